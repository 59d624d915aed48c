"""DSV-style dynamic block-sparse attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libdsa.so`` (declared in
``include/dsa.h``).  It only marshals arguments: PyTorch supplies device
memory and the current HIP stream; every step of the path (predictor scores,
top-k selection, block-sparse attention forward and backward) runs in the
library's HIP kernels.  There is no fallback: if the library is missing or a
call fails, an exception is raised.

Method: DSV: Exploiting Dynamic Sparsity to Accelerate Large-Scale Video DiT
Training (gist.science/ar/paper/2502.07590) -- a low-rank predictor (section 3a)
scores query-tile x key-block pairs, each tile of neighbouring queries keeps
its top-k key blocks (section 3b), and exact attention runs only over those
(section 4).
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "Layout", "lib", "library_path", "predict", "select", "attn_fwd", "attn_bwd",
    "bwd_workspace_bytes", "fwd_workspace_bytes", "attn_bwd_prepare", "attn_bwd_dkdv", "attn_bwd_dq", "DsaError", "F32", "BF16",
    "predict_select", "predictor_grad", "predictor_grad_workspace_bytes", "rope3d",
    "set_fwd_kernel", "get_fwd_kernel", "fwd_kernel_for", "FWD_AUTO", "FWD_ONE_TILE", "FWD_TILE_PAIR",
]

F32 = 0
BF16 = 1
FWD_AUTO, FWD_ONE_TILE, FWD_TILE_PAIR = 0, 1, 2
_LIB_NAME = "libdsa.so"
library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), _LIB_NAME)


class DsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "H", "d", "Lt", "Lh", "Lw", "tt", "th", "tw", "io")]


def _load():
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is missing: build it with "
            "`python -m dynamic_sparse_attention_lowrank_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(library_path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    sp = ctypes.POINTER(Shape)
    L.dsa_status_string.restype = ctypes.c_char_p
    L.dsa_status_string.argtypes = [ctypes.c_int]
    L.dsa_version.restype = i32
    L.dsa_version.argtypes = []
    L.dsa_predict.restype = ctypes.c_int
    L.dsa_predict.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    L.dsa_select.restype = ctypes.c_int
    L.dsa_select.argtypes = [sp, vp, vp, i32, vp, vp]
    L.dsa_predict_select.restype = ctypes.c_int
    L.dsa_predict_select.argtypes = [sp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp]
    L.dsa_predictor_grad_workspace_bytes.restype = sz
    L.dsa_predictor_grad_workspace_bytes.argtypes = [sp]
    L.dsa_predictor_grad.restype = ctypes.c_int
    L.dsa_predictor_grad.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_rope3d.restype = ctypes.c_int
    L.dsa_rope3d.argtypes = [sp, i32, f32, i32, i32, i32, i32, vp, vp, vp]
    L.dsa_attn_fwd.restype = ctypes.c_int
    L.dsa_attn_fwd.argtypes = [sp, vp, vp, vp, vp, vp, i32, f32, i32, vp, vp, vp, sz, vp]
    L.dsa_set_fwd_kernel.restype = ctypes.c_int
    L.dsa_set_fwd_kernel.argtypes = [i32]
    L.dsa_get_fwd_kernel.restype = i32
    L.dsa_get_fwd_kernel.argtypes = []
    L.dsa_fwd_kernel_for.restype = i32
    L.dsa_fwd_kernel_for.argtypes = [sp]
    L.dsa_attn_fwd_noalloc.restype = ctypes.c_int
    L.dsa_attn_fwd_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, i32, f32, i32, vp, vp, vp]
    L.dsa_attn_fwd_workspace_bytes.restype = sz
    L.dsa_attn_fwd_workspace_bytes.argtypes = [sp]
    L.dsa_attn_bwd_workspace_bytes.restype = sz
    L.dsa_attn_bwd_workspace_bytes.argtypes = [sp, i32]
    L.dsa_attn_bwd.restype = ctypes.c_int
    L.dsa_attn_bwd.argtypes = [sp, vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, f32, i32, vp, vp, vp, vp, sz, vp]
    L.dsa_attn_bwd_prepare.restype = ctypes.c_int
    L.dsa_attn_bwd_prepare.argtypes = [sp, vp, i32, vp, vp, vp, i32, vp, sz, vp]
    L.dsa_attn_bwd_dkdv.restype = ctypes.c_int
    L.dsa_attn_bwd_dkdv.argtypes = [sp, vp, vp, vp, vp, vp, i32, f32, i32, vp, vp, vp, sz, vp]
    L.dsa_attn_bwd_dq.restype = ctypes.c_int
    L.dsa_attn_bwd_dq.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, i32, f32, i32, vp, vp, sz, vp]
    return L


_lib = None


def _L():
    """The loaded library (loaded on first use, so the build module can run without it)."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def __getattr__(name):
    if name == "lib":
        return _L()
    raise AttributeError(name)


@dataclass(frozen=True)
class Layout:
    """Latent grid and tile of a video-token sequence (tokens row-major over (t, y, x))."""
    latent: Tuple[int, int, int]
    tile: Tuple[int, int, int]

    @property
    def N(self) -> int:
        return self.latent[0] * self.latent[1] * self.latent[2]

    @property
    def T(self) -> int:
        return self.tile[0] * self.tile[1] * self.tile[2]

    @property
    def NB(self) -> int:
        return self.N // self.T


def _io_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _shape(X: torch.Tensor, layout: Layout) -> Shape:
    if X.dim() != 4:
        raise ValueError("expected a [B, H, N, d] tensor")
    B, H, N, d = X.shape
    if N != layout.N:
        raise ValueError(f"tensor has N={N} tokens but the latent {layout.latent} holds {layout.N}")
    return Shape(B, H, d, *layout.latent, *layout.tile, _io_code(X))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _expect(name: str, t, shape, dtypes) -> None:
    """Shape and dtype of one argument, checked before anything reaches the library
    (a short or mis-typed buffer would otherwise be read or written past its end)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(name: str, t, need: int) -> None:
    if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 1-D uint8 tensor")
    if t.numel() < need:
        raise ValueError(f"{name} holds {t.numel()} bytes, {need} needed")


def _dev(*ts: torch.Tensor) -> None:
    """Every tensor on the same GPU (checked after the shapes and dtypes)."""
    dev = None
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must live on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices: {dev} and {t.device}")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


_IO = (torch.float32, torch.bfloat16)


def _qkv(layout: "Layout", Q: torch.Tensor, **named: torch.Tensor):
    """Q is [B, H, N, d] float32 or bfloat16 and every other named tensor matches it."""
    if not isinstance(Q, torch.Tensor) or Q.dim() != 4:
        raise ValueError("Q must be a [B, H, N, d] tensor")
    _expect("Q", Q, Q.shape, _IO)
    if Q.shape[2] != layout.N:
        raise ValueError(f"Q has N={Q.shape[2]} tokens but the latent {layout.latent} holds {layout.N}")
    for n, t in named.items():
        _expect(n, t, Q.shape, Q.dtype)
    return Q.shape


def _kvec(k: torch.Tensor, B: int, H: int) -> None:
    _expect("k", k, (B * H,), torch.int32)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(status: int) -> None:
    if status != 0:
        raise DsaError(status, _L().dsa_status_string(status).decode())


def _rank(Wq: torch.Tensor, Wk: torch.Tensor, H: int, d: int, dtype) -> int:
    """Wq, Wk are [H, d, r] in the I/O dtype; returns r."""
    if not isinstance(Wq, torch.Tensor) or Wq.dim() != 3:
        raise ValueError("Wq must be an [H, d, r] tensor")
    r = Wq.shape[-1]
    _expect("Wq", Wq, (H, d, r), dtype)
    _expect("Wk", Wk, (H, d, r), dtype)
    return r


def predict(Q: torch.Tensor, K: torch.Tensor, Wq: torch.Tensor, Wk: torch.Tensor, layout: Layout,
            out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Low-rank predictor: returns (Qbar, Kbar, S) as float32 [B,H,NB,r], [B,H,NB,r], [B,H,NB,NB]."""
    B, H, N, d = _qkv(layout, Q, K=K)
    r = _rank(Wq, Wk, H, d, Q.dtype)
    if out is None:
        Qbar = torch.empty(B, H, layout.NB, r, device=Q.device, dtype=torch.float32)
        Kbar = torch.empty_like(Qbar)
        S = torch.empty(B, H, layout.NB, layout.NB, device=Q.device, dtype=torch.float32)
    else:
        Qbar, Kbar, S = out
    _expect("Qbar", Qbar, (B, H, layout.NB, r), torch.float32)
    _expect("Kbar", Kbar, (B, H, layout.NB, r), torch.float32)
    _expect("S", S, (B, H, layout.NB, layout.NB), torch.float32)
    _dev(Q, K, Wq, Wk, Qbar, Kbar, S)
    sh = _shape(Q, layout)
    _check(_L().dsa_predict(ctypes.byref(sh), r, _ptr(Q), _ptr(K), _ptr(Wq), _ptr(Wk), _ptr(Qbar), _ptr(Kbar),
                           _ptr(S), _stream()))
    return Qbar, Kbar, S


def select(S: torch.Tensor, k: torch.Tensor, kmax: int, layout: Layout, d: int = 128,
           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-k key blocks per query tile: idx int32 [B,H,NB,kmax], ascending, -1 padded."""
    if not isinstance(S, torch.Tensor) or S.dim() != 4:
        raise ValueError("S must be a [B, H, NB, NB] tensor")
    B, H = S.shape[:2]
    _expect("S", S, (B, H, layout.NB, layout.NB), torch.float32)
    _kvec(k, B, H)
    idx = out if out is not None else torch.empty(B, H, layout.NB, kmax, device=S.device, dtype=torch.int32)
    _expect("idx", idx, (B, H, layout.NB, kmax), torch.int32)
    _dev(S, k, idx)
    sh = Shape(B, H, d, *layout.latent, *layout.tile, F32)
    _check(_L().dsa_select(ctypes.byref(sh), _ptr(S), _ptr(k), kmax, _ptr(idx), _stream()))
    return idx


def predict_select(Q: torch.Tensor, K: torch.Tensor, Wq: torch.Tensor, Wk: torch.Tensor, k: torch.Tensor, kmax: int,
                   layout: Layout, out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Predictor and top-k selection without the score matrix: returns (Qbar, Kbar, idx)."""
    B, H, N, d = _qkv(layout, Q, K=K)
    r = _rank(Wq, Wk, H, d, Q.dtype)
    _kvec(k, B, H)
    if out is None:
        Qbar = torch.empty(B, H, layout.NB, r, device=Q.device, dtype=torch.float32)
        Kbar = torch.empty_like(Qbar)
        idx = torch.empty(B, H, layout.NB, kmax, device=Q.device, dtype=torch.int32)
    else:
        Qbar, Kbar, idx = out
    _expect("Qbar", Qbar, (B, H, layout.NB, r), torch.float32)
    _expect("Kbar", Kbar, (B, H, layout.NB, r), torch.float32)
    _expect("idx", idx, (B, H, layout.NB, kmax), torch.int32)
    _dev(Q, K, Wq, Wk, k, Qbar, Kbar, idx)
    sh = _shape(Q, layout)
    _check(_L().dsa_predict_select(ctypes.byref(sh), r, _ptr(Q), _ptr(K), _ptr(Wq), _ptr(Wk), _ptr(k), kmax,
                                   _ptr(Qbar), _ptr(Kbar), _ptr(idx), _stream()))
    return Qbar, Kbar, idx


def rope3d(X: torch.Tensor, layout: Layout, base: float = 10000.0, offsets: Tuple[int, int, int] = (0, 0, 0),
           inverse: bool = False, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """3-D rotary positions of X [B,H,N,d] (bf16 or fp32); `out` may be X (in place)."""
    _qkv(layout, X)
    Y = torch.empty_like(X) if out is None else out
    _expect("out", Y, X.shape, X.dtype)
    _dev(X, Y)
    sh = _shape(X, layout)
    dt = F32 if X.dtype == torch.float32 else BF16
    _check(_L().dsa_rope3d(ctypes.byref(sh), dt, float(base), int(offsets[0]), int(offsets[1]), int(offsets[2]),
                           int(bool(inverse)), _ptr(X), _ptr(Y), _stream()))
    return Y


def predictor_grad_workspace_bytes(Q: torch.Tensor, layout: Layout) -> int:
    sh = _shape(Q, layout)
    return int(_L().dsa_predictor_grad_workspace_bytes(ctypes.byref(sh)))


def predictor_grad(Q: torch.Tensor, K: torch.Tensor, Wq: torch.Tensor, Wk: torch.Tensor, layout: Layout,
                   out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                   workspace: Optional[torch.Tensor] = None):
    """Stage-one predictor loss and weight gradients: returns (loss [B,H], dWq [H,d,r], dWk [H,d,r]), fp32."""
    B, H, N, d = _qkv(layout, Q, K=K)
    r = _rank(Wq, Wk, H, d, Q.dtype)
    if out is None:
        loss = torch.empty(B, H, device=Q.device, dtype=torch.float32)
        dWq = torch.empty(Wq.shape, device=Q.device, dtype=torch.float32)
        dWk = torch.empty(Wk.shape, device=Q.device, dtype=torch.float32)
    else:
        loss, dWq, dWk = out
    _expect("loss", loss, (B, H), torch.float32)
    _expect("dWq", dWq, (H, d, r), torch.float32)
    _expect("dWk", dWk, (H, d, r), torch.float32)
    sh = _shape(Q, layout)
    need = int(_L().dsa_predictor_grad_workspace_bytes(ctypes.byref(sh)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=Q.device, dtype=torch.uint8)
    _workspace("workspace", workspace, need)
    _dev(Q, K, Wq, Wk, loss, dWq, dWk, workspace)
    _check(_L().dsa_predictor_grad(ctypes.byref(sh), r, _ptr(Q), _ptr(K), _ptr(Wq), _ptr(Wk), _ptr(loss), _ptr(dWq),
                                   _ptr(dWk), _ptr(workspace), workspace.numel(), _stream()))
    return loss, dWq, dWk


def fwd_workspace_bytes(Q: torch.Tensor, layout: Layout) -> int:
    sh = _shape(Q, layout)
    return int(_L().dsa_attn_fwd_workspace_bytes(ctypes.byref(sh)))


def _idx(idx: torch.Tensor, B: int, H: int, layout: "Layout") -> int:
    """idx is int32 [B, H, NB, kmax]; returns kmax."""
    if not isinstance(idx, torch.Tensor) or idx.dim() != 4:
        raise ValueError("idx must be a [B, H, NB, kmax] tensor")
    _expect("idx", idx, (B, H, layout.NB, idx.shape[-1]), torch.int32)
    return idx.shape[-1]


def attn_fwd(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, idx: torch.Tensor, k: torch.Tensor, layout: Layout,
             scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
             out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None, workspace: Optional[torch.Tensor] = None):
    """Block-sparse attention forward: returns (O [B,H,N,d] out_dtype, LSE [B,H,N] float32)."""
    B, H, N, d = _qkv(layout, Q, K=K, V=V)
    kmax = _idx(idx, B, H, layout)
    _kvec(k, B, H)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    odt = out_dtype or Q.dtype
    if out is None:
        O = torch.empty(Q.shape, device=Q.device, dtype=odt)
        LSE = torch.empty(Q.shape[:3], device=Q.device, dtype=torch.float32)
    else:
        O, LSE = out
    _expect("O", O, Q.shape, _IO)
    _expect("LSE", LSE, (B, H, N), torch.float32)
    sh = _shape(Q, layout)
    need = int(_L().dsa_attn_fwd_workspace_bytes(ctypes.byref(sh)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=Q.device, dtype=torch.uint8)
    _workspace("workspace", workspace, need)
    _dev(Q, K, V, idx, k, O, LSE, workspace)
    _check(_L().dsa_attn_fwd(ctypes.byref(sh), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx), _ptr(k), kmax, scale,
                             _io_code(O), _ptr(O), _ptr(LSE), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream()))
    return O, LSE


def set_fwd_kernel(kind: int) -> None:
    """Which bf16 forward kernel runs: FWD_AUTO (by size), FWD_ONE_TILE or
    FWD_TILE_PAIR (process-wide; see dsa_set_fwd_kernel in include/dsa.h)."""
    _check(_L().dsa_set_fwd_kernel(int(kind)))


def get_fwd_kernel() -> int:
    return int(_L().dsa_get_fwd_kernel())


def fwd_kernel_for(Q: torch.Tensor, layout: Layout) -> int:
    """FWD_ONE_TILE or FWD_TILE_PAIR: the kernel attn_fwd runs for Q's shape now."""
    sh = _shape(Q, layout)
    r = int(_L().dsa_fwd_kernel_for(ctypes.byref(sh)))
    if r < 0:
        raise ValueError("invalid shape for the forward")
    return r


def attn_fwd_noalloc(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, idx: torch.Tensor, k: torch.Tensor,
                     layout: Layout, out: Tuple[torch.Tensor, torch.Tensor], scale: Optional[float] = None):
    """attn_fwd into the caller's (O, LSE) without any device allocation: the library
    uses its fixed per-GPU scratch array instead of a workspace (calls that overlap in
    time on one GPU race on it)."""
    B, H, N, d = _qkv(layout, Q, K=K, V=V)
    kmax = _idx(idx, B, H, layout)
    _kvec(k, B, H)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O, LSE = out
    _expect("O", O, Q.shape, _IO)
    _expect("LSE", LSE, (B, H, N), torch.float32)
    _dev(Q, K, V, idx, k, O, LSE)
    sh = _shape(Q, layout)
    _check(_L().dsa_attn_fwd_noalloc(ctypes.byref(sh), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx), _ptr(k), kmax, scale,
                                     _io_code(O), _ptr(O), _ptr(LSE), _stream()))
    return O, LSE


def bwd_workspace_bytes(Q: torch.Tensor, layout: Layout, kmax: int) -> int:
    sh = _shape(Q, layout)
    return int(_L().dsa_attn_bwd_workspace_bytes(ctypes.byref(sh), kmax))


def attn_bwd(Q, K, V, O, dO, LSE, idx, k, layout: Layout, scale: Optional[float] = None,
             out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None,
             out: Optional[Sequence[torch.Tensor]] = None):
    """Block-sparse attention backward (mask fixed): returns (dQ, dK, dV).

    O is the float32 forward output (it enters through D = dO . O)."""
    B, H, N, d = _qkv(layout, Q, K=K, V=V, dO=dO)
    _expect("O", O, Q.shape, torch.float32)
    _expect("LSE", LSE, (B, H, N), torch.float32)
    kmax = _idx(idx, B, H, layout)
    _kvec(k, B, H)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    odt = out_dtype or Q.dtype
    if out is None:
        dQ = torch.empty(Q.shape, device=Q.device, dtype=odt)
        dK = torch.empty_like(dQ)
        dV = torch.empty_like(dQ)
    else:
        dQ, dK, dV = out
    _expect("dQ", dQ, Q.shape, _IO)
    _expect("dK", dK, Q.shape, dQ.dtype)
    _expect("dV", dV, Q.shape, dQ.dtype)
    sh = _shape(Q, layout)
    need = int(_L().dsa_attn_bwd_workspace_bytes(ctypes.byref(sh), kmax))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=Q.device, dtype=torch.uint8)
    _workspace("workspace", workspace, need)
    _dev(Q, K, V, O, dO, LSE, idx, k, dQ, dK, dV, workspace)
    _check(_L().dsa_attn_bwd(ctypes.byref(sh), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _io_code(O), _ptr(dO), _ptr(LSE),
                            _ptr(idx),
                            _ptr(k), kmax, scale, _io_code(dQ), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream()))
    return dQ, dK, dV


def _ws_args(workspace: torch.Tensor):
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def attn_bwd_prepare(O, dO, idx, k, layout: Layout, workspace: torch.Tensor) -> None:
    """Backward phase 1: D and the reverse block index into ``workspace``."""
    B, H, N, d = _qkv(layout, dO)
    _expect("O", O, dO.shape, torch.float32)
    kmax = _idx(idx, B, H, layout)
    _kvec(k, B, H)
    sh = _shape(dO, layout)
    _workspace("workspace", workspace, int(_L().dsa_attn_bwd_workspace_bytes(ctypes.byref(sh), kmax)))
    _dev(O, dO, idx, k, workspace)
    _check(_L().dsa_attn_bwd_prepare(ctypes.byref(sh), _ptr(O), _io_code(O), _ptr(dO), _ptr(idx), _ptr(k),
                                    kmax, *_ws_args(workspace), _stream()))


def attn_bwd_dkdv(Q, K, V, dO, LSE, kmax: int, layout: Layout, workspace: torch.Tensor, dK: torch.Tensor,
                  dV: torch.Tensor, scale: Optional[float] = None) -> None:
    """Backward phase 2: dK, dV (needs a prepared workspace)."""
    B, H, N, d = _qkv(layout, Q, K=K, V=V, dO=dO)
    _expect("LSE", LSE, (B, H, N), torch.float32)
    _expect("dK", dK, Q.shape, _IO)
    _expect("dV", dV, Q.shape, dK.dtype)
    sh = _shape(Q, layout)
    _workspace("workspace", workspace, int(_L().dsa_attn_bwd_workspace_bytes(ctypes.byref(sh), kmax)))
    _dev(Q, K, V, dO, LSE, workspace, dK, dV)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(_L().dsa_attn_bwd_dkdv(ctypes.byref(sh), _ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(LSE), kmax, scale,
                                 _io_code(dK), _ptr(dK), _ptr(dV), *_ws_args(workspace), _stream()))


def attn_bwd_dq(Q, K, V, dO, LSE, idx, k, layout: Layout, workspace: torch.Tensor, dQ: torch.Tensor,
                scale: Optional[float] = None) -> None:
    """Backward phase 3: dQ (needs a prepared workspace)."""
    B, H, N, d = _qkv(layout, Q, K=K, V=V, dO=dO)
    _expect("LSE", LSE, (B, H, N), torch.float32)
    kmax = _idx(idx, B, H, layout)
    _kvec(k, B, H)
    _expect("dQ", dQ, Q.shape, _IO)
    sh = _shape(Q, layout)
    _workspace("workspace", workspace, int(_L().dsa_attn_bwd_workspace_bytes(ctypes.byref(sh), kmax)))
    _dev(Q, K, V, dO, LSE, idx, k, workspace, dQ)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(_L().dsa_attn_bwd_dq(ctypes.byref(sh), _ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(LSE), _ptr(idx), _ptr(k),
                               kmax, scale, _io_code(dQ), _ptr(dQ), *_ws_args(workspace), _stream()))
