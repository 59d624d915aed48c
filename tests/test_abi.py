"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/dsa.h, and rejects bad arguments on the host before any HIP
call (these calls return before touching the device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


@pytest.fixture(scope="module")
def L():
    lib_path = os.path.join(ROOT, "dynamic_sparse_attention_lowrank_amd", "libdsa.so")
    if not os.path.exists(lib_path):
        from dynamic_sparse_attention_lowrank_amd import build as b
        b.build()
    import dynamic_sparse_attention_lowrank_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"DSA_API\s+[\w\s\*]+?\b(dsa_\w+)\s*\(", text)


def test_header_declares_entry_points():
    names = set(declared_functions())
    assert {"dsa_predict", "dsa_select", "dsa_predict_select", "dsa_attn_fwd", "dsa_attn_bwd",
            "dsa_attn_bwd_workspace_bytes", "dsa_status_string", "dsa_version", "dsa_predictor_grad",
            "dsa_predictor_grad_workspace_bytes", "dsa_rope3d", "dsa_attn_fwd_noalloc"} <= names


def test_library_exports_every_declared_symbol(L):
    raw = ctypes.CDLL(L.library_path)
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} not exported"
    assert L.lib.dsa_version() == 200


def _shape(L, **kw):
    base = dict(B=1, H=2, d=64, Lt=4, Lh=8, Lw=8, tt=1, th=4, tw=4, io=0)
    base.update(kw)
    return L.Shape(*[base[n] for n in ("B", "H", "d", "Lt", "Lh", "Lw", "tt", "th", "tw", "io")])


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), 2), (dict(d=0), 2), (dict(B=-1), 2), (dict(Lt=0), 2),
    (dict(th=3), 3), (dict(tt=0), 3), (dict(tt=2, th=8, tw=8), 3),    # 128-token tile
    (dict(io=7), 5),
])
def test_shape_validation(L, kw, code):
    sh = _shape(L, **kw)
    st = L.lib.dsa_predict(ctypes.byref(sh), 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == code, L.lib.dsa_status_string(st)


def test_entry_point_validation(L):
    sh = _shape(L)
    lib = L.lib
    assert lib.dsa_predict(None, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.dsa_predict(ctypes.byref(sh), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 9
    assert lib.dsa_predict(ctypes.byref(sh), 65, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 9
    assert lib.dsa_predict(ctypes.byref(sh), 16, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.dsa_select(ctypes.byref(sh), FAKE, FAKE, 0, FAKE, None) == 4
    assert lib.dsa_select(ctypes.byref(sh), FAKE, FAKE, 17, FAKE, None) == 4      # kmax > NB = 16
    assert lib.dsa_select(ctypes.byref(sh), None, FAKE, 4, FAKE, None) == 1
    ps = lambda shp, r, kmax, *p: lib.dsa_predict_select(shp, r, *p[:5], kmax, *p[5:], None)
    assert ps(ctypes.byref(sh), 0, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == 9
    assert ps(ctypes.byref(sh), 16, 17, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == 4
    assert ps(ctypes.byref(sh), 16, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE) == 1
    assert ps(None, 16, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == 1
    pneed = lib.dsa_predictor_grad_workspace_bytes(ctypes.byref(sh))
    rnd = lambda x: (x + 255) // 256 * 256
    BH, NB, d, H, rbs = 2, 16, 64, 2, 64 // 16
    assert pneed == (2 * rnd(BH * NB * d * 4) + 2 * rnd(BH * d * d * 4) + rnd(H * d * d * 4)   # means, Grams, M
                     + rnd(BH * d * 64 * 4) + rnd(BH * rbs * d * 64 * 4) + rnd(BH * rbs * 4))  # partial sums
    pg = lambda shp, r, p, ws, nb: lib.dsa_predictor_grad(shp, r, *p, ws, nb, None)
    assert pg(ctypes.byref(sh), 0, [FAKE] * 7, FAKE, pneed) == 9
    assert pg(ctypes.byref(sh), 65, [FAKE] * 7, FAKE, pneed) == 9
    assert pg(ctypes.byref(sh), 16, [FAKE] * 4 + [None] + [FAKE] * 2, FAKE, pneed) == 1     # no loss output
    assert pg(ctypes.byref(sh), 16, [FAKE] * 7, None, pneed) == 6
    assert pg(ctypes.byref(sh), 16, [FAKE] * 7, FAKE, pneed - 1) == 6
    assert pg(ctypes.byref(sh), 16, [FAKE] * 7, ctypes.c_void_p(0x1010), pneed) == 6
    assert pg(None, 16, [FAKE] * 7, FAKE, pneed) == 1
    assert lib.dsa_predictor_grad_workspace_bytes(None) == 0
    rp = lambda shp, dt, base, offs, inv, x, y: lib.dsa_rope3d(shp, dt, base, *offs, inv, x, y, None)
    assert rp(ctypes.byref(sh), 7, 1e4, (0, 0, 0), 0, FAKE, FAKE) == 5
    assert rp(ctypes.byref(sh), 1, 1.0, (0, 0, 0), 0, FAKE, FAKE) == 2                  # base must exceed 1
    assert rp(ctypes.byref(sh), 1, float("nan"), (0, 0, 0), 0, FAKE, FAKE) == 2
    assert rp(ctypes.byref(sh), 1, 1e4, (0, 0, 0), 2, FAKE, FAKE) == 2                  # inverse is 0 or 1
    assert rp(ctypes.byref(sh), 1, 1e4, (2 ** 30 + 1, 0, 0), 0, FAKE, FAKE) == 2
    assert rp(ctypes.byref(sh), 1, 1e4, (0, 0, 0), 0, None, FAKE) == 1
    assert rp(ctypes.byref(sh), 0, 1e4, (0, 0, 0), 0, ctypes.c_void_p(0x1004), FAKE) == 2   # fp32 pairs: 8-byte aligned
    assert rp(None, 1, 1e4, (0, 0, 0), 0, FAKE, FAKE) == 1
    fneed = lib.dsa_attn_fwd_workspace_bytes(ctypes.byref(sh))
    assert fneed == 1 * 2 * 16 * 64 * 64 * 4                                    # V^T: B*H*NB*d*64 fp32
    sh16 = _shape(L, io=1)
    rnd16 = lambda x: (x + 255) // 256 * 256
    # bf16: the fp16 V^T copy, then 64 partial maxima and one scale pair of V per (b, h)
    assert lib.dsa_attn_fwd_workspace_bytes(ctypes.byref(sh16)) == (2 * 16 * 64 * 64 * 2 + rnd16(2 * 64 * 4)
                                                                    + rnd16(2 * 8))
    fw = [FAKE, fneed, None]
    assert lib.dsa_attn_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0.125, 3, FAKE, FAKE, *fw) == 5
    assert lib.dsa_attn_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 4, float("nan"), 0, FAKE, FAKE,
                            *fw) == 2
    assert lib.dsa_attn_fwd(ctypes.byref(sh), FAKE, FAKE, None, FAKE, FAKE, 4, 0.125, 0, FAKE, FAKE, *fw) == 1
    assert lib.dsa_attn_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0.125, 0, FAKE, FAKE, None, fneed,
                            None) == 6
    assert lib.dsa_attn_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0.125, 0, FAKE, FAKE, FAKE,
                            fneed - 1, None) == 6
    need = lib.dsa_attn_bwd_workspace_bytes(ctypes.byref(sh), 4)
    assert need > 0
    args = [ctypes.byref(sh)] + [FAKE] * 4 + [0] + [FAKE] * 4 + [4, 0.125, 0, FAKE, FAKE, FAKE]
    assert lib.dsa_attn_bwd(*args, None, need, None) == 6                       # no workspace
    assert lib.dsa_attn_bwd(*args, FAKE, need - 1, None) == 6                   # too small
    assert lib.dsa_attn_bwd(*args, ctypes.c_void_p(0x1010), need, None) == 6    # misaligned
    bad_o = [ctypes.byref(sh)] + [FAKE] * 4 + [2] + [FAKE] * 4 + [4, 0.125, 0, FAKE, FAKE, FAKE]
    assert lib.dsa_attn_bwd(*bad_o, FAKE, need, None) == 5                      # unknown O dtype
    bf16_o = [ctypes.byref(sh)] + [FAKE] * 4 + [1] + [FAKE] * 4 + [4, 0.125, 0, FAKE, FAKE, FAKE]
    assert lib.dsa_attn_bwd(*bf16_o, FAKE, need, None) == 5                     # O must be the fp32 output
    assert lib.dsa_attn_bwd_prepare(ctypes.byref(sh), FAKE, 1, FAKE, FAKE, FAKE, 4, FAKE, need, None) == 5
    for bad_scale in (0.0, -0.125, float("inf"), float("nan")):
        args_s = [ctypes.byref(sh)] + [FAKE] * 4 + [0] + [FAKE] * 4 + [4, bad_scale, 0, FAKE, FAKE, FAKE]
        assert lib.dsa_attn_bwd(*args_s, FAKE, need, None) == 2
        assert lib.dsa_attn_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 4, bad_scale, 0, FAKE, FAKE,
                                *fw) == 2
    assert lib.dsa_attn_bwd_workspace_bytes(ctypes.byref(sh), 0) == 0
    assert lib.dsa_attn_bwd_workspace_bytes(None, 4) == 0


def test_noalloc_forward_host_checks(L):
    """dsa_attn_fwd_noalloc: the checks of dsa_attn_fwd, and shapes whose single head
    needs more than the fixed 144 MiB scratch are rejected (DSA_ERR_SCRATCH) before
    any HIP call."""
    lib = L.lib
    sh = _shape(L)
    na = lib.dsa_attn_fwd_noalloc
    assert na(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0.125, 3, FAKE, FAKE, None) == 5
    assert na(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0.125, 0, FAKE, FAKE, None) == 4
    assert na(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 4, float("nan"), 0, FAKE, FAKE, None) == 2
    assert na(ctypes.byref(sh), FAKE, FAKE, None, FAKE, FAKE, 4, 0.125, 0, FAKE, FAKE, None) == 1
    assert na(None, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0.125, 0, FAKE, FAKE, None) == 1
    empty = _shape(L, B=0)
    assert na(ctypes.byref(empty), None, None, None, None, None, 4, 0.125, 0, None, None, None) == 0
    scratch = 144 << 20
    # bf16 d = 128: a head's workspace is NB*128*64*2 bytes plus two 256-byte sections
    for nb_tiles, lat, code in (((96, 96), (1, 768, 768), 10),):             # NB = 9,216
        big = _shape(L, H=1, d=128, Lt=lat[0], Lh=lat[1], Lw=lat[2], tt=1, th=8, tw=8, io=1)
        nb = nb_tiles[0] * nb_tiles[1]
        assert lib.dsa_attn_fwd_workspace_bytes(ctypes.byref(big)) == nb * 128 * 64 * 2 + 512 > scratch
        assert na(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0.125, 1, FAKE, FAKE, None) == code
    fits = _shape(L, H=1, d=128, Lt=5, Lh=8 * 19, Lw=8 * 97, tt=1, th=8, tw=8, io=1)        # NB = 9,215
    assert lib.dsa_attn_fwd_workspace_bytes(ctypes.byref(fits)) == 9215 * 128 * 64 * 2 + 512 <= scratch
    # fp32 d = 128: NB = 4,609 exceeds it (4,608 fills it exactly)
    f32 = _shape(L, H=1, d=128, Lt=11, Lh=8, Lw=8 * 419, tt=1, th=8, tw=8, io=0)
    assert lib.dsa_attn_fwd_workspace_bytes(ctypes.byref(f32)) == 4609 * 128 * 64 * 4 > scratch
    assert na(ctypes.byref(f32), FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0.125, 0, FAKE, FAKE, None) == 10
    assert b"DSA_ERR_SCRATCH" in lib.dsa_status_string(10)


def test_reverse_index_and_launch_limits(L):
    """Shapes whose per-head reverse index (NB * kmax entries, int32 offsets) or
    whose launch grids (2^32 - 1 work-items) would overflow are rejected on the host."""
    lib = L.lib
    # 65,536 single-token tiles per head: NB * kmax = 65,536 * 32,768 = 2^31 entries
    sh = _shape(L, B=1, H=1, d=64, Lt=1, Lh=256, Lw=256, tt=1, th=1, tw=1, io=1)
    assert lib.dsa_attn_bwd_workspace_bytes(ctypes.byref(sh), 32768) == 0
    assert lib.dsa_attn_bwd_workspace_bytes(ctypes.byref(sh), 32767) > 0        # 2^31 - 65,536 entries: fits
    args = [ctypes.byref(sh)] + [FAKE] * 4 + [0] + [FAKE] * 4 + [32768, 0.125, 0, FAKE, FAKE, FAKE]
    assert lib.dsa_attn_bwd(*args, FAKE, 1 << 40, None) == 4
    assert lib.dsa_attn_bwd_prepare(ctypes.byref(sh), FAKE, 0, FAKE, FAKE, FAKE, 32768, FAKE, 1 << 40, None) == 4
    # B*H*NB*512 work-items of the pooling launch: 127 heads fit, 128 do not
    ok = _shape(L, B=1, H=127, d=64, Lt=1, Lh=256, Lw=256, tt=1, th=1, tw=1, io=1)
    big = _shape(L, B=1, H=128, d=64, Lt=1, Lh=256, Lw=256, tt=1, th=1, tw=1, io=1)
    assert lib.dsa_attn_fwd_workspace_bytes(ctypes.byref(ok)) > 0
    assert lib.dsa_attn_fwd_workspace_bytes(ctypes.byref(big)) == 0
    assert lib.dsa_predict(ctypes.byref(big), 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2


def test_empty_batch_is_a_no_op(L):
    sh = _shape(L, B=0)
    assert L.lib.dsa_predict(ctypes.byref(sh), 16, None, None, None, None, None, None, None, None) == 0
    assert L.lib.dsa_attn_fwd(ctypes.byref(sh), None, None, None, None, None, 4, 0.125, 0, None, None, None, 0,
                              None) == 0
    assert L.lib.dsa_predictor_grad(ctypes.byref(sh), 16, *([None] * 8), 0, None) == 0
    assert L.lib.dsa_rope3d(ctypes.byref(sh), 1, 1e4, 0, 0, 0, 0, None, None, None) == 0


def test_workspace_formula(L):
    """D (fp32 per token) + bitmap (NB x ceil(NB/32) words) + counts + offsets + entries
    + the dK/dV block order (+ for bf16 inputs: fp16 copies of dO, Q and K; for dO, V, Q, K and V again 64
    partial maxima and one scale pair per (b, h); max |D| per (b, h) with its 64
    partial maxima; D * 2^u and LSE * log2(e) per token), each section rounded up to 256 bytes."""
    sh = _shape(L, B=2, H=3, d=128, Lt=3, Lh=16, Lw=24, tt=1, th=8, tw=8, io=1)
    BH, N, NB, kmax = 6, 3 * 16 * 24, 18, 5
    r = lambda x: (x + 255) // 256 * 256
    want = (r(BH * N * 4) + r(BH * NB * 1 * 4) + r(BH * NB * 4) + r(BH * (NB + 1) * 4) + r(BH * NB * kmax * 4)
            + r(BH * NB * 4))                                # the dK/dV block order
    part, pair, copy = r(BH * 64 * 4), r(BH * 2 * 4), r(BH * N * 128 * 2)
    bf16_extra = (copy + 2 * (part + pair)                  # fp16 dO; scales of dO and V
                  + r(BH * 4) + part + 2 * r(BH * N * 4)    # max |D|, its partial maxima, D * 2^u, LSE log2 e
                  + 2 * (copy + part + pair)                # Q and K: fp16 copy and scale
                  + part + pair)                            # V's scale for the dQ phase
    assert L.lib.dsa_attn_bwd_workspace_bytes(ctypes.byref(sh), kmax) == want + bf16_extra
    sh32 = _shape(L, B=2, H=3, d=128, Lt=3, Lh=16, Lw=24, tt=1, th=8, tw=8, io=0)
    assert L.lib.dsa_attn_bwd_workspace_bytes(ctypes.byref(sh32), kmax) == want


def test_status_strings(L):
    for code in range(12):
        assert L.lib.dsa_status_string(code).startswith(b"DSA_")


def test_fwd_kernel_choice(L):
    """dsa_set_fwd_kernel takes the three kinds and rejects others (DSA_ERR_ARG),
    leaving the setting unchanged; no device call is made."""
    lib = L.lib
    assert lib.dsa_get_fwd_kernel() == 0
    try:
        for kind in (1, 2, 0):
            assert lib.dsa_set_fwd_kernel(kind) == 0
            assert lib.dsa_get_fwd_kernel() == kind
        lib.dsa_set_fwd_kernel(2)
        for bad in (-1, 3, 1 << 30):
            assert lib.dsa_set_fwd_kernel(bad) == 11
            assert lib.dsa_get_fwd_kernel() == 2
        with pytest.raises(L.DsaError):
            L.set_fwd_kernel(5)
    finally:
        lib.dsa_set_fwd_kernel(0)
    assert L.get_fwd_kernel() == L.FWD_AUTO


def test_fwd_kernel_for_shape(L):
    """The size rule (bf16: tile-pair once one head's gathered blocks, NB*64*d*4
    bytes, reach 48 MiB), the forced settings, fp32 (always one-tile) and invalid
    shapes (-1)."""
    lib = L.lib
    f = lambda **kw: lib.dsa_fwd_kernel_for(ctypes.byref(_shape(L, **kw)))
    bf = dict(d=128, tt=1, th=8, tw=8, io=1)
    assert f(Lt=16, Lh=32, Lw=64, **bf) == 1                 # 512 blocks: 16 MiB
    assert f(Lt=24, Lh=32, Lw=64, **bf) == 1                 # 768 blocks: 24 MiB
    assert f(Lt=48, Lh=32, Lw=64, **bf) == 2                 # 1536 blocks: 48 MiB
    assert f(Lt=32, Lh=128, Lw=128, **bf) == 2               # 8192 blocks
    assert f(Lt=32, Lh=128, Lw=128, d=128, tt=1, th=8, tw=8, io=0) == 1
    assert f(Lt=16, Lh=32, Lw=64, d=96, tt=1, th=8, tw=8, io=1) == -1
    try:
        lib.dsa_set_fwd_kernel(2)
        assert f(Lt=16, Lh=32, Lw=64, **bf) == 2
        lib.dsa_set_fwd_kernel(1)
        assert f(Lt=32, Lh=128, Lw=128, **bf) == 1
    finally:
        lib.dsa_set_fwd_kernel(0)
