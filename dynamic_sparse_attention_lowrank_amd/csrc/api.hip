// C ABI of libdsa (declared in include/dsa.h): argument checks on the host,
// shape derivation, workspace carving and kernel launches.  No entry point
// allocates memory or synchronises the device; the only state is the per-device
// address of the fixed scratch array of dsa_attn_fwd_noalloc.
#include <math.h>
#include <stdint.h>

#include "dsa.h"
#include "kernels.hpp"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

using namespace dsa;

namespace {

struct Derived {
  Geo g;
  int BH;
  int d;
  int io_f32;
};

dsa_status derive(const dsa_shape* s, Derived* out) {
  if (s == nullptr) return DSA_ERR_NULL;
  if (s->io != DSA_F32 && s->io != DSA_BF16) return DSA_ERR_DTYPE;
  if (s->B < 0 || s->H < 0) return DSA_ERR_SHAPE;
  if (s->d != 64 && s->d != 128) return DSA_ERR_SHAPE;
  if (s->Lt < 1 || s->Lh < 1 || s->Lw < 1) return DSA_ERR_SHAPE;
  if (s->tt < 1 || s->th < 1 || s->tw < 1) return DSA_ERR_TILE;
  if (s->Lt % s->tt || s->Lh % s->th || s->Lw % s->tw) return DSA_ERR_TILE;
  const int64_t T = (int64_t)s->tt * s->th * s->tw;
  if (T > 64) return DSA_ERR_TILE;
  const int64_t N = (int64_t)s->Lt * s->Lh * s->Lw;
  const int64_t esz = s->io == DSA_F32 ? 4 : 2;
  const int64_t NB = N / T;
  // every per-head byte offset (token rows, and the forward's 64-position V^T
  // blocks) must fit the kernels' signed 32-bit buffer offsets
  if (N * s->d * esz > (int64_t)INT32_MAX || NB * s->d * 64 * esz > (int64_t)INT32_MAX) return DSA_ERR_SHAPE;
  const int64_t BH = (int64_t)s->B * s->H;
  // launch limits: the grid of one launch holds at most 2^32 - 1 work-items per
  // dimension, and the largest grids are the predictor's pooling (2 x 256
  // work-items per (b, h, tile)) and the attention kernels (256 per tile)
  if (BH > 65535 || BH * NB * 512 > (int64_t)UINT32_MAX) return DSA_ERR_SHAPE;
  Geo g;
  g.Lt = s->Lt; g.Lh = s->Lh; g.Lw = s->Lw;
  g.tt = s->tt; g.th = s->th; g.tw = s->tw;
  g.gt = s->Lt / s->tt; g.gh = s->Lh / s->th; g.gw = s->Lw / s->tw;
  g.N = (int)N; g.T = (int)T; g.NB = (int)NB;
  auto rcp = [](int64_t d) -> uint32_t { return d == 1 ? 0u : (uint32_t)(((int64_t)1 << 32) / d + (((int64_t)1 << 32) % d != 0)); };
  g.m_gw = rcp(g.gw);
  g.m_gwgh = rcp((int64_t)g.gw * g.gh);
  g.m_tw = rcp(g.tw);
  g.m_twth = rcp((int64_t)g.tw * g.th);
  g.fast_tiles = NB <= 65535;
  out->g = g;
  out->BH = (int)BH;
  out->d = s->d;
  out->io_f32 = s->io == DSA_F32;
  return DSA_OK;
}

dsa_status hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdLayout {
  size_t dvec, bitmap, counts, offsets, entries, order, do16, dmax, dscale, vmax, vscale;
  size_t dabs, dabs_part, du, lse2, q16, qmax, qscale, k16, kmaxp, kscale, vmax_q, vscale_q, total;
  int words;
};

BwdLayout bwd_layout(const Derived& dv, int kmax) {
  BwdLayout l;
  const size_t BH = (size_t)dv.BH, N = (size_t)dv.g.N, NB = (size_t)dv.g.NB;
  l.words = (int)((NB + 31) / 32);
  size_t off = 0;
  l.dvec = off;    off += align256(BH * N * sizeof(float));
  l.bitmap = off;  off += align256(BH * NB * (size_t)l.words * sizeof(uint32_t));
  l.counts = off;  off += align256(BH * NB * sizeof(int32_t));
  l.offsets = off; off += align256(BH * (NB + 1) * sizeof(int32_t));
  l.entries = off; off += align256(BH * NB * (size_t)kmax * sizeof(int32_t));
  l.order = off;   off += align256(BH * NB * sizeof(int32_t));
  l.do16 = off;    off += dv.io_f32 ? 0 : align256(BH * N * (size_t)dv.d * 2);
  l.dmax = off;    off += dv.io_f32 ? 0 : align256(BH * kDoChunks * sizeof(uint32_t));
  l.dscale = off;  off += dv.io_f32 ? 0 : align256(BH * 2 * sizeof(float));
  l.vmax = off;    off += dv.io_f32 ? 0 : align256(BH * kDoChunks * sizeof(uint32_t));
  l.vscale = off;  off += dv.io_f32 ? 0 : align256(BH * 2 * sizeof(float));
  // bf16: the single-pass fp16 dS products (max |D|, scaled D, LSE in log2 units, fp16 copies of Q
  // for dK/dV and of K for dQ, and their scales; V's scale again for dQ)
  const size_t part = align256(BH * kDoChunks * sizeof(uint32_t)), sc = align256(BH * 2 * sizeof(float));
  const size_t copy = align256(BH * N * (size_t)dv.d * 2);
  l.dabs = off;      off += dv.io_f32 ? 0 : align256(BH * sizeof(uint32_t));
  l.dabs_part = off; off += dv.io_f32 ? 0 : part;
  l.du = off;        off += dv.io_f32 ? 0 : align256(BH * N * sizeof(float));
  l.lse2 = off;      off += dv.io_f32 ? 0 : align256(BH * N * sizeof(float));
  l.q16 = off;       off += dv.io_f32 ? 0 : copy;
  l.qmax = off;      off += dv.io_f32 ? 0 : part;
  l.qscale = off;    off += dv.io_f32 ? 0 : sc;
  l.k16 = off;       off += dv.io_f32 ? 0 : copy;
  l.kmaxp = off;     off += dv.io_f32 ? 0 : part;
  l.kscale = off;    off += dv.io_f32 ? 0 : sc;
  l.vmax_q = off;    off += dv.io_f32 ? 0 : part;
  l.vscale_q = off;  off += dv.io_f32 ? 0 : sc;
  l.total = off;
  return l;
}

// The reverse index stores, per head, offsets into a list of at most NB * kmax
// entries as int32: larger selections are rejected.
bool csc_fits(const Derived& dv, int kmax) { return (int64_t)dv.g.NB * kmax <= (int64_t)INT32_MAX; }

// softmax scale: finite and positive (the kernels take the row maximum of the
// unscaled scores)
bool scale_ok(float scale) { return isfinite(scale) && scale > 0.f; }

// bf16 forward kernel choice (dsa_set_fwd_kernel), read at every forward call
std::atomic<int32_t> g_fwd_kernel{DSA_FWD_AUTO};

// --- fixed scratch of dsa_attn_fwd_noalloc ------------------------------------
// One array per GPU (each device that loads this code object holds its own copy,
// at its own address).  In host code `fwd_scratch` only names the symbol: its
// device address is looked up once per device with hipGetSymbolAddress and kept
// in g_scratch_addr; kernels receive that address, never the symbol.
constexpr size_t kFwdScratchBytes = (size_t)144 << 20;
static __device__ __align__(256) unsigned char fwd_scratch[kFwdScratchBytes];
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

// device address of the current device's scratch array (looked up on first use)
hipError_t fwd_scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(fwd_scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p & 255u)) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL: return "DSA_ERR_NULL: a required pointer is NULL";
    case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE: unsupported B, H, N or d";
    case DSA_ERR_TILE: return "DSA_ERR_TILE: tile does not divide the latent or holds more than 64 tokens";
    case DSA_ERR_K: return "DSA_ERR_K: kmax out of range";
    case DSA_ERR_DTYPE: return "DSA_ERR_DTYPE: unknown element type";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace too small, NULL or not 256-byte aligned";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: a HIP launch failed";
    case DSA_ERR_NOT_IMPLEMENTED: return "DSA_ERR_NOT_IMPLEMENTED";
    case DSA_ERR_RANK: return "DSA_ERR_RANK: predictor rank must be in [1, 64]";
    case DSA_ERR_SCRATCH:
      return "DSA_ERR_SCRATCH: one head's forward workspace exceeds the 144 MiB scratch of dsa_attn_fwd_noalloc";
    case DSA_ERR_ARG: return "DSA_ERR_ARG: an enumerated argument is out of range";
  }
  return "unknown dsa_status";
}

int32_t dsa_version(void) { return 200; }

dsa_status dsa_set_fwd_kernel(int32_t kind) {
  if (kind != DSA_FWD_AUTO && kind != DSA_FWD_ONE_TILE && kind != DSA_FWD_TILE_PAIR) return DSA_ERR_ARG;
  g_fwd_kernel.store(kind, std::memory_order_relaxed);
  return DSA_OK;
}

int32_t dsa_get_fwd_kernel(void) { return g_fwd_kernel.load(std::memory_order_relaxed); }

int32_t dsa_fwd_kernel_for(const dsa_shape* shape) {
  Derived dv;
  if (derive(shape, &dv) != DSA_OK) return -1;
  return attn_fwd_kernel_for(dv.g, dv.d, dv.io_f32, g_fwd_kernel.load(std::memory_order_relaxed));
}

dsa_status dsa_predict(const dsa_shape* shape, int32_t r, const void* Q, const void* K, const void* Wq,
                       const void* Wk, float* Qbar, float* Kbar, float* S, hipStream_t stream) {
  Derived dv;
  dsa_status st = derive(shape, &dv);
  if (st != DSA_OK) return st;
  if (r < 1 || r > 64) return DSA_ERR_RANK;
  if (dv.BH == 0) return DSA_OK;
  if (!Q || !K || !Wq || !Wk || !Qbar || !Kbar || !S) return DSA_ERR_NULL;
  PredictArgs a;
  a.Q = Q; a.K = K; a.Wq = Wq; a.Wk = Wk;
  a.Qbar = Qbar; a.Kbar = Kbar; a.S = S;
  a.g = dv.g; a.B = shape->B; a.H = shape->H; a.r = r;
  return hip_status(launch_predict(a, dv.io_f32, dv.d, stream));
}

dsa_status dsa_predict_select(const dsa_shape* shape, int32_t r, const void* Q, const void* K, const void* Wq,
                              const void* Wk, const int32_t* k, int32_t kmax, float* Qbar, float* Kbar, int32_t* idx,
                              hipStream_t stream) {
  Derived dv;
  dsa_status st = derive(shape, &dv);
  if (st != DSA_OK) return st;
  if (r < 1 || r > 64) return DSA_ERR_RANK;
  if (kmax < 1 || kmax > dv.g.NB) return DSA_ERR_K;
  if (dv.BH == 0) return DSA_OK;
  if (!Q || !K || !Wq || !Wk || !Qbar || !Kbar || !k || !idx) return DSA_ERR_NULL;
  PredictArgs a;
  a.Q = Q; a.K = K; a.Wq = Wq; a.Wk = Wk;
  a.Qbar = Qbar; a.Kbar = Kbar; a.S = nullptr;
  a.g = dv.g; a.B = shape->B; a.H = shape->H; a.r = r;
  hipError_t e = launch_pool_project(a, dv.io_f32, dv.d, stream);
  if (e != hipSuccess) return hip_status(e);
  FusedSelectArgs f;
  f.Qbar = Qbar; f.Kbar = Kbar; f.kvec = k; f.kmax = kmax; f.idx = idx; f.NB = dv.g.NB; f.BH = dv.BH; f.r = r;
  return hip_status(launch_fused_select(f, stream));
}

size_t dsa_predictor_grad_workspace_bytes(const dsa_shape* shape) {
  Derived dv;
  if (derive(shape, &dv) != DSA_OK) return 0;
  return predictor_grad_workspace_bytes(dv.BH, shape->H, dv.g.NB, dv.d);
}

dsa_status dsa_predictor_grad(const dsa_shape* shape, int32_t r, const void* Q, const void* K, const void* Wq,
                              const void* Wk, float* loss, float* dWq, float* dWk, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  Derived dv;
  dsa_status st = derive(shape, &dv);
  if (st != DSA_OK) return st;
  if (r < 1 || r > 64) return DSA_ERR_RANK;
  if (dv.BH == 0) return DSA_OK;
  if (!Q || !K || !Wq || !Wk || !loss || !dWq || !dWk) return DSA_ERR_NULL;
  const size_t need = predictor_grad_workspace_bytes(dv.BH, shape->H, dv.g.NB, dv.d);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return DSA_ERR_WORKSPACE;
  PGradArgs g;
  predictor_grad_carve(g, workspace, dv.BH, shape->H, dv.g.NB, dv.d);
  g.Wq = Wq; g.Wk = Wk; g.loss = loss; g.dWq = dWq; g.dWk = dWk;
  g.B = shape->B; g.H = shape->H; g.NB = dv.g.NB; g.r = r;
  // tile means only (no projection): the pooling kernel of the predictor
  PredictArgs a;
  a.Q = Q; a.K = K; a.Wq = Wq; a.Wk = Wk;
  a.Qbar = nullptr; a.Kbar = nullptr; a.S = nullptr;
  a.Pq = const_cast<float*>(g.Pq); a.Pk = const_cast<float*>(g.Pk);
  a.g = dv.g; a.B = shape->B; a.H = shape->H; a.r = r;
  hipError_t e = launch_pool_project(a, dv.io_f32, dv.d, stream);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_predictor_grad(g, dv.io_f32, dv.d, stream));
}

dsa_status dsa_rope3d(const dsa_shape* shape, int32_t dtype, float base, int32_t t0, int32_t y0, int32_t x0,
                      int32_t inverse, const void* X, void* Y, hipStream_t stream) {
  Derived dv;
  dsa_status st = derive(shape, &dv);
  if (st != DSA_OK) return st;
  if (dtype != DSA_F32 && dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (!(base > 1.f) || !(base < 3.0e38f)) return DSA_ERR_SHAPE;       // also rejects NaN
  const int32_t lim = 1 << 30;
  if (t0 < -lim || t0 > lim || y0 < -lim || y0 > lim || x0 < -lim || x0 > lim) return DSA_ERR_SHAPE;
  if (inverse != 0 && inverse != 1) return DSA_ERR_SHAPE;
  if (dv.BH == 0) return DSA_OK;
  if (!X || !Y) return DSA_ERR_NULL;
  const uintptr_t pair_bytes = dtype == DSA_F32 ? 8 : 4;
  if (((uintptr_t)X | (uintptr_t)Y) & (pair_bytes - 1)) return DSA_ERR_SHAPE;
  RopeArgs a;
  a.X = X; a.Y = Y; a.g = dv.g; a.BH = dv.BH; a.d = dv.d;
  a.t0 = t0; a.y0 = y0; a.x0 = x0;
  a.log2_base = std::log2(base);
  a.inverse = inverse;
  return hip_status(launch_rope3d(a, dtype == DSA_F32, stream));
}

dsa_status dsa_select(const dsa_shape* shape, const float* S, const int32_t* k, int32_t kmax, int32_t* idx,
                      hipStream_t stream) {
  Derived dv;
  dsa_status st = derive(shape, &dv);
  if (st != DSA_OK) return st;
  if (kmax < 1 || kmax > dv.g.NB) return DSA_ERR_K;
  if (dv.BH == 0) return DSA_OK;
  if (!S || !k || !idx) return DSA_ERR_NULL;
  SelectArgs a;
  a.S = S; a.kvec = k; a.kmax = kmax; a.idx = idx; a.NB = dv.g.NB; a.BH = dv.BH;
  return hip_status(launch_select(a, stream));
}

size_t dsa_attn_fwd_workspace_bytes(const dsa_shape* shape) {
  Derived dv;
  if (derive(shape, &dv) != DSA_OK) return 0;
  return attn_fwd_workspace_bytes(dv.BH, dv.g.NB, dv.d, dv.io_f32);
}

dsa_status dsa_attn_fwd(const dsa_shape* shape, const void* Q, const void* K, const void* V, const int32_t* idx,
                        const int32_t* k, int32_t kmax, float scale, int32_t out_dtype, void* O, float* LSE,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Derived dv;
  dsa_status st = derive(shape, &dv);
  if (st != DSA_OK) return st;
  if (out_dtype != DSA_F32 && out_dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (kmax < 1 || kmax > dv.g.NB) return DSA_ERR_K;
  if (!scale_ok(scale)) return DSA_ERR_SHAPE;
  if (dv.BH == 0) return DSA_OK;
  if (!Q || !K || !V || !idx || !k || !O || !LSE) return DSA_ERR_NULL;
  const size_t need = attn_fwd_workspace_bytes(dv.BH, dv.g.NB, dv.d, dv.io_f32);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return DSA_ERR_WORKSPACE;
  FwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.idx = idx; a.kvec = k; a.kmax = kmax;
  a.O = O; a.LSE = LSE; a.out_f32 = out_dtype == DSA_F32;
  a.c = scale * kLog2e;
  a.Vt = workspace;
  a.g = dv.g; a.BH = dv.BH;
  a.kernel = g_fwd_kernel.load(std::memory_order_relaxed);
  return hip_status(launch_attn_fwd(a, dv.io_f32, dv.d, stream));
}

dsa_status dsa_attn_fwd_noalloc(const dsa_shape* shape, const void* Q, const void* K, const void* V,
                                const int32_t* idx, const int32_t* k, int32_t kmax, float scale, int32_t out_dtype,
                                void* O, float* LSE, hipStream_t stream) {
  Derived dv;
  dsa_status st = derive(shape, &dv);
  if (st != DSA_OK) return st;
  if (out_dtype != DSA_F32 && out_dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (kmax < 1 || kmax > dv.g.NB) return DSA_ERR_K;
  if (!scale_ok(scale)) return DSA_ERR_SHAPE;
  if (dv.BH == 0) return DSA_OK;
  if (!Q || !K || !V || !idx || !k || !O || !LSE) return DSA_ERR_NULL;
  if (attn_fwd_workspace_bytes(1, dv.g.NB, dv.d, dv.io_f32) > kFwdScratchBytes) return DSA_ERR_SCRATCH;
  // heads per group: as many as the scratch holds (every head's computation is
  // independent of the others', so grouping changes no result)
  const size_t per_head = (size_t)dv.g.NB * dv.d * 64 * (dv.io_f32 ? 4 : 2);
  int G = (int)std::min<size_t>((size_t)dv.BH, kFwdScratchBytes / per_head);
  while (G > 1 && attn_fwd_workspace_bytes(G, dv.g.NB, dv.d, dv.io_f32) > kFwdScratchBytes) --G;
  void* ws = nullptr;
  const hipError_t e = fwd_scratch_address(&ws);
  if (e != hipSuccess) return DSA_ERR_HIP;
  const size_t in_head = (size_t)dv.g.N * dv.d * (dv.io_f32 ? 4 : 2);          // bytes of one head of Q, K, V
  const size_t out_head = (size_t)dv.g.N * dv.d * (out_dtype == DSA_F32 ? 4 : 2);
  for (int h0 = 0; h0 < dv.BH; h0 += G) {
    FwdArgs a;
    a.Q = static_cast<const char*>(Q) + h0 * in_head;
    a.K = static_cast<const char*>(K) + h0 * in_head;
    a.V = static_cast<const char*>(V) + h0 * in_head;
    a.idx = idx + (size_t)h0 * dv.g.NB * kmax;
    a.kvec = k + h0;
    a.kmax = kmax;
    a.O = static_cast<char*>(O) + h0 * out_head;
    a.LSE = LSE + (size_t)h0 * dv.g.N;
    a.out_f32 = out_dtype == DSA_F32;
    a.c = scale * kLog2e;
    a.Vt = ws;
    a.kernel = g_fwd_kernel.load(std::memory_order_relaxed);
    a.g = dv.g;
    a.BH = std::min(G, dv.BH - h0);
    st = hip_status(launch_attn_fwd(a, dv.io_f32, dv.d, stream));
    if (st != DSA_OK) return st;
  }
  return DSA_OK;
}

size_t dsa_attn_bwd_workspace_bytes(const dsa_shape* shape, int32_t kmax) {
  Derived dv;
  if (derive(shape, &dv) != DSA_OK) return 0;
  if (kmax < 1 || kmax > dv.g.NB || !csc_fits(dv, kmax)) return 0;
  return bwd_layout(dv, kmax).total;
}

namespace {

enum BwdPhase { kPrepare = 1, kDkdv = 2, kDq = 4 };

// shared argument checks and workspace carving of the backward entry points
dsa_status bwd_common(int phases, const dsa_shape* shape, const void* Q, const void* K, const void* V, const void* O,
                      int32_t o_dtype, const void* dO, const float* LSE, const int32_t* idx, const int32_t* k,
                      int32_t kmax, float scale, int32_t out_dtype, void* dQ, void* dK, void* dV, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  Derived dv;
  dsa_status st = derive(shape, &dv);
  if (st != DSA_OK) return st;
  if ((phases & (kDkdv | kDq)) && out_dtype != DSA_F32 && out_dtype != DSA_BF16) return DSA_ERR_DTYPE;
  // O enters the backward only through D = rowsum(dO * O); a rounded O puts a
  // coherent error into every dS of its row, so only the float32 forward output
  // is accepted
  if ((phases & kPrepare) && o_dtype != DSA_F32) return DSA_ERR_DTYPE;
  if (kmax < 1 || kmax > dv.g.NB || !csc_fits(dv, kmax)) return DSA_ERR_K;
  if ((phases & (kDkdv | kDq)) && !scale_ok(scale)) return DSA_ERR_SHAPE;
  if (dv.BH == 0) return DSA_OK;
  if ((phases & kPrepare) && (!O || !dO || !idx || !k)) return DSA_ERR_NULL;
  if ((phases & kDkdv) && (!Q || !K || !V || !dO || !LSE || !dK || !dV)) return DSA_ERR_NULL;
  if ((phases & kDq) && (!Q || !K || !V || !dO || !LSE || !idx || !k || !dQ)) return DSA_ERR_NULL;
  const BwdLayout l = bwd_layout(dv, kmax);
  if (!workspace || workspace_bytes < l.total || ((uintptr_t)workspace & 255u)) return DSA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  BwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = static_cast<const float*>(O); a.dO = dO; a.LSE = LSE;
  a.idx = idx; a.kvec = k; a.kmax = kmax;
  a.scale = scale; a.c = scale * kLog2e; a.out_f32 = out_dtype == DSA_F32;
  a.dQ = dQ; a.dK = dK; a.dV = dV;
  a.Dvec = reinterpret_cast<float*>(ws + l.dvec);
  a.bitmap = reinterpret_cast<uint32_t*>(ws + l.bitmap);
  a.counts = reinterpret_cast<int32_t*>(ws + l.counts);
  a.offsets = reinterpret_cast<int32_t*>(ws + l.offsets);
  a.entries = reinterpret_cast<int32_t*>(ws + l.entries);
  a.order = dv.g.NB <= kOrderMaxNB ? reinterpret_cast<int32_t*>(ws + l.order) : nullptr;
  a.dO16 = dv.io_f32 ? nullptr : ws + l.do16;
  a.dmax = dv.io_f32 ? nullptr : reinterpret_cast<uint32_t*>(ws + l.dmax);
  a.dscale = dv.io_f32 ? nullptr : reinterpret_cast<float2*>(ws + l.dscale);
  a.vmax = dv.io_f32 ? nullptr : reinterpret_cast<uint32_t*>(ws + l.vmax);
  a.vscale = dv.io_f32 ? nullptr : reinterpret_cast<float2*>(ws + l.vscale);
  auto at = [&](size_t o) -> char* { return dv.io_f32 ? nullptr : ws + o; };
  a.dabs = reinterpret_cast<uint32_t*>(at(l.dabs));
  a.dabs_part = reinterpret_cast<uint32_t*>(at(l.dabs_part));
  a.Du = reinterpret_cast<float*>(at(l.du));
  a.Lse2 = reinterpret_cast<float*>(at(l.lse2));
  a.q16 = at(l.q16);
  a.qmax = reinterpret_cast<uint32_t*>(at(l.qmax));
  a.qscale = reinterpret_cast<float2*>(at(l.qscale));
  a.k16 = at(l.k16);
  a.kmaxp = reinterpret_cast<uint32_t*>(at(l.kmaxp));
  a.kscale = reinterpret_cast<float2*>(at(l.kscale));
  a.vmax_q = reinterpret_cast<uint32_t*>(at(l.vmax_q));
  a.vscale_q = reinterpret_cast<float2*>(at(l.vscale_q));
  a.words = l.words;
  a.g = dv.g; a.BH = dv.BH;
  hipError_t e = hipSuccess;
  if (phases & kPrepare) e = launch_bwd_prepare(a, dv.io_f32, dv.d, stream);
  if (e == hipSuccess && (phases & kDkdv)) e = launch_bwd_dkdv(a, dv.io_f32, dv.d, stream);
  if (e == hipSuccess && (phases & kDq)) e = launch_bwd_dq(a, dv.io_f32, dv.d, stream);
  return hip_status(e);
}

}  // namespace

dsa_status dsa_attn_bwd(const dsa_shape* shape, const void* Q, const void* K, const void* V, const void* O,
                        int32_t o_dtype, const void* dO, const float* LSE, const int32_t* idx, const int32_t* k,
                        int32_t kmax, float scale, int32_t out_dtype, void* dQ, void* dK, void* dV, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  return bwd_common(kPrepare | kDkdv | kDq, shape, Q, K, V, O, o_dtype, dO, LSE, idx, k, kmax, scale, out_dtype, dQ,
                    dK, dV, workspace, workspace_bytes, stream);
}

dsa_status dsa_attn_bwd_prepare(const dsa_shape* shape, const void* O, int32_t o_dtype, const void* dO,
                                const int32_t* idx, const int32_t* k, int32_t kmax, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return bwd_common(kPrepare, shape, nullptr, nullptr, nullptr, O, o_dtype, dO, nullptr, idx, k, kmax, 1.f,
                    DSA_F32, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream);
}

dsa_status dsa_attn_bwd_dkdv(const dsa_shape* shape, const void* Q, const void* K, const void* V, const void* dO,
                             const float* LSE, int32_t kmax, float scale, int32_t out_dtype, void* dK, void* dV,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_common(kDkdv, shape, Q, K, V, nullptr, DSA_F32, dO, LSE, nullptr, nullptr, kmax, scale, out_dtype,
                    nullptr, dK, dV, workspace, workspace_bytes, stream);
}

dsa_status dsa_attn_bwd_dq(const dsa_shape* shape, const void* Q, const void* K, const void* V, const void* dO,
                           const float* LSE, const int32_t* idx, const int32_t* k, int32_t kmax, float scale,
                           int32_t out_dtype, void* dQ, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_common(kDq, shape, Q, K, V, nullptr, DSA_F32, dO, LSE, idx, k, kmax, scale, out_dtype, dQ, nullptr,
                    nullptr, workspace, workspace_bytes, stream);
}

}  // extern "C"
