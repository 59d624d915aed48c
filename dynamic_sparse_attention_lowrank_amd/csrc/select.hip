// Top-k key-block selection per query tile for gfx950 (DSV page, gist.science/
// ar/paper/2502.07590, section 3a: the predictor keeps only the small set worth
// attending to; section 3b: one set per tile of neighbouring queries).
//
// Row (b, h, tau) keeps block tau itself plus the k-1 other blocks with the
// largest scores; equal scores go to the lower block index; output ascending.
//
// One wave per row.  Scores become order-preserving 32-bit keys (canonical +0,
// NaN lowest).  The (k-1)-th largest key T is found by a 32-step bitwise search
// (each step counts keys >= candidate with one compare + ballot + popcount per
// register slot, so the counting runs on the scalar unit), then a single
// ascending sweep emits: own block, keys > T, and the lowest-index keys == T until
// k are taken.  Rows of up to 8192 blocks live in registers; longer rows are
// re-read from memory on each step (L2-resident).
//
// The fused variant (dsa_predict_select) computes each row's scores from the
// pooled features instead of reading a stored score matrix (bit-identical scores),
// so no NB x NB array is ever written: the term that grows quadratically with the
// sequence length (6.4 GB at 524,288 tokens) disappears.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (x != x) return 1u;                 // NaN ranks below every number
  if ((u << 1) == 0u) u = 0u;            // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // >= 0x007fffff for any number
}

// Per-lane view of one row: element j = 64*i + lane sits in slot i.  A key of 0
// marks "not a candidate" (padding or the own block); candidates have key >= 1.
// SLOTS > 0: keys held in registers (loops fully unrolled so they stay there).
// SLOTS == 0: keys recomputed from the row in memory on every pass.
template <int SLOTS>
struct Row {
  const float* __restrict__ s;
  int NB, tau, lane, nslots;
  uint32_t key[SLOTS > 0 ? SLOTS : 1];

  __device__ __forceinline__ uint32_t load(int i) const {
    const int j = 64 * i + lane;
    return (j < NB && j != tau) ? order_key(s[j]) : 0u;
  }
  __device__ __forceinline__ void init() {
    if constexpr (SLOTS > 0) {
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) key[i] = load(i);
    }
  }
  // number of candidates with key >= t (t >= 1)
  __device__ __forceinline__ int count_ge(uint32_t t) const {
    int cnt = 0;
    if constexpr (SLOTS > 0) {
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) cnt += __popcll(ballot(key[i] >= t));
    } else {
      for (int i = 0; i < nslots; ++i) cnt += __popcll(ballot(load(i) >= t));
    }
    return cnt;
  }
  __device__ __forceinline__ uint32_t at(int i) const {
    if constexpr (SLOTS > 0) return key[i];
    else return load(i);
  }
};

template <typename R>
__device__ __forceinline__ void sweep_slot(const R& rw, int i, uint32_t T, int kp, int need_eq,
                                           int& taken, int& eq_seen, int32_t* __restrict__ out, int kmax) {
  const int j = 64 * i + rw.lane;
  const uint32_t key = rw.at(i);
  const bool own = (j == rw.tau);
  const bool eq = kp > 0 && key == T;                  // T >= 1 whenever kp > 0
  const uint64_t eqm = ballot(eq);
  const bool pick = own || (kp > 0 && key > T) || (eq && eq_seen + lanes_below(eqm) < need_eq);
  const uint64_t pm = ballot(pick);
  const int pos = taken + lanes_below(pm);
  if (pick && pos < kmax) out[pos] = j;
  taken += __popcll(pm);
  eq_seen += __popcll(eqm);
}

// The kept blocks of one row: the kp-th largest key T by a bitwise search, then one
// ascending sweep (own block, keys > T, lowest-index keys == T), -1 padding.
template <int SLOTS, typename R>
__device__ __forceinline__ void select_row(const R& rw, int kp, int k, int32_t* __restrict__ out, int kmax) {
  // T = the kp-th largest key: the largest t with #{key >= t} >= kp
  uint32_t T = 0xffffffffu;
  int need_eq = 0;
  if (kp > 0) {
    T = 0u;
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = T | (1u << b);
      if (rw.count_ge(cand) >= kp) T = cand;
    }
    const int n_gt = T == 0xffffffffu ? 0 : rw.count_ge(T + 1u);
    need_eq = kp - n_gt;
  }

  int taken = 0, eq_seen = 0;
  if constexpr (SLOTS > 0) {
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) sweep_slot(rw, i, T, kp, need_eq, taken, eq_seen, out, kmax);
  } else {
    for (int i = 0; i < rw.nslots; ++i) sweep_slot(rw, i, T, kp, need_eq, taken, eq_seen, out, kmax);
  }
  for (int p = k + rw.lane; p < kmax; p += 64) out[p] = -1;
}

template <int SLOTS>
__global__ __launch_bounds__(64 * kWaves) void select_kernel(SelectArgs a) {
  const int lane = threadIdx.x & 63;
  const int rowid = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (rowid >= a.BH * a.NB) return;                     // whole wave exits together
  const int NB = a.NB;
  const int bh = rowid / NB;
  const int tau = rowid - bh * NB;
  int k = a.kvec[bh];
  k = k < 1 ? 1 : (k > a.kmax ? a.kmax : k);
  const int kp = k - 1;                                 // blocks to pick besides tau
  int32_t* __restrict__ out = a.idx + (size_t)rowid * a.kmax;

  Row<SLOTS> rw;
  rw.s = a.S + (size_t)rowid * NB;
  rw.NB = NB;
  rw.tau = tau;
  rw.lane = lane;
  rw.nslots = (NB + 63) / 64;
  rw.init();

  select_row<SLOTS>(rw, kp, k, out, a.kmax);
}

template <int SLOTS>
hipError_t launch_sel(const SelectArgs& a, hipStream_t s) {
  const int rows = a.BH * a.NB;
  const int grid = (rows + kWaves - 1) / kWaves;
  hipLaunchKernelGGL((select_kernel<SLOTS>), dim3(grid), dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fused scores + selection
// The scores of row (b,h,tau) computed on the fly from the pooled features, with
// the same float32 operations in the same order as the scores of dsa_predict
// (s = sum over c < RM of fma(Qbar[tau][c], Kbar[j][c], s), zero beyond r), so the
// selection is identical to dsa_predict + dsa_select without the NB x NB matrix.
// The four waves of a work-group share each Kbar row through the L1 cache.
template <int SLOTS, int RM>
struct FusedRow {
  const float* __restrict__ kb;      // Kbar of the head, [NB][r]
  float qv[RM];                      // Qbar row (zero beyond r)
  int r, NB, tau, lane, nslots;
  uint32_t key[SLOTS > 0 ? SLOTS : 1];

  __device__ __forceinline__ uint32_t load(int i) const {
    const int j = 64 * i + lane;
    if (j >= NB || j == tau) return 0u;
    const float* kr = kb + (size_t)j * r;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < RM; ++c) s = fmaf(qv[c], c < r ? kr[c] : 0.f, s);
    return order_key(s);
  }
  __device__ __forceinline__ void init() {
    if constexpr (SLOTS > 0) {
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) key[i] = load(i);
    }
  }
  __device__ __forceinline__ int count_ge(uint32_t t) const {
    int cnt = 0;
    if constexpr (SLOTS > 0) {
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) cnt += __popcll(ballot(key[i] >= t));
    } else {
      for (int i = 0; i < nslots; ++i) cnt += __popcll(ballot(load(i) >= t));
    }
    return cnt;
  }
  __device__ __forceinline__ uint32_t at(int i) const {
    if constexpr (SLOTS > 0) return key[i];
    else return load(i);
  }
};

template <int SLOTS, int RM>
__global__ __launch_bounds__(64 * kWaves) void fused_select_kernel(FusedSelectArgs a) {
  const int lane = threadIdx.x & 63;
  const int rowid = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (rowid >= a.BH * a.NB) return;                     // whole wave exits together
  const int NB = a.NB;
  const int bh = rowid / NB;
  const int tau = rowid - bh * NB;
  int k = a.kvec[bh];
  k = k < 1 ? 1 : (k > a.kmax ? a.kmax : k);
  int32_t* __restrict__ out = a.idx + (size_t)rowid * a.kmax;

  FusedRow<SLOTS, RM> rw;
  rw.kb = a.Kbar + (size_t)bh * NB * a.r;
  const float* qb = a.Qbar + (size_t)rowid * a.r;
#pragma unroll
  for (int c = 0; c < RM; ++c) rw.qv[c] = c < a.r ? qb[c] : 0.f;
  rw.r = a.r;
  rw.NB = NB;
  rw.tau = tau;
  rw.lane = lane;
  rw.nslots = (NB + 63) / 64;
  rw.init();
  select_row<SLOTS>(rw, k - 1, k, out, a.kmax);
}

template <int SLOTS, int RM>
hipError_t launch_fsel(const FusedSelectArgs& a, hipStream_t s) {
  const int rows = a.BH * a.NB;
  const int grid = (rows + kWaves - 1) / kWaves;
  hipLaunchKernelGGL((fused_select_kernel<SLOTS, RM>), dim3(grid), dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}
template <int RM>
hipError_t launch_fsel_rm(const FusedSelectArgs& a, hipStream_t s) {
  const int slots = (a.NB + 63) / 64;
  if (slots <= 1) return launch_fsel<1, RM>(a, s);
  if (slots <= 2) return launch_fsel<2, RM>(a, s);
  if (slots <= 4) return launch_fsel<4, RM>(a, s);
  if (slots <= 8) return launch_fsel<8, RM>(a, s);
  if (slots <= 16) return launch_fsel<16, RM>(a, s);
  if (slots <= 32) return launch_fsel<32, RM>(a, s);
  if (slots <= 64) return launch_fsel<64, RM>(a, s);
  if (slots <= 128) return launch_fsel<128, RM>(a, s);
  return launch_fsel<0, RM>(a, s);
}

}  // namespace

hipError_t launch_fused_select(const FusedSelectArgs& a, hipStream_t s) {
  if (a.r <= 16) return launch_fsel_rm<16>(a, s);
  if (a.r <= 32) return launch_fsel_rm<32>(a, s);
  return launch_fsel_rm<64>(a, s);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const int slots = (a.NB + 63) / 64;
  if (slots <= 1) return launch_sel<1>(a, s);
  if (slots <= 2) return launch_sel<2>(a, s);
  if (slots <= 4) return launch_sel<4>(a, s);
  if (slots <= 8) return launch_sel<8>(a, s);
  if (slots <= 16) return launch_sel<16>(a, s);
  if (slots <= 32) return launch_sel<32>(a, s);
  if (slots <= 64) return launch_sel<64>(a, s);
  if (slots <= 128) return launch_sel<128>(a, s);
  return launch_sel<0>(a, s);
}

}  // namespace dsa
