// Top-k key-block selection per query tile for gfx950 (DSV page, gist.science/
// ar/paper/2502.07590, section 3a: the predictor keeps only the small set worth
// attending to; section 3b: one set per tile of neighbouring queries).
//
// Row (b, h, tau) keeps block tau itself plus the k-1 other blocks with the
// largest scores; equal scores go to the lower block index; output ascending.
//
// One wave per row.  Scores become order-preserving 32-bit keys (canonical +0,
// NaN lowest).  The (k-1)-th largest key T is found by a 32-step bitwise search
// (each step counts the keys >= candidate: ballot + scalar popcount per register
// slot on rows of up to 1024 blocks, per-lane vector counts and one DPP wave sum on
// longer rows), then a single ascending sweep emits: own block, keys > T, and the
// lowest-index keys == T until k are taken.  Rows of up to 8192 blocks live in
// registers; rows of up to 16,384 blocks are formed once into LDS (one wave per
// work-group, at most 64 KB); longer rows are re-read from memory on each step
// (L2-resident).
//
// The fused variant (dsa_predict_select) computes each row's scores from the
// pooled features instead of reading a stored score matrix (bit-identical scores),
// so no NB x NB array is ever written: the term that grows quadratically with the
// sequence length (6.4 GB at 524,288 tokens) disappears.
#include "common.hpp"
#include "kernels.hpp"

#include <utility>

namespace dsa {

namespace {

constexpr int kWaves = 4;

// The lane id behind an empty asm: each phase derives its per-slot block ids from
// its own copy, so the compiler cannot keep one id register per slot alive from the
// loads through the search to the sweep (64-128 extra VGPRs on long rows).
__device__ __forceinline__ int fresh_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

// Sum of an int over the 64 lanes: DPP within each 16-lane row (quad swaps, then
// half-row and row mirrors leave every lane of a row holding the row's sum), then
// the four row sums on the scalar unit.  Needs all lanes active.
__device__ __forceinline__ int wave_sum(int v) {
  v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);    // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);    // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true);   // row_half_mirror
  v += __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true);   // row_mirror
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

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

  __device__ __forceinline__ uint32_t load(int i, int l) const {
    const int j = 64 * i + l;
    const uint32_t key = order_key(s[j < NB ? j : NB - 1]);   // clamped: no branch per slot
    return (j < NB && j != tau) ? key : 0u;
  }
  __device__ __forceinline__ uint32_t load(int i) const { return load(i, lane); }
  __device__ __forceinline__ void init() {
    if constexpr (SLOTS > 0) {
      const int l = fresh_lane(lane);
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) key[i] = load(i, l);
    }
  }
  // number of candidates with key >= t (t >= 1)
  // Short rows: ballot + scalar popcount per slot.  Long rows: per-lane counts on
  // the vector unit and one wave sum per call (with ballots the compiler keeps one
  // mask or partial count per slot live and spills them).
  __device__ __forceinline__ int count_ge(uint32_t t) const {
    int cnt = 0;
    if constexpr (SLOTS > 0 && SLOTS <= 16) {
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) cnt += __popcll(ballot(key[i] >= t));
      return cnt;
    } else if constexpr (SLOTS > 16) {
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) cnt += key[i] >= t ? 1 : 0;
    } else {
      for (int i = 0; i < nslots; ++i) cnt += load(i) >= t ? 1 : 0;
    }
    return wave_sum(cnt);
  }
  __device__ __forceinline__ uint32_t at(int i) const {
    if constexpr (SLOTS > 0) return key[i];
    else return load(i);
  }
};

// Rows of 8,193 to 16,384 blocks: keys in LDS, four slots of one lane per 16-byte
// word (slot 4q+e of lane l at word 64q+l, element e), so one pass of the search is
// one ds_read_b128 per four slots.  nslots is a multiple of 4; slots past the row
// hold 0 (not a candidate).
constexpr int kLdsMaxSlots = 256;             // 16,384 blocks, 64 KB of keys
struct LdsRow {
  const uint32_t* lk;
  int NB, tau, lane, nslots;
  __device__ __forceinline__ int count_ge(uint32_t t) const {
    const u32x4* p = reinterpret_cast<const u32x4*>(lk) + lane;
    int cnt = 0;
    for (int q = 0; q < nslots / 4; ++q) {
      const u32x4 v = p[64 * q];
      cnt += (v[0] >= t ? 1 : 0) + (v[1] >= t ? 1 : 0) + (v[2] >= t ? 1 : 0) + (v[3] >= t ? 1 : 0);
    }
    return wave_sum(cnt);
  }
  __device__ __forceinline__ uint32_t at(int i) const { return lk[((i >> 2) * 64 + lane) * 4 + (i & 3)]; }
};
template <typename KeyFn>
__device__ __forceinline__ void fill_lds(uint32_t* lk, int nslots, int lane, const KeyFn& key) {
  for (int q = 0; q < nslots / 4; ++q) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = key(4 * q + e, lane);
    reinterpret_cast<u32x4*>(lk)[64 * q + lane] = v;
  }
}
__host__ __device__ inline int lds_slots(int NB) { return ((NB + 63) / 64 + 3) & ~3; }

template <typename R>
__device__ __forceinline__ void sweep_slot(const R& rw, int i, int l, bool own_lane, uint32_t T, int kp,
                                           int need_eq, int& taken, int& eq_seen, int32_t* __restrict__ out,
                                           int kmax) {
  const int j = 64 * i + l;
  const uint32_t key = rw.at(i);
  // own block: a uniform slot test and one lane test (a per-slot compare of j with
  // tau would be merged with the one in init and keep a mask per slot alive)
  const bool own = (i == (rw.tau >> 6)) && own_lane;
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
  const int l = fresh_lane(rw.lane);
  const bool own_lane = l == (rw.tau & 63);
  if constexpr (SLOTS > 0) {
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) sweep_slot(rw, i, l, own_lane, T, kp, need_eq, taken, eq_seen, out, kmax);
  } else {
    for (int i = 0; i < rw.nslots; ++i) sweep_slot(rw, i, l, own_lane, T, kp, need_eq, taken, eq_seen, out, kmax);
  }
  for (int p = k + rw.lane; p < kmax; p += 64) out[p] = -1;
}

template <int SLOTS>
__global__ __launch_bounds__(64 * kWaves) void select_kernel(SelectArgs a) {
  const int lane = threadIdx.x & 63;
  const int rowid = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

// one wave per row, keys in LDS (rows of 8,193 to 16,384 blocks)
__global__ __launch_bounds__(64) void select_lds_kernel(SelectArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds_keys[];
  const int lane = threadIdx.x;
  const int rowid = blockIdx.x;
  const int NB = a.NB;
  const int bh = rowid / NB;
  const int tau = rowid - bh * NB;
  int k = a.kvec[bh];
  k = k < 1 ? 1 : (k > a.kmax ? a.kmax : k);
  int32_t* __restrict__ out = a.idx + (size_t)rowid * a.kmax;
  Row<0> src;
  src.s = a.S + (size_t)rowid * NB;
  src.NB = NB;
  src.tau = tau;
  src.lane = lane;
  const int nslots = lds_slots(NB);
  fill_lds(lds_keys, nslots, lane, [&](int i, int l) { return src.load(i, l); });
  __syncthreads();
  LdsRow rw{lds_keys, NB, tau, lane, nslots};
  select_row<0>(rw, k - 1, k, out, a.kmax);
}

hipError_t launch_sel_lds(const SelectArgs& a, hipStream_t s) {
  const size_t lds = (size_t)lds_slots(a.NB) * 64 * sizeof(uint32_t);
  hipLaunchKernelGGL(select_lds_kernel, dim3(a.BH * a.NB), dim3(64), lds, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fused scores + selection
// The scores of row (b,h,tau) computed on the fly from the pooled features, with
// the same float32 operations in the same order as the scores of dsa_predict
// (s = sum over c < RM of fma(Qbar[tau][c], Kbar[j][c], s), zero beyond r), so the
// selection is identical to dsa_predict + dsa_select without the NB x NB matrix.
// The four waves of a work-group share each Kbar row through the L1 cache.
// EXACT: r == RM (a multiple of 4): 16-byte loads of the Kbar rows, no per-term
// tests.  Otherwise r < RM or r % 4 != 0: scalar loads, terms c >= r are zero.
template <int RM, bool EXACT>
struct PooledRow {
  const float* __restrict__ kb;      // Kbar of the head, [NB][r]
  float qv[RM];                      // Qbar row (zero beyond r)
  int r, NB, tau;

  __device__ __forceinline__ uint32_t key(int i, int l) const {
    const int j = 64 * i + l;
    const float* kr = kb + (size_t)(j < NB ? j : NB - 1) * r;
    float s = 0.f;
    if constexpr (EXACT) {
#pragma unroll
      for (int c = 0; c < RM; c += 4) {
        const float4 v = *reinterpret_cast<const float4*>(kr + c);
        s = fmaf(qv[c], v.x, s);
        s = fmaf(qv[c + 1], v.y, s);
        s = fmaf(qv[c + 2], v.z, s);
        s = fmaf(qv[c + 3], v.w, s);
      }
    } else {
#pragma unroll
      for (int c = 0; c < RM; ++c) s = fmaf(qv[c], c < r ? kr[c] : 0.f, s);
    }
    return (j < NB && j != tau) ? order_key(s) : 0u;
  }
  // all slots of a register-held row, expanded at compile time (a loop this long is
  // not unrolled completely, and the key array would then live in scratch memory)
  template <int... I>
  __device__ __forceinline__ void fill_seq(uint32_t* key, int l, std::integer_sequence<int, I...>) const {
    ((key[I] = this->key(I, l)), ...);
  }
  template <int SLOTS>
  __device__ __forceinline__ void fill(uint32_t (&key)[SLOTS], int l) const {
    fill_seq(key, l, std::make_integer_sequence<int, SLOTS>{});
  }
};

// rows longer than 8192 blocks: scores recomputed on every pass
template <int RM, bool EXACT>
struct RecomputedRow {
  PooledRow<RM, EXACT> p;
  int tau, lane, nslots;
  __device__ __forceinline__ int count_ge(uint32_t t) const {
    int cnt = 0;
    for (int i = 0; i < nslots; ++i) cnt += p.key(i, lane) >= t ? 1 : 0;
    return wave_sum(cnt);
  }
  __device__ __forceinline__ uint32_t at(int i) const { return p.key(i, lane); }
};

template <int SLOTS, int RM, bool EXACT>
__global__ __launch_bounds__(64 * kWaves) void fused_select_kernel(FusedSelectArgs a) {
  const int lane = threadIdx.x & 63;
  const int rowid = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (rowid >= a.BH * a.NB) return;                     // whole wave exits together
  const int NB = a.NB;
  const int bh = rowid / NB;
  const int tau = rowid - bh * NB;
  int k = a.kvec[bh];
  k = k < 1 ? 1 : (k > a.kmax ? a.kmax : k);
  int32_t* __restrict__ out = a.idx + (size_t)rowid * a.kmax;

  PooledRow<RM, EXACT> p;
  p.kb = a.Kbar + (size_t)bh * NB * a.r;
  // the Qbar row is the same for all lanes; read through a lane-dependent-looking
  // address so it lands in VGPRs (up to 64 values would crowd the SGPRs)
  const float* qb = a.Qbar + (size_t)rowid * a.r + fresh_lane(0);
#pragma unroll
  for (int c = 0; c < RM; ++c) p.qv[c] = c < a.r ? qb[c] : 0.f;
  p.r = a.r;
  p.NB = NB;
  p.tau = tau;

  if constexpr (SLOTS > 0) {
    Row<SLOTS> rw;                 // keys only: the pooled row's scores, computed once
    rw.s = nullptr;
    rw.NB = NB;
    rw.tau = tau;
    rw.lane = lane;
    rw.nslots = SLOTS;
    p.fill(rw.key, fresh_lane(lane));
    select_row<SLOTS>(rw, k - 1, k, out, a.kmax);
  } else {
    RecomputedRow<RM, EXACT> rw;
    rw.p = p;
    rw.tau = tau;
    rw.lane = lane;
    rw.nslots = (NB + 63) / 64;
    select_row<0>(rw, k - 1, k, out, a.kmax);
  }
}

// one wave per row, keys formed once into LDS (rows of 8,193 to 16,384 blocks)
template <int RM, bool EXACT>
__global__ __launch_bounds__(64) void fused_select_lds_kernel(FusedSelectArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds_keys[];
  const int lane = threadIdx.x;
  const int rowid = blockIdx.x;
  const int NB = a.NB;
  const int bh = rowid / NB;
  const int tau = rowid - bh * NB;
  int k = a.kvec[bh];
  k = k < 1 ? 1 : (k > a.kmax ? a.kmax : k);
  int32_t* __restrict__ out = a.idx + (size_t)rowid * a.kmax;
  PooledRow<RM, EXACT> p;
  p.kb = a.Kbar + (size_t)bh * NB * a.r;
  const float* qb = a.Qbar + (size_t)rowid * a.r + fresh_lane(0);
#pragma unroll
  for (int c = 0; c < RM; ++c) p.qv[c] = c < a.r ? qb[c] : 0.f;
  p.r = a.r;
  p.NB = NB;
  p.tau = tau;
  const int nslots = lds_slots(NB);
  fill_lds(lds_keys, nslots, lane, [&](int i, int l) { return p.key(i, l); });
  __syncthreads();
  LdsRow rw{lds_keys, NB, tau, lane, nslots};
  select_row<0>(rw, k - 1, k, out, a.kmax);
}

template <int RM, bool EXACT>
hipError_t launch_fsel_lds(const FusedSelectArgs& a, hipStream_t s) {
  const size_t lds = (size_t)lds_slots(a.NB) * 64 * sizeof(uint32_t);
  hipLaunchKernelGGL((fused_select_lds_kernel<RM, EXACT>), dim3(a.BH * a.NB), dim3(64), lds, s, a);
  return hipGetLastError();
}

template <int SLOTS, int RM, bool EXACT>
hipError_t launch_fsel(const FusedSelectArgs& a, hipStream_t s) {
  const int rows = a.BH * a.NB;
  const int grid = (rows + kWaves - 1) / kWaves;
  hipLaunchKernelGGL((fused_select_kernel<SLOTS, RM, EXACT>), dim3(grid), dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}
template <int RM, bool EXACT>
hipError_t launch_fsel_rm(const FusedSelectArgs& a, hipStream_t s) {
  const int slots = (a.NB + 63) / 64;
  if (slots <= 1) return launch_fsel<1, RM, EXACT>(a, s);
  if (slots <= 2) return launch_fsel<2, RM, EXACT>(a, s);
  if (slots <= 4) return launch_fsel<4, RM, EXACT>(a, s);
  if (slots <= 8) return launch_fsel<8, RM, EXACT>(a, s);
  if (slots <= 16) return launch_fsel<16, RM, EXACT>(a, s);
  if (slots <= 32) return launch_fsel<32, RM, EXACT>(a, s);
  if (slots <= 64) return launch_fsel<64, RM, EXACT>(a, s);
  if (slots <= 128) return launch_fsel<128, RM, EXACT>(a, s);
  if (slots <= kLdsMaxSlots) return launch_fsel_lds<RM, EXACT>(a, s);
  return launch_fsel<0, RM, EXACT>(a, s);
}

}  // namespace

hipError_t launch_fused_select(const FusedSelectArgs& a, hipStream_t s) {
  const bool aligned = (reinterpret_cast<uintptr_t>(a.Kbar) & 15) == 0;   // 16-byte row loads
  if (aligned && a.r == 16) return launch_fsel_rm<16, true>(a, s);
  if (aligned && a.r == 32) return launch_fsel_rm<32, true>(a, s);
  return launch_fsel_rm<64, false>(a, s);                  // any other rank up to 64
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
  if (slots <= kLdsMaxSlots) return launch_sel_lds(a, s);
  return launch_sel<0>(a, s);
}

}  // namespace dsa
