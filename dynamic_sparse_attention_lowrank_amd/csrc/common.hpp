// Shared device helpers for the gfx950 (MI355X) kernels of libdsa.
//
// Matrix-core fragments.  Every contraction in this library is issued as a
// sequence of 32x32 output tiles with a reduction step of 16:
//   bf16: one v_mfma_f32_32x32x16_bf16 per step;
//   fp32: eight v_mfma_f32_32x32x2_f32 per step (same operand registers, one
//         element pair per instruction), so one code path serves both types.
// Operand layout (checked on the hardware): for A (32 x 16, M x K) lane l holds
// row l%32 and reduction elements 8*(l/32) .. 8*(l/32)+7; for B (16 x 32) lane l
// holds column l%32 and the same 8 reduction elements.  The 32x32 fp32 result
// gives lane l column l%32 and rows {8g + 4*(l/32) + i : g < 4, i < 4} in
// registers 4g + i.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// element-type traits
// ---------------------------------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<bf16> {
  typedef bf16x8 frag;                 // 8 reduction elements = 16 bytes
  static constexpr int kChunkElems = 8;  // elements per 16-byte chunk
  static constexpr int kFragChunks = 1;  // 16-byte chunks per fragment
};
template <> struct Elem<f16> {
  typedef f16x8 frag;
  static constexpr int kChunkElems = 8;
  static constexpr int kFragChunks = 1;
};
template <> struct Elem<float> {
  typedef f32x8 frag;                  // 8 reduction elements = 32 bytes
  static constexpr int kChunkElems = 4;
  static constexpr int kFragChunks = 2;
};

// acc += A * B over one reduction step of 16.
__device__ __forceinline__ f32x16 mma_step(bf16x8 a, bf16x8 b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_step(f16x8 a, f16x8 b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_step(f32x8 a, f32x8 b, f32x16 acc) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], acc, 0, 0, 0);
  return acc;
}

// fragment <-> raw 16-byte chunks
__device__ __forceinline__ bf16x8 frag_from_chunks(const u32x4* c, bf16*) {
  return __builtin_bit_cast(bf16x8, c[0]);
}
__device__ __forceinline__ f16x8 frag_from_chunks(const u32x4* c, f16*) {
  return __builtin_bit_cast(f16x8, c[0]);
}
__device__ __forceinline__ f32x8 frag_from_chunks(const u32x4* c, float*) {
  f32x4 lo = __builtin_bit_cast(f32x4, c[0]);
  f32x4 hi = __builtin_bit_cast(f32x4, c[1]);
  f32x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// eight fp32 values -> fragment of the element type (round to nearest even for bf16)
__device__ __forceinline__ bf16x8 to_frag(const float* v, bf16*) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)v[e];
  return r;
}
__device__ __forceinline__ f16x8 to_frag(const float* v, f16*) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (f16)v[e];
  return r;
}
__device__ __forceinline__ f32x8 to_frag(const float* v, float*) {
  f32x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = v[e];
  return r;
}

// An fp32 operand computed inside a kernel (probabilities, dS) as a bf16 pair
// hi + lo with hi = bf16(v), lo = bf16(v - hi): the pair carries about 16
// significant bits, so contractions issued twice (hi, then lo) keep fp32-level
// accuracy without relying on the range of any other 16-bit format.  For fp32
// operands there is nothing to split (lo is unused).
struct SplitBF16 {
  bf16x8 hi, lo;
};
__device__ __forceinline__ void to_split(const float* v, SplitBF16& s) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bf16 h = (bf16)v[e];
    s.hi[e] = h;
    s.lo[e] = (bf16)(v[e] - (float)h);
  }
}
struct SplitF32 {
  f32x8 hi;
};
__device__ __forceinline__ void to_split(const float* v, SplitF32& s) {
#pragma unroll
  for (int e = 0; e < 8; ++e) s.hi[e] = v[e];
}
template <typename T> struct SplitOf;
template <> struct SplitOf<bf16> { typedef SplitBF16 type; };
template <> struct SplitOf<float> { typedef SplitF32 type; };

// acc += A * (hi + lo)   /   acc += (hi + lo) * B
__device__ __forceinline__ f32x16 mma_split_b(bf16x8 a, const SplitBF16& b, f32x16 acc) {
  acc = mma_step(a, b.hi, acc);
  return mma_step(a, b.lo, acc);
}
__device__ __forceinline__ f32x16 mma_split_b(f32x8 a, const SplitF32& b, f32x16 acc) { return mma_step(a, b.hi, acc); }
__device__ __forceinline__ f32x16 mma_split_a(const SplitBF16& a, bf16x8 b, f32x16 acc) {
  acc = mma_step(a.hi, b, acc);
  return mma_step(a.lo, b, acc);
}
__device__ __forceinline__ f32x16 mma_split_a(const SplitF32& a, f32x8 b, f32x16 acc) { return mma_step(a.hi, b, acc); }

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

// ---------------------------------------------------------------------------
// tile geometry: token offsets of the members of a tile, relative to its corner
// ---------------------------------------------------------------------------
struct Geo {
  int Lt, Lh, Lw;      // latent extents
  int tt, th, tw;      // tile extents
  int gt, gh, gw;      // tile grid extents
  int N, T, NB;        // tokens, tokens per tile, tiles
  // multiply-high reciprocals ceil(2^32 / d) of gw, gw*gh, tw, tw*th (0 for d = 1):
  // floor(n / d) = mulhi(n, m) exactly when n * (d - 1) < 2^32, which holds for
  // member indices (n, d <= 64) always and for tile indices when NB <= 65535
  // (fast_tiles); otherwise tile_base divides.
  uint32_t m_gw, m_gwgh, m_tw, m_twth;
  int fast_tiles;
};

__device__ __forceinline__ int div_rcp(int n, uint32_t m) {
  return m == 0 ? n : (int)__umulhi((uint32_t)n, m);
}

// first token of tile j (its (t, y, x) corner)
__device__ __forceinline__ int tile_base(const Geo& g, int j) {
  int jx, jy, jt;
  if (g.fast_tiles) {
    const int q = div_rcp(j, g.m_gw);
    jt = div_rcp(j, g.m_gwgh);
    jx = j - q * g.gw;
    jy = q - jt * g.gh;
  } else {
    jx = j % g.gw;
    jy = (j / g.gw) % g.gh;
    jt = j / (g.gw * g.gh);
  }
  return ((jt * g.tt) * g.Lh + jy * g.th) * g.Lw + jx * g.tw;
}
// offset of the i-th member (ascending token order, 0 <= i < T <= 64) from the tile corner
__device__ __forceinline__ int member_offset(const Geo& g, int i) {
  const int q = div_rcp(i, g.m_tw);
  const int dt = div_rcp(i, g.m_twth);
  const int dx = i - q * g.tw;
  const int dy = q - dt * g.th;
  return (dt * g.Lh + dy) * g.Lw + dx;
}

// ---------------------------------------------------------------------------
// work-group placement: the attention kernels take work-group ids in their
// natural order, (head, tile) row-major.  The hardware hands consecutive ids to
// the 8 XCDs in turn, so at any moment all XCDs work on neighbouring tiles of the
// same one or two heads and the gathered K/V (or Q/dO) blocks of those tiles
// stay in the 256 MB memory-attached cache.  Giving each XCD a contiguous range
// of (head, tile) instead (8 heads in flight) was measured slower at every size:
// forward / dK,dV / dQ -1 % / -1 % / -1 % at 32K tokens, -17 % / -27 % / -30 % on
// the 55K dynamic workload, -3 % / -10 % / -15 % at 524K, where one head's blocks
// alone fill most of that cache.
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// wave helpers (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}
__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }
// max / sum over the lane pair (l, l^32) with one v_permlane32_swap (no LDS
// round trip).  Both lanes of a pair combine (low lane, high lane) in the same
// order, so they get bit-identical results.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A tile's list of kept block ids, read by the whole wave in order: 64 entries
// per vector load (lane i holds entry base + i) and handed out one at a time by
// v_readlane, so the block loop never waits on a scalar memory load.  Entries
// outside [0, nb) are skipped.  Must be used with the full wave active.
struct IdList {
  const int* p;
  int n, nb, base, val;
  uint64_t mask;                              // entries of the current 64 not yet handed out
  __device__ __forceinline__ void fill(int lane) {
    val = base + lane < n ? p[base + lane] : -1;
    mask = ballot((unsigned)val < (unsigned)nb);
  }
  __device__ __forceinline__ void init(const int* list, int count, int nblocks, int lane) {
    p = list;
    n = count;
    nb = nblocks;
    base = 0;
    fill(lane);
  }
  // next valid id, or -1 at the end (wave-uniform)
  __device__ __forceinline__ int next(int lane) {
    while (mask == 0) {
      base += 64;
      if (base >= n) return -1;
      fill(lane);
    }
    const int b = __builtin_ctzll(mask);
    mask &= mask - 1;
    return __builtin_amdgcn_readlane(val, b);
  }
};

// An IdList of tile ids that also hands out each entry's tile base (its first
// token, tile_base), computed per lane when the entries are read (on the vector
// unit, once per 64 entries), so that requesting a tile needs no scalar address
// arithmetic per block.
struct TileList {
  IdList ids;
  const Geo* g;
  int tb;                                     // tile base of this lane's entry
  int last_base;                              // tile base of the id next() returned last
  __device__ __forceinline__ void bases() {
    tb = (unsigned)ids.val < (unsigned)ids.nb ? tile_base(*g, ids.val) : 0;
  }
  __device__ __forceinline__ void init(const int* list, int count, const Geo& geo, int lane) {
    g = &geo;
    last_base = 0;
    ids.init(list, count, geo.NB, lane);
    bases();
  }
  // next valid id (and last_base), or -1 at the end (wave-uniform)
  __device__ __forceinline__ int next(int lane) {
    while (ids.mask == 0) {
      ids.base += 64;
      if (ids.base >= ids.n) return -1;
      ids.fill(lane);
      bases();
    }
    const int b = __builtin_ctzll(ids.mask);
    ids.mask &= ids.mask - 1;
    last_base = __builtin_amdgcn_readlane(tb, b);
    return __builtin_amdgcn_readlane(ids.val, b);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// position of key kk (0..15) inside a 16-key group of a transposed operand in LDS:
// swaps bits 2 and 3, so that the registers of a 32x32 result, read in order,
// form the B operand of the next contraction without any lane exchange.
__device__ __forceinline__ int perm16(int kk) {
  return (kk & 3) | (((kk >> 2) & 1) << 3) | (((kk >> 3) & 1) << 2);
}

}  // namespace dsa
