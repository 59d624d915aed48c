// LDS staging of 64-token tiles for the attention kernels (gfx950).
//
// Tiles of 64 tokens x D elements.  Two LDS layouts are used:
//
//  * row-major  [64][D]: a token row is D*sizeof(T) bytes = CPR 16-byte chunks;
//    chunk c of row r sits at slot c ^ row_swz(r) (a bijection of r mod
//    min(CPR,16)), so both the row-wise operand reads and the transposing reads
//    of 4-row groups are free of bank conflicts;
//  * transposed [D][64]: row d holds element d of all 64 tokens, with token
//    position p = 16*G + perm16(k) for token 16*G + k (see common.hpp), so that
//    one 16-byte read gives a lane the 8 tokens its MFMA operand needs.  Chunk c
//    of row d sits at c ^ ((d ^ (d >> log2 TR)) mod TR), which keeps both the
//    transposing writes and the operand reads spread over the banks.
//
// Global loads are 16-byte chunks.  A "row item" is one chunk of one token row
// (consecutive threads take consecutive chunks of a row).  A "group item" is one
// chunk column of the 8 tokens in one 8-position group of the transposed layout;
// it is written both transposed and, when needed, row-major.
#pragma once

#include "common.hpp"

namespace dsa {

constexpr int kTileThreads = 128;

template <typename T, int D>
struct TileCfg {
  static constexpr int kCE = Elem<T>::kChunkElems;            // elements per 16-byte chunk
  static constexpr int kFC = Elem<T>::kFragChunks;            // chunks per MFMA fragment
  static constexpr int kCPR = D / kCE;                        // chunks per token row
  static constexpr int kRowPer = 64 * kCPR / kTileThreads;    // row items per thread
  static constexpr int kGItems = 8 * kCPR;                    // group items per tile
  static constexpr int kGPer = (kGItems + kTileThreads - 1) / kTileThreads;
  static constexpr int kTR = 64 * (int)sizeof(T) / 16;        // chunks per transposed row
  static constexpr int kTLog = kTR == 8 ? 3 : 4;
  static constexpr int kRSw = kCPR < 16 ? kCPR : 16;
  static constexpr int kSteps = D / 16;                       // reduction steps over d
  static constexpr int kDTiles = D / 32;                      // 32-wide tiles over d
  static constexpr int kRowChunks = 64 * kCPR;                // LDS chunks of a row-major tile
  static constexpr int kTrChunks = D * kTR;                   // LDS chunks of a transposed tile
};

// Row swizzle: a bijection of r mod RSw whose bits 1-2 are r mod 4 (bit 0: bit 2 of
// r, bit 3: bit 3 of r).  16 consecutive rows reading one chunk column hit 16
// distinct slots, and 4 consecutive rows (starting at a multiple of 4) reading a
// 32-byte column pair hit 8 distinct slots -- both conflict-free at d = 128.
template <typename T, int D>
__device__ __forceinline__ int row_swz(int r) {
  return (((r & 3) << 1) | ((r >> 2) & 1) | (r & 8)) & (TileCfg<T, D>::kRSw - 1);
}
template <typename T, int D>
__device__ __forceinline__ int row_slot(int r, int c) {
  using C = TileCfg<T, D>;
  return r * C::kCPR + (c ^ row_swz<T, D>(r));
}
template <typename T, int D>
__device__ __forceinline__ int tr_slot(int d, int c) {
  using C = TileCfg<T, D>;
  return d * C::kTR + (c ^ ((d ^ (d >> C::kTLog)) & (C::kTR - 1)));
}
// token position (0..63) stored at place e of 8-position group kg
__device__ __forceinline__ int group_row(int kg, int e) { return 16 * (kg >> 1) + perm16(8 * (kg & 1) + e); }

// --- A/B operand fragments from LDS -----------------------------------------
// row-major tile: row r, reduction step s, lane half h -> elements 16s+8h..+7
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::frag frag_row(const u32x4* lds, int r, int s, int h) {
  using C = TileCfg<T, D>;
  u32x4 ch[C::kFC];
#pragma unroll
  for (int p = 0; p < C::kFC; ++p) ch[p] = lds[row_slot<T, D>(r, (2 * s + h) * C::kFC + p)];
  return frag_from_chunks(ch, (T*)nullptr);
}
// transposed tile: row d, token step s (16 tokens), lane half h -> positions 16s+8h..+7
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::frag frag_tr(const u32x4* lds, int d, int s, int h) {
  using C = TileCfg<T, D>;
  u32x4 ch[C::kFC];
#pragma unroll
  for (int p = 0; p < C::kFC; ++p) ch[p] = lds[tr_slot<T, D>(d, (2 * s + h) * C::kFC + p)];
  return frag_from_chunks(ch, (T*)nullptr);
}
// one token row straight from global memory as B operand fragments (row tok, elements 16s+8h..)
template <typename T, int D>
__device__ __forceinline__ void load_row_frags(typename Elem<T>::frag* f, const T* __restrict__ row, bool ok, int h) {
  using C = TileCfg<T, D>;
#pragma unroll
  for (int s = 0; s < C::kSteps; ++s) {
    u32x4 ch[C::kFC];
#pragma unroll
    for (int p = 0; p < C::kFC; ++p)
      ch[p] = ok ? *reinterpret_cast<const u32x4*>(row + 16 * s + 8 * h + p * C::kCE) : u32x4{0, 0, 0, 0};
    f[s] = frag_from_chunks(ch, (T*)nullptr);
  }
}

// Transposed operand fragment from a row-major tile whose rows are the reduction
// index (e.g. queries): lane l gets column col0 + l%16 (col0 = 32t + 16*((l%32)/16))
// and the 8 rows {16s+4h+0..3, 16s+8+4h+0..3} -- the perm16 order in which the
// P^T / dS^T fragments taken from a 32x32 result hold their reduction index.
// 16-bit types use gfx950's transposing LDS read (ds_read_b64_tr_b16): within
// each 16-lane group, lane j points at row r0 + j/4, columns col0 + 4*(j%4)..+3,
// and lane i receives column col0 + i of rows r0..r0+3.  fp32 reads element-wise.
template <typename T, int D>
__device__ __forceinline__ bf16x8 frag_tr_rows(const u32x4* lds, int col0, int s, int h, int i, bf16*) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const int col = col0 + 4 * (i & 3);
  const int chunk = col >> 3, byte = (col & 7) * 2;
  const int r1 = 16 * s + 4 * h + (i >> 2), r2 = r1 + 8;
  const char* base = reinterpret_cast<const char*>(lds);
  const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (bf16x4 __attribute__((address_space(3)))*)(base + row_slot<T, D>(r1, chunk) * 16 + byte));
  const bf16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (bf16x4 __attribute__((address_space(3)))*)(base + row_slot<T, D>(r2, chunk) * 16 + byte));
  return bf16x8{v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
}
template <typename T, int D>
__device__ __forceinline__ f16x8 frag_tr_rows(const u32x4* lds, int col0, int s, int h, int i, f16*) {
  typedef __fp16 h4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  const int col = col0 + 4 * (i & 3);
  const int chunk = col >> 3, byte = (col & 7) * 2;
  const int r1 = 16 * s + 4 * h + (i >> 2), r2 = r1 + 8;
  const char* base = reinterpret_cast<const char*>(lds);
  const f16x4 v1 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (h4 __attribute__((address_space(3)))*)(base + row_slot<T, D>(r1, chunk) * 16 + byte)));
  const f16x4 v2 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (h4 __attribute__((address_space(3)))*)(base + row_slot<T, D>(r2, chunk) * 16 + byte)));
  return f16x8{v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
}
template <typename T, int D>
__device__ __forceinline__ f32x8 frag_tr_rows(const u32x4* lds, int col0, int s, int h, int i, float*) {
  const int col = col0 + i;
  const int chunk = col >> 2, within = col & 3;
  const float* base = reinterpret_cast<const float*>(lds);
  f32x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int row = 16 * s + (e < 4 ? 4 * h + e : 8 + 4 * h + e - 4);
    r[e] = base[row_slot<T, D>(row, chunk) * 4 + within];
  }
  return r;
}

// --- 16x16x32 matrix-core helpers ---------------------------------------------
// v_mfma_f32_16x16x32 (bf16 / fp16; fp32 as eight 16x16x4 steps over the same
// registers).  Layout (checked on the hardware): A (16 x 32) lane l holds row l%16
// and reduction elements 8*(l/16)..+7; B (32 x 16) lane l holds column l%16 and
// the same elements; the 16x16 result gives lane l column l%16 and rows
// 4*(l/16) + i in register i.
__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f16x8 a, f16x8 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x8 a, f32x8 b, f32x4 acc) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ f32x4 mma16_split_a(const SplitBF16& a, bf16x8 b, f32x4 acc) {
  acc = mma16(a.hi, b, acc);
  return mma16(a.lo, b, acc);
}
__device__ __forceinline__ f32x4 mma16_split_a(const SplitF32& a, f32x8 b, f32x4 acc) { return mma16(a.hi, b, acc); }

// row-major tile, row r, 32-wide reduction step s, lane group q = l/16 -> elements 32s+8q..+7
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::frag frag16_row(const u32x4* lds, int r, int s, int q) {
  using C = TileCfg<T, D>;
  const int c0 = (32 * s + 8 * q) / C::kCE;
  u32x4 ch[C::kFC];
#pragma unroll
  for (int p = 0; p < C::kFC; ++p) ch[p] = lds[row_slot<T, D>(r, c0 + p)];
  return frag_from_chunks(ch, (T*)nullptr);
}
// one token row from global memory as 16x16x32 B fragments (elements 32s+8q..+7)
template <typename T, int D>
__device__ __forceinline__ void load_row_frags16(typename Elem<T>::frag* f, const T* __restrict__ row, bool ok, int q) {
  using C = TileCfg<T, D>;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    u32x4 ch[C::kFC];
#pragma unroll
    for (int p = 0; p < C::kFC; ++p)
      ch[p] = ok ? *reinterpret_cast<const u32x4*>(row + 32 * s + 8 * q + p * C::kCE) : u32x4{0, 0, 0, 0};
    f[s] = frag_from_chunks(ch, (T*)nullptr);
  }
}
// Transposed 16x16x32 operand from a row-major tile whose rows are the reduction
// index: lane l gets column col0 + l%16 of rows {r0 + e : e < 4} and {r0 + 16 + e : e < 4}
// (r0 = 32*ks + 4*(l/16) for the k-slot order of a 16x16 result taken as operand).
template <typename T, int D>
__device__ __forceinline__ bf16x8 frag16_tr(const u32x4* lds, int col0, int r0, int i, bf16*) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const int col = col0 + 4 * (i & 3);
  const int chunk = col >> 3, byte = (col & 7) * 2;
  const int r1 = r0 + (i >> 2), r2 = r1 + 16;
  const char* base = reinterpret_cast<const char*>(lds);
  const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (bf16x4 __attribute__((address_space(3)))*)(base + row_slot<T, D>(r1, chunk) * 16 + byte));
  const bf16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (bf16x4 __attribute__((address_space(3)))*)(base + row_slot<T, D>(r2, chunk) * 16 + byte));
  return bf16x8{v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
}
template <typename T, int D>
__device__ __forceinline__ f16x8 frag16_tr(const u32x4* lds, int col0, int r0, int i, f16*) {
  typedef __fp16 h4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  const int col = col0 + 4 * (i & 3);
  const int chunk = col >> 3, byte = (col & 7) * 2;
  const int r1 = r0 + (i >> 2), r2 = r1 + 16;
  const char* base = reinterpret_cast<const char*>(lds);
  const f16x4 v1 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (h4 __attribute__((address_space(3)))*)(base + row_slot<T, D>(r1, chunk) * 16 + byte)));
  const f16x4 v2 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (h4 __attribute__((address_space(3)))*)(base + row_slot<T, D>(r2, chunk) * 16 + byte)));
  return f16x8{v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
}
template <typename T, int D>
__device__ __forceinline__ f32x8 frag16_tr(const u32x4* lds, int col0, int r0, int i, float*) {
  const int col = col0 + i;
  const int chunk = col >> 2, within = col & 3;
  const float* base = reinterpret_cast<const float*>(lds);
  f32x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int row = r0 + (e < 4 ? e : 16 + e - 4);
    r[e] = base[row_slot<T, D>(row, chunk) * 4 + within];
  }
  return r;
}

// Closed forms of the two 16-bit operand reads above for the XOR-swizzled layout
// (2-byte elements, CPR = D/8 chunks per row): the lane-dependent part of the
// byte address is one constant per lane, and the reduction step (row reads) or
// the output tile t (transposed reads) enters by an XOR with 64*s or 32*t -- one
// VALU op per step -- while rows and buffers are immediate offsets.
template <int D>
__device__ __forceinline__ int row_lane16(int l16, int q) {
  constexpr int CPR = D / 8;
  const int f = row_swz<bf16, D>(l16);
  return l16 * CPR * 16 + 64 * (f >> 2) + 16 * (q ^ (f & 3));
}
template <int D>
__device__ __forceinline__ int tr_lane16(int i, int q) {
  constexpr int CPR = D / 8;
  const int x = 4 * q + (i >> 2), f = row_swz<bf16, D>(x), cl = (i >> 1) & 1;
  return x * CPR * 16 + 32 * (f >> 1) + 16 * (cl ^ (f & 1)) + 8 * (i & 1);
}
// frag16_row(lds, 16*mt + l16, s, q) for 16-bit tiles; `lane_xs` = row_lane16 ^ (64*s)
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::frag frag16_row_fast(const u32x4* lds, int mt, int lane_xs) {
  const char* p = reinterpret_cast<const char*>(lds) + mt * 16 * (D / 8) * 16 + lane_xs;
  return __builtin_bit_cast(typename Elem<T>::frag, *reinterpret_cast<const u32x4*>(p));
}
// frag16_tr(lds, 16*t, 32*ks + 4q, l16) for 16-bit tiles; `lane_xt` = tr_lane16 ^ (32*t)
template <typename T, int D>
__device__ __forceinline__ bf16x8 frag16_tr_fast(const u32x4* lds, int ks, int lane_xt, bf16*) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const char* base = reinterpret_cast<const char*>(lds) + 32 * ks * (D / 8) * 16 + lane_xt;
  const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 __attribute__((address_space(3)))*)base);
  const bf16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (bf16x4 __attribute__((address_space(3)))*)(base + 16 * (D / 8) * 16));
  return bf16x8{v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
}
template <typename T, int D>
__device__ __forceinline__ f16x8 frag16_tr_fast(const u32x4* lds, int ks, int lane_xt, f16*) {
  typedef __fp16 h4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  const char* base = reinterpret_cast<const char*>(lds) + 32 * ks * (D / 8) * 16 + lane_xt;
  const f16x4 v1 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((h4 __attribute__((address_space(3)))*)base));
  const f16x4 v2 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (h4 __attribute__((address_space(3)))*)(base + 16 * (D / 8) * 16)));
  return f16x8{v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
}

// --- direct global -> LDS tile loads (no register staging) --------------------
// A row-major tile of 64 token rows, written with the XOR-swizzled slots of
// row_slot: LDS chunk position p (row p / CPR, slot p % CPR) receives global chunk
// slot ^ (row mod RSw) of that row.  One global_load_lds_dwordx4 moves 64 chunks
// (1 KB); a work-group of W waves issues instructions w, w+W, ...  `off[i]` is the
// element offset (relative to the tile's first token) that this lane loads in its
// i-th instruction; padding rows (>= T) repeat row 0 and must be masked by the user.
template <typename T, int D, int W>
struct DmaCfg {
  static constexpr int kInstr = TileCfg<T, D>::kRowChunks / 64;   // instructions per tile
  static constexpr int kPer = kInstr / W;                          // per wave
  static_assert(kInstr % W == 0, "tile chunks must split evenly over the waves");
};
template <typename T, int D, int W>
__device__ __forceinline__ void dma_offsets(int* off, const Geo& g, int w, int lane) {
  using C = TileCfg<T, D>;
#pragma unroll
  for (int i = 0; i < DmaCfg<T, D, W>::kPer; ++i) {
    const int p = 64 * (w + W * i) + lane;
    const int r = p / C::kCPR, s = p % C::kCPR;
    const int c = s ^ row_swz<T, D>(r);
    off[i] = (r < g.T ? member_offset(g, r) : 0) * D + c * C::kCE;
  }
}
// Buffer-resource form (MUBUF "buffer_load ... lds"): unlike the global form it
// leaves the compiler's LDS-read wait counts exact.  `rsrc` covers one head;
// `tile_bytes` is the byte offset of the tile's first token row.
template <typename T, int D, int W>
__device__ __forceinline__ void dma_tile(u32x4* lds, __amdgpu_buffer_rsrc_t rsrc, int tile_bytes, const int* off, int w) {
#pragma unroll
  for (int i = 0; i < DmaCfg<T, D, W>::kPer; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(lds + 64 * (w + W * i)), 16,
                                             off[i] * (int)sizeof(T), tile_bytes, 0, 0);
}
// 64 floats of one tile row each (e.g. LSE): lane l loads the value of member row l
__device__ __forceinline__ void dma_row_stats(float* lds, __amdgpu_buffer_rsrc_t rsrc, int tile_bytes, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 4, off * 4, tile_bytes, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes, 0x00020000);
}
// wait for this wave's direct loads (vmcnt(0), other counters untouched)
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// --- staging: global -> registers -> LDS --------------------------------------
// Row items: per thread kRowPer chunks; `off[i]` = token offset (relative to the
// tile corner) of the row of item i, or -1 for a padding row.
template <typename T, int D>
struct RowStage {
  u32x4 v[TileCfg<T, D>::kRowPer];
};
template <typename T, int D>
__device__ __forceinline__ void row_offsets(int* off, const Geo& g, int tid) {
  using C = TileCfg<T, D>;
#pragma unroll
  for (int i = 0; i < C::kRowPer; ++i) {
    const int r = (tid + i * kTileThreads) / C::kCPR;
    off[i] = r < g.T ? member_offset(g, r) : -1;
  }
}
template <typename T, int D>
__device__ __forceinline__ void row_load(RowStage<T, D>& st, const T* __restrict__ X, int base, const int* off, int tid) {
  using C = TileCfg<T, D>;
#pragma unroll
  for (int i = 0; i < C::kRowPer; ++i) {
    const int c = (tid + i * kTileThreads) % C::kCPR;
    st.v[i] = off[i] >= 0 ? *reinterpret_cast<const u32x4*>(X + (size_t)(base + off[i]) * D + c * C::kCE)
                          : u32x4{0, 0, 0, 0};
  }
}
template <typename T, int D>
__device__ __forceinline__ void row_store(const RowStage<T, D>& st, u32x4* lds, int tid) {
  using C = TileCfg<T, D>;
#pragma unroll
  for (int i = 0; i < C::kRowPer; ++i) {
    const int lc = tid + i * kTileThreads;
    lds[row_slot<T, D>(lc / C::kCPR, lc % C::kCPR)] = st.v[i];
  }
}

// Group items: per thread kGPer items of 8 chunks.
template <typename T, int D>
struct GroupStage {
  u32x4 v[TileCfg<T, D>::kGPer][8];
};
template <typename T, int D>
__device__ __forceinline__ void group_offsets(int (*off)[8], const Geo& g, int tid) {
  using C = TileCfg<T, D>;
#pragma unroll
  for (int i = 0; i < C::kGPer; ++i) {
    const int kg = (tid + i * kTileThreads) / C::kCPR;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = group_row(kg & 7, e);
      off[i][e] = (kg < 8 && r < g.T) ? member_offset(g, r) : -1;
    }
  }
}
template <typename T, int D>
__device__ __forceinline__ void group_load(GroupStage<T, D>& st, const T* __restrict__ X, int base,
                                           const int (*off)[8], int tid) {
  using C = TileCfg<T, D>;
#pragma unroll
  for (int i = 0; i < C::kGPer; ++i) {
    const int c = (tid + i * kTileThreads) % C::kCPR;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      st.v[i][e] = off[i][e] >= 0 ? *reinterpret_cast<const u32x4*>(X + (size_t)(base + off[i][e]) * D + c * C::kCE)
                                  : u32x4{0, 0, 0, 0};
  }
}

// 8 tokens x one chunk -> transposed rows.  The stored element type is the
// source type, except that bf16 sources can be stored as fp16 (exact for values
// in the fp16 normal range; used for the operand of the fp16 P.V product).
__device__ __forceinline__ uint32_t bf16_half(uint32_t w, int hi) { return hi ? (w >> 16) : (w & 0xffffu); }
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ void transpose_store(u32x4* lds_t, const u32x4 (&v)[8], int kg, int c, bf16*, bf16*) {
  using C = TileCfg<bf16, 64>;  // the transposed row geometry depends only on the element size
#pragma unroll
  for (int m = 0; m < 8; ++m) {            // element m of the chunk -> row d = 8c + m
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)            // positions 2j, 2j+1 of the group
      w[j] = bf16_half(v[2 * j][m >> 1], m & 1) | (bf16_half(v[2 * j + 1][m >> 1], m & 1) << 16);
    const int d = 8 * c + m;
    lds_t[d * C::kTR + (kg ^ ((d ^ (d >> C::kTLog)) & (C::kTR - 1)))] = u32x4{w[0], w[1], w[2], w[3]};
  }
}
__device__ __forceinline__ void transpose_store(u32x4* lds_t, const u32x4 (&v)[8], int kg, int c, bf16*, f16*) {
  using C = TileCfg<f16, 64>;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16 a = (f16)bf16_bits_to_f32(bf16_half(v[2 * j][m >> 1], m & 1));
      const f16 b = (f16)bf16_bits_to_f32(bf16_half(v[2 * j + 1][m >> 1], m & 1));
      w[j] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    }
    const int d = 8 * c + m;
    lds_t[d * C::kTR + (kg ^ ((d ^ (d >> C::kTLog)) & (C::kTR - 1)))] = u32x4{w[0], w[1], w[2], w[3]};
  }
}
__device__ __forceinline__ void transpose_store(u32x4* lds_t, const u32x4 (&v)[8], int kg, int c, float*, float*) {
  using C = TileCfg<float, 64>;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int d = 4 * c + m;
    const int f = (d ^ (d >> C::kTLog)) & (C::kTR - 1);
    lds_t[d * C::kTR + ((2 * kg) ^ f)] = u32x4{v[0][m], v[1][m], v[2][m], v[3][m]};
    lds_t[d * C::kTR + ((2 * kg + 1) ^ f)] = u32x4{v[4][m], v[5][m], v[6][m], v[7][m]};
  }
}
// store group items transposed (lds_t, element type TO) and, if lds_r != nullptr,
// row-major too (source type T)
template <typename T, int D, typename TO = T>
__device__ __forceinline__ void group_store(const GroupStage<T, D>& st, u32x4* lds_t, u32x4* lds_r, int tid) {
  using C = TileCfg<T, D>;
#pragma unroll
  for (int i = 0; i < C::kGPer; ++i) {
    const int it = tid + i * kTileThreads;
    if (it < C::kGItems) {
      const int kg = it / C::kCPR, c = it % C::kCPR;
      transpose_store(lds_t, st.v[i], kg, c, (T*)nullptr, (TO*)nullptr);
      if (lds_r != nullptr) {
#pragma unroll
        for (int e = 0; e < 8; ++e) lds_r[row_slot<T, D>(group_row(kg, e), c)] = st.v[i][e];
      }
    }
  }
}

// 4 fp32 values -> output row (16 bytes fp32, or 8 bytes bf16 rounded to nearest even)
__device__ __forceinline__ void store4(void* base, size_t off, int out_f32, float v0, float v1, float v2, float v3) {
  if (out_f32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + off) = f32x4{v0, v1, v2, v3};
  } else {
    const bf16 b0 = (bf16)v0, b1 = (bf16)v1, b2 = (bf16)v2, b3 = (bf16)v3;
    const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
    const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
    *reinterpret_cast<u32x2*>(reinterpret_cast<bf16*>(base) + off) = u32x2{w0, w1};
  }
}
__device__ __forceinline__ void store1(void* base, size_t off, int out_f32, float v) {
  if (out_f32) reinterpret_cast<float*>(base)[off] = v;
  else reinterpret_cast<bf16*>(base)[off] = (bf16)v;
}

}  // namespace dsa
