// LDS tiles of 64 tokens x D elements for the attention kernels (gfx950).
//
// Layout: row-major [64][D]; a token row is D*sizeof(T) bytes = CPR 16-byte
// chunks, and chunk c of row r sits at slot c ^ row_swz(r), so both the row-wise
// operand reads and the transposing reads of 4-row groups are free of bank
// conflicts (see row_swz).
//
// Tiles are filled either by direct global->LDS loads (dma_*: the backward) or
// through registers (row_*: the forward's Q tile, 128 threads).  Global accesses
// are 16-byte chunks.
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
  static constexpr int kRSw = kCPR < 16 ? kCPR : 16;
  static constexpr int kSteps = D / 16;                       // reduction steps over d
  static constexpr int kDTiles = D / 32;                      // 32-wide tiles over d
  static constexpr int kRowChunks = 64 * kCPR;                // LDS chunks of a row-major tile
};

// Row swizzle h(r), periodic in 16 rows.  Measured on gfx950: a 16-byte-per-lane
// read is served 16 lanes at a time and is conflict-free when those lanes hit 16
// distinct 16-byte slots of a 256-byte window; the transposing 8-byte read
// (ds_read_b64_tr_b16) is served 32 lanes -- two 4-row groups, i.e. 8 consecutive
// rows -- at a time and needs their 32-byte column segments to be 8 distinct
// segments of the window.  So h must be a bijection on 16 consecutive rows (row
// reads of one chunk column) and h >> 1 a bijection on each aligned block of 8
// rows (transposing reads of one 32-byte segment):
//   d = 128 (16 slots per 256-byte row):  h = ((r & 7) << 1) | (r >> 3 & 1)
//   d = 64  (8 slots per 128-byte row, two rows per window): h = (r >> 1 & 3) << 1 |
//     (r >> 3 & 1), a bijection on each parity class of 16 rows and, with h >> 1,
//     on each parity class of an 8-row block.
template <typename T, int D>
__device__ __forceinline__ int row_swz(int r) {
  if constexpr (TileCfg<T, D>::kRSw == 16) return ((r & 7) << 1) | ((r >> 3) & 1);
  else if constexpr (TileCfg<T, D>::kRSw == 8) return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
  else return r & (TileCfg<T, D>::kRSw - 1);
}
template <typename T, int D>
__device__ __forceinline__ int row_slot(int r, int c) {
  using C = TileCfg<T, D>;
  return r * C::kCPR + (c ^ row_swz<T, D>(r));
}
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
// A contiguous run of W * PER KB copied as is (e.g. a fragment-major block): wave w
// issues chunks w, w + W, ..., lane l moving bytes 16l..16l+15 of each 1 KB chunk.
template <int PER, int W>
__device__ __forceinline__ void dma_linear(u32x4* lds, __amdgpu_buffer_rsrc_t rsrc, int src_bytes, int w, int lane) {
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = w + W * i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(lds + 64 * c), 16,
                                             lane * 16 + c * 1024, src_bytes, 0, 0);
  }
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
