// Block-sparse attention forward for gfx950.
//
// Computes, for every query token of a query tile, exact softmax attention over
// the keys of the key blocks that the tile kept (DSV page, gist.science/ar/paper/
// 2502.07590, section 4: stage two computes only the cues the predictor picked;
// section 3b: one selection per tile of neighbouring queries).
//
// Two kernels:
//  1. kv_prep: one pass over K and V that writes every key block in fragment-
//     major order into the caller's workspace: K as MFMA A fragments of S^T = K Q^T,
//     V transposed (and, for bf16 inputs, converted to fp16) as A fragments of
//     O^T = V^T P^T.  Each fragment is 64 lanes x 16 B contiguous, so every load
//     of the attention kernel reads 1 KB contiguous (8 full cache lines) instead
//     of 32 B from each of 32 rows.  A block is gathered by ~k query tiles, so one
//     reorganisation serves all of them.
//  2. attn_fwd: one work-group (2 waves) per query tile of T <= 64 tokens, two
//     waves per SIMD (<= 256 registers): while one wave runs its softmax the other
//     keeps the matrix cores busy.  Wave w takes key positions 32w..32w+31 of every
//     kept block for all 64 query rows:
//        S^T (32 keys x 64 queries) = K Q^T          16 MFMA; Q tile in LDS,
//                                                    fragments read one step ahead
//        online softmax (fp32, base 2), one query per lane and N-tile
//        O^T (d x 64 queries)      += V^T P^T        16 MFMA; P^T taken straight
//                                                    from the S^T registers
//     K(j+1) is requested as soon as S(j) has consumed K(j), V(j+1) as soon as the
//     P.V product has consumed V(j).  Each wave keeps its own running max / sum /
//     O over its key half; the halves are merged once, through LDS, at the end.
// With bf16 inputs the P.V product runs on fp16 matrix cores: kv_prep converts
// V * 2^t, with one power of two per (b, h) that puts the head's largest |v| in
// [2^14, 2^15) (launch_pow2_scale), so the conversion is exact whatever the size
// of V, and the output is multiplied by 2^-t in fp32, exactly; P is rounded to
// fp16 (2^-12 relative) and the row sum adds the same fp16 probabilities (v_dot2,
// fp32 accumulation).  The running maximum only moves when a row's maximum grows
// by more than 2^8, so most blocks skip rescaling O; this is exact (numerator and
// denominator share the maximum).
#include "kernels.hpp"
#include "tiles.hpp"

namespace dsa {

namespace {

constexpr float kRescaleSlack = 8.0f;   // log2 units

template <typename T> struct PVType;
template <> struct PVType<bf16> { typedef f16 type; };
template <> struct PVType<float> { typedef float type; };

// ------------------------------------------------------------ 1. K, V -> fragment-major blocks
// Output per (head, block j), for each 32-key half w: the K A-fragments of the
// d/16 reduction steps, then the V^T A-fragments of the (d/32) x 2 (d tile, key
// step) pairs.  A fragment is 64 lanes x 16 bytes stored lane-major, so one load
// instruction of the attention kernel reads 1 KB contiguous.
//  * K fragment chunk (w, f, lane) = 16-byte input chunk (d0 / CE) of key row
//    32w + lane%32 with d0 = 16*(f/FC) + 8*(lane/32) + CE*(f%FC): a permutation of
//    chunks, no transposition.
//  * V^T fragment chunk (w, f=(t*2+s)*PFC+p, lane) holds element d = 32t + lane%32
//    of the keys at positions 32w + 16s + 8*(lane/32) + PE*p + e (key via perm16):
//    a thread transposes a CE x CE block (CE keys x CE elements) in registers,
//    converting to the P.V element type.
// One work-group of 256 threads per (head, block); all global accesses are
// 16-byte chunks.
template <typename T, int D>
__global__ __launch_bounds__(256) void kv_prep_kernel(FwdArgs a) {
  typedef typename PVType<T>::type PT;
  constexpr int CE = Elem<T>::kChunkElems;                     // == Elem<PT>::kChunkElems
  constexpr int CPR = D / CE;
  constexpr int FC = Elem<T>::kFragChunks;
  constexpr int KF = D / 16 * FC;                              // K chunks per lane per half
  constexpr int PFC = Elem<PT>::kFragChunks;
  static_assert(Elem<PT>::kChunkElems == CE, "square register transpose");
  const Geo g = a.g;
  const int bj = blockIdx.x;
  const int bh = bj / g.NB, j = bj - bh * g.NB;
  const size_t hoff = (size_t)bh * g.N * D;
  const T* __restrict__ Kh = reinterpret_cast<const T*>(a.K) + hoff;
  const T* __restrict__ Vh = reinterpret_cast<const T*>(a.V) + hoff;
  const int base = tile_base(g, j);
  u32x4* __restrict__ ko = reinterpret_cast<u32x4*>(reinterpret_cast<T*>(a.Kf) + (size_t)bj * 64 * D);
  u32x4* __restrict__ vo = reinterpret_cast<u32x4*>(reinterpret_cast<PT*>(a.Vt) + (size_t)bj * 64 * D);
  // K: 2 * KF * 64 output chunks
  for (int it = threadIdx.x; it < 2 * KF * 64; it += 256) {
    const int lane = it % 64, f = (it / 64) % KF, w = it / (64 * KF);
    const int r = 32 * w + (lane & 31);
    const int d0 = 16 * (f / FC) + 8 * (lane >> 5) + CE * (f % FC);
    ko[it] = r < g.T ? *reinterpret_cast<const u32x4*>(Kh + (size_t)(base + member_offset(g, r)) * D + d0)
                     : u32x4{0, 0, 0, 0};
  }
  // V: (64 / CE) position groups x CPR chunk columns, one CE x CE block each
  for (int it = threadIdx.x; it < (64 / CE) * CPR; it += 256) {
    const int c = it % CPR, pg = it / CPR;                     // chunk column, position group
    u32x4 in[CE];
#pragma unroll
    for (int e = 0; e < CE; ++e) {
      const int pos = CE * pg + e;
      const int key = 16 * (pos >> 4) + perm16(pos & 15);
      in[e] = key < g.T ? *reinterpret_cast<const u32x4*>(Vh + (size_t)(base + member_offset(g, key)) * D + c * CE)
                        : u32x4{0, 0, 0, 0};
    }
    const int w = (CE * pg) / 32, s2 = ((CE * pg) % 32) / 16, hh = ((CE * pg) % 16) / 8, p = ((CE * pg) % 8) / CE;
#pragma unroll
    for (int m = 0; m < CE; ++m) {                             // element m of the chunks -> d row c*CE + m
      const int d = c * CE + m;
      PT e[CE];
#pragma unroll
      for (int q = 0; q < CE; ++q) e[q] = (PT)to_f32(reinterpret_cast<const T*>(&in[q])[m]);
      const int t = d / 32, lane = (d % 32) + 32 * hh;
      const int f = (t * 2 + s2) * PFC + p;
      vo[(w * (D / 32 * 2 * PFC) + f) * 64 + lane] = *reinterpret_cast<const u32x4*>(e);
    }
  }
}

// Same output for 16-bit inputs, through LDS: the block's K and V rows are staged
// with coalesced 16-byte loads (256 threads, every row read as one 256-byte run)
// into XOR-swizzled row-major tiles; each K output chunk is then one 16-byte LDS
// read, and each V^T output chunk (8 keys of one d) two transposing LDS reads of
// 4 keys -- with the perm16 key order the 8 keys of a chunk are two runs of 4
// consecutive keys -- converted to fp16.  Every global store is coalesced.
template <int D>
__global__ __launch_bounds__(256) void kv_prep16_kernel(FwdArgs a) {
  typedef bf16 T;
  typedef f16 PT;
  using C = TileCfg<T, D>;
  constexpr int CE = C::kCE;                                   // 8 elements per chunk
  constexpr int CPR = C::kCPR;
  constexpr int FC = Elem<T>::kFragChunks;
  constexpr int KF = D / 16 * FC;                              // K chunks per lane per half
  constexpr int NCH = 64 * CPR;                                // chunks of a 64-row tile
  static_assert(CE == 8 && Elem<PT>::kFragChunks == 1, "16-bit elements");
  __shared__ u32x4 kt[NCH], vt[NCH];
  const Geo g = a.g;
  const int bj = blockIdx.x;
  const int bh = bj / g.NB, j = bj - bh * g.NB;
  const size_t hoff = (size_t)bh * g.N * D;
  const T* __restrict__ Kh = reinterpret_cast<const T*>(a.K) + hoff;
  const T* __restrict__ Vh = reinterpret_cast<const T*>(a.V) + hoff;
  const int base = tile_base(g, j);
  const int tid = threadIdx.x;
  const float vup = a.vscale[bh].x;                            // 2^t of this head
#pragma unroll
  for (int i = 0; i < NCH / 256; ++i) {
    const int idx = tid + 256 * i, r = idx / CPR, c = idx % CPR;
    u32x4 kv = u32x4{0, 0, 0, 0}, vv = kv;
    if (r < g.T) {
      const size_t off = (size_t)(base + member_offset(g, r)) * D + c * CE;
      kv = *reinterpret_cast<const u32x4*>(Kh + off);
      vv = *reinterpret_cast<const u32x4*>(Vh + off);
    }
    kt[row_slot<T, D>(r, c)] = kv;
    vt[row_slot<T, D>(r, c)] = vv;
  }
  __syncthreads();
  u32x4* __restrict__ ko = reinterpret_cast<u32x4*>(reinterpret_cast<T*>(a.Kf) + (size_t)bj * 64 * D);
  u32x4* __restrict__ vo = reinterpret_cast<u32x4*>(reinterpret_cast<PT*>(a.Vt) + (size_t)bj * 64 * D);
  // K: output chunk (w, f, lane) = chunk d0/CE of key row 32w + lane%32
#pragma unroll
  for (int i = 0; i < 2 * KF * 64 / 256; ++i) {
    const int it = tid + 256 * i;
    const int lane = it % 64, f = (it / 64) % KF, w = it / (64 * KF);
    const int r = 32 * w + (lane & 31);
    const int d0 = 16 * (f / FC) + 8 * (lane >> 5) + CE * (f % FC);
    ko[it] = kt[row_slot<T, D>(r, d0 / CE)];
  }
  // V^T: output chunk (w, f = 2t + s, lane) = V[key(p0 + e)][32t + lane%32], e < 8,
  // p0 = 32w + 16s + 8(lane/32); lanes 16g..16g+15 read columns 32t + 16(g%2) + i
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const char* vb = reinterpret_cast<const char*>(vt);
#pragma unroll
  for (int i = 0; i < NCH / 256; ++i) {
    const int o = tid + 256 * i;
    const int lane = o % 64, wf = o / 64;
    const int w = wf / (D / 16), f = wf % (D / 16);
    const int t = f >> 1, s2 = f & 1, hh = lane >> 5, li = lane & 15;
    const int p0 = 32 * w + 16 * s2 + 8 * hh;                  // multiple of 8
    const int keyA = 16 * (p0 >> 4) + perm16(p0 & 15);         // positions p0..p0+3
    const int keyB = 16 * (p0 >> 4) + perm16((p0 & 15) + 4);   // positions p0+4..p0+7
    const int col = 32 * t + 16 * ((lane >> 4) & 1) + 4 * (li & 3);
    const int chunk = col >> 3, byte = (col & 7) * 2;
    const int ra = keyA + (li >> 2), rb = keyB + (li >> 2);
    const bf16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (bf16x4 __attribute__((address_space(3)))*)(vb + row_slot<T, D>(ra, chunk) * 16 + byte));
    const bf16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (bf16x4 __attribute__((address_space(3)))*)(vb + row_slot<T, D>(rb, chunk) * 16 + byte));
    PT e[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      e[q] = (PT)((float)x0[q] * vup);
      e[4 + q] = (PT)((float)x1[q] * vup);
    }
    vo[o] = *reinterpret_cast<const u32x4*>(e);
  }
}

// ------------------------------------------------------------ 2. attention
template <typename T, int D>
struct FwdCfg {
  typedef typename PVType<T>::type PT;
  static constexpr int kSteps = D / 16;       // reduction steps over d (S^T product)
  static constexpr int kDTiles = D / 32;      // 32-row tiles over d (O^T product)
  static constexpr int kPE = Elem<PT>::kChunkElems;
  static constexpr int kPFC = Elem<PT>::kFragChunks;
};

// Fragment loads go through buffer resources (per-head base, byte bound): one
// lane-constant 32-bit offset, the block in the scalar offset, the step in the
// immediate; reads past the bound return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// K rows of the wave's 32 keys of one block (A operand of S^T = K Q^T)
template <typename T, int D>
struct KFrags {
  typename Elem<T>::frag f[FwdCfg<T, D>::kSteps];
};
// V^T rows for the wave's 32 key positions of one block (A operand of O^T += V^T P^T)
template <typename T, int D>
struct VFrags {
  typename Elem<typename FwdCfg<T, D>::PT>::frag f[FwdCfg<T, D>::kDTiles][2];
};

// Fragment-major blocks: fragment f of half w of block j starts at
// ((j*2 + w)*F + f) * 1 KB; lane l reads bytes 16l..16l+15.
template <typename T, int D>
__device__ __forceinline__ void load_k(KFrags<T, D>& kf, __amdgpu_buffer_rsrc_t rk, int lvoff, int soff) {
  using C = FwdCfg<T, D>;
  constexpr int FC = Elem<T>::kFragChunks;
#pragma unroll
  for (int s = 0; s < C::kSteps; ++s) {
    u32x4 ch[FC];
#pragma unroll
    for (int q = 0; q < FC; ++q) ch[q] = bload(rk, lvoff + (s * FC + q) * 1024, soff);
    kf.f[s] = frag_from_chunks(ch, (T*)nullptr);
  }
}
template <typename T, int D>
__device__ __forceinline__ void load_v(VFrags<T, D>& vf, __amdgpu_buffer_rsrc_t rv, int lvoff, int soff) {
  using C = FwdCfg<T, D>;
  typedef typename C::PT PT;
  constexpr int PFC = Elem<PT>::kFragChunks;
#pragma unroll
  for (int t = 0; t < C::kDTiles; ++t) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 ch[PFC];
#pragma unroll
      for (int q = 0; q < PFC; ++q) ch[q] = bload(rv, lvoff + ((t * 2 + s) * PFC + q) * 1024, soff);
      vf.f[t][s] = frag_from_chunks(ch, (PT*)nullptr);
    }
  }
}

template <typename T, int D>
struct WaveState {
  f32x16 o[2][FwdCfg<T, D>::kDTiles];   // O^T per query N-tile and d tile
  float m[2], l[2];                      // running max (log2 units) and lane-partial sum per N-tile
};

// row sum of eight probabilities as the P.V product sees them (fp16: the same
// rounded values as the numerator, summed exactly in fp32 by v_dot2)
__device__ __forceinline__ float frag_sum(const f16x8& p, float acc) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 one = {(f16)1.0f, (f16)1.0f};
#pragma unroll
  for (int e = 0; e < 8; e += 2) acc = __builtin_amdgcn_fdot2(h2{p[e], p[e + 1]}, one, acc, false);
  return acc;
}
__device__ __forceinline__ float frag_sum(const f32x8& p, float acc) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc += p[e];
  return acc;
}

// S^T for one block: A = K rows (registers), B = Q rows (LDS, row-major tile)
template <typename T, int D>
__device__ __forceinline__ void block_scores(f32x16 (&s)[2], const KFrags<T, D>& kf, const u32x4* lds_q, int l32, int h) {
  using C = FwdCfg<T, D>;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) s[nt] = f32x16{};
  // Q fragments are read one step ahead of the MFMAs that use them
  typedef typename Elem<T>::frag Frag;
  Frag qa0 = frag_row<T, D>(lds_q, l32, 0, h), qa1 = frag_row<T, D>(lds_q, 32 + l32, 0, h);
#pragma unroll
  for (int k = 0; k < C::kSteps; ++k) {
    Frag qb0 = qa0, qb1 = qa1;
    if (k + 1 < C::kSteps) {
      qb0 = frag_row<T, D>(lds_q, l32, k + 1, h);
      qb1 = frag_row<T, D>(lds_q, 32 + l32, k + 1, h);
    }
    s[0] = mma_step(kf.f[k], qa0, s[0]);
    s[1] = mma_step(kf.f[k], qa1, s[1]);
    qa0 = qb0;
    qa1 = qb1;
    __builtin_amdgcn_sched_barrier(0);
  }
}

// online softmax of one block's scores; returns the P^T fragments (B operand of the P.V product)
template <typename T, int D, bool FULL>
__device__ __forceinline__ void block_softmax(WaveState<T, D>& st, f32x16 (&s)[2],
                                              typename Elem<typename FwdCfg<T, D>::PT>::frag (&pf)[2][2],
                                              float c2, int kvalid, int h) {
  using C = FwdCfg<T, D>;
  typedef typename C::PT PT;
  if constexpr (!FULL) {                      // padding keys of this wave's half (T < 64)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + 4 * h + (i & 3) >= kvalid) s[nt][i] = -INFINITY;
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float mb = fmaxf(fmaxf(s[nt][0], s[nt][1]), s[nt][2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mb = fmaxf(fmaxf(mb, s[nt][i]), s[nt][i + 1]);
    mb = fmaxf(mb, s[nt][15]);
    mb = pair_max(mb);
    const float mnew = mb * c2;
    if (ballot(mnew > st.m[nt] + kRescaleSlack)) {
      const float mt = fmaxf(st.m[nt], mnew);
      const float alpha = (mt == -INFINITY) ? 1.f : fast_exp2(st.m[nt] - mt);
      st.m[nt] = mt;
      st.l[nt] *= alpha;
#pragma unroll
      for (int t = 0; t < C::kDTiles; ++t) st.o[nt][t] *= alpha;
    }
    const float mneg = -st.m[nt];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(fmaf(s[nt][8 * ks + e], c2, mneg));
      pf[nt][ks] = to_frag(pv, (PT*)nullptr);
      st.l[nt] = frag_sum(pf[nt][ks], st.l[nt]);
    }
  }
}

template <typename T, int D>
__device__ __forceinline__ void block_pv(WaveState<T, D>& st, const VFrags<T, D>& vf,
                                         const typename Elem<typename FwdCfg<T, D>::PT>::frag (&pf)[2][2]) {
  using C = FwdCfg<T, D>;
#pragma unroll
  for (int t = 0; t < C::kDTiles; ++t) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) st.o[nt][t] = mma_step(vf.f[t][ks], pf[nt][ks], st.o[nt][t]);
    }
  }
}

// Two waves per SIMD (<= 256 registers each): while one wave runs its softmax
// the other keeps the matrix cores busy.
template <typename T, int D, bool FULL>
__global__ __launch_bounds__(kTileThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdArgs a) {
  using C = FwdCfg<T, D>;
  typedef typename C::PT PT;
  typedef typename Elem<PT>::frag PFrag;
  using TC = TileCfg<T, D>;
  // the Q tile (row-major, swizzled) during the block loop; the merge buffers after it
  constexpr int kQBytes = TC::kRowChunks * 16;
  constexpr int kMrgBytes = (2 * C::kDTiles * 16 * 64 + 2 * 2 * 64) * 4;
  __shared__ __attribute__((aligned(16))) char smem[kQBytes > kMrgBytes ? kQBytes : kMrgBytes];
  u32x4* lds_q = reinterpret_cast<u32x4*>(smem);
  float (*mrg_o)[C::kDTiles * 16][64] = reinterpret_cast<float (*)[C::kDTiles * 16][64]>(smem);
  float (*mrg_ml)[2][64] = reinterpret_cast<float (*)[2][64]>(smem + 2 * C::kDTiles * 16 * 64 * 4);

  const Geo g = a.g;
  const int L = blockIdx.x;                 // natural order (see common.hpp)
  const int bh = L / g.NB;
  const int tau = L - bh * g.NB;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, h = lane >> 5;

  const size_t head_off = (size_t)bh * g.N * D;
  const T* __restrict__ Qh = reinterpret_cast<const T*>(a.Q) + head_off;
  const int* __restrict__ irow = a.idx + ((size_t)bh * g.NB + tau) * a.kmax;
  int kk = a.kvec[bh];
  kk = kk < 1 ? 1 : (kk > a.kmax ? a.kmax : kk);
  const int tau_base = tile_base(g, tau);

  {  // stage the Q tile once
    int qoff[TC::kRowPer];
    row_offsets<T, D>(qoff, g, tid);
    RowStage<T, D> qs;
    row_load<T, D>(qs, Qh, tau_base, qoff, tid);
    row_store<T, D>(qs, lds_q, tid);
  }
  __syncthreads();

  const int kvalid = g.T - 32 * w;            // valid keys in this wave's half (may be <= 0)

  WaveState<T, D> st;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    st.m[nt] = -INFINITY;
    st.l[nt] = 0.f;
#pragma unroll
    for (int t = 0; t < C::kDTiles; ++t) st.o[nt][t] = f32x16{};
  }

  if (kvalid > 0) {
    const float c2 = a.c;
    const size_t hblk = (size_t)g.NB * 64 * D;   // elements per head in the fragment-major copies
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(reinterpret_cast<const T*>(a.Kf) + (size_t)bh * hblk, hblk * sizeof(T));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(reinterpret_cast<const PT*>(a.Vt) + (size_t)bh * hblk, hblk * sizeof(PT));
    const int kblk = 64 * D * (int)sizeof(T), vblk = 64 * D * (int)sizeof(PT);
    const int klv = w * (kblk / 2) + lane * 16, vlv = w * (vblk / 2) + lane * 16;
    // One register buffer for both operands: V(j) is requested once S(j) has
    // consumed K(j), K(j+1) once the P.V product has consumed V(j).  The second
    // wave on the SIMD covers the load latency.  Invalid idx entries are skipped.
    KFrags<T, D> kf;
    VFrags<T, D> vf;
    int slot = 0;
    while (slot < kk && (unsigned)irow[slot] >= (unsigned)g.NB) ++slot;
    if (slot < kk) {
      load_k<T, D>(kf, rk, klv, irow[slot] * kblk);
      load_v<T, D>(vf, rv, vlv, irow[slot] * vblk);
    }
    while (slot < kk) {
      int nxt = slot + 1;
      while (nxt < kk && (unsigned)irow[nxt] >= (unsigned)g.NB) ++nxt;
      f32x16 s[2];
      block_scores<T, D>(s, kf, lds_q, l32, h);
      if (nxt < kk) load_k<T, D>(kf, rk, klv, irow[nxt] * kblk);        // K(j+1) behind S(j)
      PFrag pf[2][2];
      block_softmax<T, D, FULL>(st, s, pf, c2, kvalid, h);
      block_pv<T, D>(st, vf, pf);
      if (nxt < kk) load_v<T, D>(vf, rv, vlv, irow[nxt] * vblk);        // V(j+1) behind P.V(j)
      slot = nxt;
    }
  }
  __syncthreads();                            // Q no longer read: reuse its LDS for the merge

  // ---- merge the two key halves: wave w stores N-tile w and hands N-tile 1-w
  // over through LDS (compile-time register indices only, selected per wave)
  const bool w1 = w != 0;
#pragma unroll
  for (int t = 0; t < C::kDTiles; ++t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) mrg_o[w][t * 16 + i][lane] = w1 ? st.o[0][t][i] : st.o[1][t][i];
  }
  mrg_ml[w][0][lane] = w1 ? st.m[0] : st.m[1];
  mrg_ml[w][1][lane] = w1 ? st.l[0] : st.l[1];
  __syncthreads();
  const int other = 1 - w;
  const float ma = w1 ? st.m[1] : st.m[0];
  const float la0 = w1 ? st.l[1] : st.l[0];
  const float la = pair_sum(la0);
  const float mb = mrg_ml[other][0][lane];
  const float lb0 = mrg_ml[other][1][lane];
  const float lb = pair_sum(lb0);
  const float mt = fmaxf(ma, mb);
  const float wa = (ma == -INFINITY) ? 0.f : fast_exp2(ma - mt);
  const float wb = (mb == -INFINITY) ? 0.f : fast_exp2(mb - mt);
  const float l_tot = wa * la + wb * lb;
  float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if constexpr (sizeof(T) == 2) inv *= a.vscale[bh].y;        // undo the fp16 copy's 2^t (exact)
  const int q = 32 * w + l32;
  if (q < g.T) {
    const int q_tok = tau_base + member_offset(g, q);
    const size_t orow = head_off + (size_t)q_tok * D;
#pragma unroll
    for (int t = 0; t < C::kDTiles; ++t) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * gq + i;
          const float own = w1 ? st.o[1][t][r] : st.o[0][t][r];
          v[i] = (wa * own + wb * mrg_o[other][t * 16 + r][lane]) * inv;
        }
        store4(a.O, orow + 32 * t + 8 * gq + 4 * h, a.out_f32, v[0], v[1], v[2], v[3]);
      }
    }
    if (h == 0) a.LSE[(size_t)bh * g.N + q_tok] = l_tot > 0.f ? (mt + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D>
hipError_t launch_fwd(const FwdArgs& a0, hipStream_t s) {
  FwdArgs a = a0;
  const size_t copy = (size_t)a0.BH * a0.g.NB * 64 * D * sizeof(T);   // one fragment-major copy
  a.Kf = a0.Vt;
  a.Vt = reinterpret_cast<char*>(a0.Vt) + copy;
  if constexpr (sizeof(T) == 2) {
    char* tail = reinterpret_cast<char*>(a0.Vt) + 2 * copy;
    a.vmax = reinterpret_cast<uint32_t*>(tail);
    a.vscale = reinterpret_cast<float2*>(tail + (((size_t)a0.BH * kDoChunks * 4 + 255) & ~(size_t)255));
    const hipError_t e = launch_pow2_scale(a.V, a.BH, (size_t)a.g.N * D, a.vmax, a.vscale, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kv_prep16_kernel<D>), dim3(a.BH * a.g.NB), dim3(256), 0, s, a);
  } else
    hipLaunchKernelGGL((kv_prep_kernel<T, D>), dim3(a.BH * a.g.NB), dim3(256), 0, s, a);
  if (a.g.T == 64) hipLaunchKernelGGL((attn_fwd_kernel<T, D, true>), dim3(a.BH * a.g.NB), dim3(kTileThreads), 0, s, a);
  else hipLaunchKernelGGL((attn_fwd_kernel<T, D, false>), dim3(a.BH * a.g.NB), dim3(kTileThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

size_t attn_fwd_workspace_bytes(int BH, int NB, int d, int io_f32) {
  const size_t copies = 2 * (size_t)BH * NB * d * 64 * (io_f32 ? 4 : 2);      // K and V^T, fragment-major
  if (io_f32) return copies;
  // bf16: partial maxima and the power-of-two scale of V, 256-byte aligned sections
  return copies + (((size_t)BH * kDoChunks * 4 + 255) & ~(size_t)255) + (((size_t)BH * 8 + 255) & ~(size_t)255);
}

hipError_t launch_attn_fwd(const FwdArgs& a, int io_f32, int d, hipStream_t s) {
  if (io_f32) return d == 64 ? launch_fwd<float, 64>(a, s) : launch_fwd<float, 128>(a, s);
  return d == 64 ? launch_fwd<bf16, 64>(a, s) : launch_fwd<bf16, 128>(a, s);
}

}  // namespace dsa
