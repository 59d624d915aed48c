// Block-sparse attention forward for gfx950.
//
// Computes, for every query token of a query tile, exact softmax attention over
// the keys of the key blocks that the tile kept (DSV page, gist.science/ar/paper/
// 2502.07590, section 4: stage two computes only the cues the predictor picked;
// section 3b: one selection per tile of neighbouring queries).
//
// Two kernels:
//  1. v_prep: one pass over V that writes every key block's V^T into the caller's
//     workspace in fragment-major order (the A operands of O^T = V^T P^T; for bf16
//     inputs converted to fp16 after a power-of-two scale per (b, h), below).  A
//     fragment is 64 lanes x 16 B stored lane-major, so it is copied into LDS by
//     one 1 KB direct load and read back by one conflict-free ds_read_b128.  A
//     block is gathered by ~k query tiles, so one reorganisation serves all of them.
//     K needs no such pass: its token rows go straight into LDS.
//  2. attn_fwd: one work-group of 4 waves per query tile of T <= 64 tokens, two
//     work-groups (8 waves) per CU.  The kept blocks stream through two LDS buffers
//     (K rows, XOR-swizzled, and the V^T fragments), filled by direct global->LDS
//     loads one block ahead of the computation.  Wave w = (qh, kh) takes queries
//     32qh..32qh+31 (their Q^T fragments stay in registers) against keys
//     32kh..32kh+31 of every block:
//        S^T (32 keys x 32 queries) = K Q^T          8 MFMA; K rows from LDS
//        online softmax (fp32, base 2), one query per lane
//        O^T (d x 32 queries)      += V^T P^T        d/16 MFMA; P^T taken straight
//                                                    from the S^T registers
//     The two key halves of a query half keep separate running max / sum / O and
//     are merged once, through LDS, at the end.  Four waves per tile (instead of
//     fewer, larger ones) keep half as many tiles in flight per XCD, so the
//     gathered blocks of the tiles that run together fit its L2 better.
//  2'. attn_fwd_pair (bf16, long sequences): one work-group of 8 waves per pair of
//     neighbouring query tiles, each tile computed as above by 4 waves, walking the
//     union of the two kept lists so that a block kept by both is gathered once;
//     by default chosen when one head's gathered blocks outgrow the caches
//     (kPairMinHeadBytes), where the gathers are bound by memory bandwidth; the
//     caller can force either kernel (dsa_set_fwd_kernel).
// With bf16 inputs the P.V product runs on fp16 matrix cores: v_prep converts
// V * 2^t, with one power of two per (b, h) that puts the head's largest |v| in
// [2^14, 2^15) (launch_pow2_scale), so the conversion is exact whatever the size
// of V, and the output is multiplied by 2^-t in fp32, exactly; P is rounded to
// fp16 (2^-12 relative) and the row sum adds the same fp16 probabilities (v_dot2,
// fp32 accumulation).  The probabilities are taken against a reference maximum m
// that is raised (with O and the sum rescaled) only when a block's probabilities
// would overflow fp16, which a lane's block sum shows: any reference gives the same
// softmax, since numerator and denominator share it.
#include "kernels.hpp"
#include "tiles.hpp"

#include <type_traits>

namespace dsa {

namespace {

constexpr int kFwdWaves = 4;
constexpr int kFwdThreads = 64 * kFwdWaves;

template <typename T> struct PVType;
template <> struct PVType<bf16> { typedef f16 type; };
template <> struct PVType<float> { typedef float type; };

// ------------------------------------------------------------ 1. V -> fragment-major V^T blocks
// Output per (head, block j), for each 32-key half w, the V^T A-fragments of the
// (d/32) x 2 (d tile t, key step s) pairs: chunk (w, f = (t*2+s)*PFC+p, lane)
// holds element d = 32t + lane%32 of the keys at positions 32w + 16s + 8*(lane/32)
// + PE*p + e (key = 16*(pos/16) + perm16(pos%16): the order in which the S^T
// result registers hold the probabilities).  Positions >= T are zero.
// One work-group of 256 threads per (head, block); all global accesses are
// 16-byte chunks.
template <typename T, int D>
__global__ __launch_bounds__(256) void v_prep_kernel(FwdArgs a) {
  typedef typename PVType<T>::type PT;
  constexpr int CE = Elem<T>::kChunkElems;                     // == Elem<PT>::kChunkElems
  constexpr int CPR = D / CE;
  constexpr int PFC = Elem<PT>::kFragChunks;
  static_assert(Elem<PT>::kChunkElems == CE, "square register transpose");
  const Geo g = a.g;
  const int bj = blockIdx.x;
  const int bh = bj / g.NB, j = bj - bh * g.NB;
  const T* __restrict__ Vh = reinterpret_cast<const T*>(a.V) + (size_t)bh * g.N * D;
  const int base = tile_base(g, j);
  u32x4* __restrict__ vo = reinterpret_cast<u32x4*>(reinterpret_cast<PT*>(a.Vt) + (size_t)bj * 64 * D);
  // (64 / CE) position groups x CPR chunk columns, one CE x CE block each
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

// Same output for bf16 inputs (fp16, scaled), through LDS: the block's V rows are
// staged with coalesced 16-byte loads (every row read as one 256-byte run) into an
// XOR-swizzled row-major tile; each V^T output chunk (8 keys of one d; with the
// perm16 order two runs of 4 consecutive keys) is then two transposing LDS reads,
// scaled by the head's 2^t and converted to fp16.  Every global store is coalesced.
template <int D>
__global__ __launch_bounds__(256) void v_prep16_kernel(FwdArgs a) {
  typedef bf16 T;
  typedef f16 PT;
  using C = TileCfg<T, D>;
  constexpr int CE = C::kCE;                                   // 8 elements per chunk
  constexpr int CPR = C::kCPR;
  constexpr int NCH = 64 * CPR;                                // chunks of a 64-row tile
  static_assert(CE == 8 && Elem<PT>::kFragChunks == 1, "16-bit elements");
  __shared__ u32x4 vt[NCH];
  const Geo g = a.g;
  const int bj = blockIdx.x;
  const int bh = bj / g.NB, j = bj - bh * g.NB;
  const T* __restrict__ Vh = reinterpret_cast<const T*>(a.V) + (size_t)bh * g.N * D;
  const int base = tile_base(g, j);
  const int tid = threadIdx.x;
  const float vup = a.vscale[bh].x;                            // 2^t of this head
#pragma unroll
  for (int i = 0; i < NCH / 256; ++i) {
    const int idx = tid + 256 * i, r = idx / CPR, c = idx % CPR;
    u32x4 vv = u32x4{0, 0, 0, 0};
    if (r < g.T) vv = *reinterpret_cast<const u32x4*>(Vh + (size_t)(base + member_offset(g, r)) * D + c * CE);
    vt[row_slot<T, D>(r, c)] = vv;
  }
  __syncthreads();
  u32x4* __restrict__ vo = reinterpret_cast<u32x4*>(reinterpret_cast<PT*>(a.Vt) + (size_t)bj * 64 * D);
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
  static constexpr int kSteps = D / 16;                  // reduction steps over d (S^T product)
  static constexpr int kDTiles = D / 32;                 // 32-row tiles over d (O^T product)
  static constexpr int kFC = Elem<T>::kFragChunks;
  static constexpr int kPFC = Elem<PT>::kFragChunks;
  static constexpr int kKBytes = 64 * D * (int)sizeof(T);          // one K tile (row-major)
  static constexpr int kVBytes = 64 * D * (int)sizeof(PT);         // one V^T block (fragment-major)
  static constexpr int kVFrag = kDTiles * 2 * kPFC;                // V^T chunks per lane per key half
  static constexpr int kVInstr = kVBytes / 1024 / kFwdWaves;       // 1 KB direct loads per wave and block
};
// two work-groups per CU for 16-bit inputs; the fp32 variants (parity checks only)
// need 128 KB of LDS and more than 256 registers and run one
template <typename T> constexpr int kFwdWavesPerEU = sizeof(T) == 2 ? 2 : 1;

// wave state: O^T over the wave's 32 queries (one d tile per register block), the
// reference maximum (log2 units) and the lane's partial row sum
template <typename T, int D>
struct WaveState {
  f32x16 o[FwdCfg<T, D>::kDTiles];
  float m, l;
};

// an empty asm that uses a value: the compiler must have computed it at this
// point of the program (keeps vector work inside the region where it overlaps the
// matrix cores instead of sinking it to its later use)
template <typename V>
__device__ __forceinline__ void pin(const V& v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(v));                  // device pass only: the host pass never runs it
#else
  (void)v;
#endif
}

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

// Probabilities of one block's S^T (lane: query l%32, keys 8g + 4h + i of the
// wave's half in register 4g+i) against the reference maximum m: P = exp2(S c - m),
// as the P^T fragments of the two key steps, and the lane's block sum.  Padding keys
// (T < 64) give 0.  m is only a reference, not necessarily the running maximum: any
// m works (numerator and denominator share it) as long as no P overflows the P.V
// element type, which the caller checks on the block sum.
template <typename T, int D, bool FULL>
__device__ __forceinline__ float block_probs(const WaveState<T, D>& st, f32x16& s,
                                             typename Elem<typename FwdCfg<T, D>::PT>::frag (&pf)[2], float c2,
                                             int kvalid, int h) {
  typedef typename FwdCfg<T, D>::PT PT;
  if constexpr (!FULL) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (8 * (i >> 2) + 4 * h + (i & 3) >= kvalid) s[i] = -INFINITY;
  }
  const float mneg = -st.m;
  float bs = 0.f;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(fmaf(s[8 * ks + e], c2, mneg));
    pf[ks] = to_frag(pv, (PT*)nullptr);
    bs = frag_sum(pf[ks], bs);
  }
  return bs;
}

// The reference maximum is raised to the row maxima of S^T (for every lane) and O
// and the row sum are rescaled; called when some lane's block sum was not below
// kSumBound (an overflowing, infinite or NaN probability, or the first block).
template <typename T, int D>
__device__ __forceinline__ void raise_max(WaveState<T, D>& st, const f32x16& s, float c2) {
  float mb = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) mb = fmaxf(fmaxf(mb, s[i]), s[i + 1]);
  mb = fmaxf(mb, s[15]);
  mb = pair_max(mb);
  const float mt = fmaxf(st.m, mb * c2);      // c2 > 0 (the host rejects scale <= 0)
  const float alpha = (st.m == -INFINITY || mt == -INFINITY) ? 0.f : fast_exp2(st.m - mt);
  st.m = mt;
  st.l *= alpha;
#pragma unroll
  for (int t = 0; t < FwdCfg<T, D>::kDTiles; ++t) st.o[t] *= alpha;
}

// a lane's sum of 16 probabilities below 2^15 guarantees that none of them
// overflows fp16 (and that none is inf or NaN)
constexpr float kSumBound = 32768.0f;

// One work-group of 4 waves per query tile (see the file comment).  LDS: two K
// tiles and two V^T blocks; after the block loop the same memory holds the merge
// of the two key halves.
// Iteration j (blocks in idx order, invalid ids skipped): wait for K(j+1) and V(j)
// to land, barrier (every wave is done with iteration j-1), request K(j+2) into K
// slot j%2 and V(j+1) into V slot (j+1)%2, read the wave's K(j+1) and V(j)
// fragments, then S(j+1) = K(j+1) Q^T on the matrix cores under P(j) =
// exp2(S(j) c - m) on the vector ALU, and O += V(j)^T P(j)^T.  The reference
// maximum m is not updated per block: it is raised (and O rescaled) only when a
// block's probabilities would overflow fp16, which the block sums show; below that
// any reference gives the same softmax.
template <typename T, int D, bool FULL>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(kFwdWavesPerEU<T>, 2)))
void attn_fwd_kernel(FwdArgs a) {
  using C = FwdCfg<T, D>;
  typedef typename C::PT PT;
  typedef typename Elem<T>::frag Frag;
  typedef typename Elem<PT>::frag PFrag;
  using TC = TileCfg<T, D>;
  constexpr int kKB = C::kKBytes, kVB = C::kVBytes;
  constexpr int kHalfT = C::kDTiles / 2 > 0 ? C::kDTiles / 2 : 1;      // d tiles each key half stores
  constexpr int kMrgBytes = kFwdWaves * (kHalfT * 16 * 64 + 2 * 64) * 4;
  static_assert(kMrgBytes <= 2 * (kKB + kVB), "merge area fits the block buffers");
  __shared__ __attribute__((aligned(16))) char smem[2 * (kKB + kVB)];

  const Geo g = a.g;
  const int L = blockIdx.x;                 // natural order (see common.hpp)
  const int bh = L / g.NB;
  const int tau = L - bh * g.NB;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int qh = w & 1, kh = w >> 1;

  const size_t head_off = (size_t)bh * g.N * D;
  const T* __restrict__ Qh = reinterpret_cast<const T*>(a.Q) + head_off;
  const int* __restrict__ irow = a.idx + ((size_t)bh * g.NB + tau) * a.kmax;
  int kk = a.kvec[bh];
  kk = kk < 1 ? 1 : (kk > a.kmax ? a.kmax : kk);
  const int tau_base = tile_base(g, tau);

  // this lane's query (column l%32 of S^T): Q^T B-fragments, elements 16s + 8h + ..
  const int qr = 32 * qh + l32;
  const bool q_ok = qr < g.T;
  const int q_tok = tau_base + (q_ok ? member_offset(g, qr) : 0);
  Frag qf[C::kSteps];
  {
    const T* qrow = Qh + (size_t)q_tok * D;
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      u32x4 ch[C::kFC];
#pragma unroll
      for (int p = 0; p < C::kFC; ++p)
        ch[p] = q_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * h + TC::kCE * p) : u32x4{0, 0, 0, 0};
      qf[s] = frag_from_chunks(ch, (T*)nullptr);
    }
  }

  const int kvalid = g.T - 32 * kh;           // valid keys in this wave's half (may be <= 0)
  WaveState<T, D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int t = 0; t < C::kDTiles; ++t) st.o[t] = f32x16{};

  // direct loads: K rows (swizzled) and the V^T block, each wave its share
  int koff[DmaCfg<T, D, kFwdWaves>::kPer];
  dma_offsets<T, D, kFwdWaves>(koff, g, w, lane);
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(reinterpret_cast<const T*>(a.K) + head_off, (size_t)g.N * D * sizeof(T));
  const size_t hblk = (size_t)g.NB * 64 * D;   // elements per head in the V^T copy
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(reinterpret_cast<const PT*>(a.Vt) + (size_t)bh * hblk, hblk * sizeof(PT));
  auto req_k = [&](int base, int slot) {      // K tile whose first token is `base`
    dma_tile<T, D, kFwdWaves>(reinterpret_cast<u32x4*>(smem + slot * kKB), rk, base * D * (int)sizeof(T), koff, w);
  };
  auto req_v = [&](int blk, int slot) {
    dma_linear<C::kVInstr, kFwdWaves>(reinterpret_cast<u32x4*>(smem + 2 * kKB + slot * kVB), rv, blk * kVB, w, lane);
  };
  const float c2 = a.c;
  // K fragments (A = rows 32kh + l32 of the K tile in `slot`) and S^T = K Q^T
  auto read_k = [&](int slot, Frag (&kf)[C::kSteps]) {
    const u32x4* lk = reinterpret_cast<const u32x4*>(smem + slot * kKB);
#pragma unroll
    for (int k = 0; k < C::kSteps; ++k) kf[k] = frag_row<T, D>(lk, 32 * kh + l32, k, h);
  };
  auto scores_from = [&](const Frag (&kf)[C::kSteps], f32x16& s) {
    s = f32x16{};
#pragma unroll
    for (int k = 0; k < C::kSteps; ++k) s = mma_step(kf[k], qf[k], s);
  };
  auto read_v = [&](int slot, PFrag (&vf)[C::kDTiles][2]) {
    const u32x4* lv = reinterpret_cast<const u32x4*>(smem + 2 * kKB + slot * kVB) + (size_t)kh * C::kVFrag * 64 + lane;
#pragma unroll
    for (int t = 0; t < C::kDTiles; ++t) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 ch[C::kPFC];
#pragma unroll
        for (int p = 0; p < C::kPFC; ++p) ch[p] = lv[((t * 2 + ks) * C::kPFC + p) * 64];
        vf[t][ks] = frag_from_chunks(ch, (PT*)nullptr);
      }
    }
  };

  // the kept blocks in idx order (invalid entries skipped); b0 = block j, b1 = j + 1
  TileList ids;
  ids.init(irow, kk, g, lane);
  int b0 = ids.next(lane);
  const int base0 = ids.last_base;
  int b1 = b0 >= 0 ? ids.next(lane) : -1;
  f32x16 sa, sb;                              // S^T of block j: sa for even j, sb for odd j
  if (b0 >= 0) {
    req_k(base0, 0);
    req_v(b0, 0);
    if (b1 >= 0) req_k(ids.last_base, 1);
    dma_wait();
    __syncthreads();
    if (kvalid > 0) {
      Frag kf[C::kSteps];
      read_k(0, kf);
      scores_from(kf, sa);
    }
  }
  // one iteration; the loop runs it for even and odd j in turn, so the buffer
  // slots are constants (immediate LDS offsets) and the scores of the next block
  // land in the other register set (no copy)
  auto step = [&](auto parity, f32x16& scur, f32x16& snext) __attribute__((always_inline)) {
    constexpr int p = decltype(parity)::value;          // j % 2
    const int b2 = b1 >= 0 ? ids.next(lane) : -1;
    dma_wait();
    __syncthreads();                          // K(j+1), V(j) landed; iteration j-1 done everywhere
    if (b2 >= 0) req_k(ids.last_base, p);
    if (b1 >= 0) req_v(b1, 1 - p);
    if (kvalid > 0) {
      // every LDS operand of the iteration is requested first: its latency is paid
      // once, under the vector work, instead of before each product (for the last
      // block the scores of a stale K slot are computed and ignored)
      Frag kf[C::kSteps];
      PFrag vf[C::kDTiles][2];
      read_k(1 - p, kf);
      read_v(p, vf);
      __builtin_amdgcn_sched_barrier(0);
      scores_from(kf, snext);
      PFrag pf[2];
      float bs = block_probs<T, D, FULL>(st, scur, pf, c2, kvalid, h);
#pragma unroll
      for (int i = 0; i < C::kSteps; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // six VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      }
      pin(pf[0]);
      pin(pf[1]);
      pin(bs);
      __builtin_amdgcn_sched_barrier(0);
      if (ballot(!(bs < kSumBound))) {        // rare: raise the reference maximum first
        raise_max(st, scur, c2);
        bs = block_probs<T, D, FULL>(st, scur, pf, c2, kvalid, h);
      }
      st.l += bs;
#pragma unroll
      for (int t = 0; t < C::kDTiles; ++t) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) st.o[t] = mma_step(vf[t][ks], pf[ks], st.o[t]);
      }
    }
    b0 = b1;
    b1 = b2;
    return b0 >= 0;
  };
  if (b0 >= 0) {
    while (step(std::integral_constant<int, 0>{}, sa, sb) && step(std::integral_constant<int, 1>{}, sb, sa)) {
    }
  }
  __syncthreads();                            // the buffers are free: reuse them for the merge

  // ---- merge the two key halves of each query half: wave (qh, kh) stores d tiles
  // [kh*DT/2, (kh+1)*DT/2) and hands the others to its partner (qh, 1-kh) through LDS
  float* mrg = reinterpret_cast<float*>(smem);
  float* mine = mrg + w * (kHalfT * 16 * 64 + 2 * 64);
  const float* theirs = mrg + (w ^ 2) * (kHalfT * 16 * 64 + 2 * 64);
  const int t0 = C::kDTiles >= 2 ? kh * kHalfT : 0;            // first d tile this wave stores
  const int o0 = C::kDTiles >= 2 ? (1 - kh) * kHalfT : 0;      // first d tile the partner stores
#pragma unroll
  for (int t = 0; t < kHalfT; ++t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = st.o[0][i];
#pragma unroll
      for (int u = 0; u < C::kDTiles; ++u)
        if (u == o0 + t) v = st.o[u][i];
      mine[(t * 16 + i) * 64 + lane] = v;
    }
  }
  mine[kHalfT * 16 * 64 + lane] = st.m;
  mine[kHalfT * 16 * 64 + 64 + lane] = st.l;
  __syncthreads();
  const float ma = st.m, la = pair_sum(st.l);
  const float mb = theirs[kHalfT * 16 * 64 + lane];
  const float lb = pair_sum(theirs[kHalfT * 16 * 64 + 64 + lane]);
  const float mt = fmaxf(ma, mb);
  const float wa = (ma == -INFINITY) ? 0.f : fast_exp2(ma - mt);
  const float wb = (mb == -INFINITY) ? 0.f : fast_exp2(mb - mt);
  const float l_tot = wa * la + wb * lb;
  float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if constexpr (sizeof(T) == 2) inv *= a.vscale[bh].y;        // undo the fp16 copy's 2^t (exact)
  if (q_ok) {
    const size_t orow = head_off + (size_t)q_tok * D;
#pragma unroll
    for (int t = 0; t < kHalfT; ++t) {
      const int td = t0 + t;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * gq + i;
          float own = st.o[0][r];
#pragma unroll
          for (int u = 0; u < C::kDTiles; ++u)
            if (u == td) own = st.o[u][r];
          v[i] = (wa * own + wb * theirs[(t * 16 + r) * 64 + lane]) * inv;
        }
        store4(a.O, orow + 32 * td + 8 * gq + 4 * h, a.out_f32, v[0], v[1], v[2], v[3]);
      }
    }
    if (kh == 0 && h == 0) a.LSE[(size_t)bh * g.N + q_tok] = l_tot > 0.f ? (mt + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// work-group barrier that orders LDS accesses only: unlike __syncthreads() it does
// not wait for this wave's global->LDS loads still in flight (the caller waits for
// exactly the ones it needs first)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);         // lgkmcnt(0): this wave's LDS accesses are done
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::: "memory");
#endif
  __builtin_amdgcn_s_barrier();
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::: "memory");
#endif
}

// wait until at most N of this wave's vector-memory loads are in flight
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// The kept-block lists of two query tiles walked as one ascending union: each step
// yields a block and a mask (bit g: tile g kept it), so a block kept by both is
// loaded once.  Every list element is yielded exactly once whatever the order of
// the lists (a list that is not ascending only loses sharing), invalid entries are
// skipped (IdList).  Wave-uniform.
struct PairMerge {
  IdList a, b;
  int ha, hb;                                 // current heads (-1: list done)
  __device__ __forceinline__ void init(const int* la, const int* lb, int k, int nb, int lane) {
    a.init(la, k, nb, lane);
    ha = a.next(lane);
    if (lb != nullptr) {
      b.init(lb, k, nb, lane);
      hb = b.next(lane);
    } else {
      hb = -1;
    }
  }
  __device__ __forceinline__ int next(int lane, int& mask) {
    if (ha < 0 && hb < 0) {
      mask = 0;
      return -1;
    }
    int blk;
    if (hb < 0 || (ha >= 0 && ha < hb)) {
      blk = ha, mask = 1;
      ha = a.next(lane);
    } else if (ha < 0 || hb < ha) {
      blk = hb, mask = 2;
      hb = b.next(lane);
    } else {
      blk = ha, mask = 3;
      ha = a.next(lane);
      hb = b.next(lane);
    }
    return blk;
  }
};

// Which attention kernel a bf16 forward runs: one head's gathered blocks (K rows
// and the fp16 V^T copy, NB * 64 * d * 4 bytes) below this size stay mostly in the
// caches, and the one-tile kernel with its deeper per-wave pipeline is faster;
// above it the gathers are bound by L2-miss bandwidth and the tile-pair kernel,
// which gathers a block kept by both tiles once, is faster.  Measured crossover at
// d = 128 (5 % kept, 1x8x8 tiles): NB = 1024 (32 MiB) pair 7 % slower, NB = 1536
// (48 MiB) 10 % faster, NB = 8192 22 % faster.
constexpr size_t kPairMinHeadBytes = (size_t)48 << 20;

// bf16 inputs: one work-group of 8 waves per pair of neighbouring query tiles
// (waves 4g..4g+3 compute tile g exactly as above: wave (qh, kh) takes 32 queries
// against a 32-key half), one work-group per CU.  The two tiles' kept blocks are
// walked as one union (PairMerge): a block that both kept -- neighbours along the
// tile grid's slowest axis keep many of the same blocks -- is gathered once for
// both, cutting the bytes gathered per attended pair.  The blocks stream through a
// ring of four LDS slots [K rows | V^T fragments] filled three blocks ahead.
// Iteration j: wait for block j (blocks j+1, j+2 may stay in flight), barrier (every
// wave is done with iteration j-1, so its slot is free), request block j+3 into it,
// and for each tile that kept block j: S = K Q^T, P against the reference maximum,
// O += V^T P^T.
template <int D, bool FULL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_pair_kernel(FwdArgs a) {
  typedef bf16 T;
  using C = FwdCfg<T, D>;
  typedef typename C::PT PT;
  typedef typename Elem<T>::frag Frag;
  typedef typename Elem<PT>::frag PFrag;
  using TC = TileCfg<T, D>;
  constexpr int W = 8;
  constexpr int NBUF = 4;
  constexpr int kKB = C::kKBytes, kVB = C::kVBytes, kSlot = kKB + kVB;
  constexpr int kVInstr = kVB / 1024 / W;                      // 1 KB direct loads per wave and block (V)
  constexpr int kDmaPerWave = DmaCfg<T, D, W>::kPer + kVInstr;
  static_assert(kVB % (1024 * W) == 0, "V^T block splits evenly over the waves");
  constexpr int kHalfT = C::kDTiles / 2 > 0 ? C::kDTiles / 2 : 1;
  constexpr int kMrgFloats = kHalfT * 16 * 64 + 2 * 64;
  static_assert(W * kMrgFloats * 4 <= NBUF * kSlot, "merge area fits the ring");
  __shared__ __attribute__((aligned(16))) char smem[NBUF * kSlot];

  const Geo g = a.g;
  const int L = blockIdx.x;                 // natural order: neighbouring pairs of one head
  const int bh = L / a.npairs;
  const int pi = L - bh * a.npairs;
  // pair pi -> tiles tau0 = (outer * E + 2p) * S + r and tau0 + S (if 2p + 1 < E)
  const int r = pi % a.pair_s, qo = pi / a.pair_s;
  const int pp = qo % a.pair_p2, outer = qo / a.pair_p2;
  const int tau0 = (outer * a.pair_e + 2 * pp) * a.pair_s + r;
  const int tau1 = 2 * pp + 1 < a.pair_e ? tau0 + a.pair_s : -1;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int grp = w >> 2, qh = w & 1, kh = (w >> 1) & 1;
  const int tau = grp == 0 ? tau0 : tau1;
  const bool active = tau >= 0;

  const size_t head_off = (size_t)bh * g.N * D;
  const T* __restrict__ Qh = reinterpret_cast<const T*>(a.Q) + head_off;
  const int* __restrict__ ibase = a.idx + (size_t)bh * g.NB * a.kmax;
  int kk = a.kvec[bh];
  kk = kk < 1 ? 1 : (kk > a.kmax ? a.kmax : kk);

  // this lane's query (column l%32 of S^T) of its group's tile: Q^T B-fragments
  const int qr = 32 * qh + l32;
  const bool q_ok = active && qr < g.T;
  const int q_tok = (active ? tile_base(g, tau) : 0) + (q_ok ? member_offset(g, qr) : 0);
  Frag qf[C::kSteps];
  {
    const T* qrow = Qh + (size_t)q_tok * D;
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      u32x4 ch[C::kFC];
#pragma unroll
      for (int p = 0; p < C::kFC; ++p)
        ch[p] = q_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * h + TC::kCE * p) : u32x4{0, 0, 0, 0};
      qf[s] = frag_from_chunks(ch, (T*)nullptr);
    }
  }

  const int kvalid = g.T - 32 * kh;           // valid keys in this wave's half (may be <= 0)
  WaveState<T, D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int t = 0; t < C::kDTiles; ++t) st.o[t] = f32x16{};

  int koff[DmaCfg<T, D, W>::kPer];
  dma_offsets<T, D, W>(koff, g, w, lane);
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(reinterpret_cast<const T*>(a.K) + head_off, (size_t)g.N * D * sizeof(T));
  const size_t hblk = (size_t)g.NB * 64 * D;
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(reinterpret_cast<const PT*>(a.Vt) + (size_t)bh * hblk, hblk * sizeof(PT));
  auto request = [&](int blk, int slot) {
    char* b = smem + slot * kSlot;
    dma_tile<T, D, W>(reinterpret_cast<u32x4*>(b), rk, tile_base(g, blk) * D * (int)sizeof(T), koff, w);
    dma_linear<kVInstr, W>(reinterpret_cast<u32x4*>(b + kKB), rv, blk * kVB, w, lane);
  };
  const float c2 = a.c;

  PairMerge mg;
  mg.init(ibase + (size_t)tau0 * a.kmax, tau1 >= 0 ? ibase + (size_t)tau1 * a.kmax : nullptr, kk, g.NB, lane);
  int blk[NBUF], msk[NBUF];                   // entries j .. j+NBUF-1 of the union
#pragma unroll
  for (int i = 0; i < NBUF; ++i) blk[i] = -1, msk[i] = 0;
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i) {
    if (i == 0 || blk[i - 1] >= 0) blk[i] = mg.next(lane, msk[i]);
    if (blk[i] >= 0) request(blk[i], i);
  }
  int slot = 0;
  while (blk[0] >= 0) {
    // block j landed; blocks j+1, j+2 may still be in flight
    if (blk[2] >= 0) vm_wait<2 * kDmaPerWave>();
    else if (blk[1] >= 0) vm_wait<kDmaPerWave>();
    else dma_wait();
    lds_barrier();                            // iteration j-1 done everywhere: its slot is free
    if (blk[2] >= 0) blk[3] = mg.next(lane, msk[3]);
    else blk[3] = -1, msk[3] = 0;
    if (blk[3] >= 0) request(blk[3], slot == 0 ? NBUF - 1 : slot - 1);
    if (active && ((msk[0] >> grp) & 1) && kvalid > 0) {
      const u32x4* lk = reinterpret_cast<const u32x4*>(smem + slot * kSlot);
      const u32x4* lv = reinterpret_cast<const u32x4*>(smem + slot * kSlot + kKB) + (size_t)kh * C::kVFrag * 64 + lane;
      Frag kf[C::kSteps];
#pragma unroll
      for (int k = 0; k < C::kSteps; ++k) kf[k] = frag_row<T, D>(lk, 32 * kh + l32, k, h);
      PFrag vf[C::kDTiles][2];
#pragma unroll
      for (int t = 0; t < C::kDTiles; ++t) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u32x4 ch[C::kPFC];
#pragma unroll
          for (int p = 0; p < C::kPFC; ++p) ch[p] = lv[((t * 2 + ks) * C::kPFC + p) * 64];
          vf[t][ks] = frag_from_chunks(ch, (PT*)nullptr);
        }
      }
      f32x16 sc = f32x16{};
#pragma unroll
      for (int k = 0; k < C::kSteps; ++k) sc = mma_step(kf[k], qf[k], sc);
      PFrag pf[2];
      float bs = block_probs<T, D, FULL>(st, sc, pf, c2, kvalid, h);
      if (ballot(!(bs < kSumBound))) {        // rare: raise the reference maximum first
        raise_max(st, sc, c2);
        bs = block_probs<T, D, FULL>(st, sc, pf, c2, kvalid, h);
      }
      st.l += bs;
#pragma unroll
      for (int t = 0; t < C::kDTiles; ++t) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) st.o[t] = mma_step(vf[t][ks], pf[ks], st.o[t]);
      }
    }
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) blk[i] = blk[i + 1], msk[i] = msk[i + 1];
    slot = slot == NBUF - 1 ? 0 : slot + 1;
  }
  __syncthreads();                            // the ring is free: reuse it for the merge

  // ---- merge the two key halves of each query half (partner: the other kh of the group)
  float* mrg = reinterpret_cast<float*>(smem);
  float* mine = mrg + w * kMrgFloats;
  const float* theirs = mrg + (w ^ 2) * kMrgFloats;
  const int t0 = C::kDTiles >= 2 ? kh * kHalfT : 0;
  const int o0 = C::kDTiles >= 2 ? (1 - kh) * kHalfT : 0;
#pragma unroll
  for (int t = 0; t < kHalfT; ++t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = st.o[0][i];
#pragma unroll
      for (int u = 0; u < C::kDTiles; ++u)
        if (u == o0 + t) v = st.o[u][i];
      mine[(t * 16 + i) * 64 + lane] = v;
    }
  }
  mine[kHalfT * 16 * 64 + lane] = st.m;
  mine[kHalfT * 16 * 64 + 64 + lane] = st.l;
  __syncthreads();
  const float ma = st.m, la = pair_sum(st.l);
  const float mb = theirs[kHalfT * 16 * 64 + lane];
  const float lb = pair_sum(theirs[kHalfT * 16 * 64 + 64 + lane]);
  const float mt = fmaxf(ma, mb);
  const float wa = (ma == -INFINITY) ? 0.f : fast_exp2(ma - mt);
  const float wb = (mb == -INFINITY) ? 0.f : fast_exp2(mb - mt);
  const float l_tot = wa * la + wb * lb;
  float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  inv *= a.vscale[bh].y;                      // undo the fp16 copy's 2^t (exact)
  if (q_ok) {
    const size_t orow = head_off + (size_t)q_tok * D;
#pragma unroll
    for (int t = 0; t < kHalfT; ++t) {
      const int td = t0 + t;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 4 * gq + i;
          float own = st.o[0][rr];
#pragma unroll
          for (int u = 0; u < C::kDTiles; ++u)
            if (u == td) own = st.o[u][rr];
          v[i] = (wa * own + wb * theirs[(t * 16 + rr) * 64 + lane]) * inv;
        }
        store4(a.O, orow + 32 * td + 8 * gq + 4 * h, a.out_f32, v[0], v[1], v[2], v[3]);
      }
    }
    if (kh == 0 && h == 0) a.LSE[(size_t)bh * g.N + q_tok] = l_tot > 0.f ? (mt + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D>
hipError_t launch_fwd(const FwdArgs& a0, hipStream_t s) {
  typedef typename PVType<T>::type PT;
  FwdArgs a = a0;
  const size_t copy = (size_t)a0.BH * a0.g.NB * 64 * D * sizeof(PT);   // the fragment-major V^T copy
  if constexpr (sizeof(T) == 2) {
    char* tail = reinterpret_cast<char*>(a0.Vt) + copy;
    a.vmax = reinterpret_cast<uint32_t*>(tail);
    a.vscale = reinterpret_cast<float2*>(tail + (((size_t)a0.BH * kDoChunks * 4 + 255) & ~(size_t)255));
    const hipError_t e = launch_pow2_scale(a.V, a.BH, (size_t)a.g.N * D, a.vmax, a.vscale, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((v_prep16_kernel<D>), dim3(a.BH * a.g.NB), dim3(256), 0, s, a);
    const Geo& g = a.g;
    if (attn_fwd_kernel_for(g, D, 0, a.kernel) == 1) {
      if (g.T == 64) hipLaunchKernelGGL((attn_fwd_kernel<T, D, true>), dim3(a.BH * g.NB), dim3(kFwdThreads), 0, s, a);
      else hipLaunchKernelGGL((attn_fwd_kernel<T, D, false>), dim3(a.BH * g.NB), dim3(kFwdThreads), 0, s, a);
      return hipGetLastError();
    }
    // pairs of tiles along the slowest tile-grid axis with more than one tile
    if (g.gt > 1) a.pair_s = g.gh * g.gw, a.pair_e = g.gt;
    else if (g.gh > 1) a.pair_s = g.gw, a.pair_e = g.gh;
    else a.pair_s = 1, a.pair_e = g.gw;
    a.pair_p2 = (a.pair_e + 1) / 2;
    a.npairs = g.NB / a.pair_e * a.pair_p2;
    const dim3 grid((unsigned)(a.BH * a.npairs));
    if (g.T == 64) hipLaunchKernelGGL((attn_fwd_pair_kernel<D, true>), grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_pair_kernel<D, false>), grid, dim3(512), 0, s, a);
    return hipGetLastError();
  } else {
    hipLaunchKernelGGL((v_prep_kernel<T, D>), dim3(a.BH * a.g.NB), dim3(256), 0, s, a);
  }
  if (a.g.T == 64) hipLaunchKernelGGL((attn_fwd_kernel<T, D, true>), dim3(a.BH * a.g.NB), dim3(kFwdThreads), 0, s, a);
  else hipLaunchKernelGGL((attn_fwd_kernel<T, D, false>), dim3(a.BH * a.g.NB), dim3(kFwdThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int attn_fwd_kernel_for(const Geo& g, int d, int io_f32, int setting) {
  if (io_f32) return 1;
  if (setting == 1 || setting == 2) return setting;
  return (size_t)g.NB * 64 * d * 4 >= kPairMinHeadBytes ? 2 : 1;
}

size_t attn_fwd_workspace_bytes(int BH, int NB, int d, int io_f32) {
  const size_t copy = (size_t)BH * NB * d * 64 * (io_f32 ? 4 : 2);       // V^T, fragment-major
  if (io_f32) return copy;
  // bf16: partial maxima and the power-of-two scale of V, 256-byte aligned sections
  return copy + (((size_t)BH * kDoChunks * 4 + 255) & ~(size_t)255) + (((size_t)BH * 8 + 255) & ~(size_t)255);
}

hipError_t launch_attn_fwd(const FwdArgs& a, int io_f32, int d, hipStream_t s) {
  if (io_f32) return d == 64 ? launch_fwd<float, 64>(a, s) : launch_fwd<float, 128>(a, s);
  return d == 64 ? launch_fwd<bf16, 64>(a, s) : launch_fwd<bf16, 128>(a, s);
}

}  // namespace dsa
