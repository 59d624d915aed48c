// Block-sparse attention backward for gfx950, block mask held fixed.
//
// The DSV page (gist.science/ar/paper/2502.07590) trains the video DiT with the
// sparse attention in its second stage (section 4), so the kept blocks need
// exact gradients: with P recomputed from the forward's log-sum-exp,
//   D_i = dO_i . O_i,  dS_in = P_in (dO_i . v_n - D_i),
//   dQ_i = scale sum_n dS_in k_n,  dK_n = scale sum_i dS_in q_i,  dV_n = sum_i P_in dO_i.
//
// Precision: P and dS are computed in fp32 inside the kernels.  With bf16 inputs
// every product runs on fp16 matrix cores with operands that are exact: dO, V, Q
// and K enter as fp16 copies scaled by a power of two per (b, h) (or, for the
// operands a work-group keeps in registers, per 64-row block), which converts
// every bf16 value exactly whatever the size of the tensors (scale.hip), and the
// products are brought back by the inverse powers in fp32, exactly.  P in [0, 1]
// is rounded to fp16 (2^-12 relative).  dS is rounded to fp16 after a power of
// two 2^u per (b, h) chosen from bounds that hold for every element (ds_exponent
// below), so it neither overflows nor leaves fp16's normal range for any value
// within 2^-29 of the bound.  fp32 inputs use fp32 throughout.  D is taken from
// O as passed in (the fp32 forward output).
//
// No floating-point atomics, so results are bit-reproducible:
//   1. prep:     the per-(b, h) scale of the fp16 dO copy, then D (fp32) for
//                every token, the scaled copy, and max |D| per (b, h);
//   2. reverse index of the block mask: a bitmap row per key block (bit tau set
//      if tile tau kept it; integer OR is order-free), popcounts, a per-head
//      exclusive scan, and an ascending compaction into CSC lists;
//   3. dK/dV:    one work-group (4 waves, 16 keys each) per key block walks the
//                query tiles that kept it (S = Q K^T and dP = dO V^T with K, V in
//                registers; dV += P^T dO and dK += dS^T Q with Q / dO read
//                transposed from LDS);
//   4. dQ:       one work-group (4 waves, 16 queries each) per query tile walks
//                its kept blocks (S^T = K Q^T, dP^T = V dO^T; dQ^T += K^T dS^T).
// Both stream their tiles through LDS filled by direct global->LDS loads, one
// tile ahead of the computation (double-buffered; dQ's V tile, read only in its
// first products, single-buffered).
#include "kernels.hpp"
#include "tiles.hpp"

namespace dsa {

namespace {

// ---------------------------------------------------------------- 1. scale of the fp16 dO copy
// dO and V enter fp16 products (dV = P^T dO, dP = dO V^T): each is converted
// after multiplying it by its own power of two per (b, h) (launch_pow2_scale), so
// the conversion is exact whatever the size of the values, and dP and dV are
// multiplied back by the inverse powers in fp32, exactly.

// Exponent u of the fp16 dS (bf16 inputs).  dS = P (dP - D) with P in [0, 1];
// |dP| <= d max|dO| max|V| < 2^(30 - s - t + log2 d), where 2^s and 2^t are the
// power-of-two scales of dO and V (they put each maximum below 2^15), and |D| is
// at most the max |D| the prepare phase measured.  With M the larger of the two
// exponents |dS| < 2^(M+1), so dS * 2^u with u = 14 - M stays below 2^15.  Scaling
// dO or V by a power of two moves u the opposite way and leaves the fp16 dS bit
// for bit unchanged.  A non-finite max |D| gives u = 0.
__device__ __forceinline__ int ds_exponent(float2 dsc, float2 vsc, uint32_t dabs, int log2d) {
  const int s = (int)(__float_as_uint(dsc.x) >> 23) - 127;
  const int t = (int)(__float_as_uint(vsc.x) >> 23) - 127;
  if (dabs >= 0x7f800000u) return 0;
  int M = 30 - s - t + log2d;
  if (dabs != 0u) M = max(M, (int)(dabs >> 23) - 126);    // |D| < 2^(exponent + 1)
  const int u = 14 - M;
  return u < -100 ? -100 : (u > 100 ? 100 : u);
}
// 2^e as a float, |e| <= 126
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }
template <int D> constexpr int kLog2D = D == 64 ? 6 : 7;

// Power-of-two exponent for a 64-row block held in registers (the same rule as
// launch_pow2_scale: the block's largest magnitude lands in [2^14, 2^15)): `m` is
// the lane's largest bf16 magnitude pattern (bits & 0x7fff); every wave of the
// work-group calls this with its own lanes; `red` is 4 words of LDS.
__device__ __forceinline__ int block_pow2(uint32_t m, uint32_t* red, int w) {
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, sh, 64));
  if ((threadIdx.x & 63) == 0) red[w] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  int e = 0;
  if (m != 0u && m < 0x7f80u) {
    const int be = (int)(m >> 7);
    e = be == 0 ? 63 : 14 - (be - 127);
    e = e < -63 ? -63 : (e > 63 ? 63 : e);
  }
  return e;
}
__device__ __forceinline__ uint32_t frag_absmax(const bf16x8* f, int n) {
  uint32_t m = 0;
  for (int i = 0; i < n; ++i) {
    const u32x4 v = __builtin_bit_cast(u32x4, f[i]);
#pragma unroll
    for (int e = 0; e < 4; ++e) m = max(m, max(v[e] & 0x7fffu, (v[e] >> 16) & 0x7fffu));
  }
  return m;
}

// ---------------------------------------------------------------- 2. D = rowsum(dO * O)
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  constexpr int CE = Elem<T>::kChunkElems;
  constexpr int CPR = D / CE;                 // lanes per token
  constexpr int TPB = 256 / CPR;              // tokens per work-group and trip
  const size_t total = (size_t)a.BH * a.g.N;
  const int c = threadIdx.x % CPR;
  for (size_t t0 = (size_t)blockIdx.x * TPB; t0 < total; t0 += (size_t)gridDim.x * TPB) {
    const size_t tok = t0 + threadIdx.x / CPR;
    float s = 0.f;
    if (tok < total) {
      const u32x4 g = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.dO) + tok * D + c * CE);
      const T* gv = reinterpret_cast<const T*>(&g);
      const float* O = a.O + tok * D + c * CE;
      float ov[CE];
#pragma unroll
      for (int q = 0; q < CE / 4; ++q) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(O + 4 * q);
        ov[4 * q] = v[0]; ov[4 * q + 1] = v[1]; ov[4 * q + 2] = v[2]; ov[4 * q + 3] = v[3];
      }
#pragma unroll
      for (int e = 0; e < CE; ++e) s = fmaf(ov[e], to_f32(gv[e]), s);
      if constexpr (sizeof(T) == 2) {            // scaled fp16 copy of dO for the fp16 products
        const float up = a.dscale[tok / a.g.N].x;
        f16x8 h;
#pragma unroll
        for (int e = 0; e < CE; ++e) h[e] = (f16)(to_f32(gv[e]) * up);
        *reinterpret_cast<f16x8*>(reinterpret_cast<f16*>(a.dO16) + tok * D + c * CE) = h;
      }
    }
#pragma unroll
    for (int m = CPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
    if (tok < total && c == 0) a.Dvec[tok] = s;
  }
}

// ---------------------------------------------------------------- 3. reverse index
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

__global__ __launch_bounds__(256) void rev_setbits_kernel(BwdArgs a) {
  const int NB = a.g.NB;
  const size_t n = (size_t)a.BH * NB * a.kmax;
  for (size_t id = (size_t)blockIdx.x * 256 + threadIdx.x; id < n; id += (size_t)gridDim.x * 256) {
    const int slot = (int)(id % a.kmax);
    const size_t row = id / a.kmax;             // bh * NB + tau
    const int bh = (int)(row / NB);
    const int tau = (int)(row % NB);
    int kk = a.kvec[bh];
    kk = kk < 1 ? 1 : (kk > a.kmax ? a.kmax : kk);
    if (slot >= kk) continue;
    const int j = a.idx[id];
    if ((unsigned)j >= (unsigned)NB) continue;
    atomicOr(&a.bitmap[((size_t)bh * NB + j) * a.words + (tau >> 5)], 1u << (tau & 31));
  }
}

// one wave per (head, key block)
__global__ __launch_bounds__(256) void rev_count_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (size_t)a.BH * a.g.NB) return;
  const uint32_t* w = a.bitmap + row * a.words;
  int cnt = 0;
  for (int i = lane; i < a.words; i += 64) cnt += __popc(w[i]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) cnt += __shfl_xor(cnt, m, 64);
  if (lane == 0) a.counts[row] = cnt;
}

// One wave per head: order[bh] = the head's key blocks by descending list length
// (count), ties by ascending block index -- the order in which the dK/dV
// work-groups take them, so that the longest lists start first and the short ones
// fill in at the end instead of one long list running on alone (measured at 32K
// tokens: dK/dV -5 %; dynamic 55K: -4 %).  A counting sort: histogram of the
// counts (<= NB) in LDS, a descending exclusive scan, then a stable placement in
// block order, 64 blocks at a time.  Integer work only: deterministic.
__global__ __launch_bounds__(64) void rev_order_kernel(BwdArgs a) {
  extern __shared__ int start[];              // [NB + 1]
  const int NB = a.g.NB, bh = blockIdx.x, lane = threadIdx.x;
  const int* cnt = a.counts + (size_t)bh * NB;
  int* ord = a.order + (size_t)bh * NB;
  for (int c = lane; c <= NB; c += 64) start[c] = 0;
  __syncthreads();
  for (int j0 = 0; j0 < NB; j0 += 8 * 64) {   // eight count loads in flight per lane
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = j0 + 64 * u + lane < NB ? cnt[j0 + 64 * u + lane] : -1;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (v[u] >= 0) atomicAdd(&start[min(v[u], NB)], 1);
  }
  __syncthreads();
  // start[c] = number of blocks whose count exceeds c (lanes take c descending)
  int run = 0;
  for (int top = NB; top >= 0; top -= 64) {
    const int c = top - lane;
    const int h = c >= 0 ? start[c] : 0;
    int incl = h;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    if (c >= 0) start[c] = run + incl - h;
    run += __shfl(incl, 63, 64);
  }
  __syncthreads();
  int c_next = lane < NB ? min(max(cnt[lane], 0), NB) : -1;
  for (int base = 0; base < NB; base += 64) {
    const int j = base + lane;
    const int c = c_next;
    c_next = j + 64 < NB ? min(max(cnt[j + 64], 0), NB) : -1;   // the next chunk's, in flight meanwhile
    int before = 0, same = 0;                  // lanes of this chunk with the same count
#pragma unroll
    for (int l = 0; l < 64; ++l) {
      const int cl = __builtin_amdgcn_readlane(c, l);
      same += cl == c;
      before += (cl == c) & (l < lane);
    }
    if (c >= 0) ord[start[c] + before] = j;
    __syncthreads();
    if (c >= 0 && before == same - 1) start[c] += same;
    __syncthreads();
  }
}

// one work-group per head: offsets[bh][j] = sum of counts before j; offsets[bh][NB] = total
__global__ __launch_bounds__(1024) void rev_scan_kernel(BwdArgs a) {
  __shared__ int part[1024];
  const int NB = a.g.NB;
  const int bh = blockIdx.x;
  const int* cnt = a.counts + (size_t)bh * NB;
  int* off = a.offsets + (size_t)bh * (NB + 1);
  const int per = (NB + 1023) / 1024;
  const int lo = threadIdx.x * per;
  int s = 0;
  for (int i = 0; i < per; ++i) s += (lo + i < NB) ? cnt[lo + i] : 0;
  part[threadIdx.x] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {        // Hillis-Steele inclusive scan
    const int v = (int)threadIdx.x >= d ? part[threadIdx.x - d] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = part[threadIdx.x] - s;            // exclusive prefix of this thread's range
  for (int i = 0; i < per; ++i) {
    if (lo + i < NB) {
      off[lo + i] = run;
      run += cnt[lo + i];
    }
  }
  if (threadIdx.x == 1023) off[NB] = part[1023];
}

// one wave per (head, key block): set bits in ascending order -> entries
__global__ __launch_bounds__(256) void rev_fill_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int NB = a.g.NB;
  if (row >= (size_t)a.BH * NB) return;
  const int bh = (int)(row / NB);
  const int j = (int)(row % NB);
  const uint32_t* w = a.bitmap + row * a.words;
  int32_t* out = a.entries + (size_t)bh * NB * a.kmax + a.offsets[(size_t)bh * (NB + 1) + j];
  int done = 0;
  for (int base = 0; base < a.words; base += 64) {
    const int i = base + lane;
    uint32_t word = i < a.words ? w[i] : 0u;
    const int pc = __popc(word);
    int incl = pc;                              // inclusive prefix over lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    int pos = done + incl - pc;
    while (word) {
      const int b = __ffs(word) - 1;
      out[pos++] = 32 * i + b;
      word &= word - 1u;
    }
    done += __shfl(incl, 63, 64);
  }
}

// The dK/dV phase's per-token statistics (bf16 inputs): Du = D * 2^u per (b, h),
// and LSE * log2(e), the fp32 product the exponent of P takes per (query, key)
// pair otherwise (written once per token instead); grid (blocks, heads)
template <int D>
__global__ __launch_bounds__(256) void scale_d_kernel(BwdArgs a) {
  const int bh = blockIdx.y;
  const float up = pow2f(ds_exponent(a.dscale[bh], a.vscale[bh], a.dabs[bh], kLog2D<D>));
  const size_t h = (size_t)bh * a.g.N;
  const float* __restrict__ src = a.Dvec + h;
  const float* __restrict__ lse = a.LSE + h;
  float* __restrict__ dst = a.Du + h;
  float* __restrict__ l2 = a.Lse2 + h;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < a.g.N; i += gridDim.x * 256) {
    dst[i] = src[i] * up;
    l2[i] = lse[i] * kLog2e;
  }
}

// ---------------------------------------------------------------- 4. dK, dV
// Operand types: with bf16 inputs every product runs on fp16 matrix cores: Q * 2^a
// from the fp16 copy of this phase, K * 2^b (b per key block) and V * 2^t converted
// when loaded, dO * 2^s from the prepare phase's copy, P in [0,1] and dS * 2^u
// rounded to fp16; the powers of two come back out in fp32, exactly.  fp32 inputs
// use fp32 throughout.
// two waves per SIMD for 16-bit inputs; the fp32 variants (parity checks only)
// need more than 256 registers and run at one
template <typename T> constexpr int kWavesPerSimd = sizeof(T) == 2 ? 2 : 1;
template <typename T> constexpr int kDqWavesPerSimd = sizeof(T) == 2 ? 3 : 1;

template <typename T> struct GradType;
template <> struct GradType<bf16> { typedef f16 type; };
template <> struct GradType<float> { typedef float type; };

__device__ __forceinline__ f16x8 to_grad_frag(bf16x8 v, float up, f16*) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (f16)((float)v[e] * up);
  return r;
}
__device__ __forceinline__ f32x8 to_grad_frag(f32x8 v, float, float*) { return v; }

// One work-group of 4 waves per key block, two waves per SIMD (<= 256 registers);
// wave w owns keys 16w..16w+15, whose K and V rows stay in registers as the B
// operands of the 16x16x32 products S = Q K^T and dP = dO V^T.  The query tiles of
// the block's CSC list stream through two LDS buffers (Q, dO, LSE and D of one
// tile each), filled by direct global->LDS loads (no register staging): tile e+1
// is requested before tile e is computed.  Per tile and wave:
//   S, dP  (64 queries x 16 keys)  A = Q / dO rows (ds_read_b128), 4 x 4 MFMA each
//   P = exp2(S c - LSE log2 e), dS = P (dP - D)     lane = key column
//   dV += P^T dO, dK += dS^T Q     A = P^T / dS^T straight from the S / dP registers
//                                  (the k-slots follow the result's row order),
//                                  B = dO / Q read transposed (ds_read_b64_tr_b16)
template <typename T, int D, bool FULL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<T>, 2)))
void bwd_dkdv_kernel(BwdArgs a) {
  typedef typename GradType<T>::type G;      // element type of every streamed tile and operand
  constexpr int W = 4;
  constexpr bool kHalf = sizeof(T) == 2;
  using CG = TileCfg<G, D>;
  typedef typename Elem<T>::frag Frag;
  typedef typename Elem<G>::frag GFrag;
  constexpr int KS = D / 32;                  // 32-wide reduction steps over d
  constexpr int DT = D / 16;                  // 16-wide output tiles over d
  __shared__ u32x4 q0[CG::kRowChunks], q1[CG::kRowChunks];
  __shared__ u32x4 g0[CG::kRowChunks], g1[CG::kRowChunks];
  __shared__ float st0[2][64], st1[2][64];    // [LSE (* log2 e), D (* 2^u)][query row]
  __shared__ uint32_t red[4];

  const Geo g = a.g;
  const int L = blockIdx.x;                 // natural head order (see common.hpp)
  const int bh = L / g.NB;
  const int r = L - bh * g.NB;
  int j = a.order != nullptr ? a.order[(size_t)bh * g.NB + r] : r;         // longest lists first
  if ((unsigned)j >= (unsigned)g.NB) j = r;   // (a workspace the prepare phase did not write)
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, q = lane >> 4;
  const size_t head_off = (size_t)bh * g.N * D;
  const G* __restrict__ Qh = (kHalf ? reinterpret_cast<const G*>(a.q16) : reinterpret_cast<const G*>(a.Q)) + head_off;
  const G* __restrict__ Gh = (kHalf ? reinterpret_cast<const G*>(a.dO16) : reinterpret_cast<const G*>(a.dO)) + head_off;
  // row statistics: LSE (fp32 inputs) or LSE * log2(e) (bf16), and D or D * 2^u
  const float* __restrict__ LSEh = (kHalf ? a.Lse2 : a.LSE) + (size_t)bh * g.N;
  const float* __restrict__ Dh = (kHalf ? a.Du : a.Dvec) + (size_t)bh * g.N;
  const int jbase = tile_base(g, j);

  // Reduction order of the 16x16x32 products that read row operands from LDS (S, dP):
  // lane group q takes the 8-element chunk qk of each 32-wide step, the two bits of
  // q swapped (16-bit tiles).  Measured on gfx950: when lanes l and l+32 read one row
  // at chunks that differ in bit 1, every ds_read_b128 pays a second pass (LDS bank
  // conflict counters: 4 of 8 cycles); chunks that differ in bit 0 cost nothing.
  const int qk = kHalf ? (((q & 1) << 1) | (q >> 1)) : q;
  // this lane's key row: B fragments of S = Q K^T and dP = dO V^T (N = keys)
  const int kr = 16 * w + l16;
  const bool k_ok = kr < g.T;
  const int k_tok = jbase + (k_ok ? member_offset(g, kr) : 0);
  GFrag kf[KS], vf[KS];
  // dinv: 2^-s of the fp16 dO copy (dV); dpinv: 2^(u-s-t) turns the fp16 dP into
  // dP * 2^u; c2: the softmax scale (log2 units) over 2^(a+b); kscale: dK's 2^-u
  float dinv = 1.f, dpinv = 1.f, c2 = a.c, kunscale = 1.f, kfac = a.scale;
  {
    Frag kt[KS], vt[KS];
    load_row_frags16<T, D>(kt, reinterpret_cast<const T*>(a.K) + head_off + (size_t)k_tok * D, k_ok, qk);
    load_row_frags16<T, D>(vt, reinterpret_cast<const T*>(a.V) + head_off + (size_t)k_tok * D, k_ok, qk);
    float kup = 1.f, vup = 1.f;
    if constexpr (kHalf) {
      const int bj = block_pow2(frag_absmax(kt, KS), red, w);   // K's exponent for this key block
      const float2 vs = a.vscale[bh], ds = a.dscale[bh];
      const int u = ds_exponent(ds, vs, a.dabs[bh], kLog2D<D>);
      kup = pow2f(bj);
      vup = vs.x;
      dinv = ds.y;
      dpinv = dinv * vs.y * pow2f(u);         // powers of two: exact while normal
      c2 = a.c * a.qscale[bh].y * pow2f(-bj);
      kunscale = pow2f(-u);
      kfac = a.scale * a.qscale[bh].y;
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kf[s] = to_grad_frag(kt[s], kup, (G*)nullptr);
      vf[s] = to_grad_frag(vt[s], vup, (G*)nullptr);
    }
  }

  int goff[DmaCfg<G, D, W>::kPer];
  dma_offsets<G, D, W>(goff, g, w, lane);     // the Q and dO tiles share one layout
  const int soff = lane < g.T ? member_offset(g, lane) : 0;   // stats row of lane (waves 0, 1)

  f32x4 dk[DT], dv[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    dk[t] = f32x4{};
    dv[t] = f32x4{};
  }
  const int* list = a.entries + (size_t)bh * g.NB * a.kmax;
  const int* off = a.offsets + (size_t)bh * (g.NB + 1);
  const int e0 = off[j], n = off[j + 1] - e0;

  // 16-bit tiles: closed-form operand addresses (one lane constant each)
  constexpr bool kFast = sizeof(T) == 2;
  const int rowl = row_lane16<D>(l16, qk), trl = tr_lane16<D>(l16, q);

  const __amdgpu_buffer_rsrc_t rq = head_rsrc(Qh, (size_t)g.N * D * sizeof(G));
  const __amdgpu_buffer_rsrc_t rg = head_rsrc(Gh, (size_t)g.N * D * sizeof(G));
  const __amdgpu_buffer_rsrc_t rs = head_rsrc(w == 0 ? LSEh : Dh, (size_t)g.N * sizeof(float));
  auto request = [&](int base, u32x4* lq, u32x4* lg, float (*lst)[64]) {   // tile whose first token is `base`
    dma_tile<G, D, W>(lq, rq, base * D * (int)sizeof(G), goff, w);
    dma_tile<G, D, W>(lg, rg, base * D * (int)sizeof(G), goff, w);
    if (w < 2) dma_row_stats(lst[w], rs, base * 4, soff);
  };
  auto compute = [&](const u32x4* lq, const u32x4* lg, const float (*lst)[64]) {
    // S and dP: lane holds key column kr, query rows 16mt + 4q + i
    f32x4 sacc[4], pacc[4];
    constexpr int NS = 4 * KS;                // (mt, s) steps
    constexpr int NT = 2 * DT;                // (t, ks) steps
    // 16-bit path: operand reads run two steps ahead of the products
    GFrag bg[4], bq[4];
    if constexpr (kFast) {
      GFrag qa[3], ga[3];
      auto rd = [&](int k, GFrag& qf, GFrag& gf) {
        const int xs = rowl ^ (64 * (k % KS));
        qf = frag16_row_fast<G, D>(lq, k / KS, xs);
        gf = frag16_row_fast<G, D>(lg, k / KS, xs);
      };
      auto rt = [&](int k, GFrag& gb, GFrag& qb) {   // step k = (t, ks) as in the dV/dK loop below
        const int t = 2 * (k / 4) + (k & 1), ks = (k >> 1) & 1;
        const int xt = trl ^ (32 * t);
        gb = frag16_tr_fast<G, D>(lg, ks, xt, (G*)nullptr);
        qb = frag16_tr_fast<G, D>(lq, ks, xt, (G*)nullptr);
      };
      rd(0, qa[0], ga[0]);
      rd(1, qa[1], ga[1]);
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        if (k + 2 < NS) rd(k + 2, qa[(k + 2) % 3], ga[(k + 2) % 3]);
        const int mt = k / KS, s = k % KS;
        if (s == 0) {
          sacc[mt] = f32x4{};
          pacc[mt] = f32x4{};
        }
        sacc[mt] = mma16(qa[k % 3], kf[s], sacc[mt]);
        pacc[mt] = mma16(ga[k % 3], vf[s], pacc[mt]);
        __builtin_amdgcn_sched_barrier(0);
      }
      rt(0, bg[0], bq[0]);                    // first transposed operands, under the softmax below
      rt(1, bg[1], bq[1]);
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        sacc[mt] = f32x4{};
        pacc[mt] = f32x4{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          sacc[mt] = mma16(frag16_row<G, D>(lq, 16 * mt + l16, s, q), kf[s], sacc[mt]);
          pacc[mt] = mma16(frag16_row<G, D>(lg, 16 * mt + l16, s, q), vf[s], pacc[mt]);
        }
        __builtin_amdgcn_sched_barrier(0);      // bounds the operand reads in flight
      }
    }
    // P and dS (* 2^u) as A operands: k-slot e of step ks <-> query 32ks + 16(e/4) + 4q + e%4
    GFrag pf[2], sf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float pv[8], sv[8];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int mt = 2 * ks + hf, r0 = 16 * mt + 4 * q;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lst[0][r0]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&lst[1][r0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = fast_exp2(fmaf(sacc[mt][i], c2, kHalf ? -l4[i] : -l4[i] * kLog2e));
          if constexpr (!FULL) p = (r0 + i < g.T) ? p : 0.f;      // padding query rows
          pv[4 * hf + i] = p;
          sv[4 * hf + i] = p * fmaf(pacc[mt][i], dpinv, -d4[i]);
        }
      }
      pf[ks] = to_frag(pv, (G*)nullptr);
      sf[ks] = to_frag(sv, (G*)nullptr);
    }
    __builtin_amdgcn_sched_barrier(0);
    // dV += P^T dO, dK += dS^T Q: lane holds d column 16t + l16, key rows 4q + i
    if constexpr (kFast) {
      // steps k = (t, ks) in the order (t0, ks), (t0+1, ks): no product depends on
      // the one issued just before it
      auto rt = [&](int k, GFrag& gb, GFrag& qb) {
        const int t = 2 * (k / 4) + (k & 1), ks = (k >> 1) & 1;
        const int xt = trl ^ (32 * t);
        gb = frag16_tr_fast<G, D>(lg, ks, xt, (G*)nullptr);
        qb = frag16_tr_fast<G, D>(lq, ks, xt, (G*)nullptr);
      };
#pragma unroll
      for (int k = 0; k < NT; k += 2) {
        if (k + 2 < NT) rt(k + 2, bg[(k + 2) % 4], bq[(k + 2) % 4]);
        if (k + 3 < NT) rt(k + 3, bg[(k + 3) % 4], bq[(k + 3) % 4]);
        const int t0 = 2 * (k / 4), ks = (k >> 1) & 1;
        const int a0 = k % 4, a1 = (k + 1) % 4;
        dv[t0] = mma16(pf[ks], bg[a0], dv[t0]);
        dv[t0 + 1] = mma16(pf[ks], bg[a1], dv[t0 + 1]);
        dk[t0] = mma16(sf[ks], bq[a0], dk[t0]);
        dk[t0 + 1] = mma16(sf[ks], bq[a1], dk[t0 + 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int t = 0; t < DT; ++t) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int r0 = 32 * ks + 4 * q;
          dv[t] = mma16(pf[ks], frag16_tr<G, D>(lg, 16 * t, r0, l16, (G*)nullptr), dv[t]);
          dk[t] = mma16(sf[ks], frag16_tr<G, D>(lq, 16 * t, r0, l16, (G*)nullptr), dk[t]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // the block's query tiles, 64 list entries per vector load (no scalar-load wait per tile)
  // (entries are tile ids written by the prepare phase, all valid: the list walk
  // hands out exactly n of them)
  TileList ids;
  ids.init(list + e0, n, g, lane);
  auto next_base = [&]() {
    (void)ids.next(lane);
    return ids.last_base;
  };
  if (n > 0) request(next_base(), q0, g0, st0);
  dma_wait();
  __syncthreads();
  // two tiles per trip so that every LDS buffer is a distinct object (the next
  // tile's direct loads never alias the reads of the current one)
  for (int e = 0; e < n; e += 2) {
    if (e + 1 < n) request(next_base(), q1, g1, st1);
    compute(q0, g0, st0);
    dma_wait();
    __syncthreads();
    if (e + 1 >= n) break;
    if (e + 2 < n) request(next_base(), q0, g0, st0);
    compute(q1, g1, st1);
    dma_wait();
    __syncthreads();
  }

  // store: lane holds d column 16t + l16, key rows 16w + 4q + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * q + i;
    if (r < g.T) {
      const size_t orow = head_off + (size_t)(jbase + member_offset(g, r)) * D;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        store1(a.dK, orow + 16 * t + l16, a.out_f32, (dk[t][i] * kunscale) * kfac);
        store1(a.dV, orow + 16 * t + l16, a.out_f32, dv[t][i] * dinv);
      }
    }
  }
}

// ---------------------------------------------------------------- 5. dQ
// One work-group of 4 waves per query tile, three work-groups per CU (16-bit
// inputs); wave w owns queries 16w..16w+15, whose Q and dO rows stay in registers
// as the B operands of the 16x16x32 products S^T = K Q^T and dP^T = V dO^T.  The
// kept blocks stream through LDS, filled by direct global->LDS loads: K rows (read
// in both halves of a block) in two buffers, one block ahead; V rows (read only by
// dP^T) in one, the next block's requested once every wave is past its dP^T
// products.  One V buffer keeps the work-group at 48 KB of LDS, so three fit on a
// CU (measured at 32K tokens: -4 % against two buffers at two per CU, outputs
// bit-identical).  With bf16 inputs K comes from this phase's fp16 copy (K * 2^b),
// Q is converted to fp16 with a power of two per query tile, dP^T = V dO^T stays
// bf16, and dS^T * 2^u is rounded to fp16.  Per block and wave:
//   S^T, dP^T (64 keys x 16 queries)   A = K / V rows (ds_read_b128), 4 x 4 MFMA each
//   P^T = exp2(S^T c - LSE log2 e), dS^T = P^T (dP^T - D)   lane = query column
//   dQ^T += K^T dS^T                   B = dS^T straight from the S^T registers,
//                                      A = K read transposed (ds_read_b64_tr_b16)
template <typename T, int D, bool FULL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kDqWavesPerSimd<T>, 3)))
void bwd_dq_kernel(BwdArgs a) {
  constexpr int W = 4;
  typedef typename GradType<T>::type G;      // K tiles, Q and dS operands
  using C = TileCfg<T, D>;
  using CG = TileCfg<G, D>;
  typedef typename Elem<T>::frag Frag;
  typedef typename Elem<G>::frag GFrag;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr bool kFast = sizeof(T) == 2;
  __shared__ u32x4 k0[CG::kRowChunks], k1[CG::kRowChunks];
  __shared__ u32x4 vt[C::kRowChunks];          // one V buffer: read in the first products only
  __shared__ uint32_t red[4];

  const Geo g = a.g;
  const int L = blockIdx.x;                 // natural order (see common.hpp)
  const int bh = L / g.NB;
  const int tau = L - bh * g.NB;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, q = lane >> 4;
  const size_t head_off = (size_t)bh * g.N * D;
  const G* __restrict__ Kh = (kFast ? reinterpret_cast<const G*>(a.k16) : reinterpret_cast<const G*>(a.K)) + head_off;
  const T* __restrict__ Vh = reinterpret_cast<const T*>(a.V) + head_off;
  const int* __restrict__ irow = a.idx + ((size_t)bh * g.NB + tau) * a.kmax;
  int kk = a.kvec[bh];
  kk = kk < 1 ? 1 : (kk > a.kmax ? a.kmax : kk);

  // reduction order of S^T and dP^T: lane group q takes chunk qk of each 32-wide step
  // (the bits of q swapped for 16-bit tiles; see the dK/dV kernel)
  const int qk = kFast ? (((q & 1) << 1) | (q >> 1)) : q;
  // this lane's query row (B fragments: N = queries)
  const int qr = 16 * w + l16;
  const bool q_ok = qr < g.T;
  const int q_tok = tile_base(g, tau) + (q_ok ? member_offset(g, qr) : 0);
  GFrag qf[KS];
  Frag gf[KS];
  load_row_frags16<T, D>(gf, reinterpret_cast<const T*>(a.dO) + head_off + (size_t)q_tok * D, q_ok, qk);
  const float nl = q_ok ? -a.LSE[(size_t)bh * g.N + q_tok] * kLog2e : -INFINITY;   // padding rows: P = 0
  float dd = q_ok ? a.Dvec[(size_t)bh * g.N + q_tok] : 0.f;
  // c2: the softmax scale (log2 units) over 2^(a+b); up: 2^u of the fp16 dS;
  // dQ = (acc * qunscale) * qfac
  float c2 = a.c, up = 1.f, qunscale = 1.f, qfac = a.scale;
  {
    Frag qt[KS];
    load_row_frags16<T, D>(qt, reinterpret_cast<const T*>(a.Q) + head_off + (size_t)q_tok * D, q_ok, qk);
    float qup = 1.f;
    if constexpr (kFast) {
      const int at = block_pow2(frag_absmax(qt, KS), red, w);   // Q's exponent for this query tile
      const int u = ds_exponent(a.dscale[bh], a.vscale_q[bh], a.dabs[bh], kLog2D<D>);
      qup = pow2f(at);
      c2 = a.c * a.kscale[bh].y * pow2f(-at);
      up = pow2f(u);
      dd *= up;
      qunscale = pow2f(-u);
      qfac = a.scale * a.kscale[bh].y;
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = to_grad_frag(qt[s], qup, (G*)nullptr);
  }

  int koff[DmaCfg<T, D, W>::kPer];
  dma_offsets<T, D, W>(koff, g, w, lane);
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(Kh, (size_t)g.N * D * sizeof(G));
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(Vh, (size_t)g.N * D * sizeof(T));
  const int rowl = kFast ? row_lane16<D>(l16, qk) : 0, trl = kFast ? tr_lane16<D>(l16, q) : 0;

  f32x4 dq[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dq[t] = f32x4{};

  auto request_k = [&](int base, u32x4* lk) {   // block whose first token is `base`
    dma_tile<G, D, W>(lk, rk, base * D * (int)sizeof(G), koff, w);   // same layout: G and T have one size
  };
  auto request_v = [&](int base) { dma_tile<T, D, W>(vt, rv, base * D * (int)sizeof(T), koff, w); };
  auto compute = [&](const u32x4* lk, const u32x4* lv, auto&& mid) {
    // S^T and dP^T: lane holds query column qr, key rows 16mt + 4q + i
    f32x4 sacc[4], pacc[4];
    GFrag ka[4];                               // transposed K operands of the first steps (prefetched)
    if constexpr (kFast) {
      GFrag ra[3];
      Frag rb[3];
      auto rd = [&](int k, GFrag& x, Frag& y) {
        const int xs = rowl ^ (64 * (k % KS));
        x = frag16_row_fast<G, D>(lk, k / KS, xs);
        y = frag16_row_fast<T, D>(lv, k / KS, xs);
      };
      rd(0, ra[0], rb[0]);
      rd(1, ra[1], rb[1]);
#pragma unroll
      for (int k = 0; k < 4 * KS; ++k) {
        if (k + 2 < 4 * KS) rd(k + 2, ra[(k + 2) % 3], rb[(k + 2) % 3]);
        const int mt = k / KS, s = k % KS;
        if (s == 0) {
          sacc[mt] = f32x4{};
          pacc[mt] = f32x4{};
        }
        sacc[mt] = mma16(ra[k % 3], qf[s], sacc[mt]);
        pacc[mt] = mma16(rb[k % 3], gf[s], pacc[mt]);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        ka[2 * k] = frag16_tr_fast<G, D>(lk, 0, trl ^ (32 * k), (G*)nullptr);
        ka[2 * k + 1] = frag16_tr_fast<G, D>(lk, 1, trl ^ (32 * k), (G*)nullptr);
      }
      mid();
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        sacc[mt] = f32x4{};
        pacc[mt] = f32x4{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          sacc[mt] = mma16(frag16_row<G, D>(lk, 16 * mt + l16, s, q), qf[s], sacc[mt]);
          pacc[mt] = mma16(frag16_row<T, D>(lv, 16 * mt + l16, s, q), gf[s], pacc[mt]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mid();
    }
    // dS^T (* 2^u) as B operands: k-slot e of step ks <-> key 32ks + 16(e/4) + 4q + e%4
    GFrag sf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float sv[8];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int mt = 2 * ks + hf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = fast_exp2(fmaf(sacc[mt][i], c2, nl));
          if constexpr (!FULL) p = (16 * mt + 4 * q + i < g.T) ? p : 0.f;     // padding keys
          sv[4 * hf + i] = p * fmaf(pacc[mt][i], up, -dd);
        }
      }
      sf[ks] = to_frag(sv, (G*)nullptr);
    }
    __builtin_amdgcn_sched_barrier(0);
    // dQ^T += K^T dS^T: lane holds query column qr, d rows 16t + 4q + i
    if constexpr (kFast) {
      GFrag kb[4];
#pragma unroll
      for (int t = 0; t < DT; t += 2) {
        const bool pre = t + 2 < DT;
        if (pre) {
          kb[0] = frag16_tr_fast<G, D>(lk, 0, trl ^ (32 * (t + 2)), (G*)nullptr);
          kb[1] = frag16_tr_fast<G, D>(lk, 1, trl ^ (32 * (t + 2)), (G*)nullptr);
          kb[2] = frag16_tr_fast<G, D>(lk, 0, trl ^ (32 * (t + 3)), (G*)nullptr);
          kb[3] = frag16_tr_fast<G, D>(lk, 1, trl ^ (32 * (t + 3)), (G*)nullptr);
        }
        // t: ka[0] (ks 0), ka[1] (ks 1); t+1: ka[2], ka[3]
        dq[t] = mma16(ka[0], sf[0], dq[t]);
        dq[t + 1] = mma16(ka[2], sf[0], dq[t + 1]);
        dq[t] = mma16(ka[1], sf[1], dq[t]);
        dq[t + 1] = mma16(ka[3], sf[1], dq[t + 1]);
        if (pre) {
#pragma unroll
          for (int x = 0; x < 4; ++x) ka[x] = kb[x];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int t = 0; t < DT; ++t) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const GFrag kt = frag16_tr<G, D>(lk, 16 * t, 32 * ks + 4 * q, l16, (G*)nullptr);
          dq[t] = mma16(kt, sf[ks], dq[t]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // the kept blocks in idx order, invalid entries skipped (wave-uniform)
  TileList ids;
  ids.init(irow, kk, g, lane);
  auto next_valid = [&]() -> int { return ids.next(lane); };
  int bcur = next_valid();
  if (bcur >= 0) {
    request_k(ids.last_base, k0);
    request_v(ids.last_base);
  }
  dma_wait();
  __syncthreads();
  int bnext = bcur >= 0 ? next_valid() : -1;
  int nbase = ids.last_base;
  // V of the next block is requested once every wave has finished its S^T, dP^T
  // products (the only reads of V); K, read in both halves, is double-buffered
  auto mid = [&]() {
    __syncthreads();
    if (bnext >= 0) request_v(nbase);
  };
  // two blocks per trip so that every K buffer is a distinct object
  while (bcur >= 0) {
    if (bnext >= 0) request_k(nbase, k1);
    compute(k0, vt, mid);
    dma_wait();
    __syncthreads();
    bcur = bnext;
    if (bcur < 0) break;
    bnext = next_valid();
    nbase = ids.last_base;
    if (bnext >= 0) request_k(nbase, k0);
    compute(k1, vt, mid);
    dma_wait();
    __syncthreads();
    bcur = bnext;
    if (bcur < 0) break;
    bnext = next_valid();
    nbase = ids.last_base;
  }

  // store: lane holds query column qr, d rows 16t + 4q + i
  if (q_ok) {
    const size_t orow = head_off + (size_t)q_tok * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
      store4(a.dQ, orow + 16 * t + 4 * q, a.out_f32, (dq[t][0] * qunscale) * qfac, (dq[t][1] * qunscale) * qfac,
             (dq[t][2] * qunscale) * qfac, (dq[t][3] * qunscale) * qfac);
  }
}

template <typename T, int D>
hipError_t launch_prepare_t(const BwdArgs& a, hipStream_t s) {
  constexpr int CPR = D / Elem<T>::kChunkElems;
  const size_t tokens = (size_t)a.BH * a.g.N;
  const int tpb = 256 / CPR;
  if constexpr (sizeof(T) == 2) {
    const hipError_t e = launch_pow2_scale(a.dO, a.BH, (size_t)a.g.N * D, a.dmax, a.dscale, s);
    if (e != hipSuccess) return e;
  }
  const size_t pgrid = (tokens + tpb - 1) / tpb;
  hipLaunchKernelGGL((bwd_prep_kernel<T, D>), dim3((unsigned)(pgrid < (1u << 20) ? pgrid : (1u << 20))), dim3(256), 0,
                     s, a);
  if constexpr (sizeof(T) == 2) {
    const hipError_t e = launch_absmax_f32(a.Dvec, a.BH, (size_t)a.g.N, a.dabs_part, a.dabs, s);
    if (e != hipSuccess) return e;
  }
  const size_t nwords = (size_t)a.BH * a.g.NB * a.words;
  const unsigned zgrid = (unsigned)((nwords + 255) / 256 < 65536 ? (nwords + 255) / 256 : 65536);
  hipLaunchKernelGGL(zero_words_kernel, dim3(zgrid), dim3(256), 0, s, a.bitmap, nwords);
  const size_t nslots = (size_t)a.BH * a.g.NB * a.kmax;
  const size_t sgrid = (nslots + 255) / 256;
  hipLaunchKernelGGL(rev_setbits_kernel, dim3((unsigned)(sgrid < (1u << 20) ? sgrid : (1u << 20))), dim3(256), 0, s, a);
  const unsigned rows4 = (unsigned)(((size_t)a.BH * a.g.NB + 3) / 4);
  hipLaunchKernelGGL(rev_count_kernel, dim3(rows4), dim3(256), 0, s, a);
  if (a.order != nullptr)
    hipLaunchKernelGGL(rev_order_kernel, dim3(a.BH), dim3(64), (size_t)(a.g.NB + 1) * sizeof(int), s, a);
  hipLaunchKernelGGL(rev_scan_kernel, dim3(a.BH), dim3(1024), 0, s, a);
  hipLaunchKernelGGL(rev_fill_kernel, dim3(rows4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prepare(const BwdArgs& a, int io_f32, int d, hipStream_t s) {
  if (io_f32) return d == 64 ? launch_prepare_t<float, 64>(a, s) : launch_prepare_t<float, 128>(a, s);
  return d == 64 ? launch_prepare_t<bf16, 64>(a, s) : launch_prepare_t<bf16, 128>(a, s);
}

template <typename T, int D>
void launch_dkdv_t(const BwdArgs& a, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    // V's and Q's scales, the fp16 copy of Q, then D * 2^u
    const size_t per_head = (size_t)a.g.N * D;
    if (launch_pow2_scale(a.V, a.BH, per_head, a.vmax, a.vscale, s) != hipSuccess) return;
    if (launch_pow2_scale(a.Q, a.BH, per_head, a.qmax, a.qscale, s) != hipSuccess) return;
    if (launch_pow2_convert(a.Q, a.BH, per_head, a.qscale, a.q16, s) != hipSuccess) return;
    const unsigned gx = (unsigned)((a.g.N + 255) / 256 < 64 ? (a.g.N + 255) / 256 : 64);
    hipLaunchKernelGGL((scale_d_kernel<D>), dim3(gx, (unsigned)a.BH), dim3(256), 0, s, a);
  }
  const dim3 grid(a.BH * a.g.NB), block(256);
  if (a.g.T == 64) hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false>), grid, block, 0, s, a);
}
hipError_t launch_bwd_dkdv(const BwdArgs& a, int io_f32, int d, hipStream_t s) {
  if (io_f32) {
    if (d == 64) launch_dkdv_t<float, 64>(a, s);
    else launch_dkdv_t<float, 128>(a, s);
  } else {
    if (d == 64) launch_dkdv_t<bf16, 64>(a, s);
    else launch_dkdv_t<bf16, 128>(a, s);
  }
  return hipGetLastError();
}

template <typename T, int D>
void launch_dq_t(const BwdArgs& a, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    // V's scale (for the exponent of dS), K's scale and the fp16 copy of K
    const size_t per_head = (size_t)a.g.N * D;
    if (launch_pow2_scale(a.V, a.BH, per_head, a.vmax_q, a.vscale_q, s) != hipSuccess) return;
    if (launch_pow2_scale(a.K, a.BH, per_head, a.kmaxp, a.kscale, s) != hipSuccess) return;
    if (launch_pow2_convert(a.K, a.BH, per_head, a.kscale, a.k16, s) != hipSuccess) return;
  }
  const dim3 grid(a.BH * a.g.NB), block(256);
  if (a.g.T == 64) hipLaunchKernelGGL((bwd_dq_kernel<T, D, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((bwd_dq_kernel<T, D, false>), grid, block, 0, s, a);
}
hipError_t launch_bwd_dq(const BwdArgs& a, int io_f32, int d, hipStream_t s) {
  if (io_f32) {
    if (d == 64) launch_dq_t<float, 64>(a, s);
    else launch_dq_t<float, 128>(a, s);
  } else {
    if (d == 64) launch_dq_t<bf16, 64>(a, s);
    else launch_dq_t<bf16, 128>(a, s);
  }
  return hipGetLastError();
}

}  // namespace dsa
