// Training signal of the low-rank predictor for gfx950 (DSV page, gist.science/
// ar/paper/2502.07590, section 4: in stage one the predictor is trained next to
// the model so that it learns which blocks matter; the page gives no loss).
//
// Reading: the predictor's score S[tau, j] = Qbar[tau] . Kbar[j] estimates the
// pooled attention logit T[tau, j] = mean over the tile x block token pairs of
// q . k = Pq[tau] . Pk[j] (Pq, Pk: tile means of Q and K), and stage one
// minimises, per (b, h), loss = ||S - T||^2 / NB^2 over Wq[h] and Wk[h] only.
//
// With the GPU's pool-then-project predictor, Qbar = Pq Wq and Kbar = Pk Wk, so
//   S - T = Pq (Wq Wk^T - I) Pk^T = Pq M Pk^T,
//   loss  = trace(M^T A M C) / NB^2         A = Pq^T Pq, C = Pk^T Pk   (d x d)
//   dloss/dWq = (2/NB^2) A M C Wk,  dloss/dWk = (2/NB^2) (A M C)^T Wq.
// Nothing of size NB x NB is formed: the work is one read of Q and K (the
// predictor's pooling kernel, storing the tile means), NB*d^2 multiply-adds per
// Gram matrix, and a few d x d products per (b, h).  All arithmetic is fp32 in a
// fixed order (bit-reproducible).
//
// Kernel gram_kernel: one work-group per (tensor, b*h, 32x32 output tile on or
//   above the diagonal, written to both mirror positions); tile means staged
//   through LDS 32 tiles at a time; each thread sums 4 outputs over all tiles in
//   ascending order.
// Kernel pg_m_kernel: M = Wq Wk^T - I per head.
// Kernel pg_x_kernel: one work-group per (b*h, 16 rows): Z = A[rows] M, X[rows] =
//   Z C with M and C in LDS (128 KB at d = 128); partial loss and gradient rows.
// Kernel pg_reduce_kernel: the partials summed in a fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int kThreads = 256;
constexpr int kGT = 32;                       // Gram output tile edge and tiles per LDS stage
constexpr int kRB = 16;                       // rows of the d x d products per work-group

template <int D>
__global__ __launch_bounds__(kThreads) void gram_kernel(PGradArgs a) {
  constexpr int TILES = D / kGT;
  constexpr int PAIRS = TILES * (TILES + 1) / 2;   // tiles on and above the diagonal
  __shared__ float pi[kGT][kGT + 1];
  __shared__ float pj[kGT][kGT + 1];
  const int BH = a.B * a.H;
  int id = blockIdx.x;
  int pr = id % PAIRS;
  id /= PAIRS;
  int ti = 0;
  while (pr >= TILES - ti) {                   // pair index -> (ti, tj), ti <= tj
    pr -= TILES - ti;
    ++ti;
  }
  const int tj = ti + pr;
  const int bh = id % BH;
  const int which = id / BH;                  // 0: Q, 1: K
  const float* __restrict__ P = (which ? a.Pk : a.Pq) + (size_t)bh * a.NB * D;
  float* __restrict__ G = (which ? a.Gk : a.Gq) + (size_t)bh * D * D;

  const int tid = threadIdx.x;
  const int ii = tid & 15, jj = tid >> 4;     // outputs (ii | ii+16) x (jj | jj+16)
  const int lrow = tid >> 3, lcol = (tid & 7) * 4;
  float acc00 = 0.f, acc01 = 0.f, acc10 = 0.f, acc11 = 0.f;
  for (int t0 = 0; t0 < a.NB; t0 += kGT) {
    const int t = t0 + lrow;
    float4 vi = make_float4(0.f, 0.f, 0.f, 0.f), vj = vi;
    if (t < a.NB) {
      vi = *reinterpret_cast<const float4*>(P + (size_t)t * D + ti * kGT + lcol);
      vj = *reinterpret_cast<const float4*>(P + (size_t)t * D + tj * kGT + lcol);
    }
    pi[lrow][lcol] = vi.x; pi[lrow][lcol + 1] = vi.y; pi[lrow][lcol + 2] = vi.z; pi[lrow][lcol + 3] = vi.w;
    pj[lrow][lcol] = vj.x; pj[lrow][lcol + 1] = vj.y; pj[lrow][lcol + 2] = vj.z; pj[lrow][lcol + 3] = vj.w;
    __syncthreads();
#pragma unroll 8
    for (int u = 0; u < kGT; ++u) {
      const float a0 = pi[u][ii], a1 = pi[u][ii + 16];
      const float b0 = pj[u][jj], b1 = pj[u][jj + 16];
      acc00 = fmaf(a0, b0, acc00);
      acc01 = fmaf(a0, b1, acc01);
      acc10 = fmaf(a1, b0, acc10);
      acc11 = fmaf(a1, b1, acc11);
    }
    __syncthreads();
  }
  // the Gram matrix is symmetric (fma(a, b) = fma(b, a), same order): the tile and
  // its mirror image get the same values
  const int r0 = ti * kGT + ii, c0 = tj * kGT + jj;
  G[(size_t)r0 * D + c0] = acc00;
  G[(size_t)r0 * D + c0 + 16] = acc01;
  G[(size_t)(r0 + 16) * D + c0] = acc10;
  G[(size_t)(r0 + 16) * D + c0 + 16] = acc11;
  G[(size_t)c0 * D + r0] = acc00;
  G[(size_t)(c0 + 16) * D + r0] = acc01;
  G[(size_t)c0 * D + r0 + 16] = acc10;
  G[(size_t)(c0 + 16) * D + r0 + 16] = acc11;
}

// Sum over the work-group, fixed order: wave partials via xor shuffles, then the
// four wave sums in wave order.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < kThreads / 64; ++q) s += red[q];
  __syncthreads();
  return s;
}

// M[h] = Wq[h] Wk[h]^T - I, one thread per element.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void pg_m_kernel(PGradArgs a) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= a.H * D * D) return;
  const int h = i / (D * D), rem = i - h * D * D;
  const int e = rem / D, f = rem - e * D;
  const int r = a.r;
  const T* __restrict__ Wq = reinterpret_cast<const T*>(a.Wq) + (size_t)h * D * r;
  const T* __restrict__ Wk = reinterpret_cast<const T*>(a.Wk) + (size_t)h * D * r;
  float m = 0.f;
  for (int c = 0; c < r; ++c) m = fmaf(to_f32(Wq[e * r + c]), to_f32(Wk[f * r + c]), m);
  a.M[i] = m - (e == f ? 1.f : 0.f);
}

// One work-group per (b*h, block of kRB rows e): with X = (A M) C,
//   Z = A[rows] M, X[rows] = Z C, loss part = sum of X[rows] o M[rows],
//   dWq part (rows)  = X[rows] Wk,   dWk part (all d rows) = X[rows]^T Wq[rows].
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void pg_x_kernel(PGradArgs a) {
  constexpr int CPT = D * kRB / kThreads;     // columns per thread (8 at d = 128, 4 at d = 64)
  constexpr int TPR = D / CPT;                // threads per row
  __shared__ float Mh[D * D];
  __shared__ float Cs[D * D];
  __shared__ float Zs[kRB * D];
  __shared__ float red[kThreads / 64];
  constexpr int RBS = D / kRB;
  const int bh = blockIdx.x / RBS;
  const int rb = blockIdx.x - bh * RBS;
  const int h = bh % a.H;
  const int e0 = rb * kRB;
  const int tid = threadIdx.x;
  const int r = a.r;
  const float* __restrict__ Mg = a.M + (size_t)h * D * D;
  const float* __restrict__ Ag = a.Gq + (size_t)bh * D * D;
  const float* __restrict__ Cg = a.Gk + (size_t)bh * D * D;
  for (int i = tid * 4; i < D * D; i += kThreads * 4) {
    *reinterpret_cast<float4*>(Mh + i) = *reinterpret_cast<const float4*>(Mg + i);
    *reinterpret_cast<float4*>(Cs + i) = *reinterpret_cast<const float4*>(Cg + i);
  }
  __syncthreads();
  const int row = tid / TPR, c0 = (tid % TPR) * CPT;
  float z[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) z[q] = 0.f;
  const float* __restrict__ arow = Ag + (size_t)(e0 + row) * D;
  for (int g = 0; g < D; ++g) {                // Z = A[rows] M
    const float av = arow[g];
#pragma unroll
    for (int q = 0; q < CPT; ++q) z[q] = fmaf(av, Mh[g * D + c0 + q], z[q]);
  }
#pragma unroll
  for (int q = 0; q < CPT; ++q) Zs[row * D + c0 + q] = z[q];
  __syncthreads();
  float x[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) x[q] = 0.f;
  for (int g = 0; g < D; ++g) {                // X[rows] = Z C
    const float zv = Zs[row * D + g];
#pragma unroll
    for (int q = 0; q < CPT; ++q) x[q] = fmaf(zv, Cs[g * D + c0 + q], x[q]);
  }
  float part = 0.f;
#pragma unroll
  for (int q = 0; q < CPT; ++q) part = fmaf(x[q], Mh[(e0 + row) * D + c0 + q], part);
  __syncthreads();                             // every thread is done reading Zs
#pragma unroll
  for (int q = 0; q < CPT; ++q) Zs[row * D + c0 + q] = x[q];    // Zs now holds X[rows]
  const float total = block_sum(part, red);    // its barriers order the X stores before the reads
  if (tid == 0) a.lpart[blockIdx.x] = total;
  const T* __restrict__ Wq = reinterpret_cast<const T*>(a.Wq) + (size_t)h * D * r;
  const T* __restrict__ Wk = reinterpret_cast<const T*>(a.Wk) + (size_t)h * D * r;
  float* __restrict__ pq = a.qpart + (size_t)bh * D * r;                     // rows e0.. of this (b,h)
  float* __restrict__ pk = a.kpart + (size_t)blockIdx.x * D * r;             // all rows, this block
  for (int i = tid; i < kRB * r; i += kThreads) {
    const int rr = i / r, c = i - rr * r;
    float sq = 0.f;
    for (int g = 0; g < D; ++g) sq = fmaf(Zs[rr * D + g], to_f32(Wk[g * r + c]), sq);
    pq[(size_t)(e0 + rr) * r + c] = sq;
  }
  for (int i = tid; i < D * r; i += kThreads) {
    const int f = i / r, c = i - f * r;
    float sk = 0.f;
#pragma unroll
    for (int rr = 0; rr < kRB; ++rr) sk = fmaf(Zs[rr * D + f], to_f32(Wq[(e0 + rr) * r + c]), sk);
    pk[i] = sk;
  }
}

// Fixed-order sums: loss[b,h] over row blocks; dWq[h] over b; dWk[h] over b, then
// row blocks.  One thread per output value (plus one per loss).
template <int D>
__global__ __launch_bounds__(kThreads) void pg_reduce_kernel(PGradArgs a) {
  constexpr int RBS = D / kRB;
  const int i = blockIdx.x * kThreads + threadIdx.x;
  const int r = a.r;
  const int nw = a.H * D * r;
  const float nb2 = (float)a.NB * (float)a.NB;
  const float cs = 2.f / nb2;
  if (i < nw) {
    const int h = i / (D * r), rem = i - h * D * r;
    float sq = 0.f, sk = 0.f;
    for (int b = 0; b < a.B; ++b) {
      const int bh = b * a.H + h;
      sq += a.qpart[(size_t)bh * D * r + rem];
      for (int rb = 0; rb < RBS; ++rb) sk += a.kpart[((size_t)bh * RBS + rb) * D * r + rem];
    }
    a.dWq[i] = cs * sq;
    a.dWk[i] = cs * sk;
  } else if (i < nw + a.B * a.H) {
    const int bh = i - nw;
    float s = 0.f;
    for (int rb = 0; rb < RBS; ++rb) s += a.lpart[bh * RBS + rb];
    a.loss[bh] = s / nb2;
  }
}

template <typename T, int D>
hipError_t launch_t(const PGradArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  constexpr int TILES = D / kGT;
  hipLaunchKernelGGL((gram_kernel<D>), dim3(2 * BH * TILES * (TILES + 1) / 2), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL((pg_m_kernel<T, D>), dim3((a.H * D * D + kThreads - 1) / kThreads), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL((pg_x_kernel<T, D>), dim3(BH * (D / kRB)), dim3(kThreads), 0, s, a);
  const int n = a.H * D * a.r + BH;
  hipLaunchKernelGGL((pg_reduce_kernel<D>), dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

size_t predictor_grad_workspace_bytes(int BH, int H, int NB, int d) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rbs = d / kRB;
  return 2 * al((size_t)BH * NB * d * 4) + 2 * al((size_t)BH * d * d * 4) + al((size_t)H * d * d * 4) +
         al((size_t)BH * d * 64 * 4) + al((size_t)BH * rbs * d * 64 * 4) + al((size_t)BH * rbs * 4);
}

void predictor_grad_carve(PGradArgs& a, void* workspace, int BH, int H, int NB, int d) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rbs = d / kRB;
  char* w = static_cast<char*>(workspace);
  const size_t sizes[8] = {al((size_t)BH * NB * d * 4), al((size_t)BH * NB * d * 4), al((size_t)BH * d * d * 4),
                           al((size_t)BH * d * d * 4),  al((size_t)H * d * d * 4),    al((size_t)BH * d * 64 * 4),
                           al((size_t)BH * rbs * d * 64 * 4), al((size_t)BH * rbs * 4)};
  float* p[8];
  for (int i = 0; i < 8; ++i) {
    p[i] = reinterpret_cast<float*>(w);
    w += sizes[i];
  }
  a.Pq = p[0]; a.Pk = p[1]; a.Gq = p[2]; a.Gk = p[3]; a.M = p[4]; a.qpart = p[5]; a.kpart = p[6]; a.lpart = p[7];
}

hipError_t launch_predictor_grad(const PGradArgs& a, int io_f32, int d, hipStream_t s) {
  if (io_f32) return d == 64 ? launch_t<float, 64>(a, s) : launch_t<float, 128>(a, s);
  return d == 64 ? launch_t<bf16, 64>(a, s) : launch_t<bf16, 128>(a, s);
}

}  // namespace dsa
