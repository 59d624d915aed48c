// Low-rank block-score predictor for gfx950 (DSV page, gist.science/ar/paper/
// 2502.07590, section 3a: a small, cheap predictor looks at the data before the
// expensive attention and names the part worth attending to).
//
// Per head h and tile tau:
//   Qbar[tau] = mean over the tile's tokens of Q[n] @ Wq[h]       (r values)
//   Kbar[tau] = mean over the tile's tokens of K[n] @ Wk[h]
//   S[tau, j] = Qbar[tau] . Kbar[j]
// By linearity the mean is taken before the projection (one d-vector per tile,
// then one d x r product), which reads Q and K exactly once.  All sums are fp32.
//
// Kernel 1 (pool_project): one work-group per (tensor, head, tile); 16-byte
//   coalesced row loads (all of a thread's rows in flight at once), fp32 column
//   sums, LDS tree over token groups in a fixed order, then the d x r projection
//   split over all threads by d segments, summed in a fixed order (optionally also
//   stores the tile means, and with no Qbar/Kbar output only those, for the
//   predictor's training signal).
// Kernel 2 (scores): one work-group per (head, 64 query tiles, 256 key blocks);
//   a thread owns one key block, keeps its Kbar row in registers and writes 64
//   coalesced scores.  Bound by writing S.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int kPoolThreads = 256;

template <typename T, int D>
__device__ __forceinline__ void pool_project_body(const PredictArgs& a) {
  constexpr int CE = Elem<T>::kChunkElems;
  constexpr int CPR = D / CE;                  // 16-byte chunks per token row
  constexpr int RPG = kPoolThreads / CPR;      // token rows loaded per pass
  __shared__ float red[RPG * D];
  __shared__ float xmean[D];

  const Geo g = a.g;
  const int BH = a.B * a.H;
  const int per = BH * g.NB;
  const int which = (int)blockIdx.x >= per;    // 0: Q, 1: K
  const int L = blockIdx.x - which * per;
  const int bh = L / g.NB;
  const int tau = L - bh * g.NB;
  const int head = bh % a.H;
  const int tid = threadIdx.x;
  const T* __restrict__ X = reinterpret_cast<const T*>(which ? a.K : a.Q) + (size_t)bh * g.N * D;
  const T* __restrict__ W = reinterpret_cast<const T*>(which ? a.Wk : a.Wq) + (size_t)head * D * a.r;
  float* __restrict__ out = which ? a.Kbar : a.Qbar;

  const int c = tid % CPR, rsub = tid / CPR;
  float acc[CE];
#pragma unroll
  for (int e = 0; e < CE; ++e) acc[e] = 0.f;
  const int base = tile_base(g, tau);
  // rows rsub, rsub + RPG, ... (T <= 64): every load issued before the first add;
  // absent rows load zeros, which leave the sums unchanged
  constexpr int MAXR = (64 + RPG - 1) / RPG;
  u32x4 ch[MAXR];
#pragma unroll
  for (int q = 0; q < MAXR; ++q) {
    const int i = rsub + q * RPG;
    ch[q] = i < g.T ? *reinterpret_cast<const u32x4*>(X + (size_t)(base + member_offset(g, i)) * D + c * CE)
                    : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int q = 0; q < MAXR; ++q) {
    const T* v = reinterpret_cast<const T*>(&ch[q]);
#pragma unroll
    for (int e = 0; e < CE; ++e) acc[e] += to_f32(v[e]);
  }
#pragma unroll
  for (int e = 0; e < CE; ++e) red[rsub * D + c * CE + e] = acc[e];
  __syncthreads();
  float* __restrict__ P = which ? a.Pk : a.Pq;
  if (tid < D) {
    float s = 0.f;
    for (int q = 0; q < RPG; ++q) s += red[q * D + tid];
    xmean[tid] = s / (float)g.T;
    if (P) P[((size_t)bh * g.NB + tau) * D + tid] = xmean[tid];
  }
  if (!out) return;                            // tile means only
  __syncthreads();
  // projection on all threads: column cc of W over one of nseg contiguous d
  // segments, then the segments summed in order (rp = r rounded up to 16/32/64)
  const int rp = a.r <= 16 ? 16 : (a.r <= 32 ? 32 : 64);
  const int nseg = kPoolThreads / rp;
  const int cc = tid % rp, sg = tid / rp, len = D / nseg;
  float o = 0.f;
  if (cc < a.r) {
    for (int e = sg * len; e < (sg + 1) * len; ++e) o = fmaf(xmean[e], to_f32(W[e * a.r + cc]), o);
  }
  red[sg * rp + cc] = o;                       // red is free once xmean is formed
  __syncthreads();
  if (tid < a.r) {
    float t = 0.f;
    for (int q = 0; q < nseg; ++q) t += red[q * rp + tid];
    out[((size_t)bh * g.NB + tau) * a.r + tid] = t;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_project_kernel(PredictArgs a) {
  pool_project_body<T, D>(a);
}

// the same body with tile means only (Qbar = Kbar = null), named apart so that
// profiles keep the predictor's pooling and the training signal's apart
template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void tile_mean_kernel(PredictArgs a) {
  pool_project_body<T, D>(a);
}

constexpr int kScoreRows = 64;
constexpr int kScoreCols = 256;

template <int RM>
__global__ __launch_bounds__(kScoreCols) void scores_kernel(PredictArgs a) {
  __shared__ float qs[kScoreRows][RM];
  const int NB = a.g.NB;
  const int r = a.r;
  const int bh = blockIdx.z;
  const int row0 = blockIdx.y * kScoreRows;
  const int j = blockIdx.x * kScoreCols + threadIdx.x;
  const float* __restrict__ Qb = a.Qbar + (size_t)bh * NB * r;
  const float* __restrict__ Kb = a.Kbar + (size_t)bh * NB * r;
  for (int t = threadIdx.x; t < kScoreRows * RM; t += kScoreCols) {
    const int rr = t / RM, cc = t % RM;
    qs[rr][cc] = (row0 + rr < NB && cc < r) ? Qb[(size_t)(row0 + rr) * r + cc] : 0.f;
  }
  float kr[RM];
#pragma unroll
  for (int cc = 0; cc < RM; ++cc) kr[cc] = (j < NB && cc < r) ? Kb[(size_t)j * r + cc] : 0.f;
  __syncthreads();
  if (j >= NB) return;
  float* __restrict__ Sb = a.S + (size_t)bh * NB * NB;
  const int rows = NB - row0 < kScoreRows ? NB - row0 : kScoreRows;
  for (int rr = 0; rr < rows; ++rr) {
    float s = 0.f;
#pragma unroll
    for (int cc = 0; cc < RM; ++cc) s = fmaf(qs[rr][cc], kr[cc], s);
    Sb[(size_t)(row0 + rr) * NB + j] = s;
  }
}

template <typename T, int D>
hipError_t launch_pool(const PredictArgs& a, hipStream_t s) {
  const int grid = 2 * a.B * a.H * a.g.NB;
  if (a.Qbar)
    hipLaunchKernelGGL((pool_project_kernel<T, D>), dim3(grid), dim3(kPoolThreads), 0, s, a);
  else
    hipLaunchKernelGGL((tile_mean_kernel<T, D>), dim3(grid), dim3(kPoolThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool_project(const PredictArgs& a, int io_f32, int d, hipStream_t s) {
  if (io_f32) return d == 64 ? launch_pool<float, 64>(a, s) : launch_pool<float, 128>(a, s);
  return d == 64 ? launch_pool<bf16, 64>(a, s) : launch_pool<bf16, 128>(a, s);
}

hipError_t launch_predict(const PredictArgs& a, int io_f32, int d, hipStream_t s) {
  hipError_t e = launch_pool_project(a, io_f32, d, s);
  if (e != hipSuccess) return e;
  const int NB = a.g.NB;
  dim3 grid((NB + kScoreCols - 1) / kScoreCols, (NB + kScoreRows - 1) / kScoreRows, a.B * a.H);
  if (a.r <= 16) hipLaunchKernelGGL((scores_kernel<16>), grid, dim3(kScoreCols), 0, s, a);
  else if (a.r <= 32) hipLaunchKernelGGL((scores_kernel<32>), grid, dim3(kScoreCols), 0, s, a);
  else hipLaunchKernelGGL((scores_kernel<64>), grid, dim3(kScoreCols), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
