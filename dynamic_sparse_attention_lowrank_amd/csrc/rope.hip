// 3-D rotary positions for gfx950 (second page, gist.science/ar/paper/2603.06664,
// section 2: a frame's time position is its chunk's start index plus its index
// inside the chunk -- a global time index -- so each device computes positions
// locally).  The page gives no formula; this library reads it as rotary encoding
// per axis: the head dimension is cut into a time, a height and a width section
// of adjacent pairs (time takes what a three-way split of the d/2 pairs leaves:
// 22/21/21 at d = 128), and pair i of a section of 2m dimensions is turned by
//   angle = (coordinate on that axis + offset) * base^(-2i / 2m).
// Applied to Q and K once per layer (the rotated tensors, stored in their own
// dtype, are what the predictor and the attention read); the inverse rotation
// maps the gradients of the rotated tensors back.
//
// Kernel: one thread per 16-byte chunk of a token row (4 bf16 or 2 fp32 pairs):
// the angles, sines and cosines of its pairs are computed once (fp32, accurate
// sincosf) and applied to those pairs in every (b, h) row, so every load and store
// is a full 16 bytes per lane and coalesced.  HBM-bound: reads and writes the
// tensor once.  Tensors that are only pair-aligned (a view at an odd offset) take
// the same arithmetic one pair per thread.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeUnroll = 4;                // (b, h) rows in flight per thread

template <typename T>
struct Pair2;
template <>
struct Pair2<bf16> {
  typedef uint32_t raw;
  static __device__ __forceinline__ void get(raw r, float& u, float& v) {
    u = __uint_as_float(r << 16);
    v = __uint_as_float(r & 0xffff0000u);
  }
  static __device__ __forceinline__ raw put(float u, float v) {
    const bf16 a = (bf16)u, b = (bf16)v;        // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  }
};
template <>
struct Pair2<float> {
  typedef float2 raw;
  static __device__ __forceinline__ void get(raw r, float& u, float& v) {
    u = r.x;
    v = r.y;
  }
  static __device__ __forceinline__ raw put(float u, float v) { return make_float2(u, v); }
};

// sine and cosine of the rotation of pair p of token n
__device__ __forceinline__ void pair_angle(const RopeArgs& a, int n, int p, float& sn, float& cs) {
  const Geo& g = a.g;
  const int pairs = a.d / 2;
  // section of pair p and its index inside the section
  const int m_t = pairs - 2 * (pairs / 3), m_s = pairs / 3;
  int axis, li, m;
  if (p < m_t) {
    axis = 0; li = p; m = m_t;
  } else if (p < m_t + m_s) {
    axis = 1; li = p - m_t; m = m_s;
  } else {
    axis = 2; li = p - m_t - m_s; m = m_s;
  }
  const int plane = g.Lh * g.Lw;
  const int pos = axis == 0 ? n / plane + a.t0 : (axis == 1 ? (n / g.Lw) % g.Lh + a.y0 : n % g.Lw + a.x0);
  const float freq = exp2f(-(float)(2 * li) / (float)(2 * m) * a.log2_base);
  sincosf((float)pos * freq, &sn, &cs);
  if (a.inverse) sn = -sn;
}

// 16-byte chunks: P pairs per thread (both tensors 16-byte aligned)
template <typename T>
__global__ __launch_bounds__(kRopeThreads) void rope3d_chunk_kernel(RopeArgs a) {
  typedef typename Pair2<T>::raw raw;
  constexpr int P = 16 / (int)sizeof(raw);
  const int cpr = a.d / 2 / P;                 // chunks per token row
  const long long i = (long long)blockIdx.x * kRopeThreads + threadIdx.x;
  if (i >= (long long)a.g.N * cpr) return;
  const int n = (int)(i / cpr), c = (int)(i - (long long)n * cpr);
  float sn[P], cs[P];
#pragma unroll
  for (int e = 0; e < P; ++e) pair_angle(a, n, c * P + e, sn[e], cs[e]);

  const u32x4* __restrict__ X = reinterpret_cast<const u32x4*>(a.X);
  u32x4* __restrict__ Y = reinterpret_cast<u32x4*>(a.Y);
  const size_t row = (size_t)a.g.N * cpr;      // chunks per (b, h)
  for (int b0 = 0; b0 < a.BH; b0 += kRopeUnroll) {
    u32x4 v[kRopeUnroll];
#pragma unroll
    for (int u = 0; u < kRopeUnroll; ++u)
      if (b0 + u < a.BH) v[u] = X[(size_t)(b0 + u) * row + i];
#pragma unroll
    for (int u = 0; u < kRopeUnroll; ++u) {
      if (b0 + u < a.BH) {
        raw r[P];
        __builtin_memcpy(r, &v[u], 16);
#pragma unroll
        for (int e = 0; e < P; ++e) {
          float x0, x1;
          Pair2<T>::get(r[e], x0, x1);
          r[e] = Pair2<T>::put(fmaf(x0, cs[e], -x1 * sn[e]), fmaf(x0, sn[e], x1 * cs[e]));
        }
        u32x4 o;
        __builtin_memcpy(&o, r, 16);
        Y[(size_t)(b0 + u) * row + i] = o;
      }
    }
  }
}

// one pair per thread (tensors aligned to a pair only)
template <typename T>
__global__ __launch_bounds__(kRopeThreads) void rope3d_kernel(RopeArgs a) {
  typedef typename Pair2<T>::raw raw;
  const Geo g = a.g;
  const int pairs = a.d / 2;
  const long long i = (long long)blockIdx.x * kRopeThreads + threadIdx.x;
  if (i >= (long long)g.N * pairs) return;
  const int n = (int)(i / pairs), p = (int)(i - (long long)n * pairs);
  float sn, cs;
  pair_angle(a, n, p, sn, cs);

  const raw* __restrict__ X = reinterpret_cast<const raw*>(a.X);
  raw* __restrict__ Y = reinterpret_cast<raw*>(a.Y);
  const size_t row = (size_t)g.N * pairs;     // pairs per (b, h)
  for (int b0 = 0; b0 < a.BH; b0 += kRopeUnroll) {
    raw v[kRopeUnroll];
#pragma unroll
    for (int u = 0; u < kRopeUnroll; ++u)
      if (b0 + u < a.BH) v[u] = X[(size_t)(b0 + u) * row + i];
#pragma unroll
    for (int u = 0; u < kRopeUnroll; ++u) {
      if (b0 + u < a.BH) {
        float x0, x1;
        Pair2<T>::get(v[u], x0, x1);
        Y[(size_t)(b0 + u) * row + i] = Pair2<T>::put(fmaf(x0, cs, -x1 * sn), fmaf(x0, sn, x1 * cs));
      }
    }
  }
}

}  // namespace

hipError_t launch_rope3d(const RopeArgs& a, int f32, hipStream_t s) {
  if ((((uintptr_t)a.X | (uintptr_t)a.Y) & 15u) == 0) {
    const long long work = (long long)a.g.N * (a.d / 2) / (f32 ? 2 : 4);
    const unsigned grid = (unsigned)((work + kRopeThreads - 1) / kRopeThreads);
    if (f32)
      hipLaunchKernelGGL((rope3d_chunk_kernel<float>), dim3(grid), dim3(kRopeThreads), 0, s, a);
    else
      hipLaunchKernelGGL((rope3d_chunk_kernel<bf16>), dim3(grid), dim3(kRopeThreads), 0, s, a);
    return hipGetLastError();
  }
  const long long work = (long long)a.g.N * (a.d / 2);
  const unsigned grid = (unsigned)((work + kRopeThreads - 1) / kRopeThreads);
  if (f32)
    hipLaunchKernelGGL((rope3d_kernel<float>), dim3(grid), dim3(kRopeThreads), 0, s, a);
  else
    hipLaunchKernelGGL((rope3d_kernel<bf16>), dim3(grid), dim3(kRopeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
