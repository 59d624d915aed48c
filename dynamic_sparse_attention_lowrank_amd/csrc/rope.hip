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
// Kernel: one thread per (token, pair): its angle, sine and cosine are computed
// once (fp32, accurate sincosf) and applied to that pair in every (b, h) row; a
// wave covers one 256-byte token row (d = 128, bf16) per (b, h), so every load and
// store is coalesced.  HBM-bound: reads and writes the tensor once.
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

template <typename T>
__global__ __launch_bounds__(kRopeThreads) void rope3d_kernel(RopeArgs a) {
  typedef typename Pair2<T>::raw raw;
  const Geo g = a.g;
  const int pairs = a.d / 2;
  const long long i = (long long)blockIdx.x * kRopeThreads + threadIdx.x;
  if (i >= (long long)g.N * pairs) return;
  const int n = (int)(i / pairs), p = (int)(i - (long long)n * pairs);
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
  float sn, cs;
  sincosf((float)pos * freq, &sn, &cs);
  if (a.inverse) sn = -sn;

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
  const long long work = (long long)a.g.N * (a.d / 2);
  const unsigned grid = (unsigned)((work + kRopeThreads - 1) / kRopeThreads);
  if (f32)
    hipLaunchKernelGGL((rope3d_kernel<float>), dim3(grid), dim3(kRopeThreads), 0, s, a);
  else
    hipLaunchKernelGGL((rope3d_kernel<bf16>), dim3(grid), dim3(kRopeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
