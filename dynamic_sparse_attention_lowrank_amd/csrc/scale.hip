// Power-of-two scale of a bf16 tensor per (b, h) for the fp16 matrix-core
// products of the attention kernels (gfx950).
//
// fp16 keeps 11 significant bits, more than bf16's 8, but only 5 exponent bits: a
// plain bf16 -> fp16 conversion overflows at 65504 and drops bits below 2^-17.
// Multiplying a head's values by 2^s, with s chosen so that the head's largest
// magnitude lands in [2^14, 2^15), makes the conversion exact for every element
// within a factor 2^31 of that maximum whatever the size of the values; the
// products are brought back by 2^-s in fp32, exactly.  Because s only depends on
// the exponent of the maximum, scaling the input by any power of two (within
// range) leaves the fp16 copy bit for bit unchanged.
//   (a) per-chunk maxima of the magnitude bits: for finite bf16 values the integer
//       order of (bits & 0x7fff) is the order of |x|, and a maximum is order-free;
//   (b) one wave per (b, h): s = 14 - floor(log2 max|x|), clamped to [-63, 63]
//       (so 2^s, 2^-s and the product of two such scales stay normal floats);
//       s = 0 for an all-zero head or one holding inf / NaN.
// Also here: the scaled fp16 copy itself (pow2_convert) and per-head maxima of
// |x| for float data (absmax_f32).
#include "kernels.hpp"

namespace dsa {

namespace {

// largest bf16 magnitude pattern among the 8 values of a 16-byte chunk
__device__ __forceinline__ uint32_t chunk_absmax(u32x4 v) {
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) m = max(m, max(v[e] & 0x7fffu, (v[e] >> 16) & 0x7fffu));
  return m;
}

// grid-stride over the chunks of one head, four loads in flight per thread
__global__ __launch_bounds__(256) void absmax_kernel(const void* X, size_t chunks16, uint32_t* partial) {
  const int bh = blockIdx.x / kDoChunks, c = blockIdx.x - bh * kDoChunks;
  const u32x4* __restrict__ p = reinterpret_cast<const u32x4*>(X) + (size_t)bh * chunks16;
  constexpr size_t kStride = (size_t)kDoChunks * 256;
  uint32_t m = 0;
  size_t i = (size_t)c * 256 + threadIdx.x;
  for (; i + 3 * kStride < chunks16; i += 4 * kStride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = p[i + u * kStride];
#pragma unroll
    for (int u = 0; u < 4; ++u) m = max(m, chunk_absmax(v[u]));
  }
  for (; i < chunks16; i += kStride) m = max(m, chunk_absmax(p[i]));
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s, 64));
  __shared__ uint32_t wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = max(max(wm[0], wm[1]), max(wm[2], wm[3]));
}

static_assert(kDoChunks == 64, "one lane per chunk");
__global__ __launch_bounds__(64) void pow2_scale_kernel(const uint32_t* partial, float2* scale) {
  const int bh = blockIdx.x;
  uint32_t m = partial[(size_t)bh * kDoChunks + threadIdx.x];
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s, 64));
  if (threadIdx.x == 0) {
    int s = 0;
    if (m != 0u && m < 0x7f80u) {
      const int e = (int)(m >> 7);            // biased exponent (0: subnormal, below 2^-126)
      s = e == 0 ? 63 : 14 - (e - 127);
      s = s < -63 ? -63 : (s > 63 ? 63 : s);
    }
    scale[bh] = make_float2(__uint_as_float((uint32_t)(127 + s) << 23), __uint_as_float((uint32_t)(127 - s) << 23));
  }
}

// out = fp16(x * 2^s) for 8 consecutive bf16 values per thread-iteration; grid
// (chunk blocks, heads)
__global__ __launch_bounds__(256) void pow2_convert_kernel(const void* X, size_t chunks_per_head, const float2* scale,
                                                           void* out) {
  const size_t head = (size_t)blockIdx.y * chunks_per_head;
  const u32x4* __restrict__ x = reinterpret_cast<const u32x4*>(X) + head;
  u32x4* __restrict__ o = reinterpret_cast<u32x4*>(out) + head;
  const float up = scale[blockIdx.y].x;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < chunks_per_head; i += (size_t)gridDim.x * 256) {
    const bf16x8 v = __builtin_bit_cast(bf16x8, x[i]);
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (f16)((float)v[e] * up);
    o[i] = __builtin_bit_cast(u32x4, h);
  }
}

// per-chunk maxima of |x| for float data (bits of fabs: integer order = order of |x|)
__global__ __launch_bounds__(256) void absmax_f32_kernel(const float* X, size_t per_head, uint32_t* partial) {
  const int bh = blockIdx.x / kDoChunks, c = blockIdx.x - bh * kDoChunks;
  const float* __restrict__ p = X + (size_t)bh * per_head;
  uint32_t m = 0;
  for (size_t i = (size_t)c * 256 + threadIdx.x; i < per_head; i += (size_t)kDoChunks * 256)
    m = max(m, __float_as_uint(p[i]) & 0x7fffffffu);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s, 64));
  __shared__ uint32_t wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = max(max(wm[0], wm[1]), max(wm[2], wm[3]));
}

__global__ __launch_bounds__(64) void max_reduce_kernel(const uint32_t* partial, uint32_t* out) {
  uint32_t m = partial[(size_t)blockIdx.x * kDoChunks + threadIdx.x];
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s, 64));
  if (threadIdx.x == 0) out[blockIdx.x] = m;
}

}  // namespace

hipError_t launch_pow2_convert(const void* X, int BH, size_t elems_per_head, const float2* scale, void* out,
                               hipStream_t s) {
  const size_t cph = elems_per_head / 8;
  const size_t gx = (cph + 255) / 256;
  hipLaunchKernelGGL(pow2_convert_kernel, dim3((unsigned)(gx < 512 ? gx : 512), (unsigned)BH), dim3(256), 0, s, X, cph,
                     scale, out);
  return hipGetLastError();
}

hipError_t launch_absmax_f32(const float* X, int BH, size_t elems_per_head, uint32_t* partial, uint32_t* out,
                             hipStream_t s) {
  hipLaunchKernelGGL(absmax_f32_kernel, dim3((unsigned)(BH * kDoChunks)), dim3(256), 0, s, X, elems_per_head, partial);
  hipLaunchKernelGGL(max_reduce_kernel, dim3((unsigned)BH), dim3(64), 0, s, partial, out);
  return hipGetLastError();
}

hipError_t launch_pow2_scale(const void* X, int BH, size_t elems_per_head, uint32_t* partial, float2* scale,
                             hipStream_t s) {
  hipLaunchKernelGGL(absmax_kernel, dim3((unsigned)(BH * kDoChunks)), dim3(256), 0, s, X, elems_per_head / 8, partial);
  hipLaunchKernelGGL(pow2_scale_kernel, dim3((unsigned)BH), dim3(64), 0, s, partial, scale);
  return hipGetLastError();
}

}  // namespace dsa
