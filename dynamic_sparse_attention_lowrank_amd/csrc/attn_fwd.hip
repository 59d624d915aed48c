// Block-sparse attention forward for gfx950.
//
// Computes, for every query token of a query tile, exact softmax attention over
// the keys of the key blocks that the tile kept (DSV page, gist.science/ar/paper/
// 2502.07590, section 4: stage two computes only the cues the predictor picked;
// section 3b: one selection per tile of neighbouring queries).
//
// One work-group (2 waves) per query tile of T <= 64 tokens; wave w owns query
// rows 32w..32w+31.  The work-group walks its kept blocks; each block's K rows
// (row-major) and V rows (transposed) are staged in LDS, and the next block's
// global loads are issued before the current block is computed.  Per block and
// wave:
//   S^T (keys x queries) = K Q^T       -- Q fragments live in registers
//   online softmax in fp32, base 2, one query per lane (lanes l and l^32 share)
//   O^T (d x queries)   += V^T P^T     -- P^T is taken straight from the S^T
//                                         registers (perm16 layout)
// With bf16 inputs the P.V product runs on fp16 matrix cores: V is converted
// to fp16 while it is transposed into LDS (exact for |v| in the fp16 normal
// range, |v| < 65504) and the probabilities are rounded to fp16 (relative error
// 2^-12 instead of bf16's 2^-9, which keeps max-abs output errors near 1e-3 even
// for peaked attention over large values).
// The running maximum only moves when a row's new maximum exceeds it by more
// than 2^8, so most blocks skip rescaling O.  This is exact: every exponential
// and the final normalisation use the same maximum.
#include "kernels.hpp"
#include "tiles.hpp"

namespace dsa {

namespace {

constexpr float kRescaleSlack = 8.0f;   // log2 units

// element type of the P.V product operands
template <typename T> struct PVType;
template <> struct PVType<bf16> { typedef f16 type; };
template <> struct PVType<float> { typedef float type; };

template <typename T, int D>
__global__ __launch_bounds__(kTileThreads) void attn_fwd_kernel(FwdArgs a) {
  using C = TileCfg<T, D>;
  typedef typename Elem<T>::frag Frag;
  typedef typename PVType<T>::type PT;
  typedef typename Elem<PT>::frag PFrag;
  __shared__ u32x4 lds_k[C::kRowChunks];
  __shared__ u32x4 lds_vt[TileCfg<PT, D>::kTrChunks];

  const Geo g = a.g;
  const int L = xcd_remap(blockIdx.x, a.BH * g.NB);
  const int bh = L / g.NB;
  const int tau = L - bh * g.NB;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, h = lane >> 5;

  const size_t head_off = (size_t)bh * g.N * D;
  const T* __restrict__ Qh = reinterpret_cast<const T*>(a.Q) + head_off;
  const T* __restrict__ Kh = reinterpret_cast<const T*>(a.K) + head_off;
  const T* __restrict__ Vh = reinterpret_cast<const T*>(a.V) + head_off;
  const int* __restrict__ irow = a.idx + ((size_t)bh * g.NB + tau) * a.kmax;
  int kk = a.kvec[bh];
  kk = kk < 1 ? 1 : (kk > a.kmax ? a.kmax : kk);

  int koff[C::kRowPer];
  row_offsets<T, D>(koff, g, tid);
  int voff[C::kGPer][8];
  group_offsets<T, D>(voff, g, tid);

  const int q = 32 * wave + l32;
  const bool q_ok = q < g.T;
  const int q_tok = tile_base(g, tau) + (q_ok ? member_offset(g, q) : 0);
  Frag qf[C::kSteps];
  load_row_frags<T, D>(qf, Qh + (size_t)q_tok * D, q_ok, h);

  f32x16 oacc[C::kDTiles];
#pragma unroll
  for (int t = 0; t < C::kDTiles; ++t) oacc[t] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c2 = a.c;

  int slot = 0;
  while (slot < kk && (unsigned)irow[slot] >= (unsigned)g.NB) ++slot;
  RowStage<T, D> kst;
  GroupStage<T, D> vst;
  if (slot < kk) {
    const int base = tile_base(g, irow[slot]);
    row_load<T, D>(kst, Kh, base, koff, tid);
    group_load<T, D>(vst, Vh, base, voff, tid);
  }

  while (slot < kk) {
    __syncthreads();
    row_store<T, D>(kst, lds_k, tid);
    group_store<T, D, PT>(vst, lds_vt, nullptr, tid);
    __syncthreads();
    int nxt = slot + 1;
    while (nxt < kk && (unsigned)irow[nxt] >= (unsigned)g.NB) ++nxt;
    if (nxt < kk) {
      const int base = tile_base(g, irow[nxt]);
      row_load<T, D>(kst, Kh, base, koff, tid);
      group_load<T, D>(vst, Vh, base, voff, tid);
    }

    // ---- S^T = K Q^T : two 32-key tiles
    f32x16 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = f32x16{};
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s)
        sacc[mt] = mma_step(frag_row<T, D>(lds_k, 32 * mt + l32, s, h), qf[s], sacc[mt]);
    }
    // ---- mask padding keys; block maximum per query
    float mb = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
        if (key >= g.T) sacc[mt][i] = -INFINITY;
        mb = fmaxf(mb, sacc[mt][i]);
      }
    }
    mb = fmaxf(mb, xor32(mb));
    const float mnew = mb * c2;
    if (ballot(mnew > m_run + kRescaleSlack)) {
      const float mt_ = fmaxf(m_run, mnew);
      const float alpha = (mt_ == -INFINITY) ? 1.f : fast_exp2(m_run - mt_);
      m_run = mt_;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < C::kDTiles; ++t) oacc[t] *= alpha;
    }
    // ---- unnormalised probabilities as B fragments of O^T += V^T P^T
    PFrag pf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = fast_exp2(fmaf(sacc[s >> 1][8 * (s & 1) + e], c2, -m_run));
        l_run += p;
        pv[e] = p;
      }
      pf[s] = to_frag(pv, (PT*)nullptr);
    }
#pragma unroll
    for (int t = 0; t < C::kDTiles; ++t) {
#pragma unroll
      for (int s = 0; s < 4; ++s) oacc[t] = mma_step(frag_tr<PT, D>(lds_vt, 32 * t + l32, s, h), pf[s], oacc[t]);
    }
    slot = nxt;
  }

  // ---- normalise and store: lane holds query q, d = 32t + 8g + 4h + i
  const float l_tot = l_run + xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    const size_t orow = head_off + (size_t)q_tok * D;
#pragma unroll
    for (int t = 0; t < C::kDTiles; ++t) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        store4(a.O, orow + 32 * t + 8 * gq + 4 * h, a.out_f32, oacc[t][4 * gq] * inv, oacc[t][4 * gq + 1] * inv,
               oacc[t][4 * gq + 2] * inv, oacc[t][4 * gq + 3] * inv);
      }
    }
    if (h == 0) a.LSE[(size_t)bh * g.N + q_tok] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd_kernel<T, D>), dim3(a.BH * a.g.NB), dim3(kTileThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const FwdArgs& a, int io_f32, int d, hipStream_t s) {
  if (io_f32) return d == 64 ? launch_fwd<float, 64>(a, s) : launch_fwd<float, 128>(a, s);
  return d == 64 ? launch_fwd<bf16, 64>(a, s) : launch_fwd<bf16, 128>(a, s);
}

}  // namespace dsa
