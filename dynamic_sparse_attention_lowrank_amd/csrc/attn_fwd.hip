// Block-sparse attention forward for gfx950.
//
// Computes, for every query token of a query tile, exact softmax attention over
// the keys of the key blocks that the tile kept (DSV page, gist.science/ar/paper/
// 2502.07590, section 4: stage two computes only the cues the predictor picked;
// section 3b: one selection per tile of neighbouring queries).
//
// Two kernels:
//  1. vt_prep: every key block's V rows, transposed to [d][64 key positions] (key
//     positions in perm16 order, padding keys zero) and, for bf16 inputs,
//     converted to fp16.  One HBM pass; afterwards a block's V^T is 16 KB of
//     contiguous memory from which MFMA A fragments load directly.  Each block
//     is gathered by ~k query tiles, so transposing once replaces k transposes.
//  2. attn_fwd: one work-group (2 waves) per query tile of T <= 64 tokens.  Wave
//     w takes key positions 32w..32w+31 of every kept block for all 64 query
//     rows, so each wave loads only its half of K and V^T, straight from L2 into
//     registers (no LDS staging), double-buffered one block ahead:
//        S^T (32 keys x 64 queries) = K Q^T          16 MFMA, Q in registers
//        online softmax (fp32, base 2), one query per lane and N-tile
//        O^T (d x 64 queries)      += V^T P^T        16 MFMA, P^T taken straight
//                                                    from the S^T registers
//     Each wave keeps its own running max / sum / O over its key half; the two
//     halves are merged once, through LDS, at the end.
// With bf16 inputs the P.V product runs on fp16 matrix cores (V converted in
// vt_prep, exact for |v| < 65504; P rounded to fp16, 2^-12 relative).  The
// running maximum only moves when a row's maximum grows by more than 2^8, so
// most blocks skip rescaling O; this is exact (numerator and denominator share
// the maximum).
#include "kernels.hpp"
#include "tiles.hpp"

namespace dsa {

namespace {

constexpr float kRescaleSlack = 8.0f;   // log2 units

template <typename T> struct PVType;
template <> struct PVType<bf16> { typedef f16 type; };
template <> struct PVType<float> { typedef float type; };

// ------------------------------------------------------------ 1. V -> V^T blocks
// One work-group of 256 threads per (head, block): rows in (coalesced 16-byte
// chunks) -> LDS [64][D] fp32 -> out as [D][64] rows of the P.V element type.
template <typename T, int D>
__global__ __launch_bounds__(256) void vt_prep_kernel(FwdArgs a) {
  typedef typename PVType<T>::type PT;
  constexpr int CE = Elem<T>::kChunkElems;
  constexpr int CPR = D / CE;
  __shared__ float tile[64][D + 1];
  const Geo g = a.g;
  const int bj = blockIdx.x;                 // bh * NB + j
  const int bh = bj / g.NB, j = bj - bh * g.NB;
  const T* __restrict__ Vh = reinterpret_cast<const T*>(a.V) + (size_t)bh * g.N * D;
  const int base = tile_base(g, j);
  for (int it = threadIdx.x; it < 64 * CPR; it += 256) {
    const int r = it / CPR, c = it % CPR;                  // r: key (member) index
    float v[CE];
    if (r < g.T) {
      const u32x4 ch = *reinterpret_cast<const u32x4*>(Vh + (size_t)(base + member_offset(g, r)) * D + c * CE);
      const T* e = reinterpret_cast<const T*>(&ch);
#pragma unroll
      for (int q = 0; q < CE; ++q) v[q] = to_f32(e[q]);
    } else {
#pragma unroll
      for (int q = 0; q < CE; ++q) v[q] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < CE; ++q) tile[r][c * CE + q] = v[q];
  }
  __syncthreads();
  PT* __restrict__ out = reinterpret_cast<PT*>(a.Vt) + (size_t)bj * D * 64;
  for (int it = threadIdx.x; it < D * 64; it += 256) {
    const int d = it >> 6, p = it & 63;                    // position p holds key 16*(p/16) + perm16(p%16)
    out[it] = (PT)tile[16 * (p >> 4) + perm16(p & 15)][d];
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

// kvoff: lane byte offset of (key row, element 8h) inside a tile; ksoff: the tile's first row
template <typename T, int D>
__device__ __forceinline__ void load_k(KFrags<T, D>& kf, __amdgpu_buffer_rsrc_t rk, int kvoff, int ksoff) {
  using C = FwdCfg<T, D>;
  constexpr int CE = Elem<T>::kChunkElems, FC = Elem<T>::kFragChunks;
#pragma unroll
  for (int s = 0; s < C::kSteps; ++s) {
    u32x4 ch[FC];
#pragma unroll
    for (int q = 0; q < FC; ++q) ch[q] = bload(rk, kvoff + (16 * s + q * CE) * (int)sizeof(T), ksoff);
    kf.f[s] = frag_from_chunks(ch, (T*)nullptr);
  }
}
// vvoff: lane byte offset of (row l32, position 32w + 8h) inside a block's V^T; vsoff: the block
template <typename T, int D>
__device__ __forceinline__ void load_v(VFrags<T, D>& vf, __amdgpu_buffer_rsrc_t rv, int vvoff, int vsoff) {
  using C = FwdCfg<T, D>;
  typedef typename C::PT PT;
  constexpr int PE = Elem<PT>::kChunkElems, PFC = Elem<PT>::kFragChunks;
#pragma unroll
  for (int t = 0; t < C::kDTiles; ++t) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 ch[PFC];
#pragma unroll
      for (int q = 0; q < PFC; ++q)
        ch[q] = bload(rv, vvoff + (16 * s + q * PE) * (int)sizeof(PT), vsoff + 32 * t * 64 * (int)sizeof(PT));
      vf.f[t][s] = frag_from_chunks(ch, (PT*)nullptr);
    }
  }
}

template <typename T, int D>
struct WaveState {
  f32x16 o[2][FwdCfg<T, D>::kDTiles];   // O^T per query N-tile and d tile
  float m[2], l[2];                      // running max (log2 units) and lane-partial sum per N-tile
};

template <typename T, int D>
__device__ __forceinline__ void attend_block(WaveState<T, D>& st, const KFrags<T, D>& kf, const VFrags<T, D>& vf,
                                             const typename Elem<T>::frag (*qf)[FwdCfg<T, D>::kSteps],
                                             float c2, int kvalid, int h) {
  using C = FwdCfg<T, D>;
  typedef typename C::PT PT;
  typedef typename Elem<PT>::frag PFrag;
  f32x16 s[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    s[nt] = f32x16{};
#pragma unroll
    for (int k = 0; k < C::kSteps; ++k) s[nt] = mma_step(kf.f[k], qf[nt][k], s[nt]);
  }
  if (kvalid < 32) {                        // padding keys of this wave's half (T < 64 only)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + 4 * h + (i & 3) >= kvalid) s[nt][i] = -INFINITY;
    }
  }
  PFrag pf[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float mb = s[nt][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mb = fmaxf(mb, s[nt][i]);
    mb = fmaxf(mb, xor32(mb));
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
      for (int e = 0; e < 8; ++e) {
        const float p = fast_exp2(fmaf(s[nt][8 * ks + e], c2, mneg));
        st.l[nt] += p;
        pv[e] = p;
      }
      pf[nt][ks] = to_frag(pv, (PT*)nullptr);
    }
  }
#pragma unroll
  for (int t = 0; t < C::kDTiles; ++t) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) st.o[nt][t] = mma_step(vf.f[t][ks], pf[nt][ks], st.o[nt][t]);
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kTileThreads) void attn_fwd_kernel(FwdArgs a) {
  using C = FwdCfg<T, D>;
  typedef typename Elem<T>::frag Frag;
  // merge buffer: per wave, the partial of the query N-tile the other wave stores
  __shared__ float mrg_o[2][C::kDTiles * 16][64];
  __shared__ float mrg_ml[2][2][64];

  const Geo g = a.g;
  const int L = xcd_remap(blockIdx.x, a.BH * g.NB);
  const int bh = L / g.NB;
  const int tau = L - bh * g.NB;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, h = lane >> 5;

  const size_t head_off = (size_t)bh * g.N * D;
  const T* __restrict__ Qh = reinterpret_cast<const T*>(a.Q) + head_off;
  const T* __restrict__ Kh = reinterpret_cast<const T*>(a.K) + head_off;
  const int* __restrict__ irow = a.idx + ((size_t)bh * g.NB + tau) * a.kmax;
  int kk = a.kvec[bh];
  kk = kk < 1 ? 1 : (kk > a.kmax ? a.kmax : kk);
  const int tau_base = tile_base(g, tau);

  // queries: N-tile nt holds rows 32nt .. 32nt+31
  Frag qf[2][C::kSteps];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int q = 32 * nt + l32;
    const bool ok = q < g.T;
    load_row_frags<T, D>(qf[nt], Qh + (size_t)(tau_base + (ok ? member_offset(g, q) : 0)) * D, ok, h);
  }
  // this lane's key row inside the wave's half of a block
  const int kr = 32 * w + l32;
  const bool k_ok = kr < g.T;
  const int koff = k_ok ? member_offset(g, kr) : 0;
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
    typedef typename C::PT PT;
    const float c2 = a.c;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh, (size_t)g.N * D * sizeof(T));
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(reinterpret_cast<const PT*>(a.Vt) + (size_t)bh * g.NB * D * 64, (size_t)g.NB * D * 64 * sizeof(PT));
    const int kvoff = (koff * D + 8 * h) * (int)sizeof(T);
    const int vvoff = (l32 * 64 + 32 * w + 8 * h) * (int)sizeof(PT);
    const int vblk = D * 64 * (int)sizeof(PT);
    // K of the next block is fetched one block ahead (ping-pong k0/k1); V of the
    // current block is fetched at its start and lands during S^T and the softmax.
    KFrags<T, D> k0, k1;
    VFrags<T, D> vf;
    int j = irow[0];
    bool v0 = (unsigned)j < (unsigned)g.NB;
    if (v0) load_k<T, D>(k0, rk, kvoff, tile_base(g, j) * D * (int)sizeof(T));
    for (int slot = 0; slot < kk; slot += 2) {
      bool v1 = false;
      int j1 = 0;
      if (slot + 1 < kk) {
        j1 = irow[slot + 1];
        v1 = (unsigned)j1 < (unsigned)g.NB;
        if (v1) load_k<T, D>(k1, rk, kvoff, tile_base(g, j1) * D * (int)sizeof(T));
      }
      if (v0) {
        load_v<T, D>(vf, rv, vvoff, j * vblk);
        attend_block<T, D>(st, k0, vf, qf, c2, kvalid, h);
      }
      if (slot + 1 >= kk) break;
      v0 = false;
      if (slot + 2 < kk) {
        j = irow[slot + 2];
        v0 = (unsigned)j < (unsigned)g.NB;
        if (v0) load_k<T, D>(k0, rk, kvoff, tile_base(g, j) * D * (int)sizeof(T));
      }
      if (v1) {
        load_v<T, D>(vf, rv, vvoff, j1 * vblk);
        attend_block<T, D>(st, k1, vf, qf, c2, kvalid, h);
      }
    }
  }

  // ---- merge the two key halves: wave w stores N-tile w, hands N-tile 1-w over
  const int give = 1 - w;
#pragma unroll
  for (int t = 0; t < C::kDTiles; ++t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) mrg_o[w][t * 16 + i][lane] = st.o[give][t][i];
  }
  mrg_ml[w][0][lane] = st.m[give];
  mrg_ml[w][1][lane] = st.l[give];
  __syncthreads();
  const int other = 1 - w;
  const float ma = st.m[w], mb = mrg_ml[other][0][lane];
  const float la = st.l[w] + xor32(st.l[w]);
  const float lb0 = mrg_ml[other][1][lane];
  const float lb = lb0 + __shfl_xor(lb0, 32, 64);
  const float mt = fmaxf(ma, mb);
  const float wa = (ma == -INFINITY) ? 0.f : fast_exp2(ma - mt);
  const float wb = (mb == -INFINITY) ? 0.f : fast_exp2(mb - mt);
  const float l_tot = wa * la + wb * lb;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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
          v[i] = (wa * st.o[w][t][r] + wb * mrg_o[other][t * 16 + r][lane]) * inv;
        }
        store4(a.O, orow + 32 * t + 8 * gq + 4 * h, a.out_f32, v[0], v[1], v[2], v[3]);
      }
    }
    if (h == 0) a.LSE[(size_t)bh * g.N + q_tok] = l_tot > 0.f ? (mt + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((vt_prep_kernel<T, D>), dim3(a.BH * a.g.NB), dim3(256), 0, s, a);
  hipLaunchKernelGGL((attn_fwd_kernel<T, D>), dim3(a.BH * a.g.NB), dim3(kTileThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

size_t attn_fwd_workspace_bytes(int BH, int NB, int d, int io_f32) {
  return (size_t)BH * NB * d * 64 * (io_f32 ? 4 : 2);
}

hipError_t launch_attn_fwd(const FwdArgs& a, int io_f32, int d, hipStream_t s) {
  if (io_f32) return d == 64 ? launch_fwd<float, 64>(a, s) : launch_fwd<float, 128>(a, s);
  return d == 64 ? launch_fwd<bf16, 64>(a, s) : launch_fwd<bf16, 128>(a, s);
}

}  // namespace dsa
