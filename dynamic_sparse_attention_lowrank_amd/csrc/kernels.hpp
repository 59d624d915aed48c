// Launch interfaces between the C-ABI layer (api.hip) and the kernel files.
// Every launcher only enqueues work on the given stream and returns the launch
// status; arguments have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace dsa {

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const int32_t* idx;
  const int32_t* kvec;
  int kmax;
  void* O;
  float* LSE;
  int out_f32;
  float c;      // scale * log2(e)
  void* Vt;     // workspace: per block, V^T in fragment-major order
  uint32_t* vmax;   // workspace [BH][kDoChunks]: partial max |V| (bf16 inputs)
  float2* vscale;   // workspace [BH]: (2^t, 2^-t), the fp16 V copy's power-of-two scale
  Geo g;
  int BH;
  // query-tile pairs (bf16 forward): tiles tau and tau + pair_s, neighbours along
  // one axis of the tile grid (extent pair_e, pair_p2 = ceil(pair_e / 2) pairs per
  // line); npairs pairs per head
  int pair_s, pair_e, pair_p2, npairs;
  int kernel;   // bf16 forward kernel: 0 by size, 1 one-tile, 2 tile-pair
};
size_t attn_fwd_workspace_bytes(int BH, int NB, int d, int io_f32);
// forward kernel a shape runs: 1 one-tile, 2 tile-pair (setting: 0 by size, 1, 2)
int attn_fwd_kernel_for(const Geo& g, int d, int io_f32, int setting);
hipError_t launch_attn_fwd(const FwdArgs& a, int io_f32, int d, hipStream_t s);

struct PredictArgs {
  const void* Q;
  const void* K;
  const void* Wq;
  const void* Wk;
  float* Qbar;
  float* Kbar;
  float* S;
  Geo g;
  int B, H, r;
  float* Pq = nullptr;   // optional: tile means of Q, [B*H][NB][d] fp32
  float* Pk = nullptr;   // optional: tile means of K
};
hipError_t launch_predict(const PredictArgs& a, int io_f32, int d, hipStream_t s);

// Stage-one predictor training: loss and weight gradients from the Gram
// matrices of the pooled Q and K.
struct PGradArgs {
  const float* Pq;      // [B*H][NB][d] tile means (pool_project with Pq/Pk set)
  const float* Pk;
  float* Gq;            // workspace [B*H][d][d]: Pq^T Pq
  float* Gk;            // workspace [B*H][d][d]: Pk^T Pk
  float* M;             // workspace [H][d][d]: Wq Wk^T - I
  float* qpart;         // workspace [B*H][d][r]: per-(b,h) dWq rows (unscaled)
  float* kpart;         // workspace [B*H][d/16][d][r]: per row block dWk parts
  float* lpart;         // workspace [B*H][d/16]: per row block loss parts
  const void* Wq;       // [H][d][r], I/O dtype
  const void* Wk;
  float* loss;          // [B][H]
  float* dWq;           // [H][d][r] fp32
  float* dWk;
  int B, H, NB, r;
};
size_t predictor_grad_workspace_bytes(int BH, int H, int NB, int d);
// points the workspace arrays of `a` (Pq, Pk, Gq, Gk, M, parts) into `workspace`
void predictor_grad_carve(PGradArgs& a, void* workspace, int BH, int H, int NB, int d);
hipError_t launch_predictor_grad(const PGradArgs& a, int io_f32, int d, hipStream_t s);

// 3-D rotary positions of one [B*H][N][d] tensor (X -> Y, Y may be X).
struct RopeArgs {
  const void* X;
  void* Y;
  Geo g;
  int BH, d;
  int t0, y0, x0;       // position offsets per axis
  float log2_base;
  int inverse;          // 1: rotate by minus the angle
};
hipError_t launch_rope3d(const RopeArgs& a, int f32, hipStream_t s);

struct SelectArgs {
  const float* S;
  const int32_t* kvec;
  int kmax;
  int32_t* idx;
  int NB;
  int BH;
};
hipError_t launch_select(const SelectArgs& a, hipStream_t s);

struct FusedSelectArgs {
  const float* Qbar;
  const float* Kbar;
  const int32_t* kvec;
  int kmax;
  int32_t* idx;
  int NB;
  int BH;
  int r;
};
hipError_t launch_fused_select(const FusedSelectArgs& a, hipStream_t s);
// pooled features only (the first half of launch_predict)
hipError_t launch_pool_project(const PredictArgs& a, int io_f32, int d, hipStream_t s);

// per-(b, h) chunks of the magnitude reductions behind the power-of-two scales
// (one wave reduces them)
constexpr int kDoChunks = 64;

// Per-(b, h) power-of-two scale of a bf16 [BH][elems_per_head] tensor (elems_per_head
// a multiple of 8, rows 16-byte aligned): scale[bh] = (2^s, 2^-s) with s such that
// the head's largest magnitude times 2^s lies in [2^14, 2^15) (s in [-63, 63]; 0 for
// an all-zero head).  `partial` holds BH * kDoChunks words.
hipError_t launch_pow2_scale(const void* X, int BH, size_t elems_per_head, uint32_t* partial, float2* scale,
                             hipStream_t s);
// out = fp16(X * scale[bh].x) for a bf16 [BH][elems_per_head] tensor (the exact
// fp16 copy that the power-of-two scale above makes possible)
hipError_t launch_pow2_convert(const void* X, int BH, size_t elems_per_head, const float2* scale, void* out,
                               hipStream_t s);
// out[bh] = bit pattern of max |X| over the head's elems_per_head floats (an order-free
// maximum of the magnitude bits; a NaN anywhere gives a pattern above +inf's)
hipError_t launch_absmax_f32(const float* X, int BH, size_t elems_per_head, uint32_t* partial, uint32_t* out,
                             hipStream_t s);

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const float* O;       // forward output, float32
  const void* dO;
  const float* LSE;
  const int32_t* idx;
  const int32_t* kvec;
  int kmax;
  float scale;
  float c;      // scale * log2(e)
  int out_f32;
  void* dQ;
  void* dK;
  void* dV;
  // workspace views
  float* Dvec;          // [BH, N]
  void* dO16;           // [BH, N, d] fp16 copy of dO * 2^s_bh (bf16 inputs; written by prepare)
  uint32_t* dmax;       // [BH, kDoChunks] partial max |dO| (bf16 magnitude bits; bf16 inputs)
  float2* dscale;       // [BH] (2^s_bh, 2^-s_bh): the fp16 copy's exact power-of-two scale
  uint32_t* vmax;       // [BH, kDoChunks] partial max |V| (bf16 inputs; written by the dK/dV phase)
  float2* vscale;       // [BH] (2^t_bh, 2^-t_bh): scale of V before its fp16 conversion in dK/dV
  // bf16 inputs: the fp16 dS products (see attn_bwd.hip)
  uint32_t* dabs;       // [BH] bits of max |D| (written by prepare)
  uint32_t* dabs_part;  // [BH, kDoChunks] its partial maxima
  float* Du;            // [BH, N] D * 2^u_bh, the scaled D of the dK/dV phase
  float* Lse2;          // [BH, N] LSE * log2(e) (fp32 product), the dK/dV phase's row statistic
  void* q16;            // [BH, N, d] fp16 Q * 2^a_bh (dK/dV phase)
  uint32_t* qmax;       // [BH, kDoChunks]
  float2* qscale;       // [BH] (2^a_bh, 2^-a_bh)
  void* k16;            // [BH, N, d] fp16 K * 2^b_bh (dQ phase)
  uint32_t* kmaxp;      // [BH, kDoChunks]
  float2* kscale;       // [BH] (2^b_bh, 2^-b_bh)
  uint32_t* vmax_q;     // [BH, kDoChunks] partial max |V| of the dQ phase
  float2* vscale_q;     // [BH] V's scale as the dQ phase computes it (same values as vscale)
  uint32_t* bitmap;     // [BH, NB, words]   bit tau of row j: tile tau kept block j
  int32_t* counts;      // [BH, NB]
  int32_t* offsets;     // [BH, NB + 1]
  int32_t* entries;     // [BH, NB * kmax]
  int32_t* order;       // [BH, NB] key blocks by descending list length (the dK/dV
                        // work-groups' order), or null: ascending block order
  int words;            // ceil(NB / 32)
  Geo g;
  int BH;
};
// longest head (in key blocks) whose dK/dV work-groups take the blocks in
// descending order of list length; longer heads keep ascending order
constexpr int kOrderMaxNB = 16383;
// backward phases: prepare (D + reverse index into the workspace), then dK/dV and
// dQ, which only read the workspace and may run in either order or concurrently
hipError_t launch_bwd_prepare(const BwdArgs& a, int io_f32, int d, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int io_f32, int d, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, int io_f32, int d, hipStream_t s);

}  // namespace dsa
