/*
 * dsa.h -- C ABI of libdsa: DSV-style dynamic block-sparse attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the one described on the DSV page (DSV: Exploiting Dynamic
 * Sparsity to Accelerate Large-Scale Video DiT Training,
 * gist.science/ar/paper/2502.07590): a cheap low-rank predictor guesses which
 * small part of the attention matters (section 3a), neighbouring tokens are
 * grouped so that one 3-D tile of queries shares one selection (section 3b), and
 * exact attention is then computed only over what was selected (section 4,
 * stage two), forward and backward.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Geometry.  A head holds N = Lt*Lh*Lw video tokens stored row-major over the
 *   latent grid (t, y, x): token n = (t*Lh + y)*Lw + x.  A tile is a tt x th x tw
 *   sub-box (tt | Lt, th | Lh, tw | Lw); tiles are numbered row-major over the
 *   tile grid, NB = (Lt/tt)(Lh/th)(Lw/tw), T = tt*th*tw tokens per tile.  Query
 *   tile tau and key block tau are the same tokens ("own block").  Within a tile,
 *   tokens are taken in ascending n.
 * Tensors.  Q, K, V, O, dO, dQ, dK, dV are dense [B, H, N, d] arrays, d
 *   innermost, in device memory.  d is 64 or 128.  Their element type is
 *   shape->io (DSA_BF16 or DSA_F32) unless an argument says otherwise.
 * Empty input.  B*H == 0 is valid: the call returns DSA_OK and enqueues nothing.
 * Limits.  N*d*esize and NB*d*64*esize below 2^31 bytes (esize = 2 for bf16, 4 for
 *   fp32), B*H <= 65535, and B*H*NB*512 <= 2^32-1 (the work-items of the largest
 *   launch grid) (DSA_ERR_SHAPE).
 * Ownership.  The caller owns every buffer and the stream.  The library never
 *   allocates memory and never synchronises the device; each call only enqueues
 *   kernels on `stream` and returns.  It keeps two pieces of state: the
 *   process-wide choice of forward kernel (dsa_set_fwd_kernel, default: by size),
 *   and the workspace of dsa_attn_fwd_noalloc, a fixed array in device memory that
 *   the library's code object holds on each GPU it runs on.
 * Errors.  All argument checks happen on the host before any HIP call; a failed
 *   check returns its status and enqueues nothing.  A failed kernel launch
 *   returns DSA_ERR_HIP.  Device-side values (k[], idx[]) cannot be checked by
 *   the host without a synchronisation, so the kernels treat them defensively
 *   (documented per entry point) and never access memory out of bounds.
 * Determinism.  For identical inputs (and the same forward-kernel choice) every
 *   entry point produces bit-identical outputs (no floating-point atomics).
 * Concurrency.  Calls on different streams may overlap only if their output
 *   buffers (and workspaces) are disjoint.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__)
#define DSA_API __attribute__((visibility("default")))
#else
#define DSA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,            /* a required pointer is NULL                        */
  DSA_ERR_SHAPE = 2,           /* B, H, N or d out of range / unsupported          */
  DSA_ERR_TILE = 3,            /* tile extents do not divide the latent, or T > 64 */
  DSA_ERR_K = 4,               /* kmax out of range                                */
  DSA_ERR_DTYPE = 5,           /* unknown element type                             */
  DSA_ERR_WORKSPACE = 6,       /* workspace too small or misaligned                */
  DSA_ERR_HIP = 7,             /* a HIP launch failed                              */
  DSA_ERR_NOT_IMPLEMENTED = 8, /* combination the library does not support         */
  DSA_ERR_RANK = 9,            /* predictor rank r out of range                    */
  DSA_ERR_SCRATCH = 10,        /* one head needs more than dsa_attn_fwd_noalloc's
                                  fixed device scratch                             */
  DSA_ERR_ARG = 11             /* an enumerated argument is out of range           */
} dsa_status;

typedef enum { DSA_F32 = 0, DSA_BF16 = 1 } dsa_dtype;

typedef struct {
  int32_t B, H, d;        /* batch, heads, head dimension (64 or 128)                 */
  int32_t Lt, Lh, Lw;     /* latent extents; N = Lt*Lh*Lw                             */
  int32_t tt, th, tw;     /* tile extents; must divide the latent; T = tt*th*tw <= 64 */
  int32_t io;             /* dsa_dtype of Q, K, V, Wq, Wk, O (bwd input), dO          */
} dsa_shape;

/* Human-readable name of a status code (static storage, never NULL). */
DSA_API const char* dsa_status_string(dsa_status s);

/* Library ABI version (major*100 + minor): 200. */
DSA_API int32_t dsa_version(void);

/*
 * dsa_predict -- low-rank predictor (DSV page, section 3a).
 *   For every (b, h) and tile tau:
 *     Qbar[b,h,tau,:] = (1/T) sum_{n in tile tau} Q[b,h,n,:] @ Wq[h]      (r values)
 *     Kbar[b,h,tau,:] = (1/T) sum_{n in tile tau} K[b,h,n,:] @ Wk[h]
 *     S[b,h,tau,j]    = Qbar[b,h,tau,:] . Kbar[b,h,j,:]                  (unscaled)
 *   Q, K: [B,H,N,d] io dtype.  Wq, Wk: [H,d,r] io dtype (per-head weights).
 *   Qbar, Kbar: outputs [B,H,NB,r] float32.  S: output [B,H,NB,NB] float32.
 *   All arithmetic is float32 (products of the stored values, float32 sums).
 *   r must lie in [1, 64] (DSA_ERR_RANK otherwise).
 */
DSA_API dsa_status dsa_predict(const dsa_shape* shape, int32_t r, const void* Q, const void* K,
                       const void* Wq, const void* Wk, float* Qbar, float* Kbar, float* S,
                       hipStream_t stream);

/*
 * dsa_select -- top-k key blocks per query tile (DSV page, sections 3a-3b).
 *   For row (b,h,tau) with k = k[b*H+h]: keep block tau itself plus the k-1 other
 *   blocks with the largest S[b,h,tau,j]; equal scores go to the lower index
 *   (+0 and -0 are equal; NaN ranks below every number).  The kept blocks are
 *   written to idx[b,h,tau,0..k-1] in ascending order and idx[b,h,tau,k..kmax-1]
 *   is set to -1.
 *   S: [B,H,NB,NB] float32.  k: device int32 [B*H].  idx: output [B,H,NB,kmax] int32.
 *   1 <= kmax <= NB is required (DSA_ERR_K).  A device value k outside
 *   [1, kmax] is clamped into that range.
 *   Cost: one wave per row; a row's keys are held in registers up to NB = 8192,
 *   in LDS up to NB = 16384, and re-read on each of the search's 33 passes above
 *   that (correct at any NB, but slow for very long rows).
 */
DSA_API dsa_status dsa_select(const dsa_shape* shape, const float* S, const int32_t* k, int32_t kmax,
                      int32_t* idx, hipStream_t stream);

/*
 * dsa_predict_select -- dsa_predict followed by dsa_select without the score
 *   matrix (the next step after the predictor and the selector: the selector
 *   computes each row's scores on the fly and keeps only the top k).
 *   Arguments mean what they mean for dsa_predict and dsa_select; Qbar and Kbar
 *   are written as by dsa_predict, idx as by dsa_select, and no [B,H,NB,NB]
 *   array is read or written.  The scores are the same float32 operations in the
 *   same order as dsa_predict's, so idx is identical to dsa_predict + dsa_select.
 *   Errors: those of dsa_predict (without S) and of dsa_select.
 */
DSA_API dsa_status dsa_predict_select(const dsa_shape* shape, int32_t r, const void* Q, const void* K,
                                      const void* Wq, const void* Wk, const int32_t* k, int32_t kmax,
                                      float* Qbar, float* Kbar, int32_t* idx, hipStream_t stream);

/*
 * dsa_predictor_grad_workspace_bytes -- device workspace that dsa_predictor_grad
 * needs (0 on invalid arguments), in float32 values: tile means 2*B*H*NB*d, Gram
 * matrices 2*B*H*d*d, M = Wq Wk^T - I H*d*d, and partial sums B*H*d*64,
 * B*H*(d/16)*d*64 and B*H*(d/16); each of the eight arrays is rounded up to 256
 * bytes.
 */
DSA_API size_t dsa_predictor_grad_workspace_bytes(const dsa_shape* shape);

/*
 * dsa_predictor_grad -- training signal of the predictor (DSV page, section 4:
 *   in stage one the predictor is trained alongside the model; the page gives
 *   no loss, so this library reads it as follows).  The predictor's score
 *   S[tau,j] (as defined by dsa_predict) estimates the pooled attention logit
 *     T[b,h,tau,j] = mean over i in tile tau, n in block j of Q[b,h,i,:] . K[b,h,n,:],
 *   and the loss of (b, h) is
 *     loss[b,h] = (1/NB^2) sum_{tau,j} (S[b,h,tau,j] - T[b,h,tau,j])^2.
 *   dWq[h] and dWk[h] are the gradients of sum_b loss[b,h] with respect to Wq[h]
 *   and Wk[h] (Q and K receive none).
 *   Q, K: [B,H,N,d] io dtype.  Wq, Wk: [H,d,r] io dtype.  loss: output [B,H]
 *   float32.  dWq, dWk: outputs [H,d,r] float32 (overwritten, not accumulated).
 *   Evaluated as loss = trace(M^T A M C)/NB^2 with M = Wq Wk^T - I and A, C the
 *   d x d Gram matrices of the tile means of Q and K: no NB x NB array is formed.
 *   All arithmetic is float32.  r must lie in [1, 64] (DSA_ERR_RANK).
 *   workspace: device memory of at least dsa_predictor_grad_workspace_bytes(shape)
 *   bytes, 256-byte aligned (DSA_ERR_WORKSPACE).
 */
DSA_API dsa_status dsa_predictor_grad(const dsa_shape* shape, int32_t r, const void* Q, const void* K,
                                      const void* Wq, const void* Wk, float* loss, float* dWq, float* dWk,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dsa_rope3d -- 3-D rotary positions (second page, gist.science/ar/paper/2603.06664,
 *   section 2: a frame's time position is its chunk's start index plus its index in
 *   the chunk, a global time index; the page gives no formula, so this library
 *   reads it as rotary encoding per axis).
 *   The d/2 adjacent pairs (X[n,2p], X[n,2p+1]) of every token row are cut into a
 *   time, a height and a width section of mt, mh, mw pairs (mh = mw = (d/2)/3,
 *   mt = d/2 - 2*mh: 22/21/21 at d = 128, 12/10/10 at d = 64).  Pair i of a section
 *   of m pairs is rotated by
 *     angle = (c + c0) * base^(-i/m),   c = the token's latent coordinate on that
 *     axis (t, y or x), c0 = t0, y0 or x0,
 *   that is Y = (u cos a - v sin a, u sin a + v cos a) for (u, v) = the pair;
 *   inverse = 1 rotates by -angle (maps gradients of rotated tensors back).
 *   X, Y: [B,H,N,d] arrays of element type `dtype` (DSA_BF16 or DSA_F32, any io);
 *   Y may equal X (in place).  Arithmetic is fp32 (sincosf), one rounding to the
 *   output type (round to nearest even for bf16).  Apply it to Q and K before
 *   dsa_predict / dsa_predict_select / dsa_attn_fwd, and with inverse = 1 to the
 *   dQ and dK of dsa_attn_bwd.
 *   Errors: base must be finite and > 1, |t0|, |y0|, |x0| <= 2^30, inverse 0 or 1,
 *   X and Y aligned to one pair (4 bytes bf16, 8 bytes fp32): DSA_ERR_SHAPE.
 */
DSA_API dsa_status dsa_rope3d(const dsa_shape* shape, int32_t dtype, float base, int32_t t0, int32_t y0, int32_t x0,
                              int32_t inverse, const void* X, void* Y, hipStream_t stream);

/*
 * dsa_attn_fwd_workspace_bytes -- device workspace that dsa_attn_fwd needs for
 * this shape (0 on invalid arguments): B*H*NB*d*64 elements of 2 bytes (bf16 io)
 * or 4 bytes (fp32 io), and for bf16 io two more 256-byte-aligned sections of
 * B*H*64 words and B*H float pairs.  dsa_attn_fwd first rewrites every key
 * block's V there, transposed (fp16 for bf16 io), in the order its matrix-core
 * fragments are loaded, after finding V's power-of-two scale per (b, h) (the two
 * small sections).
 */
DSA_API size_t dsa_attn_fwd_workspace_bytes(const dsa_shape* shape);

/*
 * dsa_attn_fwd -- exact softmax attention over the kept blocks (DSV page,
 * section 4, stage two).
 *   For each query token i of tile tau, over the keys n of the blocks
 *   idx[b,h,tau,0..k-1]:  s_in = scale * (q_i . k_n),
 *   O_i = sum_n softmax_n(s_in) v_n,  LSE_i = ln sum_n exp(s_in).
 *   Q, K, V: [B,H,N,d] io dtype.  idx: [B,H,NB,kmax] int32, k: device int32 [B*H].
 *   out_dtype: element type of O (DSA_BF16 or DSA_F32, any io).  O: [B,H,N,d].
 *   LSE: [B,H,N] float32 (natural log).  scale must be finite and > 0 (normally
 *   1/sqrt(d)); otherwise DSA_ERR_SHAPE.
 *   workspace: device memory of at least dsa_attn_fwd_workspace_bytes(shape)
 *   bytes, 256-byte aligned; contents on entry do not matter (DSA_ERR_WORKSPACE).
 *   Softmax statistics and accumulation are float32.  With bf16 io the P.V
 *   product runs on fp16 matrix cores: V is multiplied by 2^t, one power of two
 *   per (b, h) that puts the head's largest |v| in [2^14, 2^15) (t in [-63, 63]),
 *   and converted to fp16, which is exact for every element within a factor 2^31
 *   of that maximum whatever the size of V; O is multiplied back by 2^-t in fp32
 *   (exact).  The probabilities are rounded to fp16 (2^-12 relative).
 *   Device-side robustness: k is clamped to [1, kmax]; idx entries outside
 *   [0, NB) are skipped; a row with no valid block gets O = 0, LSE = -inf.
 *   Duplicate entries are the caller's responsibility (dsa_select never makes them).
 */
DSA_API dsa_status dsa_attn_fwd(const dsa_shape* shape, const void* Q, const void* K, const void* V,
                                const int32_t* idx, const int32_t* k, int32_t kmax, float scale,
                                int32_t out_dtype, void* O, float* LSE, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * dsa_set_fwd_kernel / dsa_get_fwd_kernel -- which kernel the bf16 forward
 *   (dsa_attn_fwd, dsa_attn_fwd_noalloc) runs.  Both compute the same function
 *   (the DSV page, section 4, stage two) to the same precision, in different
 *   orders of summation, so O and LSE may differ in the last bits between them:
 *     DSA_FWD_ONE_TILE:  one work-group per query tile, its kept blocks gathered
 *                        for it alone;
 *     DSA_FWD_TILE_PAIR: one work-group per two neighbouring query tiles, walking
 *                        the union of their kept blocks, so that a block both kept
 *                        is gathered once;
 *     DSA_FWD_AUTO (the default): the tile-pair kernel when one head's gathered
 *                        blocks (NB * 64 * d * 4 bytes) reach 48 MiB, where the
 *                        gathers run at L2-miss bandwidth, else the one-tile kernel.
 *   fp32 io always runs its one kernel.  The setting is process-wide, read at each
 *   forward call; an unknown kind returns DSA_ERR_ARG and changes nothing.
 */
typedef enum { DSA_FWD_AUTO = 0, DSA_FWD_ONE_TILE = 1, DSA_FWD_TILE_PAIR = 2 } dsa_fwd_kernel;
DSA_API dsa_status dsa_set_fwd_kernel(int32_t kind);
DSA_API int32_t dsa_get_fwd_kernel(void);
/* The kernel a forward of this shape runs under the current setting:
 * DSA_FWD_ONE_TILE or DSA_FWD_TILE_PAIR; -1 for an invalid shape.  Host only. */
DSA_API int32_t dsa_fwd_kernel_for(const dsa_shape* shape);

/*
 * dsa_attn_fwd_noalloc -- dsa_attn_fwd for callers that cannot allocate device
 *   memory (code under HIP graph capture, tight serving loops, harnesses that
 *   forbid hipMalloc).  Same arguments, semantics, errors and results (bit-
 *   identical O and LSE) as dsa_attn_fwd, without the workspace: its V^T copy and
 *   scale sections live in a fixed device array of 144 MiB (150,994,944 bytes),
 *   one per GPU, held from the first call on that GPU until the process ends.
 *   Heads are processed in groups that fit it (the kernels of one group, then the
 *   next, on `stream`); a shape for which one head's workspace
 *   (dsa_attn_fwd_workspace_bytes with B = H = 1) exceeds the array returns
 *   DSA_ERR_SCRATCH: at d = 128 that is NB > 9,215 key blocks for bf16 io
 *   (589,760 tokens in 64-token tiles) and NB > 4,608 for fp32 io (d = 64:
 *   18,431 and 9,216).  No hipMalloc, hipFree or allocating library routine is
 *   called; the first call on a GPU looks up the array's device address
 *   (hipGetSymbolAddress), which can fail with DSA_ERR_HIP.
 *   Every call on one GPU shares its array: calls that overlap in time on one GPU
 *   (different streams, or other host threads) race and give undefined results.
 *   The array's contents on entry do not matter.
 */
DSA_API dsa_status dsa_attn_fwd_noalloc(const dsa_shape* shape, const void* Q, const void* K, const void* V,
                                        const int32_t* idx, const int32_t* k, int32_t kmax, float scale,
                                        int32_t out_dtype, void* O, float* LSE, hipStream_t stream);

/*
 * dsa_attn_bwd_workspace_bytes -- device workspace that dsa_attn_bwd needs for
 * this shape and kmax (0 on invalid arguments, including NB*kmax > 2^31-1: the
 * reverse index keeps 32-bit offsets per head).  It holds D = rowsum(dO * O);
 * the reverse (key block -> query tiles) index of idx (for every key block, the
 * query tiles whose kept set contains it: the sums over queries of dK and dV in
 * the DSV page's stage two, section 4, run over these lists) with the order in
 * which the dK/dV phase takes each head's key blocks, longest list first (B*H*NB
 * int32); and, for bf16 inputs, what the fp16 products of the backward need:
 * fp16 copies of dO, of Q (dK/dV phase) and of K (dQ phase), B*H*N*d*2 bytes
 * each; the power-of-two scales of dO, V, Q, K and of V again for the dQ phase
 * (for each, B*H*64 partial maxima and B*H float pairs); max |D| per (b, h) with
 * its B*H*64 partial maxima; D times the fp16 dS scale and LSE times log2(e)
 * (B*H*N floats each).
 * Sections are 256-byte aligned.
 */
DSA_API size_t dsa_attn_bwd_workspace_bytes(const dsa_shape* shape, int32_t kmax);

/*
 * dsa_attn_bwd -- gradients of the block-sparse attention with the block mask
 * held fixed (no gradient reaches the predictor).  The DSV page trains the video
 * DiT through its sparse attention in stage two (section 4), so the kept blocks
 * need exact gradients:
 *   D_i = dO_i . O_i,  P from the forward's LSE,  dS_in = P_in (dO_i . v_n - D_i),
 *   dQ_i = scale sum_n dS_in k_n,  dK_n = scale sum_i dS_in q_i,  dV_n = sum_i P_in dO_i.
 *   Q, K, V, dO: [B,H,N,d] io dtype; LSE: [B,H,N] float32 from dsa_attn_fwd.
 *   O: [B,H,N,d] float32 forward output; o_dtype must be DSA_F32 (else
 *   DSA_ERR_DTYPE): O only enters through D, where a rounded O would put one
 *   coherent error into every dS of its row.
 *   idx, k, kmax, scale: as passed to dsa_attn_fwd (scale finite and > 0; NB*kmax
 *   <= 2^31-1, else DSA_ERR_K).
 *   dQ, dK, dV: outputs [B,H,N,d] of out_dtype, fully overwritten.
 *   workspace: device memory of at least dsa_attn_bwd_workspace_bytes(shape, kmax)
 *   bytes, 256-byte aligned; its contents on entry do not matter.
 *   Precision with bf16 inputs: every product runs on fp16 matrix cores.  dO, V,
 *   Q and K are converted to fp16 after multiplying each by a power of two that
 *   puts its largest magnitude (per (b, h), or per 64-row block for the rows a
 *   work-group keeps in registers) in [2^14, 2^15), so the conversions are exact
 *   for every element within a factor 2^31 of that maximum, whatever the size of
 *   the inputs; P in [0,1] is rounded to fp16; dS is rounded to fp16 after a
 *   power of two per (b, h) derived from bounds on |dO . v| and |D| that hold for
 *   every element (no overflow; 2^-12 relative for every value within 2^-29 of
 *   the bound).  All powers of two are taken back out in fp32, exactly, so
 *   scaling dO or V by a power of two scales the gradients exactly.
 *   The same device-side robustness rules as dsa_attn_fwd apply.
 */
DSA_API dsa_status dsa_attn_bwd(const dsa_shape* shape, const void* Q, const void* K, const void* V,
                                const void* O, int32_t o_dtype, const void* dO, const float* LSE,
                                const int32_t* idx, const int32_t* k, int32_t kmax, float scale,
                                int32_t out_dtype, void* dQ, void* dK, void* dV, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * Backward in phases.  dsa_attn_bwd is exactly these three calls in order on one
 * stream; callers may instead issue them separately, e.g. run dsa_attn_bwd_dkdv
 * and dsa_attn_bwd_dq concurrently on two streams once dsa_attn_bwd_prepare has
 * completed (each reads what prepare wrote and writes only workspace sections of
 * its own).  Arguments mean what they mean for dsa_attn_bwd; the workspace must
 * be the one prepared with the same idx, k, kmax, O and dO.
 *
 * dsa_attn_bwd_prepare -- D = rowsum(dO * O) and the reverse index (for every
 *   key block, the ascending list of query tiles that kept it, and each head's
 *   key blocks ordered by descending list length) into the workspace (bf16: also
 *   dO's scale and fp16 copy, and max |D|).
 * dsa_attn_bwd_dkdv    -- dK, dV: one pass per key block over the query tiles
 *   that kept it, the key blocks of a head taken longest list first so that
 *   short lists fill in at the end (bf16: it first writes V's and Q's scales, Q's
 *   fp16 copy, the scaled D and LSE * log2(e) into its sections).
 * dsa_attn_bwd_dq      -- dQ: one pass per query tile over its kept blocks
 *   (bf16: it first writes V's and K's scales and K's fp16 copy into its sections).
 */
DSA_API dsa_status dsa_attn_bwd_prepare(const dsa_shape* shape, const void* O, int32_t o_dtype, const void* dO,
                                        const int32_t* idx, const int32_t* k, int32_t kmax, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);
DSA_API dsa_status dsa_attn_bwd_dkdv(const dsa_shape* shape, const void* Q, const void* K, const void* V,
                                     const void* dO, const float* LSE, int32_t kmax, float scale,
                                     int32_t out_dtype, void* dK, void* dV, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);
DSA_API dsa_status dsa_attn_bwd_dq(const dsa_shape* shape, const void* Q, const void* K, const void* V,
                                   const void* dO, const float* LSE, const int32_t* idx, const int32_t* k,
                                   int32_t kmax, float scale, int32_t out_dtype, void* dQ, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
