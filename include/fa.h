/*
 * fa.h — C ABI of the MI355X (gfx950) attention-forward library libfa.so.
 *
 * The operation (handbook page "算子加速：注意力、编译与融合", section
 * "注意力：从 O(N²) 显存到分块", and the case-study page, section 3.1):
 *
 *     O[b,h,i,:] = sum_j softmax_j( scale * Q[b,h,i,:] . K[b,h,j,:] + M[b,h,i,j] ) V[b,h,j,:]
 *
 * computed tile by tile with a running row max and denominator so the N x N
 * score matrix never reaches device memory.  Non-causal; no dropout; forward
 * only.  The mask M is added after scaling (case-study page, section 2.3) and
 * is either an additive float32 array or a per-batch valid key count.
 *
 * Conventions shared by every entry point:
 *   - Tensors q, k, v, o are contiguous [B, H, N, D] with D fastest
 *     (essay page, sections 2.1 and 5.3, case-study page, section 3.3), in
 *     the element type `dtype`; o has the same type as the inputs.
 *   - All pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates or frees memory and never synchronises; work is queued on
 *     `hip_stream` (a hipStream_t; NULL means the null stream) and the call
 *     returns as soon as it is queued.
 *   - q, k, v, o and workspace must be 16-byte aligned; lse and mask 4-byte.
 *   - Arguments are validated on the host before anything is queued; on an
 *     error nothing is launched and a negative FA_ERR_* code is returned.
 *   - A row whose every key is masked yields O = 0 and lse = -inf.
 *   - Output is bitwise deterministic for identical inputs and launch
 *     configuration (fixed reduction order; the only atomic, in fa_fwd_ws,
 *     counts arrivals and does not order any arithmetic).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define FA_API __attribute__((visibility("default")))
#else
#define FA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype_t;

typedef enum {
  FA_MASK_NONE = 0,
  /* float32 values added to the scaled scores; -inf drops a key.  Element
   * (b,h,i,j) is read at ptr[b*stride_b + h*stride_h + i*stride_q + j*stride_k];
   * a stride of 0 broadcasts that dimension. */
  FA_MASK_ADDITIVE = 1,
  /* int32 len[B] on the device: keys j >= len[b] are dropped for every query
   * of batch entry b (padding of dynamically batched requests, case-study
   * page, section 2.2).  Values outside [0, N] are clamped to it. */
  FA_MASK_KEYLEN = 2
} fa_mask_kind_t;

typedef struct {
  int32_t kind;       /* fa_mask_kind_t */
  const void* ptr;    /* device pointer, see fa_mask_kind_t */
  int64_t stride_b, stride_h, stride_q, stride_k;   /* FA_MASK_ADDITIVE only, in elements */
} fa_mask_t;

enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,       /* B, H, N or D not positive, or the problem is too large */
  FA_ERR_UNSUPPORTED = -3, /* dtype / D / mask combination not built */
  FA_ERR_ALIGN = -4,       /* a pointer is not aligned as required */
  FA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required */
  FA_ERR_ARG = -6,         /* any other invalid argument (scale, mask kind, ...) */
  FA_ERR_HIP = -7          /* the HIP runtime rejected a launch; see fa_last_hip_error */
};

/*
 * Attention forward.
 *   q, k, v  [B,H,N,D] dtype (read)         o   [B,H,N,D] dtype (written)
 *   lse      [B,H,N] float32 or NULL: natural-log log-sum-exp of each row's
 *            scaled, masked scores (essay page, section 2.3: the Triton kernel
 *            also emits the row log-sum-exp), -inf for a fully masked row.
 *   mask     NULL or a descriptor (FA_MASK_NONE is the same as NULL).
 *   scale    multiplies Q.K; must be finite and > 0 (1/sqrt(D) is usual).
 * Supported: dtype F32, F16, BF16; D in {32, 40, 128}; N >= 1 with
 * (N + 256) * D * sizeof(dtype) < 2^32 (one head's rows are addressed with
 * 32-bit offsets; FA_ERR_SHAPE beyond that).
 */
FA_API int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           const fa_mask_t* mask, int B, int H, int N, int D, float scale,
           fa_dtype_t dtype, void* hip_stream);

/*
 * Cross-attention: queries and keys/values of different lengths, as in the
 * CrossAttention layers the case-study page (section 3.1) routes through the
 * fused kernel next to SelfAttention (UNet latents attending to text tokens).
 *   q, o [B,H,Nq,D]; k, v [B,H,Nk,D]; lse [B,H,Nq] or NULL.
 *   Additive mask element (b,h,i,j) for i < Nq, j < Nk (same strides as
 *   fa_fwd); a key-length mask counts keys, clamped to [0, Nk].
 * Everything else as fa_fwd; fa_fwd(.., N, ..) is fa_fwd_cross(.., N, N, ..).
 */
FA_API int fa_fwd_cross(const void* q, const void* k, const void* v, void* o, float* lse,
                        const fa_mask_t* mask, int B, int H, int Nq, int Nk, int D, float scale,
                        fa_dtype_t dtype, void* hip_stream);

/*
 * Attention forward (self- or cross-attention) on strided tensor views, so a
 * projection output laid out [B, N, H, D] needs no transposing copy (the
 * essay page, sections 2.1 and 5.3, and the case-study page, section 3.3,
 * transpose it to [B, H, N, D] before the kernel).  Element (b, h, n, d) of
 * each tensor is at base[b*stride_b + h*stride_h + n*stride_n + d]: D is
 * contiguous, strides are in elements.
 *   q, o: n < Nq;  k, v: n < Nk;  lse [B,H,Nq] contiguous float32 or NULL.
 * Requirements (else FA_ERR_NULL / FA_ERR_ARG / FA_ERR_ALIGN / FA_ERR_SHAPE,
 * nothing launched): stride pointers non-NULL; strides >= 0, stride_n > 0
 * (o: stride_n >= D); every stride times sizeof(dtype) a multiple of 16;
 * (rows + 256) * stride_n * sizeof(dtype) at most 2^32 - 1 for each tensor.
 * Distinct (b, h, n) of o must not overlap.  Everything else as
 * fa_fwd_cross; with contiguous strides the results are bitwise those of
 * fa_fwd_cross.
 */
typedef struct {
  int64_t stride_b, stride_h, stride_n;
} fa_stride_t;

FA_API int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                          const fa_mask_t* mask, int B, int H, int Nq, int Nk, int D,
                          const fa_stride_t* q_strides, const fa_stride_t* k_strides,
                          const fa_stride_t* v_strides, const fa_stride_t* o_strides,
                          float scale, fa_dtype_t dtype, void* hip_stream);

/*
 * fa_fwd with an even split of the key tiles over the compute units, for
 * shapes whose query blocks (256 rows) would leave the last round of
 * workgroups under 90 % full (e.g. B=1, H=24, N=4608: 432 blocks on 256
 * CUs).  One workgroup per CU takes an equal share of the (query block, key
 * tile) pairs; a block whose keys fall in two shares is computed as two
 * online softmaxes over disjoint key ranges whose unnormalised accumulators,
 * running maxima and denominators are combined by the handbook's rescale
 * (section "注意力：从 O(N²) 显存到分块": exp(m_old - m_new) on both the
 * accumulator and the denominator) by whichever part finishes second.  The
 * combination is a fixed function of (first key range, second key range),
 * so results are bitwise deterministic; they differ from fa_fwd's only by
 * rounding (a different summation order over the keys of split blocks).
 *   fa_fwd_workspace_bytes(B,H,N,D,dtype): bytes the split needs on the
 *     CURRENT device (it depends on the CU count), or 0 when the shape does
 *     not take the split: then fa_fwd_ws is fa_fwd and ignores workspace.
 *     The split is taken for dtype F16/BF16, D = 128, no mask (NULL or
 *     FA_MASK_NONE), N a multiple of 64 and above 384, at least one query
 *     block per CU.
 *   workspace: 256-byte aligned device memory of at least that size, all
 *     zero before its first use.  It begins with one arrival counter per
 *     split, and every completed call leaves the counters at zero again, so
 *     a workspace is zero-filled once and reused; the rest is scratch for
 *     partial results.  Calls that share a workspace must be ordered on one
 *     stream (concurrent calls would race on the counters).
 * Everything else as fa_fwd.  Errors: FA_ERR_WORKSPACE if the split is taken
 * and workspace is NULL or too small, FA_ERR_ALIGN if it is misaligned.
 */
FA_API size_t fa_fwd_workspace_bytes(int B, int H, int N, int D, fa_dtype_t dtype);
FA_API int fa_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse,
                     const fa_mask_t* mask, int B, int H, int N, int D, float scale,
                     fa_dtype_t dtype, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * fa_fwd_ws without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split runs on a scratch array the
 * library holds in device memory, 69,477,632 bytes per GPU it runs on, kept
 * until the process ends; it serves up to 256 compute units (one split
 * workgroup per CU): on a device with more CUs a shape that takes the split
 * returns FA_ERR_WORKSPACE (see fa_last_hip_error).  Shapes that do not take
 * the split run fa_fwd.  The call allocates nothing.  Results are bitwise
 * those of fa_fwd_ws.
 *   Every call on one GPU shares that GPU's array: calls that overlap on
 *   one GPU (different streams, or different host threads, without
 *   ordering) race on it and give wrong results.  The first call on a
 *   device looks the array up and queues a clear of its arrival counters on
 *   hip_stream, so it must not be made under graph capture.
 * Arguments as fa_fwd_ws without workspace / workspace_bytes.
 */
FA_API int fa_fwd_ws_static(const void* q, const void* k, const void* v, void* o, float* lse,
                            const fa_mask_t* mask, int B, int H, int N, int D, float scale,
                            fa_dtype_t dtype, void* hip_stream);

/*
 * INT8-QK / FP8-PV variant (handbook page, section "SageAttention").  Steps:
 *   1. kmean[b,h,:] = token mean of K (float32);
 *   2. Q and K - kmean to INT8, one float32 scale per (b, h, 64-token block),
 *      round to nearest even, codes in [-127, 127];
 *   3. V to FP8 e4m3 (OCP e4m3fn) with one float32 scale per (b, h, channel);
 *   4. S = (Q8 . K8) * sq * sk * scale on INT8 matrix cores, exact int32 sums;
 *   5. online softmax over key tiles of fa_int8qk_kv_block() keys, P taken
 *      against the running max and rounded to e4m3 as 448 * P; the
 *      denominator sums the unrounded P;
 *   6. O = (sum of P8 V8 on FP8 matrix cores, float32 accumulate) * sv / (448 l).
 * lse (if requested) is that of the smoothed, quantised scores in step 4: it
 * differs from the unquantised row log-sum-exp by -scale * q . kmean (the
 * per-row constant smoothing removes) plus quantisation error.
 * Same tensor conventions as fa_fwd.  dtype F16 or BF16, D = 128, B*H at
 * most 65535 (FA_ERR_SHAPE beyond: the prepass grids take B*H as a
 * dimension).  Masks
 * act after quantisation (kmean and the scales still run over all N
 * tokens): KEYLEN drops keys beyond the length; ADDITIVE (strides as in
 * fa_fwd) adds its float32 value to the dequantised, scaled score of step 4,
 * before the running max of step 5 (scale, then the mask: case-study page,
 * section 2.3); a row whose keys are all -inf gives O = 0 and lse = -inf.
 *   workspace        device scratch of at least
 *                    fa_fwd_int8qk_workspace_bytes(B,H,N,D) bytes, 256-byte
 *                    aligned; contents on entry are ignored.  On return it
 *                    holds the quantised operands, each region starting at
 *                    the next 256-byte boundary, in this order (Np = N rounded
 *                    up to 64, BH = B*H):
 *                      q8    int8  [BH, Np, D]   (rows >= N are 0)
 *                      k8    int8  [BH, Np, D]
 *                      v8t   e4m3  [BH, D, Np]   row d, position 64g + pi(k)
 *                            holds key 64g + k, pi(k) = 32*((k>>2)&1) +
 *                            16*(k>>5) + 4*((k>>3)&3) + (k&3)
 *                      sq    f32   [BH, Np/64]   Q scale per 64-token block
 *                      sk    f32   [BH, Np/64]   K scale per 64-token block
 *                      sv    f32   [BH, D]       V scale (absmax / 448)
 *                      vmul  f32   [BH, D]       448 / absmax
 *                      kmean f32   [BH, D]
 *                    followed by reduction scratch.  Calls that share a
 *                    workspace must be ordered on one stream.
 */
FA_API size_t fa_fwd_int8qk_workspace_bytes(int B, int H, int N, int D);
FA_API int fa_fwd_int8qk(const void* q, const void* k, const void* v, void* o, float* lse,
                  const fa_mask_t* mask, int B, int H, int N, int D, float scale,
                  fa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                  void* hip_stream);

/*
 * INT8-QK / 16-bit-PV form of the same method: steps 1, 2, 4 and 5 as for
 * fa_fwd_int8qk, then P (<= 1 against the running max) rounded to `dtype`
 * and multiplied with V as given (not quantised) on 16-bit matrix cores with
 * float32 accumulation; O = acc / l, l summing the unrounded P.  More
 * accurate than the FP8 form and slower in P V.  lse as for fa_fwd_int8qk.
 * Same arguments and support as fa_fwd_int8qk; its workspace
 * (fa_fwd_int8qk_pv16_workspace_bytes) has the same regions in the same
 * order except v8t, which holds V^T in `dtype`: [BH, D, Np], row d,
 * position 64g + 32(k >> 5) + pi16(k & 31) holds key 64g + k,
 * pi16(k) = 16*((k>>2)&1) + 4*(k>>3) + (k&3).
 */
FA_API size_t fa_fwd_int8qk_pv16_workspace_bytes(int B, int H, int N, int D);
FA_API int fa_fwd_int8qk_pv16(const void* q, const void* k, const void* v, void* o, float* lse,
                              const fa_mask_t* mask, int B, int H, int N, int D, float scale,
                              fa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                              void* hip_stream);

/*
 * The same method with Q smoothing as well (handbook page, section
 * "SageAttention": Q and K minus their block means).  pv16 = 0 runs the P V
 * of fa_fwd_int8qk (FP8), pv16 = 1 that of fa_fwd_int8qk_pv16 (16-bit).
 * Step 2 quantises Q - qbar_g instead of Q, where qbar_g is the mean of the
 * rows of 64-token block g that exist (rows < N), summed in float64 and
 * rounded once to float32 (the subtraction in float32, rows >= N stay 0);
 * step 4 adds the compensation back to every score:
 *     S = (Q8 . K8) * sq * sk * scale + scale * (qbar_g . (K_j - kmean))
 * the dot product in float64 over the float32 operands, tabulated per
 * (b, h, block, key) and rounded once to float32 (in log2 units, times
 * log2 e) — without quantisation error this is scale * Q . (K - kmean), as
 * without smoothing; with it, only each block's deviation from its mean is
 * quantised, which helps when query blocks share a large common offset.
 * lse as for fa_fwd_int8qk.  Masks: NONE or KEYLEN (ADDITIVE gives
 * FA_ERR_UNSUPPORTED); FA_ERR_ARG for pv16 outside {0, 1}; FA_ERR_SHAPE
 * also when one head's table reaches 2^31 bytes (N above 185,344);
 * otherwise the arguments and errors of fa_fwd_int8qk.
 *   workspace  at least fa_fwd_int8qk_smooth_workspace_bytes(B,H,N,D,pv16)
 *              bytes, 256-byte aligned: the regions of the chosen form's
 *              workspace, then
 *                qbar  f32  [BH, Np/64, D]   block means of Q
 *                comp  f32  [BH, Np/64, Np]  scale * log2(e) * qbar . (K - kmean)
 *              (B*H*N*N/16 bytes for the table: 14.5 GB at B=1, H=40,
 *              N=76112).  fa_fwd_int8qk_smooth_workspace_bytes returns 0 for
 *              non-positive sizes or pv16 outside {0, 1}.
 */
FA_API size_t fa_fwd_int8qk_smooth_workspace_bytes(int B, int H, int N, int D, int pv16);
FA_API int fa_fwd_int8qk_smooth(const void* q, const void* k, const void* v, void* o, float* lse,
                                const fa_mask_t* mask, int B, int H, int N, int D, float scale,
                                fa_dtype_t dtype, int pv16, void* workspace, size_t workspace_bytes,
                                void* hip_stream);

/*
 * Merge two attention results computed for the same queries over disjoint
 * key sets (K/V split along the sequence, as in ring attention: essay page,
 * section 6.2):
 *     lse = log(e^lse_a + e^lse_b),  O = O_a e^(lse_a - lse) + O_b e^(lse_b - lse)
 * in fp32, rounded to dtype.  A row empty on both sides (lse -inf) gives
 * O = 0, lse = -inf.
 *   o_a, o_b, o  [B,H,N,D] dtype;  lse_a, lse_b [B,H,N] float32 (as written
 *   by fa_fwd / fa_fwd_cross);  lse [B,H,N] float32 or NULL.
 * o may be o_a and lse may be lse_a (in-place accumulation); other overlaps
 * are not allowed.  D * sizeof(dtype) must be a multiple of 16 and at most
 * 1024 bytes.
 */
FA_API int fa_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                    void* o, float* lse, int B, int H, int N, int D, fa_dtype_t dtype,
                    void* hip_stream);

/*
 * Measurement aid, not part of the attention path: an MFMA-only throughput
 * probe giving the dense matrix-core rate the part sustains (the published
 * peaks assume the 2.4 GHz peak engine clock).  Launches `workgroups`
 * workgroups of 4 waves; every wave issues 4 x iters independent MFMAs of
 * one shape on hashed, finite operands and writes one float to
 * out[4 * workgroup + wave] (out: 4 * workgroups floats, device memory).
 *   kind 0: v_mfma_f32_32x32x16_bf16   (32768 flop each)
 *   kind 1: v_mfma_f32_32x32x64_f8f6f4 (e4m3, 131072 flop each)
 *   kind 2: v_mfma_i32_32x32x32_i8     (65536 op each)
 * Total work = workgroups * 16 * iters * (flop each); time it with events on
 * hip_stream.  Errors: FA_ERR_NULL, FA_ERR_SHAPE (workgroups or iters <= 0),
 * FA_ERR_ALIGN, FA_ERR_ARG (kind).
 */
FA_API int fa_mfma_probe(int kind, int workgroups, int iters, float* out, void* hip_stream);

/*
 * Measurement aid, not part of the attention path: the narrowing
 * conversions the kernels use, applied to n caller-given floats (n a
 * multiple of 4), so their rounding can be checked bit by bit.
 *   kind 0: float -> OCP e4m3fn byte (the quantised kernels' conversion of
 *           448 P and of V; round to nearest even), out: n bytes;
 *   kind 1: float -> bf16 (P and O in bf16 paths), out: n uint16;
 *   kind 2: float -> fp16, out: n uint16.
 * in: 16-byte aligned device floats; out: 8-byte aligned device memory.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE (n <= 0 or not a multiple of 4),
 * FA_ERR_ALIGN, FA_ERR_ARG (kind).
 */
FA_API int fa_cvt_probe(int kind, const float* in, void* out, int64_t n, void* hip_stream);

/* Keys per tile of the quantised variant's online softmax (P is rounded
 * against the running max, so the result depends on this tile size). */
FA_API int fa_int8qk_kv_block(void);

/* Static text for a status code. */
FA_API const char* fa_status_string(int status);

/* Text of the last HIP error seen by this thread (empty if none). */
FA_API const char* fa_last_hip_error(void);

/* ABI version: bumped whenever a signature or convention above changes. */
FA_API int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
