/*
 * qlora.h - C ABI of the MI355X (gfx950) QLoRA frozen-base linear layer.
 *
 * The layer keeps a frozen weight W [N, K] in 4-bit NormalFloat (NF4) with
 * double quantization, and adds a trainable low-rank bf16 adapter (A [K, r],
 * B [r, N]) on top of it.  Sources (page titles and the part of each page):
 *   - "QLoRA 原理精讲" (1.2.3), section 2.1: NF4 codebook from N(0,1) quantiles,
 *     per-block absmax (64 weights) and nearest-codeword lookup;
 *     section 2.2 and its storage figure: the fp32 block constants are
 *     quantized again to FP8, 256 per fp32 super-scale; storage is the 4-bit
 *     codes + FP8 constants + fp32 super-scales; dequantization runs in
 *     reverse order (super-scale, then constant, then weight).
 *   - "从LoRA到QLoRA：量化技术如何改变预训练模型的微调方式", section 2.3 (NF4 on
 *     [-1, 1]) and section 3.1 (storage type NF4, compute type bf16;
 *     gradients reach the LoRA adapters through the frozen base).
 *   - Volcengine article on LoRA / Q-LoRA / PortLLM, section 3.4: the QLoRA
 *     linear layer (its equation was lost in extraction; the reading used here
 *     is Y = X W'^T + s (X A) B with s = alpha / r).
 *
 * Conventions shared by every entry point
 *   - All tensors are dense row-major DEVICE pointers owned by the caller.  bf16
 *     values are passed as uint16_t bit patterns.  Every pointer must be 16-byte
 *     aligned.  The library never allocates or frees device memory and keeps
 *     no per-call state; the only global state is its immutable codebook.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it and the call returns before it completes; a device fault surfaces
 *     at the caller's next synchronisation.
 *   - Every call validates its arguments on the host BEFORE launching anything:
 *     on a status other than QLORA_ERR_DEVICE nothing has been launched and no
 *     output was touched.  QLORA_ERR_DEVICE means the HIP runtime refused a
 *     launch; kernels the same call enqueued before that one may still run, so
 *     its outputs and workspace are then unspecified.  Functions never throw
 *     across the ABI.
 *   - Blocks are 64 consecutive elements of the flattened weight, groups are 256
 *     consecutive blocks (the last group may be partial).  Both are fixed.
 *   - Inputs must be finite; the result for non-finite inputs is unspecified.
 *   - Storage of a quantized W with numel = N*K elements:
 *       codes       uint8 [numel/2]          two 4-bit codes per byte, even element in the high nibble
 *       absmax_fp8  uint8 [numel/64]         FP8 E4M3FN code of each block's absmax (scaled by the group super-scale)
 *       superscale  float [ceil(numel/16384)] one fp32 super-scale per group of 256 blocks
 */
#ifndef QLORA_MI355X_H
#define QLORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum {
    QLORA_OK = 0,
    QLORA_ERR_NULL = 1,       /* a required pointer is NULL                                  */
    QLORA_ERR_SHAPE = 2,      /* a size is out of range (numel % 64, K % 64, T < 1, r, ...)   */
    QLORA_ERR_ALIGN = 3,      /* a pointer is not 16-byte aligned                            */
    QLORA_ERR_VALUE = 4,      /* a scalar argument is not finite                             */
    QLORA_ERR_WORKSPACE = 5,  /* workspace is NULL or smaller than qlora_workspace_bytes()   */
    QLORA_ERR_DEVICE = 6      /* the HIP runtime reported an error (launch, device query)    */
} qlora_status;

#define QLORA_BLOCK 64
#define QLORA_GROUP 256
#define QLORA_MAX_RANK 256

/*
 * nf4_build_codebook - the 16 NF4 codewords, ascending (index = 4-bit code).
 *   Source: "QLoRA 原理精讲" section 2.1 and "从LoRA到QLoRA" section 2.3: N(0,1)
 *   quantiles at evenly spaced probabilities, normalised to [-1, 1].  Reading
 *   of the lost formula: 8 positive codewords Phi^-1(1/2 + j(d-1/2)/8)/z
 *   (j = 1..8), 7 negative ones -Phi^-1(1/2 + j(d-1/2)/7)/z (j = 1..7) and an
 *   exact 0, with d = ((1-1/30) + (1-1/32))/2 and z = Phi^-1(d); computed in
 *   fp64 and rounded once to fp32, so out[0] = -1, out[7] = +0, out[15] = +1.
 *   codebook_out: HOST pointer to 16 floats, written.  Pure host code, no GPU.
 *   Errors: QLORA_ERR_NULL.
 */
int nf4_build_codebook(float codebook_out[16]);

/*
 * nf4_quantize_dq - blockwise NF4 quantization with double quantization.
 *   Source: "QLoRA 原理精讲" sections 2.1-2.2.  Per block of 64: c1 = max|w|,
 *   n = fl32(w / c1), code = nearest codeword (exact ties to the lower code;
 *   an all-zero block gives code 7).  Per group of 256 blocks:
 *   s2 = fl32(max c1 / 448); each c1 becomes the E4M3FN code nearest to
 *   min(fl32(c1 / s2), 448), exact ties to the lower code (s2 = 0 -> codes 0).
 *   w          [numel] bf16 (device), read.
 *   numel      number of elements, > 0, a multiple of 64 and at most 2^43.
 *   codes      [numel/2] uint8 (device), written.
 *   absmax_fp8 [numel/64] uint8 (device), written.
 *   superscale [ceil(numel/16384)] float (device), written.
 *   Errors: NULL, SHAPE, ALIGN, DEVICE.
 */
int nf4_quantize_dq(const uint16_t* w, int64_t numel,
                    uint8_t* codes, uint8_t* absmax_fp8, float* superscale,
                    void* stream);

/*
 * nf4_dequantize_dq - double dequantization back to bf16.
 *   Source: "QLoRA 原理精讲" section 2.2 (reverse order).  For block b of group g:
 *   c1' = fl32(e4m3(absmax_fp8[b]) * superscale[g]);
 *   w'  = RNE_bf16(fl32(q[code] * c1')).
 *   codes, absmax_fp8, superscale: the storage triple (device), read.
 *   numel  > 0, multiple of 64, at most 2^43.   w_out [numel] bf16 (device), written.
 *   Errors: NULL, SHAPE, ALIGN, DEVICE.
 */
int nf4_dequantize_dq(const uint8_t* codes, const uint8_t* absmax_fp8, const float* superscale,
                      int64_t numel, uint16_t* w_out, void* stream);

/*
 * Grouped quantize / dequantize: several tensors in one launch.
 *   Source: as nf4_quantize_dq / nf4_dequantize_dq ("QLoRA 原理精讲" sections
 *   2.1-2.2); grouping changes only how the work is launched (for example all
 *   weights of a transformer layer at once, so that small tensors do not each
 *   pay a launch's ramp and tail).  Every tensor gets exactly the bytes the
 *   single-tensor call would give it.
 *   count    1 .. QLORA_MAX_TENSORS descriptors (HOST array, read during the call).
 *   Per tensor: w [numel] bf16 (read by nf4_quantize_dq_grouped, written by
 *   nf4_dequantize_dq_grouped), numel > 0, a multiple of 64 and at most
 *   2^43, and the
 *   storage triple codes [numel/2], absmax_fp8 [numel/64],
 *   superscale [ceil(numel/16384)] (written by the quantizer, read by the
 *   dequantizer); all device pointers, 16-byte aligned.  The tensors' buffers
 *   must not overlap one another.
 *   Errors: NULL, SHAPE (count, a numel, or more than 2^31 - 1 workgroups in
 *   total), ALIGN, DEVICE; nothing is launched unless every tensor is valid.
 */
#define QLORA_MAX_TENSORS 16
typedef struct nf4_tensor {
    uint16_t* w;
    int64_t numel;
    uint8_t* codes;
    uint8_t* absmax_fp8;
    float* superscale;
} nf4_tensor;
int nf4_quantize_dq_grouped(int count, const nf4_tensor* tensors, void* stream);
int nf4_dequantize_dq_grouped(int count, const nf4_tensor* tensors, void* stream);

/* qlora_linear_bwd_input flags: reuse the forward's s X A; compute the
 * adapter gradients in the dX kernel (see below). */
#define QLORA_BWD_REUSE_FORWARD 1u
#define QLORA_BWD_FUSED_GRADS 2u

/*
 * qlora_workspace_bytes - device workspace (bytes) that qlora_linear_fwd and
 *   qlora_linear_bwd_input need for these sizes (the larger of the two).
 *   Returns 0 for sizes the entry points would reject.  The size is not
 *   monotone in T: 16 < T <= 96 keeps one set of split partials per 16-token
 *   window and can need more than a larger T (for example about 34 MB at
 *   T = 96 against about 26 MB at T = 4096 on an 11008 x 4096 weight with
 *   r = 64), and a mid-size T whose 256 x 256 output tiles are too few to
 *   fill the chip splits the reduction over several workgroups with fp32
 *   partial tiles (at most 64 MiB; 64 MiB for a 4096 x 4096 weight at
 *   T = 512), so a caller that sizes one workspace for a range of T takes the
 *   maximum over that range (qlora_workspace_bytes_upto).
 */
size_t qlora_workspace_bytes(int64_t T, int64_t K, int64_t N, int64_t r);

/*
 * qlora_workspace_bytes_upto - the largest qlora_workspace_bytes(T, K, N, r)
 *   over 1 <= T <= T_max: one workspace of this size serves every call with
 *   up to T_max tokens.  Returns 0 for sizes the entry points would reject.
 */
size_t qlora_workspace_bytes_upto(int64_t T_max, int64_t K, int64_t N, int64_t r);

/*
 * qlora_workspace_bytes_bwd - device workspace (bytes) that a
 *   qlora_linear_bwd_input call with these flags needs when it computes the
 *   adapter gradients (at least the forward's part, so the forward can use the
 *   same workspace).  With QLORA_BWD_FUSED_GRADS this holds fp32 gradient
 *   partials for every 256-token tile and can exceed qlora_workspace_bytes.
 *   Returns 0 for sizes the entry points would reject or an unknown flag.
 */
size_t qlora_workspace_bytes_bwd(int64_t T, int64_t K, int64_t N, int64_t r, unsigned flags);

/*
 * qlora_linear_fwd - fused forward of one QLoRA linear layer.
 *   Source: Volcengine article section 3.4 (equation lost; reading above) and
 *   "从LoRA到QLoRA" section 3.1 (dequantize to bf16 on the fly).
 *     Y = X W'^T + scaling * (X A) B,   fp32 accumulation, bf16 output.
 *   W' is the double-dequantized bf16 weight (same values nf4_dequantize_dq
 *   writes); it is never materialised in HBM.
 *   x [T, K] bf16; codes/absmax_fp8/superscale: W [N, K] quantized as above;
 *   lora_a [K, r] bf16, lora_b [r, N] bf16 (both NULL iff r == 0);
 *   y [T, N] bf16, written.  T >= 1, K and N multiples of 64, r = 0 or a
 *   multiple of 8 up to 256.  Size limits (32-bit operand addressing):
 *   K, N <= 2^20, T <= 2^22, T*K <= 2^30, T*N <= 2^30, N*K < 2^32.
 *   workspace: device scratch of at least qlora_workspace_bytes(T, K, N, r)
 *   bytes (may be NULL if that is 0); its contents on entry do not matter.
 *   Kernels by size: T <= 16 runs the decode kernels (small-M MFMA, weight
 *   stream read once); 16 < T <= 96 runs them on 16-token windows as one
 *   grouped launch; larger T runs the 256 x 256-tile MFMA GEMM, whose
 *   reduction over K is split over up to 16 workgroups per tile (fp32
 *   partials in the workspace, added in split order by one more launch) when
 *   the tiles alone are too few for the chip.  Results are deterministic.
 *   Errors: NULL, SHAPE, ALIGN, VALUE (non-finite scaling), WORKSPACE, DEVICE.
 */
int qlora_linear_fwd(const uint16_t* x, int64_t T, int64_t K, int64_t N,
                     const uint8_t* codes, const uint8_t* absmax_fp8, const float* superscale,
                     const uint16_t* lora_a, const uint16_t* lora_b, int64_t r, float scaling,
                     uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * qlora_linear_bwd_input - backward of the layer through the frozen base.
 *   Source: "从LoRA到QLoRA" sections 1.3 and 3.1 (gradients flow through the
 *   frozen 4-bit base into the adapters; only the adapters get weight
 *   gradients); "QLoRA 原理精讲" section 3 (adapters stay bf16).
 *     dX = dY W' + scaling * (dY B^T) A^T
 *     dA = scaling * X^T (dY B^T)        (only if d_lora_a != NULL)
 *     dB = scaling * (X A)^T dY          (only if d_lora_b != NULL)
 *   fp32 accumulation, bf16 outputs.
 *   dy [T, N] bf16; W as in qlora_linear_fwd; dx [T, K] bf16, written;
 *   x [T, K] bf16, required iff d_lora_a or d_lora_b is non-NULL;
 *   d_lora_a [K, r] and d_lora_b [r, N] bf16, written when non-NULL
 *   (must be NULL when r == 0).  Sizes as for qlora_linear_fwd.  The
 *   workspace is needed even when r == 0 (block scales are staged there).
 *   flags: an OR of
 *     QLORA_BWD_REUSE_FORWARD when `workspace` still holds what a
 *       qlora_linear_fwd with the same x, lora_a, scaling and sizes left there
 *       (nothing else used it since): s X A is then taken from it instead of
 *       being recomputed for dB.  Ignored for T <= 96 (the decode-kernel
 *       forward keeps nothing).  With a stale workspace the flag gives wrong
 *       dB.
 *     QLORA_BWD_FUSED_GRADS: dA and dB come from the dX kernel itself, each
 *       of its workgroups adding the gradients of its 256-token tile after
 *       its dX tile (dA over its own k columns, dB over an even share of N),
 *       and one launch sums the tiles' fp32 partials in tile order; the
 *       separate gradient pass over X and dY is gone.  dX is the same bits as
 *       without the flag; dA and dB sum in another order (same tolerance).
 *       The workspace must hold qlora_workspace_bytes_bwd(T, K, N, r, flags)
 *       bytes.  Without d_lora_a and d_lora_b the flag changes nothing.
 *   Errors: NULL, SHAPE, ALIGN, VALUE (non-finite scaling, unknown flag),
 *   WORKSPACE, DEVICE.
 */
int qlora_linear_bwd_input(const uint16_t* dy, int64_t T, int64_t K, int64_t N,
                           const uint8_t* codes, const uint8_t* absmax_fp8, const float* superscale,
                           const uint16_t* lora_a, const uint16_t* lora_b, int64_t r, float scaling,
                           uint16_t* dx, const uint16_t* x,
                           uint16_t* d_lora_a, uint16_t* d_lora_b,
                           void* workspace, size_t workspace_bytes, unsigned flags, void* stream);

/*
 * qlora_merge_lora - the adapted layer's weight, merged back into bf16.
 *   Source: "QLoRA 原理精讲" section 2.5 (after merging, inference runs at the
 *   base model's speed: the adapter merges back into BF16 weights) and
 *   section 3, pitfall 3 (deployment from the merged BF16 weights).  Since
 *   X W'^T + s (X A) B = X (W' + s (A B)^T)^T, the merged weight is
 *     W_m[n][k] = RNE_bf16(W'[n][k] + scaling * sum_j A[k][j] B[j][n]),
 *   with W' the double-dequantized bf16 weight (the values nf4_dequantize_dq
 *   writes), the rank-r sum accumulated in fp32 and added to W' by one fused
 *   multiply-add before the single rounding.
 *   codes/absmax_fp8/superscale: W [N, K] quantized as above (device), read;
 *   lora_a [K, r] bf16 and lora_b [r, N] bf16 (device), read (both NULL iff
 *   r == 0, which writes W' itself); w_out [N, K] bf16 (device), written.
 *   K a multiple of 64, N a multiple of 8, r = 0 or a multiple of 8 up to 256,
 *   K, N <= 2^20, N*K < 2^32.  Needs no workspace.
 *   Errors: NULL, SHAPE, ALIGN, VALUE (non-finite scaling), DEVICE.
 */
int qlora_merge_lora(const uint8_t* codes, const uint8_t* absmax_fp8, const float* superscale,
                     int64_t K, int64_t N, const uint16_t* lora_a, const uint16_t* lora_b, int64_t r,
                     float scaling, uint16_t* w_out, void* stream);

/*
 * Single quantization (no double quantization).
 *   Source: "QLoRA 原理精讲" section 2.2, its engineering motivation: the first
 *   level alone keeps one fp32 scale per 64 weights (32/64 = 0.5 bit of
 *   overhead per weight, against about 0.127 bit with the second level).  The
 *   codes are those of nf4_quantize_dq (same absmax, same nearest-codeword
 *   rule); the block constant is the exact fp32 absmax c1 itself, and
 *   dequantization is w' = RNE_bf16(fl32(q[code] * c1)).  Storage of W with
 *   numel = N*K elements:
 *       codes   uint8 [numel/2]   as above
 *       absmax  float [numel/64]  fp32 absmax of each block
 *   Every _sq entry point takes `absmax` in place of the pair
 *   (absmax_fp8, superscale) and otherwise has the arguments, sizes, workspace
 *   and errors of the entry point it is named after.
 */
int nf4_quantize(const uint16_t* w, int64_t numel, uint8_t* codes, float* absmax, void* stream);
int nf4_dequantize(const uint8_t* codes, const float* absmax, int64_t numel, uint16_t* w_out, void* stream);
int qlora_linear_fwd_sq(const uint16_t* x, int64_t T, int64_t K, int64_t N,
                        const uint8_t* codes, const float* absmax,
                        const uint16_t* lora_a, const uint16_t* lora_b, int64_t r, float scaling,
                        uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);
int qlora_linear_bwd_input_sq(const uint16_t* dy, int64_t T, int64_t K, int64_t N,
                              const uint8_t* codes, const float* absmax,
                              const uint16_t* lora_a, const uint16_t* lora_b, int64_t r, float scaling,
                              uint16_t* dx, const uint16_t* x,
                              uint16_t* d_lora_a, uint16_t* d_lora_b,
                              void* workspace, size_t workspace_bytes, unsigned flags, void* stream);
int qlora_merge_lora_sq(const uint8_t* codes, const float* absmax, int64_t K, int64_t N,
                        const uint16_t* lora_a, const uint16_t* lora_b, int64_t r,
                        float scaling, uint16_t* w_out, void* stream);

/*
 * INT4 absmax quantization: the baseline of the data-type ablation.
 *   Source: "QLoRA 原理精讲" section 2.1 (why not INT4: 16 uniform integer
 *   levels [-8, 7], against NF4's equal-probability levels).  Same blocks,
 *   absmax and storage as nf4_quantize / nf4_dequantize, with the levels
 *   v_i = fl32((i - 8) / 7) in place of the NF4 codewords: code = level
 *   nearest to fl32(w / c1), exact ties to the lower code, all-zero blocks
 *   code 8; w' = RNE_bf16(fl32(v[code] * c1)).  Not used by the layer entry
 *   points; arguments and errors as for nf4_quantize / nf4_dequantize.
 */
int int4_quantize(const uint16_t* w, int64_t numel, uint8_t* codes, float* absmax, void* stream);
int int4_dequantize(const uint8_t* codes, const float* absmax, int64_t numel, uint16_t* w_out, void* stream);

/*
 * fp16 compute type.
 *   Source: "QLoRA 原理精讲" section 3, pitfall 4 (GPUs without bfloat16 switch
 *   the compute dtype to FP16).  Each _f16 entry point has the arguments,
 *   sizes, workspace and errors of the entry point it is named after, with
 *   every 16-bit tensor in IEEE fp16 instead of bf16: the weight given to
 *   nf4_quantize_dq_f16, the dequantized weight, x, y, dy, dx, lora_a,
 *   lora_b and the adapter gradients.  The storage (codes, FP8 constants,
 *   super-scales) is the same as for bf16.  Every rounding to 16 bits (the
 *   dequantized weight w' = RNE_fp16(fl32(q[code] * c1')), the outputs) is
 *   to nearest even in fp16; products accumulate in fp32 on the fp16 MFMA.
 *   The layer's intermediates s X A and s dY B^T travel as fp16 hi + lo pairs.
 */
int nf4_quantize_dq_f16(const uint16_t* w, int64_t numel,
                        uint8_t* codes, uint8_t* absmax_fp8, float* superscale, void* stream);
int nf4_dequantize_dq_f16(const uint8_t* codes, const uint8_t* absmax_fp8, const float* superscale,
                          int64_t numel, uint16_t* w_out, void* stream);
int qlora_linear_fwd_f16(const uint16_t* x, int64_t T, int64_t K, int64_t N,
                         const uint8_t* codes, const uint8_t* absmax_fp8, const float* superscale,
                         const uint16_t* lora_a, const uint16_t* lora_b, int64_t r, float scaling,
                         uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);
int qlora_linear_bwd_input_f16(const uint16_t* dy, int64_t T, int64_t K, int64_t N,
                               const uint8_t* codes, const uint8_t* absmax_fp8, const float* superscale,
                               const uint16_t* lora_a, const uint16_t* lora_b, int64_t r, float scaling,
                               uint16_t* dx, const uint16_t* x,
                               uint16_t* d_lora_a, uint16_t* d_lora_b,
                               void* workspace, size_t workspace_bytes, unsigned flags, void* stream);
int qlora_merge_lora_f16(const uint8_t* codes, const uint8_t* absmax_fp8, const float* superscale,
                         int64_t K, int64_t N, const uint16_t* lora_a, const uint16_t* lora_b, int64_t r,
                         float scaling, uint16_t* w_out, void* stream);

/*
 * Grouped decode forward: several independent layers in one launch.
 *   Source: the layer of qlora_linear_fwd (Volcengine article section 3.4,
 *   read as Y = X W'^T + s (X A) B); grouping changes only how the work is
 *   launched.  At decode sizes one linear streams too few bytes to cover the
 *   memory latency of the device, so the linears that a step can run together
 *   (q/k/v on the same X, gate/up on the same X) go into one launch pair.
 *   Each problem i computes exactly what qlora_linear_fwd computes for it:
 *     problems[i].y = problems[i].x W_i'^T + problems[i].scaling (x A_i) B_i
 *   with the same arithmetic (and so the same bits) as the single call.
 *   count      1 .. QLORA_MAX_GROUP problems (HOST array, read during the call).
 *   T          tokens of every problem, 1 .. QLORA_GROUPED_MAX_T.
 *   r          adapter rank of every problem (0 = no adapter: lora_a and
 *              lora_b NULL), rules as for qlora_linear_fwd.
 *   Per problem: x [T, K] bf16, the storage triple of W [N, K], lora_a [K, r],
 *   lora_b [r, N], y [T, N] bf16 written; K, N and alignment as for
 *   qlora_linear_fwd.  Outputs must not overlap one another or any input.
 *   workspace: at least qlora_grouped_workspace_bytes(count, problems, T, r)
 *   bytes (device); contents on entry do not matter.
 *   Errors: NULL, SHAPE (count, T, r or a problem's sizes), ALIGN, VALUE,
 *   WORKSPACE, DEVICE; nothing is launched unless every problem is valid.
 */
#define QLORA_MAX_GROUP 8
#define QLORA_GROUPED_MAX_T 16
typedef struct qlora_linear_problem {
    const uint16_t* x;            /* [T, K] bf16 (device)                    */
    const uint8_t* codes;         /* W [N, K]: packed codes [N*K/2]          */
    const uint8_t* absmax_fp8;    /* [N*K/64] FP8 E4M3FN block constants     */
    const float* superscale;      /* [ceil(N*K/16384)] fp32 super-scales     */
    const uint16_t* lora_a;       /* [K, r] bf16, or NULL when r == 0        */
    const uint16_t* lora_b;       /* [r, N] bf16, or NULL when r == 0        */
    uint16_t* y;                  /* [T, N] bf16 (device), written           */
    int64_t K, N;
    float scaling;                /* s = alpha / r                           */
} qlora_linear_problem;

/* Workspace bytes for qlora_linear_fwd_grouped (0 if any size is invalid). */
size_t qlora_grouped_workspace_bytes(int count, const qlora_linear_problem* problems, int64_t T, int64_t r);
int qlora_linear_fwd_grouped(int count, const qlora_linear_problem* problems, int64_t T, int64_t r,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * qlora_linear_fwd_grouped_ex - qlora_linear_fwd_grouped with the decode
 *   product chosen by the caller.  The layer and its dequantized weights are
 *   those above ("QLoRA 原理精讲" section 2.2; Volcengine article section 3.4);
 *   the weight stream, blocks and dequantization are the same in both forms,
 *   only the multiply-add of the dequantized bf16 weights with X differs:
 *     QLORA_DECODE_MFMA  matrix cores, X padded to 16 token rows;
 *     QLORA_DECODE_VALU  vector dot products (v_dot2 of two bf16 pairs into
 *                        fp32), no matrix-core instruction; T <= 8;
 *     0                  the library's choice for T (what
 *                        qlora_linear_fwd_grouped and qlora_linear_fwd use).
 *   The two forms sum in different orders, so their outputs may differ in the
 *   last bits; each is deterministic.
 *   Errors: those of qlora_linear_fwd_grouped, and QLORA_ERR_VALUE for any
 *   other flags value or QLORA_DECODE_VALU with T > 8.
 */
#define QLORA_DECODE_MFMA 1u
#define QLORA_DECODE_VALU 2u
int qlora_linear_fwd_grouped_ex(int count, const qlora_linear_problem* problems, int64_t T, int64_t r,
                                unsigned flags, void* workspace, size_t workspace_bytes, void* stream);

/*
 * qlora_linear_fwd_noalloc - qlora_linear_fwd for callers that cannot
 *   allocate device memory (code under HIP graph capture, tight serving
 *   loops, harnesses that forbid hipMalloc): the same computation and kernels
 *   as qlora_linear_fwd, with no workspace argument.  Its scratch is a static
 *   device array of qlora_noalloc_scratch_bytes() (32 MiB) that every GPU the
 *   library runs on holds until the process ends; the call allocates nothing.
 *   The output is bit-identical to qlora_linear_fwd's whenever the latter's
 *   forward workspace fits the scratch.  Where the tile GEMM's split-k
 *   partials (mid-size T) would not fit, the reduction is split over fewer
 *   workgroups (down to one), so the fp32 sums run in another order and the
 *   bf16 results can differ in the last bit.  Sizes whose remaining workspace
 *   still exceeds the scratch are rejected with QLORA_ERR_WORKSPACE before
 *   anything is launched; every T <= 16 decode call of the LLaMA-7B and -65B
 *   linears with r <= 64 fits, and so does every T from 129 to 4096 on the
 *   7B shapes.
 *   All calls on one GPU share its array and each leaves it in an unspecified
 *   state, so calls that may overlap on one GPU (other streams, other host
 *   threads) race and must be serialised by the caller; nothing in the array
 *   needs to start at zero.  The forward's s X A is not kept for a backward
 *   (no QLORA_BWD_REUSE_FORWARD after this call).  The stream must belong to
 *   the current device.  Arguments and errors otherwise as qlora_linear_fwd.
 */
int qlora_linear_fwd_noalloc(const uint16_t* x, int64_t T, int64_t K, int64_t N,
                             const uint8_t* codes, const uint8_t* absmax_fp8, const float* superscale,
                             const uint16_t* lora_a, const uint16_t* lora_b, int64_t r, float scaling,
                             uint16_t* y, void* stream);
size_t qlora_noalloc_scratch_bytes(void);

/* qlora_status_string - static, NUL-terminated description of a status code. */
const char* qlora_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_MI355X_H */
