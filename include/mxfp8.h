/*
 * mxfp8.h -- C ABI of libmxfp8.so, the MXFP8 dense linear layer (and its
 * top-k routed MoE variant) for AMD Instinct MI355X (gfx950).
 *
 * The dense layer, as the pages define it ("[Kernel] Add FlashInfer TRTLLM MXFP8
 * linear backend", vLLM PR #52204, §Purpose and the review of apply_weights):
 *   1. BF16 activations are quantized on the fly to E4M3 elements with one
 *      UE8M0 (power-of-two) scale per 32 elements along K;
 *   2. the MXFP8 weight and its scales are prepared once after loading, with
 *      N physically padded to a multiple of 128 and K a multiple of 256;
 *   3. a block-scaled FP8 GEMM accumulates in fp32; the padded output is cut
 *      back to the logical N, bias is added and the result is BF16.
 * The quantization rule is the OCP Microscaling (MX) v1.0 conversion:
 *   scale = 2^(floor(log2(max |v|)) - 8), elements round-to-nearest-even on
 *   the E4M3 grid, saturated to +-448; an all-zero block gets scale byte 0.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers unless stated; sizes are elements.
 *     E4M3 and UE8M0 data travel as raw bytes (uint8); BF16 as 16-bit words.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work on it: none allocates, none synchronizes, so
 *     every call can be captured into a HIP graph.  The caller owns every
 *     buffer, including workspaces and prepared weights.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     negative mxfp8_status is returned with nothing launched.  A launch
 *     failure reported by the runtime is MXFP8_E_LAUNCH.  Faults inside a
 *     kernel surface at the caller's next synchronization (HIP semantics).
 *   - M == 0 is a valid no-op (returns MXFP8_OK, launches nothing).
 */
#ifndef MXFP8_H_
#define MXFP8_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXFP8_OK = 0,
  MXFP8_E_NULLPTR = -1,   /* a required pointer is NULL */
  MXFP8_E_SHAPE = -2,     /* a size is negative / zero where it must not be, breaks K % 32, K % 256,
                             or exceeds a limit (K <= 2^24 for the packed operands of the GEMM) */
  MXFP8_E_ALIGN = -3,     /* a pointer is not aligned as documented */
  MXFP8_E_LD = -4,        /* a leading dimension is too small or not a documented multiple */
  MXFP8_E_WORKSPACE = -5, /* workspace NULL or smaller than the *_workspace_bytes query */
  MXFP8_E_DEVICE = -6,    /* the current device is not gfx950, or no device */
  MXFP8_E_LAUNCH = -7,    /* the HIP runtime reported an error at launch */
  MXFP8_E_SCRATCH = -8    /* mxfp8_linear_noalloc: the shape needs more than its static scratch */
} mxfp8_status;

/* Static, human readable text for a status code (never NULL). */
const char* mxfp8_status_string(int status);

/*
 * Activation quantization (step 1 of the layer; the on-the-fly quantize of
 * vLLM PR #52204 §Purpose).  For each row m and block b:
 *   q[m, 32b .. 32b+31] = E4M3 elements, s[m, b] = UE8M0 scale byte.
 * x_bf16 [M, K] row-major with row stride ldx (elements);
 * q_e4m3 [M, K] bytes with row stride ldq; s_e8m0 [M, K/32] bytes, stride lds.
 * Requires K % 32 == 0; ldx >= K, ldx % 8 == 0; ldq >= K, ldq % 8 == 0;
 * lds >= K/32; x_bf16 and q_e4m3 16-byte aligned.
 */
int mxfp8_quantize_act(const void* x_bf16, int64_t M, int64_t K, int64_t ldx,
                       void* q_e4m3, int64_t ldq, void* s_e8m0, int64_t lds,
                       void* stream);

/*
 * Sizes in bytes of the prepared (packed) weight for a logical [N, K] MXFP8
 * weight: *w_bytes = N_pad * K, *s_bytes = N_pad * K / 32, where
 * N_pad = ceil(N / 128) * 128.  Host-only; requires N >= 1, K % 256 == 0.
 */
int mxfp8_prepared_weight_bytes(int64_t N, int64_t K, size_t* w_bytes, size_t* s_bytes);

/*
 * One-time weight preparation (step 2; process_weights_after_loading in the
 * vLLM PR #52204 digest, "implementation breakdown": require K % 256 == 0,
 * take the logical [:N, :K/32] scale region, pad N to a multiple of 128,
 * reorder into the GEMM's layout).  Reads the MXFP8 weight as a checkpoint
 * holds it:
 *   w_e4m3   [N, K] bytes, row stride ldw (ldw >= K, ldw % 16 == 0, 16-byte aligned)
 *   w_s_e8m0 [>= N, >= K/32] bytes, row stride ldws (ldws >= K/32), any alignment
 * and writes w_packed (w_bytes) and s_packed (s_bytes), 256-byte aligned, in
 * an opaque order owned by this library.  Pad rows N..N_pad-1 are zero
 * elements with scale byte 127; they never reach the output.
 */
int mxfp8_prepare_weight(const void* w_e4m3, const void* w_s_e8m0, int64_t N, int64_t K,
                         int64_t ldw, int64_t ldws, void* w_packed, void* s_packed,
                         void* stream);

/*
 * Inverse of mxfp8_prepare_weight, for tests and tooling: writes the full
 * padded operand w_e4m3 [N_pad, K] (contiguous) and w_s_e8m0 [N_pad, K/32]
 * (contiguous).  Same size rules as mxfp8_prepare_weight.  Also unpacks the
 * packed activations of mxfp8_quantize_act_packed (pass M as N).
 */
int mxfp8_unpack_weight(const void* w_packed, const void* s_packed, int64_t N, int64_t K,
                        void* w_e4m3, void* w_s_e8m0, void* stream);

/*
 * Workspace bytes mxfp8_linear needs for this shape (host-only).  On the
 * decode kernel (M <= 16, K <= 8192) nothing is stored there (a 256-byte
 * minimum is still required); on the split-K slab kernel (M <= 128) it holds
 * fp32 partial outputs, one [M, N_pad] per K slice; otherwise (the
 * mid-M, medium-tile and large-tile GEMMs) the activations
 * quantized into the packed layout (M padded to 128 rows, plus their scales;
 * for M > 128 also the fp32 split-K partials when the shape has few tiles).
 * Which kernel a shape takes comes from the measured shape table (see
 * mxfp8_debug_force_path).  Its
 * contents need no initialization.  Calls that share one workspace must be ordered on one
 * stream (concurrent calls on one workspace race).
 */
int mxfp8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes);

/*
 * The MXFP8 dense linear layer (steps 1 + 3; apply_weights in vLLM PR
 * #52204):  y[m, n] = bf16( sum_k deq(q(x))[m, k] * deq(W)[n, k] + bias[n] )
 * for m < M, n < N, accumulated in fp32.
 *   x_bf16    [M, K] row stride ldx (ldx >= K, ldx % 8 == 0, 16-byte aligned)
 *   w_packed, s_packed  from mxfp8_prepare_weight for this (N, K)
 *   bias_bf16 [N] or NULL
 *   y_bf16    [M, N] row stride ldy (ldy >= N); columns >= N are not written
 *   workspace >= mxfp8_linear_workspace_bytes(M, N, K), 256-byte aligned
 * Requires K % 256 == 0, N >= 1.  Bias is added to the fp32 accumulator and
 * the sum is rounded to bf16 once.
 */
int mxfp8_linear(const void* x_bf16, int64_t M, int64_t K, int64_t ldx,
                 const void* w_packed, const void* s_packed, int64_t N,
                 const void* bias_bf16, void* y_bf16, int64_t ldy,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same layer for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, results and errors as mxfp8_linear, without the workspace: the
 * same kernels use a static device array of MXFP8_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that each GPU the library runs on holds until the process ends.
 * A shape whose mxfp8_linear_workspace_bytes exceeds it returns
 * MXFP8_E_SCRATCH with nothing launched (every M <= 128 at K <= 8192 fits;
 * larger M fits while its packed activations, and split-K partials, do).
 * The call allocates nothing and never synchronizes.  All calls on one GPU
 * share that GPU's array: calls that overlap on one GPU (several streams or
 * host threads at once) race; order them on one stream.
 */
#define MXFP8_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
int mxfp8_linear_noalloc(const void* x_bf16, int64_t M, int64_t K, int64_t ldx,
                         const void* w_packed, const void* s_packed, int64_t N,
                         const void* bias_bf16, void* y_bf16, int64_t ldy, void* stream);

/*
 * W4A8: MXFP4 weights (E2M1 elements, one UE8M0 scale per 32 along K) times
 * MXFP8 activations -- the "MxE2m1 weights x MxE4m3 activations" mode of
 * flashinfer's W4A8 exposure PR ("Changes": MXFP4 weights with 32-element
 * UE8M0 scales, MXFP8 activation preparation).  Same layer as mxfp8_linear
 * with the weight element format changed; E2M1 is 1 sign, 2 exponent (bias
 * 1), 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 *
 * mxfp8_prepared_weight_fp4_bytes: host-only sizes (N >= 1, K % 256 == 0):
 *   *w_bytes = N_pad * K / 2, *s_bytes = N_pad * K / 32.
 * mxfp8_prepare_weight_fp4: one-time pack.
 *   w_e2m1   [N, K/2] bytes, row stride ldw bytes (ldw >= K/2, ldw % 16 == 0,
 *            16-byte aligned); element 2j of a row in the low nibble of byte
 *            j, element 2j + 1 in the high nibble
 *   w_s_e8m0 [N, >= K/32] row stride ldws (only [:N, :K/32] is read)
 *   w_packed, s_packed  outputs of the sizes above, 256-byte aligned.  Pad
 *            rows hold zero elements and scale byte 127.
 * mxfp8_unpack_weight_fp4: inverse of mxfp8_prepare_weight_fp4, for tests
 *   and tooling: writes the full padded operand w_e2m1 [N_pad, K/2] bytes
 *   (contiguous, 16-byte aligned; pad rows zero) and w_s_e8m0 [N_pad, K/32]
 *   (contiguous; pad rows byte 127).  Same size rules as the pack.
 * mxfp8_linear_w4a8_workspace_bytes: host-only.  As mxfp8_linear's on the
 *   decode, mid-M and slab kernels (each has a 4-bit form); on the tile
 *   path, mxfp8_linear's plus N_pad * K bytes where the table splits K: the
 *   weight is then widened (exactly: every E2M1 value is an E4M3 value) to
 *   the MXFP8 tiles for the split-K tile GEMM.
 * mxfp8_linear_w4a8: y[m, n] = bf16( sum_k deq(q(x))[m, k] * deq4(W)[n, k]
 *   + bias[n] ), fp32 accumulate, one rounding; arguments as mxfp8_linear
 *   with the packed MXFP4 weight.  M <= 128 streams the 4-bit weight once
 *   (half the bytes of MXFP8).  Errors as mxfp8_linear.
 */
/*
 * bf16 -> MXFP4 (the MX rule with E2M1 elements: shared exponent
 * floor(log2 amax) - 2, RNE, saturate to +-6, all-zero block -> byte 0):
 *   x_bf16 [M, K] row stride ldx (ldx >= K, ldx % 8 == 0, 16-byte aligned);
 *   q_e2m1 [M, K/2] bytes, row stride ldq (ldq >= K/2, ldq % 4 == 0, 4-byte
 *          aligned), element 2j in the low nibble of byte j;
 *   s_e8m0 [M, K/32] row stride lds.  K % 32 == 0.
 * For making W4A8 weights from a bf16 checkpoint (the output feeds
 * mxfp8_prepare_weight_fp4).
 */
int mxfp8_quantize_fp4(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, void* q_e2m1, int64_t ldq,
                       void* s_e8m0, int64_t lds, void* stream);
int mxfp8_prepared_weight_fp4_bytes(int64_t N, int64_t K, size_t* w_bytes, size_t* s_bytes);
int mxfp8_prepare_weight_fp4(const void* w_e2m1, const void* w_s_e8m0, int64_t N, int64_t K, int64_t ldw,
                             int64_t ldws, void* w_packed, void* s_packed, void* stream);
int mxfp8_unpack_weight_fp4(const void* w_packed, const void* s_packed, int64_t N, int64_t K, void* w_e2m1,
                            void* w_s_e8m0, void* stream);
int mxfp8_linear_w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes);
int mxfp8_linear_w4a8(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const void* w_packed,
                      const void* s_packed, int64_t N, const void* bias_bf16, void* y_bf16, int64_t ldy,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two kernels of mxfp8_linear's large-M path, exposed separately (for
 * timing each, and for callers that reuse one quantized activation across
 * several weights).  The packed activation layout is the packed weight
 * layout with M in place of N: rows padded to a multiple of 128, opaque
 * order owned by this library; mxfp8_unpack_weight(qp, sp, M, K, ...)
 * returns it to plain [M_pad, K] / [M_pad, K/32] bytes.
 *
 * mxfp8_packed_act_bytes: host-only sizes for M rows (M >= 1, K % 256 == 0):
 *   *q_bytes = M_pad * K, *s_bytes = M_pad * K / 32, M_pad = ceil(M/128)*128.
 * mxfp8_quantize_act_packed: step 1 into that layout (same bytes as
 *   mxfp8_quantize_act, reordered; pad rows are zero with scale byte 0).
 *   x_bf16 as in mxfp8_quantize_act; qp, sp 256-byte aligned.
 * mxfp8_gemm_packed: step 3 (the mm_mxfp8 GEMM of vLLM PR #52204's
 *   apply_weights) + epilogue on packed activations; other arguments as
 *   mxfp8_linear.  Needs no workspace.
 */
int mxfp8_packed_act_bytes(int64_t M, int64_t K, size_t* q_bytes, size_t* s_bytes);

int mxfp8_quantize_act_packed(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, void* q_packed,
                              void* s_packed, void* stream);

int mxfp8_gemm_packed(const void* q_packed, const void* s_packed, int64_t M, int64_t K,
                      const void* w_packed, const void* ws_packed, int64_t N, const void* bias_bf16,
                      void* y_bf16, int64_t ldy, void* stream);

/*
 * Test entry: step 3 alone on activations quantized elsewhere, in the
 * boundary's row-major layout (the GEMM given quantized A: the output of
 * mxfp8_quantize_act, or of a reference quantizer, drives the block-scaled
 * GEMM + epilogue directly, so the GEMM can be checked apart from the
 * quantizer):
 *   q_e4m3 [M, K] bytes, row stride ldq (ldq >= K, ldq % 16 == 0, 16-byte aligned)
 *   s_e8m0 [M, >= K/32] bytes, row stride lds (lds >= K/32)
 *   other arguments as mxfp8_linear; workspace of at least
 *   mxfp8_gemm_prequant_workspace_bytes(M, N, K), 256-byte aligned, no
 *   initialization needed (it receives the activations in the packed layout).
 * Always the large-tile GEMM (for every M), so its output equals
 * mxfp8_linear's on that path bit for bit.
 */
int mxfp8_gemm_prequant_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes);
int mxfp8_gemm_prequant(const void* q_e4m3, int64_t ldq, const void* s_e8m0, int64_t lds, int64_t M, int64_t K,
                        const void* w_packed, const void* ws_packed, int64_t N, const void* bias_bf16, void* y_bf16,
                        int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ---------------------------------------------------------------------------
 * Top-k routed MXFP8 mixture-of-experts layer (the grouped variant).
 *
 * What is computed ("feat(moe): add unified block-scale FP8 support",
 * flashinfer PR #4026, walkthrough: BF16 activations in, MXFP8 inside;
 * "Feature/sm100 low latency nvfp4 kernels", flashinfer PR #1214, Highlights:
 * the Renormalize routing; "Add support for FlashInfer mxfp8", sglang PR
 * #18945: fused w13 = [gate; up] and w2 expert weights with 32-K UE8M0
 * scales).  For each token t:
 *   ids = the topk largest logits[t, :] (ties: lower expert id first),
 *   w   = softmax over those topk logits (fp32),
 *   for each selected e: h = deq(q(x_t)) . deq(w13[e])^T   ([2I], fp32 acc),
 *                        a = bf16( silu(h[0:I]) * h[I:2I] ),  silu(z) = z/(1+e^-z),
 *                        o_e = deq(q(a)) . deq(w2[e])^T        ([H], fp32 acc),
 *   y[t] = bf16( sum_j w_j * o_{e_j} ), the products and the sum in fp32 (slot
 *          order), rounded once.
 * q() is the MX quantization of mxfp8_quantize_act along the contraction
 * dimension (H for x, I for a).
 *
 * Shapes: H % 256 == 0, I % 256 == 0, 1 <= E <= 256, 1 <= topk <= min(E, 16),
 * T >= 0 (T == 0 is a no-op); limits H, I <= 2^20, T <= 2^24, T*topk <= 2^26
 * and (T+1)*H < 2^32 (the quantized token rows are addressed with 32-bit
 * offsets); anything else returns MXFP8_E_SHAPE.  Checkpoint layouts
 * (contiguous, row-major):
 *   w13 E4M3 [E, 2I, H] with UE8M0 [E, 2I, H/32]  (rows 0..I-1 gate, I..2I-1 up)
 *   w2  E4M3 [E, H, I]  with UE8M0 [E, H, I/32]
 * The whole layer runs in this library's kernels on `stream`; results are
 * deterministic (no atomics in any sum).
 * ---------------------------------------------------------------------------
 */

/* Host-only sizes of the prepared (packed) expert weights. */
int mxfp8_moe_prepared_bytes(int64_t E, int64_t H, int64_t I, size_t* w13_bytes, size_t* s13_bytes,
                             size_t* w2_bytes, size_t* s2_bytes);

/*
 * One-time preparation of the expert weights (the MoE counterpart of
 * mxfp8_prepare_weight): packs w13 with its gate and up rows interleaved for
 * the fused SiLU-gating epilogue, and w2, into opaque layouts owned by this
 * library.  w13_e4m3 / w2_e4m3 16-byte aligned; outputs 256-byte aligned,
 * sizes from mxfp8_moe_prepared_bytes.
 */
int mxfp8_moe_prepare_weights(const void* w13_e4m3, const void* w13_s_e8m0, const void* w2_e4m3,
                              const void* w2_s_e8m0, int64_t E, int64_t H, int64_t I, void* w13_packed,
                              void* s13_packed, void* w2_packed, void* s2_packed, void* stream);

/* Host-only workspace bytes of mxfp8_moe_grouped (contents need no init). */
int mxfp8_moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk, size_t* bytes);

/*
 * The MoE layer.  x_bf16 [T, H] contiguous, 16-byte aligned; logits_f32
 * [T, E] contiguous; y_bf16 [T, H] contiguous, 16-byte aligned (written
 * entirely); prepared weights from mxfp8_moe_prepare_weights; workspace of at
 * least mxfp8_moe_workspace_bytes, 256-byte aligned.  Calls sharing a
 * workspace must be ordered on one stream.
 */
int mxfp8_moe_grouped(const void* x_bf16, const float* logits_f32, int64_t T, int64_t H, int64_t E,
                      int64_t topk, int64_t I, const void* w13_packed, const void* s13_packed,
                      const void* w2_packed, const void* s2_packed, void* y_bf16, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Test hook: when set (all five non-NULL), every later mxfp8_moe_grouped call
 * also writes, for row t*topk + j (token t, slot j): the bf16 gated
 * activation act_bf16 [T*topk, I], its MX quantization act_e4m3 [T*topk, I]
 * and act_e8m0 [T*topk, I/32], the routed expert ids_i32 [T*topk] and the
 * routing weight wts_f32 [T*topk] (act_bf16 8-byte aligned, the others
 * 4-byte aligned).  All NULL turns it off; MXFP8_E_NULLPTR if only some are
 * NULL.  Process-wide: set it between calls, never concurrently with one.
 */
int mxfp8_moe_debug_capture(void* act_bf16, void* act_e4m3, void* act_e8m0, void* ids_i32, void* wts_f32);

/*
 * Test hook: force the GEMM path of mxfp8_linear and mxfp8_linear_w4a8.
 * 0 or 2 = automatic: the path and the tile GEMM's K splits come from the
 * shape table measured on MI355X (shape_table.inc, written by
 * mxfp8_block_scaled_amd/tune_shapes.py), within each kernel's limits
 * (decode kernel M <= 16 and K <= 8192, mid-M kernel M <= 128 and
 * K <= 8192, split-K slab kernel M <= 128; K splits s need
 * (K/64) % (4s) == 0); 1 = large-tile path with the table's splits; 3 =
 * mid-M kernel where it applies; 4 = decode kernel where it applies; 5 =
 * split-K slab kernel where it applies; 6 / 7 = medium-tile GEMM with
 * 128 x 128 / 128 x 64 tiles (MXFP8 only: mxfp8_linear_w4a8 takes the
 * large-tile path there); 16 + s (s = 1, 2, 4, 8) = large-tile path with s K
 * splits where they apply (else one).  A forced path that a
 * shape cannot take falls back to the large-tile path;
 * mxfp8_linear_workspace_bytes follows the forced choice.  Process-wide;
 * returns the previous value, or MXFP8_E_SHAPE for an unknown value.
 */
int mxfp8_debug_force_path(int path);

/*
 * Test hook (host only): the plan mxfp8_linear takes for an M x N x K call
 * under the current forcing: *path = 0 large-tile GEMM, 1 decode kernel,
 * 2 mid-M kernel, 3 split-K slab kernel, 4 / 5 medium-tile GEMM with
 * 128 / 64 activation rows per tile; *splits = the tile GEMM's K splits (1 for the other paths).
 * MXFP8_E_SHAPE for M < 1, N < 1 or K not a positive multiple of 256.
 */
int mxfp8_debug_plan(int64_t M, int64_t N, int64_t K, int* path, int* splits);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_H_ */
