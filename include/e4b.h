/*
 * e4b.h -- C ABI of the MI355X (gfx950) fused blockwise-4-bit Mixture-of-Experts
 * expert MLP: quantize / dequantize a fused expert stack, the routed SwiGLU
 * forward, and the frozen-base input gradient (dgrad).
 *
 * Sources (page titles; sections named per entry point below):
 *   [sdist]  experts4bit-qlora 0.1.0 source distribution, module
 *            experts4bit_qlora/_vendor/experts.py, class Experts4bit.
 *   [PR]     bitsandbytes pull request #1965, "Add Experts4bit for 4-bit
 *            quantization of fused MoE experts".
 *   [README] experts4bit-qlora 0.4.0 README (PyPI wheel metadata).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Stacks are row-major [E, out, in] per expert ([sdist] class docstring):
 *   gate_up is [E, 2I, H] with rows 0..I-1 the gate and rows I..2I-1 the up
 *   projection; down is [E, H, I].
 * - Packed codes: uint8 [E, out*in/2], two 4-bit codes per byte, the even
 *   element of the flattened row-major [out, in] in the high nibble.
 * - absmax: fp32 [E, out*in/64], one scale per 64 consecutive elements of a
 *   row; in % 64 == 0 so a block never straddles a row or an expert
 *   ([sdist] Experts4bit.__init__ block-alignment check). absmax is always
 *   fp32 and the codebook is a library constant chosen by enum, never a
 *   caller buffer ([PR] "Dtype-cast safety" bullet).
 * - bf16 tensors are raw IEEE bfloat16 bit patterns (uint16).
 * - Every pointer argument except the `const e4b_stack*`/`const
 *   e4b_moe_layer*` descriptors (host memory, read during the call only) is
 *   a DEVICE pointer owned by the caller; the library never allocates or
 *   frees memory and keeps no state between calls beyond its code objects.
 * - Device buffers must be 16-byte aligned (E4B_ERR_ALIGN otherwise).
 * - Asynchrony: every call validates its arguments on the host, enqueues
 *   kernels on `stream` and returns; no call synchronizes. A non-OK status is
 *   returned synchronously and nothing is enqueued for validation errors.
 * - Errors follow the pages' fail-loudly rule ([README] support matrix
 *   "Unsupported" definition): a bad argument is reported, never ignored.
 *   T == 0 is a valid no-op.
 * - Device preconditions that are NOT checked: finite weights and logits;
 *   0 <= topk_idx < E when it is an input. An id outside [0, E) never leads
 *   to an out-of-bounds access: every kernel that reads ids treats it as
 *   expert 0, so the pair's result is meaningless but the call stays in
 *   bounds (the Python binding can check the ids first). Given ids may
 *   repeat an expert within a token: each slot is a pair of its own.
 */
#ifndef E4B_H
#define E4B_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  E4B_OK = 0,
  E4B_ERR_NULL = 1,      /* a required pointer is NULL */
  E4B_ERR_SHAPE = 2,     /* a dimension <= 0, in % 64 != 0, top_k not in [1, min(E, 32)],
                            E > 1024, inconsistent gate_up/down shapes, or a size too large */
  E4B_ERR_BLOCKSIZE = 3, /* blocksize != 64 (MXFP4: != 32) */
  E4B_ERR_CODEBOOK = 4,  /* unknown codebook, or gate_up/down codebooks differ */
  E4B_ERR_DTYPE = 5,     /* unknown output dtype */
  E4B_ERR_WORKSPACE = 6, /* workspace NULL or smaller than e4b_moe_workspace_bytes() */
  E4B_ERR_ALIGN = 7,     /* a device buffer is not 16-byte aligned */
  E4B_ERR_PATH = 8,      /* unknown path, or the decode path was asked for but does not apply (a BF16, INT8 or FP8 layer, T > 8, saved != NULL, or max(H, I) above 16384) */
  E4B_ERR_HIP = 9        /* a kernel launch failed (hipGetLastError after the launch) */
} e4b_status;

/* MXFP4 = the MX storage the [0.31.1] project page names for gpt-oss experts
 * ("dequantised bit-identically") and for its native MXFP4 row, read as the
 * OCP Microscaling Formats (MX) v1.0 FP4 format: E2M1 codes (same code layout
 * and nibble order as FP4, unscaled magnitudes {0,.5,1,1.5,2,3,4,6}) with one
 * E8M0 scale 2^(s-127) per 32 consecutive elements of a row in `scales`
 * (uint8 [E, out*in/32]); blocksize 32, `absmax` unused. The dequantized
 * weight code * 2^(s-127) is exact in fp32 and bf16, so every path (grouped
 * forward, dgrad, decode GEMV, LoRA) runs on exactly the stored values.
 *
 * Storage modes. The 16-entry codebooks ([sdist] Experts4bit.__init__
 * quant_type "nf4"/"fp4"): NF4 = the NormalFloat-4 table of the QLoRA paper
 * (arXiv:2305.14314); FP4 = e2m1 (sign bit 3, magnitudes {0,.5,1,1.5,2,3,4,6}/6).
 * BF16 = the 16-bit passthrough lane of the [README] support matrix (the
 * reference baseline, no absmax buffer): `packed` holds the bf16 weight
 * [E, out*in] (two bytes per element, round-to-nearest-even of the fp32
 * weight), `absmax` is unused and may be NULL. A BF16 layer runs the grouped
 * path only (the decode GEMV reads 4-bit codes). */
/* Storage modes ([README] "Storage modes: the support matrix"): the 4-bit
 * codebooks NF4 and FP4 (two codes per byte), the bf16 passthrough lane, MXFP4
 * (E2M1 codes + E8M0 scales), and the 8-bit blockwise lanes INT8 (the
 * dynamic tree map) and FP8 (an E4M3 codebook), one code byte per element:
 * sign bit 7 | index into 128 ascending magnitudes from 0 to 1 (the tables
 * are defined in csrc/codebook8.h). The grouped GEMMs decode the code bytes
 * in their weight staging through a 256-entry table, as they decode the 4-bit
 * codes (bf16(fl32(value * absmax))); as on the pages, the 8-bit lanes have
 * no decode GEMV. */
typedef enum {
  E4B_CB_NF4 = 0,
  E4B_CB_FP4 = 1,
  E4B_CB_BF16 = 2,
  E4B_CB_MXFP4 = 3,
  E4B_CB_INT8 = 4,
  E4B_CB_FP8 = 5
} e4b_codebook;

typedef enum { E4B_F32 = 0, E4B_BF16 = 1 } e4b_dtype;

/* Forward path selection. AUTO = the decode dequant-GEMV path when T <= 8,
 * saved == NULL and the layer is a gated 4-bit one (NF4, FP4, MXFP4), else
 * the grouped MFMA path. MX8 = the MX forward of an
 * MXFP4 gated layer on gfx950's block-scaled MFMA ([0.31.1] native MXFP4
 * row): x and a = bf16(silu(g) * u) are converted per row to MXFP8 (E4M3, an
 * E8M0 scale per 32; the OCP MX v1.0 rule with emax 8: saturating,
 * round-to-nearest-even), so the result approximates the exact-weights
 * forward to about the E4M3 rounding (2^-4 relative per activation); it
 * needs H % 128 == 0, I % 128 == 0 and saved == NULL (E4B_ERR_PATH
 * otherwise). */
typedef enum {
  E4B_PATH_AUTO = 0,
  E4B_PATH_GROUPED = 1,
  E4B_PATH_DECODE = 2,
  E4B_PATH_MX8 = 3
} e4b_path;

/* One quantized stack (device pointers; the struct itself is host memory). */
typedef struct {
  const uint8_t *packed; /* [E, out*in/2]; BF16: [E, out*in] bf16; INT8, FP8: [E, out*in] codes */
  const float *absmax;   /* [E, out*in/64]; BF16, MXFP4: unused */
  int64_t E, out, in;
  int32_t blocksize; /* 64; MXFP4: 32 */
  int32_t codebook;  /* e4b_codebook */
  const uint8_t *scales; /* MXFP4: E8M0 [E, out*in/32]; other modes: unused */
} e4b_stack;

/* A MoE layer: gate_up (out = 2I, in = H) and down (out = H, in = I), same E,
 * same codebook ([README] "one module, one scheme"). A first stack of out = I
 * rows selects the ungated variant ([sdist] Experts4bit has_gate=False: a
 * plain up projection h, a = silu(h)); it runs the grouped path and takes no
 * LoRA adapters. */
typedef struct {
  e4b_stack gate_up;
  e4b_stack down;
} e4b_moe_layer;

/* Blockwise absmax quantization of an fp32 [E, out, in] stack.
 * [sdist] Experts4bit.from_float / _quantize_stack (per expert, blocksize 64,
 * no double quantization; [PR] "Non-goals" keeps absmax a plain fp32 buffer).
 * absmax = max |w| over each 64-block; code = nearest codebook entry to
 * w/absmax decided exactly (ties: NF4 lower code, FP4 smaller magnitude; FP4
 * sign bit = sign bit of w); an NF4 block of zeros stores code 7. INT8 and
 * FP8: the magnitude nearest |w|/absmax (ties: the smaller one), sign bit 7 =
 * sign bit of w, one code byte per element.
 *   w      : device fp32 [E, out, in], finite (unchecked)
 *   packed : device uint8 [E, out*in/2]; INT8, FP8: [E, out*in]   (written)
 *   absmax : device fp32  [E, out*in/64]  (written)
 * codebook E4B_CB_BF16 writes the bf16 rounding (nearest even) of w to
 * `packed` ([E, out*in] bf16) and leaves `absmax` (may be NULL) untouched.
 * Errors: NULL, SHAPE (E/out/in <= 0, in % 64 != 0), BLOCKSIZE, CODEBOOK,
 * ALIGN, HIP. */
e4b_status e4b_quantize_nf4(const float *w, int64_t E, int64_t out, int64_t in,
                            int32_t blocksize, int32_t codebook, uint8_t *packed,
                            float *absmax, hipStream_t stream);

/* MXFP4 conversion of an fp32 [E, out, in] stack (OCP MX v1.0, read for the
 * [0.31.1] project page's MXFP4 experts): per block of 32 consecutive
 * elements, shared exponent = floor(log2(max |w|)) - 2 clamped to
 * [-127, 127] (a block of zeros: -127), scale byte = shared + 127; each
 * element is w / 2^shared rounded to the nearest E2M1 value (ties to the even
 * mantissa, beyond 6 saturated), sign bit = sign bit of w.
 *   w      : device fp32 [E, out, in], finite (unchecked); in % 32 == 0
 *   packed : device uint8 [E, out*in/2]   (written)
 *   scales : device uint8 [E, out*in/32]  (written)
 * Errors: NULL, SHAPE, ALIGN, HIP. */
e4b_status e4b_quantize_mxfp4(const float *w, int64_t E, int64_t out, int64_t in, uint8_t *packed,
                              uint8_t *scales, hipStream_t stream);

/* MXFP8 conversion of bf16 activation rows, as the MX forward (E4B_PATH_MX8)
 * feeds them to the block-scaled MFMA: per block of 32 consecutive elements
 * of a row, shared exponent = floor(log2(max |x|)) - 8 clamped to
 * [-127, 127] (a block of zeros: -127), scale byte = shared + 127, element =
 * x / 2^shared rounded to E4M3 (nearest even, saturating at 448; sign bit 7).
 * Layout: codes [rows, K] with the two bytes of every element pair swapped
 * (byte 2p holds element 2p + 1), scales [rows, K/32].
 *   x_bf16 : device bf16 [rows, K]; K % 32 == 0
 * Errors: NULL, SHAPE, ALIGN, HIP. */
e4b_status e4b_mx8_rows(const void *x_bf16, int64_t rows, int64_t K, uint8_t *codes,
                        uint8_t *scales, hipStream_t stream);

/* Dequantize a whole stack: w_out[e, r, c] = fl32(code * absmax) (one fp32
 * rounding of the exact product), or its round-to-nearest-even bf16 when
 * dtype == E4B_BF16. [sdist] Experts4bit._dequantize_expert. A BF16 stack
 * gives its stored values (exact in fp32); an MXFP4 stack gives code *
 * 2^(s-127) (exact in both dtypes).
 *   st    : host descriptor of device buffers
 *   w_out : device [E, out, in] fp32 or bf16 (written)
 * Errors: NULL, SHAPE, BLOCKSIZE, CODEBOOK, DTYPE, ALIGN, HIP. */
e4b_status e4b_dequantize_nf4(const e4b_stack *st, int32_t dtype, void *w_out,
                              hipStream_t stream);

/* Asynchronous copy of one stored stack (packed codes or bf16 weights, and
 * the absmax when the mode has one) from `src` to `dst`, on `stream`
 * (hipMemcpyAsync: host-to-device from pinned host memory, or device-to-
 * device). It is the transfer of the layer-granular prefetch of the
 * [README] "Prefetched expert offload" bullet (decode with experts that
 * exceed device memory): the caller copies layer L+1 into a second set of
 * device buffers on a side stream while layer L computes, and orders the
 * two streams with events, so at most two layers are resident.
 *   dst, src : host descriptors; dst's buffers on the device, src's on the
 *              device or in pinned host memory; same E, out, in, blocksize
 *              and codebook
 * Errors: NULL, SHAPE (descriptors differ), BLOCKSIZE, CODEBOOK, ALIGN, HIP. */
e4b_status e4b_stack_copy_async(const e4b_stack *dst, const e4b_stack *src, hipStream_t stream);

/* Routed SwiGLU expert forward. [sdist] Experts4bit.forward: for each
 * (token t, slot j) with expert e = topk_idx[t, j],
 *   h = W_gu[e] x_t ; g = h[:I] ; u = h[I:] ; a = silu(g) * u ;
 *   y_t = sum_j topk_w[t, j] * (W_dn[e] a), accumulated in fp32,
 * with W the dequantized stacks (bf16 operands, fp32 accumulation); an
 * ungated layer has a = silu(W_up[e] x_t).
 *   x_bf16        : device bf16 [T, H]
 *   router_logits : device fp32 [T, E] or NULL. Given: topk_idx/topk_w are
 *                   OUTPUTS = the top_k largest logits (descending, ties to the
 *                   lower expert id) and the softmax over them. NULL: topk_idx
 *                   and topk_w are INPUTS.
 *   topk_idx      : device int32 [T, top_k]
 *   topk_w        : device fp32  [T, top_k]
 *   y_bf16        : device bf16 [T, H] (written)
 *   saved         : device buffer of e4b_moe_saved_bytes() or NULL; when given,
 *                   the bf16 gate and up projections (ungated: h) of every pair and the
 *                   routing permutation are stored for e4b_moe_dgrad
 *                   (grouped path only)
 *   ws, ws_bytes  : device workspace, >= e4b_moe_workspace_bytes()
 *   path          : e4b_path
 * Errors: NULL, SHAPE, BLOCKSIZE, CODEBOOK, WORKSPACE, ALIGN, PATH, HIP. */
e4b_status e4b_moe_forward(const e4b_moe_layer *L, int64_t T, int32_t top_k,
                           const void *x_bf16, const float *router_logits,
                           int32_t *topk_idx, float *topk_w, void *y_bf16,
                           void *saved, void *ws, size_t ws_bytes, int32_t path,
                           hipStream_t stream);

/* Frozen-base input gradient of e4b_moe_forward with routing held fixed.
 * [PR] "What this adds", recompute-in-backward bullet: each projection's
 * backward forms grad_output @ W from a re-dequantized W (never a saved W);
 * frozen-base bullet: no weight gradient. Per pair (t, j), expert e:
 *   G2 = W_dn[e]^T grad_y_t ; grad_topk_w[t, j] = G2 . a ;
 *   grad_a = topk_w[t, j] G2 ; s = sigmoid(g) ;
 *   dg = grad_a u s (1 + g (1 - s)) ; du = grad_a g s ;
 *   grad_x_t = sum_j W_gu[e]^T [dg ; du]   (ungated: dh = grad_a s (1 + h (1 - s)),
 *   grad_x_t = sum_j W_up[e]^T dh).
 *   topk_idx, topk_w : device [T, top_k] (inputs, as used by the forward)
 *   x_bf16           : device bf16 [T, H]; required when saved == NULL
 *                      (the gate/up projections are recomputed), ignored otherwise
 *   saved            : the buffer filled by e4b_moe_forward, or NULL. Its
 *                      permutation replaces topk_idx (which must be the
 *                      forward's). Recompute and saved give bitwise-identical
 *                      results.
 *   grad_y_bf16      : device bf16 [T, H]
 *   grad_x_bf16      : device bf16 [T, H] (written)
 *   grad_topk_w      : device fp32 [T, top_k] (written) or NULL
 * Errors: NULL, SHAPE, BLOCKSIZE, CODEBOOK, WORKSPACE, ALIGN, HIP. */
e4b_status e4b_moe_dgrad(const e4b_moe_layer *L, int64_t T, int32_t top_k,
                         const int32_t *topk_idx, const float *topk_w,
                         const void *x_bf16, const void *saved,
                         const void *grad_y_bf16, void *grad_x_bf16,
                         float *grad_topk_w, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* Workspace bytes that e4b_moe_forward and e4b_moe_dgrad need for (L, T,
 * top_k) (one size serves both); 0 when the arguments are invalid. */
size_t e4b_moe_workspace_bytes(const e4b_moe_layer *L, int64_t T, int32_t top_k);

/* Bytes of the `saved` buffer (its contents are internal to the library): the
 * bf16 gate and up projections of every routed pair (gated: in blocks of 256
 * sorted pairs x 128 intermediate columns, g and u side by side, one block per
 * m-tile and column block; ungated: h as [T*top_k, I]) followed by the routing
 * permutation (int32 arrays over experts, m-tiles and pairs) and room for the
 * LoRA forward's two per-pair rank projections (fp32 [T*top_k, 16] each; the
 * base forward leaves it unwritten); 0 when invalid. The forward never writes
 * the padding of the blocks (rows past an expert's pairs, blocks of m-tiles
 * the routing does not produce) and nothing reads it. */
size_t e4b_moe_saved_bytes(const e4b_moe_layer *L, int64_t T, int32_t top_k);

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): e4b_moe_forward with its workspace in a fixed per-GPU device
 * array of the library (E4B_NOALLOC_SCRATCH_BYTES) instead of a caller
 * buffer; the other arguments are those of e4b_moe_forward. Each GPU holds
 * its own copy of the array until the process ends; every call on that GPU
 * shares it and it keeps the last call's contents (no kernel of the forward
 * reads a workspace byte that the same call did not write, so nothing is
 * cleared). Calls that overlap on one GPU (two streams or two threads) race
 * on the array: the caller serializes them. No call allocates; the first
 * call on a device looks up the array's device address once.
 * Errors: as e4b_moe_forward; WORKSPACE when e4b_moe_workspace_bytes(L, T,
 * top_k) exceeds E4B_NOALLOC_SCRATCH_BYTES; HIP when the address lookup fails. */
#define E4B_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
e4b_status e4b_moe_forward_noalloc(const e4b_moe_layer *L, int64_t T, int32_t top_k,
                                   const void *x_bf16, const float *router_logits,
                                   int32_t *topk_idx, float *topk_w, void *y_bf16, void *saved,
                                   int32_t path, hipStream_t stream);

/* Per-expert LoRA adapters over the frozen base (fp32 device buffers).
 * [README] Quickstart: ExpertsLoRA(base, r=8, alpha=16) attaches trainable
 * per-expert LoRA to a frozen 4-bit stack; only the adapters train. The
 * adapter module is not printed on the pages; the usual LoRA form is used on
 * both projections of every expert e, with scale s = alpha / r:
 *   h = W_gu[e] x + s B_gu[e] (A_gu[e] x),  o = W_dn[e] a + s B_dn[e] (A_dn[e] a).
 *   A_gu : [E, r, H]    B_gu : [E, 2I, r]  (rows follow the gate | up rows)
 *   A_dn : [E, r, I]    B_dn : [E, H, r]
 * 1 <= r <= 16. The low-rank term enters each grouped GEMM as one extra
 * 16-deep MFMA slice (bf16 operands, fp32 accumulation). */
typedef struct {
  const float *A_gu, *B_gu, *A_dn, *B_dn;
  int32_t r;
  float alpha;
} e4b_lora;

/* Forward of e4b_moe_forward with LoRA adapters; always the grouped path
 * (saved, when given, is filled as by e4b_moe_forward, with the adapted g|u,
 * plus the rank projections x A_gu^T and a A_dn^T that the backward reuses).
 * ws must hold e4b_moe_lora_workspace_bytes(). Errors as e4b_moe_forward,
 * plus NULL / SHAPE for the adapter descriptor (r outside [1, 16]). */
e4b_status e4b_moe_lora_forward(const e4b_moe_layer *L, const e4b_lora *lora, int64_t T,
                                int32_t top_k, const void *x_bf16, const float *router_logits,
                                int32_t *topk_idx, float *topk_w, void *y_bf16, void *saved,
                                void *ws, size_t ws_bytes, hipStream_t stream);

/* Backward of e4b_moe_lora_forward with routing held fixed: the input
 * gradient and grad_topk_w as e4b_moe_dgrad (the base stays frozen) plus the
 * adapter gradients of sum(grad_y * y), per pair (t, j), G_o = topk_w grad_y_t:
 *   grad_a = W_dn^T G_o + s A_dn^T (B_dn^T G_o)
 *   dB_dn += s G_o (A_dn a)^T         dA_dn += s (B_dn^T G_o) a^T
 *   grad_h = [dg ; du] from grad_a     grad_x_t += W_gu^T grad_h + s A_gu^T (B_gu^T grad_h)
 *   dB_gu += s grad_h (A_gu x_t)^T     dA_gu += s (B_gu^T grad_h) x_t^T
 *   x_bf16   : device bf16 [T, H], required (the adapter gradients use it)
 *   saved    : the buffer filled by e4b_moe_lora_forward with the same
 *              adapters, or NULL (recomputes the forward's projections,
 *              bitwise equal to the saved ones)
 *   dA_gu, dB_gu, dA_dn, dB_dn : device fp32, adapter shapes (written, not
 *              accumulated); each sum runs over an expert's pairs in sorted
 *              order, so results are deterministic
 * Errors as e4b_moe_dgrad, plus NULL / SHAPE for the adapters. */
e4b_status e4b_moe_lora_backward(const e4b_moe_layer *L, const e4b_lora *lora, int64_t T,
                                 int32_t top_k, const int32_t *topk_idx, const float *topk_w,
                                 const void *x_bf16, const void *saved, const void *grad_y_bf16,
                                 void *grad_x_bf16, float *grad_topk_w, float *dA_gu,
                                 float *dB_gu, float *dA_dn, float *dB_dn, void *ws,
                                 size_t ws_bytes, hipStream_t stream);

/* Workspace bytes of the two LoRA calls (the base workspace plus the
 * adapters' per-pair projections, their bf16 operand packs and, for a
 * backward without saved state, the recomputed bf16 a [T*top_k, I]); 0 when
 * invalid. */
size_t e4b_moe_lora_workspace_bytes(const e4b_moe_layer *L, int64_t T, int32_t top_k);

/* Kernels of the forward and dgrad calls that the *_timed entry points can
 * bracket with events (benchmark instrumentation). */
typedef enum {
  E4B_K_GATE_UP_FWD = 0,   /* grouped gate_up GEMM + SiLU*up epilogue (MX path: its MX GEMM) */
  E4B_K_DOWN_FWD = 1,      /* grouped down GEMM (MX path: its MX GEMM) */
  E4B_K_DOWN_DGRAD = 2,    /* grouped GEMM on W_dn^T + SiLU-backward epilogue */
  E4B_K_GATE_UP_DGRAD = 3, /* grouped GEMM on W_gu^T */
  E4B_K_DECODE_GATE_UP = 4,/* decode dequant-GEMV, gate_up + SiLU*up (routes and groups the pairs too) */
  E4B_K_DECODE_DOWN = 5,   /* decode dequant-GEMV, down (+ the weighted combine) */
  E4B_K_ROUTE = 6,         /* top-k routing from logits */
  E4B_K_PERMUTE = 7,       /* the permutation (the first of its kernels to the last) */
  E4B_K_COMBINE = 8,       /* forward gather-combine */
  E4B_K_COMBINE_DGRAD = 9, /* dgrad gather-combine + routing-weight gradient */
  E4B_K_COUNT = 10
} e4b_kernel;

/* Per-call kernel timing. For every kernel id whose start and stop events
 * are both non-NULL, the call launches that kernel with
 * hipExtLaunchKernelGGL(start, stop), so the two events carry the start and
 * end time of that dispatch on the launch stream (hipEventElapsedTime gives
 * the kernel's duration). A kernel launched twice in one call (the gate_up
 * GEMM recomputed by a dgrad without saved state) records the last launch;
 * E4B_K_PERMUTE spans its three launches. Events are caller-owned and
 * created beforehand. The library keeps no reference after the call. */
typedef struct {
  hipEvent_t start[E4B_K_COUNT];
  hipEvent_t stop[E4B_K_COUNT];
} e4b_kernel_events;

/* e4b_moe_forward / e4b_moe_dgrad with per-call kernel timing (`events` may
 * be NULL: then identical to the untimed calls). Same arguments, results
 * and errors. */
e4b_status e4b_moe_forward_timed(const e4b_moe_layer *L, int64_t T, int32_t top_k,
                                 const void *x_bf16, const float *router_logits,
                                 int32_t *topk_idx, float *topk_w, void *y_bf16, void *saved,
                                 void *ws, size_t ws_bytes, int32_t path, hipStream_t stream,
                                 const e4b_kernel_events *events);
e4b_status e4b_moe_dgrad_timed(const e4b_moe_layer *L, int64_t T, int32_t top_k,
                               const int32_t *topk_idx, const float *topk_w, const void *x_bf16,
                               const void *saved, const void *grad_y_bf16, void *grad_x_bf16,
                               float *grad_topk_w, void *ws, size_t ws_bytes, hipStream_t stream,
                               const e4b_kernel_events *events);

/* Where the grouped forward (saved == NULL) leaves its routing permutation
 * in the workspace, for inspection (int32 arrays; byte offsets from ws):
 * counts [E], offsets [E + 1] (first sorted position of each expert),
 * tile_offsets [E + 1] (first m-tile of each expert, m-tiles of 256 sorted
 * pairs), sorted_pair [P] (flat pair id t * top_k + j at each sorted
 * position, stable: ascending within an expert), pos_of_pair [P] (its
 * inverse), tile_map [m_tiles_bound] (int32 x4 per m-tile: expert, segment
 * start, first row, rows). Errors as e4b_moe_workspace_bytes' arguments
 * (NULL for a NULL `out`). */
typedef struct {
  size_t counts, offsets, tile_offsets, sorted_pair, pos_of_pair, tile_map;
  int64_t m_tiles_bound;
} e4b_perm_layout;
e4b_status e4b_moe_perm_layout(const e4b_moe_layer *L, int64_t T, int32_t top_k,
                               e4b_perm_layout *out);

/* Static, human-readable text for a status code. */
const char *e4b_status_string(e4b_status status);

#ifdef __cplusplus
}
#endif

#endif /* E4B_H */
