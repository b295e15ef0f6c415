/*
 * moe.h - C ABI of the MI355X (gfx950) sparse mixture-of-experts FFN block.
 *
 * The block (forward pass only):
 *   logits = x W_r^T (+ logit_bias)                      router projection
 *   s      = sigmoid(logits) | softmax_E(logits)         scores, fp32
 *   chosen = top-k of (s + select_bias)                  the bias moves selection only
 *   w      = s[chosen] (/ sum, if norm_topk) * routed_scale
 *   z      = x | latent_down(x)
 *   y_r[t] = sum_j w[t,j] * down_e(swiglu(gate_e z_t, up_e z_t)),  e = chosen[t,j]
 *   latent:  y_r = latent_up(rms_norm(y_r))
 *   y      = y_r | y_r + shared(x) | c0*y_r + c1*shared(x), c = softmax(x W_c^T + b_c)
 *
 * Sources (web pages; sections named, no line numbers):
 *   - mlxcel PR #1044 "Klear sparse MoE family": point 2 (shared expert blended
 *     through a per-token 2-way softmax of a [2, hidden] head with a [2] bias),
 *     point 3 (sigmoid scoring in fp32, bias added to a copy used for selection,
 *     weights gathered unbiased, norm_topk_prob renormalises, no routed scaling),
 *     "Other guards" (top-k range 1..num_experts, full expert stacks, zero checks
 *     before divisibility checks).
 *   - libmir-metal clamped_routed/experts/mod.rs: ClampedRoutedExperts::forward
 *     (flatten leading dims to [tokens, hidden], checked token product, router,
 *     top-k, gate/up with swiglu_limit, down applying the routing weights);
 *     ExpertLayout (MXFP4 blocks/scales/bias; stacked tensors required).
 *   - ferrox-models latent_moe.rs: module doc and kimi_latent_moe_forward (latent
 *     flow), route_top_k_sigmoid_with_bias(logits, bias, k, renormalize, scaling),
 *     KimiExpertWeights (w1 gate [ffn,in], w2 down [in,ffn], w3 up [ffn,in]).
 *   - mlxcel issue #974: SwitchLinear::Quantized {weight, scales, biases,
 *     group_size, bits} applied by gather_qmm in "affine" mode; quantisation
 *     parameters validated before they are stored ("Acceptance Criteria").
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library keeps
 *     no pointer after returning and allocates no device memory: scratch space is
 *     the caller's workspace `ws`.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = default stream).
 *   - Workspace query: ws == NULL writes the required byte count to *ws_bytes and
 *     returns MOE_OK without launching anything.  Otherwise *ws_bytes is the size
 *     of `ws`; too small -> MOE_ERR_WORKSPACE.  `ws` must be 256-byte aligned.
 *   - Every argument is validated before the first launch; on any error nothing
 *     is launched and no output is touched.  The library never aborts or throws.
 *   - T == 0 is a no-op returning MOE_OK (after validating the other arguments).
 *   - Row-major layouts; "[a, b]" lists dimensions outermost first.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,        /* NULL pointer, enum out of range, non-finite scalar */
  MOE_ERR_SHAPE = 2,      /* zero/negative dimension, mismatch, overflow, unsupported multiple */
  MOE_ERR_QUANT = 3,      /* bits / group_size not valid for the weight format */
  MOE_ERR_WORKSPACE = 4,  /* ws too small or misaligned */
  MOE_ERR_DEVICE = 5,     /* a HIP call failed (launch error, no device) */
  MOE_ERR_UNSUPPORTED = 6 /* valid but unsupported dtype/format combination */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_F16 = 2 } moe_dtype;
typedef enum { MOE_SIGMOID = 0, MOE_SOFTMAX = 1 } moe_scoring;
typedef enum { MOE_W_DENSE = 0, MOE_W_AFFINE4 = 1, MOE_W_MXFP4 = 2 } moe_wformat;
typedef enum { MOE_SHARED_NONE = 0, MOE_SHARED_ADD = 1, MOE_SHARED_BLEND = 2 } moe_shared_mode;

/*
 * n stacked matrices W[e] of shape [rows = out, cols = in]; applied as y = W x (+ bias).
 *   DENSE   w: dense_dtype (F32 or BF16) [n, rows, cols]
 *   AFFINE4 w: uint32 [n, rows, cols/8], element 8j+i in bits 4i..4i+3 of word j;
 *           scales, qbias: bf16 [n, rows, cols/group_size];
 *           weight = scale * q + qbias, q in 0..15  (bits must be 4,
 *           group_size 32, 64 or 128)
 *   MXFP4   w: uint8 [n, rows, cols/2], E2M1 codes, even element in the low nibble;
 *           scales: uint8 E8M0 [n, rows, cols/32]; weight = e2m1 * 2^(scale-127)
 *           (group_size must be 32, bits 4; scale byte 255 (NaN) is out of contract)
 *   bias (optional, any format): output bias [n, rows], bf16 (f32 for DENSE F32).
 *   packed: the stream moe_pack_weights wrote for this stack (for gate/up: the one
 *           stream of the pair, set on `gate`; `up.packed` is not read).  Required by
 *           every BF16/F16-activation GEMM; there w, scales and qbias are not read
 *           (they describe the source of the stream).  Unused on the F32 path.
 *   packed_scaled (optional, MXFP4 only): the stream moe_pack_weights_scaled wrote (for
 *           gate/up: the pair's stream, set on `gate`).  When the routed experts' gate and
 *           down stacks both carry one, moe_block_forward runs prefill-sized batches of the
 *           latent layer (f16 intermediates, expert widths in whole blocks of 128) on
 *           gfx950's block-scaled FP4 x FP8 MFMA (moe_experts_forward keeps the 16-bit
 *           path): the weights
 *           as stored (codes and E8M0 scales), the activations split into two FP8 terms
 *           with E8M0 block scales of 32 (about 8 significant bits, more than bf16).
 *           NULL, or any other batch: the 16-bit MFMA path.  256-byte aligned.
 * "qbias" (the affine offset of each group) and "bias" (the linear layer's output
 * bias) are different things on purpose.
 */
typedef struct {
  int32_t fmt;          /* moe_wformat */
  int32_t dense_dtype;  /* DENSE only: MOE_F32 or MOE_BF16 */
  int32_t n, rows, cols;
  int32_t group_size;   /* AFFINE4: 32/64/128; MXFP4: 32; DENSE: ignored */
  int32_t bits;         /* AFFINE4/MXFP4: 4; DENSE: ignored */
  const void *w;
  const void *scales;
  const void *qbias;
  const void *bias;
  const void *packed;
  const void *packed_scaled;
} moe_linear;

/* SwiGLU expert stack: h = silu(gate z) * (up z) with gate/up [n, I, D], down [n, D, I].
 * swiglu_limit > 0 clamps both gate and up pre-activations to [-limit, limit]
 * (after their output bias); <= 0 disables the clamp.  Must be finite. */
typedef struct {
  moe_linear gate, up, down;
  float swiglu_limit;
} moe_mlp;

typedef struct {
  int32_t num_experts;       /* E >= 1 */
  int32_t top_k;             /* 1 <= K <= E, K <= 32 */
  int32_t scoring;           /* moe_scoring */
  int32_t norm_topk;         /* 0/1: divide the K weights by their sum */
  float routed_scale;        /* finite; multiplies the (renormalised) weights */
  const void *w;             /* [E, H], same dtype as x */
  const float *logit_bias;   /* optional [E]: added to the logits (moves weights and selection) */
  const float *select_bias;  /* optional [E]: added to the scores for selection only */
} moe_router;

typedef struct {
  int32_t hidden;            /* H */
  int32_t expert_dim;        /* D: H, or the latent width when latent_down.w != NULL */
  moe_router router;
  moe_mlp experts;           /* n = E, gate/up [E, I, D], down [E, D, I] */
  int32_t shared_mode;       /* moe_shared_mode */
  moe_mlp shared;            /* n = 1, gate/up [1, I_s, H], down [1, H, I_s]; unused when NONE */
  const void *coef_w;        /* BLEND: [2, H], dtype of x; index 1 weights the shared branch */
  const float *coef_b;       /* BLEND: [2] */
  moe_linear latent_down;    /* w == NULL: no latent projection; else DENSE BF16 [1, D, H] */
  moe_linear latent_up;      /* DENSE BF16 [1, H, D] when latent */
  const float *latent_norm_w;/* optional [D]: RMSNorm of the routed sum before latent_up */
  float norm_eps;            /* > 0 and finite when latent_norm_w != NULL */
  int32_t inter_dtype;       /* storage of z, h, expert outputs: MOE_BF16 or MOE_F16
                                (MOE_F32 when x is f32).  MOE_F16 keeps 3 more mantissa
                                bits but its range ends at 65504: a value beyond it is
                                stored as +-inf and propagates to y (no saturation, no
                                error status).  With MOE_F16 a prefill-sized batch of a
                                bf16 layer also reads x as f16 and dequantises 4-bit
                                weights to f16 (11 bits instead of 8), so x is bound by
                                the same range there.  MOE_BF16 has the fp32 range. */
} moe_block;

/*
 * moe_pack_weights - write the GEMM's packed stream of a weight stack (once, at load time).
 *   a      the stack (natural layout above: DENSE BF16, AFFINE4 or MXFP4)
 *   b      NULL: `a` alone, in blocks of 32 rows (down projections, latent maps);
 *          else the up stack of a gate/up pair (`a` = gate, same format and shape):
 *          blocks of 16 gate rows followed by the same 16 up rows
 *   out    device buffer, 256-byte aligned; NULL: write the size to *out_bytes
 *   out_bytes  in: size of out; too small -> MOE_ERR_WORKSPACE
 * The stream is a permutation of the stored codes, scales and qbias (nothing is
 * converted; AFFINE4 words hold their 8 codes with the even elements in the low
 * half-word and the odd ones in the high half-word, element 2j at bit 4j and 2j+1 at
 * bit 16+4j); rows and reduction elements are zero-padded to whole blocks of 32 rows
 * and 256 elements (64 for DENSE).  Layout: per matrix, per row block, per chunk a
 * record of 4096 bytes of weights in MFMA lane order followed by the chunk's scales
 * (AFFINE4: 4 bytes per row and group, MXFP4: 1 byte per row and block).
 * Source: the gather_qmm weight planes of mlxcel issue #974 and libmir-metal's
 * ExpertLayout, re-laid for gfx950's 16x16x32 MFMA operand order.
 */
MOE_API moe_status moe_pack_weights(const moe_linear *a, const moe_linear *b, void *out, size_t *out_bytes,
                                    void *stream);

/*
 * moe_pack_weights_scaled - the stream of MXFP4 weights for the block-scaled MFMA (once,
 * at load time; see moe_linear.packed_scaled).  Arguments, sizes (the same as
 * moe_pack_weights for the stack) and errors as moe_pack_weights; `a` must be MXFP4
 * (else MOE_ERR_UNSUPPORTED).  Each record (32 tile rows x 256 elements) holds, for each
 * of its two 128-element stages and two 16-row halves, 1 KB in the FP4 operand order of
 * the 16x16x128 MFMA (lane l: the 16 stored bytes of row l%16 at elements 32*(l/16)..+32),
 * then one word per lane whose byte 2*stage + half is the E8M0 scale of those elements.
 * A permutation of the stored codes and scales: nothing is converted.
 * Source: libmir-metal ExpertLayout::Native (the MXFP4 gate/up and down kernels read the
 * weights as stored); the layout is gfx950's MFMA operand order.
 */
MOE_API moe_status moe_pack_weights_scaled(const moe_linear *a, const moe_linear *b, void *out, size_t *out_bytes,
                                           void *stream);

/*
 * moe_route - router projection, scoring, selection and weights.
 *   x        [T, H] (x_dtype F32 or BF16; router->w has the same dtype)
 *   topk_idx [T, K] int32 out: the K chosen experts of each token in ascending id
 *            order; equal selection keys go to the lower expert id
 *   topk_w   [T, K] float out: weights gathered from the unbiased scores, in the
 *            same slot order
 *   logits   optional [T, E] float out: x W_r^T + logit_bias, fp32 (for 256 tokens
 *            or more with BF16 x, the fp32 sum of the partial sums over slices of H,
 *            added in slice order: the same values moe_block_forward selects on).
 *            The slices are fixed by (T, H, E) alone, never by the device's compute
 *            unit count, so the logits (and the selection at near-ties) are the same
 *            bits on every gfx950 device and partition.
 *   ws       holds the router's partial sums (the query reports its size)
 * Source: mlxcel PR #1044 point 3; latent_moe.rs route_top_k_sigmoid_with_bias.
 */
MOE_API moe_status moe_route(const void *x, int32_t x_dtype, int64_t T, int32_t H, const moe_router *r,
                     int32_t *topk_idx, float *topk_w, float *logits,
                     void *ws, size_t *ws_bytes, void *stream);

/*
 * moe_permute - group the T*K slots (slot p = t*K + j) by expert.
 *   counts      [E] int32 out: slots routed to each expert
 *   offsets     [E+1] int32 out: exclusive prefix sum of counts (offsets[E] = T*K)
 *   sorted_slot [T*K] int32 out: for e ascending, the slots of e in ascending p
 *   slot_pos    [T*K] int32 out: inverse permutation, sorted_slot[slot_pos[p]] == p
 * topk_idx entries must lie in [0, E) and be distinct within a token (as produced
 * by moe_route); other input is out of contract.
 * Source: the gathered-expert application of gather_qmm (mlxcel issue #974) and
 * the routing indices handed to the gate/up and down kernels (libmir-metal execute).
 */
MOE_API moe_status moe_permute(const int32_t *topk_idx, int64_t T, int32_t K, int32_t E,
                       int32_t *counts, int32_t *offsets, int32_t *sorted_slot, int32_t *slot_pos,
                       void *ws, size_t *ws_bytes, void *stream);

/*
 * moe_experts_forward - the routed experts and their weighted sum:
 *   y_routed[t] = sum_j topk_w[t,j] * down_e(swiglu(gate_e z_t, up_e z_t)), j ascending.
 *   z        [T, D], z_dtype BF16 or F16 (F32 with DENSE F32 experts)
 *   ex       expert stack, n = E, gate/up [E, I, D], down [E, D, I]
 *   topk_idx, topk_w [T, K]; offsets [E+1], sorted_slot [T*K], slot_pos [T*K] from moe_permute
 *   y_routed [T, D] float out
 *   inter_dtype: storage of h and the per-slot outputs (BF16 or F16; F32 for f32 z)
 * Source: libmir-metal execute (mxfp4_gate_up with the clamp limit, mxfp4_down
 * with the routing weights); latent_moe.rs combine loop.
 */
MOE_API moe_status moe_experts_forward(const void *z, int32_t z_dtype, int64_t T, int32_t D, const moe_mlp *ex,
                               int32_t E, int32_t K, const int32_t *topk_idx, const float *topk_w,
                               const int32_t *offsets, const int32_t *sorted_slot, const int32_t *slot_pos,
                               int32_t inter_dtype, float *y_routed,
                               void *ws, size_t *ws_bytes, void *stream);

/*
 * moe_block_forward - the whole block for T tokens.
 *   x        [T, H] (x_dtype F32 or BF16)
 *   y        [T, H] out, y_dtype F32 or BF16 (F32 when x is F32)
 *   topk_idx, topk_w: optional [T, K] outputs of the routing (may be NULL)
 * After the call (once the stream has reached it) the workspace begins with the
 * routing state the experts ran on, int32 arrays at 256-byte aligned offsets, in
 * this order: counts [E], offsets [E+1], sorted_slot [T*K], slot_pos [T*K] (as
 * moe_permute defines them), then status [1]; each array starts at the previous
 * one's offset plus its size rounded up to a multiple of 256 bytes.  status is 0,
 * or 1 if a bounded wait between workgroups of the one-launch decode path (see
 * moe_set_decode_fusion) gave up, in which case that call's outputs are invalid
 * (a wait gives up only if the device could not hold the launch's workgroups at
 * once).  The rest of the workspace is unspecified.
 * Source: all of the above; the blend of mlxcel PR #1044 point 2; the latent flow
 * of latent_moe.rs.
 */
MOE_API moe_status moe_block_forward(const void *x, int32_t x_dtype, int64_t T, const moe_block *b,
                             void *y, int32_t y_dtype, int32_t *topk_idx, float *topk_w,
                             void *ws, size_t *ws_bytes, void *stream);

/*
 * moe_block_forward_noalloc - moe_block_forward without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and validation as
 * moe_block_forward; the scratch space is a fixed array of MOE_NOALLOC_SCRATCH_BYTES in
 * the library's code object, one per GPU, held until the process ends.  The call itself
 * allocates nothing (no hipMalloc, no hipFree, no allocating library routine).
 *   - A call whose workspace would exceed MOE_NOALLOC_SCRATCH_BYTES returns
 *     MOE_ERR_WORKSPACE before launching anything (about 600 tokens of the 2048-hidden,
 *     256-expert decode layer fit).
 *   - `stream` must belong to the calling thread's current device (else MOE_ERR_ARG).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap on one GPU (on
 *     different streams or threads) race and give undefined results.  Calls ordered on
 *     one stream are safe; each call initialises all the scratch state it reads.
 *   - The first call on a device looks up the array's device address (once per device).
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
MOE_API moe_status moe_block_forward_noalloc(const void *x, int32_t x_dtype, int64_t T, const moe_block *b,
                                             void *y, int32_t y_dtype, int32_t *topk_idx, float *topk_w,
                                             void *stream);

/*
 * moe_set_decode_fusion - choose how moe_block_forward runs a decode-sized batch (at most
 * 64 tokens, top_k <= 16, at most 256 experts, bf16 activations and intermediates, a router
 * whose logits take one pass, 4-bit routed experts, a shared expert of the same format or
 * none, no latent projection):
 *   enabled = 1 (default): the router, selection and permutation in one launch, gate/up and
 *                the down projection of every slot (and of the shared expert) in one
 *                persistent launch, then the weighted combine (3 launches per block);
 *   enabled = 2: the same, except that a batch of at most 16 tokens with an f32 or bf16
 *                output and a hidden size that is a multiple of 32 (at most 8192) runs in one
 *                launch: router tiles, selection and permutation first, then the experts,
 *                and each 32-column block of the output combined by the wave that completes
 *                it (the pages' fused single-token decode kernel, mlxcel PR #1044,
 *                "Validation"; not faster than the three launches on MI355X);
 *   enabled = 0: separate router, routing, gate/up, down and combine launches (5 in all).
 * All give the same bits: the same arithmetic in the same order (unlike the pages' fused
 * MoE decode kernel, whose output was not byte-identical to the unfused path; this switch
 * mirrors theirs: MLXCEL_FUSED_MOE).
 * The launches hand work between workgroups through counters that the library keeps in its
 * code object: three blocks of 110 KiB for each of up to 16 streams per device (one for the
 * three launches, two that single launches use in turn; each call leaves the next call's
 * block zero).  A call on a 17th stream of a device, on a stream of another device than the
 * current one, or on a stream under capture (a graph replayed on another stream would share
 * the blocks) takes the separate launches.
 * Process-wide, not thread-safe; enabled must be 0, 1 or 2 (else MOE_ERR_ARG).
 */
MOE_API moe_status moe_set_decode_fusion(int32_t enabled);

/*
 * Live timing of one kernel class with HIP events, for measurement tools.
 *   kind: 0 off; 1 grouped gate/up GEMM; 2 grouped down GEMM; 3 router logits;
 *         4 scores + top-k; 5 permutation; 6 combine; 7 plain GEMMs (latent
 *         projections, a shared expert run outside the grouped launches); 8 the
 *         one-launch decode experts (gate/up + down).
 * While a kind is on, every launch of that class is bracketed by hipEventRecord on
 * the stream it is launched on (a pool of 8192 event pairs, created on the first
 * call with kind != 0; launches past a full pool are not timed).  moe_timing_read
 * waits for the recorded events, writes the number of timed launches and their
 * summed duration in milliseconds, and clears the record.  Not thread-safe.
 */
MOE_API moe_status moe_timing_enable(int32_t kind);
MOE_API moe_status moe_timing_read(int32_t *launches, double *total_ms);

/* Human-readable name of a status code (static string; never NULL). */
MOE_API const char *moe_status_str(int32_t status);

/* Text of the last validation failure on the calling thread ("" if none). */
MOE_API const char *moe_last_error(void);

/* ABI version: (major << 16) | minor.  Major 3: moe_linear.packed_scaled. */
MOE_API int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
