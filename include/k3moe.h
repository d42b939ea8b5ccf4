/*
 * k3moe.h — C ABI of the routed-expert MXFP4 MoE layer for MI355X (gfx950).
 *
 * The layer is the Kimi-K3 routed-expert FFN: each token's latent activation is
 * routed by sigmoid scores plus a per-expert bias to the top-k experts; every
 * expert is a SiLU-gated MLP whose three matrices are stored as MXFP4 (4-bit
 * E2M1 codes in 32-element blocks, one E8M0 exponent per block) in 17-byte ggml
 * blocks; the expert outputs are summed with the gate weights.
 *
 * General conventions (all entry points):
 *   - Array pointers are DEVICE pointers unless stated otherwise. The caller
 *     allocates and owns every buffer; no entry point allocates device memory
 *     or synchronizes the host. The library's state: moe_mxfp4_ffn's
 *     per-thread side stream (below) and moe_mxfp4_ffn_noalloc's fixed
 *     scratch array, one per device.
 *   - `stream` is a hipStream_t (NULL = the default stream) of the current
 *     device, which also holds every buffer passed. Every call only enqueues
 *     work on it and returns; results are ready when the stream is.
 *   - Arrays are row-major and contiguous. Inputs are never written. Outputs
 *     are fully overwritten (never accumulated into).
 *   - Every argument check runs on the host before anything is enqueued; a
 *     failing check returns a negative k3moe_status and enqueues nothing. The
 *     library never aborts the process. Device pointers must be 16-byte
 *     aligned (K3MOE_ERR_ALIGN otherwise).
 *   - Calls are reentrant; calls on different streams may run concurrently as
 *     long as their output/workspace buffers are distinct.
 */
#ifndef K3MOE_H
#define K3MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  K3MOE_OK = 0,
  K3MOE_ERR_NULL = -1,        /* a required pointer is NULL */
  K3MOE_ERR_SHAPE = -2,       /* a size argument is out of range or inconsistent */
  K3MOE_ERR_ALIGN = -3,       /* a device pointer is not 16-byte aligned */
  K3MOE_ERR_WORKSPACE = -4,   /* workspace smaller than moe_mxfp4_ffn_workspace_size() */
  K3MOE_ERR_UNSUPPORTED = -5, /* unknown enum value (activation, output dtype) */
  K3MOE_ERR_DEVICE = -6,      /* the HIP runtime refused a launch (e.g. no gfx950 device) */
  K3MOE_ERR_TOO_LARGE = -7    /* moe_mxfp4_ffn_noalloc: the sizes need more than its fixed scratch */
} k3moe_status;

/* Largest top-k the router and FFN accept. */
#define K3MOE_MAX_TOPK 64
/* Largest expert count moe_mxfp4_ffn accepts (its grouping keeps one 64-bit
   token bitmap per expert in LDS). moe_route_topk has no expert limit. */
#define K3MOE_MAX_EXPERTS_FFN 8192
/* Largest latent dim D and expert intermediate I moe_mxfp4_ffn accepts. */
#define K3MOE_MAX_DIM_FFN 65536

/* Activation hook ids ("situ" is named but not defined by the sources; the
   only hook provided is SiLU(gate) * up). */
#define K3MOE_ACT_SILU_MUL 0

/* Output dtypes of mxfp4_dequant. */
#define K3MOE_DTYPE_F32 0
#define K3MOE_DTYPE_BF16 1

/* Human-readable name of a status code (static string, never NULL). */
const char* k3moe_status_str(int status);

/*
 * moe_route_topk — sigmoid + bias top-k routing.
 * Source: llama.cpp pull request "model: add Kimi-K3 text model", review
 * comment on the converter dry run (expert count 896, experts used 16, expert
 * score gating function sigmoid, per-expert bias tensor exp_probs_b).
 *
 *   logits  f32 [T, E]   router logits z
 *   bias    f32 [E]      per-expert selection bias b, or NULL for zero
 *   topk_ids i32 [T, k]  out: selected experts, best first
 *   topk_w   f32 [T, k]  out: gate weights, aligned with topk_ids
 *
 * Score s[t,e] = 1/(1+exp(-z[t,e])) + b[e], evaluated in fp64; a NaN score
 * ranks below every number. Experts are taken in order of decreasing score,
 * the lower index first among equal scores. The gate weight of a selected
 * expert is its sigmoid(z) (the bias only steers selection), divided by the
 * sum over the k selected when `normalize` != 0, then times `route_scale`,
 * rounded once to f32.
 * Sizes: T >= 0 (T == 0 is a no-op), 1 <= k <= min(E, K3MOE_MAX_TOPK), E >= 1
 * (no upper limit). K3MOE_ERR_SHAPE otherwise.
 */
int moe_route_topk(const float* logits, const float* bias, int64_t T, int32_t E, int32_t k,
                   int32_t normalize, float route_scale, int32_t* topk_ids, float* topk_w,
                   void* stream);

/*
 * mxfp4_repack — compressed-tensors MXFP4 -> 17-byte ggml blocks (lossless).
 * Source: llama.cpp pull request "model: add Kimi-K3 text model", review
 * comment "repack_mxfp4_blocks is bit-exact — 0 mismatches over 11,010,048
 * values" (reference-side and ggml-side layouts, byte accounting).
 *
 *   packed  u8 [R, K/2]       element 2i of a row in the low nibble of byte i,
 *                             element 2i+1 in the high nibble
 *   scale   u8 [R, K/32]      E8M0 exponent of each 32-element block
 *   blocks  u8 [R, K/32, 17]  out: byte 0 = the exponent byte unchanged,
 *                             byte 1+j = code(j) | code(j+16) << 4
 *
 * Every 4-bit code and every exponent byte is copied unchanged, only moved;
 * with ggml's doubled value table and halved scale the represented values
 * are unchanged. Sizes: R >= 0 (R == 0 is a no-op), K > 0 and K % 32 == 0.
 */
int mxfp4_repack(const uint8_t* packed, const uint8_t* scale, int64_t R, int64_t K, uint8_t* blocks,
                 void* stream);

/*
 * mxfp4_tile — reorder MXFP4 matrices from ggml row order into the stage-tiled
 * order that moe_mxfp4_ffn, its variants, moe_expert_cache_route and
 * moe_latent_block read. A pure permutation of whole 17-byte blocks (the block
 * encoding is the one mxfp4_repack writes, from the same review comment); the
 * order itself is this library's own: it makes every 16-row x 512-column
 * piece of a matrix one contiguous run, so the kernels that stream weights
 * read memory front to back.
 *
 *   src  u8 [nmat, N, K/32, 17]  matrices in ggml row order (row r, block b at
 *                                block index r * K/32 + b)
 *   dst  u8 [nmat, N, K/32, 17]  out: the same blocks, stage-tiled
 *
 * Stage-tiled order of one N x nb matrix (nb = K/32): rows in groups of 16,
 * a group's blocks in stages of 16 (the last group and the last stage may be
 * shorter); groups one after another, a group stage by stage, a stage row by
 * row, a row's blocks in order. Block b of row r sits at block index
 *   16*G*nb + 16*s*rG + (r % 16)*wS + (b % 16),
 * G = r / 16, s = b / 16, rG = min(16, N - 16*G), wS = min(16, nb - 16*s).
 * mxfp4_dequant decodes blocks in storage order, so on tiled data its output
 * rows are permuted the same way. Sizes: nmat >= 0 (0 is a no-op), N >= 1,
 * K > 0, K % 32 == 0, at most 2^31 - 1 pieces of 16 x 16 blocks in all.
 * src and dst must not overlap (K3MOE_ERR_SHAPE).
 */
int mxfp4_tile(const uint8_t* src, int64_t nmat, int64_t N, int64_t K, uint8_t* dst, void* stream);

/*
 * mxfp4_dequant — decode 17-byte ggml MXFP4 blocks.
 * Source: same review comment (ggml-side decode: dequantize_row_mxfp4 with
 * kvalues_fp4 = doubled E2M1 values and the half scale 2^(x-128), whose bits
 * are (x-1) << 23 for x >= 2).
 *
 *   blocks  u8 [R, K/32, 17]
 *   out     [R, K] f32 (out_dtype K3MOE_DTYPE_F32) or bf16 (K3MOE_DTYPE_BF16)
 *
 * Element j of a block is kvalues[low nibble of byte 1+j] * 2^(x-128), element
 * j+16 uses the high nibble. The product is exact: x = 0 and 1 give fp32
 * subnormals, large x overflow to +-inf, the zero codes give +0. Every finite
 * value is also exact in bf16. Sizes: R >= 0, K > 0, K % 32 == 0.
 * Unknown out_dtype -> K3MOE_ERR_UNSUPPORTED.
 */
int mxfp4_dequant(const uint8_t* blocks, int64_t R, int64_t K, int32_t out_dtype, void* out, void* stream);

/*
 * moe_mxfp4_ffn_workspace_size — bytes of device workspace moe_mxfp4_ffn needs
 * for these sizes (0 when T == 0). Pure host computation.
 */
size_t moe_mxfp4_ffn_workspace_size(int64_t T, int32_t D, int32_t I, int32_t E, int32_t k);

/*
 * moe_mxfp4_ffn — the routed-expert FFN with MXFP4 expert weights.
 * Sources: llama.cpp pull request "model: add Kimi-K3 text model": opening
 * comment (latent MoE: routed experts run at the latent width; the "situ"
 * activation), the dry-run comment (each expert is a w1 | w2 | w3 group), the
 * repack comment (w1 of one expert is logical [3072, 3584]; ggml block layout);
 * and the LLAMA_MAX_EXPERTS comment (build_moe_ffn: route -> per-expert
 * products -> weighted sum).
 *
 *   x_bf16   bf16 [T, D]        latent activations
 *   topk_ids i32  [T, k]        routed experts of each token
 *   topk_w   f32  [T, k]        gate weights
 *   w1, w3   u8 [E, I, D/32, 17] gate / up matrices ([I, D] per expert,
 *                               blocks along D) as ggml MXFP4 blocks in the
 *                               stage-tiled order of mxfp4_tile
 *   w2       u8 [E, D, I/32, 17] down matrix ([D, I] per expert), likewise
 *   out      f32  [T, D]        out[t] = sum_j w[t,j] * W2 act(W1 x_t, W3 x_t)
 *   workspace device buffer of at least moe_mxfp4_ffn_workspace_size() bytes;
 *             its contents on entry do not matter and are clobbered
 *
 * act must be K3MOE_ACT_SILU_MUL: act(g, u) = g * sigmoid(g) * u.
 * Precision: bf16 x and exact weights, MFMA with fp32 accumulation; h =
 * act(g, u) is formed in fp32 and enters the down product either as the bf16
 * pair hi = bf16(h), lo = bf16(h - hi) (about 16 significant bits; experts with
 * few rows, and shapes outside the large-tile kernels) or, for experts served
 * by the large-tile kernels (D and I multiples of 512, I <= 16384), as fp16
 * scaled by a power of two per (row, 256-wide slice of I) (11 significant
 * bits), and those experts' outputs before the weighted sum are held as fp16
 * scaled per (row, 32 outputs) (about 3e-4 relative L2 error on K3-shaped
 * inputs in all); fp32 output.
 * The k expert outputs of a token are summed in slot order (deterministic, no
 * atomics).
 * Large batches run as consecutive chunks of tokens that reuse one workspace
 * (at most (2^31 - 1) / (2 * k * max(D, I)) tokens each, rounded down to a
 * multiple of 64: the GEMM kernels address activations with 32-bit offsets);
 * moe_mxfp4_ffn_workspace_size() is that of one chunk.
 * Side stream: when one call has experts for both GEMM kinds (many rows: the
 * large-tile kernels; at most 16 rows: the weight-streaming kernels), the
 * streaming launches run on a side stream forked from `stream` with an event
 * and joined back before the combine (a graph captured from `stream` gets two
 * parallel branches). The side stream (default priority) and its two events
 * belong to the calling host thread and the current device; they are created
 * by the thread's first such call made outside a graph capture (until then
 * the launches stay on `stream`) and destroyed when the thread exits (those of
 * the process's main thread are kept until the process ends). A side stream
 * that is part of an open capture (an earlier call of the thread during that
 * capture forked it) is used only by calls captured into that same capture;
 * the thread's other calls meanwhile launch everything on `stream`.
 * Entry (t, j) is skipped (contributes nothing, whatever its weight) when
 * topk_ids[t,j] is outside [0, E) or repeats an id earlier in the same row.
 * Sizes: T >= 0 (T == 0 is a no-op), D > 0 and I > 0 multiples of 32 and at
 * most K3MOE_MAX_DIM_FFN, 1 <= k <= min(E, K3MOE_MAX_TOPK),
 * 1 <= E <= K3MOE_MAX_EXPERTS_FFN, T * k < 2^31.
 * E8M0 exponent bytes of the weights must be <= 254 (255 is not supported).
 */
int moe_mxfp4_ffn(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1,
                  const uint8_t* w3, const uint8_t* w2, int64_t T, int32_t D, int32_t I, int32_t E, int32_t k,
                  int32_t act, float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_mxfp4_ffn_profiled — moe_mxfp4_ffn that also records caller-created
 * hipEvent_t handles on `stream` at its stage boundaries, for timing the
 * stages on the stream they run on (the layer's arithmetic is identical).
 *
 *   stage_events  host array of K3MOE_FFN_STAGE_EVENTS hipEvent_t (each may be
 *                 NULL to skip it): [0] before grouping, [1] before the gate/up
 *                 product's large-tile (or small-tile) launch, [2] before its
 *                 weight-streaming launch, [3] before the down product's
 *                 large-tile (or small-tile) launch, [4] before its
 *                 weight-streaming launch, [5] before the combine, [6] after
 *                 the combine. A stage the batch does not need leaves two
 *                 consecutive events with nothing between them. NULL array =
 *                 plain moe_mxfp4_ffn. With several token chunks every chunk
 *                 records the events, so they end up bounding the last chunk.
 *
 * Same arguments, checks and results as moe_mxfp4_ffn, except that every
 * launch stays on `stream` (no side stream, so the events bound each
 * launch); an event the runtime refuses to record gives K3MOE_ERR_DEVICE.
 */
#define K3MOE_FFN_STAGE_EVENTS 7
int moe_mxfp4_ffn_profiled(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1,
                           const uint8_t* w3, const uint8_t* w2, int64_t T, int32_t D, int32_t I, int32_t E,
                           int32_t k, int32_t act, float* out, void* workspace, size_t workspace_bytes,
                           void* stream, void* const* stage_events);

/*
 * moe_q4k_ffn_workspace_size — bytes of device workspace moe_q4k_ffn needs for
 * these sizes (0 when T == 0 or the sizes are invalid). Pure host computation.
 */
size_t moe_q4k_ffn_workspace_size(int64_t T, int32_t D, int32_t I, int32_t E, int32_t k);

/*
 * moe_q4k_ffn — the same routed-expert FFN as moe_mxfp4_ffn with the experts
 * stored as Q4_K blocks. Sources: the pages run K3 requantized (Hugging Face
 * card "K3-Stuff", scripts list: a trunk rewritten from Q8_0 to Q4_K;
 * llama.cpp page "model: add Kimi-K3 text model", a Q3_K_M deployment;
 * lucebox page, "Runtime validation": a UD-IQ1_S target) and warn that the
 * QAT-trained MXFP4 experts should stay as they are ("K3-Stuff", Key facts);
 * they name Q4_K without defining it, so the block is ggml's published
 * block_q4_K:
 *   256 consecutive weights of a row in 144 bytes: fp16 d (bytes 0-1), fp16
 *   dmin (2-3), 12 bytes (4-15) packing eight 6-bit (scale, min) pairs, one
 *   per 32-weight sub-block (sub-block j < 4: scale = b[j] & 63, min =
 *   b[j+4] & 63; j >= 4: scale = (b[j+4] & 15) | (b[j-4] >> 6) << 4, min =
 *   (b[j+4] >> 4) | (b[j] >> 6) << 4, b = those 12 bytes), and 128 bytes of
 *   4-bit codes (code bytes 32c..32c+31 hold sub-block 2c in their low and
 *   2c+1 in their high nibbles); weight = d * scale * code - dmin * min.
 *
 *   x_bf16   bf16 [T, D]            latent activations
 *   topk_ids i32  [T, k]            routed experts of each token
 *   topk_w   f32  [T, k]            gate weights
 *   w1, w3   u8 [E, I, D/256, 144]  gate / up matrices ([I, D] per expert), Q4_K
 *                                   blocks along D, in ggml's row-major order
 *                                   (no repacking)
 *   w2       u8 [E, D, I/256, 144]  down matrix ([D, I] per expert), likewise
 *   out      f32  [T, D]            out[t] = sum_j w[t,j] * W2 act(W1 x_t, W3 x_t)
 *   workspace device buffer of at least moe_q4k_ffn_workspace_size() bytes;
 *             its contents on entry do not matter and are clobbered
 *
 * act must be K3MOE_ACT_SILU_MUL. Precision: bf16 x and exact weights, bf16
 * MFMA on the exact codes with fp32 accumulation and the block's scales and
 * mins applied in fp32; h enters the down product as the bf16 pair hi =
 * bf16(h), lo = bf16(h - hi); fp32 output. The k expert outputs of a token
 * are summed in slot order (deterministic); skipped entries as in
 * moe_mxfp4_ffn. Every launch stays on `stream`; the library keeps no state.
 * Sizes: as moe_mxfp4_ffn, with D and I multiples of 256 (else
 * K3MOE_ERR_SHAPE). Large batches run in the same token chunks as
 * moe_mxfp4_ffn. Non-finite d or dmin give non-finite outputs.
 */
int moe_q4k_ffn(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1,
                const uint8_t* w3, const uint8_t* w2, int64_t T, int32_t D, int32_t I, int32_t E, int32_t k,
                int32_t act, float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_q4k_ffn_profiled — moe_q4k_ffn recording caller-created hipEvent_t
 * handles at its launch boundaries, in the slots of moe_mxfp4_ffn_profiled:
 * [0] before grouping, [1] before the gate/up product, [3] before the down
 * product, [5] before the combine, [6] after it ([2] and [4], the streaming
 * slots, follow [1] and [3] with nothing between). Same arguments, checks and
 * results as moe_q4k_ffn; an event the runtime refuses to record gives
 * K3MOE_ERR_DEVICE.
 */
int moe_q4k_ffn_profiled(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1,
                         const uint8_t* w3, const uint8_t* w2, int64_t T, int32_t D, int32_t I, int32_t E, int32_t k,
                         int32_t act, float* out, void* workspace, size_t workspace_bytes, void* stream,
                         void* const* stage_events);

/*
 * moe_mxfp4_ffn_noalloc — moe_mxfp4_ffn for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the workspace is a fixed scratch array inside the
 * library, so the caller passes only inputs and outputs.
 *
 * Same arguments (without workspace), checks and results as moe_mxfp4_ffn;
 * every launch stays on `stream` (no side stream). The scratch holds
 * K3MOE_NOALLOC_SCRATCH_BYTES on every device the library runs on, from the
 * first use there until the process ends; sizes whose
 * moe_mxfp4_ffn_workspace_size() exceeds it give K3MOE_ERR_TOO_LARGE and
 * enqueue nothing (K3 shape: up to 128 tokens at k = 16). The call calls no
 * allocating routine; its first call on a device looks up the array's
 * device address (K3MOE_ERR_DEVICE if the runtime refuses).
 * All calls on one device share its one array: calls that overlap on a
 * device (different streams, or host threads, without ordering between
 * them) race on it and give undefined results. Nothing in the array needs
 * to start at a known value.
 */
#define K3MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_mxfp4_ffn_noalloc(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1,
                          const uint8_t* w3, const uint8_t* w2, int64_t T, int32_t D, int32_t I, int32_t E,
                          int32_t k, int32_t act, float* out, void* stream);

/*
 * moe_group_workspace_size — bytes of device workspace moe_group_by_expert
 * needs (0 when T == 0 or the sizes are out of range). Pure host computation.
 */
size_t moe_group_workspace_size(int64_t T, int32_t E, int32_t k);

/*
 * moe_group_by_expert — the grouping step that moe_mxfp4_ffn runs before its
 * products, as a call of its own: the routed entries sorted by expert.
 * Source: llama.cpp pull request "model: add Kimi-K3 text model",
 * LLAMA_MAX_EXPERTS comment (build_moe_ffn runs every expert on the tokens
 * routed to it; the expert count is a run-time size, not a compile-time cap).
 *
 *   topk_ids i32 [T, k]   routed experts; entry q = t*k + j
 *   counts   i32 [E]      out: valid entries per expert
 *   offsets  i32 [E + 1]  out: exclusive prefix sum of counts; offsets[E] = n,
 *                         the number of valid entries
 *   row_tok  i32 [T * k]  out: token of grouped row r for r < n, rows ordered
 *                         by (expert, token, slot); entries from n on are left
 *                         as they were
 *   slot_row i32 [T * k]  out: grouped row of entry q, or -1 if q is skipped
 *   workspace device buffer of at least moe_group_workspace_size() bytes;
 *             its contents on entry do not matter and are clobbered
 *
 * Entry q is skipped when its id is outside [0, E) or repeats an id earlier in
 * the same row (the rule moe_mxfp4_ffn applies). Integer work only; the result
 * does not depend on thread timing.
 * Sizes: T >= 0 (T == 0 is a no-op: nothing is written), 1 <= k <=
 * K3MOE_MAX_TOPK, 1 <= E <= K3MOE_MAX_EXPERTS_FFN, T * k < 2^31;
 * K3MOE_ERR_SHAPE otherwise. Every pointer must be 16-byte aligned.
 */
int moe_group_by_expert(const int32_t* topk_ids, int64_t T, int32_t E, int32_t k, int32_t* counts, int32_t* offsets,
                        int32_t* row_tok, int32_t* slot_row, void* workspace, size_t workspace_bytes, void* stream);

/* Largest verify width (rows per sequence) of the verify-width calls. */
#define K3MOE_MAX_VERIFY_WIDTH 64

/*
 * moe_verify_width_distinct — distinct routed experts of a speculative verify
 * batch, for every verify width at once.
 * Source: lucebox pull request "feat(kimi-k3): add DSpark Q8 artifact and
 * shared speculative runtime": Summary (target cost hints so that
 * external-memory targets avoid over-verification), "Kimi-K3 DSpark workload
 * probe" (expert traffic scales with every verified row) and "DSpark
 * acceptance-contract correction" (verification is the current token plus 7
 * proposals: width 8).
 *
 *   topk_ids  i32 [S * W, k]  routed experts of the batch's rows; row
 *                             r = s * W + w is position w (0 = the current
 *                             token, 1.. = the proposals) of sequence s
 *   distinct  i32 [W]         out: distinct[w] = number of distinct ids in
 *                             [0, E) routed by the rows of position <= w of
 *                             all S sequences
 *
 * A verify pass of width w (positions 0 .. w-1 of every sequence) streams
 * distinct[w-1] experts' weights once through the FFN. Ids outside [0, E) and
 * repeats add nothing. Integer result, independent of thread timing.
 * Sizes: S >= 0 (S == 0 writes zeros), 1 <= W <= K3MOE_MAX_VERIFY_WIDTH,
 * 1 <= E <= K3MOE_MAX_EXPERTS_FFN, 1 <= k <= K3MOE_MAX_TOPK, S * W * k < 2^31.
 */
int moe_verify_width_distinct(const int32_t* topk_ids, int32_t S, int32_t W, int32_t E, int32_t k, int32_t* distinct,
                              void* stream);

/*
 * moe_verify_width_choose — the verify width a cost hint picks (HOST call:
 * every pointer is host memory; nothing is enqueued).
 * Source: as moe_verify_width_distinct (cost hints; adaptive verification
 * reduced the streamed expert payload from 73.4 to 47.4 GiB).
 *
 *   distinct      i32 [W]      distinct experts by width (host copy of
 *                              moe_verify_width_distinct's output)
 *   accept        f64 [W - 1]  accept[j-1] = probability that proposal j is
 *                              accepted given that the ones before it were, or
 *                              NULL for all ones
 *   expert_bytes  bytes of one expert's weights (17,547,264 at K3 shape)
 *   bytes_per_s   rate at which those bytes reach the GPU (HBM, or the host
 *                 link for streamed experts)
 *   fixed_s       time of a pass that moves no expert bytes
 *   best_w        out: the width in 1 .. W with the highest rate (the
 *                 smallest one among equal rates)
 *   rates         out (optional, NULL to skip) f64 [W]: expected committed
 *                 tokens per second of every width
 *
 * A pass of width w commits, per sequence, the target's next token plus the
 * accepted prefix of its w - 1 proposals, 1 + sum_{i<w} prod_{j<=i} accept[j-1]
 * tokens in expectation, and takes fixed_s + distinct[w-1] * expert_bytes /
 * bytes_per_s seconds; rate = S * committed / time.
 * K3MOE_ERR_SHAPE for W outside 1 .. K3MOE_MAX_VERIFY_WIDTH, S < 1,
 * bytes_per_s <= 0, expert_bytes or fixed_s < 0; K3MOE_ERR_NULL for a missing
 * required pointer.
 */
int moe_verify_width_choose(const int32_t* distinct, int32_t W, int32_t S, const double* accept, double expert_bytes,
                            double bytes_per_s, double fixed_s, int32_t* best_w, double* rates);

/*
 * Device expert cache — routed experts kept in an external store (any memory
 * the GPU can read: pinned, mapped host memory, or device memory) and staged
 * on demand into C expert slots in HBM.
 * Sources: Hugging Face card "K3-Stuff", llama-cpp-patches item 2 (experts
 * paged in on demand; the page cache is the hot-expert cache, with LRU
 * eviction); lucebox pull request "feat(kimi-k3): add DSpark Q8 artifact and
 * shared speculative runtime", "Runtime validation" (SSD-routed experts
 * behind an 8 GiB device expert cache).
 *
 * Policy (least recently used): a batch uses the distinct ids in [0, E) of
 * its entries; used experts already in a slot are hits; the i-th miss (in
 * increasing expert order) takes the i-th slot, in least-recently-used order,
 * that no hit holds (empty slots come first), evicting what it held; the slots
 * the batch did not touch keep their order, then come the hit slots (old
 * order), then the filled slots (miss order). At init every slot is empty,
 * listed 0 .. C-1.
 *
 * The state is a caller-allocated device buffer of
 * moe_expert_cache_state_size(E, C) bytes: this header, then i32 slot_of[E]
 * (slot of each expert, -1: not cached), i32 expert_in[C] (expert in each
 * slot, -1: empty), i32 order[C] (slots from least to most recently used) and
 * i32 fetch[2 * C] (the last batch's (expert, slot) pairs, n_fetch of them),
 * each starting on a 256-byte boundary.  The caller may copy it to the host
 * to read the counters or the tables; only init and route write it.
 */
typedef struct {
  uint32_t step;          /* batches routed since init */
  uint32_t n_fetch;       /* experts the last batch fetched (its misses) */
  uint32_t hits;          /* used experts of the last batch found cached */
  uint32_t misses;        /* = n_fetch */
  uint64_t hits_total;    /* since init */
  uint64_t misses_total;  /* since init */
  int32_t E, C;           /* sizes given at init */
  uint32_t tag;           /* K3MOE_EXPERT_CACHE_TAG once initialised */
  uint32_t reserved;
} k3moe_expert_cache_header;
#define K3MOE_EXPERT_CACHE_TAG 0x4B334543u

/* Bytes of cache state for E experts and C slots (0 if out of range:
   1 <= E, C <= K3MOE_MAX_EXPERTS_FFN). Pure host computation. */
size_t moe_expert_cache_state_size(int32_t E, int32_t C);

/* Empty cache: every slot empty, LRU order 0 .. C-1, counters zero.
   K3MOE_ERR_SHAPE / _NULL / _ALIGN / _WORKSPACE (state too small). */
int moe_expert_cache_init(void* state, size_t state_bytes, int32_t E, int32_t C, void* stream);

/*
 * moe_expert_cache_route — stage a routed batch's experts into the cache.
 *
 *   state      the cache state (same E and C as at init)
 *   topk_ids   i32 [T, k]   routed experts of the batch
 *   slot_ids   i32 [T, k]   out: the slot of each entry's expert (entries whose
 *                           id is outside [0, E) get -1); pass it with
 *                           cache_w1/w3/w2 and E = C to moe_mxfp4_ffn, which
 *                           then computes exactly what it computes on the
 *                           store's experts with topk_ids
 *   store_w1, store_w3 u8 [E, I, D/32, 17], store_w2 u8 [E, D, I/32, 17]
 *                           all experts (pinned host memory, or device
 *                           memory), stage-tiled as moe_mxfp4_ffn reads them
 *                           (whole experts are copied unchanged)
 *   cache_w1, cache_w3 u8 [C, I, D/32, 17], cache_w2 u8 [C, D, I/32, 17]
 *                           device: the slots
 *
 * Two launches on `stream`: a one-workgroup plan (the policy above; it
 * writes slot_ids, the fetch list and the header) and a copy of every missed
 * expert's three matrices from the store into its slot (GPU loads from the
 * store: over the host link for host memory). Nothing waits for the host.
 * A state whose header does not carry the tag, E and C of an init with these
 * sizes is left untouched: every slot_ids entry becomes -1 and nothing is
 * fetched (so the FFN then contributes nothing).
 * The store pointers must be device memory or pinned host memory the GPU can
 * map (checked with hipPointerGetAttributes: K3MOE_ERR_UNSUPPORTED for memory
 * the GPU cannot read, such as pageable host memory).
 * Sizes: T >= 0 (T == 0 is a no-op), 1 <= k <= K3MOE_MAX_TOPK, D and I as for
 * moe_mxfp4_ffn, C >= min(E, T * k) (any batch fits), 1 <= E, C <=
 * K3MOE_MAX_EXPERTS_FFN; K3MOE_ERR_SHAPE otherwise.
 */
int moe_expert_cache_route(void* state, size_t state_bytes, int32_t E, int32_t C, const int32_t* topk_ids, int64_t T,
                           int32_t k, int32_t* slot_ids, const uint8_t* store_w1, const uint8_t* store_w3,
                           const uint8_t* store_w2, uint8_t* cache_w1, uint8_t* cache_w3, uint8_t* cache_w2, int32_t D,
                           int32_t I, void* stream);

/*
 * moe_expert_cache_route_q4k — moe_expert_cache_route for experts stored as
 * Q4_K blocks (the encoding moe_q4k_ffn reads): store_w1 / store_w3 u8
 * [E, I, D/256, 144], store_w2 u8 [E, D, I/256, 144], the slots likewise with
 * C; pass slot_ids and the slots to moe_q4k_ffn with E = C. Same state,
 * policy, launches, checks and results, with D and I multiples of 256
 * (K3MOE_ERR_SHAPE otherwise).
 */
int moe_expert_cache_route_q4k(void* state, size_t state_bytes, int32_t E, int32_t C, const int32_t* topk_ids,
                               int64_t T, int32_t k, int32_t* slot_ids, const uint8_t* store_w1,
                               const uint8_t* store_w3, const uint8_t* store_w2, uint8_t* cache_w1,
                               uint8_t* cache_w3, uint8_t* cache_w2, int32_t D, int32_t I, void* stream);

/*
 * moe_latent_block — the latent-MoE block around the routed experts.
 * Sources: llama.cpp pull request "model: add Kimi-K3 text model": opening
 * comment (latent MoE: routed experts run at a latent width), dry-run comment
 * (per-layer gate with exp_probs_b, ffn_routed_down, ffn_routed_norm and
 * ffn_routed_up beside the experts; hidden width 7168, 896 experts, 16 used,
 * sigmoid gating), review comment (shared-expert invariants). The pages give
 * no formula for the block; the reading this library computes, for hidden
 * rows h (bf16() = round to nearest even; every product takes bf16 operands
 * and sums in fp32):
 *
 *   z    = h Wg^T                          (router logits, fp32)
 *   ids, w = moe_route_topk(z, bias, k, normalize, route_scale)
 *   xl   = bf16(gamma * d / sqrt(mean(d^2) + eps)),  d = h Wd^T
 *   yl   = bf16(moe_mxfp4_ffn(xl, ids, w, w1, w3, w2))   (routed experts at width D)
 *   s    = bf16(SiLU(h Ws1^T) * (h Ws3^T))               (shared expert)
 *   out  = yl Wu^T + s Ws2^T
 *
 *   h        bf16 [T, H]         hidden rows
 *   wg       bf16 [E, H]         gate projection
 *   bias     f32 [E] or NULL     selection bias (NULL: zero)
 *   wd       bf16 [D, H]         ffn_routed_down
 *   gamma    bf16 [D]            ffn_routed_norm
 *   w1, w3, w2                   routed experts exactly as for moe_mxfp4_ffn
 *                                (E experts, latent width D, intermediate I)
 *   wu       bf16 [H, D]         ffn_routed_up
 *   ws1, ws3 bf16 [Is, H]        shared expert gate / up
 *   ws2      bf16 [H, Is]        shared expert down
 *   out      f32 [T, H]
 *   topk_ids i32 [T, k], topk_w f32 [T, k]: optional outputs of the routing
 *                                (NULL: kept in the workspace)
 *   workspace  moe_latent_block_workspace_size(T, H, D, I, Is, E, k) bytes
 *
 * Sizes: T >= 0 (T == 0 is a no-op), H a multiple of 128, D and Is multiples
 * of 64, I a multiple of 32, H, D, I, Is <= K3MOE_MAX_DIM_FFN, 1 <= k <=
 * min(E, K3MOE_MAX_TOPK), E <= K3MOE_MAX_EXPERTS_FFN, T * k < 2^31, eps >= 0
 * (K3MOE_ERR_SHAPE otherwise). Every pointer 16-byte aligned. Launches on
 * `stream` only (the routed FFN may fork to its side stream and joins back);
 * nothing synchronizes with the host; capturable in a graph.
 */
#define K3MOE_BLOCK_STAGE_EVENTS 7
size_t moe_latent_block_workspace_size(int64_t T, int32_t H, int32_t D, int32_t I, int32_t Is, int32_t E, int32_t k);
int moe_latent_block(const void* h_bf16, const void* wg, const float* bias, const void* wd, const void* gamma,
                     const uint8_t* w1, const uint8_t* w3, const uint8_t* w2, const void* wu, const void* ws1,
                     const void* ws3, const void* ws2, int64_t T, int32_t H, int32_t D, int32_t I, int32_t Is,
                     int32_t E, int32_t k, int32_t normalize, float route_scale, float eps, float* out,
                     int32_t* topk_ids, float* topk_w, void* workspace, size_t workspace_bytes, void* stream);
/* The same block with every launch on `stream` (the FFN's side stream is not
   used) and, when `events` is not NULL, K3MOE_BLOCK_STAGE_EVENTS caller-owned
   hipEvent_t recorded on `stream` before the first product, the epilogue
   after it (logits, latent norm, shared h), the routing, the routed FFN, the
   second product, the sum of its split-K partials (no launch when it has one
   split) and after the last launch (NULL entries are skipped). */
int moe_latent_block_profiled(const void* h_bf16, const void* wg, const float* bias, const void* wd, const void* gamma,
                              const uint8_t* w1, const uint8_t* w3, const uint8_t* w2, const void* wu,
                              const void* ws1, const void* ws3, const void* ws2, int64_t T, int32_t H, int32_t D,
                              int32_t I, int32_t Is, int32_t E, int32_t k, int32_t normalize, float route_scale,
                              float eps, float* out, int32_t* topk_ids, float* topk_w, void* workspace,
                              size_t workspace_bytes, void* stream, void* const* events);

#ifdef __cplusplus
}
#endif

#endif /* K3MOE_H */
