/*
 * peagle.h -- C ABI of the MI355X (gfx950) P-EAGLE parallel-drafter library.
 *
 * What the library computes (sources cited by page title and section):
 *   - "P-EAGLE: A Technical Deep Dive into Parallel Speculative Decoding",
 *     section "2. The P-EAGLE Parallel Drafter": one forward pass drafts K
 *     tokens.  The first (next-token) position takes the new token's
 *     embedding and the target's hidden state; positions 2..K take a shared
 *     mask-token embedding and a shared hidden state h_shared.
 *   - "P-EAGLE: Parallel-Drafting EAGLE with Scalable Training" (notes on
 *     arXiv:2602.01469), section 2: the inputs are the concatenated target
 *     hidden states of three layers; the block runs through N LLaMA-3 style
 *     decoder layers with RoPE and an LM head.  Section 3.1: the attention
 *     mask is precomputed once at the maximum length and sliced per sample.
 *   - "Speeding LLM inference with P-EAGLE in vLLM Speculators", sections
 *     "A learnable mask parameter" (mask_hidden is 3H wide) and
 *     "Flex-attention mask" (who may attend to whom).
 *   - "EAGLE-4" (lightseek.org), "EAGLE-4 overview": the verifier keeps the
 *     longest agreeing prefix plus one bonus token.
 *
 * Conventions shared by every entry point:
 *   - All pointers named *device* point to GPU memory owned by the caller;
 *     *host* pointers point to CPU memory read during the call only.
 *   - Matrices are row-major [out, in] (PyTorch nn.Linear layout): y = x W^T.
 *   - "dtype" data (weights, hidden states, caches, mask embedding) is bf16
 *     or fp32 as pe_config.dtype says; accumulation is always fp32.
 *   - Validation happens before any launch: a non-OK status means nothing
 *     was enqueued.  pe_last_error() returns a thread-local message.
 *   - Work is asynchronous on the given hipStream_t (NULL = default stream);
 *     the forward entry points never allocate, free or synchronise.
 *   - Device pointers must be 16-byte aligned.
 */
#ifndef PEAGLE_H
#define PEAGLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PE_OK = 0,
  PE_ERR_INVALID_ARGUMENT = -1, /* a NULL required pointer, a bad size or shape */
  PE_ERR_UNSUPPORTED = -2,      /* valid in principle, outside this build's limits */
  PE_ERR_WORKSPACE = -3,        /* workspace NULL or smaller than the size query says */
  PE_ERR_HIP = -4               /* a HIP runtime call or launch failed */
} pe_status;

typedef enum { PE_F32 = 0, PE_BF16 = 1 } pe_dtype;

/* Build limits. */
#define PE_K_MAX 16        /* draft block length K */
#define PE_DECODE_ROWS_MAX 64 /* B*K rows per draft forward; also B+1 <= 64 */

typedef struct {
  int32_t hidden;        /* H, multiple of 16 */
  int32_t n_layers;      /* decoder layers held by the model */
  int32_t n_q_heads;     /* query heads */
  int32_t n_kv_heads;    /* key/value heads; n_q_heads % n_kv_heads == 0 */
  int32_t head_dim;      /* 64 or 128 */
  int32_t intermediate;  /* SwiGLU width I, multiple of 8 */
  int32_t vocab;         /* V, multiple of 16 */
  float rope_theta;      /* RoPE base (500000 for LLaMA-3 style drafters) */
  float rms_eps;         /* RMSNorm epsilon (1e-5) */
  int32_t dtype;         /* pe_dtype of weights and activations */
} pe_config;

/* Device pointers of one decoder layer, all in pe_config.dtype. */
typedef struct {
  const void *attn_norm; /* [H] RMSNorm gain before attention */
  const void *wq;        /* [n_q_heads*head_dim, H] */
  const void *wk;        /* [n_kv_heads*head_dim, H] */
  const void *wv;        /* [n_kv_heads*head_dim, H] */
  const void *wo;        /* [H, n_q_heads*head_dim] */
  const void *mlp_norm;  /* [H] RMSNorm gain before the MLP */
  const void *w_gate;    /* [I, H] */
  const void *w_up;      /* [I, H] */
  const void *w_down;    /* [H, I] */
} pe_layer_weights;

typedef struct {
  const void *embed;       /* [V, H] token embedding; kept by reference, must outlive the model */
  const void *fc;          /* [H, 3H] projection of the concatenated target hidden states */
  const void *final_norm;  /* [H] RMSNorm gain before the LM head */
  const void *lm_head;     /* [V, H], untied from embed */
  const pe_layer_weights *layers; /* host array of n_layers entries */
} pe_weights;

typedef struct pe_model pe_model;
typedef struct pe_mask pe_mask;

/* Copy every weight except the embedding into the library's MFMA tile layout
 * (device memory owned by the model), convert norm gains to fp32 and build
 * the RoPE frequency table in fp64.  Synchronises the stream before
 * returning; the caller may free its weight copies afterwards (not embed). */
pe_status pe_model_create(const pe_config *cfg, const pe_weights *w, void *stream, pe_model **out);
pe_status pe_model_destroy(pe_model *m);

/* Workspace bytes needed by pe_draft_forward for B sequences, block K and
 * context stride ctx_stride.  The same workspace serves any smaller call. */
pe_status pe_draft_workspace_size(const pe_model *m, int32_t B, int32_t K, int64_t ctx_stride,
                                  size_t *bytes);

/* Host-only check, no device access: whether pe_draft_forward and
 * pe_draft_extend can run B sequences of block K over caches of stride
 * ctx_stride for this configuration on a device with num_cus compute units.
 * PE_ERR_UNSUPPORTED (with the reason in pe_last_error) when a projection's
 * contraction cannot be split into chunks whose activation fragments fit the
 * GEMM's registers, when one (sequence, kv head) cache slice of
 * ctx_stride * head_dim elements exceeds 2 GiB, or when B and K exceed the
 * build limits; pe_draft_workspace_size, pe_draft_forward and
 * pe_draft_extend return the same status for such shapes. */
pe_status pe_draft_shape_check(const pe_config *cfg, int32_t B, int32_t K, int64_t ctx_stride,
                               int32_t num_cus);

/* Zero a workspace (device, ws_bytes) on the stream with a fill kernel (no
 * memset node, so it may sit in a captured graph).  Required once before a
 * workspace's first use: it holds arrival counters and argmax keys that must
 * start at zero, and every completed call leaves them at zero again.  After
 * a call that failed on the device, initialise the workspace again. */
pe_status pe_workspace_init(void *workspace, size_t ws_bytes, void *stream);

/*
 * One parallel-drafting forward ("2. The P-EAGLE Parallel Drafter").
 *
 *   N           layers to run, 0..n_layers (0 = fusion, final norm, LM head)
 *   B, K        sequences and block length; 1 <= K <= PE_K_MAX,
 *               B*K <= PE_DECODE_ROWS_MAX, B + 1 <= PE_DECODE_ROWS_MAX
 *   hidden3     device [B, 3H]  concatenated target hidden states (low|mid|high)
 *   token_ids   device int32 [B] newly generated token of each sequence
 *   mask_emb    device [H]       mask-token embedding (e.g. row mask_token_id of embed)
 *   h_shared    device [3H]      shared hidden state (the learnable mask_hidden)
 *   ctx_lens    device int32 [B] cached context length C_b, 0 <= C_b <= ctx_stride
 *   ctx_stride  C_max, the cache's position stride
 *   k_cache, v_cache
 *               host arrays of N device pointers; entry l points at layer l's
 *               cache [B, n_kv_heads, ctx_stride, head_dim] (keys already
 *               rotated).  Block row k of sequence b sits at RoPE position
 *               C_b + k and attends to cache rows [0, C_b) and block rows 0..k.
 *               The cache is only read.
 *   draft_out   device int32 [B, K]: argmax of each position's logits, the
 *               lowest index among equal maxima
 *   logits_out  device fp32 [B, K, V] or NULL
 *   workspace   device, ws_bytes >= pe_draft_workspace_size(m, B, K, ctx_stride),
 *               initialised once by pe_workspace_init; calls that share a
 *               workspace must be ordered on one stream.
 */
pe_status pe_draft_forward(const pe_model *m, int32_t N, int32_t B, int32_t K,
                           const void *hidden3, const int32_t *token_ids,
                           const void *mask_emb, const void *h_shared,
                           const int32_t *ctx_lens, int64_t ctx_stride,
                           const void *const *k_cache, const void *const *v_cache,
                           int32_t *draft_out, float *logits_out,
                           void *workspace, size_t ws_bytes, void *stream);

/*
 * pe_draft_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The same kernels run on a scratch
 * array of PE_NOALLOC_SCRATCH_BYTES bytes that the library holds per device
 * in its own code object (there from module load until the process ends);
 * this call allocates and frees nothing.  The first call on a device looks
 * the array's address up and clears it with a fill kernel on `stream`.
 * Arguments, layouts and outputs as pe_draft_forward.  Errors as
 * pe_draft_forward; PE_ERR_UNSUPPORTED also when the shape needs more
 * scratch than the array holds (the message gives both sizes; the
 * workspace forward serves such shapes).  Every call on one device shares
 * that device's array: calls that may overlap in time on one device (other
 * streams, other threads) race on it and must be ordered by the caller.
 */
#define PE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pe_status pe_draft_forward_noalloc(const pe_model *m, int32_t N, int32_t B, int32_t K,
                                   const void *hidden3, const int32_t *token_ids,
                                   const void *mask_emb, const void *h_shared,
                                   const int32_t *ctx_lens, int64_t ctx_stride,
                                   const void *const *k_cache, const void *const *v_cache,
                                   int32_t *draft_out, float *logits_out, void *stream);

/*
 * Drafter-cache extension: T real rows per sequence ("Speeding LLM inference
 * with P-EAGLE in vLLM Speculators", "Flex-attention mask": depth-0
 * positions carry real tokens and real hidden states and attend causally to
 * each other).  Two uses:
 *   - after verification, the accepted tokens with their target hidden
 *     states become drafter context (input_kind PE_INPUT_TARGET);
 *   - the autoregressive EAGLE-3 drafter that P-EAGLE replaces ("P-EAGLE: A
 *     Technical Deep Dive into Parallel Speculative Decoding", "Technical
 *     Architecture: From Sequential to Parallel": K sequential passes for K
 *     tokens): step 0 takes the new token and the target's hidden state,
 *     step j > 0 takes step j-1's draft token and its final-norm output
 *     (input_kind PE_INPUT_DRAFTER; "EAGLE-4", "EAGLE-4 overview": the
 *     final-norm state of one step is the next step's input), with pos_offset = j.
 *
 *   N, B, T     layers (0..n_layers), sequences, rows per sequence;
 *               1 <= T <= PE_K_MAX, B*T <= PE_DECODE_ROWS_MAX
 *   inputs      device; PE_INPUT_TARGET: dtype [B, T, 3H] target hidden
 *               states (row input E[token] + fc(h));
 *               PE_INPUT_DRAFTER: fp32 [B, T, H] drafter states z (row
 *               input E[token] + z)
 *   token_ids   device int32 [B, T]
 *   ctx_lens, pos_offset, ctx_stride
 *               row t of sequence b sits at position P_b + t with
 *               P_b = min(ctx_lens[b] + pos_offset, ctx_stride); it attends to
 *               cache rows [0, P_b) and block rows 0..t
 *   k_cache, v_cache
 *               host arrays of N device pointers, layout as in
 *               pe_draft_forward.  Read at [0, P_b) and WRITTEN at
 *               [P_b, P_b + T): each row's rotated key and its value; rows at
 *               positions >= ctx_stride are not written (the caller keeps
 *               ctx_lens[b] + pos_offset + T <= ctx_stride)
 *   draft_out   device int32 [B, T] argmax per row, or NULL
 *   logits_out  device fp32 [B, T, V], or NULL (with draft_out NULL as well
 *               the LM head is skipped)
 *   z_out       device fp32 [B, T, H] final-norm output of each row, or NULL
 *   workspace   as for pe_draft_forward with K = T
 */
#define PE_INPUT_TARGET 0
#define PE_INPUT_DRAFTER 1
pe_status pe_draft_extend(const pe_model *m, int32_t N, int32_t B, int32_t T, const void *inputs,
                          int32_t input_kind, const int32_t *token_ids, const int32_t *ctx_lens,
                          int32_t pos_offset, int64_t ctx_stride, void *const *k_cache, void *const *v_cache,
                          int32_t *draft_out, float *logits_out, float *z_out, void *workspace, size_t ws_bytes,
                          void *stream);

/*
 * Greedy longest-prefix acceptance ("EAGLE-4", "EAGLE-4 overview";
 * "Speeding LLM inference with P-EAGLE in vLLM Speculators", introduction).
 *   draft       device int32 [B, K]
 *   target      device int32 [B, K+1]  the verifier's greedy token at each block
 *               position plus the one after the last
 *   accept_len  device int32 [B]: largest a <= K with draft[b,i] == target[b,i] for i < a
 *   out_tokens  device int32 [B, K+1] or NULL: target[b, 0..a] then -1
 * 1 <= K <= PE_K_MAX, B >= 0 (B == 0 enqueues nothing).
 */
pe_status pe_accept(int32_t B, int32_t K, const int32_t *draft, const int32_t *target,
                    int32_t *accept_len, int32_t *out_tokens, void *stream);

/* ------------------------------------------------------------------------
 * Training-shape forward ("P-EAGLE: A Technical Deep Dive into Parallel
 * Speculative Decoding", section "Memory and Training Complexity";
 * "P-EAGLE: Parallel-Drafting EAGLE with Scalable Training", sections 3,
 * 3.1 and 3.2; visibility rules from "Speeding LLM inference with P-EAGLE
 * in vLLM Speculators", section "Flex-attention mask").
 *
 * A sequence of n positions is expanded to the n x K grid of cells (p, d):
 * position p, depth d, anchor a = p - d, grid index r = p*K + d
 * (position-major).  COD sampling keeps a subset of cells; the kept grid
 * indices ("rows") are strictly ascending, contain every depth-0 cell, and
 * are chain-closed (a kept (p, d >= 1) has (p-1, d-1) kept).  Cell (p, d)
 * takes E[x_p] + fc(h_p) at depth 0 and mask_emb + fc(h_shared) deeper, sits
 * at RoPE position p, and attends to the depth-0 cells at positions <= a and
 * to the kept cells of its own rollout (a + j, j), 1 <= j <= d.
 * ---------------------------------------------------------------------- */

/* Amortized mask: built once for the longest sequence n_max, it holds for
 * every cell of the n_max x K grid the anchor and depth that define its mask
 * row.  A sample of n positions uses the top-left n*K cells (a slice, no
 * rebuilding), then gathers its kept cells. */
pe_status pe_mask_create(int32_t n_max, int32_t K, void *stream, pe_mask **out);
pe_status pe_mask_destroy(pe_mask *m);

/* Test and debugging aid: materialise the mask of kept rows `rows` (device
 * int32 [L]) of an n-position sample from the sliced table, as bytes
 * out[i*L + j] = 1 if kept row i may attend to kept row j (device uint8
 * [L, L]).  L <= 65536. */
pe_status pe_mask_materialize(const pe_mask *m, int32_t n, const int32_t *rows, int32_t L,
                              uint8_t *out, void *stream);

/* Workspace bytes of pe_train_forward for n positions, block K and L kept rows. */
pe_status pe_train_workspace_size(const pe_model *m, int32_t n, int32_t K, int32_t L, size_t *bytes);

/*
 * Forward of the first N layers over the L kept rows of one sequence.
 *   hidden3    device [n, 3H]   target hidden states of every position
 *   token_ids  device int32 [n] token at every position (out-of-range ids clamped)
 *   mask_emb   device [H], h_shared device [3H]
 *   rows       device int32 [L], kept grid indices as above (violations give
 *              unspecified values but every access stays in bounds)
 *   logits_out device [L, V] in the model dtype, or NULL
 *   argmax_out device int32 [L] (lowest index among equal maxima), or NULL
 * Requires n <= n_max, K equal to the mask's K, and hidden and intermediate
 * multiples of 32 (bf16) or 16 (fp32); PE_ERR_UNSUPPORTED otherwise.  Row i
 * of the outputs belongs to rows[i].
 */
pe_status pe_train_forward(const pe_model *m, const pe_mask *mask, int32_t N, int32_t n, int32_t K,
                           const void *hidden3, const int32_t *token_ids, const void *mask_emb,
                           const void *h_shared, const int32_t *rows, int32_t L, void *logits_out,
                           int32_t *argmax_out, void *workspace, size_t ws_bytes, void *stream);

/*
 * COD sampling on the host ("Speeding LLM inference with P-EAGLE in vLLM
 * Speculators", section "COD sampling"; paper notes, section 3): depth 0
 * keeps every position; a cell (p, d >= 1) with p >= d is kept when its
 * parent (p-1, d-1) is kept and U[p*K + d] < r_d, where
 * r_d = max(r^d, floor) / max(r^(d-1), floor), so depth d keeps a fraction
 * max(r^d, floor) of positions.  U: host double [n*K] uniforms in [0, 1).
 * rows_out: host int32 with room for n*K entries; *L_out receives the count.
 */
pe_status pe_cod_rows(int32_t n, int32_t K, double r, double floor_rate, const double *U,
                      int32_t *rows_out, int32_t *L_out);

/*
 * Sequence partition on the host (paper notes, section 3.2): S equal-width
 * position segments [floor(s n / S), floor((s+1) n / S)); depth-0 and
 * depth-1 cells go to the segment of their position, a deeper cell to the
 * chunk of its parent (p-1, d-1).  Chunk s is completed by every depth-0
 * cell before the end of segment s.  rows: host int32 [L] (kept rows as for
 * pe_train_forward); chunk_out: host int32 [L].
 */
pe_status pe_partition(int32_t n, int32_t K, int32_t S, const int32_t *rows, int32_t L,
                       int32_t *chunk_out);

/*
 * Cells of chunk s of that partition, the unit of a chunked training
 * forward (paper notes, section 3.2: each chunk is completed by the depth-0
 * cells before the end of its segment, so chunks share no state).
 *   rows       host int32 [L], kept cells of the whole sequence as for
 *              pe_train_forward (every depth-0 cell present)
 *   cells_out  host int32 with room for L entries: the chunk's cells,
 *              ascending; the first *n_lead (the depth-0 cells of positions
 *              before segment s) belong to earlier chunks
 *   out_rows   host int32 with room for L entries: for cell *n_lead + i,
 *              its index in rows
 *   *L_chunk   number of cells; *n_chunk positions the chunk covers (its
 *              largest position + 1): the chunk forward reads hidden3 and
 *              token_ids rows [0, *n_chunk) only
 * PE_ERR_INVALID_ARGUMENT as pe_partition, for s outside [0, S), or when a
 * depth-0 cell of a position before the end of segment s is missing.
 */
pe_status pe_partition_chunk(int32_t n, int32_t K, int32_t S, int32_t s, const int32_t *rows, int32_t L,
                             int32_t *cells_out, int32_t *out_rows, int32_t *L_chunk, int32_t *n_lead,
                             int32_t *n_chunk);

/*
 * Training-shape forward of one chunk (paper notes, section 3.2), run with
 * no state from other chunks: pe_train_forward over the chunk's L cells
 * (device int32 [L], from pe_partition_chunk, n = its n_chunk), writing
 * only the cells from n_lead on, each to row out_rows[i] (device int32
 * [L - n_lead]) of the whole sequence's outputs logits_out [L_out, V] and
 * argmax_out [L_out]; rows outside [0, L_out) are dropped.  Over all chunks
 * of a partition this writes every row of pe_train_forward's outputs with
 * the same values.  Workspace: pe_train_workspace_size(m, n, K, L).  cells
 * must contain the depth-0 cell of every position up to their largest
 * anchor and be chain-closed (violations give unspecified values but every
 * access stays in bounds).
 */
pe_status pe_train_forward_chunk(const pe_model *m, const pe_mask *mask, int32_t N, int32_t n, int32_t K,
                                 const void *hidden3, const int32_t *token_ids, const void *mask_emb,
                                 const void *h_shared, const int32_t *cells, int32_t L, int32_t n_lead,
                                 const int32_t *out_rows, int32_t L_out, void *logits_out, int32_t *argmax_out,
                                 void *workspace, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Training step: loss and gradients over a COD layout ("P-EAGLE: A
 * Technical Deep Dive into Parallel Speculative Decoding", section "Memory
 * and Training Complexity": the K-depth layout trains in one forward and
 * backward pass, gradients accumulated over the chunks of a sequence
 * partition; "P-EAGLE: Parallel-Drafting EAGLE with Scalable Training",
 * sections 3 and 3.2; learnable mask embedding, hidden state and embedding
 * table from "Speeding LLM inference with P-EAGLE in vLLM Speculators",
 * sections "A learnable mask parameter" and "Learnable embedding").
 *
 * Cell (p, d) drafts the token after position p: its loss is the
 * cross-entropy of its logits against labels[p] (negative: not scored).
 * Gradients are fp32, in the weights' own [out, in] row-major layouts, and
 * are ADDED to the caller's buffers, so calls over the chunks of a
 * partition (each with the whole sequence's loss_scale) accumulate the
 * whole sequence's gradients.
 * ---------------------------------------------------------------------- */
typedef struct {
  float *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *w_gate, *w_up, *w_down;  /* NULL: not wanted */
} pe_layer_grads;

typedef struct {
  float *fc;          /* [H, 3H] */
  float *final_norm;  /* [H] */
  float *lm_head;     /* [V, H] */
  float *mask_emb;    /* [H] */
  float *h_shared;    /* [3H] */
  float *embed_rows;  /* [n, H]: gradient of the embedding row looked up at position p (depth-0 cells); the
                         caller adds row p into its table's row token_ids[p] */
  const pe_layer_grads *layers;  /* host array [N] */
} pe_grads;

/* Builds the transposed weight tiles the backward's data gradients read,
 * from the same weights the model was created from (device, row-major).
 * Allocates once (about the size of the model's own tiles); later calls
 * return PE_OK at once. */
pe_status pe_model_prepare_backward(pe_model *m, const pe_weights *w, void *stream);

/* Workspace bytes of pe_train_step for N layers, n positions, block K and L cells. */
pe_status pe_train_step_workspace_size(const pe_model *m, int32_t N, int32_t n, int32_t K, int32_t L,
                                       size_t *bytes);

/*
 * Forward, loss and backward of the first N layers over L cells (device
 * int32 [L], as for pe_train_forward or pe_train_forward_chunk; n positions).
 * The first n_lead cells are not scored (a chunk's depth-0 completion from
 * earlier segments).  labels: device int32 [n].  *loss_out (device fp32, or
 * NULL) += loss_scale * the summed cross-entropy of the scored cells; every
 * non-NULL gradient pointer in grads receives += its gradient.  Needs
 * pe_model_prepare_backward, head_dim 64 (or 128 for bf16), at most 64 query
 * heads per kv head and hidden <= 4096.
 */
pe_status pe_train_step(const pe_model *m, const pe_mask *mask, int32_t N, int32_t n, int32_t K,
                        const void *hidden3, const int32_t *token_ids, const void *mask_emb, const void *h_shared,
                        const int32_t *cells, int32_t L, int32_t n_lead, const int32_t *labels, float loss_scale,
                        float *loss_out, const pe_grads *grads, void *workspace, size_t ws_bytes, void *stream);

/* Thread-local description of the last non-OK status of this thread. */
const char *pe_last_error(void);

/* Library build string (kernel set, arch). */
const char *pe_version(void);

/* Optional per-stage timing of pe_draft_forward: when enabled, the model
 * records HIP events around its LM-head launch on the forward's stream.
 * pe_profile_read synchronises on the last event and returns the number of
 * recorded launches and their mean duration in milliseconds, then clears.
 * The event slots belong to the model: while profiling is enabled, forwards
 * of that model must be issued from one host thread at a time (they may use
 * any stream).  With profiling disabled (the default) a model is only read
 * by the forward calls, and several threads and streams may share it. */
pe_status pe_profile_enable(pe_model *m, int32_t enable);
pe_status pe_profile_read(pe_model *m, int32_t *count, double *mean_ms);

#ifdef __cplusplus
}
#endif

#endif /* PEAGLE_H */
