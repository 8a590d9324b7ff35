/*
 * dory.h -- C ABI of the MI355X (gfx950) forward pass of the looped
 * normalized-GPT described in "Dory1.0-4B: A Looped Normalized-GPT"
 * (paper body page).
 *
 * The model (sections Architecture and Training with Loops): an input block,
 * a recurrent block applied k times with every parameter shared across the k
 * invocations, and an output block. Each block is a sequence of sublayers,
 * attention-only or MLP-only. Every sublayer ends in the normalized
 * Transformer's residual update h <- N(h + alpha * (N(y) - h)), N being
 * per-token L2 normalization. Before each recurrent invocation the input
 * block's output x is added to the state and the sum normalized; the state
 * is replaced by the block's output and normalized again; the final state
 * feeds the output block and the LM head. Attention is grouped-query with an
 * input-dependent sigmoid gate on the head outputs; layers are
 * sliding-window or full attention in a 3:1 pattern, with RoPE bases and
 * window from section Long-Context Extension. Keys and values are cached per
 * loop or, with last-loop caching (section Last-Loop KV Caching), from the
 * final loop only so that the cache size does not depend on k.
 *
 * Conventions for every call below:
 *   - Device memory (weights, KV buffer, workspace, token ids, logits,
 *     hidden states) is allocated and owned by the caller. The library keeps
 *     only the pointers it is given and small host-side handles; it never
 *     allocates or frees device memory.
 *   - Matrices are row-major. "bf16" buffers hold bfloat16 bit patterns,
 *     weight matrices use the [out_features, in_features] layout.
 *   - All argument checks run on the host before anything is enqueued: on a
 *     non-OK status nothing was enqueued and the cache is unchanged.
 *   - Compute calls are asynchronous on the given HIP stream (a hipStream_t
 *     passed as void*; NULL = default stream); outputs are valid once that
 *     stream has been synchronized. A failed kernel launch returns
 *     DORY_ERR_HIP and marks the KV handle invalid until dory_kv_reset().
 *   - dory_last_error() returns a thread-local description of the last
 *     non-OK status returned on the calling thread.
 */
#ifndef DORY_H_
#define DORY_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dory_status {
  DORY_OK = 0,
  DORY_ERR_ARG = 1,          /* null pointer, k < 1, B or T <= 0, bad shape */
  DORY_ERR_MODE = 2,         /* cache-mode mismatch, or per-loop k rule */
  DORY_ERR_CAPACITY = 3,     /* cache length + T > max_seq, or B > bound batch */
  DORY_ERR_WORKSPACE = 4,    /* workspace too small */
  DORY_ERR_UNSUPPORTED = 5,  /* shape without a kernel (head_dim, widths) */
  DORY_ERR_HIP = 6,          /* a HIP launch failed */
  DORY_ERR_STATE = 7         /* KV handle invalid after a HIP failure */
} dory_status;

/* Cache policies of section Last-Loop KV Caching. */
typedef enum dory_cache_mode {
  DORY_CACHE_LAST_LOOP = 0, /* one cache per recurrent attention sublayer, holding the final loop's K/V */
  DORY_CACHE_PER_LOOP = 1   /* one cache per recurrent attention sublayer and loop */
} dory_cache_mode;

/* Sublayer kinds. Section Architecture: attention-only and MLP-only layers,
 * attention either sliding-window or full. */
typedef enum dory_layer_kind {
  DORY_LAYER_ATTN_SWA = 0,
  DORY_LAYER_ATTN_FULL = 1,
  DORY_LAYER_MLP = 2
} dory_layer_kind;

typedef struct dory_config {
  int32_t d_model;      /* d */
  int32_t n_q_heads;    /* query heads (16 in section Architecture) */
  int32_t n_kv_heads;   /* KV groups (4); n_q_heads % n_kv_heads == 0 */
  int32_t head_dim;     /* 32, 64 or 128 */
  int32_t d_ff;         /* SwiGLU width F */
  int32_t vocab;        /* V */
  int32_t n_input;      /* sublayers in the input block (16) */
  int32_t n_recurrent;  /* sublayers in the shared recurrent block (40) */
  int32_t n_output;     /* sublayers in the output block (16) */
  int32_t window;       /* sliding window W (1024): query p sees keys u with p - u < W */
  int32_t full_every;   /* default schedule: attention sublayer j is full iff j % full_every == full_every - 1 */
  int32_t has_lm_head;  /* 0: no LM head (logits unavailable) */
  double rope_base_swa;  /* 1e4 */
  double rope_base_full; /* 1e7 */
  double softmax_scale;  /* logit scale on q_hat.k_hat; <= 0 selects sqrt(head_dim) */
  /* Optional explicit schedule: n_input + n_recurrent + n_output entries of
   * dory_layer_kind. NULL: sublayers alternate attention and MLP starting
   * with attention, attention kinds by full_every. Copied at model creation. */
  const int32_t* layer_kinds;
  /* DORY_PRECISION_BF16 (0, the default): bf16 weights, K/V cache and
   * projection inputs, MFMA with fp32 accumulation, fp32 residual stream.
   * DORY_PRECISION_FP32 (1): fp32 debug build, every tensor (weights, K/V,
   * activations, logits) in fp32 on fp32 arithmetic, for checking the method
   * at a tighter tolerance; sized for small models; MXFP8, prefix copies,
   * the attention probes and decode graphs are bf16-build features. */
  int32_t precision;
} dory_config;

#define DORY_PRECISION_BF16 0
#define DORY_PRECISION_FP32 1

/* Device pointers of one sublayer. Attention sublayers use the first group,
 * MLP sublayers the second; alpha is used by both. */
/* Matrices below are bf16, or fp32 in the fp32 debug build (precision). */
typedef struct dory_sublayer_weights {
  const void* w_qkvg;   /* bf16 [2*d_q + 2*d_kv, d]: rows q (d_q = n_q*head_dim), k (d_kv), v (d_kv), gate (d_q) */
  const void* w_o;      /* bf16 [d, d_q] */
  const float* s_qk;    /* fp32 [head_dim]: scale applied to the normalized q and k heads */
  const void* w_upgate; /* bf16 [2*F, d]: rows up (F), then gate (F) */
  const void* w_down;   /* bf16 [d, F] */
  const float* s_u;     /* fp32 [F] */
  const float* s_v;     /* fp32 [F] */
  const float* alpha;   /* fp32 [d]: effective residual rate */
} dory_sublayer_weights;

typedef struct dory_weights {
  const void* embed;    /* bf16 [V, d] */
  const void* lm_head;  /* bf16 [V, d] (ignored without an LM head) */
  const float* s_z;     /* fp32 [V]: logit scale */
  const dory_sublayer_weights* sublayers; /* host array of n_input + n_recurrent + n_output; copied */
} dory_weights;

typedef struct dory_model dory_model;
typedef struct dory_kv dory_kv;

/* Location of one cache slot, for tests and tools. Entries are bf16 (fp32
 * in the fp32 debug build); keys of (b, g, position
 * u) live at k + ((b * n_kv + g) * rows + r(u)) * head_dim, values
 * transposed at v + ((b * n_kv + g) * head_dim + dim) * rows + r(u), with
 * r(u) = u mod ring when ring > 0 (sliding-window slots) and r(u) = u
 * otherwise. */
typedef struct dory_kv_slot_info {
  void* k;
  void* v;
  int64_t rows;
  int64_t ring;
} dory_kv_slot_info;

/* Validates the configuration and weight table and builds the host-side
 * schedule. Pointers are stored, not copied or dereferenced. */
dory_status dory_model_create(const dory_config* cfg, const dory_weights* w, dory_model** out);
void dory_model_destroy(dory_model* m);

/* Writes the kind of each sublayer (dory_layer_kind) into kinds_out, which
 * holds `capacity` entries. Schedule of section Architecture (27
 * sliding-window + 9 full + 36 MLP at the paper's 72 sublayers). */
dory_status dory_schedule(const dory_config* cfg, int32_t* kinds_out, int32_t capacity);

/* Bytes of KV storage for a cache bound with these parameters (closed form:
 * per attention sublayer, slots x batch x 2 x n_kv x head_dim x 2 bytes x
 * rows; recurrent sublayers hold k_max slots under per-loop caching and one
 * otherwise; sliding-window slots hold min(max_seq, window) rows, rounded up
 * to a multiple of 8, as a ring; full-attention slots hold max_seq rows
 * rounded up to a multiple of 8). Returns 0 on invalid arguments, including
 * a max_seq above the longest cache: 2^24 positions, and round8(max_seq) x
 * head_dim x 2 bytes below 2^32, i.e. at most 16,777,208 positions at
 * head_dim 128 (the attention kernels address one slab with 32-bit byte
 * offsets). */
size_t dory_kv_bytes(const dory_config* cfg, dory_cache_mode mode, int32_t k_max,
                     int32_t batch, int64_t max_seq);

/* Bytes of workspace needed by a call with B sequences of T tokens each
 * (decode: T = 1). Returns 0 on invalid arguments. */
size_t dory_workspace_bytes(const dory_config* cfg, int32_t batch, int32_t tokens);

/* Binds a caller-owned device buffer of at least dory_kv_bytes() bytes as
 * the KV cache of `batch` sequences of at most max_seq tokens, in `mode`;
 * lengths start at 0. A max_seq above the longest cache (see dory_kv_bytes)
 * returns DORY_ERR_ARG. */
dory_status dory_kv_bind(const dory_model* m, void* kv_dev, size_t kv_bytes, dory_cache_mode mode,
                         int32_t k_max, int32_t batch, int64_t max_seq, dory_kv** out);
void dory_kv_destroy(dory_kv* kv);
/* Forgets all cached tokens (length 0) and clears the invalid flag and the
 * loop count recorded for per-loop caching. Device memory is not touched. */
dory_status dory_kv_reset(dory_kv* kv);
/* Tokens cached per sequence, or -1 for a NULL handle. */
int64_t dory_kv_length(const dory_kv* kv);
/* Slot of a sublayer: loop is 0-based and only meaningful for recurrent
 * sublayers under per-loop caching. */
dory_status dory_kv_slot(const dory_kv* kv, int32_t sublayer, int32_t loop, dory_kv_slot_info* out);

/* One forward step over T new tokens per sequence at positions
 * L .. L + T - 1, where L = dory_kv_length(kv) (the same for all B rows).
 * Chunked prefill is a sequence of such calls.
 *   tokens: device int32 [B, T]; ids outside [0, V) produce NaN outputs.
 *   k >= 1: loop count (section Training with Loops). Under per-loop
 *     caching k <= k_max, and every earlier position must hold loop-k
 *     entries (written by a step with at least k loops, or declared by
 *     dory_kv_set_length): a step may use fewer loops than earlier ones,
 *     and its positions then hold only loops 1 .. k (DORY_ERR_MODE
 *     otherwise).
 *   mode: must equal the mode the cache was bound with.
 *   ws / ws_bytes: device workspace of at least dory_workspace_bytes(cfg, B, T).
 *   logits: device fp32 [B, V], logits of the last position, or NULL.
 *   next: device int32 [B], greedy token of the last position (argmax, lowest
 *     index on ties), or NULL. Needs an LM head.
 *   hidden: device fp32 [B, T, d], output of the last sublayer, or NULL.
 *   states: device fp32 [k, B, T, d], recurrent state after each loop
 *     (s_1 .. s_k), or NULL.
 * Cached keys must have been made with the layers' current s_qk (by this
 * model, or copied from a cache of it): the prefill attention bounds every
 * score by max |s_qk|^2 (section Architecture: q and k heads are s_qk times
 * unit vectors) and, when 2 max|s_qk|^2 scale log2(e) <= 120, uses that
 * bound as a fixed softmax reference instead of a running maximum.
 * On success the cache length grows by T. */
dory_status dory_prefill(dory_model* m, dory_kv* kv, const int32_t* tokens, int32_t B, int32_t T,
                         int32_t k, dory_cache_mode mode, void* ws, size_t ws_bytes,
                         float* logits, int32_t* next, float* hidden, float* states,
                         void* stream);

/* One decode step: one new token per sequence (tokens: device int32 [B]) at
 * position dory_kv_length(kv). Arguments as for dory_prefill with T = 1;
 * hidden is [B, d] and states [k, B, d]. The split-K decode attention
 * covers at most 1,048,576 keys: a step at a longer context returns
 * DORY_ERR_UNSUPPORTED before anything is enqueued (prefill chunks have no
 * such limit). Decode steps are replayed from captured HIP graphs (see
 * dory_model_set_decode_graphs). */
dory_status dory_decode_step(dory_model* m, dory_kv* kv, const int32_t* tokens, int32_t B,
                             int32_t k, dory_cache_mode mode, void* ws, size_t ws_bytes,
                             float* logits, int32_t* next, float* hidden, float* states,
                             void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): a decode
 * step like dory_decode_step, without a workspace argument. Its workspace is
 * a static device array of DORY_NOALLOC_SCRATCH_BYTES per GPU, created when
 * the library's code is loaded on that GPU and held until the process ends;
 * the call allocates nothing (no hipMalloc, no allocating library routine).
 * The scratch is laid out for exactly this step (split-K and split-attention
 * partials for its position), so that a batch of 64 sequences at 32,768
 * cached tokens fits; a step needing more returns DORY_ERR_WORKSPACE before
 * anything is enqueued. Nothing in the scratch needs to start at zero. Every
 * call on one GPU uses that GPU's single array: calls that overlap in time on
 * one GPU (other streams, other threads) race and must be serialized by the
 * caller. Other arguments, outputs and errors as for dory_decode_step. */
#define DORY_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
dory_status dory_decode_step_noalloc(dory_model* m, dory_kv* kv, const int32_t* tokens, int32_t B,
                                     int32_t k, dory_cache_mode mode, float* logits, int32_t* next,
                                     float* hidden, float* states, void* stream);

/* Steps whose sequences run different loop counts (one checkpoint served at
 * any loop count per request, section Introduction; rollouts of one batch
 * routed to different loop counts, section Post-Training, RLVR with a
 * difficulty-aware loop curriculum). k_rows: host int32 [B], each >= 1, read
 * before the call returns. Sequence b runs k_rows[b] loops of the recurrent
 * block and then the output block; the step executes max k_rows loops and a
 * sequence past its own count keeps its state (it is not updated, gets no
 * loop boundary and stores no K/V). Each sequence's K/V of the recurrent
 * attention sublayers is cached from its own last loop, so mode must be
 * DORY_CACHE_LAST_LOOP (else DORY_ERR_MODE); a model without a recurrent
 * block returns DORY_ERR_UNSUPPORTED. states[i] is written only for the
 * sequences with k_rows[b] > i. Results equal those of running each
 * sequence alone at its own loop count. Other arguments and errors as for
 * dory_prefill / dory_decode_step; the per-sequence counts are copied into
 * the workspace on the stream. */
dory_status dory_prefill_rows(dory_model* m, dory_kv* kv, const int32_t* tokens, int32_t B,
                              int32_t T, const int32_t* k_rows, dory_cache_mode mode, void* ws,
                              size_t ws_bytes, float* logits, int32_t* next, float* hidden,
                              float* states, void* stream);
dory_status dory_decode_step_rows(dory_model* m, dory_kv* kv, const int32_t* tokens, int32_t B,
                                  const int32_t* k_rows, dory_cache_mode mode, void* ws,
                                  size_t ws_bytes, float* logits, int32_t* next, float* hidden,
                                  float* states, void* stream);

/* Sets the number of cached positions of every sequence; the next step
 * starts at that position. 0 <= length <= max_seq. Shortening forgets the
 * positions past `length` (for example rejected speculative tokens);
 * lengthening declares that the new positions already hold valid K/V of
 * every loop (for example a cache restored by the caller). A
 * sliding-window sublayer's ring holds its window plus DORY_KV_ROLLBACK
 * positions, so where a ring is shorter than max_seq the cache can be
 * shortened to no less than (longest length written since the last reset
 * or copy) - DORY_KV_ROLLBACK; deeper returns DORY_ERR_ARG (the keys the
 * next step's window needs would have been overwritten). */
#define DORY_KV_ROLLBACK 64
dory_status dory_kv_set_length(dory_kv* kv, int64_t length);

/* Prefix caching (section Last-Loop KV Caching: serving reuses cached
 * prefixes). Copies the cached K/V of positions 0 .. n - 1 of sequence
 * src_seq of `src` into sequence dst_seq of `dst`, so that a prompt prefix
 * shared by several requests is computed once: the step after the copy
 * continues at position n exactly as if dst_seq had run the prefix itself
 * with the loop counts src_seq used. Both caches must be bound to the same
 * model and policy (DORY_ERR_ARG / DORY_ERR_MODE); 1 <= n <= length of src
 * (DORY_ERR_ARG); n <= max_seq of dst (DORY_ERR_CAPACITY). The length of dst
 * must be 0 or n (DORY_ERR_STATE) and becomes n: the call sets it for every
 * sequence of dst, so every sequence must receive a prefix of length n (or
 * the caller's own entries) before dst's next step. Sliding-window
 * sublayers copy the positions both rings hold (the last ring-size
 * positions). Per-loop caching: the loops copied are those whose entries
 * src holds for all n positions, up to dst's k_max; dst then holds only
 * the loops every copied sequence received, and a later step needs loop-k
 * entries as usual. src and dst may be the same cache (sequence to
 * sequence). Enqueued on `stream` (a hipStream_t, NULL for the default
 * stream); all checks happen before anything is enqueued. */
dory_status dory_kv_copy_prefix(const dory_kv* src, int32_t src_seq, dory_kv* dst, int32_t dst_seq,
                                int64_t n, void* stream);

/* One round of self-speculative greedy decoding (section Self-Speculative
 * Decoding: the same checkpoint drafts at a shallow loop count and verifies
 * at a deeper one in one batched pass over the drafted tokens). From the
 * tokens `last` (device int32 [B], not yet in the cache) at position
 * L = dory_kv_length(kv): gamma draft decode steps at k_draft, greedy; the
 * cache is rolled back to L; one verification step over the gamma + 1
 * tokens (last and the drafts) at k_verify, with the greedy token after
 * every position written to out (device int32 [gamma + 1][B]). Draft j is
 * accepted while it equals the verifier's token after position L + j - 1;
 * the batch keeps the n drafts accepted by every sequence (n_accepted, host
 * int32), the cache keeps positions up to L + n, and out rows 0 .. n are the
 * next n + 1 tokens of every sequence (row n, the verifier's own token after
 * the last accepted position, feeds the next round). With greedy selection
 * the emitted tokens are those of plain decoding at k_verify (sampled
 * decoding: dory_selfspec_step_sampled). Reuse of the drafts' input-block
 * and loop-1 activations in the verification pass is not implemented: the
 * verification recomputes them (with per-loop caching it rewrites the same
 * input-block and loop-1 entries). 1 <= gamma <= DORY_KV_ROLLBACK (the
 * cache is shortened by up to gamma positions). Per-loop caches only (as on the pages;
 * DORY_ERR_MODE otherwise): under last-loop caching the verification chunk
 * reads its own tokens' current-loop entries where token-by-token decoding
 * reads final-loop ones. scratch: device int32 of 2 B (gamma + 1)
 * elements. ws: at least dory_workspace_bytes(cfg, B, gamma + 1).
 * 1 <= k_draft <= k_verify <= k_max; needs an LM head. Synchronous: returns
 * after the round (n_accepted is read back). */
dory_status dory_selfspec_step(dory_model* m, dory_kv* kv, const int32_t* last, int32_t B,
                               int32_t gamma, int32_t k_draft, int32_t k_verify, dory_cache_mode mode,
                               void* ws, size_t ws_bytes, int32_t* scratch, int32_t* out,
                               int32_t* n_accepted, void* stream);

/* ---- Sampled decoding ---------------------------------------------------
 * Sampling by inversion (uniforms are inputs; nothing here draws random
 * numbers): out[r] (device int32 [rows]) = the smallest index i whose
 * cumulative weight exceeds u[r] times the row total, the weights being
 * softmax(logits[r] / temperature) (logits: device fp32 [rows][V], u:
 * device fp32 [rows] in [0, 1)); a token of zero probability is never
 * chosen (a row needs one finite logit; a row without gives token 0).
 * temperature > 0. Asynchronous on `stream`. */
dory_status dory_sample(const float* logits, int32_t rows, int32_t V, float temperature,
                        const float* u, int32_t* out, void* stream);

/* Rejection rule of self-speculative decoding (section Self-Speculative
 * Decoding: rejection sampling with both the drafter's and the verifier's
 * probabilities accepts proposals and corrects rejections, preserving the
 * verifier's sampling distribution). For each sequence b, with
 * q_j = softmax(draft_logits[j][b] / T) (j < gamma) and
 * p_j = softmax(verify_logits[j][b] / T) (j <= gamma): draft j
 * (drafts[j][b], sampled from q_j) is accepted while u[j][b] < p_j / q_j at
 * it; at the first rejection j the next token is sampled by inversion with
 * u[gamma][b] from max(0, p_j - q_j), and if all gamma drafts pass, from
 * p_gamma. Device buffers: draft_logits fp32 [gamma][B][V], verify_logits
 * fp32 [gamma + 1][B][V], drafts int32 [gamma][B], u fp32 [gamma + 1][B];
 * outputs n_accepted int32 [B] and out int32 [gamma + 1][B] (the accepted
 * drafts, then the next token, then -1). 1 <= gamma <= 1000. A rejection
 * whose residual has no mass in fp32 (p and q agree up to rounding; in
 * exact arithmetic a rejection implies positive residual mass) samples
 * from p_j instead. */
dory_status dory_speculative_accept(const float* draft_logits, const float* verify_logits,
                                    const int32_t* drafts, const float* u, int32_t B, int32_t V,
                                    int32_t gamma, float temperature, int32_t* n_accepted,
                                    int32_t* out, void* stream);

/* One self-speculative round with sampled decoding (section
 * Self-Speculative Decoding): gamma draft steps at k_draft, each sampling
 * its token from softmax(logits / temperature) with uniforms
 * u[0 .. gamma - 1][B]; the cache is rolled back; one verification step at
 * k_verify over the gamma + 1 tokens writes the logits after every
 * position; dory_speculative_accept with uniforms u[gamma .. 2 gamma][B]
 * decides each sequence's accepted count n_b and next token. The cache
 * keeps n = min over b of n_b drafts (one length per batch) and
 * *n_accepted (host) = n; out (device int32 [gamma + 1][B]) holds every
 * sequence's own accepted drafts and next token (dory_speculative_accept's
 * layout): rows 0 .. n are the next n + 1 tokens of every sequence (for a
 * sequence with n_b > n, row n is its accepted draft n + 1: a prefix of a
 * correctly distributed continuation is correctly distributed), and row n
 * feeds the next round. logits_buf: device fp32 [2 gamma + 1][B][V] (the
 * drafts' logits, then the verification's), scratch: device int32 of
 * 2 B (gamma + 1) elements, u: device fp32 [2 gamma + 1][B] in [0, 1).
 * 1 <= gamma <= DORY_KV_ROLLBACK, temperature > 0. Per-loop caches only;
 * other arguments and errors as for dory_selfspec_step. Synchronous (the
 * accepted counts are read back). */
dory_status dory_selfspec_step_sampled(dory_model* m, dory_kv* kv, const int32_t* last, int32_t B,
                                       int32_t gamma, int32_t k_draft, int32_t k_verify,
                                       dory_cache_mode mode, float temperature, const float* u,
                                       void* ws, size_t ws_bytes, int32_t* scratch,
                                       float* logits_buf, int32_t* out, int32_t* n_accepted,
                                       void* stream);

/* ---- MXFP8 weights (W8A16) ------------------------------------------------
 * Section Quantization (Post-Training Quantization): an MXFP8 checkpoint made
 * by post-training quantization with maximum scaling, weight-only, covering
 * every weight matrix but the token embeddings and the LM head; vectors and
 * scalars stay in full precision. Format: blocks of 32 consecutive elements
 * of a weight row share a scale 2^(c - 127) stored as the byte c; elements
 * are FP8 E4M3 codes (bias 7, 3 mantissa bits, largest finite 448). Scale
 * rule: the block's shared exponent is floor(log2(max |w|)) - 8, at least
 * -126; each w * 2^-shared is rounded to the nearest E4M3 value, ties to the
 * even code, saturating at 448, the sign of a zero kept.
 *
 * Quantizes one bf16 matrix [rows][cols] (row-major, cols a positive
 * multiple of 32): codes uint8 [rows][cols], scales uint8 [rows][cols / 32]
 * and, if deq is not NULL, the dequantized values as bf16 [rows][cols] (an
 * E4M3 value times a power of two is exact in bf16). Device pointers; w,
 * codes and deq 16-byte aligned; asynchronous on `stream`. */
dory_status dory_mxfp8_quantize(const void* w, int64_t rows, int32_t cols, void* codes,
                                void* scales, void* deq, void* stream);

/* Bytes of device memory that dory_model_quantize_mxfp8 needs: for every
 * projection matrix in sublayer order (attention: w_qkvg then w_o; MLP:
 * w_upgate then w_down) a region holding its codes, scales and bf16
 * dequantized copy, each part starting at a multiple of 256 bytes. Returns 0
 * on an invalid configuration. */
size_t dory_mxfp8_bytes(const dory_config* cfg);

/* Quantizes the model's projection matrices into the caller-owned device
 * buffer `buf` (256-byte aligned, at least dory_mxfp8_bytes() bytes; layout
 * as described there), asynchronously on `stream`, and enables them: from
 * then on every projection computes with the dequantized weights (W8A16).
 * Calls with at most 64 token rows (decode) stream the 8-bit codes through
 * the small-M kernel; larger calls read the bf16 dequantized copy. The
 * embedding and LM head stay bf16. The buffer must outlive the model's use
 * of it. DORY_ERR_CAPACITY if the buffer is too small. */
dory_status dory_model_quantize_mxfp8(dory_model* m, void* buf, size_t bytes, void* stream);

/* Decode-step graphs (on by default). A decode step at k loops is
 * 32 + 40k sublayer applications (section Training with Loops), hundreds of
 * short kernel launches; with graphs on, the first dory_decode_step with a
 * given cache, batch, loop count, policy, weight format, set of buffers
 * (tokens, workspace, outputs) and decode split size (one below and one
 * above 65,536 cached keys) is captured into a HIP graph on a library stream
 * and launched on the caller's stream, and later steps with the same
 * parameters replay it: the kernels read the step position from the
 * workspace, where the graph's first node writes it. Results are identical
 * to running the kernels directly. Steps are run directly (not captured)
 * while dory_profile_begin is active, when the caller's stream is itself
 * being captured, and when capture fails. Graphs of a cache are released by
 * dory_kv_destroy; on = 0 releases all of them. Calls on one model must not
 * overlap from several threads. */
dory_status dory_model_set_decode_graphs(dory_model* m, int32_t on);

/* Switches between the bf16 weights (on = 0) and the MXFP8 copy (on != 0,
 * only after dory_model_quantize_mxfp8; DORY_ERR_ARG otherwise). */
dory_status dory_model_use_mxfp8(dory_model* m, int32_t on);

/* Kernel classes timed by the measurement hooks below. */
typedef enum dory_kernel_class {
  DORY_K_GEMM_QKVG = 0,   /* q/k/v/gate projection */
  DORY_K_GEMM_O = 1,      /* attention output projection */
  DORY_K_GEMM_UPGATE = 2, /* SwiGLU up/gate projection (with the activation) */
  DORY_K_GEMM_DOWN = 3,   /* MLP down projection */
  DORY_K_GEMM_LM = 4,     /* LM head */
  DORY_K_ATTN = 5,        /* attention (prefill or decode, incl. split combine) */
  DORY_K_QK = 6,          /* RoPE / q-k norm / K-V placement */
  DORY_K_UPDATE = 7,      /* nGPT normalize-and-update (and loop boundary) */
  DORY_K_KV_WRITE = 8,    /* persistent cache store */
  DORY_K_OTHER = 9,       /* embedding, SwiGLU over partials, argmax, copies */
  DORY_K_NUM_CLASSES = 10
} dory_kernel_class;

/* Measurement hooks. Between dory_profile_begin and dory_profile_end, each
 * kernel launch of the model is bracketed by a pair of HIP events recorded
 * on the call's stream (at most max_launches launches are recorded; later
 * ones are not timed). dory_profile_end synchronizes those events and writes,
 * per dory_kernel_class, the number of timed launches and their summed
 * duration in milliseconds into counts[DORY_K_NUM_CLASSES] and
 * ms[DORY_K_NUM_CLASSES]. The events are host-side HIP objects; no device
 * memory is allocated. */
dory_status dory_profile_begin(dory_model* m, int32_t max_launches);
dory_status dory_profile_end(dory_model* m, int64_t* counts, double* ms);

/* Greedy selection (greedy decoding of the workload descriptions; reading:
 * the lowest index wins ties): out[r] = argmax over i < n of logits[r * n + i]
 * for each of `rows` rows. logits: device fp32 [rows, n]; out: device int32
 * [rows]. NaN entries never win; a row without a value above -inf yields 0.
 * The same kernel as the `next` output of the compute calls. Asynchronous on
 * `stream`. */
dory_status dory_greedy(const float* logits, int32_t rows, int32_t n, int32_t* out, void* stream);

/* ---- Debug probes of the production kernels (bit-exact tests) ------------
 * These run the attention kernels and index computations of the compute
 * calls on probe inputs; they exist so that tests can read the mask and the
 * cache rows those kernels actually use.
 *
 * Cache rows (section Last-Loop KV Caching; the ring of a sliding-window
 * slot): rows_out[i] (device int64 [n]) receives the row of position
 * pos_a + i in the slots of `sublayer`, evaluated on the device by the
 * function every cache-writing kernel uses (position mod ring for a
 * sliding-window slot, the position for a full-attention slot).
 * 0 <= pos_a, pos_a + n <= max_seq. */
dory_status dory_debug_kv_slots(const dory_kv* kv, int32_t sublayer, int64_t pos_a, int64_t n,
                                int64_t* rows_out, void* stream);

/* Runs the attention of attention sublayer `sublayer` (its kind: sliding
 * window or full, section Architecture; window of section Long-Context
 * Extension) exactly as a step over positions p0 .. p0 + T - 1 does, on the
 * caller's inputs: q_hat bf16 [B][n_q][T][head_dim] (already transformed),
 * the step's own keys k_new and values v_new bf16 [B][n_kv][T][head_dim], the
 * gate sigma(g) bf16 [B * T][n_q * head_dim]; z (bf16, same shape as the
 * gate) receives the gated attention output. B is the cache's bound batch.
 * Keys below p0 are read from the slot (`loop` selects it under per-loop
 * caching) as the step would read them: the caller writes them through
 * dory_kv_slot() in its layout. T = 1 runs the decode kernels (the token's
 * K/V are first stored in the slot, as a decode step stores them); T > 1 the
 * prefill kernels (the slot is not written). The cache length is not used or
 * changed; p0 + T <= max_seq. ws: at least dory_workspace_bytes(cfg, B, T). */
dory_status dory_debug_attention(dory_model* m, dory_kv* kv, int32_t sublayer, int32_t loop,
                                 int64_t p0, int32_t T, const void* q_hat, const void* k_new,
                                 const void* v_new, const void* gate, void* z, void* ws,
                                 size_t ws_bytes, void* stream);

/* Mask dump (bit-exact tests): out (device uint16 [B][n_q][T][p0 + T])
 * receives the weight, as a bf16 bit pattern, that the attention kernels of
 * `sublayer` give key position u for the query at position p0 + t of query
 * head h when all scores are equal (zero queries and keys): 1 / (number of
 * visible keys) at the visible keys and 0 at the others, so its nonzero
 * pattern is the mask the kernels apply. It is read off the kernels'
 * outputs, with one-hot values probing head_dim keys at a time
 * (ceil((p0 + T) / head_dim) runs of the kernels of dory_debug_attention,
 * decode kernels for T = 1). Overwrites the contents of the slot (`loop`
 * under per-loop caching) and the workspace; the cache length is unchanged.
 * Arguments and errors as for dory_debug_attention. */
dory_status dory_debug_mask(dory_model* m, dory_kv* kv, int32_t sublayer, int32_t loop, int64_t p0,
                            int32_t T, void* ws, size_t ws_bytes, uint16_t* out, void* stream);

const char* dory_status_string(dory_status s);
const char* dory_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DORY_H_ */
