/*
 * pe.h — C ABI of the P-EAGLE parallel-drafting hot path on one AMD Instinct MI355X (gfx950).
 *
 * The method (source: "Parallelize speculative decoding with P-EAGLE on Amazon SageMaker AI", solution
 * overview: "how P-EAGLE breaks the chain" and "step-by-step drafting process"): for every request the
 * drafter builds K input rows in one go — row 0 from the token the target just produced and the hidden
 * states captured at three target layers, rows 1..K-1 from two learned placeholders (the shared hidden
 * state h_shared and the mask-token embedding emb_mask) — runs all K rows through its transformer layers
 * and LM head in a single forward pass, and emits K draft tokens at once. The target then checks the K
 * candidates in one verification pass with the standard acceptance rule (greedy form here).
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" point to GPU memory of the device that was current at pe_init; "host"
 *     pointers to CPU memory. The caller owns every buffer it passes; the library never frees them.
 *   - Matrices are row-major. A weight matrix W of a projection y = x . W^T is stored [out, in].
 *   - Device arrays of activations, caches and logits (target_hidden, rows, logits, target_logits and
 *     the KV cache) must be 16-byte aligned; calls reject other addresses with PE_ERR_INVALID.
 *   - Element type: pe_config.dtype (PE_F32 or PE_BF16) for weights, KV cache, target hiddens and target
 *     logits. Token ids, lengths and slots are int32. Logits written by the library are float32.
 *   - Calls enqueue work on the stream given to pe_init and return without waiting for the GPU.
 *     pe_draft_step, pe_draft_rows, pe_draft_ar, pe_draft_catchup, pe_verify and pe_verify_sampled
 *     allocate nothing.
 *   - A ctx is used by one host thread at a time. Calls on one ctx run in stream order.
 *   - Errors: every call returns a pe_status. Host-checkable problems (null pointers, sizes out of
 *     range, unsupported shapes) return PE_ERR_INVALID / PE_ERR_UNSUPPORTED before anything is enqueued.
 *     HIP failures return PE_ERR_HIP; pe_last_error gives the message. Device-value preconditions
 *     (token ids < vocab, slots < n_slots, seq_len + K + 1 <= max_ctx for pe_draft_step and pe_draft_ar, seq_len + K <=
 *     max_ctx for pe_draft_rows and pe_verify) are the caller's contract; kernels
 *     skip any access that would break them and raise a flag readable through pe_device_flags.
 */
#ifndef PE_H
#define PE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PE_MAX_LAYERS 8
#define PE_MAX_BATCH 1024
#define PE_MAX_K 16

typedef enum {
  PE_OK = 0,
  PE_ERR_INVALID = 1,     /* bad argument (null pointer, size out of range) */
  PE_ERR_UNSUPPORTED = 2, /* valid but not supported here (shape, dtype, device) */
  PE_ERR_OOM = 3,         /* workspace allocation failed in pe_init */
  PE_ERR_HIP = 4          /* a HIP runtime call failed; see pe_last_error */
} pe_status;

typedef enum { PE_F32 = 0, PE_BF16 = 1 } pe_dtype;

/* Drafter shape and capacity. */
typedef struct pe_config {
  int32_t n_layers;   /* transformer layers of the drafter, 1..PE_MAX_LAYERS (4 in practice) */
  int32_t d_model;    /* width d; multiple of 32 */
  int32_t n_q_heads;  /* Hq */
  int32_t n_kv_heads; /* Hkv; Hq % Hkv == 0 (grouped-query attention, q head h reads kv head h / (Hq/Hkv)) */
  int32_t head_dim;   /* hd; 64 or 128 */
  int32_t ffn_dim;    /* F of the SwiGLU MLP; multiple of 32 */
  int32_t vocab;      /* V */
  float rms_eps;      /* RMSNorm epsilon */
  float rope_base;    /* RoPE base (rotate-half pairs (i, i+hd/2), inv_freq_i = base^(-2i/hd)) */
  int32_t dtype;      /* pe_dtype */
  int32_t max_batch;  /* largest B passed to any call, 1..PE_MAX_BATCH */
  int32_t max_k;      /* largest K passed to any call, 1..PE_MAX_K */
  int32_t max_ctx;    /* positions per KV slot */
  int32_t n_slots;    /* KV slots */
  int32_t row_concat; /* 0: input rows are sums (embedding + hidden), width d. 1: rows are the concatenation
                         [embedding || hidden] (the pages' wording for positions 1..K): layer 0's attention
                         reads the 2d-wide row, RMSNorm applied to each half with its own gain (embed_norm
                         for the embedding, attn_norm[0] for the hidden), and the residual stream is the
                         hidden half; wqkv[0] is then [(Hq + 2 Hkv) hd, 2d]. bf16 drafters and pe_draft_step
                         only: caller rows, autoregressive drafting and catch-up steps return
                         PE_ERR_UNSUPPORTED on such a ctx. */
  int32_t weight_fp8; /* 0: bf16 projection weights. 1: FP8 drafter weights (the pages' deployment
                         precision): pe_init stores every projection matrix (fc, wqkv, wo, wgate, wup,
                         wdown, lm_head) as E4M3 codes of w / s_n (round to nearest even) with one float32
                         scale per output row, s_n = max_k |w[n][k]| / 448 (1 for a zero row); a product
                         is s_n * (codes . x) with bf16 activations and fp32 accumulation. bf16 drafters
                         and summed rows only. */
} pe_config;

/* Drafter weights (device, element type = dtype). Must stay valid and unchanged until pe_destroy:
 * pe_init copies the projection matrices into its own tiled layout, but reads embed, emb_mask,
 * h_shared and the norm gains in place on every step. */
typedef struct pe_weights {
  const void* fc;          /* [d, 3d]: projection of the three captured target hidden states */
  const void* embed;       /* [V, d]: token embedding */
  const void* emb_mask;    /* [d]: learned mask-token embedding (rows 1..K-1) */
  const void* h_shared;    /* [d]: learned shared hidden state (rows 1..K-1) */
  const void* final_norm;  /* [d]: RMSNorm gain before the LM head */
  const void* lm_head;     /* [V, d] */
  const void* attn_norm[PE_MAX_LAYERS]; /* [d] */
  const void* wqkv[PE_MAX_LAYERS];      /* [(Hq + 2 Hkv) hd, d]: q heads, then k heads, then v heads */
  const void* wo[PE_MAX_LAYERS];        /* [d, Hq hd] */
  const void* mlp_norm[PE_MAX_LAYERS];  /* [d] */
  const void* wgate[PE_MAX_LAYERS];     /* [F, d] */
  const void* wup[PE_MAX_LAYERS];       /* [F, d] */
  const void* wdown[PE_MAX_LAYERS];     /* [d, F] */
  const void* embed_norm;  /* [d]: RMSNorm gain of the embedding half (row_concat only, else ignored) */
} pe_weights;

/* Drafter KV cache (device, element type = dtype), one K and one V tensor per layer, each
 * [n_slots][Hkv][max_ctx][hd]. Keys are stored already rotated by RoPE. Owned by the caller. */
typedef struct pe_kv {
  void* k[PE_MAX_LAYERS];
  void* v[PE_MAX_LAYERS];
} pe_kv;

typedef struct pe_ctx pe_ctx;

/* Host-only check of a configuration; touches no GPU. */
pe_status pe_config_validate(const pe_config* cfg);

/* Create a context on the current HIP device (which must be gfx950): validates cfg, allocates the
 * workspace for max_batch x (max_k + 1) rows, copies the projection matrices into the library's tiled layout
 * and builds the RoPE table. stream: a hipStream_t (NULL = default stream). Synchronizes before return. */
pe_status pe_init(const pe_config* cfg, const pe_weights* w, const pe_kv* kv, void* stream, pe_ctx** out);

/* The parallel draft step (solution overview, step 2). For request b (0 <= b < B):
 *   row 0     = fc . concat(target_hidden[b]) + embed[last_token[b]]
 *   rows 1..K-1 = h_shared + emb_mask
 * (with row_concat: row 0 = [embed[last_token[b]] || fc . concat(target_hidden[b])], rows 1..K-1 =
 * [emb_mask || h_shared]) at positions seq_len[b] + j. All B*K rows go through the drafter layers (RMSNorm, GQA attention over
 * the request's cache slot with a causal mask inside the K block, SwiGLU MLP) and the LM head;
 * draft_tokens[b*K + j] = argmax over the vocabulary (lowest index among equal maxima).
 * One more placeholder row (h_shared + emb_mask at position seq_len[b] + K) runs after the K draft rows;
 * it changes none of them (causal mask) and only its K and V are kept: pe_verify can accept K + 1
 * tokens (seq_len advances by accept_len), and every position it keeps then holds drafter K/V.
 * The K and V of rows 0..K are written to cache slot req_slot[b] at positions seq_len[b]..+K;
 * seq_len itself is not changed.
 *   req_slot, seq_len, last_token: device int32 [B]
 *   target_hidden: device [B, 3d] (dtype); the three captured hidden states as consecutive d-blocks
 *   draft_tokens:  device int32 [B, K] (written)
 *   logits:        device float32 [B, K, V] or NULL; written when not NULL. */
pe_status pe_draft_step(pe_ctx* ctx, int32_t B, int32_t K, const int32_t* req_slot, const int32_t* seq_len,
                        const int32_t* last_token, const void* target_hidden, int32_t* draft_tokens,
                        float* logits);

/* Same drafter pass over caller-built input rows (device float32 [B, K, d]) instead of the row
 * builder: lets a caller feed arbitrary rows, e.g. to check that row j never depends on rows after j.
 * Exactly the K given rows run (no trailing placeholder row): K/V at positions seq_len[b]..+K-1. */
pe_status pe_draft_rows(pe_ctx* ctx, int32_t B, int32_t K, const int32_t* req_slot, const int32_t* seq_len,
                        const float* rows, int32_t* draft_tokens, float* logits);

/* Autoregressive EAGLE-style drafting on the same kernels: the sequential chain the parallel step
 * removes (solution overview, "sequential dependency in autoregressive EAGLE": every draft token needs
 * the previous pass's hidden state and token, so K tokens take K forward passes). bf16 drafters only.
 * Pass 0 runs one row per request, row 0 of pe_draft_step, at position seq_len[b]. Pass i = 1..K-1 runs
 * one row per request at position seq_len[b] + i: the drafter's residual stream after its last layer
 * (before the final norm) in pass i-1 plus embed[draft of pass i-1]; it attends to the context and to the
 * rows of passes 0..i-1. draft_tokens[b*K + i] = argmax of pass i. One more pass through the layers only
 * (input: hidden of pass K-1 + embed[draft K-1], position seq_len[b] + K) writes the K/V an all-accepted
 * verify keeps, so after the call the cache holds the same positions seq_len[b]..+K as after
 * pe_draft_step. Arguments, layouts and errors as pe_draft_step; a float32 drafter returns
 * PE_ERR_UNSUPPORTED. Allocates nothing. */
pe_status pe_draft_ar(pe_ctx* ctx, int32_t B, int32_t K, const int32_t* req_slot, const int32_t* seq_len,
                      const int32_t* last_token, const void* target_hidden, int32_t* draft_tokens, float* logits);

/* Multi-row catch-up step: a parallel draft step whose input starts with several real positions, so
 * that the drafter's K/V for the tokens a verify emitted come from the target's own hidden states.
 * (Solution overview, step-by-step drafting process: the pages' position 1 pairs the token just produced
 * with the target hidden states captured while producing it; here every emitted token gets such a row.
 * The pages do not describe this step; it is a reading.) bf16 drafters only.
 *   Request b runs R + K rows at positions seq_len[b] .. seq_len[b] + R + K - 1. Rows i < n_real[b] are
 *   real: fc(target_hidden[b][i]) + embed[tokens[b][i]]; every later row is the placeholder h_shared +
 *   emb_mask. draft_tokens[b*K + j] = argmax of row n_real[b] - 1 + j (the last real row predicts the
 *   next token). Rows after the drafted ones only fill cache positions the causal mask hides from them.
 *   With R = 1 this is pe_draft_step with tokens = last_token.
 *   R: 1 .. max_k + 1 - K (real rows per request in the arrays; R = K + 1 holds a fully accepted step)
 *   req_slot, seq_len (position of the first real row), n_real (1 .. R): device int32 [B]
 *   tokens: device int32 [B, R]   target_hidden: device [B, R, 3 * d_model] (dtype); entries past
 *   n_real[b] are ignored   draft_tokens: device int32 [B, K]   logits: device float32 [B, K, V] or NULL
 *   Device contract: seq_len[b] + R + K <= max_ctx; an n_real outside 1..R is clamped into it.
 *   A float32 drafter returns PE_ERR_UNSUPPORTED. Allocates nothing. */
pe_status pe_draft_catchup(pe_ctx* ctx, int32_t B, int32_t K, int32_t R, const int32_t* req_slot,
                           const int32_t* seq_len, const int32_t* n_real, const int32_t* tokens,
                           const void* target_hidden, int32_t* draft_tokens, float* logits);

/* Greedy verification and batch-metadata rebuild (solution overview, step 2, last sentence; batch
 * metadata as in the pages' fused metadata kernels). With t[b][i] = argmax_v target_logits[b][i][v]
 * (lowest index on ties) for i = 0..K:
 *   n_b = first i < K with draft_tokens[b][i] != t[b][i], or K;   accept_len[b] = n_b + 1
 *   cu_accept[0] = 0, cu_accept[b+1] = cu_accept[b] + accept_len[b]
 *   out_tokens[cu_accept[b] + i] = t[b][i] for i <= n_b   (accepted drafts, then the bonus token)
 *   requests with finished[b] == 0 survive, in order: keep_index[0..n_keep-1] lists them and
 *   req_slot_next[i] = req_slot[keep_index[i]], seq_len_next[i] = seq_len[keep_index[i]] +
 *   accept_len[keep_index[i]], last_token_next[i] = t[keep_index[i]][n_{keep_index[i]}] (the bonus).
 *   target_logits: device [B, K+1, V] (dtype)      draft_tokens: device int32 [B, K]
 *   finished: device uint8 [B] or NULL (none finished)
 *   req_slot, seq_len: device int32 [B]
 *   outputs (device int32): accept_len [B], cu_accept [B+1], out_tokens [B*(K+1)] (first cu_accept[B]
 *   valid), keep_index [B], n_keep [1], req_slot_next / seq_len_next / last_token_next [B] (first
 *   n_keep valid). Output buffers must not alias inputs. */
pe_status pe_verify(pe_ctx* ctx, int32_t B, int32_t K, const void* target_logits, const int32_t* draft_tokens,
                    const uint8_t* finished, const int32_t* req_slot, const int32_t* seq_len,
                    int32_t* accept_len, int32_t* cu_accept, int32_t* out_tokens, int32_t* keep_index,
                    int32_t* n_keep, int32_t* req_slot_next, int32_t* seq_len_next, int32_t* last_token_next);

/* Verification in its sampling form (temperature > 0; same section, the standard acceptance rule as
 * speculative sampling applies it). Reading: the parallel drafter drafts greedily, so its proposal is a
 * point mass at each draft token; the rule "accept x with probability min(1, p(x)/q(x)), else draw from
 * the normalised max(0, p - q)" then becomes, with p_i = softmax(target_logits[b][i] / temperature):
 *   draft_tokens[b][i] is accepted iff u[b][i] < p_i(draft_tokens[b][i]), for i = 0, 1, ... in order;
 *   at the first rejection n the emitted token is drawn with v[b][n] from p_n without the draft token;
 *   after K acceptances the bonus token is drawn with v[b][K] from p_K;
 *   a draw with uniform w from weights q returns the smallest x with q_0 + ... + q_x > w (q_0 + ... + q_V-1).
 * Every emitted token is then distributed as the target's p_i. Outputs exactly as pe_verify (the emitted
 * token after the accepted drafts takes the bonus token's place). u: device float32 [B, K], v: device
 * float32 [B, K+1], uniforms in [0, 1) drawn by the caller. Decisions and draws are computed in float32,
 * so a uniform within float32 rounding of a decision boundary may go either way. vocab must be a
 * multiple of 8. Allocates nothing. */
pe_status pe_verify_sampled(pe_ctx* ctx, int32_t B, int32_t K, const void* target_logits,
                            const int32_t* draft_tokens, float temperature, const float* u, const float* v,
                            const uint8_t* finished, const int32_t* req_slot, const int32_t* seq_len,
                            int32_t* accept_len, int32_t* cu_accept, int32_t* out_tokens, int32_t* keep_index,
                            int32_t* n_keep, int32_t* req_slot_next, int32_t* seq_len_next,
                            int32_t* last_token_next);

/* Greedy verification exactly as pe_verify (same inputs, outputs, contract and results), without a ctx and
 * without allocating anything. For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Its scratch memory (the vocabulary
 * argmax partials and the per-position target tokens) is a static array inside the library, one per GPU,
 * PE_VERIFY_STATIC_SCRATCH_BYTES (256 KiB) in size; the first call on a device looks up that device's copy
 * (the device current at the call, which must be gfx950), later calls reuse it. Every call on one GPU
 * shares that array, so calls that overlap on one GPU (two streams, or two host threads) race and must be
 * serialised by the caller; consecutive calls in one stream are safe (nothing in the array needs to start
 * at zero). vocab: V, a positive multiple of 8; dtype: element type of target_logits (a pe_dtype value:
 * PE_F32 or PE_BF16, passed as int32_t so that any other value is rejected rather than read as an enum);
 * 1 <= B <= 1024, 1 <= K <= 16 (every such size fits the array; a size that would not is rejected with
 * PE_ERR_INVALID). stream: a hipStream_t (NULL = default stream). Errors before anything is enqueued
 * (PE_ERR_INVALID / PE_ERR_UNSUPPORTED / PE_ERR_HIP); pe_last_error(NULL) gives the message. */
#define PE_VERIFY_STATIC_SCRATCH_BYTES (256 * 1024)
pe_status pe_verify_static(int32_t B, int32_t K, int32_t vocab, int32_t dtype, const void* target_logits,
                           const int32_t* draft_tokens, const uint8_t* finished, const int32_t* req_slot,
                           const int32_t* seq_len, int32_t* accept_len, int32_t* cu_accept, int32_t* out_tokens,
                           int32_t* keep_index, int32_t* n_keep, int32_t* req_slot_next, int32_t* seq_len_next,
                           int32_t* last_token_next, void* stream);

/* Waits for the ctx's stream, then frees everything pe_init allocated. NULL is allowed. */
pe_status pe_destroy(pe_ctx* ctx);

/* Device flags raised by kernels that skipped an access breaking a device-value precondition
 * (bit 0: token id out of range, bit 1: slot out of range, bit 2: position beyond max_ctx).
 * Synchronizes the stream; clear != 0 resets the flags. */
pe_status pe_device_flags(pe_ctx* ctx, int32_t clear, int32_t* flags);

/* Per-launch timing of selected kernels with HIP events recorded on the ctx's stream around each launch.
 * pe_profile_enable(ctx, mask) synchronizes, resets the totals and records the kernels whose bit
 * (1 << pe_prof_kernel) is set in mask (0 stops recording); pe_profile_read synchronizes and returns the
 * summed duration in milliseconds and the number of recorded launches of one kernel. */
typedef enum {
  PE_PROF_LM_HEAD = 0,     /* LM-head GEMM with fused argmax partials */
  PE_PROF_ATTENTION = 1,   /* attention: every kernel of it, the split merge included (every layer) */
  PE_PROF_GATE_UP = 2,     /* MLP gate/up GEMM with SwiGLU (every layer) */
  PE_PROF_VERIFY_SCAN = 3, /* verify's vocabulary argmax scan */
  PE_PROF_QKV = 4,         /* QKV GEMM with RoPE and KV append (every layer) */
  PE_PROF_O_PROJ = 5,      /* attention output projection + residual (every layer) */
  PE_PROF_DOWN = 6,        /* MLP down projection + residual (every layer) */
  PE_PROF_ROWS = 7,        /* input-row build (fc projection + embeddings) */
  PE_PROF_COUNT = 8
} pe_prof_kernel;
pe_status pe_profile_enable(pe_ctx* ctx, int32_t mask);
pe_status pe_profile_read(pe_ctx* ctx, int32_t which, double* total_ms, int64_t* launches);

const char* pe_status_string(pe_status s);
/* Message of the last failed call on ctx (or of the last failed pe_init when ctx is NULL). */
const char* pe_last_error(const pe_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif /* PE_H */
