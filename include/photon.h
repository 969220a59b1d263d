/*
 * photon.h -- C ABI of the PHOTON recursive-generation (RecGen) decode path
 * on one AMD Instinct MI355X (gfx950).
 *
 * The method: PHOTON paper record (ACL 2026 long paper "PHOTON: Hierarchical
 * Autoregressive Modeling for Lightspeed and Memory-Efficient Language
 * Generation"), abstract; PHOTON explainer (mokumoku.ipfde.com, Fujitsu
 * PHOTON vertical scan): module table (Context Chunker, Context Encoder,
 * Context Converter, Context Decoder), the recursive-generation section
 * (HierGen's three steps, RecGen's feedback of the bottleneck
 * reconstruction, Theorem A.6, dropping the lower encoder caches after
 * prefill, keeping only the decoders resident), and the decode-heavy table
 * (throughput per unit memory, TPM).
 *
 * Conventions shared by every entry point:
 *   - Every call returns a photon_status; no C++ exception crosses the ABI.
 *     photon_last_error() gives a thread-local detail string for the most
 *     recent failing call on this thread.
 *   - Every shape, capacity and state check happens on the host before any
 *     HIP call; a call that fails a check has no side effect.
 *   - Device pointers ("d_" prefix) are allocated and owned by the caller.
 *     The library owns only the small host-side photon_ctx (and the HIP
 *     graphs it may instantiate for it).
 *   - Work is enqueued on the caller's stream (a hipStream_t passed as void*;
 *     NULL is the null stream) and is asynchronous: no call synchronises.
 *     A launch failure returns PHOTON_EHIP; device faults surface at the
 *     caller's next synchronisation.
 *   - A photon_ctx is not thread safe; separate contexts are independent.
 *   - Token ids are int32 in [0, vocab).
 *
 * Shapes: L levels (2 <= L <= PHOTON_MAX_LEVELS); chunk = {C1, ..., CL}:
 * C_l states of level l-1 form one level-l state (level 0 = tokens, level L
 * = the top), so a level-l state covers span(l) = C1*...*C_l tokens and one
 * top state covers S = span(L) tokens (S = C1*C2 for two levels).  The
 * explainer's module table gives a chunker and an encoder per level on the
 * way up and a converter and a decoder per level on the way down, for any
 * depth; its main setting is L = 2.  d = d_model, H = n_heads, hd = d / H,
 * F = mlp_mult * d.  K1 = S / C1 is the number of level-1 states per chunk
 * (C2 for two levels).
 */
#ifndef PHOTON_H
#define PHOTON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PHOTON_OK = 0,
  PHOTON_EINVAL = -1,      /* null pointer, bad enum, misaligned buffer */
  PHOTON_ESHAPE = -2,      /* P % S != 0, P < S, batch < 1, d % H != 0 ... */
  PHOTON_ECAPACITY = -3,   /* workspace too small or max_tokens exceeded */
  PHOTON_ESTATE = -4,      /* decode before prefill, HierGen without the
                              prefill-only weights, ... */
  PHOTON_EUNSUPPORTED = -5,/* a shape this build does not handle */
  PHOTON_EHIP = -6         /* a HIP runtime call or launch failed */
} photon_status;

typedef enum { PHOTON_F32 = 0, PHOTON_BF16 = 1 } photon_dtype;

/* RecGen feeds the level-1 decoder's reconstruction A-hat straight to the
 * top encoder; HierGen re-encodes the emitted tokens bottom-up (explainer,
 * recursive-generation section). */
typedef enum { PHOTON_RECGEN = 0, PHOTON_HIERGEN = 1 } photon_mode;

#define PHOTON_MAX_LEVELS 4

typedef struct {
  int32_t n_levels;     /* L, 2 .. PHOTON_MAX_LEVELS */
  int32_t chunk[PHOTON_MAX_LEVELS];  /* C1 .. CL, each 1 .. 16 (entries past
                                        L are ignored) */
  int32_t d_model;
  int32_t n_heads;
  int32_t mlp_mult;     /* MLP width F = mlp_mult * d_model */
  int32_t vocab;
  int32_t n_top;        /* top (level-L) encoder layers */
  int32_t n_enc1;       /* level-1 encoder layers (prefill / HierGen only) */
  int32_t n_dec1;       /* level-1 decoder layers */
  int32_t n_dec0;       /* token decoder layers */
  int32_t dtype;        /* photon_dtype: storage of weights, K/V, operands */
  float norm_eps;       /* RMSNorm epsilon */
  float rope_theta;     /* rotary base */
  /* L > 2 only: layers of the level-l encoder (prefill / HierGen only) and
   * of the level-l decoder at entry l - 2, for l = 2 .. L-1 */
  int32_t n_enc_hi[PHOTON_MAX_LEVELS - 2];
  int32_t n_dec_hi[PHOTON_MAX_LEVELS - 2];
} photon_config;

/* ------------------------------------------------------------------------
 * Memory accounting (pure host, no device call).
 *
 * photon_kv_bytes: byte counts for `batch` sequences holding `tokens` tokens
 * in `mode` (explainer, decode-heavy table: TPM = throughput / memory; the
 * RecGen section: only the top-level global KV is kept, the level-1 encoder
 * cache is dropped after prefill; the module table: the decoder's cache is
 * confined to the chunk and does not grow with the context).
 *
 * The workspace that photon_prefill/photon_decode_chunk use is laid out for
 * a capacity of `tokens` tokens: call with tokens = max_tokens to size it.
 * ---------------------------------------------------------------------- */
typedef struct {
  int64_t top_len;            /* ceil(tokens / S) top states per sequence */
  int64_t lower_len;          /* ceil(tokens / C1) level-1 states (HierGen) */
  uint64_t top_kv;            /* n_top*2*batch*top_len*d*elem bytes */
  uint64_t lower_kv;          /* HierGen: the sum over encoder levels l < L of
                                 layers*2*batch*ceil(tokens/span(l))*d*elem;
                                 RecGen 0 */
  uint64_t dec_kv;            /* n_dec0*2*batch*S*d*elem (K1 groups of C1
                                 slots per sequence), independent of tokens */
  uint64_t state;             /* h_{i-1}, positions, argmax keys, counters */
  uint64_t decode_scratch;    /* activations of one decode chunk */
  uint64_t workspace_total;   /* bytes the workspace must hold (256-aligned) */
  uint64_t weights_decode;    /* decode-resident weight blob */
  uint64_t weights_prefill_only; /* Chunker^1 + level-1 encoder blob */
  /* byte offsets of the regions inside the workspace; the top K/V region
   * is [n_top][2 (K,V)][batch][H][top_len][hd], the lower region holds
   * level 1, 2, ... L-1 in turn, each [layers][2][batch][H][ceil(tokens /
   * span(l))][hd] (256-byte aligned), the decoder region
   * [n_dec0][2][batch*K1][H][C1][hd]; h is [batch][d] at off_state. */
  uint64_t off_top_kv, off_lower_kv, off_dec_kv, off_state, off_scratch;
} photon_kv_report;

photon_status photon_kv_bytes(const photon_config* cfg, int32_t batch,
                              int64_t tokens, int32_t mode,
                              photon_kv_report* out);

/* Transient device bytes photon_prefill needs for a prompt of `prompt_len`
 * tokens per sequence (activations, and RecGen's level-1 K/V, which is not
 * kept).  The buffer may be freed once photon_prefill's work has completed. */
photon_status photon_prefill_scratch_bytes(const photon_config* cfg,
                                           int32_t batch, int32_t prompt_len,
                                           int32_t mode, uint64_t* out);

/* ------------------------------------------------------------------------
 * Weight blobs (pure host).  Two device blobs: the decode blob (embedding,
 * Chunker^L, top encoder, then Converter^l and the level-(l-1) decoder for
 * l = L down to 1, output head) and the prefill-only blob (Chunker^l and the
 * level-l encoder for l = 1 .. L-1), which RecGen never touches after
 * prefill (explainer, recursive-generation section: only the decoder side
 * must stay on the GPU).
 *
 * Tensors are the canonical ones: matrices W[out][in] (y = x W^T) stored in
 * the config dtype, row-major; norm gains float32.  Within a layer Wq, Wk, Wv
 * are adjacent so that [Wq;Wk;Wv] is one [3d][d] matrix.
 * Tensor names: "E", "W_ch<l>" and "W_cv<l>" (l = 1 .. L), "W_out",
 * "<stack>.<i>.{g1,Wq,Wk,Wv,Wo,g2,W1,W2}", "<stack>.gf" for stack in
 * enc<l> (l = 1 .. L-1), top, dec<l> (l = 0 .. L-1).
 * ---------------------------------------------------------------------- */
typedef struct {
  char name[32];
  int32_t blob;       /* 0 = decode blob, 1 = prefill-only blob */
  int32_t dtype;      /* photon_dtype of the stored elements */
  uint64_t offset;    /* byte offset inside its blob (256-aligned) */
  int64_t rows;       /* out features (vector: length) */
  int64_t cols;       /* in features (vector: 1) */
} photon_tensor_info;

photon_status photon_weight_layout(const photon_config* cfg,
                                   uint64_t* decode_bytes,
                                   uint64_t* prefill_only_bytes,
                                   int32_t* n_tensors);
photon_status photon_weight_tensor(const photon_config* cfg, int32_t index,
                                   photon_tensor_info* out);

/* ------------------------------------------------------------------------
 * Context.  d_w_decode must stay valid until photon_close.  d_w_prefill_only
 * may be NULL, or released later with photon_release_prefill_weights, after
 * which prefill and HierGen decoding return PHOTON_ESTATE.
 * ---------------------------------------------------------------------- */
typedef struct photon_ctx photon_ctx;

photon_status photon_open(const photon_config* cfg, const void* d_w_decode,
                          const void* d_w_prefill_only, photon_ctx** out);
photon_status photon_release_prefill_weights(photon_ctx* ctx);
photon_status photon_close(photon_ctx* ctx);
const char* photon_last_error(void);

/* Prefill (explainer, module table and recursive-generation section):
 * embedding, then Chunker^l -> level-l encoder (causal) for l = 1 .. L-1,
 * then Chunker^L -> top encoder (causal), writing top K/V slots 0 .. n - 1
 * (n = prompt_len / S, whole chunks) and the last top output h into the
 * workspace.  RecGen keeps no lower K/V; HierGen writes every lower level's
 * into the workspace's lower region.  HierGen needs S / span(l) in
 * {1, 2, 4} for every l < L (the queries of one encoder step per sequence;
 * else PHOTON_EUNSUPPORTED).
 * A ragged prompt (prompt_len mod S = r > 0): only whole chunks form top
 * states; the r tail tokens open chunk n, whose decoders take them as given
 * tokens (the next photon_decode_chunk reports them as its first r tokens
 * and draws the other S - r).
 *   d_prompt   [batch][prompt_len] int32 device ids.
 *   prompt_len >= S (else PHOTON_ESHAPE).
 *   max_tokens the capacity the workspace was sized for; prompt_len plus
 *              every later decoded chunk must fit (else PHOTON_ECAPACITY).
 *   d_workspace >= photon_kv_bytes(cfg, batch, max_tokens, mode)
 *              .workspace_total bytes, 256-byte aligned; it holds the whole
 *              decode state and must stay valid while decoding.
 *   d_scratch  >= photon_prefill_scratch_bytes(...) bytes, 256-aligned.
 * Resets the context's position to the end of the prompt. */
photon_status photon_prefill(photon_ctx* ctx, int32_t mode, void* d_workspace,
                             uint64_t ws_bytes, void* d_scratch,
                             uint64_t scratch_bytes, const int32_t* d_prompt,
                             int32_t batch, int32_t prompt_len,
                             int64_t max_tokens, void* stream);

/* One decode chunk of S tokens per sequence (explainer, recursive-generation
 * section).  Converter^L expands h_{i-1} into C_L conditioning vectors; the
 * level-(L-1) decoder (attention confined to the chunk) gives A-hat_i; for
 * l = L-1 down to 2 every level-l vector is expanded by Converter^l and the
 * level-(l-1) decoder over its own C_l positions; every level-1 position is
 * expanded by Converter^1 and the token decoder (in-chunk K/V of C1 slots)
 * into C1 greedy tokens; RecGen then feeds Chunker^L(A-hat_i) to the top
 * encoder, which appends slot i to the global K/V and attends over slots
 * 0..i to give h_i.  HierGen instead re-encodes the tokens through
 * Chunker^l and one level-l encoder step for l = 1 .. L-1 before the top
 * step.
 *   d_tokens  [batch][S] int32 out; token k*C1 + j is position j of level-1
 *             sub-chunk k (k < K1, in time order); greedy argmax, lowest
 *             index on ties.
 *   d_logits  NULL, or [batch][S][vocab] float32 out (the logits behind
 *             every token).
 * PHOTON_ESTATE before a prefill; PHOTON_ECAPACITY when the chunk would pass
 * max_tokens. */
photon_status photon_decode_chunk(photon_ctx* ctx, int32_t* d_tokens,
                                  float* d_logits, void* stream);

/* Consistency diagnostic: the recursive loss of the paper (explainer,
 * recursive-generation section: Eq. 1, a cosine distance that training may
 * add with weight alpha) measured on the chunk a HierGen context decoded
 * last.  d_dist [batch][C_L] float32 out: 1 - cos(A-hat_i[k], A_i[k]) between
 * the level-(L-1) decoder's reconstruction and the level-(L-1) encoder's
 * summary (the two values the top may read; level 1 for two levels) at each
 * of the chunk's C_L positions, on the stored (post-norm, storage-dtype)
 * values, float32 sums.  d_ahat, d_a: NULL, or [batch][C_L][d_model]
 * storage-dtype copies of A-hat_i and A_i.  PHOTON_ESTATE for a RecGen context (it never
 * computes A_i) or before the first decoded chunk. */
photon_status photon_consistency(photon_ctx* ctx, float* d_dist, void* d_ahat,
                                 void* d_a, void* stream);

/* Position bookkeeping: top states held and tokens (prompt + generated). */
photon_status photon_position(const photon_ctx* ctx, int64_t* top_len,
                              int64_t* tokens);

/* Move the decode position back to `tokens` (the prompt end, or a multiple
 * of S between it and the current position), enqueued on `stream`; back at
 * a ragged prompt's end, the next chunk takes the tail as given again.  The top
 * K/V slots from tokens/S on become free and are rewritten by the next
 * chunks.  The caller must first restore the workspace's h region (the
 * photon_kv_report state region, [batch][d] at off_state) to the value it
 * held at that position, e.g. from a copy taken then: this is the resume
 * half of a snapshot (copy the workspace) / restore (copy back + this call)
 * pair.  PHOTON_ESTATE before a prefill, PHOTON_ESHAPE for a bad position. */
photon_status photon_set_position(photon_ctx* ctx, int64_t tokens,
                                  void* stream);

/* Decode chunks run as captured HIP graphs by default: the first
 * photon_decode_chunk after a prefill captures the chunk (its kernels read
 * every position from device memory, so the same graphs serve every chunk)
 * and later calls replay it.  Each graph is a single chain of kernels, which
 * the runtime replays from packets recorded at instantiation.  HierGen: one
 * graph on the caller's stream.  RecGen: the chunk's prefix and token
 * decoder on the caller's stream, the top encoder step as a second graph on
 * a stream of the context, forked after the prefix and joined before the
 * position update through events, so the two run side by side and the
 * caller's stream orders everything after the call.  RecGen's decoders above the token decoder read only the previous
 * top output, so the top branch of chunk i also runs them for chunk i+1
 * (from h_i) while chunk i's tokens are decoded; the first chunk after a
 * prefill or a photon_set_position runs them first.  The results are those
 * of the sequential order.  Calls that ask for logits, and calls while tracing is on, launch
 * the same kernels directly on the caller's stream instead.  enable = 0
 * turns graphs off for this context. */
photon_status photon_use_graphs(photon_ctx* ctx, int32_t enable);

/* ------------------------------------------------------------------------
 * Flat Transformer baseline: the comparison model of the explainer's
 * decode-heavy table (a vanilla decoder whose K/V cache holds every token).
 * One causal stack of n_layers blocks -- the same pre-norm blocks as the
 * PHOTON stacks -- over the tokens, an embedding E[vocab][d] and an untied
 * output head W_out[vocab][d], in one weight blob with tensors "E",
 * "layers.<l>.{g1,Wq,Wk,Wv,Wo,g2,W1,W2}", "layers.gf", "W_out".
 * A context from photon_vanilla_open works with photon_close,
 * photon_position (top_len reports tokens), photon_set_position,
 * photon_use_graphs and the tracing calls; photon_vanilla_prefill and
 * photon_vanilla_decode take the place of photon_prefill and
 * photon_decode_chunk (each pair returns PHOTON_ESTATE on the other kind of
 * context).  Same rounding contract, limits and conventions as above.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t d_model, n_heads, mlp_mult, vocab, n_layers;
  photon_dtype dtype;
  float norm_eps, rope_theta;
  int32_t steps;          /* tokens per sequence per photon_vanilla_decode */
} photon_vanilla_config;

/* top_len / top_kv: the token K/V ([n_layers][K,V][batch][heads][tokens]
 * [head_dim]); the level-1 and decoder fields are 0; weights_decode is the
 * blob, weights_prefill_only 0. */
photon_status photon_vanilla_kv_bytes(const photon_vanilla_config* cfg,
                                      int32_t batch, int64_t tokens,
                                      photon_kv_report* out);
photon_status photon_vanilla_prefill_scratch_bytes(
    const photon_vanilla_config* cfg, int32_t batch, int32_t prompt_len,
    uint64_t* out);
photon_status photon_vanilla_weight_layout(const photon_vanilla_config* cfg,
                                           uint64_t* bytes, int32_t* n_tensors);
photon_status photon_vanilla_weight_tensor(const photon_vanilla_config* cfg,
                                           int32_t index,
                                           photon_tensor_info* out);
photon_status photon_vanilla_open(const photon_vanilla_config* cfg,
                                  const void* d_weights, photon_ctx** out);
/* The prompt through the causal stack at positions 0 .. prompt_len-1,
 * writing every position's K/V and the last position's stack output.
 * prompt_len: a positive multiple of steps.  Workspace and scratch as for
 * photon_prefill, sized by the two vanilla size queries. */
photon_status photon_vanilla_prefill(photon_ctx* ctx, void* d_workspace,
                                     uint64_t ws_bytes, void* d_scratch,
                                     uint64_t scratch_bytes,
                                     const int32_t* d_prompt, int32_t batch,
                                     int32_t prompt_len, int64_t max_tokens,
                                     void* stream);
/* `steps` greedy tokens per sequence: logits = W_out z, token = first
 * argmax, then the token's embedding through the stack at the next position
 * over every cached token gives the next z.  d_tokens [batch][steps];
 * d_logits NULL or [batch][steps][vocab].  PHOTON_ECAPACITY past
 * max_tokens. */
photon_status photon_vanilla_decode(photon_ctx* ctx, int32_t* d_tokens,
                                    float* d_logits, void* stream);

/* ------------------------------------------------------------------------
 * Stand-alone decode attention (no context, no model): the two kernels the
 * decode path runs over a cache, applied to caller buffers.
 *   PHOTON_ATTN_GLOBAL  the top encoder's attention over the global coarse
 *       K/V, the one cache that grows with the context (explainer,
 *       recursive-generation section); split over keys into partials merged
 *       by a second pass when there are few (group, head) pairs.
 *   PHOTON_ATTN_CHUNK   the decoders' attention confined to the current
 *       chunk (explainer, module table: the Context Decoder attends only
 *       within its chunk); at most 16 keys.
 *   PHOTON_ATTN_PREFILL causal self-attention over a whole prompt, the
 *       encoders' attention in prefill (explainer, module table: each
 *       Context Encoder is causal over its level's stream); queries == keys.
 *       bf16 caches run on MFMA with q and the probabilities entering each
 *       product as two bf16 terms (hi + lo: at most 2^-18 relative error per
 *       operand), float32 caches on FMA.
 * Layout: d_q [groups*queries][heads*head_dim] float32, row g*queries + t;
 * d_k, d_v [groups][heads][cap][head_dim] in `dtype` (photon_dtype);
 * d_out like d_q but in `dtype`.  Query t of group g attends to keys
 * 0 .. keys-queries+t of its (g, h) cache, softmax(q k^T / sqrt(head_dim)) v
 * with float32 softmax and accumulation; out is rounded to dtype (bf16:
 * nearest, ties to even).
 * Limits (else PHOTON_ESHAPE / PHOTON_EUNSUPPORTED): head_dim in {32, 64,
 * 96, 128}; 1 <= queries <= keys <= cap; GLOBAL: queries in {1, 2, 4};
 * CHUNK: keys <= 16; PREFILL: queries == keys.  d_scratch holds the split partials:
 * photon_attention_scratch_bytes() bytes (0 when the launch does not
 * split; d_scratch may then be NULL), 256-byte aligned.
 * ---------------------------------------------------------------------- */
typedef enum { PHOTON_ATTN_GLOBAL = 0, PHOTON_ATTN_CHUNK = 1, PHOTON_ATTN_PREFILL = 2 } photon_attn_kind;

photon_status photon_attention_scratch_bytes(int32_t kind, int32_t groups,
                                             int32_t heads, int32_t head_dim,
                                             int32_t queries, int32_t cap,
                                             uint64_t* bytes);
photon_status photon_attention(int32_t kind, int32_t dtype, const float* d_q,
                               const void* d_k, const void* d_v, void* d_out,
                               int32_t groups, int32_t heads, int32_t head_dim,
                               int32_t queries, int32_t keys, int32_t cap,
                               void* d_scratch, uint64_t scratch_bytes,
                               void* stream);

/* photon_attention for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels, same arguments and limits, with the split
 * partials in a built-in device array of PHOTON_NOALLOC_SCRATCH_BYTES
 * (8 MiB) per GPU, held until the process ends.  It calls no
 * allocator.  A launch whose partials
 * (photon_attention_scratch_bytes) exceed that size is rejected with
 * PHOTON_ECAPACITY before anything is enqueued (within the limits above a
 * launch needs at most 3.6 MB, so this only guards later changes of the
 * split rule).  Nothing in the array needs clearing: every split writes its
 * whole partial before the combine reads it.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race and may return wrong results; serialize them. */
photon_status photon_attention_noalloc(int32_t kind, int32_t dtype,
                                       const float* d_q, const void* d_k,
                                       const void* d_v, void* d_out,
                                       int32_t groups, int32_t heads,
                                       int32_t head_dim, int32_t queries,
                                       int32_t keys, int32_t cap, void* stream);
#define PHOTON_NOALLOC_SCRATCH_BYTES (8ull << 20)

/* ------------------------------------------------------------------------
 * Sampling decode and multi-query aggregation (explainer, the paragraph on
 * recovering quality: several slightly varied queries are run and bound by
 * majority vote or best-of-N).  The variation is stochastic decoding, one
 * independent random stream per sequence:
 *   - top_k = 0 keeps the whole vocabulary; k >= 1 keeps every id whose
 *     logit reaches the k-th largest logit (ties at the cut are kept);
 *   - a token is the first maximum over the kept ids of
 *     logit / temperature + G, G = -log(-log u) standard Gumbel noise
 *     (the Gumbel-max identity: this samples the tempered softmax of the
 *     kept ids);
 *   - u = ((x >> 9) + 1/2) * 2^-23 with x word (id % 4) of
 *     Philox-4x32-10 (Salmon et al., "Parallel Random Numbers: As Easy as 1,
 *     2, 3", SC 2011) keyed by `seed` (low word first), counter
 *     (id / 4, absolute token position, sequence index, 0).  The absolute
 *     position of token k*C1 + j of the chunk that starts at token T is
 *     T + k*C1 + j; prompts start at position 0.
 * The log-likelihood of a token is logit[y] - logsumexp(logits) under the
 * model's distribution (temperature 1, whole vocabulary), float32.
 * Vocabularies up to 65536 (else PHOTON_EUNSUPPORTED).
 * ---------------------------------------------------------------------- */
typedef struct {
  float temperature;   /* in [1e-4, 1e4] (else PHOTON_EINVAL) */
  int32_t top_k;       /* >= 0 */
  uint64_t seed;
} photon_sampling;

/* Bytes of the sampling workspace of a context decoding `batch` sequences:
 * the logits of one token step ([batch*K1][vocab] float32) and the chunk's
 * log-likelihoods ([batch][S] float32).  Pure host. */
photon_status photon_sampling_bytes(const photon_config* cfg, int32_t batch,
                                    uint64_t* bytes);
/* Switch a PHOTON context to sampling (s != NULL) or back to greedy
 * decoding (s == NULL; d_ws may then be NULL).  d_ws: caller-owned device
 * memory of >= photon_sampling_bytes(cfg, batch) bytes, 256-byte aligned,
 * valid while sampling; a decode chunk with a larger batch than it holds
 * returns PHOTON_ECAPACITY.  Takes effect at the next decode chunk (the
 * captured graphs are rebuilt).  PHOTON_ESTATE on a flat-baseline context. */
photon_status photon_set_sampling(photon_ctx* ctx, const photon_sampling* s,
                                  void* d_ws, uint64_t ws_bytes);
/* photon_decode_chunk plus d_logprobs: NULL, or [batch][S] float32 out, the
 * log-likelihood of every token (sampling contexts only, else
 * PHOTON_ESTATE). */
photon_status photon_decode_chunk_lp(photon_ctx* ctx, int32_t* d_tokens,
                                     float* d_logits, float* d_logprobs,
                                     void* stream);
/* The sampler alone on caller rows: row r of d_logits [rows][ld] float32
 * (ld >= vocab) draws d_ids[r] for sequence d_seq[r] at absolute position
 * d_pos[r] (int32 device arrays); d_logprobs (nullable) [rows] gets its
 * log-likelihood. */
photon_status photon_sample(int32_t rows, int32_t vocab, const float* d_logits,
                            int64_t ld, const photon_sampling* s,
                            const int32_t* d_seq, const int32_t* d_pos,
                            int32_t* d_ids, float* d_logprobs, void* stream);
/* Multi-query aggregation over groups of `group` (1..64) consecutive
 * sequences of the batch (the last group may be shorter):
 *   d_tokens [batch][tok_ld] int32, d_logprobs [batch][lp_ld] float32: the
 *   generated tokens and their log-likelihoods (first n_tok of each row).
 *   A query's score is the sum of its n_tok log-likelihoods (float32);
 *   its answer is tokens [span_begin, span_end).
 * Out, per group g (ceil(batch / group) of them), member indices within
 * the group: d_best[g] the highest score (lowest index on ties);
 * d_major[g] the member whose answer the most members share (ties: higher
 * score, then lower index); d_votes[g] how many share it.  d_scores
 * (nullable) [batch] the scores. */
photon_status photon_aggregate(int32_t batch, int32_t group, int32_t n_tok,
                               const int32_t* d_tokens, int64_t tok_ld,
                               const float* d_logprobs, int64_t lp_ld,
                               int32_t span_begin, int32_t span_end,
                               int32_t* d_best, int32_t* d_major,
                               int32_t* d_votes, float* d_scores, void* stream);

/* ------------------------------------------------------------------------
 * Tracing: per kernel class, a start and a stop HIP event recorded by the
 * kernel dispatches of every traced operation (the first kernel's start,
 * the last kernel's end; no marker packets between kernels), with the
 * algorithmic bytes and flops of each launch (weights, activations and
 * caches read or written once: no K slabs, split partials or re-reads).
 * ---------------------------------------------------------------------- */
typedef enum {
  PHOTON_K_GEMM_QKV = 0,   /* [Wq;Wk;Wv] projection */
  PHOTON_K_GEMM_O,         /* attention output projection (+ residual) */
  PHOTON_K_GEMM_UP,        /* MLP up projection + GELU */
  PHOTON_K_GEMM_DOWN,      /* MLP down projection (+ residual) */
  PHOTON_K_GEMM_HEAD,      /* output head + greedy argmax */
  PHOTON_K_GEMM_CONV,      /* Context Converter (both levels) */
  PHOTON_K_GEMM_CHUNK,     /* Context Chunker (both levels) */
  PHOTON_K_ATTN_TOP,       /* top-level / level-1 decode attention (split) */
  PHOTON_K_ATTN_CHUNK,     /* decoder attention confined to the chunk */
  PHOTON_K_ATTN_PREFILL,   /* causal prompt attention */
  PHOTON_K_NORM,           /* RMSNorm */
  PHOTON_K_ROPE_KV,        /* rotary embedding + K/V cache append */
  PHOTON_K_EMBED,          /* embedding gather / conditioning add */
  PHOTON_K_ARGMAX,         /* argmax reduction across column tiles */
  PHOTON_K_SAMPLE,         /* sampling: top-k cut + Gumbel-max per row */
  PHOTON_K_COUNT
} photon_kernel_class;

typedef struct {
  int64_t launches;
  double ms;               /* summed event time of the launches */
  double bytes;            /* summed algorithmic HBM bytes */
  double flops;            /* summed algorithmic flops */
} photon_trace_stat;

/* Enable tracing for the classes whose bit (1 << class) is set; 0 turns it
 * off.  Clears previous records.  Traced chunks launch their kernels directly
 * (no graph), one after the other on the caller's stream. */
photon_status photon_trace_enable(photon_ctx* ctx, uint32_t class_mask);
/* Wait for the recorded events, sum them per class into out[PHOTON_K_COUNT]
 * and clear the records (tracing stays enabled). */
photon_status photon_trace_read(photon_ctx* ctx, photon_trace_stat* out);

#ifdef __cplusplus
}
#endif
#endif /* PHOTON_H */
