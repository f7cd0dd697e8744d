/*
 * dflash.h — C ABI of libdflash: the block-diffusion draft step with KV
 * injection, on one AMD Instinct MI355X (gfx950).
 *
 * Sources describing the method (cited by page title and section):
 *   [Note] "DFlash: Block Diffusion for Flash Speculative Decoding" (study note):
 *          整体架构; 三大核心创新 §1 context features, §2 KV injection,
 *          §3 block diffusion decoding; Immediate Materialization.
 *   [Blog] "DFlash：用“块扩散”魔法，让大模型推理速度起飞！": 核心创新 (the
 *          generate-block / verify loop); 2. Flash Verification.
 *   [Deep] "DFlash + Spec V2 深度解析": 2.2 KV 注入; 2.3 块扩散; 4.2 训练配置
 *          (block size, diffusion steps, kv projection dim); 4.3 评估指标.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked (device) are HIP device pointers; (host) are host
 *   pointers.  The caller allocates and owns every buffer; the library never
 *   allocates or frees device memory, never synchronises the stream, and
 *   keeps no pointer after returning.
 * - All work is enqueued on the given stream and runs asynchronously.
 * - Errors found on the host are returned before anything is enqueued.  A
 *   failed launch returns DFLASH_EHIP.  Device-resident indices (block
 *   tables, positions, context lengths, tokens) are the caller's contract;
 *   kernels clamp or skip out-of-range values instead of reading or writing
 *   outside the buffers, so a wrong index gives wrong numbers, not a fault
 *   (context tokens on a page the block table leaves unmapped, -1, are left
 *   out of the attention).  A library built with DFLASH_DEBUG (the build's
 *   debug variant, libdflash_debug.so) copies those indices to the host before
 *   launching anything, synchronising the stream, and returns DFLASH_EINVAL
 *   for any outside its documented range: a context length above the call's
 *   bound, an unmapped or out-of-range page under a context or an injected
 *   position, a sequence index outside [-1, n_seqs), a token outside the
 *   vocabulary, an acceptance length outside [0, block_size].
 * - Matrices are row-major.  A weight W of shape [out, in] maps x to W x.
 * - dtype DFLASH_BF16: weights, embeddings, target hidden states and the KV
 *   pool are bfloat16; RMSNorm gains are float32; activations are float32
 *   and enter the matrix cores as a (hi, lo) pair of bfloat16 values, except
 *   the LM-head input, which is rounded to bfloat16.  dtype DFLASH_F32:
 *   everything float32.
 * - Logits, confidences and uniforms are float32; tokens and lengths int32.
 *
 * KV pool layout (one allocation shared by all sequences; prefix sharing =
 * several block-table rows naming the same physical page):
 *   pool[n_pages][n_layers][2][n_kv_heads][chunk]  with chunk = page_size*head_dim
 *   (index 0 of the third axis holds K, index 1 V)
 *   K chunk: [page_size][head_dim]   (token-major)
 *   V chunk: [head_dim][page_size]   (dimension-major)
 * A page holds every layer's K and V of its page_size tokens in one block.
 * Token t of sequence b lives in physical page block_table[b*max_pages + t/page_size],
 * slot t % page_size.  K is stored after rotary embedding at position t.
 */
#ifndef DFLASH_H_
#define DFLASH_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFLASH_OK = 0,
  DFLASH_EINVAL = -1,     /* NULL pointer or argument out of range */
  DFLASH_ESHAPE = -2,     /* inconsistent or unsupported dimensions */
  DFLASH_EDTYPE = -3,     /* unknown dtype */
  DFLASH_ECAPACITY = -4,  /* request larger than a documented limit */
  DFLASH_EWORKSPACE = -5, /* workspace NULL, misaligned (256 B) or too small */
  DFLASH_EHIP = -6        /* a HIP call or kernel launch failed */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* How the block is denoised over the n_steps forwards ([Deep] 2.3 says only
 * that a few rounds progressively fix the block's tokens; both readings are
 * offered):
 *   DFLASH_SCHEDULE_PROGRESSIVE  step s fixes the floor(sB/S)-floor((s-1)B/S)
 *       most confident still-open positions, which stay fixed (masked
 *       diffusion decoding by confidence);
 *   DFLASH_SCHEDULE_REPREDICT    every step predicts every position again
 *       from the previous step's tokens (step 1 from the all-mask block) and
 *       the block is the last step's prediction.
 * With n_steps = 1 both are one forward plus argmax. */
typedef enum { DFLASH_SCHEDULE_PROGRESSIVE = 0, DFLASH_SCHEDULE_REPREDICT = 1 } dflash_schedule;

/* Draft model dimensions.  Limits: head_dim in {64, 128}; n_q_heads a
 * multiple of n_kv_heads; hidden, intermediate, n_fuse*target_hidden and
 * n_q_heads*head_dim multiples of 64; hidden <= 8192; page_size 16; 0 <= mask_token_id <
 * vocab.  rope_base > 0 (rotate-half pairing (x_j, x_{j+d/2}), frequency
 * rope_base^(-2j/d)).  rms_eps >= 0. */
typedef struct {
  int32_t hidden;
  int32_t n_layers;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t intermediate;
  int32_t vocab;
  int32_t n_fuse;         /* number of target layers whose hidden states are fused */
  int32_t target_hidden;  /* width of one target layer's hidden state */
  int32_t page_size;      /* tokens per KV page; must be 16 */
  int32_t mask_token_id;  /* the [MASK] id a block starts from */
  float rope_base;
  float rms_eps;
  int32_t dtype;          /* dflash_dtype */
  int32_t denoise_schedule; /* dflash_schedule */
  int32_t qk_norm;        /* 1: every query and key head is RMS-normalised over head_dim
                           * (gains q_norm / k_norm, epsilon rms_eps) before the rotary
                           * embedding, the injected context keys included (the Qwen3 layer);
                           * 0: no QK-norm.  dflash_inject_kv supports QK-norm for at
                           * most 16 layers (ECAPACITY beyond). */
} dflash_config;

/* Draft weights (all device pointers; per-layer entries are host arrays of
 * n_layers device pointers).  Matrices in the storage dtype, gains float32.
 *   w_fc      [hidden, n_fuse*target_hidden]           context-feature fusion
 *   w_kv      [n_layers*2*n_kv_heads*head_dim, hidden]  per layer: K rows then V rows;
 *             used both for injected context features and for block tokens
 *   embed     [vocab, hidden];  lm_head [vocab, hidden];  final_norm [hidden]
 *   attn_norm[l], mlp_norm[l]  [hidden]
 *   w_q[l] [n_q_heads*head_dim, hidden];  w_o[l] [hidden, n_q_heads*head_dim]
 *   w_gate[l], w_up[l] [intermediate, hidden];  w_down[l] [hidden, intermediate] */
typedef struct {
  const void* w_fc;
  const void* w_kv;
  const void* embed;
  const float* final_norm;
  const void* lm_head;
  const float* const* attn_norm;
  const void* const* w_q;
  const void* const* w_o;
  const float* const* mlp_norm;
  const void* const* w_gate;
  const void* const* w_up;
  const void* const* w_down;
  const float* const* q_norm;  /* per layer [head_dim] fp32 gains; required iff qk_norm */
  const float* const* k_norm;  /* per layer [head_dim] fp32 gains; required iff qk_norm */
} dflash_weights;

/* Bytes of workspace the calls need for the given maxima (a call checks its
 * own arguments against ws_bytes).  block_size is the draft block (at most
 * 16) or a target forward's n_tok (at most 32).  max_inject_tokens bounds the
 * chunk size of one injection pass (larger injections are processed in
 * chunks of that size); max_ctx_len bounds the context any draft call
 * attends to.  Returns 0 if the configuration is invalid. */
size_t dflash_workspace_size(const dflash_config* cfg, int32_t max_batch, int32_t block_size,
                             int32_t max_inject_tokens, int32_t max_ctx_len);

/* KV injection ([Note] 三大核心创新 §1-§2, Immediate Materialization; [Deep] 2.2).
 * For each of the n_tok tokens: f = w_fc x (x = the token's target hidden
 * states of n_fuse layers, concatenated in layer order), then for every
 * draft layer l at once (one layer-batched product with w_kv):
 * K_l = RoPE(Wk_l f, pos), V_l = Wv_l f, written to the pool at the token's
 * page slot.  Only K/V persist; f is transient.  Injecting a prefix in one
 * call or in several calls gives bit-identical pool contents.
 *   target_hidden (device) [n_tok, n_fuse*target_hidden], storage dtype
 *   tok_seq (device) [n_tok] sequence index b of each token (row of block_table)
 *   tok_pos (device) [n_tok] absolute position of each token in its sequence
 *   kv_pool (device) pool of n_pages pages (layout above)
 *   block_table (device) [n_seqs, max_pages] physical page per logical page
 * Tokens whose sequence (tok_seq = -1, say), logical page or physical page
 * is out of range are skipped.  With bf16 weights, rows with tok_seq < 0 are
 * packed out on the device before the products (their cost is a few bytes
 * each, not a GEMM row), which leaves every written value unchanged.  Tokens
 * are processed in chunks of the rows the workspace holds. */
dflash_status dflash_inject_kv(const dflash_config* cfg, const dflash_weights* w,
                               const void* target_hidden, const int32_t* tok_seq,
                               const int32_t* tok_pos, int32_t n_tok, void* kv_pool,
                               int32_t n_pages, const int32_t* block_table, int32_t n_seqs,
                               int32_t max_pages, void* workspace, size_t ws_bytes,
                               hipStream_t stream);

/* Block-diffusion draft ([Deep] 2.3; [Note] 三大核心创新 §3, 整体架构).
 * Each sequence b drafts block_size tokens at positions ctx_len[b] ..
 * ctx_len[b]+block_size-1.  The block starts as all mask_token_id; each of
 * n_steps forwards runs every draft layer (RMSNorm, grouped-query attention
 * of the block over the sequence's injected context KV plus all block keys,
 * SwiGLU MLP) and the LM head.  Progressive schedule: step s commits
 * floor(sB/S)-floor((s-1)B/S) still-open positions with the highest
 * confidence (log-probability of their candidate; ties to the lower
 * position), the last step commits the rest.  Re-predict schedule: every
 * step replaces every position's token by its candidate.  Candidates:
 * argmax (temperature 0, ties to the lowest id) or
 * Gumbel-max with Philox4x32-10 noise keyed by seed and counter
 * (v/4, i, s, b) (temperature > 0).
 *   ctx_len (device) [batch]; entries are clamped to [0, min(max_ctx_len, max_pages*page_size)]
 *   max_ctx_len (host) upper bound of ctx_len, sizes the attention grid
 *   out_tokens (device) [batch, block_size]
 *   out_logits (device, optional) [batch, block_size, vocab] fp32: each position's
 *              logits at the step that committed it (re-predict: the last step)
 *   out_conf (device, optional) [batch, n_steps, block_size] fp32: confidence of each
 *              open position at each step, NaN where the position was already committed
 *              (re-predict: every position is open at every step)
 *   anchor_tokens (device, optional) [batch]: NULL for the pages' all-[MASK] block.
 *              Otherwise block position 0 of sequence b holds anchor_tokens[b] from
 *              the start, given rather than drafted, and the schedule above runs over
 *              the other block_size-1 positions.  This is the last committed token of
 *              a closed loop: its target hidden state arrives only with the next
 *              verify forward, so it cannot be injected before this call, and the
 *              context (ctx_len[b] tokens) holds everything before it.  Its
 *              out_tokens entry is the anchor, its out_logits row is not written, its
 *              out_conf entries are NaN.
 * Limits: 1 <= block_size <= 16; 1 <= n_steps <= block_size (block_size - 1 with an
 * anchor); temperature >= 0. */
dflash_status dflash_draft_block(const dflash_config* cfg, const dflash_weights* w,
                                 const void* kv_pool, int32_t n_pages,
                                 const int32_t* block_table, int32_t max_pages,
                                 const int32_t* ctx_len, int32_t max_ctx_len, int32_t batch,
                                 int32_t block_size, int32_t n_steps, float temperature,
                                 uint64_t seed, const int32_t* anchor_tokens, int32_t* out_tokens,
                                 float* out_logits, float* out_conf, void* workspace, size_t ws_bytes,
                                 hipStream_t stream);

/* Target-side verify forward ([Blog] 2. Flash Verification: the target checks
 * the whole block in one forward; [Note] 三大核心创新 §1: the drafter is fed
 * hidden states taken from several target layers).  The target model has the
 * draft's layer structure (cfg and w describe the target; w_fc is unused).
 * Sequence b runs n_tok tokens at positions ctx_len[b] .. ctx_len[b]+n_tok-1
 * (the last committed token and the draft block): token j attends to the
 * sequence's cached context (positions < ctx_len[b], read from kv_pool) and
 * causally to tokens 0..j.  Outputs:
 *   out_logits (device) [batch, n_tok, vocab] fp32: row j scores the token
 *              at position ctx_len[b] + j + 1 (the rows dflash_verify_block takes)
 *   out_hidden (device) [batch, n_tok, n_capture * hidden] bf16: the residual
 *              stream after each layer capture_layers[f] (host, distinct, in
 *              [0, n_layers)), slot f; the input of dflash_inject_kv
 * and every layer's K (rotated) and V of the n_tok tokens are written into
 * kv_pool at their positions (the target's own paged cache, the same layout
 * as the draft's), so accepted tokens need no further pass.
 * Limits: bf16 weights and head_dim 128; 1 <= n_tok <= 32 (a block of up to 31
 * and the token before it); the workspace is
 * dflash_workspace_size(cfg, max_batch, n_tok, 0, max_ctx_len). */
dflash_status dflash_target_forward(const dflash_config* cfg, const dflash_weights* w, void* kv_pool,
                                    int32_t n_pages, const int32_t* block_table, int32_t max_pages,
                                    const int32_t* ctx_len, int32_t max_ctx_len, int32_t batch, int32_t n_tok,
                                    const int32_t* tokens, const int32_t* capture_layers, int32_t n_capture,
                                    float* out_logits, void* out_hidden, void* workspace, size_t ws_bytes,
                                    hipStream_t stream);

/* Device-side bookkeeping between two drafter steps, so that inject -> draft
 * -> verify -> advance repeats with no host round trip and can be captured
 * in a HIP graph (host work between steps leaves the GPU idle: [Deep] 3.2
 * Overlap 调度; [Note] Spec V2 引擎优化).  Verification committed
 * accept_len[b] + 1 tokens of sequence b (the accepted prefix and the bonus
 * token) at positions ctx_len[b] .. ctx_len[b] + accept_len[b].  For
 * j = 0..block_size this writes injection row r = b*(block_size+1) + j:
 *   tok_seq[r] = (j <= accept_len[b]) ? b : -1,  tok_pos[r] = ctx_len[b] + j
 * and then advances ctx_len[b] by accept_len[b] + 1.  dflash_inject_kv skips
 * rows with tok_seq = -1 (and, with bf16 weights, packs them out before its
 * products, so only the accepted rows cost GEMM work), so the next injection
 * takes n_tok = batch*(block_size+1) rows of target hidden states laid out
 * [b][j] (the target's states at the block_size+1 verified positions of each
 * sequence).
 *   accept_len (device) [batch], as dflash_verify_block writes it (values
 *              are clamped to [0, block_size])
 *   ctx_len (device) [batch], read and advanced in place
 *   tok_seq, tok_pos (device) [batch*(block_size+1)] int32, written
 * The block table must already map the pages of the new positions;
 * positions past it are skipped by the injection like any unmapped one.
 * Limits: batch >= 0; 1 <= block_size <= 16. */
dflash_status dflash_advance_context(int32_t batch, int32_t block_size, const int32_t* accept_len,
                                     int32_t* ctx_len, int32_t* tok_seq, int32_t* tok_pos,
                                     hipStream_t stream);

/* Bytes of workspace dflash_verify_block needs. */
size_t dflash_verify_workspace_size(int32_t batch, int32_t block_size, int32_t vocab);

/* Block verification ([Blog] 2. Flash Verification; [Note] 整体架构 accept/reject;
 * [Deep] 4.3 acceptance length).  Row i <= block_size of target_logits is the
 * target's prediction for block position i.
 * temperature == 0: y_i = argmax row i (lowest id on ties); a = first i with
 *   y_i != draft_tokens[i] (block_size if none); out = draft[0:a], y_a, then -1.
 * temperature > 0: speculative sampling with p = softmax(target/T),
 *   q = softmax(draft/T): position i is accepted iff u[i][0]*q(d_i) < p(d_i);
 *   at the first rejection the output token is the inverse-CDF draw (with
 *   u[i][1]) from max(0, p-q); if all are accepted the bonus is drawn from
 *   p of row block_size with u[block_size][1].  Inverse CDF: smallest k with
 *   sum_{v<=k} w_v > u * sum_v w_v.
 *   target_logits (device) [batch, block_size+1, vocab] fp32
 *   draft_tokens (device) [batch, block_size] int32
 *   draft_logits (device) [batch, block_size, vocab] fp32, required iff temperature > 0
 *   uniforms (device) [batch, block_size+1, 2] fp32 in [0,1), required iff temperature > 0
 *   accept_len (device) [batch]; out_tokens (device) [batch, block_size+1]
 * Limits: 1 <= block_size <= 16. */
dflash_status dflash_verify_block(int32_t batch, int32_t block_size, int32_t vocab,
                                  const float* target_logits, const int32_t* draft_tokens,
                                  float temperature, const float* draft_logits,
                                  const float* uniforms, int32_t* accept_len,
                                  int32_t* out_tokens, void* workspace, size_t ws_bytes,
                                  hipStream_t stream);

/* dflash_verify_block for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * verification with the same arguments and results, but no workspace argument.
 * Its scratch is a fixed 8 MiB array that the library holds on each GPU it runs on
 * until the process ends; it is found once per device with hipGetSymbolAddress
 * (the stream's device must be the calling thread's current device), and nothing
 * is allocated or freed.  Capacity: dflash_verify_workspace_size(batch,
 * block_size, vocab) <= 8 MiB (batch 32, block 16, vocabulary 151936 needs about
 * 0.4 MiB); larger requests return DFLASH_ECAPACITY before anything is enqueued.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (several streams or threads at once) race on it and must be serialised by the
 * caller.  Each call writes every scratch entry it reads, so no clearing is needed. */
dflash_status dflash_verify_block_static(int32_t batch, int32_t block_size, int32_t vocab,
                                         const float* target_logits, const int32_t* draft_tokens,
                                         float temperature, const float* draft_logits,
                                         const float* uniforms, int32_t* accept_len,
                                         int32_t* out_tokens, hipStream_t stream);

/* Block size for the next drafter step, chosen from the acceptance seen so
 * far.  The pages name block sizes that adapt to how hard the input is as a
 * direction ([Deep] 7.3 短期趋势) and note that too large a block wastes draft
 * work while too small a one gives up speed ([Blog] 局限性); they give no
 * rule.  Reading taken here: acceptance is the observable measure of how
 * predictable the text is.  Each draft position matches the target with
 * probability p, independently, so a step with block B accepts
 * a = min(first mismatch, B) tokens.  The maximum-likelihood estimate of p
 * over the observed steps, with a Beta(prior_a, prior_b) prior, is
 *   p = (sum a + prior_a) / (sum a + #(a < B) + prior_a + prior_b)
 * (0.5 when that is 0/0), and the expected tokens one step commits per
 * sequence are E[a + 1 | B] = 1 + p + ... + p^B.  The choice is the
 * candidate maximising E[a + 1 | B] / step_time(B), ties to the smaller block.
 * Host-only: no device memory, no GPU work, no stream.
 *   accept_len, block_of (host) [n_obs]: accepted draft tokens of one sequence
 *              at one step (bonus excluded), and the block size it drafted with
 *   cand_block (host) [n_cand] in 1..16; step_time (host) [n_cand] > 0, any unit
 *   p_match (host, optional): receives the estimate of p
 * Returns the chosen block size, or a negative dflash_status (EINVAL: a NULL
 * array with a nonzero count, n_cand < 1, a time not > 0, a negative prior,
 * or a_i outside [0, block_of_i]; ECAPACITY: a block size outside 1..16). */
int32_t dflash_adaptive_block_size(const int32_t* accept_len, const int32_t* block_of, int32_t n_obs,
                                   const int32_t* cand_block, const float* step_time, int32_t n_cand,
                                   float prior_a, float prior_b, float* p_match);

/* Human-readable name of a status code (static string). */
const char* dflash_status_string(dflash_status s);

/* Kernel timing for measurement (the benchmark's live per-kernel rates).
 * dflash_prof_select(k) makes every later launch of kernel class k (see
 * dflash_kernel_class) record a HIP event pair on the launch stream;
 * dflash_prof_collect waits for the recorded events (the one place the library
 * blocks on the GPU), returns the summed duration in ms and the launch count,
 * and clears them.  k = DFLASH_PROF_NONE (the default) turns recording off;
 * then no call touches this state.  The event list is the library's only
 * mutable state; it is guarded by a mutex, but interleaving calls on several
 * streams while recording mixes their events. */
typedef enum {
  DFLASH_PROF_NONE = 0,
  DFLASH_PROF_ATTN = 1,       /* paged context attention (all layers, all steps) */
  DFLASH_PROF_GEMM_QKV = 2,
  DFLASH_PROF_GEMM_O = 3,
  DFLASH_PROF_GEMM_GATEUP = 4,
  DFLASH_PROF_GEMM_DOWN = 5,
  DFLASH_PROF_LMHEAD = 6,
  DFLASH_PROF_INJECT_FC = 7,
  DFLASH_PROF_INJECT_KV = 8,
  DFLASH_PROF_VERIFY = 9
} dflash_kernel_class;
dflash_status dflash_prof_select(int32_t kernel_class);
dflash_status dflash_prof_collect(float* total_ms, int32_t* n_launches);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H_ */
