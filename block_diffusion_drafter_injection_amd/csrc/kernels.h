// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace dflash {

// GEMM: C[M, N] = A[M, K] * W[N, K]^T, fp32 accumulation, fused epilogue.
enum EpiKind : int { EPI_STORE = 0, EPI_ADD = 1, EPI_SWIGLU = 2, EPI_LMHEAD = 3, EPI_KVSCATTER = 4 };

// Rows of W.  mode 0: row n of b0.  mode 1: rows [0, split) of b0 then b1.
// mode 2 (SwiGLU): each tile of BN columns holds BN/2 rows of b0 (gate) then
// the same BN/2 rows of b1 (up); a kernel may load them interleaved (16 gate
// rows, then the same 16 up rows, per 32 columns) as long as its output
// follows the same contract.
struct BRowsArgs {
  const void* b0;
  const void* b1;
  int ldb;
  int split;
  int mode;
};

struct EpiParams {
  // EPI_STORE / EPI_SWIGLU: destination
  ActOut out;
  // EPI_ADD: resid[row * ldr + col] += value
  float* resid;
  int ldr;
  // EPI_LMHEAD: per (row, column tile) partials, optional logits
  float4* part_f;        // (pmax, zmax, zsum, zc)
  int* part_i;           // argmax index
  int ntiles;
  const int* row_map;    // compact row -> b*B + i
  float* logits;         // [bt*B, V] or null
  int col0;              // vocabulary index of the launch's column 0 (set by launch_gemm)
  int ldz;               // vocabulary size: logits row stride (set by launch_gemm)
  int block;             // B
  float temperature;
  uint32_t seed_lo, seed_hi;
  int step;
  // EPI_KVSCATTER: write K (rotated) / V into the paged pool
  void* pool;
  const int* tok_seq;
  const int* tok_pos;
  const int* block_table;
  int n_seqs, max_pages, n_pages;
  const float2* rope_cs;  // [M, d/2]
  int n_layers, n_kv, head_dim;
  // EPI_KVSCATTER with QK-norm: each K head is RMS-normalised over head_dim
  // with layer l's gains k_gain[l] before the rotation
  int k_norm_on;
  float rms_eps;
  const float* k_gain[kMaxQkLayers];
};

struct GemmArgs {
  int wdtype;            // 0 f32 weights (A f32), 1 bf16 weights (A hi/lo or bf16)
  ActIn a;
  BRowsArgs b;
  int M, N, K;
  int kind;
  EpiParams e;
  bool fixed_split;      // K split chosen from (N, K) only: results independent of M
  float* part;           // split-K partials (gemm_partial_bytes of the plan), or null
  bool defer_reduce;     // EPI_ADD / EPI_STORE with a K split: leave the partials to the consumer
                         // (the next RMSNorm, or the query prep of the attention)
  const int* m_dev;      // optional device row count <= M: rows from it on are neither computed
                         // nor written (tile configuration 2 only, i.e. a fixed K split)
  size_t part_cap;       // EPI_LMHEAD: bytes at part (0: none); the last round of tiles is K-split
                         // into it when gemm_lmhead_part_bytes(M, N) fit
};

struct GemmPlan {
  int cfg;               // tile configuration
  int ksplit;            // K ranges reduced in fixed order (1 = none)
};
GemmPlan gemm_plan(int wdtype, int a_mode, int M, int N, int K, int kind, bool fixed_split);
size_t gemm_partial_bytes(const GemmPlan& p, int M, int N);
// Partial bytes the bf16 LM head over at most M rows (N columns, one activation
// plane) uses for the K split of its last, partly filled round of tiles.
size_t gemm_lmhead_part_bytes(int M, int N);
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s);
int gemm_ksplit(const GemmArgs& g);   // K split launch_gemm uses for g
int gemm_bn(int wdtype, int K);  // columns per LM-head partial (partial count = ceil(N / bn))

// Attention of the block queries over paged context KV plus in-block keys.
struct AttnParams {
  const void* pool;
  int n_pages;
  const int* block_table;
  int max_pages;
  const int* ctx_len;
  int ctx_cap;            // clamp of ctx_len
  const float* qkv;       // [M, (nq + 2 nkv) d] fp32, not yet rotated
  const float2* cs;       // rope table [M, d/2]
  int batch, B, nq, nkv, d, n_layers, layer;
  float scale;
  int n_splits, pps;      // context splits and pages per split (pps even)
  float* part_o;          // [n_splits, M*nq, d] normalised partial outputs
  float* part_lse;        // [n_splits, M*nq] their log-sum-exp
  bf16_t* q_hi;           // [batch, nkv, g*B, d] rotated queries, hi plane (bf16 pools)
  bf16_t* q_lo;           // same, lo plane
  float* kblk;            // [batch, nkv, B, d] rotated block keys, fp32 (bf16 pools)
  float* vblk;            // [batch, nkv, B, d] block values, fp32 (bf16 pools)
  const float* qkv_part;  // [qkv_ks, M, (nq + 2 nkv) d] K-split partials of qkv, or null
  int qkv_ks;             // number of partials (the query prep sums them in split order)
  const float* q_gain;    // QK-norm gains of this layer [d], or null (no QK-norm)
  const float* k_gain;
  float rms_eps;
  int causal;             // 1: block query i sees block keys j <= i only (target forward)
};
// Context splits -> partials (no launch when there is no context).
// Query rows per context workgroup for R query rows per kv head (64 or 128).
int att_query_group(int R, int wdtype, int d);
hipError_t launch_attention(const AttnParams& p, int wdtype, hipStream_t s, void (*mark)(int, hipStream_t));
// In-block keys + merge with the partials -> attention output as GEMM operand.
hipError_t launch_attn_finish(const AttnParams& p, int wdtype, ActOut out, hipStream_t s);

// Elementwise and bookkeeping kernels.
hipError_t launch_rope_table_block(const int* ctx_len, int ctx_cap, int batch, int B, int d,
                                   double base, float2* cs, hipStream_t s);
// Injection rows with tok_seq >= 0 packed to the front, in order (the rest
// marked -1); count = how many (device).
hipError_t launch_compact_rows(const int* tok_seq, const int* tok_pos, int n, int* src, int* seq_c, int* pos_c,
                               int* count, hipStream_t s);
hipError_t launch_rope_table_tokens(const int* tok_pos, int n, int d, double base, float2* cs,
                                    hipStream_t s);
// tau = mask_id, nothing committed; with anchor != null, position 0 of each block
// of B takes anchor[b] and is committed from the start.
hipError_t launch_block_init(int* tau, int* committed, int M, int B, int mask_id, const int* anchor,
                             hipStream_t s);
// QK-norm in place on the query and key heads of qkv [M, (nq + 2 nkv) d] (before RoPE).
hipError_t launch_qk_norm(float* qkv, int M, int nq, int nkv, int d, const float* q_gain, const float* k_gain,
                          float eps, hipStream_t s);
hipError_t launch_embed(const int* tau, const void* embed, int wdtype, int vocab, float* h, int M,
                        int H, hipStream_t s);
// With part != null, h += sum over the ksplit partials [ksplit][part_rows][H]
// (in split order, part_rows = M when 0) first, and the rows read are written
// back to h.
// With capture != null, the finished residual row (after the fold) is also
// stored there in its storage type (a layer's output hidden state).  Without
// committed, row_map (if given) receives the identity.
hipError_t launch_rmsnorm(float* h, const float* gain, ActOut out, int M, int H, float eps,
                          const int* committed, int B, int n_open, int* row_map, hipStream_t s,
                          const float* part = nullptr, int ksplit = 0, int part_rows = 0,
                          const ActOut* capture = nullptr);
// Rotated block K and block V of one layer (the query prep's kblk / vblk) into
// the paged bf16 pool at positions ctx_len[b] + j.
hipError_t launch_kv_append(const float* kblk, const float* vblk, const int* ctx_len, int ctx_cap, void* pool,
                            int n_pages, const int* block_table, int max_pages, int batch, int n_tok, int nkv, int d,
                            int n_layers, int layer, hipStream_t s);
// Injection rows of the tokens a verification committed, and ctx_len += a + 1.
hipError_t launch_advance_context(int batch, int B, const int* accept_len, int* ctx_len, int* tok_seq,
                                  int* tok_pos, hipStream_t s);
hipError_t launch_lm_combine(const float4* part_f, const int* part_i, int ntiles, int rows,
                             const int* row_map, int* cand, float* conf, hipStream_t s);
hipError_t launch_commit(const int* cand, const float* conf, int* tau, int* committed, float* out_conf,
                         int* out_tokens, int batch, int B, int S, int step, int k_step, int last, bool repredict,
                         hipStream_t s);

// Verification.
int verify_chunks(int vocab);
hipError_t launch_verify_greedy(int batch, int B, int V, const float* zt, const int* draft,
                                int* accept_len, int* out_tokens, void* ws, hipStream_t s);
hipError_t launch_verify_sampled(int batch, int B, int V, const float* zt, const float* zd,
                                 const int* draft, const float* uniforms, float T,
                                 int* accept_len, int* out_tokens, void* ws, hipStream_t s);
size_t verify_ws_bytes(int batch, int B, int V);

}  // namespace dflash
