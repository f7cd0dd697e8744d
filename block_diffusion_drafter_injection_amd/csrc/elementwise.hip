// Small kernels of the draft step: rotary tables, block init, embedding
// gather, RMSNorm (with the gather of still-open rows before the LM head),
// the LM-head row combine and the denoise commit.
#include "kernels.h"

namespace dflash {

// Rotary table cs[row][j] = (cos, sin)(pos * base^(-2j/d)) for j < d/2.  The
// angle reaches ~3e4 rad at long contexts, so it is formed and reduced in
// double precision; only the final cos/sin are rounded to float.
__device__ __forceinline__ float2 rope_cs(int pos, int j, int d, double base) {
  const double w = pow(base, -2.0 * (double)j / (double)d);
  double sn, c;
  sincos((double)pos * w, &sn, &c);
  return make_float2((float)c, (float)sn);
}

__global__ void rope_block_kernel(const int* ctx_len, int ctx_cap, int batch, int B, int d, double base,
                                  float2* cs) {
  const int hd = d / 2;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= batch * B * hd) return;
  const int row = idx / hd, j = idx - row * hd;
  const int b = row / B, i = row - b * B;
  int c = ctx_len[b];
  c = c < 0 ? 0 : (c > ctx_cap ? ctx_cap : c);
  cs[idx] = rope_cs(c + i, j, d, base);
}

__global__ void rope_tokens_kernel(const int* tok_pos, int n, int d, double base, float2* cs) {
  const int hd = d / 2;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * hd) return;
  const int row = idx / hd, j = idx - row * hd;
  cs[idx] = rope_cs(tok_pos[row], j, d, base);
}

__global__ void block_init_kernel(int* tau, int* committed, int M, int B, int mask_id, const int* anchor) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < M) {
    const bool given = anchor && i % B == 0;
    tau[i] = given ? anchor[i / B] : mask_id;
    committed[i] = given ? 1 : 0;
  }
}

template <typename T>
__global__ void embed_kernel(const int* tau, const T* embed, int vocab, float* h, int H) {
  const int row = blockIdx.x;
  int t = tau[row];
  t = t < 0 ? 0 : (t >= vocab ? vocab - 1 : t);
  for (int c = threadIdx.x; c < H; c += blockDim.x) h[(size_t)row * H + c] = ld_f(embed, (size_t)t * H + c);
}

// One workgroup per output row.  With committed != null the output rows are
// the still-open positions of each sequence in position order (n_open per
// sequence) and row_map receives b*B + i for each.  With part != null the
// source row first takes the sum of its K-split partials ([ksplit][Mp][H],
// indexed by the source row), which is also written back to h.
constexpr int kRmsMaxH = 8192;   // widest row
constexpr int kRmsMaxSplit = 8;   // K-split partials folded with all loads in flight (more: one at a time)

// NT threads per row (1024 when there are few rows, so more loads are in
// flight per row), VEC float4 of the row per thread.  Every global read of a
// row -- the residual and up to kRmsMaxSplit partials of each of the thread's
// VEC quads -- is issued before the first add or store, so a row costs one
// memory round trip (a store between the quads would keep the later loads
// behind it: h and the partials may alias as far as the compiler knows).
template <int NT, int VEC>
__global__ __launch_bounds__(NT) void rmsnorm_kernel(float* h, const float* gain, ActOut out, int H,
                                                      float eps, const int* committed, int B, int n_open,
                                                      int* row_map, const float* part, int ksplit, int Mp,
                                                      ActOut cap) {
  __shared__ double red[NT / 64];
  __shared__ int src_s;
  const int r = blockIdx.x, tid = threadIdx.x;
  if (tid < 64) {
    // source row: r itself, or the (r mod n_open)-th still-open position of its
    // sequence (a ballot ranks up to 64 positions per pass)
    if (committed) {
      const int b = r / n_open, jj = r - b * n_open;
      bool found = false;
      int seen = 0;
      for (int base = 0; base < B && !found; base += 64) {
        const int i = base + tid;
        const bool open = i < B && !committed[b * B + i];
        const unsigned long long m = __ballot(open);
        const int cnt = __popcll(m);
        if (jj < seen + cnt) {
          if (open && __popcll(m & ((1ull << tid) - 1ull)) == jj - seen) {
            src_s = b * B + i;
            row_map[r] = b * B + i;
          }
          found = true;
        }
        seen += cnt;
      }
      if (!found && tid == 0) {
        src_s = b * B;
        row_map[r] = b * B;
      }
    } else if (tid == 0) {
      src_s = r;
      if (row_map) row_map[r] = r;
    }
  }
  __syncthreads();
  // the row is read once into registers (H <= NT * 4 * VEC); squares are
  // summed in fp32 per thread (at most 4 * VEC terms) and in double across
  // threads
  float* x = h + (size_t)src_s * H;
  const bool fold = part && ksplit <= kRmsMaxSplit;
  const size_t stride = (size_t)Mp * H;
  float4 v[VEC];
  float4 pv[VEC][kRmsMaxSplit];
#pragma unroll
  for (int k = 0; k < VEC; ++k) {
    const int c = tid * 4 + 4 * NT * k;
    v[k] = c < H ? *(const float4*)(x + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float* pp = part + (size_t)src_s * H + c;
#pragma unroll
    for (int sp = 0; sp < kRmsMaxSplit; ++sp)
      pv[k][sp] = (fold && sp < ksplit && c < H) ? *(const float4*)(pp + sp * stride) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < VEC; ++k) {
    const int c = tid * 4 + 4 * NT * k;
    if (part && c < H) {
      // residual += sum of the split-K partials, in split order (the same sums
      // the split-K reduce would form)
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
      if (fold) {
#pragma unroll
        for (int sp = 0; sp < kRmsMaxSplit; ++sp) {
          if (sp < ksplit) { a.x += pv[k][sp].x; a.y += pv[k][sp].y; a.z += pv[k][sp].z; a.w += pv[k][sp].w; }
        }
      } else {
        const float* pp = part + (size_t)src_s * H + c;
        for (int sp = 0; sp < ksplit; ++sp) {
          const float4 q = *(const float4*)(pp + sp * stride);
          a.x += q.x; a.y += q.y; a.z += q.z; a.w += q.w;
        }
      }
      v[k].x += a.x; v[k].y += a.y; v[k].z += a.z; v[k].w += a.w;
      *(float4*)(x + c) = v[k];
    }
    // the finished residual row (a layer's output hidden state), in the storage type
    if (cap.p0 && c < H) act_store4(cap, src_s, c, v[k]);
    ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
  }
  double sd = ss;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sd += __shfl_xor(sd, o, kWave);
  if ((tid & 63) == 0) red[tid >> 6] = sd;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) tot += red[w];
  const float rs = (float)(1.0 / sqrt(tot / (double)H + (double)eps));
#pragma unroll
  for (int k = 0; k < VEC; ++k) {
    const int c = tid * 4 + 4 * NT * k;
    if (c < H) {
      const float4 gg = *(const float4*)(gain + c);
      act_store4(out, r, c, make_float4(v[k].x * rs * gg.x, v[k].y * rs * gg.y, v[k].z * rs * gg.z, v[k].w * rs * gg.w));
    }
  }
}

// Row combine of the LM-head tile partials (four waves per row): a running
// (argmax score, index, z at argmax) and a running (max z, sum of exp)
// pair per lane over a strided set of tiles, then across lanes and waves.
// Ties of the argmax score resolve to the smallest index.
struct LmAcc {
  float pmax, zmax, zsum, zc;
  int idx;
};
__device__ __forceinline__ void lm_merge(LmAcc& a, float qp, float qz, float qs, float qc, int qi) {
  if (qi >= 0 && (a.idx < 0 || qp > a.pmax || (qp == a.pmax && qi < a.idx))) {
    a.pmax = qp;
    a.idx = qi;
    a.zc = qc;
  }
  const float M = fmaxf(a.zmax, qz);
  float s = 0.f;
  if (a.zsum > 0.f) s += a.zsum * __expf(a.zmax - M);
  if (qs > 0.f) s += qs * __expf(qz - M);
  a.zmax = M;
  a.zsum = s;
}

__global__ __launch_bounds__(256) void lm_combine_kernel(const float4* part_f, const int* part_i, int ntiles,
                                                         const int* row_map, int* cand, float* conf) {
  __shared__ float sh[4][4];
  __shared__ int shi[4];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  LmAcc a{-INFINITY, -INFINITY, 0.f, -INFINITY, -1};
  // a thread's partials t = tid + 256 k, merged in k order; LMQ of them loaded
  // per pass before the first merge, so their loads are in flight together
  constexpr int LMQ = 8;
  for (int t0 = tid; t0 < ntiles; t0 += 256 * LMQ) {
    float4 f[LMQ];
    int fi[LMQ];
#pragma unroll
    for (int q = 0; q < LMQ; ++q) {
      const int t = t0 + 256 * q;
      f[q] = t < ntiles ? part_f[(size_t)r * ntiles + t] : make_float4(0.f, 0.f, 0.f, 0.f);
      fi[q] = t < ntiles ? part_i[(size_t)r * ntiles + t] : -1;
    }
#pragma unroll
    for (int q = 0; q < LMQ; ++q)
      if (t0 + 256 * q < ntiles) lm_merge(a, f[q].x, f[q].y, f[q].z, f[q].w, fi[q]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
    lm_merge(a, __shfl_xor(a.pmax, o, kWave), __shfl_xor(a.zmax, o, kWave), __shfl_xor(a.zsum, o, kWave),
             __shfl_xor(a.zc, o, kWave), __shfl_xor(a.idx, o, kWave));
  if (lane == 0) {
    sh[w][0] = a.pmax;
    sh[w][1] = a.zmax;
    sh[w][2] = a.zsum;
    sh[w][3] = a.zc;
    shi[w] = a.idx;
  }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < 4; ++k) lm_merge(a, sh[k][0], sh[k][1], sh[k][2], sh[k][3], shi[k]);
    const int dst = row_map[r];
    cand[dst] = a.idx;
    conf[dst] = a.zc - (a.zmax + logf(a.zsum));
  }
}

// Denoise commit for one sequence (one wave, lane = block position): the
// k_step most confident open positions (ties to the lower position) take
// their candidate; at the last step every open position does.  Re-predict:
// every position takes its candidate and stays open for the next step.
__global__ __launch_bounds__(64) void commit_kernel(const int* cand, const float* conf, int* tau, int* committed,
                                                    float* out_conf, int* out_tokens, int B, int S, int step,
                                                    int k_step, int last, int repredict) {
  __shared__ float cs[16];
  __shared__ int open[16];
  const int b = blockIdx.x, i = threadIdx.x;
  const int row = b * B + i;
  if (i < B) {
    open[i] = !committed[row];
    cs[i] = conf[row];
  }
  __syncthreads();
  if (i < B) {
    if (out_conf) out_conf[((size_t)b * S + step) * B + i] = open[i] ? cs[i] : __int_as_float(0x7fc00000);
    if (repredict) {
      if (open[i]) tau[row] = cand[row];   // a given anchor stays
    } else if (open[i]) {
      int rank = 0;
      for (int k = 0; k < B; ++k)
        if (open[k] && (cs[k] > cs[i] || (cs[k] == cs[i] && k < i))) ++rank;
      if (last || rank < k_step) {
        tau[row] = cand[row];
        committed[row] = 1;
      }
    }
  }
  __syncthreads();
  if (last && out_tokens && i < B) out_tokens[row] = tau[row];
}

hipError_t launch_rope_table_block(const int* ctx_len, int ctx_cap, int batch, int B, int d, double base,
                                   float2* cs, hipStream_t s) {
  const int n = batch * B * (d / 2);
  hipLaunchKernelGGL(rope_block_kernel, dim3((n + 255) / 256), dim3(256), 0, s, ctx_len, ctx_cap, batch, B, d,
                     base, cs);
  return hipGetLastError();
}

// Stable compaction of injection rows: the rows r < n with tok_seq[r] >= 0
// become rows 0..count-1 in their order (src[i] = r, seq_c[i] = tok_seq[r],
// pos_c[i] = tok_pos[r]); rows count..n-1 get seq_c = -1 and pos_c = 0, which
// the scatter skips.  One workgroup walks the rows 1024 at a time: a ballot
// ranks the rows of each wave, the wave counts give each wave's offset, and a
// running total carries over to the next 1024.
__global__ __launch_bounds__(1024) void compact_rows_kernel(const int* tok_seq, const int* tok_pos, int n, int* src,
                                                           int* seq_c, int* pos_c, int* count) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int base = 0;
  for (int r0 = 0; r0 < n; r0 += 1024) {
    const int r = r0 + tid;
    const int sq = r < n ? tok_seq[r] : -1;
    const bool v = sq >= 0;
    const unsigned long long m = __ballot(v);
    if (lane == 0) wsum[w] = __popcll(m);
    __syncthreads();
    int off = base, tot = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      off += k < w ? wsum[k] : 0;
      tot += wsum[k];
    }
    if (v) {
      const int i = off + __popcll(m & ((1ull << lane) - 1ull));
      src[i] = r;
      seq_c[i] = sq;
      pos_c[i] = tok_pos[r];
    }
    base += tot;
    __syncthreads();   // wsum is rewritten by the next block of rows
  }
  for (int i = base + tid; i < n; i += 1024) {
    src[i] = 0;
    seq_c[i] = -1;
    pos_c[i] = 0;
  }
  if (tid == 0) *count = base;
}

hipError_t launch_compact_rows(const int* tok_seq, const int* tok_pos, int n, int* src, int* seq_c, int* pos_c,
                               int* count, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(compact_rows_kernel, dim3(1), dim3(1024), 0, s, tok_seq, tok_pos, n, src, seq_c, pos_c, count);
  return hipGetLastError();
}

hipError_t launch_rope_table_tokens(const int* tok_pos, int n, int d, double base, float2* cs, hipStream_t s) {
  const int t = n * (d / 2);
  if (t <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_tokens_kernel, dim3((t + 255) / 256), dim3(256), 0, s, tok_pos, n, d, base, cs);
  return hipGetLastError();
}

// QK-norm in place, one wave per (row, query-or-key head) of qkv
// [M, (nq + 2 nkv) d] (head_dim <= 128: two values per lane at most).
__global__ __launch_bounds__(256) void qk_norm_kernel(float* qkv, int M, int nq, int nkv, int d,
                                                     const float* q_gain, const float* k_gain, float eps) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int heads = nq + nkv;
  if (wave >= M * heads) return;   // the whole wave leaves together
  const int row = wave / heads, hh = wave - row * heads;
  float* x = qkv + (size_t)row * (nq + 2 * nkv) * d + (size_t)hh * d;
  const float* g = hh < nq ? q_gain : k_gain;
  float v[2], ss = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    v[k] = c < d ? x[c] : 0.f;
    ss = fmaf(v[k], v[k], ss);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
  const float inv = 1.f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    if (c < d) x[c] = v[k] * inv * g[c];
  }
}

hipError_t launch_qk_norm(float* qkv, int M, int nq, int nkv, int d, const float* q_gain, const float* k_gain,
                          float eps, hipStream_t s) {
  const int waves = M * (nq + nkv);
  if (waves <= 0) return hipSuccess;
  if (d > 128 || !q_gain || !k_gain) return hipErrorInvalidValue;
  hipLaunchKernelGGL(qk_norm_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, qkv, M, nq, nkv, d, q_gain, k_gain, eps);
  return hipGetLastError();
}

hipError_t launch_block_init(int* tau, int* committed, int M, int B, int mask_id, const int* anchor,
                             hipStream_t s) {
  hipLaunchKernelGGL(block_init_kernel, dim3((M + 255) / 256), dim3(256), 0, s, tau, committed, M, B, mask_id,
                     anchor);
  return hipGetLastError();
}

hipError_t launch_embed(const int* tau, const void* embed, int wdtype, int vocab, float* h, int M, int H,
                        hipStream_t s) {
  if (wdtype)
    hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(M), dim3(256), 0, s, tau, (const bf16_t*)embed, vocab, h, H);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(M), dim3(256), 0, s, tau, (const float*)embed, vocab, h, H);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(float* h, const float* gain, ActOut out, int M, int H, float eps,
                          const int* committed, int B, int n_open, int* row_map, hipStream_t s,
                          const float* part, int ksplit, int part_rows, const ActOut* capture) {
  if (M <= 0) return hipSuccess;
  ActOut cap{};
  if (capture) cap = *capture;
  if (H <= 0 || H > kRmsMaxH || H % 4) return hipErrorInvalidValue;
  const int ks = part ? ksplit : 0, mp = part_rows > 0 ? part_rows : M;
#define RMS_GO(NT, VEC)                                                                                        \
  hipLaunchKernelGGL((rmsnorm_kernel<NT, VEC>), dim3(M), dim3(NT), 0, s, h, gain, out, H, eps, committed, B, n_open, \
                     row_map, part, ks, mp, cap)
  // threads per row and quads per thread: the row in one pass, at most four
  // quads (and their partials) in registers per thread
  if (M < 128) {
    if (H <= 4096) RMS_GO(1024, 1);
    else RMS_GO(1024, 2);
  } else if (H <= 1024) {
    RMS_GO(256, 1);
  } else if (H <= 2048) {
    RMS_GO(256, 2);
  } else if (H <= 4096) {
    RMS_GO(256, 4);
  } else {
    RMS_GO(512, 4);
  }
#undef RMS_GO
  return hipGetLastError();
}

// Block K (rotated, fp32) and V of n_tok tokens per sequence, for one layer,
// into the paged pool at positions ctx_len[b] + j: K chunk rows are
// token-major [slot][d], V chunks dimension-major [d][slot].  Positions
// outside the block table or unmapped pages are skipped.
__global__ __launch_bounds__(256) void kv_append_kernel(const float* kblk, const float* vblk, const int* ctx_len,
                                                        int ctx_cap, bf16_t* pool, int n_pages,
                                                        const int* block_table, int max_pages, int batch, int n_tok,
                                                        int nkv, int d, int n_layers, int layer) {
  const size_t total = (size_t)batch * nkv * n_tok * d;
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int e = (int)(t % d);
  const size_t r = t / d;
  const int j = (int)(r % n_tok);
  const int m = (int)((r / n_tok) % nkv);
  const int b = (int)(r / ((size_t)n_tok * nkv));
  const int pos = min(max(ctx_len[b], 0), ctx_cap) + j;
  const int lp = pos >> 4, slot = pos & 15;
  if (lp >= max_pages) return;
  const int phys = block_table[(size_t)b * max_pages + lp];
  if (phys < 0 || phys >= n_pages) return;
  const size_t src = (((size_t)b * nkv + m) * n_tok + j) * d + e;
  const size_t chunk = (size_t)16 * d;
  bf16_t* kc = pool + ((((size_t)phys * n_layers + layer) * 2 + 0) * nkv + m) * chunk;
  bf16_t* vc = pool + ((((size_t)phys * n_layers + layer) * 2 + 1) * nkv + m) * chunk;
  kc[slot * d + e] = f2bf(kblk[src]);
  vc[e * 16 + slot] = f2bf(vblk[src]);
}

hipError_t launch_kv_append(const float* kblk, const float* vblk, const int* ctx_len, int ctx_cap, void* pool,
                            int n_pages, const int* block_table, int max_pages, int batch, int n_tok, int nkv, int d,
                            int n_layers, int layer, hipStream_t s) {
  const size_t total = (size_t)batch * nkv * n_tok * d;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, kblk, vblk, ctx_len,
                     ctx_cap, (bf16_t*)pool, n_pages, block_table, max_pages, batch, n_tok, nkv, d, n_layers, layer);
  return hipGetLastError();
}

// One workgroup per sequence: rows j = 0..B of the next injection, then the
// context length advances (after every row has read the old value).
__global__ __launch_bounds__(64) void advance_context_kernel(int B, const int* accept_len, int* ctx_len,
                                                             int* tok_seq, int* tok_pos) {
  const int b = blockIdx.x, j = threadIdx.x;
  const int a = min(max(accept_len[b], 0), B);
  const int c = ctx_len[b];
  if (j <= B) {
    tok_seq[b * (B + 1) + j] = j <= a ? b : -1;
    tok_pos[b * (B + 1) + j] = c + j;
  }
  __syncthreads();
  if (j == 0) ctx_len[b] = c + a + 1;
}

hipError_t launch_advance_context(int batch, int B, const int* accept_len, int* ctx_len, int* tok_seq,
                                  int* tok_pos, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(advance_context_kernel, dim3(batch), dim3(64), 0, s, B, accept_len, ctx_len, tok_seq, tok_pos);
  return hipGetLastError();
}

hipError_t launch_lm_combine(const float4* part_f, const int* part_i, int ntiles, int rows, const int* row_map,
                             int* cand, float* conf, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(lm_combine_kernel, dim3(rows), dim3(256), 0, s, part_f, part_i, ntiles, row_map, cand, conf);
  return hipGetLastError();
}

hipError_t launch_commit(const int* cand, const float* conf, int* tau, int* committed, float* out_conf,
                         int* out_tokens, int batch, int B, int S, int step, int k_step, int last, bool repredict,
                         hipStream_t s) {
  hipLaunchKernelGGL(commit_kernel, dim3(batch), dim3(64), 0, s, cand, conf, tau, committed, out_conf, out_tokens,
                     B, S, step, k_step, last, repredict ? 1 : 0);
  return hipGetLastError();
}

}  // namespace dflash
