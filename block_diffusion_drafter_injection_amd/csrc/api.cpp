// libdflash C ABI: argument checks, workspace layout and the launch sequence
// of KV injection, the block-diffusion draft and block verification.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstring>
#include <mutex>
#include <vector>

#include "dflash.h"
#include "kernels.h"

using namespace dflash;

namespace {

// ---------------------------------------------------------------- timing hooks
// The only state the library keeps: measurement hooks (dflash_prof_*) that,
// when a kernel class is selected, bracket that class's launches with HIP
// events.  Off by default; guarded by a mutex.
struct Prof {
  std::atomic<int> cls{DFLASH_PROF_NONE};
  std::mutex mu;
  std::vector<hipEvent_t> pool;  // reusable events
  std::vector<std::pair<hipEvent_t, hipEvent_t>> recorded;
  hipEvent_t open = nullptr;
  size_t used = 0;
} g_prof;

hipEvent_t prof_event() {
  if (g_prof.used == g_prof.pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_prof.pool.push_back(e);
  }
  return g_prof.pool[g_prof.used++];
}

void prof_mark(int cls, int phase, hipStream_t s) {
  const int sel = g_prof.cls.load(std::memory_order_relaxed);
  if (sel == DFLASH_PROF_NONE || sel != cls) return;
  std::lock_guard<std::mutex> lock(g_prof.mu);
  hipEvent_t e = prof_event();
  if (!e) return;
  if (hipEventRecord(e, s) != hipSuccess) return;
  if (phase == 0) {
    g_prof.open = e;
  } else if (g_prof.open) {
    g_prof.recorded.emplace_back(g_prof.open, e);
    g_prof.open = nullptr;
  }
}

void prof_attn(int phase, hipStream_t s) { prof_mark(DFLASH_PROF_ATTN, phase, s); }

hipError_t gemm(int cls, const GemmArgs& g, hipStream_t s) {
  prof_mark(cls, 0, s);
  hipError_t e = launch_gemm(g, s);
  prof_mark(cls, 1, s);
  return e;
}

// ---------------------------------------------------------------- checks
bool ptr_ok(const void* p) { return p != nullptr; }

dflash_status check_cfg(const dflash_config* c) {
  if (!c) return DFLASH_EINVAL;
  if (c->dtype != DFLASH_F32 && c->dtype != DFLASH_BF16) return DFLASH_EDTYPE;
  if (c->hidden <= 0 || c->n_layers <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->intermediate <= 0 ||
      c->vocab < 2 || c->n_fuse <= 0 || c->target_hidden <= 0)
    return DFLASH_ESHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return DFLASH_ESHAPE;
  if (c->n_q_heads % c->n_kv_heads) return DFLASH_ESHAPE;
  if (c->hidden % 64 || c->intermediate % 64 || (c->n_fuse * c->target_hidden) % 64) return DFLASH_ESHAPE;
  if (c->hidden > 8192) return DFLASH_ESHAPE;
  if (c->page_size != 16) return DFLASH_ESHAPE;
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab) return DFLASH_EINVAL;
  if (c->denoise_schedule != DFLASH_SCHEDULE_PROGRESSIVE && c->denoise_schedule != DFLASH_SCHEDULE_REPREDICT)
    return DFLASH_EINVAL;
  if (c->qk_norm != 0 && c->qk_norm != 1) return DFLASH_EINVAL;
  if (!(c->rope_base > 0.f) || !(c->rms_eps >= 0.f)) return DFLASH_EINVAL;
  return DFLASH_OK;
}

dflash_status check_weights(const dflash_config* c, const dflash_weights* w, bool draft) {
  if (!w) return DFLASH_EINVAL;
  if (!ptr_ok(w->w_fc) || !ptr_ok(w->w_kv)) return DFLASH_EINVAL;
  if (c->qk_norm) {
    if (!w->k_norm || (draft && !w->q_norm)) return DFLASH_EINVAL;
    for (int l = 0; l < c->n_layers; ++l)
      if (!w->k_norm[l] || (draft && !w->q_norm[l])) return DFLASH_EINVAL;
  }
  if (!draft) return DFLASH_OK;
  if (!ptr_ok(w->embed) || !ptr_ok(w->final_norm) || !ptr_ok(w->lm_head)) return DFLASH_EINVAL;
  const void* const* arrs[7] = {(const void* const*)w->attn_norm, w->w_q, w->w_o, (const void* const*)w->mlp_norm,
                                w->w_gate, w->w_up, w->w_down};
  for (auto a : arrs) {
    if (!a) return DFLASH_EINVAL;
    for (int l = 0; l < c->n_layers; ++l)
      if (!a[l]) return DFLASH_EINVAL;
  }
  return DFLASH_OK;
}

// ---------------------------------------------------------------- workspace
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  }
};

void attn_split(int bt, int nkv, int nqg, int ctx_cap, bool valu, int& ns, int& pps) {
  const int pages = (ctx_cap + 15) / 16;
  if (pages <= 0) {
    ns = 0;
    pps = 2;
    return;
  }
  const int pairs = std::max(1, bt * nkv * nqg);
  // enough splits for kAttWgTarget workgroups; and, up to kAttBalanceSplits
  // splits, at most about kAttMaxPps pages per split, so that in a batch of
  // mixed lengths the longest sequence is spread over several workgroups
  // (splits past a shorter sequence's end exit at once).  Beyond that the
  // partials each split writes cost more than the balance gains (measured on
  // contexts of 16k-32k tokens).
  constexpr int kAttWgTarget = 512, kAttMaxPps = 132, kAttBalanceSplits = 4;
  const int by_len = std::min(kAttBalanceSplits, (pages + kAttMaxPps - 1) / kAttMaxPps);
  const int want = std::max((kAttWgTarget + pairs - 1) / pairs, by_len);
  // at least four 32-token tiles per split for the MFMA kernel (its pipeline
  // fill); the VALU kernel (fp32 pools, head_dim 64) walks a split page by
  // page and takes splits down to one tile
  const int max_ns = valu ? std::max(1, (pages + 1) / 2) : std::max(1, pages / 8);
  const int min_ns = (pages + 511) / 512;   // the context kernel stages at most 512 page ids
  ns = std::max(min_ns, std::max(1, std::min(want, max_ns)));
  pps = (pages + ns - 1) / ns;
  pps = (pps + 1) & ~1;
  ns = (pages + pps - 1) / pps;
}

int n_qgroups(const dflash_config* c, int B) {
  const int R = (c->n_q_heads / c->n_kv_heads) * B;
  const int qg = att_query_group(R, c->dtype == DFLASH_BF16 ? 1 : 0, c->head_dim);
  return (R + qg - 1) / qg;
}

struct DraftWS {
  size_t h, u_hi, u_lo, qkv, o_hi, o_lo, act_hi, act_lo, y, row_map, part_f, part_i, att_o, att_lse, cs, tau,
      committed, cand, conf, gemm_part, q_hi, q_lo, kblk, vblk, total;
  size_t gemm_part_bytes;
  int ns, pps, ntiles;
};

DraftWS draft_layout(const dflash_config* c, int bt, int B, int ctx_cap) {
  DraftWS w{};
  const size_t M = (size_t)bt * B;
  const size_t H = c->hidden, I = c->intermediate, d = c->head_dim, nq = c->n_q_heads, nkv = c->n_kv_heads;
  const size_t el = c->dtype == DFLASH_BF16 ? 2 : 4;  // one plane of an activation operand
  attn_split(bt, (int)nkv, n_qgroups(c, B), ctx_cap, !(c->dtype == DFLASH_BF16 && c->head_dim == 128), w.ns, w.pps);
  w.ntiles = (c->vocab + gemm_bn(c->dtype, c->hidden) - 1) / gemm_bn(c->dtype, c->hidden);
  Carve k;
  w.h = k.take(M * H * 4);
  w.u_hi = k.take(M * H * el);
  w.u_lo = k.take(M * H * el);
  w.qkv = k.take(M * (nq + 2 * nkv) * d * 4);
  w.o_hi = k.take(M * nq * d * el);
  w.o_lo = k.take(M * nq * d * el);
  w.act_hi = k.take(M * I * el);
  w.act_lo = k.take(M * I * el);
  w.y = k.take(M * H * 4);
  w.row_map = k.take(M * 4);
  w.part_f = k.take(M * w.ntiles * 16);
  w.part_i = k.take(M * w.ntiles * 4);
  w.att_o = k.take((size_t)std::max(w.ns, 1) * M * nq * d * 4);
  w.att_lse = k.take((size_t)std::max(w.ns, 1) * M * nq * 4);
  w.cs = k.take(M * (d / 2) * 8);
  w.tau = k.take(M * 4);
  w.committed = k.take(M * 4);
  w.cand = k.take(M * 4);
  w.conf = k.take(M * 4);
  w.q_hi = k.take(M * nq * d * 2);
  w.q_lo = k.take(M * nq * d * 2);
  w.kblk = k.take(M * nkv * d * 4);
  w.vblk = k.take(M * nkv * d * 4);
  {
    const int wd = c->dtype == DFLASH_BF16;
    const int am = wd ? ACT_HILO : ACT_F32;
    const int Mi = (int)M, Hi = (int)H, Ii = (int)I, Nq = (int)(nq * d), Nqkv = (int)((nq + 2 * nkv) * d);
    size_t pb = 0;
    pb = std::max(pb, gemm_partial_bytes(gemm_plan(wd, am, Mi, Nqkv, Hi, EPI_STORE, false), Mi, Nqkv));
    pb = std::max(pb, gemm_partial_bytes(gemm_plan(wd, am, Mi, Hi, Nq, EPI_ADD, false), Mi, Hi));
    pb = std::max(pb, gemm_partial_bytes(gemm_plan(wd, am, Mi, 2 * Ii, Hi, EPI_SWIGLU, false), Mi, 2 * Ii));
    pb = std::max(pb, gemm_partial_bytes(gemm_plan(wd, am, Mi, Hi, Ii, EPI_ADD, false), Mi, Hi));
    if (wd) pb = std::max(pb, gemm_lmhead_part_bytes(Mi, c->vocab));   // LM head's last round of tiles
    w.gemm_part = k.take(pb);
    w.gemm_part_bytes = pb;
  }
  w.total = k.off;
  return w;
}

struct InjectWS {
  size_t f_hi, f_lo, cs, gemm_part, src, seq_c, pos_c, count, total;
};

// Split-K partial bytes per injected token (the fc and KV GEMMs run one after
// the other and share the region).
size_t inject_part_per_token(const dflash_config* c) {
  const int wd = c->dtype == DFLASH_BF16;
  const int H = c->hidden, FH = c->n_fuse * c->target_hidden;
  const int Nkv = c->n_layers * 2 * c->n_kv_heads * c->head_dim;
  const GemmPlan pf = gemm_plan(wd, wd ? ACT_BF16 : ACT_F32, 1, H, FH, EPI_STORE, true);
  const GemmPlan pk = gemm_plan(wd, wd ? ACT_HILO : ACT_F32, 1, Nkv, H, EPI_KVSCATTER, true);
  return std::max(gemm_partial_bytes(pf, 1, H), gemm_partial_bytes(pk, 1, Nkv));
}

InjectWS inject_layout(const dflash_config* c, int chunk) {
  InjectWS w{};
  const size_t el = c->dtype == DFLASH_BF16 ? 2 : 4;
  Carve k;
  w.f_hi = k.take((size_t)chunk * c->hidden * el);
  w.f_lo = k.take((size_t)chunk * c->hidden * el);
  w.cs = k.take((size_t)chunk * (c->head_dim / 2) * 8);
  w.gemm_part = k.take((size_t)chunk * inject_part_per_token(c));
  w.src = k.take((size_t)chunk * 4);
  w.seq_c = k.take((size_t)chunk * 4);
  w.pos_c = k.take((size_t)chunk * 4);
  w.count = k.take(4);
  w.total = k.off;
  return w;
}

// Injection chunk the workspace holds (rows of one fused-feature pass).
int inject_chunk_capacity(const dflash_config* c, size_t ws_bytes) {
  const size_t el = c->dtype == DFLASH_BF16 ? 2 : 4;
  const size_t per = 2 * c->hidden * el + (c->head_dim / 2) * 8 + inject_part_per_token(c) + 12;
  size_t n = ws_bytes / (per + 1);
  while (n > 0 && inject_layout(c, (int)std::min<size_t>(n, 1 << 30)).total > ws_bytes) n -= std::max<size_t>(1, n / 64);
  return (int)std::min<size_t>(n, 1 << 30);
}

char* at(void* ws, size_t off) { return (char*)ws + off; }

ActOut act_out(const dflash_config* c, void* hi, void* lo, int ld) {
  ActOut o;
  o.p0 = hi;
  o.p1 = lo;
  o.ld = ld;
  o.mode = c->dtype == DFLASH_BF16 ? ACT_HILO : ACT_F32;
  return o;
}
ActIn act_in(const ActOut& o) { return ActIn{o.p0, o.p1, o.ld, o.mode}; }

// ---------------------------------------------------------------- debug build
// Built with DFLASH_DEBUG, every call copies its device-resident indices to the
// host (on the call's stream, then synchronised) and checks them before
// anything is launched: a value outside its documented range returns
// DFLASH_EINVAL.  The release build trusts the caller (its kernels clamp or skip
// such values, so a bad index gives wrong numbers rather than a fault).
#ifdef DFLASH_DEBUG
bool dbg_fetch(std::vector<int32_t>& v, const int32_t* src, size_t n, hipStream_t s) {
  v.resize(n);
  if (n == 0) return true;
  if (hipMemcpyAsync(v.data(), src, n * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess) return false;
  return hipStreamSynchronize(s) == hipSuccess;
}

// ctx_len[b] in [0, ctx_cap]; the pages of positions [0, ctx_len[b] + extra) mapped
// to a physical page in [0, n_pages).
dflash_status dbg_context(const int32_t* ctx_len, int batch, int ctx_cap, int extra, const int32_t* table,
                          int max_pages, int n_pages, hipStream_t s) {
  std::vector<int32_t> c, t;
  if (!dbg_fetch(c, ctx_len, batch, s) || !dbg_fetch(t, table, (size_t)batch * max_pages, s)) return DFLASH_EHIP;
  for (int b = 0; b < batch; ++b) {
    if (c[b] < 0 || c[b] > ctx_cap) return DFLASH_EINVAL;
    const int pages = (c[b] + extra + 15) / 16;
    if (pages > max_pages) return DFLASH_EINVAL;
    for (int lp = 0; lp < pages; ++lp) {
      const int ph = t[(size_t)b * max_pages + lp];
      if (ph < 0 || ph >= n_pages) return DFLASH_EINVAL;
    }
  }
  return DFLASH_OK;
}

// Injection rows: tok_seq -1 (skip) or a sequence in [0, n_seqs) whose page of
// tok_pos is mapped to a physical page in [0, n_pages).
dflash_status dbg_inject(const int32_t* tok_seq, const int32_t* tok_pos, int n_tok, const int32_t* table,
                         int n_seqs, int max_pages, int n_pages, hipStream_t s) {
  std::vector<int32_t> q, p, t;
  if (!dbg_fetch(q, tok_seq, n_tok, s) || !dbg_fetch(p, tok_pos, n_tok, s) ||
      !dbg_fetch(t, table, (size_t)n_seqs * max_pages, s))
    return DFLASH_EHIP;
  for (int i = 0; i < n_tok; ++i) {
    if (q[i] == -1) continue;
    if (q[i] < 0 || q[i] >= n_seqs || p[i] < 0 || p[i] / 16 >= max_pages) return DFLASH_EINVAL;
    const int ph = t[(size_t)q[i] * max_pages + p[i] / 16];
    if (ph < 0 || ph >= n_pages) return DFLASH_EINVAL;
  }
  return DFLASH_OK;
}

// Every entry of a device int32 array in [lo, hi].
dflash_status dbg_range(const int32_t* v, size_t n, int lo, int hi, hipStream_t s) {
  std::vector<int32_t> h;
  if (!dbg_fetch(h, v, n, s)) return DFLASH_EHIP;
  for (int32_t x : h)
    if (x < lo || x > hi) return DFLASH_EINVAL;
  return DFLASH_OK;
}
#define DBG_CHECK(x)                                  \
  do {                                                \
    const dflash_status dbg_st_ = (x);                \
    if (dbg_st_ != DFLASH_OK) return dbg_st_;         \
  } while (0)
#else
#define DBG_CHECK(x) \
  do {               \
  } while (0)
#endif

#define HIP_TRY(x)                              \
  do {                                          \
    if ((x) != hipSuccess) return DFLASH_EHIP;  \
  } while (0)

// Block verification behind both verify entry points; prof: the timing hooks may
// record events around it (never for the allocation-free variant).
dflash_status verify_impl(int32_t batch, int32_t block_size, int32_t vocab, const float* target_logits,
                          const int32_t* draft_tokens, float temperature, const float* draft_logits,
                          const float* uniforms, int32_t* accept_len, int32_t* out_tokens, void* workspace,
                          size_t ws_bytes, hipStream_t stream, bool prof) {
  if (batch < 0 || vocab < 1) return DFLASH_EINVAL;
  if (block_size < 1 || block_size > 16) return DFLASH_ECAPACITY;
  if (!(temperature >= 0.f)) return DFLASH_EINVAL;
  if (batch == 0) return DFLASH_OK;
  if (!target_logits || !draft_tokens || !accept_len || !out_tokens) return DFLASH_EINVAL;
  if (temperature > 0.f && (!draft_logits || !uniforms)) return DFLASH_EINVAL;
  if (!workspace || ((uintptr_t)workspace & 255)) return DFLASH_EWORKSPACE;
  if (ws_bytes < verify_ws_bytes(batch, block_size, vocab)) return DFLASH_EWORKSPACE;
  DBG_CHECK(dbg_range(draft_tokens, (size_t)batch * block_size, 0, vocab - 1, stream));
  hipError_t e;
  if (prof) prof_mark(DFLASH_PROF_VERIFY, 0, stream);
  if (temperature > 0.f)
    e = launch_verify_sampled(batch, block_size, vocab, target_logits, draft_logits, draft_tokens, uniforms,
                              temperature, accept_len, out_tokens, workspace, stream);
  else
    e = launch_verify_greedy(batch, block_size, vocab, target_logits, draft_tokens, accept_len, out_tokens,
                             workspace, stream);
  if (prof) prof_mark(DFLASH_PROF_VERIFY, 1, stream);
  return e == hipSuccess ? DFLASH_OK : DFLASH_EHIP;
}

}  // namespace

// ---------------------------------------------------------------- static scratch
// Scratch of dflash_verify_block_static, for callers that cannot allocate: one
// array per GPU the library runs on, held until the process ends.  In host code
// the array's name only stands in for it; its device address is looked up with
// hipGetSymbolAddress once per device (with that device current) and that
// address is what the kernels receive.  The verify kernels write every scratch
// entry they read within the same call, so nothing needs clearing between calls.
constexpr size_t kVerifyScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kVerifyScratchBytes];
namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of this process's scratch on the current device.
hipError_t verify_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" {

const char* dflash_status_string(dflash_status s) {
  switch (s) {
    case DFLASH_OK: return "ok";
    case DFLASH_EINVAL: return "invalid argument";
    case DFLASH_ESHAPE: return "unsupported or inconsistent shape";
    case DFLASH_EDTYPE: return "unknown dtype";
    case DFLASH_ECAPACITY: return "capacity exceeded";
    case DFLASH_EWORKSPACE: return "workspace missing, misaligned or too small";
    case DFLASH_EHIP: return "HIP error";
  }
  return "unknown status";
}

size_t dflash_workspace_size(const dflash_config* cfg, int32_t max_batch, int32_t block_size,
                             int32_t max_inject_tokens, int32_t max_ctx_len) {
  if (check_cfg(cfg) != DFLASH_OK || max_batch < 0 || block_size < 1 || block_size > 32 || max_inject_tokens < 0 ||
      max_ctx_len < 0)
    return 0;
  size_t need = 256;
  for (int bt = 1; bt <= max_batch; ++bt) need = std::max(need, draft_layout(cfg, bt, block_size, max_ctx_len).total);
  if (max_inject_tokens > 0) need = std::max(need, inject_layout(cfg, max_inject_tokens).total);
  return need;
}

dflash_status dflash_inject_kv(const dflash_config* cfg, const dflash_weights* w, const void* target_hidden,
                               const int32_t* tok_seq, const int32_t* tok_pos, int32_t n_tok, void* kv_pool,
                               int32_t n_pages, const int32_t* block_table, int32_t n_seqs, int32_t max_pages,
                               void* workspace, size_t ws_bytes, hipStream_t stream) {
  dflash_status st = check_cfg(cfg);
  if (st != DFLASH_OK) return st;
  if ((st = check_weights(cfg, w, false)) != DFLASH_OK) return st;
  // one injection launch carries every layer's QK-norm key gains
  if (cfg->qk_norm && cfg->n_layers > kMaxQkLayers) return DFLASH_ECAPACITY;
  if (n_tok < 0 || n_pages < 0 || n_seqs < 0 || max_pages < 0) return DFLASH_EINVAL;
  if (n_tok == 0) return DFLASH_OK;
  if (!target_hidden || !tok_seq || !tok_pos || !kv_pool || !block_table) return DFLASH_EINVAL;
  if (!workspace || ((uintptr_t)workspace & 255)) return DFLASH_EWORKSPACE;
  const int chunk = inject_chunk_capacity(cfg, ws_bytes);
  if (chunk < 1) return DFLASH_EWORKSPACE;
  DBG_CHECK(dbg_inject(tok_seq, tok_pos, n_tok, block_table, n_seqs, max_pages, n_pages, stream));
  const InjectWS L = inject_layout(cfg, chunk);
  const int bf = cfg->dtype == DFLASH_BF16;
  const size_t el = bf ? 2 : 4;
  const int H = cfg->hidden, FH = cfg->n_fuse * cfg->target_hidden;
  const int d = cfg->head_dim, nkv = cfg->n_kv_heads;
  for (int t0 = 0; t0 < n_tok; t0 += chunk) {
    const int n = std::min(chunk, n_tok - t0);
    // bf16: the rows to write (tok_seq >= 0) are packed to the front on the
    // device, and both GEMMs stop at their count, so rows that are skipped
    // (a step loop's unaccepted block positions) cost no GEMM work.  Each row's
    // result depends only on its own inputs (fixed K split), so packing leaves
    // every written value unchanged.
    const int* seq = tok_seq + t0;
    const int* pos = tok_pos + t0;
    const int* rows = nullptr;
    const int* count = nullptr;
    if (bf) {
      int* src = (int*)at(workspace, L.src);
      int* seq_c = (int*)at(workspace, L.seq_c);
      int* pos_c = (int*)at(workspace, L.pos_c);
      int* cnt = (int*)at(workspace, L.count);
      HIP_TRY(launch_compact_rows(seq, pos, n, src, seq_c, pos_c, cnt, stream));
      seq = seq_c;
      pos = pos_c;
      rows = src;
      count = cnt;
    }
    HIP_TRY(launch_rope_table_tokens(pos, n, d, (double)cfg->rope_base, (float2*)at(workspace, L.cs), stream));
    GemmArgs g{};
    g.wdtype = bf;
    g.a = ActIn{(const char*)target_hidden + (size_t)t0 * FH * el, nullptr, FH, bf ? ACT_BF16 : ACT_F32, rows};
    g.m_dev = count;
    g.b = BRowsArgs{w->w_fc, nullptr, FH, 0, 0};
    g.M = n;
    g.N = H;
    g.K = FH;
    g.kind = EPI_STORE;
    g.fixed_split = true;
    g.part = (float*)at(workspace, L.gemm_part);
    const ActOut f = act_out(cfg, at(workspace, L.f_hi), at(workspace, L.f_lo), H);
    g.e.out = f;
    HIP_TRY(gemm(DFLASH_PROF_INJECT_FC, g, stream));

    GemmArgs k{};
    k.wdtype = bf;
    k.a = act_in(f);
    k.b = BRowsArgs{w->w_kv, nullptr, H, 0, 0};
    k.M = n;
    k.N = cfg->n_layers * 2 * nkv * d;
    k.K = H;
    k.kind = EPI_KVSCATTER;
    k.fixed_split = true;
    k.m_dev = count;
    k.part = (float*)at(workspace, L.gemm_part);
    k.e.pool = kv_pool;
    k.e.tok_seq = seq;
    k.e.tok_pos = pos;
    k.e.block_table = block_table;
    k.e.n_seqs = n_seqs;
    k.e.max_pages = max_pages;
    k.e.n_pages = n_pages;
    k.e.rope_cs = (const float2*)at(workspace, L.cs);
    k.e.n_layers = cfg->n_layers;
    k.e.n_kv = nkv;
    k.e.head_dim = d;
    k.e.k_norm_on = cfg->qk_norm;
    k.e.rms_eps = cfg->rms_eps;
    for (int l = 0; cfg->qk_norm && l < cfg->n_layers; ++l) k.e.k_gain[l] = w->k_norm[l];
    HIP_TRY(gemm(DFLASH_PROF_INJECT_KV, k, stream));
  }
  return DFLASH_OK;
}

// Activation buffers of one forward (all in the workspace).
struct FwdBufs {
  float* h;      // residual stream [M, H] fp32
  ActOut u, o, act;
  float* qkv;
  float* gpart;  // split-K partials
};

// Every layer of the model over the rows h [M, H] (M = batch * B tokens at
// positions ctx_len[b] + i): RMSNorm, q/k/v, attention of the block over the
// context pool plus the block keys (causal or not, ap.causal), O + residual,
// RMSNorm, SwiGLU, down + residual.  pending_ks returns the K split of the
// last down projection, whose partials the caller's final norm folds in.
// append_pool: also write each layer's block K/V into that pool (bf16, head_dim
// 128).  caps: per layer, where to store that layer's output (null p0: not
// stored); the last layer's output is stored by the caller's final norm.
static dflash_status run_layers(const dflash_config* cfg, const dflash_weights* w, AttnParams& ap,
                                const FwdBufs& fb, int M, int B, void* append_pool, const ActOut* caps,
                                int& pending_ks, hipStream_t stream) {
  const int bf = cfg->dtype == DFLASH_BF16;
  const int H = cfg->hidden, I = cfg->intermediate, d = cfg->head_dim, nq = cfg->n_q_heads, nkv = cfg->n_kv_heads;
  const int Nqkv = (nq + 2 * nkv) * d;
  float* h = fb.h;
  const ActOut u = fb.u, o = fb.o, act = fb.act;
  float* qkv = fb.qkv;
  float* gpart = fb.gpart;
  pending_ks = 0;   // K splits of a down projection whose partials the next norm folds in
  for (int l = 0; l < cfg->n_layers; ++l) {
    // the previous layer's down projection left its K-split partials to this norm
    // (and, when asked, stores that finished output of layer l-1)
    const ActOut* cap = (caps && l > 0 && caps[l - 1].p0) ? &caps[l - 1] : nullptr;
    HIP_TRY(launch_rmsnorm(h, w->attn_norm[l], u, M, H, cfg->rms_eps, nullptr, B, 0, nullptr, stream,
                           pending_ks > 1 ? gpart : nullptr, pending_ks, 0, cap));
    pending_ks = 0;
    GemmArgs g{};
    g.wdtype = bf;
    g.a = act_in(u);
    g.b = BRowsArgs{w->w_q[l], (const char*)w->w_kv + (size_t)l * 2 * nkv * d * H * (bf ? 2 : 4), H, nq * d, 1};
    g.M = M;
    g.N = Nqkv;
    g.part = gpart;
    g.K = H;
    g.kind = EPI_STORE;
    g.e.out = ActOut{qkv, nullptr, Nqkv, ACT_F32};
    // the query prep (bf16 pools, head_dim 128) sums a K split itself
    g.defer_reduce = bf && d == 128;
    const int ks_qkv = g.defer_reduce ? gemm_ksplit(g) : 1;
    ap.qkv_part = ks_qkv > 1 ? gpart : nullptr;
    ap.qkv_ks = ks_qkv;
    // QK-norm: the query prep applies it (bf16, head_dim 128); otherwise it runs in
    // place on the finished q/k rows before the attention kernels read them
    ap.q_gain = cfg->qk_norm ? w->q_norm[l] : nullptr;
    ap.k_gain = cfg->qk_norm ? w->k_norm[l] : nullptr;
    ap.rms_eps = cfg->rms_eps;
    HIP_TRY(gemm(DFLASH_PROF_GEMM_QKV, g, stream));
    if (cfg->qk_norm && !g.defer_reduce)
      HIP_TRY(launch_qk_norm(qkv, M, nq, nkv, d, ap.q_gain, ap.k_gain, cfg->rms_eps, stream));

    ap.layer = l;
    HIP_TRY(launch_attention(ap, bf, stream, g_prof.cls == DFLASH_PROF_ATTN ? prof_attn : nullptr));
    // target forward: this layer's block K/V (from the query prep) join the target's own cache
    if (append_pool)
      HIP_TRY(launch_kv_append(ap.kblk, ap.vblk, ap.ctx_len, ap.ctx_cap, append_pool, ap.n_pages, ap.block_table,
                               ap.max_pages, ap.batch, B, nkv, d, cfg->n_layers, l, stream));
    HIP_TRY(launch_attn_finish(ap, bf, o, stream));

    GemmArgs go{};
    go.wdtype = bf;
    go.a = act_in(o);
    go.b = BRowsArgs{w->w_o[l], nullptr, nq * d, 0, 0};
    go.M = M;
    go.N = H;
    go.part = gpart;
    go.K = nq * d;
    go.kind = EPI_ADD;
    go.e.resid = h;
    go.e.ldr = H;
    go.defer_reduce = true;   // folded into the MLP norm below
    const int ks_o = gemm_ksplit(go);
    HIP_TRY(gemm(DFLASH_PROF_GEMM_O, go, stream));

    HIP_TRY(launch_rmsnorm(h, w->mlp_norm[l], u, M, H, cfg->rms_eps, nullptr, B, 0, nullptr, stream,
                           ks_o > 1 ? gpart : nullptr, ks_o));
    GemmArgs gu{};
    gu.wdtype = bf;
    gu.a = act_in(u);
    gu.b = BRowsArgs{w->w_gate[l], w->w_up[l], H, 0, 2};
    gu.M = M;
    gu.N = 2 * I;
    gu.part = gpart;
    gu.K = H;
    gu.kind = EPI_SWIGLU;
    gu.e.out = act;
    HIP_TRY(gemm(DFLASH_PROF_GEMM_GATEUP, gu, stream));

    GemmArgs gd{};
    gd.wdtype = bf;
    gd.a = act_in(act);
    gd.b = BRowsArgs{w->w_down[l], nullptr, I, 0, 0};
    gd.M = M;
    gd.N = H;
    gd.part = gpart;
    gd.K = I;
    gd.kind = EPI_ADD;
    gd.e.resid = h;
    gd.e.ldr = H;
    gd.defer_reduce = true;   // folded into the next attention norm, or the final norm
    pending_ks = gemm_ksplit(gd);
    HIP_TRY(gemm(DFLASH_PROF_GEMM_DOWN, gd, stream));
  }
  return DFLASH_OK;
}

dflash_status dflash_draft_block(const dflash_config* cfg, const dflash_weights* w, const void* kv_pool,
                                 int32_t n_pages, const int32_t* block_table, int32_t max_pages,
                                 const int32_t* ctx_len, int32_t max_ctx_len, int32_t batch, int32_t block_size,
                                 int32_t n_steps, float temperature, uint64_t seed, const int32_t* anchor_tokens,
                                 int32_t* out_tokens, float* out_logits, float* out_conf, void* workspace,
                                 size_t ws_bytes, hipStream_t stream) {
  dflash_status st = check_cfg(cfg);
  if (st != DFLASH_OK) return st;
  if ((st = check_weights(cfg, w, true)) != DFLASH_OK) return st;
  if (batch < 0 || n_pages < 0 || max_pages < 0 || max_ctx_len < 0) return DFLASH_EINVAL;
  if (block_size < 1 || block_size > 16) return DFLASH_ECAPACITY;
  // an anchor takes block position 0, so B - 1 positions are left to denoise
  const int given = anchor_tokens ? 1 : 0;
  if (n_steps < 1 || n_steps > block_size - given) return DFLASH_EINVAL;
  if (!(temperature >= 0.f)) return DFLASH_EINVAL;
  if (batch == 0) return DFLASH_OK;
  if (!ctx_len || !out_tokens || !block_table || (!kv_pool && max_ctx_len > 0)) return DFLASH_EINVAL;
  if (!workspace || ((uintptr_t)workspace & 255)) return DFLASH_EWORKSPACE;
  const int ctx_cap = n_pages > 0 ? (int)std::min<long long>(max_ctx_len, (long long)max_pages * 16) : 0;
  const DraftWS L = draft_layout(cfg, batch, block_size, ctx_cap);
  if (L.total > ws_bytes) return DFLASH_EWORKSPACE;
  DBG_CHECK(dbg_context(ctx_len, batch, ctx_cap, 0, block_table, max_pages, n_pages, stream));
  if (anchor_tokens) DBG_CHECK(dbg_range(anchor_tokens, (size_t)batch, 0, cfg->vocab - 1, stream));

  const int bf = cfg->dtype == DFLASH_BF16;
  const int B = block_size, M = batch * B, S = n_steps;
  const int H = cfg->hidden, I = cfg->intermediate, d = cfg->head_dim, nq = cfg->n_q_heads, nkv = cfg->n_kv_heads;
  const int Nqkv = (nq + 2 * nkv) * d;
  float* h = (float*)at(workspace, L.h);
  const ActOut u = act_out(cfg, at(workspace, L.u_hi), at(workspace, L.u_lo), H);
  const ActOut o = act_out(cfg, at(workspace, L.o_hi), at(workspace, L.o_lo), nq * d);
  const ActOut act = act_out(cfg, at(workspace, L.act_hi), at(workspace, L.act_lo), I);
  ActOut y;
  y.p0 = at(workspace, L.y);
  y.p1 = nullptr;
  y.ld = H;
  y.mode = bf ? ACT_BF16 : ACT_F32;
  float* qkv = (float*)at(workspace, L.qkv);
  int* row_map = (int*)at(workspace, L.row_map);
  int* tau = (int*)at(workspace, L.tau);
  int* committed = (int*)at(workspace, L.committed);
  int* cand = (int*)at(workspace, L.cand);
  float* conf = (float*)at(workspace, L.conf);
  float2* cs = (float2*)at(workspace, L.cs);
  float* gpart = (float*)at(workspace, L.gemm_part);
  const FwdBufs fb{h, u, o, act, qkv, gpart};

  AttnParams ap{};
  ap.pool = kv_pool;
  ap.n_pages = n_pages;
  ap.block_table = block_table;
  ap.max_pages = max_pages;
  ap.ctx_len = ctx_len;
  ap.ctx_cap = ctx_cap;
  ap.qkv = qkv;
  ap.cs = cs;
  ap.batch = batch;
  ap.B = B;
  ap.nq = nq;
  ap.nkv = nkv;
  ap.d = d;
  ap.n_layers = cfg->n_layers;
  ap.scale = 1.0f / sqrtf((float)d);
  ap.n_splits = L.ns;
  ap.pps = L.pps;
  ap.part_o = (float*)at(workspace, L.att_o);
  ap.part_lse = (float*)at(workspace, L.att_lse);
  ap.q_hi = (bf16_t*)at(workspace, L.q_hi);
  ap.q_lo = (bf16_t*)at(workspace, L.q_lo);
  ap.kblk = (float*)at(workspace, L.kblk);
  ap.vblk = (float*)at(workspace, L.vblk);

  HIP_TRY(launch_rope_table_block(ctx_len, ctx_cap, batch, B, d, (double)cfg->rope_base, cs, stream));
  HIP_TRY(launch_block_init(tau, committed, M, B, cfg->mask_token_id, anchor_tokens, stream));

  // re-predict schedule: every open position takes its candidate at every step
  const bool repredict = cfg->denoise_schedule == DFLASH_SCHEDULE_REPREDICT;
  const int Bo = B - given;   // positions the steps denoise
  int done = given;
  for (int s = 0; s < S; ++s) {
    const int k_s = repredict ? Bo : ((s + 1) * Bo) / S - (s * Bo) / S;
    const int n_open = B - done;
    const int last = s == S - 1;
    HIP_TRY(launch_embed(tau, w->embed, bf, cfg->vocab, h, M, H, stream));
    int pending_ks = 0;   // K splits of the last down projection, folded by the final norm
    {
      const dflash_status rs = run_layers(cfg, w, ap, fb, M, B, nullptr, nullptr, pending_ks, stream);
      if (rs != DFLASH_OK) return rs;
    }
    const int Ms = batch * n_open;
    HIP_TRY(launch_rmsnorm(h, w->final_norm, y, Ms, H, cfg->rms_eps, committed, B, n_open, row_map, stream,
                           pending_ks > 1 ? gpart : nullptr, pending_ks, M));
    GemmArgs gl{};
    gl.wdtype = bf;
    gl.a = ActIn{y.p0, nullptr, H, y.mode};
    gl.b = BRowsArgs{w->lm_head, nullptr, H, 0, 0};
    gl.M = Ms;
    gl.N = cfg->vocab;
    gl.K = H;
    gl.kind = EPI_LMHEAD;
    gl.e.part_f = (float4*)at(workspace, L.part_f);
    gl.e.part_i = (int*)at(workspace, L.part_i);
    gl.e.ntiles = L.ntiles;
    gl.e.row_map = row_map;
    gl.e.logits = out_logits;
    gl.e.block = B;
    gl.e.temperature = temperature;
    gl.e.seed_lo = (uint32_t)(seed & 0xffffffffu);
    gl.e.seed_hi = (uint32_t)(seed >> 32);
    gl.e.step = s;
    gl.part = gpart;
    gl.part_cap = L.gemm_part_bytes;
    HIP_TRY(gemm(DFLASH_PROF_LMHEAD, gl, stream));
    HIP_TRY(launch_lm_combine(gl.e.part_f, gl.e.part_i, L.ntiles, Ms, row_map, cand, conf, stream));
    HIP_TRY(launch_commit(cand, conf, tau, committed, out_conf, out_tokens, batch, B, S, s, k_s, last, repredict,
                          stream));
    if (!repredict) done += k_s;
  }
  return DFLASH_OK;
}

dflash_status dflash_target_forward(const dflash_config* cfg, const dflash_weights* w, void* kv_pool,
                                    int32_t n_pages, const int32_t* block_table, int32_t max_pages,
                                    const int32_t* ctx_len, int32_t max_ctx_len, int32_t batch, int32_t n_tok,
                                    const int32_t* tokens, const int32_t* capture_layers, int32_t n_capture,
                                    float* out_logits, void* out_hidden, void* workspace, size_t ws_bytes,
                                    hipStream_t stream) {
  dflash_status st = check_cfg(cfg);
  if (st != DFLASH_OK) return st;
  if (cfg->dtype != DFLASH_BF16 || cfg->head_dim != 128) return DFLASH_ESHAPE;
  if (!w || !w->w_kv || !w->embed || !w->final_norm || !w->lm_head) return DFLASH_EINVAL;
  {
    const void* const* arrs[7] = {(const void* const*)w->attn_norm, w->w_q, w->w_o,
                                  (const void* const*)w->mlp_norm, w->w_gate, w->w_up, w->w_down};
    for (auto a : arrs) {
      if (!a) return DFLASH_EINVAL;
      for (int l = 0; l < cfg->n_layers; ++l)
        if (!a[l]) return DFLASH_EINVAL;
    }
    if (cfg->qk_norm) {
      if (!w->q_norm || !w->k_norm) return DFLASH_EINVAL;
      for (int l = 0; l < cfg->n_layers; ++l)
        if (!w->q_norm[l] || !w->k_norm[l]) return DFLASH_EINVAL;
    }
  }
  if (batch < 0 || n_pages < 0 || max_pages < 0 || max_ctx_len < 0 || n_capture < 0) return DFLASH_EINVAL;
  if (n_tok < 1 || n_tok > 32) return DFLASH_ECAPACITY;
  if (n_capture > 0 && (!capture_layers || !out_hidden)) return DFLASH_EINVAL;
  std::vector<ActOut> caps(cfg->n_layers);
  for (int f = 0; f < n_capture; ++f) {
    const int l = capture_layers[f];
    if (l < 0 || l >= cfg->n_layers || caps[l].p0) return DFLASH_EINVAL;   // out of range or repeated
    caps[l] = ActOut{(bf16_t*)out_hidden + (size_t)f * cfg->hidden, nullptr, n_capture * cfg->hidden, ACT_BF16};
  }
  if (batch == 0) return DFLASH_OK;
  if (!ctx_len || !tokens || !out_logits || !block_table || !kv_pool) return DFLASH_EINVAL;
  if (!workspace || ((uintptr_t)workspace & 255)) return DFLASH_EWORKSPACE;
  const int ctx_cap = n_pages > 0 ? (int)std::min<long long>(max_ctx_len, (long long)max_pages * 16) : 0;
  const int B = n_tok, M = batch * B;
  const DraftWS L = draft_layout(cfg, batch, B, ctx_cap);
  if (L.total > ws_bytes) return DFLASH_EWORKSPACE;
  DBG_CHECK(dbg_context(ctx_len, batch, ctx_cap, n_tok, block_table, max_pages, n_pages, stream));
  DBG_CHECK(dbg_range(tokens, (size_t)batch * n_tok, 0, cfg->vocab - 1, stream));
  const int H = cfg->hidden, d = cfg->head_dim, nq = cfg->n_q_heads, nkv = cfg->n_kv_heads;
  float* h = (float*)at(workspace, L.h);
  const FwdBufs fb{h, act_out(cfg, at(workspace, L.u_hi), at(workspace, L.u_lo), H),
                   act_out(cfg, at(workspace, L.o_hi), at(workspace, L.o_lo), nq * d),
                   act_out(cfg, at(workspace, L.act_hi), at(workspace, L.act_lo), cfg->intermediate),
                   (float*)at(workspace, L.qkv), (float*)at(workspace, L.gemm_part)};
  int* row_map = (int*)at(workspace, L.row_map);
  float2* cs = (float2*)at(workspace, L.cs);

  AttnParams ap{};
  ap.pool = kv_pool;
  ap.n_pages = n_pages;
  ap.block_table = block_table;
  ap.max_pages = max_pages;
  ap.ctx_len = ctx_len;
  ap.ctx_cap = ctx_cap;
  ap.qkv = fb.qkv;
  ap.cs = cs;
  ap.batch = batch;
  ap.B = B;
  ap.nq = nq;
  ap.nkv = nkv;
  ap.d = d;
  ap.n_layers = cfg->n_layers;
  ap.scale = 1.0f / sqrtf((float)d);
  ap.n_splits = L.ns;
  ap.pps = L.pps;
  ap.part_o = (float*)at(workspace, L.att_o);
  ap.part_lse = (float*)at(workspace, L.att_lse);
  ap.q_hi = (bf16_t*)at(workspace, L.q_hi);
  ap.q_lo = (bf16_t*)at(workspace, L.q_lo);
  ap.kblk = (float*)at(workspace, L.kblk);
  ap.vblk = (float*)at(workspace, L.vblk);
  ap.causal = 1;

  HIP_TRY(launch_rope_table_block(ctx_len, ctx_cap, batch, B, d, (double)cfg->rope_base, cs, stream));
  HIP_TRY(launch_embed(tokens, w->embed, 1, cfg->vocab, h, M, H, stream));
  int pending_ks = 0;
  {
    const dflash_status rs = run_layers(cfg, w, ap, fb, M, B, kv_pool, caps.data(), pending_ks, stream);
    if (rs != DFLASH_OK) return rs;
  }
  ActOut y{at(workspace, L.y), nullptr, H, ACT_BF16};
  const ActOut* last_cap = caps[cfg->n_layers - 1].p0 ? &caps[cfg->n_layers - 1] : nullptr;
  HIP_TRY(launch_rmsnorm(h, w->final_norm, y, M, H, cfg->rms_eps, nullptr, B, 0, row_map, stream,
                         pending_ks > 1 ? fb.gpart : nullptr, pending_ks, M, last_cap));
  GemmArgs gl{};
  gl.wdtype = 1;
  gl.a = ActIn{y.p0, nullptr, H, ACT_BF16};
  gl.b = BRowsArgs{w->lm_head, nullptr, H, 0, 0};
  gl.M = M;
  gl.N = cfg->vocab;
  gl.K = H;
  gl.kind = EPI_LMHEAD;
  gl.e.part_f = (float4*)at(workspace, L.part_f);
  gl.e.part_i = (int*)at(workspace, L.part_i);
  gl.e.ntiles = L.ntiles;
  gl.e.row_map = row_map;
  gl.e.logits = out_logits;
  gl.e.block = B;
  gl.e.temperature = 0.f;
  gl.part = fb.gpart;
  gl.part_cap = L.gemm_part_bytes;
  HIP_TRY(gemm(DFLASH_PROF_LMHEAD, gl, stream));
  return DFLASH_OK;
}

size_t dflash_verify_workspace_size(int32_t batch, int32_t block_size, int32_t vocab) {
  if (batch < 0 || block_size < 1 || block_size > 16 || vocab < 1) return 0;
  return verify_ws_bytes(batch, block_size, vocab);
}

dflash_status dflash_verify_block(int32_t batch, int32_t block_size, int32_t vocab, const float* target_logits,
                                  const int32_t* draft_tokens, float temperature, const float* draft_logits,
                                  const float* uniforms, int32_t* accept_len, int32_t* out_tokens,
                                  void* workspace, size_t ws_bytes, hipStream_t stream) {
  return verify_impl(batch, block_size, vocab, target_logits, draft_tokens, temperature, draft_logits, uniforms,
                     accept_len, out_tokens, workspace, ws_bytes, stream, true);
}

dflash_status dflash_verify_block_static(int32_t batch, int32_t block_size, int32_t vocab,
                                         const float* target_logits, const int32_t* draft_tokens, float temperature,
                                         const float* draft_logits, const float* uniforms, int32_t* accept_len,
                                         int32_t* out_tokens, hipStream_t stream) {
  if (batch < 0 || vocab < 1) return DFLASH_EINVAL;
  if (block_size < 1 || block_size > 16) return DFLASH_ECAPACITY;
  if (verify_ws_bytes(batch, block_size, vocab) > kVerifyScratchBytes) return DFLASH_ECAPACITY;
  void* ws = nullptr;
  if (verify_scratch(&ws) != hipSuccess) return DFLASH_EHIP;
  return verify_impl(batch, block_size, vocab, target_logits, draft_tokens, temperature, draft_logits, uniforms,
                     accept_len, out_tokens, ws, kVerifyScratchBytes, stream, false);
}

int32_t dflash_adaptive_block_size(const int32_t* accept_len, const int32_t* block_of, int32_t n_obs,
                                   const int32_t* cand_block, const float* step_time, int32_t n_cand,
                                   float prior_a, float prior_b, float* p_match) {
  if (n_obs < 0 || n_cand < 1 || !cand_block || !step_time) return DFLASH_EINVAL;
  if (n_obs > 0 && (!accept_len || !block_of)) return DFLASH_EINVAL;
  if (!(prior_a >= 0.f) || !(prior_b >= 0.f)) return DFLASH_EINVAL;
  // maximum-likelihood match probability of the truncated-geometric acceptances
  double matches = prior_a, misses = prior_b;
  for (int32_t i = 0; i < n_obs; ++i) {
    const int32_t a = accept_len[i], b = block_of[i];
    if (b < 1 || b > 16) return DFLASH_ECAPACITY;
    if (a < 0 || a > b) return DFLASH_EINVAL;
    matches += a;
    misses += a < b ? 1.0 : 0.0;
  }
  const double p = matches + misses > 0.0 ? matches / (matches + misses) : 0.5;
  if (p_match) *p_match = (float)p;
  int32_t best = -1;
  double best_rate = -1.0;
  for (int32_t j = 0; j < n_cand; ++j) {
    const int32_t B = cand_block[j];
    if (B < 1 || B > 16) return DFLASH_ECAPACITY;
    if (!(step_time[j] > 0.f)) return DFLASH_EINVAL;
    double e = 0.0, pk = 1.0;   // 1 + p + ... + p^B
    for (int32_t k = 0; k <= B; ++k) {
      e += pk;
      pk *= p;
    }
    const double rate = e / (double)step_time[j];
    if (rate > best_rate || (rate == best_rate && B < best)) {
      best_rate = rate;
      best = B;
    }
  }
  return best;
}

dflash_status dflash_advance_context(int32_t batch, int32_t block_size, const int32_t* accept_len,
                                     int32_t* ctx_len, int32_t* tok_seq, int32_t* tok_pos, hipStream_t stream) {
  if (batch < 0) return DFLASH_EINVAL;
  if (block_size < 1 || block_size > 16) return DFLASH_ECAPACITY;
  if (batch == 0) return DFLASH_OK;
  if (!accept_len || !ctx_len || !tok_seq || !tok_pos) return DFLASH_EINVAL;
  DBG_CHECK(dbg_range(accept_len, (size_t)batch, 0, block_size, stream));
  DBG_CHECK(dbg_range(ctx_len, (size_t)batch, 0, INT32_MAX - block_size - 1, stream));
  return launch_advance_context(batch, block_size, accept_len, ctx_len, tok_seq, tok_pos, stream) == hipSuccess
             ? DFLASH_OK
             : DFLASH_EHIP;
}

dflash_status dflash_prof_select(int32_t kernel_class) {
  if (kernel_class < DFLASH_PROF_NONE || kernel_class > DFLASH_PROF_VERIFY) return DFLASH_EINVAL;
  g_prof.cls.store(kernel_class, std::memory_order_relaxed);
  return DFLASH_OK;
}

dflash_status dflash_prof_collect(float* total_ms, int32_t* n_launches) {
  if (!total_ms || !n_launches) return DFLASH_EINVAL;
  std::lock_guard<std::mutex> lock(g_prof.mu);
  double tot = 0.0;
  for (auto& pr : g_prof.recorded) {
    if (hipEventSynchronize(pr.second) != hipSuccess) return DFLASH_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess) return DFLASH_EHIP;
    tot += ms;
  }
  *total_ms = (float)tot;
  *n_launches = (int32_t)g_prof.recorded.size();
  g_prof.recorded.clear();
  g_prof.open = nullptr;
  g_prof.used = 0;
  return DFLASH_OK;
}

}  // extern "C"
