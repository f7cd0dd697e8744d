// Attention of the draft block over the injected context KV plus the block's
// own keys (every block query sees every context key and every block key).
//
// The work is split flash-decoding style: each context split (a run of
// pages of one sequence and one kv head) and one extra "block" split (the B
// in-block keys) produce a normalised partial output and its log-sum-exp;
// a combine kernel merges the splits in a fixed order (deterministic).
//
// bf16 pool, context splits: MFMA.  Per 32-token tile (two pages) one wave
// computes S^T = K Q^T (A = K rows from LDS, B = the wave's 16 queries kept
// in registers as hi/lo bf16), so each lane owns query (lane % 16) and 8
// tokens; the online-softmax probabilities are then already the B operand
// of O^T = V^T P^T, whose A operand comes from the dimension-major V page
// (one 16-byte LDS read per fragment, no transpose).  P is split hi/lo too.
// fp32 pool and the in-block split: a VALU kernel, four lanes per query row.
#include <algorithm>
#include <type_traits>

#include "kernels.h"

namespace dflash {

__device__ __forceinline__ int clamp_ctx(const AttnParams& p, int b) {
  int c = p.ctx_len[b];
  const int cap = min(p.ctx_cap, p.max_pages * 16);
  return c < 0 ? 0 : (c > cap ? cap : c);
}

__device__ __forceinline__ int phys_page(const AttnParams& p, int b, int lp) {
  const int ph = p.block_table[(size_t)b * p.max_pages + lp];
  return (ph >= 0 && ph < p.n_pages) ? ph : -1;
}

// Rotated query / block-key element dd of a head vector (rotate-half pairing).
__device__ __forceinline__ float rope_elem(const float* v, const float2* cs, int dd, int D) {
  const int h = D / 2;
  const float2 c = cs[dd < h ? dd : dd - h];
  return dd < h ? v[dd] * c.x - v[dd + h] * c.y : v[dd] * c.x + v[dd - h] * c.y;
}

// Pages [pg0, pg1) of context split `split` of a sequence with npages pages:
// the sequence's 32-token tiles are dealt evenly to the n_splits splits (so
// the splits of every sequence are balanced whatever bound the grid was sized
// for); at most p.pps pages per split.
__device__ __forceinline__ void split_pages(const AttnParams& p, int npages, int split, int& pg0, int& pg1) {
  const int tiles = (npages + 1) >> 1;
  const int tps = (tiles + p.n_splits - 1) / p.n_splits;
  pg0 = min(2 * split * tps, npages);
  pg1 = min(pg0 + 2 * tps, npages);
}

// ---------------------------------------------------------------------------
constexpr int kMaxPPS = 512;   // pages per context split (bounded by the host)
constexpr int kCachePolicyNT = 2;   // cache-policy operand of the direct loads: non-temporal
constexpr int kAttStages = 5;   // 32-token tiles resident per four-wave workgroup (two fill the 160 KiB of LDS)

// s_waitcnt on the vector-memory counter only, through the builtin so that
// the compiler's own wait insertion knows which loads have completed
// (vmcnt bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void att_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Barrier without the memory fence of __syncthreads(): the fence would also
// wait for the later tiles' loads still in flight.  Each wave waits for its
// own copies of the current tile (vmcnt) before arriving.
__device__ __forceinline__ void att_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Rotated queries of every (sequence, kv head) group as (hi, lo) bf16 planes
// in [b][kv head][r][d] order, r = j*B + i for head m*g + j and block
// position i: the context kernel then loads its MFMA operands directly.  The
// queries carry the softmax scale times log2 e, so the scores come out ready
// for the base-2 exponential.  The rotated block keys and the block values
// (fp32) are written too, [b][kv head][i][d], for the in-block part of the
// attention.  When the q/k/v projection left K-split partials, they are
// summed here in split order (the sums a separate reduction would form).
// The quads of a head row at off (dims 4e ..) and off + h (their rotate-half
// partners), each summed over the K-split partials in split order.  Up to
// kQkvMaxSplit partials of both quads are loaded before the first add, so
// their loads are in flight together; more are folded one at a time.
constexpr int kQkvMaxSplit = 8;
__device__ __forceinline__ void qkv_quads(const AttnParams& p, size_t off, size_t h, size_t plane, float4& x0,
                                          float4& x1) {
  if (p.qkv_ks <= 1) {
    x0 = *(const float4*)(p.qkv + off);
    x1 = *(const float4*)(p.qkv + off + h);
    return;
  }
  x0 = make_float4(0.f, 0.f, 0.f, 0.f);
  x1 = x0;
  auto add = [](float4& a, const float4& v) {
    a.x += v.x;
    a.y += v.y;
    a.z += v.z;
    a.w += v.w;
  };
  if (p.qkv_ks <= kQkvMaxSplit) {
    float4 v0[kQkvMaxSplit], v1[kQkvMaxSplit];
#pragma unroll
    for (int s = 0; s < kQkvMaxSplit; ++s) {
      v0[s] = s < p.qkv_ks ? *(const float4*)(p.qkv_part + s * plane + off) : make_float4(0.f, 0.f, 0.f, 0.f);
      v1[s] = s < p.qkv_ks ? *(const float4*)(p.qkv_part + s * plane + off + h) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int s = 0; s < kQkvMaxSplit; ++s)
      if (s < p.qkv_ks) {
        add(x0, v0[s]);
        add(x1, v1[s]);
      }
    return;
  }
  for (int s = 0; s < p.qkv_ks; ++s) {
    add(x0, *(const float4*)(p.qkv_part + s * plane + off));
    add(x1, *(const float4*)(p.qkv_part + s * plane + off + h));
  }
}

// Rotate-half RoPE of four consecutive first-half dims x0 (4e .. 4e+3) and
// their partners x1 (h+4e ..): y0 = x0 cos - x1 sin, y1 = x1 cos + x0 sin.
__device__ __forceinline__ void rope4(const float4& x0, const float4& x1, const float4& c01, const float4& c23,
                                      float4& y0, float4& y1) {
  y0 = make_float4(x0.x * c01.x - x1.x * c01.y, x0.y * c01.z - x1.y * c01.w, x0.z * c23.x - x1.z * c23.y,
                   x0.w * c23.z - x1.w * c23.w);
  y1 = make_float4(x1.x * c01.x + x0.x * c01.y, x1.y * c01.z + x0.y * c01.w, x1.z * c23.x + x0.z * c23.y,
                   x1.w * c23.z + x0.w * c23.w);
}

// QK-norm of one head row spread over TPR consecutive lanes (dims 4e..4e+3 in
// x0 and their rotate-half partners in x1): x * gain / rms(x).
template <int TPR, int D>
__device__ __forceinline__ void head_rmsnorm(float4& x0, float4& x1, const float* gain, int e, float eps) {
  float ss = x0.x * x0.x + x0.y * x0.y + x0.z * x0.z + x0.w * x0.w + x1.x * x1.x + x1.y * x1.y + x1.z * x1.z +
             x1.w * x1.w;
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) ss += __shfl_xor(ss, o, kWave);
  const float inv = 1.f / sqrtf(ss / (float)D + eps);
  const float4 g0 = *(const float4*)(gain + 4 * e), g1 = *(const float4*)(gain + D / 2 + 4 * e);
  x0 = make_float4(x0.x * inv * g0.x, x0.y * inv * g0.y, x0.z * inv * g0.z, x0.w * inv * g0.w);
  x1 = make_float4(x1.x * inv * g1.x, x1.y * inv * g1.y, x1.z * inv * g1.z, x1.w * inv * g1.w);
}

template <int D>
__global__ __launch_bounds__(256) void attn_qprep_kernel(AttnParams p) {
  // D/8 threads per row; thread e covers dims 4e .. 4e+3 and their
  // rotate-half partners h+4e .. h+4e+3.  Row slots u < R are queries, then
  // B block keys, then B block values, so every workgroup does equal work.
  constexpr int TPR = D / 8, RPB = 256 / TPR, h = D / 2;
  const int g = p.nq / p.nkv, R = g * p.B;
  const int ldq = (p.nq + 2 * p.nkv) * D;
  const size_t plane = (size_t)p.batch * p.B * ldq;
  const int e = threadIdx.x % TPR, u = blockIdx.x * RPB + threadIdx.x / TPR;
  const int m = blockIdx.y, b = blockIdx.z;
  if (u >= R + 2 * p.B) return;
  if (u < R) {
    const float qscale = p.scale * 1.4426950408889634f;   // scores come out in base-2 units
    const int r = u, j = r / p.B, i = r - j * p.B, row = b * p.B + i, n = m * g + j;
    const size_t off = (size_t)row * ldq + n * D + 4 * e;
    float4 x0, x1;
    qkv_quads(p, off, h, plane, x0, x1);
    if (p.q_gain) head_rmsnorm<TPR, D>(x0, x1, p.q_gain, e, p.rms_eps);
    const float4* cs = (const float4*)(p.cs + (size_t)row * h + 4 * e);   // (cos, sin) of dims 4e .. 4e+3
    float4 y0, y1;
    rope4(x0, x1, cs[0], cs[1], y0, y1);
    uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
    split_hilo2(y0.x * qscale, y0.y * qscale, h0, l0);
    split_hilo2(y0.z * qscale, y0.w * qscale, h1, l1);
    split_hilo2(y1.x * qscale, y1.y * qscale, h2, l2);
    split_hilo2(y1.z * qscale, y1.w * qscale, h3, l3);
    const size_t gr = (((size_t)b * p.nkv + m) * R + r) * (D / 2);   // in 32-bit words
    *(u32x2*)((uint32_t*)p.q_hi + gr + 2 * e) = u32x2{h0, h1};
    *(u32x2*)((uint32_t*)p.q_lo + gr + 2 * e) = u32x2{l0, l1};
    *(u32x2*)((uint32_t*)p.q_hi + gr + h / 2 + 2 * e) = u32x2{h2, h3};
    *(u32x2*)((uint32_t*)p.q_lo + gr + h / 2 + 2 * e) = u32x2{l2, l3};
    return;
  }
  const bool is_k = u < R + p.B;
  const int r = is_k ? u - R : u - R - p.B;   // block position
  const int krow = b * p.B + r;
  const size_t off = (size_t)krow * ldq + (p.nq + (is_k ? 0 : p.nkv)) * D + m * D + 4 * e;
  float4 x0, x1;
  qkv_quads(p, off, h, plane, x0, x1);
  const size_t o = (((size_t)b * p.nkv + m) * p.B + r) * D + 4 * e;
  if (is_k) {   // rotated key (QK-normed first when asked)
    if (p.k_gain) head_rmsnorm<TPR, D>(x0, x1, p.k_gain, e, p.rms_eps);
    const float4* cs = (const float4*)(p.cs + (size_t)krow * h + 4 * e);
    float4 y0, y1;
    rope4(x0, x1, cs[0], cs[1], y0, y1);
    *(float4*)(p.kblk + o) = y0;
    *(float4*)(p.kblk + o + h) = y1;
  } else {
    *(float4*)(p.vblk + o) = x0;
    *(float4*)(p.vblk + o + h) = x1;
  }
}

// Context part of the block attention, one (context split, kv head, sequence,
// query group) per workgroup of NW waves, 16 query rows per wave: four waves
// (64 rows, two workgroups per CU, kAttStages tiles each) or, when a kv head
// has more than 64 query rows (a target forward over a block and the token
// before it), eight waves (128 rows, one workgroup per CU, twice the tiles),
// so that the context is streamed once for all of them.  Tiles of 32 tokens
// (two pages: K 2 x 4 KiB, V 2 x 4 KiB) are copied global -> LDS by
// global_load_lds_dwordx4 (lane i of an instruction fills LDS bytes
// base + 16 i); wave w copies part w / 4 of page w & 1 of the tile, K for
// w % 4 < 2 and V otherwise, so it needs one physical page per tile.  The split's
// page ids come from the block table once, into registers (lane j holds tile
// j + 64 r), and a lane read picks a tile's page at its issue; unmapped pages
// become wave-uniform bit masks.  The loop has no LDS round trip besides the
// operand reads.
//
// Within a tile, MFMA block t (t = 0, 1) of S^T = K Q^T takes the 16 tokens
// 8(r / 4) + 4t + (r % 4), r = 0..15: lane (gq, q) then holds the scores of
// tokens 8 gq .. 8 gq + 7 in order, which are also the 8 consecutive tokens
// its V^T operand needs (one 16-byte read of a V row).  K rows (256 B) keep
// chunk c at c ^ kswz(row), so the sixteen rows one operand read touches land
// on distinct bank groups; V rows (32 B) keep their two halves in place: a
// probe of the shader sequencer's bank-conflict counter finds the 16-row V
// read conflict-free laid out so, and 2-way conflicted when the halves of rows
// d and d + 8 are swapped.
__device__ __forceinline__ int kswz(int krow) { return (krow & 15) ^ (((krow >> 4) & 1) << 2); }

// Maximum over lanes l, l ^ 16, l ^ 32 and l ^ 48 (lane swaps across the
// 32-lane halves and the 16-lane rows, no LDS traffic).
__device__ __forceinline__ float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

constexpr int kPidRegs = kMaxPPS / 128;   // page-id registers per wave (64 tiles of two pages each)

// vmcnt wait for a tile with k later tiles of PT copies each still in flight
template <int PT, int MAXK>
__device__ __forceinline__ void att_wait_tiles(int k) {
  if constexpr (MAXK == 0) {
    att_wait_vmcnt<0>();
  } else {
    if (k >= MAXK) att_wait_vmcnt<MAXK * PT>();
    else att_wait_tiles<PT, MAXK - 1>(k);
  }
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void attn_ctx_mfma_kernel(AttnParams p) {
  static_assert(D == 128, "context kernel is specialised for head_dim 128");
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  constexpr int STAGES = NW == 8 ? 2 * kAttStages : kAttStages;   // tiles resident (LDS of one CU either way)
  constexpr int QG = 16 * NW;                 // query rows per workgroup
  static_assert(STAGES >= 2 && STAGES <= 10, "stages");
  static_assert(kPidRegs == 4, "page-id register select");
  constexpr int KK = D / 32, NN = D / 16;
  constexpr int KBYTES = 32 * D * 2;          // K tile: 32 tokens x 256 B
  constexpr int VBYTES = 2 * D * 32;          // V tile: 2 pages x D rows x 32 B
  constexpr int TILE = KBYTES + VBYTES;       // 16 KiB
  constexpr int PER_THREAD = TILE / 1024 / NW; // load instructions per wave per tile
  static_assert(STAGES * TILE <= 160 * 1024, "LDS");
  static_assert((STAGES - 1) * PER_THREAD < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[STAGES * TILE];

  const int g = p.nq / p.nkv, R = g * p.B;
  const int nqg = (R + QG - 1) / QG;
  const int split = blockIdx.x / nqg, qg = blockIdx.x - split * nqg;
  const int m = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int ctx = clamp_ctx(p, b);
  const int npages = (ctx + 15) >> 4;
  int pg0, pg1;
  split_pages(p, npages, split, pg0, pg1);
  const int ntiles = pg1 > pg0 ? (pg1 - pg0 + 1) >> 1 : 0;

  const int r = qg * QG + wid * 16 + (lane & 15);
  const bool rvalid = r < R;
  const bool wave_active = qg * QG + wid * 16 < R;
  const int j = rvalid ? r / p.B : 0, i = rvalid ? r - (r / p.B) * p.B : 0;
  const int n = m * g + j, row = b * p.B + i;

  bf16x8 qh[KK], ql[KK];
  {
    const size_t qoff = (((size_t)b * p.nkv + m) * R + (rvalid ? r : 0)) * D + 8 * (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qh[kk] = as_bf16x8(rvalid ? *(const u32x4*)(p.q_hi + qoff + 32 * kk) : z);
      ql[kk] = as_bf16x8(rvalid ? *(const u32x4*)(p.q_lo + qoff + 32 * kk) : z);
    }
  }
  // page ids: page q (0, 1) of tile t = lane + 64 rr, -1 past the split or unmapped;
  // any_bad (wave-uniform): some page of the split has no valid physical page
  const int wid_u = __builtin_amdgcn_readfirstlane(wid);
  const int wrole = wid_u & 3, wpart = wid_u >> 2;   // copy role (K0, K1, V0, V1) and its part
  const int wpage = wrole & 1;
  int mypid[kPidRegs];
  int pid00 = -1;
  bool any_bad = false;
#pragma unroll
  for (int rr = 0; rr < kPidRegs; ++rr) {
    int ph0 = -1, ph1 = -1;
    if (64 * rr < ntiles) {
      const int pp = pg0 + 2 * (lane + 64 * rr);
      if (pp < pg1) ph0 = phys_page(p, b, pp);
      if (pp + 1 < pg1) ph1 = phys_page(p, b, pp + 1);
      any_bad |= __ballot((pp < pg1 && ph0 < 0) || (pp + 1 < pg1 && ph1 < 0)) != 0;
    }
    mypid[rr] = wpage ? ph1 : ph0;
    if (rr == 0) pid00 = __builtin_amdgcn_readlane(ph0, 0);
  }
  att_wait_vmcnt<0>();   // query fragments and page ids loaded (before any tile copy is in flight)

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 ot[NN];
#pragma unroll
  for (int nn = 0; nn < NN; ++nn) ot[nn] = f32x4{0.f, 0.f, 0.f, 0.f};

  // page-major pool: page ph holds [layer][K, V][kv head] chunks
  const size_t chunk = 16 * D;
  const size_t page_stride = (size_t)p.n_layers * 2 * p.nkv * chunk;
  const bf16_t* kbase = (const bf16_t*)p.pool + ((size_t)p.layer * 2 * p.nkv + m) * chunk;
  const bf16_t* vbase = kbase + (size_t)p.nkv * chunk;
  const uint32_t lds0 = (uint32_t)(size_t)lds;
  // stand-in source for masked pages: the split's first page, else page 0
  // (the host only attends to a context when the pool has at least one page)
  const int first_ph = (ntiles && pid00 >= 0) ? pid00 : 0;

  // copy role of this wave and the per-lane byte offsets of its PER_THREAD
  // loads within a page chunk (instruction ins = 4 wrole + qq, qq = the
  // wave's part * PER_THREAD + q, fills LDS bytes ins * 1024 .. + 1023 of the tile)
  const bf16_t* srcbase = wrole < 2 ? kbase : vbase;
  uint32_t loff[PER_THREAD];
#pragma unroll
  for (int q = 0; q < PER_THREAD; ++q) {
    const int qq = wpart * PER_THREAD + q;
    if (wrole < 2) {
      const int krow = 16 * wpage + 4 * qq + (lane >> 4);
      const int lc = (lane & 15) ^ kswz(krow);
      loff[q] = (uint32_t)((krow & 15) * (D * 2) + lc * 16);
    } else {
      const int d = 32 * qq + (lane >> 1);
      const int lh = lane & 1;
      loff[q] = (uint32_t)(d * 32 + lh * 16);
    }
  }
  // physical page this wave copies for tile t (uniform): past the split, or
  // without a valid index, the stand-in page is read (its tokens are masked out)
  auto page_of = [&](int t) __attribute__((always_inline)) {
    if (t >= ntiles) return first_ph;
    const int rr = t >> 6;
    const int v = rr == 0 ? mypid[0] : rr == 1 ? mypid[1] : rr == 2 ? mypid[2] : mypid[3];
    const int ph = __builtin_amdgcn_readlane(v, t & 63);
    return ph >= 0 ? ph : first_ph;
  };
  // page q (0, 1) of tile t lies in the split but has no valid physical page:
  // its tokens are skipped (scores masked, values zeroed), as the VALU path does
  auto unmapped = [&](int t, int q) __attribute__((always_inline)) {
    if (!any_bad) return false;   // the usual case: no table read in the loop
    const int pp = pg0 + 2 * t + q;
    return pp < pg1 && phys_page(p, b, pp) < 0;
  };
  // The pool is streamed once per layer and forward: its copies carry the
  // non-temporal hint (nt), which measured about 8% faster than the default
  // policy on the 8B-shaped batch-32 workload (117-120 against 128 us).
  auto issue = [&](int ph, int st) __attribute__((always_inline)) {
    const char* base = (const char*)(srcbase + (size_t)__builtin_amdgcn_readfirstlane(ph) * page_stride);
#pragma unroll
    for (int q = 0; q < PER_THREAD; ++q)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(base + loff[q]),
                                       (__attribute__((address_space(3))) void*)(size_t)(lds0 + st * TILE +
                                                     (4 * wrole + wpart * PER_THREAD + q) * 1024),
                                       16, 0, kCachePolicyNT);
  };

  // loop-invariant LDS operand offsets of this lane
  int koff[2][KK], voff[NN];
  {
    const int rr = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int krow = 8 * (rr >> 2) + 4 * t + (rr & 3);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) koff[t][kk] = krow * (D * 2) + (((4 * kk + gq) ^ kswz(krow)) << 4);
    }
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      const int d = 16 * nn + rr;
      voff[nn] = (gq >> 1) * (D * 32) + d * 32 + ((gq & 1) << 4);
    }
  }
  const int tok_end = min(ctx, pg1 * 16);
  const int tl = 8 * (lane >> 4);   // first of this lane's 8 tokens in a tile

  // V slots at or past the context end may hold anything (a page never
  // written), and so may the stand-in page read for an unmapped one; they are
  // zeroed so that P = 0 meets V = 0.
  auto zero_tail = [&](int t) __attribute__((always_inline)) {
    const int tok0 = (pg0 + 2 * t) * 16;
    const bool bad0 = unmapped(t, 0), bad1 = unmapped(t, 1);
    if (tok0 + 32 > ctx || bad0 || bad1) {
      unsigned char* vt = lds + (t % STAGES) * TILE + KBYTES;
      for (int c = tid; c < 2 * D * 16; c += 64 * NW) {
        const int pg = c / (D * 16), rem = c - pg * D * 16, d = rem >> 4, slot = rem & 15;
        if (tok0 + pg * 16 + slot >= ctx || (pg ? bad1 : bad0)) {
          const int lh = slot >> 3;
          *(bf16_t*)(vt + pg * (D * 32) + d * 32 + lh * 16 + (slot & 7) * 2) = 0;
        }
      }
      __syncthreads();
    }
  };
#define ATT_SCORES(T, O0, O1)                                                                                 \
  do {                                                                                                        \
    const unsigned char* kt_ = lds + ((T) % STAGES) * TILE;                                                   \
    O0 = f32x4{0.f, 0.f, 0.f, 0.f};                                                                           \
    O1 = f32x4{0.f, 0.f, 0.f, 0.f};                                                                           \
    _Pragma("unroll") for (int kk = 0; kk < KK; ++kk) {                                                       \
      const bf16x8 a0_ = as_bf16x8(*(const u32x4*)(kt_ + koff[0][kk]));                                       \
      const bf16x8 a1_ = as_bf16x8(*(const u32x4*)(kt_ + koff[1][kk]));                                       \
      O0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0_, qh[kk], O0, 0, 0, 0);                                 \
      O1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1_, qh[kk], O1, 0, 0, 0);                                 \
      O0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0_, ql[kk], O0, 0, 0, 0);                                 \
      O1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1_, ql[kk], O1, 0, 0, 0);                                 \
    }                                                                                                         \
  } while (0)
#define ATT_READ_V(T, VF)                                                                                     \
  do {                                                                                                        \
    const unsigned char* vt_ = lds + ((T) % STAGES) * TILE + KBYTES;                                          \
    _Pragma("unroll") for (int nn = 0; nn < NN; ++nn) VF[nn] = as_bf16x8(*(const u32x4*)(vt_ + voff[nn]));    \
  } while (0)

  // Software pipeline: iteration it waits for tile it+1, computes its scores
  // (MFMA) and then the softmax and P V of tile it, whose scores were computed
  // one iteration earlier, so the matrix and vector work of neighbouring tiles
  // overlap inside a wave.  Tile it+1's V fragments are read at the end of
  // iteration it, so they arrive during the next wait and barrier.  Tile it-1's
  // buffer is refilled after the barrier of iteration it (every wave is past its
  // P V by then).
  int issued = 0;   // tiles issued so far
#pragma unroll
  for (int t = 0; t < STAGES; ++t)
    if (t < ntiles) { issue(page_of(t), t); ++issued; }
  auto wait_tile = [&](int t) __attribute__((always_inline)) {
    att_wait_tiles<PER_THREAD, STAGES - 1>(issued - 1 - t);   // tiles issued after tile t
  };

  f32x4 stc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  bf16x8 vf[NN];
  if (ntiles > 0) {
    wait_tile(0);
    att_barrier();
    zero_tail(0);
    if (wave_active) {
      ATT_SCORES(0, stc[0], stc[1]);
      ATT_READ_V(0, vf);
    }
  }
  // One iteration.  FAST: tiles it and it+1 are whole and every page of the
  // split is mapped, so no score is masked and no tail is zeroed; the leading
  // iterations of a split run so, the last ones (and every iteration of a split
  // with an unmapped page) take the general path.
  auto step = [&](int it, auto fast_c) __attribute__((always_inline)) {
    constexpr bool FAST = decltype(fast_c)::value;
    const bool more = FAST || it + 1 < ntiles;
    if (more) {
      wait_tile(it + 1);
      att_barrier();
      if (it >= 1 && issued < ntiles) {
        issue(page_of(issued), (it - 1) % STAGES);   // tile it+STAGES-1 into tile it-1's buffer
        ++issued;
      }
      if constexpr (!FAST) zero_tail(it + 1);
    }
    if (wave_active) {
      // K of tile it+1 (stale and unused after the last tile)
      bf16x8 kf[2][KK];
      {
        const unsigned char* kt = lds + ((it + 1) % STAGES) * TILE;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          kf[0][kk] = as_bf16x8(*(const u32x4*)(kt + koff[0][kk]));
          kf[1][kk] = as_bf16x8(*(const u32x4*)(kt + koff[1][kk]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // scores of tile it+1 (garbage after the last tile, never used); the
      // matrix cores run them while the softmax below runs on the VALU
      f32x4 stn[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        stn[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][kk], qh[kk], stn[0], 0, 0, 0);
        stn[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][kk], qh[kk], stn[1], 0, 0, 0);
        stn[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][kk], ql[kk], stn[0], 0, 0, 0);
        stn[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][kk], ql[kk], stn[1], 0, 0, 0);
      }
      const int tok0 = (pg0 + 2 * it) * 16;
      // lane owns query (lane & 15) and tokens tok0 + tl + 4t + e, all on page
      // lane >> 5 of the tile; scores in base-2 units (the queries carry
      // scale * log2 e)
      bool bad0 = false, bad1 = false;
      if constexpr (!FAST) {
        bad0 = unmapped(it, 0);
        bad1 = unmapped(it, 1);
      }
      const bool page_ok = !((lane >> 5) ? bad1 : bad0);
      float s[8];
      if (FAST || (tok0 + 32 <= tok_end && !bad0 && !bad1)) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[t * 4 + e] = stc[t][e];
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[t * 4 + e] = (page_ok && tok0 + tl + 4 * t + e < tok_end) ? stc[t][e] : -INFINITY;
      }
      // row maximum over the four lanes holding this query's 32 tokens
      const float mx = row_max4(fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                                      fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7]))));
      // Lazy rescaling: the reference maximum m_run moves (and the running
      // sums are rescaled) only when some row's maximum exceeds it by more
      // than 8, so the probabilities stay below 2^8 and the rescale is rare.
      const float m_new = fmaxf(m_run, mx);
      if (__any(m_new > m_run + 8.f)) {
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) ot[nn] *= alpha;
        m_run = m_new;
      }
      // a row with no unmasked token yet (m_run = -inf) contributes P = 0
      const bool live = m_run != -INFINITY;
      float pv[8], ps = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        pv[k] = live ? __builtin_amdgcn_exp2f(s[k] - m_run) : 0.f;
        ps += pv[k];
      }
      l_run += ps;
      u32x4 hu, lu;
      split_hilo8(pv, hu, lu);
      const bf16x8 pbh = as_bf16x8(hu), pbl = as_bf16x8(lu);
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) ot[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[nn], pbh, ot[nn], 0, 0, 0);
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) ot[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[nn], pbl, ot[nn], 0, 0, 0);
      stc[0] = stn[0];
      stc[1] = stn[1];
      // tile it+1 landed (waited for above): its V fragments for the next P V
      if (more) ATT_READ_V(it + 1, vf);
    }
  };
  const int full = tok_end > pg0 * 16 ? min(ntiles, (tok_end - pg0 * 16) / 32) : 0;   // leading whole tiles
  const int n_fast = any_bad ? 0 : max(0, full - 1);
  int it = 0;
  for (; it < n_fast; ++it) step(it, std::true_type{});
  for (; it < ntiles; ++it) step(it, std::false_type{});
#undef ATT_SCORES
#undef ATT_READ_V

  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);
  if (!rvalid) return;
  const size_t Mq = (size_t)p.batch * p.B * p.nq;
  const size_t qrow = (size_t)row * p.nq + n;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if ((lane >> 4) == 0)
    p.part_lse[split * Mq + qrow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
  float* dst = p.part_o + (split * Mq + qrow) * D;
#pragma unroll
  for (int nn = 0; nn < NN; ++nn) {
    const int d0 = 16 * nn + 4 * (lane >> 4);
    *(float4*)(dst + d0) = make_float4(ot[nn][0] * inv, ot[nn][1] * inv, ot[nn][2] * inv, ot[nn][3] * inv);
  }
}

// ---------------------------------------------------------------------------
// VALU attention over a context split (fp32 pools, or head_dim 64): 64 query
// rows per workgroup, 4 lanes per row (D/4 dims each).
template <typename TP, int D, bool CTX>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnParams p) {
  constexpr int DQ = D / 4;
  const int g = p.nq / p.nkv, R = g * p.B;
  const int nqg = (R + 63) / 64;
  const int split = blockIdx.x / nqg;
  const int qg = blockIdx.x % nqg;
  const int m = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, q4 = tid & 3;
  const int r = qg * 64 + (tid >> 2);
  const bool rvalid = r < R;
  const int j = rvalid ? r / p.B : 0, i = rvalid ? r - (r / p.B) * p.B : 0;
  const int n = m * g + j, row = b * p.B + i;
  const int ldq = (p.nq + 2 * p.nkv) * D;

  float q[DQ], o[DQ];
  {
    const float* qv = p.qkv + (size_t)row * ldq + n * D;
    const float2* cs = p.cs + (size_t)row * (D / 2);
    // scores in base-2 units: the query carries scale * log2 e
    const float qs = p.scale * 1.4426950408889634f;
#pragma unroll
    for (int e = 0; e < DQ; ++e) {
      q[e] = rvalid ? rope_elem(qv, cs, q4 * DQ + e, D) * qs : 0.f;
      o[e] = 0.f;
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  auto consume = [&](float sc, const float* vvals) {  // vvals may point to LDS
    // vvals: this lane's DQ value entries
    const float m_new = fmaxf(m_run, sc);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new), pw = __builtin_amdgcn_exp2f(sc - m_new);
    l_run = l_run * alpha + pw;
#pragma unroll
    for (int e = 0; e < DQ; ++e) o[e] = o[e] * alpha + pw * vvals[e];
    m_run = m_new;
  };

  {
    const int ctx = clamp_ctx(p, b);
    const int npages = (ctx + 15) >> 4;
    int pg0, pg1;
    split_pages(p, npages, split, pg0, pg1);
    const TP* pool = (const TP*)p.pool;
    const size_t chunk = 16 * D;
    // Each page's K and V chunks are staged in LDS by the whole workgroup (one
    // coalesced pass, one memory round trip per page) and every query row then
    // walks the page's tokens from LDS.
    __shared__ float ks[16 * D], vs[16 * D];
    for (int pg = pg0; pg < pg1; ++pg) {
      const int ph = phys_page(p, b, pg);   // the same for every thread of the workgroup
      if (ph < 0) continue;
      const TP* Kc = pool + (((size_t)ph * p.n_layers + p.layer) * 2 * p.nkv + m) * chunk;
      const TP* Vc = Kc + (size_t)p.nkv * chunk;
      const int ns = min(16, ctx - pg * 16);
      __syncthreads();   // the previous page's reads are done
      float kv[2][16 * D / 256];   // all of a thread's loads in flight before any LDS store
#pragma unroll
      for (int t = 0; t < 16 * D / 256; ++t) {
        kv[0][t] = ld_f(Kc, tid + 256 * t);
        kv[1][t] = ld_f(Vc, tid + 256 * t);
      }
#pragma unroll
      for (int t = 0; t < 16 * D / 256; ++t) {
        ks[tid + 256 * t] = kv[0][t];
        vs[tid + 256 * t] = kv[1][t];
      }
      __syncthreads();
      for (int slot = 0; slot < ns; ++slot) {
        float sd = 0.f;
#pragma unroll
        for (int e = 0; e < DQ; ++e) sd += q[e] * ks[slot * D + q4 * DQ + e];
        sd += __shfl_xor(sd, 1, kWave);
        sd += __shfl_xor(sd, 2, kWave);
        float vv[DQ];
#pragma unroll
        for (int e = 0; e < DQ; ++e) vv[e] = vs[(q4 * DQ + e) * 16 + slot];
        consume(sd, vv);
      }
    }
  }
  if (!rvalid) return;
  const size_t Mq = (size_t)p.batch * p.B * p.nq;
  const size_t qrow = (size_t)row * p.nq + n;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  // natural-log LSE, as the finish kernel merges it
  if (q4 == 0)
    p.part_lse[split * Mq + qrow] = l_run > 0.f ? (m_run + log2f(l_run)) * 0.6931471805599453f : -INFINITY;
  float* dst = p.part_o + (split * Mq + qrow) * D + q4 * DQ;
#pragma unroll
  for (int e = 0; e < DQ; ++e) dst[e] = o[e] * inv;
}

// ---------------------------------------------------------------------------
// Block keys and merge, per (16 query rows, kv head, sequence), sixteen
// threads per query row: the B rotated block keys and their values (fp32) are
// staged in LDS; each thread keeps 1/16 of its row's rotated query in
// registers, the partial dot products of a key are summed over the row's
// lanes, the row attends to the B keys (softmax in fp32), and the result is
// merged with the n_splits context partials in split order (block part last)
// and written in the operand form of the output projection.
// Value of another lane of the same 16-lane row, by a DPP control (quad
// permutation or row rotation): no LDS round trip.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

template <int D, bool PREP, int NK = 16>
__global__ __launch_bounds__(256) void attn_finish_kernel(AttnParams p, ActOut out) {
  // NK: block keys held (16 for a draft block; 32 for a target forward of up to 32 tokens)
  constexpr int QR = 16, DPT = D / 16;   // 16 threads per query row, DPT dims each
  static_assert(DPT % 4 == 0, "dims per thread");
  // a thread's dims are C chunks of four, chunk c at c * (D / C) + 4 * part: the
  // sixteen threads of a row read each chunk as 256 contiguous bytes (no LDS
  // bank conflicts, coalesced global reads and stores)
  constexpr int C = DPT / 4;
  __shared__ __attribute__((aligned(16))) float kb[NK][D];
  __shared__ __attribute__((aligned(16))) float vb[NK][D];
  const int g = p.nq / p.nkv, R = g * p.B, h = D / 2;
  const int qg = blockIdx.x, m = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int ldq = (p.nq + 2 * p.nkv) * D;
  // Every global read is unconditional and four wide: block rows past B and
  // query rows past the group are clamped to a valid row (and masked or
  // dropped later), so all reads are in flight before the first use.
  constexpr int KV4 = NK * D / 4 / 256;   // float4 of K (and of V) per thread
#pragma unroll
  for (int k = 0; k < KV4; ++k) {
    const int c4 = tid + 256 * k, jb = (4 * c4) / D, e = 4 * c4 - jb * D;
    const int jc = min(jb, p.B - 1), krow = b * p.B + jc;
    float4 kk, vv;
    if constexpr (PREP) {
      const size_t o = (((size_t)b * p.nkv + m) * p.B + jc) * D + e;
      kk = *(const float4*)(p.kblk + o);
      vv = *(const float4*)(p.vblk + o);
    } else {
      vv = *(const float4*)(p.qkv + (size_t)krow * ldq + (p.nq + p.nkv) * D + m * D + e);
      const float* kv = p.qkv + (size_t)krow * ldq + p.nq * D + m * D;
      const float2* cs = p.cs + (size_t)krow * h;
      kk = make_float4(rope_elem(kv, cs, e, D), rope_elem(kv, cs, e + 1, D), rope_elem(kv, cs, e + 2, D),
                       rope_elem(kv, cs, e + 3, D));
    }
    *(float4*)&kb[jb][e] = kk;
    *(float4*)&vb[jb][e] = vv;
  }
  const int rl = tid >> 4, part = tid & 15, rr = qg * QR + rl;
  const bool rv = rr < R;
  const int rc = rv ? rr : R - 1;
  const int j = rc / p.B, i = rc - j * p.B;
  const int row = b * p.B + i, n = m * g + j;
  auto dch = [&](int c) { return c * (D / C) + 4 * part; };   // first dim of chunk c
  // the first context partials of this row, loaded now so their latency
  // overlaps the in-block attention (the merge below uses them in split order)
  constexpr int NPF = 2;
  const size_t Mq = (size_t)p.batch * p.B * p.nq;
  const size_t qrow = (size_t)row * p.nq + n;
  float pl[NPF];
  float4 po[NPF][DPT / 4];
#pragma unroll
  for (int k = 0; k < NPF; ++k) {
    pl[k] = k < p.n_splits ? p.part_lse[k * Mq + qrow] : -INFINITY;
#pragma unroll
    for (int e = 0; e < DPT; e += 4)
      po[k][e / 4] = k < p.n_splits ? *(const float4*)(p.part_o + (k * Mq + qrow) * D + dch(e / 4))
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float q[DPT];
  if constexpr (PREP) {
    // prepared rotated query (hi + lo), carrying scale * log2 e
    const size_t qoff = (((size_t)b * p.nkv + m) * R + rc) * D;
#pragma unroll
    for (int k = 0; k < DPT; k += 4) {
      // a bf16 is the high half of an fp32: element 2t of a word is w << 16,
      // element 2t+1 is w & 0xffff0000
      const size_t o = qoff + dch(k / 4);
      const u32x2 hv = *(const u32x2*)(p.q_hi + o), lv = *(const u32x2*)(p.q_lo + o);
      q[k] = __uint_as_float(hv.x << 16) + __uint_as_float(lv.x << 16);
      q[k + 1] = __uint_as_float(hv.x & 0xffff0000u) + __uint_as_float(lv.x & 0xffff0000u);
      q[k + 2] = __uint_as_float(hv.y << 16) + __uint_as_float(lv.y << 16);
      q[k + 3] = __uint_as_float(hv.y & 0xffff0000u) + __uint_as_float(lv.y & 0xffff0000u);
    }
  } else {
    const float* qv = p.qkv + (size_t)row * ldq + n * D;
    const float2* cs = p.cs + (size_t)row * h;
#pragma unroll
    for (int e = 0; e < DPT; ++e) q[e] = rope_elem(qv, cs, dch(e / 4) + (e & 3), D) * p.scale * 1.4426950408889634f;
  }
  __syncthreads();
  // scores in base-2 units: partial dot over this thread's dims, summed over
  // the row's sixteen lanes (DPP: lane ^ 1, lane ^ 2, then rotations by 4, 8)
  float sc[NK];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < DPT; e += 4) {
      const float4 kv = *(const float4*)&kb[k][dch(e / 4)];
      a = fmaf(q[e], kv.x, a);
      a = fmaf(q[e + 1], kv.y, a);
      a = fmaf(q[e + 2], kv.z, a);
      a = fmaf(q[e + 3], kv.w, a);
    }
    a += dpp_mov<0xB1>(a);
    a += dpp_mov<0x4E>(a);
    a += dpp_mov<0x124>(a);   // row_ror:4
    a += dpp_mov<0x128>(a);   // row_ror:8
    sc[k] = (k < p.B && (!p.causal || k <= i)) ? a : -INFINITY;
    mx = fmaxf(mx, sc[k]);
  }
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    sc[k] = k < p.B ? __builtin_amdgcn_exp2f(sc[k] - mx) : 0.f;
    sum += sc[k];
  }
  const float blse = (mx + __log2f(sum)) * 0.6931471805599453f;   // natural log, as the context partials
  const float rs = 1.f / sum;
  float ob[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) ob[e] = 0.f;
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const float w = sc[k] * rs;
#pragma unroll
    for (int e = 0; e < DPT; e += 4) {
      const float4 vv = *(const float4*)&vb[k][dch(e / 4)];
      ob[e] = fmaf(w, vv.x, ob[e]);
      ob[e + 1] = fmaf(w, vv.y, ob[e + 1]);
      ob[e + 2] = fmaf(w, vv.z, ob[e + 2]);
      ob[e + 3] = fmaf(w, vv.w, ob[e + 3]);
    }
  }
  if (!rv) return;
  float mxl = blse;
#pragma unroll
  for (int k = 0; k < NPF; ++k) mxl = fmaxf(mxl, pl[k]);
  // the remaining split maxima, eight loads in flight at a time
  for (int s0 = NPF; s0 < p.n_splits; s0 += 8) {
    float l8[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) l8[k] = s0 + k < p.n_splits ? p.part_lse[(s0 + k) * Mq + qrow] : -INFINITY;
#pragma unroll
    for (int k = 0; k < 8; ++k) mxl = fmaxf(mxl, l8[k]);
  }
  float tot = 0.f, acc[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
  // an empty split has lse = -inf and o = 0, so it adds nothing (no branch)
#pragma unroll
  for (int k = 0; k < NPF; ++k) {
    const float w = expf(pl[k] - mxl);
    tot += w;
#pragma unroll
    for (int e = 0; e < DPT; e += 4) {
      const float4 v = po[k][e / 4];
      acc[e] = fmaf(w, v.x, acc[e]);
      acc[e + 1] = fmaf(w, v.y, acc[e + 1]);
      acc[e + 2] = fmaf(w, v.z, acc[e + 2]);
      acc[e + 3] = fmaf(w, v.w, acc[e + 3]);
    }
  }
  // the remaining splits in split order, four splits' loads in flight at a time; a
  // split past the end reads as (lse -inf, o 0) and adds exactly nothing
  for (int s0 = NPF; s0 < p.n_splits; s0 += 4) {
    float l4[4];
    float4 v4[4][DPT / 4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool ok = s0 + k < p.n_splits;
      l4[k] = ok ? p.part_lse[(s0 + k) * Mq + qrow] : -INFINITY;
      const float* src = p.part_o + ((s0 + k) * Mq + qrow) * D;
#pragma unroll
      for (int e = 0; e < DPT; e += 4)
        v4[k][e / 4] = ok ? *(const float4*)(src + dch(e / 4)) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float w = expf(l4[k] - mxl);
      tot += w;
#pragma unroll
      for (int e = 0; e < DPT; e += 4) {
        const float4 v = v4[k][e / 4];
        acc[e] = fmaf(w, v.x, acc[e]);
        acc[e + 1] = fmaf(w, v.y, acc[e + 1]);
        acc[e + 2] = fmaf(w, v.z, acc[e + 2]);
        acc[e + 3] = fmaf(w, v.w, acc[e + 3]);
      }
    }
  }
  {
    const float w = expf(blse - mxl);
    tot += w;
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] = fmaf(w, ob[e], acc[e]);
  }
  const float inv = 1.f / tot;
#pragma unroll
  for (int e = 0; e < DPT; e += 4)
    act_store4(out, row, n * D + dch(e / 4),
               make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv));
}

// ---------------------------------------------------------------------------
int att_query_group(int R, int wdtype, int d) { return wdtype == 1 && d == 128 && R > 64 ? 128 : 64; }

hipError_t launch_attention(const AttnParams& p, int wdtype, hipStream_t s, void (*mark)(int, hipStream_t)) {
  const int g = p.nq / p.nkv, R = g * p.B, qgr = att_query_group(R, wdtype, p.d), nqg = (R + qgr - 1) / qgr;
  // the prepared queries and block keys also feed the finish kernel, with or
  // without context
  if (wdtype == 1 && p.d == 128) {
    hipLaunchKernelGGL(attn_qprep_kernel<128>, dim3((R + 2 * p.B + 15) / 16, p.nkv, p.batch), dim3(256), 0, s, p);
  }
  if (p.n_splits <= 0) return hipGetLastError();
  const dim3 gctx(p.n_splits * nqg, p.nkv, p.batch);
  if (mark) mark(0, s);
  if (wdtype == 1 && p.d == 128 && qgr == 128)
    hipLaunchKernelGGL((attn_ctx_mfma_kernel<128, 8>), gctx, dim3(512), 0, s, p);
  else if (wdtype == 1 && p.d == 128)
    hipLaunchKernelGGL((attn_ctx_mfma_kernel<128, 4>), gctx, dim3(256), 0, s, p);
  else if (wdtype == 1)
    hipLaunchKernelGGL((attn_valu_kernel<bf16_t, 64, true>), gctx, dim3(256), 0, s, p);
  else if (p.d == 128)
    hipLaunchKernelGGL((attn_valu_kernel<float, 128, true>), gctx, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((attn_valu_kernel<float, 64, true>), gctx, dim3(256), 0, s, p);
  if (mark) mark(1, s);
  return hipGetLastError();
}

hipError_t launch_attn_finish(const AttnParams& p, int wdtype, ActOut out, hipStream_t s) {
  const int R = (p.nq / p.nkv) * p.B;
  const dim3 grid((R + 15) / 16, p.nkv, p.batch);
  if (wdtype == 1 && p.d == 128)   // the query prep ran: prepared queries, block keys and values
    if (p.B > 16)
      hipLaunchKernelGGL((attn_finish_kernel<128, true, 32>), grid, dim3(256), 0, s, p, out);
    else
      hipLaunchKernelGGL((attn_finish_kernel<128, true>), grid, dim3(256), 0, s, p, out);
  else if (p.d == 128)
    hipLaunchKernelGGL((attn_finish_kernel<128, false>), grid, dim3(256), 0, s, p, out);
  else
    hipLaunchKernelGGL((attn_finish_kernel<64, false>), grid, dim3(256), 0, s, p, out);
  return hipGetLastError();
}

}  // namespace dflash
