// GEMM kernels: C[M, N] = A[M, K] * W[N, K]^T with fp32 accumulation.
//
// bf16 weights: MFMA v_mfma_f32_16x16x32_bf16 on gfx950.  A is either one
// bfloat16 plane (target hidden states, LM-head input) or a (hi, lo) pair of
// planes carrying an fp32 activation to ~2^-16 relative: every product is
// then two MFMAs into the same accumulator.  Weights are exact in bf16.
// fp32 weights: a plain LDS-tiled FMA kernel.
//
// Both kernels end by staging their C tile in LDS, so every epilogue sees
// whole tile rows: plain/hi-lo stores, residual add, SwiGLU (gate and up
// halves of the same tile), the LM-head argmax / log-sum-exp partials, and
// the KV-injection scatter (rotary on K pairs (j, j+d/2), then the page slot).
#include <algorithm>

#include "kernels.h"

namespace dflash {

template <typename T>
struct BRows {
  const T* b0;
  const T* b1;
  int ldb, split, mode;
  __device__ __forceinline__ const T* row(int n, int BN) const {
    if (mode == 0) return b0 + (size_t)n * ldb;
    if (mode == 1) return n < split ? b0 + (size_t)n * ldb : b1 + (size_t)(n - split) * ldb;
    const int h = BN / 2, t = n / BN, c = n - t * BN;
    return c < h ? b0 + (size_t)(t * h + c) * ldb : b1 + (size_t)(t * h + c - h) * ldb;
  }
};

// SwiGLU rows interleaved per 32 columns of a BN tile: 16 gate rows (b0),
// then the same 16 up rows (b1).
__device__ __forceinline__ const bf16_t* swiglu_il_row(const BRows<bf16_t>& b, int n, int BN) {
  const int h = BN / 2, t = n / BN, c = n - t * BN, q = c >> 5, w = c & 31;
  return (w < 16 ? b.b0 : b.b1) + (size_t)(t * h + q * 16 + (w & 15)) * b.ldb;
}
// Tile column (interleaved order) -> column in the gate-half / up-half order
// the split-K reduce expects.
__device__ __forceinline__ int swiglu_il_col(int c, int BN) {
  const int q = c >> 5, w = c & 31;
  return w < 16 ? q * 16 + w : BN / 2 + q * 16 + (w - 16);
}

// ---------------------------------------------------------------------------
// LM-head partials: over a run of columns, (max of the score the candidate
// maximises, its first index, max and sum-exp of z/T, z/T at that index).
struct LMPart {
  float pmax, zmax, zsum, zc;
  int idx;
};

__device__ __forceinline__ LMPart lm_merge(const LMPart& a, const LMPart& b) {
  // a covers lower column indices than b
  LMPart r;
  if (b.pmax > a.pmax || (a.idx < 0 && b.idx >= 0)) {
    r.pmax = b.pmax; r.idx = b.idx; r.zc = b.zc;
  } else {
    r.pmax = a.pmax; r.idx = a.idx; r.zc = a.zc;
  }
  const float M = fmaxf(a.zmax, b.zmax);
  float s = 0.f;
  if (a.zsum > 0.f) s += a.zsum * expf(a.zmax - M);
  if (b.zsum > 0.f) s += b.zsum * expf(b.zmax - M);
  r.zmax = M;
  r.zsum = s;
  return r;
}

// x / (1 + e^-x) with the hardware exp2 and reciprocal (about 1 ulp each);
// e^-x overflowing to infinity gives 0, the limit.
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

template <int KIND, int BM, int BN, int NT, typename TP>
__device__ __forceinline__ void run_epilogue(const float* Cs, int ldc, int m0, int n0, int M, int N,
                                             const EpiParams& e) {
  const int tid = threadIdx.x;
  if constexpr (KIND == EPI_STORE || KIND == EPI_ADD) {
    constexpr int C4 = BN / 4;
    for (int idx = tid; idx < BM * C4; idx += NT) {
      const int r = idx / C4, c = (idx - r * C4) * 4;
      const int row = m0 + r, col = n0 + c;
      if (row >= M || col >= N) continue;
      const float4 v = *(const float4*)(Cs + r * ldc + c);
      if constexpr (KIND == EPI_STORE) {
        act_store4(e.out, row, col, v);
      } else {
        float4* p = (float4*)(e.resid + (size_t)row * e.ldr + col);
        float4 o = *p;
        o.x += v.x; o.y += v.y; o.z += v.z; o.w += v.w;
        *p = o;
      }
    }
  } else if constexpr (KIND == EPI_SWIGLU) {
    constexpr int H2 = BN / 2, C4 = H2 / 4;
    for (int idx = tid; idx < BM * C4; idx += NT) {
      const int r = idx / C4, c = (idx - r * C4) * 4;
      const int row = m0 + r, col = n0 / 2 + c;
      if (row >= M || col >= N / 2) continue;
      const float4 g = *(const float4*)(Cs + r * ldc + c);
      const float4 u = *(const float4*)(Cs + r * ldc + H2 + c);
      float4 a;
      a.x = silu_fast(g.x) * u.x;
      a.y = silu_fast(g.y) * u.y;
      a.z = silu_fast(g.z) * u.z;
      a.w = silu_fast(g.w) * u.w;
      act_store4(e.out, row, col, a);
    }
  } else if constexpr (KIND == EPI_LMHEAD) {
    // optional logits, coalesced row segments
    if (e.logits) {
      constexpr int C4 = BN / 4;
      for (int idx = tid; idx < BM * C4; idx += NT) {
        const int r = idx / C4, c = (idx - r * C4) * 4;
        const int row = m0 + r;
        if (row >= M) continue;
        const size_t base = (size_t)e.row_map[row] * e.ldz + e.col0;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (n0 + c + q < N) e.logits[base + n0 + c + q] = Cs[r * ldc + c + q];
      }
    }
    constexpr int TPR = NT / BM;      // threads per row
    constexpr int GRP = (BN % 128 == 0) ? 128 : 64;   // columns per partial
    constexpr int CPT = GRP / TPR;    // columns per thread within a group
    static_assert(NT % BM == 0 && GRP % TPR == 0 && BN % GRP == 0, "tile split");
    const int r = tid / TPR, q = tid - r * TPR;
    const int row = m0 + r;
    const bool rv = row < M;
    const float T = e.temperature;
    const bool samp = T > 0.f;
    int bi = 0, bb = 0;
    if (rv) {
      const int rm = e.row_map[row];
      bb = rm / e.block;
      bi = rm - bb * e.block;
    }
#pragma unroll 1
    for (int gq = 0; gq < BN / GRP; ++gq) {
      LMPart P;
      P.pmax = -INFINITY; P.zmax = -INFINITY; P.zsum = 0.f; P.zc = -INFINITY; P.idx = -1;
      const int c0 = gq * GRP + q * CPT;
      if (rv) {
        for (int c = 0; c < CPT; c += 4) {
          const int v0 = n0 + c0 + c;   // launch column; vocabulary index e.col0 + v0
          uint4 w = make_uint4(0, 0, 0, 0);
          if (samp && v0 < N)
            w = philox4x32_10(
                make_uint4((uint32_t)((e.col0 + v0) >> 2), (uint32_t)bi, (uint32_t)e.step, (uint32_t)bb),
                e.seed_lo, e.seed_hi);
          const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int v = v0 + k;
            if (v >= N) break;
            const float zt = samp ? Cs[r * ldc + c0 + c + k] / T : Cs[r * ldc + c0 + c + k];
            const float sc = samp ? zt + gumbel_from_word(ww[k]) : zt;
            if (sc > P.pmax || P.idx < 0) { P.pmax = sc; P.idx = e.col0 + v; P.zc = zt; }
            P.zmax = fmaxf(P.zmax, zt);
          }
        }
        for (int c = 0; c < CPT; ++c) {
          if (n0 + c0 + c >= N) break;
          const float zt = samp ? Cs[r * ldc + c0 + c] / T : Cs[r * ldc + c0 + c];
          P.zsum += expf(zt - P.zmax);
        }
      }
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) {
        LMPart Q;
        Q.pmax = __shfl_xor(P.pmax, o, kWave);
        Q.zmax = __shfl_xor(P.zmax, o, kWave);
        Q.zsum = __shfl_xor(P.zsum, o, kWave);
        Q.zc = __shfl_xor(P.zc, o, kWave);
        Q.idx = __shfl_xor(P.idx, o, kWave);
        P = (q & o) ? lm_merge(Q, P) : lm_merge(P, Q);
      }
      if (rv && q == 0 && n0 + gq * GRP < N) {
        const size_t pi = (size_t)row * e.ntiles + (e.col0 + n0 + gq * GRP) / GRP;
        e.part_f[pi] = make_float4(P.pmax, P.zmax, P.zsum, P.zc);
        e.part_i[pi] = P.idx;
      }
    }
  } else if constexpr (KIND == EPI_KVSCATTER) {
    const int d = e.head_dim, hd = d / 2, nkv = e.n_kv;
    const int hpt = BN / d;  // heads per tile
    // QK-norm: 1 / rms of every (row, head) of the tile (head_dim >= 64, so at
    // most BN / 64 heads per row); only the K heads use it
    __shared__ float kinv[BM * (BN / 64)];
    if (e.k_norm_on) {
      for (int idx = tid; idx < BM * hpt; idx += NT) {
        const int r = idx / hpt, hb = idx - r * hpt;
        const float* x = Cs + r * ldc + hb * d;
        float ss = 0.f;
        for (int c = 0; c < d; ++c) ss = fmaf(x[c], x[c], ss);
        kinv[idx] = 1.f / sqrtf(ss / (float)d + e.rms_eps);
      }
      __syncthreads();
    }
    for (int idx = tid; idx < BM * hpt * hd; idx += NT) {
      const int r = idx / (hpt * hd);
      const int rem = idx - r * hpt * hd;
      const int hb = rem / hd, j = rem - hb * hd;
      const int row = m0 + r, col0 = n0 + hb * d;
      if (row >= M || col0 >= N) continue;
      const int head = col0 / d;           // ((l * 2 + kv) * nkv + m)
      const int m = head % nkv, kv = (head / nkv) & 1, l = head / (2 * nkv), L = e.n_layers;
      const int b = e.tok_seq[row], pos = e.tok_pos[row];
      if (b < 0 || b >= e.n_seqs || pos < 0) continue;
      const int lp = pos >> 4, slot = pos & 15;
      if (lp >= e.max_pages) continue;
      const int phys = e.block_table[(size_t)b * e.max_pages + lp];
      if (phys < 0 || phys >= e.n_pages) continue;
      float x0 = Cs[r * ldc + hb * d + j], x1 = Cs[r * ldc + hb * d + j + hd];
      TP* chunk = (TP*)e.pool + ((((size_t)phys * L + l) * 2 + kv) * nkv + m) * (size_t)(16 * d);
      if (kv == 0) {
        if (e.k_norm_on) {
          const float sc = kinv[r * hpt + hb];
          const float* gk = e.k_gain[l];
          x0 = x0 * sc * gk[j];
          x1 = x1 * sc * gk[j + hd];
        }
        const float2 cs = e.rope_cs[(size_t)row * hd + j];
        const float y0 = x0 * cs.x - x1 * cs.y, y1 = x1 * cs.x + x0 * cs.y;
        if constexpr (sizeof(TP) == 2) {
          chunk[slot * d + j] = f2bf(y0);
          chunk[slot * d + j + hd] = f2bf(y1);
        } else {
          chunk[slot * d + j] = y0;
          chunk[slot * d + j + hd] = y1;
        }
      } else {
        if constexpr (sizeof(TP) == 2) {
          chunk[j * 16 + slot] = f2bf(x0);
          chunk[(j + hd) * 16 + slot] = f2bf(x1);
        } else {
          chunk[j * 16 + slot] = x0;
          chunk[(j + hd) * 16 + slot] = x1;
        }
      }
    }
  }
}

// Tile order: consecutive block ids go to different XCDs (round robin), so
// the id is remapped to give each XCD a contiguous run of tiles, M-tiles of
// one N-tile adjacent: a weight tile is then fetched by one XCD's L2.
__device__ __forceinline__ bool tile_of(int ntm, int total, int& tm, int& tn) {
  const int per = gridDim.x / 8;
  const int L = blockIdx.x;
  const int t = (per > 0) ? (L & 7) * per + (L >> 3) : L;
  if (t >= total) return false;
  tm = t % ntm;
  tn = t / ntm;
  return true;
}

// ---------------------------------------------------------------------------
// MFMA GEMM with direct global->LDS loads (gfx950 global_load_lds_dwordx4):
// 128x128x32 tiles, four 64x64 waves, three LDS stages, one barrier per
// K-tile and no staging registers.  Each 16-byte load instruction of a wave
// fills 1 KiB of LDS lane-linearly (lane i -> base + 16 i), so the LDS tile is
// row-major with 64-byte rows; the 16-byte chunk c of row r is stored at
// chunk c ^ ((r >> 1) & 3), which keeps the MFMA operand reads of eight
// consecutive lanes (eight rows, same chunk) on distinct banks.
template <int NP>
struct DmaCfg {
  static constexpr int BM = 128, BN = 128, BK = 32, NT = 256, STAGES = 3;
  static constexpr int ROWS = NP * BM + BN;          // LDS rows per stage (64 B each)
  static constexpr int STAGE_BYTES = ROWS * 64;
  static constexpr int BLOCKS = STAGE_BYTES / 1024;   // 1 KiB load instructions per stage
  static constexpr int LPT = BLOCKS / 4;              // per wave (and per thread)
  static constexpr int LDC = BN + 4;
  static constexpr int SMEM_PIPE = STAGES * STAGE_BYTES;
  static constexpr int SMEM_EPI = BM * LDC * 4;
  static constexpr int SMEM = SMEM_PIPE > SMEM_EPI ? SMEM_PIPE : SMEM_EPI;
  static_assert(BLOCKS % 4 == 0, "blocks per wave");
};

// s_waitcnt on the vector-memory counter only, through the builtin so that
// the compiler's own wait insertion knows the copies to LDS have landed (it
// would otherwise wait for every outstanding store before each LDS read of the
// epilogue).  vmcnt sits in bits 3:0 and 15:14; expcnt and lgkmcnt stay at
// their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would also wait for the next tile's loads still in flight.  LDS data of the
// current tile is covered by each wave's own vmcnt wait before the barrier;
// LDS reads of the previous tile completed before their MFMAs issued.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// The same, after this wave's LDS reads have completed: the buffer they read
// may be refilled by any wave once every wave has passed the barrier.
__device__ __forceinline__ void lds_reads_done_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int NP, int KIND>
__global__ __launch_bounds__(256, 2) void gemm_dma_kernel(ActIn a, BRows<bf16_t> b, int M, int N, int K, int ksplit,
                                                           float* part, EpiParams e, const int* m_dev) {
  using C = DmaCfg<NP>;
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, LPT = C::LPT;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::SMEM];

  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  int t;
  {
    const int per = gridDim.x / 8, L = blockIdx.x;
    t = (per > 0) ? (L & 7) * per + (L >> 3) : L;
    if (t >= ntm * ntn * ksplit) return;
  }
  const int tm = t % ntm, tn = (t / ntm) % ntn, ks = t / (ntm * ntn);
  const int m0 = tm * BM, n0 = tn * BN;
  // rows from the device count on are left alone: tiles wholly past it leave
  // at once (the partial layout keeps the row stride of M)
  const int Mp = M;
  if (m_dev) M = min(M, max(*m_dev, 0));
  if (m0 >= M) return;
  const int nkt = K / BK;
  const int kt0 = (int)((long long)ks * nkt / ksplit), kt1 = (int)((long long)(ks + 1) * nkt / ksplit);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  // source row pointers of this lane's LPT load blocks (fixed over K)
  const bf16_t* src[LPT];
#pragma unroll
  for (int q = 0; q < LPT; ++q) {
    const int blk = wid * LPT + q;
    const int row = blk * 16 + (lane >> 2);
    const int pc = lane & 3, lc = pc ^ ((row >> 1) & 3);
    const bf16_t* base;
    if (row < NP * BM) {
      const int p = row / BM, r = row - p * BM;
      int gr = min(m0 + r, M - 1);
      if (a.rows) gr = a.rows[gr];
      base = (const bf16_t*)(p == 0 ? a.p0 : a.p1) + (size_t)gr * a.ld;
    } else {
      base = b.row(min(n0 + row - NP * BM, N - 1), BN);
    }
    src[q] = base + lc * 8;
  }
  const uint32_t lds0 = (uint32_t)(size_t)smem;

  auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
    const int k0 = kt * BK;
#pragma unroll
    for (int q = 0; q < LPT; ++q) {
      const int blk = wid * LPT + q;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(src[q] + k0),
          (__attribute__((address_space(3))) void*)(size_t)(lds0 + stage * C::STAGE_BYTES + blk * 1024), 16, 0, 0);
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nloc = kt1 - kt0;
  if (nloc > 0) issue(kt0, 0);
  if (nloc > 1) issue(kt0 + 1, 1);
  for (int it = 0; it < nloc; ++it) {
    if (it + 1 < nloc) wait_vmcnt<LPT>();   // this tile landed; the next may still be in flight
    else wait_vmcnt<0>();
    stage_barrier();                         // all lanes' data visible; stage (it+2)%3 is free
    if (it + 2 < nloc) issue(kt0 + it + 2, (it + 2) % 3);
    const unsigned char* st = smem + (it % 3) * C::STAGE_BYTES;
    const int lc = lane >> 4;
    bf16x8 af[NP][4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int row = p * BM + wm * 64 + 16 * i + (lane & 15);
        af[p][i] = as_bf16x8(*(const u32x4*)(st + row * 64 + ((lc ^ ((row >> 1) & 3)) << 4)));
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = NP * BM + wn * 64 + 16 * j + (lane & 15);
      bfr[j] = as_bf16x8(*(const u32x4*)(st + row * 64 + ((lc ^ ((row >> 1) & 3)) << 4)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int p = 0; p < NP; ++p)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[p][i], bfr[j], acc[i][j], 0, 0, 0);
  }
  __syncthreads();   // every wave is done with the pipeline buffers

  float* Cs = (float*)smem;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        Cs[(wm * 64 + 16 * i + 4 * (lane >> 4) + q) * C::LDC + wn * 64 + 16 * j + (lane & 15)] = acc[i][j][q];
  __syncthreads();
  if (ksplit > 1) {
    float* dst = part + (size_t)ks * Mp * N;
    constexpr int C4 = BN / 4;
    for (int idx = tid; idx < BM * C4; idx += 256) {
      const int r = idx / C4, c = (idx - r * C4) * 4;
      if (m0 + r < M && n0 + c < N)
        *(float4*)(dst + (size_t)(m0 + r) * N + n0 + c) = *(const float4*)(Cs + r * C::LDC + c);
    }
    return;
  }
  run_epilogue<KIND, BM, BN, 256, bf16_t>(Cs, C::LDC, m0, n0, M, N, e);
}

// Scheduling of one pipeline step: the R fragment reads of the next stage are
// spread over the Q MFMAs of the current one (Q/R MFMAs, then one read), so
// their LDS traffic overlaps the matrix work instead of following it (MFMAs
// first: the fragments they use are already in registers).
template <int R, int Q>
__device__ __forceinline__ void mfma_read_interleave() {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    __builtin_amdgcn_sched_group_barrier(0x008, Q / R, 0);  // Q/R MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // one LDS read
  }
  if constexpr (Q % R != 0) __builtin_amdgcn_sched_group_barrier(0x008, Q % R, 0);
}

// MFMA GEMM with direct global->LDS loads for large tiles: eight waves (two
// per SIMD, one workgroup per CU) of 64 x (BN/WGN), 64-deep K stages in two
// LDS buffers.  Each 1 KiB direct load covers eight whole 128-byte rows, so
// it holds eight L1 line slots instead of sixteen half-used ones (32-deep
// stages would leave each 128-byte line half used per load).  LDS rows are 128 bytes with 16-byte chunk
// c of row r stored at chunk c ^ ((r >> 1) & 7) (the sixteen rows one operand
// read touches land on distinct bank groups).  The fragment pipeline runs in
// 32-deep half stages: the reads of the next half overlap the MFMAs of the
// current one, and the one barrier per stage sits between the two halves.
template <int BM, int BN, int WGM, int WGN, int NP, int BS = 2>
struct FlCfg {
  static constexpr int NT = 64 * WGM * WGN, NW = WGM * WGN, BK = 64;
  static constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 16, FN = WN / 16;
  static constexpr int ROWS = NP * BM + BN;          // LDS rows per stage (128 B each)
  static constexpr int STAGE_BYTES = ROWS * 128;
  static constexpr int BLOCKS = ROWS / 8;             // 1 KiB load instructions per stage
  static constexpr int LPT = BLOCKS / NW;             // per wave
  static constexpr int LDC = BN + 4;
  // BS = 3: activation rows in two slots, weight rows in three (weights run a stage further ahead)
  static constexpr int A_BYTES = NP * BM * 128, B_BYTES = BN * 128, A_BLOCKS = NP * BM / 8;
  static constexpr int SMEM_PIPE = BS == 2 ? 2 * STAGE_BYTES : 2 * A_BYTES + BS * B_BYTES;
  static_assert(BS == 2 || (BS == 3 && A_BLOCKS % LPT == 0 && (NP * BM) % 16 == 0), "loader waves");
  static constexpr int SMEM_EPI = 64 * LDC * 4;
  static constexpr int SMEM = SMEM_PIPE > SMEM_EPI ? SMEM_PIPE : SMEM_EPI;
  static_assert(BLOCKS % NW == 0 && WM % 16 == 0 && WN % 16 == 0 && WM == 64, "tile shape");
  static_assert(SMEM <= 160 * 1024, "LDS");
  static_assert(LPT <= 63, "vmcnt range");
};

template <int BM, int BN, int WGM, int WGN, int NP, int KIND, int BS = 2>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_fl_kernel(ActIn a, BRows<bf16_t> b, int M, int N, int K,
                                                                     int ksplit, float* part, EpiParams e) {
  using C = FlCfg<BM, BN, WGM, WGN, NP, BS>;
  constexpr int BK = C::BK, LPT = C::LPT, FM = C::FM, FN = C::FN, NT = C::NT;
  // SwiGLU tiles load gate and up rows interleaved per 32 columns, so each
  // wave holds both halves of its output columns
  constexpr bool IL = KIND == EPI_SWIGLU && C::WN % 32 == 0;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::SMEM];

  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  int t;
  {
    const int per = gridDim.x / 8, L = blockIdx.x;
    t = (per > 0) ? (L & 7) * per + (L >> 3) : L;
    if (t >= ntm * ntn * ksplit) return;
  }
  const int tm = t % ntm, tn = (t / ntm) % ntn, ks = t / (ntm * ntn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nkt = K / BK;
  const int kt0 = (int)((long long)ks * nkt / ksplit), kt1 = (int)((long long)(ks + 1) * nkt / ksplit);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid - wm * WGN;

  // Load blocks of eight rows never straddle two buffers (the plane, split and
  // SwiGLU-half boundaries are multiples of eight rows), so each block has a
  // wave-uniform base pointer and a 32-bit per-lane byte offset.
  const int wid_u = __builtin_amdgcn_readfirstlane(wid);
  const bf16_t* bbase[LPT];
  uint32_t boff[LPT];
#pragma unroll
  for (int q = 0; q < LPT; ++q) {
    const int blk = wid_u * LPT + q;
    const int row0 = blk * 8, dr = lane >> 3;
    const int row = row0 + dr;
    const int pc = lane & 7, lc = pc ^ ((row >> 1) & 7);
    if (row0 < NP * BM) {
      const int p = row0 / BM, r = row - p * BM;
      const int gr = min(m0 + r, M - 1);
      bbase[q] = (const bf16_t*)(p == 0 ? a.p0 : a.p1);
      boff[q] = (uint32_t)(((size_t)gr * a.ld + lc * 8) * 2);
    } else {
      // rows of a block are consecutive rows of one buffer (a clamped row only
      // occurs in a block that lies past the split / half boundaries)
      const int first = min(n0 + row0 - NP * BM, N - 1);
      const bf16_t* rb = IL ? swiglu_il_row(b, first, BN) : b.row(first, BN);
      bbase[q] = rb;
      boff[q] = (uint32_t)(((size_t)(min(n0 + row - NP * BM, N - 1) - first) * b.ldb + lc * 8) * 2);
    }
  }
  const uint32_t lds0 = (uint32_t)(size_t)smem;

#define FL_ISSUE(KT, STAGE)                                                                                      \
  do {                                                                                                           \
    const uint32_t k0_ = (uint32_t)(KT) * (BK * 2);                                                              \
    _Pragma("unroll") for (int q = 0; q < LPT; ++q) {                                                            \
      __builtin_amdgcn_global_load_lds(                                                                          \
          (const __attribute__((address_space(1))) void*)((const char*)bbase[q] + (size_t)(boff[q] + k0_)),      \
          (__attribute__((address_space(3))) void*)(size_t)(lds0 + (STAGE) * C::STAGE_BYTES +                   \
                                                            (wid * LPT + q) * 1024),                             \
          16, 0, 0);                                                                                             \
    }                                                                                                            \
  } while (0)

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15, lq = lane >> 4;
#define FL_LOAD(F, STG, H)                                                                                     \
  do {                                                                                                         \
    const unsigned char* st_ = smem + (STG) * C::STAGE_BYTES;                                                  \
    const int lc_ = 4 * (H) + lq;                                                                              \
    _Pragma("unroll") for (int p = 0; p < NP; ++p) _Pragma("unroll") for (int i = 0; i < FM; ++i) {            \
      const int row = p * BM + wm * C::WM + 16 * i + lr;                                                       \
      F##a[p][i] = as_bf16x8(*(const u32x4*)(st_ + row * 128 + ((lc_ ^ ((row >> 1) & 7)) << 4)));             \
    }                                                                                                          \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                                           \
      const int row = NP * BM + wn * C::WN + 16 * j + lr;                                                      \
      F##b[j] = as_bf16x8(*(const u32x4*)(st_ + row * 128 + ((lc_ ^ ((row >> 1) & 7)) << 4)));                \
    }                                                                                                          \
  } while (0)
#define FL_MMA(F)                                                                                              \
  do {                                                                                                         \
    _Pragma("unroll") for (int p = 0; p < NP; ++p) _Pragma("unroll") for (int i = 0; i < FM; ++i)             \
        _Pragma("unroll") for (int j = 0; j < FN; ++j) acc[i][j] =                                             \
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(F##a[p][i], F##b[j], acc[i][j], 0, 0, 0);                  \
  } while (0)

  const int nloc = kt1 - kt0;
  bf16x8 f0a[NP][FM], f0b[FN], f1a[NP][FM], f1b[FN];
  if constexpr (BS == 3) {
    // Activation rows in two slots, weight rows in three: a wave's load blocks
    // are all activation rows or all weight rows, and the weight rows of stage
    // it+3 are issued at the stage boundary after stage it, two stage-times
    // before their use (the activation rows of stage it+2, one stage-time).
    const bool a_wave = wid_u * LPT < C::A_BLOCKS;
    const uint32_t dst0 = a_wave ? lds0 + (uint32_t)(wid_u * LPT) * 1024
                                 : lds0 + 2 * C::A_BYTES + (uint32_t)(wid_u * LPT - C::A_BLOCKS) * 1024;
    const uint32_t slot_bytes = a_wave ? C::A_BYTES : C::B_BYTES;
#define FL3_ISSUE(KT, SLOT)                                                                                      \
  do {                                                                                                           \
    const uint32_t k0_ = (uint32_t)(KT) * (BK * 2);                                                              \
    const uint32_t d_ = dst0 + (uint32_t)(SLOT) * slot_bytes;                                                    \
    _Pragma("unroll") for (int q = 0; q < LPT; ++q) {                                                            \
      __builtin_amdgcn_global_load_lds(                                                                          \
          (const __attribute__((address_space(1))) void*)((const char*)bbase[q] + (size_t)(boff[q] + k0_)),      \
          (__attribute__((address_space(3))) void*)(size_t)(d_ + q * 1024), 16, 0, 0);                           \
    }                                                                                                            \
  } while (0)
#define FL3_LOAD(F, SA, SB, H)                                                                                 \
  do {                                                                                                         \
    const unsigned char* sa_ = smem + (SA) * C::A_BYTES;                                                       \
    const unsigned char* sb_ = smem + 2 * C::A_BYTES + (SB) * C::B_BYTES;                                      \
    const int lc_ = 4 * (H) + lq;                                                                              \
    _Pragma("unroll") for (int p = 0; p < NP; ++p) _Pragma("unroll") for (int i = 0; i < FM; ++i) {            \
      const int row = p * BM + wm * C::WM + 16 * i + lr;                                                       \
      F##a[p][i] = as_bf16x8(*(const u32x4*)(sa_ + row * 128 + ((lc_ ^ ((row >> 1) & 7)) << 4)));             \
    }                                                                                                          \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                                           \
      const int row = wn * C::WN + 16 * j + lr;                                                                \
      F##b[j] = as_bf16x8(*(const u32x4*)(sb_ + row * 128 + ((lc_ ^ ((row >> 1) & 7)) << 4)));                \
    }                                                                                                          \
  } while (0)
    if (nloc > 0) FL3_ISSUE(kt0, 0);
    if (nloc > 1) FL3_ISSUE(kt0 + 1, 1);
    if (!a_wave && nloc > 2) FL3_ISSUE(kt0 + 2, 2);
    if (nloc > 0) {
      // stage 0 landed: an activation wave may leave stage 1 in flight, a weight
      // wave stages 1 and 2
      if (a_wave) {
        if (nloc > 1) wait_vmcnt<LPT>();
        else wait_vmcnt<0>();
      } else {
        if (nloc > 2) wait_vmcnt<2 * LPT>();
        else if (nloc > 1) wait_vmcnt<LPT>();
        else wait_vmcnt<0>();
      }
      stage_barrier();
      FL3_LOAD(f0, 0, 0, 0);
    }
    for (int it = 0; it < nloc; ++it) {
      const int sa = it & 1, sb = it % 3, sb1 = sb == 2 ? 0 : sb + 1;
      FL3_LOAD(f1, sa, sb, 1);
      FL_MMA(f0);
      mfma_read_interleave<NP * FM + FN, NP * FM * FN>();
      if (it + 1 < nloc) {
        // stage it+1 landed (a weight wave may still have stage it+2 in flight);
        // every wave holds all of stage it, so its slots take stages it+2 / it+3
        if (a_wave) {
          wait_vmcnt<0>();
        } else {
          if (it + 2 < nloc) wait_vmcnt<LPT>();
          else wait_vmcnt<0>();
        }
        lds_reads_done_barrier();
        if (a_wave) {
          if (it + 2 < nloc) FL3_ISSUE(kt0 + it + 2, sa);
        } else {
          if (it + 3 < nloc) FL3_ISSUE(kt0 + it + 3, sb);
        }
      }
      FL3_LOAD(f0, sa ^ 1, sb1, 0);
      FL_MMA(f1);
      mfma_read_interleave<NP * FM + FN, NP * FM * FN>();
    }
#undef FL3_LOAD
#undef FL3_ISSUE
  } else {
  if (nloc > 0) FL_ISSUE(kt0, 0);
  if (nloc > 1) FL_ISSUE(kt0 + 1, 1);
  if (nloc > 0) {
    if (nloc > 1) wait_vmcnt<LPT>();
    else wait_vmcnt<0>();
    stage_barrier();
    FL_LOAD(f0, 0, 0);
  }
  for (int it = 0; it < nloc; ++it) {
    const int cur = it & 1;
    // first half: MFMAs of half 0 of stage it, reads of its half 1
    FL_LOAD(f1, cur, 1);
    FL_MMA(f0);
    mfma_read_interleave<NP * FM + FN, NP * FM * FN>();
    // stage boundary: stage it+1 landed, every wave holds all of stage it in
    // registers, so its buffer takes stage it+2
    if (it + 1 < nloc) {
      wait_vmcnt<0>();
      lds_reads_done_barrier();
      if (it + 2 < nloc) FL_ISSUE(kt0 + it + 2, cur);
    }
    // second half: MFMAs of half 1, reads of half 0 of stage it+1 (stale and
    // unused after the last stage; unconditional so the MFMAs wait only for
    // their own fragments)
    FL_LOAD(f0, cur ^ 1, 0);
    FL_MMA(f1);
    mfma_read_interleave<NP * FM + FN, NP * FM * FN>();
  }
  }
#undef FL_LOAD
#undef FL_MMA
#undef FL_ISSUE
  wait_vmcnt<0>();   // every copy has landed (no-op here; tells the compiler's wait insertion)
  if constexpr (IL) {
    // MFMA blocks 2k and 2k+1 of a wave are the gate and up values of the
    // same 16 output columns, so SiLU(g) * u is formed and stored straight
    // from the accumulators.
    // Each wave stages its 64 x (WN/2) outputs in a private LDS slice, then
    // stores four consecutive columns per lane (8-byte hi and lo stores).
    if (ksplit == 1) {
      constexpr int OW = C::WN / 2, LDW = OW + 4;
      static_assert(C::NW * 64 * LDW * 4 <= C::SMEM, "per-wave output slices");
      // the slices overlap the pipeline buffers: every wave is done reading
      // them and every copy has landed before any slice is written
      __syncthreads();
      float* wl = (float*)smem + wid * (64 * LDW);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int k = 0; k < FN / 2; ++k)
            wl[(16 * i + 4 * lq + q) * LDW + 16 * k + lr] = silu_fast(acc[i][2 * k][q]) * acc[i][2 * k + 1][q];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's slice is written
      const int ocol0 = n0 / 2 + wn * OW;
      constexpr int C4 = OW / 4;
      // all slice reads first, then the stores
      float4 ov[C4];
#pragma unroll
      for (int t = 0; t < C4; ++t) {
        const int idx = lane + 64 * t, r = idx / C4, c = (idx - r * C4) * 4;
        ov[t] = *(const float4*)(wl + r * LDW + c);
      }
#pragma unroll
      for (int t = 0; t < C4; ++t) {
        const int idx = lane + 64 * t, r = idx / C4, c = (idx - r * C4) * 4;
        const int row = m0 + wm * C::WM + r;
        if (row < M && ocol0 + c < N / 2) act_store4(e.out, row, ocol0 + c, ov[t]);
      }
      return;
    }
  }
  if constexpr (KIND == EPI_LMHEAD && C::WN == 128) {
    // Greedy LM-head partials straight from the accumulators: a wave's 128
    // columns are one partial group; lane (lq, lr) holds rows 16i+4lq+q at
    // columns 16j+lr, so a row is reduced over j in the lane, then over the
    // sixteen lanes sharing lq.  Ties keep the lowest column.
    if (ksplit == 1 && e.temperature == 0.f) {
      const int cbase = n0 + wn * 128;
      if (cbase < N) {
        constexpr float kL2E = 1.4426950408889634f;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = m0 + wm * C::WM + 16 * i + 4 * lq + q;
            float mx = -INFINITY;
            int ix = -1;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int v = cbase + 16 * j + lr;
              const float z = acc[i][j][q];
              if (v < N && (ix < 0 || z > mx)) { mx = z; ix = e.col0 + v; }
            }
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
              const float qm = __shfl_xor(mx, o, kWave);
              const int qi = __shfl_xor(ix, o, kWave);
              if (qi >= 0 && (ix < 0 || qm > mx || (qm == mx && qi < ix))) { mx = qm; ix = qi; }
            }
            float sm = 0.f;
#pragma unroll
            for (int j = 0; j < FN; ++j)
              if (cbase + 16 * j + lr < N) sm += __builtin_amdgcn_exp2f((acc[i][j][q] - mx) * kL2E);
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) sm += __shfl_xor(sm, o, kWave);
            if (r < M) {
              if (lr == 0) {
                const size_t pi = (size_t)r * e.ntiles + (e.col0 + cbase) / 128;
                e.part_f[pi] = make_float4(mx, mx, sm, mx);
                e.part_i[pi] = ix;
              }
              if (e.logits) {
                const size_t base = (size_t)e.row_map[r] * e.ldz + e.col0;
#pragma unroll
                for (int j = 0; j < FN; ++j)
                  if (cbase + 16 * j + lr < N) e.logits[base + cbase + 16 * j + lr] = acc[i][j][q];
              }
            }
          }
      }
      return;
    }
  }
  __syncthreads();   // every wave is done with the pipeline buffers

  // epilogue over 64-row slices of the tile (slice sl = the rows of wave row wm == sl)
  float* Cs = (float*)smem;
#pragma unroll
  for (int sl = 0; sl < WGM; ++sl) {
    if (m0 + sl * 64 >= M) break;
    if (wm == sl) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            Cs[(16 * i + 4 * lq + q) * C::LDC + wn * C::WN + 16 * j + lr] = acc[i][j][q];
    }
    __syncthreads();
    const int ms = m0 + sl * 64;
    if (ksplit > 1) {
      float* dst = part + (size_t)ks * M * N;
      constexpr int C4 = BN / 4;
      for (int idx = tid; idx < 64 * C4; idx += NT) {
        const int r = idx / C4, c = (idx - r * C4) * 4;
        // interleaved SwiGLU columns go back to gate-half / up-half order (runs
        // of four stay within one 16-column group)
        const int cd = IL ? swiglu_il_col(c, BN) : c;
        if (ms + r < M && n0 + c < N)
          *(float4*)(dst + (size_t)(ms + r) * N + n0 + cd) = *(const float4*)(Cs + r * C::LDC + c);
      }
    } else {
      run_epilogue<KIND, 64, BN, NT, bf16_t>(Cs, C::LDC, ms, n0, M, N, e);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// GEMM for at most 16 rows (one or two sequences' blocks).  Each weight is used
// by a single MFMA fragment, so nothing is staged in LDS: every lane loads its
// 16-byte weight and activation operand fragments straight from global memory
// into registers (the activation rows, a few KiB, stay in L1/L2), U k-steps at
// a time so many loads are in flight per wave.  Eight waves of 16 columns make
// a 128-column tile; the K range is split into ksplit parts (summed later in
// split order), and with one part the tile goes through the usual epilogues.
constexpr int kSkinnyBN = 128;

template <int NP, int KIND>
__global__ __launch_bounds__(512) void gemm_skinny_kernel(ActIn a, BRows<bf16_t> b, int M, int N, int K,
                                                          int ksplit, float* part, EpiParams e) {
  // the LM head (no K split: a long K range per wave) takes sixteen steps per
  // batch, twice the bytes in flight per wave (Qwen3-4B shape, 778 MB: 156 ->
  // 143 us, 5.0 -> 5.4 TB/s)
  constexpr int BN = kSkinnyBN, LDC = BN + 4, U = KIND == EPI_LMHEAD ? 16 : 8;
  // activation fragments of one batch, in fragment order [plane][step][lane] (16 B each),
  // double-buffered; each of the NP * U fragments is one 1 KiB direct load
  constexpr int AFRAG = NP * U, ABYTES = AFRAG * 1024;
  static_assert(AFRAG % 8 == 0, "fragments per wave");
  __shared__ __attribute__((aligned(1024))) unsigned char abuf[2 * ABYTES];
  __shared__ __attribute__((aligned(16))) float Cs[16 * LDC];
  const int ntn = (N + BN - 1) / BN;
  const int tn = blockIdx.x % ntn, ks = blockIdx.x / ntn;
  if (ks >= ksplit) return;
  const int n0 = tn * BN;
  const int nkt = K / 32;
  const int kt0 = (int)((long long)ks * nkt / ksplit), kt1 = (int)((long long)(ks + 1) * nkt / ksplit);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  // weight row n of this lane (clamped; columns past N are never stored)
  const bf16_t* brow = b.row(min(n0 + wid * 16 + lr, N - 1), BN) + 8 * lq;
  // activation fragments this wave copies: f = wid * (AFRAG / 8) + t, plane f / U,
  // step f % U, from row lr (clamped; rows past M are never stored)
  const int ar = min(lr, M - 1);
  const bf16_t* asrc[AFRAG / 8];
  int astep[AFRAG / 8];
#pragma unroll
  for (int t = 0; t < AFRAG / 8; ++t) {
    const int f = wid * (AFRAG / 8) + t, p = f / U;
    asrc[t] = (const bf16_t*)(p == 0 ? a.p0 : a.p1) + (size_t)ar * a.ld + 8 * lq;
    astep[t] = f - p * U;
  }
  const uint32_t abase = (uint32_t)(size_t)abuf;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  int buf = 0;
  for (int kt = kt0; kt < kt1; kt += U, buf ^= 1) {
    // a batch of U steps; steps past the range read the last step again and
    // contribute an exact zero (their activation fragment is zeroed)
    bf16x8 bf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) bf[u] = as_bf16x8(*(const u32x4*)(brow + min(kt + u, kt1 - 1) * 32));
#pragma unroll
    for (int t = 0; t < AFRAG / 8; ++t) {
      const int k = min(kt + astep[t], kt1 - 1);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(asrc[t] + k * 32),
          (__attribute__((address_space(3))) void*)(size_t)(abase + buf * ABYTES +
                                                            (wid * (AFRAG / 8) + t) * 1024),
          16, 0, 0);
    }
    wait_vmcnt<0>();
    // the batch's activation fragments are in LDS for every wave; buffer buf was
    // last read in the batch before the previous one, finished before that barrier
    stage_barrier();
    const unsigned char* ab = abuf + buf * ABYTES + lane * 16;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      bf16x8 af[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) af[p] = as_bf16x8(*(const u32x4*)(ab + (p * U + u) * 1024));
      if (kt + u >= kt1) {
#pragma unroll
        for (int p = 0; p < NP; ++p) af[p] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
      }
#pragma unroll
      for (int p = 0; p < NP; ++p) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[p], bf[u], acc, 0, 0, 0);
    }
  }
  // lane (lq, lr) holds rows 4 lq + q of column 16 wid + lr
#pragma unroll
  for (int q = 0; q < 4; ++q) Cs[(4 * lq + q) * LDC + wid * 16 + lr] = acc[q];
  __syncthreads();
  if (ksplit > 1) {
    float* dst = part + (size_t)ks * M * N;
    for (int idx = threadIdx.x; idx < 16 * (BN / 4); idx += 512) {
      const int r = idx / (BN / 4), c = (idx - r * (BN / 4)) * 4;
      if (r < M && n0 + c < N) *(float4*)(dst + (size_t)r * N + n0 + c) = *(const float4*)(Cs + r * LDC + c);
    }
    return;
  }
  run_epilogue<KIND, 16, BN, 512, bf16_t>(Cs, LDC, 0, n0, M, N, e);
}

// The same GEMM (at most 16 rows, 128-column tiles of eight waves, K split into
// ksplit parts) with the activation fragments of the workgroup's whole K range
// copied into LDS once, in fragment order, at the start (at most MAXS 32-deep
// steps), so the loop has no barrier: each wave streams its weight fragments
// in batches of eight steps, the next batch's loads issued before the current
// batch's MFMAs.  Used for splits of more than two batches (the one-sequence
// down projection: 19.5 -> 17.4 us at the Qwen3-4B shape); the LM head keeps
// gemm_skinny_kernel.
template <int NP, int KIND, int MAXS>
__global__ __launch_bounds__(512) void gemm_skinny_a1_kernel(ActIn a, BRows<bf16_t> b, int M, int N, int K,
                                                             int ksplit, float* part, EpiParams e) {
  constexpr int BN = kSkinnyBN, LDC = BN + 4, U = 8;
  __shared__ __attribute__((aligned(1024))) unsigned char abuf[NP * MAXS * 1024];
  __shared__ __attribute__((aligned(16))) float Cs[16 * LDC];
  const int ntn = (N + BN - 1) / BN;
  const int tn = blockIdx.x % ntn, ks = blockIdx.x / ntn;
  if (ks >= ksplit) return;
  const int n0 = tn * BN;
  const int nkt = K / 32;
  const int kt0 = (int)((long long)ks * nkt / ksplit), kt1 = (int)((long long)(ks + 1) * nkt / ksplit);
  const int nk = kt1 - kt0;   // at most MAXS (the launcher checks)
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wid_u = __builtin_amdgcn_readfirstlane(wid);
  const int lr = lane & 15, lq = lane >> 4;
  // weight row of this lane (clamped; columns past N are never stored)
  const bf16_t* brow = b.row(min(n0 + wid * 16 + lr, N - 1), BN) + 8 * lq;
  // activation fragment f = p * nk + t (plane p, step kt0 + t) at abuf + 1024 f,
  // lane-ordered; wave w copies f = w, w + 8, ... (clamped to the last
  // fragment, whose copy is then repeated; rows past M read row M - 1, never
  // stored).  The copies go through registers rather than direct-to-LDS loads,
  // so the compiler's wait counting stays exact for the weight loads below.
  constexpr int AMAX = (NP * MAXS + 7) / 8;
  u32x4 av[AMAX];
  {
    const int ar = min(lr, M - 1);
#pragma unroll
    for (int i = 0; i < AMAX; ++i) {
      const int f = min(wid_u + 8 * i, NP * nk - 1), pl = f >= nk ? 1 : 0, t = f - pl * nk;
      av[i] = *(const u32x4*)((const bf16_t*)(pl == 0 ? a.p0 : a.p1) + (size_t)ar * a.ld + 8 * lq + (kt0 + t) * 32);
    }
  }
  bf16x8 bw[2][U];
#pragma unroll
  for (int u = 0; u < U; ++u) bw[0][u] = as_bf16x8(*(const u32x4*)(brow + min(kt0 + u, kt1 - 1) * 32));
#pragma unroll
  for (int i = 0; i < AMAX; ++i) {
    const int f = min(wid_u + 8 * i, NP * nk - 1);
    *(u32x4*)(abuf + f * 1024 + lane * 16) = av[i];
  }
  lds_reads_done_barrier();   // every wave's fragment stores are in LDS (the weight loads stay in flight)
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const unsigned char* al = abuf + lane * 16;
  // batches of U steps, two per iteration (register sets 0 and 1), the range
  // padded to an even number of batches; steps past the range read the last
  // step again and add an exact zero (their activation fragments are zeroed),
  // so every load and MFMA is unconditional and the loads of the next batch
  // stay in flight under the MFMAs of this one
#define SK_BATCH(CUR, NXT, KT)                                                                                 \
  do {                                                                                                         \
    _Pragma("unroll") for (int u = 0; u < U; ++u)                                                              \
        bw[NXT][u] = as_bf16x8(*(const u32x4*)(brow + min((KT) + U + u, kt1 - 1) * 32));                       \
    __builtin_amdgcn_sched_barrier(0);                                                                         \
    _Pragma("unroll") for (int u = 0; u < U; ++u) {                                                            \
      const int t_ = (KT) - kt0 + u;                                                                           \
      const uint32_t live_ = (KT) + u < kt1 ? ~0u : 0u;   /* uniform: a mask, not a branch */                  \
      bf16x8 af_[NP];                                                                                          \
      _Pragma("unroll") for (int p = 0; p < NP; ++p)                                                           \
          af_[p] = as_bf16x8(*(const u32x4*)(al + (size_t)(p * nk + min(t_, nk - 1)) * 1024) & live_);         \
      _Pragma("unroll") for (int p = 0; p < NP; ++p)                                                           \
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af_[p], bw[CUR][u], acc, 0, 0, 0);                     \
    }                                                                                                          \
  } while (0)
  for (int kt = kt0; kt < kt1; kt += 2 * U) {
    SK_BATCH(0, 1, kt);
    SK_BATCH(1, 0, kt + U);
  }
#undef SK_BATCH
  // lane (lq, lr) holds rows 4 lq + q of column 16 wid + lr
#pragma unroll
  for (int q = 0; q < 4; ++q) Cs[(4 * lq + q) * LDC + wid * 16 + lr] = acc[q];
  __syncthreads();
  if (ksplit > 1) {
    float* dst = part + (size_t)ks * M * N;
    for (int idx = threadIdx.x; idx < 16 * (BN / 4); idx += 512) {
      const int r = idx / (BN / 4), c = (idx - r * (BN / 4)) * 4;
      if (r < M && n0 + c < N) *(float4*)(dst + (size_t)r * N + n0 + c) = *(const float4*)(Cs + r * LDC + c);
    }
    return;
  }
  run_epilogue<KIND, 16, BN, 512, bf16_t>(Cs, LDC, 0, n0, M, N, e);
}

// Sum of the split-K partials of RB rows x BN columns (a row slice of one GEMM
// tile: every epilogue is row-independent), in split order, then the epilogue.
template <int RB, int BN, int KIND, typename TP>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* part, int ksplit, int M, int N,
                                                             EpiParams e, const int* m_dev) {
  constexpr int LDC = BN + 4;
  __shared__ __attribute__((aligned(16))) float Cs[RB * LDC];
  const int nrb = (M + RB - 1) / RB;
  const int rb = blockIdx.x % nrb, tn = blockIdx.x / nrb;
  const int m0 = rb * RB, n0 = tn * BN;
  const int Mp = M;   // row stride of the partials
  if (m_dev) M = min(M, max(*m_dev, 0));
  if (m0 >= M) return;
  constexpr int C4 = BN / 4;
  for (int idx = threadIdx.x; idx < RB * C4; idx += 256) {
    const int r = idx / C4, c = (idx - r * C4) * 4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (m0 + r < M && n0 + c < N) {
      for (int k = 0; k < ksplit; ++k) {
        const float4 v = *(const float4*)(part + ((size_t)k * Mp + m0 + r) * N + n0 + c);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
    }
    *(float4*)(Cs + r * LDC + c) = acc;
  }
  __syncthreads();
  run_epilogue<KIND, RB, BN, 256, TP>(Cs, LDC, m0, n0, M, N, e);
}

// ---------------------------------------------------------------------------
template <int KIND>
__global__ __launch_bounds__(256) void gemm_f32_kernel(ActIn a, BRows<float> b, int M, int N, int K,
                                                       EpiParams e) {
  constexpr int BM = 64, BN = 128, BK = 16, NT = 256, LDA = BM + 4, LDB = BN + 4, LDC = BN + 4;
  constexpr int STAGE = BK * (LDA + LDB) * 4, EPI = BM * LDC * 4;
  constexpr int SMEM = STAGE > EPI ? STAGE : EPI;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  float* As = (float*)smem;          // [BK][BM+4]
  float* Bs = As + BK * LDA;         // [BK][BN+4]
  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  int tm, tn;
  if (!tile_of(ntm, ntm * ntn, tm, tn)) return;
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const float* A = (const float*)a.p0;
  float acc[4][8] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + j * NT, r = c >> 4, k = c & 15;
      As[k * LDA + r] = (m0 + r < M) ? A[(size_t)(m0 + r) * a.ld + k0 + k] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = tid + j * NT, r = c >> 4, k = c & 15;
      Bs[k * LDB + r] = (n0 + r < N) ? b.row(n0 + r, BN)[k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float av[4], bv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[k * LDA + ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) bv[j] = Bs[k * LDB + tx * 8 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* Cs = (float*)smem;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) Cs[(ty * 4 + i) * LDC + tx * 8 + j] = acc[i][j];
  __syncthreads();
  run_epilogue<KIND, BM, BN, NT, float>(Cs, LDC, m0, n0, M, N, e);
}

// fp32 GEMM for at most 16 rows (the fp32 workloads' draft forwards and step
// injections, latency-bound): the rows' activations are copied to LDS once
// (direct 16-byte loads, all in flight together), then each wave takes groups
// of G columns, loads every weight it needs for a group at once (lanes across
// K: contiguous runs of the weight rows) and, row by row, forms the dot
// products in registers and sums them over the wave.  BN columns per
// workgroup; the usual epilogues over the 16-row tile.  KK = K / 64 rounded up
// to 4, 8 or 16; a group holds at most 64 weights per lane, so it has
// min(64 / KK, 8) columns.  Rows are 16-byte aligned with K a multiple of 4
// (checked by the host).
constexpr int kF32RowsMaxK = 1024;
template <int KIND, int BN, int KK>
__global__ __launch_bounds__(256) void gemm_f32_rows_kernel(ActIn a, BRows<float> b, int M, int N, int K,
                                                            EpiParams e) {
  constexpr int G0 = (64 / KK < BN / 4) ? 64 / KK : BN / 4, G = G0 < 8 ? G0 : 8, LDC = BN + 4, GPW = BN / 4 / G;
  static_assert(BN % (4 * G) == 0 && KK * 64 <= kF32RowsMaxK, "columns per wave");
  __shared__ __attribute__((aligned(1024))) float As[16 * kF32RowsMaxK];
  __shared__ __attribute__((aligned(16))) float Cs[16 * LDC];
  const int n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float* A = (const float*)a.p0;
  {
    // 1 KiB blocks (256 floats of a row); lanes past the row's end read its last
    // four values again (their LDS slots are never used)
    const int nkb = (K + 255) / 256;
    const uint32_t as0 = (uint32_t)(size_t)As;
    for (int f = wid; f < M * nkb; f += 4) {
      const int m = f / nkb, kb = f - m * nkb;
      const int k = min(kb * 256 + lane * 4, K - 4);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(A + (size_t)m * a.ld + k),
                                       (__attribute__((address_space(3))) void*)(size_t)(
                                           as0 + (uint32_t)(m * kF32RowsMaxK + kb * 256) * 4),
                                       16, 0, 0);
    }
    wait_vmcnt<0>();
    __syncthreads();
  }
  for (int gi = 0; gi < GPW; ++gi) {
    const int c0 = (wid * GPW + gi) * G;
    float w[G][KK];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float* br = b.row(min(n0 + c0 + j, N - 1), BN);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int k = lane + 64 * kk;
        w[j][kk] = k < K ? br[k] : 0.f;
      }
    }
    // rows: a runtime loop (the arrays are indexed by unrolled constants only)
    for (int m = 0; m < M; ++m) {
      float acc[G];
#pragma unroll
      for (int j = 0; j < G; ++j) acc[j] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int k = lane + 64 * kk;
        const float av = k < K ? As[m * kF32RowsMaxK + k] : 0.f;
#pragma unroll
        for (int j = 0; j < G; ++j) acc[j] = fmaf(av, w[j][kk], acc[j]);
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float v = acc[j];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
        if (lane == 0) Cs[m * LDC + c0 + j] = v;
      }
    }
  }
  __syncthreads();
  run_epilogue<KIND, 16, BN, 256, float>(Cs, LDC, 0, n0, M, N, e);
}

// ---------------------------------------------------------------------------
// Tile choice per GEMM kind (bf16 weights):
//   2: 128x128, four 64x64 waves, two workgroups per CU (gemm_dma_kernel;
//      injection, and K not a multiple of 64)
//   10: 128x384, eight 64x96 waves     11: 256x256, eight 64x128 waves (one plane)
//   12: 128x256, eight 64x64 waves     13: 64x256, eight 64x32 waves (one plane, at most 64 rows)
//   (gemm_fl_kernel, one workgroup per CU, two for 13)
constexpr int kCfgSwiglu = 10;       // gate/up + SwiGLU
constexpr int kCfgLmhead = 11;       // LM head (one bf16 plane)
constexpr int kCfgAdd = 12;          // O and down + residual
constexpr int kCfgStore = 10;        // q/k/v
static int tile_bn(int cfg) {
  return cfg == 10 ? 384 : cfg >= 11 ? 256 : 128;
}
static int tile_bm(int cfg) { return cfg == 11 ? 256 : cfg == 13 ? 64 : 128; }

// LM-head partials cover 128 columns each, or 64 when the tile width is not a multiple of 128
int gemm_bn(int wdtype, int K) { return wdtype && K % 32 == 0 && tile_bn(kCfgLmhead) % 128 ? 64 : 128; }

// Tile configuration and K split of one GEMM (the table above).  A split is
// used only when the tiles alone leave CUs idle; with fixed_split the split
// depends on N and K only (injection must give the same bits for any M).
constexpr int kInjectWgTarget = 256;   // workgroups the injection's fixed K split aims for
// Estimated time (us) of a SwiGLU GEMM on tile config c with its best K split
// (returned in ks): whole rounds of one tile per CU at the sustained per-CU
// MFMA rate (about 5 TFLOP/s of executed work), plus, for a split, the reduce
// pass over the fp32 partials at HBM speed (about 5 TB/s).
static double swiglu_split_us(int c, int np, int M, int N, int K, int& ks_out) {
  const int bm = tile_bm(c), bn = tile_bn(c), cus = 256;
  const int tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const double tile_us = 2.0 * np * bm * bn * (double)K / 5.1e12 * 1e6;
  const int cap = std::min(8, std::max(1, K / 32 / 16));
  double best = 1e30;
  for (int ks = 1; ks <= cap; ++ks) {
    const double rounds = (double)((tiles * ks + cus - 1) / cus);
    const double reduce_us = ks > 1 ? (ks + 0.5) * (double)M * N * 4.0 / 5e12 * 1e6 : 0.0;
    const double us = rounds * tile_us / ks + reduce_us;
    if (us < best - 1e-9) { best = us; ks_out = ks; }
  }
  return best;
}

GemmPlan gemm_plan(int wdtype, int a_mode, int M, int N, int K, int kind, bool fixed_split) {
  GemmPlan p{0, 1};
  if (wdtype == 0) return p;
  int cfg = 2;
  if (!fixed_split && K % 32 == 0) {
    if (kind == EPI_SWIGLU) cfg = kCfgSwiglu;
    else if (kind == EPI_LMHEAD) cfg = M > 64 ? kCfgLmhead : 13;
    else if (kind == EPI_ADD) cfg = kCfgAdd;
    else if (kind == EPI_STORE) cfg = kCfgStore;
    const bool one_plane = a_mode != ACT_HILO;
    if ((cfg == 11 || cfg == 13) && !one_plane) cfg = 12;
    if (cfg >= 10 && K % 64 != 0) cfg = 2;
    // SwiGLU tiles hold BN/2 gate and BN/2 up columns of the same rows
    if (kind == EPI_SWIGLU && (N / 2) % (tile_bn(cfg) / 2) != 0) cfg = (N / 2) % 128 == 0 && K % 64 == 0 ? 12 : 2;
  }
  // at most 16 rows: weights streamed straight into registers (gemm_skinny_kernel);
  // the K split gives each wave about two batches of eight 32-deep steps (at most
  // eight parts, so the consumer folds few partials) and depends on K only
  if (!fixed_split && M <= 16 && K % 32 == 0 && kind != EPI_KVSCATTER) {
    p.cfg = 20;
    const int nkt = K / 32;
    p.ksplit = kind == EPI_LMHEAD ? 1 : std::max(1, std::min({(nkt + 15) / 16, 8, nkt}));
    return p;
  }
  p.cfg = cfg;
  if (cfg == 2) {
    const int nkt = K / 32;
    const int tn = (N + 127) / 128;
    const int tiles = (fixed_split ? 1 : (M + 127) / 128) * tn;
    int ks = (kInjectWgTarget + tiles - 1) / tiles;
    ks = std::min(ks, std::max(1, nkt / 4));
    ks = std::max(ks, 1);
    if (kind == EPI_LMHEAD) ks = 1;
    p.ksplit = ks;
    return p;
  }
  if (kind == EPI_SWIGLU && (cfg == 10 || cfg == 12)) {
    // SwiGLU partials need a reduce pass of their own (the activation is not
    // linear), so the split is priced with it, and the 128x384 and 128x256
    // tiles are compared: with 544 rows the wide tile leaves a fifth row of
    // tiles that only a four-way split (and its reduce) packs into whole rounds
    int best_cfg = cfg, best_ks = 1;
    double best_us = 1e30;
    const int np = a_mode == ACT_HILO ? 2 : 1;
    for (int c : {10, 12}) {
      if ((N / 2) % (tile_bn(c) / 2) != 0 || K % 64 != 0) continue;
      int ks = 1;
      const double us = swiglu_split_us(c, np, M, N, K, ks);
      if (us < best_us - 1e-9) { best_us = us; best_cfg = c; best_ks = ks; }
    }
    p.cfg = best_cfg;
    p.ksplit = best_ks;
    return p;
  }
  // one workgroup per CU: pick the split that minimises rounds per unit of work
  const int bm = tile_bm(cfg), bn = tile_bn(cfg);
  const int tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int cap = kind == EPI_LMHEAD ? 1 : std::max(1, K / 32 / 16);
  const int cus = 256;
  double best = 1e30;
  for (int ks = 1; ks <= std::min(cap, 8); ++ks) {
    const double cost = (double)((tiles * ks + cus - 1) / cus) / ks;
    if (cost < best - 1e-9) { best = cost; p.ksplit = ks; }
  }
  (void)a_mode;
  return p;
}

size_t gemm_partial_bytes(const GemmPlan& p, int M, int N) {
  return p.ksplit > 1 ? (size_t)p.ksplit * M * N * 4 : 0;
}

template <int KIND>
static hipError_t go_f32(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 16 && g.K <= kF32RowsMaxK && g.K >= 4 && g.K % 4 == 0 && g.a.ld % 4 == 0 &&
      (uintptr_t)g.a.p0 % 16 == 0) {
    // LM-head partials and the KV scatter's rotated heads need 128-column tiles
    constexpr int BN = (KIND == EPI_LMHEAD || KIND == EPI_KVSCATTER) ? 128 : 32;
    BRows<float> b{(const float*)g.b.b0, (const float*)g.b.b1, g.b.ldb, g.b.split, g.b.mode};
    const dim3 grid((g.N + BN - 1) / BN);
    if (g.K <= 256)
      hipLaunchKernelGGL((gemm_f32_rows_kernel<KIND, BN, 4>), grid, dim3(256), 0, s, g.a, b, g.M, g.N, g.K, g.e);
    else if (g.K <= 512)
      hipLaunchKernelGGL((gemm_f32_rows_kernel<KIND, BN, 8>), grid, dim3(256), 0, s, g.a, b, g.M, g.N, g.K, g.e);
    else
      hipLaunchKernelGGL((gemm_f32_rows_kernel<KIND, BN, 16>), grid, dim3(256), 0, s, g.a, b, g.M, g.N, g.K, g.e);
    return hipGetLastError();
  }
  const int total = ((g.M + 63) / 64) * ((g.N + 127) / 128);
  const int grid = (total + 7) / 8 * 8;
  BRows<float> b{(const float*)g.b.b0, (const float*)g.b.b1, g.b.ldb, g.b.split, g.b.mode};
  hipLaunchKernelGGL((gemm_f32_kernel<KIND>), dim3(grid), dim3(256), 0, s, g.a, b, g.M, g.N, g.K, g.e);
  return hipGetLastError();
}

template <int NP, int KIND>
static hipError_t go_dma(const GemmArgs& g, int ksplit, hipStream_t s) {
  const int ntm = (g.M + 127) / 128, ntn = (g.N + 127) / 128;
  const int total = ntm * ntn * ksplit;
  const int grid = (total + 7) / 8 * 8;
  BRows<bf16_t> b{(const bf16_t*)g.b.b0, (const bf16_t*)g.b.b1, g.b.ldb, g.b.split, g.b.mode};
  hipLaunchKernelGGL((gemm_dma_kernel<NP, KIND>), dim3(grid), dim3(256), 0, s, g.a, b, g.M, g.N, g.K, ksplit, g.part,
                     g.e, g.m_dev);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || ksplit == 1 || (g.defer_reduce && (KIND == EPI_ADD || KIND == EPI_STORE))) return err;
  hipLaunchKernelGGL((splitk_reduce_kernel<16, 128, KIND, bf16_t>), dim3((g.M + 15) / 16 * ntn), dim3(256), 0, s,
                     g.part, ksplit, g.M, g.N, g.e, g.m_dev);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int NP, int KIND, int BS = 2>
static hipError_t go_fl(const GemmArgs& g, int ksplit, hipStream_t s) {
  const int ntm = (g.M + BM - 1) / BM, ntn = (g.N + BN - 1) / BN;
  const int total = ntm * ntn * ksplit;
  const int grid = (total + 7) / 8 * 8;
  BRows<bf16_t> b{(const bf16_t*)g.b.b0, (const bf16_t*)g.b.b1, g.b.ldb, g.b.split, g.b.mode};
  hipLaunchKernelGGL((gemm_fl_kernel<BM, BN, WGM, WGN, NP, KIND, BS>), dim3(grid), dim3(64 * WGM * WGN), 0, s, g.a, b,
                     g.M, g.N, g.K, ksplit, g.part, g.e);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || ksplit == 1 || (g.defer_reduce && (KIND == EPI_ADD || KIND == EPI_STORE))) return err;
  hipLaunchKernelGGL((splitk_reduce_kernel<16, BN, KIND, bf16_t>), dim3((g.M + 15) / 16 * ntn), dim3(256), 0, s,
                     g.part, ksplit, g.M, g.N, g.e, nullptr);
  return hipGetLastError();
}

template <int NP, int KIND>
static hipError_t go_skinny(const GemmArgs& g, int ksplit, hipStream_t s) {
  const int ntn = (g.N + kSkinnyBN - 1) / kSkinnyBN;
  BRows<bf16_t> b{(const bf16_t*)g.b.b0, (const bf16_t*)g.b.b1, g.b.ldb, g.b.split, g.b.mode};
  // splits of more than two batches (the down projection) stage their activations
  // once; shorter ones gain nothing from it and lose occupancy to its registers
  const int steps = (g.K / 32 + ksplit - 1) / ksplit;   // longest K range of a split
  if (KIND != EPI_LMHEAD && steps > 16 && steps <= 40)
    hipLaunchKernelGGL((gemm_skinny_a1_kernel<NP, KIND, 40>), dim3(ntn * ksplit), dim3(512), 0, s, g.a, b, g.M, g.N,
                       g.K, ksplit, g.part, g.e);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<NP, KIND>), dim3(ntn * ksplit), dim3(512), 0, s, g.a, b, g.M, g.N, g.K,
                       ksplit, g.part, g.e);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || ksplit == 1 || (g.defer_reduce && (KIND == EPI_ADD || KIND == EPI_STORE))) return err;
  hipLaunchKernelGGL((splitk_reduce_kernel<16, kSkinnyBN, KIND, bf16_t>), dim3((g.M + 15) / 16 * ntn), dim3(256), 0,
                     s, g.part, ksplit, g.M, g.N, g.e, nullptr);
  return hipGetLastError();
}

template <int NP, int KIND>
static hipError_t go_bf16(const GemmArgs& g, const GemmPlan& p, hipStream_t s) {
  constexpr bool scatter = KIND == EPI_KVSCATTER;
  switch (p.cfg) {
    case 20: if constexpr (!scatter) return go_skinny<NP, KIND>(g, p.ksplit, s); break;
    case 2: return go_dma<NP, KIND>(g, p.ksplit, s);
    case 10: if constexpr (!scatter) return go_fl<128, 384, 2, 4, NP, KIND>(g, p.ksplit, s); break;
    case 11: if constexpr (NP == 1 && !scatter) return go_fl<256, 256, 4, 2, 1, KIND, 3>(g, p.ksplit, s); break;
    case 12: if constexpr (!scatter) return go_fl<128, 256, 2, 4, NP, KIND>(g, p.ksplit, s); break;
    case 13: if constexpr (NP == 1 && !scatter) return go_fl<64, 256, 1, 8, 1, KIND>(g, p.ksplit, s); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

int gemm_ksplit(const GemmArgs& g) {
  if (g.wdtype == 0) return 1;
  return gemm_plan(g.wdtype, g.a.mode, g.M, g.N, g.K, g.kind, g.fixed_split).ksplit;
}

// LM head on 256 x 256 tiles (one workgroup per CU): the column tiles of the
// last, partly filled round run as a second launch with their K range split
// ks ways (ks partial tiles of a third or a half of the work fill the CUs the
// round would leave idle), and their partials are summed in split order before
// the argmax / log-sum-exp epilogue.  The second denoise step's 256 rows make
// 594 tiles: two whole rounds, then 82 tiles split three ways.  Returns the
// columns of the whole rounds (0: no split) and ks.
static int lmhead_split(int M, int N, int& ks) {
  ks = 1;
  if (N % 4) return 0;   // the partials are summed four columns at a time
  const int cus = 256, ntm = (M + 255) / 256, ntn = (N + 255) / 256;
  const int c = (ntm * ntn / cus) * cus / ntm;   // column tiles in whole rounds
  const int rem = ntn - c;
  ks = rem > 0 ? std::min(4, cus / (ntm * rem)) : 1;
  return (c > 0 && ks >= 2) ? c * 256 : 0;
}

size_t gemm_lmhead_part_bytes(int M, int N) {
  size_t best = 0;
  for (int ntm = 1; ntm <= (M + 255) / 256; ++ntm) {
    const int m = std::min(M, ntm * 256);
    if (m <= 64) continue;   // at most 64 rows: 64 x 256 tiles, no split
    int ks = 1;
    const int cols = lmhead_split(m, N, ks);
    if (cols > 0) best = std::max(best, (size_t)ks * m * (N - cols) * 4);
  }
  return best;
}

hipError_t launch_gemm(const GemmArgs& g_in, hipStream_t s) {
  if (g_in.M <= 0 || g_in.N <= 0) return hipSuccess;
  GemmArgs g = g_in;
  if (g.kind == EPI_LMHEAD) {
    g.e.col0 = 0;
    g.e.ldz = g.N;
  }
  if (g.wdtype == 0) {
    if (g.m_dev || g.a.rows) return hipErrorInvalidValue;
    switch (g.kind) {
      case EPI_STORE: return go_f32<EPI_STORE>(g, s);
      case EPI_ADD: return go_f32<EPI_ADD>(g, s);
      case EPI_SWIGLU: return go_f32<EPI_SWIGLU>(g, s);
      case EPI_LMHEAD: return go_f32<EPI_LMHEAD>(g, s);
      case EPI_KVSCATTER: return go_f32<EPI_KVSCATTER>(g, s);
    }
    return hipErrorInvalidValue;
  }
  const GemmPlan p = gemm_plan(g.wdtype, g.a.mode, g.M, g.N, g.K, g.kind, g.fixed_split);
  if (p.ksplit > 1 && !g.part) return hipErrorInvalidValue;
  // a device row count and a row gather are carried by tile configuration 2 only
  if ((g.m_dev || g.a.rows) && p.cfg != 2) return hipErrorInvalidValue;
  if (g.a.mode == ACT_HILO) {
    switch (g.kind) {
      case EPI_STORE: return go_bf16<2, EPI_STORE>(g, p, s);
      case EPI_ADD: return go_bf16<2, EPI_ADD>(g, p, s);
      case EPI_SWIGLU: return go_bf16<2, EPI_SWIGLU>(g, p, s);
      case EPI_KVSCATTER: return go_bf16<2, EPI_KVSCATTER>(g, p, s);
    }
  } else {
    switch (g.kind) {
      case EPI_STORE: return go_bf16<1, EPI_STORE>(g, p, s);
      case EPI_LMHEAD: {
        int ks = 1;
        const int cols = p.cfg == 11 && g.part ? lmhead_split(g.M, g.N, ks) : 0;
        if (cols == 0 || (size_t)ks * g.M * (g.N - cols) * 4 > g.part_cap) return go_bf16<1, EPI_LMHEAD>(g, p, s);
        GemmArgs g1 = g, g2 = g;
        g1.N = cols;
        g2.N = g.N - cols;
        g2.b.b0 = (const bf16_t*)g.b.b0 + (size_t)cols * g.b.ldb;
        g2.e.col0 = cols;
        const hipError_t err = go_fl<256, 256, 4, 2, 1, EPI_LMHEAD, 3>(g1, 1, s);
        if (err != hipSuccess) return err;
        return go_fl<256, 256, 4, 2, 1, EPI_LMHEAD, 3>(g2, ks, s);
      }
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace dflash
