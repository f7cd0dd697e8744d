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
      a.x = g.x / (1.f + expf(-g.x)) * u.x;
      a.y = g.y / (1.f + expf(-g.y)) * u.y;
      a.z = g.z / (1.f + expf(-g.z)) * u.z;
      a.w = g.w / (1.f + expf(-g.w)) * u.w;
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
        const size_t base = (size_t)e.row_map[row] * N;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (n0 + c + q < N) e.logits[base + n0 + c + q] = Cs[r * ldc + c + q];
      }
    }
    constexpr int TPR = NT / BM;      // threads per row
    constexpr int CPT = BN / TPR;     // columns per thread
    static_assert(NT % BM == 0 && BN % TPR == 0, "tile split");
    const int r = tid / TPR, q = tid - r * TPR;
    const int row = m0 + r;
    const bool rv = row < M;
    const float T = e.temperature;
    const bool samp = T > 0.f;
    const float invT = samp ? 1.f / T : 1.f;
    int bi = 0, bb = 0;
    if (rv) {
      const int rm = e.row_map[row];
      bb = rm / e.block;
      bi = rm - bb * e.block;
    }
    LMPart P;
    P.pmax = -INFINITY; P.zmax = -INFINITY; P.zsum = 0.f; P.zc = -INFINITY; P.idx = -1;
    const int c0 = q * CPT;
    if (rv) {
      for (int c = 0; c < CPT; c += 4) {
        const int v0 = n0 + c0 + c;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (samp && v0 < N)
          w = philox4x32_10(make_uint4((uint32_t)(v0 >> 2), (uint32_t)bi, (uint32_t)e.step, (uint32_t)bb),
                            e.seed_lo, e.seed_hi);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int v = v0 + k;
          if (v >= N) break;
          const float zt = samp ? Cs[r * ldc + c0 + c + k] / T : Cs[r * ldc + c0 + c + k];
          const float sc = samp ? zt + gumbel_from_word(ww[k]) : zt;
          if (sc > P.pmax || P.idx < 0) { P.pmax = sc; P.idx = v; P.zc = zt; }
          P.zmax = fmaxf(P.zmax, zt);
        }
      }
      for (int c = 0; c < CPT; ++c) {
        if (n0 + c0 + c >= N) break;
        const float zt = samp ? Cs[r * ldc + c0 + c] / T : Cs[r * ldc + c0 + c];
        P.zsum += expf(zt - P.zmax);
      }
    }
    (void)invT;
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
    if (rv && q == 0) {
      const size_t pi = (size_t)row * e.ntiles + n0 / BN;
      e.part_f[pi] = make_float4(P.pmax, P.zmax, P.zsum, P.zc);
      e.part_i[pi] = P.idx;
    }
  } else if constexpr (KIND == EPI_KVSCATTER) {
    const int d = e.head_dim, hd = d / 2, nkv = e.n_kv;
    const int hpt = BN / d;  // heads per tile
    for (int idx = tid; idx < BM * hpt * hd; idx += NT) {
      const int r = idx / (hpt * hd);
      const int rem = idx - r * hpt * hd;
      const int hb = rem / hd, j = rem - hb * hd;
      const int row = m0 + r, col0 = n0 + hb * d;
      if (row >= M || col0 >= N) continue;
      const int head = col0 / d;           // ((l * 2 + kv) * nkv + m)
      const int m = head % nkv, kv = (head / nkv) & 1, l = head / (2 * nkv);
      const int b = e.tok_seq[row], pos = e.tok_pos[row];
      if (b < 0 || b >= e.n_seqs || pos < 0) continue;
      const int lp = pos >> 4, slot = pos & 15;
      if (lp >= e.max_pages) continue;
      const int phys = e.block_table[(size_t)b * e.max_pages + lp];
      if (phys < 0 || phys >= e.n_pages) continue;
      const float x0 = Cs[r * ldc + hb * d + j], x1 = Cs[r * ldc + hb * d + j + hd];
      TP* chunk = (TP*)e.pool + ((((size_t)phys * e.n_layers + l) * 2 + kv) * nkv + m) * (size_t)(16 * d);
      if (kv == 0) {
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
template <int BM, int BN, int WM, int WN, bool HILO, int KIND>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_mfma_kernel(
    ActIn a, BRows<bf16_t> b, int M, int N, int K, EpiParams e) {
  constexpr int BK = 64, LDK = BK + 8;
  constexpr int NWN = BN / WN, NT = (BM / WM) * NWN * 64;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int NP = HILO ? 2 : 1;
  constexpr int APER = BM * BK / 8 / NT, BPER = BN * BK / 8 / NT;
  static_assert(APER * NT == BM * BK / 8 && BPER * NT == BN * BK / 8, "load split");
  constexpr int LDC = BN + 4;
  constexpr int STAGE = (NP * BM + BN) * LDK * 2;
  constexpr int EPI = BM * LDC * 4;
  constexpr int SMEM = STAGE > EPI ? STAGE : EPI;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  bf16_t* As = (bf16_t*)smem;
  bf16_t* Bs = As + NP * BM * LDK;

  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  int tm, tn;
  if (!tile_of(ntm, ntm * ntn, tm, tn)) return;
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / NWN, wn = wid - (wid / NWN) * NWN;

  const bf16_t* ap[2] = {(const bf16_t*)a.p0, (const bf16_t*)a.p1};
  uint4 ra[NP][APER], rb[BPER];
  const uint4 z4 = make_uint4(0, 0, 0, 0);

  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < APER; ++j) {
      const int c = tid + j * NT, r = c >> 3, kc = (c & 7) * 8;
      const int row = m0 + r;
#pragma unroll
      for (int p = 0; p < NP; ++p)
        ra[p][j] = row < M ? *(const uint4*)(ap[p] + (size_t)row * a.ld + k0 + kc) : z4;
    }
#pragma unroll
    for (int j = 0; j < BPER; ++j) {
      const int c = tid + j * NT, r = c >> 3, kc = (c & 7) * 8;
      const int n = n0 + r;
      rb[j] = n < N ? *(const uint4*)(b.row(n, BN) + k0 + kc) : z4;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int j = 0; j < APER; ++j) {
      const int c = tid + j * NT, r = c >> 3, kc = (c & 7) * 8;
#pragma unroll
      for (int p = 0; p < NP; ++p) *(uint4*)(As + (p * BM + r) * LDK + kc) = ra[p][j];
    }
#pragma unroll
    for (int j = 0; j < BPER; ++j) {
      const int c = tid + j * NT, r = c >> 3, kc = (c & 7) * 8;
      *(uint4*)(Bs + r * LDK + kc) = rb[j];
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  gload(0);
  sstore();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int kof = ks * 32 + 8 * (lane >> 4);
      bf16x8 af[NP][TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int p = 0; p < NP; ++p)
          af[p][i] = as_bf16x8(*(const uint4*)(As + (p * BM + wm * WM + 16 * i + (lane & 15)) * LDK + kof));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = as_bf16x8(*(const uint4*)(Bs + (wn * WN + 16 * j + (lane & 15)) * LDK + kof));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int p = 0; p < NP; ++p)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[p][i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      sstore();
      __syncthreads();
    }
  }

  float* Cs = (float*)smem;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        Cs[(wm * WM + 16 * i + 4 * (lane >> 4) + q) * LDC + wn * WN + 16 * j + (lane & 15)] = acc[i][j][q];
  __syncthreads();
  run_epilogue<KIND, BM, BN, NT, bf16_t>(Cs, LDC, m0, n0, M, N, e);
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

// ---------------------------------------------------------------------------
int gemm_bn(int) { return 128; }

template <int BM, int BN, int WM, int WN, bool HILO, int KIND>
static hipError_t go_mfma(const GemmArgs& g, hipStream_t s) {
  const int ntm = (g.M + BM - 1) / BM, ntn = (g.N + BN - 1) / BN;
  const int total = ntm * ntn;
  const int grid = (total + 7) / 8 * 8;
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  BRows<bf16_t> b{(const bf16_t*)g.b.b0, (const bf16_t*)g.b.b1, g.b.ldb, g.b.split, g.b.mode};
  hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WM, WN, HILO, KIND>), dim3(grid), dim3(NT), 0, s, g.a, b,
                     g.M, g.N, g.K, g.e);
  return hipGetLastError();
}

template <int KIND>
static hipError_t go_f32(const GemmArgs& g, hipStream_t s) {
  const int total = ((g.M + 63) / 64) * ((g.N + 127) / 128);
  const int grid = (total + 7) / 8 * 8;
  BRows<float> b{(const float*)g.b.b0, (const float*)g.b.b1, g.b.ldb, g.b.split, g.b.mode};
  hipLaunchKernelGGL((gemm_f32_kernel<KIND>), dim3(grid), dim3(256), 0, s, g.a, b, g.M, g.N, g.K, g.e);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.wdtype == 0) {
    switch (g.kind) {
      case EPI_STORE: return go_f32<EPI_STORE>(g, s);
      case EPI_ADD: return go_f32<EPI_ADD>(g, s);
      case EPI_SWIGLU: return go_f32<EPI_SWIGLU>(g, s);
      case EPI_LMHEAD: return go_f32<EPI_LMHEAD>(g, s);
      case EPI_KVSCATTER: return go_f32<EPI_KVSCATTER>(g, s);
    }
    return hipErrorInvalidValue;
  }
  const bool hilo = g.a.mode == ACT_HILO;
  if (hilo) {
    switch (g.kind) {
      case EPI_STORE: return go_mfma<128, 128, 64, 64, true, EPI_STORE>(g, s);
      case EPI_ADD: return go_mfma<128, 128, 64, 64, true, EPI_ADD>(g, s);
      case EPI_SWIGLU: return go_mfma<128, 128, 64, 64, true, EPI_SWIGLU>(g, s);
      case EPI_KVSCATTER: return go_mfma<128, 128, 64, 64, true, EPI_KVSCATTER>(g, s);
    }
  } else {
    switch (g.kind) {
      case EPI_STORE: return go_mfma<128, 128, 64, 64, false, EPI_STORE>(g, s);
      case EPI_LMHEAD: return go_mfma<128, 128, 64, 64, false, EPI_LMHEAD>(g, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace dflash
