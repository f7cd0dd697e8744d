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
// (two 8-byte LDS reads per fragment, no transpose).  P is split hi/lo too.
// fp32 pool and the in-block split: a VALU kernel, four lanes per query row.
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

// ---------------------------------------------------------------------------
constexpr int kMaxPPS = 512;   // pages per context split (bounded by the host)

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_ctx_mfma_kernel(AttnParams p) {
  constexpr int NT = NW * 64;
  constexpr int KK = D / 32;         // 32-wide k-steps of QK^T
  constexpr int NN = D / 16;         // 16-row tiles of O^T
  constexpr int LDK = D + 8, LDV = 32 + 8;
  constexpr int KPC = 32 * D / 8;    // 16-byte pieces of a 32-token K tile
  constexpr int VPC = 4 * D;         // 16-byte pieces of the two V pages
  constexpr int KP = (KPC + NT - 1) / NT, VP = (VPC + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[32 * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[D * LDV];
  __shared__ int ptab[kMaxPPS];

  const int g = p.nq / p.nkv, R = g * p.B;
  const int nqg = (R + 63) / 64;
  const int split = blockIdx.x / nqg, qg = blockIdx.x - split * nqg;
  const int m = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int ctx = clamp_ctx(p, b);
  const int npages = (ctx + 15) >> 4;
  const int pg0 = split * p.pps, pg1 = min(pg0 + p.pps, npages);

  for (int i = tid; i < pg1 - pg0; i += NT) ptab[i] = phys_page(p, b, pg0 + i);

  const int r = qg * 64 + wid * 16 + (lane & 15);
  const bool rvalid = r < R;
  const int j = rvalid ? r / p.B : 0, i = rvalid ? r - (r / p.B) * p.B : 0;
  const int n = m * g + j, row = b * p.B + i;
  const int ldq = (p.nq + 2 * p.nkv) * D;

  bf16x8 qh[KK], ql[KK];
  {
    const float* qv = p.qkv + (size_t)row * ldq + n * D;
    const float2* cs = p.cs + (size_t)row * (D / 2);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16_t hv[8], lv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dd = 32 * kk + 8 * (lane >> 4) + e;
        const float x = rvalid ? rope_elem(qv, cs, dd, D) : 0.f;
        split_hilo(x, hv[e], lv[e]);
      }
      u32x4 hu, lu;
      hu.x = hv[0] | ((uint32_t)hv[1] << 16); hu.y = hv[2] | ((uint32_t)hv[3] << 16);
      hu.z = hv[4] | ((uint32_t)hv[5] << 16); hu.w = hv[6] | ((uint32_t)hv[7] << 16);
      lu.x = lv[0] | ((uint32_t)lv[1] << 16); lu.y = lv[2] | ((uint32_t)lv[3] << 16);
      lu.z = lv[4] | ((uint32_t)lv[5] << 16); lu.w = lv[6] | ((uint32_t)lv[7] << 16);
      qh[kk] = as_bf16x8(hu);
      ql[kk] = as_bf16x8(lu);
    }
  }
  __syncthreads();   // ptab ready

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 ot[NN];
#pragma unroll
  for (int nn = 0; nn < NN; ++nn) ot[nn] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t chunk = 16 * D;
  const size_t kv_stride = (size_t)p.nkv * chunk;                   // K region -> V region of one layer
  const size_t page_stride = (size_t)p.n_layers * 2 * kv_stride;
  const bf16_t* base = (const bf16_t*)p.pool + (size_t)p.layer * 2 * kv_stride + (size_t)m * chunk;
  u32x4 rk[KP], rv[VP];
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  // Global -> registers for the 32-token tile starting at page pg (two pages).
#define DFLASH_ATT_LOAD(pg)                                                                    \
  do {                                                                                         \
    _Pragma("unroll") for (int q = 0; q < KP; ++q) {                                           \
      const int c = tid + q * NT;                                                              \
      const int tok = c / (D / 8), part = c - tok * (D / 8);                                   \
      const int pp = (pg) + (tok >> 4), slot = tok & 15;                                       \
      u32x4 v = z4;                                                                            \
      if (c < KPC && pp < pg1 && pp * 16 + slot < ctx) {                                       \
        const int ph = ptab[pp - pg0];                                                         \
        if (ph >= 0) v = *(const u32x4*)(base + (size_t)ph * page_stride + slot * D + part * 8); \
      }                                                                                        \
      rk[q] = v;                                                                               \
    }                                                                                          \
    _Pragma("unroll") for (int q = 0; q < VP; ++q) {                                           \
      const int c = tid + q * NT;                                                              \
      const int t = c / (2 * D), rem = c - t * 2 * D, dd = rem >> 1, half = rem & 1;           \
      const int pp = (pg) + t;                                                                 \
      u32x4 v = z4;                                                                            \
      if (c < VPC && pp < pg1) {                                                               \
        const int ph = ptab[pp - pg0];                                                         \
        if (ph >= 0) {                                                                         \
          v = *(const u32x4*)(base + kv_stride + (size_t)ph * page_stride + dd * 16 + half * 8); \
          const int valid = ctx - (pp * 16 + half * 8);                                        \
          if (valid < 8) {                                                                     \
            _Pragma("unroll") for (int e = 0; e < 8; ++e)                                      \
              if (e >= valid) v[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;                \
          }                                                                                    \
        }                                                                                      \
      }                                                                                        \
      rv[q] = v;                                                                               \
    }                                                                                          \
  } while (0)

  if (pg0 < pg1) DFLASH_ATT_LOAD(pg0);
  for (int pg = pg0; pg < pg1; pg += 2) {
    __syncthreads();   // the previous tile has been consumed
#pragma unroll
    for (int q = 0; q < KP; ++q) {
      const int c = tid + q * NT;
      if (c < KPC) {
        const int tok = c / (D / 8), part = c - tok * (D / 8);
        *(u32x4*)(Ks + tok * LDK + part * 8) = rk[q];
      }
    }
#pragma unroll
    for (int q = 0; q < VP; ++q) {
      const int c = tid + q * NT;
      if (c < VPC) {
        const int t = c / (2 * D), rem = c - t * 2 * D, dd = rem >> 1, half = rem & 1;
        *(u32x4*)(Vt + dd * LDV + t * 16 + half * 8) = rv[q];
      }
    }
    __syncthreads();
    if (pg + 2 < pg1) DFLASH_ATT_LOAD(pg + 2);   // next tile in flight during this one

    f32x4 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 a = as_bf16x8(*(const u32x4*)(Ks + (16 * t + (lane & 15)) * LDK + 32 * kk + 8 * (lane >> 4)));
        st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[kk], st[t], 0, 0, 0);
        st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[kk], st[t], 0, 0, 0);
      }
    }
    // lane owns query (lane & 15) and tokens 16t + 4(lane>>4) + e
    float s[8];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = pg * 16 + 16 * t + 4 * (lane >> 4) + e;
        const float v = (tok < pg1 * 16 && tok < ctx) ? st[t][e] * p.scale : -INFINITY;
        s[t * 4 + e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    if (m_new == -INFINITY) continue;
    const float alpha = expf(m_run - m_new);
    float ps = 0.f;
    bf16_t ph[8], pl[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float pv = expf(s[k] - m_new);
      ps += pv;
      split_hilo(pv, ph[k], pl[k]);
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
    u32x4 hu, lu;
    hu.x = ph[0] | ((uint32_t)ph[1] << 16); hu.y = ph[2] | ((uint32_t)ph[3] << 16);
    hu.z = ph[4] | ((uint32_t)ph[5] << 16); hu.w = ph[6] | ((uint32_t)ph[7] << 16);
    lu.x = pl[0] | ((uint32_t)pl[1] << 16); lu.y = pl[2] | ((uint32_t)pl[3] << 16);
    lu.z = pl[4] | ((uint32_t)pl[5] << 16); lu.w = pl[6] | ((uint32_t)pl[7] << 16);
    const bf16x8 pbh = as_bf16x8(hu), pbl = as_bf16x8(lu);
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      ot[nn] *= alpha;
      const bf16_t* vr = Vt + (16 * nn + (lane & 15)) * LDV + 4 * (lane >> 4);
      const u32x2 lo2 = *(const u32x2*)vr, hi2 = *(const u32x2*)(vr + 16);
      const u32x4 vv = {lo2.x, lo2.y, hi2.x, hi2.y};
      const bf16x8 va = as_bf16x8(vv);
      ot[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pbh, ot[nn], 0, 0, 0);
      ot[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pbl, ot[nn], 0, 0, 0);
    }
  }
#undef DFLASH_ATT_LOAD

  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);
  if (!rvalid) return;
  const size_t Mq = (size_t)p.batch * p.B * p.nq;
  const size_t qrow = (size_t)row * p.nq + n;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if ((lane >> 4) == 0) p.part_lse[split * Mq + qrow] = l_tot > 0.f ? m_run + logf(l_tot) : -INFINITY;
  float* dst = p.part_o + (split * Mq + qrow) * D;
#pragma unroll
  for (int nn = 0; nn < NN; ++nn) {
    const int d0 = 16 * nn + 4 * (lane >> 4);
    *(float4*)(dst + d0) = make_float4(ot[nn][0] * inv, ot[nn][1] * inv, ot[nn][2] * inv, ot[nn][3] * inv);
  }
}

// ---------------------------------------------------------------------------
// VALU attention: 64 query rows per workgroup, 4 lanes per row (D/4 dims each).
// CTX: keys of context split blockIdx.x / nqg from the paged pool of type TP.
// !CTX: the B in-block keys (fp32, rotated here), written as split n_splits.
template <typename TP, int D, bool CTX>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnParams p) {
  constexpr int DQ = D / 4;
  const int g = p.nq / p.nkv, R = g * p.B;
  const int nqg = (R + 63) / 64;
  const int split = CTX ? blockIdx.x / nqg : p.n_splits;
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
#pragma unroll
    for (int e = 0; e < DQ; ++e) {
      q[e] = rvalid ? rope_elem(qv, cs, q4 * DQ + e, D) : 0.f;
      o[e] = 0.f;
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  auto consume = [&](float sdot, const float* vvals) {  // vvals may point to LDS
    // vvals: this lane's DQ value entries
    const float sc = sdot * p.scale;
    const float m_new = fmaxf(m_run, sc);
    const float alpha = expf(m_run - m_new), pw = expf(sc - m_new);
    l_run = l_run * alpha + pw;
#pragma unroll
    for (int e = 0; e < DQ; ++e) o[e] = o[e] * alpha + pw * vvals[e];
    m_run = m_new;
  };

  if constexpr (CTX) {
    const int ctx = clamp_ctx(p, b);
    const int npages = (ctx + 15) >> 4;
    const int pg0 = split * p.pps, pg1 = min(pg0 + p.pps, npages);
    const TP* pool = (const TP*)p.pool;
    const size_t chunk = 16 * D;
    for (int pg = pg0; pg < pg1; ++pg) {
      const int ph = phys_page(p, b, pg);
      if (ph < 0) continue;
      const TP* Kc = pool + (((size_t)ph * p.n_layers + p.layer) * 2 * p.nkv + m) * chunk;
      const TP* Vc = pool + ((((size_t)ph * p.n_layers + p.layer) * 2 + 1) * p.nkv + m) * chunk;
      const int ns = min(16, ctx - pg * 16);
      for (int slot = 0; slot < ns; ++slot) {
        float sd = 0.f;
#pragma unroll
        for (int e = 0; e < DQ; ++e) sd += q[e] * ld_f(Kc, (size_t)slot * D + q4 * DQ + e);
        sd += __shfl_xor(sd, 1, kWave);
        sd += __shfl_xor(sd, 2, kWave);
        float vv[DQ];
#pragma unroll
        for (int e = 0; e < DQ; ++e) vv[e] = ld_f(Vc, (size_t)(q4 * DQ + e) * 16 + slot);
        consume(sd, vv);
      }
    }
  } else {
    // the B block keys (rotated) and values of kv head m, staged once
    __shared__ float kb[16 * D], vb[16 * D];
    for (int c = tid; c < p.B * D; c += 256) {
      const int jb = c / D, e = c - jb * D;
      const int krow = b * p.B + jb;
      const float* kv = p.qkv + (size_t)krow * ldq + p.nq * D + m * D;
      kb[c] = rope_elem(kv, p.cs + (size_t)krow * (D / 2), e, D);
      vb[c] = p.qkv[(size_t)krow * ldq + (p.nq + p.nkv) * D + m * D + e];
    }
    __syncthreads();
    for (int jb = 0; jb < p.B; ++jb) {
      float sd = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) sd += q[e] * kb[jb * D + q4 * DQ + e];
      sd += __shfl_xor(sd, 1, kWave);
      sd += __shfl_xor(sd, 2, kWave);
      consume(sd, vb + jb * D + q4 * DQ);
    }
  }
  if (!rvalid) return;
  const size_t Mq = (size_t)p.batch * p.B * p.nq;
  const size_t qrow = (size_t)row * p.nq + n;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  if (q4 == 0) p.part_lse[split * Mq + qrow] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
  float* dst = p.part_o + (split * Mq + qrow) * D + q4 * DQ;
#pragma unroll
  for (int e = 0; e < DQ; ++e) dst[e] = o[e] * inv;
}

// ---------------------------------------------------------------------------
// Merge the n_splits + 1 partials of every query row in split order.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p, ActOut out) {
  const size_t Mq = (size_t)p.batch * p.B * p.nq;
  const int per = 256 / (D / 4);
  const size_t qrow = (size_t)blockIdx.x * per + threadIdx.x / (D / 4);
  const int e4 = (threadIdx.x % (D / 4)) * 4;
  if (qrow >= Mq) return;
  const int S = p.n_splits + 1;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, p.part_lse[s * Mq + qrow]);
  float tot = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < S; ++s) {
    const float l = p.part_lse[s * Mq + qrow];
    if (l == -INFINITY) continue;
    const float w = expf(l - mx);
    tot += w;
    const float4 v = *(const float4*)(p.part_o + (s * Mq + qrow) * D + e4);
    acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  acc.x *= inv; acc.y *= inv; acc.z *= inv; acc.w *= inv;
  const int rowm = (int)(qrow / p.nq), n = (int)(qrow % p.nq);
  act_store4(out, rowm, n * D + e4, acc);
}

// ---------------------------------------------------------------------------
hipError_t launch_attention(const AttnParams& p, int wdtype, hipStream_t s, void (*mark)(int, hipStream_t)) {
  const int g = p.nq / p.nkv, R = g * p.B, nqg = (R + 63) / 64;
  const dim3 gctx(p.n_splits * nqg, p.nkv, p.batch), gblk(nqg, p.nkv, p.batch);
  if (p.n_splits > 0) {
  if (mark) mark(0, s);
  if (wdtype == 1) {
    const int waves = min(4, (R + 15) / 16);
#define DFLASH_ATT_GO(DD, NWV) hipLaunchKernelGGL((attn_ctx_mfma_kernel<DD, NWV>), gctx, dim3(64 * NWV), 0, s, p)
    if (p.d == 128) {
      if (waves == 4) DFLASH_ATT_GO(128, 4); else if (waves == 3) DFLASH_ATT_GO(128, 3);
      else if (waves == 2) DFLASH_ATT_GO(128, 2); else DFLASH_ATT_GO(128, 1);
    } else {
      if (waves == 4) DFLASH_ATT_GO(64, 4); else if (waves == 3) DFLASH_ATT_GO(64, 3);
      else if (waves == 2) DFLASH_ATT_GO(64, 2); else DFLASH_ATT_GO(64, 1);
    }
#undef DFLASH_ATT_GO
  } else {
    if (p.d == 128)
      hipLaunchKernelGGL((attn_valu_kernel<float, 128, true>), gctx, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((attn_valu_kernel<float, 64, true>), gctx, dim3(256), 0, s, p);
  }
  if (mark) mark(1, s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  }
  if (p.d == 128)
    hipLaunchKernelGGL((attn_valu_kernel<float, 128, false>), gblk, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((attn_valu_kernel<float, 64, false>), gblk, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnParams& p, ActOut out, hipStream_t s) {
  const size_t Mq = (size_t)p.batch * p.B * p.nq;
  const int per = 256 / (p.d / 4);
  const int grid = (int)((Mq + per - 1) / per);
  if (p.d == 128)
    hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(grid), dim3(256), 0, s, p, out);
  else
    hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(grid), dim3(256), 0, s, p, out);
  return hipGetLastError();
}

}  // namespace dflash
