// Block verification against target logits.
//
// Greedy: every row (b, i <= B) is split into vocab chunks; one workgroup per
// (chunk, row) finds the chunk's first maximum with 128-bit loads; a
// per-sequence kernel merges the chunks in order (lowest index on ties) and
// scans for the first mismatch.
//
// Sampled: the same chunking gives per-chunk (max, sum exp) of z/T for every
// target and draft row, accumulated in double; one wave per row merges its
// chunks into the row's log-sum-exp; a per-sequence workgroup runs the accept
// tests u*q(d) < p(d) in double (one thread per block position) and draws
// from the residual max(0, p - q) (or from p of the last row) by an inverse
// CDF over the whole vocabulary: contiguous per-wave segments summed in
// double, an ordered scan of the segment sums, then an in-order walk of the
// segment that holds the crossing.
#include "kernels.h"

namespace dflash {

constexpr int kVChunk = 8192;
constexpr int kMaxVerifyB = 16;   // largest block the verify call accepts
constexpr int kSeg = 128;         // vocabulary segments per sequence in the inverse CDF

int verify_chunks(int vocab) { return (vocab + kVChunk - 1) / kVChunk; }

size_t verify_ws_bytes(int batch, int B, int V) {
  const size_t rows = (size_t)batch * (2 * B + 1);
  const size_t nc = verify_chunks(V);
  // chunk (max, sum) pairs, one log-sum-exp per row, then the draw's segment masses
  return rows * nc * 16 + rows * 8 + (size_t)batch * kSeg * 8 + 256;
}

// vec4: V % 4 == 0 and a 16-byte aligned base (checked by the host), so every
// row and chunk starts on a 16-byte boundary and takes 128-bit loads.
__global__ __launch_bounds__(256) void greedy_rows_kernel(const float* z, int V, int vec4, float* pval, int* pidx) {
  const int ch = blockIdx.x, row = blockIdx.y, nc = gridDim.x;
  const int v0 = ch * kVChunk, v1 = min(V, v0 + kVChunk);
  const float* zr = z + (size_t)row * V;
  float best = -INFINITY;
  int bi = -1;
  if (vec4) {
    // the logits are read once: non-temporal loads (about 7% faster than the default policy)
    for (int v = v0 + threadIdx.x * 4; v < v1; v += 1024) {
      const f32x4 x4 = __builtin_nontemporal_load((const f32x4*)(zr + v));
      const float4 x = make_float4(x4[0], x4[1], x4[2], x4[3]);
      if (x.x > best || bi < 0) { best = x.x; bi = v; }
      if (x.y > best) { best = x.y; bi = v + 1; }
      if (x.z > best) { best = x.z; bi = v + 2; }
      if (x.w > best) { best = x.w; bi = v + 3; }
    }
  } else {
    for (int v = v0 + threadIdx.x; v < v1; v += 256) {
      const float x = zr[v];
      if (x > best || bi < 0) { best = x; bi = v; }
    }
  }
  __shared__ float sv[4];
  __shared__ int si[4];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float qv = __shfl_xor(best, o, kWave);
    const int qi = __shfl_xor(bi, o, kWave);
    if (qi >= 0 && (bi < 0 || qv > best || (qv == best && qi < bi))) { best = qv; bi = qi; }
  }
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = best; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (si[w] >= 0 && (bi < 0 || sv[w] > best || (sv[w] == best && si[w] < bi))) { best = sv[w]; bi = si[w]; }
    pval[(size_t)row * nc + ch] = best;
    pidx[(size_t)row * nc + ch] = bi;
  }
}

__global__ __launch_bounds__(64) void greedy_accept_kernel(int B, int nc, const float* pval, const int* pidx,
                                                           const int* draft, int* accept_len, int* out_tokens) {
  __shared__ int y[17];
  const int b = blockIdx.x, i = threadIdx.x;
  if (i <= B) {
    const size_t row = (size_t)b * (B + 1) + i;
    float best = -INFINITY;
    int bi = -1;
    for (int c = 0; c < nc; ++c) {
      const float v = pval[row * nc + c];
      const int ii = pidx[row * nc + c];
      if (ii >= 0 && (bi < 0 || v > best)) { best = v; bi = ii; }
    }
    y[i] = bi;
  }
  __syncthreads();
  if (i == 0) {
    int a = 0;
    while (a < B && y[a] == draft[b * B + a]) ++a;
    accept_len[b] = a;
    for (int k = 0; k <= B; ++k)
      out_tokens[b * (B + 1) + k] = k < a ? draft[b * B + k] : (k == a ? y[a] : -1);
  }
}

// e^x in double for x <= 0, table-driven (Tang's method): with n = rint(32 x / ln2),
// x = n ln2/32 + r, |r| <= ln2/64 (Cody-Waite: ln2/32 split in two, n times the
// high part exact), e^r by its Taylor series to degree 6 (truncation below 2e-17
// relative), times 2^(j/32) (j = n mod 32, from tab) and 2^floor(n/32).  Within
// about two ulps of e^x, with 15 double operations where a degree-13 series over
// |r| <= ln2/2 takes 23; terms below 2^-1020 (the log-sum-exp they join is at
// least 1) are returned as 0.
__device__ __forceinline__ double exp_nonpos_tab(double x, const double* tab) {
  constexpr double k32Log2e = 46.166241308446828384, kHi = 6.93147180369123816490e-01 / 32.0,
                   kLo = 1.90821492927058770002e-10 / 32.0;
  const double t = x * k32Log2e;
  const double n = rint(fmax(t, -32.0 * 1021.0));
  const double r = fma(-n, kLo, fma(-n, kHi, x));
  double p = 1.0 / 720.0;
  p = fma(p, r, 1.0 / 120.0);
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const int ni = (int)n;
  const double e = ldexp(tab[ni & 31] * p, ni >> 5);
  return t < -32.0 * 1020.0 ? 0.0 : e;
}

// (max, sum exp(x - max)) of x = z/T over one chunk, in double.  The chunk is
// read once into registers (128-bit loads when rows are 16-byte aligned).  The
// maximum is taken over z (dividing by T > 0 keeps the order) and divided once;
// the exponents use z * (1/T), within an ulp of z/T.
constexpr int kLsePer = kVChunk / 256;   // elements per thread
__global__ __launch_bounds__(256) void lse_rows_kernel(const float* zt, const float* zd, int nt_rows, int V,
                                                       double Td, int vec4, double2* part) {
  const int ch = blockIdx.x, row = blockIdx.y, nc = gridDim.x, tid = threadIdx.x;
  const float* zr = row < nt_rows ? zt + (size_t)row * V : zd + (size_t)(row - nt_rows) * V;
  const int v0 = ch * kVChunk, v1 = min(V, v0 + kVChunk);
  float x[kLsePer];
  if (vec4) {
    // element v0 + 4 (tid + 256 k) + e; V % 4 == 0 and 16-byte aligned bases (checked
    // by the host), so every row and chunk starts on a 16-byte boundary
#pragma unroll
    for (int k = 0; k < kLsePer / 4; ++k) {
      const int v = v0 + 4 * (tid + 256 * k);
      const float4 q = v < v1 ? *(const float4*)(zr + v) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      x[4 * k] = q.x;
      x[4 * k + 1] = q.y;
      x[4 * k + 2] = q.z;
      x[4 * k + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kLsePer; ++k) {
      const int v = v0 + tid + 256 * k;
      x[k] = v < v1 ? zr[v] : -INFINITY;
    }
  }
  float mf = -INFINITY;
#pragma unroll
  for (int k = 0; k < kLsePer; ++k) mf = fmaxf(mf, x[k]);
  __shared__ float red[4];
  __shared__ double dred[4];
  __shared__ double tab[32];   // 2^(j/32)
  if (tid < 32) tab[tid] = exp2((double)tid / 32.0);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mf = fmaxf(mf, __shfl_xor(mf, o, kWave));
  if ((tid & 63) == 0) red[tid >> 6] = mf;
  __syncthreads();
  const double mx = (double)fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) / Td;
  const double invT = 1.0 / Td;
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < kLsePer; ++k)
    if (x[k] != -INFINITY) s += exp_nonpos_tab(fmin((double)x[k] * invT - mx, 0.0), tab);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
  if ((tid & 63) == 0) dred[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) part[(size_t)row * nc + ch] = make_double2(mx, dred[0] + dred[1] + dred[2] + dred[3]);
}

// log-sum-exp of each row from its chunk pairs: one wave per row, lanes over chunks.
__global__ __launch_bounds__(256) void lse_merge_kernel(const double2* part, int rows, int nc, double* lse) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  double mx = -INFINITY;
  for (int c = lane; c < nc; c += 64) mx = fmax(mx, part[(size_t)row * nc + c].x);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, kWave));
  double s = 0.0;
  for (int c = lane; c < nc; c += 64) {
    const double2 q = part[(size_t)row * nc + c];
    if (q.y > 0.0) s += q.y * exp(q.x - mx);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
  if (lane == 0) lse[row] = mx + log(s);
}

// The accept tests of sequence b, thread i < B testing block position i (the
// first rejection decides).  Leaves in shared memory the accepted length a, the
// log-sum-exp of the target row a (and of draft row a if a < B), and the
// sampling uniform of row a.  Every thread of the block must call it.
struct AcceptState {
  double lt[kMaxVerifyB + 1], ld[kMaxVerifyB];
  int rej[kMaxVerifyB];
  int a;
  double lset, lsed, u;
};

__device__ void accept_tests(AcceptState& st, int b, int nseq, int B, int V, const float* zt, const float* zd,
                             const int* draft, const float* U, double Td, const double* lse) {
  const int tid = threadIdx.x, nt_rows = nseq * (B + 1);
  if (tid < B) {
    const size_t trow = (size_t)b * (B + 1) + tid, drow = (size_t)b * B + tid;
    const double lt = lse[trow], ld = lse[nt_rows + drow];
    int d = draft[drow];
    d = d < 0 ? 0 : (d >= V ? V - 1 : d);
    const double p = exp((double)zt[trow * V + d] / Td - lt);
    const double q = exp((double)zd[drow * V + d] / Td - ld);
    st.lt[tid] = lt;
    st.ld[tid] = ld;
    st.rej[tid] = !((double)U[trow * 2] * q < p);
  } else if (tid == B) {
    st.lt[B] = lse[(size_t)b * (B + 1) + B];
  }
  __syncthreads();
  if (tid == 0) {
    int a = B;
    for (int i = 0; i < B; ++i)
      if (st.rej[i]) { a = i; break; }
    st.a = a;
    st.lset = st.lt[a];
    st.lsed = a < B ? st.ld[a] : 0.0;
    st.u = (double)U[((size_t)b * (B + 1) + a) * 2 + 1];
  }
  __syncthreads();
}

// Mass w(v) of the distribution drawn from at row a: the residual max(0, p - q)
// after a rejection, else p of the bonus row.
struct DrawRow {
  const float *zr, *zq;
  double lt, ld, invT;
  __device__ double operator()(int v) const {
    const double p = exp((double)zr[v] * invT - lt);
    if (!zq) return p;
    const double q = exp((double)zq[v] * invT - ld);
    return p > q ? p - q : 0.0;
  }
};

__device__ DrawRow draw_row(const AcceptState& st, int b, int B, int V, const float* zt, const float* zd, double Td) {
  const int a = st.a;
  DrawRow r;
  r.zr = zt + ((size_t)b * (B + 1) + a) * V;
  r.zq = a < B ? zd + ((size_t)b * B + a) * V : nullptr;
  r.lt = st.lset;
  r.ld = st.lsed;
  r.invT = 1.0 / Td;
  return r;
}

__device__ __forceinline__ int seg_len(int V) { return ((V + kSeg - 1) / kSeg + 63) / 64 * 64; }

// Mass of each vocabulary segment of the drawn row: grid (kSeg, batch).
__global__ __launch_bounds__(256) void draw_segments_kernel(int B, int V, const float* zt, const float* zd,
                                                            const int* draft, const float* U, double Td,
                                                            const double* lse, double* segsum) {
  __shared__ AcceptState st;
  __shared__ double red[4];
  const int sg = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  accept_tests(st, b, gridDim.y, B, V, zt, zd, draft, U, Td, lse);
  const DrawRow w = draw_row(st, b, B, V, zt, zd, Td);
  const int len = seg_len(V), s0 = sg * len, s1 = min(V, s0 + len);
  double sum = 0.0;
  for (int v = s0 + tid; v < s1; v += 256) sum += w(v);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  __syncthreads();
  if (tid == 0) segsum[(size_t)b * kSeg + sg] = red[0] + red[1] + red[2] + red[3];
}

// Accept length, then the draw by inverse CDF: the segment sums are scanned in
// order, and the segment holding the crossing is walked 64 elements at a time
// with an in-order wave scan.  One wave per sequence.
__global__ __launch_bounds__(64) void draw_select_kernel(int B, int V, const float* zt, const float* zd,
                                                         const int* draft, const float* U, double Td,
                                                         const double* lse, const double* segsum, int* accept_len,
                                                         int* out_tokens) {
  __shared__ AcceptState st;
  __shared__ double s_target, s_pre;
  __shared__ int s_owner;
  const int b = blockIdx.x, lane = threadIdx.x;
  accept_tests(st, b, gridDim.x, B, V, zt, zd, draft, U, Td, lse);
  const DrawRow w = draw_row(st, b, B, V, zt, zd, Td);
  __shared__ double run[kSeg];   // this sequence's segment masses, staged for the serial scan
  for (int t = lane; t < kSeg; t += 64) run[t] = segsum[(size_t)b * kSeg + t];
  __syncthreads();
  if (lane == 0) {
    double tot = 0.0;
    for (int t = 0; t < kSeg; ++t) tot += run[t];
    const double target = st.u * tot;
    double pre = 0.0;
    int owner = -1;
    for (int t = 0; t < kSeg; ++t) {
      const double nx = pre + run[t];
      if (run[t] > 0.0 && nx > target) { owner = t; break; }
      pre = nx;
    }
    if (owner < 0) {  // rounding pushed the target past the total: last segment with mass
      for (int t = kSeg - 1; t >= 0; --t)
        if (run[t] > 0.0) { owner = t; break; }
      owner = owner < 0 ? 0 : owner;
      pre = 0.0;
      for (int t = 0; t < owner; ++t) pre += run[t];
      s_target = pre + run[owner] * 0.999999;
    } else {
      s_target = target;
    }
    s_pre = pre;
    s_owner = owner;
  }
  __syncthreads();
  const int len = seg_len(V), s0 = s_owner * len, s1 = min(V, s0 + len);
  const double target = s_target;
  double acc = s_pre;
  int k = -1, last = -1;
  for (int base = s0; base < s1 && k < 0; base += 64) {
    const int v = base + lane;
    const double x0 = v < s1 ? w(v) : 0.0;
    double x = x0;   // inclusive scan over the lanes, in vocabulary order
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double y = __shfl_up(x, o, kWave);
      if (lane >= o) x += y;
    }
    const double c = acc + x;
    const unsigned long long hit = __ballot(x0 > 0.0 && c > target);
    const unsigned long long pos = __ballot(x0 > 0.0);
    if (hit) k = base + __builtin_ctzll(hit);
    else if (pos) last = base + 63 - __builtin_clzll(pos);
    acc = __shfl(c, 63, kWave);
  }
  if (k < 0) k = last >= 0 ? last : max(s0, s1 - 1);   // no crossing: the last element with mass
  if (lane == 0) {
    const int a = st.a;
    accept_len[b] = a;
    for (int kk = 0; kk <= B; ++kk)
      out_tokens[b * (B + 1) + kk] = kk < a ? draft[b * B + kk] : (kk == a ? k : -1);
  }
}

hipError_t launch_verify_greedy(int batch, int B, int V, const float* zt, const int* draft, int* accept_len,
                                int* out_tokens, void* ws, hipStream_t s) {
  const int nc = verify_chunks(V);
  const int rows = batch * (B + 1);
  float* pval = (float*)ws;
  int* pidx = (int*)(pval + (size_t)rows * nc);
  const int vec4 = (V % 4 == 0) && ((uintptr_t)zt % 16 == 0);
  hipLaunchKernelGGL(greedy_rows_kernel, dim3(nc, rows), dim3(256), 0, s, zt, V, vec4, pval, pidx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(greedy_accept_kernel, dim3(batch), dim3(64), 0, s, B, nc, pval, pidx, draft, accept_len,
                     out_tokens);
  return hipGetLastError();
}

hipError_t launch_verify_sampled(int batch, int B, int V, const float* zt, const float* zd, const int* draft,
                                 const float* uniforms, float T, int* accept_len, int* out_tokens, void* ws,
                                 hipStream_t s) {
  const int nc = verify_chunks(V);
  const int nt_rows = batch * (B + 1), nd_rows = batch * B;
  double2* part = (double2*)ws;
  const double Td = (double)T;
  const int vec4 = (V % 4 == 0) && ((uintptr_t)zt % 16 == 0) && ((uintptr_t)zd % 16 == 0);
  hipLaunchKernelGGL(lse_rows_kernel, dim3(nc, nt_rows + nd_rows), dim3(256), 0, s, zt, zd, nt_rows, V, Td, vec4,
                     part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  double* lse = (double*)(part + (size_t)(nt_rows + nd_rows) * nc);
  const int rows = nt_rows + nd_rows;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, part, rows, nc, lse);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  double* segsum = lse + rows;
  hipLaunchKernelGGL(draw_segments_kernel, dim3(kSeg, batch), dim3(256), 0, s, B, V, zt, zd, draft, uniforms, Td, lse,
                     segsum);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(draw_select_kernel, dim3(batch), dim3(64), 0, s, B, V, zt, zd, draft, uniforms, Td, lse, segsum,
                     accept_len, out_tokens);
  return hipGetLastError();
}

}  // namespace dflash
