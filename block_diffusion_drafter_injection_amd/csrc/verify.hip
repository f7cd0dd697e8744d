// Block verification against target logits.
//
// Greedy: every row (b, i <= B) is split into vocab chunks; one workgroup per
// (chunk, row) finds the chunk's first maximum with 128-bit loads; a
// per-sequence kernel merges the chunks in order (lowest index on ties) and
// scans for the first mismatch.
//
// Sampled: the same chunking gives per-chunk (max, sum exp) of z/T for every
// target and draft row, accumulated in double; a per-sequence workgroup
// forms log-sum-exp in double, runs the accept tests u*q(d) < p(d) in double,
// and draws from the residual max(0, p - q) (or from p of the last row) by an
// inverse CDF over the whole vocabulary: contiguous per-thread runs summed in
// double, an ordered scan of the run sums, then a re-walk of the run that
// holds the crossing.
#include "kernels.h"

namespace dflash {

constexpr int kVChunk = 8192;

int verify_chunks(int vocab) { return (vocab + kVChunk - 1) / kVChunk; }

size_t verify_ws_bytes(int batch, int B, int V) {
  const size_t rows = (size_t)batch * (2 * B + 1);
  const size_t nc = verify_chunks(V);
  return rows * nc * 16 + 256;
}

__global__ __launch_bounds__(256) void greedy_rows_kernel(const float* z, int V, float* pval, int* pidx) {
  const int ch = blockIdx.x, row = blockIdx.y, nc = gridDim.x;
  const int v0 = ch * kVChunk, v1 = min(V, v0 + kVChunk);
  const float* zr = z + (size_t)row * V;
  float best = -INFINITY;
  int bi = -1;
  const bool vec = (V & 3) == 0;
  if (vec) {
    for (int v = v0 + threadIdx.x * 4; v < v1; v += 1024) {
      const float4 x = *(const float4*)(zr + v);
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

// (max, sum exp(x - max)) of x = z/T over one chunk, in double.
__global__ __launch_bounds__(256) void lse_rows_kernel(const float* zt, const float* zd, int nt_rows, int V,
                                                       double Td, double2* part) {
  const int ch = blockIdx.x, row = blockIdx.y, nc = gridDim.x;
  const float* zr = row < nt_rows ? zt + (size_t)row * V : zd + (size_t)(row - nt_rows) * V;
  const int v0 = ch * kVChunk, v1 = min(V, v0 + kVChunk);
  double mx = -INFINITY;
  for (int v = v0 + threadIdx.x; v < v1; v += 256) mx = fmax(mx, (double)zr[v] / Td);
  __shared__ double red[4];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, kWave));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  __syncthreads();
  double s = 0.0;
  for (int v = v0 + threadIdx.x; v < v1; v += 256) s += exp((double)zr[v] / Td - mx);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) part[(size_t)row * nc + ch] = make_double2(mx, red[0] + red[1] + red[2] + red[3]);
}

__device__ double lse_of(const double2* part, size_t row, int nc) {
  double mx = -INFINITY;
  for (int c = 0; c < nc; ++c) mx = fmax(mx, part[row * nc + c].x);
  double s = 0.0;
  for (int c = 0; c < nc; ++c) {
    const double2 q = part[row * nc + c];
    if (q.y > 0.0) s += q.y * exp(q.x - mx);
  }
  return mx + log(s);
}

__global__ __launch_bounds__(256) void sampled_accept_kernel(int B, int V, int nc, const float* zt, const float* zd,
                                                             const int* draft, const float* U, double Td,
                                                             const double2* part, int* accept_len,
                                                             int* out_tokens) {
  const int b = blockIdx.x, tid = threadIdx.x;
  __shared__ int s_row, s_resid;
  __shared__ double s_lset, s_lsed, s_u;
  __shared__ double run[256];
  if (tid == 0) {
    const int nt_rows = gridDim.x * (B + 1);
    int a = B;
    for (int i = 0; i < B; ++i) {
      const size_t trow = (size_t)b * (B + 1) + i, drow = (size_t)b * B + i;
      const double lt = lse_of(part, trow, nc), ld = lse_of(part, nt_rows + drow, nc);
      int d = draft[drow];
      d = d < 0 ? 0 : (d >= V ? V - 1 : d);
      const double p = exp((double)zt[trow * V + d] / Td - lt);
      const double q = exp((double)zd[drow * V + d] / Td - ld);
      if ((double)U[trow * 2] * q < p) continue;
      a = i;
      s_lset = lt;
      s_lsed = ld;
      break;
    }
    s_row = a;
    s_resid = a < B;
    if (a == B) s_lset = lse_of(part, (size_t)b * (B + 1) + B, nc);
    s_u = (double)U[((size_t)b * (B + 1) + a) * 2 + 1];
    accept_len[b] = a;
  }
  __syncthreads();
  const int a = s_row;
  const bool resid = s_resid;
  const size_t trow = (size_t)b * (B + 1) + a;
  const float* zr = zt + trow * V;
  const float* zq = resid ? zd + ((size_t)b * B + a) * V : nullptr;
  const double lt = s_lset, ld = s_lsed;
  auto wv = [&](int v) -> double {
    const double p = exp((double)zr[v] / Td - lt);
    if (!resid) return p;
    const double q = exp((double)zq[v] / Td - ld);
    return p > q ? p - q : 0.0;
  };
  const int per = (V + 255) / 256;
  const int v0 = tid * per, v1 = min(V, v0 + per);
  double sum = 0.0;
  for (int v = v0; v < v1; ++v) sum += wv(v);
  run[tid] = sum;
  __syncthreads();
  __shared__ double s_target;
  __shared__ int s_thread;
  if (tid == 0) {
    double tot = 0.0;
    for (int t = 0; t < 256; ++t) tot += run[t];
    const double target = s_u * tot;
    double pre = 0.0;
    int owner = -1;
    for (int t = 0; t < 256; ++t) {
      const double nx = pre + run[t];
      if (run[t] > 0.0 && nx > target) { owner = t; break; }
      pre = nx;
    }
    if (owner < 0) {  // rounding pushed the target past the total: last run with mass
      for (int t = 255; t >= 0; --t)
        if (run[t] > 0.0) { owner = t; break; }
      pre = 0.0;
      for (int t = 0; t < owner; ++t) pre += run[t];
      s_target = pre + run[owner] * 0.999999;
    } else {
      s_target = target;
    }
    run[0] = pre;  // prefix before the owner's run (slot reused)
    s_thread = owner;
  }
  __syncthreads();
  if (tid == s_thread) {
    double acc = run[0];
    int k = v1 - 1, last = -1;
    for (int v = v0; v < v1; ++v) {
      const double w = wv(v);
      if (w > 0.0) last = v;
      acc += w;
      if (w > 0.0 && acc > s_target) { k = v; last = -2; break; }
    }
    if (last >= 0) k = last;
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
  hipLaunchKernelGGL(greedy_rows_kernel, dim3(nc, rows), dim3(256), 0, s, zt, V, pval, pidx);
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
  hipLaunchKernelGGL(lse_rows_kernel, dim3(nc, nt_rows + nd_rows), dim3(256), 0, s, zt, zd, nt_rows, V, Td,
                     part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sampled_accept_kernel, dim3(batch), dim3(256), 0, s, B, V, nc, zt, zd, draft, uniforms, Td,
                     part, accept_len, out_tokens);
  return hipGetLastError();
}

}  // namespace dflash
