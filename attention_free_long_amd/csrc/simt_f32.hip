// fp32 path: plain SIMT kernels with fp32 arithmetic for all three steps.
//
// These serve fp32 inputs (the 1000-token, d = 64 parity workload); they favour a direct
// reading of the definitions over speed. Same definitions as the bf16 kernels: MaxSim over
// valid tokens (paperlayer.ai "Avey-B" summary, section 3), X^ = P X_cat + X_i
// (papernotes.org Avey-B note, 关键设计 4, eq. 8), S~ Z_t with eq. 6 (关键设计 2 and 3).
#include "avey_common.h"
#include "launch.h"

namespace avey {

namespace {

__device__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

__device__ float norm_f32(const float* __restrict__ v, int n) {
  float s = 0.f;
  for (int c = 0; c < n; ++c) s = fmaf(v[c], v[c], s);
  return sqrtf(s);
}

// One workgroup per ordered pair (b, i, j), over the normalised rows N(x) written by the
// preparation pass ([B][n_s * S][d], padding rows zero): the cosine is a plain dot product.
__global__ void __launch_bounds__(256) maxsim_f32_kernel(const float* __restrict__ xn, int64_t N, int d, int S,
                                                          int n_s, float* __restrict__ scores) {
  __shared__ float red[4];
  const int64_t pr = blockIdx.x;
  const int j = (int)(pr % n_s);
  const int i = (int)((pr / n_s) % n_s);
  const int64_t b = pr / ((int64_t)n_s * n_s);
  float* out = scores + pr;
  if (i == j) {
    if (threadIdx.x == 0) *out = -INFINITY;
    return;
  }
  const float* xb = xn + b * (int64_t)n_s * S * d;
  const int64_t ti0 = (int64_t)i * S, tj0 = (int64_t)j * S;
  const int ni = (int)min((int64_t)S, N - ti0), nj = (int)min((int64_t)S, N - tj0);
  float part = 0.f;
  for (int t = threadIdx.x; t < ni; t += 256) {
    const float* xt = xb + (ti0 + t) * d;
    float best = -INFINITY;
    for (int u = 0; u < nj; ++u) {
      const float* xu = xb + (tj0 + u) * d;
      float dot = 0.f;
      for (int c = 0; c < d; ++c) dot = fmaf(xt[c], xu[c], dot);
      best = fmaxf(best, dot);
    }
    part += best;
  }
  const float tot = block_sum(part, red);
  if (threadIdx.x == 0) *out = tot;
}

// One workgroup per ordered pair (b, i, j), straight from X (row stride ld): the inverse norms of
// the candidate split's valid tokens go to LDS first, then each thread takes target tokens t and
// sums rn_t max_u (x_t . x_u) rn_u, the largest cosine over the candidate's valid tokens.
__global__ void __launch_bounds__(256) maxsim_rows_f32_kernel(const float* __restrict__ x, int64_t N, int d,
                                                               int64_t ld, int S, int n_s,
                                                               float* __restrict__ scores) {
  __shared__ float rnj[512];
  __shared__ float red[4];
  const int64_t pr = blockIdx.x;
  const int j = (int)(pr % n_s);
  const int i = (int)((pr / n_s) % n_s);
  const int64_t b = pr / ((int64_t)n_s * n_s);
  float* out = scores + pr;
  if (i == j) {
    if (threadIdx.x == 0) *out = -INFINITY;
    return;
  }
  const float* xb = x + b * N * ld;
  const int64_t ti0 = (int64_t)i * S, tj0 = (int64_t)j * S;
  const int ni = (int)min((int64_t)S, N - ti0), nj = (int)min((int64_t)S, N - tj0);
  for (int u = threadIdx.x; u < nj; u += 256) {
    const float n = norm_f32(xb + (tj0 + u) * ld, d);
    rnj[u] = n > 0.f ? 1.0f / n : 0.f;
  }
  __syncthreads();
  float part = 0.f;
  for (int t = threadIdx.x; t < ni; t += 256) {
    const float* xt = xb + (ti0 + t) * ld;
    const float nt = norm_f32(xt, d);
    float best = -INFINITY;
    for (int u = 0; u < nj; ++u) {
      const float* xu = xb + (tj0 + u) * ld;
      float dot = 0.f;
      for (int c = 0; c < d; ++c) dot = fmaf(xt[c], xu[c], dot);
      best = fmaxf(best, dot * rnj[u]);
    }
    part += best * (nt > 0.f ? 1.0f / nt : 0.f);
  }
  const float tot = block_sum(part, red);
  if (threadIdx.x == 0) *out = tot;
}

// One thread per output element (b, token, feature).
__global__ void __launch_bounds__(256) compress_f32_kernel(const float* __restrict__ x, int64_t B, int64_t N, int d,
                                                            int64_t ld_x, int S, int k, int n_s,
                                                            const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                            const float* __restrict__ P, int residual,
                                                            float* __restrict__ xhat, int64_t ld_out,
                                                            LayerEpi epi) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= B * N * d) return;
  const int f = (int)(e % d);
  const int64_t bt = e / d;
  const int64_t t = bt % N, b = bt / N;
  const int i = (int)(t / S), s = (int)(t % S);
  const float* xb = x + b * N * ld_x;
  const int KP = (k + 1) * S;
  const float* prow = P + (int64_t)s * KP;
  float acc = 0.f;
  for (int blk = 0; blk <= k; ++blk) {
    int src = blk ? idx[(b * n_s + i) * k + blk - 1] : i;
    if (src < 0) continue;                 // empty block (unidirectional padding)
    src = min(src, n_s - 1);
    const float wt = blk ? w[(b * n_s + i) * k + blk - 1] : 1.f;
    for (int slot = 0; slot < S; ++slot) {
      const int64_t tok = (int64_t)src * S + slot;
      if (tok >= N) break;
      acc = fmaf(prow[blk * S + slot], wt * xb[tok * ld_x + f], acc);
    }
  }
  if (residual) acc += xb[t * ld_x + f];
  if (epi.bias) acc += epi.bias[s];
  if (epi.act) acc = fmaxf(acc, 0.f);
  xhat[(b * N + t) * ld_out + f] = acc;
}

// One workgroup per (b, token p): cosine row G_p., its sum, then the mixed output row.
__global__ void __launch_bounds__(256) dyn_f32_kernel(const float* __restrict__ z, int64_t N, int m_t, int64_t ld_z,
                                                       int S, float eps, float* __restrict__ out, int64_t ld_out,
                                                       LayerEpi epi) {
  __shared__ float g[512];
  __shared__ float red[4];
  const int64_t bt = blockIdx.x;
  const int64_t t = bt % N, b = bt / N;
  const int64_t base = (t / S) * S;
  const int nv = (int)min((int64_t)S, N - base);
  const float* zb = z + b * N * ld_z;
  const float* zp = zb + t * ld_z;
  const float np_ = norm_f32(zp, m_t);
  float part = 0.f;
  for (int q = threadIdx.x; q < nv; q += 256) {
    const float* zq = zb + (base + q) * ld_z;
    const float nq = norm_f32(zq, m_t);
    float dot = 0.f;
    for (int c = 0; c < m_t; ++c) dot = fmaf(zp[c], zq[c], dot);
    float gq = (np_ > 0.f && nq > 0.f) ? dot / (np_ * nq) : 0.f;
    if (epi.norm == kNormSoftmax) gq = expf(gq);
    g[q] = gq;
    part += epi.norm == kNormRms ? gq * gq : gq;
  }
  const float r = block_sum(part, red);   // contains a barrier: g[] is complete afterwards
  // row scale: 1 / (sum + eps) (eq. 6), 1 / sum (softmax), 1 / sqrt(mean square + eps), 1
  const float den = epi.norm == kNormSum ? r + eps
                  : epi.norm == kNormSoftmax ? r
                  : epi.norm == kNormRms ? sqrtf(r / (float)nv + eps) : 1.f;
  const float bv = epi.bias ? epi.bias[t - base] : 0.f;
  for (int f = threadIdx.x; f < m_t; f += 256) {
    float acc = 0.f;
    for (int q = 0; q < nv; ++q) acc = fmaf(g[q], zb[(base + q) * ld_z + f], acc);
    float y = acc / den + bv;
    if (epi.act) y = fmaxf(y, 0.f);
    out[(b * N + t) * ld_out + f] = y;
  }
}

// Enricher: one thread per output element (token t, feature j): ReLU(x_t . U[:, j] + b_j)^2.
__global__ void __launch_bounds__(256) enrich_f32_kernel(const float* __restrict__ x, int64_t M, int d, int64_t ld_x,
                                                          const float* __restrict__ U, int m,
                                                          const float* __restrict__ bias, float* __restrict__ z,
                                                          int64_t ld_z) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= M * m) return;
  const int j = (int)(e % m);
  const int64_t t = e / m;
  float acc = bias ? bias[j] : 0.f;
  for (int c = 0; c < d; ++c) acc = fmaf(x[t * ld_x + c], U[(int64_t)c * m + j], acc);
  const float r = fmaxf(acc, 0.f);
  z[t * ld_z + j] = r * r;
}

// Fuser: one thread per output element (token t, feature f):
// sum_j<m_h z[t][j] O[j][f] + sum_j<m_t c[t][j] O[m_h + j][f] + x_res[t][f].
__global__ void __launch_bounds__(256) fuse_f32_kernel(const float* __restrict__ z, int64_t M, int m_h, int64_t ld_z,
                                                        const float* __restrict__ c, int m_t, int64_t ld_c,
                                                        const float* __restrict__ O, int d,
                                                        const float* __restrict__ xr, int64_t ld_res,
                                                        float* __restrict__ y, int64_t ld_y) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= M * d) return;
  const int f = (int)(e % d);
  const int64_t t = e / d;
  float acc = 0.f;
  for (int j = 0; j < m_h; ++j) acc = fmaf(z[t * ld_z + j], O[(int64_t)j * d + f], acc);
  for (int j = 0; j < m_t; ++j) acc = fmaf(c[t * ld_c + j], O[(int64_t)(m_h + j) * d + f], acc);
  y[t * ld_y + f] = acc + xr[t * ld_res + f];
}

}  // namespace

hipError_t launch_enrich_f32(const float* x, int64_t M, int d, int64_t ld_x, const float* U, int m,
                             const float* bias, float* z, int64_t ld_z, hipStream_t stream) {
  hipLaunchKernelGGL(enrich_f32_kernel, dim3((unsigned)((M * m + 255) / 256)), dim3(256), 0, stream, x, M, d, ld_x,
                     U, m, bias, z, ld_z);
  return hipGetLastError();
}

hipError_t launch_fuse_f32(const float* z, int64_t M, int m_h, int64_t ld_z, const float* c, int m_t, int64_t ld_c,
                           const float* O, int d, const float* x_res, int64_t ld_res, float* y, int64_t ld_y,
                           hipStream_t stream) {
  hipLaunchKernelGGL(fuse_f32_kernel, dim3((unsigned)((M * d + 255) / 256)), dim3(256), 0, stream, z, M, m_h, ld_z,
                     c, m_t, ld_c, O, d, x_res, ld_res, y, ld_y);
  return hipGetLastError();
}

hipError_t launch_maxsim_f32(const float* xn, int64_t B, int64_t N, int d, int S, float* scores, hipStream_t stream) {
  const int n_s = (int)((N + S - 1) / S);
  const int64_t grid = B * n_s * n_s;
  hipLaunchKernelGGL(maxsim_f32_kernel, dim3((unsigned)grid), dim3(256), 0, stream, xn, N, d, S, n_s, scores);
  return hipGetLastError();
}

hipError_t launch_maxsim_rows_f32(const float* x, int64_t B, int64_t N, int d, int64_t ld, int S, float* scores,
                                  hipStream_t stream) {
  const int n_s = (int)((N + S - 1) / S);
  const int64_t grid = B * n_s * n_s;
  hipLaunchKernelGGL(maxsim_rows_f32_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, N, d, ld, S, n_s, scores);
  return hipGetLastError();
}

hipError_t launch_compress_f32(const float* x, int64_t B, int64_t N, int d, int64_t ld_x, int S, int k,
                               const int32_t* idx, const float* w, const float* P, int residual, float* xhat,
                               int64_t ld_out, hipStream_t stream, LayerEpi epi) {
  const int n_s = (int)((N + S - 1) / S);
  const int64_t total = B * N * d;
  hipLaunchKernelGGL(compress_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, x, B, N, d,
                     ld_x, S, k, n_s, idx, w, P, residual, xhat, ld_out, epi);
  return hipGetLastError();
}

hipError_t launch_dyn_f32(const float* z, int64_t B, int64_t N, int m_t, int64_t ld_z, int S, float eps, float* out,
                          int64_t ld_out, hipStream_t stream, LayerEpi epi) {
  hipLaunchKernelGGL(dyn_f32_kernel, dim3((unsigned)(B * N)), dim3(256), 0, stream, z, N, m_t, ld_z, S, eps, out,
                     ld_out, epi);
  return hipGetLastError();
}

}  // namespace avey
