// Per-split top-k with divide-by-max weights (papernotes.org Avey-B note, 方法详解/整体框架:
// keep the k most relevant candidate splits and divide their scores by the largest one;
// paperlayer.ai "Avey-B" summary, section 3).
//
// One wave per score row. Candidates are ordered by (score descending, index ascending), NaN
// ordering as -inf. With `preceding` set (the unidirectional ranker: only the splits before the
// target are candidates, paperlayer.ai "Avey-B" summary, section 3), a row with fewer than k
// candidates is completed with empty entries: index -1, weight 0. Round r picks the best candidate strictly after the round r-1 winner in
// that total order, so no "taken" set is needed: every lane scans its strided share of the
// row, then a 6-step butterfly of cross-lane shuffles finds the wave's best.
#include "avey_common.h"
#include "launch.h"

namespace avey {

namespace {

__device__ __forceinline__ bool better(float v, int j, float bv, int bj) {
  return v > bv || (v == bv && j < bj);
}

__global__ void __launch_bounds__(256) topk_norm_kernel(const float* __restrict__ scores, int64_t rows, int n_s,
                                                         int k, int preceding, int32_t* __restrict__ idx,
                                                         float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int i = (int)(row % n_s);
  const float* s = scores + row * n_s;

  float prev_v = INFINITY;
  int prev_j = -1;
  float s0 = 0.f;
  const int jend = preceding ? i : n_s;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bj = INT_MAX;
    for (int j = lane; j < jend; j += 64) {
      if (j == i) continue;
      float v = s[j];
      if (v != v) v = -INFINITY;
      const bool after = v < prev_v || (v == prev_v && j > prev_j);
      if (after && better(v, j, bv, bj)) {
        bv = v;
        bj = j;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oj = __shfl_xor(bj, o);
      if (better(ov, oj, bv, bj)) {
        bv = ov;
        bj = oj;
      }
    }
    if (bj == INT_MAX) {                       // no candidate left (preceding only)
      if (lane == 0) {
        idx[row * k + r] = -1;
        w[row * k + r] = 0.f;
      }
      continue;
    }
    if (lane == 0) {
      const float raw = s[bj];
      if (r == 0) s0 = raw;
      idx[row * k + r] = bj;
      w[row * k + r] = raw / s0;
    }
    prev_v = bv;
    prev_j = bj;
  }
}

}  // namespace

hipError_t launch_topk_norm(const float* scores, int64_t B, int64_t n_s, int k, bool preceding, int32_t* idx,
                            float* w, hipStream_t stream) {
  const int64_t rows = B * n_s;
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(topk_norm_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, scores, rows, (int)n_s, k,
                     preceding ? 1 : 0, idx, w);
  return hipGetLastError();
}

}  // namespace avey
