// Inverse L2 norm of every token: rn[b, t] = 1 / |x_t| (0 for a zero row). This is the scale of
// the cosine normalisation N(.) (papernotes.org Avey-B note, 关键设计 2) that MaxSim applies to
// both sides of every dot product. One pass over X, fp32 accumulation; 16 lanes per row.
#include "avey_common.h"
#include "launch.h"

namespace avey {

namespace {

__global__ void __launch_bounds__(256) rnorm_bf16_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t N,
                                                          int d, int64_t ld, float* __restrict__ rn) {
  const int lane16 = threadIdx.x & 15;
  const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  float s = 0.f;
  if (r < rows) {
    const uint16_t* row = x + r * ld;   // rows of all sequences are evenly strided (batch stride N * ld)
    for (int c = lane16 * 8; c < d; c += 128) s = sumsq8(*reinterpret_cast<const uint4*>(row + c), s);
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (r < rows && lane16 == 0) rn[r] = s > 0.f ? 1.0f / sqrtf(s) : 0.f;
}

__global__ void __launch_bounds__(256) rnorm_f32_kernel(const float* __restrict__ x, int64_t rows, int64_t N, int d,
                                                         int64_t ld, float* __restrict__ rn) {
  const int lane16 = threadIdx.x & 15;
  const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  float s = 0.f;
  if (r < rows) {
    const float* row = x + r * ld;
    for (int c = lane16; c < d; c += 16) s = fmaf(row[c], row[c], s);
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (r < rows && lane16 == 0) rn[r] = s > 0.f ? 1.0f / sqrtf(s) : 0.f;
}

}  // namespace

hipError_t launch_rnorm(const void* x, bool bf16, int64_t B, int64_t N, int d, int64_t ld, float* rn,
                        hipStream_t stream) {
  const int64_t rows = B * N;
  const unsigned blocks = (unsigned)((rows + 15) / 16);
  if (bf16)
    hipLaunchKernelGGL(rnorm_bf16_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const uint16_t*>(x), rows,
                       N, d, ld, rn);
  else
    hipLaunchKernelGGL(rnorm_f32_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const float*>(x), rows, N,
                       d, ld, rn);
  return hipGetLastError();
}

}  // namespace avey
