// Peak micro-benchmarks: the measured ceilings that the hot path's roofline fractions are also
// reported against, next to the datasheet peaks. Not part of the hot path.
//   * mfma_probe_kernel: one 8-wave workgroup per CU; each wave runs 16 independent
//     v_mfma_f32_32x32x16_bf16 per iteration on register operands (8 accumulator blocks, two
//     k-steps, the shape of the MaxSim and compression K loops without any memory traffic).
//     With `changing`, the operands are replaced every iteration by new bf16 bit patterns from
//     an integer hash (a few VALU operations per iteration), as operands read from memory would
//     be; without it the same operands are used throughout. The matrix pipes' power draw, and so
//     the clock the chip holds, depends on how much the operand bits toggle, so the two modes
//     bracket what a real contraction can reach.
//   * copy_probe_kernel: a grid-stride copy with 16-byte vector loads and stores.
#include "avey_common.h"
#include "launch.h"

namespace avey {

namespace {

// Eight bf16 values from a 32-bit hash: random signs and mantissas, exponents near 1.
__device__ __forceinline__ uint4 hashed_bf16x8(uint32_t h) {
  const uint32_t v = h * 0x165667B1u;
  return make_uint4((v & 0x807F807Fu) | 0x3C003C00u, ((v >> 3) & 0x807F807Fu) | 0x3C003C00u,
                    ((v >> 5) & 0x807F807Fu) | 0x3C003C00u, ((v >> 7) & 0x807F807Fu) | 0x3C003C00u);
}

__global__ void __launch_bounds__(512, 1) mfma_probe_kernel(int64_t iters, int changing, float* sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
  uint4 ra[2][4], rb[2][2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
#pragma unroll
    for (int a = 0; a < 4; ++a) ra[k][a] = hashed_bf16x8((uint32_t)(lane * 7 + a + 5 * k));
#pragma unroll
    for (int b = 0; b < 2; ++b) rb[k][b] = hashed_bf16x8((uint32_t)(lane * 5 + b + 11 * k + 1000));
  }
  for (int64_t g = 0; g < iters; ++g) {
    if (changing) {
      const uint32_t h = (uint32_t)g * 0x9E3779B9u + (uint32_t)lane * 0x85EBCA6Bu + (uint32_t)wave;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
#pragma unroll
        for (int a = 0; a < 4; ++a) ra[k][a] = hashed_bf16x8(h ^ ((uint32_t)a * 0x27D4EB2Fu + (uint32_t)k));
#pragma unroll
        for (int b = 0; b < 2; ++b) rb[k][b] = hashed_bf16x8(h ^ ((uint32_t)b * 0x61C88647u + 7u * (uint32_t)k));
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma32(as_bf16x8(ra[k][a]), as_bf16x8(rb[k][b]), acc[a][b]);
  }
  float s = 0.f;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) s += acc[a][b][lane & 15];
  // never true for finite sums of these magnitudes; keeps the MFMAs from being removed
  if (s == 1.0e30f) sink[blockIdx.x] = s;
}

__global__ void __launch_bounds__(256) copy_probe_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

int probe_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return -1;
  return cus;
}

hipError_t launch_mfma_probe(int64_t iters, int changing, float* sink, int cus, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)cus), dim3(512), 0, stream, iters, changing, sink);
  return hipGetLastError();
}

hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, int cus, hipStream_t stream) {
  // four 256-thread workgroups per CU, one 16-byte load and store per thread and step: of the
  // shapes tried (1 to 8 vectors per thread and step, 4 to 32 workgroups per CU, non-temporal
  // hints) the fastest on a 1 GiB copy
  const int64_t n16 = bytes / 16;
  const int64_t want = (n16 + 255) / 256;
  const unsigned grid = (unsigned)(want < (int64_t)cus * 4 ? want : (int64_t)cus * 4);
  hipLaunchKernelGGL(copy_probe_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace avey
