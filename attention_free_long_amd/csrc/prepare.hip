// Ranker operand preparation: every token is normalised to unit L2 length, N(x) = x / |x| with
// N(0) = 0 (papernotes.org Avey-B note, 关键设计 2), and the last split is completed with zero
// padding tokens (方法详解/整体框架: the sequence is cut into S-token splits, the last one
// zero-padded). One pass over X; the sum of squares is accumulated in fp32.
//
// Output layouts (the ranker's workspace):
//   bf16: [B][n_s][nk][S][32], nk = ceil(d / 32) -- for each split, chunk-planes of 32
//         features holding S token rows of 64 bytes, so that a block of consecutive tokens of
//         one chunk is one contiguous run of memory. Values are N(x) rounded to bf16 (round to
//         nearest even); the features d .. 32 nk - 1 of the last plane are zero.
//   fp32: [B][n_s * S][d] row-major, N(x) in fp32.
#include "avey_common.h"
#include "launch.h"

namespace avey {

namespace {

// 16 lanes per token row; rows t >= N of the last split are written as zeros. Rows of up to
// 16 * 8 * RP features are read once and kept in registers between the norm and the scaling.
template <int RP>
__global__ void __launch_bounds__(256) prepare_bf16_kernel(const uint16_t* __restrict__ x, int64_t rows_p, int64_t N,
                                                            int d, int64_t ld, int S, int n_s,
                                                            uint16_t* __restrict__ xp) {
  const int lane16 = threadIdx.x & 15;
  const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);   // padded row over all sequences
  const int64_t per_seq = (int64_t)n_s * S;
  const int64_t b = r / per_seq, tp = r % per_seq;                    // sequence, padded token
  const bool live = r < rows_p;
  const bool valid = live && tp < N;
  const uint16_t* row = x + (b * N + (valid ? tp : 0)) * ld;
  uint4 v[RP];
  float s = 0.f;
#pragma unroll
  for (int p = 0; p < RP; ++p) {
    const int c = lane16 * 8 + p * 128;
    v[p] = (valid && c < d) ? *reinterpret_cast<const uint4*>(row + c) : make_uint4(0, 0, 0, 0);
    s = sumsq8(v[p], s);
  }
  for (int c = lane16 * 8 + RP * 128; c < d; c += 128)   // rows wider than the register tile
    if (valid) s = sumsq8(*reinterpret_cast<const uint4*>(row + c), s);
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) s += __shfl_xor(s, o, 16);
  const float rn = s > 0.f ? 1.0f / sqrtf(s) : 0.f;
  if (!live) return;
  const int j = (int)(tp / S), slot = (int)(tp % S);
  const int nkc = (d + 31) / 32, dp = nkc * 32;   // features padded with zeros to whole chunks
  uint16_t* dst = xp + ((b * n_s + j) * (int64_t)nkc * S + slot) * 32;
  auto put = [&](int c, uint4 u) {
    uint4 o;
    o.x = pack_bf16(bf16lo(u.x) * rn, bf16hi(u.x) * rn);
    o.y = pack_bf16(bf16lo(u.y) * rn, bf16hi(u.y) * rn);
    o.z = pack_bf16(bf16lo(u.z) * rn, bf16hi(u.z) * rn);
    o.w = pack_bf16(bf16lo(u.w) * rn, bf16hi(u.w) * rn);
    // feature c lives in chunk c / 32 at position c % 32 of the token's 32-element row
    *reinterpret_cast<uint4*>(dst + (int64_t)(c >> 5) * S * 32 + (c & 31)) = o;
  };
#pragma unroll
  for (int p = 0; p < RP; ++p) {
    const int c = lane16 * 8 + p * 128;
    if (c < dp) put(c, v[p]);   // zero past d
  }
  for (int c = lane16 * 8 + RP * 128; c < dp; c += 128)
    put(c, (valid && c < d) ? *reinterpret_cast<const uint4*>(row + c) : make_uint4(0, 0, 0, 0));
}

__global__ void __launch_bounds__(256) prepare_f32_kernel(const float* __restrict__ x, int64_t rows_p, int64_t N,
                                                           int d, int64_t ld, int S, int n_s,
                                                           float* __restrict__ xn) {
  const int lane16 = threadIdx.x & 15;
  const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int64_t per_seq = (int64_t)n_s * S;
  const int64_t b = r / per_seq, tp = r % per_seq;
  const bool live = r < rows_p;
  const bool valid = live && tp < N;
  const float* row = x + (b * N + (valid ? tp : 0)) * ld;
  float s = 0.f;
  if (valid)
    for (int c = lane16; c < d; c += 16) s = fmaf(row[c], row[c], s);
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) s += __shfl_xor(s, o, 16);
  const float rn = s > 0.f ? 1.0f / sqrtf(s) : 0.f;
  if (!live) return;
  float* dst = xn + r * d;
  for (int c = lane16; c < d; c += 16) dst[c] = valid ? row[c] * rn : 0.f;
}

}  // namespace

hipError_t launch_prepare(const void* x, bool bf16, int64_t B, int64_t N, int d, int64_t ld, int S, void* ws,
                          hipStream_t stream) {
  const int n_s = (int)((N + S - 1) / S);
  const int64_t rows_p = B * n_s * (int64_t)S;
  const unsigned blocks = (unsigned)((rows_p + 15) / 16);
  if (bf16)
    hipLaunchKernelGGL(prepare_bf16_kernel<8>, dim3(blocks), dim3(256), 0, stream, static_cast<const uint16_t*>(x),
                       rows_p, N, d, ld, S, n_s, static_cast<uint16_t*>(ws));
  else
    hipLaunchKernelGGL(prepare_f32_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const float*>(x), rows_p,
                       N, d, ld, S, n_s, static_cast<float*>(ws));
  return hipGetLastError();
}

}  // namespace avey
