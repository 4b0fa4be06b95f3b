// Internal launchers (not exported). Argument checks happen in abi.hip before any of these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace avey {

hipError_t launch_prepare(const void* x, bool bf16, int64_t B, int64_t N, int d, int64_t ld, int S, void* ws,
                          hipStream_t stream);
// MaxSim from the packed, normalised workspace that launch_prepare wrote (d padded to whole chunks
// of 32 features), and straight from the caller's row-major X (norms on chip).
hipError_t launch_maxsim_bf16(const uint16_t* xp, int64_t B, int64_t N, int d, int S, float* scores,
                              hipStream_t stream);
hipError_t launch_maxsim_rows_bf16(const uint16_t* x, int64_t B, int64_t N, int d, int64_t ld, int S, float* scores,
                                   hipStream_t stream);
hipError_t launch_topk_norm(const float* scores, int64_t B, int64_t n_s, int k, bool preceding, int32_t* idx,
                            float* w, hipStream_t stream);

// Row normalisation of the dynamic layer's cosine matrix: divide by sum + eps (eq. 6), softmax,
// divide by the root mean square, or none.
constexpr int kNormSum = 0, kNormSoftmax = 1, kNormRms = 2, kNormNone = 3;

// Output epilogue of a contextualizer layer, y = act(v + bias[s]) with s the token's position in
// its split: bias holds S fp32 values (nullptr: no bias); act 0 is the identity, 1 is ReLU. norm
// is the dynamic layer's row normalisation (one of kNorm*; the static layer ignores it).
struct LayerEpi {
  const float* bias = nullptr;
  int act = 0;
  int norm = kNormSum;
};

constexpr int kCompressMaxBlocks = 512;   // bf16 gather + compress: k + 1 <= this
hipError_t launch_compress_bf16(const uint16_t* x, int64_t B, int64_t N, int d, int64_t ld_x, int S, int k,
                                const int32_t* idx, const float* w, const uint16_t* P, int residual, uint16_t* xhat,
                                int64_t ld_out, hipStream_t stream, LayerEpi epi = {});
hipError_t launch_dyn_bf16(const uint16_t* z, int64_t B, int64_t N, int m_t, int64_t ld_z, int S, float eps,
                           uint16_t* out, int64_t ld_out, hipStream_t stream, LayerEpi epi = {});

constexpr int kEnrichMaxWidth = 4096;   // bf16 enricher: m <= this (LDS bias table)
hipError_t launch_enrich_bf16(const uint16_t* x, int64_t M, int d, int64_t ld_x, const uint16_t* U, int m,
                              const float* bias, uint16_t* z, int64_t ld_z, hipStream_t stream);
hipError_t launch_fuse_bf16(const uint16_t* z, int64_t M, int m_h, int64_t ld_z, const uint16_t* c, int m_t,
                            int64_t ld_c, const uint16_t* O, int d, const uint16_t* x_res, int64_t ld_res,
                            uint16_t* y, int64_t ld_y, hipStream_t stream);
hipError_t launch_enrich_f32(const float* x, int64_t M, int d, int64_t ld_x, const float* U, int m,
                             const float* bias, float* z, int64_t ld_z, hipStream_t stream);
hipError_t launch_fuse_f32(const float* z, int64_t M, int m_h, int64_t ld_z, const float* c, int m_t, int64_t ld_c,
                           const float* O, int d, const float* x_res, int64_t ld_res, float* y, int64_t ld_y,
                           hipStream_t stream);

hipError_t launch_maxsim_f32(const float* xn, int64_t B, int64_t N, int d, int S, float* scores, hipStream_t stream);
hipError_t launch_maxsim_rows_f32(const float* x, int64_t B, int64_t N, int d, int64_t ld, int S, float* scores,
                                  hipStream_t stream);
hipError_t launch_compress_f32(const float* x, int64_t B, int64_t N, int d, int64_t ld_x, int S, int k,
                               const int32_t* idx, const float* w, const float* P, int residual, float* xhat,
                               int64_t ld_out, hipStream_t stream, LayerEpi epi = {});
hipError_t launch_dyn_f32(const float* z, int64_t B, int64_t N, int m_t, int64_t ld_z, int S, float eps, float* out,
                          int64_t ld_out, hipStream_t stream, LayerEpi epi = {});

// Peak micro-benchmarks (peak_probe.hip).
int probe_cus();   // compute units of the current device, or -1
hipError_t launch_mfma_probe(int64_t iters, int changing, float* sink, int cus, hipStream_t stream);
hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, int cus, hipStream_t stream);

}  // namespace avey
