// C ABI of libavey.so: argument checks and kernel launches. See include/avey.h for the contract.
#include "avey.h"
#include "avey_probe.h"

#include <stdint.h>

#include "checks.h"
#include "launch.h"

using namespace avey;

extern "C" {

int32_t avey_abi_version(void) { return AVEY_ABI_VERSION; }

const char* avey_status_str(int32_t s) {
  switch (s) {
    case AVEY_OK: return "AVEY_OK: success";
    case AVEY_ERR_NULL: return "AVEY_ERR_NULL: a required pointer is NULL";
    case AVEY_ERR_SHAPE: return "AVEY_ERR_SHAPE: a size or leading dimension is out of range";
    case AVEY_ERR_DTYPE: return "AVEY_ERR_DTYPE: unknown dtype";
    case AVEY_ERR_ALIGN: return "AVEY_ERR_ALIGN: a pointer or leading dimension is misaligned";
    case AVEY_ERR_UNSUPPORTED: return "AVEY_ERR_UNSUPPORTED: shape not implemented for this dtype";
    case AVEY_ERR_HIP: return "AVEY_ERR_HIP: the HIP runtime reported a launch error";
    default: return "unknown avey status";
  }
}

int64_t avey_rank_workspace_bytes(avey_dtype dt, int64_t B, int64_t N, int64_t d, int32_t S) {
  bool empty = false;
  const avey_status st = check_rank_shape(dt, B, N, d, S, &empty);
  if (st != AVEY_OK) return st;
  return empty ? 0 : workspace_bytes(dt, B, N, d, S);
}

avey_status avey_maxsim_prepare(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d, int64_t ld_x,
                                int32_t S, void* workspace, void* stream) {
  bool empty = false;
  AVEY_TRY(check_prepare(x, dt, B, N, d, ld_x, S, workspace, &empty));
  if (empty) return AVEY_OK;
  return hip_status(launch_prepare(x, dt == AVEY_BF16, B, N, (int)d, ld_x, pack_rows(dt, S), workspace,
                                   reinterpret_cast<hipStream_t>(stream)));
}

avey_status avey_maxsim_scores(const void* workspace, avey_dtype dt, int64_t B, int64_t N, int64_t d, int32_t S,
                               float* scores, void* stream) {
  bool empty = false;
  AVEY_TRY(check_scores(workspace, dt, B, N, d, S, scores, &empty));
  if (empty) return AVEY_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dt == AVEY_BF16)
    return hip_status(launch_maxsim_bf16(static_cast<const uint16_t*>(workspace), B, N, (int)d, S, scores, st));
  return hip_status(launch_maxsim_f32(static_cast<const float*>(workspace), B, N, (int)d, S, scores, st));
}

avey_status avey_topk_norm(const float* scores, int64_t B, int64_t n_s, int32_t k, int32_t* idx, float* w,
                           void* stream) {
  bool empty = false;
  AVEY_TRY(check_topk(scores, B, n_s, k, idx, w, &empty));
  if (empty) return AVEY_OK;
  return hip_status(launch_topk_norm(scores, B, n_s, k, false, idx, w, reinterpret_cast<hipStream_t>(stream)));
}

avey_status avey_topk_norm_preceding(const float* scores, int64_t B, int64_t n_s, int32_t k, int32_t* idx, float* w,
                                     void* stream) {
  bool empty = false;
  AVEY_TRY(check_topk(scores, B, n_s, k, idx, w, &empty));
  if (empty) return AVEY_OK;
  return hip_status(launch_topk_norm(scores, B, n_s, k, true, idx, w, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {
// MaxSim straight from X (no workspace): every check before the launch.
avey_status check_maxsim_rows(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d, int64_t ld_x,
                              int32_t S, const float* scores, bool* empty) {
  AVEY_TRY(check_rank_shape(dt, B, N, d, S, empty));
  if (*empty) return AVEY_OK;
  if (!scores) return AVEY_ERR_NULL;
  AVEY_TRY(check_rank_rows(x, dt, N, d, ld_x));
  if (!aligned(scores, 4)) return AVEY_ERR_ALIGN;
  return AVEY_OK;
}

avey_status launch_maxsim_rows(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d, int64_t ld_x,
                               int32_t S, float* scores, hipStream_t st) {
  if (dt == AVEY_BF16)
    return hip_status(launch_maxsim_rows_bf16(static_cast<const uint16_t*>(x), B, N, (int)d, ld_x, S, scores, st));
  return hip_status(launch_maxsim_rows_f32(static_cast<const float*>(x), B, N, (int)d, ld_x, S, scores, st));
}

avey_status split_rank(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d, int64_t ld_x, int32_t S,
                       int32_t k, float* scores, int32_t* idx, float* w, bool preceding, void* stream) {
  // Every check of both stages runs before the first launch.
  bool empty = false;
  AVEY_TRY(check_maxsim_rows(x, dt, B, N, d, ld_x, S, scores, &empty));
  if (empty) return AVEY_OK;
  const int64_t n_s = splits(N, S);
  AVEY_TRY(check_topk(scores, B, n_s, k, idx, w, &empty));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  AVEY_TRY(launch_maxsim_rows(x, dt, B, N, d, ld_x, S, scores, st));
  return hip_status(launch_topk_norm(scores, B, n_s, k, preceding, idx, w, st));
}
// Row-wise (position-wise) entry points: a [M, width] operand set.
avey_status check_rows(avey_dtype dt, int64_t M, bool* empty) {
  if (dt != AVEY_F32 && dt != AVEY_BF16) return AVEY_ERR_DTYPE;
  if (!size_ok(M)) return AVEY_ERR_SHAPE;
  *empty = M == 0;
  return AVEY_OK;
}

// Layer epilogue arguments: bias may be NULL (no bias), act is an avey_act.
avey_status check_epi(const float* bias, int32_t act, LayerEpi* epi) {
  if (act != AVEY_ACT_IDENTITY && act != AVEY_ACT_RELU) return AVEY_ERR_SHAPE;
  if (bias && !aligned(bias, 4)) return AVEY_ERR_ALIGN;
  epi->bias = bias;
  epi->act = act;
  return AVEY_OK;
}

avey_status dyn_layer(const void* z_tail, avey_dtype dt, int64_t B, int64_t N, int64_t m_t, int64_t ld_z, int32_t S,
                      float eps, LayerEpi epi, void* out, int64_t ld_out, void* stream) {
  bool empty = false;
  AVEY_TRY(check_common(dt, B, N, S, &empty));
  if (empty) return AVEY_OK;
  AVEY_TRY(check_tensor(z_tail, dt, N, m_t, ld_z, 8));
  AVEY_TRY(check_tensor(out, dt, N, m_t, ld_out, 8));
  AVEY_TRY(check_split_bf16(dt, S));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dt == AVEY_BF16) {
    const int64_t tiles = prod(B, splits(N, S), (S + 255) / 256, S > 256 ? 2 : 1);
    if (tiles > kI32) return AVEY_ERR_UNSUPPORTED;
    return hip_status(launch_dyn_bf16(static_cast<const uint16_t*>(z_tail), B, N, (int)m_t, ld_z, S, eps,
                                      static_cast<uint16_t*>(out), ld_out, st, epi));
  }
  if (prod(B, N) > kI32) return AVEY_ERR_UNSUPPORTED;
  return hip_status(launch_dyn_f32(static_cast<const float*>(z_tail), B, N, (int)m_t, ld_z, S, eps,
                                   static_cast<float*>(out), ld_out, st, epi));
}

}  // namespace

extern "C" {

avey_status avey_maxsim(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d, int64_t ld_x, int32_t S,
                        float* scores, void* stream) {
  bool empty = false;
  AVEY_TRY(check_maxsim_rows(x, dt, B, N, d, ld_x, S, scores, &empty));
  if (empty) return AVEY_OK;
  return launch_maxsim_rows(x, dt, B, N, d, ld_x, S, scores, reinterpret_cast<hipStream_t>(stream));
}

avey_status avey_split_rank(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d, int64_t ld_x, int32_t S,
                            int32_t k, float* scores, int32_t* idx, float* w, void* stream) {
  return split_rank(x, dt, B, N, d, ld_x, S, k, scores, idx, w, false, stream);
}

avey_status avey_split_rank_preceding(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d, int64_t ld_x,
                                      int32_t S, int32_t k, float* scores, int32_t* idx, float* w, void* stream) {
  return split_rank(x, dt, B, N, d, ld_x, S, k, scores, idx, w, true, stream);
}

avey_status avey_select_compress(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d, int64_t ld_x,
                                 int32_t S, int32_t k, const int32_t* idx, const float* w, const void* P,
                                 int32_t residual, void* xhat, int64_t ld_out, void* stream) {
  bool empty = false;
  AVEY_TRY(check_common(dt, B, N, S, &empty));
  if (empty) return AVEY_OK;
  if (!idx || !w || !P) return AVEY_ERR_NULL;
  AVEY_TRY(check_tensor(x, dt, N, d, ld_x, 8));
  AVEY_TRY(check_tensor(xhat, dt, N, d, ld_out, 8));
  if (k < 1 || (residual != 0 && residual != 1)) return AVEY_ERR_SHAPE;
  if (!aligned(idx, 4) || !aligned(w, 4)) return AVEY_ERR_ALIGN;
  if ((int64_t)S * (k + 1) * S >= (1LL << 30)) return AVEY_ERR_UNSUPPORTED;   // P byte offsets < 2^31
  AVEY_TRY(check_split_bf16(dt, S));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dt == AVEY_BF16) {
    if (!aligned(P, 16)) return AVEY_ERR_ALIGN;
    if (k + 1 > kCompressMaxBlocks) return AVEY_ERR_UNSUPPORTED;
    const int64_t tiles = prod(B, splits(N, S), (S + 255) / 256, (d + 255) / 256);
    if (tiles > kI32) return AVEY_ERR_UNSUPPORTED;
    return hip_status(launch_compress_bf16(static_cast<const uint16_t*>(x), B, N, (int)d, ld_x, S, k, idx, w,
                                           static_cast<const uint16_t*>(P), residual, static_cast<uint16_t*>(xhat),
                                           ld_out, st));
  }
  if (!aligned(P, 4)) return AVEY_ERR_ALIGN;
  if (prod(B, N, d) > 256 * kI32) return AVEY_ERR_UNSUPPORTED;
  return hip_status(launch_compress_f32(static_cast<const float*>(x), B, N, (int)d, ld_x, S, k, idx, w,
                                        static_cast<const float*>(P), residual, static_cast<float*>(xhat), ld_out, st));
}

avey_status avey_dyn_context(const void* z_tail, avey_dtype dt, int64_t B, int64_t N, int64_t m_t, int64_t ld_z,
                             int32_t S, float eps, void* out, int64_t ld_out, void* stream) {
  return dyn_layer(z_tail, dt, B, N, m_t, ld_z, S, eps, LayerEpi{}, out, ld_out, stream);
}

avey_status avey_dyn_layer(const void* z_tail, avey_dtype dt, int64_t B, int64_t N, int64_t m_t, int64_t ld_z,
                           int32_t S, float eps, int32_t norm, const float* bias, int32_t act, void* out,
                           int64_t ld_out, void* stream) {
  LayerEpi epi;
  AVEY_TRY(check_epi(bias, act, &epi));
  if (norm != AVEY_NORM_SUM && norm != AVEY_NORM_SOFTMAX && norm != AVEY_NORM_RMS && norm != AVEY_NORM_NONE)
    return AVEY_ERR_SHAPE;
  epi.norm = norm;
  return dyn_layer(z_tail, dt, B, N, m_t, ld_z, S, eps, epi, out, ld_out, stream);
}

avey_status avey_static_layer(const void* z_tail, avey_dtype dt, int64_t B, int64_t N, int64_t m_t, int64_t ld_z,
                              int32_t S, const void* V, const float* bias, int32_t act, void* out, int64_t ld_out,
                              void* stream) {
  bool empty = false;
  AVEY_TRY(check_common(dt, B, N, S, &empty));
  if (empty) return AVEY_OK;
  LayerEpi epi;
  AVEY_TRY(check_epi(bias, act, &epi));
  if (!V) return AVEY_ERR_NULL;
  AVEY_TRY(check_tensor(z_tail, dt, N, m_t, ld_z, 8));
  AVEY_TRY(check_tensor(out, dt, N, m_t, ld_out, 8));
  AVEY_TRY(check_split_bf16(dt, S));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // V Z_i is the gather + compress product with no retrieved block (k = 0: X_cat = Z_i, P = V)
  if (dt == AVEY_BF16) {
    if (!aligned(V, 16)) return AVEY_ERR_ALIGN;
    const int64_t tiles = prod(B, splits(N, S), (S + 255) / 256, (m_t + 255) / 256);
    if (tiles > kI32) return AVEY_ERR_UNSUPPORTED;
    return hip_status(launch_compress_bf16(static_cast<const uint16_t*>(z_tail), B, N, (int)m_t, ld_z, S, 0,
                                           nullptr, nullptr, static_cast<const uint16_t*>(V), 0,
                                           static_cast<uint16_t*>(out), ld_out, st, epi));
  }
  if (!aligned(V, 4)) return AVEY_ERR_ALIGN;
  if (prod(B, N, m_t) > 256 * kI32) return AVEY_ERR_UNSUPPORTED;
  return hip_status(launch_compress_f32(static_cast<const float*>(z_tail), B, N, (int)m_t, ld_z, S, 0, nullptr,
                                        nullptr, static_cast<const float*>(V), 0, static_cast<float*>(out), ld_out,
                                        st, epi));
}

avey_status avey_enrich(const void* x, avey_dtype dt, int64_t M, int64_t d, int64_t ld_x, const void* U,
                        int64_t m, const float* b, void* z, int64_t ld_z, void* stream) {
  bool empty = false;
  AVEY_TRY(check_rows(dt, M, &empty));
  if (empty) return AVEY_OK;
  if (!U) return AVEY_ERR_NULL;
  AVEY_TRY(check_tensor(x, dt, M, d, ld_x));
  AVEY_TRY(check_tensor(z, dt, M, m, ld_z));
  if (b && !aligned(b, 4)) return AVEY_ERR_ALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dt == AVEY_BF16) {
    if (!aligned(U, 16)) return AVEY_ERR_ALIGN;
    if (prod(d, m) >= (1LL << 30) || (b && m > kEnrichMaxWidth)) return AVEY_ERR_UNSUPPORTED;
    return hip_status(launch_enrich_bf16(static_cast<const uint16_t*>(x), M, (int)d, ld_x,
                                         static_cast<const uint16_t*>(U), (int)m, b, static_cast<uint16_t*>(z),
                                         ld_z, st));
  }
  if (!aligned(U, 4)) return AVEY_ERR_ALIGN;
  if (prod(M, m) > 256 * kI32) return AVEY_ERR_UNSUPPORTED;
  return hip_status(launch_enrich_f32(static_cast<const float*>(x), M, (int)d, ld_x, static_cast<const float*>(U),
                                      (int)m, b, static_cast<float*>(z), ld_z, st));
}

avey_status avey_fuse(const void* z, avey_dtype dt, int64_t M, int64_t m_h, int64_t ld_z, const void* c,
                      int64_t m_t, int64_t ld_c, const void* O, int64_t d, const void* x, int64_t ld_x,
                      void* y, int64_t ld_y, void* stream) {
  bool empty = false;
  AVEY_TRY(check_rows(dt, M, &empty));
  if (empty) return AVEY_OK;
  if (!O) return AVEY_ERR_NULL;
  if (!size_ok(m_h)) return AVEY_ERR_SHAPE;
  if (m_h > 0) AVEY_TRY(check_tensor(z, dt, M, m_h, ld_z));
  AVEY_TRY(check_tensor(c, dt, M, m_t, ld_c));
  AVEY_TRY(check_tensor(x, dt, M, d, ld_x));
  AVEY_TRY(check_tensor(y, dt, M, d, ld_y));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dt == AVEY_BF16) {
    if (m_h % 64) return AVEY_ERR_UNSUPPORTED;
    if (!aligned(O, 16)) return AVEY_ERR_ALIGN;
    if (prod(m_h + m_t, d) >= (1LL << 30)) return AVEY_ERR_UNSUPPORTED;
    return hip_status(launch_fuse_bf16(static_cast<const uint16_t*>(z), M, (int)m_h, ld_z,
                                       static_cast<const uint16_t*>(c), (int)m_t, ld_c,
                                       static_cast<const uint16_t*>(O), (int)d, static_cast<const uint16_t*>(x),
                                       ld_x, static_cast<uint16_t*>(y), ld_y, st));
  }
  if (!aligned(O, 4)) return AVEY_ERR_ALIGN;
  if (prod(M, d) > 256 * kI32) return AVEY_ERR_UNSUPPORTED;
  return hip_status(launch_fuse_f32(static_cast<const float*>(z), M, (int)m_h, ld_z, static_cast<const float*>(c),
                                    (int)m_t, ld_c, static_cast<const float*>(O), (int)d,
                                    static_cast<const float*>(x), ld_x, static_cast<float*>(y), ld_y, st));
}

int64_t avey_probe_mfma_flops(int64_t iters) {
  if (iters < 1 || iters > (1LL << 24)) return AVEY_ERR_SHAPE;
  const int cus = probe_cus();
  if (cus < 0) return AVEY_ERR_HIP;
  // per iteration and wave: 16 MFMAs of 32 x 32 x 16 multiply-adds
  return (int64_t)cus * 8 * iters * 16 * (2 * 32 * 32 * 16);
}

avey_status avey_probe_mfma_bf16(int64_t iters, int32_t changing, float* sink, void* stream) {
  if (iters < 1 || iters > (1LL << 24)) return AVEY_ERR_SHAPE;
  if (!sink) return AVEY_ERR_NULL;
  if (!aligned(sink, 4)) return AVEY_ERR_ALIGN;
  const int cus = probe_cus();
  if (cus < 0) return AVEY_ERR_HIP;
  return hip_status(launch_mfma_probe(iters, changing != 0, sink, cus, static_cast<hipStream_t>(stream)));
}

avey_status avey_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16) return AVEY_ERR_SHAPE;
  if (bytes == 0) return AVEY_OK;
  if (!src || !dst) return AVEY_ERR_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return AVEY_ERR_ALIGN;
  const int cus = probe_cus();
  if (cus < 0) return AVEY_ERR_HIP;
  return hip_status(launch_copy_probe(src, dst, bytes, cus, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
