// Host-side argument checks shared by the C entry points (abi.hip, noalloc.hip). Internal: every
// check runs before any HIP call, so a call that fails one enqueues nothing.
#pragma once

#include <stdint.h>

#include "avey.h"
#include "launch.h"

namespace avey {
namespace {

constexpr int64_t kMaxS = 512;
constexpr int64_t kI32 = 0x7fffffffLL;
// Every size argument is checked to lie in [0, kMaxDim] before it enters any arithmetic, and
// products of sizes are formed with prod(), which saturates at INT64_MAX instead of overflowing.
constexpr int64_t kMaxDim = int64_t(1) << 40;

bool size_ok(int64_t v) { return v >= 0 && v <= kMaxDim; }

int64_t prod(int64_t a) { return a; }
template <class... R>
int64_t prod(int64_t a, int64_t b, R... rest) {
  int64_t p;
  if (__builtin_mul_overflow(a, b, &p)) p = INT64_MAX;
  return prod(p, rest...);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t splits(int64_t N, int64_t S) { return (N + S - 1) / S; }

avey_status hip_status(hipError_t e) { return e == hipSuccess ? AVEY_OK : AVEY_ERR_HIP; }

// Checks common to the three tensor entry points. Returns AVEY_OK with *empty set when there is
// nothing to do.
avey_status check_common(avey_dtype dt, int64_t B, int64_t N, int32_t S, bool* empty) {
  if (dt != AVEY_F32 && dt != AVEY_BF16) return AVEY_ERR_DTYPE;
  if (!size_ok(B) || !size_ok(N) || S < 1 || S > kMaxS) return AVEY_ERR_SHAPE;
  *empty = (B == 0 || N == 0);
  return AVEY_OK;
}

// A [B, N, width] operand with row stride ld; bf16 widths must be multiples of `mult`.
avey_status check_tensor(const void* p, avey_dtype dt, int64_t N, int64_t width, int64_t ld, int64_t mult = 64) {
  if (!p) return AVEY_ERR_NULL;
  if (width < 1 || ld < width || ld > kMaxDim) return AVEY_ERR_SHAPE;
  if (dt == AVEY_BF16) {
    if (width % mult) return AVEY_ERR_UNSUPPORTED;
    if (ld % 8 || !aligned(p, 16)) return AVEY_ERR_ALIGN;
    if (prod(N, ld) >= (1LL << 30)) return AVEY_ERR_UNSUPPORTED;   // byte offsets within a sequence stay < 2^31
  } else {
    if (!aligned(p, 4)) return AVEY_ERR_ALIGN;
  }
  return AVEY_OK;
}

// bf16 split lengths: multiples of 16 (the MFMA operand tiles are padded with zero rows).
avey_status check_split_bf16(avey_dtype dt, int32_t S) {
  return (dt == AVEY_BF16 && S % 16) ? AVEY_ERR_UNSUPPORTED : AVEY_OK;
}

#define AVEY_TRY(expr)                      \
  do {                                      \
    const avey_status s_ = (expr);          \
    if (s_ != AVEY_OK) return s_;           \
  } while (0)

// Feature count of the bf16 ranker workspace: d padded with zeros to whole chunks of 32.
int64_t padded_d(avey_dtype dt, int64_t d) { return dt == AVEY_BF16 ? (d + 31) / 32 * 32 : d; }

// Bytes of the ranker workspace (normalised, padded copy of X), or a negative status.
// Rows per packed block of the bf16 workspace: S, or 256 at S = 64 and 128, where the MaxSim
// kernel takes 256 / S consecutive splits (256 consecutive tokens) as one side of a unit.
int32_t pack_rows(avey_dtype dt, int32_t S) { return (dt == AVEY_BF16 && (S == 64 || S == 128)) ? 256 : S; }

int64_t workspace_bytes(avey_dtype dt, int64_t B, int64_t N, int64_t d, int32_t S) {
  const int64_t eb = dt == AVEY_BF16 ? 2 : 4;
  const int32_t P = pack_rows(dt, S);
  return prod(B, splits(N, P), P, padded_d(dt, d), eb);
}

// Checks of the ranker (scoring, and the workspace path's preparation) on the shape alone. bf16
// takes S a multiple of 16 and d a multiple of 8.
avey_status check_rank_shape(avey_dtype dt, int64_t B, int64_t N, int64_t d, int32_t S, bool* empty) {
  AVEY_TRY(check_common(dt, B, N, S, empty));
  if (*empty) return AVEY_OK;
  if (d < 1 || d > kMaxDim) return AVEY_ERR_SHAPE;
  const int64_t n_s = splits(N, S);
  if (n_s < 2) return AVEY_ERR_SHAPE;
  const int32_t P = pack_rows(dt, S);
  const int64_t n_p = splits(N, P);                                          // packed blocks
  if (dt == AVEY_BF16) {
    if (S % 16 || d % 8) return AVEY_ERR_UNSUPPORTED;
    if (prod(n_p, P, padded_d(dt, d)) >= (1LL << 30)) return AVEY_ERR_UNSUPPORTED;   // workspace offsets < 2^31
    if (prod(n_s, n_s - 1) / 2 > kI32) return AVEY_ERR_UNSUPPORTED;
  } else {
    if (prod(B, n_s, n_s) > kI32) return AVEY_ERR_UNSUPPORTED;
  }
  if (prod(B, n_p, P) > 16 * kI32) return AVEY_ERR_UNSUPPORTED;            // prepare's grid
  if (prod(B, n_p, P, padded_d(dt, d)) > (1LL << 45)) return AVEY_ERR_UNSUPPORTED;   // workspace elements
  return AVEY_OK;
}

// The workspace-free scoring's reads of X: the kernel's byte offsets per sequence, up to the rows
// of a whole last unit past N (which it reads as zeros), stay below 2^31.
avey_status check_rank_rows(const void* x, avey_dtype dt, int64_t N, int64_t d, int64_t ld_x) {
  AVEY_TRY(check_tensor(x, dt, N, d, ld_x, 8));
  if (dt == AVEY_BF16 && prod(N + 512, ld_x) >= (1LL << 30)) return AVEY_ERR_UNSUPPORTED;
  return AVEY_OK;
}

avey_status check_prepare(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d, int64_t ld_x, int32_t S,
                          const void* ws, bool* empty) {
  AVEY_TRY(check_rank_shape(dt, B, N, d, S, empty));
  if (*empty) return AVEY_OK;
  if (!ws) return AVEY_ERR_NULL;
  AVEY_TRY(check_tensor(x, dt, N, d, ld_x, 8));
  if (!aligned(ws, 16)) return AVEY_ERR_ALIGN;
  return AVEY_OK;
}

avey_status check_scores(const void* ws, avey_dtype dt, int64_t B, int64_t N, int64_t d, int32_t S,
                         const float* scores, bool* empty) {
  AVEY_TRY(check_rank_shape(dt, B, N, d, S, empty));
  if (*empty) return AVEY_OK;
  if (!ws || !scores) return AVEY_ERR_NULL;
  if (!aligned(ws, 16) || !aligned(scores, 4)) return AVEY_ERR_ALIGN;
  return AVEY_OK;
}

avey_status check_topk(const float* scores, int64_t B, int64_t n_s, int32_t k, const int32_t* idx, const float* w,
                       bool* empty) {
  if (!size_ok(B) || !size_ok(n_s)) return AVEY_ERR_SHAPE;
  *empty = (B == 0 || n_s == 0);
  if (*empty) return AVEY_OK;
  if (!scores || !idx || !w) return AVEY_ERR_NULL;
  if (n_s < 2 || k < 1 || k > n_s - 1 || n_s > kI32) return AVEY_ERR_SHAPE;
  if (!aligned(scores, 4) || !aligned(idx, 4) || !aligned(w, 4)) return AVEY_ERR_ALIGN;
  if (prod(B, n_s) > 4 * kI32) return AVEY_ERR_UNSUPPORTED;                 // top-k grid
  return AVEY_OK;
}

}  // namespace
}  // namespace avey
