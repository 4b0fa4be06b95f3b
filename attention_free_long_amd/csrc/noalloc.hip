// avey_split_rank_noalloc: the explicit-workspace ranker (normalised split-packed copy of X,
// MaxSim over it, top-k) for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops): its workspace is a file-scope device array that the library
// holds on every GPU it runs on until the process ends, so the call allocates nothing.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address on
// the current GPU comes from hipGetSymbolAddress, once per device, and only that address is
// passed to kernels. Every call on a GPU shares that GPU's array, so calls that overlap on one GPU
// (two streams, two host threads) race; each call overwrites the part it uses completely before
// reading it, so nothing has to be cleared between calls.
#include <mutex>

#include "checks.h"
#include "launch.h"

using namespace avey;

static __device__ __align__(256) uint8_t scratch[AVEY_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array (looked up on the first call on each device).
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" avey_status avey_split_rank_noalloc(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d,
                                               int64_t ld_x, int32_t S, int32_t k, float* scores, int32_t* idx,
                                               float* w, void* stream) {
  bool empty = false;
  AVEY_TRY(check_rank_shape(dt, B, N, d, S, &empty));
  if (empty) return AVEY_OK;
  if (!scores) return AVEY_ERR_NULL;
  AVEY_TRY(check_tensor(x, dt, N, d, ld_x, 8));
  if (!aligned(scores, 4)) return AVEY_ERR_ALIGN;
  if (prod(B, N, ld_x) > (1LL << 50)) return AVEY_ERR_UNSUPPORTED;   // x's offsets stay far from overflow
  const int64_t n_s = splits(N, S);
  AVEY_TRY(check_topk(scores, B, n_s, k, idx, w, &empty));
  // one sequence's copy must fit; as many whole sequences as fit go through each pass
  const int64_t per_seq = workspace_bytes(dt, 1, N, d, S);
  if (per_seq > AVEY_NOALLOC_SCRATCH_BYTES) return AVEY_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (scratch_on_current_device(&ws) != hipSuccess) return AVEY_ERR_HIP;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t per_pass = AVEY_NOALLOC_SCRATCH_BYTES / per_seq;
  const int64_t eb = dt == AVEY_BF16 ? 2 : 4;
  for (int64_t b0 = 0; b0 < B; b0 += per_pass) {
    const int64_t nb = B - b0 < per_pass ? B - b0 : per_pass;
    const void* xb = static_cast<const uint8_t*>(x) + b0 * N * ld_x * eb;
    float* sb = scores + b0 * n_s * n_s;
    AVEY_TRY(hip_status(launch_prepare(xb, dt == AVEY_BF16, nb, N, (int)d, ld_x, pack_rows(dt, S), ws, st)));
    if (dt == AVEY_BF16)
      AVEY_TRY(hip_status(launch_maxsim_bf16(static_cast<const uint16_t*>(ws), nb, N, (int)d, S, sb, st)));
    else
      AVEY_TRY(hip_status(launch_maxsim_f32(static_cast<const float*>(ws), nb, N, (int)d, S, sb, st)));
  }
  return hip_status(launch_topk_norm(scores, B, n_s, k, false, idx, w, st));
}
