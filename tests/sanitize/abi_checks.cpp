// Host-side argument checks of libavey under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Every call below is rejected by the checks or is empty work, so no HIP call is made; the
// point is that the checks themselves (size products, alignment arithmetic, pointer offsets)
// stay free of overflow and out-of-bounds accesses for any argument values, including the
// extremes of int64_t. Exit status: 0 when every call returns the expected status; a sanitizer
// report aborts the process.
#include <stdint.h>
#include <stdio.h>

#include <initializer_list>

#include "avey.h"

namespace {

int failures = 0;

void expect(const char* what, int64_t got, int64_t want) {
  if (got != want) {
    fprintf(stderr, "%s: status %lld, expected %lld\n", what, (long long)got, (long long)want);
    ++failures;
  }
}

// A rejected call: any non-OK status counts as rejected here; its exact code is checked by the
// Python tests.
void rejected(const char* what, int64_t got) {
  if (got == AVEY_OK) {
    fprintf(stderr, "%s: accepted, expected a rejection\n", what);
    ++failures;
  }
}

void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }

}  // namespace

int main() {
  void* p16 = P(0x10000);
  float* f16 = static_cast<float*>(p16);
  int32_t* i16 = static_cast<int32_t*>(p16);
  const int64_t big[] = {INT64_MAX, INT64_MAX - 1, INT64_MIN, -1, (int64_t)1 << 62, (int64_t)1 << 40,
                         (int64_t)1 << 31, 0x7fffffff, 3};
  const int32_t bigs[] = {INT32_MAX, INT32_MIN, -1, 0, 1, 16, 512, 513};
  const avey_dtype dts[] = {AVEY_BF16, AVEY_F32, static_cast<avey_dtype>(7)};

  // empty work is accepted with NULL pointers
  expect("split_rank empty", avey_split_rank(nullptr, AVEY_BF16, 0, 1024, 64, 64, 64, 3, nullptr, nullptr, nullptr, nullptr), AVEY_OK);
  expect("maxsim empty", avey_maxsim(nullptr, AVEY_BF16, 1, 0, 64, 64, 64, nullptr, nullptr), AVEY_OK);
  expect("noalloc empty", avey_split_rank_noalloc(nullptr, AVEY_F32, 0, 5, 64, 64, 64, 3, nullptr, nullptr, nullptr, nullptr), AVEY_OK);
  expect("compress empty", avey_select_compress(nullptr, AVEY_BF16, 0, 1024, 64, 64, 64, 3, nullptr, nullptr, nullptr, 1, nullptr, 64, nullptr), AVEY_OK);
  expect("dyn empty", avey_dyn_context(nullptr, AVEY_BF16, 2, 0, 64, 64, 64, 1e-8f, nullptr, 64, nullptr), AVEY_OK);
  expect("workspace empty", avey_rank_workspace_bytes(AVEY_BF16, 0, 1000, 64, 64), 0);

  // every size argument at the extremes, each call with one required pointer NULL so that it is
  // rejected before any HIP call (no size here is 0, which would be empty work): the checks must
  // reach their verdict without overflow
  for (avey_dtype dt : dts) {
    for (int64_t B : big) {
      for (int64_t N : big) {
        for (int64_t d : big) {
          for (int32_t S : bigs) {
            const int64_t ws = avey_rank_workspace_bytes(dt, B, N, d, S);
            if (ws > ((int64_t)1 << 48)) {
              fprintf(stderr, "rank_workspace_bytes accepted an absurd size: %lld\n", (long long)ws);
              ++failures;
            }
            rejected("split_rank", avey_split_rank(p16, dt, B, N, d, d, S, 3, nullptr, i16, f16, nullptr));
            rejected("split_rank_preceding", avey_split_rank_preceding(p16, dt, B, N, d, d, S, S, f16, i16, nullptr, nullptr));
            rejected("maxsim", avey_maxsim(p16, dt, B, N, d, N, S, nullptr, nullptr));
            rejected("noalloc", avey_split_rank_noalloc(p16, dt, B, N, d, d, S, 3, f16, nullptr, f16, nullptr));
            rejected("prepare", avey_maxsim_prepare(p16, dt, B, N, d, d, S, nullptr, nullptr));
            rejected("scores", avey_maxsim_scores(p16, dt, B, N, d, S, nullptr, nullptr));
            rejected("topk", avey_topk_norm(f16, B, N, S, i16, nullptr, nullptr));
            rejected("topk_preceding", avey_topk_norm_preceding(f16, B, N, S, nullptr, f16, nullptr));
            rejected("compress", avey_select_compress(p16, dt, B, N, d, d, S, 3, i16, f16, p16, 1, nullptr, d, nullptr));
            rejected("compress P", avey_select_compress(p16, dt, B, N, d, d, S, (int32_t)N, i16, f16, nullptr, 1, p16, d, nullptr));
            rejected("dyn", avey_dyn_context(p16, dt, B, N, d, d, S, 1e-8f, nullptr, d, nullptr));
            rejected("dyn_layer", avey_dyn_layer(p16, dt, B, N, d, d, S, 1e-8f, 0, nullptr, 0, nullptr, d, nullptr));
            rejected("static", avey_static_layer(p16, dt, B, N, d, d, S, nullptr, nullptr, 0, p16, d, nullptr));
            rejected("enrich", avey_enrich(p16, dt, N, d, d, nullptr, B, nullptr, p16, B, nullptr));
            rejected("fuse", avey_fuse(p16, dt, N, B, d, p16, d, d, nullptr, B, p16, B, p16, B, nullptr));
          }
        }
      }
    }
  }
  // status strings for every code, including unknown ones
  for (int32_t c : {0, -1, -2, -3, -4, -5, -6, 7, INT32_MIN, INT32_MAX}) {
    const char* s = avey_status_str(c);
    if (!s || !s[0]) ++failures;
  }
  expect("abi version", avey_abi_version(), AVEY_ABI_VERSION);
  if (failures) fprintf(stderr, "%d unexpected results\n", failures);
  else printf("abi checks: all calls rejected or empty as expected\n");
  return failures ? 1 : 0;
}
