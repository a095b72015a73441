// Host-side exerciser of the C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_host_sanitizers.py builds it and the library's host code with them). It calls
// every entry point with extreme and inconsistent sizes, NULL, misaligned and overlapping
// (fake) pointers and undersized workspaces. It must run where no GPU is visible: a call that
// passes validation then stops at the device check, so no pointer below is ever dereferenced
// by a kernel. Every call must return a documented status code other than LCE_OK; any
// out-of-bounds access or undefined arithmetic in the validation, the size queries or the
// workspace carving aborts the program with a sanitizer report.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <vector>

#include "lce_masked.h"

extern "C" int hipGetDeviceCount(int* count);  // the runtime's int-sized hipError_t

namespace {

int failures = 0;
long calls = 0;

void expect(int rc, const char* what, int want = -1) {
  ++calls;
  const bool ok_code = rc >= LCE_OK && rc <= LCE_ERR_SCRATCH_LIMIT;
  if (!ok_code || rc == LCE_OK || (want >= 0 && rc != want)) {
    std::fprintf(stderr, "%s: status %d (wanted %s%d)\n", what, rc, want >= 0 ? "" : "nonzero ",
                 want >= 0 ? want : 0);
    ++failures;
  }
}

const int64_t kMax = std::numeric_limits<int64_t>::max();
const int64_t kMin = std::numeric_limits<int64_t>::min();
const int64_t kSizes[] = {kMin, -1, 0, 1, 7, 64, 1000, 128256, (int64_t(1) << 31) - 1,
                          int64_t(1) << 31, int64_t(1) << 40, int64_t(1) << 62, kMax};
const int64_t kChunks[] = {kMin, -1, 0, 1, 16, 1024, int64_t(1) << 40, kMax};
const uint32_t kFlags[] = {0u, 1u, 2u, 3u, 4u, 0x80000000u, 0xffffffffu};

// Fake device addresses: distinct, 256-byte aligned, far apart; `mis` is misaligned.
alignas(256) unsigned char arena[1 << 16];
void* fake(int i) { return arena + 4096 * (i % 16); }
void* mis(int i) { return arena + 4096 * (i % 16) + 1; }

}  // namespace

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == 0 && ndev > 0) {
    std::printf("skipped: a GPU is visible\n");
    return 0;
  }
  for (int code = -3; code < 16; ++code) {
    if (!lce_status_str(code) || !flce_status_str(code)) {
      std::fprintf(stderr, "status string %d is NULL\n", code);
      ++failures;
    }
  }
  size_t bytes = 0;
  expect(ce_chunked_workspace_size(10, 10, 4, nullptr), "ce ws NULL", LCE_ERR_NULL_ARG);
  expect(flce_workspace_size(10, 8, 10, 4, 0, nullptr), "flce ws NULL", LCE_ERR_NULL_ARG);
  for (int64_t n : kSizes)
    for (int64_t v : kSizes)
      for (int64_t c : kChunks) {
        const int rc = ce_chunked_workspace_size(n, v, c, &bytes);
        ++calls;
        if (rc != LCE_OK && rc != LCE_ERR_BAD_SHAPE && rc != LCE_ERR_BAD_CHUNK) {
          std::fprintf(stderr, "ce ws (%lld, %lld, %lld): %d\n", (long long)n, (long long)v,
                       (long long)c, rc);
          ++failures;
        }
        for (int64_t h : {int64_t(-8), int64_t(0), int64_t(8), int64_t(40), int64_t(4096),
                          int64_t(1) << 21, kMax})
          for (uint32_t f : kFlags) {
            const int r2 = flce_workspace_size(n, h, v, c, f, &bytes);
            ++calls;
            if (r2 != LCE_OK && r2 != LCE_ERR_BAD_SHAPE && r2 != LCE_ERR_BAD_CHUNK &&
                r2 != LCE_ERR_BAD_FLAGS) {
              std::fprintf(stderr, "flce ws: %d\n", r2);
              ++failures;
            }
          }
      }

  // CE entry points: shapes x strides x chunks, with consistent fake pointers and a large
  // workspace (validation passes only for valid shapes, then the device check stops it)
  auto* logits = static_cast<uint16_t*>(fake(0));
  auto* grad = static_cast<uint16_t*>(fake(1));
  auto* labels = static_cast<int32_t*>(fake(2));
  auto* lossp = static_cast<float*>(fake(3));
  auto* lse = static_cast<float*>(fake(4));
  auto* st = static_cast<int32_t*>(fake(5));
  void* ws = fake(6);
  auto* gout = static_cast<float*>(fake(7));
  const size_t big = size_t(1) << 60;
  for (int64_t n : kSizes)
    for (int64_t v : {int64_t(-1), int64_t(0), int64_t(1), int64_t(1000), int64_t(1) << 40, kMax})
      for (int64_t ldx : {int64_t(-1), int64_t(0), int64_t(3), int64_t(1) << 40})
        for (int64_t c : {int64_t(0), int64_t(16), kMax}) {
          // ld < v, = v, > v, far past v (saturating at the int64 range)
          const int64_t ld = ldx < 0 ? (v > kMin ? v - 1 : v) : (v <= kMax - ldx ? v + ldx : kMax);
          expect(ce_chunked_fwd(logits, n, v, ld, labels, -100, c, -1, lossp, lse, st, ws, big,
                                nullptr), "ce_chunked_fwd");
          expect(ce_chunked_bwd(logits, n, v, ld, grad, ld, labels, -100, c, -1, gout, lse, st,
                                ws, big, nullptr), "ce_chunked_bwd");
          expect(ce_chunked_bwd_inplace(logits, n, v, ld, labels, -100, c, 7, nullptr, nullptr,
                                        st, ws, big, nullptr), "ce_chunked_bwd_inplace");
          expect(ce_chunked_fwd_bwd_inplace(logits, n, v, ld, labels, -100, c, -1, gout, lossp,
                                            lse, st, ws, big, nullptr),
                 "ce_chunked_fwd_bwd_inplace");
          expect(ce_chunked_fwd_bwd_inplace_noalloc(logits, n, v, ld, labels, -100, c, -1, gout,
                                                    lossp, lse, st, nullptr),
                 "ce_chunked_fwd_bwd_inplace_noalloc");
          expect(ce_rows_fwd(logits, n, v, ld, labels, -100, c, lse, nullptr, st, ws, big,
                             nullptr), "ce_rows_fwd");
          expect(ce_rows_bwd(logits, n, v, ld, grad, ld, labels, -100, c, gout, lse, st, ws, big,
                             nullptr), "ce_rows_bwd");
        }
  // NULL, misaligned, overlapping, undersized
  expect(ce_chunked_fwd(nullptr, 4, 10, 10, labels, -100, 2, -1, lossp, lse, st, ws, big,
                        nullptr), "ce fwd NULL logits", LCE_ERR_NULL_ARG);
  expect(ce_chunked_fwd(static_cast<uint16_t*>(mis(0)), 4, 10, 10, labels, -100, 2, -1, lossp,
                        lse, st, ws, big, nullptr), "ce fwd misaligned", LCE_ERR_ALIGNMENT);
  expect(ce_chunked_fwd(logits, 4, 10, 10, labels, -100, 2, -1, lossp, lse, st, ws, 1, nullptr),
         "ce fwd small workspace", LCE_ERR_WORKSPACE);
  expect(ce_chunked_fwd(logits, 4, 10, 10, labels, -100, 2, -1,
                        reinterpret_cast<float*>(logits + 4), lse, st, ws, big, nullptr),
         "ce fwd loss inside logits", LCE_ERR_OVERLAP);
  expect(ce_chunked_bwd(logits, 4, 10, 10, logits + 5, 10, labels, -100, 2, -1, gout, lse, st,
                        ws, big, nullptr), "ce bwd grad overlapping logits", LCE_ERR_OVERLAP);
  expect(ce_chunked_fwd_bwd_inplace_noalloc(logits, int64_t(LCE_NOALLOC_MAX_ROWS) + 1, 10, 10,
                                            labels, -100, 2, -1, gout, lossp, lse, st, nullptr),
         "noalloc over the limit", LCE_ERR_SCRATCH_LIMIT);

  // FLCE entry points
  auto* hidden = static_cast<uint16_t*>(fake(8));
  auto* weight = static_cast<uint16_t*>(fake(9));
  auto* bias = static_cast<float*>(fake(10));
  auto* gh = static_cast<uint16_t*>(fake(11));
  auto* gw = static_cast<float*>(fake(12));
  auto* gb = static_cast<float*>(fake(13));
  for (int64_t n : kSizes)
    for (int64_t h : {int64_t(-8), int64_t(0), int64_t(8), int64_t(40), int64_t(4096),
                      int64_t(1) << 21, kMax})
      for (int64_t v : {int64_t(0), int64_t(1), int64_t(1000), int64_t(128256), int64_t(1) << 40,
                        kMax})
        for (int64_t c : {int64_t(0), int64_t(1), int64_t(1024), kMax})
          for (uint32_t f : {0u, 1u, 2u, 3u, 8u}) {
            expect(flce_fwd_bwd(hidden, weight, bias, labels, n, h, v, -100, c, -1, f, gout,
                                lossp, lse, gh, gw, gb, st, ws, big, nullptr), "flce_fwd_bwd");
            expect(flce_fwd(hidden, weight, bias, labels, n, h, v, -100, c, -1, lossp, lse, st,
                            ws, big, nullptr), "flce_fwd");
            expect(flce_bwd(hidden, weight, bias, labels, lse, n, h, v, -100, c, -1, f, gout, gh,
                            gw, gb, st, ws, big, nullptr), "flce_bwd");
          }
  expect(flce_fwd_bwd(hidden, weight, bias, labels, 64, 64, 1000, -100, 16, -1, 0, gout, lossp,
                      lse, gh, gw, gb, st, ws, 1, nullptr), "flce small workspace",
         LCE_ERR_WORKSPACE);
  expect(flce_fwd_bwd(hidden, weight, bias, labels, 64, 64, 1000, -100, 16, -1, 0, gout, lossp,
                      lse, hidden, gw, gb, st, ws, big, nullptr), "flce grad_hidden = hidden",
         LCE_ERR_OVERLAP);
  expect(flce_fwd_bwd(hidden, weight, bias, labels, 64, 64, 1000, -100, 16, -1, 0, gout, lossp,
                      lse, gh, reinterpret_cast<float*>(weight), gb, st, ws, big, nullptr),
         "flce grad_weight = weight", LCE_ERR_OVERLAP);
  expect(flce_fwd_bwd(hidden, static_cast<uint16_t*>(mis(9)), bias, labels, 64, 64, 1000, -100,
                      16, -1, 0, gout, lossp, lse, gh, gw, gb, st, ws, big, nullptr),
         "flce misaligned weight", LCE_ERR_ALIGNMENT);
  expect(flce_fwd_bwd(hidden, weight, bias, labels, 64, 64, 1000, -100, 16, -1, 64u, gout, lossp,
                      lse, gh, gw, gb, st, ws, big, nullptr), "flce bad flags", LCE_ERR_BAD_FLAGS);

  // timing interface
  const char* names[64];
  double ms[64];
  long long launches[64];
  int count = 0;
  lce_timing_enable(1);
  lce_timing_read(64, names, ms, launches, &count);
  lce_timing_read(0, nullptr, nullptr, nullptr, &count);
  lce_timing_enable(0);

  std::printf("%ld calls, %d failures\n", calls, failures);
  return failures ? 1 : 0;
}
