// The host-side bounds checks of debug builds (debug.hpp), and the testing
// entry points that drive them (include/lgs_testing.h).  In the product build
// only the testing entry points remain, reporting that checks are off.
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <utility>
#include <vector>

#include "debug.hpp"
#include "lgs_testing.h"

#define LGS_API extern "C" __attribute__((visibility("default")))

namespace {
std::atomic<long> g_checks{0};
std::atomic<int> g_dry_run{0};
}  // namespace

#ifdef LGS_DEBUG
namespace lgs {
namespace debug {

namespace {
thread_local std::vector<std::pair<uintptr_t, size_t>> t_spans;
}

void allow(const void* p, size_t bytes) {
  if (p && bytes) t_spans.emplace_back((uintptr_t)p, bytes);
}

void need(const void* p, size_t bytes, const char* what, const char* file, int line) {
  g_checks.fetch_add(1, std::memory_order_relaxed);
  if (!bytes) return;
  const uintptr_t a = (uintptr_t)p;
  for (const auto& s : t_spans)
    if (a >= s.first && a - s.first <= s.second && bytes <= s.second - (a - s.first)) return;
  fprintf(stderr, "lgs debug: %s:%d: %s spans [%#llx, +%zu), outside every validated buffer of the call:\n",
          file, line, what, (unsigned long long)a, bytes);
  for (const auto& s : t_spans)
    fprintf(stderr, "  [%#llx, +%zu)\n", (unsigned long long)s.first, s.second);
  abort();
}

void check(bool ok, const char* what, const char* file, int line) {
  g_checks.fetch_add(1, std::memory_order_relaxed);
  if (ok) return;
  fprintf(stderr, "lgs debug: %s:%d: check failed: %s\n", file, line, what);
  abort();
}

void end_call() { t_spans.clear(); }

bool dry_run() { return g_dry_run.load(std::memory_order_relaxed) != 0; }

}  // namespace debug
}  // namespace lgs
#endif

LGS_API int lgs_test_debug_build(void) {
#ifdef LGS_DEBUG
  return 1;
#else
  return 0;
#endif
}

LGS_API int lgs_test_set_dry_run(int on) {
#ifdef LGS_DEBUG
  g_dry_run.store(on ? 1 : 0);
  return 0;
#else
  (void)on;
  return -1;
#endif
}

LGS_API long lgs_test_debug_checks(void) { return g_checks.load(); }

LGS_API int lgs_test_debug_span(const void* allowed, size_t allowed_bytes, const void* p, size_t bytes) {
#ifdef LGS_DEBUG
  lgs::debug::allow(allowed, allowed_bytes);
  LGS_NEED(p, bytes, "lgs_test_debug_span");
  lgs::debug::end_call();
  return 0;
#else
  (void)allowed, (void)allowed_bytes, (void)p, (void)bytes;
  return -1;
#endif
}
