// Host-side bounds checks of the launchers, compiled in with -DLGS_DEBUG
// (liblgs_debug.so); in the product build every hook below is an empty
// inline function.
//
// Each entry point registers the device spans it validated (every matrix as
// ((rows - 1) * ld + width) elements, the per-token arrays, the workspace).
// Before every kernel launch the launcher computes, from the launch's own
// sizes, every span that kernel reads or writes and asserts that each lies
// inside one registered span; a failed check prints the span and aborts.
// Registered spans are thread-local and dropped when the entry point
// returns.  A dry-run switch skips every HIP call (launches, error queries,
// the static scratch's lookup) so that the checks can run without a GPU.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lgs {
namespace debug {

#ifdef LGS_DEBUG
void allow(const void* p, size_t bytes);
void need(const void* p, size_t bytes, const char* what, const char* file, int line);
void check(bool ok, const char* what, const char* file, int line);
void end_call();
bool dry_run();
#else
inline void allow(const void*, size_t) {}
inline void need(const void*, size_t, const char*, const char*, int) {}
inline void check(bool, const char*, const char*, int) {}
inline void end_call() {}
inline bool dry_run() { return false; }
#endif

// Bytes spanned by `rows` rows of `width` elements of `esz` bytes, ld apart.
inline size_t mat_bytes(int64_t rows, int64_t ld, int64_t width, size_t esz) {
  return rows > 0 && width > 0 ? (size_t)((rows - 1) * ld + width) * esz : 0;
}

}  // namespace debug
}  // namespace lgs

#define LGS_NEED(p, bytes, what) ::lgs::debug::need((p), (bytes), (what), __FILE__, __LINE__)
#define LGS_CHECK(cond) ::lgs::debug::check((cond), #cond, __FILE__, __LINE__)

// A kernel launch that a dry run skips, and the launch status it then reports.
#define LGS_LAUNCH(kernel, grid, block, shmem, stream, ...)                         \
  do {                                                                              \
    if (!::lgs::debug::dry_run())                                                   \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);           \
  } while (0)
#define LGS_LAUNCH_STATUS() (::lgs::debug::dry_run() ? hipSuccess : hipGetLastError())
