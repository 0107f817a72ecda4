// HIP-side helpers: launch bracketing for kernel timing, XCD-aware block mapping.
#pragma once

#include <hip/hip_runtime.h>

#include "rc_internal.h"

namespace rc {

// Device error word registered through rc_set_error_word (nullptr = off).
int32_t* error_word();

// Times one launch with HIP events on `stream` while timing is enabled
// (and `timed`: calls that must allocate nothing pass false).
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t stream, bool timed = true);
  ~ProfScope();

 private:
  int idx_ = -1;
  hipStream_t stream_;
};

// Check the launch that just happened.
rc_status check_launch(const char* what);

}  // namespace rc

// MI355X dispatches workgroup p of a 1-D grid to XCD p % 8.  Remap so that each
// XCD receives a contiguous run of logical work indices: neighbouring work
// (tiles of the same request and kv head, member groups of one shared range)
// then shares that XCD's L2.
__device__ __forceinline__ int xcd_remap(int p, int n) {
  const int x = p & 7, i = p >> 3;
  const int per = n >> 3, rem = n & 7;
  return x * per + (x < rem ? x : rem) + i;
}
