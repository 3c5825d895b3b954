// ceiling.h -- launchers of the measurement kernels (not part of the
// method): streams with the access pattern of the library's kernels, whose
// rates the kernels are compared with.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rbi {

// c[i] = a[i] ^ b[i] over n16 16-byte units: two reads for each write, the
// traffic mix of the backward (x and dy read, dx written).
hipError_t launch_stream_2r1w(const void* a, const void* b, void* c, int64_t n16, hipStream_t st);

}  // namespace rbi
