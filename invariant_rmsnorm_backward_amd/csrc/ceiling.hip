// ceiling.hip -- a two-reads-one-write stream at the practical HBM rate of
// the GPU, the ceiling the backward's traffic (x and dy read, dx written) is
// compared with.  Not part of the method.
#include "ceiling.h"

namespace rbi {
namespace {

typedef unsigned int u32x4c_t __attribute__((ext_vector_type(4)));

// Four 16-byte units of each input per thread per pass (grid stride), loaded
// and stored non-temporally: the most bytes in flight per lane that measured
// fastest for this mix on MI355X (4 or 8 KB per workgroup, 16,384 workgroups).
constexpr int kUnroll = 4;

__global__ __launch_bounds__(256) void stream_2r1w_kernel(const u32x4c_t* __restrict__ a,
                                                          const u32x4c_t* __restrict__ b,
                                                          u32x4c_t* __restrict__ c, int64_t n16) {
  const int64_t step = (int64_t)gridDim.x * 256 * kUnroll;
  for (int64_t i = (int64_t)blockIdx.x * 256 * kUnroll + threadIdx.x; i < n16; i += step) {
    u32x4c_t va[kUnroll], vb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = i + 256 * u;
      if (j < n16) {
        va[u] = __builtin_nontemporal_load(a + j);
        vb[u] = __builtin_nontemporal_load(b + j);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = i + 256 * u;
      if (j < n16) __builtin_nontemporal_store(va[u] ^ vb[u], c + j);
    }
  }
}

}  // namespace

hipError_t launch_stream_2r1w(const void* a, const void* b, void* c, int64_t n16, hipStream_t st) {
  if (n16 <= 0) return hipSuccess;
  int64_t g = (n16 + 256 * kUnroll - 1) / (256 * kUnroll);
  if (g > 16384) g = 16384;
  stream_2r1w_kernel<<<dim3((unsigned)g), dim3(256), 0, st>>>(static_cast<const u32x4c_t*>(a),
                                                               static_cast<const u32x4c_t*>(b),
                                                               static_cast<u32x4c_t*>(c), n16);
  return hipGetLastError();
}

}  // namespace rbi
