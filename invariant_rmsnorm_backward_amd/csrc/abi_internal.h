// abi_internal.h -- pieces shared by the C-ABI translation units: the
// per-thread error message, argument checks and the opaque layout type.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "../../include/rmsnorm_bi.h"
#include "kernels.h"
#include "plan.h"

namespace rbi {
namespace abi {

std::string& last_error();   // message of the last error on the calling thread

inline int fail(int code, const std::string& msg) {
  last_error() = msg;
  return code;
}

inline int hip_fail(hipError_t e, const char* what) {
  return fail(RMSNORM_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

inline int check_rows(int64_t rows) {
  if (rows < 0) return fail(RMSNORM_EINVAL, "rows must be non-negative");
  if (rows > INT32_MAX) return fail(RMSNORM_EUNSUPPORTED, "rows must be below 2^31");
  return RMSNORM_OK;
}

inline int check_tensor(const void* p, const char* name, size_t align) {
  if (p == nullptr) return fail(RMSNORM_EINVAL, std::string(name) + " is NULL");
  if (!aligned(p, align))
    return fail(RMSNORM_EUNSUPPORTED,
                std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
  return RMSNORM_OK;
}

}  // namespace abi
}  // namespace rbi

struct rmsnorm_layout {
  rbi::PlanHost host;
  void* d_mem = nullptr;
  rbi::PlanDev dev;
};
