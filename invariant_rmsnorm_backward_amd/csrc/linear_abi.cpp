// linear_abi.cpp -- the C-ABI of include/det_gemm_bi.h: argument checks,
// the canonical dW accumulator and kernel launches.  Every check runs on
// the host before anything is enqueued; there is no fallback path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/det_gemm_bi.h"
#include "abi_internal.h"
#include "linear.h"
#include "plan.h"

using rbi::abi::check_rows;
using rbi::abi::check_tensor;
using rbi::abi::fail;
using rbi::abi::hip_fail;
using rbi::abi::overlaps;

namespace {

constexpr int64_t kMaxFeatures = 1 << 16;

int check_features(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0) return fail(RMSNORM_EINVAL, "n and k must be positive");
  if (n % 8 != 0 || k % 8 != 0)
    return fail(RMSNORM_EUNSUPPORTED, "n and k must be multiples of 8 (16-byte bf16 vectors)");
  if (n > kMaxFeatures || k > kMaxFeatures)
    return fail(RMSNORM_EUNSUPPORTED, "n and k must be at most 65536");
  return RMSNORM_OK;
}

int check_layout(const rmsnorm_layout* layout, int64_t rows) {
  if (layout != nullptr && layout->host.rows != rows)
    return fail(RMSNORM_ELAYOUT, "layout rows (" + std::to_string(layout->host.rows) +
                                     ") differ from rows (" + std::to_string(rows) + ")");
  return RMSNORM_OK;
}

// Where a dW group's chain stands: computed at contrib time from the buffers
// of the one call that held the whole group in logical order, or staged (its
// rows copied to the logical-order staging area, the chain runs at finalize).
enum GroupState : uint8_t { kGroupNone = 0, kGroupComputed = 1, kGroupStaged = 2 };

// The groups a call holds whole, in logical order, as one run of physical
// rows: for such a group g, the physical row of logical row l is l + off[g].
struct DirectGroups {
  std::vector<int64_t> off;
  std::vector<uint8_t> whole;
};
DirectGroups direct_groups(const rbi::PlanHost& plan, int64_t T) {
  const int64_t G = rbi::lin::num_groups(T);
  DirectGroups d;
  d.off.assign(static_cast<size_t>(G), 0);
  d.whole.assign(static_cast<size_t>(G), 0);
  std::vector<int64_t> cnt(static_cast<size_t>(G), 0);
  std::vector<uint8_t> run(static_cast<size_t>(G), 1);
  for (int64_t p = 0; p < plan.rows; ++p) {
    const int64_t l = plan.row_logical[static_cast<size_t>(p)];
    if (l < 0) continue;
    const size_t g = static_cast<size_t>(l / rbi::lin::kGroupRows);
    if (cnt[g] == 0) d.off[g] = p - l;
    else if (p - l != d.off[g]) run[g] = 0;
    ++cnt[g];
  }
  for (int64_t g = 0; g < G; ++g) {
    const int64_t size = std::min(rbi::lin::kGroupRows, T - g * rbi::lin::kGroupRows);
    d.whole[static_cast<size_t>(g)] = run[static_cast<size_t>(g)] && cnt[static_cast<size_t>(g)] == size;
  }
  return d;
}

}  // namespace

struct det_gemm_dw_acc {
  rbi::AccHost host;
  int64_t n = 0, k = 0, groups = 0;
  float* d_q = nullptr;          // [groups][n][k]
  uint16_t* d_x = nullptr;       // [n_logical][k] staging, logical order
  uint16_t* d_dy = nullptr;      // [n_logical][n]
  std::vector<uint8_t> group_state;   // GroupState per group
};

extern "C" {

int det_gemm_fwd(const rmsnorm_bf16* x, const rmsnorm_bf16* w, rmsnorm_bf16* y, int64_t rows,
                 int64_t n, int64_t k, const rmsnorm_layout* layout, void* stream) {
  int rc;
  if ((rc = check_rows(rows)) || (rc = check_features(n, k)) || (rc = check_layout(layout, rows)))
    return rc;
  if (rows == 0) return RMSNORM_OK;
  if ((rc = check_tensor(x, "x", 16)) || (rc = check_tensor(w, "w", 16)) ||
      (rc = check_tensor(y, "y", 16)))
    return rc;
  if (overlaps(y, rows * n * 2, x, rows * k * 2) || overlaps(y, rows * n * 2, w, n * k * 2))
    return fail(RMSNORM_EINVAL, "y must not alias an input");
  rbi::lin::RowwiseArgs a{x, k, w, k, rows, n, k, layout ? layout->dev.row_logical : nullptr, y};
  hipError_t e = rbi::lin::launch_rowwise(a, false, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "det_gemm_fwd launch");
  return RMSNORM_OK;
}

int det_gemm_bwd_dx(const rmsnorm_bf16* dy, const rmsnorm_bf16* w, rmsnorm_bf16* dx,
                    int64_t rows, int64_t n, int64_t k, const rmsnorm_layout* layout,
                    void* stream) {
  int rc;
  if ((rc = check_rows(rows)) || (rc = check_features(n, k)) || (rc = check_layout(layout, rows)))
    return rc;
  if (rows == 0) return RMSNORM_OK;
  if ((rc = check_tensor(dy, "dy", 16)) || (rc = check_tensor(w, "w", 16)) ||
      (rc = check_tensor(dx, "dx", 16)))
    return rc;
  if (overlaps(dx, rows * k * 2, dy, rows * n * 2) || overlaps(dx, rows * k * 2, w, n * k * 2))
    return fail(RMSNORM_EINVAL, "dx must not alias an input");
  rbi::lin::RowwiseArgs a{dy, n, w, k, rows, k, n, layout ? layout->dev.row_logical : nullptr, dx};
  hipError_t e = rbi::lin::launch_rowwise(a, true, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "det_gemm_bwd_dx launch");
  return RMSNORM_OK;
}

int det_gemm_dw_acc_create(det_gemm_dw_acc** out, int64_t n_logical, int64_t n, int64_t k,
                           void* stream) {
  (void)stream;
  if (out == nullptr) return fail(RMSNORM_EINVAL, "out is NULL");
  *out = nullptr;
  int rc;
  if ((rc = check_features(n, k))) return rc;
  if (n_logical < 0) return fail(RMSNORM_EINVAL, "n_logical must be non-negative");
  if (rbi::lin::num_groups(n_logical) > rbi::lin::kMaxGroups)
    return fail(RMSNORM_EUNSUPPORTED, "n_logical must be at most " +
                                          std::to_string(rbi::lin::kMaxGroups * rbi::lin::kGroupRows));
  auto* A = new det_gemm_dw_acc();
  A->host.init(n_logical, k);
  A->n = n;
  A->k = k;
  A->groups = rbi::lin::num_groups(n_logical);
  A->group_state.assign(static_cast<size_t>(A->groups), kGroupNone);
  hipError_t e = hipSuccess;
  auto cleanup = [&](const char* what) {
    if (A->d_q) (void)hipFree(A->d_q);
    if (A->d_x) (void)hipFree(A->d_x);
    if (A->d_dy) (void)hipFree(A->d_dy);
    delete A;
    return hip_fail(e, what);
  };
  const size_t nq = std::max<int64_t>(1, A->groups) * static_cast<size_t>(n * k);
  if ((e = hipMalloc(&A->d_q, nq * sizeof(float))) != hipSuccess)
    return cleanup("group result allocation");
  if ((e = hipMalloc(&A->d_x, std::max<size_t>(8, n_logical * k) * 2)) != hipSuccess)
    return cleanup("staging allocation");
  if ((e = hipMalloc(&A->d_dy, std::max<size_t>(8, n_logical * n) * 2)) != hipSuccess)
    return cleanup("staging allocation");
  *out = A;
  return RMSNORM_OK;
}

int det_gemm_dw_contrib(const rmsnorm_bf16* x, const rmsnorm_bf16* dy, int64_t rows, int64_t n,
                        int64_t k, const rmsnorm_layout* layout, det_gemm_dw_acc* acc,
                        void* stream) {
  if (acc == nullptr) return fail(RMSNORM_EINVAL, "accumulator is NULL");
  int rc;
  if ((rc = check_rows(rows)) || (rc = check_features(n, k)) || (rc = check_layout(layout, rows)))
    return rc;
  if (n != acc->n || k != acc->k)
    return fail(RMSNORM_EINVAL, "n, k differ from the accumulator's");
  if (acc->host.finalized)
    return fail(RMSNORM_ESTATE, "accumulator already finalized; call det_gemm_dw_acc_reset first");
  if (rows > 0 && ((rc = check_tensor(x, "x", 16)) || (rc = check_tensor(dy, "dy", 16)))) return rc;
  std::string err;
  const rbi::PlanHost* plan_host = layout ? &layout->host : nullptr;
  rc = acc->host.check_call(plan_host, rows, &err);
  if (rc != RMSNORM_OK) return fail(rc, err);
  if (rows == 0) {
    acc->host.commit_call(plan_host);
    return RMSNORM_OK;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  const int64_t T = acc->host.n_logical;
  if (layout == nullptr) {
    // every row, in logical order: every group's chain runs now
    rbi::lin::DwArgs a{dy, x, T, n, k, acc->d_q};
    if ((e = rbi::lin::launch_dw_groups(a, st)) != hipSuccess) return hip_fail(e, "dW groups");
    acc->host.commit_call(plan_host);
    std::fill(acc->group_state.begin(), acc->group_state.end(), kGroupComputed);
    return RMSNORM_OK;
  }
  // Groups this call holds whole and in order run their chains now, from the
  // call's own buffers (addressed by logical row); the rows of every other
  // group are staged for the finalize.
  const DirectGroups dg = direct_groups(layout->host, T);
  uint64_t direct_mask = 0;
  bool any_staged = false;
  for (int64_t g = 0; g < acc->groups; ++g) {
    if (dg.whole[static_cast<size_t>(g)]) {
      const int64_t off = dg.off[static_cast<size_t>(g)];
      rbi::lin::DwArgs a{dy + off * n, x + off * k, T, n, k, acc->d_q, g, 1};
      if ((e = rbi::lin::launch_dw_groups(a, st)) != hipSuccess) return hip_fail(e, "dW group");
      direct_mask |= uint64_t(1) << g;
    } else {
      any_staged = true;
    }
  }
  if (any_staged &&
      (e = rbi::lin::launch_stage_rows2(x, k, acc->d_x, dy, n, acc->d_dy, rows,
                                        layout->dev.row_logical, st, direct_mask)) != hipSuccess)
    return hip_fail(e, "dW staging");
  acc->host.commit_call(plan_host);
  // a group touched by this call is either whole here (computed) or split
  // across calls (staged: all of its rows arrive through the staging copy)
  std::vector<uint8_t> touched(static_cast<size_t>(acc->groups), 0);
  for (int32_t l : layout->host.row_logical)
    if (l >= 0) touched[static_cast<size_t>(l / rbi::lin::kGroupRows)] = 1;
  for (int64_t g = 0; g < acc->groups; ++g) {
    if (!touched[static_cast<size_t>(g)]) continue;
    acc->group_state[static_cast<size_t>(g)] =
        (direct_mask >> g) & 1u ? kGroupComputed : kGroupStaged;
  }
  return RMSNORM_OK;
}

int det_gemm_dw_finalize(det_gemm_dw_acc* acc, float* dw, void* stream) {
  if (acc == nullptr) return fail(RMSNORM_EINVAL, "accumulator is NULL");
  int rc;
  if ((rc = check_tensor(dw, "dw", 4))) return rc;
  std::vector<int32_t> spilled;
  std::string err;
  rc = acc->host.prepare_finalize(&spilled, &err);
  if (rc != RMSNORM_OK) return fail(rc, err);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  const int64_t T = acc->host.n_logical, nk = acc->n * acc->k;
  if (T == 0) {
    if ((e = rbi::lin::launch_zero_f32(dw, nk, st)) != hipSuccess) return hip_fail(e, "dW zero fill");
    acc->host.finalized = true;
    return RMSNORM_OK;
  }
  // the chains of staged groups, one launch per run of consecutive ones
  for (int64_t g = 0; g < acc->groups;) {
    if (acc->group_state[static_cast<size_t>(g)] != kGroupStaged) {
      ++g;
      continue;
    }
    int64_t g1 = g;
    while (g1 < acc->groups && acc->group_state[static_cast<size_t>(g1)] == kGroupStaged) ++g1;
    rbi::lin::DwArgs a{acc->d_dy, acc->d_x, T, acc->n, acc->k, acc->d_q, g, g1 - g};
    if ((e = rbi::lin::launch_dw_groups(a, st)) != hipSuccess) return hip_fail(e, "dW groups");
    g = g1;
  }
  if ((e = rbi::lin::launch_group_tree(acc->d_q, acc->groups, nk, dw, st)) != hipSuccess)
    return hip_fail(e, "dW group tree");
  acc->host.finalized = true;
  return RMSNORM_OK;
}

int det_gemm_dw_acc_reset(det_gemm_dw_acc* acc, void* stream) {
  (void)stream;
  if (acc == nullptr) return fail(RMSNORM_EINVAL, "accumulator is NULL");
  acc->host.reset();
  std::fill(acc->group_state.begin(), acc->group_state.end(), kGroupNone);
  return RMSNORM_OK;
}

int det_gemm_dw_acc_destroy(det_gemm_dw_acc* acc) {
  if (acc == nullptr) return RMSNORM_OK;
  hipError_t e = hipDeviceSynchronize();
  (void)hipFree(acc->d_q);
  (void)hipFree(acc->d_x);
  (void)hipFree(acc->d_dy);
  delete acc;
  if (e != hipSuccess) return hip_fail(e, "accumulator destroy");
  return RMSNORM_OK;
}

}  // extern "C"
