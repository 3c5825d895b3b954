// linear.h -- launchers of the linear-layer (det_gemm) kernels, internal to
// the library.  Shapes: x[rows][k], W[n][k], dY[rows][n]; n and k are
// multiples of 8; all tensors contiguous, 16-byte aligned.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rbi {
namespace lin {

// Logical rows per dW group (the split of the canonical order, GDO-v1).
constexpr int64_t kGroupRows = 16384;
// Largest number of groups the final tree takes (rows <= 64 * 16384).
constexpr int64_t kMaxGroups = 64;

// out[rows][n] (bf16) = sum over c < k of A[row][c] * B(c, n), A row-major
// [rows][k]; B(c, n) = b[n * ldb + c] (fwd: W) or b[c * ldb + n] (dX: W).
// Rows whose map value is -1 are not read and get 0.
struct RowwiseArgs {
  const uint16_t* a;
  int64_t lda;
  const uint16_t* b;
  int64_t ldb;
  int64_t rows;
  int64_t n;   // output columns
  int64_t k;   // contraction length
  const int32_t* row_logical;
  uint16_t* out;
};

// Group results Q[g][n][k] (fp32) of dW = dY^T X over T logical rows in
// logical order: row l of dY at dy + l * n, of X at x + l * k (the caller may
// shift both pointers so that a call's buffer is addressed by logical row).
// Groups g_first .. g_first + g_count - 1 are computed (g_count = 0: all).
struct DwArgs {
  const uint16_t* dy;
  const uint16_t* x;
  int64_t T;
  int64_t n;
  int64_t k;
  float* out;
  int64_t g_first = 0;
  int64_t g_count = 0;
};

hipError_t launch_rowwise(const RowwiseArgs& a, bool b_transposed, hipStream_t stream);
int64_t num_groups(int64_t T);
hipError_t launch_dw_groups(const DwArgs& a, hipStream_t stream);
hipError_t launch_group_tree(const float* q, int64_t G, int64_t nk, float* dw, hipStream_t stream);
// Copies the call's real rows to their logical positions, except rows of the
// groups whose bit is set in skip_groups (bit g: logical rows of group g).
hipError_t launch_stage_rows(const uint16_t* src, int64_t rows, int64_t cols,
                             const int32_t* row_logical, uint16_t* dst, hipStream_t stream,
                             uint64_t skip_groups = 0);
// The same for two tensors of one call at once (x[rows][ca] -> da, dY[rows][cb] -> db).
hipError_t launch_stage_rows2(const uint16_t* a, int64_t ca, uint16_t* da, const uint16_t* b,
                              int64_t cb, uint16_t* db, int64_t rows, const int32_t* row_logical,
                              hipStream_t stream, uint64_t skip_groups = 0);
hipError_t launch_zero(uint16_t* dst, int64_t n_elems, hipStream_t stream);
hipError_t launch_zero_f32(float* dst, int64_t n, hipStream_t stream);

}  // namespace lin
}  // namespace rbi
