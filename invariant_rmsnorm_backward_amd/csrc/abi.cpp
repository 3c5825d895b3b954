// abi.cpp -- the C-ABI of include/rmsnorm_bi.h: argument checks, layouts,
// accumulators and kernel launches.  Every check runs on the host before
// anything is enqueued; there is no fallback path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/rmsnorm_bi.h"
#include "abi_internal.h"
#include "ceiling.h"
#include "kernels.h"
#include "plan.h"

namespace rbi {
namespace abi {
std::string& last_error() {
  thread_local std::string err;
  return err;
}
}  // namespace abi
}  // namespace rbi

namespace {

using rbi::abi::check_rows;
using rbi::abi::check_tensor;
using rbi::abi::fail;
using rbi::abi::hip_fail;
using rbi::abi::overlaps;

int check_hidden(int64_t hidden) {
  if (hidden <= 0) return fail(RMSNORM_EINVAL, "hidden must be positive");
  if (hidden % 8 != 0)
    return fail(RMSNORM_EUNSUPPORTED, "hidden must be a multiple of 8 (16-byte bf16 vectors)");
  if (hidden > rbi::kMaxHidden)
    return fail(RMSNORM_EUNSUPPORTED,
                "hidden " + std::to_string(hidden) + " exceeds the maximum " +
                    std::to_string(rbi::kMaxHidden));
  return RMSNORM_OK;
}

}  // namespace

// Device scratch of rmsnorm_bwd_noalloc: the block partials of one call and
// the partial levels of its block tree.  Every GPU the library runs on holds
// its own copy of the array until the process ends; host code reaches it only
// through the address hipGetSymbolAddress gives for the current device.
constexpr int64_t kNoAllocScratchFloats = int64_t(16) << 20;   // 64 MiB
static __device__ __align__(256) float scratch[kNoAllocScratchFloats];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_addr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
int scratch_of_current_device(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RMSNORM_EUNSUPPORTED, "device index " + std::to_string(dev) + " is above 63");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "address of the device scratch");
    g_scratch_addr[dev] = static_cast<float*>(addr);
  }
  *out = g_scratch_addr[dev];
  return RMSNORM_OK;
}

}  // namespace

struct rmsnorm_dw_acc {
  rbi::AccHost host;
  float* d_P = nullptr;
  float* d_S = nullptr;
  float* d_tmp = nullptr;
  float* d_Q = nullptr;           // stream sums q1..q3 of blocks in stream form
  int32_t* d_form = nullptr;      // per block: 1 = in stream form
  bool stream_form = false;       // some call since reset took the stream-owner path
  int32_t* d_spilled = nullptr;
  int32_t* h_spilled = nullptr;   // pinned staging for the spilled-block list
  hipEvent_t staged = nullptr;
  bool staging_pending = false;
};

extern "C" {

int rmsnorm_max_hidden(void) { return rbi::kMaxHidden; }

const char* rmsnorm_last_error(void) { return rbi::abi::last_error().c_str(); }

const char* rmsnorm_backend_info(void) {
  return "hip gfx950; cdo=v2 R=64 S=4, "
         "contribution fl32(fl32(dy*x)*rstd), streams fold ascending from +0.0, "
         "stream tree pairwise, block tree pairwise with +0.0 padding; "
         "row sums (x*x, dy*x*w): fmaf chain per 16-byte chunk, one wavefront sum per "
         "64-chunk group, pairwise tree over the groups with +0.0 padding; no atomics; "
         "fwd=rows_per_workgroup|lanes_per_row; bwd=fused dx+dW by resident block-owning "
         "workgroups, two or four rows in flight, next rows prefetched across blocks "
         "(calls with a few dozen blocks: one workgroup per fold stream; with fewer: "
         "row-parallel dx + 256-column dW units on one XCD per block), nt loads/stores; "
         "max_hidden=10240";
}

int rmsnorm_set_split_threshold(int64_t blocks, int64_t* previous) {
  if (previous != nullptr) *previous = rbi::split_items();
  rbi::set_split_items(blocks);
  return RMSNORM_OK;
}

int rmsnorm_set_stream_threshold(int64_t blocks, int64_t* previous) {
  if (previous != nullptr) *previous = rbi::stream_items();
  rbi::set_stream_items(blocks);
  return RMSNORM_OK;
}

int rmsnorm_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0) return fail(RMSNORM_EINVAL, "bytes must be non-negative");
  if (bytes == 0) return RMSNORM_OK;
  if (src == nullptr || dst == nullptr) return fail(RMSNORM_EINVAL, "src and dst must be non-NULL");
  if (bytes % 16 != 0) return fail(RMSNORM_EUNSUPPORTED, "bytes must be a multiple of 16");
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return fail(RMSNORM_EUNSUPPORTED, "src and dst must be 16-byte aligned");
  if (overlaps(src, static_cast<size_t>(bytes), dst, static_cast<size_t>(bytes)))
    return fail(RMSNORM_EINVAL, "src and dst must not overlap");
  const hipError_t e = rbi::launch_stream_copy(src, dst, bytes / 16, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream copy launch");
  return RMSNORM_OK;
}

int rmsnorm_stream_2r1w(const void* a, const void* b, void* c, int64_t bytes, void* stream) {
  if (bytes < 0) return fail(RMSNORM_EINVAL, "bytes must be non-negative");
  if (bytes == 0) return RMSNORM_OK;
  if (a == nullptr || b == nullptr || c == nullptr) return fail(RMSNORM_EINVAL, "a, b and c must be non-NULL");
  if (bytes % 16 != 0) return fail(RMSNORM_EUNSUPPORTED, "bytes must be a multiple of 16");
  if (reinterpret_cast<uintptr_t>(a) % 16 != 0 || reinterpret_cast<uintptr_t>(b) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(c) % 16 != 0)
    return fail(RMSNORM_EUNSUPPORTED, "a, b and c must be 16-byte aligned");
  const size_t n = static_cast<size_t>(bytes);
  if (overlaps(a, n, c, n) || overlaps(b, n, c, n)) return fail(RMSNORM_EINVAL, "c must not overlap a or b");
  const hipError_t e = rbi::launch_stream_2r1w(a, b, c, bytes / 16, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "two-read stream launch");
  return RMSNORM_OK;
}

int rmsnorm_set_workgroup_cap(int64_t groups, int64_t* previous) {
  if (previous != nullptr) *previous = rbi::wide_group_cap();
  rbi::set_wide_group_cap(groups);
  return RMSNORM_OK;
}

// Checks one forward call and fills *out; *launch is false when there is
// nothing to enqueue (rows == 0).
static int fwd_prepare(const rmsnorm_bf16* x, const rmsnorm_bf16* w, rmsnorm_bf16* y, float* rstd,
                       int64_t rows, int64_t hidden, float eps, const rmsnorm_layout* layout,
                       const rbi::RowPacking& pk, int64_t extent, rbi::FwdArgs* out, bool* launch) {
  int rc;
  *launch = false;
  if ((rc = check_rows(rows)) || (rc = check_hidden(hidden))) return rc;
  if (!(eps >= 0.0f) || std::isinf(eps)) return fail(RMSNORM_EINVAL, "eps must be finite and >= 0");
  if (layout != nullptr && layout->host.rows != rows)
    return fail(RMSNORM_ELAYOUT, "layout rows (" + std::to_string(layout->host.rows) +
                                     ") differ from rows (" + std::to_string(rows) + ")");
  if (rows == 0) return RMSNORM_OK;
  if ((rc = check_tensor(x, "x", 16)) || (rc = check_tensor(w, "w", 16)) ||
      (rc = check_tensor(y, "y", 16)))
    return rc;
  if (rstd != nullptr && (rc = check_tensor(rstd, "rstd", 4))) return rc;   // NULL: not saved
  const size_t nbytes = static_cast<size_t>(extent) * 2;
  if (overlaps(y, nbytes, x, nbytes) || overlaps(y, nbytes, w, hidden * 2) ||
      (rstd != nullptr && (overlaps(rstd, rows * 4, x, nbytes) || overlaps(rstd, rows * 4, y, nbytes))))
    return fail(RMSNORM_EINVAL, "outputs must not alias inputs or each other");
  // The forward is row-local: the map matters only for padding rows (not
  // read, written as 0).  A layout without padding rows runs as the identity,
  // so no row waits for its map entry before its loads.
  const bool pads = layout != nullptr && !layout->host.pad_rows.empty();
  *out = rbi::FwdArgs{x, w, y, rstd, rows, static_cast<int32_t>(hidden), eps,
                      pads ? layout->dev.row_logical : nullptr, pk};
  *launch = true;
  return RMSNORM_OK;
}

static int fwd_common(const rmsnorm_bf16* x, const rmsnorm_bf16* w, rmsnorm_bf16* y, float* rstd,
                      int64_t rows, int64_t hidden, float eps, const rmsnorm_layout* layout,
                      void* stream, const rbi::RowPacking& pk, int64_t extent) {
  rbi::FwdArgs a{};
  bool launch = false;
  int rc = fwd_prepare(x, w, y, rstd, rows, hidden, eps, layout, pk, extent, &a, &launch);
  if (rc != RMSNORM_OK || !launch) return rc;
  hipError_t e = rbi::launch_fwd(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rmsnorm_fwd launch");
  return RMSNORM_OK;
}

// Packed rows: tokens x heads rows of head_dim values, row (t, h) at
// t * token_stride + h * head_dim.  Returns the element extent through *extent.
static int check_packing(int64_t tokens, int64_t heads, int64_t head_dim, int64_t token_stride,
                         rbi::RowPacking* pk, int64_t* rows, int64_t* extent) {
  if (tokens < 0 || heads <= 0) return fail(RMSNORM_EINVAL, "tokens must be >= 0 and heads > 0");
  if (heads > INT32_MAX) return fail(RMSNORM_EUNSUPPORTED, "too many heads");
  if (!rbi::packed_hidden_supported(static_cast<int>(std::min<int64_t>(head_dim, 1 << 20))))
    return fail(RMSNORM_EUNSUPPORTED, "packed rows need head_dim in {8, 16, 32, 64, 128, 256}");
  if (token_stride % 8 != 0 || token_stride < heads * head_dim)
    return fail(RMSNORM_EINVAL, "token_stride must be a multiple of 8 and >= heads * head_dim");
  if (tokens > INT32_MAX / heads) return fail(RMSNORM_EUNSUPPORTED, "rows must be below 2^31");
  pk->heads = static_cast<int32_t>(heads);
  pk->token_stride = token_stride;
  *rows = tokens * heads;
  *extent = tokens == 0 ? 0 : (tokens - 1) * token_stride + heads * head_dim;
  return RMSNORM_OK;
}

// One backward call, checked and turned into kernel arguments; nothing is
// recorded in the accumulator until bwd_commit (after the launch).
struct BwdCall {
  rbi::BwdArgs a{};
  const rbi::PlanHost* plan_host = nullptr;
  rmsnorm_dw_acc* acc = nullptr;
  bool launch = false;   // rows > 0
  bool with_dx = true;
  bool recompute = false;
};

// recompute: rstd is not read (NULL) but rebuilt from x with eps.
static int bwd_prepare(const rmsnorm_bf16* x, const rmsnorm_bf16* w, const rmsnorm_bf16* dy,
                       const float* rstd, rmsnorm_bf16* dx, int64_t rows, int64_t hidden,
                       const rmsnorm_layout* layout, rmsnorm_dw_acc* acc, bool with_dx,
                       const rbi::RowPacking& pk, int64_t extent, bool recompute, float eps,
                       BwdCall* c) {
  int rc;
  if ((rc = check_rows(rows)) || (rc = check_hidden(hidden))) return rc;
  if (recompute && (!(eps >= 0.0f) || std::isinf(eps)))
    return fail(RMSNORM_EINVAL, "eps must be finite and >= 0");
  if (layout != nullptr && layout->host.rows != rows)
    return fail(RMSNORM_ELAYOUT, "layout rows (" + std::to_string(layout->host.rows) +
                                     ") differ from rows (" + std::to_string(rows) + ")");
  if (acc != nullptr) {
    if (acc->host.hidden != hidden)
      return fail(RMSNORM_EINVAL, "accumulator hidden (" + std::to_string(acc->host.hidden) +
                                      ") differs from hidden (" + std::to_string(hidden) + ")");
    if (acc->host.finalized)
      return fail(RMSNORM_ESTATE, "accumulator already finalized; call rmsnorm_dw_acc_reset first");
  }
  if (rows > 0) {
    if ((rc = check_tensor(x, "x", 16)) || (rc = check_tensor(dy, "dy", 16))) return rc;
    if (!recompute && (rc = check_tensor(rstd, "rstd", 4))) return rc;
    if (with_dx) {
      if ((rc = check_tensor(w, "w", 16)) || (rc = check_tensor(dx, "dx", 16))) return rc;
      const size_t nbytes = static_cast<size_t>(extent) * 2;
      if (overlaps(dx, nbytes, x, nbytes) || overlaps(dx, nbytes, dy, nbytes) ||
          overlaps(dx, nbytes, w, hidden * 2) ||
          (!recompute && overlaps(dx, nbytes, rstd, rows * 4)))
        return fail(RMSNORM_EINVAL, "dx must not alias an input");
    }
  }
  c->plan_host = layout ? &layout->host : nullptr;
  c->acc = acc;
  c->with_dx = with_dx;
  c->recompute = recompute;
  rbi::SpillTable spill;
  if (acc != nullptr) {
    std::string err;
    rc = acc->host.check_call(c->plan_host, rows, &err, &spill);
    if (rc != RMSNORM_OK) return fail(rc, err);
  }
  c->launch = rows > 0;
  rbi::BwdArgs& a = c->a;
  a.x = x;
  a.w = w;
  a.dy = dy;
  a.rstd = recompute ? nullptr : rstd;
  a.eps = eps;
  a.dx = with_dx ? dx : nullptr;
  a.P = acc ? acc->d_P : nullptr;
  a.S = acc ? acc->d_S : nullptr;
  a.Q = acc ? acc->d_Q : nullptr;
  a.form = acc ? acc->d_form : nullptr;
  a.spill = spill;
  a.rows = rows;
  a.hidden = static_cast<int32_t>(hidden);
  a.pack = pk;
  // A call whose rows are whole canonical blocks in logical order (no padding,
  // the first row on a block boundary, every block held completely: a B=1
  // sample or a chunked-prefill piece that starts on a block boundary) is the
  // identity map on blocks first/64 onwards: it runs the kernels without a
  // plan (no per-block lookups before the loads), with the block outputs
  // addressed from that block.  Same rows, same operations, same bits.
  const rbi::PlanHost* ph = layout ? &layout->host : nullptr;
  const bool whole_blocks = ph != nullptr && ph->contig_first >= 0 &&
                            ph->contig_first % rbi::kBlockRows == 0 && ph->n_partial == 0;
  if (layout != nullptr && !whole_blocks) {
    a.plan = layout->dev;
  } else {
    a.plan.n_items = static_cast<int32_t>(rbi::num_blocks(rows));
    a.plan.n_pad = 0;
    if (whole_blocks) {
      const int64_t b0 = ph->contig_first / rbi::kBlockRows;
      if (a.P != nullptr) a.P += b0 * hidden;
      if (a.Q != nullptr) a.Q += b0 * 3 * hidden;
      if (a.form != nullptr) a.form += b0;
    }
  }
  return RMSNORM_OK;
}

// The rows count as contributed only once their kernels are enqueued.
static void bwd_commit(const BwdCall& c) {
  if (c.acc == nullptr) return;
  c.acc->host.commit_call(c.plan_host);
  if (c.launch && rbi::bwd_path(c.a, c.with_dx, true, c.recompute) == rbi::BwdPath::kStream)
    c.acc->stream_form = true;
}

static int bwd_common(const rmsnorm_bf16* x, const rmsnorm_bf16* w, const rmsnorm_bf16* dy,
                      const float* rstd, rmsnorm_bf16* dx, int64_t rows, int64_t hidden,
                      const rmsnorm_layout* layout, rmsnorm_dw_acc* acc, void* stream,
                      bool with_dx, const rbi::RowPacking& pk, int64_t extent,
                      bool recompute = false, float eps = 0.0f) {
  BwdCall c;
  int rc = bwd_prepare(x, w, dy, rstd, dx, rows, hidden, layout, acc, with_dx, pk, extent,
                       recompute, eps, &c);
  if (rc != RMSNORM_OK) return rc;
  if (c.launch) {
    hipError_t e = rbi::launch_bwd(c.a, with_dx, acc != nullptr,
                                   reinterpret_cast<hipStream_t>(stream), recompute);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm backward launch");
  }
  bwd_commit(c);
  return RMSNORM_OK;
}

// Two packed norms in one launch: the per-token column windows of two
// outputs may interleave (Q and K heads of one tensor) but must not share
// an element.
static bool windows_disjoint(const void* a, int64_t cols_a, int64_t stride_a, int64_t extent_a,
                             const void* b, int64_t cols_b, int64_t stride_b, int64_t extent_b) {
  if (extent_a == 0 || extent_b == 0) return true;
  if (!overlaps(a, static_cast<size_t>(extent_a) * 2, b, static_cast<size_t>(extent_b) * 2))
    return true;
  if (stride_a != stride_b) return false;
  const int64_t d = (reinterpret_cast<intptr_t>(b) - reinterpret_cast<intptr_t>(a)) / 2;
  if (d >= 0) return d >= cols_a && d + cols_b <= stride_a;
  return -d >= cols_b && -d + cols_a <= stride_a;
}

int rmsnorm_fwd(const rmsnorm_bf16* x, const rmsnorm_bf16* w, rmsnorm_bf16* y, float* rstd,
                int64_t rows, int64_t hidden, float eps, const rmsnorm_layout* layout,
                void* stream) {
  return fwd_common(x, w, y, rstd, rows, hidden, eps, layout, stream, rbi::RowPacking{},
                    rows * hidden);
}

int rmsnorm_fwd_packed(const rmsnorm_bf16* x, const rmsnorm_bf16* w, rmsnorm_bf16* y,
                       float* rstd, int64_t tokens, int64_t heads, int64_t head_dim,
                       int64_t token_stride, float eps, const rmsnorm_layout* layout,
                       void* stream) {
  rbi::RowPacking pk;
  int64_t rows = 0, extent = 0;
  int rc = check_packing(tokens, heads, head_dim, token_stride, &pk, &rows, &extent);
  if (rc != RMSNORM_OK) return rc;
  return fwd_common(x, w, y, rstd, rows, head_dim, eps, layout, stream, pk, extent);
}

int rmsnorm_bwd_dx(const rmsnorm_bf16* x, const rmsnorm_bf16* w, const rmsnorm_bf16* dy,
                   const float* rstd, rmsnorm_bf16* dx, int64_t rows, int64_t hidden,
                   const rmsnorm_layout* layout, rmsnorm_dw_acc* acc, void* stream) {
  return bwd_common(x, w, dy, rstd, dx, rows, hidden, layout, acc, stream, true,
                    rbi::RowPacking{}, rows * hidden);
}

int rmsnorm_bwd_dx_recompute(const rmsnorm_bf16* x, const rmsnorm_bf16* w, const rmsnorm_bf16* dy,
                             float eps, rmsnorm_bf16* dx, int64_t rows, int64_t hidden,
                             const rmsnorm_layout* layout, rmsnorm_dw_acc* acc, void* stream) {
  return bwd_common(x, w, dy, nullptr, dx, rows, hidden, layout, acc, stream, true,
                    rbi::RowPacking{}, rows * hidden, true, eps);
}

int rmsnorm_bwd_dx_packed(const rmsnorm_bf16* x, const rmsnorm_bf16* w, const rmsnorm_bf16* dy,
                          const float* rstd, rmsnorm_bf16* dx, int64_t tokens, int64_t heads,
                          int64_t head_dim, int64_t token_stride, const rmsnorm_layout* layout,
                          rmsnorm_dw_acc* acc, void* stream) {
  rbi::RowPacking pk;
  int64_t rows = 0, extent = 0;
  int rc = check_packing(tokens, heads, head_dim, token_stride, &pk, &rows, &extent);
  if (rc != RMSNORM_OK) return rc;
  return bwd_common(x, w, dy, rstd, dx, rows, head_dim, layout, acc, stream, true, pk, extent);
}

int rmsnorm_fwd_packed_pair(const rmsnorm_bf16* x_a, const rmsnorm_bf16* w_a, rmsnorm_bf16* y_a,
                            float* rstd_a, int64_t heads_a, int64_t token_stride_a,
                            const rmsnorm_layout* layout_a, const rmsnorm_bf16* x_b,
                            const rmsnorm_bf16* w_b, rmsnorm_bf16* y_b, float* rstd_b,
                            int64_t heads_b, int64_t token_stride_b,
                            const rmsnorm_layout* layout_b, int64_t tokens, int64_t head_dim,
                            float eps, void* stream) {
  rbi::RowPacking pa, pb;
  int64_t rows_a = 0, rows_b = 0, ext_a = 0, ext_b = 0;
  int rc;
  if ((rc = check_packing(tokens, heads_a, head_dim, token_stride_a, &pa, &rows_a, &ext_a)) ||
      (rc = check_packing(tokens, heads_b, head_dim, token_stride_b, &pb, &rows_b, &ext_b)))
    return rc;
  rbi::FwdArgs a{}, b{};
  bool la = false, lb = false;
  if ((rc = fwd_prepare(x_a, w_a, y_a, rstd_a, rows_a, head_dim, eps, layout_a, pa, ext_a, &a, &la)) ||
      (rc = fwd_prepare(x_b, w_b, y_b, rstd_b, rows_b, head_dim, eps, layout_b, pb, ext_b, &b, &lb)))
    return rc;
  if (!la) return RMSNORM_OK;   // tokens == 0
  const size_t ea = static_cast<size_t>(ext_a) * 2, eb = static_cast<size_t>(ext_b) * 2;
  // each norm's outputs against the other norm's inputs and outputs
  if (overlaps(y_a, ea, x_b, eb) || overlaps(y_b, eb, x_a, ea) ||
      overlaps(y_a, ea, w_b, head_dim * 2) || overlaps(y_b, eb, w_a, head_dim * 2) ||
      !windows_disjoint(y_a, heads_a * head_dim, token_stride_a, ext_a, y_b, heads_b * head_dim,
                        token_stride_b, ext_b) ||
      (rstd_a != nullptr && (overlaps(rstd_a, rows_a * 4, x_b, eb) || overlaps(rstd_a, rows_a * 4, y_b, eb) ||
                             (rstd_b != nullptr && overlaps(rstd_a, rows_a * 4, rstd_b, rows_b * 4)))) ||
      (rstd_b != nullptr && (overlaps(rstd_b, rows_b * 4, x_a, ea) || overlaps(rstd_b, rows_b * 4, y_a, ea))))
    return fail(RMSNORM_EINVAL, "the pair's outputs must not alias its inputs or each other");
  hipError_t e = rbi::launch_fwd_pair(a, b, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rmsnorm_fwd_packed_pair launch");
  return RMSNORM_OK;
}

int rmsnorm_bwd_dx_packed_pair(const rmsnorm_bf16* x_a, const rmsnorm_bf16* w_a,
                               const rmsnorm_bf16* dy_a, const float* rstd_a, rmsnorm_bf16* dx_a,
                               int64_t heads_a, int64_t token_stride_a,
                               const rmsnorm_layout* layout_a, rmsnorm_dw_acc* acc_a,
                               const rmsnorm_bf16* x_b, const rmsnorm_bf16* w_b,
                               const rmsnorm_bf16* dy_b, const float* rstd_b, rmsnorm_bf16* dx_b,
                               int64_t heads_b, int64_t token_stride_b,
                               const rmsnorm_layout* layout_b, rmsnorm_dw_acc* acc_b,
                               int64_t tokens, int64_t head_dim, void* stream) {
  rbi::RowPacking pa, pb;
  int64_t rows_a = 0, rows_b = 0, ext_a = 0, ext_b = 0;
  int rc;
  if ((rc = check_packing(tokens, heads_a, head_dim, token_stride_a, &pa, &rows_a, &ext_a)) ||
      (rc = check_packing(tokens, heads_b, head_dim, token_stride_b, &pb, &rows_b, &ext_b)))
    return rc;
  if (acc_a != nullptr && acc_a == acc_b)
    return fail(RMSNORM_EINVAL, "the two norms of a pair need accumulators of their own");
  BwdCall ca, cb;
  if ((rc = bwd_prepare(x_a, w_a, dy_a, rstd_a, dx_a, rows_a, head_dim, layout_a, acc_a, true, pa,
                        ext_a, false, 0.0f, &ca)) ||
      (rc = bwd_prepare(x_b, w_b, dy_b, rstd_b, dx_b, rows_b, head_dim, layout_b, acc_b, true, pb,
                        ext_b, false, 0.0f, &cb)))
    return rc;
  if (ca.launch) {
    const size_t ea = static_cast<size_t>(ext_a) * 2, eb = static_cast<size_t>(ext_b) * 2;
    if (overlaps(dx_a, ea, x_b, eb) || overlaps(dx_a, ea, dy_b, eb) ||
        overlaps(dx_a, ea, w_b, head_dim * 2) || overlaps(dx_a, ea, rstd_b, rows_b * 4) ||
        overlaps(dx_b, eb, x_a, ea) || overlaps(dx_b, eb, dy_a, ea) ||
        overlaps(dx_b, eb, w_a, head_dim * 2) || overlaps(dx_b, eb, rstd_a, rows_a * 4) ||
        !windows_disjoint(dx_a, heads_a * head_dim, token_stride_a, ext_a, dx_b,
                          heads_b * head_dim, token_stride_b, ext_b))
      return fail(RMSNORM_EINVAL, "the pair's dx must not alias its inputs or each other");
    hipError_t e = rbi::launch_bwd_pair(ca.a, acc_a != nullptr, cb.a, acc_b != nullptr,
                                        reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "rmsnorm_bwd_dx_packed_pair launch");
  }
  bwd_commit(ca);
  bwd_commit(cb);
  return RMSNORM_OK;
}

int rmsnorm_dw_contrib(const rmsnorm_bf16* x, const rmsnorm_bf16* dy, const float* rstd,
                       int64_t rows, int64_t hidden, const rmsnorm_layout* layout,
                       rmsnorm_dw_acc* acc, void* stream) {
  if (acc == nullptr) return fail(RMSNORM_EINVAL, "rmsnorm_dw_contrib needs an accumulator");
  return bwd_common(x, nullptr, dy, rstd, nullptr, rows, hidden, layout, acc, stream, false,
                    rbi::RowPacking{}, rows * hidden);
}

int rmsnorm_dw_finalize(rmsnorm_dw_acc* acc, float* dweight, void* stream) {
  if (acc == nullptr) return fail(RMSNORM_EINVAL, "accumulator is NULL");
  int rc;
  if ((rc = check_tensor(dweight, "dweight", 4))) return rc;
  std::vector<int32_t> spilled, slots;
  std::string err;
  rc = acc->host.prepare_finalize(&spilled, &err, &slots);
  if (rc != RMSNORM_OK) return fail(rc, err);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int32_t H = static_cast<int32_t>(acc->host.hidden);
  hipError_t e;
  if (acc->stream_form) {
    // blocks in stream form get their in-block tree (once: a repeated
    // finalize finds them joined); before the rebuild, which rewrites every
    // spilled block whatever its flag says
    if ((e = rbi::launch_join(acc->d_P, acc->d_Q, acc->d_form, acc->host.nb, H, st)) != hipSuccess)
      return hip_fail(e, "stream-form join");
    acc->stream_form = false;
  }
  if (!spilled.empty()) {
    // The spilled-block list goes to the device through a pinned host buffer
    // that the next finalize rewrites: a captured graph would replay that
    // copy from whatever the buffer holds then.  Refuse rather than record it.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(st, &cap)) != hipSuccess) return hip_fail(e, "capture query");
    if (cap != hipStreamCaptureStatusNone)
      return fail(RMSNORM_EUNSUPPORTED,
                  "finalize of an accumulator with blocks split across calls cannot be captured in "
                  "a HIP graph (it uploads the spilled-block list); finalize outside the capture");
    if (acc->staging_pending) {
      if ((e = hipEventSynchronize(acc->staged)) != hipSuccess) return hip_fail(e, "staging wait");
      acc->staging_pending = false;
    }
    // blocks, then their spill slots
    const size_t n = spilled.size();
    std::memcpy(acc->h_spilled, spilled.data(), n * sizeof(int32_t));
    std::memcpy(acc->h_spilled + n, slots.data(), n * sizeof(int32_t));
    if ((e = hipMemcpyAsync(acc->d_spilled, acc->h_spilled, 2 * n * sizeof(int32_t),
                            hipMemcpyHostToDevice, st)) != hipSuccess)
      return hip_fail(e, "spilled-block list upload");
    if ((e = hipEventRecord(acc->staged, st)) != hipSuccess) return hip_fail(e, "event record");
    acc->staging_pending = true;
    if ((e = rbi::launch_rebuild(acc->d_S, acc->d_P, acc->d_spilled, acc->d_spilled + n,
                                 static_cast<int32_t>(n), acc->host.n_logical, H, st)) !=
        hipSuccess)
      return hip_fail(e, "spilled-block rebuild");
  }
  if ((e = rbi::launch_tree(acc->d_P, acc->host.nb, acc->d_tmp, dweight, H, st)) != hipSuccess)
    return hip_fail(e, "block tree");
  acc->host.finalized = true;
  return RMSNORM_OK;
}

int rmsnorm_bwd_noalloc(const rmsnorm_bf16* x, const rmsnorm_bf16* w, const rmsnorm_bf16* dy,
                        const float* rstd, rmsnorm_bf16* dx, float* dweight, int64_t rows,
                        int64_t hidden, void* stream) {
  int rc;
  if ((rc = check_rows(rows)) || (rc = check_hidden(hidden))) return rc;
  if ((rc = check_tensor(dweight, "dweight", 4))) return rc;
  const int64_t nb = rbi::num_blocks(rows);
  const int64_t need = (nb + rbi::tree_scratch_rows(nb)) * hidden;
  if (need > kNoAllocScratchFloats)
    return fail(RMSNORM_EUNSUPPORTED,
                "rows x hidden needs " + std::to_string(need) + " floats of scratch (block partials "
                "and block tree), above the " + std::to_string(kNoAllocScratchFloats) +
                " this entry point holds; use rmsnorm_bwd_dx with an accumulator");
  if (rows > 0) {
    if ((rc = check_tensor(x, "x", 16)) || (rc = check_tensor(dy, "dy", 16)) ||
        (rc = check_tensor(w, "w", 16)) || (rc = check_tensor(rstd, "rstd", 4)) ||
        (rc = check_tensor(dx, "dx", 16)))
      return rc;
    const size_t nbytes = static_cast<size_t>(rows * hidden) * 2;
    if (overlaps(dx, nbytes, x, nbytes) || overlaps(dx, nbytes, dy, nbytes) ||
        overlaps(dx, nbytes, w, hidden * 2) || overlaps(dx, nbytes, rstd, rows * 4) ||
        overlaps(dx, nbytes, dweight, hidden * 4))
      return fail(RMSNORM_EINVAL, "dx must not alias an input or dweight");
    if (overlaps(dweight, hidden * 4, x, nbytes) || overlaps(dweight, hidden * 4, dy, nbytes) ||
        overlaps(dweight, hidden * 4, w, hidden * 2) || overlaps(dweight, hidden * 4, rstd, rows * 4))
      return fail(RMSNORM_EINVAL, "dweight must not alias an input");
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int32_t H = static_cast<int32_t>(hidden);
  hipError_t e;
  if (rows == 0) {
    // the empty multiset: dweight = 0, no scratch used
    if ((e = rbi::launch_tree(nullptr, 0, nullptr, dweight, H, st)) != hipSuccess)
      return hip_fail(e, "dweight zero fill");
    return RMSNORM_OK;
  }
  float* scr = nullptr;
  if ((rc = scratch_of_current_device(&scr))) return rc;
  // One call holding every logical row (identity map): every block is
  // complete, so every block partial is written and nothing spills; the
  // block tree writes every scratch row it reads.  Nothing needs clearing.
  rbi::BwdArgs a{};
  a.x = x;
  a.w = w;
  a.dy = dy;
  a.rstd = rstd;
  a.dx = dx;
  a.P = scr;
  a.S = nullptr;
  a.rows = rows;
  a.hidden = H;
  a.plan.n_items = static_cast<int32_t>(nb);
  a.plan.n_pad = 0;
  if ((e = rbi::launch_bwd(a, true, true, st)) != hipSuccess) return hip_fail(e, "rmsnorm backward launch");
  if ((e = rbi::launch_tree(scr, nb, scr + nb * hidden, dweight, H, st)) != hipSuccess)
    return hip_fail(e, "block tree");
  return RMSNORM_OK;
}

int64_t rmsnorm_bwd_noalloc_max_scratch(void) { return kNoAllocScratchFloats; }

int rmsnorm_layout_check(const int32_t* row_logical_host, int64_t rows, int64_t n_logical,
                         int64_t stats[5]) {
  rbi::PlanHost plan;
  std::string err;
  int rc = rbi::build_plan(row_logical_host, rows, n_logical, &plan, &err);
  if (rc != RMSNORM_OK) return fail(rc, err);
  if (stats) {
    stats[0] = plan.n_items();
    stats[1] = plan.n_complete;
    stats[2] = plan.n_partial;
    stats[3] = static_cast<int64_t>(plan.pad_rows.size());
    stats[4] = plan.n_real;
  }
  return RMSNORM_OK;
}

int rmsnorm_layout_create(rmsnorm_layout** out, const int32_t* row_logical_host, int64_t rows,
                          int64_t n_logical, void* stream) {
  if (out == nullptr) return fail(RMSNORM_EINVAL, "out is NULL");
  *out = nullptr;
  auto* L = new rmsnorm_layout();
  std::string err;
  int rc = rbi::build_plan(row_logical_host, rows, n_logical, &L->host, &err);
  if (rc != RMSNORM_OK) {
    delete L;
    return fail(rc, err);
  }
  const rbi::PlanHost& P = L->host;
  const size_t n_info = P.item_info.size(), n_slot = P.slot_phys.size(),
               n_pad = P.pad_rows.size(), n_rl = P.row_logical.size();
  std::vector<int32_t> staging;
  staging.reserve(n_info + n_slot + n_pad + n_rl + 4);
  staging.insert(staging.end(), P.item_info.begin(), P.item_info.end());
  staging.insert(staging.end(), P.slot_phys.begin(), P.slot_phys.end());
  staging.insert(staging.end(), P.pad_rows.begin(), P.pad_rows.end());
  staging.insert(staging.end(), P.row_logical.begin(), P.row_logical.end());
  staging.push_back(0);  // never allocate zero bytes
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMalloc(&L->d_mem, staging.size() * sizeof(int32_t));
  if (e != hipSuccess) {
    delete L;
    return hip_fail(e, "layout allocation");
  }
  e = hipMemcpyAsync(L->d_mem, staging.data(), staging.size() * sizeof(int32_t),
                     hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    (void)hipFree(L->d_mem);
    delete L;
    return hip_fail(e, "layout upload");
  }
  int32_t* base = static_cast<int32_t*>(L->d_mem);
  L->dev.item_info = base;
  L->dev.slot_phys = base + n_info;
  L->dev.pad_rows = base + n_info + n_slot;
  L->dev.row_logical = base + n_info + n_slot + n_pad;
  L->dev.n_items = static_cast<int32_t>(n_info);
  L->dev.n_pad = static_cast<int32_t>(n_pad);
  *out = L;
  return RMSNORM_OK;
}

int rmsnorm_layout_destroy(rmsnorm_layout* layout) {
  if (layout == nullptr) return RMSNORM_OK;
  hipError_t e = hipFree(layout->d_mem);  // hipFree waits for the device
  delete layout;
  if (e != hipSuccess) return hip_fail(e, "layout free");
  return RMSNORM_OK;
}

// max_spill_rows < 0: spill rows for every logical row (unbounded).
static int acc_create(rmsnorm_dw_acc** out, int64_t n_logical, int64_t hidden,
                      int64_t max_spill_rows) {
  if (out == nullptr) return fail(RMSNORM_EINVAL, "out is NULL");
  *out = nullptr;
  int rc;
  if ((rc = check_hidden(hidden))) return rc;
  if (n_logical < 0) return fail(RMSNORM_EINVAL, "n_logical must be non-negative");
  if (n_logical > INT32_MAX) return fail(RMSNORM_EUNSUPPORTED, "n_logical must be below 2^31");
  auto* A = new rmsnorm_dw_acc();
  const int64_t nb_all = rbi::num_blocks(n_logical);
  // a bounded area holds whole 64-row slots, never more than every block
  const int64_t spill_slots =
      max_spill_rows < 0 ? -1 : std::min(nb_all, rbi::num_blocks(max_spill_rows));
  A->host.init(n_logical, hidden, spill_slots);
  const int64_t nb = A->host.nb;
  const size_t spill_rows = spill_slots < 0 ? static_cast<size_t>(n_logical)
                                            : static_cast<size_t>(spill_slots) * rbi::kBlockRows;
  const size_t H = static_cast<size_t>(hidden);
  hipError_t e = hipSuccess;
  auto cleanup = [&](const char* what) {
    if (A->d_P) (void)hipFree(A->d_P);
    if (A->d_S) (void)hipFree(A->d_S);
    if (A->d_tmp) (void)hipFree(A->d_tmp);
    if (A->d_Q) (void)hipFree(A->d_Q);
    if (A->d_form) (void)hipFree(A->d_form);
    if (A->d_spilled) (void)hipFree(A->d_spilled);
    if (A->h_spilled) (void)hipHostFree(A->h_spilled);
    if (A->staged) (void)hipEventDestroy(A->staged);
    delete A;
    return hip_fail(e, what);
  };
  if ((e = hipMalloc(&A->d_P, std::max<size_t>(1, nb * H) * sizeof(float))) != hipSuccess)
    return cleanup("block partial allocation");
  if ((e = hipMalloc(&A->d_S, std::max<size_t>(1, spill_rows * H) * sizeof(float))) != hipSuccess)
    return cleanup("spill allocation");
  if ((e = hipMalloc(&A->d_tmp, std::max<size_t>(1, rbi::tree_scratch_rows(nb) * H) *
                                    sizeof(float))) != hipSuccess)
    return cleanup("tree scratch allocation");
  if ((e = hipMalloc(&A->d_Q, std::max<size_t>(1, 3 * nb * H) * sizeof(float))) != hipSuccess)
    return cleanup("stream-form allocation");
  if ((e = hipMalloc(&A->d_form, std::max<size_t>(1, nb) * sizeof(int32_t))) != hipSuccess)
    return cleanup("stream-form flag allocation");
  if ((e = hipMemset(A->d_form, 0, std::max<size_t>(1, nb) * sizeof(int32_t))) != hipSuccess)
    return cleanup("stream-form flag clear");
  if ((e = hipMalloc(&A->d_spilled, std::max<size_t>(1, 2 * nb) * sizeof(int32_t))) != hipSuccess)
    return cleanup("spill list allocation");
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&A->h_spilled),
                         std::max<size_t>(1, 2 * nb) * sizeof(int32_t), hipHostMallocDefault)) !=
      hipSuccess)
    return cleanup("pinned staging allocation");
  if ((e = hipEventCreateWithFlags(&A->staged, hipEventDisableTiming)) != hipSuccess)
    return cleanup("event creation");
  *out = A;
  return RMSNORM_OK;
}

int rmsnorm_dw_acc_create(rmsnorm_dw_acc** out, int64_t n_logical, int64_t hidden, void* stream) {
  (void)stream;
  return acc_create(out, n_logical, hidden, -1);
}

int rmsnorm_dw_acc_create_bounded(rmsnorm_dw_acc** out, int64_t n_logical, int64_t hidden,
                                  int64_t max_spill_rows, void* stream) {
  (void)stream;
  if (max_spill_rows < 0) return fail(RMSNORM_EINVAL, "max_spill_rows must be non-negative");
  return acc_create(out, n_logical, hidden, max_spill_rows);
}

int rmsnorm_dw_acc_reset(rmsnorm_dw_acc* acc, void* stream) {
  (void)stream;
  if (acc == nullptr) return fail(RMSNORM_EINVAL, "accumulator is NULL");
  acc->host.reset();
  acc->stream_form = false;
  return RMSNORM_OK;
}

int rmsnorm_dw_acc_destroy(rmsnorm_dw_acc* acc) {
  if (acc == nullptr) return RMSNORM_OK;
  hipError_t e = hipDeviceSynchronize();
  (void)hipFree(acc->d_P);
  (void)hipFree(acc->d_S);
  (void)hipFree(acc->d_tmp);
  (void)hipFree(acc->d_Q);
  (void)hipFree(acc->d_form);
  (void)hipFree(acc->d_spilled);
  (void)hipHostFree(acc->h_spilled);
  (void)hipEventDestroy(acc->staged);
  delete acc;
  if (e != hipSuccess) return hip_fail(e, "accumulator destroy");
  return RMSNORM_OK;
}

}  // extern "C"
