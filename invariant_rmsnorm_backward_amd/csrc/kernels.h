// kernels.h -- launchers of the gfx950 kernels (internal C++ interface used
// by the C-ABI layer).  The arithmetic a row or a canonical block goes
// through is fixed by `hidden` alone; the row count of a call only chooses
// how that same arithmetic is spread over workgroups, so a result cannot
// depend on how many rows share its call.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace rbi {

constexpr int kMaxHidden = 10240;

// Calls that touch fewer canonical blocks than the split threshold run the
// backward in two passes (row-parallel dx, column-split dweight fold); the
// per-row and per-block arithmetic is the same code as the fused kernel's,
// so the choice never changes a bit of any output.
constexpr int64_t kDefaultSplitItems = 96;   // measured crossover: 64 vs 128 blocks
void set_split_items(int64_t n);   // n < 0 restores the default
int64_t split_items();

// Calls that touch at least the stream threshold of blocks (and fewer than
// the split threshold), and compute dx and dweight contributions together
// into an accumulator, run the stream-owner backward: one workgroup per fold
// stream of each block, x and dy read once.  Same arithmetic again.
constexpr int64_t kDefaultStreamItems = 32;
void set_stream_items(int64_t n);   // n < 0 restores the default
int64_t stream_items();

// Cap on the workgroups of the looping fused backward (hidden 2048, 3072,
// 4096; 0: what the chip holds at once, occupancy x compute units).  A
// tuning and test knob: the arithmetic of every item is the same whichever
// workgroup runs it.
void set_wide_group_cap(int64_t n);   // n <= 0 restores the default
int64_t wide_group_cap();

// Physical->logical plan as the kernels see it (device pointers).
struct PlanDev {
  const int32_t* item_info = nullptr;  // nullptr: identity map, item = block
  const int32_t* slot_phys = nullptr;  // [n_items * 64]
  const int32_t* pad_rows = nullptr;   // [n_pad]
  const int32_t* row_logical = nullptr;
  int32_t n_items = 0;
  int32_t n_pad = 0;
};

// Row placement of the bf16 row tensors (x, y, dy, dx): row r = (token t,
// head h) with r = t * heads + h starts at t * token_stride + h * hidden.
// heads = 1 and token_stride = hidden is the contiguous [rows][hidden]
// layout; heads > 1 is a per-head norm applied inside a packed tensor (the
// heads of a fused QKV projection), supported for hidden <= 256.
struct RowPacking {
  int32_t heads = 1;
  int64_t token_stride = 0;   // 0: contiguous
};

struct FwdArgs {
  const uint16_t* x;
  const uint16_t* w;
  uint16_t* y;
  float* rstd;
  int64_t rows;
  int32_t hidden;
  float eps;
  const int32_t* row_logical;  // nullptr: no padding
  RowPacking pack{};
};

struct BwdArgs {
  const uint16_t* x;
  const uint16_t* w;   // needed for dx
  const uint16_t* dy;
  const float* rstd;
  uint16_t* dx;        // nullptr when only dweight contributions are wanted
  float* P;            // block partials [nb][hidden]
  float* S;            // spill rows, 64 per slot: [slots * 64][hidden]
  int64_t rows;
  int32_t hidden;
  PlanDev plan;
  RowPacking pack{};
  float eps = 0.0f;    // used only when rstd is rebuilt
  // Fused wide backward: workgroups that loop over the work items (set by
  // the launcher; the padding-row workgroups come after them).
  int32_t item_groups = 0;
  // Stream form (both nullptr: the stream-owner backward is not used).  A
  // block in stream form has q0 in P[b], q1..q3 in Q[b*3 .. b*3+2] and
  // form[b] = 1; every other writer of a complete block's P[b] sets
  // form[b] = 0.
  float* Q = nullptr;         // [nb * 3][hidden]
  int32_t* form = nullptr;    // [nb]
  // Spill slots of the call's partial items (n = -1: slot = block).
  SpillTable spill{};
};

// Which kernel family a backward call runs (decided by hidden, the call's
// block count, the thresholds above and whether stream form is available).
enum class BwdPath { kSmall, kSplit, kStream, kFused };
BwdPath bwd_path(const BwdArgs& a, bool with_dx, bool with_dw, bool recompute);

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// Two per-head norms (hidden <= 256, row placement given by each one's
// RowPacking) in one launch, every bit as in two launch_fwd calls.
hipError_t launch_fwd_pair(const FwdArgs& a, const FwdArgs& b, hipStream_t stream);
// The same for the backward with dx; dw_a / dw_b: fold into a.P / b.P.
hipError_t launch_bwd_pair(const BwdArgs& a, bool dw_a, const BwdArgs& b, bool dw_b,
                           hipStream_t stream);
// dst[0..n16) = src[0..n16) in 16-byte units with the kernels' streaming
// access policy, one unit per thread (a practical bandwidth ceiling).
hipError_t launch_stream_copy(const void* src, void* dst, int64_t n16, hipStream_t stream);
// with_dx: write dx (and zero padding rows); with_dw: fold dweight contributions.
// recompute: rstd is not read but rebuilt from x with a.eps in the forward's
// order (bitwise the saved rstd); needs with_dx and contiguous rows.
hipError_t launch_bwd(const BwdArgs& a, bool with_dx, bool with_dw, hipStream_t stream,
                      bool recompute = false);
// P[b] = (q0 + q1) + (q2 + q3) for every block b < nb with form[b] == 1.
hipError_t launch_join(float* P, const float* Q, const int32_t* form, int64_t nb, int32_t hidden,
                       hipStream_t stream);
// Rebuild the partials of spilled blocks from their spill rows (block
// blocks[i] from slot slots[i]: rows slots[i]*64 .. +63 of S).
hipError_t launch_rebuild(const float* S, float* P, const int32_t* blocks, const int32_t* slots,
                          int32_t n_blocks, int64_t n_logical, int32_t hidden, hipStream_t stream);
// dweight = pairwise tree over P[0..nb); tmp needs ceil(nb/32) * hidden floats.
hipError_t launch_tree(const float* P, int64_t nb, float* tmp, float* dweight, int32_t hidden,
                       hipStream_t stream);
int64_t tree_scratch_rows(int64_t nb);

bool hidden_supported(int hidden);
bool packed_hidden_supported(int hidden);   // hidden values the packed-row kernels take
const char* fwd_variant(int hidden);
const char* bwd_variant(int hidden);

}  // namespace rbi
