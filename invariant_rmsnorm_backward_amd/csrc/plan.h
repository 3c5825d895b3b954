// plan.h -- host-side layout plans and dweight-accumulator bookkeeping.
//
// Pure C++ (no HIP calls), so every check here runs on a machine without a
// GPU.  A plan turns a call's physical->logical row map into the work list
// of the backward kernel: one item per canonical block of 64 logical rows
// that the call touches, with the physical row of each of its 64 slots and
// whether the call holds every present row of the block (then the kernel
// folds the block completely; otherwise it spills the rows' contributions
// for the finalize step).  The accumulator bookkeeping enforces that every
// logical row contributes exactly once ("[WS1 Closeout][Backward] Reusable
// gradient-invariance harness and operator adapters", Acceptance criteria:
// B1 and BN use the same sample set and a fixed aggregation order).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace rbi {

constexpr int kBlockRows = 64;   // logical rows per canonical block
constexpr int kStreams = 4;      // in-block fold streams
constexpr int kSlotsPerStream = kBlockRows / kStreams;

enum Status : int {
  kOk = 0,
  kEInval = -1,
  kEUnsupported = -2,
  kELayout = -3,
  kECoverage = -4,
  kEState = -5,
  kEHip = -6,
  kESpill = -7,
};

// Spill slots of one call's partial items, for an accumulator with a
// bounded spill area (n = -1: unbounded, a block's spill rows are its own
// logical rows).  Passed to the kernels by value, so a call may hold at most
// kSpillTable blocks in part.
constexpr int kSpillTable = 32;
struct SpillTable {
  int32_t n = -1;
  int32_t item[kSpillTable];   // item index in the call's plan
  int32_t slot[kSpillTable];   // 64-row spill slot of that item's block
};

inline int64_t num_blocks(int64_t n_logical) { return (n_logical + kBlockRows - 1) / kBlockRows; }

struct PlanHost {
  int64_t rows = 0;
  int64_t n_logical = 0;
  std::vector<int32_t> row_logical;  // [rows], -1 = padding
  std::vector<int32_t> item_info;    // [n_items]: block id if complete, ~block id if partial
  std::vector<int32_t> slot_phys;    // [n_items * 64]: physical row or -1
  std::vector<int32_t> pad_rows;     // physical rows mapped to -1
  std::vector<int32_t> partial_rows; // logical ids of the rows of partial items (the only
                                     // rows whose coverage is tracked one by one)
  int64_t n_real = 0;                // rows with a logical id
  int64_t contig_first = -1;         // the rows are logical rows contig_first, +1, ... in
                                     // order with no padding row; else -1
  int64_t n_complete = 0;
  int64_t n_partial = 0;
  int64_t n_items() const { return static_cast<int64_t>(item_info.size()); }
};

// Validates the map and builds the plan.  Returns kOk or kELayout / kEInval
// with a message in *err.
int build_plan(const int32_t* row_logical, int64_t rows, int64_t n_logical, PlanHost* out,
               std::string* err);

enum BlockState : uint8_t { kBlockNone = 0, kBlockDirect = 1, kBlockSpilled = 2 };

// Coverage bookkeeping costs O(1) for a call with the identity map and
// O(items + rows of partial items) for a call with a layout: a block that a
// call holds completely is recorded once (kBlockDirect), since any other
// call touching it would repeat a row; only the rows of blocks split across
// calls are tracked one by one.  The per-row state is scanned only to name
// the offending row when a check fails.
struct AccHost {
  int64_t n_logical = 0;
  int64_t hidden = 0;
  int64_t nb = 0;
  std::vector<uint8_t> covered;       // per logical row of split blocks: contributed (0/1)
  std::vector<uint8_t> block_state;   // per block: BlockState, layout calls only
  int64_t n_covered = 0;              // logical rows that have contributed
  int64_t n_spilled = 0;              // blocks marked kBlockSpilled
  bool identity_call = false;         // an identity-map call covered every row
  bool rows_dirty = false;            // covered was written
  bool blocks_dirty = false;          // block_state was written
  bool finalized = false;
  // Bounded spill area (spill_cap >= 0 slots of 64 rows): a block held in
  // part takes the next free slot at its first call and keeps it until
  // reset.  spill_cap < 0: unbounded (slot = block).
  int64_t spill_cap = -1;
  std::vector<int32_t> spill_slot;    // per block, -1 = none (bounded only)
  int64_t spill_used = 0;

  void init(int64_t T, int64_t H, int64_t spill_slots = -1);
  void reset();
  // Registers one call.  plan == nullptr means the identity map over `rows`
  // rows (all blocks complete).  check_call validates without changing any
  // state; commit_call records a call that check_call accepted, once its
  // kernels are enqueued (a launch that fails leaves the accumulator as it
  // was); register_call does both.
  // With a bounded spill area check_call also fills *table (if non-NULL)
  // with the slots of the call's partial items (kESpill when the area is
  // full, kEUnsupported above kSpillTable partial items) and commit_call
  // takes them.
  int check_call(const PlanHost* plan, int64_t rows, std::string* err,
                 SpillTable* table = nullptr) const;
  void commit_call(const PlanHost* plan);
  int register_call(const PlanHost* plan, int64_t rows, std::string* err);
  // Checks that every logical row contributed exactly once and lists the
  // spilled blocks in ascending order, with their spill slots in *slots.
  int prepare_finalize(std::vector<int32_t>* spilled, std::string* err,
                       std::vector<int32_t>* slots = nullptr) const;
};

}  // namespace rbi
