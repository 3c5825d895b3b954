// plan.cpp -- host-side layout plans and accumulator bookkeeping (no HIP).
#include "plan.h"

#include <algorithm>
#include <cstring>

namespace rbi {

int build_plan(const int32_t* row_logical, int64_t rows, int64_t n_logical, PlanHost* out,
               std::string* err) {
  if (rows < 0 || n_logical < 0) {
    *err = "rows and n_logical must be non-negative";
    return kEInval;
  }
  if (rows > 0 && row_logical == nullptr) {
    *err = "row_logical is NULL";
    return kEInval;
  }
  if (rows > INT32_MAX || n_logical > INT32_MAX) {
    *err = "rows and n_logical must be below 2^31";
    return kEUnsupported;
  }
  const int64_t nb = num_blocks(n_logical);
  std::vector<uint8_t> seen(static_cast<size_t>(n_logical), 0);
  std::vector<int32_t> in_call(static_cast<size_t>(nb), 0);  // rows of block in this call
  int64_t n_real = 0;
  for (int64_t p = 0; p < rows; ++p) {
    const int32_t l = row_logical[p];
    if (l == -1) continue;
    if (l < 0 || l >= n_logical) {
      *err = "row_logical[" + std::to_string(p) + "] = " + std::to_string(l) +
             " is outside [-1, n_logical = " + std::to_string(n_logical) + ")";
      return kELayout;
    }
    if (seen[l]) {
      *err = "logical row " + std::to_string(l) + " appears twice (second at physical row " +
             std::to_string(p) + ")";
      return kELayout;
    }
    seen[l] = 1;
    in_call[l / kBlockRows] += 1;
    ++n_real;
  }

  PlanHost& P = *out;
  P = PlanHost();
  P.rows = rows;
  P.n_logical = n_logical;
  P.row_logical.assign(row_logical, row_logical + rows);
  P.n_real = n_real;

  // Items in ascending block order.
  std::vector<int32_t> item_of_block(static_cast<size_t>(nb), -1);
  for (int64_t b = 0; b < nb; ++b) {
    if (in_call[b] == 0) continue;
    const int64_t present = std::min<int64_t>(kBlockRows, n_logical - b * kBlockRows);
    const bool complete = in_call[b] == present;
    item_of_block[b] = static_cast<int32_t>(P.item_info.size());
    P.item_info.push_back(complete ? static_cast<int32_t>(b) : ~static_cast<int32_t>(b));
    if (complete) ++P.n_complete; else ++P.n_partial;
  }
  P.slot_phys.assign(P.item_info.size() * kBlockRows, -1);
  for (int64_t p = 0; p < rows; ++p) {
    const int32_t l = row_logical[p];
    if (l < 0) {
      P.pad_rows.push_back(static_cast<int32_t>(p));
      continue;
    }
    const int32_t item = item_of_block[l / kBlockRows];
    P.slot_phys[static_cast<size_t>(item) * kBlockRows + (l % kBlockRows)] = static_cast<int32_t>(p);
    if (P.item_info[static_cast<size_t>(item)] < 0) P.partial_rows.push_back(l);
  }
  if (rows > 0 && P.pad_rows.empty()) {
    bool contig = true;
    for (int64_t p = 1; p < rows && contig; ++p) contig = row_logical[p] == row_logical[0] + p;
    if (contig) P.contig_first = row_logical[0];
  }
  return kOk;
}

void AccHost::init(int64_t T, int64_t H, int64_t spill_slots) {
  n_logical = T;
  hidden = H;
  nb = num_blocks(T);
  spill_cap = spill_slots;
  spill_slot.assign(spill_slots >= 0 ? static_cast<size_t>(nb) : 0, -1);
  spill_used = 0;
  covered.assign(static_cast<size_t>(T), 0);
  block_state.assign(static_cast<size_t>(nb), kBlockNone);
  n_covered = 0;
  n_spilled = 0;
  identity_call = false;
  rows_dirty = false;
  blocks_dirty = false;
  finalized = false;
}

void AccHost::reset() {
  if (spill_used > 0) std::fill(spill_slot.begin(), spill_slot.end(), -1);
  spill_used = 0;
  if (rows_dirty) std::fill(covered.begin(), covered.end(), 0);
  if (blocks_dirty) std::fill(block_state.begin(), block_state.end(), kBlockNone);
  n_covered = 0;
  n_spilled = 0;
  identity_call = false;
  rows_dirty = false;
  blocks_dirty = false;
  finalized = false;
}

// First registered logical row of block b (-1 if none).
static int64_t first_registered_in(const AccHost& A, int64_t b) {
  const int64_t lo = b * kBlockRows, hi = std::min<int64_t>(lo + kBlockRows, A.n_logical);
  if (A.identity_call || A.block_state[static_cast<size_t>(b)] == kBlockDirect) return lo;
  for (int64_t l = lo; l < hi; ++l)
    if (A.covered[static_cast<size_t>(l)]) return l;
  return -1;
}

// First registered logical row of the accumulator (-1 if none).
static int64_t first_registered(const AccHost& A) {
  if (A.identity_call) return 0;
  for (int64_t b = 0; b < A.nb; ++b)
    if (A.block_state[static_cast<size_t>(b)] != kBlockNone) return first_registered_in(A, b);
  return -1;
}

// First logical row the plan holds in item `it`.
static int64_t first_held(const PlanHost& P, size_t it) {
  const int32_t info = P.item_info[it];
  const int64_t b = info >= 0 ? info : ~info;
  for (int s = 0; s < kBlockRows; ++s)
    if (P.slot_phys[it * kBlockRows + s] >= 0) return b * kBlockRows + s;
  return b * kBlockRows;
}

int AccHost::check_call(const PlanHost* plan, int64_t rows, std::string* err,
                        SpillTable* table) const {
  if (table != nullptr) table->n = -1;
  if (finalized) {
    *err = "accumulator already finalized; call rmsnorm_dw_acc_reset first";
    return kEState;
  }
  auto dup = [&](int64_t l) {
    *err = "logical row " + std::to_string(l) + " already contributed";
    return kECoverage;
  };
  if (plan == nullptr) {
    if (rows != n_logical) {
      *err = "identity layout with an accumulator needs rows (" + std::to_string(rows) +
             ") == n_logical (" + std::to_string(n_logical) + ")";
      return kELayout;
    }
    if (n_covered > 0) return dup(first_registered(*this));
    return kOk;
  }
  if (plan->n_logical != n_logical) {
    *err = "layout n_logical (" + std::to_string(plan->n_logical) +
           ") differs from the accumulator's (" + std::to_string(n_logical) + ")";
    return kELayout;
  }
  // A block this call holds completely must have no registered row; a block
  // it holds in part must not be held completely by an earlier call, and its
  // rows are checked one by one.
  for (size_t it = 0; it < plan->item_info.size(); ++it) {
    const int32_t info = plan->item_info[it];
    const int64_t b = info >= 0 ? info : ~info;
    if (identity_call) return dup(first_held(*plan, it));
    const uint8_t st = block_state[static_cast<size_t>(b)];
    if (info >= 0 && st != kBlockNone) return dup(first_registered_in(*this, b));
    if (info < 0 && st == kBlockDirect) return dup(first_held(*plan, it));
  }
  for (int32_t l : plan->partial_rows)
    if (covered[static_cast<size_t>(l)]) return dup(l);
  if (spill_cap >= 0 && plan->n_partial > 0) {
    if (plan->n_partial > kSpillTable) {
      *err = "the call holds " + std::to_string(plan->n_partial) + " blocks in part; an "
             "accumulator with a bounded spill area takes at most " +
             std::to_string(kSpillTable) + " per call";
      return kEUnsupported;
    }
    // the slots commit_call will hand out: assigned ones, then new ones in
    // item order
    int64_t next = spill_used;
    int32_t n = 0;
    for (size_t it = 0; it < plan->item_info.size(); ++it) {
      const int32_t info = plan->item_info[it];
      if (info >= 0) continue;
      int32_t slot = spill_slot[static_cast<size_t>(~info)];
      if (slot < 0) {
        if (next >= spill_cap) {
          *err = "spill area full: the accumulator holds " + std::to_string(spill_cap) +
                 " blocks of spill rows (64 rows each) and this call needs more (block " +
                 std::to_string(~info) + " held in part)";
          return kESpill;
        }
        slot = static_cast<int32_t>(next++);
      }
      if (table != nullptr) {
        table->item[n] = static_cast<int32_t>(it);
        table->slot[n] = slot;
      }
      ++n;
    }
    if (table != nullptr) table->n = n;
  }
  return kOk;
}

void AccHost::commit_call(const PlanHost* plan) {
  if (plan == nullptr) {
    identity_call = true;
    n_covered = n_logical;
    return;
  }
  for (int32_t info : plan->item_info) {
    if (info >= 0) {
      block_state[static_cast<size_t>(info)] = kBlockDirect;
    } else {
      if (block_state[static_cast<size_t>(~info)] != kBlockSpilled) {
        block_state[static_cast<size_t>(~info)] = kBlockSpilled;
        ++n_spilled;
      }
      if (spill_cap >= 0 && spill_slot[static_cast<size_t>(~info)] < 0)
        spill_slot[static_cast<size_t>(~info)] = static_cast<int32_t>(spill_used++);
    }
  }
  for (int32_t l : plan->partial_rows) covered[static_cast<size_t>(l)] = 1;
  if (!plan->item_info.empty()) blocks_dirty = true;
  if (!plan->partial_rows.empty()) rows_dirty = true;
  n_covered += plan->n_real;
}

int AccHost::register_call(const PlanHost* plan, int64_t rows, std::string* err) {
  const int rc = check_call(plan, rows, err);
  if (rc == kOk) commit_call(plan);
  return rc;
}

int AccHost::prepare_finalize(std::vector<int32_t>* spilled, std::string* err,
                              std::vector<int32_t>* slots) const {
  if (n_covered != n_logical) {
    // rows are registered at most once, so fewer than n_logical means a gap
    int64_t l = 0;
    while (l < n_logical) {
      const int64_t b = l / kBlockRows;
      if (block_state[static_cast<size_t>(b)] == kBlockDirect) {
        l = (b + 1) * kBlockRows;
      } else if (covered[static_cast<size_t>(l)]) {
        ++l;
      } else {
        break;
      }
    }
    *err = "logical row " + std::to_string(l) + " has not contributed";
    return kECoverage;
  }
  spilled->clear();
  if (slots != nullptr) slots->clear();
  if (n_spilled > 0)
    for (int64_t b = 0; b < nb; ++b)
      if (block_state[b] == kBlockSpilled) {
        spilled->push_back(static_cast<int32_t>(b));
        if (slots != nullptr)
          slots->push_back(spill_cap >= 0 ? spill_slot[static_cast<size_t>(b)]
                                          : static_cast<int32_t>(b));
      }
  return kOk;
}

}  // namespace rbi
