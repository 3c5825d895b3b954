// Fuzz driver for the host-side plan and accumulator bookkeeping, built with
// AddressSanitizer + UndefinedBehaviorSanitizer by tests/test_sanitizers.py.
// Random valid maps must build plans whose slots cover exactly the real rows;
// invalid maps must be refused; accumulator coverage must catch duplicates
// and missing rows.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "plan.h"

using namespace rbi;

static int fails = 0;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

int main() {
  std::mt19937_64 rng(12345);
  for (int iter = 0; iter < 3000; ++iter) {
    const int64_t T = rng() % 700;
    // a random subset of logical rows, permuted, with random padding interleaved
    std::vector<int32_t> ids;
    for (int64_t l = 0; l < T; ++l) if (rng() % 3 != 0) ids.push_back((int32_t)l);
    std::shuffle(ids.begin(), ids.end(), rng);
    std::vector<int32_t> rl;
    for (int32_t l : ids) {
      while (rng() % 5 == 0) rl.push_back(-1);
      rl.push_back(l);
    }
    PlanHost P;
    std::string err;
    int rc = build_plan(rl.data(), (int64_t)rl.size(), T, &P, &err);
    CHECK(rc == kOk);
    // every real row appears in exactly one slot, pads in the pad list
    std::vector<int> seen(rl.size(), 0);
    for (size_t it = 0; it < P.item_info.size(); ++it) {
      const int32_t info = P.item_info[it];
      const int32_t b = info >= 0 ? info : ~info;
      int present = 0, held = 0;
      for (int s = 0; s < kBlockRows; ++s) {
        const int32_t p = P.slot_phys[it * kBlockRows + s];
        if (b * (int64_t)kBlockRows + s < T) ++present;
        if (p >= 0) {
          CHECK(p < (int32_t)rl.size());
          CHECK(rl[p] == b * kBlockRows + s);
          seen[p]++;
          ++held;
        }
      }
      CHECK((info >= 0) == (held == present));
    }
    for (int32_t p : P.pad_rows) { CHECK(rl[p] == -1); seen[p]++; }
    for (size_t p = 0; p < rl.size(); ++p) CHECK(seen[p] == 1);
    {
      bool contig = !rl.empty();
      for (size_t p = 0; p < rl.size() && contig; ++p) contig = rl[p] >= 0 && rl[p] == rl[0] + (int32_t)p;
      CHECK(P.contig_first == (contig ? rl[0] : -1));
    }
    // accumulator: one call then finalize must report missing rows unless all held
    AccHost A;
    A.init(T, 8);
    CHECK(A.register_call(&P, (int64_t)rl.size(), &err) == kOk);
    CHECK(A.register_call(&P, (int64_t)rl.size(), &err) == (ids.empty() ? kOk : kECoverage));
    std::vector<int32_t> spilled;
    const int frc = A.prepare_finalize(&spilled, &err);
    CHECK(frc == ((int64_t)ids.size() == T ? kOk : kECoverage));
    // invalid maps: out of range, duplicate, below -1
    if (!rl.empty()) {
      std::vector<int32_t> bad = rl;
      bad[rng() % bad.size()] = (int32_t)T;
      CHECK(build_plan(bad.data(), (int64_t)bad.size(), T, &P, &err) == kELayout);
      bad = rl;
      bad[rng() % bad.size()] = -7;
      CHECK(build_plan(bad.data(), (int64_t)bad.size(), T, &P, &err) == kELayout);
      if (ids.size() >= 2) {
        // copy one real row's logical id onto another real row
        std::vector<size_t> real;
        for (size_t p = 0; p < rl.size(); ++p) if (rl[p] >= 0) real.push_back(p);
        bad = rl;
        bad[real[1]] = bad[real[0]];
        CHECK(build_plan(bad.data(), (int64_t)bad.size(), T, &P, &err) == kELayout);
      }
    }
  }
  // Call sequences against a per-row reference: random subsets (contiguous
  // chunks, whole blocks, scattered rows, some repeating earlier rows) and
  // identity calls, each permuted and padded.  A call must be accepted iff
  // none of its rows contributed before; a refusal names a repeated row; the
  // finalize check passes iff every row contributed, names the first missing
  // row otherwise, and lists exactly the blocks some call held in part.
  auto named_row = [](const std::string& e) -> int64_t {
    const std::string key = "logical row ";
    const size_t at = e.find(key);
    return at == std::string::npos ? -2 : std::strtoll(e.c_str() + at + key.size(), nullptr, 10);
  };
  for (int iter = 0; iter < 3000; ++iter) {
    const int64_t T = rng() % 400;
    const int64_t nb = (T + kBlockRows - 1) / kBlockRows;
    AccHost A;
    A.init(T, 8);
    std::vector<uint8_t> ref(T, 0);
    std::vector<uint8_t> ref_split(nb, 0);
    int64_t ref_n = 0;
    const int ncalls = 1 + rng() % 6;
    std::string err;
    for (int c = 0; c < ncalls; ++c) {
      if (rng() % 10 == 0) {
        const int rc = A.register_call(nullptr, T, &err);
        CHECK((rc == kOk) == (ref_n == 0));
        if (rc != kOk) {
          CHECK(rc == kECoverage);
          const int64_t l = named_row(err);
          CHECK(l >= 0 && l < T && ref[l]);
        } else {
          std::fill(ref.begin(), ref.end(), 1);
          ref_n = T;
        }
        continue;
      }
      std::vector<int32_t> ids;
      const int mode = rng() % 3;
      if (mode == 0 && T > 0) {
        int64_t a = rng() % (T + 1), b = rng() % (T + 1);
        if (a > b) std::swap(a, b);
        for (int64_t l = a; l < b; ++l) ids.push_back((int32_t)l);
      } else if (mode == 1) {
        for (int64_t l = 0; l < T; ++l)
          if (ref[l] ? rng() % 16 == 0 : rng() % 2 == 0) ids.push_back((int32_t)l);
      } else if (T > 0) {
        const int64_t b0 = rng() % nb;
        for (int64_t l = b0 * kBlockRows; l < std::min<int64_t>(T, (b0 + 1) * kBlockRows); ++l)
          ids.push_back((int32_t)l);
      }
      std::shuffle(ids.begin(), ids.end(), rng);
      std::vector<int32_t> rl;
      for (int32_t l : ids) {
        if (rng() % 7 == 0) rl.push_back(-1);
        rl.push_back(l);
      }
      PlanHost P;
      CHECK(build_plan(rl.data(), (int64_t)rl.size(), T, &P, &err) == kOk);
      bool fresh = true;
      for (int32_t l : ids) fresh = fresh && !ref[l];
      const int rc = A.register_call(&P, (int64_t)rl.size(), &err);
      CHECK((rc == kOk) == fresh);
      if (rc != kOk) {
        CHECK(rc == kECoverage);
        const int64_t l = named_row(err);
        CHECK(l >= 0 && l < T && ref[l] && std::find(ids.begin(), ids.end(), (int32_t)l) != ids.end());
        continue;
      }
      std::vector<int> held(nb, 0);
      for (int32_t l : ids) {
        ref[l] = 1;
        ++ref_n;
        held[l / kBlockRows]++;
      }
      for (int64_t b = 0; b < nb; ++b) {
        const int64_t present = std::min<int64_t>(kBlockRows, T - b * kBlockRows);
        if (held[b] > 0 && held[b] < present) ref_split[b] = 1;
      }
    }
    std::vector<int32_t> spilled;
    const int frc = A.prepare_finalize(&spilled, &err);
    CHECK((frc == kOk) == (ref_n == T));
    if (frc == kOk) {
      std::vector<int32_t> want;
      for (int64_t b = 0; b < nb; ++b) if (ref_split[b]) want.push_back((int32_t)b);
      CHECK(spilled == want);
    } else {
      CHECK(frc == kECoverage);
      const int64_t l = named_row(err);
      CHECK(l >= 0 && l < T && !ref[l]);
      for (int64_t k = 0; k < l && k < T; ++k) CHECK(ref[k]);
    }
    A.reset();
    CHECK(A.register_call(nullptr, T, &err) == kOk);
    CHECK(A.prepare_finalize(&spilled, &err) == kOk && spilled.empty());
  }
  // identity accumulator path and state machine
  // Contiguous runs of logical rows: contig_first, and the whole-block case
  // the backward runs without a device plan (items are the consecutive
  // blocks from contig_first / 64, all complete, slot s of item i at
  // physical row 64 i + s).
  for (int iter = 0; iter < 2000; ++iter) {
    const int64_t T = 1 + rng() % 900;
    int64_t a = rng() % T;
    if (rng() % 2) a -= a % kBlockRows;
    int64_t len = 1 + rng() % (T - a);
    if (rng() % 2) len = std::min<int64_t>(T - a, (len + kBlockRows - 1) / kBlockRows * kBlockRows);
    std::vector<int32_t> rl;
    for (int64_t l = a; l < a + len; ++l) rl.push_back((int32_t)l);
    const bool pad = rng() % 5 == 0;
    if (pad) rl.push_back(-1);
    PlanHost P;
    std::string err;
    CHECK(build_plan(rl.data(), (int64_t)rl.size(), T, &P, &err) == kOk);
    CHECK(P.contig_first == (pad ? -1 : a));
    const bool whole = P.contig_first >= 0 && P.contig_first % kBlockRows == 0 && P.n_partial == 0;
    CHECK(whole == (!pad && a % kBlockRows == 0 && (len % kBlockRows == 0 || a + len == T)));
    if (whole) {
      for (size_t it = 0; it < P.item_info.size(); ++it) {
        CHECK(P.item_info[it] == (int32_t)(a / kBlockRows + (int64_t)it));
        for (int s = 0; s < kBlockRows; ++s) {
          const int64_t p = (int64_t)it * kBlockRows + s;
          CHECK(P.slot_phys[it * kBlockRows + s] == (p < len ? (int32_t)p : -1));
        }
      }
    }
  }
  AccHost A;
  std::string err;
  A.init(100, 16);
  CHECK(A.register_call(nullptr, 99, &err) == kELayout);
  CHECK(A.register_call(nullptr, 100, &err) == kOk);
  std::vector<int32_t> sp;
  CHECK(A.prepare_finalize(&sp, &err) == kOk && sp.empty());
  A.finalized = true;
  CHECK(A.register_call(nullptr, 100, &err) == kEState);
  A.reset();
  CHECK(A.register_call(nullptr, 100, &err) == kOk);
  // check_call changes nothing: a call whose launch fails after the check is
  // never counted, so the accumulator still misses its rows at finalize
  A.reset();
  CHECK(A.check_call(nullptr, 100, &err) == kOk);
  CHECK(A.prepare_finalize(&sp, &err) == kECoverage);
  CHECK(A.check_call(nullptr, 100, &err) == kOk);   // still accepted: nothing was recorded
  A.commit_call(nullptr);
  CHECK(A.prepare_finalize(&sp, &err) == kOk);
  CHECK(A.check_call(nullptr, 100, &err) == kECoverage);
  {
    PlanHost P;
    std::vector<int32_t> rl = {5, 70, 71};
    CHECK(build_plan(rl.data(), (int64_t)rl.size(), 100, &P, &err) == kOk);
    AccHost B;
    B.init(100, 16);
    CHECK(B.check_call(&P, 3, &err) == kOk);
    CHECK(B.check_call(&P, 3, &err) == kOk);          // unchanged by the first check
    B.commit_call(&P);
    CHECK(B.check_call(&P, 3, &err) == kECoverage);   // now the rows are recorded
  }
  // Bounded spill area: contiguous pieces of random lengths cover [0, T).
  // With exactly as many slots as blocks held in part, every call fits, each
  // partial item is listed once with its block's one slot, and finalize
  // reports the same slots; with one slot fewer, the call that needs it is
  // refused (kESpill) and changes nothing.
  for (int iter = 0; iter < 400; ++iter) {
    const int64_t T = 1 + rng() % 900;
    std::vector<std::vector<int32_t>> calls;
    for (int64_t a = 0; a < T;) {
      const int64_t len = std::min<int64_t>(T - a, 1 + rng() % 150);
      std::vector<int32_t> rl;
      for (int64_t l = a; l < a + len; ++l) rl.push_back((int32_t)l);
      std::shuffle(rl.begin(), rl.end(), rng);
      calls.push_back(rl);
      a += len;
    }
    std::vector<PlanHost> plans(calls.size());
    std::vector<int> partial_blocks(num_blocks(T), 0);
    std::string err;
    for (size_t c = 0; c < calls.size(); ++c) {
      CHECK(build_plan(calls[c].data(), (int64_t)calls[c].size(), T, &plans[c], &err) == kOk);
      for (int32_t info : plans[c].item_info) if (info < 0) partial_blocks[~info] = 1;
    }
    int64_t need = 0;
    for (int v : partial_blocks) need += v;
    for (int shrink = 0; shrink <= 1; ++shrink) {
      if (shrink && need == 0) continue;
      AccHost A;
      A.init(T, 8, need - shrink);
      std::vector<int32_t> slot_of(num_blocks(T), -1);
      bool refused = false;
      for (size_t c = 0; c < calls.size(); ++c) {
        SpillTable tab;
        const int rc = A.check_call(&plans[c], (int64_t)calls[c].size(), &err, &tab);
        if (rc == kESpill) {
          CHECK(shrink == 1);
          refused = true;
          // refused: nothing recorded, the same answer again
          CHECK(A.check_call(&plans[c], (int64_t)calls[c].size(), &err, &tab) == kESpill);
          break;
        }
        CHECK(rc == kOk);
        int listed = 0;
        for (size_t it = 0; it < plans[c].item_info.size(); ++it) {
          const int32_t info = plans[c].item_info[it];
          if (info >= 0) continue;
          CHECK(listed < tab.n && tab.item[listed] == (int32_t)it);
          const int32_t sl = tab.slot[listed++];
          CHECK(sl >= 0 && sl < need - shrink);
          if (slot_of[~info] < 0) {
            for (int32_t o : slot_of) CHECK(o != sl);   // a new slot is free
            slot_of[~info] = sl;
          }
          CHECK(slot_of[~info] == sl);
        }
        CHECK(tab.n == (plans[c].n_partial > 0 ? listed : -1));
        A.commit_call(&plans[c]);
      }
      CHECK(refused == (shrink == 1));
      if (!refused) {
        std::vector<int32_t> sp, sl;
        CHECK(A.prepare_finalize(&sp, &err, &sl) == kOk);
        CHECK(sp.size() == sl.size() && (int64_t)sp.size() == need);
        for (size_t i = 0; i < sp.size(); ++i) CHECK(sl[i] == slot_of[sp[i]]);
        A.reset();
        CHECK(A.spill_used == 0);
      }
    }
  }
  {
    // more blocks in part than a bounded call takes: refused when bounded,
    // accepted (slot = block) when unbounded
    std::vector<int32_t> rl;
    for (int b = 0; b < 40; ++b) rl.push_back(b * kBlockRows);   // one row of each of 40 blocks
    PlanHost P;
    CHECK(build_plan(rl.data(), (int64_t)rl.size(), 40 * kBlockRows, &P, &err) == kOk);
    AccHost B, U;
    B.init(40 * kBlockRows, 8, 1000);
    U.init(40 * kBlockRows, 8);
    SpillTable tab;
    CHECK(B.check_call(&P, (int64_t)rl.size(), &err, &tab) == kEUnsupported);
    CHECK(U.check_call(&P, (int64_t)rl.size(), &err, &tab) == kOk && tab.n == -1);
    std::vector<int32_t> sp, sl;
    U.commit_call(&P);
    CHECK(U.prepare_finalize(&sp, &err, &sl) == kECoverage);
  }
  std::printf("plan fuzz: %s\n", fails ? "FAILED" : "ok");
  return fails ? 1 : 0;
}
