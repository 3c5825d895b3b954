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
  std::printf("plan fuzz: %s\n", fails ? "FAILED" : "ok");
  return fails ? 1 : 0;
}
