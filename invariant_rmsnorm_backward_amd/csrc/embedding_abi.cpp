// embedding_abi.cpp -- the C-ABI of include/det_embedding_bi.h: argument
// checks, the batch's canonical scatter plan (built on the host), the
// accumulator and kernel launches.  No fallback path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/det_embedding_bi.h"
#include "abi_internal.h"
#include "embedding.h"
#include "linear.h"
#include "plan.h"

using rbi::abi::check_rows;
using rbi::abi::check_tensor;
using rbi::abi::fail;
using rbi::abi::hip_fail;
using rbi::abi::overlaps;

namespace {

constexpr int64_t kMaxDim = 1 << 16;
constexpr int64_t kMaxVocab = (int64_t)1 << 28;

int check_dims(int64_t vocab, int64_t dim) {
  if (vocab <= 0 || dim <= 0) return fail(RMSNORM_EINVAL, "vocab and dim must be positive");
  if (dim % 8 != 0) return fail(RMSNORM_EUNSUPPORTED, "dim must be a multiple of 8");
  if (dim > kMaxDim) return fail(RMSNORM_EUNSUPPORTED, "dim must be at most 65536");
  if (vocab > kMaxVocab) return fail(RMSNORM_EUNSUPPORTED, "vocab must be at most 2^28");
  return RMSNORM_OK;
}

enum Mode { kEmpty = 0, kComputed = 1, kStaged = 2, kDirect = 3 };

// Host plan: occurrences grouped by token (counting sort, stable in the
// logical row), cut into blocks of kBlockOcc.
struct HostPlan {
  std::vector<int32_t> occ, blk_start, blk_len, tok_first, tok_nblk, blk_order, mb_blocks, mb_tokens,
      single_tokens, zero_tokens;
};

int build_plan(const int32_t* ids, int64_t T, int64_t vocab, HostPlan* P) {
  std::vector<int64_t> cnt(static_cast<size_t>(vocab) + 1, 0);
  for (int64_t l = 0; l < T; ++l) {
    if (ids[l] < 0 || ids[l] >= vocab)
      return fail(RMSNORM_EINVAL, "token id " + std::to_string(ids[l]) + " of logical row " +
                                      std::to_string(l) + " is outside [0, vocab)");
    cnt[static_cast<size_t>(ids[l]) + 1]++;
  }
  for (int64_t v = 0; v < vocab; ++v) cnt[v + 1] += cnt[v];
  std::vector<int64_t> pos(cnt.begin(), cnt.end());
  P->occ.assign(static_cast<size_t>(T), 0);
  for (int64_t l = 0; l < T; ++l) P->occ[pos[ids[l]]++] = static_cast<int32_t>(l);
  P->blk_start.clear();
  P->blk_len.clear();
  P->tok_first.assign(static_cast<size_t>(vocab), -1);
  P->tok_nblk.assign(static_cast<size_t>(vocab), 0);
  for (int64_t v = 0; v < vocab; ++v) {
    const int64_t a = cnt[v], n = cnt[v + 1] - cnt[v];
    if (n == 0) continue;
    P->tok_first[v] = static_cast<int32_t>(P->blk_start.size());
    for (int64_t b = 0; b * rbi::emb::kBlockOcc < n; ++b) {
      P->blk_start.push_back(static_cast<int32_t>(a + b * rbi::emb::kBlockOcc));
      P->blk_len.push_back(static_cast<int32_t>(std::min<int64_t>(rbi::emb::kBlockOcc,
                                                                   n - b * rbi::emb::kBlockOcc)));
    }
    P->tok_nblk[v] = static_cast<int32_t>(P->blk_start.size()) - P->tok_first[v];
  }
  // work order: longest blocks first (does not enter any result)
  P->blk_order.resize(P->blk_start.size());
  for (size_t i = 0; i < P->blk_order.size(); ++i) P->blk_order[i] = static_cast<int32_t>(i);
  std::stable_sort(P->blk_order.begin(), P->blk_order.end(),
                   [&](int32_t a, int32_t b) { return P->blk_len[a] > P->blk_len[b]; });
  // the blocks of tokens with two or more blocks (the one-call backward folds
  // single-block tokens in its finalize), in the same work order
  P->mb_blocks.clear();
  std::vector<int32_t> blk_tok(P->blk_start.size());
  for (int64_t v = 0; v < vocab; ++v)
    for (int32_t i = 0; i < P->tok_nblk[v]; ++i) blk_tok[P->tok_first[v] + i] = static_cast<int32_t>(v);
  for (int32_t b : P->blk_order)
    if (P->tok_nblk[blk_tok[b]] > 1) P->mb_blocks.push_back(b);
  P->mb_tokens.clear();
  P->single_tokens.clear();
  P->zero_tokens.clear();
  for (int64_t v = 0; v < vocab; ++v) {
    const int32_t n = P->tok_nblk[v];
    (n > 1 ? P->mb_tokens : n == 1 ? P->single_tokens : P->zero_tokens).push_back(static_cast<int32_t>(v));
  }
  // work order of the one-call backward's items: the longest trees and folds first
  std::stable_sort(P->mb_tokens.begin(), P->mb_tokens.end(),
                   [&](int32_t a, int32_t b) { return P->tok_nblk[a] > P->tok_nblk[b]; });
  std::stable_sort(P->single_tokens.begin(), P->single_tokens.end(), [&](int32_t a, int32_t b) {
    return P->blk_len[P->tok_first[a]] > P->blk_len[P->tok_first[b]];
  });
  return RMSNORM_OK;
}

}  // namespace

struct det_embedding_dw_acc {
  rbi::AccHost host;
  int64_t vocab = 0, dim = 0;
  int32_t* d_plan = nullptr;      // occ | blk_start | blk_len | tok_first | tok_nblk | blk_order |
                                  // mb_blocks | mb_tokens | single_tokens | zero_tokens
  size_t plan_cap = 0;            // int32 entries allocated
  rbi::emb::PlanView view{};
  float* d_P = nullptr;           // [max blocks][dim]
  int64_t max_blocks = 0;
  uint16_t* d_dy = nullptr;       // [n_logical][dim] staging, logical order
  Mode mode = kEmpty;
};

namespace {

int upload_plan(det_embedding_dw_acc* A, const int32_t* ids, hipStream_t st) {
  HostPlan P;
  int rc = build_plan(ids, A->host.n_logical, A->vocab, &P);
  if (rc != RMSNORM_OK) return rc;
  const int64_t nb = static_cast<int64_t>(P.blk_start.size());
  if (nb > A->max_blocks) return fail(RMSNORM_EINVAL, "internal: block count exceeds the bound");
  std::vector<int32_t> buf;
  buf.reserve(P.occ.size() + 4 * nb + 3 * A->vocab + 1);
  buf.insert(buf.end(), P.occ.begin(), P.occ.end());
  buf.insert(buf.end(), P.blk_start.begin(), P.blk_start.end());
  buf.insert(buf.end(), P.blk_len.begin(), P.blk_len.end());
  buf.insert(buf.end(), P.tok_first.begin(), P.tok_first.end());
  buf.insert(buf.end(), P.tok_nblk.begin(), P.tok_nblk.end());
  buf.insert(buf.end(), P.blk_order.begin(), P.blk_order.end());
  buf.insert(buf.end(), P.mb_blocks.begin(), P.mb_blocks.end());
  buf.insert(buf.end(), P.mb_tokens.begin(), P.mb_tokens.end());
  buf.insert(buf.end(), P.single_tokens.begin(), P.single_tokens.end());
  buf.insert(buf.end(), P.zero_tokens.begin(), P.zero_tokens.end());
  if (buf.size() > A->plan_cap) return fail(RMSNORM_EINVAL, "internal: plan exceeds its buffer");
  hipError_t e = hipStreamSynchronize(st);   // earlier work may still read the old plan
  if (e == hipSuccess && !buf.empty())
    e = hipMemcpy(A->d_plan, buf.data(), buf.size() * sizeof(int32_t), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "embedding plan upload");
  int32_t* b = A->d_plan;
  const int64_t T = A->host.n_logical;
  A->view.occ = b;
  A->view.blk_start = b + T;
  A->view.blk_len = b + T + nb;
  A->view.tok_first = b + T + 2 * nb;
  A->view.tok_nblk = b + T + 2 * nb + A->vocab;
  A->view.blk_order = b + T + 2 * nb + 2 * A->vocab;
  A->view.mb_blocks = b + T + 3 * nb + 2 * A->vocab;
  A->view.mb_tokens = A->view.mb_blocks + P.mb_blocks.size();
  A->view.single_tokens = A->view.mb_tokens + P.mb_tokens.size();
  A->view.zero_tokens = A->view.single_tokens + P.single_tokens.size();
  A->view.n_blocks = nb;
  A->view.n_mb_blocks = static_cast<int64_t>(P.mb_blocks.size());
  A->view.n_mb_tokens = static_cast<int64_t>(P.mb_tokens.size());
  A->view.n_single_tokens = static_cast<int64_t>(P.single_tokens.size());
  A->view.n_zero_tokens = static_cast<int64_t>(P.zero_tokens.size());
  A->view.vocab = A->vocab;
  A->host.reset();
  A->mode = kEmpty;
  return RMSNORM_OK;
}

}  // namespace

extern "C" {

int det_embedding_fwd(const int32_t* ids, const rmsnorm_bf16* table, rmsnorm_bf16* y,
                      int64_t rows, int64_t vocab, int64_t dim, const rmsnorm_layout* layout,
                      void* stream) {
  int rc;
  if ((rc = check_rows(rows)) || (rc = check_dims(vocab, dim))) return rc;
  if (layout != nullptr && layout->host.rows != rows)
    return fail(RMSNORM_ELAYOUT, "layout rows differ from rows");
  if (rows == 0) return RMSNORM_OK;
  if ((rc = check_tensor(ids, "ids", 4)) || (rc = check_tensor(table, "table", 16)) ||
      (rc = check_tensor(y, "y", 16)))
    return rc;
  if (overlaps(y, rows * dim * 2, table, vocab * dim * 2) || overlaps(y, rows * dim * 2, ids, rows * 4))
    return fail(RMSNORM_EINVAL, "y must not alias an input");
  hipError_t e = rbi::emb::launch_fwd(ids, table, y, rows, vocab, dim,
                                      layout ? layout->dev.row_logical : nullptr,
                                      reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "det_embedding_fwd launch");
  return RMSNORM_OK;
}

int det_embedding_dw_acc_create(det_embedding_dw_acc** out, const int32_t* ids_host,
                                int64_t n_logical, int64_t vocab, int64_t dim, void* stream) {
  if (out == nullptr) return fail(RMSNORM_EINVAL, "out is NULL");
  *out = nullptr;
  int rc;
  if ((rc = check_dims(vocab, dim))) return rc;
  if (n_logical < 0) return fail(RMSNORM_EINVAL, "n_logical must be non-negative");
  if (n_logical > rbi::emb::kMaxRows)
    return fail(RMSNORM_EUNSUPPORTED, "n_logical must be at most 2^21");
  if (n_logical > 0 && ids_host == nullptr) return fail(RMSNORM_EINVAL, "ids_host is NULL");
  auto* A = new det_embedding_dw_acc();
  A->host.init(n_logical, dim);
  A->vocab = vocab;
  A->dim = dim;
  // every token has at most one partly filled block: blocks <= T/64 + distinct tokens
  A->max_blocks = n_logical / rbi::emb::kBlockOcc + std::min<int64_t>(n_logical, vocab);
  // occ, 4 block lists, 2 per-token arrays, 3 token lists that partition the vocabulary
  A->plan_cap = static_cast<size_t>(n_logical + 4 * A->max_blocks + 3 * vocab + 1);
  hipError_t e = hipSuccess;
  auto cleanup = [&](const char* what) {
    if (A->d_plan) (void)hipFree(A->d_plan);
    if (A->d_P) (void)hipFree(A->d_P);
    if (A->d_dy) (void)hipFree(A->d_dy);
    delete A;
    return hip_fail(e, what);
  };
  if ((e = hipMalloc(&A->d_plan, A->plan_cap * sizeof(int32_t))) != hipSuccess)
    return cleanup("plan allocation");
  if ((e = hipMalloc(&A->d_P, std::max<size_t>(1, A->max_blocks * dim) * sizeof(float))) !=
      hipSuccess)
    return cleanup("block partial allocation");
  if ((e = hipMalloc(&A->d_dy, std::max<size_t>(8, n_logical * dim) * 2)) != hipSuccess)
    return cleanup("staging allocation");
  if ((rc = upload_plan(A, ids_host, reinterpret_cast<hipStream_t>(stream))) != RMSNORM_OK) {
    (void)hipFree(A->d_plan);
    (void)hipFree(A->d_P);
    (void)hipFree(A->d_dy);
    delete A;
    return rc;
  }
  *out = A;
  return RMSNORM_OK;
}

int det_embedding_dw_acc_set_ids(det_embedding_dw_acc* acc, const int32_t* ids_host,
                                 void* stream) {
  if (acc == nullptr) return fail(RMSNORM_EINVAL, "accumulator is NULL");
  if (acc->host.n_logical > 0 && ids_host == nullptr) return fail(RMSNORM_EINVAL, "ids_host is NULL");
  return upload_plan(acc, ids_host, reinterpret_cast<hipStream_t>(stream));
}

int det_embedding_dw_contrib(const rmsnorm_bf16* dy, int64_t rows, int64_t dim,
                             const rmsnorm_layout* layout, det_embedding_dw_acc* acc,
                             void* stream) {
  if (acc == nullptr) return fail(RMSNORM_EINVAL, "accumulator is NULL");
  int rc;
  if ((rc = check_rows(rows))) return rc;
  if (dim != acc->dim) return fail(RMSNORM_EINVAL, "dim differs from the accumulator's");
  if (layout != nullptr && layout->host.rows != rows)
    return fail(RMSNORM_ELAYOUT, "layout rows differ from rows");
  if (acc->host.finalized)
    return fail(RMSNORM_ESTATE, "accumulator already finalized; call det_embedding_dw_acc_reset first");
  if (rows > 0 && (rc = check_tensor(dy, "dy", 16))) return rc;
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
  if (layout == nullptr) {
    if ((e = rbi::emb::launch_blocks(dy, acc->view, dim, acc->d_P, st)) != hipSuccess)
      return hip_fail(e, "embedding block folds");
    acc->host.commit_call(plan_host);
    acc->mode = kComputed;
    return RMSNORM_OK;
  }
  if ((e = rbi::lin::launch_stage_rows(dy, rows, dim, layout->dev.row_logical, acc->d_dy, st)) !=
      hipSuccess)
    return hip_fail(e, "embedding staging");
  acc->host.commit_call(plan_host);
  acc->mode = kStaged;
  return RMSNORM_OK;
}

int det_embedding_dw_finalize(det_embedding_dw_acc* acc, float* dE, void* stream) {
  if (acc == nullptr) return fail(RMSNORM_EINVAL, "accumulator is NULL");
  int rc;
  if ((rc = check_tensor(dE, "dE", 16))) return rc;
  if (acc->mode == kDirect)
    return fail(RMSNORM_ESTATE,
                "det_embedding_bwd keeps no block partials; call det_embedding_dw_acc_reset first");
  std::vector<int32_t> spilled;
  std::string err;
  rc = acc->host.prepare_finalize(&spilled, &err);
  if (rc != RMSNORM_OK) return fail(rc, err);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (acc->mode == kStaged) {
    // every row is staged in logical order: the one-call backward's kernels
    // (no partials for single-block tokens) give the same bits
    if ((e = rbi::emb::launch_bwd_one_call(acc->d_dy, acc->d_P, acc->view, acc->dim, dE, st)) !=
        hipSuccess)
      return hip_fail(e, "embedding folds and token trees");
  } else if ((e = rbi::emb::launch_finalize(acc->d_P, acc->view, acc->dim, dE, st)) != hipSuccess) {
    return hip_fail(e, "embedding token trees");
  }
  acc->host.finalized = true;
  return RMSNORM_OK;
}

int det_embedding_bwd(const rmsnorm_bf16* dy, int64_t rows, int64_t dim, det_embedding_dw_acc* acc,
                      float* dE, void* stream) {
  if (acc == nullptr) return fail(RMSNORM_EINVAL, "accumulator is NULL");
  int rc;
  if ((rc = check_rows(rows))) return rc;
  if (dim != acc->dim) return fail(RMSNORM_EINVAL, "dim differs from the accumulator's");
  if (acc->host.finalized || acc->mode != kEmpty)
    return fail(RMSNORM_ESTATE,
                "det_embedding_bwd needs an accumulator with no contribution; call det_embedding_dw_acc_reset first");
  if (rows != acc->host.n_logical)
    return fail(RMSNORM_ECOVERAGE, "det_embedding_bwd takes all " +
                                       std::to_string(acc->host.n_logical) + " logical rows, got " +
                                       std::to_string(rows));
  if ((rc = check_tensor(dE, "dE", 16))) return rc;
  if (rows > 0 && (rc = check_tensor(dy, "dy", 16))) return rc;
  if (rows > 0 && overlaps(dE, acc->vocab * dim * 4, dy, rows * dim * 2))
    return fail(RMSNORM_EINVAL, "dE must not alias dy");
  std::string err;
  // the one call holds every logical row: check it, enqueue, then record it
  if ((rc = acc->host.check_call(nullptr, rows, &err)) != RMSNORM_OK) return fail(rc, err);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if ((e = rbi::emb::launch_bwd_one_call(dy, acc->d_P, acc->view, dim, dE, st)) != hipSuccess)
    return hip_fail(e, "embedding one-call backward");
  acc->host.commit_call(nullptr);
  acc->mode = kDirect;
  acc->host.finalized = true;
  return RMSNORM_OK;
}

int det_embedding_dw_acc_reset(det_embedding_dw_acc* acc, void* stream) {
  (void)stream;
  if (acc == nullptr) return fail(RMSNORM_EINVAL, "accumulator is NULL");
  acc->host.reset();
  acc->mode = kEmpty;
  return RMSNORM_OK;
}

int det_embedding_dw_acc_destroy(det_embedding_dw_acc* acc) {
  if (acc == nullptr) return RMSNORM_OK;
  hipError_t e = hipDeviceSynchronize();
  (void)hipFree(acc->d_plan);
  (void)hipFree(acc->d_P);
  (void)hipFree(acc->d_dy);
  delete acc;
  if (e != hipSuccess) return hip_fail(e, "accumulator destroy");
  return RMSNORM_OK;
}

}  // extern "C"
