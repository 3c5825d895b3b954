// embedding.hip -- gfx950 kernels of the batch-invariant embedding table
// gradient (the "Embedding / LM-head" adapter of "[WS1 Closeout][Backward]
// Reusable gradient-invariance harness and operator adapters", Required
// adapters).
//
// Forward y[r] = E[id(r)] is a row gather.  The backward is a scatter-add,
// dE[v] = sum of dY over the logical rows whose token is v: the other
// order-sensitive parameter VJP next to RMSNorm's dweight.  It is reduced in
// one canonical order keyed by (token id, logical row), EDO-v1:
//   * the occurrences of token v in ascending logical row index are cut into
//     blocks of 64 consecutive occurrences;
//   * a block is folded from +0.0 in occurrence order, one FP32 rounding per
//     added row (bf16 dY widened exactly);
//   * the token's block partials meet in a perfect pairwise tree with +0.0
//     leaves up to the next power of two; absent tokens get +0.0.
// The occurrence lists come from a host-built plan of the batch's token ids
// (logical order), and the dY rows are read in logical order (the caller's
// buffer when one call holds every row in order, else rows staged by
// logical index), so no layout can change a bit.  No atomics: every output
// element has one owner.
#include "embedding.h"

namespace rbi {
namespace emb {

typedef unsigned int u32x4e_t __attribute__((ext_vector_type(4)));
typedef float f32x4e_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void widen8(const u32x4e_t v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

// One 16-byte chunk (8 columns) per thread, grid-stride over rows x chunks.
__global__ __launch_bounds__(256) void fwd_kernel(const int32_t* __restrict__ ids,
                                                  const uint16_t* __restrict__ table,
                                                  uint16_t* __restrict__ y, int64_t rows,
                                                  int64_t vocab, int64_t dim,
                                                  const int32_t* __restrict__ row_logical) {
  const int64_t nq = dim / 8;
  const int64_t total = rows * nq;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / nq, q = i % nq;
    u32x4e_t v = {0u, 0u, 0u, 0u};
    const bool pad = row_logical != nullptr && row_logical[r] < 0;
    if (!pad) {
      const int64_t id = ids[r];
      if (id >= 0 && id < vocab)   // ids outside the table read nothing and give 0
        v = *reinterpret_cast<const u32x4e_t*>(table + id * dim + 8 * q);
    }
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4e_t*>(y + r * dim + 8 * q));
  }
}

// One block of <= 64 occurrences over 512 columns: one wavefront, 8 columns
// per lane.  Lane i first loads the block's i-th logical row index; the rows
// are then loaded 16 at a time (their indices read across lanes) and added
// in occurrence order.  Workgroups take the blocks longest first (the plan's
// work order; it does not enter any result).
__global__ __launch_bounds__(64) void block_kernel(const uint16_t* __restrict__ dy, PlanView p,
                                                   int64_t dim, float* __restrict__ P) {
  const int lane = threadIdx.x;
  const int64_t b = p.blk_order[blockIdx.x];
  const int64_t q = (int64_t)blockIdx.y * 64 + lane;
  const bool on = q < dim / 8;
  const int start = p.blk_start[b], len = p.blk_len[b];
  const int my_row = p.occ[start + (lane < len ? lane : len - 1)];
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int i0 = 0; i0 < len; i0 += 16) {
    u32x4e_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      v[u] = u32x4e_t{0u, 0u, 0u, 0u};
      if (i0 + u < len) {                                   // rows past the block's end are not loaded
        const int64_t l = __builtin_amdgcn_readlane(my_row, i0 + u);
        if (on) v[u] = *reinterpret_cast<const u32x4e_t*>(dy + l * dim + 8 * q);
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (i0 + u < len) {
        float f[8];
        widen8(v[u], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] + f[e];
      }
    }
  }
  if (on) {
    f32x4e_t* dst = reinterpret_cast<f32x4e_t*>(P + b * dim + 8 * q);
    dst[0] = f32x4e_t{acc[0], acc[1], acc[2], acc[3]};
    dst[1] = f32x4e_t{acc[4], acc[5], acc[6], acc[7]};
  }
}

// The tree of token v's nb block partials (rows first .. first + nb - 1 of P)
// over the 4 columns at c0: the partials, read in order, are combined like
// the digits of a binary counter -- level k holds a finished subtree of 2^k
// leaves, a new leaf merges upward as its left neighbours complete -- which
// is the perfect pairwise tree; the pending levels are joined from the
// lowest up, which is the same tree with +0.0 leaves to the next power of
// two (x + 0.0 == x for every partial: none is -0.0, all folds start from
// +0.0).  The partials are loaded 8 at a time ahead of the merges.
__device__ __forceinline__ void token_tree(const float* __restrict__ P, int first, int nb,
                                           int64_t dim, int64_t c0, float (&r)[4]) {
  float st[kTreeLevels][4] = {};
  for (int i0 = 0; i0 < nb; i0 += 8) {
    f32x4e_t pv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u < nb ? i0 + u : nb - 1;          // in bounds; extra loads unused
      pv[u] = *reinterpret_cast<const f32x4e_t*>(P + (int64_t)(first + i) * dim + c0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u;
      if (i < nb) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = pv[u][e];
        bool placed = false;
#pragma unroll
        for (int k = 0; k < kTreeLevels; ++k) {
          if (!placed) {
            if ((i >> k) & 1) {
#pragma unroll
              for (int e = 0; e < 4; ++e) x[e] = st[k][e] + x[e];
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) st[k][e] = x[e];
              placed = true;
            }
          }
        }
      }
    }
  }
  bool have = false;
#pragma unroll
  for (int k = 0; k < kTreeLevels; ++k) {
    if ((nb >> k) & 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = have ? st[k][e] + r[e] : st[k][e];
      have = true;
    }
  }
}

// Every vocabulary row v over 4 columns per thread (1024 per workgroup):
// the token's tree, or 0 for an absent token.
__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ P, PlanView p,
                                                       int64_t dim, float* __restrict__ dE) {
  const int64_t v = blockIdx.x;
  const int64_t c0 = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 4;
  if (c0 >= dim) return;
  const int first = p.tok_first[v];
  float r[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (first >= 0) token_tree(P, first, p.tok_nblk[v], dim, c0, r);
  __builtin_nontemporal_store(f32x4e_t{r[0], r[1], r[2], r[3]},
                              reinterpret_cast<f32x4e_t*>(dE + v * dim + c0));
}

// The one-call backward in two launches.  Each workgroup takes one item of a
// work list; the lists' order is only a schedule (longest items first), no
// result depends on it, and every dE row and partial has one writer.
//   head: [0, n_mb_blocks)        a block of a token with two or more blocks:
//                                 its fold over every column -> P[b];
//         [.., + ceil(n_zero/4))  up to 4 absent tokens: their dE rows are 0;
//   tail: [0, n_mb_tokens x TS)   the tree of a token with two or more blocks
//                                 over one slice of 1024 columns (TS slices);
//         [.., + n_single_tokens) a token with a single block: the same fold,
//                                 written straight to its dE row (the tree of
//                                 one leaf is that leaf), so no partial exists.
// The trees need only the head's partials, so they run beside the
// single-block folds instead of after every other item.  Folds run over 4096
// columns at a time, 8 + 8 per thread, with the rows loaded 8 at a time ahead
// of the adds, in occurrence order from +0.0: the additions of block_kernel,
// in the same order.
constexpr int kZeroRowsPerGroup = 4;
constexpr int kTreeCols = 1024;   // columns of one tree item (256 threads x 4)

__device__ __forceinline__ void fold_to(const uint16_t* __restrict__ dy, const int32_t* __restrict__ occ,
                                        int start, int len, int64_t dim, float* __restrict__ out, int t) {
  // two 2048-column passes at a time, so that a short block's loads for both
  // are in flight together; rows past the block's end are not loaded
  for (int64_t c0 = (int64_t)t * 8; c0 < dim; c0 += 2 * 256 * 8) {
    const int64_t c1 = c0 + 256 * 8;
    const bool two = c1 < dim;
    float r0[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    float r1[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int i0 = 0; i0 < len; i0 += 8) {
      u32x4e_t q0[8], q1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (i0 + u < len) {
          const uint16_t* row = dy + (int64_t)occ[start + i0 + u] * dim;
          q0[u] = *reinterpret_cast<const u32x4e_t*>(row + c0);
          if (two) q1[u] = *reinterpret_cast<const u32x4e_t*>(row + c1);
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (i0 + u < len) {
          float f[8];
          widen8(q0[u], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) r0[e] = r0[e] + f[e];
          if (two) {
            widen8(q1[u], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) r1[e] = r1[e] + f[e];
          }
        }
      }
    }
    f32x4e_t* dst = reinterpret_cast<f32x4e_t*>(out + c0);
    __builtin_nontemporal_store(f32x4e_t{r0[0], r0[1], r0[2], r0[3]}, dst);
    __builtin_nontemporal_store(f32x4e_t{r0[4], r0[5], r0[6], r0[7]}, dst + 1);
    if (two) {
      dst = reinterpret_cast<f32x4e_t*>(out + c1);
      __builtin_nontemporal_store(f32x4e_t{r1[0], r1[1], r1[2], r1[3]}, dst);
      __builtin_nontemporal_store(f32x4e_t{r1[4], r1[5], r1[6], r1[7]}, dst + 1);
    }
  }
}

__global__ __launch_bounds__(256) void bwd_head_kernel(const uint16_t* __restrict__ dy, PlanView p,
                                                       int64_t dim, float* __restrict__ P,
                                                       float* __restrict__ dE) {
  const int64_t g = blockIdx.x;
  const int t = threadIdx.x;
  if (g < p.n_mb_blocks) {
    const int64_t b = p.mb_blocks[g];
    fold_to(dy, p.occ, p.blk_start[b], p.blk_len[b], dim, P + b * dim, t);
    return;
  }
  const int64_t z0 = (g - p.n_mb_blocks) * kZeroRowsPerGroup;
  const f32x4e_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t z = z0; z < z0 + kZeroRowsPerGroup && z < p.n_zero_tokens; ++z) {
    f32x4e_t* row = reinterpret_cast<f32x4e_t*>(dE + (int64_t)p.zero_tokens[z] * dim);
    for (int64_t q = t; q < dim / 4; q += 256) __builtin_nontemporal_store(zero, row + q);
  }
}

__global__ __launch_bounds__(256) void bwd_tail_kernel(const uint16_t* __restrict__ dy, PlanView p,
                                                       int64_t dim, const float* __restrict__ P,
                                                       float* __restrict__ dE) {
  const int64_t g = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t ts = (dim + kTreeCols - 1) / kTreeCols;
  if (g < p.n_mb_tokens * ts) {
    const int64_t v = p.mb_tokens[g / ts];
    const int64_t c0 = (g % ts) * kTreeCols + (int64_t)t * 4;
    if (c0 >= dim) return;
    float r[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    token_tree(P, p.tok_first[v], p.tok_nblk[v], dim, c0, r);
    __builtin_nontemporal_store(f32x4e_t{r[0], r[1], r[2], r[3]},
                                reinterpret_cast<f32x4e_t*>(dE + v * dim + c0));
    return;
  }
  const int64_t v = p.single_tokens[g - p.n_mb_tokens * ts];
  const int b = p.tok_first[v];
  fold_to(dy, p.occ, p.blk_start[b], p.blk_len[b], dim, dE + v * dim, t);
}

hipError_t launch_fwd(const int32_t* ids, const uint16_t* table, uint16_t* y, int64_t rows,
                      int64_t vocab, int64_t dim, const int32_t* row_logical, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  int64_t g = (rows * (dim / 8) + 255) / 256;
  if (g > 8192) g = 8192;
  fwd_kernel<<<dim3((unsigned)g), dim3(256), 0, st>>>(ids, table, y, rows, vocab, dim, row_logical);
  return hipGetLastError();
}

hipError_t launch_blocks(const uint16_t* dy, const PlanView& plan, int64_t dim, float* P,
                         hipStream_t st) {
  if (plan.n_blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)plan.n_blocks, (unsigned)((dim / 8 + 63) / 64));
  block_kernel<<<grid, dim3(64), 0, st>>>(dy, plan, dim, P);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* P, const PlanView& plan, int64_t dim, float* dE,
                           hipStream_t st) {
  if (plan.vocab == 0) return hipSuccess;
  const dim3 grid((unsigned)plan.vocab, (unsigned)((dim / 4 + 255) / 256));
  finalize_kernel<<<grid, dim3(256), 0, st>>>(P, plan, dim, dE);
  return hipGetLastError();
}

hipError_t launch_bwd_one_call(const uint16_t* dy, float* P, const PlanView& plan, int64_t dim,
                               float* dE, hipStream_t st) {
  const int64_t head = plan.n_mb_blocks + (plan.n_zero_tokens + kZeroRowsPerGroup - 1) / kZeroRowsPerGroup;
  const int64_t tail = plan.n_mb_tokens * ((dim + kTreeCols - 1) / kTreeCols) + plan.n_single_tokens;
  if (head > 0) bwd_head_kernel<<<dim3((unsigned)head), dim3(256), 0, st>>>(dy, plan, dim, P, dE);
  if (tail > 0) bwd_tail_kernel<<<dim3((unsigned)tail), dim3(256), 0, st>>>(dy, plan, dim, P, dE);
  return hipGetLastError();
}

}  // namespace emb
}  // namespace rbi
