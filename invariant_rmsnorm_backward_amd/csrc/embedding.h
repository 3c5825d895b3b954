// embedding.h -- launchers of the embedding (det_embedding) kernels,
// internal to the library.  Table rows are `dim` bf16 values, dim % 8 == 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rbi {
namespace emb {

constexpr int kBlockOcc = 64;        // occurrences per block of a token's fold (EDO-v1)
constexpr int kTreeLevels = 16;      // a token may have up to 2^16 - 1 blocks
constexpr int64_t kMaxRows = (int64_t)kBlockOcc << 15;   // so that every token fits

// Device view of a batch's canonical scatter plan: the logical rows of
// every token in ascending order, cut into blocks of <= 64 occurrences.
struct PlanView {
  const int32_t* occ;          // [n_logical] logical rows, grouped by token, ascending within a token
  const int32_t* blk_start;    // [n_blocks] first entry of the block in occ
  const int32_t* blk_len;      // [n_blocks] 1..64
  const int32_t* tok_first;    // [vocab] first block of the token, -1 if it does not occur
  const int32_t* tok_nblk;     // [vocab] number of blocks of the token
  const int32_t* blk_order;    // [n_blocks] block ids by decreasing length (work order only)
  const int32_t* mb_blocks;    // [n_mb_blocks] blocks of tokens with two or more blocks
  const int32_t* mb_tokens;    // [n_mb_tokens] tokens with two or more blocks, most blocks first
  const int32_t* single_tokens;  // [n_single_tokens] tokens with one block, longest first
  const int32_t* zero_tokens;    // [n_zero_tokens] tokens that do not occur
  int64_t n_blocks;
  int64_t n_mb_blocks;
  int64_t n_mb_tokens;
  int64_t n_single_tokens;
  int64_t n_zero_tokens;
  int64_t vocab;
};

hipError_t launch_fwd(const int32_t* ids, const uint16_t* table, uint16_t* y, int64_t rows,
                      int64_t vocab, int64_t dim, const int32_t* row_logical, hipStream_t stream);
// Block partials P[n_blocks][dim] from dY rows in logical order.
hipError_t launch_blocks(const uint16_t* dy, const PlanView& plan, int64_t dim, float* P,
                         hipStream_t stream);
// dE[vocab][dim]: each token's tree over its block partials, 0 for absent tokens.
hipError_t launch_finalize(const float* P, const PlanView& plan, int64_t dim, float* dE,
                           hipStream_t stream);
// The one-call backward: dE[vocab][dim] from dY rows in logical order, in two
// launches -- block partials into P only for tokens with two or more blocks,
// absent tokens 0; then those tokens' trees beside the single-block tokens,
// which are folded straight into dE.
hipError_t launch_bwd_one_call(const uint16_t* dy, float* P, const PlanView& plan, int64_t dim,
                               float* dE, hipStream_t stream);

}  // namespace emb
}  // namespace rbi
