// kernels.hip -- gfx950 kernels of batch-invariant RMSNorm.
//
// Forward: the backward's row shape -- one wavefront per row up to 1024
// columns, two above -- with 2 or 4 rows per workgroup (hidden >= 512, or any
// hidden that is not a power of two below 512), or one group of hidden/8
// lanes per row (hidden in {8..256}); streaming 16-byte bf16 loads and
// stores, FP32 math, DPP wavefront sums of squares.
//
// Backward: one workgroup per canonical block of 64 logical rows.  The
// dweight order (CDO-v2, following "WS1 C4 (#270) closeout evidence":
// parameter gradients from logical-row FP32 contributions reduced in a fixed
// order) is laid onto the hardware: each of the 4 fold streams is one
// wavefront (hidden <= 1024) or a pair of wavefronts (wider rows) that walks
// its slots w, w+4, ... in ascending order and keeps the running FP32 sums in
// registers, so x and dy are read from HBM once for dx and dweight together.
// The streams meet in LDS for the fixed in-block tree and the block partial
// goes to HBM; a separate pass reduces the partials with a perfect pairwise
// tree.  Blocks that a call holds only in part write their rows'
// contributions to a spill area instead, and the finalize step folds them in
// exactly the same order.  No atomics anywhere: every sum has one owner.
#include <mutex>
#include <type_traits>

#include "kernels.h"

#include "device_math.h"
#include "plan.h"

namespace rbi {

// Element offset of row r of a row tensor (see RowPacking).  PACKED is a
// compile-time switch so the contiguous kernels keep their plain addressing.
template <bool PACKED>
__device__ __forceinline__ int64_t row_off(const RowPacking& pk, int64_t r, int H) {
  if (!PACKED) return r * H;
  // rows < 2^31: a 32-bit division is enough (and much cheaper than 64-bit)
  const uint32_t t = static_cast<uint32_t>(r) / static_cast<uint32_t>(pk.heads);
  const uint32_t h = static_cast<uint32_t>(r) - t * static_cast<uint32_t>(pk.heads);
  return static_cast<int64_t>(t) * pk.token_stride + static_cast<int64_t>(h) * H;
}

// ----------------------------------------------------------------- forward
// The row's sum of squares, in the order every wide kernel uses (the
// forward here, and the backward that rebuilds rstd from x): the row's
// 16-byte chunks are grouped 64 at a time -- chunk q = 64k + l is lane l of
// group k -- and
//   s_q   = fmaf chain over the chunk's 8 squares, from +0.0, in column order
//   S_k   = wavefront sum (wave_sum) of s_{64k+l} over l (absent chunks: 0)
//   ss    = perfect pairwise tree over S_0 .. S_{K-1}, K = ceil(hidden/512),
//           padded with +0.0 to a power of two (pad_tree below).
// The padding makes the tree over any longer list with +0.0 past K the same
// value, so a kernel may hold more (empty) groups than the row has.
template <int N>
__device__ __forceinline__ float pad_tree(float (&v)[N]) {
#pragma unroll
  for (int st = 1; st < N; st *= 2)
#pragma unroll
    for (int k = 0; k + st < N; k += 2 * st) v[k] = v[k] + v[k + st];   // v + (+0.0) == v
  return v[0];
}
// The perfect pairwise tree over N = 2^m values fed one at a time, in
// order: the pending subtree roots are joined as the digits of a binary
// counter (left operand the earlier subtree), so at most m values are live.
template <int N>
struct RunningTree {
  static_assert((N & (N - 1)) == 0, "a power of two");
  static constexpr int LEVELS = N > 1 ? 1 + RunningTree<(N > 1 ? N / 2 : 1)>::LEVELS : 1;
  float pend[LEVELS];
  // value number i (0-based, compile-time in unrolled loops)
  __device__ __forceinline__ void push(int i, float v) {
#pragma unroll
    for (int l = 0; l < LEVELS; ++l) {
      if (((i >> l) & 1) == 0) {
        pend[l] = v;
        return;
      }
      v = pend[l] + v;
    }
  }
  __device__ __forceinline__ float root() const { return pend[LEVELS - 1]; }
};
template <>
struct RunningTree<1> {
  static constexpr int LEVELS = 1;
  float pend[1];
  __device__ __forceinline__ void push(int, float v) { pend[0] = v; }
  __device__ __forceinline__ float root() const { return pend[0]; }
};

__device__ __forceinline__ float chunk_squares(const uint4& v) {
  float f[8];
  unpack8(v, f);
  float c = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) c = fmaf(f[e], f[e], c);
  return c;
}

// Row shape of the wide forward, the backward's own: TW wavefronts per row
// (one up to 1024 columns, else two), V chunks per lane; lane l of wavefront
// h holds chunk groups h*V .. h*V+V-1, i.e. chunks (h*V + j)*64 + l.  A
// 256-thread workgroup takes 4/TW consecutive rows, each row's wavefronts
// swapping their group sums through LDS.  Many short workgroups that read
// their rows once and write them once keep the access stream in address
// order across the chip (measured on hidden 4096, 5120 and 8192: 74-77% of
// 8 TB/s, against 63-72% for one wavefront per row over a capped grid and
// for one chunk per thread at 5120 and 8192).
// FULL: hidden == 512*V*TW (no lane masks).  PAD: the call has padding rows.
template <int V, int TW, bool FULL, bool PAD>
__global__ __launch_bounds__(256) void fwd_row_kernel(FwdArgs a) {
  constexpr int RPW = 4 / TW;          // rows per workgroup
  constexpr int G = V * TW;            // chunk groups held (at least the row's)
  __shared__ float s_s[TW > 1 ? RPW * G : 1];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int rg = wv / TW;              // the workgroup's row
  const int half = wv % TW;            // wavefront within the row
  const int H = FULL ? 512 * G : a.hidden;
  const int nchunk = H >> 3;
  const int64_t row = (int64_t)blockIdx.x * RPW + rg;
  const bool live = row < a.rows;
  const bool real = live && (!PAD || a.row_logical[row] >= 0);   // uniform per wavefront
  const int base = (half * V * 64 + lane) * 8;                     // first column of chunk 0
  auto in_row = [&](int j) { return FULL || (half * V + j) * 64 + lane < nchunk; };
  uint4 wc[V], xv[V];
#pragma unroll
  for (int j = 0; j < V; ++j) wc[j] = in_row(j) ? load16(a.w + base + j * 512) : make_uint4(0, 0, 0, 0);
  if (real) {
    const uint16_t* xr = a.x + row * H + base;
#pragma unroll
    for (int j = 0; j < V; ++j) xv[j] = in_row(j) ? load16_stream(xr + j * 512) : make_uint4(0, 0, 0, 0);
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) xv[j] = make_uint4(0, 0, 0, 0);
  }
  float S[V];
#pragma unroll
  for (int j = 0; j < V; ++j) S[j] = wave_sum(chunk_squares(xv[j]));
  float ss;
  if constexpr (TW == 1) {
    ss = pad_tree(S);
  } else {
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < V; ++j) s_s[rg * G + half * V + j] = S[j];
    }
    __syncthreads();
    float g[G];
#pragma unroll
    for (int k = 0; k < G; ++k) g[k] = s_s[rg * G + k];
    ss = pad_tree(g);
  }
  if (!live) return;
  const float r = real ? rsqrtf(ss / (float)H + a.eps) : 0.0f;
  uint16_t* yr = a.y + row * H + base;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    if (in_row(j)) {
      uint4 out = make_uint4(0, 0, 0, 0);   // padding rows: +0.0
      if (real) {
        float f[8], g[8], o[8];
        unpack8(xv[j], f);
        unpack8(wc[j], g);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (f[e] * r) * g[e];
        out = pack8(o);
      }
      store16_stream(yr + j * 512, out);
    }
  }
  if (half == 0 && lane == 0 && a.rstd != nullptr) a.rstd[row] = r;
}

// hidden = 8L with L lanes per row (L in 1..32, a power of two); workgroup
// wg of n_wg walks row groups wg, wg + n_wg, ...
template <int L, bool PACKED>
__device__ __forceinline__ void fwd_small_rows(const FwdArgs& a, int64_t wg, int64_t n_wg) {
  constexpr int H = 8 * L;
  constexpr int GROUPS = 256 / L;
  const int g = threadIdx.x / L;
  const int sub = threadIdx.x % L;
  float wf[8];
  unpack8(load16(a.w + sub * 8), wf);
  for (int64_t base = wg * GROUPS; base < a.rows; base += n_wg * GROUPS) {
    const int64_t row = base + g;
    const bool valid = row < a.rows;
    const bool pad = valid && a.row_logical != nullptr && a.row_logical[row] < 0;
    uint4 xv = make_uint4(0, 0, 0, 0);
    const int64_t off = valid ? row_off<PACKED>(a.pack, row, H) : 0;
    if (valid && !pad) xv = load16_stream(a.x + off + sub * 8);
    float f[8];
    unpack8(xv, f);
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
    ss = group_sum<L>(ss);
    const float r = rsqrtf(ss / (float)H + a.eps);
    if (valid) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = pad ? 0.0f : (f[e] * r) * wf[e];
      store16_stream(a.y + off + sub * 8, pack8(o));
      if (sub == 0 && a.rstd != nullptr) a.rstd[row] = pad ? 0.0f : r;
    }
  }
}
template <int L, bool PACKED>
__global__ __launch_bounds__(256) void fwd_small_kernel(FwdArgs a) {
  fwd_small_rows<L, PACKED>(a, blockIdx.x, gridDim.x);
}
// Two per-head norms (the Q and K heads of a packed tensor) in one launch:
// workgroups 0 .. wg_a-1 run norm a, the rest norm b, each exactly as in its
// own launch.
template <int L>
__global__ __launch_bounds__(256) void fwd_small_pair_kernel(FwdArgs a, FwdArgs b, int wg_a) {
  if ((int)blockIdx.x < wg_a) fwd_small_rows<L, true>(a, blockIdx.x, wg_a);
  else fwd_small_rows<L, true>(b, (int)blockIdx.x - wg_a, (int)gridDim.x - wg_a);
}

// ----------------------------------------------------------------- backward
__device__ __forceinline__ int slot_row(const BwdArgs& a, int item, int blk, int s) {
  if (a.plan.item_info != nullptr) return a.plan.slot_phys[(int64_t)item * kBlockRows + s];
  const int64_t r = (int64_t)blk * kBlockRows + s;
  return r < a.rows ? (int)r : -1;
}
// Same, with the layout kind known at compile time (PLAN: a plan; else the
// identity map), so each kernel instance has one straight memory sequence.
template <bool PLAN>
__device__ __forceinline__ int slot_row_t(const BwdArgs& a, int item, int blk, int s) {
  if (PLAN) return a.plan.slot_phys[(int64_t)item * kBlockRows + s];
  const int64_t r = (int64_t)blk * kBlockRows + s;
  return r < a.rows ? (int)r : -1;
}

// First spill row of work item `item` (a block the call holds in part): its
// block's own rows, or the slot the accumulator gave the block.  The host
// lists every partial item of the call in the table.
__device__ __forceinline__ int64_t spill_row0(const BwdArgs& a, int item, int blk) {
  if (a.spill.n < 0) return (int64_t)blk * kBlockRows;
  int slot = 0;
  for (int j = 0; j < a.spill.n; ++j)
    if (a.spill.item[j] == item) slot = a.spill.slot[j];
  return (int64_t)slot * kBlockRows;
}

// Wide rows (hidden > 256).  A row is held by a team of TW wavefronts:
// wavefront h of the team holds the chunk groups h*V .. h*V+V-1, where chunk
// group g is the 64 16-byte chunks 64g .. 64g+63 and lane l holds chunk
// 64g + l.  FULL means hidden == 512*V*TW exactly, so no lane needs a mask.
//
// The row's dot = sum_j (dy_j*x_j)*w_j has one order for every wide kernel,
// whatever its shape (the same grouping as the sum of squares above):
//   d_q = fmaf chain over chunk q's 8 products (dy*x, exact) times w, from
//         +0.0, in column order
//   D_g = wave_sum of d_{64g+l} over l (absent chunks: +0.0)
//   dot = perfect pairwise tree over D_0 .. D_{K-1}, padded with +0.0.
// So dx is a function of the row and hidden alone, and each kernel may spread
// a row over as many wavefronts as suits it (the fused backward, the dx rows
// of the two-pass path and the rstd-recompute backward all give the same
// bits).  No partial sum is ever -0.0 (every chain starts from +0.0), so the
// +0.0 padding of the tree changes nothing.
template <int V, int TW, bool FULL>
struct RowLanes {
  static constexpr int G = V * TW;     // chunk groups a team holds
  static constexpr int COLS = 512 * G; // columns a team covers
  int lane, half, nchunk, base;        // base: first column of chunk 0 of this lane
  __device__ __forceinline__ bool in_row(int k) const {
    return FULL || (half * V + k) * 64 + lane < nchunk;
  }
};

// w as FP32 in LDS (columns past hidden hold 0).  FP32 rather than bf16
// saves the widening on every use: 1.2% of the hidden-4096 backward.
template <int COLS, int THREADS>
__device__ __forceinline__ void stage_w(const BwdArgs& a, float* w_s, int tid, int nchunk) {
  for (int q = tid; q < COLS / 8; q += THREADS) {
    float f[8];
    unpack8(q < nchunk ? load16(a.w + q * 8) : make_uint4(0, 0, 0, 0), f);
    store_f4(&w_s[q * 8], f[0], f[1], f[2], f[3]);
    store_f4(&w_s[q * 8 + 4], f[4], f[5], f[6], f[7]);
  }
  __syncthreads();
}

// The per-row work of a team: one row's partial sums, the team's exchange of
// its group sums through LDS (TW > 1; the workgroup meets at a barrier, so
// every team of the workgroup calls row() the same number of times), dx, and
// the row's dweight contributions c = fl32(fl32(dy*x)*rstd) -- added to the
// stream sums `acc` (a block the call holds completely) or written to the
// spill row `srow` (a block held in part).  RC: rstd is not given but
// rebuilt from the row in the forward's order, so its bits are the saved
// rstd's; the contributions then wait for it.
//
// When V is a power of two, a wavefront's V groups h*V .. h*V+V-1 are an
// aligned subtree of the padded tree over the row's groups, so the
// wavefront reduces them itself and the team exchanges one value per
// wavefront (the tree over those values, padded with +0.0, is the rest of
// the same tree); otherwise every group sum is exchanged.
template <int V, int TW, int TEAMS, bool FULL, bool DX, bool RC>
struct RowOps {
  using L = RowLanes<V, TW, FULL>;
  static constexpr int G = L::G;
  static constexpr bool SUBTREE = (V & (V - 1)) == 0;
  static constexpr int XG = SUBTREE ? TW : G;       // values a team exchanges per sum
  static constexpr int XN = RC ? 2 : 1;            // sums exchanged (dot, squares)
  static constexpr bool XCH = TW > 1 && (DX || RC);
  static constexpr int XCH_FLOATS = XCH ? 2 * TEAMS * XN * XG : 1;
  const BwdArgs& a;
  const float* w_s;
  float* xch;     // [2][TEAMS][XN][G]
  L ln;
  int team, H;

  __device__ __forceinline__ void load(int p, uint4 (&xv)[V], uint4 (&dv)[V]) const {
    // Loads are issued whether or not the slot is present (an absent slot
    // reads row 0) and whether or not the lane's chunk is inside the row (a
    // lane past the row's end reads the row's first chunk); mask() discards
    // what they read.  The same memory operations on every path and in every
    // lane keep the compiler's wait counts exact, so the rows issued ahead
    // stay in flight while this one is processed.
    const int row = p >= 0 ? p : 0;
    const uint16_t* xr = a.x + (int64_t)row * H + ln.base;
    const uint16_t* dr = a.dy + (int64_t)row * H + ln.base;
#pragma unroll
    for (int k = 0; k < V; ++k) {
      const int off = ln.in_row(k) ? k * 512 : -ln.base;
      xv[k] = load16_stream(xr + off);
      dv[k] = load16_stream(dr + off);
    }
  }
  // Zero the chunks of lanes past the row's end (after the data has arrived).
  __device__ __forceinline__ void mask(uint4 (&xv)[V], uint4 (&dv)[V]) const {
    if (FULL) return;
#pragma unroll
    for (int k = 0; k < V; ++k) {
      if (!ln.in_row(k)) {
        xv[k] = make_uint4(0, 0, 0, 0);
        dv[k] = make_uint4(0, 0, 0, 0);
      }
    }
  }

  // DW: contributions wanted; COMPLETE: into acc, else into srow.
  template <bool DW, bool COMPLETE>
  __device__ __forceinline__ void row(int j, int p, uint4 (&xv)[V], uint4 (&dv)[V], float r,
                                      float (&acc)[DW ? V * 8 : 1], float* srow) const {
    mask(xv, dv);
    // the group sums of this wavefront's chunk groups: kept one per group,
    // or (a power-of-two count) folded into the subtree as they come
    float d[SUBTREE ? 1 : V], sq[SUBTREE ? 1 : V];
    RunningTree<SUBTREE ? V : 1> td, ts;
#pragma unroll
    for (int k = 0; k < V; ++k) {
      float dk = 0.0f, sk = 0.0f;
      if (p >= 0) {
        float xf[8], df[8], c[8];
        unpack8(xv[k], xf);
        unpack8(dv[k], df);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pr = df[e] * xf[e];          // exact: two bf16 significands
          if (DX) dk = fmaf(pr, w_s[ln.base + k * 512 + e], dk);
          if (RC) sk = fmaf(xf[e], xf[e], sk);
          c[e] = pr * r;                           // the row's contribution, rounded once
          if (!RC && DW && COMPLETE) acc[k * 8 + e] = acc[k * 8 + e] + c[e];
        }
        if (!RC && DW && !COMPLETE && ln.in_row(k)) {
          store_f4_stream(srow + k * 512, c[0], c[1], c[2], c[3]);
          store_f4_stream(srow + k * 512 + 4, c[4], c[5], c[6], c[7]);
        }
      }
      if constexpr (SUBTREE) {
        if (DX) td.push(k, wave_sum(dk));
        if (RC) ts.push(k, wave_sum(sk));
      } else {
        if (DX) d[k] = wave_sum(dk);
        if (RC) sq[k] = wave_sum(sk);
      }
    }
    float dot = 0.0f;
    if (DX || RC) {
      float ss = 0.0f;
      if constexpr (!XCH) {
        // this wavefront holds every chunk group of the row
        if constexpr (SUBTREE) {
          if (DX) dot = td.root();
          if (RC) ss = ts.root();
        } else {
          if (DX) dot = pad_tree(d);
          if (RC) ss = pad_tree(sq);
        }
      } else if constexpr (SUBTREE) {
        // this wavefront's subtree, then the tree over the team's subtrees
        float* xs = xch + ((j & 1) * TEAMS + team) * XN * XG;
        if (ln.lane == 0) {
          if (DX) xs[ln.half] = td.root();
          if (RC) xs[(XN - 1) * XG + ln.half] = ts.root();
        }
        __syncthreads();
        float g[XG];
        if (DX) {
#pragma unroll
          for (int k = 0; k < XG; ++k) g[k] = xs[k];
          dot = pad_tree(g);
        }
        if (RC) {
#pragma unroll
          for (int k = 0; k < XG; ++k) g[k] = xs[(XN - 1) * XG + k];
          ss = pad_tree(g);
        }
      } else {
        float* xs = xch + ((j & 1) * TEAMS + team) * XN * XG;
        if (ln.lane == 0) {
#pragma unroll
          for (int k = 0; k < V; ++k) {
            if (DX) xs[ln.half * V + k] = d[k];
            if (RC) xs[(XN - 1) * XG + ln.half * V + k] = sq[k];
          }
        }
        __syncthreads();
        // every chunk group of the row, in group order
        float g[XG];
        if (DX) {
#pragma unroll
          for (int k = 0; k < XG; ++k) g[k] = xs[k];
          dot = pad_tree(g);
        }
        if (RC) {
#pragma unroll
          for (int k = 0; k < XG; ++k) g[k] = xs[(XN - 1) * XG + k];
          ss = pad_tree(g);
        }
      }
      if (RC) r = p >= 0 ? rsqrtf(ss / (float)H + a.eps) : 0.0f;
    }
    if (RC && DW && p >= 0) {
#pragma unroll
      for (int k = 0; k < V; ++k) {
        float xf[8], df[8], c[8];
        unpack8(xv[k], xf);
        unpack8(dv[k], df);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          c[e] = (df[e] * xf[e]) * r;
          if (COMPLETE) acc[k * 8 + e] = acc[k * 8 + e] + c[e];
        }
        if (!COMPLETE && ln.in_row(k)) {
          store_f4_stream(srow + k * 512, c[0], c[1], c[2], c[3]);
          store_f4_stream(srow + k * 512 + 4, c[4], c[5], c[6], c[7]);
        }
      }
    }
    if (DX && p >= 0) {
      const float kk = ((r * r) * r) * (dot / (float)H);
      uint16_t* xo = a.dx + (int64_t)p * H + ln.base;
      // re-derive the FP32 values from the packed registers instead of
      // keeping twice as many registers live across the exchange
      compiler_fence();
#pragma unroll
      for (int k = 0; k < V; ++k) {
        launder(xv[k]);
        launder(dv[k]);
      }
#pragma unroll
      for (int k = 0; k < V; ++k) {
        if (ln.in_row(k)) {
          float xf[8], df[8], o[8];
          unpack8(xv[k], xf);
          unpack8(dv[k], df);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float g = df[e] * w_s[ln.base + k * 512 + e];
            o[e] = fmaf(-xf[e], kk, r * g);
          }
          store16_stream(xo + k * 512, pack8(o));
        }
      }
    }
  }
};

// ------------------------------------------------------- fused backward
// One workgroup owns each canonical block of 64 logical rows it is given and
// runs dx and the dweight fold in one pass over x and dy.  The workgroup is
// TEAMS teams of TW wavefronts, each team on one row at a time:
//   TEAMS = 2 (hidden > 1024): the block is walked in two passes, streams
//     {0, 1} then {2, 3}; at step i of pass p team t takes slot 4i + 2p + t,
//     i.e. its stream 2p + t in ascending slot order.  At the end of pass 0
//     team 0 keeps q0 + q1 in registers; at the end of pass 1 it adds
//     q2 + q3 and writes P[b] = (q0 + q1) + (q2 + q3).
//   TEAMS = 4 (hidden <= 1024): one pass, team t on stream t.
// Team 0 receives the other teams' stream sums through LDS.  Two rows in
// flight per workgroup with several wavefronts per row, one resident
// workgroup per compute unit walking its blocks in turn, and the next rows
// prefetched PD steps ahead across pass and block boundaries measured about
// 5% faster than one row per stream (four rows in flight) on the hidden-4096
// backward, for the same arithmetic.
template <int V, int TW, int TEAMS, int PD, bool FULL, bool PLAN, bool DX, bool DW, bool RC>
__global__ __launch_bounds__(64 * TW * TEAMS) void bwd_team_kernel(BwdArgs a) {
  using Ops = RowOps<V, TW, TEAMS, FULL, DX, RC>;
  using L = typename Ops::L;
  constexpr int COLS = L::COLS;
  constexpr int WAVES = TW * TEAMS;
  constexpr int THREADS = 64 * WAVES;
  constexpr int STEPS = kBlockRows / TEAMS;   // slots a team takes per block
  constexpr int R = PD + 1;                   // row buffers in the ring
  static_assert(TEAMS == 2 || TEAMS == 4, "two or four teams");
  static_assert(STEPS % R == 0 && 16 % R == 0, "the ring must divide a pass");
  // TEAMS = 2 keeps q0 + q1 across the block's second pass: in registers,
  // or in LDS when a wavefront holds 4 or more chunk groups per row
  constexpr bool HQ_LDS = TEAMS == 2 && V >= 4;
  __shared__ float w_s[DX ? COLS : 1];
  __shared__ float q_s[DW ? (TEAMS / 2 + (HQ_LDS ? 1 : 0)) * COLS : 1];
  __shared__ float xch[Ops::XCH_FLOATS];

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int team = wv / TW;
  const int half = wv % TW;
  const int H = FULL ? COLS : a.hidden;
  const int nchunk = H >> 3;
  const int n_items = a.plan.n_items;
  const int groups = a.item_groups;

  if ((int)blockIdx.x >= groups) {
    // padding rows: dx = 0, nothing read (one row per wavefront)
    if (DX) {
      const int idx = ((int)blockIdx.x - groups) * WAVES + wv;
      if (idx < a.plan.n_pad) {
        uint16_t* d = a.dx + (int64_t)a.plan.pad_rows[idx] * H;
        for (int q = lane; q < nchunk; q += 64) store16_stream(d + q * 8, make_uint4(0, 0, 0, 0));
      }
    }
    return;
  }
  int item = blockIdx.x;
  if (item >= n_items) return;
  if (DX) stage_w<COLS, THREADS>(a, w_s, tid, nchunk);

  const L ln{lane, half, nchunk, (half * V * 64 + lane) * 8};
  const Ops ops{a, w_s, xch, ln, team, H};

  auto info_of = [&](int it, int& blk, bool& complete) {
    if (PLAN) {
      const int info = a.plan.item_info[it];
      complete = info >= 0;
      blk = complete ? info : ~info;
    } else {
      blk = it;
      complete = true;
    }
  };
  // step j of a team: pass j / 16, slot 4*(j % 16) + TEAMS*(j / 16) + team
  auto slot_of = [&](int j) { return 4 * (j & 15) + TEAMS * (j >> 4) + team; };
  // lane j (< STEPS) holds the physical row and rstd of step j; the step
  // loop reads them as scalars, so its only vector loads are the rows
  auto slots_of = [&](int it, int blk, int& sp, float& sr) {
    sp = slot_row_t<PLAN>(a, it, blk, slot_of(lane & (STEPS - 1)));
    if (!RC) sr = a.rstd[sp >= 0 ? sp : 0];
  };

  float acc[DW ? V * 8 : 1];
  float hq[(DW && TEAMS == 2 && !HQ_LDS) ? V * 8 : 1];
  // Stream sums (or their pairs) handed between teams through q_s: the
  // sending team writes, all meet at a barrier, the receiving team adds.
  auto hand = [&](int region, bool send) {
    if (send) {
#pragma unroll
      for (int k = 0; k < V; ++k) {
        float* dst = &q_s[region * COLS + ln.base + k * 512];
        store_f4(dst, acc[k * 8 + 0], acc[k * 8 + 1], acc[k * 8 + 2], acc[k * 8 + 3]);
        store_f4(dst + 4, acc[k * 8 + 4], acc[k * 8 + 5], acc[k * 8 + 6], acc[k * 8 + 7]);
      }
    }
    __syncthreads();
  };
  auto hand_own = [&](int region) {
#pragma unroll
    for (int k = 0; k < V; ++k) {
      float* dst = &q_s[region * COLS + ln.base + k * 512];
      store_f4(dst, acc[k * 8 + 0], acc[k * 8 + 1], acc[k * 8 + 2], acc[k * 8 + 3]);
      store_f4(dst + 4, acc[k * 8 + 4], acc[k * 8 + 5], acc[k * 8 + 6], acc[k * 8 + 7]);
    }
  };
  auto load_own = [&](int region, float (&h)[V * 8]) {
#pragma unroll
    for (int k = 0; k < V; ++k) {
      const float4 lo = *reinterpret_cast<const float4*>(&q_s[region * COLS + ln.base + k * 512]);
      const float4 hi = *reinterpret_cast<const float4*>(&q_s[region * COLS + ln.base + k * 512 + 4]);
      h[k * 8 + 0] = lo.x; h[k * 8 + 1] = lo.y; h[k * 8 + 2] = lo.z; h[k * 8 + 3] = lo.w;
      h[k * 8 + 4] = hi.x; h[k * 8 + 5] = hi.y; h[k * 8 + 6] = hi.z; h[k * 8 + 7] = hi.w;
    }
  };
  auto take = [&](int region) {
#pragma unroll
    for (int k = 0; k < V; ++k) {
      const float4 lo = *reinterpret_cast<const float4*>(&q_s[region * COLS + ln.base + k * 512]);
      const float4 hi = *reinterpret_cast<const float4*>(&q_s[region * COLS + ln.base + k * 512 + 4]);
      acc[k * 8 + 0] = acc[k * 8 + 0] + lo.x;
      acc[k * 8 + 1] = acc[k * 8 + 1] + lo.y;
      acc[k * 8 + 2] = acc[k * 8 + 2] + lo.z;
      acc[k * 8 + 3] = acc[k * 8 + 3] + lo.w;
      acc[k * 8 + 4] = acc[k * 8 + 4] + hi.x;
      acc[k * 8 + 5] = acc[k * 8 + 5] + hi.y;
      acc[k * 8 + 6] = acc[k * 8 + 6] + hi.z;
      acc[k * 8 + 7] = acc[k * 8 + 7] + hi.w;
    }
  };
  auto store_p = [&](int blk) {
    if (a.form != nullptr && tid == 0) a.form[blk] = 0;
    float* Pb = a.P + (int64_t)blk * H + ln.base;
#pragma unroll
    for (int k = 0; k < V; ++k) {
      if (ln.in_row(k)) {
        store_f4(Pb + k * 512, acc[k * 8 + 0], acc[k * 8 + 1], acc[k * 8 + 2], acc[k * 8 + 3]);
        store_f4(Pb + k * 512 + 4, acc[k * 8 + 4], acc[k * 8 + 5], acc[k * 8 + 6], acc[k * 8 + 7]);
      }
    }
  };
  // End of a pass over a complete block.
  //   TEAMS = 4 (streams 0..3 on teams 0..3): teams 1 and 3 hand q1, q3 to
  //     teams 0 and 2, which form q0 + q1 and q2 + q3; team 2 hands q2 + q3
  //     to team 0: P[b] = (q0 + q1) + (q2 + q3).
  //   TEAMS = 2: pass 0 (streams 0, 1): team 1 hands q1 to team 0, which
  //     keeps q0 + q1 in registers; pass 1 (streams 2, 3): team 0 forms
  //     q2 + q3 the same way and writes P[b] = (q0 + q1) + (q2 + q3).
  auto pass_end = [&](int pass, int blk) {
    if (TEAMS == 4) {
      hand(team >> 1, team & 1);
      if ((team & 1) == 0) take(team >> 1);
      hand(1, team == 2);
      if (team == 0) {
        take(1);
        store_p(blk);
      }
    } else {
      hand(0, team == 1);
      if (team == 0) {
        take(0);
        if constexpr (HQ_LDS) {
          // region 1 is written and read by this team's own lanes only
          if (pass == 0) {
            hand_own(1);
          } else {
            float h[V * 8];
            load_own(1, h);
#pragma unroll
            for (int i = 0; i < V * 8; ++i) acc[i] = h[i] + acc[i];
            store_p(blk);
          }
        } else if (pass == 0) {
#pragma unroll
          for (int i = 0; i < V * 8; ++i) hq[(TEAMS == 2) ? i : 0] = acc[i];
        } else {
#pragma unroll
          for (int i = 0; i < V * 8; ++i) acc[i] = hq[(TEAMS == 2) ? i : 0] + acc[i];
          store_p(blk);
        }
      }
    }
    __syncthreads();   // q_s is free again
#pragma unroll
    for (int i = 0; i < V * 8; ++i) acc[i] = 0.0f;
  };

  int blk, sp, nsp = -1;
  bool complete;
  float sr = 0.0f, nsr = 0.0f;
  info_of(item, blk, complete);
  slots_of(item, blk, sp, sr);
  uint4 xb[R][V], db[R][V];
#pragma unroll
  for (int j = 0; j < PD; ++j) ops.load(__builtin_amdgcn_readlane(sp, j), xb[j], db[j]);
  // consume the slot registers once here, so the compiler does not insert a
  // full wait (which would also wait for the rows in flight) in the loop
  asm volatile("" : "+v"(sp), "+v"(sr));
#pragma unroll
  for (int i = 0; i < (DW ? V * 8 : 1); ++i) acc[i] = 0.0f;

  // One block's steps.  The last PD steps issue the first rows of the
  // workgroup's next block (or, past the last one, dummy loads of row 0 that
  // keep the wait counts exact).
  auto run = [&](auto complete_tag, int nblk_more, int nxt_sp) {
    constexpr bool CPL = decltype(complete_tag)::value;
#pragma unroll
    for (int j0 = 0; j0 < STEPS; j0 += R) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int j = j0 + u;
        const int jn = j + PD;
        int pj;
        if (jn < STEPS) pj = __builtin_amdgcn_readlane(sp, jn);
        else pj = nblk_more ? __builtin_amdgcn_readlane(nxt_sp, jn - STEPS) : -1;
        ops.load(pj, xb[(u + PD) % R], db[(u + PD) % R]);
        const int p = __builtin_amdgcn_readlane(sp, j);
        const float r = RC ? 0.0f : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sr), j));
        float* srow = nullptr;
        if (DW && !CPL) srow = a.S + (spill_row0(a, item, blk) + slot_of(j)) * H + ln.base;
        ops.template row<DW, CPL>(j, p, xb[u], db[u], r, acc, srow);
        if (DW && CPL && (j & 15) == 15) pass_end(j >> 4, blk);
        // keep the scheduler from interleaving steps: the row loads are
        // already issued PD steps ahead, and moving work across steps only
        // raises register use
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  while (true) {
    const int nxt = item + groups;
    const bool more = nxt < n_items;
    int nblk = 0;
    bool ncomplete = true;
    if (more) {
      info_of(nxt, nblk, ncomplete);
      slots_of(nxt, nblk, nsp, nsr);
    }
    if (!PLAN || complete) run(std::true_type{}, more, nsp);
    else run(std::false_type{}, more, nsp);
    if (!more) break;
    item = nxt;
    blk = nblk;
    complete = ncomplete;
    sp = nsp;
    sr = nsr;
    asm volatile("" : "+v"(sp), "+v"(sr));
  }
}

// ------------------------------------------- stream-owner backward (mid-size calls)
// A call with a few dozen blocks would run the fused kernel on a few dozen
// compute units, and the two-pass path reads x and dy twice.  Here every
// fold stream of every block is a workgroup of its own: workgroup (item, w)
// walks the stream's slots w, w+4, ..., w+60 in ascending order with the
// fused kernel's per-row code -- dx of each row and the running FP32 sum of
// its contributions -- so x and dy are read once and the call fills four
// times as many compute units as it has blocks.  The stream sums are the
// fused kernel's q0..q3 bit for bit; they stay apart (q0 in P[b], q1..q3 in
// Q[b], form[b] = 1) until the finalize step forms P[b] = (q0 + q1) +
// (q2 + q3), the fused kernel's in-block tree.  A block held in part writes
// its rows' contributions to the spill rows, as on every path.  The team is
// TW wavefronts, V chunk groups each; PD rows are in flight ahead of the
// one being reduced.
template <int V, int TW, int PD, bool FULL, bool PLAN>
__global__ __launch_bounds__(64 * TW) void bwd_stream_kernel(BwdArgs a) {
  using Ops = RowOps<V, TW, 1, FULL, true, false>;
  using L = typename Ops::L;
  constexpr int COLS = L::COLS;
  constexpr int THREADS = 64 * TW;
  constexpr int R = PD + 1;                   // row buffers in the ring
  static_assert(kSlotsPerStream % R == 0, "the ring must divide the stream");
  __shared__ float w_s[COLS];
  __shared__ float xch[Ops::XCH_FLOATS];
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int H = FULL ? COLS : a.hidden;
  const int nchunk = H >> 3;
  const int n_wg = a.plan.n_items * kStreams;
  if ((int)blockIdx.x >= n_wg) {
    // padding rows: dx = 0, nothing read (one row per wavefront)
    const int idx = ((int)blockIdx.x - n_wg) * TW + wv;
    if (idx < a.plan.n_pad) {
      uint16_t* d = a.dx + (int64_t)a.plan.pad_rows[idx] * H;
      for (int q = lane; q < nchunk; q += 64) store16_stream(d + q * 8, make_uint4(0, 0, 0, 0));
    }
    return;
  }
  const int item = (int)blockIdx.x >> 2;
  const int w = (int)blockIdx.x & (kStreams - 1);
  int blk = item;
  bool complete = true;
  if (PLAN) {
    const int info = a.plan.item_info[item];
    complete = info >= 0;
    blk = complete ? info : ~info;
  }
  const L ln{lane, wv, nchunk, (wv * V * 64 + lane) * 8};
  const Ops ops{a, w_s, xch, ln, 0, H};
  // lane i (< 16) holds the physical row and rstd of the stream's step i
  const int sp = slot_row_t<PLAN>(a, item, blk, w + kStreams * (lane & (kSlotsPerStream - 1)));
  const float sr = a.rstd[sp >= 0 ? sp : 0];
  uint4 xb[R][V], db[R][V];
#pragma unroll
  for (int j = 0; j < PD; ++j) ops.load(__builtin_amdgcn_readlane(sp, j), xb[j], db[j]);
  stage_w<COLS, THREADS>(a, w_s, tid, nchunk);
  float acc[V * 8];
#pragma unroll
  for (int i = 0; i < V * 8; ++i) acc[i] = 0.0f;

  auto run = [&](auto complete_tag) {
    constexpr bool CPL = decltype(complete_tag)::value;
#pragma unroll
    for (int j0 = 0; j0 < kSlotsPerStream; j0 += R) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int j = j0 + u;
        const int jn = j + PD;
        // past the stream's end: dummy loads of row 0 keep the wait counts exact
        const int pj = jn < kSlotsPerStream ? __builtin_amdgcn_readlane(sp, jn) : -1;
        ops.load(pj, xb[(u + PD) % R], db[(u + PD) % R]);
        const int p = __builtin_amdgcn_readlane(sp, j);
        const float r = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sr), j));
        float* srow = nullptr;
        if (!CPL) srow = a.S + (spill_row0(a, item, blk) + w + kStreams * j) * H + ln.base;
        ops.template row<true, CPL>(j, p, xb[u], db[u], r, acc, srow);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if (!PLAN || complete) {
    run(std::true_type{});
    float* dst = w == 0 ? a.P + (int64_t)blk * H : a.Q + ((int64_t)blk * 3 + (w - 1)) * H;
    dst += ln.base;
#pragma unroll
    for (int k = 0; k < V; ++k) {
      if (ln.in_row(k)) {
        store_f4(dst + k * 512, acc[k * 8 + 0], acc[k * 8 + 1], acc[k * 8 + 2], acc[k * 8 + 3]);
        store_f4(dst + k * 512 + 4, acc[k * 8 + 4], acc[k * 8 + 5], acc[k * 8 + 6], acc[k * 8 + 7]);
      }
    }
    if (w == 0 && tid == 0) a.form[blk] = 1;
  } else {
    run(std::false_type{});
  }
}

// ------------------------------------------------- two-pass backward (few blocks)
// A call that touches few canonical blocks would leave most compute units
// idle in the fused kernel (one workgroup per block).  It runs two passes
// instead, with enough workgroups for the whole chip between them:
//   dx rows (dx_pair_part): dx, two rows of a work item per workgroup, one
//     per team, through the same per-row code as the fused kernel (RowOps
//     with the dweight part compiled out); the dot order does not depend on
//     the row shape, so every dx bit equals the fused kernel's;
//   dweight columns (dw_cols_part): the dweight contributions and the
//     in-block stream fold of one canonical block over 256 columns, with the
//     same operations in the same order as the fused kernel, so the block
//     partials and spill rows are bitwise the same.
// The passes are independent, so one launch (bwd_split_kernel) runs both,
// and the column pass reads x and dy a second time: the work list places
// both readers of a block on one XCD, so the second read is served from L2.

// One dx task: slots 2*pair + team of work item `item` (one row per team),
// through the fused kernel's per-row code with the dweight part compiled out.
// Work list of the two-pass launch (see bwd_split_kernel).
struct SplitMap {
  int groups;     // item groups: workgroup wg serves items wg % groups + groups * i
  int col_wg;     // column-unit workgroups per item (0: no dweight)
  int row_wg;     // dx workgroups per item, two rows each (0: no dx)
  int n_slices;   // 256-column slices of a row
  int task_wg;    // workgroups before the padding-row ones
};

// 8 groups (one per XCD) when the items spread evenly enough over them (at
// most 25% more workgroups than items would need); else 1, which spreads
// every item's tasks over the whole chip.
static int split_groups(int n_items) {
  const int g = 8;
  if (n_items < g) return 1;
  const int64_t padded = (int64_t)((n_items + g - 1) / g) * g;
  return padded * 4 <= (int64_t)n_items * 5 ? g : 1;
}

template <int V, int TW, bool FULL, bool PLAN>
__device__ __forceinline__ void dx_pair_part(const BwdArgs& a, float* w_s, float* xch, int item,
                                             int pair) {
  constexpr int TEAMS = 2;
  using Ops = RowOps<V, TW, TEAMS, FULL, true, false>;
  using L = typename Ops::L;
  constexpr int THREADS = 64 * TW * TEAMS;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int team = wv / TW;
  const int half = wv % TW;
  const int H = FULL ? L::COLS : a.hidden;
  const int nchunk = H >> 3;
  int blk = item;
  if (PLAN) {
    const int info = a.plan.item_info[item];
    blk = info >= 0 ? info : ~info;
  }
  // an absent slot (a block the call holds in part) reads row 0 and writes
  // nothing; both teams still reach the row's exchange
  const int p = slot_row_t<PLAN>(a, item, blk, TEAMS * pair + team);
  const float r = a.rstd[p >= 0 ? p : 0];
  const L ln{lane, half, nchunk, (half * V * 64 + lane) * 8};
  const Ops ops{a, w_s, xch, ln, team, H};
  uint4 xv[V], dv[V];
  ops.load(p, xv, dv);
  stage_w<L::COLS, THREADS>(a, w_s, tid, nchunk);
  float acc[1];
  ops.template row<false, true>(0, p, xv, dv, r, acc, nullptr);
}

// One column unit: the canonical block of work item `item` over the 256
// columns of `slice`, folded by 4 wavefronts starting at wavefront `w0`:
// wavefront w0 + w is stream w and lane l holds columns 4*(64*slice + l)
// .. +4 (8-byte loads).  All 16 rows of the stream are loaded before the
// fold, which then runs in slot order, so the unit waits for memory once.
// `live` false: no unit, but the barrier is still reached (the workgroup's
// other unit may need it).
template <bool PLAN>
__device__ __forceinline__ void dw_cols_part(const BwdArgs& a, float (*q_s)[256], int item, int slice,
                                             int w0, bool live) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int stream = __builtin_amdgcn_readfirstlane(tid >> 6) - w0;
  const int H = a.hidden;
  const int col = (slice * 64 + lane) * 4;   // this lane's first column (hidden % 8 == 0)
  const bool on = live && col < H;
  int blk = 0;
  bool complete = true;
  if (live) {
    if (PLAN) {
      const int info = a.plan.item_info[item];
      complete = info >= 0;
      blk = complete ? info : ~info;
    } else {
      blk = item;
    }
  }
  float acc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = 0.0f;
  if (live) {
    // lane i (< 16) holds the physical row and rstd of the stream's slot i
    const int sp = slot_row_t<PLAN>(a, item, blk, stream + kStreams * (lane & (kSlotsPerStream - 1)));
    const float sr = a.rstd[sp >= 0 ? sp : 0];
    uint2 xv[kSlotsPerStream], dv[kSlotsPerStream];
#pragma unroll
    for (int i = 0; i < kSlotsPerStream; ++i) {
      const int p = __builtin_amdgcn_readlane(sp, i);
      const int64_t off = (int64_t)(p >= 0 ? p : 0) * H + (on ? col : 0);
      xv[i] = load8_stream(a.x + off);
      dv[i] = load8_stream(a.dy + off);
    }
#pragma unroll
    for (int i = 0; i < kSlotsPerStream; ++i) {
      const int p = __builtin_amdgcn_readlane(sp, i);
      if (p < 0) continue;
      const float r = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sr), i));
      float xf[4], df[4], c[4];
      unpack4(xv[i], xf);
      unpack4(dv[i], df);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pr = df[e] * xf[e];          // exact: two bf16 significands
        c[e] = pr * r;                           // the row's contribution, rounded once
        acc[e] = acc[e] + c[e];
      }
      if (!complete && on) {
        float* srow = a.S + (spill_row0(a, item, blk) + stream + kStreams * i) * H + col;
        store_f4_stream(srow, c[0], c[1], c[2], c[3]);
      }
    }
  }
  const bool fold = live && complete;
  if (fold && stream > 0) store_f4(&q_s[stream - 1][lane * 4], acc[0], acc[1], acc[2], acc[3]);
  __syncthreads();
  if (fold && stream == 0 && on) {
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = stream_tree4(acc[e], q_s[0][lane * 4 + e], q_s[1][lane * 4 + e], q_s[2][lane * 4 + e]);
    store_f4(a.P + (int64_t)blk * H + col, o[0], o[1], o[2], o[3]);
    if (a.form != nullptr && slice == 0 && lane == 0) a.form[blk] = 0;
  }
}

// Both passes in one launch, as tasks of the call's work items: per item,
// m.col_wg workgroups of column units (TW/2 units of 256 columns each:
// wavefronts 4u .. 4u+3 take unit u) and m.row_wg workgroups of dx rows (two
// rows each).  Either list may be empty (dx alone, contributions alone).
// Workgroup wg serves item group g = wg % m.groups -- items g, g + groups,
// ... -- so with 8 groups all tasks of an item run on one XCD (the chip
// hands consecutive workgroups to its 8 XCDs in turn): the column units and
// the dx rows read the same rows of x and dy, and the second reader finds
// them in that XCD's L2.  Workgroups past m.task_wg zero padding rows.
template <int V, int TW, bool FULL, bool PLAN>
__global__ __launch_bounds__(128 * TW) void bwd_split_kernel(BwdArgs a, SplitMap m) {
  using Ops = RowOps<V, TW, 2, FULL, true, false>;
  constexpr int COLS = Ops::L::COLS;
  constexpr int UNITS = TW / 2;
  static_assert(TW % 2 == 0, "column units take four wavefronts");
  constexpr int ROWS_LDS = COLS + Ops::XCH_FLOATS;   // w, then the exchange
  constexpr int COLS_LDS = UNITS * (kStreams - 1) * 256;
  constexpr int LDS = ROWS_LDS > COLS_LDS ? ROWS_LDS : COLS_LDS;
  __shared__ float4 lds4[(LDS + 3) / 4];
  float* lds = reinterpret_cast<float*>(lds4);
  const int wg = blockIdx.x;
  if (wg >= m.task_wg) {
    // padding rows: dx = 0, nothing read (one row per wavefront)
    const int idx = (wg - m.task_wg) * 2 * TW + (int)(threadIdx.x >> 6);
    if (idx < a.plan.n_pad) {
      const int nchunk = a.hidden >> 3;
      uint16_t* d = a.dx + (int64_t)a.plan.pad_rows[idx] * a.hidden;
      for (int q = (int)(threadIdx.x & 63); q < nchunk; q += 64) store16_stream(d + q * 8, make_uint4(0, 0, 0, 0));
    }
    return;
  }
  const int per = m.col_wg + m.row_wg;
  const int k = wg / m.groups;
  const int item = wg % m.groups + m.groups * (k / per);
  const int t = k % per;
  if (item >= a.plan.n_items) return;   // the whole workgroup: no barrier is left waiting
  if (t < m.col_wg) {
    const int u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);   // the workgroup's unit
    const int slice = t * UNITS + u;
    const bool live = slice < m.n_slices;
    dw_cols_part<PLAN>(a, reinterpret_cast<float (*)[256]>(lds + u * (kStreams - 1) * 256), item,
                       live ? slice : 0, u * kStreams, live);
  } else {
    dx_pair_part<V, TW, FULL, PLAN>(a, lds, lds + COLS, item, t - m.col_wg);
  }
}

// Small rows: hidden = 8L (L in 1..32), one group of L lanes per row; the
// 64 slots' contributions go through LDS and the 4 streams fold them there.
// (Folding in registers instead -- each block's four streams on 4L lanes of
// one wavefront, the stream tree as lane shuffles, no LDS -- measured 10-14%
// slower at 128 columns: a quarter of the wavefronts in flight, each walking
// 16 rows.)
// RC: rstd rebuilt from the row in the forward's order (the same lanes, the
// same chain and group sum), so its bits are the saved rstd's.
template <int L, bool DX, bool DW, bool PACKED, bool RC>
__device__ __forceinline__ void bwd_small_block(const BwdArgs& a, int item) {
  constexpr int H = 8 * L;
  constexpr int GROUPS = 256 / L;
  constexpr int ITERS = (kBlockRows + GROUPS - 1) / GROUPS;
  __shared__ float c_s[DW ? kBlockRows * H : 1];
  __shared__ float q_s[DW ? kStreams * H : 1];
  const int tid = threadIdx.x;
  const int g = tid / L;
  const int sub = tid % L;

  if (item >= a.plan.n_items) {
    if (DX) {
      const int idx = (item - a.plan.n_items) * GROUPS + g;
      if (idx < a.plan.n_pad)
        store16_stream(a.dx + row_off<PACKED>(a.pack, a.plan.pad_rows[idx], H) + sub * 8,
                       make_uint4(0, 0, 0, 0));
    }
    return;
  }
  float wf[8];
  if (DX) unpack8(load16(a.w + sub * 8), wf);

  int blk;
  bool complete;
  if (a.plan.item_info != nullptr) {
    const int info = a.plan.item_info[item];
    complete = info >= 0;
    blk = complete ? info : ~info;
  } else {
    blk = item;
    complete = true;
  }

  // Every row of the group is loaded before any is processed (absent slots
  // read row 0 and are never used), so the block's loads are all in flight.
  int pp[ITERS];
  uint4 xv[ITERS], dv[ITERS];
  float rr[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int s = g + it * GROUPS;
    pp[it] = s < kBlockRows ? slot_row(a, item, blk, s) : -1;
  }
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int row = pp[it] >= 0 ? pp[it] : 0;
    const int64_t off = row_off<PACKED>(a.pack, row, H);
    xv[it] = load16_stream(a.x + off + sub * 8);
    dv[it] = load16_stream(a.dy + off + sub * 8);
    if (!RC) rr[it] = a.rstd[row];
  }
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int s = g + it * GROUPS;
    const int p = pp[it];
    float xf[8], df[8], pr[8];
    unpack8(p >= 0 ? xv[it] : make_uint4(0, 0, 0, 0), xf);
    unpack8(p >= 0 ? dv[it] : make_uint4(0, 0, 0, 0), df);
    float r;
    if (RC) {
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(xf[e], xf[e], ss);
      ss = group_sum<L>(ss);
      r = p >= 0 ? rsqrtf(ss / (float)H + a.eps) : 0.0f;
    } else {
      r = p >= 0 ? rr[it] : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) pr[e] = df[e] * xf[e];
    if (DX) {
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(pr[e], wf[e], dot);
      dot = group_sum<L>(dot);
      if (p >= 0) {
        const float kk = ((r * r) * r) * (dot / (float)H);
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(-xf[e], kk, r * (df[e] * wf[e]));
        store16_stream(a.dx + row_off<PACKED>(a.pack, p, H) + sub * 8, pack8(o));
      }
    }
    if (DW) {
      float c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) c[e] = pr[e] * r;   // +0.0 for slots this call lacks
      if (complete) {
        if (s < kBlockRows) {
          store_f4(&c_s[s * H + sub * 8], c[0], c[1], c[2], c[3]);
          store_f4(&c_s[s * H + sub * 8 + 4], c[4], c[5], c[6], c[7]);
        }
      } else if (p >= 0) {
        float* srow = a.S + (spill_row0(a, item, blk) + s) * H + sub * 8;
        store_f4_stream(srow, c[0], c[1], c[2], c[3]);
        store_f4_stream(srow + 4, c[4], c[5], c[6], c[7]);
      }
    }
  }
  if (DW && complete) {
    __syncthreads();
    for (int idx = tid; idx < kStreams * H; idx += 256) {
      const int w = idx / H, j = idx % H;
      float q = 0.0f;
#pragma unroll
      for (int i = 0; i < kSlotsPerStream; ++i) q = q + c_s[(w + kStreams * i) * H + j];
      q_s[w * H + j] = q;
    }
    __syncthreads();
    for (int j = tid; j < H; j += 256)
      a.P[(int64_t)blk * H + j] = stream_tree4(q_s[j], q_s[H + j], q_s[2 * H + j], q_s[3 * H + j]);
    if (a.form != nullptr && tid == 0) a.form[blk] = 0;
  }
}
template <int L, bool DX, bool DW, bool PACKED, bool RC>
__global__ __launch_bounds__(256) void bwd_small_kernel(BwdArgs a) {
  bwd_small_block<L, DX, DW, PACKED, RC>(a, blockIdx.x);
}
// Two per-head norms in one launch (dx, and dweight into their own
// accumulators or none): workgroups 0 .. wg_a-1 run norm a's items and
// padding rows, the rest norm b's, each exactly as in its own launch.
template <int L, bool DW>
__global__ __launch_bounds__(256) void bwd_small_pair_kernel(BwdArgs a, BwdArgs b, int wg_a) {
  if ((int)blockIdx.x < wg_a) bwd_small_block<L, true, DW, true, false>(a, blockIdx.x);
  else bwd_small_block<L, true, DW, true, false>(b, (int)blockIdx.x - wg_a);
}

// ----------------------------------------------------------------- finalize
// Blocks the stream-owner backward left in stream form: P[b] = (q0 + q1) +
// (q2 + q3) with q0 = P[b] and q1..q3 = Q[b], the fused kernel's in-block
// tree.  Workgroup g covers 1024 columns of block g / groups_per_block.
__global__ __launch_bounds__(256) void join_kernel(float* __restrict__ P, const float* __restrict__ Q,
                                                   const int32_t* __restrict__ form,
                                                   int groups_per_block, int H) {
  const int64_t b = blockIdx.x / groups_per_block;
  if (form[b] != 1) return;
  const int c = ((int)(blockIdx.x % groups_per_block) * 256 + (int)threadIdx.x) * 4;
  if (c >= H) return;   // hidden % 8 == 0, so c + 3 < H otherwise
  float* pb = P + b * H + c;
  const float* qb = Q + b * 3 * H + c;
  const float4 q0 = *reinterpret_cast<const float4*>(pb);
  const float4 q1 = *reinterpret_cast<const float4*>(qb);
  const float4 q2 = *reinterpret_cast<const float4*>(qb + H);
  const float4 q3 = *reinterpret_cast<const float4*>(qb + 2 * H);
  store_f4(pb, stream_tree4(q0.x, q1.x, q2.x, q3.x), stream_tree4(q0.y, q1.y, q2.y, q3.y),
           stream_tree4(q0.z, q1.z, q2.z, q3.z), stream_tree4(q0.w, q1.w, q2.w, q3.w));
}

// Partials of spilled blocks, folded from their spill rows in the same order
// as the backward kernel folds complete blocks.
__global__ __launch_bounds__(256) void rebuild_kernel(const float* __restrict__ S,
                                                      float* __restrict__ P,
                                                      const int32_t* __restrict__ blocks,
                                                      const int32_t* __restrict__ slots,
                                                      int64_t T, int H) {
  const int b = blocks[blockIdx.x];
  const int64_t srow0 = (int64_t)slots[blockIdx.x] * kBlockRows;
  const int j = blockIdx.y * 256 + threadIdx.x;
  if (j >= H) return;
  // every slot's value is loaded before the folds (absent slots, l >= T,
  // load nothing and add nothing), so the 64 loads are in flight together
  float v[kBlockRows];
#pragma unroll
  for (int s = 0; s < kBlockRows; ++s) {
    const int64_t l = (int64_t)b * kBlockRows + s;
    v[s] = l < T ? S[(srow0 + s) * H + j] : 0.0f;
  }
  float q[kStreams];
#pragma unroll
  for (int w = 0; w < kStreams; ++w) {
    float acc = 0.0f;
#pragma unroll
    for (int s = w; s < kBlockRows; s += kStreams)
      if ((int64_t)b * kBlockRows + s < T) acc = acc + v[s];
    q[w] = acc;
  }
  P[(int64_t)b * H + j] = stream_tree4(q[0], q[1], q[2], q[3]);
}

// One level of the cross-block tree: out[g] = perfect pairwise tree over the
// 512 leaves in[g*512 .. g*512+512), +0.0 past n_in.  A workgroup of 8
// wavefronts covers 32 columns: in wavefront w, the lanes of half h
// (lane / 32) reduce the aligned 32-leaf subtree 2w + h of column lane % 32 in
// registers (each load: 32 lanes x 4 bytes, one 128-byte line); the halves
// meet as h0 + h1 -- the 64-leaf subtree w -- and the 8 subtree roots meet in
// LDS in the same pairwise shape, so the result is the 512-leaf perfect tree.
constexpr int kTreeLeaves = 512;
constexpr int kTreeCols = 32;     // columns per workgroup
__global__ __launch_bounds__(512) void tree_kernel(const float* __restrict__ in, int64_t n_in,
                                                   float* __restrict__ out, int H) {
  __shared__ float root_s[8][kTreeCols];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int j = blockIdx.y * kTreeCols + (lane & 31);
  const int64_t g = blockIdx.x;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int64_t idx = g * kTreeLeaves + wv * 64 + h * 32 + i;
    v[i] = (idx < n_in && j < H) ? in[idx * H + j] : 0.0f;
  }
#pragma unroll
  for (int st = 1; st < 32; st *= 2)
#pragma unroll
    for (int i = 0; i < 32; i += 2 * st) v[i] = v[i] + v[i + st];
  // half 0 ends with h0 + h1; half 1's sum is unused
  const float r = v[0] + __shfl_xor(v[0], 32, 64);
  if (h == 0) root_s[wv][lane] = r;
  __syncthreads();
  if (wv == 0 && h == 0 && j < H) {
    const float r01 = root_s[0][lane] + root_s[1][lane], r23 = root_s[2][lane] + root_s[3][lane];
    const float r45 = root_s[4][lane] + root_s[5][lane], r67 = root_s[6][lane] + root_s[7][lane];
    out[g * H + j] = (r01 + r23) + (r45 + r67);
  }
}

__global__ void fill_zero_kernel(float* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// ----------------------------------------------------------------- copy
// A plain streaming copy in the shape that moves data fastest here: one
// 16-byte unit per thread, each workgroup reading and writing its 4 KB once
// (many short workgroups keep the access stream in address order).
__global__ __launch_bounds__(256) void stream_copy_kernel(const uint4* __restrict__ src,
                                                          uint4* __restrict__ dst, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    store16_stream(&dst[i], load16_stream(&src[i]));
}

// ----------------------------------------------------------------- dispatch
static int small_lanes(int hidden) {
  switch (hidden) {
    case 8: return 1;
    case 16: return 2;
    case 32: return 4;
    case 64: return 8;
    case 128: return 16;
    case 256: return 32;
    default: return 0;
  }
}

bool hidden_supported(int hidden) {
  return hidden > 0 && hidden % 8 == 0 && hidden <= kMaxHidden;
}

bool packed_hidden_supported(int hidden) { return small_lanes(hidden) != 0; }

// Forward row shape: one wavefront per row up to 1024 columns, two above.
static int fwd_tw(int hidden) { return hidden <= 1024 ? 1 : 2; }
static int fwd_v(int hidden) {
  const int per = 512 * fwd_tw(hidden);
  return (hidden + per - 1) / per;
}

// Backward shapes, by the number of 512-column chunk groups K of a row
// (chunk groups per wavefront V, wavefronts per row TW, rows in flight per
// workgroup TEAMS, rows prefetched ahead PD).  The shape decides only how
// the row's fixed arithmetic is spread over the hardware: no output bit
// depends on it.  Measured on MI355X (one call, x and dy 0.5-1.2 GB): at
// 4096 columns two rows in flight per workgroup, four wavefronts each, one
// resident workgroup per compute unit, beat four rows in flight by 5%; at
// 5120 and 8192 columns four rows in flight of two wavefronts each beat two
// rows of four or five wavefronts by 1-5% (5120 padded and permuted: two
// rows in flight 3.5% slower, three chunk groups on four wavefronts 2%
// slower, no prefetch ring the same; 8192: four chunk groups on four
// wavefronts or two on eight 5% slower, four teams of four wavefronts
// without a ring the same).
struct BwdShape {
  int v, tw, teams, pd;
};
static BwdShape fused_shape(int hidden) {
  const int K = (hidden + 511) / 512;
  if (K <= 1) return {1, 1, 4, 1};
  if (K <= 2) return {1, 2, 4, 1};
  if (K <= 4) return {1, 4, 2, 1};
  if (K <= 8) return {2, 4, 2, 1};
  if (K <= 10) return {5, 2, 4, 1};
  if (K <= 16) return {8, 2, 4, 1};
  return {10, 2, 4, 0};
}
// The rstd-recompute backward keeps the row for a second pass (the
// contributions wait for rstd): above 4096 columns it keeps no prefetch
// ring, and above 8192 it runs two teams of four wavefronts.
static BwdShape recompute_shape(int hidden) {
  const int K = (hidden + 511) / 512;
  if (K <= 8) return fused_shape(hidden);
  if (K <= 10) return {5, 2, 4, 0};
  if (K <= 16) return {8, 2, 4, 0};
  return {5, 4, 2, 0};
}
// The dx rows of the two-pass path: two teams of two wavefronts, so a
// workgroup is one 4-wavefront column unit or two dx rows.  Against four
// wavefronts per row (the earlier shape) this is 12% faster on 512-row
// chunks at 8192 columns, 18% at 4096 and 7% on B=1 samples at 5120: the
// tasks are latency chains, and smaller workgroups start sooner.
static BwdShape split_shape(int hidden) {
  const int K = (hidden + 511) / 512;
  if (K <= 2) return {1, 2, 2, 0};
  if (K <= 4) return {2, 2, 2, 0};
  if (K <= 8) return {4, 2, 2, 0};
  if (K <= 10) return {5, 2, 2, 0};
  if (K <= 16) return {8, 2, 2, 0};
  return {10, 2, 2, 0};
}

const char* fwd_variant(int hidden) {
  return small_lanes(hidden) ? "fwd_small(lanes_per_row=hidden/8)"
         : fwd_tw(hidden) == 1 ? "fwd_rows(wave_per_row, 4 rows per workgroup)"
                               : "fwd_rows(two_waves_per_row, 2 rows per workgroup)";
}
const char* bwd_variant(int hidden) {
  if (small_lanes(hidden)) return "bwd_small(lds_fold, streams=4)";
  return fused_shape(hidden).teams == 4
             ? "bwd_team(one pass, 4 teams x 1 row, streams=4; few blocks: dx_rows + dw_cols)"
             : "bwd_team(two passes, 2 teams x 1 row, streams=4; few blocks: dx_rows + dw_cols)";
}

static int grid_cap() { return 256 * 16; }

hipError_t launch_stream_copy(const void* src, void* dst, int64_t n16, hipStream_t st) {
  if (n16 <= 0) return hipSuccess;
  int64_t g = (n16 + 255) / 256;
  if (g > (int64_t(1) << 30)) g = int64_t(1) << 30;   // larger copies loop
  stream_copy_kernel<<<dim3((unsigned)g), dim3(256), 0, st>>>(static_cast<const uint4*>(src),
                                                                static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

// rows < 2^31 (checked at the C-ABI), so the grid always fits.
template <int V, int TW>
static void fwd_row_go(const FwdArgs& a, hipStream_t st) {
  constexpr int RPW = 4 / TW;
  const dim3 grid((unsigned)((a.rows + RPW - 1) / RPW)), block(256);
  const bool full = a.hidden == 512 * V * TW, pad = a.row_logical != nullptr;
  if (full && !pad) fwd_row_kernel<V, TW, true, false><<<grid, block, 0, st>>>(a);
  else if (full) fwd_row_kernel<V, TW, true, true><<<grid, block, 0, st>>>(a);
  else if (!pad) fwd_row_kernel<V, TW, false, false><<<grid, block, 0, st>>>(a);
  else fwd_row_kernel<V, TW, false, true><<<grid, block, 0, st>>>(a);
}
static bool is_packed(const RowPacking& pk, int hidden) {
  return pk.heads > 1 || (pk.token_stride != 0 && pk.token_stride != hidden);
}

template <int L>
static void fwd_small_go(const FwdArgs& a, hipStream_t st) {
  constexpr int GROUPS = 256 / L;
  int64_t g = (a.rows + GROUPS - 1) / GROUPS;
  if (g > grid_cap()) g = grid_cap();
  if (is_packed(a.pack, a.hidden))
    fwd_small_kernel<L, true><<<dim3((unsigned)g), dim3(256), 0, st>>>(a);
  else
    fwd_small_kernel<L, false><<<dim3((unsigned)g), dim3(256), 0, st>>>(a);
}

template <int L>
static void fwd_small_pair_go(const FwdArgs& a, const FwdArgs& b, hipStream_t st) {
  constexpr int GROUPS = 256 / L;
  auto groups = [](const FwdArgs& x) {
    const int64_t g = (x.rows + GROUPS - 1) / GROUPS;
    return g > grid_cap() ? (int64_t)grid_cap() : g;
  };
  const int64_t ga = groups(a), gb = groups(b);
  if (ga + gb == 0) return;
  fwd_small_pair_kernel<L><<<dim3((unsigned)(ga + gb)), dim3(256), 0, st>>>(a, b, (int)ga);
}

hipError_t launch_fwd_pair(const FwdArgs& a, const FwdArgs& b, hipStream_t st) {
  if (a.hidden != b.hidden) return hipErrorInvalidValue;
  switch (small_lanes(a.hidden)) {
    case 1: fwd_small_pair_go<1>(a, b, st); break;
    case 2: fwd_small_pair_go<2>(a, b, st); break;
    case 4: fwd_small_pair_go<4>(a, b, st); break;
    case 8: fwd_small_pair_go<8>(a, b, st); break;
    case 16: fwd_small_pair_go<16>(a, b, st); break;
    case 32: fwd_small_pair_go<32>(a, b, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  if (is_packed(a.pack, a.hidden) && !packed_hidden_supported(a.hidden)) return hipErrorInvalidValue;
  switch (small_lanes(a.hidden)) {
    case 1: fwd_small_go<1>(a, st); return hipGetLastError();
    case 2: fwd_small_go<2>(a, st); return hipGetLastError();
    case 4: fwd_small_go<4>(a, st); return hipGetLastError();
    case 8: fwd_small_go<8>(a, st); return hipGetLastError();
    case 16: fwd_small_go<16>(a, st); return hipGetLastError();
    case 32: fwd_small_go<32>(a, st); return hipGetLastError();
    default: break;
  }
  // fwd_tw wavefronts per row, fwd_v chunks per lane
  const int V = fwd_v(a.hidden);
  if (fwd_tw(a.hidden) == 1) {
    switch (V) {
      case 1: fwd_row_go<1, 1>(a, st); break;
      case 2: fwd_row_go<2, 1>(a, st); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (V) {
#define RBI_FWD(v) case v: fwd_row_go<v, 2>(a, st); break;
      RBI_FWD(1) RBI_FWD(2) RBI_FWD(3) RBI_FWD(4) RBI_FWD(5) RBI_FWD(6) RBI_FWD(7) RBI_FWD(8)
      RBI_FWD(9) RBI_FWD(10)
#undef RBI_FWD
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

// Calls touching fewer canonical blocks than this take the two-pass path
// (host-side setting, guarded by a mutex).
static std::mutex g_split_mu;
static int64_t g_split_items = kDefaultSplitItems;

void set_split_items(int64_t n) {
  std::lock_guard<std::mutex> lk(g_split_mu);
  g_split_items = n < 0 ? kDefaultSplitItems : n;
}
int64_t split_items() {
  std::lock_guard<std::mutex> lk(g_split_mu);
  return g_split_items;
}
static int64_t g_stream_items = kDefaultStreamItems;
void set_stream_items(int64_t n) {
  std::lock_guard<std::mutex> lk(g_split_mu);
  g_stream_items = n < 0 ? kDefaultStreamItems : n;
}
int64_t stream_items() {
  std::lock_guard<std::mutex> lk(g_split_mu);
  return g_stream_items;
}
static int64_t g_group_cap = 0;
void set_wide_group_cap(int64_t n) {
  std::lock_guard<std::mutex> lk(g_split_mu);
  g_group_cap = n < 0 ? 0 : n;
}
int64_t wide_group_cap() {
  std::lock_guard<std::mutex> lk(g_split_mu);
  return g_group_cap;
}

// Workgroups of the fused backward: one per work item, capped at the number
// the chip holds at once (occupancy x compute units), so with more items
// every workgroup stays resident and loops over its share.
static int compute_units() {
  static std::mutex mu;
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// Workgroups of the fused backward: one per work item, capped so that the
// workgroups walk their share of the items in turn -- one per compute unit
// with two teams (two resident workgroups per compute unit were about 4%
// slower at hidden 4096), two with four teams, and at least 8 wavefronts
// per compute unit.  With four teams the second workgroup of a compute
// unit may not fit beside the first (above 128 VGPRs); capping at what
// fits was 3.5% slower at hidden 8192 (1169 blocks): more, shorter
// workgroups balance the tail better.  Which workgroup takes an item
// changes nothing in its arithmetic.
template <int V, int TW, int TEAMS, int PD, bool FULL, bool PLAN, bool DX, bool DW, bool RC>
static void bwd_team_launch(BwdArgs a, hipStream_t st) {
  constexpr int WAVES = TW * TEAMS;
  const int64_t knob = wide_group_cap();
  const int64_t per_cu = (TEAMS == 2 ? 1 : 2) * (WAVES >= 8 ? 1 : 8 / WAVES);
  const int64_t cap = knob > 0 ? knob : per_cu * compute_units();
  a.item_groups = (int32_t)(a.plan.n_items > cap ? cap : a.plan.n_items);
  // padding rows get workgroups of their own after the item workgroups
  // (zeroing them inside the item workgroups, beside the next item's loads,
  // measured the same on the hidden-5120 padded layout)
  const int pad_groups = DX ? (a.plan.n_pad + WAVES - 1) / WAVES : 0;
  if (a.item_groups + pad_groups == 0) return;
  const dim3 grid((unsigned)(a.item_groups + pad_groups)), block(64 * WAVES);
  bwd_team_kernel<V, TW, TEAMS, PD, FULL, PLAN, DX, DW, RC><<<grid, block, 0, st>>>(a);
}

template <int V, int TW, int TEAMS, int PD, bool RC, bool FULL, bool PLAN>
static void bwd_team_go3(const BwdArgs& a, bool dx, bool dw, hipStream_t st) {
  if constexpr (RC) {
    if (dw) bwd_team_launch<V, TW, TEAMS, PD, FULL, PLAN, true, true, true>(a, st);
    else bwd_team_launch<V, TW, TEAMS, PD, FULL, PLAN, true, false, true>(a, st);
  } else {
    if (dx && dw) bwd_team_launch<V, TW, TEAMS, PD, FULL, PLAN, true, true, false>(a, st);
    else if (dx) bwd_team_launch<V, TW, TEAMS, PD, FULL, PLAN, true, false, false>(a, st);
    else bwd_team_launch<V, TW, TEAMS, PD, FULL, PLAN, false, true, false>(a, st);
  }
}
// RC: the shape serves the rstd-recompute backward (only its instances are
// built); otherwise the saved-rstd one.  With a layout plan a kernel carries
// the spill path next to the fold, and a row narrower than the shape carries
// the lane masks: at 8 or more chunk groups per wavefront the prefetch ring
// would not fit the register file beside either.
template <int V, int TW, int TEAMS, int PD, bool RC>
static void bwd_team_go(const BwdArgs& a, bool dx, bool dw, hipStream_t st) {
  constexpr int PD_LEAN = V >= 8 ? 0 : PD;
  const bool plan = a.plan.item_info != nullptr;
  if constexpr (512 * V * TW <= kMaxHidden) {
    if (a.hidden == 512 * V * TW) {
      if (plan) bwd_team_go3<V, TW, TEAMS, PD_LEAN, RC, true, true>(a, dx, dw, st);
      else bwd_team_go3<V, TW, TEAMS, PD, RC, true, false>(a, dx, dw, st);
      return;
    }
  }
  if (plan) bwd_team_go3<V, TW, TEAMS, PD_LEAN, RC, false, true>(a, dx, dw, st);
  else bwd_team_go3<V, TW, TEAMS, PD_LEAN, RC, false, false>(a, dx, dw, st);
}

template <int V, int TW, bool FULL, bool PLAN>
static void bwd_split_go2(const BwdArgs& a, bool dx, bool dw, hipStream_t st) {
  constexpr int UNITS = TW / 2;
  const int n = a.plan.n_items;
  SplitMap m;
  m.n_slices = (a.hidden + 255) / 256;
  m.col_wg = dw ? (m.n_slices + UNITS - 1) / UNITS : 0;
  m.row_wg = dx ? kBlockRows / 2 : 0;
  m.groups = split_groups(n);
  const int64_t per_group = (n + m.groups - 1) / m.groups;
  m.task_wg = (int)(m.groups * per_group * (m.col_wg + m.row_wg));
  const int pad_wg = dx ? (a.plan.n_pad + 2 * TW - 1) / (2 * TW) : 0;
  if (m.task_wg + pad_wg == 0) return;
  bwd_split_kernel<V, TW, FULL, PLAN><<<dim3((unsigned)(m.task_wg + pad_wg)), dim3(128 * TW), 0, st>>>(a, m);
}
template <int V, int TW>
static void bwd_split_go(const BwdArgs& a, bool dx, bool dw, hipStream_t st) {
  const bool full = a.hidden == 512 * V * TW, plan = a.plan.item_info != nullptr;
  if (full && plan) bwd_split_go2<V, TW, true, true>(a, dx, dw, st);
  else if (full) bwd_split_go2<V, TW, true, false>(a, dx, dw, st);
  else if (plan) bwd_split_go2<V, TW, false, true>(a, dx, dw, st);
  else bwd_split_go2<V, TW, false, false>(a, dx, dw, st);
}

// Stream-owner shape by chunk groups K: one chunk group per wavefront up to
// 16 groups (a whole row per workgroup of K wavefronts, rounded up to a
// shape that is built), two above; 3 rows in flight ahead of the one being
// reduced, 7 at up to 4096 columns (measured at 4096: 7 ahead beat 3 by 2%
// and 1 by 11%; two chunk groups per wavefront on half the wavefronts lost
// 1-3%).
static BwdShape stream_shape(int hidden) {
  const int k = (hidden + 511) / 512;
  if (k <= 2) return {1, 2, 1, 3};
  if (k <= 4) return {1, 4, 1, 3};
  if (k <= 8) return {1, 8, 1, 7};
  if (k <= 10) return {1, 10, 1, 3};
  if (k <= 12) return {1, 12, 1, 3};
  if (k <= 16) return {1, 16, 1, 3};
  return {2, 10, 1, 3};
}
template <int V, int TW, int PD, bool FULL, bool PLAN>
static void bwd_stream_go2(const BwdArgs& a, hipStream_t st) {
  const int64_t wg = (int64_t)a.plan.n_items * kStreams + (a.plan.n_pad + TW - 1) / TW;
  bwd_stream_kernel<V, TW, PD, FULL, PLAN><<<dim3((unsigned)wg), dim3(64 * TW), 0, st>>>(a);
}
template <int V, int TW, int PD>
static void bwd_stream_go(const BwdArgs& a, hipStream_t st) {
  const bool full = a.hidden == 512 * V * TW, plan = a.plan.item_info != nullptr;
  if (full && plan) bwd_stream_go2<V, TW, PD, true, true>(a, st);
  else if (full) bwd_stream_go2<V, TW, PD, true, false>(a, st);
  else if (plan) bwd_stream_go2<V, TW, PD, false, true>(a, st);
  else bwd_stream_go2<V, TW, PD, false, false>(a, st);
}

BwdPath bwd_path(const BwdArgs& a, bool dx, bool dw, bool rc) {
  if (small_lanes(a.hidden) != 0) return BwdPath::kSmall;
  if (rc) return BwdPath::kFused;
  const int64_t n = a.plan.n_items;
  if (n >= split_items()) return BwdPath::kFused;
  if (dx && dw && a.Q != nullptr && a.form != nullptr && n >= stream_items() && n > 0 &&
      !is_packed(a.pack, a.hidden))
    return BwdPath::kStream;
  return BwdPath::kSplit;
}

template <int L>
static void bwd_small_go(const BwdArgs& a, bool dx, bool dw, bool rc, hipStream_t st) {
  constexpr int GROUPS = 256 / L;
  const int pad_groups = dx ? (a.plan.n_pad + GROUPS - 1) / GROUPS : 0;
  const dim3 grid((unsigned)(a.plan.n_items + pad_groups)), block(256);
  if (rc) {   // contiguous rows only (the packed entry points read the saved rstd)
    if (dw) bwd_small_kernel<L, true, true, false, true><<<grid, block, 0, st>>>(a);
    else bwd_small_kernel<L, true, false, false, true><<<grid, block, 0, st>>>(a);
  } else if (is_packed(a.pack, a.hidden)) {
    if (dx && dw) bwd_small_kernel<L, true, true, true, false><<<grid, block, 0, st>>>(a);
    else if (dx) bwd_small_kernel<L, true, false, true, false><<<grid, block, 0, st>>>(a);
    else bwd_small_kernel<L, false, true, true, false><<<grid, block, 0, st>>>(a);
  } else {
    if (dx && dw) bwd_small_kernel<L, true, true, false, false><<<grid, block, 0, st>>>(a);
    else if (dx) bwd_small_kernel<L, true, false, false, false><<<grid, block, 0, st>>>(a);
    else bwd_small_kernel<L, false, true, false, false><<<grid, block, 0, st>>>(a);
  }
}

template <int L>
static void bwd_small_pair_go(const BwdArgs& a, const BwdArgs& b, bool dw, hipStream_t st) {
  constexpr int GROUPS = 256 / L;
  const int wa = a.plan.n_items + (a.plan.n_pad + GROUPS - 1) / GROUPS;
  const int wb = b.plan.n_items + (b.plan.n_pad + GROUPS - 1) / GROUPS;
  if (wa + wb == 0) return;
  const dim3 grid((unsigned)(wa + wb)), block(256);
  if (dw) bwd_small_pair_kernel<L, true><<<grid, block, 0, st>>>(a, b, wa);
  else bwd_small_pair_kernel<L, false><<<grid, block, 0, st>>>(a, b, wa);
}

hipError_t launch_bwd_pair(const BwdArgs& a, bool dw_a, const BwdArgs& b, bool dw_b,
                           hipStream_t st) {
  if (a.hidden != b.hidden || small_lanes(a.hidden) == 0) return hipErrorInvalidValue;
  if (dw_a != dw_b) {
    // one norm with an accumulator and one without: two launches
    hipError_t e = launch_bwd(a, true, dw_a, st);
    return e != hipSuccess ? e : launch_bwd(b, true, dw_b, st);
  }
  switch (small_lanes(a.hidden)) {
    case 1: bwd_small_pair_go<1>(a, b, dw_a, st); break;
    case 2: bwd_small_pair_go<2>(a, b, dw_a, st); break;
    case 4: bwd_small_pair_go<4>(a, b, dw_a, st); break;
    case 8: bwd_small_pair_go<8>(a, b, dw_a, st); break;
    case 16: bwd_small_pair_go<16>(a, b, dw_a, st); break;
    case 32: bwd_small_pair_go<32>(a, b, dw_a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, bool dx, bool dw, hipStream_t st, bool rc) {
  if (rc && (!dx || is_packed(a.pack, a.hidden))) return hipErrorInvalidValue;
  if (is_packed(a.pack, a.hidden) && !packed_hidden_supported(a.hidden)) return hipErrorInvalidValue;
  const int pads = dx ? a.plan.n_pad : 0;
  if (a.plan.n_items + pads == 0) return hipSuccess;
  switch (small_lanes(a.hidden)) {
    case 1: bwd_small_go<1>(a, dx, dw, rc, st); return hipGetLastError();
    case 2: bwd_small_go<2>(a, dx, dw, rc, st); return hipGetLastError();
    case 4: bwd_small_go<4>(a, dx, dw, rc, st); return hipGetLastError();
    case 8: bwd_small_go<8>(a, dx, dw, rc, st); return hipGetLastError();
    case 16: bwd_small_go<16>(a, dx, dw, rc, st); return hipGetLastError();
    case 32: bwd_small_go<32>(a, dx, dw, rc, st); return hipGetLastError();
    default: break;
  }
  const BwdPath path = bwd_path(a, dx, dw, rc);
  if (path == BwdPath::kStream) {
    const BwdShape s = stream_shape(a.hidden);
    switch (s.v * 32 + s.tw) {
      case 1 * 32 + 2: bwd_stream_go<1, 2, 3>(a, st); break;
      case 1 * 32 + 4: bwd_stream_go<1, 4, 3>(a, st); break;
      case 1 * 32 + 8: bwd_stream_go<1, 8, 7>(a, st); break;
      case 1 * 32 + 10: bwd_stream_go<1, 10, 3>(a, st); break;
      case 1 * 32 + 12: bwd_stream_go<1, 12, 3>(a, st); break;
      case 1 * 32 + 16: bwd_stream_go<1, 16, 3>(a, st); break;
      case 2 * 32 + 10: bwd_stream_go<2, 10, 3>(a, st); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (path == BwdPath::kSplit) {
    const BwdShape s = split_shape(a.hidden);
    switch (s.v * 16 + s.tw) {
      case 1 * 16 + 2: bwd_split_go<1, 2>(a, dx, dw, st); break;
      case 2 * 16 + 2: bwd_split_go<2, 2>(a, dx, dw, st); break;
      case 4 * 16 + 2: bwd_split_go<4, 2>(a, dx, dw, st); break;
      case 5 * 16 + 2: bwd_split_go<5, 2>(a, dx, dw, st); break;
      case 8 * 16 + 2: bwd_split_go<8, 2>(a, dx, dw, st); break;
      case 10 * 16 + 2: bwd_split_go<10, 2>(a, dx, dw, st); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (rc) {
    const BwdShape s = recompute_shape(a.hidden);
    switch (s.v * 16 + s.tw) {
      case 1 * 16 + 1: bwd_team_go<1, 1, 4, 1, true>(a, dx, dw, st); break;
      case 1 * 16 + 2: bwd_team_go<1, 2, 4, 1, true>(a, dx, dw, st); break;
      case 1 * 16 + 4: bwd_team_go<1, 4, 2, 1, true>(a, dx, dw, st); break;
      case 2 * 16 + 4: bwd_team_go<2, 4, 2, 1, true>(a, dx, dw, st); break;
      case 5 * 16 + 2: bwd_team_go<5, 2, 4, 0, true>(a, dx, dw, st); break;
      case 8 * 16 + 2: bwd_team_go<8, 2, 4, 0, true>(a, dx, dw, st); break;
      case 5 * 16 + 4: bwd_team_go<5, 4, 2, 0, true>(a, dx, dw, st); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const BwdShape s = fused_shape(a.hidden);
  switch (s.v * 16 + s.tw) {
    case 1 * 16 + 1: bwd_team_go<1, 1, 4, 1, false>(a, dx, dw, st); break;
    case 1 * 16 + 2: bwd_team_go<1, 2, 4, 1, false>(a, dx, dw, st); break;
    case 1 * 16 + 4: bwd_team_go<1, 4, 2, 1, false>(a, dx, dw, st); break;
    case 2 * 16 + 4: bwd_team_go<2, 4, 2, 1, false>(a, dx, dw, st); break;
    case 5 * 16 + 2: bwd_team_go<5, 2, 4, 1, false>(a, dx, dw, st); break;
    case 8 * 16 + 2: bwd_team_go<8, 2, 4, 1, false>(a, dx, dw, st); break;
    case 10 * 16 + 2: bwd_team_go<10, 2, 4, 0, false>(a, dx, dw, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_join(float* P, const float* Q, const int32_t* form, int64_t nb, int32_t hidden,
                       hipStream_t st) {
  if (nb == 0) return hipSuccess;
  const int per = (hidden + 1023) / 1024;
  join_kernel<<<dim3((unsigned)(nb * per)), dim3(256), 0, st>>>(P, Q, form, per, hidden);
  return hipGetLastError();
}

hipError_t launch_rebuild(const float* S, float* P, const int32_t* blocks, const int32_t* slots,
                          int32_t n_blocks, int64_t n_logical, int32_t hidden, hipStream_t st) {
  if (n_blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)n_blocks, (unsigned)((hidden + 255) / 256));
  rebuild_kernel<<<grid, dim3(256), 0, st>>>(S, P, blocks, slots, n_logical, hidden);
  return hipGetLastError();
}

int64_t tree_scratch_rows(int64_t nb) {
  const int64_t a = (nb + kTreeLeaves - 1) / kTreeLeaves;
  const int64_t b = (a + kTreeLeaves - 1) / kTreeLeaves;
  return a + b;
}

hipError_t launch_tree(const float* P, int64_t nb, float* tmp, float* dweight, int32_t hidden,
                       hipStream_t st) {
  const unsigned gy = (unsigned)((hidden + kTreeCols - 1) / kTreeCols);
  if (nb == 0) {
    fill_zero_kernel<<<dim3((unsigned)((hidden + 255) / 256)), dim3(256), 0, st>>>(dweight, hidden);
    return hipGetLastError();
  }
  // ping-pong between two scratch regions sized for the first two levels
  const int64_t rows_a = (nb + kTreeLeaves - 1) / kTreeLeaves;
  float* buf[2] = {tmp, tmp + rows_a * hidden};
  const float* in = P;
  int64_t n = nb;
  int which = 0;
  while (true) {
    const int64_t groups = (n + kTreeLeaves - 1) / kTreeLeaves;
    float* out = groups == 1 ? dweight : buf[which];
    tree_kernel<<<dim3((unsigned)groups, gy), dim3(512), 0, st>>>(in, n, out, hidden);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (groups == 1) break;
    in = out;
    n = groups;
    which ^= 1;
  }
  return hipSuccess;
}

}  // namespace rbi
