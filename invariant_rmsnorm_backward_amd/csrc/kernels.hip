// kernels.hip -- gfx950 kernels of batch-invariant RMSNorm.
//
// Forward: the backward's row shape -- one wavefront per row up to 1024
// columns, two above -- with 2 or 4 rows per workgroup (hidden >= 512, or any
// hidden that is not a power of two below 512), or one group of hidden/8
// lanes per row (hidden in {8..256}); streaming 16-byte bf16 loads and
// stores, FP32 math, DPP wavefront sums of squares.
//
// Backward: one workgroup per canonical block of 64 logical rows.  The
// dweight order (CDO-v1, following "WS1 C4 (#270) closeout evidence":
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

// hidden = 8L with L lanes per row (L in 1..32, a power of two).
template <int L, bool PACKED>
__global__ __launch_bounds__(256) void fwd_small_kernel(FwdArgs a) {
  constexpr int H = 8 * L;
  constexpr int GROUPS = 256 / L;
  const int g = threadIdx.x / L;
  const int sub = threadIdx.x % L;
  float wf[8];
  unpack8(load16(a.w + sub * 8), wf);
  for (int64_t base = (int64_t)blockIdx.x * GROUPS; base < a.rows;
       base += (int64_t)gridDim.x * GROUPS) {
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

// Wide rows: V chunks of 8 columns per lane, TW wavefronts per row, 4
// streams; the workgroup is 4*TW wavefronts.  Chunk q of the row held by
// lane `lane` of wave-part `half` at step k is q = (half*V + k)*64 + lane.
// FULL means hidden == 512*V*TW exactly, so no lane needs a bounds mask.
template <int V, int TW, bool FULL>
struct WideShape {
  static constexpr int S = kStreams;               // fold streams
  static constexpr int SLOTS = kSlotsPerStream;    // slots per stream
  static constexpr int WAVES = S * TW;             // wavefronts per workgroup
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int COLS = 512 * V * TW;        // columns the workgroup covers
  static constexpr int NTILE = (V * TW + 1) / 2;   // 1024-column tiles of the stream tree
};

// w as FP32 in LDS; columns past hidden hold 0 so masked lanes read zeros.
template <typename Sh>
__device__ __forceinline__ void stage_w(const BwdArgs& a, float* w_s, int tid, int nchunk) {
  for (int q = tid; q < Sh::COLS / 8; q += Sh::THREADS) {
    float f[8];
    unpack8(q < nchunk ? load16(a.w + q * 8) : make_uint4(0, 0, 0, 0), f);
    store_f4(&w_s[q * 8], f[0], f[1], f[2], f[3]);
    store_f4(&w_s[q * 8 + 4], f[4], f[5], f[6], f[7]);
  }
  __syncthreads();
}

// One canonical block: the stream's slots in ascending order.  COMPLETE: the
// call holds every present row of the block, so the contributions are folded
// in registers; otherwise they are written to the spill rows.  When two row
// buffers fit in registers the loop is software-pipelined: the next slot's
// row is loaded before the current row's reduction and dx pass.
// RC: rstd is not read but rebuilt from the row in the forward's order (the
// chunk chains, one wavefront sum per 64-chunk group, the padded pairwise
// tree over the groups; the TW wavefronts of a row swap their group sums
// through LDS), so its bits are the saved rstd's; the contributions then
// wait for it.
template <int V, int TW, bool FULL, bool PLAN, bool DX, bool DW, bool COMPLETE, bool RC = false>
struct WideBlock {
  using Sh = WideShape<V, TW, FULL>;
  const BwdArgs& a;
  int item, blk, stream, half, lane, wv, H, nchunk, base;
  const float* w_s;
  float* dot_s;
  float (&acc)[DW ? V * 8 : 1];
  float* ss_s = nullptr;
  // Lane j (< SLOTS) holds the physical row of this stream's slot j and its
  // rstd, loaded once per block; the row loop reads them as scalars, so the
  // only vector loads in the loop are the row data (in-order waits stay
  // precise and the next row's loads stay in flight).
  int slot_p = -1;
  float slot_r = 0.0f;

  __device__ __forceinline__ void load_slots() {
    // every lane loads (lanes past SLOTS repeat a slot): no divergent memory ops
    slot_p = slot_row_t<PLAN>(a, item, blk, stream + Sh::S * (lane & (Sh::SLOTS - 1)));
    if (!RC) slot_r = a.rstd[slot_p >= 0 ? slot_p : 0];
  }
  // Consume both slot registers before the row loop: the compiler then waits
  // for their loads once, instead of inserting a full vmcnt(0) wait inside
  // the loop (which would also wait for the prefetched row).  Called after
  // the first row's loads are issued, so that row is in flight meanwhile.
  __device__ __forceinline__ void settle_slots() { asm volatile("" : "+v"(slot_p), "+v"(slot_r)); }
  __device__ __forceinline__ int row_of(int i) const { return __builtin_amdgcn_readlane(slot_p, i); }
  __device__ __forceinline__ float rstd_of(int i) const {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(slot_r), i));
  }

  __device__ __forceinline__ bool in_row(int k) const {
    return FULL || (half * V + k) * 64 + lane < nchunk;
  }

  // The loads are issued whether or not the slot is present (an absent slot
  // reads row 0 and its data is never used): with the same number of memory
  // operations on every path, the compiler's wait counts stay exact and the
  // next row's loads remain in flight while the current row is processed.
  __device__ __forceinline__ void load(int p, uint4 (&xv)[V], uint4 (&dv)[V]) const {
    const int row = p >= 0 ? p : 0;
    const uint16_t* xr = a.x + (int64_t)row * H + base;
    const uint16_t* dr = a.dy + (int64_t)row * H + base;
#pragma unroll
    for (int k = 0; k < V; ++k) {
      xv[k] = in_row(k) ? load16_stream(xr + k * 512) : make_uint4(0, 0, 0, 0);
      dv[k] = in_row(k) ? load16_stream(dr + k * 512) : make_uint4(0, 0, 0, 0);
    }
  }

  __device__ __forceinline__ void process(int i, int p, uint4 (&xv)[V], uint4 (&dv)[V], float r) {
    const int s = stream + Sh::S * i;
    float dot = 0.0f, ss = 0.0f;
    // RC: the chunk chains of the forward's sum of squares; chunk k of this
    // lane is lane `lane` of chunk group half*V + k
    float sq[RC ? V : 1];
#pragma unroll
    for (int k = 0; k < (RC ? V : 1); ++k) sq[k] = 0.0f;
    if (p >= 0) {
      float* srow = COMPLETE ? nullptr : a.S + ((int64_t)blk * kBlockRows + s) * H + base;
#pragma unroll
      for (int k = 0; k < V; ++k) {
        float xf[8], df[8];
        unpack8(xv[k], xf);
        unpack8(dv[k], df);
        float c[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pr = df[e] * xf[e];          // exact: two bf16 significands
          if (DX) dot = fmaf(pr, w_s[base + k * 512 + e], dot);
          if (RC) sq[RC ? k : 0] = fmaf(xf[e], xf[e], sq[RC ? k : 0]);
          c[e] = pr * r;                           // the row's contribution, rounded once
          if (!RC && DW && COMPLETE) acc[k * 8 + e] = acc[k * 8 + e] + c[e];
        }
        if (!RC && DW && !COMPLETE && in_row(k)) {
          store_f4_stream(srow + k * 512, c[0], c[1], c[2], c[3]);
          store_f4_stream(srow + k * 512 + 4, c[4], c[5], c[6], c[7]);
        }
      }
      if (TW == 1) {
        if (DX) dot = wave_sum(dot);
        if (RC) {
          // this wavefront holds every chunk group of the row
#pragma unroll
          for (int k = 0; k < (RC ? V : 1); ++k) sq[k] = wave_sum(sq[k]);
          ss = pad_tree(sq);
        }
      }
    }
    if (DX || RC) {
      if (TW > 1) {
        // the row's wavefronts exchange their partial sums through LDS
        if (DX) dot = wave_sum(dot);
        if (RC) {
#pragma unroll
          for (int k = 0; k < (RC ? V : 1); ++k) sq[k] = wave_sum(sq[k]);
        }
        if (lane == 0) {
          if (DX) dot_s[(i & 1) * 16 + wv] = dot;
          if (RC) {
#pragma unroll
            for (int k = 0; k < (RC ? V : 1); ++k)
              ss_s[((i & 1) * Sh::S + stream) * (TW * V) + half * V + k] = sq[k];
          }
        }
        __syncthreads();
        if (DX) {
          const float* d = &dot_s[(i & 1) * 16 + stream * TW];
          dot = TW == 2 ? d[0] + d[1] : (d[0] + d[1]) + (d[2 % TW] + d[3 % TW]);
        }
        if (RC) {
          // every chunk group of the row, in group order (groups past the
          // row's end hold +0.0, which the padded tree absorbs)
          float g[RC ? TW * V : 1];
#pragma unroll
          for (int k = 0; k < (RC ? TW * V : 1); ++k)
            g[k] = ss_s[((i & 1) * Sh::S + stream) * (TW * V) + k];
          ss = pad_tree(g);
        }
      }
      if (RC) r = p >= 0 ? rsqrtf(ss / (float)H + a.eps) : 0.0f;
    }
    if (RC && DW && p >= 0) {
      float* srow = COMPLETE ? nullptr : a.S + ((int64_t)blk * kBlockRows + s) * H + base;
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
        if (!COMPLETE && in_row(k)) {
          store_f4_stream(srow + k * 512, c[0], c[1], c[2], c[3]);
          store_f4_stream(srow + k * 512 + 4, c[4], c[5], c[6], c[7]);
        }
      }
    }
    if (DX) {
      if (p >= 0) {
        const float kk = ((r * r) * r) * (dot / (float)H);
        uint16_t* xo = a.dx + (int64_t)p * H + base;
        compiler_fence();
#pragma unroll
        for (int k = 0; k < V; ++k) {
          launder(xv[k]);
          launder(dv[k]);
        }
#pragma unroll
        for (int k = 0; k < V; ++k) {
          if (in_row(k)) {
            float xf[8], df[8], o[8];
            unpack8(xv[k], xf);
            unpack8(dv[k], df);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float g = df[e] * w_s[base + k * 512 + e];
              o[e] = fmaf(-xf[e], kk, r * g);
            }
            store16_stream(xo + k * 512, pack8(o));
          }
        }
      }
    }
  }

  // Two row buffers fit in the register file only up to 8 chunks per lane
  // without masks (4 when rstd is rebuilt, which keeps the row for a second
  // pass); wider or masked rows are processed one at a time.
  static constexpr bool PIPE = FULL && V <= (RC ? 4 : 8);

  __device__ __forceinline__ void run() {
    load_slots();
    if constexpr (PIPE) run_pipelined();
    else run_sequential();
  }

  __device__ __forceinline__ void run_sequential() {
    settle_slots();
    for (int i = 0; i < Sh::SLOTS; ++i) {
      uint4 xv[V], dv[V];
      const int p = row_of(i);
      load(p, xv, dv);
      process(i, p, xv, dv, rstd_of(i));
    }
  }

  __device__ __forceinline__ void run_pipelined() {
    uint4 xa[V], da[V];
    int pa = row_of(0);
    load(pa, xa, da);
    settle_slots();
    run_from(xa, da, pa, -1, false);
  }

  // The pipelined slot loop with slot 0's row already issued into (xa, da).
  // When `more`, the last step issues the first row of the workgroup's next
  // block (lane 0 of `next_slots`, read only there) into (xa, da), so that
  // row is in flight across this block's stream tree; otherwise it issues a
  // dummy load of row 0 (never used) to keep the wait counts exact.
  __device__ __forceinline__ void run_from(uint4 (&xa)[V], uint4 (&da)[V], int pa, int next_slots,
                                           bool more) {
    static_assert(Sh::SLOTS % 2 == 0, "slots per stream must be even");
    uint4 xb[V], db[V];
#pragma unroll
    for (int i = 0; i < Sh::SLOTS; i += 2) {
      const int pb = row_of(i + 1);
      load(pb, xb, db);
      process(i, pa, xa, da, rstd_of(i));
      if (i + 2 < Sh::SLOTS) pa = row_of(i + 2);
      else pa = more ? __builtin_amdgcn_readlane(next_slots, 0) : -1;
      load(pa, xa, da);
      process(i + 1, pb, xb, db, rstd_of(i + 1));
    }
  }
};

// The in-block stream tree, 1024 columns at a time: every stream stores its
// sums for the tile, then each thread reduces its columns into P[blk].
// LOOP: the workgroup folds several blocks, so tile_s may still be read for
// the previous block when the first tile is stored (a barrier comes first).
template <int V, int TW, bool FULL, bool LOOP>
__device__ __forceinline__ void block_partial(const BwdArgs& a, int blk, int H, int tid, int stream,
                                              int half, int lane, const float (&acc)[V * 8],
                                              float* tile_s) {
  using Sh = WideShape<V, TW, FULL>;
  float* Pb = a.P + (int64_t)blk * H;
#pragma unroll
  for (int t = 0; t < Sh::NTILE; ++t) {
    if (LOOP || t > 0) __syncthreads();   // tile_s is free again
#pragma unroll
    for (int k = 0; k < V; ++k) {
      const int K = half * V + k;   // 512-column chunk index within the row
      if ((K >> 1) == t) {
        float* dst = &tile_s[stream * 1024 + ((K & 1) * 64 + lane) * 8];
        store_f4(dst, acc[k * 8 + 0], acc[k * 8 + 1], acc[k * 8 + 2], acc[k * 8 + 3]);
        store_f4(dst + 4, acc[k * 8 + 4], acc[k * 8 + 5], acc[k * 8 + 6], acc[k * 8 + 7]);
      }
    }
    __syncthreads();
    for (int c = tid; c < 1024; c += Sh::THREADS) {
      const int col = t * 1024 + c;
      if (col < H)
        Pb[col] = stream_tree4(tile_s[c], tile_s[1024 + c], tile_s[2048 + c], tile_s[3072 + c]);
    }
  }
}

// Whether the fused backward loops over several work items per workgroup:
// the pipelined two-wavefront kernels up to 4 chunks per lane (hidden 2048,
// 3072, 4096).  Measured at hidden 4096 the loop saves about 1% of the
// backward; at 5120 the loop's extra registers cost more than the block
// hand-over it hides, and the one-block kernel is kept there and above.
template <int V, int TW, bool FULL, bool RC>
constexpr bool wide_persistent() {
  return FULL && TW == 2 && V <= 4;
}

// Workgroups 0 .. item_groups-1 each take work items g, g + item_groups, ...
// (for the looping kernels item_groups is at most what the chip holds at
// once, so every workgroup is resident and they all end after the same
// number of items; otherwise it is the item count, one item each); the
// workgroups after them zero padding rows.  Which workgroup takes an item
// changes nothing in its arithmetic.  In the looping kernels the first row
// of a workgroup's next item is loaded during the last step of the current
// one, so it is in flight across the block's stream tree.
template <int V, int TW, bool FULL, bool PLAN, bool DX, bool DW, bool RC>
__global__ __launch_bounds__(256 * TW) void bwd_wide_kernel(BwdArgs a) {
  using Sh = WideShape<V, TW, FULL>;
  using BlkC = WideBlock<V, TW, FULL, PLAN, DX, DW, true, RC>;    // complete block: fold
  using BlkS = WideBlock<V, TW, FULL, PLAN, DX, DW, false, RC>;   // partial block: spill
  constexpr bool PIPE = BlkC::PIPE;
  constexpr bool LOOP = wide_persistent<V, TW, FULL, RC>();
  static_assert(!LOOP || PIPE, "the looping kernels are the pipelined ones");
  __shared__ float w_s[DX ? Sh::COLS : 1];
  __shared__ float tile_s[DW ? kStreams * 1024 : 1];
  __shared__ float dot_s[(DX && TW > 1) ? 2 * 16 : 1];
  __shared__ float ss_s[(RC && TW > 1) ? 2 * kStreams * TW * V : 1];

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wavefront
  const int lane = tid & 63;
  const int stream = wv / TW;
  const int half = wv % TW;
  const int H = FULL ? Sh::COLS : a.hidden;
  const int nchunk = H >> 3;
  const int n_items = a.plan.n_items;
  const int groups = a.item_groups;

  if ((int)blockIdx.x >= groups) {
    // padding rows: dx = 0, nothing read (one row per wavefront)
    if (DX) {
      const int idx = ((int)blockIdx.x - groups) * Sh::WAVES + wv;
      if (idx < a.plan.n_pad) {
        uint16_t* d = a.dx + (int64_t)a.plan.pad_rows[idx] * H;
        for (int q = lane; q < nchunk; q += 64) store16_stream(d + q * 8, make_uint4(0, 0, 0, 0));
      }
    }
    return;
  }
  int item = blockIdx.x;
  if (item >= n_items) return;

  if (DX) stage_w<Sh>(a, w_s, tid, nchunk);

  // item -> (canonical block, does the call hold all of its present rows)
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

  float acc[DW ? V * 8 : 1];
  const int base = half * V * 512 + lane * 8;      // this lane's first column
  int blk;
  bool complete;
  info_of(item, blk, complete);
  if constexpr (!LOOP) {
    // one item per workgroup
#pragma unroll
    for (int i = 0; i < (DW ? V * 8 : 1); ++i) acc[i] = 0.0f;
    if (!DW || complete) {
      BlkC{a, item, blk, stream, half, lane, wv, H, nchunk, base, w_s, dot_s, acc, ss_s}.run();
      if constexpr (DW) block_partial<V, TW, FULL, LOOP>(a, blk, H, tid, stream, half, lane, acc, tile_s);
    } else {
      BlkS{a, item, blk, stream, half, lane, wv, H, nchunk, base, w_s, dot_s, acc, ss_s}.run();
    }
    return;
  }
  BlkC cur{a, item, blk, stream, half, lane, wv, H, nchunk, base, w_s, dot_s, acc, ss_s};
  cur.load_slots();
  uint4 xa[V], da[V];
  int pa = cur.row_of(0);
  cur.load(pa, xa, da);
  cur.settle_slots();
  while (true) {
    const int nxt = item + groups;
    const bool more = nxt < n_items;
    int nblk = 0;
    bool ncomplete = true;
    BlkC nx{a, nxt, 0, stream, half, lane, wv, H, nchunk, base, w_s, dot_s, acc, ss_s};
    if (more) {
      info_of(nxt, nblk, ncomplete);
      nx.blk = nblk;
      nx.load_slots();
    }
#pragma unroll
    for (int i = 0; i < (DW ? V * 8 : 1); ++i) acc[i] = 0.0f;
    if (!DW || complete) {
      cur.run_from(xa, da, pa, nx.slot_p, more);
      if constexpr (DW) block_partial<V, TW, FULL, LOOP>(a, blk, H, tid, stream, half, lane, acc, tile_s);
    } else {
      BlkS sp{a, item, blk, stream, half, lane, wv, H, nchunk, base, w_s, dot_s, acc, ss_s};
      sp.slot_p = cur.slot_p;
      sp.slot_r = cur.slot_r;
      sp.run_from(xa, da, pa, nx.slot_p, more);
    }
    if (!more) break;
    item = nxt;
    blk = nblk;
    complete = ncomplete;
    cur.item = nxt;
    cur.blk = nblk;
    cur.slot_p = nx.slot_p;
    cur.slot_r = nx.slot_r;
    pa = cur.row_of(0);   // its loads were issued in the last step
    cur.settle_slots();
  }
}

// ------------------------------------------------- two-pass backward (few blocks)
// A call that touches few canonical blocks would leave most compute units
// idle in the fused kernel (one workgroup per block).  It runs two passes
// instead, with enough workgroups for the whole chip between them:
//   dx rows (dx_rows_part): dx, four physical rows per workgroup step,
//     through the very same per-row code as the fused kernel (WideBlock's
//     load + process with the dweight part compiled out), so every dx bit
//     equals the fused kernel's;
//   dweight columns (dw_cols_part): the dweight contributions and the
//     in-block stream fold of one canonical block over 512 columns, with the
//     same operations in the same order as the fused kernel, so the block
//     partials and spill rows are bitwise the same.
// The passes are independent, so one launch (bwd_split_kernel) runs both:
// its first workgroups fold column units, the rest compute dx rows, and the
// two work lists overlap on the chip.  The column pass reads x and dy a
// second time; for the calls that take this path they are small enough to
// be served largely from the last-level cache.
template <int V, int TW, bool FULL, bool PLAN>
__device__ __forceinline__ void dx_rows_part(const BwdArgs& a, float* w_s, float* dot_s, int64_t wg,
                                             int64_t n_wg) {
  using Sh = WideShape<V, TW, FULL>;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int stream = wv / TW;          // the workgroup's row slot (0..3)
  const int half = wv % TW;
  const int H = FULL ? Sh::COLS : a.hidden;
  const int nchunk = H >> 3;
  stage_w<Sh>(a, w_s, tid, nchunk);
  float acc[1];
  const int base = half * V * 512 + lane * 8;
  WideBlock<V, TW, FULL, PLAN, true, false, true> wb{a, 0, 0, stream, half, lane, wv, H, nchunk,
                                                     base, w_s, dot_s, acc};
  const int64_t step = n_wg * Sh::S;
  int i = 0;
  // the trip count is the same for every wavefront of the workgroup (the
  // TW > 1 dot exchange synchronises the workgroup once per row)
  for (int64_t r0 = wg * Sh::S; r0 < a.rows; r0 += step, ++i) {
    const int64_t row = r0 + stream;
    int p = row < a.rows ? (int)row : -1;
    if (PLAN && p >= 0 && a.plan.row_logical[p] < 0) {
      // padding row: dx = 0, nothing read
      uint16_t* d = a.dx + (int64_t)p * H + base;
#pragma unroll
      for (int k = 0; k < V; ++k)
        if (wb.in_row(k)) store16_stream(d + k * 512, make_uint4(0, 0, 0, 0));
      p = -1;
    }
    const float r = p >= 0 ? a.rstd[p] : 0.0f;
    uint4 xv[V], dv[V];
    wb.load(p, xv, dv);
    wb.process(i, p, xv, dv, r);
  }
}

// One column unit: the canonical block of work item `item` over the 512
// columns of `slice`, folded by 4 wavefronts starting at wavefront `w0`:
// wavefront w0 + w is stream w and lane l holds columns 8*(64*slice + l)
// .. +8.  The stream's 16 rows are loaded in two batches of 8 (all of a
// batch before its fold), and the fold runs in slot order across both; the
// batches keep the unit's registers near the dx rows' so the launch that
// runs both keeps its occupancy.  `live` false: no unit, but the barrier is
// still reached (the workgroup's other unit may need it).
template <bool PLAN>
__device__ __forceinline__ void dw_cols_part(const BwdArgs& a, float (*q_s)[512], int item, int slice,
                                             int w0, bool live) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int stream = __builtin_amdgcn_readfirstlane(tid >> 6) - w0;
  const int H = a.hidden;
  const int q = slice * 64 + lane;         // this lane's 8-column chunk
  const bool on = live && q < (H >> 3);
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
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  if (live) {
    // lane i (< 16) holds the physical row and rstd of the stream's slot i
    const int sp = slot_row_t<PLAN>(a, item, blk, stream + kStreams * (lane & (kSlotsPerStream - 1)));
    const float sr = a.rstd[sp >= 0 ? sp : 0];
    constexpr int B = kSlotsPerStream / 2;
#pragma unroll
    for (int b0 = 0; b0 < kSlotsPerStream; b0 += B) {
      uint4 xv[B], dv[B];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int p = __builtin_amdgcn_readlane(sp, b0 + i);
        const int64_t off = (int64_t)(p >= 0 ? p : 0) * H + (on ? q * 8 : 0);
        xv[i] = load16_stream(a.x + off);
        dv[i] = load16_stream(a.dy + off);
      }
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int p = __builtin_amdgcn_readlane(sp, b0 + i);
        if (p < 0) continue;
        const float r = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sr), b0 + i));
        float xf[8], df[8], c[8];
        unpack8(xv[i], xf);
        unpack8(dv[i], df);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pr = df[e] * xf[e];          // exact: two bf16 significands
          c[e] = pr * r;                           // the row's contribution, rounded once
          acc[e] = acc[e] + c[e];
        }
        if (!complete && on) {
          float* srow = a.S + ((int64_t)blk * kBlockRows + stream + kStreams * (b0 + i)) * H + q * 8;
          store_f4_stream(srow, c[0], c[1], c[2], c[3]);
          store_f4_stream(srow + 4, c[4], c[5], c[6], c[7]);
        }
      }
    }
  }
  const bool fold = live && complete;
  if (fold && stream > 0) {
    float* d = &q_s[stream - 1][lane * 8];
    store_f4(d, acc[0], acc[1], acc[2], acc[3]);
    store_f4(d + 4, acc[4], acc[5], acc[6], acc[7]);
  }
  __syncthreads();
  if (fold && stream == 0 && on) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      o[e] = stream_tree4(acc[e], q_s[0][lane * 8 + e], q_s[1][lane * 8 + e], q_s[2][lane * 8 + e]);
    float* dst = a.P + (int64_t)blk * H + q * 8;
    store_f4(dst, o[0], o[1], o[2], o[3]);
    store_f4(dst + 4, o[4], o[5], o[6], o[7]);
  }
}

// Both passes in one launch.  Workgroups 0 .. n_cols_wg-1 fold column units
// (TW units per workgroup: wavefronts 4u .. 4u+3 take unit TW*wg + u of the
// n_units = items x column slices); the following n_rows_wg workgroups
// compute dx rows.  Either list may be empty (dx alone, contributions alone).
template <int V, int TW, bool FULL, bool PLAN>
__global__ __launch_bounds__(256 * TW) void bwd_split_kernel(BwdArgs a, int n_cols_wg, int n_units,
                                                             int n_slices, int n_rows_wg) {
  using Sh = WideShape<V, TW, FULL>;
  constexpr int ROWS_LDS = Sh::COLS + 2 * 16;
  constexpr int COLS_LDS = TW * (kStreams - 1) * 512;
  __shared__ float lds[ROWS_LDS > COLS_LDS ? ROWS_LDS : COLS_LDS];
  const int wg = blockIdx.x;
  if (wg < n_cols_wg) {
    const int u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);   // the workgroup's unit
    const int unit = wg * TW + u;
    const bool live = unit < n_units;
    dw_cols_part<PLAN>(a, reinterpret_cast<float (*)[512]>(lds + u * (kStreams - 1) * 512),
                       live ? unit / n_slices : 0, live ? unit % n_slices : 0, u * kStreams, live);
  } else {
    dx_rows_part<V, TW, FULL, PLAN>(a, lds, lds + Sh::COLS, wg - n_cols_wg, n_rows_wg);
  }
}

// Small rows: hidden = 8L (L in 1..32), one group of L lanes per row; the
// 64 slots' contributions go through LDS and the 4 streams fold them there.
// RC: rstd rebuilt from the row in the forward's order (the same lanes, the
// same chain and group sum), so its bits are the saved rstd's.
template <int L, bool DX, bool DW, bool PACKED, bool RC>
__global__ __launch_bounds__(256) void bwd_small_kernel(BwdArgs a) {
  constexpr int H = 8 * L;
  constexpr int GROUPS = 256 / L;
  constexpr int ITERS = (kBlockRows + GROUPS - 1) / GROUPS;
  __shared__ float c_s[DW ? kBlockRows * H : 1];
  __shared__ float q_s[DW ? kStreams * H : 1];
  const int tid = threadIdx.x;
  const int g = tid / L;
  const int sub = tid % L;
  const int item = blockIdx.x;

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
        float* srow = a.S + ((int64_t)blk * kBlockRows + s) * H + sub * 8;
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
  }
}

// ----------------------------------------------------------------- finalize
// Partials of spilled blocks, folded from their spill rows in the same order
// as the backward kernel folds complete blocks.
__global__ __launch_bounds__(256) void rebuild_kernel(const float* __restrict__ S,
                                                      float* __restrict__ P,
                                                      const int32_t* __restrict__ blocks,
                                                      int64_t T, int H) {
  const int b = blocks[blockIdx.x];
  const int j = blockIdx.y * 256 + threadIdx.x;
  if (j >= H) return;
  // every slot's value is loaded before the folds (absent slots, l >= T,
  // load nothing and add nothing), so the 64 loads are in flight together
  float v[kBlockRows];
#pragma unroll
  for (int s = 0; s < kBlockRows; ++s) {
    const int64_t l = (int64_t)b * kBlockRows + s;
    v[s] = l < T ? S[l * H + j] : 0.0f;
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

// Wavefronts per row: one up to 1024 columns, two above.
static int wide_tw(int hidden) { return hidden <= 1024 ? 1 : 2; }
static int wide_v(int hidden) {
  const int per = 512 * wide_tw(hidden);
  return (hidden + per - 1) / per;
}

const char* fwd_variant(int hidden) {
  return small_lanes(hidden) ? "fwd_small(lanes_per_row=hidden/8)"
         : wide_tw(hidden) == 1 ? "fwd_rows(wave_per_row, 4 rows per workgroup)"
                                : "fwd_rows(two_waves_per_row, 2 rows per workgroup)";
}
const char* bwd_variant(int hidden) {
  if (small_lanes(hidden)) return "bwd_small(lds_fold, streams=4)";
  return wide_tw(hidden) == 1 ? "bwd_wide(wave_per_row, streams=4; few blocks: dx_rows + dw_cols)"
                              : "bwd_wide(two_waves_per_row, streams=4; few blocks: dx_rows + dw_cols)";
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
  // the backward's row shape: wide_tw wavefronts per row, wide_v chunks per lane
  const int V = wide_v(a.hidden);
  if (wide_tw(a.hidden) == 1) {
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

template <int V, int TW, bool FULL, bool PLAN, bool DX, bool DW, bool RC>
static void bwd_wide_launch(BwdArgs a, int pad_groups, hipStream_t st) {
  using Sh = WideShape<V, TW, FULL>;
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&bwd_wide_kernel<V, TW, FULL, PLAN, DX, DW, RC>),
            Sh::THREADS, 0) != hipSuccess || n <= 0)
      n = 1;
    return n;
  }();
  const int64_t knob = wide_group_cap();
  const int64_t cap = knob > 0 ? knob : (int64_t)per_cu * compute_units();
  a.item_groups = (int32_t)(wide_persistent<V, TW, FULL, RC>() && a.plan.n_items > cap ? cap
                                                                                  : a.plan.n_items);
  const dim3 grid((unsigned)(a.item_groups + pad_groups)), block(Sh::THREADS);
  bwd_wide_kernel<V, TW, FULL, PLAN, DX, DW, RC><<<grid, block, 0, st>>>(a);
}

template <int V, int TW, bool FULL, bool PLAN>
static void bwd_wide_go3(const BwdArgs& a, bool dx, bool dw, bool rc, hipStream_t st) {
  using Sh = WideShape<V, TW, FULL>;
  if (rc) {   // rstd rebuilt in the fused kernel (the two-pass path reads rstd)
    const int pad_groups = (a.plan.n_pad + Sh::WAVES - 1) / Sh::WAVES;
    if (dw) bwd_wide_launch<V, TW, FULL, PLAN, true, true, true>(a, pad_groups, st);
    else bwd_wide_launch<V, TW, FULL, PLAN, true, false, true>(a, pad_groups, st);
    return;
  }
  if (a.plan.n_items < split_items()) {
    int64_t rows_wg = 0;
    if (dx && a.rows > 0) {
      rows_wg = (a.rows + Sh::S - 1) / Sh::S;
      if (rows_wg > grid_cap()) rows_wg = grid_cap();
    }
    const int n_slices = (a.hidden / 8 + 63) / 64;
    const int64_t units = dw ? (int64_t)a.plan.n_items * n_slices : 0;
    const int64_t cols_wg = (units + TW - 1) / TW;
    if (rows_wg + cols_wg == 0) return;
    bwd_split_kernel<V, TW, FULL, PLAN><<<dim3((unsigned)(cols_wg + rows_wg)), dim3(Sh::THREADS), 0, st>>>(
        a, (int)cols_wg, (int)units, n_slices, (int)rows_wg);
    return;
  }
  const int pad_groups = dx ? (a.plan.n_pad + Sh::WAVES - 1) / Sh::WAVES : 0;
  if (dx && dw) bwd_wide_launch<V, TW, FULL, PLAN, true, true, false>(a, pad_groups, st);
  else if (dx) bwd_wide_launch<V, TW, FULL, PLAN, true, false, false>(a, pad_groups, st);
  else bwd_wide_launch<V, TW, FULL, PLAN, false, true, false>(a, pad_groups, st);
}
template <int V, int TW, bool FULL>
static void bwd_wide_go2(const BwdArgs& a, bool dx, bool dw, bool rc, hipStream_t st) {
  if (a.plan.item_info != nullptr) bwd_wide_go3<V, TW, FULL, true>(a, dx, dw, rc, st);
  else bwd_wide_go3<V, TW, FULL, false>(a, dx, dw, rc, st);
}
template <int V, int TW>
static void bwd_wide_go(const BwdArgs& a, bool dx, bool dw, bool rc, hipStream_t st) {
  if (a.hidden == 512 * V * TW) bwd_wide_go2<V, TW, true>(a, dx, dw, rc, st);
  else bwd_wide_go2<V, TW, false>(a, dx, dw, rc, st);
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
  const int tw = wide_tw(a.hidden), V = wide_v(a.hidden);
  if (tw == 1) {
    switch (V) {
      case 1: bwd_wide_go<1, 1>(a, dx, dw, rc, st); break;
      case 2: bwd_wide_go<2, 1>(a, dx, dw, rc, st); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (V) {
#define RBI_BWD2(v) case v: bwd_wide_go<v, 2>(a, dx, dw, rc, st); break;
      RBI_BWD2(2) RBI_BWD2(3) RBI_BWD2(4) RBI_BWD2(5) RBI_BWD2(6)
      RBI_BWD2(7) RBI_BWD2(8) RBI_BWD2(9) RBI_BWD2(10)
#undef RBI_BWD2
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_rebuild(const float* S, float* P, const int32_t* blocks, int32_t n_blocks,
                          int64_t n_logical, int32_t hidden, hipStream_t st) {
  if (n_blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)n_blocks, (unsigned)((hidden + 255) / 256));
  rebuild_kernel<<<grid, dim3(256), 0, st>>>(S, P, blocks, n_logical, hidden);
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
