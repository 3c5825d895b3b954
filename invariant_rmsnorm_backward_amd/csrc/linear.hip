// linear.hip -- gfx950 kernels of the batch-invariant linear-layer backward
// (the "GEMM dX/dW" gradients of "[WS1 Closeout][Backward] Reusable
// gradient-invariance harness and operator adapters", Required adapters).
//
// A linear layer y = x W^T (x[rows][K], W[N][K], bf16) has the VJP
//     dX = dY W            row-local, [rows][N] x [N][K]
//     dW = dY^T X          a sum over rows, [N][rows] x [rows][K]
// "WS1 C4 (#270) closeout evidence" puts the deterministic GEMM's dW in the
// same class as RMSNorm's dweight: a sum whose association follows the
// physical row count is not batch invariant.  Here dW is reduced in one
// canonical order over *logical* rows (GDO-v1):
//   * group g = logical rows [16384 g, 16384 (g+1)); rows >= T are zero;
//   * Q_g = the chain of v_mfma_f32_32x32x16_bf16 over the group's rows in
//     ascending 16-row steps, accumulator starting at +0.0;
//   * dW = perfect pairwise tree over Q_0 .. Q_{G-1}, +0.0 leaves up to the
//     next power of two.
// Each output element's chain is the same whatever tile or workgroup
// computes it (steps of zero rows or columns past the end add +0.0 products
// to an accumulator that started at +0.0, which changes no bit), and the
// kernel always reads the rows in logical order (the caller's buffer when one
// call holds every row in order, else rows staged by logical index), so no
// layout can change a bit.
//
// All three products run on one MFMA tile engine (Engine below):
//   * 256 x 256 output tiles, 8 wavefronts (two per SIMD) each owning a
//     128 x 64 share of 32 x 32 blocks; 128 x 128 tiles with 4 wavefronts for
//     small outputs;
//   * K stages of 64 (32 for the small tiles) in an LDS ring of NS stages,
//     filled by global_load_lds_dwordx4 (16 bytes per lane straight into LDS,
//     no staging registers); one workgroup barrier per stage;
//   * LDS rows XOR-swizzled in 16-byte chunks so that the matrix-core
//     fragment reads hit distinct banks in every 16-lane phase;
//   * operands whose K index is the slow one in memory (W in dX, both
//     operands of dW) stay in that order in LDS and are read with the
//     transposing ds_read_b64_tr_b16, so no operand is rearranged by the ALU;
//   * the 16-deep steps are software pipelined: the fragments of step s + 1
//     are read while the MFMAs of step s run, and the loads of stage
//     it + NS are issued one after each MFMA of the last step of stage it;
//   * tiles are mapped to workgroups so that the 32 workgroups one XCD runs
//     at a time share 4 row blocks and 8 column blocks (the round-robin
//     dispatch puts workgroup id on XCD id % 8), also on grids that 4 x 8
//     super-blocks do not tile (the vocabulary side of an LM head).
#include "linear.h"
#include "tile_map.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace rbi {
namespace lin {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4v_t __attribute__((ext_vector_type(4)));
#define RBI_LDS __attribute__((address_space(3)))

// 16 zero bytes: the source of every load whose rows or columns are out of range.
__device__ __align__(16) uint32_t kZero16[4];

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// Workgroup barrier without a memory fence: the engine waits for its own loads
// explicitly (a fenced barrier would wait for every load still in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
// 16 bytes per lane from global memory into LDS at lds + 16 * lane.  The LDS
// base is an input bound to m0, so the compiler sets m0 itself; the s_nop is
// the wait state between an m0 write and the load that reads it.  The
// compiler does not track this load; the engine waits for it with vmcnt.
__device__ __forceinline__ void load_to_lds(uint64_t src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds));
}
#define RBI_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

template <int MI, int NJ>
struct Acc {
  f32x16_t c[MI][NJ];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) c[i][j][r] = 0.0f;
  }
};

// One operand's tile of one K stage: ROWS tile rows (the operand's M or N
// index) x BK, loaded by NT threads.
//  KM = false (K contiguous): element (m, k) at g[m ld + k]; LDS row r holds
//      its BK values, 16-byte chunk c at position c ^ swz(r).
//  KM = true (K slow): element (m, k) at g[k ld + m]; LDS row kr holds ROWS
//      values of one k, chunk c at position c ^ swk(kr).
// Thread t loads the chunks P = NT i + t of the tile (i < NI); a wavefront's
// 64 loads fill 1 KB of LDS contiguously.
// INNER: every tile row is in range and every stage is either wholly inside
// [0, k_lim) or wholly past it, so a load needs no per-lane range test.
template <bool KM, int ROWS, int BK, int NT, bool INNER = false>
struct Operand {
  static constexpr int CHUNKS = ROWS * BK / 8;
  static constexpr int NI = CHUNKS / NT;
  static constexpr int BYTES = ROWS * BK * 2;
  static constexpr int CPR = BK / 8;                        // chunks per LDS row (KM = false)
  static constexpr int CPK = ROWS / 8;                      // chunks per LDS row (KM = true)
  static constexpr int RSTEP = KM ? NT / CPK : NT / CPR;    // tile rows between a thread's loads
  static_assert(CHUNKS % NT == 0 && NI >= 1, "tile");
  static_assert(KM ? (CPK >= 16 && NT % CPK == 0 && RSTEP % 4 == 0)
                   : (CPR <= 8 && NT % CPR == 0 && RSTEP % 16 == 0),
                "the swizzle of a thread's chunks must not depend on i");
  uint64_t base, zp;
  int64_t ld, k_lim;
  unsigned ok;   // KM: the thread's column is in range; else bit i: row of load i in range
  int kc;        // KM: the thread's row within a stage; else its k offset within a stage

  // Conflict-free for the 8- and the 16-lane phases of a 128-bit read.
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);
    else if constexpr (CPR == 4) return ((((r >> 2) ^ (r >> 3)) & 1) << 1) | (((r >> 1) ^ (r >> 2)) & 1);
    else return 0;
  }
  // Conflict-free for the transposing 64-bit reads (4 rows x 32 or 64 bytes).
  __device__ static __forceinline__ int swk(int kr) { return (2 * (kr & 3)) ^ (8 * (kr & 1)); }

  // m0: first tile row; m_lim / k_lim: rows and k at or past them read as
  // zero; rowmap (KM = false only): a row whose map value is negative reads as zero.
  __device__ __forceinline__ void init(const uint16_t* g, int64_t ld_, int64_t m0, int64_t m_lim,
                                       int64_t k_lim_, const int32_t* rowmap, int t) {
    ld = ld_;
    k_lim = k_lim_;
    zp = (uint64_t)(uintptr_t)kZero16;
    if (!KM) {
      const int r = t / CPR;
      const int c = (t % CPR) ^ swz(r);
      kc = 8 * c;
      ok = 0;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int64_t m = m0 + r + (int64_t)RSTEP * i;
        bool v = m < m_lim;
        if (v && rowmap != nullptr) v = rowmap[m] >= 0;
        ok |= (unsigned)v << i;
      }
      base = (uint64_t)(uintptr_t)(g + (m0 + r) * ld + kc);
    } else {
      const int kr = t / CPK;
      const int c = (t % CPK) ^ swk(kr);
      kc = kr;
      const int64_t m = m0 + 8 * c;
      ok = m < m_lim;
      base = (uint64_t)(uintptr_t)(g + (int64_t)kr * ld + m);
    }
  }

  template <int I>
  __device__ __forceinline__ void issue_one(uint32_t tile, int64_t k0, int w) const {
    const uint32_t dst = tile + (uint32_t)((NT * I + 64 * w) * 16);
    if constexpr (INNER) {
      // k0 is the same in every lane: a stage past the end reads zeros
      const uint64_t a = !KM ? base + (uint64_t)(((int64_t)RSTEP * I * ld + k0) * 2)
                             : base + (uint64_t)((k0 + (int64_t)RSTEP * I) * ld * 2);
      if (k0 + BK <= k_lim) load_to_lds(a, dst);
      else load_to_lds(zp, dst);
      return;
    }
    bool v;
    uint64_t a;
    if (!KM) {
      v = (bool)((ok >> I) & 1u) & (k0 + kc < k_lim);
      a = base + (uint64_t)(((int64_t)RSTEP * I * ld + k0) * 2);
    } else {
      v = (bool)ok & (k0 + kc + RSTEP * I < k_lim);
      a = base + (uint64_t)((k0 + (int64_t)RSTEP * I) * ld * 2);
    }
    load_to_lds(v ? a : zp, dst);
  }
  template <int I = 0>
  __device__ __forceinline__ void issue_all(uint32_t tile, int64_t k0, int w) const {
    if constexpr (I < NI) {
      issue_one<I>(tile, k0, w);
      issue_all<I + 1>(tile, k0, w);
    }
  }

  // Matrix-core fragment: lane l holds (tile row R0 + l % 32, k = ks + 8 (l / 32) + 0..7).
  // KM: two transposing reads; in each 16-lane group lane j addresses 4 values
  // of row kr = ks + 8 (l / 32) + j / 4 (+ 4 for the second read) at columns
  // R0 + 16 ((l / 16) % 2) + 4 (j % 4), and lane i receives column .. + i of
  // the group's 4 rows.
  __device__ __forceinline__ bf16x8_t frag(uint32_t tile, int R0, int ks, int lane) const {
    if (!KM) {
      const int R = R0 + (lane & 31);
      const int c = (ks >> 3) + (lane >> 5);
      return *(const RBI_LDS bf16x8_t*)(uintptr_t)(tile + (uint32_t)((R * CPR + (c ^ swz(R))) * 16));
    } else {
      const int j = lane & 15;
      const int m = R0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
      const int phys = (m >> 3) ^ swk(j >> 2);
      const int kr = ks + 8 * (lane >> 5) + (j >> 2);
      const uint32_t p0 = tile + (uint32_t)((kr * CPK + phys) * 16 + (m & 7) * 2);
      const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((RBI_LDS s16x4_t*)(uintptr_t)p0);
      const s16x4_t v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((RBI_LDS s16x4_t*)(uintptr_t)(p0 + 4 * CPK * 16));
      const s16x8_t v = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8_t, v);
    }
  }
};

// BM x BN output tile, K stages of BK in an LDS ring of NS stages, WGM x WGN
// wavefronts (each owning a (BM / WGM) x (BN / WGN) share of 32 x 32 blocks).
// AKM / BKM: the operand's K index is the slow one in memory.  INNER: the
// operands' loads need no range test (see Operand).
template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool AKM, bool BKM, bool INNER = false>
struct Engine {
  static constexpr int NT = 64 * WGM * WGN;
  using OA = Operand<AKM, BM, BK, NT, INNER>;
  using OB = Operand<BKM, BN, BK, NT, INNER>;
  static constexpr int STAGE = OA::BYTES + OB::BYTES;
  static constexpr int L = OA::NI + OB::NI;                  // loads per thread per stage
  static constexpr int LDS_BYTES = NS * STAGE;
  static constexpr int MI = BM / (32 * WGM), NJ = BN / (32 * WGN);
  static constexpr int STEPS = BK / 16;
  static_assert(STEPS % 2 == 0 && L <= MI * NJ && NS >= 2, "engine shape");
  static_assert((NS - 1) * L < 64, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  using AccT = Acc<MI, NJ>;

  __device__ static __forceinline__ int wm(int w) { return (w / WGN) * (BM / WGM); }
  __device__ static __forceinline__ int wn(int w) { return (w % WGN) * (BN / WGN); }

  __device__ static __forceinline__ void frags(const OA& oa, const OB& ob, uint32_t as, int ks, int m0,
                                               int n0, int lane, bf16x8_t* a, bf16x8_t* b) {
#pragma unroll
    for (int i = 0; i < MI; ++i) a[i] = oa.frag(as, m0 + 32 * i, ks, lane);
#pragma unroll
    for (int j = 0; j < NJ; ++j) b[j] = ob.frag(as + OA::BYTES, n0 + 32 * j, ks, lane);
  }

  template <int Q>
  __device__ static __forceinline__ void load_q(const OA& oa, const OB& ob, uint32_t tile, int64_t k0,
                                                int w) {
    if constexpr (Q < OA::NI) oa.template issue_one<Q>(tile, k0, w);
    else if constexpr (Q < L) ob.template issue_one<Q - OA::NI>(tile + OA::BYTES, k0, w);
  }

  // The MI x NJ MFMAs of one step; with LOADS, load Q of the next stage after MFMA Q.
  // Each block is computed transposed (B's fragment as the instruction's
  // first operand), so that a lane's results lie along a tile row (see
  // for_each4).  The instruction forms the same products and sums them in the
  // same order either way: the results are bit for bit those of the
  // untransposed product.
  template <bool LOADS, int Q = 0>
  __device__ static __forceinline__ void mma(AccT& acc, const bf16x8_t* a, const bf16x8_t* b,
                                             const OA& oa, const OB& ob, uint32_t tile, int64_t k0,
                                             int w) {
    if constexpr (Q < MI * NJ) {
      acc.c[Q / NJ][Q % NJ] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[Q % NJ], a[Q / NJ], acc.c[Q / NJ][Q % NJ], 0, 0, 0);
      if constexpr (LOADS && Q < L) {
        RBI_SCHED_FENCE();
        load_q<Q>(oa, ob, tile, k0, w);
        RBI_SCHED_FENCE();
      }
      mma<LOADS, Q + 1>(acc, a, b, oa, ob, tile, k0, w);
    }
  }

  // Step S of stage `it` (buffer `as`): the fragments of the next step (or of
  // the next stage's first step) are read into (na, nb) while the MFMAs use
  // (ca, cb).  The last step waits for the next stage, meets the other
  // wavefronts, and refills this stage's buffer with stage it + NS.
  template <int S>
  __device__ static __forceinline__ void step(uint32_t sm, uint32_t as, int it, AccT& acc,
                                              const OA& oa, const OB& ob, int64_t k_begin, int w,
                                              int m0, int n0, int lane, bf16x8_t* ca, bf16x8_t* cb,
                                              bf16x8_t* na, bf16x8_t* nb) {
    RBI_SCHED_FENCE();
    if constexpr (S == STEPS - 1) {
      wait_vm_lgkm<(NS - 2) * L>();
      lds_barrier();
      frags(oa, ob, sm + (uint32_t)(((it + 1) % NS) * STAGE), 0, m0, n0, lane, na, nb);
      RBI_SCHED_FENCE();
      mma<true>(acc, ca, cb, oa, ob, as, k_begin + (int64_t)(it + NS) * BK, w);
    } else {
      frags(oa, ob, as, 16 * (S + 1), m0, n0, lane, na, nb);
      RBI_SCHED_FENCE();
      mma<false>(acc, ca, cb, oa, ob, as, 0, w);
    }
    RBI_SCHED_FENCE();
  }
  template <int S>
  __device__ static __forceinline__ void steps(uint32_t sm, uint32_t as, int it, AccT& acc,
                                               const OA& oa, const OB& ob, int64_t k_begin, int w,
                                               int m0, int n0, int lane, bf16x8_t* a0, bf16x8_t* b0,
                                               bf16x8_t* a1, bf16x8_t* b1) {
    if constexpr (S < STEPS) {
      if constexpr (S % 2 == 0) step<S>(sm, as, it, acc, oa, ob, k_begin, w, m0, n0, lane, a0, b0, a1, b1);
      else step<S>(sm, as, it, acc, oa, ob, k_begin, w, m0, n0, lane, a1, b1, a0, b0);
      steps<S + 1>(sm, as, it, acc, oa, ob, k_begin, w, m0, n0, lane, a0, b0, a1, b1);
    }
  }

  // acc += the product over the K stages [k_begin, k_begin + nst BK) in
  // ascending order.  Every stage issues its loads (stages past the end read
  // the zero chunk into a buffer no later stage reads), so the wait counts
  // are constants.  They count the engine's own loads only: the loop issues
  // no other vector-memory load, and the row-map reads of Operand::init feed
  // the first load addresses, so they are complete before any stage is issued.
  __device__ static __forceinline__ void run(uint32_t sm, AccT& acc, const OA& oa, const OB& ob,
                                             int64_t k_begin, int nst) {
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int m0 = wm(w), n0 = wn(w);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      oa.issue_all(sm + s * STAGE, k_begin + (int64_t)s * BK, w);
      ob.issue_all(sm + s * STAGE + OA::BYTES, k_begin + (int64_t)s * BK, w);
    }
    wait_vm_lgkm<(NS - 1) * L>();
    lds_barrier();
    bf16x8_t a0[MI], b0[NJ], a1[MI], b1[NJ];
    frags(oa, ob, sm, 0, m0, n0, lane, a0, b0);
    for (int it = 0; it < nst; ++it) {
      const uint32_t as = sm + (uint32_t)((it % NS) * STAGE);
      steps<0>(sm, as, it, acc, oa, ob, k_begin, w, m0, n0, lane, a0, b0, a1, b1);
    }
    wait_vm_lgkm<0>();
  }

  // Results of wavefront w, four consecutive columns at a time: block (i, j),
  // registers 4q .. 4q + 3 of a lane hold tile row wm + 32 i + lane % 32,
  // tile columns wn + 32 j + 8 q + 4 (lane / 32) + 0 .. 3.
  template <typename F>
  __device__ static __forceinline__ void for_each4(const AccT& acc, F&& f) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int mb = wm(w), nb = wn(w);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          f(mb + 32 * i + (lane & 31), nb + 32 * j + 8 * q + 4 * (lane >> 5), acc.c[i][j][4 * q],
            acc.c[i][j][4 * q + 1], acc.c[i][j][4 * q + 2], acc.c[i][j][4 * q + 3]);
  }
};

__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
  const unsigned u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ u32x4v_t ld16_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4v_t*>(p));
}

__device__ __forceinline__ uint32_t lds_addr(RBI_LDS uint8_t* p) { return (uint32_t)(uintptr_t)p; }

// y = x W^T (fwd, B K-contiguous) and dX = dY W (B K-slow): bf16 result rows of
// the call, padding rows 0.  One workgroup per tile, 1-D grid.
template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool BT>
__global__ __launch_bounds__(64 * WGM * WGN) void rowwise_kernel(RowwiseArgs p) {
  using E = Engine<BM, BN, BK, NS, WGM, WGN, false, BT>;
  __shared__ __align__(16) uint8_t smem[E::LDS_BYTES];
  int tm, tn;
  if (!xcd_tile((int)blockIdx.x, (int)((p.rows + BM - 1) / BM), (int)((p.n + BN - 1) / BN), tm, tn)) return;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int t = threadIdx.x;
  typename E::OA oa;
  typename E::OB ob;
  oa.init(p.a, p.lda, m0, p.rows, p.k, p.row_logical, t);
  ob.init(p.b, p.ldb, n0, p.n, p.k, nullptr, t);
  typename E::AccT acc;
  acc.zero();
  E::run(lds_addr((RBI_LDS uint8_t*)smem), acc, oa, ob, 0, (int)((p.k + BK - 1) / BK));
  // padding rows were loaded as zeros; they are written as 0 explicitly
  // four bf16 results per 8-byte store (n is a multiple of 8, a column
  // group is wholly inside or outside the output)
  E::for_each4(acc, [&](int mi, int ni, float v0, float v1, float v2, float v3) {
    const int64_t m = m0 + mi, n = n0 + ni;
    if (m < p.rows && n < p.n) {
      const bool pad = p.row_logical != nullptr && p.row_logical[m] < 0;
      uint2 o = make_uint2(0u, 0u);
      if (!pad) {
        o.x = (uint32_t)to_bf16_rne(v0) | ((uint32_t)to_bf16_rne(v1) << 16);
        o.y = (uint32_t)to_bf16_rne(v2) | ((uint32_t)to_bf16_rne(v3) << 16);
      }
      *reinterpret_cast<uint2*>(p.out + m * p.n + n) = o;
    }
  });
}

// Q_g for one tile of dW and one group g of logical rows (dY and X in logical
// row order, T rows); 1-D grid, workgroup id = g * tiles + tile.
template <int BM, int BN, int BK, int NS, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void dw_group_kernel(DwArgs p) {
  using E = Engine<BM, BN, BK, NS, WGM, WGN, true, true>;
  using EI = Engine<BM, BN, BK, NS, WGM, WGN, true, true, true>;
  static_assert(kGroupRows % BK == 0, "a group holds whole stages");
  __shared__ __align__(16) uint8_t smem[E::LDS_BYTES];
  const int tmc = (int)((p.n + BM - 1) / BM), tnc = (int)((p.k + BN - 1) / BN);
  const int per_group = (int)tile_slots(tmc, tnc);
  const int g = (int)p.g_first + (int)blockIdx.x / per_group;
  int tm, tn;
  if (!xcd_tile((int)blockIdx.x % per_group, tmc, tnc, tm, tn)) return;
  const int64_t n0 = (int64_t)tm * BM, k0 = (int64_t)tn * BN;
  const int64_t r0 = (int64_t)g * kGroupRows;
  int64_t r1 = r0 + kGroupRows;
  if (r1 > p.T) r1 = (p.T + BK - 1) / BK * BK;   // the rest of the group is zero rows
  // Rows at or past the group's end read as zero: the ring's loads for the
  // stages after the last one must not reach past the group, whose rows may
  // be all a caller's buffer holds (a call that holds the group whole).
  const int64_t row_end = r0 + kGroupRows < p.T ? r0 + kGroupRows : p.T;
  const int t = threadIdx.x;
  typename E::AccT acc;
  acc.zero();
  const uint32_t sm = lds_addr((RBI_LDS uint8_t*)smem);
  if (n0 + BM <= p.n && k0 + BN <= p.k && r0 + kGroupRows <= p.T) {
    // a whole tile of a whole group: no load needs a range test (the same
    // loads into the same LDS places, so the same chain)
    typename EI::OA oa;
    typename EI::OB ob;
    oa.init(p.dy, p.n, n0, p.n, row_end, nullptr, t);
    ob.init(p.x, p.k, k0, p.k, row_end, nullptr, t);
    EI::run(sm, acc, oa, ob, r0, (int)((r1 - r0) / BK));
  } else {
    typename E::OA oa;
    typename E::OB ob;
    oa.init(p.dy, p.n, n0, p.n, row_end, nullptr, t);
    ob.init(p.x, p.k, k0, p.k, row_end, nullptr, t);
    E::run(sm, acc, oa, ob, r0, (int)((r1 - r0) / BK));
  }
  float* out = p.out + (int64_t)g * p.n * p.k;
  E::for_each4(acc, [&](int mi, int ni, float v0, float v1, float v2, float v3) {
    const int64_t n = n0 + mi, k = k0 + ni;
    if (n < p.n && k < p.k) *reinterpret_cast<float4*>(out + n * p.k + k) = make_float4(v0, v1, v2, v3);
  });
}

// dW = perfect pairwise tree over the G group results (+0.0 past G), G <= 64.
template <int L>
__global__ __launch_bounds__(256) void group_tree_kernel(const float* __restrict__ q, int G,
                                                         int64_t nk, float* __restrict__ dw) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= nk) return;
  float v[L];
#pragma unroll
  for (int i = 0; i < L; ++i) v[i] = i < G ? q[(int64_t)i * nk + e] : 0.0f;
#pragma unroll
  for (int s = 1; s < L; s *= 2)
#pragma unroll
    for (int i = 0; i < L; i += 2 * s) v[i] = v[i] + v[i + s];
  dw[e] = v[0];
}

// Rows of one call copied to their logical positions (staging for the rows
// of groups a call does not hold whole and in order); padding rows and the
// rows of groups flagged in skip_groups are skipped.
__global__ __launch_bounds__(256) void stage_rows_kernel(const uint16_t* __restrict__ src,
                                                         int64_t rows, int64_t cols,
                                                         const int32_t* __restrict__ row_logical,
                                                         uint16_t* __restrict__ dst,
                                                         uint64_t skip_groups) {
  const int64_t nchunk = cols / 8;
  const int64_t total = rows * nchunk;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t p = i / nchunk, c = i % nchunk;
    const int32_t l = row_logical[p];
    const int64_t g = l / kGroupRows;
    if (l >= 0 && !(skip_groups != 0 && g < 64 && ((skip_groups >> g) & 1u)))
      *reinterpret_cast<u32x4v_t*>(dst + (int64_t)l * cols + 8 * c) = ld16_nt(src + p * cols + 8 * c);
  }
}

// The same for the rows of two tensors of one call (x and dY) in one launch:
// unit i < rows * (ca + cb) / 8 of the call is chunk i % per of row i / per,
// from the first tensor below ca / 8 chunks, else from the second.
__global__ __launch_bounds__(256) void stage_rows2_kernel(const uint16_t* __restrict__ a, int64_t ca,
                                                          uint16_t* __restrict__ da,
                                                          const uint16_t* __restrict__ b, int64_t cb,
                                                          uint16_t* __restrict__ db, int64_t rows,
                                                          const int32_t* __restrict__ row_logical,
                                                          uint64_t skip_groups) {
  const int64_t na = ca / 8, per = na + cb / 8;
  const int64_t total = rows * per;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t p = i / per, c = i % per;
    const int32_t l = row_logical[p];
    const int64_t g = l / kGroupRows;
    if (l >= 0 && !(skip_groups != 0 && g < 64 && ((skip_groups >> g) & 1u))) {
      if (c < na)
        *reinterpret_cast<u32x4v_t*>(da + (int64_t)l * ca + 8 * c) = ld16_nt(a + p * ca + 8 * c);
      else
        *reinterpret_cast<u32x4v_t*>(db + (int64_t)l * cb + 8 * (c - na)) =
            ld16_nt(b + p * cb + 8 * (c - na));
    }
  }
}

__global__ __launch_bounds__(256) void zero_rows_kernel(uint16_t* __restrict__ dst, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    *reinterpret_cast<u32x4v_t*>(dst + 8 * i) = u32x4v_t{0u, 0u, 0u, 0u};
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = 0.0f;
}

// ----------------------------------------------------------------- launchers
// Tile shape from the output size only (the results do not depend on it:
// every output element runs the same chain whatever tile holds it).
static bool big_tiles(int64_t m, int64_t n) { return m >= 256 && n >= 256; }

template <int BM, int BN, int BK, int NS, int WGM, int WGN>
static hipError_t rowwise_go(const RowwiseArgs& a, bool bt, hipStream_t st) {
  const int64_t tiles = tile_slots((a.rows + BM - 1) / BM, (a.n + BN - 1) / BN);
  if (tiles > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tiles), block(64 * WGM * WGN);
  if (bt) rowwise_kernel<BM, BN, BK, NS, WGM, WGN, true><<<grid, block, 0, st>>>(a);
  else rowwise_kernel<BM, BN, BK, NS, WGM, WGN, false><<<grid, block, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_rowwise(const RowwiseArgs& a, bool b_transposed, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  if (big_tiles(a.rows, a.n)) return rowwise_go<256, 256, 64, 2, 2, 4>(a, b_transposed, st);
  return rowwise_go<128, 128, 32, 4, 2, 2>(a, b_transposed, st);
}

int64_t num_groups(int64_t T) { return (T + kGroupRows - 1) / kGroupRows; }

template <int BM, int BN, int BK, int NS, int WGM, int WGN>
static hipError_t dw_go(const DwArgs& a, int64_t G, hipStream_t st) {
  const int64_t tiles = tile_slots((a.n + BM - 1) / BM, (a.k + BN - 1) / BN) * G;
  if (tiles > INT32_MAX) return hipErrorInvalidValue;
  dw_group_kernel<BM, BN, BK, NS, WGM, WGN><<<dim3((unsigned)tiles), dim3(64 * WGM * WGN), 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_dw_groups(const DwArgs& a_in, hipStream_t st) {
  const int64_t total = num_groups(a_in.T);
  DwArgs a = a_in;
  if (a.g_count == 0) {
    a.g_first = 0;
    a.g_count = total;
  }
  if (a.g_count == 0) return hipSuccess;
  if (a.g_first < 0 || a.g_first + a.g_count > total) return hipErrorInvalidValue;
  if (big_tiles(a.n, a.k)) return dw_go<256, 256, 64, 2, 2, 4>(a, a.g_count, st);
  return dw_go<128, 128, 32, 4, 2, 2>(a, a.g_count, st);
}

hipError_t launch_group_tree(const float* q, int64_t G, int64_t nk, float* dw, hipStream_t st) {
  const dim3 grid((unsigned)((nk + 255) / 256));
  int L = 1;
  while (L < G) L *= 2;
  switch (L) {
    case 1: group_tree_kernel<1><<<grid, dim3(256), 0, st>>>(q, (int)G, nk, dw); break;
    case 2: group_tree_kernel<2><<<grid, dim3(256), 0, st>>>(q, (int)G, nk, dw); break;
    case 4: group_tree_kernel<4><<<grid, dim3(256), 0, st>>>(q, (int)G, nk, dw); break;
    case 8: group_tree_kernel<8><<<grid, dim3(256), 0, st>>>(q, (int)G, nk, dw); break;
    case 16: group_tree_kernel<16><<<grid, dim3(256), 0, st>>>(q, (int)G, nk, dw); break;
    case 32: group_tree_kernel<32><<<grid, dim3(256), 0, st>>>(q, (int)G, nk, dw); break;
    case 64: group_tree_kernel<64><<<grid, dim3(256), 0, st>>>(q, (int)G, nk, dw); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_stage_rows(const uint16_t* src, int64_t rows, int64_t cols,
                             const int32_t* row_logical, uint16_t* dst, hipStream_t st,
                             uint64_t skip_groups) {
  if (rows == 0) return hipSuccess;
  int64_t g = (rows * (cols / 8) + 255) / 256;
  if (g > 4096) g = 4096;
  stage_rows_kernel<<<dim3((unsigned)g), dim3(256), 0, st>>>(src, rows, cols, row_logical, dst,
                                                              skip_groups);
  return hipGetLastError();
}

hipError_t launch_stage_rows2(const uint16_t* a, int64_t ca, uint16_t* da, const uint16_t* b,
                              int64_t cb, uint16_t* db, int64_t rows, const int32_t* row_logical,
                              hipStream_t st, uint64_t skip_groups) {
  if (rows == 0) return hipSuccess;
  int64_t g = (rows * ((ca + cb) / 8) + 255) / 256;
  if (g > 4096) g = 4096;
  stage_rows2_kernel<<<dim3((unsigned)g), dim3(256), 0, st>>>(a, ca, da, b, cb, db, rows, row_logical,
                                                               skip_groups);
  return hipGetLastError();
}

hipError_t launch_zero(uint16_t* dst, int64_t n_elems, hipStream_t st) {
  const int64_t n16 = n_elems / 8;
  if (n16 == 0) return hipSuccess;
  int64_t g = (n16 + 255) / 256;
  if (g > 4096) g = 4096;
  zero_rows_kernel<<<dim3((unsigned)g), dim3(256), 0, st>>>(dst, n16);
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* dst, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  int64_t g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  zero_f32_kernel<<<dim3((unsigned)g), dim3(256), 0, st>>>(dst, n);
  return hipGetLastError();
}

}  // namespace lin
}  // namespace rbi
