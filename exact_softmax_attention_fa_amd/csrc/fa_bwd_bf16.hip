// Backward pass of exact softmax attention, bf16 inputs, for gfx950 (CDNA4).
//
// The probabilities are recomputed from q, k and the forward's saved log-normaliser instead
// of being stored (lihaoran.work, "The intermediate matrix comes first": FlashAttention
// recomputes in the backward pass). The gradients are those of the definition O = P V,
// P = softmax(scale Q K^T) row by row:
//   delta_i = sum_c dO_ic O_ic                 (= sum_k P_ik dP_ik)
//   P_ij    = exp(scale q_i.k_j - lse_i)       (0 where masked)
//   dP_ij   = dO_i . v_j
//   dS_ij   = P_ij (dP_ij - delta_i)
//   dV = P^T dO,   dK = scale dS^T Q,   dQ = scale dS K
//
// Two kernels, no atomics, launched in this order:
// * bwd_dq_kernel: a workgroup owns 128 queries (4 waves x 32). Each query's delta comes from
//   its dO row (held in registers) and its O row, and is written to the caller's workspace.
//   Then it walks the key tiles of 32, like the forward: S^T = K Q^T and dP^T = V dO^T with
//   Q and dO in registers, and dQ^T += K^T dS^T with K^T read transposed from the K tile.
// * bwd_dkdv_kernel: a workgroup owns 128 keys and walks the query blocks of 32 rows, staged
//   in LDS (Q, dO, log-normaliser, delta). Score waves form S = Q K^T and dP = dO V^T with K
//   and V held in registers as B operands (the accumulator holds one key per lane and 16
//   queries in its registers), then P and dS; accumulator waves add dV^T += dO^T P and
//   dK^T += Q^T dS with the transposed operands read by ds_read_b64_tr_b16 and P / dS as the
//   B operands (the register/key correspondence of the forward kernels, with the roles of
//   queries and keys exchanged).
// Scores stay in base-2 units (|scale| log2 e folded into one multiply); a negative scale
// negates q exactly and dQ at the end. P and dS are rounded to bf16 for the MFMAs, with fp32
// accumulation; the outputs are rounded to bf16 once.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "fa_bwd_internal.h"
#include "fa_dma.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int NW = 4;        // waves per workgroup
constexpr int NT = NW * 64;
constexpr int BLK = 32;      // rows per MFMA block (keys or queries)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// MFMA 32x32x16 bf16 with fp32 accumulation
__device__ __forceinline__ f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// Staged [32][D] bf16 tiles sit in LDS without padding: 16-byte chunk L of row r is stored at
// chunk position L ^ swz(r) (fa_dma.h), which keeps both the row reads and the transposed reads
// free of bank conflicts.
using dma::swz;
template <int D>
__device__ __forceinline__ int tile_off(int r, int chunk) { return r * D + 8 * (chunk ^ swz<D>(r)); }

// Per-lane element offsets into a swizzled tile for the two read patterns:
// * row reads: lane l takes row l%32, features 16kk + 8(l/32) .. +7 (an A operand of S);
// * transposed reads: lane l gets feature 32dt + l%32 of rows 16c + {4hh + r, 8 + 4hh + r}
//   (r = 0..3), the order in which accumulator registers 8c..8c+7 hold their rows; the
//   offsets below are for c = 0, and c = 1 adds 16 rows.
template <int D>
struct TileOffsets {
  int row[D / 16];
  int tr[D / 32][2];
  __device__ __forceinline__ explicit TileOffsets(int lane) {
    const int lr = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) row[kk] = tile_off<D>(lr, 2 * kk + hh);
    const int tr_row = 4 * hh + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        tr[dt][h] = tile_off<D>(tr_row + 8 * h, 4 * dt + (tr_col >> 3)) + (tr_col & 7);
  }
};

template <int D>
__device__ __forceinline__ u32x4 read_tr(const uint16_t* tile, int c16, const TileOffsets<D>& to, int dt) {
  const uint16_t* base = tile + c16 * 16 * D;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + to.tr[dt][0]));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + to.tr[dt][1]));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
  return (u32x4){lo2[0], lo2[1], hi2[0], hi2[1]};
}

// ---- dK, dV --------------------------------------------------------------------------------
// One 16-byte-per-lane (or 4-byte-per-lane) global -> LDS load: lane l's data lands at LDS
// byte lds_addr + 16 l (+ 4 l). Issued through inline assembly so that the compiler's wait
// insertion does not tie later LDS reads to it; completion is tracked by hand (step_barrier).
// An LDS DMA needs a wait state after the scalar write of M0 that gives its LDS address (the
// s_nop).
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory");
}

// Wait until at most n vector-memory operations of this wave are outstanding and its LDS
// accesses have completed, then join the workgroup barrier. The compiler does not see the
// LDS writes of the loads above, so this is also a compiler memory barrier.
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  // s_waitcnt encoding (gfx9): vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  constexpr int imm = (n & 15) | (7 << 4) | (0 << 8) | ((n >> 4) << 14);
  __builtin_amdgcn_s_waitcnt(imm);
}
template <int n>
__device__ __forceinline__ void step_barrier() {
  wait_vm_lgkm0<n>();
  asm volatile("s_barrier" ::: "memory");
}

// A workgroup owns 128 keys and runs 8 waves in two roles, two waves per SIMD:
// * score waves (0..3) hold K^T and V^T of 32 keys each in registers and, per query block,
//   form S = Q K^T and dP = dO V^T, the probabilities P and dS = P (dP - delta), and hand
//   P and dS (bf16, already in B-operand order) to their partner through LDS;
// * accumulator waves (4..7) hold dK^T and dV^T of the same 32 keys and, one block later,
//   add dO^T P and Q^T dS with the transposed operands read from the staged tiles.
// Each role fits in half a SIMD's registers. A score wave is software-pipelined: while the
// matrix core forms S and dP of block j+1, its VALU turns the S and dP of block j (held in
// registers since the previous step) into P and dS, and the partner accumulates block j-1
// meanwhile. The query blocks (Q and dO tiles, log-normaliser and delta rows) rotate through
// five LDS slots, loaded straight from global memory two steps ahead of their first use:
// block j+3 loading, j+2 landed, j+1 in the products, j waiting, j-1 accumulated.
// P / dS rotate through two exchange buffers.
constexpr int DKDV_NT = 2 * NT;          // 8 waves
template <int D, bool CAUSAL>
__global__ __launch_bounds__(DKDV_NT, 1)
void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int QT = BLK * D;           // swizzled Q / dO tile (elements)
  constexpr int TILEB = 2 * QT;         // bytes per tile
  constexpr int SLOTB = 2 * TILEB + 512;   // Q tile, dO tile, 64 floats of log-normaliser, 64 of delta
  constexpr int SLOTS = 5;
  constexpr int IPW = D / 64;           // 1 KiB loads per wave per block (Q and dO: 2 TILEB)
  constexpr int KB_TILE = TILEB / 1024; // 1 KiB regions per tile
  static_assert(2 * KB_TILE == 8 * IPW, "8 waves load the two tiles");

  __shared__ __attribute__((aligned(16))) uint8_t smem[SLOTS * SLOTB];
  __shared__ __attribute__((aligned(16))) u32x4 xch[2][NW][4][64];      // [buf][pair][pb0 pb1 db0 db1][lane]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & (NW - 1);
  const int lr = lane & 31, hh = lane >> 5;
  const int N = a.N;
  const float sl2 = a.sl2;

  // heads vary fastest; under a causal mask the first key blocks see the most queries, so
  // the dispatch order is already heaviest first
  const int id = blockIdx.x;
  const int kblk = id / a.BH;
  const int bh = id - kblk * a.BH;
  const int k0 = kblk * NW * BLK;
  const int kw0 = k0 + pair * BLK;      // the pair's first key
  const int key = kw0 + lr;
  const size_t head = (size_t)bh * (size_t)N * D;

  // query blocks: causal ones start at the first block that holds a query >= k0. Every pair
  // takes every block from there: a pair whose keys lie past N, or follow all of a block's
  // queries, sees only masked probabilities and adds zeros (no branches around accumulators).
  const int nqb = (N + BLK - 1) / BLK;
  const int qb0 = CAUSAL ? k0 / BLK : 0;
  const int nq = nqb - qb0;

  // ---- loads of one block into a slot -------------------------------------------------------
  // Only the score waves load, at the end of their step (they reach the barrier first).
  // Score wave w fills the 1 KiB regions 2 IPW w .. 2 IPW w + 2 IPW - 1 of the slot's two
  // tiles: lane l writes physical chunk l % NC of row kb*(512/D) + l / NC, so it loads that
  // row's logical chunk (physical ^ swz(row)). Rows past N repeat row N-1 (masked later).
  // Waves 0 and 1 also load the block's 32 log-normalisers and deltas (lanes 32..63 repeat
  // lanes 0..31).
  constexpr int RPW = 2 * IPW;          // regions per loading wave
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)smem);
  const int lw = wave;                  // loading wave index (score waves)
  const int tile_of_wave = (min(lw, NW - 1) * RPW) / KB_TILE;  // 0: Q, 1: dO
  const uint8_t* tile_src = (const uint8_t*)(tile_of_wave == 0 ? a.q : a.dout) + head * 2;
  int dma_row[RPW];
  uint32_t dma_off[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int kb = (min(lw, NW - 1) * RPW + i) % KB_TILE;
    dma_row[i] = dma::tile_row<D>(kb, lane);
    dma_off[i] = dma::tile_off<D>(kb, lane);
  }
  const float* stat_src = lw == 0 ? a.lse + (size_t)bh * N : a.delta + (size_t)bh * N;
  auto issue = [&](int qb, int slot) __attribute__((always_inline)) {
    if (wave >= NW) return;
    const int row0 = qb * BLK;
    const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(lds_base + (uint32_t)(slot * SLOTB + tile_of_wave * TILEB)));
    const uint8_t* src = tile_src + (size_t)row0 * 2 * D;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const uint32_t back = dma::past_end_back(row0, dma_row[i], N, 2 * D);
      const int kb = (lw * RPW + i) % KB_TILE;
      dma16(src, dma_off[i] - back, dst + (uint32_t)(kb * 1024));
    }
    if (lw < 2) {
      const uint32_t sdst = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)(lds_base + (uint32_t)(slot * SLOTB + 2 * TILEB + lw * 256)));
      dma4(stat_src + row0, (uint32_t)(4 * min(lr, N - 1 - row0)), sdst);
    }
  };
  // vector-memory operations per block of a loading wave; the accumulators have none in flight
  auto barrier = [&]() __attribute__((always_inline)) {
    if (wave >= NW) step_barrier<0>();
    else if (lw < 2) step_barrier<RPW + 1>();
    else step_barrier<RPW>();
  };

  const TileOffsets<D> to(lane);
  // blocks qb0 and qb0+1 (a repeat of the last block when there is none) into slots 0 and 1;
  // step t (t = 0, 1, ...) issues block qb0+t+2 into slot (t+2) mod 5
  issue(qb0, 0);
  issue(min(qb0 + 1, nqb - 1), 1);
  auto next_slot = [](int sl) { return sl == SLOTS - 1 ? 0 : sl + 1; };

  if (wave < NW) {
    // ---- score role ----
    // K^T and V^T as B operands: lane l supplies key kw0 + l%32, features 16kk + 8hh .. +7;
    // a negative scale negates the keys (exact in bf16), and dK's sign comes at the end
    const uint32_t negmask = a.neg ? 0x80008000u : 0u;
    const uint16_t* __restrict__ Kh = (const uint16_t*)a.k + head;
    const uint16_t* __restrict__ Vh = (const uint16_t*)a.v + head;
    u32x4 kf[D / 16], vf[D / 16];
    {
      const uint32_t keep = key < N ? 0xffffffffu : 0u;
      const uint16_t* krow = Kh + (size_t)min(key, N - 1) * D;
      const uint16_t* vrow = Vh + (size_t)min(key, N - 1) * D;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        kf[kk] = (*(const u32x4*)(krow + 16 * kk + 8 * hh) & keep) ^ negmask;
        vf[kk] = *(const u32x4*)(vrow + 16 * kk + 8 * hh) & keep;
      }
    }
    // the key operands are plain loads: wait for them before counting the block loads
    __builtin_amdgcn_s_waitcnt(0xc07f & ~0xc00f);   // vmcnt(0)
    barrier();   // block qb0 landed (qb0 + 1 may still be in flight)

    // S = Q K^T, dP = dO V^T of the block in slot sl: lane = key, register i = query
    // 8(i/4) + 4hh + i%4
    auto products = [&](int sl, f32x16& sc, f32x16& dp) __attribute__((always_inline)) {
      const uint16_t* Qs = (const uint16_t*)(smem + sl * SLOTB);
      const uint16_t* dOs = Qs + QT;
      sc = (f32x16){};
      dp = (f32x16){};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const u32x4 qa = *(const u32x4*)(Qs + to.row[kk]);
        const u32x4 da = *(const u32x4*)(dOs + to.row[kk]);
        sc = mfma(qa, kf[kk], sc);
        dp = mfma(da, vf[kk], dp);
      }
    };
    // P and dS of block qb (statistics in slot sl: -lse log2 e and delta) into exchange
    // buffer xb
    auto softmax = [&](int qb, int sl, int xb, const f32x16& sc, const f32x16& dp) __attribute__((always_inline)) {
      const float* st = (const float*)(smem + sl * SLOTB + 2 * TILEB);
      const int qf0 = qb * BLK;
      f32x4 l4[4], d4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        l4[g] = *(const f32x4*)(st + 8 * g + 4 * hh);
        d4[g] = *(const f32x4*)(st + 64 + 8 * g + 4 * hh);
      }
      float p[16], ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) p[4 * g + t] = __builtin_amdgcn_exp2f(fmaf(sc[4 * g + t], sl2, l4[g][t]));
      // ragged or diagonal blocks only; the empty asm keeps this a branch rather than selects
      // on every block
      const bool masked = (qf0 + BLK > N) || (kw0 + BLK > N) || (CAUSAL && qf0 < kw0 + BLK - 1);
      if (masked) {
        asm volatile("");
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int qi = qf0 + 8 * g + 4 * hh + t;
            if (qi >= N || key >= N || (CAUSAL && key > qi)) p[4 * g + t] = 0.0f;
          }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) ds[4 * g + t] = p[4 * g + t] * (dp[4 * g + t] - d4[g][t]);
      u32x4* xo = &xch[xb][pair][0][lane];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        xo[64 * c] = (u32x4){pack_bf16x2(p[8 * c + 0], p[8 * c + 1]), pack_bf16x2(p[8 * c + 2], p[8 * c + 3]),
                             pack_bf16x2(p[8 * c + 4], p[8 * c + 5]), pack_bf16x2(p[8 * c + 6], p[8 * c + 7])};
        xo[64 * (2 + c)] = (u32x4){pack_bf16x2(ds[8 * c + 0], ds[8 * c + 1]), pack_bf16x2(ds[8 * c + 2], ds[8 * c + 3]),
                                   pack_bf16x2(ds[8 * c + 4], ds[8 * c + 5]), pack_bf16x2(ds[8 * c + 6], ds[8 * c + 7])};
      }
    };

    // step 0: products of block qb0
    f32x16 sa, da, sb, db;
    products(0, sa, da);
    issue(min(qb0 + 2, nqb - 1), 2);
    barrier();
    // step t >= 1: products of block qb0+t (a repeat of the last block at t = nq, unused)
    // beside the softmax of block qb0+t-1; unrolled by two so that the two register sets
    // swap roles without copies
    int sl_prev = 0, sl_cur = 1, sl_issue = 3;
    auto step = [&](int it, const f32x16& sc, const f32x16& dp, f32x16& sc_n, f32x16& dp_n) __attribute__((always_inline)) {
      products(sl_cur, sc_n, dp_n);
      softmax(qb0 + it - 1, sl_prev, (it - 1) & 1, sc, dp);
      // block qb0+it+2 into the slot that block qb0+it-3 left (read by nobody since the last
      // barrier)
      issue(min(qb0 + it + 2, nqb - 1), sl_issue);
      sl_prev = sl_cur;
      sl_cur = next_slot(sl_cur);
      sl_issue = next_slot(sl_issue);
      barrier();   // block qb0+it+1 landed; P / dS of block qb0+it-1 visible
    };
    int it = 1;
    for (; it + 1 <= nq; it += 2) {
      step(it, sa, da, sb, db);
      step(it + 1, sb, db, sa, da);
    }
    if (it <= nq) step(it, sa, da, sb, db);
    barrier();     // the accumulators' last block
  } else {
    // ---- accumulator role ----
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) { dk[dt][i] = 0.0f; dv[dt][i] = 0.0f; }

    // At step t the first accumulator wave turns the log-normalisers of block qb0+t (landed
    // by then, read by the score waves' softmax at step t+1) into -lse log2 e in place.
    auto prescale = [&](int sl) __attribute__((always_inline)) {
      if (wave == NW) {
        float* st = (float*)(smem + sl * SLOTB + 2 * TILEB);
        st[lane] *= -kLog2e;
      }
    };
    barrier();   // block qb0 landed
    // steps 0 and 1: the score waves form block qb0's products and then its P / dS
    prescale(0);
    barrier();
    prescale(1);
    barrier();
    // step t >= 2: accumulate block qb0+t-2
    int sl_acc = 0, sl_pre = 2;
    for (int it = 2; it <= nq + 1; ++it) {
      prescale(sl_pre);
      sl_pre = next_slot(sl_pre);
      const uint16_t* Qs = (const uint16_t*)(smem + sl_acc * SLOTB);
      const uint16_t* dOs = Qs + QT;
      const u32x4* xi = &xch[it & 1][pair][0][lane];
      u32x4 tq[D / 32][2], tdo[D / 32][2];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          tdo[dt][c] = read_tr<D>(dOs, c, to, dt);
          tq[dt][c] = read_tr<D>(Qs, c, to, dt);
        }
      const u32x4 pb[2] = {xi[0], xi[64]};
      const u32x4 db[2] = {xi[128], xi[192]};
      // dV^T += dO^T P and dK^T += Q^T dS over the block's two 16-query chunks
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          dv[dt] = mfma(tdo[dt][c], pb[c], dv[dt]);
          dk[dt] = mfma(tq[dt][c], db[c], dk[dt]);
        }
      sl_acc = next_slot(sl_acc);
      barrier();
    }

    // dK = scale * (Q^T dS)^T, dV as accumulated; lane = key, registers = features
    if (key < N) {
      const float kscale = (a.neg ? -sl2 : sl2) / kLog2e;
      uint16_t* dkrow = (uint16_t*)a.dk + head + (size_t)key * D;
      uint16_t* dvrow = (uint16_t*)a.dv + head + (size_t)key * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = dt * 32 + 8 * g + 4 * hh;
          const u32x2 wk = {pack_bf16x2(dk[dt][4 * g + 0] * kscale, dk[dt][4 * g + 1] * kscale),
                            pack_bf16x2(dk[dt][4 * g + 2] * kscale, dk[dt][4 * g + 3] * kscale)};
          const u32x2 wv = {pack_bf16x2(dv[dt][4 * g + 0], dv[dt][4 * g + 1]),
                            pack_bf16x2(dv[dt][4 * g + 2], dv[dt][4 * g + 3])};
          *(u32x2*)(dkrow + col) = wk;
          *(u32x2*)(dvrow + col) = wv;
        }
    }
  }
  // loads of blocks that nothing reads may still be landing: let them finish first
  wait_vm_lgkm0<0>();
}

// ---- dQ ------------------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 2)
void bwd_dq_kernel(BwdArgs a) {
  // A step covers 64 keys, two sub-tiles of 32: slot = [K sub 0][K sub 1][V sub 0][V sub 1],
  // each a swizzled [32][D] tile. Two slots: step t works on one while step t+1's keys land
  // in the other, loaded straight from global memory at the start of step t.
  constexpr int KT = BLK * D;           // one swizzled sub-tile (elements)
  constexpr int SLOT = 4 * KT;          // elements per slot
  constexpr int KB_SUB = 2 * KT / 1024; // 1 KiB regions per sub-tile: one wave loads one sub-tile
  static_assert(KB_SUB * 1024 == 2 * KT, "sub-tile size");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;
  const int N = a.N;
  const float sl2 = a.sl2;
  const uint32_t negmask = a.neg ? 0x80008000u : 0u;

  const int nqt = (N + NW * BLK - 1) / (NW * BLK);
  const int id = blockIdx.x;
  const int qt_rev = id / a.BH;
  const int bh = id - qt_rev * a.BH;
  const int qt = CAUSAL ? (nqt - 1 - qt_rev) : qt_rev;   // causal: heaviest first
  const int q0 = qt * NW * BLK;
  const int qw0 = q0 + wave * BLK;
  const int qi = qw0 + lr;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Qh = (const uint16_t*)a.q + head;
  const uint16_t* __restrict__ dOh = (const uint16_t*)a.dout + head;

  // Q'^T and dO^T as B operands (lane = query)
  u32x4 qf[D / 16], df[D / 16];
  const uint32_t keep = qi < N ? 0xffffffffu : 0u;
  {
    const uint16_t* qrow = Qh + (size_t)min(qi, N - 1) * D;
    const uint16_t* drow = dOh + (size_t)min(qi, N - 1) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qf[kk] = (*(const u32x4*)(qrow + 16 * kk + 8 * hh) & keep) ^ negmask;
      df[kk] = *(const u32x4*)(drow + 16 * kk + 8 * hh) & keep;
    }
  }
  const float lse2 = a.lse[(size_t)bh * N + min(qi, N - 1)] * kLog2e;
  // delta_i = sum_c dO_ic O_ic: this lane holds half of the row's features (8hh .. 8hh+7 of
  // every 16), the lane 32 apart the other half
  float dlt;
  {
    const uint16_t* orow = (const uint16_t*)a.o + head + (size_t)min(qi, N - 1) * D;
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const u32x4 x = *(const u32x4*)(orow + 16 * kk + 8 * hh);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        s0 = fmaf(bf16_lo(x[t]), bf16_lo(df[kk][t]), s0);
        s1 = fmaf(bf16_hi(x[t]), bf16_hi(df[kk][t]), s1);
      }
    }
    const float part = s0 + s1;
    dlt = part + __shfl_xor(part, 32);
    if (hh == 0 && qi < N) a.delta[(size_t)bh * N + qi] = dlt;
  }

  f32x16 dq[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[dt][i] = 0.0f;

  const int kv_end = CAUSAL ? min(N, q0 + NW * BLK) : N;

  // Wave w loads sub-tile w % 2 of K (w < 2) or V (w >= 2): lane l writes physical chunk
  // l % NC of row kb*(512/D) + l / NC of the sub-tile, i.e. that row's logical chunk
  // (physical ^ swz(row)). Key rows past N repeat row N-1; their probabilities are masked.
  // The per-lane offset is unsigned, so the base row is clamped to N-1 first: a sub-tile that
  // starts past N then reads row N-1 throughout.
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)smem);
  const uint8_t* ld_src = (const uint8_t*)(wave < 2 ? a.k : a.v) + head * 2;
  int dma_row[KB_SUB];
  uint32_t dma_off[KB_SUB];
#pragma unroll
  for (int i = 0; i < KB_SUB; ++i) {
    dma_row[i] = dma::tile_row<D>(i, lane);
    dma_off[i] = dma::tile_off<D>(i, lane);
  }
  auto issue = [&](int t, int slot) __attribute__((always_inline)) {
    // first key of this wave's sub-tile, clamped so that every offset below is >= 0
    static_assert(BLK == 32, "sub-tiles of the load arithmetic");
    const int row0 = dma::dq_row0(t, wave, N);
    const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(lds_base + (uint32_t)(slot * SLOT * 2 + wave * KT * 2)));
    const uint8_t* src = ld_src + (size_t)row0 * 2 * D;
#pragma unroll
    for (int i = 0; i < KB_SUB; ++i) {
      const uint32_t back = dma::past_end_back(row0, dma_row[i], N, 2 * D);   // rows past N-1 read row N-1
      dma16(src, dma_off[i] - back, dst + (uint32_t)(i * 1024));
    }
  };

  const TileOffsets<D> to(lane);
  const int nst = (kv_end + 2 * BLK - 1) / (2 * BLK);   // 64-key steps
  issue(0, 0);
  step_barrier<0>();
  // Every wave takes every key sub-tile: sub-tiles past a wave's last query (causal) or past
  // N see only masked probabilities and add zeros, which keeps the loop free of branches.
  for (int t = 0; t < nst; ++t) {
    if (t + 1 < nst) issue(t + 1, (t + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const uint16_t* Ks = smem + (t & 1) * SLOT + sub * KT;
      const uint16_t* Vs = Ks + 2 * KT;
      const int key0 = (2 * t + sub) * BLK;
      // S^T = K Q'^T, dP^T = V dO^T: lane = query, register i = key 8(i/4) + 4hh + i%4
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const u32x4 ka = *(const u32x4*)(Ks + to.row[kk]);
        const u32x4 va = *(const u32x4*)(Vs + to.row[kk]);
        s = mfma(ka, qf[kk], s);
        dp = mfma(va, df[kk], dp);
      }
      float pv[16], ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(s[i], sl2, -lse2));
      // ragged or diagonal sub-tiles only; the empty asm keeps this a branch rather than
      // selects on every sub-tile
      const bool masked = (key0 + BLK > N) || (qw0 + BLK > N) || (CAUSAL && key0 + BLK - 1 > qw0);
      if (masked) {
        asm volatile("");
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kj = key0 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (kj >= N || qi >= N || (CAUSAL && kj > qi)) pv[i] = 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = pv[i] * (dp[i] - dlt);
      u32x4 db[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
        db[c] = (u32x4){pack_bf16x2(ds[8 * c + 0], ds[8 * c + 1]), pack_bf16x2(ds[8 * c + 2], ds[8 * c + 3]),
                        pack_bf16x2(ds[8 * c + 4], ds[8 * c + 5]), pack_bf16x2(ds[8 * c + 6], ds[8 * c + 7])};
      // dQ^T += K^T dS^T
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) dq[dt] = mfma(read_tr<D>(Ks, c, to, dt), db[c], dq[dt]);
    }
    // the next step's keys have landed (each wave waits for its own loads) and nobody reads
    // this step's slot any more
    step_barrier<0>();
  }

  // dQ = scale * (dS K): |scale| from the accumulation, sign from the flipped q
  if (qi < N) {
    const float qscale = (a.neg ? -1.0f : 1.0f) * (sl2 / kLog2e);
    uint16_t* dqrow = (uint16_t*)a.dq + head + (size_t)qi * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = dt * 32 + 8 * g + 4 * hh;
        const u32x2 w = {pack_bf16x2(dq[dt][4 * g + 0] * qscale, dq[dt][4 * g + 1] * qscale),
                         pack_bf16x2(dq[dt][4 * g + 2] * qscale, dq[dt][4 * g + 3] * qscale)};
        *(u32x2*)(dqrow + col) = w;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
  const unsigned nblk = (unsigned)((a.N + NW * BLK - 1) / (NW * BLK));
  // dQ first: it writes delta, which the dK/dV kernel reads
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)a.BH * nblk), dim3(NT), 0, stream, a);
  // the dK/dV kernel reads the delta rows the dQ kernel writes: launch it only if that launch went in
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)a.BH * nblk), dim3(DKDV_NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int bwd_rows_per_block() { return NW * BLK; }

hipError_t launch_bwd_bf16(const BwdArgs& a, bool causal, hipStream_t stream) {
  if (a.d == 64) return causal ? launch_bwd_d<64, true>(a, stream) : launch_bwd_d<64, false>(a, stream);
  return causal ? launch_bwd_d<128, true>(a, stream) : launch_bwd_d<128, false>(a, stream);
}

}  // namespace fa
