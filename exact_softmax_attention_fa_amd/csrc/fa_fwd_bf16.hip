// Fused forward pass of exact softmax attention, bf16 inputs, for gfx950 (CDNA4).
//
// Method (liminalml.com "FlashAttention", online update equations; interactiveml.org
// "FlashAttention saves the matrix, not the quadratic work"): every query row keeps a
// running maximum m, a denominator l and an unnormalised numerator u; for each block of
// keys, m' = max(m, max s), both l and u are multiplied by e^(m - m'), and the block adds
// p = e^(s - m') to l and p V to u. After the last block the row is u / l. Query and key
// dimensions are both tiled and the whole computation is fused (interactiveml.org, same
// page), so no N x N matrix leaves the chip (sadullah.online, "fused, tiled computation").
//
// gfx950 mapping
// --------------
// * One workgroup = NW waves of 64 lanes; each wave owns QW blocks of 32 query rows, so a
//   workgroup covers BR = NW*QW*32 queries of one (b, h). Q stays in VGPRs as MFMA operands.
// * K and V tiles of BC keys are staged in LDS, double-buffered: the global loads of tile
//   j+1 are issued before the MFMAs of tile j and written to the other buffer afterwards.
// * Both products use v_mfma_f32_32x32x16_bf16 with fp32 accumulation, computed transposed:
//     S^T (keys x queries) = K Q^T      and      O^T (d x queries) += V^T P^T.
//   In the 32x32 accumulator layout lane l holds column l%32, so every lane holds 16
//   scores of ONE query, and in O^T every lane holds 16 output features of ONE query.
//   Row statistics are then per-lane registers (one cross-half exchange per tile), the
//   rescale of u is a per-lane multiply, and the probabilities go from the S^T
//   accumulator straight into the B operand of the second product with no data movement:
//   accumulator register i of lane l holds key 8*(i/4) + 4*(l/32) + i%4 of the 32-key
//   block, and registers 8c..8c+7 are exactly the 8 contraction slots lane l supplies for
//   16-key chunk c, provided the A operand (V^T) supplies the same keys in those slots.
// * V^T operands are read from the row-major V tile with ds_read_b64_tr_b16 (a gfx950
//   transpose read): in each group of 16 lanes, lane 4r+q points at key row r and
//   features 4q..4q+3, and lane i receives feature i of the four rows. Two such reads give
//   the 8 keys a lane needs.
// * The scores are kept in base-2 units (scale * log2 e folded into one FMA before
//   v_exp_f32). The running maximum is only raised when the new maximum exceeds it by more
//   than 2^8 in probability terms; otherwise the stale maximum stays, probabilities may
//   reach 2^8, and l and u stay consistent because both use the same reference. The
//   result is the same function; only the rounding differs.
// * Causal: key tiles past the workgroup's last query are never loaded, a wave skips the
//   tiles past its own last query, and only tiles that straddle the diagonal (or the ragged
//   end of the keys) are masked, by setting their dead scores to -inf before the update that
//   every tile shares. Workgroups are issued heaviest first.
// * Block shapes (Cfg): per padded head width, and at width 64 per grid size (4 waves with no
//   key split on large grids, 2 waves with up to 4 key groups on small ones). A small grid
//   splits the key range over key groups inside the workgroup, which merge their (m, l, u)
//   through LDS at the end (interactiveml.org, merge of the three sufficient statistics).
// * Row loads and stores (LD): whole 16-byte chunks at the full padded width; whole chunks or
//   none when the width is a multiple of 8; element by element otherwise.
// * PARTIAL instantiations run the split-KV partial pass: the workgroup covers one column of
//   the key range (blockIdx.y) and writes its (m, l, u) to the caller's workspace for the
//   merge kernel (fa_splitkv.hip) instead of o and lse.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kRescaleThreshold = 8.0f;  // log2 units: rescale when the max rises by > 2^8

// Largest grid (workgroups) that gets a key split: one workgroup per CU of the 256, so that a
// split workgroup only needs room for its own waves.
#ifndef FA_SPLIT_MAX_WGS
#define FA_SPLIT_MAX_WGS 256
#endif

// Tile configuration per padded head width: QW query blocks of 32 per wave, NW waves per
// workgroup, BC keys per LDS tile. The defaults can be overridden at build time for sweeps.
#ifndef FA_BF16_D64_QW
#define FA_BF16_D64_QW 1
#endif
#ifndef FA_BF16_D64_NW
#define FA_BF16_D64_NW 2
#endif
#ifndef FA_BF16_D64_BC
#define FA_BF16_D64_BC 64
#endif
#ifndef FA_BF16_D128_QW
#define FA_BF16_D128_QW 1
#endif
#ifndef FA_BF16_D128_NW
#define FA_BF16_D128_NW 8
#endif
#ifndef FA_BF16_D128_BC
#define FA_BF16_D128_BC 64
#endif
// minimum waves per SIMD the register allocation must allow (1: up to 512 registers)
#ifndef FA_BF16_D64_WPE
#define FA_BF16_D64_WPE 2
#endif
#ifndef FA_BF16_D128_WPE
#define FA_BF16_D128_WPE 2
#endif
#ifndef FA_BF16_D64W_NW
#define FA_BF16_D64W_NW 4
#endif
// Grids of at least this many workgroups of the wide head-width-64 configuration use it.
#ifndef FA_BF16_D64W_MIN_WGS
#define FA_BF16_D64W_MIN_WGS 256
#endif
// NW counts the waves of one key group; a workgroup runs SPLIT key groups (MAXSPLIT at most)
// over the same queries and merges them at the end. D is the padded head width.
template <int D_> struct Cfg;
template <> struct Cfg<64> {
  static constexpr int D = 64;
  static constexpr int QW = FA_BF16_D64_QW, NW = FA_BF16_D64_NW, BC = FA_BF16_D64_BC, WPE = FA_BF16_D64_WPE;
  static constexpr int MAXSPLIT = 4;
};
// Head widths up to 64 on large grids: 4 waves share each K/V tile (half the tile loads per
// query of the 2-wave blocks), no key split; three such workgroups fit one CU (measured at
// B1 H16 N8192 against 8 waves, of which only one workgroup fits: d64 865 against 851
// TFLOP/s, d32 463 against 418). The 2-wave blocks with their key split stay the choice for
// small grids, where the wide blocks would leave CUs idle.
struct CfgD64Wide {
  static constexpr int D = 64;
  static constexpr int QW = 1, NW = FA_BF16_D64W_NW, BC = 64, WPE = 2;
  static constexpr int MAXSPLIT = 1;
};
template <> struct Cfg<128> {
  static constexpr int D = 128;
  static constexpr int QW = FA_BF16_D128_QW, NW = FA_BF16_D128_NW, BC = FA_BF16_D128_BC, WPE = FA_BF16_D128_WPE;
  static constexpr int MAXSPLIT = 1;
};
// head widths 129..256: one wave per SIMD (the 256-wide accumulators and operands need more
// than 256 registers), 4 waves of 32 query rows
template <> struct Cfg<256> {
  static constexpr int D = 256;
  static constexpr int QW = 1, NW = 4, BC = 32, WPE = 1;
  static constexpr int MAXSPLIT = 1;
};

// Whether a head-width-64 forward call over BH heads of N queries runs the wide blocks.
bool d64_wide(int64_t BH, int N) {
  constexpr int rows = CfgD64Wide::NW * CfgD64Wide::QW * 32;
  return BH * (((int64_t)N + rows - 1) / rows) >= FA_BF16_D64W_MIN_WGS;
}

__device__ __forceinline__ float pair_max(float x) {
  // lanes l and l^32 exchange x; after the swap each lane holds both halves' values
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // one v_cvt_pk_bf16_f32: both halves rounded to nearest even
  const f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// How a kernel reads rows of q, k, v and writes rows of o (d = stored head width, D = padded):
//   LD_FULL  d == D: whole 16-byte chunks
//   LD_VEC8  d a multiple of 8: a chunk lies wholly inside the row or wholly past its end, so
//            chunks are read or written whole, or skipped (zero)
//   LD_ELEM  any other d: element by element, columns past d read as zero
enum { LD_FULL = 0, LD_VEC8 = 1, LD_ELEM = 2 };

// 8 consecutive bf16 of one row, zero outside [0, d) (generic head width). The row starts at
// element row0 of base; elements are addressed by 32-bit indices off the uniform base, so that
// no 64-bit address per element stays live. The loads are unconditional (column clamped) so
// that they issue together.
__device__ __forceinline__ u32x4 load8_masked(const uint16_t* base, uint32_t row0, int col, int d) {
  uint16_t e[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint16_t x = base[row0 + (uint32_t)min(col + t, d - 1)];
    e[t] = (col + t < d) ? x : (uint16_t)0;
  }
  u32x4 r;
  r[0] = e[0] | ((uint32_t)e[1] << 16);
  r[1] = e[2] | ((uint32_t)e[3] << 16);
  r[2] = e[4] | ((uint32_t)e[5] << 16);
  r[3] = e[6] | ((uint32_t)e[7] << 16);
  return r;
}

// Everything one wave does with one K/V tile in LDS: S^T = K Q^T, the online-softmax
// update of its QW query blocks, and O^T += V^T P^T. `masked` (uniform over the wave) hides
// keys >= N and, when causal, keys past each query, by setting their scores to -inf before
// the shared update: sl2 > 0, so the tile maximum max(s) * sl2 equals max(s * sl2) and
// exp2(fma(-inf, sl2, -m)) = 0. One update path for both kinds of tile keeps a single copy
// of the accumulators in the loops that mix them.
template <int D, int QW, int BC, int KP, int VP, bool CAUSAL>
__device__ __forceinline__ void tile_step(const uint16_t* __restrict__ Ks, const uint16_t* __restrict__ Vs,
                                          const u32x4 (&qf)[QW][D / 16], f32x16 (&acc)[QW][D / 32],
                                          float (&m_run)[QW], float (&l_run)[QW],
                                          int key0, int N, int wq_lo, float sl2, int lr, int hh,
                                          int tr_row, int tr_col, bool masked) {
  // ---- S^T = K Q^T : per 32-key block, all K operands are read before the MFMA chain ----
  f32x16 s[QW][BC / 32];
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb) {
    // (head widths up to 128: all K operands of the block are read before the MFMA chain;
    // wider heads read them as the chain goes, to bound the registers)
    constexpr int KOPS = D <= 128 ? D / 16 : 1;   // (unused for wider heads)
    u32x4 kop[KOPS];
    const uint16_t* krow = Ks + (kb * 32 + lr) * KP + 8 * hh;
    if constexpr (D <= 128) {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) kop[kk] = *(const u32x4*)(krow + 16 * kk);
    }
#pragma unroll
    for (int qb = 0; qb < QW; ++qb) {
      f32x16 c = {};
      if constexpr (D <= 128) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kop[kk]),
                                                      __builtin_bit_cast(bf16x8, qf[qb][kk]), c, 0, 0, 0);
      } else {
        // two operands in flight; the scheduling barriers keep the compiler from hoisting
        // every read of the chain to its start
        u32x4 k0 = *(const u32x4*)krow, k1 = *(const u32x4*)(krow + 16);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const u32x4 kv = k0;
          k0 = k1;
          if (kk + 2 < D / 16) k1 = *(const u32x4*)(krow + 16 * (kk + 2));
          __builtin_amdgcn_sched_barrier(0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv),
                                                      __builtin_bit_cast(bf16x8, qf[qb][kk]), c, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      s[qb][kb] = c;
    }
  }

  // ---- online softmax update, one query per lane ----------------------------------------
  u32x4 pb[QW][BC / 16];   // probabilities as bf16: the B operand chunks of 16 keys
#pragma unroll
  for (int qb = 0; qb < QW; ++qb) {
    const int qi = wq_lo + qb * 32 + lr;
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (key >= N || (CAUSAL && key > qi)) s[qb][kb][i] = -INFINITY;
        }
    }
    float m0 = s[qb][0][0], m1 = s[qb][0][1];
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int i = (kb == 0 ? 2 : 0); i < 16; i += 2) {
        m0 = fmaxf(m0, s[qb][kb][i]);
        m1 = fmaxf(m1, s[qb][kb][i + 1]);
      }
    float mt = pair_max(fmaxf(m0, m1) * sl2);
    const float m_new = fmaxf(m_run[qb], mt);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run[qb] + kRescaleThreshold)) {
      const float alpha = exp2f(m_run[qb] - m_new);  // 0 while m_run is -inf
      l_run[qb] *= alpha;
      // In-place multiply: tying each output to its input register keeps the compiler from
      // copying the whole accumulator to merge the taken and not-taken paths. (The 256-wide
      // accumulators live in AGPRs, which the VGPR constraint would force out of them.) The
      // compiler does not count inline asm as a reader of a transcendental result, which needs a
      // wait state after the v_exp_f32 that may write it; the s_nop in front provides it.
      float alpha_r = alpha;
      if constexpr (D <= 128) asm volatile("s_nop 1" : "+v"(alpha_r));
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if constexpr (D <= 128) asm("v_mul_f32 %0, %0, %1" : "+v"(acc[qb][dt][i]) : "v"(alpha_r));
          else acc[qb][dt][i] *= alpha;
        }
      m_run[qb] = m_new;
    }
    const float msub = (m_run[qb] == -INFINITY) ? 0.0f : m_run[qb];
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][i], sl2, -msub));
        ls[i & 3] += p[i];
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 w;
        w[0] = pack_bf16x2(p[8 * c + 0], p[8 * c + 1]);
        w[1] = pack_bf16x2(p[8 * c + 2], p[8 * c + 3]);
        w[2] = pack_bf16x2(p[8 * c + 4], p[8 * c + 5]);
        w[3] = pack_bf16x2(p[8 * c + 6], p[8 * c + 7]);
        pb[qb][2 * kb + c] = w;
      }
    }
    l_run[qb] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  }

  // ---- O^T += V^T P^T --------------------------------------------------------------------
  auto v_operand = [&](int dt, int c16) __attribute__((always_inline)) {
    const uint16_t* base = Vs + (c16 * 16 + tr_row) * VP + dt * 32 + tr_col;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 8 * VP));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
    return (u32x4){lo2[0], lo2[1], hi2[0], hi2[1]};
  };
  if constexpr (D <= 128) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int c16 = 0; c16 < BC / 16; ++c16) {
        const u32x4 av = v_operand(dt, c16);
#pragma unroll
        for (int qb = 0; qb < QW; ++qb)
          acc[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, pb[qb][c16]), acc[qb][dt], 0, 0, 0);
      }
    }
  } else {
    // steps st = (dt, c16) in order, two operands in flight (as in the S chain above)
    constexpr int ST = (D / 32) * (BC / 16);
    u32x4 v0 = v_operand(0, 0), v1 = v_operand(1 / (BC / 16), 1 % (BC / 16));
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      const int dt = st / (BC / 16), c16 = st % (BC / 16);
      const u32x4 av = v0;
      v0 = v1;
      if (st + 2 < ST) v1 = v_operand((st + 2) / (BC / 16), (st + 2) % (BC / 16));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int qb = 0; qb < QW; ++qb)
        acc[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, pb[qb][c16]), acc[qb][dt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Minimum waves per SIMD the register allocation must allow: a workgroup of two waves or fewer
// may use the whole register file (larger ones keep the configured occupancy).
template <class C, int SPLIT> constexpr int min_waves_per_simd() { return C::NW * SPLIT <= 2 ? 1 : C::WPE; }

// PARTIAL: the workgroup covers only the keys of its split column (blockIdx.y) and writes its
// partial state (m, l, u) to the workspace instead of o and lse; a merge pass combines them.
template <class C, bool CAUSAL, int LD, int SPLIT, bool PARTIAL>
__global__ __launch_bounds__(C::NW * SPLIT * 64, (min_waves_per_simd<C, SPLIT>()))
void fwd_bf16_kernel(FwdArgs a) {
  constexpr int D = C::D, QW = C::QW, NW = C::NW, BC = C::BC;
  constexpr int NT = NW * SPLIT * 64;
  constexpr int BR = NW * QW * 32;
  constexpr int KP = D + 8;    // K row pitch (elements): conflict-free 16-byte reads of 32 rows
  constexpr int VP = D + 16;   // V row pitch: conflict-free transpose reads of 4 rows
  constexpr int KT = BC * KP, VT = BC * VP;
  constexpr int CH = BC * D / 8;      // 16-byte chunks per K (or V) tile
  constexpr int CPT = SPLIT * CH / NT;  // chunks per thread (SPLIT tiles per step)
  static_assert((SPLIT * CH) % NT == 0, "tiles must split evenly over the workgroup");
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shapes");
  // one value block per (query wave, extra key group) for the final merge
  constexpr int NV = QW * (D / 32 * 16 + 2);
  static_assert(SPLIT == 1 || NW * (SPLIT - 1) * NV * 64 * 4 <= 2 * SPLIT * (KT + VT) * 2,
                "merge area must fit in the tile buffers");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * SPLIT * (KT + VT)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = tid >> 6;
  const int grpk = wave_all / NW;    // key group: takes tiles grpk, grpk + SPLIT, ...
  const int wave = wave_all - grpk * NW;   // query wave within the workgroup
  const int lr = lane & 31, hh = lane >> 5;
  const int N = a.N, d = a.d;

  // Scheduler: heads vary fastest, so consecutive workgroups (which the dispatcher spreads
  // round-robin over the 8 XCDs) keep one head on one XCD whenever B*H is a multiple of 8.
  // (workgroups off the first XCD exit at once when the grid is packed onto one XCD; the
  // exit is uniform over the workgroup and comes before any barrier)
  if (blockIdx.x & ((1u << a.wg_shift) - 1u)) return;
  const int id = (int)(blockIdx.x >> a.wg_shift);
  const int qt_rev = id / a.BH;
  const int bh = id - qt_rev * a.BH;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - qt_rev) : qt_rev;
  const int q0 = qt * BR;

  const size_t head = (size_t)bh * (size_t)N * (size_t)d;
  const uint16_t* __restrict__ Qh = (const uint16_t*)a.q + head;
  const uint16_t* __restrict__ Kh = (const uint16_t*)a.k + head;
  const uint16_t* __restrict__ Vh = (const uint16_t*)a.v + head;
  uint16_t* __restrict__ Oh = (uint16_t*)a.o + head;

  const int wq_lo = q0 + wave * QW * 32;   // first query of this wave
  const int wq_hi = wq_lo + QW * 32 - 1;   // last query of this wave

  // Q fragments: B operand of S^T = K Q^T. Lane l supplies query l%32, features 16kk+8hh..+7.
  // (unconditional loads from a clamped row, so that they are all in flight together;
  // rows past N become 0)
  u32x4 qf[QW][D / 16];
  const uint32_t negmask = a.neg ? 0x80008000u : 0u;
#pragma unroll
  for (int qb = 0; qb < QW; ++qb) {
    const int qi = wq_lo + qb * 32 + lr;
    const uint32_t qrow0 = (uint32_t)min(qi, N - 1) * (uint32_t)d;
    const uint16_t* qrow = Qh + qrow0;
    const uint32_t keep = qi < N ? 0xffffffffu : 0u;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int col = 16 * kk + 8 * hh;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (LD == LD_FULL || (LD == LD_VEC8 && col < d)) x = *(const u32x4*)(qrow + col);
      else if (LD == LD_ELEM) x = load8_masked(Qh, qrow0, col, d);
      qf[qb][kk] = (x & keep) ^ negmask;
    }
  }

  // Key range of this workgroup: all keys up to the last query (causal) or N, restricted to
  // its split column when the key range is split over workgroups. A column that holds no key
  // any of its queries may see has nothing to contribute (the merge skips it).
  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  int key_beg = 0, key_stop = kv_end;
  if constexpr (PARTIAL) {
    key_beg = (int)blockIdx.y * a.kv_chunk;
    key_stop = min(kv_end, key_beg + a.kv_chunk);
    if (key_beg >= key_stop) return;   // uniform over the workgroup, before any barrier
  }
  const int t_beg = key_beg / BC;                       // first tile (kv_chunk is a tile multiple)
  const int nkv = (key_stop + BC - 1) / BC - t_beg;     // tiles of this workgroup

  f32x16 acc[QW][D / 32];
#pragma unroll
  for (int qb = 0; qb < QW; ++qb)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[qb][dt][i] = 0.0f;
  float m_run[QW], l_run[QW];
#pragma unroll
  for (int qb = 0; qb < QW; ++qb) { m_run[qb] = -INFINITY; l_run[qb] = 0.0f; }

  // Global -> register staging of one K/V tile. Chunk c covers row c/(D/8), features
  // 8*(c%(D/8))..+7; consecutive threads read consecutive 16-byte pieces of a row.
  u32x4 kreg[CPT], vreg[CPT];
  // step `it` stages tiles it*SPLIT .. it*SPLIT + SPLIT-1 (one per key group)
  auto gload = [&](int it) {
    const int key_lo = (t_beg + it * SPLIT) * BC;
    const bool whole = LD != LD_ELEM && key_lo + SPLIT * BC <= N;   // every staged key exists
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int c = tid + r * NT;
      const int row = c / (D / 8);      // row within the SPLIT*BC staged keys
      const int col = (c % (D / 8)) * 8;
      const int key = key_lo + row;
      // one 32-bit element offset serves K and V (N * d < 2^31), so that the loop keeps no
      // 64-bit address per chunk live
      const uint32_t e = (uint32_t)key * (uint32_t)d + (uint32_t)col;
      if (whole && LD == LD_FULL) {
        kreg[r] = *(const u32x4*)(Kh + e);
        vreg[r] = *(const u32x4*)(Vh + e);
      } else {
        u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
        if (LD == LD_VEC8) {
          if ((whole || key < N) && col < d) {
            kx = *(const u32x4*)(Kh + e);
            vx = *(const u32x4*)(Vh + e);
          }
        } else if (key < N) {
          const uint32_t row0 = (uint32_t)key * (uint32_t)d;
          kx = LD == LD_FULL ? *(const u32x4*)(Kh + e) : load8_masked(Kh, row0, col, d);
          vx = LD == LD_FULL ? *(const u32x4*)(Vh + e) : load8_masked(Vh, row0, col, d);
        }
        kreg[r] = kx;
        vreg[r] = vx;
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int c = tid + r * NT;
      const int row = c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      uint16_t* Ks = smem + (buf * SPLIT + row / BC) * (KT + VT);
      uint16_t* Vs = Ks + KT;
      const int tr = row % BC;
      *(u32x4*)(Ks + tr * KP + col) = kreg[r];
      *(u32x4*)(Vs + tr * VP + col) = vreg[r];
    }
  };
  auto tile_buf = [&](int buf) { return (const uint16_t*)smem + (buf * SPLIT + grpk) * (KT + VT); };

  const int nit = (nkv + SPLIT - 1) / SPLIT;   // steps of SPLIT tiles
  gload(0);
  swrite(0);
  __syncthreads();

  // Lane roles in the transpose read of V: in each group of 16 lanes, lane 4r+q points at
  // key row r (second read: r+8) and features 4q..4q+3 of a 16-wide half of a 32-block.
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // Tiles [0, j_split) hold only keys that every query of the workgroup may see, so they
  // take the unmasked path with no per-tile decision; the remaining tiles (the causal
  // diagonal, or the ragged last tile) take the masked path, and under a causal mask a wave
  // skips the tiles that lie entirely past its own last query. Key group g handles tiles
  // it*SPLIT + g.
  // (tile indices below are relative to t_beg; in a split column the unmasked tiles end at the
  // column's end or earlier, and may not exist at all)
  const int j_unmasked = CAUSAL ? min(N / BC, (q0 + 1) / BC) : N / BC;
  const int j_split = PARTIAL ? min(nkv, j_unmasked - t_beg) : j_unmasked;
  const int it_split = PARTIAL ? max(j_split, 0) / SPLIT : j_split / SPLIT;   // steps whose tiles are all unmasked
  int it = 0;
  for (; it < it_split; ++it) {
    const int buf = it & 1;
    if (it + 1 < nit) gload(it + 1);
    const uint16_t* Ks = tile_buf(buf);
    tile_step<D, QW, BC, KP, VP, CAUSAL>(Ks, Ks + KT, qf, acc, m_run, l_run, (t_beg + it * SPLIT + grpk) * BC, N,
                                        wq_lo, a.sl2, lr, hh, tr_row, tr_col, false);
    if (it + 1 < nit) swrite(buf ^ 1);
    __syncthreads();
  }
  for (; it < nit; ++it) {
    const int buf = it & 1;
    if (it + 1 < nit) gload(it + 1);
    const uint16_t* Ks = tile_buf(buf);
    const int t = it * SPLIT + grpk;
    const int key0 = (t_beg + t) * BC;
    if (t < nkv && (!CAUSAL || key0 <= wq_hi))
      tile_step<D, QW, BC, KP, VP, CAUSAL>(Ks, Ks + KT, qf, acc, m_run, l_run, key0, N, wq_lo, a.sl2, lr, hh,
                                          tr_row, tr_col, t >= j_split);
    if (it + 1 < nit) swrite(buf ^ 1);
    __syncthreads();
  }

  // ---- merge of the key groups (split of the key range inside the workgroup) -------------
  // Each group holds (m, l, u) for its keys; with m* = max m_g the row's state is
  // l = sum l_g 2^(m_g - m*), u = sum u_g 2^(m_g - m*) (interactiveml.org, merge of the three
  // sufficient statistics). Groups 1.. hand their state to group 0 through LDS (the tile
  // buffers are free after the last barrier of the loop).
  if constexpr (SPLIT > 1) {
    float* mb = (float*)smem;
    if (grpk > 0) {
      float* dst = mb + (size_t)((wave * (SPLIT - 1) + grpk - 1) * NV) * 64 + lane;
#pragma unroll
      for (int qb = 0; qb < QW; ++qb) {
        const int v0 = qb * (D / 32 * 16 + 2);
        dst[(v0 + 0) * 64] = m_run[qb];
        dst[(v0 + 1) * 64] = l_run[qb];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) dst[(v0 + 2 + dt * 16 + i) * 64] = acc[qb][dt][i];
      }
    }
    __syncthreads();
    if (grpk > 0) return;
#pragma unroll
    for (int g = 1; g < SPLIT; ++g) {
      const float* src = mb + (size_t)((wave * (SPLIT - 1) + g - 1) * NV) * 64 + lane;
#pragma unroll
      for (int qb = 0; qb < QW; ++qb) {
        const int v0 = qb * (D / 32 * 16 + 2);
        const float mg = src[(v0 + 0) * 64], lg = src[(v0 + 1) * 64];
        const float ms = fmaxf(m_run[qb], mg);
        // weights 2^(m - m*); a group that saw no key has m = -inf and weight 0
        const float w0 = (m_run[qb] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run[qb] - ms);
        const float wg = (mg == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mg - ms);
        l_run[qb] = l_run[qb] * w0 + lg * wg;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[qb][dt][i] = acc[qb][dt][i] * w0 + src[(v0 + 2 + dt * 16 + i) * 64] * wg;
        m_run[qb] = ms;
      }
    }
  }

  // ---- partial epilogue: the state (m, l, u) of this key range, unnormalised ---------------
  // m is the reference of the exponentials in base-2 units (-inf for a row that saw no key
  // of this range; then l = 0 and u = 0).
  if constexpr (PARTIAL) {
    const size_t col_base = (size_t)blockIdx.y * a.BH + bh;
#pragma unroll
    for (int qb = 0; qb < QW; ++qb) {
      const int qi = wq_lo + qb * 32 + lr;
      const float l_tot = pair_sum(l_run[qb]);
      if (qi < N) {
        const size_t row = col_base * N + qi;
        float* urow = a.part_u + row * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 w = {acc[qb][dt][4 * g + 0], acc[qb][dt][4 * g + 1], acc[qb][dt][4 * g + 2],
                              acc[qb][dt][4 * g + 3]};
            *(float4*)(urow + dt * 32 + 8 * g + 4 * hh) = w;
          }
        if (hh == 0) *(float2*)(a.part_ml + 2 * row) = make_float2(m_run[qb], l_tot);
      }
    }
    return;
  }

  // ---- epilogue: o = u / l, lse = (m + log2 l) * ln 2 ----------------------------------------
#pragma unroll
  for (int qb = 0; qb < QW; ++qb) {
    const int qi = wq_lo + qb * 32 + lr;
    const float l_tot = pair_sum(l_run[qb]);
    const float inv = 1.0f / l_tot;
    if (qi < N) {
      uint16_t* orow = Oh + (size_t)qi * d;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = dt * 32 + 8 * g + 4 * hh;   // 4 consecutive features
          const float x0 = acc[qb][dt][4 * g + 0] * inv, x1 = acc[qb][dt][4 * g + 1] * inv;
          const float x2 = acc[qb][dt][4 * g + 2] * inv, x3 = acc[qb][dt][4 * g + 3] * inv;
          if (LD == LD_FULL || (LD == LD_VEC8 && col < d)) {
            const u32x2 w = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
            *(u32x2*)(orow + col) = w;
          } else if (LD == LD_ELEM) {
            const float xs[4] = {x0, x1, x2, x3};
#pragma unroll
            for (int t = 0; t < 4; ++t)
              if (col + t < d) orow[col + t] = __builtin_bit_cast(uint16_t, (__bf16)xs[t]);
          }
        }
      if (a.lse != nullptr && hh == 0) {
        const float msub = (m_run[qb] == -INFINITY) ? 0.0f : m_run[qb];
        a.lse[(size_t)bh * N + qi] = (msub + log2f(l_tot)) * 0.69314718055994531f;
      }
    }
  }
}

template <class C, bool CAUSAL, int SPLIT, bool PARTIAL>
hipError_t launch_split(const FwdArgs& a, int ld, int ncol, hipStream_t stream) {
  const dim3 grid((unsigned)(a.BH * a.n_qtiles) << a.wg_shift, (unsigned)ncol);
  const dim3 block(C::NW * SPLIT * 64);
  // (head width exactly 128 runs on the tuned kernel in a single pass, so the generic 128-wide
  // kernel is built for full rows only where the split pass uses it)
  if constexpr (C::D != 128 || PARTIAL) {
    if (ld == LD_FULL) {
      hipLaunchKernelGGL((fwd_bf16_kernel<C, CAUSAL, LD_FULL, SPLIT, PARTIAL>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  }
  if (ld == LD_VEC8)
    hipLaunchKernelGGL((fwd_bf16_kernel<C, CAUSAL, LD_VEC8, SPLIT, PARTIAL>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<C, CAUSAL, LD_ELEM, SPLIT, PARTIAL>), grid, block, 0, stream, a);
  return hipGetLastError();
}

// Key groups per workgroup: split the key range as far as MAXSPLIT allows when the grid has
// at most one workgroup per CU, as long as every group still gets at least two tiles.
// `keys` is the length of one workgroup's key range, `ncol` the number of split columns.
template <class C>
int choose_split(const FwdArgs& a, int keys, int ncol) {
  const long long wgs = (long long)a.BH * a.n_qtiles * ncol;
  const int nkv = (keys + C::BC - 1) / C::BC;
  int split = 1;
  while (split * 2 <= C::MAXSPLIT && wgs <= FA_SPLIT_MAX_WGS && nkv >= 2 * split * 2) split *= 2;
  return split;
}

template <class C, bool CAUSAL, bool PARTIAL>
hipError_t launch_one(const FwdArgs& a, int ld, int ncol, hipStream_t stream) {
  if constexpr (C::MAXSPLIT >= 4) {
    const int split = choose_split<C>(a, PARTIAL ? a.kv_chunk : a.N, ncol);
    if (split == 4) return launch_split<C, CAUSAL, 4, PARTIAL>(a, ld, ncol, stream);
    if (split == 2) return launch_split<C, CAUSAL, 2, PARTIAL>(a, ld, ncol, stream);
  }
  return launch_split<C, CAUSAL, 1, PARTIAL>(a, ld, ncol, stream);
}

template <class C, bool PARTIAL>
hipError_t launch_causal(const FwdArgs& a, int ld, bool causal, int ncol, hipStream_t stream) {
  return causal ? launch_one<C, true, PARTIAL>(a, ld, ncol, stream)
                : launch_one<C, false, PARTIAL>(a, ld, ncol, stream);
}

// The split pass (PARTIAL) always runs the narrow configurations; the single pass at head
// width 64 takes the wide blocks where d64_wide says so (its grid was sized for them).
template <bool PARTIAL>
hipError_t launch_generic(const FwdArgs& a, int d_pad, bool causal, int ncol, hipStream_t stream) {
  const int ld = a.d == d_pad ? LD_FULL : (a.d % 8 == 0 ? LD_VEC8 : LD_ELEM);
  if (d_pad == 64) {
    if (!PARTIAL && d64_wide(a.BH, a.N)) return launch_causal<CfgD64Wide, false>(a, ld, causal, ncol, stream);
    return launch_causal<Cfg<64>, PARTIAL>(a, ld, causal, ncol, stream);
  }
  if (d_pad == 128) return launch_causal<Cfg<128>, PARTIAL>(a, ld, causal, ncol, stream);
  return launch_causal<Cfg<256>, PARTIAL>(a, ld, causal, ncol, stream);
}

}  // namespace

int bf16_rows_per_block(int d, int64_t BH, int N) {
  if (d == 128 || (d == 64 && bf16_tuned_d64(BH, N))) return bf16_tuned_rows_per_block();
  if (d <= 64) return d64_wide(BH, N) ? CfgD64Wide::NW * CfgD64Wide::QW * 32 : Cfg<64>::NW * Cfg<64>::QW * 32;
  if (d <= 128) return Cfg<128>::NW * Cfg<128>::QW * 32;
  return Cfg<256>::NW * Cfg<256>::QW * 32;
}

hipError_t launch_bf16(const FwdArgs& a, int d_pad, bool causal, hipStream_t stream) {
  if (a.d == 128 || (a.d == 64 && bf16_tuned_d64(a.BH, a.N))) return launch_bf16_tuned(a, causal, stream);
  return launch_generic<false>(a, d_pad, causal, 1, stream);
}

int bf16_split_rows_per_block(int d_pad) {
  return d_pad <= 64 ? Cfg<64>::NW * Cfg<64>::QW * 32
                     : (d_pad <= 128 ? Cfg<128>::NW * Cfg<128>::QW * 32 : Cfg<256>::NW * Cfg<256>::QW * 32);
}

int bf16_split_key_tile(int d_pad) {
  return d_pad <= 64 ? Cfg<64>::BC : (d_pad <= 128 ? Cfg<128>::BC : Cfg<256>::BC);
}

hipError_t launch_bf16_partial(const FwdArgs& a, int d_pad, bool causal, int nsplit, hipStream_t stream) {
  return launch_generic<true>(a, d_pad, causal, nsplit, stream);
}

}  // namespace fa
