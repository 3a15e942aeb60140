// Fused forward pass of exact softmax attention, bf16, head width exactly 128 or exactly 64:
// the tuned gfx950 kernels for long sequences (one body, instantiated for each width).
//
// Same arithmetic as the generic bf16 kernel (online softmax over key tiles: running max,
// denominator and unnormalised numerator rescaled together when the max rises; liminalml.com
// "FlashAttention", online update equations), with a schedule built for CDNA4:
//
// * 8 waves per workgroup, 32 query rows each (256 rows per workgroup), two waves per SIMD.
//   The waves form two groups (waves 0-3 and 4-7, one wave of each group per SIMD) that run
//   one phase apart. Every key tile j is handled in two phases per wave:
//     M_j: O^T += V_{j-1}^T P_{j-1}^T, then S_j^T = K_j Q^T (D/8 MFMAs each: 16 at D = 128,
//          8 at D = 64)
//     V_j: online-softmax update of S_j into P_j (exponentials and the other VALU work)
//   separated by workgroup barriers. While one group is in an M phase the other is in a V
//   phase, so each SIMD keeps its matrix unit busy with one wave while the other wave's
//   vector work runs alongside.
// * K and V tiles (64 keys x D features) go from HBM straight into LDS with
//   global_load_lds_dwordx4 (no staging registers, no LDS write instructions) into rings of
//   4 slots, requested at the start of V phases (two tiles ahead for the leading group, three
//   for the other), where the vector work leaves issue slack. Each wave's load instruction fills
//   1 KiB of LDS (lane l -> byte 16*l), so rows are stored unpadded and the 16-byte chunks of
//   each row are XOR-swizzled so that the 16-byte K operand reads of 16 consecutive rows, and
//   the V transpose reads of 4 consecutive rows and two 16-feature halves, hit distinct banks
//   (the permutations are in fa_dma.h).
// * Operand reads from LDS run a few MFMAs ahead. The first V^T operands of M_j are requested
//   at the end of the wave's V_{j-1} phase (V_{j-1} has been in LDS since M_{j-1}) and the first
//   K operands of S_j during the last steps of the V product, so that neither product of an M
//   phase starts by waiting for LDS; LDS reads may stay in flight across the phase barriers.
// * Operand layouts are those of the generic kernel: S^T and O^T accumulators hold one query
//   per lane, probabilities go from the S^T accumulator into the B operand of the second
//   product without data movement, and V^T operands come from ds_read_b64_tr_b16.
// * The softmax of a tile takes no row maximum in the common case: the exponentials use the
//   running reference directly, and only when the tile's sum shows a score far above it (more
//   than 2^59 in probability terms, or the first tile) is the tile maximum taken and the
//   reference raised, with the usual rescale of denominator and numerator. Probabilities then
//   stay below 2^64, far inside the fp32 and bf16 ranges; the reference is any value at or
//   below the true running maximum, which leaves u / l and the log-normaliser unchanged up to
//   rounding.
// * A tile is masked only where it must be (the causal diagonal, the ragged last tile): the
//   mask overwrites scores with -inf, the rest of the update is shared. Key rows past N are
//   loaded from row N-1 (finite data, weight 0).
// * The output rows leave through LDS (the K ring is idle after the last barrier of an item),
//   so that every store writes whole rows.
// * When there are more work items (query tile, head) than workgroups that fit on the chip at
//   once, that many stay resident and each runs a fixed sequence of items: no dispatch gap
//   between items, and under the causal mask a balanced total per workgroup (see the schedule
//   below).

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <atomic>

#include "fa_internal.h"
#include "fa_dma.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BC = 64;          // keys per tile
constexpr int NW = 8;           // waves per workgroup
constexpr int NT = NW * 64;
constexpr int BR = NW * 32;     // query rows per workgroup
constexpr int SLOTS = 4;
// Per head width D: bytes per key row in LDS, per K or V tile (16 KiB at D = 128, 8 KiB at 64),
// the V ring's start after the K ring, the rings' LDS (128 or 64 KiB), and the DMA instructions
// each thread issues per tile (K + V: 4 or 2).
template <int D> struct Tiles {
  static constexpr int ROWB = D * 2;
  static constexpr int TILEB = BC * ROWB;
  static constexpr int VREGION = SLOTS * TILEB;
  static constexpr int LDS_BYTES = 2 * SLOTS * TILEB;
  static constexpr int LOADS_PER_TILE = 2 * (TILEB / 16) / NT;
};
// A tile whose per-lane probability sum exceeds 2^64 raises the reference (see v_phase).
constexpr float kRaiseSum = 18446744073709551616.0f;   // 2^64
// Reference before the first tile: finite (so that masked scores give exp2(-inf) = 0, never
// a NaN), and so low that the first tile always raises it.
constexpr float kRefInit = -1.0e30f;

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// A VALU instruction that reads the result of a transcendental one (v_exp_f32) needs a wait
// state between them. The compiler provides it for the instructions it emits, but it does not
// treat inline asm as a reader, so a value that inline asm will read right after a v_exp_f32
// passes through an s_nop first (two wait states; the raise path only).
__device__ __forceinline__ float asm_ready(float x) {
  asm volatile("s_nop 1" : "+v"(x));
  return x;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

template <int V> struct IntC { static constexpr int value = V; };

// One 16-byte-per-lane global -> LDS load: lane l's data lands at LDS byte lds_addr + 16*l.
// Issued through inline assembly so that the compiler's wait insertion does not treat every
// later LDS read as dependent on it; completion is tracked by hand (phase_barrier). An LDS DMA
// needs a wait state after the scalar write of M0 that gives its LDS address (the s_nop).
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory");
}

// Wait until at most `n` vector-memory operations of this wave are outstanding and, with
// LGKM = 0, all of its LDS reads have returned (LGKM = 15: LDS reads may stay in flight).
template <int n, int LGKM = 0>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  static_assert(LGKM == 0 || LGKM == 15, "lgkmcnt: all or none");
  // s_waitcnt encoding (gfx9): vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  constexpr int imm = (n & 15) | (7 << 4) | (LGKM << 8) | ((n >> 4) << 14);
  __builtin_amdgcn_s_waitcnt(imm);
}

// Barrier between phases. `ahead` = how many tiles this wave has requested beyond the last
// tile that some wave reads in the coming phase: the DMA loads of those tiles may stay in
// flight, everything older must have landed in LDS. LDS reads may stay in flight across it:
// every read either feeds an MFMA of the phase it was issued in, or requests operands of the
// wave's next M phase from a slot that no load overwrites before that phase has ended. The
// compiler does not see the LDS writes of the DMA loads, so the barrier is also a compiler
// memory barrier.
template <int LOADS_PER_TILE>
__device__ __forceinline__ void phase_barrier(int ahead) {
  if (ahead >= 2) wait_vm<2 * LOADS_PER_TILE, 15>();
  else if (ahead == 1) wait_vm<LOADS_PER_TILE, 15>();
  else wait_vm<0, 15>();
  asm volatile("s_barrier" ::: "memory");
}

template <int D>
__device__ __forceinline__ void fwd_tuned_body(FwdArgs a, int causal_flag) {
  static_assert(D == 64 || D == 128, "head width");
  constexpr int ROWB = Tiles<D>::ROWB, TILEB = Tiles<D>::TILEB, VREGION = Tiles<D>::VREGION;
  constexpr int LDS_BYTES = Tiles<D>::LDS_BYTES, LOADS_PER_TILE = Tiles<D>::LOADS_PER_TILE;
  const bool CAUSAL = causal_flag != 0;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
  const int grp = wave >> 2;   // 0: runs ahead, 1: one phase behind
  const int N = a.N;

  // (workgroups off the first XCD exit at once when the grid is packed onto one XCD; the
  // exit is uniform over the workgroup and comes before any barrier)
  if (blockIdx.x & ((1u << a.wg_shift) - 1u)) return;
  // Work item id = qt_rev * BH + bh: query tile qt of head bh (heaviest causal tiles first,
  // heads varying fastest). With at least one workgroup per item each workgroup takes one item.
  // Otherwise the grid holds the workgroups that fit at once (a multiple of 8) and workgroup w, on XCD
  // w % 8, runs the items id = w % 8 + 8k of that XCD, so that a head's K/V stay in one L2 as
  // with one workgroup per item; k runs over the XCD's workgroups in rounds of alternating
  // direction, so that under the causal mask the heaviest items of one round meet the
  // lightest of the next. A workgroup that stays resident pays no dispatch gap between items.
  const int nitems = a.BH * a.n_qtiles;
  const bool persist = (int)(gridDim.x >> a.wg_shift) < nitems;
  const int xcd = (int)(blockIdx.x & 7u), loc = (int)(blockIdx.x >> 3), nloc = (int)(gridDim.x >> 3);
  const int nx = persist ? (nitems - xcd + 7) >> 3 : 1;
  const int nrounds = persist ? (nx + nloc - 1) / nloc : 1;
  for (int round = 0; round < nrounds; ++round) {
  int id = (int)(blockIdx.x >> a.wg_shift);
  if (persist) {
    const int k = round * nloc + ((round & 1) ? nloc - 1 - loc : loc);
    if (k >= nx) continue;
    id = xcd + 8 * k;
  }
  // (per-lane addresses are formed anew for every item rather than kept live across items)
  int lane_v = lane;
  asm volatile("" : "+v"(lane_v));
  const int lane = lane_v;
  const int lr = lane & 31, hh = lane >> 5;

  const int qt_rev = id / a.BH;
  const int bh = id - qt_rev * a.BH;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - qt_rev) : qt_rev;
  const int q0 = qt * BR;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Qh = (const uint16_t*)a.q + head;
  const uint8_t* __restrict__ Kb = (const uint8_t*)((const uint16_t*)a.k + head);
  const uint8_t* __restrict__ Vb = (const uint8_t*)((const uint16_t*)a.v + head);
  uint16_t* __restrict__ Oh = (uint16_t*)a.o + head;

  const int wq_lo = q0 + wave * 32;
  const int wq_hi = wq_lo + 31;
  const int qi = wq_lo + lr;

  // ---- Q operand fragments (B operand of S^T = K Q^T) ---------------------------------------
  // (unconditional loads from a clamped row, all in flight together; rows past N become 0)
  u32x4 qf[D / 16];
  {
    const uint32_t negmask = a.neg ? 0x80008000u : 0u;
    const uint32_t keep = qi < N ? 0xffffffffu : 0u;
    const uint16_t* qrow = Qh + (size_t)min(qi, N - 1) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const u32x4 x = *(const u32x4*)(qrow + 16 * kk + 8 * hh);
      qf[kk] = (x & keep) ^ negmask;
    }
  }

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int nkv = (kv_end + BC - 1) / BC;
  const int j_last = CAUSAL ? min(nkv - 1, wq_hi / BC) : nkv - 1;   // last tile this wave uses

  // ---- LDS DMA addressing ----------------------------------------------------------------
  // Each thread issues D/64 K and D/64 V load instructions per tile. For instruction i the wave
  // fills LDS bytes [((D/64)*wave+i)*1024, +1024) of the slot; lane l writes physical chunk
  // l%(D/8) of row ((D/64)*wave+i)*(512/D) + l/(D/8) and so fetches the logical chunk the
  // swizzle places there.
  // The per-lane byte offsets inside a tile are fixed; the tile's base address advances in
  // scalar registers, so issuing a whole tile costs no vector instructions.
  static_assert(dma::fwd_row_bytes<D>() == ROWB, "row size of the load arithmetic");
  constexpr int NLD = D / 64;   // load instructions per thread for each of K and V
  uint32_t gk_off[NLD], gv_off[NLD];
  int dma_row[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    dma_row[i] = dma::fwd_row<D>(wave, lane, i);
    gk_off[i] = dma::fwd_k_off<D>(wave, lane, i);
    gv_off[i] = dma::fwd_v_off<D>(wave, lane, i);
  }
  // LDS byte address of the buffer (address-space cast, then the 32-bit LDS offset)
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)smem);
  const uint32_t dma_lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds_base + (uint32_t)(NLD * wave * 1024)));
  int last_issued = -1;
  auto issue_tile = [&](int t) __attribute__((always_inline)) {
    last_issued = t;
    const int key0 = t * BC;
    const uint32_t slot = (uint32_t)(t & (SLOTS - 1)) * TILEB;
    const uint8_t* kt = Kb + (size_t)key0 * ROWB;
    const uint8_t* vt = Vb + (size_t)key0 * ROWB;
    if (key0 + BC <= N) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const uint32_t ldst = dma_lds + slot + (uint32_t)(i * 1024);
        dma16(kt, gk_off[i], ldst);
        dma16(vt, gv_off[i], ldst + VREGION);
      }
    } else {   // ragged last tile: rows past the end read row N-1 instead (weight 0 later)
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const uint32_t back = dma::past_end_back(key0, dma_row[i], N, ROWB);
        const uint32_t ldst = dma_lds + slot + (uint32_t)(i * 1024);
        dma16(kt, gk_off[i] - back, ldst);
        dma16(vt, gv_off[i] - back, ldst + VREGION);
      }
    }
  };

  // ---- LDS read addressing -----------------------------------------------------------------
  // Per-lane byte addresses for slot 0; slot and block offsets are compile-time immediates.
  // K operand for step kk: row lr (+32 for the second 32-key block), logical chunk 2kk+hh.
  uint32_t koff[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    koff[kk] = lds_base + (uint32_t)(lr * ROWB + (((2 * kk + hh) ^ dma::fwd_k_swz<D>(lr)) * 16));
  // V transpose reads: in each 16-lane group, lane 4r+q reads key row r (+8 for the second
  // read) at features 4q..4q+3 of the 16-wide half b of 32-feature block dt.
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int b16 = (lane >> 4) & 1;
  uint32_t voff[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int chunk = (4 * dt + 2 * b16 + ((lane & 3) >> 1)) ^ dma::fwd_v_swz<D>(tr_row);
    voff[dt] = lds_base + VREGION + (uint32_t)(tr_row * ROWB + chunk * 16 + 8 * (lane & 1));
  }

  // ---- state -------------------------------------------------------------------------------
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.0f;
  float m_run = kRefInit, l_run = 0.0f;
  f32x16 s0, s1;             // S_j^T for the two 32-key blocks of the current tile
  u32x4 pb[BC / 16];          // P_{j}, bf16, B operand chunks (consumed in M_{j+1})

  // Phase intervals are numbered k = 0, 1, 2, ...: group 0 runs M_j in interval 2j and V_j in
  // 2j+1, group 1 one interval later. In interval k+1 the newest tile any wave reads is
  // (k+1)/2 (K of an M phase; V of M_j is tile j-1), so the barrier closing interval k needs
  // every tile up to (k+1)/2 in LDS.
  // Loads are issued at the start of V phases, where the vector work leaves issue slack: group
  // 0 requests tile j+2 in V_j (interval 2j+1), group 1 tile j+3 in its V_j (interval 2j+2).
  // Tile t goes to the slot of tile t-4, whose last readers (the V products of M_{t-3}) ran in
  // intervals 2t-6 and 2t-5, before either request.
  auto barrier_after = [&](int k) __attribute__((always_inline)) {
    phase_barrier<LOADS_PER_TILE>(last_issued - ((k + 1) >> 1));
  };

  // prologue: every wave requests its share of tiles 0 and 1; tile 0 lands before interval 0
  issue_tile(0);
  if (nkv > 1) issue_tile(1);
  if (grp == 1 && nkv > 2) issue_tile(2);
  phase_barrier<LOADS_PER_TILE>(last_issued);

  // Operand reads run PF (K) and PFV (V) steps ahead of the MFMAs; scheduling barriers keep the
  // compiler from sinking them next to their uses. The reads of one product's first steps are
  // issued before it starts, in the preceding phase or product, so that no product waits for
  // LDS at its start. Shallow depths measured best (2 and 1: fewer reads in the softmax phase,
  // which is as critical as the matrix phase; deeper ones were up to 3% slower).
#ifndef FA_PF
#define FA_PF 2
#endif
#ifndef FA_PFV
#define FA_PFV 1
#endif
  constexpr int PF = FA_PF;     // K operand steps in flight
  constexpr int PFV = FA_PFV;   // V operand steps in flight (requested in the V phase before)
  constexpr int S_STEPS = D / 16;                  // S^T = K Q^T: steps of two MFMAs
  constexpr int PV_STEPS = (BC / 16) * (D / 32);   // O^T += V^T P^T: one MFMA per step
  static_assert(PF >= 1 && PF <= S_STEPS && PFV >= 1 && PFV <= PV_STEPS, "prefetch depth within a product");
  u32x4 kb0[S_STEPS], kb1[S_STEPS];   // K operands of the two 32-key blocks
  u32x4 av[PV_STEPS];                 // V^T operands
  auto k_load = [&](int kk, auto ks_tag) __attribute__((always_inline)) {
    constexpr uint32_t kslot = decltype(ks_tag)::value * TILEB;
    kb0[kk] = *(const lds_u32x4*)(uintptr_t)(koff[kk] + kslot);
    kb1[kk] = *(const lds_u32x4*)(uintptr_t)(koff[kk] + (kslot + 32 * ROWB));
  };
  auto v_load = [&](int st, auto vs_tag) __attribute__((always_inline)) {
    constexpr uint32_t vslot = decltype(vs_tag)::value * TILEB;
    const int c16 = st / (D / 32), dt = st % (D / 32);
    const uint32_t off = vslot + (uint32_t)(c16 * 16 * ROWB);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(voff[dt] + off));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(voff[dt] + (off + 8 * ROWB)));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
    av[st] = (u32x4){lo2[0], lo2[1], hi2[0], hi2[1]};
  };
  auto k_prefetch = [&](auto ks_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) k_load(kk, ks_tag);
  };
  auto v_prefetch = [&](auto vs_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < PFV; ++st) v_load(st, vs_tag);
    __builtin_amdgcn_sched_barrier(0);
  };

  // S_j^T = K_j Q^T from LDS slot KS (first PF steps already requested).
  auto s_product = [&](auto ks_tag) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    f32x16 c0 = {}, c1 = {};
#pragma unroll
    for (int kk = 0; kk < S_STEPS; ++kk) {
      if (kk + PF < S_STEPS) k_load(kk + PF, ks_tag);
      __builtin_amdgcn_sched_barrier(0);
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kb0[kk]),
                                                   __builtin_bit_cast(bf16x8, qf[kk]), c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kb1[kk]),
                                                   __builtin_bit_cast(bf16x8, qf[kk]), c1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    s0 = c0;
    s1 = c1;
  };

  // O^T += V^T P^T from LDS slot VS (first PF steps already requested); unless it is the last
  // product (KPF = 0), its last steps request the first K operands of the S product that
  // follows, from slot KS.
  auto pv_product = [&](auto vs_tag, auto ks_tag, auto kpf_tag) __attribute__((always_inline)) {
    constexpr bool KPF = decltype(kpf_tag)::value != 0;
#pragma unroll
    for (int st = 0; st < PV_STEPS; ++st) {
      if (st + PFV < PV_STEPS) v_load(st + PFV, vs_tag);
      if (KPF && st + PF >= PV_STEPS) k_load(st + PF - PV_STEPS, ks_tag);
      __builtin_amdgcn_sched_barrier(0);
      const int c16 = st / (D / 32), dt = st % (D / 32);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[st]),
                                                        __builtin_bit_cast(bf16x8, pb[c16]), acc[dt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // M phase of tile j held in LDS slot SLOT (j may equal nkv: then only the product with
  // V_{j-1} remains): first O^T += V_{j-1}^T P_{j-1}^T (its V operands were requested at the
  // end of the wave's previous V phase; V_{j-1} has been in LDS since before M_{j-1}), then
  // S_j. Tile 0 (FIRST) has only S_0; the final M phase (LAST, j = nkv) only the product with
  // V_{nkv-1}, and it reads nothing from the K ring. The wave raises its issue priority so that
  // the other wave's vector work on the same SIMD does not hold back its MFMA stream.
  auto m_phase = [&](int j, auto slot_tag, auto first_tag, auto last_tag) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_tag)::value;
    constexpr bool FIRST = decltype(first_tag)::value != 0;
    constexpr bool LAST = decltype(last_tag)::value != 0;
    __builtin_amdgcn_s_setprio(2);
    if constexpr (FIRST) {
      k_prefetch(IntC<SL>{});
      s_product(IntC<SL>{});
    } else if constexpr (LAST) {
      if (j - 1 <= j_last) pv_product(IntC<(SL + SLOTS - 1) % SLOTS>{}, IntC<SL>{}, IntC<0>{});
    } else if (j - 1 <= j_last) {   // otherwise j > j_last as well: nothing left for this wave
      pv_product(IntC<(SL + SLOTS - 1) % SLOTS>{}, IntC<SL>{}, IntC<1>{});
      if (j < nkv && j <= j_last) s_product(IntC<SL>{});
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // V phase of tile j: online-softmax update of S_j into P_j. The exponentials use the current
  // reference m_run directly; no per-tile maximum is taken unless the tile's sum shows that
  // the reference must be raised (some score more than ~2^59 above it, or the first tile,
  // whose reference is a huge negative number): then the tile maximum is found, the
  // denominator and numerator are rescaled and the exponentials are recomputed. Otherwise
  // every probability is at most 2^64, so the fp32 sums and bf16 probabilities stay finite.
  auto v_phase = [&](int j, auto slot_tag) __attribute__((always_inline)) {
    if (j > j_last) return;
    const int key0 = j * BC;
    const bool masked = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > wq_lo);
    if (masked) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (key >= N || (CAUSAL && key > qi)) s0[i] = -INFINITY;
        if (key + 32 >= N || (CAUSAL && key + 32 > qi)) s1[i] = -INFINITY;
      }
    }
    float p[32], ls;
    auto exps = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], a.sl2, -m_run));
        p[16 + i] = __builtin_amdgcn_exp2f(fmaf(s1[i], a.sl2, -m_run));
      }
      float t[4] = {p[0] + p[16], p[1] + p[17], p[2] + p[18], p[3] + p[19]};
#pragma unroll
      for (int i = 4; i < 16; ++i) t[i & 3] += p[i] + p[16 + i];
      ls = (t[0] + t[1]) + (t[2] + t[3]);
    };
    exps();
    if (__builtin_amdgcn_ballot_w64(ls > kRaiseSum)) {
      float m0 = fmaxf(s0[0], s0[1]), m1 = fmaxf(s1[0], s1[1]);
#pragma unroll
      for (int i = 2; i < 16; i += 2) {
        m0 = fmaxf(m0, fmaxf(s0[i], s0[i + 1]));
        m1 = fmaxf(m1, fmaxf(s1[i], s1[i + 1]));
      }
      const float m_new = fmaxf(m_run, pair_max(fmaxf(m0, m1) * a.sl2));
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      // In-place multiplies (inline asm, so that the compiler keeps one copy of the accumulator
      // across the branch) of a value that v_exp_f32 has just written: see asm_ready.
      const float alpha_r = asm_ready(alpha);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) asm("v_mul_f32 %0, %0, %1" : "+v"(acc[dt][i]) : "v"(alpha_r));
      m_run = m_new;
      exps();
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 w = {pack_bf16x2(p[8 * c + 0], p[8 * c + 1]), pack_bf16x2(p[8 * c + 2], p[8 * c + 3]),
                       pack_bf16x2(p[8 * c + 4], p[8 * c + 5]), pack_bf16x2(p[8 * c + 6], p[8 * c + 7])};
      pb[c] = w;
    }
    l_run += ls;
    v_prefetch(slot_tag);   // V_j operands of the next M phase (tile j has been in LDS since M_j)
  };

  // Phases: M_0 V_0 M_1 V_1 ... M_{n-1} V_{n-1} M_n, one barrier after each. Group 1 starts
  // with one extra barrier and skips the barrier after its last phase, so it always works one
  // phase behind group 0 while both pass the same number of barriers. The loop is unrolled by
  // the ring size so that every LDS slot offset is an immediate.
  const int lag = grp;   // interval of this wave's M_0
  if (grp == 1) barrier_after(0);
  auto tile = [&](int j, auto slot_tag, auto first_tag) __attribute__((always_inline)) {
    m_phase(j, slot_tag, first_tag, IntC<0>{});
    barrier_after(2 * j + lag);
    if (j + 2 + grp < nkv) issue_tile(j + 2 + grp);
    v_phase(j, slot_tag);
    barrier_after(2 * j + 1 + lag);
  };
  // Tile 0 (slot 0) is peeled off; the loop then runs tiles 1, 2, 3, 0 (mod 4) per iteration.
  tile(0, IntC<0>{}, IntC<1>{});
  int j = 1;
  for (; j + SLOTS <= nkv; j += SLOTS) {
    tile(j, IntC<1>{}, IntC<0>{});
    tile(j + 1, IntC<2>{}, IntC<0>{});
    tile(j + 2, IntC<3>{}, IntC<0>{});
    tile(j + 3, IntC<0>{}, IntC<0>{});
  }
  if (j < nkv) tile(j++, IntC<1>{}, IntC<0>{});
  if (j < nkv) tile(j++, IntC<2>{}, IntC<0>{});
  if (j < nkv) tile(j++, IntC<3>{}, IntC<0>{});
  switch (nkv & (SLOTS - 1)) {   // the final M phase (product with V_{nkv-1} only)
    case 0: m_phase(nkv, IntC<0>{}, IntC<0>{}, IntC<1>{}); break;
    case 1: m_phase(nkv, IntC<1>{}, IntC<0>{}, IntC<1>{}); break;
    case 2: m_phase(nkv, IntC<2>{}, IntC<0>{}, IntC<1>{}); break;
    default: m_phase(nkv, IntC<3>{}, IntC<0>{}, IntC<1>{}); break;
  }
  if (grp == 0) barrier_after(2 * nkv);
  wait_vm<0>();

  // ---- epilogue: o = u / l, lse = (m + log2 l) * ln 2 -----------------------------------------
  // A lane holds 4-feature pieces of one output row, so stores straight from the accumulators
  // would touch 32 rows per instruction. The rows go out through LDS instead: after the last
  // barrier nothing reads the K ring any more (the last S product ran before it, the final M
  // phase reads only the V ring and no load is in flight), so each wave stages its 32 rows
  // (64 D bytes, bf16) in its own eighth of the K ring, 16-byte chunk c of row r at
  // c ^ (r mod D/8), and reads them back as whole rows: each store writes 1 KiB contiguous
  // (512/D rows).
  const float l_tot = pair_sum(l_run);
  const float inv = 1.0f / l_tot;
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int RPS = 1024 / ROWB;    // rows per 1 KiB store
  const uint32_t stage = lds_base + (uint32_t)(wave * 32 * ROWB);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {   // features dt*32 + 8g + 4hh .. +3 = half hh of chunk 4dt + g
      const u32x2 w = {pack_bf16x2(acc[dt][4 * g + 0] * inv, acc[dt][4 * g + 1] * inv),
                       pack_bf16x2(acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv)};
      const uint32_t chunk = (uint32_t)((4 * dt + g) ^ (lr & (CPR - 1)));
      *(lds_u32x2*)(uintptr_t)(stage + (uint32_t)(lr * ROWB) + chunk * 16 + 8 * hh) = w;
    }
#pragma unroll
  for (int s = 0; s < 32 / RPS; ++s) {   // lane l: row RPS s + l/CPR, chunk l%CPR
    const int r = RPS * s + lane / CPR, c = lane % CPR;
    const u32x4 x = *(const lds_u32x4*)(uintptr_t)(stage + (uint32_t)(r * ROWB) + (uint32_t)((c ^ (r & (CPR - 1))) * 16));
    if (wq_lo + r < N) *(u32x4*)(Oh + (size_t)(wq_lo + r) * D + 8 * c) = x;
  }
  if (a.lse != nullptr && hh == 0 && qi < N) a.lse[(size_t)bh * N + qi] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
  // every wave has read its staged rows before the next item's loads refill the K ring
  __syncthreads();
  }
}

__global__ __launch_bounds__(NT, 2)
void fwd_bf16_d128_kernel(FwdArgs a, int causal_flag) { fwd_tuned_body<128>(a, causal_flag); }

__global__ __launch_bounds__(NT, 2)
void fwd_bf16_d64_kernel(FwdArgs a, int causal_flag) { fwd_tuned_body<64>(a, causal_flag); }

// Workgroups of a kernel that stay resident at once on the current device (CUs times the
// kernel's workgroups per CU), rounded down to a multiple of 8 (XCDs); cached per device.
template <int D>
int resident_workgroups() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, D == 128 ? fwd_bf16_d128_kernel : fwd_bf16_d64_kernel,
                                                     NT, 0) != hipSuccess || per_cu < 1)
      return 0;
    n = (cus * per_cu) & ~7;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D>
hipError_t launch_tuned(const FwdArgs& a, bool causal, hipStream_t stream) {
  const int64_t nitems = (int64_t)a.BH * a.n_qtiles;
  const int resident = resident_workgroups<D>();
  unsigned grid = (unsigned)(nitems << a.wg_shift);
  if (a.wg_shift == 0 && resident >= 8 && nitems > resident) grid = (unsigned)resident;   // persistent
  hipLaunchKernelGGL(D == 128 ? fwd_bf16_d128_kernel : fwd_bf16_d64_kernel, dim3(grid), dim3(NT), 0, stream, a,
                     causal ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

int bf16_tuned_rows_per_block() { return BR; }

// Head width 64 runs the tuned kernel when the grid has at least one tile of 256 queries per CU;
// smaller grids keep the generic blocks (more, smaller workgroups). FA_TUNED_D64=0 (a timing
// build) sends every width-64 call to the generic blocks.
#ifndef FA_TUNED_D64
#define FA_TUNED_D64 1
#endif
bool bf16_tuned_d64(int64_t BH, int N) { return FA_TUNED_D64 && BH * (((int64_t)N + BR - 1) / BR) >= 256; }

hipError_t launch_bf16_tuned(const FwdArgs& a, bool causal, hipStream_t stream) {
  return a.d == 128 ? launch_tuned<128>(a, causal, stream) : launch_tuned<64>(a, causal, stream);
}

}  // namespace fa
