// Fused forward pass of exact softmax attention, fp32 inputs, for gfx950 (CDNA4).
//
// Same method and data flow as the bf16 kernel (online softmax over key tiles with the
// running max, denominator and numerator rescaled together; liminalml.com
// "FlashAttention", online update equations), with fp32 operands throughout: both
// products use v_mfma_f32_32x32x2_f32 and the probabilities stay fp32.
//
// Layout (transposed products, as in the bf16 kernel):
//   S^T = K Q^T : A operand lane l = K[key l%32][feature slot], B operand = Q[query l%32][slot]
//   O^T += V^T P^T : the 16 accumulator registers of S^T hold keys 8*(i/4)+4*(l/32)+i%4 of
//   one query; register i is the B operand of one MFMA whose two contraction slots are the
//   keys of the two lane halves, and the A operand is V[that key][feature l%32], read from
//   a row-major V tile (consecutive lanes read consecutive features).
// The contraction over features is permuted: in MFMA step kk, lane half h supplies feature
// kk + h*D/2, so every lane reads one contiguous run of a K row and of its Q row.
// Unlike the bf16 kernel, the running maximum is kept on unscaled scores and the scale is
// applied after the subtraction, which the 1e-5 fp32 tolerance needs at large scores.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kRescaleThreshold = 8.0f;

// NW waves per key group, BC keys per tile; a workgroup runs up to MAXSPLIT key groups over
// the same queries (taking tiles g, g + SPLIT, ...) and merges them at the end.
template <int D> struct CfgF;
template <> struct CfgF<64>  { static constexpr int NW = 1, BC = 32, MAXSPLIT = 4; };
template <> struct CfgF<128> { static constexpr int NW = 2, BC = 32, MAXSPLIT = 2; };
template <> struct CfgF<256> { static constexpr int NW = 4, BC = 32, MAXSPLIT = 1; };

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 4 consecutive floats of one row, zero outside [0, d). The row starts at element row0 of
// base; elements are addressed by 32-bit indices off the uniform base (no 64-bit address per
// element stays live). The loads are unconditional (column clamped) so that they issue
// together.
__device__ __forceinline__ f32x4 load4_masked(const float* base, uint32_t row0, int col, int d) {
  f32x4 r;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float x = base[row0 + (uint32_t)min(col + t, d - 1)];
    r[t] = (col + t < d) ? x : 0.0f;
  }
  return r;
}

// PARTIAL: the workgroup covers only the keys of its split column (blockIdx.y) and writes its
// partial state (m, l, u) to the workspace instead of o and lse; a merge pass combines them.
template <int D, bool CAUSAL, bool FULLD, int SPLIT, bool PARTIAL>
__global__ __launch_bounds__(CfgF<D>::NW * SPLIT * 64, 1)
void fwd_f32_kernel(FwdArgs a) {
  constexpr int NW = CfgF<D>::NW, BC = CfgF<D>::BC;
  constexpr int NT = NW * SPLIT * 64;
  constexpr int BR = NW * 32;
  constexpr int KP = D + 1;   // odd pitch: the 32 rows of one read fall in distinct banks
  constexpr int VP = D + 4;
  constexpr int KT = BC * KP, VT = BC * VP;
  constexpr int CH = BC * D / 4;   // 16-byte chunks per tile
  constexpr int CPT = SPLIT * CH / NT;   // SPLIT tiles per step
  constexpr int H2 = D / 2;
  static_assert((SPLIT * CH) % NT == 0, "tiles must split evenly over the workgroup");
  constexpr int NV = D / 32 * 16 + 2;   // merge values per lane: m, l, numerator
  static_assert(SPLIT == 1 || NW * (SPLIT - 1) * NV * 64 <= 2 * SPLIT * (KT + VT),
                "merge area must fit in the tile buffers");

  __shared__ __attribute__((aligned(16))) float smem[2 * SPLIT * (KT + VT)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = tid >> 6;
  const int grpk = wave_all / NW;          // key group
  const int wave = wave_all - grpk * NW;   // query wave
  const int lr = lane & 31, hh = lane >> 5;
  const int N = a.N, d = a.d;

  // (workgroups off the first XCD exit at once when the grid is packed onto one XCD; the
  // exit is uniform over the workgroup and comes before any barrier)
  if (blockIdx.x & ((1u << a.wg_shift) - 1u)) return;
  const int id = (int)(blockIdx.x >> a.wg_shift);
  const int qt_rev = id / a.BH;
  const int bh = id - qt_rev * a.BH;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - qt_rev) : qt_rev;
  const int q0 = qt * BR;

  const size_t head = (size_t)bh * (size_t)N * (size_t)d;
  const float* __restrict__ Qh = (const float*)a.q + head;
  const float* __restrict__ Kh = (const float*)a.k + head;
  const float* __restrict__ Vh = (const float*)a.v + head;
  float* __restrict__ Oh = (float*)a.o + head;

  const int wq_lo = q0 + wave * 32;
  const int wq_hi = wq_lo + 31;
  const int qi = wq_lo + lr;

  // Q operand: step kk uses feature kk + hh*D/2. Every load is unconditional (row and column
  // clamped into range) so that they are all in flight together; out-of-range values are
  // replaced by 0 afterwards.
  float qf[H2];
  {
    const float sgn = a.neg ? -1.0f : 1.0f;
    const bool qv = qi < N;
    const uint32_t qrow0 = (uint32_t)min(qi, N - 1) * (uint32_t)d;
    const float* qrow = Qh + qrow0;
    if (FULLD) {
#pragma unroll
      for (int v = 0; v < H2 / 4; ++v) {
        const f32x4 x = *(const f32x4*)(qrow + hh * H2 + 4 * v);
#pragma unroll
        for (int t = 0; t < 4; ++t) qf[4 * v + t] = qv ? sgn * x[t] : 0.0f;
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < H2; ++kk) {
        const int col = kk + hh * H2;
        const float x = Qh[qrow0 + (uint32_t)min(col, d - 1)];
        qf[kk] = (qv && col < d) ? sgn * x : 0.0f;
      }
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

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  f32x4 kreg[CPT], vreg[CPT];
  // step `it` stages tiles it*SPLIT .. it*SPLIT + SPLIT-1 (one per key group)
  auto gload = [&](int it) {
    const int key0 = (t_beg + it * SPLIT) * BC;
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int c = tid + r * NT;
      const int row = c / (D / 4);      // row within the SPLIT*BC staged keys
      const int col = (c % (D / 4)) * 4;
      const int key = key0 + row;
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (key < N) {
        // one 32-bit element offset serves K and V (N * d < 2^31)
        const uint32_t row0 = (uint32_t)key * (uint32_t)d;
        if (FULLD) {
          kx = *(const f32x4*)(Kh + row0 + col);
          vx = *(const f32x4*)(Vh + row0 + col);
        } else {
          kx = load4_masked(Kh, row0, col, d);
          vx = load4_masked(Vh, row0, col, d);
        }
      }
      kreg[r] = kx;
      vreg[r] = vx;
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int c = tid + r * NT;
      const int row = c / (D / 4);
      const int col = (c % (D / 4)) * 4;
      float* Ks = smem + (buf * SPLIT + row / BC) * (KT + VT);
      float* Vs = Ks + KT;
      const int tr = row % BC;
#pragma unroll
      for (int t = 0; t < 4; ++t) Ks[tr * KP + col + t] = kreg[r][t];   // odd pitch: scalar stores
      *(f32x4*)(Vs + tr * VP + col) = vreg[r];
    }
  };

  const int nit = (nkv + SPLIT - 1) / SPLIT;   // steps of SPLIT tiles
  gload(0);
  swrite(0);
  __syncthreads();

  for (int it = 0; it < nit; ++it) {
    const int buf = it & 1;
    // The next step's tile is fetched into registers during this step's products, except at
    // head widths above 128: there the 128 Q and 128 accumulator registers per lane leave no
    // room for the staging registers beside the products, so the fetch follows them.
    constexpr bool kOverlapFetch = D <= 128;
    if (kOverlapFetch && it + 1 < nit) gload(it + 1);
    const float* Ks = smem + (buf * SPLIT + grpk) * (KT + VT);
    const float* Vs = Ks + KT;
    const int j = it * SPLIT + grpk;   // this key group's tile (relative to t_beg)
    const int key0 = (t_beg + j) * BC;

    if (j < nkv && (!CAUSAL || key0 <= wq_hi)) {
      f32x16 s[BC / 32];
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
        const float* krow = Ks + (kb * 32 + lr) * KP + hh * H2;
        // all operand reads first, then the MFMA chain (one LDS latency per block, not one
        // per MFMA)
        // (head widths above 64 read them as the chain goes, to bound the registers)
        constexpr int KOPS = D <= 64 ? H2 : 1;
        float kop[KOPS];
        if constexpr (D <= 64) {
#pragma unroll
          for (int kk = 0; kk < H2; ++kk) kop[kk] = krow[kk];
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kk = 0; kk < H2; ++kk)
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(D <= 64 ? kop[kk % KOPS] : krow[kk], qf[kk], s[kb], 0, 0, 0);
      }

      // Statistics are kept on the unscaled scores: p = 2^((s - m) * sl2). Subtracting
      // before scaling keeps the exponent argument accurate to fp32 rounding of s - m even
      // when the scores themselves are large (e.g. all near 1000).
      const bool masked = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > wq_lo);
      float mt = -INFINITY;
      if (masked) {
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            const bool dead = key >= N || (CAUSAL && key > qi);
            if (dead) s[kb][i] = -INFINITY;
            mt = fmaxf(mt, s[kb][i]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kb][i]);
      }
      mt = pair_max(mt);
      const float m_new = fmaxf(m_run, mt);
      if (__builtin_amdgcn_ballot_w64((m_new - m_run) * a.sl2 > kRescaleThreshold)) {
        const float alpha = exp2f((m_run - m_new) * a.sl2);  // 0 while m_run is -inf
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
        m_run = m_new;
      }
      const float msub = (m_run == -INFINITY) ? 0.0f : m_run;
      float lsum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = __builtin_amdgcn_exp2f((s[kb][i] - msub) * a.sl2);
          if (masked && s[kb][i] == -INFINITY) p = 0.0f;   // also right when scale is 0
          s[kb][i] = p;
          lsum += p;
        }
      l_run += lsum;

#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        // operand reads of the whole block first, then the MFMAs
        constexpr int VI = D <= 64 ? 16 : 1;
        float vop[VI][D / 32];
        if constexpr (D <= 64) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            const float* vrow = Vs + key * VP + lr;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) vop[i][dt] = vrow[dt * 32];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          const float* vrow = Vs + key * VP + lr;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(D <= 64 ? vop[i % VI][dt] : vrow[dt * 32], s[kb][i], acc[dt],
                                                           0, 0, 0);
        }
      }
    }

    if (!kOverlapFetch && it + 1 < nit) gload(it + 1);
    if (it + 1 < nit) swrite(buf ^ 1);
    __syncthreads();
  }

  // ---- merge of the key groups: m* = max m_g, l = sum l_g w_g, u = sum u_g w_g with
  // w_g = 2^((m_g - m*) * scale * log2 e) (interactiveml.org, merge of the three sufficient
  // statistics); groups 1.. pass their state to group 0 through LDS.
  if constexpr (SPLIT > 1) {
    float* mb = smem;
    if (grpk > 0) {
      float* dst = mb + (size_t)((wave * (SPLIT - 1) + grpk - 1) * NV) * 64 + lane;
      dst[0] = m_run;
      dst[64] = l_run;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[(2 + dt * 16 + i) * 64] = acc[dt][i];
    }
    __syncthreads();
    if (grpk > 0) return;
#pragma unroll
    for (int g = 1; g < SPLIT; ++g) {
      const float* src = mb + (size_t)((wave * (SPLIT - 1) + g - 1) * NV) * 64 + lane;
      const float mg = src[0], lg = src[64];
      const float ms = fmaxf(m_run, mg);
      // a group that saw no key has m = -inf and weight 0
      const float w0 = (m_run == -INFINITY) ? 0.0f : exp2f((m_run - ms) * a.sl2);
      const float wg = (mg == -INFINITY) ? 0.0f : exp2f((mg - ms) * a.sl2);
      l_run = l_run * w0 + lg * wg;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] = acc[dt][i] * w0 + src[(2 + dt * 16 + i) * 64] * wg;
      m_run = ms;
    }
  }

  const float l_tot = pair_sum(l_run);

  // ---- partial epilogue: the state (m, l, u) of this key range, unnormalised ---------------
  // m is the running maximum of the unscaled scores (-inf for a row that saw no key of this
  // range; then l = 0 and u = 0).
  if constexpr (PARTIAL) {
    if (qi < N) {
      const size_t row = ((size_t)blockIdx.y * a.BH + bh) * N + qi;
      float* urow = a.part_u + row * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 w = {acc[dt][4 * g + 0], acc[dt][4 * g + 1], acc[dt][4 * g + 2], acc[dt][4 * g + 3]};
          *(float4*)(urow + dt * 32 + 8 * g + 4 * hh) = w;
        }
      if (hh == 0) *(float2*)(a.part_ml + 2 * row) = make_float2(m_run, l_tot);
    }
    return;
  }

  const float inv = 1.0f / l_tot;
  if (qi < N) {
    float* orow = Oh + (size_t)qi * d;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = dt * 32 + 8 * g + 4 * hh;
        f32x4 w;
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = acc[dt][4 * g + t] * inv;
        if (FULLD) {
          *(f32x4*)(orow + col) = w;
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (col + t < d) orow[col + t] = w[t];
        }
      }
    if (a.lse != nullptr && hh == 0) {
      const float msub = (m_run == -INFINITY) ? 0.0f : m_run;
      a.lse[(size_t)bh * N + qi] = (msub * a.sl2 + log2f(l_tot)) * 0.69314718055994531f;
    }
  }
}

template <int D, bool CAUSAL, int SPLIT, bool PARTIAL>
hipError_t launch_split(const FwdArgs& a, bool fulld, int ncol, hipStream_t stream) {
  const dim3 grid((unsigned)(a.BH * a.n_qtiles) << a.wg_shift, (unsigned)ncol);
  const dim3 block(CfgF<D>::NW * SPLIT * 64);
  if (fulld) hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, true, SPLIT, PARTIAL>), grid, block, 0, stream, a);
  else       hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, false, SPLIT, PARTIAL>), grid, block, 0, stream, a);
  return hipGetLastError();
}

// Key groups per workgroup: split the key range while the grid stays small (at most 512
// workgroups) and every group still gets at least two tiles. `keys` is the length of one
// workgroup's key range, `ncol` the number of split columns.
template <int D, bool CAUSAL, bool PARTIAL>
hipError_t launch_one(const FwdArgs& a, bool fulld, int ncol, hipStream_t stream) {
  const long long wgs = (long long)a.BH * a.n_qtiles * ncol;
  const int nkv = ((PARTIAL ? a.kv_chunk : a.N) + CfgF<D>::BC - 1) / CfgF<D>::BC;
  int split = 1;
  while (split * 2 <= CfgF<D>::MAXSPLIT && wgs * split * 2 <= 512 && nkv >= 2 * split * 2) split *= 2;
  if constexpr (CfgF<D>::MAXSPLIT >= 4) {
    if (split == 4) return launch_split<D, CAUSAL, 4, PARTIAL>(a, fulld, ncol, stream);
  }
  if constexpr (CfgF<D>::MAXSPLIT >= 2) {
    if (split == 2) return launch_split<D, CAUSAL, 2, PARTIAL>(a, fulld, ncol, stream);
  }
  return launch_split<D, CAUSAL, 1, PARTIAL>(a, fulld, ncol, stream);
}

template <bool PARTIAL>
hipError_t launch_generic(const FwdArgs& a, int d_pad, bool causal, int ncol, hipStream_t stream) {
  const bool fulld = (a.d == d_pad);
  if (d_pad == 64)
    return causal ? launch_one<64, true, PARTIAL>(a, fulld, ncol, stream)
                  : launch_one<64, false, PARTIAL>(a, fulld, ncol, stream);
  if (d_pad == 128)
    return causal ? launch_one<128, true, PARTIAL>(a, fulld, ncol, stream)
                  : launch_one<128, false, PARTIAL>(a, fulld, ncol, stream);
  return causal ? launch_one<256, true, PARTIAL>(a, fulld, ncol, stream)
                : launch_one<256, false, PARTIAL>(a, fulld, ncol, stream);
}

}  // namespace

int f32_rows_per_block(int d) {
  return d <= 64 ? CfgF<64>::NW * 32 : (d <= 128 ? CfgF<128>::NW * 32 : CfgF<256>::NW * 32);
}

hipError_t launch_f32(const FwdArgs& a, int d_pad, bool causal, hipStream_t stream) {
  return launch_generic<false>(a, d_pad, causal, 1, stream);
}

int f32_split_key_tile(int d_pad) {
  return d_pad <= 64 ? CfgF<64>::BC : (d_pad <= 128 ? CfgF<128>::BC : CfgF<256>::BC);
}

hipError_t launch_f32_partial(const FwdArgs& a, int d_pad, bool causal, int nsplit, hipStream_t stream) {
  return launch_generic<true>(a, d_pad, causal, nsplit, stream);
}

}  // namespace fa
