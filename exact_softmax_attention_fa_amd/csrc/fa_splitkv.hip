// Merge pass of the split key range (split-KV): combine the partial states of every row.
//
// When the keys of a row are split into ranges handled by different workgroups, each range
// leaves the three statistics of the online softmax for that row: its reference maximum m_s,
// its denominator l_s and its unnormalised numerator u_s (a d-vector). The states merge with
// the rule for combining two blocks (interactiveml.org, "FlashAttention saves the matrix, not
// the quadratic work", merge of the three sufficient statistics):
//   m* = max_s m_s,   w_s = e^(m_s - m*),   l = sum_s w_s l_s,   u = sum_s w_s u_s,
// and then o = u / l, lse = m* + ln l. A range that saw no key of the row has m_s = -inf and
// weight 0. Here the exponentials are base 2: the partial kernels keep m either in base-2
// units of the scaled scores (bf16 kernels, weight 2^(m_s - m*)) or on the unscaled scores
// (fp32 kernel, weight 2^((m_s - m*) * scale * log2 e)).
//
// One thread per (row, 4 features): the partial numerators are read as 16-byte vectors, the
// (m, l) pairs as 8-byte ones (shared by the threads of a row). The pass reads
// nsplit * (d_pad + 2) * 4 bytes per row and writes the row of o and its lse.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 x = {lo, hi};   // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

constexpr int kMergeThreads = 256;

template <int D, bool OUT_F32>
__global__ __launch_bounds__(kMergeThreads)
void merge_kernel(FwdArgs a, int nsplit, int causal, int m_unscaled) {
  constexpr int TPR = D / 4;                 // threads per row
  constexpr int RPB = kMergeThreads / TPR;   // rows per workgroup
  const int N = a.N, d = a.d;
  const long long rows = (long long)a.BH * N;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= rows) return;
  const int c4 = (threadIdx.x % TPR) * 4;
  const int i = (int)(row % N);   // query index within its head

  // Split columns that hold keys row i may see: under the causal mask only columns starting at
  // or before key i (the partial kernels wrote nothing for the others).
  const int ns = causal ? min(nsplit, i / a.kv_chunk + 1) : nsplit;
  const size_t col_stride = (size_t)rows;   // rows per split column
  const float ms = m_unscaled ? a.sl2 : 1.0f;

  float mstar = -INFINITY;
  for (int s = 0; s < ns; ++s) mstar = fmaxf(mstar, a.part_ml[2 * (s * col_stride + row)]);

  float l = 0.0f;
  float4 u = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < ns; ++s) {
    const size_t r = s * col_stride + row;
    const float2 ml = *(const float2*)(a.part_ml + 2 * r);
    // weight 0 for a range without keys of this row (m = -inf, l = 0, u = 0)
    const float w = ml.x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((ml.x - mstar) * ms);
    const float4 us = *(const float4*)(a.part_u + r * D + c4);
    l = fmaf(w, ml.y, l);
    u.x = fmaf(w, us.x, u.x);
    u.y = fmaf(w, us.y, u.y);
    u.z = fmaf(w, us.z, u.z);
    u.w = fmaf(w, us.w, u.w);
  }

  const float inv = 1.0f / l;
  const float x[4] = {u.x * inv, u.y * inv, u.z * inv, u.w * inv};
  const size_t obase = (size_t)row * d + c4;
  if (OUT_F32) {
    float* orow = (float*)a.o + obase;
    if (c4 + 4 <= d && (d & 3) == 0) {
      *(float4*)orow = make_float4(x[0], x[1], x[2], x[3]);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (c4 + t < d) orow[t] = x[t];
    }
  } else {
    uint16_t* orow = (uint16_t*)a.o + obase;
    if (c4 + 4 <= d && (d & 3) == 0) {
      const uint2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      *(uint2*)orow = w;
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (c4 + t < d) orow[t] = __builtin_bit_cast(uint16_t, (__bf16)x[t]);
    }
  }
  if (a.lse != nullptr && c4 == 0) a.lse[row] = (mstar * ms + log2f(l)) * 0.69314718055994531f;
}

template <int D, bool OUT_F32>
hipError_t launch_merge_d(const FwdArgs& a, int nsplit, bool causal, bool m_unscaled, hipStream_t stream) {
  constexpr int RPB = kMergeThreads / (D / 4);
  const long long rows = (long long)a.BH * a.N;
  const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
  hipLaunchKernelGGL((merge_kernel<D, OUT_F32>), grid, dim3(kMergeThreads), 0, stream, a, nsplit, causal ? 1 : 0,
                     m_unscaled ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const FwdArgs& a, int d_pad, bool causal, int nsplit, bool m_unscaled, bool out_f32,
                        hipStream_t stream) {
  if (out_f32) {
    if (d_pad == 64) return launch_merge_d<64, true>(a, nsplit, causal, m_unscaled, stream);
    if (d_pad == 128) return launch_merge_d<128, true>(a, nsplit, causal, m_unscaled, stream);
    return launch_merge_d<256, true>(a, nsplit, causal, m_unscaled, stream);
  }
  if (d_pad == 64) return launch_merge_d<64, false>(a, nsplit, causal, m_unscaled, stream);
  if (d_pad == 128) return launch_merge_d<128, false>(a, nsplit, causal, m_unscaled, stream);
  return launch_merge_d<256, false>(a, nsplit, causal, m_unscaled, stream);
}

}  // namespace fa
