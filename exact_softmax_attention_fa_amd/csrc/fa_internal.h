// Internal launch interface between the C-ABI front end (fa_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Arguments shared by every forward kernel. Pointers are per-call device pointers;
// each (b, h) slice of q/k/v/o is N*d contiguous elements, lse holds N floats per slice.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;     // may be null
  int N;          // sequence length (queries = keys)
  int d;          // head dimension actually stored (<= the kernel's padded width)
  int BH;         // B * H
  int n_qtiles;   // ceil(N / rows per workgroup)
  float sl2;      // |scale| * log2(e): scores are kept in base-2 exponent units
  int neg;        // 1 when scale < 0: the kernel negates q (exact) and uses |scale|
};

// Rows of queries per workgroup of the kernel that will run for head width d (host needs it
// for the grid).
int bf16_rows_per_block(int d);
int f32_rows_per_block(int d);

// Enqueue one forward pass. d_pad (64 or 128) is the padded head width of the generic
// kernels. Return hipSuccess or the launch error.
hipError_t launch_bf16(const FwdArgs& a, int d_pad, bool causal, hipStream_t stream);
hipError_t launch_f32(const FwdArgs& a, int d_pad, bool causal, hipStream_t stream);

// Tuned bf16 kernel for head width exactly 128 (rows per workgroup, launch).
int bf16_d128_rows_per_block();
hipError_t launch_bf16_d128(const FwdArgs& a, bool causal, hipStream_t stream);

}  // namespace fa
