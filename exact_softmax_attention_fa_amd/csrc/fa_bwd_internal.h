// Internal launch interface between the C-ABI front end (fa_api.hip) and the backward kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Backward pass (bf16). Pointers as in the forward plus the saved output o, its gradient
// dout, the forward's log-normaliser lse (natural log), the gradients dq, dk, dv (written)
// and delta, a caller-provided fp32 workspace of B*H*N floats (written).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;
  int N;
  int d;          // 64 or 128
  int BH;
  float sl2;      // |scale| * log2(e)
  int neg;        // 1 when scale < 0
};
int bwd_rows_per_block();
hipError_t launch_bwd_bf16(const BwdArgs& a, bool causal, hipStream_t stream);

}  // namespace fa
