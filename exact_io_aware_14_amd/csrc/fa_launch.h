// fa_launch.h -- host-side launch entry points of the attention kernels.
// Arguments have been validated by the C-ABI layer before these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

enum { kBF16 = 0, kFP32 = 1 };

struct FwdArgs {
  const void *q, *k, *v;
  void* o;
  float* lse;
  int B, H, N, d;
  float scale;
  int causal, dtype;
  void* stream;
};

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float* lse;
  void *dq, *dk, *dv;
  float* Dvec;   // [B*H*N] workspace: D_i = dO_i . O_i
  float* dqacc;  // [B*H*N*d] workspace: float32 dQ accumulator
  int B, H, N, d;
  float scale;
  int causal, dtype;
  void* stream;
};

hipError_t launch_fwd(const FwdArgs& a);
// Backward stages (fields of BwdArgs a stage does not use may be null).
hipError_t launch_bwd_preprocess(const BwdArgs& a);
hipError_t launch_bwd_main(const BwdArgs& a);
hipError_t launch_bwd_finalize(const BwdArgs& a);

}  // namespace fa
