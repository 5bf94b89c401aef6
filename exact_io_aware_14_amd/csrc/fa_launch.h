// fa_launch.h -- host-side launch entry points of the attention kernels.
// Arguments have been validated by the C-ABI layer before these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

#include <atomic>

namespace fa {

enum { kBF16 = 0, kFP32 = 1 };

// Called right before each kernel launch: takes an error that earlier, unrelated HIP
// calls left in this thread's error slot out of it, so that the hipGetLastError()
// after the launch reports only what the launch itself caused.
inline void launch_begin() { (void)hipGetLastError(); }

// Compute units of the current device, queried once per device (0 if the query fails:
// callers then launch one workgroup per block).
inline int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Per-head row padding of the backward's D and lse workspace vectors: every
// backward query tile (32 rows) reads whole padded vectors.
constexpr int kRowPad = 32;
inline int pad_rows(int N) { return (N + kRowPad - 1) / kRowPad * kRowPad; }

// The block plan of a variable-length or windowed dK/dV launch (workspace, int32): a
// header of kPlanHead values, then one id per block of keys, at most one per 128 keys of
// every (batch, head) unit.
constexpr int kPlanHead = 16;
constexpr int kPlanKeys = 128;
inline size_t plan_ints(int B, int H, int N) {
  return kPlanHead + (size_t)B * H * ((N + kPlanKeys - 1) / kPlanKeys);
}

// Dense calls: cu_seqlens = null, N the sequence length.  Variable-length calls:
// cu_seqlens = B+1 device boundaries, tensors packed [H, T, d], N the longest length.
// window > 0: causal band, query i sees key j iff i - window < j <= i.
struct FwdArgs {
  const void *q, *k, *v;
  void* o;
  float* lse;
  int B, H, N, d;
  float scale;
  int causal, dtype;
  void* stream;
  const int* cu_seqlens = nullptr;
  int T = 0;
  int window = 0;
};

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float* lse;
  void *dq, *dk, *dv;
  float* Dvec;   // [B*H*Npad] workspace: D_i = dO_i . O_i (0 on padding rows)
  float* L2;     // [B*H*Npad] workspace: lse_i * log2(e) (+inf on padding rows)
  float* dqacc;  // [B*H*Npad*d] workspace float32 dQ accumulator (fp32 path only; null for bf16)
  int* plan;     // [plan_ints(B, H, N)] workspace: block plan of general bf16 dK/dV launches
  int B, H, N, d;
  int Npad;      // N rounded up to kRowPad
  float scale;
  int causal, dtype;
  void* stream;
  const int* cu_seqlens = nullptr;
  int T = 0;
  int window = 0;
};

// Split-KV decoding: partials of every key chunk, then their merge.
struct SplitArgs {
  const void *q, *k, *v;
  float* o_part;    // [nsplit, B, H, Nq, d]
  float* lse_part;  // [nsplit, B, H, Nq]
  int B, H, Nq, Nk, d;
  float scale;
  int causal, nsplit, dtype;
  void* stream;
};
struct MergeArgs {
  const float* o_part;
  const float* lse_part;
  void* o;
  float* lse;
  int nsplit, rows, d, dtype;
  void* stream;
};
hipError_t launch_splitkv_partial(const SplitArgs& a);
hipError_t launch_splitkv_merge(const MergeArgs& a);
hipError_t launch_fwd(const FwdArgs& a);       // dispatches on dtype
hipError_t launch_fwd_bf16(const FwdArgs& a);  // the gfx950-tuned bf16 kernel
// Backward stages (fields of BwdArgs a stage does not use may be null).
hipError_t launch_bwd_preprocess(const BwdArgs& a);
hipError_t launch_bwd_main(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);
hipError_t launch_bwd_main_bf16(const BwdArgs& a);  // gfx950-tuned bf16 dK/dV pass
hipError_t launch_bwd_dq_bf16(const BwdArgs& a);    // gfx950-tuned bf16 dQ pass
// bf16 dQ pass with the preprocess folded in: also writes D and lse*log2(e) (needs o, lse)
hipError_t launch_bwd_dq_pre_bf16(const BwdArgs& a);

}  // namespace fa
