// fa_api.hip -- the C ABI of libfa.so: argument checks and kernel dispatch.
// The contract (layout, ownership, error codes) is documented in include/fa.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fa.h"
#include "fa_launch.h"

namespace {

constexpr size_t kWsAlign = 256;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

fa_status check_sizes(int B, int H, int N, int d, float scale, int causal, int dtype) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
  // row indices (B*H*N) are kept below 2^31 so every grid fits a 32-bit id
  if ((long long)B * H * N > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale) || !(scale > 0.0f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// Workspace: D [B*H*Npad] | lse*log2(e) [B*H*Npad] (both dtypes), then for fp32
// only a dQ accumulator [B*H*Npad*d] (float32), then the int32 block plan of the
// variable-length / windowed dK/dV pass; each region 256-byte aligned.
size_t vec_bytes(int B, int H, int N) {
  return round_up((size_t)B * H * fa::pad_rows(N) * sizeof(float), kWsAlign);
}
size_t acc_bytes(int B, int H, int N, int d, int dtype) {
  const size_t prows = (size_t)B * H * fa::pad_rows(N);
  return dtype == FA_DTYPE_FP32 ? round_up(prows * d * sizeof(float), kWsAlign) : 0;
}
size_t ws_bytes(int B, int H, int N, int d, int dtype) {
  const size_t plan = round_up(fa::plan_ints(B, H, N) * sizeof(int), kWsAlign);
  return 2 * vec_bytes(B, H, N) + acc_bytes(B, H, N, d, dtype) + plan;
}

// Extra checks of the variable-length / window calls (see fa.h).
fa_status check_ex(const int* cu, int H, int total, int causal, int window) {
  if (window < 0 || (window > 0 && causal != 1)) return FA_ERR_INVALID_ARG;
  if (cu != nullptr) {
    if (!aligned4(cu) || total < 1) return FA_ERR_INVALID_ARG;
    if ((long long)H * total > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  }
  return FA_OK;
}

// Split-KV decoding sizes (see fa.h).
constexpr int kMaxSplitRows = 8;
constexpr int kMaxSplits = 256;
fa_status check_split(int B, int H, int Nq, int Nk, int d, float scale, int causal,
                      int nsplit, int dtype) {
  if (Nq < 1 || Nk < 1 || nsplit < 1) return FA_ERR_INVALID_ARG;
  fa_status st = check_sizes(B, H, Nk, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  if (Nk < Nq) return FA_ERR_INVALID_ARG;
  if (Nq > kMaxSplitRows || nsplit > kMaxSplits) return FA_ERR_UNSUPPORTED;
  if ((long long)nsplit * B * H * Nq * (d + 1) > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  return FA_OK;
}
size_t split_part_bytes(int B, int H, int Nq, int d, int nsplit) {
  return round_up((size_t)nsplit * B * H * Nq * d * sizeof(float), kWsAlign);
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return (1 << 16) | 1; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration (head dim must be 64 or 128, dtype bf16 or fp32)";
    case FA_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch or the scratch lookup";
    case FA_ERR_TOO_LARGE: return "the call needs more scratch than fa_bwd_noalloc's fixed FA_NOALLOC_SCRATCH_BYTES";
    default: return "unknown status";
  }
}

fa_status fa_fwd_check(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, int B, int H, int N, int d, float softmax_scale,
                       int causal, int dtype) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  const fa_status st = check_sizes(B, H, N, d, softmax_scale, causal, dtype);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  return FA_OK;
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                 int H, int N, int d, float softmax_scale, int causal, int dtype,
                 void* stream) {
  const fa_status st = fa_fwd_check(q, k, v, o, lse, B, H, N, d, softmax_scale, causal, dtype);
  if (st != FA_OK) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, softmax_scale, causal, dtype, stream};
  return fa::launch_fwd(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int dtype) {
  if (check_sizes(B, H, N, d, 1.0f, 0, dtype) != FA_OK) return 0;
  return ws_bytes(B, H, N, d, dtype);
}

fa_status fa_bwd_check(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, const void* dq, const void* dk,
                       const void* dv, const void* workspace, size_t workspace_bytes, int B,
                       int H, int N, int d, float softmax_scale, int causal, int dtype) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
    return FA_ERR_INVALID_ARG;
  const fa_status st = check_sizes(B, H, N, d, softmax_scale, causal, dtype);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) ||
      !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (workspace_bytes < ws_bytes(B, H, N, d, dtype)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

static fa::BwdArgs bwd_args(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            void* workspace, int B, int H, int N, int d, float scale, int causal,
                            int dtype, void* stream) {
  const size_t vb = vec_bytes(B, H, N);
  float* Dvec = (float*)workspace;
  float* L2 = (float*)((char*)workspace + vb);
  float* dqacc = dtype == FA_DTYPE_FP32 ? (float*)((char*)workspace + 2 * vb) : nullptr;
  int* plan = (int*)((char*)workspace + 2 * vb + acc_bytes(B, H, N, d, dtype));
  return fa::BwdArgs{q, k, v, o, dout, lse, dq, dk, dv, Dvec, L2, dqacc, plan,
                     B, H, N, d, fa::pad_rows(N), scale, causal, dtype, stream};
}

// The backward's launches.  bf16: the dQ pass with the preprocess folded in (it writes
// D and lse*log2(e) for the dK/dV pass), then the dK/dV pass.  fp32: preprocess, dK/dV
// pass (which adds the dQ contributions to the accumulator), dQ conversion.
// `launches` selects a subset (bit 0: the first launch, bit 1: the second, bit 2: the
// third), for callers that time them one by one.
static fa_status run_bwd(const fa::BwdArgs& a, int launches = 7) {
  if (a.dtype == FA_DTYPE_BF16) {
    if ((launches & 1) && fa::launch_bwd_dq_pre_bf16(a) != hipSuccess) return FA_ERR_LAUNCH;
    if ((launches & 2) && fa::launch_bwd_main(a) != hipSuccess) return FA_ERR_LAUNCH;
    return FA_OK;
  }
  if ((launches & 1) && fa::launch_bwd_preprocess(a) != hipSuccess) return FA_ERR_LAUNCH;
  if ((launches & 2) && fa::launch_bwd_main(a) != hipSuccess) return FA_ERR_LAUNCH;
  if ((launches & 4) && fa::launch_bwd_dq(a) != hipSuccess) return FA_ERR_LAUNCH;
  return FA_OK;
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int B, int H, int N, int d, float softmax_scale,
                 int causal, int dtype, void* stream) {
  const fa_status st = fa_bwd_check(q, k, v, o, dout, lse, dq, dk, dv, workspace,
                                    workspace_bytes, B, H, N, d, softmax_scale, causal, dtype);
  if (st != FA_OK) return st;
  const fa::BwdArgs a = bwd_args(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N, d,
                                 softmax_scale, causal, dtype, stream);
  return run_bwd(a);
}

fa_status fa_bwd_preprocess(const void* o, const void* dout, const float* lse,
                            void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                            int dtype, void* stream) {
  // the pointers this stage does not take are stood in for by `o` in the full check
  const fa_status st = fa_bwd_check(o, o, o, o, dout, lse, o, o, o, workspace,
                                    workspace_bytes, B, H, N, d, 1.0f, 0, dtype);
  if (st != FA_OK) return st;
  const fa::BwdArgs a = bwd_args(nullptr, nullptr, nullptr, o, dout, lse, nullptr, nullptr,
                                 nullptr, workspace, B, H, N, d, 1.0f, 0, dtype, stream);
  return fa::launch_bwd_preprocess(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_bwd_main(const void* q, const void* k, const void* v, const void* dout,
                      void* dk, void* dv, void* workspace, size_t workspace_bytes, int B,
                      int H, int N, int d, float softmax_scale, int causal, int dtype,
                      void* stream) {
  const fa_status st = fa_bwd_check(q, k, v, q, dout, (const float*)q, dk, dk, dv, workspace,
                                    workspace_bytes, B, H, N, d, softmax_scale, causal, dtype);
  if (st != FA_OK) return st;
  const fa::BwdArgs a = bwd_args(q, k, v, nullptr, dout, nullptr, nullptr, dk, dv, workspace, B,
                                 H, N, d, softmax_scale, causal, dtype, stream);
  return fa::launch_bwd_main(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq,
                    void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                    float softmax_scale, int causal, int dtype, void* stream) {
  const fa_status st = fa_bwd_check(q, k, v, q, dout, (const float*)q, dq, dq, dq, workspace,
                                    workspace_bytes, B, H, N, d, softmax_scale, causal, dtype);
  if (st != FA_OK) return st;
  const fa::BwdArgs a = bwd_args(q, k, v, nullptr, dout, nullptr, dq, nullptr, nullptr, workspace,
                                 B, H, N, d, softmax_scale, causal, dtype, stream);
  return fa::launch_bwd_dq(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_bwd_dq_pre(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* workspace,
                        size_t workspace_bytes, int B, int H, int N, int d, float softmax_scale,
                        int causal, int dtype, void* stream) {
  const fa_status st = fa_bwd_check(q, k, v, o, dout, lse, dq, dq, dq, workspace, workspace_bytes, B,
                                    H, N, d, softmax_scale, causal, dtype);
  if (st != FA_OK) return st;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  const fa::BwdArgs a = bwd_args(q, k, v, o, dout, lse, dq, nullptr, nullptr, workspace, B, H, N, d,
                                 softmax_scale, causal, dtype, stream);
  return fa::launch_bwd_dq_pre_bf16(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_splitkv_workspace_bytes(int B, int H, int Nq, int d, int num_splits) {
  if (check_split(B, H, Nq, Nq, d, 1.0f, 0, num_splits, FA_DTYPE_FP32) != FA_OK) return 0;
  return split_part_bytes(B, H, Nq, d, num_splits) +
         round_up((size_t)num_splits * B * H * Nq * sizeof(float), kWsAlign);
}

fa_status fa_fwd_partial(const void* q, const void* k, const void* v, float* o_part,
                         float* lse_part, int B, int H, int Nq, int Nk, int d,
                         float softmax_scale, int causal, int num_splits, int dtype,
                         void* stream) {
  if (!q || !k || !v || !o_part || !lse_part) return FA_ERR_INVALID_ARG;
  const fa_status st = check_split(B, H, Nq, Nk, d, softmax_scale, causal, num_splits, dtype);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_part) || !aligned4(lse_part))
    return FA_ERR_INVALID_ARG;
  const fa::SplitArgs a{q, k, v, o_part, lse_part, B, H, Nq, Nk, d, softmax_scale, causal,
                        num_splits, dtype, stream};
  return fa::launch_splitkv_partial(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_merge(const float* o_part, const float* lse_part, void* o, float* lse,
                   int num_splits, int rows, int d, int dtype, void* stream) {
  if (!o_part || !lse_part || !o || !lse) return FA_ERR_INVALID_ARG;
  if (num_splits < 1 || rows < 1 || d < 1 || d > 1024) return FA_ERR_INVALID_ARG;
  if (num_splits > kMaxSplits) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
  if ((long long)num_splits * rows * d > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  const size_t ea = dtype == FA_DTYPE_FP32 ? 4 : 2;
  if (!aligned4(o_part) || !aligned4(lse_part) || !aligned4(lse) || ((uintptr_t)o % ea) != 0)
    return FA_ERR_INVALID_ARG;
  const fa::MergeArgs a{o_part, lse_part, o, lse, num_splits, rows, d, dtype, stream};
  return fa::launch_splitkv_merge(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int Nq, int Nk, int d, float softmax_scale, int causal,
                         int num_splits, void* workspace, size_t workspace_bytes, int dtype,
                         void* stream) {
  if (!q || !k || !v || !o || !lse || !workspace) return FA_ERR_INVALID_ARG;
  const fa_status st = check_split(B, H, Nq, Nk, d, softmax_scale, causal, num_splits, dtype);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse) ||
      !aligned16(workspace))
    return FA_ERR_INVALID_ARG;
  if (workspace_bytes < fa_splitkv_workspace_bytes(B, H, Nq, d, num_splits)) return FA_ERR_INVALID_ARG;
  float* o_part = (float*)workspace;
  float* lse_part = (float*)((char*)workspace + split_part_bytes(B, H, Nq, d, num_splits));
  const fa::SplitArgs a{q, k, v, o_part, lse_part, B, H, Nq, Nk, d, softmax_scale, causal,
                        num_splits, dtype, stream};
  if (fa::launch_splitkv_partial(a) != hipSuccess) return FA_ERR_LAUNCH;
  const fa::MergeArgs m{o_part, lse_part, o, lse, num_splits, B * H * Nq, d, dtype, stream};
  return fa::launch_splitkv_merge(m) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens, int B, int H, int N, int total, int d,
                    float softmax_scale, int causal, int window, int dtype, void* stream) {
  fa_status st = fa_fwd_check(q, k, v, o, lse, B, H, N, d, softmax_scale, causal, dtype);
  if (st != FA_OK) return st;
  st = check_ex(cu_seqlens, H, total, causal, window);
  if (st != FA_OK) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, softmax_scale, causal, dtype, stream};
  a.cu_seqlens = cu_seqlens;
  a.T = cu_seqlens ? total : 0;
  a.window = window;
  return fa::launch_fwd(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, void* workspace,
                    size_t workspace_bytes, const int* cu_seqlens, int B, int H, int N, int total,
                    int d, float softmax_scale, int causal, int window, int dtype, void* stream) {
  return fa_bwd_ex_launches(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes,
                            cu_seqlens, B, H, N, total, d, softmax_scale, causal, window, dtype,
                            FA_BWD_ALL_LAUNCHES, stream);
}

fa_status fa_bwd_ex_launches(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, const int* cu_seqlens, int B,
                             int H, int N, int total, int d, float softmax_scale, int causal,
                             int window, int dtype, int launches, void* stream) {
  if (launches < 1 || launches > FA_BWD_ALL_LAUNCHES) return FA_ERR_INVALID_ARG;
  fa_status st = fa_bwd_check(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H,
                              N, d, softmax_scale, causal, dtype);
  if (st != FA_OK) return st;
  st = check_ex(cu_seqlens, H, total, causal, window);
  if (st != FA_OK) return st;
  fa::BwdArgs a = bwd_args(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N, d, softmax_scale,
                           causal, dtype, stream);
  a.cu_seqlens = cu_seqlens;
  a.T = cu_seqlens ? total : 0;
  a.window = window;
  return run_bwd(a, launches);
}

}  // extern "C"

// ---- fa_bwd_noalloc: fa_bwd with a library-owned workspace ---------------------------
// The workspace (D and lse*log2(e) vectors, plus the fp32 path's dQ accumulator) lives
// in this file-scope device array instead of caller memory.  Each device the library
// runs on holds its own copy from module load until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: its device address comes
// from hipGetSymbolAddress, once per device, and only that address is handed to the
// kernels.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call there).
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                    int B, int H, int N, int d, float softmax_scale, int causal,
                                    int dtype, void* stream) {
  // The checks of fa_bwd with a stand-in workspace (aligned, large enough): they do not
  // read it.
  fa_status st = fa_bwd_check(q, k, v, o, dout, lse, dq, dk, dv, (const void*)256, (size_t)-1, B,
                              H, N, d, softmax_scale, causal, dtype);
  if (st != FA_OK) return st;
  if (ws_bytes(B, H, N, d, dtype) > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return FA_ERR_LAUNCH;
  // The preprocess writes every padded row of D and lse*log2(e) and clears the fp32
  // accumulator, so nothing a previous call left in the scratch is read.
  const fa::BwdArgs a = bwd_args(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, N, d, softmax_scale,
                                 causal, dtype, stream);
  return run_bwd(a);
}
