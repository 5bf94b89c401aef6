// fa_bwd.hip -- backward pass of exact tiled attention for gfx950.
//
// Method ("FlashAttention and online softmax", ML Systems Lesson 4, section
// "Backward pass: recompute instead of store"): the forward keeps only O and the
// per-row lse; the backward rebuilds each score tile S = tau Q_i K_j^T and
// P = exp(S - lse) (no running max or sum needed), then
//   dV_j += P^T dO_i,  dP = dO_i V_j^T,  dS = P o (dP - D_i),
//   dQ_i += tau dS K_j,  dK_j += tau dS^T Q_i,   with D_i = dO_i . O_i.
//
// Three stages on the caller's stream:
//   1. bwd_pre:     D = rowsum(dO o O) and lse in base 2 per padded row, in fp32
//                   (both dtypes); for fp32 also a zeroed fp32 dQ accumulator.
//   2. main:        dK and dV.  bf16: fa_bwd_bf16.hip.  fp32: bwd_main_kernel below,
//                   one workgroup per (batch, head, block of 32*NW keys); K_j and
//                   V_j stay in registers, dK_j and dV_j accumulate in registers;
//                   query tiles stream through LDS; each wave owns 32 keys, so
//                   dK/dV never need a cross-wave reduction; dQ contributions are
//                   added with fp32 atomics into the accumulator.
//   3. dQ:          bf16: the query-stationary dQ pass (fa_bwd_dq_bf16.hip).
//                   fp32: dq_convert, dQ = tau * accumulator.
//
// gfx950 mapping.  S = Q K^T and dP = dO V^T are computed with keys on the lane
// columns of the 32x32 MFMA accumulator, which makes P^T and dS^T valid A operands
// (c-layout k order) of dV = P^T dO and dK = dS^T Q without any shuffle; their B
// operands (dO, Q) are gathered from LDS in that same k order.  dQ = dS K needs dS
// with queries on lanes, so dS takes one trip through LDS, and K^T is kept in LDS
// for the B operand of that product.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO o O), L2 = lse * log2(e) per padded row (D = 0, L2 = +inf on
//    the padding rows N .. Npad-1 of each head); zero the dQ accumulator.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O,
                                                      const T* __restrict__ dO,
                                                      const float* __restrict__ LSE,
                                                      float* __restrict__ Dvec,
                                                      float* __restrict__ L2,
                                                      float* __restrict__ dqacc, int N,
                                                      int Npad, long long prow_total,
                                                      SeqMap sm) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int TPR = D / VEC;  // threads per row (divides 64)
  static_assert(64 % TPR == 0, "a row's threads must sit in one wave");
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long prow = gid / TPR;  // padded row index (bh * Npad + q)
  const int part = (int)(gid % TPR);
  const long long bh = prow / Npad;
  const int q = (int)(prow - bh * Npad);
  int base = 0, len = 0;
  if (prow < prow_total) seq_rows(sm, (int)bh, N, base, len);
  const bool live = prow < prow_total && q < len;
  float acc = 0.0f;
  if (live) {
    const size_t off = ((size_t)base + q) * D + part * VEC;
    const T* po = O + off;
    const T* pd = dO + off;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc = fmaf(to_f32(po[e]), to_f32(pd[e]), acc);
  }
  if (dqacc != nullptr && prow < prow_total) {  // Npad accumulator rows per head: clear all
    float4* z = reinterpret_cast<float4*>(dqacc + (size_t)prow * D + part * VEC);
#pragma unroll
    for (int e = 0; e < VEC / 4; ++e) z[e] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int o = TPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (prow < prow_total && part == 0) {
    Dvec[prow] = live ? acc : 0.0f;
    L2[prow] = live ? LSE[(size_t)base + q] * kLog2e : INFINITY;
  }
}

// ---------------------------------------------------------------------------
// 3. dQ = scale * accumulator in the storage dtype (4 elements per thread).  The
//    accumulator has Npad rows per head; only the head's live rows are converted.
template <typename T>
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc,
                                                         T* __restrict__ dQ, long long n4,
                                                         int N, int Npad, int d4,
                                                         float scale, SeqMap sm) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // over B*H*Npad*d/4
  if (i >= n4) return;
  const long long prow = i / d4;  // bh * Npad + q
  const long long bh = prow / Npad;
  const int q = (int)(prow - bh * Npad);
  int base, len;
  seq_rows(sm, (int)bh, N, base, len);
  if (q >= len) return;
  const long long col4 = i - prow * d4;
  const float4 v = reinterpret_cast<const float4*>(acc)[i];
  T* p = dQ + (((size_t)base + q) * d4 + col4) * 4;
  p[0] = from_f32<T>(v.x * scale);
  p[1] = from_f32<T>(v.y * scale);
  p[2] = from_f32<T>(v.z * scale);
  p[3] = from_f32<T>(v.w * scale);
}

// ---------------------------------------------------------------------------
// 2. main kernel
template <typename T, int D, int NW>
struct BwdCfg {
  static constexpr int NT = 64 * NW;
  static constexpr int BKV = 32 * NW;         // keys per workgroup
  static constexpr int BQ = 32;               // queries per streamed tile
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int LDQ = D + VEC;         // row stride of the Q / dO tiles
  static constexpr int LDS_ = BKV + VEC;      // row stride of the dS tile
  static constexpr int LDK = BKV + VEC;       // row stride of K^T (one row per dim)
  static constexpr int CPR = D / VEC;         // 16-byte chunks per row
  static constexpr int NDT = D / 32;          // 32-wide dim tiles
  static constexpr int NKP = NW / NDT;        // key parts per dQ tile (>= 1)
  static_assert(NW % NDT == 0, "waves must cover the dQ dim tiles");
};

template <typename T, int D, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_main_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dvec,
    float* __restrict__ dqacc, T* __restrict__ dK, T* __restrict__ dV, int Nmax, int Npad,
    float scale, int causal, int nkb, SeqMap sm, int window) {
  using C = BwdCfg<T, D, NW>;
  using M = Mma<T>;
  typedef typename M::op_t op_t;
  constexpr int KPI = M::KPI, EPL = M::EPL;
  constexpr int NKK = D / KPI;
  constexpr int NDT = C::NDT;
  constexpr int NJ = 32 / KPI;

  __shared__ __attribute__((aligned(16))) T Qs[C::BQ * C::LDQ];
  __shared__ __attribute__((aligned(16))) T dOs[C::BQ * C::LDQ];
  __shared__ __attribute__((aligned(16))) T dSs[C::BQ * C::LDS_];
  __shared__ __attribute__((aligned(16))) T Kt[D * C::LDK];
  __shared__ float lse_s[C::BQ];
  __shared__ float D_s[C::BQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / nkb;
  const int kb = id - bh * nkb;  // ascending: under a causal mask block 0 has the most work
  int base, N;  // first row and length of this (batch, head)
  seq_rows(sm, bh, Nmax, base, N);
  const size_t head = (size_t)base * D;
  const int k0 = kb * C::BKV;
  if (k0 >= N) return;  // a short sequence of a variable-length batch: no keys here
  const int kw = k0 + w * 32;  // first key of this wave
  const int mykey = kw + l32;

  // K and V of this wave's 32 keys as B operands (natural k assignment).
  op_t kop[NKK], vop[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const size_t off = head + (size_t)mykey * D + kk * KPI + g * EPL;
    kop[kk] = mykey < N ? M::load(K + off) : M::zero();
    vop[kk] = mykey < N ? M::load(V + off) : M::zero();
  }
  // K^T of the whole key block into LDS (B operand of dQ = dS K).
  for (int idx = tid; idx < C::BKV * C::CPR; idx += C::NT) {
    const int r = idx / C::CPR, col = (idx % C::CPR) * C::VEC;
    const int key = k0 + r;
    T vals[C::VEC];
    if (key < N) {
      *reinterpret_cast<v16b*>(vals) = *reinterpret_cast<const v16b*>(K + head + (size_t)key * D + col);
    } else {
#pragma unroll
      for (int e = 0; e < C::VEC; ++e) vals[e] = from_f32<T>(0.0f);
    }
#pragma unroll
    for (int e = 0; e < C::VEC; ++e) Kt[(col + e) * C::LDK + r] = vals[e];
  }

  f32x16_t dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    dk[dt] = zero16();
    dv[dt] = zero16();
  }
  const float c = scale * kLog2e;
  int nqt = (N + C::BQ - 1) / C::BQ;
  const int qt0 = causal ? k0 / C::BQ : 0;  // earlier query rows see none of these keys
  if (window > 0)  // nor do rows past the last key's band
    nqt = min(nqt, (k0 + C::BKV - 1 + window - 1) / C::BQ + 1);
  const int dq_dt = w % NDT, dq_kp = w / NDT;
  constexpr int KPART = C::BKV / C::NKP;

  for (int qt = qt0; qt < nqt; ++qt) {
    const int qb0 = qt * C::BQ;
    __syncthreads();  // the previous tile's Q, dO and dS are no longer read
    for (int idx = tid; idx < C::BQ * C::CPR; idx += C::NT) {
      const int r = idx / C::CPR, col = (idx % C::CPR) * C::VEC;
      const int q = qb0 + r;
      v16b xq{0, 0, 0, 0}, xd{0, 0, 0, 0};
      if (q < N) {
        xq = *reinterpret_cast<const v16b*>(Q + head + (size_t)q * D + col);
        xd = *reinterpret_cast<const v16b*>(dO + head + (size_t)q * D + col);
      }
      *reinterpret_cast<v16b*>(Qs + r * C::LDQ + col) = xq;
      *reinterpret_cast<v16b*>(dOs + r * C::LDQ + col) = xd;
    }
    if (tid < C::BQ) {  // padded vectors: rows past N hold lse = +inf, D = 0
      lse_s[tid] = L2[(size_t)bh * Npad + qb0 + tid];
      D_s[tid] = Dvec[(size_t)bh * Npad + qb0 + tid];
    }
    __syncthreads();

    // S = Q K^T and dP = dO V^T: 32 queries (rows) x this wave's 32 keys (lanes).
    f32x16_t s = zero16(), dp = zero16();
    const T* qrow = Qs + l32 * C::LDQ + g * EPL;
    const T* drow = dOs + l32 * C::LDQ + g * EPL;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      s = M::mma(M::load(qrow + kk * KPI), kop[kk], s);
      dp = M::mma(M::load(drow + kk * KPI), vop[kk], dp);
    }
    // P = exp(S - lse) on visible pairs, dS = P o (dP - D).
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ql = crow(g, r);
      const int q = qb0 + ql;
      const bool vis = mykey < N && q < N && (!causal || mykey <= q) && (window <= 0 || mykey > q - window);
      const float p = vis ? __builtin_amdgcn_exp2f(fmaf(s[r], c, -lse_s[ql])) : 0.0f;
      s[r] = p;
      dp[r] = p * (dp[r] - D_s[ql]);
    }
    // dV += P^T dO, dK += dS^T Q  (keys x dims, contraction over the 32 queries).
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const op_t pa = M::from_acc(s, j * EPL);
      const op_t da = M::from_acc(dp, j * EPL);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        auto offs = [&](int sl) { return crow(g, j * EPL + sl) * C::LDQ; };
        const op_t bdo = M::gather(dOs + dt * 32 + l32, offs);
        const op_t bq = M::gather(Qs + dt * 32 + l32, offs);
        dv[dt] = M::mma(pa, bdo, dv[dt]);
        dk[dt] = M::mma(da, bq, dk[dt]);
      }
    }
    // dS (queries x keys) into LDS for dQ.
#pragma unroll
    for (int r = 0; r < 16; ++r) dSs[crow(g, r) * C::LDS_ + w * 32 + l32] = from_f32<T>(dp[r]);
    __syncthreads();

    // dQ tile (32 queries x 32 dims) of this wave over its share of the block's keys.
    f32x16_t dq = zero16();
    const T* arow = dSs + l32 * C::LDS_ + dq_kp * KPART + g * EPL;
    const T* brow = Kt + (dq_dt * 32 + l32) * C::LDK + dq_kp * KPART + g * EPL;
#pragma unroll
    for (int kk = 0; kk < KPART / KPI; ++kk)
      dq = M::mma(M::load(arow + kk * KPI), M::load(brow + kk * KPI), dq);
#pragma unroll
    for (int r = 0; r < 16; ++r) {  // padded accumulator rows: no bounds test
      const int q = qb0 + crow(g, r);
      unsafeAtomicAdd(dqacc + ((size_t)bh * Npad + q) * D + dq_dt * 32 + l32, dq[r]);
    }
  }

  // dK (scaled) and dV: lane = dim column, register = key row.
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw + crow(g, r);
      if (key < N) {
        const size_t off = head + (size_t)key * D + dt * 32 + l32;
        dK[off] = from_f32<T>(dk[dt][r] * scale);
        dV[off] = from_f32<T>(dv[dt][r]);
      }
    }
}

template <typename T, int D>
static hipError_t launch_pre_cfg(const BwdArgs& a) {
  const long long prows = (long long)a.B * a.H * a.Npad;
  constexpr int TPR = D / (16 / sizeof(T));
  const long long blocks = (prows * TPR + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  launch_begin();
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)a.stream, (const T*)a.o, (const T*)a.dout, a.lse, a.Dvec, a.L2,
                     a.dqacc, a.N, a.Npad, prows, SeqMap{a.cu_seqlens, a.B, a.T});
  return hipGetLastError();
}

template <typename T, int D, int NW>
static hipError_t launch_main_cfg(const BwdArgs& a) {
  using C = BwdCfg<T, D, NW>;
  const int nkb = (a.N + C::BKV - 1) / C::BKV;
  const long long grid = (long long)a.B * a.H * nkb;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  launch_begin();
  hipLaunchKernelGGL((bwd_main_kernel<T, D, NW>), dim3((unsigned)grid), dim3(C::NT), 0,
                     (hipStream_t)a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                     (const T*)a.dout, a.L2, a.Dvec, a.dqacc, (T*)a.dk, (T*)a.dv, a.N, a.Npad,
                     a.scale, a.causal, nkb, SeqMap{a.cu_seqlens, a.B, a.T}, a.window);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_fin_cfg(const BwdArgs& a) {
  const long long n4 = (long long)a.B * a.H * a.Npad * a.d / 4;
  const long long blocks = (n4 + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  launch_begin();
  hipLaunchKernelGGL((dq_convert_kernel<T>), dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)a.stream, a.dqacc, (T*)a.dq, n4, a.N, a.Npad, a.d / 4,
                     a.scale, SeqMap{a.cu_seqlens, a.B, a.T});
  return hipGetLastError();
}

hipError_t launch_bwd_preprocess(const BwdArgs& a) {
  if (a.dtype == kBF16) {
    if (a.d == 64) return launch_pre_cfg<__bf16, 64>(a);
    if (a.d == 128) return launch_pre_cfg<__bf16, 128>(a);
  } else {
    if (a.d == 64) return launch_pre_cfg<float, 64>(a);
    if (a.d == 128) return launch_pre_cfg<float, 128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_main(const BwdArgs& a) {
  if (a.dtype == kBF16) {
    return launch_bwd_main_bf16(a);
  } else {
    if (a.d == 64) return launch_main_cfg<float, 64, 4>(a);
    if (a.d == 128) return launch_main_cfg<float, 128, 4>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq(const BwdArgs& a) {
  return a.dtype == kBF16 ? launch_bwd_dq_bf16(a) : launch_fin_cfg<float>(a);
}

}  // namespace fa
