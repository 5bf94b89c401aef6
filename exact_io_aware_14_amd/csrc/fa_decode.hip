// fa_decode.hip -- split-KV attention for decoding and the merge of partials.
//
// "FlashAttention and online softmax" (ML Systems Lesson 4), section "Split-KV for
// decoding (flash-decoding)": with one (or a few) query rows per (batch, head) the
// query-tile grid has only B*H workgroups, so the key/value cache of each row is
// cut into chunks, every chunk gets workgroups of its own and returns a partial
// (o, lse), and a second kernel merges the partials with the formula of section
// "Merging two partial results".
//
// Decoding streams the whole cache once and does two multiply-adds per cached
// element and query, so the pass is bound by HBM, not by the matrix cores: a 32x32
// MFMA tile would carry one useful query row in 32.  The partial kernel therefore
// works on the vector ALUs with every load a full 16-byte row slice:
// * LPK = d*sizeof(T)/16 lanes share one key row (lane l reads bytes 16*(l % LPK)
//   .. of it), so a wave reads 64/LPK consecutive rows = 1 KiB contiguous per load
//   instruction; the dot product with each query is finished by a butterfly of
//   log2(LPK) lane exchanges.
// * The chunk is walked in sub-chunks of 256 keys.  Pass 1 writes the scores of the
//   sub-chunk (exp2 domain: q is pre-scaled by scale*log2 e) to LDS; each wave then
//   takes the max and the exponentials of some query rows; pass 2 streams the V rows
//   and accumulates p * v.  The running max moves once per sub-chunk, rescaling the
//   per-lane accumulators then (the online-softmax theorem at sub-chunk
//   granularity).  Both passes issue all of a lane's row loads for the sub-chunk
//   before using any, to keep enough bytes in flight for HBM.
// * At the end the per-lane partial outputs are summed across the key groups of a
//   wave (lane exchanges) and across the waves (LDS), normalised, and stored as
//   float32 with lse = (m + log2 l) * ln 2.
#include <stdint.h>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kSub = 256;  // keys per sub-chunk

template <typename T>
struct Vec16;
template <>
struct Vec16<__bf16> {
  typedef __bf16 vec_t __attribute__((ext_vector_type(8)));
  static constexpr int N = 8;
};
template <>
struct Vec16<float> {
  typedef float vec_t __attribute__((ext_vector_type(4)));
  static constexpr int N = 4;
};

template <typename T, int D, int NQ>
__global__ __launch_bounds__(kDecThreads) void splitkv_partial_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    float* __restrict__ OP, float* __restrict__ LP, int BH, int Nq, int Nk, int chunk,
    int nsplit, float scale, int causal) {
  using VT = typename Vec16<T>::vec_t;
  constexpr int EPL = Vec16<T>::N;       // elements per lane load
  constexpr int LPK = D / EPL;           // lanes per key row
  constexpr int KPW = 64 / LPK;          // keys per wave step
  constexpr int KPB = KPW * kDecWaves;   // keys per workgroup step
  constexpr int STEPS = kSub / KPB;      // steps per sub-chunk
  static_assert(kSub % KPB == 0 && kSub % 64 == 0, "sub-chunk shape");

  __shared__ float sc[NQ][kSub];          // scores, then weights, of the sub-chunk
  __shared__ float stat[3][NQ];           // running max, sum, last rescale factor
  __shared__ float red[kDecWaves][NQ][D]; // per-wave partial outputs

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane / LPK, sl = lane % LPK;
  const int bh = blockIdx.x / nsplit, s = blockIdx.x - bh * nsplit;
  const int kbeg = s * chunk, kend = min(Nk, kbeg + chunk);
  const size_t qhead = (size_t)bh * Nq * D, khead = (size_t)bh * Nk * D;
  const float c = scale * kLog2e;

  // This lane's slice of every query row, pre-scaled (rows >= Nq are zero, unused).
  float qv[NQ][EPL];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    if (i < Nq) {
      const VT x = *reinterpret_cast<const VT*>(Q + qhead + (size_t)i * D + sl * EPL);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[i][e] = (float)x[e] * c;
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[i][e] = 0.0f;
    }
  }
  float oacc[NQ][EPL];
#pragma unroll
  for (int i = 0; i < NQ; ++i)
#pragma unroll
    for (int e = 0; e < EPL; ++e) oacc[i][e] = 0.0f;
  if (tid < NQ) {
    stat[0][tid] = -INFINITY;  // running max (exp2 domain)
    stat[1][tid] = 0.0f;       // running sum
  }
  // last key visible to query i: i + Nk - Nq (causal), else every key
  const int vis_off = causal ? Nk - Nq : Nk;

  for (int k0 = kbeg; k0 < kend; k0 += kSub) {
    // Pass 1: scores of keys k0 .. k0+kSub-1 (all loads first).
    VT kr[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int key = k0 + st * KPB + w * KPW + grp;
      const int row = min(key, kend - 1);  // rows past the chunk: any valid row, discarded
      kr[st] = *reinterpret_cast<const VT*>(K + khead + (size_t)row * D + sl * EPL);
    }
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int kl = st * KPB + w * KPW + grp;  // key within the sub-chunk
      const int key = k0 + kl;
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = fmaf(qv[i][e], (float)kr[st][e], dot);
#pragma unroll
        for (int m = 1; m < LPK; m <<= 1) dot += __shfl_xor(dot, m);
        const bool vis = key < kend && key <= i + vis_off;
        if (sl == 0 && i < Nq) sc[i][kl] = vis ? dot : -INFINITY;
      }
    }
    __syncthreads();
    // Row max of the sub-chunk, new running max, weights and their sum: wave w takes
    // query rows w, w + 4, ...
    for (int i = w; i < NQ && i < Nq; i += kDecWaves) {
      float x[kSub / 64];
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < kSub / 64; ++t) {
        x[t] = sc[i][lane + 64 * t];
        mx = fmaxf(mx, x[t]);
      }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
      const float mold = stat[0][i];
      const float mnew = fmaxf(mold, mx);
      float sum = 0.0f;
#pragma unroll
      for (int t = 0; t < kSub / 64; ++t) {
        const float p = mnew == -INFINITY ? 0.0f : exp2f(x[t] - mnew);
        sc[i][lane + 64 * t] = p;
        sum += p;
      }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) sum += __shfl_xor(sum, m);
      const float alpha = mold == -INFINITY ? (mnew == -INFINITY ? 1.0f : 0.0f) : exp2f(mold - mnew);
      if (lane == 0) {
        stat[0][i] = mnew;
        stat[1][i] = stat[1][i] * alpha + sum;
        stat[2][i] = alpha;
      }
    }
    __syncthreads();
    // Pass 2: o = o * alpha + sum_k p_k v_k over this lane's keys.
    VT vr[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int key = k0 + st * KPB + w * KPW + grp;
      const int row = min(key, kend - 1);
      vr[st] = *reinterpret_cast<const VT*>(V + khead + (size_t)row * D + sl * EPL);
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i >= Nq) break;
      const float alpha = stat[2][i];
#pragma unroll
      for (int e = 0; e < EPL; ++e) oacc[i][e] *= alpha;
    }
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int kl = st * KPB + w * KPW + grp;
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        if (i >= Nq) break;
        const float p = sc[i][kl];  // 0 for keys past the chunk or hidden by the mask
#pragma unroll
        for (int e = 0; e < EPL; ++e) oacc[i][e] = fmaf(p, (float)vr[st][e], oacc[i][e]);
      }
    }
    __syncthreads();  // sc is rewritten by the next sub-chunk
  }

  // Sum over the KPW key groups of the wave (lanes that share sl), then the waves.
#pragma unroll
  for (int i = 0; i < NQ; ++i)
#pragma unroll
    for (int e = 0; e < EPL; ++e)
#pragma unroll
      for (int m = LPK; m < 64; m <<= 1) oacc[i][e] += __shfl_xor(oacc[i][e], m);
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < NQ; ++i)
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[w][i][sl * EPL + e] = oacc[i][e];
  }
  __syncthreads();
  const size_t prow = ((size_t)s * BH + bh) * Nq;  // first partial row of this (split, b, h)
  for (int x = tid; x < Nq * D; x += kDecThreads) {
    const int i = x / D, e = x - i * D;
    const float l = stat[1][i];
    float o = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) o += red[ww][i][e];
    OP[(prow + i) * D + e] = l > 0.0f ? o / l : 0.0f;
  }
  if (tid < Nq) {
    const float l = stat[1][tid];
    LP[prow + tid] = l > 0.0f ? (stat[0][tid] + log2f(l)) * 0.69314718055994531f : -INFINITY;
  }
}

// One workgroup per row.  Thread s < nsplit loads lse_s; the block forms
// m = max_s lse_s and the weights e^(lse_s - m) in LDS, l = sum of the weights.
// The weighted sum of the partial rows is split over `parts` groups of threads that
// each take every parts-th chunk (independent loads), then added through LDS.
constexpr int kMergeThreads = 256;
template <typename T>
__global__ __launch_bounds__(kMergeThreads) void splitkv_merge_kernel(
    const float* __restrict__ OP, const float* __restrict__ LP, T* __restrict__ O,
    float* __restrict__ LSE, int rows, int d, int nsplit) {
  __shared__ float wts[kMergeThreads];
  __shared__ float red[kMergeThreads];
  __shared__ float part[kMergeThreads];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float ls = tid < nsplit ? LP[(size_t)tid * rows + row] : -INFINITY;
  float m = ls;
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) m = fmaxf(m, __shfl_xor(m, k));
  if (lane == 0) red[wv] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float wgt = (ls == -INFINITY) ? 0.0f : __expf(ls - m);  // an empty chunk: weight 0
  wts[tid] = wgt;
  float l = wgt;
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) l += __shfl_xor(l, k);
  __syncthreads();  // red[] is reused below
  if (lane == 0) red[wv] = l;
  __syncthreads();
  l = red[0] + red[1] + red[2] + red[3];
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;  // l = 0 only when every chunk is empty
  const int parts = (d <= kMergeThreads / 4) ? 4 : (d <= kMergeThreads / 2 ? 2 : 1);
  const int span = kMergeThreads / parts;
  const int pi = tid / span, e0 = tid - pi * span;
  for (int eb = 0; eb < d; eb += span) {
    const int e = eb + e0;
    float o = 0.0f;
    if (e < d) {
#pragma unroll 8
      for (int s = pi; s < nsplit; s += parts) o = fmaf(wts[s], OP[((size_t)s * rows + row) * d + e], o);
    }
    part[tid] = o;
    __syncthreads();
    if (pi == 0 && e < d) {
      float t = o;
      for (int p2 = 1; p2 < parts; ++p2) t += part[p2 * span + e0];
      O[(size_t)row * d + e] = from_f32<T>(t * inv);
    }
    __syncthreads();
  }
  if (tid == 0) LSE[row] = l > 0.0f ? m + logf(l) : -INFINITY;
}

template <typename T, int D, int NQ>
hipError_t launch_partial_q(const SplitArgs& a) {
  const int chunk = (a.Nk + a.nsplit - 1) / a.nsplit;
  const long long grid = (long long)a.B * a.H * a.nsplit;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  launch_begin();
  hipLaunchKernelGGL((splitkv_partial_kernel<T, D, NQ>), dim3((unsigned)grid), dim3(kDecThreads), 0,
                     (hipStream_t)a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.o_part,
                     a.lse_part, a.B * a.H, a.Nq, a.Nk, chunk, a.nsplit, a.scale, a.causal);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_partial_d(const SplitArgs& a) {
  if (a.Nq <= 1) return launch_partial_q<T, D, 1>(a);
  if (a.Nq <= 2) return launch_partial_q<T, D, 2>(a);
  if (a.Nq <= 4) return launch_partial_q<T, D, 4>(a);
  return launch_partial_q<T, D, 8>(a);
}

}  // namespace

hipError_t launch_splitkv_partial(const SplitArgs& a) {
  const bool bf = a.dtype == 0;
  if (a.d == 64) return bf ? launch_partial_d<__bf16, 64>(a) : launch_partial_d<float, 64>(a);
  if (a.d == 128) return bf ? launch_partial_d<__bf16, 128>(a) : launch_partial_d<float, 128>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_splitkv_merge(const MergeArgs& a) {
  if (a.nsplit > kMergeThreads) return hipErrorInvalidValue;
  launch_begin();
  if (a.dtype == 0)
    hipLaunchKernelGGL((splitkv_merge_kernel<__bf16>), dim3((unsigned)a.rows), dim3(kMergeThreads), 0,
                       (hipStream_t)a.stream, a.o_part, a.lse_part, (__bf16*)a.o, a.lse, a.rows,
                       a.d, a.nsplit);
  else
    hipLaunchKernelGGL((splitkv_merge_kernel<float>), dim3((unsigned)a.rows), dim3(kMergeThreads), 0,
                       (hipStream_t)a.stream, a.o_part, a.lse_part, (float*)a.o, a.lse, a.rows,
                       a.d, a.nsplit);
  return hipGetLastError();
}

}  // namespace fa
