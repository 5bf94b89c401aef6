// fa_fwd.hip -- forward pass of exact tiled attention for gfx950.
//
// Method ("FlashAttention and online softmax", ML Systems Lesson 4, section "3.
// Definitions and main results", the tiled forward pass under "The online softmax
// theorem"): a workgroup owns a block of query rows and keeps them on chip; it
// streams tiles of keys and values through LDS, computes the score tile, updates
// each row's running max m, running sum l and unnormalised output o~ (both
// rescaled by exp(m_old - m_new)), and after the last tile writes O = o~ / l and
// lse = m + log l.  Causal tiles wholly above the diagonal are never loaded
// (section "Causal masks and FlashAttention-3").  Work is split over query rows
// across waves, so waves never exchange partial outputs (section "What
// FlashAttention-2 changed", point 3).
//
// gfx950 mapping.  Each wave owns 32*QT query rows.  The score tile is computed
// transposed, S^T = K Q^T, on 32x32 MFMA: the accumulator puts one query per lane
// column (lane L and lane L+32 share query L%32), so the row max and row sum are
// in-lane reductions plus a single exchange with the partner half-wave, and the
// rescale factor is a per-lane scalar.  The output is accumulated transposed too,
// O^T += V^T P^T, whose B operand is P^T taken straight from the score
// accumulator registers (c-layout k assignment), so P never leaves registers.
// Q^T stays in registers for the whole pass.  exp is v_exp_f32 (base 2) with
// scale*log2(e) folded into one FMA per score.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <typename T, int D, int BC, int NW, int QT>
struct FwdCfg {
  static constexpr int NT = 64 * NW;          // threads per workgroup
  static constexpr int BR = 32 * QT * NW;     // query rows per workgroup
  static constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte chunk
  static constexpr int LDR = D + VEC;         // LDS row stride (16-byte pad per row)
  static constexpr int CPR = D / VEC;         // 16-byte chunks per row
  static constexpr int CPT = BC * CPR / NT;   // chunks per thread per K (or V) tile
  static_assert(BC * CPR % NT == 0, "a K/V tile must split evenly over the threads");
  static_assert(BC % 32 == 0 && D % 32 == 0, "tiles are multiples of 32");
};

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* p, float a, float b, float c, float d) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  bf16x4_t v;
  v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
  *reinterpret_cast<bf16x4_t*>(p) = v;
}

template <typename T, int D, int BC, int NW, int QT>
__global__ __launch_bounds__(64 * NW) void fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    T* __restrict__ O, float* __restrict__ LSE, int Nmax, float scale, int causal, int nqb,
    SeqMap sm, int window) {
  using C = FwdCfg<T, D, BC, NW, QT>;
  using M = Mma<T>;
  typedef typename M::op_t op_t;
  constexpr int KPI = M::KPI, EPL = M::EPL;
  constexpr int NKK = D / KPI;  // instructions along d
  constexpr int NDT = D / 32;   // 32-wide dim tiles of O^T
  constexpr int NKS = BC / 32;  // 32-key sub-tiles of a K/V tile
  constexpr int NJ = 32 / KPI;  // instructions along 32 keys

  __shared__ __attribute__((aligned(16))) T Ks[BC * C::LDR];
  __shared__ __attribute__((aligned(16))) T Vs[BC * C::LDR];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / nqb;
  int qb = id - bh * nqb;
  if (causal) qb = nqb - 1 - qb;  // longest query blocks of a head start first
  int base, N;  // first row and length of this (batch, head)
  seq_rows(sm, bh, Nmax, base, N);
  const size_t head = (size_t)base * D;
  const T* Qh = Q + head;
  const T* Kh = K + head;
  const T* Vh = V + head;
  const int q0 = qb * C::BR;
  if (q0 >= N) return;  // a short sequence of a variable-length batch: no rows here
  const int qw = q0 + w * 32 * QT;  // first query row of this wave

  // Q^T as the B operand of S^T = K Q^T (natural k assignment), kept in registers.
  op_t qop[QT][NKK];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = qw + qt * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qop[qt][kk] = row < N ? M::load(Qh + (size_t)row * D + kk * KPI + g * EPL) : M::zero();
  }

  f32x16_t oacc[QT][NDT];
  float mrun[QT], lrun[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mrun[qt] = kNoMax;
    lrun[qt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[qt][dt] = zero16();
  }
  const float c = scale * kLog2e;

  const int q_last = min(q0 + C::BR, N) - 1;
  const int nkt = causal ? q_last / BC + 1 : (N + BC - 1) / BC;

  v16b kst[C::CPT], vst[C::CPT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int idx = tid + i * C::NT;
      const int r = idx / C::CPR, col = (idx % C::CPR) * C::VEC;
      const int key = kt * BC + r;
      if (key < N) {
        kst[i] = *reinterpret_cast<const v16b*>(Kh + (size_t)key * D + col);
        vst[i] = *reinterpret_cast<const v16b*>(Vh + (size_t)key * D + col);
      } else {
        kst[i] = v16b{0, 0, 0, 0};
        vst[i] = v16b{0, 0, 0, 0};
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int idx = tid + i * C::NT;
      const int r = idx / C::CPR, col = (idx % C::CPR) * C::VEC;
      *reinterpret_cast<v16b*>(Ks + r * C::LDR + col) = kst[i];
      *reinterpret_cast<v16b*>(Vs + r * C::LDR + col) = vst[i];
    }
  };

  // first key tile of the block's band (sliding window), else tile 0
  const int kt0 = window > 0 ? max(0, q0 - window + 1) / BC : 0;
  gload(kt0);
  for (int kt = kt0; kt < nkt; ++kt) {
    __syncthreads();  // every wave is done reading the previous tile
    sstore();
    __syncthreads();
    if (kt + 1 < nkt) gload(kt + 1);  // next tile's loads fly during this tile's math
    const int k0 = kt * BC;

    // S^T = K Q^T for this tile: NKS x QT accumulators of 32 keys x 32 queries.
    f32x16_t s[NKS][QT];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[ks][qt] = zero16();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const T* krow = Ks + (ks * 32 + l32) * C::LDR + g * EPL;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const op_t a = M::load(krow + kk * KPI);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) s[ks][qt] = M::mma(a, qop[qt][kk], s[ks][qt]);
      }
    }

    // Mask keys past the end and, on tiles that reach past this wave's first
    // query, keys above the diagonal.
    const bool need_mask = (k0 + BC > N) || (causal && k0 + BC - 1 > qw) ||
                           (window > 0 && k0 <= qw + 32 * QT - 1 - window);
    if (need_mask) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const int q = qw + qt * 32 + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + ks * 32 + crow(g, r);
            if (key >= N || (causal && key > q) || (window > 0 && key <= q - window))
              s[ks][qt][r] = -INFINITY;
          }
        }
    }

    // Online softmax update, one query per lane pair.
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = mrun[qt];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[ks][qt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float alpha = __builtin_amdgcn_exp2f((mrun[qt] - mx) * c);
      const float mc = mx * c;
      float rs = 0.0f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[ks][qt][r], c, -mc));
          s[ks][qt][r] = p;
          rs += p;
        }
      lrun[qt] = fmaf(lrun[qt], alpha, rs);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[qt][dt] *= alpha;
      mrun[qt] = mx;
    }

    // O^T += V^T P^T.  A = V^T gathered from LDS in the c-layout k order, B = P^T
    // from the score accumulators.
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        op_t pop[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) pop[qt] = M::from_acc(s[ks][qt], j * EPL);
        const T* vblk = Vs + (ks * 32) * C::LDR + l32;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const op_t a = M::gather(vblk + dt * 32, [&](int sl) { return crow(g, j * EPL + sl) * C::LDR; });
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) oacc[qt][dt] = M::mma(a, pop[qt], oacc[qt][dt]);
        }
      }
  }

  // Epilogue: combine the two half-wave partial sums, O = o~ / l, lse = m*scale + ln l.
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float l_tot = lrun[qt] + __shfl_xor(lrun[qt], 32);
    const int q = qw + qt * 32 + l32;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (q < N) {
      T* orow = O + head + (size_t)q * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const f32x16_t& a = oacc[qt][dt];
          store4<T>(orow + dt * 32 + 8 * rb + 4 * g, a[4 * rb] * inv, a[4 * rb + 1] * inv,
                    a[4 * rb + 2] * inv, a[4 * rb + 3] * inv);
        }
      if (g == 0)
        LSE[(size_t)base + q] = l_tot > 0.0f ? fmaf(mrun[qt], scale, logf(l_tot)) : -INFINITY;
    }
  }
}

template <typename T, int D, int BC, int NW, int QT>
static hipError_t launch_fwd_cfg(const FwdArgs& a) {
  using C = FwdCfg<T, D, BC, NW, QT>;
  const int nqb = (a.N + C::BR - 1) / C::BR;
  const long long grid = (long long)a.B * a.H * nqb;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  launch_begin();
  hipLaunchKernelGGL((fwd_kernel<T, D, BC, NW, QT>), dim3((unsigned)grid), dim3(C::NT), 0,
                     (hipStream_t)a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                     (T*)a.o, a.lse, a.N, a.scale, a.causal, nqb, SeqMap{a.cu_seqlens, a.B, a.T},
                     a.window);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.dtype == kBF16) {
    return launch_fwd_bf16(a);
  } else {
    if (a.d == 64) return launch_fwd_cfg<float, 64, 32, 4, 1>(a);
    if (a.d == 128) return launch_fwd_cfg<float, 128, 32, 4, 1>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
