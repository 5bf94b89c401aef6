// fa_bwd_dq_bf16.hip -- the bf16 dQ pass of the backward, tuned for gfx950.
//
// dQ_i = scale * sum_j dS_ij K_j with dS = P o (dP - D), P = exp(S - lse)
// ("FlashAttention and online softmax", ML Systems Lesson 4, "Backward pass:
// recompute instead of store", steps 1-4).  The dK/dV pass keeps keys stationary;
// summing its per-key-block dQ contributions would take one float atomic per key
// block per dQ element, and gfx950 retires about 3.4e11 such atomics per second,
// well below what the matrix cores need at this shape.  This pass instead keeps a
// block of 128 query rows stationary (32 per wave), like the forward, and streams
// K/V tiles, recomputing S and dP: three matrix products per tile and no atomics.
//
// Per 64-key tile, transposed products on 32x32 MFMA (queries on lane columns):
//   S^T  = K Q^T       A: K rows (natural LDS reads),  B: Q^T in registers
//   dP^T = V dO^T      A: V rows (natural LDS reads),  B: dO^T in registers
//   dS^T = P^T o (dP^T - D)  with P^T = 2^(S^T c - lse2): lse2 and D are per lane
//   dQ^T += K^T dS^T   A: K^T (transposed LDS reads),  B: dS^T from the registers
// K and V tiles are double buffered in LDS by global_load_lds_dwordx4, row-major
// with the chunk swizzle f(r) that keeps both natural and transposed reads free of
// bank conflicts.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct DqFast {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 32 * NW;  // query rows per workgroup
  static constexpr int BC = 64;       // keys per K/V tile
  static constexpr int CPR = D / 8;
  static constexpr int TILE = BC * D;
  static constexpr int LOADS = BC * CPR / 64 / NW;
  static_assert(BC * CPR % (64 * NW) == 0, "tile must split over the waves");
};

template <int D>
__device__ __forceinline__ int dq_swz(int r) {
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// PRE = true folds the backward's preprocess into this pass: each lane forms its own
// row's D = dO . O and lse * log2(e) (the same products and the same summation tree as
// bwd_pre_kernel, so the values are bit for bit those the preprocess would write), uses
// them, and writes them to the workspace vectors (padding rows: D = 0, +inf) for the
// dK/dV pass that runs next.  PRE = false reads them from the workspace.
template <int D, bool GEN, bool PRE>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, float* __restrict__ L2, float* __restrict__ Dvec,
    const __bf16* __restrict__ O, const float* __restrict__ LSE,
    __bf16* __restrict__ dQ, int Nmax, int Npad, float scale, int causal, int nqb, SeqMap sm_arg,
    int window_arg) {
  // GEN = false: dense tensors, no window; the general code folds away.
  const int window = GEN ? window_arg : 0;
  const SeqMap sm{GEN ? sm_arg.cu : nullptr, sm_arg.B, sm_arg.T};
  using C = DqFast<D>;
  constexpr int NKK = D / 16;
  constexpr int NDT = D / 32;
  constexpr int CPR = C::CPR;

  __shared__ __attribute__((aligned(1024))) __bf16 K0[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 K1[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 V0[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 V1[C::TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int g = lane >> 5, l32 = lane & 31;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  int bh = id / nqb, qb = id - bh * nqb;
  // Longest first, over groups of twice heavy_group's L2-sized count of units (capped at 8):
  // measured -0.3 to -0.6 % against heavy_group's own count on the long causal layer, at
  // N = 16384 and on the training step.
  if (causal) heavy_first(id, nqb, gridDim.x / nqb, GEN ? 1 : min(8, 2 * heavy_group(Nmax, D)), bh, qb);
  int base, N;  // first row and length of this (batch, head)
  seq_rows(sm, bh, Nmax, base, N);
  const size_t head = (size_t)base * D;
  const int q0 = qb * C::BR;
  if (q0 >= N) return;  // a short sequence of a variable-length batch: no rows here
  const int qw = q0 + w * 32;
  const int myq = qw + l32;

  // direct-load sources: slot s = r*CPR + p holds logical chunk p ^ f(r)
  int src_row[C::LOADS], src_col[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int slot = (w * C::LOADS + i) * 64 + lane;
    const int r = slot / CPR, p = slot % CPR;
    src_row[i] = r;
    src_col[i] = (p ^ dq_swz<D>(r)) * 8;
  }
  auto issue_tile = [&](int kt, __bf16* Kd, __bf16* Vd) {
    const int kbase = kt * C::BC;  // < N for every tile issued
    const __bf16* ks = K + head + (size_t)kbase * D;
    const __bf16* vs = V + head + (size_t)kbase * D;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      // keys past the end read the last row (masked later)
      const unsigned off = (unsigned)(min(src_row[i], N - 1 - kbase) * D + src_col[i]) * 2u;
      dma16(ks, off, Kd + (w * C::LOADS + i) * 512);
      dma16(vs, off, Vd + (w * C::LOADS + i) * 512);
    }
  };
  // natural A-operand reads: row ks*32 + l32, logical chunk 2*kk + g
  int nat[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) nat[kk] = l32 * D + (((2 * kk + g) ^ dq_swz<D>(l32)) << 3);
  // transposed reads of K (A of dQ^T = K^T dS^T): row 16j + 8h + 4(G>>1) + e,
  // column dt*32 + 16(G&1) + 4 q4
  const int G = lane >> 4, e4 = (lane >> 2) & 3, q4 = lane & 3;
  int trk[2][NDT];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int row = 8 * h + 4 * (G >> 1) + e4;
      const int col = dt * 32 + 16 * (G & 1) + 4 * q4;
      trk[h][dt] = row * D + (((col >> 3) ^ dq_swz<D>(row)) << 3) + (col & 7);
    }

  // Q^T and dO^T operands of this lane's query row, its lse (base 2) and D.
  bf16x8_t qop[NKK], gop[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    if (myq < N) {
      const int off = (myq - q0) * D + kk * 16 + g * 8;
      qop[kk] = *reinterpret_cast<const bf16x8_t*>(Q + head + (size_t)q0 * D + off);
      gop[kk] = *reinterpret_cast<const bf16x8_t*>(dO + head + (size_t)q0 * D + off);
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        qop[kk][t] = (__bf16)0.0f;
        gop[kk][t] = (__bf16)0.0f;
      }
    }
  }
  float lse2, dval;
  if constexpr (PRE) {
    // D: per 16-byte chunk p = 2 kk + g an fma chain over its 8 elements, then the
    // butterfly over chunks (p ^ 8, 4, 2 within the lane's chunks, p ^ 1 across the
    // half-waves): the order bwd_pre_kernel adds them in.
    float part[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      part[kk] = 0.0f;
      if (myq < N) {
        const int off = (myq - q0) * D + kk * 16 + g * 8;
        const bf16x8_t o8 = *reinterpret_cast<const bf16x8_t*>(O + head + (size_t)q0 * D + off);
#pragma unroll
        for (int t = 0; t < 8; ++t) part[kk] = fmaf((float)o8[t], (float)gop[kk][t], part[kk]);
      }
    }
#pragma unroll
    for (int x = NKK / 2; x > 0; x >>= 1) {
      float nxt[NKK];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) nxt[kk] = part[kk] + part[kk ^ x];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) part[kk] = nxt[kk];
    }
    dval = part[0] + __shfl_xor(part[0], 32);
    lse2 = myq < N ? LSE[(size_t)base + myq] * kLog2e : INFINITY;  // +inf past N: P = 0
    if (myq >= N) dval = 0.0f;
    if (g == 0 && myq < Npad) {
      Dvec[(size_t)bh * Npad + myq] = dval;
      L2[(size_t)bh * Npad + myq] = lse2;
    }
  } else {
    lse2 = L2[(size_t)bh * Npad + min(myq, Npad - 1)];  // +inf past N: P = 0
    dval = Dvec[(size_t)bh * Npad + min(myq, Npad - 1)];
  }

  f32x16_t acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = zero16();
  const float c = scale * kLog2e;
  const int q_last = min(q0 + C::BR, N) - 1;
  const int nkt = causal ? q_last / C::BC + 1 : (N + C::BC - 1) / C::BC;

  auto tile = [&](int kt, const __bf16* Kb, const __bf16* Vb, __bf16* Kn, __bf16* Vn) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile kt landed
    __syncthreads();                     // ... everyone's, and the other buffers are free
    if (kt + 1 < nkt) issue_tile(kt + 1, Kn, Vn);
    const int k0 = kt * C::BC;
    if (causal && k0 > qw + 31) return;  // tile wholly above this wave's rows
    if (window > 0 && k0 + C::BC - 1 <= qw - window) return;  // wholly below their band

    // The tile's two 32-key halves one after the other: half 1's products can run
    // while half 0's P and dS are computed, and only one half's S and dP are live.
    const bool need_mask = (k0 + C::BC > N) || (causal && k0 + C::BC - 1 > qw) ||
                           (window > 0 && k0 <= qw + 31 - window);
    // K and V operand reads run AHEAD d-steps in front of the products that use them,
    // so the LDS round trips overlap each other and the products.
    constexpr int AHEAD = NKK < 4 ? NKK : 2;
    bf16x8_t ak[NKK], av[NKK];
    auto read_kv_h = [&](int h, int kk) {
      ak[kk] = *reinterpret_cast<const bf16x8_t*>(Kb + h * 32 * D + nat[kk]);
      av[kk] = *reinterpret_cast<const bf16x8_t*>(Vb + h * 32 * D + nat[kk]);
    };
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f32x16_t s = zero16(), dp = zero16();
      auto read_kv = [&](int kk) { read_kv_h(ks, kk); };
      // Dense calls at d = 128: wave priority 1 for the S and dP products, 2 for the dQ
      // products, 0 for the softmax between them, so that of two ready waves on a SIMD the
      // one feeding the matrix cores issues first (measured: the windowed kernel and d = 64
      // are faster without).
      constexpr bool kPrio = !GEN && D == 128;
      if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
      // (the second half's first operands were read under the first half's dQ products)
      if (ks == 0) {
#pragma unroll
        for (int kk = 0; kk < AHEAD; ++kk) read_kv(kk);
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        __builtin_amdgcn_sched_barrier(0);
        if (kk + AHEAD < NKK) read_kv(kk + AHEAD);
        __builtin_amdgcn_sched_barrier(0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[kk], qop[kk], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kk], gop[kk], dp, 0, 0, 0);
      }
      if constexpr (kPrio) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
      }
      // K^T operands of this half's dQ product (transposed reads).  At d = 64 they are
      // read here, so their LDS round trips run under the softmax below; at d = 128 the
      // registers for that are not there, and each is read just before its product.
      auto read_kt = [&](int j, int dt) {
        const __bf16* kb = Kb + (ks * 32 + j * 16) * D;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(kb + trk[0][dt]));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(kb + trk[1][dt]));
        const bf16x4_t x = __builtin_bit_cast(bf16x4_t, lo), y = __builtin_bit_cast(bf16x4_t, hi);
        bf16x8_t a;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          a[t] = x[t];
          a[4 + t] = y[t];
        }
        return a;
      };
      constexpr bool kEarly = D == 64;
      bf16x8_t kt_op[2][NDT];
      if constexpr (kEarly) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) kt_op[j][dt] = read_kt(j, dt);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (need_mask) {  // keys past the end, above the diagonal or below the window: P = 0
        const int hi = causal ? min(myq, N - 1) : N - 1;
        const int lo = window > 0 ? myq - window + 1 : 0;
        mask_rows<GEN>(s, g, k0 + ks * 32, lo, hi);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lse2));
        dp[r] = p * (dp[r] - dval);
      }
      // dQ^T += K^T dS^T over this half's 32 keys (2 steps of 16, c-layout key order).
      if constexpr (kPrio) __builtin_amdgcn_s_setprio(2);
      // The second half's first K and V operands are read here, so that its S and dP
      // products need not start on an LDS round trip (the compiler places the reads among
      // these products; measured -1.0 to -1.7 % at d = 128, against -0.5 % slower when
      // they are pinned before the first of them).
      if (ks == 0) {
#pragma unroll
        for (int kk = 0; kk < AHEAD; ++kk) read_kv_h(1, kk);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8_t b;
#pragma unroll
        for (int t = 0; t < 8; ++t) b[t] = (__bf16)dp[8 * j + t];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kEarly ? kt_op[j][dt] : read_kt(j, dt), b,
                                                            acc[dt], 0, 0, 0);
      }
    }
  };

  // first key tile of the block's band (sliding window), else tile 0
  const int kt0 = window > 0 ? max(0, q0 - window + 1) / C::BC : 0;
  issue_tile(kt0, K0, V0);
  for (int kt = kt0; kt < nkt; kt += 2) {
    tile(kt, K0, V0, K1, V1);
    if (kt + 1 < nkt) tile(kt + 1, K1, V1, K0, V0);
  }

  // dQ = scale * acc: lane = query row, registers = dims 8 rb + 4 g + 0..3 of tile dt.
  if (myq < N) {
    // wave-uniform block base plus a 32-bit lane offset (no 64-bit value kept live)
    __bf16* row = dQ + head + (size_t)q0 * D + (myq - q0) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        bf16x4_t v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (__bf16)(acc[dt][4 * rb + t] * scale);
        *reinterpret_cast<bf16x4_t*>(row + dt * 32 + 8 * rb + 4 * g) = v;
      }
  }
}

template <int D, bool GEN, bool PRE>
static hipError_t launch_dq_bf16_d(const BwdArgs& a) {
  using C = DqFast<D>;
  const int nqb = (a.N + C::BR - 1) / C::BR;
  const long long grid = (long long)a.B * a.H * nqb;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  launch_begin();
  hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, GEN, PRE>), dim3((unsigned)grid), dim3(C::NT), 0,
                     (hipStream_t)a.stream, (const __bf16*)a.q, (const __bf16*)a.k,
                     (const __bf16*)a.v, (const __bf16*)a.dout, a.L2, a.Dvec,
                     (const __bf16*)a.o, a.lse, (__bf16*)a.dq, a.N, a.Npad, a.scale, a.causal,
                     nqb, SeqMap{a.cu_seqlens, a.B, a.T}, a.window);
  return hipGetLastError();
}

template <bool PRE>
static hipError_t launch_dq_bf16(const BwdArgs& a) {
  const bool gen = a.cu_seqlens != nullptr || a.window > 0;
  if (a.d == 64) return gen ? launch_dq_bf16_d<64, true, PRE>(a) : launch_dq_bf16_d<64, false, PRE>(a);
  if (a.d == 128) return gen ? launch_dq_bf16_d<128, true, PRE>(a) : launch_dq_bf16_d<128, false, PRE>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_bf16(const BwdArgs& a) { return launch_dq_bf16<false>(a); }
hipError_t launch_bwd_dq_pre_bf16(const BwdArgs& a) { return launch_dq_bf16<true>(a); }

}  // namespace fa
