// fa_fwd_bf16.hip -- the bf16 forward kernel tuned for gfx950.
//
// Same method as fa_fwd.hip ("FlashAttention and online softmax", ML Systems
// Lesson 4, the tiled forward pass under "The online softmax theorem"), with the
// data movement built around CDNA4:
//
// * K/V tiles go global -> LDS with global_load_lds_dwordx4 (no staging VGPRs),
//   double buffered: tile j+1 is in flight while tile j is computed.
// * LDS has 64 banks of 4 bytes.  K is stored chunk-major inside 16-row groups
//   (16-byte chunk c of row r at ((r/16)*CPR + c)*16 + r%16 chunks), so the 16
//   lanes of a 128-bit read phase, which read 16 consecutive rows at one chunk,
//   touch 256 contiguous bytes.  V is stored row-major with the 16-byte chunk index
//   XOR-swizzled by the row, and read transposed with ds_read_b64_tr_b16: within
//   each 16-lane group, lane i receives element i%4 of the 8 bytes loaded by lanes
//   4e + i/4, e = 0..3.  Each group then reads 4 rows x 32 bytes, and the swizzle
//   puts the 4 rows of a 32-lane phase on disjoint banks.
// * The running max used as the softmax reference is only moved when a tile's max
//   exceeds it by more than 2^8 in the exp2 domain.  The online-softmax theorem's
//   exactness needs only that l and o~ share one reference value, which stays
//   true; exponents are bounded by 2^8 instead of 1, far inside fp32 and bf16
//   range.  The rescale of o~ (64 multiplies per lane) is thereby skipped on
//   almost every tile.
// * Waves whose 32 query rows all lie above a diagonal tile skip its math.
// * The P tile enters the PV product rounded to bf16, so O is normalised by the sum
//   of those same rounded weights (v_dot2_f32_bf16 against ones): O stays an exact
//   convex combination of V rows and D = dO . O in the backward matches the P it
//   recomputes, even for rows whose softmax is nearly one-hot.  lse keeps the sum
//   of the unrounded weights.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// Bound on a lane's sum of weights in one tile before the reference must move (see the
// softmax in the tile loop); far inside fp32 and bf16 range.
constexpr float kWeightBound = 1048576.0f;  // 2^20

// d = 128: tiles of 32 keys, so that a wave fits 168 registers and three waves share each
// SIMD (three workgroups per CU): two K operand reads in flight ahead of the products, V
// operands read where the products need them.  d = 64: tiles of 64 keys, three waves per
// SIMD already; four K reads ahead, and the V operands of a tile's first 16 keys read before
// its softmax.
template <int D>
struct FwdFast {
  static constexpr int NW = 4;             // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 32 * NW;       // query rows per workgroup
  static constexpr int BC = D == 128 ? 32 : 64;  // keys per K/V tile
  static constexpr int NKS = BC / 32;      // 32-key halves of a tile
  static constexpr int OCC = D == 128 ? 3 : 2;   // waves per SIMD the registers are sized for
  static constexpr int AHEAD = D == 128 ? 2 : 4; // K operand reads in flight (d-steps)
  static constexpr bool EARLY_V = D == 64;       // first V operands read before the softmax
  // Wave priorities (s_setprio) of the S products and of the PV products; the softmax runs
  // at 0.  PRIO_GEN: whether the general (windowed / variable-length) kernel sets them too.
  static constexpr int PRIO_S = 1;
  static constexpr int PRIO_PV = 2;
  static constexpr bool PRIO_GEN = D == 128;
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int TILE = BC * D;      // elements per K (or V) tile
  static constexpr int LOADS = BC * CPR / 64 / NW;  // direct loads per wave per tile
  static_assert(BC * CPR % (64 * NW) == 0, "tile must split over the waves");
  static constexpr float kRescaleLog2 = 8.0f;  // move the reference max past 2^8 growth
};

// LDS chunk slot of K's 16-byte chunk (r, c): chunk-major inside 16-row groups.
template <int D>
__device__ __forceinline__ int k_slot(int r, int c) {
  return ((r >> 4) * (D / 8) + c) * 16 + (r & 15);
}
// V's swizzle: chunk c of row r is stored at chunk c ^ vswz(r) of that row.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

template <int D, bool GEN>
__global__ __launch_bounds__(256, FwdFast<D>::OCC) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int Nmax, float scale, int causal, int nqb,
    SeqMap sm_arg, int window_arg) {
  // GEN = false: dense tensors, no window; the general code folds away.
  const int window = GEN ? window_arg : 0;
  const SeqMap sm{GEN ? sm_arg.cu : nullptr, sm_arg.B, sm_arg.T};
  using C = FwdFast<D>;
  constexpr int NKK = D / 16;  // MFMA steps along d
  constexpr int NDT = D / 32;  // 32-wide dim tiles of O^T
  constexpr int CPR = C::CPR;

  // Two K and two V buffers as distinct objects, each named statically in the
  // (twice unrolled) tile loop, so the compiler can see that reading one buffer
  // does not depend on the direct loads still landing in the other.
  __shared__ __attribute__((aligned(1024))) __bf16 K0[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 K1[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 V0[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 V1[C::TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int g = lane >> 5, l32 = lane & 31;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  int bh = id / nqb, qb = id - bh * nqb;
  // Longest first, over groups of units twice heavy_group's L2-sized count (capped at 8): with
  // three workgroups per CU an XCD runs half again as many blocks at once as the one- and
  // two-workgroup passes, and the larger groups balance them better (measured against
  // heavy_group's own count: long causal layer -2.4 %, N = 16384 -0.9 %, training step
  // -1.6 %; four times it was 21 % slower at N = 16384).
  if (causal) heavy_first(id, nqb, gridDim.x / nqb, GEN ? 1 : min(8, 2 * heavy_group(Nmax, D)), bh, qb);
  int base, N;  // first row and length of this (batch, head)
  seq_rows(sm, bh, Nmax, base, N);
  const size_t head = (size_t)base * D;
  const __bf16* Kh = K + head;
  const __bf16* Vh = V + head;
  const int q0 = qb * C::BR;
  if (q0 >= N) return;  // a short sequence of a variable-length batch: no rows here
  const int qw = q0 + w * 32;
  const int myq = qw + l32;

  // --- per-lane address pieces -------------------------------------------------
  // Direct-load sources: wave w's load i fills chunk slots (w*LOADS + i)*64 + lane.
  int k_src_row[C::LOADS], k_src_col[C::LOADS], v_src_row[C::LOADS], v_src_col[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int slot = (w * C::LOADS + i) * 64 + lane;
    // K: slot -> (r, c) inverse of k_slot
    const int grp = slot / (CPR * 16), within = slot % (CPR * 16);
    k_src_row[i] = grp * 16 + (within & 15);
    k_src_col[i] = (within >> 4) * 8;
    // V: row-major, physical chunk p holds logical chunk p ^ vswz(r)
    const int r = slot / CPR, p = slot % CPR;
    v_src_row[i] = r;
    v_src_col[i] = (p ^ vswz<D>(r)) * 8;
  }
  // The same pieces as offsets from a tile's first row: a load is then a wave-uniform
  // tile base plus a fixed per-lane offset, with no per-tile address arithmetic.
  unsigned k_off[C::LOADS], v_off[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    k_off[i] = k_src_row[i] * D + k_src_col[i];
    v_off[i] = v_src_row[i] * D + v_src_col[i];
  }
  auto issue_tile = [&](int kt, __bf16* Kd, __bf16* Vd) {
    const int kbase = kt * C::BC;
    const __bf16* ks = Kh + (size_t)kbase * D;
    const __bf16* vs = Vh + (size_t)kbase * D;
    if (kbase + C::BC <= N) {
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        dma16(ks, k_off[i] * 2u, Kd + (w * C::LOADS + i) * 64 * 8);
        dma16(vs, v_off[i] * 2u, Vd + (w * C::LOADS + i) * 64 * 8);
      }
    } else {  // the tile runs past the end: rows past it read the last row (masked later)
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        const int kr = min(k_src_row[i], N - 1 - kbase);
        const int vr = min(v_src_row[i], N - 1 - kbase);
        dma16(ks, (unsigned)(kr * D + k_src_col[i]) * 2u, Kd + (w * C::LOADS + i) * 64 * 8);
        dma16(vs, (unsigned)(vr * D + v_src_col[i]) * 2u, Vd + (w * C::LOADS + i) * 64 * 8);
      }
    }
  };
  // K operand read (A of S^T = K Q^T): row ks*32 + l32, chunk 2*kk + g.
  const int k_rd = k_slot<D>(l32, g) * 8;  // + ks*32 rows and kk*2 chunks are immediates
  // V^T operand via transposed reads: lane (G = lane/16, e = lane%16/4, q = lane%4)
  // loads 8 bytes of row rbase + 4*(G>>1) + e at column dt*32 + 16*(G&1) + 4*q.
  const int G = lane >> 4, e4 = (lane >> 2) & 3, q4 = lane & 3;
  const int v_row = 4 * (G >> 1) + e4;
  int v_rd[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int col = dt * 32 + 16 * (G & 1) + 4 * q4;
    v_rd[dt] = v_row * D + (((col >> 3) ^ vswz<D>(v_row)) << 3) + (col & 7);
  }

  // --- Q^T operands in registers ---------------------------------------------------
  bf16x8_t qop[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    if (myq < N) {
      qop[kk] = *reinterpret_cast<const bf16x8_t*>(Q + head + (size_t)myq * D + kk * 16 + g * 8);
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) qop[kk][s] = (__bf16)0.0f;
    }
  }

  f32x16_t oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = zero16();
  float mref = kNoMax, lsum = 0.0f, lsum_bf = 0.0f;
  bool first = true;  // no reference yet: the first tile a wave computes takes the max
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones2 = {(__bf16)1.0f, (__bf16)1.0f};
  const float c = scale * kLog2e;
  const float grow = C::kRescaleLog2 / c;  // allowed growth of the raw max before a rescale

  const int q_last = min(q0 + C::BR, N) - 1;
  const int nkt = causal ? q_last / C::BC + 1 : (N + C::BC - 1) / C::BC;

  auto tile = [&](int kt, const __bf16* Kb, const __bf16* Vb, __bf16* Kn, __bf16* Vn) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile kt landed
    __syncthreads();                     // ... everyone's, and the other buffers are free
    if (kt + 1 < nkt) issue_tile(kt + 1, Kn, Vn);
    const int k0 = kt * C::BC;
    if (causal && k0 > qw + 31) return;  // tile wholly above this wave's rows
    if (window > 0 && k0 + C::BC - 1 <= qw - window) return;  // wholly below their band
    // S^T = K Q^T (a lambda: the rare path below computes it a second time)
    constexpr int NKS = C::NKS;
    // K operand reads run AHEAD d-steps in front of the products that use them, so
    // the LDS round trips overlap each other and the products instead of alternating
    // with them (at most 15 LDS reads may be outstanding for a counted wait).
    constexpr int AHEAD = C::AHEAD < NKK ? C::AHEAD : NKK;
    const bool need_mask = (k0 + C::BC > N) || (causal && k0 + C::BC - 1 > qw) ||
                           (window > 0 && k0 <= qw + 31 - window);
    f32x16_t s[NKS];
    auto scores = [&]() {
      bf16x8_t ka[NKK][NKS];
      auto read_k = [&](int kk) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          ka[kk][ks] = *reinterpret_cast<const bf16x8_t*>(
              Kb + k_rd + (ks * 2 * CPR * 16 + kk * 2 * 16) * 8);
      };
      // Wave priority raised while the wave issues its products, 0 during its softmax: when
      // several waves of a SIMD are ready, the ones feeding the matrix cores go first, and
      // the others' vector work fills in, which pushes them into different phases.  At
      // The PV products rank above the S products; at d = 128 (three waves a SIMD) the
      // general kernel uses the same order, at d = 64 its flat priority measured faster.
      if constexpr (!GEN || C::PRIO_GEN) __builtin_amdgcn_s_setprio(C::PRIO_S);
#pragma unroll
      for (int kk = 0; kk < AHEAD; ++kk) read_k(kk);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) s[ks] = zero16();
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        __builtin_amdgcn_sched_barrier(0);
        if (kk + AHEAD < NKK) read_k(kk + AHEAD);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          s[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk][ks], qop[kk], s[ks], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!GEN || C::PRIO_GEN) __builtin_amdgcn_s_setprio(0);
      if (need_mask) {  // keys past the end, above the diagonal or below the window
        const int hi = causal ? min(myq, N - 1) : N - 1;
        const int lo = window > 0 ? myq - window + 1 : 0;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) mask_rows<GEN>(s[ks], g, k0 + ks * 32, lo, hi);
      }
    };
    scores();

    // V^T operand of keys ks*32 + j*16 .. +15 for dim tile dt (two transposed reads).
    auto read_v = [&](int ks, int j, int dt) -> bf16x8_t {
      const __bf16* base = Vb + v_rd[dt] + (ks * 32 + j * 16) * D;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(base));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(base + 8 * D));
      bf16x8_t a;
      const bf16x4_t lob = __builtin_bit_cast(bf16x4_t, lo), hib = __builtin_bit_cast(bf16x4_t, hi);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a[t] = lob[t];
        a[4 + t] = hib[t];
      }
      return a;
    };
    // At d = 64 the operands of the tile's first 16 keys are read before the softmax, so
    // that their LDS latency passes under it and the PV products can start on its last
    // weight (at d = 128 the third wave of each SIMD hides that latency, and the registers
    // are needed for it).
    bf16x8_t vfirst[C::EARLY_V ? NDT : 1];
    if constexpr (C::EARLY_V) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vfirst[dt] = read_v(0, 0, dt);
      __builtin_amdgcn_sched_barrier(0);
    }

    // Online softmax against the lazily moved reference mref: p = 2^(s*c - mref*c).
    // The theorem's exactness needs only one common reference for l and o~, and the
    // reference only has to keep the weights bounded.  So after the first tile the
    // weights are formed against the current reference straight away, and the tile's
    // sum of weights per lane bounds every one of them: while no lane's sum exceeds
    // 2^20 nothing needs to move.  Otherwise (a score beyond the reference by more than
    // about 15 in the exp2 domain, or the first tile) the scores' max moves the
    // reference and the weights are formed again.  The scores for that come from
    // registers of their own at d = 64; at d = 128, where those registers would cost
    // more, the weights overwrite the scores and the rare path computes the scores
    // again from the K tile still in LDS.  The first tile and the rare case share one
    // copy of the reference move; with two, the compiler copied the weights between
    // register sets on every tile where the paths joined.
    constexpr bool kKeepScores = D == 64;
    f32x16_t pst[kKeepScores ? NKS : 1];
    auto P = [&](int ks) -> f32x16_t& {
      if constexpr (kKeepScores) return pst[ks];
      else return s[ks];
    };
    float t = 0.0f;
    bool again = first;
    if (!first) {
      const float mc = mref * c;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          P(ks)[r] = __builtin_amdgcn_exp2f(fmaf(s[ks][r], c, -mc));
          t += P(ks)[r];
        }
      again = __builtin_amdgcn_ballot_w64(!(t <= kWeightBound)) != 0;  // wave-uniform, rare
      if constexpr (!kKeepScores) {
        if (again) scores();
      }
    }
    if (again) {
      first = false;
      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int ks = 1; ks < NKS; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[ks][r]);
      {  // the other half of the wave holds the other keys of the same query columns
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const bool move = mx > mref + grow;
      if (__builtin_amdgcn_ballot_w64(move)) {
        const float mnew = move ? mx : mref;
        const float alpha = __builtin_amdgcn_exp2f((mref - mnew) * c);
        lsum *= alpha;
        lsum_bf *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
        mref = mnew;
      }
      const float mc = mref * c;
      t = 0.0f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          P(ks)[r] = __builtin_amdgcn_exp2f(fmaf(s[ks][r], c, -mc));
          t += P(ks)[r];
        }
    }
    lsum += t;

    // O^T += V^T P^T
    if constexpr (!GEN || C::PRIO_GEN) __builtin_amdgcn_s_setprio(C::PRIO_PV);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8_t pb;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) pb[sl] = (__bf16)P(ks)[j * 8 + sl];
        lsum_bf = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), ones2, lsum_bf, false);
        lsum_bf = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 2, 3), ones2, lsum_bf, false);
        lsum_bf = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 4, 5), ones2, lsum_bf, false);
        lsum_bf = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 6, 7), ones2, lsum_bf, false);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          bf16x8_t a;
          if constexpr (C::EARLY_V) a = (ks == 0 && j == 0) ? vfirst[dt] : read_v(ks, j, dt);
          else a = read_v(ks, j, dt);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[dt], 0, 0, 0);
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

  // Epilogue: O = o~ / l (l of the rounded weights), lse = mref*scale + ln l.
  const float l_tot = lsum + __shfl_xor(lsum, 32);
  const float lb_tot = lsum_bf + __shfl_xor(lsum_bf, 32);
  const float inv = lb_tot > 0.0f ? 1.0f / lb_tot : 0.0f;
  if (myq < N) {
    __bf16* orow = O + head + (size_t)myq * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        bf16x4_t v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (__bf16)(oacc[dt][4 * rb + t] * inv);
        *reinterpret_cast<bf16x4_t*>(orow + dt * 32 + 8 * rb + 4 * g) = v;
      }
    if (g == 0) LSE[(size_t)base + myq] = l_tot > 0.0f ? fmaf(mref, scale, logf(l_tot)) : -INFINITY;
  }
}

template <int D, bool GEN>
static hipError_t launch_fwd_bf16_d(const FwdArgs& a) {
  using C = FwdFast<D>;
  const int nqb = (a.N + C::BR - 1) / C::BR;
  const long long grid = (long long)a.B * a.H * nqb;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  launch_begin();
  hipLaunchKernelGGL((fwd_bf16_kernel<D, GEN>), dim3((unsigned)grid), dim3(C::NT), 0,
                     (hipStream_t)a.stream, (const __bf16*)a.q, (const __bf16*)a.k,
                     (const __bf16*)a.v, (__bf16*)a.o, a.lse, a.N, a.scale, a.causal, nqb,
                     SeqMap{a.cu_seqlens, a.B, a.T}, a.window);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  const bool gen = a.cu_seqlens != nullptr || a.window > 0;
  if (a.d == 64) return gen ? launch_fwd_bf16_d<64, true>(a) : launch_fwd_bf16_d<64, false>(a);
  if (a.d == 128) return gen ? launch_fwd_bf16_d<128, true>(a) : launch_fwd_bf16_d<128, false>(a);
  return hipErrorInvalidValue;
}

}  // namespace fa
