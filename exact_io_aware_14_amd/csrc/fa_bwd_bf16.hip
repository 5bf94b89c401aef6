// fa_bwd_bf16.hip -- the bf16 dK/dV pass of the backward, tuned for gfx950.
//
// Method ("FlashAttention and online softmax", ML Systems Lesson 4, "Backward pass:
// recompute instead of store"): one workgroup at a time per block of keys (32 per wave at
// d = 128, two blocks of 32 per wave at d = 64), K_j and V_j in registers, dK_j and dV_j
// accumulated in registers, query tiles of 32 rows streamed; per tile
//   S = Q_i K_j^T, P = exp2(S*scale*log2e - lse_i*log2e),  dP = dO_i V_j^T,
//   dS = P o (dP - D_i),  dV_j += P^T dO_i,  dK_j += dS^T Q_i.
// dQ is computed by its own query-stationary pass (fa_bwd_dq_bf16.hip), which
// avoids one float atomic per key block per dQ element.
//
// Data movement for CDNA4:
// * Q_i, dO_i and the tile's lse/D values go global -> LDS by global_load_lds_dwordx4,
//   in four rotating buffer sets: tile i+2 lands while tiles i-1, i and i+1 are read.
// * Q and dO live in LDS row-major with the 16-byte chunk index XOR-swizzled by
//   f(r).  The same f makes both reads conflict-free on 64 banks: the natural
//   128-bit reads of 16 consecutive rows at one chunk (A operands of S and dP), and
//   the transposed ds_read_b64_tr_b16 reads of 4 rows x 32 bytes per 16-lane group
//   (B operands of dV = P^T dO and dK = dS^T Q).
// * S = Q K^T and dP = dO V^T put keys on the lane columns of the accumulators, so
//   P^T and dS^T feed dV and dK as A operands straight from registers.
// * One wave per SIMD (K, V, dK and dV alone hold 192 registers per lane at
//   d = 128, and as many for the two key blocks of a wave at d = 64, all in AGPRs), so
//   the overlap comes from inside the wave: the loop is
//   software pipelined.  Step i runs tile i's S products from Q rows already in
//   AGPRs, with the step's LDS reads (tile i-1's dO and Q transposed, tile i's lse and
//   D) under them; then its dP products, with most of P = 2^(S*scale*log2e - lse2) on
//   the vector ALUs under those; then tile i-1's dV/dK products alternate with the
//   rest of tile i's softmax (dS, and both kept as bf16 for the next step) and with
//   the reads of tile i+1's rows into AGPRs.
// * Dense calls run one workgroup per CU, each looping over its blocks of keys (a
//   block's K and V rows are staged in LDS by direct loads and read into AGPRs from
//   there).  A workgroup stages its next block's rows while it finishes the current
//   one, so a block starts without a round trip to HBM and without a new dispatch.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct BwdFast {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  // 32-key blocks per wave: at d = 64, K, V, dK and dV of two blocks fit the registers
  // that one block takes at d = 128, and every Q/dO operand read from LDS then feeds
  // the products of both.
  static constexpr int KB = D == 64 ? 2 : 1;
  static constexpr int BKV = 32 * KB * NW;  // keys per workgroup
  static constexpr int BQ = 32;        // query rows per streamed tile (== kRowPad)
  static constexpr int CPR = D / 8;    // 16-byte chunks per row
  static constexpr int QTILE = BQ * D;
  static constexpr int QLOADS = BQ * CPR / 64 / NW;  // direct loads per wave per Q tile
  static constexpr int NDT = D / 32;
  static_assert(BQ == kRowPad, "query tiles are the padded row unit");
  static_assert(BQ * CPR % (64 * NW) == 0, "tiles split over waves");
};

// Chunk swizzle of the Q and dO tiles (see the file comment).
template <int D>
__device__ __forceinline__ int bswz(int r) {
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// Swizzle of the epilogue's [column][key] transpose (4-key chunks XOR-ed by a function
// of the column): conflict-free on 64 banks both for the 8-byte writes in the accumulator
// layout (32 consecutive columns, one chunk) and for the transposing reads (4 columns x 4
// chunks per 16-lane group, two groups 8 columns apart per half-wave).
template <int D>
__device__ __forceinline__ int epi_swz(int col) {
  if (D == 128) {  // 4 columns per 256-byte bank row: swap bits 1 and 2 of col / 4
    const int x = (col >> 2) & 7;
    return (x & 1) | (((x >> 1) & 1) << 2) | (((x >> 2) & 1) << 1);
  }
  const int x = (col >> 1) & 15;  // 2 columns per bank row: bits 0,1,2,3 -> 2,0,3,1
  return ((x & 1) << 2) | ((x >> 1) & 1) | (((x >> 2) & 1) << 3) | (((x >> 3) & 1) << 1);
}

__device__ __forceinline__ bf16x8_t tr_pair(const __bf16* lo, const __bf16* hi) {
  const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)lo);
  const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)hi);
  const bf16x4_t x = __builtin_bit_cast(bf16x4_t, a), y = __builtin_bit_cast(bf16x4_t, b);
  bf16x8_t r;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    r[t] = x[t];
    r[4 + t] = y[t];
  }
  return r;
}

// Query tiles qt0 .. nqt-1 that see a block of keys k0 .. k0+BKV-1 of a sequence of n
// rows: causal rows before k0 see none of its keys, and in a window rows past the last
// key's band see none.
template <int BKV, int BQ>
__device__ __forceinline__ void key_block_tiles(int n, int k0, int causal, int window, int& qt0, int& nqt) {
  nqt = (n + BQ - 1) / BQ;
  qt0 = causal ? k0 / BQ : 0;
  if (window > 0) nqt = min(nqt, (k0 + BKV - 1 + window - 1) / BQ + 1);
}

// The plan of a variable-length or windowed dK/dV launch, built on the device from the
// sequence table by one workgroup right before it.  Blocks of keys (id = unit * nkb + key
// block) that hold keys are split into 8 contiguous id ranges of about equal cost (steps
// plus a fixed cost per block), one per XCD, so that a unit's blocks share an L2; each
// range is sorted by steps, most first, so that the workgroups of an XCD, taking its
// list in rounds, end close together.  Layout: plan[x] = start of XCD x's list,
// plan[8] = end of the last, ids from plan[kPlanHead] on.
constexpr int kPlanThreads = 1024;
constexpr int kPlanBins = 1024;    // steps classes of the sort (steps >> shift)
constexpr int kPlanFix = 3;        // a block's prologue and stores, in steps
constexpr int kPlanCache = 16384;  // blocks whose steps are kept in LDS between the passes
static_assert(kPlanHead >= 9, "plan header");

template <int BKV, int BQ>
__global__ __launch_bounds__(kPlanThreads) void bwd_plan_kernel(SeqMap sm, int Nmax, int causal, int window,
                                                               int nkb, int total, int* __restrict__ plan) {
  constexpr int NWV = kPlanThreads / 64;
  __shared__ long long wsum[NWV];
  __shared__ int bins[8 * kPlanBins];
  __shared__ unsigned short cache[kPlanCache];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  // Inclusive prefix sum over the workgroup's threads (within each wave by shuffles, then
  // over the waves' sums); `all` receives the total.
  auto scan = [&](long long v, long long& all) -> long long {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long a = __shfl_up(v, off, 64);
      if (lane >= off) v += a;
    }
    if (lane == 63) wsum[wv] = v;
    __syncthreads();
    long long before = 0;
    all = 0;
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
      const long long x = wsum[i];
      before += i < wv ? x : 0;
      all += x;
    }
    __syncthreads();  // wsum is free for the next scan
    return v + before;
  };
  // Each thread walks a contiguous run of ids; a run spans few units, whose length it keeps.
  // The first pass keeps each block's steps in LDS (when they fit) for the other two.
  const int seg = total / kPlanThreads + (total % kPlanThreads != 0);
  const int i0 = min(t * seg, total), i1 = min(i0 + seg, total);
  const int smax = (Nmax + BQ - 1) / BQ;
  const bool cached = total <= kPlanCache && smax < 65536;
  int unit = -1, n = 0;
  auto steps = [&](int id) -> int {  // 0: no keys in this block
    const int u = id / nkb, kb = id - u * nkb;
    if (u != unit) {
      int base;
      seq_rows(sm, u, Nmax, base, n);
      unit = u;
    }
    if (kb * BKV >= n) return 0;
    int qt0, nqt;
    key_block_tiles<BKV, BQ>(n, kb * BKV, causal, window, qt0, nqt);
    return nqt - qt0;
  };
  auto steps_again = [&](int id) -> int { return cached ? (int)cache[id] : steps(id); };
  int shift = 0;
  while ((smax >> shift) >= kPlanBins) ++shift;
  auto bin_of = [&](int st) { return kPlanBins - 1 - min(st >> shift, kPlanBins - 1); };

  for (int i = t; i < 8 * kPlanBins; i += kPlanThreads) bins[i] = 0;
  long long mine = 0;
  for (int id = i0; id < i1; ++id) {
    const int st = steps(id);
    if (cached) cache[id] = (unsigned short)st;
    if (st > 0) mine += st + kPlanFix;
  }
  long long ctot;
  const long long incl = scan(mine, ctot);  // (its barriers also order the zeroed bins)
  // XCD of a block: the eighth of the total cost that holds the block's midpoint (in
  // double precision: the same rounding in both passes that use it, and no 64-bit division).
  const double per = ctot > 0 ? 4.0 / (double)ctot : 0.0;
  auto xcd_of = [&](long long p, int cost) -> int {
    return min(7, (int)((double)(2 * p + cost) * per));
  };
  long long p = incl - mine;
  for (int id = i0; id < i1; ++id) {
    const int st = steps_again(id);
    if (st > 0) {
      atomicAdd(&bins[xcd_of(p, st + kPlanFix) * kPlanBins + bin_of(st)], 1);
      p += st + kPlanFix;
    }
  }
  __syncthreads();
  // Counts -> list positions: XCD-major, and within an XCD the most steps first.
  constexpr int PER = 8 * kPlanBins / kPlanThreads;
  int cnt[PER], sum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    cnt[j] = bins[t * PER + j];
    sum += cnt[j];
  }
  long long count;
  int run = (int)(scan(sum, count) - sum);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    bins[t * PER + j] = run;
    run += cnt[j];
  }
  __syncthreads();
  if (t < 8) plan[t] = bins[t * kPlanBins];
  if (t == 8) plan[8] = (int)count;
  __syncthreads();
  p = incl - mine;
  for (int id = i0; id < i1; ++id) {
    const int st = steps_again(id);
    if (st > 0) {
      const int at = atomicAdd(&bins[xcd_of(p, st + kPlanFix) * kPlanBins + bin_of(st)], 1);
      plan[kPlanHead + at] = id;
      p += st + kPlanFix;
    }
  }
}

template <int D, bool GEN>
__global__ __launch_bounds__(256) void bwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dvec,
    __bf16* __restrict__ dK, __bf16* __restrict__ dV, int Nmax, int Npad, float scale, int causal,
    int nkb, int total, SeqMap sm_arg, int window_arg, const int* __restrict__ plan) {
  // GEN = false: dense tensors, no window; the general code folds away.
  const int window = GEN ? window_arg : 0;
  const SeqMap sm{GEN ? sm_arg.cu : nullptr, sm_arg.B, sm_arg.T};
  using C = BwdFast<D>;
  constexpr int NKK = D / 16;
  constexpr int NDT = C::NDT;
  constexpr int CPR = C::CPR;

  // Four sets of Q, dO, lse and D tile buffers, each named statically in the (four
  // times unrolled) step loop: tile t+2 lands while tiles t-1, t and t+1 are read.
  // Each set holds its Q tile followed by its dO tile, so one address reaches a row of
  // both (the dO read adds a fixed instruction offset).
  __shared__ __attribute__((aligned(1024))) __bf16 S0[2 * C::QTILE];
  __shared__ __attribute__((aligned(1024))) __bf16 S1[2 * C::QTILE];
  __shared__ __attribute__((aligned(1024))) __bf16 S2[2 * C::QTILE];
  __shared__ __attribute__((aligned(1024))) __bf16 S3[2 * C::QTILE];
  __bf16* const Q0 = S0;
  __bf16* const Q1 = S1;
  __bf16* const Q2 = S2;
  __bf16* const Q3 = S3;
  __bf16* const G0 = S0 + C::QTILE;  // dO
  __bf16* const G1 = S1 + C::QTILE;
  __bf16* const G2 = S2 + C::QTILE;
  __bf16* const G3 = S3 + C::QTILE;
  __shared__ __attribute__((aligned(16))) float L0[C::BQ];
  __shared__ __attribute__((aligned(16))) float L1[C::BQ];
  __shared__ __attribute__((aligned(16))) float L2s[C::BQ];
  __shared__ __attribute__((aligned(16))) float L3[C::BQ];
  __shared__ __attribute__((aligned(16))) float E0[C::BQ];  // D values
  __shared__ __attribute__((aligned(16))) float E1[C::BQ];
  __shared__ __attribute__((aligned(16))) float E2[C::BQ];
  __shared__ __attribute__((aligned(16))) float E3[C::BQ];
  // K and V rows of a block, staged by direct loads and then read into AGPRs: chunk c of
  // row r (16-byte units) at ((r/16)*CPR + c)*16 + r%16, so the 16 lanes of a 128-bit read
  // phase, 16 consecutive rows at one chunk, touch 256 contiguous bytes.  A block's rows
  // are loaded while the block before it ends (see the block loop below).
  __shared__ __attribute__((aligned(1024))) __bf16 KVs[2 * C::BKV * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int g = lane >> 5, l32 = lane & 31;
  constexpr int KB = C::KB;
  // Dense calls: logical blocks (id: unit and key block, heaviest first when causal) are
  // taken in rounds k = 0, 1, ... of nwg = gridDim.x at a time.  A launch of one workgroup
  // per block runs one round.  A persistent launch (fewer workgroups, each looping) walks
  // every second round backwards within its XCD (nwg a multiple of 8), so a workgroup's
  // blocks alternate between the heavy and the light end of a round; blocks stay on the
  // XCD whose L2 holds their unit's rows, as with one workgroup per block.
  // General calls (always persistent, nwg a multiple of 8): workgroup wi runs on XCD
  // wi % 8 and takes that XCD's list in the plan (most steps first) in the same rounds.
  const int nwg = gridDim.x;
  int lbeg = 0, lend = 0;
  if constexpr (GEN) {
    lbeg = plan[blockIdx.x & 7];
    lend = plan[(blockIdx.x & 7) + 1];
  }
  auto vindex = [&](int k) -> int {
    const int wi = blockIdx.x;
    if constexpr (GEN) {
      const int nx = nwg >> 3, li = wi >> 3;
      return k * nx + ((k & 1) ? nx - 1 - li : li);
    }
    if ((nwg & 7) != 0 || !(k & 1)) return k * nwg + wi;
    return k * nwg + (nwg - 8 - (wi & ~7)) + (wi & 7);
  };
  auto has = [&](int v) -> bool { return GEN ? lbeg + v < lend : v < total; };
  auto block_of = [&](int v, int& bh_, int& kb_) {
    if constexpr (GEN) {
      const int id = plan[kPlanHead + lbeg + v];
      bh_ = id / nkb;
      kb_ = id - bh_ * nkb;
      return;
    }
    const int id = xcd_remap(v, total);
    bh_ = id / nkb;
    kb_ = id - bh_ * nkb;
    if (causal) {  // the first key blocks see the most query tiles: heaviest first
      int t;
      heavy_first(id, nkb, total / nkb, heavy_group(Nmax, D), bh_, t);
      kb_ = nkb - 1 - t;
    }
  };
  // The current block: unit bh, rows base.. of its sequence (length N), keys k0.. (this
  // wave's from kw), query tiles qt0..nqt-1.
  int bh = 0, kb = 0, base = 0, N = 0, k0 = 0, kw = 0, nqt = 0, qt0 = 0;
  size_t head = 0, hpad = 0;
  auto set_block = [&](int v) {
    block_of(v, bh, kb);
    seq_rows(sm, bh, Nmax, base, N);
    head = (size_t)base * D;
    hpad = (size_t)bh * Npad;
    k0 = kb * C::BKV;
    kw = k0 + w * 32 * KB;
    // query tiles of this sequence that see these keys (its padded rows hold lse = +inf:
    // P = 0 there)
    key_block_tiles<C::BKV, C::BQ>(N, k0, causal, window, qt0, nqt);
  };

  // --- direct-load source offsets ------------------------------------------------
  // Row-major swizzled tiles: chunk slot s = r*CPR + p holds logical chunk p ^ f(r).
  int q_row[C::QLOADS], q_col[C::QLOADS];
#pragma unroll
  for (int i = 0; i < C::QLOADS; ++i) {
    const int slot = (w * C::QLOADS + i) * 64 + lane;
    const int r = slot / CPR, p = slot % CPR;
    q_row[i] = r;
    q_col[i] = (p ^ bswz<D>(r)) * 8;
  }
  auto issue_q = [&](int qt, __bf16* Qd, __bf16* Gd, float* Ld, float* Ed) {
    const int qb0 = qt * C::BQ;  // < N: every streamed tile holds a valid row
    const __bf16* qs = Q + head + (size_t)qb0 * D;
    const __bf16* gs = dO + head + (size_t)qb0 * D;
#pragma unroll
    for (int i = 0; i < C::QLOADS; ++i) {
      // padding rows past N read the last row (P = 0 there)
      const unsigned off = (unsigned)(min(q_row[i], N - 1 - qb0) * D + q_col[i]) * 2u;
      dma16(qs, off, Qd + (w * C::QLOADS + i) * 512);
      dma16(gs, off, Gd + (w * C::QLOADS + i) * 512);
    }
    if (w < 2) {  // lse on wave 0, D on wave 1: 16 bytes per lane of lanes 0..BQ/4-1
      // the lane index read afresh, so that it need not stay live across the loop
      unsigned ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      if (ln < C::BQ / 4) dma16((w == 0 ? L2 : Dvec) + hpad + qb0, 16u * ln, w == 0 ? Ld : Ed);
    }
  };
  // --- per-lane LDS read offsets -------------------------------------------------
  // Natural A-operand read of row l32, logical chunk 2*kk + g.
  int nat[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) nat[kk] = l32 * D + (((2 * kk + g) ^ bswz<D>(l32)) << 3);
  // Transposed reads: lane (G, e, q4) loads 8 bytes of row base + 8h + 4(G>>1) + e at
  // column col0 + 16(G&1) + 4 q4, base a multiple of 16.  For the swizzled tiles the
  // chunk depends on h (rows 0-7 vs 8-15 of the 16) and on the 32-column tile.
  const int G = lane >> 4, e4 = (lane >> 2) & 3, q4 = lane & 3;
  int trq[2][NDT];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int row = 8 * h + 4 * (G >> 1) + e4;
      const int col = dt * 32 + 16 * (G & 1) + 4 * q4;
      trq[h][dt] = row * D + ((((col >> 3) ^ bswz<D>(row))) << 3) + (col & 7);
    }

  // --- K and V of this wave's keys as B operands (natural k order), in AGPRs -------
  // K and V only ever feed the matrix cores, which read A/B operands from AGPRs as
  // well; keeping them there leaves the VGPRs for operand prefetch.
  bf16x8_t kop[KB][NKK], vop[KB][NKK];
  constexpr int KVL = C::BKV * CPR / 64 / C::NW;  // direct loads per wave and tensor
  static_assert(C::BKV * CPR % (64 * C::NW) == 0, "K/V rows split over the waves");
  // Stage keys kk0.. of the unit whose rows start at element hd (sequence length n); rows
  // past the end read the last row (their S is masked, so P = 0 and dS = 0 there).
  auto issue_kv = [&](size_t hd, int kk0, int n) {
    // The bases come out of this block's index arithmetic right here, partly on the vector
    // ALUs: wait states between their last write and the loads.
    const unsigned long long ks = sgpr_ptr(K + hd + (size_t)kk0 * D);
    const unsigned long long vs = sgpr_ptr(V + hd + (size_t)kk0 * D);
    sgpr_wait(ks, vs);
    // the lane index read afresh, so that no offset stays live across the steps
    unsigned ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
#pragma unroll
    for (int i = 0; i < KVL; ++i) {
      const int slot = (w * KVL + i) * 64 + (int)ln;
      const int grp = slot / (CPR * 16), within = slot % (CPR * 16);
      const int r = min(grp * 16 + (within & 15), n - 1 - kk0);
      const unsigned off = (unsigned)(r * D + (within >> 4) * 8) * 2u;
      dma16_s(ks, off, KVs + (w * KVL + i) * 64 * 8);
      dma16_s(vs, off, KVs + C::BKV * D + (w * KVL + i) * 64 * 8);
    }
  };
  // The staged rows into AGPRs (then waited for: lgkmcnt(0)).
  auto read_kv = [&]() {
    unsigned ln;  // read afresh, as in issue_kv
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const int l32f = (int)ln & 31, gf = (int)ln >> 5;
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int r = w * 32 * KB + 32 * b + l32f, c = 2 * kk + gf;
        const int e = (((r >> 4) * CPR + c) * 16 + (r & 15)) * 8;
        lds_read_a(kop[b][kk], KVs + e);
        lds_read_a(vop[b][kk], KVs + C::BKV * D + e);
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  };
  // The next block's rows (round kcur + 1) are staged right after this block's last
  // tile load: they load under its last steps, products and stores, whose waits leave
  // those KVN loads in flight (kv_inflight).
  constexpr int KVN = 2 * KVL;
  static_assert(KVN < 64, "vmcnt range");
  int kcur = 0;
  bool kv_inflight = false;
  auto issue_kv_next = [&]() {
    int bhn, kbn, basen, nn;
    block_of(vindex(kcur + 1), bhn, kbn);
    seq_rows(sm, bhn, Nmax, basen, nn);
    issue_kv((size_t)basen * D, kbn * C::BKV, nn);
  };

  // dK^T, dV^T accumulators in AGPRs (written by v_accvgpr_write: 4 wait states
  // before the first product accumulates into them).
  f32x16_t dk[KB][NDT], dv[KB][NDT];
  auto zero_acc = [&]() {
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        dk[b][dt] = zero16();
        dv[b][dt] = zero16();
        asm volatile("s_nop 3" : "+a"(dk[b][dt]), "+a"(dv[b][dt]));
      }
  };
  const float c = scale * kLog2e;

  // P^T and dS^T of the previous tile, as bf16 A operands (j = 0, 1 query halves).
  // They start at zero, so the first step's dV/dK products add nothing.
  bf16x8_t pa[KB][2], da[KB][2];
  auto zero_pd = [&]() {
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          pa[b][j][t] = (__bf16)0.0f;
          da[b][j][t] = (__bf16)0.0f;
        }
  };
  // Q and dO rows of the next tile (A operands of its S and dP), read one step ahead
  // straight into AGPRs: the S and dP products of a step then start right after its
  // barrier, and these reads run under the previous step's dV/dK products.
  bf16x8_t aq[NKK], ag[NKK];
  auto prefetch_rows = [&](const __bf16* Qb, const __bf16* Gb, int kk) {
    (void)Gb;  // == Qb + QTILE
    lds_read_a_pair<C::QTILE * 2>(aq[kk], ag[kk], Qb + nat[kk]);
  };

  // Step qt (tile t in buffer set (t - qt0) % 4; p = tile qt-1, c = tile qt, n = tile
  // qt+1, i = tile qt+2):
  //   wait until tile qt+1 has landed everywhere and this wave's reads of tile qt's
  //   rows are back; start tile qt+2 (its set last held tile qt-2, whose final reads
  //   were in step qt-1);
  //   S, dP of tile qt from the prefetched rows; read tile qt-1's transposed dO and Q
  //   (B operands of its dV, dK) and tile qt's lse and D while they run;
  //   tile qt-1's dV/dK products, each followed by a slice of tile qt's softmax and
  //   two reads of tile qt+1's rows (past the last tile: stale, never used).
  auto step = [&](int qt, const __bf16* Qp, const __bf16* Gp, const float* Lc, const float* Ec,
                  const __bf16* Qn, const __bf16* Gn, __bf16* Qi, __bf16* Gi, float* Li, float* Ei) {
    __builtin_amdgcn_sched_barrier(0);  // no code motion across steps
    if (kv_inflight)  // all but the next block's K/V rows: vmcnt(KVN) lgkmcnt(0)
      __builtin_amdgcn_s_waitcnt(((KVN >> 4) << 14) | (KVN & 15) | 0x0070);
    else
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int qb0 = qt * C::BQ;

    // S = Q K^T and dP = dO V^T: queries on rows, this wave's keys on lanes; the
    // results land in VGPRs, where the softmax below reads them.  Between the
    // products go the step's other operand reads: tile qt-1's dO and Q transposed
    // (B operands of its dV/dK) and tile qt's lse and D, so those LDS round trips
    // start at once and run under the products instead of after them.
    f32x16_t s[KB], dp[KB];
    bf16x8_t bg[2][NDT], bq[2][NDT];
    float lv[16], dvv[16];
    constexpr int NTR = 4 * NDT;        // transposed 16-byte operands to read
    constexpr int NRD = NKK < 4 ? NKK : 4;  // d-steps the reads are spread over
    constexpr int TPK = NTR / NRD;      // ... per d-step of the products
    constexpr int LPK = 8 / NRD;        // lse/D 128-bit reads per d-step
    static_assert(NTR % NRD == 0 && 8 % NRD == 0, "reads must split over the d-steps");
    auto read_tr = [&](int t) {  // t = (j * NDT + dt) * 2 + (0: dO, 1: Q)
      const int j = t / (2 * NDT), dt = (t / 2) % NDT;
      const __bf16* b = (t & 1) ? Qp : Gp;
      const bf16x8_t v = tr_pair(b + j * 16 * D + trq[0][dt], b + j * 16 * D + trq[1][dt]);
      if (t & 1) bq[j][dt] = v;
      else bg[j][dt] = v;
    };
    auto read_le = [&](int t) {  // rows 8(t/2) + 4g + 0..3: lse for even t, D for odd t,
      const int b = t >> 1;        // in the order the softmax below consumes them
      const float4 x = *reinterpret_cast<const float4*>(((t & 1) ? Ec : Lc) + 8 * b + 4 * g);
      float* dst = (t & 1) ? dvv : lv;
      dst[4 * b] = x.x, dst[4 * b + 1] = x.y, dst[4 * b + 2] = x.z, dst[4 * b + 3] = x.w;
    };
    // S = Q K^T alone first: its chain of dependent products runs back to back.  The
    // step's LDS reads go under it.
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        if (kk == 0) mma_v_first_aa(s[b], aq[0], kop[b][0]);
        else mma_v_aa(s[b], aq[kk], kop[b][kk]);
      }
      if (kk < NRD) {
#pragma unroll
        for (int t = kk * TPK; t < kk * TPK + TPK; ++t) read_tr(t);
#pragma unroll
        for (int t = kk * LPK; t < kk * LPK + LPK; ++t) read_le(t);
      }
      // tile qt+2 starts loading once the first products are under way
      if (kk == 1 && qt + 2 < nqt) issue_q(qt + 2, Qi, Gi, Li, Ei);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Then dP = dO V^T, with P = 2^(s*c - lse2) of the first N1 elements on the vector
    // ALUs under it (element e is row 8 * (e / (8*KB)) + e % 8 of key block (e / 8) % KB).
    constexpr int NDP = NKK * KB;
    constexpr int N1 = 2 * (NDP - 2) < 16 * KB ? 2 * (NDP - 2) : 16 * KB;
    // Keys past the end and, on tiles crossing the diagonal, keys above it: S = -inf,
    // so P = 2^-inf = 0 and dS = 0.  Only those tiles pay for the per-element test.
    const bool need_mask = (kw + 32 * KB > N) || (causal && kw + 32 * KB - 1 > qb0) ||
                           (window > 0 && qb0 + 31 >= kw + window);
#pragma unroll
    for (int m = 0; m < NDP; ++m) {
      const int kk = m / KB, b = m % KB;
      if (kk == 0) mma_v_first_aa(dp[b], ag[0], vop[b][0]);
      else mma_v_aa(dp[b], ag[kk], vop[b][kk]);
      if (m == 1) {  // two products after the last of S: its wait states run under them
        mfma_v_ready1(s[KB - 1]);
#pragma unroll
        for (int bb = 0; bb < KB - 1; ++bb) asm volatile("" : "+v"(s[bb]));
        if (need_mask) {
#pragma unroll
          for (int bb = 0; bb < KB; ++bb) {
            const int key = kw + 32 * bb + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int q = qb0 + crow(g, r);
              const bool dead = (key >= N) | (causal & (key > q)) | ((window > 0) & (q - key >= window));
              s[bb][r] = dead ? -INFINITY : s[bb][r];
            }
          }
        }
      }
      if (m >= 2) {
#pragma unroll
        for (int e = 2 * (m - 2); e < 2 * (m - 2) + 2 && e < N1; ++e) {
          const int eb = (e / 8) % KB, r = 8 * (e / (8 * KB)) + e % 8;
          s[eb][r] = __builtin_amdgcn_exp2f(fmaf(s[eb][r], c, -lv[r]));
          asm volatile("" : "+v"(s[eb][r]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // All of this phase's LDS reads (transposed operands, lse, D) are waited for here,
    // before the next tile's row reads below are issued: those are inline assembly the
    // compiler does not count, so a wait it places later for one of this phase's reads
    // would also wait for them.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    // The first dV product reads neither S nor dP: it runs while dP's last products
    // drain, under the wait states the vector ALUs need before reading them.
    mma_a(dv[0][0], pa[0][0], bg[0][0]);
    mfma_v_ready1(dp[KB - 1]);
#pragma unroll
    for (int b = 0; b < KB - 1; ++b) asm volatile("" : "+v"(dp[b]));  // after the wait states

    // The previous tile's dV/dK products (accumulating in AGPRs), each followed by
    // elements of this tile's P = 2^(s*c - lse2) and dS = P (dP - D) on the vector
    // ALUs and by reads of the next tile's rows; sched_barrier keeps that interleave.
    constexpr int NSTEP = 2 * NDT * KB, EPS = 16 * KB / NSTEP;  // product pairs; elements per pair
    // Each slice's P and dS are pinned where they are computed (empty asm reading
    // them): the compiler would otherwise sink the dS arithmetic and the bf16
    // conversions below the last product, where they run with the matrix cores idle.
    // The first query half's bf16 operands are formed as soon as this step's last
    // product reading the previous half-0 operands is issued; the second half's after
    // the loop.
    auto to_bf16 = [&](int j) {
#pragma unroll
      for (int b = 0; b < KB; ++b) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          pa[b][j][t] = (__bf16)s[b][8 * j + t];
          da[b][j][t] = (__bf16)dp[b][8 * j + t];
        }
        asm volatile("" : "+v"(pa[b][j]), "+v"(da[b][j]));
      }
    };
    // Pair i multiplies query half j = i / (KB*NDT) of key block (i / NDT) % KB; element e
    // is row 8 * (e / (8*KB)) + e % 8 of key block (e / 8) % KB, so the first NSTEP/2
    // pairs both read and (by their end) compute exactly query half 0.
    static_assert(EPS * (NSTEP / 2) == 8 * KB && NSTEP / 2 == NDT * KB, "half 0 is done by slot NSTEP/2");
    // Row reads of the next tile go in the first half of the pairs, so they are back
    // well before the next step's wait.
    constexpr int RPP = (NKK + NSTEP / 2 - 1) / (NSTEP / 2);  // row-operand steps per pair
    auto elems = [&](int e0, int e1) {  // P of elements below N1 is already formed
#pragma unroll
      for (int e = e0; e < e1; ++e) {
        const int b = (e / 8) % KB, r = 8 * (e / (8 * KB)) + e % 8;
        const float p = e < N1 ? s[b][r] : __builtin_amdgcn_exp2f(fmaf(s[b][r], c, -lv[r]));
        s[b][r] = p;
        dp[b][r] = p * (dp[b][r] - dvv[r]);
        asm volatile("" : "+v"(s[b][r]), "+v"(dp[b][r]));
      }
    };
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      const int j = i / (NDT * KB), b = (i / NDT) % KB, dt = i % NDT;
      // Each product is followed by half the pair's vector work, so both products of
      // the pair run under it.
      if (i > 0) mma_a(dv[b][dt], pa[b][j], bg[j][dt]);
      if (i == NSTEP / 2) to_bf16(0);  // products 0 .. NSTEP/2-1 read half 0
      elems(i * EPS, i * EPS + EPS / 2);
      __builtin_amdgcn_sched_barrier(0);
      mma_a(dk[b][dt], da[b][j], bq[j][dt]);
#pragma unroll
      for (int kk = i * RPP; kk < i * RPP + RPP && kk < NKK; ++kk) prefetch_rows(Qn, Gn, kk);
      elems(i * EPS + EPS / 2, i * EPS + EPS);
      __builtin_amdgcn_sched_barrier(0);
    }
    to_bf16(1);
#pragma unroll
    for (int b = 0; b < KB; ++b) valu_ready(pa[b][0], pa[b][1], da[b][0], da[b][1]);  // read next step
  };

  // Q3/G3 start at zero: the first step of a workgroup's first block reads its "previous"
  // dV/dK operands there (with P^T = dS^T = 0), and 0 * (an Inf or NaN bit pattern) would
  // not be 0; later blocks find finite rows of earlier tiles there.  The first block's
  // barrier orders these writes before those reads.
  for (int i = tid; i < C::QTILE / 8; i += C::NT) {
    reinterpret_cast<v16b*>(Q3)[i] = v16b{0, 0, 0, 0};
    reinterpret_cast<v16b*>(G3)[i] = v16b{0, 0, 0, 0};
  }
  // A block after a workgroup's first finds its K/V rows staged by the one before it
  // (kv_inflight).  Neither dense blocks nor planned ones are ever empty; should a planned
  // one be, its staged rows are waited for and the next block loads its own.
  for (int k = 0;; ++k) {
    const int v = vindex(k);
    if (!has(v)) break;
    set_block(v);
    // Prologue: K/V rows (unless staged), tiles qt0 and qt0+1 loading; once all have
    // landed, K/V into AGPRs and tile qt0's rows.
    if constexpr (GEN) {
      if (k0 >= N) {  // no keys here
        if (kv_inflight) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        kv_inflight = false;
        continue;
      }
      if (k > 0) __builtin_amdgcn_s_barrier();  // the last block's tiles are no longer read
      if (!kv_inflight) issue_kv(head, k0, N);
    } else {
      if (k0 >= N) continue;  // (never taken; kept for the compiler's register allocation)
      if (k > 0) __builtin_amdgcn_s_barrier();  // as above
      else issue_kv(head, k0, N);
    }
    issue_q(qt0, Q0, G0, L0, E0);
    if (qt0 + 1 < nqt) issue_q(qt0 + 1, Q1, G1, L1, E1);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    kv_inflight = false;
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_kv();
    zero_acc();
    zero_pd();
    kcur = k;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) prefetch_rows(Q0, G0, kk);
    int qt = qt0;
    for (; qt + 3 < nqt; qt += 4) {  // whole rotations: no conditional steps in the body
      step(qt, Q3, G3, L0, E0, Q1, G1, Q2, G2, L2s, E2);
      step(qt + 1, Q0, G0, L1, E1, Q2, G2, Q3, G3, L3, E3);
      step(qt + 2, Q1, G1, L2s, E2, Q3, G3, Q0, G0, L0, E0);
      step(qt + 3, Q2, G2, L3, E3, Q0, G0, Q1, G1, L1, E1);
    }
    // Stage the next block's rows after step nqt - 3, which issues the last tile load (or
    // after the first step if there is none), so that they are the newest loads in flight;
    // past the first step's barrier every wave has read this block's K/V.
    const bool stage = has(vindex(k + 1));
    auto stage_next = [&]() {
      issue_kv_next();
      kv_inflight = true;
    };
    if (stage && qt > qt0 && qt >= nqt - 2) stage_next();
    if (qt < nqt) step(qt, Q3, G3, L0, E0, Q1, G1, Q2, G2, L2s, E2);
    if (stage && !kv_inflight) stage_next();
    if (qt + 1 < nqt) step(qt + 1, Q0, G0, L1, E1, Q2, G2, Q3, G3, L3, E3);
    if (qt + 2 < nqt) step(qt + 2, Q1, G1, L2s, E2, Q3, G3, Q0, G0, L0, E0);
    // dV/dK of the last tile (buffer set (nqt - 1 - qt0) % 4, intact: no later loads)
    {
      const int last = (nqt - 1 - qt0) % 4;
      const __bf16* Qp = last == 0 ? Q0 : last == 1 ? Q1 : last == 2 ? Q2 : Q3;
      const __bf16* Gp = last == 0 ? G0 : last == 1 ? G1 : last == 2 ? G2 : G3;
      // The transposed-read offsets formed afresh (as trq): nothing the steps keep in
      // registers needs to live on to here.
      unsigned ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      int trf[2][NDT];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int row = 8 * h + 4 * ((int)ln >> 5) + (((int)ln >> 2) & 3);
          const int col = dt * 32 + 16 * (((int)ln >> 4) & 1) + 4 * ((int)ln & 3);
          trf[h][dt] = row * D + ((((col >> 3) ^ bswz<D>(row))) << 3) + (col & 7);
        }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8_t bg = tr_pair(Gp + j * 16 * D + trf[0][dt], Gp + j * 16 * D + trf[1][dt]);
          const bf16x8_t bq = tr_pair(Qp + j * 16 * D + trf[0][dt], Qp + j * 16 * D + trf[1][dt]);
#pragma unroll
          for (int b = 0; b < KB; ++b) {
            mma_a(dv[b][dt], pa[b][j], bg);
            mma_a(dk[b][dt], da[b][j], bq);
          }
        }
    }
    // The last step's reads of the next tile's rows (stale: never used) are back.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)

    // MFMA results in AGPRs: 16 wait states before v_accvgpr_read may take them.
    asm volatile("s_nop 7\n\ts_nop 7" : "+a"(dk[0][0]), "+a"(dv[0][0]));
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) asm volatile("" : "+a"(dk[b][dt]), "+a"(dv[b][dt]));
    // dK (scaled) and dV, one tensor at a time, transposed through this wave's query-tile
    // set (free now: once every wave has passed the barrier below, all have done their
    // last products, and the next block loads its tiles only after its own barrier).
    // Lane (g, c) holds column c of key rows crow(g, r); rows r = 4i .. 4i+3 are four
    // consecutive keys and go to LDS as one 8-byte write in a [column][key] layout.
    // Transposing reads of that layout give each lane 4 consecutive columns of one key, two
    // reads 8, which leave with one 16-byte store: 16 stores per lane instead of 128.
    __builtin_amdgcn_s_barrier();
    {
      unsigned ln;  // read afresh: nothing below is formed before the barrier
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      constexpr int KW = 32 * KB;   // keys per wave
      constexpr int NKH = KW / 16;  // 16-key groups per wave
      __bf16* const reg = w == 0 ? S0 : w == 1 ? S1 : w == 2 ? S2 : S3;  // KW x D bf16 fit
      static_assert(KW * D <= 2 * C::QTILE, "a wave's tile fits its set");
      auto loff = [](int col, int kc) { return col * KW + 4 * (kc ^ epi_swz<D>(col)); };
      const int lg = (int)ln >> 5, lc = (int)ln & 31;
      const int q = (int)ln >> 4, e = ((int)ln >> 2) & 3, j = (int)ln & 3, i16 = (int)ln & 15;
      auto put = [&](f32x16_t (&acc)[KB][NDT], float mul, __bf16* dst) {
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              bf16x4_t x;
#pragma unroll
              for (int t = 0; t < 4; ++t) x[t] = (__bf16)(acc[b][dt][4 * i + t] * mul);
              *reinterpret_cast<bf16x4_t*>(reg + loff(dt * 32 + lc, 8 * b + 2 * i + lg)) = x;
            }
        // lane (q, e, j) of read h fetches column 32cb + 8q + 4h + e, keys 16kh + 4j ..
        // +3; lane (q, i) receives columns 32cb + 8q + 4h .. +3 of key 16kh + i.
#pragma unroll
        for (int s = 0; s < NKH * NDT; ++s) {
          const int kh = s % NKH, cb = s / NKH;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(reg + loff(32 * cb + 8 * q + e, 4 * kh + j)));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(reg + loff(32 * cb + 8 * q + 4 + e, 4 * kh + j)));
          const int key = kw + 16 * kh + i16;
          if (key < N) {
            const v16b val = __builtin_bit_cast(v16b, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            *reinterpret_cast<v16b*>(dst + head + (size_t)key * D + 32 * cb + 8 * q) = val;
          }
        }
      };
      put(dk, scale, dK);
      put(dv, 1.0f, dV);
    }
  }
  // No direct load may still be in flight when the wave ends.
  __builtin_amdgcn_s_waitcnt(0x0070);
}

template <int D, bool GEN>
static hipError_t launch_bwd_bf16_d(const BwdArgs& a) {
  using C = BwdFast<D>;
  const int nkb = (a.N + C::BKV - 1) / C::BKV;
  const long long total = (long long)a.B * a.H * nkb;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // One wave per SIMD fills a CU: the pass runs one persistent workgroup per CU (a
  // multiple of 8, for the rounds' XCD order), each taking its blocks in turn and staging
  // the next one's K/V while it finishes the current one.  Variable-length and windowed
  // calls, whose blocks differ irregularly in cost, take them from a plan sorted by cost.
  const int ncu = compute_units();
  long long grid = total;
  const SeqMap sm{a.cu_seqlens, a.B, a.T};
  launch_begin();
  if (!GEN) {
    if (ncu >= 8 && total > ncu) grid = ncu - ncu % 8;
  } else {
    // The plan first (one workgroup), then one workgroup per CU, a multiple of 8.
    hipLaunchKernelGGL((bwd_plan_kernel<C::BKV, C::BQ>), dim3(1), dim3(kPlanThreads), 0,
                       (hipStream_t)a.stream, sm, a.N, a.causal, a.window, nkb, (int)total, a.plan);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    grid = ncu >= 8 ? ncu - ncu % 8 : 8;
  }
  hipLaunchKernelGGL((bwd_bf16_kernel<D, GEN>), dim3((unsigned)grid), dim3(C::NT), 0,
                     (hipStream_t)a.stream, (const __bf16*)a.q, (const __bf16*)a.k,
                     (const __bf16*)a.v, (const __bf16*)a.dout, a.L2, a.Dvec, (__bf16*)a.dk,
                     (__bf16*)a.dv, a.N, a.Npad, a.scale, a.causal, nkb, (int)total, sm,
                     a.window, GEN ? (const int*)a.plan : nullptr);
  return hipGetLastError();
}

hipError_t launch_bwd_main_bf16(const BwdArgs& a) {
  const bool gen = a.cu_seqlens != nullptr || a.window > 0;
  if (a.d == 64) return gen ? launch_bwd_bf16_d<64, true>(a) : launch_bwd_bf16_d<64, false>(a);
  if (a.d == 128) return gen ? launch_bwd_bf16_d<128, true>(a) : launch_bwd_bf16_d<128, false>(a);
  return hipErrorInvalidValue;
}

}  // namespace fa
