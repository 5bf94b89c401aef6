// fa_device.h -- device-side building blocks of the attention kernels (gfx950).
//
// Matrix products run on the CDNA4 32x32 MFMA instructions with fp32 accumulation:
//   bf16 operands: v_mfma_f32_32x32x16_bf16 (each lane feeds 8 bf16 of A and of B)
//   fp32 operands: v_mfma_f32_32x32x2_f32   (each lane feeds 1 float of A and of B)
//
// Lane layout of a 32x32 accumulator (16 floats per lane, wave64): lane L holds
// column  n = L % 32  and, in register r, row  m = 8*(r/4) + 4*(L/32) + (r%4).
// The contraction index of one instruction is split over the two half-waves
// g = L/32: the kernels only need A and B to agree on which logical k each
// (g, slot) carries, so they use two assignments:
//   natural : slot s of half g carries k = g*EPL + s            (contiguous reads)
//   c-layout: slot s of instruction j, half g carries the row of accumulator
//             register j*EPL + s, i.e. k = crow(g, j*EPL + s)   (feeds a product
//             straight from a previous accumulator, no shuffle needed)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Row of accumulator register r held by half-wave g.
__device__ __forceinline__ constexpr int crow(int g, int r) {
  return 8 * (r >> 2) + 4 * g + (r & 3);
}

template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
  static constexpr int KPI = 16;  // contraction length of one instruction
  static constexpr int EPL = 8;   // operand elements per lane
  typedef bf16x8_t op_t;
  static __device__ __forceinline__ f32x16_t mma(op_t a, op_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // EPL contiguous elements starting at p (16-byte aligned).
  static __device__ __forceinline__ op_t load(const __bf16* p) {
    return *reinterpret_cast<const op_t*>(p);
  }
  // One element per slot from p + offs(s) (strided / gathered operand).
  template <typename F>
  static __device__ __forceinline__ op_t gather(const __bf16* p, F offs) {
    op_t v;
#pragma unroll
    for (int s = 0; s < EPL; ++s) v[s] = p[offs(s)];
    return v;
  }
  // Operand from accumulator registers r0 .. r0+EPL-1 (rounded to nearest even).
  static __device__ __forceinline__ op_t from_acc(const f32x16_t& c, int r0) {
    op_t v;
#pragma unroll
    for (int s = 0; s < EPL; ++s) v[s] = (__bf16)c[r0 + s];
    return v;
  }
  static __device__ __forceinline__ op_t zero() {
    op_t v;
#pragma unroll
    for (int s = 0; s < EPL; ++s) v[s] = (__bf16)0.0f;
    return v;
  }
};

template <>
struct Mma<float> {
  static constexpr int KPI = 2;
  static constexpr int EPL = 1;
  typedef float op_t;
  static __device__ __forceinline__ f32x16_t mma(op_t a, op_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ op_t load(const float* p) { return *p; }
  template <typename F>
  static __device__ __forceinline__ op_t gather(const float* p, F offs) {
    return p[offs(0)];
  }
  static __device__ __forceinline__ op_t from_acc(const f32x16_t& c, int r0) { return c[r0]; }
  static __device__ __forceinline__ op_t zero() { return 0.0f; }
};

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// 16-byte vector copy type.
struct alignas(16) v16b {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// One direct global -> LDS load of 16 bytes per lane: lane l's bytes come from
// base + voff (base wave-uniform, voff in bytes) and land at lds_wave + 16*l, so the
// loaded data never passes through VGPRs.  Issued as inline assembly: with the
// compiler builtin for this load, the compiler counts it as an LDS access of
// unknown order and then uses full drains (lgkmcnt(0)) for every LDS wait in the
// kernel, so LDS reads can no longer run ahead of the matrix products that consume
// them.  The compiler therefore does not track these loads: every caller waits for
// them itself (s_waitcnt vmcnt(0), then a barrier) before the tile is read.
// LDS byte address of a pointer into a __shared__ array.  A generic pointer to LDS
// carries the LDS offset in its low 32 bits (the high bits are the shared aperture),
// so truncation gives it without the null test an address-space cast emits.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(unsigned long long)p;
}

__device__ __forceinline__ void dma16(const void* base, unsigned voff, const void* lds_wave) {
  const unsigned long long t = (unsigned long long)base;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)t);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(t >> 32));
  const unsigned long long sbase = ((unsigned long long)hi << 32) | lo;
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave));
  // M0 (the LDS destination) is bound as an operand, so the compiler sets it itself.
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

// A wave-uniform pointer as a 64-bit scalar register pair.
__device__ __forceinline__ unsigned long long sgpr_ptr(const void* p) {
  const unsigned long long t = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)t);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(t >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
// dma16 from a base already in scalar registers (sgpr_ptr).  A vector-ALU write of the
// base (v_readfirstlane) needs five wait states before a load reads it; callers that form
// the base right before their loads separate the two with sgpr_wait.
__device__ __forceinline__ void dma16_s(unsigned long long sbase, unsigned voff, const void* lds_wave) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave));
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}
// Five wait states after the scalar registers of a and b were last written.
__device__ __forceinline__ void sgpr_wait(unsigned long long a, unsigned long long b) {
  asm volatile("s_nop 4" ::"s"(a), "s"(b));
}

// Block id -> logical work id.  Consecutive workgroup ids are spread round robin
// over the 8 XCDs (each with its own L2); the remap hands each XCD a contiguous
// range of logical ids, so the tiles of one (batch, head) share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int id, int n) {
  constexpr int kXcd = 8;
  if (n % kXcd != 0) return id;
  return (id % kXcd) * (n / kXcd) + id / kXcd;
}

// Logical work id -> (unit, tile) when a unit's tiles differ in cost (causal: the last
// query block of a head costs the most).  Units are taken in groups of G, and within a
// group tiles go heaviest first, alternating over the group's units.  With G = 2 an
// XCD's contiguous range of ids works on about two units at a time and the heaviest tiles
// of every pair start before its light ones, so the grid does not end with a few CUs
// finishing heavy tiles while the rest idle; G = 1 is plain unit-by-unit order (heaviest
// tile of each unit first).  Ids cover nunits * nt.
__device__ __forceinline__ void heavy_first(int id, int nt, int nunits, int G, int& unit, int& tile) {
  const int group = id / (G * nt);
  const int within = id - group * G * nt;
  const int gs = min(G, nunits - group * G);  // the last group may hold fewer units
  const int rank = within / gs;
  unit = group * G + (within - rank * gs);
  tile = nt - 1 - rank;
}
// Units per group for heavy_first: as many as keep the group's K and V (2 * N * D bf16
// per unit) within about 4 MiB, an XCD's L2 (1 to 8): two heads of 4096 x 128, eight of
// 2048 x 64.  Larger groups balance small grids (few blocks per CU, where the longest
// blocks set the time); past one head per group the extra K/V re-reads miss L2 for no gain.
// Variable-length batches keep groups of one: their units differ in length, and grouping
// measured slower there.
__device__ __forceinline__ int heavy_group(int N, int D) {
  const long long nd = (long long)N * D;
  return nd >= (1 << 20) ? 1 : (int)min(8LL, (1LL << 20) / nd);
}

// Rows of one (batch, head) unit of work.  Dense: [B, H, N, d], unit bh = b*H + h
// owns rows bh*N .. bh*N + N-1.  Variable length (cu != null): tensors are packed
// head-major [H, T, d] with sequence b in rows cu[b] .. cu[b+1]-1 of every head, and
// unit bh = h*B + b owns rows h*T + cu[b] ...  The boundaries are device data the
// host cannot see: they are clamped to 0 <= cu[b] <= cu[b+1] <= T and the length to
// Nmax, so that a malformed table can give wrong rows but never an access outside
// the tensors.
struct SeqMap {
  const int* cu;  // null: dense
  int B;          // sequences (varlen)
  int T;          // rows per head (varlen)
};
__device__ __forceinline__ void seq_rows(const SeqMap& m, int bh, int Nmax, int& base, int& len) {
  if (m.cu == nullptr) {
    base = bh * Nmax;
    len = Nmax;
    return;
  }
  const int h = bh / m.B, b = bh - h * m.B;
  const int c0 = min(max(m.cu[b], 0), m.T);
  const int c1 = min(max(m.cu[b + 1], c0), m.T);
  base = h * m.T + c0;
  len = min(c1 - c0, Nmax);
}

// --- Matrix products with fixed register files ----------------------------------
// The compiler picks one form for every MFMA builtin of a kernel: when a kernel
// may use more than 256 registers, all accumulators go to AGPRs, and scores that
// the vector ALUs must read are then copied out on every tile.  The wrappers below
// state each operand's file instead (S in VGPRs next to the softmax, O in AGPRs,
// Q^T in AGPRs).  The compiler does not model the hazards of an instruction inside
// inline asm, so the code that mixes these with vector code keeps the wait states
// gfx950 requires with the mfma_*_ready helpers:
//   * a vector-ALU read or write of an MFMA result: 16 wait states after the MFMA
//     (the compiler itself inserts 12-13 for this 8-pass instruction);
//   * an MFMA reading a register just written by the vector ALU or by
//     v_accvgpr_write: 4 (the documented need is 2).
// Dependent MFMAs (one accumulating into the result of an earlier one) need no
// wait states of their own.
// acc += a * b; acc in AGPRs, a and b in VGPRs.
__device__ __forceinline__ void mma_a(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// acc = a * b (first product of a chain); acc in VGPRs, a and b in AGPRs.
__device__ __forceinline__ void mma_v_first_aa(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "a"(a), "a"(b));
}
// acc += a * b; acc in VGPRs, a and b in AGPRs.
__device__ __forceinline__ void mma_v_aa(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "a"(a), "a"(b));
}
// 16 bytes of LDS at p (16-byte aligned) straight into AGPRs.  The compiler does not
// count this read: the caller waits for it (s_waitcnt lgkmcnt(0)) before any
// instruction reads dst, and keeps it in order with the products that consume dst
// by issuing those as inline assembly too.
__device__ __forceinline__ void lds_read_a(bf16x8_t& dst, const __bf16* p) {
  const unsigned addr = lds_addr(p);
  asm volatile("ds_read_b128 %0, %1" : "=a"(dst) : "v"(addr) : "memory");
}
// Two 16-byte LDS reads into AGPRs from one address: p and p + OFF bytes (OFF an
// instruction offset).  Same waiting rules as lds_read_a.
template <int OFF>
__device__ __forceinline__ void lds_read_a_pair(bf16x8_t& d0, bf16x8_t& d1, const __bf16* p) {
  const unsigned addr = lds_addr(p);
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:%3" : "=&a"(d0), "=a"(d1) : "v"(addr), "i"(OFF) : "memory");
}
// An MFMA result in VGPRs may now be touched by vector code.
__device__ __forceinline__ void mfma_v_ready1(f32x16_t& x) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(x));
}
// Vector-written MFMA operands in VGPRs may now be read by an MFMA.
__device__ __forceinline__ void valu_ready(bf16x8_t& a, bf16x8_t& b, bf16x8_t& c, bf16x8_t& d) {
  asm volatile("s_nop 3" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

// Accumulator elements whose row index base + crow(g, r) lies outside [lo, hi] become
// -inf.  crow(g, r) = 4g + off(r) with off(r) = 8(r/4) + r%4 a constant per register, so
// each bound is one compare against a per-lane threshold; CHECK_LO = false drops the
// lower bound.  |lo|, |hi| and base stay well inside int range at every call.
template <bool CHECK_LO>
__device__ __forceinline__ void mask_rows(f32x16_t& s, int g, int base, int lo, int hi) {
  const int tlo = lo - base - 4 * g, thi = hi - base - 4 * g;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int off = 8 * (r >> 2) + (r & 3);
    const bool dead = (off > thi) || (CHECK_LO && off < tlo);
    s[r] = dead ? -INFINITY : s[r];
  }
}

constexpr float kLog2e = 1.4426950408889634f;
// Start value of the running max: finite, so that exp2((m_old - m_new) * c) and
// s * c - m * c never form -inf - (-inf) while a row has seen no visible key.
constexpr float kNoMax = -1.0e30f;

}  // namespace fa
