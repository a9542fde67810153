// Device-side building blocks shared by the ditnorm kernels (gfx950 / CDNA4).
//
// bf16 handling: a bf16 value widens to fp32 exactly by a 16-bit shift; fp32
// results round back to bf16 nearest-even with the hardware v_cvt_pk_bf16_f32
// (two values per instruction).  That is the per-op-boundary rounding of the
// eager chain the GLM-Image page describes ("What rounding-faithful means
// here": every elementwise boundary rounds to bf16).
//
// Row statistics are accumulated in binary64.  Sums of bf16 values and of
// their squares are exact (or within 1e-16) in binary64, so the fp32 mean and
// rstd derived from them do not depend on the order of the reduction.  The
// wavefront reductions use DPP lane permutations (quad_perm, row_half_mirror,
// row_mirror) arranged as an xor-butterfly, so that every lane of a group ends
// with the same bits; cross-wave combination goes through LDS in a fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ditnorm {

// --------------------------------------------------------------------------
// bf16 <-> fp32
// --------------------------------------------------------------------------

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round two fp32 values to bf16 (nearest-even) and pack them (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_rn(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Round-trip through bf16: the value an eager bf16 kernel boundary would keep.
// Packing (0, a) puts bf16(a) in the high half above a zero low half, which
// is already the rounded value as fp32: one conversion per value, where
// packing two values costs one conversion and two shift/mask instructions.
__device__ __forceinline__ float round1(float a) { return __uint_as_float(pack_rn(0.0f, a)); }

__device__ __forceinline__ void round2(float &a, float &b) {
  a = round1(a);
  b = round1(b);
}

// 8 bf16 values of a 16-byte vector <-> 8 floats.
__device__ __forceinline__ void unpack8(const uint4 v, float f[8]) {
  f[0] = bf_lo(v.x); f[1] = bf_hi(v.x);
  f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
  f[4] = bf_lo(v.z); f[5] = bf_hi(v.z);
  f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}

__device__ __forceinline__ uint4 pack8(const float f[8]) {
  uint4 v;
  v.x = pack_rn(f[0], f[1]);
  v.y = pack_rn(f[2], f[3]);
  v.z = pack_rn(f[4], f[5]);
  v.w = pack_rn(f[6], f[7]);
  return v;
}

// Opaque to the optimiser: after this the packed value must be re-widened
// where it is used again, instead of keeping every widened copy live across
// a reduction (which would multiply the register footprint).
__device__ __forceinline__ void launder(uint4 &v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// Index of this wavefront within its workgroup, as a wave-uniform (scalar)
// value: the compiler cannot prove threadIdx.x / 64 uniform by itself, and
// would otherwise keep row indices, batch tests and 64-bit address
// arithmetic in vector registers behind exec-mask branches.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// --------------------------------------------------------------------------
// global memory: 16-byte vectors
// --------------------------------------------------------------------------

__device__ __forceinline__ uint4 ld16(const uint16_t *p) {
  return *reinterpret_cast<const uint4 *>(p);
}
__device__ __forceinline__ void st16(uint16_t *p, uint4 v) {
  *reinterpret_cast<uint4 *>(p) = v;
}
__device__ __forceinline__ float4 ld16f(const float *p) {
  return *reinterpret_cast<const float4 *>(p);
}

// Streaming variants for data touched exactly once (activations in and out):
// the nontemporal hint keeps them from displacing reused lines (modulation
// rows, weights) in the caches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16s(const uint16_t *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  uint4 r;
  r.x = v.x; r.y = v.y; r.z = v.z; r.w = v.w;
  return r;
}
__device__ __forceinline__ void st16s(uint16_t *p, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}
// Streaming stores that write through to memory.  A buffer resource over
// the bytes from a wavefront-uniform base, and 16-byte stores at a per-lane
// byte offset from it carrying the streaming hint and device scope (nt sc1):
// the lines go through the L2 instead of sitting in it dirty until the end
// of the kernel.  A plain 16-byte copy of 113 MB measured 19.5 us with
// streaming stores and 18.75 us with these (56 MB: 10.8 -> 10.5 us; 613 MB
// within 0.5%); loads keep the streaming hint alone (device scope on the
// loads measured no faster).  Kernels that compute between their loads and
// stores mostly lose by it (the row kernels 2-13%, the standalone modulate
// 3-5%, the Wan kernels up to 1%), so only the copy, qk_layernorm and the
// backward's d_x use it (about 1% faster each).  The base must be the same
// in every lane: the resource lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wt_rsrc(const void *base) {
  // stride 0, the whole 32-bit offset range, the raw-buffer format word
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, -1, 0x00020000);
}
__device__ __forceinline__ void st16w(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  constexpr int kNtSc1 = 2 | 16;  // cache policy: nt (bit 1), sc1 (bit 4)
  __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)byte_off, 0, kNtSc1);
}

// streaming (NT) or ordinary load, chosen at compile time
template <bool NT>
__device__ __forceinline__ uint4 ld16x(const uint16_t *p) {
  if constexpr (NT) return ld16s(p);
  else return ld16(p);
}

// --------------------------------------------------------------------------
// DPP reductions in binary64
// --------------------------------------------------------------------------

// DPP control codes (GFX9 encoding).
constexpr int DPP_QUAD_XOR1 = 0xB1;      // quad_perm(1,0,3,2)
constexpr int DPP_QUAD_XOR2 = 0x4E;      // quad_perm(2,3,0,1)
constexpr int DPP_ROW_MIRROR = 0x140;    // lane i <- lane 15-i within a row of 16
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i <- lane 7-i within 8 lanes

// Every control code used here reads a valid lane of the same row for every
// lane, so bound_ctrl never applies and no "old" value has to be materialised.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Sum over each aligned group of 4 lanes; every lane of the group gets the
// same bits (each step adds the same two operands, in either order).
__device__ __forceinline__ double sum4(double v) {
  v += dpp_f64<DPP_QUAD_XOR1>(v);
  v += dpp_f64<DPP_QUAD_XOR2>(v);
  return v;
}

// Sum over each aligned group of 8 lanes (quads hold equal values, so the
// half-row mirror pairs quad 0 with quad 1).
__device__ __forceinline__ double sum8(double v) {
  v = sum4(v);
  v += dpp_f64<DPP_ROW_HALF_MIRROR>(v);
  return v;
}

// Sum over each row of 16 lanes, identical in all 16 lanes.
__device__ __forceinline__ double sum16(double v) {
  v = sum8(v);
  v += dpp_f64<DPP_ROW_MIRROR>(v);
  return v;
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the whole wavefront of 64 lanes; uniform result.
__device__ __forceinline__ double sum64(double v) {
  v = sum16(v);
  const double r0 = readlane_f64(v, 0), r1 = readlane_f64(v, 16);
  const double r2 = readlane_f64(v, 32), r3 = readlane_f64(v, 48);
  return (r0 + r1) + (r2 + r3);
}

// Sum over aligned groups of L lanes (L = 4, 8, 16 or 64).
template <int L>
__device__ __forceinline__ double group_sum(double v) {
  static_assert(L == 4 || L == 8 || L == 16 || L == 64, "unsupported group");
  if constexpr (L == 4) return sum4(v);
  else if constexpr (L == 8) return sum8(v);
  else if constexpr (L == 16) return sum16(v);
  else return sum64(v);
}

// --------------------------------------------------------------------------
// 16-bit storage types: DT 0 bf16, 1 fp16.  widen8 is exact; narrow8 rounds
// to nearest even (fp16: overflow to infinity, subnormals kept); round8 is
// the value a storage-type kernel boundary keeps.
// --------------------------------------------------------------------------

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ void widen8(const uint4 v, float f[8]) {
  if constexpr (DT == 0) {
    unpack8(v, f);
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 p = __builtin_convertvector(__builtin_bit_cast(f16x2, w[i]), f32x2);
      f[2 * i] = p.x;
      f[2 * i + 1] = p.y;
    }
  }
}

template <int DT>
__device__ __forceinline__ uint4 narrow8(const float f[8]) {
  if constexpr (DT == 0) {
    return pack8(f);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 p = {f[2 * i], f[2 * i + 1]};
      w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, f16x2));
    }
    uint4 r;
    r.x = w[0]; r.y = w[1]; r.z = w[2]; r.w = w[3];
    return r;
  }
}

// the value a storage-type kernel boundary keeps
// a 16-byte vector as four fp16 pairs, and back
__device__ __forceinline__ void as_f16x2(const uint4 v, f16x2 h[4]) {
  h[0] = __builtin_bit_cast(f16x2, v.x);
  h[1] = __builtin_bit_cast(f16x2, v.y);
  h[2] = __builtin_bit_cast(f16x2, v.z);
  h[3] = __builtin_bit_cast(f16x2, v.w);
}
__device__ __forceinline__ uint4 from_f16x2(const f16x2 h[4]) {
  uint4 v;
  v.x = __builtin_bit_cast(uint32_t, h[0]);
  v.y = __builtin_bit_cast(uint32_t, h[1]);
  v.z = __builtin_bit_cast(uint32_t, h[2]);
  v.w = __builtin_bit_cast(uint32_t, h[3]);
  return v;
}

template <int DT>
__device__ __forceinline__ void round8(float f[8]) {
  const uint4 p = narrow8<DT>(f);
  widen8<DT>(p, f);
}

// --------------------------------------------------------------------------
// workgroup barrier for LDS traffic only (global loads stay in flight)
// --------------------------------------------------------------------------

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// --------------------------------------------------------------------------
// statistics -> the fp32 values the chain consumes
// --------------------------------------------------------------------------

// Single-pass moments.  For bf16 inputs S1 = sum(x) and S2 = sum(x^2) are
// exact in binary64 (a bf16 square has 16 significant bits) unless a row
// spans more than ~2^37 in magnitude, so the mean S1/N is the correctly
// rounded binary64 quotient of the exact sum, and the biased variance
// (S2 - S1*mean)/N loses only the cancellation of S1*mean against S2 (about
// 1e-16 times (mean^2 + var)/var, relative).
struct Moments {
  double s1, s2;
};

__device__ __forceinline__ void accumulate(Moments &m, float x) {
  const double d = (double)x;
  m.s1 += d;
  m.s2 = __builtin_fma(d, d, m.s2);
}

// The variance S2/N - mean*S1/N clamped at 0 against its last-bit rounding
// on near-constant rows.  A comparison, not fmax: a row holding an infinity
// or a NaN has a NaN variance (inf - inf), and fmax would turn it into 0.
__device__ __forceinline__ double clamp_var(double v) { return v < 0.0 ? 0.0 : v; }

// rstd = fp32(1 / sqrt(v)), v = var + eps in binary64 (correctly rounded
// binary64 square root and division, then one rounding to binary32).
__device__ __forceinline__ float rstd_from(double v) {
  return (float)(1.0 / __builtin_sqrt(v));
}

}  // namespace ditnorm
