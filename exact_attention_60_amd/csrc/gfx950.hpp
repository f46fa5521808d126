// gfx950 (CDNA4) building blocks shared by the attention kernels.
//
// Lane layouts relied on (wave64; verified on the device by a layout probe):
//  * v_mfma_f32_32x32x16_bf16: A operand lane l holds A[l%32][k-slots of half
//    l/32], B operand lane l holds B[k-slots of half l/32][l%32], the k-slots
//    being the same for A and B; accumulator register r of lane l holds
//    C[8*(r/4) + 4*(l/32) + r%4][l%32].
//  * ds_read_b64_tr_b16: in each group of 16 lanes, lane j receives element
//    j%4 of the 4-element (64-bit) row addressed by lane 4*e + j/4, for
//    e = 0..3.
//  * v_permlane32_swap with both operands equal returns the lower half of the
//    wave broadcast to both halves (first result) and the upper half (second).
//  * the float -> bf16 conversion (v_cvt_pk_bf16_f32) rounds to nearest even.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

namespace attn {

// Causal launch order.  Workgroups are dealt to the 8 XCDs round robin
// (XCD = i % 8).  Workgroup i gets head h in [0, NH) and query tile qt so that
// each XCD takes NH / 8 whole heads (every K/V tile of a head is then read
// through one L2), and within an XCD the 32 heaviest query tiles of one head
// come first -- one per CU of the XCD, all streaming the same K/V tiles at
// the same time -- then those of the XCD's next head, then the next 32 tiles
// of each head, down to the lightest.  NH must be a multiple of 8 and the
// grid NH * n_qt workgroups.
__device__ __forceinline__ void causal_xcd_order(int i, int NH, int n_qt, int& h, int& qt) {
  constexpr int BAND = 32;
  const int x = i & 7, j = i >> 3;
  const int hpx = NH >> 3;               // heads per XCD
  const int full = n_qt / BAND;          // full bands of 32 tiles
  const int in_full = full * hpx * BAND;
  int hl, row;
  if (j < in_full) {
    const int band = j / (hpx * BAND);
    const int r = j - band * hpx * BAND;
    hl = r / BAND;
    row = band * BAND + (r - hl * BAND);
  } else {
    const int t = j - in_full;
    const int rows_t = n_qt - full * BAND;
    hl = t / rows_t;
    row = full * BAND + (t - hl * rows_t);
  }
  h = x * hpx + hl;
  qt = n_qt - 1 - row;
}


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define ATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Value of lane (l ^ 32), for a wave64.
__device__ __forceinline__ float xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const bool upper = (threadIdx.x & 32) != 0;
  return __uint_as_float(upper ? r[0] : r[1]);
}
__device__ __forceinline__ float max_halves(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}
// bf16 bits of x (in the upper half of the result) by integer arithmetic on
// the sign-magnitude encoding: adding HALF (0x8000, half a bf16 spacing, for
// RTNA; 0 for RTZ) to the magnitude and dropping the low 16 bits.  With
// 0x8000 a tie carries into the kept bits, i.e. away from zero, and values from
// half a spacing past the largest finite bf16 carry into the exponent and give
// inf; with 0 it is truncation.  NaN becomes the quiet NaN 0x7FC0 with x's
// sign.
template <uint32_t HALF>
__device__ __forceinline__ uint32_t bf16_bits_hi(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t nan = (u & 0x80000000u) | 0x7fc00000u;
  return ((u & 0x7fffffffu) > 0x7f800000u ? nan : u + HALF) & 0xffff0000u;
}
// two floats -> packed bf16 under the rounding rule MODE (kRound*)
template <int MODE>
__device__ __forceinline__ uint32_t pack_bf16_as(float lo, float hi) {
  if constexpr (MODE == kRoundRTNE) {
    return pack_bf16(lo, hi);
  } else {
    constexpr uint32_t half = MODE == kRoundRTNA ? 0x8000u : 0u;
    return (bf16_bits_hi<half>(lo) >> 16) | bf16_bits_hi<half>(hi);
  }
}
// Calls f(std::integral_constant<int, MODE>) for the run-time rule `mode`, so
// that the conversion code is chosen once, outside the caller's loops.
template <class F>
__device__ __forceinline__ void with_rounding(int mode, F&& f) {
  if (mode == kRoundRTNA) f(std::integral_constant<int, kRoundRTNA>{});
  else if (mode == kRoundRTZ) f(std::integral_constant<int, kRoundRTZ>{});
  else f(std::integral_constant<int, kRoundRTNE>{});
}
// two floats -> packed fp16 (v_cvt_pk_f16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), f16x2));
}
// The row sums below avoid the dot-product instructions (v_dot2*): measured
// on gfx950, a dot instruction of one wave waits for the matrix core while
// another wave of the SIMD runs MFMAs (about 70 cycles each instead of 5),
// whereas ordinary VALU instructions, v_fma_mix_f32 included, issue beside
// them.
// sum of the two fp16 halves of u added to acc in fp32: each half widened
// exactly and added with one rounding (v_fma_mix_f32 with 1.0: lo, then hi)
__device__ __forceinline__ float sum2_f16(uint32_t u, float acc) {
  float r, t;
  asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(t) : "v"(u), "v"(acc));
  asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(u), "v"(t));
  return r;
}
// sum of the two bf16 halves of u added to acc in fp32 (each half widened
// exactly by a shift or mask)
__device__ __forceinline__ float sum2_bf16(uint32_t u, float acc) {
  return (acc + __uint_as_float(u << 16)) + __uint_as_float(u & 0xffff0000u);
}
// two bf16 (packed in u) -> two fp16 (packed); exact for |x| in the fp16
// normal range, |x| >= 65520 becomes +-inf
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t u) {
  return pack_f16(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}

// One 1 KB asynchronous copy (buffer_load_dwordx4 ... lds): lane i's 16 bytes
// at byte offset voff of the buffer land at LDS byte lds + 16*i.  Written as
// an asm statement so that the compiler does not see an LDS write in flight:
// it would otherwise wait for every outstanding copy before the wave's next
// LDS read, and a copy could not stay in flight across the wave's operand
// reads.  The callers order the copies with explicit vmcnt waits and
// barriers (vector memory loads complete in order).  M0 holds the LDS
// address (one wait state before the copy reads it).
__device__ __forceinline__ void lds_copy16_at(const u32x4& rsrc, uint32_t voff, uint32_t lds_addr) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
// the same with the LDS destination as a pointer into __shared__ memory
__device__ __forceinline__ void lds_copy16(const u32x4& rsrc, uint32_t voff, const char* lds) {
  lds_copy16_at(rsrc, voff, (uint32_t)(uintptr_t)(const ATTN_LDS char*)lds);
}

// Buffer descriptor: base address, no stride, nrec bytes, raw dword access.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* p, uint32_t nrec) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, nrec, 0x00020000u};
}

// p must point into __shared__ memory (8-byte aligned).
__device__ __forceinline__ bf16x4 lds_read_tr(const void* p) {
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(p));
  return __builtin_bit_cast(bf16x4, t);
}

// True if any lane of the wave has `pred` set (wave-uniform result).
__device__ __forceinline__ bool wave_any(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred) != 0;
}

}  // namespace attn
