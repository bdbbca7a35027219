// Device helpers shared by the gfx950 kernels: vector types, MFMA wrappers,
// 8-bit conversions, 16-bit packing.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lamp {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// MFMA 32x32 wrappers.  Operand layout (all of them): lane l holds row/column
// (l % 32) and one contiguous run of the reduction index selected by l / 32.
// The kernels only rely on A and B sharing that mapping.  Output layout:
// lane l, register i -> column l % 32, row 8*(i/4) + 4*(l/32) + (i%4).
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

__device__ __forceinline__ i32x16 mfma_i8(u32x4 a, u32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                               __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// Wait states after the last v_mfma_scale_f32_32x32x64_f8f6f4 of a chain
// before its result is read.  With fp8 operands the instruction takes 16
// passes; hipcc (ROCm 7.2) lets a v_accvgpr_read of the result follow 12
// wait states after it, which returned stale accumulator values on MI355X.
// The scheduling barriers keep every read behind the 20 explicit wait states.
__device__ __forceinline__ void xdl16_settle() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n\ts_nop 3");
  __builtin_amdgcn_sched_barrier(0);
}

// OCP e4m3 x e4m3, K = 64, unit block scales (E8M0 127 = 2^0).
__device__ __forceinline__ f32x16 mfma_e4m3(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x16 c) {
  i32x8 a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  i32x8 b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// The same product with a power-of-two scale 2^(sa - 127) on operand A (sa
// is the E8M0 code, i.e. the biased exponent field of an fp32 power of two).
__device__ __forceinline__ f32x16 mfma_e4m3_sa(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x16 c,
                                               int sa) {
  i32x8 a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  i32x8 b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, 127);
}

// ---------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------

// four fp32 -> four OCP e4m3 codes, a in byte 0 .. d in byte 3
// (round-to-nearest-even; callers keep |x| <= 448 so no value saturates or
// overflows).  The second conversion writes the upper half of the first's
// result.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  // the high half of the first word is overwritten by the second conversion,
  // so any dead value serves as its old contents (saves a register clear)
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// e4m3 codes in bytes 2 HI, 2 HI + 1 -> two fp32 (exact)
template <bool HI>
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t codes) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, HI);
}

// e4m3 codes in bytes 2 HI, 2 HI + 1 -> two packed 16-bit values (exact:
// every e4m3 value is a bf16 and an fp16 value; scale 1)
template <bool BF16, bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_16(uint32_t codes) {
  if constexpr (BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)codes, 1.f, HI));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)codes, 1.f, HI));
  }
}

template <bool BF16>
__device__ __forceinline__ uint32_t pack16x2(float a, float b) {
  if constexpr (BF16) {
    bf16x2 r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
  } else {
    f16x2 r = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, r);
  }
}

template <bool BF16>
__device__ __forceinline__ float from16(uint32_t bits16) {
  if constexpr (BF16) {
    return __builtin_bit_cast(float, bits16 << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  }
}

// c + lo + hi of two packed 16-bit values (v_dot2c_f32_{bf16,f16} with the
// multiplier pair (1, 1): the products are exact).
template <bool BF16>
__device__ __forceinline__ float sum16x2(uint32_t v, float c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v),
                                           __builtin_bit_cast(bf16x2, 0x3F803F80u), c, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, v), __builtin_bit_cast(f16x2, 0x3C003C00u),
                                  c, false);
  }
}

// int32 accumulators started at kMagicBits hold the float kMagic + acc for
// |acc| < 2^22 (floats in [2^23, 2^24) have unit spacing).
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23

// c >= 0 rounded to 21 significant bits (ties away from zero).  kMagic * c is
// then exact in fp32: 3 * c needs at most 23 significant bits and 2^22 only
// moves the exponent.  The relative change of c is at most 2^-21.
__device__ __forceinline__ float round_sig21(float c) {
  return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, c) + 4u) & ~7u);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// memory helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld_lds16(const char* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st_lds16(char* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st_lds8(char* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane i's 16 bytes land at lds_base + 16 * i, lds_base being wave-uniform.
// Completion is tracked by vmcnt like any global load.
__device__ __forceinline__ void dma16(const void* gsrc, char* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// Wait until every outstanding vector-memory operation of this wave (loads,
// stores and direct-to-LDS copies) has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// result lane 4a + j receives element j of the 8-byte reads of source lanes
// a, a + 4, a + 8, a + 12 (in that order): a 4x4 transpose of 16-bit values.
__device__ __forceinline__ u32x2 ld_lds_tr16(const char* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
  return __builtin_bit_cast(u32x2, r);
}

// Load of a wave-uniform value that nothing writes during the kernel, through
// the constant address space: the compiler emits a scalar load.
template <class T>
__device__ __forceinline__ T ld_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// x of the lane in the other 32-lane half (lane l gets x[l ^ 32]).
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; with x in both operands the lower-half lanes
// find x[l + 32] in the second result and the upper-half lanes x[l - 32] in
// the first, whether or not the compiler gives both operands one register.
__device__ __forceinline__ float other_half(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto pr = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r = (__lane_id() & 32) ? pr[0] : pr[1];
  return __builtin_bit_cast(float, r);
}
__device__ __forceinline__ float halves_max(float x) { return fmaxf(x, other_half(x)); }
__device__ __forceinline__ float halves_sum(float x) { return x + other_half(x); }

// Raw buffer resource over [base, base + bytes): buffer loads at offsets at
// or beyond `bytes` return zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Direct buffer -> LDS copy of 16 bytes per lane at byte offset voff + soff;
// lane i's bytes land at lds_base + 16 * i.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                          char* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                           voff, soff, 0, 0);
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

// 8-bit exponential of one e4m3 code c (LampAttention, Abstract: exponentials
// in 8-bit formats): E4M3(exp(value(c))), the value decoded by the hardware
// conversion, exp taken through exp2, the result rounded to e4m3.  Code 0xFF,
// which the fp32 -> e4m3 conversion gives logits below -464, -inf and NaN,
// weighs 0, as a logit clamped to -448 would (its exponential is below half
// the smallest e4m3 subnormal).
__device__ __forceinline__ uint32_t exp8_code(uint32_t c) {
  if (c == 0xFFu) return 0u;
  const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
  const int r = __builtin_amdgcn_cvt_pk_fp8_f32(exp2_fast(v.x * kLog2e), 0.f, 0, false);
  return (uint32_t)r & 0xFFu;
}

}  // namespace lamp
