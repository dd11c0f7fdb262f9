// Device-side helpers for the gfx950 kernels: element widening, MFMA wrappers,
// exp2/log2 and cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fi_internal.h"

namespace fi {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& x) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, x);
}

// 16-byte global loads; the streaming form marks the lines non-temporal (each
// KV byte is read once per call).
__device__ __forceinline__ uint4 load16(const void* p) {
  return bitcast<uint4>(*reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  return bitcast<uint4>(__builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

// ---------------------------------------------------------------------------
// fp8 -> 2-byte widening.
//
// gfx950 converts OCP fp8 natively: v_cvt_scalef32_pk_{f16,bf16}_{fp8,bf8}
// takes two codes (the low or the high 16-bit half of a dword, per word_sel)
// and multiplies by an fp32 scale.  With scale 1.0 the result is the exact
// value: every finite e4m3 / e5m2 value, subnormals included, is representable
// in fp16 and in bf16 (the oracle's tables test this), so no rounding occurs.
// The k / v scales are not applied here but in fp32 (logit scale and output).
// ---------------------------------------------------------------------------
// fnuz codes (the gfx942 layouts: e4m3 bias 8, e5m2 bias 16, no inf, no -0,
// NaN only at 0x80) have no conversion instruction on gfx950; their 2-byte
// form is built from the bits, exactly.  A byte permute puts codes b0, b1 in
// the high bytes of two 16-bit halves (x = b1 << 24 | b0 << 8), sign bits at
// 15 and 31.  Then, per half:
//  * e4m3fnuz: the 7 magnitude bits shifted to bits 13..7 form the fp16 of
//    value * 2^-7 (exponent field e at bias 15 against the code's 8, and the
//    subnormals line up too); the caller folds 2^7 into its scales.
//  * e5m2fnuz: the 7 magnitude bits at 14..8 form the fp16 of 2 * value
//    (bias 15 against 16), infinite where the code's exponent is 31; halving
//    in the integer domain -- one exponent step down for exponent >= 2, a
//    right shift below, i.e. max(sat(mag - 0x400), mag >> 1) -- gives the
//    value exactly, the top binade 2^15 .. 57344 included.
// The NaN code 0x80 (sign set, magnitude zero: the format's only NaN) gives a
// half of exactly 0x8000 after the shifts above; it is turned into the quiet
// NaN 0xFE00, so a NaN stored in an fnuz cache propagates as it does from an
// OCP one.  bf16 is then reached from fp16 exactly (every fnuz value has at
// most 4 significant bits and lies within fp16's range; NaN stays NaN).
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

template <int KVF>
__device__ __forceinline__ uint32_t fnuz2_f16(uint32_t x) {
  uint32_t r;
  if constexpr (KVF == FMT_E4M3_FNUZ) {
    r = ((x >> 1) & 0x3F803F80u) | (x & 0x80008000u);
  } else {
    const u16x2_t mag = bitcast<u16x2_t>(x & 0x7F007F00u);
    const u16x2_t step = {0x0400, 0x0400};
    const u16x2_t m = __builtin_elementwise_max(__builtin_elementwise_sub_sat(mag, step), mag >> (unsigned short)1);
    r = bitcast<uint32_t>(m) | (x & 0x80008000u);
  }
  // the NaN code: a half equal to 0x8000 becomes 0xFE00
  const u16x2_t h = bitcast<u16x2_t>(r);
  const u16x2_t eq = __builtin_convertvector(h == (unsigned short)0x8000, u16x2_t);  // all ones where equal
  const u16x2_t nan_bits = {0x7E00, 0x7E00};
  return r | bitcast<uint32_t>(eq & nan_bits);
}

template <bool QBF16, int KVF>
__device__ __forceinline__ uint2 fnuz4(uint32_t w) {
  uint2 r = make_uint2(fnuz2_f16<KVF>(__builtin_amdgcn_perm(w, w, 0x010c000cu)),
                       fnuz2_f16<KVF>(__builtin_amdgcn_perm(w, w, 0x030c020cu)));
  if constexpr (QBF16) {
    const f16x2_t a = bitcast<f16x2_t>(r.x), b = bitcast<f16x2_t>(r.y);
    const bf16x2_t ab = {(__bf16)(float)a.x, (__bf16)(float)a.y};
    const bf16x2_t bb = {(__bf16)(float)b.x, (__bf16)(float)b.y};
    r = make_uint2(bitcast<uint32_t>(ab), bitcast<uint32_t>(bb));
  }
  return r;
}

// Fast form for e4m3fnuz: apart from 0x7F / 0xFF (+-240, which OCP e4m3
// reads as NaN) and the NaN code 0x80 (which OCP reads as -0) the same bits
// read as OCP e4m3 are exactly twice the fnuz value (bias 7 against 8), so
// the OCP converter with scale 2^-8 gives value * 2^-7 -- bit for bit what
// fnuz4 builds.  The caller checks its codes with e4m3fnuz_outside first.
template <bool QBF16>
__device__ __forceinline__ uint2 widen4_e4m3fnuz_ocp(uint32_t w) {
  constexpr float k = 0.00390625f;  // 2^-8
  uint2 r;
  if constexpr (QBF16) {
    r.x = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, k, false));
    r.y = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, k, true));
  } else {
    r.x = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, k, false));
    r.y = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, k, true));
  }
  return r;
}
// Bit 7 of byte i of the result is set iff byte i of w is 0x7F, 0xFF or 0x80.
// With m = the low 7 bits of each byte (no byte carries out of the sums
// below): m + 1 reaches bit 7 iff m is all ones (+-240); m + 0x7F reaches bit
// 7 iff m is nonzero, so a set sign bit without it is the NaN code.
__device__ __forceinline__ uint32_t e4m3fnuz_outside(uint32_t w) {
  const uint32_t m = w & 0x7F7F7F7Fu;
  return ((m + 0x01010101u) | (w & ~(m + 0x7F7F7F7Fu))) & 0x80808080u;
}

// Fast form for e5m2fnuz: a code whose exponent field is 2 or more, with
// that field lowered by one (4 subtracted from the byte), reads as OCP e5m2
// (bias 15 against 16) with exactly the fnuz value -- the top binade, which
// OCP keeps for inf/NaN, included; the zero code 0x00 stays as it is.  Codes
// with exponent 0 or 1 and a nonzero magnitude (below 2^-14: tiny values)
// have no such reading, nor has the NaN code 0x80 (OCP reads it as -0); the
// caller checks for them with e5m2fnuz_outside first.
__device__ __forceinline__ uint32_t e5m2fnuz_big(uint32_t w) {  // bit 7 of a byte: exponent >= 2
  return ((w & 0x78787878u) + 0x78787878u) & 0x80808080u;
}
// bit 7 of a byte: a nonzero magnitude with exponent 0/1, or the NaN code
// (magnitude zero, sign set) -- per byte, nonzero ? !big : sign
__device__ __forceinline__ uint32_t e5m2fnuz_outside(uint32_t w) {
  const uint32_t nz = (w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu;
  return ((nz & ~e5m2fnuz_big(w)) | (~nz & w)) & 0x80808080u;
}
template <bool QBF16>
__device__ __forceinline__ uint2 widen4_e5m2fnuz_ocp(uint32_t w) {
  const uint32_t x = w - (e5m2fnuz_big(w) >> 5);
  uint2 r;
  if constexpr (QBF16) {
    r.x = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(x, 1.0f, false));
    r.y = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(x, 1.0f, true));
  } else {
    r.x = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_bf8(x, 1.0f, false));
    r.y = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_bf8(x, 1.0f, true));
  }
  return r;
}

// Either fnuz format: the test for codes outside the OCP reading, and the
// fast widening valid for all other codes.
template <int KVF>
__device__ __forceinline__ uint32_t fnuz_outside_ocp(uint32_t w) {
  if constexpr (KVF == FMT_E4M3_FNUZ)
    return e4m3fnuz_outside(w);
  else
    return e5m2fnuz_outside(w);
}
template <bool QBF16, int KVF>
__device__ __forceinline__ uint2 widen4_fnuz_ocp(uint32_t w) {
  if constexpr (KVF == FMT_E4M3_FNUZ)
    return widen4_e4m3fnuz_ocp<QBF16>(w);
  else
    return widen4_e5m2fnuz_ocp<QBF16>(w);
}

// The two word_sel immediates must be compile-time constants.
template <bool QBF16, int KVF>
__device__ __forceinline__ uint2 widen4(uint32_t w) {
  if constexpr (KVF == FMT_E4M3_FNUZ || KVF == FMT_E5M2_FNUZ) return fnuz4<QBF16, KVF>(w);
  uint2 r;
  if constexpr (!QBF16) {
    if constexpr (KVF == FMT_E4M3) {
      r.x = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
      r.y = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
    } else {
      r.x = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, false));
      r.y = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, true));
    }
  } else {
    if constexpr (KVF == FMT_E4M3) {
      r.x = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
      r.y = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
    } else {
      r.x = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, false));
      r.y = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, true));
    }
  }
  return r;
}

// 8 fp8 codes (two dwords) -> one MFMA operand of 8 2-byte values.
template <bool QBF16, int KVF>
__device__ __forceinline__ uint4 widen8(uint32_t lo, uint32_t hi) {
  uint2 a = widen4<QBF16, KVF>(lo);
  uint2 b = widen4<QBF16, KVF>(hi);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// Exact split of fp16 values into bf16 pairs: v == hi + lo with hi = bf16(v)
// (round to nearest even) and lo = bf16(v - hi).  An fp16 value has 11
// significant bits; hi keeps 8 and the residual has at most 3, so lo holds it
// exactly, and bf16's exponent range covers every fp16 value.  Used when an
// fp16 operand meets a bf16 one (mixed 2-byte decode): the MFMA runs in bf16 on
// hi and lo, so no value is rounded and none can overflow.
__device__ __forceinline__ void split_f16x2(uint32_t w, uint32_t& hi, uint32_t& lo) {
  const f16x2_t h = bitcast<f16x2_t>(w);
  const float a = (float)h.x, b = (float)h.y;
  const __bf16 ah = (__bf16)a, bh = (__bf16)b;
  const bf16x2_t vh = {ah, bh};
  const bf16x2_t vl = {(__bf16)(a - (float)ah), (__bf16)(b - (float)bh)};
  hi = bitcast<uint32_t>(vh);
  lo = bitcast<uint32_t>(vl);
}

__device__ __forceinline__ void split_f16x8(uint4 x, uint4& hi, uint4& lo) {
  split_f16x2(x.x, hi.x, lo.x);
  split_f16x2(x.y, hi.y, lo.y);
  split_f16x2(x.z, hi.z, lo.z);
  split_f16x2(x.w, hi.w, lo.w);
}

// ---------------------------------------------------------------------------
// LDS transposed reads (gfx950).  Within each group of 16 lanes:
//  * lds_tr8  (ds_read_b64_tr_b8):  lanes 2r and 2r+1 give the addresses of the
//    two 8-byte halves of row r (r = 0..7); lane i receives byte column i of
//    the 8 rows, row r in byte r.
//  * lds_tr16 (ds_read_b64_tr_b16): lanes 4r..4r+3 give the four 8-byte pieces
//    of row r (r = 0..3); lane i receives 16-bit column i of the 4 rows.
// Rows are whatever the addresses name, so any token order can be gathered.
// ---------------------------------------------------------------------------
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 lds_tr8(const uint8_t* p) {
  const i32x2_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(p));
  return bitcast<uint2>(r);
}
__device__ __forceinline__ uint2 lds_tr16(const uint8_t* p) {
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
  return bitcast<uint2>(r);
}

// ---------------------------------------------------------------------------
// MFMA wrappers (operands as raw dwords).
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ f32x4_t mfma16x16x32(uint4 a, uint4 b, f32x4_t c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(a), bitcast<bf16x8_t>(b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8_t>(a), bitcast<f16x8_t>(b), c, 0, 0, 0);
  }
}

template <bool BF16>
__device__ __forceinline__ f32x4_t mfma16x16x16(uint2 a, uint2 b, f32x4_t c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bitcast<i16x4_t>(a), bitcast<i16x4_t>(b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(bitcast<f16x4_t>(a), bitcast<f16x4_t>(b), c, 0, 0, 0);
  }
}

template <bool BF16>
__device__ __forceinline__ f32x16_t mfma32x32x16(uint4 a, uint4 b, f32x16_t c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8_t>(a), bitcast<bf16x8_t>(b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<f16x8_t>(a), bitcast<f16x8_t>(b), c, 0, 0, 0);
  }
}

// fp8 x fp8 -> fp32, 32x32 outputs over k = 64 (v_mfma_f32_32x32x64_f8f6f4,
// unscaled).  Each lane supplies 32 bytes of A (row lane % 32) and of B
// (column lane % 32); A and B share the assignment of (lane / 32, byte) to k,
// so any split of the 64 k positions works as long as both operands use it.
// The output layout is that of the 16-bit 32x32 MFMAs.  FA / FB name the
// operands' formats (FMT_E4M3 or FMT_E5M2).
typedef int i32x8_t __attribute__((ext_vector_type(8)));

template <int FA, int FB>
__device__ __forceinline__ f32x16_t mfma32x32x64_f8(uint4 a0, uint4 a1, uint4 b0, uint4 b1, f32x16_t c) {
  const i32x8_t a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8_t b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA == FMT_E5M2 ? 1 : 0, FB == FMT_E5M2 ? 1 : 0, 0, 0,
                                                         0, 0);
}

// ---------------------------------------------------------------------------
// Scalars
// ---------------------------------------------------------------------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
// A row's sum of probabilities is +0 (no visible key), positive, or NaN (a
// NaN read from the cache).  The test reads the bits through an empty asm
// statement: in code compiled with NaNs assumed absent the compiler would
// otherwise fold a test of the bits (it can prove the sum is never -0) into
// an ordered float compare, which takes NaN for +0.
__device__ __forceinline__ bool has_weight(float l) {
  uint32_t b = __float_as_uint(l);
  asm volatile("" : "+v"(b));
  return b != 0u;
}

// Round an fp32 to q's 2-byte type and return (bits, value as fp32).
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (BF16) {
    bf16x2_t r = {(__bf16)a, (__bf16)b};
    return bitcast<uint32_t>(r);
  } else {
    f16x2_t r = {(_Float16)a, (_Float16)b};
    return bitcast<uint32_t>(r);
  }
}

// c + w.lo + w.hi for a packed pair of 2-byte values, summed in fp32
// (v_dot2_f32_{f16,bf16} against (1, 1): the products are exact)
template <bool BF16>
__device__ __forceinline__ float sum2(uint32_t w, float c) {
  if constexpr (BF16) {
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(w), one, c, false);
  } else {
    const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(bitcast<f16x2_t>(w), one, c, false);
  }
}

template <bool BF16>
__device__ __forceinline__ float2 unpack2(uint32_t w) {
  if constexpr (BF16) {
    return make_float2(bitcast<float>(w << 16), bitcast<float>(w & 0xffff0000u));
  } else {
    f16x2_t h = bitcast<f16x2_t>(w);
    return make_float2((float)h.x, (float)h.y);
  }
}

template <bool BF16>
__device__ __forceinline__ uint16_t to_bits(float a) {
  if constexpr (BF16) {
    return bitcast<uint16_t>((__bf16)a);
  } else {
    return bitcast<uint16_t>((_Float16)a);
  }
}

// Cross-lane max / sum over lanes l, l^16, l^32, l^48 (ds_swizzle-free: bpermute).
// A value the caller knows to be equal on every lane of the wave, moved to a
// scalar register so that branches on it are scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Max / sum of v and v from the lane 32 away, through v_permlane32_swap (a
// register exchange between the wave's halves: no LDS round trip).  With both
// operands v, the two results are v and its partner in the same order on
// every lane, so both halves compute the identical value.
__device__ __forceinline__ float max_half_swap(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_half_swap(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float xor_max(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask)); }
__device__ __forceinline__ float xor_sum(float v, int mask) { return v + __shfl_xor(v, mask); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

}  // namespace fi
