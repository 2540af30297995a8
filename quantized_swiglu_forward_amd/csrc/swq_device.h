// Device helpers shared by the HIP kernels of the fused quantized SwiGLU.
//
// Dequantization scheme.  A weight is w = s*q + b (affine group quantization;
// "mlx-bun 0.0.7 -> 0.0.9" diff, page 42, gemma4-base.ts QuantizedLinear and
// fused-swiglu-kernel.ts support predicate).  The kernels rewrite it as
//
//     w = s*(q - z) + (b + z*s),        z = 8 for 4-bit codes
//     w = 16s*(hi - 8) + s*(lo - 8) + (b + 136*s)   for 8-bit codes q = 16*hi + lo
//
// Every code offset (q - 8), (hi - 8), (lo - 8) lies in [-8, 7], so with a
// bf16 scale (8 significant bits) the product s*(q - 8) has at most 11
// significant bits and is EXACT in binary16 as long as |s| is in
// [2^-17, 2^8).  The sum over K therefore runs on f16 MFMA / dot2 with exact
// products and float32 accumulation, and the per-group constant (b + z*s)
// multiplies the per-group sum of x, which is carried separately.
//
// Code extraction places a nibble into the mantissa of a binary16 "magic"
// number: nibble bits [0,4) OR 0x6400 is 1024 + q, nibble bits [4,8) OR 0x5400
// is 64 + q.  Subtracting 1032 or 72 (exact) gives q - 8.  A 32-bit word
// holds two f16 lanes, so one AND/OR pair extracts two codes at once; the
// pairs come out as (code j, code j+4) of an 8-code block, and every x
// operand is stored in the matching order [0,4,1,5,2,6,3,7] within each
// block of 8 consecutive k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swq {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float round_to_bf16(float f) {
  return bf16_to_f32(f32_to_bf16(f));
}

// Activation types: bf16 (swiglu_q_forward) or binary16 (swiglu_q_forward_f16)
// for x, the scales and biases, and the 16-bit output.
enum : int { kActBf16 = 0, kActF16 = 1 };

__device__ __forceinline__ float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint16_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ float act_to_f32(uint16_t b, int act) {
  return act == kActF16 ? f16_to_f32(b) : bf16_to_f32(b);
}
__device__ __forceinline__ uint16_t f32_to_act(float f, int act) {
  return act == kActF16 ? f32_to_f16(f) : f32_to_bf16(f);
}
__device__ __forceinline__ float round_to_act(float f, int act) {
  return act == kActF16 ? (float)(_Float16)f : round_to_bf16(f);
}

// Exponent e of a row's (or chunk's) largest magnitude, from its bits without
// the sign (bf16: 8-bit exponent field; binary16: 5-bit), so that x 2^-e lies
// below 2 and its largest element in [1, 2) (a subnormal maximum: e one
// below the smallest normal exponent, x 2^-e still below 2), an all-zero row 0.
__device__ __forceinline__ int x_exponent(uint32_t amax_bits, int act) {
  if (amax_bits == 0) return 0;
  if (act == kActF16) {
    const int field = (int)(amax_bits >> 10);
    return field == 0 ? -15 : field - 15;
  }
  const int field = (int)(amax_bits >> 7);
  return field == 0 ? -127 : field - 127;
}

// A binary16 scale (times its row's 2^-k) as two parts for two MFMA planes:
// hi = s rounded to 8 significant bits, lo = s - hi (exact, at most 3
// significant bits), so that hi (q - z) and lo (q - z) are each exact in
// binary16 where a bf16 scale's product is (lo: 8-bit codes too).
__device__ __forceinline__ f16x2 split_scale(float s) {
  const float hi = round_to_bf16(s);
  return (f16x2){(_Float16)hi, (_Float16)(s - hi)};
}

__device__ __forceinline__ f16x2 as_h2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// bf16 value -> (v, v) as two binary16 lanes (exact inside the documented range).
__device__ __forceinline__ f16x2 bf16_to_h2(uint16_t b) {
  _Float16 h = (_Float16)bf16_to_f32(b);
  return (f16x2){h, h};
}

// Nibble masks and f16 magic numbers of the unpack: a nibble in bits [0,4)
// of a binary16 lane ORed with 0x6400 is 1024 + q; in bits [4,8) ORed with
// 0x5400 it is 64 + q.  As literals (the default) or, from
// nibble_consts_in_regs(), in registers: then each mask-and-OR is one
// v_and_or_b32 (a VOP3 instruction cannot take two literals on this target).
struct NibbleK {
  uint32_t m_lo, m_hi, g_lo, g_hi;
};
constexpr NibbleK kNibbleLiterals = {0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x54005400u};
__device__ __forceinline__ NibbleK nibble_consts_in_regs() {
  NibbleK k;
  asm volatile("s_mov_b32 %0, 0xf000f" : "=s"(k.m_lo));
  asm volatile("s_mov_b32 %0, 0xf000f0" : "=s"(k.m_hi));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(k.g_lo));
  asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(k.g_hi));
  return k;
}

// Eight 4-bit codes of one word -> s*(q-8) as four f16 pairs in the order
// (q0,q4) (q1,q5) (q2,q6) (q3,q7).
__device__ __forceinline__ void dequant4(uint32_t w, f16x2 s2, uint32_t out[4], const NibbleK& k = kNibbleLiterals) {
  const f16x2 c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2 c72 = {(_Float16)72.0f, (_Float16)72.0f};
  const uint32_t w8 = w >> 8;
  f16x2 p0 = as_h2((w & k.m_lo) | k.g_lo) - c1032;
  f16x2 p1 = as_h2((w & k.m_hi) | k.g_hi) - c72;
  f16x2 p2 = as_h2((w8 & k.m_lo) | k.g_lo) - c1032;
  f16x2 p3 = as_h2((w8 & k.m_hi) | k.g_hi) - c72;
  out[0] = as_u32(p0 * s2);
  out[1] = as_u32(p1 * s2);
  out[2] = as_u32(p2 * s2);
  out[3] = as_u32(p3 * s2);
}

// Eight 4-bit codes of one word -> (q-8) as four f16 pairs, same order, no scale.
__device__ __forceinline__ void codes4(uint32_t w, uint32_t out[4]) {
  const f16x2 c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2 c72 = {(_Float16)72.0f, (_Float16)72.0f};
  const uint32_t w8 = w >> 8;
  out[0] = as_u32(as_h2((w & 0x000F000Fu) | 0x64006400u) - c1032);
  out[1] = as_u32(as_h2((w & 0x00F000F0u) | 0x54005400u) - c72);
  out[2] = as_u32(as_h2((w8 & 0x000F000Fu) | 0x64006400u) - c1032);
  out[3] = as_u32(as_h2((w8 & 0x00F000F0u) | 0x54005400u) - c72);
}

// Eight 8-bit codes in two words (wa: codes 0..3, wb: codes 4..7) -> the low
// and high nibble planes (lo-8) and (hi-8) as f16 pairs in the order
// (c0,c4) (c1,c5) (c2,c6) (c3,c7).  v_perm_b32 gathers byte j of wa and byte j
// of wb into bytes 0 and 2 of one register.  With `full`, also the whole
// codes q - 136 (a byte ORed with 0x6400 is 1024 + q; exact in binary16).
__device__ __forceinline__ void codes8(uint32_t wa, uint32_t wb, uint32_t lo[4], uint32_t hi[4],
                                       const NibbleK& k = kNibbleLiterals, uint32_t* full = nullptr) {
  const f16x2 c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2 c72 = {(_Float16)72.0f, (_Float16)72.0f};
  const f16x2 c1160 = {(_Float16)1160.0f, (_Float16)1160.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + j) << 16) | (uint32_t)j;
    const uint32_t t = __builtin_amdgcn_perm(wb, wa, sel);
    lo[j] = as_u32(as_h2((t & k.m_lo) | k.g_lo) - c1032);
    hi[j] = as_u32(as_h2((t & k.m_hi) | k.g_hi) - c72);
    if (full) full[j] = as_u32(as_h2((t & 0x00FF00FFu) | 0x64006400u) - c1160);
  }
}

// 2-bit codes run through the 4-bit arithmetic: the eight 2-bit fields of
// a 16-bit block (code j in bits [2j, 2j+2)) spread to eight nibbles of a
// word (code j in bits [4j, 4j+4)), the 4-bit layout.  A code q <= 3 is a
// 4-bit code too, and s*(q - 8) stays exact in binary16.
__device__ __forceinline__ uint32_t spread2(uint32_t b16) {
  uint32_t v = b16 & 0xFFFFu;
  v = (v | (v << 8)) & 0x00FF00FFu;
  v = (v | (v << 4)) & 0x0F0F0F0Fu;
  v = (v | (v << 2)) & 0x33333333u;
  return v;
}

// Width at which a code is computed: 2-bit codes as 4-bit ones.
template <int BITS>
inline constexpr int kCodeWidth = BITS == 2 ? 4 : BITS;

// Offset z of the rewrite w = s*(q - z) + (b + z*s).
template <int BITS>
struct CodeOffset;
template <>
struct CodeOffset<2> { static constexpr float z = 8.0f; };
template <>
struct CodeOffset<4> { static constexpr float z = 8.0f; };
template <>
struct CodeOffset<8> { static constexpr float z = 136.0f; };

// Weight-row exponent.  Every kernel that forms binary16 operands s (q - z)
// and c = b + z s first multiplies a row's scales and constants by a power
// of two 2^-k of its own: with m the largest over the row's groups of
// |s| F and |c| (F the largest code offset times its plane weight: 8 for
// codes of at most 4 bits, 128 for the 8-bit high plane 16 (hi - 8)) and m in
// [2^E, 2^(E+1)), k = E - 14.  Every operand is then below 2^15 (finite in
// binary16), the largest in [2^14, 2^15), and the row's sums are multiplied
// by 2^k at the end.  A group whose own largest term is at least 2^-28 (8-bit:
// 2^-24) of m keeps s 2^-k at or above 2^-17, where its 8 significant bits
// times an offset of at most 3 significant bits are exact in binary16.
template <int BITS>
inline constexpr float kPlaneMax = kCodeWidth<BITS> == 8 ? 128.0f : 8.0f;

__device__ __forceinline__ float group_term_max(float s, float b, float z, float F) {
  return fmaxf(fabsf(s) * F, fabsf(fmaf(z, s, b)));
}

__device__ __forceinline__ int row_exponent_k(float m) {
  if (!(m > 0.0f)) return 0;
  const int E = __builtin_amdgcn_frexp_expf(m) - 1;     // m in [2^E, 2^(E+1))
  return min(max(E - 14, -200), 200);
}

// silu(g) u = g sigma(g) u with sigma(g) = 1 / (1 + 2^b), b = -g log2(e),
// from the hardware exp2 and reciprocal (about 1 ulp each).  Past b = 64
// (g < -44.4) the 1 in the denominator is below float32's resolution, so
// sigma(g) = 2^-b to within 2^-64, taken as 2^64 rcp(2^(b - 64)): the
// reciprocal stays a normal number down to b = 190 (g = -131.7), where
// sigma(g) itself has long left float32's normal range, and the product
// leaves that range only at its last step, one rounding (float32's own
// subnormals).  Below b = 190 the true value is under half float32's
// smallest subnormal whenever |g u| < 2^40.
__device__ __forceinline__ float silu_times(float g, float u) {
  const float b = g * -1.4426950408889634f;
  const bool deep = b > 64.0f;
  const float e = __builtin_amdgcn_exp2f(b - (deep ? 64.0f : 0.0f));
  const float r = __builtin_amdgcn_rcpf(e + (deep ? 0.0f : 1.0f));
  return ldexpf(g * r * u, deep ? -64 : 0);
}

// Debug build (-DSWQ_LDS_POISON): every kernel fills its LDS with a poison
// pattern before using it -- NaN bits for floating-point data, 2^30 for
// integer exponents -- so that a read of LDS the kernel did not write first
// shows in its results (the pages' threadgroup-zeroing diagnostic, with a
// pattern that cannot pass for data).  The product build has none of it.
#ifdef SWQ_LDS_POISON
constexpr uint32_t kPoisonFloat = 0xFFFFFFFFu;   // NaN as float32 and as binary16 pairs
constexpr uint32_t kPoisonExp = 0x40000000u;     // an exponent of 2^30
__device__ __forceinline__ void lds_poison(void* p, size_t bytes, uint32_t pattern) {
  for (size_t i = threadIdx.x; i < bytes / 4; i += blockDim.x) reinterpret_cast<uint32_t*>(p)[i] = pattern;
}
#endif

// Precision modes (values fixed by the public header).
enum : int { kMatch = 0, kF32 = 1, kF32Bf16Out = 2 };
// (the linear's epilogue kinds kLinBf16 / kLinF32 are in swq_kernels.h)

// The epilogue on one element: gate g and up u in float32 (MATCH rounds them
// to the activation type first).
__device__ __forceinline__ float swiglu_epilogue(float g, float u, int mode, int act = kActBf16) {
  if (mode == kMatch) {
    g = round_to_act(g, act);
    u = round_to_act(u, act);
  }
  return silu_times(g, u);
}

// ------------------------------------------------ LDS-writing loads ----

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer descriptor in scalar registers: base, no stride, `bytes` records
// (hardware bounds check: reads past the end return zero).
__device__ __forceinline__ i32x4 make_srsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return (i32x4){(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uint64_t)(lds_ptr_t)p;
}

// Buffer loads that write LDS: lane i's 16 bytes land at base + 16 i.  They
// are issued from inline assembly so that the compiler does not serialise
// every later LDS read behind them (it cannot tell the stages apart); the
// kernel orders them itself with explicit vmcnt waits and barriers.  m0
// carries the LDS base.  The whole byte offset rides in the VGPR offset (the
// SGPR offset is 0): a raw buffer's range check covers the VGPR offset only,
// so every load past the end of its buffer -- including the loads the
// pipeline issues ahead past the last K-step -- returns zeros and touches no
// memory.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(i32x4 rs, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               ::"s"(lds_base), "v"(voff), "s"(rs) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace swq
