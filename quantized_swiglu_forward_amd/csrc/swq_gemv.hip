// Matrix-vector path (M < threshold) of the fused quantized SwiGLU.
//
// At decode the two projections are memory-bound matrix-vector products and
// reading Wg/Wu dominates ("mlx-bun 0.0.7 -> 0.0.9" diff, page 42,
// fused-swiglu-kernel.ts, the comment on where the fusion pays off, and the
// M-threshold function below which the caller keeps this path).  Lanes
// stream packed rows with 16-byte loads, turn codes into exact binary16
// operands, and per 32-input chunk (always inside one quantization group)
// the chunk's share of sum_k x'(s q + b) is formed exactly up to float32
// accumulation; the same epilogue as the matrix-matrix path writes hidden.
//
// Two kernels:
//  * swq_gemv1_kernel: M = 1 with at most four chunks per lane (H <= 8192),
//    and 2 <= M <= 4 with a whole wave per column and at most two chunks
//    per lane (2048 <= H <= 4096), each weight chunk loaded once for all
//    rows.  Codes enter mixed-precision FMAs (MATCH: v_dot2_f32_f16) as
//    exact binary16 subnormals with no offset, each chunk of x scaled by its
//    own power of two; the block shares x through LDS (described above the
//    kernel).
//  * swq_skinny_kernel: 1 <= M <= 32 otherwise.  x' is converted by the
//    waves themselves (M <= 16), built in LDS by every block, or staged by
//    the prep kernel; codes become exact binary16 s (q - z) and
//    16 x 16 x 32 MFMAs multiply them with one or two tiles of 16 rows at
//    once (described above the kernel).
// 2-bit codes are spread to nibbles as they are loaded and take the 4-bit
// arithmetic.  The activation type (bf16 or binary16) is a template
// parameter of both kernels.
//
// This file is compiled twice: on its own (SWQ_GEMV_ACT unset) for the bf16
// instances, the shared host functions and the dispatcher, and through
// swq_gemv_f16.hip for the binary16 instances only, so that the two halves
// build in parallel.
#include <cstring>
#include <mutex>
#include <type_traits>

#include "swq_device.h"
#include "swq_kernels.h"

#ifndef SWQ_GEMV_ACT
#define SWQ_GEMV_ACT 0
#endif

namespace swq {

// Raw weight data of one (column, chunk) item for one matrix.
template <int BITS>
struct RawChunk {
  u32x4 w[kCodeWidth<BITS> / 4];   // 32 codes: 16 bytes (4-bit, or 2-bit spread to nibbles) or 32 bytes (8-bit)
  uint32_t sb;         // bf16 scale (low half) and bias (high half) of the chunk's group
};

// Chunk loads through buffer descriptors whose base is the wave's first column:
// 32-bit offsets (one VALU op per address), and the descriptor's record count
// returns zeros for columns past the end.
struct MatBufs {
  __amdgpu_buffer_rsrc_t w, s, b;
  int rw, ng, lg_gs;
};

__device__ __forceinline__ MatBufs mat_bufs(const uint32_t* W, const uint16_t* S, const uint16_t* B, int64_t n0,
                                            int ncols, int H, int bits, int gs) {
  MatBufs m;
  m.rw = H * bits / 32;
  m.lg_gs = __builtin_ctz(gs);
  m.ng = H >> m.lg_gs;
  m.w = __builtin_amdgcn_make_buffer_rsrc((void*)(W + n0 * m.rw), (short)0, ncols * m.rw * 4, 0x00020000);
  m.s = __builtin_amdgcn_make_buffer_rsrc((void*)(S + n0 * m.ng), (short)0, ncols * m.ng * 2, 0x00020000);
  m.b = __builtin_amdgcn_make_buffer_rsrc((void*)(B + n0 * m.ng), (short)0, ncols * m.ng * 2, 0x00020000);
  return m;
}

// Chunk kc of column n0 + rel; code loads are nontemporal (each byte is read once).
template <int BITS>
__device__ __forceinline__ void load_chunk_buf(RawChunk<BITS>& r, const MatBufs& m, int rel, int kc) {
  const int wo = (rel * m.rw + kc * BITS) * 4;
  if constexpr (BITS == 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(m.w, wo, 0, 2);
    r.w[0] = (u32x4){spread2(v[0]), spread2(v[0] >> 16), spread2(v[1]), spread2(v[1] >> 16)};
  } else {
#pragma unroll
    for (int i = 0; i < BITS / 4; ++i) r.w[i] = __builtin_amdgcn_raw_buffer_load_b128(m.w, wo + 16 * i, 0, 2);
  }
  const int go = (rel * m.ng + ((kc * 32) >> m.lg_gs)) * 2;
  r.sb = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(m.s, go, 0, 0) |
         ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(m.b, go, 0, 0) << 16);
}


// (act: the activation type, a constant in every caller)
__device__ __forceinline__ void store_out(const GemvParams& p, int m, int n, float g, float u, int act) {
  const int64_t o = (int64_t)m * p.ldo + n;
  if (p.dbg_g) {
    p.dbg_g[o] = g;
    p.dbg_u[o] = u;
  } else if (p.mode >= kLinBf16) {
    if (p.res) {   // the residual of a whole MLP, added in float32 before the one rounding
      g += bf16_to_f32(p.res[o]);
      if (n < p.I_u) u += bf16_to_f32(p.res[o + p.I]);
    }
    if (p.mode == kLinF32) {
      reinterpret_cast<float*>(p.out)[o] = g;
      if (n < p.I_u) reinterpret_cast<float*>(p.out)[o + p.I] = u;
    } else {
      reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16(g);
      if (n < p.I_u) reinterpret_cast<uint16_t*>(p.out)[o + p.I] = f32_to_bf16(u);
    }
  } else {
    const float h = swiglu_epilogue(g, u, p.mode, act);
    if (p.mode == kF32) reinterpret_cast<float*>(p.out)[o] = h;
    else reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_act(h, act);
  }
}



// ------------------------------------------------------------- M == 1 ----
//
// Codes as binary16 subnormals.  A 4-bit code q in bits [0,4) of a binary16
// lane, with the exponent field zero, is the subnormal q * 2^-24; in bits
// [4,8) it is 16q * 2^-24.  So one AND per code pair of a word yields exact
// binary16 operands (no magic constant, no offset), and mixed-precision FMAs
// (or v_dot2_f32_f16) form exact products x' * q in float32.  The x' pairs that meet a code in
// bits [0,4) are stored pre-multiplied by 16 (exact: a power of two, and
// 16 max|x'| < 32), so every product lands in the same unit 2^-20:
//
//   P = sum_k 16 x'_k q_k 2^-24 = 2^-20 sum_k x'_k q_k
//
// and a 32-code chunk adds s * P + b * Sx'' with Sx'' = 2^-20 * sum x' over
// the chunk (the same unit).  x' = x * 2^-e uses the exponent e of the
// chunk's own largest magnitude; the chunk's scale and the unit are removed
// with one ldexp by (e + 20) per chunk.  No offset is subtracted, so nothing
// cancels beyond what w = s*q + b itself does.
//
// 8-bit codes: v_perm_b32 gathers byte j of the word holding codes 0..3 and
// byte j of the word holding codes 4..7 into one register; its low nibbles
// (mask 0x000F000F) and high nibbles (mask 0x00F000F0, worth 16 * lo units)
// both meet 16 x', which is what q = 16 hi + lo needs.
//

// Two exact binary16 products x c, each added to p with one float32 rounding
// (v_fma_mix_f32).  v_dot2_f32_f16 would take both in one instruction, but
// its sum of two products and the accumulator is not rounded to nearest
// when their exponents differ widely (measured: a downward bias of about
// 2^-22 of the sum per step), which sums of many same-sign products turn
// into errors well above float32 accumulation.
// (Contraction is off here: the compiler would fold the two FMAs back into
// v_dot2.)
__device__ __forceinline__ float fma2(uint32_t xv, uint32_t cv, float p) {
#pragma clang fp contract(off)
  const f16x2 x = as_h2(xv), c = as_h2(cv);
  p = __builtin_fmaf((float)x[0], (float)c[0], p);
  return __builtin_fmaf((float)x[1], (float)c[1], p);
}

// The same two products, summed by v_dot2_f32_f16 (DOT) or by fma2.  The M = 1
// kernel takes v_dot2 in MATCH, where gate and up are rounded to the 16-bit
// activation type: its summation error (measured: at most about 5e-5 of the
// column's cancellation-free scale on rows of one-signed x) lies far inside
// that rounding's tie allowance, and one instruction per pair halves the
// arithmetic that follows the loads.  The float32 modes take fma2.
template <bool DOT>
__device__ __forceinline__ float pair2(uint32_t xv, uint32_t cv, float p) {
  if constexpr (DOT) return __builtin_amdgcn_fdot2(as_h2(xv), as_h2(cv), p, false);
  else return fma2(xv, cv, p);
}

// Unscaled dot of one chunk in units of 2^-20: xa holds the 16x pairs
// (codes at bits [0,4)), xb the 1x pairs (codes at bits [4,8)).
template <int BITS, bool DOT>
__device__ __forceinline__ float chunk_dot_sub(const RawChunk<BITS>& r, const uint32_t xa[8], const uint32_t xb[8]) {
  float p = 0.0f;
  if (kCodeWidth<BITS> == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = r.w[0][j];
      const uint32_t w8 = w >> 8;
      p = pair2<DOT>(xa[2 * j], w & 0x000F000Fu, p);
      p = pair2<DOT>(xb[2 * j], w & 0x00F000F0u, p);
      p = pair2<DOT>(xa[2 * j + 1], w8 & 0x000F000Fu, p);
      p = pair2<DOT>(xb[2 * j + 1], w8 & 0x00F000F0u, p);
    }
  } else {
    // xa / xb interleave as (pair 0, pair 2) / (pair 1, pair 3) of each 8-block;
    // 8-bit needs 16x' on every pair: xb pairs are scaled here
    const f16x2 c16 = {(_Float16)16.0f, (_Float16)16.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4& wv = r.w[j / 2];
      const uint32_t wa = wv[2 * (j & 1)], wb = wv[2 * (j & 1) + 1];
      uint32_t xq[4] = {xa[2 * j], as_u32(as_h2(xb[2 * j]) * c16), xa[2 * j + 1],
                        as_u32(as_h2(xb[2 * j + 1]) * c16)};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + t) << 16) | (uint32_t)t;
        const uint32_t v = __builtin_amdgcn_perm(wb, wa, sel);
        p = pair2<DOT>(xq[t], v & 0x000F000Fu, p);
        p = pair2<DOT>(xq[t], v & 0x00F000F0u, p);
      }
    }
  }
  return p;
}

// Sum over aligned groups of `width` lanes (a power of two); every lane of a
// group ends with the group's sum.
__device__ __forceinline__ float group_sum(float v, int width) {
  if (width >= 2) v += __shfl_xor(v, 1);
  if (width >= 4) v += __shfl_xor(v, 2);
  if (width >= 8) v += __shfl_xor(v, 4);
  if (width >= 16) v += __shfl_xor(v, 8);
  if (width >= 32) v += __shfl_xor(v, 16);
  if (width >= 64) v += __shfl_xor(v, 32);
  return v;
}

// Sum over the whole wavefront, uniform result: DPP within rows of 16
// lanes (xor 1, xor 2, half-row mirror, row mirror), then the four row sums.
__device__ __forceinline__ float wave_sum(float v) {
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xF, 0xF, false);   // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xF, 0xF, false);   // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Row sum over 16 lanes; every lane of the row ends with it.
__device__ __forceinline__ float row_sum(float v) {
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xF, 0xF, false);   // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xF, 0xF, false);   // row_mirror
  return v;
}

// v_permlane32_swap: a' = (a lanes 0-31, b lanes 0-31), b' = (a lanes 32-63,
// b lanes 32-63), so a' + b' holds a's half-wave partial sums in lanes 0-31
// and b's in lanes 32-63.  v_permlane16_swap does the same with the odd and
// even 16-lane rows: a' = (a.r0, b.r0, a.r2, b.r2), b' = (a.r1, b.r1, a.r3, b.r3).
__device__ __forceinline__ float fold32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float fold16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Lane i < 32 receives lane i + 32's value.
__device__ __forceinline__ float upper_half(float a) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return __uint_as_float(r[1]);
}

// One lane's x chunk (32 values) as exact binary16 pairs for the
// subnormal-code dot products, scaled by its own power of two: x' = x 2^-e
// with e the exponent of the chunk's largest magnitude (every element at
// least 2^-17 of that maximum converts exactly).  xa holds the pairs that
// meet codes in bits [0,4) as 16x', xb the others as x'; sx is the chunk's
// sum of x' in the dot products' unit 2^-20.
struct XChunk {
  uint32_t xa[8], xb[8];
  float sx;
  int e;
};

// Largest H of the M = 1 kernel: 64 lanes x 2 chunks of 32.
constexpr int kGemv1MaxH = 8192;

// The block converts x once and shares it through LDS.  Thread t converts
// the 8-value blocks t, t + 256, ...; the four blocks of a 32-value chunk
// sit in four consecutive lanes, which agree on the chunk's exponent and
// sum with two DPP steps.  Block j of a chunk is stored as the 16 bytes
// (16x'0, 16x'4), (x'1, x'5), (16x'2, 16x'6), (x'3, x'7): the operands of
// code word j in the order the dot products take them.  Lanes past the end
// of x carry zeros (a quad is all in or all out: H is a multiple of 32).
__device__ __forceinline__ void stage_x_block(const u32x4& raw, int blk, bool valid, u32x4* xs, float2* xinfo,
                                              int act) {
  uint32_t amax = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) amax = max(amax, max(raw[j] & 0x7FFFu, (raw[j] >> 16) & 0x7FFFu));
  amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  const int e = x_exponent(amax, act);
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = act_to_f32((uint16_t)(raw[j] & 0xFFFFu), act);
    f[2 * j + 1] = act_to_f32((uint16_t)(raw[j] >> 16), act);
  }
  u32x4 v;
  v[0] = as_u32((f16x2){(_Float16)ldexpf(f[0], 4 - e), (_Float16)ldexpf(f[4], 4 - e)});
  v[1] = as_u32((f16x2){(_Float16)ldexpf(f[1], -e), (_Float16)ldexpf(f[5], -e)});
  v[2] = as_u32((f16x2){(_Float16)ldexpf(f[2], 4 - e), (_Float16)ldexpf(f[6], 4 - e)});
  v[3] = as_u32((f16x2){(_Float16)ldexpf(f[3], -e), (_Float16)ldexpf(f[7], -e)});
  // the chunk's sum of x' (exact values, float32 adds)
  float sx = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) sx += ldexpf(f[j], -e);
  sx += __builtin_amdgcn_update_dpp(0.0f, sx, 0xB1, 0xF, 0xF, false);
  sx += __builtin_amdgcn_update_dpp(0.0f, sx, 0x4E, 0xF, 0xF, false);
  if (valid) {
    xs[blk] = v;
    if ((blk & 3) == 0) xinfo[blk >> 2] = make_float2(ldexpf(sx, -20), __int_as_float(e));
  }
}

__device__ __forceinline__ void read_x_chunk(const u32x4* xs, const float2* xinfo, int kc, XChunk& c) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 v = xs[4 * kc + q];
    c.xa[2 * q] = v[0];
    c.xb[2 * q] = v[1];
    c.xa[2 * q + 1] = v[2];
    c.xb[2 * q + 1] = v[3];
  }
  const float2 inf = xinfo[kc];
  c.sx = inf.x;
  c.e = __float_as_int(inf.y);
}

// The chunk's share of sum_k x_k (s q_k + b), in the chunk's own scale 2^(e+20).
template <int BITS, bool DOT>
__device__ __forceinline__ float chunk_term(const RawChunk<BITS>& r, const XChunk& x, int act) {
  const float P = chunk_dot_sub<BITS, DOT>(r, x.xa, x.xb);
  const float s = act_to_f32((uint16_t)(r.sb & 0xFFFFu), act);
  const float b = act_to_f32((uint16_t)(r.sb >> 16), act);
  return fmaf(s, P, b * x.sx);
}

// M = 1.  Lane sl of a column group of lpc = 2^lg lanes owns the 32-code
// chunks sl, sl + lpc, ... of its column; a wave owns R rounds of 64/lpc
// columns.  Every thread issues its x load and then its whole weight stream
// before any arithmetic; the block converts x into LDS while the weights
// arrive (one barrier, which the weight loads stay in flight across).  With
// a whole wave per column, the R columns' sums end wave-uniform and lane r
// runs the epilogue of column r, so one pass serves all R columns.  FULL:
// H = 2048 CPL exactly (64 lanes per column, every lane CPL chunks).
// MR > 1 serves MR = M rows (R <= 2): every row's x is staged and dotted
// with the same weight chunks, which are loaded once; the reduction and
// epilogue run per row.
template <int BITS_G, int BITS_U, int CPL, int R, bool FULL, int WPB, int MR, int ACT>
__global__ __launch_bounds__(64 * WPB) void swq_gemv1_kernel(GemvParams p, int lg) {
  static_assert(MR >= 1 && MR <= 4 && (MR == 1 || R <= 2), "several rows: at most two columns per wave");
  constexpr int NT = 64 * WPB;
  constexpr int XI = (256 * CPL + NT - 1) / NT;   // 8-value blocks of one row of x per thread
  __shared__ u32x4 xs[MR][256 * CPL];
  __shared__ float2 xinfo[MR][64 * CPL];
#ifdef SWQ_LDS_POISON
  lds_poison(xs, sizeof(xs), kPoisonFloat);
  lds_poison(xinfo, sizeof(xinfo), kPoisonFloat);
  __syncthreads();
#endif
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  if constexpr (FULL) lg = 6;
  const int lpc = 1 << lg;
  const int wave_global = blockIdx.x * WPB + __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int sub = lane >> lg, sl = lane & (lpc - 1);
  const int cpw = 64 >> lg;
  const int nchunk = p.H / 32, nblk = p.H / 8;

  // 1. this thread's 8-value blocks of x (loads complete in issue order: x
  //    first, so it is not held up behind the weight stream)
  u32x4 xraw[MR][XI];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int blk = tid + NT * i;
      xraw[m][i] = *reinterpret_cast<const u32x4*>(p.x + (int64_t)m * p.H + 8 * min(blk, nblk - 1));
    }

  // 2. all weight loads of this lane: R columns x CPL chunks x 2 matrices
  const int64_t n0 = (int64_t)wave_global * R * cpw;           // the wave's first column
  const int ncols = (int)max((int64_t)0, min((int64_t)R * cpw, (int64_t)p.I - n0));
  const MatBufs mg = mat_bufs(p.wg, p.sg, p.bg, n0, ncols, p.H, BITS_G, p.gs_g);
  const int ncols_u = (int)max((int64_t)0, min((int64_t)ncols, (int64_t)p.I_u - n0));
  const MatBufs mu = mat_bufs(p.wu, p.su, p.bu, n0, ncols_u, p.H, BITS_U, p.gs_u);
  RawChunk<BITS_G> rg[R][CPL];
  RawChunk<BITS_U> ru[R][CPL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rel = r * cpw + sub;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int kc = min(sl + c * lpc, nchunk - 1);
      load_chunk_buf<BITS_G>(rg[r][c], mg, rel, kc);
      load_chunk_buf<BITS_U>(ru[r][c], mu, rel, kc);
    }
  }

  // every load is issued before the first wait (for x) below
  __builtin_amdgcn_sched_barrier(0);

  // 3. x' into LDS, shared by the block's four waves
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int i = 0; i < XI; ++i) stage_x_block(xraw[m][i], tid + NT * i, tid + NT * i < nblk, xs[m], xinfo[m], ACT);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // 4. per column: chunk terms, reduction over the column group, epilogue
  // (row m of the output); the products summed by v_dot2 in MATCH, by FMAs
  // otherwise (pair2)
  auto columns = [&](auto dot_tag) {
    constexpr bool DOT = decltype(dot_tag)::value;
    auto finish = [&](const float (&ag)[R], const float (&au)[R], int m) __attribute__((always_inline)) {
      if (R <= 2 && (FULL || lpc == 64)) {
        // Sums of the 2R values of the wave with two lane-swap folds and one row
        // sum: row 0 ends with column 0's gate, row 2 with its up, rows 1 and 3
        // with column 1's (R = 2); lane 16 r then runs column r's epilogue.
        const float t0 = fold32(ag[0], au[0]);
        const float t = R == 2 ? fold16(t0, fold32(ag[R - 1], au[R - 1])) : fold16(t0, t0);
        const float g = row_sum(t);
        const float u = upper_half(g);
        const int col = lane >> 4;
        const int64_t n = (int64_t)wave_global * R + col;
        if ((lane & 15) == 0 && col < R && n < p.I) store_out(p, m, (int)n, g, u, ACT);
      } else if (FULL || lpc == 64) {
        float g = 0.0f, u = 0.0f;
  #pragma unroll
        for (int r = 0; r < R; ++r) {
          const float gr = wave_sum(ag[r]), ur = wave_sum(au[r]);
          if (lane == r) {
            g = gr;
            u = ur;
          }
        }
        const int n = wave_global * R + lane;
        if (lane < R && n < p.I) store_out(p, m, n, g, u, ACT);
      } else if constexpr (!FULL) {
  #pragma unroll
        for (int r = 0; r < R; ++r) {
          const float g = group_sum(ag[r], lpc), u = group_sum(au[r], lpc);
          const int n = (wave_global * R + r) * cpw + sub;
          if (sl == 0 && n < p.I) store_out(p, m, n, g, u, ACT);
        }
      }
    };
    if constexpr (MR > 1) {
      // A whole wave per column (the launcher's condition).  Every row's sums
      // first (each row's x chunk read from LDS once for the R columns), then
      // the rows' reductions side by side, then one store branch for all rows:
      // the rows' dependency chains overlap instead of running one after the
      // other.  Per row the arithmetic is the single-row case's, in its order.
      float ag[MR][R], au[MR][R];
  #pragma unroll
      for (int m = 0; m < MR; ++m)
  #pragma unroll
        for (int r = 0; r < R; ++r) {
          ag[m][r] = 0.0f;
          au[m][r] = 0.0f;
        }
  #pragma unroll
      for (int c = 0; c < CPL; ++c) {
        if (FULL || sl + c * lpc < nchunk) {
  #pragma unroll
          for (int m = 0; m < MR; ++m) {
            XChunk xc;   // per row and chunk: all of them at once would not fit in registers
            read_x_chunk(xs[m], xinfo[m], sl + c * lpc, xc);
  #pragma unroll
            for (int r = 0; r < R; ++r) {
              ag[m][r] += ldexpf(chunk_term<BITS_G, DOT>(rg[r][c], xc, ACT), xc.e + 20);
              au[m][r] += ldexpf(chunk_term<BITS_U, DOT>(ru[r][c], xc, ACT), xc.e + 20);
            }
          }
        }
      }
      float gm[MR], um[MR];
  #pragma unroll
      for (int m = 0; m < MR; ++m) {
        const float t0 = fold32(ag[m][0], au[m][0]);
        const float t = R == 2 ? fold16(t0, fold32(ag[m][R - 1], au[m][R - 1])) : fold16(t0, t0);
        gm[m] = row_sum(t);
        um[m] = upper_half(gm[m]);
      }
      // every lane of a 16-lane row holds its column's sums of every row:
      // lane 16 col + m runs the epilogue of row m, all rows at once
      const int col = lane >> 4, mrow = lane & 15;
      const int64_t n = (int64_t)wave_global * R + col;
      float g = gm[0], u = um[0];
  #pragma unroll
      for (int m = 1; m < MR; ++m)
        if (mrow == m) {
          g = gm[m];
          u = um[m];
        }
      if (mrow < MR && col < R && n < p.I) store_out(p, mrow, (int)n, g, u, ACT);
    } else {
      XChunk xc[CPL];
  #pragma unroll
      for (int c = 0; c < CPL; ++c) read_x_chunk(xs[0], xinfo[0], min(sl + c * lpc, nchunk - 1), xc[c]);
      float ag[R], au[R];
  #pragma unroll
      for (int r = 0; r < R; ++r) {
        ag[r] = 0.0f;
        au[r] = 0.0f;
  #pragma unroll
        for (int c = 0; c < CPL; ++c) {
          if (FULL || sl + c * lpc < nchunk) {
            ag[r] += ldexpf(chunk_term<BITS_G, DOT>(rg[r][c], xc[c], ACT), xc[c].e + 20);
            au[r] += ldexpf(chunk_term<BITS_U, DOT>(ru[r][c], xc[c], ACT), xc[c].e + 20);
          }
        }
      }
      finish(ag, au, 0);
    }
  };
  if (p.mode == kMatch) columns(std::true_type{});
  else columns(std::false_type{});
}

// --------------------------------------------------------- 2 <= M <= 32 --
//
// Matrix-vector products for a few rows.  The rows of x, staged once per call
// as x' = x 2^-e (binary16, per-row power of two, in the code-pair order of
// the dequantized weights, 32 inputs per chunk), are the A operand of
// v_mfma_f32_16x16x32_f16 (RT tiles of 16 rows, M of them live); the
// dequantized weights s (q - z) of 16 output columns are the B operand, so
// one unpack serves every row of every tile.  A block of up to 16 waves owns 16 columns of both matrices:
// wave w takes the chunk quads w, w + W, ... (W waves), and lane group
// h = lane / 16 takes chunk 4 quad + h: the MFMA's K slots of group h are
// that chunk's 8-code block, on the A side x' of the same inputs.  With 4-bit
// codes at most 64 registers per lane let two such blocks share a CU, so a
// whole decode-sized grid is resident at once.  A fifth MFMA per chunk adds
// the bias term sum_chunk x' * c (c = b + z s) with the chunk sum of x' and c
// each split into binary16 hi + lo, as on the matrix-matrix path.  The waves'
// partial sums meet in LDS; wave 4 t + j sums element j of row tile t, applies
// 2^e and runs that row's epilogue.  x' comes from one of three sources (XS):
//  * kXSelf (a row fits one pass of the block's waves; M <= 16, or up to 32
//    rows in two tiles with narrow codes and one chunk quad per wave): each
//    wave copies the rows of x over its own chunks into its own LDS region
//    (loads that write LDS, four lanes per 64-byte piece of a row), reads
//    them back in the MFMA's lane order, takes the largest magnitude of each
//    row over its chunks (two lane swaps) and converts in registers; its
//    partial sums are multiplied by its own 2^e, so no other wave, block or
//    kernel is involved;
//  * kXStage (M*H at most kSkinnyStageMax): every block builds x' in LDS with
//    the prep kernel's row powers of two, conversion and layout;
//  * kXPrep: the prep kernel stages x' and the row exponents first.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
constexpr int kSkinnyMaxWaves = 16;

template <int BITS_G, int BITS_U, int RT, int CT>
struct SkinnyChunk {
  // codes of each column tile as loaded (the line-friendly lane order, 2-bit
  // codes not yet spread), then in the MFMA's order
  u32x4 cg[CT][kCodeWidth<BITS_G> / 4], cu[CT][kCodeWidth<BITS_U> / 4], x[RT][4];
  uint32_t sg[CT], bg[CT], su[CT], bu[CT];   // raw 16-bit bits, converted where used (after every load is issued)
  float sx[RT];              // x converted by the wave: the lane's sum of x' (float32 adds)
  bool live;
};

// Scales and biases of a chunk quad (or of two adjacent quads): per array one
// dword per lane, lane 4 rl + hl holding groups w + 2 hl and w + 2 hl + 1 of
// column rl, where the window [w, w + 8) is the block of 8 groups, aligned to
// 8, around the quad's first input; it holds every group of those 128 (or
// 256) inputs.
template <int CT>
struct SbWindow {
  uint32_t v[CT][4];   // per column tile: sg, bg, su, bu
  int wg, wu;          // window starts (gate, up)
};

// RT: row tiles of 16 (M <= 16 RT = 1; M <= 32 RT = 2, whose second tile of x'
// and accumulators need twice the registers: half the waves per SIMD).  Q2:
// two chunk quads in flight per wave (codes of at most 4 bits, x' from the
// prep kernel), with half the waves per SIMD.  CT: column tiles of 16 per
// block (CT = 2 with x converted by the waves, one chunk quad per wave and
// narrow codes: one conversion of x serves 32 columns, for grids of more
// tiles than CUs).
template <int BITS_G, int BITS_U, int XS, int RT, bool Q2, int ACT, int CT>
__global__ __launch_bounds__(64 * kSkinnyMaxWaves)
__attribute__((amdgpu_waves_per_eu(CT == 2 || Q2 ? 4 : (BITS_G == 4 && BITS_U == 4 ? 6 : 4) / RT))) void swq_skinny_kernel(GemvParams pin) {
  constexpr bool STAGE = XS == kXStage, SELF = XS == kXSelf;
  // rows of this block: row group blockIdx.y of kGemvMaxM rows (x, its
  // staged exponents and the stores offset by m0; p.M the group's rows)
  const int m0 = (int)blockIdx.y * kGemvMaxM;
  GemvParams p = pin;
  p.x = pin.x + (int64_t)m0 * pin.H;
  p.M = min(kGemvMaxM, pin.M - m0);
  if constexpr (XS == kXPrep) p.xexp = pin.xexp + m0;
  // 16-row tiles of x' staged by the prep kernel (every group's), and this group's first
  const int xtiles = RT * (int)gridDim.y, xtile0 = RT * (int)blockIdx.y;
  static_assert(!Q2 || (!STAGE && BITS_G <= 4 && BITS_G == BITS_U), "two quads in flight: narrow codes, x' in registers");
  static_assert(!SELF || RT == 1 || !Q2, "x converted by the waves: two row tiles with one quad per wave");
  static_assert(CT == 1 || (CT == 2 && SELF && !Q2 && BITS_G <= 4 && BITS_G == BITS_U),
                "two column tiles: x converted by the waves, one quad per wave, narrow codes");
  (void)xtile0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = blockDim.x >> 6;
  const int r = lane & 15, h = lane >> 4;             // A row / B and D column; K-slot group
  const int64_t n0 = (int64_t)blockIdx.x * 16 * CT;
  const int col = (int)n0 + r;                        // (column tile 0; tile c: col + 16 c)
  // x' row of this lane per tile: from the prep kernel, a row past M reads
  // zeros (see load); from LDS, clamped to the last row
  bool rowok[RT];
  int rowl[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    rowok[t] = 16 * t + r < p.M;
    rowl[t] = min(16 * t + r, p.M - 1);
  }
  const int nchunk = p.H >> 5;
  // the block's 16 CT columns through buffer descriptors (columns past I read zeros)
  const int ncols = (int)min((int64_t)16 * CT, (int64_t)p.I - n0);
  const MatBufs mg = mat_bufs(p.wg, p.sg, p.bg, n0, ncols, p.H, BITS_G, p.gs_g);
  const int ncols_u = (int)max((int64_t)0, min((int64_t)ncols, (int64_t)p.I_u - n0));
  const MatBufs mu = mat_bufs(p.wu, p.su, p.bu, n0, ncols_u, p.H, BITS_U, p.gs_u);
  // x' from the prep kernel in this kernel's lane order (kSkinnyXUnitsPerQuadTile)
  const int nquad_all = (nchunk + 3) >> 2;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.xa, (short)0, nquad_all * xtiles * kSkinnyXUnitsPerQuadTile * 16, 0x00020000);
  // exponents of this lane's accumulator rows 16 t + 4 h + j (prep-fed x'; the
  // block's own in LDS otherwise), loaded with the first weights and packed
  // as four biased bytes per tile (each lies in [-127, 127]); two row tiles
  // with two quads in flight, and 2-bit codes (spread as they are loaded),
  // have no registers to spare and load them at the end
  // (SELF: the wave's own exponents, packed the same way once its x is in)
  constexpr bool kPreE = XS == kXPrep && !(Q2 && RT == 2) && BITS_G != 2 && BITS_U != 2;
  uint32_t xrow_e[RT];
  if constexpr (kPreE) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      xrow_e[t] = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = 16 * t + 4 * h + j;
        xrow_e[t] |= (uint32_t)((m < p.M ? p.xexp[m] : 0) + 128) << (8 * j);
      }
    }
  }
  const NibbleK nk = nibble_consts_in_regs();

  // Codes, scales and biases are loaded in a line-friendly lane order and then
  // moved to the MFMA's order with ds_bpermute.  In the MFMA's order adjacent
  // lanes hold adjacent columns, each in its own cache line, and the vector
  // L1 looks up one tag per cache line for every four lanes of a load; in the
  // load order the four lanes 4 rl + hl (hl = 0..3) read one piece of column
  // rl (its chunk 4 quad + hl, or one window of groups).  Lane 16 h + r of
  // the MFMA's order takes its codes from lane 4 r + h.
  const int rl = lane >> 2, hl = lane & 3;
  const int perm = (4 * r + h) * 4;   // ds_bpermute byte address of that lane
  // the windows of groups in dwords when every row of the four arrays starts
  // on a dword boundary (else in two halves)
  const bool sb_dword = (((mg.ng | mu.ng) & 1) == 0) &&
                        ((((uintptr_t)p.sg | (uintptr_t)p.bg | (uintptr_t)p.su | (uintptr_t)p.bu) & 3) == 0);

  // STAGE: x' in LDS as [H/32][M][32] binary16 (16-byte pieces), row exponents beside it
  __shared__ u32x4 xs[STAGE ? kSkinnyStageMax / 8 : 1];
  __shared__ int xe[STAGE ? kGemvMaxM : 1];
  __shared__ uint32_t xmax[STAGE ? kGemvMaxM : 1];
  // SELF: the waves' regions (skinny_self_region bytes each), launched as dynamic LDS
  extern __shared__ u32x4 swq_dyn[];
  constexpr int kSelfChunks = Q2 ? 8 : 4;   // chunks per wave
  const int rb = SELF ? skinny_self_region(p.M, kSelfChunks, CT * RT) : 0;
  unsigned char* const xreg = reinterpret_cast<unsigned char*>(swq_dyn) + w * rb;

  // Row exponents k of the block's 16 columns of both matrices
  // (row_exponent_k): the scales and constants below are taken times 2^-k
  // and the sums multiplied by 2^k in the epilogue.  With x' from the prep
  // kernel, its column blocks computed them; with STAGE the block does:
  // thread t scans column
  // t % 16 of both matrices over groups t / 16, t / 16 + nt / 16, ...,
  // loaded after the first weights (the block barrier below waits for the
  // slowest wave's weights either way); the lanes of a column reduce with
  // two swaps, and the waves meet in LDS.
  __shared__ float kred[STAGE ? kSkinnyMaxWaves : 1][32];
  // the waves' partial sums (after the K loop; SELF: in each wave's own region)
  __shared__ f32x4 red[SELF ? 1 : kSkinnyMaxWaves][SELF ? 1 : 2 * RT][64];
  auto red_at = [&](int ww, int i) -> f32x4* {
    if constexpr (SELF) return reinterpret_cast<f32x4*>(reinterpret_cast<unsigned char*>(swq_dyn) + ww * rb) + 64 * i;
    else return red[ww][i];
  };
#ifdef SWQ_LDS_POISON
  lds_poison(xs, sizeof(xs), kPoisonFloat);
  lds_poison(xe, sizeof(xe), kPoisonExp);
  lds_poison(xmax, sizeof(xmax), kPoisonExp);
  lds_poison(kred, sizeof(kred), kPoisonFloat);
  lds_poison(red, sizeof(red), kPoisonFloat);
  if constexpr (SELF) lds_poison(swq_dyn, nw * rb, kPoisonFloat);
  __syncthreads();
#endif
  auto row_k_finish = [&]() {
    const int kstride = blockDim.x >> 4;
    float kmax_g = 0.0f, kmax_u = 0.0f;
#pragma unroll 2
    for (int g = tid >> 4; g < max(mg.ng, mu.ng); g += kstride) {
      const int gg = min(g, mg.ng - 1), gu = min(g, mu.ng - 1);
      const uint16_t s_g = __builtin_amdgcn_raw_buffer_load_b16(mg.s, (r * mg.ng + gg) * 2, 0, 0);
      const uint16_t b_g = __builtin_amdgcn_raw_buffer_load_b16(mg.b, (r * mg.ng + gg) * 2, 0, 0);
      const uint16_t s_u = __builtin_amdgcn_raw_buffer_load_b16(mu.s, (r * mu.ng + gu) * 2, 0, 0);
      const uint16_t b_u = __builtin_amdgcn_raw_buffer_load_b16(mu.b, (r * mu.ng + gu) * 2, 0, 0);
      if (g < mg.ng)
        kmax_g = fmaxf(kmax_g, group_term_max(act_to_f32(s_g, ACT), act_to_f32(b_g, ACT), CodeOffset<BITS_G>::z,
                                              kPlaneMax<BITS_G>));
      if (g < mu.ng)
        kmax_u = fmaxf(kmax_u, group_term_max(act_to_f32(s_u, ACT), act_to_f32(b_u, ACT), CodeOffset<BITS_U>::z,
                                              kPlaneMax<BITS_U>));
    }
    kmax_g = fmaxf(kmax_g, __shfl_xor(kmax_g, 16));
    kmax_g = fmaxf(kmax_g, __shfl_xor(kmax_g, 32));
    kmax_u = fmaxf(kmax_u, __shfl_xor(kmax_u, 16));
    kmax_u = fmaxf(kmax_u, __shfl_xor(kmax_u, 32));
    if (lane < 16) {
      kred[w][lane] = kmax_g;
      kred[w][16 + lane] = kmax_u;
    }
  };
  // this lane's column exponents: from the prep kernel (x' staged there),
  // else from the block's own pass, after a barrier.  Both in one register
  // (each in [-200, 200]): gate in the low half, up in the high half.
  uint32_t kpack[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) kpack[ct] = 0;
  auto set_k = [&](int ct, int kg_, int ku_) { kpack[ct] = ((uint32_t)kg_ & 0xFFFFu) | ((uint32_t)ku_ << 16); };
  auto k_gate = [&](int ct) { return (int)(int16_t)(kpack[ct] & 0xFFFFu); };
  auto k_up = [&](int ct) { return (int)kpack[ct] >> 16; };
  if constexpr (XS == kXPrep) {
    const int nquad_ = (nchunk + 3) >> 2;
    if (nquad_ > (Q2 ? 2 : 1) * nw && col < p.I) set_k(0, p.kexp[col], p.kexp[p.I + col]);
  }
  auto row_k_read = [&]() {
    float mg_ = 0.0f, mu_ = 0.0f;
    for (int ww = 0; ww < nw; ++ww) {
      mg_ = fmaxf(mg_, kred[ww][r]);
      mu_ = fmaxf(mu_, kred[ww][16 + r]);
    }
    set_k(0, row_exponent_k(mg_), row_exponent_k(mu_));
  };

  // the window of groups around quad `quad` (issue before the quad's codes)
  auto load_sb = [&](int quad, SbWindow<CT>& sw) {
    sw.wg = ((128 * quad) >> mg.lg_gs) & ~7;
    sw.wu = ((128 * quad) >> mu.lg_gs) & ~7;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int og = ((16 * ct + rl) * mg.ng + sw.wg + 2 * hl) * 2, ou = ((16 * ct + rl) * mu.ng + sw.wu + 2 * hl) * 2;
      if (sb_dword) {
        sw.v[ct][0] = __builtin_amdgcn_raw_buffer_load_b32(mg.s, og, 0, 0);
        sw.v[ct][1] = __builtin_amdgcn_raw_buffer_load_b32(mg.b, og, 0, 0);
        sw.v[ct][2] = __builtin_amdgcn_raw_buffer_load_b32(mu.s, ou, 0, 0);
        sw.v[ct][3] = __builtin_amdgcn_raw_buffer_load_b32(mu.b, ou, 0, 0);
      } else {
        auto two = [](const __amdgpu_buffer_rsrc_t& rs, int off) {
          return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0) |
                 ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, off + 2, 0, 0) << 16);
        };
        sw.v[ct][0] = two(mg.s, og);
        sw.v[ct][1] = two(mg.b, og);
        sw.v[ct][2] = two(mu.s, ou);
        sw.v[ct][3] = two(mu.b, ou);
      }
    }
  };
  // this lane's scale and bias (chunk 4 quad + h of column r) from the window
  auto pick_sb = [&](const SbWindow<CT>& sw, int quad, SkinnyChunk<BITS_G, BITS_U, RT, CT>& d) {
    const int c = 4 * quad + h;
    const int ig = ((32 * c) >> mg.lg_gs) - sw.wg, iu = ((32 * c) >> mu.lg_gs) - sw.wu;   // in [0, 8)
    const int ag = (4 * r + (ig >> 1)) * 4, au = (4 * r + (iu >> 1)) * 4;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const uint32_t s_g = (uint32_t)__builtin_amdgcn_ds_bpermute(ag, (int)sw.v[ct][0]);
      const uint32_t b_g = (uint32_t)__builtin_amdgcn_ds_bpermute(ag, (int)sw.v[ct][1]);
      const uint32_t s_u = (uint32_t)__builtin_amdgcn_ds_bpermute(au, (int)sw.v[ct][2]);
      const uint32_t b_u = (uint32_t)__builtin_amdgcn_ds_bpermute(au, (int)sw.v[ct][3]);
      d.sg[ct] = (ig & 1) ? s_g >> 16 : s_g & 0xFFFFu;
      d.bg[ct] = (ig & 1) ? b_g >> 16 : b_g & 0xFFFFu;
      d.su[ct] = (iu & 1) ? s_u >> 16 : s_u & 0xFFFFu;
      d.bu[ct] = (iu & 1) ? b_u >> 16 : b_u & 0xFFFFu;
    }
  };

  auto load = [&](int quad, SkinnyChunk<BITS_G, BITS_U, RT, CT>& d) {
    const int c = 4 * quad + h;
    d.live = c < nchunk;
    // codes in the load order: chunk 4 quad + hl of column rl of each column
    // tile (chunk 0 past the end)
    const int cl = 4 * quad + hl < nchunk ? 4 * quad + hl : 0;
    auto codes = [](const __amdgpu_buffer_rsrc_t& rs, int off, u32x4* dst, auto bits_tag) {
      constexpr int BITS = decltype(bits_tag)::value;
      if constexpr (BITS == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 2);
        dst[0] = (u32x4){v[0], v[1], 0u, 0u};   // spread after the move
      } else {
#pragma unroll
        for (int i = 0; i < BITS / 4; ++i) dst[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * i, 0, 2);
      }
    };
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int og = ((16 * ct + rl) * mg.rw + cl * BITS_G) * 4, ou = ((16 * ct + rl) * mu.rw + cl * BITS_U) * 4;
      codes(mg.w, og, d.cg[ct], std::integral_constant<int, BITS_G>{});
      codes(mu.w, ou, d.cu[ct], std::integral_constant<int, BITS_U>{});
    }
    if constexpr (XS == kXPrep) {
      // one contiguous kilobyte per instruction; a row past M or a chunk past
      // H reads zeros (offset past the buffer's range)
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const bool ok = d.live && rowok[t];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ox = ok ? (((quad * xtiles + xtile0 + t) * 4 + q) * 64 + lane) * 16 : 0x7FFFFFF0;
          d.x[t][q] = __builtin_amdgcn_raw_buffer_load_b128(rx, ox, 0, 0);
        }
      }
    }
    // every load of the chunk is in flight before the first use of any of them
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load_x_lds = [&](int quad, SkinnyChunk<BITS_G, BITS_U, RT, CT>& d) {
    const int c = min(4 * quad + h, nchunk - 1);
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) d.x[t][q] = xs[(c * p.M + rowl[t]) * 4 + q];
  };

  // one matrix's 8-code block kb of a chunk, multiplied into every row tile:
  // one B operand (4-bit) or two (8-bit planes), built once
  // s2 = (s, s), or with binary16 scales (split) its two parts (hi, lo):
  // then each part takes its own plane (split_scale)
  auto block_mfma = [&]<int BITS>(const u32x4* cw, f16x2 s2, bool split, int kb, const f16x8 (&a)[RT],
                                  f32x4 (&acc)[RT]) {
    auto mfma_b = [&](const u32x4& v) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], __builtin_bit_cast(f16x8, v), acc[t], 0, 0, 0);
    };
    if constexpr (kCodeWidth<BITS> == 4) {
      if (split) {
        const f16x2 shi = {s2[0], s2[0]}, slo = {s2[1], s2[1]};
        uint32_t q[4];
        codes4(cw[0][kb], q);
        u32x4 vh, vl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vh[j] = as_u32(as_h2(q[j]) * shi);
          vl[j] = as_u32(as_h2(q[j]) * slo);
        }
        mfma_b(vh);
        mfma_b(vl);
      } else {
        uint32_t o[4];
        dequant4(cw[0][kb], s2, o, nk);
        mfma_b((u32x4){o[0], o[1], o[2], o[3]});
      }
    } else {
      uint32_t lo[4], hi[4], full[4];
      codes8(cw[kb >> 1][2 * (kb & 1)], cw[kb >> 1][2 * (kb & 1) + 1], lo, hi, nk, split ? full : nullptr);
      const f16x2 sh = split ? (f16x2){s2[0], s2[0]} : s2;
      const f16x2 s16 = sh * (f16x2){(_Float16)16.0f, (_Float16)16.0f};
      u32x4 vl, vh;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vl[j] = as_u32(as_h2(lo[j]) * sh);
        vh[j] = as_u32(as_h2(hi[j]) * s16);
      }
      mfma_b(vl);
      mfma_b(vh);
      if (split) {
        const f16x2 slo = {s2[1], s2[1]};
        u32x4 vf;
#pragma unroll
        for (int j = 0; j < 4; ++j) vf[j] = as_u32(as_h2(full[j]) * slo);
        mfma_b(vf);
      }
    }
  };

  f32x4 ag[CT][RT], au[CT][RT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      ag[ct][t] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
      au[ct][t] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    }
  // the codes into the MFMA's order (lane 16 h + r from lane 4 r + h)
  auto arrange = [&](SkinnyChunk<BITS_G, BITS_U, RT, CT>& d, int ct) {
    auto move = [&](u32x4* cw, auto bits_tag) {
      constexpr int BITS = decltype(bits_tag)::value;
      if constexpr (BITS == 2) {
        const uint32_t v0 = (uint32_t)__builtin_amdgcn_ds_bpermute(perm, (int)cw[0][0]);
        const uint32_t v1 = (uint32_t)__builtin_amdgcn_ds_bpermute(perm, (int)cw[0][1]);
        cw[0] = (u32x4){spread2(v0), spread2(v0 >> 16), spread2(v1), spread2(v1 >> 16)};
      } else {
#pragma unroll
        for (int i = 0; i < BITS / 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) cw[i][j] = (uint32_t)__builtin_amdgcn_ds_bpermute(perm, (int)cw[i][j]);
      }
    };
    move(d.cg[ct], std::integral_constant<int, BITS_G>{});
    move(d.cu[ct], std::integral_constant<int, BITS_U>{});
  };
  auto compute = [&](SkinnyChunk<BITS_G, BITS_U, RT, CT>& d) {
#pragma unroll
   for (int ct = 0; ct < CT; ++ct) {
    arrange(d, ct);
    // a chunk past the end gets zero scales and biases: its B operands vanish
    // (scaled by the column's 2^-k)
    const int kg_ = k_gate(ct), ku_ = k_up(ct);
    const float sg = d.live ? ldexpf(act_to_f32((uint16_t)d.sg[ct], ACT), -kg_) : 0.0f;
    const float bg = d.live ? ldexpf(act_to_f32((uint16_t)d.bg[ct], ACT), -kg_) : 0.0f;
    const float su = d.live ? ldexpf(act_to_f32((uint16_t)d.su[ct], ACT), -ku_) : 0.0f;
    const float bu = d.live ? ldexpf(act_to_f32((uint16_t)d.bu[ct], ACT), -ku_) : 0.0f;
    constexpr bool split = ACT == kActF16;
    const f16x2 sg2 = split ? split_scale(sg) : (f16x2){(_Float16)sg, (_Float16)sg};
    const f16x2 su2 = split ? split_scale(su) : (f16x2){(_Float16)su, (_Float16)su};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f16x8 a[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) a[t] = __builtin_bit_cast(f16x8, d.x[t][kb]);
      block_mfma.template operator()<BITS_G>(d.cg[ct], sg2, split, kb, a, ag[ct]);
      block_mfma.template operator()<BITS_U>(d.cu[ct], su2, split, kb, a, au[ct]);
    }
    // bias term sum_k x'_k c of this chunk (c = b + z s split into two
    // binary16 parts, c_hi + c_lo; every product exact):
    const float cgf = fmaf(CodeOffset<BITS_G>::z, sg, bg), cuf = fmaf(CodeOffset<BITS_U>::z, su, bu);
    const _Float16 cgh = (_Float16)cgf, cgl = (_Float16)(cgf - (float)cgh);
    const _Float16 cuh = (_Float16)cuf, cul = (_Float16)(cuf - (float)cuh);
    if constexpr (SELF) {
      // x converted by the wave, which summed x' as it went: K slots
      // (hi, hi, lo) of that sum against (c_hi, c_lo, c_hi)
      const _Float16 z0 = (_Float16)0.0f;
      const f16x8 beg = {cgh, cgl, cgh, z0, z0, z0, z0, z0};
      const f16x8 beu = {cuh, cul, cuh, z0, z0, z0, z0, z0};
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const float sx = d.sx[t];
        const _Float16 xhi = (_Float16)sx, xlo = (_Float16)(sx - (float)xhi);
        const f16x8 ae = {xhi, xhi, xlo, z0, z0, z0, z0, z0};
        ag[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ae, beg, ag[ct][t], 0, 0, 0);
        au[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ae, beu, au[ct][t], 0, 0, 0);
      }
    } else {
      // x' staged elsewhere: the block's A operands once more against
      // B = c_hi and B = c_lo in every K slot of the lane's chunk (MFMAs
      // instead of a VALU sum of x')
      const f16x8 bgh = {cgh, cgh, cgh, cgh, cgh, cgh, cgh, cgh}, bgl = {cgl, cgl, cgl, cgl, cgl, cgl, cgl, cgl};
      const f16x8 buh = {cuh, cuh, cuh, cuh, cuh, cuh, cuh, cuh}, bul = {cul, cul, cul, cul, cul, cul, cul, cul};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const f16x8 a = __builtin_bit_cast(f16x8, d.x[t][kb]);
          ag[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bgh, ag[ct][t], 0, 0, 0);
          au[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, buh, au[ct][t], 0, 0, 0);
          ag[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bgl, ag[ct][t], 0, 0, 0);
          au[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bul, au[ct][t], 0, 0, 0);
        }
    }
   }
  };

  // chunk quads w, w + nw, ... (Q2: 2w and 2w + 1 in one pass, then 2(w + nw), ...).
  // When one pass loads every quad of the row, each wave takes its own
  // column exponents from the scales and biases its loads brought (the
  // largest term of its chunks of the column: two swaps, no barrier); its
  // partial sums are multiplied by 2^k before the waves add them, so waves
  // may differ.  A wave's maximum is at most the row's, so exactness holds
  // as for the row's k.  Otherwise the exponents come from the prep kernel
  // (x' staged there) or the block's own pass (STAGE).
  const int nquad = (nchunk + 3) >> 2;
  const bool single = nquad <= (Q2 ? 2 : 1) * nw;

  // SELF: the rows of x over the wave's chunks chunk0 .. chunk0 + kSelfChunks
  // - 1 into its region, one (chunk slot s, row m) pair of 64 bytes per four
  // lanes, at (s M + m) 64, its 16-byte pieces permuted by (m >> 2) & 3 so
  // that the reads below (16 rows, one piece) spread over all banks.  A chunk
  // past H, or a pair past the last, reads zeros.  Issued before every other
  // load of the wave, so one vmcnt wait covers them.
  const i32x4 rxs = make_srsrc(p.x, (uint32_t)(p.M * p.H * 2));
  // pr / M as (pr * ceil(2^16 / M)) >> 16: exact for pr < 2^16 / M, and pr < 16 kSelfChunks here
  const uint32_t inv_m = (65536u + (uint32_t)p.M - 1u) / (uint32_t)p.M;
  auto dma_x = [&](int chunk0) {
    const int np = kSelfChunks * p.M;
    for (int j = 0; 16 * j < np; ++j) {
      const int pr = 16 * j + (lane >> 2);
      const int sl = (int)(((uint32_t)pr * inv_m) >> 16), m = pr - sl * p.M;
      const int c = chunk0 + sl;
      const int kb = (lane & 3) ^ ((m >> 2) & 3);
      const uint32_t off = (pr < np && c < nchunk) ? (uint32_t)((m * p.H + 32 * c + 8 * kb) * 2) : 0x7FFFFFF0u;
      dma16(rxs, lds_addr(xreg) + 1024 * j, off);
    }
  };
  // ... chunk slot 4 qs + h of row r back, as the MFMA's A operand (bf16
  // bits).  A lane of a row past M reads row M - 1 again: A's rows past M
  // only reach D's rows past M, which are never stored.
  auto read_x = [&](int qs, SkinnyChunk<BITS_G, BITS_U, RT, CT>& d) {
    const int sl = 4 * qs + h;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int m = rowl[t];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        d.x[t][q] = *reinterpret_cast<const u32x4*>(xreg + (sl * p.M + m) * 64 + 16 * (q ^ ((m >> 2) & 3)));
    }
  };
  // loads the wave issues after its x: the windows of groups (at least 4)
  // and the codes of its quads
  constexpr int kLoadsAfterX = CT * (4 + (Q2 ? 2 : 1) * ((BITS_G == 8 ? 2 : 1) + (BITS_U == 8 ? 2 : 1)));

  // SELF: the largest bf16 magnitude of each of this lane's rows (packed
  // halves, folded at the end), over the wave's chunks ...
  uint32_t xam[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) xam[t] = 0;
  auto x_amax = [&](const SkinnyChunk<BITS_G, BITS_U, RT, CT>& d) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xam[t] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, xam[t]),
                                                                          __builtin_bit_cast(u16x2, d.x[t][q][j] & 0x7FFF7FFFu)));
  };
  // ... the row exponents e (the lanes of a row meet with two swaps; the
  // accumulator rows' exponents packed as in the preload) ...  When every
  // row's largest magnitude lies in [1, 2^10) (0 <= e <= 9) the wave takes
  // e = 0 instead, x' = x: x fits binary16, a chunk's sum of x' (carried as
  // binary16 hi + lo) stays below 2^15, and an element is exact in binary16
  // down to 2^-17 (binary16 x: 2^-14), not 2^(e - 17): at least as exact as
  // with the row's own power of two.
  int xe_self[RT];
  bool xe_zero = false;
  auto x_rows = [&]() {
    bool in_range = true;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      uint32_t a = max(xam[t] & 0xFFFFu, xam[t] >> 16);
      a = max(a, (uint32_t)__shfl_xor((int)a, 16));
      a = max(a, (uint32_t)__shfl_xor((int)a, 32));
      xe_self[t] = x_exponent(a, ACT);
      in_range = in_range && xe_self[t] >= 0 && xe_self[t] <= 9;
    }
    xe_zero = __all(in_range);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      if (xe_zero) xe_self[t] = 0;
      xrow_e[t] = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) xrow_e[t] |= (uint32_t)(__shfl(xe_self[t], 4 * h + j) + 128) << (8 * j);
    }
  };
  // ... and x' = x 2^-e in binary16, in the code-pair order (word j of a
  // block holds inputs j and j + 4), in place, with the lane's sum of x'
  // for the bias term (float32 adds of x 2^-e, which is x' wherever binary16
  // holds it exactly; done here, while the weights are still in flight)
  auto x_convert = [&](SkinnyChunk<BITS_G, BITS_U, RT, CT>& d) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      d.sx[t] = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 v = d.x[t][q];
        float f[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f[2 * j] = act_to_f32((uint16_t)(v[j] & 0xFFFFu), ACT);
          f[2 * j + 1] = act_to_f32((uint16_t)(v[j] >> 16), ACT);
        }
        if (!xe_zero) {
#pragma unroll
          for (int j = 0; j < 8; ++j) f[j] = ldexpf(f[j], -xe_self[t]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) d.x[t][q][j] = as_u32((f16x2){(_Float16)f[j], (_Float16)f[j + 4]});
#pragma unroll
        for (int j = 0; j < 8; ++j) d.sx[t] += f[j];
      }
    }
  };
  float cmax_g[CT], cmax_u[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) cmax_g[ct] = cmax_u[ct] = 0.0f;
  auto chunk_k = [&](const SkinnyChunk<BITS_G, BITS_U, RT, CT>& d) {
    if (!d.live) return;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      cmax_g[ct] = fmaxf(cmax_g[ct], group_term_max(act_to_f32((uint16_t)d.sg[ct], ACT), act_to_f32((uint16_t)d.bg[ct], ACT),
                                                    CodeOffset<BITS_G>::z, kPlaneMax<BITS_G>));
      cmax_u[ct] = fmaxf(cmax_u[ct], group_term_max(act_to_f32((uint16_t)d.su[ct], ACT), act_to_f32((uint16_t)d.bu[ct], ACT),
                                                    CodeOffset<BITS_U>::z, kPlaneMax<BITS_U>));
    }
  };
  auto chunk_k_wave = [&]() {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      float g = cmax_g[ct], u = cmax_u[ct];
      g = fmaxf(g, __shfl_xor(g, 16));
      g = fmaxf(g, __shfl_xor(g, 32));
      u = fmaxf(u, __shfl_xor(u, 16));
      u = fmaxf(u, __shfl_xor(u, 32));
      set_k(ct, row_exponent_k(g), row_exponent_k(u));
    }
  };
  if constexpr (STAGE) {
    // the first quad's weights are in flight while the block builds x'
    SkinnyChunk<BITS_G, BITS_U, RT, CT> d;
    SbWindow<CT> sw;
    if (w < nquad) {
      load_sb(w, sw);
      load(w, d);
    }
    if (single) {
      if (w < nquad) {
        pick_sb(sw, w, d);
        chunk_k(d);
      }
      chunk_k_wave();
    } else {
      row_k_finish();
    }
    const int nt = blockDim.x, nblk = p.M * (p.H >> 3);   // 8-value blocks of x
    if (tid < p.M) xmax[tid] = 0;
    __syncthreads();
    if (!single) row_k_read();
    for (int b = tid; b < nblk; b += nt) {              // row maxima of |x| (bf16 magnitude bits)
      const u32x4 v = *reinterpret_cast<const u32x4*>(p.x + 8 * (int64_t)b);
      uint32_t amax = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) amax = max(amax, max(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
      atomicMax(&xmax[b / (p.H >> 3)], amax);
    }
    __syncthreads();
    if (tid < p.M) xe[tid] = x_exponent(xmax[tid], ACT);
    __syncthreads();
    for (int b = tid; b < nblk; b += nt) {              // x' = x 2^-e in the code-pair order
      const int m = b / (p.H >> 3), k8 = b - m * (p.H >> 3);
      const u32x4 v = *reinterpret_cast<const u32x4*>(p.x + 8 * (int64_t)b);
      const int e = xe[m];
      float f[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[2 * j] = ldexpf(act_to_f32((uint16_t)(v[j] & 0xFFFFu), ACT), -e);
        f[2 * j + 1] = ldexpf(act_to_f32((uint16_t)(v[j] >> 16), ACT), -e);
      }
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = as_u32((f16x2){(_Float16)f[j], (_Float16)f[j + 4]});
      xs[((k8 >> 2) * p.M + m) * 4 + (k8 & 3)] = o;
    }
    __syncthreads();
    for (int q0 = w; q0 < nquad; q0 += nw) {
      if (q0 != w) {
        load_sb(q0, sw);
        load(q0, d);
      }
      load_x_lds(q0, d);
      pick_sb(sw, q0, d);
      compute(d);
    }
  } else if constexpr (!Q2) {
    if (single) {
      SkinnyChunk<BITS_G, BITS_U, RT, CT> d;
      SbWindow<CT> sw;
      if (w < nquad) {
        if constexpr (SELF) dma_x(4 * w);
        load_sb(w, sw);
        load(w, d);
        if constexpr (SELF) {   // x arrives first (L2): convert it while the weights are in flight
          wait_vmcnt<kLoadsAfterX>();
          read_x(0, d);
          x_amax(d);
        }
      }
      if constexpr (SELF) x_rows();
      if (w < nquad) {
        if constexpr (SELF) x_convert(d);
        pick_sb(sw, w, d);
        chunk_k(d);
      }
      chunk_k_wave();
      if (w < nquad) compute(d);
    } else if constexpr (!SELF) {   // (SELF is launched for one pass only)
      for (int q0 = w; q0 < nquad; q0 += nw) {
        SkinnyChunk<BITS_G, BITS_U, RT, CT> d;
        SbWindow<CT> sw;
        load_sb(q0, sw);
        load(q0, d);
        pick_sb(sw, q0, d);
        compute(d);
      }
    }
  } else {
    // two adjacent chunk quads in flight per wave, half the waves (a quad
    // past the end loads chunk 0 with zero scales and adds nothing)
    if (single) {
      SkinnyChunk<BITS_G, BITS_U, RT, CT> d0, d1;
      SbWindow<CT> sw;   // one window holds both quads' groups
      if (2 * w < nquad) {
        if constexpr (SELF) dma_x(8 * w);
        load_sb(2 * w, sw);
        load(2 * w, d0);
        load(2 * w + 1, d1);
        if constexpr (SELF) {   // x arrives first (L2): convert it while the weights are in flight
          wait_vmcnt<kLoadsAfterX>();
          read_x(0, d0);
          read_x(1, d1);
          x_amax(d0);
          x_amax(d1);
        }
      }
      if constexpr (SELF) x_rows();
      if (2 * w < nquad) {
        if constexpr (SELF) {
          x_convert(d0);
          x_convert(d1);
        }
        pick_sb(sw, 2 * w, d0);
        pick_sb(sw, 2 * w + 1, d1);
        chunk_k(d0);
        chunk_k(d1);
      }
      chunk_k_wave();
      if (2 * w < nquad) {
        compute(d0);
        compute(d1);
      }
    } else if constexpr (!SELF) {
      for (int pq = w; 2 * pq < nquad; pq += nw) {   // adjacent quads: their code rows share lines
        SkinnyChunk<BITS_G, BITS_U, RT, CT> d0, d1;
        SbWindow<CT> sw;
        load_sb(2 * pq, sw);
        load(2 * pq, d0);
        load(2 * pq + 1, d1);
        pick_sb(sw, 2 * pq, d0);
        pick_sb(sw, 2 * pq + 1, d1);
        compute(d0);
        compute(d1);
      }
    }
  }

  // the waves' partial sums in their true scale, times 2^(k + e) (weight
  // column and x row; one scaling, so no intermediate leaves the range of
  // the sums themselves); D element j of lane l is row 4 (l / 16) + j,
  // column l % 16
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int kg_ = k_gate(ct), ku_ = k_up(ct);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      f32x4 a = ag[ct][t], b = au[ct][t];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = 16 * t + 4 * h + j;
        int e;
        if constexpr (kPreE || SELF) e = (int)((xrow_e[t] >> (8 * j)) & 0xFFu) - 128;
        else if constexpr (STAGE) e = m < p.M ? xe[m] : 0;
        else e = m < p.M ? p.xexp[m] : 0;
        a[j] = ldexpf(a[j], kg_ + e);
        b[j] = ldexpf(b[j], ku_ + e);
      }
      red_at(w, 2 * (ct * RT + t))[lane] = a;
      red_at(w, 2 * (ct * RT + t) + 1)[lane] = b;
    }
  }
  __syncthreads();
  // element j of D (row 16 t + 4 h + j) of row tile t and column tile ct:
  // wave 4 (ct RT + t) + j sums it over the waves (in wave order) and runs
  // its epilogue, so the 4 RT CT epilogues of a lane run on different waves
  // at once
  for (int k = w; k < 4 * RT * CT; k += nw) {
    const int tt = k >> 2, j = k & 3;                 // tt = ct RT + t
    const int t = tt % RT, c16 = col + 16 * (tt / RT);
    float g = 0.0f, u = 0.0f;
    for (int ww = 0; ww < nw; ++ww) {
      g += red_at(ww, 2 * tt)[lane][j];
      u += red_at(ww, 2 * tt + 1)[lane][j];
    }
    const int m = 16 * t + 4 * h + j;
    if (m < p.M && c16 < p.I) store_out(p, m0 + m, c16, g, u, ACT);
  }
}

// ------------------------------------------------------------ launchers ----

// lanes per column: one 32-input chunk per lane, at most a wavefront
static int gemv_lanes_per_column(int H) {
  const int chunks = H / 32;
  int l = 1;
  while (l * 2 <= chunks && l * 2 <= 64) l *= 2;
  return l;
}

template <int BG, int BU, int CPL, bool FULL, int ACT>
static hipError_t launch_gemv1_t(const GemvParams& p, int R, hipStream_t stream) {
  constexpr int WPB = 4;
  const int lpc = gemv_lanes_per_column(p.H);
  int lg = 0;
  while ((1 << lg) < lpc) ++lg;
  const int cpw = 64 / lpc;
  const int cols_per_wave = cpw * R;
  const int waves = (p.I + cols_per_wave - 1) / cols_per_wave;
  if (p.H > kGemv1MaxH || p.H / 8 > 256 * CPL) return hipErrorInvalidValue;
  const int blocks = (waves + WPB - 1) / WPB;
  switch (R) {
    case 1: hipLaunchKernelGGL((swq_gemv1_kernel<BG, BU, CPL, 1, FULL, WPB, 1, ACT>), dim3(blocks), dim3(64 * WPB), 0, stream, p, lg); break;
    case 2: hipLaunchKernelGGL((swq_gemv1_kernel<BG, BU, CPL, 2, FULL, WPB, 1, ACT>), dim3(blocks), dim3(64 * WPB), 0, stream, p, lg); break;
    case 4: hipLaunchKernelGGL((swq_gemv1_kernel<BG, BU, CPL, 4, FULL, WPB, 1, ACT>), dim3(blocks), dim3(64 * WPB), 0, stream, p, lg); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The several-row form (gemv1_rows_shape): a whole wave per column, R (one
// or two) columns per wave.
template <int BG, int BU, int CPL, bool FULL, int ACT>
static hipError_t launch_gemv1_rows_t(const GemvParams& p, int R, hipStream_t stream) {
  constexpr int WPB = 4;
  const int lpc = gemv_lanes_per_column(p.H);
  int lg = 0;
  while ((1 << lg) < lpc) ++lg;
  const int cols_per_wave = 64 / lpc * R;
  const int waves = (p.I + cols_per_wave - 1) / cols_per_wave;
  if (!gemv1_rows_shape(p.M, p.H) || lpc != 64 || p.H / 8 > 256 * CPL) return hipErrorInvalidValue;
  static_assert(kGemv1MaxRows == 4, "one instance per row count");
  const int blocks = (waves + WPB - 1) / WPB;
  const dim3 g(blocks), b(64 * WPB);
  switch (R * 8 + p.M) {
    case 8 + 2: hipLaunchKernelGGL((swq_gemv1_kernel<BG, BU, CPL, 1, FULL, WPB, 2, ACT>), g, b, 0, stream, p, lg); break;
    case 8 + 3: hipLaunchKernelGGL((swq_gemv1_kernel<BG, BU, CPL, 1, FULL, WPB, 3, ACT>), g, b, 0, stream, p, lg); break;
    case 8 + 4: hipLaunchKernelGGL((swq_gemv1_kernel<BG, BU, CPL, 1, FULL, WPB, 4, ACT>), g, b, 0, stream, p, lg); break;
    case 16 + 2: hipLaunchKernelGGL((swq_gemv1_kernel<BG, BU, CPL, 2, FULL, WPB, 2, ACT>), g, b, 0, stream, p, lg); break;
    case 16 + 3: hipLaunchKernelGGL((swq_gemv1_kernel<BG, BU, CPL, 2, FULL, WPB, 3, ACT>), g, b, 0, stream, p, lg); break;
    case 16 + 4: hipLaunchKernelGGL((swq_gemv1_kernel<BG, BU, CPL, 2, FULL, WPB, 4, ACT>), g, b, 0, stream, p, lg); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Columns per wave: two, or one when that leaves fewer than 2048 waves
// (fewer columns than 4096), so that a small output still spreads over the
// chip.  SWIGLU_Q_GEMV_ROUNDS (1, 2 or 4) overrides.
static int gemv1_rounds(int I) {
  static const int r = [] {
    const char* s = getenv("SWIGLU_Q_GEMV_ROUNDS");
    const int v = s ? atoi(s) : 0;
    return (v == 1 || v == 2 || v == 4) ? v : 0;
  }();
  return r ? r : (I >= 4096 ? 2 : 1);
}

#if SWQ_GEMV_ACT == 0
// SWIGLU_Q_GEMV1_ROWS=0 sends 2 <= M <= kGemv1MaxRows to the few-row MFMA
// kernel instead (for comparisons).
bool gemv1_rows_enabled() {
  static const bool on = [] {
    const char* s = getenv("SWIGLU_Q_GEMV1_ROWS");
    return !(s && s[0] == '0');
  }();
  return on;
}
#endif

// Waves per block of the few-row kernel and whether it takes two chunk quads
// per pass (the launcher's choice below), for x source xs.
static void skinny_shape(int64_t M, int64_t H, int bits_g, int bits_u, int xs, int* waves, bool* two) {
  const int quads = (int)((H / 32 + 3) / 4);
  // (equal widths of at most 4 bits: mixed 2- and 4-bit codes would not fit
  // two quads in the registers of four waves per SIMD).  x' from the prep
  // kernel: two quads measured faster with two row tiles everywhere, and with
  // one up to H = 2048 (slower beyond, at half the waves per SIMD, where the
  // rows take several passes); x converted by the waves themselves (M <= 16):
  // two quads whenever the codes allow, which doubles the row one pass covers
  const bool narrow = bits_g <= 4 && bits_u <= 4 && bits_g == bits_u;
  // (SWIGLU_Q_SKINNY_QUADS=1, read on every call: one quad per wave, for
  // comparisons and tests)
  const char* q = getenv("SWIGLU_Q_SKINNY_QUADS");
  if (xs == kXSelf) *two = narrow && M <= 16 && !(q && q[0] == '1' && q[1] == 0);
  else *two = narrow && xs == kXPrep && (M > 16 || H <= 2048);
  const int per = *two ? (quads + 1) / 2 : quads;
  *waves = per < kSkinnyMaxWaves ? per : kSkinnyMaxWaves;
}

// x' converted by each wave itself for M <= 16 whenever a row fits one pass
// of the block's waves, their LDS regions fit kSkinnySelfMaxLds and the block
// has more than one wave (no second launch, no workspace); for 16 < M <= 32
// (two row tiles) likewise with narrow codes and one chunk quad per wave,
// within kSkinnySelfRt2MaxLds; else built in LDS by each block for
// M*H <= kSkinnyStageMax; else from the prep kernel.
// SWIGLU_Q_SKINNY_X=prep or =stage (where M*H allows) overrides, for
// comparisons and for tests of those sources.
#if SWQ_GEMV_ACT == 0
int skinny_x_source(int64_t M, int64_t H, int bits_g, int bits_u) {
  const char* env = getenv("SWIGLU_Q_SKINNY_X");
  if (env && strcmp(env, "prep") == 0) return kXPrep;
  if (env && strcmp(env, "stage") == 0 && M <= kGemvMaxM && M * H <= kSkinnyStageMax) return kXStage;
  // (more than kGemvMaxM rows: row groups of kGemvMaxM, never built in the block)
  const int64_t Mg = M > kGemvMaxM ? kGemvMaxM : M;
  int waves;
  bool two;
  skinny_shape(Mg, H, bits_g, bits_u, kXSelf, &waves, &two);
  const bool stage = M <= kGemvMaxM && M * H <= kSkinnyStageMax;
  // (a one-wave block, H <= 256 with two quads per wave, converts faster in
  // the block: measured 4.4 against 4.9 us at M = 6, H = 256, I = 768)
  if (Mg <= 16 && (H / 32 + 3) / 4 <= (two ? 2 : 1) * waves &&
      waves * skinny_self_region((int)Mg, two ? 8 : 4) <= kSkinnySelfMaxLds && !(waves == 1 && stage))
    return kXSelf;
  const bool narrow = bits_g <= 4 && bits_u <= 4 && bits_g == bits_u;
  if (Mg > 16 && narrow && (H / 32 + 3) / 4 <= waves && waves > 1 &&
      waves * skinny_self_region((int)Mg, 4, 4) <= kSkinnySelfRt2MaxLds)
    return kXSelf;
  return stage ? kXStage : kXPrep;
}

bool skinny_needs_kexp(int M, int H, int bits_g, int bits_u) {
  int waves;
  bool two;
  skinny_shape(M > kGemvMaxM ? kGemvMaxM : M, H, bits_g, bits_u, kXPrep, &waves, &two);
  return (H / 32 + 3) / 4 > (two ? 2 : 1) * waves;
}
#endif

// Column tiles per block of the few-row kernel: two (with one chunk quad per
// wave, the row in one pass of at most kSkinnyMaxWaves waves) when each wave
// converts x itself, the codes are narrow, and the 16-column tiles are more
// than the device's CUs -- with one row tile, at most twice as many: each
// conversion of x serves both tiles, instead of some CUs taking a second
// block of 16 (measured at H = 2048: I = 5632, M = 8 / 16: 9.04 / 10.12 ->
// 8.59 / 9.21 us; one tile stays ahead at most one round of tiles, and with
// one row tile at 3.5 rounds, where two of its blocks share a CU).
// SWIGLU_Q_SKINNY_CT=1 or 2 (read on every call) overrides where two are
// possible, for comparisons and tests.
static int skinny_ct(int64_t I, int xs, bool narrow, int quads, int rt) {
  if (xs != kXSelf || !narrow || quads > kSkinnyMaxWaves) return 1;
  if (const char* s = getenv("SWIGLU_Q_SKINNY_CT"); s && (s[0] == '1' || s[0] == '2') && s[1] == 0) return s[0] - '0';
  const int64_t tiles = (I + 15) / 16, cus = device_cus();
  return tiles > cus && (rt == 2 || tiles <= 2 * cus) ? 2 : 1;
}

// Two row tiles with x converted by the waves: regions past 64 KB of
// dynamic LDS, allowed once per instance (and device) before the launch.
template <int BG, int BU, int ACT, int CT>
static void launch_self_rt2(dim3 g, dim3 b, int lds, hipStream_t stream, const GemvParams& p) {
  auto kern = swq_skinny_kernel<BG, BU, kXSelf, 2, false, ACT, CT>;
  constexpr int kDevices = 64;
  static std::once_flag once[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kDevices)
    std::call_once(once[dev], [&] {
      (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kSkinnySelfRt2MaxLds);
    });
  hipLaunchKernelGGL(kern, g, b, lds, stream, p);
}

template <int BG, int BU, int ACT>
static hipError_t launch_gemv_bits(const GemvParams& p, hipStream_t stream) {
  const int lpc = gemv_lanes_per_column(p.H);
  const int cpl = (p.H / 32 + lpc - 1) / lpc;
  if (p.M == 1 && cpl <= 4) {
    const bool full = lpc == 64 && p.H == 2048 * cpl;
    const int r = gemv1_rounds(p.I);
    switch (cpl) {
      case 1: return full ? launch_gemv1_t<BG, BU, 1, true, ACT>(p, r, stream) : launch_gemv1_t<BG, BU, 1, false, ACT>(p, r, stream);
      case 2: return full ? launch_gemv1_t<BG, BU, 2, true, ACT>(p, r, stream) : launch_gemv1_t<BG, BU, 2, false, ACT>(p, r, stream);
      case 3: return full ? launch_gemv1_t<BG, BU, 3, true, ACT>(p, r, stream) : launch_gemv1_t<BG, BU, 3, false, ACT>(p, r, stream);
      default: return full ? launch_gemv1_t<BG, BU, 4, true, ACT>(p, r, stream) : launch_gemv1_t<BG, BU, 4, false, ACT>(p, r, stream);
    }
  }
  if (gemv1_rows_shape(p.M, p.H)) {
    static_assert(kGemv1RowsMaxH <= 2 * 2048, "at most two chunks per lane");
    const bool full = lpc == 64 && p.H == 2048 * cpl;
    const int r = gemv1_rounds(p.I) >= 2 ? 2 : 1;
    if (cpl == 1) return full ? launch_gemv1_rows_t<BG, BU, 1, true, ACT>(p, r, stream) : hipErrorInvalidValue;   // H = 2048
    return full ? launch_gemv1_rows_t<BG, BU, 2, true, ACT>(p, r, stream) : launch_gemv1_rows_t<BG, BU, 2, false, ACT>(p, r, stream);
  }
  if (p.M < 1 || p.M > kGemvGroupsMaxM) return hipErrorInvalidValue;
  // row groups of kGemvMaxM rows (grid y); Mg: the rows of a full group
  const int groups = (p.M + kGemvMaxM - 1) / kGemvMaxM;
  const int Mg = groups > 1 ? kGemvMaxM : p.M;
  // one wave per chunk quad (or pair of quads), at most kSkinnyMaxWaves per
  // block of 16 columns
  constexpr bool kNarrow = BG <= 4 && BU <= 4 && BG == BU;
  const int xs = p.xa != nullptr ? kXPrep : skinny_x_source(p.M, p.H, BG, BU);
  int waves;
  bool two;
  skinny_shape(Mg, p.H, BG, BU, xs, &waves, &two);
  const int quads = (p.H / 32 + 3) / 4;
  if (xs == kXPrep && (p.xa == nullptr || (p.kexp == nullptr && skinny_needs_kexp(p.M, p.H, BG, BU))))
    return hipErrorInvalidValue;
  if (xs == kXStage && (groups > 1 || (int64_t)p.M * p.H > kSkinnyStageMax)) return hipErrorInvalidValue;
  const int rt = Mg > 16 ? 2 : 1;
  const int ct = skinny_ct(p.I, xs, kNarrow, quads, rt);
  if (ct == 2) {   // one quad per wave
    two = false;
    waves = quads;
  }
  const int lds = xs == kXSelf ? waves * skinny_self_region(Mg, two ? 8 : 4, ct * rt) : 0;
  if (xs == kXSelf && (quads > (two ? 2 : 1) * waves || (rt == 2 && (two || !kNarrow)) ||
                       lds > (rt == 2 ? kSkinnySelfRt2MaxLds : kSkinnySelfMaxLds)))
    return hipErrorInvalidValue;   // one pass, regions within bounds; two row tiles: one quad per wave
  const dim3 g((p.I + 16 * ct - 1) / (16 * ct), groups), b(64 * waves);
  auto go = [&](auto xs_tag, auto two_tag) {
    constexpr int XS = decltype(xs_tag)::value;
    constexpr bool TWO = decltype(two_tag)::value;
    if constexpr (XS == kXSelf && kNarrow && !TWO) {
      if (rt == 2) {
        if (ct == 2) launch_self_rt2<BG, BU, ACT, 2>(g, b, lds, stream, p);
        else launch_self_rt2<BG, BU, ACT, 1>(g, b, lds, stream, p);
      } else if (ct == 2) {
        hipLaunchKernelGGL((swq_skinny_kernel<BG, BU, XS, 1, TWO, ACT, 2>), g, b, lds, stream, p);
      } else {
        hipLaunchKernelGGL((swq_skinny_kernel<BG, BU, XS, 1, TWO, ACT, 1>), g, b, lds, stream, p);
      }
    } else if constexpr (XS == kXSelf) {
      hipLaunchKernelGGL((swq_skinny_kernel<BG, BU, XS, 1, TWO, ACT, 1>), g, b, lds, stream, p);
    } else if (Mg <= 16) {
      hipLaunchKernelGGL((swq_skinny_kernel<BG, BU, XS, 1, TWO, ACT, 1>), g, b, 0, stream, p);
    } else {
      hipLaunchKernelGGL((swq_skinny_kernel<BG, BU, XS, 2, TWO, ACT, 1>), g, b, 0, stream, p);
    }
  };
  using F = std::false_type;
  using T = std::true_type;
  if (xs == kXStage) go(std::integral_constant<int, kXStage>{}, F{});
  else if (!two) {
    if (xs == kXSelf) go(std::integral_constant<int, kXSelf>{}, F{});
    else go(std::integral_constant<int, kXPrep>{}, F{});
  } else if constexpr (kNarrow) {
    if (xs == kXSelf) go(std::integral_constant<int, kXSelf>{}, T{});
    else go(std::integral_constant<int, kXPrep>{}, T{});
  }
  return hipGetLastError();
}

template <int BG, int ACT>
static hipError_t launch_gemv_g(const GemvParams& p, int bits_u, hipStream_t stream) {
  if (bits_u == 2) return launch_gemv_bits<BG, 2, ACT>(p, stream);
  if (bits_u == 4) return launch_gemv_bits<BG, 4, ACT>(p, stream);
  if (bits_u == 8) return launch_gemv_bits<BG, 8, ACT>(p, stream);
  return hipErrorInvalidValue;
}

template <int ACT>
hipError_t launch_gemv_act(const GemvParams& p, int bits_g, int bits_u, hipStream_t stream) {
  if (bits_g == 2) return launch_gemv_g<2, ACT>(p, bits_u, stream);
  if (bits_g == 4) return launch_gemv_g<4, ACT>(p, bits_u, stream);
  if (bits_g == 8) return launch_gemv_g<8, ACT>(p, bits_u, stream);
  return hipErrorInvalidValue;
}

template hipError_t launch_gemv_act<SWQ_GEMV_ACT>(const GemvParams&, int, int, hipStream_t);

#if SWQ_GEMV_ACT == 0
extern template hipError_t launch_gemv_act<kActF16>(const GemvParams&, int, int, hipStream_t);

hipError_t launch_gemv(const GemvParams& p, int bits_g, int bits_u, hipStream_t stream) {
  if (p.act == kActF16) return launch_gemv_act<kActF16>(p, bits_g, bits_u, stream);
  if (p.act == kActBf16) return launch_gemv_act<kActBf16>(p, bits_g, bits_u, stream);
  return hipErrorInvalidValue;
}
#endif

}  // namespace swq
