// Matrix-matrix path (M >= threshold) of the fused quantized SwiGLU:
//   hidden[M, I] = silu(x Wg^T) * (x Wu^T)
// One dispatch produces a BM x 128 tile of BOTH projections from one staged
// x tile, then applies the epilogue in registers ("mlx-bun 0.0.7 -> 0.0.9"
// diff, page 42, fused-swiglu-kernel.ts: header comment and kernel source,
// where x is read once for two GEMMs and down_proj stays separate).
//
// Exactness.  A weight w = s*q + b is split as  s*(q - z) + c  with
// c = b + z*s per group (z = 8 for 4-bit codes, and for 2-bit codes, which
// are spread to nibbles and computed as 4-bit ones; for 8-bit codes
// q = 16 hi + lo and s*q = 16s*(hi - 8) + s*(lo - 8) + 136 s).  Each output
// feature of each matrix first gets its own power of two 2^-k, chosen from
// the row's largest |s| times code offset and largest |c| (see the column
// blocks below), so that s 2^-k (code - 8) and c 2^-k are finite in binary16
// and, with a bf16 scale's 8 significant bits and an offset of at most 4,
// exact for every group within 2^28 (8-bit: 2^24) of the row's largest
// term.  The K loop therefore runs on f16 MFMA with exact products and
// float32 accumulation, and the epilogue multiplies by 2^k.  The constant
// part sum_g Sx[m,g] * c[n,g] runs on the same MFMAs as extra K columns: the
// group sum of x' (float32) split into binary16 hi + lo, against c 2^-k split
// into binary16 c_hi + c_lo, three columns per group: (hi, hi, lo) x
// (c_hi, c_lo, c_hi); the dropped lo*c_lo term is below 2^-22 of the group
// term.
//
// Two kernels:
//  1. swq_prep_kernel.  Blocks [0, M): one row of x each.  It picks a
//     power-of-two row scale 2^-e so that max|x'| lies in [1, 2), writes
//     x' = x * 2^-e as binary16 in the [0,4,1,5,2,6,3,7] order that matches
//     the dequantized weight pairs, and appends the extra columns
//     (hi, hi, lo) of every group of g0 = min(gs_g, gs_u) inputs.  Every bf16
//     x whose magnitude is at least 2^-17 of the row maximum converts
//     exactly.  The column blocks then write, for a run of consecutive
//     output features of both matrices each, the row exponents k, the
//     extra-column B rows (c_hi, c_lo, c_hi) and the scale tiles (binary16
//     scale pairs per K-step, 128 columns at a time).
//  2. swq_mfma_kernel: f16 MFMA 32x32x16 with float32 accumulators over the
//     H columns (packed codes, dequantized in registers) and then the extra
//     columns (precomputed binary16 rows); epilogue 2^(e + k), then
//     silu(g) * u per precision mode, or the two projections as they are for
//     the quantized linear (W's rows split between the gate and up slots).
#include <type_traits>
#include <utility>

#include "swq_device.h"

#include "swq_kernels.h"

namespace swq {

// ---------------------------------------------------------------- prep ----

__device__ __forceinline__ void prep_x_row(const PrepParams& p, int m) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint16_t* xrow = p.x + (int64_t)m * p.H;
  // x' is stored K-step major: the 32 columns [32s, 32s + 32) of row m at
  // ((s * M) + m) * 32 halves, so a row tile of one K-step is contiguous
  auto xa_at = [&](int k) { return p.xa + ((int64_t)(k >> 5) * p.M + m) * 32 + (k & 31); };
  const int nchunk = p.H / 8;

  // 1. row maximum of |x| (on the bf16 magnitude bits: monotone for finite
  //    values); the first kXRegs 8-value blocks of this thread stay in
  //    registers for step 2 (all of them for H <= 8192), the rest are read again
  constexpr int kXRegs = 4;
  u32x4 keep[kXRegs];
  uint32_t amax = 0;
  auto fold = [&](const u32x4& v) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = max(amax, v[j] & 0x7FFFu);
      amax = max(amax, (v[j] >> 16) & 0x7FFFu);
    }
  };
#pragma unroll
  for (int i = 0; i < kXRegs; ++i) {
    const int c = tid + 256 * i;
    keep[i] = c < nchunk ? *reinterpret_cast<const u32x4*>(xrow + 8 * c) : (u32x4){0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < kXRegs; ++i) fold(keep[i]);
  for (int c = tid + 256 * kXRegs; c < nchunk; c += 256) fold(*reinterpret_cast<const u32x4*>(xrow + 8 * c));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
  __shared__ uint32_t red[4];
#ifdef SWQ_LDS_POISON
  lds_poison(red, sizeof(red), kPoisonFloat);
  __syncthreads();
#endif
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = max(max(red[0], red[1]), max(red[2], red[3]));
  // exponent of the row maximum: max|x| in [2^e, 2^(e+1))
  const int e = x_exponent(amax, p.act);
  if (tid == 0) p.xexp[m] = e;

  // 2. scaled binary16 copy in pair order, and per-group sums
  const int gchunks = p.g0 / 8;
  const int ngroups = p.H / p.g0;
  for (int base = 0, i = 0; base < nchunk; base += 256, ++i) {
    const int c = base + tid;
    float part = 0.0f;
    if (c < nchunk) {
      u32x4 v;
      if (i < kXRegs) {
#pragma unroll
        for (int q = 0; q < kXRegs; ++q)
          if (q == i) v = keep[q];
      } else {
        v = *reinterpret_cast<const u32x4*>(xrow + 8 * c);
      }
      float f[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[2 * j] = ldexpf(act_to_f32((uint16_t)(v[j] & 0xFFFFu), p.act), -e);
        f[2 * j + 1] = ldexpf(act_to_f32((uint16_t)(v[j] >> 16), p.act), -e);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) part += f[j];
      f16x8 h;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[2 * j] = (_Float16)f[j];
        h[2 * j + 1] = (_Float16)f[j + 4];
      }
      if (p.xlane) {                                   // the few-row kernel's lane order
        const int chunk = c >> 2, kb = c & 3;
        const int64_t unit = ((int64_t)((chunk >> 2) * p.xlane + (m >> 4)) * 4 + kb) * 64 + (chunk & 3) * 16 + (m & 15);
        *reinterpret_cast<f16x8*>(p.xa + unit * 8) = h;
      } else {
        *reinterpret_cast<f16x8*>(xa_at(8 * c)) = h;
      }
    }
    // a group is g0/8 consecutive 8-value blocks = consecutive lanes
    for (int off = 1; off < gchunks; off <<= 1) part += __shfl_xor(part, off);
    if (!p.xlane && c < nchunk && (c % gchunks) == 0) {
      const int g = c / gchunks;
      const _Float16 hi = (_Float16)part;
      const _Float16 lo = (_Float16)(part - (float)hi);
      *xa_at(p.H + 3 * g) = hi;
      *xa_at(p.H + 3 * g + 1) = hi;
      *xa_at(p.H + 3 * g + 2) = lo;
    }
  }
  // zero padding of the extra columns
  if (!p.xlane)
    for (int k = 3 * ngroups + tid; k < p.kext; k += 256) *xa_at(p.H + k) = (_Float16)0.0f;
}

// Weight rows.  Thread ((n * 2 + matrix) << lg) + c owns extra-column slot c
// (eight g0-groups) of output feature n of one matrix and the scale-tile
// words of the K-steps those groups cover.  The 2^lg threads of a row are
// consecutive lanes of one wave (2^lg <= 64), so the row exponent k
// (row_exponent_k) is a maximum over those lanes; a row with more than 64
// slots gives each thread slots c, c + 64, ... (loaded once for the maximum
// and again for the stores).  Each thread then writes
//  - the slot's extra-column B row entries (c_hi, c_lo, c_hi) of c 2^-k, with
//    c = b + z s in float32 and zeros past the last group, as three 16-byte
//    stores (a row is kext*2 bytes, a multiple of 64, so each store lies
//    wholly inside or outside it);
//  - for every K-step (32 inputs) of its groups below H, the scale-tile word
//    (s 2^-k, s 2^-k) in binary16 of that K-step's group (binary16 scales:
//    split_scale(s 2^-k), the two parts of two MFMA planes): through LDS,
//    where the block stores its features' words as whole 16-byte pieces
//    (see kPrepWordsLds), else one store per word;
//  - (slot 0) k itself, for the MFMA kernel's epilogue.
// With k_only (the matrix-vector path) only k is written.  The MFMA kernel
// never reads scale-tile words of K-steps past H or of columns past the rows,
// and they are left unwritten.
struct RowSpec {
  const uint16_t* S;
  const uint16_t* B;
  int lg_gs;      // log2 of the group size
  int ng;         // groups per row
  float z, F;     // code offset; largest |offset| times plane weight
  int act;        // type of the scales and biases (kActBf16, kActF16)
};

__device__ __forceinline__ RowSpec row_spec(const PrepParams& p, int mat) {
  RowSpec r;
  const int gs = mat ? p.gs_u : p.gs_g, bits = mat ? p.bits_u : p.bits_g;
  r.S = mat ? p.su : p.sg;
  r.B = mat ? p.bu : p.bg;
  r.lg_gs = __builtin_ctz(gs);
  r.ng = p.H >> r.lg_gs;
  r.z = bits == 8 ? 136.0f : 8.0f;
  r.F = bits == 8 ? 128.0f : 8.0f;
  r.act = p.act;
  return r;
}

// Raw scales and biases of the eight g0-groups of slot `slot` of row n
// (indices clamped into the row).
__device__ __forceinline__ void load_slot(const RowSpec& r, int64_t n, int lg_g0, int ngroups, int slot,
                                          uint16_t (&sv)[8], uint16_t (&bv)[8]) {
  if (lg_g0 == r.lg_gs && 8 * slot + 8 <= ngroups) {   // eight whole groups of the row, one load each
    const uint16_t* ps = r.S + n * r.ng + 8 * slot;
    const uint16_t* pb = r.B + n * r.ng + 8 * slot;
    if ((((uintptr_t)ps | (uintptr_t)pb) & 15) == 0) {
      const u32x4 vs = *reinterpret_cast<const u32x4*>(ps), vb = *reinterpret_cast<const u32x4*>(pb);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sv[2 * j] = (uint16_t)(vs[j] & 0xFFFFu);
        sv[2 * j + 1] = (uint16_t)(vs[j] >> 16);
        bv[2 * j] = (uint16_t)(vb[j] & 0xFFFFu);
        bv[2 * j + 1] = (uint16_t)(vb[j] >> 16);
      }
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int G = min(8 * slot + j, ngroups - 1);
    const int64_t gi = n * r.ng + ((G << lg_g0) >> r.lg_gs);
    sv[j] = r.S[gi];
    bv[j] = r.B[gi];
  }
}

__device__ __forceinline__ float slot_max(const RowSpec& r, int ngroups, int slot, const uint16_t (&sv)[8],
                                          const uint16_t (&bv)[8]) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (8 * slot + j < ngroups)
      m = fmaxf(m, group_term_max(act_to_f32(sv[j], r.act), act_to_f32(bv[j], r.act), r.z, r.F));
  return m;
}

// The scale-tile word of g0-group j of a slot: (s 2^-k, s 2^-k) in binary16,
// or with binary16 scales split_scale(s 2^-k).
__device__ __forceinline__ uint32_t scale_word(const RowSpec& r, int k, uint16_t sv) {
  const float sk = ldexpf(act_to_f32(sv, r.act), -k);
  const _Float16 hs = (_Float16)sk;
  return r.act == kActF16 ? as_u32(split_scale(sk)) : as_u32((f16x2){hs, hs});
}

// The slot's extra-column entries (see above).
__device__ __forceinline__ void store_ext(const PrepParams& p, const RowSpec& r, int mat, int64_t n, int ngroups,
                                          int slot, int k, const uint16_t (&sv)[8], const uint16_t (&bv)[8]) {
  f16x8 h[3];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    _Float16 chi = (_Float16)0.0f, clo = (_Float16)0.0f;
    if (8 * slot + j < ngroups) {
      const float cv = ldexpf(fmaf(r.z, act_to_f32(sv[j], r.act), act_to_f32(bv[j], r.act)), -k);
      chi = (_Float16)cv;
      clo = (_Float16)(cv - (float)chi);
    }
    h[(3 * j) >> 3][(3 * j) & 7] = chi;
    h[(3 * j + 1) >> 3][(3 * j + 1) & 7] = clo;
    h[(3 * j + 2) >> 3][(3 * j + 2) & 7] = chi;
  }
  unsigned char* row = reinterpret_cast<unsigned char*>((mat ? p.bext_u : p.bext_g) + n * p.kext);
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const int off = 48 * slot + 16 * q;
    if (off < p.kext * 2) *reinterpret_cast<f16x8*>(row + off) = h[q];
  }
}

// The slot's scale-tile words, one store per K-step (K-steps (8 slot + j)
// g0/32 + u, u < g0/32, take group sv[j]); rows whose block cannot gather
// its words in LDS (see prep_weight_rows).
__device__ __forceinline__ void store_slot_words(const PrepParams& p, const RowSpec& r, int mat, int64_t n,
                                                 int lg_g0, int slot, int k, const uint16_t (&sv)[8]) {
  const int s_main = p.H >> 5, per = 1 << (lg_g0 - 5);
  uint32_t* tile = p.scl + (n >> 7) * (int64_t)p.nss * kScaleTileWords + mat * kScaleTileCols + (n & 127);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t word = scale_word(r, k, sv[j]);
    const int t0 = (8 * slot + j) * per;
    for (int u = 0; u < per; ++u) {
      const int t = t0 + u;
      if (t < s_main) tile[(int64_t)(t >> 2) * kScaleTileWords + (t & 3) * 2 * kScaleTileCols] = word;
    }
  }
}

// Threads per weight row: the slots (padding included) rounded up to a
// power of two, at most a wavefront.  Host and device agree on it.
__host__ __device__ inline int prep_row_lg(int kext) {
  const int per_row = (kext + 23) / 24;
  int lg = 0;
  while ((1 << lg) < per_row && lg < 6) ++lg;
  return lg;
}

// Scale-tile words gathered per block: with one slot per thread (2^lg >=
// the slots of a row) and 2^lg <= 32, the block's 256 >> lg rows are
// C = 128 >> lg consecutive output features of both matrices, and its words
// (2 H/g0 C, at most kPrepWordsLds) meet in LDS as [matrix][g0-group][C];
// after a barrier the block stores them per K-step as 16-byte pieces of four
// features, C * 4 contiguous bytes per (K-step, matrix).
constexpr int kPrepWordsLds = 2048;

__device__ __forceinline__ void prep_weight_rows(const PrepParams& p, int64_t idx) {
  const int lg = prep_row_lg(p.kext);
  const int c = (int)(idx & ((1 << lg) - 1));
  const int64_t pair = idx >> lg;
  const int64_t n = pair >> 1;
  const int mat = (int)(pair & 1);
  const RowSpec r = row_spec(p, mat);
  const int lg_g0 = __builtin_ctz(p.g0);
  const int ngroups = p.H >> lg_g0;
  const int per_row = (p.kext + 23) / 24;
  const int step = 1 << lg;
  const int C = 128 >> lg;
  const bool gather = !p.k_only && per_row <= step && lg <= 5 && 2 * ngroups * C <= kPrepWordsLds;
  if (!gather && n >= p.I) return;                      // whole rows: the lanes of a row leave together
  const bool live = n < p.I && n < (mat ? p.I_u : p.I); // up rows past I_u: none (k = 0)
  float vmax = 0.0f;
  int k;
  if (per_row <= step) {                                // one slot per thread: keep it in registers
    uint16_t sv[8], bv[8];
    const bool mine = live && c < per_row;
    if (mine) {
      load_slot(r, n, lg_g0, ngroups, c, sv, bv);
      vmax = slot_max(r, ngroups, c, sv, bv);
    }
    for (int off = 1; off < step; off <<= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off));
    k = row_exponent_k(vmax);
    if (mine && !p.k_only) {
      store_ext(p, r, mat, n, ngroups, c, k, sv, bv);
      if (!gather) store_slot_words(p, r, mat, n, lg_g0, c, k, sv);
    }
    if (gather) {
      __shared__ __align__(16) uint32_t words[kPrepWordsLds];
      const int64_t nb0 = (idx - threadIdx.x) >> (lg + 1);   // the block's first feature (a multiple of C)
      const int cl = (int)(n - nb0);
#ifdef SWQ_LDS_POISON
      lds_poison(words, sizeof(words), kPoisonFloat);
      __syncthreads();
#endif
      if (c < per_row) {                                 // zeros for rows past I (or I_u)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (8 * c + j < ngroups) words[(mat * ngroups + 8 * c + j) * C + cl] = mine ? scale_word(r, k, sv[j]) : 0u;
      }
      __syncthreads();
      const int s_main = p.H >> 5, per = 1 << (lg_g0 - 5);
      const int lq = 5 - lg;                             // log2 of the 16-byte pieces per row of C words
      for (int i = threadIdx.x; i < (2 * ngroups) << lq; i += blockDim.x) {
        const int q = i & ((1 << lq) - 1), mg = i >> lq;  // piece, (matrix, g0-group)
        const int m = mg >= ngroups ? 1 : 0, G = mg - m * ngroups;
        const int64_t n4 = nb0 + 4 * q;
        if (n4 >= p.I) continue;                         // (pieces past I lie in the last tile of 128)
        const u32x4 v = *reinterpret_cast<const u32x4*>(&words[mg * C + 4 * q]);
        uint32_t* tile = p.scl + (n4 >> 7) * (int64_t)p.nss * kScaleTileWords + m * kScaleTileCols + (n4 & 127);
        for (int u = 0; u < per; ++u) {
          const int t = G * per + u;
          if (t < s_main) *reinterpret_cast<u32x4*>(tile + (int64_t)(t >> 2) * kScaleTileWords + (t & 3) * 2 * kScaleTileCols) = v;
        }
      }
    }
  } else {
    for (int slot = c; live && slot < per_row; slot += step) {
      uint16_t sv[8], bv[8];
      load_slot(r, n, lg_g0, ngroups, slot, sv, bv);
      vmax = fmaxf(vmax, slot_max(r, ngroups, slot, sv, bv));
    }
    for (int off = 1; off < step; off <<= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off));
    k = row_exponent_k(vmax);
    for (int slot = c; live && !p.k_only && slot < per_row; slot += step) {
      uint16_t sv[8], bv[8];
      load_slot(r, n, lg_g0, ngroups, slot, sv, bv);
      store_ext(p, r, mat, n, ngroups, slot, k, sv, bv);
      store_slot_words(p, r, mat, n, lg_g0, slot, k, sv);
    }
  }
  if (c == 0 && n < p.I) p.kexp[(int64_t)mat * p.I + n] = k;
}

// Blocks [0, M): x rows.  Then the weight rows, 2^lg threads each (whole
// rows per wave: 256 is a multiple of 2^lg).
__global__ __launch_bounds__(256) void swq_prep_kernel(PrepParams p) {
  if ((int)blockIdx.x < p.M) {
    prep_x_row(p, blockIdx.x);
    return;
  }
  prep_weight_rows(p, ((int64_t)blockIdx.x - p.M) * 256 + threadIdx.x);
}

__host__ __device__ inline int64_t prep_row_blocks(int I, int kext) {
  return ((2 * (int64_t)I << prep_row_lg(kext)) + 255) / 256;
}

// ----------------------------------------------------------- MFMA GEMM ----
//
// Work split.  A block of four wavefronts (one per SIMD) computes a BM x 128
// tile of both projections.  Wave w owns all BM rows and columns
// [32w, 32w + 32) of the gate AND the up tile: BM/32 MFMA 32x32x16
// fragments per matrix.  Each column's codes are dequantized by exactly one
// wave; every A fragment read from LDS feeds the gate and the up MFMA.
//
// Staging.  A ring of four LDS stages, each holding one K-step of 32: the x'
// tile (BM rows x 64 bytes) and the B side (packed codes of both matrices, or
// for the extra-column steps their binary16 rows).  Global data goes
// straight to LDS with buffer loads that write LDS (no VGPR round trip),
// issued three K-steps ahead; one barrier per K-step.  Rows of 64 bytes are
// stored as four 16-byte chunks permuted by (row >> 2) & 3, so the MFMA
// operand reads (32 rows, one chunk) spread over all banks.
//
// Software pipeline per K-step t (two k16 sub-steps): while the MFMAs of one
// sub-step run, the A fragments of the next are read from LDS and its codes
// dequantized in registers (lane l: column l % 32, 8-code blocks
// 2 (l / 32) + ks, the MFMA's own K order).
//
// Tile order: blocks are dealt round-robin to the 8 XCDs; the kernel remaps
// them so that each XCD runs a contiguous range of logical tiles, grouped four
// (or eight) row tiles at a time, so the tiles running together on one XCD
// share x' rows and weight rows in its L2.

// Barrier without the memory fence of __syncthreads (which would wait for the
// loads in flight for later stages); the asm statements keep the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Dequantized B operands of one k16 sub-step (one 8-code block per lane) of one matrix.
template <int BITS, bool A16>
__device__ __forceinline__ void dequant_block(const uint32_t* w, f16x2 s2, f16x8& b0, f16x8& b1, f16x8& b2,
                                              const NibbleK& k) {
  if (kCodeWidth<BITS> == 4) {
    if constexpr (A16) {   // s2 = (hi, lo): planes hi (q - 8) and lo (q - 8)
      const f16x2 shi = {s2[0], s2[0]}, slo = {s2[1], s2[1]};
      const f16x2 c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
      const f16x2 c72 = {(_Float16)72.0f, (_Float16)72.0f};
      const uint32_t w8 = w[0] >> 8;
      const f16x2 q[4] = {as_h2((w[0] & k.m_lo) | k.g_lo) - c1032, as_h2((w[0] & k.m_hi) | k.g_hi) - c72,
                          as_h2((w8 & k.m_lo) | k.g_lo) - c1032, as_h2((w8 & k.m_hi) | k.g_hi) - c72};
      u32x4 vh, vl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vh[j] = as_u32(q[j] * shi);
        vl[j] = as_u32(q[j] * slo);
      }
      b0 = __builtin_bit_cast(f16x8, vh);
      b1 = __builtin_bit_cast(f16x8, vl);
    } else {
      uint32_t o[4];
      dequant4(w[0], s2, o, k);
      b0 = __builtin_bit_cast(f16x8, (u32x4){o[0], o[1], o[2], o[3]});
    }
  } else {
    // planes s (lo - 8) and 16 s (hi - 8); A16: with s = hi part, and a third
    // plane lo part times the whole code q - 136
    uint32_t lo[4], hi[4], full[4];
    codes8(w[0], w[1], lo, hi, k, A16 ? full : nullptr);
    const f16x2 sh = A16 ? (f16x2){s2[0], s2[0]} : s2;
    const f16x2 s16 = sh * (f16x2){(_Float16)16.0f, (_Float16)16.0f};
    u32x4 vl, vh;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vl[j] = as_u32(as_h2(lo[j]) * sh);
      vh[j] = as_u32(as_h2(hi[j]) * s16);
    }
    b0 = __builtin_bit_cast(f16x8, vl);
    b1 = __builtin_bit_cast(f16x8, vh);
    if constexpr (A16) {
      const f16x2 slo = {s2[1], s2[1]};
      u32x4 vf;
#pragma unroll
      for (int j = 0; j < 4; ++j) vf[j] = as_u32(as_h2(full[j]) * slo);
      b2 = __builtin_bit_cast(f16x8, vf);
    }
  }
}

// MFMA planes per matrix: 8-bit codes two (nibbles), binary16 scales one more.
template <int BITS, bool A16>
inline constexpr int kPlanes = (kCodeWidth<BITS> == 8 ? 2 : 1) + (A16 ? 1 : 0);

template <int BITS_G, int BITS_U, int BM, int WN, int OCC, bool A16, bool KSPLIT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void swq_mfma_kernel(MfmaParams p) {
  constexpr int NT = 256;
  constexpr int STAGES = 4;                            // x' / extra-column ring: K-steps in flight
  constexpr int SS = 4;                                // K-steps per code super-step (the code ring's unit)
  constexpr int BN = 4 * WN;                           // columns per matrix of the block tile
  constexpr int MF = BM / 32, NF = WN / 32;            // A and B fragments per wave
  constexpr int A_BYTES = BM * 64;                     // x' rows of one K-step
  constexpr int EXT_BYTES = BN * 64;                   // extra-column rows of one matrix, one K-step
  constexpr int STAGE = A_BYTES + EXT_BYTES;
  // code super-step: SS K-steps of codes per row = BITS 16-byte chunks per row and matrix,
  // then the scales of its groups (4 slots per row and matrix, a dword each)
  constexpr int CPR_G = BITS_G, CPR_U = BITS_U;
  constexpr int SSG_BYTES = BN * CPR_G * 16, SSU_BYTES = BN * CPR_U * 16;
  constexpr int SS_CODE_BYTES = SSG_BYTES + SSU_BYTES;
  constexpr int SS_SLOT = SS_CODE_BYTES + 2 * BN * 16;
  constexpr int A_INSTR = BM * 4 / NT;
  constexpr int B_EXT_INSTR = EXT_BYTES / 16 / NT;
  constexpr int SS_CODE_INSTR = SS_CODE_BYTES / 16 / NT;
  constexpr int SS_SCALE_INSTR = kScaleTileWords * 4 / 16 / NT;   // one 4 KB scale tile
  constexpr int N_SS = SS_CODE_INSTR + SS_SCALE_INSTR;  // buffer loads a thread issues per super-step
  constexpr int N_MAIN = A_INSTR;                       // ... per code K-step
  constexpr int N_EXT = A_INSTR + B_EXT_INSTR;          // ... per extra-column K-step
  constexpr int GM = 4;                                // row tiles per group of the tile order
  static_assert(SSG_BYTES % (16 * NT) == 0 && SSU_BYTES % (16 * NT) == 0 && (BN * 4) % NT == 0,
                "each code or scale DMA instruction reads one matrix");
  static_assert(BM <= NT && A_INSTR >= 1 && B_EXT_INSTR >= 1 && SS_SCALE_INSTR == 1, "tile shape");
  static_assert(BN == kScaleTileCols && kScaleTileWords * 4 == 2 * BN * 16, "scale tile = ring slot scale area");
  static_assert(STAGES == SS, "a stage slot and the super-step phase are both t % 4");
  static_assert(STAGES * STAGE + 2 * SS_SLOT + BM * 4 + 2 * BN * 4 <= 160 * 1024, "LDS");
  static_assert(2 * BN == NT, "one thread per (matrix, column) of the tile for the row exponents k");

  __shared__ __attribute__((aligned(16))) unsigned char smem[STAGES * STAGE + 2 * SS_SLOT];
  __shared__ int rexp[BM];
  __shared__ int rk[2][BN];
#ifdef SWQ_LDS_POISON
  lds_poison(smem, sizeof(smem), kPoisonFloat);
  lds_poison(rexp, sizeof(rexp), kPoisonExp);
  lds_poison(rk, sizeof(rk), kPoisonExp);
  __syncthreads();
#endif
  unsigned char* const ssmem = smem + STAGES * STAGE;   // code ring: two super-step slots

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform (scalar)
  const int half = lane >> 5, l32 = lane & 31;

  // ---- tile of this block
  const int T = gridDim.x;
  const int q8 = T / 8, r8 = T % 8;
  const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const int logical = xcd < r8 ? xcd * (q8 + 1) + local : r8 * (q8 + 1) + (xcd - r8) * q8 + local;
  const int mtiles = (p.M + BM - 1) / BM, ntiles = (p.n_end - p.n_begin + BN - 1) / BN;
  const int per_group = GM * ntiles;
  const int grp = logical / per_group;
  const int first_m = grp * GM;
  const int gsz = min(mtiles - first_m, GM);
  const int in_grp = logical - grp * per_group;
  const int m0 = (first_m + in_grp % gsz) * BM;
  const int n0 = p.n_begin + (in_grp / gsz) * BN;
  const int rows = min(BM, p.M - m0);
  const int cols = min(BN, p.n_end - n0);
  const int cols_u = max(0, min(cols, p.I_u - n0));   // up rows of the tile (fewer for a split linear weight)

  const int s_main = p.H / 32;
  const int s_ext = p.kext / 32;
  const int s_total = s_main + 2 * s_ext;              // extra-column steps: gate then up, per 32 columns
  // K split (KSPLIT; grid y = the splits): this block runs the code K-steps
  // [kb0, kb1) (p.kchunk per split, whole super-steps) and, in the last
  // split, the extra columns; its float32 sums go to its own slice of the
  // partial buffers (dbg_g, dbg_u), which swq_ksplit_epilogue adds in split
  // order and finishes
  const int kb0 = KSPLIT ? (int)blockIdx.y * p.kchunk : 0;
  const int kb1 = KSPLIT ? min(s_main, kb0 + p.kchunk) : s_main;
  const bool klast = !KSPLIT || kb1 == s_main;
  const int rw_g = p.H * BITS_G / 32, rw_u = p.H * BITS_U / 32;

  // x' tile rows of K-step s: (s * M + m0 + row) * 64 bytes from the start of x'
  const i32x4 rs_a = make_srsrc(p.xa + (int64_t)m0 * 32, (uint32_t)(((int64_t)(p.ldx / 32) * p.M - m0) * 64));
  const uint32_t a_step = (uint32_t)p.M * 64;
  const i32x4 rs_wg = make_srsrc(p.wg + (int64_t)n0 * rw_g, (uint32_t)cols * rw_g * 4);
  const i32x4 rs_wu = make_srsrc(p.wu + (int64_t)n0 * rw_u, (uint32_t)cols_u * rw_u * 4);
  const i32x4 rs_sc = make_srsrc(p.scl + (int64_t)(n0 / BN) * p.nss * kScaleTileWords,
                                 (uint32_t)p.nss * kScaleTileWords * 4);
  const i32x4 rs_eg = make_srsrc(p.bext_g + (int64_t)n0 * p.kext, (uint32_t)cols * p.kext * 2);
  const i32x4 rs_eu = make_srsrc(p.bext_u + (int64_t)n0 * p.kext, (uint32_t)cols_u * p.kext * 2);

  // ---- per-thread DMA offsets (bytes)
  // A: LDS piece L = j*NT + tid holds row L/4, chunk (L%4) ^ ((row>>2)&3)
  uint32_t a_voff[A_INSTR];
#pragma unroll
  for (int j = 0; j < A_INSTR; ++j) {
    const int L = j * NT + tid, row = L >> 2, c = (L & 3) ^ ((row >> 2) & 3);
    a_voff[j] = (uint32_t)(row * 64 + c * 16);
  }
  // super-step codes: LDS piece L < BN*CPR_G is gate row r = L / CPR_G, chunk
  // (L % CPR_G) ^ swz(r), then the up rows; the permutation spreads a K-step's
  // reads over the banks
  auto swz = [](int r, int cpr) { return (r * cpr / 16) % cpr; };
  uint32_t c_voff[SS_CODE_INSTR];
#pragma unroll
  for (int j = 0; j < SS_CODE_INSTR; ++j) {
    const int L = j * NT + tid;
    if (j * NT < BN * CPR_G) {
      const int r = L / CPR_G, c = (L % CPR_G) ^ swz(r, CPR_G);
      c_voff[j] = (uint32_t)(r * rw_g * 4 + c * 16);
    } else {
      const int L2 = L - BN * CPR_G, r = L2 / CPR_U, c = (L2 % CPR_U) ^ swz(r, CPR_U);
      c_voff[j] = (uint32_t)(r * rw_u * 4 + c * 16);
    }
  }
  // extra columns of one matrix: piece L = row*4 + phys, chunk phys ^ ((row>>2)&3)
  uint32_t e_voff[B_EXT_INSTR];
#pragma unroll
  for (int j = 0; j < B_EXT_INSTR; ++j) {
    const int L = j * NT + tid, row = L >> 2, c = (L & 3) ^ ((row >> 2) & 3);
    e_voff[j] = (uint32_t)(row * p.kext * 2 + c * 16);
  }
  // super-step scales: the tile's 4 KB block, 16 bytes per thread in order
  const uint32_t s_voff[SS_SCALE_INSTR] = {(uint32_t)tid * 16};

  const NibbleK nk = nibble_consts_in_regs();            // unpack constants in registers

  // row exponents of the tile (x rows e, weight rows k: thread = (matrix, column)):
  // loaded first, published through LDS after the K loop
  const int my_exp = tid < rows ? p.xexp[m0 + tid] : 0;
  const int kc = tid & (BN - 1), km = tid >> 7;
  const int my_k = n0 + kc < (km ? min(p.n_end, p.I_u) : p.n_end) ? p.kexp[(int64_t)km * p.I + n0 + kc] : 0;

  // issue the x' (and for an extra-column step the B) loads of K-step s into stage `slot`
  const uint32_t smem0 = lds_addr(smem);
  auto issue = [&](int slot, int s, bool ext) {
    const uint32_t st = smem0 + slot * STAGE;
    const int es = s - s_main;                         // extra-column step: block es/2, matrix es%2
    const uint32_t soff_a = (uint32_t)(ext ? s_main + (es >> 1) : s) * a_step;
#pragma unroll
    for (int j = 0; j < A_INSTR; ++j) dma16(rs_a, st + (j * NT + w * 64) * 16, a_voff[j] + soff_a);
    if (ext) {
      const uint32_t sb = st + A_BYTES;
      const i32x4 rs_e = (es & 1) ? rs_eu : rs_eg;
      const uint32_t soff_e = (uint32_t)(es >> 1) * 64;
#pragma unroll
      for (int j = 0; j < B_EXT_INSTR; ++j) dma16(rs_e, sb + (j * NT + w * 64) * 16, e_voff[j] + soff_e);
    }
  };
  // issue the codes and scales of super-step j (K-steps SS*j .. SS*j + SS-1) into its slot
  const uint32_t ssmem0 = lds_addr(ssmem);
  auto issue_ss = [&](int j) {
    const uint32_t sl = ssmem0 + (j & 1) * SS_SLOT;
#pragma unroll
    for (int q = 0; q < SS_CODE_INSTR; ++q) {
      if (q * NT < BN * CPR_G) dma16(rs_wg, sl + (q * NT + w * 64) * 16, c_voff[q] + (uint32_t)(j * CPR_G * 16));
      else dma16(rs_wu, sl + (q * NT + w * 64) * 16, c_voff[q] + (uint32_t)(j * CPR_U * 16));
    }
#pragma unroll
    for (int q = 0; q < SS_SCALE_INSTR; ++q)
      dma16(rs_sc, sl + SS_CODE_BYTES + w * 64 * 16, s_voff[q] + (uint32_t)j * kScaleTileWords * 4);
  };

  f32x16 acc_g[MF][NF], acc_u[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc_g[i][f][r] = 0.0f;
        acc_u[i][f][r] = 0.0f;
      }

  // operand registers of the two sub-steps of a K-step
  f16x8 a0[MF], a1[MF];
  f16x8 g0a[NF], g0b[NF], g0c[NF], u0a[NF], u0b[NF], u0c[NF];   // sub-step 0: gate planes, up planes
  f16x8 g1a[NF], g1b[NF], g1c[NF], u1a[NF], u1b[NF], u1c[NF];   // sub-step 1
  constexpr int PL_G = kPlanes<BITS_G, A16>, PL_U = kPlanes<BITS_U, A16>;
  // this lane's codes and scales of two consecutive code K-steps: step t
  // uses set P and loads step t+1 into set P^1 (in the unrolled main loop P
  // alternates; elsewhere P = 0 and set 1 is copied back after the step)
  constexpr int WG = kCodeWidth<BITS_G>, WU = kCodeWidth<BITS_U>;   // 2-bit codes held as nibbles
  uint32_t cw_g[2][NF][WG / 2], cw_u[2][NF][WU / 2];
  f16x2 s_g2[2][NF], s_u2[2][NF];

  const uint32_t sw = (uint32_t)((l32 >> 2) & 3);
  const uint32_t a_lds0 = (uint32_t)(l32 * 64) + (((2 * half) ^ sw) * 16);
  const uint32_t a_lds1 = (uint32_t)(l32 * 64) + (((2 * half + 1) ^ sw) * 16);

  // A fragments of sub-step ks from stage `slot`
  auto read_a = [&](int slot, int ks, f16x8 (&a)[MF]) {
    const unsigned char* st = smem + slot * STAGE + (ks ? a_lds1 : a_lds0);
#pragma unroll
    for (int i = 0; i < MF; ++i) a[i] = *reinterpret_cast<const f16x8*>(st + i * 32 * 64);
  };
  // this lane's codes and scales of code K-step t, from the code ring
  auto load_codes = [&](int t, uint32_t (&cg)[NF][WG / 2], uint32_t (&cu)[NF][WU / 2], f16x2 (&s_g)[NF],
                        f16x2 (&s_u)[NF]) {
    const unsigned char* ring = ssmem + ((t / SS) & 1) * SS_SLOT;
    const int q = t % SS;                              // K-step within the super-step
    const uint32_t* sc = reinterpret_cast<const uint32_t*>(ring + SS_CODE_BYTES);

#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int n = w * WN + f * 32 + l32;
      s_g[f] = as_h2(sc[(2 * q) * BN + n]);
      s_u[f] = as_h2(sc[(2 * q + 1) * BN + n]);
      // 4-bit: chunk q holds the K-step, this lane's two 8-code blocks at half * 8;
      // 8-bit: chunks 2q, 2q+1 hold it, this lane's blocks are chunk 2q + half;
      // 2-bit: chunk q/2 holds it at 8 (q % 2), this lane's blocks at half * 4
      auto code_at = [&](int bits, int cpr, int base) {
        return bits == 4 ? ring + base + n * (cpr * 16) + ((q ^ swz(n, cpr)) * 16) + half * 8
             : bits == 8 ? ring + base + n * (cpr * 16) + (((2 * q + half) ^ swz(n, cpr)) * 16)
                         : ring + base + n * (cpr * 16) + (((q >> 1) ^ swz(n, cpr)) * 16) + 8 * (q & 1) + half * 4;
      };
      const unsigned char* qg = code_at(BITS_G, CPR_G, 0);
      const unsigned char* qu = code_at(BITS_U, CPR_U, SSG_BYTES);
      if constexpr (BITS_G == 2) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(qg);
        cg[f][0] = spread2(v); cg[f][1] = spread2(v >> 16);
      } else if constexpr (BITS_G == 4) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(qg);
        cg[f][0] = v[0]; cg[f][1] = v[1];
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(qg);
        cg[f][0] = v[0]; cg[f][1] = v[1]; cg[f][2] = v[2]; cg[f][3] = v[3];
      }
      if constexpr (BITS_U == 2) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(qu);
        cu[f][0] = spread2(v); cu[f][1] = spread2(v >> 16);
      } else if constexpr (BITS_U == 4) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(qu);
        cu[f][0] = v[0]; cu[f][1] = v[1];
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(qu);
        cu[f][0] = v[0]; cu[f][1] = v[1]; cu[f][2] = v[2]; cu[f][3] = v[3];
      }
    }
  };
  // B operands of sub-step ks from codes and scales in registers
  auto dequant = [&](int ks, const uint32_t (&cg)[NF][WG / 2], const uint32_t (&cu)[NF][WU / 2],
                     const f16x2 (&s_g)[NF], const f16x2 (&s_u)[NF], f16x8 (&ga)[NF], f16x8 (&gb)[NF],
                     f16x8 (&gc)[NF], f16x8 (&ua)[NF], f16x8 (&ub)[NF], f16x8 (&uc)[NF]) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      dequant_block<BITS_G, A16>(&cg[f][ks * (WG / 4)], s_g[f], ga[f], gb[f], gc[f], nk);
      dequant_block<BITS_U, A16>(&cu[f][ks * (WU / 4)], s_u[f], ua[f], ub[f], uc[f], nk);
    }
  };
  // B operands of sub-step ks of an extra-column step from stage `slot` (one
  // matrix per step; its operands go to the gate slots)
  auto read_ext = [&](int slot, int ks, f16x8 (&ga)[NF]) {
    const unsigned char* sb = smem + slot * STAGE + A_BYTES;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int n = w * WN + f * 32 + l32;
      ga[f] = *reinterpret_cast<const f16x8*>(sb + n * 64 + (((2 * half + ks) ^ sw) * 16));
    }
  };
  // kind 0: code step (both matrices); 1: extra columns of the gate; 2: of the up matrix
  auto mfma = [&](int kind, const f16x8 (&a)[MF], const f16x8 (&ga)[NF], const f16x8 (&gb)[NF],
                  const f16x8 (&gc)[NF], const f16x8 (&ua)[NF], const f16x8 (&ub)[NF], const f16x8 (&uc)[NF]) {
    if (kind == 0) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int i = 0; i < MF; ++i) {
          acc_g[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ga[f], a[i], acc_g[i][f], 0, 0, 0);
          acc_u[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ua[f], a[i], acc_u[i][f], 0, 0, 0);
          if (PL_G >= 2) acc_g[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(gb[f], a[i], acc_g[i][f], 0, 0, 0);
          if (PL_U >= 2) acc_u[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ub[f], a[i], acc_u[i][f], 0, 0, 0);
          if (PL_G >= 3) acc_g[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(gc[f], a[i], acc_g[i][f], 0, 0, 0);
          if (PL_U >= 3) acc_u[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(uc[f], a[i], acc_u[i][f], 0, 0, 0);
        }
    } else if (kind == 1) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int i = 0; i < MF; ++i)
          acc_g[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ga[f], a[i], acc_g[i][f], 0, 0, 0);
    } else {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int i = 0; i < MF; ++i)
          acc_u[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ga[f], a[i], acc_u[i][f], 0, 0, 0);
    }
  };

  // Order of one sub-step's instructions: the MFMAs interleaved with the LDS
  // reads and the dequantization that prepare the next sub-step, so that the
  // matrix pipe stays fed while the vector ALU works (the reads go with the
  // first MFMAs, their results are needed by the dequantization).
  constexpr int MF_MAIN = MF * NF * (PL_G + PL_U);   // MFMAs of a code sub-step
  constexpr int DQ_VALU = NF * (BITS_G == 8 ? 40 : 20) * (A16 ? 3 : 2) / 2 + NF * (BITS_U == 8 ? 40 : 20) * (A16 ? 3 : 2) / 2;
  auto interleave = [&]<int NMFMA, int NDS, int NVALU>() {
    constexpr int LEAD = NMFMA < 8 ? NMFMA / 2 : 4;
    constexpr int DS_PER = (NDS + LEAD - 1) / LEAD;
    constexpr int V_PER = (NVALU + (NMFMA - LEAD) - 1) / (NMFMA - LEAD);
#pragma unroll
    for (int i = 0; i < LEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, DS_PER, 0);   // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
    }
#pragma unroll
    for (int i = LEAD; i < NMFMA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, V_PER, 0);    // VALU
    }
  };

  // Loads of K-step s are issued STAGES - 1 = 3 steps ahead, after the
  // barrier of step s - 3, and the codes and scales of super-step j at the
  // start of step SS*(j-1) + 1 (before that step's x' loads).  At the barrier
  // of step t everything issued before step t-1's x' loads must have landed:
  // only those (K-step t+2) may still be in flight, and in a step that issued
  // a super-step, the super-step too.  A super-step has therefore landed at the
  // barrier of the step after the one that issued it, a step before its first
  // codes are read (in the first half of step SS*j - 1).

  // one K-step t in stage ph = t % STAGES: sub-step (t, 0) while (t, 1) is
  // prepared from the same stage, then the barrier, then sub-step (t, 1)
  // while (t+1, 0) is prepared.  D = 0: steps t+1 .. t+3 are code steps;
  // D in [1, 3]: D = s_main - t (steps t+D and later are extra-column steps);
  // D = -1 / -2: extra-column step of the gate / the up matrix.  Every kind is
  // a compile-time constant.
  auto step = [&]<int D, int P = 0, bool COPY = true>(int t, int ph) {
    constexpr int KIND = D >= 0 ? 0 : -D;                      // MFMA kind of step t
    constexpr bool NXT_EXT = D < 0 || D == 1;
    constexpr bool W2_EXT = D < 0 || D == 1 || D == 2;         // is step t+2 an extra-column step
    constexpr bool IS_EXT = D != 0;
    constexpr int NA = W2_EXT ? N_EXT : N_MAIN;
    const int nx = (ph + 1) % STAGES, is = (ph + STAGES - 1) % STAGES;
    // codes and scales of the next super-step, apart from the x' loads that follow the barrier
    if (ph == 1) issue_ss(t / SS + 1);
    read_a(ph, 1, a1);
    if constexpr (KIND == 0) dequant(1, cw_g[P], cw_u[P], s_g2[P], s_u2[P], g1a, g1b, g1c, u1a, u1b, u1c);
    else read_ext(ph, 1, g1a);
    // the next code step's codes: its super-step landed before the previous barrier
    if constexpr (!NXT_EXT) load_codes(t + 1, cw_g[P ^ 1], cw_u[P ^ 1], s_g2[P ^ 1], s_u2[P ^ 1]);
    mfma(KIND, a0, g0a, g0b, g0c, u0a, u0b, u0c);
    if (D == 0) interleave.template operator()<MF_MAIN, MF + 4 * NF, DQ_VALU + 4 * NF>();
    // stage t+1 and its super-step complete for every wave, and every wave is done with stage t-1
    // (scheduling fences keep the first half's MFMAs ahead of the wait)
    __builtin_amdgcn_sched_barrier(0);
    if (ph == 1) wait_vmcnt<NA + N_SS>();
    else wait_vmcnt<NA>();
    block_barrier();
    issue(is, t + STAGES - 1, IS_EXT);
    read_a(nx, 0, a0);
    if constexpr (!NXT_EXT) dequant(0, cw_g[P ^ 1], cw_u[P ^ 1], s_g2[P ^ 1], s_u2[P ^ 1], g0a, g0b, g0c, u0a, u0b, u0c);
    else read_ext(nx, 0, g0a);
    mfma(KIND, a1, g1a, g1b, g1c, u1a, u1b, u1c);
    if (D == 0) interleave.template operator()<MF_MAIN, MF, DQ_VALU>();
    __builtin_amdgcn_sched_barrier(0);   // each step is its own scheduling region
    if constexpr (COPY && !NXT_EXT) {
      static_assert(P == 0, "copies go back to set 0");
#pragma unroll
      for (int f = 0; f < NF; ++f) {
#pragma unroll
        for (int j = 0; j < WG / 2; ++j) cw_g[0][f][j] = cw_g[1][f][j];
#pragma unroll
        for (int j = 0; j < WU / 2; ++j) cw_u[0][f][j] = cw_u[1][f][j];
        s_g2[0][f] = s_g2[1][f];
        s_u2[0][f] = s_u2[1][f];
      }
    }
  };

  // ---- prologue: super-step 0 and K-steps 0 .. 2 in flight, step 0 complete, its first operands read
  issue_ss(kb0 / SS);
  issue(0, kb0, kb0 >= s_main);
  issue(1, kb0 + 1, kb0 + 1 >= s_main);
  issue(2, kb0 + 2, kb0 + 2 >= s_main);
  if (kb0 + 2 < s_main) {
    wait_vmcnt<2 * N_MAIN>();
  } else if (kb0 + 1 < s_main) {
    wait_vmcnt<N_MAIN + N_EXT>();
  } else {
    wait_vmcnt<2 * N_EXT>();
  }
  block_barrier();
  read_a(0, 0, a0);
  if (kb0 < s_main) {
    load_codes(kb0, cw_g[0], cw_u[0], s_g2[0], s_u2[0]);
    dequant(0, cw_g[0], cw_u[0], s_g2[0], s_u2[0], g0a, g0b, g0c, u0a, u0b, u0c);
  } else {
    read_ext(0, 0, g0a);
  }

  // ---- K loop: code steps, the last three code steps, extra-column steps in gate/up pairs
  const int t_code = max(kb0, kb1 - 3);
  int t = kb0;
  for (; t + STAGES <= t_code; t += STAGES) {
    step.template operator()<0, 0, false>(t, 0);
    step.template operator()<0, 1, false>(t + 1, 1);
    step.template operator()<0, 0, false>(t + 2, 2);
    step.template operator()<0, 1, false>(t + 3, 3);
  }
  for (; t < t_code; ++t) step.template operator()<0>(t, t % STAGES);
  if (kb1 - kb0 >= 3) step.template operator()<3>(kb1 - 3, (kb1 - 3) % STAGES);
  if (kb1 - kb0 >= 2) step.template operator()<2>(kb1 - 2, (kb1 - 2) % STAGES);
  step.template operator()<1>(kb1 - 1, (kb1 - 1) % STAGES);
  if (klast) {
    for (t = s_main; t < s_total; t += 2) {
      step.template operator()<-1>(t, t % STAGES);
      step.template operator()<-2>(t + 1, (t + 1) % STAGES);
    }
  }
  wait_vmcnt<0>();                                   // nothing left in flight at exit
  if (tid < BM) rexp[tid] = my_exp;
  rk[km][kc] = my_k;
  __syncthreads();

  // ---- epilogue.  The MFMAs compute W x'^T, so in fragment (i, f) lane l holds
  // token row i*32 + l32 and, in accumulator entry 4j + c, feature
  // w*WN + 32f + 8j + 4*half + c: four consecutive features per j, written
  // with one vector store when the output allows it (p.vec).
  // four consecutive outputs at element offset o of a float32 or bf16 array,
  // columns c0 .. c0 + 3 stored while below lim
  constexpr int ACT = A16 ? kActF16 : kActBf16;   // 16-bit output type
  auto put4 = [&](auto* base, int64_t o, int c0, int lim, const float (&v)[4]) {
    constexpr bool F32 = std::is_same_v<std::remove_pointer_t<decltype(base)>, float>;
    if (p.vec && c0 + 4 <= lim) {
      if constexpr (F32) {
        *reinterpret_cast<f32x4*>(base + o) = (f32x4){v[0], v[1], v[2], v[3]};
      } else {
        const uint32_t lo = (uint32_t)f32_to_act(v[0], ACT) | ((uint32_t)f32_to_act(v[1], ACT) << 16);
        const uint32_t hi = (uint32_t)f32_to_act(v[2], ACT) | ((uint32_t)f32_to_act(v[3], ACT) << 16);
        *reinterpret_cast<u32x2*>(base + o) = (u32x2){lo, hi};
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c0 + c >= lim) continue;
        if constexpr (F32) base[o + c] = v[c];
        else base[o + c] = f32_to_act(v[c], ACT);
      }
    }
  };
  // MODE 0..2: precision mode; 3: debug gate/up; kLinBf16, kLinF32: the linear
  auto epilogue = [&]<int MODE>() {
    constexpr bool LIN = MODE == kLinBf16 || MODE == kLinF32;
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int lr = i * 32 + l32;
      const int e = rexp[lr];
      const bool row_ok = lr < rows;
      const int64_t orow = (int64_t)(m0 + lr) * p.ldo;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int cl = w * WN + f * 32 + 8 * j + 4 * half;
          const int c0 = n0 + cl;
          float g[4], u[4], h[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            g[c] = ldexpf(acc_g[i][f][4 * j + c], e + rk[0][cl + c]);
            u[c] = ldexpf(acc_u[i][f][4 * j + c], e + rk[1][cl + c]);
            if constexpr (MODE < 3) h[c] = swiglu_epilogue(g[c], u[c], MODE, ACT);
          }
          if (!row_ok) continue;
          const int64_t o = orow + c0;
          if constexpr (MODE == 3) {
            const int64_t ko = KSPLIT ? (int64_t)blockIdx.y * p.M * p.ldo : 0;   // this split's slice
            put4(p.dbg_g + ko, o, c0, p.n_end, g);
            put4(p.dbg_u + ko, o, c0, p.n_end, u);
          } else if constexpr (LIN) {
            if (p.res) {   // the residual of a whole MLP, added in float32 before the one rounding
              const int lg_ = p.n_end - c0, lu_ = min(p.n_end, p.I_u) - c0;
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                if (c < lg_) g[c] += bf16_to_f32(p.res[o + c]);
                if (c < lu_) u[c] += bf16_to_f32(p.res[o + p.I + c]);
              }
            }
            auto* y = reinterpret_cast<std::conditional_t<MODE == kLinF32, float, uint16_t>*>(p.out);
            put4(y, o, c0, p.n_end, g);
            put4(y, o + p.I, c0, min(p.n_end, p.I_u), u);
          } else if constexpr (MODE == kF32) {
            put4(reinterpret_cast<float*>(p.out), o, c0, p.n_end, h);
          } else {
            put4(reinterpret_cast<uint16_t*>(p.out), o, c0, p.n_end, h);
          }
        }
      }
    }
  };
  if (p.dbg_g) epilogue.template operator()<3>();
  else if (p.mode == kMatch) epilogue.template operator()<kMatch>();
  else if (p.mode == kF32) epilogue.template operator()<kF32>();
  else if (p.mode == kF32Bf16Out) epilogue.template operator()<kF32Bf16Out>();
  else if (p.mode == kLinBf16) epilogue.template operator()<kLinBf16>();
  else epilogue.template operator()<kLinF32>();
}

// ------------------------------------------------------------ launchers ----

hipError_t launch_prep(const PrepParams& p, hipStream_t stream) {
  const int64_t blocks = p.M + prep_row_blocks(p.I, p.kext);
  hipLaunchKernelGGL(swq_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// The K split's second pass: for each output feature n < p.I of row m the
// splits' float32 gate and up sums (true scale; [split][M][p.I] planes),
// added in split order, then the epilogue of p.mode: the forward's SwiGLU,
// or the linear's two output columns n and p.I + n (the residual added in
// float32 before the one rounding).
__global__ __launch_bounds__(256) void swq_ksplit_epilogue(MfmaParams p, const float* __restrict__ part_g,
                                                           const float* __restrict__ part_u, int ksplit) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)p.M * p.I) return;
  const int m = (int)(i / p.I), n = (int)(i - (int64_t)m * p.I);
  const int64_t slice = (int64_t)p.M * p.I;
  float g = part_g[i], u = part_u[i];
  for (int k = 1; k < ksplit; ++k) {
    g += part_g[k * slice + i];
    u += part_u[k * slice + i];
  }
  const int64_t o = (int64_t)m * p.ldo + n;
  if (p.mode == kLinBf16 || p.mode == kLinF32) {
    const bool up = n < p.I_u;
    if (p.res) {
      g += bf16_to_f32(p.res[o]);
      if (up) u += bf16_to_f32(p.res[o + p.I]);
    }
    if (p.mode == kLinF32) {
      reinterpret_cast<float*>(p.out)[o] = g;
      if (up) reinterpret_cast<float*>(p.out)[o + p.I] = u;
    } else {
      reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_act(g, p.act);
      if (up) reinterpret_cast<uint16_t*>(p.out)[o + p.I] = f32_to_act(u, p.act);
    }
    return;
  }
  const float h = swiglu_epilogue(g, u, p.mode, p.act);
  if (p.mode == kF32) reinterpret_cast<float*>(p.out)[o] = h;
  else reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_act(h, p.act);
}

hipError_t launch_ksplit_epilogue(const MfmaParams& p, const float* part_g, const float* part_u, int ksplit,
                                  hipStream_t stream) {
  const int64_t n = (int64_t)p.M * p.I;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(swq_ksplit_epilogue, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, part_g,
                     part_u, ksplit);
  return hipGetLastError();
}

hipError_t launch_prep_rows(const PrepParams& p, hipStream_t stream) {
  const int64_t blocks = p.M + (p.k_only ? prep_row_blocks(p.I, p.kext) : 0);
  hipLaunchKernelGGL(swq_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int BG, int BU, int BM, int WN, int OCC, bool A16 = false, bool KSPLIT = false>
static hipError_t launch_mfma_t(const MfmaParams& p, hipStream_t stream, int ksplit = 1) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.n_end - p.n_begin + 4 * WN - 1) / (4 * WN));
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((swq_mfma_kernel<BG, BU, BM, WN, OCC, A16, KSPLIT>), dim3(tiles, KSPLIT ? ksplit : 1), dim3(256),
                     0, stream, p);
  return hipGetLastError();
}

template <int BG, int BU, bool A16>
static hipError_t launch_mfma_cfg(const MfmaParams& p, int cfg, int n_split, int ksplit, hipStream_t stream) {
  // K split: 128-row tiles (64-row ones for at most 64 rows), the splits
  // along grid y (the host's choice: few tiles)
  if (ksplit > 1) {
    if (p.M <= 64) return launch_mfma_t<BG, BU, 64, 32, 1, A16, true>(p, stream, ksplit);
    return launch_mfma_t<BG, BU, 128, 32, 1, A16, true>(p, stream, ksplit);
  }
  // 8-bit codes in both matrices need the larger code ring: 128-row tiles only
  if (cfg == 1 || (BG == 8 && BU == 8)) return launch_mfma_t<BG, BU, 128, 32, 1, A16>(p, stream);
  if constexpr (!(BG == 8 && BU == 8)) {
    if (n_split <= 0 || n_split >= p.I) return launch_mfma_t<BG, BU, 256, 32, 1, A16>(p, stream);
    // columns [0, n_split) in whole rounds of 256 x 128 tiles, the rest in 128 x 128 tiles
    MfmaParams a = p, b = p;
    a.n_end = n_split;
    b.n_begin = n_split;
    const hipError_t e = launch_mfma_t<BG, BU, 256, 32, 1, A16>(a, stream);
    if (e != hipSuccess) return e;
    return launch_mfma_t<BG, BU, 128, 32, 1, A16>(b, stream);
  }
  return hipErrorInvalidValue;
}

// binary16 activations take the instances with the split-scale planes
template <int BG, int BU>
static hipError_t launch_mfma_bits(const MfmaParams& p, int cfg, int n_split, int ksplit, hipStream_t stream) {
  if (p.act == kActF16) return launch_mfma_cfg<BG, BU, true>(p, cfg, n_split, ksplit, stream);
  return launch_mfma_cfg<BG, BU, false>(p, cfg, n_split, ksplit, stream);
}

template <int BG>
static hipError_t launch_mfma_g(const MfmaParams& p, int cfg, int n_split, int ksplit, int bits_u, hipStream_t stream) {
  if (bits_u == 2) return launch_mfma_bits<BG, 2>(p, cfg, n_split, ksplit, stream);
  if (bits_u == 4) return launch_mfma_bits<BG, 4>(p, cfg, n_split, ksplit, stream);
  if (bits_u == 8) return launch_mfma_bits<BG, 8>(p, cfg, n_split, ksplit, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_mfma(const MfmaParams& p, int cfg, int n_split, int ksplit, int bits_g, int bits_u,
                       hipStream_t stream) {
  if (bits_g == 2) return launch_mfma_g<2>(p, cfg, n_split, ksplit, bits_u, stream);
  if (bits_g == 4) return launch_mfma_g<4>(p, cfg, n_split, ksplit, bits_u, stream);
  if (bits_g == 8) return launch_mfma_g<8>(p, cfg, n_split, ksplit, bits_u, stream);
  return hipErrorInvalidValue;
}

}  // namespace swq
