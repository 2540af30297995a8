// Matrix-matrix path (M >= threshold) of the fused quantized SwiGLU:
//   hidden[M, I] = silu(x Wg^T) * (x Wu^T)
// One dispatch produces a BM x BN tile of BOTH projections from one staged
// x tile, then applies the epilogue in registers ("mlx-bun 0.0.7 -> 0.0.9"
// diff, page 42, fused-swiglu-kernel.ts: header comment and kernel source,
// where x is read once for two GEMMs and down_proj stays separate).
//
// Two kernels:
//  1. swq_prep_kernel.  Blocks [0, M): one row of x each.  It picks a
//     power-of-two row scale 2^-e so that max|x'| lies in [1, 2), writes
//     x' = x * 2^-e as binary16 in the [0,4,1,5,2,6,3,7] order that matches
//     the dequantized weight pairs, and appends, per group of
//     g0 = min(gs_g, gs_u) inputs, the group sum Sx of x' split as hi + lo
//     binary16 values, in four extra K columns (hi, lo, hi, lo).  Every bf16
//     x whose magnitude is at least 2^-17 of the row maximum converts
//     exactly.  The remaining blocks write the B rows of those extra
//     columns for every output feature: (b, b, 8s, 8s) per group (exact in
//     binary16), and for an 8-bit matrix a second plane (128s, 128s, 0, 0),
//     so that the extra columns add sum_g Sx[m,g] * (b[n,g] + z*s[n,g]).
//  2. swq_mfma_kernel: f16 MFMA 32x32x16 with float32 accumulators.  The K
//     loop streams the packed codes, dequantizes them to the exact binary16
//     values s*(q - z) and feeds them to the MFMA, then runs over the extra
//     columns.  The epilogue multiplies by 2^e (exact), then computes
//     silu(g) * u per precision mode.
#include "swq_device.h"
#include "swq_kernels.h"

namespace swq {

// ---------------------------------------------------------------- prep ----

__device__ __forceinline__ void prep_x_row(const PrepParams& p, int m) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint16_t* xrow = p.x + (int64_t)m * p.H;
  _Float16* arow = p.xa + (int64_t)m * p.ldx;
  const int nchunk = p.H / 8;

  // 1. row maximum of |x| (on the bf16 magnitude bits: monotone for finite values)
  uint32_t amax = 0;
  for (int c = tid; c < nchunk; c += 256) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xrow + 8 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = max(amax, v[j] & 0x7FFFu);
      amax = max(amax, (v[j] >> 16) & 0x7FFFu);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
  __shared__ uint32_t red[4];
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = max(max(red[0], red[1]), max(red[2], red[3]));
  // exponent of the row maximum: max|x| in [2^e, 2^(e+1))
  int e = 0;
  if (amax != 0) {
    const int field = (int)(amax >> 7);
    e = (field == 0) ? -127 : field - 127;
  }
  if (tid == 0) p.xexp[m] = e;

  // 2. scaled binary16 copy in pair order, and per-group sums
  const int gchunks = p.g0 / 8;
  const int ngroups = p.H / p.g0;
  _Float16* ext = arow + p.H;
  for (int base = 0; base < nchunk; base += 256) {
    const int c = base + tid;
    float part = 0.0f;
    if (c < nchunk) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(xrow + 8 * c);
      float f[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[2 * j] = ldexpf(bf16_to_f32((uint16_t)(v[j] & 0xFFFFu)), -e);
        f[2 * j + 1] = ldexpf(bf16_to_f32((uint16_t)(v[j] >> 16)), -e);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) part += f[j];
      f16x8 h;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[2 * j] = (_Float16)f[j];
        h[2 * j + 1] = (_Float16)f[j + 4];
      }
      *reinterpret_cast<f16x8*>(arow + 8 * c) = h;
    }
    // a group is g0/8 consecutive 8-value blocks = consecutive lanes
    for (int off = 1; off < gchunks; off <<= 1) part += __shfl_xor(part, off);
    if (c < nchunk && (c % gchunks) == 0) {
      const int g = c / gchunks;
      const _Float16 hi = (_Float16)part;
      const _Float16 lo = (_Float16)(part - (float)hi);
      *reinterpret_cast<f16x2*>(ext + 4 * g) = (f16x2){hi, lo};
      *reinterpret_cast<f16x2*>(ext + 4 * g + 2) = (f16x2){hi, lo};
    }
  }
  // zero padding of the extra columns
  for (int k = 4 * ngroups + tid; k < p.kext; k += 256) ext[k] = (_Float16)0.0f;
}

// B rows of the extra columns for one matrix: thread (n, G) writes columns
// [4G, 4G+4) of row n (zeros in the padding).
__device__ __forceinline__ void prep_ext_rows(const uint16_t* S, const uint16_t* B, int gs, int bits, int g0,
                                              int H, int I, int kext, _Float16* lo, _Float16* hi,
                                              int64_t idx) {
  const int per_row = kext / 4;
  if (idx >= (int64_t)I * per_row) return;
  const int n = (int)(idx / per_row), G = (int)(idx % per_row);
  f16x2 v0 = {(_Float16)0.0f, (_Float16)0.0f}, v1 = v0, h0 = v0;
  if (G < H / g0) {
    const int g = G * g0 / gs;
    const int ng = H / gs;
    const float b = bf16_to_f32(B[(int64_t)n * ng + g]);
    const float s = bf16_to_f32(S[(int64_t)n * ng + g]);
    const _Float16 bb = (_Float16)b, s8 = (_Float16)(8.0f * s), s128 = (_Float16)(128.0f * s);
    v0 = (f16x2){bb, bb};
    v1 = (f16x2){s8, s8};
    h0 = (f16x2){s128, s128};
  }
  const int64_t o = (int64_t)n * kext + 4 * G;
  *reinterpret_cast<f16x2*>(lo + o) = v0;
  *reinterpret_cast<f16x2*>(lo + o + 2) = v1;
  if (bits == 8) {
    *reinterpret_cast<f16x2*>(hi + o) = h0;
    *reinterpret_cast<f16x2*>(hi + o + 2) = (f16x2){(_Float16)0.0f, (_Float16)0.0f};
  }
}

__global__ __launch_bounds__(256) void swq_prep_kernel(PrepParams p) {
  if ((int)blockIdx.x < p.M) {
    prep_x_row(p, blockIdx.x);
    return;
  }
  const int64_t idx = (int64_t)(blockIdx.x - p.M) * 256 + threadIdx.x;
  const int64_t per_mat = (int64_t)p.I * (p.kext / 4);
  if (idx < per_mat)
    prep_ext_rows(p.sg, p.bg, p.gs_g, p.bits_g, p.g0, p.H, p.I, p.kext, p.bext_g, p.bext_g2, idx);
  else
    prep_ext_rows(p.su, p.bu, p.gs_u, p.bits_u, p.g0, p.H, p.I, p.kext, p.bext_u, p.bext_u2, idx - per_mat);
}

// ----------------------------------------------------------- MFMA GEMM ----
//
// Work split.  A block of four wavefronts (one per SIMD) computes a 256 x 128
// tile of both projections.  Wave (wm, wn) owns rows [128 wm, 128 wm + 128)
// and columns [64 wn, 64 wn + 64) of the gate AND the up tile: 4 x 2 MFMA
// 32x32x16 fragments per matrix, 256 float32 accumulators per lane.
//  * x' (the A operand) goes through a 3-stage LDS ring; its global loads are
//    issued two K-steps ahead and written to LDS one K-step ahead.
//  * The B side is staged in LDS per super-step: four K-steps of packed codes
//    (64 or 128 bytes per row) with their scales, or one K-step of the
//    precomputed extra-column rows (64 bytes per plane).  Rows are read as
//    whole segments, one super-step ahead.  Each lane then reads the codes
//    of its columns and two 8-code blocks from LDS and dequantizes them in
//    registers just before the MFMA: lane l holds column l%32 and blocks
//    2(l/32), 2(l/32)+1 of the 32-wide K-step, one per MFMA k16 step (A is
//    read for the same blocks).
//  * Global accesses are buffer loads: per-lane offsets fixed for the whole
//    loop, the K position as a scalar offset.

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Dequantized B operands of one k-block (8 codes) of one matrix.
template <int BITS>
__device__ __forceinline__ void code_operands(const uint32_t* w, f16x2 s2, f16x8& b0, f16x8& b1) {
  if (BITS == 4) {
    uint32_t o[4];
    dequant4(w[0], s2, o);
    b0 = __builtin_bit_cast(f16x8, (u32x4){o[0], o[1], o[2], o[3]});
  } else {
    uint32_t lo[4], hi[4];
    codes8(w[0], w[1], lo, hi);
    const f16x2 s16 = s2 * (f16x2){(_Float16)16.0f, (_Float16)16.0f};
    u32x4 vl, vh;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vl[j] = as_u32(as_h2(lo[j]) * s2);
      vh[j] = as_u32(as_h2(hi[j]) * s16);
    }
    b0 = __builtin_bit_cast(f16x8, vl);
    b1 = __builtin_bit_cast(f16x8, vh);
  }
}

template <int BITS_G, int BITS_U>
__global__ __launch_bounds__(256) void swq_mfma_kernel(MfmaParams p) {
  constexpr int NT = 256;
  constexpr int BM = 256, BN = 128;
  constexpr int LDK = 40;                        // A row pitch in halves (80 bytes)
  constexpr int A_IT = BM * 4 / NT;              // 16-byte x' chunks per thread per step
  constexpr int RBG = BITS_G * 16, RBU = BITS_U * 16;   // staged bytes per row per super-step
  constexpr int PG = RBG + 16, PU = RBU + 16;           // LDS row pitches
  constexpr int CHG = RBG / 16, CHU = RBU / 16;         // 16-byte pieces per row
  constexpr int SS_CH = BN * (CHG + CHU);
  constexpr int SS_IT = SS_CH / NT;
  constexpr int IT_G = BN * CHG / NT;            // slots [0, IT_G) stage gate rows, the rest up rows
  static_assert(SS_IT * NT == SS_CH && IT_G * NT == BN * CHG, "staged pieces must divide evenly");
  static_assert(A_IT * NT == BM * 4, "x' chunks must divide evenly");

  __shared__ __attribute__((aligned(16))) _Float16 As[3][BM * LDK];
  __shared__ __attribute__((aligned(16))) unsigned char Bq[2][BN * (PG + PU)];
  __shared__ __attribute__((aligned(16))) uint16_t Sq[2][2][BN * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;

  // XCD-aware tile order: consecutive tiles land on the same XCD (blocks are
  // dealt round-robin to the 8 XCDs); within an XCD's range the row tile
  // varies fastest, so concurrent blocks share weights and x' in its L2.
  const int T = gridDim.x;
  const int q8 = T / 8, r8 = T % 8;
  const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const int logical = xcd < r8 ? xcd * (q8 + 1) + local : r8 * (q8 + 1) + (xcd - r8) * q8 + local;
  const int mtiles = (p.M + BM - 1) / BM;
  const int m0 = (logical % mtiles) * BM;
  const int n0 = (logical / mtiles) * BN;
  const int rows = min(BM, p.M - m0);
  const int cols = min(BN, p.I - n0);

  const int s_main = p.H / 32;                   // multiple of 1; super-steps of 4
  const int s_ext = p.kext / 32;
  const int rw_g = p.H * BITS_G / 32, rw_u = p.H * BITS_U / 32;
  const int ng_g = p.H / p.gs_g, ng_u = p.H / p.gs_u;

  const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(p.xa + (int64_t)m0 * p.ldx, (uint32_t)rows * p.ldx * 2);
  const __amdgpu_buffer_rsrc_t rs_wg = make_rsrc(p.wg + (int64_t)n0 * rw_g, (uint32_t)cols * rw_g * 4);
  const __amdgpu_buffer_rsrc_t rs_wu = make_rsrc(p.wu + (int64_t)n0 * rw_u, (uint32_t)cols * rw_u * 4);
  const __amdgpu_buffer_rsrc_t rs_sg = make_rsrc(p.sg + (int64_t)n0 * ng_g, (uint32_t)cols * ng_g * 2);
  const __amdgpu_buffer_rsrc_t rs_su = make_rsrc(p.su + (int64_t)n0 * ng_u, (uint32_t)cols * ng_u * 2);
  // the second plane of an 8-bit matrix follows its first plane at p.ext_plane bytes
  const uint32_t ebytes = (uint32_t)cols * p.kext * 2;
  const __amdgpu_buffer_rsrc_t rs_eg =
      make_rsrc(p.bext_g + (int64_t)n0 * p.kext, ebytes + (BITS_G == 8 ? (uint32_t)p.ext_plane : 0u));
  const __amdgpu_buffer_rsrc_t rs_eu =
      make_rsrc(p.bext_u + (int64_t)n0 * p.kext, ebytes + (BITS_U == 8 ? (uint32_t)p.ext_plane : 0u));

  uint32_t aoff[A_IT];
#pragma unroll
  for (int it = 0; it < A_IT; ++it) {
    const int c = tid + it * NT;
    aoff[it] = (uint32_t)((min(c >> 2, rows - 1) * p.ldx + (c & 3) * 8) * 2);
  }
  // staged B piece it of this thread: (matrix, row, 16-byte part)
  uint32_t qoff[SS_IT];
#pragma unroll
  for (int it = 0; it < SS_IT; ++it) {
    const bool g = it < IT_G;
    const int cc = g ? tid + it * NT : tid + (it - IT_G) * NT;
    const int per = g ? CHG : CHU;
    const int row = min(cc / per, cols - 1), part = cc % per;
    qoff[it] = (uint32_t)(row * (g ? rw_g : rw_u) * 4 + part * 16);
  }
  // scale staging: thread t owns (matrix t / BN, row t % BN); uniform per wave
  const bool s_gate = __builtin_amdgcn_readfirstlane(tid) < BN;
  const int s_row = tid % BN;
  const uint32_t s_off = (uint32_t)(min(s_row, cols - 1) * (s_gate ? ng_g : ng_u) * 2);
  const int s_gs = s_gate ? p.gs_g : p.gs_u;

  f32x16 acc_g[4][2], acc_u[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc_g[i][j][r] = 0.0f;
        acc_u[i][j][r] = 0.0f;
      }

  u32x4 ra[3][A_IT];
  u32x4 qs[SS_IT];          // staged codes of the next super-step
  uint32_t ss_s[4];         // staged scales of the next super-step

  // ---- loads (unconditional: past-the-end loads are harmless and unused)
  auto issue_a = [&](int kcol, u32x4 (&a)[A_IT]) {
#pragma unroll
    for (int it = 0; it < A_IT; ++it) a[it] = __builtin_amdgcn_raw_buffer_load_b128(rs_a, aoff[it], kcol * 2, 0);
  };
  auto issue_ss = [&](int ss) {
#pragma unroll
    for (int it = 0; it < SS_IT; ++it) {
      if (it < IT_G) qs[it] = __builtin_amdgcn_raw_buffer_load_b128(rs_wg, qoff[it], ss * RBG, 0);
      else qs[it] = __builtin_amdgcn_raw_buffer_load_b128(rs_wu, qoff[it], ss * RBU, 0);
    }
    const int g0i = (ss * 128) / s_gs;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      ss_s[q] = s_gate ? __builtin_amdgcn_raw_buffer_load_b16(rs_sg, s_off, (g0i + q) * 2, 0)
                       : __builtin_amdgcn_raw_buffer_load_b16(rs_su, s_off, (g0i + q) * 2, 0);
  };
  auto write_ss = [&](int buf) {
#pragma unroll
    for (int it = 0; it < SS_IT; ++it) {
      const bool g = it < IT_G;
      const int cc = g ? tid + it * NT : tid + (it - IT_G) * NT;
      const int per = g ? CHG : CHU;
      const int row = cc / per, part = cc % per;
      const int o = g ? row * PG + part * 16 : BN * PG + row * PU + part * 16;
      *reinterpret_cast<u32x4*>(&Bq[buf][o]) = qs[it];
    }
    uint16_t* d = &Sq[buf][s_gate ? 0 : 1][s_row * 4];
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = (uint16_t)ss_s[q];
  };
  auto write_a = [&](int stage, const u32x4 (&a)[A_IT]) {
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
      const int c = tid + it * NT;
      *reinterpret_cast<u32x4*>(&As[stage][(c >> 2) * LDK + (c & 3) * 8]) = a[it];
    }
  };

  auto mfma4 = [&](const f16x8 (&a)[4], int f, const f16x8& bg0, const f16x8& bg1, const f16x8& bu0,
                   const f16x8& bu1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc_g[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], bg0, acc_g[i][f], 0, 0, 0);
      if (BITS_G == 8) acc_g[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], bg1, acc_g[i][f], 0, 0, 0);
      acc_u[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], bu0, acc_u[i][f], 0, 0, 0);
      if (BITS_U == 8) acc_u[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], bu1, acc_u[i][f], 0, 0, 0);
    }
  };

  // K-step with sub-step Q (0..3) of super-step buffer BUF, A stage STAGE
  auto compute_main = [&]<int Q>(int stage, int buf) {
    const _Float16* abase = &As[stage][(wm * 128 + l32) * LDK];
    f16x2 sg2[2], su2[2];
    uint32_t wgv[2][4], wuv[2][4];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int cl = wn * 64 + f * 32 + l32;
      const unsigned char* qg = &Bq[buf][cl * PG + Q * (BITS_G * 4) + half * (BITS_G * 2)];
      const unsigned char* qu = &Bq[buf][BN * PG + cl * PU + Q * (BITS_U * 4) + half * (BITS_U * 2)];
      if (BITS_G == 4) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(qg);
        wgv[f][0] = v[0]; wgv[f][1] = v[1];
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(qg);
        wgv[f][0] = v[0]; wgv[f][1] = v[1]; wgv[f][2] = v[2]; wgv[f][3] = v[3];
      }
      if (BITS_U == 4) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(qu);
        wuv[f][0] = v[0]; wuv[f][1] = v[1];
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(qu);
        wuv[f][0] = v[0]; wuv[f][1] = v[1]; wuv[f][2] = v[2]; wuv[f][3] = v[3];
      }
      sg2[f] = bf16_to_h2(Sq[buf][0][cl * 4 + (Q * 32) / p.gs_g]);
      su2[f] = bf16_to_h2(Sq[buf][1][cl * 4 + (Q * 32) / p.gs_u]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kk = (2 * half + ks) * 8;
      f16x8 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const f16x8*>(abase + i * 32 * LDK + kk);
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        f16x8 bg0, bg1, bu0, bu1;
        code_operands<BITS_G>(&wgv[f][ks * (BITS_G / 4)], sg2[f], bg0, bg1);
        code_operands<BITS_U>(&wuv[f][ks * (BITS_U / 4)], su2[f], bu0, bu1);
        mfma4(a, f, bg0, bg1, bu0, bu1);
      }
    }
  };

  // main K-step t = 12*it + K (K static): A stage K%3, super-step sub-step K%4
  auto main_step = [&]<int K>(int t) {
    constexpr int U = K % 3, Q = K % 4;
    __syncthreads();
    issue_a((t + 2) * 32, ra[(U + 2) % 3]);
    const int j = t >> 2;                      // super-step of this K-step
    if constexpr (Q == 0) issue_ss(j + 1);
    compute_main.template operator()<Q>(U, j & 1);
    write_a((U + 1) % 3, ra[(U + 1) % 3]);
    if constexpr (Q == 3) write_ss((j + 1) & 1);
  };

  // prologue: steps 0, 1 of A, super-step 0 of B
  issue_a(0, ra[0]);
  issue_a(32, ra[1]);
  issue_ss(0);
  write_a(0, ra[0]);
  write_ss(0);
  const int full = s_main / 12;
  int t = 0;
  for (int it = 0; it < full; ++it, t += 12) {
    main_step.template operator()<0>(t);
    main_step.template operator()<1>(t + 1);
    main_step.template operator()<2>(t + 2);
    main_step.template operator()<3>(t + 3);
    main_step.template operator()<4>(t + 4);
    main_step.template operator()<5>(t + 5);
    main_step.template operator()<6>(t + 6);
    main_step.template operator()<7>(t + 7);
    main_step.template operator()<8>(t + 8);
    main_step.template operator()<9>(t + 9);
    main_step.template operator()<10>(t + 10);
    main_step.template operator()<11>(t + 11);
  }
  // tail: the remaining s_main % 12 steps (runs once)
  {
    const int rem = s_main - t;
    if (rem > 0) main_step.template operator()<0>(t);
    if (rem > 1) main_step.template operator()<1>(t + 1);
    if (rem > 2) main_step.template operator()<2>(t + 2);
    if (rem > 3) main_step.template operator()<3>(t + 3);
    if (rem > 4) main_step.template operator()<4>(t + 4);
    if (rem > 5) main_step.template operator()<5>(t + 5);
    if (rem > 6) main_step.template operator()<6>(t + 6);
    if (rem > 7) main_step.template operator()<7>(t + 7);
    if (rem > 8) main_step.template operator()<8>(t + 8);
    if (rem > 9) main_step.template operator()<9>(t + 9);
    if (rem > 10) main_step.template operator()<10>(t + 10);
  }

  // ---- extra columns of the bias term: A = group sums of x', B = precomputed rows
  // staged in As[0] and Bq[0] with one step of prefetch
  {
    constexpr int EP_G = BITS_G == 8 ? 2 : 1, EP_U = BITS_U == 8 ? 2 : 1;
    u32x4 ea[A_IT];
    u32x4 eb[SS_IT];
    auto issue_e = [&](int e) {
      issue_a(p.H + e * 32, ea);
      // 64 bytes per plane-row per step: the same piece layout as the codes
#pragma unroll
      for (int it = 0; it < SS_IT; ++it) {
        const bool g = it < IT_G;
        const int cc = g ? tid + it * NT : tid + (it - IT_G) * NT;
        const int per = g ? CHG : CHU;
        const int row = min(cc / per, cols - 1), part = cc % per;
        // plane part/4: the second plane starts p.ext_plane bytes after the first
        const uint32_t off = (uint32_t)(row * p.kext * 2 + (part & 3) * 16 + (part >> 2) * p.ext_plane);
        if (g) eb[it] = __builtin_amdgcn_raw_buffer_load_b128(rs_eg, off, e * 64, 0);
        else eb[it] = __builtin_amdgcn_raw_buffer_load_b128(rs_eu, off, e * 64, 0);
      }
    };
    issue_e(0);
    for (int e = 0; e < s_ext; ++e) {
      __syncthreads();                        // previous users of As[0] / Bq[0] are done
      write_a(0, ea);
#pragma unroll
      for (int it = 0; it < SS_IT; ++it) qs[it] = eb[it];
      write_ss(0);
      __syncthreads();
      if (e + 1 < s_ext) issue_e(e + 1);
      const _Float16* abase = &As[0][(wm * 128 + l32) * LDK];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int kk = (2 * half + ks) * 8;
        f16x8 a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const f16x8*>(abase + i * 32 * LDK + kk);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int cl = wn * 64 + f * 32 + l32;
          const unsigned char* rg = &Bq[0][cl * PG];
          const unsigned char* ru = &Bq[0][BN * PG + cl * PU];
          const int kb = (2 * half + ks) * 16;
          const f16x8 bg0 = *reinterpret_cast<const f16x8*>(rg + kb);
          const f16x8 bu0 = *reinterpret_cast<const f16x8*>(ru + kb);
          f16x8 bg1 = bg0, bu1 = bu0;
          if (EP_G == 2) bg1 = *reinterpret_cast<const f16x8*>(rg + 64 + kb);
          if (EP_U == 2) bu1 = *reinterpret_cast<const f16x8*>(ru + 64 + kb);
          mfma4(a, f, bg0, bg1, bu0, bu1);
        }
      }
    }
  }

  // epilogue: lane holds rows 8*(r/4) + 4*(lane/32) + r%4 of column lane%32
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int ocol = n0 + wn * 64 + f * 32 + l32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
        if (row >= p.M || ocol >= p.I) continue;
        const int e = p.xexp[row];
        const float g = ldexpf(acc_g[i][f][r], e);
        const float u = ldexpf(acc_u[i][f][r], e);
        const int64_t o = (int64_t)row * p.I + ocol;
        if (p.dbg_g) {
          p.dbg_g[o] = g;
          p.dbg_u[o] = u;
        } else {
          const float h = swiglu_epilogue(g, u, p.mode);
          if (p.mode == kF32) reinterpret_cast<float*>(p.out)[o] = h;
          else reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16(h);
        }
      }
    }
  }
}

// ------------------------------------------------------------ launchers ----

hipError_t launch_prep(const PrepParams& p, hipStream_t stream) {
  const int64_t ext_threads = 2 * (int64_t)p.I * (p.kext / 4);
  const int64_t blocks = p.M + (ext_threads + 255) / 256;
  hipLaunchKernelGGL(swq_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int BG, int BU>
static hipError_t launch_mfma_bits(const MfmaParams& p, int cfg, hipStream_t stream) {
  (void)cfg;
  const int tiles = ((p.M + 255) / 256) * ((p.I + 127) / 128);
  hipLaunchKernelGGL((swq_mfma_kernel<BG, BU>), dim3(tiles), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_mfma(const MfmaParams& p, int cfg, int bits_g, int bits_u, hipStream_t stream) {
  if (bits_g == 4 && bits_u == 4) return launch_mfma_bits<4, 4>(p, cfg, stream);
  if (bits_g == 8 && bits_u == 4) return launch_mfma_bits<8, 4>(p, cfg, stream);
  if (bits_g == 4 && bits_u == 8) return launch_mfma_bits<4, 8>(p, cfg, stream);
  if (bits_g == 8 && bits_u == 8) return launch_mfma_bits<8, 8>(p, cfg, stream);
  return hipErrorInvalidValue;
}

}  // namespace swq
