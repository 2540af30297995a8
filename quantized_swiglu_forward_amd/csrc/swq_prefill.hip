// Matrix-matrix path (M >= threshold) of the fused quantized SwiGLU:
//   hidden[M, I] = silu(x Wg^T) * (x Wu^T)
// One dispatch produces a BM x BN tile of BOTH projections from one staged
// x tile, then applies the epilogue in registers ("mlx-bun 0.0.7 -> 0.0.9"
// diff, page 42, fused-swiglu-kernel.ts: header comment and kernel source,
// where x is read once for two GEMMs and down_proj stays separate).
//
// Two kernels:
//  1. swq_prep_kernel  (one block per row of x): picks a power-of-two row
//     scale 2^-e so that max|x'| lies in [1, 2), writes x' = x * 2^-e as
//     binary16 in the [0,4,1,5,2,6,3,7] order that matches the dequantized
//     weight pairs, and appends per-group sums of x' (split hi + lo in
//     binary16, plain and times the code offset z) as extra K columns.
//     Every bf16 x whose magnitude is at least 2^-18 of the row maximum
//     converts exactly.
//  2. swq_mfma_kernel: f16 MFMA 32x32x16 with float32 accumulators.  The
//     main K loop streams packed codes, dequantizes them to the exact
//     binary16 values s*(q - z) and feeds them to the MFMA; two short extra
//     K loops add sum_g Sx[m,g] * (b[n,g] + z*s[n,g]) with the bias and
//     scale as exact binary16 B operands.  The epilogue multiplies by 2^e
//     (exact), then computes silu(g) * u per precision mode.
#include "swq_device.h"
#include "swq_kernels.h"

namespace swq {

// ---------------------------------------------------------------- prep ----

__global__ __launch_bounds__(256) void swq_prep_kernel(PrepParams p) {
  const int m = blockIdx.x;
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
  const int gchunks_g = p.gs_g / 8, gchunks_u = p.gs_u / 8;
  const int ngroups_g = p.H / p.gs_g, ngroups_u = p.H / p.gs_u;
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
    // group sums: a group is gs/8 consecutive chunks = consecutive lanes
    float sg = part, su = part;
    for (int off = 1; off < gchunks_g; off <<= 1) sg += __shfl_xor(sg, off);
    for (int off = 1; off < gchunks_u; off <<= 1) su += __shfl_xor(su, off);
    if (c < nchunk && (c % gchunks_g) == 0) {
      const int g = c / gchunks_g;
      const float zs = p.z_g * sg;
      const _Float16 h0 = (_Float16)sg, h2 = (_Float16)zs;
      _Float16* dst = arow + p.H + 4 * g;
      dst[0] = h0;
      dst[1] = (_Float16)(sg - (float)h0);
      dst[2] = h2;
      dst[3] = (_Float16)(zs - (float)h2);
    }
    if (c < nchunk && (c % gchunks_u) == 0) {
      const int g = c / gchunks_u;
      const float zs = p.z_u * su;
      const _Float16 h0 = (_Float16)su, h2 = (_Float16)zs;
      _Float16* dst = arow + p.H + p.kext_g + 4 * g;
      dst[0] = h0;
      dst[1] = (_Float16)(su - (float)h0);
      dst[2] = h2;
      dst[3] = (_Float16)(zs - (float)h2);
    }
  }
  // zero padding of the extra columns
  for (int k = 4 * ngroups_g + tid; k < p.kext_g; k += 256) arow[p.H + k] = (_Float16)0.0f;
  for (int k = 4 * ngroups_u + tid; k < p.kext_u; k += 256) arow[p.H + p.kext_g + k] = (_Float16)0.0f;
}

// ----------------------------------------------------------- MFMA GEMM ----

template <int BITS_G, int BITS_U, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64, 1) void swq_mfma_kernel(MfmaParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int BK = 32;           // K per pipeline step (two MFMA k16 steps)
  constexpr int LDK = BK + 8;      // LDS row pitch in halves (80 bytes)
  constexpr int PG = BITS_G == 8 ? 2 : 1;
  constexpr int PU = BITS_U == 8 ? 2 : 1;
  constexpr int NPL = PG + PU;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int CG = BITS_G / 4, CU = BITS_U / 4;   // 16-byte code chunks per row per step
  constexpr int A_CH = BM * 4;                      // 16-byte x chunks per step
  constexpr int A_IT = (A_CH + NT - 1) / NT;
  constexpr int B_CH = BN * (CG + CU);
  constexpr int B_IT = (B_CH + NT - 1) / NT;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");

  __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][NPL][BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const int ntn = (p.I + BN - 1) / BN;
  const int tile = blockIdx.x;
  const int n0 = (tile % ntn) * BN;
  const int m0 = (tile / ntn) * BM;

  const int ksteps_main = p.H / BK;
  const int ksteps_g = p.kext_g / BK;
  const int ksteps_u = p.kext_u / BK;
  const int ksteps = ksteps_main + ksteps_g + ksteps_u;
  const int rw_g = p.H * BITS_G / 32;   // words per packed row
  const int rw_u = p.H * BITS_U / 32;
  const int ng_g = p.H / p.gs_g, ng_u = p.H / p.gs_u;

  f32x16 acc_g[FM][FN], acc_u[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc_g[i][j][r] = 0.0f;
        acc_u[i][j][r] = 0.0f;
      }

  // staged global data of one step
  u32x4 ra[A_IT];
  u32x4 rb[B_IT];
  uint32_t rs[B_IT];          // bf16 scale of the chunk's group (main phase)
  uint32_t rx[B_IT][8];       // ext phase: 8 (bias, scale) pairs as packed bf16x2

  auto load_step = [&](int t) {
    int kcol;
    if (t < ksteps_main) kcol = t * BK;
    else if (t < ksteps_main + ksteps_g) kcol = p.H + (t - ksteps_main) * BK;
    else kcol = p.H + p.kext_g + (t - ksteps_main - ksteps_g) * BK;
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
      const int c = tid + it * NT;
      if (c < A_CH) {
        const int row = c >> 2, part = c & 3;
        const int gm = min(m0 + row, p.M - 1);
        ra[it] = *reinterpret_cast<const u32x4*>(p.xa + (int64_t)gm * p.ldx + kcol + part * 8);
      }
    }
    if (t < ksteps_main) {
      const int k0 = t * BK;
#pragma unroll
      for (int it = 0; it < B_IT; ++it) {
        const int c = tid + it * NT;
        if (c < B_CH) {
          if (c < BN * CG) {
            const int row = c / CG, part = c % CG;
            const int gn = min(n0 + row, p.I - 1);
            rb[it] = *reinterpret_cast<const u32x4*>(p.wg + (int64_t)gn * rw_g + (k0 * BITS_G) / 32 + part * 4);
            rs[it] = p.sg[(int64_t)gn * ng_g + k0 / p.gs_g];
          } else {
            const int cc = c - BN * CG;
            const int row = cc / CU, part = cc % CU;
            const int gn = min(n0 + row, p.I - 1);
            rb[it] = *reinterpret_cast<const u32x4*>(p.wu + (int64_t)gn * rw_u + (k0 * BITS_U) / 32 + part * 4);
            rs[it] = p.su[(int64_t)gn * ng_u + k0 / p.gs_u];
          }
        }
      }
    } else {
      const bool gate = t < ksteps_main + ksteps_g;
      const int ke = gate ? (t - ksteps_main) * BK : (t - ksteps_main - ksteps_g) * BK;
      const uint16_t* bsrc = gate ? p.bg : p.bu;
      const uint16_t* ssrc = gate ? p.sg : p.su;
      const int ng = gate ? ng_g : ng_u;
#pragma unroll
      for (int it = 0; it < B_IT; ++it) {
        const int row = tid + it * NT;
        if (row < BN) {
          const int gn = min(n0 + row, p.I - 1);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int g = ke / 4 + j;
            uint32_t v = 0;
            if (g < ng) {
              v = (uint32_t)bsrc[(int64_t)gn * ng + g] | ((uint32_t)ssrc[(int64_t)gn * ng + g] << 16);
            }
            rx[it][j] = v;
          }
        }
      }
    }
  };

  auto store_step = [&](int t, int buf) {
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
      const int c = tid + it * NT;
      if (c < A_CH) {
        const int row = c >> 2, part = c & 3;
        *reinterpret_cast<u32x4*>(&As[buf][row * LDK + part * 8]) = ra[it];
      }
    }
    if (t < ksteps_main) {
#pragma unroll
      for (int it = 0; it < B_IT; ++it) {
        const int c = tid + it * NT;
        if (c < B_CH) {
          const bool gate = c < BN * CG;
          const int cc = gate ? c : c - BN * CG;
          const int bits = gate ? BITS_G : BITS_U;
          const int per = gate ? CG : CU;
          const int row = cc / per, part = cc % per;
          const int plane0 = gate ? 0 : PG;
          const f16x2 s2 = bf16_to_h2((uint16_t)rs[it]);
          if (bits == 4) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              uint32_t o[4];
              dequant4(rb[it][kb], s2, o);
              *reinterpret_cast<u32x4*>(&Bs[buf][plane0][row * LDK + kb * 8]) =
                  (u32x4){o[0], o[1], o[2], o[3]};
            }
          } else {
            const f16x2 s16 = s2 * (f16x2){(_Float16)16.0f, (_Float16)16.0f};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              uint32_t lo[4], hi[4];
              codes8(rb[it][2 * h], rb[it][2 * h + 1], lo, hi);
              const int kb = part * 2 + h;
              u32x4 vl, vh;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                vl[j] = as_u32(as_h2(lo[j]) * s2);
                vh[j] = as_u32(as_h2(hi[j]) * s16);
              }
              *reinterpret_cast<u32x4*>(&Bs[buf][plane0][row * LDK + kb * 8]) = vl;
              *reinterpret_cast<u32x4*>(&Bs[buf][plane0 + 1][row * LDK + kb * 8]) = vh;
            }
          }
        }
      }
    } else {
      const bool gate = t < ksteps_main + ksteps_g;
      const int plane = gate ? 0 : PG;
#pragma unroll
      for (int it = 0; it < B_IT; ++it) {
        const int row = tid + it * NT;
        if (row < BN) {
          // ext column 4g+j: B = b, b, s, s
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            u32x4 v;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t bs = rx[it][2 * q + h];
              const _Float16 b = (_Float16)bf16_to_f32((uint16_t)(bs & 0xFFFFu));
              const _Float16 s = (_Float16)bf16_to_f32((uint16_t)(bs >> 16));
              v[2 * h] = as_u32((f16x2){b, b});
              v[2 * h + 1] = as_u32((f16x2){s, s});
            }
            *reinterpret_cast<u32x4*>(&Bs[buf][plane][row * LDK + q * 8]) = v;
          }
        }
      }
    }
  };

  auto compute_step = [&](int t, int buf) {
    const bool main_phase = t < ksteps_main;
    const bool do_g = main_phase || t < ksteps_main + ksteps_g;
    const bool do_u = main_phase || !do_g;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kk = ks * 16 + (lane >> 5) * 8;
      f16x8 a[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = *reinterpret_cast<const f16x8*>(&As[buf][(wm * TM + i * 32 + (lane & 31)) * LDK + kk]);
      if (do_g) {
        const int npl = main_phase ? PG : 1;
        for (int pl = 0; pl < npl; ++pl) {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const f16x8 b = *reinterpret_cast<const f16x8*>(
                &Bs[buf][pl][(wn * TN + j * 32 + (lane & 31)) * LDK + kk]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
              acc_g[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b, acc_g[i][j], 0, 0, 0);
          }
        }
      }
      if (do_u) {
        const int npl = main_phase ? PU : 1;
        for (int pl = 0; pl < npl; ++pl) {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const f16x8 b = *reinterpret_cast<const f16x8*>(
                &Bs[buf][PG + pl][(wn * TN + j * 32 + (lane & 31)) * LDK + kk]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
              acc_u[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b, acc_u[i][j], 0, 0, 0);
          }
        }
      }
    }
  };

  // software pipeline: global loads of step t+1 overlap the MFMAs of step t
  load_step(0);
  store_step(0, 0);
  __syncthreads();
  for (int t = 0; t < ksteps; ++t) {
    const int buf = t & 1;
    if (t + 1 < ksteps) load_step(t + 1);
    compute_step(t, buf);
    if (t + 1 < ksteps) store_step(t + 1, buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 8*(r/4) + 4*(lane/32) + r%4 of column lane%32
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * TM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      if (row >= p.M) continue;
      const int e = p.xexp[row];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * TN + j * 32 + (lane & 31);
        if (col >= p.I) continue;
        const float g = ldexpf(acc_g[i][j][r], e);
        const float u = ldexpf(acc_u[i][j][r], e);
        const int64_t o = (int64_t)row * p.I + col;
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
  hipLaunchKernelGGL(swq_prep_kernel, dim3(p.M), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int BG, int BU, int BM, int BN, int WM, int WN>
static hipError_t launch_mfma_t(const MfmaParams& p, hipStream_t stream) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.I + BN - 1) / BN);
  hipLaunchKernelGGL((swq_mfma_kernel<BG, BU, BM, BN, WM, WN>), dim3(tiles), dim3(WM * WN * 64), 0,
                     stream, p);
  return hipGetLastError();
}

template <int BG, int BU>
static hipError_t launch_mfma_bits(const MfmaParams& p, int cfg, hipStream_t stream) {
  switch (cfg) {
    case 0: return launch_mfma_t<BG, BU, 128, 128, 2, 2>(p, stream);
    case 1: return launch_mfma_t<BG, BU, 256, 128, 2, 2>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_mfma(const MfmaParams& p, int cfg, int bits_g, int bits_u, hipStream_t stream) {
  if (bits_g == 4 && bits_u == 4) return launch_mfma_bits<4, 4>(p, cfg, stream);
  if (bits_g == 8 && bits_u == 4) return launch_mfma_bits<8, 4>(p, cfg, stream);
  if (bits_g == 4 && bits_u == 8) return launch_mfma_bits<4, 8>(p, cfg, stream);
  if (bits_g == 8 && bits_u == 8) return launch_mfma_bits<8, 8>(p, cfg, stream);
  return hipErrorInvalidValue;
}

}  // namespace swq
