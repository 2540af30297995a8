// Matrix-vector path (M < threshold) of the fused quantized SwiGLU.
//
// At decode the two projections are memory-bound matrix-vector products and
// reading Wg/Wu dominates ("mlx-bun 0.0.7 -> 0.0.9" diff, page 42,
// fused-swiglu-kernel.ts, the comment on where the fusion pays off, and the
// M-threshold function below which the caller keeps this path).  No MFMA
// here: lanes stream packed rows with 16-byte loads, turn codes into exact
// binary16 (q - 8) pairs and accumulate x'(q - 8) with v_dot2_f32_f16; per
// 32-input chunk (always inside one quantization group) the partial sum P
// and the chunk's sum of x' give  s*P + (b + z*s)*Sx  in float32.  A
// cross-lane reduction per column then yields gate and up, and the same
// epilogue as the matrix-matrix path writes hidden.
//
// x is used as x' = x * 2^-e in binary16 (e = exponent of the row maximum;
// exact for every element at least 2^-17 of the maximum), in the
// [0,4,1,5,2,6,3,7] order of the code pairs.
//
// Work split: a column group of `lpc` lanes (a power of two, at most 64)
// owns one output column at a time; lane sl of the group handles the
// 32-input chunks sl, sl + lpc, ...  Every lane issues its weight loads
// before anything else, so the whole weight stream is in flight while x is
// prepared.
//
// Two kernels:
//  * swq_gemv1_kernel: M = 1 with at most two chunks per lane.  Each lane
//    keeps its own x chunks in registers; the row maximum is a reduction over
//    the column group, which covers the whole row.  No LDS, no barriers.
//  * swq_gemvm_kernel: 1 <= M <= 16.  The block stages x' and per-chunk sums
//    in LDS; the loads of the next (column, chunk) item are in flight while
//    the current one is computed.
#include "swq_device.h"
#include "swq_kernels.h"

namespace swq {

// Raw weight data of one (column, chunk) item for one matrix.
template <int BITS>
struct RawChunk {
  u32x4 w[BITS / 4];   // 32 codes: 16 bytes (4-bit) or 32 bytes (8-bit)
  uint32_t sb;         // bf16 scale (low half) and bias (high half) of the chunk's group
};

template <int BITS>
__device__ __forceinline__ void load_chunk(RawChunk<BITS>& r, const uint32_t* W, const uint16_t* S,
                                           const uint16_t* B, int64_t row, int rw, int ng, int gs,
                                           int kc) {
  const uint32_t* base = W + row * rw + (int64_t)kc * (BITS);   // BITS words per 32-code chunk
#pragma unroll
  for (int i = 0; i < BITS / 4; ++i) r.w[i] = *reinterpret_cast<const u32x4*>(base + 4 * i);
  const int64_t gi = row * ng + (kc * 32) / gs;
  r.sb = (uint32_t)S[gi] | ((uint32_t)B[gi] << 16);
}

// sum over the chunk of x'(q - z) as float32, split as  s*P + (b + z s)*Sx.
template <int BITS>
__device__ __forceinline__ float chunk_dot(const RawChunk<BITS>& r, const uint32_t xv[16], float sx) {
  float p = 0.0f;
  if (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t q[4];
      codes4(r.w[0][j], q);
#pragma unroll
      for (int t = 0; t < 4; ++t) p = __builtin_amdgcn_fdot2(as_h2(xv[4 * j + t]), as_h2(q[t]), p, false);
    }
  } else {
    float ph = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t lo[4], hi[4];
      const u32x4& w = r.w[j / 2];
      codes8(w[2 * (j & 1)], w[2 * (j & 1) + 1], lo, hi);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        p = __builtin_amdgcn_fdot2(as_h2(xv[4 * j + t]), as_h2(lo[t]), p, false);
        ph = __builtin_amdgcn_fdot2(as_h2(xv[4 * j + t]), as_h2(hi[t]), ph, false);
      }
    }
    p = fmaf(16.0f, ph, p);
  }
  const float s = bf16_to_f32((uint16_t)(r.sb & 0xFFFFu));
  const float b = bf16_to_f32((uint16_t)(r.sb >> 16));
  const float c = fmaf(CodeOffset<BITS>::z, s, b);   // b + z*s
  return fmaf(s, p, c * sx);
}

__device__ __forceinline__ void store_out(const GemvParams& p, int m, int n, float g, float u) {
  const int64_t o = (int64_t)m * p.I + n;
  if (p.dbg_g) {
    p.dbg_g[o] = g;
    p.dbg_u[o] = u;
  } else {
    const float h = swiglu_epilogue(g, u, p.mode);
    if (p.mode == kF32) reinterpret_cast<float*>(p.out)[o] = h;
    else reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16(h);
  }
}

// bf16 x chunk (32 values) -> x' = x * 2^-e as binary16 pairs in code-pair order, and its sum.
__device__ __forceinline__ float convert_chunk(const u32x4 raw[4], int e, uint32_t xv[16]) {
  float sum = 0.0f;
#pragma unroll
  for (int b = 0; b < 4; ++b) {            // block of 8 values
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = ldexpf(bf16_to_f32((uint16_t)(raw[b][j] & 0xFFFFu)), -e);
      f[2 * j + 1] = ldexpf(bf16_to_f32((uint16_t)(raw[b][j] >> 16)), -e);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += f[j];
#pragma unroll
    for (int j = 0; j < 4; ++j) xv[4 * b + j] = as_u32((f16x2){(_Float16)f[j], (_Float16)f[j + 4]});
  }
  return sum;
}

__device__ __forceinline__ uint32_t chunk_absmax(const u32x4 raw[4]) {
  uint32_t a = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) a = max(a, max(raw[b][j] & 0x7FFFu, (raw[b][j] >> 16) & 0x7FFFu));
  return a;
}

__device__ __forceinline__ int row_exponent(uint32_t amax_bits) {
  if (amax_bits == 0) return 0;
  const int field = (int)(amax_bits >> 7);
  return field == 0 ? -127 : field - 127;
}

// ------------------------------------------------------------- M == 1 ----

template <int BITS_G, int BITS_U, int CPL, int R>
__global__ __launch_bounds__(256) void swq_gemv1_kernel(GemvParams p, int lpc) {
  const int lane = threadIdx.x & 63;
  const int wave_global = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int sub = lane / lpc, sl = lane % lpc;
  const int cpw = 64 / lpc;
  const int nchunk = p.H / 32;
  const int ng_g = p.H / p.gs_g, ng_u = p.H / p.gs_u;
  const int rw_g = p.H * BITS_G / 32, rw_u = p.H * BITS_U / 32;

  // 1. all weight loads of this lane's R columns x CPL chunks
  RawChunk<BITS_G> rg[R][CPL];
  RawChunk<BITS_U> ru[R][CPL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = (wave_global * R + r) * cpw + sub;
    const int nn = min(n, p.I - 1);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int kc = min(sl + c * lpc, nchunk - 1);
      load_chunk<BITS_G>(rg[r][c], p.wg, p.sg, p.bg, nn, rw_g, ng_g, p.gs_g, kc);
      load_chunk<BITS_U>(ru[r][c], p.wu, p.su, p.bu, nn, rw_u, ng_u, p.gs_u, kc);
    }
  }

  // 2. this lane's x chunks, the row exponent, x' and chunk sums
  u32x4 raw[CPL][4];
  uint32_t amax = 0;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int kc = sl + c * lpc;
    if (kc < nchunk) {
#pragma unroll
      for (int b = 0; b < 4; ++b) raw[c][b] = *reinterpret_cast<const u32x4*>(p.x + kc * 32 + 8 * b);
      amax = max(amax, chunk_absmax(raw[c]));
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) raw[c][b] = (u32x4){0u, 0u, 0u, 0u};
    }
  }
  for (int off = lpc >> 1; off > 0; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
  const int e = row_exponent(amax);
  uint32_t xv[CPL][16];
  float sx[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) sx[c] = convert_chunk(raw[c], e, xv[c]);

  // 3. per column: dot products, group reduction, epilogue
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float ag = 0.0f, au = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      if (sl + c * lpc < nchunk) {
        ag += chunk_dot<BITS_G>(rg[r][c], xv[c], sx[c]);
        au += chunk_dot<BITS_U>(ru[r][c], xv[c], sx[c]);
      }
    }
    for (int off = lpc >> 1; off > 0; off >>= 1) {
      ag += __shfl_xor(ag, off);
      au += __shfl_xor(au, off);
    }
    const int n = (wave_global * R + r) * cpw + sub;
    if (sl == 0 && n < p.I) store_out(p, 0, n, ldexpf(ag, e), ldexpf(au, e));
  }
}

// ---------------------------------------------------------- 1 <= M <= 16 --

template <int BITS_G, int BITS_U, int MAXM>
__global__ __launch_bounds__(256) void swq_gemvm_kernel(GemvParams p, int lpc, int rounds) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int H = p.H, M = p.M;
  const int nchunk = H / 32;
  _Float16* xs = reinterpret_cast<_Float16*>(smem);                   // [M][H]
  float* sxs = reinterpret_cast<float*>(smem + (size_t)M * H * 2);     // [M][H/32]
  __shared__ uint32_t rowmax[MAXM];
  __shared__ int rowexp[MAXM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane / lpc, sl = lane % lpc;
  const int cpw = 64 / lpc;
  const int cpl = (nchunk + lpc - 1) / lpc;
  const int items = rounds * cpl;
  const int ng_g = H / p.gs_g, ng_u = H / p.gs_u;
  const int rw_g = H * BITS_G / 32, rw_u = H * BITS_U / 32;
  const int col0 = blockIdx.x * rounds * 4 * cpw;

  auto item_col = [&](int j) { return col0 + (j / cpl) * 4 * cpw + wave * cpw + sub; };
  auto item_chunk = [&](int j) { return sl + (j % cpl) * lpc; };

  RawChunk<BITS_G> cg, ng;
  RawChunk<BITS_U> cu, nu;
  auto load_item = [&](int j, RawChunk<BITS_G>& a, RawChunk<BITS_U>& b) {
    const int nn = min(item_col(j), p.I - 1);
    const int kc = min(item_chunk(j), nchunk - 1);
    load_chunk<BITS_G>(a, p.wg, p.sg, p.bg, nn, rw_g, ng_g, p.gs_g, kc);
    load_chunk<BITS_U>(b, p.wu, p.su, p.bu, nn, rw_u, ng_u, p.gs_u, kc);
  };
  load_item(0, cg, cu);     // weights first: in flight while x is staged

  // ---- stage x rows
  if (tid < MAXM) rowmax[tid] = 0;
  __syncthreads();
  const int nchunk8 = M * (H / 8);
  for (int c = tid; c < nchunk8; c += 256) {
    const int m = c / (H / 8), k8 = c % (H / 8);
    const u32x4 v = *reinterpret_cast<const u32x4*>(p.x + (int64_t)m * H + 8 * k8);
    uint32_t a = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) a = max(a, max(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
    atomicMax(&rowmax[m], a);
  }
  __syncthreads();
  if (tid < M) rowexp[tid] = row_exponent(rowmax[tid]);
  __syncthreads();
  for (int base = 0; base < nchunk8; base += 256) {
    const int c = base + tid;
    float part = 0.0f;
    if (c < nchunk8) {
      const int m = c / (H / 8), k8 = c % (H / 8);
      const int e = rowexp[m];
      const u32x4 v = *reinterpret_cast<const u32x4*>(p.x + (int64_t)m * H + 8 * k8);
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
      *reinterpret_cast<f16x8*>(xs + (size_t)m * H + 8 * k8) = h;
    }
    // four consecutive 8-value blocks (consecutive lanes) form one 32-input chunk
    part += __shfl_xor(part, 1);
    part += __shfl_xor(part, 2);
    if (c < nchunk8 && (c & 3) == 0) {
      const int m = c / (H / 8), k8 = c % (H / 8);
      sxs[(size_t)m * nchunk + k8 / 4] = part;
    }
  }
  __syncthreads();

  float ag[MAXM], au[MAXM];
#pragma unroll
  for (int m = 0; m < MAXM; ++m) {
    ag[m] = 0.0f;
    au[m] = 0.0f;
  }
  for (int j = 0; j < items; ++j) {
    if (j + 1 < items) load_item(j + 1, ng, nu);
    const int kc = item_chunk(j);
    if (kc < nchunk) {
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        if (m < M) {
          const uint32_t* xr = reinterpret_cast<const uint32_t*>(xs + (size_t)m * H + kc * 32);
          uint32_t xv[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4 t = *reinterpret_cast<const u32x4*>(xr + 4 * q);
            xv[4 * q] = t[0];
            xv[4 * q + 1] = t[1];
            xv[4 * q + 2] = t[2];
            xv[4 * q + 3] = t[3];
          }
          const float sx = sxs[(size_t)m * nchunk + kc];
          ag[m] += chunk_dot<BITS_G>(cg, xv, sx);
          au[m] += chunk_dot<BITS_U>(cu, xv, sx);
        }
      }
    }
    if (j % cpl == cpl - 1) {
      // end of a column: reduce over the group, write, reset
      const int n = item_col(j);
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        if (m < M) {
          float g = ag[m], u = au[m];
          for (int off = lpc >> 1; off > 0; off >>= 1) {
            g += __shfl_xor(g, off);
            u += __shfl_xor(u, off);
          }
          if (sl == 0 && n < p.I) store_out(p, m, n, ldexpf(g, rowexp[m]), ldexpf(u, rowexp[m]));
          ag[m] = 0.0f;
          au[m] = 0.0f;
        }
      }
    }
    cg = ng;
    cu = nu;
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

template <int BG, int BU, int CPL>
static hipError_t launch_gemv1_t(const GemvParams& p, int R, hipStream_t stream) {
  const int lpc = gemv_lanes_per_column(p.H);
  const int cpw = 64 / lpc;
  const int cols_per_wave = cpw * R;
  const int waves = (p.I + cols_per_wave - 1) / cols_per_wave;
  const int blocks = (waves + 3) / 4;
  switch (R) {
    case 1: hipLaunchKernelGGL((swq_gemv1_kernel<BG, BU, CPL, 1>), dim3(blocks), dim3(256), 0, stream, p, lpc); break;
    case 2: hipLaunchKernelGGL((swq_gemv1_kernel<BG, BU, CPL, 2>), dim3(blocks), dim3(256), 0, stream, p, lpc); break;
    case 4: hipLaunchKernelGGL((swq_gemv1_kernel<BG, BU, CPL, 4>), dim3(blocks), dim3(256), 0, stream, p, lpc); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BG, int BU, int MAXM>
static hipError_t launch_gemvm_t(const GemvParams& p, hipStream_t stream) {
  const int lpc = gemv_lanes_per_column(p.H);
  const int cpw = 64 / lpc;
  const int rounds = 2;
  const int cols_per_block = 4 * cpw * rounds;
  const int blocks = (p.I + cols_per_block - 1) / cols_per_block;
  const size_t lds = (size_t)gemv_lds_bytes(p.M, p.H);
  hipLaunchKernelGGL((swq_gemvm_kernel<BG, BU, MAXM>), dim3(blocks), dim3(256), lds, stream, p, lpc, rounds);
  return hipGetLastError();
}

static int gemv1_rounds() {
  static const int r = [] {
    const char* s = getenv("SWIGLU_Q_GEMV_ROUNDS");
    const int v = s ? atoi(s) : 0;
    return (v == 1 || v == 2 || v == 4) ? v : 2;
  }();
  return r;
}

template <int BG, int BU>
static hipError_t launch_gemv_bits(const GemvParams& p, hipStream_t stream) {
  const int lpc = gemv_lanes_per_column(p.H);
  const int cpl = (p.H / 32 + lpc - 1) / lpc;
  if (p.M == 1 && cpl <= 2 && !getenv("SWIGLU_Q_GEMV_GENERAL")) {
    if (cpl == 1) return launch_gemv1_t<BG, BU, 1>(p, gemv1_rounds(), stream);
    return launch_gemv1_t<BG, BU, 2>(p, gemv1_rounds(), stream);
  }
  if (p.M <= 1) return launch_gemvm_t<BG, BU, 1>(p, stream);
  if (p.M <= 2) return launch_gemvm_t<BG, BU, 2>(p, stream);
  if (p.M <= 4) return launch_gemvm_t<BG, BU, 4>(p, stream);
  if (p.M <= 8) return launch_gemvm_t<BG, BU, 8>(p, stream);
  if (p.M <= kGemvMaxM) return launch_gemvm_t<BG, BU, kGemvMaxM>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(const GemvParams& p, int bits_g, int bits_u, hipStream_t stream) {
  if (bits_g == 4 && bits_u == 4) return launch_gemv_bits<4, 4>(p, stream);
  if (bits_g == 8 && bits_u == 4) return launch_gemv_bits<8, 4>(p, stream);
  if (bits_g == 4 && bits_u == 8) return launch_gemv_bits<4, 8>(p, stream);
  if (bits_g == 8 && bits_u == 8) return launch_gemv_bits<8, 8>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace swq
