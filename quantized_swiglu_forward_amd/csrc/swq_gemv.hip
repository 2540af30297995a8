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
// The block first stages its x rows in LDS as x' = x * 2^-e (e = exponent of
// the row maximum; the product is exact) in binary16 and the
// [0,4,1,5,2,6,3,7] order of the code pairs, plus one float32 sum per
// 32-input chunk.
#include "swq_device.h"
#include "swq_kernels.h"

namespace swq {

template <int BITS_G, int BITS_U, int MAXM>
__global__ __launch_bounds__(256) void swq_gemv_kernel(GemvParams p, int lpc, int cols_per_block) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int H = p.H, M = p.M;
  const int nchunk32 = H / 32;
  _Float16* xs = reinterpret_cast<_Float16*>(smem);                           // [M][H]
  float* sxs = reinterpret_cast<float*>(smem + (size_t)M * H * 2);             // [M][H/32]
  __shared__ uint32_t rowmax[MAXM];
  __shared__ int rowexp[MAXM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- stage x rows
  if (tid < MAXM) rowmax[tid] = 0;
  __syncthreads();
  const int nchunk8 = M * (H / 8);
  for (int c = tid; c < nchunk8; c += 256) {
    const int m = c / (H / 8), kc = c % (H / 8);
    const u32x4 v = *reinterpret_cast<const u32x4*>(p.x + (int64_t)m * H + 8 * kc);
    uint32_t a = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) a = max(a, max(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
    atomicMax(&rowmax[m], a);
  }
  __syncthreads();
  if (tid < M) {
    const uint32_t a = rowmax[tid];
    const int field = (int)(a >> 7);
    rowexp[tid] = (a == 0) ? 0 : ((field == 0) ? -127 : field - 127);
  }
  __syncthreads();
  for (int base = 0; base < nchunk8; base += 256) {
    const int c = base + tid;
    float part = 0.0f;
    if (c < nchunk8) {
      const int m = c / (H / 8), kc = c % (H / 8);
      const int e = rowexp[m];
      const u32x4 v = *reinterpret_cast<const u32x4*>(p.x + (int64_t)m * H + 8 * kc);
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
      *reinterpret_cast<f16x8*>(xs + (size_t)m * H + 8 * kc) = h;
    }
    // four consecutive 8-chunks (consecutive lanes) form one 32-chunk
    part += __shfl_xor(part, 1);
    part += __shfl_xor(part, 2);
    if (c < nchunk8 && (c & 3) == 0) {
      const int m = c / (H / 8), kc = c % (H / 8);
      sxs[(size_t)m * nchunk32 + kc / 4] = part;
    }
  }
  __syncthreads();

  // ---- columns: each group of lpc lanes owns one column at a time
  const int sub = lane / lpc;          // column slot inside the wave
  const int sl = lane % lpc;           // lane inside the column group
  const int cpw = 64 / lpc;
  const int ng_g = H / p.gs_g, ng_u = H / p.gs_u;
  const int rw_g = H * BITS_G / 32, rw_u = H * BITS_U / 32;
  const float zg = CodeOffset<BITS_G>::z, zu = CodeOffset<BITS_U>::z;
  const int col0 = blockIdx.x * cols_per_block;

  for (int slot = wave * cpw + sub; slot < cols_per_block; slot += 4 * cpw) {
    const int n = col0 + slot;
    const bool valid = n < p.I;
    const int nn = valid ? n : p.I - 1;
    float ag[MAXM], au[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      ag[m] = 0.0f;
      au[m] = 0.0f;
    }
    for (int kc = sl; kc < nchunk32; kc += lpc) {
      const int k0 = kc * 32;
      // gate codes -> (q-8) pairs; 8-bit codes split into two planes
      uint32_t qg[BITS_G == 8 ? 32 : 16];
      if (BITS_G == 4) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p.wg + (int64_t)nn * rw_g + kc * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) codes4(w[j], &qg[4 * j]);
      } else {
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(p.wg + (int64_t)nn * rw_g + kc * 8);
        const u32x4 w1 = *reinterpret_cast<const u32x4*>(p.wg + (int64_t)nn * rw_g + kc * 8 + 4);
        codes8(w0[0], w0[1], &qg[0], &qg[16]);
        codes8(w0[2], w0[3], &qg[4], &qg[20]);
        codes8(w1[0], w1[1], &qg[8], &qg[24]);
        codes8(w1[2], w1[3], &qg[12], &qg[28]);
      }
      uint32_t qu[BITS_U == 8 ? 32 : 16];
      if (BITS_U == 4) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p.wu + (int64_t)nn * rw_u + kc * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) codes4(w[j], &qu[4 * j]);
      } else {
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(p.wu + (int64_t)nn * rw_u + kc * 8);
        const u32x4 w1 = *reinterpret_cast<const u32x4*>(p.wu + (int64_t)nn * rw_u + kc * 8 + 4);
        codes8(w0[0], w0[1], &qu[0], &qu[16]);
        codes8(w0[2], w0[3], &qu[4], &qu[20]);
        codes8(w1[0], w1[1], &qu[8], &qu[24]);
        codes8(w1[2], w1[3], &qu[12], &qu[28]);
      }
      const int gg = k0 / p.gs_g, gu = k0 / p.gs_u;
      const float s_g = bf16_to_f32(p.sg[(int64_t)nn * ng_g + gg]);
      const float b_g = bf16_to_f32(p.bg[(int64_t)nn * ng_g + gg]);
      const float s_u = bf16_to_f32(p.su[(int64_t)nn * ng_u + gu]);
      const float b_u = bf16_to_f32(p.bu[(int64_t)nn * ng_u + gu]);
      const float c_g = fmaf(zg, s_g, b_g);   // exact for bf16 s, b in range
      const float c_u = fmaf(zu, s_u, b_u);
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        if (m < M) {
          const uint32_t* xr = reinterpret_cast<const uint32_t*>(xs + (size_t)m * H + k0);
          uint32_t xv[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4 t = *reinterpret_cast<const u32x4*>(xr + 4 * q);
            xv[4 * q] = t[0];
            xv[4 * q + 1] = t[1];
            xv[4 * q + 2] = t[2];
            xv[4 * q + 3] = t[3];
          }
          const float sx = sxs[(size_t)m * nchunk32 + kc];
          float pg = 0.0f, pu = 0.0f;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            pg = __builtin_amdgcn_fdot2(as_h2(xv[j]), as_h2(qg[j]), pg, false);
            pu = __builtin_amdgcn_fdot2(as_h2(xv[j]), as_h2(qu[j]), pu, false);
          }
          if (BITS_G == 8) {
            float ph = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) ph = __builtin_amdgcn_fdot2(as_h2(xv[j]), as_h2(qg[16 + j]), ph, false);
            pg = fmaf(16.0f, ph, pg);
          }
          if (BITS_U == 8) {
            float ph = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) ph = __builtin_amdgcn_fdot2(as_h2(xv[j]), as_h2(qu[16 + j]), ph, false);
            pu = fmaf(16.0f, ph, pu);
          }
          ag[m] = fmaf(s_g, pg, fmaf(c_g, sx, ag[m]));
          au[m] = fmaf(s_u, pu, fmaf(c_u, sx, au[m]));
        }
      }
    }
    // reduce over the lpc lanes of the column group (aligned power-of-two block)
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      if (m < M) {
        for (int off = lpc >> 1; off > 0; off >>= 1) {
          ag[m] += __shfl_xor(ag[m], off);
          au[m] += __shfl_xor(au[m], off);
        }
      }
    }
    if (valid && sl == 0) {
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        if (m < M) {
          const float g = ldexpf(ag[m], rowexp[m]);
          const float u = ldexpf(au[m], rowexp[m]);
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
      }
    }
  }
}

// lanes per column: one 32-input chunk per lane, at most a wavefront
static int gemv_lanes_per_column(int H) {
  const int chunks = H / 32;
  int l = 1;
  while (l * 2 <= chunks && l * 2 <= 64) l *= 2;
  return l;
}

template <int BG, int BU, int MAXM>
static hipError_t launch_gemv_t(const GemvParams& p, hipStream_t stream) {
  const int lpc = gemv_lanes_per_column(p.H);
  const int cpw = 64 / lpc;
  const int cols_per_block = 4 * cpw * 2;   // two rounds per wave
  const int blocks = (p.I + cols_per_block - 1) / cols_per_block;
  const size_t lds = (size_t)gemv_lds_bytes(p.M, p.H);
  hipLaunchKernelGGL((swq_gemv_kernel<BG, BU, MAXM>), dim3(blocks), dim3(256), lds, stream, p, lpc,
                     cols_per_block);
  return hipGetLastError();
}

template <int BG, int BU>
static hipError_t launch_gemv_bits(const GemvParams& p, hipStream_t stream) {
  if (p.M <= 1) return launch_gemv_t<BG, BU, 1>(p, stream);
  if (p.M <= 2) return launch_gemv_t<BG, BU, 2>(p, stream);
  if (p.M <= 4) return launch_gemv_t<BG, BU, 4>(p, stream);
  if (p.M <= 8) return launch_gemv_t<BG, BU, 8>(p, stream);
  if (p.M <= kGemvMaxM) return launch_gemv_t<BG, BU, kGemvMaxM>(p, stream);
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
