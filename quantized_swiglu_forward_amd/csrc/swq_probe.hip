// Measurement yardsticks for the benchmark (libswq_probe.so): not part of the
// forward's path, and nothing in libswiglu_q.so calls them.
//
//  * swq_probe_mfma_f16: the sustained rate of back-to-back
//    v_mfma_f32_32x32x16_f16 on this GPU.  Dense f16 MFMA is power limited
//    here, so the rate depends on the operand bits; pattern 0 fills both
//    operands with random binary16 values of full 11-bit precision, pattern 1
//    with operands shaped like the fused kernel's (A: x' with a full
//    significand in [1, 2) and random sign; B: s (q - 8) with an 8-bit
//    significand scale and random 4-bit codes).
//  * swq_probe_read: a read-only stream of `bytes` bytes with 16-byte
//    nontemporal loads, every load issued before any arithmetic, one store
//    per block: the cost of reading a decode call's weight bytes once, which
//    the matrix-vector kernel cannot beat.
//
//  * swq_probe_empty, swq_probe_grid_barrier, swq_probe_atomic_add,
//    swq_probe_read_slices: the parts a whole MLP in one dispatch would pay
//    at decode -- the launch it saves (a trivial kernel), a grid-wide barrier
//    between its two phases, f32 atomic accumulation of every I-block's
//    partial output, and reads of the down projection's rows in the I-slices
//    the blocks of the first phase own.
//
// All return 0, or -1 when the launch fails (or the arguments are invalid).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t mix(uint32_t v) {   // integer hash (xorshift-multiply)
  v ^= v >> 16;
  v *= 0x7feb352dU;
  v ^= v >> 15;
  v *= 0x846ca68bU;
  v ^= v >> 16;
  return v;
}

__device__ __forceinline__ _Float16 rand_f16(uint32_t h, int pattern, bool a_side) {
  if (pattern == 0) {                                   // full significand, exponent in [-1, 1]
    const uint16_t bits = (uint16_t)(((h & 1) << 15) | ((14 + (h >> 1) % 3) << 10) | ((h >> 4) & 0x3FF));
    return __builtin_bit_cast(_Float16, bits);
  }
  if (a_side) {                                         // x': [1, 2), full significand, random sign
    const uint16_t bits = (uint16_t)(((h & 1) << 15) | (15 << 10) | ((h >> 4) & 0x3FF));
    return __builtin_bit_cast(_Float16, bits);
  }
  // s (q - 8): scale with an 8-bit significand near 2^11, code 0..15
  const float s = 2048.0f * (1.0f + (float)((h >> 8) & 0x7F) / 128.0f);
  return (_Float16)(s * (float)((int)(h & 15) - 8) / 4096.0f);
}

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, int pattern, float* sink) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  f16x8 a[2], b[2];
#pragma unroll
  for (int v = 0; v < 2; ++v)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[v][j] = rand_f16(mix(t * 64u + v * 16u + j), pattern, true);
      b[v][j] = rand_f16(mix(t * 64u + v * 16u + 8u + j + 0x9E3779B9u), pattern, false);
    }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[c & 1], b[c >> 1], acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[t] = s;
}

constexpr int kReadPerThread = 2;   // 16-byte pieces per thread (1 and 2 measured fastest, 4 slower)

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* src, int64_t pieces, float* sink) {
  const int64_t base = (int64_t)blockIdx.x * 256 * kReadPerThread + threadIdx.x;
  u32x4 v[kReadPerThread];
#pragma unroll
  for (int i = 0; i < kReadPerThread; ++i) {
    const int64_t at = base + (int64_t)i * 256;
    v[i] = at < pieces ? __builtin_nontemporal_load(src + at) : (u32x4){0, 0, 0, 0};
  }
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < kReadPerThread; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
  // one value per block leaves the kernel (so the loads are kept)
  x ^= __shfl_xor(x, 1);
  x ^= __shfl_xor(x, 2);
  x ^= __shfl_xor(x, 4);
  if (threadIdx.x == 0) sink[blockIdx.x] = (float)(x & 0xFFFF);
}

__global__ __launch_bounds__(64) void probe_empty_kernel(float* sink) {
  if (threadIdx.x == 0) sink[blockIdx.x] = (float)blockIdx.x;
}

// Every block arrives once (ticket = its position in the arrivals so far,
// over every launch), then waits until the whole launch has arrived: the
// counter never resets, so each launch waits for the next multiple of
// `blocks`.  The wait gives up after max_spin polls and records that in the
// block's sink slot (1), so the kernel ends whether or not every block of a
// launch is resident.
__global__ __launch_bounds__(256) void probe_grid_barrier_kernel(unsigned* counter, unsigned blocks, int max_spin,
                                                                 float* sink) {
  __shared__ int timed_out;
  if (threadIdx.x == 0) {
    const unsigned ticket = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned target = (ticket / blocks + 1u) * blocks;
    int spin = 0;
    while ((int)(__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - target) < 0 &&
           spin < max_spin)
      ++spin;
    timed_out = spin >= max_spin;
  }
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = (float)timed_out;
}

// blocks x n f32 atomic adds: block b adds (b + 1) to each of y[0..n).
__global__ __launch_bounds__(256) void probe_atomic_add_kernel(float* y, int n) {
  const float v = (float)(blockIdx.x + 1);
  for (int j = threadIdx.x; j < n; j += 256) __hip_atomic_fetch_add(y + j, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block b reads bytes [b piece, (b + 1) piece) of every one of `rows` rows
// of row_bytes (piece: 8 or 16 bytes, one load per row), threads over rows.
__global__ __launch_bounds__(256) void probe_read_slices_kernel(const unsigned char* src, int rows, int row_bytes,
                                                                int piece, float* sink) {
  uint32_t x = 0;
  for (int r = threadIdx.x; r < rows; r += 256) {
    const unsigned char* at = src + (int64_t)r * row_bytes + (int64_t)blockIdx.x * piece;
    if (piece == 16) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(at));
      x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    } else {
      const uint64_t v = __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(at));
      x ^= (uint32_t)v ^ (uint32_t)(v >> 32);
    }
  }
  x ^= __shfl_xor(x, 1);
  x ^= __shfl_xor(x, 2);
  if (threadIdx.x == 0) sink[blockIdx.x] = (float)(x & 0xFFFF);
}

}  // namespace

extern "C" {

// blocks x 256 threads, each wave `iters` x 4 MFMAs (32 x 32 x 16 f16); sink:
// float32 [blocks * 256] device buffer.  Work: blocks * 4 * iters * 4 * 32768 flops.
int swq_probe_mfma_f16(int blocks, int iters, int pattern, float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0 || !sink) return -1;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, pattern, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Read `bytes` (a multiple of 16, src 16-byte aligned) once; sink: float32
// [swq_probe_read_blocks(bytes)] device buffer.
int64_t swq_probe_read_blocks(int64_t bytes) { return (bytes / 16 + 256 * kReadPerThread - 1) / (256 * kReadPerThread); }

int swq_probe_read(const void* src, int64_t bytes, float* sink, void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 || ((uintptr_t)src & 15)) return -1;
  const int64_t blocks = swq_probe_read_blocks(bytes);
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// One trivial block per `blocks`; sink: float32 [blocks].
int swq_probe_empty(int blocks, float* sink, void* stream) {
  if (blocks <= 0 || !sink) return -1;
  hipLaunchKernelGGL(probe_empty_kernel, dim3(blocks), dim3(64), 0, (hipStream_t)stream, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// counter: one uint32 in device memory, zero before the first launch and
// never written by the host afterwards; sink: float32 [blocks] (1 where a
// block gave up waiting after max_spin polls).
int swq_probe_grid_barrier(int blocks, unsigned* counter, int max_spin, float* sink, void* stream) {
  if (blocks <= 0 || !counter || !sink || max_spin <= 0) return -1;
  hipLaunchKernelGGL(probe_grid_barrier_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, counter,
                     (unsigned)blocks, max_spin, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// y: float32 [n] device buffer.
int swq_probe_atomic_add(int blocks, int n, float* y, void* stream) {
  if (blocks <= 0 || n <= 0 || !y) return -1;
  hipLaunchKernelGGL(probe_atomic_add_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, y, n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// src: rows x row_bytes (16-byte aligned rows), blocks * piece <= row_bytes,
// piece 8 or 16; sink: float32 [blocks].
int swq_probe_read_slices(const void* src, int rows, int row_bytes, int piece, int blocks, float* sink,
                          void* stream) {
  if (!src || !sink || rows <= 0 || blocks <= 0 || (piece != 8 && piece != 16) || row_bytes % 16 ||
      ((uintptr_t)src & 15) || (int64_t)blocks * piece > row_bytes)
    return -1;
  hipLaunchKernelGGL(probe_read_slices_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const unsigned char*)src, rows, row_bytes, piece, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
