// Internal interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swq {

// Epilogue kinds of the quantized linear y = x W^T (after the precision modes
// 0..2 of the fused forward).  It runs on the same kernels with W's rows split
// in two, the first ceil(N/2) in the gate slot and the rest in the up slot; the
// epilogue stores both projections as they are, gate column n at n and up
// column n at I + n (I = ceil(N/2)), rounded to bf16 or as float32.
constexpr int kLinBf16 = 4, kLinF32 = 5;

// Row staging of x for the matrix-matrix path, and the extra-column rows
// that carry the per-group bias term.
struct PrepParams {
  const uint16_t* x;   // bf16 [M, H]
  const uint16_t* sg;  // scales and biases of both matrices (bf16 [I, H/gs])
  const uint16_t* bg;
  const uint16_t* su;
  const uint16_t* bu;
  int M, H, I;
  int I_u;             // rows of the up matrix: I, or fewer (the second half of a split linear weight)
  int gs_g, gs_u, bits_g, bits_u;
  int g0;              // min(gs_g, gs_u): granularity of the group sums
  int ldx;             // columns of x': H + kext (a multiple of 32)
  int kext;            // extra K columns: 3 per g0-group, padded to 32
  _Float16* xa;        // out: [ldx / 32][M][32], K-step major
  int* xexp;           // out: [M] row exponents e (x' = x * 2^-e)
  _Float16* bext_g;    // out: [I, kext] extra-column B rows of the gate (c_hi, c_lo, c_hi per group)
  _Float16* bext_u;    // out: same for the up matrix
  uint32_t* scl;       // out: scale tiles, see kScaleTileWords
  int nss;             // super-steps of 128 inputs: ceil(H / 128)
  int* kexp;           // out: [2][I] row exponents k of the gate and up rows (scales and constants
                       //      are stored times 2^-k; the sums are multiplied by 2^k)
  int k_only;          // 1: the column blocks write kexp only (no extra-column rows, no scale tiles)
  int xlane;           // 0: x' K-step major for the MFMA kernel (with the extra columns);
                       // 1 or 2: in the few-row kernel's lane order with that many 16-row tiles
                       // (see kSkinnyXUnit), no extra columns
  int act;             // kActBf16 or kActF16: the type of x, the scales and the biases (binary16:
                       // x' = x, e = 0; scale tiles hold (hi, lo) parts, split_scale)
};

// x' of the few-row kernel, in its MFMA lane order: for chunk quad Q (128
// inputs), row tile t (16 rows), 8-input block kb and lane l = 16 h + r, the
// 16 bytes x'[16 t + r][128 Q + 32 h + 8 kb .. + 8] at 16-byte unit
// ((Q * RT + t) * 4 + kb) * 64 + l: every load instruction of a wave reads
// one contiguous kilobyte.  Rows past M and inputs past H are never written
// and never read (the kernel masks them).
constexpr int kSkinnyXUnitsPerQuadTile = 4 * 64;

struct MfmaParams {
  const _Float16* xa;
  const int* xexp;
  const uint32_t* wg;
  const uint16_t* sg;
  const uint32_t* wu;
  const uint16_t* su;
  int M, H, I;
  int I_u;             // rows of the up matrix (I, or fewer for a split linear weight)
  int ldo;             // output row stride in elements (I, or N for the linear)
  int n_begin, n_end;  // output columns [n_begin, n_end) of this launch
  const uint32_t* scl; // scale tiles written by the prep kernel
  int nss;
  int gs_g, gs_u;
  int ldx, kext;
  const _Float16* bext_g;
  const _Float16* bext_u;
  const int* kexp;     // [2][I] row exponents of the gate and up rows, from the prep kernel
  int mode;
  void* out;
  float* dbg_g;        // non-null: write float32 gate/up instead of hidden
  float* dbg_u;
  const uint16_t* res; // the linear only: bf16 [M, ldo] added to its sums before the store, or null
  int vec;             // 1: the output rows allow 16-byte (f32) / 8-byte (bf16) stores of 4 features
  int act;             // kActBf16 or kActF16 (output type of modes 0 and 2, MATCH rounding)
  int kchunk;          // K split: code K-steps per split (a multiple of 4), else 0
};

struct GemvParams {
  const uint16_t* x;   // bf16 (or binary16, act) [M, H]
  const uint32_t* wg;
  const uint16_t* sg;
  const uint16_t* bg;
  const uint32_t* wu;
  const uint16_t* su;
  const uint16_t* bu;
  int M, H, I;
  int I_u;             // rows of the up matrix (I, or fewer for a split linear weight)
  int ldo;             // output row stride in elements (I, or N for the linear)
  int gs_g, gs_u;
  int mode;
  void* out;
  float* dbg_g;
  float* dbg_u;
  const uint16_t* res; // the linear only: bf16 [M, ldo] added to its sums before the store, or null
  const _Float16* xa;  // x' staged by the prep kernel in the few-row kernel's lane order, or null
  const int* xexp;     // and its row exponents
  const int* kexp;     // with xa: [2][I] weight-row exponents k from the prep kernel's column blocks
  int act;             // kActBf16 or kActF16: the type of x, the scales and biases, and the output
};

// Scale tiles: for every 128 output columns and every 128 inputs (a
// super-step of four K-steps of 32), the scale of each column's group in
// each K-step and matrix as a binary16 pair (s, s) -- binary16 scales: its
// two parts (hi, lo), see split_scale -- ordered
// [K-step q][matrix][column]: 4 * 2 * 128 words, one contiguous 4 KB block.
constexpr int kScaleTileCols = 128;
constexpr int kScaleTileWords = 4 * 2 * kScaleTileCols;

// Tile shapes of the MFMA kernel: rows, and columns per matrix.
constexpr int kMfmaConfigs = 2;
constexpr int kMfmaBM[kMfmaConfigs] = {256, 128};
constexpr int kMfmaBN[kMfmaConfigs] = {128, 128};

// Rows of one launch group of the few-row kernel (two 16-row MFMA tiles).
constexpr int kGemvMaxM = 32;
// ... the few-row kernel takes up to kGemvGroupsMaxM rows as row groups of
// kGemvMaxM (one grid row per group; x' and the weights read once per group)
constexpr int kGemvGroupsMaxM = 128;
// 16-row tiles of x' the prep kernel stages for the few-row kernel: one for
// M <= 16, else two per row group
inline int64_t gemv_x_tiles(int64_t M) { return M > 16 ? 2 * ((M + kGemvMaxM - 1) / kGemvMaxM) : 1; }
// Where the few-row kernel's x' comes from (skinny_x_source): the prep
// kernel (staged in the workspace), the block's own LDS (M*H up to
// kSkinnyStageMax), or each wave's own registers (a row fits one pass of the
// block's waves).  The last two need no workspace and no second launch.
constexpr int kXPrep = 0, kXStage = 1, kXSelf = 2;
constexpr int kSkinnyStageMax = 8192;
// kXSelf (M <= 16): each wave's LDS region in bytes -- its chunks' rows of x
// as loaded (64 bytes per chunk and row, written 1 KB per load instruction),
// later its partial sums (2 KB per column tile) -- for `nch` chunks per wave
// and `ct` column tiles per block; the block's regions together stay within
// kSkinnySelfMaxLds.
__host__ __device__ inline int skinny_self_region(int M, int nch, int ct = 1) {
  const int x = (nch * M + 15) / 16 * 1024;
  return x > 2048 * ct ? x : 2048 * ct;
}
constexpr int kSkinnySelfMaxLds = 65536;
// ... and with two row tiles (16 < M <= 32, one chunk quad per wave): 8 KB
// regions for up to 16 waves (the device allows 160 KB per block)
constexpr int kSkinnySelfRt2MaxLds = 131072;
// the matrix-vector kernel's several-row form (no staging pass): 2 <= M <=
// kGemv1MaxRows with a whole wave per column (H >= 2048) and at most two
// chunks per lane (H <= 4096); below H = 2048 the few-row kernel is faster
constexpr int kGemv1MaxRows = 4;
constexpr int kGemv1RowsMinH = 2048;
constexpr int kGemv1RowsMaxH = 4096;
bool gemv1_rows_enabled();
inline bool gemv1_rows_shape(int64_t M, int64_t H) {
  return M >= 2 && M <= kGemv1MaxRows && H >= kGemv1RowsMinH && H <= kGemv1RowsMaxH && gemv1_rows_enabled();
}

inline int kext_columns(int64_t H, int g0) {
  const int64_t c = 3 * (H / g0);
  return (int)((c + 31) / 32 * 32);
}

hipError_t launch_prep(const PrepParams& p, hipStream_t stream);
// The x rows of the prep kernel (x' and row exponents), and with k_only its
// weight rows' exponents, for the matrix-vector path.
hipError_t launch_prep_rows(const PrepParams& p, hipStream_t stream);
// cfg: tile shape (kMfmaBM/kMfmaBN); n_split > 0 with cfg 0: columns
// [0, n_split) as 256 x 128 tiles and [n_split, I) as 128 x 128 tiles, two launches.
// ksplit > 1: 128 x 128 tiles with the code K-steps split ksplit ways
// (p.kchunk each), the float32 sums of split k at dbg_g / dbg_u + k M ldo.
hipError_t launch_mfma(const MfmaParams& p, int cfg, int n_split, int ksplit, int bits_g, int bits_u,
                       hipStream_t stream);
// The K split's second pass: out = epilogue(sum over the splits) for p.mode
// (forward or linear), the splits' sums in [ksplit][M][p.I] planes.
hipError_t launch_ksplit_epilogue(const MfmaParams& p, const float* part_g, const float* part_u, int ksplit,
                                  hipStream_t stream);
hipError_t launch_gemv(const GemvParams& p, int bits_g, int bits_u, hipStream_t stream);
// the instances of one activation type (kActBf16 / kActF16), each compiled in
// its own translation unit
template <int ACT>
hipError_t launch_gemv_act(const GemvParams& p, int bits_g, int bits_u, hipStream_t stream);
// The few-row kernel's x source for a call of M rows (kXPrep, kXStage or kXSelf).
int skinny_x_source(int64_t M, int64_t H, int bits_g, int bits_u);
// compute units of the current device (cached per device)
int device_cus();
// Whether the few-row kernel, fed x' by the prep kernel, needs the weight-row
// exponents from the prep kernel's k-only rows (a row longer than one pass of
// its waves); otherwise it takes them from the scales its first pass loads.
bool skinny_needs_kexp(int M, int H, int bits_g, int bits_u);

}  // namespace swq
