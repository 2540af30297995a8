// C-ABI boundary of the fused quantized SwiGLU library (declared in
// include/swiglu_q.h): argument validation, the M-threshold dispatcher,
// per-path call counters, and the per-(device, stream) workspace (x' and
// the matrix-matrix path's staging).
//
// The dispatcher mirrors the pages' M threshold ("mlx-bun 0.0.7 -> 0.0.9"
// diff, page 42, fused-swiglu-kernel.ts: below a small row count the
// projections are matrix-vector products and a different path runs; the
// threshold defaults to 2 there, benchmarks are to set it, and it can be set
// from the environment) and the support predicate of the same file (bf16
// activations, affine biases, 2-, 4- or 8-bit codes, group size a multiple
// of 32, H a multiple of 32).  Here the default is 65, or 33 for wide
// weights (H * I >= 3 * 2^23 with I >= 4096), or 129 for small ones
// (H * I <= 2^23).  Measured on this GPU, the
// matrix-vector kernels beat the matrix-matrix kernel for every M <= 32 on
// every weight shape measured (2-3x on the decode and prefill weight shapes
// for M <= 16).  With two row groups of 32 (33 <= M <= 64) they are faster
// on weights up to 2^24 elements (17-67 %) and on fewer than 4096 columns.
// On wide weights they are 24-66 % slower than the matrix-matrix kernel with
// its K split.  The few-row kernel takes at most 128 rows (four
// groups).  A threshold set by API or environment applies to every shape.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>
#include <vector>

#include "../../include/swiglu_q.h"
#include "swq_device.h"
#include "swq_kernels.h"

using namespace swq;

// Compute units of the current device (cached per device).
int swq::device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  cache[dev] = cus;
  return cus;
}

namespace {

// Default M thresholds: the matrix-vector path up to two row groups (M <= 64),
// or up to one (M <= 32) for wide weights (H * I >= 3 * 2^23 and I >= 4096),
// where the MFMA path with its K split is faster from 33 rows on.  With
// fewer columns its split blocks do not fill the chip (a linear of 2048
// columns per slot and K = 14336: 57.5 against 41.5 us at M = 48).
// Small weights (H * I <= 2^23) keep the matrix-vector path up to its 128
// rows (H = 1024, I = 4096: 15.6 against 25.6 us at M = 128).
constexpr int kDefaultThreshold = 2 * kGemvMaxM + 1;
constexpr int kDefaultThresholdWide = kGemvMaxM + 1;
constexpr int kDefaultThresholdSmall = kGemvGroupsMaxM + 1;
constexpr int64_t kSmallWeights = int64_t(1) << 23;
constexpr int64_t kWideWeights = int64_t(3) << 23;
constexpr int64_t kWideColumns = 4096;

std::atomic<int> g_threshold{-1};
std::atomic<uint64_t> g_calls[2];
// Call cap (<0: none; -2: not yet read from the environment)
std::atomic<int64_t> g_max_calls{-2};

int64_t max_calls_now() {
  int64_t v = g_max_calls.load();
  if (v != -2) return v;
  v = -1;
  if (const char* s = getenv("SWIGLU_Q_MAXCALLS")) {
    char* end = nullptr;
    const long long t = strtoll(s, &end, 10);
    if (end != s && t >= 0) v = t;
  }
  int64_t expected = -2;
  g_max_calls.compare_exchange_strong(expected, v);
  return g_max_calls.load();
}
std::mutex g_ws_mutex;

struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
// slot 0: the kernels' own staging; slot 1: the whole MLP's hidden tensor
std::map<std::tuple<int, uintptr_t, int>, Workspace> g_ws;
// Buffers replaced by a larger one.  They stay allocated until
// swiglu_q_release_workspace(): work already queued on the stream, and HIP
// graphs captured while they were current, may still read and write them.
std::vector<std::pair<int, void*>> g_retired;

// The threshold set by swiglu_q_set_m_threshold, else by SWIGLU_Q_MMIN (read
// once), else -1 (the default rule).
int explicit_threshold() {
  const int t = g_threshold.load(std::memory_order_relaxed);
  if (t >= 0) return t;
  static const int env = [] {
    if (const char* s = getenv("SWIGLU_Q_MMIN")) {
      char* end = nullptr;
      long v = strtol(s, &end, 10);
      if (end != s && v > 0 && v < (1L << 30)) return (int)v;
    }
    return -1;
  }();
  return env;
}

// The threshold for weights of H x I.
int threshold_for(int64_t H, int64_t I) {
  const int t = explicit_threshold();
  if (t >= 0) return t;
  if (H * I <= kSmallWeights) return kDefaultThresholdSmall;
  return (H * I >= kWideWeights && I >= kWideColumns) ? kDefaultThresholdWide : kDefaultThreshold;
}

bool logging() {
  static const bool on = [] {
    const char* s = getenv("SWIGLU_Q_LOG");
    return s && s[0] == '1';
  }();
  return on;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool spec_ok(int bits, int gs) {
  return (bits == 2 || bits == 4 || bits == 8) && (gs == 32 || gs == 64 || gs == 128);
}

// Validation shared by every entry point; nothing touches HIP here.  With
// has_x false, x is library-owned (the whole MLP's hidden tensor) and not checked.
int validate(const void* x, const uint32_t* Wg, const void* sg, const void* bg, const uint32_t* Wu,
             const void* su, const void* bu, int64_t M, int64_t H, int64_t I, int bits_g, int gs_g,
             int bits_u, int gs_u, bool has_x = true) {
  if ((has_x && !x) || !Wg || !sg || !bg || !Wu || !su || !bu) return SWQ_ERR_NULL;
  if (!spec_ok(bits_g, gs_g) || !spec_ok(bits_u, gs_u)) return SWQ_ERR_UNSUPPORTED;
  if (M < 0 || H <= 0 || I <= 0) return SWQ_ERR_SHAPE;
  if (H % 32 != 0 || H % gs_g != 0 || H % gs_u != 0) return SWQ_ERR_SHAPE;
  // kernels index rows, columns and tiles with 32-bit counters, and address a
  // block's rows of x' and of the weights with 32-bit buffer offsets
  if (M > (1LL << 30) || H > (1LL << 20) || I > (1LL << 30)) return SWQ_ERR_SHAPE;
  if (((M + 127) / 128) * ((I + 127) / 128) >= (1LL << 31)) return SWQ_ERR_SHAPE;
  // the staged x' ([H + extra columns] x M binary16) is addressed with 32-bit byte offsets
  if (M * (H + kext_columns(H, gs_g < gs_u ? gs_g : gs_u)) * 2 >= (1LL << 32)) return SWQ_ERR_SHAPE;
  if ((has_x && !aligned(x, 16)) || !aligned(Wg, 16) || !aligned(Wu, 16)) return SWQ_ERR_ALIGN;
  if (!aligned(sg, 2) || !aligned(bg, 2) || !aligned(su, 2) || !aligned(bu, 2)) return SWQ_ERR_ALIGN;
  return SWQ_OK;
}

bool gemv_fits(int64_t M, int64_t H);

// The dispatcher's rule.
int auto_path(int64_t M, int64_t H, int64_t I) {
  return (M < threshold_for(H, I) && gemv_fits(M, H)) ? SWQ_PATH_GEMV : SWQ_PATH_MFMA;
}

bool gemv_fits(int64_t M, int64_t H) {
  (void)H;
  return M >= 1 && M <= kGemvGroupsMaxM;
}

// The matrix-vector kernel reads x itself (M = 1 with H <= 8192, and its
// several-row form), and the few-row kernel converts x itself where
// skinny_x_source says so; otherwise the prep kernel stages x' first (in the
// workspace).
bool gemv_needs_rows(int64_t M, int64_t H, int bits_g, int bits_u) {
  if (M == 1 && H <= 8192) return false;
  if (gemv1_rows_shape(M, H)) return false;
  return skinny_x_source(M, H, bits_g, bits_u) == kXPrep;
}

// Tile shape of the MFMA kernel: 256 x 128 unless that leaves CUs idle
// (fewer than two tiles per CU of the 256), then 128 x 128.  The environment
// variable SWIGLU_Q_MFMA_CFG (0 .. kMfmaConfigs-1) overrides the choice.
int choose_mfma_config(int64_t M, int64_t I) {
  if (const char* s = getenv("SWIGLU_Q_MFMA_CFG")) {
    char* end = nullptr;
    const long v = strtol(s, &end, 10);
    if (end != s && v >= 0 && v < kMfmaConfigs) return (int)v;
  }
  const int64_t tiles256 = ((M + 255) / 256) * ((I + 127) / 128);
  return tiles256 >= 512 ? 0 : 1;
}

// With 256 x 128 tiles (one per CU at a time), a partly filled last round
// leaves CUs idle for a whole tile time.  The columns past the last whole
// round then go to a second launch of 128 x 128 tiles when that is at most
// one round of them.  Returns the first column of the second launch, or 0
// for a single launch.  SWIGLU_Q_MFMA_SPLIT=0 turns this off.
int choose_column_split(int64_t M, int64_t I, int cfg, int bits_g, int bits_u) {
  if (cfg != 0 || (bits_g == 8 && bits_u == 8)) return 0;
  if (const char* s = getenv("SWIGLU_Q_MFMA_SPLIT"); s && s[0] == '0') return 0;
  const int64_t cus = device_cus();
  const int64_t mt = (M + 255) / 256, nt = (I + 127) / 128;
  const int64_t full = mt * nt / cus;
  if (full == 0 || mt * nt == full * cus) return 0;
  const int64_t nt1 = full * cus / mt;
  if (nt1 <= 0 || nt1 >= nt) return 0;
  const int64_t rest = ((M + 127) / 128) * ((I - 128 * nt1 + 127) / 128);
  if (rest > cus) return 0;
  return (int)(128 * nt1);
}

// K split of the MFMA path: with few 128 x 128 tiles (at most half the CUs)
// and H >= 2048, each tile's code K-steps are split across blocks in whole
// super-steps (at least four per split), up to 8 ways, 16 from H = 8192 on
// (more than two only while their float32 partial sums stay below 32 MB); a second kernel adds the splits in order and runs
// the epilogue.  Shorter splits, or more partial sums, measured slower (at
// H = 1024 the split loses from M = 128 on).  Forward
// precision modes only.  SWIGLU_Q_MFMA_KSPLIT=n caps the splits at n (0 or 1:
// no split).
struct KSplit {
  int n = 1;       // splits (1: none)
  int chunk = 0;   // code K-steps per split
};
KSplit choose_ksplit(int64_t M, int64_t H, int64_t I, int cfg, int n_split) {
  KSplit k;
  const int64_t steps = H / 32;
  int64_t cap = steps >= 256 ? 16 : 8;
  if (const char* s = getenv("SWIGLU_Q_MFMA_KSPLIT"); s && *s) cap = std::min<int64_t>(cap, atol(s));
  if (cap < 2 || cfg != 1 || n_split != 0 || M <= 0 || I <= 0) return k;
  const int64_t cus = device_cus();
  const int64_t tiles = ((M + 127) / 128) * ((I + 127) / 128);
  if (2 * tiles > cus || steps < 64) return k;
  int64_t n = std::min<int64_t>(std::min<int64_t>(cus / tiles, steps / 16), cap);
  while (n > 2 && n * 2 * M * I * 4 >= (int64_t(32) << 20)) --n;
  if (n < 2) return k;
  const int64_t chunk = ((steps + n - 1) / n + 3) / 4 * 4;
  const int64_t nn = (steps + chunk - 1) / chunk;
  if (nn < 2) return k;
  k.n = (int)nn;
  k.chunk = (int)chunk;
  return k;
}

// Workspace of the matrix-matrix path, in order: x' rows [M, H + kext]
// (binary16), row exponents [M] (int32), the extra-column B rows [I, kext]
// (binary16) of the gate and of the up matrix, the scale tiles (4 KB per
// 128 columns and 128 inputs), then the weight rows' exponents k [2][I] (int32).
struct WsLayout {
  int64_t xa, xexp, eg, eu, sc, kx, part, total;
};

int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

WsLayout ws_layout(int64_t M, int64_t H, int64_t I, int bits_g, int gs_g, int bits_u, int gs_u) {
  const int64_t kext = kext_columns(H, gs_g < gs_u ? gs_g : gs_u);
  const int64_t plane = align256(I * kext * 2);
  WsLayout w;
  w.xa = 0;
  w.xexp = align256(M * (H + kext) * 2);
  w.eg = w.xexp + align256(M * 4);
  w.eu = w.eg + plane;
  w.sc = w.eu + plane;
  const int64_t tiles = (I + kScaleTileCols - 1) / kScaleTileCols * ((H + 127) / 128);
  w.kx = w.sc + align256(tiles * kScaleTileWords * 4);
  w.part = w.kx + align256(2 * I * 4);
  // the K split's float32 partial sums (gate, up) per split, when it applies
  const int cfg = choose_mfma_config(M, I);
  const KSplit ks = choose_ksplit(M, H, I, cfg, choose_column_split(M, I, cfg, bits_g, bits_u));
  w.total = w.part + (ks.n > 1 ? align256(2 * (int64_t)ks.n * M * I * 4) : 0);
  return w;
}

int get_workspace(hipStream_t stream, size_t need, void** out, int slot = 0) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SWQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& w = g_ws[{dev, (uintptr_t)stream, slot}];
  if (w.bytes < need) {
    // at least double, so that a sequence of growing calls retires a bounded
    // total (under the size of the last buffer); no synchronisation: the old
    // buffer is retired, not freed
    const size_t grain = 2u << 20;
    const size_t want = need > 2 * w.bytes ? need : 2 * w.bytes;
    const size_t bytes = (want + grain - 1) / grain * grain;
    void* fresh = nullptr;
    if (hipMalloc(&fresh, bytes) != hipSuccess) {
      (void)hipGetLastError();
      return SWQ_ERR_WORKSPACE;
    }
    if (w.ptr) g_retired.emplace_back(dev, w.ptr);
    w.ptr = fresh;
    w.bytes = bytes;
  }
  *out = w.ptr;
  return SWQ_OK;
}

// Staging of the matrix-vector path when the prep kernel stages x' (x' in the
// few-row kernel's lane order: 4 KB per chunk quad and 16-row tile, two
// tiles per row group past 16 rows; the row exponents; then the weight
// rows' exponents k [2][I]).
int64_t gemv_x_bytes(int64_t M, int64_t H) {
  return align256(((H + 127) / 128) * gemv_x_tiles(M) * kSkinnyXUnitsPerQuadTile * 16);
}
int64_t gemv_stage_bytes(int64_t M, int64_t H, int64_t I) {
  return gemv_x_bytes(M, H) + align256(M * 4) + align256(2 * I * 4);
}

// Device staging bytes of a call that takes `path` (0: none).
int64_t staging_bytes(int64_t M, int64_t H, int64_t I, int bits_g, int gs_g, int bits_u, int gs_u, int path) {
  if (M <= 0) return 0;
  if (path == SWQ_PATH_GEMV) return gemv_needs_rows(M, H, bits_g, bits_u) ? gemv_stage_bytes(M, H, I) : 0;
  return ws_layout(M, H, I, bits_g, gs_g, bits_u, gs_u).total;
}

// The staging buffer of a call: the caller's fixed one (fixed != null; it
// must hold `need` bytes) or the library's per-(device, stream) workspace.
int acquire(hipStream_t stream, size_t need, void** out, void* fixed, size_t fixed_bytes) {
  if (fixed) {
    if (need > fixed_bytes) return SWQ_ERR_TOO_LARGE;
    *out = fixed;
    return SWQ_OK;
  }
  return get_workspace(stream, need, out);
}

// I_u: rows of the up matrix (I, or fewer for the linear's split weight);
// ldo: output row stride in elements (I, or N for the linear); res: the
// linear's residual (bf16 [M, ldo]) or null; fixed: a caller-chosen staging
// buffer of fixed_bytes (null: the library's workspace).
int run(const void* x, const uint32_t* Wg, const void* sg, const void* bg, const uint32_t* Wu,
        const void* su, const void* bu, int64_t M, int64_t H, int64_t I, int64_t I_u, int64_t ldo,
        int bits_g, int gs_g, int bits_u, int gs_u, int mode, void* out, float* dbg_g, float* dbg_u,
        const void* res, int path, void* stream_v, void* fixed = nullptr, size_t fixed_bytes = 0,
        int act = kActBf16) {
  hipStream_t stream = (hipStream_t)stream_v;
  if (M == 0) return SWQ_OK;
  if (path == SWQ_PATH_AUTO) {
    path = auto_path(M, H, I);
  }
  if (path == SWQ_PATH_GEMV && !gemv_fits(M, H)) return SWQ_ERR_UNSUPPORTED;

  if (path == SWQ_PATH_GEMV) {
    GemvParams p;
    p.x = (const uint16_t*)x;
    p.wg = Wg; p.sg = (const uint16_t*)sg; p.bg = (const uint16_t*)bg;
    p.wu = Wu; p.su = (const uint16_t*)su; p.bu = (const uint16_t*)bu;
    p.M = (int)M; p.H = (int)H; p.I = (int)I;
    p.I_u = (int)I_u; p.ldo = (int)ldo;
    p.gs_g = gs_g; p.gs_u = gs_u; p.mode = mode;
    p.out = out; p.dbg_g = dbg_g; p.dbg_u = dbg_u; p.res = (const uint16_t*)res;
    p.xa = nullptr; p.xexp = nullptr; p.kexp = nullptr;
    p.act = act;
    if (logging())
      fprintf(stderr, "[swiglu_q] gemv M=%lld H=%lld I=%lld bits %d/%d gs %d/%d mode %d\n",
              (long long)M, (long long)H, (long long)I, bits_g, bits_u, gs_g, gs_u, mode);
    (void)hipGetLastError();
    if (gemv_needs_rows(M, H, bits_g, bits_u)) {
      // x' rows, their exponents and the weight rows' exponents k from the
      // prep kernel's column blocks (gemv_stage_bytes)
      const int kext = kext_columns(H, 32);
      const int64_t xa_bytes = gemv_x_bytes(M, H);
      const int64_t xe_bytes = align256(M * 4);
      void* ws = nullptr;
      int rc = acquire(stream, (size_t)gemv_stage_bytes(M, H, I), &ws, fixed, fixed_bytes);
      if (rc != SWQ_OK) return rc;
      PrepParams pp{};
      pp.x = (const uint16_t*)x;
      pp.sg = (const uint16_t*)sg; pp.bg = (const uint16_t*)bg;
      pp.su = (const uint16_t*)su; pp.bu = (const uint16_t*)bu;
      pp.M = (int)M; pp.H = (int)H; pp.I = (int)I; pp.I_u = (int)I_u;
      pp.gs_g = gs_g; pp.gs_u = gs_u; pp.bits_g = bits_g; pp.bits_u = bits_u;
      pp.g0 = 32; pp.ldx = (int)H + kext; pp.kext = kext;
      pp.xa = (_Float16*)ws;
      pp.xexp = (int*)((char*)ws + xa_bytes);
      pp.kexp = (int*)((char*)ws + xa_bytes + xe_bytes);
      pp.nss = (int)((H + 127) / 128);
      // the weight rows' exponents only when the few-row kernel cannot take
      // them from the scales of its first pass
      pp.k_only = skinny_needs_kexp((int)M, (int)H, bits_g, bits_u) ? 1 : 0;
      pp.xlane = (int)gemv_x_tiles(M);
      pp.act = act;
      p.xa = pp.xa;
      p.xexp = pp.xexp;
      p.kexp = pp.k_only ? pp.kexp : nullptr;
      if (launch_prep_rows(pp, stream) != hipSuccess) return SWQ_ERR_HIP;
    }
    if (launch_gemv(p, bits_g, bits_u, stream) != hipSuccess) return SWQ_ERR_HIP;
    g_calls[SWQ_PATH_GEMV].fetch_add(1, std::memory_order_relaxed);
    return SWQ_OK;
  }

  const WsLayout L = ws_layout(M, H, I, bits_g, gs_g, bits_u, gs_u);
  void* ws = nullptr;
  int rc = acquire(stream, (size_t)L.total, &ws, fixed, fixed_bytes);
  if (rc != SWQ_OK) return rc;
  char* wsb = (char*)ws;
  const int g0 = gs_g < gs_u ? gs_g : gs_u;
  const int kext = kext_columns(H, g0);
  const int ldx = (int)H + kext;
  _Float16* xa = (_Float16*)(wsb + L.xa);
  int* xexp = (int*)(wsb + L.xexp);
  _Float16* eg = (_Float16*)(wsb + L.eg);
  _Float16* eu = (_Float16*)(wsb + L.eu);
  uint32_t* scl = (uint32_t*)(wsb + L.sc);
  const int nss = (int)((H + 127) / 128);

  PrepParams pp;
  pp.x = (const uint16_t*)x;
  pp.sg = (const uint16_t*)sg; pp.bg = (const uint16_t*)bg;
  pp.su = (const uint16_t*)su; pp.bu = (const uint16_t*)bu;
  pp.M = (int)M; pp.H = (int)H; pp.I = (int)I; pp.I_u = (int)I_u;
  pp.gs_g = gs_g; pp.gs_u = gs_u; pp.bits_g = bits_g; pp.bits_u = bits_u;
  pp.g0 = g0; pp.ldx = ldx; pp.kext = kext;
  pp.xa = xa; pp.xexp = xexp;
  pp.bext_g = eg; pp.bext_u = eu;
  pp.scl = scl; pp.nss = nss;
  pp.kexp = (int*)(wsb + L.kx);
  pp.k_only = 0;
  pp.xlane = 0;
  pp.act = act;

  MfmaParams p;
  p.xa = xa; p.xexp = xexp;
  p.wg = Wg; p.sg = (const uint16_t*)sg;
  p.wu = Wu; p.su = (const uint16_t*)su;
  p.M = (int)M; p.H = (int)H; p.I = (int)I;
  p.I_u = (int)I_u; p.ldo = (int)ldo;
  p.n_begin = 0; p.n_end = (int)I;
  p.scl = scl; p.nss = nss;
  p.gs_g = gs_g; p.gs_u = gs_u;
  p.ldx = ldx; p.kext = kext;
  p.bext_g = eg; p.bext_u = eu;
  p.kexp = pp.kexp;
  p.mode = mode; p.out = out; p.dbg_g = dbg_g; p.dbg_u = dbg_u; p.res = (const uint16_t*)res;
  p.act = act;
  p.kchunk = 0;
  {
    const auto a16 = [](const void* q) { return q == nullptr || ((uintptr_t)q & 15) == 0; };
    p.vec = (I % 4 == 0) && (ldo % 4 == 0) && a16(out) && a16(dbg_g) && a16(dbg_u);
  }
  const int cfg = choose_mfma_config(M, I);
  const int n_split = choose_column_split(M, I, cfg, bits_g, bits_u);
  if (logging())
    fprintf(stderr, "[swiglu_q] mfma cfg %d (%dx%d) split %d M=%lld H=%lld I=%lld bits %d/%d gs %d/%d mode %d\n",
            cfg, kMfmaBM[cfg], kMfmaBN[cfg], n_split, (long long)M, (long long)H, (long long)I, bits_g, bits_u,
            gs_g, gs_u, mode);
  // the forward's and the linear's modes may split K (choose_ksplit): partial
  // sums in the workspace ([split][M][I], rows of I), then the second pass
  // writes the output
  const bool can_split = mode == SWQ_MATCH || mode == SWQ_F32 || mode == SWQ_F32_BF16OUT || mode == kLinBf16 ||
                         mode == kLinF32;
  const KSplit ks = (can_split && !dbg_g) ? choose_ksplit(M, H, I, cfg, n_split) : KSplit{};
  (void)hipGetLastError();
  if (launch_prep(pp, stream) != hipSuccess) return SWQ_ERR_HIP;
  if (ks.n > 1) {
    MfmaParams q = p;
    float* part_g = (float*)(wsb + L.part);
    float* part_u = part_g + (int64_t)ks.n * M * I;
    q.dbg_g = part_g;
    q.dbg_u = part_u;
    q.ldo = (int)I;
    q.res = nullptr;
    q.kchunk = ks.chunk;
    q.vec = (I % 4 == 0);
    if (logging()) fprintf(stderr, "[swiglu_q] mfma K split %d x %d K-steps\n", ks.n, ks.chunk);
    if (launch_mfma(q, cfg, 0, ks.n, bits_g, bits_u, stream) != hipSuccess) return SWQ_ERR_HIP;
    if (launch_ksplit_epilogue(p, part_g, part_u, ks.n, stream) != hipSuccess) return SWQ_ERR_HIP;
  } else if (launch_mfma(p, cfg, n_split, 1, bits_g, bits_u, stream) != hipSuccess) {
    return SWQ_ERR_HIP;
  }
  g_calls[SWQ_PATH_MFMA].fetch_add(1, std::memory_order_relaxed);
  return SWQ_OK;
}

int validate_linear(const void* x, const uint32_t* W, const void* s, const void* b, int64_t M, int64_t K,
                    int64_t N, int bits, int gs, int out_mode, const void* out, bool has_x = true) {
  const int64_t Ig = N > 0 ? (N + 1) / 2 : 0;
  int rc = validate(x, W, s, b, W, s, b, M, K, Ig, bits, gs, bits, gs, has_x);
  if (rc != SWQ_OK) return rc;
  if (out_mode != SWQ_LINEAR_BF16 && out_mode != SWQ_LINEAR_F32) return SWQ_ERR_UNSUPPORTED;
  if (!out) return SWQ_ERR_NULL;
  if (!aligned(out, out_mode == SWQ_LINEAR_F32 ? 4 : 2)) return SWQ_ERR_ALIGN;
  return SWQ_OK;
}

// y = x W^T (+ res): W's rows [0, Ig) run in the gate slot of the fused
// kernels, [Ig, N) in the up slot
int linear_run(const void* x, const uint32_t* W, const void* s, const void* b, const void* res, int64_t M,
               int64_t K, int64_t N, int bits, int gs, int out_mode, void* out, void* stream) {
  const int64_t Ig = N > 0 ? (N + 1) / 2 : 0, Iu = N - Ig;
  const uint32_t* Wu = W + Ig * (K * bits / 32);
  const uint16_t* su = (const uint16_t*)s + Ig * (K / gs);
  const uint16_t* bu = (const uint16_t*)b + Ig * (K / gs);
  return run(x, W, s, b, Wu, su, bu, M, K, Ig, Iu, N, bits, gs, bits, gs,
             out_mode == SWQ_LINEAR_F32 ? swq::kLinF32 : swq::kLinBf16, out, nullptr, nullptr, res, SWQ_PATH_AUTO,
             stream);
}

// ---- allocation-free forward ------------------------------------------------
//
// swiglu_q_forward_noalloc stages into this file-scope device array instead of
// the per-stream workspace.  Each GPU the library runs on holds its own copy
// (kScratchBytes of device memory until the process ends).  In host code the
// name `scratch` is only a stand-in: the device address of the copy on the
// current GPU comes from hipGetSymbolAddress, taken once per device at the
// entry point's first call there and kept in g_scratch.  Every call on one GPU
// shares that GPU's copy, so calls that overlap in time on one GPU race.  No
// byte of it needs to start at zero: the prep kernel writes everything the
// GEMM kernels read before they read it.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];   // device address of each GPU's copy, or null before its first call

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SWQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return SWQ_ERR_HIP;
    }
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return SWQ_OK;
}

}  // namespace

extern "C" {

int swiglu_q_forward(const void* x, const uint32_t* Wg, const void* sg, const void* bg,
                     const uint32_t* Wu, const void* su, const void* bu, int64_t M, int64_t H, int64_t I,
                     int bits_g, int gs_g, int bits_u, int gs_u, int precision_mode, void* out,
                     void* stream) {
  int rc = validate(x, Wg, sg, bg, Wu, su, bu, M, H, I, bits_g, gs_g, bits_u, gs_u);
  if (rc != SWQ_OK) return rc;
  if (precision_mode < SWQ_MATCH || precision_mode > SWQ_F32_BF16OUT) return SWQ_ERR_UNSUPPORTED;
  if (!out) return SWQ_ERR_NULL;
  if (!aligned(out, precision_mode == SWQ_F32 ? 4 : 2)) return SWQ_ERR_ALIGN;
  return run(x, Wg, sg, bg, Wu, su, bu, M, H, I, I, I, bits_g, gs_g, bits_u, gs_u, precision_mode, out,
             nullptr, nullptr, nullptr, SWQ_PATH_AUTO, stream);
}

int swiglu_q_forward_f16(const void* x, const uint32_t* Wg, const void* sg, const void* bg,
                         const uint32_t* Wu, const void* su, const void* bu, int64_t M, int64_t H, int64_t I,
                         int bits_g, int gs_g, int bits_u, int gs_u, int precision_mode, void* out,
                         void* stream) {
  int rc = validate(x, Wg, sg, bg, Wu, su, bu, M, H, I, bits_g, gs_g, bits_u, gs_u);
  if (rc != SWQ_OK) return rc;
  if (precision_mode < SWQ_MATCH || precision_mode > SWQ_F32_BF16OUT) return SWQ_ERR_UNSUPPORTED;
  if (!out) return SWQ_ERR_NULL;
  if (!aligned(out, precision_mode == SWQ_F32 ? 4 : 2)) return SWQ_ERR_ALIGN;
  return run(x, Wg, sg, bg, Wu, su, bu, M, H, I, I, I, bits_g, gs_g, bits_u, gs_u, precision_mode, out,
             nullptr, nullptr, nullptr, SWQ_PATH_AUTO, stream, nullptr, 0, kActF16);
}

int swiglu_q_forward_noalloc(const void* x, const uint32_t* Wg, const void* sg, const void* bg,
                             const uint32_t* Wu, const void* su, const void* bu, int64_t M, int64_t H,
                             int64_t I, int bits_g, int gs_g, int bits_u, int gs_u, int precision_mode,
                             void* out, void* stream) {
  int rc = validate(x, Wg, sg, bg, Wu, su, bu, M, H, I, bits_g, gs_g, bits_u, gs_u);
  if (rc != SWQ_OK) return rc;
  if (precision_mode < SWQ_MATCH || precision_mode > SWQ_F32_BF16OUT) return SWQ_ERR_UNSUPPORTED;
  if (!out) return SWQ_ERR_NULL;
  if (!aligned(out, precision_mode == SWQ_F32 ? 4 : 2)) return SWQ_ERR_ALIGN;
  if (M == 0) return SWQ_OK;
  // the size check comes before any HIP call
  const int path = auto_path(M, H, I);
  if (staging_bytes(M, H, I, bits_g, gs_g, bits_u, gs_u, path) > (int64_t)kScratchBytes) return SWQ_ERR_TOO_LARGE;
  void* ptr = nullptr;
  rc = scratch_address(&ptr);
  if (rc != SWQ_OK) return rc;
  return run(x, Wg, sg, bg, Wu, su, bu, M, H, I, I, I, bits_g, gs_g, bits_u, gs_u, precision_mode, out, nullptr,
             nullptr, nullptr, path, stream, ptr, kScratchBytes);
}

int swiglu_q_linear(const void* x, const uint32_t* W, const void* s, const void* b, int64_t M, int64_t K,
                    int64_t N, int bits, int gs, int out_mode, void* out, void* stream) {
  int rc = validate_linear(x, W, s, b, M, K, N, bits, gs, out_mode, out);
  if (rc != SWQ_OK) return rc;
  return linear_run(x, W, s, b, nullptr, M, K, N, bits, gs, out_mode, out, stream);
}

int swiglu_q_mlp(const void* x, const uint32_t* Wg, const void* sg, const void* bg, const uint32_t* Wu,
                 const void* su, const void* bu, const uint32_t* Wd, const void* sd, const void* bd,
                 const void* residual, int64_t M, int64_t H, int64_t I, int64_t Ho, int bits_g, int gs_g,
                 int bits_u, int gs_u, int bits_d, int gs_d, int out_mode, void* out, void* stream) {
  int rc = validate(x, Wg, sg, bg, Wu, su, bu, M, H, I, bits_g, gs_g, bits_u, gs_u);
  if (rc != SWQ_OK) return rc;
  // the down projection (K = I, N = Ho) reads the library's hidden tensor
  rc = validate_linear(nullptr, Wd, sd, bd, M, I, Ho, bits_d, gs_d, out_mode, out, false);
  if (rc != SWQ_OK) return rc;
  if (!aligned(residual, 2)) return SWQ_ERR_ALIGN;
  if (M == 0) return SWQ_OK;
  void* hidden = nullptr;
  rc = get_workspace((hipStream_t)stream, (size_t)align256(M * I * 2), &hidden, 1);
  if (rc != SWQ_OK) return rc;
  rc = run(x, Wg, sg, bg, Wu, su, bu, M, H, I, I, I, bits_g, gs_g, bits_u, gs_u, SWQ_MATCH, hidden, nullptr,
           nullptr, nullptr, SWQ_PATH_AUTO, stream);
  if (rc != SWQ_OK) return rc;
  return linear_run(hidden, Wd, sd, bd, residual, M, I, Ho, bits_d, gs_d, out_mode, out, stream);
}

int swiglu_q_debug_gemm(const void* x, const uint32_t* Wg, const void* sg, const void* bg,
                        const uint32_t* Wu, const void* su, const void* bu, int64_t M, int64_t H,
                        int64_t I, int bits_g, int gs_g, int bits_u, int gs_u, int path, float* gate_out,
                        float* up_out, void* stream) {
  int rc = validate(x, Wg, sg, bg, Wu, su, bu, M, H, I, bits_g, gs_g, bits_u, gs_u);
  if (rc != SWQ_OK) return rc;
  if (path != SWQ_PATH_AUTO && path != SWQ_PATH_GEMV && path != SWQ_PATH_MFMA) return SWQ_ERR_UNSUPPORTED;
  if (!gate_out || !up_out) return SWQ_ERR_NULL;
  if (!aligned(gate_out, 4) || !aligned(up_out, 4)) return SWQ_ERR_ALIGN;
  return run(x, Wg, sg, bg, Wu, su, bu, M, H, I, I, I, bits_g, gs_g, bits_u, gs_u, SWQ_F32, nullptr, gate_out,
             up_out, nullptr, path, stream);
}

int swiglu_q_supported(int64_t H, int bits_g, int gs_g, int bits_u, int gs_u, int precision_mode) {
  if (!spec_ok(bits_g, gs_g) || !spec_ok(bits_u, gs_u)) return 0;
  if (precision_mode < SWQ_MATCH || precision_mode > SWQ_F32_BF16OUT) return 0;
  if (H <= 0 || H % 32 != 0 || H % gs_g != 0 || H % gs_u != 0 || H > (1LL << 20)) return 0;
  return 1;
}

void swiglu_q_set_m_threshold(int T) { g_threshold.store(T < 0 ? -1 : T); }

int swiglu_q_get_m_threshold(void) {
  const int t = explicit_threshold();
  return t >= 0 ? t : kDefaultThreshold;
}

int swiglu_q_path_for(int64_t M, int64_t H, int64_t I) {
  if (M < 1 || H < 1 || I < 1) return -1;
  return auto_path(M, H, I);
}

uint64_t swiglu_q_call_count(int path) {
  if (path != SWQ_PATH_GEMV && path != SWQ_PATH_MFMA) return 0;
  return g_calls[path].load();
}

void swiglu_q_set_max_calls(int64_t n) { g_max_calls.store(n < 0 ? -1 : n); }

int swiglu_q_under_cap(void) {
  const int64_t cap = max_calls_now();
  return cap < 0 || (int64_t)(g_calls[0].load() + g_calls[1].load()) < cap;
}

void swiglu_q_reset_counts(void) {
  g_calls[0].store(0);
  g_calls[1].store(0);
}

const char* swiglu_q_strerror(int status) {
  switch (status) {
    case SWQ_OK: return "ok";
    case SWQ_ERR_NULL: return "a required pointer is NULL";
    case SWQ_ERR_SHAPE: return "invalid shape (M<0, H<=0, I<=0, H not a multiple of 32 or of a group size)";
    case SWQ_ERR_UNSUPPORTED: return "unsupported bits, group size, precision mode or path";
    case SWQ_ERR_ALIGN: return "misaligned pointer (x, Wg, Wu need 16 bytes; others their element size)";
    case SWQ_ERR_HIP: return "HIP launch or runtime error";
    case SWQ_ERR_WORKSPACE: return "workspace allocation failed";
    case SWQ_ERR_TOO_LARGE: return "the call needs more staging than the allocation-free entry point's fixed 64 MiB";
    default: return "unknown status";
  }
}

int64_t swiglu_q_workspace_bytes(int64_t M, int64_t H, int64_t I, int bits_g, int gs_g, int bits_u,
                                 int gs_u) {
  if (M <= 0 || H <= 0 || I <= 0 || !spec_ok(bits_g, gs_g) || !spec_ok(bits_u, gs_u)) return 0;
  if (H % gs_g != 0 || H % gs_u != 0) return 0;
  return ws_layout(M, H, I, bits_g, gs_g, bits_u, gs_u).total;
}

int64_t swiglu_q_staging_bytes(int64_t M, int64_t H, int64_t I, int bits_g, int gs_g, int bits_u, int gs_u,
                               int path) {
  if (M <= 0 || H <= 0 || I <= 0 || !spec_ok(bits_g, gs_g) || !spec_ok(bits_u, gs_u)) return 0;
  if (H % 32 != 0 || H % gs_g != 0 || H % gs_u != 0) return 0;
  if (path == SWQ_PATH_AUTO) path = auto_path(M, H, I);
  if (path == SWQ_PATH_GEMV && !gemv_fits(M, H)) return 0;
  if (path != SWQ_PATH_GEMV && path != SWQ_PATH_MFMA) return 0;
  return staging_bytes(M, H, I, bits_g, gs_g, bits_u, gs_u, path);
}

int swiglu_q_release_workspace(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int rc = SWQ_OK;
  int prev = 0;
  (void)hipGetDevice(&prev);
  for (auto& kv : g_ws) g_retired.emplace_back(std::get<0>(kv.first), kv.second.ptr);
  for (auto& r : g_retired) {
    if (!r.second) continue;
    if (hipSetDevice(r.first) != hipSuccess) { rc = SWQ_ERR_HIP; continue; }
    if (hipDeviceSynchronize() != hipSuccess) rc = SWQ_ERR_HIP;
    if (hipFree(r.second) != hipSuccess) rc = SWQ_ERR_HIP;
  }
  (void)hipSetDevice(prev);
  g_ws.clear();
  g_retired.clear();
  return rc;
}

const char* swiglu_q_version(void) { return "swiglu_q 0.1.0 (gfx950)"; }

}  // extern "C"
