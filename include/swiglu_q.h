/*
 * swiglu_q — fused quantized SwiGLU expansion for AMD Instinct MI355X (gfx950).
 *
 *   hidden[M, I] = silu(x · Wgᵀ) ⊙ (x · Wuᵀ),   silu(t) = t · σ(t),  σ(t) = 1 / (1 + e^(−t))
 *
 * Wg and Wu are affine group-quantized: each weight is stored as an unsigned
 * integer code q of `bits` bits, and every group of `gs` consecutive codes
 * along K (the hidden dimension H) has one bf16 scale s and one bf16 bias b,
 * so that w = s·q + b.  The down projection is not part of this call.
 *
 * Sources (pages of the "mlx-bun" package diffs):
 *  - the operation, one dispatch computing both projections from one read of
 *    x, and the down projection left as a separate call:
 *    "mlx-bun 0.0.7 -> 0.0.9" (page 42), fused-swiglu-kernel.ts, header comment;
 *  - the host entry (x, then gate weight/scales/biases, then up
 *    weight/scales/biases, then the two quantization specs, gate and up
 *    specs independent), its shapes and "caller owns the result":
 *    same file, host entry and its docstring;
 *  - the two precision variants: same file, precision-variants comment;
 *  - the support predicate (bf16 or float16 activations, affine biases
 *    present, group size a multiple of 32, H a multiple of 32): same file,
 *    support predicate; the kernel's element type is x's (its template
 *    dtype argument), so scales, biases and result share it;
 *  - the M threshold below which the caller keeps the matrix-vector path:
 *    same file, M-threshold function and the "where the win is" comment.
 *
 * Memory layout (all row-major, contiguous, no strides):
 *   x        bf16    [M, H]
 *   Wg, Wu   uint32  [I, H·bits/32]   codes along K, 32/bits per word, code j of
 *                                     a word in bits [bits·j, bits·j + bits)
 *                                     (least significant first)
 *   sg,bg,su,bu bf16 [I, H/gs]        scale and bias of each group
 *   out      [M, I]  bf16 for SWQ_MATCH and SWQ_F32_BF16OUT, float32 for SWQ_F32
 *
 * Ownership and synchronisation: every pointer passed to the forward calls
 * is a DEVICE pointer owned by the caller; the library never frees or keeps
 * them.  Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 * and the call returns without synchronising.  A matrix-vector call whose
 * kernel cannot convert x itself needs a device workspace for the staged x
 * (swiglu_q_staging_bytes says how much; most calls with 4-bit or 2-bit
 * codes, H <= 2048 and M <= 128 need none),
 * and every matrix-matrix call needs one for x and the weights' extra rows,
 * scale tiles and row exponents (and, where few output tiles split K across
 * blocks, the float32 partial sums): the library keeps one per (device, stream),
 * allocated on
 * first use and replaced by a larger one (at least twice the size) when a call
 * needs more.  Growth never synchronises: a replaced buffer is kept, not freed,
 * until swiglu_q_release_workspace(), so work already queued on the stream and
 * HIP graphs captured while it was current still have valid memory.  Calls and
 * graph replays that use one stream's workspace must not run at the same time
 * (on that stream they are ordered).  HIP graphs: a call recorded into a graph
 * must not need to grow a buffer (allocation cannot be captured; such a call
 * returns SWQ_ERR_HIP or SWQ_ERR_WORKSPACE), so make one call of the largest
 * shape on the same stream before capturing; the kernels write every output
 * element and need no clearing between replays.
 *
 * Exactness: the weights are dequantized exactly (no rounding of s·q + b), and
 * gate and up are float32 dot products, for any finite bf16 scales and biases.
 * Before a kernel forms 16-bit operands it multiplies each weight row's scales
 * and constants (c = b + z·s, z the code offset 8, or 136 for 8-bit codes) by a
 * power of two of that row's own, chosen from the row's largest |s|·(largest
 * code offset) and |c|, and multiplies the row's sums back at the end.  Every
 * group whose largest such term is at least 2^-28 (8-bit codes: 2^-24) of the
 * row's largest is then exact in binary16; a smaller group's weights are
 * rounded to binary16's grid at the row's scale, an error below 2^-39 of the
 * row's largest term per weight.  Results are finite whenever the float32
 * sums are (the M = 1 kernel applies s and b in float32 throughout).
 * Binary16 scales (swiglu_q_forward_f16) have 11 significant bits; they are
 * split into a part of 8 significant bits and a remainder of at most 3, each
 * with its own MFMA operand, and the window becomes 2^-25 (8-bit codes:
 * 2^-21) of the row's largest term, with the same bound outside it.
 *
 * Errors: every entry point validates its arguments on the host before any
 * HIP call and returns a status; nothing is launched on error.
 */
#ifndef SWIGLU_Q_H
#define SWIGLU_Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SWQ_OK               0
#define SWQ_ERR_NULL         1  /* a required pointer is NULL                       */
#define SWQ_ERR_SHAPE        2  /* M < 0, H <= 0, I <= 0, H % gs != 0, H % 32 != 0,
                                   H > 2^20, M or I > 2^30, or a staged copy of x
                                   (2 bytes x M x about 1.05 H) of 4 GiB or more   */
#define SWQ_ERR_UNSUPPORTED  3  /* bits not in {2, 4, 8}, gs not in {32, 64, 128},
                                   unknown precision mode or path                   */
#define SWQ_ERR_ALIGN        4  /* a pointer is not 16-byte aligned                 */
#define SWQ_ERR_HIP          5  /* a HIP call or kernel launch failed               */
#define SWQ_ERR_WORKSPACE    6  /* the workspace could not be allocated             */
#define SWQ_ERR_TOO_LARGE    7  /* swiglu_q_forward_noalloc: the call's staging would
                                   exceed its fixed 64 MiB                          */

/* Precision modes (the pages' two variants; the wide one with two output types). */
#define SWQ_MATCH        0  /* gate and up rounded to bf16 (RNE) before silu·up;
                               product computed in float32, rounded once to bf16   */
#define SWQ_F32          1  /* gate, up, silu and product in float32; float32 out  */
#define SWQ_F32_BF16OUT  2  /* as SWQ_F32, rounded once to bf16 at the store       */

/* Kernel paths chosen by the M-threshold dispatcher. */
#define SWQ_PATH_GEMV    0  /* M < threshold (M <= 128): matrix-vector kernels     */
#define SWQ_PATH_MFMA    1  /* M >= threshold: dequantizing bf16/f16 MFMA GEMM      */
#define SWQ_PATH_AUTO   -1

/*
 * Fused forward: out = silu(x·Wgᵀ) ⊙ (x·Wuᵀ) in the given precision mode.
 *   x            bf16 [M, H] device pointer
 *   Wg, sg, bg   gate codes [I, H·bits_g/32], scales and biases [I, H/gs_g]
 *   Wu, su, bu   up codes [I, H·bits_u/32], scales and biases [I, H/gs_u]
 *   M, H, I      rows of x, hidden size, intermediate size
 *   bits_*, gs_* quantization spec of each matrix: bits in {2, 4, 8},
 *                gs in {32, 64, 128}, H a multiple of gs and of 32
 *   precision_mode  SWQ_MATCH, SWQ_F32 or SWQ_F32_BF16OUT
 *   out          [M, I] device pointer, bf16 or float32 by mode
 *   stream       hipStream_t (NULL = null stream)
 * M == 0 returns SWQ_OK with nothing launched.  x, Wg and Wu must be 16-byte
 * aligned, the scales, biases and out aligned to their element size
 * (SWQ_ERR_ALIGN otherwise).
 */
int swiglu_q_forward(const void *x,
                     const uint32_t *Wg, const void *sg, const void *bg,
                     const uint32_t *Wu, const void *su, const void *bu,
                     int64_t M, int64_t H, int64_t I,
                     int bits_g, int gs_g, int bits_u, int gs_u,
                     int precision_mode, void *out, void *stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, validation, kernels and results (bit for bit)
 * as swiglu_q_forward, but the call allocates nothing: the staging that
 * swiglu_q_forward keeps in its per-stream workspace lives in a fixed
 * 64 MiB device array that each GPU the library runs on holds from the first
 * such call until the process ends.  Returns SWQ_ERR_TOO_LARGE, before any
 * HIP call, when the call would need more than that (the matrix-matrix path
 * needs swiglu_q_workspace_bytes(...); M = 8192, H = 2560, I = 10240 with an
 * 8-bit gs 32 gate fits).  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU, on any streams, race and give wrong
 * results; order them (one stream, or events).
 */
/*
 * Fused forward with binary16 activations: x, sg, bg, su and bu are float16
 * (IEEE binary16) instead of bf16, and out is float16 for SWQ_MATCH (gate and
 * up rounded to float16, RNE) and SWQ_F32_BF16OUT (float32 internal, rounded
 * once to float16), float32 for SWQ_F32.  Everything else -- arguments,
 * layout, validation, status codes, workspace, dispatch -- is as in
 * swiglu_q_forward.  Source: the support predicate accepts float16
 * activations and the kernel's element type follows x ("mlx-bun 0.0.7 ->
 * 0.0.9", page 42, fused-swiglu-kernel.ts, support predicate and host
 * entry).  The matrix-matrix path runs the bf16 tile shapes with one more
 * MFMA per code block (the scales' two parts), the matrix-vector kernels as
 * for bf16.
 */
int swiglu_q_forward_f16(const void *x,
                         const uint32_t *Wg, const void *sg, const void *bg,
                         const uint32_t *Wu, const void *su, const void *bu,
                         int64_t M, int64_t H, int64_t I,
                         int bits_g, int gs_g, int bits_u, int gs_u,
                         int precision_mode, void *out, void *stream);

int swiglu_q_forward_noalloc(const void *x,
                             const uint32_t *Wg, const void *sg, const void *bg,
                             const uint32_t *Wu, const void *su, const void *bu,
                             int64_t M, int64_t H, int64_t I,
                             int bits_g, int gs_g, int bits_u, int gs_u,
                             int precision_mode, void *out, void *stream);

/* Output types of swiglu_q_linear. */
#define SWQ_LINEAR_BF16  0  /* float32 sums rounded once to bf16 (RNE) at the store */
#define SWQ_LINEAR_F32   1  /* float32 sums stored as float32                      */

/*
 * Quantized linear: out = x·Wᵀ, the plain projection the fused forward's
 * output feeds (the down projection; "mlx-bun 0.0.7 -> 0.0.9" diff, page 43,
 * steel-linear-kernel.ts: its header comment defines it as y = x·Wᵀ over an
 * affine-quantized W, stored in the activation type).
 *   x         bf16 [M, K] device pointer
 *   W, s, b   codes [N, K·bits/32], scales and biases [N, K/gs] (same packing
 *             and dequantization w = s·q + b as the forward)
 *   M, K, N   rows of x, input size, output size
 *   bits, gs  bits in {2, 4, 8}, gs in {32, 64, 128}, K a multiple of gs and 32
 *   out_mode  SWQ_LINEAR_BF16 or SWQ_LINEAR_F32
 *   out       [M, N] device pointer, bf16 or float32 by out_mode
 *   stream    hipStream_t (NULL = null stream)
 * The sums are float32 dot products of the exactly dequantized weights (the
 * forward's arithmetic).  It runs on the forward's kernels and dispatcher
 * (threshold, workspace and counters included), W's first ceil(N/2) rows in
 * the gate slot and the rest in the up slot.  Same status codes, limits and
 * alignment rules as swiglu_q_forward with H = K and I = ceil(N/2).
 */
int swiglu_q_linear(const void *x, const uint32_t *W, const void *s, const void *b,
                    int64_t M, int64_t K, int64_t N, int bits, int gs,
                    int out_mode, void *out, void *stream);

/*
 * Whole MLP: out = residual + (silu(x·Wgᵀ) ⊙ (x·Wuᵀ))·Wdᵀ.  The pages' fused
 * MLP ("mlx-bun 0.0.7 -> 0.0.9" diff, page 42, fused-mlp-kernel.ts, header
 * comment and the fusedMlp host function) computes the SwiGLU hidden tensor
 * of an (M, I) tile once, multiplies it into the down projection and returns
 * the result in the activation type; the model's MLP ("mlx-bun 0.0.8 ->
 * 0.0.10" diff, page 41, minicpm5.ts, LlamaMLP.forward) passes the layer
 * input as a residual that the call adds to the MLP output.
 *   x, Wg..bu, M, H, I, bits_g..gs_u   as swiglu_q_forward
 *   Wd, sd, bd  down codes [Ho, I·bits_d/32], scales and biases [Ho, I/gs_d];
 *               I a multiple of gs_d and of 32
 *   residual    bf16 [M, Ho] device pointer, or NULL for none
 *   Ho          output size (the model's hidden size)
 *   out_mode    SWQ_LINEAR_BF16 or SWQ_LINEAR_F32
 *   out         [M, Ho] device pointer, bf16 or float32 by out_mode
 * Two launches on `stream`: the fused forward in SWQ_MATCH writes the hidden
 * tensor (bf16 [M, I]) into a buffer the library keeps per (device, stream)
 * beside its workspace (grown on demand, freed by swiglu_q_release_workspace),
 * then the quantized linear of Wd reads it and adds the residual in float32
 * before its one rounding.  Deterministic: no atomics.  Status codes and
 * alignment rules as swiglu_q_forward and swiglu_q_linear; residual aligned
 * to 2 bytes.  Calls that overlap on one stream's buffers are ordered by the
 * stream.
 */
int swiglu_q_mlp(const void *x,
                 const uint32_t *Wg, const void *sg, const void *bg,
                 const uint32_t *Wu, const void *su, const void *bu,
                 const uint32_t *Wd, const void *sd, const void *bd,
                 const void *residual,
                 int64_t M, int64_t H, int64_t I, int64_t Ho,
                 int bits_g, int gs_g, int bits_u, int gs_u, int bits_d, int gs_d,
                 int out_mode, void *out, void *stream);

/* 1 if the combination is supported by swiglu_q_forward, else 0 (mirrors the
 * pages' support predicate, restricted to what this library implements). */
int swiglu_q_supported(int64_t H, int bits_g, int gs_g, int bits_u, int gs_u,
                       int precision_mode);

/* M threshold T of the dispatcher: M < T takes SWQ_PATH_GEMV, M >= T takes
 * SWQ_PATH_MFMA; the matrix-vector path takes at most 128 rows (past 32, as
 * row groups of 32 that each read the weights once), so M > 128 always runs
 * the MFMA path.  T is the value given to swiglu_q_set_m_threshold (T >= 0),
 * else the environment variable SWIGLU_Q_MMIN when set to a positive integer,
 * and applies to every weight shape.  Without either, the default rule
 * applies: T = 65, or T = 33 for wide weights (H * I >= 3 * 2^23 with
 * I >= 4096), or T = 129 for small weights (H * I <= 2^23; the matrix-vector
 * path up to its 128 rows); the linear's I is ceil(N / 2).
 * (Measured: the matrix-vector path is faster for every M <= 32 on every
 * weight shape measured.  For 33 <= M <= 64 it is 17-67 % faster up to
 * H * I = 2^24, e.g. H = 2048, I = 5632, and on fewer columns.  It is
 * 24-66 % slower on wide weights, e.g. H = 4096, I = 14336, where the MFMA
 * path splits K.)
 * swiglu_q_set_m_threshold with T < 0 restores the default rule; T <= 1
 * sends every M >= 1 to the MFMA path.  swiglu_q_get_m_threshold returns the
 * threshold set, else 65 (the default rule's value for weights that are not wide). */
void swiglu_q_set_m_threshold(int T);
int swiglu_q_get_m_threshold(void);

/* The path (SWQ_PATH_GEMV or SWQ_PATH_MFMA) a call with M rows, hidden size
 * H and intermediate size I takes under the current threshold, by the same
 * rule as the calls (M < T and M <= 128 take the matrix-vector path; the
 * linear's rule is that of I = ceil(N / 2)); -1 for M, H or I below 1.
 * Host only: touches no device. */
int swiglu_q_path_for(int64_t M, int64_t H, int64_t I);

/* Number of forward (and debug) calls that launched each path since load
 * or the last reset.  path: SWQ_PATH_GEMV or SWQ_PATH_MFMA.  Mirrors the
 * pages' dispatch counter, which a gate test asserts on to prove that the
 * kernel ran ("mlx-bun 0.0.7 -> 0.0.9" diff, page 42, fused-swiglu-kernel.ts,
 * dispatch counter). */
uint64_t swiglu_q_call_count(int path);
void swiglu_q_reset_counts(void);

/* Call cap for bisecting, the pages' debug cap on how many fused calls run
 * ("mlx-bun 0.0.7 -> 0.0.9" diff, page 42, fused-swiglu-kernel.ts, the cap
 * function and its caller's predicate): a caller that keeps an unfused path
 * asks swiglu_q_under_cap() before each call and takes its own path once it
 * returns 0.  The cap counts launched calls of both paths (the sum of
 * swiglu_q_call_count); n < 0 removes it.  The default comes from the
 * environment variable SWIGLU_Q_MAXCALLS (a non-negative integer), else no
 * cap.  Host only: the library itself never refuses a call. */
void swiglu_q_set_max_calls(int64_t n);
int swiglu_q_under_cap(void);

/* Human-readable text of a status code (static storage). */
const char *swiglu_q_strerror(int status);

/*
 * Test hook (the pages' debug-gate switch, which writes the raw gate
 * projection instead of hidden: "mlx-bun 0.0.7 -> 0.0.9" diff, page 42,
 * fused-swiglu-kernel.ts, kernel source): the pre-epilogue gate and up
 * projections in float32,
 * gate_out[M, I] and up_out[M, I] (device pointers, caller-owned), computed
 * by the kernel of `path` (SWQ_PATH_AUTO = what the dispatcher would pick).
 * Same validation and status codes as swiglu_q_forward.
 */
int swiglu_q_debug_gemm(const void *x,
                        const uint32_t *Wg, const void *sg, const void *bg,
                        const uint32_t *Wu, const void *su, const void *bu,
                        int64_t M, int64_t H, int64_t I,
                        int bits_g, int gs_g, int bits_u, int gs_u,
                        int path, float *gate_out, float *up_out, void *stream);

/* Bytes of workspace the MFMA path uses for this shape (0 when M == 0 or
 * the arguments are invalid), including the K split's float32 partial sums
 * where the shape takes it (the choice depends on the current device's CU
 * count and on SWIGLU_Q_MFMA_KSPLIT). */
int64_t swiglu_q_workspace_bytes(int64_t M, int64_t H, int64_t I, int bits_g, int gs_g,
                                 int bits_u, int gs_u);

/* Bytes of device staging a call of this shape takes on `path`
 * (SWQ_PATH_AUTO: the dispatcher's choice): what swiglu_q_forward takes from
 * its workspace, and swiglu_q_forward_noalloc from its static array.  0 when
 * the call stages nothing (the matrix-vector kernels read x themselves: M =
 * 1, and the few-row kernel whenever a row fits one pass of its waves), when
 * M == 0, or when the arguments are invalid. */
int64_t swiglu_q_staging_bytes(int64_t M, int64_t H, int64_t I, int bits_g, int gs_g,
                               int bits_u, int gs_u, int path);

/* Free every cached workspace (synchronises the device first). */
int swiglu_q_release_workspace(void);

/* Library version string. */
const char *swiglu_q_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_Q_H */
