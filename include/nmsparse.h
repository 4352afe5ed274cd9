/*
 * nmsparse.h - C ABI of the MI355X (gfx950) N:M semi-structured sparsity library.
 *
 * The library implements the data-parallel hot path of post-training N:M
 * sparsification of LLM linear layers: importance scores, per-group top-N mask
 * selection, packing of kept values with their in-group positions, the
 * sliding-window decomposition of (2N-2):2N into overlapping 2:4 windows, and
 * the structured-sparse linear layer Y = X * W_hat^T on packed weights
 * (bf16, and int8 activations x ternary int8 weights).
 *
 * Conventions shared by every entry point
 *  - Pointers are DEVICE pointers owned by the caller unless the comment says
 *    host.  The library never allocates, frees or synchronises; work is enqueued
 *    on `stream` (a hipStream_t passed as void*, NULL = the null stream) and the
 *    call returns immediately.  NM_OK means "enqueued"; results are valid once
 *    the caller synchronises the stream.
 *  - Every argument is validated before anything is enqueued; on an error
 *    nothing is written and the status says why.  nm_last_error() then returns
 *    a message (thread-local, valid until the next call on this thread).
 *    A failed kernel launch returns NM_ERR_DEVICE with HIP's message.
 *  - Matrices are row-major with an explicit leading dimension (in elements,
 *    except where noted).  Weights are [R = out_features, K = in_features];
 *    activations are [tokens, K]; an N:M group is M consecutive weights of a
 *    row along K.
 *  - Mask bits: one bit per weight, LSB-first, uint8 [R, ldm bytes], ldm >= ceil(K/8).
 *  - Packed weights: vals [R, ldv] holds the kept values of group g at
 *    vals[g*N .. g*N+N-1] in ascending in-group position; idx [R, ldi uint32
 *    words] is an LSB-first bitstream of b = ceil(log2 M)-bit in-group
 *    positions, field j of a row at bits j*b .. j*b+b-1.  For 2:4 this is two
 *    2-bit positions per group, 16 fields per word.  Every group always
 *    carries N distinct ascending positions (padded with value 0 when a mask
 *    row has fewer than N bits in a group).
 *  - Lifted (slide) format: the 2:4 packed format over K' = (2 - 2/N) K, one
 *    2:4 group per window, windows of a 2N-group in order.
 *  - Alignment: base pointers must be 16-byte aligned and leading dimensions
 *    multiples of 16 bytes where a kernel uses vector access (NM_ERR_ALIGN).
 *  - Aliasing: outputs must not overlap inputs (NM_ERR_ALIAS).
 *  - Calls are stateless and thread-safe; calls on different streams may overlap.
 *    The one exception to "never synchronises" is NM_FLAG_VALIDATE (below).
 */
#ifndef NMSPARSE_H
#define NMSPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NM_ABI_VERSION 2

typedef void* nm_stream_t;

typedef enum {
    NM_OK = 0,
    NM_ERR_NULL = 1,      /* required pointer is NULL */
    NM_ERR_SHAPE = 2,     /* sizes negative, inconsistent, or beyond int32 exactness */
    NM_ERR_PATTERN = 3,   /* unsupported N:M (or slide N) */
    NM_ERR_DTYPE = 4,     /* unsupported dtype combination */
    NM_ERR_ALIGN = 5,     /* pointer / leading dimension alignment */
    NM_ERR_WORKSPACE = 6, /* workspace NULL or too small */
    NM_ERR_DEVICE = 7,    /* HIP error (launch or device query) */
    NM_ERR_ALIAS = 8      /* an output overlaps an input */
} nm_status;

/* NM_FP8: OCP FP8 e4m3 codes, one byte each (1 sign, 4 exponent bits with bias 7,
 * 3 mantissa bits; no infinities, 0x7f/0xff NaN, largest finite 448).  FP8 is
 * one of the precisions the sliding-window product runs in ("SlideSparse",
 * section 3); here it is carried as raw codes by the packers and multiplied by
 * nm_spmm with f32 accumulation. */
typedef enum { NM_F32 = 0, NM_BF16 = 1, NM_I8 = 2, NM_I32 = 3, NM_FP8 = 4 } nm_dtype;

typedef enum { NM_SCORE_HESSIAN = 0, NM_SCORE_MAGNITUDE = 1 } nm_score_mode;

/* flags of the calls that pack a caller's mask (nm_pack, nm_slide_decompose).
 * NM_FLAG_VALIDATE: before anything is written, count on the device the groups
 * whose mask holds more bits than the format keeps (more than N of an N:M group,
 * more than 2N-2 of a 2N slide group: "Sparse-BitNet", section 1 and "SlideSparse",
 * section 2A), wait for the count (the call synchronises `stream`) and return
 * NM_ERR_PATTERN, with the count in nm_last_error(), if there are any; nothing is
 * packed then.  Without the flag such groups keep their first N (2N-2) set bits.
 * Validating calls share one counter per device and are serialised within the
 * process.  Other flag bits are rejected (NM_ERR_SHAPE). */
#define NM_FLAG_VALIDATE 1u

int nm_abi_version(void);
const char* nm_last_error(void);

/* ---------------------------------------------------------------- curvature
 * Diagonal Gauss-Newton proxy of a linear layer's Hessian from calibration
 * activations: H[k] = sum_i X[i,k]^2.  ("Sparsity Induction", section 2C: the
 * diagonal proxy lets importance scores refresh in O(d_in).)
 * X: [n, K] bf16 or f32, leading dim ldx elements.  H: [K] f32 out.
 * The squares (exact in f64) are summed in f64 in a fixed (run-to-run identical)
 * order and the sum is rounded to f32 once: H is the f32 rounding of the exact sum
 * up to the f64 summation error (about n * 2^-53 relative).
 * ws: device workspace of nm_colsumsq_workspace(n, K) bytes; the current kernel needs none
 *     (the call returns 0) and ws may be NULL. */
size_t nm_colsumsq_workspace(int64_t n, int64_t K);
nm_status nm_hdiag_colsumsq(const void* X, nm_dtype xdt, int64_t n, int64_t K, int64_t ldx,
                            float* H, void* ws, size_t ws_bytes, nm_stream_t stream);

/* Hutchinson estimate of the Hessian diagonal of the layer's quadratic output
 * energy L(W) = ||X W^T||_F^2 with Rademacher probes ("SparseForge", Methodology
 * 2: the diagonal is estimated stochastically because the full Hessian is
 * prohibitive):  D = (1/P) sum_p V_p .* (H V_p),  H V = 2 (V X^T) X.
 * V_p[o,k] in {-1,+1} is bit (k mod 64) of SplitMix64 output number
 * p*2^40 + o*ceil(K/64) + floor(k/64) of a generator seeded with `seed`
 * (bit set -> -1); it is generated in registers, never stored.
 * X: [n, K] bf16 (ldx elements).  D: [R, K] f32 out (ldd elements).
 * Both products run on bf16 MFMA with f32 accumulation; V X^T is rounded to
 * bf16 before the second product.  Requires K % 64 == 0, n % 64 == 0.
 * ws: nm_hutchinson_workspace(n, K, R, probes) bytes. */
size_t nm_hutchinson_workspace(int64_t n, int64_t K, int64_t R, int probes);
nm_status nm_hdiag_hutchinson(const void* X, int64_t n, int64_t K, int64_t ldx, int64_t R, int probes,
                              uint64_t seed, float* D, int64_t ldd, void* ws, size_t ws_bytes,
                              nm_stream_t stream);

/* Hutchinson diagonal, score and its statistics in one pass over the curvature
 * ("SparseForge", Methodology 2: the Hutchinson/Rademacher diagonal D of the Hessian
 * weights the score s = (D + eps) * W^2, and the scores are standardised per tensor):
 * S = (D + eps) * W^2 with D as nm_hdiag_hutchinson computes it and the score's
 * arithmetic of nm_score, so S equals nm_hdiag_hutchinson followed by nm_score bit for
 * bit; D itself is never stored.  stats (nullable, device f64 [2]): mean and population
 * standard deviation of S as nm_score_stats gives them (combined in another fixed order:
 * equal to about 1e-15 relative).  W: bf16 [R, K] (ldw, 8-byte aligned rows); S: f32
 * [R, K] (lds, 16-byte aligned rows).  Requirements of nm_hdiag_hutchinson, plus
 * probes * R * n * 2 < 2^32 (NM_ERR_SHAPE otherwise) and a 16-byte aligned workspace.
 * ws: nm_hutchinson_score_workspace(n, K, R, probes) bytes. */
size_t nm_hutchinson_score_workspace(int64_t n, int64_t K, int64_t R, int probes);
nm_status nm_hutchinson_score(const void* X, int64_t n, int64_t K, int64_t ldx, int64_t R, int probes,
                              uint64_t seed, const void* W, nm_dtype wdt, int64_t ldw, float eps,
                              float* S, int64_t lds, double* stats, void* ws, size_t ws_bytes,
                              nm_stream_t stream);

/* ---------------------------------------------------------------- score
 * Importance score ("SparseForge", Methodology 2: s = (H + eps) * W^2 with H a
 * Hessian-diagonal approximation; "Sparse-BitNet", section 2: magnitude |W|).
 * HESSIAN: s = (h + eps) * (w * w) in f32, one rounding per operation in the
 * order t = w*w, u = h + eps, s = u*t.  MAGNITUDE: s = |w| (H ignored).
 * W: [R, K] bf16 or f32 (ldw).  H: f32, ldh == 0 -> one [K] vector for all rows,
 * ldh >= K -> [R, K] (e.g. a Hutchinson diagonal).  S: [R, K] f32 out (lds). */
nm_status nm_score(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw,
                   const float* H, int64_t ldh, float eps, nm_score_mode mode,
                   float* S, int64_t lds, nm_stream_t stream);

/* Per-tensor standardisation statistics of a score matrix ("SparseForge",
 * Methodology 2: scores are standardised before the temperature sigmoid).
 * stats[0] = mean, stats[1] = population standard deviation, both f64, from one
 * pass: per-thread shifted sums turned into (count, mean, squared deviations),
 * combined pairwise in a fixed order (run-to-run identical; equal to a two-pass
 * f64 evaluation to about 1e-15 relative).  ws: nm_stats_workspace(R, K) bytes. */
size_t nm_stats_workspace(int64_t R, int64_t K);
nm_status nm_score_stats(const float* S, int64_t R, int64_t K, int64_t lds, double* stats,
                         void* ws, size_t ws_bytes, nm_stream_t stream);

/* Soft gate and annealing to a hard N:M mask ("SparseForge", Methodology 2
 * and 3).  With z = (s - mean)/std (z = 0 when std == 0), for t = 0..steps-1:
 *   T_t = T0 * rho^t,  beta_t = t/(steps-1),  g_t = sigmoid(z / T_t)
 *   (f32, hardware 2^x and reciprocal: about 1e-7 relative),
 *   m_t = (1 - beta_t) g_t + beta_t h,   h = top-N of s per group,
 *   lmid[t] = sum m_t (1 - m_t)   (summed over 8 consecutive scores in f32, then
 *   in f64 in a fixed order).
 * The final projection keeps the top-N of m_{steps-1} per group -> hard_mask.
 * m (nullable): m_t of step t = m_step (0 <= m_step < steps) as f32 [R, K] (ldf);
 * m_step = steps-1 gives the last blend, which equals h because beta = 1 there,
 * an earlier step shows the temperature sigmoid itself.  stats: device [2] from
 * nm_score_stats.  lmid: device f64 [steps].  Requires K % M == 0,
 * 1 <= steps <= 64.  ws: nm_gate_workspace(R, K, steps) bytes. */
size_t nm_gate_workspace(int64_t R, int64_t K, int steps);
nm_status nm_gate(const float* S, int64_t R, int64_t K, int64_t lds, const double* stats,
                  int N, int M, float T0, float rho, int steps, int m_step,
                  float* m, int64_t ldf, uint8_t* hard_mask, int64_t ldm, double* lmid,
                  void* ws, size_t ws_bytes, nm_stream_t stream);

/* ---------------------------------------------------------------- mask
 * N:M top-N selection ("Sparse-BitNet", sections 1-2: keep the N largest of
 * every M consecutive weights; "SparseForge", Methodology 3: the hard target is
 * the top-N per group).  Ties go to the lower index, NaN ranks lowest, -0 equals
 * +0; exactly N bits are set per group.  S: [R, K] f32 (lds).
 * Supported: M in {4, 8}, 1 <= N < M, K % M == 0. */
nm_status nm_mask(const float* S, int64_t R, int64_t K, int64_t lds, int N, int M,
                  uint8_t* mask, int64_t ldm, nm_stream_t stream);

/* ---------------------------------------------------------------- pack
 * Pack kept values and in-group positions (the compressed storage of an N:M
 * weight; "SlideSparse", section 2C: weights are packed once, off the request
 * path).  For each group the first N set mask bits (ascending) are kept;
 * groups with fewer bits are padded with value 0 at the smallest unused
 * positions.  W: [R, K] (ldw) of dtype wdt; vals: [R, ldv] of dtype vdt
 * (f32 -> bf16 rounds to nearest even; otherwise the dtype must match);
 * idx: [R, ldi] uint32 words.  Supported: M in {4, 8}, 1 <= N < M.
 * flags: 0 or NM_FLAG_VALIDATE. */
nm_status nm_pack(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw,
                  const uint8_t* mask, int64_t ldm, int N, int M, nm_dtype vdt,
                  void* vals, int64_t ldv, uint32_t* idx, int64_t ldi, unsigned flags,
                  nm_stream_t stream);

/* The gate/anneal of nm_gate and the packing of W under its hard mask (nm_pack
 * of hard_mask) in one call ("SparseForge", Methodology 3: the anneal ends in
 * the hard top-N target, the mask the compressed weight is then stored with).
 * S, stats, N, M, T0, rho, steps, m_step, m, hard_mask, lmid and the workspace
 * (nm_gate_workspace(R, K, steps) bytes) as in nm_gate; W [R, K] (ldw) of dtype
 * wdt, vals [R, ldv] of dtype vdt and idx [R, ldi] as in nm_pack.  Every output
 * is bit for bit that of nm_gate followed by nm_pack on the same stream.  For
 * 2:4 with the default 8 steps, bf16 W and vals, K a multiple of 32, 16-byte
 * aligned S, W and m rows and 8-byte aligned vals rows, one pass reads S and W
 * once (the pack rides along the gate's vector-bound pass); otherwise the two
 * kernels run one after the other.  No input may overlap an output or the
 * workspace, nor outputs each other (NM_ERR_ALIAS). */
nm_status nm_gate_pack(const float* S, int64_t R, int64_t K, int64_t lds, const double* stats,
                       int N, int M, float T0, float rho, int steps, int m_step,
                       float* m, int64_t ldf, uint8_t* hard_mask, int64_t ldm, double* lmid,
                       const void* W, nm_dtype wdt, int64_t ldw, nm_dtype vdt, void* vals, int64_t ldv,
                       uint32_t* idx, int64_t ldi, void* ws, size_t ws_bytes, nm_stream_t stream);

/* Fused score -> top-N mask -> pack in one pass over the weight.  The score is
 * taken from Wsc (dtype sdt, lds_ elements; HESSIAN with H/ldh/eps as in
 * nm_score, or MAGNITUDE), the packed values from Wv (dtype wdt, ldwv), which
 * may be the same tensor.  Distinct tensors give "quantise then mask"
 * ("Sparse-BitNet", section 2): the mask comes from high-precision master
 * weights and is applied to their ternary code.  mask may be NULL. */
nm_status nm_prune_pack(const void* Wsc, nm_dtype sdt, int64_t ldsc, const float* H, int64_t ldh,
                        float eps, nm_score_mode mode,
                        const void* Wv, nm_dtype wdt, int64_t ldwv, int64_t R, int64_t K, int N, int M,
                        uint8_t* mask, int64_t ldm, nm_dtype vdt, void* vals, int64_t ldv,
                        uint32_t* idx, int64_t ldi, nm_stream_t stream);

/* ---------------------------------------------------------------- slide
 * Sliding-window decomposition ("SlideSparse", section 2A): every 2N-wide group
 * with at most 2N-2 kept positions is covered by N-1 windows of width 4 and
 * stride 2 (window w covers positions 2w..2w+3), each a 2:4 group of the
 * lifted weight of width K' = (2 - 2/N) K.  Kept positions (first 2N-2 set
 * mask bits) are visited in ascending order and assigned to the earliest
 * covering window with a free slot; windows are padded with value 0 at their
 * smallest unused positions.  Output: lifted 2:4 vals [R, ldv] (ldv >= K'/2)
 * and idx [R, ldi] (ldi >= K'/32).  Supported: 2 <= Ns <= 8, K % (2 Ns) == 0.
 * Positions beyond a window's capacity (masks with more than 2N-2 bits in a
 * group) are dropped; NM_FLAG_VALIDATE in flags reports such groups instead. */
nm_status nm_slide_decompose(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw,
                             const uint8_t* mask, int64_t ldm, int Ns, nm_dtype vdt,
                             void* vals, int64_t ldv, uint32_t* idx, int64_t ldi, unsigned flags,
                             nm_stream_t stream);

/* Fused (2Ns-2):2Ns mask selection and slide decomposition: top-(2Ns-2) of
 * every 2Ns by the score of Wsc (as nm_prune_pack), then the decomposition of
 * Wv under that mask.  mask may be NULL.  (The fused calls select exactly N, or
 * 2N-2, positions per group themselves, so they take no validation flag.) */
nm_status nm_prune_slide(const void* Wsc, nm_dtype sdt, int64_t ldsc, const float* H, int64_t ldh,
                         float eps, nm_score_mode mode,
                         const void* Wv, nm_dtype wdt, int64_t ldwv, int64_t R, int64_t K, int Ns,
                         uint8_t* mask, int64_t ldm, nm_dtype vdt, void* vals, int64_t ldv,
                         uint32_t* idx, int64_t ldi, nm_stream_t stream);

/* Online step of the slide path ("SlideSparse", sections 2B-2C: the
 * activation lift is an index remap fused into the per-token quantisation
 * kernel, ahead of the sparse GEMM; INT8 and FP8 are among its precisions).
 * Token row m of X (bf16 [Mtok, K], ldx), all in f32 with one rounding per
 * operation (the quotients decide the codes):
 *   qdt == NM_I8:  x_scale[m] = max_k |X[m,k]| / 127,
 *                  q = rint(X[m,k] / x_scale[m]) clamped to [-127, 127] (ties to even);
 *   qdt == NM_FP8: x_scale[m] = max_k |X[m,k]| / 448,
 *                  q = the e4m3 code nearest X[m,k] / x_scale[m] (ties to even; the
 *                  quotient is within 448, and is clamped to it);
 *   a zero row gives x_scale = 0 and codes 0.
 * Written lifted when Ns >= 3 ((2Ns-2):2Ns, 3 <= Ns <= 8): window w of group g
 * (Ns - 1 windows of 4 codes per group of 2Ns) is Xq[m, 4(Ns-1)g + 4w + l] =
 * q[m, 2Ns g + 2w + l] -- for Ns == 4 (6:8) Xq[m, 12g + 4w + l] = q[m, 8g + 2w + l] --
 * one byte per code, [Mtok, K' = (2 - 2/Ns) K] (ldq >= K'), the activation nm_spmm
 * multiplies with Ns = 0 over K' against a slide-decomposed weight; Ns == 0
 * writes q as is (ldq >= K).  Requires K % 8 == 0 and K % 2Ns == 0, X 16-byte
 * aligned with 16-byte row strides, Xq 4-byte (lifted) or 8-byte aligned rows.
 * x_scale: device f32 [Mtok].  Allocates nothing. */
nm_status nm_quant_lift(const void* X, nm_dtype xdt, int64_t Mtok, int64_t K, int64_t ldx, int Ns, nm_dtype qdt,
                        void* Xq, int64_t ldq, float* x_scale, nm_stream_t stream);

/* Per-tensor scale of a ternary layer: alpha = mean |W| over R x K, reduced in
 * f64 in a fixed order and rounded to f32 ("Sparse-BitNet", section 1-2:
 * 1.58-bit weights carry one high-precision scale).  W: f32, bf16, int8 or
 * int32 (not FP8).  alpha: device f32 [1].  ws: nm_stats_workspace(R, K) bytes. */
nm_status nm_absmean(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw, float* alpha,
                     void* ws, size_t ws_bytes, nm_stream_t stream);

/* ---------------------------------------------------------------- sparse GEMM
 * Structured-sparse linear layer Y = X * W_hat^T on packed weights
 * ("SlideSparse", sections 2B-2C: the lifted activation is an index remap of X;
 * the product then runs on 2:4 sparse matrix instructions).  Runs on gfx950
 * SMFMAC (the packed weight is the sparse operand).  With Ns == 4 (6:8) and up to
 * 256 tokens (bf16) or 64 (one-byte codes) the lift happens inside the product's
 * activation loads; otherwise X is lifted once into the workspace.
 *   X: [Mtok, K] (ldx elements), K the ORIGINAL input width.
 *   vals/idx: 2:4 packed weight over K (Ns == 0) or over the lifted width
 *   K' = (2 - 2/Ns) K ((2Ns-2):2Ns, 3 <= Ns <= 8), rows R;
 *   ldv >= K'/2, ldi >= ceil(K'/32).
 *   xdt/vdt: BF16/BF16 (f32 accumulation), I8/I8 (exact int32 accumulation) or
 *   FP8/FP8 (e4m3 codes; exact products, f32 accumulation).
 *   ydt: for BF16 inputs BF16 or F32; for I8 inputs I32 (raw sums), F32 or BF16;
 *   for FP8 inputs F32 or BF16.
 *   Float outputs are y = acc when x_scale == NULL and w_scale == 1, else
 *   y = (w_scale * x_scale[m]) * acc in f32 (x_scale NULL counts as 1).
 *   Requires K % 2Ns == 0 (Ns >= 3) and K' a multiple of 16 (bf16) or 32 (one-byte
 *   types), K' = K for Ns == 0 (NM_ERR_SHAPE otherwise).
 *   int8 requires K' * 127 * 127 < 2^31 so that int32 accumulation is exact.
 * ws: nm_spmm_workspace(...) bytes, 16-byte aligned (NM_ERR_ALIGN otherwise): 0 for most
 * plain 2:4 shapes; the split-K partials for few tokens on few rows (summed in split order
 * by a second kernel); the lifted activation [Mtok, K'] where the lift is not done in the
 * product.  Its contents need not be initialised, but one workspace must not serve two
 * calls that may overlap. */
size_t nm_spmm_workspace(int64_t Mtok, int64_t K, int64_t R, int Ns, nm_dtype xdt);
nm_status nm_spmm(const void* X, nm_dtype xdt, int64_t Mtok, int64_t K, int64_t ldx,
                  const void* vals, nm_dtype vdt, const uint32_t* idx, int64_t R, int64_t ldv, int64_t ldi,
                  int Ns, const float* x_scale, float w_scale, void* Y, nm_dtype ydt, int64_t ldy,
                  void* ws, size_t ws_bytes, nm_stream_t stream);

/* ---------------------------------------------------------------- no-allocation variant
 * For callers that cannot allocate device memory or pass a workspace: code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc.  nm_spmm with the
 * same arguments minus the workspace; the workspace the call needs (the split-K
 * partials and the lifted activation, nm_spmm_workspace(...) bytes) comes from a
 * library-owned static device buffer of NM_SPMM_SCRATCH_BYTES per GPU, which each GPU
 * the library runs on holds until the process ends.
 *  - A call needing more than NM_SPMM_SCRATCH_BYTES returns NM_ERR_WORKSPACE before
 *    anything is enqueued (use nm_spmm with a workspace then).
 *  - Every call on a GPU shares that GPU's buffer: calls that overlap on one GPU (on
 *    different streams, or from different host threads without ordering) race on it
 *    and must be serialised by the caller.  Nothing in it needs to start at zero.
 *  - stream must belong to the current device (NM_ERR_DEVICE otherwise).  The first
 *    call on a device looks up the buffer's address on it; no call allocates, frees or
 *    synchronises.
 * Results are bit-identical to nm_spmm's for the same arguments. */
#define NM_SPMM_SCRATCH_BYTES ((size_t)64 << 20)
nm_status nm_spmm_noalloc(const void* X, nm_dtype xdt, int64_t Mtok, int64_t K, int64_t ldx,
                          const void* vals, nm_dtype vdt, const uint32_t* idx, int64_t R, int64_t ldv,
                          int64_t ldi, int Ns, const float* x_scale, float w_scale, void* Y, nm_dtype ydt,
                          int64_t ldy, nm_stream_t stream);

/* Sparse layer with stacked low-rank adapters ("SALR", section 3: every adapter of a
 * layer, the fine-tuning one and the truncated-SVD adapter of the pruning residual of
 * section 2, is stacked along the rank so that one product serves them all):
 *   Y = X W_hat^T + u B^T,   u = bf16(X A^T)   (u rounded once to nearest even from its
 *   f32 sum; every other sum in f32, output rounded once to ydt).
 *   X: bf16 [Mtok, K] (ldx), K the original width; vals/idx: bf16 2:4 packed weight as for
 *   nm_spmm (Ns 0, or 3 <= Ns <= 8 over K' = (2 - 2/Ns) K); A: bf16 [rank, K] (lda), the stacked
 *   down-projections; B: bf16 [R, rank] (ldb), the stacked up-projections (the row-major
 *   weights of a LoRA pair of linear layers).  rank: a multiple of 8 in [8, 256].
 *   Y: [Mtok, R] (ldy), bf16 or f32.  No scales.
 *   Requires K % 16 == 0, and for Ns >= 3 K % 2Ns == 0 and K' % 16 == 0; X, vals, idx, A
 *   and B 16-byte aligned with 16-byte row strides.
 * ws: nm_spmm_lowrank_workspace(Mtok, K, R, Ns, rank) bytes, 16-byte aligned (u and its
 * K-split partials, the sparse product's own workspace as for nm_spmm, and for products
 * that are not run by the many-token kernels an f32 copy of the sparse product).
 * Allocates nothing. */
size_t nm_spmm_lowrank_workspace(int64_t Mtok, int64_t K, int64_t R, int Ns, int rank);
nm_status nm_spmm_lowrank(const void* X, int64_t Mtok, int64_t K, int64_t ldx, const void* vals, const uint32_t* idx,
                          int64_t R, int64_t ldv, int64_t ldi, int Ns, const void* A, int64_t lda, const void* B,
                          int64_t ldb, int rank, void* Y, nm_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes,
                          nm_stream_t stream);

/* Bitmap format of a pruned weight ("SALR", section 4: a bitmap of the kept positions
 * and a compact array of the kept values, with a lookup table that locates each
 * sub-block's values for the decode; any sparsity pattern, e.g. unstructured 50% or
 * (2N-2):2N without the sliding-window expansion).
 *   mask [R, ldm] bytes: the bitmap (the 1-bit mask of nm_mask: bit k%8 of byte k/8).
 *   vals [R, ldv] bf16: row r's kept values in column order at positions 0 .. nnz_r - 1
 *     (a kept value at position >= ldv is not stored and reads as zero; size ldv to the
 *     largest row count, offs[r, K/64]).
 *   offs [R, ldo] int32: offs[r, b] = kept values of row r before column 64 b,
 *     offs[r, K/64] = nnz_r (ldo >= K/64 + 1).
 * nm_bitmap_encode writes vals and offs from W (bf16 [R, K], ldw) and the mask.
 * Requires K % 64 == 0, W 16-byte aligned with ldw % 8 == 0, mask 8-byte aligned with
 * ldm % 8 == 0.  Allocates nothing. */
nm_status nm_bitmap_encode(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw, const uint8_t* mask,
                           int64_t ldm, void* vals, int64_t ldv, int32_t* offs, int64_t ldo, nm_stream_t stream);

/* Y = X W_hat^T with W_hat in the bitmap format above: each K step of a block's tile is
 * first rebuilt dense in LDS from the bitmap, the table and the values, then multiplied
 * with dense bf16 MFMA (f32 accumulation; the two stages of the pages' pipeline).
 *   X: bf16 [Mtok, K] (ldx, 16-byte aligned rows); vals with 16-byte aligned rows
 *   (ldv % 8 == 0); Y: [Mtok, R] bf16 or f32 (ldy), rounded once.  Requires K % 64 == 0.
 * ws: nm_spmm_bitmap_workspace(Mtok, K, R) bytes: 0 up to 4 tokens (the rows are
 * streamed, one wave per weight row); from 512 tokens a dense bf16 copy of the weight
 * (the decode then runs once, not once per token tile); f32 partials of a K split when
 * the tiles alone leave the chip short of blocks. */
size_t nm_spmm_bitmap_workspace(int64_t Mtok, int64_t K, int64_t R);
nm_status nm_spmm_bitmap(const void* X, int64_t Mtok, int64_t K, int64_t ldx, const void* vals, int64_t ldv,
                         const uint8_t* mask, int64_t ldm, const int32_t* offs, int64_t ldo, int64_t R, void* Y,
                         nm_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes, nm_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NMSPARSE_H */
