/*
 * int8mm.h - C ABI of libint8mm.so: the LLM.int8() mixed-precision
 * decomposed matrix multiply on MI355X (gfx950).
 *
 * Sources (web pages on the method, cited by title and section):
 *   [Abstract]  "LLM.int8(): 8-bit Matrix Multiplication for Transformers at
 *               Scale" (mlsanity.com paper index), "Abstract (arXiv)".
 *   [Summary]   "8-bit Matrix Multiplication for Large Language Models"
 *               (legiblepapers.com), "Summary & Methodology Analysis".
 *   [Blog]      "Compress your LLMs" (samsena.com), bullets "Vector-wise
 *               quantization" and "Mixed-precision decomposition".
 *   [Explainer] "What is 8-bit LLM quantization?" (machinoai.in), "How does
 *               INT8 quantization work?".
 *
 * Notation: X fp16 [M, K] row-major activations (rows = tokens, columns =
 * feature dimensions). W fp16 weights, K input features x N output features.
 * Wq: the int8 weight in the "unit-tiled" layout the kernels read: element (n, k)
 * of the [N, K] matrix is at byte
 *     ((n / 16) * KS + k / 64) * 1024 + (n % 16) * 64 + k % 64,   KS = ceil(K / 64),
 * i.e. 16-row x 64-byte units stored contiguously, K-fastest within a group of 16
 * rows; bytes with k >= K are zero. Size: int8_prepared_weight_bytes(K, N) =
 * N * KS * 64 bytes. Codes are symmetric in
 * [-127, 127]: q = round-half-even(127 * v / a) for absmax constant a, and
 * q = 0 when a = 0. An outlier column j is one where some row has
 * |X[i, j]| >= threshold.
 *
 * Conventions shared by every call:
 *  - Every pointer argument is a DEVICE pointer on the current HIP device,
 *    owned by the caller. The library never allocates device memory, never
 *    frees, and keeps no pointer after returning. Inputs are never written;
 *    outputs are fully overwritten. Buffers must not overlap.
 *  - Every pointer must be 16-byte aligned. K and N must be multiples of 16
 *    (>= 16). 1 <= M, N <= 2^24. K <= 133144, which keeps |int32 accumulators|
 *    <= 127*127*K < 2^31. 0 <= max_outliers <= min(K, 8192).
 *  - Calls are stream-ordered and asynchronous on `stream` (0 = the null
 *    stream). They make no host synchronisation and read no device data on
 *    the host (int8mm_read_status and int8mm_timing_read excepted).
 *  - Argument errors are found on the host before any HIP call and returned
 *    synchronously (nothing is launched). A failed launch returns
 *    INT8MM_E_HIP. Inputs must be finite.
 */
#ifndef INT8MM_H_
#define INT8MM_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum int8mm_status {
  INT8MM_OK = 0,
  INT8MM_E_NULL = 1,      /* a required pointer is NULL */
  INT8MM_E_SHAPE = 2,     /* M, K, N or max_outliers outside the limits above,
                             or a bad layout flag */
  INT8MM_E_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  INT8MM_E_THRESHOLD = 4, /* threshold is NaN or negative */
  INT8MM_E_WORKSPACE = 5, /* workspace smaller than int8_mixed_matmul_workspace_bytes() */
  INT8MM_E_HIP = 6,       /* a HIP runtime call or kernel launch failed */
  INT8MM_E_TOO_MANY_OUTLIERS = 7, /* asynchronous: more outlier columns than max_outliers;
                                     reported only through int8mm_read_status */
  INT8MM_E_SCRATCH = 8    /* int8_mixed_matmul_noalloc: the shape needs more workspace
                             than INT8MM_NOALLOC_SCRATCH_BYTES */
} int8mm_status;

/*
 * Weight conversion, once per weight ([Abstract]: a 16/32-bit checkpoint is
 * converted to Int8 at load; [Blog] "Vector-wise quantization": one constant
 * per column of the weight matrix).
 *   W         fp16 weights. w_layout 0: [K, N] row-major (x @ W);
 *             w_layout 1: [N, K] row-major (the nn.Linear weight layout).
 *   Wq        out, int8_prepared_weight_bytes(K, N) bytes, unit-tiled (see the
 *             notation above): element (n, k) = q(W(k, n), w_absmax[n]).
 *   w_absmax  out, fp32 [N]: max over all K of |W(k, n)| (an exact fp16 value).
 */
int int8_prepare_weight(const void* W, int64_t K, int64_t N, int w_layout, int8_t* Wq,
                        float* w_absmax, hipStream_t stream);

/*
 * An int8 weight that is already quantized ([Abstract]: a checkpoint converted to Int8
 * is used as it is loaded; one fp32 constant per output column), handed over as the
 * plain [N, K] matrix: copies it into the unit-tiled layout the matmul calls read.
 * Layout only, no arithmetic: the caller's constants w_absmax [N] are used unchanged
 * with the result (the codes must be those of q(W, w_absmax), in [-127, 127], for the
 * product to be the method's). The unit-tiled layout is what every matmul call takes
 * in place of a plain [N, K] Wq.
 *   Wq_nk     int8 [N, K] row-major (K contiguous).
 *   Wq        out, int8_prepared_weight_bytes(K, N) bytes, unit-tiled; the K padding of
 *             each row's last unit is zero.
 * Errors: NULL pointers, K or N outside the limits above, pointers not 16-byte aligned.
 */
int int8_tile_weight(const int8_t* Wq_nk, int64_t K, int64_t N, int8_t* Wq, hipStream_t stream);

/*
 * Outlier detection plus vector-wise row quantization of the activations
 * ([Blog] "Vector-wise quantization": one constant per input row;
 * [Abstract]/[Summary]: outlier feature dimensions are isolated).
 *   X             fp16 [M, K] row-major.
 *   threshold     >= 0. +inf: no outliers. 0: every column is an outlier.
 *   Xq            out, int8 [M, K]: 0 in outlier columns, else q(X[i,j], x_absmax[i]).
 *   x_absmax      out, fp32 [M]: max |X[i, j]| over non-outlier columns j (0 if none).
 *   outlier_mask  out, uint32 [ceil(K/32)]: bit (j % 32) of word j / 32 set iff
 *                 column j is an outlier.
 *   outlier_idx   out, int32 [max_outliers] (may be NULL when max_outliers == 0):
 *                 the first min(count, max_outliers) outlier columns, ascending.
 *   n_outliers    out, int32 [1]: the true outlier count (may exceed max_outliers).
 */
int int8_quant_rows(const void* X, int64_t M, int64_t K, float threshold, int8_t* Xq,
                    float* x_absmax, uint32_t* outlier_mask, int32_t* outlier_idx,
                    int32_t* n_outliers, int64_t max_outliers, hipStream_t stream);

/* Bytes of a prepared (unit-tiled) int8 weight: N * ceil(K / 64) * 64 (0 on bad shapes). */
size_t int8_prepared_weight_bytes(int64_t K, int64_t N);

/* Bytes of workspace int8_mixed_matmul needs for this shape (0 on bad arguments). */
size_t int8_mixed_matmul_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t max_outliers);

/*
 * The decomposed product Y = dequant(Xq Wq^T) + X[:, O] W^[O, :] in fp16
 * ([Summary]: the int8 product is dequantized by the outer product of the
 * row and column constants, and the outlier and regular outputs are summed
 * into 16-bit floating-point outputs; [Blog] "Mixed-precision
 * decomposition": outlier dimensions in 16 bit, the rest in 8 bit).
 *   X, M, K       fp16 activations [M, K].
 *   Wq, w_absmax  unit-tiled int8 weight and fp32 [N] from int8_prepare_weight.
 *   threshold     outlier threshold, as for int8_quant_rows.
 *   max_outliers  capacity for outlier columns, 0 <= max_outliers <= min(K, 8192). If the
 *                 call finds more, Y is filled with fp16 NaN and the workspace
 *                 status becomes INT8MM_E_TOO_MANY_OUTLIERS.
 *   Y             out, fp16 [M, N] row-major.
 *   workspace     device scratch of at least workspace_bytes; contents on entry
 *                 are ignored. It also holds the status word of the last call.
 *   acc_i32       optional out (NULL to skip), int32 [M, N]: the exact int8
 *                 accumulators sum_k Xq[i,k] Wq[n,k], for verification.
 * Sums: int32 exact for the int8 part; the outlier part uses fp16 operands
 * (X values and Wq*w_absmax/127 rounded to fp16) with fp32 accumulation; the
 * epilogue combines both in fp32 and rounds once to fp16.
 * M <= 16 with K <= 4096, and M <= 8 with K <= 8192, run as one bandwidth-bound kernel
 * (int8_mixed_matmul_is_decode); otherwise the activation quantization (K <= 32768: one
 * pass over X, then a two-launch fix-up for the outlier column set, the rows it changes
 * and the outlier gathers; larger K: an outlier-mask launch, then row quantization with
 * the gathers) and the MFMA GEMM. The GEMM is tiled (256 x 256, 128 x 256 or 128 x 128
 * outputs per block, whichever is estimated fastest; when 256 x 256 tiles leave a partial
 * last wave, the features that fill whole waves and the rest run as two launches) or, for
 * a few tokens (M <= 32, or M <= 64 with N K <= 2^26; K >= 1024), a weight stream with
 * one block per 16-64 output features; both compute every output with the same
 * arithmetic, so Y does not depend on which one runs.
 */
int int8_mixed_matmul(const void* X, int64_t M, int64_t K, const int8_t* Wq,
                      const float* w_absmax, int64_t N, float threshold, int64_t max_outliers,
                      void* Y, void* workspace, size_t workspace_bytes, int32_t* acc_i32,
                      hipStream_t stream);

/*
 * int8_mixed_matmul without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). The call allocates nothing and frees nothing: its workspace is a
 * fixed array of INT8MM_NOALLOC_SCRATCH_BYTES in the library's device code, one copy
 * per GPU, held from the library's load until the process ends. Its address is
 * looked up on the first call on each device (make that first call outside graph
 * capture). Same kernels, same arguments and same result as int8_mixed_matmul on a
 * workspace of its own: Y and acc_i32 equal that call's bit for bit.
 *   Shapes whose int8_mixed_matmul_workspace_bytes(M, K, N, max_outliers) exceeds
 *   INT8MM_NOALLOC_SCRATCH_BYTES are rejected with INT8MM_E_SCRATCH before anything
 *   is launched (every decode shape fits; so do prefill shapes up to, for example,
 *   M x K = 2048 x 4096 with N = 16384 and 256 outlier columns).
 * Every call on one GPU shares that GPU's scratch and leaves its contents behind
 * (none of it needs to start at zero): calls that overlap in time on one GPU (two
 * streams, two host threads) race and must be serialised by the caller. The status
 * word lives in the scratch and is not readable; an outlier overflow still shows as
 * NaN in Y. Other errors as for int8_mixed_matmul.
 */
#define INT8MM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int int8_mixed_matmul_noalloc(const void* X, int64_t M, int64_t K, const int8_t* Wq,
                              const float* w_absmax, int64_t N, float threshold,
                              int64_t max_outliers, void* Y, int32_t* acc_i32,
                              hipStream_t stream);

/* 1 if int8_mixed_matmul takes the single-kernel decode path for (M, K), else 0. */
int int8_mixed_matmul_is_decode(int64_t M, int64_t K);

/*
 * The activation side once, for several weights that share the same input (the
 * projections fed by one X: [Abstract], the decomposition applies to the
 * feed-forward and attention projection layers). int8_quantize_activations runs
 * the outlier detection and row quantization of int8_mixed_matmul into `state`;
 * int8_mixed_matmul_q then runs the weight side (int8 MFMA GEMM whose epilogue
 * dequantizes the outlier columns' weights, fp16 outlier product, dequant) for one
 * weight from that state. Y equals int8_mixed_matmul's bit for bit when
 * int8_mixed_matmul takes its multi-kernel path (int8_mixed_matmul_is_decode(M, K) is
 * 0); for decode shapes the same values are reached through the GEMM instead of the
 * single decode kernel.
 *   state         device buffer of int8_quant_state_bytes(M, K, max_outliers),
 *                 written by int8_quantize_activations, read by int8_mixed_matmul_q;
 *                 it holds the status word (int8mm_read_status works on it).
 *   workspace     (int8_mixed_matmul_q) at least int8_mixed_matmul_q_workspace_bytes(N,
 *                 max_outliers) bytes, a fixed 256: reserved (the weight side needs no
 *                 scratch; the GEMM dequantizes the outlier columns' weights itself).
 * M, K, max_outliers and the threshold's outcome are those of the quantization
 * call; arguments are validated as for int8_mixed_matmul.
 */
size_t int8_quant_state_bytes(int64_t M, int64_t K, int64_t max_outliers);
/*
 * Where the quantization results sit inside a state buffer of int8_quant_state_bytes(M,
 * K, max_outliers) bytes, so that a caller can read them: on success out[] holds byte
 * offsets from the start of the state, out[0] a_x (fp32 [M], the row constants), out[1]
 * Xq (int8, unit-tiled like a prepared weight with M rows: rows padded to a multiple of
 * 16, K to a multiple of 64), out[2] Xo (fp16 [M][out[5]], the outlier columns' values
 * in rank order, zeros past the count), out[3] the ascending outlier column list
 * (int32 [max_outliers]; the first min(count, max_outliers) are valid), out[4] the
 * outlier count (int32), and out[5] is Xo's row stride in elements. Host-only: no
 * device access. Returns INT8MM_E_NULL for a null out, INT8MM_E_SHAPE for bad sizes.
 */
int int8_quant_state_layout(int64_t M, int64_t K, int64_t max_outliers, int64_t out[6]);
int int8_quantize_activations(const void* X, int64_t M, int64_t K, float threshold,
                              int64_t max_outliers, void* state, size_t state_bytes,
                              hipStream_t stream);
size_t int8_mixed_matmul_q_workspace_bytes(int64_t N, int64_t max_outliers);
int int8_mixed_matmul_q(const void* state, int64_t M, int64_t K, int64_t max_outliers,
                        const int8_t* Wq, const float* w_absmax, int64_t N, void* Y,
                        void* workspace, size_t workspace_bytes, int32_t* acc_i32,
                        hipStream_t stream);

/*
 * int8_mixed_matmul_q for G <= 8 weights at once, in one GEMM launch (for a few
 * tokens, where the weight-stream kernel fills the GPU by itself, one per weight): the weights'
 * output tiles form one grid, so projections too narrow to fill the GPU on their
 * own (Q, K, V of one layer) run side by side ([Abstract]: the attention and
 * feed-forward projection layers share the input the state was made from).
 *   G             1 <= G <= 8.
 *   Wq, w_absmax, N, Y   host arrays of G entries (read during the call, not kept):
 *                 each weight's unit-tiled int8 matrix, fp32 [N[q]] constants, output
 *                 width (multiple of 16) and fp16 output [M, N[q]].
 *   workspace     at least int8_mixed_matmul_q_grouped_workspace_bytes(G, N,
 *                 max_outliers) bytes (reserved, 256 per weight).
 * Each Y[q] equals int8_mixed_matmul_q's output for that weight bit for bit. No
 * int32 sums output. Errors as for int8_mixed_matmul_q; G out of range or a bad
 * N[q] is INT8MM_E_SHAPE, a null entry INT8MM_E_NULL.
 */
size_t int8_mixed_matmul_q_grouped_workspace_bytes(int64_t G, const int64_t* N,
                                                    int64_t max_outliers);
int int8_mixed_matmul_q_grouped(const void* state, int64_t M, int64_t K, int64_t max_outliers,
                                int64_t G, const int8_t* const* Wq, const float* const* w_absmax,
                                const int64_t* N, void* const* Y, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * Weight-only int8 product for a handful of tokens: Y = X · Ŵ with
 * Ŵ[k, n] = Wq[n, k] · w_absmax[n] / 127, no activation quantization and no
 * outlier decomposition ("What is 8-bit LLM quantization?", What is special about
 * LLM.int8()?: int8 weights may be paired with 16-bit activations and arithmetic;
 * Does INT8 always improve speed?: at decode time the gain is the smaller weight
 * stream). The comparison point for the decode path above.
 *   X, M, K       fp16 activations [M, K], 1 <= M <= 16 and M K < 2^30 (X is
 *                 read through a buffer resource, whose byte offsets are 31-bit).
 *   Wq, w_absmax  unit-tiled int8 weight and fp32 [N] from int8_prepare_weight.
 *   Y             out, fp16 [M, N] row-major.
 * Sums: the products of fp16 X and the int8 codes are exact in fp32 and accumulate
 * in fp32; each output is scaled by w_absmax[n] / 127 once and rounded to fp16.
 * Errors: as for int8_mixed_matmul (shapes outside the limits above are
 * INT8MM_E_SHAPE). No workspace.
 */
int int8_weight_only_matmul(const void* X, int64_t M, int64_t K, const int8_t* Wq,
                            const float* w_absmax, int64_t N, void* Y, hipStream_t stream);

/*
 * Synchronises `stream`, then returns the status word the last
 * int8_mixed_matmul call left in `workspace` (INT8MM_OK or
 * INT8MM_E_TOO_MANY_OUTLIERS), or INT8MM_E_HIP / INT8MM_E_NULL.
 * n_outliers (nullable) receives that call's outlier count.
 */
int int8mm_read_status(const void* workspace, int32_t* n_outliers, hipStream_t stream);

/* Static description of a status code. */
const char* int8mm_strerror(int code);

/*
 * Optional event timing, for benchmarks. int8mm_timing_enable(mode): 0 off; 1: each call
 * records a HIP event pair on its stream around its main kernels (the MFMA GEMM: one
 * launch, or two when a partial last wave of 256 x 256 tiles is split off; the decode
 * kernel; the weight-only kernel); 2: also around each of the two activation
 * quantization phases. Other modes are INT8MM_E_SHAPE. Not for calls under graph
 * capture (the events would be captured). int8mm_timing_read_phases synchronises on the
 * recorded events and returns, per phase, the summed milliseconds and the number of
 * bracketed calls since the last read: phase 0 is the pass over X (flags, provisional
 * row constants and codes; for K > 32768 the outlier-mask kernel), phase 1 the fix-up
 * (two launches: the outlier column set, then the rows it changes and the outlier
 * gathers; for K > 32768 the row-quantization kernel), phase 2 the main kernels. It then
 * starts a new period; int8mm_timing_read does the same and returns phase 2 only. Not
 * thread-safe.
 */
int int8mm_timing_enable(int mode);
int int8mm_timing_read(double* total_ms, int64_t* launches);
int int8mm_timing_read_phases(double* ms /*[3]*/, int64_t* launches /*[3]*/);

#ifdef __cplusplus
}
#endif

#endif /* INT8MM_H_ */
