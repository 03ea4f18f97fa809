// C ABI of libint8mm.so: argument validation, workspace layout, kernel dispatch.
// Declarations and the contract of each call are in include/int8mm.h.
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <utility>
#include <vector>

#include "common.hpp"
#include "int8mm.h"
#include "launch.hpp"

namespace {

constexpr int64_t kMaxK = 133144;          // 127 * 127 * K < 2^31
constexpr int64_t kMaxMN = int64_t(1) << 24;
constexpr int64_t kMaxOutliers = 8192;     // LDS holds the ranked outlier list

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool bad_k(int64_t K) { return K < 16 || K % 16 != 0 || K > kMaxK; }
bool bad_n(int64_t N) { return N < 16 || N % 16 != 0 || N > kMaxMN; }
bool bad_m(int64_t M) { return M < 1 || M > kMaxMN; }
bool bad_outliers(int64_t mo, int64_t K) { return mo < 0 || mo > K || mo > kMaxOutliers; }
bool bad_threshold(float t) { return isnan(t) || t < 0.0f; }

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Row chunks of the outlier-mask launch: enough blocks to cover the chip.
int mask_row_chunks(int64_t M, int64_t K) {
  const int64_t strips = (K + 63) / 64;
  int64_t r = (1024 + strips - 1) / strips;
  const int64_t max_r = (M + 31) / 32;
  if (r > max_r) r = max_r;
  if (r > 64) r = 64;
  return r < 1 ? 1 : static_cast<int>(r);
}

struct Layout {
  size_t status = 0, partial = 0, a_x = 0, xq = 0, xo = 0, idx = 0, wot = 0, total = 0;
  size_t lists = 0, masks = 0, jstar = 0, gmask = 0;  // one-pass quantization's scratch
  int R = 1, o_stride = 0;
  bool fused = false;  // one pass over X and a fix-up, else the two-launch path
  int rows_per_block = 0, nblk = 0;
};

// Quantized-activation state (int8_quantize_activations): [status, count] header, the
// quantization scratch (one-pass path: the pass-1 blocks' published column lists and
// masks and the per-row candidate columns; two-launch path: the row-chunk column
// flags), a_x, unit-tiled Xq (rows padded to 16, K to 64), Xo and the ascending outlier
// column list, each 256-byte aligned. The one-call workspace (prefill) is the same
// followed by WoT, the outlier columns' weights gathered by the quantization's spare
// blocks; the quantize-once calls have none, and their GEMM epilogue dequantizes those
// weights from Wq itself.
Layout prefill_layout(int64_t M, int64_t K, int64_t max_outliers) {
  Layout L;
  size_t off = 256;
  const size_t W = (K + 31) / 32;
  const size_t m_rows = (M + 15) & ~int64_t(15);
  L.o_stride = static_cast<int>((max_outliers + 15) & ~int64_t(15));
  L.fused = i8mm::quant_fused_supported(K);
  if (L.fused) {
    i8mm::quant_fused_geometry(M, K, &L.rows_per_block, &L.nblk);
    // sized for min(M, kFusedMaxBlocks) >= nblk blocks, so that the size grows with M
    const size_t nb = size_t(M < i8mm::kFusedMaxBlocks ? M : i8mm::kFusedMaxBlocks);
    L.lists = off; off += round256(nb * (4 + i8mm::kFlagListCap) * 4);
    L.masks = off; off += round256(nb * W * 4);
    L.jstar = off; off += round256(size_t(M) * 16);
    L.gmask = off; off += round256(W * 4);
  } else {
    L.R = mask_row_chunks(M, K);
    L.partial = off; off += round256(size_t(L.R) * W * 4);
  }
  L.a_x = off;     off += round256(size_t(M) * 4);
  L.xq = off;      off += round256(m_rows * i8mm::unit_ks(int(K)) * i8mm::kUnitK);
  L.xo = off;      off += round256(size_t(M) * L.o_stride * 2);
  L.idx = off;     off += round256(size_t(max_outliers) * 4);
  L.wot = L.total = off;
  return L;
}

Layout layout(int64_t M, int64_t K, int64_t N, int64_t max_outliers) {
  if (i8mm::decode_supported(M, K)) {
    Layout L;
    L.total = 256;
    return L;
  }
  Layout L = prefill_layout(M, K, max_outliers);
  L.total = L.wot + round256(size_t(N) * L.o_stride * 2);
  return L;
}

// The weight side needs no scratch: a fixed, reserved size.
constexpr size_t kQWorkspaceBytes = 256;

// Optional event timing (int8mm_timing_enable): mode 1 brackets the main kernel of each
// call (the MFMA GEMM, the decode kernel, the weight-only kernel), mode 2 also the
// outlier-mask and row-quantization kernels. Each record is an event pair and a phase.
enum Phase { kPhaseMask = 0, kPhaseQuant = 1, kPhaseMain = 2, kPhases = 3 };
int g_timing = 0;
struct TimedLaunch {
  hipEvent_t begin, end;
  int phase;
};
std::vector<TimedLaunch> g_events;
size_t g_events_used = 0;

bool timed(int phase) { return g_timing == 2 || (g_timing == 1 && phase == kPhaseMain); }

int timing_begin(hipStream_t s, int phase = kPhaseMain) {
  if (!timed(phase)) return INT8MM_OK;
  if (g_events_used == g_events.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess) return INT8MM_E_HIP;
    if (hipEventCreate(&b) != hipSuccess) return INT8MM_E_HIP;
    g_events.push_back({a, b, 0});
  }
  g_events[g_events_used].phase = phase;
  return hipEventRecord(g_events[g_events_used].begin, s) == hipSuccess ? INT8MM_OK : INT8MM_E_HIP;
}

int timing_end(hipStream_t s, int phase = kPhaseMain) {
  if (!timed(phase)) return INT8MM_OK;
  if (hipEventRecord(g_events[g_events_used].end, s) != hipSuccess) return INT8MM_E_HIP;
  ++g_events_used;
  return INT8MM_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? INT8MM_OK : INT8MM_E_HIP; }

// Validation shared by int8_mixed_matmul and int8_mixed_matmul_noalloc (everything but
// the workspace).
int check_mixed_args(const void* X, int64_t M, int64_t K, const int8_t* Wq,
                     const float* w_absmax, int64_t N, float threshold, int64_t max_outliers,
                     const void* Y, const int32_t* acc_i32) {
  if (!X || !Wq || !w_absmax || !Y) return INT8MM_E_NULL;
  if (bad_m(M) || bad_k(K) || bad_n(N) || bad_outliers(max_outliers, K)) return INT8MM_E_SHAPE;
  if (bad_threshold(threshold)) return INT8MM_E_THRESHOLD;
  if (!aligned16(X) || !aligned16(Wq) || !aligned16(w_absmax) || !aligned16(Y) ||
      (acc_i32 && !aligned16(acc_i32)))
    return INT8MM_E_ALIGN;
  return INT8MM_OK;
}

// Activation quantization into the state at ws (layout L): the outlier column list and
// count, a_x, unit-tiled Xq and Xo, plus WoT when wot is given (the one-call path). The
// two kernels are timed as phases 0 and 1.
int quantize_into(const _Float16* x, int64_t M, int64_t K, float threshold, int64_t max_outliers,
                  char* ws, const Layout& L, const int8_t* Wq, const float* w_absmax, int64_t N,
                  _Float16* wot, hipStream_t stream) {
  int32_t* status = reinterpret_cast<int32_t*>(ws + L.status);
  int rc;
  if (L.fused) {
    i8mm::FusedQuantArgs f{};
    f.X = x; f.M = int(M); f.K = int(K); f.t = threshold;
    f.Xq = reinterpret_cast<int8_t*>(ws + L.xq);
    f.a_x = reinterpret_cast<float*>(ws + L.a_x);
    f.jstar = reinterpret_cast<int32_t*>(ws + L.jstar);
    f.lists = reinterpret_cast<int32_t*>(ws + L.lists);
    f.masks = reinterpret_cast<uint32_t*>(ws + L.masks);
    f.rows_per_block = L.rows_per_block; f.nblk = L.nblk;
    f.gmask = reinterpret_cast<uint32_t*>(ws + L.gmask);
    f.idx_out = max_outliers > 0 ? reinterpret_cast<int32_t*>(ws + L.idx) : nullptr;
    f.count_out = status + 1; f.status_out = status;
    f.max_outliers = int(max_outliers);
    f.Xo = reinterpret_cast<_Float16*>(ws + L.xo); f.o_stride = L.o_stride;
    f.Wq = Wq; f.a_w = w_absmax; f.N = int(N); f.WoT = wot;
    if ((rc = timing_begin(stream, kPhaseMask)) != INT8MM_OK) return rc;
    if (i8mm::launch_quant_pass(f, stream) != hipSuccess) return INT8MM_E_HIP;
    if ((rc = timing_end(stream, kPhaseMask)) != INT8MM_OK) return rc;
    if ((rc = timing_begin(stream, kPhaseQuant)) != INT8MM_OK) return rc;
    if (i8mm::launch_quant_fixup(f, stream) != hipSuccess) return INT8MM_E_HIP;
    return timing_end(stream, kPhaseQuant);
  }
  uint32_t* partial = reinterpret_cast<uint32_t*>(ws + L.partial);
  if ((rc = timing_begin(stream, kPhaseMask)) != INT8MM_OK) return rc;
  if (i8mm::launch_outlier_mask(x, int(M), int(K), threshold, L.R, partial, stream) != hipSuccess)
    return INT8MM_E_HIP;
  if ((rc = timing_end(stream, kPhaseMask)) != INT8MM_OK) return rc;
  i8mm::QuantRowsArgs q{};
  q.X = x; q.M = int(M); q.K = int(K);
  q.partial = partial; q.R = L.R;
  q.Xq = reinterpret_cast<int8_t*>(ws + L.xq); q.xq_tiled = 1;
  q.a_x = reinterpret_cast<float*>(ws + L.a_x);
  q.idx_out = max_outliers > 0 ? reinterpret_cast<int32_t*>(ws + L.idx) : nullptr;
  q.count_out = status + 1; q.status_out = status;
  q.max_outliers = int(max_outliers);
  q.Xo = reinterpret_cast<_Float16*>(ws + L.xo); q.o_stride = L.o_stride;
  q.Wq = Wq; q.a_w = w_absmax; q.N = int(N); q.WoT = wot;
  if ((rc = timing_begin(stream, kPhaseQuant)) != INT8MM_OK) return rc;
  if (i8mm::launch_quant_rows(q, stream) != hipSuccess) return INT8MM_E_HIP;
  return timing_end(stream, kPhaseQuant);
}

// The whole decomposed product into a workspace of layout(M, K, N, max_outliers).total
// bytes (arguments already validated).
int run_mixed(const void* X, int64_t M, int64_t K, const int8_t* Wq, const float* w_absmax,
              int64_t N, float threshold, int64_t max_outliers, void* Y, void* workspace,
              int32_t* acc_i32, hipStream_t stream);

constexpr size_t kNoAllocScratchBytes = INT8MM_NOALLOC_SCRATCH_BYTES;
static_assert(kNoAllocScratchBytes % 256 == 0, "scratch size");

}  // namespace

// Scratch of int8_mixed_matmul_noalloc: a file-scope device array, one copy per GPU the
// library runs on, held until the process ends. Host code never uses its name as an
// address (on the host it is only a stand-in for the symbol): each device's address is
// looked up once with hipGetSymbolAddress, with that device current, and kept below.
static __device__ __attribute__((aligned(256))) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch` (resolved on the first call on the device).
int device_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return INT8MM_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return INT8MM_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return INT8MM_OK;
}

}  // namespace

extern "C" {

int int8_prepare_weight(const void* W, int64_t K, int64_t N, int w_layout, int8_t* Wq,
                        float* w_absmax, hipStream_t stream) {
  if (!W || !Wq || !w_absmax) return INT8MM_E_NULL;
  if (bad_k(K) || bad_n(N) || (w_layout != 0 && w_layout != 1)) return INT8MM_E_SHAPE;
  if (!aligned16(W) || !aligned16(Wq) || !aligned16(w_absmax)) return INT8MM_E_ALIGN;
  return hip_status(i8mm::launch_prepare_weight(static_cast<const _Float16*>(W), int(K), int(N),
                                                w_layout, Wq, w_absmax, stream));
}

int int8_tile_weight(const int8_t* Wq_nk, int64_t K, int64_t N, int8_t* Wq, hipStream_t stream) {
  if (!Wq_nk || !Wq) return INT8MM_E_NULL;
  if (bad_k(K) || bad_n(N)) return INT8MM_E_SHAPE;
  if (!aligned16(Wq_nk) || !aligned16(Wq)) return INT8MM_E_ALIGN;
  return hip_status(i8mm::launch_tile_weight(Wq_nk, int(K), int(N), Wq, stream));
}

int int8_quant_rows(const void* X, int64_t M, int64_t K, float threshold, int8_t* Xq,
                    float* x_absmax, uint32_t* outlier_mask, int32_t* outlier_idx,
                    int32_t* n_outliers, int64_t max_outliers, hipStream_t stream) {
  if (!X || !Xq || !x_absmax || !outlier_mask || !n_outliers) return INT8MM_E_NULL;
  if (max_outliers > 0 && !outlier_idx) return INT8MM_E_NULL;
  if (bad_m(M) || bad_k(K) || bad_outliers(max_outliers, K)) return INT8MM_E_SHAPE;
  if (bad_threshold(threshold)) return INT8MM_E_THRESHOLD;
  if (!aligned16(X) || !aligned16(Xq) || !aligned16(x_absmax) || !aligned16(outlier_mask) ||
      !aligned16(n_outliers) || (outlier_idx && !aligned16(outlier_idx)))
    return INT8MM_E_ALIGN;
  const _Float16* x = static_cast<const _Float16*>(X);
  // the column flags of mask_row_chunks(M, K) row chunks, merged into the caller's mask
  hipError_t e = i8mm::launch_outlier_mask_merged(x, int(M), int(K), threshold,
                                                  mask_row_chunks(M, K), outlier_mask, stream);
  if (e != hipSuccess) return INT8MM_E_HIP;
  i8mm::QuantRowsArgs q{};
  q.X = x; q.M = int(M); q.K = int(K);
  q.partial = outlier_mask; q.R = 1;
  q.Xq = Xq; q.xq_tiled = 0; q.a_x = x_absmax;
  q.idx_out = max_outliers > 0 ? outlier_idx : nullptr;
  q.count_out = n_outliers; q.status_out = nullptr;
  q.max_outliers = int(max_outliers);
  return hip_status(i8mm::launch_quant_rows(q, stream));
}

size_t int8_prepared_weight_bytes(int64_t K, int64_t N) {
  if (bad_k(K) || bad_n(N)) return 0;
  return static_cast<size_t>(N) * i8mm::unit_ks(int(K)) * i8mm::kUnitK;
}

size_t int8_mixed_matmul_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t max_outliers) {
  if (bad_m(M) || bad_k(K) || bad_n(N) || bad_outliers(max_outliers, K)) return 0;
  return layout(M, K, N, max_outliers).total;
}

int int8_mixed_matmul_is_decode(int64_t M, int64_t K) {
  return i8mm::decode_supported(M, K) ? 1 : 0;
}

int int8_mixed_matmul(const void* X, int64_t M, int64_t K, const int8_t* Wq,
                      const float* w_absmax, int64_t N, float threshold, int64_t max_outliers,
                      void* Y, void* workspace, size_t workspace_bytes, int32_t* acc_i32,
                      hipStream_t stream) {
  if (!workspace) return INT8MM_E_NULL;
  int rc = check_mixed_args(X, M, K, Wq, w_absmax, N, threshold, max_outliers, Y, acc_i32);
  if (rc != INT8MM_OK) return rc;
  if (!aligned16(workspace)) return INT8MM_E_ALIGN;
  if (workspace_bytes < layout(M, K, N, max_outliers).total) return INT8MM_E_WORKSPACE;
  return run_mixed(X, M, K, Wq, w_absmax, N, threshold, max_outliers, Y, workspace, acc_i32,
                   stream);
}

int int8_mixed_matmul_noalloc(const void* X, int64_t M, int64_t K, const int8_t* Wq,
                              const float* w_absmax, int64_t N, float threshold,
                              int64_t max_outliers, void* Y, int32_t* acc_i32,
                              hipStream_t stream) {
  int rc = check_mixed_args(X, M, K, Wq, w_absmax, N, threshold, max_outliers, Y, acc_i32);
  if (rc != INT8MM_OK) return rc;
  if (layout(M, K, N, max_outliers).total > kNoAllocScratchBytes) return INT8MM_E_SCRATCH;
  void* ws = nullptr;
  if ((rc = device_scratch(&ws)) != INT8MM_OK) return rc;
  return run_mixed(X, M, K, Wq, w_absmax, N, threshold, max_outliers, Y, ws, acc_i32, stream);
}

}  // extern "C"

namespace {

int run_mixed(const void* X, int64_t M, int64_t K, const int8_t* Wq, const float* w_absmax,
              int64_t N, float threshold, int64_t max_outliers, void* Y, void* workspace,
              int32_t* acc_i32, hipStream_t stream) {
  const Layout L = layout(M, K, N, max_outliers);
  char* ws = static_cast<char*>(workspace);
  int32_t* status = reinterpret_cast<int32_t*>(ws + L.status);
  const _Float16* x = static_cast<const _Float16*>(X);
  _Float16* y = static_cast<_Float16*>(Y);
  int rc;

  if (i8mm::decode_supported(M, K)) {
    i8mm::DecodeArgs d{};
    d.X = x; d.M = int(M); d.K = int(K); d.t = threshold;
    d.Wq = Wq; d.a_w = w_absmax; d.N = int(N);
    d.max_outliers = int(max_outliers);
    d.Y = y; d.acc_out = acc_i32; d.status = status;
    if ((rc = timing_begin(stream)) != INT8MM_OK) return rc;
    if (i8mm::launch_decode(d, stream) != hipSuccess) return INT8MM_E_HIP;
    return timing_end(stream);
  }

  float* a_x = reinterpret_cast<float*>(ws + L.a_x);
  int8_t* xq = reinterpret_cast<int8_t*>(ws + L.xq);
  _Float16* xo = reinterpret_cast<_Float16*>(ws + L.xo);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + L.idx);
  _Float16* wot = reinterpret_cast<_Float16*>(ws + L.wot);
  if ((rc = quantize_into(x, M, K, threshold, max_outliers, ws, L, Wq, w_absmax, N, wot,
                          stream)) != INT8MM_OK)
    return rc;

  i8mm::GemmArgs g{};
  g.Wq = Wq; g.Xq = xq; g.M = int(M); g.N = int(N); g.K = int(K);
  g.a_x = a_x; g.a_w = w_absmax;
  g.Xo = xo; g.WoT = wot; g.idx = idx; g.o_stride = L.o_stride;
  g.count = status + 1; g.max_outliers = int(max_outliers);
  g.Y = y; g.acc_out = acc_i32;
  if ((rc = timing_begin(stream)) != INT8MM_OK) return rc;
  if (i8mm::launch_gemm(g, stream) != hipSuccess) return INT8MM_E_HIP;
  return timing_end(stream);
}

}  // namespace

extern "C" {

size_t int8_quant_state_bytes(int64_t M, int64_t K, int64_t max_outliers) {
  if (bad_m(M) || bad_k(K) || bad_outliers(max_outliers, K)) return 0;
  return prefill_layout(M, K, max_outliers).total;
}

int int8_quant_state_layout(int64_t M, int64_t K, int64_t max_outliers, int64_t out[6]) {
  if (!out) return INT8MM_E_NULL;
  if (bad_m(M) || bad_k(K) || bad_outliers(max_outliers, K)) return INT8MM_E_SHAPE;
  const Layout L = prefill_layout(M, K, max_outliers);
  out[0] = int64_t(L.a_x);
  out[1] = int64_t(L.xq);
  out[2] = int64_t(L.xo);
  out[3] = int64_t(L.idx);
  out[4] = int64_t(L.status) + 4;
  out[5] = L.o_stride;
  return INT8MM_OK;
}

size_t int8_mixed_matmul_q_workspace_bytes(int64_t N, int64_t max_outliers) {
  if (bad_n(N) || max_outliers < 0 || max_outliers > kMaxOutliers) return 0;
  return kQWorkspaceBytes;
}

int int8_quantize_activations(const void* X, int64_t M, int64_t K, float threshold,
                              int64_t max_outliers, void* state, size_t state_bytes,
                              hipStream_t stream) {
  if (!X || !state) return INT8MM_E_NULL;
  if (bad_m(M) || bad_k(K) || bad_outliers(max_outliers, K)) return INT8MM_E_SHAPE;
  if (bad_threshold(threshold)) return INT8MM_E_THRESHOLD;
  if (!aligned16(X) || !aligned16(state)) return INT8MM_E_ALIGN;
  const Layout L = prefill_layout(M, K, max_outliers);
  if (state_bytes < L.total) return INT8MM_E_WORKSPACE;
  return quantize_into(static_cast<const _Float16*>(X), M, K, threshold, max_outliers,
                       static_cast<char*>(state), L, nullptr, nullptr, 0, nullptr, stream);
}

int int8_mixed_matmul_q(const void* state, int64_t M, int64_t K, int64_t max_outliers,
                        const int8_t* Wq, const float* w_absmax, int64_t N, void* Y,
                        void* workspace, size_t workspace_bytes, int32_t* acc_i32,
                        hipStream_t stream) {
  if (!state || !Wq || !w_absmax || !Y || !workspace) return INT8MM_E_NULL;
  if (bad_m(M) || bad_k(K) || bad_n(N) || bad_outliers(max_outliers, K)) return INT8MM_E_SHAPE;
  if (!aligned16(state) || !aligned16(Wq) || !aligned16(w_absmax) || !aligned16(Y) ||
      !aligned16(workspace) || (acc_i32 && !aligned16(acc_i32)))
    return INT8MM_E_ALIGN;
  if (workspace_bytes < int8_mixed_matmul_q_workspace_bytes(N, max_outliers))
    return INT8MM_E_WORKSPACE;
  const Layout L = prefill_layout(M, K, max_outliers);
  const char* st = static_cast<const char*>(state);
  const int32_t* status = reinterpret_cast<const int32_t*>(st + L.status);
  i8mm::GemmArgs g{};
  g.Wq = Wq; g.Xq = reinterpret_cast<const int8_t*>(st + L.xq); g.M = int(M); g.N = int(N);
  g.K = int(K);
  g.a_x = reinterpret_cast<const float*>(st + L.a_x); g.a_w = w_absmax;
  g.Xo = reinterpret_cast<const _Float16*>(st + L.xo);
  g.idx = reinterpret_cast<const int32_t*>(st + L.idx); g.o_stride = L.o_stride;
  g.count = status + 1; g.max_outliers = int(max_outliers);
  g.Y = static_cast<_Float16*>(Y); g.acc_out = acc_i32;
  int rc;
  if ((rc = timing_begin(stream)) != INT8MM_OK) return rc;
  if (i8mm::launch_gemm(g, stream) != hipSuccess) return INT8MM_E_HIP;
  return timing_end(stream);
}

size_t int8_mixed_matmul_q_grouped_workspace_bytes(int64_t G, const int64_t* N,
                                                    int64_t max_outliers) {
  if (G < 1 || G > i8mm::kMaxGroups || !N) return 0;
  size_t total = 0;
  for (int64_t q = 0; q < G; ++q) {
    const size_t b = int8_mixed_matmul_q_workspace_bytes(N[q], max_outliers);
    if (b == 0) return 0;
    total += b;
  }
  return total;
}

int int8_mixed_matmul_q_grouped(const void* state, int64_t M, int64_t K, int64_t max_outliers,
                                int64_t G, const int8_t* const* Wq, const float* const* w_absmax,
                                const int64_t* N, void* const* Y, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (!state || !Wq || !w_absmax || !N || !Y || !workspace) return INT8MM_E_NULL;
  if (G < 1 || G > i8mm::kMaxGroups) return INT8MM_E_SHAPE;
  for (int64_t q = 0; q < G; ++q)
    if (!Wq[q] || !w_absmax[q] || !Y[q]) return INT8MM_E_NULL;
  if (bad_m(M) || bad_k(K) || bad_outliers(max_outliers, K)) return INT8MM_E_SHAPE;
  for (int64_t q = 0; q < G; ++q)
    if (bad_n(N[q])) return INT8MM_E_SHAPE;
  if (!aligned16(state) || !aligned16(workspace)) return INT8MM_E_ALIGN;
  for (int64_t q = 0; q < G; ++q)
    if (!aligned16(Wq[q]) || !aligned16(w_absmax[q]) || !aligned16(Y[q])) return INT8MM_E_ALIGN;
  if (workspace_bytes < int8_mixed_matmul_q_grouped_workspace_bytes(G, N, max_outliers))
    return INT8MM_E_WORKSPACE;
  const Layout L = prefill_layout(M, K, max_outliers);
  const char* st = static_cast<const char*>(state);
  const int32_t* status = reinterpret_cast<const int32_t*>(st + L.status);
  i8mm::GroupedGemmArgs ga{};
  i8mm::GemmArgs& g = ga.base;
  g.Xq = reinterpret_cast<const int8_t*>(st + L.xq); g.M = int(M); g.K = int(K);
  g.a_x = reinterpret_cast<const float*>(st + L.a_x);
  g.Xo = reinterpret_cast<const _Float16*>(st + L.xo);
  g.idx = reinterpret_cast<const int32_t*>(st + L.idx); g.o_stride = L.o_stride;
  g.count = status + 1; g.max_outliers = int(max_outliers); g.acc_out = nullptr;
  ga.G = int(G);
  for (int64_t q = 0; q < G; ++q) {
    ga.Wq[q] = Wq[q]; ga.a_w[q] = w_absmax[q];
    ga.Y[q] = static_cast<_Float16*>(Y[q]); ga.N[q] = int(N[q]);
  }
  int rc;
  if ((rc = timing_begin(stream)) != INT8MM_OK) return rc;
  if (i8mm::launch_gemm_grouped(ga, stream) != hipSuccess) return INT8MM_E_HIP;
  return timing_end(stream);
}

int int8_weight_only_matmul(const void* X, int64_t M, int64_t K, const int8_t* Wq,
                            const float* w_absmax, int64_t N, void* Y, hipStream_t stream) {
  if (!X || !Wq || !w_absmax || !Y) return INT8MM_E_NULL;
  if (bad_m(M) || bad_k(K) || bad_n(N) || !i8mm::weight_only_supported(M, K)) return INT8MM_E_SHAPE;
  if (!aligned16(X) || !aligned16(Wq) || !aligned16(w_absmax) || !aligned16(Y)) return INT8MM_E_ALIGN;
  i8mm::WeightOnlyArgs a{};
  a.X = static_cast<const _Float16*>(X); a.M = int(M); a.K = int(K);
  a.Wq = Wq; a.a_w = w_absmax; a.N = int(N); a.Y = static_cast<_Float16*>(Y);
  int rc;
  if ((rc = timing_begin(stream)) != INT8MM_OK) return rc;
  if (i8mm::launch_weight_only(a, stream) != hipSuccess) return INT8MM_E_HIP;
  return timing_end(stream);
}

int int8mm_read_status(const void* workspace, int32_t* n_outliers, hipStream_t stream) {
  if (!workspace) return INT8MM_E_NULL;
  if (hipStreamSynchronize(stream) != hipSuccess) return INT8MM_E_HIP;
  int32_t h[2] = {0, 0};
  if (hipMemcpy(h, workspace, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return INT8MM_E_HIP;
  if (n_outliers) *n_outliers = h[1];
  return h[0];
}

const char* int8mm_strerror(int code) {
  switch (code) {
    case INT8MM_OK: return "ok";
    case INT8MM_E_NULL: return "a required pointer is NULL";
    case INT8MM_E_SHAPE: return "bad shape: need M >= 1, K and N multiples of 16 (>= 16), "
                                "K <= 133144, M and N <= 2^24, 0 <= max_outliers <= min(K, 8192), "
                                "layout 0 or 1";
    case INT8MM_E_ALIGN: return "a pointer is not 16-byte aligned";
    case INT8MM_E_THRESHOLD: return "threshold is NaN or negative";
    case INT8MM_E_WORKSPACE: return "workspace smaller than int8_mixed_matmul_workspace_bytes()";
    case INT8MM_E_HIP: return "HIP runtime error or failed kernel launch";
    case INT8MM_E_TOO_MANY_OUTLIERS: return "more outlier columns than max_outliers (Y is NaN)";
    case INT8MM_E_SCRATCH: return "shape needs more than the allocation-free call's fixed "
                                  "scratch (INT8MM_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown int8mm status code";
  }
}

int int8mm_timing_enable(int mode) {
  if (mode < 0 || mode > 2) return INT8MM_E_SHAPE;
  g_timing = mode;
  return INT8MM_OK;
}

int int8mm_timing_read_phases(double* ms, int64_t* launches) {
  if (!ms || !launches) return INT8MM_E_NULL;
  for (int p = 0; p < kPhases; ++p) {
    ms[p] = 0.0;
    launches[p] = 0;
  }
  for (size_t i = 0; i < g_events_used; ++i) {
    if (hipEventSynchronize(g_events[i].end) != hipSuccess) return INT8MM_E_HIP;
    float t = 0.0f;
    if (hipEventElapsedTime(&t, g_events[i].begin, g_events[i].end) != hipSuccess)
      return INT8MM_E_HIP;
    ms[g_events[i].phase] += t;
    ++launches[g_events[i].phase];
  }
  g_events_used = 0;
  return INT8MM_OK;
}

int int8mm_timing_read(double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return INT8MM_E_NULL;
  double ms[kPhases];
  int64_t n[kPhases];
  const int rc = int8mm_timing_read_phases(ms, n);
  if (rc != INT8MM_OK) return rc;
  *total_ms = ms[kPhaseMain];
  *launches = n[kPhaseMain];
  return INT8MM_OK;
}

}  // extern "C"
