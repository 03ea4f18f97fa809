// The int8 GEMM with the outlier fp16 product and the dequantizing epilogue, for a
// handful of token rows (M <= 64) on the multi-kernel path: the same product as
// k_gemm ("Compress your LLMs", Mixed-precision decomposition: 8-bit matrix
// multiplication for the non-outlier dimensions, 16-bit for the outlier columns; "8-bit
// Matrix Multiplication for Large Language Models", Summary & Methodology Analysis:
// dequantization by the outer product of the row and column constants), shaped for a
// weight stream. With so few rows the product is bound by reading Wq once from HBM,
// and 128 x 128 tiles would leave most of the GPU idle (N / 128 blocks) and multiply
// padding rows; here a block owns 16 RG output features and all of M, so there are
// N / (16 RG) blocks.
//
// Per block: 8 waves split the K steps (wave w takes steps w, w + 8, ...); per step a
// lane loads 16 bytes of each of the RG weight units and the G activation units (one
// 1 KB unit is exactly one 16 x 64 operand of v_mfma_i32_16x16x64_i8), in batches of
// kSkBatch steps, double-buffered in registers so that the next batch is in flight
// while this one multiplies. The waves' int32 partials are summed exactly through LDS.
// The epilogue is k_gemm's: per 16 x 16 block of (feature, token), dequantize in fp32
// as acc * (a_x * 1/127^2) * a_w, add the outlier product with v_mfma_f32_16x16x16_f16
// over the same 16-column chunks of Xo and the dequantized outlier weights in the same
// order, round once to fp16; so Y is bit-identical to k_gemm's for the same inputs.
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace i8mm {

constexpr int kSkWaves = 8, kSkThreads = 64 * kSkWaves;
constexpr int kSkBatch = 4;   // K steps per wave per load batch
constexpr int kSkMaxM = 64;

// K >= 1024 (at least two K steps per wave; below that a block is mostly fixed
// costs); up to 32 tokens, or 33..64 tokens while the weight is at most 64 MB (beyond
// that the activation units, re-read for every 16 features, cost more than the tiles'
// padding rows).
bool gemm_skinny_supported(int64_t M, int64_t N, int64_t K) {
  return K >= 1024 && M >= 1 && (M <= 32 || (M <= kSkMaxM && N * K <= (int64_t(1) << 26)));
}

// Source of the loads past a wave's share of K steps: one 16-byte line for all lanes.
__device__ __attribute__((aligned(16))) const int kSkZero[4] = {0, 0, 0, 0};

// G: token groups of 16 (M <= 16 G), RG: groups of 16 output features per block.
template <int G, int RG>
__global__ __launch_bounds__(kSkThreads) void k_gemm_skinny(GemmArgs g) {
  constexpr int NR = 16 * RG, NM = 16 * G;                   // features, tokens per block
  constexpr int OS = 24;   // staged row stride in halves (16 columns + 8 of padding)
  __shared__ int red[kSkWaves][RG * G * 256];
  __shared__ int sum_s[RG * G * 256];
  __shared__ float aw_s[NR], ax_s[NM];
  __shared__ __attribute__((aligned(16))) _Float16 wo_s[NR * OS];
  __shared__ __attribute__((aligned(16))) _Float16 xo_s[NM * OS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = g.M, N = g.N, ks = unit_ks(g.K);
  const int n0 = blockIdx.x * NR;

  // 16x16x64 operand of one unit: lane l reads row l % 16, K bytes 16 (l / 16) .. + 15
  const int lane_off = (lane & 15) * kUnitK + 16 * (lane >> 4);
  const int8_t* wrow[RG];
  const int8_t* xrow[G];
#pragma unroll
  for (int r = 0; r < RG; ++r)
    wrow[r] = g.Wq + static_cast<size_t>(min(n0 / 16 + r, N / 16 - 1)) * ks * kUnitBytes + lane_off;
#pragma unroll
  for (int q = 0; q < G; ++q)
    xrow[q] = g.Xq + static_cast<size_t>(min(q, (M - 1) / 16)) * ks * kUnitBytes + lane_off;

  // this wave's K steps: wave + 8 i for i < nmine. Loads are unconditional (a guarded
  // load becomes a branch whose join waits for every load in flight): slots past the
  // wave's share read one zero line and are not multiplied, and so do the lanes of
  // activation rows past M (their products land in discarded outputs), which spares
  // most of the activation reads when M is well below 16.
  const int nmine = ks > wave ? (ks - wave + kSkWaves - 1) / kSkWaves : 0;
  const int8_t* zero = reinterpret_cast<const int8_t*>(kSkZero);
  bool tok_in[G];
#pragma unroll
  for (int q = 0; q < G; ++q) tok_in[q] = 16 * q + (lane & 15) < M;
  v4i acc[RG][G];
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int q = 0; q < G; ++q) acc[r][q] = v4i{};
  v4i wa[kSkBatch][RG], xa[kSkBatch][G], wb[kSkBatch][RG], xb[kSkBatch][G];
  // the weight units non-temporally (each is read once per call), the activation units
  // cached (every block reads them)
  auto load = [&](v4i (&w)[kSkBatch][RG], v4i (&x)[kSkBatch][G], int i0) {
#pragma unroll
    for (int b = 0; b < kSkBatch; ++b) {
      const bool in = i0 + b < nmine;  // wave-uniform
      const size_t off = static_cast<size_t>(wave + kSkWaves * (i0 + b)) * kUnitBytes;
#pragma unroll
      for (int r = 0; r < RG; ++r)
        w[b][r] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(in ? wrow[r] + off : zero));
#pragma unroll
      for (int q = 0; q < G; ++q)
        x[b][q] = *reinterpret_cast<const v4i*>(in && tok_in[q] ? xrow[q] + off : zero);
    }
  };
  auto mma = [&](const v4i (&w)[kSkBatch][RG], const v4i (&x)[kSkBatch][G], int i0) {
#pragma unroll
    for (int b = 0; b < kSkBatch; ++b)
      if (i0 + b < nmine)  // wave-uniform
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
          for (int q = 0; q < G; ++q)
            acc[r][q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[b][r], x[b][q], acc[r][q], 0, 0, 0);
  };
  load(wa, xa, 0);
  for (int i0 = 0; i0 < nmine; i0 += 2 * kSkBatch) {  // wave-uniform trip count
    load(wb, xb, i0 + kSkBatch);
    mma(wa, xa, i0);
    load(wa, xa, i0 + 2 * kSkBatch);
    mma(wb, xb, i0 + kSkBatch);
  }

  // partials: 16x16 accumulator layout, lane l, register e -> token l % 16 of group q,
  // feature 4 (l / 16) + e of group r; block (r, q) holds [feature][token]
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        red[wave][(r * G + q) * 256 + (4 * (lane >> 4) + e) * 16 + (lane & 15)] = acc[r][q][e];
  const int count = *g.count;
  const bool overflow = count > g.max_outliers;
  const int o_pad = min((count + 15) & ~15, g.o_stride);
  const int nvalid = min(count, g.max_outliers);
  for (int t = tid; t < NR; t += kSkThreads) aw_s[t] = g.a_w[min(n0 + t, N - 1)];
  for (int t = tid; t < NM; t += kSkThreads) ax_s[t] = g.a_x[min(t, M - 1)];
  // the outlier columns s0 .. s0 + 15: the block's weight rows (gathered beforehand, or
  // dequantized from Wq) and Xo
  auto stage_outliers = [&](int s0) {
    for (int t = tid; t < (NR + NM) * 2; t += kSkThreads) {
      const int row = t >> 1, h = t & 1;
      if (row < NR)
        *reinterpret_cast<v8h*>(wo_s + row * OS + 8 * h) =
            g.WoT ? *reinterpret_cast<const v8h*>(g.WoT + static_cast<size_t>(min(n0 + row, N - 1)) * g.o_stride + s0 + 8 * h)
                  : outlier_weights(g, min(n0 + row, N - 1), s0 + 8 * h, nvalid, ks);
      else
        *reinterpret_cast<v8h*>(xo_s + (row - NR) * OS + 8 * h) = *reinterpret_cast<const v8h*>(
            g.Xo + static_cast<size_t>(min(row - NR, M - 1)) * g.o_stride + s0 + 8 * h);
    }
  };
  if (o_pad > 0) stage_outliers(0);
  __syncthreads();
  for (int t = tid; t < RG * G * 256; t += kSkThreads) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < kSkWaves; ++w) s += red[w][t];
    sum_s[t] = s;
  }
  __syncthreads();

  // epilogue: wave e < RG G takes the 16 x 16 block (features 16 (e / G) .., tokens
  // 16 (e % G) ..); 16x16 layout: lane l, register v -> token l % 16, feature
  // 4 (l / 16) + v
  const bool ep = wave < RG * G;
  const int en = ep ? wave / G : 0, em = ep ? wave % G : 0;
  const int l16 = lane & 15, lq = lane >> 4;
  const int mloc = 16 * em + l16, nloc = 16 * en + 4 * lq, n = n0 + nloc;
  v4f y;
  if (ep) {
    const float sx = ax_s[mloc] * kInvQMax2;
    const int* blk = sum_s + (en * G + em) * 256 + (4 * lq) * 16 + l16;
    v4i av;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      av[v] = blk[16 * v];
      y[v] = static_cast<float>(av[v]) * sx * aw_s[nloc + v];
    }
    if (g.acc_out && mloc < M && n < N)
      *reinterpret_cast<v4i*>(g.acc_out + static_cast<size_t>(mloc) * N + n) = av;
  }
  for (int s0 = 0; s0 < o_pad; s0 += 16) {  // block-uniform trip count
    if (s0 > 0) {
      __syncthreads();
      stage_outliers(s0);
      __syncthreads();
    }
    if (ep) {
      const v4h fa = *reinterpret_cast<const v4h*>(wo_s + (16 * en + l16) * OS + 4 * lq);
      const v4h fb = *reinterpret_cast<const v4h*>(xo_s + (16 * em + l16) * OS + 4 * lq);
      y = __builtin_amdgcn_mfma_f32_16x16x16f16(fa, fb, y, 0, 0, 0);
    }
  }
  if (ep && mloc < M && n < N) {
    v4h out;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      out[e] = overflow ? static_cast<_Float16>(__builtin_nanf("")) : static_cast<_Float16>(y[e]);
    *reinterpret_cast<v4h*>(g.Y + static_cast<size_t>(mloc) * N + n) = out;
  }
}

// Features per block: 16, or 32 / 64 where N leaves more than 2048 / 4096 blocks of
// 16 (fewer, longer blocks re-read the activation units fewer times).
hipError_t launch_gemm_skinny(const GemmArgs& g, hipStream_t s) {
  const int G = (g.M + 15) / 16;
  const int nrg = g.N / 16;
  int rg = nrg > 4096 ? 4 : nrg > 2048 ? 2 : 1;
  while (rg * G > 4) rg >>= 1;
  const dim3 grid((nrg + rg - 1) / rg), block(kSkThreads);
#define I8MM_SK(GV, RV)                                              \
  if (G == GV && rg == RV) {                                         \
    hipLaunchKernelGGL((k_gemm_skinny<GV, RV>), grid, block, 0, s, g); \
    return hipGetLastError();                                        \
  }
  I8MM_SK(1, 1) I8MM_SK(1, 2) I8MM_SK(1, 4) I8MM_SK(2, 1) I8MM_SK(2, 2) I8MM_SK(3, 1) I8MM_SK(4, 1)
#undef I8MM_SK
  return hipErrorInvalidValue;
}

}  // namespace i8mm
