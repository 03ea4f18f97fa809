// Weight-only int8 decode: Y = X * dequant(Wq)^T with fp16 activations, no activation
// quantization and no outlier decomposition.
//
// "What is 8-bit LLM quantization?", What is special about LLM.int8()?: 8-bit weight
// storage does not imply that every activation or operation is INT8; and Does INT8
// always improve speed?: for the decoding workload the gain is the smaller weight
// stream. This is the variant that keeps only the weight in int8: the fp16 X
// multiplies the int8 weight dequantized by its column constant, Ŵ[k, n] =
// Wq[n, k] a_w[n] / 127, with fp32 accumulation; the constant is applied once per
// output.
//
// One block per 16 output features (one 16-row group of the unit-tiled Wq), 16 waves.
// X is staged in LDS first (its loads go out before the weight stream). Wave w takes
// k-steps w, w + 16, ... (64 columns each) in batches of kWoBatch: every
// weight load reads one whole 1 KB unit, the int8 bytes become exact fp16 values
// (1024 + (q + 128) built bitwise, then 1152 subtracted in packed fp16), and each
// step is two v_mfma_f32_16x16x32_f16 with the unit as the 16-row operand and 16
// tokens of X (zero past M) as the other. Partials of the waves are summed in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace i8mm {

constexpr int kWoWaves = 16, kWoBatch = 4;

// 4 int8 codes (one dword) -> 4 fp16 of the same values, as 2 dwords.
__device__ __forceinline__ v2u int8x4_to_half(unsigned d) {
  const unsigned u = d ^ 0x80808080u;  // q + 128 as unsigned bytes
  typedef _Float16 v2h __attribute__((ext_vector_type(2)));
  const v2h bias = {_Float16(1152.0f), _Float16(1152.0f)};
  // halves 0x64bb = 1024 + b; selector bytes 0-3 take u's bytes, 4-7 the constant's
  const unsigned lo = __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u);
  const unsigned hi = __builtin_amdgcn_perm(0x64646464u, u, 0x05030402u);
  v2u o;
  o[0] = __builtin_bit_cast(unsigned, __builtin_bit_cast(v2h, lo) - bias);
  o[1] = __builtin_bit_cast(unsigned, __builtin_bit_cast(v2h, hi) - bias);
  return o;
}

__global__ __launch_bounds__(64 * kWoWaves) void k_weight_only(WeightOnlyArgs a) {
  extern __shared__ __attribute__((aligned(16))) _Float16 x_s[];  // [M][K + 8]
  __shared__ float red[kWoWaves][16][17];
  const int K = a.K, M = a.M, xs = K + 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int ks = unit_ks(K);
  const int g = lane >> 4, tok = lane & 15;
  // X (small, L2-resident) is issued first and staged in LDS; the first batch of
  // weight loads goes out before X is written to LDS, so the weight stream is not
  // held up by the staging
  const int nchunk = M * (K / 8);
  constexpr int kStage = 64 * kWoWaves * kWoBatch;  // chunks of 8 halves per pass
  auto x_chunk = [&](int c) { return *reinterpret_cast<const v8h*>(a.X + static_cast<size_t>(min(c, nchunk - 1)) * 8); };
  auto x_store = [&](int c, const v8h& v) {
    if (c < nchunk) {
      const int row = c / (K / 8), col = (c - row * (K / 8)) * 8;
      *reinterpret_cast<v8h*>(x_s + row * xs + col) = v;
    }
  };
  v8h xv[kWoBatch];
#pragma unroll
  for (int j = 0; j < kWoBatch; ++j) xv[j] = x_chunk(tid + 64 * kWoWaves * j);
  __builtin_amdgcn_sched_barrier(0);  // keep every X load ahead of the weight loads

  const int8_t* wunit = a.Wq + static_cast<size_t>(n0 >> 4) * ks * kUnitBytes + (lane & 15) * kUnitK + 16 * g;
  auto load_batch = [&](int base, v4u (&wf)[kWoBatch]) {
#pragma unroll
    for (int j = 0; j < kWoBatch; ++j) {
      const int s = base + kWoWaves * j;
      wf[j] = *reinterpret_cast<const v4u*>(wunit + static_cast<size_t>(s < ks ? s : 0) * kUnitBytes);
    }
  };
  v4u wf[kWoBatch];
  load_batch(wave, wf);
  const float aw_pre = a.a_w[n0 + (tid & 15)];  // epilogue constant, loaded early
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int j = 0; j < kWoBatch; ++j) x_store(tid + 64 * kWoWaves * j, xv[j]);
  for (int c0 = kStage; c0 < nchunk; c0 += kStage) {  // only for M K > 32768
#pragma unroll
    for (int j = 0; j < kWoBatch; ++j) xv[j] = x_chunk(c0 + tid + 64 * kWoWaves * j);
#pragma unroll
    for (int j = 0; j < kWoBatch; ++j) x_store(c0 + tid + 64 * kWoWaves * j, xv[j]);
  }
  lds_barrier();

  const bool tok_ok = tok < M;
  const _Float16* xrow = x_s + min(tok, M - 1) * xs;
  v4f acc = v4f{};
  for (int base = wave;;) {
#pragma unroll
    for (int j = 0; j < kWoBatch; ++j) {
      const int s = base + kWoWaves * j;
      if (s < ks) {  // wave-uniform
        // K is a multiple of 16, so a 16-column piece is either inside the row or past it
        const int k = 64 * s + 16 * g;
        const bool ok = tok_ok && k < K;
        const int kc = k < K ? k : K - 16;
        const v8h t0 = *reinterpret_cast<const v8h*>(xrow + kc);
        const v8h t1 = *reinterpret_cast<const v8h*>(xrow + kc + 8);
        const v2u h0 = int8x4_to_half(wf[j][0]), h1 = int8x4_to_half(wf[j][1]);
        const v2u h2 = int8x4_to_half(wf[j][2]), h3 = int8x4_to_half(wf[j][3]);
        const v4u wa = {h0[0], h0[1], h1[0], h1[1]};
        const v4u wb = {h2[0], h2[1], h3[0], h3[1]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, wa), ok ? t0 : v8h{}, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, wb), ok ? t1 : v8h{}, acc, 0, 0, 0);
      }
    }
    base += kWoWaves * kWoBatch;
    if (base >= ks) break;
    load_batch(base, wf);
  }
  // 16x16 accumulator layout: lane l, register r -> column (token) l % 16, row 4 (l / 16) + r
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][4 * g + r][tok] = acc[r];
  lds_barrier();
  const int m = tid >> 4, nl = tid & 15, n = n0 + nl;
  if (m < M) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kWoWaves; ++w) s += red[w][nl][m];
    a.Y[static_cast<size_t>(m) * a.N + n] = static_cast<_Float16>(s * __fdiv_rn(aw_pre, 127.0f));
  }
}

// X is staged whole in LDS: M (K + 8) halves.
bool weight_only_supported(int64_t M, int64_t K) {
  return M >= 1 && M <= 16 && M * (K + 8) * 2 <= 128 * 1024;
}

hipError_t launch_weight_only(const WeightOnlyArgs& a, hipStream_t s) {
  const size_t lds = static_cast<size_t>(a.M) * (a.K + 8) * 2;
  hipLaunchKernelGGL(k_weight_only, dim3(a.N / 16), dim3(64 * kWoWaves), lds, s, a);
  return hipGetLastError();
}

}  // namespace i8mm
