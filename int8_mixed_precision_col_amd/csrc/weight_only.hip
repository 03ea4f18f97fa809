// Weight-only int8 decode: Y = X * dequant(Wq)^T with fp16 activations, no activation
// quantization and no outlier decomposition.
//
// "What is 8-bit LLM quantization?", What is special about LLM.int8()? (keeping the
// weights in 8 bits leaves the activations and the arithmetic free to stay 16-bit) and
// Does INT8 always improve speed? (at decode time the win is reading fewer weight
// bytes). This is the variant that keeps only the weight in int8: the fp16 X
// multiplies the int8 weight dequantized by its column constant, Ŵ[k, n] =
// Wq[n, k] a_w[n] / 127, with fp32 accumulation; the constant is applied once per
// output.
//
// One block per 16 RG output features (RG 16-row groups of the unit-tiled Wq; RG = 2
// where N leaves more than 256 blocks of 16, so that fewer blocks re-read X), W waves:
// 8 (16 where RG = 2). Wave w takes k-steps w, w + W, ... (64 columns each) in batches of
// kWoBatch (8; 2 where RG = 2), the batch's loads in flight together; per
// step every lane loads one 16-byte slice of the step's 1 KB weight unit and the two
// 8-column pieces of X (its token, the same columns) that the MFMAs pair with it,
// straight into registers: no staging, no barrier before the products. X loads go
// through a buffer resource, so tokens past M and columns past K read zeros without
// touching memory. The int8 bytes become exact fp16 values (1024 + (q + 128) built
// bitwise, then 1152 subtracted in packed fp16), and each step is two
// v_mfma_f32_16x16x32_f16 with the unit as the 16-row operand and 16 tokens of X as
// the other. Partials of the waves are summed in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace i8mm {

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

// XL: X staged once per block in LDS (rows of K halves, 16 bytes of padding between rows:
// conflict-free fragment reads) by DMA, 1 KB per instruction straight from global memory,
// instead of two 16-byte register loads per lane and step (half of them for tokens past
// M): a third of the vector memory instructions. Needs K a multiple of 512 (whole 1 KB
// row segments) and M x K x 2 <= kWoXLdsMax bytes.
constexpr int kWoXLdsMax = 64 << 10;

template <int RG, bool XL, int kWoWaves, int kWoBatch>
__global__ __launch_bounds__(64 * kWoWaves) void k_weight_only(WeightOnlyArgs a) {
  static_assert(kWoBatch * RG + 1 <= 15, "the X-staging wait counts loads in 4 bits");
  __shared__ float red[kWoWaves][16 * RG][17];
  extern __shared__ __attribute__((aligned(16))) char xs[];  // XL: [M][2 K + 16]
  const int K = a.K, M = a.M, N = a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16 * RG;
  const int ks = unit_ks(K);
  const int g = lane >> 4, tok = lane & 15;
  const int xstride = 2 * K + 16;
  if constexpr (XL) {
    // X rows into LDS: segment q of row m (1 KB) by one DMA instruction
    const int segs = (2 * K) >> 10;
    for (int t = wave; t < M * segs; t += kWoWaves) {
      const int m = t / segs, q = t - m * segs;
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const char*>(a.X) + static_cast<size_t>(m) * 2 * K + q * 1024 + 16 * lane,
          (__attribute__((address_space(3))) void*)(xs + m * xstride + q * 1024), 16, 0, 0);
    }
  }
  const int8_t* wunit[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r)
    wunit[r] = a.Wq + static_cast<size_t>(min(n0 / 16 + r, N / 16 - 1)) * ks * kUnitBytes +
               (lane & 15) * kUnitK + 16 * g;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, static_cast<unsigned>(M) * K * 2u);
  // byte offset of this lane's X piece at k-step s (K is a multiple of 16: a 16-column
  // piece is either inside the row or past it); out of range past M or K
  auto x_off = [&](int s) -> unsigned {
    const int k = 64 * s + 16 * g;
    return tok < M && k < K ? static_cast<unsigned>(tok * K + k) * 2u : kOOB;
  };
  v4u wf[kWoBatch][RG], x0[kWoBatch], x1[kWoBatch];
  // non-temporal weight loads: each byte is read once per call (8x4096x4096 6.12 -> 5.9 us)
  auto load_batch = [&](int base) {
#pragma unroll
    for (int j = 0; j < kWoBatch; ++j) {
      const int s = base + kWoWaves * j;
#pragma unroll
      for (int r = 0; r < RG; ++r)
        wf[j][r] = __builtin_nontemporal_load(
            reinterpret_cast<const v4u*>(wunit[r] + static_cast<size_t>(s < ks ? s : 0) * kUnitBytes));
      if constexpr (!XL) {
        const unsigned o = s < ks ? x_off(s) : kOOB;
        x0[j] = buf_load16(xr, o);
        x1[j] = buf_load16(xr, o == kOOB ? kOOB : o + 16u);
      }
    }
  };
  load_batch(wave);
  // this thread's output (token m, feature n0 + nl) and its constant, loaded early
  const int m = tid / (16 * RG), nl = tid % (16 * RG), n = n0 + nl;
  const float aw_pre = a.a_w[min(n, N - 1)];
  if constexpr (XL) {
    // the DMA of every wave has landed (this thread's, then the barrier for the others';
    // the weight loads issued after it may still be in flight)
    __builtin_amdgcn_s_waitcnt(0x0F70 | (kWoBatch * RG + 1));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  // tokens past M read row M - 1: their products land in discarded outputs
  const char* xrow = xs + min(tok, M - 1) * xstride + 32 * g;

  v4f acc[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) acc[r] = v4f{};
  for (int base = wave;;) {
#pragma unroll
    for (int j = 0; j < kWoBatch; ++j) {
      const int s = base + kWoWaves * j;
      if (s < ks) {  // wave-uniform
        if constexpr (XL) {
          x0[j] = *reinterpret_cast<const v4u*>(xrow + 128 * s);
          x1[j] = *reinterpret_cast<const v4u*>(xrow + 128 * s + 16);
        }
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          const v2u h0 = int8x4_to_half(wf[j][r][0]), h1 = int8x4_to_half(wf[j][r][1]);
          const v2u h2 = int8x4_to_half(wf[j][r][2]), h3 = int8x4_to_half(wf[j][r][3]);
          const v4u wa = {h0[0], h0[1], h1[0], h1[1]};
          const v4u wb = {h2[0], h2[1], h3[0], h3[1]};
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, wa), __builtin_bit_cast(v8h, x0[j]), acc[r], 0, 0, 0);
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, wb), __builtin_bit_cast(v8h, x1[j]), acc[r], 0, 0, 0);
        }
      }
    }
    base += kWoWaves * kWoBatch;
    if (base >= ks) break;
    load_batch(base);
  }
  // 16x16 accumulator layout: lane l, register e -> column (token) l % 16, row 4 (l / 16) + e
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][16 * r + 4 * g + e][tok] = acc[r][e];
  lds_barrier();
  if (m < M && n < N) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kWoWaves; ++w) s += red[w][nl][m];
    a.Y[static_cast<size_t>(m) * N + n] = static_cast<_Float16>(s * __fdiv_rn(aw_pre, 127.0f));
  }
}

// X is read through a buffer resource whose size must stay below 2^31 bytes.
bool weight_only_supported(int64_t M, int64_t K) {
  return M >= 1 && M <= 16 && M * K * 2 < (int64_t(1) << 31);
}

// Measured per call (HIP graphs over rotated weights): 32 features per block pays from
// 512 groups of 16 on (4 x 8192 x 8192: 14.8-15.0 against 16.2 us with 16 per block;
// 8 x 4096 x 4096: 7.0 against 6.2 us); X staged in LDS pays with many tokens (16 x 2048
// x 4096: 4.8 against 5.7 us) and costs its barrier with few (8 x 4096 x 4096: 6.45
// against 6.2 us). Waves x batch: 8 x 8 against 16 x 4 at one row group per block
// (8 x 4096 x 4096 5.62 against 5.83 us, 1 x 4096^2 4.88 against 5.02, 16 x 4096^2 6.95
// against 7.13), 16 x 2 at two (4 x 8192 x 8192 13.9 against 15.5 us; 8 x 8 17.6).
hipError_t launch_weight_only(const WeightOnlyArgs& a, hipStream_t s) {
  const int nrg = a.N / 16;
  if (nrg > 256) {
    hipLaunchKernelGGL((k_weight_only<2, false, 16, 2>), dim3((nrg + 1) / 2), dim3(64 * 16), 0, s, a);
  } else if (a.M >= 12 && a.K % 512 == 0 && static_cast<int64_t>(a.M) * a.K * 2 <= kWoXLdsMax) {
    const size_t lds = static_cast<size_t>(a.M) * (2 * a.K + 16);
    hipLaunchKernelGGL((k_weight_only<1, true, 8, 8>), dim3(nrg), dim3(64 * 8), lds, s, a);
  } else {
    hipLaunchKernelGGL((k_weight_only<1, false, 8, 8>), dim3(nrg), dim3(64 * 8), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace i8mm
