// Device helpers shared by the int8mm kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8mm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

constexpr int kQMax = 127;
constexpr float kInvQMax2 = 1.0f / 16129.0f;  // 1 / 127^2

// int8 code of v under absmax constant a: round-half-to-even of 127 v / a, and 0 when
// a == 0 ("What is 8-bit LLM quantization?", How does INT8 quantization work?: the
// stored integer is the rounded quotient by the scale, here a / 127).
// 127 * v is exact in fp32 for fp16 v (11-bit significand times a 7-bit integer);
// __fdiv_rn is the IEEE correctly rounded divide and rint rounds ties to even. For
// |v| <= a this is exactly round-half-even of the rational 127 v / a: a quotient
// that is not a tie lies at least 2^-18 |q| away from the nearest half-integer,
// farther than the 2^-24 |q| error of the rounded fp32 quotient.
__device__ __forceinline__ int quant_code(float v, float a) {
  return a == 0.0f ? 0 : static_cast<int>(__builtin_rintf(__fdiv_rn(127.0f * v, a)));
}

// Per-row reciprocal for quant_code_fast: 127 / a correctly rounded, 0 for a == 0.
__device__ __forceinline__ float quant_scale(float a) {
  return a == 0.0f ? 0.0f : __fdiv_rn(127.0f, a);
}

// quant_code without a divide per element. With r = quant_scale(a), t = v * r is
// within 127 * 2^-23 < 2^-16 of the exact quotient 127 v / a, so whenever t lies
// farther than 2^-15 from a half-integer, rint(t) is already the exact
// round-half-even; only such near-ties fall back to the correctly rounded divide.
__device__ __forceinline__ int quant_code_fast(float v, float a, float r) {
  const float t = v * r;
  const float q0 = __builtin_rintf(t);
  if (__builtin_expect(fabsf(t - q0) <= 0.5f - 0x1p-15f, 1)) return static_cast<int>(q0);
  return quant_code(v, a);
}

// Pack four codes in [-127, 127] into one little-endian dword.
__device__ __forceinline__ unsigned pack4(int a, int b, int c, int d) {
  return (static_cast<unsigned>(a) & 0xFFu) | ((static_cast<unsigned>(b) & 0xFFu) << 8) |
         ((static_cast<unsigned>(c) & 0xFFu) << 16) | (static_cast<unsigned>(d) << 24);
}

// fp32 1.5 * 2^23. For |p| < 2^22, the fused fma(x, r, kRoundMagic) rounds the exact
// product p = x r to an integer (half-even, in the adder) and leaves that integer, as
// kRoundMagic + q, in the result's low bits: its low byte is q as an int8.
constexpr float kRoundMagic = 12582912.0f;

// The two fp32 neighbours of RN(127 / a), which bracket the exact 127 / a; both 0 for
// a == 0. For a finite a > 0, RN(127 / a) is a normal float and so are its neighbours.
struct QuantBracket {
  float lo, hi;
};
__device__ __forceinline__ QuantBracket quant_bracket(float a) {
  if (a == 0.0f) return {0.0f, 0.0f};
  const unsigned r = __builtin_bit_cast(unsigned, __fdiv_rn(127.0f, a));
  return {__builtin_bit_cast(float, r - 1u), __builtin_bit_cast(float, r + 1u)};
}

// Low bytes of four dwords, packed little-endian (v_perm_b32 selects bytes of {S0, S1}:
// selector 0-3 takes S1's bytes, 4-7 S0's, 0x0c gives 0).
__device__ __forceinline__ unsigned pack_low_bytes(unsigned b0, unsigned b1, unsigned b2,
                                                   unsigned b3) {
  const unsigned lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  const unsigned hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Exact code of one half under absmax a (quant8_exact: 8 halves), for elements where the quant8_fast pair
// disagreed. With w = |x| and q1 = RNE(w * lo) (lo = quant_bracket(a).lo <= 127 / a),
// the code of w is q1 or q1 + 1; it is q1 + 1 exactly when 127 w / a > q1 + 1/2, or
// equals it with q1 odd (half-even). That comparison, 254 w against (2 q1 + 1) a, is
// made exactly: 254 w and (2 q1 + 1) a are exact in fp32 (18- and 19-bit products of
// fp16 values and small integers), and one fused multiply-add gives the sign of their
// difference. No divide; the sign of x is applied at the end.
__device__ __forceinline__ int quant_exact1(float xf, float a, float lo) {
  const float w = fabsf(xf);
  const float q1 = __builtin_fmaf(w, lo, kRoundMagic) - kRoundMagic;
  const float d = __builtin_fmaf(2.0f * q1 + 1.0f, a, -254.0f * w);
  const int qi = static_cast<int>(q1);
  const int q = qi + ((d < 0.0f || (d == 0.0f && (qi & 1))) ? 1 : 0);
  return xf < 0.0f ? -q : q;
}
__device__ __forceinline__ v2u quant8_exact(const v8h& x, float a, float lo) {
  int c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) c[e] = quant_exact1(static_cast<float>(x[e]), a, lo);
  v2u o;
  o[0] = pack4(c[0], c[1], c[2], c[3]);
  o[1] = pack4(c[4], c[5], c[6], c[7]);
  return o;
}

// Bit e set where the bracketing pair lo < 127 / a < hi rounds element e of x to two
// different integers: the elements quant_exact1 has to settle.
__device__ __forceinline__ unsigned quant8_disagreement(const v8h& x, float lo, float hi) {
  unsigned em = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float xf = static_cast<float>(x[e]);
    em |= (__builtin_fmaf(xf, lo, kRoundMagic) != __builtin_fmaf(xf, hi, kRoundMagic) ? 1u : 0u) << e;
  }
  return em;
}

// Clears the halves of v whose bit is set in drop (outlier columns: their codes are 0
// and they do not enter the row constant). Branch-free: one keep-mask per dword.
__device__ __forceinline__ void drop_halves(v8h& v, unsigned drop) {
  v4u u = __builtin_bit_cast(v4u, v);
#pragma unroll
  for (int d = 0; d < 4; ++d)
    u[d] &= ((drop >> (2 * d)) & 1u ? 0u : 0x0000ffffu) |
            ((drop >> (2 * d + 1)) & 1u ? 0u : 0xffff0000u);
  v = __builtin_bit_cast(v8h, u);
}

// Codes of 8 halves under absmax a from the bracketing pair br = quant_bracket(a).
// p_lo = x br.lo and p_hi = x br.hi bracket the exact 127 x / a, and round-half-even
// is monotonic, so where both round to the same integer that integer is the exact
// code. Returns the lower bracket's codes and sets dis != 0 where the pair disagrees
// (a value within about 2^-15 of a half-integer, or an exact tie); those groups take
// quant8_exact.
__device__ __forceinline__ v2u quant8_fast(const v8h& x, QuantBracket br, unsigned& dis) {
  unsigned b1[8], b2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float xf = static_cast<float>(x[e]);
    b1[e] = __builtin_bit_cast(unsigned, __builtin_fmaf(xf, br.lo, kRoundMagic));
    b2[e] = __builtin_bit_cast(unsigned, __builtin_fmaf(xf, br.hi, kRoundMagic));
  }
  v2u o;
  o[0] = pack_low_bytes(b1[0], b1[1], b1[2], b1[3]);
  o[1] = pack_low_bytes(b1[4], b1[5], b1[6], b1[7]);
  dis = (o[0] ^ pack_low_bytes(b2[0], b2[1], b2[2], b2[3])) |
        (o[1] ^ pack_low_bytes(b2[4], b2[5], b2[6], b2[7]));
  return o;
}

// The smallest fp16 magnitude (as bits) that is >= t, so that for every finite or
// infinite half x, |x| >= t exactly when (bits(x) & 0x7fff) >= the result.
__device__ __forceinline__ unsigned threshold_bits(float t) {
  if (!(t > 0.0f)) return 0u;
  if (t > 65504.0f) return 0x7c00u;
  const _Float16 h = static_cast<_Float16>(t);
  const unsigned b = __builtin_bit_cast(unsigned short, h);
  return static_cast<float>(h) < t ? b + 1u : b;
}

// Lane-wise max of two pairs of u16.
__device__ __forceinline__ unsigned pk_max_u16(unsigned a, unsigned b) {
  unsigned d;
  asm("v_pk_max_u16 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// Wave-wide reductions with DPP: row_shr 1, 2, 4, 8 within each row of 16 lanes (lanes
// shifted in from outside the row read 0, the identity here), then row_bcast15 (lane 15
// of rows 0 and 2 into rows 1 and 3) and row_bcast31 (lane 31 into rows 2 and 3).
// After these steps lane i holds the reduction over lanes 0..i.
template <typename Op>
__device__ __forceinline__ int wave_scan_dpp(int v, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false));
  return v;
}
// Inclusive prefix sum over the 64 lanes (lane i: sum of lanes 0..i).
__device__ __forceinline__ int wave_prefix_sum(int v) {
  return wave_scan_dpp(v, [](int a, int b) { return a + b; });
}
// Largest value over the 64 lanes, in every lane (0 is the identity: unsigned values).
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
  const int s = wave_scan_dpp(static_cast<int>(v), [](int a, int b) {
    return static_cast<int>(max(static_cast<unsigned>(a), static_cast<unsigned>(b)));
  });
  return static_cast<unsigned>(__builtin_amdgcn_readlane(s, 63));
}

// Largest magnitude (fp16 bits, two per dword) over the wave, as a float.
__device__ __forceinline__ float wave_max_half_pairs(unsigned pm) {
  const unsigned h = wave_max_u32(max(pm & 0xffffu, pm >> 16));
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(h)));
}

// Block barrier for LDS traffic only: waits for this thread's LDS operations, not for
// its outstanding global loads (__syncthreads would also drain those). The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// The int8 operand layout of the GEMM and decode kernels ("unit-tiled"): the matrix is
// cut into units of 16 rows x 64 K-bytes, each stored as 1 KB contiguous (row-major
// inside), units ordered K-fastest within a 16-row group. KS = ceil(K / 64) units per
// group; K is zero-padded to 64 * KS. A unit is exactly the 16 x 64 operand of
// v_mfma_i32_16x16x64_i8, and a 16-row group's whole K extent is contiguous.
constexpr int kUnitRows = 16, kUnitK = 64, kUnitBytes = kUnitRows * kUnitK;
__host__ __device__ __forceinline__ int unit_ks(int K) { return (K + kUnitK - 1) / kUnitK; }
__host__ __device__ __forceinline__ size_t unit_offset(int r, int k, int ks) {
  return (static_cast<size_t>(r >> 4) * ks + (k >> 6)) * kUnitBytes + (r & 15) * kUnitK + (k & 63);
}

// Raw buffer resource over [base, base + bytes). Loads whose offset lies outside
// return zeros, which the kernels use for ragged tiles instead of branches.
// bytes must be < 2^31 so that kOOB below is always out of range.
constexpr unsigned kOOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}
__device__ __forceinline__ v4u buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0);
}

}  // namespace i8mm
