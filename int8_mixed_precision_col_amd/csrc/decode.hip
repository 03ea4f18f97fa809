// Decode path: the whole decomposed product for a handful of tokens in one kernel.
//
// "What is 8-bit LLM quantization?", Does INT8 always improve speed?: for the decoding
// workload the gain comes from the smaller weights cutting memory traffic. With
// M <= 16 tokens the int8 weight stream (N x K bytes) is the whole cost, so one
// launch does every step and reads each Wq byte from HBM exactly once:
//   1. each block issues the loads of its 16 Wq rows (all K) into registers first;
//   2. while they are in flight it reads all of X (small, L2-resident): wave w owns
//      rows w, w+4, ..., lane l owns the 8-column chunks l, l+64, ...; it finds the
//      outlier columns (|X| >= t in any row), ranks them, takes each row's absmax over
//      the other columns and writes Xq into LDS. Every block repeats this for the
//      whole of X, which costs L2 reads and VALU time but no second launch and no
//      grid-wide wait;
//   3. v_mfma_i32_16x16x64_i8 with Wq rows as the 16-row operand and Xq rows as the
//      16-column operand (tokens past M are zero), K split over the 4 waves;
//   4. the four int32 partials are summed exactly through LDS; the epilogue applies
//      the outer-product dequant and adds the outlier columns' product in fp32
//      (exact fp16 X times the int8 weight dequantized by a_w / 127, both staged in
//      LDS) before the single rounding to fp16.
#include "common.hpp"
#include "launch.hpp"

namespace i8mm {

constexpr int kDecMaxM = 16, kDecMaxK = 8192, kDecMaxMK = 32768;
constexpr int kOutChunk = 64;  // outlier columns staged in LDS per epilogue pass

static int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}
static int rows_per_wave(int64_t M) { return pow2_at_least(static_cast<int>((M + 3) / 4)); }
static int chunks_per_lane(int64_t K) { return pow2_at_least(static_cast<int>((K + 511) / 512)); }

bool decode_supported(int64_t M, int64_t K) {
  return M >= 1 && M <= kDecMaxM && K <= kDecMaxK && M * K <= kDecMaxMK &&
         rows_per_wave(M) * chunks_per_lane(K) <= 32;
}

// Largest |x| of 8 halves, as fp16 magnitude bits (finite halves order like their
// bit patterns). Written with scalar AND / BFE / MAX: this compiler folds a packed
// u16 max of vector-element bit casts down to its first operand.
__device__ __forceinline__ unsigned chunk_mag_max(const v8h& v) {
  const v4u u = __builtin_bit_cast(v4u, v);
  unsigned r = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) r = max(r, max(u[i] & 0x7fffu, (u[i] >> 16) & 0x7fffu));
  return r;
}

__device__ __forceinline__ float half_bits_to_float(unsigned h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(h)));
}

// RW: rows per wave (wave w owns rows w + 4 i), CL: 8-column chunks per lane
// (lane l owns chunks l + 64 j). Each wave holds 2 CL k-steps of 64 for the MFMA.
template <int RW, int CL>
__global__ __launch_bounds__(256) void k_decode(DecodeArgs a) {
  constexpr int SPW = 2 * CL;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int red[4][16][17];
  __shared__ int wave_tot[4];
  __shared__ float rowmax_s[kDecMaxM];
  const int K = a.K, M = a.M;
  const int W = (K + 31) / 32, nchunk = K / 8, xs = K + 16;
  int8_t* xq_s = reinterpret_cast<int8_t*>(lds);
  uint32_t* mask_s = reinterpret_cast<uint32_t*>(lds + ((M * xs + 15) & ~15));
  short* idx_s = reinterpret_cast<short*>(mask_s + W);
  float* xo_s = reinterpret_cast<float*>(lds + ((((M * xs + 15) & ~15) + W * 4 + K * 2 + 15) & ~15));
  float* wo_s = xo_s + kOutChunk * 16;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;

  // 1. activations into registers (loaded first: the vmcnt wait for them then leaves
  // every weight load in flight)
  v8h xv[RW][CL];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int m = wave + 4 * i;
#pragma unroll
    for (int j = 0; j < CL; ++j) {
      const int c = lane + 64 * j;
      const v8h v = *reinterpret_cast<const v8h*>(a.X + static_cast<size_t>(min(m, M - 1)) * K +
                                                  min(c, nchunk - 1) * 8);
      xv[i][j] = (m < M && c < nchunk) ? v : v8h{};
    }
  }
  // 2. the weight stream. Wq is unit-tiled: the block's 16 rows are one contiguous
  // run of KS units, and unit s is exactly the 16 x 64 A operand of k-step s, so each
  // load instruction reads one whole 1 KB unit. Wave w takes steps w, w + 4, ...; each
  // block starts at a different step so that concurrent blocks spread over HBM
  // channels instead of all hitting the same offsets. The K padding holds zeros.
  const int ks = unit_ks(K);
  const int nsteps = ks;
  const int kl = 16 * (lane >> 4);
  v4i wf[SPW];
  int wstep[SPW];
  const int8_t* wunit = a.Wq + static_cast<size_t>(n0 >> 4) * ks * kUnitBytes + (lane & 15) * kUnitK + kl;
  const int nmine = (nsteps - wave + 3) / 4;  // steps of this wave
  const int rot = nmine > 0 ? static_cast<int>(blockIdx.x * 5u % static_cast<unsigned>(nmine)) : 0;
  // Loads are unconditional (a guarded load becomes a branch whose join waits for the
  // data): slots past this wave's share re-read unit 0 and are skipped by the MFMA.
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    int j = i + rot;
    j = j >= nmine ? j - nmine : j;
    const int step = i < nmine ? wave + 4 * j : 0;
    wstep[i] = i < nmine ? step : -1;
    wf[i] = *reinterpret_cast<const v4i*>(wunit + static_cast<size_t>(step) * kUnitBytes);
  }

  for (int w = tid; w < W; w += 256) mask_s[w] = 0;
  lds_barrier();

  // outlier flags of this wave's rows, per owned chunk (OR over rows), into LDS
#pragma unroll
  for (int j = 0; j < CL; ++j) {
    const int c = lane + 64 * j;
    unsigned mx = 0;
#pragma unroll
    for (int i = 0; i < RW; ++i) mx = max(mx, chunk_mag_max(xv[i][j]));
    const float cmax = half_bits_to_float(mx);
    if (c < nchunk && cmax >= a.t) {  // rare: find which columns
      unsigned f = 0;
#pragma unroll
      for (int i = 0; i < RW; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          f |= static_cast<unsigned>(fabsf(static_cast<float>(xv[i][j][e])) >= a.t) << e;
      atomicOr(&mask_s[c >> 2], f << ((c & 3) << 3));
    }
  }
  lds_barrier();

  // 3. rank outlier columns (thread t owns words [t*per, (t+1)*per))
  const int per = (W + 255) / 256;
  const int w0 = min(W, tid * per), w1 = min(W, w0 + per);
  int mine = 0;
  for (int w = w0; w < w1; ++w) mine += __popc(mask_s[w]);
  const int incl = wave_inclusive_sum(mine);
  if (lane == 63) wave_tot[wave] = incl;

  // row absmax over the kept columns, then quantize into LDS (this wave's rows)
  unsigned mbyte[CL];
#pragma unroll
  for (int j = 0; j < CL; ++j) {
    const int c = lane + 64 * j;
    mbyte[j] = c < nchunk ? (mask_s[c >> 2] >> ((c & 3) << 3)) & 0xFFu : 0u;
  }
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int m = wave + 4 * i;
    if (m >= M) break;  // wave-uniform
    unsigned mb = 0;
#pragma unroll
    for (int j = 0; j < CL; ++j) {
      v8h v = xv[i][j];
      if (mbyte[j]) {  // drop the outlier columns of this chunk
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((mbyte[j] >> e) & 1u) v[e] = _Float16(0);
      }
      mb = max(mb, chunk_mag_max(v));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mb = max(mb, static_cast<unsigned>(__shfl_xor(static_cast<int>(mb), o, 64)));
    const float am = half_bits_to_float(mb);
    const float r = quant_scale(am);
    if (lane == 0) rowmax_s[m] = am;
#pragma unroll
    for (int j = 0; j < CL; ++j) {
      const int c = lane + 64 * j;
      if (c < nchunk) {
        const v2u o = quant8(xv[i][j], mbyte[j], am, r);
        *reinterpret_cast<v2u*>(xq_s + m * xs + c * 8) = o;
      }
    }
  }
  lds_barrier();
  int before = incl - mine;
  for (int i = 0; i < wave; ++i) before += wave_tot[i];
  const int count = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
  for (int w = w0, r = before; w < w1; ++w) {
    uint32_t bits = mask_s[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      idx_s[r++] = static_cast<short>(w * 32 + b);
    }
  }

  // 4. int8 MFMA: D[n_local][m] += Wq[n0 + n_local, k] * Xq[m, k]
  v4i acc = v4i{};
  const int mtok = lane & 15;
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    if (wstep[i] >= 0) {  // wave-uniform
      const int k = 64 * wstep[i] + kl;
      const v4i xf = (mtok < M && k < K) ? *reinterpret_cast<const v4i*>(xq_s + mtok * xs + k)
                                         : v4i{};
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[i], xf, acc, 0, 0, 0);
    }
  }
  // 16x16 accumulator layout: lane l, register r -> column m = l % 16, row 4 (l / 16) + r
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][4 * (lane >> 4) + r][mtok] = acc[r];
  lds_barrier();

  // 5. epilogue: thread -> (token m, output feature n0 + nl)
  const int m = tid >> 4, nl = tid & 15, n = n0 + nl;
  float yo = 0.0f;
  for (int r0 = 0; r0 < count; r0 += kOutChunk) {  // block-uniform trip count
    const int rn = min(kOutChunk, count - r0);
    for (int t = tid; t < rn * 16; t += 256) {
      const int r = t >> 4, q = t & 15;
      const int col = idx_s[r0 + r];
      wo_s[r * 16 + q] = static_cast<float>(a.Wq[unit_offset(n0 + q, col, ks)]);
      xo_s[r * 16 + q] = q < M ? static_cast<float>(a.X[static_cast<size_t>(q) * K + col]) : 0.0f;
    }
    lds_barrier();
    for (int r = 0; r < rn; ++r) yo += xo_s[r * 16 + m] * wo_s[r * 16 + nl];
    lds_barrier();
  }
  const bool overflow = count > a.max_outliers;
  if (m < M) {
    const int s = red[0][nl][m] + red[1][nl][m] + red[2][nl][m] + red[3][nl][m];
    const float aw = a.a_w[n];
    const float y = static_cast<float>(s) * (rowmax_s[m] * kInvQMax2) * aw + yo * __fdiv_rn(aw, 127.0f);
    a.Y[static_cast<size_t>(m) * a.N + n] =
        overflow ? static_cast<_Float16>(__builtin_nanf("")) : static_cast<_Float16>(y);
    if (a.acc_out) a.acc_out[static_cast<size_t>(m) * a.N + n] = s;
  }
  if (blockIdx.x == 0 && tid == 0) {
    a.status[0] = overflow ? 7 : 0;
    a.status[1] = count;
  }
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  const int W = (a.K + 31) / 32;
  const size_t head = ((static_cast<size_t>(a.M) * (a.K + 16) + 15) & ~size_t(15)) + W * 4 +
                      static_cast<size_t>(a.K) * 2;
  const size_t lds = ((head + 15) & ~size_t(15)) + 2 * kOutChunk * 16 * sizeof(float);
  const int rw = rows_per_wave(a.M), cl = chunks_per_lane(a.K);
  const dim3 grid(a.N / 16), block(256);
#define I8MM_DEC(R, C)                                                              \
  if (rw == R && cl == C) {                                                         \
    hipLaunchKernelGGL((k_decode<R, C>), grid, block, lds, s, a);                   \
    return hipGetLastError();                                                       \
  }
  I8MM_DEC(1, 1) I8MM_DEC(1, 2) I8MM_DEC(1, 4) I8MM_DEC(1, 8) I8MM_DEC(1, 16)
  I8MM_DEC(2, 1) I8MM_DEC(2, 2) I8MM_DEC(2, 4) I8MM_DEC(2, 8) I8MM_DEC(2, 16)
  I8MM_DEC(4, 1) I8MM_DEC(4, 2) I8MM_DEC(4, 4) I8MM_DEC(4, 8)
#undef I8MM_DEC
  return hipErrorInvalidValue;
}

}  // namespace i8mm
