// Decode path: the whole decomposed product for a handful of tokens in one kernel.
//
// "What is 8-bit LLM quantization?", Does INT8 always improve speed?: for the decoding
// workload the gain comes from the smaller weights cutting memory traffic. With
// M <= 16 tokens the int8 weight stream (N x K bytes) is the whole cost, so one
// launch does every step and reads each Wq byte from HBM exactly once:
//   1. each block issues the loads of its 16 Wq rows (all K) into registers first;
//   2. while they are in flight it reads all of X (small, L2-resident), finds the
//      outlier columns (|X| >= t in any row), ranks them, takes each row's absmax over
//      the other columns and writes Xq into LDS - every block does this redundantly,
//      which costs L2 reads but no extra launch or grid-wide wait;
//   3. v_mfma_i32_16x16x64_i8 with Wq rows as the 16-row operand and Xq rows as the
//      16-column operand (tokens past M are zero), K split over the 4 waves;
//   4. the four int32 partials are summed exactly through LDS; the epilogue applies
//      the outer-product dequant, adds the outlier columns' product in fp32 (exact
//      fp16 X times the int8 weight dequantized by a_w / 127) and rounds once to fp16.
#include "common.hpp"
#include "launch.hpp"

namespace i8mm {

constexpr int kDecMaxM = 16, kDecMaxK = 8192, kDecMaxMK = 32768;

bool decode_supported(int64_t M, int64_t K) {
  return M >= 1 && M <= kDecMaxM && K <= kDecMaxK && M * K <= kDecMaxMK;
}

// SPW: k-steps of 64 per wave held in registers (wave w takes steps w, w+4, ...).
// XC: 8-half chunks of X per thread (chunk e = tid + 256 i of the M*K/8 chunks).
template <int SPW, int XC>
__global__ __launch_bounds__(256) void k_decode(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int red[4][16][17];
  __shared__ unsigned rowmax[kDecMaxM];
  __shared__ int wave_tot[4];
  const int K = a.K, M = a.M;
  const int W = (K + 31) / 32, nchunk = K / 8, xs = K + 16;
  int8_t* xq_s = reinterpret_cast<int8_t*>(lds);
  uint32_t* mask_s = reinterpret_cast<uint32_t*>(lds + ((M * xs + 15) & ~15));
  short* idx_s = reinterpret_cast<short*>(mask_s + W);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int nsteps = (K + 63) / 64;
  const int kl = 16 * (lane >> 4);

  // 1. the weight stream
  v4i wf[SPW];
  const int8_t* wrow = a.Wq + static_cast<size_t>(n0 + (lane & 15)) * K + kl;
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int step = wave + 4 * i;
    wf[i] = (step < nsteps && 64 * step + kl < K)
                ? *reinterpret_cast<const v4i*>(wrow + 64 * step)
                : v4i{};
  }

  // 2. activations
  const int nx = M * nchunk;
  v8h xv[XC];
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int e = tid + 256 * i;
    xv[i] = e < nx ? *reinterpret_cast<const v8h*>(a.X + static_cast<size_t>(e) * 8) : v8h{};
  }
  for (int w = tid; w < W; w += 256) mask_s[w] = 0;
  if (tid < kDecMaxM) rowmax[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int e = tid + 256 * i;
    if (e < nx) {
      unsigned f = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        f |= static_cast<unsigned>(fabsf(static_cast<float>(xv[i][q])) >= a.t) << q;
      const int c = e % nchunk;
      if (f) atomicOr(&mask_s[c >> 2], f << ((c & 3) << 3));
    }
  }
  __syncthreads();
  // rank outlier columns (thread t owns words [t*per, (t+1)*per)) and row absmax
  const int per = (W + 255) / 256;
  const int w0 = min(W, tid * per), w1 = min(W, w0 + per);
  int mine = 0;
  for (int w = w0; w < w1; ++w) mine += __popc(mask_s[w]);
  const int incl = wave_inclusive_sum(mine);
  if (lane == 63) wave_tot[wave] = incl;
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int e = tid + 256 * i;
    if (e < nx) {
      const int c = e % nchunk;
      const unsigned mb = (mask_s[c >> 2] >> ((c & 3) << 3)) & 0xFFu;
      float m = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (!((mb >> q) & 1u)) m = fmaxf(m, fabsf(static_cast<float>(xv[i][q])));
      // non-negative floats order like their bit patterns
      if (m > 0.0f) atomicMax(&rowmax[e / nchunk], __float_as_uint(m));
    }
  }
  __syncthreads();
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
  // quantize into LDS (outlier columns -> 0)
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int e = tid + 256 * i;
    if (e < nx) {
      const int row = e / nchunk, c = e % nchunk;
      const unsigned mb = (mask_s[c >> 2] >> ((c & 3) << 3)) & 0xFFu;
      const float m = __uint_as_float(rowmax[row]);
      int q[8];
#pragma unroll
      for (int z = 0; z < 8; ++z) q[z] = ((mb >> z) & 1u) ? 0 : quant_code(xv[i][z], m);
      v2u o;
      o[0] = pack4(q[0], q[1], q[2], q[3]);
      o[1] = pack4(q[4], q[5], q[6], q[7]);
      *reinterpret_cast<v2u*>(xq_s + row * xs + c * 8) = o;
    }
  }
  __syncthreads();

  // 3. int8 MFMA: D[n_local][m] += Wq[n0 + n_local, k] * Xq[m, k]
  v4i acc = v4i{};
  const int mtok = lane & 15;
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int step = wave + 4 * i;
    if (step < nsteps) {
      const int k = 64 * step + kl;
      const v4i xf = (mtok < M && k < K) ? *reinterpret_cast<const v4i*>(xq_s + mtok * xs + k)
                                         : v4i{};
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[i], xf, acc, 0, 0, 0);
    }
  }
  // 16x16 accumulator layout: lane l, register r -> column m = l % 16, row 4 (l / 16) + r
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][4 * (lane >> 4) + r][mtok] = acc[r];
  __syncthreads();

  // 4. epilogue: thread -> (token m, output feature n0 + nl)
  const int m = tid >> 4, nl = tid & 15, n = n0 + nl;
  const bool overflow = count > a.max_outliers;
  if (m < M) {
    const int s = red[0][nl][m] + red[1][nl][m] + red[2][nl][m] + red[3][nl][m];
    const float aw = a.a_w[n];
    const float ax = __uint_as_float(rowmax[m]);
    float yo = 0.0f;
    const _Float16* xr = a.X + static_cast<size_t>(m) * K;
    const int8_t* wr = a.Wq + static_cast<size_t>(n) * K;
    for (int r = 0; r < count; ++r) {
      const int col = idx_s[r];
      yo += static_cast<float>(xr[col]) * static_cast<float>(wr[col]);
    }
    const float y = static_cast<float>(s) * (ax * kInvQMax2) * aw + yo * __fdiv_rn(aw, 127.0f);
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
  const size_t lds = ((static_cast<size_t>(a.M) * (a.K + 16) + 15) & ~size_t(15)) + W * 4 +
                     static_cast<size_t>(a.K) * 2;
  const int nsteps = (a.K + 63) / 64;
  const int spw = (nsteps + 3) / 4;
  const int xc = (a.M * (a.K / 8) + 255) / 256;
  const dim3 grid(a.N / 16), block(256);
#define I8MM_DEC(S, X) hipLaunchKernelGGL((k_decode<S, X>), grid, block, lds, s, a)
  if (xc <= 4) {
    if (spw <= 4) I8MM_DEC(4, 4);
    else if (spw <= 8) I8MM_DEC(8, 4);
    else if (spw <= 16) I8MM_DEC(16, 4);
    else I8MM_DEC(32, 4);
  } else {
    if (spw <= 4) I8MM_DEC(4, 16);
    else if (spw <= 8) I8MM_DEC(8, 16);
    else if (spw <= 16) I8MM_DEC(16, 16);
    else I8MM_DEC(32, 16);
  }
#undef I8MM_DEC
  return hipGetLastError();
}

}  // namespace i8mm
