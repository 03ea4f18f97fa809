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
constexpr int kDecWaves = 8, kDecThreads = 64 * kDecWaves;
constexpr int kOutChunk = 64;  // outlier columns staged in LDS per epilogue pass
constexpr int kPre = kDecThreads / 16;  // outlier columns gathered before the MFMA (32)

static int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}
static int rows_per_wave(int64_t M) {
  return pow2_at_least(static_cast<int>((M + kDecWaves - 1) / kDecWaves));
}
static int chunks_per_lane(int64_t K) { return pow2_at_least(static_cast<int>((K + 511) / 512)); }

bool decode_supported(int64_t M, int64_t K) {
  return M >= 1 && M <= kDecMaxM && K <= kDecMaxK && M * K <= kDecMaxMK &&
         rows_per_wave(M) * chunks_per_lane(K) <= 16;
}

__device__ __forceinline__ float half_bits_to_float(unsigned h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(h)));
}

// RW: rows per wave (wave w owns rows w + 8 i), CL: 8-column chunks per lane (lane l
// owns chunks l + 64 j). Wave w's MFMA k-steps are w, w + 8, ... (at most CL of them).
template <int RW, int CL>
__global__ __launch_bounds__(kDecThreads) void k_decode(DecodeArgs a) {
  constexpr int SPW = CL;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int red[kDecWaves][16][17];
  __shared__ int wave_tot[kDecWaves];
  __shared__ float rowmax_s[kDecMaxM];
  const int K = a.K, M = a.M;
  const int W = (K + 31) / 32, nchunk = K / 8, xs = K + 16;
  // LDS: Xq [M][K + 16] | per-chunk flag bytes of each wave [nchunk][8] | combined mask
  // words [W] | outlier column list [K] (short) | outlier staging
  int8_t* xq_s = reinterpret_cast<int8_t*>(lds);
  const int off_flag = (M * xs + 15) & ~15;
  unsigned char* flag_s = reinterpret_cast<unsigned char*>(lds + off_flag);
  uint32_t* mask_s = reinterpret_cast<uint32_t*>(lds + off_flag + nchunk * kDecWaves);
  short* idx_s = reinterpret_cast<short*>(mask_s + W);
  float* xo_s = reinterpret_cast<float*>(
      lds + ((off_flag + nchunk * kDecWaves + W * 4 + K * 2 + 15) & ~15));
  float* wo_s = xo_s + kOutChunk * 16;
  // 8 bytes per lane that absorb the stores of chunks past K (branch-free stores)
  int8_t* sink_s = reinterpret_cast<int8_t*>(wo_s + kOutChunk * 16);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;

  // 1. activations into registers (issued first: waiting for them then leaves every
  // weight load in flight). Every block reads all of X, so each block walks its
  // chunks from a different starting group: register j holds chunk group
  // (j + xrot) mod CL, and concurrent blocks of one XCD (block ids 8 apart) hit
  // different L2 channels instead of all requesting the same lines at once.
  const int xrot = (blockIdx.x >> 3) & (CL - 1);
  v8h xv[RW][CL];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int m = wave + kDecWaves * i;
#pragma unroll
    for (int j = 0; j < CL; ++j) {
      const int c = lane + 64 * ((j + xrot) & (CL - 1));
      const v8h v = *reinterpret_cast<const v8h*>(a.X + static_cast<size_t>(min(m, M - 1)) * K +
                                                  min(c, nchunk - 1) * 8);
      xv[i][j] = (m < M && c < nchunk) ? v : v8h{};
    }
  }
  // 2. the weight stream. Wq is unit-tiled: the block's 16 rows are one contiguous run
  // of KS units, and unit s is exactly the 16 x 64 A operand of k-step s, so each load
  // instruction reads one whole 1 KB unit. Each block starts its share at a different
  // step (also among the blocks of one XCD) so that concurrent blocks spread over HBM
  // channels. The K padding holds zeros.
  // Loads are unconditional (a guarded load becomes a branch whose join waits for the
  // data): slots past this wave's share re-read unit 0 and are skipped by the MFMA.
  const int ks = unit_ks(K);
  const int kl = 16 * (lane >> 4);
  v4i wf[SPW];
  int wstep[SPW];
  const int8_t* wunit =
      a.Wq + static_cast<size_t>(n0 >> 4) * ks * kUnitBytes + (lane & 15) * kUnitK + kl;
  const int nmine = (ks - wave + kDecWaves - 1) / kDecWaves;
  const int rot = nmine > 0 ? static_cast<int>((blockIdx.x * 5u + (blockIdx.x >> 3) * 3u) %
                                               static_cast<unsigned>(nmine))
                            : 0;
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    int j = i + rot;
    j = j >= nmine ? j - nmine : j;
    const int step = i < nmine ? wave + kDecWaves * j : 0;
    wstep[i] = i < nmine ? step : -1;
    wf[i] = *reinterpret_cast<const v4i*>(wunit + static_cast<size_t>(step) * kUnitBytes);
  }
  // the epilogue's column constant, loaded now so that its latency hides under the rest
  const float aw_pre = a.a_w[n0 + (tid & 15)];

  // 3. outlier flags ("LLM.int8()", Mixed-precision decomposition: a feature column is
  // an outlier when any of its values reaches the threshold). Magnitudes as fp16 bits:
  // mag[i][j][d] holds two halves; the per-chunk max over this wave's rows decides
  // whether the exact per-column test is needed. Each wave writes one flag byte per
  // chunk (no zeroing, no atomics); the OR over waves is taken after the barrier.
  const unsigned tb = threshold_bits(a.t);
#pragma unroll
  for (int j = 0; j < CL; ++j) {
    const int c = lane + 64 * ((j + xrot) & (CL - 1));
    unsigned f = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      unsigned cm = 0;
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const unsigned mg = __builtin_bit_cast(v4u, xv[i][j])[d] & 0x7fff7fffu;
        cm = i == 0 ? mg : pk_max_u16(cm, mg);
      }
      f |= static_cast<unsigned>((cm & 0xffffu) >= tb) << (2 * d);
      f |= static_cast<unsigned>((cm >> 16) >= tb) << (2 * d + 1);
    }
    *(c < nchunk ? reinterpret_cast<unsigned char*>(flag_s + c * kDecWaves + wave)
                 : reinterpret_cast<unsigned char*>(sink_s + lane)) = static_cast<unsigned char>(f);
  }
  lds_barrier();

  // 4. combined flags of the owned chunks; outlier values are zeroed in the registers
  // (their codes are 0 and they do not enter the row constant), branch-free: bit e of
  // the chunk's flags clears half e through a keep-mask per dword
#pragma unroll
  for (int j = 0; j < CL; ++j) {
    const int c = lane + 64 * ((j + xrot) & (CL - 1));
    const v2u fw = *reinterpret_cast<const v2u*>(flag_s + min(c, nchunk - 1) * kDecWaves);
    const unsigned o = fw[0] | fw[1];
    const unsigned keep = c < nchunk ? ~(o | (o >> 8) | (o >> 16) | (o >> 24)) : ~0u;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const unsigned km = ((keep >> (2 * d)) & 1u ? 0x0000ffffu : 0u) |
                          ((keep >> (2 * d + 1)) & 1u ? 0xffff0000u : 0u);
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        v4u u = __builtin_bit_cast(v4u, xv[i][j]);
        u[d] &= km;
        xv[i][j] = __builtin_bit_cast(v8h, u);
      }
    }
  }
  // 5. mask words and their ranks: thread t < W owns word t (chunks 4t .. 4t + 3)
  int mine = 0;
  if (tid < W) {
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = 4 * tid + q;
      if (c < nchunk) {
        const v2u fw = *reinterpret_cast<const v2u*>(flag_s + c * kDecWaves);
        const unsigned o = fw[0] | fw[1];
        word |= ((o | (o >> 8) | (o >> 16) | (o >> 24)) & 0xffu) << (8 * q);
      }
    }
    mask_s[tid] = word;
    mine = __popc(word);
  }
  const int incl = wave_prefix_sum(mine);
  if (lane == 63) wave_tot[wave] = incl;

  // 6. row absmax over the kept columns ("LLM.int8()", Vector-wise quantization: one
  // constant per row of X) and the row's codes into LDS
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int m = wave + kDecWaves * i;
    if (m >= M) break;  // wave-uniform
    unsigned pm = 0;
#pragma unroll
    for (int j = 0; j < CL; ++j)
#pragma unroll
      for (int d = 0; d < 4; ++d)
        pm = pk_max_u16(pm, __builtin_bit_cast(v4u, xv[i][j])[d] & 0x7fff7fffu);
    const unsigned mb = wave_max_u32(max(pm & 0xffffu, pm >> 16));
    const float am = half_bits_to_float(mb);
    const QuantBracket br = quant_bracket(am);
    if (lane == 0) rowmax_s[m] = am;
    // codes from the bracketing pair (see quant8_bracket); chunks where the pair
    // disagrees (values at or within about 2^-15 of a half-integer) are rewritten
    // with quant8_exact after the loop, behind one wave-uniform test
    unsigned redo = 0;
#pragma unroll
    for (int j = 0; j < CL; ++j) {
      const int c = lane + 64 * ((j + xrot) & (CL - 1));
      unsigned b1[8], b2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xf = static_cast<float>(xv[i][j][e]);
        b1[e] = __builtin_bit_cast(unsigned, __builtin_fmaf(xf, br.lo, kRoundMagic));
        b2[e] = __builtin_bit_cast(unsigned, __builtin_fmaf(xf, br.hi, kRoundMagic));
      }
      v2u o;
      o[0] = pack_low_bytes(b1[0], b1[1], b1[2], b1[3]);
      o[1] = pack_low_bytes(b1[4], b1[5], b1[6], b1[7]);
      const unsigned dis = (o[0] ^ pack_low_bytes(b2[0], b2[1], b2[2], b2[3])) |
                           (o[1] ^ pack_low_bytes(b2[4], b2[5], b2[6], b2[7]));
      redo |= dis != 0u ? 1u << j : 0u;
      *reinterpret_cast<v2u*>(c < nchunk ? xq_s + m * xs + c * 8 : sink_s + lane * 8) = o;
    }
    // One pass of a do-while always runs, so its code is fetched in order on every
    // launch (a rarely taken branch into cold code costs microseconds here): each lane
    // selects its lowest pending chunk (or none) and rewrites it with quant8_exact.
    unsigned pend = redo;
    do {
      const unsigned jb = __builtin_ctz(pend | (1u << CL));  // CL: nothing pending
      v8h xs8 = v8h{};
      int cs = 0;
#pragma unroll
      for (int j = 0; j < CL; ++j) {
        const bool hit = jb == static_cast<unsigned>(j);
        xs8 = hit ? xv[i][j] : xs8;
        cs = hit ? lane + 64 * ((j + xrot) & (CL - 1)) : cs;
      }
      const v2u o = quant8_exact(xs8, am, br.lo);
      *reinterpret_cast<v2u*>(jb < CL && cs < nchunk ? xq_s + m * xs + cs * 8 : sink_s + lane * 8) = o;
      pend &= pend - 1u;
    } while (__ballot(pend != 0u) != 0);
  }
  lds_barrier();
  int before = incl - mine;
  for (int i = 0; i < wave; ++i) before += wave_tot[i];
  int count = 0;
#pragma unroll
  for (int i = 0; i < kDecWaves; ++i) count += wave_tot[i];
  if (tid < W) {
    uint32_t bits = mask_s[tid];
    for (int r = before; bits; ++r) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      idx_s[r] = static_cast<short>(tid * 32 + b);
    }
  }
  lds_barrier();
  // The values of the first kPre outlier columns (one (column, row) pair per thread)
  // are loaded now, so that their latency overlaps the MFMA (unconditional loads at a
  // valid column, discarded past the count); they go to LDS with the partials.
  const int m = (tid >> 4) & 15, nl = tid & 15, n = n0 + nl;
  const int npre = min(count, kPre);
  const int pr = tid >> 4, pq = tid & 15;
  const int pcol = pr < npre ? idx_s[pr] : 0;
  const int pw = a.Wq[unit_offset(n0 + pq, pcol, ks)];
  const _Float16 px = a.X[static_cast<size_t>(min(pq, M - 1)) * K + pcol];

  // 7. int8 MFMA: D[n_local][m] += Wq[n0 + n_local, k] * Xq[m, k]; the Xq fragments
  // are read (at clamped addresses, discarded past M or K) before the MFMA chain
  // (in batches of at most 8 steps, to bound the registers the fragments take)
  const int mtok = lane & 15;
  constexpr int XB = SPW < 8 ? SPW : 8;
  v4i acc = v4i{};
#pragma unroll
  for (int i0 = 0; i0 < SPW; i0 += XB) {
    v4i xf[XB];
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      const int k = 64 * max(wstep[i0 + i], 0) + kl;
      const v4i t = *reinterpret_cast<const v4i*>(xq_s + min(mtok, M - 1) * xs + min(k, K - 16));
      xf[i] = (mtok < M && k < K) ? t : v4i{};
    }
#pragma unroll
    for (int i = 0; i < XB; ++i)
      if (wstep[i0 + i] >= 0)  // wave-uniform
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[i0 + i], xf[i], acc, 0, 0, 0);
  }
  // 16x16 accumulator layout: lane l, register r -> column m = l % 16, row 4 (l / 16) + r
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][4 * (lane >> 4) + r][mtok] = acc[r];
  wo_s[pr * 16 + pq] = pr < npre ? static_cast<float>(pw) : 0.0f;
  xo_s[pr * 16 + pq] = pr < npre && pq < M ? static_cast<float>(px) : 0.0f;
  lds_barrier();

  // 8. epilogue: thread t < 256 -> (token m, output feature n0 + nl). The int32
  // partials of the waves are summed exactly; the outlier columns' product is taken
  // in fp32 from the exact fp16 X and the int8 weight dequantized by a_w / 127.
  float yo = 0.0f;
  if (tid < 256)
    for (int r = 0; r < npre; ++r) yo += xo_s[r * 16 + m] * wo_s[r * 16 + nl];
  for (int r0 = kPre; r0 < count; r0 += kOutChunk) {  // block-uniform trip count
    lds_barrier();  // the staged values above are read
    const int rn = min(kOutChunk, count - r0);
    for (int t = tid; t < rn * 16; t += kDecThreads) {
      const int r = t >> 4, q = t & 15;
      const int col = idx_s[r0 + r];
      wo_s[r * 16 + q] = static_cast<float>(a.Wq[unit_offset(n0 + q, col, ks)]);
      xo_s[r * 16 + q] = q < M ? static_cast<float>(a.X[static_cast<size_t>(q) * K + col]) : 0.0f;
    }
    lds_barrier();
    if (tid < 256)
      for (int r = 0; r < rn; ++r) yo += xo_s[r * 16 + m] * wo_s[r * 16 + nl];
    lds_barrier();
  }
  const bool overflow = count > a.max_outliers;
  if (tid < 256 && m < M) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) s += red[w][nl][m];
    const float aw = aw_pre;
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
  const int W = (a.K + 31) / 32, nchunk = a.K / 8;
  const size_t off_flag = (static_cast<size_t>(a.M) * (a.K + 16) + 15) & ~size_t(15);
  const size_t head = off_flag + static_cast<size_t>(nchunk) * kDecWaves + W * 4 +
                      static_cast<size_t>(a.K) * 2;
  const size_t lds = ((head + 15) & ~size_t(15)) + 2 * kOutChunk * 16 * sizeof(float) + 64 * 8;
  const int rw = rows_per_wave(a.M), cl = chunks_per_lane(a.K);
  const dim3 grid(a.N / 16), block(kDecThreads);
#define I8MM_DEC(R, C)                                                              \
  if (rw == R && cl == C) {                                                         \
    hipLaunchKernelGGL((k_decode<R, C>), grid, block, lds, s, a);                   \
    return hipGetLastError();                                                       \
  }
  I8MM_DEC(1, 1) I8MM_DEC(1, 2) I8MM_DEC(1, 4) I8MM_DEC(1, 8) I8MM_DEC(1, 16)
  I8MM_DEC(2, 1) I8MM_DEC(2, 2) I8MM_DEC(2, 4) I8MM_DEC(2, 8)
#undef I8MM_DEC
  return hipErrorInvalidValue;
}

}  // namespace i8mm
