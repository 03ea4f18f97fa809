// Decode path: the whole decomposed product for a handful of tokens in one kernel.
//
// "What is 8-bit LLM quantization?", Does INT8 always improve speed?: for the decoding
// workload the gain comes from the smaller weights cutting memory traffic. With
// M <= 16 tokens the int8 weight stream (N x K bytes) is the whole cost, so one
// launch does every step and reads each Wq byte from HBM exactly once. One block of
// 8 waves per 16 output features:
//   1. each thread loads its 8-column chunks of X for every token row, then issues its
//      wave's share of the block's 16 Wq rows (whole 1 KB units) into registers;
//   2. while the weights are in flight: per chunk, the largest magnitude over the
//      rows against the threshold gives the outlier columns (a keep-mask per column,
//      one byte of outlier bits per chunk in LDS); per row, the absmax over the kept
//      columns, reduced over the wave with DPP and over the block through LDS; the
//      rows' brackets of 127 / a_x; the codes of every (row, chunk) into LDS, with an
//      exact pass for the rare values where the bracket cannot decide; the outlier
//      columns' ranks. Every block repeats this for the whole of X, which costs L2
//      reads and VALU time but no second launch and no grid-wide wait;
//   3. v_mfma_i32_16x16x64_i8 with Wq rows as the 16-row operand and Xq rows as the
//      16-column operand (tokens past M are zero), K split over the 8 waves;
//   4. the eight int32 partials are summed exactly through LDS; the epilogue applies
//      the outer-product dequant and adds the outlier columns' product in fp32
//      (exact fp16 X times the int8 weight dequantized by a_w / 127, both staged in
//      LDS) before the single rounding to fp16.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace i8mm {

constexpr int kDecMaxM = 16, kDecMaxK = 8192;
// dynamic LDS a block may take (160 KB per CU, less the kernel's static arrays)
constexpr size_t kDecMaxDynLds = 150 * 1024;
constexpr int kDecWaves = 8, kDecThreads = 64 * kDecWaves;
constexpr int kOutChunk = 64;  // outlier columns staged in LDS per epilogue pass
constexpr int kPre = kDecThreads / 16;  // outlier columns gathered before the MFMA (32)

static int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}
// token rows held per thread: M rounded up to a power of two, at least 2
static int rows_held(int64_t M) { return max(2, pow2_at_least(static_cast<int>(M))); }
// MFMA k-steps (64 columns each) per wave: ceil(K / 512) rounded up, at least 2
static int steps_per_wave(int64_t K) {
  return max(2, pow2_at_least(static_cast<int>((K + 511) / 512)));
}

// X chunks a thread holds in registers: rows_held(M) x (one per 4096 columns of K),
// at most 16 (64 registers): M <= 16 up to K = 4096, M <= 8 up to K = 8192.
bool decode_supported(int64_t M, int64_t K) {
  if (M < 1 || M > kDecMaxM || K > kDecMaxK) return false;
  return rows_held(M) * (K > 4096 ? 2 : 1) <= 16;
}

// Dynamic LDS of one block; with x_staged, the masked copy of X is included.
static size_t decode_lds_bytes(int64_t M, int64_t K, bool x_staged) {
  const size_t nchunk = static_cast<size_t>(K) / 8;
  const size_t off_flag = (x_staged ? static_cast<size_t>(M) * K * 2 : 0) +
                          ((static_cast<size_t>(M) * (K + 16) + 15) & ~size_t(15));
  const size_t head = off_flag + ((nchunk + 3) & ~size_t(3)) + static_cast<size_t>(K) * 2;
  return ((head + 15) & ~size_t(15)) + 2 * kOutChunk * 16 * sizeof(float) + 64 * 16;
}

__device__ __forceinline__ float half_bits_to_float(unsigned h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(h)));
}

typedef unsigned short v2us __attribute__((ext_vector_type(2)));
typedef short v2ss __attribute__((ext_vector_type(2)));

// Per half of a dword of magnitudes (fp16 bits, sign cleared): 0xffff where the
// magnitude is below the threshold bits (tb2 holds them in both halves), 0 where it
// reaches them. Both are below 2^15, so mag - tb wraps (sets bit 15) exactly when
// mag < tb; an arithmetic shift spreads that bit over its half.
__device__ __forceinline__ unsigned keep_halves(unsigned mag2, unsigned tb2) {
  const v2us d = __builtin_bit_cast(v2us, mag2) - __builtin_bit_cast(v2us, tb2);
  return __builtin_bit_cast(unsigned, __builtin_bit_cast(v2ss, d) >> (v2ss){15, 15});
}

// Largest value over the 64 lanes of each of N unsigned values, in every lane: the
// DPP steps of wave_scan_dpp, taken for all N values before the next step so that
// the independent chains fill each other's DPP wait states.
template <int N>
__device__ __forceinline__ void wave_max_u32_n(unsigned (&v)[N]) {
  auto step = [&](auto ctrl, auto rmask, auto bound) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      v[i] = max(v[i], static_cast<unsigned>(__builtin_amdgcn_update_dpp(
                           0, static_cast<int>(v[i]), decltype(ctrl)::value,
                           decltype(rmask)::value, 0xF, decltype(bound)::value)));
  };
  using T = std::true_type;
  using F = std::false_type;
  step(std::integral_constant<int, 0x111>{}, std::integral_constant<int, 0xF>{}, T{});
  step(std::integral_constant<int, 0x112>{}, std::integral_constant<int, 0xF>{}, T{});
  step(std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0xF>{}, T{});
  step(std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0xF>{}, T{});
  step(std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xA>{}, F{});
  step(std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xC>{}, F{});
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(v[i]), 63));
}

// MR: token rows held per thread (M <= MR), SPW: MFMA k-steps per wave (slots for the
// weight units), XS: the masked X is staged in LDS for the exact pass (else that pass
// reads X from global memory, where the larger shapes leave no room in LDS). Thread t owns the 8-column chunks c = 64 ((w + xrot) mod 8) + l + 512 j
// (w its wave, l its lane, j < CC) of every row, so a chunk's outlier test over all
// rows and its keep-mask are computed once, in registers.
template <int MR, int SPW, bool XS>
__global__ __launch_bounds__(kDecThreads) void k_decode(DecodeArgs a) {
  constexpr int CC = SPW > 8 ? 2 : 1;  // chunks per thread: K <= 4096 needs one
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int red[kDecWaves][16][17];
  __shared__ int count_s;
  __shared__ unsigned rmax_w[kDecWaves][MR];  // each wave's row maxima (fp16 bits)
  __shared__ float rowmax_s[kDecMaxM];
  const int K = a.K, M = a.M;
  const int W = (K + 31) / 32, nchunk = K / 8, xs = K + 16;
  const int nflag = (nchunk + 3) & ~3;
  // LDS: X with its outlier columns cleared [M][K] (XS only) | Xq [M][K + 16] |
  // outlier bits, one byte per chunk [nflag] | outlier column list [K] (short) |
  // outlier staging | sink
  _Float16* x_s = reinterpret_cast<_Float16*>(lds);
  const int off_xq = XS ? M * K * 2 : 0;
  int8_t* xq_s = reinterpret_cast<int8_t*>(lds + off_xq);
  const int off_flag = off_xq + ((M * xs + 15) & ~15);
  unsigned char* flag_s = reinterpret_cast<unsigned char*>(lds + off_flag);
  short* idx_s = reinterpret_cast<short*>(lds + off_flag + nflag);
  float* xo_s = reinterpret_cast<float*>(lds + ((off_flag + nflag + K * 2 + 15) & ~15));
  float* wo_s = xo_s + kOutChunk * 16;
  // 16 bytes per lane that absorb the stores of chunks past K (branch-free stores)
  int8_t* sink_s = reinterpret_cast<int8_t*>(wo_s + kOutChunk * 16);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;

  // 1. activations into registers (issued first: waiting for them then leaves every
  // weight load in flight). Every block reads all of X; the chunk groups of its waves
  // are rotated per block so that concurrent blocks of one XCD (block ids 8 apart)
  // start on different L2 channels. Rows past M and chunks past K read the last valid
  // row or chunk: repeats change neither a maximum nor an OR, and their codes go to
  // the sink.
  const int xrot = (blockIdx.x >> 3) & 7;
  const int cbase = 64 * ((wave + xrot) & 7) + lane;
  v8h xv[MR][CC];
#pragma unroll
  for (int j = 0; j < CC; ++j) {
    const int c = min(cbase + 512 * j, nchunk - 1);
#pragma unroll
    for (int m = 0; m < MR; ++m)
      xv[m][j] = *reinterpret_cast<const v8h*>(a.X + static_cast<size_t>(min(m, M - 1)) * K + c * 8);
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

  // 3. outlier columns ("LLM.int8()", Mixed-precision decomposition: a feature column is
  // an outlier when any of its values reaches the threshold). Magnitudes as fp16 bits,
  // two per dword: the largest over the rows, compared with the threshold bits, gives
  // a keep-mask per half (0 on outlier columns) and one byte of outlier bits per chunk.
  const unsigned tb = threshold_bits(a.t), tb2 = tb * 0x10001u;
  v4u keep[CC];
#pragma unroll
  for (int j = 0; j < CC; ++j) {
    const int c = cbase + 512 * j;
    v4u cm = __builtin_bit_cast(v4u, xv[0][j]) & 0x7fff7fffu;
#pragma unroll
    for (int m = 1; m < MR; ++m)
#pragma unroll
      for (int d = 0; d < 4; ++d)
        cm[d] = pk_max_u16(cm[d], __builtin_bit_cast(v4u, xv[m][j])[d] & 0x7fff7fffu);
#pragma unroll
    for (int d = 0; d < 4; ++d) keep[j][d] = keep_halves(cm[d], tb2);
    // one byte of each half's keep-mask (halves 0-3, then 4-7), a different bit taken
    // from each byte, summed: bit e is set where column 8 c + e is kept
    const unsigned p = __builtin_amdgcn_perm(keep[j][1], keep[j][0], 0x06040200u);
    const unsigned q = __builtin_amdgcn_perm(keep[j][3], keep[j][2], 0x06040200u);
    const unsigned kb = __builtin_amdgcn_sad_u8((p & 0x08040201u) | (q & 0x80402010u), 0u, 0u);
    *(c < nchunk ? flag_s + c : reinterpret_cast<unsigned char*>(sink_s + lane)) =
        static_cast<unsigned char>(~kb);
  }

  // 4. row absmax over the kept columns ("LLM.int8()", Vector-wise quantization: one
  // constant per row of X): this thread's maximum of each row, then the wave's (the
  // rows' DPP reductions are independent, so their steps interleave), then (after the
  // barrier) the block's
  unsigned rmx[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    unsigned v = 0;
#pragma unroll
    for (int j = 0; j < CC; ++j)
#pragma unroll
      for (int d = 0; d < 4; ++d)
        v = pk_max_u16(v, __builtin_bit_cast(v4u, xv[m][j])[d] & 0x7fff7fffu & keep[j][d]);
    rmx[m] = max(v & 0xffffu, v >> 16);
  }
  wave_max_u32_n<MR>(rmx);
  if (lane == 0)
#pragma unroll
    for (int m = 0; m < MR; ++m) rmax_w[wave][m] = rmx[m];
  lds_barrier();

  // 5. row constants: lane r of every wave combines row r's maxima over the waves and
  // takes its quantization bracket; the rows' values are read from those lanes below
  float am_l;
  QuantBracket br_l;
  {
    const int r = min(lane, MR - 1);
    unsigned v = 0;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) v = max(v, rmax_w[w][r]);
    am_l = half_bits_to_float(v);
    br_l = quant_bracket(am_l);
  }
  if (wave == 0 && lane < M) rowmax_s[lane] = am_l;

  // 6. the outlier column list, ascending: wave 0, lane l takes the mask words
  // 4l .. 4l + 3 (W <= 256), whose little-endian bytes are the outlier bytes of chunks
  // 16l .. 16l + 15; a prefix sum over the lanes gives each word's first rank
  if (wave == 0) {
    const v4u f = *reinterpret_cast<const v4u*>(flag_s + 16 * min(lane, (W - 1) >> 2));
    unsigned wd[4];
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = 4 * lane + q, valid = nchunk - 4 * t;  // chunks of word t inside K
      wd[q] = t >= W ? 0u : valid >= 4 ? f[q] : f[q] & ((1u << (8 * valid)) - 1u);
      cnt += __popc(wd[q]);
    }
    const int incl = wave_prefix_sum(cnt);
    int r = incl - cnt;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      for (unsigned bits = wd[q]; bits; bits &= bits - 1u)
        idx_s[r++] = static_cast<short>((4 * lane + q) * 32 + __builtin_ctz(bits));
    if (lane == 63) count_s = incl;
  }
  lds_barrier();
  const int count = count_s;
  // The values of the first kPre outlier columns (one (column, row) pair per thread)
  // are loaded now, so that their latency hides under the quantization and the MFMA
  // (unconditional loads at a valid column, discarded past the count); they go to LDS
  // with the partials.
  const int npre = min(count, kPre);
  const int pr = tid >> 4, pq = tid & 15;
  const int pcol = pr < npre ? idx_s[pr] : 0;
  const int pw = a.Wq[unit_offset(n0 + pq, pcol, ks)];
  const _Float16 px = a.X[static_cast<size_t>(min(pq, M - 1)) * K + pcol];

  // 7. codes into LDS, outlier columns cleared first (their codes are 0). The bracketing
  // pair (see quant8_fast) decides; (row, chunk) slots where it disagrees (values at
  // or within about 2^-15 of a half-integer) are rewritten with quant8_exact below.
  unsigned redo = 0;
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    // a skipped body rather than an early exit: the loop must unroll fully so that
    // xv stays in registers (a loop with a second exit is left rolled at MR = 16,
    // and xv[m] then lives in scratch memory)
    if (m >= M) continue;  // block-uniform
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, br_l.lo), m));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, br_l.hi), m));
#pragma unroll
    for (int j = 0; j < CC; ++j) {
      const int c = cbase + 512 * j;
      v4u u = __builtin_bit_cast(v4u, xv[m][j]);
#pragma unroll
      for (int d = 0; d < 4; ++d) u[d] &= keep[j][d];
      xv[m][j] = __builtin_bit_cast(v8h, u);
      if constexpr (XS)
        *reinterpret_cast<v8h*>(c < nchunk ? reinterpret_cast<char*>(x_s + m * K + c * 8)
                                           : reinterpret_cast<char*>(sink_s + lane * 16)) = xv[m][j];
      unsigned b1[8], b2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xf = static_cast<float>(xv[m][j][e]);
        b1[e] = __builtin_bit_cast(unsigned, __builtin_fmaf(xf, lo, kRoundMagic));
        b2[e] = __builtin_bit_cast(unsigned, __builtin_fmaf(xf, hi, kRoundMagic));
      }
      v2u o;
      o[0] = pack_low_bytes(b1[0], b1[1], b1[2], b1[3]);
      o[1] = pack_low_bytes(b1[4], b1[5], b1[6], b1[7]);
      const unsigned dis = (o[0] ^ pack_low_bytes(b2[0], b2[1], b2[2], b2[3])) |
                           (o[1] ^ pack_low_bytes(b2[4], b2[5], b2[6], b2[7]));
      redo |= dis != 0u && c < nchunk ? 1u << (m * CC + j) : 0u;
      *reinterpret_cast<v2u*>(c < nchunk ? xq_s + m * xs + c * 8 : sink_s + lane * 8) = o;
    }
  }
  // Exact codes where the pair disagreed, one element per lane per pass. One pass of the
  // loop always runs, so its code is fetched in order on every launch (a rarely taken
  // branch into cold code costs microseconds here). A pass takes the lane's lowest
  // pending slot, reads that chunk back from LDS (this lane wrote it), redoes the pair
  // to find the elements that differ, and settles the lowest one not yet settled with
  // the exact comparison of quant8_exact, patching its code byte.
  unsigned pend = redo, done = 0;
  do {
    const unsigned jb = __builtin_ctz(pend | (1u << (MR * CC)));  // MR * CC: nothing pending
    const bool any = jb < static_cast<unsigned>(MR * CC);
    const int ms = any ? static_cast<int>(jb) / CC : 0;
    const int cs = cbase + 512 * (any ? static_cast<int>(jb) % CC : 0);
    // the pending chunk: the masked copy in LDS, or X itself, whose outlier columns
    // are then left out below (their codes are 0 already)
    const v8h x = XS ? *reinterpret_cast<const v8h*>(x_s + (any ? ms * K + cs * 8 : 0))
                     : *reinterpret_cast<const v8h*>(a.X + (any ? static_cast<size_t>(ms) * K + cs * 8 : 0));
    const float am = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(ms << 2, __builtin_bit_cast(int, am_l)));
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(ms << 2, __builtin_bit_cast(int, br_l.lo)));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(ms << 2, __builtin_bit_cast(int, br_l.hi)));
    unsigned diff = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xf = static_cast<float>(x[e]);
      const unsigned t1 = __builtin_bit_cast(unsigned, __builtin_fmaf(xf, lo, kRoundMagic));
      const unsigned t2 = __builtin_bit_cast(unsigned, __builtin_fmaf(xf, hi, kRoundMagic));
      diff |= t1 != t2 ? 1u << e : 0u;
    }
    diff &= ~done;
    if constexpr (!XS) diff &= ~static_cast<unsigned>(flag_s[any ? cs : 0]);
    const int e = __builtin_ctz(diff | 0x100u);  // 8: nothing left in this slot
    const unsigned xd = __builtin_bit_cast(v4u, x)[(e >> 1) & 3];
    const float xf = half_bits_to_float((e & 1) ? xd >> 16 : xd & 0xffffu);
    const float w = fabsf(xf);
    const float q1 = __builtin_fmaf(w, lo, kRoundMagic) - kRoundMagic;
    const float d = __builtin_fmaf(2.0f * q1 + 1.0f, am, -254.0f * w);
    const int qi = static_cast<int>(q1);
    const int q = qi + ((d < 0.0f || (d == 0.0f && (qi & 1))) ? 1 : 0);
    const bool ok = any && e < 8;
    *(ok ? xq_s + ms * xs + cs * 8 + e : sink_s + lane * 16) =
        static_cast<int8_t>(xf < 0.0f ? -q : q);
    const bool slot_done = (diff & (diff - 1u)) == 0u;  // e was the last one (or none)
    done = slot_done ? 0u : done | (1u << e);
    pend = slot_done ? pend & (pend - 1u) : pend;
  } while (__ballot(pend != 0u) != 0);
  lds_barrier();
  const int m = (tid >> 4) & 15, nl = tid & 15, n = n0 + nl;

  // 8. int8 MFMA: D[n_local][m] += Wq[n0 + n_local, k] * Xq[m, k]; the Xq fragments
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

  // 9. epilogue: thread t < 256 -> (token m, output feature n0 + nl). The int32
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
  const bool xs = decode_lds_bytes(a.M, a.K, true) <= kDecMaxDynLds;
  const size_t lds = decode_lds_bytes(a.M, a.K, xs);
  const int mr = rows_held(a.M), spw = steps_per_wave(a.K);
  const dim3 grid(a.N / 16), block(kDecThreads);
#define I8MM_DEC(R, P, X)                                                           \
  if (mr == R && spw == P && xs == X) {                                             \
    hipLaunchKernelGGL((k_decode<R, P, X>), grid, block, lds, s, a);                \
    return hipGetLastError();                                                       \
  }
  I8MM_DEC(2, 2, true) I8MM_DEC(2, 4, true) I8MM_DEC(2, 8, true) I8MM_DEC(2, 16, true)
  I8MM_DEC(4, 2, true) I8MM_DEC(4, 4, true) I8MM_DEC(4, 8, true) I8MM_DEC(4, 16, true)
  I8MM_DEC(8, 2, true) I8MM_DEC(8, 4, true) I8MM_DEC(8, 8, true) I8MM_DEC(8, 16, true)
  I8MM_DEC(16, 2, true) I8MM_DEC(16, 4, true) I8MM_DEC(16, 8, true)
  // shapes whose masked X does not fit beside Xq (M = 16 from K = 2880, M = 8 from
  // K = 5536)
  I8MM_DEC(8, 16, false) I8MM_DEC(16, 8, false)
#undef I8MM_DEC
  return hipErrorInvalidValue;
}

}  // namespace i8mm
