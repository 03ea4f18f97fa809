// Decode path: the whole decomposed product for a handful of tokens in one kernel.
//
// "What is 8-bit LLM quantization?", Does INT8 always improve speed?: at decode time the
// gain of int8 weights is the smaller weight stream. With M <= 16 tokens the N x K
// bytes of Wq are the whole cost, so one launch does every step and reads each Wq byte
// from HBM exactly once. One block per 16 output features (32 where N has more 16-row
// groups than the GPU has CUs and 5-8 token rows are held), all of K, P pairs of waves
// (8; 2 for 513-1024 columns of K, 4 for 1025-2048); pair p owns the K-steps (64 columns
// each) SPW p .. SPW p + SPW - 1:
//   * compute wave p loads the 8-column chunks of X of exactly those columns for every
//     token row (these requests go out first: the stream wave of the pair sends only a
//     few weight requests until this X has arrived), finds the outlier columns among
//     them (a keep-mask
//     per column from the largest magnitude over the rows; no exchange: a lane holds
//     every row of its chunks), the rows' partial absmax over the kept columns (DPP
//     over the wave) and its outlier columns in ascending order. The eight compute
//     waves meet through an LDS counter (the stream waves take no part); then each
//     has the row constants, the outlier count and ranks; it loads the weight bytes of
//     its first outlier columns, quantizes its columns into its own LDS rows (an exact
//     pass for the rare values the bracketing pair cannot decide), flags them ready and
//     stages the outlier columns' X and dequantized weights for the epilogue;
//   * stream wave p issues the pair's Wq units (one 1 KB unit per load instruction,
//     straight into registers). A wave that issues this many loads stalls in issue
//     until the memory system accepts them; keeping the stream in waves of its own
//     keeps those stalls away from the activation work. When its compute wave's codes
//     are ready it runs v_mfma_i32_16x16x64_i8 over the pair's steps (Wq unit as the
//     16-row operand, the codes of up to 16 tokens as the other) and stores its int32
//     partials;
//   * after one block barrier, the epilogue sums the eight int32 partials exactly,
//     applies the outer-product dequantization and adds the outlier columns' product,
//     fp16 X times the fp16-rounded dequantized weight fp16(q a_w / 127) summed in fp32
//     in ascending column order, before the single rounding to fp16.
// The compute waves wait for nothing issued after their own X loads, so the activation
// quantization overlaps the weight stream.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace i8mm {

constexpr int kDecMaxM = 16, kDecMaxK = 8192;
constexpr int kPre = 16;    // outlier columns staged while the codes are made
constexpr int kChunkO = 32; // outlier columns per later epilogue pass (at most)
#ifndef I8MM_DEC_EARLY
#define I8MM_DEC_EARLY 2
#endif
constexpr int kEarly = I8MM_DEC_EARLY;  // weight units per stream wave sent before X arrives
// Bound of the LDS waits between the waves of a block (each pass sleeps ~64 clocks: some
// ms in all). Every wave the waits depend on belongs to the same block and runs; the
// bound only guarantees that the kernel ends. On expiry the block writes NaN.
constexpr int kSpinLimit = 1 << 17;

static int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}
// token rows held per thread: M rounded up to a power of two
static int rows_held(int64_t M) { return pow2_at_least(static_cast<int>(M)); }
// Pairs of waves per block (compute waves = stream waves): 8, or fewer where K leaves a
// pair fewer than 8 K-steps and at least 4 token rows are held, so that every lane of a
// compute wave owns a chunk: a wave issues the same instructions however many of its
// lanes hold data, and with 4-16 rows the activation phase is bound by the instructions
// each SIMD issues (9-16 K-steps: 2 pairs, 17-32: 4). With 1-2 rows the work is small and
// 8 pairs, more loads in flight, measured faster.
static int decode_pairs(int64_t M, int64_t K) {
  const int ks = unit_ks(static_cast<int>(K));
  if (rows_held(M) < 4) return 8;
  return ks > 8 && ks <= 16 ? 2 : ks > 16 && ks <= 32 ? 4 : 8;
}
// K-steps (64 columns) per pair: ceil(ceil(K / 64) / pairs) rounded up to a power of two
static int steps_per_wave(int64_t M, int64_t K) {
  const int P = decode_pairs(M, K);
  return pow2_at_least(static_cast<int>((unit_ks(static_cast<int>(K)) + P - 1) / P));
}

// X chunks a thread holds in registers: rows_held(M) x (1, or 2 past 4096 columns), at
// most 16 (64 registers): M <= 16 up to K = 4096, M <= 8 up to K = 8192.
bool decode_supported(int64_t M, int64_t K) {
  if (M < 1 || M > kDecMaxM || K < 16 || K > kDecMaxK) return false;
  return rows_held(M) * (K > 4096 ? 2 : 1) <= 16;
}

// Dynamic LDS: each pair's code rows [rows_held(M)][64 SPW + 16] (rows from M on are
// scratch), the outlier column lists (one segment of 64 SPW shorts per pair), and a sink of
// 8 bytes per lane for the code stores of lanes that own no chunk.
static size_t decode_lds_bytes(int64_t M, int64_t K) {
  const size_t spw = static_cast<size_t>(steps_per_wave(M, K)), P = static_cast<size_t>(decode_pairs(M, K));
  return P * static_cast<size_t>(rows_held(M)) * (64 * spw + 16) + P * 64 * spw * 2 + 64 * 8;
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

// The pair holding outlier rank r (0 <= r < count): the last pair whose first rank is at
// most r (wb: first rank of each pair, nondecreasing).
template <int P>
__device__ __forceinline__ int pair_of_rank(const int (&wb)[P + 1], int r) {
  int w = 0;
#pragma unroll
  for (int i = 1; i < P; ++i) w += r >= wb[i] ? 1 : 0;
  return w;
}

// Half e (runtime, 0..7) of v, as fp16 bits.
__device__ __forceinline__ unsigned half_at(const v8h& v, int e) {
  const v4u u = __builtin_bit_cast(v4u, v);
  const int d = e >> 1;
  const unsigned w = d == 0 ? u[0] : d == 1 ? u[1] : d == 2 ? u[2] : u[3];
  return (e & 1) ? w >> 16 : w & 0xffffu;
}

// Codes of 8 halves from the bracketing pair lo < 127 / a < hi (see quant8_fast): the
// lower bracket's codes, and whether the two disagree anywhere. Both results of a fused
// multiply-add are kRoundMagic + code exactly, so comparing them whole (two at a time)
// compares the codes.
__device__ __forceinline__ v2u quant8_pair(const v8h& x, float lo, float hi, bool& dis) {
  unsigned b1[8], b2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float xf = static_cast<float>(x[e]);
    b1[e] = __builtin_bit_cast(unsigned, __builtin_fmaf(xf, lo, kRoundMagic));
    b2[e] = __builtin_bit_cast(unsigned, __builtin_fmaf(xf, hi, kRoundMagic));
  }
  bool d = false;
#pragma unroll
  for (int e = 0; e < 8; e += 2)
    d |= __builtin_bit_cast(unsigned long long, v2u{b1[e], b1[e + 1]}) !=
         __builtin_bit_cast(unsigned long long, v2u{b2[e], b2[e + 1]});
  dis = d;
  v2u o;
  o[0] = pack_low_bytes(b1[0], b1[1], b1[2], b1[3]);
  o[1] = pack_low_bytes(b1[4], b1[5], b1[6], b1[7]);
  return o;
}

// Waits until the LDS counter reaches target; false if the bound expired.
__device__ __forceinline__ bool lds_wait_geq(int* counter, int target) {
  for (int i = 0; i < kSpinLimit; ++i) {
    if (__hip_atomic_load(counter, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target)
      return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// MR: token rows held per compute thread (M <= MR). SPW: K-steps per pair; a compute
// lane owns the chunks c = 8 SPW p + l + 64 j (j < CC) of every row. RG: 16-row groups of
// Wq per block (2 where N leaves more row groups than the GPU has CUs, at most 8 K-steps
// per pair and 8 rows held: one activation pass then serves 32 output features). The
// two-group form differs in the stream waves, the staged outlier weights and the
// epilogue; each of those has its own branch below, the one-group code unchanged.
template <int MR, int SPW, int P, int RG>
__global__ __launch_bounds__(128 * P) void k_decode(DecodeArgs a) {
  constexpr int kDecPairs = P;
  constexpr int NF = 16 * RG;  // output features per block
  constexpr int CO = kChunkO < 8 * P ? kChunkO : 8 * P;  // later epilogue pass: 16 CO threads
  constexpr int CC = SPW > 8 ? SPW / 8 : 1;  // chunks per lane
  constexpr int WCH = 8 * SPW;               // chunks per pair
  constexpr int WCOLS = 64 * SPW;            // columns per pair
  constexpr int XS = WCOLS + 16;             // code row stride (padding: conflict-free reads)
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int red[kDecPairs][NF][17];
  __shared__ unsigned rmax_s[kDecPairs][16];
  __shared__ int cnt_s[kDecPairs];
  __shared__ float rowmax_s[16];
  __shared__ float xo_s[kChunkO * 16], wo_s[kChunkO * NF];
  // [0]: compute waves past their row maxima; [1 + p]: pair p's codes ready; [9]: a
  // wait expired; [10 + p]: pair p's X has arrived
  __shared__ int sync_s[2 * kDecPairs + 2];

  const int K = a.K, M = a.M, N = a.N;
  const int nchunk = K >> 3, ks = unit_ks(K);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p = wave & (kDecPairs - 1);
  const int n0 = blockIdx.x * NF;
  int8_t* xq_p = reinterpret_cast<int8_t*>(lds) + p * MR * XS;  // pair p's codes [MR][XS]
  short* list_s = reinterpret_cast<short*>(lds + kDecPairs * MR * XS);
  int8_t* sink = reinterpret_cast<int8_t*>(list_s + kDecPairs * WCOLS) + lane * 8;
  // the epilogue's column constant of feature n0 + t % 16 (two row groups: of feature
  // n0 + t % 32, clamped to N - 1): loaded by the compute waves, and by the stream waves
  // too with fewer than 8 pairs or two row groups (the epilogue's threads, or its later
  // outlier passes, then span both)
  float aw_c = 0.0f;

  if (wave < kDecPairs) {
    // ---------------------------------------------------------------- compute wave p
    const int cw = WCH * p;  // first chunk of this pair
    // 1. X. Chunks outside the pair's range or past K read the last chunk (repeats change
    // no maximum; such chunks are masked out below); rows past M read zeros through the
    // buffer resource's range check, without a memory access, so that they add nothing
    // to the maxima and quantize to 0 with no exact work.
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, static_cast<unsigned>(M) * K * 2u);
    v8h xv[MR][CC];
    bool cval[CC];
#pragma unroll
    for (int j = 0; j < CC; ++j) {
      const int lc = lane + 64 * j, c = cw + lc;
      cval[j] = lc < WCH && c < nchunk;
      const int cc = min(c, nchunk - 1);
#pragma unroll
      for (int m = 0; m < MR; ++m)
        xv[m][j] = __builtin_bit_cast(
            v8h, buf_load16(xr, m < M ? static_cast<unsigned>(m * K + cc * 8) * 2u : kOOB));
    }
    if constexpr (RG == 1)
      aw_c = a.a_w[n0 + (tid & 15)];
    else
      aw_c = a.a_w[min(n0 + tid % NF, N - 1)];
    if (tid == 0)
#pragma unroll
      for (int i = 0; i < 2 * kDecPairs + 2; ++i) sync_s[i] = 0;
    lds_barrier();  // the counters are set and the X requests are out
    // X has arrived (this wave has no other load in flight): the stream wave of the pair
    // may send the rest of its weight requests
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): expcnt and lgkmcnt left open
    if (lane == 0)
      __hip_atomic_fetch_add(&sync_s[2 + kDecPairs + p], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);

    // 2. outlier columns ("LLM.int8()", Mixed-precision decomposition: a feature column
    // is an outlier when one of its values reaches the threshold). Magnitudes as fp16
    // bits, two per dword: the largest over the rows against the threshold bits gives
    // a keep-mask per half (0 on outlier columns and on chunks the lane does not own).
    const unsigned tb2 = threshold_bits(a.t) * 0x10001u;
    v4u keep[CC];
    unsigned ob[CC];  // bit e: column 8 c + e of chunk j is an outlier
#pragma unroll
    for (int j = 0; j < CC; ++j) {
      v4u cm = __builtin_bit_cast(v4u, xv[0][j]) & 0x7fff7fffu;
#pragma unroll
      for (int m = 1; m < MR; ++m)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          cm[d] = pk_max_u16(cm[d], __builtin_bit_cast(v4u, xv[m][j])[d] & 0x7fff7fffu);
#pragma unroll
      for (int d = 0; d < 4; ++d) keep[j][d] = cval[j] ? keep_halves(cm[d], tb2) : 0u;
      // one byte of each half's keep-mask (halves 0-3, then 4-7), a different bit taken
      // from each byte, summed: bit e is set where column 8 c + e is kept
      const unsigned p0 = __builtin_amdgcn_perm(keep[j][1], keep[j][0], 0x06040200u);
      const unsigned q0 = __builtin_amdgcn_perm(keep[j][3], keep[j][2], 0x06040200u);
      const unsigned kb = __builtin_amdgcn_sad_u8((p0 & 0x08040201u) | (q0 & 0x80402010u), 0u, 0u);
      ob[j] = cval[j] ? ~kb & 0xFFu : 0u;
    }

    // 3. row absmax over the kept columns ("LLM.int8()", Vector-wise quantization: one
    // constant per row of X): this thread's, then the wave's (DPP), to LDS
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
      for (int m = 0; m < MR; ++m) rmax_s[p][m] = rmx[m];

    // 4. this pair's outlier columns, ascending (chunk group j, then lane, then bit),
    // into its list segment; the count to LDS
    short* list_p = list_s + p * WCOLS;
    int wcount = 0;
#pragma unroll
    for (int j = 0; j < CC; ++j) {
      const int cj = __popc(ob[j]);
      const int incl = wave_prefix_sum(cj);
      int r = wcount + incl - cj;  // local rank of this lane's first outlier column
      for (unsigned bits = ob[j]; bits; bits &= bits - 1u)
        list_p[r++] = static_cast<short>((cw + lane + 64 * j) * 8 + __builtin_ctz(bits));
      wcount += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) {
      cnt_s[p] = wcount;
      __hip_atomic_fetch_add(&sync_s[0], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }

    // 5. gathers for the pair's first kPre outlier columns, the epilogue's operands, sent
    // before the meeting below so that their latency hides under the codes: the weight
    // bytes (lane: column 4 i + l / 16 of the list, feature l % 16) and the fp16 X values
    // (lane: column l % 16, token row l / 16 + 4 i). Which of them the epilogue takes
    // depends on the global ranks, known after the meeting; the extra ones are unused.
    // The list was written to LDS by this wave above, and a wave's LDS accesses complete
    // in order.
    constexpr int kStageLoads = kPre / 4;        // 4 columns per load (16 lanes each)
    constexpr int kXoLoads = (MR + 3) / 4;       // 4 token rows per load
    const int ngather = min(wcount, kPre);       // wave-uniform
    int qv[kStageLoads];
#pragma unroll
    for (int i = 0; i < kStageLoads; ++i) {
      const int k = 4 * i + (lane >> 4);
      const int col = k < ngather ? list_p[k] : 0;
      qv[i] = a.Wq[unit_offset(n0 + (lane & 15), col, ks)];
    }
    // second row group: the same columns for features n0 + 16 + l % 16 (clamped), and
    // the column constants of both of this lane's staged features
    int qv2[RG > 1 ? kStageLoads : 1];
    float aw_st[2] = {0.0f, 0.0f};
    if constexpr (RG > 1) {
      const int nf = min(n0 + 16 + (lane & 15), N - 1);
#pragma unroll
      for (int i = 0; i < kStageLoads; ++i) {
        const int k = 4 * i + (lane >> 4);
        const int col = k < ngather ? list_p[k] : 0;
        qv2[i] = a.Wq[unit_offset(nf, col, ks)];
      }
      aw_st[0] = a.a_w[n0 + (lane & 15)];
      aw_st[1] = a.a_w[nf];
    }
    // (MR <= 2: the X values are copied from the registers below instead, a divergent
    // loop over the few lanes holding an outlier column; measured faster at one token,
    // slower from four on)
    constexpr bool kXoGather = MR > 2;
    unsigned short xg[kXoLoads];
    if constexpr (kXoGather) {
      const int k = lane & 15;
      const int col = k < ngather ? list_p[k] : 0;
#pragma unroll
      for (int i = 0; i < kXoLoads; ++i) {
        const int m = min((lane >> 4) + 4 * i, M - 1);
        xg[i] = reinterpret_cast<const unsigned short*>(a.X)[static_cast<size_t>(m) * K + col];
      }
    }
    if (!lds_wait_geq(&sync_s[0], kDecPairs)) sync_s[kDecPairs + 1] = 1;

    // 6. row constants: lane r combines row r's maxima over the pairs and takes its
    // quantization bracket; the rows' values are read from those lanes below
    float am_l;
    QuantBracket br_l;
    {
      const int r = min(lane, MR - 1);
      unsigned v = 0;
#pragma unroll
      for (int w = 0; w < kDecPairs; ++w) v = max(v, rmax_s[w][r]);
      am_l = half_bits_to_float(v);
      br_l = quant_bracket(am_l);
    }
    if (p == 0 && lane < M) rowmax_s[lane] = am_l;
    int first = 0;  // first global rank of this pair
#pragma unroll
    for (int w = 0; w < kDecPairs; ++w) first += w < p ? cnt_s[w] : 0;
    if constexpr (!kXoGather) {
#pragma unroll
      for (int j = 0; j < CC; ++j) {
        const int cj = __popc(ob[j]);
        const int incl = wave_prefix_sum(cj);
        int r = first + incl - cj;  // global rank of this lane's first outlier column
        for (unsigned bits = ob[j]; bits && r < kPre; bits &= bits - 1u, ++r) {
          const int e = __builtin_ctz(bits);
#pragma unroll
          for (int m = 0; m < MR; ++m)
            if (m < M) xo_s[r * 16 + m] = half_bits_to_float(half_at(xv[m][j], e));
        }
      }
    }

    // 7. codes of this pair's columns into its LDS rows, outlier columns cleared (their
    // codes are 0). Rows past M (zeros) fill the scratch rows. The
    // bracketing pair decides; (row, chunk) slots where it disagrees in some lane are
    // redone with quant8_exact below.
    unsigned long long dm[MR][CC];  // lanes where the pair disagreed
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, br_l.lo), m));
      const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, br_l.hi), m));
#pragma unroll
      for (int j = 0; j < CC; ++j) {
        const int lc = lane + 64 * j;
        v4u u = __builtin_bit_cast(v4u, xv[m][j]);
#pragma unroll
        for (int d = 0; d < 4; ++d) u[d] &= keep[j][d];
        xv[m][j] = __builtin_bit_cast(v8h, u);
        bool dis;
        const v2u o = quant8_pair(xv[m][j], lo, hi, dis);
        dm[m][j] = __ballot(dis);
        *reinterpret_cast<v2u*>(lc < WCH ? xq_p + m * XS + lc * 8 : sink) = o;
      }
    }
    // 8. exact codes where the pair disagreed (values at or within about 2^-15 of a
    // half-integer, exact ties included: in fp16 data every element equal to half its
    // row's absmax is one): per (row, chunk) slot with a disagreement, a wave-uniform
    // branch; in it each lane finds which of its 8 elements disagree and settles them one
    // at a time, each with an exact comparison, its code stored as one byte
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int j = 0; j < CC; ++j)
        if (dm[m][j] != 0) {
          const float am = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, am_l), m));
          const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, br_l.lo), m));
          const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, br_l.hi), m));
          const int lc = lane + 64 * j;
          unsigned em = (dm[m][j] >> lane) & 1u ? quant8_disagreement(xv[m][j], lo, hi) : 0u;
          int8_t* row = lc < WCH ? xq_p + m * XS + lc * 8 : sink;
          while (__ballot(em != 0u) != 0) {  // wave-uniform
            if (em != 0u) {
              const int e = __builtin_ctz(em);
              em &= em - 1u;
              row[e] = static_cast<int8_t>(quant_exact1(half_bits_to_float(half_at(xv[m][j], e)), am, lo));
            }
          }
        }
    // the gathered operands of the pair's outlier columns of global rank < kPre: X as
    // fp32, and W^ = fp16(q a_w / 127), the int8 weight dequantized as the GEMM epilogue
    // forms it
    const int nstage = max(0, min(wcount, kPre - first));  // wave-uniform
#pragma unroll
    for (int i = 0; i < kStageLoads; ++i) {
      const int k = 4 * i + (lane >> 4);
      if constexpr (RG == 1) {
        if (k < nstage)
          wo_s[(first + k) * 16 + (lane & 15)] =
              static_cast<float>(static_cast<_Float16>(__fdiv_rn(static_cast<float>(qv[i]) * aw_c, 127.0f)));
      } else {
        if (k < nstage) {
          wo_s[(first + k) * NF + (lane & 15)] =
              static_cast<float>(static_cast<_Float16>(__fdiv_rn(static_cast<float>(qv[i]) * aw_st[0], 127.0f)));
          wo_s[(first + k) * NF + 16 + (lane & 15)] =
              static_cast<float>(static_cast<_Float16>(__fdiv_rn(static_cast<float>(qv2[i]) * aw_st[1], 127.0f)));
        }
      }
    }
    if constexpr (kXoGather) {
#pragma unroll
      for (int i = 0; i < kXoLoads; ++i) {
        const int k = lane & 15, m = (lane >> 4) + 4 * i;
        if (k < nstage && m < M) xo_s[(first + k) * 16 + m] = half_bits_to_float(xg[i]);
      }
    }
    if (lane == 0)
      __hip_atomic_fetch_add(&sync_s[1 + p], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    // ---------------------------------------------------------------- stream wave p
    lds_barrier();  // after the X requests
    // The weight stream. Wq is unit-tiled: the block's 16 rows are one contiguous run of
    // ks units and unit s is exactly the 16 x 64 A operand of K-step s. Loads are
    // unconditional (steps past K re-read the last unit and are not multiplied). The
    // first kEarly units go out at once, the rest when the pair's X has arrived: sent
    // together, the whole stream queues ahead of the activations in the memory system.
    // Non-temporal loads: each weight byte is read once per call (8x4096x4096 8.20 ->
    // 7.86 us per call).
    const int8_t* wrow =
        a.Wq + static_cast<size_t>(n0 >> 4) * ks * kUnitBytes + (lane & 15) * kUnitK + 16 * (lane >> 4);
    constexpr int E = kEarly < SPW ? kEarly : SPW;
    v4i wf[SPW];
#pragma unroll
    for (int i = 0; i < E; ++i)
      wf[i] = __builtin_nontemporal_load(
          reinterpret_cast<const v4i*>(wrow + static_cast<size_t>(min(SPW * p + i, ks - 1)) * kUnitBytes));
    if (!lds_wait_geq(&sync_s[2 + kDecPairs + p], 1)) sync_s[kDecPairs + 1] = 1;
#pragma unroll
    for (int i = E; i < SPW; ++i)
      wf[i] = __builtin_nontemporal_load(
          reinterpret_cast<const v4i*>(wrow + static_cast<size_t>(min(SPW * p + i, ks - 1)) * kUnitBytes));
    // second row group (clamped to the last one of Wq past N: its products land in
    // outputs that are not stored), all its units after the first group's
    v4i wf2[RG > 1 ? SPW : 1];
    if constexpr (RG > 1) {
      const int8_t* wrow2 = a.Wq + static_cast<size_t>(min((n0 >> 4) + 1, (N >> 4) - 1)) * ks * kUnitBytes +
                            (lane & 15) * kUnitK + 16 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < SPW; ++i)
        wf2[i] = __builtin_nontemporal_load(
            reinterpret_cast<const v4i*>(wrow2 + static_cast<size_t>(min(SPW * p + i, ks - 1)) * kUnitBytes));
    }
    if constexpr (kDecPairs < 8) aw_c = a.a_w[n0 + (tid & 15)];
    if constexpr (RG > 1) aw_c = a.a_w[min(n0 + tid % NF, N - 1)];
    if (!lds_wait_geq(&sync_s[1 + p], 1)) sync_s[kDecPairs + 1] = 1;

    // 9. int8 MFMA: D[feature][token] += Wq[n0 + feature, k] * Xq[token, k] over the
    // pair's steps; tokens past M multiply zeros
    const int tok = lane & 15, kg = lane >> 4;
    v4i acc = v4i{}, acc2 = v4i{};
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const v4i t = *reinterpret_cast<const v4i*>(xq_p + min(tok, M - 1) * XS + 64 * i + 16 * kg);
      const v4i b = tok < M ? t : v4i{};
      if (SPW * p + i < ks) {  // wave-uniform
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[i], b, acc, 0, 0, 0);
        if constexpr (RG > 1) acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf2[i], b, acc2, 0, 0, 0);
      }
    }
    // 16x16 accumulator layout: lane l, register r -> token l % 16, feature 4 (l / 16) + r
#pragma unroll
    for (int r = 0; r < 4; ++r) red[p][4 * kg + r][tok] = acc[r];
    if constexpr (RG > 1)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[p][16 + 4 * kg + r][tok] = acc2[r];
  }
  lds_barrier();

  // 11. epilogue: thread t < 256 -> (token m, output feature n0 + nl). The int32 partials
  // of the pairs are summed exactly; the outlier product in fp32, ascending columns, the
  // first kPre from the staged values, the rest CO at a time from global memory.
  int wb[kDecPairs + 1];
  wb[0] = 0;
#pragma unroll
  for (int w = 0; w < kDecPairs; ++w) wb[w + 1] = wb[w] + cnt_s[w];
  const int count = wb[kDecPairs];
  const int npre = min(count, kPre);
  if constexpr (RG == 1) {
    const int m = tid >> 4, nl = tid & 15;
    float yo = 0.0f;
    if (tid < 256)
      for (int r = 0; r < npre; ++r) yo = __builtin_fmaf(xo_s[r * 16 + m], wo_s[r * 16 + nl], yo);
    for (int r0 = kPre; r0 < count; r0 += CO) {  // block-uniform trip count
      lds_barrier();  // the staged values above are read
      const int rn = min(CO, count - r0);
      if (tid < CO * 16) {
        const int pr = tid >> 4, pq = tid & 15;
        int col = 0;
        if (pr < rn) {
          const int w = pair_of_rank<kDecPairs>(wb, r0 + pr);
          col = list_s[w * WCOLS + r0 + pr - wb[w]];
        }
        const int q = a.Wq[unit_offset(n0 + pq, col, ks)];
        const _Float16 x = a.X[static_cast<size_t>(min(pq, M - 1)) * K + col];
        wo_s[pr * 16 + pq] = pr < rn ? static_cast<float>(static_cast<_Float16>(
                                           __fdiv_rn(static_cast<float>(q) * aw_c, 127.0f)))
                                     : 0.0f;
        xo_s[pr * 16 + pq] = pr < rn && pq < M ? static_cast<float>(x) : 0.0f;
      }
      lds_barrier();
      if (tid < 256)
        for (int r = 0; r < rn; ++r) yo = __builtin_fmaf(xo_s[r * 16 + m], wo_s[r * 16 + nl], yo);
    }
    const bool overflow = count > a.max_outliers;
    const bool expired = sync_s[kDecPairs + 1] != 0;
    if (tid < 256 && m < M) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < kDecPairs; ++w) s += red[w][nl][m];
      const float y = static_cast<float>(s) * (rowmax_s[m] * kInvQMax2) * aw_c + yo;
      a.Y[static_cast<size_t>(m) * N + n0 + nl] =
          overflow || expired ? static_cast<_Float16>(__builtin_nanf("")) : static_cast<_Float16>(y);
      if (a.acc_out) a.acc_out[static_cast<size_t>(m) * N + n0 + nl] = s;
    }
  } else {
    // two row groups: thread t < 16 NF -> (token t / NF, feature n0 + t % NF); later
    // passes stage weights by thread t < CO NF (rank t / NF, feature t % NF, that of its
    // own column constant) and X by thread t < 16 CO (rank t / 16, token t % 16)
    const int m = tid / NF, nl = tid % NF;
    float yo = 0.0f;
    if (tid < 16 * NF)
      for (int r = 0; r < npre; ++r) yo = __builtin_fmaf(xo_s[r * 16 + m], wo_s[r * NF + nl], yo);
    auto col_of_rank = [&](int r) {
      const int w = pair_of_rank<kDecPairs>(wb, r);
      return static_cast<int>(list_s[w * WCOLS + r - wb[w]]);
    };
    for (int r0 = kPre; r0 < count; r0 += CO) {  // block-uniform trip count
      lds_barrier();  // the staged values above are read
      const int rn = min(CO, count - r0);
      if (tid < CO * NF) {
        const int pr = tid / NF;
        const int col = pr < rn ? col_of_rank(r0 + pr) : 0;
        const int q = a.Wq[unit_offset(min(n0 + nl, N - 1), col, ks)];
        wo_s[pr * NF + nl] = pr < rn ? static_cast<float>(static_cast<_Float16>(
                                           __fdiv_rn(static_cast<float>(q) * aw_c, 127.0f)))
                                     : 0.0f;
      }
      if (tid < CO * 16) {
        const int pr = tid >> 4, pq = tid & 15;
        const int col = pr < rn ? col_of_rank(r0 + pr) : 0;
        const _Float16 x = a.X[static_cast<size_t>(min(pq, M - 1)) * K + col];
        xo_s[pr * 16 + pq] = pr < rn && pq < M ? static_cast<float>(x) : 0.0f;
      }
      lds_barrier();
      if (tid < 16 * NF)
        for (int r = 0; r < rn; ++r) yo = __builtin_fmaf(xo_s[r * 16 + m], wo_s[r * NF + nl], yo);
    }
    const bool overflow = count > a.max_outliers;
    const bool expired = sync_s[kDecPairs + 1] != 0;
    if (tid < 16 * NF && m < M && n0 + nl < N) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < kDecPairs; ++w) s += red[w][nl][m];
      const float y = static_cast<float>(s) * (rowmax_s[m] * kInvQMax2) * aw_c + yo;
      a.Y[static_cast<size_t>(m) * N + n0 + nl] =
          overflow || expired ? static_cast<_Float16>(__builtin_nanf("")) : static_cast<_Float16>(y);
      if (a.acc_out) a.acc_out[static_cast<size_t>(m) * N + n0 + nl] = s;
    }
  }
  if (blockIdx.x == 0 && tid == 0) {
    a.status[0] = count > a.max_outliers ? 7 : 0;
    a.status[1] = count;
  }
}

static int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      return 256;
    cus = v;
  }
  return cus;
}

// Row groups per block: 2 where the 16-row groups of Wq outnumber the CUs (with one per
// block the blocks would run in several rounds, each repeating the activation work), with
// 8 pairs of waves, at most 8 K-steps per pair (the stream waves then hold 2 x 8 units)
// and 8 token rows held. Measured per call: 8 x 4096 x 8192 14.0 -> 9.4 us, 8 x 4096 x
// 16384 26.0 -> 16.9; with 1-4 rows, where the activation work is small, the doubled
// weight stream per block lost (1 x 4096 x 12288 11.6 -> 14.3, 4 x 4096 x 11008 13.0 ->
// 14.4), and 16 rows leave the compute waves no registers for it.
static int decode_row_groups(int64_t M, int64_t K, int64_t N) {
  return decode_pairs(M, K) == 8 && steps_per_wave(M, K) <= 8 && rows_held(M) == 8 &&
                 N / 16 > device_cus()
             ? 2
             : 1;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  const size_t lds = decode_lds_bytes(a.M, a.K);
  const int mr = rows_held(a.M), spw = steps_per_wave(a.M, a.K), pairs = decode_pairs(a.M, a.K);
  const int rg = decode_row_groups(a.M, a.K, a.N);
  const dim3 grid((a.N / 16 + rg - 1) / rg), block(128 * pairs);
#define I8MM_DEC(R, W, P, G)                                                     \
  if (mr == R && spw == W && pairs == P && rg == G) {                            \
    hipLaunchKernelGGL((k_decode<R, W, P, G>), grid, block, lds, s, a);          \
    return hipGetLastError();                                                    \
  }
  I8MM_DEC(1, 1, 8, 1) I8MM_DEC(1, 2, 8, 1) I8MM_DEC(1, 4, 8, 1) I8MM_DEC(1, 8, 8, 1) I8MM_DEC(1, 16, 8, 1)
  I8MM_DEC(2, 1, 8, 1) I8MM_DEC(2, 2, 8, 1) I8MM_DEC(2, 4, 8, 1) I8MM_DEC(2, 8, 8, 1) I8MM_DEC(2, 16, 8, 1)
  I8MM_DEC(4, 1, 8, 1) I8MM_DEC(4, 2, 8, 1) I8MM_DEC(4, 4, 8, 1) I8MM_DEC(4, 8, 8, 1) I8MM_DEC(4, 16, 8, 1)
  I8MM_DEC(8, 1, 8, 1) I8MM_DEC(8, 2, 8, 1) I8MM_DEC(8, 4, 8, 1) I8MM_DEC(8, 8, 8, 1) I8MM_DEC(8, 16, 8, 1)
  I8MM_DEC(16, 1, 8, 1) I8MM_DEC(16, 2, 8, 1) I8MM_DEC(16, 4, 8, 1) I8MM_DEC(16, 8, 8, 1)
  I8MM_DEC(4, 8, 2, 1) I8MM_DEC(8, 8, 2, 1) I8MM_DEC(16, 8, 2, 1)
  I8MM_DEC(4, 8, 4, 1) I8MM_DEC(8, 8, 4, 1) I8MM_DEC(16, 8, 4, 1)
  I8MM_DEC(8, 1, 8, 2) I8MM_DEC(8, 2, 8, 2) I8MM_DEC(8, 4, 8, 2) I8MM_DEC(8, 8, 8, 2)
#undef I8MM_DEC
  return hipErrorInvalidValue;
}

}  // namespace i8mm
