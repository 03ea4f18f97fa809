// Outlier detection and vector-wise row quantization of the activations.
//
// "8-bit Matrix Multiplication for Large Language Models", Summary & Methodology
// Analysis, and "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale",
// Abstract: the emergent outlier feature dimensions (columns of X) are isolated and
// multiplied in 16 bit; everything else is quantized with one normalization constant
// per inner product. "Compress your LLMs", Vector-wise quantization: one constant per
// row of the input matrix. A column j is an outlier when some row has |X[i,j]| >= t;
// the row constant is the absmax over the remaining columns.
//
// Two launches, because every row needs the complete column mask before it can pick
// its constant:
//   k_outlier_mask  column strips x row chunks -> per-chunk column flag words (no
//                   atomics and no pre-zeroed memory: every word is written).
//   k_quant_rows    ORs the chunk flags, ranks the outlier columns with a block scan,
//                   then one wave per row: absmax over kept columns, quantize, store
//                   Xq (row-major, or unit-tiled for the GEMM); gathers the fp16
//                   outlier activations Xo; block 0 stores the ranked column list.
//                   Extra blocks (one-call path) gather the dequantized int8 weight
//                   rows of the outlier columns, WoT.
// Both are HBM-bound streaming kernels (X read, Xq written).
#include "common.hpp"
#include "launch.hpp"

namespace i8mm {

// Block (strip, chunk): 64 columns x rows [chunk*rpc, +rpc). 8 threads x 16 B per row;
// each thread keeps the running magnitude max of its 8 columns as packed u16 (finite
// and infinite halves order like their magnitude bits) and tests it against the
// threshold once at the end.
__global__ __launch_bounds__(256) void k_outlier_mask(const _Float16* __restrict__ X, int M, int K,
                                                      float t, int rpc,
                                                      uint32_t* __restrict__ partial, int W,
                                                      int merge) {
  const int tid = threadIdx.x;
  const int cg = tid & 7;
  const int col0 = blockIdx.x * 64 + cg * 8;
  const int r_begin = blockIdx.y * rpc;
  const int r_end = min(M, r_begin + rpc);
  unsigned cm[4] = {0u, 0u, 0u, 0u};
  if (col0 < K) {
#pragma unroll 8
    for (int r = r_begin + (tid >> 3); r < r_end; r += 32) {
      const v4u u = *reinterpret_cast<const v4u*>(X + static_cast<size_t>(r) * K + col0);
#pragma unroll
      for (int d = 0; d < 4; ++d) cm[d] = pk_max_u16(cm[d], u[d] & 0x7fff7fffu);
    }
  }
  const unsigned tb = threshold_bits(t);
  unsigned flags = 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    flags |= static_cast<unsigned>((cm[d] & 0xffffu) >= tb) << (2 * d);
    flags |= static_cast<unsigned>((cm[d] >> 16) >= tb) << (2 * d + 1);
  }
  if (col0 >= K || r_begin >= r_end) flags = 0;
  flags |= __shfl_xor(flags, 8, 64);
  flags |= __shfl_xor(flags, 16, 64);
  flags |= __shfl_xor(flags, 32, 64);
  __shared__ unsigned s[4][8];
  if ((tid & 63) < 8) s[tid >> 6][cg] = flags;
  __syncthreads();
  if (tid < 2) {
    unsigned word = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = tid * 4 + g;
      word |= (s[0][c] | s[1][c] | s[2][c] | s[3][c]) << (8 * g);
    }
    const int w = blockIdx.x * 2 + tid;
    if (merge) {
      if (w < W && word) atomicOr(partial + w, word);
    } else if (w < W) {
      partial[static_cast<size_t>(blockIdx.y) * W + w] = word;
    }
  }
}

__global__ __launch_bounds__(256) void k_zero_words(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// One wave quantizes one row. CH > 0: the row is held in registers (CH chunks of 8
// halves per lane, K <= 512 * CH) and read once; CH == 0: streamed twice.
// Xq goes row-major (ks == 0) or unit-tiled with ks = unit_ks(K) units per row group,
// in which case the row's K padding is written as zero codes.
// Outlier columns are cleared in the registers (drop_halves), the row constant is a
// packed u16 magnitude max reduced over the wave with DPP, and the codes come from the
// bracketing pair of fused multiply-adds (quant8_fast); groups where the pair
// disagrees take quant8_exact.
// Loads a row into registers for quant_one_row<CH> (CH > 0): chunk c = t + STRIDE i
// (STRIDE threads share the row), through a buffer resource over the row so that chunks
// past its end read as zeros. (A select of the loaded value against zero would make
// each load wait for its data before the next one issues.) NT: non-temporal loads
// (cache-policy bit nt), for a single streaming pass over a large X.
template <int CH, int STRIDE = 64, bool NT = false>
__device__ __forceinline__ void load_row(const _Float16* __restrict__ xr, int K, int t,
                                         v8h (&v)[CH > 0 ? CH : 1]) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(xr, static_cast<unsigned>(K) * 2u);
#pragma unroll
  for (int i = 0; i < (CH > 0 ? CH : 1); ++i) {
    const int off = static_cast<int>(static_cast<unsigned>(t + STRIDE * i) * 16u);
    v[i] = __builtin_bit_cast(v8h, NT ? __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2)
                                      : __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  }
}

template <int CH>
__device__ __forceinline__ void quant_one_row(const _Float16* __restrict__ xr, int K,
                                              const uint32_t* words, int8_t* __restrict__ Xq,
                                              int row, int ks, float* a_x_row, int lane,
                                              v8h (&v)[CH > 0 ? CH : 1]) {
  const int nchunk = K >> 3;
  auto dst = [&](int c) -> int8_t* {
    return ks ? Xq + unit_offset(row, c * 8, ks) : Xq + static_cast<size_t>(row) * K + c * 8;
  };
  auto chunk_mask = [&](int c) -> unsigned { return (words[c >> 2] >> ((c & 3) << 3)) & 0xFFu; };
  float m;
  if constexpr (CH > 0) {
    unsigned pm = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = lane + 64 * i;
      const unsigned mb = c < nchunk ? chunk_mask(c) : 0u;
      if (mb) drop_halves(v[i], mb);  // outlier columns are rare
      const v4u u = __builtin_bit_cast(v4u, v[i]);
#pragma unroll
      for (int d = 0; d < 4; ++d) pm = pk_max_u16(pm, u[d] & 0x7fff7fffu);
    }
    m = wave_max_half_pairs(pm);
    const QuantBracket br = quant_bracket(m);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = lane + 64 * i;
      unsigned dis;
      v2u o = quant8_fast(v[i], br, dis);
      if (dis) o = quant8_exact(v[i], m, br.lo);  // rare; many waves share the code
      if (c < nchunk) *reinterpret_cast<v2u*>(dst(c)) = o;
    }
  } else {
    unsigned pm = 0;
    for (int c = lane; c < nchunk; c += 64) {
      v8h t = *reinterpret_cast<const v8h*>(xr + c * 8);
      const unsigned mb = chunk_mask(c);
      if (mb) drop_halves(t, mb);
      const v4u u = __builtin_bit_cast(v4u, t);
#pragma unroll
      for (int d = 0; d < 4; ++d) pm = pk_max_u16(pm, u[d] & 0x7fff7fffu);
    }
    m = wave_max_half_pairs(pm);
    const QuantBracket br = quant_bracket(m);
    for (int c = lane; c < nchunk; c += 64) {
      v8h t = *reinterpret_cast<const v8h*>(xr + c * 8);
      const unsigned mb = chunk_mask(c);
      if (mb) drop_halves(t, mb);
      unsigned dis;
      v2u o = quant8_fast(t, br, dis);
      if (dis) o = quant8_exact(t, m, br.lo);
      *reinterpret_cast<v2u*>(dst(c)) = o;
    }
  }
  if (lane == 0) *a_x_row = m;
  if (ks)
    for (int c = nchunk + lane; c < ks * 8; c += 64) *reinterpret_cast<v2u*>(dst(c)) = v2u{0u, 0u};
}

// One row quantized by a whole 256-thread block (for a handful of rows, where a wave
// per row would leave the GPU idle and make each row a long serial chain): thread t
// takes chunks t + 256 i (CH > 0, held in registers), the row constant is reduced over
// the wave with DPP and over the 4 waves through red_s, then the same codes as
// quant_one_row.
template <int CH>
__device__ __forceinline__ void quant_row_block(const _Float16* __restrict__ xr, int K,
                                                const uint32_t* words, int8_t* __restrict__ Xq,
                                                int row, int ks, float* a_x_row, int tid,
                                                v8h (&v)[CH], unsigned* red_s) {
  static_assert(CH > 0, "registers only");
  const int nchunk = K >> 3;
  auto dst = [&](int c) -> int8_t* {
    return ks ? Xq + unit_offset(row, c * 8, ks) : Xq + static_cast<size_t>(row) * K + c * 8;
  };
  unsigned pm = 0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + 256 * i;
    const unsigned mb = c < nchunk ? (words[c >> 2] >> ((c & 3) << 3)) & 0xFFu : 0u;
    if (mb) drop_halves(v[i], mb);  // outlier columns are rare
    const v4u u = __builtin_bit_cast(v4u, v[i]);
#pragma unroll
    for (int d = 0; d < 4; ++d) pm = pk_max_u16(pm, u[d] & 0x7fff7fffu);
  }
  const unsigned wm = wave_max_u32(max(pm & 0xffffu, pm >> 16));
  if ((tid & 63) == 0) red_s[tid >> 6] = wm;
  lds_barrier();
  const unsigned h = max(max(red_s[0], red_s[1]), max(red_s[2], red_s[3]));
  const float m = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(h)));
  const QuantBracket br = quant_bracket(m);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + 256 * i;
    unsigned dis;
    v2u o = quant8_fast(v[i], br, dis);
    if (dis) o = quant8_exact(v[i], m, br.lo);
    if (c < nchunk) *reinterpret_cast<v2u*>(dst(c)) = o;
  }
  if (tid == 0) *a_x_row = m;
  if (ks)
    for (int c = nchunk + tid; c < ks * 8; c += 256) *reinterpret_cast<v2u*>(dst(c)) = v2u{0u, 0u};
}

// Blocks [0, nrow): rows 4b..4b+3 (one wave each; WIDE: row b, the whole block).
// Blocks [nrow, nrow + ngather): WoT
// rows n = 256 (b - nrow) + tid. Dynamic LDS: W mask words, then o_lds ranked columns.
template <int CH, bool WIDE>
__global__ __launch_bounds__(256) void k_quant_rows(QuantRowsArgs a, int W, int o_lds, int nrow) {
  extern __shared__ uint32_t lds[];
  uint32_t* words = lds;
  int* idx_s = reinterpret_cast<int*>(lds + W);
  __shared__ int wave_tot[4];
  __shared__ unsigned red_s[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool row_block = static_cast<int>(blockIdx.x) < nrow;
  const int row = WIDE ? static_cast<int>(blockIdx.x) : blockIdx.x * 4 + wave;
  // 1. column mask = OR of the row-chunk flags. The loads of two words x 8 row chunks
  // are issued together (chunk indices clamped to the last one: a repeat changes no
  // OR), so that a block waits about once for them rather than once per chunk.
  for (int w0 = tid; w0 < W; w0 += 512) {
    const int w1 = min(w0 + 256, W - 1);  // a repeat of word W - 1 past the end
    uint32_t v0 = 0, v1 = 0;
    for (int rc0 = 0; rc0 < a.R; rc0 += 8) {
      uint32_t t0[8], t1[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const size_t base = static_cast<size_t>(min(rc0 + q, a.R - 1)) * W;
        t0[q] = a.partial[base + w0];
        t1[q] = a.partial[base + w1];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        v0 |= t0[q];
        v1 |= t1[q];
      }
    }
    words[w0] = v0;
    if (w0 + 256 < W) words[w0 + 256] = v1;
  }
  lds_barrier();
  // 2. rank the outlier columns: thread t owns words [t*per, (t+1)*per)
  const int per = (W + 255) / 256;
  const int w0 = min(W, tid * per), w1 = min(W, w0 + per);
  int mine = 0;
  for (int w = w0; w < w1; ++w) mine += __popc(words[w]);
  const int incl = wave_prefix_sum(mine);
  if (lane == 63) wave_tot[wave] = incl;
  lds_barrier();
  int before = incl - mine;
  for (int i = 0; i < wave; ++i) before += wave_tot[i];
  const int count = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
  for (int w = w0, r = before; w < w1; ++w) {
    uint32_t bits = words[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (r < o_lds) idx_s[r] = w * 32 + b;
      ++r;
    }
  }
  lds_barrier();

  if (blockIdx.x == 0) {
    if (tid == 0) {
      if (a.count_out) a.count_out[0] = count;
      if (a.status_out) a.status_out[0] = count > a.max_outliers ? 7 : 0;
    }
    if (a.idx_out)
      for (int r = tid; r < min(count, a.max_outliers); r += 256) a.idx_out[r] = idx_s[r];
  }
  // outlier columns actually carried (padded to the 16-wide fp16 MFMA step)
  const int o_pad = min((count + 15) & ~15, a.o_stride);

  if (row_block) {
    if (row >= a.M) return;  // block-uniform when WIDE
    const _Float16* xr = a.X + static_cast<size_t>(row) * a.K;
    v8h v[CH > 0 ? CH : 1];
    if constexpr (WIDE) {
      load_row<CH, 256>(xr, a.K, tid, v);
      quant_row_block<CH>(xr, a.K, words, a.Xq, row, a.xq_tiled ? unit_ks(a.K) : 0, a.a_x + row,
                          tid, v, red_s);
    } else {
      if constexpr (CH > 0) load_row<CH>(xr, a.K, lane, v);
      quant_one_row<CH>(xr, a.K, words, a.Xq, row, a.xq_tiled ? unit_ks(a.K) : 0, a.a_x + row, lane, v);
    }
    if (a.Xo) {
      _Float16* xo = a.Xo + static_cast<size_t>(row) * a.o_stride;
      const int t0 = WIDE ? tid : lane, ts = WIDE ? 256 : 64;
      for (int r = t0; r < o_pad; r += ts) xo[r] = r < count ? xr[idx_s[r]] : _Float16(0);
    }
  } else {
    // WoT[n, r] = fp16(Wq[n, O_r] * a_w[n] / 127): the outlier columns' weights,
    // dequantized from the int8 copy that is the only weight kept in memory.
    const int n = (blockIdx.x - nrow) * 256 + tid;
    if (n >= a.N) return;
    const float aw = a.a_w[n];
    const int ks = unit_ks(a.K);
    _Float16* dst = a.WoT + static_cast<size_t>(n) * a.o_stride;
    for (int r0 = 0; r0 < o_pad; r0 += 8) {
      v8h o;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = r0 + e;
        o[e] = r < count ? static_cast<_Float16>(
                               __fdiv_rn(static_cast<float>(a.Wq[unit_offset(n, idx_s[r], ks)]) * aw, 127.0f))
                         : _Float16(0);
      }
      *reinterpret_cast<v8h*>(dst + r0) = o;
    }
  }
}

hipError_t launch_outlier_mask(const _Float16* X, int M, int K, float t, int R,
                               uint32_t* partial, hipStream_t s) {
  const int W = (K + 31) / 32;
  const int rpc = (M + R - 1) / R;
  hipLaunchKernelGGL(k_outlier_mask, dim3((K + 63) / 64, R), dim3(256), 0, s, X, M, K, t, rpc,
                     partial, W, 0);
  return hipGetLastError();
}

hipError_t launch_outlier_mask_merged(const _Float16* X, int M, int K, float t, int R,
                                      uint32_t* mask, hipStream_t s) {
  const int W = (K + 31) / 32;
  const int rpc = (M + R - 1) / R;
  hipLaunchKernelGGL(k_zero_words, dim3((W + 255) / 256), dim3(256), 0, s, mask, W);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_outlier_mask, dim3((K + 63) / 64, R), dim3(256), 0, s, X, M, K, t, rpc, mask,
                     W, 1);
  return hipGetLastError();
}

// A row per wave, or, below 256 rows (where M waves would leave most of the GPU idle
// and each row one long serial chain), a row per 4-wave block.
hipError_t launch_quant_rows(const QuantRowsArgs& a, hipStream_t s) {
  const int W = (a.K + 31) / 32;
  const int o_lds = a.o_stride > a.max_outliers ? a.o_stride : a.max_outliers;
  const size_t lds = static_cast<size_t>(W + o_lds) * 4;
  const int nchunk = a.K / 8;
  const bool wide = a.M < 256 && (nchunk + 255) / 256 <= 16;
  const int nrow = wide ? a.M : (a.M + 3) / 4;
  const int ngather = a.WoT ? (a.N + 255) / 256 : 0;
  const dim3 grid(nrow + ngather), block(256);
#define I8MM_QR(CHV, WV) hipLaunchKernelGGL((k_quant_rows<CHV, WV>), grid, block, lds, s, a, W, o_lds, nrow)
  if (wide) {
    const int per_thread = (nchunk + 255) / 256;
    if (per_thread <= 1) I8MM_QR(1, true);
    else if (per_thread <= 2) I8MM_QR(2, true);
    else if (per_thread <= 4) I8MM_QR(4, true);
    else if (per_thread <= 8) I8MM_QR(8, true);
    else I8MM_QR(16, true);
  } else {
    const int per_lane = (nchunk + 63) / 64;
    if (per_lane <= 1) I8MM_QR(1, false);
    else if (per_lane <= 2) I8MM_QR(2, false);
    else if (per_lane <= 4) I8MM_QR(4, false);
    else if (per_lane <= 8) I8MM_QR(8, false);
    else if (per_lane <= 16) I8MM_QR(16, false);
    else if (per_lane <= 24) I8MM_QR(24, false);
    else if (per_lane <= 32) I8MM_QR(32, false);
    else if (per_lane <= 40) I8MM_QR(40, false);
    else I8MM_QR(0, false);
  }
#undef I8MM_QR
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// One pass over X (k_quant_pass), then a two-launch fix-up (k_quant_or, k_quant_fix).
//
// The outlier set O is global (a column is an outlier when any row reaches t), yet a
// row needs O only to leave columns out of its constant and its codes. Pass 1 therefore
// quantizes each row, as it streams by, under the provisional constant
// a' = max{|x| : |x| < t} of that row, its own flagged entries cleared. a' bounds the
// exact constant a = max{|x_j| : j not in O} from above, and equals it whenever some
// column where the row reaches a' is not in O: then every code already is the exact one,
// except at outlier columns flagged only by other rows, which must become 0. Each block
// ORs the flags of its rows into an LDS column mask and publishes it (a short ascending
// column list, or the whole mask). k_quant_or ORs the published flags into the call's
// mask of O; each k_quant_fix block ranks O and, per row, either zeroes the provisional
// codes at the outlier columns or, when every column that reached a' is an outlier (or
// O is too large to patch), reads the row again and requantizes it under the exact
// mask. Either way the codes, the row constants and the ranked column list are those of
// the two-launch path above.

bool quant_fused_supported(int64_t K) { return K <= 256 * 8 * kFusedMaxChunks; }

// Enough pass-1 blocks to fill the chip once: 256 CUs times the blocks one CU holds at
// the kernel's register use for this row length (a block's rows are a serial chain of
// load latencies, so fewer rows per block is faster while the blocks still fit), at
// most kFusedMaxBlocks (every fix-up block reads every block's published flags).
void quant_fused_geometry(int64_t M, int64_t K, int* rows_per_block, int* nblk) {
  const int64_t per = (K / 8 + 255) / 256;
  const int64_t per_cu = per <= 2 ? 8 : per <= 4 ? 5 : per <= 6 ? 4 : per <= 8 ? 3 : per <= 12 ? 2 : 1;
  int64_t target = 256 * per_cu;
  if (target > kFusedMaxBlocks) target = kFusedMaxBlocks;
  const int64_t rpb = (M + target - 1) / target;
  *rows_per_block = static_cast<int>(rpb);
  *nblk = static_cast<int>((M + rpb - 1) / rpb);
}

constexpr int kListSlot = 4 + kFlagListCap;  // ints per published list: count, 3 pad, columns

// Block b: rows b, b + nblk, b + 2 nblk, ... (at most rows_per_block of them), each held
// by the whole block (thread t takes chunks t + 256 i), the next row's loads in flight
// while the current one is processed. Interleaved rather than consecutive rows: the
// blocks' first loads then cover one contiguous stretch of X (13B down pass: 62 -> 58 us).
template <int CH, bool NT>
__global__ __launch_bounds__(256) void k_quant_pass(FusedQuantArgs a) {
  extern __shared__ uint32_t mask_s[];  // the block's column flags, ceil(K / 32) words
  __shared__ unsigned red_s[2][4];
  __shared__ int tot_s[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, W = (K + 31) >> 5, nchunk = K >> 3, ks = unit_ks(K);
  const unsigned tb = threshold_bits(a.t);
  for (int w = tid; w < W; w += 256) mask_s[w] = 0u;
  // block 0 clears the call's outlier mask, which the fix-up's first launch ORs into
  if (blockIdx.x == 0)
    for (int w = tid; w < W; w += 256) a.gmask[w] = 0u;
  lds_barrier();
  const int S = a.nblk, first = blockIdx.x, last = first + (a.M - 1 - first) / S * S;

  auto process = [&](v8h (&v)[CH], int row, int par) {
    // flags |x| >= t (rare: their halves are cleared and ORed into the block mask) and
    // the largest kept magnitude, per chunk and over the row
    unsigned cmx[CH];
    unsigned pm = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 256 * i;
      v4u u = __builtin_bit_cast(v4u, v[i]) & 0x7fff7fffu;
      unsigned cm = pk_max_u16(pk_max_u16(u[0], u[1]), pk_max_u16(u[2], u[3]));
      if (max(cm & 0xffffu, cm >> 16) >= tb && c < nchunk) {
        unsigned fm = 0;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          fm |= static_cast<unsigned>((u[d] & 0xffffu) >= tb) << (2 * d);
          fm |= static_cast<unsigned>((u[d] >> 16) >= tb) << (2 * d + 1);
        }
        drop_halves(v[i], fm);
        atomicOr(&mask_s[c >> 2], fm << ((c & 3) << 3));
        u = __builtin_bit_cast(v4u, v[i]) & 0x7fff7fffu;
        cm = pk_max_u16(pk_max_u16(u[0], u[1]), pk_max_u16(u[2], u[3]));
      }
      cmx[i] = max(cm & 0xffffu, cm >> 16);
      pm = max(pm, cmx[i]);
    }
    const unsigned wm = wave_max_u32(pm);
    if (lane == 0) red_s[par][wave] = wm;
    lds_barrier();
    const unsigned hm = max(max(red_s[par][0], red_s[par][1]), max(red_s[par][2], red_s[par][3]));
    const float m = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(hm)));
    const QuantBracket br = quant_bracket(m);
    // codes under a' (K padding included: those chunks hold zeros), and the smallest
    // column of this wave whose magnitude is a', kept as 0x7fffffff - column so that
    // the wave's unsigned max finds it (0: none)
    // Stores go through a buffer resource over the row's 16-row group, so that chunks
    // past the K padding fall outside it and are dropped: every store is issued, and the
    // compiler can count them when it waits for the next row's loads. (256 CH >= ks * 8
    // always, since ks * 8 is nchunk rounded up to a multiple of 8 and 256 CH is it
    // rounded up to a multiple of 256: the padding chunks are all covered here.)
    const __amdgpu_buffer_rsrc_t qs =
        make_rsrc(a.Xq + static_cast<size_t>(row >> 4) * ks * kUnitBytes,
                  static_cast<unsigned>(ks) * kUnitBytes);
    const unsigned row_off = static_cast<unsigned>(row & 15) * kUnitK;
    unsigned best = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 256 * i;
      unsigned dis;
      v2u o = quant8_fast(v[i], br, dis);
      if (dis) o = quant8_exact(v[i], m, br.lo);
      __builtin_amdgcn_raw_buffer_store_b64(
          o, qs, static_cast<int>((c >> 3) * kUnitBytes + row_off + (c & 7) * 8), 0, 0);
      if (hm != 0u && cmx[i] == hm) {
        const v4u u = __builtin_bit_cast(v4u, v[i]);
        int e = 0;
#pragma unroll
        for (int d = 3; d >= 0; --d) {
          if (((u[d] >> 16) & 0x7fffu) == hm) e = 2 * d + 1;
          if ((u[d] & 0x7fffu) == hm) e = 2 * d;
        }
        best = max(best, 0x7fffffffu - static_cast<unsigned>(c * 8 + e));
      }
    }
    const unsigned wb = wave_max_u32(best);
    if (lane == 0)
      a.jstar[static_cast<size_t>(row) * 4 + wave] = wb ? static_cast<int>(0x7fffffffu - wb) : -1;
    if (tid == 0) a.a_x[row] = m;
  };

  // The next row's loads are always issued (past the block's last row they re-read it):
  // loads under a condition make the compiler wait for them where the paths join.
  {
    v8h A[CH], B[CH];
    load_row<CH, 256, NT>(a.X + static_cast<size_t>(first) * K, K, tid, A);
    for (int row = first; row <= last; row += 2 * S) {
      load_row<CH, 256, NT>(a.X + static_cast<size_t>(min(row + S, last)) * K, K, tid, B);
      process(A, row, 0);
      if (row + S > last) break;
      load_row<CH, 256, NT>(a.X + static_cast<size_t>(min(row + 2 * S, last)) * K, K, tid, A);
      process(B, row + S, 1);
    }
  }

  // publish the block's flags: the column list (ascending) when short, else the whole
  // mask. Thread t owns mask words [t*per, (t+1)*per); a block prefix sum places them.
  lds_barrier();
  const int per = (W + 255) / 256;
  const int w0 = min(W, tid * per), w1 = min(W, w0 + per);
  int mine = 0;
  for (int w = w0; w < w1; ++w) mine += __popc(mask_s[w]);
  const int incl = wave_prefix_sum(mine);
  if (lane == 63) tot_s[wave] = incl;
  lds_barrier();
  int before = incl - mine, total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    before += i < wave ? tot_s[i] : 0;
    total += tot_s[i];
  }
  int32_t* lst = a.lists + static_cast<size_t>(blockIdx.x) * kListSlot;
  if (total <= kFlagListCap) {
    for (int w = w0, r = before; w < w1; ++w) {
      uint32_t bits = mask_s[w];
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1;
        lst[4 + r++] = w * 32 + b;
      }
    }
    if (tid == 0) lst[0] = total;
  } else {
    uint32_t* msk = a.masks + static_cast<size_t>(blockIdx.x) * W;
    for (int w = tid; w < W; w += 256) msk[w] = mask_s[w];
    if (tid == 0) lst[0] = -1;
  }
}

// The fix-up's first launch ORs the pass-1 blocks' flags into the call's outlier mask
// (cleared by pass 1): thread t of block b reads the list published by pass-1 block
// 256 b + t (its count and first 32 columns in one go; the slot is always there to read
// and entries past the count are ignored; columns beyond 32 only when a list is longer),
// or that block's whole mask when it listed too many, and ORs it into the block's LDS
// copy of the mask; the block then ORs its nonzero words into the call's mask. A list
// equal to list 0 is skipped (the lists are ascending, so equal column sets are equal
// ints): most lists hold the same columns, whose atomics would all pile onto the same
// few words. Dynamic LDS: ceil(K / 32) words.
__global__ __launch_bounds__(256) void k_quant_or(FusedQuantArgs a) {
  extern __shared__ uint32_t m_s[];
  const int W = (a.K + 31) >> 5;
  const int tid = threadIdx.x, pb = blockIdx.x * 256 + tid;
  const int b = min(pb, a.nblk - 1);
  const v4i* slot = reinterpret_cast<const v4i*>(a.lists + static_cast<size_t>(b) * kListSlot);
  const v4i* ref = reinterpret_cast<const v4i*>(a.lists);
  const v4i head = slot[0], rhead = ref[0];
  v4i e[8], re[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    e[q] = slot[1 + q];
    re[q] = ref[1 + q];
  }
  __shared__ int novf_s;
  __shared__ int ovf_s[256];
  for (int w = tid; w < W; w += 256) m_s[w] = 0u;
  if (tid == 0) novf_s = 0;
  lds_barrier();
  auto set_bit = [&](int col) {
    const uint32_t bit = 1u << (col & 31);
    if (!(m_s[col >> 5] & bit)) atomicOr(&m_s[col >> 5], bit);
  };
  if (pb < a.nblk) {
    const int h = head[0];
    if (h < 0) ovf_s[atomicAdd(&novf_s, 1)] = pb;
    bool same = pb > 0 && h >= 0 && h <= 32 && h == rhead[0];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (4 * q + k < h && e[q][k] != re[q][k]) same = false;
    if (!same && h >= 0) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (4 * q + k < h) set_bit(e[q][k]);
      for (int r = 32; r < h; ++r) set_bit(a.lists[static_cast<size_t>(pb) * kListSlot + 4 + r]);
    }
  }
  lds_barrier();
  // whole masks of the blocks that listed too many, a word per thread
  const int nov = novf_s;
  for (int i = 0; i < nov; ++i) {
    const uint32_t* msk = a.masks + static_cast<size_t>(ovf_s[i]) * W;
    for (int w = tid; w < W; w += 256) m_s[w] |= msk[w];
  }
  lds_barrier();
  for (int w = tid; w < W; w += 256)
    if (const uint32_t m = m_s[w]) atomicOr(&a.gmask[w], m);
}

// Blocks [0, nfix): rows 16 b .. 16 b + 15 (wave w patches rows 16 b + 4 r + w; rows to
// requantize are collected and then done by the whole block, the row held in
// registers, CH chunks per thread). Blocks from nfix on: the WoT gather, 64 weight rows
// each (WoT rows n = 64 (b - nfix) + t % 64, ranks r = t / 64 + 4 j). Dynamic LDS: the
// outlier mask (ceil(K / 32) words), then o_lds ranked columns.
template <int CH>
__global__ __launch_bounds__(256) void k_quant_fix(FusedQuantArgs a, int o_lds, int nfix) {
  extern __shared__ uint32_t lds[];
  const int K = a.K, W = (K + 31) >> 5, ks = unit_ks(K);
  uint32_t* g_s = lds;
  int* idx_s = reinterpret_cast<int*>(lds + W);
  __shared__ int nredo_s;
  __shared__ int redo_s[16];
  __shared__ unsigned red_s[4];
  __shared__ int wave_tot[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool row_block = static_cast<int>(blockIdx.x) < nfix;
  // a_x and the candidate columns of the wave's rows go out with the column set's loads
  const int rbase = blockIdx.x * 16 + wave;
  float ax[4];
  v4i js[4];
  if (row_block) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = min(rbase + 4 * rr, a.M - 1);
      ax[rr] = a.a_x[row];
      js[rr] = *reinterpret_cast<const v4i*>(a.jstar + static_cast<size_t>(row) * 4);
    }
  }
  // the outlier set: rank the mask's columns (thread t owns words [t*per, (t+1)*per))
  for (int w = tid; w < W; w += 256) g_s[w] = a.gmask[w];
  if (tid == 0) nredo_s = 0;
  lds_barrier();
  const int per = (W + 255) / 256;
  const int w0 = min(W, tid * per), w1 = min(W, w0 + per);
  int mine = 0;
  for (int w = w0; w < w1; ++w) mine += __popc(g_s[w]);
  const int incl = wave_prefix_sum(mine);
  if (lane == 63) wave_tot[wave] = incl;
  lds_barrier();
  int before = incl - mine, count = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    before += i < wave ? wave_tot[i] : 0;
    count += wave_tot[i];
  }
  // rows: patch (zero the provisional codes at every outlier column) when some column
  // reaching the provisional constant is not an outlier, else requantize; decided as
  // soon as the mask and the count are known, the ranking below alongside
  const bool patch = count <= min(kFixZeroMax, o_lds);
  bool redo[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int row = rbase + 4 * rr;
    redo[rr] = row_block && row < a.M && !patch;
    if (row_block && row < a.M && patch && count > 0 && ax[rr] > 0.0f) {
      bool keep = false;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = js[rr][k];
        keep = keep || (c >= 0 && !((g_s[c >> 5] >> (c & 31)) & 1u));
      }
      redo[rr] = !keep;
    }
    if (redo[rr] && lane == 0) redo_s[atomicAdd(&nredo_s, 1)] = row;
  }
  for (int w = w0, r = before; w < w1; ++w) {
    uint32_t bits = g_s[w];
    while (bits) {
      const int bb = __ffs(bits) - 1;
      bits &= bits - 1;
      if (r < o_lds) idx_s[r] = w * 32 + bb;
      ++r;
    }
  }
  lds_barrier();
  const int nr = min(count, o_lds);
  if (blockIdx.x == 0) {
    if (tid == 0) {
      a.count_out[0] = count;
      if (a.status_out) a.status_out[0] = count > a.max_outliers ? 7 : 0;
    }
    if (a.idx_out)
      for (int r = tid; r < min(count, a.max_outliers); r += 256) a.idx_out[r] = idx_s[r];
  }
  const int o_pad = min((count + 15) & ~15, a.o_stride);
  const _Float16* __restrict__ X = a.X;

  if (row_block) {
    const int nredo = nredo_s;
    // the outlier values of the wave's rows (for up to 64 ranks, all four rows' loads
    // before any store: the pointers do not alias) and the zeroed codes
    _Float16* __restrict__ Xo = a.Xo;
    int8_t* __restrict__ Xq = a.Xq;
    auto patch_rows = [&]() {
      if (Xo && o_pad <= 64) {
        const int col = lane < nr ? idx_s[lane] : 0;
        _Float16 g[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int row = min(rbase + 4 * rr, a.M - 1);
          g[rr] = lane < count ? X[static_cast<size_t>(row) * K + col] : _Float16(0);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int row = rbase + 4 * rr;
          if (row < a.M && lane < o_pad) Xo[static_cast<size_t>(row) * a.o_stride + lane] = g[rr];
        }
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = rbase + 4 * rr;
        if (row >= a.M) break;
        if (!redo[rr])
          for (int r = lane; r < count; r += 64) Xq[unit_offset(row, idx_s[r], ks)] = 0;
        if (Xo && o_pad > 64) {
          const _Float16* xr = X + static_cast<size_t>(row) * K;
          _Float16* xo = Xo + static_cast<size_t>(row) * a.o_stride;
          for (int r = lane; r < o_pad; r += 64) xo[r] = r < count ? xr[idx_s[r]] : _Float16(0);
        }
      }
    };
    if (nredo == 0) {
      patch_rows();
    } else {
      // the first row to requantize is loaded before the patching, under it (inside this
      // branch: registers loaded under a condition and used after the join would make
      // the compiler wait for them at the join)
      v8h v[CH];
      load_row<CH, 256>(X + static_cast<size_t>(redo_s[0]) * K, K, tid, v);
      patch_rows();
      for (int i = 0; i < nredo; ++i) {
        const int row = redo_s[i];
        const _Float16* xr = X + static_cast<size_t>(row) * K;
        if (i > 0) load_row<CH, 256>(xr, K, tid, v);
        quant_row_block<CH>(xr, K, g_s, Xq, row, ks, a.a_x + row, tid, v, red_s);
        lds_barrier();  // red_s is reused by the next row
      }
    }
  } else {
    // WoT[n, r] = fp16(Wq[n, O_r] * a_w[n] / 127), as in k_quant_rows: thread t takes
    // row n = 64 (b - nfix) + t % 64 and ranks t / 64 + 4 j, all its loads at once
    const int n = (blockIdx.x - nfix) * 64 + lane;
    if (n >= a.N) return;
    const float aw = a.a_w[n];
    const int8_t* __restrict__ Wq = a.Wq;
    _Float16* __restrict__ dst = a.WoT + static_cast<size_t>(n) * a.o_stride;
    for (int r0 = wave; r0 < o_pad; r0 += 64) {
      int8_t q[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = r0 + 4 * j;
        q[j] = r < count ? Wq[unit_offset(n, idx_s[min(r, o_lds - 1)], ks)] : int8_t(0);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = r0 + 4 * j;
        if (r < o_pad)
          dst[r] = static_cast<_Float16>(__fdiv_rn(static_cast<float>(q[j]) * aw, 127.0f));
      }
    }
  }
}

template <int CH>
static void launch_pass_ch(const FusedQuantArgs& a, size_t lds, bool nt, hipStream_t s) {
  if (nt) hipLaunchKernelGGL((k_quant_pass<CH, true>), dim3(a.nblk), dim3(256), lds, s, a);
  else hipLaunchKernelGGL((k_quant_pass<CH, false>), dim3(a.nblk), dim3(256), lds, s, a);
}

hipError_t launch_quant_pass(const FusedQuantArgs& a, hipStream_t s) {
  const int per = (a.K / 8 + 255) / 256;
  const size_t lds = static_cast<size_t>((a.K + 31) / 32) * 4;
  // X read non-temporally when it is large: at 100-170 MB the pass ran 7-9% faster so
  // (175B share 41.4 -> 37.5 us, 13B down 58.3 -> 54.0 us); at 16 MB (6.7B up) 5% slower
  const bool nt = static_cast<int64_t>(a.M) * a.K * 2 >= (int64_t(64) << 20);
#define I8MM_QP(CHV) launch_pass_ch<CHV>(a, lds, nt, s)
  if (per <= 1) I8MM_QP(1);
  else if (per <= 2) I8MM_QP(2);
  else if (per <= 4) I8MM_QP(4);
  else if (per <= 6) I8MM_QP(6);
  else if (per <= 8) I8MM_QP(8);
  else if (per <= 10) I8MM_QP(10);
  else if (per <= 12) I8MM_QP(12);
  else I8MM_QP(16);
#undef I8MM_QP
  return hipGetLastError();
}

hipError_t launch_quant_fixup(const FusedQuantArgs& a, hipStream_t s) {
  const int W = (a.K + 31) / 32;
  const int o_lds = a.o_stride > a.max_outliers ? a.o_stride : a.max_outliers;
  const size_t lds = static_cast<size_t>(W + o_lds) * 4;
  hipLaunchKernelGGL(k_quant_or, dim3((a.nblk + 255) / 256), dim3(256), static_cast<size_t>(W) * 4,
                     s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nfix = (a.M + 15) / 16;
  const int ngather = a.WoT ? (a.N + 63) / 64 : 0;
  const int per = (a.K / 8 + 255) / 256;
  const dim3 grid(nfix + ngather), block(256);
#define I8MM_QF(CHV) hipLaunchKernelGGL((k_quant_fix<CHV>), grid, block, lds, s, a, o_lds, nfix)
  if (per <= 1) I8MM_QF(1);
  else if (per <= 2) I8MM_QF(2);
  else if (per <= 4) I8MM_QF(4);
  else if (per <= 8) I8MM_QF(8);
  else if (per <= 12) I8MM_QF(12);
  else I8MM_QF(16);
#undef I8MM_QF
  return hipGetLastError();
}

}  // namespace i8mm
