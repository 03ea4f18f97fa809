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
                                                      uint32_t* __restrict__ partial, int W) {
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
    if (w < W) partial[static_cast<size_t>(blockIdx.y) * W + w] = word;
  }
}

// One wave quantizes one row. CH > 0: the row is held in registers (CH chunks of 8
// halves per lane, K <= 512 * CH) and read once; CH == 0: streamed twice.
// Xq goes row-major (ks == 0) or unit-tiled with ks = unit_ks(K) units per row group,
// in which case the row's K padding is written as zero codes.
// Outlier columns are cleared in the registers (drop_halves), the row constant is a
// packed u16 magnitude max reduced over the wave with DPP, and the codes come from the
// bracketing pair of fused multiply-adds (quant8_fast); groups where the pair
// disagrees take quant8_exact.
// Loads a row into registers for quant_one_row<CH> (CH > 0): chunk c = lane + 64 i;
// unconditional loads at clamped addresses, zeros past the row.
// (STRIDE threads share the row: chunk c = t + STRIDE i.)
template <int CH, int STRIDE = 64>
__device__ __forceinline__ void load_row(const _Float16* __restrict__ xr, int K, int t,
                                         v8h (&v)[CH > 0 ? CH : 1]) {
  const int nchunk = K >> 3;
#pragma unroll
  for (int i = 0; i < (CH > 0 ? CH : 1); ++i) {
    const int c = t + STRIDE * i;
    const v8h t = *reinterpret_cast<const v8h*>(xr + min(c, nchunk - 1) * 8);
    v[i] = c < nchunk ? t : v8h{};
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
                     partial, W);
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

}  // namespace i8mm
