// The int8 GEMM with the outlier fp16 product and the dequantizing epilogue.
//
// acc[m, n] = sum_k Xq[m, k] Wq[n, k]  (exact int32; "Compress your LLMs",
//   Mixed-precision decomposition: 8-bit matrix multiplication for the non-outlier
//   dimensions),
// Y[m, n]   = fp16( acc * a_x[m] * a_w[n] / 127^2              (outer-product dequant,
//                   "8-bit Matrix Multiplication for Large Language Models", Summary &
//                   Methodology Analysis)
//                 + sum_r Xo[m, r] WoT[n, r] )                  (16-bit product over the
//                   outlier columns, summed into the same fp16 output)
//
// gfx950 design. Both operands are K-contiguous, so the block computes D = Wq_tile *
// Xq_tile^T with v_mfma_i32_32x32x32_i8: lane l feeds row l%32 with 16 consecutive K
// bytes of each operand, and the A/B roles are chosen so that every lane ends up
// holding 4 consecutive output columns n of one row m (8-byte fp16 stores).
// A 256-thread block (4 waves, one per SIMD) owns a TN x TM tile; each wave a
// (TN/2) x (TM/2) sub-tile of 32x32 blocks whose int32 accumulators live in registers.
// K is walked in BK-byte slabs: global -> registers (buffer loads; rows past the edge
// and K past the end read as zeros) -> LDS (double buffered, XOR-swizzled 16-byte
// chunks so that ds_read_b128 fragment reads are free of bank conflicts) -> MFMA.
// The next slab's global loads are in flight while the current slab is multiplied.
// The outlier product runs after the K loop on v_mfma_f32_32x32x16_f16, reading the
// small Xo / WoT fragments straight from global memory (L2-resident), and is added in
// fp32 before the single rounding to fp16.
#include "common.hpp"
#include "launch.hpp"

namespace i8mm {

template <int TN_, int TM_, int BK_, int WGN_, int WGM_>
struct GemmCfg {
  static constexpr int TN = TN_, TM = TM_, BK = BK_, WGN = WGN_, WGM = WGM_;
  static constexpr int NT = WGN * WGM * 64;
  static constexpr int WTN = TN / WGN, WTM = TM / WGM;
  static constexpr int BN = WTN / 32, BM = WTM / 32;
  static constexpr int CPR = BK / 16;  // 16-byte chunks per LDS row
  static constexpr int AC = TN * CPR / NT, BC = TM * CPR / NT;
  static constexpr int A_BYTES = TN * BK, B_BYTES = TM * BK;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static_assert(AC * NT == TN * CPR && BC * NT == TM * CPR, "tile / thread mismatch");
  static_assert(BK % 32 == 0 && WTN % 32 == 0 && WTM % 32 == 0, "shape");
};

// XOR swizzle of the 16-byte chunk index within an LDS row. For the fragment reads
// (lanes 0..31 read rows r0..r0+31 at one chunk, lanes 32..63 the next chunk) every
// group of 8 lanes hits 8 distinct 16-byte slots of a 128-byte window and every group
// of 16 lanes 16 distinct slots of a 256-byte window; the same holds for the
// row-major ds_write_b128 stores.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 4) return ((r >> 1) ^ (r >> 2)) & 3;
  else return (r ^ (r >> 1)) & 7;
}
template <int BK>
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * BK + 16 * (c ^ swz<BK / 16>(r));
}

// Block -> output tile. The hardware hands workgroup b to XCD b % 8; renumber so that
// each XCD owns a contiguous run of tiles, then walk the run in groups of group_m
// m-tiles per n-tile so that concurrently running tiles on one XCD share operand
// slabs in that XCD's L2.
__device__ __forceinline__ void tile_of(int bid, int nblocks, int tiles_m, int group_m, int& tn,
                                        int& tm) {
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nblocks >> 3, extra = nblocks & 7;
  const int pid = xcd < extra ? xcd * (per + 1) + local : extra * (per + 1) + (xcd - extra) * per + local;
  const int tiles_n = nblocks / tiles_m;
  const int per_group = group_m * tiles_n;
  const int grp = pid / per_group;
  const int first_m = grp * group_m;
  const int gsz = min(tiles_m - first_m, group_m);
  const int in = pid - grp * per_group;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

template <class C>
__global__ __launch_bounds__(C::NT) void k_gemm(GemmArgs g, int tiles_m, int group_m) {
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % C::WGN, wm = wave / C::WGN;
  int tn, tm;
  tile_of(blockIdx.x, gridDim.x, tiles_m, group_m, tn, tm);
  const int n0 = tn * C::TN, m0 = tm * C::TM;
  const int K = g.K;

  const unsigned rows_a = min(C::TN, g.N - n0), rows_b = min(C::TM, g.M - m0);
  const auto ra = make_rsrc(g.Wq + static_cast<size_t>(n0) * K, rows_a * K);
  const auto rb = make_rsrc(g.Xq + static_cast<size_t>(m0) * K, rows_b * K);

  // Chunk i of this thread's share of a stage is row r0 + i * (NT / CPR), chunk c: the
  // XOR swizzle only sees the row's low bits, which NT / CPR (a multiple of 8) keeps.
  constexpr int RSTEP = C::NT / C::CPR;
  static_assert(RSTEP % 8 == 0, "row step must preserve the swizzle");
  const int r0 = tid / C::CPR, c0 = tid % C::CPR;
  const unsigned g_base = r0 * K + c0 * 16, g_step = RSTEP * K;
  const int l_base = lds_off<C::BK>(r0, c0);
  const int kc = c0 * 16;

  v4u va[C::AC], vb[C::BC];
  auto gload = [&](int kt) {
    const int k0 = kt * C::BK;
    const unsigned off = k0 + kc < K ? g_base + k0 : kOOB;
    const unsigned stp = k0 + kc < K ? g_step : 0u;
#pragma unroll
    for (int i = 0; i < C::AC; ++i) va[i] = buf_load16(ra, off + i * stp);
#pragma unroll
    for (int i = 0; i < C::BC; ++i) vb[i] = buf_load16(rb, off + i * stp);
  };
  auto lstore = [&](int buf) {
    char* s = smem + buf * C::STAGE + l_base;
#pragma unroll
    for (int i = 0; i < C::AC; ++i) *reinterpret_cast<v4u*>(s + i * RSTEP * C::BK) = va[i];
#pragma unroll
    for (int i = 0; i < C::BC; ++i)
      *reinterpret_cast<v4u*>(s + C::A_BYTES + i * RSTEP * C::BK) = vb[i];
  };

  v16i acc[C::BN][C::BM];
#pragma unroll
  for (int i = 0; i < C::BN; ++i)
#pragma unroll
    for (int j = 0; j < C::BM; ++j) acc[i][j] = v16i{};

  const int l32 = lane & 31, lhi = lane >> 5;
  auto compute = [&](int buf) {
    const char* As = smem + buf * C::STAGE;
    const char* Bs = As + C::A_BYTES;
#pragma unroll
    for (int s = 0; s < C::BK / 32; ++s) {
      const int c = 2 * s + lhi;
      v4i af[C::BN], bf[C::BM];
#pragma unroll
      for (int i = 0; i < C::BN; ++i)
        af[i] = *reinterpret_cast<const v4i*>(As + lds_off<C::BK>(wn * C::WTN + i * 32 + l32, c));
#pragma unroll
      for (int j = 0; j < C::BM; ++j)
        bf[j] = *reinterpret_cast<const v4i*>(Bs + lds_off<C::BK>(wm * C::WTM + j * 32 + l32, c));
#pragma unroll
      for (int i = 0; i < C::BN; ++i)
#pragma unroll
        for (int j = 0; j < C::BM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  const int nk = (K + C::BK - 1) / C::BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk - 1; ++kt) {
    gload(kt + 1);  // in flight while slab kt is multiplied
    compute(kt & 1);
    lstore((kt + 1) & 1);
    __syncthreads();
  }
  compute((nk - 1) & 1);

  // Epilogue. 32x32 accumulator layout: lane l, register r holds column m = l % 32
  // and row n = 8 (r / 4) + 4 (l / 32) + r % 4 of the block (rows are n here).
  // Per block: store the int32 sums if asked, dequantize in place to fp32, let the
  // fp16 outlier MFMA accumulate on top of that, round once to fp16.
  const int count = *g.count;
  const bool overflow = count > g.max_outliers;
  const int o_pad = min((count + 15) & ~15, g.o_stride);
  const int M = g.M, N = g.N;
#pragma unroll
  for (int i = 0; i < C::BN; ++i) {
    const int nb = n0 + wn * C::WTN + i * 32;
    const _Float16* wo_row = g.WoT + static_cast<size_t>(min(nb + l32, N - 1)) * g.o_stride;
#pragma unroll
    for (int j = 0; j < C::BM; ++j) {
      const int m = m0 + wm * C::WTM + j * 32 + l32;
      const int mc = min(m, M - 1);
      const float sx = g.a_x[mc] * kInvQMax2;
      v16f y;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nb + 8 * q + 4 * lhi;
        const v4f aw = n < N ? *reinterpret_cast<const v4f*>(g.a_w + n) : v4f{};
        if (g.acc_out && m < M && n < N) {
          const v4i av = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                          acc[i][j][4 * q + 3]};
          *reinterpret_cast<v4i*>(g.acc_out + static_cast<size_t>(m) * N + n) = av;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          y[4 * q + e] = static_cast<float>(acc[i][j][4 * q + e]) * sx * aw[e];
      }
      const _Float16* xo_row = g.Xo + static_cast<size_t>(mc) * g.o_stride;
      for (int s = 0; s < o_pad; s += 16) {
        const v8h fa = *reinterpret_cast<const v8h*>(wo_row + s + 8 * lhi);
        const v8h fb = *reinterpret_cast<const v8h*>(xo_row + s + 8 * lhi);
        y = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, fb, y, 0, 0, 0);
      }
      if (m < M) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nb + 8 * q + 4 * lhi;
          if (n < N) {
            v4h out;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              out[e] = overflow ? static_cast<_Float16>(__builtin_nanf(""))
                                : static_cast<_Float16>(y[4 * q + e]);
            *reinterpret_cast<v4h*>(g.Y + static_cast<size_t>(m) * N + n) = out;
          }
        }
      }
    }
  }
}

using CfgL = GemmCfg<256, 256, 64, 2, 2>;  // large problems
using CfgS = GemmCfg<128, 128, 64, 2, 2>;  // small or skinny problems

template <class C>
static hipError_t run(const GemmArgs& g, hipStream_t s) {
  const int tiles_n = (g.N + C::TN - 1) / C::TN, tiles_m = (g.M + C::TM - 1) / C::TM;
  const int group_m = tiles_m < 8 ? tiles_m : 8;
  hipLaunchKernelGGL(k_gemm<C>, dim3(tiles_n * tiles_m), dim3(C::NT), 0, s, g, tiles_m, group_m);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  const long tiles_l = static_cast<long>((g.N + 255) / 256) * ((g.M + 255) / 256);
  if (g.M >= 256 && tiles_l >= 256) return run<CfgL>(g, s);
  return run<CfgS>(g, s);
}

}  // namespace i8mm
