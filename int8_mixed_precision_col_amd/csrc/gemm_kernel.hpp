// The int8 GEMM with the outlier fp16 product and the dequantizing epilogue.
//
// acc[m, n] = sum_k Xq[m, k] Wq[n, k]  (exact int32; "Compress your LLMs",
//   Mixed-precision decomposition: 8-bit matrix multiplication for the non-outlier
//   dimensions),
// Y[m, n]   = fp16( acc * a_x[m] * a_w[n] / 127^2              (outer-product dequant,
//                   "8-bit Matrix Multiplication for Large Language Models", Summary &
//                   Methodology Analysis)
//                 + sum_r Xo[m, r] W^[O_r, n] )                 (16-bit product over the
//                   outlier columns O_r, summed into the same fp16 output; W^ is the
//                   int8 weight dequantized, fp16(Wq a_w / 127))
//
// gfx950 design. Both operands are K-contiguous, so a block computes D = Wq_tile *
// Xq_tile^T with v_mfma_i32_16x16x64_i8: lane l feeds row l%16 with 16 consecutive K
// bytes (chunk l/16 of a 64-byte slab row) of each operand, and the A/B roles are
// chosen so that every lane ends up holding 4 consecutive output columns n of one row
// m (8-byte fp16 stores). Under the board's power limit the 16x16x64 form sustains
// more int8 operations per second than 32x32x32 on the same operands: it moves half
// the accumulator bits per operation.
// A block of WGN x WGM waves owns a TN x TM tile; each wave a (TN/WGN) x (TM/WGM)
// sub-tile of 16x16 blocks whose int32 accumulators live in registers.
// K is walked in BK-byte slabs through a ring of STAGES LDS buffers filled by
// global_load_lds_dwordx4 (global memory straight into LDS, no VGPR staging) from
// unit-tiled operands (16 rows x 64 K-bytes per contiguous 1 KB unit), so that each
// DMA instruction reads whole cache lines: rows past the tile edge are clamped to the
// last row (their outputs are discarded), the K padding holds zeros and slabs past it
// read a 16-byte zero constant, and each lane fetches the global 16-byte chunk that
// belongs at its LDS slot under an XOR swizzle, so that the ds_read_b128 fragment
// reads are free of bank conflicts. Slab kt + STAGES - 1 is in
// flight while slab kt is multiplied; one barrier per slab.
// The outlier product runs after the K loop on v_mfma_f32_16x16x16_f16, with the
// small Xo / W^ fragments staged through LDS (W^ gathered beforehand, or dequantized
// from the Wq bytes of the outlier columns as they are staged), accumulating on top of
// the already
// dequantized fp32 values before the single rounding to fp16.
#pragma once

#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace i8mm {

// CPOL: cache-policy bits of the DMA loads (gfx950: 1 = sc0, 2 = nt, 16 = sc1).
template <int TN_, int TM_, int BK_, int WGN_, int WGM_, int STAGES_, int CPOL_ = 0>
struct GemmCfg {
  static constexpr int TN = TN_, TM = TM_, BK = BK_, WGN = WGN_, WGM = WGM_, STAGES = STAGES_;
  static constexpr int CPOL = CPOL_;
  static constexpr int NW = WGN * WGM, NT = NW * 64;
  static constexpr int WTN = TN / WGN, WTM = TM / WGM;
  static constexpr int BN = WTN / 16, BM = WTM / 16;
  static constexpr int CPR = BK / 16;                  // 16-byte chunks per LDS row
  static constexpr int A_BYTES = TN * BK, B_BYTES = TM * BK;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int AI = A_BYTES / (1024 * NW);    // 1 KB DMA instructions per wave, A
  static constexpr int BI = B_BYTES / (1024 * NW);    // ... and B
  static_assert(AI * 1024 * NW == A_BYTES && BI * 1024 * NW == B_BYTES, "tile / wave mismatch");
  static_assert(BK == 64 && WTN % 32 == 0 && WTM % 32 == 0, "shape");
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");
};

// XOR swizzle of the 16-byte chunk index within an LDS row. For the fragment reads
// (lanes 16c .. 16c + 15 read rows r0 .. r0 + 15, r0 a multiple of 16, at chunk c) every
// group of 8 lanes hits 8 distinct 16-byte slots of a 128-byte window and every group
// of 16 lanes 16 distinct slots of a 256-byte window.
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
  const int pid =
      xcd < extra ? xcd * (per + 1) + local : extra * (per + 1) + (xcd - extra) * per + local;
  const int tiles_n = nblocks / tiles_m;
  const int per_group = group_m * tiles_n;
  const int grp = pid / per_group;
  const int first_m = grp * group_m;
  const int gsz = min(tiles_m - first_m, group_m);
  const int in = pid - grp * per_group;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

#define I8MM_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// One 16-byte-per-lane DMA from global memory into LDS (base + 16 * lane). The cache
// policy must reach the builtin as a literal.
template <int CPOL>
__device__ __forceinline__ void dma16(const void* src, __attribute__((address_space(3))) void* dst) {
  if constexpr (CPOL == 1) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 1);
  else if constexpr (CPOL == 2) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 2);
  else if constexpr (CPOL == 3) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 3);
  else __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// Source of the K-tail chunks: multiplying by zeros adds nothing to the int32 sums.
__device__ __attribute__((aligned(16))) const int kZero16[4] = {0, 0, 0, 0};

// Waits until at most `pending` of this thread's buffer loads are outstanding and all
// its LDS reads are done, then joins the block barrier. The empty asm statements keep
// the compiler from moving memory accesses across the barrier.
// Waits for this thread's outstanding LDS reads only (vmcnt and expcnt left open).
__device__ __forceinline__ void lds_reads_done() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}

template <int PENDING>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(PENDING >= 0 && PENDING < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14]
  __builtin_amdgcn_s_waitcnt((PENDING & 0xF) | (0x7 << 4) | (0x0 << 8) | ((PENDING >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The LDS ring: one __shared__ object per stage, so that the compiler can tell which
// stage a DMA writes and a fragment read reads (a single array indexed by stage makes
// it wait for every outstanding DMA before each read).
template <class C, int S>
__device__ __forceinline__ char* stage_buf() {
  __shared__ __attribute__((aligned(1024))) char buf[C::STAGE];
  return buf;
}

// The LDS slice of wave w for staging its fp16 output sub-tile (WTM rows of WTN halves):
// slices are packed into the ring's stages, as many per stage as fit.
template <class C>
__device__ __forceinline__ char* wave_slice(int w) {
  constexpr int PW = C::WTM * C::WTN * 2, PER = C::STAGE / PW;
  static_assert(PER >= 1 && C::NW <= PER * C::STAGES, "the ring holds every wave's output");
  const int st = w / PER, off = (w % PER) * PW;
  if constexpr (C::STAGES > 3)
    if (st == 3) return stage_buf<C, 3>() + off;
  if constexpr (C::STAGES > 2)
    if (st == 2) return stage_buf<C, 2>() + off;
  return (st == 1 ? stage_buf<C, 1>() : stage_buf<C, 0>()) + off;
}
// Chunk swizzle of a staged output row: spreads the 16 rows written by one fragment store
// (half of a 16-byte chunk each, two lanes per chunk) over 16 distinct bank groups.
template <int CH>
__device__ __forceinline__ int ysw(int r) {
  static_assert(CH == 16 || CH == 8, "staged row width");
  if constexpr (CH == 16) return r & 15;
  else return (r >> 1) & 7;
}

// Epilogue. 16x16 accumulator layout: lane l, register r holds column m = l % 16 and
// row n = 4 (l / 16) + r of the block (rows are n here). The tile's
// a_w / a_x and the outlier fragments (16 columns of W^ and Xo per pass) are staged
// in stage 0 of the ring first (free once the K loop is done), so that no global
// load waits inside the per-block loops; reading them straight from global memory,
// one block at a time, took ~13 us per tile against ~8 us now. Per block:
// store the int32 sums if asked, dequantize in place to fp32, let the fp16 outlier
// MFMA accumulate on top of that, round once to fp16.
template <class C, bool GATHER>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, v4i (&acc)[C::BN][C::BM],
                                                     int n0, int m0, int wn, int wm, int lane,
                                                     int tid) {
  constexpr int OS = 24;  // staged row stride in halves (16 columns + 8 of padding)
  static_assert((C::TN + C::TM) * 4 + (C::TN + C::TM) * OS * 2 <= C::STAGE, "staging fits a stage");
  char* base = stage_buf<C, 0>();
  float* aw_s = reinterpret_cast<float*>(base);
  float* ax_s = aw_s + C::TN;
  _Float16* wo_s = reinterpret_cast<_Float16*>(ax_s + C::TM);
  _Float16* xo_s = wo_s + C::TN * OS;
  const int l16 = lane & 15, lq = lane >> 4;
  const int count = *g.count;
  const bool overflow = count > g.max_outliers;
  const int o_pad = min((count + 15) & ~15, g.o_stride);
  const int nvalid = min(count, g.max_outliers);
  const int M = g.M, N = g.N, ks = unit_ks(g.K);
  const size_t ldy = g.ldy > 0 ? g.ldy : N;
  auto stage_outliers = [&](int s0) {
    for (int t = tid; t < (C::TN + C::TM) * 2; t += C::NT) {
      const int row = t >> 1, h = t & 1;
      if (row < C::TN) {
        if constexpr (GATHER)
          *reinterpret_cast<v8h*>(wo_s + row * OS + 8 * h) =
              outlier_weights(g, min(n0 + row, N - 1), s0 + 8 * h, nvalid, ks);
        else
          *reinterpret_cast<v8h*>(wo_s + row * OS + 8 * h) = *reinterpret_cast<const v8h*>(
              g.WoT + static_cast<size_t>(min(n0 + row, N - 1)) * g.o_stride + s0 + 8 * h);
      } else
        *reinterpret_cast<v8h*>(xo_s + (row - C::TN) * OS + 8 * h) = *reinterpret_cast<const v8h*>(
            g.Xo + static_cast<size_t>(min(m0 + row - C::TN, M - 1)) * g.o_stride + s0 + 8 * h);
    }
  };
  lds_reads_done();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();  // every wave is done reading the ring
  asm volatile("" ::: "memory");
  for (int t = tid; t < C::TN + C::TM; t += C::NT) {
    if (t < C::TN) aw_s[t] = g.a_w[min(n0 + t, N - 1)];
    else ax_s[t - C::TN] = g.a_x[min(m0 + t - C::TN, M - 1)];
  }
  if (o_pad > 0) stage_outliers(0);
  lds_barrier();
#pragma unroll
  for (int i = 0; i < C::BN; ++i) {
    const int nl = wn * C::WTN + i * 16;
    const int nq = nl + 4 * lq;
    const v4f aw = *reinterpret_cast<const v4f*>(aw_s + nq);
#pragma unroll
    for (int j = 0; j < C::BM; ++j) {
      const int ml = wm * C::WTM + j * 16;
      const int m = m0 + ml + l16;
      const float sx = ax_s[ml + l16] * kInvQMax2;
      if (g.acc_out && m < M && n0 + nq < N)
        *reinterpret_cast<v4i*>(g.acc_out + m * ldy + n0 + nq) = acc[i][j];
      v4f y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = static_cast<float>(acc[i][j][e]) * sx * aw[e];
      acc[i][j] = __builtin_bit_cast(v4i, y);
    }
  }
  for (int s0 = 0; s0 < o_pad; s0 += 16) {
    if (s0 > 0) {
      lds_barrier();
      stage_outliers(s0);
      lds_barrier();
    }
#pragma unroll
    for (int i = 0; i < C::BN; ++i) {
      const int nl = wn * C::WTN + i * 16;
#pragma unroll
      for (int j = 0; j < C::BM; ++j) {
        const int ml = wm * C::WTM + j * 16;
        const v4h fa = *reinterpret_cast<const v4h*>(wo_s + (nl + l16) * OS + 4 * lq);
        const v4h fb = *reinterpret_cast<const v4h*>(xo_s + (ml + l16) * OS + 4 * lq);
        acc[i][j] = __builtin_bit_cast(v4i, __builtin_amdgcn_mfma_f32_16x16x16f16(
                                                fa, fb, __builtin_bit_cast(v4f, acc[i][j]), 0, 0, 0));
      }
    }
  }
  // Y: each wave rounds its sub-tile to fp16 into a private slice of the ring (free now:
  // the barrier below also retires the staged scales and outlier fragments), then stores
  // whole row segments, 16 bytes per lane and 64 / CH rows per instruction. Straight from
  // the accumulator layout every store would cover 32 rows x 16 bytes, four times the
  // memory requests for the same bytes.
  lds_barrier();
  char* ys = wave_slice<C>(wn + C::WGN * wm);
  constexpr int CH = C::WTN / 8;   // 16-byte chunks per staged row
  constexpr int RB = C::WTN * 2;   // staged row bytes
#pragma unroll
  for (int i = 0; i < C::BN; ++i) {
#pragma unroll
    for (int j = 0; j < C::BM; ++j) {
      const int r = j * 16 + l16;
      const v4f y = __builtin_bit_cast(v4f, acc[i][j]);
      v4h out;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        out[e] = overflow ? static_cast<_Float16>(__builtin_nanf("")) : static_cast<_Float16>(y[e]);
      *reinterpret_cast<v4h*>(ys + r * RB + 16 * ((2 * i + (lane >> 5)) ^ ysw<CH>(r)) +
                              8 * (lq & 1)) = out;
    }
  }
  constexpr int RPI = 64 / CH;     // rows per store instruction
  const int c = lane % CH;
  const int n = n0 + wn * C::WTN + 8 * c;
#pragma unroll
  for (int t = 0; t < C::WTM / RPI; ++t) {
    const int r = t * RPI + lane / CH;
    const v4u v = *reinterpret_cast<const v4u*>(ys + r * RB + 16 * (c ^ ysw<CH>(r)));
    const int m = m0 + wm * C::WTM + r;
    if (m < M && n < N) *reinterpret_cast<v4u*>(g.Y + m * ldy + n) = v;
  }
}

template <class C>
struct GemmBlock {
  const GemmArgs& g;
  const int8_t* a_src[C::AI];   // per-instruction global chunk addresses of slab 0
  const int8_t* b_src[C::BI];
  int a_k[C::AI], b_k[C::BI];   // K offset of this lane's chunk within a slab
  int wave, lane, wn, wm;
  int rn0, rm0;   // first fragment row of this lane in the A / B tile
  v4i acc[C::BN][C::BM];

  // Issue the DMA of slab kt into stage S (one 1 KB LDS block per instruction).
  // Slab kt starts kt * BK / 64 units further along each row group.
  template <int S>
  __device__ __forceinline__ void issue(int kt) {
    const int k0 = kt * C::BK;
    const size_t step = static_cast<size_t>(kt) * (C::BK / kUnitK) * kUnitBytes;
    const int kpad = unit_ks(g.K) * kUnitK;
    char* base = stage_buf<C, S>();
    const int8_t* zero = reinterpret_cast<const int8_t*>(kZero16);
#pragma unroll
    for (int i = 0; i < C::AI; ++i)
      dma16<C::CPOL>(k0 + a_k[i] < kpad ? a_src[i] + step : zero,
                     I8MM_LDS(base + (i * C::NW + wave) * 1024));
#pragma unroll
    for (int i = 0; i < C::BI; ++i)
      dma16<C::CPOL>(k0 + b_k[i] < kpad ? b_src[i] + step : zero,
                     I8MM_LDS(base + C::A_BYTES + (i * C::NW + wave) * 1024));
  }

  // One DMA instruction (q < AI: A chunk q, else B chunk q - AI) of slab kt into stage S.
  template <int S>
  __device__ __forceinline__ void issue_one(int kt, int q) {
    const int k0 = kt * C::BK;
    const size_t step = static_cast<size_t>(kt) * (C::BK / kUnitK) * kUnitBytes;
    const int kpad = unit_ks(g.K) * kUnitK;
    char* base = stage_buf<C, S>();
    const int8_t* zero = reinterpret_cast<const int8_t*>(kZero16);
    if (q < C::AI) {
      dma16<C::CPOL>(k0 + a_k[q] < kpad ? a_src[q] + step : zero,
                     I8MM_LDS(base + (q * C::NW + wave) * 1024));
    } else {
      const int i = q - C::AI;
      dma16<C::CPOL>(k0 + b_k[i] < kpad ? b_src[i] + step : zero,
                     I8MM_LDS(base + C::A_BYTES + (i * C::NW + wave) * 1024));
    }
  }

  struct Frags {
    v4i a[C::BN], b[C::BM];
  };

  // Fragments of the slab held in stage S: chunk l / 16 of rows l % 16 of each block.
  template <int S>
  __device__ __forceinline__ void load_frags(Frags& f) const {
    const char* As = stage_buf<C, S>();
    const char* Bs = As + C::A_BYTES;
    const int c = lane >> 4;
#pragma unroll
    for (int i = 0; i < C::BN; ++i)
      f.a[i] = *reinterpret_cast<const v4i*>(As + lds_off<C::BK>(rn0 + i * 16, c));
#pragma unroll
    for (int j = 0; j < C::BM; ++j)
      f.b[j] = *reinterpret_cast<const v4i*>(Bs + lds_off<C::BK>(rm0 + j * 16, c));
  }

  // The MFMAs of one substep with the DMA of slab kt into stage S spread between them:
  // issued as a burst right after the barrier, the DMA instructions of all waves stall
  // their issue queues together and the matrix cores idle meanwhile.
  template <int S>
  __device__ __forceinline__ void mma_dma(const Frags& f, int kt) {
    constexpr int NQ = C::AI + C::BI, NMM = C::BN * C::BM;
    constexpr int EVERY = NMM / NQ > 0 ? NMM / NQ : 1;
#pragma unroll
    for (int i = 0; i < C::BN; ++i)
#pragma unroll
      for (int j = 0; j < C::BM; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
        if ((i * C::BM + j) % EVERY == EVERY - 1 && (i * C::BM + j) / EVERY < NQ) {
          __builtin_amdgcn_sched_barrier(0);
          issue_one<S>(kt, (i * C::BM + j) / EVERY);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
    for (int q = NMM / EVERY; q < NQ; ++q) issue_one<S>(kt, q);
  }

  // One K slab held in stage CUR, whose fragments are already in f: wait until slab
  // kt + 1 has landed (this thread's DMA, then the barrier for everyone else's; the
  // slabs up to kt + STAGES - 1 may still be in flight), read slab kt + 1's fragments,
  // and run the MFMAs of slab kt with the refill of stage CUR - free now that every
  // wave has read all of slab kt - by slab kt + STAGES spread between them.
  // sched_barrier(0) keeps the compiler from sinking the fragment reads down to their
  // MFMAs, which would expose the LDS latency once per slab.
  template <int CUR>
  __device__ __forceinline__ void step(int kt, Frags& f) {
    constexpr int S = C::STAGES;
    Frags nxt;
    wait_and_barrier<(S - 2) * (C::AI + C::BI)>();
    load_frags<(CUR + 1) % S>(nxt);
    __builtin_amdgcn_sched_barrier(0);
    mma_dma<CUR>(f, kt + S);
    __builtin_amdgcn_sched_barrier(0);
    f = nxt;
  }
};

// One output tile (tn, tm) of the product described by g: the whole K loop and the
// epilogue. GATHER: the outlier columns' weights are dequantized from Wq in the
// epilogue (g.WoT unused); otherwise they are read from the gathered rows g.WoT.
template <class C, bool GATHER>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, int tn, int tm) {
  GemmBlock<C> b{g};
  const int tid = threadIdx.x;
  b.lane = tid & 63;
  b.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  b.wn = b.wave % C::WGN;
  b.wm = b.wave / C::WGN;
  {
    // The wave's row offsets enter the fragment addresses as per-lane values: folded
    // in as a scalar they hide which LDS stage a read touches, and the compiler then
    // waits for every outstanding DMA before each fragment read.
    const int vw = tid >> 6;
    b.rn0 = (vw % C::WGN) * C::WTN + (b.lane & 15);
    b.rm0 = (vw / C::WGN) * C::WTM + (b.lane & 15);
  }
  const int n0 = tn * C::TN, m0 = tm * C::TM;
  const int K = g.K;
  // LDS slot p = 64 (i NW + wave) + lane of a tile holds row p / CPR, chunk
  // (p % CPR) ^ swz(row): fetch that global chunk so the ring holds swizzled tiles.
  // The operands are unit-tiled (common.hpp), so every 1 KB DMA instruction reads
  // whole 64-byte unit rows (BK = 64: one contiguous unit). Rows past the edge are
  // clamped to the last row (their outputs are discarded); Xq rows are padded to 16.
  const int ks = unit_ks(K);
  const int m_rows = (g.M + 15) & ~15;
#pragma unroll
  for (int i = 0; i < C::AI; ++i) {
    const int p = (i * C::NW + b.wave) * 64 + b.lane;
    const int r = p / C::CPR, c = (p % C::CPR) ^ swz<C::CPR>(r);
    b.a_src[i] = g.Wq + unit_offset(min(n0 + r, g.N - 1), c * 16, ks);
    b.a_k[i] = c * 16;
  }
#pragma unroll
  for (int i = 0; i < C::BI; ++i) {
    const int p = (i * C::NW + b.wave) * 64 + b.lane;
    const int r = p / C::CPR, c = (p % C::CPR) ^ swz<C::CPR>(r);
    b.b_src[i] = g.Xq + unit_offset(min(m0 + r, m_rows - 1), c * 16, ks);
    b.b_k[i] = c * 16;
  }
#pragma unroll
  for (int i = 0; i < C::BN; ++i)
#pragma unroll
    for (int j = 0; j < C::BM; ++j) b.acc[i][j] = v4i{};

  // K slabs, padded to a multiple of STAGES: the padding slabs read as zeros and add
  // nothing to the exact int32 sums.
  const int nk = (ks * kUnitK + C::BK - 1) / C::BK;
  const int nk_pad = (nk + C::STAGES - 1) / C::STAGES * C::STAGES;
  b.template issue<0>(0);
  b.template issue<1>(1);
  if constexpr (C::STAGES >= 3) b.template issue<2>(2);
  if constexpr (C::STAGES >= 4) b.template issue<3>(3);
  typename GemmBlock<C>::Frags f;
  wait_and_barrier<(C::STAGES - 1) * (C::AI + C::BI)>();   // slab 0 landed
  b.template load_frags<0>(f);
  for (int kt = 0; kt < nk_pad; kt += C::STAGES) {
    b.template step<0>(kt, f);
    b.template step<1>(kt + 1, f);
    if constexpr (C::STAGES >= 3) b.template step<2>(kt + 2, f);
    if constexpr (C::STAGES >= 4) b.template step<3>(kt + 3, f);
  }
  // no DMA may still be writing this block's LDS when the block exits
  __builtin_amdgcn_s_waitcnt(0);
  gemm_epilogue<C, GATHER>(g, b.acc, n0, m0, b.wn, b.wm, b.lane, tid);
}

template <class C, bool GATHER>
__global__ __launch_bounds__(C::NT) void k_gemm(GemmArgs g, int tiles_m, int group_m) {
  int tn, tm;
  tile_of(blockIdx.x, gridDim.x, tiles_m, group_m, tn, tm);
  gemm_tile<C, GATHER>(g, tn, tm);
}

// Several weights against one quantized activation in one launch: the groups' column
// tiles are laid side by side (group q owns virtual tile columns [tn_first[q],
// tn_first[q + 1])), the XCD-aware order runs over that combined grid, and each block
// multiplies with its group's weight, constants and output (the outlier columns'
// weights dequantized from that weight in the epilogue).
template <class C>
__global__ __launch_bounds__(C::NT) void k_gemm_grouped(GroupedGemmArgs ga, int tiles_m,
                                                        int group_m) {
  int tnv, tm;
  tile_of(blockIdx.x, gridDim.x, tiles_m, group_m, tnv, tm);
  int q = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroups; ++i) q += (i < ga.G && tnv >= ga.tn_first[i]) ? 1 : 0;
  GemmArgs g = ga.base;
  g.Wq = ga.Wq[q];
  g.a_w = ga.a_w[q];
  g.Y = ga.Y[q];
  g.N = ga.N[q];
  gemm_tile<C, true>(g, tnv - ga.tn_first[q], tm);
}

#undef I8MM_LDS

}  // namespace i8mm
