// Launcher of the int8 MFMA GEMM (kernel in gemm_kernel.hpp): picks the tile shape.
#include "gemm_kernel.hpp"

namespace i8mm {

// 256 x 256 tiles, 8 waves (two per SIMD, 128 x 64 each), 4-stage ring (128 KB of LDS).
using CfgL = GemmCfg<256, 256, 64, 2, 4, 4>;
// 128 features x 256 tokens, 8 waves (64 x 64 each), 4-stage ring (96 KB).
using CfgM = GemmCfg<128, 256, 64, 2, 4, 4>;
// 128 x 128 tiles, 8 waves (64 x 32 each), 4-stage ring (64 KB).
using CfgS = GemmCfg<128, 128, 64, 2, 4, 4>;

// Which tile shape: the one with the least estimated time, counted in waves of tiles
// over the CUs times the tile's cost relative to a 256 x 256 tile (its area over its
// measured rate: 1, 0.9 and 0.85 of the 256 x 256 rate on full waves). A last, partial
// wave of tiles costs at least 0.6 of a full one: its tiles run alone but not faster
// in proportion. On MI355X this picks the measured fastest shape, or one within 3% of
// it, for 2048 x 4096 x {4096, 12288, 16384}, 4096 x 4096 x 4096, 4096 x 20480 x 5120,
// 4096 x 12288 x 49152, 1024 x 4096 x 4096 and 512 x 8192 x 8192.
enum class Tile { L, M, S };
static int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
    else
      return 256;
  }
  return cus;
}
static double wave_cost(long tiles) {
  const double w = static_cast<double>(tiles) / device_cus();
  const double full = static_cast<double>(static_cast<long>(w)), frac = w - full;
  return full + (frac > 0.0 ? (frac > 0.6 ? frac : 0.6) : 0.0);
}
// tiles(tn, tm): tile count for a tile of tn features x tm tokens
template <class F>
static Tile pick_tile(F tiles) {
  const double cl = wave_cost(tiles(256, 256));
  const double cm = wave_cost(tiles(128, 256)) * (0.5 / 0.9);
  const double cs = wave_cost(tiles(128, 128)) * (0.25 / 0.85);
  if (cl <= cm && cl <= cs) return Tile::L;
  return cm <= cs ? Tile::M : Tile::S;
}

template <class C>
static hipError_t run(const GemmArgs& g, hipStream_t s, int group_m) {
  const int tiles_n = (g.N + C::TN - 1) / C::TN, tiles_m = (g.M + C::TM - 1) / C::TM;
  if (group_m > tiles_m) group_m = tiles_m;
  if (g.WoT)
    hipLaunchKernelGGL((k_gemm<C, false>), dim3(tiles_n * tiles_m), dim3(C::NT), 0, s, g, tiles_m, group_m);
  else
    hipLaunchKernelGGL((k_gemm<C, true>), dim3(tiles_n * tiles_m), dim3(C::NT), 0, s, g, tiles_m, group_m);
  return hipGetLastError();
}

template <class C>
static hipError_t run_grouped(GroupedGemmArgs& a, hipStream_t s, int group_m) {
  const int tiles_m = (a.base.M + C::TM - 1) / C::TM;
  int tn = 0;
  for (int q = 0; q < a.G; ++q) {
    a.tn_first[q] = tn;
    tn += (a.N[q] + C::TN - 1) / C::TN;
  }
  for (int q = a.G; q <= kMaxGroups; ++q) a.tn_first[q] = tn;
  if (group_m > tiles_m) group_m = tiles_m;
  hipLaunchKernelGGL(k_gemm_grouped<C>, dim3(tn * tiles_m), dim3(C::NT), 0, s, a, tiles_m, group_m);
  return hipGetLastError();
}

static hipError_t run_grouped_tile(Tile t, GroupedGemmArgs& a, hipStream_t s) {
  if (t == Tile::L) return run_grouped<CfgL>(a, s, 8);
  if (t == Tile::M) return run_grouped<CfgM>(a, s, 8);
  return run_grouped<CfgS>(a, s, 8);
}

// Groups [q0, q1) of a as a grouped product of their own.
static GroupedGemmArgs group_range(const GroupedGemmArgs& a, int q0, int q1) {
  GroupedGemmArgs r = a;
  r.G = q1 - q0;
  for (int q = 0; q < r.G; ++q) {
    r.Wq[q] = a.Wq[q0 + q];
    r.a_w[q] = a.a_w[q0 + q];
    r.Y[q] = a.Y[q0 + q];
    r.N[q] = a.N[q0 + q];
  }
  return r;
}

// Cost, in waves of 256 x 256 tiles, of the best single tile shape for the tile counts
// tiles(tn, tm).
template <class F>
static double best_cost(F tiles, Tile* t) {
  *t = pick_tile(tiles);
  if (*t == Tile::L) return wave_cost(tiles(256, 256));
  if (*t == Tile::M) return wave_cost(tiles(128, 256)) * (0.5 / 0.9);
  return wave_cost(tiles(128, 128)) * (0.25 / 0.85);
}

// Same choice of kernel and tile shape as launch_gemm, on the combined tile count. A
// handful of tokens takes the skinny kernel once per weight: its blocks fill the GPU
// at any width, and each output is then computed exactly as by the one-weight call.
hipError_t launch_gemm_grouped(GroupedGemmArgs& a, hipStream_t s) {
  bool skinny = true;
  for (int q = 0; q < a.G; ++q) skinny = skinny && gemm_skinny_supported(a.base.M, a.N[q], a.base.K);
  if (skinny) {
    for (int q = 0; q < a.G; ++q) {
      GemmArgs g = a.base;
      g.Wq = a.Wq[q];
      g.a_w = a.a_w[q];
      g.Y = a.Y[q];
      g.N = a.N[q];
      const hipError_t e = launch_gemm_skinny(g, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // tile count of groups [q0, q1) for tiles of tn features x tm tokens
  auto tiles_in = [&](int q0, int q1) {
    return [&a, q0, q1](int tn, int tm) {
      long n = 0;
      for (int q = q0; q < q1; ++q) n += static_cast<long>((a.N[q] + tn - 1) / tn) * ((a.base.M + tm - 1) / tm);
      return n;
    };
  };
  const Tile t = pick_tile(tiles_in(0, a.G));
  // A split at a group boundary, as launch_gemm splits a product: when the leading groups'
  // 256 x 256 tiles fill whole waves and the single launch would end on a partial wave,
  // the leading groups take one launch of 256 x 256 tiles and the rest a second launch
  // with the shape that suits them. The grouped epilogue dequantizes the outlier columns'
  // weights in every tile, and a partial last wave measured costlier here than on the
  // one-weight path (Q, K, V of 2048 x 4096: half a wave took 0.77 of a full one; the
  // split took the grouped GEMM from 114.6 to 107.3 us), so the single launch's partial
  // wave is counted as at least 0.75 of a wave.
  if (t == Tile::L) {
    const long cus = device_cus(), total = tiles_in(0, a.G)(256, 256);
    const double w = static_cast<double>(total) / cus, full = static_cast<double>(total / cus);
    const double single = full + (w > full ? (w - full > 0.75 ? w - full : 0.75) : 0.0);
    long lead = 0;
    for (int j = 1; j < a.G && total % cus != 0; ++j) {
      lead += tiles_in(j - 1, j)(256, 256);
      if (lead % cus != 0) continue;
      Tile t2;
      const double split = static_cast<double>(lead / cus) + best_cost(tiles_in(j, a.G), &t2) + 0.05;
      if (split < single) {
        GroupedGemmArgs a1 = group_range(a, 0, j), a2 = group_range(a, j, a.G);
        const hipError_t e = run_grouped<CfgL>(a1, s, 8);
        if (e != hipSuccess) return e;
        return run_grouped_tile(t2, a2, s);
      }
      break;
    }
  }
  return run_grouped_tile(t, a, s);
}

// Features [n0, n1) of the product g as a product of its own (n0 a multiple of 16: the
// slice starts at a unit-row boundary of Wq), writing into the same Y rows.
static GemmArgs feature_slice(const GemmArgs& g, int n0, int n1) {
  GemmArgs s = g;
  s.Wq = g.Wq + static_cast<size_t>(n0 / kUnitRows) * unit_ks(g.K) * kUnitBytes;
  s.a_w = g.a_w + n0;
  if (g.WoT) s.WoT = g.WoT + static_cast<size_t>(n0) * g.o_stride;
  s.Y = g.Y + n0;
  if (g.acc_out) s.acc_out = g.acc_out + n0;
  s.N = n1 - n0;
  s.ldy = g.ldy > 0 ? g.ldy : g.N;
  return s;
}

static hipError_t run_tile(Tile t, const GemmArgs& g, hipStream_t s) {
  if (t == Tile::L) return run<CfgL>(g, s, 8);
  if (t == Tile::M) return run<CfgM>(g, s, 8);
  return run<CfgS>(g, s, 8);
}

// Cost, in waves of 256 x 256 tiles, of the best single tile shape over M x N.
static double best_cost(long M, long N, Tile* t) {
  return best_cost([&](int tn, int tm) { return ((N + tn - 1) / tn) * ((M + tm - 1) / tm); }, t);
}

// A last, partial wave of 256 x 256 tiles leaves CUs idle for a whole tile's time (the
// 4096 x 20480 x 5120 product has 1.25 waves of them). When the output holds at least
// one whole wave, the leading feature columns that fill whole waves take 256 x 256
// tiles and the remaining features a second launch with the tile shape that suits
// them, if the estimate (plus a twentieth of a wave for the second launch) is lower.
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (gemm_skinny_supported(g.M, g.N, g.K)) return launch_gemm_skinny(g, s);
  Tile t1;
  const double single = best_cost(g.M, g.N, &t1);
  const long cus = device_cus(), tiles_m = (g.M + 255) / 256;
  const long waves = static_cast<long>((g.N + 255) / 256) * tiles_m / cus;
  const long n_split = waves * cus / tiles_m * 256;
  if (waves >= 1 && n_split > 0 && n_split < g.N) {
    Tile t2;
    const double rest = best_cost(g.M, g.N - n_split, &t2);
    const double lead = wave_cost(n_split / 256 * tiles_m);
    if (lead + rest + 0.05 < single) {
      const hipError_t e = run<CfgL>(feature_slice(g, 0, int(n_split)), s, 8);
      if (e != hipSuccess) return e;
      return run_tile(t2, feature_slice(g, int(n_split), g.N), s);
    }
  }
  return run_tile(t1, g, s);
}

}  // namespace i8mm
