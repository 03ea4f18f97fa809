// Launcher of the int8 MFMA GEMM (kernel in gemm_kernel.hpp): picks the tile shape.
#include "gemm_kernel.hpp"

namespace i8mm {

// 256 x 256 tiles, 8 waves (two per SIMD, 128 x 64 each), 4-stage ring (128 KB of LDS).
using CfgL = GemmCfg<256, 256, 64, 2, 4, 4>;
// 128 features x 256 tokens, 8 waves (64 x 64 each), 4-stage ring (96 KB).
using CfgM = GemmCfg<128, 256, 64, 2, 4, 4>;
// 128 x 128 tiles, 4 waves, 3-stage ring.
using CfgS = GemmCfg<128, 128, 64, 2, 2, 3>;

// Which tile shape: the one with the least estimated time, counted in waves of tiles
// over the CUs times the tile's cost relative to a 256 x 256 tile (its area over its
// measured rate: 1, 0.9 and 0.85 of the 256 x 256 rate on full waves). A last, partial
// wave of tiles costs at least 0.6 of a full one: its tiles run alone but not faster
// in proportion. On MI355X this picks the measured fastest shape for 2048 x 4096 x
// {4096, 12288, 16384}, 4096 x 20480 x 5120, 4096 x 12288 x 49152, 1024 x 4096 x 4096 and
// 512 x 8192 x 8192.
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
  const Tile t = pick_tile([&](int tn, int tm) {
    long n = 0;
    for (int q = 0; q < a.G; ++q) n += static_cast<long>((a.N[q] + tn - 1) / tn) * ((a.base.M + tm - 1) / tm);
    return n;
  });
  if (t == Tile::L) return run_grouped<CfgL>(a, s, 8);
  if (t == Tile::M) return run_grouped<CfgM>(a, s, 8);
  return run_grouped<CfgS>(a, s, 8);
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (gemm_skinny_supported(g.M, g.N, g.K)) return launch_gemm_skinny(g, s);
  const Tile t = pick_tile([&](int tn, int tm) {
    return static_cast<long>((g.N + tn - 1) / tn) * ((g.M + tm - 1) / tm);
  });
  if (t == Tile::L) return run<CfgL>(g, s, 8);
  if (t == Tile::M) return run<CfgM>(g, s, 8);
  return run<CfgS>(g, s, 8);
}

}  // namespace i8mm
