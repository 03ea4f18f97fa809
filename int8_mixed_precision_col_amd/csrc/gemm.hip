// Launcher of the int8 MFMA GEMM (kernel in gemm_kernel.hpp): picks the tile shape.
#include "gemm_kernel.hpp"

namespace i8mm {

// Large problems: 256 x 256 tiles, 8 waves (two per SIMD, 128 x 64 each), 4-stage ring
// (128 KB of LDS).
using CfgL = GemmCfg<256, 256, 64, 2, 4, 4>;
// Small or skinny problems: 128 x 128 tiles, 4 waves.
using CfgS = GemmCfg<128, 128, 64, 2, 2, 3>;

template <class C>
static hipError_t run(const GemmArgs& g, hipStream_t s, int group_m) {
  const int tiles_n = (g.N + C::TN - 1) / C::TN, tiles_m = (g.M + C::TM - 1) / C::TM;
  if (group_m > tiles_m) group_m = tiles_m;
  hipLaunchKernelGGL(k_gemm<C>, dim3(tiles_n * tiles_m), dim3(C::NT), 0, s, g, tiles_m, group_m);
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
  long tiles_l = 0;
  for (int q = 0; q < a.G; ++q) tiles_l += static_cast<long>((a.N[q] + 255) / 256) * ((a.base.M + 255) / 256);
  if (a.base.M >= 256 && tiles_l >= 256) return run_grouped<CfgL>(a, s, 8);
  return run_grouped<CfgS>(a, s, 8);
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (gemm_skinny_supported(g.M, g.N, g.K)) return launch_gemm_skinny(g, s);
  const long tiles_l = static_cast<long>((g.N + 255) / 256) * ((g.M + 255) / 256);
  if (g.M >= 256 && tiles_l >= 256) return run<CfgL>(g, s, 8);
  return run<CfgS>(g, s, 8);
}

}  // namespace i8mm
