// Device helper shared by the GEMM epilogues (k_gemm, k_gemm_skinny).
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace i8mm {

// The weights of outlier ranks r0 .. r0 + 7 in output row n (the same values as the
// gathered rows WoT of the one-call path, by the same expression), dequantized from the int8
// copy that is the only weight kept in memory: fp16(Wq[n, O_r] a_w[n] / 127) ("LLM.int8():
// 8-bit Matrix Multiplication for Transformers at Scale", Abstract: the weights are
// converted to Int8 at load; the outlier columns are multiplied in 16 bit). Ranks from
// nvalid on (padding up to the 16-wide MFMA step) give 0.
__device__ __forceinline__ v8h outlier_weights(const GemmArgs& g, int n, int r0, int nvalid,
                                               int ks) {
  const float aw = g.a_w[n];
  v8h o;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = r0 + e;
    o[e] = r < nvalid ? static_cast<_Float16>(__fdiv_rn(
                            static_cast<float>(g.Wq[unit_offset(n, g.idx[r], ks)]) * aw, 127.0f))
                      : _Float16(0);
  }
  return o;
}

}  // namespace i8mm
