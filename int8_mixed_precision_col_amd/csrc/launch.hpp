// Host-side launchers of the int8mm kernels (internal to libint8mm.so).
// Each returns hipSuccess or the launch error; arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8mm {

// Weight conversion: W fp16 [K, N] (layout 0) or [N, K] (layout 1) -> unit-tiled Wq, a_w [N].
hipError_t launch_prepare_weight(const _Float16* W, int K, int N, int layout, int8_t* Wq,
                                 float* a_w, hipStream_t s);

// Layout only: int8 [N, K] row-major -> unit-tiled, K padding zeroed.
hipError_t launch_tile_weight(const int8_t* Wnk, int K, int N, int8_t* Wq, hipStream_t s);

// Column outlier flags: partial[rc * W + w] for row chunk rc < R, word w < W = ceil(K/32).
hipError_t launch_outlier_mask(const _Float16* X, int M, int K, float t, int R,
                               uint32_t* partial, hipStream_t s);
// The same over R row chunks, merged into one mask [W] (cleared first, then each chunk's
// nonzero words ORed in atomically).
hipError_t launch_outlier_mask_merged(const _Float16* X, int M, int K, float t, int R,
                                      uint32_t* mask, hipStream_t s);

struct QuantRowsArgs {
  const _Float16* X;
  int M, K;
  const uint32_t* partial;  // [R][W] column flags from launch_outlier_mask
  int R;
  int8_t* Xq;
  int xq_tiled;         // 0: Xq row-major [M][K]; 1: unit-tiled (GEMM operand layout)
  float* a_x;
  int32_t* idx_out;     // [max_outliers] ascending outlier columns (the first
                        // min(count, max_outliers)), nullable
  int32_t* count_out;   // [1]
  int32_t* status_out;  // [1], nullable
  int max_outliers;
  _Float16* Xo;         // nullable: [M][o_stride] fp16 outlier activations
  int o_stride;         // multiple of 16, >= max_outliers
  const int8_t* Wq;     // unit-tiled, for the WoT gather (nullable = no gather)
  const float* a_w;
  int N;
  _Float16* WoT;        // [N][o_stride] fp16 dequantized outlier weight rows, nullable
};
hipError_t launch_quant_rows(const QuantRowsArgs& a, hipStream_t s);

// One pass over X for the outlier flags, a provisional row constant and provisional
// codes (launch_quant_pass), then a small fix-up (launch_quant_fixup: a launch that ORs
// the blocks' flags into the column set, then one for the rows it changes and the
// gathers).
constexpr int kFlagListCap = 64;      // columns a pass-1 block lists before it stores
                                      // its whole flag mask instead
constexpr int kFixZeroMax = 64;       // more outlier columns than this: every row is
                                      // requantized in the fix-up rather than patched
constexpr int kFusedMaxChunks = 16;   // 8-half chunks per thread: K <= 32768
constexpr int kFusedMaxBlocks = 1024; // pass-1 blocks at most
struct FusedQuantArgs {
  const _Float16* X;
  int M, K;
  float t;
  int8_t* Xq;           // unit-tiled [M (padded to 16)][K (padded to 64)]
  float* a_x;           // [M]: provisional after pass 1, final after the fix-up
  int32_t* jstar;       // [M][4]: per wave of the row's block, a column reaching the
                        // provisional constant, or -1
  int32_t* lists;       // [nblk][1 + kFlagListCap]: flagged-column count (-1: see masks),
                        // then the columns
  uint32_t* masks;      // [nblk][ceil(K / 32)]: a block's flags when it lists too many
  int rows_per_block, nblk;
  uint32_t* gmask;      // [ceil(K / 32)]: the outlier columns (cleared by pass 1, ORed
                        // by the fix-up's first launch)
  int32_t* idx_out;     // [max_outliers] ascending outlier columns, nullable
  int32_t* count_out;   // [1]
  int32_t* status_out;  // [1], nullable
  int max_outliers;
  _Float16* Xo;         // nullable [M][o_stride]
  int o_stride;
  const int8_t* Wq;     // WoT gather as in QuantRowsArgs (nullable = none)
  const float* a_w;
  int N;
  _Float16* WoT;
};
bool quant_fused_supported(int64_t K);
// Pass-1 blocks for M rows of K columns, and the rows each takes.
void quant_fused_geometry(int64_t M, int64_t K, int* rows_per_block, int* nblk);
hipError_t launch_quant_pass(const FusedQuantArgs& a, hipStream_t s);
hipError_t launch_quant_fixup(const FusedQuantArgs& a, hipStream_t s);

struct GemmArgs {
  const int8_t* Wq;   // unit-tiled [N][K]
  const int8_t* Xq;   // unit-tiled [M][K] (rows padded to a multiple of 16)
  int M, N, K;
  const float* a_x;
  const float* a_w;
  const _Float16* Xo;   // [M][o_stride]
  const _Float16* WoT;  // nullable [N][o_stride]: the outlier columns' weights, gathered
                        // beforehand; when null, the epilogue dequantizes them from Wq
  const int32_t* idx;   // ascending outlier columns, the first min(count, max_outliers) valid
  int o_stride;
  const int32_t* count;
  int max_outliers;
  _Float16* Y;          // [M][ldy]
  int32_t* acc_out;     // nullable [M][ldy]
  int ldy;              // row stride of Y and acc_out in elements (0: N)
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
// A handful of tokens: the weight-stream form of the same product (one block per 16
// to 64 output features, all tokens), which launch_gemm picks for those shapes.
bool gemm_skinny_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t s);

// Up to kMaxGroups weights sharing one activation state (base holds the shared fields;
// its Wq, a_w, Y, N are unused).
constexpr int kMaxGroups = 8;
struct GroupedGemmArgs {
  GemmArgs base;
  int G;
  const int8_t* Wq[kMaxGroups];
  const float* a_w[kMaxGroups];
  _Float16* Y[kMaxGroups];
  int N[kMaxGroups];
  int tn_first[kMaxGroups + 1];  // first virtual tile column of each group (filled by the launcher)
};
hipError_t launch_gemm_grouped(GroupedGemmArgs& a, hipStream_t s);

struct DecodeArgs {
  const _Float16* X;  // [M][K]
  int M, K;
  float t;
  const int8_t* Wq;   // unit-tiled [N][K]
  const float* a_w;
  int N;
  int max_outliers;
  _Float16* Y;
  int32_t* acc_out;   // nullable
  int32_t* status;    // [0] = status, [1] = outlier count
};
bool decode_supported(int64_t M, int64_t K);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

struct WeightOnlyArgs {
  const _Float16* X;  // [M][K]
  int M, K;
  const int8_t* Wq;   // unit-tiled [N][K]
  const float* a_w;
  int N;
  _Float16* Y;        // [M][N]
};
bool weight_only_supported(int64_t M, int64_t K);
hipError_t launch_weight_only(const WeightOnlyArgs& a, hipStream_t s);

}  // namespace i8mm
