// Weight conversion: fp16 W -> int8 Wq (unit-tiled, see common.hpp) + fp32 column absmax.
//
// "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale", Abstract: a
// 16/32-bit checkpoint is converted to Int8 when it is loaded. "Compress your LLMs",
// Vector-wise quantization: every column of the weight matrix (an output feature) has
// its own scaling constant, here the absmax of that column over all K inputs.
// Runs once per weight, outside the timed matmul; HBM-bound.
#include "common.hpp"
#include "launch.hpp"

namespace i8mm {

// a_w[n] = max_k |W[k, n]| for W [K, N] row-major. One block per 64-column strip:
// 8 threads x 16 B cover a 128-byte row segment, 32 rows per pass.
__global__ __launch_bounds__(256) void k_colmax_kn(const _Float16* __restrict__ W, int K, int N,
                                                   float* __restrict__ a_w) {
  const int tid = threadIdx.x;
  const int cg = tid & 7;
  const int col0 = blockIdx.x * 64 + cg * 8;
  float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (col0 < N) {
#pragma unroll 4
    for (int k = tid >> 3; k < K; k += 32) {
      // non-temporal: 0.64 -> 0.59 ms for the whole conversion of the 175B-share weight
      // (also making the second pass's loads or the Wq stores non-temporal was slower)
      v8h v = __builtin_nontemporal_load(
          reinterpret_cast<const v8h*>(W + static_cast<size_t>(k) * N + col0));
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], fabsf(static_cast<float>(v[e])));
    }
  }
  __shared__ float red[4][64];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float v = m[e];
    v = fmaxf(v, __shfl_xor(v, 8, 64));
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    v = fmaxf(v, __shfl_xor(v, 32, 64));
    m[e] = v;
  }
  if ((tid & 63) < 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tid >> 6][cg * 8 + e] = m[e];
  }
  __syncthreads();
  if (tid < 64) {
    const int n = blockIdx.x * 64 + tid;
    float v = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
    if (n < N) a_w[n] = v;
  }
}

// Wq(n, k) = q(W[k, n], a_w[n]) for a 64 (k) x 64 (n) tile, transposed through LDS;
// K-padding bytes (k >= K in the last unit) are written as zero codes.
__global__ __launch_bounds__(256) void k_quant_transpose_kn(const _Float16* __restrict__ W, int K,
                                                            int N, const float* __restrict__ a_w,
                                                            int8_t* __restrict__ Wq) {
  __shared__ _Float16 tile[64][64 + 2];
  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  // load: 64 rows (k) x 8 chunks of 8 halves
  for (int i = tid; i < 512; i += 256) {
    const int r = i >> 3, c = i & 7;
    const int k = k0 + r, n = n0 + c * 8;
    v8h v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (k < K && n < N) v = *reinterpret_cast<const v8h*>(W + static_cast<size_t>(k) * N + n);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[r][c * 8 + e] = v[e];
  }
  __syncthreads();
  // store: thread -> (n row, 16 consecutive k)
  const int nl = tid >> 2, kseg = (tid & 3) * 16;
  const int n = n0 + nl, k = k0 + kseg;
  if (n >= N) return;  // k < 64 * unit_ks(K): loaded as zeros past K, so codes are 0
  const float a = a_w[n], r = quant_scale(a);
  int q[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) q[e] = quant_code_fast(static_cast<float>(tile[kseg + e][nl]), a, r);
  v4u out;
  out[0] = pack4(q[0], q[1], q[2], q[3]);
  out[1] = pack4(q[4], q[5], q[6], q[7]);
  out[2] = pack4(q[8], q[9], q[10], q[11]);
  out[3] = pack4(q[12], q[13], q[14], q[15]);
  *reinterpret_cast<v4u*>(Wq + unit_offset(n, k, unit_ks(K))) = out;
}

// W [N, K] row-major (output-feature rows): one wave per row, absmax then quantize;
// the row's K padding is written as zero codes.
__global__ __launch_bounds__(256) void k_quant_rows_nk(const _Float16* __restrict__ W, int K, int N,
                                                       int8_t* __restrict__ Wq,
                                                       float* __restrict__ a_w) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const _Float16* row = W + static_cast<size_t>(n) * K;
  const int nchunk = K >> 3;
  float m = 0.0f;
  for (int c = lane; c < nchunk; c += 64) {
    v8h v = *reinterpret_cast<const v8h*>(row + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(static_cast<float>(v[e])));
  }
  m = wave_max(m);
  if (lane == 0) a_w[n] = m;
  const float r = quant_scale(m);
  for (int c = lane; c < nchunk; c += 64) {
    v8h v = *reinterpret_cast<const v8h*>(row + c * 8);
    v2u o;
    o[0] = pack4(quant_code_fast(v[0], m, r), quant_code_fast(v[1], m, r),
                 quant_code_fast(v[2], m, r), quant_code_fast(v[3], m, r));
    o[1] = pack4(quant_code_fast(v[4], m, r), quant_code_fast(v[5], m, r),
                 quant_code_fast(v[6], m, r), quant_code_fast(v[7], m, r));
    *reinterpret_cast<v2u*>(Wq + unit_offset(n, c * 8, unit_ks(K))) = o;
  }
  const int ks = unit_ks(K);
  for (int c = nchunk + lane; c < ks * 8; c += 64)
    *reinterpret_cast<v2u*>(Wq + unit_offset(n, c * 8, ks)) = v2u{0u, 0u};
}

// Layout only: an int8 [N, K] row-major matrix into the unit-tiled layout, the K
// padding as zero bytes. Thread t writes the 16-byte piece t of the output: unit
// t / 64 (group g = unit / KS, unit s = unit % KS), row (t / 4) % 16, bytes 16 (t % 4)
// of the unit's 64; its source is row 16 g + that row, columns 64 s + 16 (t % 4) ..
// + 15 (K is a multiple of 16, so a piece lies wholly inside K or wholly past it).
__global__ __launch_bounds__(256) void k_tile_weight(const int8_t* __restrict__ Wnk, int K, int ks,
                                                     int8_t* __restrict__ Wq, long pieces) {
  const long t = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= pieces) return;
  const long unit = t >> 6;
  const int r = static_cast<int>((t >> 2) & 15), c = static_cast<int>(t & 3);
  const long g = unit / ks;
  const int su = static_cast<int>(unit - g * ks);
  const int k = 64 * su + 16 * c;
  v4u v = {0u, 0u, 0u, 0u};
  if (k < K) v = *reinterpret_cast<const v4u*>(Wnk + (g * 16 + r) * static_cast<long>(K) + k);
  *reinterpret_cast<v4u*>(Wq + t * 16) = v;
}

hipError_t launch_tile_weight(const int8_t* Wnk, int K, int N, int8_t* Wq, hipStream_t s) {
  const int ks = unit_ks(K);
  const long pieces = static_cast<long>(N) * ks * 4;
  hipLaunchKernelGGL(k_tile_weight, dim3(static_cast<unsigned>((pieces + 255) / 256)), dim3(256), 0, s,
                     Wnk, K, ks, Wq, pieces);
  return hipGetLastError();
}

hipError_t launch_prepare_weight(const _Float16* W, int K, int N, int layout, int8_t* Wq,
                                 float* a_w, hipStream_t s) {
  if (layout == 0) {
    hipLaunchKernelGGL(k_colmax_kn, dim3((N + 63) / 64), dim3(256), 0, s, W, K, N, a_w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_quant_transpose_kn, dim3((N + 63) / 64, (K + 63) / 64), dim3(256), 0, s,
                       W, K, N, a_w, Wq);
  } else {
    hipLaunchKernelGGL(k_quant_rows_nk, dim3((N + 3) / 4), dim3(256), 0, s, W, K, N, Wq, a_w);
  }
  return hipGetLastError();
}

}  // namespace i8mm
