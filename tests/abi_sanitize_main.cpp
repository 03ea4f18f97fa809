// Host-only driver for the sanitizer build of the C ABI's argument validation (no GPU):
// every call below is rejected before the library touches the HIP runtime, so under
// AddressSanitizer and UndefinedBehaviorSanitizer this exercises the validation code,
// the size helpers and the status strings alone. Exit status 0 when every return value
// is the documented one.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "int8mm.h"

static int failures = 0;

static void expect(const char* what, long long got, long long want) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: got %lld, want %lld\n", what, got, want);
    ++failures;
  }
}

int main() {
  // fake, 16-byte-aligned device addresses: never dereferenced, the calls fail first
  void* P = reinterpret_cast<void*>(uintptr_t(0x10000));
  void* U = reinterpret_cast<void*>(uintptr_t(0x10008));
  int8_t* Pi = static_cast<int8_t*>(P);
  float* Pf = static_cast<float*>(P);
  int32_t* Pl = static_cast<int32_t*>(P);
  uint32_t* Pu = static_cast<uint32_t*>(P);
  const size_t big = size_t(1) << 40;

  // prepare / tile
  expect("prepare null", int8_prepare_weight(nullptr, 64, 64, 0, Pi, Pf, nullptr), INT8MM_E_NULL);
  expect("prepare K", int8_prepare_weight(P, 60, 64, 0, Pi, Pf, nullptr), INT8MM_E_SHAPE);
  expect("prepare layout", int8_prepare_weight(P, 64, 64, 7, Pi, Pf, nullptr), INT8MM_E_SHAPE);
  expect("prepare align", int8_prepare_weight(U, 64, 64, 1, Pi, Pf, nullptr), INT8MM_E_ALIGN);
  expect("tile null", int8_tile_weight(nullptr, 64, 64, Pi, nullptr), INT8MM_E_NULL);
  expect("tile N", int8_tile_weight(Pi, 64, 8, Pi, nullptr), INT8MM_E_SHAPE);
  expect("tile align", int8_tile_weight(static_cast<int8_t*>(U), 64, 64, Pi, nullptr), INT8MM_E_ALIGN);

  // quant rows
  expect("quant null idx", int8_quant_rows(P, 4, 64, 6.0f, Pi, Pf, Pu, nullptr, Pl, 4, nullptr), INT8MM_E_NULL);
  expect("quant mo", int8_quant_rows(P, 4, 64, 6.0f, Pi, Pf, Pu, Pl, Pl, 65, nullptr), INT8MM_E_SHAPE);
  expect("quant t", int8_quant_rows(P, 4, 64, -1.0f, Pi, Pf, Pu, Pl, Pl, 4, nullptr), INT8MM_E_THRESHOLD);
  expect("quant nan", int8_quant_rows(P, 4, 64, __builtin_nanf(""), Pi, Pf, Pu, Pl, Pl, 4, nullptr),
         INT8MM_E_THRESHOLD);

  // mixed matmul, every argument class, at the limits of the int64 arguments too
  const int64_t shapes[][3] = {{0, 64, 64}, {-1, 64, 64}, {1, 0, 64}, {1, 63, 64}, {1, 64, 0},
                               {1, 64, 24}, {1, 133152, 64}, {int64_t(1) << 25, 64, 64},
                               {1, INT64_MAX, 64}, {INT64_MAX, 64, INT64_MAX}, {1, 64, INT64_MIN}};
  for (const auto& s : shapes) {
    expect("mm shape", int8_mixed_matmul(P, s[0], s[1], Pi, Pf, s[2], 6.0f, 0, P, P, big, nullptr, nullptr),
           INT8MM_E_SHAPE);
    expect("ws bytes 0", static_cast<long long>(int8_mixed_matmul_workspace_bytes(s[0], s[1], s[2], 0)), 0);
    expect("noalloc shape", int8_mixed_matmul_noalloc(P, s[0], s[1], Pi, Pf, s[2], 6.0f, 0, P, nullptr, nullptr),
           INT8MM_E_SHAPE);
  }
  expect("mm ws null", int8_mixed_matmul(P, 8, 64, Pi, Pf, 64, 6.0f, 4, P, nullptr, big, nullptr, nullptr),
         INT8MM_E_NULL);
  expect("mm ws small", int8_mixed_matmul(P, 300, 1040, Pi, Pf, 528, 6.0f, 4, P, P, 16, nullptr, nullptr),
         INT8MM_E_WORKSPACE);
  expect("mm acc align", int8_mixed_matmul(P, 8, 64, Pi, Pf, 64, 6.0f, 4, P, P, big, static_cast<int32_t*>(U), nullptr),
         INT8MM_E_ALIGN);
  expect("mm mo", int8_mixed_matmul(P, 8, 64, Pi, Pf, 64, 6.0f, 8193, P, P, big, nullptr, nullptr), INT8MM_E_SHAPE);
  expect("noalloc scratch", int8_mixed_matmul_noalloc(P, 8192, 8192, Pi, Pf, 256, 6.0f, 256, P, nullptr, nullptr),
         INT8MM_E_SCRATCH);
  expect("is decode", int8_mixed_matmul_is_decode(8, 4096), 1);
  expect("is decode big", int8_mixed_matmul_is_decode(INT64_MAX, INT64_MAX), 0);
  const size_t wb = int8_mixed_matmul_workspace_bytes(4096, 133136, int64_t(1) << 24, 8192);
  expect("ws huge nonzero", wb > (size_t(1) << 30), 1);
  expect("prepared bytes", static_cast<long long>(int8_prepared_weight_bytes(1040, 528)), 528 * 1088);
  expect("prepared bytes bad", static_cast<long long>(int8_prepared_weight_bytes(INT64_MAX, 16)), 0);

  // quantize once / grouped
  expect("state bytes bad", static_cast<long long>(int8_quant_state_bytes(INT64_MAX, 64, 4)), 0);
  int64_t lay[6];
  expect("state layout", int8_quant_state_layout(4096, 20480, 256, lay), INT8MM_OK);
  expect("state layout null", int8_quant_state_layout(4096, 20480, 256, nullptr), INT8MM_E_NULL);
  expect("state layout bad", int8_quant_state_layout(INT64_MAX, 64, 4, lay), INT8MM_E_SHAPE);
  expect("qa short", int8_quantize_activations(P, 64, 256, 6.0f, 16, P, 1, nullptr), INT8MM_E_WORKSPACE);
  expect("mmq null", int8_mixed_matmul_q(P, 64, 256, 16, nullptr, Pf, 128, P, P, 256, nullptr, nullptr),
         INT8MM_E_NULL);
  const int64_t ns[9] = {64, 64, 64, 64, 64, 64, 64, 64, 64};
  const int8_t* wq[9] = {Pi, Pi, Pi, Pi, Pi, Pi, Pi, Pi, Pi};
  const float* aw[9] = {Pf, Pf, Pf, Pf, Pf, Pf, Pf, Pf, Pf};
  void* ys[9] = {P, P, P, P, P, P, P, P, P};
  expect("grouped G", int8_mixed_matmul_q_grouped(P, 64, 256, 16, 9, wq, aw, ns, ys, P, big, nullptr),
         INT8MM_E_SHAPE);
  expect("grouped G0", int8_mixed_matmul_q_grouped(P, 64, 256, 16, 0, wq, aw, ns, ys, P, big, nullptr),
         INT8MM_E_SHAPE);
  expect("grouped ws", static_cast<long long>(int8_mixed_matmul_q_grouped_workspace_bytes(9, ns, 16)), 0);
  expect("weight-only M", int8_weight_only_matmul(P, 17, 64, Pi, Pf, 64, P, nullptr), INT8MM_E_SHAPE);

  // status strings and the timing hook without launches
  for (int c = -3; c < 12; ++c) expect("strerror", strlen(int8mm_strerror(c)) > 0, 1);
  expect("timing mode", int8mm_timing_enable(3), INT8MM_E_SHAPE);
  expect("timing mode neg", int8mm_timing_enable(-1), INT8MM_E_SHAPE);
  double ms[3];
  int64_t n[3];
  expect("timing read", int8mm_timing_read_phases(ms, n), INT8MM_OK);
  expect("timing read null", int8mm_timing_read_phases(nullptr, n), INT8MM_E_NULL);
  expect("status null", int8mm_read_status(nullptr, nullptr, nullptr), INT8MM_E_NULL);

  if (failures) fprintf(stderr, "%d failures\n", failures);
  else printf("abi sanitize driver: all checks passed\n");
  return failures ? 1 : 0;
}
