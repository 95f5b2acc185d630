// Drives every entry point of kda_api.cpp through its argument checks
// (NULL, shape, alignment, workspace, dtype, unsupported head size) and a
// valid call, host-only, with the launchers replaced by counting doubles.
// Built with -fsanitize=address,undefined by tests/test_sanitizers.py; exits
// non-zero on the first unexpected status.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kda.h"

namespace kda { extern int g_launches; }

static int failures = 0;
#define EXPECT(call, want)                                                                         \
  do {                                                                                             \
    const int before = kda::g_launches;                                                            \
    const kda_status got = (call);                                                                 \
    if (got != (want)) {                                                                           \
      std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got, want);   \
      ++failures;                                                                                  \
    }                                                                                              \
    if ((want) != KDA_OK && kda::g_launches != before) {                                           \
      std::fprintf(stderr, "line %d: a launcher ran before the check failed\n", __LINE__);          \
      ++failures;                                                                                  \
    }                                                                                              \
  } while (0)

int main() {
  // host buffers stand in for device pointers: nothing here dereferences them
  std::vector<float> buf(1 << 16);
  void* p = buf.data();
  void* mis = static_cast<char*>(p) + 4;   // not 16-byte aligned
  const float* fp = buf.data();
  float* wp = buf.data();
  const int32_t* cu = reinterpret_cast<const int32_t*>(buf.data());
  std::vector<unsigned char> ws(1 << 20);
  const int N = 2, H = 2, D = 64;
  const int64_t T = 100;
  const size_t need = kda_prefill_workspace_size(N, T, H, D, D, KDA_BF16);
  if (need == 0 || need > ws.size()) { std::fprintf(stderr, "workspace size %zu\n", need); return 2; }

  // prefill and its forms
  EXPECT(kda_prefill_varlen(p, p, p, fp, p, cu, nullptr, p, wp, N, T, H, D, D, KDA_BF16, ws.data(), ws.size(), nullptr), KDA_OK);
  EXPECT(kda_prefill_varlen(nullptr, p, p, fp, p, cu, nullptr, p, wp, N, T, H, D, D, KDA_BF16, ws.data(), ws.size(), nullptr), KDA_ERR_NULL);
  EXPECT(kda_prefill_varlen(p, p, p, fp, p, nullptr, nullptr, p, wp, N, T, H, D, D, KDA_BF16, ws.data(), ws.size(), nullptr), KDA_ERR_NULL);
  EXPECT(kda_prefill_varlen(mis, p, p, fp, p, cu, nullptr, p, wp, N, T, H, D, D, KDA_BF16, ws.data(), ws.size(), nullptr), KDA_ERR_ALIGN);
  EXPECT(kda_prefill_varlen(p, p, p, fp, p, cu, nullptr, p, wp, N, T, H, D, D, KDA_BF16, ws.data(), need - 1, nullptr), KDA_ERR_WORKSPACE);
  EXPECT(kda_prefill_varlen(p, p, p, fp, p, cu, nullptr, p, wp, N, T, H, D, D, KDA_BF16, nullptr, 0, nullptr), KDA_ERR_WORKSPACE);
  EXPECT(kda_prefill_varlen(p, p, p, fp, p, cu, nullptr, p, wp, N, T, H, 96, 96, KDA_BF16, ws.data(), ws.size(), nullptr), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_prefill_varlen(p, p, p, fp, p, cu, nullptr, p, wp, N, T, H, 128, 64, KDA_BF16, ws.data(), ws.size(), nullptr), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_prefill_varlen(p, p, p, fp, p, cu, nullptr, p, wp, N, T, H, D, D, (kda_dtype)7, ws.data(), ws.size(), nullptr), KDA_ERR_DTYPE);
  EXPECT(kda_prefill_varlen(p, p, p, fp, p, cu, nullptr, p, wp, 0, T, H, D, D, KDA_BF16, ws.data(), ws.size(), nullptr), KDA_ERR_SHAPE);
  EXPECT(kda_prefill_varlen(p, p, p, fp, p, cu, nullptr, p, wp, N, -1, H, D, D, KDA_BF16, ws.data(), ws.size(), nullptr), KDA_ERR_SHAPE);
  EXPECT(kda_prefill_varlen(p, p, p, fp, p, cu, nullptr, p, wp, N, T, 0, D, D, KDA_BF16, ws.data(), ws.size(), nullptr), KDA_ERR_SHAPE);
  EXPECT(kda_prefill_varlen(nullptr, nullptr, nullptr, nullptr, nullptr, cu, fp, nullptr, wp, N, 0, H, D, D, KDA_BF16, nullptr, 0, nullptr), KDA_OK);
  EXPECT(kda_gdn_prefill_varlen(p, p, p, fp, p, cu, fp, p, wp, N, T, H, D, D, KDA_F32, ws.data(), ws.size(), nullptr), KDA_OK);
  EXPECT(kda_prefill_varlen_raw(p, p, p, fp, p, cu, nullptr, p, wp, N, T, H, D, D, KDA_BF16, ws.data(), ws.size(), nullptr), KDA_OK);
  EXPECT(kda_prefill_varlen_raw(p, p, p, fp, nullptr, cu, nullptr, p, wp, N, T, H, D, D, KDA_BF16, ws.data(), ws.size(), nullptr), KDA_ERR_NULL);
  const int32_t* sidx = cu;
  EXPECT(kda_prefill_varlen_pooled(p, p, p, fp, p, cu, sidx, wp, 4, 1, p, N, T, H, D, D, KDA_BF16, ws.data(), ws.size(), nullptr), KDA_OK);
  EXPECT(kda_prefill_varlen_pooled(p, p, p, fp, p, cu, nullptr, wp, 4, 1, p, N, T, H, D, D, KDA_BF16, ws.data(), ws.size(), nullptr), KDA_ERR_NULL);
  EXPECT(kda_prefill_varlen_pooled(p, p, p, fp, p, cu, sidx, wp, -1, 1, p, N, T, H, D, D, KDA_BF16, ws.data(), ws.size(), nullptr), KDA_ERR_SHAPE);

  // decode and its forms
  EXPECT(kda_decode_step(p, p, p, fp, p, wp, p, N, H, D, D, KDA_BF16, nullptr), KDA_OK);
  EXPECT(kda_decode_step(p, p, p, fp, p, nullptr, p, N, H, D, D, KDA_BF16, nullptr), KDA_ERR_NULL);
  EXPECT(kda_decode_step(p, p, p, fp, p, wp, mis, N, H, D, D, KDA_BF16, nullptr), KDA_ERR_ALIGN);
  EXPECT(kda_decode_step(p, p, p, fp, p, wp, p, N, H, 32, 32, KDA_BF16, nullptr), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_decode_step(p, p, p, fp, p, wp, p, -1, H, D, D, KDA_BF16, nullptr), KDA_ERR_SHAPE);
  EXPECT(kda_decode_step(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, H, D, D, KDA_BF16, nullptr), KDA_OK);
  EXPECT(kda_gdn_decode_step(p, p, p, fp, p, wp, p, N, H, D, D, KDA_F32, nullptr), KDA_OK);
  EXPECT(kda_decode_step_raw(p, p, p, fp, p, wp, p, N, H, D, D, KDA_BF16, nullptr), KDA_OK);
  EXPECT(kda_decode_step_pooled(p, p, p, fp, p, sidx, wp, 4, p, N, H, D, D, KDA_BF16, nullptr), KDA_OK);
  EXPECT(kda_decode_step_pooled(p, p, p, fp, p, sidx, nullptr, 4, p, N, H, D, D, KDA_BF16, nullptr), KDA_ERR_NULL);

  // backward
  const size_t bneed = kda_prefill_backward_workspace_size(N, T, H, D, D, KDA_F32);
  std::vector<unsigned char> bws(bneed + 16);
  EXPECT(kda_prefill_backward(p, p, p, fp, p, cu, nullptr, p, nullptr, wp, wp, wp, wp, wp, nullptr, N, T, H, D, D,
                              KDA_F32, bws.data(), bneed, nullptr), KDA_OK);
  EXPECT(kda_prefill_backward(p, p, p, fp, p, cu, nullptr, nullptr, nullptr, wp, wp, wp, wp, wp, nullptr, N, T, H, D,
                              D, KDA_F32, bws.data(), bneed, nullptr), KDA_ERR_NULL);
  EXPECT(kda_prefill_backward(p, p, p, fp, p, cu, nullptr, p, nullptr, wp, wp, wp, wp, wp, nullptr, N, T, H, D, D,
                              KDA_F32, bws.data(), bneed - 1, nullptr), KDA_ERR_WORKSPACE);

  // sizes and strings
  if (kda_prefill_workspace_size(N, T, H, 96, 96, KDA_BF16) != 0) ++failures;
  if (kda_prefill_status_offset(N, T, H, 96, 96, KDA_BF16) != SIZE_MAX) ++failures;
  for (int s = -1; s < 12; ++s)
    if (!kda_status_string((kda_status)s)) ++failures;
  std::printf("abi driver: %d failures, %d launches\n", failures, kda::g_launches);
  return failures == 0 ? 0 : 1;
}
