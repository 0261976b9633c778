// Host-side checks of the library's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (test infrastructure; tests/test_host_sanitizers.py
// builds and runs it on a machine without a GPU).
//
// The library's sources are built with the sanitizers on their host code
// and linked into this program, which runs only where no GPU is present
// (it checks, and its test skips otherwise): a call that passes validation
// ends at its launch with TQ_E_HIP.  Every pointer handed over is a fake,
// aligned address that the host code must never dereference.  What runs is every
// validation path, the pure host helpers, and counts and strides at the ends
// of their ranges, where an unchecked product would overflow.  A wrong status
// or any sanitizer report fails the run.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include <hip/hip_runtime_api.h>

#include "../../include/tq.h"

namespace {

int g_fails = 0;
int g_checks = 0;

void expect(long long got, long long want, const char* what, int line) {
  ++g_checks;
  if (got != want) {
    std::fprintf(stderr, "line %d: %s -> %lld, expected %lld\n", line, what, got, want);
    ++g_fails;
  }
}
#define EXPECT(expr, want) expect((long long)(expr), (long long)(want), #expr, __LINE__)

// A call that passed validation: it either had nothing to do or reached its
// launch, which fails without device code.
void expect_launch(int32_t got, const char* what, int line) {
  ++g_checks;
  if (got != TQ_E_HIP) {
    std::fprintf(stderr, "line %d: %s -> %d, expected the launch to fail (%d)\n", line, what, got, TQ_E_HIP);
    ++g_fails;
  }
}
#define EXPECT_LAUNCH(expr) expect_launch((expr), #expr, __LINE__)

template <typename T>
T* fake(uintptr_t addr) {
  return reinterpret_cast<T*>(addr);
}

const uintptr_t A = uintptr_t(1) << 32;  // fake device addresses, 1 GiB apart
uintptr_t at(int i) { return A + (uintptr_t(i) << 30); }

tq_planes planes_at(int first) {
  return tq_planes{fake<void>(at(first)), fake<void>(at(first + 1)), fake<void>(at(first + 2)),
                   fake<void>(at(first + 3)), fake<void>(at(first + 4))};
}

bool served_d(int d) { return d == 64 || d == 128 || d == 256 || d == 512; }
bool served_k(int b) { return b == 2 || b == 4 || b == 5 || b == 8; }
bool served_v(int b) { return b == 2 || b == 3 || b == 4 || b == 5 || b == 8; }

void schemes_and_helpers() {
  EXPECT(tq_check_scheme(nullptr), TQ_E_NULL);
  const int dims[] = {INT_MIN, -128, 0, 1, 32, 63, 64, 96, 128, 256, 384, 512, 1024, INT_MAX};
  const int bits[] = {INT_MIN, -1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 16, INT_MAX};
  for (int d : dims)
    for (int kb : bits)
      for (int vb : bits) {
        const tq_scheme s{d, kb, vb};
        const int32_t want = !served_d(d) ? TQ_E_HEAD_DIM : (!served_k(kb) || !served_v(vb)) ? TQ_E_BITS : TQ_OK;
        EXPECT(tq_check_scheme(&s), want);
        int64_t total = 0;
        for (int p = -2; p < 7; ++p) {
          const int64_t rb = tq_plane_row_bytes(&s, p);
          if (want != TQ_OK) {
            EXPECT(rb, want);
          } else if (p < 0 || p > 4) {
            EXPECT(rb, TQ_E_PLANE);
          } else {
            const int64_t g = d / 32;
            const int64_t expect_rb = p == TQ_PLANE_K_Q ? (kb == 8 ? d : d * kb / 8)
                                      : p == TQ_PLANE_V_Q ? d * vb / 8 : 2 * g;
            EXPECT(rb, expect_rb);
            total += rb;
          }
        }
        EXPECT(tq_row_bytes(&s), want == TQ_OK ? total : want);
      }
  const tq_scheme k8v3{128, 8, 3};
  EXPECT(tq_row_bytes(&k8v3), 200);
  EXPECT(tq_plane_row_bytes(nullptr, 0), TQ_E_NULL);
  EXPECT(tq_row_bytes(nullptr), TQ_E_NULL);

  static float cen[256], bnd[255];
  for (int b : bits) {
    const bool ok = b == 1 || b == 2 || b == 3 || b == 4 || b == 5 || b == 8;
    EXPECT(tq_codebook(b, cen, bnd), ok ? TQ_OK : TQ_E_BITS);
    if (ok) {
      for (int i = 0; i + 1 < (1 << b); ++i) {
        EXPECT(cen[i] < bnd[i] && bnd[i] < cen[i + 1], 1);
      }
    }
    EXPECT(tq_codebook(b, nullptr, bnd), ok ? TQ_E_NULL : TQ_E_BITS);
    EXPECT(tq_codebook(b, cen, nullptr), ok ? TQ_E_NULL : TQ_E_BITS);
  }
  for (int st = -40; st <= 40; ++st) {
    const char* m = tq_status_string(st);
    EXPECT(m != nullptr && std::strlen(m) > 0, 1);
  }
  EXPECT(tq_status_string(INT_MIN) != nullptr, 1);
  EXPECT(tq_status_string(INT_MAX) != nullptr, 1);

  EXPECT(tq_grown_capacity(0), 0);
  EXPECT(tq_grown_capacity(1), 256);
  EXPECT(tq_grown_capacity(256), 256);
  EXPECT(tq_grown_capacity(257), 512);
  EXPECT(tq_grown_capacity((int64_t)INT32_MAX - 255), (int64_t)INT32_MAX - 255);
  EXPECT(tq_grown_capacity((int64_t)INT32_MAX - 254), TQ_E_SHAPE);
  EXPECT(tq_grown_capacity(INT32_MAX), TQ_E_SHAPE);
  EXPECT(tq_grown_capacity(INT64_MAX), TQ_E_SHAPE);
  EXPECT(tq_grown_capacity(-1), TQ_E_SHAPE);
  EXPECT(tq_grown_capacity(INT64_MIN), TQ_E_SHAPE);
}

void codec_calls() {
  const tq_scheme s{128, 8, 3};
  const tq_planes p = planes_at(0);
  const uint16_t* k = fake<const uint16_t>(at(10));
  const uint16_t* v = fake<const uint16_t>(at(11));
  const int8_t* sg = fake<const int8_t>(at(12));
  uint16_t* ko = fake<uint16_t>(at(13));
  uint16_t* vo = fake<uint16_t>(at(14));
  const tq_rows r{4, 100, 8, 800, 8, 1};
  EXPECT_LAUNCH(tq_quantize_kv(&s, k, v, &r, sg, &p, &r, nullptr));
  EXPECT_LAUNCH(tq_dequantize_kv(&s, &p, &r, sg, ko, vo, &r, nullptr));
  EXPECT_LAUNCH(tq_dequantize_kv(&s, &p, &r, nullptr, ko, nullptr, &r, nullptr));
  EXPECT(tq_quantize_kv(&s, k, v, nullptr, sg, &p, &r, nullptr), TQ_E_NULL);
  EXPECT(tq_quantize_kv(&s, k, v, &r, sg, &p, nullptr, nullptr), TQ_E_NULL);
  EXPECT(tq_quantize_kv(&s, k, v, &r, sg, nullptr, &r, nullptr), TQ_E_NULL);
  EXPECT(tq_dequantize_kv(&s, &p, &r, sg, nullptr, nullptr, &r, nullptr), TQ_E_NULL);
  // counts and strides at the ends of their ranges
  const int64_t big[] = {INT64_MIN, -1, 0, 1, 1 << 16, (int64_t)1 << 31, INT32_MAX, INT64_MAX};
  for (int64_t a : big)
    for (int64_t b : big) {
      const tq_rows x{a, b, 3, 0, 0, 0};
      const tq_rows y{2, 3, 4, a, b, a};
      const bool neg = a < 0 || b < 0;
      const int64_t lim = (int64_t)1 << 31;
      const bool huge = !neg && (a >= lim || b >= lim || (__int128)a * b * 3 >= lim);
      const int32_t want_x = neg || huge ? TQ_E_SHAPE : (a == 0 || b == 0 ? TQ_OK : TQ_E_HIP);
      EXPECT(tq_quantize_kv(&s, k, v, &x, sg, &p, &x, nullptr), want_x);
      EXPECT(tq_dequantize_kv(&s, &p, &x, sg, ko, vo, &x, nullptr), want_x);
      EXPECT(tq_unrotate_rows(128, k, &x, sg, ko, &x, nullptr), want_x);
      EXPECT(tq_quantize_kv(&s, k, v, &y, sg, &p, &y, nullptr), neg ? TQ_E_SHAPE : TQ_E_HIP);
    }
  const tq_rows r2{4, 100, 9, 900, 9, 1};
  EXPECT(tq_quantize_kv(&s, k, v, &r, sg, &p, &r2, nullptr), TQ_E_SHAPE);
  EXPECT(tq_unrotate_rows(96, k, &r, sg, ko, &r, nullptr), TQ_E_HEAD_DIM);
  EXPECT(tq_unrotate_rows(128, k + 1, &r, sg, ko, &r, nullptr), TQ_E_ALIGN);
  EXPECT_LAUNCH(tq_unrotate_rows(512, k, &r, sg, ko, &r, nullptr));
  // every served scheme reaches its launch
  for (int d : {64, 128, 256, 512})
    for (int kb : {2, 4, 5, 8})
      for (int vb : {2, 3, 4, 5, 8}) {
        const tq_scheme t{d, kb, vb};
        EXPECT_LAUNCH(tq_quantize_kv(&t, k, v, &r, sg, &p, &r, nullptr));
        EXPECT_LAUNCH(tq_dequantize_kv(&t, &p, &r, sg, ko, vo, &r, nullptr));
      }
}

void cache_calls() {
  const tq_scheme s{128, 8, 3};
  const tq_planes c = planes_at(0);
  const uint16_t* k = fake<const uint16_t>(at(10));
  const int8_t* sg = fake<const int8_t>(at(12));
  const int32_t* pos = fake<const int32_t>(at(15));
  uint16_t* ko = fake<uint16_t>(at(13));
  EXPECT_LAUNCH(tq_append_kv(&s, k, k, 4, 1, 8, sg, &c, 8 * 512, 512, pos, 512, nullptr));
  EXPECT(tq_append_kv(&s, k, k, INT32_MAX, INT32_MAX, INT32_MAX, sg, &c, INT64_MAX, INT64_MAX, pos, INT32_MAX,
                      nullptr),
         TQ_E_SHAPE);
  EXPECT(tq_append_kv(&s, k, k, INT32_MAX, 1, 1, sg, &c, INT64_MAX, INT64_MAX, pos, INT32_MAX, nullptr),
         TQ_E_HIP);
  EXPECT(tq_append_kv(&s, k, k, INT32_MIN, 1, 1, sg, &c, 1, 1, pos, 1, nullptr), TQ_E_SHAPE);
  EXPECT_LAUNCH(tq_fetch_kv(&s, &c, 4, 8, 8 * 512, 512, 512, pos, 600, sg, 0, ko, ko + 8, nullptr));
  EXPECT_LAUNCH(tq_fetch_kv(&s, &c, 4, 8, 8 * 512, 512, 512, pos, 600, nullptr, 1, nullptr, ko, nullptr));
  EXPECT(tq_fetch_kv(&s, &c, INT32_MAX, INT32_MAX, INT64_MAX, INT64_MAX, INT32_MAX, pos, INT32_MAX, sg, 0, ko,
                     ko, nullptr),
         TQ_E_SHAPE);
  EXPECT(tq_fetch_kv(&s, &c, 4, 8, 8 * 512, 512, 512, pos, 600, nullptr, 0, ko, ko, nullptr), TQ_E_NULL);

  // growth: layouts, overlaps and the ends of the ranges
  const tq_planes d = planes_at(20);
  EXPECT_LAUNCH(tq_grow_kv(&s, 4, 8, &c, 8 * 512, 512, 512, &d, 8 * 768, 768, 768, nullptr));
  EXPECT_LAUNCH(tq_grow_kv(&s, 4, 8, &c, 8 * 512, 512, 512, &d, 8 * 300, 300, 300, nullptr));
  EXPECT_LAUNCH(tq_grow_kv(&s, 4, 8, &c, 512, 4 * 512, 512, &d, 768, 4 * 768, 768, nullptr));
  EXPECT(tq_grow_kv(&s, 4, 8, &c, 8 * 512, 512, 512, &d, 8 * 768, 767, 768, nullptr), TQ_E_SHAPE);
  EXPECT(tq_grow_kv(&s, 4, 8, &c, 8 * 512, 512, 512, &c, 8 * 768, 768, 768, nullptr), TQ_E_OVERLAP);
  EXPECT(tq_grow_kv(&s, 0, 8, &c, 0, 0, 512, &c, 0, 0, 768, nullptr), TQ_OK);
  EXPECT(tq_grow_kv(&s, 4, 8, &c, 8 * 512, 512, 512, &d, 8 * 768, 768, 0, nullptr), TQ_OK);
  const int64_t strides[] = {0, 1, 767, 768, (int64_t)1 << 40, INT64_MAX / 1024, INT64_MAX};
  for (int32_t B : {1, 2, INT32_MAX})
    for (int32_t H : {1, 3, INT32_MAX})
      for (int64_t ss : strides)
        for (int64_t hs : strides)
          for (int32_t cap : {0, 1, 768, INT32_MAX}) {
            const int32_t got = tq_grow_kv(&s, B, H, &c, ss, hs, cap, &d, ss, hs, cap, nullptr);
            ++g_checks;
            if (got != TQ_OK && got != TQ_E_SHAPE && got != TQ_E_OVERLAP && got != TQ_E_HIP) {
              std::fprintf(stderr, "tq_grow_kv(B=%d H=%d ss=%lld hs=%lld cap=%d) -> %d\n", B, H, (long long)ss,
                           (long long)hs, cap, got);
              ++g_fails;
            }
          }
}

void attention_calls() {
  const tq_scheme s{128, 8, 3};
  const tq_planes c = planes_at(0);
  const uint16_t* q = fake<const uint16_t>(at(10));
  const int32_t* ctx = fake<const int32_t>(at(15));
  const int8_t* sg = fake<const int8_t>(at(12));
  uint16_t* out = fake<uint16_t>(at(13));
  void* ws = fake<void>(at(16));
  const size_t need = tq_decode_attn_workspace_bytes(&s, 16, 32, 8, 32768);
  EXPECT(need > 0, 1);
  EXPECT_LAUNCH(tq_decode_attn_quant(&s, q, 16, 32, 8, &c, 8 * 32768, 32768, ctx, 32768, 0.088f, sg, out, ws, need,
                                     nullptr));
  EXPECT(tq_decode_attn_quant(&s, q, 16, 32, 8, &c, 8 * 32768, 32768, ctx, 32768, 0.088f, sg, out, ws, need - 1,
                              nullptr),
         TQ_E_WORKSPACE);
  EXPECT(tq_decode_attn_quant(&s, q, 16, 30, 8, &c, 8 * 32768, 32768, ctx, 32768, 0.088f, sg, out, ws, need,
                              nullptr),
         TQ_E_SHAPE);
  for (int d : {64, 128, 256, 512})
    for (int kb : {2, 4, 5, 8})
      for (int vb : {2, 3, 4, 5, 8})
        for (int M : {1, 4, 9})
          for (int rep : {1, 4, 6}) {
            const tq_scheme t{d, kb, vb};
            const size_t w = tq_attn_quant_workspace_bytes(&t, 3, M, 2 * rep, 2, 1000);
            EXPECT(w > 0, 1);
            EXPECT_LAUNCH(tq_attn_quant(&t, q, 3, M, 2 * rep, 2, &c, 2 * 1000, 1000, ctx, 1000, 0.1f, sg, out, ws,
                                        w, nullptr));
          }
  const int32_t ends[] = {INT32_MIN, -1, 0, 1, 7, 1 << 16, INT32_MAX};
  for (int32_t B : ends)
    for (int32_t M : ends)
      for (int32_t Hq : {1, 8, INT32_MAX})
        for (int32_t Hkv : {1, 8, INT32_MAX})
          for (int32_t N : ends) {
            const size_t w = tq_attn_quant_workspace_bytes(&s, B, M, Hq, Hkv, N);
            const bool bad =
                B < 0 || M < 1 || Hq % Hkv != 0 || N < 1 || (__int128)B * M * Hq >= ((__int128)1 << 30);
            if (bad) EXPECT(w, 0);
            const int32_t got = tq_attn_quant(&s, q, B, M, Hq, Hkv, &c, INT64_MAX, INT64_MAX, ctx, N, 0.1f, sg, out,
                                              ws, w, nullptr);
            EXPECT(got, bad ? TQ_E_SHAPE : (B == 0 ? TQ_OK : TQ_E_HIP));
          }
  // the allocation-free form refuses before it looks for its scratch
  EXPECT(tq_attn_quant_noalloc(&s, q, 64, 8, 64, 8, &c, 8 * 32768, 32768, ctx, 32768, 0.1f, sg, out, nullptr),
         TQ_E_WORKSPACE);
  EXPECT(tq_attn_quant_noalloc(&s, q, 2, 1, 8, 2, &c, 2 * 100, 100, ctx, 100, 0.1f, sg, out, nullptr), TQ_E_HIP);
}

void dense_calls() {
  EXPECT(tq_dense_check_scheme(nullptr), TQ_E_NULL);
  for (int d : {INT_MIN, 0, 32, 64, 128, 256, 512})
    for (int b : {INT_MIN, 0, 1, 2, 3, 4, 5, INT_MAX})
      for (int qjl : {-1, 0, 1, 2}) {
        const tq_dense_scheme s{d, b, qjl};
        const bool dok = d == 64 || d == 128 || d == 256;
        const bool bok = b >= 1 && b <= 4 && (qjl == 0 || qjl == 1);
        const int32_t want = !dok ? TQ_E_HEAD_DIM : !bok ? TQ_E_BITS : (qjl && d > 128) ? TQ_E_HEAD_DIM : TQ_OK;
        EXPECT(tq_dense_check_scheme(&s), want);
        for (int p = -1; p < 5; ++p) {
          const int64_t rb = tq_dense_plane_row_bytes(&s, p);
          if (want != TQ_OK)
            EXPECT(rb, want);
          else if (p < 0 || p > 3)
            EXPECT(rb, TQ_E_PLANE);
          else
            EXPECT(rb >= 0, 1);
        }
        if (want == TQ_OK) {
          const tq_dense_planes pl{fake<void>(at(0)), fake<float>(at(1)), fake<void>(at(2)), fake<float>(at(3))};
          const tq_rows r{1, 1000, 1, 1000, 1, 1};
          const uint16_t* x = fake<const uint16_t>(at(10));
          const uint16_t* m = fake<const uint16_t>(at(11));
          EXPECT_LAUNCH(tq_dense_quantize(&s, x, &r, m, m, &pl, &r, nullptr));
          EXPECT_LAUNCH(tq_dense_dequantize(&s, &pl, &r, m, m, fake<uint16_t>(at(12)), &r, nullptr));
          EXPECT(tq_dense_quantize(&s, x, &r, m, qjl ? nullptr : m, &pl, &r, nullptr), qjl ? TQ_E_NULL : TQ_E_HIP);
          const tq_rows huge{INT64_MAX, INT64_MAX, INT64_MAX, 1, 1, 1};
          EXPECT(tq_dense_quantize(&s, x, &huge, m, m, &pl, &huge, nullptr), TQ_E_SHAPE);
        }
      }
}

}  // namespace

int main() {
  // The fake addresses would reach real launches where a GPU is present.
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) == hipSuccess && n_dev > 0) {
    std::printf("abi host checks: a GPU is present, not run\n");
    return 77;
  }
  schemes_and_helpers();
  codec_calls();
  cache_calls();
  attention_calls();
  dense_calls();
  std::printf("abi host checks: %d checks, %d failures\n", g_checks, g_fails);
  return g_fails ? 1 : 0;
}
