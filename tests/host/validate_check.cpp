// Host-only check of the C ABI's argument validation (csrc/validate.h),
// built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitize.py.  Every LTXA_E_* path of every check is
// driven, and the 64-bit overflow guards are pushed to their limits: a
// signed overflow or an out-of-bounds read of a host array (max_pos, opts)
// aborts the program.  Device pointers are never dereferenced by the checks,
// so plain integers stand in for them; host arrays are heap blocks of exactly
// the size the ABI documents, so that ASan sees any read past them.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>
#include <vector>

#include "validate.h"

namespace {

int g_cases = 0, g_failures = 0;

void expect(int got, int want, const char* what, int line) {
  ++g_cases;
  if (got != want) {
    std::printf("FAIL line %d: %s returned %d, expected %d\n", line, what, got, want);
    ++g_failures;
  }
}
#define EXPECT(expr, code) expect((expr), (code), #expr, __LINE__)

const void* dev(uintptr_t a) { return reinterpret_cast<const void*>(a); }
const int32_t* devpos(uintptr_t a) { return reinterpret_cast<const int32_t*>(a); }
float* devf(uintptr_t a) { return reinterpret_cast<float*>(a); }

// Distinct, 16-byte aligned stand-ins for device buffers, far apart.
constexpr uintptr_t kA = uintptr_t(1) << 40, kB = uintptr_t(2) << 40, kC = uintptr_t(3) << 40,
                    kD = uintptr_t(4) << 40, kE = uintptr_t(5) << 40, kF = uintptr_t(6) << 40;
constexpr double kNan = std::numeric_limits<double>::quiet_NaN();
constexpr double kInf = std::numeric_limits<double>::infinity();

void perm_checks() {
  using ltxa::check_perm;
  ltxa::PermPlan plan{};
  EXPECT(check_perm(dev(kA), dev(kB), 1, 232, 4, 64, 4, 2, &plan), LTXA_OK);
  EXPECT(int(plan.bytes == 232 * 4 * 64 * 2 && plan.rows == 232 && plan.chunk == 128), 1);
  EXPECT(check_perm(nullptr, dev(kB), 1, 232, 4, 64, 4, 2, &plan), LTXA_E_NULL);
  EXPECT(check_perm(dev(kA), nullptr, 1, 232, 4, 64, 4, 2, &plan), LTXA_E_NULL);
  EXPECT(check_perm(dev(kA), dev(kB), 0, 232, 4, 64, 4, 2, &plan), LTXA_E_SHAPE);
  EXPECT(check_perm(dev(kA), dev(kB), 1, 0, 4, 64, 4, 2, &plan), LTXA_E_SHAPE);
  EXPECT(check_perm(dev(kA), dev(kB), 1, 232, 0, 64, 4, 2, &plan), LTXA_E_SHAPE);
  EXPECT(check_perm(dev(kA), dev(kB), 1, 232, 4, 0, 4, 2, &plan), LTXA_E_SHAPE);
  EXPECT(check_perm(dev(kA), dev(kB), 1, 232, 4, 64, 0, 2, &plan), LTXA_E_SHAPE);
  EXPECT(check_perm(dev(kA), dev(kB), 1, 232, 4, 64, 4, 3, &plan), LTXA_E_SHAPE);
  EXPECT(check_perm(dev(kA), dev(kB), 1, 232, 2, 64, 4, 2, &plan), LTXA_E_DIVISIBILITY);  // heads % P
  EXPECT(check_perm(dev(kA), dev(kB), 1, 231, 4, 64, 4, 2, &plan), LTXA_E_DIVISIBILITY);  // tokens % P
  EXPECT(check_perm(dev(kA), dev(kB), INT64_MAX, INT64_MAX - 3, 4, 64, 4, 8, &plan), LTXA_E_RANGE);
  EXPECT(check_perm(dev(kA), dev(kB), 1, int64_t(1) << 30, 32, 128, 8, 2, &plan), LTXA_E_RANGE);  // 2^43 B
  EXPECT(check_perm(dev(kA), dev(kB), 1, 65536, 65536, 1, 65536, 1, &plan), LTXA_E_RANGE);       // P > 65535
  EXPECT(check_perm(dev(kA), dev(kA + 16), 1, 232, 4, 64, 4, 2, &plan), LTXA_E_ALIAS);
  EXPECT(check_perm(dev(kA), dev(kA + 232 * 4 * 64 * 2), 1, 232, 4, 64, 4, 2, &plan), LTXA_OK);  // adjacent
}

void rope_checks() {
  using ltxa::check_rope;
#ifdef LTXA_CHECK_PLANT_SHORT_ARRAY
  // Planted caller mistake: a 3-axis call given only 2 max_pos values.  The
  // sanitizer build must stop at the read past the array.
  std::vector<double> mp3 = {3.0, 7.0}, mp1 = {1000.0};
#else
  std::vector<double> mp3 = {3.0, 7.0, 11.0}, mp1 = {1000.0};
#endif
  const double* m3 = mp3.data();
  const double* m1 = mp1.data();
  EXPECT(check_rope(dev(kA), devpos(kC), 232, 3, m3, dev(kB), devpos(kC), 232, 3, m3, 1, 2, 64, 1e4), LTXA_OK);
  EXPECT(check_rope(dev(kA), devpos(kC), 232, 3, m3, nullptr, nullptr, 0, 0, nullptr, 1, 2, 64, 1e4), LTXA_OK);
  EXPECT(check_rope(nullptr, nullptr, 0, 0, nullptr, dev(kB), devpos(kD), 1024, 1, m1, 1, 2, 64, 1e4), LTXA_OK);
  EXPECT(check_rope(nullptr, nullptr, 0, 0, nullptr, nullptr, nullptr, 0, 0, nullptr, 1, 2, 64, 1e4),
         LTXA_E_NULL);
  EXPECT(check_rope(dev(kA), nullptr, 232, 3, m3, nullptr, nullptr, 0, 0, nullptr, 1, 2, 64, 1e4), LTXA_E_NULL);
  EXPECT(check_rope(dev(kA), devpos(kC), 232, 3, nullptr, nullptr, nullptr, 0, 0, nullptr, 1, 2, 64, 1e4),
         LTXA_E_NULL);
  auto q_only = [&](int64_t n, int32_t axes, const double* mp, int64_t batch, int32_t heads, int32_t hd,
                    double theta, uintptr_t q = kA, uintptr_t pos = kC) {
    return check_rope(dev(q), devpos(pos), n, axes, mp, nullptr, nullptr, 0, 0, nullptr, batch, heads, hd, theta);
  };
  EXPECT(q_only(232, 3, m3, 0, 2, 64, 1e4), LTXA_E_SHAPE);
  EXPECT(q_only(232, 3, m3, 1, 0, 64, 1e4), LTXA_E_SHAPE);
  EXPECT(q_only(232, 3, m3, 1, 2, 63, 1e4), LTXA_E_SHAPE);   // odd head_dim
  EXPECT(q_only(232, 3, m3, 1, 2, 258, 1e4), LTXA_E_SHAPE);  // above 256
  EXPECT(q_only(232, 3, m3, 1, 2, 0, 1e4), LTXA_E_SHAPE);
  EXPECT(q_only(232, 3, m3, 1, 2, 64, 0.0), LTXA_E_SHAPE);
  EXPECT(q_only(232, 3, m3, 1, 2, 64, -1.0), LTXA_E_SHAPE);
  EXPECT(q_only(232, 3, m3, 1, 2, 64, kInf), LTXA_E_SHAPE);
  EXPECT(q_only(232, 3, m3, 1, 2, 64, kNan), LTXA_E_SHAPE);
  EXPECT(q_only(232, 3, m3, 1, 2, 6, 1e4), LTXA_E_ALIGN);    // 12-byte rows
  EXPECT(q_only(0, 3, m3, 1, 2, 64, 1e4), LTXA_E_SHAPE);
  EXPECT(q_only(232, 0, m3, 1, 2, 64, 1e4), LTXA_E_SHAPE);
  EXPECT(q_only(232, 4, m3, 1, 2, 64, 1e4), LTXA_E_SHAPE);
  std::vector<double> bad = {3.0, 0.0, 11.0};
  EXPECT(q_only(232, 3, bad.data(), 1, 2, 64, 1e4), LTXA_E_SHAPE);
  bad[1] = kNan;
  EXPECT(q_only(232, 3, bad.data(), 1, 2, 64, 1e4), LTXA_E_SHAPE);
  bad[1] = -kInf;
  EXPECT(q_only(232, 3, bad.data(), 1, 2, 64, 1e4), LTXA_E_SHAPE);
  EXPECT(q_only(232, 3, m3, 1, 2, 64, 1e4, kA + 8), LTXA_E_ALIGN);
  EXPECT(q_only(232, 3, m3, 1, 2, 64, 1e4, kA, kC + 4), LTXA_E_ALIGN);
  EXPECT(q_only(INT64_MAX, 3, m3, 1, 2, 64, 1e4), LTXA_E_RANGE);
  EXPECT(q_only(int64_t(1) << 41, 1, m1, 1, 1, 16, 1e4), LTXA_E_RANGE);   // beyond the grid
  EXPECT(check_rope(dev(kA), devpos(kC), 232, 3, m3, dev(kA + 64), devpos(kC), 232, 3, m3, 1, 2, 64, 1e4),
         LTXA_E_ALIAS);
}

void attn_checks() {
  using ltxa::check_attn;
  const float s = 0.125f;
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), devf(kE), 1, 4, 128, 32768, 32768, 32768, s), LTXA_OK);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, 8, 4, 64, 24576, 1024, 1000, s), LTXA_OK);
  EXPECT(check_attn(nullptr, dev(kB), dev(kC), dev(kD), nullptr, 1, 4, 128, 64, 64, 64, s), LTXA_E_NULL);
  EXPECT(check_attn(dev(kA), nullptr, dev(kC), dev(kD), nullptr, 1, 4, 128, 64, 64, 64, s), LTXA_E_NULL);
  EXPECT(check_attn(dev(kA), dev(kB), nullptr, dev(kD), nullptr, 1, 4, 128, 64, 64, 64, s), LTXA_E_NULL);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), nullptr, nullptr, 1, 4, 128, 64, 64, 64, s), LTXA_E_NULL);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, 0, 4, 128, 64, 64, 64, s), LTXA_E_SHAPE);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, 1, 0, 128, 64, 64, 64, s), LTXA_E_SHAPE);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, 1, 4, 128, 0, 64, 64, s), LTXA_E_SHAPE);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, 1, 4, 128, 64, 0, 1, s), LTXA_E_SHAPE);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, 1, 4, 96, 64, 64, 64, s), LTXA_E_SHAPE);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, 1, 4, 128, 64, 64, 0, s), LTXA_E_SHAPE);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, 1, 4, 128, 64, 64, 65, s), LTXA_E_SHAPE);
  for (float bad : {0.0f, -1.0f, std::numeric_limits<float>::infinity(), std::numeric_limits<float>::quiet_NaN()})
    EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, 1, 4, 128, 64, 64, 64, bad), LTXA_E_SHAPE);
  EXPECT(check_attn(dev(kA + 2), dev(kB), dev(kC), dev(kD), nullptr, 1, 4, 128, 64, 64, 64, s), LTXA_E_ALIGN);
  EXPECT(check_attn(dev(kA), dev(kB + 8), dev(kC), dev(kD), nullptr, 1, 4, 128, 64, 64, 64, s), LTXA_E_ALIGN);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC + 4), dev(kD), nullptr, 1, 4, 128, 64, 64, 64, s), LTXA_E_ALIGN);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD + 2), nullptr, 1, 4, 128, 64, 64, 64, s), LTXA_E_ALIGN);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), devf(kE + 4), 1, 4, 128, 64, 64, 64, s), LTXA_E_ALIGN);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, INT64_MAX, 4, 128, INT64_MAX, 64, 64, s),
         LTXA_E_RANGE);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, 1, 1 << 20, 128, 64, 64, 64, s), LTXA_E_RANGE);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, 1 << 20, 64, 64, 1 << 20, 64, 64, s),
         LTXA_E_RANGE);  // grid beyond 2^31 workgroups
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kA + 256), nullptr, 1, 4, 128, 64, 64, 64, s), LTXA_E_ALIAS);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kB), nullptr, 1, 4, 128, 64, 64, 64, s), LTXA_E_ALIAS);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kC + 16), nullptr, 1, 4, 128, 64, 64, 64, s), LTXA_E_ALIAS);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), devf(kD + 16), 1, 4, 128, 64, 64, 64, s), LTXA_E_ALIAS);
  EXPECT(check_attn(dev(kA), dev(kB), dev(kC), dev(kD), devf(kA), 1, 4, 128, 64, 64, 64, s), LTXA_E_ALIAS);
  // q, k and v may share memory (they are only read).
  EXPECT(check_attn(dev(kA), dev(kA), dev(kA), dev(kD), devf(kE), 1, 4, 128, 64, 64, 64, s), LTXA_OK);

  using ltxa::check_attn_unpack;
  EXPECT(check_attn_unpack(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, 1, 32, 128, 32768, 32768, 32761, s, 8),
         LTXA_OK);
  EXPECT(check_attn_unpack(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, 1, 32, 128, 64, 64, 64, s, 0),
         LTXA_E_SHAPE);
  EXPECT(check_attn_unpack(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, 1, 30, 128, 64, 64, 64, s, 8),
         LTXA_E_DIVISIBILITY);
  EXPECT(check_attn_unpack(dev(kA), dev(kB), dev(kC), dev(kD), nullptr, INT64_MAX, 32, 128, 64, 64, 64, s, 8),
         LTXA_E_RANGE);
  EXPECT(check_attn_unpack(nullptr, dev(kB), dev(kC), dev(kD), nullptr, 1, 32, 128, 64, 64, 64, s, 8),
         LTXA_E_NULL);
}

void pack_rope_checks() {
  using ltxa::check_pack_rope;
  std::vector<double> mp3 = {16.0, 32.0, 64.0};
  const double* m = mp3.data();
  EXPECT(check_pack_rope(dev(kA), dev(kB), devpos(kC), 32768, 3, m, 1, 32, 128, 8, 1e4), LTXA_OK);
  EXPECT(check_pack_rope(nullptr, dev(kB), devpos(kC), 32768, 3, m, 1, 32, 128, 8, 1e4), LTXA_E_NULL);
  EXPECT(check_pack_rope(dev(kA), nullptr, devpos(kC), 32768, 3, m, 1, 32, 128, 8, 1e4), LTXA_E_NULL);
  EXPECT(check_pack_rope(dev(kA), dev(kB), nullptr, 32768, 3, m, 1, 32, 128, 8, 1e4), LTXA_E_NULL);
  EXPECT(check_pack_rope(dev(kA), dev(kB), devpos(kC), 32768, 3, m, 1, 32, 128, 0, 1e4), LTXA_E_SHAPE);
  EXPECT(check_pack_rope(dev(kA), dev(kB), devpos(kC), 32768, 3, m, 1, 32, 127, 8, 1e4), LTXA_E_SHAPE);
  EXPECT(check_pack_rope(dev(kA), dev(kB), devpos(kC), 32768, 3, m, 1, 32, 128, 8, kNan), LTXA_E_SHAPE);
  EXPECT(check_pack_rope(dev(kA), dev(kB), devpos(kC), 32768, 3, m, 1, 32, 6, 8, 1e4), LTXA_E_ALIGN);
  EXPECT(check_pack_rope(dev(kA), dev(kB + 2), devpos(kC), 32768, 3, m, 1, 32, 128, 8, 1e4), LTXA_E_ALIGN);
  EXPECT(check_pack_rope(dev(kA), dev(kB), devpos(kC), 32768, 3, m, 1, 30, 128, 8, 1e4), LTXA_E_DIVISIBILITY);
  EXPECT(check_pack_rope(dev(kA), dev(kB), devpos(kC), 32761, 3, m, 1, 32, 128, 8, 1e4), LTXA_E_DIVISIBILITY);
  EXPECT(check_pack_rope(dev(kA), dev(kB), devpos(kC), int64_t(1) << 42, 3, m, 1, 32, 128, 8, 1e4),
         LTXA_E_RANGE);
  EXPECT(check_pack_rope(dev(kA), dev(kA + 1024), devpos(kC), 32768, 3, m, 1, 32, 128, 8, 1e4), LTXA_E_ALIAS);
  // Output scale of the scaled rotary pack.
  EXPECT(ltxa::check_out_scale(0.12752f), LTXA_OK);
  EXPECT(ltxa::check_out_scale(1.0f), LTXA_OK);
  EXPECT(ltxa::check_out_scale(0.0f), LTXA_E_SHAPE);
  EXPECT(ltxa::check_out_scale(-0.5f), LTXA_E_SHAPE);
  EXPECT(ltxa::check_out_scale(std::numeric_limits<float>::infinity()), LTXA_E_SHAPE);
  EXPECT(ltxa::check_out_scale(std::numeric_limits<float>::quiet_NaN()), LTXA_E_SHAPE);
  EXPECT(ltxa::check_out_scale(std::numeric_limits<float>::denorm_min()), LTXA_OK);
}

void rope_opts_checks() {
  using ltxa::check_rope_ex;
  std::vector<double> mp1 = {1024.0};
  const double* m = mp1.data();
  auto opts = [](int32_t type, int32_t grid, int32_t off, int32_t f64, int32_t mid, float scale) {
    ltxa_rope_opts* o = new ltxa_rope_opts{type, grid, off, f64, mid, scale};
    return o;
  };
  auto run = [&](const ltxa_rope_opts* o, int32_t heads = 32, int32_t hd = 128) {
    const int rc = check_rope_ex(dev(kA), devpos(kC), 1024, 1, m, 2, heads, hd, 1e4, o);
    delete o;
    return rc;
  };
  EXPECT(check_rope_ex(dev(kA), devpos(kC), 1024, 1, m, 2, 32, 128, 1e4, nullptr), LTXA_OK);
  EXPECT(check_rope_ex(nullptr, devpos(kC), 1024, 1, m, 2, 32, 128, 1e4, nullptr), LTXA_E_NULL);
  // Q and K in one launch: k present, aligned, disjoint from q and the
  // positions; k_scale 0 or finite and > 0.
  auto qk = [&](uintptr_t k, float ks) {
    return ltxa::check_rope_qk_ex(dev(kA), dev(k), devpos(kC), 1024, 1, m, 2, 32, 128, 1e4, nullptr, ks);
  };
  EXPECT(qk(kB, 0.0f), LTXA_OK);
  EXPECT(qk(kB, 0.5f), LTXA_OK);
  EXPECT(ltxa::check_rope_qk_ex(dev(kA), nullptr, devpos(kC), 1024, 1, m, 2, 32, 128, 1e4, nullptr, 0.0f),
         LTXA_E_NULL);
  EXPECT(qk(kB, -0.5f), LTXA_E_SHAPE);
  EXPECT(qk(kB, std::numeric_limits<float>::infinity()), LTXA_E_SHAPE);
  EXPECT(qk(kB + 8, 0.0f), LTXA_E_ALIGN);
  EXPECT(qk(kA + 4096, 0.0f), LTXA_E_ALIAS);
  EXPECT(qk(kC, 0.0f), LTXA_E_ALIAS);
  EXPECT(run(opts(0, 32, 0, 0, 0, 0)), LTXA_OK);
  EXPECT(run(opts(1, 32, 0, 1, 1, 0)), LTXA_OK);
  EXPECT(run(opts(2, 0, 0, 0, 0, 0)), LTXA_E_SHAPE);
  EXPECT(run(opts(0, 0, 0, 2, 0, 0)), LTXA_E_SHAPE);
  EXPECT(run(opts(0, 0, 0, 0, 2, 0)), LTXA_E_SHAPE);
  EXPECT(run(opts(0, 0, 0, 0, 0, 0.18033688f)), LTXA_OK);   // out_scale = log2(e) / 8
  EXPECT(run(opts(0, 0, 0, 0, 0, -1.0f)), LTXA_E_SHAPE);
  EXPECT(run(opts(0, 0, 0, 0, 0, std::numeric_limits<float>::infinity())), LTXA_E_SHAPE);
  EXPECT(run(opts(0, 0, 0, 0, 0, std::numeric_limits<float>::quiet_NaN())), LTXA_E_SHAPE);
  EXPECT(run(opts(0, -1, 0, 0, 0, 0)), LTXA_E_SHAPE);
  EXPECT(run(opts(0, 32, -1, 0, 0, 0)), LTXA_E_SHAPE);
  EXPECT(run(opts(0, 31, 0, 0, 0, 0)), LTXA_E_SHAPE);        // 32 heads do not fit in 31
  EXPECT(run(opts(0, 40, 9, 0, 0, 0)), LTXA_E_SHAPE);        // offset 9 + 32 heads > 40
  EXPECT(run(opts(0, 70000, 0, 0, 0, 0), 70000), LTXA_E_RANGE);  // heads beyond the grid's y limit
  EXPECT(run(opts(1, 0, 0, 0, 0, 0), 32, 40), LTXA_E_ALIGN);  // split needs head_dim % 16 == 0
}

void rope_table_checks() {
  using ltxa::check_pack_rope_table;
  using ltxa::check_rope_angles;
  std::vector<double> mp3 = {16.0, 32.0, 64.0};
  const double* m = mp3.data();
  auto angles = [&](const ltxa_rope_opts* o, int64_t n = 32768, int32_t axes = 3, int32_t hd = 128,
                    uintptr_t pos = kC, uintptr_t table = kD) {
    return check_rope_angles(devpos(pos), n, axes, m, hd, 1e4, o, devf(table));
  };
  EXPECT(angles(nullptr), LTXA_OK);
  EXPECT(check_rope_angles(nullptr, 32768, 3, m, 128, 1e4, nullptr, devf(kD)), LTXA_E_NULL);
  EXPECT(check_rope_angles(devpos(kC), 32768, 3, nullptr, 128, 1e4, nullptr, devf(kD)), LTXA_E_NULL);
  EXPECT(check_rope_angles(devpos(kC), 32768, 3, m, 128, 1e4, nullptr, nullptr), LTXA_E_NULL);
  EXPECT(angles(nullptr, 0), LTXA_E_SHAPE);
  EXPECT(angles(nullptr, 32768, 4), LTXA_E_SHAPE);
  EXPECT(angles(nullptr, 32768, 3, 127), LTXA_E_SHAPE);
  EXPECT(check_rope_angles(devpos(kC), 32768, 3, m, 128, kInf, nullptr, devf(kD)), LTXA_E_SHAPE);
  EXPECT(angles(nullptr, 32768, 3, 6), LTXA_E_ALIGN);
  EXPECT(angles(nullptr, 32768, 3, 128, kC, kD + 4), LTXA_E_ALIGN);
  EXPECT(angles(nullptr, 32768, 3, 128, kC + 4), LTXA_E_ALIGN);
  {
    ltxa_rope_opts o1{0, 0, 0, 1, 1, 0.0f}, o2{1, 0, 0, 0, 0, 0.0f}, o3{0, 4, 0, 0, 0, 0.0f},
        o4{0, 0, 0, 0, 0, 0.5f}, o5{3, 0, 0, 0, 0, 0.0f};
    EXPECT(angles(&o1), LTXA_OK);  // fp64 angles, cell middles
    EXPECT(angles(&o2), LTXA_OK);  // split pairing: same angles
    EXPECT(angles(&o3), LTXA_E_SHAPE);
    EXPECT(angles(&o4), LTXA_E_SHAPE);
    EXPECT(angles(&o5), LTXA_E_SHAPE);
  }
  EXPECT(angles(nullptr, 32768, 3, 128, kC, kC + 64), LTXA_E_ALIAS);
  EXPECT(angles(nullptr, int64_t(1) << 33), LTXA_E_RANGE);
  EXPECT(angles(nullptr, INT64_MAX / 2), LTXA_E_RANGE);

  auto pack = [&](int64_t n, int64_t b, int32_t h, int32_t hd, int32_t p, int32_t type, float sc,
                  uintptr_t src = kA, uintptr_t dst = kB, uintptr_t table = kD) {
    return check_pack_rope_table(dev(src), dev(dst), devf(table), n, b, h, hd, p, type, sc);
  };
  EXPECT(pack(32768, 1, 32, 128, 8, 0, 0.0f), LTXA_OK);
  EXPECT(pack(32768, 1, 32, 128, 8, 1, 0.18033688f), LTXA_OK);
  EXPECT(check_pack_rope_table(nullptr, dev(kB), devf(kD), 32768, 1, 32, 128, 8, 0, 0.0f), LTXA_E_NULL);
  EXPECT(check_pack_rope_table(dev(kA), nullptr, devf(kD), 32768, 1, 32, 128, 8, 0, 0.0f), LTXA_E_NULL);
  EXPECT(check_pack_rope_table(dev(kA), dev(kB), nullptr, 32768, 1, 32, 128, 8, 0, 0.0f), LTXA_E_NULL);
  EXPECT(pack(0, 1, 32, 128, 8, 0, 0.0f), LTXA_E_SHAPE);
  EXPECT(pack(32768, 0, 32, 128, 8, 0, 0.0f), LTXA_E_SHAPE);
  EXPECT(pack(32768, 1, 32, 130, 8, 0, 0.0f), LTXA_E_ALIGN);
  EXPECT(pack(32768, 1, 32, 258, 8, 0, 0.0f), LTXA_E_SHAPE);
  EXPECT(pack(32768, 1, 32, 128, 8, 2, 0.0f), LTXA_E_SHAPE);
  EXPECT(pack(32768, 1, 32, 128, 8, 0, -2.0f), LTXA_E_SHAPE);
  EXPECT(pack(32768, 1, 32, 128, 8, 0, std::numeric_limits<float>::quiet_NaN()), LTXA_E_SHAPE);
  EXPECT(pack(32768, 1, 32, 40, 8, 1, 0.0f), LTXA_E_ALIGN);  // split: head_dim % 16
  EXPECT(pack(32768, 1, 32, 128, 8, 0, 0.0f, kA + 8), LTXA_E_ALIGN);
  EXPECT(pack(32768, 1, 32, 128, 8, 0, 0.0f, kA, kB, kD + 8), LTXA_E_ALIGN);
  EXPECT(pack(32768, 1, 30, 128, 8, 0, 0.0f), LTXA_E_DIVISIBILITY);
  EXPECT(pack(32761, 1, 32, 128, 8, 0, 0.0f), LTXA_E_DIVISIBILITY);
  EXPECT(pack(32768, 1, 32, 128, 8, 0, 0.0f, kA, kA + 4096), LTXA_E_ALIAS);
  EXPECT(pack(32768, 1, 32, 128, 8, 0, 0.0f, kA, kB, kB + 4096), LTXA_E_ALIAS);
  EXPECT(pack(int64_t(1) << 40, int64_t(1) << 13, 32, 128, 8, 0, 0.0f), LTXA_E_RANGE);
  EXPECT(pack(int64_t(1) << 36, 1, 8, 128, 8, 0, 0.0f), LTXA_E_RANGE);  // grid above 2^31 workgroups

  // Q and K in one launch: each pair as above, and no destination on the
  // other pair's tensors (256 MiB per tensor at these sizes).
  auto qk = [&](uintptr_t q, uintptr_t qd, float qs, uintptr_t k, uintptr_t kd, float ks, int32_t type = 0,
                int64_t n = 32768) {
    return ltxa::check_pack_rope_qk_table(dev(q), dev(qd), qs, dev(k), dev(kd), ks, devf(kD), n, 1, 32, 128, 8,
                                          type);
  };
  EXPECT(qk(kA, kB, 0.18033688f, kC, kE, 0.0f), LTXA_OK);
  EXPECT(qk(kA, kB, 0.0f, kA, kE, 0.0f, 1), LTXA_OK);  // the sources may overlap
  EXPECT(qk(kA, kB, 0.0f, 0, kE, 0.0f), LTXA_E_NULL);
  EXPECT(qk(kA, kB, 0.0f, kC, 0, 0.0f), LTXA_E_NULL);
  EXPECT(qk(kA, kB, 0.0f, kC, kE, -1.0f), LTXA_E_SHAPE);
  EXPECT(qk(kA, kB, 0.0f, kC + 8, kE, 0.0f), LTXA_E_ALIGN);
  EXPECT(qk(kA, kB, 0.0f, kC, kE, 0.0f, 0, 32761), LTXA_E_DIVISIBILITY);
  EXPECT(qk(kA, kB, 0.0f, kB + 4096, kE, 0.0f), LTXA_E_ALIAS);  // q_dst on k
  EXPECT(qk(kA, kB, 0.0f, kC, kB + 4096, 0.0f), LTXA_E_ALIAS);  // the destinations overlap
  EXPECT(qk(kA, kB, 0.0f, kC, kA + 4096, 0.0f), LTXA_E_ALIAS);  // k_dst on q
  EXPECT(qk(kA, kB, 0.0f, kC, kD + 4096, 0.0f), LTXA_E_ALIAS);  // k_dst on the table
  // 2^31 tokens: a grid of 2^30 workgroups per tensor is valid for one
  // tensor, not for two (16 TiB tensors, so the addresses are 32 TiB apart).
  constexpr uintptr_t kT = uintptr_t(1) << 45;
  EXPECT(pack(int64_t(1) << 31, 1, 32, 128, 8, 0, 0.0f, kT, 2 * kT), LTXA_OK);
  EXPECT(qk(kT, 2 * kT, 0.0f, 3 * kT, 4 * kT, 0.0f, 0, int64_t(1) << 31), LTXA_E_RANGE);
}

void mul_checks() {
  EXPECT(int(ltxa::mul_capped(INT64_MAX, INT64_MAX)), -1);
  EXPECT(int(ltxa::mul_capped(-1, 5)), -1);
  EXPECT(int(ltxa::mul_capped(0, INT64_MAX)), 0);
  EXPECT(int(ltxa::mul_capped(ltxa::kMaxBytes, 1) == ltxa::kMaxBytes), 1);
  EXPECT(int(ltxa::mul_capped(ltxa::kMaxBytes, 2)), -1);
  EXPECT(int(ltxa::mul4_capped(1 << 20, 1 << 20, 1 << 20, 1 << 20)), -1);
  EXPECT(int(ltxa::mul4_capped(2, 3, 5, 7)), 210);
}

}  // namespace

int main() {
  perm_checks();
  rope_checks();
  attn_checks();
  pack_rope_checks();
  rope_opts_checks();
  rope_table_checks();
  mul_checks();
  std::printf("validate_check: %d cases, %d failures\n", g_cases, g_failures);
  return g_failures == 0 ? 0 : 1;
}
