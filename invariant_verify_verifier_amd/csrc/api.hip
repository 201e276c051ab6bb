// Error state, version and host-side tables of libbiverify.
#include <cmath>

#include "biv_internal.h"

namespace biv {

static thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

}  // namespace biv

extern "C" int biv_abi_version(void) { return 2; }

extern "C" const char* biv_last_error(void) { return biv::g_last_error; }

// Rotate-half RoPE angles in fp64, rounded once to fp32.
extern "C" biv_status biv_rope_table(float* cos_sin, int max_pos, int D, double theta) {
  BIV_REQUIRE(cos_sin != nullptr, "biv_rope_table: cos_sin is NULL");
  BIV_REQUIRE(max_pos >= 1 && D >= 2 && D % 2 == 0, "biv_rope_table: bad max_pos=%d or D=%d", max_pos, D);
  BIV_REQUIRE(theta > 0.0, "biv_rope_table: theta must be > 0");
  const int half = D / 2;
  for (int i = 0; i < half; ++i) {
    const double inv = std::pow(theta, -2.0 * i / D);
    for (int p = 0; p < max_pos; ++p) {
      const double a = p * inv;
      cos_sin[((int64_t)p * half + i) * 2 + 0] = (float)std::cos(a);
      cos_sin[((int64_t)p * half + i) * 2 + 1] = (float)std::sin(a);
    }
  }
  return BIV_OK;
}
