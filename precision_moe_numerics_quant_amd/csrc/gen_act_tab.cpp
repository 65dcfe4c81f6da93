// Build-time generator of the SiLU / SiLU' tables compiled into libmoe4.
//
// For every bf16 value u with |u| in [2**-8, 2**8) (sign x 16 binades x 128
// mantissas = 4096 entries, indexed as act_index() in act.h), it writes the
// float32 values of silu(u) = u / (1 + exp(-u)) and
// silu'(u) = s * (1 + u * (1 - s)), s = 1 / (1 + exp(-u)), evaluated in double
// precision and rounded once to float32.  The double evaluation's error
// (a few units of 2**-53) is far below the distance of each of these values
// from a float32 rounding boundary (more than 1e-13 relative over this range),
// so each entry is the correctly rounded float32 value.  Output: the two
// tables as C hexadecimal float literals, silu first, to be included as the
// initialiser of a float[2][4096] array.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

static double bf16_value(uint32_t b) {
  const uint32_t u = b << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return (double)f;
}

int main() {
  constexpr int N = 4096;
  for (int which = 0; which < 2; ++which) {
    std::printf("/* %s */\n", which == 0 ? "silu" : "silu'");
    for (int i = 0; i < N; ++i) {
      const uint32_t s = (uint32_t)i >> 11, ex = (((uint32_t)i >> 7) & 15u) + 119u, m = (uint32_t)i & 0x7Fu;
      const double x = bf16_value((s << 15) | (ex << 7) | m);
      const double sg = 1.0 / (1.0 + std::exp(-x));
      const double v = which == 0 ? x / (1.0 + std::exp(-x)) : sg * (1.0 + x * (1.0 - sg));
      std::printf("%af,%s", (double)(float)v, (i % 4 == 3) ? "\n" : " ");
    }
  }
  return 0;
}
