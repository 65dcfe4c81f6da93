// Build-time generator of the SiLU / SiLU' tables compiled into libmoe4.
//
// For every bf16 value u with |u| in [2**-16, 2**8) (sign x 24 binades x 128
// mantissas = 6144 entries, indexed as act_index() in act.h), it writes the
// correctly rounded float32 values of silu(u) = u / (1 + exp(-u)) and
// silu'(u) = s * (1 + u * (1 - s)), s = 1 / (1 + exp(-u)):
//  * |u| >= 2**-8: the formula evaluated in double precision and rounded once
//    to float32.  The double evaluation's error (a few units of 2**-53) is far
//    below the distance of each of these values from a float32 rounding
//    boundary (more than 1e-13 relative over this range).
//  * |u| < 2**-8: the Taylor series u/2 + u**2/4 - u**4/48 (silu) and
//    1/2 + u/2 - u**3/12 (silu').  The double sum of the first two terms is
//    exact for a bf16 u in this range; the remaining terms are smaller than the
//    distance of that sum from any float32 rounding boundary it does not sit
//    on, so they only decide exact float32 midpoints, by their sign.
// Output: the two tables as C hexadecimal float literals, silu first, to be
// included as the initialiser of a float[2][6144] array.
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

// Round a to float32; an exact midpoint of two float32 values goes downward
// (down) or upward.
static float round_midpoint(double a, bool down) {
  const float r = (float)a;
  const double d = a - (double)r;
  if (d == 0.0) return r;
  const float n = std::nextafter(r, d > 0 ? INFINITY : -INFINITY);
  if ((double)n - a == d) return down ? std::fmin(r, n) : std::fmax(r, n);  // a halfway between r and n
  return r;
}

int main() {
  constexpr int N = 6144, HALF = N / 2;
  for (int which = 0; which < 2; ++which) {
    std::printf("/* %s */\n", which == 0 ? "silu" : "silu'");
    for (int i = 0; i < N; ++i) {
      const uint32_t s = (uint32_t)i / HALF, t = (uint32_t)i % HALF;
      const uint32_t ex = (t >> 7) + 111u, m = t & 0x7Fu;
      const double x = bf16_value((s << 15) | (ex << 7) | m);
      float v;
      if (ex >= 119u) {
        const double sg = 1.0 / (1.0 + std::exp(-x));
        v = (float)(which == 0 ? x / (1.0 + std::exp(-x)) : sg * (1.0 + x * (1.0 - sg)));
      } else if (which == 0) {
        v = round_midpoint(0.5 * x + 0.25 * (x * x), true);  // next term -u**4/48 < 0
      } else {
        v = round_midpoint(0.5 + 0.5 * x, x > 0.0);  // next term -u**3/12
      }
      std::printf("%af,%s", (double)v, (i % 4 == 3) ? "\n" : " ");
    }
  }
  return 0;
}
