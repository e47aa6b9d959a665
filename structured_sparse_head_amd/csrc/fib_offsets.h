// Offset generation shared by the host entry points and the kernels.
//
// Fibottention paper (arXiv 2406.19391), method section: head i attends the
// pairs (j, k) with |j - k| a term of the generalized Fibonacci sequence
// Fib(a, b) and |j - k| <= w.  The project README's Algorithm 1 builds the
// sequence from [a, b] by repeated sums.  Here the terms are produced in
// ascending order without duplicates and cut at `lim` = min(w, N - 1) (a
// distance of N or more has no pair).
//
// With a >= 0 and b >= 1 the third term a + b is >= max(a, b), equal only
// when a = 0 (then it repeats b), and every later term is strictly larger
// than the one before.  So sorting reduces to ordering the first two terms,
// and duplicates can only be a == b or the repeated b when a == 0.
#pragma once

#include <stdint.h>

// Functions shared with device code carry __host__ __device__ under the HIP
// compiler; the host layer is also built by a plain C++ compiler.
#if defined(__HIPCC__)
#define FIBATT_HD __host__ __device__
#else
#define FIBATT_HD
#endif

namespace fibatt {

// Largest number of distinct distances a head can have for lim < 2^31:
// (a, b) = (0, 1) gives 0 and the Fibonacci numbers up to 2^31, 47 terms.
constexpr int kMaxOffsets = 64;

// Writes up to `cap` distances into `out` (ascending) and returns how many
// exist in total.  Requires a >= 0, b >= 1, lim >= 0.
FIBATT_HD inline int fib_offsets_gen(int64_t a, int64_t b, int64_t lim,
                                               int32_t* out, int cap) {
  int n = 0;
  const int64_t lo = a < b ? a : b;
  const int64_t hi = a < b ? b : a;
  if (lo <= lim) {
    if (n < cap) out[n] = static_cast<int32_t>(lo);
    ++n;
  }
  if (hi != lo && hi <= lim) {
    if (n < cap) out[n] = static_cast<int32_t>(hi);
    ++n;
  }
  int64_t x = a, y = b;
  for (;;) {
    const int64_t z = x + y;
    if (z > lim) break;
    if (z != hi) {  // z == hi only for the third term when a == 0
      if (n < cap) out[n] = static_cast<int32_t>(z);
      ++n;
    }
    x = y;
    y = z;
  }
  return n;
}

}  // namespace fibatt
