// Correctly rounded fp64 quotient a / b from y = RN(1 / b), in three dependent operations.
//
// q = RN(a y); r = a - b q, exact with one fused multiply-add; the result RN(q + r y). With y the
// correctly rounded reciprocal and finite normal operands (no overflow or underflow on the way), this is
// Markstein's final correction step, and it returns the same value as an IEEE division: checked on the
// host against IEEE division on random and adversarial operand pairs, and exhaustively over all
// significand pairs of narrow binary formats (tests/test_divide_host.py).
#pragma once

#include <cmath>

#ifndef GPTQ_HOST_DEVICE
#define GPTQ_HOST_DEVICE __host__ __device__
#endif

namespace gptq {

GPTQ_HOST_DEVICE inline double div_rn(double a, double b, double y) {
  const double q = a * y;
  const double r = fma(-b, q, a);
  return fma(r, y, q);
}

}  // namespace gptq
