// Device-side trigonometry in revolutions shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace ncmri {

// sin(2 pi u) and cos(2 pi u) for an angle u in turns (|u| < 2^22).
// u is split exactly as u = q/4 + r with q = rint(4u) and |r| <= 1/8, then
// sin(2 pi r) = r P(r^2) and cos(2 pi r) = 1 + r^2 Q(r^2), and the pair is
// rotated by q quarter turns (swaps and sign flips, exact).  P and Q are our
// own fits (weighted least squares on Chebyshev nodes, Lawson-reweighted
// towards minimax, coefficients rounded to fp32); evaluated in fp32 Horner
// form the results are within 1.7 ulp (sin) and 1.0 ulp (cos) of the true
// values on the reduced range.
__device__ __forceinline__ void sincos_turns(float u, float& s, float& c) {
  const float q = __builtin_rintf(4.0f * u);
  const float r = __builtin_fmaf(q, -0.25f, u);  // exact
  const float r2 = r * r;
  float p = __builtin_fmaf(-75.39374542236328f, r2, 81.59236145019531f);
  p = __builtin_fmaf(p, r2, -41.3416633605957f);
  p = __builtin_fmaf(p, r2, 6.2831854820251465f);
  const float sp = p * r;
  float k = __builtin_fmaf(59.245967864990234f, r2, -85.44374084472656f);
  k = __builtin_fmaf(k, r2, 64.93932342529297f);
  k = __builtin_fmaf(k, r2, -19.739208221435547f);
  const float cp = __builtin_fmaf(k, r2, 1.0f);
  const int qi = (int)q;
  const bool odd = (qi & 1) != 0;
  const float s1 = odd ? cp : sp;
  const float c1 = odd ? sp : cp;
  s = __builtin_bit_cast(float, __builtin_bit_cast(unsigned, s1) ^ ((unsigned)(qi & 2) << 30));
  c = __builtin_bit_cast(float, __builtin_bit_cast(unsigned, c1) ^ ((unsigned)((qi + 1) & 2) << 30));
}

}  // namespace ncmri
