// Device helpers of the grid-factored matrix-core gathers (PMPP ch. 17
// "Iterative MRI reconstruction", section 17.3): a wave's regularity vote,
// the sample range of a launch row, and a group phase's cosine and sine with
// the three-product A entries.  Shared by the fp32 engines and the
// half-split engine.
#pragma once

#include "fhd_internal.h"
#include "fhd_trig.h"

namespace ncmri {
namespace {

// ---------------------------------------------------------------------------
// Wave w of either gather kernel owns the voxel groups G w .. G w + G - 1 of V
// voxels each (G = 32 for the two-sample engine, 16 for the four-sample
// engine), i.e. voxels [G V w, G V (w + 1)).  The wave is "regular" when every
// group's voxels sit at the offsets of the first group (exact double
// comparison of the coordinate differences); the 64 / G lanes l = i mod G of
// group i split its voxels.  Returns the wave-uniform vote.
template <int V, int G = 32>
__device__ __forceinline__ bool wave_regular(const float* __restrict__ x, const float* __restrict__ y,
                                             const float* __restrict__ z, int64_t N, int64_t n0,
                                             int lane, float gx, float gy, float gz) {
  constexpr int parts = 64 / G, per = (V + parts - 1) / parts;
  bool reg = true;
  const double bx = x[0], by = y[0], bz = z[0];
  const int r = lane / G;
  // offsets j = r per + t of the group (j >= 1), unrolled so that the
  // coordinate loads of several offsets are in flight together
#pragma unroll 8
  for (int t = 0; t < per; ++t) {
    const int j = r * per + t;
    const int64_t n = n0 + j;
    if (j >= 1 && j < V && n < N)
      reg &= ((double)x[n] - (double)gx == (double)x[j] - bx) &
             ((double)y[n] - (double)gy == (double)y[j] - by) &
             ((double)z[n] - (double)gz == (double)z[j] - bz);
  }
  return __all(reg);
}

// Samples [lo, hi) of launch row `row`.
__device__ __forceinline__ void row_range(int64_t m_split, int64_t mpad, int32_t row, int64_t& lo,
                                          int64_t& hi) {
  const int64_t lo64 = (int64_t)row * m_split;
  lo = lo64 < mpad ? lo64 : mpad;
  hi = lo64 + m_split < mpad ? lo64 + m_split : mpad;
}

// ---------------------------------------------------------------------------
// cos and sin of the phase 2 pi k.x of one point (x, y, z) from a sample
// header hs: HW trig reduces the phase in turns with fract and feeds v_sin /
// v_cos; the accurate path reduces kh.x exactly (kh a multiple of 2^-12, so
// kh.x is exact for integer or half-integer coordinates of moderate size),
// adds kl.x and evaluates the quarter-turn polynomials.
template <int TRIG>
__device__ __forceinline__ void phase_sincos(const float* hs, float x, float y, float z, float& c,
                                             float& s) {
  if constexpr (TRIG == kTrigHw) {
    const float t = __builtin_fmaf(hs[2], z, __builtin_fmaf(hs[1], y, hs[0] * x));
    const float f = __builtin_amdgcn_fractf(t);
    s = __builtin_amdgcn_sinf(f);
    c = __builtin_amdgcn_cosf(f);
  } else {
    float th = __builtin_fmaf(hs[2], z, __builtin_fmaf(hs[1], y, hs[0] * x));
    th = th - __builtin_rintf(th);
    const float tl = __builtin_fmaf(hs[6], z, __builtin_fmaf(hs[5], y, hs[4] * x));
    sincos_turns(th + tl, s, c);
  }
}

// A-operand entries of a group phase in the three-product form: (c + s, c - s, s).
template <int TRIG>
__device__ __forceinline__ void group_entries(const float* hs, float gx, float gy, float gz,
                                              float (&av)[3]) {
  float c, s;
  phase_sincos<TRIG>(hs, gx, gy, gz, c, s);
  av[0] = c + s;
  av[1] = c - s;
  av[2] = s;
}

}  // namespace
}  // namespace ncmri
