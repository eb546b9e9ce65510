// Device helpers shared by the forward operator's matrix-core engines (PMPP
// ch. 17 "Iterative MRI reconstruction", section 17.2's F; section 17.3 step 3):
// the per-lane sample wave-vector with its phase, cosine and sine, the A
// entries of the three-product form, and the finish of the four-group
// engines (G through LDS, contracted with exp(-i 2 pi k . d_j), times phi).
#pragma once

#include "fhd_internal.h"
#include "fhd_mfma_common.h"
#include "fhd_trig.h"

namespace ncmri {
namespace {

// Per-lane sample wave-vector: k (HW) or its exact split k = kh + kl, kh a
// multiple of 2^-12 (accurate), as the adjoint's records kernel forms it.
template <int TRIG>
struct SampleK {
  static constexpr int NK = TRIG == kTrigHw ? 3 : 6;
  float v[NK];
  __device__ void load(const FwdArgs& a, int64_t m, bool valid) {
    const float kx = valid ? a.kx[m] : 0.0f, ky = valid ? a.ky[m] : 0.0f, kz = valid ? a.kz[m] : 0.0f;
    if constexpr (TRIG == kTrigHw) {
      v[0] = kx; v[1] = ky; v[2] = kz;
    } else {
      v[0] = __builtin_rintf(kx * 4096.0f) * (1.0f / 4096.0f);
      v[1] = __builtin_rintf(ky * 4096.0f) * (1.0f / 4096.0f);
      v[2] = __builtin_rintf(kz * 4096.0f) * (1.0f / 4096.0f);
      v[3] = kx - v[0]; v[4] = ky - v[1]; v[5] = kz - v[2];
    }
  }
  // cos and sin of 2 pi k . p.
  __device__ __forceinline__ void sincos_phase(float px, float py, float pz, float& c, float& s) const {
    if constexpr (TRIG == kTrigHw) {
      const float t = __builtin_fmaf(v[2], pz, __builtin_fmaf(v[1], py, v[0] * px));
      const float f = __builtin_amdgcn_fractf(t);
      s = __builtin_amdgcn_sinf(f);
      c = __builtin_amdgcn_cosf(f);
    } else {
      float th = __builtin_fmaf(v[2], pz, __builtin_fmaf(v[1], py, v[0] * px));
      th = th - __builtin_rintf(th);
      const float tl = __builtin_fmaf(v[5], pz, __builtin_fmaf(v[4], py, v[3] * px));
      sincos_turns(th + tl, s, c);
    }
  }
};

// A entries (c - s, c + s, s) of one lane's (sample, group) phase in the
// three-product form of (c - i s)(rr + i ri).
template <int TRIG>
__device__ __forceinline__ void fwd_entries(const SampleK<TRIG>& k, const float (&hs)[3], float (&av)[3]) {
  float c, s;
  k.sincos_phase(hs[0], hs[1], hs[2], c, s);
  av[0] = c - s;
  av[1] = c + s;
  av[2] = s;
}

// Finish of a four-group engine wave (16 samples, T units of 16 complex
// columns, groups of V = 16 T / BC voxels): ore / oim hold the wave's G block
// (Re, Im) in the 16x16 accumulator layout; lds holds at least NW blocks of
// GH float4s and every wave of the workgroup has passed its last barrier.
template <int T, int BC, int TRIG>
__device__ __forceinline__ void fwd_finish(const FwdArgs& a, float4* lds, int wig, int lane, bool valid, int64_t m,
                                           int32_t row, const SampleK<TRIG>& k, const f32x4 (&ore)[T],
                                           const f32x4 (&oim)[T]) {
  constexpr int V = 16 * T / BC;
  constexpr int HC = 8 * T;                  // G columns per half
  constexpr int GH = 16 * HC * 2 / 4;        // float4s of one wave's half G block
  // Finish.  Every wave has passed the last barrier, so the staging buffers
  // are free.  Per half of the columns (units t of one half): each wave
  // stores its 16 x 8 T complex block of G there ...
  float2* gl = reinterpret_cast<float2*>(lds + wig * GH);
  const float2* gr = gl + (lane & 15) * HC;
  const int c = lane & 15;
  float dre[BC], dim[BC];
#pragma unroll
  for (int b = 0; b < BC; ++b) { dre[b] = 0.0f; dim[b] = 0.0f; }
  // offsets relative to the reference column (0, or jref < N with mirror pairs)
  const bool any_voxel = a.N > 0;
  const float x0 = any_voxel ? a.x[a.jref] : 0.0f, y0 = any_voxel ? a.y[a.jref] : 0.0f,
              z0 = any_voxel ? a.z[a.jref] : 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h > 0) __syncthreads();   // the first half's reads are done
#pragma unroll
    for (int u = 0; u < T / 2; ++u) {
      const int t = h * (T / 2) + u;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (lane >> 4) + r;
        gl[i * HC + 16 * u + c] = make_float2(ore[t][r], oim[t][r]);
      }
    }
    __syncthreads();
    // ... and lane l contracts the offsets j = l / 16 (mod 4) of row l % 16
    // (its sample) with exp(-i 2 pi k . d_j).  One vector: this half holds
    // the offsets [h HC, (h + 1) HC); several: it holds vectors
    // [h BC/2, (h + 1) BC/2), every offset.
    if (valid) {
      constexpr int JN = BC == 1 ? HC : V;
      const int j0 = BC == 1 ? h * HC : 0;
      for (int jj = lane >> 4; jj < JN && j0 + jj < a.N; jj += 4) {
        const int j = j0 + jj;
        float cj = 1.0f, sj = 0.0f;
        if (j != a.jref) k.sincos_phase(a.x[j] - x0, a.y[j] - y0, a.z[j] - z0, cj, sj);
#pragma unroll
        for (int bb = 0; bb < (BC == 1 ? 1 : BC / 2); ++bb) {
          const int b = BC == 1 ? 0 : h * (BC / 2) + bb;
          const float2 gv = gr[bb * V + jj];
          // (cj - i sj)(gre + i gim)
          dre[b] = __builtin_fmaf(cj, gv.x, __builtin_fmaf(sj, gv.y, dre[b]));
          dim[b] = __builtin_fmaf(cj, gv.y, __builtin_fmaf(-sj, gv.x, dim[b]));
        }
      }
    }
  }
  // the four lanes of a row add their sums, (p0 + p1) + (p2 + p3), and one
  // of them multiplies by phi_m
#pragma unroll
  for (int b = 0; b < BC; ++b) {
    dre[b] += __shfl_xor(dre[b], 16);
    dim[b] += __shfl_xor(dim[b], 16);
    dre[b] += __shfl_xor(dre[b], 32);
    dim[b] += __shfl_xor(dim[b], 32);
  }
  if (lane >= 16 || !valid) return;
  const float2 ph = a.phi[m];
  float2* dst = a.partial ? a.partial + (int64_t)row * BC * a.M : a.out;
#pragma unroll
  for (int b = 0; b < BC; ++b)
    dst[(int64_t)b * a.M + m] = make_float2(ph.x * dre[b] - ph.y * dim[b], ph.x * dim[b] + ph.y * dre[b]);
}

}  // namespace
}  // namespace ncmri
