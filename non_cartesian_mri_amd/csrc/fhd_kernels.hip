// gfx950 kernels for F^H D and Q (PMPP ch. 17 "Iterative MRI reconstruction").
//
// Two kernels, as loop fission splits the computation (section 17.3 step 1,
// Figs. 17.6 and 17.7):
//
//  * records_kernel -- one lane per k-space sample.  Forms Mu = conj(phi) D
//    (or the real weight |phi|^2 for Q) and packs everything the gather needs
//    for that sample into one array-of-structures record (the pages move k
//    from three arrays into one array of structs, Figs. 17.14-17.16, so the
//    values a step needs share one cache line).
//
//  * gather_kernel -- one lane owns V voxels (the pages' gather after loop
//    interchange, Figs. 17.9/17.10, with "several voxels per thread" from the
//    same section's remark on larger images).  Voxel coordinates and all
//    accumulators live in VGPRs for the whole sum (register promotion, Fig.
//    17.11).  Every lane of a wave reads the same record at the same time, so
//    records are fetched with wave-uniform scalar loads into SGPRs and fed to
//    the VALU as its one scalar operand -- the broadcast the pages obtain from
//    constant memory (Figs. 17.12/17.13), without the 64 KB chunking and
//    repeated host launches: one launch walks any number of samples.
//
// Phase factoring.  On gfx950 a v_sin_f32 / v_cos_f32 costs about two VALU
// issue slots and shares the issue port with FMAs, so the direct form costs
// ~12 slots per (voxel, sample).  When a lane's V voxels sit at offsets d_j
// from its first voxel x0 (identical offsets for every lane, as on a Cartesian
// grid), exp(i2pi k.(x0+d_j)) = exp(i2pi k.x0) * exp(i2pi k.d_j), and the
// second factor does not depend on the lane.  The records kernel therefore
// stores f_j = Mu * exp(i2pi k.d_j) (in double, rounded once), and the gather
// evaluates one sin/cos per sample for x0 and then only multiply-accumulates
// f_j * (c + i s) for the other voxels.  The complex MAC uses three real FMAs
// (Gauss): with E = c + i s and f = fr + i fi,
//     A += c (fr+fi),  B += (c+s) fi,  C += (s-c) fr   ==>  Re = A - B, Im = A + C.
// Waves whose voxels do not have the common offsets (any non-grid coordinate
// set) evaluate the phase of every voxel directly.  Both paths compute the
// same sum; only the rounding differs.
//
// Trig paths (section 17.3 step 3, Fig. 17.17: hardware trig functions):
//  * HW: t = k.x in revolutions (fp32 FMA chain), fract(t), v_sin_f32 and
//    v_cos_f32 -- these instructions take their argument in revolutions.
//  * accurate: k is split as kh + kl with kh a multiple of 2^-12; for integer
//    or half-integer coordinates of moderate size kh.x is exact in fp32, so
//    its fractional part is exact and only the small kl.x term rounds; the
//    reduced phase then goes through the library's sincospi.
//
// Summation: per-tile partial sums are folded into running totals (blocked);
// optionally the fold is Kahan-compensated (the reduction article's
// compensated-summation section).
#include "fhd_internal.h"

namespace ncmri {
namespace {

__device__ __forceinline__ void phase_sincos_hw(const float* r, float x, float y, float z,
                                                float& c, float& s) {
  float t = __builtin_fmaf(r[2], z, __builtin_fmaf(r[1], y, r[0] * x));
  float f = __builtin_amdgcn_fractf(t);
  s = __builtin_amdgcn_sinf(f);
  c = __builtin_amdgcn_cosf(f);
}

__device__ __forceinline__ void phase_sincos_acc(const float* r, float x, float y, float z,
                                                 float& c, float& s) {
  float th = __builtin_fmaf(r[2], z, __builtin_fmaf(r[1], y, r[0] * x));
  th = th - __builtin_rintf(th);
  float tl = __builtin_fmaf(r[5], z, __builtin_fmaf(r[4], y, r[3] * x));
  float u = th + tl;
  sincospif(2.0f * u, &s, &c);
}

template <int TRIG>
__device__ __forceinline__ void phase_sincos(const float* r, float x, float y, float z,
                                             float& c, float& s) {
  if constexpr (TRIG == kTrigHw) phase_sincos_hw(r, x, y, z, c, s);
  else phase_sincos_acc(r, x, y, z, c, s);
}

// ---------------------------------------------------------------------------
// Per-sample kernel: Mu and record packing (one lane per padded sample).
__global__ void __launch_bounds__(kWorkgroup)
records_kernel(RecordArgs a, int is_q, int trig, int V, int BC, int stride) {
  const int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= a.mpad) return;
  float* r = a.rec + m * stride;
  if (m >= a.M) {  // padding sample: contributes exactly zero
    for (int i = 0; i < stride; ++i) r[i] = 0.0f;
    return;
  }
  const float kx = a.kx[m], ky = a.ky[m], kz = a.kz[m];
  int o = 0;
  if (trig == kTrigHw) {
    r[0] = kx; r[1] = ky; r[2] = kz;
    o = 3;
  } else {
    // kh = nearest multiple of 2^-12 (exact scaling by powers of two), kl = k - kh (exact).
    const float khx = __builtin_rintf(kx * 4096.0f) * (1.0f / 4096.0f);
    const float khy = __builtin_rintf(ky * 4096.0f) * (1.0f / 4096.0f);
    const float khz = __builtin_rintf(kz * 4096.0f) * (1.0f / 4096.0f);
    r[0] = khx; r[1] = khy; r[2] = khz;
    r[3] = kx - khx; r[4] = ky - khy; r[5] = kz - khz;
    o = 6;
  }
  const double pr = a.phi[m].x, pim = a.phi[m].y;
  const double x0 = a.x[0], y0 = a.y[0], z0 = a.z[0];
  for (int j = 0; j < V; ++j) {
    // phase factor of voxel offset j relative to the group's first voxel
    double cj = 1.0, sj = 0.0;
    if (j > 0) {
      const double p = (double)kx * ((double)a.x[j] - x0) + (double)ky * ((double)a.y[j] - y0) +
                       (double)kz * ((double)a.z[j] - z0);
      sincospi(2.0 * p, &sj, &cj);
    }
    if (is_q) {
      const double w = pr * pr + pim * pim;
      if (j == 0) {
        r[o++] = (float)w;
      } else {
        const double fr = w * cj, fi = w * sj;
        r[o++] = (float)(fr + fi); r[o++] = (float)fr; r[o++] = (float)fi;
      }
    } else {
      for (int b = 0; b < BC; ++b) {
        const float2 d = a.D[(int64_t)b * a.M + m];
        // Mu = conj(phi) * D
        const double mr = pr * d.x + pim * d.y;
        const double mi = pr * d.y - pim * d.x;
        const double fr = mr * cj - mi * sj, fi = mr * sj + mi * cj;
        r[o++] = (float)(fr + fi); r[o++] = (float)fr; r[o++] = (float)fi;
      }
    }
  }
  for (; o < stride; ++o) r[o] = 0.0f;
}

// ---------------------------------------------------------------------------
// Gather kernel.
template <int V, int BC, bool QW, int TRIG, bool KAHAN>
struct Gather {
  static constexpr int S = V * BC;                       // weight sets per record
  static constexpr int H = header_dwords(TRIG);
  static constexpr int STRIDE = record_dwords(QW ? 1 : 0, TRIG, V, BC);

  // dword offset of set s inside a record
  static constexpr int set_off(int s) { return QW ? (s == 0 ? H : H + 1 + 3 * (s - 1)) : H + 3 * s; }

  __device__ static void run(const GatherArgs& a) {
    const int64_t lane = (int64_t)blockIdx.x * kWorkgroup + threadIdx.x;
    const int64_t n0 = lane * V;

    float vx[V], vy[V], vz[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t n = n0 + j;
      const bool ok = n < a.N;
      vx[j] = ok ? a.x[n] : 0.0f;
      vy[j] = ok ? a.y[n] : 0.0f;
      vz[j] = ok ? a.z[n] : 0.0f;
    }
    // Does this lane's group have the common offsets d_j of the first group?
    bool reg = true;
    if constexpr (V > 1) {
      const double bx = a.x[0], by = a.y[0], bz = a.z[0];
#pragma unroll
      for (int j = 1; j < V; ++j) {
        if (n0 + j < a.N) {
          reg = reg && ((double)vx[j] - (double)vx[0] == (double)a.x[j] - bx) &&
                ((double)vy[j] - (double)vy[0] == (double)a.y[j] - by) &&
                ((double)vz[j] - (double)vz[0] == (double)a.z[j] - bz);
        }
      }
    }
    const bool wave_regular = __all(reg);

    // real-form sets (Q weight w applied directly): re += w c, im += w s
    auto real_form = [&](int s) -> bool { return QW && (s == 0 || !wave_regular); };

    float A[S], Bq[S], Cr[S];          // tile partials
    float Tre[S], Tim[S];              // running totals
    float Kre[KAHAN ? S : 1], Kim[KAHAN ? S : 1];  // Kahan compensations
#pragma unroll
    for (int s = 0; s < S; ++s) {
      Tre[s] = 0.0f; Tim[s] = 0.0f;
      if constexpr (KAHAN) { Kre[s] = 0.0f; Kim[s] = 0.0f; }
    }

    const float* __restrict__ rec = a.rec;
    for (int64_t t0 = 0; t0 < a.mpad; t0 += a.tile) {
      const int64_t t1 = (t0 + a.tile < a.mpad) ? t0 + a.tile : a.mpad;
#pragma unroll
      for (int s = 0; s < S; ++s) { A[s] = 0.0f; Bq[s] = 0.0f; Cr[s] = 0.0f; }

      if (wave_regular) {
        for (int64_t m = t0; m < t1; m += kUnroll) {
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            const float* r = rec + (m + u) * STRIDE;
            float c, s;
            phase_sincos<TRIG>(r, vx[0], vy[0], vz[0], c, s);
            const float cps = c + s, smc = s - c;
#pragma unroll
            for (int q = 0; q < S; ++q) {
              const int o = set_off(q);
              if (QW && q == 0) {
                A[0] = __builtin_fmaf(r[o], c, A[0]);
                Bq[0] = __builtin_fmaf(r[o], s, Bq[0]);
              } else {
                A[q] = __builtin_fmaf(r[o], c, A[q]);
                Bq[q] = __builtin_fmaf(r[o + 2], cps, Bq[q]);
                Cr[q] = __builtin_fmaf(r[o + 1], smc, Cr[q]);
              }
            }
          }
        }
      } else {
        // direct evaluation of every voxel's phase; sets (0, b) carry Mu_b
        for (int64_t m = t0; m < t1; m += kUnroll) {
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            const float* r = rec + (m + u) * STRIDE;
#pragma unroll
            for (int j = 0; j < V; ++j) {
              float c, s;
              phase_sincos<TRIG>(r, vx[j], vy[j], vz[j], c, s);
              if constexpr (QW) {
                A[j] = __builtin_fmaf(r[H], c, A[j]);
                Bq[j] = __builtin_fmaf(r[H], s, Bq[j]);
              } else {
                const float cps = c + s, smc = s - c;
#pragma unroll
                for (int b = 0; b < BC; ++b) {
                  const int q = j * BC + b;
                  const int o = set_off(b);
                  A[q] = __builtin_fmaf(r[o], c, A[q]);
                  Bq[q] = __builtin_fmaf(r[o + 2], cps, Bq[q]);
                  Cr[q] = __builtin_fmaf(r[o + 1], smc, Cr[q]);
                }
              }
            }
          }
        }
      }
      // fold the tile into the totals
#pragma unroll
      for (int q = 0; q < S; ++q) {
        const bool rf = real_form(q);
        const float dre = rf ? A[q] : A[q] - Bq[q];
        const float dim = rf ? Bq[q] : A[q] + Cr[q];
        if constexpr (KAHAN) {
          const float yr = dre - Kre[q];
          const float tr = Tre[q] + yr;
          Kre[q] = (tr - Tre[q]) - yr;
          Tre[q] = tr;
          const float yi = dim - Kim[q];
          const float ti = Tim[q] + yi;
          Kim[q] = (ti - Tim[q]) - yi;
          Tim[q] = ti;
        } else {
          Tre[q] += dre;
          Tim[q] += dim;
        }
      }
    }
    // write-out: out[b][n0 + j]
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t n = n0 + j;
      if (n < a.N) {
#pragma unroll
        for (int b = 0; b < BC; ++b) {
          const int q = j * BC + b;
          a.out[(int64_t)b * a.N + n] = make_float2(Tre[q], Tim[q]);
        }
      }
    }
  }
};

template <int V, int BC, bool QW, int TRIG, bool KAHAN>
__global__ void __launch_bounds__(kWorkgroup) gather_kernel(GatherArgs a) {
  Gather<V, BC, QW, TRIG, KAHAN>::run(a);
}

using GatherFn = void (*)(GatherArgs);

template <int V, int BC, bool QW>
GatherFn pick(int trig, bool kahan) {
  if (trig == kTrigHw)
    return kahan ? gather_kernel<V, BC, QW, kTrigHw, true> : gather_kernel<V, BC, QW, kTrigHw, false>;
  return kahan ? gather_kernel<V, BC, QW, kTrigAccurate, true>
               : gather_kernel<V, BC, QW, kTrigAccurate, false>;
}

GatherFn select(const Layout& L, bool kahan) {
  if (L.is_q) {
    switch (L.V) {
      case 1: return pick<1, 1, true>(L.trig, kahan);
      case 2: return pick<2, 1, true>(L.trig, kahan);
      case 4: return pick<4, 1, true>(L.trig, kahan);
      case 8: return pick<8, 1, true>(L.trig, kahan);
      case 16: return pick<16, 1, true>(L.trig, kahan);
      default: return nullptr;
    }
  }
  if (L.BC == 1) {
    switch (L.V) {
      case 1: return pick<1, 1, false>(L.trig, kahan);
      case 2: return pick<2, 1, false>(L.trig, kahan);
      case 4: return pick<4, 1, false>(L.trig, kahan);
      case 8: return pick<8, 1, false>(L.trig, kahan);
      case 16: return pick<16, 1, false>(L.trig, kahan);
      default: return nullptr;
    }
  }
  if (L.V != 1) return nullptr;
  switch (L.BC) {
    case 2: return pick<1, 2, false>(L.trig, kahan);
    case 4: return pick<1, 4, false>(L.trig, kahan);
    case 8: return pick<1, 8, false>(L.trig, kahan);
    case 16: return pick<1, 16, false>(L.trig, kahan);
    default: return nullptr;
  }
}

}  // namespace

bool gather_supported(int is_q, int V, int BC) {
  Layout L{is_q, kTrigHw, V, BC, 0, 0};
  return select(L, false) != nullptr;
}

hipError_t launch_records(const Layout& L, const RecordArgs& a, hipStream_t s) {
  if (a.mpad <= 0) return hipSuccess;
  const int64_t blocks = (a.mpad + kWorkgroup - 1) / kWorkgroup;
  hipLaunchKernelGGL(records_kernel, dim3((unsigned)blocks), dim3(kWorkgroup), 0, s, a, L.is_q,
                     L.trig, L.V, L.BC, L.stride);
  return hipGetLastError();
}

hipError_t launch_gather(const Layout& L, bool kahan, const GatherArgs& a, hipStream_t s) {
  GatherFn fn = select(L, kahan);
  if (!fn) return hipErrorInvalidValue;
  if (a.N <= 0) return hipSuccess;
  const int64_t lanes = (a.N + L.V - 1) / L.V;
  const int64_t blocks = (lanes + kWorkgroup - 1) / kWorkgroup;
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kWorkgroup), 0, s, a);
  return hipGetLastError();
}

}  // namespace ncmri
