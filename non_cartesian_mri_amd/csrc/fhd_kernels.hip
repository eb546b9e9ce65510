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
//    reduced phase then goes through sincos_turns (exact quarter-turn
//    reduction and fitted polynomials, within 2 ulp).
//
// Summation: per-tile partial sums are folded into running totals (blocked);
// optionally the fold is Kahan-compensated (the reduction article's
// compensated-summation section).
#include "fhd_internal.h"
#include "fhd_trig.h"

namespace ncmri {
namespace {

// Keeps the compiler's scheduler from moving instructions across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

template <typename R>
__device__ __forceinline__ void phase_sincos_hw(const R& r, float p0, float x, float y, float z,
                                                float& c, float& s) {
  float t = __builtin_fmaf(r[2], z, __builtin_fmaf(r[1], y, p0));
  float f = __builtin_amdgcn_fractf(t);
  s = __builtin_amdgcn_sinf(f);
  c = __builtin_amdgcn_cosf(f);
}

template <typename R>
__device__ __forceinline__ void phase_sincos_acc(const R& r, float p0, float x, float y, float z,
                                                 float& c, float& s) {
  float th = __builtin_fmaf(r[2], z, __builtin_fmaf(r[1], y, p0));
  th = th - __builtin_rintf(th);
  float tl = __builtin_fmaf(r[5], z, __builtin_fmaf(r[4], y, r[3] * x));
  sincos_turns(th + tl, s, c);
}

// p0 must be r[0] * x (the first product of the phase); passing it in lets a
// caller consume the record's first dword early.
template <int TRIG, typename R>
__device__ __forceinline__ void phase_sincos(const R& r, float p0, float x, float y, float z,
                                             float& c, float& s) {
  if constexpr (TRIG == kTrigHw) phase_sincos_hw(r, p0, x, y, z, c, s);
  else phase_sincos_acc(r, p0, x, y, z, c, s);
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
  // Double-buffer the records in SGPRs when two of them fit and a sample
  // carries enough VALU work to cover the next record's load (measured: a
  // gain for 24-32 dword records, a loss for shorter ones).
  static constexpr bool PIPE = STRIDE >= 24 && 2 * STRIDE <= 64 && kUnroll % 2 == 0;
  // Samples per step of the plain regular loop (kUnroll must be a multiple).
  // Measured on MI355X for 52-56 dword records: 4 is fastest for F^H D and
  // the batched passes; Q spills scalar registers at 4 and runs best at 2.
  static constexpr int RU = (STRIDE > 40 && QW) ? 2 : kUnroll;

  // dword offset of set s inside a record
  static constexpr int set_off(int s) { return QW ? (s == 0 ? H : H + 1 + 3 * (s - 1)) : H + 3 * s; }

  __device__ static __forceinline__ void load_record(float (&dst)[STRIDE], const float* src) {
#pragma unroll
    for (int i = 0; i < STRIDE; ++i) dst[i] = src[i];
  }

  // One sample for a regular wave: phase of the group's first voxel (p0 =
  // r[0] * x0 already formed), then the three-FMA complex MAC for every set.
  template <typename R>
  __device__ static __forceinline__ void regular_step(const R& r, float p0, float x0, float y0,
                                                      float z0, float (&A)[S], float (&Bq)[S],
                                                      float (&Cr)[S]) {
    float c, s;
    phase_sincos<TRIG>(r, p0, x0, y0, z0, c, s);
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

  // One sample for a wave whose voxels are not on the common offsets: every
  // voxel's phase is evaluated; the sets of offset 0 carry Mu_b (or w).
  __device__ static __forceinline__ void direct_step(const float* r, const float (&vx)[V],
                                                     const float (&vy)[V], const float (&vz)[V],
                                                     float (&A)[S], float (&Bq)[S], float (&Cr)[S]) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      float c, s;
      phase_sincos<TRIG>(r, r[0] * vx[j], vx[j], vy[j], vz[j], c, s);
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

  // Folds one tile's partial sums into the running totals (optionally
  // Kahan-compensated).  rf_all: every set is in real form (Q, direct path).
  __device__ static __forceinline__ void fold(bool direct, float (&A)[S], float (&Bq)[S],
                                              float (&Cr)[S], float (&Tre)[S], float (&Tim)[S],
                                              float (&Kre)[KAHAN ? S : 1],
                                              float (&Kim)[KAHAN ? S : 1]) {
#pragma unroll
    for (int q = 0; q < S; ++q) {
      // real-form sets (Q weight w applied directly): re += w c, im += w s
      const bool rf = QW && (q == 0 || direct);
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

  // Sums the samples [lo, hi) (both multiples of kUnroll) tile by tile into
  // the totals.  The regular (factored) and direct forms are separate
  // instantiations so that the regular loop keeps only the group's first
  // voxel in registers.
  template <bool REG>
  __device__ static __forceinline__ void sum_range(const float* __restrict__ rec, int32_t lo,
                                                   int32_t hi, int32_t tile,
                                                   const float (&vx)[V], const float (&vy)[V],
                                                   const float (&vz)[V], float (&Tre)[S],
                                                   float (&Tim)[S], float (&Kre)[KAHAN ? S : 1],
                                                   float (&Kim)[KAHAN ? S : 1]) {
    float A[S], Bq[S], Cr[S];  // tile partials
    for (int32_t t0 = lo; t0 < hi; t0 += tile) {
      const int32_t t1 = (hi - t0 > tile) ? t0 + tile : hi;
#pragma unroll
      for (int q = 0; q < S; ++q) { A[q] = 0.0f; Bq[q] = 0.0f; Cr[q] = 0.0f; }
      const float* p = rec + (int64_t)t0 * STRIDE;
      const float* pend = rec + (int64_t)t1 * STRIDE;
      if constexpr (REG && PIPE) {
        // Ping-pong over two SGPR-resident records.  Scalar loads may return
        // out of order, so a wait covers every load in flight: the current
        // record's first dword is consumed (forcing its wait) before the next
        // record's loads are issued, and the fences keep the scheduler from
        // hoisting those loads above that first use.  The next record's
        // latency then overlaps one sample's VALU work.
        const float x0 = vx[0], y0 = vy[0], z0 = vz[0];
        float ra[STRIDE], rb[STRIDE];
        load_record(ra, p);
        for (; p < pend; p += 2 * STRIDE) {
          const float pa = ra[0] * x0;
          sched_fence();
          load_record(rb, p + STRIDE);
          sched_fence();
          regular_step(ra, pa, x0, y0, z0, A, Bq, Cr);
          const float pb = rb[0] * x0;
          sched_fence();
          load_record(ra, (p + 2 * STRIDE < pend) ? p + 2 * STRIDE : p);
          sched_fence();
          regular_step(rb, pb, x0, y0, z0, A, Bq, Cr);
        }
      } else if constexpr (REG) {
        const float x0 = vx[0], y0 = vy[0], z0 = vz[0];
        for (; p < pend; p += RU * STRIDE) {
#pragma unroll
          for (int u = 0; u < RU; ++u) {
            const float* r = p + u * STRIDE;
            regular_step(r, r[0] * x0, x0, y0, z0, A, Bq, Cr);
          }
        }
      } else {
        for (; p < pend; p += kUnroll * STRIDE) {
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) direct_step(p + u * STRIDE, vx, vy, vz, A, Bq, Cr);
        }
      }
      fold(!REG, A, Bq, Cr, Tre, Tim, Kre, Kim);
    }
  }

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

    float Tre[S], Tim[S];                          // running totals
    float Kre[KAHAN ? S : 1], Kim[KAHAN ? S : 1];  // Kahan compensations
#pragma unroll
    for (int q = 0; q < S; ++q) {
      Tre[q] = 0.0f; Tim[q] = 0.0f;
      if constexpr (KAHAN) { Kre[q] = 0.0f; Kim[q] = 0.0f; }
    }

    // This launch row's share of the samples (the sample dimension is split
    // across gridDim.y rows; the rows' partial sums are added by reduce_kernel).
    const int32_t split = (int32_t)blockIdx.y;
    const int32_t mpad = (int32_t)a.mpad;
    const int64_t lo64 = (int64_t)split * a.m_split;
    const int32_t lo = (int32_t)(lo64 < mpad ? lo64 : mpad);
    const int32_t hi = (int32_t)(lo64 + a.m_split < mpad ? lo64 + a.m_split : mpad);
    if (wave_regular)
      sum_range<true>(a.rec, lo, hi, (int32_t)a.tile, vx, vy, vz, Tre, Tim, Kre, Kim);
    else
      sum_range<false>(a.rec, lo, hi, (int32_t)a.tile, vx, vy, vz, Tre, Tim, Kre, Kim);

    // write-out: out[b][n0 + j], or this row's partial sums
    float2* dst = a.partial ? a.partial + (int64_t)split * BC * a.N : a.out;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t n = n0 + j;
      if (n < a.N) {
#pragma unroll
        for (int b = 0; b < BC; ++b) {
          const int q = j * BC + b;
          dst[(int64_t)b * a.N + n] = make_float2(Tre[q], Tim[q]);
        }
      }
    }
  }
};

// Adds the partial sums of the sample splits in split order (fixed, so the
// result is deterministic): out[i] = sum_p partial[p][i], i < count.
__global__ void __launch_bounds__(kWorkgroup)
reduce_kernel(const float2* __restrict__ partial, float2* __restrict__ out, int64_t count,
              int32_t splits, int32_t kahan) {
  const int64_t i = (int64_t)blockIdx.x * kWorkgroup + threadIdx.x;
  if (i >= count) return;
  float re = 0.0f, im = 0.0f, cr = 0.0f, ci = 0.0f;
  for (int32_t p = 0; p < splits; ++p) {
    const float2 v = partial[(int64_t)p * count + i];
    if (kahan) {
      const float yr = v.x - cr, tr = re + yr;
      cr = (tr - re) - yr;
      re = tr;
      const float yi = v.y - ci, ti = im + yi;
      ci = (ti - im) - yi;
      im = ti;
    } else {
      re += v.x;
      im += v.y;
    }
  }
  out[i] = make_float2(re, im);
}

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

hipError_t launch_gather(const Layout& L, bool kahan, int32_t splits, const GatherArgs& a,
                         hipStream_t s) {
  GatherFn fn = select(L, kahan);
  if (!fn || splits < 1 || (splits > 1) != (a.partial != nullptr)) return hipErrorInvalidValue;
  if (a.N <= 0) return hipSuccess;
  const int64_t lanes = (a.N + L.V - 1) / L.V;
  const int64_t blocks = (lanes + kWorkgroup - 1) / kWorkgroup;
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks, (unsigned)splits), dim3(kWorkgroup), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reduce(int BC, bool kahan, int32_t splits, const GatherArgs& a, hipStream_t s) {
  if (splits < 2 || !a.partial || a.N <= 0) return hipSuccess;
  const int64_t count = (int64_t)BC * a.N;
  const int64_t rblocks = (count + kWorkgroup - 1) / kWorkgroup;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)rblocks), dim3(kWorkgroup), 0, s, a.partial,
                     a.out, count, splits, kahan ? 1 : 0);
  return hipGetLastError();
}

}  // namespace ncmri
