/*
 * Oracle for F^H D and Q -- TEST INFRASTRUCTURE, not part of the product.
 *
 * A plain, slow, double-precision CPU evaluation of the definitions, used only
 * by the tests, the smoke check and the CPU-baseline leg of the benchmark.  It
 * shares no code with the HIP library and never calls it.
 *
 * What it computes (PMPP ch. 17 "Iterative MRI reconstruction"):
 *   - Section 17.2 / Fig. 17.3: the reconstruction needs the matrix-vector
 *     product F^H D, where F models the imaging physics and D holds the scan
 *     samples, and Q, a structure with the same core computation that lets
 *     the solver apply F^H F without forming it.
 *   - Section 17.1, Eq. 17.1: each sample contributes with weight times data
 *     times exp(+i 2 pi k_j . r).
 *   - Section 17.3 (sequential code, Fig. 17.4, and its loop-fission form,
 *     Fig. 17.6): per k-space sample first form Mu (real and imaginary parts),
 *     then add that sample's contribution to every voxel.
 *   - The register-promoted kernel printed on the study-notes page for step 2
 *     ("FHD Kernel memory bandwidth optimisation") fixes the complex
 *     multiply-accumulate: re += rMu cos - iMu sin, im += iMu cos + rMu sin,
 *     with the angle 2*pi*(kx x + ky y + kz z).
 * Mu = conj(phi) * D (the pages never print Mu; this reading makes the sum
 * equal to the conjugate transpose of F[m][n] = phi_m exp(-i 2 pi k_m . x_n)
 * applied to D).  Q uses the real weight |phi_m|^2 in place of Mu.
 *
 * The forward model F itself (section 17.2: F models the imaging physics
 * relating the image to the scan data; section 17.3 step 3 synthesises scan
 * data from an image by this "inverse process"):
 *
 *   D[b][m]   = phi[m] * sum_n rho[b][n] exp(-i 2 pi (kx[m]x[n]+ky[m]y[n]+kz[m]z[n]))
 *
 *   FhD[b][n] = sum_m conj(phi[m]) D[b][m] exp(+i 2 pi (kx[m]x[n]+ky[m]y[n]+kz[m]z[n]))
 *   Q[n]      = sum_m |phi[m]|^2          exp(+i 2 pi (kx[m]x[n]+ky[m]y[n]+kz[m]z[n]))
 *
 * All float32 inputs are promoted exactly to double; the angle is formed in
 * double with 2*pi as 2*M_PI; cos/sin are libm's; the sum over m runs in
 * order m = 0..M-1 for every voxel.  No blocking, no reordering.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (never -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

/* Complex numbers are interleaved (re, im) float32 pairs on input and
 * (re, im) double pairs on output. */

static int threads_used(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * oracle_fhd: out[(b*nidx + i)*2 + {0,1}] = FhD[b][n] with n = idx[i] (or n = i
 * if idx is NULL, then nidx must equal N).  Returns 0 on success, -1 on bad
 * arguments, -2 on allocation failure.  *threads receives the OpenMP thread
 * count (may be NULL).
 */
int oracle_fhd(const float* kx, const float* ky, const float* kz,
               const float* x, const float* y, const float* z,
               const float* phi, const float* D,
               int64_t M, int64_t N, int32_t B,
               const int64_t* idx, int64_t nidx,
               double* out, int32_t* threads) {
  if (M < 0 || N < 0 || B < 1 || nidx < 0) return -1;
  if (!idx && nidx != N) return -1;
  if (threads) *threads = threads_used();
  if (nidx == 0) return 0;
  /* Stage 1 (loop fission, first loop): Mu for every sample and vector. */
  double* mu = (double*)malloc(sizeof(double) * 2 * (size_t)(M > 0 ? M : 1) * (size_t)B);
  if (!mu) return -2;
  for (int32_t b = 0; b < B; ++b) {
    for (int64_t m = 0; m < M; ++m) {
      double pr = phi[2 * m], pi = phi[2 * m + 1];
      double dr = D[2 * ((int64_t)b * M + m)], di = D[2 * ((int64_t)b * M + m) + 1];
      /* conj(phi) * D = (pr - i pi)(dr + i di) */
      mu[2 * ((int64_t)b * M + m)] = pr * dr + pi * di;
      mu[2 * ((int64_t)b * M + m) + 1] = pr * di - pi * dr;
    }
  }
  /* Stage 2 (loop fission, second loop, interchanged so voxels are outer). */
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nidx; ++i) {
    int64_t n = idx ? idx[i] : i;
    double xn = x[n], yn = y[n], zn = z[n];
    for (int32_t b = 0; b < B; ++b) {
      out[2 * ((int64_t)b * nidx + i)] = 0.0;
      out[2 * ((int64_t)b * nidx + i) + 1] = 0.0;
    }
    for (int64_t m = 0; m < M; ++m) {
      double arg = 2.0 * M_PI * ((double)kx[m] * xn + (double)ky[m] * yn + (double)kz[m] * zn);
      double c = cos(arg), s = sin(arg);
      for (int32_t b = 0; b < B; ++b) {
        double rmu = mu[2 * ((int64_t)b * M + m)], imu = mu[2 * ((int64_t)b * M + m) + 1];
        out[2 * ((int64_t)b * nidx + i)] += rmu * c - imu * s;
        out[2 * ((int64_t)b * nidx + i) + 1] += imu * c + rmu * s;
      }
    }
  }
  free(mu);
  return 0;
}

/* oracle_q: out[i*2 + {0,1}] = Q[n], n = idx[i] (or i).  Same return codes. */
int oracle_q(const float* kx, const float* ky, const float* kz,
             const float* x, const float* y, const float* z,
             const float* phi, int64_t M, int64_t N,
             const int64_t* idx, int64_t nidx,
             double* out, int32_t* threads) {
  if (M < 0 || N < 0 || nidx < 0) return -1;
  if (!idx && nidx != N) return -1;
  if (threads) *threads = threads_used();
  if (nidx == 0) return 0;
  double* w = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
  if (!w) return -2;
  for (int64_t m = 0; m < M; ++m) {
    double pr = phi[2 * m], pi = phi[2 * m + 1];
    w[m] = pr * pr + pi * pi;
  }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nidx; ++i) {
    int64_t n = idx ? idx[i] : i;
    double xn = x[n], yn = y[n], zn = z[n];
    double re = 0.0, im = 0.0;
    for (int64_t m = 0; m < M; ++m) {
      double arg = 2.0 * M_PI * ((double)kx[m] * xn + (double)ky[m] * yn + (double)kz[m] * zn);
      re += w[m] * cos(arg);
      im += w[m] * sin(arg);
    }
    out[2 * i] = re;
    out[2 * i + 1] = im;
  }
  free(w);
  return 0;
}

/*
 * oracle_forward: out[(b*nidx + i)*2 + {0,1}] = D[b][m] = (F rho_b)[m] with
 * m = idx[i] (or m = i if idx is NULL, then nidx must equal M), for the
 * forward model F[m][n] = phi_m exp(-i 2 pi k_m . x_n) applied to the images
 * rho[b][n] (complex, vector-major).  For every sample the voxel sum runs in
 * order n = 0..N-1 in double, then the sum is multiplied by phi_m.  Same
 * return codes as oracle_fhd.
 */
int oracle_forward(const float* kx, const float* ky, const float* kz,
                   const float* x, const float* y, const float* z,
                   const float* phi, const float* rho,
                   int64_t M, int64_t N, int32_t B,
                   const int64_t* idx, int64_t nidx,
                   double* out, int32_t* threads) {
  if (M < 0 || N < 0 || B < 1 || nidx < 0) return -1;
  if (!idx && nidx != M) return -1;
  if (threads) *threads = threads_used();
  if (nidx == 0) return 0;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nidx; ++i) {
    int64_t m = idx ? idx[i] : i;
    double km[3] = {kx[m], ky[m], kz[m]};
    double pr = phi[2 * m], pi = phi[2 * m + 1];
    for (int32_t b = 0; b < B; ++b) {
      double re = 0.0, im = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        double arg = 2.0 * M_PI * (km[0] * (double)x[n] + km[1] * (double)y[n] + km[2] * (double)z[n]);
        double c = cos(arg), s = sin(arg);
        double rr = rho[2 * ((int64_t)b * N + n)], ri = rho[2 * ((int64_t)b * N + n) + 1];
        /* rho * exp(-i arg) = (rr + i ri)(c - i s) */
        re += rr * c + ri * s;
        im += ri * c - rr * s;
      }
      /* phi * sum */
      out[2 * ((int64_t)b * nidx + i)] = pr * re - pi * im;
      out[2 * ((int64_t)b * nidx + i) + 1] = pr * im + pi * re;
    }
  }
  return 0;
}
