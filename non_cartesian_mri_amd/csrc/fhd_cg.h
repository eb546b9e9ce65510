// Internal interface of the reconstruction module (fhd_cg.hip): Toeplitz
// F^H F through the FFT of Q on the grid of coordinate differences, the
// regulariser, and conjugate gradient.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace ncmri {

// Device buffers of one CG solve / normal-operator application on an
// nx x ny x nz grid (n = nx ny nz voxels).
struct CgWorkspace {
  float2* P;        // [8n] padded grid
  float2* X;        // [8n] its spectrum
  float2* r;        // [n] residual
  float2* p;        // [n] search direction
  float2* Ap;       // [n] operator applied to p
  double* partial;  // [1024] stage-1 sums of the dot products
  double* state;    // [8] <r,r>, <p,Ap>, alpha, beta
};

constexpr int kCgPartials = 1024;

// Bytes of a CgWorkspace for an nx x ny x nz grid and the layout within it.
inline size_t cg_align(size_t b) { return (b + 255) / 256 * 256; }
inline size_t cg_workspace_bytes(int64_t n) {
  return 2 * cg_align((size_t)(8 * n) * 8) + 3 * cg_align((size_t)n * 8) +
         cg_align(kCgPartials * sizeof(double)) + cg_align(8 * sizeof(double));
}
inline CgWorkspace cg_workspace(void* base, int64_t n) {
  char* c = (char*)base;
  CgWorkspace w;
  w.P = (float2*)c;  c += cg_align((size_t)(8 * n) * 8);
  w.X = (float2*)c;  c += cg_align((size_t)(8 * n) * 8);
  w.r = (float2*)c;  c += cg_align((size_t)n * 8);
  w.p = (float2*)c;  c += cg_align((size_t)n * 8);
  w.Ap = (float2*)c; c += cg_align((size_t)n * 8);
  w.partial = (double*)c; c += cg_align(kCgPartials * sizeof(double));
  w.state = (double*)c;
  return w;
}

// Each returns nullptr on success, else a static description of the failure.
const char* fft3(int nx, int ny, int nz, float2* in, float2* out, bool forward, hipStream_t s);
const char* normal_apply(const float2* Qhat, int nx, int ny, int nz, float lambda, const float2* p,
                         float2* Ap, float2* P, float2* X, double* partial, hipStream_t s);
const char* cg_run(const float2* Qhat, int nx, int ny, int nz, float lambda, const float2* b,
                   float2* x, int iters, double* resid, const CgWorkspace& w, hipStream_t s);
hipError_t launch_diff_grid(int nx, int ny, int nz, float* x, float* y, float* z, hipStream_t s);
hipError_t launch_scale(float2* v, int64_t n, float f, hipStream_t s);

}  // namespace ncmri
