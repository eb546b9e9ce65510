// Internal interface of the reconstruction module (fhd_cg.hip): Toeplitz
// F^H F through the FFT of Q on a padded grid of coordinate differences, the
// regulariser, and conjugate gradient.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace ncmri {

// FFT length along an axis of n voxels: the smallest power of two >= 2n
// (a cyclic convolution of that length holds every difference in (-n, n)).
inline int toeplitz_len(int n) {
  int p = 2;
  while (p < 2 * n) p *= 2;
  return p;
}
constexpr int kToeplitzMaxLen = 1024;   // longest transform the line FFTs take

struct ToeplitzDims {
  int nx, ny, nz;   // image grid
  int px, py, pz;   // transform lengths
  int64_t voxels() const { return (int64_t)nx * ny * nz; }
  int64_t spectrum() const { return (int64_t)px * py * pz; }
  int64_t lines() const { return (int64_t)nz * py * px; }   // the working grid: nz planes of py x px
};
inline ToeplitzDims toeplitz_dims(int nx, int ny, int nz) {
  return ToeplitzDims{nx, ny, nz, toeplitz_len(nx), toeplitz_len(ny), toeplitz_len(nz)};
}

// Device buffers of one CG solve / normal-operator application.
struct CgWorkspace {
  float2* T;        // [nz][py][px] working grid of the transforms
  float2* T2;       // the same nz py px values after the y transform, in z-line blocks (fhd_cg.hip)
  float2* r;        // [n] residual
  float2* p;        // [n] search direction
  float2* Ap;       // [n] operator applied to p
  double* partial;  // [kCgPartials] stage-1 sums of <p, Ap> (and of the initial <r, r>)
  double* partial2; // [kCgPartials] stage-1 sums of <r, r> in the iterations
  double* state;    // [8] <r,r> (two slots), <p,Ap>, alpha, beta
};

constexpr int kCgPartials = 1024;

inline size_t cg_align(size_t b) { return (b + 255) / 256 * 256; }
inline size_t cg_workspace_bytes(const ToeplitzDims& d) {
  return 2 * cg_align((size_t)d.lines() * 8) + 3 * cg_align((size_t)d.voxels() * 8) +
         2 * cg_align(kCgPartials * sizeof(double)) + cg_align(8 * sizeof(double));
}
inline CgWorkspace cg_workspace(void* base, const ToeplitzDims& d) {
  char* c = (char*)base;
  CgWorkspace w;
  w.T = (float2*)c;  c += cg_align((size_t)d.lines() * 8);
  w.T2 = (float2*)c; c += cg_align((size_t)d.lines() * 8);
  w.r = (float2*)c;  c += cg_align((size_t)d.voxels() * 8);
  w.p = (float2*)c;  c += cg_align((size_t)d.voxels() * 8);
  w.Ap = (float2*)c; c += cg_align((size_t)d.voxels() * 8);
  w.partial = (double*)c; c += cg_align(kCgPartials * sizeof(double));
  w.partial2 = (double*)c; c += cg_align(kCgPartials * sizeof(double));
  w.state = (double*)c;
  return w;
}

// Scratch of toeplitz_spectrum: the padded complex grid [pz][py][px].
inline size_t toeplitz_scratch_bytes(const ToeplitzDims& d) { return (size_t)d.spectrum() * 8; }

// Each returns nullptr on success, else a static description of the failure.
// Q2 holds Q on the (2nz, 2ny, 2nx) circular difference grid (index i < n is
// difference i, i >= n is i - 2n); Qhat (real, [pz][py][px]) receives the
// spectrum of its embedding in the padded grid, divided by px py pz.
const char* toeplitz_spectrum(const ToeplitzDims& d, const float2* Q2, float2* G, float* Qhat,
                              hipStream_t s);
const char* normal_apply(const ToeplitzDims& d, const float* Qhat, float lambda, const float2* p,
                         float2* Ap, float2* T, float2* T2, double* partial, hipStream_t s);
const char* cg_run(const ToeplitzDims& d, const float* Qhat, float lambda, const float2* b, float2* x,
                   int iters, double* resid, const CgWorkspace& w, hipStream_t s);
hipError_t launch_diff_grid(int nx, int ny, int nz, float* x, float* y, float* z, hipStream_t s);
// Q2's planes dz < 0 from the planes dz > 0 by Q(-d) = conj Q(d) (only the
// first nz planes of Q2 need computing).
hipError_t launch_hermitian_fill(int nx, int ny, int nz, float2* Q2, hipStream_t s);

// Gridding reconstruction (fhd_grid.hip): image (complex [nz][ny][nx], each
// axis a power of two in [2, kToeplitzMaxLen]) = the centred lattice inverse
// DFT of the trilinearly gridded conj(phi) D.  scratch: gridding_scratch_bytes
// (the sorted deposit entries, two per sample, and the per-plane counts),
// 16-byte aligned.
size_t gridding_scratch_bytes(int64_t M, int nz);
const char* gridding_run(const float* kx, const float* ky, const float* kz, const float2* phi, const float2* D,
                         int64_t M, int nx, int ny, int nz, float2* image, void* scratch, hipStream_t s);

}  // namespace ncmri
