// Gridding reconstruction, the baseline the pages compare the iterative image
// with (PMPP ch. 17 "Iterative MRI reconstruction": section 17.1, Fig. 17.1B,
// and the bilinear gridding/iFFT image of section 17.3 step 3, Fig. 17.19).
//
// Each sample's value Mu = conj(phi) D (the weight of F^H D) is spread onto
// the image's own k-lattice kappa_j = (j - n/2) / n (cycles per voxel, per
// axis) with trilinear weights on the 8 lattice points around it; the lattice
// is periodic with period 1 (voxel coordinates are integers), so neighbours
// wrap.  The image at voxel coordinates x_i = i - n/2 is then
//
//   image[i] = sum_j G[j] exp(+i 2 pi kappa_j . x_i)
//            = s (-1)^(ix+iy+iz) IDFT( (-1)^(jx+jy+jz) G )[i],   s = prod_axes i^n,
//
// an unnormalised inverse DFT of the sign-alternated lattice (the centring of
// both index sets), run as three passes of the library's line FFTs in place
// in the output.  Deposits are float atomics, so the rounding of a lattice
// value depends on the order in which samples land (results are not
// bitwise reproducible); the lattice position and weights are computed in
// double from the float32 k, so every sample lands in the cells its exact
// coordinate selects.
#include "fhd.h"
#include "fhd_cg.h"
#include "fhd_lines.h"

namespace ncmri {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 4096;

__global__ void __launch_bounds__(kThreads) zero_kernel(float2* __restrict__ a, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    a[i] = make_float2(0.0f, 0.0f);
}

// Cell and fraction of coordinate k on an n-point lattice: u = k n + n/2,
// cell = floor(u) mod n, fraction = u - floor(u).
__device__ __forceinline__ void lattice_cell(float k, int n, int& j, double& f) {
  const double u = (double)k * n + (double)(n / 2);
  const double fl = floor(u);
  f = u - fl;
  int64_t c = (int64_t)fl % n;
  j = (int)(c < 0 ? c + n : c);
}

__global__ void __launch_bounds__(kThreads)
scatter_kernel(const float* __restrict__ kx, const float* __restrict__ ky, const float* __restrict__ kz,
               const float2* __restrict__ phi, const float2* __restrict__ D, int64_t M, int nx, int ny, int nz,
               float2* __restrict__ G) {
  float* g = reinterpret_cast<float*>(G);
  for (int64_t m = (int64_t)blockIdx.x * kThreads + threadIdx.x; m < M; m += (int64_t)gridDim.x * kThreads) {
    const float2 p = phi[m], d = D[m];
    // conj(phi) D
    const float mr = __builtin_fmaf(p.x, d.x, p.y * d.y);
    const float mi = __builtin_fmaf(p.x, d.y, -(p.y * d.x));
    int jx, jy, jz;
    double fx, fy, fz;
    lattice_cell(kx[m], nx, jx, fx);
    lattice_cell(ky[m], ny, jy, fy);
    lattice_cell(kz[m], nz, jz, fz);
#pragma unroll
    for (int dz = 0; dz < 2; ++dz) {
      const int cz = jz + dz == nz ? 0 : jz + dz;
      const double wz = dz ? fz : 1.0 - fz;
#pragma unroll
      for (int dy = 0; dy < 2; ++dy) {
        const int cy = jy + dy == ny ? 0 : jy + dy;
        const double wy = dy ? fy : 1.0 - fy;
#pragma unroll
        for (int dx = 0; dx < 2; ++dx) {
          const int cx = jx + dx == nx ? 0 : jx + dx;
          const double wx = dx ? fx : 1.0 - fx;
          float w = (float)(wx * wy * wz);
          if ((cx + cy + cz) & 1) w = -w;
          const int64_t idx = ((int64_t)cz * ny + cy) * nx + cx;
          unsafeAtomicAdd(g + 2 * idx, w * mr);
          unsafeAtomicAdd(g + 2 * idx + 1, w * mi);
        }
      }
    }
  }
}

// image[i] *= s (-1)^(ix+iy+iz)
__global__ void __launch_bounds__(kThreads)
sign_kernel(float2* __restrict__ a, int nx, int ny, int nz, float s) {
  const int64_t n = (int64_t)nx * ny * nz;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int ix = (int)(i % nx), iy = (int)((i / nx) % ny), iz = (int)(i / ((int64_t)nx * ny));
    const float f = ((ix + iy + iz) & 1) ? -s : s;
    const float2 v = a[i];
    a[i] = make_float2(v.x * f, v.y * f);
  }
}

int blocks(int64_t n) {
  const int64_t b = (n + kThreads - 1) / kThreads;
  return (int)(b < kMaxBlocks ? (b > 0 ? b : 1) : kMaxBlocks);
}

// i^n for a power of two n >= 2: -1 for n = 2, +1 otherwise
float quarter_power(int n) { return n % 4 == 0 ? 1.0f : -1.0f; }

}  // namespace

const char* gridding_run(const float* kx, const float* ky, const float* kz, const float2* phi, const float2* D,
                         int64_t M, int nx, int ny, int nz, float2* image, hipStream_t s) {
  const int64_t n = (int64_t)nx * ny * nz;
  hipLaunchKernelGGL(zero_kernel, dim3(blocks(n)), dim3(kThreads), 0, s, image, n);
  if (hipGetLastError() != hipSuccess) return "zero kernel launch failed";
  if (M > 0) {
    hipLaunchKernelGGL(scatter_kernel, dim3(blocks(M)), dim3(kThreads), 0, s, kx, ky, kz, phi, D, M, nx, ny, nz,
                       image);
    if (hipGetLastError() != hipSuccess) return "scatter kernel launch failed";
  }
  const int64_t plane = (int64_t)nx * ny;
  if (launch_lines(true, kLineInv, nx, line_pass(image, image, (int64_t)nz * ny, 1, nx, 0, 1, nx, nx), s) !=
      hipSuccess)
    return "x transform launch failed";
  if (launch_lines(false, kLineInv, ny, line_pass(image, image, (int64_t)nz * nx, nx, plane, 1, nx, ny, ny), s) !=
      hipSuccess)
    return "y transform launch failed";
  if (launch_lines(false, kLineInv, nz, line_pass(image, image, plane, 1, 1, 0, plane, nz, nz), s) != hipSuccess)
    return "z transform launch failed";
  const float sg = quarter_power(nx) * quarter_power(ny) * quarter_power(nz);
  hipLaunchKernelGGL(sign_kernel, dim3(blocks(n)), dim3(kThreads), 0, s, image, nx, ny, nz, sg);
  if (hipGetLastError() != hipSuccess) return "sign kernel launch failed";
  return nullptr;
}

}  // namespace ncmri
