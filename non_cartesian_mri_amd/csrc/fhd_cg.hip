// Iterative reconstruction on the voxel grid (PMPP ch. 17 "Iterative MRI
// reconstruction", section 17.2 / Fig. 17.3): conjugate gradient on
//
//   (F^H F + lambda W^H W) rho = F^H D,
//
// with F^H F applied through Q (computed once per trajectory).  On a grid with
// unit steps, (F^H F p)[n] = sum_n' Q(x_n - x_n') p[n'] is a convolution with
// Q at the coordinate differences d in (-n, n) per axis; embedded circularly
// in a grid of twice the size it is a cyclic convolution, so
//
//   F^H F p = crop( IFFT( Qhat * FFT( zero-pad(p) ) ) ),
//   Qhat    = FFT( Q on the 2n grid of differences, circular order ) / (8 nx ny nz).
//
// Q comes from the library's own Q path (q_compute on the difference grid:
// the matrix-core engine, since the circular grid's rows still hold whole
// voxel groups); the FFTs are hipFFT library calls; the padding, spectral
// product, crop, regulariser and every CG step are the kernels below.  W is
// the first-difference stand-in for the pages' anatomical prior: W^H W p is
// the 6-neighbour graph Laplacian.  CG's scalars (<r,r>, <p,Ap>, alpha, beta)
// stay in device memory, so an iteration needs no host synchronisation; dot
// products are accumulated in double with a fixed-order two-stage reduction,
// so results are deterministic.
#include "fhd.h"
#include "fhd_cg.h"

#include <hipfft/hipfft.h>

#include <map>
#include <mutex>
#include <tuple>

namespace ncmri {
namespace {

constexpr int kThreads = 256;
constexpr int kBlocks = kCgPartials;  // grid of every reduction stage 1 (fixed: deterministic sums)

// Circular coordinates of the difference grid: index i < n is d = i, i >= n is d = i - 2n.
__global__ void __launch_bounds__(kThreads)
diff_grid_kernel(int nx, int ny, int nz, float* x, float* y, float* z) {
  const int64_t n2 = (int64_t)8 * nx * ny * nz;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n2; i += (int64_t)gridDim.x * kThreads) {
    const int ix = (int)(i % (2 * nx));
    const int iy = (int)((i / (2 * nx)) % (2 * ny));
    const int iz = (int)(i / ((int64_t)4 * nx * ny));
    x[i] = (float)(ix < nx ? ix : ix - 2 * nx);
    y[i] = (float)(iy < ny ? iy : iy - 2 * ny);
    z[i] = (float)(iz < nz ? iz : iz - 2 * nz);
  }
}

__global__ void __launch_bounds__(kThreads) scale_kernel(float2* v, int64_t n, float s) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const float2 a = v[i];
    v[i] = make_float2(a.x * s, a.y * s);
  }
}

// P (2nz x 2ny x 2nx) = p in the low corner, zeros elsewhere.
__global__ void __launch_bounds__(kThreads)
pad_kernel(const float2* __restrict__ p, float2* __restrict__ P, int nx, int ny, int nz) {
  const int64_t n2 = (int64_t)8 * nx * ny * nz;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n2; i += (int64_t)gridDim.x * kThreads) {
    const int ix = (int)(i % (2 * nx));
    const int iy = (int)((i / (2 * nx)) % (2 * ny));
    const int iz = (int)(i / ((int64_t)4 * nx * ny));
    P[i] = (ix < nx && iy < ny && iz < nz) ? p[((int64_t)iz * ny + iy) * nx + ix] : make_float2(0.0f, 0.0f);
  }
}

// X *= Qhat (complex).
__global__ void __launch_bounds__(kThreads)
spectral_kernel(float2* __restrict__ X, const float2* __restrict__ Qhat, int64_t n2) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n2; i += (int64_t)gridDim.x * kThreads) {
    const float2 a = X[i], q = Qhat[i];
    X[i] = make_float2(a.x * q.x - a.y * q.y, a.x * q.y + a.y * q.x);
  }
}

// Block sum of a double in LDS (fixed tree: deterministic).
__device__ double block_sum(double v, double* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

// Ap = crop(P) + lambda (W^H W p); partial[block] = sum Re(conj(p) Ap).
__global__ void __launch_bounds__(kThreads)
crop_kernel(const float2* __restrict__ P, const float2* __restrict__ p, float2* __restrict__ Ap,
            int nx, int ny, int nz, float lambda, double* __restrict__ partial) {
  __shared__ double sh[kThreads];
  const int64_t n = (int64_t)nx * ny * nz;
  double acc = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int ix = (int)(i % nx);
    const int iy = (int)((i / nx) % ny);
    const int iz = (int)(i / ((int64_t)nx * ny));
    float2 v = P[((int64_t)iz * 2 * ny + iy) * 2 * nx + ix];
    const float2 c = p[i];
    if (lambda != 0.0f) {
      float lr = 0.0f, li = 0.0f;
      // sum over the existing neighbours of p[i] - p[neighbour]
      if (ix > 0) { const float2 q = p[i - 1]; lr += c.x - q.x; li += c.y - q.y; }
      if (ix + 1 < nx) { const float2 q = p[i + 1]; lr += c.x - q.x; li += c.y - q.y; }
      if (iy > 0) { const float2 q = p[i - nx]; lr += c.x - q.x; li += c.y - q.y; }
      if (iy + 1 < ny) { const float2 q = p[i + nx]; lr += c.x - q.x; li += c.y - q.y; }
      if (iz > 0) { const float2 q = p[i - (int64_t)nx * ny]; lr += c.x - q.x; li += c.y - q.y; }
      if (iz + 1 < nz) { const float2 q = p[i + (int64_t)nx * ny]; lr += c.x - q.x; li += c.y - q.y; }
      v.x = __builtin_fmaf(lambda, lr, v.x);
      v.y = __builtin_fmaf(lambda, li, v.y);
    }
    Ap[i] = v;
    acc += (double)c.x * v.x + (double)c.y * v.y;
  }
  const double s = block_sum(acc, sh);
  if (threadIdx.x == 0 && partial) partial[blockIdx.x] = s;
}

// Sums kBlocks partials in fixed order into a CG state slot, then derives:
//   what 0: state[RS] = sum (and resid[0])                        -- initial <r, r>
//   what 1: state[PAP] = sum, state[ALPHA] = state[RS] / sum      -- after A p
//   what 2: state[BETA] = sum / state[RS], state[RS] = sum (and resid[it])
enum { RS = 0, PAP = 1, ALPHA = 2, BETA = 3 };
__global__ void __launch_bounds__(kThreads)
finalize_kernel(const double* __restrict__ partial, double* __restrict__ state, int what,
                double* __restrict__ resid) {
  __shared__ double sh[kThreads];
  double acc = 0.0;
  for (int i = threadIdx.x; i < kBlocks; i += kThreads) acc += partial[i];
  const double s = block_sum(acc, sh);
  if (threadIdx.x != 0) return;
  if (what == 0) {
    state[RS] = s;
    if (resid) resid[0] = s;
  } else if (what == 1) {
    state[PAP] = s;
    state[ALPHA] = s != 0.0 ? state[RS] / s : 0.0;
  } else {
    state[BETA] = state[RS] != 0.0 ? s / state[RS] : 0.0;
    state[RS] = s;
    if (resid) *resid = s;
  }
}

// r = b - Ax, p = r; partial = sum |r|^2.
__global__ void __launch_bounds__(kThreads)
residual_kernel(const float2* __restrict__ b, const float2* __restrict__ Ax, float2* __restrict__ r,
                float2* __restrict__ pv, int64_t n, double* __restrict__ partial) {
  __shared__ double sh[kThreads];
  double acc = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const float2 v = make_float2(b[i].x - Ax[i].x, b[i].y - Ax[i].y);
    r[i] = v;
    pv[i] = v;
    acc += (double)v.x * v.x + (double)v.y * v.y;
  }
  const double s = block_sum(acc, sh);
  if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

// x += alpha p, r -= alpha Ap; partial = sum |r|^2.
__global__ void __launch_bounds__(kThreads)
step_kernel(float2* __restrict__ x, float2* __restrict__ r, const float2* __restrict__ pv,
            const float2* __restrict__ Ap, int64_t n, const double* __restrict__ state,
            double* __restrict__ partial) {
  __shared__ double sh[kThreads];
  const float alpha = (float)state[ALPHA];
  double acc = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const float2 p = pv[i], a = Ap[i];
    float2 xv = x[i], rv = r[i];
    xv.x = __builtin_fmaf(alpha, p.x, xv.x);
    xv.y = __builtin_fmaf(alpha, p.y, xv.y);
    rv.x = __builtin_fmaf(-alpha, a.x, rv.x);
    rv.y = __builtin_fmaf(-alpha, a.y, rv.y);
    x[i] = xv;
    r[i] = rv;
    acc += (double)rv.x * rv.x + (double)rv.y * rv.y;
  }
  const double s = block_sum(acc, sh);
  if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

// p = r + beta p.
__global__ void __launch_bounds__(kThreads)
direction_kernel(const float2* __restrict__ r, float2* __restrict__ pv, int64_t n,
                 const double* __restrict__ state) {
  const float beta = (float)state[BETA];
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const float2 rv = r[i], p = pv[i];
    pv[i] = make_float2(__builtin_fmaf(beta, p.x, rv.x), __builtin_fmaf(beta, p.y, rv.y));
  }
}

int blocks_for(int64_t n) {
  const int64_t b = (n + kThreads - 1) / kThreads;
  return (int)(b < kBlocks ? (b > 0 ? b : 1) : kBlocks);
}

// hipFFT plans for (2nz, 2ny, 2nx) C2C, one per device, stream and size, kept
// until the process ends (plan creation is expensive).  A plan's work area is
// used by every transform run with it, so plans are not shared across streams:
// work on different streams may overlap, work on one stream is ordered.
std::mutex g_plan_mu;
std::map<std::tuple<int, hipStream_t, int, int, int>, hipfftHandle> g_plans;

const char* fft_name(hipfftResult r) {
  switch (r) {
    case HIPFFT_SUCCESS: return "HIPFFT_SUCCESS";
    case HIPFFT_ALLOC_FAILED: return "HIPFFT_ALLOC_FAILED";
    case HIPFFT_INVALID_VALUE: return "HIPFFT_INVALID_VALUE";
    case HIPFFT_INVALID_SIZE: return "HIPFFT_INVALID_SIZE";
    case HIPFFT_EXEC_FAILED: return "HIPFFT_EXEC_FAILED";
    default: return "hipFFT error";
  }
}

}  // namespace

// Runs one C2C transform of the (2nz, 2ny, 2nx) grid on `stream`.
const char* fft3(int nx, int ny, int nz, float2* in, float2* out, bool forward, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return "hipGetDevice failed";
  std::lock_guard<std::mutex> lk(g_plan_mu);
  auto key = std::make_tuple(dev, stream, nx, ny, nz);
  auto it = g_plans.find(key);
  hipfftHandle plan;
  if (it == g_plans.end()) {
    hipfftResult r = hipfftPlan3d(&plan, 2 * nz, 2 * ny, 2 * nx, HIPFFT_C2C);
    if (r != HIPFFT_SUCCESS) return fft_name(r);
    g_plans[key] = plan;
  } else {
    plan = it->second;
  }
  hipfftResult r = hipfftSetStream(plan, stream);
  if (r != HIPFFT_SUCCESS) return fft_name(r);
  r = hipfftExecC2C(plan, reinterpret_cast<hipfftComplex*>(in), reinterpret_cast<hipfftComplex*>(out),
                    forward ? HIPFFT_FORWARD : HIPFFT_BACKWARD);
  return r == HIPFFT_SUCCESS ? nullptr : fft_name(r);
}

hipError_t launch_diff_grid(int nx, int ny, int nz, float* x, float* y, float* z, hipStream_t s) {
  const int64_t n2 = (int64_t)8 * nx * ny * nz;
  hipLaunchKernelGGL(diff_grid_kernel, dim3(blocks_for(n2)), dim3(kThreads), 0, s, nx, ny, nz, x, y, z);
  return hipGetLastError();
}

hipError_t launch_scale(float2* v, int64_t n, float f, hipStream_t s) {
  hipLaunchKernelGGL(scale_kernel, dim3(blocks_for(n)), dim3(kThreads), 0, s, v, n, f);
  return hipGetLastError();
}

// Ap = F^H F p + lambda W^H W p (and the <p, Ap> partials when `partial`).
const char* normal_apply(const float2* Qhat, int nx, int ny, int nz, float lambda, const float2* p,
                         float2* Ap, float2* P, float2* X, double* partial, hipStream_t s) {
  const int64_t n = (int64_t)nx * ny * nz, n2 = 8 * n;
  hipLaunchKernelGGL(pad_kernel, dim3(blocks_for(n2)), dim3(kThreads), 0, s, p, P, nx, ny, nz);
  if (hipGetLastError() != hipSuccess) return "pad kernel launch failed";
  if (const char* e = fft3(nx, ny, nz, P, X, true, s)) return e;
  hipLaunchKernelGGL(spectral_kernel, dim3(blocks_for(n2)), dim3(kThreads), 0, s, X, Qhat, n2);
  if (hipGetLastError() != hipSuccess) return "spectral kernel launch failed";
  if (const char* e = fft3(nx, ny, nz, X, P, false, s)) return e;
  hipLaunchKernelGGL(crop_kernel, dim3(kBlocks), dim3(kThreads), 0, s, P, p, Ap, nx, ny, nz, lambda, partial);
  if (hipGetLastError() != hipSuccess) return "crop kernel launch failed";
  return nullptr;
}

const char* cg_run(const float2* Qhat, int nx, int ny, int nz, float lambda, const float2* b,
                   float2* x, int iters, double* resid, const CgWorkspace& w, hipStream_t s) {
  const int64_t n = (int64_t)nx * ny * nz;
  // r = b - A x, p = r, <r, r>
  if (const char* e = normal_apply(Qhat, nx, ny, nz, lambda, x, w.Ap, w.P, w.X, nullptr, s)) return e;
  hipLaunchKernelGGL(residual_kernel, dim3(kBlocks), dim3(kThreads), 0, s, b, w.Ap, w.r, w.p, n, w.partial);
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(kThreads), 0, s, w.partial, w.state, 0, resid);
  if (hipGetLastError() != hipSuccess) return "CG kernel launch failed";
  for (int it = 0; it < iters; ++it) {
    if (const char* e = normal_apply(Qhat, nx, ny, nz, lambda, w.p, w.Ap, w.P, w.X, w.partial, s)) return e;
    hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(kThreads), 0, s, w.partial, w.state, 1, nullptr);
    hipLaunchKernelGGL(step_kernel, dim3(kBlocks), dim3(kThreads), 0, s, x, w.r, w.p, w.Ap, n, w.state, w.partial);
    hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(kThreads), 0, s, w.partial, w.state, 2,
                       resid ? resid + it + 1 : nullptr);
    hipLaunchKernelGGL(direction_kernel, dim3(blocks_for(n)), dim3(kThreads), 0, s, w.r, w.p, n, w.state);
    if (hipGetLastError() != hipSuccess) return "CG kernel launch failed";
  }
  return nullptr;
}

}  // namespace ncmri
