// Iterative reconstruction on the voxel grid (PMPP ch. 17 "Iterative MRI
// reconstruction", section 17.2 / Fig. 17.3): conjugate gradient on
//
//   (F^H F + lambda W^H W) rho = F^H D,
//
// with F^H F applied through Q (computed once per trajectory).  On a grid with
// unit steps, (F^H F p)[n] = sum_n' Q(x_n - x_n') p[n'] is a convolution with
// Q at the coordinate differences d in (-n, n) per axis.  Embedded in a grid
// of P >= 2n points per axis (Q at d placed at d mod P, zeros elsewhere) it is
// a cyclic convolution, so
//
//   F^H F p = crop( IDFT( Qhat * DFT( zero-pad(p) ) ) ),
//   Qhat    = DFT( embedded Q ) / (Px Py Pz).
//
// Q(-d) = conj(Q(d)), so the embedded grid is Hermitian and Qhat is real; the
// entry at d = -n, never used by the product, is left zero to keep it so.
// Qhat is stored in the order the z pass reads it: the (ky, kx) columns in
// blocks of W = 32 consecutive ones (kx fastest), each block holding its W
// columns point by point along kz (W floats = 128 bytes per kz), so a tile of
// the z pass reads one contiguous 128 KB block (at Pz = 1024) instead of a
// short row in each of Pz planes, which costs an address translation apiece.
//
// The transforms are the library's own line FFTs (fhd_fft.h), one kernel per
// axis, and the product skips what the padding makes trivial:
//   x pass   rows (z < nz, y < ny) of p, zero-extended to Px       -> T
//   y pass   columns (z < nz, kx) of T, zero-extended to Py         -> T
//   z pass   columns (ky, kx): nz points zero-extended to Pz, DFT, times Qhat,
//            inverse DFT, first nz points kept                      -> T
//   y pass   inverse, first ny points kept                          -> T
//   x pass   inverse, first nx points kept, plus lambda W^H W p and the
//            partial sums of <p, Ap>                                -> Ap
// T holds nz planes of Py x Px points; nothing else is stored between passes.
// W is the first-difference stand-in for the pages' anatomical prior: W^H W p
// is the 6-neighbour graph Laplacian.  CG's scalars (<r,r>, <p,Ap>, alpha,
// beta) stay in device memory, so an iteration needs no host synchronisation;
// dot products are accumulated in double with a fixed-order two-stage
// reduction, so results are deterministic.
#include "fhd.h"
#include "fhd_cg.h"
#include "fhd_fft.h"
#include "fhd_lines.h"

namespace ncmri {
namespace {

constexpr int kThreads = 256;
constexpr int kBlocks = kCgPartials;  // grid of every reduction stage 1 (fixed: deterministic sums)
static_assert(kBlocks % 64 == 0, "whole waves of partial sums");
static_assert(kThreads == fft::kThreads, "one block size");

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

// Q(-d) = sum_m |phi_m|^2 exp(-i 2 pi k_m . d) = conj Q(d): the planes with
// dz < 0 (index iz in (nz, 2 nz)) are the conjugates of the computed planes
// dz = -(iz - 2 nz) in [1, nz), with dx, dy negated (index (2n - i) mod 2n).
// Plane iz = nz (dz = -nz) is zeroed, and the entries dx = -nx or dy = -ny
// (index nx or ny, whose negation is not on the grid) take another entry's
// value: the embedding reads only differences |d| < n per axis.
__global__ void __launch_bounds__(kThreads)
hermitian_fill_kernel(float2* __restrict__ Q2, int nx, int ny, int nz) {
  const int64_t plane = (int64_t)4 * nx * ny;
  const int64_t n = plane * nz;                       // planes iz = nz .. 2 nz - 1
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int iz = nz + (int)(i / plane);
    const int64_t r = i - (int64_t)(iz - nz) * plane;
    const int iy = (int)(r / (2 * nx)), ix = (int)(r - (int64_t)iy * 2 * nx);
    float2 v = make_float2(0.0f, 0.0f);
    if (iz > nz) {
      const int sz = 2 * nz - iz, sy = iy == 0 ? 0 : 2 * ny - iy, sx = ix == 0 ? 0 : 2 * nx - ix;
      const float2 q = Q2[((int64_t)sz * 2 * ny + sy) * 2 * nx + sx];
      v = make_float2(q.x, -q.y);
    }
    Q2[(int64_t)iz * plane + r] = v;
  }
}

// Index in the circular 2n grid of the difference held at padded index a
// (a < n: d = a; a > P - n: d = a - P), or -1 where the padded grid is zero.
__device__ __forceinline__ int embed_src(int a, int n, int P) {
  return a < n ? a : (a > P - n ? a - P + 2 * n : -1);
}

__global__ void __launch_bounds__(kThreads)
embed_kernel(const float2* __restrict__ Q2, float2* __restrict__ G, int nx, int ny, int nz, int px, int py,
             int pz) {
  const int64_t total = (int64_t)px * py * pz;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
    const int a1 = (int)(i % px);
    const int a2 = (int)((i / px) % py);
    const int a3 = (int)(i / ((int64_t)px * py));
    const int s1 = embed_src(a1, nx, px), s2 = embed_src(a2, ny, py), s3 = embed_src(a3, nz, pz);
    G[i] = (s1 >= 0 && s2 >= 0 && s3 >= 0) ? Q2[((int64_t)s3 * 2 * ny + s2) * 2 * nx + s1]
                                            : make_float2(0.0f, 0.0f);
  }
}

__global__ void __launch_bounds__(kThreads)
real_scale_kernel(const float2* __restrict__ G, float* __restrict__ Qhat, int64_t n, float scale, int64_t plane,
                  int pz, int shift) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    // G[kz][ky][kx] -> column c = ky px + kx, point kz of its block
    const int64_t z = i / plane, c = i - z * plane;
    Qhat[(c >> shift) * ((int64_t)pz << shift) + (z << shift) + (c & ((1 << shift) - 1))] = G[i].x * scale;
  }
}

// log2 of the spectrum's block width: 32 columns, fewer on grids with fewer.
int spectrum_block_shift(int64_t plane) {
  int s = 0;
  while (s < 5 && ((int64_t)2 << s) <= plane) ++s;
  return s;
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

// Rows (z < nz, y < ny) of T, the first stage's inputs of the last pass.
struct TRows {
  const float2* T;
  int c0, count, ny, py, px;
  template <int RN, int STEP>
  __device__ __forceinline__ void get(int l, int j, float2* w) const {
    const int c = c0 + l;
    const bool ok = c < count;
    const int z = c / ny, y = c - z * ny;
    const float2* t = T + (((int64_t)z * py + y) * px + j);
#pragma unroll
    for (int r = 0; r < RN; ++r) w[r] = ok ? t[r * STEP] : make_float2(0.0f, 0.0f);
  }
};

// Last pass of the normal operator: inverse transforms of the rows (z < nz,
// y < ny) of T, the first nx points of each, plus lambda (W^H W p); writes Ap
// and partial[block] = sum Re(conj(p) Ap) over the block's rows.  Launched on
// kBlocks blocks that stride over the row groups in a fixed order.
template <int N>
__global__ void __launch_bounds__(fft::kThreads)
crop_kernel(const float2* __restrict__ T, int py, const float2* __restrict__ p, float2* __restrict__ Ap,
            int nx, int ny, int nz, float lambda, double* __restrict__ partial) {
  using L = fft::Lds<N, fft::kRows>;
  using S = fft::Sched<N>;
  __shared__ float2 buf[L::kSize];
  __shared__ float2 tw[N];
  __shared__ double sh[kThreads];
  fft::fill_twiddles<N>(tw);
  const int count = ny * nz;
  const int groups = (count + L::kLines - 1) / L::kLines;
  const int64_t plane = (int64_t)nx * ny;
  // nx <= N / 2: only outputs r < RL / 2 of each last-stage butterfly are kept
  constexpr int RL = S::last(false), kStep = N / RL;
  double acc = 0.0;
  for (int g = blockIdx.x; g < groups; g += gridDim.x) {
    const int c0 = g * L::kLines;
    float2 v[fft::kPerThread];
    fft::transform<N, fft::kRows, true, false, false>(TRows{T, c0, count, ny, py, N}, buf, tw, v);
    // the last stage's outputs: point j + r kStep of line c0 + l
#pragma unroll
    for (int k = 0; k < fft::kPerThread / RL; ++k) {
      int l, j;
      fft::locate<N, RL, fft::kRows>(k, l, j);
      const int c = c0 + l;
      if (c >= count) continue;
      const int z = c / ny, y = c - z * ny;
#pragma unroll
      for (int r = 0; r < RL / 2; ++r) {
        const int i = j + r * kStep;
        if (i >= nx) continue;
        const int64_t vox = (int64_t)c * nx + i;
        float2 a = v[k * RL + r];
        const float2 cv = p[vox];
        if (lambda != 0.0f) {
          float lr = 0.0f, li = 0.0f;
          // sum over the existing neighbours of p[vox] - p[neighbour]
          if (i > 0) { const float2 q = p[vox - 1]; lr += cv.x - q.x; li += cv.y - q.y; }
          if (i + 1 < nx) { const float2 q = p[vox + 1]; lr += cv.x - q.x; li += cv.y - q.y; }
          if (y > 0) { const float2 q = p[vox - nx]; lr += cv.x - q.x; li += cv.y - q.y; }
          if (y + 1 < ny) { const float2 q = p[vox + nx]; lr += cv.x - q.x; li += cv.y - q.y; }
          if (z > 0) { const float2 q = p[vox - plane]; lr += cv.x - q.x; li += cv.y - q.y; }
          if (z + 1 < nz) { const float2 q = p[vox + plane]; lr += cv.x - q.x; li += cv.y - q.y; }
          a.x = __builtin_fmaf(lambda, lr, a.x);
          a.y = __builtin_fmaf(lambda, li, a.y);
        }
        Ap[vox] = a;
        acc += (double)cv.x * a.x + (double)cv.y * a.y;
      }
    }
  }
  const double s = block_sum(acc, sh);
  if (threadIdx.x == 0 && partial) partial[blockIdx.x] = s;
}

// CG state slots.  <r, r> alternates between two slots by iteration, so the
// blocks of the direction update can read the old value while one of them
// stores the new one.
enum { RS0 = 0, RS1 = 1, PAP = 2, ALPHA = 3, BETA = 4 };

// Sum of partial[0 .. kBlocks) in a fixed order, formed by every wave on its
// own (no barrier): lane i adds partial[i + 64 k] for k = 0, 1, ..., then an
// xor butterfly over the lanes.  Floating-point addition is commutative, so
// both partners of each butterfly step get the same value: every lane of
// every wave ends with the same bits.
__device__ __forceinline__ double sum_partials(const double* __restrict__ partial) {
  const int lane = threadIdx.x & 63;
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < kBlocks; i += 64) acc += partial[i + lane];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  return acc;
}

// The initial <r, r>: state[RS0] (and resid[0]).
__global__ void __launch_bounds__(kThreads)
initial_rs_kernel(const double* __restrict__ partial, double* __restrict__ state, double* __restrict__ resid) {
  const double s = sum_partials(partial);
  if (threadIdx.x != 0) return;
  state[RS0] = s;
  if (resid) resid[0] = s;
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

// alpha = <r, r> / <p, Ap> (every wave sums the <p, Ap> partials itself, while
// its first elements load); x += alpha p, r -= alpha Ap; rr_partial = sum |r|^2.
__global__ void __launch_bounds__(kThreads)
step_kernel(float2* __restrict__ x, float2* __restrict__ r, const float2* __restrict__ pv,
            const float2* __restrict__ Ap, int64_t n, double* __restrict__ state, int slot,
            const double* __restrict__ pap_partial, double* __restrict__ rr_partial) {
  __shared__ double sh[kThreads];
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  float2 p{}, a{}, xv{}, rv{};
  if (i < n) {
    p = pv[i];
    a = Ap[i];
    xv = x[i];
    rv = r[i];
  }
  const double pap = sum_partials(pap_partial);
  const double alpha_d = pap != 0.0 ? state[RS0 + slot] / pap : 0.0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    state[PAP] = pap;
    state[ALPHA] = alpha_d;
  }
  const float alpha = (float)alpha_d;
  double acc = 0.0;
  while (i < n) {
    xv.x = __builtin_fmaf(alpha, p.x, xv.x);
    xv.y = __builtin_fmaf(alpha, p.y, xv.y);
    rv.x = __builtin_fmaf(-alpha, a.x, rv.x);
    rv.y = __builtin_fmaf(-alpha, a.y, rv.y);
    x[i] = xv;
    r[i] = rv;
    acc += (double)rv.x * rv.x + (double)rv.y * rv.y;
    i += stride;
    if (i < n) {
      p = pv[i];
      a = Ap[i];
      xv = x[i];
      rv = r[i];
    }
  }
  const double s = block_sum(acc, sh);
  if (threadIdx.x == 0) rr_partial[blockIdx.x] = s;
}

// Sum of the partials into *out (the <r, r> after the last iteration).
__global__ void __launch_bounds__(kThreads) store_sum_kernel(const double* __restrict__ partial, double* __restrict__ out) {
  const double s = sum_partials(partial);
  if (threadIdx.x == 0) *out = s;
}

// Rows (z < nz, y < ny) of the new direction p = r + beta p as the first
// stage's inputs of the x transform: each point is read, updated, written
// back to p and handed to the transform exactly once.
struct DirRows {
  const float2* r;
  float2* p;
  float beta;
  int c0, count, nx;
  template <int RN, int STEP>
  __device__ __forceinline__ void get(int l, int j, float2* w) const {
    const int c = c0 + l;
    const bool ok = c < count;
    const int64_t base = (int64_t)(ok ? c : 0) * nx;
#pragma unroll
    for (int q = 0; q < RN; ++q) {
      const int i = j + q * STEP;
      float2 v = make_float2(0.0f, 0.0f);
      if (ok && i < nx) {
        const float2 rv = r[base + i], pv = p[base + i];
        v = make_float2(__builtin_fmaf(beta, pv.x, rv.x), __builtin_fmaf(beta, pv.y, rv.y));
        p[base + i] = v;
      }
      w[q] = v;
    }
  }
};

// First pass of a CG iteration after the first: beta = <r, r>_new / <r, r>_old
// from the step's partials (every wave sums them itself, as in
// step_kernel), p = r + beta p on the rows (z < nz, y < ny), and the
// zero-extended forward transforms of those rows -> rows of T.  The new
// <r, r> goes to the other state slot (and to *resid).  Launched on
// ceil(nz ny / lines) blocks.
template <int N>
__global__ void __launch_bounds__(fft::kThreads)
direction_x_kernel(const float2* __restrict__ r, float2* __restrict__ pv, float2* __restrict__ T, int nx, int ny,
                   int nz, int py, double* __restrict__ state, int slot, const double* __restrict__ rr_partial,
                   double* __restrict__ resid) {
  using L = fft::Lds<N, fft::kRows>;
  using S = fft::Sched<N>;
  __shared__ float2 buf[L::kSize];
  __shared__ float2 tw[N];
  fft::fill_twiddles<N>(tw);
  const double rs_new = sum_partials(rr_partial);
  const double rs = state[RS0 + slot];
  const double beta_d = rs != 0.0 ? rs_new / rs : 0.0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    state[BETA] = beta_d;
    state[RS0 + (slot ^ 1)] = rs_new;
    if (resid) *resid = rs_new;
  }
  const int count = ny * nz;
  const int c0 = blockIdx.x * L::kLines;
  float2 v[fft::kPerThread];
  // nx <= N / 2: the inputs from N/2 on are zero
  fft::transform<N, fft::kRows, false, false, true>(DirRows{r, pv, (float)beta_d, c0, count, nx}, buf, tw, v);
  constexpr int RL = S::last(false), kStep = N / RL;
#pragma unroll
  for (int k = 0; k < fft::kPerThread / RL; ++k) {
    int l, j;
    fft::locate<N, RL, fft::kRows>(k, l, j);
    const int c = c0 + l;
    if (c >= count) continue;
    const int z = c / ny, y = c - z * ny;
    float2* t = T + (((int64_t)z * py + y) * N + j);
#pragma unroll
    for (int q = 0; q < RL; ++q) t[q * kStep] = v[k * RL + q];
  }
}

int blocks_for(int64_t n) {
  const int64_t b = (n + kThreads - 1) / kThreads;
  return (int)(b < kBlocks ? (b > 0 ? b : 1) : kBlocks);
}

template <int N>
hipError_t launch_crop_n(const ToeplitzDims& d, const float2* T, const float2* p, float2* Ap, float lambda,
                         double* partial, hipStream_t s) {
  hipLaunchKernelGGL(crop_kernel<N>, dim3(kBlocks), dim3(fft::kThreads), 0, s, T, d.py, p, Ap, d.nx, d.ny, d.nz,
                     lambda, partial);
  return hipGetLastError();
}

template <int N>
hipError_t launch_direction_x_n(const ToeplitzDims& d, const float2* r, float2* p, float2* T, double* state, int slot,
                                const double* rr_partial, double* resid, hipStream_t s) {
  constexpr int lines = fft::Lds<N, fft::kRows>::kLines;
  const int64_t count = (int64_t)d.ny * d.nz;
  hipLaunchKernelGGL(direction_x_kernel<N>, dim3((unsigned)((count + lines - 1) / lines)), dim3(fft::kThreads), 0, s,
                     r, p, T, d.nx, d.ny, d.nz, d.py, state, slot, rr_partial, resid);
  return hipGetLastError();
}

hipError_t launch_direction_x(const ToeplitzDims& d, const float2* r, float2* p, float2* T, double* state, int slot,
                              const double* rr_partial, double* resid, hipStream_t s) {
  if (2 * d.nx > d.px) return hipErrorInvalidValue;   // the transform reads the first half of each row only
  switch (d.px) {
    case 2: return launch_direction_x_n<2>(d, r, p, T, state, slot, rr_partial, resid, s);
    case 4: return launch_direction_x_n<4>(d, r, p, T, state, slot, rr_partial, resid, s);
    case 8: return launch_direction_x_n<8>(d, r, p, T, state, slot, rr_partial, resid, s);
    case 16: return launch_direction_x_n<16>(d, r, p, T, state, slot, rr_partial, resid, s);
    case 32: return launch_direction_x_n<32>(d, r, p, T, state, slot, rr_partial, resid, s);
    case 64: return launch_direction_x_n<64>(d, r, p, T, state, slot, rr_partial, resid, s);
    case 128: return launch_direction_x_n<128>(d, r, p, T, state, slot, rr_partial, resid, s);
    case 256: return launch_direction_x_n<256>(d, r, p, T, state, slot, rr_partial, resid, s);
    case 512: return launch_direction_x_n<512>(d, r, p, T, state, slot, rr_partial, resid, s);
    case 1024: return launch_direction_x_n<1024>(d, r, p, T, state, slot, rr_partial, resid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_crop(const ToeplitzDims& d, const float2* T, const float2* p, float2* Ap, float lambda,
                       double* partial, hipStream_t s) {
  if (2 * d.nx > d.px) return hipErrorInvalidValue;   // the kernel keeps the first half of each row only
  switch (d.px) {
    case 2: return launch_crop_n<2>(d, T, p, Ap, lambda, partial, s);
    case 4: return launch_crop_n<4>(d, T, p, Ap, lambda, partial, s);
    case 8: return launch_crop_n<8>(d, T, p, Ap, lambda, partial, s);
    case 16: return launch_crop_n<16>(d, T, p, Ap, lambda, partial, s);
    case 32: return launch_crop_n<32>(d, T, p, Ap, lambda, partial, s);
    case 64: return launch_crop_n<64>(d, T, p, Ap, lambda, partial, s);
    case 128: return launch_crop_n<128>(d, T, p, Ap, lambda, partial, s);
    case 256: return launch_crop_n<256>(d, T, p, Ap, lambda, partial, s);
    case 512: return launch_crop_n<512>(d, T, p, Ap, lambda, partial, s);
    case 1024: return launch_crop_n<1024>(d, T, p, Ap, lambda, partial, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_hermitian_fill(int nx, int ny, int nz, float2* Q2, hipStream_t s) {
  const int64_t n = (int64_t)4 * nx * ny * nz;
  hipLaunchKernelGGL(hermitian_fill_kernel, dim3(blocks_for(n)), dim3(kThreads), 0, s, Q2, nx, ny, nz);
  return hipGetLastError();
}

hipError_t launch_diff_grid(int nx, int ny, int nz, float* x, float* y, float* z, hipStream_t s) {
  const int64_t n2 = (int64_t)8 * nx * ny * nz;
  hipLaunchKernelGGL(diff_grid_kernel, dim3(blocks_for(n2)), dim3(kThreads), 0, s, nx, ny, nz, x, y, z);
  return hipGetLastError();
}

const char* toeplitz_spectrum(const ToeplitzDims& d, const float2* Q2, float2* G, float* Qhat, hipStream_t s) {
  const int64_t total = d.spectrum();
  const int64_t plane = (int64_t)d.px * d.py;
  hipLaunchKernelGGL(embed_kernel, dim3(blocks_for(total)), dim3(kThreads), 0, s, Q2, G, d.nx, d.ny, d.nz, d.px,
                     d.py, d.pz);
  if (hipGetLastError() != hipSuccess) return "embed kernel launch failed";
  // x: rows (kz, ky); y: columns (kz, kx); z: columns (ky, kx) -- all in place, full length
  if (launch_lines(true, kLineFwd, d.px, line_pass(G, G, (int64_t)d.pz * d.py, 1, d.px, 0, 1, d.px, d.px), s) != hipSuccess)
    return "x transform launch failed";
  if (launch_lines(false, kLineFwd, d.py, line_pass(G, G, (int64_t)d.pz * d.px, d.px, plane, 1, d.px, d.py, d.py), s) !=
      hipSuccess)
    return "y transform launch failed";
  if (launch_lines(false, kLineFwd, d.pz, line_pass(G, G, plane, 1, 1, 0, plane, d.pz, d.pz), s) != hipSuccess)
    return "z transform launch failed";
  hipLaunchKernelGGL(real_scale_kernel, dim3(blocks_for(total)), dim3(kThreads), 0, s, G, Qhat, total,
                     (float)(1.0 / (double)total), plane, d.pz, spectrum_block_shift(plane));
  if (hipGetLastError() != hipSuccess) return "spectrum scale kernel launch failed";
  return nullptr;
}

// Ap = F^H F p + lambda W^H W p (and the <p, Ap> partials when `partial`).
namespace {

// Passes 2 to 5 of the normal operator, after the x transform of p is in T.
//
// The y transform writes its output to T2 in z-line blocks: the value at
// (z, ky, kx) sits at ((kx >> w) py + ky) W nz + z W + (kx mod W), W = 2^w =
// min(32, px), so the W lines (ky, kx) of a block hold their nz points in one
// contiguous run of W nz values.  The z pass then reads and writes whole
// blocks instead of one short row in each of nz planes a whole plane apart
// (whose address translations missed in the GPU's L1 TLB), and the inverse y
// transform reads the blocks back into T's plane layout.  (Blocks of 16
// lines measured the same at 512^3; blocks of 8 made the y passes' 64-byte
// rows slower.)
LinePass blocked_y_side(LinePass a, const ToeplitzDims& d, bool in) {
  const int w = spectrum_block_shift((int64_t)d.px);   // log2 min(32, px)
  const int64_t W = (int64_t)1 << w;
  if (in) {
    a.in_os = W; a.in_ws = 1; a.in_sh = w; a.in_wh = (int64_t)d.py * W * d.nz; a.in_es = W * d.nz;
  } else {
    a.out_os = W; a.out_ws = 1; a.out_sh = w; a.out_wh = (int64_t)d.py * W * d.nz; a.out_es = W * d.nz;
  }
  return a;
}

const char* normal_apply_rest(const ToeplitzDims& d, const float* Qhat, float lambda, const float2* p, float2* Ap,
                              float2* T, float2* T2, double* partial, hipStream_t s) {
  const int64_t plane = (int64_t)d.px * d.py;
  const int w = spectrum_block_shift((int64_t)d.px);
  const int64_t W = (int64_t)1 << w;
  // y: columns (z < nz, kx) of T, ny points in; py points out into T2's blocks
  LinePass y = blocked_y_side(line_pass(T, T2, (int64_t)d.nz * d.px, d.px, plane, 1, d.px, d.ny, d.py), d, false);
  if (launch_lines(false, kLineFwd, d.py, y, s) != hipSuccess) return "y transform launch failed";
  // z: columns (ky, kx) = line ky px + kx of T2 (in place): nz points, spectral product, nz points back
  LinePass zq = line_pass(T2, T2, plane, d.px, W * d.nz, 1, W, d.nz, d.nz);
  zq.in_sh = zq.out_sh = w;
  zq.in_wh = zq.out_wh = (int64_t)d.py * W * d.nz;
  zq.q = Qhat;
  zq.q_shift = spectrum_block_shift(plane);
  zq.q_bs = (int64_t)d.pz << zq.q_shift;
  if (launch_lines(false, kLineFwdQInv, d.pz, zq, s) != hipSuccess) return "z transform launch failed";
  // y inverse: columns (z, kx) of T2's blocks, py points in; ny out into T's planes
  LinePass yi = blocked_y_side(line_pass(T2, T, (int64_t)d.nz * d.px, d.px, plane, 1, d.px, d.py, d.ny), d, true);
  if (launch_lines(false, kLineInv, d.py, yi, s) != hipSuccess) return "y inverse transform launch failed";
  if (launch_crop(d, T, p, Ap, lambda, partial, s) != hipSuccess) return "x inverse transform launch failed";
  return nullptr;
}

}  // namespace

const char* normal_apply(const ToeplitzDims& d, const float* Qhat, float lambda, const float2* p, float2* Ap,
                         float2* T, float2* T2, double* partial, hipStream_t s) {
  // x: rows (z < nz, y < ny) of p -> rows of T
  LinePass a = line_pass(p, T, (int64_t)d.nz * d.ny, d.ny, 0, 0, 1, d.nx, d.px);
  a.in_os = (int64_t)d.nx * d.ny;
  a.in_ws = d.nx;
  a.out_os = (int64_t)d.px * d.py;
  a.out_ws = d.px;
  if (launch_lines(true, kLineFwd, d.px, a, s) != hipSuccess) return "x transform launch failed";
  return normal_apply_rest(d, Qhat, lambda, p, Ap, T, T2, partial, s);
}

const char* cg_run(const ToeplitzDims& d, const float* Qhat, float lambda, const float2* b, float2* x, int iters,
                   double* resid, const CgWorkspace& w, hipStream_t s) {
  const int64_t n = d.voxels();
  // r = b - A x, p = r, <r, r>
  if (const char* e = normal_apply(d, Qhat, lambda, x, w.Ap, w.T, w.T2, nullptr, s)) return e;
  hipLaunchKernelGGL(residual_kernel, dim3(kBlocks), dim3(kThreads), 0, s, b, w.Ap, w.r, w.p, n, w.partial);
  hipLaunchKernelGGL(initial_rs_kernel, dim3(1), dim3(kThreads), 0, s, w.partial, w.state, resid);
  if (hipGetLastError() != hipSuccess) return "CG kernel launch failed";
  for (int it = 0; it < iters; ++it) {
    const int slot = it & 1;
    if (it == 0) {
      if (const char* e = normal_apply(d, Qhat, lambda, w.p, w.Ap, w.T, w.T2, w.partial, s)) return e;
    } else {
      // p = r + beta p of the previous step, fused with the x transform of p
      if (launch_direction_x(d, w.r, w.p, w.T, w.state, slot ^ 1, w.partial2, resid ? resid + it : nullptr, s) !=
          hipSuccess)
        return "CG direction launch failed";
      if (const char* e = normal_apply_rest(d, Qhat, lambda, w.p, w.Ap, w.T, w.T2, w.partial, s)) return e;
    }
    hipLaunchKernelGGL(step_kernel, dim3(kBlocks), dim3(kThreads), 0, s, x, w.r, w.p, w.Ap, n, w.state, slot,
                       w.partial, w.partial2);
    if (hipGetLastError() != hipSuccess) return "CG kernel launch failed";
  }
  // <r, r> after the last step (its direction update is never needed)
  if (iters > 0 && resid) {
    hipLaunchKernelGGL(store_sum_kernel, dim3(1), dim3(kThreads), 0, s, w.partial2, resid + iters);
    if (hipGetLastError() != hipSuccess) return "CG kernel launch failed";
  }
  return nullptr;
}

}  // namespace ncmri
