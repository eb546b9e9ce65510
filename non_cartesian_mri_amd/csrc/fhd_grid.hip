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
//   image[i] = sum_j G[j] exp(+i 2 pi kappa_j . x_i).
//
// Per axis, (j - n/2)(i - n/2) = j i - (n/2)(i + j) + n^2/4, so the sum is
// i^n (-1)^i IDFT((-1)^j G)[i], and multiplying an inverse DFT's output by
// (-1)^i is the same as rolling its input by n/2; i^n (-1)^(n/2) = 1 for every
// power of two n >= 2.  Hence
//
//   image = IDFT(L),   L[j'] = (-1)^(j'x + j'y + j'z) G[j' - n/2 (mod n, per axis)],
//
// an unnormalised inverse DFT of the rolled, sign-alternated lattice: the x
// transform inside the deposit kernel (a tile holds whole x-rows of a
// plane), then two passes of the library's line FFTs (y, z) in place in the
// output.
//
// The spreading uses no global atomics (scattered float atomics run at a
// fraction of the rate of scattered stores).  A counting sort lists every
// (sample, z plane) deposit under its lattice plane: a sample lands on planes
// jz and jz + 1 (mod nz), so it makes two entries, each holding the sample's
// x / y cell, x / y fractions and Mu times its z weight.  Then one workgroup
// per tile of TY rows of a plane (TY nx <= 4096 cells) adds the entries of its
// plane that touch its rows into the tile, then transforms the tile's rows
// (rolled and sign-alternated: rows of L) along x and writes them once.  The
// tile sums are 64-bit fixed point with LDS integer atomics (on this GPU an LDS float atomic add runs at about a ninth
// of the rate of an integer one): with c the largest |Re| or |Im| of any Mu,
// no cell receives more than M contributions of size <= c, so terms scaled by
// 2^s with M c 2^s < 2^61 cannot overflow, and each term is the double
// product rounded to an integer (relative rounding ~1e-16 for the largest
// terms, far below float32's).  Integer sums do not depend on the order in
// which entries land, so the lattice, and the image, are bitwise
// reproducible.  The lattice cell and fractions come from the float32 k in
// double, so every sample lands in the cells its exact coordinate selects.
#include "fhd.h"
#include "fhd_cg.h"
#include "fhd_fft.h"
#include "fhd_lines.h"

namespace ncmri {
namespace {

constexpr int kThreads = 256;
constexpr int kBinSamples = 512;             // samples per binning block (2 per thread)
constexpr int kPerThread = kBinSamples / kThreads;
constexpr int kTileCells = 4096;             // lattice cells of a deposit tile
constexpr int kMaxPlanes = kToeplitzMaxLen;  // nz <= 1024: one LDS counter per plane
constexpr int kMaxSlots = 64;                // the largest |Mu| component, spread over 64 words

// Cell and fraction of coordinate k on an n-point lattice: u = k n + n/2,
// cell = floor(u) mod n, fraction = u - floor(u).
__device__ __forceinline__ void lattice_cell(float k, int n, int& j, double& f) {
  const double u = (double)k * n + (double)(n / 2);
  const double fl = floor(u);
  f = u - fl;
  int64_t c = (int64_t)fl % n;
  j = (int)(c < 0 ? c + n : c);
}

__device__ __forceinline__ int z_cell(float k, int nz) {
  int j;
  double f;
  lattice_cell(k, nz, j, f);
  return j;
}

__global__ void __launch_bounds__(kThreads) clear_counts(unsigned* __restrict__ count, int nz,
                                                         unsigned* __restrict__ maxbits) {
  for (int b = threadIdx.x; b < nz; b += kThreads) count[b] = 0u;
  if (threadIdx.x < kMaxSlots) maxbits[threadIdx.x] = 0u;
}

// Entries per plane: an LDS histogram per block of kBinSamples samples, then
// one global atomic per plane the block touches.
__global__ void __launch_bounds__(kThreads)
count_kernel(const float* __restrict__ kz, int64_t M, int nz, unsigned* __restrict__ count) {
  __shared__ unsigned hist[kMaxPlanes];
  for (int b = threadIdx.x; b < nz; b += kThreads) hist[b] = 0u;
  __syncthreads();
  const int64_t m0 = (int64_t)blockIdx.x * kBinSamples;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int64_t m = m0 + k * kThreads + threadIdx.x;
    if (m < M) {
      const int jz = z_cell(kz[m], nz);
      atomicAdd(&hist[jz], 1u);
      atomicAdd(&hist[jz + 1 == nz ? 0 : jz + 1], 1u);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < nz; b += kThreads)
    if (hist[b]) atomicAdd(&count[b], hist[b]);
}

// start[b] = cursor[b] = sum of count[b'] over b' < b (one block; nz <= 1024).
__global__ void __launch_bounds__(kThreads)
scan_kernel(const unsigned* __restrict__ count, unsigned* __restrict__ start, unsigned* __restrict__ cursor,
            int nz) {
  __shared__ unsigned part[kThreads];
  constexpr int kPer = kMaxPlanes / kThreads;   // planes per thread
  unsigned v[kPer], run = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = threadIdx.x * kPer + i;
    v[i] = b < nz ? count[b] : 0u;
    run += v[i];
  }
  part[threadIdx.x] = run;
  __syncthreads();
  // inclusive scan of the per-thread totals (Hillis-Steele)
  for (int d = 1; d < kThreads; d *= 2) {
    const unsigned add = (int)threadIdx.x >= d ? part[threadIdx.x - d] : 0u;
    __syncthreads();
    part[threadIdx.x] += add;
    __syncthreads();
  }
  unsigned base = part[threadIdx.x] - run;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = threadIdx.x * kPer + i;
    if (b < nz) {
      start[b] = base;
      cursor[b] = base;
    }
    base += v[i];
  }
}

// The entries: each block ranks its samples per plane in LDS, reserves one
// range per plane with a global atomic, and writes (cell, fractions, value).
// cell = jx | jy << 16; val = (fx, fy, Re, Im of Mu times the z weight).  The
// largest |Re Mu|, |Im Mu| goes to maxbits[block mod 64] (as float bits:
// non-negative floats order like their bit patterns, so an integer max is
// exact and independent of order; 64 words keep the atomics of different
// blocks off one address).
__global__ void __launch_bounds__(kThreads)
fill_kernel(const float* __restrict__ kx, const float* __restrict__ ky, const float* __restrict__ kz,
            const float2* __restrict__ phi, const float2* __restrict__ D, int64_t M, int nx, int ny, int nz,
            unsigned* __restrict__ cursor, unsigned* __restrict__ cell, float4* __restrict__ val,
            unsigned* __restrict__ maxbits) {
  __shared__ unsigned hist[kMaxPlanes];
  __shared__ unsigned base[kMaxPlanes];
  __shared__ unsigned wmax[kThreads / 64];
  for (int b = threadIdx.x; b < nz; b += kThreads) hist[b] = 0u;
  __syncthreads();
  const int64_t m0 = (int64_t)blockIdx.x * kBinSamples;
  int jz[kPerThread];
  unsigned r0[kPerThread], r1[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int64_t m = m0 + k * kThreads + threadIdx.x;
    jz[k] = 0;
    r0[k] = r1[k] = 0u;
    if (m < M) {
      jz[k] = z_cell(kz[m], nz);
      r0[k] = atomicAdd(&hist[jz[k]], 1u);
      r1[k] = atomicAdd(&hist[jz[k] + 1 == nz ? 0 : jz[k] + 1], 1u);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < nz; b += kThreads)
    if (hist[b]) base[b] = atomicAdd(&cursor[b], hist[b]);
  __syncthreads();
  unsigned tmax = 0u;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int64_t m = m0 + k * kThreads + threadIdx.x;
    if (m >= M) continue;
    const float2 p = phi[m], d = D[m];
    // conj(phi) D
    const float mr = __builtin_fmaf(p.x, d.x, p.y * d.y);
    const float mi = __builtin_fmaf(p.x, d.y, -(p.y * d.x));
    const unsigned bits = __float_as_uint(__builtin_fmaxf(__builtin_fabsf(mr), __builtin_fabsf(mi)));
    tmax = bits > tmax ? bits : tmax;
    int jx, jy, jzz;
    double fx, fy, fz;
    lattice_cell(kx[m], nx, jx, fx);
    lattice_cell(ky[m], ny, jy, fy);
    lattice_cell(kz[m], nz, jzz, fz);
    const unsigned c = (unsigned)jx | ((unsigned)jy << 16);
    const float w0 = (float)(1.0 - fz), w1 = (float)fz;
    const unsigned e0 = base[jz[k]] + r0[k];
    const unsigned e1 = base[jz[k] + 1 == nz ? 0 : jz[k] + 1] + r1[k];
    cell[e0] = c;
    val[e0] = make_float4((float)fx, (float)fy, w0 * mr, w0 * mi);
    cell[e1] = c;
    val[e1] = make_float4((float)fx, (float)fy, w1 * mr, w1 * mi);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const unsigned o = __shfl_xor(tmax, m, 64);
    tmax = o > tmax ? o : tmax;
  }
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = tmax;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned b = 0u;
    for (int w = 0; w < kThreads / 64; ++w) b = wmax[w] > b ? wmax[w] : b;
    if (b) atomicMax(&maxbits[blockIdx.x % kMaxSlots], b);
  }
}

// One tile: rows [row0, row0 + TY) of plane z.  The plane's entries that
// touch those rows go into the tile as 64-bit fixed-point sums (LDS integer
// atomics).
__device__ __forceinline__ void add_fixed(unsigned long long* t, int i, double re, double im) {
  atomicAdd(&t[2 * i], (unsigned long long)(long long)__builtin_rint(re));
  atomicAdd(&t[2 * i + 1], (unsigned long long)(long long)__builtin_rint(im));
}

// f = (fx, fy, Re, Im of the value); scale = 2^s.
__device__ __forceinline__ void deposit_entry(unsigned long long* t, unsigned c, const float4& f, int nx, int ny,
                                              int ty, int row0, double scale) {
  const int jx = (int)(c & 0xffffu), jy = (int)(c >> 16);
  const int ra = jy - row0, rb = (jy + 1 == ny ? 0 : jy + 1) - row0;
  const int xb = jx + 1 == nx ? 0 : jx + 1;
  const double vr = (double)f.z * scale, vi = (double)f.w * scale;
  const double wx1 = (double)f.x, wx0 = 1.0 - wx1, wy1 = (double)f.y, wy0 = 1.0 - wy1;
  if ((unsigned)ra < (unsigned)ty) {
    const double a = wx0 * wy0, b = wx1 * wy0;
    add_fixed(t, ra * nx + jx, vr * a, vi * a);
    add_fixed(t, ra * nx + xb, vr * b, vi * b);
  }
  if ((unsigned)rb < (unsigned)ty) {
    const double a = wx0 * wy1, b = wx1 * wy1;
    add_fixed(t, rb * nx + jx, vr * a, vi * a);
    add_fixed(t, rb * nx + xb, vr * b, vi * b);
  }
}

// The deposit with the inverse x transform fused in: a tile holds whole
// x-rows of its plane, so after the fixed-point sums its rows are
// transformed in LDS and written to the image already x-transformed (one
// pass over the lattice fewer).  The row transforms take the first
// Lds<N, kRows>::kThreads threads; the others only keep the barriers in step.
constexpr int kFusedThreads = 512;

// First-stage inputs: point x' of tile row l is L[x'] =
// (-1)^(x' + yr + zr) G[(x' + nx/2) mod nx] (rolled, sign-alternated), from
// the tile's fixed-point sums.
struct TileRows {
  const unsigned long long* tile;
  int nx, ty, row0, ny, zr;
  double unscale;
  template <int RN, int STEP>
  __device__ __forceinline__ void get(int l, int j, float2* w) const {
    const bool ok = l < ty;
    const int yr = (row0 + l + ny / 2) & (ny - 1);
    const int s0 = (yr + zr) & 1;
#pragma unroll
    for (int r = 0; r < RN; ++r) {
      const int xp = j + r * STEP;
      const int k = l * nx + ((xp + nx / 2) & (nx - 1));
      const float re = ok ? (float)((double)(long long)tile[2 * k] * unscale) : 0.0f;
      const float im = ok ? (float)((double)(long long)tile[2 * k + 1] * unscale) : 0.0f;
      w[r] = ((xp + s0) & 1) ? make_float2(-re, -im) : make_float2(re, im);
    }
  }
};

// Last-stage outputs: transformed row l to image[zr][yr][x].
struct ImageRows {
  float2* image;
  int nx, ty, row0, ny, zr;
  template <int RN, int STEP>
  __device__ __forceinline__ void put(int l, int j, const float2* w) const {
    if (l >= ty) return;
    const int yr = (row0 + l + ny / 2) & (ny - 1);
    float2* p = image + (((int64_t)zr * ny + yr) * nx + j);
#pragma unroll
    for (int r = 0; r < RN; ++r) p[r * STEP] = w[r];
  }
};

template <int N>
__global__ void __launch_bounds__(kFusedThreads)
deposit_x_kernel(const unsigned* __restrict__ start, const unsigned* __restrict__ count,
                 const unsigned* __restrict__ cell, const float4* __restrict__ val,
                 const unsigned* __restrict__ maxbits, int64_t M, int ny, int nz, int ty,
                 float2* __restrict__ image) {
  using L = fft::Lds<N, fft::kRows>;
  static_assert(L::kSize * sizeof(float2) <= 2 * kTileCells * sizeof(unsigned long long), "buffer in the tile");
  static_assert(L::kThreads <= kFusedThreads && L::kLines * N == kTileCells, "a tile is one transform group");
  constexpr int nx = N;
  __shared__ unsigned long long tile[2 * kTileCells];   // 64 KB: (Re, Im) per cell
  __shared__ float2 tw[N];
  fft::fill_twiddles<N>(tw);
  const int z = (int)(blockIdx.x % (unsigned)nz), row0 = (int)(blockIdx.x / (unsigned)nz) * ty;
  const int cells = ty * nx;
  for (int i = threadIdx.x; i < 2 * cells; i += kFusedThreads) tile[i] = 0ull;
  unsigned cb = maxbits[threadIdx.x & (kMaxSlots - 1)];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const unsigned o = __shfl_xor(cb, m, 64);
    cb = o > cb ? o : cb;
  }
  const float cmax = __uint_as_float(cb);
  const int e = cmax > 0.0f ? ilogb((double)M * (double)cmax) + 1 : 0;
  const double scale = ldexp(1.0, 61 - e), unscale = ldexp(1.0, e - 61);
  __syncthreads();
  const unsigned e0 = start[z], e1 = e0 + count[z];
  unsigned i = e0 + threadIdx.x;
  for (; (int64_t)i + kFusedThreads < (int64_t)e1; i += 2 * kFusedThreads) {
    const unsigned ca = cell[i], cb2 = cell[i + kFusedThreads];
    const float4 fa = val[i], fb = val[i + kFusedThreads];
    deposit_entry(tile, ca, fa, nx, ny, ty, row0, scale);
    deposit_entry(tile, cb2, fb, nx, ny, ty, row0, scale);
  }
  if (i < e1) deposit_entry(tile, cell[i], val[i], nx, ny, ty, row0, scale);
  __syncthreads();
  const int zr = (z + nz / 2) & (nz - 1);
  if (threadIdx.x < L::kThreads) {
    float2 v[fft::kPerThread];
    // the first stage reads the tile; the exchanges reuse its LDS after a barrier
    fft::transform<N, fft::kRows, true, false, false>(TileRows{tile, nx, ty, row0, ny, zr, unscale},
                                                      reinterpret_cast<float2*>(tile), tw, v);
    fft::last_stage<N, fft::kRows, false, false>(ImageRows{image, nx, ty, row0, ny, zr}, v);
  } else {
    for (int b = 0; b < 2 * (fft::Sched<N>::kStages - 1); ++b) __syncthreads();
  }
}

template <int N>
hipError_t launch_deposit_x(int64_t blocks, const unsigned* start, const unsigned* count, const unsigned* cell,
                            const float4* val, const unsigned* maxbits, int64_t M, int ny, int nz, int ty,
                            float2* image, hipStream_t s) {
  hipLaunchKernelGGL(deposit_x_kernel<N>, dim3((unsigned)blocks), dim3(kFusedThreads), 0, s, start, count, cell,
                     val, maxbits, M, ny, nz, ty, image);
  return hipGetLastError();
}

hipError_t launch_deposit_x_n(int nx, int64_t blocks, const unsigned* start, const unsigned* count,
                              const unsigned* cell, const float4* val, const unsigned* maxbits, int64_t M, int ny,
                              int nz, int ty, float2* image, hipStream_t s) {
  switch (nx) {
    case 2: return launch_deposit_x<2>(blocks, start, count, cell, val, maxbits, M, ny, nz, ty, image, s);
    case 4: return launch_deposit_x<4>(blocks, start, count, cell, val, maxbits, M, ny, nz, ty, image, s);
    case 8: return launch_deposit_x<8>(blocks, start, count, cell, val, maxbits, M, ny, nz, ty, image, s);
    case 16: return launch_deposit_x<16>(blocks, start, count, cell, val, maxbits, M, ny, nz, ty, image, s);
    case 32: return launch_deposit_x<32>(blocks, start, count, cell, val, maxbits, M, ny, nz, ty, image, s);
    case 64: return launch_deposit_x<64>(blocks, start, count, cell, val, maxbits, M, ny, nz, ty, image, s);
    case 128: return launch_deposit_x<128>(blocks, start, count, cell, val, maxbits, M, ny, nz, ty, image, s);
    case 256: return launch_deposit_x<256>(blocks, start, count, cell, val, maxbits, M, ny, nz, ty, image, s);
    case 512: return launch_deposit_x<512>(blocks, start, count, cell, val, maxbits, M, ny, nz, ty, image, s);
    case 1024: return launch_deposit_x<1024>(blocks, start, count, cell, val, maxbits, M, ny, nz, ty, image, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t gridding_scratch_bytes(int64_t M, int nz) {
  const size_t entries = 2 * (size_t)M;
  return entries * sizeof(float4) + cg_align(entries * sizeof(unsigned)) + 3 * cg_align((size_t)nz * sizeof(unsigned)) +
         cg_align(kMaxSlots * sizeof(unsigned));
}

const char* gridding_run(const float* kx, const float* ky, const float* kz, const float2* phi, const float2* D,
                         int64_t M, int nx, int ny, int nz, float2* image, void* scratch, hipStream_t s) {
  if (nx > 0xffff || ny > 0xffff || nz > kMaxPlanes || M < 0 || 2 * M > (int64_t)0xffffffffLL)
    return "gridding sizes out of range";
  const size_t entries = 2 * (size_t)M;
  char* c = (char*)scratch;
  float4* val = (float4*)c;            c += entries * sizeof(float4);
  unsigned* cell = (unsigned*)c;       c += cg_align(entries * sizeof(unsigned));
  unsigned* count = (unsigned*)c;      c += cg_align((size_t)nz * sizeof(unsigned));
  unsigned* start = (unsigned*)c;      c += cg_align((size_t)nz * sizeof(unsigned));
  unsigned* cursor = (unsigned*)c;    c += cg_align((size_t)nz * sizeof(unsigned));
  unsigned* maxbits = (unsigned*)c;
  hipLaunchKernelGGL(clear_counts, dim3(1), dim3(kThreads), 0, s, count, nz, maxbits);
  if (hipGetLastError() != hipSuccess) return "clear kernel launch failed";
  const int64_t bins = (M + kBinSamples - 1) / kBinSamples;
  if (M > 0) {
    hipLaunchKernelGGL(count_kernel, dim3((unsigned)bins), dim3(kThreads), 0, s, kz, M, nz, count);
    if (hipGetLastError() != hipSuccess) return "count kernel launch failed";
  }
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kThreads), 0, s, count, start, cursor, nz);
  if (hipGetLastError() != hipSuccess) return "scan kernel launch failed";
  if (M > 0) {
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)bins), dim3(kThreads), 0, s, kx, ky, kz, phi, D, M, nx, ny, nz,
                       cursor, cell, val, maxbits);
    if (hipGetLastError() != hipSuccess) return "fill kernel launch failed";
  }
  const int ty = ny < kTileCells / nx ? ny : kTileCells / nx;   // powers of two: ty divides ny
  // deposit + inverse x transform of the tile rows, straight into the image
  if (launch_deposit_x_n(nx, (int64_t)nz * (ny / ty), start, count, cell, val, maxbits, M, ny, nz, ty, image, s) !=
      hipSuccess)
    return "deposit kernel launch failed";
  const int64_t plane = (int64_t)nx * ny;
  if (launch_lines(false, kLineInv, ny, line_pass(image, image, (int64_t)nz * nx, nx, plane, 1, nx, ny, ny), s) !=
      hipSuccess)
    return "y transform launch failed";
  if (launch_lines(false, kLineInv, nz, line_pass(image, image, plane, 1, 1, 0, plane, nz, nz), s) != hipSuccess)
    return "z transform launch failed";
  return nullptr;
}

}  // namespace ncmri
