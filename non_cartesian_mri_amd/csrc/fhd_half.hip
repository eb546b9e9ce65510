// gfx950 half-split matrix-core engine for F^H D and Q (PMPP ch. 17
// "Iterative MRI reconstruction", section 17.3): the grid-factored sum of
// the four-sample engine (groups of 128 / vectors voxels, 16 groups per
// wave, the three real products P1 = sum (c + s) fr, P2 = sum (c - s) fi,
// P3 = sum s (fr + fi)), with every fp32 product formed from fp16 parts on
// the fp16 matrix cores: x = hi + lo, hi = fp16(x), lo = fp16(x - hi), and
// x y ~ hi_x hi_y + hi_x lo_y + lo_x hi_y, accumulated in fp32 by
// v_mfma_f32_16x16x32_f16 (K = 32 samples).  The dropped lo lo term and lo's
// rounding leave ~2^-22 relative error per product (fp32: 2^-24).  This is
// the split-precision emulation of fp32 products on half-precision matrix
// units (Markidis et al. 2018; Ootomo and Yokota 2022).
//
// The factor side (fr, fi, fr + fi = Mu e^{i 2 pi k.d}) is scaled by a power
// of two that puts its largest part near 2^14 and unscaled at the store (both
// exact); the group side (c + s, c - s, s) lies within +-sqrt(2).
//
// Data flow as in the fp32 engines: per 32-sample chunk the factor parts of
// all 8 tiles (48 KB) are copied once per 8-wave workgroup into LDS by LDS
// DMA, double-buffered; each lane evaluates the phases of its group at 8
// samples of the chunk and splits (c + s, c - s, s) into the A operands;
// each tile takes 9 MFMAs per chunk (hi hi, hi lo, lo hi for each product).
// Waves off the common offsets run per voxel in fp32 (half_direct_kernel).
#include "fhd_internal.h"
#include "fhd_trig.h"
#include "fhd_mfma_common.h"
#include "fhd_groups.h"
#include "fhd_half_common.h"

namespace ncmri {
namespace {

using MfmaFn = void (*)(MfmaArgs);
using DirectFn = void (*)(MfmaArgs);

// The factors' scale: 2^e with sqrt(2) max_m,b |Mu_b[m]| 2^e <= 2^14, so that
// every factor part (|fr|, |fi| <= |Mu|, |fr + fi| <= sqrt(2) |Mu|) stays
// below fp16's 65504 with room for rounding.  Two passes: kHalfScaleBlocks
// workgroups write the largest |Mu_b[m]| of their samples to scale[2 + w],
// then one workgroup takes the largest of those (a maximum: order-free).
constexpr int kHalfScaleBlocks = 256;

__global__ void __launch_bounds__(256)
half_scale_partial_kernel(MfmaRecordArgs a, int is_q, int BC, float* __restrict__ scale) {
  __shared__ float sh[256];
  float mx = 0.0f;
  for (int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x; m < a.M; m += (int64_t)kHalfScaleBlocks * 256) {
    const double pr = a.phi[m].x, pim = a.phi[m].y;
    for (int b = 0; b < BC; ++b) {
      double mr, mi;
      if (is_q) {
        mr = pr * pr + pim * pim;
        mi = 0.0;
      } else {
        const float2 d = a.D[(int64_t)b * a.M + m];
        mr = pr * d.x + pim * d.y;
        mi = pr * d.y - pim * d.x;
      }
      const float v = (float)sqrt(mr * mr + mi * mi);
      mx = v > mx ? v : mx;
    }
  }
  sh[threadIdx.x] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] = sh[threadIdx.x] > sh[threadIdx.x + s] ? sh[threadIdx.x] : sh[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) scale[2 + blockIdx.x] = sh[0];
}

__global__ void __launch_bounds__(256) half_scale_kernel(float* __restrict__ scale) {
  __shared__ float sh[256];
  sh[threadIdx.x] = scale[2 + threadIdx.x];
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] = sh[threadIdx.x] > sh[threadIdx.x + s] ? sh[threadIdx.x] : sh[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    // max |Mu| rounded to fp32: the largest part ends in [2^13, 2^14), far
    // under fp16's 65504, so the rounding is harmless
    const double top = 1.4142135623730951 * (double)sh[0];   // bound of every factor part
    int e = 0;
    if (top > 0.0 && isfinite(top)) {
      e = 14 - ilogb(top) - 1;
      e = e < -120 ? -120 : (e > 120 ? 120 : e);
    }
    scale[0] = ldexpf(1.0f, e);
    scale[1] = ldexpf(1.0f, -e);
  }
}

// Records: one lane per (octet of samples o, complex column cc < 128): the
// factors of column cc for samples 8 o .. 8 o + 7, scaled and split, as the
// six 16-byte B parts of lane c + 16 (o % 4) of tile t = cc / 16 in block
// o / 4.  Column cc holds vector b = cc / V at offset j = cc % V; the lanes
// with j = 0 also write Mu_b in fp32, and those of column 0 the headers.
__global__ void __launch_bounds__(kWorkgroup)
half_records_kernel(HalfRecordArgs h, int is_q, int trig, int BC) {
  const MfmaRecordArgs& a = h.r;
  const int64_t idx = (int64_t)blockIdx.x * kWorkgroup + threadIdx.x;
  const int64_t o = idx >> 7;
  const int cc = (int)(idx & 127);
  if (o * 8 >= a.mpad) return;
  const int V = 128 / BC, b = cc / V, j = cc % V;
  const int HF = mfma_header_floats(trig);
  const float sc = h.scale[0];
  const double x0 = a.x[0], y0 = a.y[0], z0 = a.z[0];
  const double dx = j < a.N ? (double)a.x[j] - x0 : 0.0, dy = j < a.N ? (double)a.y[j] - y0 : 0.0,
               dz = j < a.N ? (double)a.z[j] - z0 : 0.0;
  half8 part[3][2];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t m = o * 8 + e;
    double vr = 0.0, vi = 0.0;
    if (m < a.M) {
      const float kx = a.kx[m], ky = a.ky[m], kz = a.kz[m];
      const double pr = a.phi[m].x, pim = a.phi[m].y;
      double mr, mi;
      if (is_q) {
        mr = pr * pr + pim * pim;
        mi = 0.0;
      } else {
        const float2 d = a.D[(int64_t)b * a.M + m];
        mr = pr * d.x + pim * d.y;  // Mu = conj(phi) * D
        mi = pr * d.y - pim * d.x;
      }
      double cj = 1.0, sj = 0.0;
      if (j > 0 && j < a.N) sincospi(2.0 * ((double)kx * dx + (double)ky * dy + (double)kz * dz), &sj, &cj);
      vr = mr * cj - mi * sj;
      vi = mr * sj + mi * cj;
      if (j == 0) h.mu[m * BC + b] = make_float2((float)mr, (float)mi);
      if (cc == 0) {
        float* hp = a.hdr + m * HF;
        if (trig == kTrigHw) {
          hp[0] = kx; hp[1] = ky; hp[2] = kz; hp[3] = 0.0f;
        } else {
          const float khx = __builtin_rintf(kx * 4096.0f) * (1.0f / 4096.0f);
          const float khy = __builtin_rintf(ky * 4096.0f) * (1.0f / 4096.0f);
          const float khz = __builtin_rintf(kz * 4096.0f) * (1.0f / 4096.0f);
          hp[0] = khx; hp[1] = khy; hp[2] = khz; hp[3] = 0.0f;
          hp[4] = kx - khx; hp[5] = ky - khy; hp[6] = kz - khz; hp[7] = 0.0f;
        }
      }
    } else if (m < a.mpad) {  // padding sample: contributes exactly zero
      if (j == 0) h.mu[m * BC + b] = make_float2(0.0f, 0.0f);
      if (cc == 0)
        for (int i = 0; i < HF; ++i) a.hdr[m * HF + i] = 0.0f;
    }
    // scaled products (fr, fi, fr + fi), each rounded once to fp32, then split
    const float v[3] = {(float)(vr * sc), (float)(vi * sc), (float)((vr + vi) * sc)};
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      _Float16 hi, lo;
      split_half(v[u], hi, lo);
      part[u][0][e] = hi;
      part[u][1][e] = lo;
    }
  }
  const int64_t q = o >> 2;
  const int t = cc >> 4, lane = (cc & 15) + 16 * (int)(o & 3);
  uint4* w = reinterpret_cast<uint4*>(h.wh);
#pragma unroll
  for (int u = 0; u < 3; ++u)
#pragma unroll
    for (int s = 0; s < 2; ++s)
      w[(((q * 8 + t) * 3 + u) * 2 + s) * 64 + lane] = *reinterpret_cast<const uint4*>(&part[u][s]);
}

// Gather (regular waves): a wave owns 16 groups of V = 128 / BC voxels; per
// 32-sample chunk each lane evaluates the phases of its group (lane % 16) at
// samples 8 (lane / 16) .. + 7, splits (c + s, c - s, s) into A parts, and
// for each tile t reads the six B parts from LDS and issues 9 MFMAs (the
// three products, each as hi hi + hi lo + lo hi).  Chunks are staged into LDS
// by LDS DMA, double buffered, shared by the 8 waves of the workgroup.
// FOLD: tiles of a.tile samples are folded (as Re, Im) into running totals
// (blocked summation within the row); without it the launch row is one
// summation block.  Rows are added by the reduction kernel in a fixed order.
template <int BC, int TRIG, bool FOLD>
struct HalfGather {
  static constexpr int T = 8;
  static constexpr int V = 16 * T / BC;
  static constexpr int HF = mfma_header_floats(TRIG);
  static constexpr int C = kHalfChunk;
  static constexpr int NW = kHalfWaves;
  static constexpr int BQ = T * 6 * 64;     // 16-byte B parts per chunk (48 KB)
  static constexpr int NH = C * HF / 4;     // header float4s per chunk
  static_assert(BQ % (64 * NW) == 0 && NH <= 64, "chunk staging");

  __device__ static __forceinline__ void stage(const MfmaArgs& a, int64_t c, int wig, int lane, uint4* lb,
                                               float4* lh) {
    const __amdgpu_buffer_rsrc_t rb =
        buffer_rsrc(reinterpret_cast<const uint4*>(a.wb) + (c / C) * BQ, BQ * 16);
#pragma unroll
    for (int i = 0; i < BQ / 64 / NW; ++i) {
      const int blk = i * NW + wig;   // wave-uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_ptr)(lb + blk * 64), 16, lane * 16, blk * 1024, 0, 0);
    }
    // headers transposed in LDS: sample m = 8 g + e of the chunk at slot
    // 4 e + g, so that the four lane groups, which read samples 8 g + e at
    // once, hit consecutive slots (samples 8 apart would share banks)
    if (wig == 0 && lane < NH) {
      constexpr int P4 = HF / 4;   // float4s per header
      const int j = lane / P4, part = lane % P4, m = 8 * (j % 4) + j / 4;
      lds_dma16(buffer_rsrc(reinterpret_cast<const float4*>(a.hdr) + c * P4, NH * 16), (m * P4 + part) * 16, lh);
    }
  }

  __device__ static __forceinline__ void publish() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  __device__ static __forceinline__ void chunk(const float* __restrict__ hb, const uint4* __restrict__ lb,
                                               int lane, float gx, float gy, float gz, f32x4 (&acc)[3][T]) {
    half8 ah[3], al[3];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float av0[3], av1[3];   // samples 8 (lane / 16) + 2 p and + 2 p + 1
      group_entries<TRIG>(hb + (4 * (2 * p) + (lane >> 4)) * HF, gx, gy, gz, av0);
      group_entries<TRIG>(hb + (4 * (2 * p + 1) + (lane >> 4)) * HF, gx, gy, gz, av1);
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        uint32_t hi, lo;
        split_pair(av0[u], av1[u], hi, lo);
        const half2v h = __builtin_bit_cast(half2v, hi), l = __builtin_bit_cast(half2v, lo);
        ah[u][2 * p] = h[0];
        ah[u][2 * p + 1] = h[1];
        al[u][2 * p] = l[0];
        al[u][2 * p + 1] = l[1];
      }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      half8 bh[3], bl[3];
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const uint4 wh = lb[((t * 3 + u) * 2) * 64 + lane], wl = lb[((t * 3 + u) * 2 + 1) * 64 + lane];
        bh[u] = *reinterpret_cast<const half8*>(&wh);
        bl[u] = *reinterpret_cast<const half8*>(&wl);
      }
      // each accumulator is revisited after the other two products' MFMAs
#pragma unroll
      for (int u = 0; u < 3; ++u) acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[u], bh[u], acc[u][t], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 3; ++u) acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[u], bl[u], acc[u][t], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 3; ++u) acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[u], bh[u], acc[u][t], 0, 0, 0);
    }
  }

  __device__ static void run(const MfmaArgs& a) {
    __shared__ uint4 sb0[BQ], sb1[BQ];
    __shared__ float4 sh0[NH], sh1[NH];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wig = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t wave = (int64_t)blockIdx.x * NW + wig;
    const int64_t vbase = wave * 16 * V;
    const int64_t n0 = vbase + (int64_t)(lane & 15) * V;
    const bool gin = n0 < a.N;
    const float gx = gin ? a.x[n0] : 0.0f, gy = gin ? a.y[n0] : 0.0f, gz = gin ? a.z[n0] : 0.0f;
    const bool regular = wave_regular<V, 16>(a.x, a.y, a.z, a.N, n0, lane, gx, gy, gz);
    if (blockIdx.y == 0 && lane == 0 && vbase < a.N) a.flags[wave] = regular ? 1 : 0;
    if (!__syncthreads_or(regular)) return;
    const int32_t row = (int32_t)blockIdx.y;
    int64_t lo, hi;
    row_range(a.m_split, a.mpad, row, lo, hi);
    const int32_t nch = (int32_t)((hi - lo) / C);
    const int32_t cpt = (int32_t)(a.tile / C);
    if (nch > 0) stage(a, lo, wig, lane, sb0, sh0);
    publish();
    f32x4 acc[3][T], tre[FOLD ? T : 1], tim[FOLD ? T : 1];
#pragma unroll
    for (int t = 0; t < T; ++t) { acc[0][t] = f32x4{}; acc[1][t] = f32x4{}; acc[2][t] = f32x4{}; }
    if constexpr (FOLD) {
#pragma unroll
      for (int t = 0; t < T; ++t) { tre[t] = f32x4{}; tim[t] = f32x4{}; }
    }
    int32_t left = cpt;
    auto tile_end = [&]() {
      if constexpr (FOLD) {
        if (--left == 0) {
#pragma unroll
          for (int t = 0; t < T; ++t) {
            tre[t] += acc[0][t] - acc[2][t];
            tim[t] += acc[1][t] + acc[2][t];
            acc[0][t] = f32x4{}; acc[1][t] = f32x4{}; acc[2][t] = f32x4{};
          }
          left = cpt;
        }
      }
    };
    int32_t ch = 0;
    for (; ch + 1 < nch; ch += 2) {
      stage(a, lo + (int64_t)(ch + 1) * C, wig, lane, sb1, sh1);
      if (regular) chunk(reinterpret_cast<const float*>(sh0), sb0, lane, gx, gy, gz, acc);
      tile_end();
      publish();
      if (ch + 2 < nch) stage(a, lo + (int64_t)(ch + 2) * C, wig, lane, sb0, sh0);
      if (regular) chunk(reinterpret_cast<const float*>(sh1), sb1, lane, gx, gy, gz, acc);
      tile_end();
      publish();
    }
    if (ch < nch) {
      if (regular) chunk(reinterpret_cast<const float*>(sh0), sb0, lane, gx, gy, gz, acc);
      tile_end();
      publish();
    }
    if (!regular) return;
    if constexpr (FOLD) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        tre[t] += acc[0][t] - acc[2][t];
        tim[t] += acc[1][t] + acc[2][t];
      }
    }
    const float inv = a.scale[1];
    float2* dst = a.partial ? a.partial + (int64_t)row * BC * a.N : a.out;
    const int c = lane & 15;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int cc = 16 * t + c;
      const int b = cc / V, j = cc % V;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (lane >> 4) + r;
        const int64_t n = vbase + (int64_t)i * V + j;
        if (n >= a.N) continue;
        // Re = P1 - P3, Im = P2 + P3, scale undone (a power of two: exact)
        if constexpr (FOLD)
          dst[(int64_t)b * a.N + n] = make_float2(tre[t][r] * inv, tim[t][r] * inv);
        else
          dst[(int64_t)b * a.N + n] =
              make_float2((acc[0][t][r] - acc[2][t][r]) * inv, (acc[1][t][r] + acc[2][t][r]) * inv);
      }
    }
  }
};

// Direct gather for the irregular waves of the half-split engine: as
// MfmaDirect4 (tiles of a.tile samples folded into running totals), with
// Mu_b read in fp32 from the records' Mu array.
template <int BC, int TRIG>
struct HalfDirect {
  static constexpr int V = 128 / BC;
  static constexpr int ND = V / 4;
  static constexpr int NV = ND < 4 ? ND : 4;

  __device__ static void run(const MfmaArgs& a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kWorkgroup / 64) + (threadIdx.x >> 6);
    const int64_t vbase = wave * 16 * V;
    const int32_t row = (int32_t)blockIdx.y;
    int64_t lo, hi;
    row_range(a.m_split, a.mpad, row, lo, hi);
    if (vbase >= a.N) return;
    if (a.flags[wave]) return;
    constexpr int HF = mfma_header_floats(TRIG);
    for (int i0 = 0; i0 < ND; i0 += NV) {
      float vx[NV], vy[NV], vz[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int64_t n = vbase + lane + 64 * (i0 + i);
        const bool ok = n < a.N;
        vx[i] = ok ? a.x[n] : 0.0f;
        vy[i] = ok ? a.y[n] : 0.0f;
        vz[i] = ok ? a.z[n] : 0.0f;
      }
      float tre[NV][BC], tim[NV][BC];
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int b = 0; b < BC; ++b) { tre[i][b] = 0.0f; tim[i][b] = 0.0f; }
      for (int64_t t0 = lo; t0 < hi; t0 += a.tile) {
        const int64_t t1 = (hi - t0 > a.tile) ? t0 + a.tile : hi;
        float are[NV][BC], aim[NV][BC];
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
          for (int b = 0; b < BC; ++b) { are[i][b] = 0.0f; aim[i][b] = 0.0f; }
        for (int64_t m = t0; m < t1; ++m) {
          const float* hs = a.hdr + m * HF;
          float mr[BC], mi[BC];
#pragma unroll
          for (int b = 0; b < BC; ++b) {
            const float2 w = a.mu[m * BC + b];
            mr[b] = w.x;
            mi[b] = w.y;
          }
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            float c, sn;
            phase_sincos<TRIG>(hs, vx[i], vy[i], vz[i], c, sn);
#pragma unroll
            for (int b = 0; b < BC; ++b) {
              are[i][b] = __builtin_fmaf(mr[b], c, __builtin_fmaf(-mi[b], sn, are[i][b]));
              aim[i][b] = __builtin_fmaf(mi[b], c, __builtin_fmaf(mr[b], sn, aim[i][b]));
            }
          }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
          for (int b = 0; b < BC; ++b) { tre[i][b] += are[i][b]; tim[i][b] += aim[i][b]; }
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int64_t n = vbase + lane + 64 * (i0 + i);
        if (n >= a.N) continue;
#pragma unroll
        for (int b = 0; b < BC; ++b) {
          float2* dst = a.partial ? a.partial + (int64_t)row * BC * a.N : a.out;
          dst[(int64_t)b * a.N + n] = make_float2(tre[i][b], tim[i][b]);
        }
      }
    }
  }
};

template <int BC, int TRIG, bool FOLD>
__global__ void __launch_bounds__(64 * kHalfWaves) __attribute__((amdgpu_waves_per_eu(2)))
half_gather_kernel(MfmaArgs a) {
  HalfGather<BC, TRIG, FOLD>::run(a);
}

template <int BC, int TRIG>
__global__ void __launch_bounds__(kWorkgroup) half_direct_kernel(MfmaArgs a) {
  HalfDirect<BC, TRIG>::run(a);
}

struct HalfPair {
  MfmaFn gather;      // tiles folded into running totals
  DirectFn direct;
  MfmaFn gather_row;  // the launch row is one summation block
};

template <int BC>
HalfPair pick_half(int trig) {
  if (trig == kTrigHw)
    return {half_gather_kernel<BC, kTrigHw, true>, half_direct_kernel<BC, kTrigHw>,
            half_gather_kernel<BC, kTrigHw, false>};
  return {half_gather_kernel<BC, kTrigAccurate, true>, half_direct_kernel<BC, kTrigAccurate>,
          half_gather_kernel<BC, kTrigAccurate, false>};
}

HalfPair select_half(int trig, int BC) {
  switch (BC) {
    case 1: return pick_half<1>(trig);
    case 2: return pick_half<2>(trig);
    case 4: return pick_half<4>(trig);
    case 8: return pick_half<8>(trig);
    case 16: return pick_half<16>(trig);
    default: return {nullptr, nullptr, nullptr};
  }
}

}  // namespace

bool half_supported(int BC) { return select_half(kTrigHw, BC).gather != nullptr; }

hipError_t launch_half_records(int is_q, int trig, int BC, const HalfRecordArgs& a, hipStream_t s) {
  if (!half_supported(BC) || a.r.mpad % kMfmaChunk != 0 || !a.scale) return hipErrorInvalidValue;
  // the scale first, also for M = 0 (then 1: the gather multiplies its zero sums by it)
  hipLaunchKernelGGL(half_scale_partial_kernel, dim3(kHalfScaleBlocks), dim3(256), 0, s, a.r, is_q, BC, a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(half_scale_kernel, dim3(1), dim3(256), 0, s, a.scale);
  e = hipGetLastError();
  if (e != hipSuccess || a.r.mpad <= 0) return e;
  if (!a.wh || !a.mu) return hipErrorInvalidValue;
  const int64_t lanes = a.r.mpad / 8 * 128;
  hipLaunchKernelGGL(half_records_kernel, dim3((unsigned)((lanes + kWorkgroup - 1) / kWorkgroup)), dim3(kWorkgroup), 0,
                     s, a, is_q, trig, BC);
  return hipGetLastError();
}

hipError_t launch_half_gather(int trig, int BC, int32_t splits, const MfmaArgs& a, hipStream_t s) {
  HalfPair fn = select_half(trig, BC);
  if (!fn.gather || splits < 1 || (splits > 1) != (a.partial != nullptr) || !a.flags || !a.mu || !a.scale)
    return hipErrorInvalidValue;
  if (a.mpad % kMfmaChunk != 0 || a.m_split % kMfmaChunk != 0 || a.tile % kHalfChunk != 0 || a.tile <= 0)
    return hipErrorInvalidValue;
  if (a.N <= 0) return hipSuccess;
  const int64_t waves = mfma_gather_waves(a.N, 8, BC);
  const int64_t blocks = (waves + kHalfWaves - 1) / kHalfWaves;
  const int64_t dblocks = (waves + kWorkgroup / 64 - 1) / (kWorkgroup / 64);
  // a tile as long as the launch row never folds: the kernel without running totals
  const MfmaFn g = a.tile >= a.m_split ? fn.gather_row : fn.gather;
  hipLaunchKernelGGL(g, dim3((unsigned)blocks, (unsigned)splits), dim3(64 * kHalfWaves), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn.direct, dim3((unsigned)dblocks, (unsigned)splits), dim3(kWorkgroup), 0, s, a);
  return hipGetLastError();
}

}  // namespace ncmri
