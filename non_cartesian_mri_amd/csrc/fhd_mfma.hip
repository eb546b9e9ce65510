// gfx950 matrix-core engine for F^H D and Q (PMPP ch. 17 "Iterative MRI
// reconstruction").
//
// The pages' gather (section 17.3, Figs. 17.9-17.11) evaluates, for every
// voxel and sample, one phase, its sine and cosine, and a complex
// multiply-accumulate.  Phase factoring turns most of that into a dense
// product.  Split the voxels into groups of V that sit at common offsets d_j
// from their group's first voxel x_g (on a Cartesian grid: V consecutive
// voxels of one row).  Then
//
//   out[b][x_g + d_j] = sum_m  (c + i s)_m[g] * (fr + i fi)_m[j][b],
//   (c, s)_m[g] = (cos, sin)(2 pi k_m.x_g),
//   f_m[j][b]   = Mu_b[m] exp(i 2 pi k_m.d_j)   (Mu = conj(phi) D, or |phi|^2 for Q)
//
// a complex matrix product (groups x samples) * (samples x columns).  It is
// computed with three real products instead of four (the three-multiplication
// form of a complex product, usually credited to Gauss):
//
//   P1 = sum (c + s) fr,   P2 = sum (c - s) fi,   P3 = sum s (fr + fi),
//   Re = P1 - P3,          Im = P2 + P3.
//
// This variant keeps a sample at k = 0 exact: with s = 0 the products are
// c fr, c fi and 0.  Each real product over 32 groups, 32 columns and two
// samples is one v_mfma_f32_32x32x2_f32 (K = 2 = the samples of a pair), so a
// pair of samples costs 3 MFMAs per tile of 32 complex columns where the
// four-product form needs 4, and each lane evaluates one phase (3 FMAs), its
// sine and its cosine per pair of samples.  The factor values (fr, fi,
// fr + fi) do not depend on the voxel; the records kernel forms them once
// per sample, in double, rounded once to fp32, already laid out as the MFMA B
// operands.
//
// Operand layouts of v_mfma_f32_32x32x2_f32 (wave64), checked on gfx950:
//   A[i][k] = lane 32 k + i,  B[k][j] = lane 32 k + j,
//   D[i][j] = register (i / 8) * 4 + i % 4 of lane 32 * ((i / 4) % 2) + j.
// So lane l supplies group i = l % 32 at sample 2 h + l / 32 of pair h, and
// the B entry of column j at that sample.
//
// Data flow.  The 4 waves of a workgroup walk the same samples, so each
// 32-sample chunk of records is copied from memory once per workgroup into LDS
// and read from there by every wave -- the role the pages give constant memory
// (Figs. 17.12/17.13).  The copy uses gfx950's LDS DMA (buffer_load_dwordx4 ...
// lds: lane i's 16 bytes land at the LDS base + 16 i, no VGPRs involved), double
// buffered in two separate LDS arrays: the next chunk's copy is in flight
// while the current one is consumed, with one wait and workgroup barrier per
// chunk.  The headers (k) are read from LDS, two addresses per wave.
//
// Waves whose voxels are not on the common offsets (any non-grid coordinate
// set) only help stage the chunks (a workgroup of such waves only leaves at
// once); a second kernel (mfma_direct_kernel) evaluates every voxel phase of
// those waves directly on the vector ALU from the same records (the offset-0
// columns hold fr, fi = Mu_b), and exits at once for the other waves: the
// gather's first launch row records each wave's decision in a flag array.
//
// Summation is blocked as in the VALU engine: tile partial sums in the MFMA
// accumulators, folded (as Re, Im) into running totals at tile ends.
#include "fhd_internal.h"
#include "fhd_trig.h"
#include "fhd_mfma_common.h"
#include "fhd_groups.h"

namespace ncmri {
namespace {

// ---------------------------------------------------------------------------
// Records of the two-sample engine: one lane per (padded sample, complex
// column).
__global__ void __launch_bounds__(kWorkgroup)
mfma_records_kernel(MfmaRecordArgs a, int is_q, int trig, int T, int BC) {
  const int cols = 16 * T;
  const int P = T / 2;
  const int64_t idx = (int64_t)blockIdx.x * kWorkgroup + threadIdx.x;
  const int64_t m = idx / cols;
  const int cc = (int)(idx - m * cols);
  if (m >= a.mpad) return;
  const int HF = mfma_header_floats(trig);
  const int V = cols / BC;
  float* h = a.hdr + m * HF;
  // two-sample engine (T = 2, 4): entry of column c = cc % 32 of tile
  // t = cc / 32 at row m % 2 of the pair
  const int t = cc / 32, lp = 32 * (int)(m & 1) + cc % 32;
  float* pair = a.wb + (m >> 1) * (192 * P);
  float* wr = pair + lp * (2 * P) + t;  // fr; fi at + P
  float* wi = wr + P;
  float* ws = pair + 128 * P + lp * P + t;  // fr + fi
  if (m >= a.M) {  // padding sample: contributes exactly zero
    if (cc == 0)
      for (int i = 0; i < HF; ++i) h[i] = 0.0f;
    wr[0] = 0.0f; wi[0] = 0.0f; ws[0] = 0.0f;
    return;
  }
  const float kx = a.kx[m], ky = a.ky[m], kz = a.kz[m];
  if (cc == 0) {
    if (trig == kTrigHw) {
      h[0] = kx; h[1] = ky; h[2] = kz; h[3] = 0.0f;
    } else {
      // kh = nearest multiple of 2^-12 (exact scaling by powers of two), kl = k - kh (exact)
      const float khx = __builtin_rintf(kx * 4096.0f) * (1.0f / 4096.0f);
      const float khy = __builtin_rintf(ky * 4096.0f) * (1.0f / 4096.0f);
      const float khz = __builtin_rintf(kz * 4096.0f) * (1.0f / 4096.0f);
      h[0] = khx; h[1] = khy; h[2] = khz; h[3] = 0.0f;
      h[4] = kx - khx; h[5] = ky - khy; h[6] = kz - khz; h[7] = 0.0f;
    }
  }
  const int b = cc / V, j = cc % V;
  // phase factor of offset j relative to the group's first voxel (columns of
  // offsets beyond a voxel set smaller than one group are never written out)
  double cj = 1.0, sj = 0.0;
  if (j > 0 && j < a.N) {
    const double p = (double)kx * ((double)a.x[j] - (double)a.x[0]) +
                     (double)ky * ((double)a.y[j] - (double)a.y[0]) +
                     (double)kz * ((double)a.z[j] - (double)a.z[0]);
    sincospi(2.0 * p, &sj, &cj);
  }
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
  const double fr = mr * cj - mi * sj, fi = mr * sj + mi * cj;
  wr[0] = (float)fr; wi[0] = (float)fi; ws[0] = (float)(fr + fi);
}

// Records of the four-sample engine (T = 8): one lane per (padded sample m,
// column c < 16, tile group g < 2) forms the factors of the four columns
// cc = 16 t + c, t = 4 g .. 4 g + 3, and writes fr, fi and fr + fi of them as
// three float4 slices (slices g, 2 + g and 4 + g of lane p = 16 (m % 4) + c;
// 16 consecutive lanes fill 256 contiguous bytes).
__global__ void __launch_bounds__(kWorkgroup)
mfma4_records_kernel(MfmaRecordArgs a, int is_q, int trig, int BC) {
  constexpr int T = 8;
  const int64_t idx = (int64_t)blockIdx.x * kWorkgroup + threadIdx.x;
  const int64_t m = idx >> 5;
  const int r = (int)(idx & 31), c = r & 15, g = r >> 4;
  if (m >= a.mpad) return;
  const int HF = mfma_header_floats(trig);
  const int V = 16 * T / BC;
  float* h = a.hdr + m * HF;
  float4* blk = reinterpret_cast<float4*>(a.wb) + (m >> 2) * (192 * T / 4);
  const int p = 16 * (int)(m & 3) + c;
  float4* wr = blk + g * 64 + p;
  float4* wi = blk + (2 + g) * 64 + p;
  float4* ws = blk + (4 + g) * 64 + p;
  if (m >= a.M) {  // padding sample: contributes exactly zero
    if (r == 0)
      for (int i = 0; i < HF; ++i) h[i] = 0.0f;
    *wr = make_float4(0.0f, 0.0f, 0.0f, 0.0f); *wi = *wr; *ws = *wr;
    return;
  }
  const float kx = a.kx[m], ky = a.ky[m], kz = a.kz[m];
  if (r == 0) {
    if (trig == kTrigHw) {
      h[0] = kx; h[1] = ky; h[2] = kz; h[3] = 0.0f;
    } else {
      const float khx = __builtin_rintf(kx * 4096.0f) * (1.0f / 4096.0f);
      const float khy = __builtin_rintf(ky * 4096.0f) * (1.0f / 4096.0f);
      const float khz = __builtin_rintf(kz * 4096.0f) * (1.0f / 4096.0f);
      h[0] = khx; h[1] = khy; h[2] = khz; h[3] = 0.0f;
      h[4] = kx - khx; h[5] = ky - khy; h[6] = kz - khz; h[7] = 0.0f;
    }
  }
  const double pr = a.phi[m].x, pim = a.phi[m].y;
  // offsets relative to the reference column jref (< N): its factor is Mu_b itself
  const double x0 = a.x[a.jref], y0 = a.y[a.jref], z0 = a.z[a.jref];
  float fr[4], fi[4], fs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int cc = 16 * (4 * g + i) + c;
    const int b = cc / V, j = cc % V;
    double cj = 1.0, sj = 0.0;
    if (j != a.jref && j < a.N) {
      const double ph = (double)kx * ((double)a.x[j] - x0) + (double)ky * ((double)a.y[j] - y0) +
                        (double)kz * ((double)a.z[j] - z0);
      sincospi(2.0 * ph, &sj, &cj);
    }
    double mr, mi;
    if (is_q) {
      mr = pr * pr + pim * pim;
      mi = 0.0;
    } else {
      const float2 d = a.D[(int64_t)b * a.M + m];
      mr = pr * d.x + pim * d.y;  // Mu = conj(phi) * D
      mi = pr * d.y - pim * d.x;
    }
    const double vr = mr * cj - mi * sj, vi = mr * sj + mi * cj;
    fr[i] = (float)vr; fi[i] = (float)vi; fs[i] = (float)(vr + vi);
  }
  *wr = make_float4(fr[0], fr[1], fr[2], fr[3]);
  *wi = make_float4(fi[0], fi[1], fi[2], fi[3]);
  *ws = make_float4(fs[0], fs[1], fs[2], fs[3]);
}

// ---------------------------------------------------------------------------
// Matrix-core gather (regular waves).
template <int T, int BC, int TRIG>
struct MfmaGather {
  static constexpr int V = 16 * T / BC;                // voxels per group
  static constexpr int P = T / 2;                      // tiles of 32 complex columns
  static constexpr int HF = mfma_header_floats(TRIG);  // header floats per sample
  static constexpr int C = kMfmaChunk;
  static constexpr int NW = kWorkgroup / 64;           // waves per workgroup
  static constexpr int PF = 192 * P;                   // factor floats per pair of samples
  static constexpr int NB = C / 2 * PF * 4 / 1024;     // 1 KiB factor blocks per chunk
  static constexpr int NH = C * HF / 4;                // header float4s per chunk
  static_assert(P >= 1 && V >= 2 && V * BC == 16 * T, "group shape");
  static_assert(NB % NW == 0 && NH <= 64, "chunk staging");

  static constexpr int HK = TRIG == kTrigHw ? 3 : 7;  // header floats a sample's phase reads

  // Header of the lane's sample and its B-operand entries of pair h of the
  // chunk in LDS: fr (P), fi (P) in one read, fr + fi (P) in another.
  __device__ static __forceinline__ void load_pair(const float* __restrict__ hb,
                                                   const float* __restrict__ wb, int h, int lane,
                                                   float (&hs)[HK], float (&bv)[3 * P]) {
    const float* hp = hb + (2 * h + (lane >> 5)) * HF;
#pragma unroll
    for (int i = 0; i < HK; ++i) hs[i] = hp[i];
    const float* pp = wb + h * PF;
    if constexpr (P == 2) {
      const float4 v = *reinterpret_cast<const float4*>(pp + lane * 4);
      const float2 u = *reinterpret_cast<const float2*>(pp + 256 + lane * 2);
      bv[0] = v.x; bv[1] = v.y; bv[2] = v.z; bv[3] = v.w; bv[4] = u.x; bv[5] = u.y;
    } else if constexpr (P == 1) {
      const float2 v = *reinterpret_cast<const float2*>(pp + lane * 2);
      bv[0] = v.x; bv[1] = v.y; bv[2] = pp[128 + lane];
    } else {
#pragma unroll
      for (int i = 0; i < 2 * P; ++i) bv[i] = pp[lane * 2 * P + i];
#pragma unroll
      for (int t = 0; t < P; ++t) bv[2 * P + t] = pp[128 * P + lane * P + t];
    }
  }

  __device__ static __forceinline__ void mfmas(const float (&av)[3], const float (&bv)[3 * P],
                                               f32x16 (&acc)[3][P]) {
#pragma unroll
    for (int t = 0; t < P; ++t) {
      acc[0][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[0], bv[t], acc[0][t], 0, 0, 0);
      acc[1][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[1], bv[P + t], acc[1][t], 0, 0, 0);
      acc[2][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[2], bv[2 * P + t], acc[2][t], 0, 0, 0);
    }
  }

  // One chunk for a wave on the common offsets, software-pipelined by one
  // pair: the next pair's LDS reads are issued before this pair's MFMAs (the
  // fences keep the scheduler from moving them).  The A entries of the HW
  // path (three FMAs, fract, sine, cosine) are computed right before the
  // pair's own MFMAs; the accurate path's longer chain (exact reduction and
  // polynomials) is computed one pair ahead, right after the previous pair's
  // MFMAs, so it runs while the matrix pipe works.
  __device__ static __forceinline__ void regular_chunk(const float* __restrict__ hb,
                                                       const float* __restrict__ wb, int lane,
                                                       float gx, float gy, float gz,
                                                       f32x16 (&acc)[3][P]) {
    constexpr int NP = C / 2;
    float hc[HK], bc[3 * P], av[3];
    load_pair(hb, wb, 0, lane, hc, bc);
    if constexpr (TRIG == kTrigHw) {
#pragma unroll
      for (int h = 0; h < NP; ++h) {
        float hn[HK], bn[3 * P];
        if (h + 1 < NP) load_pair(hb, wb, h + 1, lane, hn, bn);
        sched_fence();
        group_entries<TRIG>(hc, gx, gy, gz, av);
        mfmas(av, bc, acc);
        sched_fence();
        if (h + 1 < NP) {
#pragma unroll
          for (int i = 0; i < HK; ++i) hc[i] = hn[i];
#pragma unroll
          for (int i = 0; i < 3 * P; ++i) bc[i] = bn[i];
        }
      }
    } else {
      group_entries<TRIG>(hc, gx, gy, gz, av);
#pragma unroll
      for (int h = 0; h < NP; ++h) {
        float hn[HK], bn[3 * P];
        if (h + 1 < NP) load_pair(hb, wb, h + 1, lane, hn, bn);
        sched_fence();
        mfmas(av, bc, acc);
        sched_fence();
        if (h + 1 < NP) {
          group_entries<TRIG>(hn, gx, gy, gz, av);
#pragma unroll
          for (int i = 0; i < 3 * P; ++i) bc[i] = bn[i];
        }
        sched_fence();
      }
    }
  }

  // Starts the copy of the chunk at sample c into (lb, lh): wave w copies the
  // factor blocks w, w + NW, ... and wave 0 the headers.
  __device__ static __forceinline__ void stage(const MfmaArgs& a, int64_t c, int wave_in_wg,
                                               int lane, float4* lb, float4* lh) {
    const __amdgpu_buffer_rsrc_t rb =
        buffer_rsrc(reinterpret_cast<const float4*>(a.wb) + (c / 2) * (PF / 4), NB * 64 * 16);
#pragma unroll
    for (int i = 0; i < NB / NW; ++i) {
      const int blk = i * NW + wave_in_wg;
      lds_dma16(rb, (blk * 64 + lane) * 16, lb + blk * 64);
    }
    if (wave_in_wg == 0 && lane < NH)
      lds_dma16(buffer_rsrc(reinterpret_cast<const float4*>(a.hdr) + c * (HF / 4), NH * 16), lane * 16, lh);
  }

  // Chunk copies complete (this wave's) and visible to the workgroup.
  __device__ static __forceinline__ void publish() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Tile end: Re = P1 - P3, Im = P2 + P3 into the running totals.
  __device__ static __forceinline__ void fold(f32x16 (&acc)[3][P], f32x16 (&tre)[P],
                                              f32x16 (&tim)[P]) {
#pragma unroll
    for (int t = 0; t < P; ++t) {
      tre[t] += acc[0][t] - acc[2][t];
      tim[t] += acc[1][t] + acc[2][t];
      acc[0][t] = f32x16{}; acc[1][t] = f32x16{}; acc[2][t] = f32x16{};
    }
  }

  __device__ static void run(const MfmaArgs& a) {
    __shared__ float4 sb0[C / 2 * PF / 4], sb1[C / 2 * PF / 4];
    __shared__ float4 sh0[NH], sh1[NH];
    const int tid = threadIdx.x, lane = tid & 63, wig = tid >> 6;
    const int64_t wave = (int64_t)blockIdx.x * NW + wig;
    const int64_t vbase = wave * 32 * V;   // first voxel of the wave
    const int64_t n0 = vbase + (int64_t)(lane & 31) * V;  // first voxel of the lane's group
    const bool gin = n0 < a.N;
    const float gx = gin ? a.x[n0] : 0.0f, gy = gin ? a.y[n0] : 0.0f, gz = gin ? a.z[n0] : 0.0f;
    const bool regular = wave_regular<V>(a.x, a.y, a.z, a.N, n0, lane, gx, gy, gz);
    // the decision for the direct kernel, once per wave
    if (blockIdx.y == 0 && lane == 0 && vbase < a.N) a.flags[wave] = regular ? 1 : 0;
    // a workgroup without a regular wave has no chunk to stage for anyone
    if (!__syncthreads_or(regular)) return;
    const int32_t row = (int32_t)blockIdx.y;
    int64_t lo, hi;
    row_range(a.m_split, a.mpad, row, lo, hi);

    // Chunks alternate between the two buffers; tiles (a whole number of
    // chunks, counted from lo) fold into the totals.
    const int32_t nch = (int32_t)((hi - lo) / C);
    const int32_t cpt = (int32_t)(a.tile / C);
    if (nch > 0) stage(a, lo, wig, lane, sb0, sh0);
    publish();
    f32x16 acc[3][P], tre[P], tim[P];
#pragma unroll
    for (int t = 0; t < P; ++t) {
      acc[0][t] = f32x16{}; acc[1][t] = f32x16{}; acc[2][t] = f32x16{};
      tre[t] = f32x16{}; tim[t] = f32x16{};
    }
    int32_t left = cpt;  // chunks left in the current tile
    for (int32_t ch = 0; ch < nch; ch += 2) {
      if (ch + 1 < nch) stage(a, lo + (int64_t)(ch + 1) * C, wig, lane, sb1, sh1);
      if (regular)
        regular_chunk(reinterpret_cast<const float*>(sh0), reinterpret_cast<const float*>(sb0), lane,
                      gx, gy, gz, acc);
      if (--left == 0) {
        fold(acc, tre, tim);
        left = cpt;
      }
      publish();
      if (ch + 1 >= nch) break;
      if (ch + 2 < nch) stage(a, lo + (int64_t)(ch + 2) * C, wig, lane, sb0, sh0);
      if (regular)
        regular_chunk(reinterpret_cast<const float*>(sh1), reinterpret_cast<const float*>(sb1), lane,
                      gx, gy, gz, acc);
      if (--left == 0) {
        fold(acc, tre, tim);
        left = cpt;
      }
      publish();
    }
    fold(acc, tre, tim);  // the last (partial) tile

    // write-out: out[b][n], or this row's partial sums (irregular waves are
    // written by mfma_direct_kernel)
    if (!regular) return;
    float2* dst = a.partial ? a.partial + (int64_t)row * BC * a.N : a.out;
    const int c = lane & 31;
#pragma unroll
    for (int t = 0; t < P; ++t) {
      const int cc = 32 * t + c;
      const int b = cc / V, j = cc % V;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = (v / 4) * 8 + (lane / 32) * 4 + (v % 4);
        const int64_t n = vbase + (int64_t)i * V + j;
        if (n < a.N) dst[(int64_t)b * a.N + n] = make_float2(tre[t][v], tim[t][v]);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Direct gather for the irregular waves, over the same launch rows as the
// gather (row blockIdx.y sums its share of the samples into its partial-sum
// row; one row writes the output).  Lane l of wave w owns voxels
// 32 V w + l + 64 i, i < V / 2, and evaluates each voxel's phase; records are
// read with wave-uniform scalar loads.
template <int T, int BC, int TRIG>
struct MfmaDirect {
  static constexpr int V = 16 * T / BC;
  static constexpr int P = T / 2;
  static constexpr int HF = mfma_header_floats(TRIG);
  static constexpr int ND = V / 2;

  __device__ static void run(const MfmaArgs& a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kWorkgroup / 64) + (threadIdx.x >> 6);
    const int64_t vbase = wave * 32 * V;
    const int32_t row = (int32_t)blockIdx.y;
    int64_t lo, hi;
    row_range(a.m_split, a.mpad, row, lo, hi);
    if (vbase >= a.N) return;
    if (a.flags[wave]) return;   // a regular wave: the gather kernel summed it

    float vx[ND], vy[ND], vz[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int64_t n = vbase + lane + 64 * i;
      const bool ok = n < a.N;
      vx[i] = ok ? a.x[n] : 0.0f;
      vy[i] = ok ? a.y[n] : 0.0f;
      vz[i] = ok ? a.z[n] : 0.0f;
    }
    float tre[ND][BC], tim[ND][BC];
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int b = 0; b < BC; ++b) { tre[i][b] = 0.0f; tim[i][b] = 0.0f; }
    for (int64_t t0 = lo; t0 < hi; t0 += a.tile) {
      const int64_t t1 = (hi - t0 > a.tile) ? t0 + a.tile : hi;
      float are[ND][BC], aim[ND][BC];
#pragma unroll
      for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int b = 0; b < BC; ++b) { are[i][b] = 0.0f; aim[i][b] = 0.0f; }
      for (int64_t m = t0; m < t1; ++m) {
        const float* hs = a.hdr + m * HF;
        const float* wm = a.wb + (m >> 1) * (192 * P);
        const int k = (int)(m & 1);
        float mr[BC], mi[BC];
#pragma unroll
        for (int b = 0; b < BC; ++b) {
          // Mu_b is the offset-0 column of vector b: (fr, fi) of column cc
          const int cc = b * V;
          const float* e = wm + (32 * k + cc % 32) * (2 * P) + cc / 32;
          mr[b] = e[0];
          mi[b] = e[P];
        }
#pragma unroll
        for (int i = 0; i < ND; ++i) {
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
      for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int b = 0; b < BC; ++b) { tre[i][b] += are[i][b]; tim[i][b] += aim[i][b]; }
    }
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int64_t n = vbase + lane + 64 * i;
      if (n >= a.N) continue;
#pragma unroll
      for (int b = 0; b < BC; ++b) {
        float2* dst = a.partial ? a.partial + (int64_t)row * BC * a.N : a.out;
        dst[(int64_t)b * a.N + n] = make_float2(tre[i][b], tim[i][b]);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Four-sample matrix-core gather (regular waves), v_mfma_f32_16x16x4_f32:
// A[i][k] = lane 16 k + i, B[k][j] = lane 16 k + j, D[i][j] = register i % 4
// of lane 16 (i / 4) + j (checked on gfx950).  A wave owns 16 groups of V
// voxels; lane l supplies group l % 16 at sample 4 q + l / 16 of block q, so
// each lane evaluates one phase with its sine and cosine per four samples and
// the 16 x 16 products take 3 T MFMAs per block: with T = 8 tiles of 16
// complex columns that is 24 MFMAs (768 matrix cycles) per phase, twice the
// two-sample engine's 6 per pair at the same register count.  Records stream
// through LDS in 16-sample chunks (4 blocks, 24 KB with T = 8) shared by the
// 4 waves of a workgroup; two workgroups per CU (2 waves per SIMD, one of
// each), so that one workgroup's barrier or copy burst is covered by the
// other's MFMAs.  (One 8-wave workgroup per CU with 32-sample chunks was
// 1.5 % slower at 128^3: its two waves on a SIMD wait at the same barrier.)
// FOLD: tiles shorter than the launch row fold into running totals (blocked
// summation within the row).  Without FOLD the row is one summation block:
// the accumulators hold the row's sums, no totals are kept (64 VGPRs fewer:
// 3 waves per SIMD on the HW path), and the rows are added in a fixed order
// by the reduction kernel.
template <int T, int BC, int TRIG, bool FOLD>
struct MfmaGather4 {
  static constexpr int V = 16 * T / BC;                // voxels per group
  static constexpr int HF = mfma_header_floats(TRIG);
  static constexpr int C = kMfma4Chunk;
  static constexpr int NW = kMfma4Waves;               // waves per workgroup
  static constexpr int QF = 192 * T;                   // factor floats per block of 4 samples
  static constexpr int NS = 3 * T / 4;                 // float4 slices per lane and block
  static constexpr int NB = C / 4 * QF * 4 / 1024;     // 1 KiB factor blocks per chunk
  static constexpr int NH = C * HF / 4;                // header float4s per chunk
  static constexpr int HK = TRIG == kTrigHw ? 3 : 7;
  static_assert(T % 4 == 0 && V >= 1 && V * BC == 16 * T, "group shape");
  static_assert(NB % NW == 0 && NH <= 64, "chunk staging");

  __device__ static __forceinline__ void load_block(const float* __restrict__ hb,
                                                    const float* __restrict__ wb, int q, int lane,
                                                    float (&hs)[HK], float (&bv)[3 * T]) {
    const float* hp = hb + (4 * q + (lane >> 4)) * HF;
#pragma unroll
    for (int i = 0; i < HK; ++i) hs[i] = hp[i];
    const float* pp = wb + q * QF;
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      const float4 v = *reinterpret_cast<const float4*>(pp + (sl * 64 + lane) * 4);
      bv[4 * sl] = v.x; bv[4 * sl + 1] = v.y; bv[4 * sl + 2] = v.z; bv[4 * sl + 3] = v.w;
    }
  }

  __device__ static __forceinline__ void mfmas(const float (&av)[3], const float (&bv)[3 * T],
                                               f32x4 (&acc)[3][T]) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[0], bv[t], acc[0][t], 0, 0, 0);
      acc[1][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[1], bv[T + t], acc[1][t], 0, 0, 0);
      acc[2][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[2], bv[2 * T + t], acc[2][t], 0, 0, 0);
    }
  }

  // Slices of block q for the units t of one half h: slices h, 2 + h, 4 + h
  // (the three products' entries for t in [4h, 4h + 4)).
  __device__ static __forceinline__ void load_half(const float* __restrict__ wb, int q, int lane, int h,
                                                   float (&bv)[3 * T]) {
    static_assert(T == 8, "half-block slices 2 p + h of four units each: the layout of T = 8");
    const float* pp = wb + q * QF;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const int sl = 2 * p + h;
      const float4 v = *reinterpret_cast<const float4*>(pp + (sl * 64 + lane) * 4);
      bv[4 * sl] = v.x; bv[4 * sl + 1] = v.y; bv[4 * sl + 2] = v.z; bv[4 * sl + 3] = v.w;
    }
  }

  __device__ static __forceinline__ void load_header(const float* __restrict__ hb, int q, int lane,
                                                     float (&hs)[HK]) {
    const float* hp = hb + (4 * q + (lane >> 4)) * HF;
#pragma unroll
    for (int i = 0; i < HK; ++i) hs[i] = hp[i];
  }

  template <int H>
  __device__ static __forceinline__ void mfmas_half(const float (&av)[3], const float (&bv)[3 * T],
                                                    f32x4 (&acc)[3][T]) {
#pragma unroll
    for (int u = 0; u < T / 2; ++u) {
      const int t = H * (T / 2) + u;
      acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[0], bv[t], acc[0][t], 0, 0, 0);
      acc[1][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[1], bv[T + t], acc[1][t], 0, 0, 0);
      acc[2][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[2], bv[2 * T + t], acc[2][t], 0, 0, 0);
    }
  }

  // One chunk.  HW trig: one set of B entries; the next block's first-half
  // slices are read once this block's first-half MFMAs have issued, its
  // second half after the rest (each half a block of MFMAs ahead of its use),
  // and the A entries are formed right before the block's MFMAs.  Accurate
  // trig: software-pipelined by one whole block (A entries one block ahead,
  // right after the previous block's MFMAs), as in the two-sample engine.
  __device__ static __forceinline__ void regular_chunk(const float* __restrict__ hb,
                                                       const float* __restrict__ wb, int lane,
                                                       float gx, float gy, float gz,
                                                       f32x4 (&acc)[3][T]) {
    constexpr int NQ = C / 4;
    if constexpr (TRIG == kTrigHw) {
      float hc[HK], bv[3 * T], av[3];
      load_header(hb, 0, lane, hc);
      load_half(wb, 0, lane, 0, bv);
      load_half(wb, 0, lane, 1, bv);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        float hn[HK];
        if (q + 1 < NQ) load_header(hb, q + 1, lane, hn);
        sched_fence();
        group_entries<TRIG>(hc, gx, gy, gz, av);
        mfmas_half<0>(av, bv, acc);
        sched_fence();
        if (q + 1 < NQ) load_half(wb, q + 1, lane, 0, bv);
        sched_fence();
        mfmas_half<1>(av, bv, acc);
        sched_fence();
        if (q + 1 < NQ) {
          load_half(wb, q + 1, lane, 1, bv);
#pragma unroll
          for (int i = 0; i < HK; ++i) hc[i] = hn[i];
        }
        sched_fence();
      }
    } else {
      float hc[HK], bc[3 * T], av[3];
      load_block(hb, wb, 0, lane, hc, bc);
      group_entries<TRIG>(hc, gx, gy, gz, av);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        float hn[HK], bn[3 * T];
        if (q + 1 < NQ) load_block(hb, wb, q + 1, lane, hn, bn);
        sched_fence();
        mfmas(av, bc, acc);
        sched_fence();
        if (q + 1 < NQ) {
          group_entries<TRIG>(hn, gx, gy, gz, av);
#pragma unroll
          for (int i = 0; i < 3 * T; ++i) bc[i] = bn[i];
        }
        sched_fence();
      }
    }
  }

  // Starts the copy of the chunk at sample c: wave w copies the factor blocks
  // w, w + NW, ... and wave 0 the headers.
  // Starts the copy of the chunk at sample c: wave w copies the factor blocks
  // w, w + NW, ... and wave 0 the headers.
  __device__ static __forceinline__ void stage(const MfmaArgs& a, int64_t c, int wave_in_wg,
                                               int lane, float4* lb, float4* lh) {
    const __amdgpu_buffer_rsrc_t rb =
        buffer_rsrc(reinterpret_cast<const float4*>(a.wb) + (c / 4) * (QF / 4), NB * 64 * 16);
#pragma unroll
    for (int i = 0; i < NB / NW; ++i) {
      const int blk = i * NW + wave_in_wg;   // wave-uniform: an SGPR offset
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_ptr)(lb + blk * 64), 16, lane * 16,
                                               blk * 1024, 0, 0);
    }
    if (wave_in_wg == 0 && lane < NH)
      lds_dma16(buffer_rsrc(reinterpret_cast<const float4*>(a.hdr) + c * (HF / 4), NH * 16), lane * 16, lh);
  }

  // Chunk copies complete (this wave's) and visible to the workgroup.
  __device__ static __forceinline__ void publish() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  template <int NT>
  __device__ static __forceinline__ void fold(f32x4 (&acc)[3][T], f32x4 (&tre)[NT], f32x4 (&tim)[NT]) {
    static_assert(NT == T, "fold needs the running totals");
#pragma unroll
    for (int t = 0; t < T; ++t) {
      tre[t] += acc[0][t] - acc[2][t];
      tim[t] += acc[1][t] + acc[2][t];
      acc[0][t] = f32x4{}; acc[1][t] = f32x4{}; acc[2][t] = f32x4{};
    }
  }

  __device__ static void run(const MfmaArgs& a) {
    __shared__ float4 sb0[C / 4 * QF / 4], sb1[C / 4 * QF / 4];
    __shared__ float4 sh0[NH], sh1[NH];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wig = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave in the workgroup
    const int64_t wave = (int64_t)blockIdx.x * NW + wig;
    const int64_t vbase = wave * 16 * V;                  // first voxel of the wave
    const int64_t n0 = vbase + (int64_t)(lane & 15) * V;  // first voxel of the lane's group
    const bool gin = n0 < a.N;
    const float gx = gin ? a.x[n0] : 0.0f, gy = gin ? a.y[n0] : 0.0f, gz = gin ? a.z[n0] : 0.0f;
    const bool regular = wave_regular<V, 16>(a.x, a.y, a.z, a.N, n0, lane, gx, gy, gz);
    // the decision for the direct kernel, once per wave
    if (blockIdx.y == 0 && lane == 0 && vbase < a.N) a.flags[wave] = regular ? 1 : 0;
    // a workgroup without a regular wave has no chunk to stage for anyone
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
    for (int t = 0; t < T; ++t) {
      acc[0][t] = f32x4{}; acc[1][t] = f32x4{}; acc[2][t] = f32x4{};
    }
    if constexpr (FOLD) {
#pragma unroll
      for (int t = 0; t < T; ++t) { tre[t] = f32x4{}; tim[t] = f32x4{}; }
    }
    int32_t left = cpt;
    auto tile_end = [&]() {
      if constexpr (FOLD) {
        if (--left == 0) {
          fold(acc, tre, tim);
          left = cpt;
        }
      }
    };
    // pairs of chunks (sb0, then sb1), then an odd last chunk, already in
    // sb0: one exit from the loop, so the accumulators are updated in place
    int32_t ch = 0;
    for (; ch + 1 < nch; ch += 2) {
      stage(a, lo + (int64_t)(ch + 1) * C, wig, lane, sb1, sh1);
      if (regular)
        regular_chunk(reinterpret_cast<const float*>(sh0), reinterpret_cast<const float*>(sb0), lane,
                      gx, gy, gz, acc);
      tile_end();
      publish();
      if (ch + 2 < nch) stage(a, lo + (int64_t)(ch + 2) * C, wig, lane, sb0, sh0);
      if (regular)
        regular_chunk(reinterpret_cast<const float*>(sh1), reinterpret_cast<const float*>(sb1), lane,
                      gx, gy, gz, acc);
      tile_end();
      publish();
    }
    if (ch < nch) {
      if (regular)
        regular_chunk(reinterpret_cast<const float*>(sh0), reinterpret_cast<const float*>(sb0), lane,
                      gx, gy, gz, acc);
      tile_end();
      publish();
    }
    if constexpr (FOLD) fold(acc, tre, tim);
    (void)left;

    if (!regular) return;
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
        if constexpr (FOLD)
          dst[(int64_t)b * a.N + n] = make_float2(tre[t][r], tim[t][r]);
        else  // Re = P1 - P3, Im = P2 + P3 of the row's sums
          dst[(int64_t)b * a.N + n] =
              make_float2(acc[0][t][r] - acc[2][t][r], acc[1][t][r] + acc[2][t][r]);
      }
    }
  }
};

// Direct gather for the irregular waves of the four-sample engine, over the
// gather's launch rows as in MfmaDirect: lane l of wave w owns voxels
// 16 V w + l + 64 i, i < V / 4, taken four at a time; records are read with
// wave-uniform scalar loads (Mu_b = (fr, fi) of the reference column jref of
// vector b).  With a pair plan the launch rows are the plan's.
template <int T, int BC, int TRIG>
struct MfmaDirect4 {
  static constexpr int V = 16 * T / BC;
  static constexpr int ND = V / 4;     // voxels per lane
  static constexpr int NV = ND < 4 ? ND : 4;  // voxels per pass over the samples

  __device__ static void run(const MfmaArgs& a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kWorkgroup / 64) + (threadIdx.x >> 6);
    const int64_t vbase = wave * 16 * V;
    const int32_t row = (int32_t)blockIdx.y;
    int64_t m_split = a.m_split;
    if (a.pairs) {
      if (row >= a.pairs[2]) return;
      m_split = a.pairs[3];
    }
    int64_t lo, hi;
    row_range(m_split, a.mpad, row, lo, hi);
    if (vbase >= a.N) return;
    if (a.flags[wave]) return;   // a regular wave: the gather kernel summed it
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
          const float* blk = a.wb + (m >> 2) * (192 * T);
          const int k = (int)(m & 3);
          float mr[BC], mi[BC];
#pragma unroll
          for (int b = 0; b < BC; ++b) {
            const int cc = b * V + a.jref, t = cc / 16, p = 16 * k + cc % 16;
            mr[b] = blk[((t >> 2) * 64 + p) * 4 + (t & 3)];
            mi[b] = blk[(((T + t) >> 2) * 64 + p) * 4 + ((T + t) & 3)];
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

// ---------------------------------------------------------------------------
// Mirror pairs of the four-sample engine.  Take each group's reference at column jref, x_g = x[g V + jref],
// with factors f_j = Mu exp(i 2 pi k.(x_j - x_jref)).  A group h whose
// reference is exactly -x_g holds at column j the voxel -x_g + (x_j - x_jref)
// (both groups on the common offsets), so with (c, s) = (cos, sin)(2 pi k.x_g)
//   out[g][j] = sum_m (c + i s) f_j,      out[h][j] = sum_m (c - i s) f_j
// (e^{-i t} = conj e^{i t} for a real phase t).  Four real products
//   Pcr = sum c fr,  Pci = sum c fi,  Psr = sum s fr,  Psi = sum s fi
// give out[g] = (Pcr - Psi, Pci + Psr) and out[h] = (Pcr + Psi, Pci - Psr):
// one phase and 4 MFMAs per tile for two groups, where the three-product form
// takes two phases and 6 MFMAs.  On a grid with coordinates i - L/2 and jref
// the middle column, the partner of row (y, z) is row (-y, -z).

// Regularity of the gather's waves (the vote of the gather kernels), also
// requiring every present group's reference voxel to exist.
template <int V>
__global__ void __launch_bounds__(kWorkgroup) pair_flags_kernel(PairPlanArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kWorkgroup / 64) + (threadIdx.x >> 6);
  const int64_t vbase = wave * 16 * V;
  if (vbase >= a.N) return;
  const int64_t n0 = vbase + (int64_t)(lane & 15) * V;
  const bool gin = n0 < a.N;
  const float gx = gin ? a.x[n0] : 0.0f, gy = gin ? a.y[n0] : 0.0f, gz = gin ? a.z[n0] : 0.0f;
  bool reg = wave_regular<V, 16>(a.x, a.y, a.z, a.N, n0, lane, gx, gy, gz);
  const bool has_ref = gin && n0 + a.jref < a.N;
  reg = __all(reg && (!gin || has_ref));
  if (lane == 0) a.flags[wave] = reg ? 1 : 0;
  // each group's reference voxel, packed for the list kernel's reads
  const int64_t g = wave * 16 + lane;
  if (lane < 16 && g < a.G) {
    const int64_t r = n0 + a.jref;
    a.refs[g] = has_ref ? make_float4(a.x[r], a.y[r], a.z[r], 0.0f) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
}

constexpr int kListThreads = 1024;
constexpr int kListPer = 8;   // groups per thread and step of the list kernel

// Block-wide max / min of an int64 (every thread gets the result).
__device__ __forceinline__ int64_t block_reduce64(int64_t v, bool is_max, int64_t* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const int64_t o = __shfl_xor(v, d);
    v = is_max ? (o > v ? o : v) : (o < v ? o : v);
  }
  if (lane == 0) sh[w] = v;
  __syncthreads();
  v = sh[0];
  for (int i = 1; i < kListThreads / 64; ++i) v = is_max ? (sh[i] > v ? sh[i] : v) : (sh[i] < v ? sh[i] : v);
  __syncthreads();
  return v;
}

// Exclusive block scan of two counts; also returns the block totals.
__device__ __forceinline__ void block_exscan2(int a, int b, int& ea, int& eb, int& ta, int& tb, int* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int ia = a, ib = b;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int xa = __shfl_up(ia, d), xb = __shfl_up(ib, d);
    if (lane >= d) { ia += xa; ib += xb; }
  }
  if (lane == 63) { sh[w] = ia; sh[16 + w] = ib; }
  __syncthreads();
  int oa = 0, ob = 0;
  ta = 0; tb = 0;
  for (int i = 0; i < kListThreads / 64; ++i) {
    if (i < w) { oa += sh[i]; ob += sh[16 + i]; }
    ta += sh[i]; tb += sh[16 + i];
  }
  __syncthreads();
  ea = oa + ia - a;
  eb = ob + ib - b;
}

// One workgroup: finds the index sum S of the mirror pairs from the last full
// group of a regular wave and its mirror, classifies every group (partner
// h = S - g checked exactly: both full, on regular waves, reference -x_g;
// the smaller index of a pair is listed with its partner, the larger not at
// all; every other group of a regular wave alone) and lists them in index
// order, then picks the launch rows: in [rows_lo, rows_hi] the count whose
// workgroups (Q per row) fill whole rounds of the resident slots best, the
// fewest rows among equals.
__global__ void __launch_bounds__(kListThreads) pair_list_kernel(PairPlanArgs a) {
  __shared__ int64_t red[kListThreads / 64];
  __shared__ int scan[32];
  const int tid = threadIdx.x;
  const int64_t V = a.V, G = a.G, Gfull = a.N / a.V;
  const int64_t waves = (G + 15) / 16;
  int64_t last = -1;
  for (int64_t w = tid; w < waves; w += kListThreads) {
    if (!a.flags[w]) continue;
    int64_t g = 16 * w + 15;
    if (g > Gfull - 1) g = Gfull - 1;
    if (g >= 16 * w && g > last) last = g;
  }
  last = block_reduce64(last, true, red);
  int64_t S = -1;
  const float4* refs = a.refs;
  if (a.pair && last >= 0) {
    const float4 rl = refs[last];
    const float tx = -rl.x, ty = -rl.y, tz = -rl.z;
    for (int64_t base = 0; base < Gfull; base += (int64_t)kListThreads * kListPer) {
      int64_t mine = INT64_MAX;
      for (int i = 0; i < kListPer; ++i) {
        const int64_t g = base + (int64_t)i * kListThreads + tid;
        if (g < Gfull && a.flags[g >> 4]) {
          const float4 r = refs[g];
          if (r.x == tx && r.y == ty && r.z == tz && g < mine) mine = g;
        }
      }
      const int64_t found = block_reduce64(mine, false, red);
      if (found != INT64_MAX) {
        S = last + found;
        break;
      }
    }
  }
  int2* list = reinterpret_cast<int2*>(a.plan + kPairHeader);
  int64_t cp = 0, cs = 0;
  for (int64_t base = 0; base < G; base += (int64_t)kListThreads * kListPer) {
    const int64_t g0 = base + (int64_t)tid * kListPer;
    int part[kListPer];  // -2: not listed, -1: alone, else the partner
    int np = 0, ns = 0;
#pragma unroll
    for (int i = 0; i < kListPer; ++i) {
      const int64_t g = g0 + i;
      part[i] = -2;
      if (g >= G || !a.flags[g >> 4]) continue;
      part[i] = -1;
      const int64_t h = S - g;
      if (S >= 0 && g < Gfull && h >= 0 && h < Gfull && h != g && a.flags[h >> 4]) {
        const float4 rg = refs[g], rh = refs[h];
        if (rh.x == -rg.x && rh.y == -rg.y && rh.z == -rg.z) part[i] = h > g ? (int)h : -2;
      }
      np += part[i] >= 0;
      ns += part[i] == -1;
    }
    int ep, es, tp, ts;
    block_exscan2(np, ns, ep, es, tp, ts, scan);
    int64_t wp = cp + ep, wsg = cs + es;
#pragma unroll
    for (int i = 0; i < kListPer; ++i) {
      const int g = (int)(g0 + i);
      if (part[i] >= 0) list[wp++] = make_int2(g, part[i]);
      else if (part[i] == -1) list[G - 1 - (wsg++)] = make_int2(g, -1);
    }
    cp += tp;
    cs += ts;
  }
  if (tid == 0) {
    const int64_t E = cp + cs, U = (E + 15) / 16, Q = (U + kMfma4Waves - 1) / kMfma4Waves;
    int32_t R = a.rows_lo;
    int64_t ms = 0;
    double best = -1.0;
    for (int32_t r = a.rows_lo; r <= a.rows_hi; ++r) {
      int64_t m = (a.mpad + r - 1) / r;
      m = (m + kMfmaChunk - 1) / kMfmaChunk * kMfmaChunk;
      const int64_t reff = m > 0 ? (a.mpad + m - 1) / m : 1;
      if (reff != r && r != a.rows_lo) continue;  // a count that leaves empty rows
      const int64_t items = Q * reff, rounds = (items + a.resident - 1) / a.resident;
      const double eff = rounds > 0 ? (double)items / (double)(rounds * a.resident) : 1.0;
      if (eff > best + 1e-3) {
        best = eff;
        R = (int32_t)(reff < 1 ? 1 : reff);
        ms = m;
      }
    }
    a.plan[0] = (int32_t)E;
    a.plan[1] = (int32_t)cp;
    a.plan[2] = R;
    a.plan[3] = (int32_t)ms;
    a.plan[4] = (int32_t)U;
    a.plan[5] = (int32_t)Q;
    a.plan[6] = (int32_t)(S < 0 ? -1 : S);
  }
}

// The gather over the pair plan's list: workgroup item = (row, Q slot),
// row-major, each wave 16 list entries, all summed in the four-product form
// (a group without a partner gets its own sums only: on the grids the
// pairing is made for these are the few rows without a mirror row, and one
// form keeps the kernel at 3 waves per SIMD).  The chunk staging and loop
// shape are MfmaGather4's.
// The pair gather sums each launch row in blocks of a.tile samples (a
// multiple of the 16-sample chunk): each block's sums are added into the
// row's outputs in memory, which the wave owns in that row -- blocked
// summation with the running totals in memory instead of registers.
template <int BC, int TRIG>
struct MfmaPairGather4 {
  static constexpr int T = 8;
  using Base = MfmaGather4<T, BC, TRIG, false>;
  static constexpr int V = Base::V, C = Base::C, NW = Base::NW, QF = Base::QF, HK = Base::HK, NH = Base::NH;

  // fr (u = 0) and fi (u = 1) slices 2 u + h of block q: bv[u T + t], t in half h
  __device__ static __forceinline__ void load_pair_half(const float* __restrict__ wb, int q, int lane, int h,
                                                        float (&bv)[2 * T]) {
    const float* pp = wb + q * QF;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int sl = 2 * u + h;
      const float4 v = *reinterpret_cast<const float4*>(pp + (sl * 64 + lane) * 4);
      bv[4 * sl] = v.x; bv[4 * sl + 1] = v.y; bv[4 * sl + 2] = v.z; bv[4 * sl + 3] = v.w;
    }
  }

  template <int H>
  __device__ static __forceinline__ void mfmas_pair_half(float c, float s, const float (&bv)[2 * T],
                                                         f32x4 (&acc)[3][T], f32x4 (&accx)[T]) {
#pragma unroll
    for (int u = 0; u < T / 2; ++u) {
      const int t = H * (T / 2) + u;
      acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(c, bv[t], acc[0][t], 0, 0, 0);
      acc[1][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(c, bv[T + t], acc[1][t], 0, 0, 0);
      acc[2][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(s, bv[t], acc[2][t], 0, 0, 0);
      accx[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(s, bv[T + t], accx[t], 0, 0, 0);
    }
  }

  // One chunk of the four-product form, pipelined as the three-product HW
  // chunk (B entries half a block ahead, the phase right before its MFMAs).
  __device__ static __forceinline__ void pair_chunk(const float* __restrict__ hb, const float* __restrict__ wb,
                                                    int lane, float rx, float ry, float rz, f32x4 (&acc)[3][T],
                                                    f32x4 (&accx)[T]) {
    constexpr int NQ = C / 4;
    float hc[HK], bv[2 * T];
    Base::load_header(hb, 0, lane, hc);
    load_pair_half(wb, 0, lane, 0, bv);
    load_pair_half(wb, 0, lane, 1, bv);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float hn[HK];
      if (q + 1 < NQ) Base::load_header(hb, q + 1, lane, hn);
      sched_fence();
      float c, s;
      phase_sincos<TRIG>(hc, rx, ry, rz, c, s);
      mfmas_pair_half<0>(c, s, bv, acc, accx);
      sched_fence();
      if (q + 1 < NQ) load_pair_half(wb, q + 1, lane, 0, bv);
      sched_fence();
      mfmas_pair_half<1>(c, s, bv, acc, accx);
      sched_fence();
      if (q + 1 < NQ) {
        load_pair_half(wb, q + 1, lane, 1, bv);
#pragma unroll
        for (int i = 0; i < HK; ++i) hc[i] = hn[i];
      }
      sched_fence();
    }
  }

  __device__ static __forceinline__ int2 entry(const int2* list, int64_t e, int64_t E, int64_t Cp, int64_t gcap) {
    if (e >= E) return make_int2(-1, -1);
    return list[e < Cp ? e : gcap - 1 - (e - Cp)];
  }

  __device__ static void run(const MfmaArgs& a) {
    __shared__ float4 sb0[C / 4 * QF / 4], sb1[C / 4 * QF / 4];
    __shared__ float4 sh0[NH], sh1[NH];
    const int32_t* P = a.pairs;
    const int64_t E = P[0], Cp = P[1], U = P[4], Q = P[5];
    const int32_t R = P[2];
    const int64_t m_split = P[3];
    const int64_t item = blockIdx.x;
    if (item >= Q * R) return;   // the whole workgroup
    const int tid = threadIdx.x, lane = tid & 63;
    const int wig = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int32_t row = (int32_t)(item / Q);
    const int64_t slot = (item - (int64_t)row * Q) * NW + wig;
    const bool live = slot < U;   // waves past the list only help stage the chunks
    const int2* list = reinterpret_cast<const int2*>(P + kPairHeader);
    const int2 me = entry(list, slot * 16 + (lane & 15), E, Cp, a.gcap);
    float rx = 0.0f, ry = 0.0f, rz = 0.0f;
    if (me.x >= 0) {
      const int64_t r = (int64_t)me.x * V + a.jref;
      rx = a.x[r]; ry = a.y[r]; rz = a.z[r];
    }
    int64_t lo, hi;
    row_range(m_split, a.mpad, row, lo, hi);
    const int32_t nch = (int32_t)((hi - lo) / C);
    f32x4 acc[3][T], accx[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      acc[0][t] = f32x4{}; acc[1][t] = f32x4{}; acc[2][t] = f32x4{}; accx[t] = f32x4{};
    }
    float2* dst = a.partial ? a.partial + (int64_t)row * BC * a.N : a.out;
    const int c = lane & 15;
    // out[g] = (Pcr - Psi, Pci + Psr); out[h] = (Pcr + Psi, Pci - Psr) for a partner h.
    // ADD: the block's sums are added to what earlier blocks of the row wrote.
    auto write = [&](bool add) {
      const int64_t e0 = slot * 16;
      float2* out = dst;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (lane >> 4) + r;
        const int2 en = entry(list, e0 + i, E, Cp, a.gcap);
        if (en.x < 0) continue;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const int cc = 16 * t + c;
          const int b = cc / V, j = cc % V;
          const int64_t n = (int64_t)en.x * V + j;
          float2 vg = make_float2(acc[0][t][r] - accx[t][r], acc[1][t][r] + acc[2][t][r]);
          if (n < a.N) {
            float2* o = out + (int64_t)b * a.N + n;
            if (add) { const float2 w = *o; vg.x += w.x; vg.y += w.y; }
            *o = vg;
          }
          if (en.y >= 0) {
            float2 vh = make_float2(acc[0][t][r] + accx[t][r], acc[1][t][r] - acc[2][t][r]);
            float2* o = out + (int64_t)b * a.N + (int64_t)en.y * V + j;
            if (add) { const float2 w = *o; vh.x += w.x; vh.y += w.y; }
            *o = vh;
          }
        }
      }
    };
    // blocks of a.tile samples (an even number of chunks): each block's sums
    // are added into the row's outputs (this wave owns them in this row) and
    // the accumulators restart.  The block loop is outside the double-buffered
    // chunk loop, which keeps its pipeline across block ends (the last pair
    // of a block stages the next block's first chunk); a per-chunk block test
    // inside it measured 11 % slower.
    const int32_t block = (int32_t)(a.tile / C);
    bool written = false;
    auto chunk = [&](const float4* sh, const float4* sb) {
      if (live)
        pair_chunk(reinterpret_cast<const float*>(sh), reinterpret_cast<const float*>(sb), lane, rx, ry, rz,
                   acc, accx);
    };
    if (nch > 0) Base::stage(a, lo, wig, lane, sb0, sh0);
    Base::publish();
    int32_t ch = 0;
    while (ch < nch) {
      const int32_t end = nch - ch > block ? ch + block : nch;
      for (; ch + 1 < end; ch += 2) {
        Base::stage(a, lo + (int64_t)(ch + 1) * C, wig, lane, sb1, sh1);
        chunk(sh0, sb0);
        Base::publish();
        if (ch + 2 < nch) Base::stage(a, lo + (int64_t)(ch + 2) * C, wig, lane, sb0, sh0);
        chunk(sh1, sb1);
        Base::publish();
      }
      if (ch < end) {  // an odd last chunk of the row (blocks hold an even number)
        chunk(sh0, sb0);
        Base::publish();
        ++ch;
      }
      if (ch < nch && live) {
        write(written);
        written = true;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          acc[0][t] = f32x4{}; acc[1][t] = f32x4{}; acc[2][t] = f32x4{}; accx[t] = f32x4{};
        }
      }
    }
    if (!live) return;
    write(written);
  }
};

// Adds the pair plan's launch rows of partial sums in row order.
__global__ void __launch_bounds__(kWorkgroup)
reduce_dev_rows_kernel(const float2* __restrict__ partial, float2* __restrict__ out, int64_t count,
                       const int32_t* __restrict__ plan) {
  const int64_t i = (int64_t)blockIdx.x * kWorkgroup + threadIdx.x;
  if (i >= count) return;
  const int32_t rows = plan[2];
  float re = 0.0f, im = 0.0f;
  for (int32_t p = 0; p < rows; ++p) {
    const float2 v = partial[(int64_t)p * count + i];
    re += v.x;
    im += v.y;
  }
  out[i] = make_float2(re, im);
}

// Resident waves per SIMD the gather is compiled for: 4 with one tile of 32
// complex columns (48 accumulators + 32 running totals, <= 128 VGPRs; 25 KB
// of LDS per 4-wave workgroup), 2 with two tiles (96 accumulators + 64
// running totals, <= 256 VGPRs; 50 KB of LDS per workgroup).
template <int T>
constexpr int mfma_waves_per_simd() { return T == 2 ? 4 : 2; }

template <int T, int BC, int TRIG>
__global__ void __launch_bounds__(kWorkgroup) __attribute__((amdgpu_waves_per_eu(mfma_waves_per_simd<T>())))
mfma_gather_kernel(MfmaArgs a) {
  MfmaGather<T, BC, TRIG>::run(a);
}

template <int T, int BC, int TRIG>
__global__ void __launch_bounds__(kWorkgroup) mfma_direct_kernel(MfmaArgs a) {
  MfmaDirect<T, BC, TRIG>::run(a);
}

// Four-sample engine: 4-wave workgroups of ~49 KB of LDS.  With running
// totals 2 waves per SIMD (two workgroups per CU); without them (the launch
// row one summation block) the kernel fits 168 VGPRs: 3 waves per SIMD,
// three workgroups per CU.
template <bool FOLD>
constexpr int mfma4_waves_per_simd() { return FOLD ? 2 : 3; }

template <int T, int BC, int TRIG, bool FOLD>
__global__ void __launch_bounds__(64 * kMfma4Waves)
__attribute__((amdgpu_waves_per_eu(mfma4_waves_per_simd<FOLD>())))
mfma4_gather_kernel(MfmaArgs a) {
  MfmaGather4<T, BC, TRIG, FOLD>::run(a);
}

template <int T, int BC, int TRIG>
__global__ void __launch_bounds__(kWorkgroup) mfma4_direct_kernel(MfmaArgs a) {
  MfmaDirect4<T, BC, TRIG>::run(a);
}

// Mirror-pair gather: 128 accumulators, 2 waves per SIMD (two 4-wave
// workgroups of ~49 KB of LDS per CU, pair_resident_wgs in all).  (At 3 waves
// per SIMD the HW kernel fits 168 VGPRs only by spilling the block write's
// addresses into the chunk loop, 2 % slower; without the block write it
// fitted, but measured no faster than at 2 waves: the matrix pipe is busy
// 0.93 of the time either way.)
template <int BC, int TRIG>
__global__ void __launch_bounds__(64 * kMfma4Waves) __attribute__((amdgpu_waves_per_eu(2)))
mfma4_pair_kernel(MfmaArgs a) {
  MfmaPairGather4<BC, TRIG>::run(a);
}

struct PairFns {
  void (*flags)(PairPlanArgs);
  void (*gather)(MfmaArgs);
  void (*direct)(MfmaArgs);
};

template <int BC>
PairFns pair_fns(int trig) {
  if (trig == kTrigHw)
    return {pair_flags_kernel<128 / BC>, mfma4_pair_kernel<BC, kTrigHw>, mfma4_direct_kernel<8, BC, kTrigHw>};
  return {pair_flags_kernel<128 / BC>, mfma4_pair_kernel<BC, kTrigAccurate>,
          mfma4_direct_kernel<8, BC, kTrigAccurate>};
}

PairFns select_pair(int BC, int trig) {
  switch (BC) {
    case 1: return pair_fns<1>(trig);
    case 2: return pair_fns<2>(trig);
    case 4: return pair_fns<4>(trig);
    case 8: return pair_fns<8>(trig);
    case 16: return pair_fns<16>(trig);
    default: return {nullptr, nullptr, nullptr};
  }
}

using MfmaFn = void (*)(MfmaArgs);
using DirectFn = void (*)(MfmaArgs);

struct MfmaPair {
  MfmaFn gather;
  DirectFn direct;
  MfmaFn gather_row;  // four-sample engine: the row is one summation block
};

template <int T, int BC>
MfmaPair pick_mfma(int trig) {
  if constexpr (T == 8) {
    if (trig == kTrigHw)
      return {mfma4_gather_kernel<T, BC, kTrigHw, true>, mfma4_direct_kernel<T, BC, kTrigHw>,
              mfma4_gather_kernel<T, BC, kTrigHw, false>};
    return {mfma4_gather_kernel<T, BC, kTrigAccurate, true>, mfma4_direct_kernel<T, BC, kTrigAccurate>,
            mfma4_gather_kernel<T, BC, kTrigAccurate, false>};
  } else {
    if (trig == kTrigHw) return {mfma_gather_kernel<T, BC, kTrigHw>, mfma_direct_kernel<T, BC, kTrigHw>, nullptr};
    return {mfma_gather_kernel<T, BC, kTrigAccurate>, mfma_direct_kernel<T, BC, kTrigAccurate>, nullptr};
  }
}

template <int T>
MfmaPair select_bc(int trig, int BC) {
  switch (BC) {
    case 1: return pick_mfma<T, 1>(trig);
    case 2: return pick_mfma<T, 2>(trig);
    case 4: return pick_mfma<T, 4>(trig);
    case 8: return pick_mfma<T, 8>(trig);
    case 16: return pick_mfma<T, 16>(trig);
    default: return {nullptr, nullptr, nullptr};
  }
}

MfmaPair select_mfma(int trig, int T, int BC) {
  if (T == 2) return select_bc<2>(trig, BC);
  if (T == 4) return select_bc<4>(trig, BC);
  if (T == 8) return select_bc<8>(trig, BC);
  return {nullptr, nullptr, nullptr};
}


}  // namespace

bool mfma_supported(int T, int BC) { return select_mfma(kTrigHw, T, BC).gather != nullptr; }

hipError_t launch_mfma_records(int is_q, int trig, int T, int BC, const MfmaRecordArgs& a,
                               hipStream_t s) {
  if (a.mpad <= 0) return hipSuccess;
  if (!mfma_supported(T, BC) || a.mpad % kMfmaChunk != 0) return hipErrorInvalidValue;
  if (T == 8) {  // 32 lanes per sample, four columns each
    const int64_t blocks = (a.mpad * 32 + kWorkgroup - 1) / kWorkgroup;
    hipLaunchKernelGGL(mfma4_records_kernel, dim3((unsigned)blocks), dim3(kWorkgroup), 0, s, a, is_q,
                       trig, BC);
    return hipGetLastError();
  }
  const int64_t lanes = a.mpad * 16 * T;
  const int64_t blocks = (lanes + kWorkgroup - 1) / kWorkgroup;
  hipLaunchKernelGGL(mfma_records_kernel, dim3((unsigned)blocks), dim3(kWorkgroup), 0, s, a, is_q,
                     trig, T, BC);
  return hipGetLastError();
}

hipError_t launch_mfma_pair_gather(int trig, int BC, const PairPlanArgs& pa, const MfmaArgs& a, hipStream_t s) {
  const PairFns fn = select_pair(BC, trig);
  if (!fn.gather || !a.pairs || a.pairs != pa.plan || !a.flags || a.flags != pa.flags || pa.V != 128 / BC ||
      pa.refs != reinterpret_cast<const float4*>(reinterpret_cast<const char*>(pa.plan) + pair_list_bytes(pa.G)) ||
      pa.rows_lo < 1 || pa.rows_hi < pa.rows_lo || (pa.rows_hi > 1 && !a.partial) || pa.jref < 0 ||
      pa.jref >= pa.V || (pa.N > 0 && pa.jref >= pa.N) || a.jref != pa.jref || a.gcap != pa.G ||
      pa.G != (pa.N + pa.V - 1) / pa.V || a.N != pa.N || a.mpad != pa.mpad || a.mpad % kMfmaChunk != 0 ||
      a.tile <= 0 || a.tile % (2 * kMfma4Chunk) != 0 || pa.resident != pair_resident_wgs(trig))
    return hipErrorInvalidValue;
  if (a.N <= 0) return hipSuccess;
  const int64_t waves = mfma_gather_waves(a.N, 8, BC);
  const int64_t fblocks = (waves + kWorkgroup / 64 - 1) / (kWorkgroup / 64);
  hipLaunchKernelGGL(fn.flags, dim3((unsigned)fblocks), dim3(kWorkgroup), 0, s, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pair_list_kernel, dim3(1), dim3(kListThreads), 0, s, pa);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // workgroup items: at most every wave alone (Q <= waves / 4) on the most rows
  const int64_t qmax = (waves + kMfma4Waves - 1) / kMfma4Waves;
  hipLaunchKernelGGL(fn.gather, dim3((unsigned)(qmax * pa.rows_hi)), dim3(64 * kMfma4Waves), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn.direct, dim3((unsigned)fblocks, (unsigned)pa.rows_hi), dim3(kWorkgroup), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pair_plan(int BC, const PairPlanArgs& pa, hipStream_t s) {
  const PairFns fn = select_pair(BC, kTrigHw);
  if (!fn.flags || !pa.plan || !pa.flags || pa.V != 128 / BC || pa.jref < 0 || pa.jref >= pa.V ||
      (pa.N > 0 && pa.jref >= pa.N) || pa.G != (pa.N + pa.V - 1) / pa.V || pa.rows_lo < 1 || pa.rows_hi < pa.rows_lo ||
      pa.refs != reinterpret_cast<const float4*>(reinterpret_cast<const char*>(pa.plan) + pair_list_bytes(pa.G)))
    return hipErrorInvalidValue;
  if (pa.N <= 0) return hipSuccess;
  const int64_t waves = (pa.G + 15) / 16;
  const int64_t fblocks = (waves + kWorkgroup / 64 - 1) / (kWorkgroup / 64);
  hipLaunchKernelGGL(fn.flags, dim3((unsigned)fblocks), dim3(kWorkgroup), 0, s, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pair_list_kernel, dim3(1), dim3(kListThreads), 0, s, pa);
  return hipGetLastError();
}

hipError_t launch_reduce_dev_rows(int BC, const int32_t* plan, const GatherArgs& a, hipStream_t s) {
  if (!a.partial || a.N <= 0) return hipSuccess;
  if (!plan) return hipErrorInvalidValue;
  const int64_t count = (int64_t)BC * a.N;
  const int64_t rblocks = (count + kWorkgroup - 1) / kWorkgroup;
  hipLaunchKernelGGL(reduce_dev_rows_kernel, dim3((unsigned)rblocks), dim3(kWorkgroup), 0, s, a.partial, a.out,
                     count, plan);
  return hipGetLastError();
}

// Launches the matrix-core kernel (regular waves) and the direct kernel
// (irregular waves), each with one launch row per sample split.
hipError_t launch_mfma_gather(int trig, int T, int BC, int32_t splits, const MfmaArgs& a,
                              hipStream_t s) {
  MfmaPair fn = select_mfma(trig, T, BC);
  if (!fn.gather || splits < 1 || (splits > 1) != (a.partial != nullptr) || !a.flags) return hipErrorInvalidValue;
  if (a.mpad % kMfmaChunk != 0 || a.m_split % kMfmaChunk != 0 || a.tile % kMfmaChunk != 0 ||
      a.tile <= 0)
    return hipErrorInvalidValue;
  if (a.N <= 0) return hipSuccess;
  const int64_t waves = mfma_gather_waves(a.N, T, BC);
  // gather: workgroups of kWorkgroup / 64 waves (two-sample engine) or
  // kMfma4Waves (four-sample engine); direct: workgroups of kWorkgroup / 64
  // waves over the same wave numbering
  const int wg_waves = T == 8 ? kMfma4Waves : kWorkgroup / 64;
  const int64_t blocks = (waves + wg_waves - 1) / wg_waves;
  const int64_t dblocks = (waves + kWorkgroup / 64 - 1) / (kWorkgroup / 64);
  // a tile as long as a launch row never folds: the four-sample engine then
  // keeps no running totals
  const MfmaFn g = (fn.gather_row && a.tile >= a.m_split) ? fn.gather_row : fn.gather;
  hipLaunchKernelGGL(g, dim3((unsigned)blocks, (unsigned)splits), dim3(64 * wg_waves), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn.direct, dim3((unsigned)dblocks, (unsigned)splits), dim3(kWorkgroup), 0, s, a);
  return hipGetLastError();
}

}  // namespace ncmri
