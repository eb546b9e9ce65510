// gfx950 matrix-core forward operator (PMPP ch. 17 "Iterative MRI
// reconstruction", section 17.2: F models the imaging physics, F[m][n] =
// phi_m exp(-i 2 pi k_m . x_n), the matrix whose conjugate transpose the F^H D
// kernels apply; section 17.3 step 3 synthesises scan data from an image):
//
//   D[b][m] = phi_m sum_n rho_b[n] exp(-i 2 pi k_m . x_n)
//
// The adjoint engine with the roles of samples and voxels swapped.  With the
// voxels in groups of V at the first group's offsets d_j (x_n = x_g + d_j),
//
//   D[b][m] = phi_m sum_j exp(-i 2 pi k_m . d_j) G[m][j][b],
//   G[m][j][b] = sum_g exp(-i 2 pi k_m . x_g) rho_b[x_g + d_j],
//
// and for 32 samples and 16 T complex columns (j, b) the sum over groups is a
// complex matrix product (samples x groups) * (groups x columns) with entries
// (c - i s)(rr + i ri), (c, s) = (cos, sin)(2 pi k_m . x_g).  As in the
// adjoint it is formed with three real products (the three-multiplication
// form of a complex product):
//
//   P1 = sum (c - s) rr,   P2 = sum (c + s) ri,   P3 = sum s (rr + ri),
//   Re = P1 + P3,          Im = P2 - P3,
//
// each one v_mfma_f32_32x32x2_f32 per tile of 32 complex columns with K = 2
// running over a pair of groups.  Each wave owns 32 samples (lane l: sample
// l % 32 at group 2 h + l / 32 of pair h; one phase, its sine and its cosine
// per lane and pair); the packed image is streamed through LDS in 32-group
// chunks by LDS DMA, shared by the 4 waves of a workgroup, exactly as the
// adjoint streams its sample records.  After the last group the wave writes G
// to LDS and lanes 0-31 contract their sample's row with
// exp(-i 2 pi k_m . d_j) and multiply by phi_m.
//
// Groups whose voxels are not on the first group's offsets are packed as
// zeros and flagged; one workgroup then lists them in increasing order
// (fwd_list_kernel) and fwd_direct_kernel adds their voxels per sample on the
// VALU after the launch rows have been reduced (it returns at once when the
// list is empty, as on a grid).
#include "fhd_internal.h"
#include "fhd_mfma_common.h"
#include "fhd_trig.h"
#include "fhd_forward_common.h"

namespace ncmri {
namespace {

// Group g of V voxels (first voxel n0 = g V) is on the common offsets when
// every voxel n0 + j < N satisfies x[n0 + j] - x[n0] == x[j] - x[0] (exact,
// in double; likewise y, z).  This checks one offset j.
__device__ bool voxel_on_offsets(const float* __restrict__ x, const float* __restrict__ y,
                                 const float* __restrict__ z, int64_t N, int64_t n0, int j) {
  const int64_t n = n0 + j;
  if (j == 0 || n >= N) return true;
  return (double)x[n] - (double)x[n0] == (double)x[j] - (double)x[0] &&
         (double)y[n] - (double)y[n0] == (double)y[j] - (double)y[0] &&
         (double)z[n] - (double)z[n0] == (double)z[j] - (double)z[0];
}

// ---------------------------------------------------------------------------
// Packing: one lane per (padded group, complex column); the 16 T lanes of a
// group (a divisor of the workgroup) check one offset each and combine the
// result in LDS.
__global__ void __launch_bounds__(kWorkgroup) fwd_pack_kernel(FwdArgs a, int T, int BC) {
  __shared__ int regular_s[kWorkgroup / 32];
  const int cols = 16 * T;
  const int64_t idx = (int64_t)blockIdx.x * kWorkgroup + threadIdx.x;
  const int64_t g = idx / cols;
  const int cc = (int)(idx - g * cols);
  const int lg = threadIdx.x / cols;  // the group's slot in this workgroup
  const bool live = g < a.gpad;
  const int V = cols / BC;
  const int64_t n0 = g * V;
  const bool inside = live && n0 < a.N;
  if (threadIdx.x < kWorkgroup / cols) regular_s[threadIdx.x] = 1;
  __syncthreads();
  if (inside && cc < V && !voxel_on_offsets(a.x, a.y, a.z, a.N, n0, cc)) regular_s[lg] = 0;
  __syncthreads();
  const bool reg = regular_s[lg] != 0;
  if (!live) return;
  if (cc == 0) {
    float* h = a.ghdr + g * 4;
    h[0] = inside ? a.x[n0] : 0.0f;
    h[1] = inside ? a.y[n0] : 0.0f;
    h[2] = inside ? a.z[n0] : 0.0f;
    h[3] = reg ? 0.0f : 1.0f;
  }
  const int b = cc / V, j = cc % V;
  const int64_t n = n0 + j;
  const float2 r = (inside && reg && n < a.N) ? a.rho[(int64_t)b * a.N + n] : make_float2(0.0f, 0.0f);
  if (T == 8) {
    // four-group engine: entry e = u T + t (u = re, im, re + im; tile t =
    // cc / 16) of lane p = 16 (g % 4) + cc % 16 in float4 slices of a block of
    // four groups: [g / 4][e / 4][p][e % 4]
    const int t = cc / 16, lp = 16 * (int)(g & 3) + cc % 16;
    float* blk = a.gwb + (g >> 2) * (192 * T);
    blk[((t >> 2) * 64 + lp) * 4 + (t & 3)] = r.x;
    blk[(((T + t) >> 2) * 64 + lp) * 4 + ((T + t) & 3)] = r.y;
    blk[(((2 * T + t) >> 2) * 64 + lp) * 4 + ((2 * T + t) & 3)] = r.x + r.y;
    return;
  }
  // entry of column c = cc % 32 of tile t = cc / 32 at row g % 2 of the pair
  const int P = T / 2;
  const int t = cc / 32, lp = 32 * (int)(g & 1) + cc % 32;
  float* pair = a.gwb + (g >> 1) * (192 * P);
  float* wr = pair + lp * (2 * P) + t;
  wr[0] = r.x; wr[P] = r.y;
  pair[128 * P + lp * P + t] = r.x + r.y;
}

// Lists the flagged groups: each of the workgroup's lanes counts the flags of
// a contiguous range of groups, an exclusive scan of the counts in LDS gives
// each range's place, and the ranges write their group indices in order.
// glist[0] = count, glist[1 + i] = i-th flagged group.
__global__ void __launch_bounds__(kWorkgroup) fwd_list_kernel(FwdArgs a, int V) {
  __shared__ int32_t cnt[kWorkgroup];
  const int tid = threadIdx.x;
  const int64_t G = (a.N + V - 1) / V;
  const int64_t per = (G + kWorkgroup - 1) / kWorkgroup;
  const int64_t g0 = tid * per < G ? tid * per : G;
  const int64_t g1 = g0 + per < G ? g0 + per : G;
  // flagged: off the common offsets, or (mirror pairs) in an irregular wave
  auto flagged = [&](int64_t g) { return a.wflags ? a.wflags[g >> 4] == 0 : a.ghdr[g * 4 + 3] != 0.0f; };
  int32_t c = 0;
  for (int64_t g = g0; g < g1; ++g) c += flagged(g) ? 1 : 0;
  cnt[tid] = c;
  __syncthreads();
  // exclusive prefix sum (Hillis-Steele on the inclusive sums, then shift)
  for (int off = 1; off < kWorkgroup; off *= 2) {
    const int32_t v = tid >= off ? cnt[tid - off] : 0;
    __syncthreads();
    cnt[tid] += v;
    __syncthreads();
  }
  int32_t pos = cnt[tid] - c;
  if (tid == kWorkgroup - 1) a.glist[0] = cnt[tid];
  for (int64_t g = g0; g < g1; ++g)
    if (flagged(g)) a.glist[1 + pos++] = (int32_t)g;
}

// ---------------------------------------------------------------------------
// Matrix-core gather over the regular groups.
template <int T, int BC, int TRIG>
struct FwdGather {
  static constexpr int V = 16 * T / BC;
  static constexpr int P = T / 2;                 // tiles of 32 complex columns
  static constexpr int C = kMfmaChunk;
  static constexpr int NW = kWorkgroup / 64;
  static constexpr int PF = 192 * P;              // image floats per pair of groups
  static constexpr int NB = C / 2 * PF * 4 / 1024;  // 1 KiB image blocks per chunk
  static constexpr int NH = C;                    // header float4s per chunk (one per group)
  static constexpr int SB = C / 2 * PF / 4;       // float4s of one staging buffer
  static constexpr int GW = 32 * 32 * P * 2 / 4;  // float4s of one wave's G block
  static constexpr int LDS4 = 2 * SB > NW * GW ? 2 * SB : NW * GW;
  static_assert(P >= 1 && V >= 1 && V * BC == 16 * T, "group shape");
  static_assert(NB % NW == 0 && NH <= 64, "chunk staging");

  __device__ static __forceinline__ void stage(const FwdArgs& a, int64_t g, int wig, int lane,
                                               float4* lb, float4* lh) {
    const __amdgpu_buffer_rsrc_t rb =
        buffer_rsrc(reinterpret_cast<const float4*>(a.gwb) + (g / 2) * (PF / 4), NB * 64 * 16);
#pragma unroll
    for (int i = 0; i < NB / NW; ++i) {
      const int blk = i * NW + wig;
      lds_dma16(rb, (blk * 64 + lane) * 16, lb + blk * 64);
    }
    if (wig == 0 && lane < NH)
      lds_dma16(buffer_rsrc(reinterpret_cast<const float4*>(a.ghdr) + g, NH * 16), lane * 16, lh);
  }

  __device__ static __forceinline__ void publish() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Header of the lane's group and its B entries of pair h of the chunk.
  __device__ static __forceinline__ void load_pair(const float* __restrict__ hb,
                                                   const float* __restrict__ wb, int h, int lane,
                                                   float (&hs)[3], float (&bv)[3 * P]) {
    const float* hp = hb + (2 * h + (lane >> 5)) * 4;
#pragma unroll
    for (int i = 0; i < 3; ++i) hs[i] = hp[i];
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

  // One chunk of 32 groups (16 pairs), pipelined by one pair like the
  // adjoint's loop (and, on the accurate path, with the next pair's A entries
  // computed right after this pair's MFMAs, as the adjoint does).
  __device__ static __forceinline__ void chunk(const float* __restrict__ hb, const float* __restrict__ wb,
                                               int lane, const SampleK<TRIG>& k, f32x16 (&acc)[3][P]) {
    constexpr int NP = C / 2;
    float hc[3], bc[3 * P], av[3];
    load_pair(hb, wb, 0, lane, hc, bc);
    if constexpr (TRIG != kTrigHw) fwd_entries<TRIG>(k, hc, av);
#pragma unroll
    for (int h = 0; h < NP; ++h) {
      float hn[3], bn[3 * P];
      if (h + 1 < NP) load_pair(hb, wb, h + 1, lane, hn, bn);
      sched_fence();
      if constexpr (TRIG == kTrigHw) fwd_entries<TRIG>(k, hc, av);
      mfmas(av, bc, acc);
      sched_fence();
      if (h + 1 < NP) {
        if constexpr (TRIG != kTrigHw) fwd_entries<TRIG>(k, hn, av);
#pragma unroll
        for (int i = 0; i < 3; ++i) hc[i] = hn[i];
#pragma unroll
        for (int i = 0; i < 3 * P; ++i) bc[i] = bn[i];
      }
      sched_fence();
    }
  }

  // Tile end: Re = P1 + P3, Im = P2 - P3 into the running totals.
  __device__ static __forceinline__ void fold(f32x16 (&acc)[3][P], f32x16 (&tre)[P],
                                              f32x16 (&tim)[P]) {
#pragma unroll
    for (int t = 0; t < P; ++t) {
      tre[t] += acc[0][t] + acc[2][t];
      tim[t] += acc[1][t] - acc[2][t];
      acc[0][t] = f32x16{}; acc[1][t] = f32x16{}; acc[2][t] = f32x16{};
    }
  }

  __device__ static void run(const FwdArgs& a) {
    // two staging buffers while the groups stream, then the waves' G blocks
    __shared__ float4 lds[LDS4];
    __shared__ float4 sh0[NH], sh1[NH];
    float4* sb0 = lds;
    float4* sb1 = lds + SB;
    const int tid = threadIdx.x, lane = tid & 63, wig = tid >> 6;
    const int64_t wave = (int64_t)blockIdx.x * NW + wig;
    const int64_t m = wave * 32 + (lane & 31);   // this lane's sample
    const bool valid = m < a.M;
    SampleK<TRIG> k;
    k.load(a, m, valid);

    // this launch row's groups
    const int32_t row = (int32_t)blockIdx.y;
    const int64_t lo64 = (int64_t)row * a.g_split;
    const int64_t lo = lo64 < a.gpad ? lo64 : a.gpad;
    const int64_t hi = lo64 + a.g_split < a.gpad ? lo64 + a.g_split : a.gpad;
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
    int32_t left = cpt;
    for (int32_t ch = 0; ch < nch; ch += 2) {
      if (ch + 1 < nch) stage(a, lo + (int64_t)(ch + 1) * C, wig, lane, sb1, sh1);
      chunk(reinterpret_cast<const float*>(sh0), reinterpret_cast<const float*>(sb0), lane, k, acc);
      if (--left == 0) {
        fold(acc, tre, tim);
        left = cpt;
      }
      publish();
      if (ch + 1 >= nch) break;
      if (ch + 2 < nch) stage(a, lo + (int64_t)(ch + 2) * C, wig, lane, sb0, sh0);
      chunk(reinterpret_cast<const float*>(sh1), reinterpret_cast<const float*>(sb1), lane, k, acc);
      if (--left == 0) {
        fold(acc, tre, tim);
        left = cpt;
      }
      publish();
    }
    fold(acc, tre, tim);

    // Finish.  Every wave has passed the last barrier, so the staging buffers
    // are free: each wave stores its 32 x 32 P complex block of G there ...
    float2* gl = reinterpret_cast<float2*>(lds + wig * GW);
    const int c = lane & 31;
#pragma unroll
    for (int t = 0; t < P; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = (v / 4) * 8 + (lane / 32) * 4 + (v % 4);
        gl[i * (32 * P) + 32 * t + c] = make_float2(tre[t][v], tim[t][v]);
      }
    __syncthreads();
    // ... and lane i < 32 contracts row i (its sample) with exp(-i 2 pi k . d_j)
    // over the offsets j, then multiplies by phi_m.
    if (lane >= 32 || !valid) return;
    const float2* gr = gl + lane * (32 * P);
    float dre[BC], dim[BC];
#pragma unroll
    for (int b = 0; b < BC; ++b) { dre[b] = 0.0f; dim[b] = 0.0f; }
    const bool any_voxel = a.N > 0;
    const float x0 = any_voxel ? a.x[0] : 0.0f, y0 = any_voxel ? a.y[0] : 0.0f, z0 = any_voxel ? a.z[0] : 0.0f;
    for (int j = 0; j < V && j < a.N; ++j) {
      float cj = 1.0f, sj = 0.0f;
      if (j > 0) k.sincos_phase(a.x[j] - x0, a.y[j] - y0, a.z[j] - z0, cj, sj);
#pragma unroll
      for (int b = 0; b < BC; ++b) {
        const float2 gv = gr[b * V + j];
        // (cj - i sj)(gre + i gim)
        dre[b] = __builtin_fmaf(cj, gv.x, __builtin_fmaf(sj, gv.y, dre[b]));
        dim[b] = __builtin_fmaf(cj, gv.y, __builtin_fmaf(-sj, gv.x, dim[b]));
      }
    }
    const float2 ph = a.phi[m];
    float2* dst = a.partial ? a.partial + (int64_t)row * BC * a.M : a.out;
#pragma unroll
    for (int b = 0; b < BC; ++b)
      dst[(int64_t)b * a.M + m] = make_float2(ph.x * dre[b] - ph.y * dim[b], ph.x * dim[b] + ph.y * dre[b]);
  }
};

// ---------------------------------------------------------------------------
// Four-group matrix-core gather (T = 8, groups of 128 voxels for one image):
// v_mfma_f32_16x16x4_f32 with K = a block of four groups.  A wave owns 16
// samples; lane l supplies sample l % 16 at group 4 q + l / 16, so each lane
// evaluates one phase with its sine and cosine per block and it serves
// 3 T = 24 MFMAs (768 matrix cycles), twice the pair engine's.  The packed
// groups stream through LDS in 16-group chunks (24 KB) shared by the 4 waves
// of a workgroup.  After the last group each wave writes its 16 x 128
// complex block of G to LDS, one half of the columns at a time, and all 64
// lanes contract it: four lanes per sample take every fourth offset, and
// their sums are combined in a fixed order.  FOLD: tiles shorter than the
// launch row fold into running totals; without it the launch row is one
// summation block and the kernel keeps no totals (fewer registers, 3 waves
// per SIMD on the HW path).
template <int T, int BC, int TRIG, bool FOLD>
struct FwdGather4 {
  static constexpr int V = 16 * T / BC;
  static constexpr int C = kMfma4Chunk;           // groups per chunk
  static constexpr int NW = kWorkgroup / 64;
  static constexpr int QF = 192 * T;              // image floats per block of four groups
  static constexpr int NS = 3 * T / 4;            // float4 slices per lane and block
  static constexpr int NB = C / 4 * QF * 4 / 1024;  // 1 KiB image blocks per chunk
  static constexpr int NH = C;                    // header float4s per chunk (one per group)
  static constexpr int SB = C / 4 * QF / 4;       // float4s of one staging buffer
  static constexpr int HC = 8 * T;                // G columns per half
  static constexpr int GH = 16 * HC * 2 / 4;       // float4s of one wave's half G block
  static constexpr int LDS4 = 2 * SB > NW * GH ? 2 * SB : NW * GH;
  static_assert(T % 4 == 0 && V >= 1 && V * BC == 16 * T, "group shape");
  static_assert(BC == 1 ? V == 2 * HC : HC % V == 0, "a half holds whole data vectors");
  static_assert(NB % NW == 0 && NH <= 64, "chunk staging");

  __device__ static __forceinline__ void stage(const FwdArgs& a, int64_t g, int wig, int lane,
                                               float4* lb, float4* lh) {
    const __amdgpu_buffer_rsrc_t rb =
        buffer_rsrc(reinterpret_cast<const float4*>(a.gwb) + (g / 4) * (QF / 4), NB * 64 * 16);
#pragma unroll
    for (int i = 0; i < NB / NW; ++i) {
      const int blk = i * NW + wig;   // wave-uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_ptr)(lb + blk * 64), 16, lane * 16, blk * 1024, 0, 0);
    }
    if (wig == 0 && lane < NH)
      lds_dma16(buffer_rsrc(reinterpret_cast<const float4*>(a.ghdr) + g, NH * 16), lane * 16, lh);
  }

  __device__ static __forceinline__ void publish() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Header of the lane's group and its B entries of block q of the chunk.
  __device__ static __forceinline__ void load_block(const float* __restrict__ hb,
                                                    const float* __restrict__ wb, int q, int lane,
                                                    float (&hs)[3], float (&bv)[3 * T]) {
    const float* hp = hb + (4 * q + (lane >> 4)) * 4;
#pragma unroll
    for (int i = 0; i < 3; ++i) hs[i] = hp[i];
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

  // Slices [sl] of block q for units t of one half: half h = slices h, 2 + h,
  // 4 + h (the three products' entries for t in [4h, 4h + 4)).
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
                                                     float (&hs)[3]) {
    const float* hp = hb + (4 * q + (lane >> 4)) * 4;
#pragma unroll
    for (int i = 0; i < 3; ++i) hs[i] = hp[i];
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

  // One chunk of 16 groups (4 blocks).  HW trig: one set of B entries; the
  // next block's first-half slices are read once this block's first-half
  // MFMAs have issued, its second half after the rest (each a half block of
  // MFMAs ahead of its use).  Accurate trig: pipelined by one whole block as
  // in the pair engine.
  __device__ static __forceinline__ void chunk(const float* __restrict__ hb, const float* __restrict__ wb,
                                               int lane, const SampleK<TRIG>& k, f32x4 (&acc)[3][T]) {
    constexpr int NQ = C / 4;
    if constexpr (TRIG == kTrigHw) {
      float hc[3], bv[3 * T], av[3];
      load_header(hb, 0, lane, hc);
      load_half(wb, 0, lane, 0, bv);
      load_half(wb, 0, lane, 1, bv);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        float hn[3];
        if (q + 1 < NQ) load_header(hb, q + 1, lane, hn);
        sched_fence();
        fwd_entries<TRIG>(k, hc, av);
        mfmas_half<0>(av, bv, acc);
        sched_fence();
        if (q + 1 < NQ) load_half(wb, q + 1, lane, 0, bv);
        sched_fence();
        mfmas_half<1>(av, bv, acc);
        sched_fence();
        if (q + 1 < NQ) {
          load_half(wb, q + 1, lane, 1, bv);
#pragma unroll
          for (int i = 0; i < 3; ++i) hc[i] = hn[i];
        }
        sched_fence();
      }
    } else {
      float hc[3], bc[3 * T], av[3];
      load_block(hb, wb, 0, lane, hc, bc);
      fwd_entries<TRIG>(k, hc, av);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        float hn[3], bn[3 * T];
        if (q + 1 < NQ) load_block(hb, wb, q + 1, lane, hn, bn);
        sched_fence();
        mfmas(av, bc, acc);
        sched_fence();
        if (q + 1 < NQ) {
          fwd_entries<TRIG>(k, hn, av);
#pragma unroll
          for (int i = 0; i < 3 * T; ++i) bc[i] = bn[i];
        }
        sched_fence();
      }
    }
  }

  // Tile end: Re = P1 + P3, Im = P2 - P3 into the running totals.
  template <int NT>
  __device__ static __forceinline__ void fold(f32x4 (&acc)[3][T], f32x4 (&tre)[NT], f32x4 (&tim)[NT]) {
    static_assert(NT == T, "fold needs the running totals");
#pragma unroll
    for (int t = 0; t < T; ++t) {
      tre[t] += acc[0][t] + acc[2][t];
      tim[t] += acc[1][t] - acc[2][t];
      acc[0][t] = f32x4{}; acc[1][t] = f32x4{}; acc[2][t] = f32x4{};
    }
  }

  __device__ static void run(const FwdArgs& a) {
    // two staging buffers while the groups stream, then the waves' G blocks
    __shared__ float4 lds[LDS4];
    __shared__ float4 sh0[NH], sh1[NH];
    float4* sb0 = lds;
    float4* sb1 = lds + SB;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wig = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t wave = (int64_t)blockIdx.x * NW + wig;
    const int64_t m = wave * 16 + (lane & 15);   // this lane's sample
    const bool valid = m < a.M;
    SampleK<TRIG> k;
    k.load(a, m, valid);

    // this launch row's groups
    const int32_t row = (int32_t)blockIdx.y;
    const int64_t lo64 = (int64_t)row * a.g_split;
    const int64_t lo = lo64 < a.gpad ? lo64 : a.gpad;
    const int64_t hi = lo64 + a.g_split < a.gpad ? lo64 + a.g_split : a.gpad;
    const int32_t nch = (int32_t)((hi - lo) / C);
    const int32_t cpt = (int32_t)(a.tile / C);
    if (nch > 0) stage(a, lo, wig, lane, sb0, sh0);
    publish();
    f32x4 acc[3][T], tre[FOLD ? T : 1], tim[FOLD ? T : 1];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      acc[0][t] = f32x4{}; acc[1][t] = f32x4{}; acc[2][t] = f32x4{};
    }
#pragma unroll
    for (int t = 0; t < (FOLD ? T : 1); ++t) { tre[t] = f32x4{}; tim[t] = f32x4{}; }
    int32_t left = cpt;
    auto tile_end = [&]() {
      if constexpr (FOLD) {
        if (--left == 0) {
          fold(acc, tre, tim);
          left = cpt;
        }
      }
    };
    int32_t ch = 0;
    for (; ch + 1 < nch; ch += 2) {
      stage(a, lo + (int64_t)(ch + 1) * C, wig, lane, sb1, sh1);
      chunk(reinterpret_cast<const float*>(sh0), reinterpret_cast<const float*>(sb0), lane, k, acc);
      tile_end();
      publish();
      if (ch + 2 < nch) stage(a, lo + (int64_t)(ch + 2) * C, wig, lane, sb0, sh0);
      chunk(reinterpret_cast<const float*>(sh1), reinterpret_cast<const float*>(sb1), lane, k, acc);
      tile_end();
      publish();
    }
    if (ch < nch) {
      chunk(reinterpret_cast<const float*>(sh0), reinterpret_cast<const float*>(sb0), lane, k, acc);
      tile_end();
      publish();
    }
    if constexpr (FOLD) fold(acc, tre, tim);
    (void)left;
    // the block's Re = P1 + P3, Im = P2 - P3 (the accumulators end here)
    f32x4 ore[T], oim[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      ore[t] = FOLD ? tre[FOLD ? t : 0] : acc[0][t] + acc[2][t];
      oim[t] = FOLD ? tim[FOLD ? t : 0] : acc[1][t] - acc[2][t];
    }

    fwd_finish<T, BC, TRIG>(a, lds, wig, lane, valid, m, row, k, ore, oim);
  }
};

// ---------------------------------------------------------------------------
// Mirror pairs (four-group engine).  With each group's reference at column
// jref (x_g = x[g V + jref], offsets d_j = x_j - x_jref) a group h whose
// reference is exactly -x_g holds at column j the voxel -x_g + d_j, so its
// phase is the conjugate of g's at every sample, and
//   e^{-i 2 pi k.x_g} rho_g[j] + e^{+i 2 pi k.x_g} rho_h[j]
//     = c u - i s w,  u = rho_g + rho_h, w = rho_g - rho_h,
// (c, s) = (cos, sin)(2 pi k.x_g): Re = c ur + s wi, Im = c ui - s wr, four
// real products for two groups where the three-product form takes six.  The
// K dimension of the product runs over the pair plan's entries (a group with
// its partner, or a group alone: w = u).
//
// Packing of the entries: one lane per (entry slot e, complex column cc);
// slots past the list (to the next multiple of the chunk) are zero.  Layout
// per block of four entries: value q (ur, ui, wi, wr) of tile t = cc / 16 at
// e' = q T + t, lane p = 16 (e % 4) + cc % 16: [e / 4][e' / 4][p][e' % 4]
// (256 T floats per block); the entry's header is its group's reference.
__global__ void __launch_bounds__(kWorkgroup) fwd_pair_pack_kernel(FwdArgs a, int BC) {
  constexpr int T = 8;
  const int64_t idx = (int64_t)blockIdx.x * kWorkgroup + threadIdx.x;
  const int64_t e = idx >> 7;
  const int cc = (int)(idx & 127);
  const int64_t E = a.pairs[0], Cp = a.pairs[1];
  const int64_t Epad = (E + kMfmaChunk - 1) / kMfmaChunk * kMfmaChunk;
  if (e >= Epad || e >= a.gpad) return;
  const int2* list = reinterpret_cast<const int2*>(a.pairs + kPairHeader);
  const int2 en = e < E ? list[e < Cp ? e : a.gcap - 1 - (e - Cp)] : make_int2(-1, -1);
  if (cc == 0) {
    const float4 r = en.x >= 0 ? a.refs[en.x] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    reinterpret_cast<float4*>(a.ghdr)[e] = make_float4(r.x, r.y, r.z, 0.0f);
  }
  const int V = 128 / BC;
  const int b = cc / V, j = cc % V;
  float2 rg = make_float2(0.0f, 0.0f), rh = make_float2(0.0f, 0.0f);
  if (en.x >= 0) {
    const int64_t n = (int64_t)en.x * V + j;
    if (n < a.N) rg = a.rho[(int64_t)b * a.N + n];
  }
  if (en.y >= 0) rh = a.rho[(int64_t)b * a.N + (int64_t)en.y * V + j];
  const float v[4] = {rg.x + rh.x, rg.y + rh.y, rg.y - rh.y, rg.x - rh.x};   // ur, ui, wi, wr
  const int t = cc / 16, lp = 16 * (int)(e & 3) + cc % 16;
  float* blk = a.gwb + (e >> 2) * (256 * T);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ep = q * T + t;
    blk[((ep >> 2) * 64 + lp) * 4 + (ep & 3)] = v[q];
  }
}

// The four-group engine over the pair plan's entries: FwdGather4's staging,
// pipelining and finish with four products per tile.  The launch rows split
// the padded entries evenly (chunks of 32), and each row is one summation
// block: the plan bounds a row's entries (blocked summation through the rows'
// partial sums), so the kernel keeps no running totals (with them, 128
// accumulators, 64 totals and 32 B entries spill past 256 VGPRs).
template <int BC, int TRIG>
struct FwdPairGather4 {
  static constexpr int T = 8;
  static constexpr int V = 16 * T / BC;
  static constexpr int C = kMfma4Chunk;             // entries per chunk
  static constexpr int NW = kWorkgroup / 64;
  static constexpr int QF = 256 * T;                // image floats per block of four entries
  static constexpr int NB = C / 4 * QF * 4 / 1024;  // 1 KiB image blocks per chunk
  static constexpr int NH = C;
  static constexpr int SB = C / 4 * QF / 4;
  static constexpr int HC = 8 * T;
  static constexpr int GH = 16 * HC * 2 / 4;
  static constexpr int LDS4 = 2 * SB > NW * GH ? 2 * SB : NW * GH;
  static_assert(NB % NW == 0 && NH <= 64, "chunk staging");

  __device__ static __forceinline__ void stage(const FwdArgs& a, int64_t g, int wig, int lane, float4* lb,
                                               float4* lh) {
    const __amdgpu_buffer_rsrc_t rb =
        buffer_rsrc(reinterpret_cast<const float4*>(a.gwb) + (g / 4) * (QF / 4), NB * 64 * 16);
#pragma unroll
    for (int i = 0; i < NB / NW; ++i) {
      const int blk = i * NW + wig;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_ptr)(lb + blk * 64), 16, lane * 16, blk * 1024, 0, 0);
    }
    if (wig == 0 && lane < NH)
      lds_dma16(buffer_rsrc(reinterpret_cast<const float4*>(a.ghdr) + g, NH * 16), lane * 16, lh);
  }

  __device__ static __forceinline__ void publish() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  __device__ static __forceinline__ void load_header(const float* __restrict__ hb, int q, int lane, float (&hs)[3]) {
    const float* hp = hb + (4 * q + (lane >> 4)) * 4;
#pragma unroll
    for (int i = 0; i < 3; ++i) hs[i] = hp[i];
  }

  // slices 2 q + h of block qb (values q = ur, ui, wi, wr of tiles 4h .. 4h + 3): bv[q T + t]
  __device__ static __forceinline__ void load_half(const float* __restrict__ wb, int qb, int lane, int h,
                                                   float (&bv)[4 * T]) {
    const float* pp = wb + qb * QF;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int sl = 2 * q + h;
      const float4 v = *reinterpret_cast<const float4*>(pp + (sl * 64 + lane) * 4);
      bv[4 * sl] = v.x; bv[4 * sl + 1] = v.y; bv[4 * sl + 2] = v.z; bv[4 * sl + 3] = v.w;
    }
  }

  template <int H>
  __device__ static __forceinline__ void mfmas_half(float c, float s, const float (&bv)[4 * T], f32x4 (&acc)[4][T]) {
#pragma unroll
    for (int u = 0; u < T / 2; ++u) {
      const int t = H * (T / 2) + u;
      acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(c, bv[t], acc[0][t], 0, 0, 0);           // c ur
      acc[1][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(c, bv[T + t], acc[1][t], 0, 0, 0);       // c ui
      acc[2][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(s, bv[2 * T + t], acc[2][t], 0, 0, 0);   // s wi
      acc[3][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(s, bv[3 * T + t], acc[3][t], 0, 0, 0);   // s wr
    }
  }

  // One chunk of 16 entries (4 blocks): B slices half a block ahead, the
  // phase right before its MFMAs (the HW-path pipeline of FwdGather4).
  __device__ static __forceinline__ void chunk(const float* __restrict__ hb, const float* __restrict__ wb, int lane,
                                               const SampleK<TRIG>& k, f32x4 (&acc)[4][T]) {
    constexpr int NQ = C / 4;
    float hc[3], bv[4 * T];
    load_header(hb, 0, lane, hc);
    load_half(wb, 0, lane, 0, bv);
    load_half(wb, 0, lane, 1, bv);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float hn[3];
      if (q + 1 < NQ) load_header(hb, q + 1, lane, hn);
      sched_fence();
      float c, s;
      k.sincos_phase(hc[0], hc[1], hc[2], c, s);
      mfmas_half<0>(c, s, bv, acc);
      sched_fence();
      if (q + 1 < NQ) load_half(wb, q + 1, lane, 0, bv);
      sched_fence();
      mfmas_half<1>(c, s, bv, acc);
      sched_fence();
      if (q + 1 < NQ) {
        load_half(wb, q + 1, lane, 1, bv);
#pragma unroll
        for (int i = 0; i < 3; ++i) hc[i] = hn[i];
      }
      sched_fence();
    }
  }

  __device__ static void run(const FwdArgs& a) {
    __shared__ float4 lds[LDS4];
    __shared__ float4 sh0[NH], sh1[NH];
    float4* sb0 = lds;
    float4* sb1 = lds + SB;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wig = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t wave = (int64_t)blockIdx.x * NW + wig;
    const int64_t m = wave * 16 + (lane & 15);
    const bool valid = m < a.M;
    SampleK<TRIG> k;
    k.load(a, m, valid);
    // this launch row's entries: the padded list split evenly over the rows
    const int64_t E = a.pairs[0];
    const int64_t Epad = (E + kMfmaChunk - 1) / kMfmaChunk * kMfmaChunk;
    const int32_t rows = (int32_t)gridDim.y, row = (int32_t)blockIdx.y;
    int64_t gs = (Epad + rows - 1) / rows;
    gs = (gs + kMfmaChunk - 1) / kMfmaChunk * kMfmaChunk;
    const int64_t lo64 = (int64_t)row * gs;
    const int64_t lo = lo64 < Epad ? lo64 : Epad;
    const int64_t hi = lo64 + gs < Epad ? lo64 + gs : Epad;
    const int32_t nch = (int32_t)((hi - lo) / C);
    if (nch > 0) stage(a, lo, wig, lane, sb0, sh0);
    publish();
    f32x4 acc[4][T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      acc[0][t] = f32x4{}; acc[1][t] = f32x4{}; acc[2][t] = f32x4{}; acc[3][t] = f32x4{};
    }
    int32_t ch = 0;
    for (; ch + 1 < nch; ch += 2) {
      stage(a, lo + (int64_t)(ch + 1) * C, wig, lane, sb1, sh1);
      chunk(reinterpret_cast<const float*>(sh0), reinterpret_cast<const float*>(sb0), lane, k, acc);
      publish();
      if (ch + 2 < nch) stage(a, lo + (int64_t)(ch + 2) * C, wig, lane, sb0, sh0);
      chunk(reinterpret_cast<const float*>(sh1), reinterpret_cast<const float*>(sb1), lane, k, acc);
      publish();
    }
    if (ch < nch) {
      chunk(reinterpret_cast<const float*>(sh0), reinterpret_cast<const float*>(sb0), lane, k, acc);
      publish();
    }
    // G = sum over entries of (c ur + s wi) + i (c ui - s wr)
    f32x4 ore[T], oim[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      ore[t] = acc[0][t] + acc[2][t];
      oim[t] = acc[1][t] - acc[3][t];
    }
    fwd_finish<T, BC, TRIG>(a, lds, wig, lane, valid, m, row, k, ore, oim);
  }
};

// ---------------------------------------------------------------------------
// Direct evaluation of the listed groups: one lane per sample, the groups in
// increasing order (indices and voxels read as wave-uniform scalars); the sum
// is blocked by `tile` listed groups and added into the (already reduced)
// output.
template <int T, int BC, int TRIG>
__global__ void __launch_bounds__(kWorkgroup) fwd_direct_kernel(FwdArgs a) {
  constexpr int V = 16 * T / BC;
  const int32_t count = a.glist[0];
  if (count == 0) return;
  const int64_t m = (int64_t)blockIdx.x * kWorkgroup + threadIdx.x;
  const bool valid = m < a.M;
  SampleK<TRIG> k;
  k.load(a, m, valid);
  float tre[BC], tim[BC], are[BC], aim[BC];
#pragma unroll
  for (int b = 0; b < BC; ++b) { tre[b] = 0.0f; tim[b] = 0.0f; are[b] = 0.0f; aim[b] = 0.0f; }
  int64_t left = a.tile;
  for (int32_t i = 0; i < count; ++i) {
    const int64_t g = a.glist[1 + i];
    for (int j = 0; j < V; ++j) {
      const int64_t n = g * V + j;
      if (n >= a.N) break;
      float c, s;
      k.sincos_phase(a.x[n], a.y[n], a.z[n], c, s);
#pragma unroll
      for (int b = 0; b < BC; ++b) {
        const float2 r = a.rho[(int64_t)b * a.N + n];
        // (rr + i ri)(c - i s)
        are[b] = __builtin_fmaf(r.x, c, __builtin_fmaf(r.y, s, are[b]));
        aim[b] = __builtin_fmaf(r.y, c, __builtin_fmaf(-r.x, s, aim[b]));
      }
    }
    if (--left == 0) {
#pragma unroll
      for (int b = 0; b < BC; ++b) { tre[b] += are[b]; tim[b] += aim[b]; are[b] = 0.0f; aim[b] = 0.0f; }
      left = a.tile;
    }
  }
  if (!valid) return;
  const float2 ph = a.phi[m];
#pragma unroll
  for (int b = 0; b < BC; ++b) {
    const float re = tre[b] + are[b], im = tim[b] + aim[b];
    float2* o = a.out + (int64_t)b * a.M + m;
    const float2 prev = *o;
    *o = make_float2(prev.x + (ph.x * re - ph.y * im), prev.y + (ph.x * im + ph.y * re));
  }
}

template <int T, int BC, int TRIG>
__global__ void __launch_bounds__(kWorkgroup) __attribute__((amdgpu_waves_per_eu(T == 2 ? 4 : 2)))
fwd_gather_kernel(FwdArgs a) {
  FwdGather<T, BC, TRIG>::run(a);
}

template <int BC, int TRIG, bool FOLD>
constexpr int fwd4_waves_per_simd() { return (!FOLD && TRIG == kTrigHw) ? 3 : 2; }

template <int T, int BC, int TRIG, bool FOLD>
__global__ void __launch_bounds__(kWorkgroup)
__attribute__((amdgpu_waves_per_eu(fwd4_waves_per_simd<BC, TRIG, FOLD>())))
fwd4_gather_kernel(FwdArgs a) {
  FwdGather4<T, BC, TRIG, FOLD>::run(a);
}

using FwdFn = void (*)(FwdArgs);

// Mirror-pair forward gather: 128 accumulators, 2 waves per SIMD.
template <int BC, int TRIG>
__global__ void __launch_bounds__(kWorkgroup) __attribute__((amdgpu_waves_per_eu(2)))
fwd4_pair_gather_kernel(FwdArgs a) {
  FwdPairGather4<BC, TRIG>::run(a);
}

template <int BC>
void pick_pair(int trig, FwdFn& f) {
  f = trig == kTrigHw ? fwd4_pair_gather_kernel<BC, kTrigHw> : fwd4_pair_gather_kernel<BC, kTrigAccurate>;
}

bool select_pair_fwd(int trig, int BC, FwdFn& f) {
  switch (BC) {
    case 1: pick_pair<1>(trig, f); return true;
    case 2: pick_pair<2>(trig, f); return true;
    case 4: pick_pair<4>(trig, f); return true;
    case 8: pick_pair<8>(trig, f); return true;
    case 16: pick_pair<16>(trig, f); return true;
    default: return false;
  }
}

// gather: the kernel for tiles shorter than a launch row; gather_row (four-
// group engine only) the one for a tile that spans the row.
struct FwdKernels { FwdFn gather; FwdFn direct; FwdFn gather_row; };

template <int T, int BC, int TRIG>
FwdKernels pick() {
  if constexpr (T == 8)
    return {fwd4_gather_kernel<T, BC, TRIG, true>, fwd_direct_kernel<T, BC, TRIG>,
            fwd4_gather_kernel<T, BC, TRIG, false>};
  else
    return {fwd_gather_kernel<T, BC, TRIG>, fwd_direct_kernel<T, BC, TRIG>, nullptr};
}

template <int T>
bool select_bc(int trig, int BC, FwdKernels& fn) {
  const bool hw = trig == kTrigHw;
  switch (BC) {
    case 1: fn = hw ? pick<T, 1, kTrigHw>() : pick<T, 1, kTrigAccurate>(); return true;
    case 2: fn = hw ? pick<T, 2, kTrigHw>() : pick<T, 2, kTrigAccurate>(); return true;
    case 4: fn = hw ? pick<T, 4, kTrigHw>() : pick<T, 4, kTrigAccurate>(); return true;
    case 8: fn = hw ? pick<T, 8, kTrigHw>() : pick<T, 8, kTrigAccurate>(); return true;
    case 16: fn = hw ? pick<T, 16, kTrigHw>() : pick<T, 16, kTrigAccurate>(); return true;
    default: return false;
  }
}

bool select_fwd(int trig, int T, int BC, FwdKernels& fn) {
  if (T == 2) return select_bc<2>(trig, BC, fn);
  if (T == 4) return select_bc<4>(trig, BC, fn);
  if (T == 8) return select_bc<8>(trig, BC, fn);
  return false;
}

}  // namespace

hipError_t launch_fwd_pack(int T, int BC, const FwdArgs& a, hipStream_t s) {
  FwdKernels fn;
  if (!select_fwd(kTrigHw, T, BC, fn) || a.gpad % kMfmaChunk != 0) return hipErrorInvalidValue;
  if (a.gpad <= 0) return hipSuccess;
  if (!a.glist) return hipErrorInvalidValue;
  const int64_t lanes = a.gpad * 16 * T;
  const int64_t blocks = (lanes + kWorkgroup - 1) / kWorkgroup;
  hipLaunchKernelGGL(fwd_pack_kernel, dim3((unsigned)blocks), dim3(kWorkgroup), 0, s, a, T, BC);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fwd_list_kernel, dim3(1), dim3(kWorkgroup), 0, s, a, 16 * T / BC);
  return hipGetLastError();
}

hipError_t launch_fwd_gather(int trig, int T, int BC, int32_t splits, const FwdArgs& a,
                             hipStream_t s) {
  FwdKernels fn;
  if (!select_fwd(trig, T, BC, fn) || splits < 1 || (splits > 1) != (a.partial != nullptr))
    return hipErrorInvalidValue;
  if (a.gpad % kMfmaChunk != 0 || a.g_split % kMfmaChunk != 0 || a.tile % kMfmaChunk != 0 ||
      a.tile <= 0)
    return hipErrorInvalidValue;
  if (a.M <= 0) return hipSuccess;
  // a wave owns 32 samples (pair engine) or 16 (four-group engine, T = 8)
  const int64_t per_wave = T == 8 ? 16 : 32;
  const int64_t waves = (a.M + per_wave - 1) / per_wave;
  const int64_t blocks = (waves + kWorkgroup / 64 - 1) / (kWorkgroup / 64);
  const FwdFn g = (fn.gather_row && a.tile >= a.g_split) ? fn.gather_row : fn.gather;
  hipLaunchKernelGGL(g, dim3((unsigned)blocks, (unsigned)splits), dim3(kWorkgroup), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd_pair_pack(int BC, const FwdArgs& a, hipStream_t s) {
  FwdFn f;
  if (!select_pair_fwd(kTrigHw, BC, f) || a.gpad % kMfmaChunk != 0 || !a.pairs || !a.refs || !a.wflags ||
      a.gcap != (a.N + 128 / BC - 1) / (128 / BC) || a.gpad < a.gcap)
    return hipErrorInvalidValue;
  if (a.gpad <= 0) return hipSuccess;
  if (!a.glist) return hipErrorInvalidValue;
  const int64_t lanes = a.gpad * 128;
  const int64_t blocks = (lanes + kWorkgroup - 1) / kWorkgroup;
  hipLaunchKernelGGL(fwd_pair_pack_kernel, dim3((unsigned)blocks), dim3(kWorkgroup), 0, s, a, BC);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fwd_list_kernel, dim3(1), dim3(kWorkgroup), 0, s, a, 128 / BC);
  return hipGetLastError();
}

hipError_t launch_fwd_pair_gather(int trig, int BC, int32_t splits, const FwdArgs& a, hipStream_t s) {
  FwdFn f;
  if (!select_pair_fwd(trig, BC, f) || splits < 1 || (splits > 1) != (a.partial != nullptr) || !a.pairs)
    return hipErrorInvalidValue;
  if (a.gpad % kMfmaChunk != 0) return hipErrorInvalidValue;
  if (a.M <= 0) return hipSuccess;
  const int64_t waves = (a.M + 15) / 16;
  const int64_t blocks = (waves + kWorkgroup / 64 - 1) / (kWorkgroup / 64);
  hipLaunchKernelGGL(f, dim3((unsigned)blocks, (unsigned)splits), dim3(kWorkgroup), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd_direct(int trig, int T, int BC, const FwdArgs& a, hipStream_t s) {
  FwdKernels fn;
  if (!select_fwd(trig, T, BC, fn) || a.tile <= 0) return hipErrorInvalidValue;
  if (a.M <= 0 || a.N <= 0 || a.gpad <= 0) return hipSuccess;
  if (!a.glist) return hipErrorInvalidValue;
  const int64_t blocks = (a.M + kWorkgroup - 1) / kWorkgroup;
  hipLaunchKernelGGL(fn.direct, dim3((unsigned)blocks), dim3(kWorkgroup), 0, s, a);
  return hipGetLastError();
}

}  // namespace ncmri
