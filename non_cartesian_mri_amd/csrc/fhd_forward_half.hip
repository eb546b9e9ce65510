// gfx950 half-split forward operator (PMPP ch. 17 "Iterative MRI
// reconstruction", section 17.2's F; section 17.3 step 3 synthesises scan
// data from an image):
//
//   D[b][m] = phi_m sum_j exp(-i 2 pi k_m . d_j) G[m][j][b],
//   G[m][j][b] = sum_g exp(-i 2 pi k_m . x_g) rho_b[x_g + d_j],
//
// as in the four-group engine (groups of 128 / BC voxels at common offsets,
// 16 samples per wave, the three real products P1 = sum (c - s) rr,
// P2 = sum (c + s) ri, P3 = sum s (rr + ri), Re = P1 + P3, Im = P2 - P3), with
// every fp32 product of the sum over groups formed from fp16 parts on
// v_mfma_f32_16x16x32_f16 (K = 32 groups per MFMA): x = hi + lo, x y ~ hi hi +
// hi lo + lo hi with fp32 accumulation, ~2^-22 relative error per product.
// The image entries (rr, ri, rr + ri) are scaled by a power of two that puts
// the largest near 2^14, split into parts once per pass, and the scale is
// undone on G; the contraction of G with exp(-i 2 pi k . d_j) and phi runs in
// fp32 as in the four-group engine.  Groups off the common offsets are packed
// as zeros and added afterwards by the four-group engine's direct kernel.
#include "fhd_forward_common.h"
#include "fhd_forward_half.h"
#include "fhd_half_common.h"

namespace ncmri {
namespace {

constexpr int kScaleBlocks = 256;

// Per-block maxima of |entry| over the packed image's n floats.
__global__ void __launch_bounds__(256) fwd_half_scale_partial_kernel(const float* __restrict__ gwb, int64_t n,
                                                                     float* __restrict__ scale) {
  __shared__ float sh[256];
  float mx = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)kScaleBlocks * 256) {
    const float v = __builtin_fabsf(gwb[i]);
    mx = v > mx ? v : mx;
  }
  sh[threadIdx.x] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] = sh[threadIdx.x] > sh[threadIdx.x + s] ? sh[threadIdx.x] : sh[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) scale[2 + blockIdx.x] = sh[0];
}

// scale[0] = 2^e with the largest entry times 2^e in [2^13, 2^14) (far below
// fp16's 65504), scale[1] = 2^-e; 1 for an all-zero image.
__global__ void __launch_bounds__(256) fwd_half_scale_kernel(float* __restrict__ scale) {
  __shared__ float sh[256];
  sh[threadIdx.x] = scale[2 + threadIdx.x];
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] = sh[threadIdx.x] > sh[threadIdx.x + s] ? sh[threadIdx.x] : sh[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float top = sh[0];
    int e = 0;
    if (top > 0.0f && isfinite(top)) {
      e = 14 - ilogbf(top) - 1;
      e = e < -120 ? -120 : (e > 120 ? 120 : e);
    }
    scale[0] = ldexpf(1.0f, e);
    scale[1] = ldexpf(1.0f, -e);
  }
}

// Slot v = 8 j + e (octet j < 4, element e < 8) of a 32-group chunk holds
// group (j mod s) + s e + 8 s (j div s) of the chunk, s = 1, 2 or 4: s = 1 the
// identity; on a grid whose x rows hold s groups, s makes every octet a run
// of equally spaced groups (one from each of 8 consecutive rows).
__device__ __forceinline__ int chunk_slot_group(int v, int s) {
  const int j = v >> 3, e = v & 7;
  return (j % s) + s * e + 8 * s * (j / s);
}

// Order: one thread per chunk picks the s under which most of its octets are
// equally spaced (the smallest s on ties) and writes the gather's headers in
// slot order: x, y, z of the slot's group; w of the octet's element 0: 1 when
// its bases are equally spaced (exact float comparisons), elements 1-3: the
// spacing, element 4 of octet 0: s.
__global__ void __launch_bounds__(kWorkgroup) fwd_half_order_kernel(FwdHalfArgs h) {
  const int64_t q = (int64_t)blockIdx.x * kWorkgroup + threadIdx.x;
  if (q * 32 >= h.f.gpad) return;
  const float4* gh = reinterpret_cast<const float4*>(h.f.ghdr) + q * 32;
  int best = 1, best_n = -1;
  for (int s = 1; s <= 4; s *= 2) {
    int n = 0;
    for (int j = 0; j < 4; ++j) {
      const float4 a = gh[chunk_slot_group(8 * j, s)], b = gh[chunk_slot_group(8 * j + 1, s)];
      const float dx = b.x - a.x, dy = b.y - a.y, dz = b.z - a.z;
      bool even = true;
      for (int e = 2; e < 8; ++e) {
        const float4 c = gh[chunk_slot_group(8 * j + e, s)];
        even = even && c.x - a.x == (float)e * dx && c.y - a.y == (float)e * dy && c.z - a.z == (float)e * dz;
      }
      n += even ? 1 : 0;
    }
    if (n > best_n) { best = s; best_n = n; }
  }
  float4* out = h.hh + q * 32;
  for (int j = 0; j < 4; ++j) {
    const float4 a = gh[chunk_slot_group(8 * j, best)], b = gh[chunk_slot_group(8 * j + 1, best)];
    const float dx = b.x - a.x, dy = b.y - a.y, dz = b.z - a.z;
    bool even = true;
    for (int e = 2; e < 8; ++e) {
      const float4 c = gh[chunk_slot_group(8 * j + e, best)];
      even = even && c.x - a.x == (float)e * dx && c.y - a.y == (float)e * dy && c.z - a.z == (float)e * dz;
    }
    const float wv[5] = {even ? 1.0f : 0.0f, dx, dy, dz, j == 0 ? (float)best : 0.0f};
    for (int e = 0; e < 8; ++e) {
      const float4 c = gh[chunk_slot_group(8 * j + e, best)];
      out[8 * j + e] = make_float4(c.x, c.y, c.z, e < 5 ? wv[e] : 0.0f);
    }
  }
}

// Parts: one lane per (octet of slots o, complex column cc < 128).  Entry u
// (rr, ri, rr + ri) of group g and column cc sits in the four-group engine's
// packed image at block g / 4, float4 slice (8 u + t) / 4 (t = cc / 16) of
// lane 16 (g % 4) + cc % 16; the lane scales and splits the entries of the
// groups in slots 8 o .. 8 o + 7 (the order kernel's s of chunk o / 4) and
// stores them as the B parts of lane cc % 16 + 16 (o % 4) of tile t in that
// chunk: B[k][j] = element k % 8 of lane j + 16 (k / 8), k the slot within the
// chunk, j the column within the tile.
__global__ void __launch_bounds__(kWorkgroup) fwd_half_pack_kernel(FwdHalfArgs h) {
  const FwdArgs& a = h.f;
  const int64_t idx = (int64_t)blockIdx.x * kWorkgroup + threadIdx.x;
  const int64_t o = idx >> 7;
  const int cc = (int)(idx & 127);
  if (o * 8 >= a.gpad) return;
  const float sc = h.scale[0];
  const int t = cc >> 4;
  const int64_t q = o >> 2;
  const int so = (int)h.hh[q * 32 + 4].w;
  half8 part[3][2];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t g = q * 32 + chunk_slot_group(8 * (int)(o & 3) + e, so);
    const float* blk = a.gwb + (g >> 2) * 1536;
    const int lp = 16 * (int)(g & 3) + (cc & 15);
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int en = 8 * u + t;
      const float v = blk[((en >> 2) * 64 + lp) * 4 + (en & 3)] * sc;   // exact: a power of two
      _Float16 hi, lo;
      split_half(v, hi, lo);
      part[u][0][e] = hi;
      part[u][1][e] = lo;
    }
  }
  const int lane = (cc & 15) + 16 * (int)(o & 3);
  uint4* w = reinterpret_cast<uint4*>(h.wh);
#pragma unroll
  for (int u = 0; u < 3; ++u)
#pragma unroll
    for (int s = 0; s < 2; ++s)
      w[(((q * 8 + t) * 3 + u) * 2 + s) * 64 + lane] = *reinterpret_cast<const uint4*>(&part[u][s]);
}

// Gather: a wave owns 16 samples (lane l: sample l % 16); per 32-group chunk
// lane l forms the phases of its sample at the groups of slots 8 (l / 16) ..
// + 7 (each evaluated, or stepped by rotations where the octet's bases are
// equally spaced, as on a grid), splits (c - s, c + s, s) into A parts, and
// for each tile of 16 columns reads the six B parts from LDS and issues 9
// MFMAs.  Chunks are staged into LDS by LDS DMA, double buffered, shared by
// the 8 waves of the workgroup; the headers are stored transposed in LDS
// (slot 8 (j % 4) + j / 4 at LDS slot j) so that the four lane groups, which
// read slots 8 g + e at once, hit consecutive LDS slots.  FOLD: tiles of
// a.tile groups fold into running totals; without it the launch row is one
// summation block.
template <int BC, int TRIG, bool FOLD>
struct FwdHalfGather {
  static constexpr int T = 8;
  static constexpr int C = 32;                 // groups per chunk: one MFMA K block
  static constexpr int NW = kFwdHalfWaves;
  static constexpr int BQ = T * 6 * 64;        // 16-byte B parts per chunk (48 KB)
  static constexpr int GH = 16 * (8 * T) * 2 / 4;   // float4s of one wave's half G block (fwd_finish)
  static_assert(BQ % (64 * NW) == 0, "chunk staging");
  static_assert(NW * GH <= 2 * BQ, "the G blocks fit in the staging buffers");

  __device__ static __forceinline__ void stage(const FwdHalfArgs& h, int64_t g0, int wig, int lane, uint4* lb,
                                               float4* lh) {
    const __amdgpu_buffer_rsrc_t rb =
        buffer_rsrc(reinterpret_cast<const uint4*>(h.wh) + (g0 / C) * BQ, BQ * 16);
#pragma unroll
    for (int i = 0; i < BQ / 64 / NW; ++i) {
      const int blk = i * NW + wig;   // wave-uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_ptr)(lb + blk * 64), 16, lane * 16, blk * 1024, 0, 0);
    }
    if (wig == 0 && lane < C) {
      const int m = 8 * (lane % 4) + lane / 4;
      lds_dma16(buffer_rsrc(h.hh + g0, C * 16), m * 16, lh);
    }
  }

  __device__ static __forceinline__ void publish() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  __device__ static __forceinline__ void chunk(const float4* __restrict__ hb, const uint4* __restrict__ lb, int lane,
                                               const SampleK<TRIG>& k, f32x4 (&acc)[3][T]) {
    // A entries (c - s, c + s, s) of groups 8 (lane / 16) + e, e < 8, of the
    // chunk (slot 4 e + lane / 16).  Equally spaced bases: the first group's
    // phase and the spacing's (each as the trig path evaluates a phase), then
    // seven rotations by the spacing's (2 sines and cosines per octet instead
    // of 8 of each; each rotation adds about one rounding to c and s, and
    // after seven they stay within ~5e-7 of the exact values, against ~1e-7
    // for one accurate evaluation); otherwise per group.
    const int oc = lane >> 4;
    float ent[8][3];
    const float4 h0 = hb[oc];
    if (h0.w != 0.0f) {
      float c, s, cd, sd;
      k.sincos_phase(h0.x, h0.y, h0.z, c, s);
      k.sincos_phase(hb[4 + oc].w, hb[8 + oc].w, hb[12 + oc].w, cd, sd);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ent[e][0] = c - s;
        ent[e][1] = c + s;
        ent[e][2] = s;
        if (e < 7) {
          const float cn = __builtin_fmaf(c, cd, -(s * sd));
          s = __builtin_fmaf(s, cd, c * sd);
          c = cn;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4 he = hb[4 * e + oc];
        const float hs[3] = {he.x, he.y, he.z};
        fwd_entries<TRIG>(k, hs, ent[e]);
      }
    }
    half8 ah[3], al[3];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        uint32_t hi, lo;
        split_pair(ent[2 * p][u], ent[2 * p + 1][u], hi, lo);
        const half2v hh = __builtin_bit_cast(half2v, hi), ll = __builtin_bit_cast(half2v, lo);
        ah[u][2 * p] = hh[0];
        ah[u][2 * p + 1] = hh[1];
        al[u][2 * p] = ll[0];
        al[u][2 * p + 1] = ll[1];
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
#pragma unroll
      for (int u = 0; u < 3; ++u) acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[u], bh[u], acc[u][t], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 3; ++u) acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[u], bl[u], acc[u][t], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 3; ++u) acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[u], bh[u], acc[u][t], 0, 0, 0);
    }
  }

  __device__ static void run(const FwdHalfArgs& h) {
    const FwdArgs& a = h.f;
    __shared__ uint4 lds[2 * BQ];
    __shared__ float4 sh0[C], sh1[C];
    uint4* sb0 = lds;
    uint4* sb1 = lds + BQ;
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
    if (nch > 0) stage(h, lo, wig, lane, sb0, sh0);
    publish();
    f32x4 acc[3][T], tre[FOLD ? T : 1], tim[FOLD ? T : 1];
#pragma unroll
    for (int t = 0; t < T; ++t) { acc[0][t] = f32x4{}; acc[1][t] = f32x4{}; acc[2][t] = f32x4{}; }
#pragma unroll
    for (int t = 0; t < (FOLD ? T : 1); ++t) { tre[t] = f32x4{}; tim[t] = f32x4{}; }
    int32_t left = cpt;
    auto tile_end = [&]() {
      if constexpr (FOLD) {
        if (--left == 0) {
#pragma unroll
          for (int t = 0; t < T; ++t) {
            tre[t] += acc[0][t] + acc[2][t];
            tim[t] += acc[1][t] - acc[2][t];
            acc[0][t] = f32x4{}; acc[1][t] = f32x4{}; acc[2][t] = f32x4{};
          }
          left = cpt;
        }
      }
    };
    int32_t ch = 0;
    for (; ch + 1 < nch; ch += 2) {
      stage(h, lo + (int64_t)(ch + 1) * C, wig, lane, sb1, sh1);
      chunk(sh0, sb0, lane, k, acc);
      tile_end();
      publish();
      if (ch + 2 < nch) stage(h, lo + (int64_t)(ch + 2) * C, wig, lane, sb0, sh0);
      chunk(sh1, sb1, lane, k, acc);
      tile_end();
      publish();
    }
    if (ch < nch) {
      chunk(sh0, sb0, lane, k, acc);
      tile_end();
      publish();
    }
    (void)left;
    // the block's Re = P1 + P3, Im = P2 - P3, the image's scale undone
    const float inv = h.scale[1];
    f32x4 ore[T], oim[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if constexpr (FOLD) {
        ore[t] = (tre[t] + acc[0][t] + acc[2][t]) * inv;
        oim[t] = (tim[t] + acc[1][t] - acc[2][t]) * inv;
      } else {
        ore[t] = (acc[0][t] + acc[2][t]) * inv;
        oim[t] = (acc[1][t] - acc[2][t]) * inv;
      }
    }
    fwd_finish<T, BC, TRIG>(a, reinterpret_cast<float4*>(lds), wig, lane, valid, m, row, k, ore, oim);
  }
};

template <int BC, int TRIG, bool FOLD>
__global__ void __launch_bounds__(64 * kFwdHalfWaves) __attribute__((amdgpu_waves_per_eu(2)))
fwd_half_gather_kernel(FwdHalfArgs h) {
  FwdHalfGather<BC, TRIG, FOLD>::run(h);
}

using FwdHalfFn = void (*)(FwdHalfArgs);

struct FwdHalfPair {
  FwdHalfFn gather;       // tiles folded into running totals
  FwdHalfFn gather_row;   // the launch row is one summation block
};

template <int BC>
FwdHalfPair pick_fwd_half(int trig) {
  if (trig == kTrigHw) return {fwd_half_gather_kernel<BC, kTrigHw, true>, fwd_half_gather_kernel<BC, kTrigHw, false>};
  return {fwd_half_gather_kernel<BC, kTrigAccurate, true>, fwd_half_gather_kernel<BC, kTrigAccurate, false>};
}

FwdHalfPair select_fwd_half(int trig, int BC) {
  switch (BC) {
    case 1: return pick_fwd_half<1>(trig);
    case 2: return pick_fwd_half<2>(trig);
    case 4: return pick_fwd_half<4>(trig);
    case 8: return pick_fwd_half<8>(trig);
    case 16: return pick_fwd_half<16>(trig);
    default: return {nullptr, nullptr};
  }
}

}  // namespace

bool fwd_half_supported(int BC) { return select_fwd_half(kTrigHw, BC).gather != nullptr; }

hipError_t launch_fwd_half_pack(int BC, const FwdHalfArgs& h, hipStream_t s) {
  if (!fwd_half_supported(BC) || h.f.gpad % 32 != 0 || !h.scale) return hipErrorInvalidValue;
  if (h.f.gpad > 0 && (!h.wh || !h.hh)) return hipErrorInvalidValue;
  // the scale first, also for an empty pass (then 1)
  const int64_t n = h.f.gpad * 384;   // floats of the packed image (T = 8)
  hipLaunchKernelGGL(fwd_half_scale_partial_kernel, dim3(kScaleBlocks), dim3(256), 0, s, h.f.gwb, n, h.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fwd_half_scale_kernel, dim3(1), dim3(256), 0, s, h.scale);
  e = hipGetLastError();
  if (e != hipSuccess || h.f.gpad <= 0) return e;
  const int64_t chunks = h.f.gpad / 32;
  hipLaunchKernelGGL(fwd_half_order_kernel, dim3((unsigned)((chunks + kWorkgroup - 1) / kWorkgroup)), dim3(kWorkgroup),
                     0, s, h);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t lanes = h.f.gpad / 8 * 128;
  hipLaunchKernelGGL(fwd_half_pack_kernel, dim3((unsigned)((lanes + kWorkgroup - 1) / kWorkgroup)), dim3(kWorkgroup), 0,
                     s, h);
  return hipGetLastError();
}

hipError_t launch_fwd_half_gather(int trig, int BC, int32_t splits, const FwdHalfArgs& h, hipStream_t s) {
  const FwdArgs& a = h.f;
  FwdHalfPair fn = select_fwd_half(trig, BC);
  if (!fn.gather || splits < 1 || (splits > 1) != (a.partial != nullptr) || !h.scale || !h.wh || !h.hh)
    return hipErrorInvalidValue;
  if (a.gpad % 32 != 0 || a.g_split % 32 != 0 || a.tile % 32 != 0 || a.tile <= 0) return hipErrorInvalidValue;
  if (a.M <= 0) return hipSuccess;
  const int64_t waves = (a.M + 15) / 16;
  const int64_t blocks = (waves + kFwdHalfWaves - 1) / kFwdHalfWaves;
  const FwdHalfFn g = a.tile >= a.g_split ? fn.gather_row : fn.gather;
  hipLaunchKernelGGL(g, dim3((unsigned)blocks, (unsigned)splits), dim3(64 * kFwdHalfWaves), 0, s, h);
  return hipGetLastError();
}

}  // namespace ncmri
