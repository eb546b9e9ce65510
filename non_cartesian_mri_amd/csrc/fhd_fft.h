// Batched power-of-two FFTs of lines (gfx950), for the Toeplitz normal
// operator and the gridding reconstruction.
//
// A workgroup transforms Lds<N, LAY>::kLines lines of N points (N = 2^p,
// 2 <= N <= 1024); every thread holds 16 complex values per stage, so the
// register footprint does not depend on N.  The transform is the
// self-sorting (Stockham) formulation: stage s with radix R combines R
// sub-transforms of length Ns (the product of the earlier radices) into
// transforms of length Ns R; butterfly j reads its R inputs at j + r N/R,
// multiplies input r by w_N^(r (j mod Ns) N / (Ns R)), takes an R-point DFT in
// registers and writes output r to (j div Ns) Ns R + (j mod Ns) + r Ns.
// Radices: 16s and, when p is not a multiple of 4, one stage of 2, 4 or 8,
// either first (ascending order) or last (descending order); N = 256 takes
// two stages.  The R-point DFTs are radix-2 decimation in frequency in
// registers with the sixteenth-turn twiddles as constants; w_N^t =
// e^(-2 pi i t / N) comes from a per-workgroup table computed with the
// library's own sincos in turns.
//
// Only the exchanges between stages go through LDS.  The first stage takes
// its inputs from the caller (global memory: butterfly j's inputs j + r N/R
// are points of one line, and consecutive threads take consecutive lines in a
// column tile or consecutive points in a row tile, so the reads coalesce), and
// the last stage hands its outputs to the caller at their final positions:
// the last stage has Ns R = N, so butterfly j writes points j + r N/R, the
// same positions it would read.  The first stage of a transform in the
// descending order reads exactly the points that the last stage of one in
// the ascending order wrote from the same butterflies (both radix 16, or
// both the single stage when N <= 16), so a forward transform, a pointwise
// product and an inverse transform chain in registers with no LDS exchange
// in between.
//
// Two LDS layouts for the exchanges:
//   row    -- line l, point i at l * pitch + swizzle(i): lines that are
//             contiguous in memory (x axis); 4096 values per workgroup (256
//             threads); the XOR swizzle within 16-point chunks and the
//             16-point pad keep the stage reads and writes of a half-wave on
//             distinct banks for N = 256.
//   column -- point i of line l at i * (lines + 1) + l: lines that are
//             adjacent columns in memory (y, z axes), at least 16 columns
//             (128 bytes) per workgroup so that every row of the tile is one
//             full cache line: 4096 values (256 threads) up to N = 256, 16 N
//             values (N threads) beyond;
//   narrow column -- 8 columns (64-byte rows, 8 N values, N / 2 threads) and
//             no pad, for N = 1024: 64 KB, so that two workgroups fit a CU's
//             LDS (the fused spectral-product pass, where overlapping one
//             workgroup's loads with another's transforms pays more than
//             full-line rows).  A one-point pad (72 KB + the 8 KB twiddles,
//             exactly 80 KB) measured slower: 5.84 against 5.69 ms for the
//             512^3 pass.
#pragma once

#include <hip/hip_runtime.h>

#include "fhd_trig.h"

namespace ncmri {
namespace fft {

constexpr int kThreads = 256;   // threads of a 4096-value workgroup
constexpr int kPerThread = 16;  // complex values per thread and stage
constexpr int kMaxLen = 1024;

__host__ __device__ constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

// LDS layouts (template parameter LAY of the helpers below)
enum Layout { kRows = 0, kCols = 1, kColsNarrow = 2 };

template <int N, int LAY>
struct Lds {
  static constexpr bool ROW = LAY == kRows;
  static constexpr int kColLines = LAY == kColsNarrow ? 8 : (N > 256 ? 16 : 4096 / N);
  static constexpr int kElems = ROW ? 4096 : kColLines * N;  // values per workgroup
  static constexpr int kThreads = kElems / kPerThread;
  static constexpr int kLines = kElems / N;
  static constexpr int kRowPitch = N >= 32 ? N + 16 : N;
  static constexpr int kColPitch = LAY == kColsNarrow ? kLines : kLines + 1;
  static constexpr int kSize = ROW ? kLines * kRowPitch : N * kColPitch;
  __device__ static __forceinline__ int addr(int l, int i) {
    if constexpr (ROW) {
      return l * kRowPitch + (i ^ ((i >> 4) & 15));
    } else {
      return i * kColPitch + l;
    }
  }
};

// Radix schedule of an N-point transform.
template <int N>
struct Sched {
  static_assert(N >= 2 && N <= kMaxLen && (N & (N - 1)) == 0, "power of two in [2, 1024]");
  static constexpr int kP = ilog2(N);
  static constexpr int kRem = kP % 4;
  static constexpr int kStages = (kP + 3) / 4;
  // DESC: the short stage (radix 2^(p mod 4)) last instead of first
  static constexpr int radix(int s, bool desc) {
    return kRem == 0 ? 16 : (s == (desc ? kStages - 1 : 0) ? (1 << kRem) : 16);
  }
  static constexpr int ns(int s, bool desc) {
    int n = 1;
    for (int i = 0; i < s; ++i) n *= radix(i, desc);
    return n;
  }
  static constexpr int first(bool desc) { return radix(0, desc); }
  static constexpr int last(bool desc) { return radix(kStages - 1, desc); }
};

// Butterfly k (< 16 / R) of this thread in a radix-R stage: line l of the
// workgroup and butterfly j < N / R of that line.  Column tiles give
// consecutive threads consecutive lines, row tiles consecutive butterflies.
template <int N, int R, int LAY>
__device__ __forceinline__ void locate(int k, int& l, int& j) {
  using L = Lds<N, LAY>;
  constexpr unsigned kBf = N / R;
  const unsigned b = threadIdx.x + (unsigned)(k * L::kThreads);
  if constexpr (L::ROW) {
    l = (int)(b / kBf);
    j = (int)(b % kBf);
  } else {
    l = (int)(b % (unsigned)L::kLines);
    j = (int)(b / (unsigned)L::kLines);
  }
}

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 w) {
  return make_float2(__builtin_fmaf(a.x, w.x, -(a.y * w.y)), __builtin_fmaf(a.x, w.y, a.y * w.x));
}

// a * e^(-+2 pi i t / 16) for a compile-time t in [0, 8) (after unrolling).
template <bool INV>
__device__ __forceinline__ float2 rot16(float2 a, int t) {
  // cos and sin of t/16 turns, t = 0..7
  constexpr float c16[8] = {1.0f, 0.92387953251128674f, 0.70710678118654752f, 0.38268343236508978f,
                            0.0f, -0.38268343236508978f, -0.70710678118654752f, -0.92387953251128674f};
  constexpr float s16[8] = {0.0f, 0.38268343236508978f, 0.70710678118654752f, 0.92387953251128674f,
                            1.0f, 0.92387953251128674f, 0.70710678118654752f, 0.38268343236508978f};
  if (t == 0) return a;
  if (t == 4) return INV ? make_float2(-a.y, a.x) : make_float2(a.y, -a.x);
  return cmul(a, make_float2(c16[t], INV ? s16[t] : -s16[t]));
}

__host__ __device__ constexpr int bitrev(int i, int bits) {
  int r = 0;
  for (int b = 0; b < bits; ++b) r |= ((i >> b) & 1) << (bits - 1 - b);
  return r;
}

// In-register R-point DFT (R = 2, 4, 8, 16), natural order in and out.
// HALF_IN: inputs R/2 .. R-1 are zero (not read), which turns the first
// butterfly level into copies and rotations.
template <int R, bool INV, bool HALF_IN = false>
__device__ __forceinline__ void dft(float2* v) {
#pragma unroll
  for (int half = R / 2; half >= 1; half /= 2) {
#pragma unroll
    for (int start = 0; start < R; start += 2 * half) {
#pragma unroll
      for (int k = 0; k < half; ++k) {
        if (HALF_IN && half == R / 2) {
          v[start + k + half] = rot16<INV>(v[start + k], k * (16 / (2 * half)));
        } else {
          const float2 a = v[start + k], b = v[start + k + half];
          v[start + k] = cadd(a, b);
          v[start + k + half] = rot16<INV>(csub(a, b), k * (16 / (2 * half)));
        }
      }
    }
  }
  float2 o[R];
#pragma unroll
  for (int i = 0; i < R; ++i) o[bitrev(i, ilog2(R))] = v[i];
#pragma unroll
  for (int i = 0; i < R; ++i) v[i] = o[i];
}

// The R-point DFTs of a thread's 16 / R butterflies; butterfly k's values
// are v[k R .. k R + R).
template <int R, bool INV, bool HALF_IN = false>
__device__ __forceinline__ void dft_all(float2* v) {
#pragma unroll
  for (int k = 0; k < kPerThread / R; ++k) dft<R, INV, HALF_IN>(v + k * R);
}

// Stage inputs from LDS, twiddled.
template <int N, int R, int NS, int LAY, bool INV>
__device__ __forceinline__ void read_stage(const float2* buf, const float2* tw, float2* v) {
  using L = Lds<N, LAY>;
  constexpr int kBf = N / R;
#pragma unroll
  for (int k = 0; k < kPerThread / R; ++k) {
    int l, j;
    locate<N, R, LAY>(k, l, j);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float2 a = buf[L::addr(l, j + r * kBf)];
      if (NS > 1 && r > 0) {
        float2 w = tw[r * (j % NS) * (N / (NS * R))];
        if (INV) w.y = -w.y;
        a = cmul(a, w);
      }
      v[k * R + r] = a;
    }
  }
}

// Stage outputs to LDS.
template <int N, int R, int NS, int LAY>
__device__ __forceinline__ void write_stage(float2* buf, const float2* v) {
  using L = Lds<N, LAY>;
#pragma unroll
  for (int k = 0; k < kPerThread / R; ++k) {
    int l, j;
    locate<N, R, LAY>(k, l, j);
    const int d = (j / NS) * NS * R + (j % NS);
#pragma unroll
    for (int r = 0; r < R; ++r) buf[L::addr(l, d + r * NS)] = v[k * R + r];
  }
}

// Stages S .. last through LDS.  On entry v holds the outputs of stage S - 1
// (after its DFTs), on exit those of the last stage.  Starts with a barrier,
// so the buffer may still be read by earlier code, and ends without one.
template <int N, int LAY, bool INV, bool DESC, int S = 1>
__device__ __forceinline__ void through_lds(float2* buf, const float2* tw, float2* v) {
  using Sc = Sched<N>;
  if constexpr (S < Sc::kStages) {
    constexpr int Rp = Sc::radix(S - 1, DESC), NSp = Sc::ns(S - 1, DESC);
    constexpr int R = Sc::radix(S, DESC), NS = Sc::ns(S, DESC);
    __syncthreads();
    write_stage<N, Rp, NSp, LAY>(buf, v);
    __syncthreads();
    read_stage<N, R, NS, LAY, INV>(buf, tw, v);
    dft_all<R, INV>(v);
    through_lds<N, LAY, INV, DESC, S + 1>(buf, tw, v);
  }
}

// The first stage (no twiddles: Ns = 1) with inputs from the caller:
// load.template get<RN, STEP>(l, j, w) fills w[r], r < RN, with point
// j + r STEP of line l.  HALF_IN: the points from N/2 on are zero, which are
// inputs r >= R/2 of every butterfly (j < N/R), so only RN = R/2 are read.
template <int N, int LAY, bool INV, bool DESC, bool HALF_IN, class Load>
__device__ __forceinline__ void first_stage(const Load& load, float2* v) {
  constexpr int R = Sched<N>::first(DESC);
  constexpr int RN = HALF_IN ? R / 2 : R;
#pragma unroll
  for (int k = 0; k < kPerThread / R; ++k) {
    int l, j;
    locate<N, R, LAY>(k, l, j);
    load.template get<RN, N / R>(l, j, v + k * R);
  }
  dft_all<R, INV, HALF_IN>(v);
}

// Unnormalised DFT (forward: e^(-2 pi i jk/N); inverse: e^(+2 pi i jk/N)) of
// the workgroup's lines: inputs from `load` (as in first_stage), outputs of
// the last stage left in v (see last_stage).  The twiddle table may be
// filled just before the call: the barriers of the LDS exchanges order it.
template <int N, int LAY, bool INV, bool DESC, bool HALF_IN, class Load>
__device__ __forceinline__ void transform(const Load& load, float2* buf, const float2* tw, float2* v) {
  first_stage<N, LAY, INV, DESC, HALF_IN>(load, v);
  through_lds<N, LAY, INV, DESC>(buf, tw, v);
}

// The last stage's outputs to the caller: store.template put<RN, STEP>(l, j, w)
// takes w[r], r < RN, as point j + r STEP of line l.  HALF_OUT: only the
// points below N/2 are wanted, outputs r < R/2 of every butterfly (the
// computation of the others is then dead code).
template <int N, int LAY, bool DESC, bool HALF_OUT, class Store>
__device__ __forceinline__ void last_stage(const Store& store, const float2* v) {
  constexpr int R = Sched<N>::last(DESC);
  constexpr int RN = HALF_OUT ? R / 2 : R;
#pragma unroll
  for (int k = 0; k < kPerThread / R; ++k) {
    int l, j;
    locate<N, R, LAY>(k, l, j);
    store.template put<RN, N / R>(l, j, v + k * R);
  }
}

// tw[t] = e^(-2 pi i t / N), t < N.
template <int N>
__device__ __forceinline__ void fill_twiddles(float2* tw) {
  for (int t = threadIdx.x; t < N; t += blockDim.x) {
    float s, c;
    sincos_turns((float)t * (1.0f / (float)N), s, c);
    tw[t] = make_float2(c, -s);
  }
}

}  // namespace fft
}  // namespace ncmri
