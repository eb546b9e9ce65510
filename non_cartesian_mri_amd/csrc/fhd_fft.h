// Batched power-of-two FFTs of lines held in LDS (gfx950), for the Toeplitz
// normal operator and the gridding reconstruction.
//
// A workgroup transforms lines of N points (N = 2^p, 2 <= N <= 1024) held in
// LDS; every thread holds 16 complex values per stage, so the register
// footprint does not depend on N.  The transform is the self-sorting
// (Stockham) formulation: stage s with radix R combines R sub-transforms of
// length Ns (the product of the earlier radices) into transforms of length
// Ns R; the butterfly j reads its R inputs at j + r N/R, multiplies input r by
// w_N^(r (j mod Ns) N / (Ns R)), takes an R-point DFT in registers and writes
// output r to (j div Ns) Ns R + (j mod Ns) + r Ns.  Radices: 2, 4 or 8 first
// (N's bits mod 4), then 16s, so N = 256 takes two stages through LDS.  The
// R-point DFTs are radix-2 decimation in frequency in registers with the
// sixteenth-turn twiddles as constants.  w_N^t = e^(-2 pi i t / N) comes from a
// per-workgroup table computed with the library's own sincos in turns.
//
// Two LDS layouts:
//   row    -- line l, point i at l * pitch + swizzle(i): lines that are
//             contiguous in memory (x axis); 4096 values per workgroup (256
//             threads); the XOR swizzle within 16-point chunks and the
//             16-point pad keep the stage reads and writes of a half-wave on
//             distinct banks for N = 256.
//   column -- point i of line l at i * (lines + 1) + l: lines that are
//             adjacent columns in memory (y, z axes), at least 16 columns
//             (128 bytes) per workgroup so that every row of the tile is one
//             full cache line: 4096 values (256 threads) up to N = 256, 16 N
//             values (N threads) beyond.
#pragma once

#include <hip/hip_runtime.h>

#include "fhd_trig.h"

namespace ncmri {
namespace fft {

constexpr int kThreads = 256;   // threads of a 4096-value workgroup
constexpr int kPerThread = 16;  // complex values per thread and stage
constexpr int kMaxLen = 1024;

__host__ __device__ constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

template <int N, bool ROW>
struct Lds {
  static constexpr int kElems = ROW ? 4096 : (16 * N > 4096 ? 16 * N : 4096);  // values per workgroup
  static constexpr int kThreads = kElems / kPerThread;
  static constexpr int kLines = kElems / N;
  static constexpr int kRowPitch = N >= 32 ? N + 16 : N;
  static constexpr int kColPitch = kLines + 1;
  static constexpr int kSize = ROW ? kLines * kRowPitch : N * kColPitch;
  __device__ static __forceinline__ int addr(int l, int i) {
    if constexpr (ROW) {
      return l * kRowPitch + (i ^ ((i >> 4) & 15));
    } else {
      return i * kColPitch + l;
    }
  }
  // Threads of a row tile of N >= 256 points each keep one line (N / 16
  // threads per line, 16 points each); a column tile's threads keep one line
  // when the thread count is a multiple of the line count.
  static constexpr bool kThreadLine = ROW ? N >= 256 : kThreads % kLines == 0;
  static constexpr int kPointStep = ROW ? N / 16 : kThreads / kLines;  // for kThreadLine
  // element e of the workgroup's kElems in load/store order: consecutive
  // threads take consecutive points of a line (row) or consecutive lines
  // (column); element t + k kThreads of thread t is point i0 + k kPointStep
  // of the thread's line when kThreadLine
  __device__ static __forceinline__ void element(int e, int& l, int& i) {
    if constexpr (ROW && N >= 256) {
      const int t = e % kThreads, k = e / kThreads;
      l = t / (N / 16);
      i = t % (N / 16) + k * (N / 16);
    } else if constexpr (ROW) {
      l = e / N;
      i = e % N;
    } else {
      l = e % kLines;
      i = e / kLines;
    }
  }
};

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
template <int R, bool INV>
__device__ __forceinline__ void dft(float2* v) {
#pragma unroll
  for (int half = R / 2; half >= 1; half /= 2) {
#pragma unroll
    for (int start = 0; start < R; start += 2 * half) {
#pragma unroll
      for (int k = 0; k < half; ++k) {
        const float2 a = v[start + k], b = v[start + k + half];
        v[start + k] = cadd(a, b);
        v[start + k + half] = rot16<INV>(csub(a, b), k * (16 / (2 * half)));
      }
    }
  }
  float2 o[R];
#pragma unroll
  for (int i = 0; i < R; ++i) o[bitrev(i, ilog2(R))] = v[i];
#pragma unroll
  for (int i = 0; i < R; ++i) v[i] = o[i];
}

// One radix-R stage over all lines of the workgroup (in place, two barriers).
template <int N, int R, int NS, bool ROW, bool INV>
__device__ __forceinline__ void stage(float2* buf, const float2* tw) {
  using L = Lds<N, ROW>;
  constexpr int kBf = N / R;                              // butterflies per line
  constexpr int kPer = L::kLines * kBf / L::kThreads;     // butterflies per thread (16 / R)
  static_assert(kPer * R == kPerThread, "16 values per thread");
  float2 v[kPer][R];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int b = threadIdx.x + k * L::kThreads;
    const int l = ROW ? b / kBf : b % L::kLines;
    const int j = ROW ? b % kBf : b / L::kLines;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float2 a = buf[L::addr(l, j + r * kBf)];
      if (NS > 1 && r > 0) {
        float2 w = tw[r * (j % NS) * (N / (NS * R))];
        if (INV) w.y = -w.y;
        a = cmul(a, w);
      }
      v[k][r] = a;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int b = threadIdx.x + k * L::kThreads;
    const int l = ROW ? b / kBf : b % L::kLines;
    const int j = ROW ? b % kBf : b / L::kLines;
    dft<R, INV>(v[k]);
    const int d = (j / NS) * NS * R + (j % NS);
#pragma unroll
    for (int r = 0; r < R; ++r) buf[L::addr(l, d + r * NS)] = v[k][r];
  }
  __syncthreads();
}

// Unnormalised DFT (forward: e^(-2 pi i jk/N); inverse: e^(+2 pi i jk/N)) of
// every line in LDS.  Expects a barrier between the last writes to buf / tw
// and the call; ends with a barrier.
template <int N, bool ROW, bool INV>
__device__ __forceinline__ void transform(float2* buf, const float2* tw) {
  static_assert(N >= 2 && N <= kMaxLen && (N & (N - 1)) == 0, "power of two in [2, 1024]");
  constexpr int p = ilog2(N);
  constexpr int rem = p % 4;
  constexpr int ns1 = rem != 0 ? (1 << rem) : 1;
  if constexpr (rem != 0) stage<N, (1 << rem), 1, ROW, INV>(buf, tw);
  if constexpr (p >= 4) stage<N, 16, ns1, ROW, INV>(buf, tw);
  if constexpr (p >= 8) stage<N, 16, ns1 * 16, ROW, INV>(buf, tw);
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
