// Batched line transforms over one axis of a 3-D array (see fhd_lines.h).
// A workgroup loads Lds<N, ROW>::kLines lines (zero-extending past nin points), runs
// the LDS transform of fhd_fft.h (optionally forward, times a real spectrum,
// inverse) and stores the first nout points of each line.
#include "fhd_fft.h"
#include "fhd_lines.h"

namespace ncmri {
namespace {

template <int N, bool ROW, int MODE>
__global__ void __launch_bounds__((fft::Lds<N, ROW>::kThreads)) line_fft_kernel(LinePass a) {
  using L = fft::Lds<N, ROW>;
  __shared__ float2 buf[L::kSize];
  __shared__ float2 tw[N];
  fft::fill_twiddles<N>(tw);
  const int c0 = blockIdx.x * L::kLines;
  float qv[fft::kPerThread];
  // the spectrum is read before the transform where registers allow (it
  // then arrives while the transform runs); the 1024-thread tiles read it after
  constexpr bool kPrefetchQ = L::kThreads <= 512;
  if constexpr (L::kThreadLine) {
    // one line per thread: its address and bounds once, then a running pointer
    int l0, i0;
    L::element(threadIdx.x, l0, i0);
    constexpr int di = L::kPointStep;
    const int c = c0 + l0;
    const bool ok = c < a.count;
    const int o = c / a.inner, w = c - o * a.inner;
    const float2* p = a.in + (o * a.in_os + w * a.in_ws + i0 * a.in_es);
    const int64_t st = (int64_t)di * a.in_es;
    const float* qp = a.q + (c + (int64_t)i0 * a.q_es);
    const int64_t qst = (int64_t)di * a.q_es;
#pragma unroll
    for (int k = 0; k < fft::kPerThread; ++k) {
      const int i = i0 + k * di;
      buf[L::addr(l0, i)] = (ok && i < a.nin) ? *p : make_float2(0.0f, 0.0f);
      p += st;
      if constexpr (MODE == kLineFwdQInv && kPrefetchQ) {
        qv[k] = ok ? *qp : 0.0f;
        qp += qst;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < fft::kPerThread; ++k) {
      int l, i;
      L::element(threadIdx.x + k * L::kThreads, l, i);
      const int c = c0 + l;
      float2 v = make_float2(0.0f, 0.0f);
      if (c < a.count && i < a.nin) {
        const int o = c / a.inner, w = c - o * a.inner;
        v = a.in[o * a.in_os + w * a.in_ws + i * a.in_es];
      }
      buf[L::addr(l, i)] = v;
      if constexpr (MODE == kLineFwdQInv && kPrefetchQ) qv[k] = c < a.count ? a.q[c + i * a.q_es] : 0.0f;
    }
  }
  __syncthreads();
  fft::transform<N, ROW, MODE == kLineInv>(buf, tw);
  if constexpr (MODE == kLineFwdQInv) {
#pragma unroll
    for (int k = 0; k < fft::kPerThread; ++k) {
      int l, i;
      L::element(threadIdx.x + k * L::kThreads, l, i);
      float q;
      if constexpr (kPrefetchQ) {
        q = qv[k];
      } else {
        const int c = c0 + l;
        q = c < a.count ? a.q[c + i * a.q_es] : 0.0f;
      }
      const float2 v = buf[L::addr(l, i)];
      buf[L::addr(l, i)] = make_float2(v.x * q, v.y * q);
    }
    __syncthreads();
    fft::transform<N, ROW, true>(buf, tw);
  }
  if constexpr (L::kThreadLine) {
    int l0, i0;
    L::element(threadIdx.x, l0, i0);
    constexpr int di = L::kPointStep;
    const int c = c0 + l0;
    if (c < a.count) {
      const int o = c / a.inner, w = c - o * a.inner;
      float2* p = a.out + (o * a.out_os + w * a.out_ws + i0 * a.out_es);
      const int64_t st = (int64_t)di * a.out_es;
#pragma unroll
      for (int k = 0; k < fft::kPerThread; ++k) {
        const int i = i0 + k * di;
        if (i < a.nout) *p = buf[L::addr(l0, i)];
        p += st;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < fft::kPerThread; ++k) {
      int l, i;
      L::element(threadIdx.x + k * L::kThreads, l, i);
      const int c = c0 + l;
      if (c < a.count && i < a.nout) {
        const int o = c / a.inner, w = c - o * a.inner;
        a.out[o * a.out_os + w * a.out_ws + i * a.out_es] = buf[L::addr(l, i)];
      }
    }
  }
}

template <int N, bool ROW, int MODE>
hipError_t launch_lines_n(const LinePass& a, hipStream_t s) {
  constexpr int lines = fft::Lds<N, ROW>::kLines;
  const int grid = (a.count + lines - 1) / lines;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((line_fft_kernel<N, ROW, MODE>), dim3(grid), dim3(fft::Lds<N, ROW>::kThreads), 0, s, a);
  return hipGetLastError();
}

template <bool ROW, int MODE>
hipError_t launch_mode(int N, const LinePass& a, hipStream_t s) {
  switch (N) {
    case 2: return launch_lines_n<2, ROW, MODE>(a, s);
    case 4: return launch_lines_n<4, ROW, MODE>(a, s);
    case 8: return launch_lines_n<8, ROW, MODE>(a, s);
    case 16: return launch_lines_n<16, ROW, MODE>(a, s);
    case 32: return launch_lines_n<32, ROW, MODE>(a, s);
    case 64: return launch_lines_n<64, ROW, MODE>(a, s);
    case 128: return launch_lines_n<128, ROW, MODE>(a, s);
    case 256: return launch_lines_n<256, ROW, MODE>(a, s);
    case 512: return launch_lines_n<512, ROW, MODE>(a, s);
    case 1024: return launch_lines_n<1024, ROW, MODE>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// A pass whose input and output share one layout.
LinePass line_pass(const float2* in, float2* out, int64_t count, int64_t inner, int64_t os, int64_t ws, int64_t es,
              int nin, int nout) {
  LinePass a{};
  a.in = in;
  a.out = out;
  a.q = nullptr;
  a.count = (int)count;
  a.inner = (int)inner;
  a.in_os = a.out_os = os;
  a.in_ws = a.out_ws = ws;
  a.in_es = a.out_es = es;
  a.q_es = 0;
  a.nin = nin;
  a.nout = nout;
  return a;
}


hipError_t launch_lines(bool row, int mode, int N, const LinePass& a, hipStream_t s) {
  if (row) {
    if (mode == kLineFwd) return launch_mode<true, kLineFwd>(N, a, s);
    if (mode == kLineInv) return launch_mode<true, kLineInv>(N, a, s);
    return hipErrorInvalidValue;
  }
  if (mode == kLineFwd) return launch_mode<false, kLineFwd>(N, a, s);
  if (mode == kLineInv) return launch_mode<false, kLineInv>(N, a, s);
  if (mode == kLineFwdQInv) return launch_mode<false, kLineFwdQInv>(N, a, s);
  return hipErrorInvalidValue;
}

}  // namespace ncmri
