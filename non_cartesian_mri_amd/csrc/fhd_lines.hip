// Batched line transforms over one axis of a 3-D array (see fhd_lines.h).
// A workgroup takes Lds<N, LAY>::kLines lines (zero-extending past nin
// points) straight from global memory into the first stage of the
// transforms of fhd_fft.h (forward, inverse, or forward then the product
// with a real spectrum then inverse, chained in registers) and stores the
// first nout points of each line from the last stage.  Where nin <= N/2 (a
// zero-padded line) or nout <= N/2 (a cropped one) the launch takes a
// variant that neither reads the known zeros nor computes the discarded
// half.
#include "fhd_fft.h"
#include "fhd_lines.h"

namespace ncmri {
namespace {

// Offset of line c: outer index o = c / inner, inner index w = c mod inner,
// w split into blocks of 2^sh lines wh apart.
__device__ __forceinline__ int64_t line_offset(int c, int inner, int64_t os, int64_t ws, int sh, int64_t wh) {
  const int o = c / inner, w = c - o * inner;
  return o * os + (int64_t)(w >> sh) * wh + (int64_t)(w & ((1 << sh) - 1)) * ws;
}

// Inputs of the first stage: point i of line c0 + l, zero past nin points
// or past the last line.
struct LineLoad {
  const float2* in;
  int c0, count, inner, nin;
  int64_t os, ws, es;
  int sh;
  int64_t wh;
  template <int RN, int STEP>
  __device__ __forceinline__ void get(int l, int j, float2* w) const {
    const int c = c0 + l;
    const bool ok = c < count;
    const float2* p = in + (line_offset(ok ? c : 0, inner, os, ws, sh, wh) + j * es);
    const int64_t st = (int64_t)STEP * es;
#pragma unroll
    for (int r = 0; r < RN; ++r) {
      w[r] = (ok && j + r * STEP < nin) ? *p : make_float2(0.0f, 0.0f);
      p += st;
    }
  }
};

// Outputs of the last stage: the first nout points of each existing line.
struct LineStore {
  float2* out;
  int c0, count, inner, nout;
  int64_t os, ws, es;
  int sh;
  int64_t wh;
  template <int RN, int STEP>
  __device__ __forceinline__ void put(int l, int j, const float2* w) const {
    const int c = c0 + l;
    if (c >= count) return;
    float2* p = out + (line_offset(c, inner, os, ws, sh, wh) + j * es);
    const int64_t st = (int64_t)STEP * es;
#pragma unroll
    for (int r = 0; r < RN; ++r) {
      if (j + r * STEP < nout) *p = w[r];
      p += st;
    }
  }
};

// PRUNE: bit 0 -- nin <= N/2, bit 1 -- nout <= N/2.
enum { kPruneIn = 1, kPruneOut = 2 };

// Tile of block b when G consecutive column tiles share 128-byte lines (G = 2:
// 64-byte rows of complex values or of 16 spectrum floats; G = 4: 32-byte
// rows of 8 spectrum floats).  Workgroups go to the 8 XCDs in turn (block b
// to XCD b mod 8), each with its own L2, so tiles Gk .. Gk + G - 1 are given
// blocks 8Gm + i + 8q (q < G), which share an XCD.  The grid is a multiple of
// 8G blocks.
template <int G>
__device__ __forceinline__ int grouped_tile(int b) {
  if constexpr (G == 1) {
    return b;
  } else {
    return (b / (8 * G)) * (8 * G) + (b % 8) * G + (b / 8) % G;
  }
}

// LDS layout of a pass: rows, or column tiles (narrow ones for the 1024-point
// spectral product, see fhd_fft.h).
template <int N, bool ROW, int MODE>
constexpr int layout() {
  return ROW ? fft::kRows : (MODE == kLineFwdQInv && N >= 1024 ? fft::kColsNarrow : fft::kCols);
}

// Tiles per line-sharing group: complex rows need 16 columns per 128-byte
// line, spectrum rows (the product pass) 32.
template <int N, bool ROW, int MODE>
constexpr int tile_group() {
  if constexpr (ROW) {
    return 1;
  } else {
    constexpr int lines = fft::Lds<N, layout<N, ROW, MODE>()>::kLines;
    constexpr int per = MODE == kLineFwdQInv ? 32 : 16;
    return lines >= per ? 1 : per / lines;
  }
}

template <int N, bool ROW, int MODE, int PRUNE>
__global__ void __launch_bounds__((fft::Lds<N, layout<N, ROW, MODE>()>::kThreads)) line_fft_kernel(LinePass a) {
  constexpr bool kHalfIn = (PRUNE & kPruneIn) != 0, kHalfOut = (PRUNE & kPruneOut) != 0;
  constexpr int LAY = layout<N, ROW, MODE>();
  using L = fft::Lds<N, LAY>;
  using S = fft::Sched<N>;
  __shared__ float2 buf[L::kSize];
  __shared__ float2 tw[N];
  fft::fill_twiddles<N>(tw);
  const int tile = grouped_tile<tile_group<N, ROW, MODE>()>((int)blockIdx.x);
  const int c0 = tile * L::kLines;   // past the last line (padding blocks): nothing read or written
  const LineLoad load{a.in, c0, a.count, a.inner, a.nin, a.in_os, a.in_ws, a.in_es, a.in_sh, a.in_wh};
  const LineStore store{a.out, c0, a.count, a.inner, a.nout, a.out_os, a.out_ws, a.out_es, a.out_sh, a.out_wh};
  float2 v[fft::kPerThread];
  if constexpr (MODE == kLineFwdQInv) {
    static_assert(!ROW, "the spectral product runs on column tiles");
    // The spectrum at the points of the forward transform's last stage; read
    // before the transform where registers allow (it then arrives while the
    // transform runs), after it for the 1024-thread tiles.
    constexpr int RL = S::last(false), kStep = N / RL;
    static_assert(RL == S::first(true), "the inverse's first stage takes the forward's last outputs");
    float qv[fft::kPerThread];
    auto load_q = [&]() {
#pragma unroll
      for (int k = 0; k < fft::kPerThread / RL; ++k) {
        int l, j;
        fft::locate<N, RL, LAY>(k, l, j);
        const int c = c0 + l;
        const float* qp = a.q + ((int64_t)(c >> a.q_shift) * a.q_bs + (c & ((1 << a.q_shift) - 1)) +
                                 ((int64_t)j << a.q_shift));
        const int64_t qst = (int64_t)kStep << a.q_shift;
#pragma unroll
        for (int r = 0; r < RL; ++r) {
          qv[k * RL + r] = c < a.count ? *qp : 0.0f;
          qp += qst;
        }
      }
    };
    constexpr bool kPrefetchQ = L::kThreads <= 512;
    if constexpr (kPrefetchQ) load_q();
    fft::transform<N, LAY, false, false, kHalfIn>(load, buf, tw, v);
    if constexpr (!kPrefetchQ) load_q();
#pragma unroll
    for (int i = 0; i < fft::kPerThread; ++i) v[i] = make_float2(v[i].x * qv[i], v[i].y * qv[i]);
    fft::dft_all<S::first(true), true>(v);
    fft::through_lds<N, LAY, true, true>(buf, tw, v);
    fft::last_stage<N, LAY, true, kHalfOut>(store, v);
  } else {
    fft::transform<N, LAY, MODE == kLineInv, false, kHalfIn>(load, buf, tw, v);
    fft::last_stage<N, LAY, false, kHalfOut>(store, v);
  }
}

template <int N, bool ROW, int MODE, int PRUNE>
hipError_t launch_grid(const LinePass& a, hipStream_t s) {
  using L = fft::Lds<N, layout<N, ROW, MODE>()>;
  constexpr int lines = L::kLines;
  int grid = (a.count + lines - 1) / lines;
  if (grid == 0) return hipSuccess;
  constexpr int kGroup = 8 * tile_group<N, ROW, MODE>();
  grid = (grid + kGroup - 1) / kGroup * kGroup;   // whole groups for grouped_tile
  hipLaunchKernelGGL((line_fft_kernel<N, ROW, MODE, PRUNE>), dim3(grid), dim3(L::kThreads), 0, s, a);
  return hipGetLastError();
}

// The pruned variants that the passes use: a forward transform of a
// zero-padded line, an inverse whose output is cropped, and the spectral
// product with both; every mode also has the full one.
template <int N, bool ROW, int MODE>
hipError_t launch_lines_n(const LinePass& a, hipStream_t s) {
  const bool half_in = a.nin <= N / 2, half_out = a.nout <= N / 2;
  if constexpr (MODE == kLineFwd) {
    if (half_in) return launch_grid<N, ROW, MODE, kPruneIn>(a, s);
  } else if constexpr (MODE == kLineInv) {
    if (half_out) return launch_grid<N, ROW, MODE, kPruneOut>(a, s);
  } else {
    if (half_in && half_out) return launch_grid<N, ROW, MODE, kPruneIn | kPruneOut>(a, s);
  }
  return launch_grid<N, ROW, MODE, 0>(a, s);
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
  a.in_sh = a.out_sh = 30;
  a.in_wh = a.out_wh = 0;
  a.q_shift = 0;
  a.q_bs = 0;
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
