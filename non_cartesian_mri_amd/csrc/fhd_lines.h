// Batched line transforms over one axis of a 3-D array (fhd_lines.hip): the
// LDS line FFTs of fhd_fft.h applied to every line of an axis, shared by the
// Toeplitz normal operator and the gridding reconstruction.  Internal; not
// part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ncmri {

// One axis of transforms over a batch of lines.  Line c sits at outer index
// o = c / inner and inner index w = c % inner; its point i is at
// o * os + (w >> sh) * wh + (w mod 2^sh) * ws + i * es of the array (sh = 30,
// wh = 0 for the plain o * os + w * ws; a smaller sh splits w into blocks of
// 2^sh lines that sit wh apart).  In and out may be the same array when they
// share a layout: every line is read whole before any of it is written.
struct LinePass {
  const float2* in;
  float2* out;
  // kLineFwdQInv: the real spectrum in blocks of W = 2^q_shift lines, point-major
  // within a block: point i of line c at q[(c >> q_shift) q_bs + (c mod W) + i W]
  const float* q;
  int count;       // lines
  int inner;
  int64_t in_os, in_ws, in_es;
  int64_t out_os, out_ws, out_es;
  int in_sh, out_sh;
  int64_t in_wh, out_wh;
  int q_shift;
  int64_t q_bs;
  int nin;         // points read per line (the rest are zero)
  int nout;        // points written per line (the first nout)
};

enum LineMode {
  kLineFwd = 0,     // unnormalised forward DFT, e^(-2 pi i jk/N)
  kLineInv = 1,     // unnormalised inverse DFT, e^(+2 pi i jk/N)
  kLineFwdQInv = 2  // forward DFT, times q, inverse DFT
};

// A pass whose input and output share one layout.
LinePass line_pass(const float2* in, float2* out, int64_t count, int64_t inner, int64_t os, int64_t ws,
                   int64_t es, int nin, int nout);

// Launches the transforms of a.count lines of N points (N a power of two in
// [2, 1024]); `row` selects the LDS layout for lines contiguous in memory
// (es == 1), otherwise lines are adjacent columns.  kLineFwdQInv takes the
// column layout only.
hipError_t launch_lines(bool row, int mode, int N, const LinePass& a, hipStream_t s);

}  // namespace ncmri
