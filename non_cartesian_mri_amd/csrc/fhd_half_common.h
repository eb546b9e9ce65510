// fp16 hi/lo splitting for the half-split matrix-core engines (F^H D, Q and
// the forward operator): an fp32 value x becomes hi + lo with hi = fp16(x),
// lo = fp16(x - hi), and a product x y is formed as hi hi + hi lo + lo hi on
// v_mfma_f32_16x16x32_f16 with fp32 accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ncmri {
namespace {

// Operand layouts of v_mfma_f32_16x16x32_f16 (wave64): A[i][k] = lane i + 16 (k / 8), element k % 8;
// B[k][j] = lane j + 16 (k / 8), element k % 8; D[i][j] = element i % 4 of
// lane j + 16 (i / 4) (checked on gfx950).
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

// hi = fp16(x), lo = fp16(x - hi): x = hi + lo to 2^-22 relative (the
// difference x - hi is exact in fp32); lo underflows to a subnormal only for
// |x| below ~2^-3, where its absolute error (< 2^-25) stays far below the
// operands' scale.
__device__ __forceinline__ void split_half(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

// Two values at once: hi = (fp16(x0), fp16(x1)) packed by one conversion,
// and lo = fp16(x - hi) formed by the mixed-precision FMA, which reads the
// fp16 hi from either half of the packed register, adds x in fp32 (exact:
// x - hi is representable) and rounds once to fp16 into the low or high
// half of lo: the same bits as split_half, in 3 instructions instead of 8.
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const half2v h = {(_Float16)x0, (_Float16)x1};
  hi = __builtin_bit_cast(uint32_t, h);
  uint32_t l;
  asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(l) : "v"(hi), "v"(x0));
  asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(l) : "v"(hi), "v"(x1));
  lo = l;
}

}  // namespace
}  // namespace ncmri
