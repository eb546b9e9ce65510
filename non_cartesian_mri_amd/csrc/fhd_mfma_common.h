// Device helpers shared by the gfx950 matrix-core kernels (F^H D / Q gather
// and the forward operator).
#pragma once

#include <hip/hip_runtime.h>

namespace ncmri {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Keeps the compiler's scheduler from moving instructions across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Raw buffer resource over [base, base + bytes) (stride 0; the third config
// dword of gfx9-family targets).  Loads outside the range return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// LDS DMA, 16 bytes per lane: the bytes at offset voff (per lane) of the
// buffer land at lds + 16 i for lane i (lds is wave-uniform).  The buffer
// (MUBUF) form is used rather than global_load_lds: it counts only in vmcnt,
// so the compiler keeps exact lgkmcnt waits for the LDS reads that follow.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, int voff, float4* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)lds, 16, voff, 0, 0, 0);
}

}  // namespace ncmri
