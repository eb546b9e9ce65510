// Internal interface of the half-split forward operator (fhd_forward_half.hip):
// the four-group forward engine with every fp32 product formed from fp16
// parts on v_mfma_f32_16x16x32_f16.  Not part of the ABI.
#pragma once

#include "fhd_internal.h"

namespace ncmri {

// One pass of the half-split forward operator: f as for the four-group engine
// (groups of 128 / BC voxels, its packed image f.gwb is the source of the
// parts), wh the fp16 parts [gpad / 32][8 tiles][3][2][64 lanes] (uint4 each:
// gpad x 1536 bytes; each 32-group chunk in the slot order its order kernel
// picks), hh the gather's headers [gpad] in the same order (x, y, z of the
// slot's group's first voxel; w: per octet of slots 8 o .. 8 o + 7, element
// 0 holds 1 when the octet's bases are equally spaced, elements 1-3 the
// spacing; element 4 of a chunk's first octet the chunk's order), scale
// [2 + 256] floats (2^e, 2^-e, per-block maxima).
struct FwdHalfArgs {
  FwdArgs f;
  void* wh;
  float4* hh;
  float* scale;
};

constexpr int kFwdHalfWaves = 8;   // waves per workgroup of the half-split forward gather

inline size_t fwd_half_parts_bytes(int64_t gpad) { return (size_t)gpad * 1536; }
inline size_t fwd_half_header_bytes(int64_t gpad) { return (size_t)gpad * 16; }
constexpr int kFwdHalfScaleFloats = 2 + 256;

bool fwd_half_supported(int BC);
// The scale of the packed image's entries and their fp16 parts (after
// launch_fwd_pack with T = 8 has written f.gwb).
hipError_t launch_fwd_half_pack(int BC, const FwdHalfArgs& a, hipStream_t s);
// The launch rows of the gather over the regular groups.
hipError_t launch_fwd_half_gather(int trig, int BC, int32_t splits, const FwdHalfArgs& a, hipStream_t s);

}  // namespace ncmri
