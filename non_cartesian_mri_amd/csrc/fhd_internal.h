// Internal interface between the C-ABI host code (fhd_api.hip) and the gfx950
// kernels (fhd_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ncmri {

constexpr int kWorkgroup = 256;   // lanes per workgroup (4 wave64)
#ifndef NCMRI_UNROLL
#define NCMRI_UNROLL 4
#endif
constexpr int kUnroll = NCMRI_UNROLL;  // samples per unrolled step; records are padded to it

enum Trig : int { kTrigAccurate = 0, kTrigHw = 1 };

// Record layout of one k-space sample as the per-sample kernel packs it and
// the gather kernel reads it (all dwords are float32):
//   header  HW trig:       kx, ky, kz                       (3 dwords)
//           accurate trig: khx, khy, khz, klx, kly, klz     (6 dwords)
//           k = kh + kl exactly, kh a multiple of 2^-12 (see fhd_kernels.hip)
//   then one weight set per (voxel offset j, vector b), set index s = j*BC + b:
//     complex set: (fr + fi, fr, fi) where f = Mu_b * exp(i 2 pi k.d_j)
//     real set (Q, j = 0 only): w = |phi|^2 (1 dword)
//   padded with zeros to a multiple of 4 dwords.
struct Layout {
  int is_q;      // 0: F^H D (complex Mu), 1: Q (real |phi|^2)
  int trig;      // Trig
  int V;         // voxels per lane (group size)
  int BC;        // data vectors per gather pass
  int header;    // header dwords
  int stride;    // dwords per record
};

inline constexpr int header_dwords(int trig) { return trig == kTrigHw ? 3 : 6; }

inline constexpr int record_dwords(int is_q, int trig, int V, int BC) {
  int w = is_q ? (1 + 3 * (V - 1)) : 3 * V * BC;
  int d = header_dwords(trig) + w;
  return (d + 3) / 4 * 4;
}

struct RecordArgs {
  const float* kx; const float* ky; const float* kz;
  const float* x; const float* y; const float* z;   // only x[0..V-1] etc. are read
  const float2* phi;
  const float2* D;       // first vector of this pass ([BC][M]); unused for Q
  int64_t M;             // real samples
  int64_t mpad;          // padded sample count (multiple of kUnroll)
  float* rec;            // [mpad][stride]
};

struct GatherArgs {
  const float* rec;      // [mpad][stride]
  int64_t mpad;
  int64_t tile;          // samples per summation tile (multiple of kUnroll)
  const float* x; const float* y; const float* z;
  int64_t N;
  float2* out;           // first output vector of this pass ([BC][N])
  int64_t m_split;       // samples per launch row (gridDim.y rows split the samples)
  float2* partial;       // [rows][BC][N] partial sums when rows > 1, else nullptr
};

// Launchers: return hipSuccess or the launch error.
hipError_t launch_records(const Layout& L, const RecordArgs& a, hipStream_t s);
// With splits > 1 the gather writes the rows' partial sums to a.partial and
// launch_reduce adds them into a.out (a no-op for splits == 1).
hipError_t launch_gather(const Layout& L, bool kahan, int32_t splits, const GatherArgs& a,
                         hipStream_t s);
hipError_t launch_reduce(int BC, bool kahan, int32_t splits, const GatherArgs& a, hipStream_t s);
bool gather_supported(int is_q, int V, int BC);

// ---------------------------------------------------------------------------
// Matrix-core (MFMA) engine.  Each wave owns 32 voxel groups of V voxels
// (V x BC = 16 T complex columns, i.e. T / 2 tiles of 32); per pair of
// samples it evaluates one phase per group and lane and accumulates three
// real products per tile (the three-multiplication complex product) with
// v_mfma_f32_32x32x2_f32, the K dimension running over the two samples.
constexpr int kMfmaChunk = 32;   // samples per LDS chunk; records are padded to it
constexpr int kMfma4Waves = 4;   // waves per workgroup of the four-sample engine (T = 8)
constexpr int kMfma4Chunk = 16;  // samples per LDS chunk of the four-sample engine (divides kMfmaChunk)

// Waves of a gather launch row: 32 groups per wave (T = 2, 4: two samples
// per v_mfma_f32_32x32x2_f32) or 16 (T = 8: four samples per
// v_mfma_f32_16x16x4_f32), groups of V = 16 T / BC voxels.
inline int64_t mfma_gather_waves(int64_t N, int T, int BC) {
  const int64_t V = 16 * T / BC, G = T == 8 ? 16 : 32;
  return ((N + V - 1) / V + G - 1) / G;
}

inline constexpr int mfma_header_floats(int trig) { return trig == kTrigHw ? 4 : 8; }
// factor floats per sample: 3 values per complex column
inline constexpr int mfma_factor_floats(int T) { return 48 * T; }
// dwords of one sample's records (header + factors)
inline constexpr int mfma_record_dwords(int trig, int T) { return mfma_header_floats(trig) + mfma_factor_floats(T); }

// Records of one sample m for the MFMA engine (all float32):
//   header hdr[m][]  HW trig:       kx, ky, kz, 0
//                    accurate trig: khx, khy, khz, 0, klx, kly, klz, 0
//   factors, T = 8 (four-sample engine): per block of four samples q = m / 4,
//     entry e = u T + t (u = 0: fr, 1: fi, 2: fr + fi; tile t of 16 complex
//     columns, cc = 16 t + c) of lane p = 16 (m % 4) + c at
//     wb[q][e / 4][p][e % 4] (192 T floats per block);
//   factors, T = 2, 4 (two-sample engine), per pair of samples h = m / 2 (P = T / 2 tiles of 32 complex
//     columns; complex column cc = 32 t + c holds f = Mu_b exp(i 2 pi k.d_j)
//     with b = cc / V, j = cc % V, V = 16 T / BC), 192 P floats per pair:
//       wb[h][p][2 P]   : [t] = fr, [P + t] = fi
//       wb[h][128 P + p P + t] : fr + fi (rounded once)
//     where p = 32 (m % 2) + c is the lane that supplies the entry as the
//     MFMA B operand (row k = m % 2, column c).
struct MfmaRecordArgs {
  const float* kx; const float* ky; const float* kz;
  const float* x; const float* y; const float* z;  // x[0..min(V,N)-1] etc. are read
  const float2* phi;
  const float2* D;       // first vector of this pass ([BC][M]); unused for Q
  int64_t M, N, mpad;    // mpad: multiple of kMfmaChunk
  float* hdr;            // [mpad][mfma_header_floats]
  float* wb;             // [mpad / 2][192 P] (P = T / 2)
  int32_t jref;          // reference column: factors hold Mu_b exp(i 2 pi k.(x_j - x_jref))
};

struct MfmaArgs {
  const float* hdr;
  const float* wb;
  int64_t mpad;
  int64_t tile;          // samples per summation tile (multiple of kMfmaChunk)
  const float* x; const float* y; const float* z;
  int64_t N;
  float2* out;           // first output vector of this pass ([BC][N])
  int64_t m_split;       // samples per launch row (multiple of kMfmaChunk)
  float2* partial;       // [rows][BC][N] when rows > 1, else nullptr
  int32_t* flags;        // [waves]: 1 when the gather wave's groups sit at common
                         // offsets (written by the gather's row 0, read by the
                         // direct kernel, which then skips the wave)
  // half-split engine only (nullptr otherwise)
  const float2* mu;      // [mpad][BC] Mu_b of each sample in fp32 (the direct kernel's weights)
  const float* scale;    // [2]: the factors' scale 2^e and its inverse (of a [2 + 256] buffer)
  // four-sample engine with mirror pairs (nullptr / 0 otherwise)
  const int32_t* pairs;  // pair plan: kPairHeader int32 then the int2 list (see below)
  int32_t jref;          // reference column of the factors (0 without pairs)
  int64_t gcap;          // list slots (groups of the pass)
};

// Mirror pairs (four-sample engine).  The pair plan, written on the device
// before the gather:
//   [0] E list entries, [1] Cp of them paired (the first Cp), [2] launch rows R,
//   [3] samples per row, [4] wave slots U = ceil(E / 16), [5] workgroup slots
//   Q = ceil(U / kMfma4Waves) per row, [6] the index sum S of a pair (-1: none),
//   then int2 entries (g, partner or -1): paired entries e < Cp at slot e,
//   the others at slot gcap - 1 - (e - Cp); then (16-byte aligned) each
//   group's reference voxel as a float4 (x, y, z, 0).
constexpr int kPairHeader = 16;
// resident 4-wave workgroups of the pair gather: 2 per CU on either trig path
inline constexpr int pair_resident_wgs(int) { return 2 * 256; }
inline size_t pair_list_bytes(int64_t groups) { return ((size_t)kPairHeader * 4 + (size_t)groups * 8 + 15) / 16 * 16; }
inline size_t pair_plan_bytes(int64_t groups) { return pair_list_bytes(groups) + (size_t)groups * 16; }

struct PairPlanArgs {
  const float* x; const float* y; const float* z;
  int64_t N;
  int32_t V, jref;
  int64_t G;             // groups ceil(N / V): the list's slots
  int32_t* flags;        // [ceil(G / 16)] regular waves
  int32_t* plan;         // pair plan
  float4* refs;          // [G] reference voxels (inside the pair plan buffer)
  int32_t pair;          // 0: every group alone (no partner search)
  int32_t rows_lo, rows_hi;  // the device picks the launch rows in this range
  int64_t mpad;
  int32_t resident;      // resident workgroups of the gather (pair_resident_wgs)
};

// ---------------------------------------------------------------------------
// Half-split matrix-core engine (F^H D and Q, groups of 128 / BC voxels, 16
// groups per wave as the four-sample engine): every fp32 product is formed
// from fp16 parts, x = hi + lo with hi = fp16(x) and lo = fp16(x - hi), as
// hi_a hi_b + hi_a lo_b + lo_a hi_b on v_mfma_f32_16x16x32_f16 (K = 32
// samples), accumulated in fp32.  The factors are scaled by a power of two
// 2^e that puts the largest near 2^14 (fp16 range), undone at the store.
// Records per pass: headers as the four-sample engine; factor parts per
// 32-sample block q: for tile t < 8 (16 complex columns cc = 16 t + c),
// product u < 3 (fr, fi, fr + fi) and part s < 2 (hi, lo), 64 lanes x 8 fp16
// (lane c + 16 (k / 8) holds samples 32 q + k, k = 8 (lane / 16) .. + 7) at
// wh[(((q * 8 + t) * 3 + u) * 2 + s) * 64 + lane] (16 bytes each; 1536 bytes
// per sample); Mu_b per sample in fp32 for the direct kernel; the scale pair.
constexpr int kHalfChunk = 32;    // samples per chunk: one MFMA K block (divides kMfmaChunk)
constexpr int kHalfWaves = 8;     // waves per workgroup (one workgroup per CU: 96 KB of LDS)
inline constexpr size_t half_factor_bytes(int64_t mpad) { return (size_t)mpad * 1536; }

struct HalfRecordArgs {
  MfmaRecordArgs r;      // hdr as the four-sample engine; r.wb unused
  void* wh;              // factor parts (uint4 units), see above
  float2* mu;            // [mpad][BC]
  float* scale;          // [2 + 256]: the scale pair, then per-workgroup maxima
};

// ---------------------------------------------------------------------------
// Forward operator D[b][m] = phi_m sum_n rho_b[n] exp(-i 2 pi k_m . x_n) on the
// matrix cores: waves own 32 samples, the K dimension runs over voxel groups.
// Packed image of one pass (groups g < gpad, gpad a multiple of kMfmaChunk):
//   header ghdr[g][4]: x, y, z of the group's first voxel, and 1.0 when the
//     group is not on the first group's offsets (0.0 otherwise);
//   image, per pair of groups h = g / 2 (P = T / 2 tiles of 32 complex
//     columns; complex column cc = 32 t + c holds r = rho_b[g V + j] with
//     b = cc / V, j = cc % V; zero past N and in irregular groups), 192 P floats:
//       gwb[h][p][2 P] : [t] = re, [P + t] = im;   gwb[h][128 P + p P + t] = re + im,
//     p = 32 (g % 2) + c the lane that supplies the MFMA B entry.
struct FwdArgs {
  const float* kx; const float* ky; const float* kz;
  const float* x; const float* y; const float* z;
  const float2* phi;
  const float2* rho;     // first image of this pass ([BC][N])
  int64_t M, N;
  int64_t gpad;          // padded group count
  int64_t tile;          // groups per summation tile (multiple of kMfmaChunk)
  int64_t g_split;       // groups per launch row (multiple of kMfmaChunk)
  float* ghdr;           // [gpad][4]
  float* gwb;            // [gpad / 2][192 P]
  int32_t* glist;        // [1 + groups]: count of groups off the common offsets, then their
                         // indices in increasing order
  float2* out;           // first output vector of this pass ([BC][M])
  float2* partial;       // [rows][BC][M] when rows > 1, else nullptr
  // mirror pairs (four-group engine; nullptr / 0 otherwise): the K dimension
  // runs over the pair plan's entries instead of groups; ghdr then holds each
  // entry's reference voxel and gwb its packed (rho_g + rho_h, rho_g - rho_h)
  const int32_t* pairs;  // pair plan (kPairHeader int32, int2 list, group references)
  const float4* refs;    // the plan's group references
  const int32_t* wflags; // regular waves of 16 groups (groups of the others go to glist)
  int32_t jref;          // reference column (0 without pairs)
  int64_t gcap;          // list slots (groups of the pass)
};

// Packs the image (and lists the groups off the common offsets).
hipError_t launch_fwd_pack(int T, int BC, const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_gather(int trig, int T, int BC, int32_t splits, const FwdArgs& a,
                             hipStream_t s);
// Adds the groups off the common offsets into a.out (after the rows' reduction).
hipError_t launch_fwd_direct(int trig, int T, int BC, const FwdArgs& a, hipStream_t s);

// T: units of 16 complex columns per group phase (2 or 4; T / 2 tiles of 32
// complex columns); BC: vectors of the pass.
hipError_t launch_mfma_records(int is_q, int trig, int T, int BC, const MfmaRecordArgs& a,
                               hipStream_t s);
// Mirror-pair gather of the four-sample engine (a.tile: the summation block
// in samples): pair plan kernels, the gather over the plan's list and the direct
// kernel for irregular waves, with the device's launch rows (at most
// pa.rows_hi; a.partial holds that many rows when pa.rows_hi > 1).
hipError_t launch_mfma_pair_gather(int trig, int BC, const PairPlanArgs& pa, const MfmaArgs& a, hipStream_t s);
// The pair plan alone (flags, references, list), for the forward operator.
hipError_t launch_pair_plan(int BC, const PairPlanArgs& pa, hipStream_t s);
// Forward operator with mirror pairs: packs the plan's entries (and lists the
// groups of irregular waves), then the gather over the entries.
hipError_t launch_fwd_pair_pack(int BC, const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_pair_gather(int trig, int BC, int32_t splits, const FwdArgs& a, hipStream_t s);
// Adds the device-chosen rows' partial sums (rows from the pair plan).
hipError_t launch_reduce_dev_rows(int BC, const int32_t* plan, const GatherArgs& a, hipStream_t s);
hipError_t launch_mfma_gather(int trig, int T, int BC, int32_t splits, const MfmaArgs& a,
                              hipStream_t s);
// Half-split engine: scale, records; gather (regular waves) + direct kernel.
bool half_supported(int BC);
hipError_t launch_half_records(int is_q, int trig, int BC, const HalfRecordArgs& a, hipStream_t s);
hipError_t launch_half_gather(int trig, int BC, int32_t splits, const MfmaArgs& a, hipStream_t s);
bool mfma_supported(int T, int BC);

}  // namespace ncmri
