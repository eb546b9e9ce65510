// C ABI of the F^H D / Q library: argument checks, planning, workspace and the
// two stream-ordered launches (see include/fhd.h for the contract).
#include "fhd.h"
#include "fhd_cg.h"
#include "fhd_forward_half.h"
#include "fhd_internal.h"

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#define NCMRI_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

fhd_status fail(fhd_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

fhd_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FHD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FHD_ERR_UNSUPPORTED_DEVICE, "device index %d", dev);
  int st = g_dev_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return fail(FHD_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    st = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(FHD_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
  return FHD_OK;
}

struct Range {
  const void* p;
  size_t bytes;
};

bool overlaps(Range a, Range b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes, b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
  return a0 < b1 && b0 < a1;
}

struct Plan {
  int op;              // fhd_op
  int is_q;
  int trig;
  int sum;
  int engine;          // FHD_ENGINE_VALU, FHD_ENGINE_MFMA or FHD_ENGINE_MFMA16
  int tiles;           // MFMA: 32-column factor tiles per group phase (2 or 4)
  int V;               // group size of the first pass
  int stages;
  int64_t M, N, mpad, tile;
  int32_t splits;      // launch rows splitting the samples (partial sums + reduce when > 1)
  int64_t m_split;     // samples per row
  size_t partial_bytes;
  int batch;
  int npass;           // gather passes (batch groups)
  int bc[40];          // vectors per pass (<= 31 + 4 for batch <= 512)
  size_t pass_bytes[40];
  size_t hdr_bytes;    // MFMA: header part of each pass's records (256-aligned)
  size_t flag_bytes;   // MFMA: per-wave regularity flags shared by the passes
  int64_t gpad[40];    // forward: padded group count of each pass
  int64_t g_split[40]; // forward: groups per launch row of each pass
  int pair;            // four-sample engine, HW trig, row blocks: mirror-pair gather
  int32_t rows_lo, rows_hi;  // launch rows the device picks from (pair); else both = splits
  size_t pair_bytes;   // pair plan (header + list) shared by the passes
  size_t ws_bytes;
};


// Launch-shape choices when the caller leaves them to the library; all
// measured on MI355X (256 CUs x 4 SIMDs).  Waves of one gather launch all do
// the same work, so the total wave count should be a whole number of
// "rounds" of resident waves: 3 per SIMD for the 16-voxel kernels (129-170
// VGPRs), 4 for smaller ones -- hence multiples of 1024 x lcm(3, 4) = 12288.
constexpr int64_t kSimds = 256LL * 4;
constexpr int64_t kWaveQuantum = kSimds * 12;
constexpr int64_t kMinSplitSamples = 256;  // samples per launch row at least (VALU engine)
// the matrix-core engines' rows may be shorter: when the voxels are few, more
// and shorter rows shorten each wave's serial chain of MFMAs (32^3 x 2048:
// 16 rows of 128 samples 0.032 ms per call against 0.037 with 8 of 256)
constexpr int64_t kMinSplitSamplesMfma = 128;
constexpr int32_t kMaxSplits = 1024;

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

int64_t waves_for(int64_t N, int V) { return ((N + V - 1) / V + 63) / 64; }

int32_t max_splits(int64_t mpad, int64_t min_row = kMinSplitSamples) {
  int64_t cap = mpad / min_row;
  if (cap > kMaxSplits) cap = kMaxSplits;
  return (int32_t)(cap < 1 ? 1 : cap);
}

// Voxel group: 16 voxels per lane (fastest for both trig paths at 128^3),
// unless even the most sample splits cannot give every SIMD 3 waves; then the
// largest group that can (or 1).
int auto_voxels_per_lane(int64_t N, int64_t mpad) {
  const int64_t smax = max_splits(mpad);
  for (int v = 16; v > 1; v /= 2)
    if (waves_for(N, v) * smax >= 3 * kSimds) return v;
  return 1;
}

// The MFMA gather runs 4 waves per SIMD with T = 2 (one wave per 32 voxel
// groups) and 2 with T = 4 (32 groups per wave) or T = 8 (16 groups per wave,
// the four-sample engine).
int64_t mfma_wave_quantum(int T) { return kSimds * (T == 2 ? 4 : 2); }

// Edge L of a cubic voxel count N = L^3, else 0.
int64_t cube_edge(int64_t N) {
  if (N <= 0) return 0;
  int64_t L = (int64_t)std::llround(std::cbrt((double)N));
  for (int64_t c = L > 1 ? L - 1 : 1; c <= L + 1; ++c)
    if (c * c * c == N) return c;
  return 0;
}

// Reference column of a mirror-pair pass.  On an L^3 grid with coordinates
// (i - L/2) step, x fastest: a group of V <= L voxels is a segment of a row
// and its middle column V / 2 mirrors the middle of the opposite segment of
// the mirror row (segment q of L / V onto L / V - 1 - q); a group of V = k L
// voxels is k whole rows, and the voxel x = 0 of its row k / 2, column
// V / 2 + L / 2, mirrors that of the group whose rows are mirrored in reverse
// order.  Either way every group whose rows have a mirror row is paired.
// Other voxel sets take the middle column.  Column 0 when the voxels do not
// reach the choice.
int32_t pair_jref(int64_t N, int V) {
  const int64_t L = cube_edge(N);
  int64_t j = V / 2;
  if (L > 0 && V > L && V % L == 0) j = V / 2 + L / 2;
  return N > j ? (int32_t)j : 0;
}

// Summation block of the mirror-pair gather in samples: the plan's tile,
// at most kPairBlockSamples unless the sum is plain (one running sum per row
// by definition).  A coherent sum -- Q at x = 0, the reference voxel of the
// self-mirrored group, where every product is |phi|^2 -- misses by 2e-5 in
// fp32 over one 131,072-sample block, by a few 1e-6 in blocks of 16,384.
constexpr int64_t kPairBlockSamples = 16384;
constexpr int64_t kPairAccurateTile = 2048;

int64_t pair_block(const Plan& p) {
  if (p.sum == FHD_SUM_PLAIN) return p.mpad > 0 ? p.mpad : ncmri::kMfmaChunk;
  return p.tile < kPairBlockSamples ? p.tile : kPairBlockSamples;
}

// Whether groups of V consecutive voxels (x fastest) of an L^3 grid all sit
// at the first group's offsets: V divides a row, or V is whole rows of a plane.
bool groups_regular(int64_t L, int64_t V) { return L % V == 0 || (V % L == 0 && (L * L) % V == 0); }

// Units of 16 complex columns per group phase (T).  Groups of 16 T / BC
// consecutive voxels only take the factored path when they are regular on
// the grid; more columns per phase cut the phase and sine work per MFMA but
// give fewer, longer waves, so the largest T <= tmax is chosen whose groups
// every pass keeps regular when N is a cube and, given mpad > 0, whose waves
// times the most sample rows still fill the GPU's resident-wave slots (else
// 2).  T = 8 (groups of 128 voxels for one vector) runs the four-sample
// engine.  For the forward operator (fwd_M > 0 samples; mpad unused) the
// waves own 16 or 32 samples and the launch rows split the groups, at least
// 256 groups each.
int auto_mfma_tiles(int64_t N, const int* bc, int npass, int tmax, int64_t mpad, int64_t fwd_M = 0) {
  const int64_t L = cube_edge(N);
  if (L == 0) return 2;
  for (int T = tmax; T > 2; T /= 2) {
    bool ok = true;
    for (int i = 0; i < npass; ++i) {
      const int64_t V = 16 * T / bc[i];
      if (!groups_regular(L, V)) ok = false;
    }
    int64_t capacity;  // waves x the most launch rows
    if (fwd_M > 0) {
      const int64_t per_wave = T == 8 ? 16 : 32, V = 16 * T / bc[0];
      int64_t rows = ((N + V - 1) / V) / 256;
      rows = rows < 1 ? 1 : (rows > kMaxSplits ? kMaxSplits : rows);
      capacity = (fwd_M + per_wave - 1) / per_wave * rows;
    } else {
      capacity = ncmri::mfma_gather_waves(N, T, bc[0]) * max_splits(mpad, kMinSplitSamplesMfma);
    }
    if (ok && capacity < mfma_wave_quantum(T)) ok = false;
    if (ok) return T;
  }
  return 2;
}

// Sample splits.  Rows that start at different points of the record stream
// keep the waves of a CU from all waiting on the same scalar-cache line, and
// extra rows fill the GPU when the voxel set is small.  Measured on MI355X:
// gains saturate around 16K samples per row (128^3 x 262,144: 62.9 ms with 1
// row, 54.5-54.9 ms with 12-96; Q 128^3 x 2^20: 282 ms -> 215 ms at 48 rows).
// So: enough rows for a whole quantum of waves when the voxels alone do not
// give one, and at most kSplitSamples samples per row, within a 2 GiB cap on
// the rows' partial sums.
constexpr int64_t kSplitSamples = 16384;
constexpr int64_t kMaxPartialBytes = 2LL << 30;
// Forward operator, HW path: largest row (in bytes of packed voxel groups)
// summed as one block by the kernel without running totals.
constexpr int64_t kRowBlockBytes = 256LL << 20;

int32_t auto_splits(int64_t waves, int64_t quantum, int64_t N, int BC, int64_t mpad, int64_t min_row) {
  if (waves <= 0 || mpad <= 0) return 1;
  const int32_t smax = max_splits(mpad, min_row);
  int64_t s_fill = 1;
  if (waves < quantum) {
    s_fill = (quantum + waves - 1) / waves;
    for (int32_t s = 1; s <= smax; ++s)
      if ((waves * s) % quantum == 0) { s_fill = s; break; }
  }
  int64_t s = (mpad + kSplitSamples - 1) / kSplitSamples;
  if (s < s_fill) s = s_fill;
  const int64_t row_bytes = (int64_t)BC * N * (int64_t)sizeof(fhd_c32);
  const int64_t s_mem = row_bytes > 0 ? kMaxPartialBytes / row_bytes : s;
  if (s > s_mem) s = s_mem;
  if (s > smax) s = smax;
  return (int32_t)(s < 1 ? 1 : s);
}

// Checks shared by every operation's plan.
fhd_status validate(int64_t M, int64_t N, int32_t batch, const fhd_opts* o) {
  if (M < 0 || N < 0) return fail(FHD_ERR_INVALID_ARGUMENT, "negative size (M=%lld, N=%lld)", (long long)M, (long long)N);
  if (M > 0x7fffffffLL || N > 0x7fffffffLL) return fail(FHD_ERR_INVALID_ARGUMENT, "M and N must be < 2^31");
  if (batch < 1) return fail(FHD_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", batch);
  if (batch > 16 * 32) return fail(FHD_ERR_INVALID_ARGUMENT, "batch must be <= 512 (got %d)", batch);
  if (o->trig != FHD_TRIG_ACCURATE && o->trig != FHD_TRIG_HW) return fail(FHD_ERR_INVALID_ARGUMENT, "unknown trig %d", o->trig);
  if (o->sum != FHD_SUM_BLOCKED && o->sum != FHD_SUM_KAHAN && o->sum != FHD_SUM_PLAIN) return fail(FHD_ERR_INVALID_ARGUMENT, "unknown sum %d", o->sum);
  if (o->tile < 0) return fail(FHD_ERR_INVALID_ARGUMENT, "tile must be >= 0");
  if (o->stages < 0 || o->stages > FHD_STAGE_ALL) return fail(FHD_ERR_INVALID_ARGUMENT, "unknown stages mask %d", o->stages);
  if ((o->stages & FHD_STAGE_MU) && (o->stages & FHD_STAGE_REDUCE) && !(o->stages & FHD_STAGE_GATHER))
    return fail(FHD_ERR_INVALID_ARGUMENT, "stages mask %d skips the gather between mu and reduce", o->stages);
  if (o->sample_splits < 0 || o->sample_splits > kMaxSplits)
    return fail(FHD_ERR_INVALID_ARGUMENT, "sample_splits must be in [0, %d] (got %d)", kMaxSplits, o->sample_splits);
  const int V = o->voxels_per_lane;
  if (V != 0 && V != 1 && V != 2 && V != 4 && V != 8 && V != 16 && V != 32 && V != 64 && V != 128)
    return fail(FHD_ERR_INVALID_ARGUMENT, "voxels_per_lane must be 0, 1, 2, 4, 8, 16, 32, 64 or 128 (got %d)", V);
  if (o->engine != FHD_ENGINE_AUTO && o->engine != FHD_ENGINE_VALU && o->engine != FHD_ENGINE_MFMA &&
      o->engine != FHD_ENGINE_MFMA16)
    return fail(FHD_ERR_INVALID_ARGUMENT, "unknown engine %d", o->engine);
  if (o->flags & ~FHD_FLAG_NO_MIRROR_PAIRS) return fail(FHD_ERR_INVALID_ARGUMENT, "unknown opts.flags bits 0x%x", o->flags);
  return FHD_OK;
}

fhd_status make_plan(Plan& p, int is_q, int64_t M, int64_t N, int32_t batch, const fhd_opts* o) {
  fhd_opts d;
  fhd_default_opts(&d);
  if (!o) o = &d;
  fhd_status vst = validate(M, N, batch, o);
  if (vst != FHD_OK) return vst;
  int V = o->voxels_per_lane;
  int engine = o->engine;
  if (engine == FHD_ENGINE_AUTO)
    engine = (o->sum == FHD_SUM_KAHAN || (V != 0 && V <= 16)) ? FHD_ENGINE_VALU : FHD_ENGINE_MFMA;
  if (engine == FHD_ENGINE_MFMA && o->sum == FHD_SUM_KAHAN)
    return fail(FHD_ERR_INVALID_ARGUMENT, "the MFMA engine sums blocked or plain, not Kahan");
  const bool half = engine == FHD_ENGINE_MFMA16;
  if (half && o->sum == FHD_SUM_KAHAN)
    return fail(FHD_ERR_INVALID_ARGUMENT, "the half-split engine sums blocked or plain, not Kahan");
  if (half && V != 0 && V != 128)
    return fail(FHD_ERR_INVALID_ARGUMENT, "the half-split engine takes groups of 128 voxels (got %d)", V);
  if (engine == FHD_ENGINE_MFMA && V != 0 && V < 32)
    return fail(FHD_ERR_INVALID_ARGUMENT, "MFMA group sizes are 32, 64 or 128 voxels (got %d)", V);
  if (engine == FHD_ENGINE_VALU && V > 16)
    return fail(FHD_ERR_INVALID_ARGUMENT, "VALU group sizes are 1 to 16 voxels (got %d)", V);
  const bool mfma = engine == FHD_ENGINE_MFMA || half;
  const int64_t pad = mfma ? ncmri::kMfmaChunk : ncmri::kUnroll;
  p.engine = engine;
  p.op = is_q ? FHD_OP_Q : FHD_OP_FHD;
  p.is_q = is_q;
  p.trig = o->trig;
  p.sum = o->sum;
  p.stages = o->stages == 0 ? FHD_STAGE_ALL : o->stages;
  p.M = M;
  p.N = N;
  p.batch = is_q ? 1 : batch;
  p.mpad = (M + pad - 1) / pad * pad;
  // batch groups: 16, 8, 4, 2, 1 vectors per gather pass
  p.npass = 0;
  int left = p.batch;
  for (int g = 16; g >= 1; g /= 2)
    while (left >= g) { p.bc[p.npass++] = g; left -= g; }
  p.tiles = 0;
  if (mfma) {
    p.tiles = half ? 8 : (V != 0 ? V / 16 : auto_mfma_tiles(N, p.bc, p.npass, 8, p.mpad));
    V = 16 * p.tiles / p.bc[0];  // columns of a group: voxels x vectors
  } else if (p.batch > 1) {
    V = 1;  // batched passes amortise the phase over the vectors instead of voxels
  } else if (V == 0) {
    V = auto_voxels_per_lane(N, p.mpad);
  }
  if (!mfma)
    while (V > 1 && V > N) V /= 2;  // the first group must be complete
  p.V = V;
  if (o->sum == FHD_SUM_PLAIN) {
    p.tile = p.mpad > 0 ? p.mpad : pad;
  } else if (o->tile > 0) {
    p.tile = ((int64_t)o->tile + pad - 1) / pad * pad;
  } else {
    // about sqrt(M) samples per tile; the matrix-core engine's HW-trig path
    // takes about 4 sqrt(M): its error is set by the hardware sine and the
    // fp32 phase, far above the blocked sum's, and each tile fold costs
    // (128^3 x 262,144: tile 2048 is 1 % faster than 512)
    const int64_t f = (mfma && o->trig == FHD_TRIG_HW) ? 16 : 1;
    int64_t t = 64;
    while (t * t < f * p.mpad && t < 8192) t *= 2;
    p.tile = t;
  }
  // sample splits: one launch row per split, partial sums reduced afterwards
  int32_t splits = o->sample_splits;
  if (o->sum == FHD_SUM_PLAIN) splits = 1;  // a single running sum by definition
  else if (splits == 0)
    splits = mfma ? auto_splits(ncmri::mfma_gather_waves(N, p.tiles, p.bc[0]), mfma_wave_quantum(p.tiles),
                                N, p.bc[0], p.mpad, kMinSplitSamplesMfma)
                  : auto_splits(waves_for(N, V), kWaveQuantum, N, p.bc[0], p.mpad, kMinSplitSamples);
  if (p.mpad == 0) splits = 1;
  p.m_split = p.mpad;
  if (splits > 1) {
    p.m_split = (p.mpad + splits - 1) / splits;
    p.m_split = (p.m_split + pad - 1) / pad * pad;
    splits = (int32_t)((p.mpad + p.m_split - 1) / p.m_split);  // no empty rows
  }
  p.splits = splits;
  // the four-sample engine's HW path sums each launch row as one block: no
  // tile folds, so its kernel keeps no running totals (3 waves per SIMD)
  if (mfma && p.tiles == 8 && o->trig == FHD_TRIG_HW && o->tile == 0 && p.tile < p.m_split)
    p.tile = p.m_split;
  // the half-split engine's HW path sums each launch row as one block, as
  // the four-sample engine's does; its accurate path folds tiles of ~sqrt(M)
  if (half && o->trig == FHD_TRIG_HW && o->tile == 0) p.tile = p.m_split;
  if (half && p.tile > p.m_split && p.m_split > 0) p.tile = p.m_split;
  // mirror pairs: the four-sample engine on either trig path; with automatic
  // rows the device picks between half and twice the count above (or what
  // fills every SIMD when pairing halves the waves)
  p.pair = engine == FHD_ENGINE_MFMA && p.tiles == 8 && !(o->flags & FHD_FLAG_NO_MIRROR_PAIRS);
  // the pair gather adds each block's sums into the row's outputs in memory
  // (64 KB per wave and block): the accurate path's automatic tile is
  // kPairAccurateTile there (128^3 x 262,144: 18.4 ms with blocks of 512, the
  // old ~sqrt(M) tile, 16.6 ms with blocks of 16,384; rel-L2 ~1e-6 at 2048)
  if (p.pair && o->tile == 0 && o->sum != FHD_SUM_PLAIN && o->trig == FHD_TRIG_ACCURATE && p.tile < kPairAccurateTile)
    p.tile = kPairAccurateTile;
  p.rows_lo = p.rows_hi = p.splits;
  if (p.pair && o->sample_splits == 0 && o->sum != FHD_SUM_PLAIN && p.mpad > 0) {
    // at most twice the rows, or enough for every SIMD's 3 waves when about
    // half the waves remain after pairing (plus a quarter for the device to
    // round to whole rounds)
    int64_t hi = 2 * (int64_t)p.splits;
    const int64_t half = (ncmri::mfma_gather_waves(N, p.tiles, p.bc[0]) + 1) / 2;
    const int64_t fill = (ncmri::pair_resident_wgs(o->trig == FHD_TRIG_HW ? ncmri::kTrigHw : ncmri::kTrigAccurate) *
                              ncmri::kMfma4Waves + half - 1) / half;
    if (fill + fill / 4 > hi) hi = fill + fill / 4;
    const int64_t cap = max_splits(p.mpad, kMinSplitSamplesMfma);
    const int64_t row_bytes = (int64_t)p.bc[0] * N * (int64_t)sizeof(fhd_c32);
    if (hi > cap) hi = cap;
    if (row_bytes > 0 && hi > kMaxPartialBytes / row_bytes) hi = kMaxPartialBytes / row_bytes;
    const int64_t lo = (p.splits + 1) / 2;
    p.rows_lo = (int32_t)lo;
    p.rows_hi = (int32_t)(hi > lo ? hi : lo);
  }
  p.pair_bytes = 0;
  if (p.pair) {
    int64_t g = 0;
    for (int i = 0; i < p.npass; ++i) {
      const int64_t V = 16 * p.tiles / p.bc[i], gi = (N + V - 1) / V;
      g = gi > g ? gi : g;
    }
    p.pair_bytes = align256(ncmri::pair_plan_bytes(g));
  }
  p.ws_bytes = 0;
  p.hdr_bytes = mfma ? align256((size_t)p.mpad * ncmri::mfma_header_floats(p.trig) * sizeof(float)) : 0;
  for (int i = 0; i < p.npass; ++i) {
    if (half) {
      if (!ncmri::half_supported(p.bc[i])) return fail(FHD_ERR_INTERNAL, "no half-split kernel for BC=%d", p.bc[i]);
      p.pass_bytes[i] = p.hdr_bytes + align256(ncmri::half_factor_bytes(p.mpad)) +
                        align256((size_t)p.mpad * p.bc[i] * sizeof(fhd_c32)) + align256((2 + 256) * sizeof(float));
    } else if (mfma) {
      if (!ncmri::mfma_supported(p.tiles, p.bc[i])) return fail(FHD_ERR_INTERNAL, "no MFMA kernel for T=%d BC=%d", p.tiles, p.bc[i]);
      p.pass_bytes[i] = p.hdr_bytes + (size_t)p.mpad * ncmri::mfma_factor_floats(p.tiles) * sizeof(float);
    } else {
      if (!ncmri::gather_supported(is_q, p.V, p.bc[i])) return fail(FHD_ERR_INTERNAL, "no kernel for V=%d BC=%d", p.V, p.bc[i]);
      int stride = ncmri::record_dwords(is_q, p.trig, p.V, p.bc[i]);
      p.pass_bytes[i] = (size_t)p.mpad * (size_t)stride * sizeof(float);
    }
    p.ws_bytes += align256(p.pass_bytes[i]);
  }
  // one partial-sum buffer, reused by every pass (passes run in stream order)
  p.partial_bytes = p.rows_hi > 1 ? (size_t)p.rows_hi * (size_t)p.bc[0] * (size_t)N * sizeof(fhd_c32) : 0;
  p.ws_bytes += align256(p.partial_bytes);
  // the matrix-core gather's per-wave regularity flags (the first pass has
  // the most waves: the most vectors per pass, the largest groups)
  p.flag_bytes = 0;
  if (mfma && p.npass > 0) {
    int64_t w = 0;
    for (int i = 0; i < p.npass; ++i) {
      const int64_t wi = ncmri::mfma_gather_waves(N, p.tiles, p.bc[i]);
      w = wi > w ? wi : w;
    }
    p.flag_bytes = (size_t)w * sizeof(int32_t);
  }
  p.ws_bytes += align256(p.flag_bytes);
  p.ws_bytes += p.pair_bytes;
  return FHD_OK;
}

// Forward operator: matrix-core engine only; waves own 32 samples and the
// launch rows split the voxel groups.
int64_t fwd_gpad(int64_t N, int T, int BC) {
  const int V = 16 * T / BC;
  const int64_t G = (N + V - 1) / V;
  return (G + ncmri::kMfmaChunk - 1) / ncmri::kMfmaChunk * ncmri::kMfmaChunk;
}

fhd_status make_fwd_plan(Plan& p, int64_t M, int64_t N, int32_t batch, const fhd_opts* o) {
  fhd_opts d;
  fhd_default_opts(&d);
  if (!o) o = &d;
  fhd_status vst = validate(M, N, batch, o);
  if (vst != FHD_OK) return vst;
  const int V = o->voxels_per_lane;
  if (o->engine == FHD_ENGINE_VALU)
    return fail(FHD_ERR_INVALID_ARGUMENT, "the forward operator runs on the MFMA engine only (fp32 or half-split)");
  const bool half = o->engine == FHD_ENGINE_MFMA16;
  if (o->sum == FHD_SUM_KAHAN)
    return fail(FHD_ERR_INVALID_ARGUMENT, "the forward operator sums blocked or plain, not Kahan");
  if (half && V != 0 && V != 128)
    return fail(FHD_ERR_INVALID_ARGUMENT, "the half-split engine takes groups of 128 voxels (got %d)", V);
  if (V != 0 && V < 32)
    return fail(FHD_ERR_INVALID_ARGUMENT, "MFMA group sizes are 32, 64 or 128 voxels (got %d)", V);
  const int64_t C = ncmri::kMfmaChunk;
  p.op = FHD_OP_FORWARD;
  p.is_q = 0;
  p.pair = 0;
  p.pair_bytes = 0;
  p.engine = half ? FHD_ENGINE_MFMA16 : FHD_ENGINE_MFMA;
  p.trig = o->trig;
  p.sum = o->sum;
  p.stages = o->stages == 0 ? FHD_STAGE_ALL : o->stages;
  p.M = M;
  p.N = N;
  p.batch = batch;
  p.mpad = M;
  p.npass = 0;
  int left = batch;
  for (int g = 16; g >= 1; g /= 2)
    while (left >= g) { p.bc[p.npass++] = g; left -= g; }
  p.tiles = half ? 8 : (V != 0 ? V / 16 : auto_mfma_tiles(N, p.bc, p.npass, 8, 0, M));
  p.V = 16 * p.tiles / p.bc[0];
  int64_t gmax = 0, gmin = -1;
  for (int i = 0; i < p.npass; ++i) {
    if (half && !ncmri::fwd_half_supported(p.bc[i]))
      return fail(FHD_ERR_INTERNAL, "no half-split forward kernel for BC=%d", p.bc[i]);
    if (!ncmri::mfma_supported(p.tiles, p.bc[i])) return fail(FHD_ERR_INTERNAL, "no MFMA kernel for T=%d BC=%d", p.tiles, p.bc[i]);
    p.gpad[i] = fwd_gpad(N, p.tiles, p.bc[i]);
    if (p.gpad[i] > gmax) gmax = p.gpad[i];
    if (gmin < 0 || p.gpad[i] < gmin) gmin = p.gpad[i];
  }
  // summation tile in groups
  if (o->sum == FHD_SUM_PLAIN) {
    p.tile = gmax > 0 ? gmax : C;
  } else if (o->tile > 0) {
    p.tile = ((int64_t)o->tile + C - 1) / C * C;
  } else {
    // about sqrt(G) groups per tile, about 4 sqrt(G) on the HW-trig path (as
    // for the adjoint: 128^3, tile 512 is 2.5 % faster than 128)
    const int64_t f = o->trig == FHD_TRIG_HW ? 16 : 1;
    int64_t t = 64;
    while (t * t < f * gmax && t < 8192) t *= 2;
    p.tile = t;
  }
  // launch rows over the groups: enough for whole rounds of resident waves
  // when the samples alone give fewer; at least 64 groups per row (32^3 x
  // 2048: 16 rows 0.034 / 0.035 ms HW / accurate against 0.042 / 0.051 with
  // the 4 rows of 256 groups)
  int32_t splits = o->sample_splits;
  const int64_t waves = p.tiles == 8 ? (M + 15) / 16 : (M + 31) / 32;  // samples per wave
  if (o->sum == FHD_SUM_PLAIN) {
    splits = 1;
  } else if (splits == 0) {
    const int64_t quantum = mfma_wave_quantum(p.tiles);
    int64_t smax = gmin / 64;
    if (smax > kMaxSplits) smax = kMaxSplits;
    if (smax < 1) smax = 1;
    int64_t s = 1;
    if (waves > 0 && waves < quantum) {
      s = (quantum + waves - 1) / waves;
      for (int64_t c = 1; c <= smax; ++c)
        if ((waves * c) % quantum == 0) { s = c; break; }
    }
    const int64_t row_bytes = (int64_t)p.bc[0] * M * (int64_t)sizeof(fhd_c32);
    if (row_bytes > 0 && s > kMaxPartialBytes / row_bytes) s = kMaxPartialBytes / row_bytes;
    if (s > smax) s = smax;
    splits = (int32_t)(s < 1 ? 1 : s);
  }
  if (gmax == 0 || M == 0) splits = 1;
  p.splits = splits;
  p.rows_lo = p.rows_hi = splits;
  for (int i = 0; i < p.npass; ++i) {
    int64_t gs = (p.gpad[i] + splits - 1) / splits;
    gs = (gs + C - 1) / C * C;
    p.g_split[i] = gs > 0 ? gs : C;
  }
  // the four-group engine's HW path sums each launch row as one block: no
  // tile folds, so its kernel keeps no running totals (3 waves per SIMD).
  // Every wave streams its row's packed groups, so this is kept to rows of at
  // most kRowBlockBytes of packed groups: measured, 128^3 (25 MB per row) and
  // the 16-image 96^3 pass (170 MB) gain from it, while at 512^3 (1.6 GB) the
  // three resident workgroups per CU were 1.2 % slower than two with tiles.
  if (p.tiles == 8 && o->trig == FHD_TRIG_HW && o->tile == 0 && o->sum != FHD_SUM_PLAIN) {
    int64_t gs = 0;
    for (int i = 0; i < p.npass; ++i) gs = p.g_split[i] > gs ? p.g_split[i] : gs;
    const int64_t row_bytes = gs * ncmri::mfma_factor_floats(p.tiles) * (int64_t)sizeof(float);
    if (row_bytes <= kRowBlockBytes && gs > p.tile) p.tile = gs;
  }
  // the half-split engine's HW path likewise sums rows of at most
  // kRowBlockBytes of packed groups as one block (its kernel keeps no running
  // totals either way: one resident workgroup of eight waves per CU); longer
  // rows fold tiles, which keeps its error at 512^3 at the fp32 engine's
  if (half && o->trig == FHD_TRIG_HW && o->tile == 0 && o->sum != FHD_SUM_PLAIN) {
    int64_t gs = 0;
    for (int i = 0; i < p.npass; ++i) gs = p.g_split[i] > gs ? p.g_split[i] : gs;
    const int64_t row_bytes = gs * ncmri::mfma_factor_floats(p.tiles) * (int64_t)sizeof(float);
    if (row_bytes <= kRowBlockBytes && gs > p.tile) p.tile = gs;
  }
  // mirror pairs (the fp32 four-group engine): the K dimension runs over the
  // pair plan's entries; each launch row is one summation block of at most
  // kPairBlockSamples entries (HW) or kPairAccurateTile (accurate), or the
  // caller's tile, through the rows' partial sums (the pair gather keeps no
  // running totals); sample_splits, if given, is the row count
  p.pair = !half && p.tiles == 8 && !(o->flags & FHD_FLAG_NO_MIRROR_PAIRS);
  if (p.pair && gmax > 0 && M > 0 && o->sum != FHD_SUM_PLAIN && o->sample_splits == 0) {
    const int64_t block = o->tile > 0 ? p.tile : (o->trig == FHD_TRIG_HW ? kPairBlockSamples : kPairAccurateTile);
    int64_t G = 0;
    for (int i = 0; i < p.npass; ++i) {
      const int64_t Vi = 16 * p.tiles / p.bc[i], gi = (N + Vi - 1) / Vi;
      G = gi > G ? gi : G;
    }
    int64_t rows = (G + block - 1) / block;
    if (rows < p.splits) rows = p.splits;
    const int64_t row_bytes = (int64_t)p.bc[0] * M * (int64_t)sizeof(fhd_c32);
    if (row_bytes > 0 && rows > kMaxPartialBytes / row_bytes) rows = kMaxPartialBytes / row_bytes;
    if (rows > kMaxSplits) rows = kMaxSplits;
    if (rows < 1) rows = 1;
    p.splits = (int32_t)rows;
    p.tile = block;
  }
  p.rows_lo = p.rows_hi = p.splits;
  p.pair_bytes = 0;
  p.m_split = 0;
  p.hdr_bytes = 0;
  p.ws_bytes = 0;
  for (int i = 0; i < p.npass; ++i) {
    if (p.pair && p.gpad[i] > 0) {
      // entry headers [gpad][4], entries [gpad][64 T] (ur, ui, wi, wr), list of
      // groups of irregular waves [1 + gpad], wave flags, the pair plan
      const int64_t Vi = 16 * p.tiles / p.bc[i], Gi = (N + Vi - 1) / Vi;
      p.pass_bytes[i] = align256((size_t)p.gpad[i] * 4 * sizeof(float)) +
                        align256((size_t)p.gpad[i] * 64 * p.tiles * sizeof(float)) +
                        align256((size_t)(p.gpad[i] + 1) * sizeof(int32_t)) +
                        align256((size_t)((Gi + 15) / 16) * sizeof(int32_t)) + ncmri::pair_plan_bytes(Gi);
      p.ws_bytes += align256(p.pass_bytes[i]);
      continue;
    }
    // header [gpad][4], image [gpad][48 T], list of flagged groups [1 + gpad] int32
    p.pass_bytes[i] = p.gpad[i] == 0 ? 0
                      : align256((size_t)p.gpad[i] * 4 * sizeof(float)) +
                            align256((size_t)p.gpad[i] * ncmri::mfma_factor_floats(p.tiles) * sizeof(float)) +
                            (size_t)(p.gpad[i] + 1) * sizeof(int32_t);
    // half-split: the fp16 parts of the packed image and its scale
    if (half && p.gpad[i] > 0)
      p.pass_bytes[i] = align256(p.pass_bytes[i]) + align256(ncmri::fwd_half_parts_bytes(p.gpad[i])) +
                        align256(ncmri::fwd_half_header_bytes(p.gpad[i])) +
                        align256(ncmri::kFwdHalfScaleFloats * sizeof(float));
    p.ws_bytes += align256(p.pass_bytes[i]);
  }
  p.partial_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)p.bc[0] * (size_t)M * sizeof(fhd_c32) : 0;
  p.ws_bytes += align256(p.partial_bytes);
  return FHD_OK;
}

fhd_status make_any_plan(Plan& p, int op, int64_t M, int64_t N, int32_t batch, const fhd_opts* o) {
  if (op == FHD_OP_FORWARD) return make_fwd_plan(p, M, N, batch, o);
  if (op == FHD_OP_FHD || op == FHD_OP_Q) return make_plan(p, op == FHD_OP_Q ? 1 : 0, M, N, batch, o);
  return fail(FHD_ERR_INVALID_ARGUMENT, "unknown operation %d", op);
}

// Workspace handling shared by the operations: the caller's buffer (checked)
// or a stream-ordered allocation.
struct Workspace {
  void* ptr = nullptr;
  bool own = false;
};

fhd_status acquire_workspace(const Plan& p, const fhd_opts* opts, const Range* ins, int nins,
                             Range outr, hipStream_t s, Workspace& w) {
  void* ws = opts ? opts->workspace : nullptr;
  const size_t ws_given = opts ? opts->workspace_bytes : 0;
  if (ws) {
    if ((uintptr_t)ws % 16 != 0)
      return fail(FHD_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    if (ws_given < p.ws_bytes)
      return fail(FHD_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_given, p.ws_bytes);
    Range wr{ws, ws_given};
    if (overlaps(wr, outr)) return fail(FHD_ERR_INVALID_ARGUMENT, "workspace overlaps the output");
    for (int i = 0; i < nins; ++i)
      if (overlaps(wr, ins[i])) return fail(FHD_ERR_INVALID_ARGUMENT, "workspace overlaps an input array");
  } else if (p.stages != FHD_STAGE_ALL && p.ws_bytes > 0) {
    return fail(FHD_ERR_WORKSPACE, "running stages separately needs a caller workspace");
  }
  if (p.npass > 1 && p.splits > 1 &&
      ((p.stages & FHD_STAGE_GATHER) != 0) != ((p.stages & FHD_STAGE_REDUCE) != 0))
    return fail(FHD_ERR_INVALID_ARGUMENT,
                "batch passes share the partial-sum buffer: run GATHER and REDUCE in the same call");
  w.ptr = ws;
  w.own = false;
  return FHD_OK;
}

fhd_status run_forward(const float* kx, const float* ky, const float* kz, const float* x,
                       const float* y, const float* z, const fhd_c32* phi, const fhd_c32* rho,
                       fhd_c32* out, int64_t M, int64_t N, int32_t batch, const fhd_opts* opts,
                       void* stream) {
  g_err[0] = '\0';
  Plan p;
  fhd_status st = make_fwd_plan(p, M, N, batch, opts);
  if (st != FHD_OK) return st;
  const size_t fm = (size_t)M * sizeof(float), cm = (size_t)M * sizeof(fhd_c32);
  const size_t fn = (size_t)N * sizeof(float), cn = (size_t)N * sizeof(fhd_c32);
  const size_t outb = (size_t)M * (size_t)batch * sizeof(fhd_c32);
  if (M > 0 && (!kx || !ky || !kz || !phi || !out))
    return fail(FHD_ERR_INVALID_ARGUMENT, "null sample or output array with M=%lld", (long long)M);
  if (N > 0 && (!x || !y || !z || !rho))
    return fail(FHD_ERR_INVALID_ARGUMENT, "null voxel or image array with N=%lld", (long long)N);
  Range outr{out, outb};
  Range ins[] = {{kx, fm}, {ky, fm}, {kz, fm}, {x, fn}, {y, fn}, {z, fn}, {phi, cm},
                 {rho, cn * (size_t)batch}};
  for (const Range& r : ins)
    if (overlaps(outr, r)) return fail(FHD_ERR_INVALID_ARGUMENT, "output overlaps an input array");
  hipStream_t s = (hipStream_t)stream;
  Workspace w;
  st = acquire_workspace(p, opts, ins, 8, outr, s, w);
  if (st != FHD_OK) return st;
  if (M == 0) return FHD_OK;
  st = check_device();
  if (st != FHD_OK) return st;
  if (!w.ptr && p.ws_bytes > 0) {
    hipError_t e = hipMallocAsync(&w.ptr, p.ws_bytes, s);
    if (e != hipSuccess) return fail(FHD_ERR_HIP, "hipMallocAsync(%zu): %s", p.ws_bytes, hipGetErrorString(e));
    w.own = true;
  }
  fhd_status result = FHD_OK;
  char* base = (char*)w.ptr;
  float2* partial = nullptr;
  if (p.partial_bytes > 0) {
    size_t recs = 0;
    for (int i = 0; i < p.npass; ++i) recs += align256(p.pass_bytes[i]);
    partial = (float2*)(base + recs);
  }
  int b0 = 0;
  for (int i = 0; i < p.npass && result == FHD_OK; ++i) {
    const int bc = p.bc[i];
    const size_t hb = align256((size_t)p.gpad[i] * 4 * sizeof(float));
    const size_t ib = align256((size_t)p.gpad[i] * ncmri::mfma_factor_floats(p.tiles) * sizeof(float));
    ncmri::FwdArgs fa{kx, ky, kz, x, y, z, (const float2*)phi,
                      (const float2*)(rho ? rho + (int64_t)b0 * N : nullptr), M, N, p.gpad[i], p.tile,
                      p.g_split[i], (float*)base, (float*)(base + hb),
                      p.gpad[i] > 0 ? (int32_t*)(base + hb + ib) : nullptr,
                      (float2*)(out + (int64_t)b0 * M), p.splits > 1 ? partial : nullptr};
    const bool half = p.engine == FHD_ENGINE_MFMA16;
    ncmri::FwdHalfArgs ha{fa, nullptr, nullptr, nullptr};
    if (half && p.gpad[i] > 0) {
      const size_t lb = align256(hb + ib + (size_t)(p.gpad[i] + 1) * sizeof(int32_t));
      const size_t pb = align256(ncmri::fwd_half_parts_bytes(p.gpad[i]));
      ha.wh = base + lb;
      ha.hh = (float4*)(base + lb + pb);
      ha.scale = (float*)(base + lb + pb + align256(ncmri::fwd_half_header_bytes(p.gpad[i])));
    }
    hipError_t e = hipSuccess;
    const char* what = "pack";
    ncmri::PairPlanArgs pa{};
    if (p.pair && p.gpad[i] > 0) {
      const int Vp = 16 * p.tiles / bc;
      const int64_t Gi = (N + Vp - 1) / Vp;
      const size_t hb2 = align256((size_t)p.gpad[i] * 4 * sizeof(float));
      const size_t ib2 = align256((size_t)p.gpad[i] * 64 * p.tiles * sizeof(float));
      const size_t lb2 = align256((size_t)(p.gpad[i] + 1) * sizeof(int32_t));
      int32_t* wflags = (int32_t*)(base + hb2 + ib2 + lb2);
      int32_t* plan = (int32_t*)((char*)wflags + align256((size_t)((Gi + 15) / 16) * sizeof(int32_t)));
      const int32_t jref = pair_jref(N, Vp);
      pa = ncmri::PairPlanArgs{x, y, z, N, Vp, jref, Gi, wflags, plan,
                               (float4*)((char*)plan + ncmri::pair_list_bytes(Gi)), 1, 1, 1, 0,
                               ncmri::pair_resident_wgs(ncmri::kTrigHw)};
      fa.gwb = (float*)(base + hb2);
      fa.glist = (int32_t*)(base + hb2 + ib2);
      fa.pairs = plan;
      fa.refs = pa.refs;
      fa.wflags = wflags;
      fa.jref = jref;
      fa.gcap = Gi;
    }
    if (p.stages & FHD_STAGE_MU) {
      if (p.pair && p.gpad[i] > 0) {
        e = ncmri::launch_pair_plan(bc, pa, s);
        if (e == hipSuccess) e = ncmri::launch_fwd_pair_pack(bc, fa, s);
      } else {
        e = ncmri::launch_fwd_pack(p.tiles, bc, fa, s);
      }
      if (e == hipSuccess && half && p.gpad[i] > 0) e = ncmri::launch_fwd_half_pack(bc, ha, s);
    }
    if (e == hipSuccess && (p.stages & FHD_STAGE_GATHER)) {
      what = "gather";
      e = half && p.gpad[i] > 0  ? ncmri::launch_fwd_half_gather(p.trig, bc, p.splits, ha, s)
          : p.pair && p.gpad[i] > 0 ? ncmri::launch_fwd_pair_gather(p.trig, bc, p.splits, fa, s)
                                    : ncmri::launch_fwd_gather(p.trig, p.tiles, bc, p.splits, fa, s);
    }
    if (e == hipSuccess && (p.stages & FHD_STAGE_REDUCE)) {
      what = "reduce";
      // the rows' partial sums -> output ([BC][M] values), then the groups
      // off the common offsets are added
      ncmri::GatherArgs ga{nullptr, 0, p.tile, x, y, z, M, fa.out, 0, fa.partial};
      e = ncmri::launch_reduce(bc, false, p.splits, ga, s);
      if (e == hipSuccess) e = ncmri::launch_fwd_direct(p.trig, p.tiles, bc, fa, s);
    }
    if (e != hipSuccess) result = fail(FHD_ERR_HIP, "forward %s kernel launch: %s", what, hipGetErrorString(e));
    base += align256(p.pass_bytes[i]);
    b0 += bc;
  }
  if (w.own) {
    hipError_t e = hipFreeAsync(w.ptr, s);
    if (e != hipSuccess && result == FHD_OK) result = fail(FHD_ERR_HIP, "hipFreeAsync: %s", hipGetErrorString(e));
  }
  return result;
}

// ---------------------------------------------------------------------------
// Allocation-free F^H D: the workspace is a fixed device array of the library
// (one copy per GPU, held until the process ends).  In host code the array's
// name is only a registration handle; its device address is taken once per
// device with hipGetSymbolAddress and only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = FHD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

fhd_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FHD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FHD_ERR_UNSUPPORTED_DEVICE, "device index %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(FHD_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FHD_OK;
}

fhd_status run(int is_q, const float* kx, const float* ky, const float* kz, const float* x,
               const float* y, const float* z, const fhd_c32* phi, const fhd_c32* D, fhd_c32* out,
               int64_t M, int64_t N, int32_t batch, const fhd_opts* opts, void* stream,
               bool lib_scratch = false) {
  g_err[0] = '\0';
  Plan p;
  fhd_status st = make_plan(p, is_q, M, N, batch, opts);
  if (st != FHD_OK) return st;
  const size_t fm = (size_t)M * sizeof(float), cm = (size_t)M * sizeof(fhd_c32);
  const size_t fn = (size_t)N * sizeof(float);
  const size_t outb = (size_t)N * (size_t)p.batch * sizeof(fhd_c32);
  if (M > 0 && (!kx || !ky || !kz || !phi || (!is_q && !D)))
    return fail(FHD_ERR_INVALID_ARGUMENT, "null sample array with M=%lld", (long long)M);
  if (N > 0 && (!x || !y || !z || !out))
    return fail(FHD_ERR_INVALID_ARGUMENT, "null voxel or output array with N=%lld", (long long)N);
  void* ws = opts ? opts->workspace : nullptr;
  const size_t ws_given = opts ? opts->workspace_bytes : 0;
  Range outr{out, outb};
  Range ins[] = {{kx, fm}, {ky, fm}, {kz, fm}, {x, fn}, {y, fn}, {z, fn}, {phi, cm},
                 {is_q ? nullptr : D, cm * (size_t)p.batch}};
  for (const Range& r : ins)
    if (overlaps(outr, r)) return fail(FHD_ERR_INVALID_ARGUMENT, "output overlaps an input array");
  if (ws) {
    if ((uintptr_t)ws % 16 != 0)
      return fail(FHD_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    if (ws_given < p.ws_bytes)
      return fail(FHD_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_given, p.ws_bytes);
    Range wr{ws, ws_given};
    if (overlaps(wr, outr)) return fail(FHD_ERR_INVALID_ARGUMENT, "workspace overlaps the output");
    for (const Range& r : ins)
      if (overlaps(wr, r)) return fail(FHD_ERR_INVALID_ARGUMENT, "workspace overlaps an input array");
  } else if (p.stages != FHD_STAGE_ALL && p.ws_bytes > 0) {
    return fail(FHD_ERR_WORKSPACE, "running stages separately needs a caller workspace");
  }
  if (p.npass > 1 && p.rows_hi > 1 &&
      ((p.stages & FHD_STAGE_GATHER) != 0) != ((p.stages & FHD_STAGE_REDUCE) != 0))
    return fail(FHD_ERR_INVALID_ARGUMENT,
                "batch passes share the partial-sum buffer: run GATHER and REDUCE in the same call");
  if (N == 0) return FHD_OK;
  st = check_device();
  if (st != FHD_OK) return st;

  hipStream_t s = (hipStream_t)stream;
  bool own = false;
  if (lib_scratch) {  // the allocation-free entry point: the library's fixed array
    st = scratch_for_current_device(&ws);
    if (st != FHD_OK) return st;
  } else if (!ws && p.ws_bytes > 0) {
    hipError_t e = hipMallocAsync(&ws, p.ws_bytes, s);
    if (e != hipSuccess) return fail(FHD_ERR_HIP, "hipMallocAsync(%zu): %s", p.ws_bytes, hipGetErrorString(e));
    own = true;
  }
  fhd_status result = FHD_OK;
  char* base = (char*)ws;
  float2* partial = nullptr;
  int32_t* flags = nullptr;
  int32_t* pairplan = nullptr;
  {
    size_t recs = 0;
    for (int i = 0; i < p.npass; ++i) recs += align256(p.pass_bytes[i]);
    if (p.partial_bytes > 0) partial = (float2*)(base + recs);
    if (p.flag_bytes > 0) flags = (int32_t*)(base + recs + align256(p.partial_bytes));
    if (p.pair_bytes > 0) pairplan = (int32_t*)(base + recs + align256(p.partial_bytes) + align256(p.flag_bytes));
  }
  int b0 = 0;
  const bool kahan = p.sum == FHD_SUM_KAHAN;
  for (int i = 0; i < p.npass && result == FHD_OK; ++i) {
    const int bc = p.bc[i];
    const fhd_c32* Dp = is_q ? nullptr : D + (int64_t)b0 * M;
    float2* outp = (float2*)(out + (int64_t)b0 * N);
    // the reduction only needs the output, partial buffer and sizes
    ncmri::GatherArgs ga{nullptr, p.mpad, p.tile, x, y, z, N, outp, p.m_split,
                         p.rows_hi > 1 ? partial : nullptr};
    const int Vp = p.pair ? 16 * p.tiles / bc : 0;
    const int32_t jref = p.pair ? pair_jref(N, Vp) : 0;
    hipError_t e = hipSuccess;
    const char* what = "records";
    if (p.engine == FHD_ENGINE_MFMA16) {
      float* hdr = (float*)base;
      char* wh = base + p.hdr_bytes;
      float2* mu = (float2*)(wh + align256(ncmri::half_factor_bytes(p.mpad)));
      float* scale = (float*)((char*)mu + align256((size_t)p.mpad * bc * sizeof(fhd_c32)));
      if (p.stages & FHD_STAGE_MU) {
        ncmri::HalfRecordArgs ha{{kx, ky, kz, x, y, z, (const float2*)phi, (const float2*)Dp, M, N, p.mpad, hdr,
                                  nullptr},
                                 wh, mu, scale};
        e = ncmri::launch_half_records(is_q, p.trig, bc, ha, s);
      }
      if (e == hipSuccess && (p.stages & FHD_STAGE_GATHER)) {
        what = "gather";
        ncmri::MfmaArgs ma{hdr, (const float*)wh, p.mpad, p.tile, x, y, z, N, outp, p.m_split,
                           p.splits > 1 ? partial : nullptr, flags, mu, scale};
        e = ncmri::launch_half_gather(p.trig, bc, p.splits, ma, s);
      }
    } else if (p.engine == FHD_ENGINE_MFMA) {
      float* hdr = (float*)base;
      float* wb = (float*)(base + p.hdr_bytes);
      if (p.stages & FHD_STAGE_MU) {
        ncmri::MfmaRecordArgs ra{kx, ky, kz, x, y, z, (const float2*)phi, (const float2*)Dp,
                                 M, N, p.mpad, hdr, wb, jref};
        e = ncmri::launch_mfma_records(is_q, p.trig, p.tiles, bc, ra, s);
      }
      if (e == hipSuccess && (p.stages & FHD_STAGE_GATHER)) {
        what = "gather";
        if (p.pair) {
          const int64_t G = (N + Vp - 1) / Vp;
          float4* refs = (float4*)((char*)pairplan + ncmri::pair_list_bytes(G));
          ncmri::PairPlanArgs pa{x, y, z, N, Vp, jref, G, flags, pairplan, refs, 1, p.rows_lo, p.rows_hi, p.mpad,
                                 ncmri::pair_resident_wgs(p.trig == FHD_TRIG_HW ? ncmri::kTrigHw : ncmri::kTrigAccurate)};
          ncmri::MfmaArgs ma{hdr, wb, p.mpad, pair_block(p), x, y, z, N, outp, p.m_split,
                             p.rows_hi > 1 ? partial : nullptr, flags, nullptr, nullptr, pairplan, jref, G};
          e = ncmri::launch_mfma_pair_gather(p.trig == FHD_TRIG_HW ? ncmri::kTrigHw : ncmri::kTrigAccurate, bc, pa,
                                             ma, s);
        } else {
          ncmri::MfmaArgs ma{hdr, wb, p.mpad, p.tile, x, y, z, N, outp, p.m_split,
                             p.splits > 1 ? partial : nullptr, flags};
          e = ncmri::launch_mfma_gather(p.trig, p.tiles, bc, p.splits, ma, s);
        }
      }
    } else {
      ncmri::Layout L{is_q, p.trig, p.V, bc, ncmri::header_dwords(p.trig),
                      ncmri::record_dwords(is_q, p.trig, p.V, bc)};
      float* rec = (float*)base;
      ga.rec = rec;
      if (p.stages & FHD_STAGE_MU) {
        ncmri::RecordArgs ra{kx, ky, kz, x, y, z, (const float2*)phi, (const float2*)Dp, M, p.mpad, rec};
        e = ncmri::launch_records(L, ra, s);
      }
      if (e == hipSuccess && (p.stages & FHD_STAGE_GATHER)) {
        what = "gather";
        e = ncmri::launch_gather(L, kahan, p.splits, ga, s);
      }
    }
    if (e == hipSuccess && (p.stages & FHD_STAGE_REDUCE)) {
      what = "reduce";
      e = p.pair ? ncmri::launch_reduce_dev_rows(bc, pairplan, ga, s)
                 : ncmri::launch_reduce(bc, kahan, p.splits, ga, s);
    }
    if (e != hipSuccess) result = fail(FHD_ERR_HIP, "%s kernel launch: %s", what, hipGetErrorString(e));
    base += align256(p.pass_bytes[i]);
    b0 += bc;
  }
  if (own) {
    hipError_t e = hipFreeAsync(ws, s);
    if (e != hipSuccess && result == FHD_OK) result = fail(FHD_ERR_HIP, "hipFreeAsync: %s", hipGetErrorString(e));
  }
  return result;
}

fhd_status run_noalloc(const float* kx, const float* ky, const float* kz, const float* x,
                       const float* y, const float* z, const fhd_c32* phi, const fhd_c32* D,
                       fhd_c32* out, int64_t M, int64_t N, int32_t batch, const fhd_opts* opts,
                       void* stream) {
  g_err[0] = '\0';
  fhd_opts o;
  if (opts) o = *opts;
  else fhd_default_opts(&o);
  if (o.workspace || o.workspace_bytes)
    return fail(FHD_ERR_INVALID_ARGUMENT, "fhd_compute_noalloc uses the library's scratch; opts.workspace must be NULL");
  if (o.stages != 0 && o.stages != FHD_STAGE_ALL)
    return fail(FHD_ERR_INVALID_ARGUMENT, "fhd_compute_noalloc runs all stages in one call");
  Plan p;
  fhd_status st = make_plan(p, 0, M, N, batch, &o);
  if (st != FHD_OK) return st;
  // an automatic row count is lowered until the rows' partial sums fit beside
  // the records (fewer rows: the same sums in a different order)
  if (o.sample_splits == 0 && p.ws_bytes > kNoAllocScratchBytes) {
    for (int32_t s = p.splits - 1; s >= 1 && p.ws_bytes > kNoAllocScratchBytes; --s) {
      o.sample_splits = s;
      st = make_plan(p, 0, M, N, batch, &o);
      if (st != FHD_OK) return st;
    }
  }
  if (p.ws_bytes > kNoAllocScratchBytes)
    return fail(FHD_ERR_WORKSPACE,
                "this plan needs %zu bytes of workspace; fhd_compute_noalloc holds at most %zu "
                "(fewer sample_splits, a smaller group or fewer samples per call fit in less)",
                p.ws_bytes, kNoAllocScratchBytes);
  return run(0, kx, ky, kz, x, y, z, phi, D, out, M, N, batch, &o, stream, true);
}

}  // namespace

NCMRI_API void fhd_default_opts(fhd_opts* o) {
  if (!o) return;
  std::memset(o, 0, sizeof(*o));
  o->trig = FHD_TRIG_ACCURATE;
  o->sum = FHD_SUM_BLOCKED;
  o->stages = FHD_STAGE_ALL;
  o->engine = FHD_ENGINE_AUTO;
}

NCMRI_API size_t fhd_workspace_bytes(int64_t M, int64_t N, int32_t batch, int32_t op,
                                     const fhd_opts* opts) {
  try {
    Plan p;
    if (make_any_plan(p, op, M, N, batch, opts) != FHD_OK) return 0;
    return p.ws_bytes;
  } catch (...) {
    return 0;
  }
}

NCMRI_API fhd_status fhd_describe_plan(int64_t M, int64_t N, int32_t batch, int32_t op,
                                       const fhd_opts* opts, fhd_plan_info* info) {
  try {
    g_err[0] = '\0';
    if (!info) return fail(FHD_ERR_INVALID_ARGUMENT, "info is NULL");
    Plan p;
    fhd_status st = make_any_plan(p, op, M, N, batch, opts);
    if (st != FHD_OK) return st;
    info->voxels_per_lane = p.V;
    info->tile = (int32_t)p.tile;
    info->passes = p.npass;
    info->record_dwords = p.npass == 0 ? 0
                          : p.op == FHD_OP_FORWARD ? 4 + ncmri::mfma_factor_floats(p.tiles)
                          : p.engine == FHD_ENGINE_MFMA ? ncmri::mfma_record_dwords(p.trig, p.tiles)
                          : p.engine == FHD_ENGINE_MFMA16 ? ncmri::mfma_header_floats(p.trig) + 384 + 2 * p.bc[0]
                                                         : ncmri::record_dwords(p.is_q, p.trig, p.V, p.bc[0]);
    info->padded_samples = p.mpad;
    info->workspace_bytes = p.ws_bytes;
    info->sample_splits = p.splits;
    info->engine = p.engine;
    info->mirror_pairs = p.pair;
    info->max_sample_splits = p.rows_hi;
    return FHD_OK;
  } catch (...) {
    return fail(FHD_ERR_INTERNAL, "unexpected C++ exception");
  }
}

NCMRI_API fhd_status fhd_compute(const float* kx, const float* ky, const float* kz, const float* x,
                                 const float* y, const float* z, const fhd_c32* phi,
                                 const fhd_c32* D, fhd_c32* FhD, int64_t M, int64_t N,
                                 int32_t batch, const fhd_opts* opts, void* stream) {
  try {
    return run(0, kx, ky, kz, x, y, z, phi, D, FhD, M, N, batch, opts, stream);
  } catch (...) {
    return fail(FHD_ERR_INTERNAL, "unexpected C++ exception");
  }
}

NCMRI_API fhd_status fhd_compute_noalloc(const float* kx, const float* ky, const float* kz,
                                         const float* x, const float* y, const float* z,
                                         const fhd_c32* phi, const fhd_c32* D, fhd_c32* FhD,
                                         int64_t M, int64_t N, int32_t batch, const fhd_opts* opts,
                                         void* stream) {
  try {
    return run_noalloc(kx, ky, kz, x, y, z, phi, D, FhD, M, N, batch, opts, stream);
  } catch (...) {
    return fail(FHD_ERR_INTERNAL, "unexpected C++ exception");
  }
}

NCMRI_API fhd_status fhd_forward(const float* kx, const float* ky, const float* kz, const float* x,
                                 const float* y, const float* z, const fhd_c32* phi,
                                 const fhd_c32* rho, fhd_c32* D, int64_t M, int64_t N,
                                 int32_t batch, const fhd_opts* opts, void* stream) {
  try {
    return run_forward(kx, ky, kz, x, y, z, phi, rho, D, M, N, batch, opts, stream);
  } catch (...) {
    return fail(FHD_ERR_INTERNAL, "unexpected C++ exception");
  }
}

// ---------------------------------------------------------------------------
// Reconstruction: Toeplitz kernel, normal operator, conjugate gradient.
namespace {

bool grid_ok(int32_t nx, int32_t ny, int32_t nz) {
  if (nx < 1 || ny < 1 || nz < 1) return false;
  if (nx > ncmri::kToeplitzMaxLen / 2 || ny > ncmri::kToeplitzMaxLen / 2 || nz > ncmri::kToeplitzMaxLen / 2)
    return false;
  const ncmri::ToeplitzDims d = ncmri::toeplitz_dims(nx, ny, nz);
  return (int64_t)8 * d.voxels() <= 0x7fffffffLL && d.spectrum() <= 0x7fffffffLL;
}

fhd_status check_grid(int32_t nx, int32_t ny, int32_t nz) {
  if (nx < 1 || ny < 1 || nz < 1)
    return fail(FHD_ERR_INVALID_ARGUMENT, "grid sizes must be >= 1 (got %d x %d x %d)", nx, ny, nz);
  if (!grid_ok(nx, ny, nz))
    return fail(FHD_ERR_INVALID_ARGUMENT, "grid %d x %d x %d too large: at most %d voxels per axis and "
                "8 nx ny nz < 2^31", nx, ny, nz, ncmri::kToeplitzMaxLen / 2);
  return FHD_OK;
}

fhd_status check_cg_ws(const ncmri::ToeplitzDims& d, void* ws, size_t bytes) {
  if (!ws) return fail(FHD_ERR_WORKSPACE, "a workspace of fhd_cg_workspace_bytes() bytes is required");
  if ((uintptr_t)ws % 16 != 0) return fail(FHD_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  const size_t need = ncmri::cg_workspace_bytes(d);
  if (bytes < need) return fail(FHD_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", bytes, need);
  return FHD_OK;
}

}  // namespace

NCMRI_API size_t fhd_toeplitz_bytes(int32_t nx, int32_t ny, int32_t nz) {
  if (!grid_ok(nx, ny, nz)) return 0;
  return (size_t)ncmri::toeplitz_dims(nx, ny, nz).spectrum() * sizeof(float);
}

NCMRI_API size_t fhd_cg_workspace_bytes(int32_t nx, int32_t ny, int32_t nz) {
  if (!grid_ok(nx, ny, nz)) return 0;
  return ncmri::cg_workspace_bytes(ncmri::toeplitz_dims(nx, ny, nz));
}

NCMRI_API fhd_status fhd_toeplitz_kernel(const float* kx, const float* ky, const float* kz,
                                         const fhd_c32* phi, int64_t M, int32_t nx, int32_t ny,
                                         int32_t nz, float* Qhat, const fhd_opts* opts,
                                         void* stream) {
  try {
    g_err[0] = '\0';
    fhd_status st = check_grid(nx, ny, nz);
    if (st != FHD_OK) return st;
    if (M < 0 || M > 0x7fffffffLL) return fail(FHD_ERR_INVALID_ARGUMENT, "M must be in [0, 2^31)");
    if (!Qhat) return fail(FHD_ERR_INVALID_ARGUMENT, "Qhat is NULL");
    if (M > 0 && (!kx || !ky || !kz || !phi))
      return fail(FHD_ERR_INVALID_ARGUMENT, "null sample array with M=%lld", (long long)M);
    if (opts && (opts->workspace || (opts->stages != 0 && opts->stages != FHD_STAGE_ALL)))
      return fail(FHD_ERR_INVALID_ARGUMENT, "fhd_toeplitz_kernel allocates its own scratch; pass no workspace or stages");
    const ncmri::ToeplitzDims d = ncmri::toeplitz_dims(nx, ny, nz);
    const int64_t n2 = 8 * d.voxels();
    const size_t fm = (size_t)M * sizeof(float), cm = (size_t)M * sizeof(fhd_c32);
    Range outr{Qhat, (size_t)d.spectrum() * sizeof(float)};
    Range ins[] = {{kx, fm}, {ky, fm}, {kz, fm}, {phi, cm}};
    for (const Range& r : ins)
      if (overlaps(outr, r)) return fail(FHD_ERR_INVALID_ARGUMENT, "Qhat overlaps an input array");
    st = check_device();
    if (st != FHD_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    // scratch: difference-grid coordinates, Q on that grid, the padded grid
    const size_t coord_bytes = align256((size_t)3 * n2 * sizeof(float));
    const size_t q_bytes = align256((size_t)n2 * sizeof(fhd_c32));
    char* scratch = nullptr;
    hipError_t e = hipMallocAsync((void**)&scratch, coord_bytes + q_bytes + ncmri::toeplitz_scratch_bytes(d), s);
    if (e != hipSuccess) return fail(FHD_ERR_HIP, "hipMallocAsync: %s", hipGetErrorString(e));
    float* coords = (float*)scratch;
    fhd_c32* Q2 = (fhd_c32*)(scratch + coord_bytes);
    float2* G = (float2*)(scratch + coord_bytes + q_bytes);
    fhd_status result = FHD_OK;
    e = ncmri::launch_diff_grid(nx, ny, nz, coords, coords + n2, coords + 2 * n2, s);
    if (e != hipSuccess) result = fail(FHD_ERR_HIP, "difference grid kernel: %s", hipGetErrorString(e));
    // Q on the difference grid through the library's Q path: the planes dz >= 0
    // (the first half of the grid), the others by Hermitian symmetry
    if (result == FHD_OK)
      result = run(1, kx, ky, kz, coords, coords + n2, coords + 2 * n2, phi, nullptr, Q2, M, n2 / 2, 1, opts, stream);
    if (result == FHD_OK) {
      e = ncmri::launch_hermitian_fill(nx, ny, nz, (float2*)Q2, s);
      if (e != hipSuccess) result = fail(FHD_ERR_HIP, "Hermitian fill kernel: %s", hipGetErrorString(e));
    }
    if (result == FHD_OK) {
      if (const char* fe = ncmri::toeplitz_spectrum(d, (const float2*)Q2, G, Qhat, s))
        result = fail(FHD_ERR_HIP, "spectrum of Q: %s", fe);
    }
    e = hipFreeAsync(scratch, s);
    if (e != hipSuccess && result == FHD_OK) result = fail(FHD_ERR_HIP, "hipFreeAsync: %s", hipGetErrorString(e));
    return result;
  } catch (...) {
    return fail(FHD_ERR_INTERNAL, "unexpected C++ exception");
  }
}

NCMRI_API fhd_status fhd_normal_apply(const float* Qhat, int32_t nx, int32_t ny, int32_t nz,
                                      float lambda, const fhd_c32* p, fhd_c32* Ap, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  try {
    g_err[0] = '\0';
    fhd_status st = check_grid(nx, ny, nz);
    if (st != FHD_OK) return st;
    if (!Qhat || !p || !Ap) return fail(FHD_ERR_INVALID_ARGUMENT, "null array");
    if (!(lambda >= 0.0f) || !(lambda < INFINITY)) return fail(FHD_ERR_INVALID_ARGUMENT, "lambda must be finite and >= 0");
    const ncmri::ToeplitzDims d = ncmri::toeplitz_dims(nx, ny, nz);
    const size_t nb = (size_t)d.voxels() * 8;
    st = check_cg_ws(d, workspace, workspace_bytes);
    if (st != FHD_OK) return st;
    Range ar{Ap, nb}, pr{p, nb}, qr{Qhat, (size_t)d.spectrum() * sizeof(float)}, wr{workspace, workspace_bytes};
    if (overlaps(ar, pr) || overlaps(ar, qr) || overlaps(wr, ar) || overlaps(wr, pr) || overlaps(wr, qr))
      return fail(FHD_ERR_INVALID_ARGUMENT, "overlapping arrays");
    st = check_device();
    if (st != FHD_OK) return st;
    ncmri::CgWorkspace w = ncmri::cg_workspace(workspace, d);
    if (const char* e = ncmri::normal_apply(d, Qhat, lambda, (const float2*)p, (float2*)Ap, w.T, w.T2, nullptr,
                                            (hipStream_t)stream))
      return fail(FHD_ERR_HIP, "normal operator: %s", e);
    return FHD_OK;
  } catch (...) {
    return fail(FHD_ERR_INTERNAL, "unexpected C++ exception");
  }
}

NCMRI_API fhd_status fhd_cg_solve(const float* Qhat, int32_t nx, int32_t ny, int32_t nz,
                                  float lambda, const fhd_c32* b, fhd_c32* x, int32_t iters,
                                  double* resid, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  try {
    g_err[0] = '\0';
    fhd_status st = check_grid(nx, ny, nz);
    if (st != FHD_OK) return st;
    if (!Qhat || !b || !x) return fail(FHD_ERR_INVALID_ARGUMENT, "null array");
    if (!(lambda >= 0.0f) || !(lambda < INFINITY)) return fail(FHD_ERR_INVALID_ARGUMENT, "lambda must be finite and >= 0");
    if (iters < 0) return fail(FHD_ERR_INVALID_ARGUMENT, "iters must be >= 0");
    const ncmri::ToeplitzDims d = ncmri::toeplitz_dims(nx, ny, nz);
    const size_t nb = (size_t)d.voxels() * 8;
    st = check_cg_ws(d, workspace, workspace_bytes);
    if (st != FHD_OK) return st;
    Range xr{x, nb}, br{b, nb}, qr{Qhat, (size_t)d.spectrum() * sizeof(float)}, wr{workspace, workspace_bytes},
        rr{resid, resid ? (size_t)(iters + 1) * sizeof(double) : 0};
    if (overlaps(xr, br) || overlaps(xr, qr) || overlaps(wr, xr) || overlaps(wr, br) || overlaps(wr, qr) ||
        overlaps(rr, xr) || overlaps(rr, br) || overlaps(rr, qr) || overlaps(rr, wr))
      return fail(FHD_ERR_INVALID_ARGUMENT, "overlapping arrays");
    st = check_device();
    if (st != FHD_OK) return st;
    ncmri::CgWorkspace w = ncmri::cg_workspace(workspace, d);
    if (const char* e = ncmri::cg_run(d, Qhat, lambda, (const float2*)b, (float2*)x, iters, resid, w,
                                      (hipStream_t)stream))
      return fail(FHD_ERR_HIP, "conjugate gradient: %s", e);
    return FHD_OK;
  } catch (...) {
    return fail(FHD_ERR_INTERNAL, "unexpected C++ exception");
  }
}

NCMRI_API fhd_status fhd_gridding(const float* kx, const float* ky, const float* kz, const fhd_c32* phi,
                                  const fhd_c32* D, int64_t M, int32_t nx, int32_t ny, int32_t nz,
                                  fhd_c32* image, void* stream) {
  try {
    g_err[0] = '\0';
    auto pow2 = [](int32_t n) { return n >= 2 && n <= ncmri::kToeplitzMaxLen && (n & (n - 1)) == 0; };
    if (!pow2(nx) || !pow2(ny) || !pow2(nz))
      return fail(FHD_ERR_INVALID_ARGUMENT, "gridding needs powers of two in [2, %d] per axis (got %d x %d x %d)",
                  ncmri::kToeplitzMaxLen, nx, ny, nz);
    const int64_t n = (int64_t)nx * ny * nz;
    if (n > 0x7fffffffLL) return fail(FHD_ERR_INVALID_ARGUMENT, "nx ny nz must be < 2^31");
    if (M < 0 || M > 0x7fffffffLL) return fail(FHD_ERR_INVALID_ARGUMENT, "M must be in [0, 2^31)");
    if (!image) return fail(FHD_ERR_INVALID_ARGUMENT, "image is NULL");
    if (M > 0 && (!kx || !ky || !kz || !phi || !D))
      return fail(FHD_ERR_INVALID_ARGUMENT, "null sample array with M=%lld", (long long)M);
    const size_t fm = (size_t)M * sizeof(float), cm = (size_t)M * sizeof(fhd_c32);
    Range outr{image, (size_t)n * sizeof(fhd_c32)};
    Range ins[] = {{kx, fm}, {ky, fm}, {kz, fm}, {phi, cm}, {D, cm}};
    for (const Range& r : ins)
      if (overlaps(outr, r)) return fail(FHD_ERR_INVALID_ARGUMENT, "image overlaps an input array");
    fhd_status st = check_device();
    if (st != FHD_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    void* scratch = nullptr;
    const size_t sb = ncmri::gridding_scratch_bytes(M, nz);
    hipError_t e = hipMallocAsync(&scratch, sb, s);
    if (e != hipSuccess) return fail(FHD_ERR_HIP, "hipMallocAsync(%zu): %s", sb, hipGetErrorString(e));
    fhd_status result = FHD_OK;
    if (const char* m = ncmri::gridding_run(kx, ky, kz, (const float2*)phi, (const float2*)D, M, nx, ny, nz,
                                            (float2*)image, scratch, s))
      result = fail(FHD_ERR_HIP, "gridding: %s", m);
    e = hipFreeAsync(scratch, s);
    if (e != hipSuccess && result == FHD_OK) result = fail(FHD_ERR_HIP, "hipFreeAsync: %s", hipGetErrorString(e));
    return result;
  } catch (...) {
    return fail(FHD_ERR_INTERNAL, "unexpected C++ exception");
  }
}

NCMRI_API fhd_status q_compute(const float* kx, const float* ky, const float* kz, const float* x,
                               const float* y, const float* z, const fhd_c32* phi, fhd_c32* Q,
                               int64_t M, int64_t N, const fhd_opts* opts, void* stream) {
  try {
    return run(1, kx, ky, kz, x, y, z, phi, nullptr, Q, M, N, 1, opts, stream);
  } catch (...) {
    return fail(FHD_ERR_INTERNAL, "unexpected C++ exception");
  }
}

NCMRI_API const char* fhd_status_string(fhd_status s) {
  switch (s) {
    case FHD_OK: return "FHD_OK";
    case FHD_ERR_INVALID_ARGUMENT: return "FHD_ERR_INVALID_ARGUMENT";
    case FHD_ERR_WORKSPACE: return "FHD_ERR_WORKSPACE";
    case FHD_ERR_HIP: return "FHD_ERR_HIP";
    case FHD_ERR_UNSUPPORTED_DEVICE: return "FHD_ERR_UNSUPPORTED_DEVICE";
    case FHD_ERR_INTERNAL: return "FHD_ERR_INTERNAL";
  }
  return "FHD_UNKNOWN_STATUS";
}

NCMRI_API const char* fhd_last_error(void) { return g_err; }

NCMRI_API const char* fhd_version(void) { return "ncmri-fhd 0.1.0 gfx950"; }
