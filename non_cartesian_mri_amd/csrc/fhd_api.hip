// C ABI of the F^H D / Q library: argument checks, planning, workspace and the
// two stream-ordered launches (see include/fhd.h for the contract).
#include "fhd.h"
#include "fhd_internal.h"

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

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
  int is_q;
  int trig;
  int sum;
  int V;
  int stages;
  int64_t M, N, mpad, tile;
  int batch;
  int npass;           // gather passes (batch groups)
  int bc[40];          // vectors per pass (<= 31 + 4 for batch <= 512)
  size_t pass_bytes[40];
  size_t ws_bytes;
};

// Voxel-group size when the caller leaves it to the library (measured on
// MI355X at 128^3 x 262,144 and Q at 128^3 x 2^20: 16 voxels per lane is
// fastest for both trig paths).  Smaller N shrinks the group so that at least
// ~2 waves per SIMD remain (256 CUs x 4 SIMDs x 2 waves x 64 lanes).
int auto_voxels_per_lane(int64_t N, int trig) {
  (void)trig;
  const int64_t lanes_wanted = 256LL * 4 * 2 * 64;
  int v = 16;
  while (v > 1 && (N + v - 1) / v < lanes_wanted) v /= 2;
  return v;
}

fhd_status make_plan(Plan& p, int is_q, int64_t M, int64_t N, int32_t batch, const fhd_opts* o) {
  fhd_opts d;
  fhd_default_opts(&d);
  if (!o) o = &d;
  if (M < 0 || N < 0) return fail(FHD_ERR_INVALID_ARGUMENT, "negative size (M=%lld, N=%lld)", (long long)M, (long long)N);
  if (M > 0x7fffffffLL || N > 0x7fffffffLL) return fail(FHD_ERR_INVALID_ARGUMENT, "M and N must be < 2^31");
  if (batch < 1) return fail(FHD_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", batch);
  if (batch > 16 * 32) return fail(FHD_ERR_INVALID_ARGUMENT, "batch must be <= 512 (got %d)", batch);
  if (o->trig != FHD_TRIG_ACCURATE && o->trig != FHD_TRIG_HW) return fail(FHD_ERR_INVALID_ARGUMENT, "unknown trig %d", o->trig);
  if (o->sum != FHD_SUM_BLOCKED && o->sum != FHD_SUM_KAHAN && o->sum != FHD_SUM_PLAIN) return fail(FHD_ERR_INVALID_ARGUMENT, "unknown sum %d", o->sum);
  if (o->tile < 0) return fail(FHD_ERR_INVALID_ARGUMENT, "tile must be >= 0");
  if (o->stages < 0 || o->stages > FHD_STAGE_ALL) return fail(FHD_ERR_INVALID_ARGUMENT, "unknown stages mask %d", o->stages);
  if (o->reserved != 0) return fail(FHD_ERR_INVALID_ARGUMENT, "reserved field must be 0");
  int V = o->voxels_per_lane;
  if (V != 0 && V != 1 && V != 2 && V != 4 && V != 8 && V != 16) return fail(FHD_ERR_INVALID_ARGUMENT, "voxels_per_lane must be 0, 1, 2, 4, 8 or 16 (got %d)", V);
  p.is_q = is_q;
  p.trig = o->trig;
  p.sum = o->sum;
  p.stages = o->stages == 0 ? FHD_STAGE_ALL : o->stages;
  p.M = M;
  p.N = N;
  p.batch = is_q ? 1 : batch;
  p.mpad = (M + ncmri::kUnroll - 1) / ncmri::kUnroll * ncmri::kUnroll;
  // batch groups: 16, 8, 4, 2, 1 vectors per gather pass
  p.npass = 0;
  int left = p.batch;
  for (int g = 16; g >= 1; g /= 2)
    while (left >= g) { p.bc[p.npass++] = g; left -= g; }
  if (p.batch > 1) {
    V = 1;  // batched passes amortise the phase over the vectors instead of voxels
  } else if (V == 0) {
    V = auto_voxels_per_lane(N, o->trig);
  }
  while (V > 1 && V > N) V /= 2;  // the first group must be complete
  p.V = V;
  if (o->sum == FHD_SUM_PLAIN) {
    p.tile = p.mpad > 0 ? p.mpad : ncmri::kUnroll;
  } else if (o->tile > 0) {
    p.tile = ((int64_t)o->tile + ncmri::kUnroll - 1) / ncmri::kUnroll * ncmri::kUnroll;
  } else {
    int64_t t = 64;
    while (t * t < p.mpad && t < 8192) t *= 2;
    p.tile = t;
  }
  p.ws_bytes = 0;
  for (int i = 0; i < p.npass; ++i) {
    int stride = ncmri::record_dwords(is_q, p.trig, p.V, p.bc[i]);
    p.pass_bytes[i] = (size_t)p.mpad * (size_t)stride * sizeof(float);
    p.ws_bytes += (p.pass_bytes[i] + 255) / 256 * 256;
    if (!ncmri::gather_supported(is_q, p.V, p.bc[i])) return fail(FHD_ERR_INTERNAL, "no kernel for V=%d BC=%d", p.V, p.bc[i]);
  }
  return FHD_OK;
}

fhd_status run(int is_q, const float* kx, const float* ky, const float* kz, const float* x,
               const float* y, const float* z, const fhd_c32* phi, const fhd_c32* D, fhd_c32* out,
               int64_t M, int64_t N, int32_t batch, const fhd_opts* opts, void* stream) {
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
    if (ws_given < p.ws_bytes)
      return fail(FHD_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_given, p.ws_bytes);
    Range wr{ws, ws_given};
    if (overlaps(wr, outr)) return fail(FHD_ERR_INVALID_ARGUMENT, "workspace overlaps the output");
    for (const Range& r : ins)
      if (overlaps(wr, r)) return fail(FHD_ERR_INVALID_ARGUMENT, "workspace overlaps an input array");
  } else if (p.stages != FHD_STAGE_ALL && p.ws_bytes > 0) {
    return fail(FHD_ERR_WORKSPACE, "running one stage alone needs a caller workspace");
  }
  if (N == 0) return FHD_OK;
  st = check_device();
  if (st != FHD_OK) return st;

  hipStream_t s = (hipStream_t)stream;
  bool own = false;
  if (!ws && p.ws_bytes > 0) {
    hipError_t e = hipMallocAsync(&ws, p.ws_bytes, s);
    if (e != hipSuccess) return fail(FHD_ERR_HIP, "hipMallocAsync(%zu): %s", p.ws_bytes, hipGetErrorString(e));
    own = true;
  }
  fhd_status result = FHD_OK;
  char* base = (char*)ws;
  int b0 = 0;
  for (int i = 0; i < p.npass && result == FHD_OK; ++i) {
    ncmri::Layout L{is_q, p.trig, p.V, p.bc[i], ncmri::header_dwords(p.trig),
                    ncmri::record_dwords(is_q, p.trig, p.V, p.bc[i])};
    float* rec = (float*)base;
    if (p.stages & FHD_STAGE_MU) {
      ncmri::RecordArgs ra{kx, ky, kz, x, y, z, (const float2*)phi,
                           is_q ? nullptr : (const float2*)(D + (int64_t)b0 * M), M, p.mpad, rec};
      hipError_t e = ncmri::launch_records(L, ra, s);
      if (e != hipSuccess) result = fail(FHD_ERR_HIP, "records kernel launch: %s", hipGetErrorString(e));
    }
    if (result == FHD_OK && (p.stages & FHD_STAGE_GATHER)) {
      ncmri::GatherArgs ga{rec, p.mpad, p.tile, x, y, z, N, (float2*)(out + (int64_t)b0 * N)};
      hipError_t e = ncmri::launch_gather(L, p.sum == FHD_SUM_KAHAN, ga, s);
      if (e != hipSuccess) result = fail(FHD_ERR_HIP, "gather kernel launch: %s", hipGetErrorString(e));
    }
    base += (p.pass_bytes[i] + 255) / 256 * 256;
    b0 += p.bc[i];
  }
  if (own) {
    hipError_t e = hipFreeAsync(ws, s);
    if (e != hipSuccess && result == FHD_OK) result = fail(FHD_ERR_HIP, "hipFreeAsync: %s", hipGetErrorString(e));
  }
  return result;
}

}  // namespace

NCMRI_API void fhd_default_opts(fhd_opts* o) {
  if (!o) return;
  std::memset(o, 0, sizeof(*o));
  o->trig = FHD_TRIG_ACCURATE;
  o->sum = FHD_SUM_BLOCKED;
  o->stages = FHD_STAGE_ALL;
}

NCMRI_API size_t fhd_workspace_bytes(int64_t M, int64_t N, int32_t batch, int32_t is_q,
                                     const fhd_opts* opts) {
  try {
    Plan p;
    if (make_plan(p, is_q ? 1 : 0, M, N, batch, opts) != FHD_OK) return 0;
    return p.ws_bytes;
  } catch (...) {
    return 0;
  }
}

NCMRI_API fhd_status fhd_describe_plan(int64_t M, int64_t N, int32_t batch, int32_t is_q,
                                       const fhd_opts* opts, fhd_plan_info* info) {
  try {
    g_err[0] = '\0';
    if (!info) return fail(FHD_ERR_INVALID_ARGUMENT, "info is NULL");
    Plan p;
    fhd_status st = make_plan(p, is_q ? 1 : 0, M, N, batch, opts);
    if (st != FHD_OK) return st;
    info->voxels_per_lane = p.V;
    info->tile = (int32_t)p.tile;
    info->passes = p.npass;
    info->record_dwords = p.npass > 0 ? ncmri::record_dwords(p.is_q, p.trig, p.V, p.bc[0]) : 0;
    info->padded_samples = p.mpad;
    info->workspace_bytes = p.ws_bytes;
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
