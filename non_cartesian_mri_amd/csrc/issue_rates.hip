// Issue-rate microbenchmarks for gfx950 that back the gather kernel's cost
// model: FP32 FMA throughput, v_sin_f32 throughput, whether transcendentals
// share the VALU issue port with FMAs (mixed loops), whether the group-phase
// VALU work overlaps FP32 MFMAs (the matrix-core gather's inner loop with and
// without it, for both MFMA shapes), the same inner loop with its products
// formed from fp16 high/low parts on the fp16 matrix cores (a design option
// weighed and not built), the shader clock, and the absolute error of
// v_sin_f32/v_cos_f32 and of sincospif over one turn.
// Standalone program: built by non_cartesian_mri_amd/build.py
// (build_issue_rates) and run by `python bench.py --issue-rates`.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cmath>
#include <vector>
#include <cstdlib>
#include <type_traits>

#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e), __LINE__); exit(1);} } while(0)

template <int K>
__global__ void __launch_bounds__(256) k_fma(float* out, int iters, float a, float b) {
  float acc[K];
#pragma unroll
  for (int j = 0; j < K; ++j) acc[j] = threadIdx.x * 1e-3f + j;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < K; ++j) acc[j] = __builtin_fmaf(acc[j], a, b);
  }
  float s = 0;
#pragma unroll
  for (int j = 0; j < K; ++j) s += acc[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// T chains of sin; K independent fma chains per iteration.
template <int T, int K>
__global__ void __launch_bounds__(256) k_mix(float* out, int iters, float a, float b) {
  float u[T];
  float acc[K > 0 ? K : 1];
#pragma unroll
  for (int j = 0; j < T; ++j) u[j] = threadIdx.x * 1e-4f + j * 0.01f;
#pragma unroll
  for (int j = 0; j < (K > 0 ? K : 1); ++j) acc[j] = threadIdx.x * 1e-3f + j;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < T; ++j) u[j] = __builtin_amdgcn_sinf(u[j]);
#pragma unroll
    for (int j = 0; j < K; ++j) acc[j] = __builtin_fmaf(acc[j], a, b);
  }
  float s = 0;
#pragma unroll
  for (int j = 0; j < T; ++j) s += u[j];
#pragma unroll
  for (int j = 0; j < K; ++j) s += acc[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The matrix-core gather's inner loop without its memory traffic: per block
// of KS samples, 3 NT MFMAs (the three-product form; NT tiles) and, with
// PHASE, the group phase (3 FMAs), fract, v_sin, v_cos, c + s and c - s of
// one lane.  KS = 2: v_mfma_f32_32x32x2_f32 (64 cycles); KS = 4:
// v_mfma_f32_16x16x4_f32 (32 cycles).  The phase inputs are made opaque each
// block so that the VALU work is not hoisted.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
template <int KS, int NT, bool PHASE>
__global__ void __launch_bounds__(512) k_mfma_mix(float* out, int blocks_per_wave, float k0, float k1,
                                                  float k2) {
  extern __shared__ float occupancy_pad[];  // sized by the launch to fix waves per SIMD
  const int lane = threadIdx.x & 63;
  const float gx = (float)(lane & 15) - 8.0f, gy = 3.0f, gz = -5.0f;
  float hk[3] = {k0, k1, k2};
  float bv[3 * NT];
#pragma unroll
  for (int i = 0; i < 3 * NT; ++i) bv[i] = 0.01f * (i + 1) + 1e-4f * lane;
  using Acc = typename std::conditional<KS == 2, f32x16_t, f32x4_t>::type;
  Acc acc[3][NT];
#pragma unroll
  for (int u = 0; u < 3; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[u][t] = Acc{};
  for (int q = 0; q < blocks_per_wave; ++q) {
    float av[3];
    if constexpr (PHASE) {
      const float ph = __builtin_fmaf(hk[2], gz, __builtin_fmaf(hk[1], gy, hk[0] * gx));
      const float f = __builtin_amdgcn_fractf(ph);
      const float sn = __builtin_amdgcn_sinf(f), cs = __builtin_amdgcn_cosf(f);
      av[0] = cs + sn; av[1] = cs - sn; av[2] = sn;
      asm volatile("" : "+v"(hk[0]), "+v"(hk[1]), "+v"(hk[2]));
    } else {
      av[0] = hk[0]; av[1] = hk[1]; av[2] = hk[2];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        if constexpr (KS == 2)
          acc[u][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[u], bv[u * NT + t], acc[u][t], 0, 0, 0);
        else
          acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], bv[u * NT + t], acc[u][t], 0, 0, 0);
      }
  }
  float sum = 0.0f;
#pragma unroll
  for (int u = 0; u < 3; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t)
      for (int v = 0; v < (KS == 2 ? 16 : 4); ++v) sum += acc[u][t][v];
  if (blocks_per_wave < 0) { occupancy_pad[threadIdx.x] = sum; __syncthreads(); sum += occupancy_pad[lane]; }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

// The matrix-core gather's inner loop with each fp32 product formed from fp16
// parts: x = hi + lo (hi = fp16(x), lo = fp16(x - hi)), x y ~ hi_x hi_y +
// hi_x lo_y + lo_x hi_y with fp32 accumulation, on v_mfma_f32_16x16x32_f16
// (K = 32 samples per MFMA; A[i][k] = lane i + 16 (k / 8), element k % 8).
// Per 32-sample block a wave evaluates 8 group phases per lane (16 groups),
// splits (c + s, c - s, s) into hi / lo, reads the B parts of 8 tiles of 16
// columns from LDS (3 products x 2 parts, 16 bytes per lane each) and issues
// 8 x 3 x 3 = 72 MFMAs (16 cycles each): the four-sample engine's pairs per
// block (16 groups x 128 columns x 32 samples).  STAGE 0: MFMAs only; 1: with
// the phases and splits; 2: also the B parts from LDS.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
template <int STAGE>
__global__ void __launch_bounds__(512) k_mfma16(float* out, int blocks_per_wave, float k0, float k1, float k2) {
  constexpr int CT = 8;
  __shared__ uint4 lb[CT * 6 * 64];
  __shared__ float hdr[32 * 3];
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < CT * 6 * 64; i += 512) {
    const unsigned v = 0x3c003c00u ^ (unsigned)(i & 7);
    lb[i] = make_uint4(v, v, v, v);
  }
  for (int i = threadIdx.x; i < 96; i += 512) hdr[i] = (i % 3 == 0 ? k0 : i % 3 == 1 ? k1 : k2) * (1 + i);
  __syncthreads();
  const float gx = (float)(lane & 15) - 8.0f, gy = 3.0f, gz = -5.0f;
  f32x4_t acc[3][CT];
#pragma unroll
  for (int u = 0; u < 3; ++u)
#pragma unroll
    for (int t = 0; t < CT; ++t) acc[u][t] = f32x4_t{};
  half8_t A[3][2];
#pragma unroll
  for (int u = 0; u < 3; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) { A[u][0][e] = (_Float16)(0.01f * (lane + e + u)); A[u][1][e] = (_Float16)0.0f; }
  float hk = k0;
  for (int q = 0; q < blocks_per_wave; ++q) {
    if constexpr (STAGE >= 1) {
      float v[8][3];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float* h = &hdr[(8 * (lane >> 4) + e) * 3];
        const float ph = __builtin_fmaf(h[2], gz, __builtin_fmaf(h[1], gy, h[0] * gx + hk));
        const float f = __builtin_amdgcn_fractf(ph);
        const float sn = __builtin_amdgcn_sinf(f), cs = __builtin_amdgcn_cosf(f);
        v[e][0] = cs + sn;
        v[e][1] = cs - sn;
        v[e][2] = sn;
      }
      // hi pairs by one packed conversion, lo = fp16(x - hi) by the
      // mixed-precision FMA into either half (the gather's split)
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int u = 0; u < 3; ++u) {
          const half2_t h = {(_Float16)v[2 * p][u], (_Float16)v[2 * p + 1][u]};
          const unsigned hb = __builtin_bit_cast(unsigned, h);
          unsigned lb2;
          asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(lb2) : "v"(hb), "v"(v[2 * p][u]));
          asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
              : "+v"(lb2) : "v"(hb), "v"(v[2 * p + 1][u]));
          const half2_t l = __builtin_bit_cast(half2_t, lb2);
          A[u][0][2 * p] = h[0];
          A[u][0][2 * p + 1] = h[1];
          A[u][1][2 * p] = l[0];
          A[u][1][2 * p + 1] = l[1];
        }
      asm volatile("" : "+v"(hk));
    }
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      half8_t B[3][2];
#pragma unroll
      for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if constexpr (STAGE >= 2) {
            const uint4 w = lb[((t * 3 + u) * 2 + s) * 64 + lane];
            B[u][s] = *reinterpret_cast<const half8_t*>(&w);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) B[u][s][e] = (_Float16)(0.5f + 0.001f * (t + u + s + e));
          }
        }
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[u][0], B[u][0], acc[u][t], 0, 0, 0);
        acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[u][0], B[u][1], acc[u][t], 0, 0, 0);
        acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[u][1], B[u][0], acc[u][t], 0, 0, 0);
      }
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int u = 0; u < 3; ++u)
#pragma unroll
    for (int t = 0; t < CT; ++t) sum += acc[u][t][0] + acc[u][t][3];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

// The per-pair gather body of the pages' kernel without its memory traffic:
// one voxel per lane; per sample the phase (1 mul + 2 FMA), fract, v_sin,
// v_cos and the complex multiply-accumulate -- four FMAs (re += mr c - mi s,
// im += mi c + mr s) or, with GAUSS, c + s and s - c then three FMAs on
// (fr + fi, fr, fi) as the VALU engine's records hold them.  The sample's k
// and weights are wave-uniform values whose bit patterns advance by scalar
// integer adds each sample, so they cost no VALU work and nothing is hoisted.
template <int U, bool GAUSS>
__global__ void __launch_bounds__(256) k_pair(float* out, int iters, int kb0, int kb1, int kb2) {
  const float x = (float)(threadIdx.x & 63) - 32.0f, y = (float)(blockIdx.x & 127) - 64.0f;
  const float z = (float)(threadIdx.x >> 6) - 2.0f;
  float re = 0.0f, im = 0.0f, cr = 0.0f;
  int kxb = kb0, kyb = kb1, kzb = kb2, mrb = 0x3e99999a, mib = 0xbf333333, sb = 0xbecccccd;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float kx = __builtin_bit_cast(float, kxb), ky = __builtin_bit_cast(float, kyb);
      const float kz = __builtin_bit_cast(float, kzb), mr = __builtin_bit_cast(float, mrb);
      const float mi = __builtin_bit_cast(float, mib), mpi = __builtin_bit_cast(float, sb);
      const float t = __builtin_fmaf(kz, z, __builtin_fmaf(ky, y, kx * x));
      const float f = __builtin_amdgcn_fractf(t);
      const float sn = __builtin_amdgcn_sinf(f), cs = __builtin_amdgcn_cosf(f);
      if constexpr (GAUSS) {
        const float cps = cs + sn, smc = sn - cs;
        re = __builtin_fmaf(mpi, cs, re);        // (fr + fi) is a record value: uniform
        im = __builtin_fmaf(mi, cps, im);
        cr = __builtin_fmaf(mr, smc, cr);
      } else {
        re = __builtin_fmaf(mr, cs, __builtin_fmaf(-mi, sn, re));
        im = __builtin_fmaf(mi, cs, __builtin_fmaf(mr, sn, im));
      }
      kxb += 17; kyb -= 29; kzb += 13; mrb += 7; mib -= 11; sb += 5;
    }
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = re + im + cr;
}

__global__ void k_clock(long long* out, int iters, float a, float b, float* sink) {
  long long c0 = clock64();
  long long w0 = wall_clock64();
  float x = threadIdx.x;
  for (int i = 0; i < iters; ++i) x = __builtin_fmaf(x, a, b);
  long long c1 = clock64();
  long long w1 = wall_clock64();
  if (threadIdx.x == 0) { out[0] = c1 - c0; out[1] = w1 - w0; }
  sink[threadIdx.x] = x;
}

__global__ void k_trig_acc(const float* r, float* s_hw, float* c_hw, float* s_pi, float* c_pi, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float x = r[i];
  s_hw[i] = __builtin_amdgcn_sinf(x);
  c_hw[i] = __builtin_amdgcn_cosf(x);
  float s, c;
  sincospif(2.0f * x, &s, &c);
  s_pi[i] = s; c_pi[i] = c;
}

template <typename F>
double time_it(F f, int reps) {
  hipEvent_t e0, e1; CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
  f(); CK(hipDeviceSynchronize());
  CK(hipEventRecord(e0));
  for (int r = 0; r < reps; ++r) f();
  CK(hipEventRecord(e1)); CK(hipEventSynchronize(e1));
  float ms; CK(hipEventElapsedTime(&ms, e0, e1));
  return ms / reps * 1e-3;
}

int main() {
  hipDeviceProp_t p; CK(hipGetDeviceProperties(&p, 0));
  printf("device %s arch %s CUs %d clock %d kHz\n", p.name, p.gcnArchName, p.multiProcessorCount, p.clockRate);
  const int CU = p.multiProcessorCount;
  float* out; CK(hipMalloc(&out, 64 << 20));
  long long* clk; CK(hipMalloc(&clk, 64));
  // clock estimate
  {
    int iters = 1 << 22;
    hipLaunchKernelGGL(k_clock, dim3(1), dim3(64), 0, 0, clk, iters, 0.999f, 0.001f, out);
    CK(hipDeviceSynchronize());
    long long h[2]; CK(hipMemcpy(h, clk, 16, hipMemcpyDeviceToHost));
    printf("clock: %lld shader cycles in %lld wall ticks (100MHz) -> %.3f GHz, cycles/dep-fma %.2f\n", h[0], h[1], h[0] / (h[1] * 10.0), (double)h[0] / iters);
  }
  const int waves_per_simd = 8;
  const int blocks = CU * 4 * waves_per_simd / 4;  // 256 threads = 4 waves per block
  const int iters = 4096;
  double threads = (double)blocks * 256;
  {
    double t = time_it([&] { hipLaunchKernelGGL(k_fma<16>, dim3(blocks), dim3(256), 0, 0, out, iters, 0.999f, 0.001f); }, 10);
    double fl = threads * iters * 16 * 2;
    printf("MB-FMA: %.2f TFLOP/s (%.3f ms)\n", fl / t * 1e-12, t * 1e3);
  }
  {
    double t = time_it([&] { hipLaunchKernelGGL((k_mix<8, 0>), dim3(blocks), dim3(256), 0, 0, out, iters, 0.999f, 0.001f); }, 10);
    double tr = threads * iters * 8;
    printf("MB-TRANS: %.3f Tsin/s = %.2f per clk per CU at 2.4GHz (%.3f ms)\n", tr / t * 1e-12, tr / t / (CU * 2.4e9), t * 1e3);
  }
#define MIX(T, K) { double t = time_it([&] { hipLaunchKernelGGL((k_mix<T, K>), dim3(blocks), dim3(256), 0, 0, out, iters, 0.999f, 0.001f); }, 10); \
    double wi = (double)blocks * 4 * iters; /* wave-iterations */ \
    double slots = t * CU * 2.4e9 / wi; /* cycles per wave-iteration per CU */ \
    printf("MB-MIX T=%d K=%2d: %.3f ms, CU-cycles per wave-iter %.2f (x4 SIMD = %.2f SIMD-cycles)\n", T, K, t * 1e3, slots, slots * 4); }
  MIX(2, 0) MIX(2, 2) MIX(2, 4) MIX(2, 6) MIX(2, 8) MIX(2, 12) MIX(2, 16) MIX(2, 24)
  MIX(4, 0) MIX(4, 8) MIX(4, 16)
  // the per-pair body: pairs/s at 8 waves per SIMD (the pages' form and the
  // VALU engine's three-FMA form)
#define PAIR(U, G, NAME) { double t = time_it([&] { hipLaunchKernelGGL((k_pair<U, G>), dim3(blocks), dim3(256), 0, 0, out, iters, 0x3d4ccccd, 0xbe19999a, 0x3c23d70a); }, 10); \
    double pairs = threads * iters * U; \
    printf("MB-PAIR %s: %.3e pairs/s, %.2f CU-cycles per wave-pair at 2.4 GHz (%.3f ms)\n", NAME, pairs / t, \
           t * CU * 2.4e9 / (pairs / 64), t * 1e3); }
  PAIR(4, false, "4-FMA MAC (pages' form)") PAIR(4, true, "3-FMA MAC + c+s, s-c")
  // FP32 MFMA with and without the per-block phase work, 2 waves per SIMD
  // (LDS padding: two 4-wave workgroups or one 8-wave workgroup per CU)
  {
    const int bpw = 16384;
#define MFMA_MIX(KS, NT, WG, LDSB, NAME, CYC)                                                        \
    {                                                                                               \
      const int wgs = CU * 8 / (WG / 64);                                                           \
      CK(hipFuncSetAttribute((const void*)k_mfma_mix<KS, NT, false>,                                \
                             hipFuncAttributeMaxDynamicSharedMemorySize, LDSB));                     \
      CK(hipFuncSetAttribute((const void*)k_mfma_mix<KS, NT, true>,                                 \
                             hipFuncAttributeMaxDynamicSharedMemorySize, LDSB));                     \
      double t0 = time_it([&] { hipLaunchKernelGGL((k_mfma_mix<KS, NT, false>), dim3(wgs), dim3(WG), LDSB, 0, out, bpw, 0.013f, 0.027f, -0.031f); }, 5); \
      double t1 = time_it([&] { hipLaunchKernelGGL((k_mfma_mix<KS, NT, true>), dim3(wgs), dim3(WG), LDSB, 0, out, bpw, 0.013f, 0.027f, -0.031f); }, 5); \
      CK(hipGetLastError());                                                                        \
      const double mfma_cycles = (double)wgs * (WG / 64) * bpw * 3 * NT * CYC;                     \
      const double ideal = mfma_cycles / (CU * 4 * 2.4e9);                                          \
      printf("MB-MFMA %s: MFMA only %.3f ms (matrix busy %.3f at 2.4 GHz); + phase/fract/sin/cos/c+s/c-s %.3f ms (%.3f): +%.1f SIMD-cycles per phase over %d MFMA-cycles\n", \
             NAME, t0 * 1e3, ideal / t0, t1 * 1e3, ideal / t1, (t1 - t0) * CU * 4 * 2.4e9 / ((double)wgs * (WG / 64) * bpw), 3 * NT * CYC); \
    }
    MFMA_MIX(2, 2, 256, 70 * 1024, "32x32x2 (2 samples, 6 MFMAs per phase)", 64)
    MFMA_MIX(4, 8, 512, 100 * 1024, "16x16x4 (4 samples, 24 MFMAs per phase)", 32)
  }
  // the same work per pair with fp16 high/low products (one 8-wave workgroup per CU)
  {
    const int bpw = 2048;
    double t[3];
    t[0] = time_it([&] { hipLaunchKernelGGL(k_mfma16<0>, dim3(CU), dim3(512), 0, 0, out, bpw, 0.013f, 0.027f, -0.031f); }, 5);
    t[1] = time_it([&] { hipLaunchKernelGGL(k_mfma16<1>, dim3(CU), dim3(512), 0, 0, out, bpw, 0.013f, 0.027f, -0.031f); }, 5);
    t[2] = time_it([&] { hipLaunchKernelGGL(k_mfma16<2>, dim3(CU), dim3(512), 0, 0, out, bpw, 0.013f, 0.027f, -0.031f); }, 5);
    CK(hipGetLastError());
    const double pairs = (double)CU * 8 * bpw * 16 * 128 * 32;
    const double ideal = (double)CU * 8 * bpw * 72 * 16 / (CU * 4 * 2.4e9);
    printf("MB-MFMA16 fp16 hi/lo 16x16x32 (32 samples, 72 MFMAs per 8 phases): MFMA only %.3e pairs/s (matrix busy %.3f); "
           "+ phases and splits %.3e; + B parts from LDS %.3e pairs/s (%.0f SIMD-cycles per 32-sample block over %d MFMA-cycles)\n",
           pairs / t[0], ideal / t[0], pairs / t[1], pairs / t[2], t[2] * CU * 4 * 2.4e9 / ((double)CU * 8 * bpw), 72 * 16);
  }
  // accuracy of builtins on r in [0,1)
  {
    const int n = 1 << 24;
    std::vector<float> r(n);
    for (int i = 0; i < n; ++i) r[i] = (float)((double)i / n) ;
    float *dr, *a, *b, *c, *d;
    CK(hipMalloc(&dr, n * 4)); CK(hipMalloc(&a, n * 4)); CK(hipMalloc(&b, n * 4)); CK(hipMalloc(&c, n * 4)); CK(hipMalloc(&d, n * 4));
    CK(hipMemcpy(dr, r.data(), n * 4, hipMemcpyHostToDevice));
    hipLaunchKernelGGL(k_trig_acc, dim3(n / 256), dim3(256), 0, 0, dr, a, b, c, d, n);
    CK(hipDeviceSynchronize());
    std::vector<float> sh(n), ch(n), sp(n), cp(n);
    CK(hipMemcpy(sh.data(), a, n * 4, hipMemcpyDeviceToHost)); CK(hipMemcpy(ch.data(), b, n * 4, hipMemcpyDeviceToHost));
    CK(hipMemcpy(sp.data(), c, n * 4, hipMemcpyDeviceToHost)); CK(hipMemcpy(cp.data(), d, n * 4, hipMemcpyDeviceToHost));
    double mh = 0, mp = 0, rh = 0, rp = 0;
    for (int i = 0; i < n; ++i) {
      double th = 2 * M_PI * (double)r[i];
      double es = sin(th), ec = cos(th);
      double e1 = fmax(fabs(sh[i] - es), fabs(ch[i] - ec));
      double e2 = fmax(fabs(sp[i] - es), fabs(cp[i] - ec));
      mh = fmax(mh, e1); mp = fmax(mp, e2);
      rh += (sh[i] - es) * (sh[i] - es) + (ch[i] - ec) * (ch[i] - ec);
      rp += (sp[i] - es) * (sp[i] - es) + (cp[i] - ec) * (cp[i] - ec);
    }
    printf("trig accuracy over 2^24 pts in [0,1) rev: HW max abs %.3e rms %.3e | sincospif max abs %.3e rms %.3e\n", mh, sqrt(rh / (2.0 * n)), mp, sqrt(rp / (2.0 * n)));
  }
  printf("done\n");
  return 0;
}
