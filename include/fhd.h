/*
 * fhd.h -- C ABI of the gfx950 F^H D / Q library (libncmri_fhd.so).
 *
 * The operations (PMPP ch. 17 "Iterative MRI reconstruction"):
 *
 *   F^H D  (section 17.2, Fig. 17.3; section 17.3, Figs. 17.4-17.17)
 *     FhD[b][n] = sum_{m<M} conj(phi[m]) * D[b][m]
 *                          * exp(+i 2 pi (kx[m] x[n] + ky[m] y[n] + kz[m] z[n]))
 *
 *   Q      (section 17.2: computed once per trajectory, same core structure)
 *     Q[n]      = sum_{m<M} |phi[m]|^2 * exp(+i 2 pi (kx[m] x[n] + ky[m] y[n] + kz[m] z[n]))
 *
 *   F rho  (section 17.2: F models the imaging physics; section 17.3 step 3
 *           synthesises scan data from an image, the "inverse process")
 *     D[b][m]   = phi[m] * sum_{n<N} rho[b][n] * exp(-i 2 pi (kx[m] x[n] + ky[m] y[n] + kz[m] z[n]))
 *
 * k is in cycles per voxel and x, y, z in voxel units, so k.x is the phase in
 * revolutions (Eq. 17.1 uses exp(i 2 pi k_j . r)).  The exponent sign and the
 * complex multiply-accumulate follow the register-promoted kernel on the
 * study-notes page for step 2 ("FHD Kernel memory bandwidth optimisation"):
 * re += rMu cos - iMu sin, im += iMu cos + rMu sin, with Mu = conj(phi) D (the
 * pages never print Mu; conj(phi) D makes the sum the conjugate transpose of
 * F[m][n] = phi[m] exp(-i 2 pi k_m . x_n) applied to D).
 *
 * The reconstruction entry points (fhd_toeplitz_kernel, fhd_normal_apply,
 * fhd_cg_solve) solve for the image with these operators; they are declared
 * below with their own conventions.
 *
 * Work is split as the pages' loop fission does (section 17.3 step 1, Figs.
 * 17.6/17.7): a per-sample kernel forms Mu and packs one k-space record per
 * sample; then a gather kernel over groups of voxels sums every sample (Figs.
 * 17.9/17.10 gather after loop interchange), on the vector ALU or, for voxel
 * groups on a common grid, as a matrix-core product (fhd_engine).
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers (hipMalloc / torch CUDA memory),
 *     caller-owned, naturally aligned (float: 4 B, fhd_c32: 8 B).
 *   - Complex data are interleaved (re, im) float32 pairs: fhd_c32.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *     null stream) and the call returns without synchronising.  Inputs must
 *     stay alive and unmodified until the stream has passed the work.
 *   - The output is overwritten (not accumulated into).  M == 0 writes zeros;
 *     N == 0 does nothing and returns FHD_OK.
 *   - Argument errors are reported before anything is enqueued.  Kernel faults
 *     surface at the caller's next synchronisation as a HIP error.
 *   - No C++ exception crosses this interface.  Calls are re-entrant; the only
 *     global state is a per-device property cache and the thread-local text
 *     returned by fhd_last_error().
 */
#ifndef NCMRI_FHD_H
#define NCMRI_FHD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One complex float32 sample, layout-compatible with torch.complex64. */
typedef struct fhd_c32 {
  float re, im;
} fhd_c32;

typedef enum fhd_status {
  FHD_OK = 0,
  FHD_ERR_INVALID_ARGUMENT = 1, /* null pointer with nonzero size, negative size,
                                   batch < 1, unknown enum, overlapping output */
  FHD_ERR_WORKSPACE = 2,        /* workspace too small / missing for split stages */
  FHD_ERR_HIP = 3,              /* a HIP runtime call or launch failed */
  FHD_ERR_UNSUPPORTED_DEVICE = 4, /* current device is not gfx950 */
  FHD_ERR_INTERNAL = 5          /* unexpected internal failure */
} fhd_status;

/* How sin/cos of the phase are evaluated (section 17.3 step 3, Fig. 17.17:
 * hardware trigonometry trades a little accuracy for speed). */
typedef enum fhd_trig {
  FHD_TRIG_ACCURATE = 0, /* exact reduction of the phase in revolutions + polynomial sincos (<= 2 ulp) */
  FHD_TRIG_HW = 1        /* fract() of the phase, then the v_sin_f32 / v_cos_f32 instructions */
} fhd_trig;

/* How the fp32 accumulators sum over the samples. */
typedef enum fhd_sum {
  FHD_SUM_BLOCKED = 0, /* per-tile partial sums folded into running totals; with
                          tile = 0 the matrix-core four-sample engine on the HW
                          trig path makes each launch row one tile ("row-block":
                          the row's sums stay in the MFMA accumulators, rows are
                          added in a fixed order afterwards) */
  FHD_SUM_KAHAN = 1,   /* as BLOCKED, with Kahan-compensated folding of the tiles */
  FHD_SUM_PLAIN = 2    /* one running fp32 sum over all samples */
} fhd_sum;

/* Which kernels evaluate the gather.  Both compute the same sums (only the
 * fp32 rounding differs) and share records, sample splits and reduction. */
typedef enum fhd_engine {
  FHD_ENGINE_AUTO = 0, /* MFMA, except with FHD_SUM_KAHAN or an explicit voxels_per_lane */
  FHD_ENGINE_VALU = 1, /* vector-ALU kernels: a lane owns voxels_per_lane voxels, three-FMA
                          complex multiply-accumulate per voxel and sample */
  FHD_ENGINE_MFMA = 2  /* matrix-core kernels: groups of consecutive voxels share one
                          phase per sample and the sum over samples is a complex matrix
                          product (group phases x per-sample factor columns) in three
                          real products: v_mfma_f32_16x16x4_f32 over blocks of four
                          samples for groups of 128 voxels (the default on cubic grids),
                          v_mfma_f32_32x32x2_f32 over pairs of samples for groups of 32
                          or 64 (blocked or plain summation only).  Waves whose groups do
                          not sit at common offsets (any non-grid coordinates) are
                          evaluated per voxel on the vector ALU over the same launch
                          rows, at about the rate of the VALU engine's per-voxel path */,
  FHD_ENGINE_MFMA16 = 3 /* half-split matrix-core kernels (F^H D, Q and the forward
                          operator; opt-in, never chosen by FHD_ENGINE_AUTO): the same
                          factored sum in groups of
                          128 / vectors voxels, each fp32 product formed from fp16 parts
                          (x = hi + lo, hi = fp16(x), lo = fp16(x - hi); hi hi + hi lo +
                          lo hi) on v_mfma_f32_16x16x32_f16 with fp32 accumulation, the
                          factors scaled by a power of two into fp16 range.  Products
                          carry ~2^-22 relative error (fp32: 2^-24).  FHD_SUM_BLOCKED
                          or PLAIN: on the HW path each launch row is one summation
                          block; the accurate path folds tiles of about sqrt(M)
                          samples (tile rounds up to a multiple of 32).  Irregular
                          waves run per voxel in fp32 as above */
} fhd_engine;

/* Operation codes of fhd_workspace_bytes and fhd_describe_plan. */
typedef enum fhd_op {
  FHD_OP_FHD = 0,     /* fhd_compute */
  FHD_OP_Q = 1,       /* q_compute */
  FHD_OP_FORWARD = 2  /* fhd_forward */
} fhd_op;

/* Pipeline stages: the two loops produced by loop fission, plus the
 * reduction of the sample-split rows' partial sums. */
enum {
  FHD_STAGE_MU = 1,     /* per-sample kernel: Mu (or |phi|^2) and sample records */
  FHD_STAGE_GATHER = 2, /* per-voxel gather kernel (one launch row per sample split) */
  FHD_STAGE_REDUCE = 4, /* adds the rows' partial sums into the output (no-op with one row) */
  FHD_STAGE_ALL = 7
};

/* Option bits (fhd_opts.flags).
 *
 * FHD_FLAG_NO_MIRROR_PAIRS: turn off mirror pairing on the four-sample
 *   matrix-core engine's hardware-trig path.  With pairing on (the default),
 *   voxel groups of 16 T / vectors consecutive voxels take their reference
 *   voxel at column V / 2; a group whose reference is exactly the negated
 *   reference of another has, at every sample, the conjugate group phase
 *   (e^{-i2 pi k.x} = conj e^{i2 pi k.x} for real k and x: PMPP ch. 17
 *   section 17.3, the phase of Eq. 17.1), so one phase and four real products
 *   give both groups' sums where two groups otherwise take two phases and
 *   six products.  The pairing is found on the device and checked exactly
 *   (coordinate equality); groups without a partner are summed alone.  On
 *   this path the launch rows are chosen on the device too, between half and
 *   twice the automatic count (exactly sample_splits when that is given), so
 *   that the paired waves fill whole rounds of resident workgroups. */
enum { FHD_FLAG_NO_MIRROR_PAIRS = 1 };

/* Options; pass NULL for all defaults (accurate trig, blocked sum, automatic
 * engine and tuning, library-allocated workspace, all stages).  Start from
 * fhd_default_opts() so that fields added later keep their defaults. */
typedef struct fhd_opts {
  int32_t trig;            /* fhd_trig, default FHD_TRIG_ACCURATE */
  int32_t sum;             /* fhd_sum, default FHD_SUM_BLOCKED */
  int32_t voxels_per_lane; /* group size; 0 = automatic.  VALU engine: 1, 2, 4, 8 or 16
                              voxels per lane.  MFMA engine: 32, 64 or 128 voxels sharing
                              one group phase in single-vector passes (T = 2, 4 or 8 units
                              of 16 complex columns; batched passes keep T, groups of
                              16 T / vectors; 128 runs the four-sample engine).
                              With FHD_ENGINE_AUTO, 1-16 select VALU and 32-128 MFMA */
  int32_t tile;            /* samples per summation tile; 0 = automatic: ~sqrt(M) (VALU,
                              accurate trig), ~4 sqrt(M) on the matrix cores with HW trig,
                              the whole launch row on the four-sample engine with HW trig */
  int32_t stages;          /* FHD_STAGE_* mask; 0 means FHD_STAGE_ALL.  Stages run in
                              separate calls must use the same sizes, options and
                              workspace, in the order MU, GATHER, REDUCE */
  int32_t sample_splits;   /* 0 = automatic; else 1..1024 launch rows that each sum a
                              contiguous share of the samples (partial sums, then a
                              fixed-order reduction); FHD_SUM_PLAIN always uses 1 */
  int32_t engine;          /* fhd_engine, default FHD_ENGINE_AUTO */
  int32_t flags;           /* FHD_FLAG_* bits; 0 = defaults */
  void* workspace;         /* device buffer (16-byte aligned), or NULL: the library then allocates it
                              stream-ordered (hipMallocAsync/hipFreeAsync) for this
                              call; running the stages in separate calls requires a
                              caller workspace that persists between them */
  size_t workspace_bytes;  /* size of `workspace` */
} fhd_opts;

/* Fills *opts with the defaults. */
void fhd_default_opts(fhd_opts* opts);

/* Workspace bytes the operation `op` (fhd_op: fhd_compute, q_compute or
 * fhd_forward) needs for these sizes and options (opts may be NULL).  Returns
 * 0 on invalid arguments.  The workspace holds the packed records (one per
 * sample and batch group for F^H D and Q, one per voxel group for the forward
 * operator) and, when the work is split across launch rows, the rows'
 * partial sums. */
size_t fhd_workspace_bytes(int64_t M, int64_t N, int32_t batch, int32_t op,
                           const fhd_opts* opts);

/*
 * F^H D for `batch` data vectors sharing one trajectory.
 *   kx, ky, kz : float[M]            k-space sample coordinates (cycles/voxel)
 *   x, y, z    : float[N]            voxel coordinates (voxel units), any set;
 *                                    regular grids run fastest
 *   phi        : fhd_c32[M]          per-sample complex weight
 *   D          : fhd_c32[batch][M]   scan data, vector-major
 *   FhD        : fhd_c32[batch][N]   output, overwritten; must not overlap any input
 * Returns FHD_OK or an error code (see fhd_last_error()).
 */
fhd_status fhd_compute(const float* kx, const float* ky, const float* kz,
                       const float* x, const float* y, const float* z,
                       const fhd_c32* phi, const fhd_c32* D, fhd_c32* FhD,
                       int64_t M, int64_t N, int32_t batch,
                       const fhd_opts* opts, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): F^H D as
 * fhd_compute, with the workspace taken from a fixed device array inside the
 * library instead of the caller or the stream-ordered allocator.  The array
 * holds FHD_NOALLOC_SCRATCH_BYTES (512 MiB); every GPU the library's code is
 * loaded on holds its own copy until the process ends.  The call allocates
 * nothing (no hipMalloc, hipMallocAsync or hipFree).
 *   Arguments, layouts, semantics and errors are those of fhd_compute, plus:
 *   - opts->workspace must be NULL and opts->stages FHD_STAGE_ALL (or 0),
 *     else FHD_ERR_INVALID_ARGUMENT;
 *   - with sample_splits = 0 the planned row count is lowered until the
 *     plan's workspace fits the array (the same sums in another order);
 *     a plan that still needs more than FHD_NOALLOC_SCRATCH_BYTES returns
 *     FHD_ERR_WORKSPACE before anything is enqueued (fhd_workspace_bytes
 *     gives a plan's need).
 *   Every call on one GPU shares that GPU's array and leaves the last call's
 *   contents in it: calls that overlap on one GPU (other host threads, or
 *   other streams before the earlier call's work has finished) race and give
 *   undefined results.  Calls ordered on one stream are safe.
 */
#define FHD_NOALLOC_SCRATCH_BYTES ((size_t)512 << 20)

fhd_status fhd_compute_noalloc(const float* kx, const float* ky, const float* kz,
                               const float* x, const float* y, const float* z,
                               const fhd_c32* phi, const fhd_c32* D, fhd_c32* FhD,
                               int64_t M, int64_t N, int32_t batch,
                               const fhd_opts* opts, void* stream);

/*
 * Q for one trajectory: as fhd_compute with the real weight |phi[m]|^2 in place
 * of conj(phi[m]) D[m].   Q : fhd_c32[N] output, overwritten.
 */
fhd_status q_compute(const float* kx, const float* ky, const float* kz,
                     const float* x, const float* y, const float* z,
                     const fhd_c32* phi, fhd_c32* Q,
                     int64_t M, int64_t N,
                     const fhd_opts* opts, void* stream);

/*
 * The forward model F applied to `batch` images on one trajectory:
 *   kx, ky, kz : float[M]            k-space sample coordinates (cycles/voxel)
 *   x, y, z    : float[N]            voxel coordinates (voxel units); groups of
 *                                    consecutive voxels on a common grid run on
 *                                    the matrix cores, others are evaluated directly
 *   phi        : fhd_c32[M]          per-sample complex weight
 *   rho        : fhd_c32[batch][N]   images, vector-major
 *   D          : fhd_c32[batch][M]   output scan data, overwritten; must not
 *                                    overlap any input
 * D[b][m] = phi[m] sum_n rho[b][n] exp(-i 2 pi k_m . x_n), so that
 * <F rho, d> = <rho, F^H d> with fhd_compute.  Runs on the matrix-core engine
 * only (FHD_ENGINE_VALU and FHD_SUM_KAHAN are rejected); voxels_per_lane may
 * be 0, 32, 64 or 128; sample_splits here splits the voxel groups across launch
 * rows.  FHD_ENGINE_MFMA16 sums over the voxel groups from fp16 parts of the
 * image entries (scaled by a power of two; groups of 128 / vectors voxels,
 * 32 groups per MFMA), the rest as on the fp32 engine.  N == 0 writes zeros; M == 0 does nothing.  Returns FHD_OK or an error
 * code as fhd_compute does.
 */
fhd_status fhd_forward(const float* kx, const float* ky, const float* kz,
                       const float* x, const float* y, const float* z,
                       const fhd_c32* phi, const fhd_c32* rho, fhd_c32* D,
                       int64_t M, int64_t N, int32_t batch,
                       const fhd_opts* opts, void* stream);

/*
 * Iterative reconstruction (section 17.2, Fig. 17.3): conjugate gradient on
 *
 *   (F^H F + lambda W^H W) rho = F^H D
 *
 * for an image on a unit voxel grid: nx x ny x nz voxels, x fastest, voxel
 * (ix, iy, iz) at coordinates (ix - nx/2, iy - ny/2, iz - nz/2) (any shift of
 * the grid gives the same operator).  F^H F is applied through Q, which is
 * computed once per trajectory (section 17.2): its entry for voxels n, n' is
 * Q at x_n - x_n', so F^H F is a convolution with Q over the coordinate
 * differences, run as a cyclic convolution on a padded grid of
 * px x py x pz points, p_a = the smallest power of two >= 2 n_a (transforms by
 * the library's own FFT kernels).  W is the first difference between face
 * neighbours (a stand-in for the pages' anatomical prior), so W^H W p at a
 * voxel is the sum of p[n] - p[n'] over its up to 6 neighbours.  All arrays
 * are device arrays; complex images are fhd_c32[nz][ny][nx].  Grids: 1 to 512
 * voxels per axis and 8 nx ny nz < 2^31.
 */

/* Bytes of the Toeplitz spectrum Qhat: px py pz floats (0 for an invalid grid). */
size_t fhd_toeplitz_bytes(int32_t nx, int32_t ny, int32_t nz);

/*
 * Qhat = DFT(Q embedded in the padded grid) / (px py pz), real, px py pz floats.
 * Q at difference d sits at d mod p per axis for |d| < n, zero elsewhere; as
 * Q(-d) = conj(Q(d)) the spectrum is real and only its real part is kept.
 * Layout (read by fhd_normal_apply / fhd_cg_solve only): the (ky, kx) columns
 * c = ky px + kx in blocks of W = min(32, px py) consecutive ones, each block
 * float[pz][W]; Qhat(kz, ky, kx) is at (c / W) pz W + kz W + c mod W.  Q
 * is computed by the q_compute path on the (2nz, 2ny, 2nx) grid of
 * differences (opts as for q_compute, without workspace or stages: the call
 * allocates its scratch with hipMallocAsync on `stream`).  Qhat is
 * overwritten; it must not overlap the inputs.  M == 0 gives Qhat = 0.
 */
fhd_status fhd_toeplitz_kernel(const float* kx, const float* ky, const float* kz,
                               const fhd_c32* phi, int64_t M,
                               int32_t nx, int32_t ny, int32_t nz,
                               float* Qhat, const fhd_opts* opts, void* stream);

/* Workspace bytes of fhd_normal_apply / fhd_cg_solve (0 for an invalid grid):
 * two nz x py x px working grids of the transforms (the second holds the y
 * transform's output in the blocks the z pass reads), three images and two
 * sets of 1024 dot-product partial sums. */
size_t fhd_cg_workspace_bytes(int32_t nx, int32_t ny, int32_t nz);

/*
 * Ap = F^H F p + lambda W^H W p with Qhat from fhd_toeplitz_kernel.
 *   p, Ap     : fhd_c32[nz][ny][nx]; Ap is overwritten and must not overlap p
 *   lambda    : finite, >= 0
 *   workspace : >= fhd_cg_workspace_bytes() bytes, 16-byte aligned, caller-owned
 */
fhd_status fhd_normal_apply(const float* Qhat, int32_t nx, int32_t ny, int32_t nz,
                            float lambda, const fhd_c32* p, fhd_c32* Ap,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * `iters` conjugate-gradient iterations from the start image in x (updated in
 * place): r = b - A x, p = r; then alpha = <r,r>/<p,Ap>, x += alpha p,
 * r -= alpha Ap, beta = <r',r'>/<r,r>, p = r' + beta p, with A the operator of
 * fhd_normal_apply.  Dot products are summed in double in a fixed order (the
 * result does not depend on scheduling); alpha and beta stay on the device,
 * so the call enqueues every iteration without synchronising.
 *   b     : fhd_c32[nz][ny][nx] right-hand side (F^H D)
 *   x     : fhd_c32[nz][ny][nx] start image in, solution out
 *   resid : NULL or a DEVICE double[iters + 1] receiving <r, r> before the
 *           first and after each iteration
 * A zero <p, Ap> or <r, r> sets the step to 0 (x then stays put).
 */
fhd_status fhd_cg_solve(const float* Qhat, int32_t nx, int32_t ny, int32_t nz,
                        float lambda, const fhd_c32* b, fhd_c32* x, int32_t iters,
                        double* resid, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Gridding reconstruction, the baseline of section 17.1 (Fig. 17.1B) that the
 * pages compare with the iterative image (section 17.3 step 3, Fig. 17.19):
 * each sample's conj(phi[m]) D[m] is spread with trilinear weights onto the 8
 * nearest points of the image's k-lattice kappa_j = (j - n/2)/n per axis
 * (periodic: neighbours past the edge wrap), and
 *   image[iz][iy][ix] = sum_j G[j] exp(+i 2 pi kappa_j . x_i),  x_i = i - n/2,
 * by the library's FFT kernels.  On a Cartesian trajectory (every sample on a
 * lattice point) this equals fhd_compute on the grid x_i.
 *   nx, ny, nz : powers of two in [2, 1024]
 *   image      : fhd_c32[nz][ny][nx], overwritten; must not overlap the inputs
 * The deposits are sorted by lattice plane (two entries of 20 bytes per
 * sample, in scratch the call allocates and frees stream-ordered) and summed
 * per tile of a plane in 64-bit fixed point (scaled by a power of two from M
 * and the largest |Re|, |Im| of conj(phi) D, so that no sum can overflow):
 * the result is bitwise reproducible, whatever the order of the samples.
 * NaN or infinite inputs give an undefined image.
 */
fhd_status fhd_gridding(const float* kx, const float* ky, const float* kz,
                        const fhd_c32* phi, const fhd_c32* D, int64_t M,
                        int32_t nx, int32_t ny, int32_t nz, fhd_c32* image, void* stream);

/* The launch plan the library derives from sizes and options. */
typedef struct fhd_plan_info {
  int32_t voxels_per_lane;  /* voxel group size of the first pass (VALU: voxels owned by one
                               lane; MFMA: voxels sharing one group phase) */
  int32_t tile;             /* samples per summation tile */
  int32_t passes;           /* gather launches (batch groups of 16, 8, 4, 2, 1 vectors) */
  int32_t record_dwords;    /* dwords per record of the first pass (forward: per voxel group) */
  int64_t padded_samples;   /* M rounded up to the record padding (forward: M) */
  size_t workspace_bytes;   /* = fhd_workspace_bytes(...) */
  int32_t sample_splits;    /* launch rows splitting the samples (forward: the voxel
                               groups); 1: no reduction step */
  int32_t engine;           /* FHD_ENGINE_VALU or FHD_ENGINE_MFMA */
  int32_t mirror_pairs;     /* 1: the gather pairs mirror groups (FHD_FLAG_NO_MIRROR_PAIRS);
                               the device then picks the launch rows, at most
                               max_sample_splits */
  int32_t max_sample_splits;/* most launch rows the plan's partial-sum buffer holds */
} fhd_plan_info;

/* Fills *info with the plan for these sizes and options (opts may be NULL);
 * returns FHD_ERR_INVALID_ARGUMENT (and leaves *info untouched) for the same
 * argument errors fhd_compute / q_compute report.  No device call. */
fhd_status fhd_describe_plan(int64_t M, int64_t N, int32_t batch, int32_t op,
                             const fhd_opts* opts, fhd_plan_info* info);

/* Static text for a status code. */
const char* fhd_status_string(fhd_status s);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* fhd_last_error(void);

/* Library version string. */
const char* fhd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NCMRI_FHD_H */
