/*
 * swe.h - C ABI of the MI355X (gfx950) shallow-water step library.
 *
 * One explicit time step of the first-order Roe finite-volume scheme for the
 * 2D shallow-water equations, as defined in
 *   [IR] de la Asuncion, Mantas, Castro, Fernandez-Nieto, "An MPI-CUDA
 *        implementation of an improved Roe method for two-layer shallow
 *        water systems", Sec. 2.1 (Eq. (1): the one/two-layer model; Eqs.
 *        (2)-(3): rotational invariance) and Sec. 2.2 (Eq. (4): the update
 *        W_i^{n+1} = W_i^n - dt/|V_i| sum_j |G_ij| F^-_ij with the IR-Roe
 *        flux of steps 1-4; Eq. (5): the CFL condition that fixes dt);
 *   [MG] Vinas et al., "A multi-GPU shallow-water simulation with transport
 *        of contaminants", abstract (one-layer SWE with a pollutant carried
 *        by a transport equation, first-order Roe finite volumes).
 * A step has three parts: (i) a Roe flux per edge with the path-conservative
 * bed term and the upwinded transverse momentum / pollutant flux;
 * (ii) per-cell accumulation of the flux contributions and of the CFL wave
 * speeds, then a global minimum for dt; (iii) the conserved-variable update.
 *
 * Every entry point returns an int status (SWE_OK = 0 or a negative
 * SWE_E_* code) unless stated otherwise; no C++ exception crosses the ABI
 * (any call that runs out of host or device memory returns SWE_E_NOMEM).
 * A context is not thread-safe; separate contexts are independent.
 * All GPU work of a context is ordered on one HIP stream.
 */
#ifndef SWE_H
#define SWE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWE_ABI_VERSION 2

typedef struct swe_ctx swe_ctx; /* opaque; owns every device allocation */

enum swe_status {
    SWE_OK = 0,
    SWE_E_INVAL = -1,          /* bad argument, bad mesh, call out of order  */
    SWE_E_NOMEM = -2,          /* host or device allocation failed          */
    SWE_E_HIP = -3,            /* a HIP runtime call failed                 */
    SWE_E_NOSTATE = -4,        /* swe_step / swe_get_state before set_state */
    SWE_E_DEPTH = -5,          /* a layer depth became <= 0 during a step   */
    SWE_E_NONFINITE = -6,      /* a state value became NaN or infinite      */
    SWE_E_NONHYPERBOLIC = -7   /* two-layer Roe matrix with complex speeds  */
};

enum swe_mesh_kind { SWE_MESH_CART = 0, SWE_MESH_TRI = 1 };
enum swe_precision { SWE_F64 = 0, SWE_F32 = 1 };
enum swe_bc { SWE_BC_WALL = 0, SWE_BC_PERIODIC = 1 };

/* Kernel path.  AUTO picks the fused one-launch-per-step path (Cartesian
 * one-layer grids and triangle meshes); EDGE forces the generic
 * explicit-edge-list path (three launches per step) on any mesh; FUSED
 * requests the fused path and fails with SWE_E_INVAL where none exists
 * (two layers on a Cartesian grid are rejected anyway).  RECOMPUTE is the
 * fused path in the "recomputation" organisation that [MG] contrasts with
 * its ghost-cell decoupling kernel: every cell evaluates all of its edges
 * (fluxes and Eq. (5) speeds) itself, so each interior edge is evaluated
 * twice, instead of once with the two cells sharing the result.  Same
 * results as FUSED up to rounding; an ablation.  IR-Roe flux only
 * (SWE_E_INVAL otherwise); on triangle meshes it runs the one-workgroup-
 * per-block kernel. */
enum swe_path { SWE_PATH_AUTO = 0, SWE_PATH_EDGE = 1, SWE_PATH_FUSED = 2, SWE_PATH_RECOMPUTE = 3 };

/* Numerical flux.  SWE_SCHEME_IR_ROE: the IR-Roe scheme of [IR] Sec. 2.2 --
 * the Roe matrix of the normal subsystem (2x2 for one layer, 4x4 for two),
 * with the transverse momentum and the pollutant carried by the mass flux
 * and upwinded by its sign.  SWE_SCHEME_ROE: the classical Roe scheme that
 * [IR] contrasts it with -- the Roe matrix of the whole edge system
 * ((h, q_n, q_t, hc) for one layer, 6x6 for two), whose transverse momentum
 * and pollutant rows are contact waves of each layer's Roe velocity,
 * upwinded like the other waves.  Both use the same walls and the same
 * Eq. (5) time step. */
enum swe_scheme { SWE_SCHEME_IR_ROE = 0, SWE_SCHEME_ROE = 1 };

/* Entropy fix.  [IR] Sec. 2.2 notes that the Roe solution needs one where
 * sonic rarefactions occur and names the Harten-Hyman fix.
 * SWE_ENTROPY_FIX_HH: that fix in its wave-splitting form, on the two
 * acoustic waves of the one-layer flux (IR-Roe or classical; the classical
 * flux's contact waves need none): with b = K^-1 (W_b - W_a) the state jumps of
 * the two Roe waves and W* = W_a + b_1 r_1 the state between them, a wave
 * whose characteristic speed changes sign from < 0 on its left state to > 0
 * on its right state is split into a left-moving part at the left speed and
 * a right-moving part at the right speed (fractions chosen so that the
 * wave's total flux jump is kept); the source term is untouched.  Available
 * for one layer on the FUSED and EDGE paths. */
enum swe_entropy_fix { SWE_ENTROPY_FIX_NONE = 0, SWE_ENTROPY_FIX_HH = 1 };

typedef struct swe_mesh_desc {
    int32_t abi_version; /* must be SWE_ABI_VERSION                          */
    int32_t mesh_kind;   /* SWE_MESH_CART or SWE_MESH_TRI                    */
    int32_t nlayers;     /* 1 or 2 (2: triangle meshes, no pollutant)        */
    int32_t ntracers;    /* 0 or 1 pollutant (one layer only)                */
    int32_t precision;   /* SWE_F64 or SWE_F32: storage and arithmetic type  */
    int32_t path;        /* enum swe_path                                    */
    int32_t scheme;      /* enum swe_scheme                                  */
    int32_t entropy_fix; /* 0: none; 1: Harten-Hyman (one layer)             */
    double g;            /* gravity, > 0                                     */
    double r;            /* density ratio rho1/rho2 in (0, 1) (two layers)   */

    /* Cartesian grid: nx * ny cells of dx * dy; cell k = j * nx + i has
     * centre ((i + 1/2) dx, (j + 1/2) dy).  Sides are walls or periodic. */
    int64_t nx, ny;      /* each >= 2                                        */
    double dx, dy;       /* > 0                                              */
    int32_t bc_x, bc_y;  /* enum swe_bc                                      */

    /* Triangle mesh: node coordinates (x, y) interleaved, 2 * nnodes values,
     * and 3 node ids per cell listed counter-clockwise.  Edges are derived:
     * an edge used by one cell is a reflective wall.  Both arrays are read
     * during swe_create_mesh only (the library keeps its own copies). */
    int64_t nnodes, ncells;
    const double *node_xy;
    const int32_t *tri;

    /* hipStream_t on which every call of the context enqueues its work, or
     * NULL for a stream owned by the context.  A caller stream must outlive
     * the context. */
    void *hip_stream;
} swe_mesh_desc;

/* Environment (read at swe_create_mesh; for tuning and tests, not needed in
 * normal use -- results do not depend on them beyond rounding):
 *   SWE_CART_TY=n, SWE_CART_ALT=0|1  rows per tile (4..4096) and alternating
 *                                    march of the fused Cartesian kernel;
 *   SWE_CART_STREAM=0|1              its streaming mode (non-temporal state
 *                                    loads, tile order reversed every other
 *                                    step), by default on where the two state
 *                                    copies and the bed exceed 256 MiB;
 *   SWE_TRI_B=n                      cells per triangle block (64..512, a
 *                                    multiple of 8), before the size checks;
 *   SWE_TRI_LDS=bytes                LDS cap per triangle block;
 *   SWE_TRI_NT=256                   256-thread triangle workgroups;
 *   SWE_TRI_PIPE=0|1                 the pipelined persistent triangle kernel
 *                                    (one layer) on or off;
 *   SWE_TRI_WGS=n                    its number of persistent workgroups
 *                                    (>= 8; by default as many as fit). */

/* Create a context for a mesh and upload its geometry ([IR] Sec. 2.2: cells
 * V_i with area |V_i|, edges G_ij with length |G_ij| and unit normal eta_ij
 * pointing from V_i to V_j; [IR] Sec. 3: the mesh is built once from the
 * input data, before the time loop).
 * Errors: SWE_E_INVAL for a NULL pointer, a wrong abi_version, nlayers not 1
 * or 2, a pollutant with two layers, two layers on a Cartesian grid,
 * nx or ny < 2, dx, dy or g <= 0, r outside (0, 1), a node id out of range,
 * a triangle with area <= 0, an edge shared by more than two triangles,
 * path, scheme or entropy_fix outside their enums, SWE_PATH_FUSED where no
 * fused path exists, SWE_PATH_RECOMPUTE with the classical scheme, the
 * entropy fix with two layers or SWE_PATH_RECOMPUTE,
 * a grid too large for 32-bit byte offsets of a field (fused Cartesian
 * path), a triangle mesh whose blocks cannot be formed or whose per-block
 * arrays exceed 32-bit byte offsets (fused and recomputation paths);
 * SWE_E_NOMEM / SWE_E_HIP on allocation or runtime failure.  On error *out
 * is set to NULL and nothing leaks. */
int swe_create_mesh(const swe_mesh_desc *desc, swe_ctx **out);

/* Upload the bed elevation and the conserved state ([IR] Eq. (1): W; the
 * depth function is H = -z_bed).  Host arrays of ncells doubles in the
 * caller's cell order:
 *   one layer:  cons[0..2] = h, qx, qy and, with a pollutant, cons[3] = h*c;
 *   two layers: cons[0..5] = h1, q1x, q1y, h2, q2x, q2y (layer 1 on top).
 * Float32 contexts round the values to float32.  Copies synchronously.
 * Errors: SWE_E_INVAL for NULL pointers; SWE_E_HIP on a copy failure. */
int swe_set_state(swe_ctx *ctx, const double *z_bed, const double *const *cons);

/* The bed and the state W of [IR] Eq. (1), as swe_set_state, from device
 * arrays of the context's precision (float or double), caller cell order,
 * ordered on the context stream (no host sync; the caller keeps its arrays
 * unchanged until the stream has passed this call).
 * Errors: SWE_E_INVAL for NULL pointers; SWE_E_HIP. */
int swe_set_state_device(swe_ctx *ctx, const void *z_bed, const void *const *cons);

/* Advance nsteps explicit steps ([IR] Eq. (4)) with CFL number cfl = gamma
 * of [IR] Eq. (5): dt = min_i 2 gamma |V_i| / sum_j |G_ij| ||D_ij||_inf,
 * taken from the state at the start of each step.  The steps run on the
 * context stream without host round trips; the call returns after the last
 * one finished.  t_advanced (nullable) receives the sum of the dt taken,
 * last_dt (nullable) the last one.  nsteps = 0 is a no-op.  Consecutive
 * calls continue one time stepping: on the fused paths a call with the same
 * cfl as the previous call starts from the dt that call's last step already
 * computed for the state it left (no separate dt pass), so n calls of one
 * step give bit for bit the result of one call of n steps; the first call
 * after a set_state, or with another cfl, computes dt of the state first.
 * Errors: SWE_E_INVAL for nsteps < 0 or cfl outside (0, 1];
 * SWE_E_NOSTATE before any set_state; SWE_E_DEPTH / SWE_E_NONFINITE /
 * SWE_E_NONHYPERBOLIC when a step produced such a state (the state is then
 * undefined until the next set_state); SWE_E_HIP on a runtime failure. */
int swe_step(swe_ctx *ctx, int32_t nsteps, double cfl, double *t_advanced,
             double *last_dt);

/* For callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): swe_step without
 * any allocation.  Same arguments, results and errors as swe_step (the
 * same kernels, bit for bit, and the context continues exactly as after
 * swe_step: swe_get_dt_history, a following swe_step or swe_step_noalloc).
 * The batch's bookkeeping (partial dt minima, block counters, time, error
 * flags, dt history) lives in one static device array per GPU (about 15.9
 * KB, held until the process ends) instead of buffers of the context, and
 * the call makes no hipMalloc / hipFree or other allocating call.  nsteps
 * must not exceed SWE_NOALLOC_MAX_STEPS (else SWE_E_INVAL, nothing run).
 * Every call on a GPU shares that GPU's array: calls that overlap in time on
 * one GPU (other threads, or contexts on streams that run concurrently) race
 * and must be serialised by the caller. */
#define SWE_NOALLOC_MAX_STEPS 1024
int swe_step_noalloc(swe_ctx *ctx, int32_t nsteps, double cfl, double *t_advanced, double *last_dt);

/* Download the conserved state W of [IR] Eq. (1) (after the steps taken so
 * far, W^n of Eq. (4)) into caller-allocated host arrays of ncells doubles
 * (layout as in swe_set_state).  Synchronous.
 * Errors: SWE_E_INVAL for NULL pointers; SWE_E_NOSTATE; SWE_E_HIP. */
int swe_get_state(swe_ctx *ctx, double *const *cons_out);

/* The state W of [IR] Eq. (1), as swe_get_state, into device arrays of the
 * context's precision (float or double), caller cell order, ordered on the
 * context stream (no host sync).  The caller owns the arrays; they must hold
 * ncells values each.
 * Errors: SWE_E_INVAL for NULL pointers; SWE_E_NOSTATE; SWE_E_HIP. */
int swe_get_state_device(swe_ctx *ctx, void *const *cons_out);

/* The dt of every step of the last swe_step call, in order: the global
 * minimum of [IR] Eq. (5) that each step of Eq. (4) used.  Copies at most
 * cap values into the caller's host array out and stores the number of steps
 * in *count.
 * Errors: SWE_E_INVAL for NULL pointers or cap < 0; SWE_E_HIP. */
int swe_get_dt_history(swe_ctx *ctx, double *out, int64_t cap, int64_t *count);

/* Release every resource of the context (the mesh of [IR] Sec. 3 built by
 * swe_create_mesh, both state copies and the step bookkeeping); waits for the
 * context's outstanding work first.  NULL is a no-op. */
void swe_destroy(swe_ctx *ctx);

/* Static description of a status code (never NULL). */
const char *swe_strerror(int status);

/* Detail of the last error on this context (never NULL; "" if none).  With
 * ctx = NULL: the detail of the calling thread's last failed
 * swe_create_mesh. */
const char *swe_last_error(const swe_ctx *ctx);

/* Number of conserved variables per cell, the components of W in [IR]
 * Eq. (1): 3 (h, qx, qy), 4 (with the pollutant h c of [MG]) or 6 (two
 * layers); -1 for NULL. */
int swe_nvars(const swe_ctx *ctx);

/* Number of cells; -1 for NULL. */
int64_t swe_ncells(const swe_ctx *ctx);

/* The kernel path the context runs (SWE_PATH_EDGE, SWE_PATH_FUSED or
 * SWE_PATH_RECOMPUTE); -1 for NULL. */
int swe_path(const swe_ctx *ctx);

/* What the context runs, as one line of text for logs: the kernel and its
 * launch shape (structured tiles and march order, triangle block size and
 * kernel, or the edge-list path).  Owned by the context and valid until
 * swe_destroy; "" for NULL.  Informational only: its wording may change. */
const char *swe_describe(const swe_ctx *ctx);

#ifdef __cplusplus
}
#endif

#endif /* SWE_H */
