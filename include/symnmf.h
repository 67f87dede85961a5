/*
 * symnmf.h - C ABI of libsymnmf, the MI355X (gfx950) SymNMF clustering hot path.
 *
 * Pages cited below:
 *   P1 = "GPU-Accelerated Clustering for Financial Instruments at Scale"
 *   P2 = "GPU-Accelerated SymNMF Clustering Scales to a Million Financial
 *         Instruments" (the same post; it holds the displayed AdaGrad update and
 *         the AdaptGrow algorithm sketch)
 *   P3 = the paper-card page "GEM-KMeans: Memory-Efficient and Accurate
 *         Clustering on Massive Scale with GPU Optimization", second abstract
 *         (the SymNMF study)
 *
 * Conventions for every entry point:
 *   - Array arguments are DEVICE pointers unless the name ends in _host.
 *   - Matrices are row-major. S is n x n with leading dimension lds >= n,
 *     lds a multiple of 4, and S 16-byte aligned. X is T x n (day-major, row t
 *     holds the n returns of day t) with leading dimension ldx >= n. Factors
 *     H, G, P are n x k with leading dimension k (dense).
 *   - The caller owns every buffer. The library allocates no device memory
 *     and frees nothing: scratch space is the caller's workspace `ws` of at
 *     least symnmf_workspace_bytes(...) bytes, 256-byte aligned. (The one
 *     exception is symnmf_sh_noalloc's static 64 MiB device scratch, which
 *     comes with the library's code object on each device it runs on.)
 *   - All device work is enqueued on `hip_stream` (a hipStream_t; NULL is the
 *     null stream). Calls that fill _host outputs synchronise that stream
 *     before they return; symnmf_labels is asynchronous.
 *   - Return value: 0 = OK, > 0 = warning, < 0 = error (enum below). Arguments
 *     are validated on the host before any device work is enqueued; an
 *     invalid call returns SYMNMF_E_INVALID / SYMNMF_E_WORKSPACE and touches
 *     nothing. No C++ exception crosses this boundary.
 *   - Calls on one stream are serialised by the stream; concurrent calls need
 *     distinct workspaces.
 *   - Results are deterministic: every reduction runs in a fixed order, so the
 *     same inputs on the same device give bitwise identical outputs.
 */
#ifndef SYMNMF_H
#define SYMNMF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif
#pragma GCC visibility push(default)

#define SYMNMF_ABI_VERSION 5

enum symnmf_status {
    SYMNMF_OK = 0,
    SYMNMF_W_NOT_CONVERGED = 1, /* the fit stopped at max_iters */
    SYMNMF_E_INVALID = -1,      /* bad argument (null pointer, size, layout) */
    SYMNMF_E_WORKSPACE = -2,    /* workspace missing, misaligned or too small */
    SYMNMF_E_HIP = -3,          /* a HIP runtime call failed */
    SYMNMF_E_NONFINITE = -4,    /* NaN/Inf in the input or in the objective */
    SYMNMF_E_DEGENERATE = -5,   /* a constant column (correlation undefined) */
    SYMNMF_E_TOO_LARGE = -6     /* beyond symnmf_sh_noalloc's static scratch    */
};

/* Dependence matrix kinds (P1 introduction; P3). */
enum symnmf_kind { SYMNMF_ABSCORR = 0, SYMNMF_TPDM = 1 };

/* Solvers (P1 "Factorizing with SymNMF", "Why this solver"; P2 sketch). */
enum symnmf_solver { SYMNMF_AUTO = 0, SYMNMF_FULL = 1, SYMNMF_BLOCK_SVRG = 2 };

/* The S.H product of the fit's full-batch steps and anchor refreshes.
 * ROWS streams all of S in row panels (symnmf_sh). UPPER reads only the 32 x 32
 * blocks on or above the diagonal, each serving both of its products
 * (symnmf_sh_sym; P1 "Factorization at scale"; S = S^T since P1's introduction
 * defines S as an absolute correlation or a TPDM, both symmetric): half
 * the bytes of S per step, for k <= 32, with a workspace larger by about
 * 3 k n^2 / 512 bytes. The Block-SVRG sampled steps read row panels either way. */
enum symnmf_sh_pass { SYMNMF_SH_ROWS = 0, SYMNMF_SH_UPPER = 1 };

/* Initialisation of H (P1 "Factorizing with SymNMF": the same fixed-seed
 * initialisation for every window; P2 sketch: scale-matched). */
enum symnmf_init {
    SYMNMF_INIT_UNIFORM = 0,       /* H0 = init_scale * u(seed, i*k + c)                */
    SYMNMF_INIT_SCALE_MATCHED = 1, /* H0 = 2 sqrt(mean(S)/k) * u(seed, i*k + c)         */
    SYMNMF_INIT_CALLER = 2         /* H holds H0 on entry                               */
};

/* Operations for symnmf_workspace_bytes. */
enum symnmf_op {
    SYMNMF_OP_BUILD_S = 0,
    SYMNMF_OP_PROBE = 1,
    SYMNMF_OP_FIT = 2,
    SYMNMF_OP_SH = 3,
    SYMNMF_OP_KMEANS = 4, /* k_or_p = k */
    SYMNMF_OP_SQ = 5,     /* k_or_p = w */
    SYMNMF_OP_SH_SYM = 6  /* k_or_p = k */
};

/* u(seed, c) above: the top 24 bits of output c+1 of SplitMix64 (Steele, Lea
 * and Flood, OOPSLA 2014) started at state `seed`, times 2^-24. */

typedef struct symnmf_fit_params {
    int32_t solver;        /* enum symnmf_solver; default AUTO                          */
    int32_t max_iters;     /* most update steps; default 2000 (P2 sketch: steps=2000)   */
    double lr;             /* step eta; <= 0 selects sqrt(mean(S)/k)                    */
    double eps;            /* AdaGrad epsilon, outside the root; default 1e-8 (P2)      */
    int32_t block_rows;    /* rows per sampled block b; default 1024                    */
    int32_t init;          /* enum symnmf_init; default SCALE_MATCHED                   */
    double phi0;           /* > 0: initial sampled fraction, |B|0 = ceil(phi0 nb);
                              <= 0: seeded from gamma_{k+1}                              */
    double gap_threshold;  /* gamma_{k+1} >= this selects the full gradient; default 5  */
    double tol_rel;        /* stop when |f_{t-1} - f_t| < tol_rel max(|f_{t-1}|,
                              obj_floor ||S||^2) (full batch; per step of the epoch
                              between Block-SVRG anchors); 0 = never; default 1e-6       */
    double stall_tol;      /* sampled branch: anchor objective decrease below
                              stall_tol * previous anchor doubles |B|; default 1e-3     */
    double init_scale;     /* INIT_UNIFORM scale; default 0.1                           */
    uint64_t seed;         /* init and block-sampler seed; default 0                    */
    int32_t check_every;   /* host polls the device stop flag every this many steps;
                              results do not depend on it; default 16                   */
    int32_t resume;        /* 1: G holds the AdaGrad accumulator on entry (needs G)     */
    double rms_decay;      /* 0 (default): AdaGrad, G += g*g. In (0, 1): RMSprop, one of
                              the AdaGrad-family solvers of P3's abstract (Tieleman and
                              Hinton 2012): G = rms_decay G + (1 - rms_decay) g*g; the
                              projected step is unchanged. Applies to every step.      */
    int32_t sh_pass;       /* enum symnmf_sh_pass: the S.H product of the full-batch
                              steps and anchors; default ROWS                           */
    double obj_floor;      /* the stop test's denominator never falls below
                              obj_floor ||S||^2; default 0.05 (>= 0)                     */
    int32_t start_iter;    /* absolute step index of the entry H: the Block-SVRG block
                              lists of step t are drawn for start_iter + t; default 0;
                              with resume = 1 and a state, it must equal state->iter  */
} symnmf_fit_params;

/* The AdaptGrow controller's state at a returned H, for resuming a fit so that
 * the resumed call takes the same steps as one uninterrupted call. Host
 * struct; the two anchor buffers are caller-owned device arrays (n x k, ld k),
 * both required whenever a state is passed. symnmf_fit writes the state of the
 * H it returns (iter = start_iter + iterations) and reads it when resume = 1. */
typedef struct symnmf_fit_state {
    int32_t iter;          /* absolute step index of H                              */
    int32_t blocks;        /* |B|; n_blocks means the full-batch branch              */
    int32_t anchor_iter;   /* absolute step of the current Block-SVRG anchor; -1: none */
    int32_t f_prev_valid;  /* 1: f_prev is the exact objective of step iter - 1     */
    double f_anchor;       /* exact objective at anchor_iter                          */
    double f_prev;
    float* H_anchor;       /* device: H~, the anchor's H                             */
    float* P_anchor;       /* device: P~ = S H~                                      */
} symnmf_fit_state;

typedef struct symnmf_fit_report {
    int32_t iterations;     /* update steps taken in this call; H returned is
                               H_{start_iter + iterations}                               */
    int32_t converged;      /* 1 if the tol_rel test stopped the run                    */
    int32_t start_branch;   /* 0 full batch, 1 Block-SVRG                               */
    int32_t final_branch;
    int32_t blocks_final;   /* |B| at the end (n_blocks when full)                      */
    int32_t n_blocks;       /* nb = ceil(n / block_rows)                                */
    int32_t doublings;      /* number of |B| doublings                                  */
    int32_t zero_rows;      /* rows of the returned H that are all zero (label 0)       */
    int32_t f_last_iter;    /* step index of f_last within this call (its obj_trace)    */
    int32_t anchors;        /* Block-SVRG anchor refreshes                              */
    double gamma;           /* gamma_{k+1} used for the branch choice (NaN if unused)   */
    double lr_used;
    double init_scale_used; /* U(0, a) bound used for H0 (NaN for INIT_CALLER)          */
    double f_last;          /* last exact objective ||S - H H^T||_F^2 evaluated         */
    double S_fro2;          /* ||S||_F^2                                                */
    double S_mean;          /* mean(S)                                                  */
    double seconds;         /* wall time of the call                                    */
} symnmf_fit_report;

/* Fills *p with the defaults listed above. */
void symnmf_fit_params_default(symnmf_fit_params* p);

/* Bytes of workspace `op` needs for an n x n problem of rank/width k_or_p
 * (fit: k; probe: p; sh: k) and, for BUILD_S, T days. `prm` is read for FIT
 * (max_iters, block_rows) and may be NULL (defaults). Returns 0 for invalid
 * sizes. Always O(n k + n T + max_iters): no n x n scratch (P1 "Factorization
 * at scale": peak storage ~4 n^2 bytes, the caller's S, plus factor buffers). */
size_t symnmf_workspace_bytes(int op, int64_t n, int32_t k_or_p, int64_t T,
                              const symnmf_fit_params* prm);

/* Builds the dense dependence matrix S (n x n, fp32, lds) from the returns
 * window X (T x n, fp32, ldx) on the device.
 *   kind = SYMNMF_ABSCORR (P1 introduction: absolute Pearson correlation):
 *     z_ti = (x_ti - mu_i)/||x_.i - mu_i||_2 (moments in fp64), S = |Z^T Z|,
 *     a contraction over the T days on the bf16 matrix cores with exactly
 *     split fp32 operands (fp32 products, fp32 sums); the diagonal is kept.
 *     tail_frac is ignored.
 *   kind = SYMNMF_TPDM (P1 introduction; P3): losses -X, per-column ordinal
 *     ranks R (ties to the earlier day), F = R/(T+1), Frechet alpha = 2 margins
 *     x = (-1/ln F)^(1/2), day radius r_t = ||x_t.||_2 (fp64), the
 *     m = ceil(tail_frac T - 1e-4) largest-radius days (ties to the earlier day;
 *     the 1e-4 slack keeps a float tail_frac whose product with T is an
 *     integer up to rounding at that integer),
 *     theta_t = x_t./r_t, S = (1/m) Theta^T Theta (fp32 MFMA, K = m).
 * S is computed on upper-triangle tiles and mirrored, so it is bitwise
 * symmetric. Every element of S (columns < n of rows < n) is written.
 * S_fro2_host (nullable) receives ||S||_F^2 (fp64).
 * Errors: E_INVALID (T < 2, n < 1, ldx < n, lds < n or lds % 4, null
 * pointers, TPDM tail_frac not in (0, 1]); E_WORKSPACE; E_NONFINITE (NaN/Inf
 * in X); E_DEGENERATE (a constant column, ABSCORR only); E_HIP. */
int symnmf_build_S(int kind, const float* X, int64_t T, int64_t n, int64_t ldx,
                   float tail_frac, float* S, int64_t lds, double* S_fro2_host,
                   void* ws, size_t ws_bytes, void* hip_stream);

/* Spectral probe (P1 "Choosing the rank k", "Why this solver"): the p
 * eigenvalues of symmetric S of largest magnitude, by subspace iteration on
 * w = max(round_up(p + 16, 16), min(round_up(2p, 16), 128, n rounded down
 * to 16)) columns. Q0 = 2 u(seed, i*w + c) - 1; each step
 * forms Y = S Q with symnmf_sq's pass, takes the Ritz values of Q^T S Q (fp64
 * Householder tridiagonalisation and implicit QR on the host) and
 * orthonormalises Y by CholeskyQR2 (fp64 Cholesky on the host). Stops when every one of the top p Ritz values moved by at most
 * tol |theta_1| since the previous step, or after max_iters steps.
 * eigvals_host[p] receives the values in descending |lambda| with the sign
 * kept; iters_host (nullable) the steps taken. Requires 1 <= p and
 * w <= n. Errors: E_INVALID, E_WORKSPACE, E_NONFINITE, E_HIP. Returns
 * W_NOT_CONVERGED if max_iters was reached. */
int symnmf_spectral_probe(const float* S, int64_t n, int64_t lds, int32_t p,
                          int32_t max_iters, double tol, uint64_t seed,
                          double* eigvals_host, int32_t* iters_host, void* ws,
                          size_t ws_bytes, void* hip_stream);

/* One S.H pass (the dominant product, P1 "Factorization at scale"; P2):
 * P = S H (n x k, fp32) for symmetric S, and tr_host (nullable) receives
 * tr(H^T S H) = sum_i <H_i, P_i> in fp64. The pass streams S once in row
 * panels and uses S = S^T. Requires 1 <= k <= 128. A 16-byte aligned H
 * lets the pass use its faster kernels (compile-time widths, and for k > 40
 * a direct-to-LDS ring); the result is bit for bit the same either way. */
int symnmf_sh(const float* S, int64_t n, int64_t lds, const float* H, int32_t k,
              float* P, double* tr_host, void* ws, size_t ws_bytes, void* hip_stream);

/* symnmf_sh for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation). Same
 * product with the same kernels, so P and the trace are bit for bit those of
 * symnmf_sh: P = S H (n x k, ld k) and, if tr is non-null, *tr = tr(H^T S H)
 * written on the DEVICE (one double, 8-byte aligned). No workspace argument:
 * the scratch is a static device array of 64 MiB that each device the library
 * runs on holds until the process ends. A problem whose symnmf_sh workspace
 * (symnmf_workspace_bytes(SYMNMF_OP_SH, n, k, 0, NULL)) exceeds 64 MiB is
 * rejected with SYMNMF_E_TOO_LARGE before any device work (n up to ~21 800 at
 * k = 24). Asynchronous on hip_stream; the call allocates nothing and never
 * synchronises. Every call on a device shares that device's scratch, so calls
 * that overlap on one device (other streams, other threads) race; serialise
 * them. Requires 1 <= k <= 128, lds >= n, lds % 4 == 0, S 16-byte aligned.
 * Errors: E_INVALID, E_TOO_LARGE, E_HIP. */
int symnmf_sh_noalloc(const float* S, int64_t n, int64_t lds, const float* H, int32_t k,
                      float* P, double* tr, void* hip_stream);

/* The S.H pass from the upper triangle (P1 "Factorization at scale": the
 * S H products dominate; P1 introduction: S, an absolute correlation or a
 * TPDM, is symmetric by definition). Same contract as
 * symnmf_sh (P = S H, n x k, ld k; tr_host nullable) for 1 <= k <= 32, but
 * it reads only the 32 x 32 blocks of S on or above the diagonal, each once
 * (2 n^2 bytes instead of 4 n^2): an off-diagonal block S_ab adds S_ab H_b to
 * the rows of block a and S_ab^T H_a to the rows of block b. S must be
 * symmetric; below-diagonal blocks never enter the result, so for a
 * non-symmetric S it is that of its block-upper mirror (diagonal blocks as
 * stored). Products run on the bf16
 * matrix cores with exactly split operands, as symnmf_sq: within fp32
 * rounding of symnmf_sh, not bit for bit. Deterministic (fixed-order sums of
 * per-strip and per-chunk partials). S 16-byte aligned, lds % 4 == 0.
 * Errors: E_INVALID, E_WORKSPACE, E_HIP. */
int symnmf_sh_sym(const float* S, int64_t n, int64_t lds, const float* H, int32_t k,
                  float* P, double* tr_host, void* ws, size_t ws_bytes, void* hip_stream);

/* The spectral probe's product (P1 "Choosing the rank k", "Why this
 * solver": the top eigenvalues of S): Y = S Q for S n x n (lds, 16-byte
 * aligned) and Q, Y n x w dense (ld w), 1 <= w <= 128. Rows of S are read as
 * stored (S need not be symmetric). Computed on the bf16 matrix cores: every
 * fp32 operand is split exactly into three bf16 parts, x = x1 + x2 + x3, and
 * the six products x1y1, x1y2, x2y1, x1y3, x2y2, x3y1 accumulate in fp32; the
 * three dropped products are at most ~2^-23 |x y|, so Y agrees with an fp32
 * product to fp32 rounding (not bit for bit with symnmf_sh). Exact splitting
 * needs |S_ij|, |Q_jc| >= ~1e-31 or zero (smaller values lose low bits).
 * Deterministic: a fixed split of the columns of S and a fixed-order sum.
 * Errors: E_INVALID, E_WORKSPACE, E_HIP. */
int symnmf_sq(const float* S, int64_t n, int64_t lds, const float* Q, int32_t w,
              float* Y, void* ws, size_t ws_bytes, void* hip_stream);

/* SymNMF fit S ~ H H^T, H >= 0 (P1 "Factorizing with SymNMF", "Why this
 * solver"; P2 AdaGrad update and AdaptGrow sketch; P3).
 * Objective f(H) = ||S||^2 - 2 tr(H^T S H) + ||H^T H||^2 = ||S - H H^T||_F^2,
 * evaluated without n x n intermediates (P1 "Factorization at scale").
 * Full-batch step t: P = S H_t, f_t, stop test, g = 4 (H_t (H_t^T H_t) - P),
 * G += g*g, H_{t+1} = max(H_t - lr g/(sqrt(G) + eps), 0). The stop test ends
 * the run at H_t when |f_{t-1} - f_t| < tol_rel max(|f_{t-1}|, obj_floor
 * ||S||^2) (a relative change; the floor keeps it meaningful when S can be
 * factored almost exactly and f tends to zero, as for a TPDM of rank below k).
 * Block-SVRG steps replace P by P~ + (nb/|B|) sum_{rows i in B} S[i,:]^T
 * (H - H~)[i,:] over |B| sampled row blocks (B drawn for the absolute step
 * index); a step is an anchor (H~ = H_t, P~ = S H_t, f exact, exact gradient)
 * when ceil(nb/|B|) steps have passed since the last one. At an anchor E_j
 * steps after the previous one: |f~prev - f~| < tol_rel E_j max(|f~prev|,
 * obj_floor ||S||^2) stops the run at this H (converged); otherwise a
 * decrease below stall_tol f~prev doubles |B|, until the run is full batch
 * (AUTO and BLOCK_SVRG), G kept.
 * AUTO chooses the branch from gamma_{k+1} = lambda_{k+1}/|lambda_{k+2}| of
 * eigvals_host (>= gap_threshold: full; else |B|0 = 2^floor(log2(max(1,
 * gamma/gap_threshold nb)))), unless phi0 > 0. The denominator is floored at
 * 1e-6 |lambda_1|. eigvals_host needs n_eig >= k + 2 entries in descending
 * |lambda| when used.
 * H (n x k): output (and input for INIT_CALLER). G (nullable, n x k): receives
 * the accumulator of the returned H (input too when resume = 1).
 * obj_trace_host (nullable): f_t for the steps of this call, t < min(
 * obj_trace_cap, steps evaluated); NaN for Block-SVRG steps (f is exact only at
 * anchors).
 * rep_host (nullable): the report.
 * state (nullable, host): the controller state of the returned H, written on
 * every successful return; with resume = 1 also read on entry (branch, |B|,
 * anchor, previous objectives), which skips the branch choice. Without a
 * state, resume = 1 restores only G (exact for full-batch runs without a stop
 * test).
 * Requires S symmetric and nonnegative, 1 <= k <= 64, k <= n.
 * Returns OK, W_NOT_CONVERGED, or E_INVALID / E_WORKSPACE / E_NONFINITE /
 * E_HIP. */
int symnmf_fit(const float* S, int64_t n, int64_t lds, int32_t k,
               const symnmf_fit_params* prm, const double* eigvals_host,
               int32_t n_eig, float* H, float* G, double* obj_trace_host,
               int32_t obj_trace_cap, symnmf_fit_report* rep_host,
               symnmf_fit_state* state, void* ws, size_t ws_bytes, void* hip_stream);

/* Hard labels (P1 "Factorizing with SymNMF": the row-wise argmax of H):
 * labels[i] = argmax_c H[i, c], lowest index on ties; an all-zero row gets 0.
 * n = 0 is a no-op (the pointers are not used). Asynchronous.
 * Errors: E_INVALID, E_HIP. */
int symnmf_labels(const float* H, int64_t n, int32_t k, int32_t* labels, void* hip_stream);

/* Spherical k-means on the L2-normalised rows of S, the hard-clustering
 * baseline (P1 "Spherical k-means for direct hard clustering": rows of S
 * compared by cosine similarity; "Between spherical k-means and SymNMF").
 * x_i = S[i,:] / ||S[i,:]||; the k initial centroids are the rows
 * x_{r_0} < ... < x_{r_{k-1}} drawn without replacement by the Block-SVRG
 * sampler's generator with this seed and step 0 (nb = n). Each iteration
 * assigns every row to its most similar centroid (argmax_j <x_i, c_j>, lowest
 * j on ties; computed as the row argmax of S C^T, S symmetric) and stops when
 * no label changed; otherwise each centroid becomes the normalised sum of its
 * rows (a cluster left empty keeps its centroid). Two passes over S per
 * iteration.
 * labels (n int32, device): the final assignment (made against the final
 * centroids). centroids (nullable, device, n x k, ld k): column j holds c_j.
 * iters_host (nullable): centroid updates made; converged_host (nullable): 1
 * when the last assignment changed nothing; objective_host (nullable):
 * sum_i <x_i, c_{labels[i]}> of the final assignment (fp64).
 * Requires S symmetric, 1 <= k <= 64, k <= n, max_iters >= 0.
 * Returns OK, W_NOT_CONVERGED (max_iters updates made and the last assignment
 * still moved rows), or E_INVALID / E_WORKSPACE / E_HIP. */
int symnmf_spherical_kmeans(const float* S, int64_t n, int64_t lds, int32_t k,
                            int32_t max_iters, uint64_t seed, int32_t* labels,
                            float* centroids, int32_t* iters_host,
                            int32_t* converged_host, double* objective_host,
                            void* ws, size_t ws_bytes, void* hip_stream);

const char* symnmf_status_string(int status);
int symnmf_abi_version(void);

/* Kernel timing, for measurement. When enabled, the library brackets every
 * launch of the kernels below with HIP events on the launch stream and
 * accumulates their durations (read back on symnmf_profile_read, which
 * synchronises the recorded events). Disabled by default; enabling adds an
 * event pair per launch. */
enum symnmf_prof_kernel {
    SYMNMF_PROF_SH_FULL = 0,    /* the full S.H pass (fit, symnmf_sh)          */
    SYMNMF_PROF_SH_SAMPLED = 1, /* the Block-SVRG sampled row-panel pass       */
    SYMNMF_PROF_SH_PROBE = 2,   /* the probe's S.Q pass                        */
    SYMNMF_PROF_BUILD_GRAM = 3, /* the MFMA Z^T Z / Theta^T Theta build        */
    SYMNMF_PROF_UPDATE = 4,     /* fused reduce + gradient + AdaGrad + Gram    */
    SYMNMF_PROF_SH_KMEANS = 5,  /* the spherical k-means passes over S         */
    SYMNMF_PROF_SH_SYM = 6,     /* the upper-triangle S.H pass (symnmf_sh_sym) */
    SYMNMF_PROF_COUNT = 7
};
void symnmf_profile_enable(int on);
void symnmf_profile_reset(void);
/* launches, summed milliseconds and summed algorithmic bytes (the bytes the
 * operation must move at least: S panels read plus factor reads and writes)
 * of kernel `which`. Returns E_INVALID for an unknown kernel. */
int symnmf_profile_read(int which, int64_t* launches, double* total_ms, double* total_bytes);

#pragma GCC visibility pop
#ifdef __cplusplus
}
#endif
#endif /* SYMNMF_H */
