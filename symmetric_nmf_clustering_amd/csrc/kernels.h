// Internal launcher interface between the host controller (symnmf.cpp) and the
// gfx950 kernels (k_*.hip). Every launcher enqueues on `st` and returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace symnmf {

constexpr int kMaxK = 64;         // widest factor the fit supports
constexpr int kMaxWidth = 128;    // widest S.H pass (probe subspace)
constexpr int kShTileCols = 256;  // columns of S per S.H workgroup (4 waves x 64)
constexpr int kUpdRows = 64;      // rows per workgroup of the fused update kernel
constexpr int kGramTile = 128;    // S-build workgroup tile (2 x 2 waves of 64 x 64)

constexpr int kMaxSplits = 32;   // row splits of one S.H pass (fixed-order sum)

// Which rows of S one split of the S.H pass streams.
//  contiguous (blocks == nullptr): split s covers
//      [s * rows_per_split, min(n, (s + 1) * rows_per_split))
//  sampled, sub > 1: split s covers rows [s%sub * seg, +seg) of block
//      blocks[s / sub] (clipped to the block and to n)
//  sampled, sub == 1: split s covers the whole blocks
//      blocks[s * bps .. min(nsel, (s + 1) * bps) - 1]
struct RowPlan {
    int n;
    int rows_per_split;
    const int* blocks;
    int nsel;
    int block_rows;
    int sub;
    int seg;
    int bps;
    const int* done;  // nullable: a set flag (a fit that has stopped) skips the pass
};

// Device state of one fit, in the caller's workspace.
struct FitDev {
    double S_fro2;
    double K2;          // ||H_t^T H_t||_F^2 for the current H_t
    double f_prev;      // last exact objective
    double tol;         // relative convergence tolerance (0: no test)
    double floor_abs;   // the stop test's denominator is max(|f_prev|, floor_abs)
    int f_prev_valid;
    int done;           // once set, every later kernel of the fit returns at once
    int stop_iter;
    int status;         // 0 running, 1 converged, -4 non-finite objective
    double tr;            // finalisation scratch: tr(H_t^T P_t)
    double K2next;        // finalisation scratch: ||H_{t+1}^T H_{t+1}||^2
    double Kd[kMaxK * kMaxK];  // finalisation scratch: Gram entries (fp64)
    float K[kMaxK * kMaxK];    // H_t^T H_t (fp32, full symmetric, ld kMaxK)
};

// ---- S.H pass ---------------------------------------------------------------
// part[s][i][c] (ld ldp = round_up(width, 4), split stride n*ldp) =
//   sum over rows j of split s of S[j][i] * X[j][c]
// which is (S X)[i][c] restricted to those rows, for symmetric S. Only the
// rows of the plan are read from X.
hipError_t launch_sh_panel(const float* S, int64_t lds, const float* X, int width,
                           const RowPlan& rp, int nsplit, float* part, int ldp, hipStream_t st);
// Rows per split of a full pass: at most kMaxSplits splits of at least 64 rows
// (a multiple of 4), so one output accumulates at most ceil(n / kMaxSplits)
// rows in fp32 before the fixed-order split sum. Every split is non-empty.
inline int sh_full_rows_per_split(int n) {
    const int per = (n + kMaxSplits - 1) / kMaxSplits;
    return ((per > 64 ? per : 64) + 3) / 4 * 4;
}
// ---- the probe's S.Q pass on the bf16 matrix cores (k_sq.hip) -------------
// Q is packed once per pass into the matrix core's B operands (each fp32 value
// split exactly into three bf16 parts); the pass then writes
// part[s][i][c] (ld ldp, split stride n*ldp) = sum over the K blocks of split s
// of S[i][j] Q[j][c], rows of S read directly (no symmetry assumed).
struct SqPlan {
    int nt;             // 16-column tiles of Q (width <= 16 nt)
    int nsplit;         // K splits (every one non-empty)
    int kb_per_split;   // 32-column K blocks per split
    size_t packed_bytes;  // size of the packed Q
};
SqPlan sq_plan(int n, int width);
hipError_t launch_sq_pack(const float* Q, int64_t ldq, int n, int width, const SqPlan& p,
                          void* Qs, hipStream_t st);
hipError_t launch_sq_split(const float* S, int64_t lds, const void* Qs, int n, int width,
                           const SqPlan& p, float* part, int ldp, hipStream_t st);
// ---- the symmetric S.H pass on the bf16 matrix cores (k_sym.hip) ----------
// Uses the 32 x 32 blocks of S on or above the diagonal once each; H is
// packed twice (launch_sym_pack: the column side's and the row side's K maps).
// The pass writes row-side partials P1 (one per 512-column strip and row,
// compact: strip s holds rows [0, min(n, 512 (s + 1)))) and column-side
// partials P2 (one per 2048-row chunk, strip and column of the strip); the
// fold adds them in a fixed order into P (n x k, ld ldP), with the trace
// partials as launch_reduce_partials (Hdot n x k, ld k).
constexpr int kSymStrip = 512;   // columns per strip
constexpr int kSymChunk = 2048;  // rows per chunk
constexpr int kSymMaxK = 32;     // widest factor of the symmetric pass
struct SymPlan {
    int nt;                   // 16-column tiles of H
    int ns;                   // strips
    int nq;                   // chunks of the tallest strip
    size_t p1_floats;         // size of P1
    size_t p2_floats;         // size of P2
    int nkb_col, nkb_row;     // K blocks of the two packings of H
    size_t packed_col_bytes;  // sizes of the two packings
    size_t packed_row_bytes;
    bool half;                // the last tile holds at most 8 factors (two parts per operand)
};
SymPlan sym_plan(int n, int k);
// `done` (nullable, device): a set flag skips the launch's work (a fit that
// has already stopped).
hipError_t launch_sym_pack(const float* H, int n, int k, const SymPlan& p, void* HsR, void* HsC,
                           const int* done, hipStream_t st);
hipError_t launch_sym(const float* S, int64_t lds, const void* HsR, const void* HsC, int n, int k,
                      const SymPlan& p, float* P1, float* P2, const int* done, hipStream_t st);
hipError_t launch_sym_fold(const float* P1, const float* P2, int n, int k, const SymPlan& p,
                           float* P, int ldP, const float* Hdot, double* tr_part, const int* done,
                           hipStream_t st);
// D[j][c] = H[j][c] - Ha[j][c] (fp32) for the rows j of the nsel listed row
// blocks of block_rows rows (the Block-SVRG correction's input); other rows
// of D are left as they are.
hipError_t launch_block_diff(const float* H, const float* Ha, const int* blocks, int nsel,
                             int block_rows, int n, int k, float* D, const int* done,
                             hipStream_t st);
// P[i][c] = sum_s part[s][i][c] (c < width, ld width); if Hdot: tr_part[b] =
// sum over the rows of block b of <Hdot_i, P_i> (fp64). Blocks of kUpdRows rows.
hipError_t launch_reduce_partials(const float* part, int nsplit, int n, int width, int ldp,
                                  float* P, const float* Hdot, double* tr_part, hipStream_t st);

// ---- fit --------------------------------------------------------------------
constexpr int kStatsRows = 16;  // rows of S per block of the statistics pass
// part2[2b], part2[2b+1] = sum and sum of squares of S over rows
// [kStatsRows b, kStatsRows (b+1)) (fp64); ceil(n / kStatsRows) blocks.
hipError_t launch_s_stats(const float* S, int64_t lds, int n, double* part2, hipStream_t st);
hipError_t launch_s_stats_final(const double* part2, int nblk, double* out2, hipStream_t st);
hipError_t launch_init_uniform(float* H, int64_t count, double scale, double shift, uint64_t seed,
                               hipStream_t st);
hipError_t launch_fill(float* p, int64_t count, float v, hipStream_t st);
hipError_t launch_copy(float* dst, const float* src, int64_t count, hipStream_t st);

struct UpdateArgs {
    int n, k, ldp;
    const float* part;   // nsplit partial products (nullable for gram-only)
    int nsplit;
    int64_t pstride;
    const float* Pt;     // Block-SVRG anchor product P~ (nullable: exact pass)
    float pscale;        // nb / |B|
    const float* H;      // H_t
    const float* G;      // G_t
    float* Hn;           // H_{t+1}
    float* Gn;           // G_{t+1}
    float* Ha;           // anchor H~ <- H_t (nullable)
    float* Pa;           // anchor P~ <- P_t (nullable)
    FitDev* fd;
    float lr, eps;
    float decay;         // 0: AdaGrad accumulator; in (0, 1): RMSprop moving average
    double* tr_part;     // per block <H_t, P_t> (nullable)
    float* gram_part;    // per block partial Gram of the rows written (k x k)
    int gram_only;       // 1: no update, Gram partials of H
};
hipError_t launch_update(const UpdateArgs& a, hipStream_t st);
// flags: 1 exact objective this step, 2 convergence test, 4 fold Gram partials into K
hipError_t launch_finalize(FitDev* fd, double* f_trace, int t, int nblk, int k,
                           const double* tr_part, const float* gram_part, int flags,
                           hipStream_t st);
hipError_t launch_count_zero_rows(const float* H, int n, int k, int* out, hipStream_t st);
hipError_t launch_labels(const float* H, int64_t n, int k, int32_t* labels, hipStream_t st);

// ---- spherical k-means (k_kmeans.hip) -----------------------------------------
// rinv[i] = 1/||S[i,:]||_2 (fp64 sum of squares; 0 for a zero row).
hipError_t launch_row_norm_inv(const float* S, int64_t lds, int n, float* rinv, hipStream_t st);
// Ct[l][j] = S[idx[j]][l] * rinv[idx[j]] (n x k, ld k).
hipError_t launch_gather_centroids(const float* S, int64_t lds, int n, const int* idx,
                                   const float* rinv, int k, float* Ct, hipStream_t st);
// *changes += #{i : lab[i] != lab_prev[i]}; obj_part[b] = sum over rows of
// block b (256 rows) of rinv[i] * P[i][lab[i]] (fp64).
hipError_t launch_kmeans_assign_stats(const float* P, int n, int k, const int32_t* lab,
                                      const int32_t* lab_prev, const float* rinv, int* changes,
                                      double* obj_part, hipStream_t st);
// W[i][j] = lab[i] == j ? rinv[i] : 0.
hipError_t launch_onehot_scaled(const int32_t* lab, const float* rinv, int n, int k, float* W,
                                hipStream_t st);
// Ct[:, j] = C[:, j] / ||C[:, j]|| where that norm is > 0 (else Ct[:, j] kept);
// part: ceil(n/256) * k doubles, norm: k doubles.
hipError_t launch_normalize_columns(const float* C, int n, int k, double* part, double* norm,
                                    float* Ct, hipStream_t st);
hipError_t launch_fill_int(int32_t* p, int64_t count, int32_t v, hipStream_t st);

// ---- probe helpers ----------------------------------------------------------
// C = A^T B (w x w, fp64) for n x w matrices A, B (ld w): per-block fp32
// partials, then a fixed-order fp64 reduction into C.
hipError_t launch_crossgram(const float* A, const float* B, int n, int w, float* part,
                            int nblk, double* C, hipStream_t st);
int crossgram_blocks(int n);
// Q[i][:] = Y[i][:] M (M w x w fp32, row-major)
hipError_t launch_rowmat(const float* Y, const float* M, int n, int w, float* Q, hipStream_t st);

// ---- S build ----------------------------------------------------------------
// Z (Tp x ldz): standardised columns (c < n), zero padding; flags[0] |= 1 on a
// non-finite input, flags[1] |= 1 on a constant column.
hipError_t launch_standardize(const float* X, int T, int n, int64_t ldx, float* Z, int Tp,
                              int64_t ldz, int* flags, hipStream_t st);
hipError_t launch_tpdm_ranks(const float* X, int T, int n, int64_t ldx, int* R, int* hist,
                             int* flags, hipStream_t st);
hipError_t launch_tpdm_select(const int* hist, int T, int m, double* radius, int* sel,
                              hipStream_t st);
hipError_t launch_tpdm_theta(const int* R, int T, int n, const int* sel, const double* radius,
                             int m, int mp, float* Theta, int64_t ldz, hipStream_t st);
// S = scale * (|A^T A| if absval else A^T A), A = Z (Kp x ldz), upper-triangle
// tiles mirrored; part2[tile] = partial ||S||^2 (fp64). split: the bf16 matrix
// cores with exactly split operands, Kp % 32 == 0; otherwise fp32 MFMA,
// Kp % 4 == 0 (another Kp: hipErrorInvalidValue).
hipError_t launch_gram_build(const float* Z, int Kp, int64_t ldz, int n, float scale, int absval,
                             bool split, float* S, int64_t lds, double* part2,
                             int64_t* ntiles_out, hipStream_t st);
int64_t gram_build_tiles(int n);
hipError_t launch_sum_doubles(const double* part, int64_t count, double* out, hipStream_t st);

}  // namespace symnmf
