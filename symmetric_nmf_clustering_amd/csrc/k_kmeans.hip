// Spherical k-means on the L2-normalised rows of S (P1 "Spherical k-means for
// direct hard clustering": cosine similarity between rows of S; "Between
// spherical k-means and SymNMF": the hard-clustering baseline).
//
// With x_i = S[i,:] / ||S[i,:]|| and unit centroids c_j stored as the columns
// of C^T (n x k), the similarities <x_i, c_j> are (S C^T)[i, j] / ||S[i,:]||
// (S symmetric), so an assignment is the row argmax of one S.H pass, and the
// update c_j ~ sum_{i in j} x_i is C^T ~ S (D^-1 Z), a second S.H pass with
// the one-hot assignment matrix Z scaled by D^-1 = diag(1/||S[i,:]||). The
// kernels here are the small ones around those two passes.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace symnmf {

// rinv[i] = 1 / ||S[i, :]||_2 (0 for an all-zero row), the sum of squares in
// fp64. One wave per row, 16-byte loads (lds is a multiple of 4 and S is
// 16-byte aligned, so every row starts aligned).
__global__ __launch_bounds__(256) void row_norm_inv_kernel(const float* __restrict__ S,
                                                           int64_t lds, int n,
                                                           float* __restrict__ rinv) {
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= n) return;
    const float* row = S + i * lds;
    const int n4 = n >> 2;
    double acc = 0.0;
    for (int q = lane; q < n4; q += 64) {
        const float4 v = *reinterpret_cast<const float4*>(row + 4 * q);
        acc += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
    }
    for (int c = 4 * n4 + lane; c < n; c += 64) acc += (double)row[c] * row[c];
    acc = wave_sum(acc);
    if (lane == 0) rinv[i] = acc > 0.0 ? (float)(1.0 / sqrt(acc)) : 0.f;
}

hipError_t launch_row_norm_inv(const float* S, int64_t lds, int n, float* rinv, hipStream_t st) {
    hipLaunchKernelGGL(row_norm_inv_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, st, S,
                       lds, n, rinv);
    return hipGetLastError();
}

// Initial centroids: column j of C^T is row idx[j] of S scaled to unit length.
__global__ __launch_bounds__(256) void gather_centroids_kernel(const float* __restrict__ S,
                                                               int64_t lds, int n,
                                                               const int* __restrict__ idx,
                                                               const float* __restrict__ rinv,
                                                               int k, float* __restrict__ Ct) {
    const int j = blockIdx.y;
    const int64_t l = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (l >= n) return;
    const int r = idx[j];
    Ct[l * k + j] = S[(int64_t)r * lds + l] * rinv[r];
}

hipError_t launch_gather_centroids(const float* S, int64_t lds, int n, const int* idx,
                                   const float* rinv, int k, float* Ct, hipStream_t st) {
    hipLaunchKernelGGL(gather_centroids_kernel, dim3((unsigned)((n + 255) / 256), (unsigned)k),
                       dim3(256), 0, st, S, lds, n, idx, rinv, k, Ct);
    return hipGetLastError();
}

// Per block of 256 rows: the number of rows whose label changed (added to
// *changes) and the fp64 partial of sum_i <x_i, c_{label_i}> =
// sum_i rinv[i] * P[i, label_i] (the objective the iteration raises).
__global__ __launch_bounds__(256) void kmeans_assign_stats_kernel(
    const float* __restrict__ P, int n, int k, const int32_t* __restrict__ lab,
    const int32_t* __restrict__ lab_prev, const float* __restrict__ rinv,
    int* __restrict__ changes, double* __restrict__ obj_part) {
    __shared__ double red[4];
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    double v = 0.0;
    int ch = 0;
    if (i < n) {
        const int c = lab[i];
        v = (double)rinv[i] * (double)P[i * k + c];
        ch = c != lab_prev[i];
    }
    const double s = block_sum256(v, red);
    if (threadIdx.x == 0) obj_part[blockIdx.x] = s;
    // integer count: the order of the atomic additions does not change it
    const unsigned long long ballot = __ballot(ch);
    if ((threadIdx.x & 63) == 0 && ballot) atomicAdd(changes, __popcll(ballot));
}

hipError_t launch_kmeans_assign_stats(const float* P, int n, int k, const int32_t* lab,
                                      const int32_t* lab_prev, const float* rinv, int* changes,
                                      double* obj_part, hipStream_t st) {
    hipLaunchKernelGGL(kmeans_assign_stats_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256),
                       0, st, P, n, k, lab, lab_prev, rinv, changes, obj_part);
    return hipGetLastError();
}

// W = D^-1 Z: W[i, j] = rinv[i] if lab[i] == j else 0.
__global__ __launch_bounds__(256) void onehot_scaled_kernel(const int32_t* __restrict__ lab,
                                                            const float* __restrict__ rinv,
                                                            int n, int k, float* __restrict__ W) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)n * k) return;
    const int64_t i = e / k;
    const int j = (int)(e - i * k);
    W[e] = lab[i] == j ? rinv[i] : 0.f;
}

hipError_t launch_onehot_scaled(const int32_t* lab, const float* rinv, int n, int k, float* W,
                                hipStream_t st) {
    const int64_t count = (int64_t)n * k;
    hipLaunchKernelGGL(onehot_scaled_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                       st, lab, rinv, n, k, W);
    return hipGetLastError();
}

// Column sums of squares of C (n x k), fp64 partials per block of 256 rows:
// part[b * k + j]. Block (b, j) reduces column j over its 256 rows in a fixed
// order.
__global__ __launch_bounds__(256) void col_sumsq_kernel(const float* __restrict__ C, int n, int k,
                                                        double* __restrict__ part) {
    __shared__ double red[4];
    const int j = blockIdx.y;
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    double v = 0.0;
    if (r < n) {
        const double c = C[r * k + j];
        v = c * c;
    }
    v = block_sum256(v, red);
    if (threadIdx.x == 0) part[(int64_t)blockIdx.x * k + j] = v;
}

// norm[j] = sqrt(sum_b part[b * k + j]), blocks folded in order.
__global__ __launch_bounds__(64) void col_fold_kernel(const double* __restrict__ part, int nblk,
                                                      int k, double* __restrict__ norm) {
    const int j = threadIdx.x;
    if (j >= k) return;
    double s = 0.0;
    for (int b = 0; b < nblk; ++b) s += part[(int64_t)b * k + j];
    norm[j] = sqrt(s);
}

// Ct[:, j] = C[:, j] / norm[j]; a cluster left empty (norm 0) keeps its
// previous centroid.
__global__ __launch_bounds__(256) void col_scale_kernel(const float* __restrict__ C, int n, int k,
                                                        const double* __restrict__ norm,
                                                        float* __restrict__ Ct) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)n * k) return;
    const int j = (int)(e % k);
    const double nj = norm[j];
    if (nj > 0.0) Ct[e] = (float)((double)C[e] / nj);
}

hipError_t launch_normalize_columns(const float* C, int n, int k, double* part, double* norm,
                                    float* Ct, hipStream_t st) {
    const int nblk = (n + 255) / 256;
    hipLaunchKernelGGL(col_sumsq_kernel, dim3((unsigned)nblk, (unsigned)k), dim3(256), 0, st, C, n,
                       k, part);
    hipLaunchKernelGGL(col_fold_kernel, dim3(1), dim3(64), 0, st, part, nblk, k, norm);
    const int64_t count = (int64_t)n * k;
    hipLaunchKernelGGL(col_scale_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st,
                       C, n, k, norm, Ct);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_int_kernel(int32_t* __restrict__ p, int64_t count,
                                                       int32_t v) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e < count) p[e] = v;
}

hipError_t launch_fill_int(int32_t* p, int64_t count, int32_t v, hipStream_t st) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_int_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st,
                       p, count, v);
    return hipGetLastError();
}

}  // namespace symnmf
