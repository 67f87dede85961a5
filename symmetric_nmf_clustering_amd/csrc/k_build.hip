// S build: |Pearson correlation| and TPDM from a T x n returns window
// (P1 introduction: absolute Pearson correlation for broad co-movement, TPDM
// for joint behaviour in extreme observations; P3: TPDM from extreme value
// theory). Both end in one fp32 MFMA contraction S = scale * A^T A over a
// short K (T days, or the m extreme days), written once per upper-triangle
// tile and mirrored so that S is bitwise symmetric.
#include <math.h>

#include "bf16split.h"
#include "common.h"
#include "kernels.h"

namespace symnmf {

// ---- |corr|: column standardisation ----------------------------------------
// One thread per column (coalesced across threads: X is day-major). Mean and
// centred sum of squares in fp64; z = (x - mu)/sqrt(ss) so Z^T Z is the
// correlation matrix with no ddof convention.
__global__ __launch_bounds__(256) void standardize_kernel(const float* __restrict__ X, int T,
                                                          int n, int64_t ldx,
                                                          float* __restrict__ Z, int Tp,
                                                          int64_t ldz, int* flags) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= ldz) return;
    if (i >= n) {
        for (int t = 0; t < Tp; ++t) Z[(int64_t)t * ldz + i] = 0.f;
        return;
    }
    double s = 0.0;
    bool finite = true;
    for (int t = 0; t < T; ++t) {
        const float v = X[(int64_t)t * ldx + i];
        finite = finite && isfinite(v);
        s += (double)v;
    }
    if (!finite) {
        atomicOr(&flags[0], 1);
        for (int t = 0; t < Tp; ++t) Z[(int64_t)t * ldz + i] = 0.f;
        return;
    }
    const double mu = s / (double)T;
    double ss = 0.0;
    for (int t = 0; t < T; ++t) {
        const double d = (double)X[(int64_t)t * ldx + i] - mu;
        ss += d * d;
    }
    if (!(ss > 0.0)) {
        atomicOr(&flags[1], 1);
        for (int t = 0; t < Tp; ++t) Z[(int64_t)t * ldz + i] = 0.f;
        return;
    }
    const double inv = 1.0 / sqrt(ss);
    for (int t = 0; t < T; ++t)
        Z[(int64_t)t * ldz + i] = (float)(((double)X[(int64_t)t * ldx + i] - mu) * inv);
    for (int t = T; t < Tp; ++t) Z[(int64_t)t * ldz + i] = 0.f;
}

hipError_t launch_standardize(const float* X, int T, int n, int64_t ldx, float* Z, int Tp,
                              int64_t ldz, int* flags, hipStream_t st) {
    hipLaunchKernelGGL(standardize_kernel, dim3((unsigned)((ldz + 255) / 256)), dim3(256), 0, st,
                       X, T, n, ldx, Z, Tp, ldz, flags);
    return hipGetLastError();
}

// ---- TPDM -----------------------------------------------------------------------
// Ordinal rank of the loss -x_ti within column i: 1 + #{s : -x_si < -x_ti}
// + #{s < t : x_si == x_ti}, i.e. ties go to the earlier day. Each column's
// ranks are a permutation of 1..T. hist[t][R] counts the columns whose rank on
// day t is R; the day radius depends on the ranks only, so summing the
// histogram in rank order makes equal rank multisets give bitwise equal radii.
__global__ __launch_bounds__(256) void tpdm_ranks_kernel(const float* __restrict__ X, int T, int n,
                                                         int64_t ldx, int* __restrict__ R,
                                                         int* __restrict__ hist, int* flags) {
    // windows longer than the LDS stage: one thread per (day t, column i); the
    // column's losses are read from L2 (the same address across the wave)
    const int nbt = (T + 255) / 256;  // day blocks per column
    const int i = (int)(blockIdx.x / nbt);
    const int t = (int)(blockIdx.x % nbt) * 256 + threadIdx.x;
    if (i >= n || t >= T) return;
    const float lt = -X[(int64_t)t * ldx + i];
    if (!isfinite(lt)) {
        atomicOr(&flags[0], 1);  // the build stops with E_NONFINITE
        return;
    }
    int rank = 1;
    for (int s = 0; s < T; ++s) {
        const float ls = -X[(int64_t)s * ldx + i];
        rank += (ls < lt) || (ls == lt && s < t);
    }
    R[(int64_t)t * n + i] = rank;
    atomicAdd(&hist[(int64_t)t * (T + 1) + rank], 1);
}

// The same ranks with C columns of the window staged in LDS (losses, T x C):
// the T x C (day, column) pairs of a workgroup each count, against the staged
// column, the days with a smaller loss or an equal loss on an earlier day.
// Consecutive threads take consecutive columns, so the LDS reads of a wave
// fall in consecutive banks. A column with a non-finite value is skipped and
// flagged, as above.
constexpr int kRankLdsFloats = 16000;  // 62.5 KiB of losses per workgroup (+ 256 B of flags)

__global__ __launch_bounds__(256) void tpdm_ranks_lds_kernel(const float* __restrict__ X, int T,
                                                             int n, int64_t ldx, int C,
                                                             int* __restrict__ R,
                                                             int* __restrict__ hist, int* flags) {
    extern __shared__ float L[];  // L[s * C + c] = loss of day s, column i0 + c
    __shared__ int bad[64];
    const int i0 = blockIdx.x * C;
    const int cols = min(C, n - i0);
    const int tid = threadIdx.x;
    if (tid < C) bad[tid] = 0;
    __syncthreads();
    for (int e = tid; e < T * C; e += 256) {
        const int sday = e / C, c = e - (e / C) * C;
        float v = 0.f;
        if (c < cols) {
            v = -X[(int64_t)sday * ldx + i0 + c];
            if (!isfinite(v)) bad[c] = 1;
        }
        L[e] = v;
    }
    __syncthreads();
    if (tid < cols && bad[tid]) atomicOr(&flags[0], 1);
    for (int e = tid; e < T * C; e += 256) {
        const int t = e / C, c = e - (e / C) * C;
        if (c >= cols || bad[c]) continue;
        const float lt = L[e];
        int rank = 1;
        for (int sday = 0; sday < T; ++sday) {
            const float ls = L[sday * C + c];
            rank += (ls < lt) || (ls == lt && sday < t);
        }
        R[(int64_t)t * n + i0 + c] = rank;
        atomicAdd(&hist[(int64_t)t * (T + 1) + rank], 1);
    }
}

hipError_t launch_tpdm_ranks(const float* X, int T, int n, int64_t ldx, int* R, int* hist,
                             int* flags, hipStream_t st) {
    if (T <= kRankLdsFloats) {
        const int C = min(64, kRankLdsFloats / T);
        hipLaunchKernelGGL(tpdm_ranks_lds_kernel, dim3((unsigned)((n + C - 1) / C)), dim3(256),
                           (size_t)T * C * sizeof(float), st, X, T, n, ldx, C, R, hist, flags);
    } else {
        const int64_t blocks = (int64_t)((T + 255) / 256) * n;
        if (blocks > INT32_MAX) return hipErrorInvalidValue;
        hipLaunchKernelGGL(tpdm_ranks_kernel, dim3((unsigned)blocks), dim3(256), 0, st, X, T, n, ldx,
                           R, hist, flags);
    }
    return hipGetLastError();
}

// Frechet (alpha = 2) margin of rank R among T days: x^2 = -1/ln(R/(T+1)).
__device__ __forceinline__ double frechet_sq(int R, int T) {
    return -1.0 / log((double)R / (double)(T + 1));
}

// radius[t] = sqrt(sum_R hist[t][R] x(R)^2) in fp64, one wave per day: lane
// l sums R = 1 + l, 65 + l, ... in order, then the lanes are folded by a fixed
// xor tree, so days with equal rank histograms get bitwise equal radii.
__global__ __launch_bounds__(256) void tpdm_radius_kernel(const int* __restrict__ hist, int T,
                                                          double* __restrict__ radius) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= T) return;
    const int* h = hist + (int64_t)t * (T + 1);
    double s = 0.0;
    for (int Rk = 1 + lane; Rk <= T; Rk += 64) {
        const int c = h[Rk];
        if (c) s += (double)c * frechet_sq(Rk, T);
    }
    s = wave_sum(s);
    if (lane == 0) radius[t] = sqrt(s);
}

// The m largest radii (ties to the earlier day) fill sel[0..m) in descending
// radius: day t's position is the number of days ranked before it.
__global__ __launch_bounds__(256) void tpdm_select_kernel(const double* __restrict__ radius, int T,
                                                          int m, int* __restrict__ sel) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    const double rt = radius[t];
    int pos = 0;
    for (int s = 0; s < T; ++s) {
        const double rs = radius[s];
        pos += (rs > rt) || (rs == rt && s < t);
    }
    if (pos < m) sel[pos] = t;
}

hipError_t launch_tpdm_select(const int* hist, int T, int m, double* radius, int* sel,
                              hipStream_t st) {
    hipLaunchKernelGGL(tpdm_radius_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, hist, T,
                       radius);
    hipLaunchKernelGGL(tpdm_select_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st,
                       radius, T, m, sel);
    return hipGetLastError();
}

// Theta[p][i] = x(R[sel[p]][i]) / radius[sel[p]] for p < m; zero rows m..mp-1 and
// zero columns n..ldz-1.
__global__ __launch_bounds__(256) void tpdm_theta_kernel(const int* __restrict__ R, int T, int n,
                                                         const int* __restrict__ sel,
                                                         const double* __restrict__ radius, int m,
                                                         int mp, float* __restrict__ Theta,
                                                         int64_t ldz) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int p = blockIdx.y;
    if (i >= ldz) return;
    float v = 0.f;
    if (p < m && i < n) {
        const int t = min(max(sel[p], 0), T - 1);
        const int rk = R[(int64_t)t * n + i];
        v = (float)(sqrt(frechet_sq(rk, T)) / radius[t]);
    }
    Theta[(int64_t)p * ldz + i] = v;
}

hipError_t launch_tpdm_theta(const int* R, int T, int n, const int* sel, const double* radius,
                             int m, int mp, float* Theta, int64_t ldz, hipStream_t st) {
    dim3 grid((unsigned)((ldz + 255) / 256), (unsigned)mp);
    hipLaunchKernelGGL(tpdm_theta_kernel, grid, dim3(256), 0, st, R, T, n, sel, radius, m, mp,
                       Theta, ldz);
    return hipGetLastError();
}

// ---- MFMA Gram with mirrored upper-triangle tiles -------------------------------
// Workgroup tile 128 x 128 of S (waves 2 x 2, 64 x 64 each), tiles (I, J) with
// I <= J only. In the fp32 path, per 4-day step a lane loads one float4 of the A panel
// (day t0 + lane/16, columns i0 + 4 (lane%16) .. +3) and one of the B panel;
// element qa of the A float4 and qb of the B float4 feed MFMA tile (qa, qb),
// which owns S[i0 + 4 m + qa][j0 + 4 n + qb]. The result element r of tile
// (qa, qb) in lane l is S[i0 + 16 (l/16) + 4 r + qa][j0 + 4 (l%16) + qb]: for
// fixed (qa, r) the four qb tiles give a float4 along a row of S, and for
// fixed (qb, r) the four qa tiles give a float4 along a row of S^T, so both the
// tile and its mirror are written with 16-byte stores.
int64_t gram_build_tiles(int n) {
    const int64_t nt = (n + kGramTile - 1) / kGramTile;
    return nt * (nt + 1) / 2;
}

__device__ __forceinline__ void decode_upper(int64_t b, int& I, int& J) {
    // b = J (J + 1) / 2 + I with 0 <= I <= J
    int64_t j = (int64_t)((sqrt(8.0 * (double)b + 1.0) - 1.0) * 0.5);
    while (j * (j + 1) / 2 > b) --j;
    while ((j + 1) * (j + 2) / 2 <= b) ++j;
    J = (int)j;
    I = (int)(b - j * (j + 1) / 2);
}

// SPLIT: 32-day steps on the bf16 matrix cores with exactly split operands
// (bf16split.h; Kp % 32 == 0). Lane l = 16g + c loads, per step, the float4s
// of days 32 ks + 4 m + g (m = 0..7) at columns i0 + 4c .. +3 (A) and
// j0 + 4c .. +3 (B): element m of column 4c + q is element m of lane group g
// of a 16x16x32 operand, the same K order on both sides, so A's column q and
// B's column q' feed tile (q, q') with its result in the same lanes as the
// fp32 path's. Six products per operand pair (fp32-exact), against 32 fp32
// 16x16x4 steps per 32 days in the fp32 path.
template <bool SPLIT>
__global__ __launch_bounds__(256) void gram_build_kernel(const float* __restrict__ Z, int Kp,
                                                         int64_t ldz, int n, float scale,
                                                         int absval, float* __restrict__ S,
                                                         int64_t lds, int64_t ntiles,
                                                         int64_t chunk,
                                                         double* __restrict__ part2) {
    // XCD-aware order: consecutive workgroups go to different XCDs, so give
    // each XCD a contiguous run of tiles (they share Z panels through its L2).
    const int64_t b = (int64_t)(blockIdx.x % 8) * chunk + blockIdx.x / 8;
    __shared__ double red[4];
    __shared__ floatx4 mir[4][64 * 16];  // per wave: a 64 x 64 tile of S^T (16 KiB)
    if (b >= ntiles) return;
    int I, J;
    decode_upper(b, I, J);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wi = wave >> 1, wj = wave & 1;
    const int i0 = I * kGramTile + wi * 64;
    const int j0 = J * kGramTile + wj * 64;
    const bool diag_tile = (I == J);
    const bool active = !(diag_tile && wi > wj);  // below-diagonal wave of a diagonal tile
    const bool diag_wave = diag_tile && wi == wj;
    const int r = lane >> 4;
    const int cl = lane & 15;

    double fro = 0.0;
    if (active) {
        floatx4 acc[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[a][c] = floatx4{0.f, 0.f, 0.f, 0.f};
        if constexpr (SPLIT) {
            const float* Ap = Z + (int64_t)r * ldz + i0 + 4 * cl;
            const float* Bp = Z + (int64_t)r * ldz + j0 + 4 * cl;
            floatx4 ra[8], rb[8];
            auto load = [&](int ks) {
                const int64_t off = (int64_t)32 * ks * ldz;
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    ra[m] = *reinterpret_cast<const floatx4*>(Ap + off + (int64_t)4 * m * ldz);
                    rb[m] = *reinterpret_cast<const floatx4*>(Bp + off + (int64_t)4 * m * ldz);
                }
            };
            const int nks = Kp / 32;
            load(0);
            for (int ks = 0; ks < nks; ++ks) {
                u32x4 ya[4][3], yb[4][3];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float ca[8], cb[8];
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        ca[m] = ra[m][q];
                        cb[m] = rb[m][q];
                    }
                    split3_8(ca, ya[q][0], ya[q][1], ya[q][2]);
                    split3_8(cb, yb[q][0], yb[q][1], yb[q][2]);
                }
                load(min(ks + 1, nks - 1));  // the next step's days, in flight during the products
#pragma unroll
                for (int qa = 0; qa < 4; ++qa)
#pragma unroll
                    for (int qb = 0; qb < 4; ++qb)
                        acc[qa][qb] = mfma_split6(ya[qa][0], ya[qa][1], ya[qa][2], yb[qb][0],
                                                  yb[qb][1], yb[qb][2], acc[qa][qb]);
            }
        } else {
            const float* Ap = Z + i0 + 4 * cl;
            const float* Bp = Z + j0 + 4 * cl;
            for (int t0 = 0; t0 < Kp; t0 += 4) {
                const int64_t off = (int64_t)(t0 + r) * ldz;
                const float4 av = *reinterpret_cast<const float4*>(Ap + off);
                const float4 bv = *reinterpret_cast<const float4*>(Bp + off);
                const float a4[4] = {av.x, av.y, av.z, av.w};
                const float b4[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                for (int qa = 0; qa < 4; ++qa)
#pragma unroll
                    for (int qb = 0; qb < 4; ++qb)
                        acc[qa][qb] = mfma16x16x4(a4[qa], b4[qb], acc[qa][qb]);
            }
        }
#pragma unroll
        for (int qa = 0; qa < 4; ++qa)
#pragma unroll
            for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v = acc[qa][qb][e] * scale;
                    acc[qa][qb][e] = absval ? fabsf(v) : v;
                }

        if (!diag_wave) {
            // off-diagonal block: every element written twice (S and S^T)
            const int jj = j0 + 4 * cl;
#pragma unroll
            for (int qa = 0; qa < 4; ++qa)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = i0 + 16 * r + 4 * e + qa;
                    const float4 v = {acc[qa][0][e], acc[qa][1][e], acc[qa][2][e], acc[qa][3][e]};
                    if (i < n) {
                        float* dst = S + (int64_t)i * lds + jj;
                        if (jj + 4 <= n) {
                            *reinterpret_cast<float4*>(dst) = v;
                        } else {
                            if (jj < n) dst[0] = v.x;
                            if (jj + 1 < n) dst[1] = v.y;
                            if (jj + 2 < n) dst[2] = v.z;
                        }
                        if (jj < n) fro += 2.0 * (double)v.x * v.x;
                        if (jj + 1 < n) fro += 2.0 * (double)v.y * v.y;
                        if (jj + 2 < n) fro += 2.0 * (double)v.z * v.z;
                        if (jj + 3 < n) fro += 2.0 * (double)v.w * v.w;
                    }
                }
            // the mirror S^T of the block, turned in the wave's LDS tile: lane
            // (r, cl) puts the float4 of rows i0 + 16 r + 4 e .. +3 of column
            // j0 + 4 cl + qb into tile row 4 cl + qb, 16-byte slot 4 r + e, and
            // tile rows come back whole, so each store writes 256 contiguous
            // bytes of four rows of S (written straight from the lanes, a
            // store covered 64 bytes of each of 16 rows, which cost a third of
            // the build). Slot s of tile row t sits at s ^ (t / 4): the 16
            // lanes of a write and of a read each touch 16 bank groups.
            floatx4* const tile = mir[wave];
#pragma unroll
            for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    tile[(4 * cl + qb) * 16 + ((4 * r + e) ^ cl)] =
                        floatx4{acc[0][qb][e], acc[1][qb][e], acc[2][qb][e], acc[3][qb][e]};
            wave_lds_sync();
            const int ic = i0 + 4 * cl;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int j = j0 + 4 * t + r;
                const floatx4 v = tile[(4 * t + r) * 16 + (cl ^ t)];
                if (j < n) {
                    float* dst = S + (int64_t)j * lds + ic;
                    if (ic + 4 <= n) {
                        *reinterpret_cast<floatx4*>(dst) = v;
                    } else {
                        if (ic < n) dst[0] = v[0];
                        if (ic + 1 < n) dst[1] = v[1];
                        if (ic + 2 < n) dst[2] = v[2];
                    }
                }
            }
        } else {
            // diagonal block: element (i, j) with i <= j is written at (i, j)
            // and, for i < j, mirrored to (j, i); i > j is left to its mirror
#pragma unroll
            for (int qa = 0; qa < 4; ++qa)
#pragma unroll
                for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = i0 + 16 * r + 4 * e + qa;
                        const int j = j0 + 4 * cl + qb;
                        if (i <= j && j < n) {
                            const float v = acc[qa][qb][e];
                            S[(int64_t)i * lds + j] = v;
                            if (i < j) {
                                S[(int64_t)j * lds + i] = v;
                                fro += 2.0 * (double)v * v;
                            } else {
                                fro += (double)v * v;
                            }
                        }
                    }
        }
    }
    const double tot = block_sum256(fro, red);
    if (threadIdx.x == 0) part2[b] = tot;
}

hipError_t launch_gram_build(const float* Z, int Kp, int64_t ldz, int n, float scale, int absval,
                             bool split, float* S, int64_t lds, double* part2,
                             int64_t* ntiles_out, hipStream_t st) {
    if (Kp % (split ? 32 : 4)) return hipErrorInvalidValue;
    const int64_t ntiles = gram_build_tiles(n);
    const int64_t chunk = (ntiles + 7) / 8;
    if (ntiles_out) *ntiles_out = ntiles;
    if (split)
        hipLaunchKernelGGL(gram_build_kernel<true>, dim3((unsigned)(chunk * 8)), dim3(256), 0, st,
                           Z, Kp, ldz, n, scale, absval, S, lds, ntiles, chunk, part2);
    else
        hipLaunchKernelGGL(gram_build_kernel<false>, dim3((unsigned)(chunk * 8)), dim3(256), 0, st,
                           Z, Kp, ldz, n, scale, absval, S, lds, ntiles, chunk, part2);
    return hipGetLastError();
}

// Fixed-order sum of `count` doubles (one workgroup).
__global__ __launch_bounds__(256) void sum_doubles_kernel(const double* __restrict__ part,
                                                          int64_t count, double* __restrict__ out) {
    __shared__ double red[4];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < count; i += 256) s += part[i];
    s = block_sum256(s, red);
    if (threadIdx.x == 0) *out = s;
}
hipError_t launch_sum_doubles(const double* part, int64_t count, double* out, hipStream_t st) {
    hipLaunchKernelGGL(sum_doubles_kernel, dim3(1), dim3(256), 0, st, part, count, out);
    return hipGetLastError();
}

}  // namespace symnmf
