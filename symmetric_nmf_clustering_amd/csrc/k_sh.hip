// The tall-skinny S.H pass (P1 "Factorization at scale": the dominant S H
// products; P2 AdaptGrow sketch: S @ H in every full-batch step).
//
// Layout and mapping (gfx950, wave64, fp32 MFMA 16x16x4):
//  * S is row-major and symmetric, so (S X)[i][c] = sum_j S[j][i] X[j][c]: the
//    pass streams contiguous ROW panels of S and produces output columns.
//  * A workgroup (4 waves) owns 256 consecutive columns i of S and one split
//    (a set of rows j). Each lane loads one float4 of S per 4-row group:
//    row j0 + (lane / 16), columns i0 + 4 (lane % 16) .. +3, so the four rows
//    of a group are each read as 256 contiguous bytes per wave (1 KiB per
//    workgroup).
//  * Element q of the float4 feeds MFMA tile q as its B operand, so tile q
//    owns output columns i0 + 4 n + q (n = 0..15); the A operand is X^T for 16
//    columns of X (c-tile), taken straight from L1/L2 (X is small and reused by
//    every column tile of a split).
//  * Each output (i, c) accumulates one split's rows in fp32 (a few thousand
//    terms at most), and splits are summed later in a fixed order, so the
//    result is deterministic and its rounding error stays ~1e-6 relative.
//  * Block b of the 1-D grid takes split b % nsplit and column tile
//    b / nsplit; with nsplit a multiple of 8, every workgroup of a split lands
//    on the same XCD, so that split's rows of X stay in one L2.
#include "common.h"
#include "kernels.h"

namespace symnmf {

// Row segment `g` of split `s` (at most rp.bps segments); false when none.
__device__ __forceinline__ bool split_segment(const RowPlan& rp, int s, int g, int& jb, int& je) {
    if (rp.blocks == nullptr) {
        if (g > 0) return false;
        jb = s * rp.rows_per_split;
        je = min(rp.n, jb + rp.rows_per_split);
    } else if (rp.sub > 1) {
        if (g > 0) return false;
        const int blk = rp.blocks[s / rp.sub];
        const int base = blk * rp.block_rows;
        const int bend = min(rp.n, base + rp.block_rows);
        jb = base + (s % rp.sub) * rp.seg;
        je = min(bend, jb + rp.seg);
    } else {
        const int idx = s * rp.bps + g;
        if (g >= rp.bps || idx >= rp.nsel) return false;
        const int blk = rp.blocks[idx];
        jb = blk * rp.block_rows;
        je = min(rp.n, jb + rp.block_rows);
    }
    if (jb > je) jb = je;
    return true;
}

template <int NC, bool DIFF>
__global__ __launch_bounds__(256) void sh_panel_kernel(const float* __restrict__ S, int64_t lds,
                                                       const float* __restrict__ X,
                                                       const float* __restrict__ Xa, int width,
                                                       RowPlan rp, int nsplit,
                                                       float* __restrict__ part, int ldp) {
    const int split = blockIdx.x % nsplit;
    const int tile = blockIdx.x / nsplit;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane >> 4;   // row of the 4-row group this lane loads
    const int cl = lane & 15;  // column quad / MFMA row index
    const int n = rp.n;
    const int col = tile * kShTileCols + wave * 64 + 4 * cl;

    floatx4 acc[NC][4];
#pragma unroll
    for (int ct = 0; ct < NC; ++ct)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[ct][q] = floatx4{0.f, 0.f, 0.f, 0.f};

    const bool colok = col < n;
    const bool colfull = col + 4 <= n;
    const float* __restrict__ Sc = S + col;

    int jb, je;
    for (int g = 0; split_segment(rp, split, g, jb, je); ++g) {
    constexpr int U = 4;  // 4-row groups per main-loop trip (16 rows)
    int j0 = jb;
    for (; j0 + 4 * U <= je; j0 += 4 * U) {
        float4 sv[U];
        float av[U][NC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + 4 * u + r;
            if (colok) {
                sv[u] = *reinterpret_cast<const float4*>(Sc + (int64_t)j * lds);
            } else {
                sv[u] = float4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ct = 0; ct < NC; ++ct) {
                const int c = 16 * ct + cl;
                float v = 0.f;
                if (c < width) {
                    v = X[(int64_t)j * width + c];
                    if (DIFF) v -= Xa[(int64_t)j * width + c];
                }
                av[u][ct] = v;
            }
        }
        if (!colfull) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (col + 1 >= n) sv[u].y = 0.f;
                if (col + 2 >= n) sv[u].z = 0.f;
                if (col + 3 >= n) sv[u].w = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int ct = 0; ct < NC; ++ct) {
                acc[ct][0] = mfma16x16x4(av[u][ct], sv[u].x, acc[ct][0]);
                acc[ct][1] = mfma16x16x4(av[u][ct], sv[u].y, acc[ct][1]);
                acc[ct][2] = mfma16x16x4(av[u][ct], sv[u].z, acc[ct][2]);
                acc[ct][3] = mfma16x16x4(av[u][ct], sv[u].w, acc[ct][3]);
            }
        }
    }
    // ragged tail: groups with rows past the split end contribute zeros
    for (; j0 < je; j0 += 4) {
        const int j = j0 + r;
        const bool ok = j < je;
        float4 s4 = float4{0.f, 0.f, 0.f, 0.f};
        if (ok && colok) s4 = *reinterpret_cast<const float4*>(Sc + (int64_t)j * lds);
        if (!colfull) {
            if (col + 1 >= n) s4.y = 0.f;
            if (col + 2 >= n) s4.z = 0.f;
            if (col + 3 >= n) s4.w = 0.f;
        }
        float av[NC];
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            const int c = 16 * ct + cl;
            float v = 0.f;
            if (ok && c < width) {
                v = X[(int64_t)j * width + c];
                if (DIFF) v -= Xa[(int64_t)j * width + c];
            }
            av[ct] = v;
        }
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            acc[ct][0] = mfma16x16x4(av[ct], s4.x, acc[ct][0]);
            acc[ct][1] = mfma16x16x4(av[ct], s4.y, acc[ct][1]);
            acc[ct][2] = mfma16x16x4(av[ct], s4.z, acc[ct][2]);
            acc[ct][3] = mfma16x16x4(av[ct], s4.w, acc[ct][3]);
        }
    }
    }  // segments

    // lane holds, for tile (ct, q), output columns c = 16 ct + 4 r + 0..3 of
    // row i = col + q: one aligned float4 store each.
    float* __restrict__ dst = part + (int64_t)split * ((int64_t)n * ldp);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = col + q;
        if (i < n) {
#pragma unroll
            for (int ct = 0; ct < NC; ++ct) {
                const int c0 = 16 * ct + 4 * r;
                if (c0 < ldp) {
                    const floatx4 v = acc[ct][q];
                    *reinterpret_cast<float4*>(dst + (int64_t)i * ldp + c0) =
                        float4{v[0], v[1], v[2], v[3]};
                }
            }
        }
    }
}

template <int NC>
static hipError_t launch_sh_nc(const float* S, int64_t lds, const float* X, const float* Xa,
                               int width, const RowPlan& rp, int nsplit, float* part, int ldp,
                               hipStream_t st) {
    const int ntiles = (rp.n + kShTileCols - 1) / kShTileCols;
    dim3 grid((unsigned)ntiles * (unsigned)nsplit);
    if (Xa)
        hipLaunchKernelGGL((sh_panel_kernel<NC, true>), grid, dim3(256), 0, st, S, lds, X, Xa,
                           width, rp, nsplit, part, ldp);
    else
        hipLaunchKernelGGL((sh_panel_kernel<NC, false>), grid, dim3(256), 0, st, S, lds, X,
                           nullptr, width, rp, nsplit, part, ldp);
    return hipGetLastError();
}

hipError_t launch_sh_panel(const float* S, int64_t lds, const float* X, const float* Xa,
                           int width, const RowPlan& rp, int nsplit, float* part, int ldp,
                           hipStream_t st) {
    const int nc = (width + 15) / 16;
    switch (nc) {
        case 1: return launch_sh_nc<1>(S, lds, X, Xa, width, rp, nsplit, part, ldp, st);
        case 2: return launch_sh_nc<2>(S, lds, X, Xa, width, rp, nsplit, part, ldp, st);
        case 3: return launch_sh_nc<3>(S, lds, X, Xa, width, rp, nsplit, part, ldp, st);
        case 4: return launch_sh_nc<4>(S, lds, X, Xa, width, rp, nsplit, part, ldp, st);
        case 5: return launch_sh_nc<5>(S, lds, X, Xa, width, rp, nsplit, part, ldp, st);
        case 6: return launch_sh_nc<6>(S, lds, X, Xa, width, rp, nsplit, part, ldp, st);
        case 7: return launch_sh_nc<7>(S, lds, X, Xa, width, rp, nsplit, part, ldp, st);
        case 8: return launch_sh_nc<8>(S, lds, X, Xa, width, rp, nsplit, part, ldp, st);
        default: return hipErrorInvalidValue;
    }
}

// P = sum of the split partials in split order; optional fp64 <Hdot, P> per block.
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ part,
                                                              int nsplit, int n, int width,
                                                              int ldp, float* __restrict__ P,
                                                              const float* __restrict__ Hdot,
                                                              double* __restrict__ tr_part) {
    __shared__ double red[4];
    const int row0 = blockIdx.x * kUpdRows;
    const int rows = min(kUpdRows, n - row0);
    const int64_t pstride = (int64_t)n * ldp;
    double acc = 0.0;
    for (int e = threadIdx.x; e < rows * width; e += 256) {
        const int i = row0 + e / width;
        const int c = e % width;
        const float* p = part + (int64_t)i * ldp + c;
        float s = 0.f;
        for (int sp = 0; sp < nsplit; ++sp) s += p[sp * pstride];
        P[(int64_t)i * width + c] = s;
        if (Hdot) acc += (double)Hdot[(int64_t)i * width + c] * (double)s;
    }
    if (tr_part) {
        const double t = block_sum256(acc, red);
        if (threadIdx.x == 0) tr_part[blockIdx.x] = t;
    }
}

hipError_t launch_reduce_partials(const float* part, int nsplit, int n, int width, int ldp,
                                  float* P, const float* Hdot, double* tr_part, hipStream_t st) {
    const int nblk = (n + kUpdRows - 1) / kUpdRows;
    hipLaunchKernelGGL(reduce_partials_kernel, dim3(nblk), dim3(256), 0, st, part, nsplit, n,
                       width, ldp, P, Hdot, tr_part);
    return hipGetLastError();
}

}  // namespace symnmf
