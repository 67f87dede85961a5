// The symmetric S.H pass: P = S H from the upper triangle of S alone. The
// S H products are the dominant cost of the fit (P1 "Factorization at scale"),
// and S = S^T by construction (P1 "The problem"), so every off-diagonal
// element can serve both of the products it takes part in.
//
// S is cut into 32 x 32 blocks; block (a, b) holds rows 32a..32a+31 and
// columns 32b..32b+31. The pass reads the blocks with a <= b, once each. A
// block with a < b adds
//     S_ab H_b     to rows 32a.. of P   (the row side)
//     S_ab^T H_a   to rows 32b.. of P   (the column side: S_ba = S_ab^T)
// and a diagonal block adds S_aa H_a only. For a symmetric S that is the full
// product, summed in another order; the off-diagonal half of S is never read.
//
// Both sides run on the bf16 matrix cores with exactly split fp32 operands
// (bf16split.h); H is packed once into B operands (sq_pack_q_kernel), whose K
// map over the rows of H serves both sides. Row side: lane l holds row l % 16
// of a 16-row subtile and the 8 columns 4g+e (e < 4), 16+4g+(e-4) (e >= 4),
// g = l / 16, of the block, straight from global memory (two float4 pieces per
// row). Column side: the matrix core contracts over the index held within a
// lane, which here has to be the row, so each wave writes the block's fp32
// values to an LDS area of its own and reads them back with the column along
// the lanes and the rows in the same K map.
//
// Work: strips of 512 columns (8 waves of 2 blocks), each walked down in
// chunks of 4096 rows. Workgroup (strip s, chunk q) covers rows
// [4096 q, min(4096 (q + 1), E_s)), E_s = min(n, 512 (s + 1)): the part of the
// strip on or above the diagonal. Per 32-row panel the four waves' row-side
// sums meet in LDS and leave as one partial P1[s][i] per (strip, row); the
// column side accumulates in registers over the chunk and leaves as
// P2[q][s][j] per (chunk, column). The fold adds, for row i of strip
// s(i) = i / 512,
//     sum over s = s(i) .. NS-1 of P1[s][i], then
//     sum over the chunks q of strip s(i) of P2[q][s(i)][i],
// in that fixed order, so the result does not depend on timing.
#include <algorithm>

#include "bf16split.h"
#include "common.h"
#include "kernels.h"

namespace symnmf {
namespace {

constexpr int kSymStripBlocks = kSymStrip / 32;  // 32-column blocks per strip
constexpr int kSymWaves = 8;                       // waves per workgroup
constexpr int kSymPitch = 36;  // floats per row of a wave's transpose area (16-byte rows,
                               // no bank conflicts for the column reads)

// rows of P1 held by the strips before strip s (each 512 (s' + 1) rows)
__host__ __device__ inline int64_t p1_rows_before(int s) {
    return (int64_t)(kSymStrip / 2) * s * (s + 1);
}

template <int NT, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void sym_kernel(const float* __restrict__ S, int64_t lds,
                                                  const u32x4* __restrict__ Hs, int n, int k,
                                                  float* __restrict__ P1, float* __restrict__ P2) {
    constexpr int WB = kSymStripBlocks / WAVES;  // column blocks per wave
    constexpr int NTH = 64 * WAVES;
    constexpr int HB = NT * 3 * 64;  // 16-byte pieces of one packed K block of H
    constexpr int HPER = (HB + NTH - 1) / NTH;
    __shared__ u32x4 hbuf[2][HB];
    __shared__ __attribute__((aligned(16))) float tbuf[WAVES][32 * kSymPitch];
    __shared__ floatx4 red[2][WAVES][2][NT][64];

    const int s = blockIdx.x;
    const int q = blockIdx.y;
    const int NS = gridDim.x;
    const int E = min(n, kSymStrip * (s + 1));
    const int r0 = kSymChunk * q;
    if (r0 >= E) return;  // the whole workgroup: no barrier is skipped by part of it
    const int r1 = min(E, r0 + kSymChunk);
    const int a0 = r0 >> 5;
    const int a1 = (r1 + 31) >> 5;
    const int nkb = (n + 31) >> 5;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int lr = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bw0 = s * kSymStripBlocks + wave * WB;  // first column block of the wave

    // row side B operands of the wave's column blocks, kept for the whole chunk
    u32x4 hj[WB][NT][3];
    // start of each float4 piece within a row; a piece that would start at
    // column >= n (ragged last block) reads the row's first 16 bytes instead,
    // and a block past n reads the last block, so no load sits in a branch;
    // compute zeroes what lies at columns >= n before use
    int coff[WB][2];
#pragma unroll
    for (int bb = 0; bb < WB; ++bb) {
        const int kb = min(bw0 + bb, nkb - 1);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int p = 0; p < 3; ++p) hj[bb][t][p] = Hs[((kb * NT + t) * 3 + p) * 64 + lane];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int col = 32 * kb + 16 * p + 4 * g;
            coff[bb][p] = col < n ? col : 0;
        }
    }

    typedef float Panel[WB][2][8];
    // panel a: rows 32a + 16 s2 + lr (rows past n read row n - 1, whose
    // products meet the zero rows of the packed H or are not stored)
    auto load = [&](int a, Panel& v) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const float* rp = S + (int64_t)min(32 * a + 16 * s2 + lr, n - 1) * lds;
#pragma unroll
            for (int bb = 0; bb < WB; ++bb)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const floatx4 t = __builtin_nontemporal_load(
                        reinterpret_cast<const floatx4*>(rp + coff[bb][p]));
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[bb][s2][4 * p + e] = t[e];
                }
        }
    };
    u32x4 hst[HPER];
    auto load_h = [&](int a) {
        const u32x4* src = Hs + (int64_t)min(a, nkb - 1) * HB;
#pragma unroll
        for (int m = 0; m < HPER; ++m) hst[m] = src[min(tid + NTH * m, HB - 1)];
    };
    auto store_h = [&](int buf) {
#pragma unroll
        for (int m = 0; m < HPER; ++m) {
            const int e = tid + NTH * m;
            if (HB % NTH == 0 || e < HB) hbuf[buf][e] = hst[m];
        }
    };

    floatx4 acc2[WB][2][NT];
#pragma unroll
    for (int bb = 0; bb < WB; ++bb)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc2[bb][u][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    float* __restrict__ tw = tbuf[wave];
    const int64_t p1base = p1_rows_before(s);

    auto compute = [&](int a, Panel& v) {
        const int hb = a & 1;
        u32x4 hi[NT][3];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int p = 0; p < 3; ++p) hi[t][p] = hbuf[hb][(3 * t + p) * 64 + lane];
        floatx4 acc1[2][NT];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc1[s2][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int bb = 0; bb < WB; ++bb) {
            const int b = bw0 + bb;
            if (b < nkb && a <= b) {
                if (32 * b + 32 > n) {
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int jc = 32 * b + (e < 4 ? 4 * g + e : 12 + 4 * g + e);
                            v[bb][s2][e] = jc < n ? v[bb][s2][e] : 0.f;
                        }
                }
                u32x4 x1[2], x2[2], x3[2];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) split3_8(v[bb][s2], x1[s2], x2[s2], x3[s2]);
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        acc1[s2][t] = mfma_split6(x1[s2], x2[s2], x3[s2], hj[bb][t][0],
                                                  hj[bb][t][1], hj[bb][t][2], acc1[s2][t]);
                if (a < b) {
                    // the block through LDS: written by rows, read by columns
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        float* rowp = tw + (16 * s2 + lr) * kSymPitch + 4 * g;
                        *reinterpret_cast<floatx4*>(rowp) =
                            floatx4{v[bb][s2][0], v[bb][s2][1], v[bb][s2][2], v[bb][s2][3]};
                        *reinterpret_cast<floatx4*>(rowp + 16) =
                            floatx4{v[bb][s2][4], v[bb][s2][5], v[bb][s2][6], v[bb][s2][7]};
                    }
                    float w[2][8];
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int row = e < 4 ? 4 * g + e : 12 + 4 * g + e;
                            w[u][e] = tw[row * kSymPitch + 16 * u + lr];
                        }
                    u32x4 y1[2], y2[2], y3[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) split3_8(w[u], y1[u], y2[u], y3[u]);
#pragma unroll
                    for (int t = 0; t < NT; ++t)
#pragma unroll
                        for (int u = 0; u < 2; ++u)
                            acc2[bb][u][t] = mfma_split6(y1[u], y2[u], y3[u], hi[t][0], hi[t][1],
                                                         hi[t][2], acc2[bb][u][t]);
                }
            }
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int t = 0; t < NT; ++t) red[hb][wave][s2][t][lane] = acc1[s2][t];
    };

    // the waves' row-side sums of panel a, in wave order, to P1
    auto reduce_rows = [&](int a) {
        const float* rf = reinterpret_cast<const float*>(&red[a & 1][0][0][0][0]);
        constexpr int WSTRIDE = 2 * NT * 64 * 4;  // floats per wave in red
        // a fixed trip count, no loop: a loop here makes the compiler wait for
        // every load in flight (the next panel's) before entering it
#pragma unroll
        for (int m = 0; m < (32 * 16 * NT + NTH - 1) / NTH; ++m) {
            const int o = tid + NTH * m;
            if (o >= 32 * k) break;
            const int rr = o / k;
            const int c = o - rr * k;
            const int i = 32 * a + rr;
            const int s2 = rr >> 4;
            const int gg = (rr >> 2) & 3;
            const int r = rr & 3;
            const int t = c >> 4;
            const int idx = ((s2 * NT + t) * 64 + 16 * gg + (c & 15)) * 4 + r;
            float sum = rf[idx];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) sum += rf[w * WSTRIDE + idx];
            if (i < n) P1[(p1base + i) * k + c] = sum;
        }
    };

    // One panel: issue the next panel's packed H rows and S, multiply this
    // one, stage the next H block, one barrier, then the row-side reduction.
    // Loads are issued on every path (clamped to the chunk's last panel), so
    // the compiler's wait counts stay tight; past the chunk's end only the
    // arithmetic is skipped.
    auto panel = [&](int a, Panel& cur, Panel& nxt) {
        const int an = min(a + 1, a1 - 1);
        load_h(an);  // first: waiting for it before the barrier leaves the S loads in flight
        load(an, nxt);
        if (a < a1) compute(a, cur);
        store_h((a + 1) & 1);  // that buffer was last read before the previous barrier
        __syncthreads();
        if (a < a1) reduce_rows(a);
    };

    Panel va, vb;
    load(a0, va);
    load_h(a0);
    store_h(a0 & 1);
    __syncthreads();
    for (int a = a0; a < a1; a += 2) {
        panel(a, va, vb);
        panel(a + 1, vb, va);
    }

    // column side of the chunk: lane l holds columns 16u + 4g + r of each
    // block, factor column 16t + l % 16
    float* __restrict__ dst = P2 + ((int64_t)q * NS + s) * kSymStrip * k;
#pragma unroll
    for (int bb = 0; bb < WB; ++bb)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int jl = (wave * WB + bb) * 32 + 16 * u + 4 * g + r;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int c = 16 * t + lr;
                    if (c < k) dst[(int64_t)jl * k + c] = acc2[bb][u][t][r];
                }
            }
}

// P[i][c] = sum over s >= i / 512 of P1[s][i][c], then over the chunks of
// strip i / 512 of P2[q][s(i)][i][c]; tr_part[b] = sum over the rows of block
// b of <Hdot_i, P_i> (fp64), blocks of kUpdRows rows.
__global__ __launch_bounds__(256) void sym_fold_kernel(const float* __restrict__ P1,
                                                       const float* __restrict__ P2, int n, int k,
                                                       int NS, float* __restrict__ P,
                                                       const float* __restrict__ Hdot,
                                                       double* __restrict__ tr_part) {
    __shared__ double redd[4];
    const int row0 = blockIdx.x * kUpdRows;
    const int rows = min(kUpdRows, n - row0);
    double acc = 0.0;
    for (int e = threadIdx.x; e < rows * k; e += 256) {
        const int i = row0 + e / k;
        const int c = e % k;
        const int si = i / kSymStrip;
        float sum = 0.f;
        int sp = si;
        for (; sp + 8 <= NS; sp += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = P1[(p1_rows_before(sp + u) + i) * k + c];
#pragma unroll
            for (int u = 0; u < 8; ++u) sum += v[u];
        }
        for (; sp < NS; ++sp) sum += P1[(p1_rows_before(sp) + i) * k + c];
        const int nch = (min(n, kSymStrip * (si + 1)) + kSymChunk - 1) / kSymChunk;
        const int64_t qstride = (int64_t)NS * kSymStrip * k;
        sum += ordered_strided_sum(
            P2 + ((int64_t)si * kSymStrip + (i - si * kSymStrip)) * k + c, nch, qstride);
        P[(int64_t)i * k + c] = sum;
        if (Hdot) acc += (double)Hdot[(int64_t)i * k + c] * (double)sum;
    }
    if (tr_part) {
        const double t = block_sum256(acc, redd);
        if (threadIdx.x == 0) tr_part[blockIdx.x] = t;
    }
}

}  // namespace

SymPlan sym_plan(int n, int k) {
    SymPlan p;
    p.nt = (k + 15) / 16;
    p.ns = (n + kSymStrip - 1) / kSymStrip;
    p.nq = (n + kSymChunk - 1) / kSymChunk;
    p.p1_floats = (size_t)(p1_rows_before(p.ns - 1) + n) * k;
    p.p2_floats = (size_t)p.nq * p.ns * kSymStrip * k;
    return p;
}

hipError_t launch_sym(const float* S, int64_t lds, const void* Hs, int n, int k,
                      const SymPlan& p, float* P1, float* P2, hipStream_t st) {
    const u32x4* h = static_cast<const u32x4*>(Hs);
    const dim3 grid((unsigned)p.ns, (unsigned)p.nq);
    const dim3 block(64 * kSymWaves);
    switch (p.nt) {
        case 1:
            hipLaunchKernelGGL((sym_kernel<1, kSymWaves>), grid, block, 0, st, S, lds, h, n, k, P1,
                               P2);
            break;
        case 2:
            hipLaunchKernelGGL((sym_kernel<2, kSymWaves>), grid, block, 0, st, S, lds, h, n, k, P1,
                               P2);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_sym_fold(const float* P1, const float* P2, int n, int k, const SymPlan& p,
                           float* P, const float* Hdot, double* tr_part, hipStream_t st) {
    const int nblk = (n + kUpdRows - 1) / kUpdRows;
    hipLaunchKernelGGL(sym_fold_kernel, dim3(nblk), dim3(256), 0, st, P1, P2, n, k, p.ns, P, Hdot,
                       tr_part);
    return hipGetLastError();
}

}  // namespace symnmf
