// The symmetric S.H pass: P = S H from the upper triangle of S alone. The
// S H products are the dominant cost of the fit (P1 "Factorization at scale"),
// and S = S^T by definition (P1 introduction: S is an absolute Pearson
// correlation or a tail pairwise dependence matrix, both symmetric in i, j), so
// every off-diagonal element can serve both of the products it takes part in.
//
// S is cut into 32 x 32 blocks; block (a, b) holds rows 32a..32a+31 and
// columns 32b..32b+31. The pass uses the blocks with a <= b, once each. A
// block with a < b adds
//     S_ab H_b     to rows 32a.. of P   (the row side)
//     S_ab^T H_a   to rows 32b.. of P   (the column side: S_ba = S_ab^T)
// and a diagonal block adds S_aa H_a only. For a symmetric S that is the full
// product, summed in another order; the off-diagonal half of S is not needed.
//
// Both sides run on the bf16 matrix cores with exactly split fp32 operands
// (bf16split.h). A wave owns 64 columns c0..c0+63 and reads a 32-row panel of
// them as 8 float4 loads: load m gives lane l = 16g + c (g = l / 16) the four
// columns c0 + 4c + q (q = 0..3) of row 4m + g, so each load instruction reads
// 256 contiguous bytes of 4 rows (the pattern that streams fastest).
//  * Column side: for fixed q the panel is a matrix-core B operand as loaded:
//    column c0 + 4c + q along the lanes, the 32 rows within them (row 4e + g
//    is element e of lane group g). A = H^T of the panel's rows in that K map
//    (packed once, "column map"); the result lands as Z[column][factor].
//  * Row side: the matrix core contracts over the index held within a lane,
//    which here has to be the column. Multiplying each bf16 part (taken as an
//    A operand) by a 0/1 selector on the matrix core returns it with the row
//    along the lanes and 16 consecutive columns within each lane group, exactly
//    (one nonzero term per output). The 64 columns then form two K blocks,
//    columns c0 + 16g + 8h + e for half h; H's rows are packed in that map
//    ("row map"), once per pass.
//
// The row-side products run as D^T = H^T (factor x column) times the parts
// (column x row), so a lane ends with four consecutive factors of one row: the
// per-panel sum over the eight waves is then one float2 per thread and one
// store per thread (see reduce_rows).
//
// Work: strips of 512 columns (8 waves), each walked down in chunks of 4096
// rows. Workgroup (strip s, chunk qc) covers rows [4096 qc, min(4096 (qc+1),
// E_s)), E_s = min(n, 512 (s + 1)): the part of the strip on or above the
// diagonal. Per 32-row panel the eight waves' row-side sums meet in LDS and
// leave as one partial P1[s][i] per (strip, row; rows of p1_ld(k) floats);
// the column side accumulates
// in registers over the chunk and leaves as P2[qc][s][j] per (chunk, column).
// The fold adds, for row i of strip s(i) = i / 512,
//     sum over s = s(i) .. NS-1 of P1[s][i], then
//     sum over the chunks qc of strip s(i) of P2[qc][s(i)][i],
// in that fixed order, so the result does not depend on timing.
#include <algorithm>

#include "bf16split.h"
#include "common.h"
#include "kernels.h"

namespace symnmf {
namespace {

constexpr int kSymWaves = kSymStrip / 64;  // waves per workgroup, 64 columns each

// rows of P1 held by the strips before strip s (each 512 (s' + 1) rows)
__host__ __device__ inline int64_t p1_rows_before(int s) {
    return (int64_t)(kSymStrip / 2) * s * (s + 1);
}
// row pitch of P1: the row-side sums are stored as float2 pairs of factors
__host__ __device__ inline int p1_ld(int k) { return (k + 3) / 4 * 4; }
// floats of the store sink after P1 (one float2 per thread of a workgroup)
constexpr int kSymSinkFloats = 2 * 64 * kSymWaves;

// (a, b) -> the bf16 pair of two fp32 values that are bf16-exact (their high
// halves; a in the low half, as the matrix core reads a pair)
__device__ __forceinline__ uint32_t pack_hi(float a, float b) {
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a),
                                 0x07060302u);
}

// H (n x k, ld k) -> B/A operands of every 32-row K block kb, 16-column tile t
// and part p at out[((kb * NT + t) * 3 + p) * 64 + l], lane l = 16g + c holding
// H[row(kb, g, e)][16t + c], e = 0..7, split exactly into three bf16 parts:
//   column map: row = 32 kb + 4e + g
//   row map:    row = 64 (kb / 2) + 16g + 8 (kb % 2) + e
// Rows >= n and columns >= k are zero.
__global__ __launch_bounds__(256) void sym_pack_kernel(const float* __restrict__ H, int n, int k,
                                                       int NT, int nkb, int rowmap,
                                                       u32x4* __restrict__ out,
                                                       const int* __restrict__ done) {
    if (done && *done) return;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)nkb * NT * 64) return;
    const int lane = (int)(t & 63);
    const int64_t kt = t >> 6;
    const int tile = (int)(kt % NT);
    const int kb = (int)(kt / NT);
    const int g = lane >> 4;
    const int c = 16 * tile + (lane & 15);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int row = rowmap ? 64 * (kb >> 1) + 16 * g + 8 * (kb & 1) + e : 32 * kb + 4 * e + g;
        v[e] = (row < n && c < k) ? H[(int64_t)row * k + c] : 0.f;
    }
    u32x4 x1, x2, x3;
    split3_8(v, x1, x2, x3);
    u32x4* dst = out + kt * 3 * 64 + lane;
    dst[0] = x1;
    dst[64] = x2;
    dst[128] = x3;
}

template <int NT>
__global__ __launch_bounds__(64 * kSymWaves) void sym_kernel(
    const float* __restrict__ S, int64_t lds, const u32x4* __restrict__ HsR,
    const u32x4* __restrict__ HsC, int n, int k, float* __restrict__ P1, float* __restrict__ P2,
    const int* __restrict__ done) {
    if (done && *done) return;  // uniform over the workgroup, before any barrier
    constexpr int WAVES = kSymWaves;
    constexpr int NTH = 64 * WAVES;
    constexpr int HB = NT * 3 * 64;  // 16-byte pieces of one packed K block of H
    constexpr int HPER = (HB + NTH - 1) / NTH;
    __shared__ u32x4 hbuf[2][HB];
    __shared__ floatx4 red[2][WAVES][2][NT][64];

    const int s = blockIdx.x;
    const int qc = blockIdx.y;
    const int NS = gridDim.x;
    const int E = min(n, kSymStrip * (s + 1));
    const int r0 = kSymChunk * qc;
    if (r0 >= E) return;  // the whole workgroup: no barrier is skipped by part of it
    const int r1 = min(E, r0 + kSymChunk);
    const int a0 = r0 >> 5;
    const int a1 = (r1 + 31) >> 5;
    const int nkb = (n + 31) >> 5;
    const int ngr = (n + 63) >> 6;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int lr = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c0 = s * kSymStrip + 64 * wave;  // first column of the wave
    const int b0 = c0 >> 5;                    // its first 32-column block
    const bool active = c0 < n;

    // row side B operands (row map) of the wave's two K blocks, for the chunk
    u32x4 hj[2][NT][3];
    {
        const int G = min(c0 >> 6, ngr - 1);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    hj[h][t][p] = HsR[(((2 * G + h) * NT + t) * 3 + p) * 64 + lane];
    }
    // sel[rho]: picks row 16 rho + lr of a panel in the column map (row 4e + g
    // is element e of lane group g): bf16 1.0 at element 4 rho + lr / 4 of lane
    // group lr % 4, zero elsewhere
    u32x4 sel[2];
#pragma unroll
    for (int rho = 0; rho < 2; ++rho)
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            const int e = 4 * rho + (lr >> 2);
            const bool hit = g == (lr & 3) && (e >> 1) == w2;
            sel[rho][w2] = hit ? (e & 1 ? 0x3F800000u : 0x00003F80u) : 0u;
        }
    // a float4 that would start at column >= n (ragged edge, or a wave past n)
    // reads the row's first 16 bytes instead, so no load sits in a branch; the
    // values at columns >= n are zeroed before use. A float4 starting below n
    // lies inside the row (lds is a multiple of 4).
    const int col = c0 + 4 * lr;
    const int coff = col < n ? col : 0;

    typedef floatx4 Panel[8];
    auto load = [&](int a, Panel& v) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float* rp = S + (int64_t)min(32 * a + 4 * m + g, n - 1) * lds + coff;
            v[m] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(rp));
        }
    };
    u32x4 hst[HPER];
    auto load_h = [&](int a) {
        const u32x4* src = HsC + (int64_t)min(a, nkb - 1) * HB;
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

    floatx4 acc2[4][NT];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc2[q][t] = floatx4{0.f, 0.f, 0.f, 0.f};
    const int64_t p1base = p1_rows_before(s);

    auto compute = [&](int a, Panel& v) {
        const int hb = a & 1;
        floatx4 acc1[2][NT];
#pragma unroll
        for (int rho = 0; rho < 2; ++rho)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc1[rho][t] = floatx4{0.f, 0.f, 0.f, 0.f};
        // lanes lr < 8 hold block b0, lanes lr >= 8 block b0 + 1. Row side:
        // blocks b >= a; column side: blocks b > a. Both skip columns >= n.
        if (active && a <= b0 + 1) {
            if (a == b0 + 1 || c0 + 64 > n) {
                const bool keep_blk = a <= b0 + (lr >> 3);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const bool keep = keep_blk && col + q < n;
#pragma unroll
                    for (int m = 0; m < 8; ++m) v[m][q] = keep ? v[m][q] : 0.f;
                }
            }
            // the parts, as column side B operands: y[q][p] element e of lane
            // group g = part p of row 4e + g, column c0 + 4 lr + q
            u32x4 y[4][3];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float col8[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) col8[m] = v[m][q];
                split3_8(col8, y[q][0], y[q][1], y[q][2]);
            }
            if (a <= b0) {
                const bool ck = a < b0 + (lr >> 3);  // the diagonal block is row side only
                const u32x4* hl = &hbuf[hb][lane];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    u32x4 z1 = y[q][0], z2 = y[q][1], z3 = y[q][2];
                    if (a == b0) {
                        z1 = ck ? z1 : u32x4{0u, 0u, 0u, 0u};
                        z2 = ck ? z2 : u32x4{0u, 0u, 0u, 0u};
                        z3 = ck ? z3 : u32x4{0u, 0u, 0u, 0u};
                    }
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        acc2[q][t] = mfma_split6(hl[(3 * t) * 64], hl[(3 * t + 1) * 64],
                                                 hl[(3 * t + 2) * 64], z1, z2, z3, acc2[q][t]);
                }
            }
            // row side, one part at a time (smallest first): the part with the
            // row along the lanes, then its terms of the six-term product
#pragma unroll
            for (int p = 2; p >= 0; --p) {
#pragma unroll
                for (int rho = 0; rho < 2; ++rho) {
                    floatx4 d[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        d[q] = mfma_bf16(y[q][p], sel[rho], floatx4{0.f, 0.f, 0.f, 0.f});
                    // lane (lr, g') now holds part p of row 32a + 16 rho + lr,
                    // columns c0 + 16 g' + 4 r + q in d[q][r]; K block h takes
                    // columns c0 + 16 g' + 8 h + e, e = 4 (r - 2h) + q
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const u32x4 ap = {pack_hi(d[0][2 * h], d[1][2 * h]),
                                          pack_hi(d[2][2 * h], d[3][2 * h]),
                                          pack_hi(d[0][2 * h + 1], d[1][2 * h + 1]),
                                          pack_hi(d[2][2 * h + 1], d[3][2 * h + 1])};
#pragma unroll
                        for (int t = 0; t < NT; ++t) {
                            // the terms a_p b_r with p + r <= 4 (parts numbered 1..3)
                            // as D^T: hj (H^T, factor x column) is the A
                            // operand and the part (column x row) the B one
                            if (p == 2) {
                                acc1[rho][t] = mfma_bf16(hj[h][t][0], ap, acc1[rho][t]);
                            } else if (p == 1) {
                                acc1[rho][t] = mfma_bf16(hj[h][t][1], ap, acc1[rho][t]);
                                acc1[rho][t] = mfma_bf16(hj[h][t][0], ap, acc1[rho][t]);
                            } else {
                                acc1[rho][t] = mfma_bf16(hj[h][t][2], ap, acc1[rho][t]);
                                acc1[rho][t] = mfma_bf16(hj[h][t][1], ap, acc1[rho][t]);
                                acc1[rho][t] = mfma_bf16(hj[h][t][0], ap, acc1[rho][t]);
                            }
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int rho = 0; rho < 2; ++rho)
#pragma unroll
            for (int t = 0; t < NT; ++t) red[hb][wave][rho][t][lane] = acc1[rho][t];
    };

    // The waves' row-side sums of panel a, in wave order, to P1. Lane
    // (lr, g') of acc1[rho][t] holds factors 16 t + 4 g' .. +3 of row
    // 32 a + 16 rho + lr, so thread h sums one float2 (half h & 1 of the
    // float4 at h >> 1 of each wave's block) over the eight waves and stores
    // it. Every thread stores exactly once (a thread without an output, or
    // an output past n or past k, writes the sink): with no branch around
    // the store, the compiler counts it exactly and never waits for it when
    // it waits for the next panel's loads (a store in a branch made every
    // panel wait for the previous panel's stores to complete).
    const int ldp1 = p1_ld(k);
    float* __restrict__ sink = P1 + (p1_rows_before(NS - 1) + n) * (int64_t)ldp1 + 2 * tid;
    auto reduce_rows = [&](int a) {
        constexpr int HALVES = 4 * NT * 64;  // float2 outputs of a panel
        static_assert(HALVES <= NTH, "one output per thread at most");
        const int h = tid < HALVES ? tid : 0;
        const f32x2* rq = reinterpret_cast<const f32x2*>(&red[a & 1][0][0][0][0]);
        f32x2 sum = rq[h];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) sum += rq[w * HALVES + h];
        const int o = h >> 1;
        const int ln = o & 63, t = (o >> 6) % NT, rho = o / (64 * NT);
        const int fq = 16 * t + 4 * (ln >> 4) + 2 * (h & 1);
        const int i = 32 * a + 16 * rho + (ln & 15);
        const bool ok = tid < HALVES && fq < k && i < n;
        float* dstp = ok ? P1 + (p1base + i) * ldp1 + fq : sink;
        *reinterpret_cast<f32x2*>(dstp) = sum;
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

    // column side of the chunk: lane (lr, g') holds column c0 + 4 lr + q,
    // factor columns 16t + 4g' + r
    // (rows of p1_ld(k) floats: one float4 of four factors per store)
    float* __restrict__ dst = P2 + ((int64_t)qc * NS + s) * kSymStrip * ldp1;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int c = 16 * t + 4 * g;
            if (c < ldp1)
                *reinterpret_cast<floatx4*>(dst + (int64_t)(64 * wave + 4 * lr + q) * ldp1 + c) =
                    acc2[q][t];
        }
}

// P[i][c] (ld ldP) = sum over s >= i / 512 of P1[s][i][c], then over the chunks of
// strip i / 512 of P2[qc][s(i)][i][c]; tr_part[b] = sum over the rows of block
// b of <Hdot_i, P_i> (fp64), blocks of kUpdRows rows. A thread sums four
// factors at once (float4 loads of the p1_ld(k)-float rows of P1 and P2), each
// in the same order as a scalar sum would.
__global__ __launch_bounds__(256) void sym_fold_kernel(const float* __restrict__ P1,
                                                       const float* __restrict__ P2, int n, int k,
                                                       int NS, float* __restrict__ P, int ldP,
                                                       const float* __restrict__ Hdot,
                                                       double* __restrict__ tr_part,
                                                       const int* __restrict__ done) {
    if (done && *done) return;
    __shared__ double redd[4];
    const int ldp1 = p1_ld(k);
    const int kq = ldp1 / 4;
    const int row0 = blockIdx.x * kUpdRows;
    const int rows = min(kUpdRows, n - row0);
    double acc = 0.0;
    for (int e = threadIdx.x; e < rows * kq; e += 256) {
        const int i = row0 + e / kq;
        const int c = 4 * (e % kq);
        const int si = i / kSymStrip;
        floatx4 sum = {0.f, 0.f, 0.f, 0.f};
        int sp = si;
        for (; sp + 8 <= NS; sp += 8) {
            floatx4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = *reinterpret_cast<const floatx4*>(P1 + (p1_rows_before(sp + u) + i) * ldp1 + c);
#pragma unroll
            for (int u = 0; u < 8; ++u) sum += v[u];
        }
        for (; sp < NS; ++sp)
            sum += *reinterpret_cast<const floatx4*>(P1 + (p1_rows_before(sp) + i) * ldp1 + c);
        const int nch = (min(n, kSymStrip * (si + 1)) + kSymChunk - 1) / kSymChunk;
        const int64_t qstride = (int64_t)NS * kSymStrip * ldp1;
        const float* p2 = P2 + ((int64_t)si * kSymStrip + (i - si * kSymStrip)) * ldp1 + c;
        for (int q = 0; q < nch; ++q) sum += *reinterpret_cast<const floatx4*>(p2 + q * qstride);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (c + j < k) {
                P[(int64_t)i * ldP + c + j] = sum[j];
                if (Hdot) acc += (double)Hdot[(int64_t)i * k + c + j] * (double)sum[j];
            }
        }
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
    p.p1_floats = (size_t)(p1_rows_before(p.ns - 1) + n) * p1_ld(k) + kSymSinkFloats;
    p.p2_floats = (size_t)p.nq * p.ns * kSymStrip * p1_ld(k);
    p.nkb_col = (n + 31) / 32;
    p.nkb_row = 2 * ((n + 63) / 64);
    p.packed_col_bytes = (size_t)p.nkb_col * p.nt * 3 * 64 * 16;
    p.packed_row_bytes = (size_t)p.nkb_row * p.nt * 3 * 64 * 16;
    return p;
}

hipError_t launch_sym_pack(const float* H, int n, int k, const SymPlan& p, void* HsR, void* HsC,
                           const int* done, hipStream_t st) {
    for (int rowmap = 0; rowmap < 2; ++rowmap) {
        const int nkb = rowmap ? p.nkb_row : p.nkb_col;
        const int64_t threads = (int64_t)nkb * p.nt * 64;
        hipLaunchKernelGGL(sym_pack_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                           st, H, n, k, p.nt, nkb, rowmap,
                           static_cast<u32x4*>(rowmap ? HsR : HsC), done);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_sym(const float* S, int64_t lds, const void* HsR, const void* HsC, int n, int k,
                      const SymPlan& p, float* P1, float* P2, const int* done,
                      hipStream_t st) {
    const u32x4* hr = static_cast<const u32x4*>(HsR);
    const u32x4* hc = static_cast<const u32x4*>(HsC);
    const dim3 grid((unsigned)p.ns, (unsigned)p.nq);
    const dim3 block(64 * kSymWaves);
    switch (p.nt) {
        case 1:
            hipLaunchKernelGGL((sym_kernel<1>), grid, block, 0, st, S, lds, hr, hc, n, k, P1, P2, done);
            break;
        case 2:
            hipLaunchKernelGGL((sym_kernel<2>), grid, block, 0, st, S, lds, hr, hc, n, k, P1, P2, done);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_sym_fold(const float* P1, const float* P2, int n, int k, const SymPlan& p,
                           float* P, int ldP, const float* Hdot, double* tr_part,
                           const int* done, hipStream_t st) {
    const int nblk = (n + kUpdRows - 1) / kUpdRows;
    hipLaunchKernelGGL(sym_fold_kernel, dim3(nblk), dim3(256), 0, st, P1, P2, n, k, p.ns, P, ldP,
                       Hdot, tr_part, done);
    return hipGetLastError();
}

}  // namespace symnmf
