// The spectral probe's product Y = S Q (P1 "Choosing the rank k", "Why this
// solver": the leading eigenvalues of S) on the bf16 matrix cores.
//
// Every fp32 operand is split exactly into three bf16 parts (bf16split.h), so
// the pass matches an fp32 product to fp32 rounding while its matrix work runs
// at the bf16 rate: 6 bf16 MFMAs per 32 rows of K against 8 fp32 16x16x4 ones,
// each 16 times cheaper (2.5 PFLOP/s bf16 against 157.3 TFLOP/s fp32 dense).
//
// Orientation: (S Q)[i][c] = sum_j S[i][j] Q[j][c] reads row i of S
// contiguously, so the A operand (16 rows x 32 columns of S) comes straight
// from memory, no symmetry needed. Lane l of a wave owns row l % 16 of each of
// its 16-row subtiles and, in K block kb, the 8 columns
//     32 kb + 4 g + e (e = 0..3) and 32 kb + 16 + 4 g + (e - 4) (e = 4..7),
// g = l / 16: two float4 loads per row and subtile, and each load instruction
// reads 64 contiguous bytes of 16 rows. The matrix core pairs element e of
// lane group g in A with element e of lane group g in B, so Q's K index uses
// the same map, which the Q packing below applies.
#include <algorithm>

#include "bf16split.h"
#include "common.h"
#include "kernels.h"

namespace symnmf {
namespace {

constexpr int kSqWaveTiles = 2;                  // 16-row subtiles per wave
constexpr int kSqTileRows = 4 * 16 * kSqWaveTiles;  // rows of S per workgroup

// Q (n x width, ld ldq) -> Qs, the B operands of every K block: for block kb,
// column tile t (16 columns) and part p, 64 lanes x 16 bytes at
//     Qs[((kb * NT + t) * 3 + p) * 64 + l],
// lane l = 16 g + c holding Q[j(g, e)][16 t + c] for e = 0..7 (the K map of
// the file comment). Rows >= n and columns >= width are zero.
__global__ __launch_bounds__(256) void sq_pack_q_kernel(const float* __restrict__ Q, int64_t ldq,
                                                        int n, int width, int NT,
                                                        u32x4* __restrict__ Qs) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int nkb = (n + 31) >> 5;
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
        const int j = 32 * kb + (e < 4 ? 4 * g + e : 12 + 4 * g + e);
        v[e] = (j < n && c < width) ? Q[(int64_t)j * ldq + c] : 0.f;
    }
    u32x4 x1, x2, x3;
    split3_8(v, x1, x2, x3);
    u32x4* dst = Qs + kt * 3 * 64 + lane;
    dst[0] = x1;
    dst[64] = x2;
    dst[128] = x3;
}

// part[s][i][c] = sum over the K blocks of split s of S[i][j] Q[j][c].
// Workgroup (tile, split): rows [tile * kSqTileRows, +kSqTileRows), wave w
// the 16 kSqWaveTiles rows from tile * kSqTileRows + 32 w; K blocks
// [split * kb_per_split, +kb_per_split). The K block's packed Q (NT * 3 KiB)
// is staged in LDS, double-buffered, one barrier per block; each wave's S rows
// go straight to registers, one block ahead of the multiply.
template <int NT>
// Three workgroups per CU (three waves per SIMD: 164 registers, 48 KiB of LDS).
__global__ __launch_bounds__(256, 3) void sq_split_kernel(const float* __restrict__ S, int64_t lds,
                                                       const u32x4* __restrict__ Qs, int n,
                                                       int kb_per_split, float* __restrict__ part,
                                                       int ldp, int width) {
    constexpr int WM = kSqWaveTiles;
    constexpr int BLK = NT * 3 * 64;          // 16-byte pieces of one K block of Qs
    constexpr int PER = (BLK + 255) / 256;    // pieces per thread
    __shared__ u32x4 qs[2][BLK];
    const int nkb = (n + 31) >> 5;
    const int ntiles = (n + kSqTileRows - 1) / kSqTileRows;
    const int tile = blockIdx.x % ntiles;
    const int split = blockIdx.x / ntiles;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int kb0 = split * kb_per_split;
    const int kb1 = min(nkb, kb0 + kb_per_split);
    const int row0 = tile * kSqTileRows + wave * 16 * WM;

    const float* arow[WM];
#pragma unroll
    for (int s = 0; s < WM; ++s) {
        const int i = min(row0 + 16 * s + (lane & 15), n - 1);  // rows past n: loaded, not stored
        arow[s] = S + (int64_t)i * lds + 4 * g;
    }

    // the K block's S values: v[s][e], e in the K map's order. No load sits
    // in a branch (the compiler's wait counting stays exact): a piece that
    // would start at column >= n (only in the ragged last block) reads the
    // row's first 16 bytes instead, and mask_tail zeroes columns >= n when the
    // block is used. A piece starting below n lies inside the row (lds is a
    // multiple of 4).
    auto load_a = [&](int kb, float (&v)[WM][8]) {
        const int j = 32 * kb;
#pragma unroll
        for (int s = 0; s < WM; ++s)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int col = j + 16 * p + 4 * g < n ? j + 16 * p : -4 * g;
                const floatx4 t =
                    __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(arow[s] + col));
#pragma unroll
                for (int e = 0; e < 4; ++e) v[s][4 * p + e] = t[e];
            }
    };
    auto mask_tail = [&](int kb, float (&v)[WM][8]) {
        const int j = 32 * kb;
        if (j + 32 > n) {
#pragma unroll
            for (int s = 0; s < WM; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int jc = j + (e < 4 ? 4 * g + e : 12 + 4 * g + e);
                    v[s][e] = jc < n ? v[s][e] : 0.f;
                }
        }
    };
    u32x4 qst[PER];
    auto load_q = [&](int kb) {
        const u32x4* src = Qs + (int64_t)kb * BLK;
#pragma unroll
        for (int q = 0; q < PER; ++q) qst[q] = src[min(tid + 256 * q, BLK - 1)];
    };
    auto store_q = [&](int buf) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = tid + 256 * q;
            if (BLK % 256 == 0 || e < BLK) qs[buf][e] = qst[q];
        }
    };

    floatx4 acc[WM][NT];
#pragma unroll
    for (int s = 0; s < WM; ++s)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[s][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    // One K block: the S values of block kb were loaded one block earlier;
    // this step issues block kb + 1's packed Q and S values, multiplies, then
    // stages Q (its wait does not cover the later S loads,
    // which stay in flight across the barrier). Every step issues its loads,
    // past the split's end of a clamped (valid) block, so that every path
    // holds the same loads and the compiler's wait counts stay tight; only
    // the multiply is skipped there.
    int buf = 0;
    auto step = [&](int kb, float (&cur)[WM][8], float (&pre)[WM][8]) {
        load_q(min(kb + 1, kb1 - 1));
        load_a(min(kb + 1, kb1 - 1), pre);
        if (kb < kb1) {
            mask_tail(kb, cur);
            u32x4 a1[WM], a2[WM], a3[WM];
#pragma unroll
            for (int s = 0; s < WM; ++s) split3_8(cur[s], a1[s], a2[s], a3[s]);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const u32x4 b1 = qs[buf][(3 * t + 0) * 64 + lane];
                const u32x4 b2 = qs[buf][(3 * t + 1) * 64 + lane];
                const u32x4 b3 = qs[buf][(3 * t + 2) * 64 + lane];
#pragma unroll
                for (int s = 0; s < WM; ++s) {
                    acc[s][t] = mfma_split6(a1[s], a2[s], a3[s], b1, b2, b3, acc[s][t]);
                }
            }
        }
        store_q(buf ^ 1);  // last read in the previous block, before its barrier
        __syncthreads();
        buf ^= 1;
    };

    float a0[WM][8], a1[WM][8];
    load_q(kb0);
    load_a(kb0, a0);
    store_q(0);
    __syncthreads();
    // two register sets in rotation, unrolled so that none is copied (one set
    // fewer than two blocks ahead would need leaves room for a third wave per
    // SIMD, which hides more of the matrix-core and LDS latency)
    for (int kb = kb0; kb < kb1; kb += 2) {
        step(kb, a0, a1);
        step(kb + 1, a1, a0);
    }

    // lane l holds rows 4 g + r of each subtile, column 16 t + l % 16
    float* __restrict__ dst = part + (int64_t)split * ((int64_t)n * ldp);
#pragma unroll
    for (int s = 0; s < WM; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = row0 + 16 * s + 4 * g + r;
            if (i < n) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int c = 16 * t + (lane & 15);
                    if (c < width) dst[(int64_t)i * ldp + c] = acc[s][t][r];
                }
            }
        }
}

template <int NT>
hipError_t launch_sq_nt(const float* S, int64_t lds, const u32x4* Qs, int n, int nsplit,
                        int kb_per_split, float* part, int ldp, int width, hipStream_t st) {
    const int ntiles = (n + kSqTileRows - 1) / kSqTileRows;
    hipLaunchKernelGGL((sq_split_kernel<NT>), dim3((unsigned)ntiles * (unsigned)nsplit), dim3(256),
                       0, st, S, lds, Qs, n, kb_per_split, part, ldp, width);
    return hipGetLastError();
}

}  // namespace

SqPlan sq_plan(int n, int width) {
    SqPlan p;
    p.nt = (width + 15) / 16;
    const int nkb = (n + 31) / 32;
    const int ntiles = (n + kSqTileRows - 1) / kSqTileRows;
    // about 6144 workgroups (eight rounds of three per CU, so the last,
    // partial round is a small share), at most kMaxSplits splits, none empty
    const int ns = std::max(1, std::min({kMaxSplits, nkb, (6144 + ntiles - 1) / ntiles}));
    p.kb_per_split = (nkb + ns - 1) / ns;
    p.nsplit = (nkb + p.kb_per_split - 1) / p.kb_per_split;
    p.packed_bytes = (size_t)nkb * p.nt * 3 * 64 * 16;
    return p;
}

hipError_t launch_sq_pack(const float* Q, int64_t ldq, int n, int width, const SqPlan& p,
                          void* Qs, hipStream_t st) {
    const int64_t threads = (int64_t)((n + 31) / 32) * p.nt * 64;
    hipLaunchKernelGGL(sq_pack_q_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                       Q, ldq, n, width, p.nt, static_cast<u32x4*>(Qs));
    return hipGetLastError();
}

hipError_t launch_sq_split(const float* S, int64_t lds, const void* Qs, int n, int width,
                           const SqPlan& p, float* part, int ldp, hipStream_t st) {
    const u32x4* q = static_cast<const u32x4*>(Qs);
    switch (p.nt) {
        case 1: return launch_sq_nt<1>(S, lds, q, n, p.nsplit, p.kb_per_split, part, ldp, width, st);
        case 2: return launch_sq_nt<2>(S, lds, q, n, p.nsplit, p.kb_per_split, part, ldp, width, st);
        case 3: return launch_sq_nt<3>(S, lds, q, n, p.nsplit, p.kb_per_split, part, ldp, width, st);
        case 4: return launch_sq_nt<4>(S, lds, q, n, p.nsplit, p.kb_per_split, part, ldp, width, st);
        case 5: return launch_sq_nt<5>(S, lds, q, n, p.nsplit, p.kb_per_split, part, ldp, width, st);
        case 6: return launch_sq_nt<6>(S, lds, q, n, p.nsplit, p.kb_per_split, part, ldp, width, st);
        case 7: return launch_sq_nt<7>(S, lds, q, n, p.nsplit, p.kb_per_split, part, ldp, width, st);
        case 8: return launch_sq_nt<8>(S, lds, q, n, p.nsplit, p.kb_per_split, part, ldp, width, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace symnmf
