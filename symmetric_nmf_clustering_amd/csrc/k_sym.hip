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
// them as 8 float4 buffer loads: load m gives lane l = 16g + c (g = l / 16)
// the four columns c0 + 4c + q (q = 0..3) of row 4m + g, so each load
// instruction reads 256 contiguous bytes of 4 rows. The panel's base is a
// scalar and the lane offsets are fixed; rows past n read as zero (the buffer
// ends at S's last row).
//  * Column side: for fixed q the panel's parts are matrix-core B operands as
//    loaded: column c0 + 4c + q along the lanes, the 32 rows within them (row
//    4e + g is element e of lane group g). A = H^T of the panel's rows in that
//    K order ("column map", packed once per pass); the result lands as
//    Z[factor][column].
//  * Row side: the contraction runs over the columns, which the loaded layout
//    holds across lanes. Each wave writes the parts of one 16-row half of the
//    panel to its own LDS area (eight bytes per lane, part and column: four
//    rows of one column) and reads them back with the 16-bit transposed LDS
//    read, which hands every lane eight consecutive columns of one row: the B
//    operand of D^T = H^T (factor x column) times the part (column x row), with
//    H's rows packed in column order ("row map"). A lane of the result holds
//    four consecutive factors of one row, so the per-panel sum over the eight
//    waves is one float2 per thread and one store per thread (reduce_rows).
//  * A factor tile that holds at most 8 factors (the last one when k % 16 is
//    1..8) carries two parts of H per operand, rows 8..15 of the tile holding
//    the same factors as rows 0..7 (tile_mma): four matrix-core steps per K
//    block instead of six. The two halves of the result are added at the end.
//
// Work: strips of 512 columns (8 waves), each walked down in chunks of 2048
// rows. Workgroup (strip s, chunk qc) covers rows [2048 qc, min(2048 (qc+1),
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
// per wave: the three bf16 parts of one 16-row half of a panel (part_slot)
constexpr int kSymPartBytes = 3 * 256 * 8;

// rows of P1 held by the strips before strip s (each 512 (s' + 1) rows)
__host__ __device__ inline int64_t p1_rows_before(int s) {
    return (int64_t)(kSymStrip / 2) * s * (s + 1);
}
// row pitch of P1: the row-side sums are stored as float2 pairs of factors
__host__ __device__ inline int p1_ld(int k) { return (k + 3) / 4 * 4; }
// floats of the store sink after P1 (one float2 per thread of a workgroup)
constexpr int kSymSinkFloats = 2 * 64 * kSymWaves;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The 8-byte slot (of a part's 256) that holds quad b (rows 4e + b, e = 0..3,
// of a 16-row half) of local column j. The low four bits are swizzled so that
// the 16 lanes of a write (columns 4l + q of one quad) and the 16 lanes of a
// transposed read (four columns of four quads) each touch 16 different 8-byte
// bank groups.
__device__ __forceinline__ int part_slot(int b, int j) {
    return 64 * b + 16 * (j & 3) + (((j >> 2) ^ (4 * (j & 3) + b)) & 15);
}

// 16-bit transposed LDS read (gfx950): within each 16-lane group, lane 4a + b
// reads four 16-bit values at its address, and lane 4b + e receives value e
// of lane 4a + b as its element a (a, b, e = 0..3).
__device__ __forceinline__ u32x2 lds_read_tr16(char* p) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const bf16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)((__attribute__((address_space(3))) char*)p));
    return __builtin_bit_cast(u32x2, r);
}

// acc += A B over one 32-deep K block of one factor tile, A given by three
// operands of H (sym_pack_kernel) and B by the three parts of S, smallest
// terms first. A full tile takes the six terms of mfma_split6. A half tile
// holds its (at most 8) factors in rows 0..7 of A and of the result; operand
// 0 carries part 1 of H there and part 2 in rows 8..15, operand 1 part 3 and
// operand 2 part 1 (rows 8..15 zero). The four products give the same six
// terms: rows 0..7 get H1 S1, H3 S1, H1 S2, H1 S3, rows 8..15 get H2 S1, H2 S2.
__device__ __forceinline__ floatx4 tile_mma(bool half, const u32x4 (&A)[3], const u32x4& b1,
                                            const u32x4& b2, const u32x4& b3, floatx4 acc) {
    if (half) {
        acc = mfma_bf16(A[1], b1, acc);
        acc = mfma_bf16(A[2], b3, acc);
        acc = mfma_bf16(A[0], b2, acc);
        acc = mfma_bf16(A[0], b1, acc);
        return acc;
    } else {
        return mfma_split6(A[0], A[1], A[2], b1, b2, b3, acc);
    }
}

// H (n x k, ld k) -> the A operands of every 32-row K block kb, tile t and
// operand o at out[((kb * NT + t) * 3 + o) * 64 + l]: lane l = 16g + c holds
// rows row(kb, g, e), e = 0..7, of factor slot c:
//   column map: row = 32 kb + 4 e + g   (the K order of a loaded panel's rows)
//   row map:    row = 32 kb + 8 g + e   (columns in order)
// A full tile's operand o is part o + 1 (bf16split.h) of factor 16 t + c. A
// half tile (the last one, when half) holds factor 16 t + (c & 7): operand 0
// part 1 for c < 8 and part 2 for c >= 8, operands 1 and 2 parts 3 and 1 for
// c < 8 and zero for c >= 8 (tile_mma). Rows >= n and factors >= k are zero.
__global__ __launch_bounds__(256) void sym_pack_kernel(const float* __restrict__ H, int n, int k,
                                                       int NT, int half, int nkb, int rowmap,
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
    const int c = lane & 15;
    const bool ht = half && tile == NT - 1;
    const int f = 16 * tile + (ht ? (c & 7) : c);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int row = rowmap ? 32 * kb + 8 * g + e : 32 * kb + 4 * e + g;
        v[e] = (row < n && f < k) ? H[(int64_t)row * k + f] : 0.f;
    }
    u32x4 x1, x2, x3;
    split3_8(v, x1, x2, x3);
    if (ht) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 o0 = c < 8 ? x1 : x2;
        const u32x4 o1 = c < 8 ? x3 : z;
        const u32x4 o2 = c < 8 ? x1 : z;
        x1 = o0;
        x2 = o1;
        x3 = o2;
    }
    u32x4* dst = out + kt * 3 * 64 + lane;
    dst[0] = x1;
    dst[64] = x2;
    dst[128] = x3;
}

template <int NT, bool HALF>
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
    __shared__ __attribute__((aligned(16))) char parts[WAVES][kSymPartBytes];

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

    // row side A operands (row map) of the wave's two K blocks, for the chunk
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
    // a float4 that would start at column >= n (ragged edge, or a wave past n)
    // reads the row's first 16 bytes instead; the values at columns >= n are
    // zeroed before use. A float4 starting below n lies inside the row (lds is
    // a multiple of 4).
    const int col = c0 + 4 * lr;
    const int coff = col < n ? col : 0;
    const int voff = (g * (int)lds + coff) * 4;  // bytes; 32 rows of S stay below 2^31

    typedef floatx4 Panel[8];
    auto load = [&](int a, Panel& v) {
        const int64_t row0 = 32 * (int64_t)min(a, a1 - 1);
        // bytes from the panel to S's end; a panel past the chunk gets an empty
        // buffer, whose loads return zeros without a memory access
        const int64_t rest = a < a1 ? ((int64_t)n - row0) * lds * 4 : 0;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(S + row0 * lds), (short)0, (int)min(rest, (int64_t)0x7fffffff), 0x00020000);
#pragma unroll
        for (int m = 0; m < 8; ++m)
            v[m] = __builtin_bit_cast(
                floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + m * 16 * (int)lds, 0, 2));
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

    // the wave's parts area: lane (lr, g) writes quad g of columns 4 lr + q;
    // lane 4a + b of group g reads quad b of columns 32 h + 8 g + 4 r + a
    char* const area = parts[wave];
    const int la = lr >> 2, lb = lr & 3;
    // a half tile's rows 8..15 (lanes 32..63) added to its rows 0..7 (lanes
    // 0..31) through the wave's area (free between panels); lanes 32..63 of
    // the result are not used
    auto fold_half = [&](floatx4 (&x)[4], int cnt) {
        floatx4* const st = reinterpret_cast<floatx4*>(area);
        for (int j = 0; j < cnt; ++j) st[64 * j + lane] = x[j];
        wave_lds_sync();
        for (int j = 0; j < cnt; ++j) x[j] += st[64 * j + (lane ^ 32)];
        wave_lds_sync();
    };

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
                u32x4 hc[NT][3];
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int o = 0; o < 3; ++o) hc[t][o] = hbuf[hb][(3 * t + o) * 64 + lane];
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
                        acc2[q][t] = tile_mma(HALF && t == NT - 1, hc[t], z1, z2, z3, acc2[q][t]);
                }
            }
            // row side, one 16-row half at a time: element pair 2 rho, 2 rho + 1
            // of y[q][p] is quad g (rows 4e + g, e = 0..3) of that half
#pragma unroll
            for (int rho = 0; rho < 2; ++rho) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int p = 0; p < 3; ++p)
                        *reinterpret_cast<u32x2*>(area + p * 2048 + 8 * part_slot(g, 4 * lr + q)) =
                            u32x2{y[q][p][2 * rho], y[q][p][2 * rho + 1]};
                wave_lds_sync();
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    // B operand of part p: lane (N, g) holds columns 32 h + 8 g .. + 7
                    // of row 16 rho + 4 (N & 3) + (N >> 2)
                    u32x4 bp[3];
#pragma unroll
                    for (int p = 0; p < 3; ++p) {
                        const u32x2 lo =
                            lds_read_tr16(area + p * 2048 + 8 * part_slot(lb, 32 * h + 8 * g + la));
                        const u32x2 hi = lds_read_tr16(
                            area + p * 2048 + 8 * part_slot(lb, 32 * h + 8 * g + 4 + la));
                        bp[p] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                    }
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        acc1[rho][t] =
                            tile_mma(HALF && t == NT - 1, hj[h][t], bp[0], bp[1], bp[2], acc1[rho][t]);
                }
                wave_lds_sync();  // the next writes to the area come after these reads
            }
        }
        if constexpr (HALF) {
            floatx4 hx[4] = {acc1[0][NT - 1], acc1[1][NT - 1]};
            fold_half(hx, 2);
            acc1[0][NT - 1] = hx[0];
            acc1[1][NT - 1] = hx[1];
        }
#pragma unroll
        for (int rho = 0; rho < 2; ++rho)
#pragma unroll
            for (int t = 0; t < NT; ++t) red[hb][wave][rho][t][lane] = acc1[rho][t];
    };

    // The waves' row-side sums of panel a, in wave order, to P1. Lane
    // (N, g') of acc1[rho][t] holds factors 16 t + 4 g' .. +3 of row
    // 32 a + 16 rho + 4 (N & 3) + (N >> 2), so thread h sums one float2 (half
    // h & 1 of the float4 at h >> 1 of each wave's block) over the eight
    // waves and stores it. Every thread stores exactly once (a thread without
    // an output, or an output past n or past k, writes the sink): with no
    // branch around the store, the compiler counts it exactly and never waits
    // for it when it waits for the next panel's loads (a store in a branch
    // made every panel wait for the previous panel's stores to complete).
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
        const int N = ln & 15;
        const int i = 32 * a + 16 * rho + 4 * (N & 3) + (N >> 2);
        const bool ok = tid < HALVES && fq < k && i < n;
        float* dstp = ok ? P1 + (p1base + i) * ldp1 + fq : sink;
        *reinterpret_cast<f32x2*>(dstp) = sum;
    };

    // One panel: issue the next panel's packed H rows and S, multiply this
    // one, reduce the previous panel's row sums, stage the next H block, one
    // barrier. The reduction of panel a - 1 reads the red buffer its waves
    // wrote before the last barrier, and panel a + 1 writes that buffer only
    // after the coming one; reducing it here rather than right after the
    // barrier lets the next loads go out as soon as the barrier is passed.
    // Loads are issued on every path, so the compiler's wait counts stay
    // tight: the S loads of a panel past the chunk's end read an empty buffer
    // (zeros, no memory access) and the H loads are clamped to the last block;
    // past the chunk's end only the arithmetic is skipped.
    auto panel = [&](int a, Panel& cur, Panel& nxt) {
        const int an = min(a + 1, a1 - 1);
        load_h(an);  // first: waiting for it before the barrier leaves the S loads in flight
        load(a + 1, nxt);
        if (a < a1) compute(a, cur);
        if (a > a0 && a - 1 < a1) reduce_rows(a - 1);
        store_h((a + 1) & 1);  // that buffer was last read before the previous barrier
        __syncthreads();
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
    // an even panel count ends on a computed panel whose sums no call reduced
    if ((a1 - a0) % 2 == 0) reduce_rows(a1 - 1);

    // column side of the chunk: lane (lr, g') holds column c0 + 4 lr + q,
    // factors 16t + 4g' + r (a half tile's rows 8..15 folded into 0..7 first)
    // (rows of p1_ld(k) floats: one float4 of four factors per store)
    if constexpr (HALF) {
        floatx4 hx[4] = {acc2[0][NT - 1], acc2[1][NT - 1], acc2[2][NT - 1], acc2[3][NT - 1]};
        fold_half(hx, 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc2[q][NT - 1] = hx[q];
    }
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
// b of <Hdot_i, P_i> (fp64), blocks of kUpdRows rows. One thread per row and
// four factors (blockDim = kUpdRows * p1_ld(k) / 4: float4 loads of the
// p1_ld(k)-float rows of P1 and P2), each summed in the same order as a scalar
// sum would. A row adds up to ns strip partials (rows near the top the most)
// and up to n / 2048 chunk partials (rows near the bottom): kFoldInFlight and
// 8 loads are issued before their additions, so neither sum waits for a
// memory round trip per partial.
constexpr int kFoldInFlight = 16;
__global__ __launch_bounds__(512) void sym_fold_kernel(const float* __restrict__ P1,
                                                       const float* __restrict__ P2, int n, int k,
                                                       int NS, float* __restrict__ P, int ldP,
                                                       const float* __restrict__ Hdot,
                                                       double* __restrict__ tr_part,
                                                       const int* __restrict__ done) {
    if (done && *done) return;
    __shared__ double redd[8];
    const int ldp1 = p1_ld(k);
    const int kq = ldp1 / 4;
    const int i = blockIdx.x * kUpdRows + (int)threadIdx.x / kq;
    const int c = 4 * ((int)threadIdx.x % kq);
    double acc = 0.0;
    if (i < n) {
        const int si = i / kSymStrip;
        floatx4 sum = {0.f, 0.f, 0.f, 0.f};
        int sp = si;
        for (; sp + kFoldInFlight <= NS; sp += kFoldInFlight) {
            floatx4 v[kFoldInFlight];
#pragma unroll
            for (int u = 0; u < kFoldInFlight; ++u)
                v[u] = *reinterpret_cast<const floatx4*>(P1 + (p1_rows_before(sp + u) + i) * ldp1 + c);
#pragma unroll
            for (int u = 0; u < kFoldInFlight; ++u) sum += v[u];
        }
        for (; sp < NS; ++sp)
            sum += *reinterpret_cast<const floatx4*>(P1 + (p1_rows_before(sp) + i) * ldp1 + c);
        const int nch = (min(n, kSymStrip * (si + 1)) + kSymChunk - 1) / kSymChunk;
        const int64_t qstride = (int64_t)NS * kSymStrip * ldp1;
        const float* p2 = P2 + ((int64_t)si * kSymStrip + (i - si * kSymStrip)) * ldp1 + c;
        int q = 0;
        for (; q + 8 <= nch; q += 8) {
            floatx4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = *reinterpret_cast<const floatx4*>(p2 + (q + u) * qstride);
#pragma unroll
            for (int u = 0; u < 8; ++u) sum += v[u];
        }
        for (; q < nch; ++q) sum += *reinterpret_cast<const floatx4*>(p2 + q * qstride);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (c + j < k) {
                P[(int64_t)i * ldP + c + j] = sum[j];
                if (Hdot) acc += (double)Hdot[(int64_t)i * k + c + j] * (double)sum[j];
            }
        }
    }
    if (tr_part) {
        // the block's waves in order (blockDim is a multiple of 64)
        acc = wave_sum(acc);
        const int w = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) redd[w] = acc;
        __syncthreads();
        if (threadIdx.x == 0) {
            double t = 0.0;
            for (int v = 0; v < (int)(blockDim.x >> 6); ++v) t += redd[v];
            tr_part[blockIdx.x] = t;
        }
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
    p.half = k % 16 != 0 && k % 16 <= 8;
    return p;
}

hipError_t launch_sym_pack(const float* H, int n, int k, const SymPlan& p, void* HsR, void* HsC,
                           const int* done, hipStream_t st) {
    for (int rowmap = 0; rowmap < 2; ++rowmap) {
        const int nkb = rowmap ? p.nkb_row : p.nkb_col;
        const int64_t threads = (int64_t)nkb * p.nt * 64;
        hipLaunchKernelGGL(sym_pack_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                           st, H, n, k, p.nt, (int)p.half, nkb, rowmap,
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
#define SYMNMF_SYM_LAUNCH(NT_, HALF_)                                                         \
    hipLaunchKernelGGL((sym_kernel<NT_, HALF_>), grid, block, 0, st, S, lds, hr, hc, n, k, P1, P2, \
                       done)
    if (p.nt == 1 && !p.half) SYMNMF_SYM_LAUNCH(1, false);
    else if (p.nt == 1) SYMNMF_SYM_LAUNCH(1, true);
    else if (p.nt == 2 && !p.half) SYMNMF_SYM_LAUNCH(2, false);
    else if (p.nt == 2) SYMNMF_SYM_LAUNCH(2, true);
    else return hipErrorInvalidValue;
#undef SYMNMF_SYM_LAUNCH
    return hipGetLastError();
}

hipError_t launch_sym_fold(const float* P1, const float* P2, int n, int k, const SymPlan& p,
                           float* P, int ldP, const float* Hdot, double* tr_part,
                           const int* done, hipStream_t st) {
    const int nblk = (n + kUpdRows - 1) / kUpdRows;
    const int threads = kUpdRows * (p1_ld(k) / 4);  // one per row and four factors
    hipLaunchKernelGGL(sym_fold_kernel, dim3(nblk), dim3(threads), 0, st, P1, P2, n, k, p.ns, P,
                       ldP, Hdot, tr_part, done);
    return hipGetLastError();
}

}  // namespace symnmf
