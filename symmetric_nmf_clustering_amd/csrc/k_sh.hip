// The tall-skinny S.H pass (P1 "Factorization at scale": the dominant S H
// products; P2 AdaptGrow sketch: S @ H in every full-batch step).
//
// Layout and mapping (gfx950, wave64, fp32 MFMA 16x16x4):
//  * S is row-major and symmetric, so (S X)[i][c] = sum_j S[j][i] X[j][c]: the
//    pass streams contiguous ROW panels of S and produces output columns.
//  * A workgroup (4 waves) owns 256 CW consecutive columns i of S and one
//    split (a set of rows j). Per 4-row group each lane loads CW float4s of S:
//    row j0 + (lane / 16), columns i0 + 64 w + 4 (lane % 16) .. +3, so every
//    row of the group is read as 256 CW contiguous bytes per wave (1 KiB CW
//    per workgroup).
//  * Element q of a float4 feeds MFMA tile q as its B operand, so tile q owns
//    output columns i0 + 4 n + q (n = 0..15); the A operand is X^T for 16
//    columns of X (one c-tile), read straight from L1/L2 (X is small and
//    shared by every column tile of a split).
//  * Columns past the last full 16-column tile (4 or 8 of them, e.g. 16..23
//    for k = 24) run as plain fp32 FMAs on the vector ALU instead of a padded
//    MFMA tile: the matrix core and the vector ALU issue side by side, and no
//    MFMA work is spent on padding. (fp32 MFMA is what keeps up with HBM at
//    k = 24: the vector ALU alone, without packed fp32, would need ~90% of
//    its issue slots.)
//  * Each output (i, c) accumulates one split's rows in fp32 (n / 32 terms at
//    most), and splits are summed later in a fixed order, so the result is
//    deterministic and its rounding error stays ~1e-6 relative.
//  * Block b of the 1-D grid takes column tile b % ntiles and split
//    b / ntiles: the workgroups resident together sweep the same rows of S.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace symnmf {

// How a split's rows are found: contiguous ranges of rows_per_split rows (a
// full pass), or row blocks of a sampled list with one range per split
// (blocks cut into `sub` sub-ranges) or several whole blocks per split.
enum RowMode : int { kRowsContiguous = 0, kRowsBlocks = 1, kRowsBlocksMulti = 2 };

// Row segment `g` of split `s` (at most rp.bps segments); false when none.
template <int RM>
__device__ __forceinline__ bool split_segment(const RowPlan& rp, int s, int g, int& jb, int& je) {
    if constexpr (RM == kRowsContiguous) {
        if (g > 0) return false;
        jb = s * rp.rows_per_split;
        je = min(rp.n, jb + rp.rows_per_split);
    } else if constexpr (RM == kRowsBlocks) {
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

// 4-row groups per main-loop trip. The narrow shapes (CW = 2 with at most one
// MFMA tile beside the vector-ALU columns, i.e. k <= 24, or MFMA tiles only)
// are bound by HBM: the more rows of S one wave has in flight the better, and
// six groups (24 rows, 12 KiB per wave) still leave two waves per SIMD. The
// wide shapes (CW = 1, three or more MFMA tiles) are bound by the matrix
// core, where more waves per SIMD beat deeper trips: one group per trip keeps
// the 80-column probe pass at four waves per SIMD (15.7 ms at n = 100 000
// against 17.3 ms with two groups and three waves). The multi-segment variant
// carries an extra loop level and keeps two groups.
constexpr int sh_rows_per_trip(int ncm, int nv, int cw, int rm) {
    if (cw < 2) return 1;
    return (rm != kRowsBlocksMulti && (ncm <= 1 || nv == 0)) ? 6 : 2;
}

// NCM MFMA column tiles (16 columns each) plus NV <= 8 columns on the vector
// ALU, CW float4 column groups per lane (64 CW columns per wave). XVEC: the
// width is exactly 16 NCM + NV (a multiple of 4) and X is 16-byte aligned, so
// the vector-ALU columns are read as float4s and every width-dependent offset
// is a compile-time constant (k = 24 isolated: 6.62-6.64 against 6.74-6.75 ms).
// RM: how a split finds its rows (RowMode).
template <int NCM, int NV, int CW, bool XVEC, int RM>
__global__ __launch_bounds__(256) void sh_panel_kernel(const float* __restrict__ S, int64_t lds,
                                                       const float* __restrict__ X, int width_arg,
                                                       RowPlan rp, int nsplit,
                                                       float* __restrict__ part, int ldp_arg) {
    if (rp.done && *rp.done) return;  // uniform over the workgroup
    const int width = XVEC ? 16 * NCM + NV : width_arg;
    const int ldp = XVEC ? 16 * NCM + NV : ldp_arg;
    constexpr int U = sh_rows_per_trip(NCM, NV, CW, RM);
    constexpr int WCOLS = 64 * CW;    // columns per wave
    constexpr int NCM1 = NCM > 0 ? NCM : 1;
    constexpr int NV1 = NV > 0 ? NV : 1;
    const int n = rp.n;
    const int ntiles = (n + 4 * WCOLS - 1) / (4 * WCOLS);
    // column tile fastest: the workgroups running together sweep the same rows
    const int tile = blockIdx.x % ntiles;
    const int split = blockIdx.x / ntiles;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane >> 4;   // row of the 4-row group this lane loads
    const int cl = lane & 15;  // column quad / MFMA row index
    const int colbase = tile * (4 * WCOLS) + wave * WCOLS + 4 * cl;
    const int c_v = 16 * NCM;  // first vector-ALU column
    const bool tile_full = (tile + 1) * (4 * WCOLS) <= n;  // uniform over the workgroup

    floatx4 macc[CW][NCM1][4];
    float vacc[CW][4][NV1];
#pragma unroll
    for (int w = 0; w < CW; ++w)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int ct = 0; ct < NCM; ++ct) macc[w][ct][q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NV; ++c) vacc[w][q][c] = 0.f;
        }

    // Loads are unconditional: an out-of-range column reads a clamped, valid
    // address and the value is replaced by zero (edge tile only).
    int scol[CW];
#pragma unroll
    for (int w = 0; w < CW; ++w) {
        const int c0 = colbase + 64 * w;
        scol[w] = c0 < n ? c0 : 0;
    }

    // this lane's X values of row j: MFMA A operands and vector-ALU columns
    auto load_x = [&](int64_t j, bool rowok, float (&a)[NCM1], float (&hv)[NV1]) {
        const float* px = X + j * width;
#pragma unroll
        for (int ct = 0; ct < NCM; ++ct) {
            const int c = 16 * ct + cl;
            const bool ok = rowok && c < width;
            const int off = c < width ? c : 0;
            const float v = px[off];
            a[ct] = ok ? v : 0.f;
        }
        if (NV > 0) {
            if (XVEC) {
#pragma unroll
                for (int c4 = 0; c4 < NV; c4 += 4) {
                    const float4 v = *reinterpret_cast<const float4*>(px + c_v + c4);
                    hv[c4 + 0] = rowok ? v.x : 0.f;
                    hv[c4 + 1] = rowok ? v.y : 0.f;
                    hv[c4 + 2] = rowok ? v.z : 0.f;
                    hv[c4 + 3] = rowok ? v.w : 0.f;
                }
            } else {
#pragma unroll
                for (int c = 0; c < NV; ++c) {
                    const bool ok = rowok && c_v + c < width;
                    const int off = c_v + c < width ? c_v + c : 0;
                    const float v = px[off];
                    hv[c] = ok ? v : 0.f;
                }
            }
        }
    };
    auto load_s = [&](int64_t j, bool edge, float4 (&sv)[CW]) {
        const float* ps = S + j * lds;
#pragma unroll
        for (int w = 0; w < CW; ++w) {
            // S is streamed once per pass: a non-temporal load keeps it from
            // displacing X, which every column tile of a split re-reads
            const floatx4 t = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(ps + scol[w]));
            float4 v = float4{t[0], t[1], t[2], t[3]};
            if (edge) {
                const int c0 = colbase + 64 * w;
                v.x = c0 < n ? v.x : 0.f;
                v.y = c0 + 1 < n ? v.y : 0.f;
                v.z = c0 + 2 < n ? v.z : 0.f;
                v.w = c0 + 3 < n ? v.w : 0.f;
            }
            sv[w] = v;
        }
    };
    auto compute = [&](const float4 (&sv)[CW], const float (&a)[NCM1], const float (&hv)[NV1]) {
#pragma unroll
        for (int w = 0; w < CW; ++w) {
            const float s4[4] = {sv[w].x, sv[w].y, sv[w].z, sv[w].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int ct = 0; ct < NCM; ++ct)
                    macc[w][ct][q] = mfma16x16x4(a[ct], s4[q], macc[w][ct][q]);
#pragma unroll
                for (int c = 0; c < NV; ++c) vacc[w][q][c] = fmaf(s4[q], hv[c], vacc[w][q][c]);
            }
        }
    };

    // rows [jb, je) of S; EDGE (compile time): the workgroup's column tile
    // crosses n, so loaded values past column n are zeroed
    auto run_rows = [&](int jb, int je, auto edge_c) {
        constexpr bool EDGE = decltype(edge_c)::value;
        int j0 = jb;
        for (; j0 + 4 * U <= je; j0 += 4 * U) {
            float4 sv[U][CW];
            float a[U][NCM1];
            float hv[U][NV1];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t j = j0 + 4 * u + r;
                load_s(j, EDGE, sv[u]);
                load_x(j, true, a[u], hv[u]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) compute(sv[u], a[u], hv[u]);
        }
        // ragged tail: a row past the range end reads its first row (a valid
        // address) and contributes zero
        for (; j0 < je; j0 += 4) {
            const bool ok = j0 + r < je;
            const int64_t j = ok ? (int64_t)(j0 + r) : (int64_t)jb;
            float4 sv[CW];
            float a[NCM1];
            float hv[NV1];
            load_s(j, EDGE, sv);
            if (!ok)
#pragma unroll
                for (int w = 0; w < CW; ++w) sv[w] = float4{0.f, 0.f, 0.f, 0.f};
            load_x(j, ok, a, hv);
            compute(sv, a, hv);
        }
    };
    auto run = [&](int jb, int je) {
        if (tile_full) run_rows(jb, je, std::false_type{});
        else run_rows(jb, je, std::true_type{});
    };
    int jb, je;
    if constexpr (RM == kRowsBlocksMulti) {
        for (int g = 0; split_segment<RM>(rp, split, g, jb, je); ++g) run(jb, je);
    } else {
        split_segment<RM>(rp, split, 0, jb, je);
        run(jb, je);
    }

    // Output rows i = colbase + 64 w + q. MFMA tile ct: this lane holds
    // columns 16 ct + 4 r .. +3. Vector-ALU columns: the four row lanes
    // r = 0..3 hold partial sums over their rows; fold them with two xor
    // shuffles, then lane r writes columns c_v + NV/4 r .. + NV/4 - 1.
    float* __restrict__ dst = part + (int64_t)split * ((int64_t)n * ldp);
#pragma unroll
    for (int w = 0; w < CW; ++w)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int c = 0; c < NV; ++c) {
                float v = vacc[w][q][c];
                v += __shfl_xor(v, 16, 64);
                v += __shfl_xor(v, 32, 64);
                vacc[w][q][c] = v;
            }
            const int i = colbase + 64 * w + q;
            if (i < n) {
                float* row = dst + (int64_t)i * ldp;
#pragma unroll
                for (int ct = 0; ct < NCM; ++ct) {
                    const int c0 = 16 * ct + 4 * r;
                    if (c0 < ldp) {
                        const floatx4 v = macc[w][ct][q];
                        *reinterpret_cast<float4*>(row + c0) = float4{v[0], v[1], v[2], v[3]};
                    }
                }
                if (NV > 0) {
                    constexpr int per = NV / 4;  // 1 or 2 columns per row lane
#pragma unroll
                    for (int e = 0; e < per; ++e) {
                        float v = 0.f;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
                            if (r == rr) v = vacc[w][q][per * rr + e];
                        const int c = c_v + per * r + e;
                        if (c < ldp) row[c] = v;
                    }
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Wide widths (three or more MFMA tiles, e.g. the probe's 80 columns) are bound
// by the matrix core, and with one 4-row group per trip the panel kernel has
// only 1 KiB of S per wave in flight, so MFMA issue waits on memory. The ring
// variant below moves each wave's S tile and the trip's 4 rows of X straight
// into a wave-private LDS ring with direct-to-LDS loads (no VGPR destination),
// kRingDepth trips ahead: 4 KiB of S per wave in flight at four waves per SIMD
// (80 columns at n = 100 000: 15.9 -> 14.0 ms). Nothing is shared between
// waves, so there are no barriers; the lanes, operands and accumulation order
// are the panel kernel's (CW = 1, one group per trip), so results are bitwise
// equal. Contiguous row splits only.
constexpr int kRingDepth = 4;

typedef __attribute__((address_space(3))) float* lds_float_ptr;

// 16 bytes per lane from global memory to LDS at byte address m0 + 16 lane.
// Written as asm so that the compiler does not treat the LDS write as pending
// on every later LDS read (it would wait for the whole ring); the ring waits
// for exactly the trip it reads with vmcnt below.
__device__ __forceinline__ void dma_to_lds16(const float* g, uint32_t lds_byte) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_byte), "v"(g)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}
// s_waitcnt lgkmcnt(0): this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lgkm0() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    asm volatile("" ::: "memory");
}

// X DMA instructions per trip: the trip's 4 X rows are 4 width floats, one
// 16-byte piece per lane.
constexpr int sh_ring_xdma(int ncm, int nv) { return (16 * ncm + nv + 63) / 64; }

template <int NCM, int NV>
__global__ __launch_bounds__(256) void sh_ring_kernel(const float* __restrict__ S, int64_t lds,
                                                      const float* __restrict__ X, int width,
                                                      RowPlan rp, float* __restrict__ part,
                                                      int ldp) {
    if (rp.done && *rp.done) return;  // uniform over the workgroup
    constexpr int WMAX = 16 * NCM + NV;
    constexpr int NXI = sh_ring_xdma(NCM, NV);
    constexpr int PER = 1 + NXI;                 // DMA instructions per trip and wave
    constexpr int SLOT = 256 + 4 * WMAX;         // floats: S tile, then 4 X rows
    constexpr int D = kRingDepth;
    constexpr int NV1 = NV > 0 ? NV : 1;
    __shared__ __attribute__((aligned(16))) float ring[4][D * SLOT];
    const int n = rp.n;
    const int ntiles = (n + 255) / 256;
    const int tile = blockIdx.x % ntiles;
    const int split = blockIdx.x / ntiles;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane >> 4;
    const int cl = lane & 15;
    const int colbase = tile * 256 + wave * 64 + 4 * cl;
    const int c_v = 16 * NCM;
    const bool tile_full = (tile + 1) * 256 <= n;
    const int jb = split * rp.rows_per_split;
    const int je = min(n, jb + rp.rows_per_split);
    const int ntrips = je > jb ? (je - jb + 3) / 4 : 0;
    const int xs_floats = 4 * width;
    const int64_t xcount = (int64_t)n * width;
    float* myring = ring[wave];
    const uint32_t ring_byte = (uint32_t)(uintptr_t)(lds_float_ptr)(myring);
    // a column past n loads a valid address (its value is replaced by zero)
    const int scol = colbase < n ? colbase : 0;

    // trip t: rows jb + 4 t .. +3 into slot t % D
    auto issue = [&](int t) {
        const uint32_t slot_byte = ring_byte + 4u * (uint32_t)((t % D) * SLOT);
        const int j0 = jb + 4 * t;
        const int jr = j0 + r;
        const int64_t j = jr < je ? jr : jb;
        dma_to_lds16(S + j * lds + scol, slot_byte);
#pragma unroll
        for (int i = 0; i < NXI; ++i) {
            const int f = 256 * i + 4 * lane;  // float offset in the trip's X block
            const int64_t off = (int64_t)j0 * width + f;
            const int64_t offc = off + 3 < xcount ? off : 0;
            if (f < xs_floats) dma_to_lds16(X + offc, slot_byte + 4u * (uint32_t)(256 + 256 * i));
        }
    };

    floatx4 macc[NCM][4];
    float vacc[4][NV1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int ct = 0; ct < NCM; ++ct) macc[ct][q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NV; ++c) vacc[q][c] = 0.f;
    }

#pragma unroll
    for (int t = 0; t < D; ++t)
        if (t < ntrips) issue(t);
    for (int t = 0; t < ntrips; ++t) {
        // loads complete in issue order: trip t is in LDS once at most the
        // PER * later instructions of the trips behind it are outstanding
        const int later = min(D - 1, ntrips - 1 - t);
        if (later >= 3) wait_vmcnt<PER * 3>();
        else if (later == 2) wait_vmcnt<PER * 2>();
        else if (later == 1) wait_vmcnt<PER * 1>();
        else wait_vmcnt<0>();
        const float* sl = myring + (t % D) * SLOT;
        const float* xr = sl + 256 + r * width;
        float4 sv = *reinterpret_cast<const float4*>(sl + 4 * lane);
        float a[NCM];
        float hv[NV1];
#pragma unroll
        for (int ct = 0; ct < NCM; ++ct) {
            const int c = 16 * ct + cl;
            a[ct] = c < width ? xr[c] : 0.f;
        }
#pragma unroll
        for (int c4 = 0; c4 < NV; c4 += 4) {
            const float4 v = *reinterpret_cast<const float4*>(xr + c_v + c4);
            hv[c4] = v.x;
            hv[c4 + 1] = v.y;
            hv[c4 + 2] = v.z;
            hv[c4 + 3] = v.w;
        }
        // the slot is read: refill it with trip t + D
        wait_lgkm0();
        if (t + D < ntrips) issue(t + D);
        if (jb + 4 * t + r >= je) {
#pragma unroll
            for (int ct = 0; ct < NCM; ++ct) a[ct] = 0.f;
#pragma unroll
            for (int c = 0; c < NV; ++c) hv[c] = 0.f;
        }
        if (!tile_full) {
            sv.x = colbase < n ? sv.x : 0.f;
            sv.y = colbase + 1 < n ? sv.y : 0.f;
            sv.z = colbase + 2 < n ? sv.z : 0.f;
            sv.w = colbase + 3 < n ? sv.w : 0.f;
        }
        const float s4[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int ct = 0; ct < NCM; ++ct) macc[ct][q] = mfma16x16x4(a[ct], s4[q], macc[ct][q]);
#pragma unroll
            for (int c = 0; c < NV; ++c) vacc[q][c] = fmaf(s4[q], hv[c], vacc[q][c]);
        }
    }

    // the panel kernel's epilogue with CW = 1
    float* __restrict__ dst = part + (int64_t)split * ((int64_t)n * ldp);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int c = 0; c < NV; ++c) {
            float v = vacc[q][c];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            vacc[q][c] = v;
        }
        const int i = colbase + q;
        if (i < n) {
            float* row = dst + (int64_t)i * ldp;
#pragma unroll
            for (int ct = 0; ct < NCM; ++ct) {
                const int c0 = 16 * ct + 4 * r;
                if (c0 < ldp) {
                    const floatx4 v = macc[ct][q];
                    *reinterpret_cast<float4*>(row + c0) = float4{v[0], v[1], v[2], v[3]};
                }
            }
            if (NV > 0) {
                constexpr int per = NV / 4;
#pragma unroll
                for (int e = 0; e < per; ++e) {
                    float v = 0.f;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        if (r == rr) v = vacc[q][per * rr + e];
                    const int c = c_v + per * r + e;
                    if (c < ldp) row[c] = v;
                }
            }
        }
    }
}

// The ring needs X 16-byte aligned (16-byte DMA pieces), a fixed number of X
// pieces per trip for the shape, and, with vector-ALU columns, float4 reads of
// them inside each row.
template <int NCM, int NV>
static bool sh_ring_fits(const float* X, int width, const RowPlan& rp) {
    if (rp.blocks != nullptr || rp.rows_per_split % 4 != 0) return false;
    if ((reinterpret_cast<uintptr_t>(X) % 16) != 0) return false;
    if ((width + 63) / 64 != sh_ring_xdma(NCM, NV)) return false;
    if (NV > 0 && (width % 4 != 0 || 16 * NCM + NV > width)) return false;
    return true;
}

template <int NCM, int NV>
static hipError_t launch_sh_ring(const float* S, int64_t lds, const float* X, int width,
                                 const RowPlan& rp, int nsplit, float* part, int ldp,
                                 hipStream_t st) {
    const int ntiles = (rp.n + 255) / 256;
    hipLaunchKernelGGL((sh_ring_kernel<NCM, NV>), dim3((unsigned)ntiles * (unsigned)nsplit),
                       dim3(256), 0, st, S, lds, X, width, rp, part, ldp);
    return hipGetLastError();
}

template <int NCM, int NV, int CW, int RM>
static hipError_t launch_sh_t(const float* S, int64_t lds, const float* X, int width,
                              const RowPlan& rp, int nsplit, float* part, int ldp, hipStream_t st) {
    const int ntiles = (rp.n + 256 * CW - 1) / (256 * CW);
    dim3 grid((unsigned)ntiles * (unsigned)nsplit);
    const bool xvec = width == 16 * NCM + NV && ldp == width &&
                      (reinterpret_cast<uintptr_t>(X) % 16) == 0;
    if (xvec)
        hipLaunchKernelGGL((sh_panel_kernel<NCM, NV, CW, true, RM>), grid, dim3(256), 0, st, S,
                           lds, X, width, rp, nsplit, part, ldp);
    else
        hipLaunchKernelGGL((sh_panel_kernel<NCM, NV, CW, false, RM>), grid, dim3(256), 0, st, S,
                           lds, X, width, rp, nsplit, part, ldp);
    return hipGetLastError();
}

template <int NCM, int NV, int CW>
static hipError_t launch_sh_any(const float* S, int64_t lds, const float* X, int width,
                                const RowPlan& rp, int nsplit, float* part, int ldp,
                                hipStream_t st) {
    if constexpr (CW == 1) {
        // matrix-core-bound widths: the ring keeps more of S in flight
        if (sh_ring_fits<NCM, NV>(X, width, rp))
            return launch_sh_ring<NCM, NV>(S, lds, X, width, rp, nsplit, part, ldp, st);
    }
    if (rp.blocks == nullptr)
        return launch_sh_t<NCM, NV, CW, kRowsContiguous>(S, lds, X, width, rp, nsplit, part, ldp, st);
    // sampled row blocks: fit widths only (k <= 64)
    if constexpr (16 * NCM + NV <= kMaxK) {
        if (rp.sub == 1 && rp.bps > 1)
            return launch_sh_t<NCM, NV, CW, kRowsBlocksMulti>(S, lds, X, width, rp, nsplit, part, ldp, st);
        return launch_sh_t<NCM, NV, CW, kRowsBlocks>(S, lds, X, width, rp, nsplit, part, ldp, st);
    }
    return hipErrorInvalidValue;
}

// Split a width into full 16-column MFMA tiles plus a vector-ALU remainder of
// 4 or 8 columns (a remainder above 8 takes one more, padded, MFMA tile).
hipError_t launch_sh_panel(const float* S, int64_t lds, const float* X, int width,
                           const RowPlan& rp, int nsplit, float* part, int ldp, hipStream_t st) {
    int ncm = width / 16;
    int rem = width - 16 * ncm;
    int nv = rem == 0 ? 0 : (rem <= 4 ? 4 : (rem <= 8 ? 8 : 0));
    if (rem > 8) ++ncm;
#define SH_CASE(M, V, C) \
    if (ncm == M && nv == V) return launch_sh_any<M, V, C>(S, lds, X, width, rp, nsplit, part, ldp, st);
    SH_CASE(0, 4, 2) SH_CASE(0, 8, 2)
    SH_CASE(1, 0, 2) SH_CASE(1, 4, 2) SH_CASE(1, 8, 2)
    SH_CASE(2, 0, 2) SH_CASE(2, 4, 2) SH_CASE(2, 8, 2)
    SH_CASE(3, 0, 1) SH_CASE(3, 4, 1) SH_CASE(3, 8, 1)
    SH_CASE(4, 0, 1) SH_CASE(4, 4, 1) SH_CASE(4, 8, 1)
    SH_CASE(5, 0, 1) SH_CASE(5, 4, 1) SH_CASE(5, 8, 1)
    SH_CASE(6, 0, 1) SH_CASE(6, 4, 1) SH_CASE(6, 8, 1)
    SH_CASE(7, 0, 1) SH_CASE(7, 4, 1) SH_CASE(7, 8, 1)
    SH_CASE(8, 0, 1)
#undef SH_CASE
    return hipErrorInvalidValue;
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
        const float s = ordered_strided_sum(p, nsplit, pstride);
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
