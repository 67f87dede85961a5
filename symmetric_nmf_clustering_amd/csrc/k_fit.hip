// Fit kernels: S statistics, initialisation, the fused reduce + gradient +
// projected AdaGrad + Gram kernel, the per-step finalisation, labels, and the
// small dense helpers of the spectral probe.
//
// P1 "Factorizing with SymNMF" (diagonal AdaGrad, element-wise) and P2 (the
// displayed update G <- G + g*g, H <- max(H - eta g/(sqrt(G) + eps), 0); the
// AdaptGrow sketch's gradient 4 (H (H^T H) - S H)); P1 "Factorization at
// scale" (objective by the trace identity, no n x n intermediates).
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace symnmf {

// ---- S statistics: per kStatsRows-row block, sum S and sum S^2 (fp64) ---------
// 16-byte loads (lds is a multiple of 4 and S 16-byte aligned) and eight
// independent fp64 accumulators per thread, so the pass is bound by HBM rather
// than by the latency of one fp64 addition chain. The summation order depends
// only on n, so the result is reproducible.
__global__ __launch_bounds__(256) void s_stats_kernel(const float* __restrict__ S, int64_t lds,
                                                      int n, double* __restrict__ part2) {
    __shared__ double red[4];
    const int row0 = blockIdx.x * kStatsRows;
    const int rows = min(kStatsRows, n - row0);
    const int n4 = n >> 2;
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    double b0 = 0.0, b1 = 0.0, b2 = 0.0, b3 = 0.0;
    for (int rr = 0; rr < rows; ++rr) {
        const float* row = S + (int64_t)(row0 + rr) * lds;
        for (int q = threadIdx.x; q < n4; q += 256) {
            const float4 v = *reinterpret_cast<const float4*>(row + 4 * q);
            const double x = v.x, y = v.y, z = v.z, w = v.w;
            a0 += x;
            a1 += y;
            a2 += z;
            a3 += w;
            b0 = fma(x, x, b0);
            b1 = fma(y, y, b1);
            b2 = fma(z, z, b2);
            b3 = fma(w, w, b3);
        }
        for (int c = 4 * n4 + (int)threadIdx.x; c < n; c += 256) {
            const double x = row[c];
            a0 += x;
            b0 = fma(x, x, b0);
        }
    }
    const double t1 = block_sum256((a0 + a1) + (a2 + a3), red);
    const double t2 = block_sum256((b0 + b1) + (b2 + b3), red);
    if (threadIdx.x == 0) {
        part2[2 * blockIdx.x] = t1;
        part2[2 * blockIdx.x + 1] = t2;
    }
}

__global__ __launch_bounds__(256) void s_stats_final_kernel(const double* __restrict__ part2,
                                                            int nblk, double* __restrict__ out2) {
    __shared__ double red[4];
    double a = 0.0, b = 0.0;
    for (int i = threadIdx.x; i < nblk; i += 256) {
        a += part2[2 * i];
        b += part2[2 * i + 1];
    }
    a = block_sum256(a, red);
    b = block_sum256(b, red);
    if (threadIdx.x == 0) {
        out2[0] = a;
        out2[1] = b;
    }
}

hipError_t launch_s_stats(const float* S, int64_t lds, int n, double* part2, hipStream_t st) {
    const int nblk = (n + kStatsRows - 1) / kStatsRows;
    hipLaunchKernelGGL(s_stats_kernel, dim3(nblk), dim3(256), 0, st, S, lds, n, part2);
    return hipGetLastError();
}
hipError_t launch_s_stats_final(const double* part2, int nblk, double* out2, hipStream_t st) {
    hipLaunchKernelGGL(s_stats_final_kernel, dim3(1), dim3(256), 0, st, part2, nblk, out2);
    return hipGetLastError();
}

// ---- element-wise helpers -------------------------------------------------------
// H[i] = scale * u(seed, i) + shift, formed in fp64 and rounded once to fp32.
__global__ void init_uniform_kernel(float* __restrict__ H, int64_t count, double scale,
                                    double shift, uint64_t seed) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) H[i] = (float)(scale * (double)uniform24(seed, (uint64_t)i) + shift);
}
hipError_t launch_init_uniform(float* H, int64_t count, double scale, double shift, uint64_t seed,
                               hipStream_t st) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(init_uniform_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                       st, H, count, scale, shift, seed);
    return hipGetLastError();
}

__global__ void fill_kernel(float* __restrict__ p, int64_t count, float v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) p[i] = v;
}
hipError_t launch_fill(float* p, int64_t count, float v, hipStream_t st) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, p,
                       count, v);
    return hipGetLastError();
}

__global__ void copy_kernel(float* __restrict__ d, const float* __restrict__ s, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) d[i] = s[i];
}
hipError_t launch_copy(float* dst, const float* src, int64_t count, hipStream_t st) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, dst,
                       src, count);
    return hipGetLastError();
}

// ---- fused update ------------------------------------------------------------
// One workgroup per kUpdRows rows. For each element (i, c):
//   P   = sum_s part[s][i][c]            (exact pass, fixed split order)
//      or P~[i][c] + pscale * sum_s ...  (Block-SVRG estimate)
//   g   = 4 ((H K)[i][c] - P)
//   G'  = G + g*g   (RMSprop: decay G + (1 - decay) g*g)
//   H'  = max(H - lr g / (sqrt(G') + eps), 0)
// plus <H_t, P> per block (fp64) for the trace identity and the partial Gram
// H'^T H' of the block's rows for the next step's K.
__global__ __launch_bounds__(256) void update_kernel(UpdateArgs a) {
    if (a.fd->done) return;
    extern __shared__ float smem[];
    const int k = a.k;
    float* Hs = smem;                  // kUpdRows x k   H_t rows
    float* Hn_s = Hs + kUpdRows * k;   // kUpdRows x k   H_{t+1} rows
    float* Ks = Hn_s + kUpdRows * k;   // k x k
    __shared__ double red[4];

    const int row0 = blockIdx.x * kUpdRows;
    const int rows = min(kUpdRows, a.n - row0);
    const int nel = rows * k;
    const int tid = threadIdx.x;

    for (int e = tid; e < kUpdRows * k; e += 256) {
        const int i = e / k;
        Hs[e] = (i < rows) ? a.H[(int64_t)row0 * k + e] : 0.f;
    }
    if (!a.gram_only)
        for (int e = tid; e < k * k; e += 256) Ks[e] = a.fd->K[(e / k) * kMaxK + (e % k)];
    __syncthreads();

    double tr = 0.0;
    if (a.gram_only) {
        for (int e = tid; e < kUpdRows * k; e += 256) Hn_s[e] = Hs[e];
    } else {
        for (int e = tid; e < kUpdRows * k; e += 256) {
            if (e >= nel) {
                Hn_s[e] = 0.f;
                continue;
            }
            const int i = e / k;
            const int c = e % k;
            const int64_t gi = (int64_t)(row0 + i);
            const float* p = a.part + gi * a.ldp + c;
            const float s = ordered_strided_sum(p, a.nsplit, a.pstride);
            float P = s;
            if (a.Pt) P = a.Pt[gi * k + c] + a.pscale * s;
            float hk = 0.f;
            const float* hrow = Hs + i * k;
            for (int d = 0; d < k; ++d) hk = fmaf(hrow[d], Ks[d * k + c], hk);
            const float h = hrow[c];
            const float g = 4.f * (hk - P);
            const float Gold = a.G[gi * k + c];
            const float Gv = a.decay > 0.f ? a.decay * Gold + (1.f - a.decay) * (g * g)
                                           : Gold + g * g;
            const float hn = fmaxf(h - a.lr * g / (sqrtf(Gv) + a.eps), 0.f);
            a.Gn[gi * k + c] = Gv;
            a.Hn[gi * k + c] = hn;
            Hn_s[e] = hn;
            if (a.Ha) a.Ha[gi * k + c] = h;
            if (a.Pa) a.Pa[gi * k + c] = P;
            tr += (double)h * (double)P;
        }
    }
    __syncthreads();
    if (a.tr_part) {
        const double t = block_sum256(tr, red);
        if (tid == 0) a.tr_part[blockIdx.x] = t;
    }
    // partial Gram of the rows written (upper triangle, fp32 over <= 64 rows)
    float* gp = a.gram_part + (int64_t)blockIdx.x * k * k;
    for (int idx = tid; idx < k * k; idx += 256) {
        const int x = idx / k;
        const int y = idx % k;
        if (x <= y) {
            float s = 0.f;
            for (int i = 0; i < kUpdRows; ++i) s = fmaf(Hn_s[i * k + x], Hn_s[i * k + y], s);
            gp[idx] = s;
        }
    }
}

hipError_t launch_update(const UpdateArgs& a, hipStream_t st) {
    const int nblk = (a.n + kUpdRows - 1) / kUpdRows;
    const size_t sm = (size_t)(2 * kUpdRows * a.k + a.k * a.k) * sizeof(float);
    if (sm > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)update_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(update_kernel, dim3(nblk), dim3(256), sm, st, a);
    return hipGetLastError();
}

// ---- per-step finalisation ----------------------------------------------------
// Two launches in stream order (no atomics or fences between workgroups):
//  * fold: workgroup w < k(k+1)/2 folds upper-triangle Gram entry w (row-major
//    over x <= y) over the update blocks; the next workgroup folds the trace
//    partials. Each sum is split over 256 threads in a fixed stride and
//    combined by a fixed-order tree, so it is deterministic.
//  * finish (one workgroup): forms f_t = ||S||^2 - 2 tr + ||K_t||^2, runs the
//    stop test and publishes K_{t+1}.
__global__ __launch_bounds__(256) void finalize_fold_kernel(FitDev* fd, int nblk, int k,
                                                            const double* __restrict__ tr_part,
                                                            const float* __restrict__ gram_part,
                                                            int flags) {
    if (fd->done) return;
    __shared__ double red[4];
    const int tid = threadIdx.x;
    const int nup = k * (k + 1) / 2;
    const int wg = blockIdx.x;
    if (wg < nup) {
        if (!(flags & 4)) return;
        // upper-triangle entry number wg -> (x, y), x <= y
        int x = 0, rem = wg;
        while (rem >= k - x) {
            rem -= k - x;
            ++x;
        }
        const int y = x + rem;
        const int e = x * k + y;
        const int kk = k * k;
        double s = 0.0;
        for (int b = tid; b < nblk; b += 256) s += (double)gram_part[(int64_t)b * kk + e];
        s = block_sum256(s, red);
        if (tid == 0) fd->Kd[e] = s;
    } else if (flags & 1) {
        double s = 0.0;
        for (int b = tid; b < nblk; b += 256) s += tr_part[b];
        s = block_sum256(s, red);
        if (tid == 0) fd->tr = s;
    }
}

__global__ __launch_bounds__(256) void finalize_finish_kernel(FitDev* fd, double* f_trace, int t,
                                                              int k, int flags) {
    if (fd->done) return;
    __shared__ double red[4];
    const int tid = threadIdx.x;
    const int kk = k * k;
    if (flags & 4) {
        double k2 = 0.0;
        for (int idx = tid; idx < kk; idx += 256) {
            const int x = idx / k;
            const int y = idx % k;
            if (x <= y) {
                const double s = fd->Kd[idx];
                fd->K[x * kMaxK + y] = (float)s;
                fd->K[y * kMaxK + x] = (float)s;
                k2 += (x == y ? 1.0 : 2.0) * s * s;
            }
        }
        k2 = block_sum256(k2, red);
        if (tid == 0) fd->K2next = k2;
    }
    if (tid == 0) {
        if (flags & 8) {
            // initial Gram only: no objective, no trace entry
        } else if (flags & 1) {
            const double f = fd->S_fro2 - 2.0 * fd->tr + fd->K2;
            if (f_trace) f_trace[t] = f;
            if (!isfinite(f)) {
                fd->status = -4;
                fd->done = 1;
                fd->stop_iter = t;
            } else if ((flags & 2) && fd->tol > 0.0 && fd->f_prev_valid &&
                       fabs(fd->f_prev - f) < fd->tol * fmax(fabs(fd->f_prev), fd->floor_abs)) {
                fd->status = 1;
                fd->done = 1;
                fd->stop_iter = t;
            }
            fd->f_prev = f;
            fd->f_prev_valid = 1;
        } else {
            if (f_trace) f_trace[t] = __builtin_nan("");
            fd->f_prev_valid = 0;
        }
        if (flags & 4) fd->K2 = fd->K2next;
    }
}

hipError_t launch_finalize(FitDev* fd, double* f_trace, int t, int nblk, int k,
                           const double* tr_part, const float* gram_part, int flags,
                           hipStream_t st) {
    const int nup = k * (k + 1) / 2;
    hipLaunchKernelGGL(finalize_fold_kernel, dim3(nup + 1), dim3(256), 0, st, fd, nblk, k, tr_part,
                       gram_part, flags);
    hipLaunchKernelGGL(finalize_finish_kernel, dim3(1), dim3(256), 0, st, fd, f_trace, t, k, flags);
    return hipGetLastError();
}

// ---- labels (P1 "Factorizing with SymNMF": row-wise argmax) --------------------
__global__ void labels_kernel(const float* __restrict__ H, int64_t n, int k,
                              int32_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float* h = H + i * k;
    int best = 0;
    float bv = h[0];
    for (int c = 1; c < k; ++c) {
        const float v = h[c];
        if (v > bv) {  // strict: the lowest index wins ties
            bv = v;
            best = c;
        }
    }
    out[i] = best;
}
hipError_t launch_labels(const float* H, int64_t n, int k, int32_t* labels, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(labels_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, H, n,
                       k, labels);
    return hipGetLastError();
}

// Rows of the selected blocks only: blockIdx.y is the block's position in the
// list, blockIdx.x strides over its block_rows * k entries.
__global__ __launch_bounds__(256) void block_diff_kernel(const float* __restrict__ H,
                                                         const float* __restrict__ Ha,
                                                         const int* __restrict__ blocks,
                                                         int block_rows, int n, int k,
                                                         float* __restrict__ D,
                                                         const int* __restrict__ done) {
    if (done && *done) return;
    const int64_t base = (int64_t)blocks[blockIdx.y] * block_rows;
    const int64_t end = min((int64_t)n, base + block_rows) * k;
    for (int64_t e = base * k + (int64_t)blockIdx.x * 256 + threadIdx.x; e < end;
         e += (int64_t)gridDim.x * 256)
        D[e] = H[e] - Ha[e];
}

hipError_t launch_block_diff(const float* H, const float* Ha, const int* blocks, int nsel,
                             int block_rows, int n, int k, float* D, const int* done,
                             hipStream_t st) {
    if (nsel <= 0) return hipSuccess;
    const int64_t per = (int64_t)block_rows * k;
    const unsigned gx = (unsigned)std::min<int64_t>(64, (per + 255) / 256);
    hipLaunchKernelGGL(block_diff_kernel, dim3(gx, (unsigned)nsel), dim3(256), 0, st, H, Ha,
                       blocks, block_rows, n, k, D, done);
    return hipGetLastError();
}

__global__ void zero_rows_kernel(const float* __restrict__ H, int n, int k, int* out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    bool z = true;
    for (int c = 0; c < k; ++c) z = z && (H[(int64_t)i * k + c] == 0.f);
    if (z) atomicAdd(out, 1);
}
hipError_t launch_count_zero_rows(const float* H, int n, int k, int* out, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_rows_kernel, dim3((n + 255) / 256), dim3(256), 0, st, H, n, k, out);
    return hipGetLastError();
}

// ---- probe helpers ---------------------------------------------------------------
// C = A^T B partials over blocks of kCgRows rows. Thread (tx, ty) of a 16 x 16
// grid owns the TB x TB block of C at rows tx TB.., columns ty TB.. (w <= 16 TB):
// per staged row it reads TB values of A and TB of B from LDS and does TB^2
// FMAs. Each block's fp32 partial covers kCgRows rows; the blocks are folded in
// fp64 in a fixed order.
constexpr int kCgRows = 64;

template <int TB>
__global__ __launch_bounds__(256) void crossgram_kernel(const float* __restrict__ A,
                                                        const float* __restrict__ B, int n, int w,
                                                        float* __restrict__ part) {
    __shared__ float As[kCgRows][16 * TB + 1];
    __shared__ float Bs[kCgRows][16 * TB + 1];
    const int row0 = blockIdx.x * kCgRows;
    const int rows = min(kCgRows, n - row0);
    const int tid = threadIdx.x;
    for (int e = tid; e < kCgRows * w; e += 256) {
        const int i = e / w, c = e % w;
        As[i][c] = i < rows ? A[(int64_t)(row0 + i) * w + c] : 0.f;
        Bs[i][c] = i < rows ? B[(int64_t)(row0 + i) * w + c] : 0.f;
    }
    __syncthreads();
    const int tx = tid & 15, ty = tid >> 4;
    float acc[TB][TB];
#pragma unroll
    for (int a = 0; a < TB; ++a)
#pragma unroll
        for (int b = 0; b < TB; ++b) acc[a][b] = 0.f;
    const int x0 = tx * TB, y0 = ty * TB;
    if (x0 < w && y0 < w) {
        for (int i = 0; i < kCgRows; ++i) {
            float av[TB], bv[TB];
#pragma unroll
            for (int a = 0; a < TB; ++a) av[a] = (x0 + a < w) ? As[i][x0 + a] : 0.f;
#pragma unroll
            for (int b = 0; b < TB; ++b) bv[b] = (y0 + b < w) ? Bs[i][y0 + b] : 0.f;
#pragma unroll
            for (int a = 0; a < TB; ++a)
#pragma unroll
                for (int b = 0; b < TB; ++b) acc[a][b] = fmaf(av[a], bv[b], acc[a][b]);
        }
        float* out = part + (int64_t)blockIdx.x * w * w;
#pragma unroll
        for (int a = 0; a < TB; ++a)
#pragma unroll
            for (int b = 0; b < TB; ++b)
                if (x0 + a < w && y0 + b < w) out[(x0 + a) * w + y0 + b] = acc[a][b];
    }
}

// C[idx] = sum over blocks of part[b][idx] in fp64, fixed order: thread t of
// workgroup idx sums blocks t, t + 256, ...; then a fixed-order tree.
__global__ __launch_bounds__(256) void crossgram_final_kernel(const float* __restrict__ part,
                                                              int nblk, int ww,
                                                              double* __restrict__ C) {
    __shared__ double red[4];
    const int idx = blockIdx.x;
    double s = 0.0;
    for (int b = threadIdx.x; b < nblk; b += 256) s += (double)part[(int64_t)b * ww + idx];
    s = block_sum256(s, red);
    if (threadIdx.x == 0) C[idx] = s;
}

// Widths that are multiples of 16 (every probe width) run on the matrix core:
// C = A^T B partials over blocks of kCgRowsM rows with v_mfma_f32_16x16x4_f32
// (K = 4 rows per step). Wave v owns the 16 x 16 tiles (ti, tj) of C with
// ti = v, v + 4, ...; lane l = 16 g + m supplies A[row0 + g][16 ti + m] and
// B[row0 + g][16 tj + m] and holds C[16 ti + 4 g + r][16 tj + m]. Rows past
// n read row n - 1 and count zero.
constexpr int kCgRowsM = 512;

template <int NT>
__global__ __launch_bounds__(256) void crossgram_mfma_kernel(const float* __restrict__ A,
                                                             const float* __restrict__ B, int n,
                                                             float* __restrict__ part) {
    constexpr int w = 16 * NT;
    constexpr int TI = (NT + 3) / 4;  // tile rows per wave
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4, m = lane & 15;
    const int row0 = blockIdx.x * kCgRowsM;
    const int row1 = min(n, row0 + kCgRowsM);
    floatx4 acc[TI][NT];
#pragma unroll
    for (int a = 0; a < TI; ++a)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[a][t] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int r = row0; r < row1; r += 4) {
        const int row = r + g;
        const bool ok = row < row1;
        const int64_t base = (int64_t)(ok ? row : n - 1) * w + m;
        float av[TI], bv[NT];
#pragma unroll
        for (int a = 0; a < TI; ++a) {
            const int ti = wave + 4 * a;
            av[a] = (ti < NT && ok) ? A[base + 16 * ti] : 0.f;
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) bv[t] = ok ? B[base + 16 * t] : 0.f;
#pragma unroll
        for (int a = 0; a < TI; ++a)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[a][t] = mfma16x16x4(av[a], bv[t], acc[a][t]);
    }
    float* out = part + (int64_t)blockIdx.x * w * w;
#pragma unroll
    for (int a = 0; a < TI; ++a) {
        const int ti = wave + 4 * a;
        if (ti < NT)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) out[(16 * ti + 4 * g + r) * w + 16 * t + m] = acc[a][t][r];
    }
}

// C[idx] = sum over blocks b in order of part[b][idx] (fp64), one thread per
// entry, so consecutive threads read consecutive entries of each block.
__global__ __launch_bounds__(256) void crossgram_fold_kernel(const float* __restrict__ part,
                                                             int nblk, int ww,
                                                             double* __restrict__ C) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= ww) return;
    double s = 0.0;
    for (int b = 0; b < nblk; ++b) s += (double)part[(int64_t)b * ww + idx];
    C[idx] = s;
}

int crossgram_blocks(int n) {
    return std::max((n + kCgRows - 1) / kCgRows, (n + kCgRowsM - 1) / kCgRowsM);
}

hipError_t launch_crossgram(const float* A, const float* B, int n, int w, float* part, int nblk,
                            double* C, hipStream_t st) {
    if (w % 16 == 0 && w <= 128) {
        const int nb = (n + kCgRowsM - 1) / kCgRowsM;
        if (nb > nblk) return hipErrorInvalidValue;
        switch (w / 16) {
#define CGM_CASE(T)                                                                          \
    case T:                                                                                  \
        hipLaunchKernelGGL(crossgram_mfma_kernel<T>, dim3(nb), dim3(256), 0, st, A, B, n, part); \
        break;
            CGM_CASE(1) CGM_CASE(2) CGM_CASE(3) CGM_CASE(4) CGM_CASE(5) CGM_CASE(6) CGM_CASE(7)
            CGM_CASE(8)
#undef CGM_CASE
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int ww = w * w;
        hipLaunchKernelGGL(crossgram_fold_kernel, dim3((ww + 255) / 256), dim3(256), 0, st, part,
                           nb, ww, C);
        return hipGetLastError();
    }
    const int tb = (w + 15) / 16;
    switch (tb) {
#define CG_CASE(T)                                                                            \
    case T:                                                                                   \
        hipLaunchKernelGGL(crossgram_kernel<T>, dim3(nblk), dim3(256), 0, st, A, B, n, w, part); \
        break;
        CG_CASE(1) CG_CASE(2) CG_CASE(3) CG_CASE(4) CG_CASE(5) CG_CASE(6) CG_CASE(7) CG_CASE(8)
#undef CG_CASE
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ww = w * w;
    hipLaunchKernelGGL(crossgram_final_kernel, dim3(ww), dim3(256), 0, st, part, nblk, ww, C);
    return hipGetLastError();
}

// Q = Y M, one thread per output element, M staged in LDS.
__global__ __launch_bounds__(256) void rowmat_kernel(const float* __restrict__ Y,
                                                     const float* __restrict__ M, int n, int w,
                                                     float* __restrict__ Q) {
    extern __shared__ float Ms[];
    for (int e = threadIdx.x; e < w * w; e += 256) Ms[e] = M[e];
    __syncthreads();
    const int64_t total = (int64_t)n * w;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * 256) {
        const int64_t i = e / w;
        const int c = (int)(e % w);
        const float* y = Y + i * w;
        float s = 0.f;
        for (int d = 0; d < w; ++d) s = fmaf(y[d], Ms[d * w + c], s);
        Q[e] = s;
    }
}
// Q = Y M on the matrix core for w a multiple of 16: a wave computes 16 rows x
// all w columns; per 16-column K block lane l = 16 g + m loads Y[row m][16 kb
// + 4 g .. + 3] as one float4 and runs 4 x NT v_mfma_f32_16x16x4_f32 with B =
// M[16 kb + 4 g + e][16 t + m] from LDS (M staged once per workgroup).
template <int NT>
__global__ __launch_bounds__(256) void rowmat_mfma_kernel(const float* __restrict__ Y,
                                                          const float* __restrict__ M, int n,
                                                          float* __restrict__ Q) {
    constexpr int w = 16 * NT;
    extern __shared__ float Ms[];
    for (int e = threadIdx.x; e < w * w; e += 256) Ms[e] = M[e];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4, m = lane & 15;
    const int row0 = (blockIdx.x * 4 + wave) * 16;
    if (row0 >= n) return;
    const float* y = Y + (int64_t)min(row0 + m, n - 1) * w + 4 * g;
    floatx4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NT; ++kb) {
        const float4 y4 = *reinterpret_cast<const float4*>(y + 16 * kb);
        const float yv[4] = {y4.x, y4.y, y4.z, y4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float* mrow = Ms + (16 * kb + 4 * g + e) * w + m;
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = mfma16x16x4(yv[e], mrow[16 * t], acc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = row0 + 4 * g + r;
            if (i < n) Q[(int64_t)i * w + 16 * t + m] = acc[t][r];
        }
}

hipError_t launch_rowmat(const float* Y, const float* M, int n, int w, float* Q, hipStream_t st) {
    if (w % 16 == 0 && w <= 128 && reinterpret_cast<uintptr_t>(Y) % 16 == 0) {
        const unsigned blocks = (unsigned)((n + 63) / 64);
        const size_t shm = (size_t)w * w * sizeof(float);
        switch (w / 16) {
#define RM_CASE(T)                                                                             \
    case T:                                                                                    \
        hipLaunchKernelGGL(rowmat_mfma_kernel<T>, dim3(blocks), dim3(256), shm, st, Y, M, n, Q); \
        break;
            RM_CASE(1) RM_CASE(2) RM_CASE(3) RM_CASE(4) RM_CASE(5) RM_CASE(6) RM_CASE(7) RM_CASE(8)
#undef RM_CASE
        }
        return hipGetLastError();
    }
    const int64_t total = (int64_t)n * w;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(rowmat_kernel, dim3((unsigned)blocks), dim3(256),
                       (size_t)w * w * sizeof(float), st, Y, M, n, w, Q);
    return hipGetLastError();
}

}  // namespace symnmf
