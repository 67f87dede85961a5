// libsymnmf host side: the C ABI of include/symnmf.h, argument validation,
// workspace layout, the AdaptGrow controller, the spectral probe's small fp64
// algebra and kernel timing. Every step of the path runs in the gfx950
// kernels of k_*.hip; this file only sequences launches and handles scalars.
//
// Pages: P1 "GPU-Accelerated Clustering for Financial Instruments at Scale";
// P2 "GPU-Accelerated SymNMF Clustering Scales to a Million Financial
// Instruments" (AdaGrad update, AdaptGrow sketch); P3 the SymNMF study
// abstract on the paper-card page "GEM-KMeans: ...".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstddef>
#include <cstring>
#include <limits>
#include <mutex>
#include <vector>

#include "common.h"
#include "kernels.h"
#include "symnmf.h"

using namespace symnmf;

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Bump allocator over the caller's workspace. With base == nullptr it only
// measures.
struct Carve {
    char* base;
    size_t off = 0;
    explicit Carve(void* b) : base(static_cast<char*>(b)) {}
    template <class T>
    T* take(size_t count) {
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off = align_up(off + count * sizeof(T));
        return p;
    }
};

// ---------------------------------------------------------------------------
// kernel timing
struct ProfEntry {
    hipEvent_t a, b;
    int which;
    double bytes;
    int64_t tag;  // -1, or (fit call << 32 | step) for launches a stopped fit may skip
};
struct Prof {
    std::mutex mu;
    std::atomic<bool> on{false};  // read by launches on any thread
    std::vector<ProfEntry> pending;
    int64_t launches[SYMNMF_PROF_COUNT] = {};
    double ms[SYMNMF_PROF_COUNT] = {};
    double bytes[SYMNMF_PROF_COUNT] = {};
};
Prof& prof() {
    static Prof p;
    return p;
}

struct ProfScope {
    hipEvent_t a = nullptr, b = nullptr;
    hipStream_t st;
    int which;
    double bytes;
    int64_t tag;
    ProfScope(int w, double by, hipStream_t s, int64_t tg = -1)
        : st(s), which(w), bytes(by), tag(tg) {
        Prof& p = prof();
        if (!p.on) return;
        if (hipEventCreate(&a) != hipSuccess) {
            a = nullptr;
            return;
        }
        if (hipEventCreate(&b) != hipSuccess) {
            (void)hipEventDestroy(a);
            a = b = nullptr;
            return;
        }
        (void)hipEventRecord(a, st);
    }
    ~ProfScope() {
        if (!a) return;
        (void)hipEventRecord(b, st);
        Prof& p = prof();
        std::lock_guard<std::mutex> g(p.mu);
        p.pending.push_back({a, b, which, bytes, tag});
    }
};

void prof_drain() {
    Prof& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    for (auto& e : p.pending) {
        (void)hipEventSynchronize(e.b);
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, e.a, e.b) == hipSuccess) {
            p.launches[e.which] += 1;
            p.ms[e.which] += ms;
            p.bytes[e.which] += e.bytes;
        }
        (void)hipEventDestroy(e.a);
        (void)hipEventDestroy(e.b);
    }
    p.pending.clear();
}

// Drops the pending timings tagged [lo, hi]: launches a fit enqueued after its
// device stop flag was set, which returned without doing their work (their
// durations would pull the kernels' averages down).
void prof_discard(int64_t lo, int64_t hi) {
    Prof& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    size_t keep = 0;
    for (size_t i = 0; i < p.pending.size(); ++i) {
        ProfEntry& e = p.pending[i];
        if (e.tag >= lo && e.tag <= hi) {
            (void)hipEventSynchronize(e.b);
            (void)hipEventDestroy(e.a);
            (void)hipEventDestroy(e.b);
        } else {
            p.pending[keep++] = e;
        }
    }
    p.pending.resize(keep);
}
std::atomic<int64_t> g_fit_calls{0};

#define HIPCHK(x)                                   \
    do {                                            \
        hipError_t _e = (x);                        \
        if (_e != hipSuccess) return SYMNMF_E_HIP;  \
    } while (0)

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---------------------------------------------------------------------------
// S.H pass planning
struct FullPlan {
    RowPlan rp;
    int nsplit;
};
FullPlan full_plan(int n) {
    const int rps = sh_full_rows_per_split(n);
    FullPlan fp;
    fp.nsplit = (int)cdiv(n, rps);
    fp.rp = RowPlan{n, rps, nullptr, 0, 0, 1, 0, 1};
    return fp;
}
FullPlan sampled_plan(int n, const int* blocks_dev, int nsel, int block_rows) {
    FullPlan fp;
    RowPlan rp{n, 0, blocks_dev, nsel, block_rows, 1, 0, 1};
    if (nsel < kMaxSplits) {
        int sub = std::max(1, std::min(kMaxSplits / nsel, block_rows / 64));
        rp.sub = sub;
        rp.seg = (int)round_up(cdiv(block_rows, sub), 4);
        rp.bps = 1;
        fp.nsplit = nsel * sub;
    } else {
        rp.sub = 1;
        rp.seg = block_rows;  // read when one block per split remains (nsel == kMaxSplits)
        rp.bps = (int)cdiv(nsel, kMaxSplits);
        fp.nsplit = (int)cdiv(nsel, rp.bps);
    }
    fp.rp = rp;
    return fp;
}
inline int ldp_of(int width) { return (int)round_up(width, 4); }

// ---------------------------------------------------------------------------
// Small dense fp64 algebra for the probe (host side; w <= 128).

// Cyclic Jacobi eigen-decomposition of a symmetric w x w matrix A (row-major,
// destroyed). Eigenvalues to ev; eigenvectors (columns of V) if V != nullptr.
void jacobi_eig(int w, std::vector<double>& A, std::vector<double>& ev, std::vector<double>* V) {
    if (V) {
        V->assign((size_t)w * w, 0.0);
        for (int i = 0; i < w; ++i) (*V)[(size_t)i * w + i] = 1.0;
    }
    for (int sweep = 0; sweep < 100; ++sweep) {
        double off = 0.0, diag = 0.0;
        for (int i = 0; i < w; ++i)
            for (int j = 0; j < w; ++j) {
                const double a = A[(size_t)i * w + j];
                if (i != j) off += a * a; else diag += a * a;
            }
        if (off <= 1e-30 * diag || off == 0.0) break;
        for (int p = 0; p < w - 1; ++p)
            for (int q = p + 1; q < w; ++q) {
                const double apq = A[(size_t)p * w + q];
                if (apq == 0.0) continue;
                const double app = A[(size_t)p * w + p], aqq = A[(size_t)q * w + q];
                const double theta = (aqq - app) / (2.0 * apq);
                const double t = (theta >= 0 ? 1.0 : -1.0) /
                                 (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
                const double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
                for (int r = 0; r < w; ++r) {  // columns p, q
                    const double arp = A[(size_t)r * w + p], arq = A[(size_t)r * w + q];
                    A[(size_t)r * w + p] = c * arp - s * arq;
                    A[(size_t)r * w + q] = s * arp + c * arq;
                }
                for (int r = 0; r < w; ++r) {  // rows p, q
                    const double apr = A[(size_t)p * w + r], aqr = A[(size_t)q * w + r];
                    A[(size_t)p * w + r] = c * apr - s * aqr;
                    A[(size_t)q * w + r] = s * apr + c * aqr;
                }
                if (V)
                    for (int r = 0; r < w; ++r) {
                        const double vrp = (*V)[(size_t)r * w + p], vrq = (*V)[(size_t)r * w + q];
                        (*V)[(size_t)r * w + p] = c * vrp - s * vrq;
                        (*V)[(size_t)r * w + q] = s * vrp + c * vrq;
                    }
            }
    }
    ev.resize(w);
    for (int i = 0; i < w; ++i) ev[i] = A[(size_t)i * w + i];
}

// Eigenvalues of a symmetric w x w matrix A (row-major, destroyed): Householder
// reduction to tridiagonal form, then implicit symmetric QR steps with
// Wilkinson shifts and deflation (Golub and Van Loan, "Matrix Computations",
// Algorithms 8.3.1 and 8.3.2). O(w^3) once, then O(w) per QR step; at most
// 64 w steps (a few per eigenvalue are the norm).
void sym_eigvals(int w, std::vector<double>& A, std::vector<double>& ev) {
    auto at = [&](int i, int j) -> double& { return A[(size_t)i * w + j]; };
    std::vector<double> v(w), p(w);
    for (int k = 0; k + 2 < w; ++k) {
        const int m = w - k - 1;  // entries k+1 .. w-1 of column k
        double xn2 = 0.0;
        for (int i = 0; i < m; ++i) xn2 += at(k + 1 + i, k) * at(k + 1 + i, k);
        const double xn = std::sqrt(xn2);
        if (xn == 0.0) continue;
        const double x0 = at(k + 1, k);
        const double alpha = x0 >= 0.0 ? -xn : xn;
        for (int i = 0; i < m; ++i) v[i] = at(k + 1 + i, k);
        v[0] -= alpha;
        double vtv = 0.0;
        for (int i = 0; i < m; ++i) vtv += v[i] * v[i];
        if (vtv == 0.0) continue;
        const double beta = 2.0 / vtv;
        // p = beta B v for the trailing block B = A[k+1.., k+1..]
        double vtp = 0.0;
        for (int i = 0; i < m; ++i) {
            double s = 0.0;
            for (int j = 0; j < m; ++j) s += at(k + 1 + i, k + 1 + j) * v[j];
            p[i] = beta * s;
            vtp += v[i] * p[i];
        }
        const double gam = 0.5 * beta * vtp;
        for (int i = 0; i < m; ++i) p[i] -= gam * v[i];  // q
        for (int i = 0; i < m; ++i)
            for (int j = 0; j < m; ++j) at(k + 1 + i, k + 1 + j) -= v[i] * p[j] + p[i] * v[j];
        at(k + 1, k) = at(k, k + 1) = alpha;
        for (int i = 1; i < m; ++i) at(k + 1 + i, k) = at(k, k + 1 + i) = 0.0;
    }
    std::vector<double> d(w), e(w, 0.0);
    for (int i = 0; i < w; ++i) d[i] = at(i, i);
    for (int i = 0; i + 1 < w; ++i) e[i] = at(i + 1, i);
    const double eps = std::numeric_limits<double>::epsilon();
    int hi = w - 1, guard = 0;
    while (hi > 0 && guard < 64 * w) {
        if (std::fabs(e[hi - 1]) <= eps * (std::fabs(d[hi - 1]) + std::fabs(d[hi]))) {
            e[hi - 1] = 0.0;
            --hi;
            continue;
        }
        int lo = hi - 1;
        while (lo > 0 && std::fabs(e[lo - 1]) > eps * (std::fabs(d[lo - 1]) + std::fabs(d[lo]))) --lo;
        ++guard;
        // Wilkinson shift: the eigenvalue of the trailing 2 x 2 closer to d[hi]
        const double a = d[hi - 1], b = e[hi - 1], c = d[hi];
        const double delta = 0.5 * (a - c);
        const double sg = delta >= 0.0 ? 1.0 : -1.0;
        const double mu = c - b * b / (delta + sg * std::hypot(delta, b));
        double x = d[lo] - mu, z = e[lo];
        for (int k = lo; k < hi; ++k) {
            const double r = std::hypot(x, z);
            const double cs = r == 0.0 ? 1.0 : x / r, sn = r == 0.0 ? 0.0 : z / r;
            if (k > lo) e[k - 1] = r;
            const double dk = d[k], ek = e[k], dk1 = d[k + 1];
            d[k] = cs * cs * dk + 2.0 * cs * sn * ek + sn * sn * dk1;
            d[k + 1] = sn * sn * dk - 2.0 * cs * sn * ek + cs * cs * dk1;
            e[k] = cs * sn * (dk1 - dk) + (cs * cs - sn * sn) * ek;
            if (k + 1 < hi) {
                const double f = e[k + 1];
                z = sn * f;
                e[k + 1] = cs * f;
                x = e[k];
            }
        }
    }
    ev = d;
}

// sum_{k < len} a[k] b[k] with four interleaved partial sums (fixed order).
inline double dot4(const double* a, const double* b, int len) {
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    int k = 0;
    for (; k + 4 <= len; k += 4) {
        s0 += a[k] * b[k];
        s1 += a[k + 1] * b[k + 1];
        s2 += a[k + 2] * b[k + 2];
        s3 += a[k + 3] * b[k + 3];
    }
    for (; k < len; ++k) s0 += a[k] * b[k];
    return (s0 + s1) + (s2 + s3);
}

// G = L L^T with L lower triangular (row-major, so every inner product below
// runs over contiguous memory); false on a pivot below rel * G_jj.
bool cholesky_lower(int w, const std::vector<double>& G, std::vector<double>& L, double rel) {
    L.assign((size_t)w * w, 0.0);
    for (int j = 0; j < w; ++j) {
        const double* Lj = &L[(size_t)j * w];
        const double d = G[(size_t)j * w + j] - dot4(Lj, Lj, j);
        if (!(d > rel * G[(size_t)j * w + j]) || !std::isfinite(d)) return false;
        const double ljj = std::sqrt(d);
        L[(size_t)j * w + j] = ljj;
        for (int i = j + 1; i < w; ++i)
            L[(size_t)i * w + j] = (G[(size_t)i * w + j] - dot4(&L[(size_t)i * w], Lj, j)) / ljj;
    }
    return true;
}

// Ri = (L^T)^-1 (upper triangular) = (L^-1)^T: row j of Ri is column j of
// L^-1, by forward substitution on L x = e_j.
void lower_inverse_transposed(int w, const std::vector<double>& L, std::vector<double>& Ri) {
    Ri.assign((size_t)w * w, 0.0);
    for (int j = 0; j < w; ++j) {
        double* x = &Ri[(size_t)j * w];
        x[j] = 1.0 / L[(size_t)j * w + j];
        for (int i = j + 1; i < w; ++i) {
            const double* Li = &L[(size_t)i * w];
            x[i] = -dot4(Li + j, x + j, i - j) / Li[i];
        }
    }
}

// ---------------------------------------------------------------------------
// workspace layouts

struct ShLayout {
    float* part;
    double* tr_part;
    double* tr_out;
};
size_t sh_layout(void* ws, int64_t n, int width, ShLayout* L) {
    Carve c(ws);
    FullPlan fp = full_plan((int)n);
    ShLayout l;
    l.part = c.take<float>((size_t)fp.nsplit * n * ldp_of(width));
    l.tr_part = c.take<double>((size_t)cdiv(n, kUpdRows));
    l.tr_out = c.take<double>(1);
    if (L) *L = l;
    return c.off;
}

struct KmeansLayout {
    float *rinv, *Ct, *W, *C, *part;
    int32_t *lab[2], *idx, *changes;
    double *obj_part, *obj, *col_part, *norm;
};
size_t kmeans_layout(void* ws, int64_t n, int k, KmeansLayout* L) {
    Carve c(ws);
    FullPlan fp = full_plan((int)n);
    const int64_t nblk = cdiv(n, 256);
    KmeansLayout l;
    l.rinv = c.take<float>((size_t)n);
    l.Ct = c.take<float>((size_t)n * k);
    l.W = c.take<float>((size_t)n * k);
    l.C = c.take<float>((size_t)n * k);
    l.part = c.take<float>((size_t)fp.nsplit * n * ldp_of(k));
    for (int i = 0; i < 2; ++i) l.lab[i] = c.take<int32_t>((size_t)n);
    l.idx = c.take<int32_t>((size_t)k);
    l.changes = c.take<int32_t>(1);
    l.obj_part = c.take<double>((size_t)nblk);
    l.obj = c.take<double>(1);
    l.col_part = c.take<double>((size_t)nblk * k);
    l.norm = c.take<double>((size_t)k);
    if (L) *L = l;
    return c.off;
}

struct SqLayout {
    void* qs;  // Q packed into the matrix core's B operands
    float* part;
};
size_t sq_layout(void* ws, int64_t n, int width, SqLayout* L) {
    Carve c(ws);
    const SqPlan sp = sq_plan((int)n, width);
    SqLayout l;
    l.qs = c.take<char>(sp.packed_bytes);
    l.part = c.take<float>((size_t)sp.nsplit * n * ldp_of(width));
    if (L) *L = l;
    return c.off;
}

struct SymLayout {
    void* hsr;  // H packed for the row side
    void* hsc;  // H packed for the column side
    float* p1;
    float* p2;
    double* tr_part;
    double* tr_out;
};
size_t sym_layout(void* ws, int64_t n, int k, SymLayout* L) {
    Carve c(ws);
    const SymPlan sp = sym_plan((int)n, k);
    SymLayout l;
    l.hsr = c.take<char>(sp.packed_row_bytes);
    l.hsc = c.take<char>(sp.packed_col_bytes);
    l.p1 = c.take<float>(sp.p1_floats);
    l.p2 = c.take<float>(sp.p2_floats);
    l.tr_part = c.take<double>((size_t)cdiv(n, kUpdRows));
    l.tr_out = c.take<double>(1);
    if (L) *L = l;
    return c.off;
}

struct ProbeLayout {
    float *Q, *Y, *part, *M, *cg_part;
    double* C;
    void* qs;
};
// Subspace width: 2p columns (rounded up to 16) where the widest pass (128)
// and n allow, and never fewer than p + 16. Convergence goes with
// |lambda_{w+1} / lambda_p| per step, while a pass costs little more at 128
// columns than at 80 on the bf16 matrix cores, so the wide block converges in
// less time overall.
int probe_width(int p, int64_t n) {
    const int64_t base = round_up(p + 16, 16);
    const int64_t wide = std::min<int64_t>(round_up(2 * (int64_t)p, 16),
                                           std::min<int64_t>(kMaxWidth, n / 16 * 16));
    return (int)std::max(base, wide);
}
size_t probe_layout(void* ws, int64_t n, int p, ProbeLayout* L) {
    Carve c(ws);
    const int w = probe_width(p, n);
    ProbeLayout l;
    const SqPlan sp = sq_plan((int)n, w);
    l.Q = c.take<float>((size_t)n * w);
    l.Y = c.take<float>((size_t)n * w);
    l.part = c.take<float>((size_t)sp.nsplit * n * ldp_of(w));
    l.qs = c.take<char>(sp.packed_bytes);
    l.M = c.take<float>((size_t)w * w);
    l.cg_part = c.take<float>((size_t)crossgram_blocks((int)n) * w * w);
    l.C = c.take<double>((size_t)w * w);
    if (L) *L = l;
    return c.off;
}

struct FitLayout {
    FitDev* fd;
    double* f_trace;
    float *Hb[2], *Gb[2], *Ha[2], *Pa[2], *D, *part, *gram_part;
    void *sym_hsr, *sym_hsc;  // upper-triangle pass (sh_pass UPPER only)
    float *sym_p1, *sym_p2;
    double *tr_part, *stats_part, *stats_out;
    int *blocks, *zero_rows;
};
size_t fit_layout(void* ws, int64_t n, int k, int max_iters, int block_rows, int sh_pass,
                  FitLayout* L) {
    Carve c(ws);
    const int nb = (int)cdiv(n, block_rows);
    const int nblk = (int)cdiv(n, kUpdRows);
    FitLayout l;
    l.fd = c.take<FitDev>(1);
    l.f_trace = c.take<double>((size_t)std::max(1, max_iters));
    for (int i = 0; i < 2; ++i) l.Hb[i] = c.take<float>((size_t)n * k);
    for (int i = 0; i < 2; ++i) l.Gb[i] = c.take<float>((size_t)n * k);
    for (int i = 0; i < 2; ++i) l.Ha[i] = c.take<float>((size_t)n * k);
    for (int i = 0; i < 2; ++i) l.Pa[i] = c.take<float>((size_t)n * k);
    l.D = c.take<float>((size_t)n * k);
    l.part = c.take<float>((size_t)kMaxSplits * n * ldp_of(k));
    l.gram_part = c.take<float>((size_t)nblk * k * k);
    l.tr_part = c.take<double>((size_t)nblk);
    l.stats_part = c.take<double>((size_t)2 * cdiv(n, kStatsRows));
    l.stats_out = c.take<double>(2);
    l.blocks = c.take<int>((size_t)2 * nb + 16);
    l.zero_rows = c.take<int>(1);
    l.sym_hsr = l.sym_hsc = nullptr;
    l.sym_p1 = l.sym_p2 = nullptr;
    if (sh_pass == SYMNMF_SH_UPPER) {
        const SymPlan sp = sym_plan((int)n, k);
        l.sym_hsr = c.take<char>(sp.packed_row_bytes);
        l.sym_hsc = c.take<char>(sp.packed_col_bytes);
        l.sym_p1 = c.take<float>(sp.p1_floats);
        l.sym_p2 = c.take<float>(sp.p2_floats);
    }
    if (L) *L = l;
    return c.off;
}

struct BuildLayout {
    float* Z;  // Z or Theta
    int *R, *hist, *sel, *flags;
    double *radius, *part2, *fro;
};
size_t build_layout(void* ws, int kind, int64_t T, int64_t n, BuildLayout* L) {
    Carve c(ws);
    const int64_t ldz = round_up(n, kGramTile);
    BuildLayout l{};
    if (kind == SYMNMF_ABSCORR) {
        // days padded to whole 32-day steps of the split Gram pass
        l.Z = c.take<float>((size_t)round_up(T, 32) * ldz);
    } else {
        // Theta needs m_p = round_up(ceil(tail_frac T), 4) <= round_up(T, 4) rows
        l.Z = c.take<float>((size_t)round_up(T, 4) * ldz);
        l.R = c.take<int>((size_t)T * n);
        l.hist = c.take<int>((size_t)T * (T + 1));
        l.sel = c.take<int>((size_t)T);
        l.radius = c.take<double>((size_t)T);
    }
    l.flags = c.take<int>(2);
    l.part2 = c.take<double>((size_t)gram_build_tiles((int)n));
    l.fro = c.take<double>(1);
    if (L) *L = l;
    return c.off;
}

bool ws_ok(void* ws, size_t ws_bytes, size_t need) {
    return ws != nullptr && aligned(ws, kAlign) && ws_bytes >= need;
}

}  // namespace

// ===========================================================================
extern "C" {

int symnmf_abi_version(void) { return SYMNMF_ABI_VERSION; }

const char* symnmf_status_string(int status) {
    switch (status) {
        case SYMNMF_OK: return "ok";
        case SYMNMF_W_NOT_CONVERGED: return "not converged within max_iters";
        case SYMNMF_E_INVALID: return "invalid argument";
        case SYMNMF_E_WORKSPACE: return "workspace missing, misaligned or too small";
        case SYMNMF_E_HIP: return "HIP runtime error";
        case SYMNMF_E_NONFINITE: return "non-finite value in input or objective";
        case SYMNMF_E_DEGENERATE: return "constant column: correlation undefined";
        case SYMNMF_E_TOO_LARGE:
            return "problem too large for the 64 MiB static scratch of symnmf_sh_noalloc";
        default: return "unknown status";
    }
}

void symnmf_fit_params_default(symnmf_fit_params* p) {
    if (!p) return;
    std::memset(p, 0, sizeof(*p));
    p->solver = SYMNMF_AUTO;
    p->max_iters = 2000;
    p->lr = 0.0;
    p->eps = 1e-8;
    p->block_rows = 1024;
    p->init = SYMNMF_INIT_SCALE_MATCHED;
    p->phi0 = 0.0;
    p->gap_threshold = 5.0;
    p->tol_rel = 1e-6;
    p->stall_tol = 1e-3;
    p->init_scale = 0.1;
    p->seed = 0;
    p->check_every = 16;
    p->resume = 0;
    p->rms_decay = 0.0;
    p->sh_pass = SYMNMF_SH_ROWS;
    p->obj_floor = 0.05;
    p->start_iter = 0;
}

size_t symnmf_workspace_bytes(int op, int64_t n, int32_t k_or_p, int64_t T,
                              const symnmf_fit_params* prm) {
    if (n < 1 || n > INT32_MAX / 2) return 0;
    switch (op) {
        case SYMNMF_OP_BUILD_S:
            if (T < 2 || T > 65536) return 0;
            return std::max(build_layout(nullptr, SYMNMF_ABSCORR, T, n, nullptr),
                            build_layout(nullptr, SYMNMF_TPDM, T, n, nullptr));
        case SYMNMF_OP_PROBE:
            if (k_or_p < 1 || probe_width(k_or_p, n) > kMaxWidth) return 0;
            return probe_layout(nullptr, n, k_or_p, nullptr);
        case SYMNMF_OP_SH:
            if (k_or_p < 1 || k_or_p > kMaxWidth) return 0;
            return sh_layout(nullptr, n, k_or_p, nullptr);
        case SYMNMF_OP_SQ:
            if (k_or_p < 1 || k_or_p > kMaxWidth) return 0;
            return sq_layout(nullptr, n, k_or_p, nullptr);
        case SYMNMF_OP_SH_SYM:
            if (k_or_p < 1 || k_or_p > kSymMaxK) return 0;
            return sym_layout(nullptr, n, k_or_p, nullptr);
        case SYMNMF_OP_KMEANS:
            if (k_or_p < 1 || k_or_p > kMaxK || k_or_p > n) return 0;
            return kmeans_layout(nullptr, n, k_or_p, nullptr);
        case SYMNMF_OP_FIT: {
            if (k_or_p < 1 || k_or_p > kMaxK) return 0;
            symnmf_fit_params d;
            symnmf_fit_params_default(&d);
            const symnmf_fit_params* p = prm ? prm : &d;
            if (p->max_iters < 0 || p->block_rows < 4) return 0;
            if (p->sh_pass == SYMNMF_SH_UPPER && k_or_p > kSymMaxK) return 0;
            return fit_layout(nullptr, n, k_or_p, p->max_iters, p->block_rows, p->sh_pass,
                              nullptr);
        }
        default: return 0;
    }
}

void symnmf_profile_enable(int on) {
    Prof& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    p.on = on != 0;
}
void symnmf_profile_reset(void) {
    prof_drain();
    Prof& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    for (int i = 0; i < SYMNMF_PROF_COUNT; ++i) {
        p.launches[i] = 0;
        p.ms[i] = 0.0;
        p.bytes[i] = 0.0;
    }
}
int symnmf_profile_read(int which, int64_t* launches, double* total_ms, double* total_bytes) {
    if (which < 0 || which >= SYMNMF_PROF_COUNT) return SYMNMF_E_INVALID;
    prof_drain();
    Prof& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    if (launches) *launches = p.launches[which];
    if (total_ms) *total_ms = p.ms[which];
    if (total_bytes) *total_bytes = p.bytes[which];
    return SYMNMF_OK;
}

// ---------------------------------------------------------------------------
int symnmf_labels(const float* H, int64_t n, int32_t k, int32_t* labels, void* hip_stream) {
    if (n == 0 && k >= 1) return SYMNMF_OK;  // empty input: nothing to do, pointers unused
    if (!H || !labels || n < 0 || k < 1 || n > INT32_MAX) return SYMNMF_E_INVALID;
    HIPCHK(launch_labels(H, n, k, labels, as_stream(hip_stream)));
    return SYMNMF_OK;
}

// ---------------------------------------------------------------------------
int symnmf_sh(const float* S, int64_t n, int64_t lds, const float* H, int32_t k, float* P,
              double* tr_host, void* ws, size_t ws_bytes, void* hip_stream) {
    if (!S || !H || !P || n < 1 || n > INT32_MAX / 2 || k < 1 || k > kMaxWidth || lds < n ||
        lds % 4 || !aligned(S, 16) || !aligned(P, 4))
        return SYMNMF_E_INVALID;
    const size_t need = sh_layout(nullptr, n, k, nullptr);
    if (!ws_ok(ws, ws_bytes, need)) return SYMNMF_E_WORKSPACE;
    ShLayout L;
    sh_layout(ws, n, k, &L);
    hipStream_t st = as_stream(hip_stream);
    FullPlan fp = full_plan((int)n);
    const int ldp = ldp_of(k);
    {
        ProfScope ps(SYMNMF_PROF_SH_FULL, 4.0 * n * (double)n + 8.0 * n * k, st);
        HIPCHK(launch_sh_panel(S, lds, H, k, fp.rp, fp.nsplit, L.part, ldp, st));
    }
    HIPCHK(launch_reduce_partials(L.part, fp.nsplit, (int)n, k, ldp, P, H, L.tr_part, st));
    if (tr_host) {
        HIPCHK(launch_sum_doubles(L.tr_part, cdiv(n, kUpdRows), L.tr_out, st));
        HIPCHK(hipMemcpyAsync(tr_host, L.tr_out, sizeof(double), hipMemcpyDeviceToHost, st));
        HIPCHK(hipStreamSynchronize(st));
    }
    return SYMNMF_OK;
}

int symnmf_sq(const float* S, int64_t n, int64_t lds, const float* Q, int32_t w, float* Y,
              void* ws, size_t ws_bytes, void* hip_stream) {
    if (!S || !Q || !Y || n < 1 || n > INT32_MAX / 2 || w < 1 || w > kMaxWidth || lds < n ||
        lds % 4 || !aligned(S, 16) || !aligned(Q, 4) || !aligned(Y, 4))
        return SYMNMF_E_INVALID;
    const size_t need = sq_layout(nullptr, n, w, nullptr);
    if (!ws_ok(ws, ws_bytes, need)) return SYMNMF_E_WORKSPACE;
    SqLayout L;
    sq_layout(ws, n, w, &L);
    hipStream_t st = as_stream(hip_stream);
    const SqPlan sp = sq_plan((int)n, w);
    const int ldp = ldp_of(w);
    HIPCHK(launch_sq_pack(Q, w, (int)n, w, sp, L.qs, st));
    {
        ProfScope ps(SYMNMF_PROF_SH_PROBE, 4.0 * n * (double)n + 8.0 * n * w, st);
        HIPCHK(launch_sq_split(S, lds, L.qs, (int)n, w, sp, L.part, ldp, st));
    }
    HIPCHK(launch_reduce_partials(L.part, sp.nsplit, (int)n, w, ldp, Y, nullptr, nullptr, st));
    return SYMNMF_OK;
}

int symnmf_sh_sym(const float* S, int64_t n, int64_t lds, const float* H, int32_t k, float* P,
                  double* tr_host, void* ws, size_t ws_bytes, void* hip_stream) {
    if (!S || !H || !P || n < 1 || n > INT32_MAX / 2 || k < 1 || k > kSymMaxK || lds < n ||
        lds % 4 || !aligned(S, 16) || !aligned(H, 4) || !aligned(P, 4))
        return SYMNMF_E_INVALID;
    const size_t need = sym_layout(nullptr, n, k, nullptr);
    if (!ws_ok(ws, ws_bytes, need)) return SYMNMF_E_WORKSPACE;
    SymLayout L;
    sym_layout(ws, n, k, &L);
    hipStream_t st = as_stream(hip_stream);
    const SymPlan sp = sym_plan((int)n, k);
    HIPCHK(launch_sym_pack(H, (int)n, k, sp, L.hsr, L.hsc, nullptr, st));
    {
        ProfScope ps(SYMNMF_PROF_SH_SYM, 2.0 * n * (double)(n + 1) + 8.0 * n * k, st);
        HIPCHK(launch_sym(S, lds, L.hsr, L.hsc, (int)n, k, sp, L.p1, L.p2, nullptr, st));
    }
    HIPCHK(launch_sym_fold(L.p1, L.p2, (int)n, k, sp, P, k, H, L.tr_part, nullptr, st));
    if (tr_host) {
        HIPCHK(launch_sum_doubles(L.tr_part, cdiv(n, kUpdRows), L.tr_out, st));
        HIPCHK(hipMemcpyAsync(tr_host, L.tr_out, sizeof(double), hipMemcpyDeviceToHost, st));
        HIPCHK(hipStreamSynchronize(st));
    }
    return SYMNMF_OK;
}

// ---------------------------------------------------------------------------
int symnmf_build_S(int kind, const float* X, int64_t T, int64_t n, int64_t ldx, float tail_frac,
                   float* S, int64_t lds, double* S_fro2_host, void* ws, size_t ws_bytes,
                   void* hip_stream) {
    if ((kind != SYMNMF_ABSCORR && kind != SYMNMF_TPDM) || !X || !S || T < 2 || T > 65536 ||
        n < 1 || n > INT32_MAX / 2 || ldx < n || lds < n || lds % 4 || !aligned(S, 16))
        return SYMNMF_E_INVALID;
    if (kind == SYMNMF_TPDM && !(tail_frac > 0.f && tail_frac <= 1.f)) return SYMNMF_E_INVALID;
    const size_t need = build_layout(nullptr, kind, T, n, nullptr);
    if (!ws_ok(ws, ws_bytes, need)) return SYMNMF_E_WORKSPACE;
    BuildLayout L;
    build_layout(ws, kind, T, n, &L);
    hipStream_t st = as_stream(hip_stream);
    const int64_t ldz = round_up(n, kGramTile);
    HIPCHK(launch_fill(reinterpret_cast<float*>(L.flags), 2, 0.f, st));
    int Kp = 0;
    float scale = 1.f;
    int absval = 1;
    bool split = false;
    if (kind == SYMNMF_ABSCORR) {
        // the T-deep contraction runs on the bf16 matrix cores (exact split
        // operands); the TPDM's few extreme days (m = ceil(tail_frac T)) stay
        // on the fp32 path, where padding m to 32 days would cost more
        Kp = (int)round_up(T, 32);
        split = true;
        HIPCHK(launch_standardize(X, (int)T, (int)n, ldx, L.Z, Kp, ldz, L.flags, st));
    } else {
        // m = ceil(tail_frac T) extreme days
        int m = (int)std::ceil((double)tail_frac * (double)T - 1e-4);
        m = std::max(1, std::min((int)T, m));
        Kp = (int)round_up(m, 4);
        HIPCHK(launch_fill(reinterpret_cast<float*>(L.hist), T * (T + 1), 0.f, st));
        HIPCHK(launch_fill(reinterpret_cast<float*>(L.sel), T, 0.f, st));
        HIPCHK(launch_tpdm_ranks(X, (int)T, (int)n, ldx, L.R, L.hist, L.flags, st));
        int fl[2] = {0, 0};
        HIPCHK(hipMemcpyAsync(fl, L.flags, sizeof(fl), hipMemcpyDeviceToHost, st));
        HIPCHK(hipStreamSynchronize(st));
        if (fl[0]) return SYMNMF_E_NONFINITE;
        HIPCHK(launch_tpdm_select(L.hist, (int)T, m, L.radius, L.sel, st));
        HIPCHK(launch_tpdm_theta(L.R, (int)T, (int)n, L.sel, L.radius, m, Kp, L.Z, ldz, st));
        scale = (float)(1.0 / (double)m);
        absval = 0;
    }
    int flags[2] = {0, 0};
    HIPCHK(hipMemcpyAsync(flags, L.flags, sizeof(flags), hipMemcpyDeviceToHost, st));
    HIPCHK(hipStreamSynchronize(st));
    if (flags[0]) return SYMNMF_E_NONFINITE;
    if (flags[1]) return SYMNMF_E_DEGENERATE;
    int64_t ntiles = 0;
    {
        // algorithmic traffic: S written once (4 n^2 bytes) plus the panels read
        ProfScope ps(SYMNMF_PROF_BUILD_GRAM, 4.0 * n * (double)n + 4.0 * Kp * (double)n, st);
        HIPCHK(launch_gram_build(L.Z, Kp, ldz, (int)n, scale, absval, split, S, lds, L.part2,
                                 &ntiles, st));
    }
    if (S_fro2_host) {
        HIPCHK(launch_sum_doubles(L.part2, ntiles, L.fro, st));
        HIPCHK(hipMemcpyAsync(S_fro2_host, L.fro, sizeof(double), hipMemcpyDeviceToHost, st));
        HIPCHK(hipStreamSynchronize(st));
    }
    return SYMNMF_OK;
}

// ---------------------------------------------------------------------------
namespace {

// Q <- orthonormal basis of span(Y) (n x w) by two rounds of Cholesky QR; a
// round whose Gram is numerically singular (rank-deficient S, e.g. a TPDM of
// rank m < w) falls back to Q = Y V diag(1/sqrt(max(mu, tau))) from the Gram
// eigenpairs, which keeps the well-determined directions orthonormal and
// leaves the null directions near zero. On return `Q` holds the basis (the two
// buffers may be swapped).
// Host staging of the orthonormalisation's R^-1. Its uploads are
// asynchronous, so it lives as long as the probe call (each round rewrites it
// only after a stream synchronisation) and the stream is drained before it
// goes away, on every return path.
struct ProbeHostStaging {
    std::vector<float> M;
    hipStream_t st;
    ProbeHostStaging(int w, hipStream_t s) : M((size_t)w * w), st(s) {}
    ~ProbeHostStaging() { (void)hipStreamSynchronize(st); }
};

int orthonormalize(float*& Y, float*& Q, int n, int w, ProbeLayout& L, std::vector<float>& M,
                   hipStream_t st) {
    const int nblk = crossgram_blocks(n);
    std::vector<double> G((size_t)w * w), Lf, Ri, V, ev;
    for (int round = 0; round < 2; ++round) {
        HIPCHK(launch_crossgram(Y, Y, n, w, L.cg_part, nblk, L.C, st));
        HIPCHK(hipMemcpyAsync(G.data(), L.C, sizeof(double) * w * w, hipMemcpyDeviceToHost, st));
        HIPCHK(hipStreamSynchronize(st));
        for (double v : G)
            if (!std::isfinite(v)) return SYMNMF_E_NONFINITE;
        for (int i = 0; i < w; ++i)
            for (int j = i + 1; j < w; ++j) {
                const double s = 0.5 * (G[(size_t)i * w + j] + G[(size_t)j * w + i]);
                G[(size_t)i * w + j] = G[(size_t)j * w + i] = s;
            }
        if (cholesky_lower(w, G, Lf, 1e-10)) {
            lower_inverse_transposed(w, Lf, Ri);
            for (size_t e = 0; e < M.size(); ++e) M[e] = (float)Ri[e];
        } else {
            std::vector<double> A = G;
            jacobi_eig(w, A, ev, &V);
            double mx = 0.0;
            for (double v : ev) mx = std::max(mx, v);
            const double tau = std::max(1e-300, 1e-12 * mx);
            for (int r = 0; r < w; ++r)
                for (int c = 0; c < w; ++c)
                    M[(size_t)r * w + c] = (float)(V[(size_t)r * w + c] / std::sqrt(std::max(ev[c], tau)));
        }
        HIPCHK(hipMemcpyAsync(L.M, M.data(), sizeof(float) * w * w, hipMemcpyHostToDevice, st));
        HIPCHK(launch_rowmat(Y, L.M, n, w, Q, st));
        std::swap(Y, Q);
    }
    std::swap(Y, Q);
    return SYMNMF_OK;
}

}  // namespace

int symnmf_spectral_probe(const float* S, int64_t n, int64_t lds, int32_t p, int32_t max_iters,
                          double tol, uint64_t seed, double* eigvals_host, int32_t* iters_host,
                          void* ws, size_t ws_bytes, void* hip_stream) {
    if (!S || !eigvals_host || n < 1 || n > INT32_MAX / 2 || lds < n || lds % 4 ||
        !aligned(S, 16) || p < 1 || max_iters < 1 || !(tol >= 0.0))
        return SYMNMF_E_INVALID;
    const int w = probe_width(p, n);
    if (w > kMaxWidth || w > n) return SYMNMF_E_INVALID;
    const size_t need = probe_layout(nullptr, n, p, nullptr);
    if (!ws_ok(ws, ws_bytes, need)) return SYMNMF_E_WORKSPACE;
    ProbeLayout L;
    probe_layout(ws, n, p, &L);
    hipStream_t st = as_stream(hip_stream);
    const int nn = (int)n;
    const SqPlan sp = sq_plan(nn, w);
    const int ldp = ldp_of(w);
    const int nblk = crossgram_blocks(nn);

    float* Q = L.Q;
    float* Y = L.Y;
    HIPCHK(launch_init_uniform(Y, (int64_t)n * w, 2.0, -1.0, seed, st));
    ProbeHostStaging staging(w, st);
    int rc = orthonormalize(Y, Q, nn, w, L, staging.M, st);
    if (rc != SYMNMF_OK) return rc;

    // One step: Y = S Q and the Rayleigh quotient Q^T Y into L.C, enqueued.
    auto stage = [&]() -> int {
        HIPCHK(launch_sq_pack(Q, w, nn, w, sp, L.qs, st));
        {
            ProfScope ps(SYMNMF_PROF_SH_PROBE, 4.0 * n * (double)n + 8.0 * n * w, st);
            HIPCHK(launch_sq_split(S, lds, L.qs, nn, w, sp, L.part, ldp, st));
        }
        HIPCHK(launch_reduce_partials(L.part, sp.nsplit, nn, w, ldp, Y, nullptr, nullptr, st));
        HIPCHK(launch_crossgram(Q, Y, nn, w, L.cg_part, nblk, L.C, st));
        return SYMNMF_OK;
    };
    // The host eigen-solve of step `it` (which only decides whether to stop)
    // runs while the device already computes step it+1 from the next Q; if
    // step `it` converged, that extra step is discarded. The values and the
    // step count are those of the plain loop.
    std::vector<double> T((size_t)w * w), ev, prev, theta;
    int it = 0;
    bool converged = false;
    if ((rc = stage())) return rc;
    for (it = 1; it <= max_iters; ++it) {
        HIPCHK(hipMemcpyAsync(T.data(), L.C, sizeof(double) * w * w, hipMemcpyDeviceToHost, st));
        HIPCHK(hipStreamSynchronize(st));
        for (int i = 0; i < w; ++i)
            for (int j = i + 1; j < w; ++j) {
                const double s = 0.5 * (T[(size_t)i * w + j] + T[(size_t)j * w + i]);
                T[(size_t)i * w + j] = T[(size_t)j * w + i] = s;
            }
        for (double v : T)
            if (!std::isfinite(v)) return SYMNMF_E_NONFINITE;
        if (it < max_iters) {
            rc = orthonormalize(Y, Q, nn, w, L, staging.M, st);
            if (rc != SYMNMF_OK) return rc;
            if ((rc = stage())) return rc;
        }
        std::vector<double> A = T;
        sym_eigvals(w, A, ev);
        std::vector<int> order(w);
        for (int i = 0; i < w; ++i) order[i] = i;
        std::stable_sort(order.begin(), order.end(),
                         [&](int a, int b) { return std::fabs(ev[a]) > std::fabs(ev[b]); });
        theta.assign(p, 0.0);
        for (int i = 0; i < p; ++i) theta[i] = ev[order[i]];
        if (!prev.empty()) {
            double mx = 0.0;
            for (int i = 0; i < p; ++i) mx = std::max(mx, std::fabs(theta[i] - prev[i]));
            if (mx <= tol * std::fabs(theta[0])) {
                converged = true;
                break;
            }
        }
        prev = theta;
        if (it == max_iters) break;
    }
    HIPCHK(hipStreamSynchronize(st));  // a discarded step may still be running
    for (int i = 0; i < p; ++i) eigvals_host[i] = theta[i];
    if (iters_host) *iters_host = std::min(it, (int)max_iters);
    return converged ? SYMNMF_OK : SYMNMF_W_NOT_CONVERGED;
}

// ---------------------------------------------------------------------------
namespace {

// gamma_{k+1} = lambda_{k+1} / |lambda_{k+2}| (1-based, descending |lambda|),
// denominator floored at 1e-6 |lambda_1| (P1 "Why this solver").
double gap_ratio(const double* ev, int k) {
    const double lam1 = std::fabs(ev[0]);
    double den = std::fabs(ev[k + 1]);
    if (den <= 1e-6 * lam1) den = 1e-6 * lam1;
    return ev[k] / den;
}

// |B|0 from gamma: 2^floor(log2(max(1, gamma/threshold nb))), capped at nb.
int initial_blocks(double gamma, int nb, double threshold) {
    if (gamma >= threshold) return nb;
    const double x = std::max(1.0, gamma / threshold * (double)nb);
    int e = (int)std::floor(std::log2(x));
    int64_t v = (int64_t)1 << std::min(e, 30);
    return (int)std::min<int64_t>(nb, v);
}

// Fisher-Yates over [0, nb) keyed by (seed, t); the first nsel slots, sorted.
void sample_blocks(uint64_t seed, int t, int nb, int nsel, std::vector<int>& perm, int* out) {
    perm.resize(nb);
    for (int i = 0; i < nb; ++i) perm[i] = i;
    const uint64_t key = seed ^ kSamplerKeyXor;
    for (int j = 0; j < nsel; ++j) {
        const uint64_t r = splitmix64(key, ((uint64_t)(uint32_t)t << 32) + (uint64_t)j);
        const int pick = j + (int)(r % (uint64_t)(nb - j));
        std::swap(perm[j], perm[pick]);
    }
    std::sort(perm.begin(), perm.begin() + nsel);
    for (int j = 0; j < nsel; ++j) out[j] = perm[j];
}

}  // namespace

int symnmf_fit(const float* S, int64_t n, int64_t lds, int32_t k, const symnmf_fit_params* prm,
               const double* eigvals_host, int32_t n_eig, float* H, float* G,
               double* obj_trace_host, int32_t obj_trace_cap, symnmf_fit_report* rep_host,
               symnmf_fit_state* state, void* ws, size_t ws_bytes, void* hip_stream) {
    const auto t_start = std::chrono::steady_clock::now();
    symnmf_fit_params P;
    if (prm) P = *prm; else symnmf_fit_params_default(&P);
    if (!S || !H || n < 1 || n > INT32_MAX / 2 || k < 1 || k > kMaxK || k > n || lds < n ||
        lds % 4 || !aligned(S, 16) || !aligned(H, 4))
        return SYMNMF_E_INVALID;
    if (P.solver < 0 || P.solver > 2 || P.max_iters < 0 || !(P.eps > 0.0) || P.block_rows < 4 ||
        !(P.rms_decay >= 0.0 && P.rms_decay < 1.0) || P.sh_pass < 0 || P.sh_pass > 1 ||
        (P.sh_pass == SYMNMF_SH_UPPER && k > kSymMaxK) ||
        !(P.tol_rel >= 0.0) || !(P.stall_tol >= 0.0) || P.init < 0 || P.init > 2 ||
        !(P.obj_floor >= 0.0) || !std::isfinite(P.obj_floor) || P.start_iter < 0 ||
        (int64_t)P.start_iter + P.max_iters > INT32_MAX ||
        !(P.gap_threshold > 0.0) || (P.resume && !G) || (obj_trace_cap > 0 && !obj_trace_host) ||
        obj_trace_cap < 0 || !std::isfinite(P.lr) || !std::isfinite(P.phi0))
        return SYMNMF_E_INVALID;
    if (P.init == SYMNMF_INIT_UNIFORM && !(P.init_scale > 0.0)) return SYMNMF_E_INVALID;
    const int nb = (int)cdiv(n, P.block_rows);
    const bool restore = P.resume && state;
    if (state) {
        if (!state->H_anchor || !state->P_anchor || !aligned(state->H_anchor, 4) ||
            !aligned(state->P_anchor, 4))
            return SYMNMF_E_INVALID;
        if (restore && (state->iter != P.start_iter || state->blocks < 1 || state->blocks > nb ||
                        state->anchor_iter > state->iter || state->anchor_iter < -1 ||
                        (state->anchor_iter >= 0 && !std::isfinite(state->f_anchor)) ||
                        (state->f_prev_valid && !std::isfinite(state->f_prev))))
            return SYMNMF_E_INVALID;
    }
    const bool need_eig = !restore && P.solver != SYMNMF_FULL && !(P.phi0 > 0.0) && nb > 1;
    if (need_eig && (!eigvals_host || n_eig < k + 2)) return SYMNMF_E_INVALID;
    const size_t need = fit_layout(nullptr, n, k, P.max_iters, P.block_rows, P.sh_pass, nullptr);
    if (!ws_ok(ws, ws_bytes, need)) return SYMNMF_E_WORKSPACE;
    FitLayout L;
    fit_layout(ws, n, k, P.max_iters, P.block_rows, P.sh_pass, &L);
    hipStream_t st = as_stream(hip_stream);
    const int nn = (int)n;
    const int64_t nk = (int64_t)n * k;
    const int ldp = ldp_of(k);
    const int nblk = (int)cdiv(n, kUpdRows);
    const int* done_dev = &L.fd->done;  // device address of the stop flag
    const int64_t call_tag = (g_fit_calls.fetch_add(1) + 1) << 32;

    // ---- ||S||^2 and mean(S) (one pass over S)
    HIPCHK(launch_s_stats(S, lds, nn, L.stats_part, st));
    HIPCHK(launch_s_stats_final(L.stats_part, (int)cdiv(n, kStatsRows), L.stats_out, st));
    double stats[2];
    HIPCHK(hipMemcpyAsync(stats, L.stats_out, sizeof(stats), hipMemcpyDeviceToHost, st));
    HIPCHK(hipStreamSynchronize(st));
    const double S_sum = stats[0], S_fro2 = stats[1];
    if (!std::isfinite(S_sum) || !std::isfinite(S_fro2)) return SYMNMF_E_NONFINITE;
    const double S_mean = S_sum / ((double)n * (double)n);
    const double floor_abs = P.obj_floor * S_fro2;

    // ---- readings for the undefined scale-matched init and default lr
    const double a_sm = 2.0 * std::sqrt(std::max(0.0, S_mean) / k);
    const double lr = P.lr > 0.0 ? P.lr : std::sqrt(std::max(0.0, S_mean) / k);
    double init_scale = std::nan("");
    if (P.init == SYMNMF_INIT_CALLER) {
        HIPCHK(launch_copy(L.Hb[0], H, nk, st));
    } else {
        init_scale = P.init == SYMNMF_INIT_UNIFORM ? P.init_scale : a_sm;
        HIPCHK(launch_init_uniform(L.Hb[0], nk, init_scale, 0.0, P.seed, st));
    }
    if (P.resume) HIPCHK(launch_copy(L.Gb[0], G, nk, st));
    else HIPCHK(launch_fill(L.Gb[0], nk, 0.f, st));

    // ---- controller state: fresh, or restored from the caller's state
    int ab = 0;                // anchor buffer of the current anchor
    int anchor_abs = -1;       // absolute step of the current anchor
    double f_anchor = std::nan("");
    if (restore && state->anchor_iter >= 0) {
        anchor_abs = state->anchor_iter;
        f_anchor = state->f_anchor;
        HIPCHK(launch_copy(L.Ha[0], state->H_anchor, nk, st));
        HIPCHK(launch_copy(L.Pa[0], state->P_anchor, nk, st));
    }

    // ---- device state
    {
        FitDev h;
        std::memset(&h, 0, sizeof(h));
        h.S_fro2 = S_fro2;
        h.tol = P.tol_rel;
        h.floor_abs = floor_abs;
        if (restore && state->f_prev_valid) {
            h.f_prev = state->f_prev;
            h.f_prev_valid = 1;
        }
        HIPCHK(hipMemcpyAsync(L.fd, &h, sizeof(FitDev), hipMemcpyHostToDevice, st));
        HIPCHK(hipStreamSynchronize(st));
    }
    // K_0 = H_0^T H_0
    {
        UpdateArgs a{};
        a.n = nn; a.k = k; a.ldp = ldp; a.H = L.Hb[0]; a.fd = L.fd; a.gram_part = L.gram_part;
        a.gram_only = 1;
        HIPCHK(launch_update(a, st));
        HIPCHK(launch_finalize(L.fd, nullptr, 0, nblk, k, nullptr, L.gram_part, 4 | 8, st));
    }

    // ---- branch choice (P1 "Why this solver"; P2 sketch)
    double gamma = std::nan("");
    int nsel = nb;
    if (restore) {
        nsel = state->blocks;
    } else if (P.solver == SYMNMF_FULL || nb <= 1) {
        nsel = nb;
    } else if (P.phi0 > 0.0) {
        nsel = (int)std::min<int64_t>(nb, std::max<int64_t>(1, (int64_t)std::ceil(P.phi0 * nb - 1e-12)));
    } else {
        gamma = gap_ratio(eigvals_host, k);
        nsel = initial_blocks(gamma, nb, P.gap_threshold);
    }
    bool full = nsel >= nb;
    const int start_branch = full ? 0 : 1;

    FullPlan fpl = full_plan(nn);
    fpl.rp.done = done_dev;
    const double sh_bytes = 4.0 * n * (double)n + 8.0 * (double)nk;
    const double sym_bytes = 2.0 * n * (double)(n + 1) + 8.0 * (double)nk;
    const int T0 = P.start_iter;
    int cur = 0, t = 0, doublings = 0, anchors = 0, last_exact = -1;
    FitDev hd;
    std::vector<int> perm, lists;

    const bool upper = P.sh_pass == SYMNMF_SH_UPPER;
    const SymPlan symp = sym_plan(nn, k);
    // one exact step at local index t (P_t = S H_t); with anchor >= 0 it also
    // writes H~ = H_t, P~ = P_t into anchor buffer `anchor`
    auto exact_step = [&](int anchor, int flags) -> int {
        const int64_t tag = call_tag | t;
        if (upper) {
            // P_t = S H_t from the upper triangle, folded into the first
            // partial slot (the update then reads one partial)
            HIPCHK(launch_sym_pack(L.Hb[cur], nn, k, symp, L.sym_hsr, L.sym_hsc, done_dev, st));
            {
                ProfScope ps(SYMNMF_PROF_SH_SYM, sym_bytes, st, tag);
                HIPCHK(launch_sym(S, lds, L.sym_hsr, L.sym_hsc, nn, k, symp, L.sym_p1, L.sym_p2,
                                  done_dev, st));
            }
            HIPCHK(launch_sym_fold(L.sym_p1, L.sym_p2, nn, k, symp, L.part, ldp, nullptr, nullptr,
                                   done_dev, st));
        } else {
            ProfScope ps(SYMNMF_PROF_SH_FULL, sh_bytes, st, tag);
            HIPCHK(launch_sh_panel(S, lds, L.Hb[cur], k, fpl.rp, fpl.nsplit, L.part, ldp, st));
        }
        const int nsplit = upper ? 1 : fpl.nsplit;
        UpdateArgs a{};
        a.n = nn; a.k = k; a.ldp = ldp; a.part = L.part; a.nsplit = nsplit;
        a.pstride = (int64_t)n * ldp; a.H = L.Hb[cur]; a.G = L.Gb[cur];
        a.Hn = L.Hb[cur ^ 1]; a.Gn = L.Gb[cur ^ 1];
        a.Ha = anchor >= 0 ? L.Ha[anchor] : nullptr; a.Pa = anchor >= 0 ? L.Pa[anchor] : nullptr;
        a.fd = L.fd; a.lr = (float)lr; a.eps = (float)P.eps; a.decay = (float)P.rms_decay;
        a.tr_part = L.tr_part; a.gram_part = L.gram_part;
        {
            ProfScope ps(SYMNMF_PROF_UPDATE, (double)nk * 4.0 * (5 + nsplit), st, tag);
            HIPCHK(launch_update(a, st));
        }
        HIPCHK(launch_finalize(L.fd, L.f_trace, t, nblk, k, L.tr_part, L.gram_part, flags, st));
        cur ^= 1;
        ++t;
        return SYMNMF_OK;
    };
    auto sampled_step = [&](const int* blocks_dev) -> int {
        FullPlan sp = sampled_plan(nn, blocks_dev, nsel, P.block_rows);
        sp.rp.done = done_dev;
        {
            const double rows = std::min<double>((double)nsel * P.block_rows, (double)n);
            ProfScope ps(SYMNMF_PROF_SH_SAMPLED, 4.0 * rows * (double)n + 8.0 * (double)nk, st);
            // D = H - H~ on the sampled rows, then the correction sum over them
            HIPCHK(launch_block_diff(L.Hb[cur], L.Ha[ab], blocks_dev, nsel, P.block_rows, nn, k,
                                     L.D, done_dev, st));
            HIPCHK(launch_sh_panel(S, lds, L.D, k, sp.rp, sp.nsplit, L.part, ldp, st));
        }
        UpdateArgs a{};
        a.n = nn; a.k = k; a.ldp = ldp; a.part = L.part; a.nsplit = sp.nsplit;
        a.pstride = (int64_t)n * ldp; a.Pt = L.Pa[ab]; a.pscale = (float)((double)nb / nsel);
        a.H = L.Hb[cur]; a.G = L.Gb[cur]; a.Hn = L.Hb[cur ^ 1]; a.Gn = L.Gb[cur ^ 1];
        a.fd = L.fd; a.lr = (float)lr; a.eps = (float)P.eps; a.decay = (float)P.rms_decay;
        a.gram_part = L.gram_part;
        {
            ProfScope ps(SYMNMF_PROF_UPDATE, (double)nk * 4.0 * (6 + sp.nsplit), st);
            HIPCHK(launch_update(a, st));
        }
        HIPCHK(launch_finalize(L.fd, L.f_trace, t, nblk, k, nullptr, L.gram_part, 4, st));
        cur ^= 1;
        ++t;
        return SYMNMF_OK;
    };
    auto read_state = [&]() -> int {
        HIPCHK(hipMemcpyAsync(&hd, L.fd, offsetof(FitDev, Kd), hipMemcpyDeviceToHost, st));
        HIPCHK(hipStreamSynchronize(st));
        return SYMNMF_OK;
    };

    int rc = SYMNMF_OK;
    bool stopped = false;         // device stop flag seen (full branch)
    bool anchor_stop = false;     // the anchor stop test fired (sampled branch)
    // ---- Block-SVRG branch (P1 "Factorizing with SymNMF": SVRG-corrected
    // block-sampled gradient, sample grown toward the full gradient when
    // progress stalls)
    while (!full && t < P.max_iters) {
        const int E = (int)cdiv(nb, nsel);
        const int tabs = T0 + t;
        if (anchor_abs < 0 || tabs - anchor_abs >= E) {
            rc = exact_step(ab ^ 1, 1 | 4);
            if (rc) return rc;
            if ((rc = read_state())) return rc;
            if (hd.status == -4) return SYMNMF_E_NONFINITE;
            const double f = hd.f_prev;
            if (anchor_abs >= 0) {
                const int Ej = tabs - anchor_abs;
                if (P.tol_rel > 0.0 &&
                    std::fabs(f_anchor - f) < P.tol_rel * Ej * std::max(std::fabs(f_anchor), floor_abs)) {
                    // converged: return H_t (the anchor's update went to the
                    // other buffer and is dropped; the current anchor stays)
                    anchor_stop = true;
                    cur ^= 1;
                    --t;
                    last_exact = t;
                    break;
                }
                if ((f_anchor - f) < P.stall_tol * f_anchor) {
                    nsel = std::min(2 * nsel, nb);
                    ++doublings;
                    if (nsel >= nb) full = true;
                }
            }
            ab ^= 1;
            anchor_abs = tabs;
            f_anchor = f;
            ++anchors;
            last_exact = t - 1;
            continue;
        }
        const int steps = std::min(anchor_abs + E - tabs, P.max_iters - t);
        lists.assign((size_t)steps * nsel, 0);
        for (int s2 = 0; s2 < steps; ++s2)
            sample_blocks(P.seed, tabs + s2, nb, nsel, perm, &lists[(size_t)s2 * nsel]);
        HIPCHK(hipMemcpyAsync(L.blocks, lists.data(), sizeof(int) * lists.size(), hipMemcpyHostToDevice, st));
        HIPCHK(hipStreamSynchronize(st));
        for (int s2 = 0; s2 < steps; ++s2) {
            rc = sampled_step(L.blocks + (size_t)s2 * nsel);
            if (rc) return rc;
        }
    }
    // ---- full-batch branch (P2 sketch: g = 4 (H (H^T H) - S H))
    if (full && !anchor_stop) {
        const int t0 = t, cur0 = cur;
        const int every = std::max(1, P.check_every);
        while (t < P.max_iters) {
            const int batch = std::min(every, P.max_iters - t);
            for (int b = 0; b < batch; ++b) {
                rc = exact_step(-1, 1 | 2 | 4);
                if (rc) return rc;
            }
            if ((rc = read_state())) return rc;
            if (hd.done) {
                stopped = true;
                break;
            }
        }
        if (stopped) {
            if (hd.status == -4) return SYMNMF_E_NONFINITE;
            // launches after the stop step returned at once: not timings
            prof_discard(call_tag | (hd.stop_iter + 1), call_tag | 0xFFFFFFFFll);
            t = hd.stop_iter;
            cur = (cur0 + (t - t0)) & 1;
            last_exact = t;
        } else if (t > t0) {
            last_exact = t - 1;
        }
    } else if (!anchor_stop) {
        if ((rc = read_state())) return rc;
    }
    const bool converged = (stopped && hd.status == 1) || anchor_stop;
    const int iters = t;

    // ---- outputs
    HIPCHK(launch_copy(H, L.Hb[cur], nk, st));
    if (G) HIPCHK(launch_copy(G, L.Gb[cur], nk, st));
    HIPCHK(launch_fill(reinterpret_cast<float*>(L.zero_rows), 1, 0.f, st));
    HIPCHK(launch_count_zero_rows(L.Hb[cur], nn, k, L.zero_rows, st));
    int zero_rows = 0;
    HIPCHK(hipMemcpyAsync(&zero_rows, L.zero_rows, sizeof(int), hipMemcpyDeviceToHost, st));
    const int evaluated = converged ? iters + 1 : iters;
    const int ncopy = std::min(obj_trace_cap, evaluated);
    if (ncopy > 0)
        HIPCHK(hipMemcpyAsync(obj_trace_host, L.f_trace, sizeof(double) * ncopy, hipMemcpyDeviceToHost, st));
    double f_last = std::nan("");
    if (last_exact >= 0)
        HIPCHK(hipMemcpyAsync(&f_last, L.f_trace + last_exact, sizeof(double), hipMemcpyDeviceToHost, st));
    // the objective of the step before the returned H (NaN after a sampled
    // step), for the state
    double f_before = std::nan("");
    if (iters >= 1)
        HIPCHK(hipMemcpyAsync(&f_before, L.f_trace + iters - 1, sizeof(double), hipMemcpyDeviceToHost, st));
    if (state && anchor_abs >= 0) {
        HIPCHK(launch_copy(state->H_anchor, L.Ha[ab], nk, st));
        HIPCHK(launch_copy(state->P_anchor, L.Pa[ab], nk, st));
    }
    HIPCHK(hipStreamSynchronize(st));

    if (state) {
        state->iter = T0 + iters;
        state->blocks = nsel;
        state->anchor_iter = anchor_abs;
        state->f_anchor = anchor_abs >= 0 ? f_anchor : std::nan("");
        if (iters >= 1) {
            state->f_prev_valid = std::isfinite(f_before) ? 1 : 0;
            state->f_prev = f_before;
        } else if (!restore) {
            state->f_prev_valid = 0;
            state->f_prev = std::nan("");
        }  // no step taken after a restore: the entry values stand
    }
    if (rep_host) {
        symnmf_fit_report& r = *rep_host;
        std::memset(&r, 0, sizeof(r));
        r.iterations = iters;
        r.converged = converged ? 1 : 0;
        r.start_branch = start_branch;
        r.final_branch = full ? 0 : 1;
        r.blocks_final = nsel;
        r.n_blocks = nb;
        r.doublings = doublings;
        r.zero_rows = zero_rows;
        r.f_last_iter = last_exact;
        r.anchors = anchors;
        r.gamma = gamma;
        r.lr_used = lr;
        r.init_scale_used = init_scale;
        r.f_last = f_last;
        r.S_fro2 = S_fro2;
        r.S_mean = S_mean;
        r.seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t_start).count();
    }
    if (converged || P.tol_rel == 0.0) return SYMNMF_OK;
    return SYMNMF_W_NOT_CONVERGED;
}

// ---------------------------------------------------------------------------
// Spherical k-means (P1 "Spherical k-means for direct hard clustering").
int symnmf_spherical_kmeans(const float* S, int64_t n, int64_t lds, int32_t k,
                            int32_t max_iters, uint64_t seed, int32_t* labels,
                            float* centroids, int32_t* iters_host, int32_t* converged_host,
                            double* objective_host, void* ws, size_t ws_bytes,
                            void* hip_stream) {
    if (!S || !labels || n < 1 || n > INT32_MAX / 2 || k < 1 || k > kMaxK || k > n ||
        max_iters < 0 || lds < n || lds % 4 || !aligned(S, 16) || !aligned(labels, 4) ||
        (centroids && !aligned(centroids, 4)))
        return SYMNMF_E_INVALID;
    const size_t need = kmeans_layout(nullptr, n, k, nullptr);
    if (!ws_ok(ws, ws_bytes, need)) return SYMNMF_E_WORKSPACE;
    KmeansLayout L;
    kmeans_layout(ws, n, k, &L);
    hipStream_t st = as_stream(hip_stream);
    const int nn = (int)n;
    const FullPlan fp = full_plan(nn);
    const int ldp = ldp_of(k);
    const double pass_bytes = 4.0 * n * (double)n + 8.0 * (double)n * k;
    const int64_t nblk = cdiv(n, 256);

    // x_i = S[i,:] / ||S[i,:]||; the seeded initial rows become the centroids
    HIPCHK(launch_row_norm_inv(S, lds, nn, L.rinv, st));
    {
        std::vector<int> perm, idx(k);
        sample_blocks(seed, 0, nn, k, perm, idx.data());
        HIPCHK(hipMemcpyAsync(L.idx, idx.data(), sizeof(int) * k, hipMemcpyHostToDevice, st));
        HIPCHK(launch_gather_centroids(S, lds, nn, L.idx, L.rinv, k, L.Ct, st));
        HIPCHK(hipStreamSynchronize(st));  // idx lives on the host stack
    }
    // labels before the first assignment: k, which no assignment produces
    HIPCHK(launch_fill_int(L.lab[0], n, k, st));
    int cur = 0;  // lab[cur]: labels of the last assignment
    int updates = 0, changes = 0;
    bool converged = false;
    double obj = 0.0;
    for (;;) {
        // assignment: the row argmax of S C^T
        {
            ProfScope ps(SYMNMF_PROF_SH_KMEANS, pass_bytes, st);
            HIPCHK(launch_sh_panel(S, lds, L.Ct, k, fp.rp, fp.nsplit, L.part, ldp, st));
        }
        HIPCHK(launch_reduce_partials(L.part, fp.nsplit, nn, k, ldp, L.C, nullptr, nullptr, st));
        int32_t* lab_new = L.lab[cur ^ 1];
        HIPCHK(launch_labels(L.C, n, k, lab_new, st));
        HIPCHK(launch_fill_int(L.changes, 1, 0, st));
        HIPCHK(launch_kmeans_assign_stats(L.C, nn, k, lab_new, L.lab[cur], L.rinv, L.changes,
                                          L.obj_part, st));
        HIPCHK(launch_sum_doubles(L.obj_part, nblk, L.obj, st));
        HIPCHK(hipMemcpyAsync(&changes, L.changes, sizeof(int), hipMemcpyDeviceToHost, st));
        HIPCHK(hipMemcpyAsync(&obj, L.obj, sizeof(double), hipMemcpyDeviceToHost, st));
        HIPCHK(hipStreamSynchronize(st));
        cur ^= 1;
        if (!std::isfinite(obj)) return SYMNMF_E_NONFINITE;
        if (changes == 0) {
            converged = true;
            break;
        }
        if (updates >= max_iters) break;
        // update: C^T = normalise(S D^-1 Z), empty clusters keep their centroid
        HIPCHK(launch_onehot_scaled(L.lab[cur], L.rinv, nn, k, L.W, st));
        {
            ProfScope ps(SYMNMF_PROF_SH_KMEANS, pass_bytes, st);
            HIPCHK(launch_sh_panel(S, lds, L.W, k, fp.rp, fp.nsplit, L.part, ldp, st));
        }
        HIPCHK(launch_reduce_partials(L.part, fp.nsplit, nn, k, ldp, L.C, nullptr, nullptr, st));
        HIPCHK(launch_normalize_columns(L.C, nn, k, L.col_part, L.norm, L.Ct, st));
        ++updates;
    }
    HIPCHK(hipMemcpyAsync(labels, L.lab[cur], sizeof(int32_t) * n, hipMemcpyDeviceToDevice, st));
    if (centroids)
        HIPCHK(hipMemcpyAsync(centroids, L.Ct, sizeof(float) * n * k, hipMemcpyDeviceToDevice, st));
    HIPCHK(hipStreamSynchronize(st));
    if (iters_host) *iters_host = updates;
    if (converged_host) *converged_host = converged ? 1 : 0;
    if (objective_host) *objective_host = obj;
    return converged ? SYMNMF_OK : SYMNMF_W_NOT_CONVERGED;
}

}  // extern "C"
