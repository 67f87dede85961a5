// symnmf_sh_noalloc: the S.H pass of symnmf_sh for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation). Its scratch (the per-split partial
// products and the trace partials) lives in one file-scope device array of
// kScratchBytes, resolved once per device with hipGetSymbolAddress; the call
// then launches the same kernels as symnmf_sh on that memory, so its results
// are bit for bit those of symnmf_sh.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "symnmf.h"

namespace symnmf {
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

// The scratch. Host code never passes this name to a kernel (on the host it is
// a stand-in, not a device address): it uses the address resolved below.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

inline size_t up256(size_t x) { return (x + 255) / 256 * 256; }

// Device address of `scratch` on the current device (resolved on the first
// call there); nullptr on a HIP error.
void* scratch_address(hipError_t* err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_addr[dev]) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_addr[dev] = p;
    }
    return g_addr[dev];
}

}  // namespace
}  // namespace symnmf

using namespace symnmf;

extern "C" int symnmf_sh_noalloc(const float* S, int64_t n, int64_t lds, const float* H,
                                 int32_t k, float* P, double* tr, void* hip_stream) {
    if (!S || !H || !P || n < 1 || n > INT32_MAX / 2 || k < 1 || k > kMaxWidth || lds < n ||
        lds % 4 || reinterpret_cast<uintptr_t>(S) % 16 || reinterpret_cast<uintptr_t>(P) % 4 ||
        (tr && reinterpret_cast<uintptr_t>(tr) % 8))
        return SYMNMF_E_INVALID;
    // the layout of symnmf_sh's workspace: partials, the trace partials, and
    // its one-double trace slot (unused here: the trace goes to *tr)
    const int nn = (int)n;
    const int rps = sh_full_rows_per_split(nn);
    const int nsplit = (nn + rps - 1) / rps;
    const int ldp = (k + 3) / 4 * 4;
    const int64_t nblk = (n + kUpdRows - 1) / kUpdRows;
    const size_t part_bytes = up256((size_t)nsplit * (size_t)n * ldp * sizeof(float));
    const size_t need = part_bytes + up256((size_t)nblk * sizeof(double)) + up256(sizeof(double));
    if (need > kScratchBytes) return SYMNMF_E_TOO_LARGE;
    hipError_t err;
    unsigned char* base = static_cast<unsigned char*>(scratch_address(&err));
    if (!base) return SYMNMF_E_HIP;
    float* part = reinterpret_cast<float*>(base);
    double* tr_part = reinterpret_cast<double*>(base + part_bytes);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const RowPlan rp{nn, rps, nullptr, 0, 0, 1, 0, 1, nullptr};
    if ((err = launch_sh_panel(S, lds, H, k, rp, nsplit, part, ldp, st)) != hipSuccess)
        return SYMNMF_E_HIP;
    if ((err = launch_reduce_partials(part, nsplit, nn, k, ldp, P, tr ? H : nullptr,
                                      tr ? tr_part : nullptr, st)) != hipSuccess)
        return SYMNMF_E_HIP;
    if (tr && (err = launch_sum_doubles(tr_part, nblk, tr, st)) != hipSuccess) return SYMNMF_E_HIP;
    return SYMNMF_OK;
}
