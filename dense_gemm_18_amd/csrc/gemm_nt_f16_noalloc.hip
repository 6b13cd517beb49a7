// gemm_nt_f16_noalloc.hip -- gemm_nt_f16_ws_noalloc: the stream-K form of
// the fp16 GEMM for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops), with its workspace in a static
// device array instead of caller memory.  Kernels, planning and launch
// helpers are in gemm_kernels.h.
#include "gemm_kernels.h"

// The workspace: stream-K header, flags and fp32 partial sums for a grid of
// up to 256 workgroups on the largest stream-K tile, 128 x 128 (16 MiB +
// 1.25 KiB), one copy per GPU, held until the process ends.  In host code this name is only a stand-in for the device
// symbol, never an address: kernels get the pointer hipGetSymbolAddress
// returns for the current device.
static __device__ __align__(256) unsigned char
    scratch[kSkHdrBytes + 256 * 4 + (int64_t)256 * 128 * 128 * 4];

namespace {
constexpr int64_t kScratchBytes = (int64_t)sizeof(scratch);
constexpr int kMaxDevices = 64;
// Per device: the scratch address, and 0 (not looked up yet), 1 (ready) or
// 2 (the lookup failed).
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::atomic<int> g_scratch_state[kMaxDevices];

// Zero-fills `words` 32-bit words with a kernel, so that a caller's graph
// capture records no memset node.
__global__ void fill_words_kernel(uint32_t *__restrict__ p, int words)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < words; i += gridDim.x * blockDim.x)
        p[i] = 0u;
}

// The current device's scratch address.  The first call on a device looks
// it up (with that device current, as every call is) and enqueues the
// zero-fill of the header and flags on `stream`, ahead of the GEMM.
void *scratch_on_device(hipStream_t stream)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    const int st = g_scratch_state[dev].load(std::memory_order_acquire);
    if (st == 1)
        return g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (st == 2)
        return nullptr;
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
        g_scratch_state[dev].store(2, std::memory_order_release);
        return nullptr;
    }
    constexpr int words = (int)((kSkHdrBytes + 256 * 4) / 4);
    hipLaunchKernelGGL(fill_words_kernel, dim3(1), dim3(256), 0, stream, (uint32_t *)ptr, words);
    g_scratch_ptr[dev].store(ptr, std::memory_order_relaxed);
    g_scratch_state[dev].store(1, std::memory_order_release);
    return ptr;
}
} // namespace

extern "C" {
int gemm_nt_f16_ws_noalloc(const void *A, const void *B, void *D, int64_t M, int64_t N,
                           int64_t K, hipStream_t stream)
{
    const int rc = validate(A, B, D, M, N, K);
    if (rc != GEMM_OK)
        return rc;
    const int lb = load_bytes(A, B, M, N, K);
    if (M == 0 || N == 0 || K == 0 || lb == 0)
        return gemm_nt_f16(A, B, D, M, N, K, stream);
    const Plan pl = make_plan(M, N, K, lb, device_cus());
    if (!pl.sk)
        return gemm_nt_f16(A, B, D, M, N, K, stream);
    if (workspace_bytes(pl) > kScratchBytes)
        return GEMM_ESCRATCH;
    void *ws = scratch_on_device(stream);
    if (!ws)
        return GEMM_ELAUNCH;
    SkPlan sp = pl.split;
    bind_workspace(sp, ws, pl.grid);
    launch_sk(A, B, D, (int)M, (int)N, (int)K, stream, sp, pl.grid, pl.tile);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ELAUNCH;
}

} // extern "C"
