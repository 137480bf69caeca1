// gemm_w8a8_g128_noalloc: the W8A8 G128 linear with its scratch memory in a static
// device array instead of a caller-provided workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The scratch array holds, as a gemm_w8a8_g128 workspace does, the split-K arrival
// counters (64 KiB at offset 0), the quantised activations when x is passed, and the
// split-K partial sums.  It is a file-scope __device__ array, so every GPU the
// library runs on holds its own copy until the process ends.  Host code never uses
// the array's name as an address: at the first call on a device (with that device
// current) hipGetSymbolAddress gives the device address, kept per device, and that
// address is what the kernels receive.
#include <mutex>

#include "internal.h"

namespace i8gs {
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;  // 16 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

// Zeroes the counter region (first call on a device only; afterwards every completed
// call leaves the counters it used at zero).  A kernel rather than hipMemsetAsync,
// so that it records cleanly when the first call happens under graph capture.
__global__ __launch_bounds__(256) void zero_words_kernel(int *__restrict__ p, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

struct DeviceScratch {
    std::once_flag once;
    char *ptr = nullptr;
    hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

// Device address of this device's scratch array (resolved once per device, with the
// device current), and whether this call is the first on the device.
int scratch_for_current_device(char **out, bool *first) {
    int dev = 0;
    I8GS_TRY(hip_check(hipGetDevice(&dev), "hipGetDevice"));
    if (dev < 0 || dev >= kMaxDevices) return fail(I8GS_ERR_UNSUPPORTED_DEVICE, "device index out of range");
    DeviceScratch &d = g_scratch[dev];
    bool ran = false;
    std::call_once(d.once, [&] {
        ran = true;
        void *p = nullptr;
        d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        d.ptr = d.err == hipSuccess ? static_cast<char *>(p) : nullptr;
    });
    if (d.err != hipSuccess || d.ptr == nullptr)
        return hip_check(d.err != hipSuccess ? d.err : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    *out = d.ptr;
    *first = ran;
    return I8GS_OK;
}

}  // namespace
}  // namespace i8gs

using namespace i8gs;

extern "C" size_t i8gs_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int gemm_w8a8_g128_noalloc(const void *x, int64_t ldx, const int8_t *qa, const float *a_scale,
                                      const int32_t *qweight, const float *w_scale, void *y, int64_t ldy,
                                      int64_t M, int64_t N, int64_t K, void *stream) {
    W8A8Plan plan;
    I8GS_TRY(w8a8_validate(x, ldx, qa, a_scale, qweight, w_scale, y, ldy, M, N, K, I8GS_KERNEL_AUTO, 0, &plan));
    if (M == 0 || N == 0) return ok();
    // The counters and the quantised activations must fit; the prefill kernel's split
    // pieces are used only where they fit too (otherwise it runs whole tiles, as with a
    // workspace that has no room for them).
    const size_t fixed = kCounterBytes + (plan.have_x ? plan.quant_bytes : 0);
    const size_t need = fixed + (plan.decode ? plan.gemm_bytes : 0);
    if (need > kNoAllocScratchBytes)
        return fail(I8GS_ERR_WORKSPACE,
                    std::string("the call needs ") + std::to_string(need) + " bytes of scratch; the no-allocation "
                    "entry point holds " + std::to_string(kNoAllocScratchBytes) +
                    " (pass qa/a_scale, or use gemm_w8a8_g128 with a workspace)");
    I8GS_TRY(check_device());
    char *base = nullptr;
    bool first = false;
    I8GS_TRY(scratch_for_current_device(&base, &first));
    hipStream_t s = (hipStream_t)stream;
    if (first) {
        zero_words_kernel<<<16, 256, 0, s>>>(reinterpret_cast<int *>(base), int(kCounterBytes / sizeof(int)));
        I8GS_TRY(hip_check(hipGetLastError(), "scratch counter clear"));
    }
    // Layout: counters, the quantised activations (only when x is given), the split pieces.
    char *const quant = base + kCounterBytes;
    return w8a8_launch(plan, x, ldx, qa, a_scale, qweight, w_scale, y, ldy, base, quant, base + fixed,
                       kNoAllocScratchBytes - fixed, s);
}
