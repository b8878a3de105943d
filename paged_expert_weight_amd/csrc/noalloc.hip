// The routing + layer forward for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): moe_route_forward with its workspace in a static device array
// of this library instead of a caller's allocation.
//
// The array is file-scope device memory of a fixed size; every GPU the library
// runs on holds its own copy until the process ends.  In host code the array's
// name only stands for the symbol: its device address on the current device is
// looked up once per device with hipGetSymbolAddress, and that address is what
// the kernels receive.  Nothing in the workspace has to start at zero (every
// kernel writes what it later reads: route counts, h rows of real picks, the
// combine rows, the atomic accumulator, which its launch clears with a fill
// kernel), so the array's contents left by an earlier call do not matter; two
// calls on one GPU that overlap in time share the array and race.
#include "moe.h"
#include "internal.h"

#include <mutex>
#include <string>

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices]; // device address of `scratch` on each device (null until looked up)

// The current device's address of the scratch array, looked up on the first
// call on that device.
int scratch_ptr(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return pmoe::set_error(MOE_ERR_HIP, (std::string("hipGetDevice: ") + hipGetErrorString(e)).c_str());
    }
    if (dev < 0 || dev >= kMaxDevices)
        return pmoe::set_error(MOE_ERR_UNSUPPORTED, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return pmoe::set_error(MOE_ERR_HIP,
                                   (std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e)).c_str());
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

} // namespace

extern "C" int moe_route_forward_noalloc(moe_pool *pool, const float *logits, const void *x, int64_t T,
                                         int32_t block_m, int32_t *topk_ids, float *topk_w, int32_t *sorted_ids,
                                         int32_t *block_expert, int32_t *num_padded, int32_t active_buf, void *y,
                                         uint32_t flags, void *stream)
{
    if (!pool)
        return pmoe::set_error(MOE_ERR_INVALID_ARG, "pool is null");
    size_t need = 0;
    int rc = moe_workspace_bytes(pool, T, block_m, flags, &need);
    if (rc != MOE_OK)
        return rc;
    if (need > kScratchBytes)
        return pmoe::set_error(MOE_ERR_WORKSPACE,
                               ("moe_route_forward_noalloc: T=" + std::to_string(T) + ", block_m=" +
                                std::to_string(block_m) + " needs " + std::to_string(need) +
                                " bytes of workspace, the static scratch holds " + std::to_string(kScratchBytes) +
                                "; use moe_route_forward with a caller workspace")
                                   .c_str());
    void *ws = nullptr;
    rc = scratch_ptr(&ws);
    if (rc != MOE_OK)
        return rc;
    return moe_route_forward(pool, logits, x, T, block_m, topk_ids, topk_w, sorted_ids, block_expert, num_padded,
                             active_buf, y, ws, kScratchBytes, flags, stream);
}
