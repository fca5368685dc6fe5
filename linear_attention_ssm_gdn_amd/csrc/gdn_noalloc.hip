// gdn_noalloc.hip -- gdn_recurrent_seq_noalloc: the token-by-token entry
// point for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The token-by-token kernels keep small counters beside the inputs and
// outputs: one arrival counter per (page, key head), through which the last
// workgroup to read a shared conv window writes the rolled one, and the work
// counter from which the decode kernel hands out items.  gdn_recurrent_seq
// takes them from the caller (gdn_conv_pool.sync); this entry point keeps
// them in `scratch`, a file-scope device array of GDN_NOALLOC_SYNC_WORDS
// words that every GPU the library runs on holds until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gdn.h"
#include "gdn_kernels.h"

#define GDN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

__device__ __align__(256) uint32_t scratch[GDN_NOALLOC_SYNC_WORDS];

// The device address of `scratch` on each device, taken once per device
// with that device current.  In host code the array's name is only a
// host-side stand-in; kernels and fills get this address.
constexpr int kMaxDevices = 64;
uint32_t* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

hipError_t scratch_on_current_device(uint32_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = static_cast<uint32_t*>(p);
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

// Zero n words (a fill kernel rather than a memset, so a captured call
// records only kernel nodes).
__global__ __launch_bounds__(256) void k_zero_words(uint32_t* __restrict__ p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

}  // namespace

GDN_EXPORT int32_t gdn_recurrent_seq_noalloc(const gdn_dims* dims, const gdn_params* params, const void* x,
                                             int64_t x_stride, const void* a, const void* b, int64_t ab_stride,
                                             const gdn_batch* batch, gdn_conv_pool conv, gdn_state_pool state,
                                             float* o, int32_t* err, void* stream) {
    gdn::SeqArgs A{};
    int32_t st = gdn::seq_call_args_nosync(dims, params, x, x_stride, a, b, ab_stride, batch, conv, state, o, err, &A);
    if (st != GDN_OK || batch->n_seqs == 0) return st;
    // the arrival counters of every page, then the work counter
    const int64_t words = (int64_t)conv.n_pages * dims->h_k + 1;
    if (words > GDN_NOALLOC_SYNC_WORDS) return GDN_ERR_ARG;
    uint32_t* sync = nullptr;
    if (scratch_on_current_device(&sync) != hipSuccess) return GDN_ERR_LAUNCH;
    A.sync = sync;
    const hipStream_t s = (hipStream_t)stream;
    const int64_t blocks = (words + 255) / 256;
    hipLaunchKernelGGL(k_zero_words, dim3((unsigned)(blocks < 64 ? blocks : 64)), dim3(256), 0, s, sync, words);
    if (hipGetLastError() != hipSuccess) return GDN_ERR_LAUNCH;
    return gdn::launch_seq(A, dims->d_k, dims->act_dtype, dims->state_dtype, batch->max_seqlen, s) == hipSuccess
               ? GDN_OK
               : GDN_ERR_LAUNCH;
}
