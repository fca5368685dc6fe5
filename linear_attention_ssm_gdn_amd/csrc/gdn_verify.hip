// gdn_verify.hip -- one speculative verify step (Gated DeltaNet part (d)):
// the launcher of the workgroup in gdn_verify_block.hpp.
#include "gdn_verify_block.hpp"

namespace gdn {

template <typename ActT, typename StT, int DK, int CPL, int LAYOUT>
__global__ __launch_bounds__(BLOCK_THREADS) void k_gdn_verify(const VerifyArgs A) {
    verify_block<ActT, StT, DK, CPL, LAYOUT>(A, blockIdx.x);
}

template <typename ActT, typename StT, int DK, int CPL>
static hipError_t launch_verify_t(const VerifyArgs& a, int layout, hipStream_t s) {
    const int nblk = a.d_v / (32 * CPL);
    const int64_t grid = (int64_t)a.n_req * a.h_v * nblk;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (layout == GDN_SPEC_ONEPAGE)
        hipLaunchKernelGGL((k_gdn_verify<ActT, StT, DK, CPL, GDN_SPEC_ONEPAGE>), dim3((unsigned)grid),
                           dim3(BLOCK_THREADS), 0, s, a);
    else
        hipLaunchKernelGGL((k_gdn_verify<ActT, StT, DK, CPL, GDN_SPEC_SLOTS>), dim3((unsigned)grid),
                           dim3(BLOCK_THREADS), 0, s, a);
    return hipGetLastError();
}

template <typename ActT, typename StT, int DK>
static hipError_t launch_verify_shape(const VerifyArgs& a, int layout, hipStream_t s) {
    if (a.d_v % 128 == 0) return launch_verify_t<ActT, StT, DK, 4>(a, layout, s);
    return launch_verify_t<ActT, StT, DK, 1>(a, layout, s);
}

template <typename ActT, typename StT>
static hipError_t launch_verify_dk(const VerifyArgs& a, int d_k, int layout, hipStream_t s) {
    switch (d_k) {
        case 32: return launch_verify_shape<ActT, StT, 32>(a, layout, s);
        case 64: return launch_verify_shape<ActT, StT, 64>(a, layout, s);
        case 128: return launch_verify_shape<ActT, StT, 128>(a, layout, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_verify(const VerifyArgs& a, int d_k, int act_dtype, int state_dtype, int layout,
                         hipStream_t s) {
    if (act_dtype == GDN_BF16)
        return state_dtype == GDN_BF16 ? launch_verify_dk<bf16_t, bf16_t>(a, d_k, layout, s)
                                       : launch_verify_dk<bf16_t, float>(a, d_k, layout, s);
    return state_dtype == GDN_BF16 ? launch_verify_dk<float, bf16_t>(a, d_k, layout, s)
                                   : launch_verify_dk<float, float>(a, d_k, layout, s);
}

}  // namespace gdn
