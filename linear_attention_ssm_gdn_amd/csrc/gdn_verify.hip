// gdn_verify.hip -- one speculative verify step (Gated DeltaNet part (d)):
// the launcher of the workgroup in gdn_verify_block.hpp, and the copy that
// restores cached prefixes into fresh speculative pages.
#include "gdn_verify_block.hpp"

namespace gdn {

template <typename ActT, typename StT, int DK, int CPL, int LAYOUT, bool CACHE>
__global__ __launch_bounds__(BLOCK_THREADS) void k_gdn_verify(const VerifyArgs A) {
    verify_block<ActT, StT, DK, CPL, LAYOUT, CACHE>(A, blockIdx.x);
}

template <typename ActT, typename StT, int DK, int CPL, bool CACHE>
static hipError_t launch_verify_c(const VerifyArgs& a, int layout, hipStream_t s) {
    const int nblk = a.d_v / (32 * CPL);
    const int64_t grid = (int64_t)a.n_req * a.h_v * nblk;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (layout == GDN_SPEC_ONEPAGE)
        hipLaunchKernelGGL((k_gdn_verify<ActT, StT, DK, CPL, GDN_SPEC_ONEPAGE, CACHE>), dim3((unsigned)grid),
                           dim3(BLOCK_THREADS), 0, s, a);
    else
        hipLaunchKernelGGL((k_gdn_verify<ActT, StT, DK, CPL, GDN_SPEC_SLOTS, CACHE>), dim3((unsigned)grid),
                           dim3(BLOCK_THREADS), 0, s, a);
    return hipGetLastError();
}

template <typename ActT, typename StT, int DK, int CPL>
static hipError_t launch_verify_t(const VerifyArgs& a, int layout, hipStream_t s) {
    if (a.cache_entry) return launch_verify_c<ActT, StT, DK, CPL, true>(a, layout, s);
    return launch_verify_c<ActT, StT, DK, CPL, false>(a, layout, s);
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

// Restore of cached prefixes: one workgroup per (request, value head) copies
// that head's cached state into the page's state region (the one-page
// checkpoint, or slot 0 of the slot design: both start at state_off), and
// its share of the cached window's channels into conv rows 0 .. rows-1;
// head 0 also writes the all-zero header of a fresh page.  Pure data
// movement, element by element in the stored dtypes.
constexpr int RESTORE_THREADS = 256;

template <typename ActT, typename StT>
__global__ __launch_bounds__(RESTORE_THREADS) void k_prefix_restore(const RestoreArgs A) {
    const int h = blockIdx.x % A.h_v;
    const int req = blockIdx.x / A.h_v;
    const int tid = threadIdx.x;
    const int e = A.entry[req];
    const int page = A.req_page[req];
    if (e < 0 || page < 0) return;
    if (e >= A.cache_state_n || e >= A.cache_conv_n) {
        if (h == 0 && tid == 0) set_err(A.err, GDN_DEVERR_CACHE);
        return;
    }
    if (page >= A.n_pages || page >= A.conv_n_pages) {
        if (h == 0 && tid == 0) set_err(A.err, GDN_DEVERR_PAGE);
        return;
    }
    uint8_t* pg = A.pages + (int64_t)page * A.page_bytes;
    const int64_t head_elems = (int64_t)A.d_k * A.d_v;
    const StT* __restrict__ src = static_cast<const StT*>(A.cache_state) + (int64_t)e * A.cache_state_stride +
                                  (int64_t)h * head_elems;
    StT* __restrict__ dst = reinterpret_cast<StT*>(pg + A.state_off) + (int64_t)h * head_elems;
    for (int64_t i = tid; i < head_elems; i += RESTORE_THREADS) dst[i] = src[i];
    const int64_t per = (A.C + A.h_v - 1) / A.h_v;
    const int64_t c0 = (int64_t)h * per, c1 = (c0 + per < A.C) ? c0 + per : A.C;
    const ActT* __restrict__ wsrc = static_cast<const ActT*>(A.cache_conv) + (int64_t)e * A.cache_conv_stride;
    ActT* __restrict__ wdst = static_cast<ActT*>(A.conv_base) + (int64_t)page * A.conv_page_stride;
    for (int r = 0; r < A.conv_rows; ++r)
        for (int64_t c = c0 + tid; c < c1; c += RESTORE_THREADS) wdst[(int64_t)r * A.C + c] = wsrc[(int64_t)r * A.C + c];
    if (h == 0 && tid < (int)(sizeof(gdn_spec_header) / 4))
        reinterpret_cast<uint32_t*>(pg + A.header_off)[tid] = 0u;
}

template <typename ActT, typename StT>
static hipError_t launch_restore_t(const RestoreArgs& a, hipStream_t s) {
    const int64_t grid = (int64_t)a.n_req * a.h_v;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_prefix_restore<ActT, StT>), dim3((unsigned)grid), dim3(RESTORE_THREADS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_restore(const RestoreArgs& a, int act_dtype, int state_dtype, hipStream_t s) {
    if (act_dtype == GDN_BF16)
        return state_dtype == GDN_BF16 ? launch_restore_t<bf16_t, bf16_t>(a, s) : launch_restore_t<bf16_t, float>(a, s);
    return state_dtype == GDN_BF16 ? launch_restore_t<float, bf16_t>(a, s) : launch_restore_t<float, float>(a, s);
}

}  // namespace gdn
