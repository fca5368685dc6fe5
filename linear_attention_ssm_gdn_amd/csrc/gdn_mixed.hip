// gdn_mixed.hip -- one launch for a serving step that mixes token-by-token
// sequences (prefill or decode rows of a ragged batch) with speculative
// verify requests ("r9700-stack v0.2.3", section "1. Time to first token":
// the prefill and verify kernels read their rows in place, so a mixed step
// gathers nothing; "r9700-stack v0.2.4" names the mixed-step path beside
// the one-page verify).
//
// Grid, in the order workgroups are handed out: the workgroups of the
// token-by-token part (gdn_seq_block.hpp, 32 columns each, ranked longest
// sequence first), then
// those of the verify step (gdn_verify_block.hpp), which fill the slots that
// shorter sequences free.  (Handing the verify workgroups out right after the
// longest sequence's was measured slower: 396 against 368 us for the
// short-prefill batch plus 32 verify requests, with the longest sequence's
// waves at raised issue priority.)  Each workgroup runs exactly
// the code of its stand-alone kernel, so the step's results are those of the
// two separate launches, bit for bit.
#include "gdn_seq_block.hpp"
#include "gdn_verify_block.hpp"

namespace gdn {

template <typename ActT, typename StT, int DK, int VCPL, int LAYOUT>
__global__ __launch_bounds__(BLOCK_THREADS) void k_gdn_mixed(const SeqArgs S, const VerifyArgs V,
                                                            const int n_seq_blocks) {
    const int b = blockIdx.x;
    if (b < n_seq_blocks)
        seq_block<ActT, StT, DK, 1, 16>(S, b);
    else
        verify_block<ActT, StT, DK, VCPL, LAYOUT>(V, b - n_seq_blocks);
}

template <typename ActT, typename StT, int DK, int VCPL>
static hipError_t launch_mixed_t(const SeqArgs& s, const VerifyArgs& v, int layout, hipStream_t st) {
    const int64_t nseq = s.n_seqs > 0 ? (int64_t)s.n_seqs * s.h_v * (s.d_v / 32) : 0;
    const int64_t nver = v.n_req > 0 ? (int64_t)v.n_req * v.h_v * (v.d_v / (32 * VCPL)) : 0;
    const int64_t grid = nseq + nver;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (layout == GDN_SPEC_ONEPAGE)
        hipLaunchKernelGGL((k_gdn_mixed<ActT, StT, DK, VCPL, GDN_SPEC_ONEPAGE>), dim3((unsigned)grid),
                           dim3(BLOCK_THREADS), 0, st, s, v, (int)nseq);
    else
        hipLaunchKernelGGL((k_gdn_mixed<ActT, StT, DK, VCPL, GDN_SPEC_SLOTS>), dim3((unsigned)grid),
                           dim3(BLOCK_THREADS), 0, st, s, v, (int)nseq);
    return hipGetLastError();
}

template <typename ActT, typename StT, int DK>
static hipError_t launch_mixed_shape(const SeqArgs& s, const VerifyArgs& v, int layout, hipStream_t st) {
    if (v.d_v % 128 == 0) return launch_mixed_t<ActT, StT, DK, 4>(s, v, layout, st);
    return launch_mixed_t<ActT, StT, DK, 1>(s, v, layout, st);
}

template <typename ActT, typename StT>
static hipError_t launch_mixed_dk(const SeqArgs& s, const VerifyArgs& v, int d_k, int layout, hipStream_t st) {
    switch (d_k) {
        case 32: return launch_mixed_shape<ActT, StT, 32>(s, v, layout, st);
        case 64: return launch_mixed_shape<ActT, StT, 64>(s, v, layout, st);
        case 128: return launch_mixed_shape<ActT, StT, 128>(s, v, layout, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mixed(const SeqArgs& s, const VerifyArgs& v, int d_k, int act_dtype, int state_dtype, int layout,
                        hipStream_t st) {
    if (act_dtype == GDN_BF16)
        return state_dtype == GDN_BF16 ? launch_mixed_dk<bf16_t, bf16_t>(s, v, d_k, layout, st)
                                       : launch_mixed_dk<bf16_t, float>(s, v, d_k, layout, st);
    return state_dtype == GDN_BF16 ? launch_mixed_dk<float, bf16_t>(s, v, d_k, layout, st)
                                   : launch_mixed_dk<float, float>(s, v, d_k, layout, st);
}

}  // namespace gdn
