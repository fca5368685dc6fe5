// gdn_conv.hip -- causal depthwise conv (width 4) + optional SiLU over a
// ragged batch, with the rolling conv window (Gated DeltaNet part (a)).
//
// Grid: (sequence, tile of 256 channels, segment of CONV_TS tokens); one
// channel per thread, tokens of the segment in order.  Rows before a
// segment's first token come from x (segments > 0) or from the page's window
// (segment 0).  Only segment 0 reads the old window, so segment 0 alone writes
// the rolled one, after its own reads: no other workgroup touches the window.
#include "gdn_block.hpp"
#include "gdn_kernels.h"
#include "../../include/gdn.h"

namespace gdn {

constexpr int CONV_THREADS = 256;
constexpr int CONV_TS = 64;

template <typename ActT, typename YT>
__global__ __launch_bounds__(CONV_THREADS) void k_conv_update(const ConvArgs A, int n_tiles, int n_seg,
                                                               int seg_len) {
    int bid = blockIdx.x;
    const int seg = bid % n_seg;
    bid /= n_seg;
    const int tile = bid % n_tiles;
    const int seq = bid / n_tiles;
    const int tid = threadIdx.x;
    const int64_t C = A.C;
    const int64_t c = (int64_t)tile * CONV_THREADS + tid;

    const int page = A.page_idx[seq];
    if (page < 0) return;
    if (page >= A.conv_n_pages) {
        if (tid == 0 && tile == 0 && seg == 0) set_err(A.err, GDN_DEVERR_PAGE);
        return;
    }
    const int r0 = A.cu[seq], r1 = A.cu[seq + 1];
    if (r0 < 0 || r1 < r0 || (int64_t)r1 > A.n_rows) {
        if (tid == 0 && tile == 0 && seg == 0) set_err(A.err, GDN_DEVERR_BATCH);
        return;
    }
    const int T = r1 - r0;
    const int64_t t_beg = (int64_t)seg * seg_len;
    if (seg == n_seg - 1 && t_beg + seg_len < T && tid == 0 && tile == 0) set_err(A.err, GDN_DEVERR_BATCH);
    if (t_beg >= T || c >= C) return;
    const int t_end = (int)((t_beg + seg_len < T) ? t_beg + seg_len : T);
    const bool init = A.has_init ? (A.has_init[seq] != 0) : true;

    const ActT* __restrict__ X = static_cast<const ActT*>(A.x) + (int64_t)r0 * A.x_stride + c;
    ActT* __restrict__ win = static_cast<ActT*>(A.conv_base) + (int64_t)page * A.conv_page_stride + c;
    YT* __restrict__ Y = static_cast<YT*>(A.y) + (int64_t)r0 * A.y_stride + c;
    const ActT* Wc = static_cast<const ActT*>(A.conv_w) + c * 4;
    float w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = to_f32(Wc[e]);

    // the three rows before t_beg, oldest first
    float xm[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int64_t t = t_beg - 3 + j;
        if (t >= 0) xm[j] = to_f32(X[t * A.x_stride]);
        else xm[j] = init ? to_f32(win[(3 + t) * C]) : 0.0f;
    }
    const bool act = A.activation != 0;
    for (int t = (int)t_beg; t < t_end; ++t) {
        const float x0 = to_f32(X[(int64_t)t * A.x_stride]);
        const float z = conv4(w, xm[0], xm[1], xm[2], x0);
        Y[(int64_t)t * A.y_stride] = from_f32<YT>(act ? silu(z) : z);
        xm[0] = xm[1];
        xm[1] = xm[2];
        xm[2] = x0;
    }
    if (seg == 0) {
        // rolled window: last 3 rows of (window ++ x); rows already in xm when
        // this segment reached the end of the sequence
        if (t_end < T) {
#pragma unroll
            for (int j = 0; j < 3; ++j) xm[j] = to_f32(X[(int64_t)(T - 3 + j) * A.x_stride]);
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) win[j * C] = from_f32<ActT>(xm[j]);
    }
}

template <typename ActT, typename YT>
static hipError_t launch_conv_t(const ConvArgs& a, int max_seqlen, hipStream_t s) {
    const int n_tiles = (a.C + CONV_THREADS - 1) / CONV_THREADS;
    const int n_seg = max_seqlen > 0 ? (max_seqlen + CONV_TS - 1) / CONV_TS : 1;
    const int seg_len = max_seqlen > 0 ? CONV_TS : 0x7fffffff;
    const int64_t grid = (int64_t)a.n_seqs * n_tiles * n_seg;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_conv_update<ActT, YT>), dim3((unsigned)grid), dim3(CONV_THREADS), 0, s, a, n_tiles,
                       n_seg, seg_len);
    return hipGetLastError();
}

hipError_t launch_conv(const ConvArgs& a, int act_dtype, int y_dtype, int max_seqlen, hipStream_t s) {
    if (act_dtype == GDN_BF16)
        return y_dtype == GDN_BF16 ? launch_conv_t<bf16_t, bf16_t>(a, max_seqlen, s)
                                   : launch_conv_t<bf16_t, float>(a, max_seqlen, s);
    return y_dtype == GDN_BF16 ? launch_conv_t<float, bf16_t>(a, max_seqlen, s)
                               : launch_conv_t<float, float>(a, max_seqlen, s);
}

}  // namespace gdn
