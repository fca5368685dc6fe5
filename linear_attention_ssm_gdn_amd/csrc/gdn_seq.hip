// gdn_seq.hip -- token-by-token GDN layer core: conv + SiLU + gating + gated
// delta rule fused in one launch (decode is T = 1).
//
// Grid: one workgroup per (sequence, value head h, block of 32 value
// columns).  The state block (d_k x 32) stays in VGPRs for the whole
// sequence.  Tokens are processed in chunks of TT:
//   A1  conv + SiLU of the chunk for the key head's q and k channels and the
//       block's v channels, one channel per thread, the window in registers;
//   A2  per token, L2 norms of q and k, k.q, e^g and beta (one wave per token);
//   B   the delta rule token by token (gdn::delta_step).
// The next chunk's x, a and b are loaded before B runs so their latency
// hides under the recurrence.
//
// Conv window ownership: v channels of the block are read and written only by
// this workgroup.  q/k channels of a key head are read by the r * (d_v/32)
// workgroups of that head; each arrives on the page's sync word once its
// window reads are done, and the last to arrive writes the rolled q/k window.
#include "gdn_block.hpp"
#include "gdn_kernels.h"
#include "../../include/gdn.h"

namespace gdn {

constexpr int SEQ_TT = 16;

template <typename ActT, typename StT, int DK>
__global__ __launch_bounds__(BLOCK_THREADS) void k_gdn_seq(const SeqArgs A) {
    constexpr int TT = SEQ_TT;
    constexpr int R = DK / 8;
    constexpr int NLC = 2 * DK + BV;  // local conv channels: q, k (key head), v (block)
    constexpr int NCH = (NLC + BLOCK_THREADS - 1) / BLOCK_THREADS;
    constexpr int PH = TT * (2 * DK + BV + 4);
    constexpr int ST = DK * STAGE_LD;
    __shared__ __attribute__((aligned(16))) float smem[PH > ST ? PH : ST];
    __shared__ int sh_last;
    float* sq = smem;                 // [TT][DK]  scale * q-hat
    float* sk = sq + TT * DK;         // [TT][DK]  k-hat
    float* sv = sk + TT * DK;         // [TT][BV]
    float* ssc = sv + TT * BV;        // [TT][4]   e^g, beta, k.q

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nblk = A.d_v / BV;
    int bid = blockIdx.x;
    const int blk = bid % nblk;
    bid /= nblk;
    const int h = bid % A.h_v;
    const int seq = bid / A.h_v;
    const int rr = A.h_v / A.h_k;
    const int ki = h / rr;
    const int colbase = blk * BV;
    const int64_t C = 2 * (int64_t)A.h_k * DK + (int64_t)A.h_v * A.d_v;

    const int page = A.page_idx[seq];
    if (page < 0) return;
    if (page >= A.conv_n_pages || page >= A.state_n_pages) {
        if (tid == 0 && h == 0 && blk == 0) set_err(A.err, GDN_DEVERR_PAGE);
        return;
    }
    const int r0 = A.cu[seq], r1 = A.cu[seq + 1];
    if (r0 < 0 || r1 < r0 || (int64_t)r1 > A.n_rows) {
        if (tid == 0 && h == 0 && blk == 0) set_err(A.err, GDN_DEVERR_BATCH);
        return;
    }
    const int T = r1 - r0;
    if (T == 0) return;
    const bool init = A.has_init ? (A.has_init[seq] != 0) : true;

    const ActT* __restrict__ X = static_cast<const ActT*>(A.x);
    const ActT* __restrict__ Wc = static_cast<const ActT*>(A.conv_w);
    ActT* __restrict__ win = static_cast<ActT*>(A.conv_base) + (int64_t)page * A.conv_page_stride;
    StT* __restrict__ Sg = static_cast<StT*>(A.state) + (int64_t)page * A.state_page_stride +
                           (int64_t)h * DK * A.d_v + colbase;

    // ---- conv channels of this thread
    int64_t gc[NCH];
    float w[NCH][4], xm3[NCH], xm2[NCH], xm1[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int lc = tid + j * BLOCK_THREADS;
        gc[j] = -1;
        if (lc < NLC) {
            gc[j] = lc < DK ? (int64_t)ki * DK + lc
                  : lc < 2 * DK ? (int64_t)A.h_k * DK + (int64_t)ki * DK + (lc - DK)
                  : 2 * (int64_t)A.h_k * DK + (int64_t)h * A.d_v + colbase + (lc - 2 * DK);
#pragma unroll
            for (int e = 0; e < 4; ++e) w[j][e] = to_f32(Wc[gc[j] * 4 + e]);
            xm3[j] = init ? to_f32(win[0 * C + gc[j]]) : 0.0f;
            xm2[j] = init ? to_f32(win[1 * C + gc[j]]) : 0.0f;
            xm1[j] = init ? to_f32(win[2 * C + gc[j]]) : 0.0f;
        }
    }
    const float exp_alog = expf(A.a_log[h]);
    const float dtb = A.dt_bias[h];

    // ---- state block into registers
    float s[R];
    if (init) {
        load_state_block<StT, DK>(Sg, A.d_v, smem, s, tid);
    } else {
#pragma unroll
        for (int m = 0; m < R; ++m) s[m] = 0.0f;
    }

    // ---- prefetch of chunk inputs
    float xp[NCH][TT];
    float pa[TT / 4], pb[TT / 4];
    auto prefetch = [&](int t0) {
#pragma unroll
        for (int j = 0; j < NCH; ++j)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
                xp[j][tt] = (gc[j] >= 0 && t0 + tt < T)
                                ? to_f32(X[(int64_t)(r0 + t0 + tt) * A.x_stride + gc[j]]) : 0.0f;
#pragma unroll
        for (int i = 0; i < TT / 4; ++i) {
            const int tt = wv + 4 * i;
            const bool ok = t0 + tt < T;
            const int64_t row = (int64_t)(r0 + t0 + tt) * A.ab_stride + h;
            pa[i] = ok ? to_f32(static_cast<const ActT*>(A.a)[row]) : 0.0f;
            pb[i] = ok ? to_f32(static_cast<const ActT*>(A.b)[row]) : 0.0f;
        }
    };
    prefetch(0);

    const int col = lane_col(tid), rb = lane_rowgroup(tid) * R;
    float* __restrict__ O = A.o + (int64_t)r0 * A.h_v * A.d_v + (int64_t)h * A.d_v + colbase + col;
    const int64_t o_stride = (int64_t)A.h_v * A.d_v;

    for (int t0 = 0; t0 < T; t0 += TT) {
        const int nt = (T - t0 < TT) ? (T - t0) : TT;
        // A1: conv + SiLU into LDS
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            if (gc[j] < 0) continue;
            const int lc = tid + j * BLOCK_THREADS;
            float* dst = lc < DK ? sq + lc : lc < 2 * DK ? sk + (lc - DK) : sv + (lc - 2 * DK);
            const int ld = lc < 2 * DK ? DK : BV;
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                if (tt < nt) {
                    const float x0 = xp[j][tt];
                    dst[tt * ld] = silu(conv4(w[j], xm3[j], xm2[j], xm1[j], x0));
                    xm3[j] = xm2[j];
                    xm2[j] = xm1[j];
                    xm1[j] = x0;
                }
            }
        }
        __syncthreads();
        if (t0 == 0 && tid == 0)  // every window read of this workgroup is done
            sh_last = arrive_last(A.sync + (int64_t)page * A.h_k + ki, (uint32_t)(rr * nblk)) ? 1 : 0;
        // A2: gating, one wave per token
#pragma unroll
        for (int i = 0; i < TT / 4; ++i) {
            const int tt = wv + 4 * i;
            if (tt < nt) {
                const float kq = gate_qk<DK>(sq + tt * DK, sk + tt * DK, A.scale, A.eps, lane);
                float eg, beta;
                gate_scalars(pa[i], pb[i], exp_alog, dtb, eg, beta);
                if (lane == 0) {
                    ssc[tt * 4 + 0] = eg;
                    ssc[tt * 4 + 1] = beta;
                    ssc[tt * 4 + 2] = kq;
                }
            }
        }
        __syncthreads();
        if (t0 + TT < T) prefetch(t0 + TT);
        // B: the recurrence
        for (int tt = 0; tt < nt; ++tt) {
            float k[R], q[R];
#pragma unroll
            for (int m = 0; m < R; m += 4) {
                const float4 kv4 = *reinterpret_cast<const float4*>(sk + tt * DK + rb + m);
                const float4 qv4 = *reinterpret_cast<const float4*>(sq + tt * DK + rb + m);
                k[m] = kv4.x; k[m + 1] = kv4.y; k[m + 2] = kv4.z; k[m + 3] = kv4.w;
                q[m] = qv4.x; q[m + 1] = qv4.y; q[m + 2] = qv4.z; q[m + 3] = qv4.w;
            }
            const float v = sv[tt * BV + col];
            const float eg = ssc[tt * 4 + 0], beta = ssc[tt * 4 + 1], kq = ssc[tt * 4 + 2];
            const float o = delta_step<R>(s, k, q, v, eg, beta, kq);
            if (lane_rowgroup(tid) == 0) O[(int64_t)(t0 + tt) * o_stride] = o;
        }
        __syncthreads();
    }

    // ---- epilogue: state, then the rolled windows
    store_state_block<StT, DK>(Sg, A.d_v, smem, s, tid);
    const bool last = sh_last != 0;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        if (gc[j] < 0) continue;
        const int lc = tid + j * BLOCK_THREADS;
        if (lc < 2 * DK && !last) continue;
        win[0 * C + gc[j]] = from_f32<ActT>(xm3[j]);
        win[1 * C + gc[j]] = from_f32<ActT>(xm2[j]);
        win[2 * C + gc[j]] = from_f32<ActT>(xm1[j]);
    }
}

template <typename ActT, typename StT, int DK>
static hipError_t launch_seq_t(const SeqArgs& a, hipStream_t s) {
    const int nblk = a.d_v / BV;
    const int64_t grid = (int64_t)a.n_seqs * a.h_v * nblk;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((k_gdn_seq<ActT, StT, DK>), dim3((unsigned)grid), dim3(BLOCK_THREADS), 0, s, a);
    return hipGetLastError();
}

template <typename ActT, typename StT>
static hipError_t launch_seq_dk(const SeqArgs& a, int d_k, hipStream_t s) {
    switch (d_k) {
        case 32: return launch_seq_t<ActT, StT, 32>(a, s);
        case 64: return launch_seq_t<ActT, StT, 64>(a, s);
        case 128: return launch_seq_t<ActT, StT, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

bool seq_supported(int d_k, int d_v) {
    return (d_k == 32 || d_k == 64 || d_k == 128) && d_v > 0 && d_v % BV == 0;
}

hipError_t launch_seq(const SeqArgs& a, int d_k, int act_dtype, int state_dtype, hipStream_t s) {
    if (act_dtype == GDN_BF16) {
        return state_dtype == GDN_BF16 ? launch_seq_dk<bf16_t, bf16_t>(a, d_k, s)
                                       : launch_seq_dk<bf16_t, float>(a, d_k, s);
    }
    return state_dtype == GDN_BF16 ? launch_seq_dk<float, bf16_t>(a, d_k, s)
                                   : launch_seq_dk<float, float>(a, d_k, s);
}

}  // namespace gdn
