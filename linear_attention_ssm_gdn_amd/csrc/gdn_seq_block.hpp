// gdn_seq_block.hpp -- one workgroup of the token-by-token GDN layer core,
// as a device function of its block index, so that the token-by-token
// kernel and the mixed-step kernel run the same code: conv + SiLU + gating
// + gated delta rule fused (decode is T = 1).
//
// Grid: one workgroup per (sequence, value head h, block of 32*CPL value
// columns).  The state block stays in VGPRs for the whole sequence; it is
// loaded straight into the lane layout of gdn_block.hpp right after the small
// conv inputs, so its bytes are in flight while the first chunk's conv and
// gating run.  Tokens are processed in
// chunks of TT:
//   A1  conv + SiLU of the chunk for the key head's q and k channels and the
//       block's v channels, one channel per thread, the window in registers;
//   A2  per token, L2 norms of q and k, k.q, e^g and beta (one wave per token);
//   B   the delta rule token by token (gdn::delta_step).
// The next chunk's x, a and b are loaded before B runs so their latency hides
// under the recurrence.
//
// Conv window ownership: v channels of the block are read and written only by
// this workgroup.  q/k channels of a key head are read by the r * (d_v/BV)
// workgroups of that head; each arrives on the page's sync word once its
// window reads are consumed, and the last to arrive writes the rolled q/k
// window (gdn::arrive_last).
#pragma once

#include "gdn_block.hpp"
#include "gdn_kernels.h"
#include "../../include/gdn.h"

namespace gdn {

template <typename ActT, typename StT, int DK, int CPL, int TT>
__device__ __forceinline__ void seq_block(const SeqArgs& A, const int block) {
    constexpr int R = DK / 16;
    constexpr int BV = 32 * CPL;
    constexpr int NLC = 2 * DK + BV;  // local conv channels: q, k (key head), v (block)
    static_assert(TT <= 32, "one 16-lane row per token of a chunk");
    static_assert(NLC <= BLOCK_THREADS, "one conv channel per thread");
    __shared__ __attribute__((aligned(16))) float sq[TT * DK];   // scale * q-hat
    __shared__ __attribute__((aligned(16))) float sk[TT * DK];   // k-hat
    __shared__ __attribute__((aligned(16))) float sv[TT * BV];
    __shared__ float ssc[TT * 4];                                // e^g, beta, k.q
    __shared__ int sh_last;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nblk = A.d_v / BV;
    int bid = block;
    const int blk = bid % nblk;
    bid /= nblk;
    const int h = bid % A.h_v;
    // Dispatch order: workgroups are handed out in index order, so when the
    // grid exceeds what stays resident, index v is mapped to the v-th longest
    // sequence (ties by position) and the longest sequences, which set the
    // kernel's critical path, start first.  Every workgroup ranks the lengths
    // itself (batches of up to one sequence per thread; larger batches keep
    // their order).
    int seq = bid / A.h_v;
    if (A.n_seqs > 1 && A.n_seqs <= BLOCK_THREADS) {
        int* len = reinterpret_cast<int*>(sq);  // free until the first conv
        __shared__ int sh_seq;
        const int n = A.n_seqs;
        int my = 0;
        if (tid < n) {
            my = A.cu[tid + 1] - A.cu[tid];
            len[tid] = my;
        }
        __syncthreads();
        if (tid < n) {
            int rank = 0;
            for (int j = 0; j < n; ++j) {
                const int lj = len[j];
                rank += (lj > my || (lj == my && j < tid)) ? 1 : 0;
            }
            if (rank == seq) sh_seq = tid;
        }
        __syncthreads();
        seq = sh_seq;
    }
    const int rr = A.h_v / A.h_k;
    const int ki = h / rr;
    const int colbase = blk * BV;
    const int64_t C = 2 * (int64_t)A.h_k * DK + (int64_t)A.h_v * A.d_v;

    const int page = A.page_idx[seq];
    const int r0 = A.cu[seq], r1 = A.cu[seq + 1];
    if (page < 0) return;
    if (page >= A.conv_n_pages || page >= A.state_n_pages || (A.spec_pages && page >= A.spec_n_pages)) {
        if (tid == 0 && h == 0 && blk == 0) set_err(A.err, GDN_DEVERR_PAGE);
        return;
    }
    if (r0 < 0 || r1 < r0 || (int64_t)r1 > A.n_rows) {
        if (tid == 0 && h == 0 && blk == 0) set_err(A.err, GDN_DEVERR_BATCH);
        return;
    }
    const int T = r1 - r0;
    if (T == 0) return;
    const bool init = A.has_init ? (A.has_init[seq] != 0) : true;
    // The sequence's speculative page, if any, is left fresh (all-zero
    // header fields: live slot 0 with no record rows, parity 0).
    if (A.spec_pages && tid == 0 && h == 0 && blk == 0) {
        uint32_t* hw = reinterpret_cast<uint32_t*>(A.spec_pages + (int64_t)page * A.spec_page_bytes);
        hw[0] = 0u; hw[1] = 0u; hw[2] = 0u; hw[3] = 0u;
    }

    // ---- this thread's conv channel
    const ActT* __restrict__ X = static_cast<const ActT*>(A.x);
    ActT* __restrict__ win = static_cast<ActT*>(A.conv_base) + (int64_t)page * A.conv_page_stride;
    const int lc = tid;
    int64_t gc = -1;
    float w[4] = {0.0f, 0.0f, 0.0f, 0.0f}, xm3 = 0.0f, xm2 = 0.0f, xm1 = 0.0f;
    if (lc < NLC) {
        gc = lc < DK ? (int64_t)ki * DK + lc
           : lc < 2 * DK ? (int64_t)A.h_k * DK + (int64_t)ki * DK + (lc - DK)
           : 2 * (int64_t)A.h_k * DK + (int64_t)h * A.d_v + colbase + (lc - 2 * DK);
        const ActT* Wc = static_cast<const ActT*>(A.conv_w) + gc * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = to_f32(Wc[e]);
        if (init) {
            xm3 = to_f32(win[0 * C + gc]);
            xm2 = to_f32(win[1 * C + gc]);
            xm1 = to_f32(win[2 * C + gc]);
        }
    }
    float* ydst = lc < DK ? sq + qk_pos<DK>(lc) : lc < 2 * DK ? sk + qk_pos<DK>(lc - DK) : sv + (lc - 2 * DK);
    const int yld = lc < 2 * DK ? DK : BV;
    const float exp_alog = expf(A.a_log[h]);
    const float dtb = A.dt_bias[h];

    // ---- chunk inputs, loaded one chunk ahead
    float xp[TT];
    // The last wave holds no conv channel; its thread 64*7 + tt takes the
    // gate inputs of token tt and computes its gate scalars during the conv.
    constexpr int GATE0 = BLOCK_THREADS - 64;
    static_assert(NLC <= GATE0 && TT <= 64, "a gate thread per token of a chunk, in a wave without conv channels");
    float pa = 0.0f, pb = 0.0f;
    const int gsel = tid - GATE0;              // the token of this gate thread, if in 0..TT-1
    const int gtok = (wv << 2) + (lane >> 4);  // the token row of this thread's 16-lane row
    // Loads are unconditional (row and channel clamped into range) so all of
    // them stay in flight together; values past the sequence are zeroed.
    const int64_t gcl = gc >= 0 ? gc : 0;
    auto prefetch = [&](int t0) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int t = t0 + tt < T ? t0 + tt : T - 1;
            const float xv = to_f32(X[(int64_t)(r0 + t) * A.x_stride + gcl]);
            xp[tt] = (gc >= 0 && t0 + tt < T) ? xv : 0.0f;
        }
        const bool ok = gsel >= 0 && gsel < TT && t0 + gsel < T;
        const int t = ok ? t0 + gsel : T - 1;
        const int64_t row = (int64_t)(r0 + t) * A.ab_stride + h;
        const float av = to_f32(static_cast<const ActT*>(A.a)[row]);
        const float bv = to_f32(static_cast<const ActT*>(A.b)[row]);
        pa = ok ? av : 0.0f;
        pb = ok ? bv : 0.0f;
    };
    prefetch(0);

    // ---- state block into registers.  Issued after the small loads above:
    // loads complete in order, so the conv and gating of the first chunk only
    // wait for x, the window and the taps while the state is still in flight.
    StT* __restrict__ Sg = static_cast<StT*>(A.state) + (int64_t)page * A.state_page_stride +
                           (int64_t)h * DK * A.d_v + colbase;
    float s[CPL][R];
    if (init) {
        load_state<StT, DK, CPL>(Sg, A.d_v, s, tid);
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int m = 0; m < R; ++m) s[c][m] = 0.0f;
    }


    const int cg = lane_colgroup(tid);
    const bool writer = lane_rowgroup(tid) == 0;
    float* __restrict__ O = A.o + (int64_t)r0 * A.h_v * A.d_v + (int64_t)h * A.d_v + colbase + cg * CPL;
    const int64_t o_stride = (int64_t)A.h_v * A.d_v;
    bool my_last = false;

    // The barriers in the chunk loop order LDS only: a full workgroup barrier
    // would also wait for every outstanding global store and for the next
    // chunk's prefetch.  Each thread's own loads are waited for where their
    // registers are used.
    for (int t0 = 0; t0 < T; t0 += TT) {
        const int nt = (T - t0 < TT) ? (T - t0) : TT;
        // A1: conv + SiLU into LDS
        if (gc >= 0) {
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                if (tt < nt) {
                    const float x0 = xp[tt];
                    ydst[tt * yld] = silu_hw(conv4(w, xm3, xm2, xm1, x0));
                    xm3 = xm2;
                    xm2 = xm1;
                    xm1 = x0;
                }
            }
        } else if (gsel >= 0 && gsel < nt) {
            float eg, beta;
            gate_scalars(pa, pb, exp_alog, dtb, eg, beta);
            ssc[gsel * 4 + 0] = eg;
            ssc[gsel * 4 + 1] = beta;
        }
        lds_barrier();
        if (t0 == 0 && tid == 0)  // every window read of this workgroup has been consumed
            my_last = arrive_last(A.sync + (int64_t)page * A.h_k + ki, (uint32_t)(rr * nblk));
        // A2: gating, one 16-lane row per token
        if (gtok < nt) {
            const float kq = gate_qk<DK>(sq + gtok * DK, sk + gtok * DK, A.scale, A.eps, lane & 15);
            if ((lane & 15) == 0) ssc[gtok * 4 + 2] = kq;
        }
        lds_barrier();
        if (t0 + TT < T) prefetch(t0 + TT);
        // B: the recurrence, two tokens per trip with two operand sets, each
        // set's LDS reads issued one token ahead of its use
        struct Opnd { float k[R], q[R], v[CPL], eg, beta, kq; };
        auto operands = [&](Opnd& p, int tt) {
            lds_rows<R>(sk + tt * DK, tid, p.k);
            lds_rows<R>(sq + tt * DK, tid, p.q);
            lds_cols<CPL>(sv + tt * BV, tid, p.v);
            p.eg = ssc[tt * 4 + 0];
            p.beta = ssc[tt * 4 + 1];
            p.kq = ssc[tt * 4 + 2];
        };
        auto step = [&](const Opnd& p, int tt) {
            float o[CPL];
            delta_step<R, CPL>(s, p.k, p.q, p.v, p.eg, p.beta, p.kq, o);
            if (writer) {
                float* dst = O + (int64_t)(t0 + tt) * o_stride;
                if constexpr (CPL == 4) {
                    *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
                } else {
#pragma unroll
                    for (int c = 0; c < CPL; ++c) dst[c] = o[c];
                }
            }
        };
        Opnd pa_, pb_;
        operands(pa_, 0);
        for (int tt = 0; tt < nt; tt += 2) {
            operands(pb_, tt + 1 < nt ? tt + 1 : tt);
            step(pa_, tt);
            if (tt + 1 < nt) {
                operands(pa_, tt + 2 < nt ? tt + 2 : tt + 1);
                step(pb_, tt + 1);
            }
        }
        lds_barrier();
    }

    // ---- epilogue: state, then the rolled windows
    store_state<StT, DK, CPL>(Sg, A.d_v, s, tid);
    if (tid == 0) sh_last = my_last ? 1 : 0;
    __syncthreads();
    if (gc >= 0 && (lc >= 2 * DK || sh_last)) {
        win[0 * C + gc] = from_f32<ActT>(xm3);
        win[1 * C + gc] = from_f32<ActT>(xm2);
        win[2 * C + gc] = from_f32<ActT>(xm1);
    }
}

}  // namespace gdn
