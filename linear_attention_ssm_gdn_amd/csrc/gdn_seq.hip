// gdn_seq.hip -- token-by-token GDN layer core: conv + SiLU + gating + gated
// delta rule fused in one launch (decode is T = 1).  The workgroup of the
// general kernel is gdn_seq_block.hpp; this file holds its launcher and the
// persistent short-sequence (decode) kernel.
#include "gdn_seq_block.hpp"

namespace gdn {

template <typename ActT, typename StT, int DK, int CPL, int TT>
__global__ __launch_bounds__(BLOCK_THREADS) void k_gdn_seq(const SeqArgs A) {
    seq_block<ActT, StT, DK, CPL, TT>(A, blockIdx.x);
}

// Persistent variant for short sequences (decode): the grid holds only as
// many workgroups as stay resident, and workgroup b walks the items (sequence,
// head, 32 CPL-column block) b, b + grid, b + 2 grid, ...  While item i is
// convolved, gated, updated and stored from registers, everything item i+1
// reads -- its state block, x row, gate inputs, taps and conv window -- is
// already streaming into LDS by direct global->LDS loads, which hold no
// registers while in flight.  HBM then sees the reads of the next item
// overlap the writes of the current one, instead of every resident
// workgroup loading, computing and storing in lockstep.
//
// Waits: the vector-memory counter completes in order, so any wait for a
// load issued after the prefetch would also wait for the prefetch.  Inside
// an item the kernel therefore issues no vector load whose result it needs
// early: per-item metadata comes through scalar loads and barriers order LDS
// only.  The one wait per item sits after its last token and before its
// state stores, so it covers the prefetch and the arrival but never the
// store acknowledgements.  Items longer than one token (not the decode case)
// load their later tokens synchronously.
//
// The arithmetic per column is the token-by-token kernel's (same conv,
// gate_qk, gate_scalars and delta_step), so the two agree bit for bit.
template <typename ActT, typename StT, int DK, int CPL>
__global__ __launch_bounds__(BLOCK_THREADS) __attribute__((amdgpu_waves_per_eu(4))) void k_gdn_seq_stream(
    const SeqArgs A) {
    constexpr int R = DK / 16, BV = 32 * CPL;
    constexpr int NLC = 2 * DK + BV;       // conv channels of an item: q, k (key head), v (block)
    constexpr int SL = LDS_ELEM_SLOT;      // bytes per lane slot of a staged element
    using Stage = StateStage<StT, DK, CPL>;
    static_assert(NLC <= BLOCK_THREADS && NLC % 64 == 0, "whole waves of conv channels");
    static_assert(NLC <= 7 * 64, "wave 7 holds no conv channel: it takes the gate scalars");
    // Staged small inputs: fields of NLC slots (taps 0..3, window rows 0..2,
    // x), then 64 slots each of a and b for wave 0.
    constexpr int F_TAP = 0, F_WIN = 4, F_X = 7, N_CH_FIELDS = 8;
    constexpr int AB_OFF = N_CH_FIELDS * NLC * SL;
    __shared__ __attribute__((aligned(16))) unsigned char sin[AB_OFF + 2 * 64 * SL];
    __shared__ __attribute__((aligned(16))) unsigned char stage[Stage::BYTES];
    __shared__ __attribute__((aligned(16))) float sq[DK];
    __shared__ __attribute__((aligned(16))) float sk[DK];
    __shared__ __attribute__((aligned(16))) float sv[BV];
    __shared__ float ssc[4];
    __shared__ int sh_last;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // Per-lane offsets recomputed at each use (cheap integer work) rather than
    // hoisted out of the item loop, where they would hold registers for its
    // whole length.
    auto fresh_tid = [&]() {
        int t = tid;
        asm volatile("" : "+v"(t));
        return t;
    };
    const int nblk = A.d_v / BV;
    const int n_items = A.n_seqs * A.h_v * nblk;
    const int rr = A.h_v / A.h_k;
    const int64_t C = 2 * (int64_t)A.h_k * DK + (int64_t)A.h_v * A.d_v;
    const ActT* __restrict__ X = static_cast<const ActT*>(A.x);
    const ActT* __restrict__ Ag = static_cast<const ActT*>(A.a);
    const ActT* __restrict__ Bg = static_cast<const ActT*>(A.b);
    const int lc = tid;
    const bool has_ch = lc < NLC;  // whole waves
    const int cg = lane_colgroup(tid);
    const bool writer = lane_rowgroup(tid) == 0;
    const int64_t o_stride = (int64_t)A.h_v * A.d_v;
    float* ydst = lc < DK ? sq + qk_pos<DK>(lc) : lc < 2 * DK ? sk + qk_pos<DK>(lc - DK) : sv + (lc - 2 * DK);

    struct Item {
        int h, colbase, page, r0, T;
        bool init;
        float a_log, dt_bias;
    };
    // Decode item j; false when it has nothing to compute (unused page, empty
    // sequence or a reported error).  Every field is workgroup-uniform; the
    // metadata comes in one batch of scalar loads.
    auto resolve = [&](int j, Item& it) -> bool {
        const int blk = j % nblk;
        const int hs = j / nblk;
        const int seq = hs / A.h_v;
        it.h = hs % A.h_v;
        it.colbase = blk * BV;
        const uintptr_t ia = reinterpret_cast<uintptr_t>(A.has_init ? A.has_init + seq : nullptr);
        const void* const ptrs[6] = {A.page_idx + seq, A.cu + seq, A.cu + seq + 1,
                                     A.has_init ? reinterpret_cast<const void*>(ia & ~(uintptr_t)3)
                                                : static_cast<const void*>(A.cu + seq),
                                     A.a_log + it.h, A.dt_bias + it.h};
        uint32_t m[6];
        sload_u32_n<6>(ptrs, m);
        it.page = (int32_t)m[0];
        const int r0 = (int32_t)m[1], r1 = (int32_t)m[2];
        if (it.page < 0) return false;
        if (it.page >= A.conv_n_pages || it.page >= A.state_n_pages) {
            if (tid == 0 && it.h == 0 && blk == 0) set_err(A.err, GDN_DEVERR_PAGE);
            return false;
        }
        if (r0 < 0 || r1 < r0 || (int64_t)r1 > A.n_rows) {
            if (tid == 0 && it.h == 0 && blk == 0) set_err(A.err, GDN_DEVERR_BATCH);
            return false;
        }
        it.r0 = r0;
        it.T = r1 - r0;
        if (it.T == 0) return false;
        it.init = A.has_init ? (((m[3] >> ((ia & 3u) * 8u)) & 0xffu) != 0) : true;
        it.a_log = __uint_as_float(m[4]);
        it.dt_bias = __uint_as_float(m[5]);
        return true;
    };
    // This thread's conv channel of an item (meaningful when has_ch).
    auto channel = [&](const Item& it) -> int64_t {
        const int ki = it.h / rr;
        return lc < DK ? (int64_t)ki * DK + lc
             : lc < 2 * DK ? (int64_t)A.h_k * DK + (int64_t)ki * DK + (lc - DK)
             : 2 * (int64_t)A.h_k * DK + (int64_t)it.h * A.d_v + it.colbase + (lc - 2 * DK);
    };
    // Issue every load of a resolved item into LDS (token 0's inputs; the
    // state block last).
    auto fetch = [&](const Item& it) {
        if (has_ch) {
            const int64_t gc = channel(it);
            unsigned char* wb = sin + (tid & ~63) * SL;
            const ActT* Wc = static_cast<const ActT*>(A.conv_w) + gc * 4;
            const ActT* win = static_cast<const ActT*>(A.conv_base) + (int64_t)it.page * A.conv_page_stride + gc;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                load_lds_elem(Wc + e, wb + (F_TAP + e) * NLC * SL);
#pragma unroll
            for (int r = 0; r < 3; ++r)
                load_lds_elem(win + r * C, wb + (F_WIN + r) * NLC * SL);
            load_lds_elem(X + (int64_t)it.r0 * A.x_stride + gc, wb + F_X * NLC * SL);
        }
        if (wv == 0) {
            const int64_t row = (int64_t)it.r0 * A.ab_stride + it.h;
            load_lds_elem(Ag + row, sin + AB_OFF);
            load_lds_elem(Bg + row, sin + AB_OFF + 64 * SL);
        }
        if (it.init) {
            const StT* Sg = static_cast<const StT*>(A.state) + (int64_t)it.page * A.state_page_stride +
                            (int64_t)it.h * DK * A.d_v + it.colbase;
            Stage::fetch(Sg, A.d_v, stage, fresh_tid());
        }
    };
    auto staged = [&](int field) -> float {
        return to_f32(*reinterpret_cast<const ActT*>(sin + (field * NLC + lc) * SL));
    };

    // In the iteration that processes item i the workgroup also issues item
    // i+1's loads and resolves item i+2's metadata, under the wait for those
    // loads.  Workgroup b takes items b, b+g and b+2g; when there are more,
    // the rest are handed out from the work counter that follows the
    // arrival counters: a workgroup claims item i+3 in the iteration of item
    // i (the claim returns under the same wait), so workgroups whose loads
    // are served faster take more items.  Each workgroup makes exactly one
    // claim past the end; the maker of the last claim of all returns the
    // counter to zero.
    const int g = gridDim.x;
    auto clamp_item = [&](int64_t j) -> int { return j < n_items ? (int)j : n_items; };
    const bool dyn = (int64_t)n_items > 3 * (int64_t)g;
    uint32_t* work = A.sync + (int64_t)A.conv_n_pages * A.h_k;
    __shared__ int sh_claim;
    int cur_j = blockIdx.x, nxt_j = clamp_item((int64_t)blockIdx.x + g);
    int nn_j = clamp_item((int64_t)blockIdx.x + 2 * (int64_t)g);
    Item cur{}, nxt{};
    bool cur_ok = cur_j < n_items && resolve(cur_j, cur);
    if (cur_ok) fetch(cur);
    bool pending = cur_ok;  // staged loads not yet waited for
    bool nxt_ok = nxt_j < n_items && resolve(nxt_j, nxt);

    while (cur_j < n_items) {
        if (pending) wait_vmem();
        lds_barrier();  // staged by other waves too; also orders the reuse of sh_last
        // ---- the current item's inputs, out of LDS
        float w[4] = {0.0f, 0.0f, 0.0f, 0.0f}, xm3 = 0.0f, xm2 = 0.0f, xm1 = 0.0f, x0 = 0.0f, pa = 0.0f, pb = 0.0f;
        float s[CPL][R];
        if (cur_ok) {
            if (has_ch) {
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = staged(F_TAP + e);
                if (cur.init) {
                    xm3 = staged(F_WIN + 0);
                    xm2 = staged(F_WIN + 1);
                    xm1 = staged(F_WIN + 2);
                }
                x0 = staged(F_X);
            }
            if (wv == 7) {  // the gate scalars' wave (it holds no conv channel)
                pa = to_f32(*reinterpret_cast<const ActT*>(sin + AB_OFF + lane * SL));
                pb = to_f32(*reinterpret_cast<const ActT*>(sin + AB_OFF + (64 + lane) * SL));
            }
        }
        if (cur_ok && cur.init) {
            Stage::read(stage, fresh_tid(), s);
        } else {
#pragma unroll
            for (int c = 0; c < CPL; ++c)
#pragma unroll
                for (int m = 0; m < R; ++m) s[c][m] = 0.0f;
        }
        // ---- the next item's loads, once every wave has read the stage
        if (nxt_ok) {
            lds_barrier();
            fetch(nxt);
        }
        pending = nxt_ok;
        // ---- claim the item after item i+2 (issued after the loads above, so
        // the wait for them covers its result)
        const bool claiming = dyn && nn_j < n_items;
        uint32_t claimed = 0;
        if (claiming && tid == 0) claimed = fetch_add_late(work, 1u);

        // ---- the current item, one token at a time
        const int64_t gc = channel(cur);
        uint32_t* sync = A.sync + (int64_t)cur.page * A.h_k + cur.h / rr;
        uint32_t arrived_before = 0;
        if (cur_ok) {
            const float exp_alog = expf(cur.a_log);
            float* __restrict__ O =
                A.o + (int64_t)cur.r0 * o_stride + (int64_t)cur.h * A.d_v + cur.colbase + cg * CPL;
            for (int t = 0; t < cur.T; ++t) {
                if (t > 0) {  // later tokens of a longer item: plain loads
                    const int64_t row = (int64_t)(cur.r0 + t);
                    if (has_ch) x0 = to_f32(X[row * A.x_stride + gc]);
                    if (wv == 7) {
                        pa = to_f32(Ag[row * A.ab_stride + cur.h]);
                        pb = to_f32(Bg[row * A.ab_stride + cur.h]);
                    }
                }
                if (has_ch) {
                    *ydst = silu_hw(conv4(w, xm3, xm2, xm1, x0));
                    xm3 = xm2;
                    xm2 = xm1;
                    xm1 = x0;
                }
                if (wv == 7) {  // the gate scalars alongside the conv
                    float eg, beta;
                    gate_scalars(pa, pb, exp_alog, cur.dt_bias, eg, beta);
                    if (lane == 0) {
                        ssc[0] = eg;
                        ssc[1] = beta;
                    }
                }
                lds_barrier();
                if (t == 0 && tid == 0)  // every window read of this item has been consumed
                    arrived_before = arrive(sync);
                if (tid < 16) {
                    const float kq = gate_qk<DK>(sq, sk, A.scale, A.eps, tid);
                    if (tid == 0) ssc[2] = kq;
                }
                lds_barrier();
                {
                    float k[R], q[R], v[CPL], o[CPL];
                    lds_rows<R>(sk, tid, k);
                    lds_rows<R>(sq, tid, q);
                    lds_cols<CPL>(sv, tid, v);
                    delta_step<R, CPL>(s, k, q, v, ssc[0], ssc[1], ssc[2], o);
                    if (writer) store_cols<CPL>(O + (int64_t)t * o_stride, o);
                }
                lds_barrier();
            }
        }

        // ---- item i+2's metadata, under the wait for item i+1's loads
        Item nn{};
        const bool nn_ok = nn_j < n_items && resolve(nn_j, nn);

        if (cur_ok || claiming) {
            // This wave's staged loads of the next item (and the arrival and
            // the claim) have landed once this returns; the barrier below
            // makes that true for every wave.
            wait_vmem();
            pending = false;
        }
        if (tid == 0) {
            int nnn_j = clamp_item((int64_t)nn_j + g);
            if (dyn) {
                nnn_j = n_items;
                if (claiming) {
                    asm volatile("" : "+v"(claimed) : : "memory");
                    nnn_j = clamp_item(3 * (int64_t)g + claimed);
                    if ((int64_t)claimed == (int64_t)n_items - 2 * (int64_t)g - 1)  // the last claim of all
                        __hip_atomic_store(work, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            sh_claim = nnn_j;
        }
        // The arrival's result is taken here, on every path and before the
        // state stores are issued, so no wait covers the stores' acknowledgements.
        asm volatile("" : "+v"(arrived_before) : : "memory");
        const bool last = tid == 0 && cur_ok && arrived_last(sync, arrived_before, (uint32_t)(rr * nblk));
        if (cur_ok) {
            StT* __restrict__ Sg = static_cast<StT*>(A.state) + (int64_t)cur.page * A.state_page_stride +
                                   (int64_t)cur.h * DK * A.d_v + cur.colbase;
            store_state<StT, DK, CPL>(Sg, A.d_v, s, fresh_tid());
        }
        if (tid == 0) sh_last = last ? 1 : 0;
        lds_barrier();
        if (cur_ok && has_ch && (lc >= 2 * DK || sh_last)) {
            ActT* win = static_cast<ActT*>(A.conv_base) + (int64_t)cur.page * A.conv_page_stride;
            win[0 * C + gc] = from_f32<ActT>(xm3);
            win[1 * C + gc] = from_f32<ActT>(xm2);
            win[2 * C + gc] = from_f32<ActT>(xm1);
        }
        cur_j = nxt_j;
        cur = nxt;
        cur_ok = nxt_ok;
        nxt_j = nn_j;
        nxt = nn;
        nxt_ok = nn_ok;
        nn_j = sh_claim;  // written before the barrier above; rewritten only after the next one
    }
}

// Compute units of the current device and the workgroups of `kernel` that
// stay resident on one of them (cached per device; the figures only size the
// grid, never the results).  Returns false if the runtime cannot tell.
constexpr int MAX_CACHED_DEVICES = 64;
static bool resident_shape(const void* kernel, int (&cache)[MAX_CACHED_DEVICES][2], int& ncu, int& per_cu) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    if (dev >= 0 && dev < MAX_CACHED_DEVICES) {
        const int c = __atomic_load_n(&cache[dev][0], __ATOMIC_RELAXED);
        const int p = __atomic_load_n(&cache[dev][1], __ATOMIC_RELAXED);
        if (c > 0 && p > 0) {
            ncu = c;
            per_cu = p;
            return true;
        }
    }
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, BLOCK_THREADS, 0) != hipSuccess)
        return false;
    if (ncu <= 0) ncu = 1;
    if (per_cu <= 0) per_cu = 1;
    if (dev >= 0 && dev < MAX_CACHED_DEVICES) {
        __atomic_store_n(&cache[dev][0], ncu, __ATOMIC_RELAXED);
        __atomic_store_n(&cache[dev][1], per_cu, __ATOMIC_RELAXED);
    }
    return true;
}

template <typename ActT, typename StT, int DK, int CPL>
static hipError_t launch_seq_stream(const SeqArgs& a, hipStream_t s) {
    static int cache[MAX_CACHED_DEVICES][2] = {};
    const int64_t items = (int64_t)a.n_seqs * a.h_v * (a.d_v / (32 * CPL));
    if (items == 0) return hipSuccess;
    if (items > 0x40000000) return hipErrorInvalidValue;  // item indices up to 2 items stay in int
    const void* k = reinterpret_cast<const void*>(&k_gdn_seq_stream<ActT, StT, DK, CPL>);
    int ncu = 0, per_cu = 0;
    if (!resident_shape(k, cache, ncu, per_cu)) return hipErrorInvalidValue;
    // More than four items per compute unit: one workgroup per CU (the
    // second resident workgroup of a CU starts its first item only after the
    // first one's 64 KiB have come in, and ends that much later; measured at
    // 40-128 sequences x 32 heads: 46.2 against 47.0 us at 5 items per CU,
    // 65.5 against 67.4 at 8).  Up to four, every resident slot (at 4 items
    // per CU: 38.7 against 40.4 us).
    const int64_t slots = items > 4 * (int64_t)ncu ? ncu : (int64_t)ncu * per_cu;
    const int grid = items < slots ? (int)items : (int)slots;
    hipLaunchKernelGGL((k_gdn_seq_stream<ActT, StT, DK, CPL>), dim3(grid), dim3(BLOCK_THREADS), 0, s, a);
    return hipGetLastError();
}

template <typename ActT, typename StT, int DK, int CPL, int TT>
static hipError_t launch_seq_t(const SeqArgs& a, hipStream_t s) {
    const int nblk = a.d_v / (32 * CPL);
    const int64_t grid = (int64_t)a.n_seqs * a.h_v * nblk;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_gdn_seq<ActT, StT, DK, CPL, TT>), dim3((unsigned)grid), dim3(BLOCK_THREADS), 0, s, a);
    return hipGetLastError();
}

// Few tokens per sequence (decode): the streaming persistent kernel on 128-
// (else 64-) column items.  Longer sequences: 32 columns per workgroup,
// the shortest per-token critical path.
template <typename ActT, typename StT, int DK>
static hipError_t launch_seq_shape(const SeqArgs& a, int max_seqlen, hipStream_t s) {
    if (max_seqlen >= 1 && max_seqlen <= 4) {
        // 128-column items where the head allows them: at the 64 x 1 decode
        // shape 64-column items measured slower (77.0 against 67.5 us per
        // step; each item's conv, gating and barrier chain is a fixed cost).
        if (a.d_v % 128 == 0) return launch_seq_stream<ActT, StT, DK, 4>(a, s);
        if (a.d_v % 64 == 0) return launch_seq_stream<ActT, StT, DK, 2>(a, s);
    }
    return launch_seq_t<ActT, StT, DK, 1, 16>(a, s);
}

template <typename ActT, typename StT>
static hipError_t launch_seq_dk(const SeqArgs& a, int d_k, int max_seqlen, hipStream_t s) {
    switch (d_k) {
        case 32: return launch_seq_shape<ActT, StT, 32>(a, max_seqlen, s);
        case 64: return launch_seq_shape<ActT, StT, 64>(a, max_seqlen, s);
        case 128: return launch_seq_shape<ActT, StT, 128>(a, max_seqlen, s);
        default: return hipErrorInvalidValue;
    }
}

bool seq_supported(int d_k, int d_v) {
    return (d_k == 32 || d_k == 64 || d_k == 128) && d_v > 0 && d_v % 32 == 0;
}

hipError_t launch_seq(const SeqArgs& a, int d_k, int act_dtype, int state_dtype, int max_seqlen, hipStream_t s) {
    if (act_dtype == GDN_BF16) {
        return state_dtype == GDN_BF16 ? launch_seq_dk<bf16_t, bf16_t>(a, d_k, max_seqlen, s)
                                       : launch_seq_dk<bf16_t, float>(a, d_k, max_seqlen, s);
    }
    return state_dtype == GDN_BF16 ? launch_seq_dk<float, bf16_t>(a, d_k, max_seqlen, s)
                                   : launch_seq_dk<float, float>(a, d_k, max_seqlen, s);
}

}  // namespace gdn
