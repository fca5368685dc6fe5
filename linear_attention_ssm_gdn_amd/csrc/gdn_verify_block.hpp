// gdn_verify_block.hpp -- one workgroup of the speculative verify step, as a
// device function of its block index, so that the verify kernel and the
// mixed-step kernel run the same code.
//
// The one-page design of "r9700-stack v0.2.4: one GDN state page per
// request" (section "What it does"): each request keeps one state
// checkpoint plus a record of the previous step's candidate rows (post-conv
// q|k|v and the a/b gate inputs) in two slots and a flag word (live slot,
// parity, done counter).  A step replays the accepted rows of the live slot
// into the checkpoint, stores it, then runs the new candidates from the
// stored value and records them in the other slot.  The comparison design
// keeps one state page per candidate instead.  Both designs run through this
// one kernel template and the same per-token functions, which is what makes
// them bit-identical.
//
// Grid: one workgroup per (request, value head, block of 32*CPL value
// columns), the lane layout of gdn_block.hpp.  Candidates per step <= 16.
//
// With CACHE, a request may also leave a committed prefix in a cache entry:
// the state after replayed record row j (the running state of the replay,
// rounded to the state dtype as a checkpoint is) and the conv window that
// ends at that row, buffer rows j .. j+W-2.  The slot design holds that
// state already, in slot j, and copies it; an empty live record caches the
// checkpoint as it is with window rows 0 .. W-2.
#pragma once

#include "gdn_block.hpp"
#include "gdn_kernels.h"
#include "../../include/gdn.h"

namespace gdn {

constexpr int VER_TT = 16;

template <typename ActT, typename StT, int DK, int CPL, int LAYOUT, bool CACHE = false>
__device__ __forceinline__ void verify_block(const VerifyArgs& A, const int block) {
    constexpr int TT = VER_TT;
    constexpr int R = DK / 16;
    constexpr int BV = 32 * CPL;
    constexpr int NLC = 2 * DK + BV;
    static_assert(TT <= 32, "one 16-lane row per token of a chunk");
    static_assert(NLC <= BLOCK_THREADS, "one conv channel per thread");
    __shared__ __attribute__((aligned(16))) float sq[TT * DK];
    __shared__ __attribute__((aligned(16))) float sk[TT * DK];
    __shared__ __attribute__((aligned(16))) float sv[TT * BV];
    __shared__ float ssc[TT * 4];
    __shared__ int sh_last;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nblk = A.d_v / BV;
    int bid = block;
    const int blk = bid % nblk;
    bid /= nblk;
    const int h = bid % A.h_v;
    const int req = bid / A.h_v;
    const int rr = A.h_v / A.h_k;
    const int ki = h / rr;
    const int colbase = blk * BV;
    const int64_t C = 2 * (int64_t)A.h_k * DK + (int64_t)A.h_v * A.d_v;
    const bool reporter = (h == 0 && blk == 0 && tid == 0);

    const int page = A.req_page[req];
    if (page < 0) return;
    if (page >= A.n_pages || page >= A.conv_n_pages) {
        if (reporter) set_err(A.err, GDN_DEVERR_PAGE);
        return;
    }
    uint8_t* pg = A.pages + (int64_t)page * A.page_bytes;
    gdn_spec_header* hdr = reinterpret_cast<gdn_spec_header*>(pg + A.header_off);
    // The header words, the step parity, the acceptance and the head's decay
    // parameters in one batch of scalar loads (uniform addresses; one wait
    // instead of a dependent vector load and wait each).  The live slot and
    // parity bits change only when the request's last workgroup flips the
    // flag, after every workgroup of the request has read it, and a launch
    // starts with the scalar cache clean.
    uint32_t hw[8];
    const uintptr_t par_addr = reinterpret_cast<uintptr_t>(A.step_parity + req);
    {
        const void* const ptrs[8] = {&hdr->flag, &hdr->n_rows[0], &hdr->n_rows[1], A.num_accepted + req,
                                     reinterpret_cast<const void*>(par_addr & ~(uintptr_t)3), A.a_log + h,
                                     A.dt_bias + h, A.req_page + req};
        sload_u32_n<8>(ptrs, hw);
    }
    const uint32_t flag = hw[0];
    const int L = (int)(flag & 1u);
    const int P = (int)((flag >> 1) & 1u);
    const int nr = (int)(L ? hw[2] : hw[1]);
    const int par = (int)((hw[4] >> ((par_addr & 3u) * 8u)) & 1u);
    if (par == P) {
        if (reporter) set_err(A.err, GDN_DEVERR_PARITY);
        return;
    }
    int acc = 0;
    if (nr > 0) {
        acc = (int32_t)hw[3];
        if (acc < 0 || acc >= nr || nr > A.n_spec + 1) {
            if (reporter) set_err(A.err, GDN_DEVERR_ACCEPTED);
            return;
        }
    }
    // ---- prefix cache: entry `cache_e` takes the committed prefix that ends
    // at replayed row `cache_j` (0 .. acc), or the checkpoint itself when the
    // live record holds no rows
    int cache_e = -1, cache_j = 0;
    if constexpr (CACHE) {
        cache_e = A.cache_entry[req];
        if (cache_e >= 0) {
            cache_j = nr > 0 ? A.cache_row[req] : 0;
            if (cache_e >= A.cache_state_n || cache_e >= A.cache_conv_n || cache_j < 0 || cache_j > acc) {
                if (reporter) set_err(A.err, GDN_DEVERR_CACHE);
                return;
            }
        }
    }
    const int n_replay = (LAYOUT == GDN_SPEC_ONEPAGE && nr > 0) ? acc + 1 : 0;
    const int nc = A.n_cand;

    // ---- done counter: the last workgroup of the request to get here flips the
    // flag at the end.  The counter stands for "this workgroup has read the
    // header", which is true now, so it is counted now; its result is read
    // once the state has arrived (issued before it, so already back).
    uint32_t done_before = 0;
    if (tid == 0) done_before = fetch_add_late(&hdr->flag, 256u);

    // ---- starting state: the checkpoint, or slot[acc]
    const int64_t head_elems = (int64_t)DK * A.d_v;
    StT* __restrict__ st_base = reinterpret_cast<StT*>(pg + A.state_off);
    StT* __restrict__ Sload = (LAYOUT == GDN_SPEC_ONEPAGE)
                                  ? st_base + (int64_t)h * head_elems + colbase
                                  : st_base + ((int64_t)acc * A.h_v + h) * head_elems + colbase;

    // ---- this thread's conv channel: weights, window rows acc..acc+2 of the conv buffer
    ActT* __restrict__ cbuf = static_cast<ActT*>(A.conv_base) + (int64_t)page * A.conv_page_stride;
    // Every small input is loaded raw first and converted only once all of
    // them are in flight, so they share one wait.
    const int lc = tid;
    int64_t gc = -1;
    float w[4] = {0.0f, 0.0f, 0.0f, 0.0f}, xw0 = 0.0f, xw1 = 0.0f, xw2 = 0.0f;
    if (lc < NLC)
        gc = lc < DK ? (int64_t)ki * DK + lc
           : lc < 2 * DK ? (int64_t)A.h_k * DK + (int64_t)ki * DK + (lc - DK)
           : 2 * (int64_t)A.h_k * DK + (int64_t)h * A.d_v + colbase + (lc - 2 * DK);
    // unconditional (threads without a channel read channel 0 and drop it):
    // a load inside a branch would take its conversion, and its wait, with it
    const int64_t gc0 = gc >= 0 ? gc : 0;
    ActT wr[4], xr0, xr1, xr2;
    {
        const ActT* Wc = static_cast<const ActT*>(A.conv_w) + gc0 * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) wr[e] = Wc[e];
        xr0 = cbuf[(int64_t)(acc + 0) * C + gc0];
        xr1 = cbuf[(int64_t)(acc + 1) * C + gc0];
        xr2 = cbuf[(int64_t)(acc + 2) * C + gc0];
    }
    // the cached prefix's window: buffer rows cache_j .. cache_j+2
    float cw0 = 0.0f, cw1 = 0.0f, cw2 = 0.0f;
    ActT cr0 = {}, cr1 = {}, cr2 = {};
    if constexpr (CACHE) {
        cr0 = cbuf[(int64_t)(cache_j + 0) * C + gc0];
        cr1 = cbuf[(int64_t)(cache_j + 1) * C + gc0];
        cr2 = cbuf[(int64_t)(cache_j + 2) * C + gc0];
    }
    float* ydst = lc < DK ? sq + qk_pos<DK>(lc) : lc < 2 * DK ? sk + qk_pos<DK>(lc - DK) : sv + (lc - 2 * DK);
    const int yld = lc < 2 * DK ? DK : BV;
    float exp_alog_v = expf(__uint_as_float(hw[5]));
    float dtb = __uint_as_float(hw[6]);
    asm volatile("" : "+v"(dtb));
    const float& exp_alog = exp_alog_v;

    // ---- LDS rows: when both the replayed rows and the candidates fit in
    // half of the TT token rows ("split"), the replayed rows take rows
    // 0 .. TT/2-1 and the candidates rows TT/2 .. TT-1, so the candidates'
    // conv and every gate run while the state is still in flight; otherwise
    // both start at row 0 and the candidates follow the replay.
    const bool split = (nc <= TT / 2) && (n_replay <= TT / 2);
    const int crow = split ? TT / 2 : 0;       // first candidate row
    const int gtok = (wv << 2) + (lane >> 4);  // the token row of this thread's 16-lane row
    const int cidx = gtok - crow;              // the candidate of that row (if any)

    // ---- small inputs first, then the state: loads complete in order, so
    // everything above the state is usable while the state is in flight
    float xp[TT];
    ActT xr[TT];
    float pa = 0.0f, pb = 0.0f;   // gate inputs of candidate cidx
    ActT par_raw = {}, pbr_raw = {};
    const bool cand_ok = cidx >= 0 && cidx < nc;
    const int64_t row_bytes = A.record_row_bytes;
    const int64_t rows_per_slot = A.n_spec + 1;
    float ra = 0.0f, rb = 0.0f;   // gate inputs of replayed row gtok
    const uint8_t* rec = pg + A.record_off + (int64_t)L * rows_per_slot * row_bytes;
    if (n_replay > 0) {
        const float* rrow = reinterpret_cast<const float*>(rec + (gtok < n_replay ? gtok : 0) * row_bytes);
        ra = rrow[C + h];
        rb = rrow[C + A.h_v + h];
    }
    // One-page: this lane's channel of the replayed rows.  With the split
    // layout (at most TT/2 rows) they come into registers, in flight with the
    // other small inputs and the state, and go to their LDS rows once the
    // state's loads are issued; otherwise row by row, here.  No direct
    // global->LDS loads: with one of those in flight the compiler waits for
    // every vector load before using any loaded register, which would put the
    // state's latency after the small inputs' instead of beside it.
    constexpr int RP = TT / 2;
    float rv[RP];
    const bool replay_regs = LAYOUT == GDN_SPEC_ONEPAGE && n_replay > 0 && split;
    if (replay_regs) {
        const int64_t gcl = gc >= 0 ? gc : 0;
#pragma unroll
        for (int i = 0; i < RP; ++i)
            rv[i] = reinterpret_cast<const float*>(rec + (int64_t)(i < n_replay ? i : 0) * row_bytes)[gcl];
    } else if (LAYOUT == GDN_SPEC_ONEPAGE && n_replay > 0) {
        if (lc < NLC)
            for (int i = 0; i < n_replay; ++i)
                ydst[i * yld] = reinterpret_cast<const float*>(rec + i * row_bytes)[gc];
    }
    {
        // unconditional loads (row and channel clamped into range) stay in flight
        // together; values past the candidates are zeroed
        const ActT* X = static_cast<const ActT*>(A.x);
        const int64_t gcl = gc >= 0 ? gc : 0;
        if (nc > 0) {
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const int t = tt < nc ? tt : nc - 1;
                xr[tt] = X[((int64_t)req * nc + t) * A.x_stride + gcl];
            }
            {
                const int64_t row = ((int64_t)req * nc + (cand_ok ? cidx : nc - 1)) * A.ab_stride + h;
                par_raw = static_cast<const ActT*>(A.a)[row];
                pbr_raw = static_cast<const ActT*>(A.b)[row];
            }
        } else {
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) xr[tt] = ActT{};
        }
    }
    // The state's loads are issued before any small input is used, so the two
    // latencies overlap: loads complete in order, and the waits for the small
    // inputs below leave the state's loads in flight.
    float s[CPL][R];
    load_state<StT, DK, CPL>(Sload, A.d_v, s, tid);
    asm volatile("" ::: "memory");
    // Every raw small input passes through an empty asm statement here, after
    // the state's loads: volatile asm keeps its place, so the compiler waits
    // for these values here (the state still in flight) rather than hoisting
    // their conversions, and its waits, above the state's loads.
    {
#pragma unroll
        for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(wr[e]));
        asm volatile("" : "+v"(xr0), "+v"(xr1), "+v"(xr2), "+v"(par_raw), "+v"(pbr_raw), "+v"(ra), "+v"(rb));
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) asm volatile("" : "+v"(xr[tt]));
        if constexpr (CACHE) asm volatile("" : "+v"(cr0), "+v"(cr1), "+v"(cr2));
        if (replay_regs) {
#pragma unroll
            for (int i = 0; i < RP; ++i) asm volatile("" : "+v"(rv[i]));
        }
    }
    {
        const bool has_ch = gc >= 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = has_ch ? to_f32(wr[e]) : 0.0f;
        xw0 = has_ch ? to_f32(xr0) : 0.0f;
        xw1 = has_ch ? to_f32(xr1) : 0.0f;
        xw2 = has_ch ? to_f32(xr2) : 0.0f;
        if constexpr (CACHE) {
            cw0 = (has_ch && cache_e >= 0) ? to_f32(cr0) : 0.0f;
            cw1 = (has_ch && cache_e >= 0) ? to_f32(cr1) : 0.0f;
            cw2 = (has_ch && cache_e >= 0) ? to_f32(cr2) : 0.0f;
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) xp[tt] = (gc >= 0 && tt < nc) ? to_f32(xr[tt]) : 0.0f;
        pa = cand_ok ? to_f32(par_raw) : 0.0f;
        pb = cand_ok ? to_f32(pbr_raw) : 0.0f;
        float exp_pin = exp_alog;
        asm volatile("" : "+v"(exp_pin), "+v"(pa), "+v"(pb), "+v"(ra), "+v"(rb), "+v"(xw0), "+v"(xw1), "+v"(xw2));
        asm volatile("" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
        if constexpr (CACHE) asm volatile("" : "+v"(cw0), "+v"(cw1), "+v"(cw2));
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) asm volatile("" : "+v"(xp[tt]));
        exp_alog_v = exp_pin;
    }
    if (replay_regs && gc >= 0) {
#pragma unroll
        for (int i = 0; i < RP; ++i)
            if (i < n_replay) ydst[i * yld] = rv[i];
    }

    StT* __restrict__ cst = nullptr;  // this workgroup's block of the cache entry's state
    if constexpr (CACHE) {
        if (cache_e >= 0) {
            cst = static_cast<StT*>(A.cache_state) + (int64_t)cache_e * A.cache_state_stride +
                  (int64_t)h * head_elems + colbase;
            if (LAYOUT == GDN_SPEC_SLOTS && cache_j != acc) {
                // slot cache_j holds the prefix's state; this workgroup owns its
                // columns in every slot, and no slot is written before this copy
                const StT* src = st_base + ((int64_t)cache_j * A.h_v + h) * head_elems + colbase;
                for (int i = tid; i < DK * BV; i += BLOCK_THREADS)
                    cst[(int64_t)(i / BV) * A.d_v + (i % BV)] = src[(int64_t)(i / BV) * A.d_v + (i % BV)];
            } else if (LAYOUT == GDN_SPEC_SLOTS || n_replay == 0) {
                // the loaded state is the prefix's state (stored values: exact)
                store_state<StT, DK, CPL>(cst, A.d_v, s, tid);
            }
        }
    }
    const int cache_at = (CACHE && LAYOUT == GDN_SPEC_ONEPAGE && cache_e >= 0 && n_replay > 0) ? cache_j : -1;

    // ---- candidates: conv (+ record) into rows crow.., then gating
    const bool qk_writer = (h == ki * rr) && (blk == 0);
    uint8_t* recw = pg + A.record_off + (int64_t)(1 - L) * rows_per_slot * row_bytes;
    auto cand_conv = [&]() {
        if (gc >= 0) {
            if (nc > 0) {
                const bool rec_this = (LAYOUT == GDN_SPEC_ONEPAGE) && (lc >= 2 * DK || qk_writer);
                float x3 = xw0, x2 = xw1, x1 = xw2;
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    if (tt < nc) {
                        const float x0 = xp[tt];
                        const float y = silu_hw(conv4(w, x3, x2, x1, x0));
                        ydst[(crow + tt) * yld] = y;
                        if (rec_this) reinterpret_cast<float*>(recw + tt * row_bytes)[gc] = y;
                        x3 = x2; x2 = x1; x1 = x0;
                    }
                }
            } else {
                // commit only: consume the window loads before arriving
                ydst[crow * yld] = xw0 + xw1 + xw2;
            }
        }
    };
    // the gates of this thread's token row: a replayed row or a candidate
    auto gates = [&](bool replay_rows, bool cand_rows) {
        if (replay_rows && gtok < n_replay) {
            (void)gate_qk<DK>(sq + gtok * DK, sk + gtok * DK, A.scale, A.eps, lane & 15);
            float eg, beta;
            gate_scalars(ra, rb, exp_alog, dtb, eg, beta);
            if ((lane & 15) == 0) {
                ssc[gtok * 4 + 0] = eg;
                ssc[gtok * 4 + 1] = beta;
            }
        }
        if (cand_rows && cidx >= 0 && cidx < nc) {
            const float kq = gate_qk<DK>(sq + gtok * DK, sk + gtok * DK, A.scale, A.eps, lane & 15);
            float eg, beta;
            gate_scalars(pa, pb, exp_alog, dtb, eg, beta);
            if ((lane & 15) == 0) {
                ssc[gtok * 4 + 0] = eg;
                ssc[gtok * 4 + 1] = beta;
                ssc[gtok * 4 + 2] = kq;
                if (LAYOUT == GDN_SPEC_ONEPAGE && blk == 0) {
                    float* rrow = reinterpret_cast<float*>(recw + cidx * row_bytes);
                    rrow[C + h] = pa;
                    rrow[C + A.h_v + h] = pb;
                }
            }
        }
    };
    if (split) {
        cand_conv();
        lds_barrier();
        gates(true, nc > 0);
        lds_barrier();
    } else if (LAYOUT == GDN_SPEC_ONEPAGE && n_replay > 0) {
        lds_barrier();
        gates(true, false);
        lds_barrier();
    }

    // ---- one-page: replay rows 0..acc of the live record, store the checkpoint
    if (LAYOUT == GDN_SPEC_ONEPAGE && n_replay > 0) {
        // two rows per trip with two operand sets, each set's LDS reads
        // issued one row ahead of its use
        struct ROpnd { float k[R], v[CPL], eg, beta; };
        auto roperands = [&](ROpnd& p, int tt) {
            lds_rows<R>(sk + tt * DK, tid, p.k);
            lds_cols<CPL>(sv + tt * BV, tid, p.v);
            p.eg = ssc[tt * 4 + 0];
            p.beta = ssc[tt * 4 + 1];
        };
        ROpnd r0, r1;
        roperands(r0, 0);
        for (int tt = 0; tt < n_replay; tt += 2) {
            roperands(r1, tt + 1 < n_replay ? tt + 1 : tt);
            delta_update<R, CPL>(s, r0.k, r0.v, r0.eg, r0.beta);
            if (CACHE && tt == cache_at) store_state<StT, DK, CPL>(cst, A.d_v, s, tid);
            if (tt + 1 < n_replay) {
                roperands(r0, tt + 2 < n_replay ? tt + 2 : tt + 1);
                delta_update<R, CPL>(s, r1.k, r1.v, r1.eg, r1.beta);
                if (CACHE && tt + 1 == cache_at) store_state<StT, DK, CPL>(cst, A.d_v, s, tid);
            }
        }
    }

    // ---- window arrival, before any store: the window values are in registers
    // (their loads were issued before the state's, which has been consumed),
    // and the barrier also separates the replay's LDS reads from the
    // candidates' writes.  The atomic's result is read at the end: reading it
    // is a wait on the in-order vector-memory counter, and by then the stores
    // issued after it no longer stand in anyone's way.
    asm volatile("" : "+v"(xw0), "+v"(xw1), "+v"(xw2), "+v"(done_before));
    lds_barrier();
    uint32_t arrived_before = 0;
    if (tid == 0) arrived_before = arrive(A.sync + (int64_t)page * A.h_k + ki);

    if (LAYOUT == GDN_SPEC_ONEPAGE) {
        // the checkpoint; continue from its stored (rounded) value
        store_state<StT, DK, CPL>(Sload, A.d_v, s, tid);
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int m = 0; m < R; ++m) s[c][m] = round_as<StT>(s[c][m]);
    }

    if (!split) {
        cand_conv();
        lds_barrier();
        if (nc > 0) gates(false, true);
        lds_barrier();
    }
    if (nc > 0) {
        const int cg = lane_colgroup(tid);
        const bool writer = lane_rowgroup(tid) == 0;
        float* __restrict__ O = A.o + (int64_t)req * nc * A.h_v * A.d_v + (int64_t)h * A.d_v + colbase + cg * CPL;
        const int64_t o_stride = (int64_t)A.h_v * A.d_v;
        // two tokens per trip with two operand sets, each set's LDS reads
        // issued one token ahead of its use
        struct Opnd { float k[R], q[R], v[CPL], eg, beta, kq; };
        auto operands = [&](Opnd& p, int tt) {
            const int r = crow + tt;
            lds_rows<R>(sk + r * DK, tid, p.k);
            lds_rows<R>(sq + r * DK, tid, p.q);
            lds_cols<CPL>(sv + r * BV, tid, p.v);
            p.eg = ssc[r * 4 + 0];
            p.beta = ssc[r * 4 + 1];
            p.kq = ssc[r * 4 + 2];
        };
        auto step = [&](const Opnd& p, int tt) {
            float o[CPL];
            // one-page: nothing reads the state after the last candidate (the
            // next step replays from the checkpoint), so its update is skipped
            delta_step<R, CPL>(s, p.k, p.q, p.v, p.eg, p.beta, p.kq, o,
                               !(LAYOUT == GDN_SPEC_ONEPAGE && tt == nc - 1));
            if (writer) {
                float* dst = O + (int64_t)tt * o_stride;
                if constexpr (CPL == 4) {
                    *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
                } else {
#pragma unroll
                    for (int c = 0; c < CPL; ++c) dst[c] = o[c];
                }
            }
            if (LAYOUT == GDN_SPEC_SLOTS)
                store_state<StT, DK, CPL>(st_base + ((int64_t)tt * A.h_v + h) * head_elems + colbase, A.d_v, s,
                                          tid);
        };
        Opnd p0, p1;
        operands(p0, 0);
        for (int tt = 0; tt < nc; tt += 2) {
            operands(p1, tt + 1 < nc ? tt + 1 : tt);
            step(p0, tt);
            if (tt + 1 < nc) {
                operands(p0, tt + 2 < nc ? tt + 2 : tt + 1);
                step(p1, tt + 1);
            }
        }
    } else if (LAYOUT == GDN_SPEC_SLOTS) {
        store_state<StT, DK, CPL>(st_base + (int64_t)h * head_elems + colbase, A.d_v, s, tid);
    }
    asm volatile("" : "+v"(arrived_before));  // keep the read of the result here, not at the atomic
    if (tid == 0)
        sh_last = arrived_last(A.sync + (int64_t)page * A.h_k + ki, arrived_before, (uint32_t)(rr * nblk)) ? 1 : 0;
    lds_barrier();

    // ---- conv buffer: [a'+1, a'+2, candidates] or [a', a'+1, a'+2]
    if (gc >= 0 && (lc >= 2 * DK || sh_last)) {
        if (nc > 0) {
            cbuf[0 * C + gc] = from_f32<ActT>(xw1);
            cbuf[1 * C + gc] = from_f32<ActT>(xw2);
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
                if (tt < nc) cbuf[(int64_t)(2 + tt) * C + gc] = from_f32<ActT>(xp[tt]);
        } else {
            cbuf[0 * C + gc] = from_f32<ActT>(xw0);
            cbuf[1 * C + gc] = from_f32<ActT>(xw1);
            cbuf[2 * C + gc] = from_f32<ActT>(xw2);
        }
    }

    // ---- the cached prefix's window (v channels by every workgroup, q/k
    // channels by the key head's recording workgroup)
    if constexpr (CACHE) {
        if (cache_e >= 0 && gc >= 0 && (lc >= 2 * DK || qk_writer)) {
            ActT* __restrict__ cc = static_cast<ActT*>(A.cache_conv) + (int64_t)cache_e * A.cache_conv_stride;
            cc[0 * C + gc] = from_f32<ActT>(cw0);
            cc[1 * C + gc] = from_f32<ActT>(cw1);
            cc[2 * C + gc] = from_f32<ActT>(cw2);
        }
    }

    // ---- the last workgroup of the request to count itself flips the flag.
    // Every workgroup of the request read the header before counting, so the
    // last one may rewrite it; relaxed for the reason given at arrive_last.
    if (tid == 0) {
        const uint32_t total = (uint32_t)(A.h_v * nblk);
        if ((done_before >> 8) + 1u == total) {
            hdr->n_rows[1 - L] = (uint32_t)nc;
            hdr->accepted = (uint32_t)acc;
            __hip_atomic_store(&hdr->flag, (uint32_t)((1 - L) | (par << 1)), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace gdn
