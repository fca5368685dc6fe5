// gdn_chunked.hip -- chunked WY/UT prefill of the GDN layer core (Gated
// DeltaNet part (c), chunked form) on bf16 matrix cores with fp32
// accumulation, conv + SiLU + gating fused in.
//
// Grid: one workgroup of 4 waves per (sequence, value head h, block of 64
// value columns).  Wave w owns the 16-column tile w of the block; its share
// of the fp32 state S (128 x 16) lives in MFMA accumulator registers for the
// whole sequence.  Chunks of C = 64 tokens run in order.  Per chunk, with
// chunk-local cumulative decay G and start state S0:
//   P1  conv + SiLU, one channel per thread; raw post-conv q and k go to LDS
//       as bf16 hi/lo pairs, token-major (for contractions over d) and k also
//       transposed (for contractions over tokens); v transposed.
//   P2  per-token norms (16 lanes per token), k.q, gates, the scan of G.  The
//       L2 norms stay per-token factors rq (with the output scale) and rk,
//       folded into every product below instead of rescaling the arrays.
//   P3  Q K^T (three-pass hi/lo) and K K^T on MFMA; P_ts = rq_t rk_s (q_t.k_s)
//       e^{G_t-G_s} and A_ts = beta_t rk_t rk_s (k_t.k_s) e^{G_t-G_s} for s < t,
//       masked before the exponential.
//   P4  UT transform T = (I + A)^{-1}: 16x16 diagonal blocks by the doubling
//       identity (I+N)^{-1} = (I-N)(I+N^2)(I+N^4)(I+N^8) with both N-powers
//       and their transposes in registers, then the three block sub-diagonals.
//   P5  W = T diag(beta e^G rk) K (exact diagonal + MFMA for T - I).
//   P6  U = T diag(beta) V; D = U - W S; O = diag(e^G rq) Q S + diag(k.q) D +
//       P D; S <- e^{G_last} S + K^T diag(rk e^{G_last-G}) D, the last row of
//       the chunk as an exact fp32 outer product.
// Rounding points were chosen by emulating the error against the fp64
// recurrence: single bf16 roundings that multiply a weight-one term (the
// diagonal of T and of Q K^T, the last row of the state update) would cost up
// to 2^-8 each, so those terms stay fp32, and P, D and K take hi/lo splits in
// the products where they dominate.
#include "gdn_block.hpp"
#include "gdn_kernels.h"
#include "../../include/gdn.h"

namespace gdn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int DK = 128;        // key head dim
constexpr int CH = 64;         // chunk length
constexpr int BVC = 64;        // value columns per workgroup
constexpr int NTH = 256;       // threads per workgroup
constexpr int LQK = 136;       // bf16 row stride of token-major [64][128] arrays
constexpr int LT = 72;         // bf16 row stride of [..][64] arrays
constexpr int LAF = 68;        // fp32 row stride of A [64][64]

// LDS arena (bytes)
constexpr int SZ_TOK = CH * LQK * 2;          // 17408
constexpr int SZ_REG = 18432;                  // regions that later hold two [64][72] bf16 arrays
constexpr int OFF_QH = 0;
constexpr int OFF_KH = OFF_QH + SZ_TOK;        // then T (first half) + LTbg (second half)
constexpr int OFF_QL = OFF_KH + SZ_REG;        // then A (fp32), then W
constexpr int OFF_KL = OFF_QL + SZ_REG;        // then LTb
constexpr int OFF_KTH = OFF_KL + SZ_REG;       // [128][72]
constexpr int OFF_KTL = OFF_KTH + DK * LT * 2;
constexpr int OFF_VTH = OFF_KTL + DK * LT * 2; // [64][72]
constexpr int OFF_VTL = OFF_VTH + BVC * LT * 2;
constexpr int OFF_PH = OFF_VTL + BVC * LT * 2; // [64][72]
constexpr int OFF_PL = OFF_PH + CH * LT * 2;
constexpr int OFF_SC = OFF_PL + CH * LT * 2;   // 8 x [64] fp32 scalars
constexpr int OFF_KLAST = OFF_SC + 8 * CH * 4; // [128] fp32
constexpr int OFF_WV = OFF_KLAST + DK * 4;       // [64][4] fp32 v-channel conv taps
constexpr int LDS_BYTES = OFF_WV + BVC * 4 * 4;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert(CH * LAF * 4 <= SZ_REG && CH * LQK * 2 <= SZ_REG, "region sizes");

// scalar rows in the SC block
enum { SC_RQ = 0, SC_RK, SC_KQ, SC_BETA, SC_GAM, SC_BGR, SC_WDR, SC_G };

__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Operand loaders.  Lane l of a 16x16x32 product reads 8 consecutive
// K-elements of row (l & 15); a 16x16x16 product reads 4 at offset 4*(l>>4).
__device__ __forceinline__ bf16x8 ld8(const __bf16* base, int ld, int row, int col) {
    return *reinterpret_cast<const bf16x8*>(base + row * ld + col);
}
__device__ __forceinline__ bf16x4 ld4(const __bf16* base, int ld, int row, int col) {
    return *reinterpret_cast<const bf16x4*>(base + row * ld + col);
}
__device__ __forceinline__ bf16x4 to_bf4(float a, float b, float c, float d) {
    bf16x4 r;
    r[0] = (__bf16)a; r[1] = (__bf16)b; r[2] = (__bf16)c; r[3] = (__bf16)d;
    return r;
}
__device__ __forceinline__ bf16x4 to_bf4(const f32x4& v) { return to_bf4(v[0], v[1], v[2], v[3]); }
__device__ __forceinline__ void split4(const f32x4& v, bf16x4& hi, bf16x4& lo) {
    hi = to_bf4(v);
    lo = to_bf4(v[0] - (float)hi[0], v[1] - (float)hi[1], v[2] - (float)hi[2], v[3] - (float)hi[3]);
}
__device__ __forceinline__ float silu_fast(float z) { return __fdividef(z, 1.0f + __expf(-z)); }

template <typename ActT, typename StT>
__global__ __launch_bounds__(NTH) void k_gdn_chunk(const ChunkArgs A) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    __shared__ int sh_last;
    __bf16* Qh = reinterpret_cast<__bf16*>(lds + OFF_QH);
    __bf16* Kh = reinterpret_cast<__bf16*>(lds + OFF_KH);
    __bf16* Ql = reinterpret_cast<__bf16*>(lds + OFF_QL);
    __bf16* Kl = reinterpret_cast<__bf16*>(lds + OFF_KL);
    __bf16* KTh = reinterpret_cast<__bf16*>(lds + OFF_KTH);
    __bf16* KTl = reinterpret_cast<__bf16*>(lds + OFF_KTL);
    __bf16* VTh = reinterpret_cast<__bf16*>(lds + OFF_VTH);
    __bf16* VTl = reinterpret_cast<__bf16*>(lds + OFF_VTL);
    __bf16* Ph = reinterpret_cast<__bf16*>(lds + OFF_PH);
    __bf16* Pl = reinterpret_cast<__bf16*>(lds + OFF_PL);
    float* Af = reinterpret_cast<float*>(lds + OFF_QL);                    // after P3
    __bf16* Tm = reinterpret_cast<__bf16*>(lds + OFF_KH);                  // after P3
    __bf16* LTbg = reinterpret_cast<__bf16*>(lds + OFF_KH + CH * LT * 2);  // after P4
    __bf16* LTb = reinterpret_cast<__bf16*>(lds + OFF_KL);                 // after P4
    __bf16* Wm = reinterpret_cast<__bf16*>(lds + OFF_QL);                  // after P5
    float* sc = reinterpret_cast<float*>(lds + OFF_SC);
    float* klast = reinterpret_cast<float*>(lds + OFF_KLAST);
    float* wv4 = reinterpret_cast<float*>(lds + OFF_WV);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;  // MFMA row-in-tile / lane group
    const int nblk = A.d_v / BVC;
    int bid = blockIdx.x;
    const int blk = bid % nblk;
    bid /= nblk;
    const int h = bid % A.h_v;
    const int seq = bid / A.h_v;
    const int rr = A.h_v / A.h_k;
    const int ki = h / rr;
    const int colbase = blk * BVC;
    const int64_t C = 2 * (int64_t)A.h_k * DK + (int64_t)A.h_v * A.d_v;

    const int page = A.page_idx[seq];
    const int r0 = A.cu[seq], r1 = A.cu[seq + 1];
    if (page < 0) return;
    if (page >= A.conv_n_pages || page >= A.state_n_pages) {
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

    // ---- state: wave w holds S[16 dt + 4 lg + j][16 w + lr], dt = 0..7
    StT* __restrict__ Sg = static_cast<StT*>(A.state) + (int64_t)page * A.state_page_stride +
                           (int64_t)h * DK * A.d_v + colbase + 16 * wv + lr;
    f32x4 s[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s[dt][j] = init ? to_f32(Sg[(int64_t)(16 * dt + 4 * lg + j) * A.d_v]) : 0.0f;

    // ---- conv channels: q/k channel `tid`, and v channel `tid` for tid < 64
    const ActT* __restrict__ X = static_cast<const ActT*>(A.x);
    ActT* __restrict__ win = static_cast<ActT*>(A.conv_base) + (int64_t)page * A.conv_page_stride;
    const ActT* Wc = static_cast<const ActT*>(A.conv_w);
    const bool is_q = tid < DK;
    const int64_t gq = is_q ? (int64_t)ki * DK + tid : (int64_t)A.h_k * DK + (int64_t)ki * DK + (tid - DK);
    const bool has_v = tid < BVC;
    const int64_t gv = 2 * (int64_t)A.h_k * DK + (int64_t)h * A.d_v + colbase + tid;
    float wq[4];
    float q3 = 0.0f, q2 = 0.0f, q1 = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) wq[e] = to_f32(Wc[gq * 4 + e]);
    if (init) {
        q3 = to_f32(win[0 * C + gq]); q2 = to_f32(win[1 * C + gq]); q1 = to_f32(win[2 * C + gq]);
    }
    if (has_v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) wv4[4 * tid + e] = to_f32(Wc[gv * 4 + e]);
    }
    __syncthreads();
    const float exp_alog = expf(A.a_log[h]);
    const float dtb = A.dt_bias[h];
    bool my_last = false;
    float* __restrict__ Og = A.o + (int64_t)r0 * A.h_v * A.d_v + (int64_t)h * A.d_v + colbase + 16 * wv + lr;
    const int64_t o_stride = (int64_t)A.h_v * A.d_v;

    // ---- a chunk's raw inputs, loaded one chunk ahead into spare registers
    // (issued once the current chunk's own loads are consumed, so no wait in
    // a chunk ever covers them): x of channel gq for the 64 tokens, x of v
    // channel (tid & 63) for tokens 16 (tid >> 6) .. +15 and the three rows
    // before them, and the gate inputs of token `lane` (wave 0).  Rows are
    // clamped into the sequence, so every load is unconditional.
    ActT nq[CH], nv[16], nh[3], na = ActT(0), nb = ActT(0);
    const int vc = tid & 63, tq = tid >> 6;
    const int64_t gvc = 2 * (int64_t)A.h_k * DK + (int64_t)h * A.d_v + colbase + vc;
    auto prefetch = [&](int cs) {
        const ActT* xq = X + (int64_t)r0 * A.x_stride + gq;
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            const int tt = cs + t < T ? cs + t : T - 1;
            nq[t] = xq[(int64_t)tt * A.x_stride];
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int t = cs + 16 * tq - 3 + j;  // sequence-relative row
            if (t >= 0) {                        // uniform per wave for cs > 0
                nh[j] = X[(int64_t)(r0 + (t < T ? t : T - 1)) * A.x_stride + gvc];
            } else {
                nh[j] = init ? win[(int64_t)(3 + t) * C + gvc] : ActT(0);
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = cs + 16 * tq + i;
            nv[i] = X[(int64_t)(r0 + (t < T ? t : T - 1)) * A.x_stride + gvc];
        }
        if (wv == 0) {
            const int t = cs + lane < T ? cs + lane : T - 1;
            const int64_t row = (int64_t)(r0 + t) * A.ab_stride + h;
            na = static_cast<const ActT*>(A.a)[row];
            nb = static_cast<const ActT*>(A.b)[row];
        }
    };
    prefetch(0);

    // A chunk's output tile (wave w: columns 16 w .. +15) is stored during the
    // next chunk, right after that chunk's prefetch is issued.
    f32x4 o_tile[4];
    int o_c0 = 0, o_n = 0;
    auto store_o = [&]() {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * mt + 4 * lg + j;
                if (t < o_n) Og[(int64_t)(o_c0 + t) * o_stride] = o_tile[mt][j];
            }
        o_n = 0;
    };

    for (int c0 = 0; c0 < T; c0 += CH) {
        const int n = (T - c0 < CH) ? (T - c0) : CH;
        // ================================================================ P1
        {
            // q/k: channel `tid` over the 64 tokens in order (the window slides in
            // registers); padded values are zeroed.
            __bf16* qkh = is_q ? Qh + tid : Kh + (tid - DK);
            __bf16* qkl = is_q ? Ql + tid : Kl + (tid - DK);
            for (int t0 = 0; t0 < CH; t0 += 32) {
                float xs[32];
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    const int t = t0 + i;
                    xs[i] = t < n ? to_f32(nq[t]) : 0.0f;
                }
#pragma unroll
                for (int i = 0; i < 32; i += 2) {
                    float y[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int t = t0 + i + u;
                        y[u] = 0.0f;
                        if (t < n) {
                            y[u] = silu_fast(conv4(wq, q3, q2, q1, xs[i + u]));
                            q3 = q2; q2 = q1; q1 = xs[i + u];
                        }
                    }
                    const __bf16 h0 = (__bf16)y[0], h1 = (__bf16)y[1];
                    const __bf16 l0 = (__bf16)(y[0] - (float)h0), l1 = (__bf16)(y[1] - (float)h1);
                    const int t = t0 + i;
                    qkh[t * LQK] = h0; qkh[(t + 1) * LQK] = h1;
                    qkl[t * LQK] = l0; qkl[(t + 1) * LQK] = l1;
                    if (!is_q) {
                        const bf16x2 ph = {h0, h1}, pl = {l0, l1};
                        *reinterpret_cast<bf16x2*>(KTh + (tid - DK) * LT + t) = ph;
                        *reinterpret_cast<bf16x2*>(KTl + (tid - DK) * LT + t) = pl;
                    }
                }
            }
            // v: channel (tid & 63), tokens 16 (tid >> 6) .. +15, with the three rows
            // before them (from x, or the window before the first token)
            {
                const float* wvc = wv4 + 4 * vc;
                float hx[3];
#pragma unroll
                for (int j = 0; j < 3; ++j) hx[j] = to_f32(nh[j]);
                float xs[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int t = 16 * tq + i;
                    xs[i] = t < n ? to_f32(nv[i]) : 0.0f;
                }
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    float y[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int t = 16 * tq + i + u;
                        y[u] = t < n ? silu_fast(conv4(wvc, hx[0], hx[1], hx[2], xs[i + u])) : 0.0f;
                        hx[0] = hx[1]; hx[1] = hx[2]; hx[2] = xs[i + u];
                    }
                    const __bf16 h0 = (__bf16)y[0], h1 = (__bf16)y[1];
                    const bf16x2 ph = {h0, h1};
                    const bf16x2 pl = {(__bf16)(y[0] - (float)h0), (__bf16)(y[1] - (float)h1)};
                    *reinterpret_cast<bf16x2*>(VTh + vc * LT + 16 * tq + i) = ph;
                    *reinterpret_cast<bf16x2*>(VTl + vc * LT + 16 * tq + i) = pl;
                }
            }
        }
        lds_barrier();
        if (c0 == 0 && tid == 0)  // every window read of this workgroup has been consumed
            my_last = arrive_last(A.sync + (int64_t)page * A.h_k + ki, (uint32_t)(rr * nblk));
        // ================================================================ P2
        {
            // norms: 16 lanes per token, tokens grp + 16 i
            const int grp = tid >> 4, l16 = tid & 15;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = grp + 16 * i;
                float sq = 0.0f, sk = 0.0f, qk = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int d = 8 * l16 + e;
                    const float qv = (float)Qh[t * LQK + d] + (float)Ql[t * LQK + d];
                    const float kv = (float)Kh[t * LQK + d] + (float)Kl[t * LQK + d];
                    sq = fmaf(qv, qv, sq);
                    sk = fmaf(kv, kv, sk);
                    qk = fmaf(qv, kv, qk);
                }
                sq = reduce16(sq);
                sk = reduce16(sk);
                qk = reduce16(qk);
                if (l16 == 0) {
                    const bool ok = t < n;
                    const float rq = ok ? A.scale / sqrtf(sq + A.eps) : 0.0f;
                    const float rk = ok ? 1.0f / sqrtf(sk + A.eps) : 0.0f;
                    sc[SC_RQ * CH + t] = rq;
                    sc[SC_RK * CH + t] = rk;
                    sc[SC_KQ * CH + t] = rq * rk * qk;
                }
            }
            // gates and the cumulative decay: wave 0, lane = token
            if (wv == 0) {
                const int t = lane;
                const float av = to_f32(na);
                const float bv = to_f32(nb);
                const float g = t < n ? -exp_alog * softplus(av + dtb) : 0.0f;
                const float beta = t < n ? sigmoid(bv) : 0.0f;
                float G = g;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float o = __shfl_up(G, off, 64);
                    if (lane >= off) G += o;
                }
                const float Glast = __shfl(G, 63, 64);
                sc[SC_G * CH + t] = G;
                sc[SC_BETA * CH + t] = beta;
                sc[SC_GAM * CH + t] = expf(G);
                sc[SC_WDR * CH + t] = expf(Glast - G);  // rk folded in below
            }
        }
        lds_barrier();
        {
            const int t = tid & 63;
            if (tid < CH) {
                const float rk = sc[SC_RK * CH + t];
                sc[SC_BGR * CH + t] = sc[SC_BETA * CH + t] * sc[SC_GAM * CH + t] * rk;
                // the last row of the chunk enters the state update exactly, not through the MFMA
                sc[SC_WDR * CH + t] = (t == n - 1) ? 0.0f : sc[SC_WDR * CH + t] * rk;
            }
            if (tid < DK) {
                const int tl = n - 1;
                klast[tid] = sc[SC_RK * CH + tl] * ((float)KTh[tid * LT + tl] + (float)KTl[tid * LT + tl]);
            }
        }
        lds_barrier();
        // the next chunk's inputs: every load of this chunk has been consumed
        if (c0 + CH < T) prefetch(c0 + CH);
        // then the previous chunk's outputs: a wait for the prefetch above (in
        // order) never covers stores issued after it
        store_o();
        // ================================================================ P3
        {
            // the 10 tiles on or below the diagonal, round-robin over the waves
            f32x4 accq[3], acck[3];
            int tmt[3], tnt[3];
            int cnt = 0;
            for (int idx = wv, k = 0; k < 3; ++k, idx += 4) {
                tmt[k] = -1;
                if (idx >= 10) continue;
                int mt = 0, rem = idx;
                while (rem > mt) { rem -= mt + 1; ++mt; }
                const int nt = rem;
                tmt[k] = mt; tnt[k] = nt;
                f32x4 aq = {0.0f, 0.0f, 0.0f, 0.0f}, ak = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int col = 32 * ks + 8 * lg;
                    const bf16x8 qh = ld8(Qh, LQK, 16 * mt + lr, col);
                    const bf16x8 ql = ld8(Ql, LQK, 16 * mt + lr, col);
                    const bf16x8 khm = ld8(Kh, LQK, 16 * mt + lr, col);
                    const bf16x8 khn = ld8(Kh, LQK, 16 * nt + lr, col);
                    const bf16x8 kln = ld8(Kl, LQK, 16 * nt + lr, col);
                    aq = mma32(qh, khn, aq);
                    aq = mma32(qh, kln, aq);
                    aq = mma32(ql, khn, aq);
                    ak = mma32(khm, khn, ak);
                }
                accq[k] = aq; acck[k] = ak;
                ++cnt;
            }
            lds_barrier();  // Ql is about to be overwritten by A
            for (int k = 0; k < 3; ++k) {
                if (tmt[k] < 0) continue;
                const int mt = tmt[k], nt = tnt[k];
                const int sidx = 16 * nt + lr;
                const float Gs = sc[SC_G * CH + sidx], rks = sc[SC_RK * CH + sidx];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = 16 * mt + 4 * lg + j;
                    float p = 0.0f, a = 0.0f;
                    if (sidx < t) {
                        const float e = expf(sc[SC_G * CH + t] - Gs);
                        const float rkt = sc[SC_RK * CH + t];
                        p = sc[SC_RQ * CH + t] * rks * accq[k][j] * e;
                        a = sc[SC_BETA * CH + t] * rkt * rks * acck[k][j] * e;
                    }
                    const __bf16 ph = (__bf16)p;
                    Ph[t * LT + sidx] = ph;
                    Pl[t * LT + sidx] = (__bf16)(p - (float)ph);
                    Af[t * LAF + sidx] = a;
                }
            }
            (void)cnt;
        }
        lds_barrier();
        // ================================================================ P4
        {
            // diagonal block b = wv: T_bb = (I - N)(I + N^2)(I + N^4)(I + N^8)
            const int b = wv;
            f32x4 nB, ntB, eye;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * lg + j;
                nB[j] = Af[(16 * b + r) * LAF + 16 * b + lr];   // N[r][lr]
                ntB[j] = Af[(16 * b + lr) * LAF + 16 * b + r];  // N^T[r][lr]
                eye[j] = (r == lr) ? 1.0f : 0.0f;
            }
            const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
            f32x4 Y = nB, Z = ntB;                 // N^(2^k) and its transpose, accumulator layout
            f32x4 R = eye - nB;                    // running product, starts at I - N
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const f32x4 Yn = mma16(to_bf4(Z), to_bf4(Y), zero);  // Y <- Y Y (A operand = layout of Y^T = Z)
                const f32x4 Zn = mma16(to_bf4(Y), to_bf4(Z), zero);  // Z <- Z Z
                Y = Yn; Z = Zn;
                R = mma16(to_bf4(eye + Z), to_bf4(R), zero);         // R <- (I + Y) R
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) Tm[(16 * b + 4 * lg + j) * LT + 16 * b + lr] = (__bf16)R[j];
        }
        lds_barrier();
        // off-diagonal blocks by sub-diagonal level: T_bc = -T_bb sum_{d=c}^{b-1} A_bd T_dc
        for (int lev = 1; lev < 4; ++lev) {
            if (wv < 4 - lev) {
                const int c = wv, b = wv + lev;
                const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
                f32x4 Xacc = zero;
                for (int d = c; d < b; ++d) {
                    // A operand: A_bd[lr][4 lg + i]; B operand: T_dc[4 lg + i][lr]
                    const float* ar = Af + (16 * b + lr) * LAF + 16 * d + 4 * lg;
                    const bf16x4 aop = to_bf4(ar[0], ar[1], ar[2], ar[3]);
                    const bf16x4 bop = {Tm[(16 * d + 4 * lg + 0) * LT + 16 * c + lr],
                                        Tm[(16 * d + 4 * lg + 1) * LT + 16 * c + lr],
                                        Tm[(16 * d + 4 * lg + 2) * LT + 16 * c + lr],
                                        Tm[(16 * d + 4 * lg + 3) * LT + 16 * c + lr]};
                    Xacc = mma16(aop, bop, Xacc);
                }
                const bf16x4 tbb = ld4(Tm, LT, 16 * b + lr, 16 * b + 4 * lg);
                const f32x4 Yv = mma16(tbb, to_bf4(Xacc), zero);
#pragma unroll
                for (int j = 0; j < 4; ++j) Tm[(16 * b + 4 * lg + j) * LT + 16 * c + lr] = (__bf16)(-Yv[j]);
            }
            lds_barrier();
        }
        // LT = T - I (strictly lower), column-scaled by beta and by beta e^G rk
        for (int e = tid; e < CH * CH; e += NTH) {
            const int t = e >> 6, sidx = e & 63;
            const float lt = (sidx < t) ? (float)Tm[t * LT + sidx] : 0.0f;
            LTb[t * LT + sidx] = (__bf16)(lt * sc[SC_BETA * CH + sidx]);
            LTbg[t * LT + sidx] = (__bf16)(lt * sc[SC_BGR * CH + sidx]);
        }
        lds_barrier();
        // ================================================================ P5
        {
            // W[t][d] = bgr_t K[t][d] + (LTbg K)[t][d]; 32 tiles, 8 per wave
            f32x4 wacc[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int idx = wv + 4 * k, mt = idx >> 3, dt = idx & 7;
                const int d = 16 * dt + lr;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = 16 * mt + 4 * lg + j;
                    wacc[k][j] = sc[SC_BGR * CH + t] * ((float)KTh[d * LT + t] + (float)KTl[d * LT + t]);
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8 aop = ld8(LTbg, LT, 16 * mt + lr, 32 * ks + 8 * lg);
                    const bf16x8 bop = ld8(KTh, LT, d, 32 * ks + 8 * lg);
                    wacc[k] = mma32(aop, bop, wacc[k]);
                }
            }
            // A (in the same region) is dead since the LT pass; W takes its place
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int idx = wv + 4 * k, mt = idx >> 3, dt = idx & 7;
#pragma unroll
                for (int j = 0; j < 4; ++j) Wm[(16 * mt + 4 * lg + j) * LQK + 16 * dt + lr] = (__bf16)wacc[k][j];
            }
        }
        lds_barrier();
        // ================================================================ P6
        {
            const int colv = 16 * wv + lr;  // this lane's column within the block
            bf16x4 sb[8];
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) sb[dt] = to_bf4(s[dt]);
            f32x4 D[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                // U = beta V + LTb V
                f32x4 u;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = 16 * mt + 4 * lg + j;
                    u[j] = sc[SC_BETA * CH + t] * ((float)VTh[colv * LT + t] + (float)VTl[colv * LT + t]);
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    u = mma32(ld8(LTb, LT, 16 * mt + lr, 32 * ks + 8 * lg), ld8(VTh, LT, colv, 32 * ks + 8 * lg), u);
                // W S
                f32x4 ws = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) ws = mma16(ld4(Wm, LQK, 16 * mt + lr, 16 * kt + 4 * lg), sb[kt], ws);
                D[mt] = u - ws;
            }
            bf16x4 dh[4], dl[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) split4(D[mt], dh[mt], dl[mt]);
            // O = diag(e^G rq) Q S + diag(k.q) D + P D
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 qs = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) qs = mma16(ld4(Qh, LQK, 16 * mt + lr, 16 * kt + 4 * lg), sb[kt], qs);
                f32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = 16 * mt + 4 * lg + j;
                    o[j] = sc[SC_GAM * CH + t] * sc[SC_RQ * CH + t] * qs[j] + sc[SC_KQ * CH + t] * D[mt][j];
                }
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    if (kt > mt) continue;
                    const bf16x4 ph = ld4(Ph, LT, 16 * mt + lr, 16 * kt + 4 * lg);
                    const bf16x4 pl = ld4(Pl, LT, 16 * mt + lr, 16 * kt + 4 * lg);
                    o = mma16(ph, dh[kt], o);
                    o = mma16(ph, dl[kt], o);
                    o = mma16(pl, dh[kt], o);
                }
                o_tile[mt] = o;
            }
            o_c0 = c0;
            o_n = n;
            // S <- e^{G_last} S + K^T diag(rk e^{G_last - G}) D  (+ the last row exactly)
            bf16x4 wh[4], wl[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                f32x4 dw;
#pragma unroll
                for (int j = 0; j < 4; ++j) dw[j] = D[kt][j] * sc[SC_WDR * CH + 16 * kt + 4 * lg + j];
                split4(dw, wh[kt], wl[kt]);
            }
            const int tl = n - 1;
            float dsel = 0.0f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (16 * kt + 4 * lg + j == tl) dsel = D[kt][j];
            // the lane of group (tl % 16) / 4 holds D[tl][colv]
            const float dlast = __shfl(dsel, ((tl & 15) >> 2) * 16 + lr, 64);
            const float glast = sc[SC_GAM * CH + tl];
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                f32x4 acc = s[dt] * glast;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    const bf16x4 kh = ld4(KTh, LT, 16 * dt + lr, 16 * kt + 4 * lg);
                    const bf16x4 kl = ld4(KTl, LT, 16 * dt + lr, 16 * kt + 4 * lg);
                    acc = mma16(kh, wh[kt], acc);
                    acc = mma16(kh, wl[kt], acc);
                    acc = mma16(kl, wh[kt], acc);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = fmaf(klast[16 * dt + 4 * lg + j], dlast, acc[j]);
                s[dt] = acc;
            }
        }
        lds_barrier();
    }

    store_o();  // the last chunk's outputs

    // ---- epilogue: state, then the rolled windows
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) Sg[(int64_t)(16 * dt + 4 * lg + j) * A.d_v] = from_f32<StT>(s[dt][j]);
    if (tid == 0) sh_last = my_last ? 1 : 0;
    lds_barrier();
    if (sh_last) {
        win[0 * C + gq] = from_f32<ActT>(q3);
        win[1 * C + gq] = from_f32<ActT>(q2);
        win[2 * C + gq] = from_f32<ActT>(q1);
    }
    if (has_v) {
        // rolled v window: the last three rows of (window ++ sequence), read
        // before any write (this workgroup alone owns these channels)
        float vw[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int t = T - 3 + j;
            const float xa = to_f32(X[(int64_t)(r0 + (t < 0 ? 0 : t)) * A.x_stride + gv]);
            const float wa = init ? to_f32(win[(int64_t)(3 + (t < 0 ? t : -1)) * C + gv]) : 0.0f;
            vw[j] = t >= 0 ? xa : wa;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) win[(int64_t)j * C + gv] = from_f32<ActT>(vw[j]);
    }
}

template <typename ActT, typename StT>
hipError_t launch_chunk_t(const ChunkArgs& a, hipStream_t s) {
    const int nblk = a.d_v / BVC;
    const int64_t grid = (int64_t)a.n_seqs * a.h_v * nblk;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_gdn_chunk<ActT, StT>), dim3((unsigned)grid), dim3(NTH), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool chunked_supported(int d_k, int d_v, int chunk) { return d_k == DK && d_v > 0 && d_v % BVC == 0 && chunk == CH; }

hipError_t launch_chunked(const ChunkArgs& a, int d_k, int act_dtype, int state_dtype, hipStream_t s) {
    if (!chunked_supported(d_k, a.d_v, CH)) return hipErrorInvalidValue;
    if (act_dtype == GDN_BF16)
        return state_dtype == GDN_BF16 ? launch_chunk_t<bf16_t, bf16_t>(a, s) : launch_chunk_t<bf16_t, float>(a, s);
    return state_dtype == GDN_BF16 ? launch_chunk_t<float, bf16_t>(a, s) : launch_chunk_t<float, float>(a, s);
}

}  // namespace gdn
