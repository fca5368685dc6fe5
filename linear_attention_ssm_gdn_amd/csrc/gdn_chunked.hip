// gdn_chunked.hip -- chunked WY/UT prefill of the GDN layer core (Gated
// DeltaNet part (c), chunked form) on bf16 matrix cores with fp32
// accumulation, conv + SiLU + gating fused in.
//
// Grid: one workgroup of 4 waves per (sequence, value head h, block of 64
// value columns).  Wave w owns the 16-column tile w of the block; its share
// of the fp32 state S (128 x 16) lives in MFMA accumulator registers for the
// whole sequence.  Chunks of C = 64 tokens run in order.  Per chunk, with
// chunk-local cumulative decay G and start state S0:
//   P1  conv + SiLU on register tiles (q/k: 8 channels x 8 tokens per thread,
//       v: 4 x 4), fed by 16-byte row loads issued one chunk ahead.  Raw
//       post-conv q and k go to LDS as bf16 hi/lo pairs, token-major (for
//       contractions over d) and k also transposed (for contractions over
//       tokens); v transposed.  The per-token sums of squares are reduced from
//       the same registers (16 lanes hold one token group), giving the L2-norm
//       factors rq (with the output scale) and rk, which stay per-token factors
//       folded into every product below instead of rescaling the arrays.
//       Wave 0 also takes the gates and the scan of the cumulative decay G.
//   P3  Q K^T (three-pass hi/lo) and K K^T on MFMA; P_ts = rq_t rk_s (q_t.k_s)
//       e^{G_t-G_s} and A_ts = beta_t rk_t rk_s (k_t.k_s) e^{G_t-G_s} for s < t,
//       masked before the exponential; the diagonal gives k_t.q_t.
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
constexpr int OFF_WQK = OFF_WV + BVC * 4 * 4;    // [256][4] fp32 q and k channel conv taps
constexpr int LDS_BYTES = OFF_WQK + 2 * DK * 4 * 4;
constexpr int LOS = 68;                          // fp32 row stride of the output staging tile (in P's region)
static_assert(CH * LOS * 4 <= 2 * CH * LT * 2, "output staging fits P");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert(CH * LAF * 4 <= SZ_REG && CH * LQK * 2 <= SZ_REG, "region sizes");

// scalar rows in the SC block
enum { SC_RQ = 0, SC_RK, SC_KQ, SC_BETA, SC_GAM, SC_BGR, SC_WDR, SC_G };

// A vector instruction that reads a matrix-core result must not issue
// within the product's write-back.  The compiler schedules such reads (or the
// copies out of the accumulator registers) 8 wait states after a 16x16x32
// product, and on this part those reads have returned stale values now and
// then: outputs of identical launches differed in the first two accumulator
// registers of some lanes, and 16 more wait states made every launch
// bit-identical, while a rarer mismatch remained (about one launch in a
// few hundred); the wait is 32 wait states.  Every product chain whose result
// vector instructions read ends with settle(): the wait states take the
// accumulators as accumulator-register operands, so they follow the last
// product that writes them and precede every read or copy of them.  The one
// chain that feeds a 16x16x32 result into 16x16x16 products (different pass
// counts) settles in between as well.  Results of 16x16x16 products (the UT
// solve's diagonal blocks and sub-diagonals) are read at the compiler's 8
// wait states: while 16x16x32 reads failed in nearly every launch, the
// states, which depend on every UT solve, never differed.
#define GDN_SETTLE_NOPS "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
__device__ __forceinline__ void settle(f32x4& a) { asm volatile(GDN_SETTLE_NOPS : "+a"(a)); }
__device__ __forceinline__ void settle(f32x4& a, f32x4& b) { asm volatile(GDN_SETTLE_NOPS : "+a"(a), "+a"(b)); }
__device__ __forceinline__ void settle4(f32x4 (&a)[4]) {
    asm volatile(GDN_SETTLE_NOPS : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]));
}
__device__ __forceinline__ void settle8(f32x4 (&a)[8]) {
    asm volatile(GDN_SETTLE_NOPS : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]), "+a"(a[4]), "+a"(a[5]),
                 "+a"(a[6]), "+a"(a[7]));
}

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
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }
__device__ __forceinline__ void split4(const f32x4& v, bf16x4& hi, bf16x4& lo) {
    hi = to_bf4(v);
    lo = to_bf4(v[0] - (float)hi[0], v[1] - (float)hi[1], v[2] - (float)hi[2], v[3] - (float)hi[3]);
}
// SiLU through the hardware exponential and reciprocal (about one ulp each,
// far inside the error of the bf16 products that consume it).
__device__ __forceinline__ float silu_fast(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
// The same for z given as log2(e) z, returning log2(e) silu(z).
__device__ __forceinline__ float silu_log2e(float zl) { return zl * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zl)); }
constexpr float LOG2E = 1.44269504088896341f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
// Two floats rounded to bf16 (nearest even) and packed, a in the low half.
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
    const bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
}
// hi/lo split of a pair: hi = bf16(a, b), lo = bf16 of what hi misses.
__device__ __forceinline__ void split_pk(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = pack_bf2(a, b);
    lo = pack_bf2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// K^T [128][LT] is stored with its token columns XOR-swizzled in blocks of 8
// by bits 3..5 of the row, so that the conv threads' 16-byte column writes
// (eight channels of one token block per lane group) spread over all banks.
// Every 4- and 8-token operand read stays inside one block.
__device__ __forceinline__ int kt_at(int row, int col) { return row * LT + (col ^ (row & 0x38)); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// N consecutive channels of one activation row, loaded as one vector.
template <typename ActT, int N> struct RowVec;
template <int N> struct RowVec<bf16_t, N> {
    typedef uint32_t V __attribute__((ext_vector_type(N / 2)));
    V v;
    __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const V*>(p); }
    __device__ __forceinline__ void zero() { v = V(0u); }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t w = v[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};
template <int N> struct RowVec<float, N> {
    f32x4 v[N / 4];
    __device__ __forceinline__ void load(const float* p) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) v[i] = *reinterpret_cast<const f32x4*>(p + 4 * i);
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) v[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    __device__ __forceinline__ float get(int e) const { return v[e >> 2][e & 3]; }
};

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
    __bf16* Wm = reinterpret_cast<__bf16*>(lds + OFF_QL);                  // -W, after P5
    float* Os = reinterpret_cast<float*>(lds + OFF_PH);                    // from P6's end to the next P3
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
    // Dispatch order: with more workgroups than stay resident (one per CU),
    // index v takes the v-th longest sequence (ties by position), so the
    // longest sequences start first.  Batches of up to one sequence per
    // thread are ranked; larger ones keep their order.
    int seq = bid / A.h_v;
    if (A.n_seqs > 1 && A.n_seqs <= NTH) {
        int* len = reinterpret_cast<int*>(lds + OFF_SC);  // free until the first chunk's gates
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
            if (rank == seq) sh_last = tid;
        }
        __syncthreads();
        seq = sh_last;
        __syncthreads();  // sh_last is reused at the end
    }
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

    // ---- conv taps to LDS: q/k channel `tid` (q for tid < 128), v channel `tid`
    const ActT* __restrict__ X = static_cast<const ActT*>(A.x);
    ActT* __restrict__ win = static_cast<ActT*>(A.conv_base) + (int64_t)page * A.conv_page_stride;
    const ActT* Wc = static_cast<const ActT*>(A.conv_w);
    const int64_t gq = tid < DK ? (int64_t)ki * DK + tid : (int64_t)A.h_k * DK + (int64_t)ki * DK + (tid - DK);
    const bool has_v = tid < BVC;
    const int64_t gv = 2 * (int64_t)A.h_k * DK + (int64_t)h * A.d_v + colbase + tid;
    float* wqk = reinterpret_cast<float*>(lds + OFF_WQK);
    // q and k are only ever used through their L2-norm factors, so they are
    // carried scaled by log2(e) (conv taps scaled here, eps by log2(e)^2 in
    // the norms), which puts the SiLU's exponential on exp2 directly
#pragma unroll
    for (int e = 0; e < 4; ++e) wqk[4 * tid + e] = LOG2E * to_f32(Wc[gq * 4 + e]);
    if (has_v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) wv4[4 * tid + e] = to_f32(Wc[gv * 4 + e]);
    }
    __syncthreads();
    const float exp_alog = expf(A.a_log[h]);
    const float dtb = A.dt_bias[h];
    bool my_last = false;
    float* __restrict__ Og = A.o + (int64_t)r0 * A.h_v * A.d_v + (int64_t)h * A.d_v + colbase;
    const int64_t o_stride = (int64_t)A.h_v * A.d_v;

    // ---- conv tiles.  q/k: part (q, then k) = tid >> 7, tokens 8 tgp .. +7,
    // channels 8 cgl .. +7 of the key head, so the 16 lanes of a DPP row hold
    // one token group over all 128 channels.  v: tokens 4 tq4 .. +3, channels
    // 4 vc4 .. +3 of the block.  The lane-derived offsets are recomputed at
    // each use from an opaque copy of tid (cheap integer work) rather than
    // hoisted out of the chunk loop, where they would hold registers for its
    // whole length.
    auto fresh_tid = [&]() {
        int t = tid;
        asm volatile("" : "+v"(t));
        return t;
    };
    // the same for the MFMA phases' lane indices (the wave index made scalar)
#define PHASE_IDS                                                                      \
    const int tid = fresh_tid(), lane = tid & 63, lr = lane & 15, lg = lane >> 4;     \
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);                          \
    (void)lane; (void)lr; (void)lg; (void)wv

    // ---- a chunk's raw inputs, loaded one chunk ahead into spare registers
    // (issued once the current chunk's own loads are consumed, so no wait in
    // a chunk ever covers them): each tile's rows with the three before them
    // (from x, or the window before the first token), and the gate inputs of
    // token `lane` (wave 0).  Rows past the end are clamped into the sequence
    // (their outputs are masked), so every load is unconditional.
    RowVec<ActT, 8> nqk[11];
    RowVec<ActT, 4> nvv[7];
    ActT na = ActT(0), nb = ActT(0);
    auto prefetch = [&](int cs) {
        const int ft = fresh_tid();
        const int tgp = (ft >> 4) & 7, tq4 = ft & 15;
        const int64_t gq8 = (int64_t)(ft >> 7) * A.h_k * DK + (int64_t)ki * DK + 8 * (ft & 15);
        const int64_t gv4 = 2 * (int64_t)A.h_k * DK + (int64_t)h * A.d_v + colbase + 4 * (ft >> 4);
#pragma unroll
        for (int j = 0; j < 11; ++j) {
            const int t = cs + 8 * tgp - 3 + j;  // sequence-relative row; < 0 only in the first chunk
            if (t >= 0)
                nqk[j].load(X + (int64_t)(r0 + (t < T ? t : T - 1)) * A.x_stride + gq8);
            else if (init)
                nqk[j].load(win + (int64_t)(3 + t) * C + gq8);
            else
                nqk[j].zero();
        }
#pragma unroll
        for (int j = 0; j < 7; ++j) {
            const int t = cs + 4 * tq4 - 3 + j;
            if (t >= 0)
                nvv[j].load(X + (int64_t)(r0 + (t < T ? t : T - 1)) * A.x_stride + gv4);
            else if (init)
                nvv[j].load(win + (int64_t)(3 + t) * C + gv4);
            else
                nvv[j].zero();
        }
        if (wv == 0) {
            const int t = cs + lane < T ? cs + lane : T - 1;
            const int64_t row = (int64_t)(r0 + t) * A.ab_stride + h;
            na = static_cast<const ActT*>(A.a)[row];
            nb = static_cast<const ActT*>(A.b)[row];
        }
    };
    prefetch(0);

    // A chunk's output tile (wave w: columns 16 w .. +15, in MFMA accumulator
    // layout) goes to LDS once the chunk's last read of P is done, and to
    // memory as 16-byte row pieces during the next chunk, right after that
    // chunk's prefetch is issued.
    f32x4 o_tile[4];
    int o_c0 = 0, o_n = 0;
    auto stage_o = [&]() {
        PHASE_IDS;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) Os[(16 * mt + 4 * lg + j) * LOS + 16 * wv + lr] = o_tile[mt][j];
    };
    auto store_o = [&]() {
        const int ft = fresh_tid();
        const int c4 = ft & 15, r = ft >> 4;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int t = r + 16 * it;
            if (t < o_n)
                *reinterpret_cast<f32x4*>(Og + (int64_t)(o_c0 + t) * o_stride + 4 * c4) =
                    *reinterpret_cast<const f32x4*>(Os + t * LOS + 4 * c4);
        }
        o_n = 0;
    };

    for (int c0 = 0; c0 < T; c0 += CH) {
        const int n = (T - c0 < CH) ? (T - c0) : CH;
        // ================================================================ P1
        {
            // q/k tile, two channels at a time over the 8 tokens: each pair packs
            // into one dword of every token-major row.  Outputs of tokens past
            // the end are left unmasked: their inputs are clamped real rows, so
            // they are finite, and every product that reads them is scaled by a
            // zero factor (rq, rk or beta of the padded token).
            const int ft = fresh_tid();
            const int part = ft >> 7, tgp = (ft >> 4) & 7, cgl = ft & 15;
            const int tq4 = ft & 15, vc4 = ft >> 4;
            const float* wrow = wqk + 4 * (part * DK + 8 * cgl);
            u32x4 ph[8], pl[8];
            float ss[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) ss[i] = 0.0f;
#pragma unroll
            for (int ep = 0; ep < 4; ++ep) {
                float y[2][8];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int e = 2 * ep + u;
                    const f32x4 w4 = *reinterpret_cast<const f32x4*>(wrow + 4 * e);
                    const float w[4] = {w4[0], w4[1], w4[2], w4[3]};
                    float xv[11];
#pragma unroll
                    for (int j = 0; j < 11; ++j) xv[j] = nqk[j].get(e);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        y[u][i] = silu_log2e(conv4(w, xv[i], xv[i + 1], xv[i + 2], xv[i + 3]));
                        ss[i] = fmaf(y[u][i], y[u][i], ss[i]);
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    uint32_t hi, lo;
                    split_pk(y[0][i], y[1][i], hi, lo);
                    ph[i][ep] = hi;
                    pl[i][ep] = lo;
                }
                if (part) {  // k also transposed: rows 2 ep (low halves) and 2 ep + 1 (high halves)
                    u32x4 h0, h1, l0, l1;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const uint32_t a = ph[2 * m][ep], b = ph[2 * m + 1][ep];
                        const uint32_t c = pl[2 * m][ep], d = pl[2 * m + 1][ep];
                        h0[m] = (a & 0xffffu) | (b << 16);
                        h1[m] = (a >> 16) | (b & 0xffff0000u);
                        l0[m] = (c & 0xffffu) | (d << 16);
                        l1[m] = (c >> 16) | (d & 0xffff0000u);
                    }
                    const int c = 8 * cgl + 2 * ep;
                    *reinterpret_cast<u32x4*>(KTh + kt_at(c, 8 * tgp)) = h0;
                    *reinterpret_cast<u32x4*>(KTh + kt_at(c + 1, 8 * tgp)) = h1;
                    *reinterpret_cast<u32x4*>(KTl + kt_at(c, 8 * tgp)) = l0;
                    *reinterpret_cast<u32x4*>(KTl + kt_at(c + 1, 8 * tgp)) = l1;
                }
            }
            {
                __bf16* rowh = (part ? Kh : Qh) + (8 * tgp) * LQK + 8 * cgl;
                __bf16* rowl = (part ? Kl : Ql) + (8 * tgp) * LQK + 8 * cgl;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    *reinterpret_cast<u32x4*>(rowh + i * LQK) = ph[i];
                    *reinterpret_cast<u32x4*>(rowl + i * LQK) = pl[i];
                }
            }
            // L2-norm factors: lane cgl (< 8) of the row writes token 8 tgp + cgl
            float mine = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float sum = reduce16(ss[i]);
                if ((cgl & 7) == i) mine = sum;
            }
            if (cgl < 8) {
                const int t = 8 * tgp + cgl;
                sc[(part ? SC_RK : SC_RQ) * CH + t] =
                    t < n ? (part ? 1.0f : A.scale) / sqrtf(mine + (LOG2E * LOG2E) * A.eps) : 0.0f;
            }

            // v tile: channel by channel, 4 tokens each, stored transposed
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int col = 4 * vc4 + e;
                const f32x4 w4 = *reinterpret_cast<const f32x4*>(wv4 + 4 * col);
                const float w[4] = {w4[0], w4[1], w4[2], w4[3]};
                float xv[7];
#pragma unroll
                for (int j = 0; j < 7; ++j) xv[j] = nvv[j].get(e);
                float y[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = silu_fast(conv4(w, xv[i], xv[i + 1], xv[i + 2], xv[i + 3]));
                uint32_t h0, l0, h1, l1;
                split_pk(y[0], y[1], h0, l0);
                split_pk(y[2], y[3], h1, l1);
                const u32x2 th = {h0, h1}, tl = {l0, l1};
                *reinterpret_cast<u32x2*>(VTh + col * LT + 4 * tq4) = th;
                *reinterpret_cast<u32x2*>(VTl + col * LT + 4 * tq4) = tl;
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
                sc[SC_G * CH + t] = G * LOG2E;  // P3 takes exp2 of differences
                sc[SC_BETA * CH + t] = beta;
                sc[SC_GAM * CH + t] = expf(G);
                sc[SC_WDR * CH + t] = expf(Glast - G);  // rk folded in below
            }
        }
        lds_barrier();
        if (c0 == 0 && tid == 0)  // every window read of this workgroup has been consumed
            my_last = arrive_last(A.sync + (int64_t)page * A.h_k + ki, (uint32_t)(rr * nblk));
        // the next chunk's inputs: every load of this chunk has been consumed
        if (c0 + CH < T) prefetch(c0 + CH);
        // then the previous chunk's outputs: a wait for the prefetch above (in
        // order) never covers stores issued after it
        store_o();
        // ================================================================ P3
        {
            PHASE_IDS;
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
                    // transposed tiles (rows s, columns t), so that each lane holds
                    // four consecutive s of one t and writes them as one vector
                    aq = mma32(khn, qh, aq);
                    aq = mma32(kln, qh, aq);
                    aq = mma32(khn, ql, aq);
                    ak = mma32(khn, khm, ak);
                }
                settle(aq, ak);
                accq[k] = aq; acck[k] = ak;
                ++cnt;
            }
            lds_barrier();  // Ql is about to be overwritten by A
            if (tid < CH) {
                const int t = tid;
                const float rk = sc[SC_RK * CH + t];
                sc[SC_BGR * CH + t] = sc[SC_BETA * CH + t] * sc[SC_GAM * CH + t] * rk;
                // the last row of the chunk enters the state update exactly, not through the MFMA
                sc[SC_WDR * CH + t] = (t == n - 1) ? 0.0f : sc[SC_WDR * CH + t] * rk;
            } else if (tid < CH + DK) {
                const int d = tid - CH, tl = n - 1;
                klast[d] = sc[SC_RK * CH + tl] * ((float)KTh[kt_at(d, tl)] + (float)KTl[kt_at(d, tl)]);
            }
            for (int k = 0; k < 3; ++k) {
                if (tmt[k] < 0) continue;
                const int mt = tmt[k], nt = tnt[k];
                const int t = 16 * mt + lr, s0 = 16 * nt + 4 * lg;
                const float g2t = sc[SC_G * CH + t], rqt = sc[SC_RQ * CH + t];
                const float rkt = sc[SC_RK * CH + t], bt = sc[SC_BETA * CH + t];
                const f32x4 g2s = *reinterpret_cast<const f32x4*>(sc + SC_G * CH + s0);
                const f32x4 rks = *reinterpret_cast<const f32x4*>(sc + SC_RK * CH + s0);
                float p[4];
                f32x4 a;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // computed for every s and selected: for s >= t the exponential
                    // may overflow, and is discarded
                    const float e = __builtin_amdgcn_exp2f(g2t - g2s[j]);
                    const float pv = rqt * rks[j] * accq[k][j] * e;
                    const float av = bt * rkt * rks[j] * acck[k][j] * e;
                    p[j] = s0 + j < t ? pv : 0.0f;
                    a[j] = s0 + j < t ? av : 0.0f;
                    if (s0 + j == t) sc[SC_KQ * CH + t] = rqt * rkt * accq[k][j];
                }
                uint32_t h0, l0, h1, l1;
                split_pk(p[0], p[1], h0, l0);
                split_pk(p[2], p[3], h1, l1);
                *reinterpret_cast<u32x2*>(Ph + t * LT + s0) = u32x2{h0, h1};
                *reinterpret_cast<u32x2*>(Pl + t * LT + s0) = u32x2{l0, l1};
                *reinterpret_cast<f32x4*>(Af + t * LAF + s0) = a;
            }
            (void)cnt;
        }
        lds_barrier();
        // ================================================================ P4
        {
            PHASE_IDS;
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
                f32x4 Yn = mma16(to_bf4(Z), to_bf4(Y), zero);  // Y <- Y Y (A operand = layout of Y^T = Z)
                f32x4 Zn = mma16(to_bf4(Y), to_bf4(Z), zero);  // Z <- Z Z
                Y = Yn; Z = Zn;
                R = mma16(to_bf4(eye + Z), to_bf4(R), zero);         // R <- (I + Y) R
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) Tm[(16 * b + 4 * lg + j) * LT + 16 * b + lr] = (__bf16)R[j];
        }
        lds_barrier();
        // off-diagonal blocks by sub-diagonal level: T_bc = -T_bb sum_{d=c}^{b-1} A_bd T_dc
        for (int lev = 1; lev < 4; ++lev) {
            PHASE_IDS;
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
                f32x4 Yv = mma16(tbb, to_bf4(Xacc), zero);
#pragma unroll
                for (int j = 0; j < 4; ++j) Tm[(16 * b + 4 * lg + j) * LT + 16 * c + lr] = (__bf16)(-Yv[j]);
            }
            lds_barrier();
        }
        // LT = T - I (strictly lower), column-scaled by beta and by beta e^G rk
        // (8 columns of one row per thread and pass)
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int e = fresh_tid() + NTH * pass;
            const int t = e >> 3, s0 = 8 * (e & 7);
            const bf16x8 tv = *reinterpret_cast<const bf16x8*>(Tm + t * LT + s0);
            const f32x4 b0 = *reinterpret_cast<const f32x4*>(sc + SC_BETA * CH + s0);
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(sc + SC_BETA * CH + s0 + 4);
            const f32x4 g0 = *reinterpret_cast<const f32x4*>(sc + SC_BGR * CH + s0);
            const f32x4 g1 = *reinterpret_cast<const f32x4*>(sc + SC_BGR * CH + s0 + 4);
            float lt[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) lt[k] = s0 + k < t ? (float)tv[k] : 0.0f;
            const u32x4 ob = {pack_bf2(lt[0] * b0[0], lt[1] * b0[1]), pack_bf2(lt[2] * b0[2], lt[3] * b0[3]),
                              pack_bf2(lt[4] * b1[0], lt[5] * b1[1]), pack_bf2(lt[6] * b1[2], lt[7] * b1[3])};
            const u32x4 og = {pack_bf2(lt[0] * g0[0], lt[1] * g0[1]), pack_bf2(lt[2] * g0[2], lt[3] * g0[3]),
                              pack_bf2(lt[4] * g1[0], lt[5] * g1[1]), pack_bf2(lt[6] * g1[2], lt[7] * g1[3])};
            *reinterpret_cast<u32x4*>(LTb + t * LT + s0) = ob;
            *reinterpret_cast<u32x4*>(LTbg + t * LT + s0) = og;
        }
        lds_barrier();
        // ================================================================ P5
        {
            PHASE_IDS;
            // W[t][d] = bgr_t K[t][d] + (LTbg K)[t][d]; 32 tiles, 8 per wave
            f32x4 wacc[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int idx = wv + 4 * k, mt = idx >> 3, dt = idx & 7;
                const int d = 16 * dt + lr;
                const int ko = kt_at(d, 16 * mt + 4 * lg);
                const bf16x4 kh = *reinterpret_cast<const bf16x4*>(KTh + ko);
                const bf16x4 kl = *reinterpret_cast<const bf16x4*>(KTl + ko);
                const f32x4 bg = *reinterpret_cast<const f32x4*>(sc + SC_BGR * CH + 16 * mt + 4 * lg);
#pragma unroll
                for (int j = 0; j < 4; ++j) wacc[k][j] = bg[j] * ((float)kh[j] + (float)kl[j]);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8 aop = ld8(LTbg, LT, 16 * mt + lr, 32 * ks + 8 * lg);
                    const bf16x8 bop = *reinterpret_cast<const bf16x8*>(KTh + kt_at(d, 32 * ks + 8 * lg));
                    wacc[k] = mma32(aop, bop, wacc[k]);
                }
            }
            settle8(wacc);
            // A (in the same region) is dead since the LT pass; W takes its place
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int idx = wv + 4 * k, mt = idx >> 3, dt = idx & 7;
#pragma unroll
                for (int j = 0; j < 4; ++j) Wm[(16 * mt + 4 * lg + j) * LQK + 16 * dt + lr] = (__bf16)(-wacc[k][j]);
            }
        }
        lds_barrier();
        // ================================================================ P6
        {
            PHASE_IDS;
            const int colv = 16 * wv + lr;  // this lane's column within the block
            // Contractions over d and over tokens run as 16x16x32 products on
            // accumulator-layout operands: lane group lg supplies K indices
            // 16 k + 4 lg + (0..3) of two consecutive 16-blocks k, which is a
            // permutation of the 32 K indices shared by both operands.
            bf16x8 sb[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) sb[kk] = cat8(to_bf4(s[2 * kk]), to_bf4(s[2 * kk + 1]));
            f32x4 D[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                // D = U - W S = beta V + LTb V + (-W) S, one accumulator chain
                const int t0 = 16 * mt + 4 * lg;
                const bf16x4 vh = ld4(VTh, LT, colv, t0), vl = ld4(VTl, LT, colv, t0);
                const f32x4 bt = *reinterpret_cast<const f32x4*>(sc + SC_BETA * CH + t0);
                f32x4 u;
#pragma unroll
                for (int j = 0; j < 4; ++j) u[j] = bt[j] * ((float)vh[j] + (float)vl[j]);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    u = mma32(ld8(LTb, LT, 16 * mt + lr, 32 * ks + 8 * lg), ld8(VTh, LT, colv, 32 * ks + 8 * lg), u);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    u = mma32(cat8(ld4(Wm, LQK, 16 * mt + lr, 32 * kk + 4 * lg), ld4(Wm, LQK, 16 * mt + lr, 32 * kk + 16 + 4 * lg)),
                              sb[kk], u);
                D[mt] = u;
            }
            settle4(D);
            bf16x4 dh[4], dl[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) split4(D[mt], dh[mt], dl[mt]);
            // O = diag(e^G rq) Q S + diag(k.q) D + P D  (P is lower triangular by
            // 16-blocks: block pairs below the diagonal, then the diagonal block
            // alone where it starts a pair)
            f32x4 qs[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int row = 16 * mt + lr;
                qs[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    qs[mt] = mma32(cat8(ld4(Qh, LQK, row, 32 * kk + 4 * lg), ld4(Qh, LQK, row, 32 * kk + 16 + 4 * lg)),
                                   sb[kk], qs[mt]);
            }
            settle4(qs);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int row = 16 * mt + lr;
                const int t0 = 16 * mt + 4 * lg;
                const f32x4 gm = *reinterpret_cast<const f32x4*>(sc + SC_GAM * CH + t0);
                const f32x4 rq = *reinterpret_cast<const f32x4*>(sc + SC_RQ * CH + t0);
                const f32x4 kq = *reinterpret_cast<const f32x4*>(sc + SC_KQ * CH + t0);
                f32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = gm[j] * rq[j] * qs[mt][j] + kq[j] * D[mt][j];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (2 * kk + 1 > mt) continue;
                    const bf16x8 ph = cat8(ld4(Ph, LT, row, 32 * kk + 4 * lg), ld4(Ph, LT, row, 32 * kk + 16 + 4 * lg));
                    const bf16x8 pl = cat8(ld4(Pl, LT, row, 32 * kk + 4 * lg), ld4(Pl, LT, row, 32 * kk + 16 + 4 * lg));
                    const bf16x8 bh = cat8(dh[2 * kk], dh[2 * kk + 1]), bl = cat8(dl[2 * kk], dl[2 * kk + 1]);
                    o = mma32(ph, bh, o);
                    o = mma32(ph, bl, o);
                    o = mma32(pl, bh, o);
                }
                if ((mt & 1) == 0) {
                    if (mt > 0) settle(o);
                    const bf16x4 ph = ld4(Ph, LT, row, 16 * mt + 4 * lg);
                    const bf16x4 pl = ld4(Pl, LT, row, 16 * mt + 4 * lg);
                    o = mma16(ph, dh[mt], o);
                    o = mma16(ph, dl[mt], o);
                    o = mma16(pl, dh[mt], o);
                }
                o_tile[mt] = o;
            }
            o_c0 = c0;
            o_n = n;
            // S <- e^{G_last} S + K^T diag(rk e^{G_last - G}) D  (+ the last row exactly)
            bf16x4 wh[4], wl[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const f32x4 wd = *reinterpret_cast<const f32x4*>(sc + SC_WDR * CH + 16 * kt + 4 * lg);
                split4(D[kt] * wd, wh[kt], wl[kt]);
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
            bf16x8 wh2[2], wl2[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                wh2[kk] = cat8(wh[2 * kk], wh[2 * kk + 1]);
                wl2[kk] = cat8(wl[2 * kk], wl[2 * kk + 1]);
            }
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const int row = 16 * dt + lr;
                f32x4 acc = s[dt] * glast;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int k0 = kt_at(row, 32 * kk + 4 * lg), k1 = kt_at(row, 32 * kk + 16 + 4 * lg);
                    const bf16x8 kh = cat8(*reinterpret_cast<const bf16x4*>(KTh + k0), *reinterpret_cast<const bf16x4*>(KTh + k1));
                    const bf16x8 kl = cat8(*reinterpret_cast<const bf16x4*>(KTl + k0), *reinterpret_cast<const bf16x4*>(KTl + k1));
                    acc = mma32(kh, wh2[kk], acc);
                    acc = mma32(kh, wl2[kk], acc);
                    acc = mma32(kl, wh2[kk], acc);
                }
                s[dt] = acc;
            }
            settle8(s);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const f32x4 kv = *reinterpret_cast<const f32x4*>(klast + 16 * dt + 4 * lg);
#pragma unroll
                for (int j = 0; j < 4; ++j) s[dt][j] = fmaf(kv[j], dlast, s[dt][j]);
            }
        }
        lds_barrier();
        stage_o();  // P is dead until the next chunk's P3
    }

    lds_barrier();
    store_o();  // the last chunk's outputs

    // ---- epilogue: state, then the rolled windows
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) Sg[(int64_t)(16 * dt + 4 * lg + j) * A.d_v] = from_f32<StT>(s[dt][j]);
    if (tid == 0) sh_last = my_last ? 1 : 0;
    lds_barrier();
    // rolled windows: the last three rows of (window ++ sequence) per channel,
    // each read before its thread writes.  The v channels belong to this
    // workgroup alone; the q/k channels are shared by the workgroups of the
    // key head and written by the last of them to arrive, after every other
    // has consumed its window reads.
    auto roll = [&](int64_t ch) {
        float vw[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int t = T - 3 + j;
            const float xa = to_f32(X[(int64_t)(r0 + (t < 0 ? 0 : t)) * A.x_stride + ch]);
            const float wa = init ? to_f32(win[(int64_t)(3 + (t < 0 ? t : -1)) * C + ch]) : 0.0f;
            vw[j] = t >= 0 ? xa : wa;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) win[(int64_t)j * C + ch] = from_f32<ActT>(vw[j]);
    };
    if (sh_last) roll(gq);
    if (has_v) roll(gv);
}

#undef PHASE_IDS

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
