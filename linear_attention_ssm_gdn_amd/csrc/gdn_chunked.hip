// gdn_chunked.hip -- chunked WY/UT prefill of the GDN layer core (Gated
// DeltaNet part (c), chunked form) on bf16 matrix cores with fp32
// accumulation, conv + SiLU + gating fused in.  Two launches:
//
// k_chunk_prep: one workgroup of 4 waves per (sequence, chunk of C = 64 rows,
// key head), every chunk at once.  With the chunk-local cumulative decay G:
//   conv + SiLU of q and k on register tiles (8 channels x 8 tokens per
//       thread); hi/lo bf16 rows token-major in LDS, k^T straight into the
//       record.  Per-token sums of squares reduced from the same registers
//       give the L2-norm factors rq (with the output scale) and rk, which stay
//       per-token factors folded into every product instead of rescaling the
//       arrays.
//   Q K^T (three-pass hi/lo) and K K^T on MFMA, kept in registers.
//   Per value head of the key head's group: the gates and the scan of G;
//       P_ts = rq_t rk_s (q_t.k_s) e^{G_t-G_s} and A_ts = beta_t rk_t rk_s
//       (k_t.k_s) e^{G_t-G_s} for s < t, masked before the exponential; the
//       UT transform T = (I + A)^{-1} (16x16 diagonal blocks by the doubling
//       identity (I+N)^{-1} = (I-N)(I+N^2)(I+N^4)(I+N^8), then the three block
//       sub-diagonals) and (T - I) diag(beta).  All of it goes to the chunk's
//       workspace records.
// k_chunk_state: one workgroup of 8 waves per (sequence, value head, 64 value
// columns): four waves hold the fp32 state S (128 x 16 columns each) and run
// the chain, four run the v conv and the outputs (details at the kernel).
// Chunks run in order, their records streamed into LDS one step ahead:
//   v conv + SiLU (4 channels x 4 tokens per thread) into a transposed hi/lo tile;
//   D = U - W S with the WY matrices U = T diag(beta) V and W = T diag(beta
//       e^G rk) K, computed as D = T diag(beta) E, E = V - diag(e^G rk) K S:
//       one product K S, then D = beta E + (T - I) diag(beta) E, so W is
//       never formed;
//   O = diag(e^G rq) Q S + diag(k.q) D + P D;
//   S <- e^{G_last} S + K^T diag(rk e^{G_last-G}) D, the chunk's last row as
//   an exact fp32 outer product.
// Rounding points were chosen by emulating the error against the fp64
// recurrence: single bf16 roundings that multiply a weight-one term (the
// diagonal of T and of Q K^T, the last row of the state update, beta E) would
// cost up to 2^-8 each, so those terms stay fp32, and P, D, E and K take
// hi/lo splits in the products where they dominate.
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

// LDS of the prep kernel (bytes): token-major q and k hi/lo; after the
// products the k hi region holds T, the q-lo region A.
constexpr int SZ_TOK = CH * LQK * 2;          // 17408
constexpr int SZ_REG = 18432;                  // regions that later hold two [64][72] bf16 arrays
constexpr int OFF_QH = 0;
constexpr int OFF_KH = OFF_QH + SZ_TOK;        // then T
constexpr int OFF_QL = OFF_KH + SZ_REG;        // then A (fp32)
constexpr int OFF_KL = OFF_QL + SZ_REG;
constexpr int PREP_LDS = OFF_KL + SZ_REG;
static_assert(CH * LAF * 4 <= SZ_REG && CH * LQK * 2 <= SZ_REG && 2 * CH * LT * 2 <= SZ_REG, "region sizes");

// scalar rows in the SC block
enum { SC_RQ = 0, SC_RK, SC_KQ, SC_BETA, SC_GAM, SC_WDR, SC_G };

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
__device__ __forceinline__ void settle(f32x4& a, f32x4& b) { asm volatile(GDN_SETTLE_NOPS : "+a"(a), "+a"(b)); }
// The same wait on accumulators held in architectural registers (kernels
// whose register budget is shared by two waves per SIMD keep MFMA results
// there rather than split the budget with accumulator registers).
__device__ __forceinline__ void settle_v(f32x4& a) { asm volatile(GDN_SETTLE_NOPS : "+v"(a)); }
__device__ __forceinline__ void settle4_v(f32x4 (&a)[4]) {
    asm volatile(GDN_SETTLE_NOPS : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
}
__device__ __forceinline__ void settle8_v(f32x4 (&a)[8]) {
    asm volatile(GDN_SETTLE_NOPS : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),
                 "+v"(a[6]), "+v"(a[7]));
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
// An 8-byte LDS read kept as an instruction of its own: the compiler would
// pair neighbouring 8-byte reads into one ds_read2_b64, which takes twice the
// LDS cycles of the two single reads (measured with the LDS counters).
typedef __attribute__((address_space(3))) const volatile bf16x4 lds_bf16x4_v;
__device__ __forceinline__ bf16x4 ld4s(const __bf16* p) { return *(lds_bf16x4_v*)(p); }
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

// ============================================================================
// Workspace: chunk c of sequence s has slot s + (cu[s] >> 6) + c (distinct
// for packed sequences, fewer than n_seqs + ceil(n_rows / 64) in all); a slot
// holds h_k key-head records, then h_v value-head records, in the LDS
// layouts the state kernel reads.
constexpr int LTB_ELEMS = 32 * 32 + 32 * CH;      // 3072 (ltb_at)
constexpr int KR_QH = 0;                         // bf16 [64][128] (qk_at): q hi
constexpr int KR_KH = KR_QH + CH * DK * 2;       // bf16 [64][128] (qk_at): k hi
constexpr int KR_KTH = KR_KH + CH * DK * 2;      // bf16 [128][64] (sw64): k^T hi
constexpr int KR_KTL = KR_KTH + DK * CH * 2;     // bf16 [128][64] (sw64): k^T lo
constexpr int KR_KLAST = KR_KTL + DK * CH * 2;   // fp32 [128]: rk k of the chunk's last row
constexpr int KR_RQ = KR_KLAST + DK * 4;         // fp32 [64]: rq (with the output scale)
constexpr int KR_KQ = KR_RQ + CH * 4;            // fp32 [64]: rq rk (q.k) of each row
constexpr int KREC_BYTES = KR_KQ + CH * 4;       // 66560
constexpr int VR_LTB = 0;                        // bf16, ltb_at layout: (T - I) diag(beta)
constexpr int VR_BETA = VR_LTB + LTB_ELEMS * 2;  // fp32 [64]
constexpr int VR_GRK = VR_BETA + CH * 4;         // fp32 [64]: e^G rk
// P holds only its tiles on or below the diagonal: the 16 rows of tile row
// tb keep their first 16 (tb + 1) columns, at a row pitch of 24 + 16 tb
// elements (p_row); the pitches are 12, 20, 28 and 36 words, four times an
// odd number, so the 16 rows of an 8-byte operand read start in 16 distinct
// groups of four banks.
__host__ __device__ constexpr int p_pitch(int tb) { return 24 + 16 * tb; }
__host__ __device__ constexpr int p_row(int t) {
    return 16 * (24 * (t >> 4) + 8 * (t >> 4) * ((t >> 4) - 1)) + (t & 15) * p_pitch(t >> 4);
}
constexpr int P_ELEMS = p_row(CH);               // 3072
static_assert(P_ELEMS == 3072 && p_row(63) + 64 <= P_ELEMS, "P tiles on and below the diagonal");
constexpr int VR_PH = VR_GRK + CH * 4;           // bf16, p_row layout: P hi
constexpr int VR_PL = VR_PH + P_ELEMS * 2;       // bf16, p_row layout: P lo
constexpr int VR_GRQ = VR_PL + P_ELEMS * 2;      // fp32 [64]: e^G rq
constexpr int VR_GAM = VR_GRQ + CH * 4;          // fp32 [64]: e^G
constexpr int VR_WDR = VR_GAM + CH * 4;          // fp32 [64]: rk e^{G_last - G}, 0 for the last row
constexpr int VREC_BYTES = VR_WDR + CH * 4;      // 21760, a multiple of 256
static_assert(VREC_BYTES % 256 == 0 && KREC_BYTES % 256 == 0, "records keep 256-byte alignment");
static_assert(VR_WDR + CH * 4 <= VREC_BYTES && KREC_BYTES % 256 == 0 && VREC_BYTES % 256 == 0, "records");

__device__ __forceinline__ int64_t chunk_slot(int seq, int r0, int c) { return (int64_t)seq + (r0 >> 6) + c; }

// LDS layouts of the state kernel's matrix operands.  LDS has 64 four-byte
// banks; an 8-byte read serves 32 consecutive lanes per cycle and a 16-byte
// read the lanes {0-7, 24-31} and {8-15, 16-23} of each half wave (measured
// with the bank-conflict counter).  An MFMA operand read takes row lr = lane
// & 15 and column group lg = lane >> 4.
//  - P's rows (p_row): 8-byte reads of rows 12, 20, 28 or 36 words apart
//    fill all 64 banks for every 32 lanes.
//  - qk_at ([64][128], q and k rows): rows 256 bytes apart, the 8-byte piece
//    XORed with 2 (row & 15); an 8-byte read of 16 rows and two adjacent
//    pieces by 32 lanes covers all 64 banks.
//  - sw64 ([rows][64], k^T, the v tile and rows 32-63 of LTb, read both 8 and 16 bytes wide):
//    rows 128 bytes apart, the 16-byte column group XORed with (row >> 1) & 7;
//    conflict free for both read widths, and for the v conv's 8-byte writes
//    when four consecutive lanes share a channel group (all measured).
__device__ __forceinline__ int sw64(int row, int col) { return row * CH + (col ^ (((row >> 1) & 7) << 3)); }
__device__ __forceinline__ int ktr_at(int row, int col) { return sw64(row, col); }  // k^T [128][64]
__device__ __forceinline__ int qk_at(int row, int col) {
    return row * DK + (((col >> 2) ^ ((row & 15) << 1)) << 2) + (col & 3);
}
// (T - I) diag(beta) is strictly lower triangular, and its row tiles 0 and 1
// are read in columns 0-31 only: rows 0-31 keep 32 columns (64-byte rows,
// the 8-byte piece XORed with 2 ((row >> 2) & 3): rows 16 words apart then
// cover all 64 banks in an 8-byte read of 32 lanes), rows 32-63 all 64
// (sw64 rows, whose banks do not change by starting 2 KiB later).
__host__ __device__ constexpr int ltb_at(int row, int col) {
    return row < 32 ? row * 32 + (((col >> 2) ^ (((row >> 2) & 3) << 1)) << 2) + (col & 3)
                    : 32 * 32 + (row - 32) * CH + (col ^ ((((row - 32) >> 1) & 7) << 3));
}

// Copy BYTES (a multiple of 64) from global memory into LDS with direct
// global->LDS loads, 16 bytes per lane: wave w copies the w-th quarter in
// copy_instrs(BYTES) instructions (the last one partly masked), so every wave
// issues the same, compile-time number of loads.  The loads are
// asynchronous: the reader waits for them (vector-memory counter) and a
// barrier publishes them.
constexpr int copy_instrs(int bytes) { return (bytes / 64 + 63) / 64; }
// One 16-byte direct global->LDS load per lane from sbase + voff (sbase
// wave-uniform, in scalar registers; voff per lane) into LDS byte address
// lds_base + 16 lane, written as an instruction the compiler does not see as
// an LDS write: it would otherwise order every later LDS read after every
// such load in flight (a full vector-memory wait at each read), while the
// kernel orders them itself with counted waits and barriers.  The load has
// no result register; M0 takes the LDS base one wait state before the load.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
                 "s"(lds_base)
                 : "memory", "m0");
}
// A wave-uniform pointer moved to scalar registers (the builtin returns a
// signed 32-bit value: each half is taken back as unsigned before widening).
// A wave-uniform element offset moved to scalar registers; added to a
// kernel-argument pointer it keeps that pointer's global address space (a
// pointer rebuilt from an integer would be addressed as flat memory, whose
// operations also count against the LDS wait counter).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)((hi << 32) | lo);
}
template <typename T> __device__ __forceinline__ T* uniform_ptr(T* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<T*>((uintptr_t)((hi << 32) | lo));
}
template <int BYTES>
__device__ __forceinline__ void copy_to_lds(const unsigned char* src, unsigned char* dst, int wv, int lane) {
    static_assert(BYTES % 64 == 0, "whole 16-byte pieces in four equal shares");
    constexpr int PW = BYTES / 64;  // pieces per wave
    const int w0 = wv * PW;
    const uint32_t base = (uint32_t)(uintptr_t)dst + (uint32_t)w0 * 16u;
    const unsigned char* sw = src + (int64_t)w0 * 16;
#pragma unroll
    for (int j = 0; j < copy_instrs(BYTES); ++j) {
        if (64 * j + lane < PW)
            dma16(uniform_ptr(sw + 1024 * j), 16u * (uint32_t)lane, __builtin_amdgcn_readfirstlane(base + 1024u * j));
    }
}
// q or k rows from a [64][LQK] LDS array into the record's qk_at layout,
// through registers, 16 bytes per thread and pass.
__device__ __forceinline__ void store_qk_rows(const __bf16* src, __bf16* dst, int tid) {
    for (int p = tid; p < CH * (DK / 8); p += NTH) {
        const int r = p / (DK / 8), c = 8 * (p % (DK / 8));
        *reinterpret_cast<u32x4*>(dst + qk_at(r, c)) = *reinterpret_cast<const u32x4*>(src + r * LQK + c);
    }
}

// ---------------------------------------------------------------- prep
template <typename ActT>
__global__ __launch_bounds__(NTH, 2) void k_chunk_prep(const ChunkArgs A, const int nck) {
    // Qh, Kh, Ql, Kl (k^T goes to the record only):
    // under 80 KB with the scalars and taps, so two workgroups share a CU
    __shared__ __attribute__((aligned(16))) unsigned char lds[PREP_LDS];
    __shared__ __attribute__((aligned(16))) float sc[8 * CH];
    __shared__ __attribute__((aligned(16))) float wqk[2 * DK * 4];
    __bf16* Qh = reinterpret_cast<__bf16*>(lds + OFF_QH);
    __bf16* Kh = reinterpret_cast<__bf16*>(lds + OFF_KH);
    __bf16* Ql = reinterpret_cast<__bf16*>(lds + OFF_QL);
    __bf16* Kl = reinterpret_cast<__bf16*>(lds + OFF_KL);
    float* Af = reinterpret_cast<float*>(lds + OFF_QL);    // after Q K^T
    __bf16* Tm = reinterpret_cast<__bf16*>(lds + OFF_KH);  // after Q K^T

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // Chunks are handed out last-first, so the records the state kernel reads
    // first are the last written, the likeliest to be in the last-level cache.
    int bid = blockIdx.x;
    const int ki = bid % A.h_k;
    bid /= A.h_k;
    const int c = nck - 1 - bid / A.n_seqs;
    const int seq = bid % A.n_seqs;
    const int page = A.page_idx[seq];
    // invalid pages and batches are reported by the state kernel
    if (page < 0 || page >= A.conv_n_pages || page >= A.state_n_pages) return;
    const int r0 = A.cu[seq], r1 = A.cu[seq + 1];
    if (r0 < 0 || r1 < r0 || (int64_t)r1 > A.n_rows) return;
    const int T = r1 - r0;
    const int c0 = c * CH;
    if (c0 >= T) return;
    const int n = (T - c0 < CH) ? (T - c0) : CH;
    const bool init = A.has_init ? (A.has_init[seq] != 0) : true;
    const int rr = A.h_v / A.h_k;
    const int64_t C = 2 * (int64_t)A.h_k * DK + (int64_t)A.h_v * A.d_v;
    unsigned char* slot = static_cast<unsigned char*>(A.workspace) +
                          chunk_slot(seq, r0, c) * ((int64_t)A.h_k * KREC_BYTES + (int64_t)A.h_v * VREC_BYTES);
    unsigned char* krec = slot + (int64_t)ki * KREC_BYTES;
    __bf16* KTh = reinterpret_cast<__bf16*>(krec + KR_KTH);  // the record's k^T (the state kernel's)
    __bf16* KTl = reinterpret_cast<__bf16*>(krec + KR_KTL);

    const ActT* __restrict__ X = static_cast<const ActT*>(A.x);
    const ActT* __restrict__ win = static_cast<const ActT*>(A.conv_base) + (int64_t)page * A.conv_page_stride;
    const ActT* Wc = static_cast<const ActT*>(A.conv_w);
    {
        const int64_t gq = tid < DK ? (int64_t)ki * DK + tid : (int64_t)A.h_k * DK + (int64_t)ki * DK + (tid - DK);
#pragma unroll
        for (int e = 0; e < 4; ++e) wqk[4 * tid + e] = LOG2E * to_f32(Wc[gq * 4 + e]);
    }
    // this thread's q/k tile: part (q, then k) = tid >> 7, tokens 8 tgp .. +7,
    // channels 8 cgl .. +7 of the key head
    const int part = tid >> 7, tgp = (tid >> 4) & 7, cgl = tid & 15;
    RowVec<ActT, 8> nqk[11];
    {
        const int64_t gq8 = (int64_t)part * A.h_k * DK + (int64_t)ki * DK + 8 * cgl;
#pragma unroll
        for (int j = 0; j < 11; ++j) {
            const int t = c0 + 8 * tgp - 3 + j;  // < 0 only in the first chunk
            if (t >= 0)
                nqk[j].load(X + (int64_t)(r0 + (t < T ? t : T - 1)) * A.x_stride + gq8);
            else if (init)
                nqk[j].load(win + (int64_t)(3 + t) * C + gq8);
            else
                nqk[j].zero();
        }
    }
    // the gate inputs of the key head's first two value heads (wave 0, lane =
    // token), issued with the x rows so that their latency hides under the conv
    float ga0 = 0.0f, gb0 = 0.0f, ga1 = 0.0f, gb1 = 0.0f;
    if (wv == 0) {
        const int64_t row = (int64_t)(r0 + c0 + (lane < n ? lane : n - 1)) * A.ab_stride + (int64_t)ki * rr;
        ga0 = to_f32(static_cast<const ActT*>(A.a)[row]);
        gb0 = to_f32(static_cast<const ActT*>(A.b)[row]);
        if (rr > 1) {
            ga1 = to_f32(static_cast<const ActT*>(A.a)[row + 1]);
            gb1 = to_f32(static_cast<const ActT*>(A.b)[row + 1]);
        }
    }
    __syncthreads();
    // ---- conv + SiLU of q and k (log2(e)-scaled), hi/lo rows, k^T, norms
    {
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
            if (part) {
                u32x4 h0, h1, l0, l1;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint32_t a = ph[2 * m][ep], b = ph[2 * m + 1][ep];
                    const uint32_t cc = pl[2 * m][ep], d = pl[2 * m + 1][ep];
                    h0[m] = (a & 0xffffu) | (b << 16);
                    h1[m] = (a >> 16) | (b & 0xffff0000u);
                    l0[m] = (cc & 0xffffu) | (d << 16);
                    l1[m] = (cc >> 16) | (d & 0xffff0000u);
                }
                const int ch = 8 * cgl + 2 * ep;
                *reinterpret_cast<u32x4*>(KTh + ktr_at(ch, 8 * tgp)) = h0;
                *reinterpret_cast<u32x4*>(KTh + ktr_at(ch + 1, 8 * tgp)) = h1;
                *reinterpret_cast<u32x4*>(KTl + ktr_at(ch, 8 * tgp)) = l0;
                *reinterpret_cast<u32x4*>(KTl + ktr_at(ch + 1, 8 * tgp)) = l1;
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
    }
    lds_barrier();
    // ---- the key head's record: q hi, k hi, the last row of rk k (the same
    // bits as k^T holds), rq; k^T went there from the conv
    store_qk_rows(reinterpret_cast<const __bf16*>(lds + OFF_QH), reinterpret_cast<__bf16*>(krec + KR_QH), tid);
    store_qk_rows(reinterpret_cast<const __bf16*>(lds + OFF_KH), reinterpret_cast<__bf16*>(krec + KR_KH), tid);
    if (tid < DK) {
        const int d = tid, tl = n - 1;
        reinterpret_cast<float*>(krec + KR_KLAST)[d] =
            sc[SC_RK * CH + tl] * ((float)Kh[tl * LQK + d] + (float)Kl[tl * LQK + d]);
    } else if (tid < DK + CH) {
        reinterpret_cast<float*>(krec + KR_RQ)[tid - DK] = sc[SC_RQ * CH + tid - DK];
    }
    // ---- Q K^T (three-pass hi/lo) and K K^T: the 10 tiles on or below the
    // diagonal, round-robin over the waves, kept in registers for every value head
    const int lr = lane & 15, lg = lane >> 4;
    const int wvs = __builtin_amdgcn_readfirstlane(wv);
    f32x4 accq[3], acck[3];
    int tmt[3], tnt[3];
    for (int idx = wvs, k = 0; k < 3; ++k, idx += 4) {
        tmt[k] = -1;
        tnt[k] = 0;
        accq[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        acck[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (idx >= 10) continue;
        int mt = 0, rem = idx;
        while (rem > mt) { rem -= mt + 1; ++mt; }
        const int nt = rem;
        tmt[k] = mt;
        tnt[k] = nt;
        f32x4 aq = {0.0f, 0.0f, 0.0f, 0.0f}, ak = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int col = 32 * ks + 8 * lg;
            const bf16x8 qh = ld8(Qh, LQK, 16 * mt + lr, col);
            const bf16x8 ql = ld8(Ql, LQK, 16 * mt + lr, col);
            const bf16x8 khm = ld8(Kh, LQK, 16 * mt + lr, col);
            const bf16x8 khn = ld8(Kh, LQK, 16 * nt + lr, col);
            const bf16x8 kln = ld8(Kl, LQK, 16 * nt + lr, col);
            aq = mma32(khn, qh, aq);
            aq = mma32(kln, qh, aq);
            aq = mma32(khn, ql, aq);
            ak = mma32(khn, khm, ak);
        }
        settle(aq, ak);
        accq[k] = aq;
        acck[k] = ak;
    }
    // k_t.q_t from the diagonal tiles (the same for every value head)
    for (int k = 0; k < 3; ++k) {
        if (tmt[k] < 0 || tmt[k] != tnt[k]) continue;
        const int t = 16 * tmt[k] + lr, s0 = 16 * tnt[k] + 4 * lg;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (s0 + j == t) sc[SC_KQ * CH + t] = sc[SC_RQ * CH + t] * sc[SC_RK * CH + t] * accq[k][j];
    }
    lds_barrier();  // every product read of Q, K (token-major) is done; KQ is published
    if (tid < CH) reinterpret_cast<float*>(krec + KR_KQ)[tid] = sc[SC_KQ * CH + tid];
    for (int jv = 0; jv < rr; ++jv) {
        const int h = ki * rr + jv;
        unsigned char* vrec = slot + (int64_t)A.h_k * KREC_BYTES + (int64_t)h * VREC_BYTES;
        // ---- gates and the cumulative decay of this value head: wave 0, lane = token
        if (wv == 0) {
            const int t = lane;
            const int tt = c0 + (t < n ? t : n - 1);
            const int64_t row = (int64_t)(r0 + tt) * A.ab_stride + h;
            const float av = jv == 0 ? ga0 : jv == 1 ? ga1 : to_f32(static_cast<const ActT*>(A.a)[row]);
            const float bv = jv == 0 ? gb0 : jv == 1 ? gb1 : to_f32(static_cast<const ActT*>(A.b)[row]);
            const float exp_alog = expf(A.a_log[h]);
            const float g = t < n ? -exp_alog * softplus(av + A.dt_bias[h]) : 0.0f;
            const float beta = t < n ? sigmoid(bv) : 0.0f;
            float G = g;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(G, off, 64);
                if (lane >= off) G += o;
            }
            const float Glast = __shfl(G, 63, 64);
            const float gam = expf(G);
            const float rk = sc[SC_RK * CH + t];
            sc[SC_G * CH + t] = G * LOG2E;
            sc[SC_BETA * CH + t] = beta;
            sc[SC_GAM * CH + t] = gam;
            // the last row of the chunk enters the state update exactly, not through the MFMA
            const float wdr = (t == n - 1) ? 0.0f : expf(Glast - G) * rk;
            sc[SC_WDR * CH + t] = wdr;
            float* vs = reinterpret_cast<float*>(vrec);
            vs[VR_BETA / 4 + t] = beta;
            vs[VR_GRK / 4 + t] = gam * rk;
            vs[VR_GRQ / 4 + t] = gam * sc[SC_RQ * CH + t];
            vs[VR_GAM / 4 + t] = gam;
            vs[VR_WDR / 4 + t] = wdr;
        }
        lds_barrier();
        // ---- P (to the record) and A (to LDS) from the raw products
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
                const float e = __builtin_amdgcn_exp2f(g2t - g2s[j]);
                const float pv = rqt * rks[j] * accq[k][j] * e;
                const float av = bt * rkt * rks[j] * acck[k][j] * e;
                p[j] = s0 + j < t ? pv : 0.0f;
                a[j] = s0 + j < t ? av : 0.0f;
            }
            uint32_t h0, l0, h1, l1;
            split_pk(p[0], p[1], h0, l0);
            split_pk(p[2], p[3], h1, l1);
            *reinterpret_cast<u32x2*>(vrec + VR_PH + (p_row(t) + s0) * 2) = u32x2{h0, h1};
            *reinterpret_cast<u32x2*>(vrec + VR_PL + (p_row(t) + s0) * 2) = u32x2{l0, l1};
            *reinterpret_cast<f32x4*>(Af + t * LAF + s0) = a;
        }
        lds_barrier();
        // ---- UT transform: diagonal block b = wave by the doubling identity
        {
            const int b = wvs;
            f32x4 nB, ntB, eye;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * lg + j;
                nB[j] = Af[(16 * b + r) * LAF + 16 * b + lr];
                ntB[j] = Af[(16 * b + lr) * LAF + 16 * b + r];
                eye[j] = (r == lr) ? 1.0f : 0.0f;
            }
            const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
            f32x4 Y = nB, Z = ntB;
            f32x4 R = eye - nB;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                f32x4 Yn = mma16(to_bf4(Z), to_bf4(Y), zero);
                f32x4 Zn = mma16(to_bf4(Y), to_bf4(Z), zero);
                Y = Yn;
                Z = Zn;
                R = mma16(to_bf4(eye + Z), to_bf4(R), zero);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) Tm[(16 * b + 4 * lg + j) * LT + 16 * b + lr] = (__bf16)R[j];
        }
        lds_barrier();
        for (int lev = 1; lev < 4; ++lev) {
            if (wvs < 4 - lev) {
                const int cb = wvs, b = wvs + lev;
                const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
                f32x4 Xacc = zero;
                for (int d = cb; d < b; ++d) {
                    const float* ar = Af + (16 * b + lr) * LAF + 16 * d + 4 * lg;
                    const bf16x4 aop = to_bf4(ar[0], ar[1], ar[2], ar[3]);
                    const bf16x4 bop = {Tm[(16 * d + 4 * lg + 0) * LT + 16 * cb + lr],
                                        Tm[(16 * d + 4 * lg + 1) * LT + 16 * cb + lr],
                                        Tm[(16 * d + 4 * lg + 2) * LT + 16 * cb + lr],
                                        Tm[(16 * d + 4 * lg + 3) * LT + 16 * cb + lr]};
                    Xacc = mma16(aop, bop, Xacc);
                }
                const bf16x4 tbb = ld4(Tm, LT, 16 * b + lr, 16 * b + 4 * lg);
                f32x4 Yv = mma16(tbb, to_bf4(Xacc), zero);
#pragma unroll
                for (int j = 0; j < 4; ++j) Tm[(16 * b + 4 * lg + j) * LT + 16 * cb + lr] = (__bf16)(-Yv[j]);
            }
            lds_barrier();
        }
        // LT = T - I (strictly lower), column-scaled by beta
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int e = tid + NTH * pass;
            const int t = e >> 3, s0 = 8 * (e & 7);
            if (t < 32 && s0 >= 32) continue;  // not stored (ltb_at)
            const bf16x8 tv = *reinterpret_cast<const bf16x8*>(Tm + t * LT + s0);
            const f32x4 b0 = *reinterpret_cast<const f32x4*>(sc + SC_BETA * CH + s0);
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(sc + SC_BETA * CH + s0 + 4);
            float lt[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) lt[k] = s0 + k < t ? (float)tv[k] : 0.0f;
            const u32x4 ob = {pack_bf2(lt[0] * b0[0], lt[1] * b0[1]), pack_bf2(lt[2] * b0[2], lt[3] * b0[3]),
                              pack_bf2(lt[4] * b1[0], lt[5] * b1[1]), pack_bf2(lt[6] * b1[2], lt[7] * b1[3])};
            *reinterpret_cast<u32x4*>(vrec + VR_LTB + ltb_at(t, s0) * 2) = ob;
        }
        lds_barrier();  // T, A and the scalars are rewritten by the next value head
    }
}

// ---------------------------------------------------------------- state
// k_chunk_state runs 8 waves per workgroup, two per SIMD.  Waves 0-3 (the
// chain) hold the state and do only what the next chunk's state depends on;
// waves 4-7 (the output side) run the v conv, Q S and the outputs from the
// state and D that the chain hands over in LDS, so the two interleave on
// every SIMD.  Wave w of either side owns value columns 16 (w & 3) .. +15 of
// the block.  A chunk takes two steps, each closed by a barrier:
//   step A(c)  chain:  refill G4 <- chunk c;  D(c) = T diag(beta) (V - diag(e^G rk) K S(c))
//              output: x rows of chunk c+1 -> registers;  Q S(c);  O(c-1)
//   step B(c)  chain:  refill G1 <- chunk c+1;  D(c) -> LDS;  S(c+1);
//                      hi(S(c+1)) -> LDS
//              output: v conv of chunk c+1 -> LDS;  refill G2 <- c+1, G3 <- c
// and O of the last chunk after the loop.  Each refill is issued after the
// barrier that ends the last read of its buffer and is awaited (vector
// memory count 0 in the waves that issued it) before the barrier that
// precedes its first read.
//   G1 (D):           LTb, beta, e^G rk     <- value-head record [0, VR_PH)
//                     k hi                  <- key-head record [KR_KH, KR_KTH)
//   G2 (Q S):         q hi                  <- key-head record [0, KR_KTH)
//   G4 (S update):    k^T hi/lo, klast      <- key-head record [KR_KTH, KR_RQ)
//                     gam, wdr              <- value-head record [VR_GAM, VR_WDR + 256)
//   G3 (P D, output): P hi/lo, e^G rq       <- value-head record [VR_PH, VR_GAM)
//                     kq                    <- key-head record [KR_KQ, KREC_BYTES)
constexpr int SNTH = 512;                              // threads of the state kernel
constexpr int G1V_BYTES = VR_PH;                       // 6656
constexpr int G1K_BYTES = KR_KTH - KR_KH;              // 16384
constexpr int G1_BYTES = G1V_BYTES + G1K_BYTES;
constexpr int G2_BYTES = KR_KH;                        // 16384
constexpr int G4K_BYTES = KR_RQ - KR_KTH;              // 33280
constexpr int G4V_BYTES = VR_WDR + CH * 4 - VR_GAM;    // 512
constexpr int G3V_BYTES = VR_GAM - VR_PH;              // 12544
constexpr int G3K_BYTES = KREC_BYTES - KR_KQ;          // 256
constexpr int XCH_BYTES = 4 * 4 * 64 * 16;             // one 16-byte vector per (chain wave, tile, lane)
static_assert(G1V_BYTES == 6656 && G1K_BYTES == 16384 && G4K_BYTES == 33280 && G3V_BYTES == 12544,
              "refill group sizes");
constexpr int S_LDS = G1_BYTES + 2 * G2_BYTES + G4K_BYTES + G4V_BYTES + G3V_BYTES + G3K_BYTES + 2 * BVC * CH * 2 +
                      2 * XCH_BYTES + BVC * 4 * 4;
static_assert(S_LDS <= 160 * 1024, "state kernel LDS");
// The v taps of channel c sit at 16-byte slot 16 (c & 3) + c / 4, so the
// 16-byte reads of channels 4 vc4 + e (vc4 = 0..15) hit 16 different slots.
__device__ __forceinline__ int tap_at(int c) { return ((c & 3) << 4) | (c >> 2); }

#define GDN_WAIT_VM(n) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory")

template <typename ActT, typename StT>
__global__ __launch_bounds__(SNTH) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_chunk_state(const ChunkArgs A, const int nck) {
    // One LDS object per operand group and hand-over buffer.
    __shared__ __attribute__((aligned(16))) unsigned char g1s[G1_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char g2s[2 * G2_BYTES];  // q rows of chunks c (even, odd)
    __shared__ __attribute__((aligned(16))) unsigned char g4s[G4K_BYTES + G4V_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char g3s[G3V_BYTES + G3K_BYTES];
    __shared__ __attribute__((aligned(16))) __bf16 VTh[BVC * CH];  // v^T hi, sw64
    __shared__ __attribute__((aligned(16))) __bf16 VTl[BVC * CH];  // v^T lo, sw64
    __shared__ __attribute__((aligned(16))) f32x4 Dx[4 * 4 * 64];   // D: (chain wave, row tile, lane)
    __shared__ __attribute__((aligned(16))) bf16x8 Sx[4 * 4 * 64];  // hi(S) operand: (chain wave, k step, lane)
    __shared__ __attribute__((aligned(16))) float wv4[BVC * 4];
    __shared__ int sh_last;
    const __bf16* LTb = reinterpret_cast<const __bf16*>(g1s + VR_LTB);
    const float* sbeta = reinterpret_cast<const float*>(g1s + VR_BETA);
    const float* sgrk = reinterpret_cast<const float*>(g1s + VR_GRK);
    const __bf16* Kr = reinterpret_cast<const __bf16*>(g1s + G1V_BYTES);
    const __bf16* Qh = reinterpret_cast<const __bf16*>(g2s);
    const __bf16* KTh = reinterpret_cast<const __bf16*>(g4s);
    const __bf16* KTl = reinterpret_cast<const __bf16*>(g4s + DK * CH * 2);
    const float* klast = reinterpret_cast<const float*>(g4s + 2 * DK * CH * 2);
    const float* sgam4 = reinterpret_cast<const float*>(g4s + G4K_BYTES);
    const float* swdr = reinterpret_cast<const float*>(g4s + G4K_BYTES + CH * 4);
    const __bf16* Ph = reinterpret_cast<const __bf16*>(g3s);
    const __bf16* Pl = reinterpret_cast<const __bf16*>(g3s + VR_PL - VR_PH);
    const float* sgrq = reinterpret_cast<const float*>(g3s + VR_GRQ - VR_PH);
    const float* skq = reinterpret_cast<const float*>(g3s + G3V_BYTES);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wvs = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool chain = wvs < 4;
    const int w4 = wvs & 3;    // column tile of this wave, either side
    const int t4 = tid & 255;  // thread index within its side
    const int lr = lane & 15, lg = lane >> 4;
    const int nblk = A.d_v / BVC;
    const int rr = A.h_v / A.h_k;
    // The M = rr * nblk workgroups of one (sequence, key head) group read the
    // same key-head record and, in pairs, the same value-head records, chunk
    // by chunk in lockstep.  Consecutive workgroup indices go to the 8 XCDs
    // in turn, so group g's members take indices 8 M (g / 8) + 8 m + (g % 8):
    // one XCD, one L2, dispatched together.
    const int M = rr * nblk;
    const int bx = blockIdx.x;
    const int grp = 8 * (bx / (8 * M)) + (bx % 8);
    const int mem = (bx / 8) % M;
    if (grp >= A.n_seqs * A.h_k) return;
    const int ki = grp % A.h_k;
    const int blk = mem % nblk;
    const int h = ki * rr + mem / nblk;
    // the v-th group row takes the v-th longest sequence (ties by position)
    int seq = grp / A.h_k;
    if (A.n_seqs > 1 && A.n_seqs <= 256) {
        int* len = reinterpret_cast<int*>(Dx);
        const int ns = A.n_seqs;
        int my = 0;
        if (tid < ns) {
            my = A.cu[tid + 1] - A.cu[tid];
            len[tid] = my;
        }
        __syncthreads();
        if (tid < ns) {
            int rank = 0;
            for (int j = 0; j < ns; ++j) {
                const int lj = len[j];
                rank += (lj > my || (lj == my && j < tid)) ? 1 : 0;
            }
            if (rank == seq) sh_last = tid;
        }
        __syncthreads();
        seq = sh_last;
        __syncthreads();
    }
    seq = __builtin_amdgcn_readfirstlane(seq);
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
    const int nch = (T + CH - 1) / CH;
    if (nch > nck) {  // longer than the bound the records were made for
        if (tid == 0 && h == 0 && blk == 0) set_err(A.err, GDN_DEVERR_BATCH);
        return;
    }
    const bool init = A.has_init ? (A.has_init[seq] != 0) : true;
    const int64_t slot_bytes = (int64_t)A.h_k * KREC_BYTES + (int64_t)A.h_v * VREC_BYTES;
    const unsigned char* ws = static_cast<const unsigned char*>(A.workspace);
    auto krec = [&](int c) { return ws + chunk_slot(seq, r0, c) * slot_bytes + (int64_t)ki * KREC_BYTES; };
    auto vrec = [&](int c) {
        return ws + chunk_slot(seq, r0, c) * slot_bytes + (int64_t)A.h_k * KREC_BYTES + (int64_t)h * VREC_BYTES;
    };
    // refills, each split over the four waves of the side that reads it
    auto fill_g1 = [&](int c) {
        copy_to_lds<G1V_BYTES>(vrec(c), g1s, w4, lane);
        copy_to_lds<G1K_BYTES>(krec(c) + KR_KH, g1s + G1V_BYTES, w4, lane);
    };
    auto fill_g4 = [&](int c) {
        copy_to_lds<G4K_BYTES>(krec(c) + KR_KTH, g4s, w4, lane);
        copy_to_lds<G4V_BYTES>(vrec(c) + VR_GAM, g4s + G4K_BYTES, w4, lane);
    };
    auto fill_g2 = [&](int c) { copy_to_lds<G2_BYTES>(krec(c), g2s + (c & 1) * G2_BYTES, w4, lane); };
    auto fill_g3 = [&](int c) {
        copy_to_lds<G3V_BYTES>(vrec(c) + VR_PH, g3s, w4, lane);
        copy_to_lds<G3K_BYTES>(krec(c) + KR_KQ, g3s + G3V_BYTES, w4, lane);
    };

    const ActT* __restrict__ X = static_cast<const ActT*>(A.x);
    ActT* __restrict__ win = static_cast<ActT*>(A.conv_base) + (int64_t)page * A.conv_page_stride;
    const ActT* Wc = static_cast<const ActT*>(A.conv_w);

    // ---- chain: wave w holds S[16 dt + 4 lg + j][16 w + lr], dt = 0..7
    StT* __restrict__ Sg = static_cast<StT*>(A.state) + (int64_t)page * A.state_page_stride +
                           (int64_t)h * DK * A.d_v + colbase + 16 * w4 + lr;
    f32x4 s[8];
    // the hi(S) operand of the chain's products and of the output side's Q S
    auto publish_s = [&](bf16x8 (&sb)[4]) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            sb[kk] = cat8(to_bf4(s[2 * kk]), to_bf4(s[2 * kk + 1]));
            Sx[(w4 * 4 + kk) * 64 + lane] = sb[kk];
        }
    };
    bf16x8 sb[4];

    // ---- output side: v rows and taps; lane l of wave w takes channels
    // 4 vc4 .. +3 (vc4 = l >> 2) and tokens 4 tq4 .. +3 (tq4 = (l & 3) + 4 w)
    // of a chunk
    const int vc4 = lane >> 2, tq4 = (lane & 3) + 4 * w4;
    const int64_t gv = 2 * (int64_t)A.h_k * DK + (int64_t)h * A.d_v + colbase + t4;  // channel t4 (< 64)
    RowVec<ActT, 4> nvv[7];
    auto load_v = [&](int cs) {
        const int64_t gv4 = 2 * (int64_t)A.h_k * DK + (int64_t)h * A.d_v + colbase + 4 * vc4;
        // rows cs - 3 .. cs + 63 (clamped to the sequence) as 32-bit offsets
        // from a wave-uniform base row
        const int tb = cs >= 3 ? cs - 3 : 0;
        const ActT* xb = X + uniform64((int64_t)(r0 + tb) * A.x_stride + 2 * (int64_t)A.h_k * DK +
                                       (int64_t)h * A.d_v + colbase);
#pragma unroll
        for (int j = 0; j < 7; ++j) {
            const int t = cs + 4 * tq4 - 3 + j;
            if (t >= 0)
                nvv[j].load(xb + (uint32_t)(((t < T ? t : T - 1) - tb) * (int)A.x_stride + 4 * vc4));
            else if (init)
                nvv[j].load(win + (int64_t)(3 + t) * C + gv4);
            else
                nvv[j].zero();
        }
    };
    // v conv + SiLU of a chunk from its rows, stored transposed (hi/lo)
    auto conv_v = [&]() {
        u32x2 th[4], tl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int col = 4 * vc4 + e;
            const f32x4 w4v = *reinterpret_cast<const f32x4*>(wv4 + 4 * tap_at(col));
            const float w[4] = {w4v[0], w4v[1], w4v[2], w4v[3]};
            float xv[7];
#pragma unroll
            for (int j = 0; j < 7; ++j) xv[j] = nvv[j].get(e);
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = silu_fast(conv4(w, xv[i], xv[i + 1], xv[i + 2], xv[i + 3]));
            uint32_t h0, l0, h1, l1;
            split_pk(y[0], y[1], h0, l0);
            split_pk(y[2], y[3], h1, l1);
            th[e] = u32x2{h0, h1};
            tl[e] = u32x2{l0, l1};
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int at = sw64(4 * vc4 + e, 4 * tq4);
            *reinterpret_cast<u32x2*>(VTh + at) = th[e];
            *reinterpret_cast<u32x2*>(VTl + at) = tl[e];
        }
    };
    float* __restrict__ Og0 = A.o + (int64_t)r0 * A.h_v * A.d_v + (int64_t)h * A.d_v + colbase;
    const int64_t o_stride = (int64_t)A.h_v * A.d_v;
    const int ocol = 16 * w4 + lr;
    f32x4 qs[4], Dp[4];
    bf16x4 dh[4], dl[4];
    // D of a chunk from the chain (LDS) into registers, with its hi/lo split
    auto take_d = [&]() {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            Dp[mt] = Dx[(w4 * 4 + mt) * 64 + lane];
            split4(Dp[mt], dh[mt], dl[mt]);
        }
    };
    // O of chunk pc (n_p rows) from its Q S (qs), D (Dp, dh, dl) and G3: wave
    // w's column tile, written straight from the accumulator layout (16 lanes
    // = 64 contiguous bytes of one row)
    auto output = [&](int pc, int n_p) {
        // every operand read first (P tiles on and below the diagonal), then the products
        bf16x8 pa[4][2][2];  // [row tile][k step][hi, lo] for the 16x16x32 products
        bf16x4 pd[2][2];     // [even row tile / 2][hi, lo] for the diagonal 16x16x16 products
        f32x4 grq[4], kq[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int prow = p_row(16 * mt) + lr * p_pitch(mt);  // row 16 mt + lr
            const int t0 = 16 * mt + 4 * lg;
            grq[mt] = *reinterpret_cast<const f32x4*>(sgrq + t0);
            kq[mt] = *reinterpret_cast<const f32x4*>(skq + t0);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (2 * kk + 1 > mt) continue;
                pa[mt][kk][0] = cat8(ld4s(Ph + prow + 32 * kk + 4 * lg), ld4s(Ph + prow + 32 * kk + 16 + 4 * lg));
                pa[mt][kk][1] = cat8(ld4s(Pl + prow + 32 * kk + 4 * lg), ld4s(Pl + prow + 32 * kk + 16 + 4 * lg));
            }
            if ((mt & 1) == 0) {
                pd[mt >> 1][0] = ld4s(Ph + prow + 16 * mt + 4 * lg);
                pd[mt >> 1][1] = ld4s(Pl + prow + 16 * mt + 4 * lg);
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
        f32x4 o_tile[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            f32x4 o;
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = grq[mt][j] * qs[mt][j] + kq[mt][j] * Dp[mt][j];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (2 * kk + 1 > mt) continue;
                const bf16x8 bh = cat8(dh[2 * kk], dh[2 * kk + 1]), bl = cat8(dl[2 * kk], dl[2 * kk + 1]);
                o = mma32(pa[mt][kk][0], bh, o);
                o = mma32(pa[mt][kk][0], bl, o);
                o = mma32(pa[mt][kk][1], bh, o);
            }
            if ((mt & 1) == 0) {
                if (mt > 0) settle_v(o);
                o = mma16(pd[mt >> 1][0], dh[mt], o);
                o = mma16(pd[mt >> 1][0], dl[mt], o);
                o = mma16(pd[mt >> 1][1], dh[mt], o);
            }
            o_tile[mt] = o;
        }
        settle4_v(o_tile);  // tiles 1 and 3 end with a 16x16x32 product
        // rows of this chunk as 32-bit offsets from a wave-uniform base
        float* ob = Og0 + uniform64((int64_t)pc * CH * o_stride);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * mt + 4 * lg + j;
                if (t < n_p) ob[(uint32_t)(t * (int)o_stride + ocol)] = o_tile[mt][j];
            }
    };

    // The two sides run separate copies of the chunk loop (their registers
    // never overlap); every barrier of one has its counterpart in the other,
    // in the same order.
    if (chain) {
        // ---- prologue: the state and its hi operand, G1 of the first chunk
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s[dt][j] = init ? to_f32(Sg[(int64_t)(16 * dt + 4 * lg + j) * A.d_v]) : 0.0f;
        publish_s(sb);
        fill_g1(0);
        lds_barrier();  // (the output side's taps)
        GDN_WAIT_VM(0);
        lds_barrier();  // v tile, hi(S), G1 and G2 of chunk 0
        const int colv = 16 * w4 + lr;
        for (int ci = 0; ci < nch; ++ci) {
            const int n = (T - ci * CH < CH) ? (T - ci * CH) : CH;
            // ================================ step A: D = U - W S with W = T diag(beta e^G rk) K, computed
            // as D = T diag(beta) E, E = V - diag(e^G rk) K S: Z = K S, then
            // D = beta E + LTb E with E split hi/lo (LTb = (T - I) diag(beta))
            fill_g4(ci);
            f32x4 Z[4], D[4];
            const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
            // two row tiles at a time: their k reads are issued before their products
#pragma unroll
            for (int mp = 0; mp < 4; mp += 2) {
                bf16x8 ka[2][4];
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2) {
                    const int mt = mp + m2;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        ka[m2][kk] = cat8(ld4s(Kr + qk_at(16 * mt + lr, 32 * kk + 4 * lg)),
                                          ld4s(Kr + qk_at(16 * mt + lr, 32 * kk + 16 + 4 * lg)));
                }
                __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2) {
                    f32x4 z = zero4;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) z = mma32(ka[m2][kk], sb[kk], z);
                    Z[mp + m2] = z;
                }
            }
            // the LTb operands (K index permuted as E's: lane group lg supplies
            // rows 32 ks + 4 lg + 0..3 and 32 ks + 16 + 4 lg + 0..3); LTb is
            // strictly lower triangular, so row tiles 0 and 1 need ks = 0 only
            bf16x8 la[4][2];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (ks > 0 && mt < 2) continue;
                    la[mt][ks] = cat8(ld4s(LTb + ltb_at(16 * mt + lr, 32 * ks + 4 * lg)),
                                      ld4s(LTb + ltb_at(16 * mt + lr, 32 * ks + 16 + 4 * lg)));
                }
            settle4_v(Z);
            bf16x4 eh[4], el[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int t0 = 16 * mt + 4 * lg;
                const bf16x4 vh = *reinterpret_cast<const bf16x4*>(VTh + sw64(colv, t0));
                const bf16x4 vl = *reinterpret_cast<const bf16x4*>(VTl + sw64(colv, t0));
                const f32x4 grk = *reinterpret_cast<const f32x4*>(sgrk + t0);
                const f32x4 bt = *reinterpret_cast<const f32x4*>(sbeta + t0);
                f32x4 e;
#pragma unroll
                for (int j = 0; j < 4; ++j) e[j] = ((float)vh[j] + (float)vl[j]) - grk[j] * Z[mt][j];
                split4(e, eh[mt], el[mt]);
                D[mt] = bt * e;
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 ebh = cat8(eh[2 * ks], eh[2 * ks + 1]), ebl = cat8(el[2 * ks], el[2 * ks + 1]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    if (ks > 0 && mt < 2) continue;
                    D[mt] = mma32(la[mt][ks], ebh, D[mt]);
                    D[mt] = mma32(la[mt][ks], ebl, D[mt]);
                }
            }
            settle4_v(D);
            GDN_WAIT_VM(0);  // G4 of this chunk
            lds_barrier();
            // ================================ step B: hand D over; S <- e^{G_last} S + K^T diag(rk e^{G_last - G}) D
            if (ci + 1 < nch) fill_g1(ci + 1);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) Dx[(w4 * 4 + mt) * 64 + lane] = D[mt];
            bf16x4 wh[4], wl[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const f32x4 wd = *reinterpret_cast<const f32x4*>(swdr + 16 * kt + 4 * lg);
                split4(D[kt] * wd, wh[kt], wl[kt]);
            }
            const int tl = n - 1;
            float dsel = D[3][3];  // row 63 of a full chunk (lanes with lg = 3)
            if (n < CH) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (16 * kt + 4 * lg + j == tl) dsel = D[kt][j];
            }
            const float dlast = __shfl(dsel, ((tl & 15) >> 2) * 16 + lr, 64);
            const float glast = sgam4[tl];
            bf16x8 wh2[2], wl2[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                wh2[kk] = cat8(wh[2 * kk], wh[2 * kk + 1]);
                wl2[kk] = cat8(wl[2 * kk], wl[2 * kk + 1]);
            }
            // k^T operands of four row tiles at a time, read before their products
#pragma unroll
            for (int dh = 0; dh < 8; dh += 4) {
                bf16x8 kh[4][2], kl[4][2];
#pragma unroll
                for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const int row = 16 * (dh + d4) + lr;
                        const int k0 = ktr_at(row, 32 * kk + 4 * lg), k1 = ktr_at(row, 32 * kk + 16 + 4 * lg);
                        kh[d4][kk] = cat8(ld4s(KTh + k0), ld4s(KTh + k1));
                        kl[d4][kk] = cat8(ld4s(KTl + k0), ld4s(KTl + k1));
                    }
                __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
                for (int d4 = 0; d4 < 4; ++d4) {
                    f32x4 acc = s[dh + d4] * glast;
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        acc = mma32(kh[d4][kk], wh2[kk], acc);
                        acc = mma32(kh[d4][kk], wl2[kk], acc);
                        acc = mma32(kl[d4][kk], wh2[kk], acc);
                    }
                    s[dh + d4] = acc;
                }
            }
            settle8_v(s);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const f32x4 kv = *reinterpret_cast<const f32x4*>(klast + 16 * dt + 4 * lg);
#pragma unroll
                for (int j = 0; j < 4; ++j) s[dt][j] = fmaf(kv[j], dlast, s[dt][j]);
            }
            publish_s(sb);
            GDN_WAIT_VM(0);  // G1 of the next chunk
            lds_barrier();
        }
        // ---- the final state
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) Sg[(int64_t)(16 * dt + 4 * lg + j) * A.d_v] = from_f32<StT>(s[dt][j]);
    } else {
        // ---- prologue: taps, the first chunk's v tile, G2 of the first chunk
        if (t4 < BVC) {
#pragma unroll
            for (int e = 0; e < 4; ++e) wv4[4 * tap_at(t4) + e] = to_f32(Wc[gv * 4 + e]);
        }
        load_v(0);
        fill_g2(0);
        lds_barrier();  // taps
        conv_v();
        GDN_WAIT_VM(0);
        lds_barrier();  // v tile, hi(S), G1 and G2 of chunk 0
        for (int ci = 0; ci < nch; ++ci) {
            // ================================ step A: Q S of this chunk, O of the previous one
            if (ci + 1 < nch) load_v((ci + 1) * CH);
            // the next chunk's q rows into the other buffer (last read in the
            // previous step A), after the x rows: loads complete in order, and
            // the v conv waits for the x rows only
            if (ci + 1 < nch) fill_g2(ci + 1);
            const __bf16* Qc = Qh + (ci & 1) * (G2_BYTES / 2);
            f32x4 qn[4];
            bf16x8 sbo[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) sbo[kk] = Sx[(w4 * 4 + kk) * 64 + lane];
#pragma unroll
            for (int mp = 0; mp < 4; mp += 2) {
                bf16x8 qa[2][4];
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2) {
                    const int row = 16 * (mp + m2) + lr;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        qa[m2][kk] = cat8(ld4s(Qc + qk_at(row, 32 * kk + 4 * lg)), ld4s(Qc + qk_at(row, 32 * kk + 16 + 4 * lg)));
                }
                __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2) {
                    f32x4 q = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) q = mma32(qa[m2][kk], sbo[kk], q);
                    qn[mp + m2] = q;
                }
            }
            if (ci > 0) {
                take_d();
                output(ci - 1, CH);
            }
            settle4_v(qn);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) qs[mt] = qn[mt];
            lds_barrier();
            // ================================ step B: refills (under the conv); the next chunk's v tile
            fill_g3(ci);
            if (ci + 1 < nch) conv_v();
            GDN_WAIT_VM(0);  // G2 of the next chunk (issued in step A), G3 of this one
            lds_barrier();
        }
        // ---- the last chunk's outputs (its D and G3 arrived in the last step)
        take_d();
        output(nch - 1, T - (nch - 1) * CH);
    }

    // ---- the rolled windows (this block's v channels; the key head's q/k
    // channels by its first value head's first block: the prep kernel, the
    // only reader of the old q/k window, has finished)
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
    if (!chain && t4 < BVC) roll(gv);
    if (chain && h == ki * rr && blk == 0) {
        const int64_t gq = t4 < DK ? (int64_t)ki * DK + t4 : (int64_t)A.h_k * DK + (int64_t)ki * DK + (t4 - DK);
        roll(gq);
    }
}

template <typename ActT, typename StT>
hipError_t launch_chunk2_t(const ChunkArgs& a, int max_len, hipStream_t s) {
    const int nblk = a.d_v / BVC;
    const int nck = (max_len + CH - 1) / CH;
    const int64_t gprep = (int64_t)a.n_seqs * nck * a.h_k;
    const int64_t groups = (int64_t)a.n_seqs * a.h_k;
    const int64_t gstate = ((groups + 7) / 8) * 8 * ((int64_t)(a.h_v / a.h_k) * nblk);
    if (gstate == 0 || nck == 0) return hipSuccess;
    if (gprep > 0x7fffffff || gstate > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_chunk_prep<ActT>), dim3((unsigned)gprep), dim3(NTH), 0, s, a, nck);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_chunk_state<ActT, StT>), dim3((unsigned)gstate), dim3(SNTH), 0, s, a, nck);
    return hipGetLastError();
}

}  // namespace

bool chunked_supported(int d_k, int d_v, int chunk) { return d_k == DK && d_v > 0 && d_v % BVC == 0 && chunk == CH; }

size_t chunked_workspace_bytes(int h_k, int h_v, int n_seqs, int64_t n_rows) {
    const int64_t slots = (int64_t)n_seqs + (n_rows + CH - 1) / CH;
    return (size_t)slots * ((size_t)h_k * KREC_BYTES + (size_t)h_v * VREC_BYTES);
}

hipError_t launch_chunked(const ChunkArgs& a, int d_k, int act_dtype, int state_dtype, int max_len, hipStream_t s) {
    if (!chunked_supported(d_k, a.d_v, CH)) return hipErrorInvalidValue;
    if (act_dtype == GDN_BF16)
        return state_dtype == GDN_BF16 ? launch_chunk2_t<bf16_t, bf16_t>(a, max_len, s)
                                       : launch_chunk2_t<bf16_t, float>(a, max_len, s);
    return state_dtype == GDN_BF16 ? launch_chunk2_t<float, bf16_t>(a, max_len, s)
                                   : launch_chunk2_t<float, float>(a, max_len, s);
}

}  // namespace gdn
