// gdn_block.hpp -- workgroup-level pieces shared by the token-by-token and
// verify kernels.
//
// Work layout: one workgroup of 512 threads (8 waves of 64) owns BV = 32*CPL
// state columns of one value head for one sequence (or request).  The 16
// lanes of a DPP row hold the d_k rows of the same CPL columns, R = d_k/16
// rows per lane, so each d_k-long dot product reduces inside the row with
// four DPP steps and no LDS traffic:
//   wave w, lane l:  row group rg = l & 15  (rows rg*R .. rg*R+R-1),
//                    column group cg = 4w + (l >> 4)  (columns cg*CPL .. +CPL-1).
// CPL = 1 suits long token loops (fewest operations per token on the
// critical path); CPL = 4 suits decode and verify (a whole 128-column head
// per workgroup, loaded with 16-byte vector loads straight into registers);
// CPL = 2 serves decode on heads of 64 columns.
#pragma once

#include "gdn_device.hpp"

namespace gdn {

constexpr int BLOCK_THREADS = 512;

__device__ __forceinline__ int lane_rowgroup(int tid) { return tid & 15; }
__device__ __forceinline__ int lane_colgroup(int tid) { return ((tid >> 6) << 2) + ((tid & 63) >> 4); }

// CPL consecutive state elements of one row.
template <typename StT, int CPL> struct RowVec;
template <> struct RowVec<float, 1> {
    __device__ static void load(const float* p, float (&v)[1]) { v[0] = *p; }
    __device__ static void store(float* p, const float (&v)[1]) { *p = v[0]; }
};
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
template <> struct RowVec<float, 4> {
    __device__ static void load(const float* p, float (&v)[4]) {
        const f32x4v t = *reinterpret_cast<const f32x4v*>(p);
        v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
    }
    __device__ static void store(float* p, const float (&v)[4]) {
        const f32x4v t = {v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4v*>(p) = t;
    }
};
template <> struct RowVec<float, 2> {
    __device__ static void load(const float* p, float (&v)[2]) {
        const float2 t = *reinterpret_cast<const float2*>(p);
        v[0] = t.x; v[1] = t.y;
    }
    __device__ static void store(float* p, const float (&v)[2]) {
        *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    }
};
template <> struct RowVec<bf16_t, 1> {
    __device__ static void load(const bf16_t* p, float (&v)[1]) { v[0] = to_f32(*p); }
    __device__ static void store(bf16_t* p, const float (&v)[1]) { *p = f32_to_bf16(v[0]); }
};
template <> struct RowVec<bf16_t, 2> {
    __device__ static void load(const bf16_t* p, float (&v)[2]) {
        const uint32_t t = *reinterpret_cast<const uint32_t*>(p);
        v[0] = __uint_as_float(t << 16); v[1] = __uint_as_float(t & 0xffff0000u);
    }
    __device__ static void store(bf16_t* p, const float (&v)[2]) {
        *reinterpret_cast<uint32_t*>(p) = f32x2_to_bf16x2(v[0], v[1]);
    }
};
template <> struct RowVec<bf16_t, 4> {
    __device__ static void load(const bf16_t* p, float (&v)[4]) {
        const u32x2v t = *reinterpret_cast<const u32x2v*>(p);
        v[0] = __uint_as_float(t[0] << 16); v[1] = __uint_as_float(t[0] & 0xffff0000u);
        v[2] = __uint_as_float(t[1] << 16); v[3] = __uint_as_float(t[1] & 0xffff0000u);
    }
    __device__ static void store(bf16_t* p, const float (&v)[4]) {
        const u32x2v t = {f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2v*>(p) = t;
    }
};

// Load this lane's R x CPL part of a state block; `blk` points at row 0,
// column 0 of the workgroup's block, rows ld elements apart.
template <typename StT, int DK, int CPL>
__device__ __forceinline__ void load_state(const StT* __restrict__ blk, int64_t ld, float (&s)[CPL][DK / 16],
                                           int tid) {
    constexpr int R = DK / 16;
    const StT* p = blk + (int64_t)(lane_rowgroup(tid) * R) * ld + lane_colgroup(tid) * CPL;
#pragma unroll
    for (int m = 0; m < R; ++m) {
        float v[CPL];
        RowVec<StT, CPL>::load(p + (int64_t)m * ld, v);
#pragma unroll
        for (int c = 0; c < CPL; ++c) s[c][m] = v[c];
    }
}

template <typename StT, int DK, int CPL>
__device__ __forceinline__ void store_state(StT* __restrict__ blk, int64_t ld, const float (&s)[CPL][DK / 16],
                                            int tid) {
    constexpr int R = DK / 16;
    StT* p = blk + (int64_t)(lane_rowgroup(tid) * R) * ld + lane_colgroup(tid) * CPL;
#pragma unroll
    for (int m = 0; m < R; ++m) {
        float v[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[c] = s[c][m];
        RowVec<StT, CPL>::store(p + (int64_t)m * ld, v);
    }
}

// ------------------------------------------------------ LDS state staging
// A state block can be fetched into LDS with gfx950's direct global->LDS
// loads, which take no VGPRs while in flight: a workgroup holds one block
// in registers and the next one in LDS at the same time.
//
// Each load instruction of a wave covers one contiguous run of the block
// (fp32: 1 KiB = two rows; bf16: 256 B = one row): HBM serves such runs
// markedly faster than the register layout's 16-row x 64-byte footprint.  The
// lane that lands a piece in LDS is therefore not the lane that computes on
// it, so after every wave's loads have completed a workgroup barrier must
// precede reading, and another must separate reading from the next fetch.
//
// Where a piece lands: the hardware puts lane l of a wave's load at
// wave_base + l * stride (stride 16 for 16-byte loads, 4 for 4-byte ones).
// Which piece a lane loads is ours to choose: within a row the piece index is
// XORed with a function of the row's row group, so that the 16 lanes of a DPP
// row -- 16 row groups, one piece index -- read 16 different LDS banks.
typedef __attribute__((address_space(1))) void gmem_void;
typedef __attribute__((address_space(3))) void lds_void;

// One activation element per lane into LDS.  For 1-, 2- and 4-byte loads
// the hardware places lane l's data at wave_base + 4 l, zero-extended to a
// dword (12- and 16-byte loads use a 16-byte lane stride); LDS_ELEM_SLOT is
// that stride.  A 2-byte element reads back from the low half of its slot.
constexpr int LDS_ELEM_SLOT = 4;
__device__ __forceinline__ void load_lds_elem(const float* g, unsigned char* wave_base) {
    __builtin_amdgcn_global_load_lds((gmem_void*)g, (lds_void*)wave_base, 4, 0, 0);
}
__device__ __forceinline__ void load_lds_elem(const bf16_t* g, unsigned char* wave_base) {
    __builtin_amdgcn_global_load_lds((gmem_void*)g, (lds_void*)wave_base, 2, 0, 0);
}

template <typename StT, int DK, int CPL> struct StateStage;

// fp32, 4 columns (a 128-column block): a row is 32 pieces of 16 bytes.
// Load instruction m of wave w covers rows 2(wR+m) and 2(wR+m)+1; lane l
// takes row 2(wR+m) + l/32, piece (l mod 32) ^ rowgroup(row), and lands at
// m * 8 KiB + w * 1 KiB + 16 l.
template <int DK> struct StateStage<float, DK, 4> {
    static constexpr int R = DK / 16;
    static constexpr int BYTES = R * BLOCK_THREADS * 16;
    __device__ static void fetch(const float* blk, int64_t ld, unsigned char* stage, int tid) {
        const int w = tid >> 6, l = tid & 63;
        unsigned char* wbase = stage + w * 1024;
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const int r = 2 * (w * R + m) + (l >> 5);
            const int piece = (l & 31) ^ ((r / R) & 15);
            __builtin_amdgcn_global_load_lds((gmem_void*)(blk + (int64_t)r * ld + piece * 4),
                                             (lds_void*)(wbase + m * BLOCK_THREADS * 16), 16, 0, 0);
        }
    }
    // This lane's rows rg*R .. rg*R+R-1, piece cg (columns 4cg .. 4cg+3).
    __device__ static void read(const unsigned char* stage, int tid, float (&s)[4][R]) {
        const int rg = lane_rowgroup(tid), cg = lane_colgroup(tid);
#pragma unroll
        for (int mm = 0; mm < R; ++mm) {
            const int r = rg * R + mm;
            const int w = (r >> 1) / R, m = (r >> 1) % R;
            const int l = ((r & 1) << 5) | (cg ^ rg);
            const f32x4v t = *reinterpret_cast<const f32x4v*>(stage + m * BLOCK_THREADS * 16 + w * 1024 + l * 16);
            s[0][mm] = t[0]; s[1][mm] = t[1]; s[2][mm] = t[2]; s[3][mm] = t[3];
        }
    }
};

// bf16, 4 columns: a row is 64 pieces of 4 bytes (two columns each).  Load
// instruction m of wave w covers row 2wR + m; lane l takes piece
// l ^ 2 rowgroup(row) and lands at m * 2 KiB + w * 256 B + 4 l.  A lane's
// four columns 4cg .. 4cg+3 are pieces 2cg and 2cg+1, which stay adjacent.
template <int DK> struct StateStage<bf16_t, DK, 4> {
    static constexpr int R = DK / 16;
    static constexpr int BYTES = 2 * R * BLOCK_THREADS * 4;
    __device__ static void fetch(const bf16_t* blk, int64_t ld, unsigned char* stage, int tid) {
        const int w = tid >> 6, l = tid & 63;
        unsigned char* wbase = stage + w * 256;
#pragma unroll
        for (int m = 0; m < 2 * R; ++m) {
            const int r = 2 * R * w + m;
            const int piece = l ^ (2 * ((r / R) & 15));
            __builtin_amdgcn_global_load_lds((gmem_void*)(blk + (int64_t)r * ld + 2 * piece),
                                             (lds_void*)(wbase + m * BLOCK_THREADS * 4), 4, 0, 0);
        }
    }
    __device__ static void read(const unsigned char* stage, int tid, float (&s)[4][R]) {
        const int rg = lane_rowgroup(tid), cg = lane_colgroup(tid);
#pragma unroll
        for (int mm = 0; mm < R; ++mm) {
            const int r = rg * R + mm;
            const int w = r / (2 * R), m = r % (2 * R);
            const int l = (2 * cg) ^ (2 * rg);
            const u32x2v t = *reinterpret_cast<const u32x2v*>(stage + m * BLOCK_THREADS * 4 + w * 256 + l * 4);
            s[0][mm] = __uint_as_float(t[0] << 16); s[1][mm] = __uint_as_float(t[0] & 0xffff0000u);
            s[2][mm] = __uint_as_float(t[1] << 16); s[3][mm] = __uint_as_float(t[1] & 0xffff0000u);
        }
    }
};

// fp32, 2 columns (a 64-column block): a row is 16 pieces of 16 bytes.
// Load instruction m of wave w covers rows 4(wR/2+m) .. 4(wR/2+m)+3; lane l
// takes row 4(wR/2+m) + l/16, piece (l mod 16) ^ rowgroup(row), and lands at
// m * 8 KiB + w * 1 KiB + 16 l.  A lane's two columns 2cg, 2cg+1 are the
// half (cg mod 2) of piece cg/2.
template <int DK> struct StateStage<float, DK, 2> {
    static constexpr int R = DK / 16;
    static_assert(R % 2 == 0, "four rows per wave load");
    static constexpr int BYTES = R * BLOCK_THREADS * 8;
    __device__ static void fetch(const float* blk, int64_t ld, unsigned char* stage, int tid) {
        const int w = tid >> 6, l = tid & 63;
        unsigned char* wbase = stage + w * 1024;
#pragma unroll
        for (int m = 0; m < R / 2; ++m) {
            const int r = 4 * (w * (R / 2) + m) + (l >> 4);
            const int piece = (l & 15) ^ ((r / R) & 15);
            __builtin_amdgcn_global_load_lds((gmem_void*)(blk + (int64_t)r * ld + piece * 4),
                                             (lds_void*)(wbase + m * BLOCK_THREADS * 16), 16, 0, 0);
        }
    }
    __device__ static void read(const unsigned char* stage, int tid, float (&s)[2][R]) {
        const int rg = lane_rowgroup(tid), cg = lane_colgroup(tid);
#pragma unroll
        for (int mm = 0; mm < R; ++mm) {
            const int r = rg * R + mm;
            const int q = r >> 2, w = q / (R / 2), m = q % (R / 2);
            const int l = ((r & 3) << 4) | ((cg >> 1) ^ rg);
            const float2 t = *reinterpret_cast<const float2*>(stage + m * BLOCK_THREADS * 16 + w * 1024 + l * 16 +
                                                              (cg & 1) * 8);
            s[0][mm] = t.x; s[1][mm] = t.y;
        }
    }
};

// bf16, 2 columns: a row is 32 pieces of 4 bytes (two columns each).  Load
// instruction m of wave w covers rows 2(wR+m) and 2(wR+m)+1; lane l takes
// row 2(wR+m) + l/32, piece (l mod 32) ^ rowgroup(row), and lands at
// m * 2 KiB + w * 256 B + 4 l.  A lane's two columns are piece cg.
template <int DK> struct StateStage<bf16_t, DK, 2> {
    static constexpr int R = DK / 16;
    static constexpr int BYTES = R * BLOCK_THREADS * 4;
    __device__ static void fetch(const bf16_t* blk, int64_t ld, unsigned char* stage, int tid) {
        const int w = tid >> 6, l = tid & 63;
        unsigned char* wbase = stage + w * 256;
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const int r = 2 * (w * R + m) + (l >> 5);
            const int piece = (l & 31) ^ ((r / R) & 15);
            __builtin_amdgcn_global_load_lds((gmem_void*)(blk + (int64_t)r * ld + 2 * piece),
                                             (lds_void*)(wbase + m * BLOCK_THREADS * 4), 4, 0, 0);
        }
    }
    __device__ static void read(const unsigned char* stage, int tid, float (&s)[2][R]) {
        const int rg = lane_rowgroup(tid), cg = lane_colgroup(tid);
#pragma unroll
        for (int mm = 0; mm < R; ++mm) {
            const int r = rg * R + mm;
            const int q = r >> 1, w = q / R, m = q % R;
            const int l = ((r & 1) << 5) | (cg ^ rg);
            const uint32_t t = *reinterpret_cast<const uint32_t*>(stage + m * BLOCK_THREADS * 4 + w * 256 + l * 4);
            s[0][mm] = __uint_as_float(t << 16); s[1][mm] = __uint_as_float(t & 0xffff0000u);
        }
    }
};

// Wait for every vector-memory operation of this wave, direct global->LDS
// loads included.  The compiler does not reliably order reads of LDS
// written by such loads when the loads were issued in an earlier loop
// iteration, so code that stages through LDS waits explicitly.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until this wave's LDS reads have returned, so a following fetch may
// overwrite the slots they read.  The memory clobber keeps the compiler from
// moving those reads past the wait.
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Layout of a d_k-long q or k row in LDS.  Lane g of a 16-lane row owns
// elements g*R .. g*R+R-1 (R = d_k/16).  With d_k = 128 a lane reads its 8
// elements as two 16-byte pieces; stored in element order those pieces sit
// 32 bytes apart across the 16 lanes, so lanes g and g+8 meet in the same
// banks.  The row therefore holds every lane's first piece (elements g*8 ..
// g*8+3 at 4g), then every lane's second piece (g*8+4 .. g*8+7 at 64+4g): each
// read instruction of the 16 lanes covers 256 consecutive bytes.  Smaller
// d_k already read 256 contiguous bytes per instruction in element order.
template <int DK>
__device__ __forceinline__ int qk_pos(int e) {
    if constexpr (DK == 128) return ((e & 7) >> 2) * 64 + (e >> 3) * 4 + (e & 3);
    else return e;
}
// The element stored at position p (the inverse of qk_pos).
template <int DK>
__device__ __forceinline__ int qk_elem(int p) {
    if constexpr (DK == 128) return ((p & 63) >> 2) * 8 + (p >> 6) * 4 + (p & 3);
    else return p;
}

// This lane's R elements of a q or k row in the qk_pos layout.
template <int R>
__device__ __forceinline__ void lds_rows(const float* row, int tid, float (&out)[R]) {
    if constexpr (R == 8) {
        const int g = lane_rowgroup(tid);
        const float4 t0 = *reinterpret_cast<const float4*>(row + 4 * g);
        const float4 t1 = *reinterpret_cast<const float4*>(row + 64 + 4 * g);
        out[0] = t0.x; out[1] = t0.y; out[2] = t0.z; out[3] = t0.w;
        out[4] = t1.x; out[5] = t1.y; out[6] = t1.z; out[7] = t1.w;
        return;
    }
    const float* p = row + lane_rowgroup(tid) * R;
    if constexpr (R % 4 == 0) {
#pragma unroll
        for (int m = 0; m < R; m += 4) {
            const float4 t = *reinterpret_cast<const float4*>(p + m);
            out[m] = t.x; out[m + 1] = t.y; out[m + 2] = t.z; out[m + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int m = 0; m < R; m += 2) {
            const float2 t = *reinterpret_cast<const float2*>(p + m);
            out[m] = t.x; out[m + 1] = t.y;
        }
    }
}

template <int CPL>
__device__ __forceinline__ void lds_cols(const float* row, int tid, float (&out)[CPL]) {
    const float* p = row + lane_colgroup(tid) * CPL;
    if constexpr (CPL == 4) {
        const float4 t = *reinterpret_cast<const float4*>(p);
        out[0] = t.x; out[1] = t.y; out[2] = t.z; out[3] = t.w;
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) out[c] = p[c];
    }
}

// This lane's CPL output columns, one store.
template <int CPL>
__device__ __forceinline__ void store_cols(float* p, const float (&v)[CPL]) {
    if constexpr (CPL == 4) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else if constexpr (CPL == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) p[c] = v[c];
    }
}

// Gating of one token by the 16 lanes of a DPP row (part (b)): L2-normalise
// the post-conv q and k rows of the key head in place (q also takes the output
// scale) and return k-hat . (scale q-hat).  Lane l16 holds elements
// l16*E .. l16*E+E-1 (E = d_k/16); each lane sums its elements with fused
// multiply-adds in order, then reduce16 combines the 16 partial sums.
template <int DK>
__device__ __forceinline__ float gate_qk(float* qrow, float* krow, float scale, float eps, int l16) {
    constexpr int E = DK / 16;
    float qv[E], kv[E];
    lds_rows<E>(qrow + 0, l16, qv);
    lds_rows<E>(krow + 0, l16, kv);
    float sq = 0.0f, sk = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        sq = fmaf(qv[e], qv[e], sq);
        sk = fmaf(kv[e], kv[e], sk);
    }
    sq = reduce16(sq);
    sk = reduce16(sk);
    const float rq = scale * __builtin_amdgcn_rsqf(sq + eps);  // hardware 1/sqrt, about one ulp
    const float rk = __builtin_amdgcn_rsqf(sk + eps);
    float kq = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        qv[e] *= rq;
        kv[e] *= rk;
        kq = fmaf(kv[e], qv[e], kq);
    }
    if constexpr (E == 8) {  // the qk_pos layout of d_k = 128
        *reinterpret_cast<float4*>(qrow + 4 * l16) = make_float4(qv[0], qv[1], qv[2], qv[3]);
        *reinterpret_cast<float4*>(qrow + 64 + 4 * l16) = make_float4(qv[4], qv[5], qv[6], qv[7]);
        *reinterpret_cast<float4*>(krow + 4 * l16) = make_float4(kv[0], kv[1], kv[2], kv[3]);
        *reinterpret_cast<float4*>(krow + 64 + 4 * l16) = make_float4(kv[4], kv[5], kv[6], kv[7]);
    } else {
        float* qd = qrow + l16 * E;
        float* kd = krow + l16 * E;
#pragma unroll
        for (int e = 0; e < E; ++e) { qd[e] = qv[e]; kd[e] = kv[e]; }
    }
    return reduce16(kq);
}

// Decay factor e^g and beta of one (token, value head) (part (b)).
__device__ __forceinline__ void gate_scalars(float a, float b, float exp_alog, float dt_bias, float& eg,
                                             float& beta) {
    const float g = -exp_alog * softplus(a + dt_bias);
    eg = expf(g);
    beta = sigmoid(b);
}

}  // namespace gdn
