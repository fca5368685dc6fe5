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
// per workgroup, loaded with 16-byte vector loads straight into registers).
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
template <> struct RowVec<bf16_t, 1> {
    __device__ static void load(const bf16_t* p, float (&v)[1]) { v[0] = to_f32(*p); }
    __device__ static void store(bf16_t* p, const float (&v)[1]) { *p = f32_to_bf16(v[0]); }
};
template <> struct RowVec<bf16_t, 4> {
    __device__ static void load(const bf16_t* p, float (&v)[4]) {
        const u32x2v t = *reinterpret_cast<const u32x2v*>(p);
        v[0] = __uint_as_float(t[0] << 16); v[1] = __uint_as_float(t[0] & 0xffff0000u);
        v[2] = __uint_as_float(t[1] << 16); v[3] = __uint_as_float(t[1] & 0xffff0000u);
    }
    __device__ static void store(bf16_t* p, const float (&v)[4]) {
        const u32x2v t = {(uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                          (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)};
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

// This lane's R rows of a d_k-long LDS row.
template <int R>
__device__ __forceinline__ void lds_rows(const float* row, int tid, float (&out)[R]) {
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
    const float rq = scale / sqrtf(sq + eps);
    const float rk = 1.0f / sqrtf(sk + eps);
    float kq = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        qv[e] *= rq;
        kv[e] *= rk;
        kq = fmaf(kv[e], qv[e], kq);
    }
    float* qd = qrow + l16 * E;
    float* kd = krow + l16 * E;
#pragma unroll
    for (int e = 0; e < E; ++e) { qd[e] = qv[e]; kd[e] = kv[e]; }
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
