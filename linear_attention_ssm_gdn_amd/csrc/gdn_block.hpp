// gdn_block.hpp -- workgroup-level pieces shared by the token-by-token and
// verify kernels.
//
// Work layout: one workgroup of 256 threads (4 waves of 64) owns one value
// head's BV = 32 state columns for one sequence (or request).  In the
// recurrence every lane holds R = d_k/8 rows of one column: lane l of wave
// w owns column 8w + (l >> 3) and rows (l & 7)*R .. (l & 7)*R + R - 1, so
// the d_k-long dot products reduce inside an aligned group of 8 lanes with
// three DPP steps and no LDS round trip.  State blocks move between HBM and
// this layout through an LDS stage so that global accesses stay 16-byte and
// row-contiguous.
#pragma once

#include "gdn_device.hpp"

namespace gdn {

constexpr int BLOCK_THREADS = 256;
constexpr int BV = 32;  // value columns per workgroup

__device__ __forceinline__ int lane_col(int tid) { return ((tid >> 6) << 3) + ((tid & 63) >> 3); }
__device__ __forceinline__ int lane_rowgroup(int tid) { return tid & 7; }

// 16-byte vector of state elements.
template <typename StT> struct Vec16;
template <> struct Vec16<float> {
    static constexpr int N = 4;
    __device__ static void load(const float* p, float (&v)[4]) {
        const float4 t = *reinterpret_cast<const float4*>(p);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    }
    __device__ static void store(float* p, const float (&v)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};
template <> struct Vec16<bf16_t> {
    static constexpr int N = 8;
    __device__ static void load(const bf16_t* p, float (&v)[8]) {
        const uint4 t = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ static void store(bf16_t* p, const float (&v)[8]) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
        *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
};

constexpr int STAGE_LD = BV + 1;  // padded LDS row of the state stage

// Load a d_k x BV state block (row stride ld elements) into the lane layout.
// `stage` holds DK * STAGE_LD floats; the call ends with a barrier so the
// stage may be reused.
template <typename StT, int DK>
__device__ __forceinline__ void load_state_block(const StT* __restrict__ src, int64_t ld, float* stage,
                                                 float (&s)[DK / 8], int tid) {
    using V = Vec16<StT>;
    constexpr int TPR = BV / V::N;             // threads per row
    constexpr int RPP = BLOCK_THREADS / TPR;   // rows per pass
    const int c = (tid % TPR) * V::N;
    for (int r = tid / TPR; r < DK; r += RPP) {
        float v[V::N];
        V::load(src + (int64_t)r * ld + c, v);
#pragma unroll
        for (int e = 0; e < V::N; ++e) stage[r * STAGE_LD + c + e] = v[e];
    }
    __syncthreads();
    constexpr int R = DK / 8;
    const int col = lane_col(tid), rb = lane_rowgroup(tid) * R;
#pragma unroll
    for (int m = 0; m < R; ++m) s[m] = stage[(rb + m) * STAGE_LD + col];
    __syncthreads();
}

// Store the lane-layout block back (rounded to StT); ends with a barrier.
template <typename StT, int DK>
__device__ __forceinline__ void store_state_block(StT* __restrict__ dst, int64_t ld, float* stage,
                                                  const float (&s)[DK / 8], int tid) {
    using V = Vec16<StT>;
    constexpr int R = DK / 8;
    const int col = lane_col(tid), rb = lane_rowgroup(tid) * R;
#pragma unroll
    for (int m = 0; m < R; ++m) stage[(rb + m) * STAGE_LD + col] = s[m];
    __syncthreads();
    constexpr int TPR = BV / V::N;
    constexpr int RPP = BLOCK_THREADS / TPR;
    const int c = (tid % TPR) * V::N;
    for (int r = tid / TPR; r < DK; r += RPP) {
        float v[V::N];
#pragma unroll
        for (int e = 0; e < V::N; ++e) v[e] = stage[r * STAGE_LD + c + e];
        V::store(dst + (int64_t)r * ld + c, v);
    }
    __syncthreads();
}

// Gating of one token by one wave (part (b)): L2-normalise the post-conv q
// and k rows of the key head in place (q also takes the output scale) and
// return k-hat . (scale q-hat).  Reduction order is fixed: each lane sums its
// elements lane, lane+64, ... with fused multiply-adds, then a 64-lane
// butterfly.
template <int DK>
__device__ __forceinline__ float gate_qk(float* qrow, float* krow, float scale, float eps, int lane) {
    constexpr int J = (DK + 63) / 64;
    float qv[J], kv[J];
    float sq = 0.0f, sk = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int e = lane + 64 * j;
        qv[j] = (e < DK) ? qrow[e] : 0.0f;
        kv[j] = (e < DK) ? krow[e] : 0.0f;
        sq = fmaf(qv[j], qv[j], sq);
        sk = fmaf(kv[j], kv[j], sk);
    }
    sq = reduce64(sq);
    sk = reduce64(sk);
    const float rq = scale / sqrtf(sq + eps);
    const float rk = 1.0f / sqrtf(sk + eps);
    float kq = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int e = lane + 64 * j;
        const float qn = qv[j] * rq, kn = kv[j] * rk;
        if (e < DK) { qrow[e] = qn; krow[e] = kn; }
        kq = fmaf(kn, qn, kq);
    }
    return reduce64(kq);
}

// Decay factor e^g and beta of one (token, value head) (part (b)).
__device__ __forceinline__ void gate_scalars(float a, float b, float exp_alog, float dt_bias, float& eg,
                                             float& beta) {
    const float g = -exp_alog * softplus(a + dt_bias);
    eg = expf(g);
    beta = sigmoid(b);
}

}  // namespace gdn
