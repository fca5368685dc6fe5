// gdn_device.hpp -- device helpers shared by the libgdn kernels (gfx950).
//
// Everything here is arithmetic the kernels must perform identically
// wherever the same value is produced, so that the one-page verify, the
// per-candidate-slot verify and the token-by-token sequence kernel agree
// bit for bit: one conv op order, one reduction tree per quantity, one
// gating formula and one state-update formula.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Activation / state element types: fp32 as float, bf16 as its raw bits.
using bf16_t = uint16_t;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN), by gfx950's
// conversion instruction (v_cvt_pk_bf16_f32), one instruction per pair.
typedef float gdn_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 gdn_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
// Two values converted together and packed, a in the low half.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((gdn_f32x2){a, b}, gdn_bf16x2));
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// Round through the storage type (identity for fp32).
template <typename T> __device__ __forceinline__ float round_as(float v) { return to_f32(from_f32<T>(v)); }

// ------------------------------------------------------------- gating (b)
// SiLU(z) = z / (1 + e^{-z}).
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
// The fused kernels' SiLU: the hardware exponential and reciprocal (about one
// ulp each, so a few ulp overall).  Every token-by-token kernel (sequence,
// streaming decode, verify) uses this one, which keeps them bit-identical to
// each other.
__device__ __forceinline__ float silu_hw(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// softplus(u) = log(1 + e^u); for u > 20 it equals u to within 2e-9 relative.
__device__ __forceinline__ float softplus(float u) { return u > 20.0f ? u : log1pf(expf(u)); }

__device__ __forceinline__ float sigmoid(float b) { return 1.0f / (1.0f + expf(-b)); }

// Depthwise causal conv of one channel, width 4: acc = 0, then one fused
// multiply-add per tap, oldest row first (x3 oldest ... x0 newest).
__device__ __forceinline__ float conv4(const float w[4], float x3, float x2, float x1, float x0) {
    float acc = fmaf(w[0], x3, 0.0f);
    acc = fmaf(w[1], x2, acc);
    acc = fmaf(w[2], x1, acc);
    acc = fmaf(w[3], x0, acc);
    return acc;
}

// ------------------------------------------------------------- reductions
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of an aligned DPP row; every lane of the row
// receives the same bits.  Tree: xor 1, xor 2, mirrored half-row (the other
// quad of the 8), mirrored row (the other 8):
//   (((x0+x1)+(x2+x3)) + ((x4+x5)+(x6+x7))) + (same over x8..x15).
__device__ __forceinline__ float reduce16(float x) {
    x = x + dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    x = x + dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    x = x + dpp_mov<0x141>(x);  // row_half_mirror
    x = x + dpp_mov<0x140>(x);  // row_mirror
    return x;
}

// Butterfly sum over the 64 lanes of a wave; every lane receives the same bits.
__device__ __forceinline__ float reduce64(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = x + __shfl_xor(x, m, 64);
    return x;
}

// --------------------------------------------------- the delta rule (c)
// One token of the gated delta rule for CPL state columns.  The 16 lanes of
// a DPP row together hold the d_k = 16R rows of each of their columns; this
// lane holds rows rg*R .. rg*R+R-1 (rg = lane & 15) of CPL columns.
// k, q: this lane's rows of k-hat and scale*q-hat.  Per column, a single pass
// over S_{t-1}: u = S^T k and w = S^T q (each lane: even rows and odd rows in
// two fused multiply-add chains, then reduce16), then
//   delta = beta (v - e^g u),  o = e^g w + (k.q) delta,
//   S <- e^g S + k delta^T.
// The operations per column do not depend on CPL, so every kernel built on
// this function produces the same bits for the same column.  update = false
// (uniform across the workgroup) gives the same o and leaves S as it was, for
// a token whose successor state nothing reads.
template <int R, int CPL>
__device__ __forceinline__ void delta_step(float (&s)[CPL][R], const float (&k)[R], const float (&q)[R],
                                           const float (&v)[CPL], float eg, float beta, float kq,
                                           float (&o)[CPL], bool update = true) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        float u0 = 0.0f, u1 = 0.0f, w0 = 0.0f, w1 = 0.0f;
#pragma unroll
        for (int m = 0; m < R; m += 2) {
            u0 = fmaf(s[c][m], k[m], u0);
            w0 = fmaf(s[c][m], q[m], w0);
            if (m + 1 < R) {
                u1 = fmaf(s[c][m + 1], k[m + 1], u1);
                w1 = fmaf(s[c][m + 1], q[m + 1], w1);
            }
        }
        const float u = reduce16(u0 + u1);
        const float w = reduce16(w0 + w1);
        const float d = beta * (v[c] - eg * u);
        o[c] = fmaf(kq, d, eg * w);
        if (update) {
#pragma unroll
            for (int m = 0; m < R; ++m) s[c][m] = fmaf(k[m], d, eg * s[c][m]);
        }
    }
}

// Replay variant: the same state update without the output.
template <int R, int CPL>
__device__ __forceinline__ void delta_update(float (&s)[CPL][R], const float (&k)[R], const float (&v)[CPL],
                                             float eg, float beta) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        float u0 = 0.0f, u1 = 0.0f;
#pragma unroll
        for (int m = 0; m < R; m += 2) {
            u0 = fmaf(s[c][m], k[m], u0);
            if (m + 1 < R) u1 = fmaf(s[c][m + 1], k[m + 1], u1);
        }
        const float u = reduce16(u0 + u1);
        const float d = beta * (v[c] - eg * u);
#pragma unroll
        for (int m = 0; m < R; ++m) s[c][m] = fmaf(k[m], d, eg * s[c][m]);
    }
}

// ---------------------------------------------------------- arrival count
// Workgroup arrival on a device-scope counter that returns to zero: the
// last of `group` arrivals (in any order) gets true and resets the word.
// Call from one thread after a workgroup barrier that follows every read the
// arrival stands for, with each read value already consumed (so the loads
// have completed).  No data moves between workgroups through memory inside
// the kernel: the last arrival only writes what the others have finished
// reading, and the end of the kernel publishes those writes.  The atomic is
// therefore relaxed; an acquire/release at device scope would write back and
// invalidate the whole L2 of the XCD for every workgroup.
__device__ __forceinline__ bool arrive_last(uint32_t* word, uint32_t group) {
    const uint32_t prev = __hip_atomic_fetch_add(word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev + 1u == group) {
        __hip_atomic_store(word, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    }
    return false;
}

// Split form of the same arrival for callers that want the atomic's result
// late: arrive() issues it, arrived_last() (same thread, later) decides and
// resets.  Reading the result is a wait on the vector-memory counter, which
// completes in order, so reading it early would also wait for every load
// issued before the atomic.
// Relaxed device-scope fetch-add by one lane whose result is read later.  A
// zero offset passed through an empty asm hides that the address is uniform:
// for a uniform address the compiler rewrites a one-lane atomic into a
// wave-aggregated one plus a prefix sum, and that rewrite reads the result
// right after issuing it.
__device__ __forceinline__ uint32_t fetch_add_late(uint32_t* word, uint32_t v) {
    uint32_t zero = 0;
    asm volatile("" : "+v"(zero));
    return __hip_atomic_fetch_add(word + zero, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t arrive(uint32_t* word) { return fetch_add_late(word, 1u); }
__device__ __forceinline__ bool arrived_last(uint32_t* word, uint32_t prev, uint32_t group) {
    if (prev + 1u == group) {
        __hip_atomic_store(word, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    }
    return false;
}

// ------------------------------------------------- ordering-light helpers
// Workgroup barrier that orders LDS only: wait for this wave's LDS
// accesses, then s_barrier.  __syncthreads() (and a workgroup fence, even one
// restricted to LDS) also waits for outstanding vector-memory operations --
// global stores, and direct global->LDS loads, which count as LDS writes --
// and with an in-order counter that means every load in flight, including a
// prefetch of the next block.  Use where waves exchange data through plain
// LDS reads and writes alone.  The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Workgroup-uniform loads through the scalar unit.  The compiler only picks
// scalar loads when it can prove nothing earlier in the kernel stored to the
// address; these are read-only kernel inputs, but a loop that also stores
// defeats that proof and the fallback (a vector load, then a wait) stalls on
// every vector load in flight.  `p` must be uniform and 4-byte aligned.
__device__ __forceinline__ uint32_t sload_u32(const void* p) {
    uint32_t v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
}
// Several such loads in flight together, one wait: a[i] = *p[i].
template <int N>
__device__ __forceinline__ void sload_u32_n(const void* const (&p)[N], uint32_t (&a)[N]);
template <>
__device__ __forceinline__ void sload_u32_n<6>(const void* const (&p)[6], uint32_t (&a)[6]) {
    asm volatile(
        "s_load_dword %0, %6, 0x0\n\t"
        "s_load_dword %1, %7, 0x0\n\t"
        "s_load_dword %2, %8, 0x0\n\t"
        "s_load_dword %3, %9, 0x0\n\t"
        "s_load_dword %4, %10, 0x0\n\t"
        "s_load_dword %5, %11, 0x0\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&s"(a[0]), "=&s"(a[1]), "=&s"(a[2]), "=&s"(a[3]), "=&s"(a[4]), "=&s"(a[5])
        : "s"(p[0]), "s"(p[1]), "s"(p[2]), "s"(p[3]), "s"(p[4]), "s"(p[5])
        : "memory");
}
template <>
__device__ __forceinline__ void sload_u32_n<8>(const void* const (&p)[8], uint32_t (&a)[8]) {
    asm volatile(
        "s_load_dword %0, %8, 0x0\n\t"
        "s_load_dword %1, %9, 0x0\n\t"
        "s_load_dword %2, %10, 0x0\n\t"
        "s_load_dword %3, %11, 0x0\n\t"
        "s_load_dword %4, %12, 0x0\n\t"
        "s_load_dword %5, %13, 0x0\n\t"
        "s_load_dword %6, %14, 0x0\n\t"
        "s_load_dword %7, %15, 0x0\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&s"(a[0]), "=&s"(a[1]), "=&s"(a[2]), "=&s"(a[3]), "=&s"(a[4]), "=&s"(a[5]), "=&s"(a[6]), "=&s"(a[7])
        : "s"(p[0]), "s"(p[1]), "s"(p[2]), "s"(p[3]), "s"(p[4]), "s"(p[5]), "s"(p[6]), "s"(p[7])
        : "memory");
}
__device__ __forceinline__ int32_t sload_i32(const int32_t* p) { return (int32_t)sload_u32(p); }
__device__ __forceinline__ float sload_f32(const float* p) { return __uint_as_float(sload_u32(p)); }
// One byte: the aligned dword that holds it (same page, so always mapped).
__device__ __forceinline__ uint32_t sload_u8(const uint8_t* p) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return (sload_u32(reinterpret_cast<const void*>(a & ~(uintptr_t)3)) >> ((a & 3u) * 8u)) & 0xffu;
}

__device__ __forceinline__ void set_err(int32_t* err, uint32_t bit) {
    if (err) __hip_atomic_fetch_or(err, (int32_t)bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace gdn
