// oal_device.h -- gfx950 device helpers: MFMA fragments over a 32-wide K-step.
//
// A 16x16 output tile is built from K-steps of 32: in every K-step, lane l of the wave
// owns operand row/column (l % 16) and the 8 K-positions e = 0..7 of lane group g = l / 16.
//   bf16 operands: one v_mfma_f32_16x16x32_bf16 (K = 8 g + e).
//   fp32 operands: eight v_mfma_f32_16x16x4_f32, the e-th using K-position g.
// Both orders put the same 32 products into the same accumulator, so every kernel below is
// written once for both operand types. Accumulator layout (both): lane l holds column
// l % 16 and rows 4 (l / 16) + i, i = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 oal_bf16x8 __attribute__((ext_vector_type(8)));
typedef float oal_f32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct OalFrag;

template <> struct OalFrag<__bf16> {
    oal_bf16x8 v;
    __device__ inline void set(const float (&x)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)x[e];
    }
    __device__ inline void zero() {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)0.0f;
    }
    __device__ inline void load(const void *p) { v = *reinterpret_cast<const oal_bf16x8 *>(p); }
    __device__ inline void store(void *p) const { *reinterpret_cast<oal_bf16x8 *>(p) = v; }
    // two groups of 4 consecutive elements (8-byte aligned each)
    __device__ inline void load4x2(const __bf16 *p0, const __bf16 *p1) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 a = *reinterpret_cast<const bf16x4 *>(p0);
        bf16x4 b = *reinterpret_cast<const bf16x4 *>(p1);
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
    }
    static constexpr int kBytes = 16;  // per lane
};

template <> struct OalFrag<float> {
    float v[8];
    __device__ inline void set(const float (&x)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = x[e];
    }
    __device__ inline void zero() {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
    __device__ inline void load(const void *p) {
        const float4 *q = reinterpret_cast<const float4 *>(p);
        float4 a = q[0], b = q[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    __device__ inline void store(void *p) const {
        float4 *q = reinterpret_cast<float4 *>(p);
        q[0] = make_float4(v[0], v[1], v[2], v[3]);
        q[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
    __device__ inline void load4x2(const float *p0, const float *p1) {
        float4 a = *reinterpret_cast<const float4 *>(p0);
        float4 b = *reinterpret_cast<const float4 *>(p1);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    static constexpr int kBytes = 32;
};

__device__ inline oal_f32x4 oal_mma(const OalFrag<__bf16> &a, const OalFrag<__bf16> &b, oal_f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ inline oal_f32x4 oal_mma(const OalFrag<float> &a, const OalFrag<float> &b, oal_f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
    return c;
}

template <typename T> __device__ inline float oal_ld(const T *p);
template <> __device__ inline float oal_ld<float>(const float *p) { return *p; }
template <> __device__ inline float oal_ld<__bf16>(const __bf16 *p) { return (float)*p; }

__device__ inline oal_f32x4 oal_splat(float x) {
    oal_f32x4 r;
    r[0] = x; r[1] = x; r[2] = x; r[3] = x;
    return r;
}

// Cross-workgroup publish (the decode and contribution combines): a workgroup stores its
// partial sums with agent-scope atomic stores, which are coherent across the XCDs' L2
// caches, then one thread counts the workgroup in with an agent-scope RMW on an arrival
// counter. The stores of every wave must be performed before that RMW: each wave waits for
// its own outstanding stores (gfx9 counts stores in vmcnt; this is s_waitcnt vmcnt(0) with
// the other counters left at their maxima, expcnt 7 and lgkmcnt 15) before the barrier that
// precedes the RMW. A release fence at agent scope would do the same and also write back the
// whole L2 (full of the state rows the decode just wrote), which costs far more.
__device__ inline void oal_wait_own_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// An empty asm statement that clobbers memory: loads issued before it cannot be moved after
// it. Without it the optimizer turns a prefetch ring (load in step k, use in step k + d) back
// into load-and-use in step k + d (the loads' sources are read-only and unaliased, so moving
// a load to its use is legal), and every step then waits for its own loads.
__device__ inline void oal_pin_loads() { asm volatile("" ::: "memory"); }

