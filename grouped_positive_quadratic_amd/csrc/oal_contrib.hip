// oal_contrib.hip -- causal contribution scores of the q/k dims on gfx950.
//
// Definition (reproduction notes of arXiv 2610.13674, section "核心公式", first display;
// the per-prompt causal statistics that precede the grouping in the method's flowchart):
//   chi[p,h,r] = (1/|Omega_p|) sum_{i} sum_{j<=i} |q[p,h,i,r] k[p,kv,j,r]| / sqrt(d_h)
// with |Omega_p| = T (T+1) / 2 causal pairs, and chi_mean[h,r] the mean over the prompts.
//
// Linear-time form: |q_ir k_jr| = |q_ir| |k_jr|, so the pair sum of a dim is
//   sum_i |q_ir| K_ir,  K_ir = sum_{j<=i} |k_jr|   (an inclusive prefix sum over tokens).
// For a run of consecutive tokens R keep (P_R, A_R, K_R): the pair sum inside R, the sum of
// |q_ir| and the sum of |k_jr| over R. Two adjacent runs R, S (R first) fold into
//   P = P_R + P_S + A_S K_R,  A = A_R + A_S,  K = K_R + K_S,
// and the whole prompt is the fold of its runs in token order; chi is its P / (sqrt(d)|Omega|).
//
// The work is a stream over q and k with a few flops per element: bound by HBM bandwidth,
// plain VALU code with 16-byte coalesced loads, one kernel per call:
//   * a workgroup takes one query head and a range of 32*RS tokens; each lane (8 dims x one
//     "stream" of RS consecutive tokens) loads its K and Q rows at once and runs the prefix
//     sequentially, so no cross-lane scan is needed;
//   * the 32 streams are folded through LDS (8 per wave, then the 4 waves) into the range's
//     (P, A, K), published at agent scope;
//   * the last workgroup of a (prompt, head) to arrive (arrival counter) folds the ranges in
//     order and writes chi; the last prompt of a head to arrive writes the prompt mean,
//     summing the prompts in order (deterministic, no float atomics). Counters are two-level
//     on purpose: a single counter per head, hit by every workgroup of the head, serialises
//     its atomics and delays the whole kernel.
//   The n_rep workgroups of one (KV head, range) read the same K rows: their ids are spaced
//   8 apart so that they land on the same XCD (workgroups are dealt to the 8 XCDs round-robin)
//   and the K rows come from that XCD's L2 after the first read.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "oal.h"
#include "oal_device.h"
#include "oal_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kStreams = 32;    // token streams per workgroup: 4 waves x 8 lanes per dim group
constexpr int kXcds = 8;
constexpr int kCounterStride = 32;   // unsigned ints between arrival counters (one 128-byte line each)

typedef unsigned int oal_u32x4 __attribute__((ext_vector_type(4)));
typedef float oal_f32x4v __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes from `base` (raw, stride 0): a load whose offset is past
// the end returns zero, which is how the rows past the last token are masked.
__device__ inline __amdgpu_buffer_rsrc_t oal_rsrc(const void *base, unsigned int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// 8 consecutive elements of a row, kept in their input format until used.
template <typename T> struct Raw8;

template <> struct Raw8<__bf16> {
    oal_u32x4 w;
    __device__ inline void load(__amdgpu_buffer_rsrc_t r, int byte_off) {
        w = __builtin_bit_cast(oal_u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
    }
    __device__ inline void zero() { w = oal_u32x4{0u, 0u, 0u, 0u}; }
    __device__ inline float get(int e) const {   // e is a compile-time index after unrolling
        unsigned int x = w[e >> 1];
        return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
    }
};

template <> struct Raw8<float> {
    oal_f32x4v a, b;
    __device__ inline void load(__amdgpu_buffer_rsrc_t r, int byte_off) {
        a = __builtin_bit_cast(oal_f32x4v, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
        b = __builtin_bit_cast(oal_f32x4v, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off + 16, 0, 0));
    }
    __device__ inline void zero() { a = b = oal_f32x4v{0.0f, 0.0f, 0.0f, 0.0f}; }
    __device__ inline float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// Tokens per stream (RS), requested in NB batches of RL rows (16-byte loads): 64 VGPRs of K
// and Q rows per batch keeps four workgroups per CU resident.
template <typename T> struct ChiRows;
template <> struct ChiRows<__bf16> { static constexpr int RL = 8, NB = 2, RS = RL * NB; };
template <> struct ChiRows<float> { static constexpr int RL = 4, NB = 2, RS = RL * NB; };

__device__ inline void st_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_agent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// fold of (P, A, K) with a later run (p, a, k)
__device__ inline void fold(float &P, float &A, float &K, float p, float a, float k) {
    P += p + a * K;
    A += a;
    K += k;
}

template <typename T>
__global__ __launch_bounds__(kThreads, 4) void oal_chi_kernel(
    int T_len, int batch, int n_q_heads, int n_kv_heads, int nrange, int nunits, float scale,
    const T *__restrict__ q, const T *__restrict__ k, float *__restrict__ part,
    unsigned int *__restrict__ counters, float *__restrict__ chi, float *__restrict__ chi_mean) {
    constexpr int RS = ChiRows<T>::RS;
    constexpr int RB = kStreams * RS;
    __shared__ __attribute__((aligned(16))) float s_st[3][kStreams][OAL_D];   // per stream: P, A, K
    __shared__ float s_w[3][4][OAL_D];           // per wave
    __shared__ int s_last;
    const int n_rep = n_q_heads / n_kv_heads;
    // id = ((u / 8) * n_rep + hh) * 8 + u % 8: the heads of unit u share its XCD
    const int id = blockIdx.x;
    const int rest = id / kXcds;
    const int hh = rest % n_rep;
    const int u = (rest / n_rep) * kXcds + id % kXcds;
    if (u >= nunits) return;
    const int bkv = u / nrange, rg = u % nrange;
    const int b = bkv / n_kv_heads, kv = bkv % n_kv_heads, h = kv * n_rep + hh;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int seg = lane & 7, stream = wave * 8 + (lane >> 3);
    const int row0 = rg * RB + stream * RS;

    // 1. this lane's stream: 8 dims x RS consecutive tokens, rows past the end read as zero
    const __amdgpu_buffer_rsrc_t kr_src =
        oal_rsrc(k + (size_t)bkv * T_len * OAL_D, (unsigned int)((size_t)T_len * OAL_D * sizeof(T)));
    const __amdgpu_buffer_rsrc_t qr_src =
        oal_rsrc(q + ((size_t)b * n_q_heads + h) * T_len * OAL_D, (unsigned int)((size_t)T_len * OAL_D * sizeof(T)));
    const int off0 = (row0 * OAL_D + 8 * seg) * (int)sizeof(T);
    constexpr int RL = ChiRows<T>::RL;
    float P[8], A[8], K[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) P[e] = A[e] = K[e] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < ChiRows<T>::NB; ++nb) {
        Raw8<T> kr[RL], qr[RL];
#pragma unroll
        for (int t = 0; t < RL; ++t) {
            const int off = off0 + (nb * RL + t) * OAL_D * (int)sizeof(T);
            kr[t].load(kr_src, off);
            qr[t].load(qr_src, off);
        }
#pragma unroll
        for (int t = 0; t < RL; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                K[e] += fabsf(kr[t].get(e));          // prefix of |k| up to and including this row
                float x = fabsf(qr[t].get(e));
                P[e] = fmaf(x, K[e], P[e]);
                A[e] += x;
            }
        // keep the next batch's loads behind this batch's arithmetic (register budget)
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
        *reinterpret_cast<float4 *>(&s_st[0][stream][8 * seg + e]) = make_float4(P[e], P[e + 1], P[e + 2], P[e + 3]);
        *reinterpret_cast<float4 *>(&s_st[1][stream][8 * seg + e]) = make_float4(A[e], A[e + 1], A[e + 2], A[e + 3]);
        *reinterpret_cast<float4 *>(&s_st[2][stream][8 * seg + e]) = make_float4(K[e], K[e + 1], K[e + 2], K[e + 3]);
    }
    __syncthreads();
    // 2. fold the streams: each wave its 8 (lane = dim), then wave 0 the 4 waves
    {
        float p = 0.0f, a = 0.0f, kk = 0.0f;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
            const int st = wave * 8 + s8;
            fold(p, a, kk, s_st[0][st][lane], s_st[1][st][lane], s_st[2][st][lane]);
        }
        s_w[0][wave][lane] = p;
        s_w[1][wave][lane] = a;
        s_w[2][wave][lane] = kk;
    }
    __syncthreads();
    float *pp = part + ((size_t)u * n_rep + hh) * 3 * OAL_D;
    if (wave == 0) {
        float p = 0.0f, a = 0.0f, kk = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) fold(p, a, kk, s_w[0][w][lane], s_w[1][w][lane], s_w[2][w][lane]);
        st_agent(pp + lane, p);
        st_agent(pp + OAL_D + lane, a);
        st_agent(pp + 2 * OAL_D + lane, kk);
    }
    // 3. arrival: the last range of a (prompt, head) to arrive folds its ranges in order and
    //    writes chi. The agent-scope stores and loads are coherent across the XCDs' L2 caches;
    //    the storing wave waits for its stores to complete before the barrier that precedes
    //    the counter RMW, so they are performed before it (no L2 write-back). Each counter has
    //    a 128-byte line of its own.
    oal_wait_own_stores();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    const int bh = b * n_q_heads + h;
    if (tid == 0) {
        unsigned int old = __hip_atomic_fetch_add(counters + (size_t)bh * kCounterStride, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == (unsigned int)(nrange - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    {
        // wave w folds a contiguous quarter of the ranges, 8 requested at a time
        const int per = (nrange + 3) / 4;
        const int r0 = wave * per, r1 = min(nrange, r0 + per);
        float p = 0.0f, a = 0.0f, kk = 0.0f;
        const size_t ustride = (size_t)n_rep * 3 * OAL_D;
        const float *pb = part + ((size_t)bkv * nrange * n_rep + hh) * 3 * OAL_D + lane;
        for (int rb = r0; rb < r1; rb += 8) {
            float v[8][3];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const size_t o = (size_t)min(rb + j, r1 - 1) * ustride;   // clamped: always valid
#pragma unroll
                for (int c = 0; c < 3; ++c) v[j][c] = ld_agent(pb + o + c * OAL_D);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool in = rb + j < r1;
                fold(p, a, kk, in ? v[j][0] : 0.0f, in ? v[j][1] : 0.0f, in ? v[j][2] : 0.0f);
            }
        }
        s_w[0][wave][lane] = p;
        s_w[1][wave][lane] = a;
        s_w[2][wave][lane] = kk;
    }
    __syncthreads();
    if (wave == 0) {
        float p = 0.0f, a = 0.0f, kk = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) fold(p, a, kk, s_w[0][w][lane], s_w[1][w][lane], s_w[2][w][lane]);
        st_agent(chi + (size_t)bh * OAL_D + lane, p * scale);
    }
    if (tid == 0)
        __hip_atomic_store(counters + (size_t)bh * kCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!chi_mean) return;
    // 4. arrival per head: the last prompt writes the mean over prompts, in prompt order (its
    //    chi stores completed before the counter RMW, as above)
    oal_wait_own_stores();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    unsigned int *hc = counters + ((size_t)batch * n_q_heads + h) * kCounterStride;
    if (tid == 0) {
        unsigned int old = __hip_atomic_fetch_add(hc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == (unsigned int)(batch - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (wave == 0) {
        float sum = 0.0f;
        for (int b0 = 0; b0 < batch; b0 += 16) {
            float v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                v[j] = ld_agent(chi + ((size_t)min(b0 + j, batch - 1) * n_q_heads + h) * OAL_D + lane);
#pragma unroll
            for (int j = 0; j < 16; ++j) sum += (b0 + j < batch) ? v[j] : 0.0f;
        }
        chi_mean[(size_t)h * OAL_D + lane] = sum / (float)batch;
    }
    if (tid == 0) __hip_atomic_store(hc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct ChiLayout {
    int nrange, nunits;
    size_t counter_bytes, part_bytes;
};

template <typename T> ChiLayout chi_layout(const oal_dims &d, int T_len) {
    constexpr int RB = kStreams * ChiRows<T>::RS;
    const int n_rep = d.n_q_heads / d.n_kv_heads;
    ChiLayout l;
    l.nrange = (T_len + RB - 1) / RB;
    l.nunits = d.batch * d.n_kv_heads * l.nrange;
    l.counter_bytes = (((size_t)d.batch * d.n_q_heads + d.n_q_heads) * kCounterStride * sizeof(unsigned int) + 255) / 256 * 256;
    l.part_bytes = (size_t)l.nunits * n_rep * 3 * OAL_D * sizeof(float);
    return l;
}

template <typename T>
hipError_t launch(const oal_dims &d, int T_len, const void *q, const void *k, void *ws, float *chi,
                  float *chi_mean, hipStream_t stream) {
    const ChiLayout l = chi_layout<T>(d, T_len);
    const int n_rep = d.n_q_heads / d.n_kv_heads;
    unsigned int *counters = reinterpret_cast<unsigned int *>(ws);
    float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + l.counter_bytes);
    const long long nblocks = (long long)(l.nunits + kXcds - 1) / kXcds * kXcds * n_rep;
    // 1 / (sqrt(d) |Omega|), |Omega| = T (T+1) / 2, rounded once
    const double n_pairs = (double)T_len * ((double)T_len + 1.0) / 2.0;
    const float scale = (float)(1.0 / (8.0 * n_pairs));
    hipLaunchKernelGGL((oal_chi_kernel<T>), dim3((unsigned int)nblocks), dim3(kThreads), 0, stream, T_len,
                       d.batch, d.n_q_heads, d.n_kv_heads, l.nrange, l.nunits, scale,
                       reinterpret_cast<const T *>(q), reinterpret_cast<const T *>(k), part, counters,
                       chi, chi_mean);
    return hipGetLastError();
}

}  // namespace

size_t oal_contribution_ws_bytes_impl(const oal_dims &d, int T_len) {
    const ChiLayout l = d.dtype == OAL_BF16 ? chi_layout<__bf16>(d, T_len) : chi_layout<float>(d, T_len);
    return l.counter_bytes + (l.part_bytes + 255) / 256 * 256;
}

hipError_t oal_launch_contribution(const oal_dims &d, int T_len, const void *q, const void *k, void *ws,
                                   float *chi, float *chi_mean, hipStream_t stream) {
    if (d.dtype == OAL_BF16) return launch<__bf16>(d, T_len, q, k, ws, chi, chi_mean, stream);
    return launch<float>(d, T_len, q, k, ws, chi, chi_mean, stream);
}
