// oal_contrib.hip -- causal contribution scores of the q/k dims on gfx950.
//
// Definition (reproduction notes of arXiv 2610.13674, section "核心公式", first display;
// the per-prompt causal statistics that precede the grouping in the method's flowchart):
//   chi[p,h,r] = (1/|Omega_p|) sum_{i} sum_{j<=i} |q[p,h,i,r] k[p,kv,j,r]| / sqrt(d_h)
// with |Omega_p| = T (T+1) / 2 causal pairs, and chi_mean[h,r] the mean over the prompts.
//
// Linear-time form: |q_ir k_jr| = |q_ir| |k_jr|, so the pair sum of a dim is
//   sum_i |q_ir| K_ir,  K_ir = sum_{j<=i} |k_jr|   (an inclusive prefix sum over tokens).
// Split the tokens into 64-row chunks c. With A_c = sum_{i in c} |q_ir|, Ks_c = the chunk's
// sum of |k_jr| and I_c = sum_{i in c} |q_ir| (prefix of |k| inside the chunk up to i),
//   pair sum = sum_c ( I_c + A_c * sum_{c' < c} Ks_c' ).
// The same identity combines any run of consecutive chunks, which is how the per-chunk
// partials are folded in two levels below.
//
// The work is a stream over q and k (every byte read once) with a few flops per element:
// bound by HBM bandwidth, so the kernels are plain VALU code with 16-byte coalesced loads.
//   oal_chi_partials -- one workgroup per (sequence, KV head, 64-token chunk). Each wave
//                       loads the K chunk (lane = 8 dims x 8 consecutive rows), forms the
//                       in-chunk prefix of |k| (thread-local over its 8 rows, then a scan
//                       over the 8 lanes that share its dims), and for each of its query
//                       heads reduces I_c and A_c over the rows. Waves split the query heads
//                       of the KV head; the K chunk is re-read by each wave from L2.
//   oal_chi_combine  -- one workgroup per (sequence, query head); lane = dim. Each wave
//                       folds a contiguous quarter of the chunks, wave 0 folds the quarters
//                       in order and scales by 1 / (sqrt(d) |Omega|).
//   oal_chi_mean     -- the prompt mean, summed in prompt order (deterministic).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "oal.h"
#include "oal_internal.h"

namespace {

constexpr int kChunk = 64;    // tokens per chunk partial
constexpr int kRowsPerLane = 8;
constexpr int kWaves = 4;

typedef unsigned int oal_u32x4 __attribute__((ext_vector_type(4)));
typedef float oal_f32x4v __attribute__((ext_vector_type(4)));

// 8 consecutive elements of a row, kept in their input format until used.
template <typename T> struct Raw8;

template <> struct Raw8<__bf16> {
    oal_u32x4 w;
    __device__ inline void load(const __bf16 *p) { w = *reinterpret_cast<const oal_u32x4 *>(p); }
    __device__ inline void zero() { w = oal_u32x4{0u, 0u, 0u, 0u}; }
    __device__ inline float get(int e) const {   // e is a compile-time index after unrolling
        unsigned int x = w[e >> 1];
        return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
    }
};

template <> struct Raw8<float> {
    oal_f32x4v a, b;
    __device__ inline void load(const float *p) {
        a = reinterpret_cast<const oal_f32x4v *>(p)[0];
        b = reinterpret_cast<const oal_f32x4v *>(p)[1];
    }
    __device__ inline void zero() { a = b = oal_f32x4v{0.0f, 0.0f, 0.0f, 0.0f}; }
    __device__ inline float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// Partials of one (sequence, KV head, chunk): [Ks 64][I_0 64][A_0 64] ... [I_{rep-1}][A_{rep-1}].
__host__ __device__ inline size_t part_floats(int n_rep) { return (size_t)OAL_D * (1 + 2 * n_rep); }

template <typename T>
__global__ __launch_bounds__(256) void oal_chi_partials(int T_len, int n_q_heads, int n_kv_heads,
                                                        int nchunks, const T *__restrict__ q,
                                                        const T *__restrict__ k,
                                                        float *__restrict__ part) {
    const int c = blockIdx.x, bkv = blockIdx.y;
    const int b = bkv / n_kv_heads, kv = bkv % n_kv_heads;
    const int n_rep = n_q_heads / n_kv_heads;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nwaves = blockDim.x >> 6;
    const int seg = lane & 7, rho = lane >> 3;   // dims 8*seg.., rows 8*rho.. of the chunk
    const int row0 = c * kChunk + rho * kRowsPerLane;
    const int nrows = min(kRowsPerLane, max(0, T_len - row0));

    float *pc = part + ((size_t)bkv * nchunks + c) * part_floats(n_rep);

    // K rows -> prefix of |k| over this lane's rows
    const T *kb = k + ((size_t)bkv * T_len + row0) * OAL_D + 8 * seg;
    Raw8<T> kr[kRowsPerLane];
#pragma unroll
    for (int u = 0; u < kRowsPerLane; ++u) {
        if (u < nrows) kr[u].load(kb + (size_t)u * OAL_D);
        else kr[u].zero();
    }
    // first query head's rows, requested before the scan
    int hh = wave;
    Raw8<T> qa[kRowsPerLane];
    auto load_q = [&](int head, Raw8<T> (&dst)[kRowsPerLane]) {
        const T *qb = q + (((size_t)b * n_q_heads + kv * n_rep + head) * T_len + row0) * OAL_D + 8 * seg;
#pragma unroll
        for (int u = 0; u < kRowsPerLane; ++u) {
            if (u < nrows) dst[u].load(qb + (size_t)u * OAL_D);
            else dst[u].zero();
        }
    };
    if (hh < n_rep) load_q(hh, qa);

    float kp[kRowsPerLane][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) kp[0][e] = fabsf(kr[0].get(e));
#pragma unroll
    for (int u = 1; u < kRowsPerLane; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) kp[u][e] = kp[u - 1][e] + fabsf(kr[u].get(e));
    // inclusive scan of the lane totals over rho (lanes seg + 8 rho), then shift by one lane
    float inc[8], exc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) inc[e] = kp[kRowsPerLane - 1][e];
#pragma unroll
    for (int dl = 1; dl < 8; dl <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float y = __shfl_up(inc[e], 8 * dl);
            if (rho >= dl) inc[e] += y;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float y = __shfl_up(inc[e], 8);
        exc[e] = rho >= 1 ? y : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kRowsPerLane; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) kp[u][e] += exc[e];
    if (wave == 0 && rho == 7) {
        float4 *dst = reinterpret_cast<float4 *>(pc + 8 * seg);
        dst[0] = make_float4(inc[0], inc[1], inc[2], inc[3]);
        dst[1] = make_float4(inc[4], inc[5], inc[6], inc[7]);
    }

    for (; hh < n_rep; hh += nwaves) {
        float I[8], A[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = fabsf(qa[0].get(e));
            I[e] = x * kp[0][e];
            A[e] = x;
        }
#pragma unroll
        for (int u = 1; u < kRowsPerLane; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = fabsf(qa[u].get(e));
                I[e] = fmaf(x, kp[u][e], I[e]);
                A[e] += x;
            }
        // the next head's rows are requested while this one is reduced and stored
        if (hh + nwaves < n_rep) load_q(hh + nwaves, qa);
#pragma unroll
        for (int off = 8; off < 64; off <<= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                I[e] += __shfl_xor(I[e], off);
                A[e] += __shfl_xor(A[e], off);
            }
        if (rho == 0) {
            float4 *di = reinterpret_cast<float4 *>(pc + OAL_D * (1 + 2 * hh) + 8 * seg);
            float4 *da = reinterpret_cast<float4 *>(pc + OAL_D * (2 + 2 * hh) + 8 * seg);
            di[0] = make_float4(I[0], I[1], I[2], I[3]);
            di[1] = make_float4(I[4], I[5], I[6], I[7]);
            da[0] = make_float4(A[0], A[1], A[2], A[3]);
            da[1] = make_float4(A[4], A[5], A[6], A[7]);
        }
    }
}

__global__ __launch_bounds__(256) void oal_chi_combine(int n_q_heads, int n_kv_heads, int nchunks,
                                                       float scale, const float *__restrict__ part,
                                                       float *__restrict__ chi) {
    __shared__ float s_t[kWaves][OAL_D], s_a[kWaves][OAL_D], s_k[kWaves][OAL_D];
    const int bh = blockIdx.x;
    const int b = bh / n_q_heads, h = bh % n_q_heads;
    const int n_rep = n_q_heads / n_kv_heads;
    const int kv = h / n_rep, hh = h % n_rep;
    const int wave = threadIdx.x >> 6, r = threadIdx.x & 63;
    const size_t stride = part_floats(n_rep);
    const float *pb = part + (size_t)(b * n_kv_heads + kv) * nchunks * stride;
    const int per = (nchunks + kWaves - 1) / kWaves;
    const int c0 = wave * per, c1 = min(nchunks, c0 + per);
    float t = 0.0f, a = 0.0f, ks = 0.0f;   // folded pair sum, sum of A, sum of Ks
    constexpr int U = 8;
    for (int cb = c0; cb < c1; cb += U) {
        float vi[U], va[U], vk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (cb + u < c1) {
                const float *pc = pb + (size_t)(cb + u) * stride;
                vk[u] = pc[r];
                vi[u] = pc[OAL_D * (1 + 2 * hh) + r];
                va[u] = pc[OAL_D * (2 + 2 * hh) + r];
            } else {
                vk[u] = vi[u] = va[u] = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            t += vi[u] + va[u] * ks;
            ks += vk[u];
            a += va[u];
        }
    }
    s_t[wave][r] = t;
    s_a[wave][r] = a;
    s_k[wave][r] = ks;
    __syncthreads();
    if (wave == 0) {
        float tot = 0.0f, kex = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            tot += s_t[w][r] + s_a[w][r] * kex;
            kex += s_k[w][r];
        }
        chi[(size_t)bh * OAL_D + r] = tot * scale;
    }
}

__global__ __launch_bounds__(64) void oal_chi_mean(int batch, int n_q_heads, const float *__restrict__ chi,
                                                   float *__restrict__ chi_mean) {
    const int h = blockIdx.x, r = threadIdx.x;
    float s = 0.0f;
    for (int b = 0; b < batch; ++b) s += chi[((size_t)b * n_q_heads + h) * OAL_D + r];
    chi_mean[(size_t)h * OAL_D + r] = s / (float)batch;
}

template <typename T>
hipError_t launch(const oal_dims &d, int T_len, const void *q, const void *k, void *ws, float *chi,
                  float *chi_mean, hipStream_t stream) {
    const int n_rep = d.n_q_heads / d.n_kv_heads;
    const int nchunks = (T_len + kChunk - 1) / kChunk;
    const int nw = n_rep < kWaves ? n_rep : kWaves;
    float *part = reinterpret_cast<float *>(ws);
    hipLaunchKernelGGL((oal_chi_partials<T>), dim3(nchunks, d.batch * d.n_kv_heads), dim3(64 * nw), 0,
                       stream, T_len, d.n_q_heads, d.n_kv_heads, nchunks,
                       reinterpret_cast<const T *>(q), reinterpret_cast<const T *>(k), part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // 1 / (sqrt(d) |Omega|), |Omega| = T (T+1) / 2, rounded once
    const double n_pairs = (double)T_len * ((double)T_len + 1.0) / 2.0;
    const float scale = (float)(1.0 / (8.0 * n_pairs));
    hipLaunchKernelGGL(oal_chi_combine, dim3(d.batch * d.n_q_heads), dim3(64 * kWaves), 0, stream,
                       d.n_q_heads, d.n_kv_heads, nchunks, scale, part, chi);
    e = hipGetLastError();
    if (e != hipSuccess || !chi_mean) return e;
    hipLaunchKernelGGL(oal_chi_mean, dim3(d.n_q_heads), dim3(OAL_D), 0, stream, d.batch, d.n_q_heads,
                       chi, chi_mean);
    return hipGetLastError();
}

}  // namespace

size_t oal_contribution_ws_bytes_impl(const oal_dims &d, int T_len) {
    const int n_rep = d.n_q_heads / d.n_kv_heads;
    const size_t nchunks = ((size_t)T_len + kChunk - 1) / kChunk;
    size_t bytes = (size_t)d.batch * d.n_kv_heads * nchunks * part_floats(n_rep) * sizeof(float);
    return (bytes + 255) / 256 * 256;
}

hipError_t oal_launch_contribution(const oal_dims &d, int T_len, const void *q, const void *k, void *ws,
                                   float *chi, float *chi_mean, hipStream_t stream) {
    if (d.dtype == OAL_BF16) return launch<__bf16>(d, T_len, q, k, ws, chi, chi_mean, stream);
    return launch<float>(d, T_len, q, k, ws, chi, chi_mean, stream);
}
