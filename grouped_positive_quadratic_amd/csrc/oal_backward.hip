// oal_backward.hip -- gfx950 kernels of the prefill backward: dq, dk, dv (and the gradients of
// the kernel coefficients L, eps, and of the incoming prefix state) of sum(dy * y) for the
// causal attention y of a prefill that continues from a given (or an empty) prefix state.
//
// The forward (reproduction notes of arXiv 2610.13674, section "核心公式": the kernel kappa,
// the H-state recurrence and the readout u~ = phi(q) . H, y = u~[0:64] / u~[64]) is
//   u_i = sum_{j <= i} kappa_ij [v_j; 1],  kappa_ij = phi_h(q_i) . psi(k_j)
// with psi(k) = [1, k_r, k_r k_t (r <= t)] and phi_h(q) = wdec_h o [1, q_r, q_r q_t]. Its
// backward, by the chain rule through the chunked form of the same sum:
//   g_i       = (dy_i / den_i, -(dy_i . y_i) / den_i)          (65 values per query and head)
//   dkappa_ij = g_i . [v_j; 1]
//   dq_i = Jphi_h(q_i)^T (S_c g_i)         + sum_{j <= i, same chunk} dkappa_ij dkappa_ij/dq_i
//   dv_j = (R_c^T psi(k_j))[0:64]          + sum_h sum_{i >= j, same chunk} kappa_ij g_i[0:64]
//   dk_j = Jpsi(k_j)^T (R_c [v_j; 1])      + sum_h sum_{i >= j, same chunk} dkappa_ij dkappa_ij/dk_j
// where S_c is the incoming state S_0 plus psi(k_j) [v_j; 1]^T summed over the chunks before c
// (the forward's prefix state) and R_c sums phi_h(q_i) g_i^T over the chunks after c and the
// query heads h of the KV head; the gradient of S_0 is that sum over every chunk.
// Inside a chunk kappa is taken from its z-terms, as in the forward's intra-chunk part:
//   z_m = [m = 0] L00 + sum_r Lz[m][r] q_r k_r,   kappa = eps + sum_{m <= G} z_m^2,
//   dkappa/dq_r = 2 k_r sum_m z_m Lz[m][r]        (and the same with q and k exchanged);
// for a (query tile, key tile) pair each z-term is the product (Q o Lz[m]) K^T on MFMA.
//
// Every kernel computes to fp32 accuracy (inputs of either dtype are widened on load). The
// state contractions (the readout's u, the increments, the state parts of dq, dk and dv) and
// most products over the pairs inside a chunk run on bf16 MFMA (v_mfma_f32_16x16x32_bf16) with
// every fp32 operand split in three bf16 parts and up to six products per fp32 product (split3
// below); the rest of the intra-chunk products of dk, dv run on fp32 MFMA
// (v_mfma_f32_16x16x4_f32). With packed fp32 off, the VALU bound is the non-packed FMA rate
// (256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz = 78.6 TFLOP/s); fp32 MFMA reaches 157.3,
// bf16 MFMA 2500 (about 417 for the six-term fp32 products).
//
// Launch order (all on the caller's stream):
//   1. oal_bwd_increments<keys>:    per chunk psi(K_c)^T [V_c; 1]           -> workspace states
//   2. oal_bwd_scan (forward):      exclusive prefix over chunks: S_c
//   3. oal_bwd_readout_g:           u_i (inter + intra), y, den -> g_i     -> workspace g
//   4. oal_bwd_dstate_x6, oal_bwd_dq_intra_mfma: dq (state part, then the pairs inside the
//      chunk)
//   5. oal_bwd_dkv_intra_mfma:      dk, dv partials of the pairs inside the chunk
//   6. oal_bwd_increments<queries>: per chunk sum_h phi_h(Q_c)^T G_c       -> workspace states
//   7. oal_bwd_scan (reverse):      exclusive suffix over chunks: R_c
//   8. oal_bwd_dstate_x6<keys>, oal_bwd_dv_x6: dk, dv partials of the state part
//   9. oal_bwd_kv_reduce:           dk, dv (the partials added in a fixed order)
// With coefficient gradients, also oal_bwd_dw_intra (before 6), the per-head partials of 6,
// and oal_bwd_dw_sum, oal_bwd_coef (after 6): dL, deps.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <type_traits>

#include "oal_device.h"
#include "oal_internal.h"

namespace {

constexpr int kThreads = 256;                 // four waves
constexpr int kFeatBlock = 128;               // features per increment workgroup
constexpr int kIncThreads = 512;              // its eight waves, 16 features each
constexpr int kDkSplits = 4;                  // dk state part: its t steps over 4 workgroups

__device__ inline const OalHeadDev *bwd_head(const unsigned char *params, int h) {
    return reinterpret_cast<const OalHeadDev *>(params + sizeof(OalParamsHeader) + (size_t)h * OAL_HEAD_BYTES);
}

__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// first feature of the quadratic row r, minus r: feature (r, t) is quad_base(r) + t
__device__ inline int quad_base(int r) { return 1 + OAL_D + r * OAL_D - (r * (r - 1)) / 2 - r; }







// 16-byte loads of a row segment as fp32: 8 bf16 or 4 fp32 elements.
template <typename T> struct RowVec;
template <> struct RowVec<__bf16> {
    static constexpr int N = 8;
    __device__ static inline void load(const __bf16 *p, float *out) {
        const oal_bf16x8 x = *reinterpret_cast<const oal_bf16x8 *>(p);
#pragma unroll
        for (int u = 0; u < 8; ++u) out[u] = (float)x[u];
    }
};
template <> struct RowVec<float> {
    static constexpr int N = 4;
    __device__ static inline void load(const float *p, float *out) {
        const float4 x = *reinterpret_cast<const float4 *>(p);
        out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    }
};

// Element slot s (0..15) of this thread in a 64 x 64 tile loaded with RowVec<T>: row n, column col.
template <typename T>
__device__ inline void tile_slot(int s, int &n, int &col) {
    constexpr int N = RowVec<T>::N, PER = 64 / N;       // vectors per row
    const int e = threadIdx.x + kThreads * (s / N);
    n = e / PER;
    col = (e % PER) * N + s % N;
}

// This thread's 16 elements of rows t0 .. t0 + 63 (zero past T) of a [*, T, 64] tensor.
template <typename T>
__device__ inline void load_tile(float (&out)[16], const T *src, size_t row0, int t0, int T_len) {
    constexpr int N = RowVec<T>::N;
#pragma unroll
    for (int m = 0; m < 16 / N; ++m) {
        int n, col;
        tile_slot<T>(m * N, n, col);
        if (t0 + n < T_len) {
            RowVec<T>::load(src + (row0 + t0 + n) * OAL_D + col, out + m * N);
        } else {
#pragma unroll
            for (int u = 0; u < N; ++u) out[m * N + u] = 0.0f;
        }
    }
}

template <typename T>
__device__ inline void store_tile(float *dst, int stride, const float (&in)[16]) {
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        int n, col;
        tile_slot<T>(s, n, col);
        dst[n * stride + col] = in[s];
    }
}

// Stage 64 rows (tokens t0 .. t0 + 63, zero past T) of a [*, T, 64] tensor into LDS with the
// given row stride, as fp32; column 64 (if the stride has room) gets `one`.
// One 16-byte vector at a time, so that only a vector's worth of registers is live (the
// callers hold large accumulator arrays).
template <typename T>
__device__ inline void stage_rows(float *dst, int stride, const T *src, size_t row0, int t0, int T_len, float one) {
    constexpr int N = RowVec<T>::N;
#pragma unroll 1
    for (int m = 0; m < 16 / N; ++m) {
        int n, col;
        tile_slot<T>(m * N, n, col);
        float tmp[N];
        if (t0 + n < T_len) {
            RowVec<T>::load(src + (row0 + t0 + n) * OAL_D + col, tmp);
        } else {
#pragma unroll
            for (int u = 0; u < N; ++u) tmp[u] = 0.0f;
        }
#pragma unroll
        for (int u = 0; u < N; ++u) dst[n * stride + col + u] = tmp[u];
    }
    if (stride > 64 && threadIdx.x < 64) dst[threadIdx.x * stride + 64] = one;
}

// Stage 64 rows of g (64 values from gv, the 65th from gd; zero past T) with row stride 68.
__device__ inline void stage_g(float *dst, const float *gv, const float *gd, size_t row0, int t0, int T_len) {
    stage_rows(dst, 68, gv, row0, t0, T_len, 0.0f);
    if (threadIdx.x < 64) dst[threadIdx.x * 68 + 64] = t0 + (int)threadIdx.x < T_len ? gd[row0 + t0 + threadIdx.x] : 0.0f;
}

// ---------------------------------------------------------------------------------------------
// Stage 64 rows (tokens t0 .. t0 + 63, zero past T) of a [*, T, 64] tensor into LDS transposed,
// dst[dim * 68 + token] (dims 0 .. 63), as fp32. Thread's share: tokens 4 (tid % 16) .. + 3,
// dims 4 (tid / 16) .. + 3 (16-byte writes).
template <typename T>
__device__ inline void stage_cols(float *dst, const T *src, size_t row0, int t0, int T_len) {
    const int r0 = 4 * (threadIdx.x & 15), dc = 4 * (threadIdx.x >> 4);
    float x[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[u][j] = 0.0f;
        if (t0 + r0 + u < T_len) {
            const T *p = src + (row0 + t0 + r0 + u) * OAL_D + dc;
#pragma unroll
            for (int j = 0; j < 4; ++j) x[u][j] = oal_ld(p + j);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4 *>(dst + (dc + j) * 68 + r0) = make_float4(x[0][j], x[1][j], x[2][j], x[3][j]);
}

// fp32 x = x0 + x1 + x2 (+ a remainder below 2^-24 |x|) in bf16 parts, each difference exact in
// fp32: x0 = bf16(x), x1 = bf16(x - x0), x2 = bf16(x - x0 - x1). A product x y is taken as the
// six terms x_i y_j with i + j <= 2 (Henry, Tang and Heinecke, "Leveraging the bfloat16
// artificial intelligence datatype for higher-precision computations", 2019: the "bf16x6"
// product); the dropped terms are below about 2^-22 |x y|, and each 16x16x32 bf16 MFMA is exact
// in its products and accumulates in fp32.
__device__ inline void split3(float x, __bf16 &x0, __bf16 &x1, __bf16 &x2) {
    x0 = (__bf16)x;
    const float r = x - (float)x0;
    x1 = (__bf16)r;
    x2 = (__bf16)(r - (float)x1);
}

typedef __bf16 oal_bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 oal_bf16x2 __attribute__((ext_vector_type(2)));

// Sum over the 16 lanes of a DPP row, left in every lane of the row: row rotations by 8, 4,
// 2 and 1 lanes (VALU data movement, no LDS round trip).
__device__ inline float row16_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
    return x;
}


// Eight consecutive fp32 values (16-byte aligned, LDS) in N bf16 parts (split3; N = 1 when the
// values are exact in bf16).
template <int N>
__device__ inline void split_frag(const float *p, oal_bf16x8 (&out)[3]) {
    const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        __bf16 x0, x1, x2;
        split3(x[e], x0, x1, x2);
        out[0][e] = x0;
        if constexpr (N > 1) out[1][e] = x1;
        if constexpr (N > 2) out[2][e] = x2;
    }
}

// P[r][c] = sum_{k < 64} X[r][k] Y[c][k] for the wave's 16 rows of X (this lane's row lr) and
// the 64 rows of Y (LDS tiles, row stride 68), on bf16 MFMA with NX and NY parts per operand
// (the terms of order <= 2). P[ct][jj]: row 4 kg + jj, column 16 ct + lr.
template <int NX, int NY>
__device__ inline void mfma_xyt(const float *X, const float *Y, int lr, int kg, oal_f32x4 (&P)[4]) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) P[ct] = oal_splat(0.0f);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        oal_bf16x8 a[3];
        split_frag<NX>(X + lr * 68 + 32 * ks + 8 * kg, a);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            oal_bf16x8 bq[3];
            split_frag<NY>(Y + (16 * ct + lr) * 68 + 32 * ks + 8 * kg, bq);
#pragma unroll
            for (int ord = 2; ord >= 0; --ord)
#pragma unroll
                for (int i = 0; i < NX; ++i) {
                    const int j = ord - i;
                    if (j < 0 || j >= NY) continue;
                    P[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bq[j], P[ct], 0, 0, 0);
                }
        }
    }
}

// A z-term tile Z = (X o s) Y^T + z0 for the wave's 16 rows of X (this lane's row lr) and the
// 64 rows of Y (LDS tiles, row stride 68), s = a row of Lz (64 floats, 16-byte aligned), on
// bf16 MFMA: X o s in three parts, Y in NY parts (the terms of order <= 2). Z[ct][jj]: row
// 4 kg + jj, column 16 ct + lr.
// The lane's 16 scale values of a z term: Lz[m][32 ks + 8 kg + e], ks = 0, 1, e = 0..7
// (fetched a term ahead by the callers, so that no term waits for its Lz row).
struct ZScale {
    float4 v[4];
};
__device__ inline void zscale_load(const float *sc, int kg, ZScale &z) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        z.v[2 * ks] = *reinterpret_cast<const float4 *>(sc + 32 * ks + 8 * kg);
        z.v[2 * ks + 1] = *reinterpret_cast<const float4 *>(sc + 32 * ks + 8 * kg + 4);
    }
}
template <int NY>
__device__ inline void mfma_zterm(const float *X, const ZScale &zs, const float *Y, float z0, int lr, int kg,
                                  oal_f32x4 (&Z)[4]) {
    // the constant term seeds the accumulators
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) Z[ct] = oal_splat(z0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int k0 = 32 * ks + 8 * kg;
        const float4 x0 = *reinterpret_cast<const float4 *>(X + lr * 68 + k0);
        const float4 x1 = *reinterpret_cast<const float4 *>(X + lr * 68 + k0 + 4);
        const float4 s0 = zs.v[2 * ks];
        const float4 s1 = zs.v[2 * ks + 1];
        const float xs[8] = {x0.x * s0.x, x0.y * s0.y, x0.z * s0.z, x0.w * s0.w,
                             x1.x * s1.x, x1.y * s1.y, x1.z * s1.z, x1.w * s1.w};
        oal_bf16x8 a[3];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            __bf16 p0, p1, p2;
            split3(xs[e], p0, p1, p2);
            a[0][e] = p0;
            a[1][e] = p1;
            a[2][e] = p2;
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            oal_bf16x8 bq[3];
            split_frag<NY>(Y + (16 * ct + lr) * 68 + k0, bq);
#pragma unroll
            for (int ord = 2; ord >= 0; --ord)
#pragma unroll
                for (int j = 0; j < NY; ++j) {
                    const int i = ord - j;
                    if (i < 0) continue;
                    Z[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bq[j], Z[ct], 0, 0, 0);
                }
        }
    }
}
static_assert(offsetof(OalHeadDev, Lz) % 16 == 0, "Lz rows are read as float4");

// Four consecutive elements as fp32 (8-byte aligned for bf16, 16-byte for fp32).
__device__ inline void oal_ld4(const float *p, float (&o)[4]) {
    const float4 t = *reinterpret_cast<const float4 *>(p);
    o[0] = t.x; o[1] = t.y; o[2] = t.z; o[3] = t.w;
}
__device__ inline void oal_ld4(const __bf16 *p, float (&o)[4]) {
    const oal_bf16x4 t = *reinterpret_cast<const oal_bf16x4 *>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (float)t[e];
}

// 1 / 5. Per-chunk increments of one (sequence, KV head): out_c[f][col] = sum_n a_n(f) b_n[col]
//   keys:    a_n = psi_f(k_n),                 b_n = [v_n; 1]   (n over the chunk's keys)
//   queries: a_n = wdec_h[f] mono_f(q_n),      b_n = g_n        (n over the chunk's queries of
//                                                                every head h of the KV head);
//            with dwp, also the state part of each head's coefficient gradient (see below)
// bf16 MFMA (16x16x32) on split operands: M = features, N = the 64 value columns (four
// 16-column tiles), K = rows, 32 per K-step; column 64 (the 1 of the keys, g's 65th value of
// the queries) on the VALU. Operand parts: mono_f(x) = x_r x_t is exact in two bf16 parts for
// bf16 inputs (16 significant bits), three otherwise; v is exact in one part for bf16 inputs,
// g takes three; the products are the terms of order <= 2 of split3 (keys with bf16 inputs:
// two exact terms). Workgroup = (128 features, chunk, sequence x KV head), eight waves, wave w
// the features 16 w .. 16 w + 15; rows are staged 64 at a time, transposed: x as fp32
// [dim][row] (dim 64 holds the 1), b in bf16 parts [column][row] (the queries' g parts come
// ready from oal_bwd_readout_g), so that a lane's 8 rows are contiguous. A
// operand: lane l holds mono_f(x_n) of feature 16 w + l % 16, rows n = 32 ks + 8 (l / 16) + e;
// B operand: b_n[16 tile + l % 16] of the same rows. Accumulators: the head's tile D (lane l
// holds features 16 w + 4 (l / 16) + j, column 16 tile + l % 16), folded into the total with
// the head's coefficients after its rows.
template <typename T, bool QSIDE>
__global__ __launch_bounds__(kIncThreads) void oal_bwd_increments(int T_len, int C, int nch, int n_q_heads,
                                                                int n_kv_heads, const T *__restrict__ x,
                                                                const T *__restrict__ v, const float *__restrict__ gv,
                                                                const float *__restrict__ gd,
                                                                const __bf16 *__restrict__ gpl,
                                                                const unsigned char *__restrict__ params,
                                                                float *__restrict__ st, float *__restrict__ dwp) {
    constexpr int NA = sizeof(T) == 2 ? 2 : 3;                 // parts of mono_f(x)
    constexpr int NB = (!QSIDE && sizeof(T) == 2) ? 1 : 3;     // parts of b
    constexpr int XT = 68, PS = 72;                            // row strides (fp32 / bf16)
    __shared__ __align__(16) float xt[65 * XT];
    __shared__ __align__(16) __bf16 bpl[NB * 64 * PS];
    __shared__ __align__(16) float b64s[64];
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, kg = lane >> 4, w = wave_id();
    const int c = blockIdx.y, bkv = blockIdx.z;
    const int b = bkv / n_kv_heads, kv = bkv % n_kv_heads, n_rep = n_q_heads / n_kv_heads;
    const int fbase = blockIdx.x * kFeatBlock + 16 * w;      // this wave's 16 features
    const int fa_lane = fbase + lr;                           // A operand feature of this lane
    int ia = OAL_D, ib = OAL_D;                    // its dims; dim 64 reads the 1
    if (fa_lane >= 1 && fa_lane <= OAL_D) {
        ia = fa_lane - 1;
    } else if (fa_lane > OAL_D && fa_lane < OAL_NFEAT) {
        int idx = fa_lane - 1 - OAL_D, r = 0;
        while (idx >= OAL_D - r) { idx -= OAL_D - r; ++r; }
        ia = r;
        ib = r + idx;
    }
    float *out = st + ((size_t)bkv * nch + c) * OAL_STATE_STRIDE;
    // output positions of this lane: features fo + j (j = 0..3), column 16 ct + lr; column 64
    // of feature fa_lane
    const int fo = fbase + 4 * kg;
    // queries with dwp: the state S_c this kernel overwrites, for the coefficient gradient
    // dw_h[f] = sum_{i in chunk} mono_f(q_i) (S_c g_i)[f] = S_c[f] . (sum_i mono_f(q_i) g_i)
    const bool coef = QSIDE && dwp != nullptr;
    oal_f32x4 sv[4], tot[4];
    float sv64[4] = {0.0f, 0.0f, 0.0f, 0.0f}, tot64 = 0.0f;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) sv[ct] = tot[ct] = oal_splat(0.0f);
    if (coef) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int f = fo + j;
            if (f < OAL_NFEAT) {
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) sv[ct][j] = out[(size_t)f * OAL_D + 16 * ct + lr];
                sv64[j] = out[(size_t)OAL_NFEAT * OAL_D + f];
            }
        }
    }
    const int nsrc = QSIDE ? n_rep : 1;
    const int tend = min(c * C + C, T_len);
    // the (row tile, head) steps in order; each step's x and b rows are loaded into registers
    // one step ahead: thread's share rows r0 + u (u < 4), dims / columns dc + j (j < 4), and
    // b[64] of row tid
    const int ntile = (tend - c * C + 63) / 64, nstep = nsrc * ntile;
    const int r0 = 2 * (tid & 31), dc = 4 * (tid >> 5);
    float px[2][4], pb[2][4], pb64 = 0.0f;
    uint4 pg0, pg1, pg2;                           // queries: g's parts as written by the readout
    auto load_step = [&](int stp) {
        const int hs = stp / ntile, t0 = c * C + (stp % ntile) * 64;
        const int h = kv * n_rep + hs;
        const size_t row0 = QSIDE ? ((size_t)b * n_q_heads + h) * T_len : ((size_t)b * n_kv_heads + kv) * T_len;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = t0 + r0 + u;
            const size_t o = (row0 + t) * OAL_D + dc;
#pragma unroll
            for (int j = 0; j < 4; ++j) px[u][j] = pb[u][j] = 0.0f;
            if (t < T_len) {
                oal_ld4(x + o, px[u]);
                if constexpr (!QSIDE) oal_ld4(v + o, pb[u]);
            }
        }
        if constexpr (QSIDE) {                     // 16-byte piece tid of each part
            const __bf16 *gp = gpl + ((size_t)((size_t)b * n_q_heads + h) * ((T_len + 63) / 64) + t0 / 64) * 3 * 4096;
            pg0 = *reinterpret_cast<const uint4 *>(gp + 8 * tid);
            pg1 = *reinterpret_cast<const uint4 *>(gp + 4096 + 8 * tid);
            pg2 = *reinterpret_cast<const uint4 *>(gp + 2 * 4096 + 8 * tid);
        }
        if (tid < 64) {
            const bool ok = t0 + tid < T_len;
            if constexpr (QSIDE) pb64 = ok ? gd[row0 + t0 + tid] : 0.0f;
            else pb64 = ok ? 1.0f : 0.0f;
        }
    };
    if (nstep > 0) load_step(0);
    int stp = 0;
    for (int hs = 0; hs < nsrc; ++hs) {
        const int h = kv * n_rep + hs;
        oal_f32x4 D[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) D[ct] = oal_splat(0.0f);
        float dsum = 0.0f;                         // column 64: feature fa_lane, the lane's rows
        for (int t0 = c * C; t0 < tend; t0 += 64, ++stp) {
            __syncthreads();                       // the previous tile is consumed
            if constexpr (QSIDE) {                 // piece tid: column tid / 8, queries 8 (tid % 8) .. + 7
                const int o = (tid >> 3) * PS + 8 * (tid & 7);
                *reinterpret_cast<uint4 *>(bpl + o) = pg0;
                *reinterpret_cast<uint4 *>(bpl + 64 * PS + o) = pg1;
                *reinterpret_cast<uint4 *>(bpl + 2 * 64 * PS + o) = pg2;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                *reinterpret_cast<float2 *>(xt + (dc + j) * XT + r0) = make_float2(px[0][j], px[1][j]);
                if constexpr (QSIDE) continue;
                oal_bf16x2 p0, p1, p2;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    __bf16 x0, x1, x2;
                    split3(pb[u][j], x0, x1, x2);
                    p0[u] = x0;
                    p1[u] = x1;
                    p2[u] = x2;
                }
                const int o = (dc + j) * PS + r0;
                *reinterpret_cast<oal_bf16x2 *>(bpl + o) = p0;
                if constexpr (NB > 1) {
                    *reinterpret_cast<oal_bf16x2 *>(bpl + 64 * PS + o) = p1;
                    *reinterpret_cast<oal_bf16x2 *>(bpl + 2 * 64 * PS + o) = p2;
                }
            }
            if (tid < 64) {
                xt[OAL_D * XT + tid] = 1.0f;
                b64s[tid] = pb64;
            }
            __syncthreads();
            if (stp + 1 < nstep) load_step(stp + 1);
            oal_pin_loads();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int rr = 32 * ks + 8 * kg;   // the lane's first row
                float m[8];
                {
                    const float4 xa0 = *reinterpret_cast<const float4 *>(xt + ia * XT + rr);
                    const float4 xa1 = *reinterpret_cast<const float4 *>(xt + ia * XT + rr + 4);
                    const float4 xb0 = *reinterpret_cast<const float4 *>(xt + ib * XT + rr);
                    const float4 xb1 = *reinterpret_cast<const float4 *>(xt + ib * XT + rr + 4);
                    const float4 g0 = *reinterpret_cast<const float4 *>(b64s + rr);
                    const float4 g1 = *reinterpret_cast<const float4 *>(b64s + rr + 4);
                    m[0] = xa0.x * xb0.x; m[1] = xa0.y * xb0.y; m[2] = xa0.z * xb0.z; m[3] = xa0.w * xb0.w;
                    m[4] = xa1.x * xb1.x; m[5] = xa1.y * xb1.y; m[6] = xa1.z * xb1.z; m[7] = xa1.w * xb1.w;
                    dsum += m[0] * g0.x + m[1] * g0.y + m[2] * g0.z + m[3] * g0.w + m[4] * g1.x + m[5] * g1.y +
                            m[6] * g1.z + m[7] * g1.w;
                }
                oal_bf16x8 a[3];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    __bf16 x0, x1, x2;
                    split3(m[e], x0, x1, x2);
                    a[0][e] = x0;
                    a[1][e] = x1;
                    a[2][e] = x2;
                }
                oal_bf16x8 bb[4][NB];
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                    for (int p = 0; p < NB; ++p)
                        bb[ct][p] = *reinterpret_cast<const oal_bf16x8 *>(bpl + p * 64 * PS + (16 * ct + lr) * PS + rr);
                // the terms a_i b_j with i + j <= 2, small ones first
#pragma unroll
                for (int ord = 2; ord >= 0; --ord)
#pragma unroll
                    for (int i = 0; i < NA; ++i) {
                        const int jb = ord - i;
                        if (jb < 0 || jb >= NB) continue;
#pragma unroll
                        for (int ct = 0; ct < 4; ++ct)
                            D[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[ct][jb], D[ct], 0, 0, 0);
                    }
            }
        }
        // column 64 of feature fa_lane: the four row groups
        dsum += __shfl_xor(dsum, 16);
        dsum += __shfl_xor(dsum, 32);
        // fold: total += wdec_h[f] D (keys: weight 1); coefficient-gradient partial per feature
        float wj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            wj[j] = QSIDE ? (fo + j < OAL_NFEAT ? bwd_head(params, h)->wdec[fo + j] : 0.0f) : 1.0f;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) tot[ct][j] += wj[j] * D[ct][j];
        tot64 += (QSIDE ? (fa_lane < OAL_NFEAT ? bwd_head(params, h)->wdec[fa_lane] : 0.0f) : 1.0f) * dsum;
        if (coef) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float pdw = 0.0f;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) pdw += sv[ct][j] * D[ct][j];
                pdw = row16_sum(pdw);              // the 64 columns of the feature
                const float d64 = __shfl(dsum, 4 * kg + j);   // column 64 of feature fo + j
                if (lr == 0 && fo + j < OAL_NFEAT)
                    dwp[(((size_t)b * n_q_heads + h) * nch + c) * OAL_NFEAT + fo + j] = pdw + sv64[j] * d64;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int f = fo + j;
        if (f < OAL_NFEAT) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) out[(size_t)f * OAL_D + 16 * ct + lr] = tot[ct][j];
        }
    }
    if (kg == 0 && fa_lane < OAL_NFEAT) out[(size_t)OAL_NFEAT * OAL_D + fa_lane] = tot64;
}

// 2 / 6. Exclusive prefix (reverse = 0) or suffix (reverse = 1) sum over the chunks of each
// (sequence x KV head), in place; one thread per state element. The running sum starts from
// init (the incoming state of the forward, NULL: zero) and its final value, the sum over all
// chunks, is written to total when given (the reverse scan's total is the gradient of the
// incoming state: every chunk's state contains it).
__global__ __launch_bounds__(kThreads) void oal_bwd_scan(int nch, int reverse, float *__restrict__ st,
                                                         const float *__restrict__ init, float *__restrict__ total) {
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= OAL_NFEAT * OAL_V1) return;
    float *p = st + (size_t)blockIdx.y * nch * OAL_STATE_STRIDE + e;
    float run = init ? init[(size_t)blockIdx.y * OAL_STATE_STRIDE + e] : 0.0f;
#pragma unroll 4
    for (int i = 0; i < nch; ++i) {
        const size_t o = (size_t)(reverse ? nch - 1 - i : i) * OAL_STATE_STRIDE;
        const float t = p[o];
        p[o] = run;
        run += t;
    }
    if (total) total[(size_t)blockIdx.y * OAL_STATE_STRIDE + e] = run;
}

constexpr int kXcds = 8;                       // MI355X: workgroups go round-robin to 8 XCDs

// Workgroup coordinates renumbered so that each XCD takes a contiguous range of the work
// items, blockIdx.y varying fastest: the workgroups that read the same state (the query heads
// of a KV head, the splits of a key tile) run on one XCD at about the same time and share its
// L2. Falls back to the plain numbering when the grid does not divide by the XCD count.
__device__ inline void xcd_order(int &x, int &y, int &z) {
    const int gx = gridDim.x, gy = gridDim.y, n = gx * gy * gridDim.z;
    const int id = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
    int item = n % kXcds == 0 ? (id % kXcds) * (n / kXcds) + id / kXcds : id;
    y = item % gy;
    item /= gy;
    x = item % gx;
    z = item / gx;
}


// Keys of the chunk that query lane i of tile qt sees, tile kt: all of an earlier tile, up to
// and including its own position in its own tile.
__device__ inline bool sees(int kt, int qt, int jj, int i) { return kt < qt || jj <= i; }

// 3. u_i = phi_h(q_i) . S_c + sum_{j <= i in the chunk} kappa_ij [v_j; 1]; y = u[0:64] / u[64];
//    g_i = (dy_i / den, -(dy_i . y_i) / den). Workgroup = (64-query tile, head, sequence).
//    State part U = phi(Q) S_c on split-bf16 MFMA (below), wave w computing the queries
//    16 w .. 16 w + 15 against the 64 value columns, K over the features in blocks of 64, each
//    block of S_c split and staged once in LDS; the normaliser column on the VALU. Pairs
//    inside the chunk on fp32 MFMA: lane = query, the four waves split the keys.
template <typename T>
__global__ __launch_bounds__(kThreads) void oal_bwd_readout_g(int s0, int T_len, int C, int nch, int n_q_heads,
                                                               int n_kv_heads, const T *__restrict__ q,
                                                               const T *__restrict__ k, const T *__restrict__ v,
                                                               const float *__restrict__ dy,
                                                               const unsigned char *__restrict__ params,
                                                               const float *__restrict__ st, float *__restrict__ gv,
                                                               float *__restrict__ gd, __bf16 *__restrict__ gpl) {
    __shared__ __align__(16) float xq[64 * 68];
    __shared__ __align__(16) float ks[64 * 68];    // keys; before them the coefficient tables
    // values (vs) and kappa / u (uin); before them the split block of S_c across both
    __shared__ __align__(16) float vu[64 * 80 + 64 * 68];
    float *const vs = vu, *const uin = vu + 64 * 80;
    int bx, by, bz;
    xcd_order(bx, by, bz);
    const int tpc = C / 64, c = bx / tpc, qt = bx % tpc;
    const int h = by, b = bz, n_rep = n_q_heads / n_kv_heads, kv = h / n_rep;
    const int i = threadIdx.x & 63, w = wave_id();
    const int t0 = c * C + qt * 64, t = t0 + i;
    const bool valid = t < T_len;
    const OalHeadDev *hd = bwd_head(params, h);
    const int G = hd->G;
    const size_t qrow = ((size_t)b * n_q_heads + h) * T_len, krow = ((size_t)b * n_kv_heads + kv) * T_len;
    stage_rows(xq, 68, q, qrow, t0, T_len, 1.0f);
    constexpr int NFP = 2176;                      // features padded to 34 blocks of 64
    float *wdl = ks;                               // wdec_h[f], zero past 2145
    unsigned short *fdl = reinterpret_cast<unsigned short *>(ks + NFP);   // dims of f: a | b << 8
    for (int f = threadIdx.x; f < NFP; f += kThreads) {
        wdl[f] = f < OAL_NFEAT ? hd->wdec[f] : 0.0f;
        int fa = OAL_D, fb = OAL_D;
        if (f >= 1 && f <= OAL_D) {
            fa = f - 1;
        } else if (f > OAL_D && f < OAL_NFEAT) {
            int idx = f - 1 - OAL_D, r = 0;
            while (idx >= OAL_D - r) { idx -= OAL_D - r; ++r; }
            fa = r;
            fb = r + idx;
        }
        fdl[f] = (unsigned short)(fa | (fb << 8));
    }
    __syncthreads();

    const int lr = threadIdx.x & 15, kg = (threadIdx.x >> 4) & 3;       // MFMA lane roles
    const float *xa = xq + (16 * w + lr) * 68;                         // A row: query 16 w + lr
    oal_f32x4 D[5];                                 // u: query 16 w + 4 kg + j, column 16 ct + lr
#pragma unroll
    for (int ct = 0; ct < 5; ++ct) D[ct] = oal_splat(0.0f);
    if (c > 0 || s0) {                             // S_0 = 0 without an incoming state
        // U = phi(Q) S_c = mono(Q) (wdec_h o S_c) on bf16 MFMA (16x16x32) with split operands
        // (the terms of order <= 2 of split3; mono_f(q) = q_r q_t is exact in two bf16 parts for
        // bf16 inputs): K = the features in blocks of 64 (two K-steps), N = the 64 value columns
        // in four tiles; the normaliser column 64 on the VALU. A operand: lane (lr, kg) holds
        // mono_f(q) of query 16 w + lr for the features 32 ks + 8 kg + e of the block, formed
        // and split in registers. B operand: the block of wdec_h[f] S_c[f] staged in LDS
        // transposed, plane row = value column, 64 features (stride PS), so that a lane's 8
        // features are one 16-byte read.
        constexpr int PS = 72;
        __bf16 *pb = reinterpret_cast<__bf16 *>(vs);              // 3 planes x 64 columns x PS
        float *sdb = vs + 3 * 64 * PS / 2;                         // column 64 of the block
        const float *S = st + ((size_t)((size_t)b * n_kv_heads + kv) * nch + c) * OAL_STATE_STRIDE;
        const float *Sd = S + (size_t)OAL_NFEAT * OAL_D;
        // staging share: features sf + u (u < 4), columns sc + j (j < 4)
        const int sf = 4 * (threadIdx.x & 15), sc = 4 * (threadIdx.x >> 4);
        float4 pre[4];
        float pre64 = 0.0f;
        auto load_block = [&](int f0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int f = f0 + sf + u;
                pre[u] = f < OAL_NFEAT ? *reinterpret_cast<const float4 *>(S + (size_t)f * OAL_D + sc)
                                       : make_float4(0, 0, 0, 0);
            }
            if (threadIdx.x < 64) pre64 = f0 + (int)threadIdx.x < OAL_NFEAT ? Sd[f0 + threadIdx.x] : 0.0f;
        };
        constexpr int NQP = sizeof(T) == 2 ? 2 : 3;    // parts of mono_f(q)
        float dpart = 0.0f;                        // normaliser of query 16 w + lr, the lane's features
        load_block(0);
        for (int f0 = 0; f0 < NFP; f0 += 64) {
            __syncthreads();                       // the previous block is consumed
            float wf[4];                           // wdec_h of the thread's four features
#pragma unroll
            for (int u = 0; u < 4; ++u) wf[u] = wdl[f0 + sf + u];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                oal_bf16x4 p0, p1, p2;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float x = wf[u] * (j == 0 ? pre[u].x : j == 1 ? pre[u].y : j == 2 ? pre[u].z : pre[u].w);
                    __bf16 x0, x1, x2;
                    split3(x, x0, x1, x2);
                    p0[u] = x0;
                    p1[u] = x1;
                    p2[u] = x2;
                }
                const int o = (sc + j) * PS + sf;
                *reinterpret_cast<oal_bf16x4 *>(pb + o) = p0;
                *reinterpret_cast<oal_bf16x4 *>(pb + 64 * PS + o) = p1;
                *reinterpret_cast<oal_bf16x4 *>(pb + 2 * 64 * PS + o) = p2;
            }
            if (threadIdx.x < 64) sdb[threadIdx.x] = wdl[f0 + threadIdx.x] * pre64;
            __syncthreads();
            if (f0 + 64 < NFP) load_block(f0 + 64);
            oal_pin_loads();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int fl = 32 * ks + 8 * kg;   // the lane's first feature in the block
                oal_bf16x8 a0, a1, a2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int f = f0 + fl + e;
                    const unsigned short ab = fdl[f];
                    const float ph = xa[ab & 0xff] * xa[ab >> 8];
                    dpart += ph * sdb[fl + e];
                    __bf16 x0, x1, x2;
                    split3(ph, x0, x1, x2);
                    a0[e] = x0;
                    a1[e] = x1;
                    a2[e] = x2;
                }
                oal_bf16x8 b0[4], b1[4], b2[4];
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const int o = (16 * ct + lr) * PS + fl;
                    b0[ct] = *reinterpret_cast<const oal_bf16x8 *>(pb + o);
                    b1[ct] = *reinterpret_cast<const oal_bf16x8 *>(pb + 64 * PS + o);
                    b2[ct] = *reinterpret_cast<const oal_bf16x8 *>(pb + 2 * 64 * PS + o);
                }
                // small terms first (a2 = 0 for bf16 inputs)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) D[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1[ct], D[ct], 0, 0, 0);
                if constexpr (NQP > 2) {
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct) D[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, b0[ct], D[ct], 0, 0, 0);
                }
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) D[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b2[ct], D[ct], 0, 0, 0);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) D[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b0[ct], D[ct], 0, 0, 0);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) D[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b1[ct], D[ct], 0, 0, 0);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) D[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0[ct], D[ct], 0, 0, 0);
            }
        }
        // the normaliser of query 16 w + lr summed over the four lanes kg, then moved to the
        // accumulator layout of column 64: lane (0, kg) holds query 16 w + 4 kg + jj
        dpart += __shfl_xor(dpart, 16);
        dpart += __shfl_xor(dpart, 32);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float dj = __shfl(dpart, 4 * kg + jj);
            D[4][jj] = lr == 0 ? dj : 0.0f;
        }
    }

    // pairs inside the chunk (split-bf16 MFMA): per key tile and z-term m, Z_m = (Q o Lz[m]) K^T
    // (+ L00 for m = 0); kappa = eps + sum_m Z_m^2 on the pairs that see each other; then
    // D += kappa V (V staged transposed) and the normaliser column += the row sums of kappa.
    // kappa passes through uin (the wave's own rows) to be an A operand.
    {
        const float *Lz = hd->Lz;
        const float L00 = hd->L00, eps = hd->eps;
        for (int kt = 0; kt <= qt; ++kt) {
            const int k0 = c * C + kt * 64;
            __syncthreads();
            stage_rows(ks, 68, k, krow, k0, T_len, 0.0f);
            stage_cols(vs, v, krow, k0, T_len);    // [column][key]
            __syncthreads();
            oal_f32x4 kap[4];                       // query 16 w + 4 kg + jj, key 16 jt + lr
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) kap[jt] = oal_splat(0.0f);
            ZScale zn, zc;
            zscale_load(Lz, kg, zn);
            for (int m = 0; m <= G; ++m) {
                zc = zn;
                if (m < G) zscale_load(Lz + (m + 1) * OAL_D, kg, zn);
                oal_f32x4 Z[4];
                mfma_zterm<sizeof(T) == 2 ? 1 : 3>(xq + 16 * w * 68, zc, ks, m == 0 ? L00 : 0.0f, lr, kg, Z);
#pragma unroll
                for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) kap[jt][jj] += Z[jt][jj] * Z[jt][jj];
            }
            float ksum[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // row sums of kappa: query 16 w + 4 kg + jj
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int il = 16 * w + 4 * kg + jj, jl = 16 * jt + lr;
                    const float x = sees(kt, qt, jl, il) ? eps + kap[jt][jj] : 0.0f;
                    uin[il * 68 + jl] = x;
                    ksum[jj] += x;
                }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float sj = row16_sum(ksum[jj]);
                if (lr == 0) D[4][jj] += sj;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // the wave reads its own rows
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            oal_f32x4 P[4];
            mfma_xyt<3, sizeof(T) == 2 ? 1 : 3>(uin + 16 * w * 68, vs, lr, kg, P);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) D[ct] += P[ct];
        }
    }
    // u into uin (row = query, columns 0..64), then the epilogue of wave 0
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < 5; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = 16 * ct + lr;
            if (col <= 64) uin[(16 * w + 4 * kg + j) * 68 + col] = D[ct][j];
        }
    __syncthreads();
    float acc[65];
    float *gt = xq;                                // g transposed: [column][query], stride 65
    if (w == 0) {
        if (valid) {
#pragma unroll
            for (int e = 0; e < 65; ++e) acc[e] = uin[i * 68 + e];
            const float inv = 1.0f / acc[64];
            const float *dyr = dy + (qrow + t) * OAL_D;
            float *gr = gv + (qrow + t) * OAL_D;
            float dot = 0.0f;
#pragma unroll
            for (int e = 0; e < 64; e += 4) {
                const float4 d4 = *reinterpret_cast<const float4 *>(dyr + e);
                dot += d4.x * (acc[e] * inv) + d4.y * (acc[e + 1] * inv) + d4.z * (acc[e + 2] * inv) +
                       d4.w * (acc[e + 3] * inv);
                const float4 g4 = make_float4(d4.x * inv, d4.y * inv, d4.z * inv, d4.w * inv);
                *reinterpret_cast<float4 *>(gr + e) = g4;
                gt[e * 65 + i] = g4.x;
                gt[(e + 1) * 65 + i] = g4.y;
                gt[(e + 2) * 65 + i] = g4.z;
                gt[(e + 3) * 65 + i] = g4.w;
            }
            gd[qrow + t] = -dot * inv;
        } else {
#pragma unroll 8
            for (int e = 0; e < 64; ++e) gt[e * 65 + i] = 0.0f;
        }
    }
    __syncthreads();
    // g[0:64] of the tile also in three bf16 parts, transposed, for the query increments:
    // gpl[tile][part][column][query], tile = (sequence x head, t0 / 64); thread's share: column
    // tid / 4, queries 16 (tid % 4) .. + 15 (a tile past the sequence has no slot)
    if (t0 < T_len) {
        const int col = threadIdx.x >> 2, q0 = 16 * (threadIdx.x & 3);
        __bf16 *gp = gpl + ((size_t)((size_t)b * n_q_heads + h) * ((T_len + 63) / 64) + t0 / 64) * 3 * 4096 + col * 64 + q0;
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
            oal_bf16x8 p0, p1, p2;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                __bf16 x0, x1, x2;
                split3(gt[col * 65 + q0 + 8 * hv + e], x0, x1, x2);
                p0[e] = x0;
                p1[e] = x1;
                p2[e] = x2;
            }
            *reinterpret_cast<oal_bf16x8 *>(gp + 8 * hv) = p0;
            *reinterpret_cast<oal_bf16x8 *>(gp + 4096 + 8 * hv) = p1;
            *reinterpret_cast<oal_bf16x8 *>(gp + 2 * 4096 + 8 * hv) = p2;
        }
    }
}


// 4a. The state parts dq_i = Jphi_h(q_i)^T (S_c g_i) and (keys) dk_j = Jpsi(k_j)^T (R_c [v_j; 1])
//     in one pass over the features, on bf16 MFMA with every fp32 operand split in three
//     bf16 parts.
//
//     Products as six bf16 terms (split3). When the A operand is exact in bf16 (the keys'
//     [v; 1] for bf16 inputs) only its first part is non-zero and three terms remain.
//
//     Work: W = G S^T over the 2145 features (K = the 64 value columns on MFMA, column 64 as a
//     rank-1 update on the VALU), each feature visited once: feature (r, t), r <= t, adds
//     c_f q[t] W_f to dq[r] and c_f q[r] W_f to dq[t] (c_f = wdec_h[f] for queries, 1 for keys;
//     for r = t the two adds give the factor 2 of the square), a linear feature 1 + s adds
//     c_f W_f to dq[s]. Features are taken in tiles of 16 along a row r of the triangle
//     (t = 16 m .. 16 m + 15, lanes with t < r masked), two rows per stage: r = a and
//     r = 63 - a, five tiles for every a in 0..31; stage 0 holds the 64 linear features.
//     A stage's 80 state rows are staged in LDS once per workgroup as three bf16 planes and
//     read by every wave as B operands. Wave w owns the queries (keys) 16 w .. 16 w + 15 and
//     all 64 dims: lane l holds dq of query 16 w + 4 (l / 16) + jj, dim 16 m + l % 16; the
//     dq[r] sums of a row are reduced over the 16 lanes of a row group at the end of the stage.
//     Keys: the 33 stages are split over kDkSplits workgroups, each writing its own slot.


template <typename T, bool KEYS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void oal_bwd_dstate_x6(
    int s0, int T_len, int C, int nch, int n_q_heads, int n_kv_heads, const T *__restrict__ x, const T *__restrict__ v,
    const unsigned char *__restrict__ params, const float *__restrict__ st, const float *__restrict__ gv,
    const float *__restrict__ gd, float *__restrict__ out) {
    constexpr int NR = 80, PS = 72, NSTAGE = 33;   // rows per stage, plane row stride (bf16), stages
    constexpr bool kAExact = KEYS && sizeof(T) == 2;
    __shared__ __align__(16) __bf16 pl[3][NR * PS];
    __shared__ float sdl[NR];                      // column 64 of the staged rows
    __shared__ __align__(16) float xq[64 * 68];    // query (key) tile
    __shared__ float wdl[KEYS ? 1 : 2176];         // wdec of the head
    int bx, by, bz;
    xcd_order(bx, by, bz);
    const int tpc = C / 64, c = bx / tpc, qt = bx % tpc;
    const int h = KEYS ? by / kDkSplits : by, b = bz, n_rep = n_q_heads / n_kv_heads;
    const int kv = KEYS ? h : h / n_rep, psplit = KEYS ? by % kDkSplits : 0;
    const int sbeg = KEYS ? NSTAGE * psplit / kDkSplits : 0;
    const int send = KEYS ? NSTAGE * (psplit + 1) / kDkSplits : NSTAGE;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, kg = lane >> 4, w = wave_id();
    const int t0 = c * C + qt * 64;
    if (t0 >= T_len) return;                       // a tile past the sequence (uniform)
    const size_t row0 = KEYS ? ((size_t)b * n_kv_heads + kv) * T_len : ((size_t)b * n_q_heads + h) * T_len;
    stage_rows(xq, 68, x, row0, t0, T_len, 0.0f);
    if constexpr (!KEYS) {
        const OalHeadDev *hd = bwd_head(params, h);
        for (int f = tid; f < 2176; f += kThreads) wdl[f] = f < OAL_NFEAT ? hd->wdec[f] : 0.0f;
    }
    oal_f32x4 acc[4];                              // query 16 w + 4 kg + jj, dim 16 m + lr
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = oal_splat(0.0f);
    if (KEYS ? c < nch - 1 : (c > 0 || s0)) {      // R of the last chunk = 0; S_0 = 0 without
                                                   // an incoming state
        const float *S = st + ((size_t)((size_t)b * n_kv_heads + kv) * nch + c) * OAL_STATE_STRIDE;
        const float *Sd = S + (size_t)OAL_NFEAT * OAL_D;
        // A operand: g (keys: [v; 1]) of row 16 w + lr, columns 32 ks + 8 kg + e, three parts
        oal_bf16x8 ga[2][3];
        float g64[4];
        {
            const int ta = t0 + 16 * w + lr;
            const bool ok = ta < T_len;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float e8[8];
                const size_t o = (row0 + ta) * OAL_D + 32 * ks + 8 * kg;
#pragma unroll
                for (int e = 0; e < 8; ++e) e8[e] = 0.0f;
                if (ok) {
                    if constexpr (KEYS) {
                        RowVec<T>::load(v + o, e8);
                        if constexpr (RowVec<T>::N == 4) RowVec<T>::load(v + o + 4, e8 + 4);
                    } else {
                        RowVec<float>::load(gv + o, e8);
                        RowVec<float>::load(gv + o + 4, e8 + 4);
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    __bf16 x0, x1, x2;
                    split3(e8[e], x0, x1, x2);
                    ga[ks][0][e] = x0;
                    ga[ks][1][e] = x1;
                    ga[ks][2][e] = x2;
                }
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int tq = t0 + 16 * w + 4 * kg + jj;
                g64[jj] = tq < T_len ? (KEYS ? 1.0f : gd[row0 + tq]) : 0.0f;
            }
        }
        __syncthreads();                           // xq staged
        float qreg[4][4];                          // x[query 16 w + 4 kg + jj][16 m + lr]
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) qreg[m][jj] = xq[(16 * w + 4 * kg + jj) * 68 + 16 * m + lr];
        // first feature of tile i of stage s
        auto tile_f0 = [](int s, int i) -> int {
            if (s == 0) return 1 + 16 * (i & 3);
            const int a = s - 1;
            if (a < 16) return i < 4 ? quad_base(a) + 16 * i : quad_base(63 - a) + 48;
            return i < 3 ? quad_base(a) + 16 * (i + 1) : quad_base(63 - a) + 16 * (i - 1);
        };
        // this thread's staging share: float4 e = tid + 256 u of the 80 x 64 rows (row e / 16,
        // columns 4 (e % 16)), and column 64 of row tid
        float4 pre[5];
        float pre64 = 0.0f;
        auto load_stage = [&](int s) {
#pragma unroll
            for (int u = 0; u < 5; ++u) {
                const int e = tid + kThreads * u, row = e >> 4;
                pre[u] = *reinterpret_cast<const float4 *>(S + (size_t)(tile_f0(s, row >> 4) + (row & 15)) * OAL_D +
                                                           (e & 15) * 4);
            }
            if (tid < NR) pre64 = Sd[tile_f0(s, tid >> 4) + (tid & 15)];
        };
        auto store_stage = [&]() {
#pragma unroll
            for (int u = 0; u < 5; ++u) {
                const int e = tid + kThreads * u, row = e >> 4, col = (e & 15) * 4;
                const float xs[4] = {pre[u].x, pre[u].y, pre[u].z, pre[u].w};
                oal_bf16x4 p0, p1, p2;
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                    __bf16 x0, x1, x2;
                    split3(xs[k4], x0, x1, x2);
                    p0[k4] = x0;
                    p1[k4] = x1;
                    p2[k4] = x2;
                }
                *reinterpret_cast<oal_bf16x4 *>(&pl[0][row * PS + col]) = p0;
                *reinterpret_cast<oal_bf16x4 *>(&pl[1][row * PS + col]) = p1;
                *reinterpret_cast<oal_bf16x4 *>(&pl[2][row * PS + col]) = p2;
            }
            if (tid < NR) sdl[tid] = pre64;
        };
        // W of the stage's NT tiles: row 16 w + 4 kg + jj, feature (tile) lane lr
        auto products = [&](auto nt_c, oal_f32x4 (&W)[5]) {
            constexpr int NT = decltype(nt_c)::value;
#pragma unroll
            for (int i = 0; i < NT; ++i) W[i] = oal_splat(0.0f);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                oal_bf16x8 bp[NT][3];
#pragma unroll
                for (int i = 0; i < NT; ++i)
#pragma unroll
                    for (int p = 0; p < 3; ++p)
                        bp[i][p] = *reinterpret_cast<const oal_bf16x8 *>(&pl[p][(16 * i + lr) * PS + 32 * ks + 8 * kg]);
                // small terms first
                if constexpr (!kAExact) {
#pragma unroll
                    for (int i = 0; i < NT; ++i) W[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga[ks][1], bp[i][1], W[i], 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < NT; ++i) W[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga[ks][2], bp[i][0], W[i], 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < NT; ++i) W[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga[ks][0], bp[i][2], W[i], 0, 0, 0);
                if constexpr (!kAExact) {
#pragma unroll
                    for (int i = 0; i < NT; ++i) W[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga[ks][1], bp[i][0], W[i], 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < NT; ++i) W[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga[ks][0], bp[i][1], W[i], 0, 0, 0);
#pragma unroll
                for (int i = 0; i < NT; ++i) W[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga[ks][0], bp[i][0], W[i], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < NT; ++i) {         // column 64: rank-1 update
                const float sdv = sdl[16 * i + lr];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) W[i][jj] += g64[jj] * sdv;
            }
        };
        // a row stage: KIND 1 (a < 16): tiles (a, 0..3), (63 - a, 3); KIND 2: (a, 1..3), (63 - a, 2..3)
        auto row_stage = [&](auto kind_c, int a) {
            constexpr int KIND = decltype(kind_c)::value;
            oal_f32x4 W[5];
            products(std::integral_constant<int, 5>{}, W);
            const int rb = 63 - a;
            float xa[4], xb[4], ra[4], rs[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                xa[jj] = xq[(16 * w + 4 * kg + jj) * 68 + a];
                xb[jj] = xq[(16 * w + 4 * kg + jj) * 68 + rb];
                ra[jj] = rs[jj] = 0.0f;
            }
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const bool second = KIND == 1 ? i == 4 : i >= 3;
                const int m = KIND == 1 ? (i < 4 ? i : 3) : (i < 3 ? i + 1 : i - 1);
                const int r = second ? rb : a, t = 16 * m + lr;
                // lanes with t < r read the coefficient of another feature (in range) and drop it
                const float wraw = KEYS ? 1.0f : wdl[quad_base(r) + t];
                const float cf = t >= r ? wraw : 0.0f;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float wv = W[i][jj] * cf;
                    if (second) {
                        rs[jj] += wv * qreg[m][jj];
                        acc[m][jj] += wv * xb[jj];
                    } else {
                        ra[jj] += wv * qreg[m][jj];
                        acc[m][jj] += wv * xa[jj];
                    }
                }
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {       // the row sums over the 16 lanes of the group
                ra[jj] = row16_sum(ra[jj]);
                rs[jj] = row16_sum(rs[jj]);
            }
            constexpr int MA = KIND == 1 ? 0 : 1, MB = KIND == 1 ? 3 : 2;
            const int la = a - 16 * MA, lb = rb - 16 * MB;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                if (lr == la) acc[MA][jj] += ra[jj];
                if (lr == lb) acc[MB][jj] += rs[jj];
            }
        };
        load_stage(sbeg);
        for (int s = sbeg; s < send; ++s) {
            __syncthreads();                       // the previous stage is consumed
            store_stage();
            __syncthreads();
            if (s + 1 < send) load_stage(s + 1);
            oal_pin_loads();
            if (s == 0) {                          // linear features 1 + s
                oal_f32x4 W[5];
                products(std::integral_constant<int, 4>{}, W);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float cf = KEYS ? 1.0f : wdl[1 + 16 * m + lr];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc[m][jj] += cf * W[m][jj];
                }
            } else if (s <= 16) {
                row_stage(std::integral_constant<int, 1>{}, s - 1);
            } else {
                row_stage(std::integral_constant<int, 2>{}, s - 1);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int tq = t0 + 16 * w + 4 * kg + jj;
            if (tq < T_len) {
                if constexpr (KEYS)   // part slot psplit, dk half; rows = B Hkv T
                    out[((size_t)psplit * gridDim.z * n_kv_heads * T_len + row0 + tq) * 128 + 16 * m + lr] = acc[m][jj];
                else
                    out[(row0 + tq) * OAL_D + 16 * m + lr] = acc[m][jj];
            }
        }
}

// 4b. dq_i += sum_{j <= i in the chunk} dkappa_ij dkappa_ij/dq_i, dkappa_ij = g_i . [v_j; 1], on
//     split-bf16 MFMA (mfma_xyt, mfma_zterm). dkappa/dq_ir = 2 k_jr sum_m z_m Lz[m][r] with
//     z_m = (Q diag(Lz[m]) K^T)_ij (+ L00 for m = 0), so per (query tile, key tile) pair and
//     z-term m: Z_m = (Q o Lz[m]) K^T, E_m = dkappa o Z_m (the dkappa tile is masked to
//     j <= i), dq += 2 Lz[m] o (E_m K) -- two 64 x 64 x 64 products. Wave w owns the queries
//     16 w .. 16 w + 15 of every product; E_m passes through LDS (the wave's own rows) to become
//     the A operand of the second. Rows of Lz past G are zero, so m runs to G.
template <typename T>
__global__ __launch_bounds__(kThreads) void oal_bwd_dq_intra_mfma(int T_len, int C, int n_q_heads, int n_kv_heads,
                                                                   const T *__restrict__ q, const T *__restrict__ k,
                                                                   const T *__restrict__ v,
                                                                   const unsigned char *__restrict__ params,
                                                                   const float *__restrict__ gv,
                                                                   const float *__restrict__ gd, float *__restrict__ dq) {
    __shared__ __align__(16) float ks[64 * 68];    // key tile [key][dim]
    __shared__ __align__(16) float kts[64 * 68];   // key tile transposed [dim][key]
    __shared__ __align__(16) float gs[64 * 68];    // g tile, then E_m
    __shared__ __align__(16) float vs[64 * 68];    // v tile, then the query tile
    float *qs = vs;
    const int tpc = C / 64, c = blockIdx.x / tpc, qt = blockIdx.x % tpc;
    const int h = blockIdx.y, b = blockIdx.z, n_rep = n_q_heads / n_kv_heads, kv = h / n_rep;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, kg = lane >> 4, w = wave_id();
    const int t0 = c * C + qt * 64;
    const OalHeadDev *hd = bwd_head(params, h);
    const int G = hd->G;
    const float L00 = hd->L00;
    const float *Lz = hd->Lz;
    const size_t qrow = ((size_t)b * n_q_heads + h) * T_len, krow = ((size_t)b * n_kv_heads + kv) * T_len;
    constexpr int NK = sizeof(T) == 2 ? 1 : 3;     // parts of k (exact in bf16 for bf16 inputs)
    if (t0 >= T_len) return;                       // a tile past the sequence (uniform)
    oal_f32x4 acc[4];                              // dq: query 16 w + 4 kg + j, dim 16 rt + lr
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = oal_splat(0.0f);
    for (int kt = 0; kt <= qt; ++kt) {
        const int k0 = c * C + kt * 64;
        __syncthreads();                           // previous pair consumed
        stage_g(gs, gv, gd, qrow, t0, T_len);
        stage_rows(vs, 68, v, krow, k0, T_len, 1.0f);
        stage_rows(ks, 68, k, krow, k0, T_len, 0.0f);
        stage_cols(kts, k, krow, k0, T_len);
        __syncthreads();
        // dkappa = G V^T + g64 on the wave's 16 queries, masked, kept in registers in the
        // accumulator layout of Z_m (query 16 w + 4 kg + jj, key 16 jt + lr)
        oal_f32x4 dk[4];
        {
            oal_f32x4 P[4];
            mfma_xyt<3, NK>(gs + 16 * w * 68, vs, lr, kg, P);
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int i = 16 * w + 4 * kg + jj, j = 16 * jt + lr;
                    dk[jt][jj] = (kt < qt || j <= i) ? P[jt][jj] + gs[i * 68 + 64] : 0.0f;
                }
        }
        __syncthreads();                           // gs and vs are free
        stage_rows(qs, 68, q, qrow, t0, T_len, 0.0f);
        __syncthreads();
        float *es = gs;
        ZScale zn, zc;
        zscale_load(Lz, kg, zn);
        for (int m = 0; m <= G; ++m) {
            const float *lzm = Lz + m * OAL_D;
            zc = zn;
            if (m < G) zscale_load(lzm + OAL_D, kg, zn);
            // Z_m for the wave's 16 queries x 64 keys
            oal_f32x4 Z[4];
            mfma_zterm<NK>(qs + 16 * w * 68, zc, ks, m == 0 ? L00 : 0.0f, lr, kg, Z);
            // E_m = dkappa o Z_m into the wave's rows of es (row = query, column = key)
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) es[(16 * w + 4 * kg + jj) * 68 + 16 * jt + lr] = dk[jt][jj] * Z[jt][jj];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // the wave reads its own rows
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            // F = E_m K for the wave's 16 queries x 64 dims (split bf16: E in three parts, K
            // transposed), then dq += 2 Lz[m][r] F
            oal_f32x4 F[4];
            mfma_xyt<3, NK>(es + 16 * w * 68, kts, lr, kg, F);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const float l2 = 2.0f * lzm[16 * rt + lr];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc[rt][jj] += l2 * F[rt][jj];
            }
            __builtin_amdgcn_s_barrier();           // es rows rewritten by the next m
        }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int t = t0 + 16 * w + 4 * kg + jj;
            if (t < T_len) dq[(qrow + t) * OAL_D + 16 * rt + lr] += acc[rt][jj];
        }
}

// 7. dk and dv. Each 64-key tile is covered by:
//    - oal_bwd_dstate_x6<KEYS>: the state part of dk, dk_j += Jpsi(k_j)^T (R_c [v_j; 1]);
//    - kInterSplits workgroups of oal_bwd_dv_x6: split p takes its share of the 34 feature
//      blocks of the state part of dv, dv_j += psi_f(k_j) R_c[f][0:64];
//    - one workgroup of oal_bwd_dkv_intra_mfma per query head h of the KV head: the pairs inside
//      the chunk, i >= j: dv_j += kappa_ij g_i[0:64], dk_j += dkappa_ij dkappa_ij/dk_j.
//    Each writes partial rows of 128 floats (dk, then dv) per key into part[slot]: slots
//    0 .. kInterSplits-1 the state parts (dv's 8 splits; dk's 4 splits in slots 0 .. 3, the dk
//    half of slots 4 .. 7 unused), then one slot per query head. oal_bwd_kv_reduce adds the slots
//    in order.
constexpr int kInterSplits = 8;

__device__ inline float *part_row(float *part, int slot, size_t rows, size_t row) {
    return part + ((size_t)slot * rows + row) * 128;
}


// dv's state part dv_j += (R_c^T psi(k_j))[0:64] on split-bf16 MFMA: M = the 64 keys of the tile
// (wave w: keys 16 w .. 16 w + 15), N = the 64 value columns, K = the features in blocks of 64.
// A operand: psi_f(k) of the lane's key for the features 32 ks + 8 kg + e of the block (exact in
// two bf16 parts for bf16 inputs, three otherwise); B operand: the block of R_c split in three
// parts and staged transposed in LDS ([column][feature]), as in the readout gradient. The 34
// feature blocks are split over kInterSplits workgroups per key tile; split p writes the dv half
// of partial slot p.
template <typename T>
__global__ __launch_bounds__(kThreads) void oal_bwd_dv_x6(int T_len, int C, int nch, int n_kv_heads,
                                                           const T *__restrict__ k, const float *__restrict__ st,
                                                           float *__restrict__ part) {
    constexpr int PS = 72, NFB = 34;               // plane row stride (bf16), feature blocks of 64
    constexpr int NA = sizeof(T) == 2 ? 2 : 3;     // parts of psi_f(k)
    __shared__ __align__(16) float xk[64 * 68];    // key tile, column 64 = 1
    __shared__ __align__(16) __bf16 pb[3 * 64 * PS];
    __shared__ unsigned short fdl[NFB * 64];       // dims of feature f: a | b << 8 (64 reads the 1)
    const int tpc = C / 64, c = blockIdx.x / tpc, kt = blockIdx.x % tpc;
    const int p = blockIdx.y % kInterSplits, kv = blockIdx.y / kInterSplits, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, kg = lane >> 4, w = wave_id();
    const int t0 = c * C + kt * 64;
    if (t0 >= T_len) return;                       // a tile past the sequence (uniform)
    const size_t krow = ((size_t)b * n_kv_heads + kv) * T_len, rows = (size_t)gridDim.z * n_kv_heads * T_len;
    const int fb0 = NFB * p / kInterSplits, fb1 = NFB * (p + 1) / kInterSplits;
    oal_f32x4 D[4];                                // key 16 w + 4 kg + jj, column 16 ct + lr
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) D[ct] = oal_splat(0.0f);
    if (c < nch - 1) {                             // R of the last chunk = 0
        stage_rows(xk, 68, k, krow, t0, T_len, 1.0f);
        for (int f = 64 * fb0 + tid; f < 64 * fb1; f += kThreads) {
            int fa = OAL_D, fb = OAL_D;
            if (f >= 1 && f <= OAL_D) {
                fa = f - 1;
            } else if (f > OAL_D && f < OAL_NFEAT) {
                int idx = f - 1 - OAL_D, r = 0;
                while (idx >= OAL_D - r) { idx -= OAL_D - r; ++r; }
                fa = r;
                fb = r + idx;
            }
            fdl[f] = (unsigned short)(fa | (fb << 8));
        }
        const float *R = st + ((size_t)((size_t)b * n_kv_heads + kv) * nch + c) * OAL_STATE_STRIDE;
        const float *xa = xk + (16 * w + lr) * 68;
        // staging share: features sf + u (u < 4), columns sc + j (j < 4)
        const int sf = 4 * (tid & 15), sc = 4 * (tid >> 4);
        float4 pre[4];
        auto load_block = [&](int f0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int f = f0 + sf + u;
                pre[u] = f < OAL_NFEAT ? *reinterpret_cast<const float4 *>(R + (size_t)f * OAL_D + sc)
                                       : make_float4(0, 0, 0, 0);
            }
        };
        load_block(64 * fb0);
        for (int fbk = fb0; fbk < fb1; ++fbk) {
            const int f0 = 64 * fbk;
            __syncthreads();                       // the previous block is consumed (and xk, fdl staged)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                oal_bf16x4 p0, p1, p2;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float x = j == 0 ? pre[u].x : j == 1 ? pre[u].y : j == 2 ? pre[u].z : pre[u].w;
                    __bf16 x0, x1, x2;
                    split3(x, x0, x1, x2);
                    p0[u] = x0;
                    p1[u] = x1;
                    p2[u] = x2;
                }
                const int o = (sc + j) * PS + sf;
                *reinterpret_cast<oal_bf16x4 *>(pb + o) = p0;
                *reinterpret_cast<oal_bf16x4 *>(pb + 64 * PS + o) = p1;
                *reinterpret_cast<oal_bf16x4 *>(pb + 2 * 64 * PS + o) = p2;
            }
            __syncthreads();
            if (fbk + 1 < fb1) load_block(f0 + 64);
            oal_pin_loads();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int fl = 32 * ks + 8 * kg;   // the lane's first feature in the block
                oal_bf16x8 a[3];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const unsigned short ab = fdl[f0 + fl + e];
                    __bf16 x0, x1, x2;
                    split3(xa[ab & 0xff] * xa[ab >> 8], x0, x1, x2);
                    a[0][e] = x0;
                    a[1][e] = x1;
                    a[2][e] = x2;
                }
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const int o = (16 * ct + lr) * PS + fl;
                    oal_bf16x8 bq[3];
#pragma unroll
                    for (int q3 = 0; q3 < 3; ++q3) bq[q3] = *reinterpret_cast<const oal_bf16x8 *>(pb + q3 * 64 * PS + o);
#pragma unroll
                    for (int ord = 2; ord >= 0; --ord)
#pragma unroll
                        for (int i = 0; i < NA; ++i) {
                            const int jb = ord - i;
                            if (jb < 0 || jb > 2) continue;
                            D[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bq[jb], D[ct], 0, 0, 0);
                        }
                }
            }
        }
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int t = t0 + 16 * w + 4 * kg + jj;
            if (t < T_len) part_row(part, p, rows, krow + t)[64 + 16 * ct + lr] = D[ct][jj];
        }
}

// dk and dv pairs inside the chunk for one query head, on fp32 MFMA (16x16x4). Workgroup =
// (64-key tile, query head, sequence); wave w owns the keys 16 w .. 16 w + 15 of every product.
// Per query tile (qt >= kt) and z-term m: Z_m = (K o Lz[m]) Q^T (keys x queries, + L00 for
// m = 0), kappa += Z_m^2, E_m = dkappa^T o Z_m, dk += 2 Lz[m] o (E_m Q); after the z-terms,
// kappa = eps + sum_m Z_m^2 on the pairs that see each other, and dv += kappa G. E_m and kappa
// pass through LDS (the wave's own rows) to become A operands. Writes part[8 + head slot].
template <typename T>
__global__ __launch_bounds__(kThreads) void oal_bwd_dkv_intra_mfma(int T_len, int C, int n_q_heads, int n_kv_heads,
                                                                    const T *__restrict__ q, const T *__restrict__ k,
                                                                    const T *__restrict__ v,
                                                                    const unsigned char *__restrict__ params,
                                                                    const float *__restrict__ gv,
                                                                    const float *__restrict__ gd, float *__restrict__ part) {
    __shared__ __align__(16) float ks[64 * 68];    // key tile (row = key)
    __shared__ __align__(16) float qs[64 * 68];    // query tile (row = query)
    __shared__ __align__(16) float gs[64 * 68];    // g tile (row = query, column 64 = g64)
    __shared__ __align__(16) float es[64 * 68];    // v tile, then E_m, then kappa (row = key, col = query)
    const int tpc = C / 64, c = blockIdx.x / tpc, kt = blockIdx.x % tpc;
    const int n_rep = n_q_heads / n_kv_heads;
    const int hs = blockIdx.y % n_rep, kv = blockIdx.y / n_rep, b = blockIdx.z, h = kv * n_rep + hs;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, kg = lane >> 4, w = wave_id();
    const int t0 = c * C + kt * 64;
    const size_t krow = ((size_t)b * n_kv_heads + kv) * T_len, rows = (size_t)gridDim.z * n_kv_heads * T_len;
    const size_t qrow = ((size_t)b * n_q_heads + h) * T_len;
    const OalHeadDev *hd = bwd_head(params, h);
    const int G = hd->G;
    const float L00 = hd->L00, eps = hd->eps;
    const float *Lz = hd->Lz;
    if (t0 >= T_len) return;                       // a tile past the sequence (uniform)
    oal_f32x4 dkacc[4], dvacc[4];                  // key 16 w + 4 kg + jj, dim / column 16 rt + lr
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) dkacc[rt] = dvacc[rt] = oal_splat(0.0f);
    for (int qt = kt; qt < tpc; ++qt) {
        const int q0 = c * C + qt * 64;
        if (q0 >= T_len) break;
        __syncthreads();                           // previous tile consumed
        stage_rows(ks, 68, k, krow, t0, T_len, 0.0f);
        stage_rows(qs, 68, q, qrow, q0, T_len, 0.0f);
        stage_g(gs, gv, gd, qrow, q0, T_len);
        stage_rows(es, 68, v, krow, t0, T_len, 1.0f);
        __syncthreads();
        // dkappa[i][j] = g_i . [v_j; 1] on the pairs j <= i, in the accumulator layout:
        // dkr[it][jj] for key j = 16 w + 4 kg + jj, query i = 16 it + lr (V G^T on MFMA)
        float dkr[4][4];
        {
            oal_f32x4 P[4];
            mfma_xyt<sizeof(T) == 2 ? 1 : 3, 3>(es + 16 * w * 68, gs, lr, kg, P);
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const float g64 = gs[(16 * it + lr) * 68 + 64];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int j = 16 * w + 4 * kg + jj, i = 16 * it + lr;
                    dkr[it][jj] = (kt < qt || j <= i) ? P[it][jj] + g64 : 0.0f;
                }
            }
        }
        __syncthreads();                           // the v tile is consumed
        oal_f32x4 kap[4];                          // sum_m Z_m^2: key 16 w + 4 kg + jj, query 16 it + lr
#pragma unroll
        for (int it = 0; it < 4; ++it) kap[it] = oal_splat(0.0f);
        ZScale zn, zc;
        zscale_load(Lz, kg, zn);
        for (int m = 0; m <= G; ++m) {
            const float *lzm = Lz + m * OAL_D;
            zc = zn;
            if (m < G) zscale_load(lzm + OAL_D, kg, zn);
            oal_f32x4 Z[4];
            mfma_zterm<sizeof(T) == 2 ? 1 : 3>(ks + 16 * w * 68, zc, qs, m == 0 ? L00 : 0.0f, lr, kg, Z);
#pragma unroll
            for (int it = 0; it < 4; ++it)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int j = 16 * w + 4 * kg + jj, i = 16 * it + lr;
                    kap[it][jj] += Z[it][jj] * Z[it][jj];
                    es[j * 68 + i] = dkr[it][jj] * Z[it][jj];
                }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // the wave reads its own rows
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            oal_f32x4 F[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) F[rt] = oal_splat(0.0f);
#pragma unroll 4
            for (int st = 0; st < 16; ++st) {
                const int i = 4 * st + kg;
                const float a = es[(16 * w + lr) * 68 + i];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
                    F[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qs[i * 68 + 16 * rt + lr], F[rt], 0, 0, 0);
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const float l2 = 2.0f * lzm[16 * rt + lr];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) dkacc[rt][jj] += l2 * F[rt][jj];
            }
            __builtin_amdgcn_s_barrier();           // es rows rewritten next
        }
        // kappa on the visible pairs, then dv += kappa G
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int j = 16 * w + 4 * kg + jj, i = 16 * it + lr;
                es[j * 68 + i] = (kt < qt || j <= i) ? eps + kap[it][jj] : 0.0f;
            }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll 4
        for (int st = 0; st < 16; ++st) {
            const int i = 4 * st + kg;
            const float a = es[(16 * w + lr) * 68 + i];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                dvacc[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, gs[i * 68 + 16 * rt + lr], dvacc[rt], 0, 0, 0);
        }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int t = t0 + 16 * w + 4 * kg + jj;
            if (t < T_len) {
                float *o = part_row(part, kInterSplits + hs, rows, krow + t);
                o[16 * rt + lr] = dkacc[rt][jj];
                o[64 + 16 * rt + lr] = dvacc[rt][jj];
            }
        }
}

// Sum the nslots partial rows in slot order: dk, dv [rows][64] from part [slot][rows][128].
__global__ __launch_bounds__(kThreads) void oal_bwd_kv_reduce(size_t rows, int nslots, const float *__restrict__ part,
                                                              float *__restrict__ dk, float *__restrict__ dv) {
    const size_t e = (size_t)blockIdx.x * kThreads + threadIdx.x;   // one float4 of a row
    if (e >= rows * 32) return;
    const size_t row = e / 32, col = (e % 32) * 4;
    float4 s = *reinterpret_cast<const float4 *>(part + row * 128 + col);
    // dk: slots 0 .. kDkSplits - 1 hold its state part (slots up to kInterSplits - 1 are dv's only)
    for (int p = 1; p < nslots; ++p) {
        if (col < 64 && p >= kDkSplits && p < kInterSplits) continue;
        const float4 x = *reinterpret_cast<const float4 *>(part + ((size_t)p * rows + row) * 128 + col);
        s.x += x.x; s.y += x.y; s.z += x.z; s.w += x.w;
    }
    float *o = col < 64 ? dk + row * 64 + col : dv + row * 64 + (col - 64);
    *reinterpret_cast<float4 *>(o) = s;
}

// 10. Coefficient gradients. kappa_ij = sum_f wdec_h[f] mono_f(q_i) mono_f(k_j), so the
//     gradient of the coefficient of feature f is dw_h[f] = sum_{j <= i} dkappa_ij mono_f(q_i)
//     mono_f(k_j): its pairs across chunks come from the query increments above (S_c against
//     the head's sum of mono_f(q_i) g_i), the pairs inside a chunk from oal_bwd_dw_intra. With
//     kappa = eps + sbar^T M sbar (M = L L^T), dLoss/dM[g][g'] = sum dkappa sbar_g sbar_g' is a
//     sum of dw over the features whose dims lie in groups g and g' (oal_bwd_coef), then
//     dL = 2 (dLoss/dM) L and deps = dLoss/dM[0][0].
//
// Pairs inside chunk c for head h: workgroup = (chunk, head, sequence). Per (query tile, key
// tile) pair: the tile of dkappa (masked to j <= i) in LDS, then on split-bf16 MFMA (16x16x32,
// the terms of order <= 2 of split3; psi_f(k) = k_r k_t is exact in two bf16 parts for bf16
// inputs) Y = dkappa psi(K) (M = 64 queries in four 16-row tiles, N = features, K = 64 keys in
// two K-steps) and dw[f] += sum_i mono_f(q_i) Y[i][f]. Wave w takes the feature tiles w, w + 4,
// ...; lane l holds the A operand dkappa[16 it + l % 16][32 ks + 8 (l / 16) + e] in three bf16
// parts in registers for the whole pair and builds the B operand psi_f(k_j)
// (f = 16 ft + l % 16, the same keys j) from the key tile. The query and key tiles are staged
// transposed ([dim][token], dim 64 holding the 1) so that a lane's 8 keys, and the 4 queries
// of its accumulator rows, are 16-byte reads.
template <typename T>
__global__ __launch_bounds__(kThreads) void oal_bwd_dw_intra(int T_len, int C, int nch, int n_q_heads,
                                                              int n_kv_heads, const T *__restrict__ q,
                                                              const T *__restrict__ k, const T *__restrict__ v,
                                                              const float *__restrict__ gv, const float *__restrict__ gd,
                                                              float *__restrict__ dwp) {
    constexpr int NFP = 2176, NFT = NFP / 16;      // features padded to 136 tiles of 16
    constexpr int NBP = sizeof(T) == 2 ? 2 : 3;    // parts of psi_f(k)
    __shared__ __align__(16) float ta[65 * 68];   // g tile [query][col], then the query tile [dim][query]
    __shared__ __align__(16) float tb[65 * 68];   // v tile [key][col], then the key tile [dim][key]
    __shared__ __align__(16) float dk[64 * 68];   // dkappa tile
    __shared__ float dwl[NFP];                     // dw of this (chunk, head)
    __shared__ unsigned short fdl[NFP];            // dims of feature f: a | b << 8 (64 reads the 1)
    const int tpc = C / 64, c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int n_rep = n_q_heads / n_kv_heads, kv = h / n_rep, tid = threadIdx.x;
    const int lane = tid & 63, lr = lane & 15, kg = lane >> 4, w = wave_id();
    const size_t qrow = ((size_t)b * n_q_heads + h) * T_len, krow = ((size_t)b * n_kv_heads + kv) * T_len;
    for (int f = tid; f < NFP; f += kThreads) {
        int fa = OAL_D, fb = OAL_D;
        if (f >= 1 && f <= OAL_D) {
            fa = f - 1;
        } else if (f > OAL_D && f < OAL_NFEAT) {
            int idx = f - 1 - OAL_D, r = 0;
            while (idx >= OAL_D - r) { idx -= OAL_D - r; ++r; }
            fa = r;
            fb = r + idx;
        }
        fdl[f] = (unsigned short)(fa | (fb << 8));
        dwl[f] = 0.0f;
    }
    // transposed staging of 64 tokens (zero past T): thread's share tokens r0 .. r0 + 3, dims
    // dc .. dc + 3; row 64 = 1
    const int r0 = 4 * (tid & 15), dc = 4 * (tid >> 4);
    auto stage_t = [&](float *dst, const T *src, size_t row0, int t0) {
        float x[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int j = 0; j < 4; ++j) x[u][j] = 0.0f;
            if (t0 + r0 + u < T_len) oal_ld4(src + (row0 + t0 + r0 + u) * OAL_D + dc, x[u]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<float4 *>(dst + (dc + j) * 68 + r0) = make_float4(x[0][j], x[1][j], x[2][j], x[3][j]);
        if (tid < 64) dst[OAL_D * 68 + tid] = 1.0f;
    };
    for (int qt = 0; qt < tpc; ++qt) {
        const int q0 = c * C + qt * 64;
        if (q0 >= T_len) break;
        for (int kt = 0; kt <= qt; ++kt) {
            const int k0 = c * C + kt * 64;
            __syncthreads();
            stage_g(ta, gv, gd, qrow, q0, T_len);
            stage_rows(tb, 68, v, krow, k0, T_len, 1.0f);
            __syncthreads();
            {                                      // dkappa = G V^T + g64 on the wave's 16 queries
                oal_f32x4 P[4];
                mfma_xyt<3, sizeof(T) == 2 ? 1 : 3>(ta + 16 * w * 68, tb, lr, kg, P);
#pragma unroll
                for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int i = 16 * w + 4 * kg + jj, j = 16 * jt + lr;
                        dk[i * 68 + j] = (kt < qt || j <= i) ? P[jt][jj] + ta[i * 68 + 64] : 0.0f;
                    }
            }
            __syncthreads();
            stage_t(ta, q, qrow, q0);
            stage_t(tb, k, krow, k0);
            __syncthreads();
            oal_bf16x8 A[4][2][3];                 // dkappa[16 it + lr][32 ks + 8 kg + e], three parts
#pragma unroll
            for (int it = 0; it < 4; ++it)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const float *src = dk + (16 * it + lr) * 68 + 32 * ks + 8 * kg;
                    const float4 x0 = *reinterpret_cast<const float4 *>(src);
                    const float4 x1 = *reinterpret_cast<const float4 *>(src + 4);
                    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        __bf16 p0, p1, p2;
                        split3(xs[e], p0, p1, p2);
                        A[it][ks][0][e] = p0;
                        A[it][ks][1][e] = p1;
                        A[it][ks][2][e] = p2;
                    }
                }
            for (int ft = w; ft < NFT; ft += 4) {
                const int fB = 16 * ft + lr;                         // B operand feature of this lane
                const unsigned short abB = fdl[fB];
                const int fa = abB & 0xff, fb = abB >> 8;
                oal_f32x4 D[4];
#pragma unroll
                for (int it = 0; it < 4; ++it) D[it] = oal_splat(0.0f);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const float *ka = tb + fa * 68 + 32 * ks + 8 * kg, *kb = tb + fb * 68 + 32 * ks + 8 * kg;
                    const float4 a0 = *reinterpret_cast<const float4 *>(ka), a1 = *reinterpret_cast<const float4 *>(ka + 4);
                    const float4 b0 = *reinterpret_cast<const float4 *>(kb), b1 = *reinterpret_cast<const float4 *>(kb + 4);
                    const float ps[8] = {a0.x * b0.x, a0.y * b0.y, a0.z * b0.z, a0.w * b0.w,
                                         a1.x * b1.x, a1.y * b1.y, a1.z * b1.z, a1.w * b1.w};
                    oal_bf16x8 B[3];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        __bf16 p0, p1, p2;
                        split3(ps[e], p0, p1, p2);
                        B[0][e] = p0;
                        B[1][e] = p1;
                        B[2][e] = p2;
                    }
                    // the terms A_i B_j with i + j <= 2, small ones first
#pragma unroll
                    for (int ord = 2; ord >= 0; --ord)
#pragma unroll
                        for (int jb = 0; jb < NBP; ++jb) {
                            const int ia = ord - jb;
                            if (ia < 0) continue;
#pragma unroll
                            for (int it = 0; it < 4; ++it)
                                D[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[it][ks][ia], B[jb], D[it], 0, 0, 0);
                        }
                }
                // D[it][jj]: query 16 it + 4 kg + jj, feature 16 ft + lr
                float sum = 0.0f;
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const float4 qa = *reinterpret_cast<const float4 *>(ta + fa * 68 + 16 * it + 4 * kg);
                    const float4 qb = *reinterpret_cast<const float4 *>(ta + fb * 68 + 16 * it + 4 * kg);
                    sum += qa.x * qb.x * D[it][0] + qa.y * qb.y * D[it][1] + qa.z * qb.z * D[it][2] +
                           qa.w * qb.w * D[it][3];
                }
                sum += __shfl_xor(sum, 16);                          // the four query groups
                sum += __shfl_xor(sum, 32);
                if (kg == 0) dwl[fB] += sum;                         // feature tile of this wave alone
            }
        }
    }
    __syncthreads();
    for (int f = tid; f < OAL_NFEAT; f += kThreads)
        dwp[(((size_t)b * n_q_heads + h) * nch + c) * OAL_NFEAT + f] = dwl[f];
}

// dw_h[f]: the partials summed over sequences and chunks (state part, then the pairs inside
// chunks, in a fixed order). Thread = (feature, head).
__global__ __launch_bounds__(kThreads) void oal_bwd_dw_sum(int batch, int nch, int n_q_heads,
                                                            const float *__restrict__ dwp, float *__restrict__ dwt) {
    const int f = blockIdx.x * kThreads + threadIdx.x, h = blockIdx.y;
    if (f >= OAL_NFEAT) return;
    const size_t half = (size_t)batch * n_q_heads * nch * OAL_NFEAT;
    float s = 0.0f;
    for (int part = 0; part < 2; ++part)
        for (int b = 0; b < batch; ++b) {
            const float *p = dwp + part * half + ((size_t)b * n_q_heads + h) * nch * OAL_NFEAT + f;
#pragma unroll 8
            for (int c = 0; c < nch; ++c) s += p[(size_t)c * OAL_NFEAT];
        }
    dwt[(size_t)h * OAL_NFEAT + f] = s;
}

// Per head: dLoss/dM from dw; dL = 2 (dLoss/dM) L, deps.
//   dLoss/dM[0][0] = dw[constant]; [0][g] = [g][0] = sum_{r in g} dw[linear r] / 8;
//   [g][g'] = sum_{r in g, t in g'} dw[quad(min(r,t), max(r,t))] / 64
// (sbar_0 = 1, sbar_g = sum_{r in group g-1} q_r k_r / 8). First each dim r sums its row of
// quadratic features by the group of the other dim (rs[r][g']), then each entry adds the rows
// of its group; both loops are branch-free and in a fixed order.
__global__ __launch_bounds__(kThreads) void oal_bwd_coef(const unsigned char *__restrict__ params,
                                                          const float *__restrict__ dwt, float *__restrict__ dL,
                                                          float *__restrict__ deps) {
    __shared__ float dw[2176];
    __shared__ float rs[64 * 65];
    __shared__ float gm[65 * 65];
    __shared__ int gid[64];                        // group id + 1 of each dim
    const int h = blockIdx.x, tid = threadIdx.x;
    const OalHeadDev *hd = bwd_head(params, h);
    const int G = hd->G, n = G + 1;
    if (tid < 64) gid[tid] = hd->gamma[tid] + 1;
    for (int f = tid; f < OAL_NFEAT; f += kThreads) dw[f] = dwt[(size_t)h * OAL_NFEAT + f];
    for (int e = tid; e < 64 * 65; e += kThreads) rs[e] = 0.0f;
    __syncthreads();
    if (tid < 64) {
        const int r = tid;
        for (int t = 0; t < OAL_D; ++t) {
            const float x = dw[r <= t ? quad_base(r) + t : quad_base(t) + r];
            rs[r * 65 + gid[t]] += x;              // row r belongs to this thread alone
        }
    }
    __syncthreads();
    for (int e = tid; e < n * n; e += kThreads) {
        const int g = e / n, g2 = e % n;
        float x = 0.0f;
        if (g == 0 && g2 == 0) {
            x = dw[0];
        } else if (g == 0 || g2 == 0) {
            const int gg = g + g2;
#pragma unroll 8
            for (int r = 0; r < OAL_D; ++r) x += gid[r] == gg ? dw[1 + r] : 0.0f;
            x *= 0.125f;
        } else {
#pragma unroll 8
            for (int r = 0; r < OAL_D; ++r) x += gid[r] == g ? rs[r * 65 + g2] : 0.0f;
            x *= 1.0f / 64.0f;
        }
        gm[g * 65 + g2] = x;
    }
    __syncthreads();
    for (int e = tid; e < 65 * 65; e += kThreads) {
        const int a = e / 65, m = e % 65;
        float x = 0.0f;
        if (a <= G && m <= a) {
            for (int g2 = m; g2 <= G; ++g2) x += gm[a * 65 + g2] * hd->Lt[g2 * 65 + m];
            x *= 2.0f;
        }
        dL[(size_t)h * 65 * 65 + e] = x;
    }
    if (tid == 0) deps[h] = gm[0];
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <typename T>
hipError_t launch_backward(const oal_dims &d, int T_len, int C, const void *q_, const void *k_, const void *v_,
                           const float *dy, const unsigned char *params, const float *state_in, void *ws, float *dq,
                           float *dk, float *dv, float *dstate_in, float *dL, float *deps, hipStream_t stream) {
    const T *q = static_cast<const T *>(q_), *k = static_cast<const T *>(k_), *v = static_cast<const T *>(v_);
    const int B = d.batch, Hq = d.n_q_heads, Hkv = d.n_kv_heads;
    const int nch = (T_len + C - 1) / C, tpc = C / 64;
    float *st = static_cast<float *>(ws);
    float *gv = reinterpret_cast<float *>(static_cast<unsigned char *>(ws) +
                                          align256((size_t)B * Hkv * nch * OAL_STATE_STRIDE * 4));
    float *gd = reinterpret_cast<float *>(reinterpret_cast<unsigned char *>(gv) + align256((size_t)B * Hq * T_len * 64 * 4));
    float *part = reinterpret_cast<float *>(reinterpret_cast<unsigned char *>(gd) + align256((size_t)B * Hq * T_len * 4));
    const size_t kvrows = (size_t)B * Hkv * T_len;
    float *dwp = reinterpret_cast<float *>(reinterpret_cast<unsigned char *>(part) +
                                           align256((size_t)(kInterSplits + Hq / Hkv) * kvrows * 128 * 4));
    // g in three bf16 parts per 64-query tile (oal_bwd_readout_g -> query increments)
    __bf16 *gpl = reinterpret_cast<__bf16 *>(reinterpret_cast<unsigned char *>(dwp) +
                                             align256(((size_t)2 * B * nch + 1) * Hq * OAL_NFEAT * 4));
    const bool coef = dL != nullptr;
    const dim3 blk(kThreads);
    const dim3 g_inc((OAL_NFEAT + kFeatBlock - 1) / kFeatBlock, nch, B * Hkv);
    const dim3 g_scan((OAL_NFEAT * OAL_V1 + kThreads - 1) / kThreads, B * Hkv);
    const dim3 g_q(nch * tpc, Hq, B), g_ki(nch * tpc, Hkv * kInterSplits, B), g_kh(nch * tpc, Hq, B);
    const dim3 g_red((unsigned)((kvrows * 32 + kThreads - 1) / kThreads));
    const int nslots = kInterSplits + Hq / Hkv;
    hipLaunchKernelGGL((oal_bwd_increments<T, false>), g_inc, dim3(kIncThreads), 0, stream, T_len, C, nch, Hq, Hkv, k, v,
                       (const float *)nullptr, (const float *)nullptr, (const __bf16 *)nullptr, params, st,
                       (float *)nullptr);
    hipLaunchKernelGGL(oal_bwd_scan, g_scan, blk, 0, stream, nch, 0, st, state_in, (float *)nullptr);
    const int s0 = state_in != nullptr;
    hipLaunchKernelGGL(oal_bwd_readout_g<T>, g_q, blk, 0, stream, s0, T_len, C, nch, Hq, Hkv, q, k, v, dy, params, st,
                       gv, gd, gpl);
    hipLaunchKernelGGL((oal_bwd_dstate_x6<T, false>), g_q, blk, 0, stream, s0, T_len, C, nch, Hq, Hkv, q,
                       (const T *)nullptr, params, st, gv, gd, dq);
    hipLaunchKernelGGL(oal_bwd_dq_intra_mfma<T>, g_q, blk, 0, stream, T_len, C, Hq, Hkv, q, k, v, params, gv, gd, dq);
    hipLaunchKernelGGL(oal_bwd_dkv_intra_mfma<T>, g_kh, blk, 0, stream, T_len, C, Hq, Hkv, q, k, v, params, gv, gd,
                       part);
    if (coef)
        hipLaunchKernelGGL(oal_bwd_dw_intra<T>, dim3(nch, Hq, B), blk, 0, stream, T_len, C, nch, Hq, Hkv, q, k, v,
                           gv, gd, dwp + (size_t)B * Hq * nch * OAL_NFEAT);
    hipLaunchKernelGGL((oal_bwd_increments<T, true>), g_inc, dim3(kIncThreads), 0, stream, T_len, C, nch, Hq, Hkv, q,
                       (const T *)nullptr, gv, gd, gpl, params, st, coef ? dwp : (float *)nullptr);
    if (coef) {
        float *dwt = dwp + 2 * (size_t)B * Hq * nch * OAL_NFEAT;
        hipLaunchKernelGGL(oal_bwd_dw_sum, dim3((OAL_NFEAT + kThreads - 1) / kThreads, Hq), blk, 0, stream, B, nch,
                           Hq, dwp, dwt);
        hipLaunchKernelGGL(oal_bwd_coef, dim3(Hq), blk, 0, stream, params, dwt, dL, deps);
    }
    hipLaunchKernelGGL(oal_bwd_scan, g_scan, blk, 0, stream, nch, 1, st, (const float *)nullptr, dstate_in);
    hipLaunchKernelGGL((oal_bwd_dstate_x6<T, true>), dim3(nch * tpc, Hkv * kDkSplits, B), blk, 0, stream, s0, T_len, C,
                       nch, Hq, Hkv, k, v, params, st, gv, gd, part);
    hipLaunchKernelGGL(oal_bwd_dv_x6<T>, g_ki, blk, 0, stream, T_len, C, nch, Hkv, k, st, part);
    hipLaunchKernelGGL(oal_bwd_kv_reduce, g_red, blk, 0, stream, kvrows, nslots, part, dk, dv);
    return hipGetLastError();
}

}  // namespace

size_t oal_backward_ws_bytes_impl(const oal_dims &d, int T_len, int C) {
    const size_t nch = (size_t)(T_len + C - 1) / C;
    return align256((size_t)d.batch * d.n_kv_heads * nch * OAL_STATE_STRIDE * 4) +
           align256((size_t)d.batch * d.n_q_heads * T_len * 64 * 4) + align256((size_t)d.batch * d.n_q_heads * T_len * 4) +
           align256((size_t)(kInterSplits + d.n_q_heads / d.n_kv_heads) * d.batch * d.n_kv_heads * T_len * 128 * 4) +
           align256(((size_t)2 * d.batch * nch + 1) * d.n_q_heads * OAL_NFEAT * 4) +
           align256((size_t)d.batch * d.n_q_heads * ((T_len + 63) / 64) * 3 * 4096 * 2);
}

hipError_t oal_launch_backward(const oal_dims &d, int T_len, int C, const void *q, const void *k, const void *v,
                               const float *dy, const void *params, const float *state_in, void *ws, float *dq,
                               float *dk, float *dv, float *dstate_in, float *dL, float *deps, hipStream_t stream) {
    const unsigned char *p = static_cast<const unsigned char *>(params);
    if (d.dtype == OAL_BF16)
        return launch_backward<__bf16>(d, T_len, C, q, k, v, dy, p, state_in, ws, dq, dk, dv, dstate_in, dL, deps,
                                       stream);
    return launch_backward<float>(d, T_len, C, q, k, v, dy, p, state_in, ws, dq, dk, dv, dstate_in, dL, deps, stream);
}
