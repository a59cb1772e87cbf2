// oal_backward.hip -- gfx950 kernels of the prefill backward: dq, dk, dv (and the gradients of
// the kernel coefficients L, eps) of sum(dy * y) for the causal attention y of a prefill from
// an empty prefix.
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
// where S_c sums psi(k_j) [v_j; 1]^T over the chunks before c (the forward's prefix state) and
// R_c sums phi_h(q_i) g_i^T over the chunks after c and the query heads h of the KV head.
// Inside a chunk kappa is taken from its z-terms, as in the forward's intra-chunk part:
//   z_m = [m = 0] L00 + sum_r Lz[m][r] q_r k_r,   kappa = eps + sum_{m <= G} z_m^2,
//   dkappa/dq_r = 2 k_r sum_m z_m Lz[m][r]        (and the same with q and k exchanged);
// for a (query tile, key tile) pair each z-term is the product (Q o Lz[m]) K^T on MFMA.
//
// Every kernel computes in fp32 (inputs of either dtype are widened on load). The state
// contractions and the products over the pairs inside a chunk run on fp32 MFMA
// (v_mfma_f32_16x16x4_f32), except dv's state part, which runs on the VALU with the state row
// read at a wave-uniform address through the constant address space, so that it arrives in
// scalar registers and feeds the FMAs directly. With packed fp32 off, the VALU bound is the
// non-packed FMA rate (256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz = 78.6 TFLOP/s); fp32
// MFMA reaches 157.3.
//
// Launch order (all on the caller's stream):
//   1. oal_bwd_increments<keys>:    per chunk psi(K_c)^T [V_c; 1]           -> workspace states
//   2. oal_bwd_scan (forward):      exclusive prefix over chunks: S_c
//   3. oal_bwd_readout_g:           u_i (inter + intra), y, den -> g_i     -> workspace g
//   4. oal_bwd_dq_inter_mfma, oal_bwd_dq_intra_mfma: dq (state part, then the pairs inside
//      the chunk)
//   5. oal_bwd_dkv_intra_mfma:      dk, dv partials of the pairs inside the chunk
//   6. oal_bwd_increments<queries>: per chunk sum_h phi_h(Q_c)^T G_c       -> workspace states
//   7. oal_bwd_scan (reverse):      exclusive suffix over chunks: R_c
//   8. oal_bwd_dq_inter_mfma<keys>, oal_bwd_dv_inter: dk, dv partials of the state part
//   9. oal_bwd_kv_reduce:           dk, dv (the partials added in a fixed order)
// With coefficient gradients, also oal_bwd_dw_intra (before 6), the per-head partials of 6,
// and oal_bwd_dw_sum, oal_bwd_coef (after 6): dL, deps.
#include <hip/hip_runtime.h>

#include "oal_device.h"
#include "oal_internal.h"

namespace {

constexpr int kThreads = 256;                 // four waves
constexpr int kFeatBlock = 64;                // features per increment workgroup
constexpr int kDkSplits = 4;                  // dk state part: its t steps over 4 workgroups

typedef const float __attribute__((address_space(4))) cfloat;   // wave-uniform reads

__device__ inline const OalHeadDev *bwd_head(const unsigned char *params, int h) {
    return reinterpret_cast<const OalHeadDev *>(params + sizeof(OalParamsHeader) + (size_t)h * OAL_HEAD_BYTES);
}

__device__ inline const cfloat *uni(const float *p) { return (const cfloat *)p; }

__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// first feature of the quadratic row r, minus r: feature (r, t) is quad_base(r) + t
__device__ inline int quad_base(int r) { return 1 + OAL_D + r * OAL_D - (r * (r - 1)) / 2 - r; }


// acc[0:NC] += a S[f][0:NC] (NC = 64 or 65, column 64 from the separate vector)
template <int NC>
__device__ inline void row_axpy(float (&acc)[NC], float a, const cfloat *S, const cfloat *Sd, int f) {
    const cfloat *row = S + (size_t)f * OAL_D;
#pragma unroll
    for (int c = 0; c < 64; ++c) acc[c] += a * row[c];
    if constexpr (NC == 65) acc[64] += a * Sd[f];
}





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
// 1 / 5. Per-chunk increments of one (sequence, KV head): out_c[f][col] = sum_n a_n(f) b_n[col]
//   keys:    a_n = psi_f(k_n),                 b_n = [v_n; 1]   (n over the chunk's keys)
//   queries: a_n = wdec_h[f] mono_f(q_n),      b_n = g_n        (n over the chunk's queries of
//                                                                every head h of the KV head);
//            with dwp, also the state part of each head's coefficient gradient (see below)
// fp32 MFMA (16x16x4): M = features, N = value columns (five 16-column tiles, the fifth
// holding column 64), K = rows. Workgroup = (64 features, chunk, sequence x KV head), wave w
// the features 16 w .. 16 w + 15; rows are staged 64 at a time. A operand: lane l holds
// mono_f(x_n) of feature 16 w + l % 16 and row n = 4 K-step + l / 16 (the feature's dims are
// fixed per lane); B operand: b_n[16 tile + l % 16]. Accumulators: the head's tile D (lane l
// holds features 16 w + 4 (l / 16) + j, column 16 tile + l % 16), folded into the total with
// the head's coefficients after its rows.
template <typename T, bool QSIDE>
__global__ __launch_bounds__(kThreads) void oal_bwd_increments(int T_len, int C, int nch, int n_q_heads,
                                                                int n_kv_heads, const T *__restrict__ x,
                                                                const T *__restrict__ v, const float *__restrict__ gv,
                                                                const float *__restrict__ gd,
                                                                const unsigned char *__restrict__ params,
                                                                float *__restrict__ st, float *__restrict__ dwp) {
    // row stride 80 (16 mod 32 banks): the four row groups of a wave's MFMA operand reads fall
    // on two bank halves, the two-pass minimum for 64 lanes (65 or 68 gave up to 4-way conflicts)
    constexpr int XS = 80;
    __shared__ __align__(16) float xs[64 * XS];
    __shared__ __align__(16) float bs[64 * XS];
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
    // output positions of this lane: features fo + j (j = 0..3), column 16 ct + lr
    const int fo = fbase + 4 * kg;
    // queries with dwp: the state S_c this kernel overwrites, for the coefficient gradient
    // dw_h[f] = sum_{i in chunk} mono_f(q_i) (S_c g_i)[f] = S_c[f] . (sum_i mono_f(q_i) g_i)
    const bool coef = QSIDE && dwp != nullptr;
    oal_f32x4 sv[5], tot[5];
#pragma unroll
    for (int ct = 0; ct < 5; ++ct) sv[ct] = tot[ct] = oal_splat(0.0f);
    if (coef) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int f = fo + j;
            if (f < OAL_NFEAT) {
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) sv[ct][j] = out[(size_t)f * OAL_D + 16 * ct + lr];
                sv[4][j] = lr == 0 ? out[(size_t)OAL_NFEAT * OAL_D + f] : 0.0f;
            }
        }
    }
    const int nsrc = QSIDE ? n_rep : 1;
    const int tend = min(c * C + C, T_len);
    // the (row tile, head) steps in order; each step's x and b rows are loaded into registers
    // one step ahead (thread's share: 16 elements of each, plus one b[64])
    const int ntile = (tend - c * C + 63) / 64, nstep = nsrc * ntile;
    float px[16], pb[16], pb64 = 0.0f;
    auto load_step = [&](int stp) {
        const int hs = stp / ntile, t0 = c * C + (stp % ntile) * 64;
        const int h = kv * n_rep + hs;
        const size_t row0 = QSIDE ? ((size_t)b * n_q_heads + h) * T_len : ((size_t)b * n_kv_heads + kv) * T_len;
        load_tile(px, x, row0, t0, T_len);
        if constexpr (QSIDE) load_tile(pb, gv, row0, t0, T_len);
        else load_tile(pb, v, row0, t0, T_len);
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
        oal_f32x4 D[5];
#pragma unroll
        for (int ct = 0; ct < 5; ++ct) D[ct] = oal_splat(0.0f);
        for (int t0 = c * C; t0 < tend; t0 += 64, ++stp) {
            __syncthreads();                       // the previous tile is consumed
            store_tile<T>(xs, XS, px);
            if constexpr (QSIDE) store_tile<float>(bs, XS, pb);
            else store_tile<T>(bs, XS, pb);
            if (tid < 64) {
                xs[tid * XS + 64] = 1.0f;
                bs[tid * XS + 64] = pb64;
            }
            __syncthreads();
            if (stp + 1 < nstep) load_step(stp + 1);
#pragma unroll 4
            for (int kst = 0; kst < 16; ++kst) {
                const int n = 4 * kst + kg;
                const float a = xs[n * XS + ia] * xs[n * XS + ib];
                const float *br = bs + n * XS;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
                    D[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, br[16 * ct + lr], D[ct], 0, 0, 0);
                D[4] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, lr == 0 ? br[64] : 0.0f, D[4], 0, 0, 0);
            }
        }
        // fold: total += wdec_h[f] D (keys: weight 1); coefficient-gradient partial per feature
        float wj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            wj[j] = QSIDE ? (fo + j < OAL_NFEAT ? bwd_head(params, h)->wdec[fo + j] : 0.0f) : 1.0f;
#pragma unroll
        for (int ct = 0; ct < 5; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) tot[ct][j] += wj[j] * D[ct][j];
        if (coef) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float pdw = 0.0f;
#pragma unroll
                for (int ct = 0; ct < 5; ++ct) pdw += sv[ct][j] * D[ct][j];
                pdw += __shfl_xor(pdw, 1);         // the 16 columns of the tile row
                pdw += __shfl_xor(pdw, 2);
                pdw += __shfl_xor(pdw, 4);
                pdw += __shfl_xor(pdw, 8);
                if (lr == 0 && fo + j < OAL_NFEAT)
                    dwp[(((size_t)b * n_q_heads + h) * nch + c) * OAL_NFEAT + fo + j] = pdw;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int f = fo + j;
        if (f < OAL_NFEAT) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) out[(size_t)f * OAL_D + 16 * ct + lr] = tot[ct][j];
            if (lr == 0) out[(size_t)OAL_NFEAT * OAL_D + f] = tot[4][j];
        }
    }
}

// 2 / 6. Exclusive prefix (reverse = 0) or suffix (reverse = 1) sum over the chunks of each
// (sequence x KV head), in place; one thread per state element.
__global__ __launch_bounds__(kThreads) void oal_bwd_scan(int nch, int reverse, float *__restrict__ st) {
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= OAL_NFEAT * OAL_V1) return;
    float *p = st + (size_t)blockIdx.y * nch * OAL_STATE_STRIDE + e;
    float run = 0.0f;
#pragma unroll 4
    for (int i = 0; i < nch; ++i) {
        const size_t o = (size_t)(reverse ? nch - 1 - i : i) * OAL_STATE_STRIDE;
        const float t = p[o];
        p[o] = run;
        run += t;
    }
}

// Keys of the chunk that query lane i of tile qt sees, tile kt: all of an earlier tile, up to
// and including its own position in its own tile.
__device__ inline bool sees(int kt, int qt, int jj, int i) { return kt < qt || jj <= i; }

// 3. u_i = phi_h(q_i) . S_c + sum_{j <= i in the chunk} kappa_ij [v_j; 1]; y = u[0:64] / u[64];
//    g_i = (dy_i / den, -(dy_i . y_i) / den). Workgroup = (64-query tile, head, sequence).
//    State part on fp32 MFMA (v_mfma_f32_16x16x4_f32): U = phi(Q) S_c, wave w computing the
//    queries 16 w .. 16 w + 15 against 80 columns (five 16 x 16 tiles; the fifth holds the
//    column 64 of S_c, the normaliser) with K over the features in blocks of 64, each block
//    of S_c staged once in LDS (row stride 80: the four K rows of an operand read fall on two
//    bank halves). A operand: lane l holds phi_f(q) of query l % 16 and feature
//    f = 4 K-step + l / 16, built from the query tile, the head's coefficients and the dims of
//    f (LDS tables); B operand: S_c[f][col], col = 16 tile + l % 16. The result goes to an LDS
//    tile. Pairs inside the chunk: lane = query, the four waves split the keys.
template <typename T>
__global__ __launch_bounds__(kThreads) void oal_bwd_readout_g(int T_len, int C, int nch, int n_q_heads,
                                                               int n_kv_heads, const T *__restrict__ q,
                                                               const T *__restrict__ k, const T *__restrict__ v,
                                                               const float *__restrict__ dy,
                                                               const unsigned char *__restrict__ params,
                                                               const float *__restrict__ st, float *__restrict__ gv,
                                                               float *__restrict__ gd) {
    __shared__ float xq[64 * 65];
    __shared__ __align__(16) float ks[64 * 68];    // keys; before them the coefficient tables
    __shared__ __align__(16) float vs[64 * 80];    // values; before them a block of S_c (stride 80)
    __shared__ __align__(16) float uin[64 * 68];   // state part of u per query
    const int tpc = C / 64, c = blockIdx.x / tpc, qt = blockIdx.x % tpc;
    const int h = blockIdx.y, b = blockIdx.z, n_rep = n_q_heads / n_kv_heads, kv = h / n_rep;
    const int i = threadIdx.x & 63, w = wave_id();
    const int t0 = c * C + qt * 64, t = t0 + i;
    const bool valid = t < T_len;
    const OalHeadDev *hd = bwd_head(params, h);
    const int G = hd->G;
    const size_t qrow = ((size_t)b * n_q_heads + h) * T_len, krow = ((size_t)b * n_kv_heads + kv) * T_len;
    stage_rows(xq, 65, q, qrow, t0, T_len, 1.0f);
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
    const float *xa = xq + (16 * w + lr) * 65;                         // A row: query 16 w + lr
    oal_f32x4 D[5];                                 // u: query 16 w + 4 kg + j, column 16 ct + lr
    {
        oal_f32x4 E[5];                             // even and odd K-steps: independent chains
#pragma unroll
        for (int ct = 0; ct < 5; ++ct) D[ct] = E[ct] = oal_splat(0.0f);
        if (c > 0) {                               // S_0 = 0
            const float *S = st + ((size_t)((size_t)b * n_kv_heads + kv) * nch + c) * OAL_STATE_STRIDE;
            const float *Sd = S + (size_t)OAL_NFEAT * OAL_D;
            float *sblk = vs;
            // block f0 .. f0 + 63 of S_c: thread's share (4 float4 of the 64 columns, one
            // normaliser entry), loaded into registers one block ahead of its use
            float4 pre[4];
            float pre64 = 0.0f;
            auto load_block = [&](int f0) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int e = threadIdx.x + kThreads * m, kk = e >> 4, c4 = (e & 15) * 4, f = f0 + kk;
                    pre[m] = f < OAL_NFEAT ? *reinterpret_cast<const float4 *>(S + (size_t)f * OAL_D + c4)
                                           : make_float4(0, 0, 0, 0);
                }
                if (threadIdx.x < 64) pre64 = f0 + (int)threadIdx.x < OAL_NFEAT ? Sd[f0 + threadIdx.x] : 0.0f;
            };
            load_block(0);
            for (int f0 = 0; f0 < NFP; f0 += 64) {
                __syncthreads();                   // the previous block is consumed
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int e = threadIdx.x + kThreads * m, kk = e >> 4, c4 = (e & 15) * 4;
                    *reinterpret_cast<float4 *>(sblk + kk * 80 + c4) = pre[m];
                }
                if (threadIdx.x < 64) sblk[threadIdx.x * 80 + 64] = pre64;
                __syncthreads();
                if (f0 + 64 < NFP) load_block(f0 + 64);
#pragma unroll 2
                for (int kst = 0; kst < 16; kst += 2) {
                    const int kk = 4 * kst + kg, f = f0 + kk;
                    const unsigned short ab = fdl[f], ab2 = fdl[f + 4];
                    const float a = wdl[f] * xa[ab & 0xff] * xa[ab >> 8];
                    const float a2 = wdl[f + 4] * xa[ab2 & 0xff] * xa[ab2 >> 8];
                    const float *brow = sblk + kk * 80, *brow2 = brow + 4 * 80;
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct) {
                        D[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, brow[16 * ct + lr], D[ct], 0, 0, 0);
                        E[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, brow2[16 * ct + lr], E[ct], 0, 0, 0);
                    }
                    D[4] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, lr == 0 ? brow[64] : 0.0f, D[4], 0, 0, 0);
                    E[4] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, lr == 0 ? brow2[64] : 0.0f, E[4], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int ct = 0; ct < 5; ++ct) D[ct] += E[ct];
    }

    // pairs inside the chunk (fp32 MFMA): per key tile and z-term m, Z_m = (Q o Lz[m]) K^T
    // (+ L00 for m = 0); kappa = eps + sum_m Z_m^2 on the pairs that see each other; then
    // D += kappa [V; 1]. kappa passes through uin (the wave's own rows) to be an A operand.
    {
        const float *Lz = hd->Lz;
        const float L00 = hd->L00, eps = hd->eps;
        for (int kt = 0; kt <= qt; ++kt) {
            const int k0 = c * C + kt * 64;
            __syncthreads();
            stage_rows(ks, 68, k, krow, k0, T_len, 0.0f);
            stage_rows(vs, 68, v, krow, k0, T_len, 1.0f);
            __syncthreads();
            oal_f32x4 kap[4];                       // query 16 w + 4 kg + jj, key 16 jt + lr
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) kap[jt] = oal_splat(0.0f);
            for (int m = 0; m <= G; ++m) {
                const float *lzm = Lz + m * OAL_D;
                oal_f32x4 Z[4];
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) Z[jt] = oal_splat(m == 0 ? L00 : 0.0f);
#pragma unroll 4
                for (int st = 0; st < 16; ++st) {
                    const int r = 4 * st + kg;
                    const float a = xa[r] * lzm[r];
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt)
                        Z[jt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, ks[(16 * jt + lr) * 68 + r], Z[jt], 0, 0, 0);
                }
#pragma unroll
                for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) kap[jt][jj] += Z[jt][jj] * Z[jt][jj];
            }
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int il = 16 * w + 4 * kg + jj, jl = 16 * jt + lr;
                    uin[il * 68 + jl] = sees(kt, qt, jl, il) ? eps + kap[jt][jj] : 0.0f;
                }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // the wave reads its own rows
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll 4
            for (int st = 0; st < 16; ++st) {
                const int j = 4 * st + kg;
                const float a = uin[(16 * w + lr) * 68 + j];
                const float *vr = vs + j * 68;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
                    D[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, vr[16 * ct + lr], D[ct], 0, 0, 0);
                D[4] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, lr == 0 ? vr[64] : 0.0f, D[4], 0, 0, 0);
            }
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
    if (w == 0 && valid) {
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
            *reinterpret_cast<float4 *>(gr + e) = make_float4(d4.x * inv, d4.y * inv, d4.z * inv, d4.w * inv);
        }
        gd[qrow + t] = -dot * inv;
    }
}


// 4a. dq_i = Jphi_h(q_i)^T (S_c g_i) (the state part) on fp32 MFMA. With c_st = wdec of the
//     feature (min(s,t), max(s,t)), doubled for s = t (the square), dq_i[s] = wdec_{1+s}
//     (S_c[1+s] . g_i) + sum_t c_st q_i[t] (S_c[(s,t)] . g_i): per t, X_t = G T_t^T with
//     T_t[s] = S_c[pair(s, t)] (K = the 65 columns), then dq += c_st q_i[t] X_t; the linear
//     features are one more step (T[s] = S_c[1 + s], q factor 1). Workgroup = (64-query tile,
//     head, sequence); wave w owns the queries 16 w .. 16 w + 15 and all 64 dims. The A
//     operand (g) stays in registers for every step; T_t is prefetched into registers one step
//     ahead and staged in LDS.
// State row of T_t[s] (the feature (min(s,t), max(s,t))); t = 64: the linear feature 1 + s.
__device__ inline int dq_row_of(int s, int t) {
    return t == OAL_D ? 1 + s : (s <= t ? quad_base(s) + t : quad_base(t) + s);
}

//     KEYS: the same for dk_j = Jpsi(k_j)^T (R_c [v_j; 1]) -- psi has no coefficients (c_st = 1,
//     2 for s = t, 1 for the linear features), the A operand is [v_j; 1], the rows come from R_c
//     (zero for the last chunk); workgroup = (64-key tile, KV head x 4 splits of the t steps,
//     sequence), each split's result going to the dk half of its partial slot.
template <typename T, bool KEYS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void oal_bwd_dq_inter_mfma(
    int T_len, int C, int nch, int n_q_heads, int n_kv_heads, const T *__restrict__ q, const T *__restrict__ v,
    const unsigned char *__restrict__ params, const float *__restrict__ st, const float *__restrict__ gv,
    const float *__restrict__ gd, float *__restrict__ dq) {
    __shared__ __align__(16) float xq[64 * 68];   // query tile
    __shared__ __align__(16) float tb[64 * 68];   // T_t: row s, 65 columns, zero to 68
    __shared__ float wdl[2176];                    // wdec of the head
    const int tpc = C / 64, c = blockIdx.x / tpc, qt = blockIdx.x % tpc;
    // keys: blockIdx.y = KV head x kDkSplits, split p taking the steps t = 16 p .. 16 p + 15 (p = 0
    // also the linear step)
    const int h = KEYS ? blockIdx.y / kDkSplits : blockIdx.y, b = blockIdx.z, n_rep = n_q_heads / n_kv_heads;
    const int kv = KEYS ? h : h / n_rep, psplit = KEYS ? blockIdx.y % kDkSplits : 0;
    const int tbeg = KEYS ? 16 * psplit : 0;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, kg = lane >> 4, w = wave_id();
    const int t0 = c * C + qt * 64;
    if (t0 >= T_len) return;                       // a tile past the sequence (uniform)
    const size_t qrow = KEYS ? ((size_t)b * n_kv_heads + kv) * T_len : ((size_t)b * n_q_heads + h) * T_len;
    stage_rows(xq, 68, q, qrow, t0, T_len, 0.0f);
    if constexpr (!KEYS) {
        const OalHeadDev *hd = bwd_head(params, h);
        for (int f = tid; f < 2176; f += kThreads) wdl[f] = f < OAL_NFEAT ? hd->wdec[f] : 0.0f;
    }
    float ga[17];                                  // g of query 16 w + lr, column 4 s + kg
    {
        const int ta = t0 + 16 * w + lr;
        const bool ok = ta < T_len;
#pragma unroll
        for (int ks = 0; ks < 17; ++ks) {
            const int col = 4 * ks + kg;
            if constexpr (KEYS)
                ga[ks] = !ok ? 0.0f : col < 64 ? oal_ld(v + (qrow + ta) * OAL_D + col) : col == 64 ? 1.0f : 0.0f;
            else
                ga[ks] = !ok ? 0.0f : col < 64 ? gv[(qrow + ta) * OAL_D + col] : col == 64 ? gd[qrow + ta] : 0.0f;
        }
    }
    oal_f32x4 acc[4];                              // dq: query 16 w + 4 kg + jj, dim 16 st + lr
#pragma unroll
    for (int sti = 0; sti < 4; ++sti) acc[sti] = oal_splat(0.0f);
    if (KEYS ? c < nch - 1 : c > 0) {              // S_0 = 0, R of the last chunk = 0
        const float *S = st + ((size_t)((size_t)b * n_kv_heads + kv) * nch + c) * OAL_STATE_STRIDE;
        const float *Sd = S + (size_t)OAL_NFEAT * OAL_D;
        // T of the next step, this thread's share: rows s = (tid + 256 m) / 16, 4 columns each
        const int s0 = tid >> 4, c4 = (tid & 15) * 4;
        auto ld4 = [&](int srow, int t) {
            return *reinterpret_cast<const float4 *>(S + (size_t)dq_row_of(srow, t) * OAL_D + c4);
        };
        // queries: n = t (64 = the linear step); keys: t = 16 p + n, and n = 16 (split 0 only) the
        // linear step
        auto step_t = [&](int n) { return KEYS ? (n < 16 ? tbeg + n : OAL_D) : n; };
        const int nsteps = KEYS ? (psplit == 0 ? 17 : 16) : OAL_D + 1;
        float4 p0 = ld4(s0, step_t(0)), p1 = ld4(s0 + 16, step_t(0)), p2 = ld4(s0 + 32, step_t(0)),
               p3 = ld4(s0 + 48, step_t(0));
        float p64 = Sd[dq_row_of(tid & 63, step_t(0))];
        for (int n = 0; n < nsteps; ++n) {
            const int t = step_t(n);
            __syncthreads();                       // the previous T is consumed
            *reinterpret_cast<float4 *>(tb + s0 * 68 + c4) = p0;
            *reinterpret_cast<float4 *>(tb + (s0 + 16) * 68 + c4) = p1;
            *reinterpret_cast<float4 *>(tb + (s0 + 32) * 68 + c4) = p2;
            *reinterpret_cast<float4 *>(tb + (s0 + 48) * 68 + c4) = p3;
            if (tid < 64) {
                tb[tid * 68 + 64] = p64;
                tb[tid * 68 + 65] = tb[tid * 68 + 66] = tb[tid * 68 + 67] = 0.0f;
            }
            __syncthreads();
            {                                      // the last step reloads its own T (harmless)
                const int tn = step_t(n + 1 < nsteps ? n + 1 : n);
                p0 = ld4(s0, tn);
                p1 = ld4(s0 + 16, tn);
                p2 = ld4(s0 + 32, tn);
                p3 = ld4(s0 + 48, tn);
                p64 = Sd[dq_row_of(tid & 63, tn)];
            }
            oal_f32x4 X[4];
#pragma unroll
            for (int sti = 0; sti < 4; ++sti) X[sti] = oal_splat(0.0f);
#pragma unroll
            for (int ks = 0; ks < 17; ++ks) {
                const int col = 4 * ks + kg;
#pragma unroll
                for (int sti = 0; sti < 4; ++sti)
                    X[sti] = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[ks], tb[(16 * sti + lr) * 68 + col], X[sti], 0, 0, 0);
            }
#pragma unroll
            for (int sti = 0; sti < 4; ++sti) {
                const int sd = 16 * sti + lr;
                const float cst = KEYS ? (sd == t ? 2.0f : 1.0f)
                                       : t == OAL_D ? wdl[1 + sd] : (sd == t ? 2.0f : 1.0f) * wdl[dq_row_of(sd, t)];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float qf = t == OAL_D ? 1.0f : xq[(16 * w + 4 * kg + jj) * 68 + t];
                    acc[sti][jj] += cst * qf * X[sti][jj];
                }
            }
        }
    }
#pragma unroll
    for (int sti = 0; sti < 4; ++sti)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int tq = t0 + 16 * w + 4 * kg + jj;
            if (tq < T_len) {
                if constexpr (KEYS)   // part slot psplit, dk half; rows = B Hkv T
                    dq[((size_t)psplit * gridDim.z * n_kv_heads * T_len + qrow + tq) * 128 + 16 * sti + lr] = acc[sti][jj];
                else
                    dq[(qrow + tq) * OAL_D + 16 * sti + lr] = acc[sti][jj];
            }
        }
}

// 4b. dq_i += sum_{j <= i in the chunk} dkappa_ij dkappa_ij/dq_i, dkappa_ij = g_i . [v_j; 1], on
//     fp32 MFMA (16x16x4). dkappa/dq_ir = 2 k_jr sum_m z_m Lz[m][r] with
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
    __shared__ __align__(16) float ks[64 * 68];
    __shared__ __align__(16) float dks[64 * 68];   // dkappa tile
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
        __syncthreads();
        for (int e = tid; e < 64 * 64; e += kThreads) {
            const int i = e >> 6, j = e & 63;
            float x = 0.0f;
            if (kt < qt || j <= i) {
                const float *gi = gs + i * 68, *vj = vs + j * 68;
                float x1 = 0.0f;
                for (int cc = 0; cc < 64; cc += 2) {
                    x += gi[cc] * vj[cc];
                    x1 += gi[cc + 1] * vj[cc + 1];
                }
                x += x1 + gi[64];
            }
            dks[i * 68 + j] = x;
        }
        __syncthreads();                           // dkappa ready; gs and vs are free
        stage_rows(qs, 68, q, qrow, t0, T_len, 0.0f);
        __syncthreads();
        float *es = gs;
        for (int m = 0; m <= G; ++m) {
            const float *lzm = Lz + m * OAL_D;
            // Z_m for the wave's 16 queries x 64 keys
            oal_f32x4 Z[4];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) Z[jt] = oal_splat(m == 0 ? L00 : 0.0f);
#pragma unroll 4
            for (int st = 0; st < 16; ++st) {
                const int r = 4 * st + kg;
                const float a = qs[(16 * w + lr) * 68 + r] * lzm[r];
#pragma unroll
                for (int jt = 0; jt < 4; ++jt)
                    Z[jt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, ks[(16 * jt + lr) * 68 + r], Z[jt], 0, 0, 0);
            }
            // E_m = dkappa o Z_m into the wave's rows of es (row = query, column = key)
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int i = 16 * w + 4 * kg + jj, j = 16 * jt + lr;
                    es[i * 68 + j] = dks[i * 68 + j] * Z[jt][jj];
                }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // the wave reads its own rows
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            // F = E_m K for the wave's 16 queries x 64 dims, then dq += 2 Lz[m][r] F
            oal_f32x4 F[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) F[rt] = oal_splat(0.0f);
#pragma unroll 4
            for (int st = 0; st < 16; ++st) {
                const int j = 4 * st + kg;
                const float a = es[(16 * w + lr) * 68 + j];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
                    F[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, ks[j * 68 + 16 * rt + lr], F[rt], 0, 0, 0);
            }
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
//    - oal_bwd_dq_inter_mfma<KEYS>: the state part of dk, dk_j += Jpsi(k_j)^T (R_c [v_j; 1]);
//    - kInterSplits workgroups of oal_bwd_dv_inter: the 32 waves of the splits (worker
//      4 p + w) take the feature-row pairs {worker, 63 - worker} (65 features each) of the
//      state part of dv, dv_j += psi_f(k_j) R_c[f][0:64];
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


template <typename T>
__global__ __launch_bounds__(kThreads) void oal_bwd_dv_inter(int T_len, int C, int nch, int n_kv_heads,
                                                              const T *__restrict__ k, const float *__restrict__ st,
                                                              float *__restrict__ part) {
    __shared__ float xk[64 * 65];
    __shared__ float red[64 * 65];
    const int tpc = C / 64, c = blockIdx.x / tpc, kt = blockIdx.x % tpc;
    const int p = blockIdx.y % kInterSplits, kv = blockIdx.y / kInterSplits, b = blockIdx.z;
    const int j = threadIdx.x & 63, w = wave_id(), worker = p * 4 + w;
    const int t0 = c * C + kt * 64, t = t0 + j;
    const bool valid = t < T_len;
    const size_t krow = ((size_t)b * n_kv_heads + kv) * T_len, rows = (size_t)gridDim.z * n_kv_heads * T_len;
    stage_rows(xk, 65, k, krow, t0, T_len, 1.0f);
    __syncthreads();
    const float *xj = xk + j * 65;
    float a[64];
#pragma unroll
    for (int e = 0; e < 64; ++e) a[e] = 0.0f;
    if (c < nch - 1) {
        const float *Rg = st + ((size_t)((size_t)b * n_kv_heads + kv) * nch + c) * OAL_STATE_STRIDE;
        const cfloat *R = uni(Rg), *Rd = uni(Rg + (size_t)OAL_NFEAT * OAL_D);
        if (worker == 0) row_axpy<64>(a, 1.0f, R, Rd, 0);      // constant feature
        for (int half = 0; half < 2; ++half) {
            const int r = half ? 63 - worker : worker;
            const float kr = xj[r];
            const int base = quad_base(r);
            row_axpy<64>(a, kr, R, Rd, 1 + r);
#pragma unroll 4
            for (int tt = r; tt < OAL_D; ++tt) row_axpy<64>(a, kr * xj[tt], R, Rd, base + tt);
        }
    }
    for (int s = 0; s < 4; ++s) {
        __syncthreads();
        if (w == s) {
#pragma unroll
            for (int e = 0; e < 64; ++e) red[j * 65 + e] = (s == 0 ? 0.0f : red[j * 65 + e]) + a[e];
        }
    }
    __syncthreads();
    if (valid) {
        float *o = part_row(part, p, rows, krow + t) + 64 + w * 16;
        const float *src = red + j * 65 + w * 16;
#pragma unroll
        for (int e = 0; e < 16; e += 4)
            *reinterpret_cast<float4 *>(o + e) = make_float4(src[e], src[e + 1], src[e + 2], src[e + 3]);
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
        // dkr[it][jj] for key j = 16 w + 4 kg + jj, query i = 16 it + lr
        float dkr[4][4];
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int j = 16 * w + 4 * kg + jj, i = 16 * it + lr;
                float x = 0.0f;
                if (kt < qt || j <= i) {
                    const float *gi = gs + i * 68, *vj = es + j * 68;
                    float x1 = 0.0f;
                    for (int cc = 0; cc < 64; cc += 2) {
                        x += gi[cc] * vj[cc];
                        x1 += gi[cc + 1] * vj[cc + 1];
                    }
                    x += x1 + gi[64];
                }
                dkr[it][jj] = x;
            }
        __syncthreads();                           // the v tile is consumed
        oal_f32x4 kap[4];                          // sum_m Z_m^2: key 16 w + 4 kg + jj, query 16 it + lr
#pragma unroll
        for (int it = 0; it < 4; ++it) kap[it] = oal_splat(0.0f);
        for (int m = 0; m <= G; ++m) {
            const float *lzm = Lz + m * OAL_D;
            oal_f32x4 Z[4];
#pragma unroll
            for (int it = 0; it < 4; ++it) Z[it] = oal_splat(m == 0 ? L00 : 0.0f);
#pragma unroll 4
            for (int st = 0; st < 16; ++st) {
                const int r = 4 * st + kg;
                const float a = ks[(16 * w + lr) * 68 + r] * lzm[r];
#pragma unroll
                for (int it = 0; it < 4; ++it)
                    Z[it] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qs[(16 * it + lr) * 68 + r], Z[it], 0, 0, 0);
            }
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
// tile) pair: the tile of dkappa (masked to j <= i) in LDS, then on fp32 MFMA (16x16x4)
// Y = dkappa psi(K) (M = 64 queries in four 16-row tiles, N = features, K = 64 keys) and
// dw[f] += sum_i mono_f(q_i) Y[i][f]. Wave w takes the feature tiles w, w + 4, ...; lane l
// holds the A operand dkappa[16 it + l % 16][4 s + l / 16] in registers for the whole pair and
// builds the B operand psi_f(k_j) (f = 16 ft + l % 16, j = 4 s + l / 16) from the key tile.
template <typename T>
__global__ __launch_bounds__(kThreads) void oal_bwd_dw_intra(int T_len, int C, int nch, int n_q_heads,
                                                              int n_kv_heads, const T *__restrict__ q,
                                                              const T *__restrict__ k, const T *__restrict__ v,
                                                              const float *__restrict__ gv, const float *__restrict__ gd,
                                                              float *__restrict__ dwp) {
    constexpr int NFP = 2176, NFT = NFP / 16;      // features padded to 136 tiles of 16
    __shared__ __align__(16) float ta[64 * 68];   // g tile, then the query tile
    __shared__ __align__(16) float tb[64 * 68];   // v tile, then the key tile
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
    for (int qt = 0; qt < tpc; ++qt) {
        const int q0 = c * C + qt * 64;
        if (q0 >= T_len) break;
        for (int kt = 0; kt <= qt; ++kt) {
            const int k0 = c * C + kt * 64;
            __syncthreads();
            stage_g(ta, gv, gd, qrow, q0, T_len);
            stage_rows(tb, 68, v, krow, k0, T_len, 1.0f);
            __syncthreads();
            for (int e = tid; e < 64 * 64; e += kThreads) {
                const int i = e >> 6, j = e & 63;
                float x = 0.0f;
                if (kt < qt || j <= i) {
                    const float *gi = ta + i * 68, *vj = tb + j * 68;
                    float x1 = 0.0f;
                    for (int cc = 0; cc < 64; cc += 2) {
                        x += gi[cc] * vj[cc];
                        x1 += gi[cc + 1] * vj[cc + 1];
                    }
                    x += x1 + gi[64];
                }
                dk[i * 68 + j] = x;
            }
            __syncthreads();
            stage_rows(ta, 68, q, qrow, q0, T_len, 1.0f);
            stage_rows(tb, 68, k, krow, k0, T_len, 1.0f);
            __syncthreads();
            float A[4][16];                        // dkappa[16 it + lr][4 s + kg]
#pragma unroll
            for (int it = 0; it < 4; ++it)
#pragma unroll
                for (int st = 0; st < 16; ++st) A[it][st] = dk[(16 * it + lr) * 68 + 4 * st + kg];
            for (int ft = w; ft < NFT; ft += 4) {
                const int fB = 16 * ft + lr;                         // B operand feature of this lane
                const unsigned short abB = fdl[fB];
                oal_f32x4 D[4];
#pragma unroll
                for (int it = 0; it < 4; ++it) D[it] = oal_splat(0.0f);
#pragma unroll
                for (int st = 0; st < 16; ++st) {
                    const float *kr = tb + (4 * st + kg) * 68;
                    const float bpsi = kr[abB & 0xff] * kr[abB >> 8];
#pragma unroll
                    for (int it = 0; it < 4; ++it)
                        D[it] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[it][st], bpsi, D[it], 0, 0, 0);
                }
                // D[it][jj]: query 16 it + 4 kg + jj, feature 16 ft + lr
                float sum = 0.0f;
#pragma unroll
                for (int it = 0; it < 4; ++it)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float *qi = ta + (16 * it + 4 * kg + jj) * 68;
                        sum += qi[abB & 0xff] * qi[abB >> 8] * D[it][jj];
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
                           const float *dy, const unsigned char *params, void *ws, float *dq, float *dk, float *dv,
                           float *dL, float *deps, hipStream_t stream) {
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
    const bool coef = dL != nullptr;
    const dim3 blk(kThreads);
    const dim3 g_inc((OAL_NFEAT + kFeatBlock - 1) / kFeatBlock, nch, B * Hkv);
    const dim3 g_scan((OAL_NFEAT * OAL_V1 + kThreads - 1) / kThreads, B * Hkv);
    const dim3 g_q(nch * tpc, Hq, B), g_ki(nch * tpc, Hkv * kInterSplits, B), g_kh(nch * tpc, Hq, B);
    const dim3 g_red((unsigned)((kvrows * 32 + kThreads - 1) / kThreads));
    const int nslots = kInterSplits + Hq / Hkv;
    hipLaunchKernelGGL((oal_bwd_increments<T, false>), g_inc, blk, 0, stream, T_len, C, nch, Hq, Hkv, k, v,
                       (const float *)nullptr, (const float *)nullptr, params, st, (float *)nullptr);
    hipLaunchKernelGGL(oal_bwd_scan, g_scan, blk, 0, stream, nch, 0, st);
    hipLaunchKernelGGL(oal_bwd_readout_g<T>, g_q, blk, 0, stream, T_len, C, nch, Hq, Hkv, q, k, v, dy, params, st,
                       gv, gd);
    hipLaunchKernelGGL((oal_bwd_dq_inter_mfma<T, false>), g_q, blk, 0, stream, T_len, C, nch, Hq, Hkv, q,
                       (const T *)nullptr, params, st, gv, gd, dq);
    hipLaunchKernelGGL(oal_bwd_dq_intra_mfma<T>, g_q, blk, 0, stream, T_len, C, Hq, Hkv, q, k, v, params, gv, gd, dq);
    hipLaunchKernelGGL(oal_bwd_dkv_intra_mfma<T>, g_kh, blk, 0, stream, T_len, C, Hq, Hkv, q, k, v, params, gv, gd,
                       part);
    if (coef)
        hipLaunchKernelGGL(oal_bwd_dw_intra<T>, dim3(nch, Hq, B), blk, 0, stream, T_len, C, nch, Hq, Hkv, q, k, v,
                           gv, gd, dwp + (size_t)B * Hq * nch * OAL_NFEAT);
    hipLaunchKernelGGL((oal_bwd_increments<T, true>), g_inc, blk, 0, stream, T_len, C, nch, Hq, Hkv, q,
                       (const T *)nullptr, gv, gd, params, st, coef ? dwp : (float *)nullptr);
    if (coef) {
        float *dwt = dwp + 2 * (size_t)B * Hq * nch * OAL_NFEAT;
        hipLaunchKernelGGL(oal_bwd_dw_sum, dim3((OAL_NFEAT + kThreads - 1) / kThreads, Hq), blk, 0, stream, B, nch,
                           Hq, dwp, dwt);
        hipLaunchKernelGGL(oal_bwd_coef, dim3(Hq), blk, 0, stream, params, dwt, dL, deps);
    }
    hipLaunchKernelGGL(oal_bwd_scan, g_scan, blk, 0, stream, nch, 1, st);
    hipLaunchKernelGGL((oal_bwd_dq_inter_mfma<T, true>), dim3(nch * tpc, Hkv * kDkSplits, B), blk, 0, stream, T_len, C, nch, Hq,
                       Hkv, k, v, params, st, gv, gd, part);
    hipLaunchKernelGGL(oal_bwd_dv_inter<T>, g_ki, blk, 0, stream, T_len, C, nch, Hkv, k, st, part);
    hipLaunchKernelGGL(oal_bwd_kv_reduce, g_red, blk, 0, stream, kvrows, nslots, part, dk, dv);
    return hipGetLastError();
}

}  // namespace

size_t oal_backward_ws_bytes_impl(const oal_dims &d, int T_len, int C) {
    const size_t nch = (size_t)(T_len + C - 1) / C;
    return align256((size_t)d.batch * d.n_kv_heads * nch * OAL_STATE_STRIDE * 4) +
           align256((size_t)d.batch * d.n_q_heads * T_len * 64 * 4) + align256((size_t)d.batch * d.n_q_heads * T_len * 4) +
           align256((size_t)(kInterSplits + d.n_q_heads / d.n_kv_heads) * d.batch * d.n_kv_heads * T_len * 128 * 4) +
           align256(((size_t)2 * d.batch * nch + 1) * d.n_q_heads * OAL_NFEAT * 4);
}

hipError_t oal_launch_backward(const oal_dims &d, int T_len, int C, const void *q, const void *k, const void *v,
                               const float *dy, const void *params, void *ws, float *dq, float *dk, float *dv,
                               float *dL, float *deps, hipStream_t stream) {
    const unsigned char *p = static_cast<const unsigned char *>(params);
    if (d.dtype == OAL_BF16)
        return launch_backward<__bf16>(d, T_len, C, q, k, v, dy, p, ws, dq, dk, dv, dL, deps, stream);
    return launch_backward<float>(d, T_len, C, q, k, v, dy, p, ws, dq, dk, dv, dL, deps, stream);
}
