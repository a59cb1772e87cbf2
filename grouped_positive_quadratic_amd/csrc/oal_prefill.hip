// oal_prefill.hip -- chunked causal prefill on gfx950 MFMA.
//
// Method (reproduction notes of arXiv 2610.13674, section "核心公式"): the prefix states
// H = sum_{j<=i} psi(k_j)[v_j;1]^T (H0, H1, H2) and the readout u~_i = phi(q_i) . H turn
// the causal kernel sum into a linear-time recurrence. Tokens are processed in chunks of
// C: query i of chunk c reads the state S_c built from all tokens before the chunk, plus
// the exact kernel sum over keys j <= i of its own chunk:
//   u~_i = phi_h(q_i) . S_c + sum_{j in chunk c, j <= i} kappa_h(q_i, k_j) [v_j;1]
//
// Kernels, in launch order:
//  1. oal_scan<.., kTotals>  (only when the chunks are split into several segments)
//     per (sequence x KV head, segment, K-step): the state increment of the segment, and
//     for segment 0 a copy of the incoming state, into `totals`.
//  2. oal_scan<.., kSnapshots>
//     per (sequence x KV head, segment, K-step): start from the incoming state plus the
//     increments of the earlier segments, then walk the segment's chunks writing the state
//     before each chunk (bf16 or fp32, scaled, in the MFMA operand order of the readout)
//     and adding psi(K_c)^T [V_c;1] on MFMA. The last segment writes the final state back.
//  3. oal_readout
//     per (sequence x KV head x head group, chunk, 16-query tile): the query heads of one
//     KV head share every snapshot fragment. Two waves split the 72 K-steps of
//     phi(Q) . S_c (odd/even rq) and the intra-chunk heads, then combine through LDS and
//     divide: y = u~[0:64] / u~[64].
#include <hip/hip_runtime.h>

#include "oal.h"
#include "oal_device.h"
#include "oal_internal.h"

namespace {

constexpr int kScanWaves = 8;                 // K-steps per scan workgroup (72 = 9 x 8)
constexpr int kScanBlocks = OAL_KSTEPS / kScanWaves;
constexpr int kTotalsPerLane = 40;            // 2 tiles x 5 column tiles x 4 rows
enum { kTotals = 0, kSnapshots = 1 };

template <typename T> constexpr int snap_kstep_bytes() { return 4 * 64 * OalFrag<T>::kBytes + 4 * OalFrag<T>::kBytes; }

__device__ inline const OalHeadDev *head_ptr(const unsigned char *params, int h) {
    return reinterpret_cast<const OalHeadDev *>(params + sizeof(OalParamsHeader) + (size_t)h * OAL_HEAD_BYTES);
}

__device__ inline void kstep_decode(int s, int &tb, int &rq) {
    tb = 0;
    while ((tb + 1) * (tb + 2) <= s) ++tb;
    rq = s - tb * (tb + 1);
}

// scale of a slot in the snapshot state (relative to H) and its state row; -1 = empty slot
__device__ inline int slot_row(int tb, int rq, int g, int e, float &scale) {
    int ra, rb;
    int kind = oal_slot_kind(tb, rq, g, e, &ra, &rb);
    if (kind == OAL_SLOT_QUAD) { scale = (ra < rb ? 2.0f : 1.0f) / 64.0f; return oal_quad_row(ra, rb); }
    if (kind == OAL_SLOT_LIN) { scale = 0.125f; return 1 + ra; }
    if (kind == OAL_SLOT_CONST) { scale = 1.0f; return 0; }
    scale = 0.0f;
    return -1;
}

// ------------------------------------------------------------------------------------
// chunk-state scan
template <typename T, int C, int MODE>
__global__ __launch_bounds__(64 * kScanWaves) void oal_scan(
    int T_len, int nchunks, int nseg, int seg_len, const T *__restrict__ k,
    const T *__restrict__ v, float *__restrict__ state, float *__restrict__ totals,
    unsigned char *__restrict__ snap) {
    constexpr int LD = C + 16 / (int)sizeof(T) * 2;     // padded row (keeps 16-byte alignment)
    extern __shared__ __align__(16) unsigned char smem[];
    T *s_kT = reinterpret_cast<T *>(smem);              // [65][LD], row 64 = valid-token ones
    T *s_vT = s_kT + 65 * LD;                           // [64][LD]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lr = lane & 15;
    const int s = blockIdx.x * kScanWaves + wave;
    const int sigma = blockIdx.y;
    const int bkv = blockIdx.z;
    int tb, rq;
    kstep_decode(s, tb, rq);

    // A operand (psi^T): this lane's feature row lr of tile h is slot (lr/4, 4h + lr%4)
    int ra[2], rb[2];
    float sig[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int a, bb;
        int kind = oal_slot_kind(tb, rq, lr >> 2, 4 * h + (lr & 3), &a, &bb);
        ra[h] = a;
        rb[h] = bb;
        sig[h] = kind == OAL_SLOT_QUAD ? (a < bb ? 2.0f : 1.0f) / 64.0f
               : kind == OAL_SLOT_LIN  ? 0.125f
               : kind == OAL_SLOT_CONST ? 1.0f : 0.0f;
    }

    oal_f32x4 acc[2][5];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int n = 0; n < 5; ++n) acc[h][n] = oal_splat(0.0f);

    float *Sst = state + (size_t)bkv * OAL_NFEAT * OAL_V1;
    auto read_state = [&]() {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int n = 0; n < 5; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float sc;
                    int f = slot_row(tb, rq, g, 4 * h + i, sc);
                    int col = n < 4 ? 16 * n + lr : (lr == 0 ? OAL_D : -1);
                    acc[h][n][i] = (f >= 0 && col >= 0) ? Sst[(size_t)f * OAL_V1 + col] * sc : 0.0f;
                }
    };
    auto totals_at = [&](int idx) {
        return totals + (((size_t)bkv * nseg + idx) * OAL_KSTEPS + s) * kTotalsPerLane * 64 + lane;
    };

    const int c0 = sigma * seg_len, c1 = min(nchunks, c0 + seg_len);
    if (MODE == kTotals) {
        if (sigma == 0) {
            read_state();
            float *tp = totals_at(0);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int n = 0; n < 5; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        tp[((h * 5 + n) * 4 + i) * 64] = acc[h][n][i];
                        acc[h][n][i] = 0.0f;
                    }
        }
    } else {
        if (nseg == 1) {
            read_state();
        } else {
            for (int sg = 0; sg <= sigma; ++sg) {
                const float *tp = totals_at(sg);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int n = 0; n < 5; ++n)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[h][n][i] += tp[((h * 5 + n) * 4 + i) * 64];
            }
        }
    }

    const T *kb = k + (size_t)bkv * T_len * OAL_D;
    const T *vb = v + (size_t)bkv * T_len * OAL_D;
    OalFrag<T> ones, zeros;
    {
        float o[8], zz[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) { o[e] = 1.0f; zz[e] = 0.0f; }
        ones.set(o);
        zeros.set(zz);
    }
    constexpr int KB = snap_kstep_bytes<T>();

    for (int c = c0; c < c1; ++c) {
        __syncthreads();
        for (int idx = tid; idx < C * OAL_D; idx += 64 * kScanWaves) {
            int tok = idx / OAL_D, dim = idx % OAL_D;
            int pos = c * C + tok;
            bool ok = pos < T_len;
            s_kT[dim * LD + tok] = ok ? kb[(size_t)pos * OAL_D + dim] : (T)0.0f;
            s_vT[dim * LD + tok] = ok ? vb[(size_t)pos * OAL_D + dim] : (T)0.0f;
            if (dim == 0) s_kT[OAL_D * LD + tok] = ok ? (T)1.0f : (T)0.0f;
        }
        __syncthreads();
        if (MODE == kSnapshots) {
            unsigned char *sp = snap + (((size_t)bkv * nchunks + c) * OAL_KSTEPS + s) * KB;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                float x[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) { x[i] = acc[0][n][i]; x[4 + i] = acc[1][n][i]; }
                OalFrag<T> f;
                f.set(x);
                f.store(sp + (n * 64 + lane) * OalFrag<T>::kBytes);
            }
            if (lr == 0) {
                float x[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) { x[i] = acc[0][4][i]; x[4 + i] = acc[1][4][i]; }
                OalFrag<T> f;
                f.set(x);
                f.store(sp + (4 * 64 + g) * OalFrag<T>::kBytes);
            }
        }
#pragma unroll
        for (int sb = 0; sb < C / 32; ++sb) {
            const int t0 = 32 * sb + 8 * g;
            OalFrag<T> a[2], bf[4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    x[e] = sig[h] * (float)s_kT[ra[h] * LD + t0 + e] * (float)s_kT[rb[h] * LD + t0 + e];
                a[h].set(x);
            }
#pragma unroll
            for (int n = 0; n < 4; ++n) bf[n].load(s_vT + (16 * n + lr) * LD + t0);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int n = 0; n < 4; ++n) acc[h][n] = oal_mma(a[h], bf[n], acc[h][n]);
                acc[h][4] = oal_mma(a[h], lr == 0 ? ones : zeros, acc[h][4]);
            }
        }
    }

    if (MODE == kTotals) {
        float *tp = totals_at(sigma + 1);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int n = 0; n < 5; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) tp[((h * 5 + n) * 4 + i) * 64] = acc[h][n][i];
    } else if (sigma == nseg - 1) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int n = 0; n < 5; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float sc;
                    int f = slot_row(tb, rq, g, 4 * h + i, sc);
                    int col = n < 4 ? 16 * n + lr : (lr == 0 ? OAL_D : -1);
                    if (f >= 0 && col >= 0) Sst[(size_t)f * OAL_V1 + col] = acc[h][n][i] / sc;
                }
    }
}

// ------------------------------------------------------------------------------------
// readout
constexpr int kPS = 68;   // padded LDS row of the per-query tables (16-byte aligned rows)

template <typename T, int C, int R>
__global__ __launch_bounds__(128) void oal_readout(
    int T_len, int n_q_heads, int n_kv_heads, int nchunks, int n_hgroups,
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const unsigned char *__restrict__ params, const unsigned char *__restrict__ snap,
    float *__restrict__ y) {
    constexpr int LDV = C + 16 / (int)sizeof(T) * 2;
    extern __shared__ __align__(16) unsigned char smem[];
    float *s_p = reinterpret_cast<float *>(smem);      // [R][16][kPS]  w0[r] q_r
    float *s_q = s_p + R * 16 * kPS;                   // [R][16][kPS]  q_r
    T *s_vT = reinterpret_cast<T *>(s_q + R * 16 * kPS);   // [64][LDV]

    const int qt = blockIdx.x, c = blockIdx.y;
    const int bkv = blockIdx.z / n_hgroups, hg = blockIdx.z % n_hgroups;
    const int b = bkv / n_kv_heads, kv = bkv % n_kv_heads;
    const int n_rep = n_q_heads / n_kv_heads;
    const int h0 = kv * n_rep + hg * R;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lr = lane & 15;
    const int pos0 = c * C + qt * 16;
    if (pos0 >= T_len) return;

    // 1. query tables
    for (int idx = tid; idx < R * 16 * OAL_D; idx += 128) {
        int i = idx / (16 * OAL_D), qi = (idx / OAL_D) % 16, r = idx % OAL_D;
        int pos = pos0 + qi;
        float qv = pos < T_len ? oal_ld(q + (((size_t)b * n_q_heads + h0 + i) * T_len + pos) * OAL_D + r) : 0.0f;
        s_q[(i * 16 + qi) * kPS + r] = qv;
        s_p[(i * 16 + qi) * kPS + r] = head_ptr(params, h0 + i)->w0[r] * qv;
    }
    // 2. V^T of this chunk's keys that the tile can see (rounded up to 32; zero past T)
    const int nkeys = ((qt + 2) / 2) * 32;
    const T *vb = v + (size_t)bkv * T_len * OAL_D;
    for (int idx = tid; idx < nkeys * OAL_D; idx += 128) {
        int key = idx / OAL_D, col = idx % OAL_D;
        int pos = c * C + key;
        s_vT[col * LDV + key] = pos < T_len ? vb[(size_t)pos * OAL_D + col] : (T)0.0f;
    }
    __syncthreads();

    oal_f32x4 acc[R][5];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int n = 0; n < 5; ++n) acc[i][n] = oal_splat(0.0f);

    // 3. inter-chunk: phi(Q) . S_c over this wave's 36 K-steps (rq = 2 j + wave)
    constexpr int KB = snap_kstep_bytes<T>();
    const unsigned char *sbase = snap + ((size_t)bkv * nchunks + c) * OAL_KSTEPS * KB;
    auto load_b = [&](OalFrag<T> (&bf)[5], int s) {
        const unsigned char *sp = sbase + (size_t)s * KB;
#pragma unroll
        for (int n = 0; n < 4; ++n) bf[n].load(sp + (n * 64 + lane) * OalFrag<T>::kBytes);
        if (lr == 0) bf[4].load(sp + (4 * 64 + g) * OalFrag<T>::kBytes);
        else bf[4].zero();
    };
    {
        OalFrag<T> bcur[5], bnext[5];
        float pt[R][8];
        int tb = 0, j = 0;
        load_b(bcur, oal_kstep(0, wave));
        for (int it = 0; it < OAL_KSTEPS / 2; ++it) {
            const int rq = 2 * j + wave;
            const int s = oal_kstep(tb, rq);
            int ntb = tb, nj = j + 1;
            if (nj > tb) { ntb = tb + 1; nj = 0; }
            if (it + 1 < OAL_KSTEPS / 2) load_b(bnext, oal_kstep(ntb, 2 * nj + wave));
            if (j == 0) {
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const float4 *pp = reinterpret_cast<const float4 *>(s_p + (i * 16 + lr) * kPS + 8 * tb);
                    float4 x0 = pp[0], x1 = pp[1];
                    pt[i][0] = x0.x; pt[i][1] = x0.y; pt[i][2] = x0.z; pt[i][3] = x0.w;
                    pt[i][4] = x1.x; pt[i][5] = x1.y; pt[i][6] = x1.z; pt[i][7] = x1.w;
                }
            }
            const bool lin_step = (rq == 2 * tb + 1);
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const OalHeadDev *hd = head_ptr(params, h0 + i);
                const float *qrow = s_q + (i * 16 + lr) * kPS;
                const float pr = s_p[(i * 16 + lr) * kPS + 4 * rq + g];
                float phi[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) phi[e] = pr * pt[i][e];
                if (lin_step) {
                    const int r0 = 8 * tb + 2 * g;
                    phi[0] = hd->lin[r0] * qrow[r0];
                    phi[1] = hd->lin[r0 + 1] * qrow[r0 + 1];
                    if (tb == 0 && g == 0) phi[2] = hd->a;
                }
                if ((hd->corr[s >> 5] >> (s & 31)) & 1u) {
                    const int r = 4 * rq + g;
                    const int gr = hd->gamma[r];
                    const float qr = qrow[r];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int t = 8 * tb + e;
                        const int gt = hd->gamma[t];
                        if (gt != hd->bulk && r <= t) phi[e] += hd->Dg[gr * OAL_D + gt] * qr * qrow[t];
                    }
                }
                OalFrag<T> a;
                a.set(phi);
#pragma unroll
                for (int n = 0; n < 5; ++n) acc[i][n] = oal_mma(a, bcur[n], acc[i][n]);
            }
#pragma unroll
            for (int n = 0; n < 5; ++n) bcur[n] = bnext[n];
            tb = ntb;
            j = nj;
        }
    }

    // 4. intra-chunk: kappa = eps + sum_m z_m^2 with z_m = L00 [m==0] + sum_r Lz[m][r] q_r k_r,
    //    z_m^T tiles (16 keys x 16 queries) on MFMA, then kappa [V;1] on MFMA.
    const T *kb = k + (size_t)bkv * T_len * OAL_D;
    OalFrag<T> ones, zeros;
    {
        float o[8], zz[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) { o[e] = 1.0f; zz[e] = 0.0f; }
        ones.set(o);
        zeros.set(zz);
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        if ((i & 1) != wave) continue;
        const OalHeadDev *hd = head_ptr(params, h0 + i);
        const float *qrow = s_q + (i * 16 + lr) * kPS;
        oal_f32x4 kap[C / 16];
#pragma unroll
        for (int kt = 0; kt < C / 16; ++kt) kap[kt] = oal_splat(hd->eps);
        const int G = hd->G;
        for (int m = 0; m <= G; ++m) {
            OalFrag<T> bq[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    int r = 32 * hh + 8 * g + e;
                    x[e] = hd->Lz[m * OAL_D + r] * qrow[r];
                }
                bq[hh].set(x);
            }
            const oal_f32x4 cinit = oal_splat(m == 0 ? hd->L00 : 0.0f);
#pragma unroll
            for (int kt = 0; kt < C / 16; ++kt) {
                if (kt <= qt) {
                    const int kpos = c * C + 16 * kt + lr;
                    OalFrag<T> ak[2];
                    if (kpos < T_len) {
                        ak[0].load(kb + (size_t)kpos * OAL_D + 8 * g);
                        ak[1].load(kb + (size_t)kpos * OAL_D + 32 + 8 * g);
                    } else {
                        ak[0].zero();
                        ak[1].zero();
                    }
                    oal_f32x4 z = oal_mma(ak[0], bq[0], cinit);
                    z = oal_mma(ak[1], bq[1], z);
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) kap[kt][ii] += z[ii] * z[ii];
                }
            }
        }
        // causal mask (key <= query, key < T), then kappa [V;1]
        const int qpos = pos0 + lr;
#pragma unroll
        for (int kt = 0; kt < C / 16; ++kt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                int kp = c * C + 16 * kt + 4 * g + ii;
                if (!(kt <= qt && kp <= qpos && kp < T_len)) kap[kt][ii] = 0.0f;
            }
#pragma unroll
        for (int p = 0; p < C / 32; ++p) {
            if (2 * p <= qt) {
                float x[8];
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    x[ii] = kap[2 * p][ii];
                    x[4 + ii] = kap[2 * p + 1][ii];
                }
                OalFrag<T> a;
                a.set(x);
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    const T *vr = s_vT + (16 * n + lr) * LDV + 32 * p + 4 * g;
                    OalFrag<T> bv;
                    bv.load4x2(vr, vr + 16);
                    acc[i][n] = oal_mma(a, bv, acc[i][n]);
                }
                acc[i][4] = oal_mma(a, lr == 0 ? ones : zeros, acc[i][4]);
            }
        }
    }

    // 5. combine the two waves' partial sums and divide
    __syncthreads();
    float *s_x = reinterpret_cast<float *>(smem);      // [R][5][4][64]
#pragma unroll
    for (int i = 0; i < R; ++i)
        if ((i & 1) != wave)
#pragma unroll
            for (int n = 0; n < 5; ++n)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) s_x[((i * 5 + n) * 4 + ii) * 64 + lane] = acc[i][n][ii];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < R; ++i) {
        if ((i & 1) != wave) continue;
#pragma unroll
        for (int n = 0; n < 5; ++n)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) acc[i][n][ii] += s_x[((i * 5 + n) * 4 + ii) * 64 + lane];
        float *yh = y + ((size_t)b * n_q_heads + h0 + i) * T_len * OAL_D;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            float den = __shfl(acc[i][4][ii], lane & 48);
            int pos = pos0 + 4 * g + ii;
            if (pos < T_len) {
#pragma unroll
                for (int n = 0; n < 4; ++n) yh[(size_t)pos * OAL_D + 16 * n + lr] = acc[i][n][ii] / den;
            }
        }
    }
}

template <typename T, int C>
size_t scan_lds() { return (size_t)(65 + 64) * (C + 16 / sizeof(T) * 2) * sizeof(T); }

template <typename T, int C, int R>
size_t readout_lds() {
    size_t tables = (size_t)2 * R * 16 * kPS * sizeof(float);
    size_t vt = (size_t)64 * (C + 16 / sizeof(T) * 2) * sizeof(T);
    size_t x = (size_t)R * 5 * 4 * 64 * sizeof(float);
    size_t a = tables + vt;
    return a > x ? a : x;
}

struct PrefillPlan {
    int nchunks, nseg, seg_len;
    size_t snap_bytes, totals_bytes;
};

template <typename T>
PrefillPlan make_plan(const oal_dims &d, int T_len, int C) {
    PrefillPlan p;
    size_t bkv = (size_t)d.batch * d.n_kv_heads;
    p.nchunks = (T_len + C - 1) / C;
    int target = 1;
    const char *env = getenv("OAL_NSEG");
    if (env && atoi(env) > 0) {
        target = atoi(env);
    } else {
        size_t waves = bkv * OAL_KSTEPS;
        target = (int)((1024 + waves / 2) / waves);
        if (target < 1) target = 1;
    }
    if (target > p.nchunks) target = p.nchunks;
    if (target < 1) target = 1;
    p.seg_len = (p.nchunks + target - 1) / target;
    p.nseg = (p.nchunks + p.seg_len - 1) / p.seg_len;
    p.snap_bytes = bkv * p.nchunks * OAL_KSTEPS * (size_t)snap_kstep_bytes<T>();
    p.snap_bytes = (p.snap_bytes + 255) / 256 * 256;
    p.totals_bytes = p.nseg > 1 ? bkv * p.nseg * OAL_KSTEPS * (size_t)kTotalsPerLane * 64 * sizeof(float) : 0;
    return p;
}

template <typename T, int C, int R>
hipError_t launch_readout(const oal_dims &d, int T_len, const PrefillPlan &p, const void *q,
                          const void *k, const void *v, const void *params,
                          const unsigned char *snap, float *y, hipStream_t stream) {
    int n_rep = d.n_q_heads / d.n_kv_heads;
    int n_hg = n_rep / R;
    size_t lds = readout_lds<T, C, R>();
    auto kern = oal_readout<T, C, R>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    dim3 grid(C / 16, p.nchunks, d.batch * d.n_kv_heads * n_hg);
    hipLaunchKernelGGL(kern, grid, dim3(128), lds, stream, T_len, d.n_q_heads, d.n_kv_heads,
                       p.nchunks, n_hg, reinterpret_cast<const T *>(q), reinterpret_cast<const T *>(k),
                       reinterpret_cast<const T *>(v), reinterpret_cast<const unsigned char *>(params),
                       snap, y);
    return hipGetLastError();
}

template <typename T, int C>
hipError_t launch_all(const oal_dims &d, int T_len, const void *q, const void *k, const void *v,
                      const void *params, float *state, void *ws, float *y, hipStream_t stream,
                      hipEvent_t *marks) {
    PrefillPlan p = make_plan<T>(d, T_len, C);
    if (marks && hipEventRecord(marks[0], stream) != hipSuccess) return hipErrorUnknown;
    unsigned char *snap = reinterpret_cast<unsigned char *>(ws);
    float *totals = reinterpret_cast<float *>(snap + p.snap_bytes);
    int bkv = d.batch * d.n_kv_heads;
    size_t lds = scan_lds<T, C>();
    const T *kk = reinterpret_cast<const T *>(k), *vv = reinterpret_cast<const T *>(v);
    if (p.nseg > 1) {
        auto kern = oal_scan<T, C, kTotals>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(kScanBlocks, p.nseg - 1, bkv), dim3(64 * kScanWaves), lds, stream,
                           T_len, p.nchunks, p.nseg, p.seg_len, kk, vv, state, totals, snap);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
        auto kern = oal_scan<T, C, kSnapshots>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(kScanBlocks, p.nseg, bkv), dim3(64 * kScanWaves), lds, stream,
                           T_len, p.nchunks, p.nseg, p.seg_len, kk, vv, state, totals, snap);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (marks && hipEventRecord(marks[1], stream) != hipSuccess) return hipErrorUnknown;
    int n_rep = d.n_q_heads / d.n_kv_heads;
    hipError_t e;
    if (n_rep % 8 == 0) e = launch_readout<T, C, 8>(d, T_len, p, q, k, v, params, snap, y, stream);
    else if (n_rep % 7 == 0) e = launch_readout<T, C, 7>(d, T_len, p, q, k, v, params, snap, y, stream);
    else if (n_rep % 4 == 0) e = launch_readout<T, C, 4>(d, T_len, p, q, k, v, params, snap, y, stream);
    else if (n_rep % 2 == 0) e = launch_readout<T, C, 2>(d, T_len, p, q, k, v, params, snap, y, stream);
    else e = launch_readout<T, C, 1>(d, T_len, p, q, k, v, params, snap, y, stream);
    if (e == hipSuccess && marks) e = hipEventRecord(marks[2], stream);
    return e;
}

}  // namespace

size_t oal_prefill_ws_bytes_impl(const oal_dims &d, int T_len, int C) {
    PrefillPlan p = d.dtype == OAL_BF16 ? make_plan<__bf16>(d, T_len, C) : make_plan<float>(d, T_len, C);
    return p.snap_bytes + p.totals_bytes;
}

hipError_t oal_launch_prefill(const oal_dims &d, int T_len, int C, const void *q, const void *k,
                              const void *v, const void *params, float *state, void *ws, float *y,
                              hipStream_t stream, hipEvent_t *marks) {
    if (d.dtype == OAL_BF16) {
        if (C == 64) return launch_all<__bf16, 64>(d, T_len, q, k, v, params, state, ws, y, stream, marks);
        if (C == 128) return launch_all<__bf16, 128>(d, T_len, q, k, v, params, state, ws, y, stream, marks);
        return launch_all<__bf16, 256>(d, T_len, q, k, v, params, state, ws, y, stream, marks);
    }
    if (C == 64) return launch_all<float, 64>(d, T_len, q, k, v, params, state, ws, y, stream, marks);
    if (C == 128) return launch_all<float, 128>(d, T_len, q, k, v, params, state, ws, y, stream, marks);
    return launch_all<float, 256>(d, T_len, q, k, v, params, state, ws, y, stream, marks);
}
