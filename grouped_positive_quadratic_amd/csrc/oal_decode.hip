// oal_decode.hip -- one decode step: stream each (sequence, KV head) state once.
//
// For the new token (reproduction notes of arXiv 2610.13674, section "核心公式"):
//   H <- H + psi(k) [v;1]^T           (prefix-state recurrence, H_i = H_{i-1} + term_i)
//   u~_h = phi_h(q_h) . H   for every query head h of the KV head (readout display)
//   y_h = u~_h[0:64] / u~_h[64]
// with psi(k) = [1, k_r, k_r k_t (r <= t)] and phi_h(q) = wdec_h o [1, q_r, q_r q_t].
//
// The state row f of a KV head holds 65 floats: 64 in a 256-byte row of the v part and one
// in the separate column-64 vector (the state layout keeps the v part line-aligned).
// Workgroup (split, bkv) owns 192 rows (384 for large batches); wave w walks a quarter of them
// in batches of 16 with lane c
// on column c (one aligned 256-byte row read and write per row) and the batch's 16
// column-64 entries (64 contiguous bytes) on lanes 0..15. With 260-byte rows (column 64
// inline) the rows straddled cache lines and the kernel wrote 17% more bytes than the state
// holds; the split layout brought a step from 31-32 to 30 us. The next batch is loaded while the
// current one is updated, and the first batch is requested together with everything the
// set-up reads (k, q, v, decode coefficients): the set-up costs one memory round trip, spent
// while the first rows arrive. Every byte of the state is read once and written once.
// Readout partial sums per split go to the workspace; the last workgroup of a (sequence, KV
// head) to arrive sums the splits in a fixed order, divides and writes y, then resets the
// arrival counter. No device-wide fence is used: it would write back the whole L2, full of
// fresh state rows.
#include <hip/hip_runtime.h>

#include <atomic>

#include "oal.h"
#include "oal_device.h"
#include "oal_internal.h"

namespace {

// State rows per workgroup: 192 (12 splits) up to kBigBatchBkv (sequence, KV head) blocks,
// 384 (6 splits) from there on. Measured on MI355X, 14q/2kv bf16 steps: 64 sequences 30.6 us
// with 192 rows, 31.5 us with 384; 512 sequences 276 us with 192 rows, 254 us with 384 (each
// workgroup's set-up is paid over more rows once the grid runs in several rounds).
constexpr int kThreads = 256;
constexpr int kRowsSmall = 192, kRowsBig = 384;
constexpr int kBigBatchBkv = 512;
constexpr int splits_of(int rows) { return (OAL_NFEAT + rows - 1) / rows; }
constexpr int kSplits = splits_of(kRowsSmall);   // the most splits: sizes the partial sums
constexpr int kBatch = 16;                  // rows per load batch of a wave
static_assert(8 * OAL_D % kThreads == 0, "query staging");

// Dims of state row f: (-1, -1) the constant, (r, -1) linear feature r, else the quadratic
// pair (r, t), r <= t, whose rows start at 65 + start(r), start(r) = 64 r - r (r - 1) / 2.
// r is the root of start(r) = i rounded down (fp32 square root, then a +-1 correction; exact
// for every i < 2080).
__device__ inline int quad_start(int r) { return OAL_D * r - (r * (r - 1)) / 2; }
__device__ inline void row_dims(int f, int &r, int &t) {
    if (f == 0) { r = -1; t = -1; return; }
    if (f <= OAL_D) { r = f - 1; t = -1; return; }
    const int i = f - 1 - OAL_D;
    int rr = (int)floorf((129.0f - sqrtf(16641.0f - 8.0f * (float)i)) * 0.5f);
    if (quad_start(rr + 1) <= i) ++rr;
    if (quad_start(rr) > i) --rr;
    r = rr;
    t = rr + (i - quad_start(rr));
}

template <typename T, int MAXH, int kRows>
__global__ __launch_bounds__(kThreads) void oal_decode_kernel(
    int n_q_heads, int n_kv_heads, const T *__restrict__ q, const T *__restrict__ k,
    const T *__restrict__ v, const unsigned char *__restrict__ params, float *__restrict__ state,
    const int *__restrict__ slots, int pool_size, float *__restrict__ partial,
    unsigned int *__restrict__ counters, float *__restrict__ y) {
    static_assert(kRows % 4 == 0 && kRows <= 2 * kThreads, "rows per workgroup");
    constexpr int kRowsPerWave = kRows / 4;
    constexpr int NSPL = splits_of(kRows);
    const int split = blockIdx.x;
    const int bkv = blockIdx.y;
    const int b = bkv / n_kv_heads, kv = bkv % n_kv_heads;
    const int n_rep = n_q_heads / n_kv_heads;
    const int h0 = kv * n_rep;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int f0 = split * kRows;
    // state block: sequence b's own, or pool block slots[b] (indexed decode). A slot outside
    // the pool streams no rows: the sequence's sums stay zero and its y is 0/0 = NaN.
    const int sb = slots ? slots[b] : b;
    const bool valid = sb >= 0 && sb < pool_size;
    const int nrows = valid ? min(kRows, OAL_NFEAT - f0) : 0;

    __shared__ float s_k[OAL_D];
    __shared__ float s_q[MAXH][OAL_D];
    __shared__ float s_psi[kRows];
    __shared__ __align__(16) float s_phi[kRows][MAXH];
    __shared__ float s_red[4][MAXH][OAL_V1];
    __shared__ int s_last;

    float *S = state + ((size_t)(valid ? sb : 0) * n_kv_heads + kv) * OAL_STATE_STRIDE;
    const int rbeg = wave * kRowsPerWave, rend = min(nrows, rbeg + kRowsPerWave);
    // one batch: 16 rows with lane = column, and column 64 of the same rows on lanes 0..15
    auto load_batch = [&](int rr, float *x, float &x64) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            x[u] = (rr + u < rend) ? S[(size_t)(f0 + rr + u) * OAL_D + lane] : 0.0f;
        x64 = (lane < kBatch && rr + lane < rend) ? S[(size_t)OAL_NFEAT * OAL_D + f0 + rr + lane] : 0.0f;
    };

    // 1. every global load of the set-up in one round trip: the first state batch, k, the
    //    queries, v, and the decode coefficients of this thread's rows
    float s[kBatch], s64;
    load_batch(rbeg, s, s64);
    const float kk = tid < OAL_D ? oal_ld(k + (size_t)bkv * OAL_D + tid) : 0.0f;
    const T *qb = q + ((size_t)b * n_q_heads + h0) * OAL_D;
    constexpr int kQIters = MAXH * OAL_D / kThreads;
    float qv[kQIters];
#pragma unroll
    for (int it = 0; it < kQIters; ++it)
        qv[it] = tid + it * kThreads < n_rep * OAL_D ? oal_ld(qb + tid + it * kThreads) : 0.0f;
    const float vv = oal_ld(v + (size_t)bkv * OAL_D + lane);
    constexpr int kRowIters = (kRows + kThreads - 1) / kThreads;
    float w[kRowIters][MAXH];
#pragma unroll
    for (int it = 0; it < kRowIters; ++it) {
        const int rr = tid + it * kThreads;
#pragma unroll
        for (int h = 0; h < MAXH; ++h) {
            const OalHeadDev *hd = reinterpret_cast<const OalHeadDev *>(
                params + sizeof(OalParamsHeader) + (size_t)(h0 + min(h, n_rep - 1)) * OAL_HEAD_BYTES);
            w[it][h] = (rr < nrows && h < n_rep) ? hd->wdec[f0 + rr] : 0.0f;
        }
    }
    if (tid < OAL_D) s_k[tid] = kk;
#pragma unroll
    for (int it = 0; it < kQIters; ++it) {
        const int idx = tid + it * kThreads;
        if (idx < n_rep * OAL_D) s_q[idx / OAL_D][idx % OAL_D] = qv[it];
    }
    __syncthreads();

    // 2. features of this workgroup's rows: psi (key) and phi_h (query, with coefficient)
#pragma unroll
    for (int it = 0; it < kRowIters; ++it) {
        const int rr = tid + it * kThreads;
        if (rr < kRows) {
            float psi = 0.0f;
            float ph[MAXH];
#pragma unroll
            for (int h = 0; h < MAXH; ++h) ph[h] = 0.0f;
            if (rr < nrows) {
                int r, t;
                row_dims(f0 + rr, r, t);
                psi = (r < 0) ? 1.0f : (t < 0 ? s_k[r] : s_k[r] * s_k[t]);
#pragma unroll
                for (int h = 0; h < MAXH; ++h) {
                    float mono = (r < 0) ? 1.0f : (t < 0 ? s_q[h][r] : s_q[h][r] * s_q[h][t]);
                    ph[h] = w[it][h] * mono;
                }
            }
#pragma unroll
            for (int h = 0; h < MAXH; ++h) s_phi[rr][h] = ph[h];
            s_psi[rr] = psi;
        }
    }
    __syncthreads();

    // 3. stream the rows: S += psi [v;1], written back; readout sums of the updated rows.
    //    The next batch is in flight while the current one is updated.
    float acc[MAXH], accd[MAXH];
#pragma unroll
    for (int h = 0; h < MAXH; ++h) { acc[h] = 0.0f; accd[h] = 0.0f; }
    for (int rr = rbeg; rr < rend; rr += kBatch) {
        float sn[kBatch], sn64 = 0.0f;
        const bool more = rr + kBatch < rend;
        if (more) load_batch(rr + kBatch, sn, sn64);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (rr + u < rend) {
                s[u] += s_psi[rr + u] * vv;
                S[(size_t)(f0 + rr + u) * OAL_D + lane] = s[u];
#pragma unroll
                for (int h = 0; h < MAXH; ++h) acc[h] += s_phi[rr + u][h] * s[u];
            }
        }
        if (lane < kBatch && rr + lane < rend) {
            s64 += s_psi[rr + lane];
            S[(size_t)OAL_NFEAT * OAL_D + f0 + rr + lane] = s64;
#pragma unroll
            for (int h = 0; h < MAXH; ++h) accd[h] += s_phi[rr + lane][h] * s64;
        }
        if (more) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u) s[u] = sn[u];
            s64 = sn64;
        }
    }
#pragma unroll
    for (int h = 0; h < MAXH; ++h) {
        float x = accd[h];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
        s_red[wave][h][lane] = acc[h];
        if (lane == 0) s_red[wave][h][OAL_D] = x;
    }
    __syncthreads();
    // 4. cross-workgroup combine. Partials are written and read with agent-scope atomics, which
    //    are coherent across the XCDs' L2 caches. Every wave waits for its partial stores to
    //    complete before the barrier, so all of them are performed before thread 0's arrival
    //    RMW; the last workgroup to arrive issues its loads only after its own RMW returned,
    //    so it reads every split's partial (no L2 write-back is needed for that).
    float *mypart = partial + ((size_t)bkv * NSPL + split) * MAXH * OAL_V1;
    for (int idx = tid; idx < n_rep * OAL_V1; idx += kThreads) {
        int h = idx / OAL_V1, c = idx % OAL_V1;
        __hip_atomic_store(mypart + idx, s_red[0][h][c] + s_red[1][h][c] + s_red[2][h][c] + s_red[3][h][c],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    oal_wait_own_stores();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (tid == 0) {
        unsigned int old = __hip_atomic_fetch_add(counters + bkv, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == (unsigned int)(NSPL - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const float *allpart = partial + (size_t)bkv * NSPL * MAXH * OAL_V1;
    // all splits are requested at once, then summed in split order (deterministic)
    for (int idx = tid; idx < n_rep * OAL_D; idx += kThreads) {
        int h = idx / OAL_D, c = idx % OAL_D;
        float pn[NSPL], pd[NSPL];
#pragma unroll
        for (int sp = 0; sp < NSPL; ++sp) {
            const float *pp = allpart + (size_t)sp * MAXH * OAL_V1 + h * OAL_V1;
            pn[sp] = __hip_atomic_load(pp + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            pd[sp] = __hip_atomic_load(pp + OAL_D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int sp = 0; sp < NSPL; ++sp) { num += pn[sp]; den += pd[sp]; }
        y[((size_t)b * n_q_heads + h0 + h) * OAL_D + c] = num / den;
    }
    if (tid == 0) __hip_atomic_store(counters + bkv, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int MAXH>
hipError_t launch(const oal_dims &d, const void *q, const void *k, const void *v,
                  const void *params, float *state, const int *slots, int pool_size, void *ws, float *y,
                  hipStream_t stream) {
    int bkv = d.batch * d.n_kv_heads;
    unsigned int *counters = reinterpret_cast<unsigned int *>(ws);
    size_t cbytes = ((size_t)bkv * sizeof(unsigned int) + 255) / 256 * 256;
    float *partial = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + cbytes);
    if (bkv >= kBigBatchBkv) {
        hipLaunchKernelGGL((oal_decode_kernel<T, MAXH, kRowsBig>), dim3(splits_of(kRowsBig), bkv), dim3(kThreads),
                           0, stream, d.n_q_heads, d.n_kv_heads, reinterpret_cast<const T *>(q),
                           reinterpret_cast<const T *>(k), reinterpret_cast<const T *>(v),
                           reinterpret_cast<const unsigned char *>(params), state, slots, pool_size, partial,
                           counters, y);
    } else {
        hipLaunchKernelGGL((oal_decode_kernel<T, MAXH, kRowsSmall>), dim3(splits_of(kRowsSmall), bkv),
                           dim3(kThreads), 0, stream, d.n_q_heads, d.n_kv_heads, reinterpret_cast<const T *>(q),
                           reinterpret_cast<const T *>(k), reinterpret_cast<const T *>(v),
                           reinterpret_cast<const unsigned char *>(params), state, slots, pool_size, partial,
                           counters, y);
    }
    return hipGetLastError();
}

}  // namespace

size_t oal_decode_ws_bytes_impl(const oal_dims &d) {
    size_t bkv = (size_t)d.batch * d.n_kv_heads;
    size_t cbytes = (bkv * sizeof(unsigned int) + 255) / 256 * 256;
    return cbytes + bkv * kSplits * 16 * OAL_V1 * sizeof(float);
}

hipError_t oal_launch_decode(const oal_dims &d, const void *q, const void *k, const void *v,
                             const void *params, float *state, const int *slots, int pool_size, void *ws,
                             float *y, hipStream_t stream);

// ---- allocation-free variant --------------------------------------------------------------
// The workspace of up to OAL_DECODE_NOALLOC_MAX_BLOCKS (sequence, KV head) blocks as a static
// device array of the library: each GPU the library runs on holds its own copy until the
// process ends. Host code never passes the array's name to a kernel (on the host it is only a
// stand-in symbol): its device address is looked up once per device with that device current
// and kept, and that address is what the kernels receive.
namespace {
constexpr size_t kNoAllocBytes =
    ((size_t)OAL_DECODE_NOALLOC_MAX_BLOCKS * sizeof(unsigned int) + 255) / 256 * 256 +
    (size_t)OAL_DECODE_NOALLOC_MAX_BLOCKS * kSplits * 16 * OAL_V1 * sizeof(float);
constexpr int kNoAllocDevices = 64;
std::atomic<void *> g_scratch_addr[kNoAllocDevices];

// arrival counters of the combine back to zero (a kernel, not a memset: a caller may capture
// the call into a graph)
__global__ __launch_bounds__(256) void oal_zero_counters(unsigned int *__restrict__ c, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) c[i] = 0u;
}
}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

hipError_t oal_decode_scratch_addr(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kNoAllocDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

hipError_t oal_launch_decode_noalloc(const oal_dims &d, const void *q, const void *k, const void *v,
                                     const void *params, float *state, float *y, hipStream_t stream) {
    static_assert(kNoAllocBytes % 256 == 0, "scratch size");
    void *ws = nullptr;
    hipError_t e = oal_decode_scratch_addr(&ws);
    if (e != hipSuccess) return e;
    if (oal_decode_ws_bytes_impl(d) > kNoAllocBytes) return hipErrorInvalidValue;   // checked by the caller too
    const int bkv = d.batch * d.n_kv_heads;
    // the array keeps the previous call's contents: its counters start at zero here
    hipLaunchKernelGGL(oal_zero_counters, dim3((bkv + 255) / 256), dim3(256), 0, stream,
                       reinterpret_cast<unsigned int *>(ws), bkv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return oal_launch_decode(d, q, k, v, params, state, nullptr, 0, ws, y, stream);
}

hipError_t oal_launch_decode(const oal_dims &d, const void *q, const void *k, const void *v,
                             const void *params, float *state, const int *slots, int pool_size, void *ws,
                             float *y, hipStream_t stream) {
    int n_rep = d.n_q_heads / d.n_kv_heads;
    if (!slots) pool_size = d.batch;
    if (d.dtype == OAL_BF16) {
        if (n_rep <= 8) return launch<__bf16, 8>(d, q, k, v, params, state, slots, pool_size, ws, y, stream);
        return launch<__bf16, 16>(d, q, k, v, params, state, slots, pool_size, ws, y, stream);
    }
    if (n_rep <= 8) return launch<float, 8>(d, q, k, v, params, state, slots, pool_size, ws, y, stream);
    return launch<float, 16>(d, q, k, v, params, state, slots, pool_size, ws, y, stream);
}

// ---- workspace clear ------------------------------------------------------------------------
namespace {
__global__ __launch_bounds__(256) void oal_fill_zero(unsigned int *__restrict__ p, size_t n) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) p[i] = 0u;
}
}  // namespace

// zero n 4-byte words with a fill kernel (capturable: no memset node)
hipError_t oal_launch_zero_words(void *p, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    size_t grid = (n + 255) / 256;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(oal_fill_zero, dim3((unsigned)grid), dim3(256), 0, stream,
                       reinterpret_cast<unsigned int *>(p), n);
    return hipGetLastError();
}

