// oal_host.cpp -- C ABI: argument validation, coefficient tables, kernel launches.
//
// Coefficients (reproduction notes of arXiv 2610.13674, section "核心公式"): the kernel
// kappa = eps + s-bar^T M s-bar with M = L L^T expands, with s_g = sum_{r in g} q_r k_r / 8,
// into the readout's a H0 + (1/8) sum_r b_r q_r H1_r + (1/64) sum_rt C_rt q_r q_t H2_rt with
//   a = eps + M_00,  b_r = 2 M_{0,g(r)},  C_rt = M_{g(r),g(t)}   (g(r): s-bar index of dim r)
// All of it is computed here in fp64 and rounded once to fp32.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <utility>
#include <vector>

#include "oal.h"
#include "oal_internal.h"

hipError_t oal_launch_decode(const oal_dims &d, const void *q, const void *k, const void *v,
                             const void *params, float *state, const int *slots, int pool_size, void *ws,
                             float *y, hipStream_t stream);
hipError_t oal_launch_prefill(const oal_dims &d, int T_len, const int *lens, const int *cu, long long total, int C,
                              const void *q, const void *k,
                              const void *v, const void *params, float *state, void *ws, float *y,
                              hipStream_t stream, hipEvent_t *marks);
size_t oal_decode_ws_bytes_impl(const oal_dims &d);
hipError_t oal_launch_decode_noalloc(const oal_dims &d, const void *q, const void *k, const void *v,
                                     const void *params, float *state, float *y, hipStream_t stream);
hipError_t oal_launch_contribution(const oal_dims &d, int T_len, const void *q, const void *k, void *ws,
                                   float *chi, float *chi_mean, hipStream_t stream);
size_t oal_contribution_ws_bytes_impl(const oal_dims &d, int T_len);
size_t oal_prefill_ws_bytes_impl(const oal_dims &d, int T_len, int C);
hipError_t oal_launch_backward(const oal_dims &d, int T_len, int C, const void *q, const void *k, const void *v,
                               const float *dy, const void *params, const float *state_in, void *ws, float *dq,
                               float *dk, float *dv, float *dstate_in, float *dL, float *deps, hipStream_t stream);
size_t oal_backward_ws_bytes_impl(const oal_dims &d, int T_len, int C);
hipError_t oal_launch_zero_words(void *p, size_t n, hipStream_t stream);

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// prefill chunk lengths: 16, 32, 64, 128, 256 tokens
bool prefill_chunk_ok(int32_t c) { return c == 16 || c == 32 || c == 64 || c == 128 || c == 256; }

oal_status check_dims(const oal_dims *d) {
    if (!d) return OAL_E_ARG;
    if (d->dtype != OAL_F32 && d->dtype != OAL_BF16) return OAL_E_DTYPE;
    if (d->batch < 0 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->d_h < 1 || d->d_v < 1)
        return OAL_E_SHAPE;
    if (d->n_q_heads % d->n_kv_heads) return OAL_E_SHAPE;
    if (d->d_h != OAL_D || d->d_v != OAL_D) return OAL_E_UNSUPPORTED;
    if ((long long)d->batch * d->n_kv_heads > 65535) return OAL_E_UNSUPPORTED;
    return OAL_OK;
}

oal_status check_params(const oal_dims *d, const oal_head_params *hp) {
    if (!hp || !hp->n_groups || !hp->group_of_dim || !hp->L || !hp->eps) return OAL_E_ARG;
    if (hp->g_max < 1 || hp->g_max > OAL_MAX_G) return OAL_E_ARG;
    const int gm1 = hp->g_max + 1;
    for (int h = 0; h < d->n_q_heads; ++h) {
        int G = hp->n_groups[h];
        if (G < 1 || G > d->d_h || G > hp->g_max) return OAL_E_ARG;
        for (int r = 0; r < d->d_h; ++r)
            if (hp->group_of_dim[(size_t)h * d->d_h + r] >= G) return OAL_E_ARG;
        float e = hp->eps[h];
        if (!(e >= 0.0f) || !std::isfinite(e)) return OAL_E_ARG;
        const float *Lh = hp->L + (size_t)h * gm1 * gm1;
        for (int a = 0; a <= G; ++a)
            for (int b = 0; b <= a; ++b)
                if (!std::isfinite(Lh[a * gm1 + b])) return OAL_E_ARG;
    }
    return OAL_OK;
}

// Per-head coefficients. D receives the non-bulk remainder D[a][b] (config group ids,
// G x G, zero where a or b is the bulk group); Mg the group block M[a+1][b+1].
void pack_head(const oal_head_params *hp, int h, OalHeadDev *out, std::vector<double> &D,
               std::vector<double> &Mg) {
    const int gm1 = hp->g_max + 1;
    const int G = hp->n_groups[h];
    const float *Lh = hp->L + (size_t)h * gm1 * gm1;
    const uint8_t *gam = hp->group_of_dim + (size_t)h * OAL_D;
    // lower triangle of L (rows/cols 0..G), fp64
    std::vector<double> L((G + 1) * (G + 1), 0.0), M((G + 1) * (G + 1), 0.0);
    for (int a = 0; a <= G; ++a)
        for (int b = 0; b <= a; ++b) L[a * (G + 1) + b] = Lh[a * gm1 + b];
    for (int a = 0; a <= G; ++a)
        for (int b = 0; b <= G; ++b) {
            double s = 0.0;
            for (int m = 0; m <= G; ++m) s += L[a * (G + 1) + m] * L[b * (G + 1) + m];
            M[a * (G + 1) + b] = s;
        }
    auto Mq = [&](int a, int b) { return M[(a + 1) * (G + 1) + (b + 1)]; };  // config ids
    // bulk group: most dims (lowest id on ties)
    int count[OAL_MAX_G] = {0};
    for (int r = 0; r < OAL_D; ++r) count[gam[r]]++;
    int bulk = 0;
    for (int g = 1; g < G; ++g)
        if (count[g] > count[bulk]) bulk = g;
    // rank-1 factor through the bulk column of the group block of M (M is PSD, so a zero
    // M[bulk][bulk] means a zero bulk row and column)
    std::vector<double> w0(G, 0.0);
    double mbb = Mq(bulk, bulk);
    if (mbb > 0.0) {
        double sq = std::sqrt(mbb);
        for (int a = 0; a < G; ++a) w0[a] = Mq(a, bulk) / sq;
    }
    D.assign((size_t)G * G, 0.0);
    Mg.assign((size_t)G * G, 0.0);
    for (int a = 0; a < G; ++a)
        for (int b = 0; b < G; ++b) {
            Mg[a * G + b] = Mq(a, b);
            if (a != bulk && b != bulk) D[a * G + b] = Mq(a, b) - w0[a] * w0[b];
        }
    std::memset(out, 0, sizeof(OalHeadDev));
    out->G = G;
    out->bulk = bulk;
    out->eps = hp->eps[h];
    out->a = (float)((double)hp->eps[h] + M[0]);
    out->L00 = (float)L[0];
    for (int r = 0; r < OAL_D; ++r) {
        out->gamma[r] = gam[r];
        out->lin[r] = (float)(2.0 * M[0 * (G + 1) + 1 + gam[r]]);
        out->w0[r] = (float)w0[gam[r]];
    }
    for (int m = 0; m <= G; ++m)
        for (int r = 0; r < OAL_D; ++r) {
            int gr = 1 + gam[r];
            out->Lz[m * OAL_D + r] = gr >= m ? (float)(L[gr * (G + 1) + m] / 8.0) : 0.0f;
        }
    for (int a = 0; a <= G; ++a)
        for (int b = 0; b <= a; ++b) out->Lt[a * 65 + b] = (float)L[a * (G + 1) + b];
    // decode coefficients per state row
    out->wdec[0] = out->a;
    for (int r = 0; r < OAL_D; ++r) out->wdec[1 + r] = (float)(2.0 * M[1 + gam[r]] / 8.0);
    for (int r = 0; r < OAL_D; ++r)
        for (int t = r; t < OAL_D; ++t)
            out->wdec[oal_quad_row(r, t)] = (float)((r < t ? 2.0 : 1.0) * Mq(gam[r], gam[t]) / 64.0);
}

// Tail pairs of the query heads [h0, h1) of one KV head: every (r <= t) whose remainder
// D[g(r)][g(t)] is nonzero for at least one of the heads, in (r, t) order.
std::vector<std::pair<int, int>> tail_pairs(const oal_head_params *hp, int h0, int h1,
                                            const std::vector<std::vector<double>> &D) {
    std::vector<std::pair<int, int>> pairs;
    for (int r = 0; r < OAL_D; ++r)
        for (int t = r; t < OAL_D; ++t) {
            bool need = false;
            for (int h = h0; h < h1 && !need; ++h) {
                const uint8_t *gam = hp->group_of_dim + (size_t)h * OAL_D;
                int G = hp->n_groups[h];
                need = D[h][gam[r] * G + gam[t]] != 0.0;
            }
            if (need) pairs.emplace_back(r, t);
        }
    return pairs;
}

}  // namespace

extern "C" {

const char *oal_status_string(oal_status s) {
    switch (s) {
    case OAL_OK: return "ok";
    case OAL_E_ARG: return "invalid argument";
    case OAL_E_SHAPE: return "inconsistent shape";
    case OAL_E_DTYPE: return "unsupported dtype";
    case OAL_E_ALIGN: return "device pointer not 16-byte aligned";
    case OAL_E_UNSUPPORTED: return "unsupported configuration";
    case OAL_E_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t oal_params_bytes(const oal_dims *d) {
    if (check_dims(d) != OAL_OK) return 0;
    return sizeof(OalParamsHeader) + (size_t)d->n_q_heads * OAL_HEAD_BYTES +
           (size_t)d->n_kv_heads * OAL_KV_BYTES;
}

size_t oal_state_bytes(const oal_dims *d) {
    if (check_dims(d) != OAL_OK) return 0;
    return (size_t)d->batch * d->n_kv_heads * OAL_STATE_STRIDE * sizeof(float);
}

size_t oal_prefill_workspace_bytes(const oal_dims *d, int32_t T, int32_t chunk) {
    if (check_dims(d) != OAL_OK || T < 0) return 0;
    if (!prefill_chunk_ok(chunk)) return 0;
    if (T == 0 || d->batch == 0) return 0;
    return oal_prefill_ws_bytes_impl(*d, T, chunk);
}

size_t oal_decode_workspace_bytes(const oal_dims *d) {
    if (check_dims(d) != OAL_OK) return 0;
    if (d->n_q_heads / d->n_kv_heads > 16) return 0;
    return oal_decode_ws_bytes_impl(*d);
}

oal_status oal_params_pack(const oal_dims *d, const oal_head_params *hp, void *blob, size_t bytes) {
    oal_status st = check_dims(d);
    if (st != OAL_OK) return st;
    if (!blob) return OAL_E_ARG;
    if ((st = check_params(d, hp)) != OAL_OK) return st;
    if (bytes < oal_params_bytes(d)) return OAL_E_ARG;
    unsigned char *p = static_cast<unsigned char *>(blob);
    std::memset(p, 0, oal_params_bytes(d));
    OalParamsHeader *hdr = reinterpret_cast<OalParamsHeader *>(p);
    hdr->magic = OAL_PARAMS_MAGIC;
    hdr->n_q_heads = d->n_q_heads;
    hdr->d_h = d->d_h;
    hdr->d_v = d->d_v;
    hdr->head_bytes = OAL_HEAD_BYTES;
    hdr->n_kv_heads = d->n_kv_heads;
    const int nq = d->n_q_heads, nkv = d->n_kv_heads, n_rep = nq / nkv;
    auto head = [&](int h) {
        return reinterpret_cast<OalHeadDev *>(p + sizeof(OalParamsHeader) + (size_t)h * OAL_HEAD_BYTES);
    };
    auto kvrec = [&](int kv) {
        return reinterpret_cast<OalKvDev *>(p + sizeof(OalParamsHeader) + (size_t)nq * OAL_HEAD_BYTES +
                                            (size_t)kv * OAL_KV_BYTES);
    };
    std::vector<std::vector<double>> D(nq), Mg(nq);
    for (int h = 0; h < nq; ++h) pack_head(hp, h, head(h), D[h], Mg[h]);
    std::vector<std::vector<std::pair<int, int>>> pairs(nkv);
    for (int kv = 0; kv < nkv; ++kv) {
        pairs[kv] = tail_pairs(hp, kv * n_rep, (kv + 1) * n_rep, D);
        if ((int)pairs[kv].size() > OAL_TAIL_PAIRS - OAL_TAIL_FIXED) hdr->general = 1;
    }
    for (int kv = 0; kv < nkv; ++kv) {
        OalKvDev *kr = kvrec(kv);
        // entries 0..63: linear feature r = (r, 64); 64: the constant (64, 64); then the
        // non-bulk pairs (none in a general blob)
        const int np = hdr->general ? 0 : (int)pairs[kv].size();
        kr->npairs = OAL_TAIL_FIXED + np;
        kr->nsteps = (kr->npairs + 31) / 32;
        for (int j = 0; j <= OAL_D; ++j) {
            kr->ra[j] = (uint8_t)j;
            kr->rb[j] = (uint8_t)OAL_D;
        }
        for (int m = 0; m < np; ++m) {
            kr->ra[OAL_TAIL_FIXED + m] = (uint8_t)pairs[kv][m].first;
            kr->rb[OAL_TAIL_FIXED + m] = (uint8_t)pairs[kv][m].second;
        }
        for (int h = kv * n_rep; h < (kv + 1) * n_rep; ++h) {
            OalHeadDev *hd = head(h);
            const uint8_t *gam = hp->group_of_dim + (size_t)h * OAL_D;
            int G = hp->n_groups[h];
            for (int r = 0; r < OAL_D; ++r) hd->tail[r] = hd->lin[r];
            hd->tail[OAL_D] = hd->a;
            for (int m = 0; m < np; ++m)
                hd->tail[OAL_TAIL_FIXED + m] = (float)D[h][gam[pairs[kv][m].first] * G + gam[pairs[kv][m].second]];
        }
    }
    if (hdr->general) {
        // every quadratic slot carries its full coefficient; the rank-1 factor becomes 1
        for (int h = 0; h < nq; ++h) {
            OalHeadDev *hd = head(h);
            const uint8_t *gam = hp->group_of_dim + (size_t)h * OAL_D;
            int G = hp->n_groups[h];
            for (int r = 0; r < OAL_D; ++r) hd->w0[r] = 1.0f;
            for (int tb = 0; tb < 8; ++tb)
                for (int rq = 0; rq <= 2 * tb + 1; ++rq)
                    for (int g = 0; g < 4; ++g)
                        for (int e = 0; e < 8; ++e) {
                            int ra, rb;
                            if (oal_slot_kind(tb, rq, g, e, &ra, &rb) != OAL_SLOT_QUAD) continue;
                            hd->wslot[oal_kstep(tb, rq) * 32 + 8 * g + e] = (float)Mg[h][gam[ra] * G + gam[rb]];
                        }
        }
    }
    return OAL_OK;
}

oal_status oal_state_init(const oal_dims *d, const oal_head_params *hp, void *params_dev,
                          float *state_dev, hipStream_t stream) {
    oal_status st = check_dims(d);
    if (st != OAL_OK) return st;
    if (!params_dev) return OAL_E_ARG;
    if (!aligned16(params_dev) || (state_dev && !aligned16(state_dev))) return OAL_E_ALIGN;
    if ((st = check_params(d, hp)) != OAL_OK) return st;
    size_t bytes = oal_params_bytes(d);
    std::vector<unsigned char> blob(bytes);
    if ((st = oal_params_pack(d, hp, blob.data(), bytes)) != OAL_OK) return st;
    if (hipMemcpyAsync(params_dev, blob.data(), bytes, hipMemcpyHostToDevice, stream) != hipSuccess)
        return OAL_E_HIP;
    if (state_dev && oal_state_bytes(d) > 0 &&
        hipMemsetAsync(state_dev, 0, oal_state_bytes(d), stream) != hipSuccess)
        return OAL_E_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return OAL_E_HIP;
    return OAL_OK;
}

static oal_status prefill_impl(const oal_dims *d, int32_t T, const int32_t *lens, const int32_t *cu,
                               int64_t total, int32_t chunk, const void *q, const void *k, const void *v,
                               const void *params_dev, float *state_dev, void *workspace, size_t ws_bytes,
                               float *y, hipStream_t stream, hipEvent_t *marks) {
    oal_status st = check_dims(d);
    if (st != OAL_OK) return st;
    if (T < 0) return OAL_E_SHAPE;
    if (!prefill_chunk_ok(chunk)) return OAL_E_UNSUPPORTED;
    if (T == 0 || d->batch == 0) return OAL_OK;
    // y == NULL: advance the state only (q is then not read and may be NULL)
    if ((y && !q) || !k || !v || !params_dev || !state_dev || !workspace) return OAL_E_ARG;
    if ((q && !aligned16(q)) || !aligned16(k) || !aligned16(v) || !aligned16(params_dev) ||
        !aligned16(state_dev) || !aligned16(workspace) || (y && !aligned16(y)) ||
        (reinterpret_cast<uintptr_t>(lens) & 3u) || (reinterpret_cast<uintptr_t>(cu) & 3u))
        return OAL_E_ALIGN;
    if ((T + chunk - 1) / chunk > 65535) return OAL_E_UNSUPPORTED;
    if (ws_bytes < oal_prefill_ws_bytes_impl(*d, T, chunk)) return OAL_E_ARG;
    hipError_t e = oal_launch_prefill(*d, T, lens, cu, (long long)total, chunk, q, k, v, params_dev, state_dev,
                                      workspace, y, stream, marks);
    if (e != hipSuccess) {
        (void)hipGetLastError();   // do not leave a sticky error for the caller's next HIP call
        return OAL_E_HIP;
    }
    return OAL_OK;
}

oal_status oal_prefill(const oal_dims *d, int32_t T, int32_t chunk, const void *q, const void *k,
                       const void *v, const void *params_dev, float *state_dev, void *workspace,
                       size_t workspace_bytes, float *y, hipStream_t stream) {
    return prefill_impl(d, T, nullptr, nullptr, 0, chunk, q, k, v, params_dev, state_dev, workspace,
                        workspace_bytes, y, stream, nullptr);
}

oal_status oal_prefill_timed(const oal_dims *d, int32_t T, int32_t chunk, const void *q,
                             const void *k, const void *v, const void *params_dev,
                             float *state_dev, void *workspace, size_t workspace_bytes, float *y,
                             hipStream_t stream, hipEvent_t marks[3]) {
    if (!marks || !marks[0] || !marks[1] || !marks[2]) return OAL_E_ARG;
    return prefill_impl(d, T, nullptr, nullptr, 0, chunk, q, k, v, params_dev, state_dev, workspace,
                        workspace_bytes, y, stream, marks);
}

oal_status oal_prefill_varlen(const oal_dims *d, int32_t T, const int32_t *lengths, int32_t chunk,
                              const void *q, const void *k, const void *v, const void *params_dev,
                              float *state_dev, void *workspace, size_t workspace_bytes, float *y,
                              hipStream_t stream) {
    if (!lengths && check_dims(d) == OAL_OK && T > 0 && d->batch > 0) return OAL_E_ARG;
    return prefill_impl(d, T, lengths, nullptr, 0, chunk, q, k, v, params_dev, state_dev, workspace,
                        workspace_bytes, y, stream, nullptr);
}

oal_status oal_prefill_packed(const oal_dims *d, int32_t T, const int32_t *cu_seqlens, int64_t total_tokens,
                              int32_t chunk, const void *q, const void *k, const void *v,
                              const void *params_dev, float *state_dev, void *workspace,
                              size_t workspace_bytes, float *y, hipStream_t stream) {
    if (total_tokens < 0) return OAL_E_SHAPE;
    if (check_dims(d) == OAL_OK && T > 0 && d->batch > 0) {
        if (!cu_seqlens) return OAL_E_ARG;
        if (total_tokens == 0) return OAL_OK;     // every sequence is empty
    }
    return prefill_impl(d, T, nullptr, cu_seqlens, total_tokens, chunk, q, k, v, params_dev, state_dev,
                        workspace, workspace_bytes, y, stream, nullptr);
}

oal_status oal_decode_step(const oal_dims *d, const void *q, const void *k, const void *v,
                           const void *params_dev, float *state_dev, void *workspace, size_t workspace_bytes,
                           float *y, hipStream_t stream) {
    oal_status st = check_dims(d);
    if (st != OAL_OK) return st;
    if (d->n_q_heads / d->n_kv_heads > 16) return OAL_E_UNSUPPORTED;
    if (d->batch == 0) return OAL_OK;
    if (!q || !k || !v || !params_dev || !state_dev || !workspace || !y) return OAL_E_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(params_dev) ||
        !aligned16(state_dev) || !aligned16(workspace) || !aligned16(y))
        return OAL_E_ALIGN;
    if (workspace_bytes < oal_decode_ws_bytes_impl(*d)) return OAL_E_ARG;
    hipError_t e = oal_launch_decode(*d, q, k, v, params_dev, state_dev, nullptr, 0, workspace, y, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return OAL_E_HIP;
    }
    return OAL_OK;
}

oal_status oal_decode_step_indexed(const oal_dims *d, const int32_t *slots, int32_t pool_size,
                                   const void *q, const void *k, const void *v, const void *params_dev,
                                   float *state_pool, void *workspace, size_t workspace_bytes, float *y,
                                   hipStream_t stream) {
    oal_status st = check_dims(d);
    if (st != OAL_OK) return st;
    if (d->n_q_heads / d->n_kv_heads > 16) return OAL_E_UNSUPPORTED;
    if (pool_size < 1) return OAL_E_SHAPE;
    if (d->batch == 0) return OAL_OK;
    if (!slots || !q || !k || !v || !params_dev || !state_pool || !workspace || !y) return OAL_E_ARG;
    if ((reinterpret_cast<uintptr_t>(slots) & 3u) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
        !aligned16(params_dev) || !aligned16(state_pool) || !aligned16(workspace) || !aligned16(y))
        return OAL_E_ALIGN;
    if (workspace_bytes < oal_decode_ws_bytes_impl(*d)) return OAL_E_ARG;
    hipError_t e = oal_launch_decode(*d, q, k, v, params_dev, state_pool, slots, pool_size, workspace, y, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return OAL_E_HIP;
    }
    return OAL_OK;
}

oal_status oal_decode_step_noalloc(const oal_dims *d, const void *q, const void *k, const void *v,
                                   const void *params_dev, float *state_dev, float *y, hipStream_t stream) {
    oal_status st = check_dims(d);
    if (st != OAL_OK) return st;
    if (d->n_q_heads / d->n_kv_heads > 16) return OAL_E_UNSUPPORTED;
    if ((long long)d->batch * d->n_kv_heads > OAL_DECODE_NOALLOC_MAX_BLOCKS) return OAL_E_UNSUPPORTED;
    if (d->batch == 0) return OAL_OK;
    if (!q || !k || !v || !params_dev || !state_dev || !y) return OAL_E_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(params_dev) || !aligned16(state_dev) ||
        !aligned16(y))
        return OAL_E_ALIGN;
    hipError_t e = oal_launch_decode_noalloc(*d, q, k, v, params_dev, state_dev, y, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return OAL_E_HIP;
    }
    return OAL_OK;
}

oal_status oal_workspace_clear(void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (workspace_bytes == 0) return OAL_OK;
    if (!workspace || workspace_bytes % 4) return OAL_E_ARG;
    if (reinterpret_cast<uintptr_t>(workspace) & 3u) return OAL_E_ALIGN;
    if (oal_launch_zero_words(workspace, workspace_bytes / 4, stream) != hipSuccess) {
        (void)hipGetLastError();
        return OAL_E_HIP;
    }
    return OAL_OK;
}

size_t oal_contribution_workspace_bytes(const oal_dims *d, int32_t T) {
    if (check_dims(d) != OAL_OK || T < 1 || T > OAL_CHI_MAX_T || d->batch < 1) return 0;
    return oal_contribution_ws_bytes_impl(*d, T);
}

oal_status oal_contribution(const oal_dims *d, int32_t T, const void *q, const void *k,
                            void *workspace, size_t workspace_bytes, float *chi, float *chi_mean,
                            hipStream_t stream) {
    oal_status st = check_dims(d);
    if (st != OAL_OK) return st;
    if (T < 1 || d->batch < 1) return OAL_E_SHAPE;
    if (T > OAL_CHI_MAX_T) return OAL_E_UNSUPPORTED;
    if (!q || !k || !workspace || !chi) return OAL_E_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(workspace) || !aligned16(chi) ||
        (chi_mean && !aligned16(chi_mean)))
        return OAL_E_ALIGN;
    if (workspace_bytes < oal_contribution_ws_bytes_impl(*d, T)) return OAL_E_ARG;
    hipError_t e = oal_launch_contribution(*d, T, q, k, workspace, chi, chi_mean, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return OAL_E_HIP;
    }
    return OAL_OK;
}

// grid limits of the backward's launches: chunks (dimension y of the increments and the
// coefficient kernels), query heads and 8 workgroups per KV head (dimension y elsewhere)
static bool backward_shape_ok(const oal_dims *d, int32_t T, int32_t chunk) {
    return (T + chunk - 1) / chunk <= 65535 && d->n_q_heads + 3 * d->n_kv_heads <= 65535 &&
           d->n_kv_heads * 8 <= 65535;
}

size_t oal_prefill_backward_workspace_bytes(const oal_dims *d, int32_t T, int32_t chunk) {
    if (check_dims(d) != OAL_OK || T < 0 || (chunk != 64 && chunk != 128 && chunk != 256)) return 0;
    if (!backward_shape_ok(d, T, chunk)) return 0;
    return oal_backward_ws_bytes_impl(*d, T, chunk);
}

oal_status oal_prefill_backward(const oal_dims *d, int32_t T, int32_t chunk, const void *q, const void *k,
                                const void *v, const float *dy, const void *params_dev, const float *state_in,
                                void *workspace, size_t workspace_bytes, float *dq, float *dk, float *dv,
                                float *dstate_in, float *dL, float *deps, hipStream_t stream) {
    oal_status st = check_dims(d);
    if (st != OAL_OK) return st;
    if (T < 0) return OAL_E_SHAPE;
    if (chunk != 64 && chunk != 128 && chunk != 256) return OAL_E_UNSUPPORTED;
    if (T == 0 || d->batch == 0) return OAL_OK;
    if (!backward_shape_ok(d, T, chunk)) return OAL_E_UNSUPPORTED;
    if (!q || !k || !v || !dy || !params_dev || !workspace || !dq || !dk || !dv || (!dL != !deps))
        return OAL_E_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dy) || !aligned16(params_dev) ||
        !aligned16(workspace) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
        (state_in && !aligned16(state_in)) || (dstate_in && !aligned16(dstate_in)) ||
        (reinterpret_cast<uintptr_t>(dL) & 3u) || (reinterpret_cast<uintptr_t>(deps) & 3u))
        return OAL_E_ALIGN;
    if (workspace_bytes < oal_backward_ws_bytes_impl(*d, T, chunk)) return OAL_E_ARG;
    hipError_t e = oal_launch_backward(*d, T, chunk, q, k, v, dy, params_dev, state_in, workspace, dq, dk, dv,
                                       dstate_in, dL, deps, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return OAL_E_HIP;
    }
    return OAL_OK;
}

oal_status oal_timing_event_create(hipEvent_t *event) {
    if (!event) return OAL_E_ARG;
    if (hipEventCreateWithFlags(event, hipEventDisableSystemFence) != hipSuccess) {
        (void)hipGetLastError();
        *event = nullptr;
        return OAL_E_HIP;
    }
    return OAL_OK;
}

oal_status oal_timing_event_destroy(hipEvent_t event) {
    if (!event) return OAL_OK;
    if (hipEventDestroy(event) != hipSuccess) {
        (void)hipGetLastError();
        return OAL_E_HIP;
    }
    return OAL_OK;
}

oal_status oal_timing_event_record(hipEvent_t event, hipStream_t stream) {
    if (!event) return OAL_E_ARG;
    if (hipEventRecord(event, stream) != hipSuccess) {
        (void)hipGetLastError();
        return OAL_E_HIP;
    }
    return OAL_OK;
}

oal_status oal_timing_elapsed_ms(hipEvent_t start, hipEvent_t end, float *ms) {
    if (!start || !end || !ms) return OAL_E_ARG;
    if (hipEventSynchronize(end) != hipSuccess || hipEventElapsedTime(ms, start, end) != hipSuccess) {
        (void)hipGetLastError();
        return OAL_E_HIP;
    }
    return OAL_OK;
}

}  // extern "C"
