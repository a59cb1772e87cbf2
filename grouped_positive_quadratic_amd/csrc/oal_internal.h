// oal_internal.h -- layouts shared by the host library and the gfx950 kernels.
//
// Feature space (reproduction notes of arXiv 2610.13674, section "核心公式", H-state and
// readout displays): the readout is u~ = phi(q) . H with features
//   constant (H0), linear r (H1_r, coefficient b_r / sqrt(d)) and quadratic (r,t)
//   (H2_rt, coefficient C_rt / d, counted once for r <= t with r < t doubled).
// With d = 64 that is 1 + 64 + 2080 = 2145 features per KV head and 65 value columns
// (64 components of v plus the "1" of [v;1]).
//
// Prefill kernels use a padded "slot" order of the features so that the MFMA operand of a
// query can be generated from registers with static indices. The 2304 slots of the main
// part form 72 K-steps of 32; K-step s <-> (tb, rq), s = tb*(tb+1) + rq, tb in 0..7,
// rq in 0..2tb+1. Inside a K-step, MFMA lane group g (0..3) holds 8 slots e = 0..7 with
// nominal (r, t) = (4 rq + g, 8 tb + e): r <= t is the quadratic feature (r, t), anything
// else an empty slot (zero state row). The linear features, the constant and the non-bulk
// pairs of a KV head follow in up to 8 "tail" K-steps listed per KV head (OalKvDev):
// entry j < 64 is linear feature r = j (pair (j, 64)), entry 64 the constant (pair
// (64, 64)), entries from 65 on the non-bulk quadratic pairs; dim 64 stands for a 1.
// Snapshot states in this order are pre-scaled so that the query side needs no constant:
//   quadratic: H2_rt * (r < t ? 2 : 1) / 64, linear: H1_r / 8, constant: H0.
#pragma once

#include <stdint.h>

#include "oal.h"

#define OAL_D 64
#define OAL_V1 65
#define OAL_NFEAT 2145
#define OAL_NQUAD 2080
#define OAL_KSTEPS 72
#define OAL_TAIL_STEPS 8          // extra K-steps: linear, constant, non-bulk pairs (per KV head)
#define OAL_TAIL_PAIRS (32 * OAL_TAIL_STEPS)
#define OAL_TAIL_FIXED 65         // tail entries 0..64: linear features and the constant
#define OAL_SNAP_KSTEPS (OAL_KSTEPS + OAL_TAIL_STEPS)
#define OAL_PARAMS_MAGIC 0x314C414Fu  // "OAL1"
#define OAL_MAX_G 64
static_assert(OAL_STATE_STRIDE % 64 == 0 && OAL_STATE_STRIDE >= OAL_NFEAT * OAL_V1, "state block stride");

#if defined(__HIPCC__)
#define OAL_HD __host__ __device__
#else
#define OAL_HD
#endif

enum { OAL_SLOT_EMPTY = 0, OAL_SLOT_QUAD = 1 };

// Kind of main slot (tb, rq, g, e); ra/rb receive the dims of a quadratic slot.
OAL_HD inline int oal_slot_kind(int tb, int rq, int g, int e, int *ra, int *rb) {
    int r = 4 * rq + g, t = 8 * tb + e;
    *ra = OAL_D;
    *rb = OAL_D;
    if (r <= t) { *ra = r; *rb = t; return OAL_SLOT_QUAD; }
    return OAL_SLOT_EMPTY;
}

// Row of the state layout for quadratic feature (r, t), r <= t.
OAL_HD inline int oal_quad_row(int r, int t) { return 1 + OAL_D + r * OAL_D - (r * (r - 1)) / 2 + (t - r); }

// K-step index of (tb, rq).
OAL_HD inline int oal_kstep(int tb, int rq) { return tb * (tb + 1) + rq; }

// Per-query-head coefficient record in the device parameter blob.
//   Quadratic coefficients M[g(r)+1][g(t)+1] (M = L L^T) are split into a rank-1 part
//   w0[r] * w0[t] that covers every pair touching the bulk group, and a remainder D for
//   pairs of two non-bulk dims. The tail list of the KV head (OalKvDev) carries the linear
//   features, the constant and the non-bulk pairs of all its query heads; head h multiplies
//   tail entry j by tail[j] q_a q_b (q_64 = 1): the linear coefficient, a, or D. If some KV
//   head has more non-bulk pairs than the list holds, the blob is "general": w0 = 1, the
//   list keeps only the linear features and the constant, and the prefill reads the full
//   coefficient of every main slot from wslot.
struct OalHeadDev {
    int32_t G;          // number of groups
    int32_t bulk;       // config id of the group carried by the rank-1 term
    float eps;
    float a;            // eps + M[0][0]: constant-feature coefficient
    float L00;          // L[0][0]: constant part of z_0 = (L^T s-bar)_0
    float pad0[3];
    uint8_t gamma[64];  // config group id of each dim
    float lin[64];      // 2 M[0][g(r)+1]: linear coefficient (times q_r H1_r / 8)
    float w0[64];       // rank-1 factor of dim r's group (1 in a general blob)
    float tail[OAL_TAIL_PAIRS];        // coefficient of the KV head's tail entry j
    float Lz[65 * 64];  // Lz[m][r] = L[g(r)+1][m] / 8 (zero where g(r)+1 < m), m = 0..64
    float wslot[OAL_KSTEPS * 32];      // general blob: M[g(r)+1][g(t)+1] per quadratic slot
    float wdec[2176];   // per state row f < 2145: coefficient of mono_f(q) . H_f (unscaled state)
    float Lt[65 * 65];  // L[a][b] for b <= a <= G (row stride 65), zero elsewhere
};

// Per-KV-head record: the tail list. Entries 0..64: linear features and the constant;
// from 65 on, the union over the KV head's query heads of the pairs (r <= t) whose dims
// are both outside the head's bulk group with a nonzero remainder D.
struct OalKvDev {
    int32_t npairs;     // entries listed (>= 65)
    int32_t nsteps;     // tail K-steps used: ceil(npairs / 32)
    int32_t pad[62];
    uint8_t ra[OAL_TAIL_PAIRS];
    uint8_t rb[OAL_TAIL_PAIRS];
};

struct OalParamsHeader {
    uint32_t magic;
    int32_t n_q_heads;
    int32_t d_h;
    int32_t d_v;
    int32_t head_bytes;
    int32_t n_kv_heads;
    int32_t general;    // 1: some KV head has more non-bulk pairs than its tail list holds
    int32_t pad[57];    // 256 bytes
};

#define OAL_HEAD_BYTES ((int)((sizeof(OalHeadDev) + 255) / 256 * 256))
#define OAL_KV_BYTES ((int)((sizeof(OalKvDev) + 255) / 256 * 256))
