/*
 * oal.h -- C ABI of the OAL causal-attention library for AMD Instinct MI355X (gfx950).
 *
 * What it computes (reproduction notes of arXiv 2610.13674 on daiwk.github.io, section
 * "核心公式"; arXiv abstract page of 2610.13674v1):
 *
 *   per query head h with KV head kv = h / (n_q_heads / n_kv_heads) (contiguous GQA map):
 *     s_g    = sum_{r in group g} q_r k_r / sqrt(d_h),   s-bar = [1, s_1, ..., s_G]
 *     kappa  = eps_h + s-bar^T L_h L_h^T s-bar            (> 0 by the PSD parameterisation)
 *     y_i    = sum_{j<=i} kappa(q_i,k_j) v_j / sum_{j<=i} kappa(q_i,k_j)
 *   evaluated in linear time through the prefix states of the KV head
 *     H0 = sum_{j<=i} [v_j;1],  H1_r = sum k_{j,r} [v_j;1],  H2_rt = sum k_{j,r} k_{j,t} [v_j;1]
 *   and the readout u~_i = a H0 + (1/sqrt d_h) sum_r b_r q_r H1_r + (1/d_h) sum_rt C_rt q_r q_t H2_rt,
 *   y_i = u~_i[0:d_v] / u~_i[d_v], with a = eps + M_00, b_r = 2 M_{0,g(r)}, C_rt = M_{g(r),g(t)},
 *   M = L L^T (the expansion of s-bar^T M s-bar; g(r) = s-bar index of dim r's group).
 *
 * Version 1 supports d_h = d_v = 64, q/k/v in fp32 or bf16 (fp32 accumulation), y in fp32.
 *
 * Layouts (all row-major, contiguous, device memory unless stated otherwise):
 *   q      [batch, n_q_heads,  T, 64]  dtype of oal_dims.dtype
 *   k, v   [batch, n_kv_heads, T, 64]
 *   y      [batch, n_q_heads,  T, 64]  fp32
 *   state  [batch, n_kv_heads] blocks of OAL_STATE_STRIDE (139456) fp32, one per (sequence,
 *          KV head), 256-byte aligned. The prefix state is a [2145, 65] matrix H (feature
 *          row f, column c) stored in two parts: columns 0..63 (the components of v) as a
 *          [2145, 64] row-major matrix in the first 2145 * 64 floats (256-byte rows), then
 *          column 64 (the "1" of [v;1], the denominators' state) as 2145 contiguous floats;
 *          H[f][c] is at f * 64 + c for c < 64 and at 2145 * 64 + f for c = 64
 *          (OAL_STATE_INDEX). The last 31 floats are padding (zero after oal_state_init; the
 *          kernels keep them finite). Row 0 = H0; rows 1..64 = H1_r (r = 0..63); rows 65.. =
 *          H2_rt for r <= t in row-major order of the upper triangle (the symmetric H2
 *          stored once, r < t not doubled).
 *   For a decode step T = 1 and the T axis is dropped: q [batch, n_q_heads, 64] etc.
 *
 * Ownership: the caller allocates and owns every device buffer (params, state, workspace,
 * q, k, v, y). The library allocates no memory in oal_prefill / oal_decode_step and keeps
 * no global mutable state. Host arrays passed in oal_head_params are read during the call.
 *
 * Streams: every call enqueues work on `stream` and returns; the caller synchronises.
 * oal_state_init additionally waits for its host-to-device copy before returning.
 *
 * Workspaces: every call that takes a `workspace` also takes `workspace_bytes`, the size of
 * the buffer the caller passes. It must be at least the matching *_workspace_bytes() value
 * for the call's dims (and T, chunk); a smaller buffer gives OAL_E_ARG and nothing is
 * enqueued, so an undersized workspace is an error code, never a write past its end.
 *
 * Errors: arguments are validated on the host before anything is enqueued; on any error
 * nothing is enqueued and a status code is returned. HIP launch failures map to OAL_E_HIP.
 * NaN/Inf in q, k, v propagate to y. eps = 0 together with a singular L can make a
 * denominator zero; y is then NaN or Inf for that row (kappa > 0 needs eps > 0 or L L^T PD).
 */
#ifndef OAL_H
#define OAL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    OAL_OK = 0,
    OAL_E_ARG = 1,          /* null pointer or invalid scalar argument */
    OAL_E_SHAPE = 2,        /* inconsistent sizes (n_q_heads % n_kv_heads != 0, T < 0, ...) */
    OAL_E_DTYPE = 3,        /* dtype is not OAL_F32 / OAL_BF16 */
    OAL_E_ALIGN = 4,        /* a device pointer is not 16-byte aligned */
    OAL_E_UNSUPPORTED = 5,  /* valid but not implemented (d_h or d_v != 64, chunk size) */
    OAL_E_HIP = 6           /* a HIP runtime call or kernel launch failed */
} oal_status;

typedef enum { OAL_F32 = 0, OAL_BF16 = 1 } oal_dtype;

typedef struct {
    int32_t batch;       /* sequences (>= 0) */
    int32_t n_q_heads;   /* query heads (>= 1) */
    int32_t n_kv_heads;  /* KV heads (>= 1, divides n_q_heads) */
    int32_t d_h;         /* q/k head dim (64) */
    int32_t d_v;         /* v head dim (64) */
    int32_t dtype;       /* oal_dtype of q, k, v */
} oal_dims;

/* Per-query-head kernel parameters (host memory, read during the call).
 * The group map and L are those of the kernel kappa = eps + s-bar^T L L^T s-bar
 * (reproduction notes, section "核心公式", kernel display; Figure 2(a) for the bulk + tail
 * grouping). There is no cap on the number of groups other than G <= d_h. */
typedef struct {
    int32_t g_max;               /* max G over heads, 1..64; L's per-head stride is (g_max+1)^2 */
    const int32_t *n_groups;     /* [n_q_heads]: G_h in 1..d_h and <= g_max */
    const uint8_t *group_of_dim; /* [n_q_heads][d_h]: config group id of each dim, < G_h;
                                    config group g is entry g+1 of s-bar. Empty groups allowed. */
    const float *L;              /* [n_q_heads][g_max+1][g_max+1] row-major; the lower triangle
                                    (rows/cols 0..G_h) is read, the rest ignored. Row/column 0
                                    belong to the constant entry of s-bar. Zero or negative
                                    diagonal entries are accepted. Must be finite. */
    const float *eps;            /* [n_q_heads]: eps_h >= 0, finite */
} oal_head_params;

/* Bytes of the device parameter blob (coefficient tables for every query head). */
size_t oal_params_bytes(const oal_dims *dims);

/* Floats per (sequence, KV head) block of the state buffer: 2145 * 65 rounded up to 64. */
#define OAL_STATE_STRIDE 139456
/* Offset in a state block of H[f][c] (feature row f < 2145, column c <= 64). */
#define OAL_STATE_INDEX(f, c) ((c) < 64 ? (size_t)(f) * 64 + (size_t)(c) : (size_t)2145 * 64 + (size_t)(f))

/* Bytes of the state buffer: batch * n_kv_heads * OAL_STATE_STRIDE * 4. */
size_t oal_state_bytes(const oal_dims *dims);

/* Bytes of the scratch buffer oal_prefill needs for T tokens at this chunk size
 * (per-chunk state snapshots and per-segment partial states). 0 on invalid input. */
size_t oal_prefill_workspace_bytes(const oal_dims *dims, int32_t T, int32_t chunk);

/* Bytes of the scratch buffer oal_decode_step needs (per-split partial readouts and one
 * arrival counter per (sequence, KV head, head group)). */
size_t oal_decode_workspace_bytes(const oal_dims *dims);

/* Build the parameter blob in HOST memory (what oal_state_init uploads). `blob` must hold
 * oal_params_bytes(dims) bytes. Runs on the CPU only; no device is needed. */
oal_status oal_params_pack(const oal_dims *dims, const oal_head_params *hp, void *blob,
                           size_t blob_bytes);

/* Validate the parameters, upload the parameter blob to `params_dev`
 * (oal_params_bytes(dims) bytes, device) and zero `state_dev` (oal_state_bytes(dims) bytes,
 * device; may be NULL to leave it untouched). A zero state is an empty prefix.
 * Passage: reproduction notes, section "核心公式" -- the kernel's parameters (the group map
 * of the dims, the lower-triangular factor L with M = L L^T, eps) and the prefix states
 * H0, H1, H2, which are all zero before the first token. */
oal_status oal_state_init(const oal_dims *dims, const oal_head_params *hp, void *params_dev,
                          float *state_dev, hipStream_t stream);

/* Chunked causal prefill of T new tokens per sequence, continuing from `state_dev`.
 * Passage: reproduction notes, section "核心公式" -- for every new token, the readout display
 * u~ = phi_h(q) . H over the prefix states and y = u~[0:64] / u~[64], with H advanced by the
 * H-state recurrence over the tokens. The chunking is this library's evaluation order: it
 * gives the same causal kernel sums up to rounding.
 *   chunk      -- chunk length C in {16, 32, 64, 128, 256}: the tokens of a chunk see the state
 *                 before the chunk plus an exact intra-chunk kernel sum.
 *   q, k, v    -- [batch, heads, T, 64] of dims->dtype (device).
 *   state_dev  -- in: prefix states of the tokens before these T; out: states after them.
 *   workspace  -- oal_prefill_workspace_bytes(dims, T, chunk) bytes of device scratch. Its
 *                 contents on entry do not matter.
 *   y          -- [batch, n_q_heads, T, 64] fp32 output (device), or NULL to only advance
 *                 the state (ingesting a context whose outputs are not needed; q is then
 *                 not read and may be NULL).
 * Position i of this call attends to every earlier token of the sequence (those folded
 * into the input state and tokens 0..i of this call). T = 0 is a no-op. */
oal_status oal_prefill(const oal_dims *dims, int32_t T, int32_t chunk, const void *q,
                       const void *k, const void *v, const void *params_dev, float *state_dev,
                       void *workspace, size_t workspace_bytes, float *y, hipStream_t stream);

/* oal_prefill for measurement: identical work, and additionally records the caller-owned
 * events marks[0] on `stream` before the first kernel, marks[1] after the chunk-state scan
 * kernels and marks[2] after the readout kernel (hipEventElapsedTime between them gives
 * the per-phase device time). The events are created and destroyed by the caller; events
 * from oal_timing_event_create keep the recording cheap. */
oal_status oal_prefill_timed(const oal_dims *dims, int32_t T, int32_t chunk, const void *q,
                             const void *k, const void *v, const void *params_dev,
                             float *state_dev, void *workspace, size_t workspace_bytes, float *y,
                             hipStream_t stream, hipEvent_t marks[3]);

/* oal_prefill for a ragged batch (sequences of different lengths, padded to T): sequence b
 * takes the first lengths[b] tokens of its rows of q, k, v ([batch, heads, T, 64], as in
 * oal_prefill) and its state advances by that many tokens; y rows at positions >= lengths[b]
 * are not written. Same kernels, chunk sizes and workspace as oal_prefill with this T.
 *   lengths -- [batch] int32 (device, 4-byte aligned); each value is clamped to [0, T] in
 *              the kernels (0 leaves the sequence's state unchanged).
 * A batch whose lengths are all T gives the results of oal_prefill. */
oal_status oal_prefill_varlen(const oal_dims *dims, int32_t T, const int32_t *lengths, int32_t chunk,
                              const void *q, const void *k, const void *v, const void *params_dev,
                              float *state_dev, void *workspace, size_t workspace_bytes, float *y,
                              hipStream_t stream);

/* oal_prefill for a packed ragged batch: the sequences are concatenated along the token axis,
 * sequence b being tokens cu_seqlens[b] .. cu_seqlens[b+1] - 1 of every head.
 *   cu_seqlens   -- [batch + 1] int32 (device, 4-byte aligned), nondecreasing, from 0 to
 *                   total_tokens. The kernels clamp each offset to [0, total_tokens] and each
 *                   length to [0, min(T, total_tokens - offset)].
 *   total_tokens -- tokens in the packed tensors (>= 0; 0 is a no-op).
 *   T            -- at least the longest sequence (a longer one is cut to its first T tokens);
 *                   it sizes the chunk grid and the workspace, oal_prefill_workspace_bytes(dims,
 *                   T, chunk).
 *   q, y         -- [n_q_heads, total_tokens, 64] (q of dims->dtype, y fp32);
 *   k, v         -- [n_kv_heads, total_tokens, 64].
 * Sequence b's state advances by its length; its y rows are written, no others. Results equal
 * those of oal_prefill_varlen on the same sequences padded to T, bit for bit. */
oal_status oal_prefill_packed(const oal_dims *dims, int32_t T, const int32_t *cu_seqlens,
                              int64_t total_tokens, int32_t chunk, const void *q, const void *k,
                              const void *v, const void *params_dev, float *state_dev,
                              void *workspace, size_t workspace_bytes, float *y, hipStream_t stream);

/* One decode step: appends one token per sequence to the prefix states and reads out the
 * attention of each query head over all tokens so far (the new one included).
 * Passage: reproduction notes, section "核心公式" -- one step of the H-state recurrence,
 * H <- H + psi(k) [v;1]^T, then the readout display for the new token.
 *   q [batch, n_q_heads, 64], k, v [batch, n_kv_heads, 64] of dims->dtype (device);
 *   state_dev updated in place; y [batch, n_q_heads, 64] fp32.
 *   workspace -- oal_decode_workspace_bytes(dims) bytes of device scratch that must be
 *                zero-filled before its first use and then left to the library: every call
 *                returns its counters to zero. The layout depends on dims: a workspace
 *                serves calls of one shape, and must be zero-filled again before it serves
 *                another. Calls that share a workspace must be ordered (same stream or
 *                synchronised). */
oal_status oal_decode_step(const oal_dims *dims, const void *q, const void *k, const void *v,
                           const void *params_dev, float *state_dev, void *workspace,
                           size_t workspace_bytes, float *y, hipStream_t stream);

/* Zero a workspace of oal_decode_step, oal_decode_step_indexed or oal_contribution (its
 * arrival counters and partial sums) with a fill kernel on `stream`: no memset node, so the
 * call may be captured into a graph. A workspace needs it before its first use, before it
 * serves calls of another shape, and after a call that did not run to completion (a device
 * error or an abandoned stream): those calls return their counters to zero only as they
 * finish. workspace 4-byte aligned (OAL_E_ALIGN), workspace_bytes a multiple of 4
 * (OAL_E_ARG); 0 bytes is a no-op. Not a step of the method: the callers are those that keep
 * workspaces across calls. */
oal_status oal_workspace_clear(void *workspace, size_t workspace_bytes, hipStream_t stream);

/* oal_decode_step without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * kernel, arguments (minus the workspace) and results as oal_decode_step, bit for bit. Its
 * workspace is a static device array inside the library, one per GPU, sized for
 * OAL_DECODE_NOALLOC_MAX_BLOCKS (sequence, KV head) blocks (about 12.8 MB) and held until the
 * process ends; the call allocates nothing and zeroes the array's counters itself (with a
 * kernel) before the step. batch * n_kv_heads above the maximum gives OAL_E_UNSUPPORTED.
 * All calls on one GPU share that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must not be issued; order them on one stream. */
#define OAL_DECODE_NOALLOC_MAX_BLOCKS 256
oal_status oal_decode_step_noalloc(const oal_dims *dims, const void *q, const void *k, const void *v,
                                   const void *params_dev, float *state_dev, float *y,
                                   hipStream_t stream);

/* Causal contribution scores of the q/k dims (reproduction notes, section "核心公式", first
 * display; the per-prompt causal statistics that feed the tail grouping in the method's
 * flowchart). For every prompt p (a sequence of the batch), query head h (KV head
 * kv = h / (n_q_heads / n_kv_heads)) and dim r:
 *   chi[p,h,r]    = (1/|Omega_p|) sum_{i} sum_{j<=i} |q[p,h,i,r] k[p,kv,j,r]| / sqrt(d_h),
 *                   |Omega_p| = T (T+1) / 2, the number of causal pairs of the prompt;
 *   chi_mean[h,r] = (1/batch) sum_p chi[p,h,r]   (the average over prompts).
 * The pair sum is evaluated in linear time as sum_i |q_ir| * (prefix sum of |k_jr| up to i),
 * in fp32, in a fixed order (repeated calls give identical bits).
 *   T          -- tokens per prompt (equal lengths), >= 1.
 *   q, k       -- [batch, n_q_heads, T, 64] and [batch, n_kv_heads, T, 64] of dims->dtype
 *                 (device). v is not involved; dims->d_v must still be valid (64).
 *   workspace  -- oal_contribution_workspace_bytes(dims, T) bytes of device scratch (arrival
 *                 counters and per-range partial sums) that must be zero-filled before its
 *                 first use and then left to the library: every call returns its counters to
 *                 zero (the partial sums need no initialisation). The layout depends on
 *                 dims and T: a workspace serves calls of one shape, and must be zero-filled
 *                 again before it serves another. Calls that share a workspace must be
 *                 ordered (same stream or synchronised).
 *   chi        -- [batch, n_q_heads, 64] fp32 out (device).
 *   chi_mean   -- [n_q_heads, 64] fp32 out (device), or NULL to skip the prompt average.
 * batch >= 1 and T >= 1 are required (OAL_E_SHAPE otherwise): the averages are over a
 * non-empty set. T > OAL_CHI_MAX_T gives OAL_E_UNSUPPORTED (a sequence's rows are addressed
 * with 32-bit byte offsets). */
#define OAL_CHI_MAX_T (1 << 22)
size_t oal_contribution_workspace_bytes(const oal_dims *dims, int32_t T);
oal_status oal_contribution(const oal_dims *dims, int32_t T, const void *q, const void *k,
                            void *workspace, size_t workspace_bytes, float *chi, float *chi_mean,
                            hipStream_t stream);

/* Backward of oal_prefill (reproduction notes of arXiv 2610.13674, section "核心公式": kappa,
 * the H-state recurrence and the readout; the gradients follow by the chain rule through the
 * chunked form). For y = oal_prefill(q, k, v) of T tokens per sequence continuing from the
 * prefix states state_in (NULL: a zero state, an empty prefix), and the loss sum(dy * y), it
 * writes
 *   dq [batch, n_q_heads, T, 64], dk and dv [batch, n_kv_heads, T, 64], all fp32 (device);
 *   dstate_in, unless NULL: dLoss/dstate_in, in the state layout (the gradient of each stored
 *        element of H; the 31 padding floats of a block are not written). Chained with the
 *        backward of the call that produced state_in (whose outputs' loss then also depends
 *        on its states through later calls), it trains over a sequence prefilled in pieces.
 * and, unless dL and deps are NULL, the gradients of the kernel coefficients of every query
 * head (summed over the batch):
 *   dL   [n_q_heads][65][65] fp32 (device, 4-byte aligned): entry [h][a][b] is dLoss/dL[a][b]
 *        of head h for b <= a <= n_groups[h]; every other entry is written as 0;
 *   deps [n_q_heads] fp32 (device, 4-byte aligned): dLoss/deps.
 * (Both NULL, or both given: OAL_E_ARG otherwise.) The forward quantities it needs (the
 * prefix states, y and the normaliser per query) are recomputed in fp32 from q, k, v; the
 * caller passes no saved output.
 *   T          -- tokens per sequence (equal lengths), >= 0; T = 0 or batch = 0 is a no-op.
 *   chunk      -- 64, 128 or 256: tokens per chunk of the chunked form.
 *   q, k, v    -- as for oal_prefill ([batch, heads, T, 64] of dims->dtype, device).
 *   dy         -- [batch, n_q_heads, T, 64] fp32 (device).
 *   params_dev -- the blob oal_state_init uploaded.
 *   state_in   -- [batch, n_kv_heads] state blocks (oal_state_bytes(dims) bytes, device) that
 *                 the forward call started from, or NULL for an empty prefix.
 *   workspace  -- oal_prefill_backward_workspace_bytes(dims, T, chunk) bytes of device scratch
 *                 (per-chunk states, one block of OAL_STATE_STRIDE floats per sequence, KV
 *                 head and chunk; the per-query readout gradients, also in three bf16 parts
 *                 per 64-query tile; partial dq, key and coefficient gradients); contents on
 *                 entry do not matter.
 * All arithmetic is to fp32 accuracy whatever dims->dtype is (bf16 inputs are widened on load;
 * the state contractions run on bf16 MFMA with each fp32 operand split in three bf16 parts and
 * the six products of order <= 2, the rest on fp32 MFMA or the VALU). Every
 * pointer but dL and deps must be 16-byte aligned (OAL_E_ALIGN; state_in and dstate_in when
 * given). T = 0 writes nothing. More than 65535 chunks per sequence,
 * n_q_heads + 3 n_kv_heads > 65535 or n_kv_heads > 8191 give OAL_E_UNSUPPORTED (grid limits). */
size_t oal_prefill_backward_workspace_bytes(const oal_dims *dims, int32_t T, int32_t chunk);
oal_status oal_prefill_backward(const oal_dims *dims, int32_t T, int32_t chunk, const void *q,
                                const void *k, const void *v, const float *dy,
                                const void *params_dev, const float *state_in, void *workspace,
                                size_t workspace_bytes, float *dq, float *dk, float *dv,
                                float *dstate_in, float *dL, float *deps, hipStream_t stream);

/* Decode step for sequences whose states live in a pool (serving: a batch of active
 * sequences over a larger set of state blocks). Sequence b of the batch uses pool block
 * slots[b]; otherwise identical to oal_decode_step (same kernels, same results bit for bit
 * as oal_decode_step on a state buffer holding those blocks in batch order).
 *   slots      -- [batch] int32 (device, 4-byte aligned): pool block of each sequence. The
 *                 slots of one call must be distinct (two sequences on one block race).
 *                 A slot outside [0, pool_size) is not an error: that sequence's state is not
 *                 touched and its y is NaN (the kernels check every slot).
 *   pool_size  -- blocks in the pool, >= 1 (OAL_E_SHAPE otherwise).
 *   state_pool -- [pool_size, n_kv_heads] blocks of OAL_STATE_STRIDE floats, the state
 *                 layout above (a state buffer with batch = pool_size); updated in place at
 *                 the slots of the batch, every other block left as it is.
 *   workspace  -- oal_decode_workspace_bytes(dims) bytes, same contract as oal_decode_step
 *                 (dims->batch is the number of active sequences, not the pool size).
 * q, k, v, y, params_dev: as in oal_decode_step, indexed by the batch position b. A pool is
 * filled by oal_state_init (batch = pool_size) or by oal_prefill on one block (batch = 1,
 * state_dev = the block's address). */
oal_status oal_decode_step_indexed(const oal_dims *dims, const int32_t *slots, int32_t pool_size,
                                   const void *q, const void *k, const void *v,
                                   const void *params_dev, float *state_pool, void *workspace,
                                   size_t workspace_bytes, float *y, hipStream_t stream);

/* Timing events for oal_prefill_timed and for bracketing a timed region. A default HIP event
 * performs a system-scope release when it is recorded, which writes back the L2: between two
 * kernels that leave many dirty lines that costs several microseconds and would be counted
 * as kernel time. These events are created with hipEventDisableSystemFence: their timestamps
 * are the same, only the release is skipped, so they must not be used to order memory
 * accesses with the host.
 *   oal_timing_event_create  -- *event receives a new event (OAL_E_HIP on failure).
 *   oal_timing_event_destroy -- releases it (NULL is accepted).
 *   oal_timing_event_record  -- records it on `stream`.
 *   oal_timing_elapsed_ms    -- waits for `end` to complete, then *ms = time from start to
 *                               end; both must have been recorded. */
oal_status oal_timing_event_create(hipEvent_t *event);
oal_status oal_timing_event_destroy(hipEvent_t event);
oal_status oal_timing_event_record(hipEvent_t event, hipStream_t stream);
oal_status oal_timing_elapsed_ms(hipEvent_t start, hipEvent_t end, float *ms);

/* Static description of a status code. */
const char *oal_status_string(oal_status status);

#ifdef __cplusplus
}
#endif

#endif /* OAL_H */
