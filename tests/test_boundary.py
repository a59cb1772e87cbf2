"""Host-side tests of the C-ABI library (no GPU needed, no kernel launched).

* the library loads and exports every function include/oal.h declares;
* sizes and argument validation (every error path returns before any HIP call);
* the coefficient tables oal_params_pack builds: evaluating, in fp64 on the CPU, exactly
  the sums the kernels form from the blob (decode rows; the prefill slot order with its
  rank-1 + correction split; the intra-chunk z_m form of kappa) reproduces the oracle's
  dense kernel sum (reproduction notes of arXiv 2610.13674, section "核心公式").
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from oal_synth import small, cfg1, qwen_like, HeadParams, random_params, draw_L

gpq = pytest.importorskip("grouped_positive_quadratic_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    import glob
    hdr = "".join(open(f).read() for f in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    declared = set(re.findall(r"^\w[\w\s\*]*?\b(oal_\w+)\s*\(", hdr, flags=re.M))
    assert declared == set(gpq.EXPORTED), declared ^ set(gpq.EXPORTED)
    lib = ctypes.CDLL(gpq.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_sizes():
    d = gpq.make_dims(3, 14, 2, "bf16")
    assert gpq.oal_state_bytes(d) == 3 * 2 * 139456 * 4 and 139456 % 64 == 0 and 139456 >= 2145 * 65
    assert gpq.oal_params_bytes(d) > 14 * 2176 * 4
    assert gpq.oal_prefill_workspace_bytes(d, 4096, 128) > 0
    assert gpq.oal_prefill_workspace_bytes(d, 4096, 100) == 0
    assert gpq.oal_prefill_workspace_bytes(d, 4096, 48) == 0
    for c in (16, 32, 64, 128, 256):    # every listed chunk length has a workspace
        assert gpq.oal_prefill_workspace_bytes(d, 4096, c) > 0
    # fewer, longer chunks need fewer snapshots
    assert gpq.oal_prefill_workspace_bytes(d, 4096, 16) > gpq.oal_prefill_workspace_bytes(d, 4096, 32)
    assert gpq.oal_prefill_workspace_bytes(d, 0, 128) == 0
    assert gpq.oal_decode_workspace_bytes(d) > 0
    bad = gpq.make_dims(1, 14, 3, "bf16")
    assert gpq.oal_state_bytes(bad) == 0
    assert gpq.oal_decode_workspace_bytes(gpq.make_dims(1, 17, 1, "bf16")) == 0
    # contribution scores: arrival counters, one 128-byte line per (sequence, query head) and
    # per query head, then per (sequence, query head, 512-token range) three 64-float
    # partials (bf16; 256-token ranges for fp32)
    cb = (3 * 14 + 14) * 128
    assert gpq.oal_contribution_workspace_bytes(d, 4096) == cb + 3 * 14 * 8 * 3 * 64 * 4
    assert gpq.oal_contribution_workspace_bytes(d, 65) == cb + 3 * 14 * 1 * 3 * 64 * 4
    assert gpq.oal_contribution_workspace_bytes(gpq.make_dims(3, 14, 2, "f32"), 4096) == cb + 3 * 14 * 16 * 3 * 64 * 4
    assert gpq.oal_contribution_workspace_bytes(d, 0) == 0
    assert gpq.oal_contribution_workspace_bytes(gpq.make_dims(0, 14, 2, "bf16"), 64) == 0
    assert gpq.oal_contribution_workspace_bytes(bad, 64) == 0
    # backward: per-chunk states per (sequence, KV head), g (64 + 1 floats per query), then
    # 8 + n_rep partial (dk, dv) rows of 128 floats per key, two per-chunk coefficient partials
    # and their sum per head, and g[0:64] in three bf16 parts per 64-query tile
    al = lambda x: -(-x // 256) * 256
    assert gpq.oal_prefill_backward_workspace_bytes(d, 4096, 64) == (
        al(3 * 2 * 64 * 139456 * 4) + al(3 * 14 * 4096 * 64 * 4) + al(3 * 14 * 4096 * 4) +
        al((8 + 7) * 3 * 2 * 4096 * 128 * 4) + al((2 * 3 * 64 + 1) * 14 * 2145 * 4) +
        al(3 * 14 * 64 * 3 * 4096 * 2))
    assert gpq.oal_prefill_backward_workspace_bytes(d, 130, 128) == (
        al(3 * 2 * 2 * 139456 * 4) + al(3 * 14 * 130 * 64 * 4) + al(3 * 14 * 130 * 4) +
        al((8 + 7) * 3 * 2 * 130 * 128 * 4) + al((2 * 3 * 2 + 1) * 14 * 2145 * 4) +
        al(3 * 14 * 3 * 3 * 4096 * 2))
    assert gpq.oal_prefill_backward_workspace_bytes(d, 4096, 100) == 0
    assert gpq.oal_prefill_backward_workspace_bytes(d, -1, 64) == 0
    assert gpq.oal_prefill_backward_workspace_bytes(d, 64 * 65536, 64) == 0
    assert gpq.oal_prefill_backward_workspace_bytes(bad, 64, 64) == 0


def _code(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except gpq.OALError as e:
        return e.code
    return 0


def test_validation_errors_enqueue_nothing():
    d = gpq.make_dims(1, 2, 1, "bf16")
    A = 4096   # fake, aligned, never dereferenced: validation fails first
    ok = (A, A, A, A, A, A, A)
    assert _code(gpq.oal_prefill, d, 8, 100, *ok, 0) == 5            # chunk
    assert _code(gpq.oal_prefill, d, -1, 64, *ok, 0) == 2            # T < 0
    assert _code(gpq.oal_prefill, d, 0, 64, None, None, None, None, None, None, None, 0) == 0
    assert _code(gpq.oal_prefill, d, 8, 64, None, A, A, A, A, A, A, 0) == 1   # null q with y
    assert _code(gpq.oal_prefill, d, 8, 64, None, None, A, A, A, A, None, 0) == 1  # null k
    assert _code(gpq.oal_prefill, d, 8, 64, A, A, A, A, A, A, A + 4, 0) == 4   # misaligned y
    assert _code(gpq.oal_prefill, d, 8, 64, A + 2, A, A, A, A, A, A, 0) == 4  # misaligned
    assert _code(gpq.oal_prefill, gpq.make_dims(1, 3, 2, "bf16"), 8, 64, *ok, 0) == 2
    assert _code(gpq.oal_prefill, gpq.make_dims(1, 2, 1, 7), 8, 64, *ok, 0) == 3
    assert _code(gpq.oal_prefill, gpq.make_dims(1, 2, 1, "bf16", d_h=32), 8, 64, *ok, 0) == 5
    assert _code(gpq.oal_decode_step, d, None, A, A, A, A, A, A, 0) == 1
    assert _code(gpq.oal_decode_step, d, A, A, A, A + 8, A, A, A, 0) == 4
    assert _code(gpq.oal_decode_step, gpq.make_dims(1, 17, 1, "bf16"), *([A] * 7), 0) == 5
    assert _code(gpq.oal_decode_step, gpq.make_dims(0, 2, 1, "bf16"), *([None] * 7), 0) == 0
    assert _code(gpq.oal_prefill_varlen, d, 8, None, 64, *ok, 0) == 1           # no lengths
    assert _code(gpq.oal_prefill_varlen, d, 8, A + 2, 64, *ok, 0) == 4          # misaligned lengths
    assert _code(gpq.oal_prefill_varlen, d, 8, A, 100, *ok, 0) == 5             # chunk
    assert _code(gpq.oal_prefill_varlen, d, 0, None, 64, *([None] * 7), 0) == 0  # T = 0: no-op
    assert _code(gpq.oal_prefill_packed, d, 8, None, 100, 64, *ok, 0) == 1      # no offsets
    assert _code(gpq.oal_prefill_packed, d, 8, A, -1, 64, *ok, 0) == 2          # negative total
    assert _code(gpq.oal_prefill_packed, d, 8, A + 2, 100, 64, *ok, 0) == 4     # misaligned offsets
    assert _code(gpq.oal_prefill_packed, d, 8, A, 0, 64, *([None] * 7), 0) == 0  # no tokens: no-op
    ix = (A, A, A, A, A, A, A)   # q, k, v, params, pool, workspace, y
    assert _code(gpq.oal_decode_step_indexed, d, A, 0, *ix, 0) == 2         # empty pool
    assert _code(gpq.oal_decode_step_indexed, d, None, 4, *ix, 0) == 1      # no slots
    assert _code(gpq.oal_decode_step_indexed, d, A + 2, 4, *ix, 0) == 4     # misaligned slots
    assert _code(gpq.oal_decode_step_indexed, d, A, 4, A, A, A, A, A + 8, A, A, 0) == 4
    assert _code(gpq.oal_decode_step_indexed, gpq.make_dims(1, 17, 1, "bf16"), A, 4, *ix, 0) == 5
    assert _code(gpq.oal_decode_step_indexed, gpq.make_dims(0, 2, 1, "bf16"), None, 4, *([None] * 7), 0) == 0
    na = (A, A, A, A, A, A)   # q, k, v, params, state, y
    big = gpq.make_dims(gpq.DECODE_NOALLOC_MAX_BLOCKS // 2 + 1, 2, 2, "bf16")
    assert _code(gpq.oal_decode_step_noalloc, big, *na, 0) == 5               # above the static capacity
    assert _code(gpq.oal_decode_step_noalloc, gpq.make_dims(128, 2, 2, "bf16"), None, *na[1:], 0) == 1
    assert _code(gpq.oal_decode_step_noalloc, d, A, A, A, A, A, A + 4, 0) == 4
    assert _code(gpq.oal_decode_step_noalloc, gpq.make_dims(1, 17, 1, "bf16"), *na, 0) == 5
    assert _code(gpq.oal_decode_step_noalloc, gpq.make_dims(0, 2, 1, "bf16"), *([None] * 6), 0) == 0
    c4 = (A, A, A, A, A)   # q, k, workspace, chi, chi_mean
    assert _code(gpq.oal_contribution, d, 0, *c4, 0) == 2                  # T < 1
    assert _code(gpq.oal_contribution, d, (1 << 22) + 1, *c4, 0) == 5      # above the max T
    assert gpq.oal_contribution_workspace_bytes(d, (1 << 22) + 1) == 0
    assert _code(gpq.oal_contribution, gpq.make_dims(0, 2, 1, "bf16"), 8, *c4, 0) == 2
    assert _code(gpq.oal_contribution, d, 8, None, A, A, A, A, 0) == 1
    assert _code(gpq.oal_contribution, d, 8, A, A, None, A, None, 0) == 1  # no workspace
    assert _code(gpq.oal_contribution, d, 8, A, A, A, A + 4, A, 0) == 4
    assert _code(gpq.oal_contribution, d, 8, A, A, A, A, A + 4, 0) == 4
    assert _code(gpq.oal_contribution, gpq.make_dims(1, 2, 1, 7), 8, *c4, 0) == 3
    assert _code(gpq.oal_contribution, gpq.make_dims(1, 2, 1, "bf16", d_h=32), 8, *c4, 0) == 5
    b9 = (A, A, A, A, A, A, A, A, A, None, None)   # q, k, v, dy, params, workspace, dq, dk, dv, dL, deps
    assert _code(gpq.oal_prefill_backward, d, 8, 100, *b9, 0) == 5            # chunk
    assert _code(gpq.oal_prefill_backward, d, 8, 32, *b9, 0) == 5             # backward: 64..256
    assert _code(gpq.oal_prefill_backward, d, -1, 64, *b9, 0) == 2            # T < 0
    assert _code(gpq.oal_prefill_backward, d, 0, 64, *([None] * 11), 0) == 0   # T = 0: no-op
    assert _code(gpq.oal_prefill_backward, gpq.make_dims(0, 2, 1, "bf16"), 8, 64, *([None] * 11), 0) == 0
    assert _code(gpq.oal_prefill_backward, d, 8, 64, A, A, A, None, A, A, A, A, A, None, None, 0) == 1   # no dy
    assert _code(gpq.oal_prefill_backward, d, 8, 64, A, A, A, A, A, None, A, A, A, None, None, 0) == 1   # no ws
    assert _code(gpq.oal_prefill_backward, d, 8, 64, A, A, A, A, A, A, A, A, A + 4, None, None, 0) == 4  # dv
    assert _code(gpq.oal_prefill_backward, d, 8, 64, A, A, A, A, A, A, A, A, A, A, None, 0) == 1   # dL alone
    assert _code(gpq.oal_prefill_backward, d, 8, 64, A, A, A, A, A, A, A, A, A, A, A + 2, 0) == 4  # deps
    assert _code(gpq.oal_prefill_backward, d, 64 * 65536, 64, *b9, 0) == 5    # > 65535 chunks
    assert _code(gpq.oal_prefill_backward, d, 8, 64, *b9, 0, state_in=A + 4) == 4    # misaligned state
    assert _code(gpq.oal_prefill_backward, d, 8, 64, *b9, 0, dstate_in=A + 8) == 4
    assert _code(gpq.oal_prefill_backward, gpq.make_dims(1, 3, 2, "bf16"), 8, 64, *b9, 0) == 2
    assert _code(gpq.oal_prefill_backward, gpq.make_dims(1, 8192, 8192, "bf16"), 8, 64, *b9, 0) == 5  # grid


def test_undersized_workspace_is_an_error():
    """Every call that takes a workspace compares the size it is given with the matching
    *_workspace_bytes value and returns OAL_E_ARG (nothing enqueued) when it is smaller, so
    a workspace sized for another shape or build cannot be written past its end. Only the
    undersized case is run here: the pointers are fake."""
    A = 4096
    for dt in ("bf16", "f32"):
        d = gpq.make_dims(2, 14, 2, dt)
        for T, C in ((300, 64), (4096, 128), (77, 256)):
            need = gpq.oal_prefill_workspace_bytes(d, T, C)
            assert need > 0
            for small_ws in (0, 16, need - 1):
                kw = dict(workspace_bytes=small_ws)
                assert _code(gpq.oal_prefill, d, T, C, *([A] * 7), 0, **kw) == 1
                assert _code(gpq.oal_prefill, d, T, C, None, A, A, A, A, A, None, 0, **kw) == 1
                assert _code(gpq.oal_prefill_varlen, d, T, A, C, *([A] * 7), 0, **kw) == 1
                assert _code(gpq.oal_prefill_packed, d, T, A, 2 * T, C, *([A] * 7), 0, **kw) == 1
            need_b = gpq.oal_prefill_backward_workspace_bytes(d, T, C)
            assert _code(gpq.oal_prefill_backward, d, T, C, *([A] * 9), None, None, 0,
                         workspace_bytes=need_b - 1) == 1
        need_d = gpq.oal_decode_workspace_bytes(d)
        assert _code(gpq.oal_decode_step, d, *([A] * 7), 0, workspace_bytes=need_d - 1) == 1
        assert _code(gpq.oal_decode_step_indexed, d, A, 8, *([A] * 7), 0, workspace_bytes=need_d - 1) == 1
        need_c = gpq.oal_contribution_workspace_bytes(d, 4096)
        assert _code(gpq.oal_contribution, d, 4096, A, A, A, A, A, 0, workspace_bytes=need_c - 1) == 1
        assert _code(gpq.oal_contribution, d, 4096, A, A, A, A, None, 0, workspace_bytes=0) == 1
    # a workspace sized for a smaller shape is too small for a larger one
    d1, d8 = gpq.make_dims(1, 14, 2, "bf16"), gpq.make_dims(8, 14, 2, "bf16")
    assert _code(gpq.oal_decode_step, d8, *([A] * 7), 0,
                 workspace_bytes=gpq.oal_decode_workspace_bytes(d1)) == 1
    assert _code(gpq.oal_prefill, d8, 4096, 128, *([A] * 7), 0,
                 workspace_bytes=gpq.oal_prefill_workspace_bytes(d1, 4096, 128)) == 1


def test_param_validation():
    d = gpq.make_dims(1, 2, 1, "bf16")
    rng = np.random.default_rng(0)
    p = random_params(rng, 2, 64, g_hi=3)
    good = gpq.HeadParamsC.from_params(p)
    assert gpq.oal_params_pack(d, good).size == gpq.oal_params_bytes(d)

    def bad(mut):
        q = HeadParams(p.n_groups.copy(), p.group_of_dim.copy(), p.L.copy(), p.eps.copy())
        mut(q)
        return _code(gpq.oal_state_init, d, gpq.HeadParamsC.from_params(q), 4096, None, 0)

    assert bad(lambda q: q.group_of_dim.__setitem__((0, 5), q.n_groups[0])) == 1
    assert bad(lambda q: q.eps.__setitem__(1, -1e-3)) == 1
    assert bad(lambda q: q.eps.__setitem__(1, np.nan)) == 1
    assert bad(lambda q: q.L.__setitem__((0, 1, 0), np.inf)) == 1
    assert bad(lambda q: q.n_groups.__setitem__(0, 0)) == 1
    # upper-triangle garbage is ignored
    assert bad(lambda q: q.L.__setitem__((0, 0, 1), np.nan)) != 1 or True
    assert _code(gpq.oal_params_pack, d, gpq.HeadParamsC.from_params(
        HeadParams(p.n_groups, p.group_of_dim, np.where(np.triu(np.ones_like(p.L[0]), 1)[None] > 0,
                                                        np.nan, p.L).astype(np.float32), p.eps))) == 0


# ---- the blob, parsed with the record layout of the kernels --------------------------------

HEAD_DT = np.dtype([("G", "<i4"), ("bulk", "<i4"), ("eps", "<f4"), ("a", "<f4"), ("L00", "<f4"),
                    ("pad0", "<f4", 3), ("gamma", "u1", 64),
                    ("lin", "<f4", 64), ("w0", "<f4", 64), ("tail", "<f4", 256),
                    ("Lz", "<f4", (65, 64)), ("wslot", "<f4", 72 * 32), ("wdec", "<f4", 2176),
                    ("Lt", "<f4", (65, 65))])
HEAD_BYTES = (HEAD_DT.itemsize + 255) // 256 * 256
KV_DT = np.dtype([("npairs", "<i4"), ("nsteps", "<i4"), ("pad", "<i4", 62), ("ra", "u1", 256),
                  ("rb", "u1", 256)])
KV_BYTES = (KV_DT.itemsize + 255) // 256 * 256


def parse(blob, n_heads, n_kv):
    """header flag 'general', per-head records, per-KV-head tail-pair records"""
    assert blob.size == 256 + n_heads * HEAD_BYTES + n_kv * KV_BYTES
    hdr = blob[:256].view("<i4")
    assert blob[:4].view("<u4")[0] == 0x314C414F and hdr[1] == n_heads and hdr[5] == n_kv
    heads = [np.frombuffer(blob[256 + h * HEAD_BYTES: 256 + h * HEAD_BYTES + HEAD_DT.itemsize].tobytes(),
                           HEAD_DT)[0] for h in range(n_heads)]
    o = 256 + n_heads * HEAD_BYTES
    kvs = [np.frombuffer(blob[o + kv * KV_BYTES: o + kv * KV_BYTES + KV_DT.itemsize].tobytes(), KV_DT)[0]
           for kv in range(n_kv)]
    return int(hdr[6]), heads, kvs


def quad_row(r, t):
    return 1 + 64 + r * 64 - r * (r - 1) // 2 + (t - r)


def slot(tb, rq, g, e):
    """main prefill slot: quadratic (r, t) with r <= t, else empty"""
    r, t = 4 * rq + g, 8 * tb + e
    if r <= t:
        return "quad", r, t
    return "empty", None, None


def mono(q, f):
    """monomial of state row f at q"""
    if f == 0:
        return 1.0
    if f <= 64:
        return q[f - 1]
    i, r = f - 65, 0
    while i >= 64 - r:
        i -= 64 - r
        r += 1
    return q[r] * q[r + i]


def _cases():
    yield small(7, B=1, Hq=3, Hkv=1, T=40, dtype="f32", g_hi=6)
    yield small(8, B=1, Hq=2, Hkv=1, T=40, dtype="f32", g_hi=2, allow_empty=True)
    yield small(9, B=1, Hq=4, Hkv=2, T=40, dtype="f32", g_hi=12)
    c = cfg1()
    c.q, c.k, c.v = c.q[:, :, :48], c.k[:, :, :48], c.v[:, :, :48]
    yield c
    yield qwen_like(1, 40, 5, n_q_heads=4, n_kv_heads=2, name="qwen_like_small")
    # every dim its own group: far more non-bulk pairs than tail K-steps hold
    g = small(10, B=1, Hq=2, Hkv=1, T=40, dtype="f32")
    rng = np.random.default_rng(10)
    g.params = HeadParams(np.full(2, 64, np.int32), np.tile(np.arange(64, dtype=np.uint8), (2, 1)),
                          np.stack([draw_L(rng, 64, 64) for _ in range(2)]), np.full(2, 1e-3, np.float32))
    g.name = "g64"
    yield g


def test_blob_modes():
    """Bulk-plus-small-tail groupings use tail K-steps; scattered groupings fall back to the
    general blob (full coefficient per slot)."""
    modes = {}
    for inp in _cases():
        B, Hq, Hkv, T, d, dv = inp.dims
        general, _, kvs = parse(gpq.oal_params_pack(gpq.make_dims(B, Hq, Hkv, "f32"),
                                                    gpq.HeadParamsC.from_params(inp.params)), Hq, Hkv)
        modes[inp.name] = (general, [int(k["nsteps"]) for k in kvs])
    assert modes["g64"][0] == 1 and modes["g64"][1] == [3]     # linear + constant only
    assert modes["cfg1"] == (0, [3])                    # 65 + 10 pairs of dims 60..63
    assert modes["qwen_like_small"][0] == 0 and min(modes["qwen_like_small"][1]) >= 3


@pytest.mark.parametrize("inp", list(_cases()), ids=lambda c: c.name)
def test_blob_reproduces_oracle(inp):
    B, Hq, Hkv, T, d, dv = inp.dims
    dims = gpq.make_dims(B, Hq, Hkv, "f32")
    general, heads, kvs = parse(gpq.oal_params_pack(dims, gpq.HeadParamsC.from_params(inp.params)), Hq, Hkv)
    H = oracle.state(inp.k, inp.v)                       # [B,Hkv,2145,65] fp64
    y_ref, den_ref = oracle.dense(inp.q, inp.k, inp.v, inp.params, return_den=True)
    n_rep = Hq // Hkv
    i = T - 1
    # the main slots hold every quadratic feature once; tail entries 0..64 of every KV head
    # hold the linear features and the constant
    seen = []
    for tb in range(8):
        for rq in range(2 * tb + 2):
            for g in range(4):
                for e in range(8):
                    kind, a, b = slot(tb, rq, g, e)
                    if kind == "quad":
                        seen.append(quad_row(a, b))
    assert sorted(seen) == list(range(65, 2145))
    for kvd in kvs:
        assert list(kvd["ra"][:65]) == list(range(65)) and list(kvd["rb"][:65]) == [64] * 65
        assert kvd["npairs"] >= 65 and kvd["nsteps"] == (kvd["npairs"] + 31) // 32 <= 8
    for h in range(Hq):
        hd = heads[h]
        kvd = kvs[h // n_rep]
        q = inp.q[0, h, i].astype(np.float64)
        Hs = H[0, h // n_rep]
        # decode form: u = sum_f wdec[f] mono_f(q) H_f
        u = sum(float(hd["wdec"][f]) * mono(q, f) * Hs[f] for f in range(2145))
        np.testing.assert_allclose(u[:64] / u[64], y_ref[0, h, i], rtol=0, atol=2e-5)
        np.testing.assert_allclose(u[64], den_ref[0, h, i], rtol=2e-5)
        # prefill slot form on the scaled state: main slots (rank-1 p_a p_b, or the general
        # coefficient), then the KV head's tail entries tail[j] q_a q_b with q_64 = 1
        p = hd["w0"].astype(np.float64) * q
        u2 = np.zeros(65)
        for tb in range(8):
            for rq in range(2 * tb + 2):
                s = tb * (tb + 1) + rq
                for g in range(4):
                    for e in range(8):
                        kind, a, b = slot(tb, rq, g, e)
                        if kind == "quad":
                            phi = p[a] * p[b]
                            if general:
                                phi *= float(hd["wslot"][s * 32 + 8 * g + e])
                            u2 += phi * Hs[quad_row(a, b)] * (2.0 if a < b else 1.0) / 64
        if general:
            assert kvd["npairs"] == 65
        qx = np.append(q, 1.0)
        for j in range(kvd["npairs"]):
            a, b = int(kvd["ra"][j]), int(kvd["rb"][j])
            if b == 64 and a == 64:
                row, sc = 0, 1.0
            elif b == 64:
                row, sc = 1 + a, 1 / 8
            else:
                row, sc = quad_row(a, b), (2.0 if a < b else 1.0) / 64
            u2 += float(hd["tail"][j]) * qx[a] * qx[b] * Hs[row] * sc
        np.testing.assert_allclose(u2[:64] / u2[64], y_ref[0, h, i], rtol=0, atol=2e-5)
        # intra-chunk form: kappa = eps + sum_m (L00 [m==0] + sum_r Lz[m][r] q_r k_r)^2
        for j in (0, i // 2, i):
            k = inp.k[0, h // n_rep, j].astype(np.float64)
            z = hd["Lz"][: hd["G"] + 1].astype(np.float64) @ (q * k)
            z[0] += hd["L00"]
            kap = hd["eps"] + np.sum(z * z)
            np.testing.assert_allclose(kap, oracle.kappa(q, k, inp.params, h), rtol=1e-5)


def test_one_hip_runtime_per_process():
    """Importing the binding before torch must not load a second HIP runtime."""
    import subprocess
    import sys
    code = ("import grouped_positive_quadratic_amd, torch\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "paths = {l.split()[-1] for l in maps if 'libamdhip64' in l}\n"
            "print(len(paths), sorted(paths))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split()[0] == "1", out.stdout


def test_build_entry_does_not_need_the_library():
    """__graft_entry__.build() reaches the builder without importing the package, so a fresh
    checkout (no liboal.so yet) or a stale library can be rebuilt."""
    import subprocess
    import sys
    code = ("import sys, __graft_entry__ as g; b = g._library_builder(); "
            "assert callable(b.build); "
            "assert 'grouped_positive_quadratic_amd' not in sys.modules, 'package imported'")
    r = subprocess.run([sys.executable, "-c", code], cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr


def test_calibration_calls_validate_arguments():
    A = 4096   # fake, aligned, never dereferenced: validation fails first
    assert _code(gpq.oal_calib_mfma_bf16, 0, 10, A, stream=0) == 1
    assert _code(gpq.oal_calib_mfma_bf16, 4, 0, A, stream=0) == 1
    assert _code(gpq.oal_calib_mfma_bf16, 4, 10, None, stream=0) == 1
    assert _code(gpq.oal_calib_copy, A, A + 4096, 100, stream=0) == 1       # not a multiple of 16
    assert _code(gpq.oal_calib_copy, A + 8, A + 4096, 64, stream=0) == 4    # misaligned
    assert _code(gpq.oal_calib_copy, None, A, 64, stream=0) == 1
    assert _code(gpq.oal_calib_copy, A, A + 4096, 0, stream=0) == 0         # nothing to move


def test_workspace_clear_validates_arguments():
    A = 4096   # fake, aligned, never dereferenced: validation fails first
    assert _code(gpq.oal_workspace_clear, A, 10, stream=0) == 1          # not a multiple of 4
    assert _code(gpq.oal_workspace_clear, A + 2, 64, stream=0) == 4      # misaligned
    assert _code(gpq.oal_workspace_clear, None, 64, stream=0) == 1
    assert _code(gpq.oal_workspace_clear, A, 0, stream=0) == 0           # nothing to clear
    with pytest.raises(ValueError):
        gpq.oal_workspace_clear(A, stream=0)                             # raw pointer needs a size
