"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Tolerances (row-normwise max relative error, max over rows of
||y_i - y*_i||_inf / ||y*_i||_inf): 1e-5 for fp32 inputs, 3e-2 for bf16 inputs with fp32
accumulation. States are compared blockwise (max abs error over max abs value).
"""
import numpy as np
import pytest

import oracle
from oal_synth import small, cfg1, cfg2, qwen_like, HeadParams, round_bf16, draw_L

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import Session, session_for, to_dev, state_error, state_ok, TOL  # noqa: E402
import grouped_positive_quadratic_amd as gpq  # noqa: E402


def _report(name, err):
    print(f"[parity] {name}: err={err:.3e}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


# ---------------------------------------------------------------------------------------

def test_decode_from_zero_cfg1():
    inp = cfg1()
    sess = session_for(inp)
    T = inp.q.shape[2]
    ys = []
    for i in range(T):
        ys.append(sess.decode(inp.q[:, :, i], inp.k[:, :, i], inp.v[:, :, i]))
    y = torch.stack(ys, dim=2).cpu().numpy()
    err = oracle.row_error(y, oracle.dense(inp.q, inp.k, inp.v, inp.params))
    _report("decode cfg1 (256 steps from zero)", err)
    assert err <= TOL["f32"]
    serr = state_error(sess.state_np(), oracle.state(inp.k, inp.v))
    _report("decode cfg1 state", serr)
    assert serr <= 1e-5


@pytest.mark.parametrize("chunk", [16, 32, 64, 128, 256])
def test_prefill_cfg1(chunk):
    inp = cfg1()
    sess = session_for(inp, chunk)
    y = sess.prefill(inp.q, inp.k, inp.v, chunk).cpu().numpy()
    err = oracle.row_error(y, oracle.dense(inp.q, inp.k, inp.v, inp.params))
    _report(f"prefill cfg1 C={chunk}", err)
    assert err <= TOL["f32"]
    serr = state_error(sess.state_np(), oracle.state(inp.k, inp.v))
    _report(f"prefill cfg1 C={chunk} state", serr)
    assert serr <= 1e-5


SMALL = [  # seed, B, Hq, Hkv, T, chunk
    (11, 1, 7, 1, 200, 64),
    (12, 2, 4, 2, 77, 128),
    (13, 1, 14, 2, 300, 128),
    (14, 1, 2, 1, 1, 64),
    (15, 1, 8, 1, 129, 256),
    (16, 2, 3, 1, 64, 64),
    (17, 1, 14, 2, 520, 64),
    (18, 1, 16, 1, 150, 128),   # 16 query heads per KV head: two readout head groups, two heads per intra wave
    (19, 1, 12, 1, 130, 64),    # 12 per KV head: readout head groups of 4
    (20, 2, 5, 1, 90, 128),     # 5 per KV head: head groups of 1
    (21, 1, 6, 6, 70, 64),      # one query head per KV head (no GQA)
    (23, 1, 14, 2, 101, 16),    # chunks of one query tile (ragged tail)
    (24, 2, 7, 1, 77, 32),      # chunks of two query tiles
    (25, 1, 14, 2, 40, 16),     # T = 2.5 chunks
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "s{}_B{}_H{}x{}_T{}_C{}".format(*c))
def test_prefill_small(case, dtype):
    seed, B, Hq, Hkv, T, chunk = case
    inp = small(seed, B, Hq, Hkv, T, dtype=dtype)
    sess = session_for(inp, chunk)
    y = sess.prefill(inp.q, inp.k, inp.v, chunk).cpu().numpy()
    err = oracle.row_error(y, oracle.dense(inp.q, inp.k, inp.v, inp.params))
    _report(f"prefill {dtype} {case}", err)
    assert err <= TOL[dtype]
    assert state_ok(sess.state_np(), inp.k, inp.v, dtype)


@pytest.mark.parametrize("shape", [(16, 1), (12, 2), (6, 6)], ids=["H16x1", "H12x2", "H6x6"])
def test_prefill_then_decode_head_counts(shape):
    # decode with more than 8 query heads per KV head (the 16-head decode kernel) and without
    # GQA, after a prefill of the same sequences
    Hq, Hkv = shape
    inp = small(25, 2, Hq, Hkv, 140, dtype="bf16")
    T0 = 120
    sess = session_for(inp, 64)
    y0 = sess.prefill(inp.q[:, :, :T0], inp.k[:, :, :T0], inp.v[:, :, :T0], 64)
    ys = [sess.decode(inp.q[:, :, i], inp.k[:, :, i], inp.v[:, :, i]) for i in range(T0, 140)]
    y = np.concatenate([y0.cpu().numpy(), torch.stack(ys, 2).cpu().numpy()], axis=2)
    err = oracle.row_error(y, oracle.dense(inp.q, inp.k, inp.v, inp.params))
    _report(f"prefill+decode H{Hq}x{Hkv}", err)
    assert err <= TOL["bf16"]
    assert state_ok(sess.state_np(), inp.k, inp.v, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_then_decode(dtype):
    inp = small(21, 2, 14, 2, 160, dtype=dtype)
    T0 = 100
    sess = session_for(inp, 64)
    y0 = sess.prefill(inp.q[:, :, :T0], inp.k[:, :, :T0], inp.v[:, :, :T0], 64)
    ys = [sess.decode(inp.q[:, :, i], inp.k[:, :, i], inp.v[:, :, i]) for i in range(T0, 160)]
    y = np.concatenate([y0.cpu().numpy(), torch.stack(ys, 2).cpu().numpy()], axis=2)
    err = oracle.row_error(y, oracle.dense(inp.q, inp.k, inp.v, inp.params))
    _report(f"prefill+decode {dtype}", err)
    assert err <= TOL[dtype]
    assert state_ok(sess.state_np(), inp.k, inp.v, dtype)


def test_workspace_clear_recovers_a_poisoned_decode_workspace():
    """A decode workspace whose arrival counters hold garbage (as after a call that did not
    finish) gives wrong results; oal_workspace_clear makes it serve exactly like a fresh one."""
    inp = small(22, 2, 14, 2, 40, dtype="bf16")
    a, b = session_for(inp, 64), session_for(inp, 64)
    for sess in (a, b):
        sess.prefill(inp.q[:, :, :32], inp.k[:, :, :32], inp.v[:, :, :32], 64)
    b.dws.fill_(0xA5)                       # poisoned counters and partial sums
    gpq.oal_workspace_clear(b.dws)
    for i in range(32, 40):
        ya = a.decode(inp.q[:, :, i], inp.k[:, :, i], inp.v[:, :, i])
        yb = b.decode(inp.q[:, :, i], inp.k[:, :, i], inp.v[:, :, i])
        assert torch.equal(ya, yb), i
    assert np.array_equal(a.state_np(), b.state_np())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_state_only_prefill(dtype):
    """y = NULL (q = NULL) advances the state exactly as a full prefill does; decode continues."""
    inp = small(23, 2, 14, 2, 200, dtype=dtype)
    T0 = 190
    full = session_for(inp, 64)
    full.prefill(inp.q[:, :, :T0], inp.k[:, :, :T0], inp.v[:, :, :T0], 64)
    only = session_for(inp, 64)
    only.ensure_ws(T0, 64)
    gpq.oal_prefill(only.dims, T0, 64, None, to_dev(inp.k[:, :, :T0], dtype),
                    to_dev(inp.v[:, :, :T0], dtype), only.params, only.state, only.ws, None)
    S_only, S_full = only.state_np(), full.state_np()
    assert np.array_equal(S_only, S_full)
    ys = [only.decode(inp.q[:, :, i], inp.k[:, :, i], inp.v[:, :, i]) for i in range(T0, 200)]
    y = torch.stack(ys, 2).cpu().numpy()
    err = oracle.row_error(y, oracle.dense(inp.q, inp.k, inp.v, inp.params)[:, :, T0:])
    _report(f"state-only prefill + decode {dtype}", err)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_continuation(dtype):
    inp = small(22, 1, 7, 1, 333, dtype=dtype)
    sess = session_for(inp, 128)
    ya = sess.prefill(inp.q[:, :, :150], inp.k[:, :, :150], inp.v[:, :, :150], 128)
    yb = sess.prefill(inp.q[:, :, 150:], inp.k[:, :, 150:], inp.v[:, :, 150:], 64)
    y = np.concatenate([ya.cpu().numpy(), yb.cpu().numpy()], axis=2)
    err = oracle.row_error(y, oracle.dense(inp.q, inp.k, inp.v, inp.params))
    _report(f"prefill continuation {dtype}", err)
    assert err <= TOL[dtype]
    assert state_ok(sess.state_np(), inp.k, inp.v, dtype)


def test_gqa_duplicate_heads_and_determinism():
    inp = small(23, 1, 7, 1, 257, dtype="bf16")
    inp.q[:, 3] = inp.q[:, 1]
    p = inp.params
    p.n_groups[3], p.group_of_dim[3], p.L[3], p.eps[3] = p.n_groups[1], p.group_of_dim[1], p.L[1], p.eps[1]
    y1 = session_for(inp, 128).prefill(inp.q, inp.k, inp.v, 128).cpu().numpy()
    y2 = session_for(inp, 128).prefill(inp.q, inp.k, inp.v, 128).cpu().numpy()
    assert np.array_equal(y1[:, 3], y1[:, 1])
    assert np.array_equal(y1, y2)


def test_causality():
    inp = small(24, 1, 7, 1, 300, dtype="bf16")
    y1 = session_for(inp, 64).prefill(inp.q, inp.k, inp.v, 64).cpu().numpy()
    k2, v2 = inp.k.copy(), inp.v.copy()
    k2[:, :, 170] = round_bf16(k2[:, :, 170] + 1.0)
    v2[:, :, 170] = round_bf16(v2[:, :, 170] - 2.0)
    y2 = session_for(inp, 64).prefill(inp.q, k2, v2, 64).cpu().numpy()
    assert np.array_equal(y1[:, :, :170], y2[:, :, :170])
    assert np.abs(y1[:, :, 170:] - y2[:, :, 170:]).max() > 0


# --- degenerate parameterisations --------------------------------------------------------

def _with_params(inp, mut):
    mut(inp.params)
    return inp


def _g1_taylor(p):
    eps = 1e-3
    c = np.sqrt(1 - eps)
    p.n_groups[:] = 1
    p.group_of_dim[:] = 0
    p.L[:] = 0
    p.L[:, 0, 0] = c
    p.L[:, 1, 0] = 1 / (2 * c)
    p.L[:, 1, 1] = np.sqrt((1 - 2 * eps) / (4 * (1 - eps)))
    p.eps[:] = eps


def _zero_diag(p):
    p.L[:, 1, 1] = 0.0
    p.L[:, 0, 0] = 0.0


def _many_groups():
    rng = np.random.default_rng(31)
    inp = small(31, 1, 2, 1, 150, dtype="bf16", g_hi=2)
    G = 64
    L = np.zeros((2, G + 1, G + 1), np.float32)
    for h in range(2):
        L[h] = np.tril(rng.normal(0, 0.3, (G + 1, G + 1)))
        np.fill_diagonal(L[h], np.abs(np.diag(L[h])) + 0.1)
    inp.params = HeadParams(np.full(2, G, np.int32),
                            np.stack([rng.permutation(64), np.arange(64)]).astype(np.uint8), L,
                            np.full(2, 1e-3, np.float32))
    return inp


@pytest.mark.parametrize("name", ["g1_taylor", "zero_diag", "empty_groups", "g64", "eps0"])
def test_degenerate_params(name):
    if name == "g1_taylor":
        inp = _with_params(small(32, 1, 7, 1, 200, dtype="bf16"), _g1_taylor)
    elif name == "zero_diag":
        inp = _with_params(small(33, 1, 7, 1, 200, dtype="bf16"), _zero_diag)
    elif name == "empty_groups":
        inp = small(34, 1, 4, 1, 200, dtype="bf16", g_hi=12, allow_empty=True)
    elif name == "g64":
        inp = _many_groups()
    else:
        inp = _with_params(small(35, 1, 4, 1, 200, dtype="bf16"), lambda p: p.eps.__setitem__(slice(None), 0.0))
    for chunk in (64, 128):
        y = session_for(inp, chunk).prefill(inp.q, inp.k, inp.v, chunk).cpu().numpy()
        err = oracle.row_error(y, oracle.dense(inp.q, inp.k, inp.v, inp.params))
        _report(f"degenerate {name} C={chunk}", err)
        assert err <= TOL["bf16"]


# --- bulk + small-tail groupings: the tail K-steps of the prefill ---------------------------

def _bulk_tail_params(seed, n_heads, tails, n_tail_groups):
    """Head h: tail dims tails[h] split into n_tail_groups groups (ids 1..), bulk = the rest (id 0)."""
    rng = np.random.default_rng(seed)
    G = 1 + n_tail_groups
    gamma = np.zeros((n_heads, 64), np.uint8)
    for h in range(n_heads):
        t = np.asarray(tails[h], dtype=np.int64)
        lab = np.concatenate([np.arange(1, G), rng.integers(1, G, size=max(0, len(t) - (G - 1)))])
        gamma[h, t] = lab[: len(t)]
    L = np.stack([draw_L(rng, G, G) for _ in range(n_heads)])
    return HeadParams(np.full(n_heads, G, np.int32), gamma, L, np.full(n_heads, 1e-3, np.float32))


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_tail_path_gqa(chunk):
    """Qwen-shaped heads (bulk + 2-5 tail groups), 2 sequences, ragged T, then decode."""
    inp = qwen_like(2, 333 + 3, 41, name="qwen_small")
    T0 = 333
    sess = session_for(inp, chunk)
    y0 = sess.prefill(inp.q[:, :, :T0], inp.k[:, :, :T0], inp.v[:, :, :T0], chunk)
    ys = [sess.decode(inp.q[:, :, i], inp.k[:, :, i], inp.v[:, :, i]) for i in range(T0, T0 + 3)]
    y = np.concatenate([y0.cpu().numpy(), torch.stack(ys, 2).cpu().numpy()], axis=2)
    err = oracle.row_error(y, oracle.dense(inp.q, inp.k, inp.v, inp.params))
    _report(f"tail path qwen-shaped C={chunk}", err)
    assert err <= TOL["bf16"]
    assert state_ok(sess.state_np(), inp.k, inp.v, "bf16")


def test_tail_path_continuation_deterministic():
    """Tail-mode heads continuing from a nonzero state (the tail slots repeat state rows that
    the prefill overwrites): oracle parity, and two runs give identical bits."""
    inp = qwen_like(2, 300, 44, name="qwen_cont")
    outs = []
    for _ in range(2):
        sess = session_for(inp, 128)
        ya = sess.prefill(inp.q[:, :, :130], inp.k[:, :, :130], inp.v[:, :, :130], 128)
        yb = sess.prefill(inp.q[:, :, 130:], inp.k[:, :, 130:], inp.v[:, :, 130:], 128)
        outs.append((np.concatenate([ya.cpu().numpy(), yb.cpu().numpy()], axis=2), sess.state_np()))
    err = oracle.row_error(outs[0][0], oracle.dense(inp.q, inp.k, inp.v, inp.params))
    _report("tail path continuation", err)
    assert err <= TOL["bf16"]
    assert state_ok(outs[0][1], inp.k, inp.v, "bf16")
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tail_path_eight_steps(dtype):
    """18 tail dims per head (171 pairs: with the 65 linear/constant entries, all 8 tail
    K-steps) on one KV head, none on the other."""
    inp = small(42, 1, 8, 2, 290, dtype=dtype)
    tails = [list(range(20, 38))] * 4 + [[]] * 4
    inp.params = _bulk_tail_params(42, 8, tails, 3)
    inp.params.n_groups[4:] = 1
    inp.params.group_of_dim[4:] = 0
    for chunk in (64, 128):
        sess = session_for(inp, chunk)
        y = sess.prefill(inp.q, inp.k, inp.v, chunk).cpu().numpy()
        err = oracle.row_error(y, oracle.dense(inp.q, inp.k, inp.v, inp.params))
        _report(f"tail path 8 steps {dtype} C={chunk}", err)
        assert err <= TOL[dtype]
        assert state_ok(sess.state_np(), inp.k, inp.v, dtype)


def test_tail_union_differs_per_head():
    """Heads of one KV head with different tail dims: the tail list is their union."""
    inp = small(43, 1, 7, 1, 260, dtype="bf16")
    rng = np.random.default_rng(43)
    tails = [sorted(rng.choice(64, size=rng.integers(2, 6), replace=False)) for _ in range(7)]
    inp.params = _bulk_tail_params(43, 7, tails, 2)
    y = session_for(inp, 128).prefill(inp.q, inp.k, inp.v, 128).cpu().numpy()
    err = oracle.row_error(y, oracle.dense(inp.q, inp.k, inp.v, inp.params))
    _report("tail union over heads", err)
    assert err <= TOL["bf16"]


# --- the Qwen2.5-0.5B-shaped workload at full size ----------------------------------------

def test_cfg2_full():
    inp = cfg2()
    ref = oracle.dense(inp.q, inp.k, inp.v, inp.params)
    for chunk in (64, 128, 256):
        sess = session_for(inp, chunk)
        y = sess.prefill(inp.q, inp.k, inp.v, chunk).cpu().numpy()
        err = oracle.row_error(y, ref)
        _report(f"cfg2 T=4096 C={chunk}", err)
        assert err <= TOL["bf16"]
        assert state_ok(sess.state_np(), inp.k, inp.v, "bf16")


def test_prefill_timed_with_timing_events():
    """oal_prefill_timed with the library's fence-free timing events: same output as
    oal_prefill, phases ordered and positive."""
    inp = qwen_like(1, 300, 2, name="timed")
    a, b = session_for(inp), session_for(inp)
    y_ref = a.prefill(inp.q, inp.k, inp.v)
    q, k, v = (to_dev(x, inp.dtype) for x in (inp.q, inp.k, inp.v))
    y = torch.empty_like(y_ref)
    marks = [gpq.TimingEvent() for _ in range(3)]
    b.ensure_ws(300, 128)
    gpq.oal_prefill_timed(b.dims, 300, 128, q, k, v, b.params, b.state, b.ws, y, marks)
    t_scan, t_read = marks[0].elapsed_time(marks[1]), marks[1].elapsed_time(marks[2])
    print(f"[timed] scan {t_scan * 1e3:.1f} us, readout {t_read * 1e3:.1f} us", flush=True)
    assert t_scan > 0 and t_read > 0
    assert torch.equal(y, y_ref)
    assert np.array_equal(a.state_np(), b.state_np())


# --- the other workloads at full size: sampled rows against the oracle ---------------------

def _sample_positions(T, chunk, rng, n_random=6):
    """Sequence start and end, both sides of chunk boundaries, and random positions."""
    pos = {0, 1, chunk - 1, chunk, 2 * chunk - 1, T // 2 - 1, T // 2, T - 2, T - 1}
    pos.update(int(x) for x in rng.integers(0, T, size=n_random))
    return sorted(p for p in pos if 0 <= p < T)


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_cfg3_batch8_sampled(chunk):
    """B=8 x T=4096 (32k tokens), the chunk sizes of the sweep; 16 rows per (sequence, head)
    against the oracle, and the final states of every sequence (one chunk size)."""
    from oal_synth import cfg3
    inp = cfg3()
    B, Hq, Hkv, T, _, _ = inp.dims
    sess = session_for(inp, chunk)
    y = sess.prefill(inp.q, inp.k, inp.v, chunk).cpu().numpy()
    rng = np.random.default_rng(30 + chunk)
    rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in _sample_positions(T, chunk, rng)]
    ref = oracle.dense_rows(inp.q, inp.k, inp.v, inp.params, rows)
    got = np.stack([y[b, h, i] for b, h, i in rows])
    err = oracle.row_error(got, ref)
    _report(f"cfg3 B=8 T=4096 C={chunk} ({len(rows)} sampled rows)", err)
    assert np.isfinite(y).all()
    assert err <= TOL["bf16"]
    if chunk == 128:
        assert state_ok(sess.state_np(), inp.k, inp.v, "bf16")


def test_cfg4_long_context_sampled():
    """T=32768, chunk 128 (the launch configuration of the benchmark's prefill): sampled rows
    across the whole sequence, and the final state."""
    from oal_synth import cfg4
    inp = cfg4()
    B, Hq, Hkv, T, _, _ = inp.dims
    sess = session_for(inp, 128)
    y = sess.prefill(inp.q, inp.k, inp.v, 128).cpu().numpy()
    rng = np.random.default_rng(44)
    rows = [(0, h, i) for h in range(Hq) for i in _sample_positions(T, 128, rng, n_random=10)]
    ref = oracle.dense_rows(inp.q, inp.k, inp.v, inp.params, rows)
    got = np.stack([y[b, h, i] for b, h, i in rows])
    err = oracle.row_error(got, ref)
    _report(f"cfg4 T=32768 ({len(rows)} sampled rows)", err)
    assert np.isfinite(y).all()
    assert err <= TOL["bf16"]
    assert state_ok(sess.state_np(), inp.k, inp.v, "bf16")


def test_cfg5_decode_64_sequences_sampled():
    """The decode workload as the benchmark runs it: 64 sequences whose states are built by a
    state-only prefill of 4096 tokens, then 256 decode steps. Outputs of 8 sequences at
    several steps, and their final states, against the oracle over prefix + steps."""
    from oal_synth import cfg5_prefix, cfg5_steps
    nseq, steps, T0 = 64, 256, 4096
    pre, tok = cfg5_prefix(n_seq=nseq), cfg5_steps(n_seq=nseq, steps=steps)
    sess = Session(nseq, 14, 2, "bf16", pre.params, T0, 128)
    k = to_dev(pre.k, "bf16")
    v = to_dev(pre.v, "bf16")
    gpq.oal_prefill(sess.dims, T0, 128, None, k, v, sess.params, sess.state, sess.ws, None)
    del k, v
    tq, tk, tv = (to_dev(x, "bf16").permute(2, 0, 1, 3).contiguous() for x in (tok.q, tok.k, tok.v))
    ys = []
    for s in range(steps):
        ys.append(sess.decode(tq[s], tk[s], tv[s]))
    y = torch.stack(ys).cpu().numpy()                 # [steps, nseq, 14, 64]
    assert np.isfinite(y).all()
    sel = [0, 9, 18, 27, 36, 45, 54, 63]              # sequences checked against the oracle
    check_steps = [0, 1, 127, 255]
    q_all = np.concatenate([np.zeros_like(pre.q[sel]), tok.q[sel]], axis=2)
    k_all = np.concatenate([pre.k[sel], tok.k[sel]], axis=2)
    v_all = np.concatenate([pre.v[sel], tok.v[sel]], axis=2)
    rows = [(bi, h, T0 + s) for bi in range(len(sel)) for h in range(14) for s in check_steps]
    ref = oracle.dense_rows(q_all, k_all, v_all, pre.params, rows)
    got = np.stack([y[s - T0, sel[bi], h] for bi, h, s in rows])
    err = oracle.row_error(got, ref)
    _report(f"cfg5 decode 64 seqs x 256 steps ({len(rows)} sampled outputs)", err)
    assert err <= TOL["bf16"]
    S = sess.state_np()[sel[:2]]
    assert state_ok(S, k_all[:2], v_all[:2], "bf16")


def test_state_layout_raw_offsets():
    # One decode step from an empty state: H0 = [v;1], H1_r = k_r [v;1], H2_rt = k_r k_t [v;1].
    # Read the raw buffer at the documented offsets (v part [2145, 64] row-major, then the
    # column-64 vector) for each (sequence, KV head) block.
    rng = np.random.default_rng(91)
    B, Hq, Hkv = 2, 4, 2
    q = round_bf16(rng.standard_normal((B, Hq, 64)))
    k = round_bf16(rng.standard_normal((B, Hkv, 64)))
    v = round_bf16(rng.standard_normal((B, Hkv, 64)))
    p = small(91, B, Hq, Hkv, 4).params
    sess = Session(B, Hq, Hkv, "bf16", p)
    sess.decode(q, k, v)
    torch.cuda.synchronize()
    raw = sess.state.view(B, Hkv, gpq.STATE_STRIDE).cpu().numpy().astype(np.float64)
    for b in range(B):
        for kv in range(Hkv):
            blk, kk, vv = raw[b, kv], k[b, kv].astype(np.float64), v[b, kv].astype(np.float64)
            # rows: H0; H1_5; H2_(2,3) at 65 + idx(2,3), idx(r,t) = 64 r - r(r-1)/2 + (t - r)
            for f, mono in ((0, 1.0), (6, kk[5]), (65 + 2 * 64 - 1 + 1, kk[2] * kk[3])):
                for c in (0, 17, 63):
                    assert abs(blk[gpq.state_index(f, c)] - mono * vv[c]) <= 1e-6 * (1 + abs(mono * vv[c]))
                assert abs(blk[gpq.state_index(f, 64)] - mono) <= 1e-6 * (1 + abs(mono))
                assert gpq.state_index(f, 64) == 2145 * 64 + f
            assert np.all(blk[2145 * 65:] == 0.0)
