"""GPU: decode over a state pool (oal_decode_step_indexed) against the plain decode step and
the oracle. The indexed step runs the same kernels on pool blocks chosen per sequence, so its
outputs and updated blocks must equal, bit for bit, those of oal_decode_step on a state buffer
holding the same blocks in batch order; blocks not in the batch stay untouched."""
import numpy as np
import pytest

import oracle
from oal_synth import small, qwen_like

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import Session, to_dev, TOL  # noqa: E402
import grouped_positive_quadratic_amd as gpq  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


def _pool_from_prefix(inp, T0, chunk=128):
    """Pool with one block per sequence of `inp`, filled by a prefill of its first T0 tokens."""
    B, Hq, Hkv, _, _, _ = inp.dims
    pool = Session(B, Hq, Hkv, inp.dtype, inp.params, T0, chunk)
    gpq.oal_prefill(pool.dims, T0, chunk, None, to_dev(inp.k[:, :, :T0], inp.dtype),
                    to_dev(inp.v[:, :, :T0], inp.dtype), pool.params, pool.state, pool.ws, None)
    torch.cuda.synchronize()
    return pool


def _blocks(state, idx, Hkv):
    return state.view(-1, Hkv, gpq.STATE_STRIDE)[idx].clone()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_indexed_decode_matches_plain_decode_and_oracle(dtype):
    P, Hq, Hkv, T0, steps = 6, 4, 2, 150, 3
    inp = small(501, P, Hq, Hkv, T0 + steps, dtype)
    pool = _pool_from_prefix(inp, T0)
    slots_l = [4, 0, 2]
    slots = torch.tensor(slots_l, dtype=torch.int32, device="cuda")
    untouched = [1, 3, 5]
    before = _blocks(pool.state, untouched, Hkv)
    # reference: a plain state buffer holding the three blocks in batch order
    ref = Session(3, Hq, Hkv, dtype, inp.params)
    ref.state.view(3, Hkv, gpq.STATE_STRIDE).copy_(_blocks(pool.state, slots_l, Hkv))
    dims = gpq.make_dims(3, Hq, Hkv, dtype)
    dws = torch.zeros(gpq.oal_decode_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    for st in range(steps):
        i = T0 + st
        q = to_dev(inp.q[slots_l, :, i], dtype)
        k = to_dev(inp.k[slots_l, :, i], dtype)
        v = to_dev(inp.v[slots_l, :, i], dtype)
        y = torch.empty((3, Hq, 64), dtype=torch.float32, device="cuda")
        gpq.oal_decode_step_indexed(dims, slots, P, q, k, v, pool.params, pool.state, dws, y)
        y_ref = ref.decode(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"step {st}: indexed and plain decode differ"
        rows = [(j, h, i) for j in range(3) for h in range(Hq)]
        want = oracle.dense_rows(inp.q[slots_l], inp.k[slots_l], inp.v[slots_l], inp.params, rows)
        err = oracle.row_error(y.cpu().numpy().reshape(-1, 64), want)
        print(f"[parity] indexed decode {dtype} step {st}: err={err:.2e}", flush=True)
        assert err <= TOL[dtype]
    assert torch.equal(_blocks(pool.state, slots_l, Hkv), ref.state.view(3, Hkv, gpq.STATE_STRIDE))
    assert torch.equal(_blocks(pool.state, untouched, Hkv), before)


def test_indexed_decode_slot_outside_pool_gives_nan_and_touches_nothing():
    P, Hq, Hkv, T0 = 3, 4, 2, 64
    inp = small(502, P, Hq, Hkv, T0 + 1, "bf16")
    pool = _pool_from_prefix(inp, T0)
    before = pool.state.clone()
    slots_l = [1, 7, -1]
    slots = torch.tensor(slots_l, dtype=torch.int32, device="cuda")
    dims = gpq.make_dims(3, Hq, Hkv, "bf16")
    dws = torch.zeros(gpq.oal_decode_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    src = [1, 0, 2]       # token rows fed to the three batch positions
    q, k, v = (to_dev(x[src, :, T0], "bf16") for x in (inp.q, inp.k, inp.v))
    y = torch.empty((3, Hq, 64), dtype=torch.float32, device="cuda")
    gpq.oal_decode_step_indexed(dims, slots, P, q, k, v, pool.params, pool.state, dws, y)
    torch.cuda.synchronize()
    yc = y.cpu().numpy()
    assert np.isnan(yc[1]).all() and np.isnan(yc[2]).all() and np.isfinite(yc[0]).all()
    blocks = pool.state.view(P, Hkv, gpq.STATE_STRIDE)
    assert torch.equal(blocks[[0, 2]], before.view(P, Hkv, gpq.STATE_STRIDE)[[0, 2]])
    want = oracle.dense_rows(inp.q[[1]], inp.k[[1]], inp.v[[1]], inp.params, [(0, h, T0) for h in range(Hq)])
    assert oracle.row_error(yc[0], want) <= TOL["bf16"]
    assert int(dws[:256].count_nonzero()) == 0      # counters returned to zero


def test_indexed_decode_serving_shape_bitwise():
    # 64 active sequences over a pool of 96 blocks (14q/2kv, bf16), slots in shuffled order
    P, B, T0 = 96, 64, 256
    inp = qwen_like(P, T0 + 1, 7, name="pool")
    pool = _pool_from_prefix(inp, T0)
    rng = np.random.default_rng(8)
    slots_l = [int(x) for x in rng.permutation(P)[:B]]
    slots = torch.tensor(slots_l, dtype=torch.int32, device="cuda")
    others = sorted(set(range(P)) - set(slots_l))
    before = _blocks(pool.state, others, 2)
    ref = Session(B, 14, 2, "bf16", inp.params)
    ref.state.view(B, 2, gpq.STATE_STRIDE).copy_(_blocks(pool.state, slots_l, 2))
    q, k, v = (to_dev(x[slots_l, :, T0], "bf16") for x in (inp.q, inp.k, inp.v))
    dims = gpq.make_dims(B, 14, 2, "bf16")
    dws = torch.zeros(gpq.oal_decode_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    y = torch.empty((B, 14, 64), dtype=torch.float32, device="cuda")
    gpq.oal_decode_step_indexed(dims, slots, P, q, k, v, pool.params, pool.state, dws, y)
    y_ref = ref.decode(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(_blocks(pool.state, slots_l, 2), ref.state.view(B, 2, gpq.STATE_STRIDE))
    assert torch.equal(_blocks(pool.state, others, 2), before)
    rows = [(j, h, T0) for j in (0, 31, 63) for h in (0, 7, 13)]
    sel = [slots_l[j] for j in (0, 31, 63)]
    want = oracle.dense_rows(inp.q[sel], inp.k[sel], inp.v[sel], inp.params,
                             [(n, h, T0) for n in range(3) for h in (0, 7, 13)])
    got = np.stack([y[j, h].cpu().numpy() for j, h, _ in rows])
    assert oracle.row_error(got, want) <= TOL["bf16"]


# ---------------------------------------------------------------------------------------
# ragged prefill (oal_prefill_varlen): sequence b of a batch padded to T takes lengths[b] tokens

def _varlen_run(inp, lengths, chunk, sentinel=7.0):
    B, Hq, Hkv, T, _, _ = inp.dims
    sess = Session(B, Hq, Hkv, inp.dtype, inp.params, T, chunk)
    lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    y = torch.full((B, Hq, T, 64), sentinel, dtype=torch.float32, device="cuda")
    gpq.oal_prefill_varlen(sess.dims, T, lens, chunk, to_dev(inp.q, inp.dtype), to_dev(inp.k, inp.dtype),
                           to_dev(inp.v, inp.dtype), sess.params, sess.state, sess.ws, y)
    torch.cuda.synchronize()
    return sess, y.cpu().numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [64, 128])
def test_varlen_prefill_small(dtype, chunk):
    lengths = [300, 129, 1, 0, 64]
    inp = small(601, len(lengths), 4, 2, 300, dtype)
    sess, y = _varlen_run(inp, lengths, chunk)
    S = sess.state_np()
    from gpu_util import state_ok
    for b, L in enumerate(lengths):
        assert np.all(y[b, :, L:] == 7.0), f"sequence {b}: rows past its length were written"
        if L == 0:
            assert np.all(S[b] == 0.0)
            continue
        sl = slice(b, b + 1)
        ref = oracle.dense(inp.q[sl, :, :L], inp.k[sl, :, :L], inp.v[sl, :, :L], inp.params)
        err = oracle.row_error(y[sl, :, :L], ref)
        print(f"[parity] varlen {dtype} C={chunk} seq {b} len {L}: err={err:.2e}", flush=True)
        assert err <= TOL[dtype]
        assert state_ok(S[sl], inp.k[sl, :, :L], inp.v[sl, :, :L], dtype)


def test_varlen_full_lengths_equal_plain_prefill_and_clamping():
    inp = small(602, 3, 14, 2, 257, "bf16")
    B, Hq, Hkv, T, _, _ = inp.dims
    # lengths above T are clamped to T, negative ones to 0
    sess, y = _varlen_run(inp, [T, T + 50, -3], 128)
    plain = Session(B, Hq, Hkv, "bf16", inp.params, T, 128)
    y_plain = plain.prefill(inp.q, inp.k, inp.v, 128).cpu().numpy()
    assert np.array_equal(y[:2], y_plain[:2])
    S, S_plain = sess.state_np(), plain.state_np()
    assert np.array_equal(S[:2], S_plain[:2]) and np.all(S[2] == 0.0) and np.all(y[2] == 7.0)


def test_varlen_then_decode():
    lengths = [200, 77]
    inp = small(603, 2, 4, 2, 201, "bf16")
    sess, _ = _varlen_run(inp, lengths, 128)
    # next token of each sequence = its token at position lengths[b]
    q = to_dev(np.stack([inp.q[b, :, L] for b, L in enumerate(lengths)]), "bf16")
    k = to_dev(np.stack([inp.k[b, :, L] for b, L in enumerate(lengths)]), "bf16")
    v = to_dev(np.stack([inp.v[b, :, L] for b, L in enumerate(lengths)]), "bf16")
    yd = sess.decode(q, k, v).cpu().numpy()
    for b, L in enumerate(lengths):
        sl = slice(b, b + 1)
        want = oracle.dense_rows(inp.q[sl, :, :L + 1], inp.k[sl, :, :L + 1], inp.v[sl, :, :L + 1],
                                 inp.params, [(0, h, L) for h in range(4)])
        assert oracle.row_error(yd[b], want) <= TOL["bf16"]


def test_varlen_batch8_4096_sampled():
    # ragged serving batch at the layer's full size: 8 sequences padded to 4096 tokens
    inp = qwen_like(8, 4096, 11, name="ragged", per_seq_seeds=[1100 + b for b in range(8)])
    lengths = [4096, 1, 4095, 2048, 129, 3000, 64, 1777]
    sess, y = _varlen_run(inp, lengths, 128)
    rng = np.random.default_rng(12)
    for b, L in enumerate(lengths):
        assert np.all(y[b, :, L:] == 7.0)
        pos = sorted({0, L - 1, *rng.integers(0, L, size=3).tolist()})
        heads = (0, 7, 13)
        sl = slice(b, b + 1)
        want = oracle.dense_rows(inp.q[sl, :, :L], inp.k[sl, :, :L], inp.v[sl, :, :L], inp.params,
                                 [(0, h, i) for h in heads for i in pos])
        got = np.stack([y[b, h, i] for h in heads for i in pos])
        err = oracle.row_error(got, want)
        print(f"[parity] varlen B=8x4096 seq {b} len {L}: err={err:.2e}", flush=True)
        assert err <= TOL["bf16"]
    from gpu_util import state_ok
    S = sess.state_np()
    for b in (3, 6):
        L = lengths[b]
        assert state_ok(S[b:b + 1], inp.k[b:b + 1, :, :L], inp.v[b:b + 1, :, :L], "bf16")


# ---------------------------------------------------------------------------------------
# packed ragged prefill (oal_prefill_packed): sequences concatenated along the token axis

def _pack(x, lengths, starts, total):
    """[B, H, T, d] padded -> [H, total, d] packed at the given starts."""
    B, H, T, d = x.shape
    out = np.zeros((H, total, d), dtype=x.dtype)
    for b, (L, s0) in enumerate(zip(lengths, starts)):
        out[:, s0:s0 + L] = x[b, :, :L]
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_packed_prefill_equals_varlen(dtype):
    lengths = [300, 129, 1, 0, 64]
    B, T = len(lengths), 300
    inp = small(701, B, 4, 2, T, dtype)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).tolist()
    total = int(sum(lengths)) + 37            # 37 trailing rows that belong to no sequence
    cu = torch.tensor(starts + [sum(lengths)], dtype=torch.int32, device="cuda")
    qp, kp, vp = (to_dev(_pack(x, lengths, starts, total), dtype) for x in (inp.q, inp.k, inp.v))
    sess = Session(B, 4, 2, dtype, inp.params, T, 128)
    yp = torch.full((4, total, 64), 7.0, dtype=torch.float32, device="cuda")
    gpq.oal_prefill_packed(sess.dims, T, cu, total, 128, qp, kp, vp, sess.params, sess.state, sess.ws, yp)
    torch.cuda.synchronize()
    ref_sess, y_ref = _varlen_run(inp, lengths, 128)
    ypn = yp.cpu().numpy()
    for b, (L, s0) in enumerate(zip(lengths, starts)):
        assert np.array_equal(ypn[:, s0:s0 + L], y_ref[b, :, :L]), f"sequence {b} differs from the padded run"
    assert np.all(ypn[:, sum(lengths):] == 7.0), "rows outside every sequence were written"
    assert torch.equal(sess.state, ref_sess.state)


def test_packed_prefill_inconsistent_offsets_are_clamped():
    # offsets that run backwards or past the end give empty or shortened sequences, never an
    # access outside the packed tensors: cu = [30, 30, 20, 500] over 80 rows gives sequence 0
    # empty, sequence 1 empty (negative length), sequence 2 rows 20..79 (its length 480 cut to
    # min(T, 80 - 20) = 60)
    B, T, total = 3, 64, 80
    inp = small(702, B, 2, 1, T, "bf16")
    cu = torch.tensor([30, 30, 20, 500], dtype=torch.int32, device="cuda")
    rows = lambda x: np.concatenate([np.zeros_like(x[2, :, :20]), x[2, :, :60]], axis=1)
    q, k, v = (to_dev(rows(x), "bf16") for x in (inp.q, inp.k, inp.v))
    sess = Session(B, 2, 1, "bf16", inp.params, T, 64)
    y = torch.full((2, total, 64), 7.0, dtype=torch.float32, device="cuda")
    gpq.oal_prefill_packed(sess.dims, T, cu, total, 64, q, k, v, sess.params, sess.state, sess.ws, y)
    torch.cuda.synchronize()
    S = sess.state_np()
    assert np.all(S[0] == 0.0) and np.all(S[1] == 0.0)
    yn = y.cpu().numpy()
    assert np.all(yn[:, :20] == 7.0)
    ref = oracle.dense(inp.q[2:3, :, :60], inp.k[2:3, :, :60], inp.v[2:3, :, :60], inp.params)
    assert oracle.row_error(yn[None, :, 20:80], ref) <= TOL["bf16"]
    from gpu_util import state_ok
    assert state_ok(S[2:3], inp.k[2:3, :, :60], inp.v[2:3, :, :60], "bf16")


def test_packed_prefill_serving_shape():
    # 8 sequences of mixed lengths packed into 14q/2kv tensors, B = 8, T = 4096
    lengths = [4096, 1, 4095, 2048, 129, 3000, 64, 1777]
    inp = qwen_like(8, 4096, 11, name="ragged", per_seq_seeds=[1100 + b for b in range(8)])
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).tolist()
    total = int(sum(lengths))
    cu = torch.tensor(starts + [total], dtype=torch.int32, device="cuda")
    qp, kp, vp = (to_dev(_pack(x, lengths, starts, total), "bf16") for x in (inp.q, inp.k, inp.v))
    sess = Session(8, 14, 2, "bf16", inp.params, 4096, 128)
    yp = torch.empty((14, total, 64), dtype=torch.float32, device="cuda")
    gpq.oal_prefill_packed(sess.dims, 4096, cu, total, 128, qp, kp, vp, sess.params, sess.state, sess.ws, yp)
    torch.cuda.synchronize()
    ypn = yp.cpu().numpy()
    rng = np.random.default_rng(13)
    for b, (L, s0) in enumerate(zip(lengths, starts)):
        pos = sorted({0, L - 1, *rng.integers(0, L, size=2).tolist()})
        heads = (0, 13)
        sl = slice(b, b + 1)
        want = oracle.dense_rows(inp.q[sl, :, :L], inp.k[sl, :, :L], inp.v[sl, :, :L], inp.params,
                                 [(0, h, i) for h in heads for i in pos])
        got = np.stack([ypn[h, s0 + i] for h in heads for i in pos])
        assert oracle.row_error(got, want) <= TOL["bf16"]
