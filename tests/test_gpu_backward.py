"""GPU parity of the prefill backward (oal_prefill_backward) against the oracle backward.

The oracle differentiates the dense O(T^2) definition in fp64 (pinned by finite differences,
the L = 0 closed form and the scale invariance in the CPU suite); the library runs the
chunked linear-time form in fp32 on the same (dtype-exact) inputs. The error measure is
blockwise: per (sequence, head) slice of dq, dk or dv, max |x - x*| / max |x*|.
"""
import numpy as np
import pytest

import oracle
from oal_synth import small, HeadParams

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import to_dev  # noqa: E402
import grouped_positive_quadratic_amd as gpq  # noqa: E402

# fp32 arithmetic throughout (the inputs are exact in fp32 for both dtypes): the bound of
# the fp32 forward tests. Measured errors are below 2e-6.
BWD_TOL = 1e-5
# dL and deps sum dkappa_ij sbar sbar^T over every causal pair, and each query's dkappa row is
# orthogonal to its kappa row (sum_j kappa_ij dkappa_ij = g_i . u_i = 0): the result is a small
# difference of large terms, so the same fp32 roundings give a larger error relative to it.
# Measured up to 1.1e-4 over these cases; the bound keeps a margin of about 9 over that.
COEF_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


def run_backward(inp, dy, chunk, coef=True):
    B, Hq, Hkv, T, _, _ = inp.dims
    dims = gpq.make_dims(B, Hq, Hkv, inp.dtype)
    hp = gpq.HeadParamsC.from_params(inp.params)
    params = torch.empty(max(gpq.oal_params_bytes(dims), 16), dtype=torch.uint8, device="cuda")
    gpq.oal_state_init(dims, hp, params, None)
    q, k, v = (to_dev(x, inp.dtype) for x in (inp.q, inp.k, inp.v))
    dyd = torch.from_numpy(np.ascontiguousarray(dy, np.float32)).cuda()
    ws = torch.empty(max(gpq.oal_prefill_backward_workspace_bytes(dims, T, chunk), 16), dtype=torch.uint8,
                     device="cuda")
    dq = torch.full((B, Hq, T, 64), np.nan, dtype=torch.float32, device="cuda")
    dk = torch.full((B, Hkv, T, 64), np.nan, dtype=torch.float32, device="cuda")
    dv = torch.full((B, Hkv, T, 64), np.nan, dtype=torch.float32, device="cuda")
    dL = torch.full((Hq, 65, 65), np.nan, dtype=torch.float32, device="cuda") if coef else None
    deps = torch.full((Hq,), np.nan, dtype=torch.float32, device="cuda") if coef else None
    gpq.oal_prefill_backward(dims, T, chunk, q, k, v, dyd, params, ws, dq, dk, dv, dL, deps)
    torch.cuda.synchronize()
    out = (dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy())
    return out + ((dL.cpu().numpy(), deps.cpu().numpy()) if coef else ())


def coef_err(dL, deps, rL, reps):
    """Per head: max(|dL - dL*|, |deps - deps*|) / max(|dL*|, |deps*|); dL [Hq, 65, 65] against
    the oracle's [Hq, g+1, g+1], everything outside the oracle's block must be exactly 0."""
    gm1 = rL.shape[1]
    assert np.all(dL[:, gm1:, :] == 0.0) and np.all(dL[:, :, gm1:] == 0.0)
    a = dL[:, :gm1, :gm1].astype(np.float64)
    num = np.maximum(np.abs(a - rL).reshape(len(rL), -1).max(-1), np.abs(deps - reps))
    den = np.maximum(np.abs(rL).reshape(len(rL), -1).max(-1), np.abs(reps))
    return float((num / np.maximum(den, 1e-300)).max())


def slice_err(x, ref):
    """max over (sequence, head) slices of max |x - ref| / max |ref|; a slice whose reference
    is below 1e-3 of the tensor's largest entry is measured against that 1e-3 instead."""
    x = np.asarray(x, np.float64)
    num = np.abs(x - ref).reshape(ref.shape[0], ref.shape[1], -1).max(-1)
    den = np.abs(ref).reshape(ref.shape[0], ref.shape[1], -1).max(-1)
    return float((num / np.maximum(den, max(1e-3 * den.max(), 1e-300))).max())


def check(inp, chunk, seed, tol=BWD_TOL, name=""):
    B, Hq, Hkv, T, _, _ = inp.dims
    dy = np.random.default_rng(seed).normal(0.0, 1.0, (B, Hq, T, 64)).astype(np.float32)
    dq, dk, dv, dL, deps = run_backward(inp, dy, chunk)
    rq, rk, rv, rL, reps = oracle.backward(inp.q, inp.k, inp.v, inp.params, dy)
    ec = coef_err(dL, deps, rL, reps) if T > 1 else 0.0
    if T == 1:
        # one token: y = v_0 whatever q and k are, so dq = dk = 0; both sides hold rounding
        # residue of dkappa = g . [v; 1] (a difference of two equal terms)
        scale = np.abs(dy).max() * np.abs(inp.v).max()
        assert np.abs(rq).max() <= 1e-12 * scale and np.abs(rk).max() <= 1e-12 * scale
        assert np.abs(dq).max() <= 1e-5 * scale and np.abs(dk).max() <= 1e-5 * scale
        rq, rk = dq, dk
        # the coefficient gradients are 2 dkappa sbar sbar^T L and dkappa: residue as well,
        # |sbar_g| <= 64 max|q| max|k| / 8
        sb = 1.0 + 8.0 * np.abs(inp.q).max() * np.abs(inp.k).max()
        bound = 1e-5 * scale * 2.0 * sb * sb * max(1.0, np.abs(inp.params.L).max())
        assert np.abs(rL).max() <= 1e-9 * bound and np.abs(dL).max() <= bound
        assert np.abs(deps).max() <= 1e-5 * scale
        ec = 0.0
    e = (slice_err(dq, rq), slice_err(dk, rk), slice_err(dv, rv))
    print(f"[parity] backward {name} {inp.dims[:4]} C={chunk} {inp.dtype}: "
          f"dq={e[0]:.2e} dk={e[1]:.2e} dv={e[2]:.2e} dL,deps={ec:.2e} tol={tol:.0e}/{COEF_TOL:.0e}",
          flush=True)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    assert max(e) <= tol and ec <= COEF_TOL
    return dq, dk, dv


SMALL = [  # seed, B, Hq, Hkv, T, chunk: ragged tails, one token, several chunks, n_rep 1/4/7/16
    (41, 1, 7, 1, 200, 64),
    (42, 2, 4, 2, 77, 128),
    (43, 1, 2, 1, 1, 64),
    (44, 1, 8, 1, 300, 256),
    (45, 2, 3, 1, 64, 64),
    (46, 1, 14, 2, 330, 64),
    (47, 1, 16, 1, 130, 128),
    (48, 1, 3, 3, 150, 64),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", SMALL, ids=[f"s{c[0]}" for c in SMALL])
def test_backward_small(case, dtype):
    seed, B, Hq, Hkv, T, chunk = case
    check(small(seed, B, Hq, Hkv, T, dtype), chunk, seed + 1000)


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_backward_chunk_sizes_agree(chunk):
    """Same inputs at every chunk size: each against the oracle."""
    check(small(51, 1, 7, 1, 260, "bf16"), chunk, 51)


@pytest.mark.parametrize("chunk", [64, 128])
def test_backward_many_groups(chunk):
    """64 groups (one per dim): the z-terms run in several register blocks. T = 300 spans
    several chunks of both sizes and a ragged tail."""
    rng = np.random.default_rng(52)
    inp = small(52, 1, 2, 1, 300, dtype="bf16", g_hi=2)
    G = 64
    L = np.zeros((2, G + 1, G + 1), np.float32)
    for h in range(2):
        L[h] = np.tril(rng.normal(0, 0.3, (G + 1, G + 1)))
        np.fill_diagonal(L[h], np.abs(np.diag(L[h])) + 0.1)
    inp.params = HeadParams(np.full(2, G, np.int32),
                            np.stack([rng.permutation(64), np.arange(64)]).astype(np.uint8), L,
                            np.full(2, 1e-3, np.float32))
    check(inp, chunk, 52, name="g64")


def test_backward_l_zero_closed_form():
    """L = 0: kappa = eps, y_i is the prefix mean of v, so dq = dk = 0 and
    dv_j = sum_{i >= j} dy_i / (i + 1) summed over the query heads of the KV head."""
    inp = small(53, 1, 4, 1, 150, "bf16")
    inp.params.L[:] = 0.0
    inp.params.eps[:] = 0.5
    B, Hq, Hkv, T, _, _ = inp.dims
    dy = np.random.default_rng(53).normal(0.0, 1.0, (B, Hq, T, 64)).astype(np.float32)
    dq, dk, dv, dL, deps = run_backward(inp, dy, 64)
    assert np.all(dq == 0.0) and np.all(dk == 0.0) and np.all(dL == 0.0)
    # deps = sum of dkappa over all pairs = sum_i g_i . u_i = sum_i (dy.y - dy.y) / den = 0
    assert np.abs(deps).max() <= 1e-5 * np.abs(dy).sum(axis=(0, 2, 3)).max()
    w = dy.astype(np.float64) / np.arange(1, T + 1)[None, None, :, None]
    ref = np.flip(np.cumsum(np.flip(w, 2), 2), 2).sum(1, keepdims=True)
    assert slice_err(dv, ref) <= BWD_TOL


def test_backward_deterministic():
    inp = small(54, 1, 7, 1, 200, "bf16")
    dy = np.random.default_rng(54).normal(0.0, 1.0, (1, 7, 200, 64)).astype(np.float32)
    a = run_backward(inp, dy, 64)
    b = run_backward(inp, dy, 64)
    assert len(a) == 5
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_matches_forward_directional_derivative():
    """<dq, e_q> + <dk, e_k> + <dv, e_v> equals the derivative of sum(dy * y) along
    (e_q, e_k, e_v), y being the dense definition in fp64 (central difference, step 1e-3)."""
    inp = small(55, 1, 4, 1, 96, "f32")
    B, Hq, Hkv, T, _, _ = inp.dims
    rng = np.random.default_rng(55)
    dy = rng.normal(0.0, 1.0, (B, Hq, T, 64)).astype(np.float32)
    dq, dk, dv = run_backward(inp, dy, 64, coef=False)
    eq, ek, ev = (rng.normal(0.0, 1.0, x.shape).astype(np.float64) for x in (inp.q, inp.k, inp.v))
    pred = float((dq * eq).sum() + (dk * ek).sum() + (dv * ev).sum())
    h = 1e-3

    def loss(s):
        y = oracle.dense(inp.q + s * eq, inp.k + s * ek, inp.v + s * ev, inp.params)
        return float((dy * y).sum())

    fd = (loss(h) - loss(-h)) / (2 * h)
    print(f"[parity] backward directional: pred={pred:.6e} fd={fd:.6e}", flush=True)
    assert abs(pred - fd) <= 1e-3 * max(1.0, abs(fd))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_coefficient_scale_invariance(dtype):
    """y is unchanged under (L, eps) -> (a L, a^2 eps), so d/da at a = 1 vanishes:
    sum L o dL + 2 eps deps = 0 per head (checked on the library's own gradients)."""
    inp = small(56, 1, 7, 1, 200, dtype)
    B, Hq, Hkv, T, _, _ = inp.dims
    dy = np.random.default_rng(56).normal(0.0, 1.0, (B, Hq, T, 64)).astype(np.float32)
    _, _, _, dL, deps = run_backward(inp, dy, 64)
    p = inp.params
    for h in range(Hq):
        G = int(p.n_groups[h])
        Lh = np.tril(p.L[h][: G + 1, : G + 1]).astype(np.float64)
        terms = Lh * dL[h, : G + 1, : G + 1]
        total = terms.sum() + 2.0 * float(p.eps[h]) * float(deps[h])
        scale = np.abs(terms).sum() + 2.0 * abs(float(p.eps[h]) * float(deps[h]))
        assert abs(total) <= 1e-4 * scale, (h, total, scale)


def test_backward_empty_and_validation():
    dims = gpq.make_dims(1, 2, 1, "f32")
    x = torch.zeros(16, dtype=torch.float32, device="cuda")
    ws = torch.zeros(16, dtype=torch.uint8, device="cuda")
    # T = 0: no-op
    gpq.oal_prefill_backward(dims, 0, 64, x, x, x, x, ws, ws, x, x, x)
    with pytest.raises(gpq.OALError, match="OAL_E_UNSUPPORTED"):
        gpq.oal_prefill_backward(dims, 10, 32, x, x, x, x, ws, ws, x, x, x)


def _to_state_buffer(S):
    """[B, Hkv, 2145, 65] states (the oracle's layout) -> the library's state buffer (fp32):
    per block the [2145, 64] v part, then column 64, then zero padding."""
    B, Hkv = S.shape[:2]
    blk = np.zeros((B, Hkv, gpq.STATE_STRIDE), np.float32)
    blk[..., : 2145 * 64] = S[..., :64].reshape(B, Hkv, -1)
    blk[..., 2145 * 64: 2145 * 65] = S[..., 64]
    return torch.from_numpy(blk.reshape(-1)).cuda()


def _psi_pairs():
    """(a, b) of the quadratic state rows 65.. (a <= b, row-major upper triangle)."""
    return np.array([(a, b) for a in range(64) for b in range(a, 64)], np.int64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [64, 128])
def test_backward_from_a_prefix_state(dtype, chunk):
    """Backward of a prefill that continues from the state of a prefix (the state built by the
    oracle from the prefix tokens). Reference: the oracle's dense backward over prefix + new
    tokens with dy = 0 on the prefix rows. dq, dk, dv of the new tokens and dL, deps match it;
    the incoming-state gradient dS0 must give, by the chain rule through
    S0 = sum_j psi(k_j) [v_j; 1]^T, the oracle's dv_j = (psi(k_j)^T dS0)[0:64] and
    dk_j = Jpsi(k_j)^T (dS0 [v_j; 1]) of every prefix token j."""
    T0, T1 = 150, 200
    full = small(61, 2, 4, 2, T0 + T1, dtype=dtype)
    B, Hq, Hkv = 2, 4, 2
    qp, kp, vp = (x[:, :, :T0] for x in (full.q, full.k, full.v))
    qn, kn, vn = (np.ascontiguousarray(x[:, :, T0:]) for x in (full.q, full.k, full.v))
    S0 = oracle.state(kp, vp)                                   # [B, Hkv, 2145, 65], fp64
    dims = gpq.make_dims(B, Hq, Hkv, dtype)
    params = torch.empty(max(gpq.oal_params_bytes(dims), 16), dtype=torch.uint8, device="cuda")
    gpq.oal_state_init(dims, gpq.HeadParamsC.from_params(full.params), params, None)
    state_in = _to_state_buffer(S0)
    q, k, v = (to_dev(x, dtype) for x in (qn, kn, vn))
    dy = np.random.default_rng(62).normal(0.0, 1.0, (B, Hq, T1, 64)).astype(np.float32)
    ws = torch.empty(gpq.oal_prefill_backward_workspace_bytes(dims, T1, chunk), dtype=torch.uint8, device="cuda")
    dq = torch.full((B, Hq, T1, 64), np.nan, dtype=torch.float32, device="cuda")
    dk = torch.full((B, Hkv, T1, 64), np.nan, dtype=torch.float32, device="cuda")
    dv = torch.full_like(dk, np.nan)
    dL = torch.full((Hq, 65, 65), np.nan, dtype=torch.float32, device="cuda")
    deps = torch.full((Hq,), np.nan, dtype=torch.float32, device="cuda")
    dS0 = torch.zeros_like(state_in)
    gpq.oal_prefill_backward(dims, T1, chunk, q, k, v, torch.from_numpy(dy).cuda(), params, ws, dq, dk, dv,
                             dL, deps, state_in=state_in, dstate_in=dS0)
    torch.cuda.synchronize()
    dy_full = np.concatenate([np.zeros((B, Hq, T0, 64), np.float32), dy], axis=2)
    rq, rk, rv, rL, reps = oracle.backward(full.q, full.k, full.v, full.params, dy_full)
    e = (slice_err(dq.cpu().numpy(), rq[:, :, T0:]), slice_err(dk.cpu().numpy(), rk[:, :, T0:]),
         slice_err(dv.cpu().numpy(), rv[:, :, T0:]))
    ec = coef_err(dL.cpu().numpy(), deps.cpu().numpy(), rL, reps)
    # chain rule for the prefix tokens
    G = gpq.state_view(dS0, B, Hkv).cpu().numpy().astype(np.float64)   # [B, Hkv, 2145, 65]
    pr = _psi_pairs()
    kp64, vp64 = np.asarray(kp, np.float64), np.asarray(vp, np.float64)
    psi = np.concatenate([np.ones(kp64.shape[:3] + (1,)), kp64, kp64[..., pr[:, 0]] * kp64[..., pr[:, 1]]], -1)
    pv = np.einsum("bhjf,bhfc->bhjc", psi, G[..., :64])              # predicted dv of prefix tokens
    w = np.einsum("bhfc,bhjc->bhjf", G[..., :64], vp64) + G[..., 64][:, :, None, :]
    pk = w[..., 1:65].copy()                                          # linear rows: d k_r / d k_r = 1
    wq = w[..., 65:]                                                  # pair rows: d (k_a k_b)
    for f, (a, b) in enumerate(pr):
        pk[..., a] += wq[..., f] * kp64[..., b]
        pk[..., b] += wq[..., f] * kp64[..., a]
    es = (slice_err(pv, rv[:, :, :T0]), slice_err(pk, rk[:, :, :T0]))
    print(f"[parity] backward from a {T0}-token prefix state, {T1} tokens C={chunk} {dtype}: "
          f"dq={e[0]:.2e} dk={e[1]:.2e} dv={e[2]:.2e} dL,deps={ec:.2e} dS0->dv={es[0]:.2e} dS0->dk={es[1]:.2e}",
          flush=True)
    assert max(e) <= BWD_TOL and ec <= COEF_TOL
    assert max(es) <= BWD_TOL
