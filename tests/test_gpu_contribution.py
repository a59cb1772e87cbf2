"""GPU parity of the causal contribution scores chi (oal_contribution) against the oracle.

chi is a sum of non-negative terms, so its fp32 evaluation has an elementwise relative
error of at most m * 2^-24 (first order), m being the longest chain of roundings that
reaches an output: 8 rows summed in a lane, a 4-step scan over lanes, the product with
|q|, 8 rows and a 3-step reduction for the chunk partial, then the fold over chunks --
about two roundings per chunk of the longest of four chunk runs -- the fold of the four
runs, the scale and its own rounding. The tests take m = 48 + 2 * ceil(chunks / 4) (+ batch
for the prompt mean), with chunks = ceil(T / 64). Inputs are exact in fp32 (bf16 or fp32
values), so the oracle (fp64) sees the same numbers.
"""
import math

import numpy as np
import pytest

import oracle
from oal_synth import small, cfg2, cfg3, cfg4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import to_dev  # noqa: E402
import grouped_positive_quadratic_amd as gpq  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


def chi_tol(T, B=0):
    chunks = -(-T // 64)
    return (48 + 2 * -(-chunks // 4) + B) * 2.0 ** -24


def rel_err(x, ref):
    x = np.asarray(x, np.float64)
    return float((np.abs(x - ref) / np.abs(ref)).max())


def run_chi(q, k, dtype, with_mean=True, ws_fill=None):
    B, Hq, T, _ = q.shape
    Hkv = k.shape[1]
    dims = gpq.make_dims(B, Hq, Hkv, dtype)
    qd = q if isinstance(q, torch.Tensor) else to_dev(q, dtype)
    kd = k if isinstance(k, torch.Tensor) else to_dev(k, dtype)
    ws = torch.zeros(max(gpq.oal_contribution_workspace_bytes(dims, T), 16), dtype=torch.uint8,
                     device="cuda")
    if ws_fill is not None:
        # only the arrival counters (a 128-byte line per (prompt, head) and per head) must start at zero
        cbytes = -(-(B * Hq + Hq) * 128 // 256) * 256
        ws[cbytes:].view(torch.float32).fill_(ws_fill)
    chi = torch.empty((B, Hq, 64), dtype=torch.float32, device="cuda")
    chi_mean = torch.empty((Hq, 64), dtype=torch.float32, device="cuda") if with_mean else None
    gpq.oal_contribution(dims, T, qd, kd, ws, chi, chi_mean)
    torch.cuda.synchronize()
    return chi.cpu().numpy(), (chi_mean.cpu().numpy() if with_mean else None)


SMALL = [  # (B, Hq, Hkv, T): ragged tails, single token, n_rep 1 / 5 / 7 / 16
    (2, 4, 2, 200), (1, 2, 2, 1), (3, 14, 2, 64), (1, 5, 1, 65), (2, 16, 1, 129),
    (1, 3, 3, 300), (2, 7, 1, 63),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SMALL, ids=[f"B{b}_H{h}x{kv}_T{t}" for b, h, kv, t in SMALL])
def test_contribution_small(shape, dtype):
    B, Hq, Hkv, T = shape
    inp = small(700 + T, B, Hq, Hkv, T, dtype)
    chi, chi_mean = run_chi(inp.q, inp.k, dtype)
    ref, ref_mean = oracle.contribution(inp.q, inp.k)
    e, em = rel_err(chi, ref), rel_err(chi_mean, ref_mean)
    print(f"[parity] chi small {shape} {dtype}: err={e:.2e} mean={em:.2e} tol={chi_tol(T):.2e}",
          flush=True)
    assert e <= chi_tol(T) and em <= chi_tol(T, B)


def test_contribution_workspace_reuse_and_repeat_bitwise():
    # one workspace serves successive calls of one shape (new data each time): the partial
    # sums may hold anything on entry and the counters come back to zero after each call
    dims = gpq.make_dims(3, 14, 2, "bf16")
    ws = torch.zeros(gpq.oal_contribution_workspace_bytes(dims, 1500), dtype=torch.uint8, device="cuda")
    first = None
    for seed in (78, 79, 78):
        x = small(seed, 3, 14, 2, 1500, "bf16")
        chi = torch.empty((3, 14, 64), dtype=torch.float32, device="cuda")
        chi_mean = torch.empty((14, 64), dtype=torch.float32, device="cuda")
        gpq.oal_contribution(dims, 1500, to_dev(x.q, "bf16"), to_dev(x.k, "bf16"), ws, chi, chi_mean)
        ref, ref_mean = oracle.contribution(x.q, x.k)
        got = chi.cpu().numpy()
        assert rel_err(got, ref) <= chi_tol(1500)
        assert rel_err(chi_mean.cpu().numpy(), ref_mean) <= chi_tol(1500, 3)
        if first is None:
            first = got
    assert np.array_equal(first, got)
    cb = -(-(3 * 14 + 14) * 128 // 256) * 256
    assert int(ws[:cb].count_nonzero()) == 0


def test_contribution_partials_contents_do_not_matter_and_repeat_bitwise():
    inp = small(77, 2, 14, 2, 333, "bf16")
    a, am = run_chi(inp.q, inp.k, "bf16", ws_fill=float("nan"))
    b, bm = run_chi(inp.q, inp.k, "bf16", ws_fill=1e30)
    c, _ = run_chi(inp.q, inp.k, "bf16", with_mean=False)
    assert np.array_equal(a, b) and np.array_equal(am, bm) and np.array_equal(a, c)
    ref, _ = oracle.contribution(inp.q, inp.k)
    assert rel_err(a, ref) <= chi_tol(333)


def test_contribution_cfg2_full():
    inp = cfg2()
    chi, chi_mean = run_chi(inp.q, inp.k, "bf16")
    ref, ref_mean = oracle.contribution(inp.q, inp.k)
    e = rel_err(chi, ref)
    print(f"[parity] chi cfg2 B=1 T=4096: err={e:.2e} tol={chi_tol(4096):.2e}", flush=True)
    assert e <= chi_tol(4096) and rel_err(chi_mean, ref_mean) <= chi_tol(4096, 1)


def test_contribution_cfg3_batch8_full():
    inp = cfg3()
    chi, chi_mean = run_chi(inp.q, inp.k, "bf16")
    ref, ref_mean = oracle.contribution(inp.q, inp.k)
    e, em = rel_err(chi, ref), rel_err(chi_mean, ref_mean)
    print(f"[parity] chi cfg3 B=8 T=4096: err={e:.2e} mean={em:.2e}", flush=True)
    assert e <= chi_tol(4096) and em <= chi_tol(4096, 8)


def test_contribution_cfg4_long_context_two_heads():
    # every head is computed on the GPU; the oracle checks one query head per KV head
    inp = cfg4()
    chi, _ = run_chi(inp.q, inp.k, "bf16")
    heads = [0, 7]
    ref, _ = oracle.contribution(inp.q[:, heads], inp.k)
    e = rel_err(chi[:, heads], ref)
    print(f"[parity] chi cfg4 T=32768 heads {heads}: err={e:.2e} tol={chi_tol(32768):.2e}", flush=True)
    assert e <= chi_tol(32768)
