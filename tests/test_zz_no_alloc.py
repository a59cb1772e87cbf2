"""GPU test of oal_decode_step_noalloc (the decode step whose workspace is a static device
array inside the library, for callers that cannot allocate): through the C ABI, two calls in a
row, the second with a smaller batch, each compared bit for bit with oal_decode_step on a
caller workspace (same kernel, same summation order) and with the oracle."""
import numpy as np
import pytest

import oracle
from oal_synth import small

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import to_dev  # noqa: E402
import grouped_positive_quadratic_amd as gpq  # noqa: E402


def _step_both(seed, B, Hq, Hkv, T, dtype):
    """Prefill T tokens, then one decode step twice from the same states: once with a caller
    workspace, once without. Returns both outputs, both updated states and the oracle row."""
    dev = "cuda"
    inp = small(seed, B, Hq, Hkv, T + 1, dtype)
    dims = gpq.make_dims(B, Hq, Hkv, dtype)
    params, state, ws, dws = gpq.alloc_buffers(dims, T, 64, device=dev)
    gpq.oal_state_init(dims, gpq.HeadParamsC.from_params(inp.params), params, state)
    q, k, v = (to_dev(x[:, :, :T], dtype) for x in (inp.q, inp.k, inp.v))
    gpq.oal_prefill(dims, T, 64, None, k, v, params, state, ws, None)
    qd, kd, vd = (to_dev(np.ascontiguousarray(x[:, :, T]), dtype) for x in (inp.q, inp.k, inp.v))
    state2 = state.clone()
    y_ws = torch.full((B, Hq, 64), np.nan, dtype=torch.float32, device=dev)
    y_na = torch.full((B, Hq, 64), np.nan, dtype=torch.float32, device=dev)
    gpq.oal_decode_step(dims, qd, kd, vd, params, state, dws, y_ws)
    gpq.oal_decode_step_noalloc(dims, qd, kd, vd, params, state2, y_na)
    torch.cuda.synchronize()
    ref = oracle.dense(inp.q, inp.k, inp.v, inp.params)[:, :, T]
    return y_ws.cpu().numpy(), y_na.cpu().numpy(), state.cpu().numpy(), state2.cpu().numpy(), ref


def test_noalloc_decode_two_calls_second_smaller():
    # first call 12 sequences x 2 KV heads, second 3 x 2 on the same static array: the
    # counters and partials the first call left behind must not leak into the second
    for seed, B, dtype in ((71, 12, "bf16"), (72, 3, "bf16")):
        print(f"[noalloc] seed={seed} B={B} Hq=14 Hkv=2 T=200 {dtype}", flush=True)
        y_ws, y_na, st_ws, st_na, ref = _step_both(seed, B, 14, 2, 200, dtype)
        assert np.isfinite(y_na).all()
        assert np.array_equal(y_ws, y_na)
        assert np.array_equal(st_ws, st_na)
        assert oracle.row_error(y_na, ref) <= 3e-2


def test_noalloc_decode_fp32_and_limit():
    y_ws, y_na, st_ws, st_na, ref = _step_both(73, 2, 4, 2, 130, "f32")
    assert np.array_equal(y_ws, y_na) and np.array_equal(st_ws, st_na)
    assert oracle.row_error(y_na, ref) <= 1e-5
    # above the static array's capacity: an error, nothing launched
    big = gpq.make_dims(gpq.DECODE_NOALLOC_MAX_BLOCKS // 2 + 1, 14, 2, "bf16")
    x = torch.zeros(16, dtype=torch.float32, device="cuda")
    with pytest.raises(gpq.OALError, match="OAL_E_UNSUPPORTED"):
        gpq.oal_decode_step_noalloc(big, x, x, x, x, x, x)
