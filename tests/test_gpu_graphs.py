"""GPU: the library's calls captured into a HIP graph (torch.cuda.CUDAGraph on ROCm) and
replayed. The calls enqueue kernels only (no memset, no allocation), and every workspace
counter is returned to zero by the kernels, so each replay must reproduce the eager results
bit for bit. Each replay is checked, with eager work and synchronisations in between."""
import numpy as np
import pytest

from oal_synth import small

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import Session, to_dev  # noqa: E402
import grouped_positive_quadratic_amd as gpq  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


def test_prefill_and_decode_graph_replays_match_eager():
    B, Hq, Hkv, T = 2, 14, 2, 300
    inp = small(801, B, Hq, Hkv, T + 1, "bf16")
    q, k, v = (to_dev(x[:, :, :T], "bf16") for x in (inp.q, inp.k, inp.v))
    q1, k1, v1 = (to_dev(x[:, :, T], "bf16") for x in (inp.q, inp.k, inp.v))

    # eager reference: prefill from zero, then one decode step
    ref = Session(B, Hq, Hkv, "bf16", inp.params, T, 128)
    y_ref = ref.prefill(q, k, v, 128)
    yd_ref = ref.decode(q1, k1, v1)
    torch.cuda.synchronize()
    state_ref = ref.state.clone()

    sess = Session(B, Hq, Hkv, "bf16", inp.params, T, 128)
    y = torch.empty((B, Hq, T, 64), dtype=torch.float32, device="cuda")
    yd = torch.empty((B, Hq, 64), dtype=torch.float32, device="cuda")
    zero_state = sess.state.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):     # warm-up on the capture stream (code objects, attributes)
        gpq.oal_prefill(sess.dims, T, 128, q, k, v, sess.params, sess.state, sess.ws, y)
        gpq.oal_decode_step(sess.dims, q1, k1, v1, sess.params, sess.state, sess.dws, yd)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpq.oal_prefill(sess.dims, T, 128, q, k, v, sess.params, sess.state, sess.ws, y)
        gpq.oal_decode_step(sess.dims, q1, k1, v1, sess.params, sess.state, sess.dws, yd)
    for rep in range(4):
        sess.state.copy_(zero_state)           # eager work between replays
        y.fill_(float("nan"))
        yd.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep}: prefill output differs"
        assert torch.equal(yd, yd_ref), f"replay {rep}: decode output differs"
        assert torch.equal(sess.state, state_ref), f"replay {rep}: state differs"
    assert int(sess.dws[:256].count_nonzero()) == 0


def test_decode_loop_graph_replays_match_eager():
    # a captured loop of decode steps (a serving inner loop), replayed from the same state
    B, Hq, Hkv, T0, steps = 4, 14, 2, 64, 8
    inp = small(802, B, Hq, Hkv, T0 + steps, "bf16")
    base = Session(B, Hq, Hkv, "bf16", inp.params, T0, 64)
    base.prefill(inp.q[:, :, :T0], inp.k[:, :, :T0], inp.v[:, :, :T0], 64)
    torch.cuda.synchronize()
    start = base.state.clone()
    toks = [tuple(to_dev(x[:, :, T0 + s], "bf16") for x in (inp.q, inp.k, inp.v)) for s in range(steps)]
    ys_ref = [base.decode(*t) for t in toks]
    torch.cuda.synchronize()
    end_ref = base.state.clone()
    base.state.copy_(start)
    ys = [torch.empty((B, Hq, 64), dtype=torch.float32, device="cuda") for _ in range(steps)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for t, yy in zip(toks, ys):
            gpq.oal_decode_step(base.dims, *t, base.params, base.state, base.dws, yy)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t, yy in zip(toks, ys):
            gpq.oal_decode_step(base.dims, *t, base.params, base.state, base.dws, yy)
    for rep in range(3):
        base.state.copy_(start)
        for yy in ys:
            yy.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            assert torch.equal(ys[s], ys_ref[s]), f"replay {rep} step {s}"
        assert torch.equal(base.state, end_ref)


def test_concurrent_streams_match_sequential():
    # independent sequences on two streams at once (their own params, states, workspaces):
    # the library keeps no global mutable state, so results equal those of sequential calls
    B, Hq, Hkv, T = 2, 14, 2, 513
    ins = [small(811 + i, B, Hq, Hkv, T + 1, "bf16") for i in range(2)]
    seq_out = []
    for inp in ins:
        s = Session(B, Hq, Hkv, "bf16", inp.params, T, 128)
        y = s.prefill(inp.q[:, :, :T], inp.k[:, :, :T], inp.v[:, :, :T], 128)
        yd = s.decode(inp.q[:, :, T], inp.k[:, :, T], inp.v[:, :, T])
        torch.cuda.synchronize()
        seq_out.append((y.clone(), yd.clone(), s.state.clone()))
    sessions = [Session(B, Hq, Hkv, "bf16", inp.params, T, 128) for inp in ins]
    dev = [tuple(to_dev(x[:, :, :T], "bf16") for x in (inp.q, inp.k, inp.v)) for inp in ins]
    dev1 = [tuple(to_dev(x[:, :, T], "bf16") for x in (inp.q, inp.k, inp.v)) for inp in ins]
    ys = [torch.empty((B, Hq, T, 64), dtype=torch.float32, device="cuda") for _ in ins]
    yds = [torch.empty((B, Hq, 64), dtype=torch.float32, device="cuda") for _ in ins]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for i, st in enumerate(streams):
        with torch.cuda.stream(st):
            s = sessions[i]
            gpq.oal_prefill(s.dims, T, 128, *dev[i], s.params, s.state, s.ws, ys[i], stream=st)
            gpq.oal_decode_step(s.dims, *dev1[i], s.params, s.state, s.dws, yds[i], stream=st)
    torch.cuda.synchronize()
    for i in range(2):
        assert torch.equal(ys[i], seq_out[i][0]) and torch.equal(yds[i], seq_out[i][1])
        assert torch.equal(sessions[i].state, seq_out[i][2])


def test_backward_graph_replays_match_eager():
    """The backward (with the coefficient gradients) enqueues kernels only: captured once, every
    replay gives the eager call's dq, dk, dv, dL, deps bit for bit."""
    B, Hq, Hkv, T, C = 1, 7, 1, 200, 64
    inp = small(802, B, Hq, Hkv, T, "bf16")
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    dims = gpq.make_dims(B, Hq, Hkv, "bf16")
    params = torch.empty(gpq.oal_params_bytes(dims), dtype=torch.uint8, device="cuda")
    gpq.oal_state_init(dims, gpq.HeadParamsC.from_params(inp.params), params, None)
    dy = torch.from_numpy(np.random.default_rng(802).normal(0.0, 1.0, (B, Hq, T, 64)).astype(np.float32)).cuda()
    ws = torch.empty(gpq.oal_prefill_backward_workspace_bytes(dims, T, C), dtype=torch.uint8, device="cuda")

    def outs():
        return [torch.empty((B, Hq, T, 64), device="cuda"), torch.empty((B, Hkv, T, 64), device="cuda"),
                torch.empty((B, Hkv, T, 64), device="cuda"), torch.empty((Hq, 65, 65), device="cuda"),
                torch.empty((Hq,), device="cuda")]

    ref = outs()
    gpq.oal_prefill_backward(dims, T, C, q, k, v, dy, params, ws, *ref)
    torch.cuda.synchronize()
    got = outs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gpq.oal_prefill_backward(dims, T, C, q, k, v, dy, params, ws, *got)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpq.oal_prefill_backward(dims, T, C, q, k, v, dy, params, ws, *got)
    for rep in range(3):
        for x in got:
            x.fill_(float("nan"))
        ws.fill_(7)                                # the workspace needs no initialisation
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "dL", "deps"), got, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs"
