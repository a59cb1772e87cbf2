"""Helpers for the GPU tests: upload seeded inputs, run the library through its C ABI."""
import numpy as np
import torch

import grouped_positive_quadratic_amd as gpq

TOL = {"f32": 1e-5, "bf16": 3e-2}


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda().contiguous()


class Session:
    """Device buffers for one workload: params, state, workspaces."""

    def __init__(self, B, Hq, Hkv, dtype, params, T=0, chunk=128):
        self.dims = gpq.make_dims(B, Hq, Hkv, dtype)
        self.dtype = dtype
        self.hp = gpq.HeadParamsC.from_params(params)
        self.params, self.state, self.ws, self.dws = gpq.alloc_buffers(self.dims, T, chunk)
        gpq.oal_state_init(self.dims, self.hp, self.params, self.state)
        self.B, self.Hq, self.Hkv = B, Hq, Hkv

    def ensure_ws(self, T, chunk):
        need = gpq.oal_prefill_workspace_bytes(self.dims, T, chunk)
        if self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def prefill(self, q, k, v, chunk=128):
        q, k, v = (to_dev(x, self.dtype) if isinstance(x, np.ndarray) else x for x in (q, k, v))
        T = q.shape[2]
        self.ensure_ws(T, chunk)
        y = torch.empty((self.B, self.Hq, T, 64), dtype=torch.float32, device="cuda")
        gpq.oal_prefill(self.dims, T, chunk, q, k, v, self.params, self.state, self.ws, y)
        return y

    def decode(self, q, k, v):
        q, k, v = (to_dev(x, self.dtype) if isinstance(x, np.ndarray) else x for x in (q, k, v))
        y = torch.empty((self.B, self.Hq, 64), dtype=torch.float32, device="cuda")
        gpq.oal_decode_step(self.dims, q, k, v, self.params, self.state, self.dws, y)
        return y

    def state_np(self):
        torch.cuda.synchronize()
        return gpq.state_view(self.state, self.B, self.Hkv).cpu().numpy().astype(np.float64)


def session_for(inp, chunk=128):
    B, Hq, Hkv, T, d, dv = inp.dims
    return Session(B, Hq, Hkv, inp.dtype, inp.params, T, chunk)


def state_ok(S, k, v, dtype):
    """Final prefix states against the oracle's.

    fp32 inputs: blockwise relative error <= 1e-5. bf16 inputs: the scan feeds each feature
    psi(k) = k_r k_t (exact in fp32) to the MFMA rounded once to bf16 (<= 2^-9 relative), and
    each chunk's increment sum_{j in chunk} psi(k_j) [v_j;1] (fp32 on the MFMA) is stored once
    in bf16 (<= 2^-9 of its absolute sum) before the fp32 sum over chunks, so each element obeys
    |S - S*| <= 2^-8 * sum_j |psi_f(k_j)| |[v_j;1]_c| up to fp32 terms; the bound 2^-7 keeps a
    2x margin. The right-hand side is the oracle's state of |k|, |v|.
    """
    import oracle
    S_ref = oracle.state(k, v)
    if dtype == "f32":
        return state_error(S, S_ref) <= 1e-5
    S_abs = oracle.state(np.abs(k), np.abs(v))
    return bool(np.all(np.abs(S - S_ref) <= 2.0 ** -7 * S_abs + 1e-6 * S_abs.max()))


def state_error(S, S_ref):
    """max |S - S_ref| / max |S_ref| per (sequence, KV head) block."""
    num = np.abs(S - S_ref).reshape(S.shape[0], S.shape[1], -1).max(-1)
    den = np.abs(S_ref).reshape(S.shape[0], S.shape[1], -1).max(-1)
    return float((num / den).max())
