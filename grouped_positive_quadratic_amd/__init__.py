"""Python binding of liboal (OAL causal attention on MI355X): argument marshalling only.

Every entry point has the name of the C function in ``include/oal.h`` that it calls. Device
buffers are torch tensors on the GPU (torch provides memory and streams, nothing else);
all computation happens in the library's HIP kernels. Importing this module fails loudly
when the library has not been built (``python grouped_positive_quadratic_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liboal.so")

OAL_F32, OAL_BF16 = 0, 1
NFEAT, V1, D = 2145, 65, 64
STATE_STRIDE = 139456          # floats per (sequence, KV head) block of the state buffer
STATUS = {0: "OAL_OK", 1: "OAL_E_ARG", 2: "OAL_E_SHAPE", 3: "OAL_E_DTYPE", 4: "OAL_E_ALIGN",
          5: "OAL_E_UNSUPPORTED", 6: "OAL_E_HIP"}
EXPORTED = ("oal_params_bytes", "oal_state_bytes", "oal_prefill_workspace_bytes",
            "oal_decode_workspace_bytes", "oal_params_pack", "oal_state_init", "oal_prefill",
            "oal_prefill_timed", "oal_decode_step", "oal_status_string", "oal_timing_event_create",
            "oal_timing_event_destroy", "oal_timing_event_record", "oal_timing_elapsed_ms",
            "oal_contribution_workspace_bytes", "oal_contribution", "oal_decode_step_indexed",
            "oal_prefill_varlen", "oal_prefill_packed", "oal_prefill_backward_workspace_bytes",
            "oal_prefill_backward", "oal_decode_step_noalloc", "oal_calib_mfma_bf16", "oal_calib_copy",
            "oal_workspace_clear")
DECODE_NOALLOC_MAX_BLOCKS = 256   # OAL_DECODE_NOALLOC_MAX_BLOCKS


class OALError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({status_string(code)})")


class oal_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class oal_head_params(ctypes.Structure):
    _fields_ = [("g_max", ctypes.c_int32), ("n_groups", ctypes.c_void_p),
                ("group_of_dim", ctypes.c_void_p), ("L", ctypes.c_void_p),
                ("eps", ctypes.c_void_p)]


def _load():
    # torch ships its own HIP runtime. Loading it first makes the dynamic linker bind
    # liboal.so to that same runtime instance; loaded the other way round, the process would
    # hold two runtimes and torch's device pointers and streams would be foreign to liboal.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python grouped_positive_quadratic_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    dp = ctypes.POINTER(oal_dims)
    hp = ctypes.POINTER(oal_head_params)
    lib.oal_params_bytes.argtypes, lib.oal_params_bytes.restype = [dp], S
    lib.oal_state_bytes.argtypes, lib.oal_state_bytes.restype = [dp], S
    lib.oal_prefill_workspace_bytes.argtypes, lib.oal_prefill_workspace_bytes.restype = [dp, I, I], S
    lib.oal_decode_workspace_bytes.argtypes, lib.oal_decode_workspace_bytes.restype = [dp], S
    lib.oal_params_pack.argtypes, lib.oal_params_pack.restype = [dp, hp, P, S], ctypes.c_int
    lib.oal_state_init.argtypes, lib.oal_state_init.restype = [dp, hp, P, P, P], ctypes.c_int
    lib.oal_prefill.argtypes = [dp, I, I, P, P, P, P, P, P, S, P, P]
    lib.oal_prefill.restype = ctypes.c_int
    lib.oal_prefill_timed.argtypes = [dp, I, I, P, P, P, P, P, P, S, P, P, ctypes.POINTER(P)]
    lib.oal_prefill_timed.restype = ctypes.c_int
    lib.oal_prefill_varlen.argtypes = [dp, I, P, I, P, P, P, P, P, P, S, P, P]
    lib.oal_prefill_varlen.restype = ctypes.c_int
    lib.oal_prefill_packed.argtypes = [dp, I, P, ctypes.c_int64, I, P, P, P, P, P, P, S, P, P]
    lib.oal_prefill_packed.restype = ctypes.c_int
    lib.oal_decode_step.argtypes = [dp, P, P, P, P, P, P, S, P, P]
    lib.oal_decode_step.restype = ctypes.c_int
    lib.oal_decode_step_indexed.argtypes = [dp, P, I, P, P, P, P, P, P, S, P, P]
    lib.oal_decode_step_indexed.restype = ctypes.c_int
    lib.oal_decode_step_noalloc.argtypes = [dp, P, P, P, P, P, P, P]
    lib.oal_decode_step_noalloc.restype = ctypes.c_int
    lib.oal_status_string.argtypes, lib.oal_status_string.restype = [ctypes.c_int], ctypes.c_char_p
    lib.oal_calib_mfma_bf16.argtypes = [I, I, P, ctypes.POINTER(ctypes.c_double), P]
    lib.oal_calib_mfma_bf16.restype = ctypes.c_int
    lib.oal_calib_copy.argtypes, lib.oal_calib_copy.restype = [P, P, S, P], ctypes.c_int
    lib.oal_workspace_clear.argtypes, lib.oal_workspace_clear.restype = [P, S, P], ctypes.c_int
    lib.oal_timing_event_create.argtypes, lib.oal_timing_event_create.restype = [ctypes.POINTER(P)], ctypes.c_int
    lib.oal_timing_event_destroy.argtypes, lib.oal_timing_event_destroy.restype = [P], ctypes.c_int
    lib.oal_timing_event_record.argtypes, lib.oal_timing_event_record.restype = [P, P], ctypes.c_int
    lib.oal_timing_elapsed_ms.argtypes = [P, P, ctypes.POINTER(ctypes.c_float)]
    lib.oal_timing_elapsed_ms.restype = ctypes.c_int
    lib.oal_contribution_workspace_bytes.argtypes = [dp, I]
    lib.oal_contribution_workspace_bytes.restype = S
    lib.oal_contribution.argtypes, lib.oal_contribution.restype = [dp, I, P, P, P, S, P, P, P], ctypes.c_int
    lib.oal_prefill_backward_workspace_bytes.argtypes = [dp, I, I]
    lib.oal_prefill_backward_workspace_bytes.restype = S
    lib.oal_prefill_backward.argtypes = [dp, I, I, P, P, P, P, P, P, P, S, P, P, P, P, P, P, P]
    lib.oal_prefill_backward.restype = ctypes.c_int
    return lib


_lib = _load()


def status_string(code: int) -> str:
    return _lib.oal_status_string(int(code)).decode()


def make_dims(batch: int, n_q_heads: int, n_kv_heads: int, dtype: str = "bf16",
              d_h: int = 64, d_v: int = 64) -> oal_dims:
    dt = {"bf16": OAL_BF16, "f32": OAL_F32}.get(dtype, dtype)
    return oal_dims(int(batch), int(n_q_heads), int(n_kv_heads), int(d_h), int(d_v), int(dt))


class HeadParamsC:
    """Host arrays of the per-head parameters, kept alive for the duration of a call."""

    def __init__(self, n_groups, group_of_dim, L, eps):
        self.n_groups = np.ascontiguousarray(n_groups, dtype=np.int32)
        self.group_of_dim = np.ascontiguousarray(group_of_dim, dtype=np.uint8)
        self.L = np.ascontiguousarray(L, dtype=np.float32)
        self.eps = np.ascontiguousarray(eps, dtype=np.float32)
        self.c = oal_head_params(int(self.L.shape[1]) - 1,
                                 self.n_groups.ctypes.data, self.group_of_dim.ctypes.data,
                                 self.L.ctypes.data, self.eps.ctypes.data)

    @classmethod
    def from_params(cls, p) -> "HeadParamsC":
        return cls(p.n_groups, p.group_of_dim, p.L, p.eps)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("device buffers must be GPU tensors")
    if not t.is_contiguous():
        raise ValueError("device buffers must be contiguous")
    return t.data_ptr()


# a raw integer pointer carries no size: the caller vouches for it (tests of argument checks)
_UNSIZED = (1 << 63) - 1


def _nbytes(t, given=None) -> int:
    """Size in bytes of a device buffer: `given` if the caller states it, else the tensor's."""
    if given is not None:
        return int(given)
    if t is None:
        return 0
    if isinstance(t, int):
        return _UNSIZED
    return int(t.numel() * t.element_size())


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, code: int):
    if code != 0:
        raise OALError(fn, code)


# ---- sizes -----------------------------------------------------------------------------

def oal_params_bytes(dims: oal_dims) -> int:
    return int(_lib.oal_params_bytes(ctypes.byref(dims)))


def oal_state_bytes(dims: oal_dims) -> int:
    return int(_lib.oal_state_bytes(ctypes.byref(dims)))


def oal_prefill_workspace_bytes(dims: oal_dims, T: int, chunk: int) -> int:
    return int(_lib.oal_prefill_workspace_bytes(ctypes.byref(dims), int(T), int(chunk)))


def oal_decode_workspace_bytes(dims: oal_dims) -> int:
    return int(_lib.oal_decode_workspace_bytes(ctypes.byref(dims)))


# ---- calls -----------------------------------------------------------------------------

def oal_params_pack(dims: oal_dims, params: HeadParamsC) -> np.ndarray:
    """Host-side parameter blob (uint8 array) exactly as oal_state_init uploads it."""
    n = oal_params_bytes(dims)
    blob = np.zeros(max(n, 1), dtype=np.uint8)
    _check("oal_params_pack", _lib.oal_params_pack(ctypes.byref(dims), ctypes.byref(params.c),
                                                   blob.ctypes.data, n))
    return blob[:n]


def oal_state_init(dims: oal_dims, params: HeadParamsC, params_dev, state_dev=None, stream=None):
    _check("oal_state_init", _lib.oal_state_init(ctypes.byref(dims), ctypes.byref(params.c),
                                                 _ptr(params_dev), _ptr(state_dev), _stream(stream)))


def oal_prefill(dims: oal_dims, T: int, chunk: int, q, k, v, params_dev, state_dev, workspace, y,
                stream=None, workspace_bytes=None):
    """y=None (and then q may be None) only advances the state."""
    _check("oal_prefill", _lib.oal_prefill(ctypes.byref(dims), int(T), int(chunk), _ptr(q), _ptr(k),
                                           _ptr(v), _ptr(params_dev), _ptr(state_dev),
                                           _ptr(workspace), _nbytes(workspace, workspace_bytes), _ptr(y),
                                           _stream(stream)))


def oal_prefill_varlen(dims: oal_dims, T: int, lengths, chunk: int, q, k, v, params_dev, state_dev,
                       workspace, y, stream=None, workspace_bytes=None):
    """Ragged batch padded to T: lengths is a device int32 tensor [batch]."""
    _check("oal_prefill_varlen", _lib.oal_prefill_varlen(
        ctypes.byref(dims), int(T), _ptr(lengths), int(chunk), _ptr(q), _ptr(k), _ptr(v),
        _ptr(params_dev), _ptr(state_dev), _ptr(workspace), _nbytes(workspace, workspace_bytes), _ptr(y),
        _stream(stream)))


def oal_prefill_packed(dims: oal_dims, T: int, cu_seqlens, total_tokens: int, chunk: int, q, k, v,
                       params_dev, state_dev, workspace, y, stream=None, workspace_bytes=None):
    """Packed ragged batch: q, y [n_q_heads, total, 64], k, v [n_kv_heads, total, 64];
    cu_seqlens is a device int32 tensor [batch + 1]."""
    _check("oal_prefill_packed", _lib.oal_prefill_packed(
        ctypes.byref(dims), int(T), _ptr(cu_seqlens), int(total_tokens), int(chunk), _ptr(q), _ptr(k),
        _ptr(v), _ptr(params_dev), _ptr(state_dev), _ptr(workspace), _nbytes(workspace, workspace_bytes),
        _ptr(y), _stream(stream)))


def oal_prefill_timed(dims: oal_dims, T: int, chunk: int, q, k, v, params_dev, state_dev, workspace,
                      y, marks, stream=None, workspace_bytes=None):
    """oal_prefill plus three caller-owned events (torch.cuda.Event, already created) recorded
    before the scan, between scan and readout, and after the readout."""
    handles = (ctypes.c_void_p * 3)(*[int(m.cuda_event) for m in marks])
    _check("oal_prefill_timed", _lib.oal_prefill_timed(
        ctypes.byref(dims), int(T), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(params_dev),
        _ptr(state_dev), _ptr(workspace), _nbytes(workspace, workspace_bytes), _ptr(y), _stream(stream),
        handles))


def oal_workspace_clear(workspace, workspace_bytes=None, stream=None):
    n = _nbytes(workspace, workspace_bytes)
    if n == _UNSIZED:
        raise ValueError("oal_workspace_clear: give workspace_bytes for a raw pointer")
    _check("oal_workspace_clear", _lib.oal_workspace_clear(_ptr(workspace), n, _stream(stream)))


def oal_calib_mfma_bf16(blocks: int, iters: int, out, stream=None) -> float:
    """Matrix-core loop (measurement aid); returns the dense flop count it enqueued."""
    flops = ctypes.c_double()
    _check("oal_calib_mfma_bf16", _lib.oal_calib_mfma_bf16(blocks, iters, _ptr(out), ctypes.byref(flops),
                                                           _stream(stream)))
    return float(flops.value)


def oal_calib_copy(src, dst, nbytes: int, stream=None):
    """Streaming device copy of nbytes (measurement aid)."""
    _check("oal_calib_copy", _lib.oal_calib_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


class TimingEvent:
    """A HIP event from oal_timing_event_create (no system-scope release when recorded)."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check("oal_timing_event_create", _lib.oal_timing_event_create(ctypes.byref(h)))
        self.cuda_event = h.value

    def record(self, stream=None):
        _check("oal_timing_event_record", _lib.oal_timing_event_record(ctypes.c_void_p(self.cuda_event),
                                                                       _stream(stream)))

    def elapsed_time(self, end: "TimingEvent") -> float:
        ms = ctypes.c_float()
        _check("oal_timing_elapsed_ms", _lib.oal_timing_elapsed_ms(ctypes.c_void_p(self.cuda_event),
                                                                   ctypes.c_void_p(end.cuda_event),
                                                                   ctypes.byref(ms)))
        return float(ms.value)

    def __del__(self):
        if getattr(self, "cuda_event", None) and _lib is not None:
            _lib.oal_timing_event_destroy(ctypes.c_void_p(self.cuda_event))
            self.cuda_event = None


def oal_decode_step(dims: oal_dims, q, k, v, params_dev, state_dev, workspace, y, stream=None,
                    workspace_bytes=None):
    _check("oal_decode_step", _lib.oal_decode_step(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v),
                                                   _ptr(params_dev), _ptr(state_dev),
                                                   _ptr(workspace), _nbytes(workspace, workspace_bytes),
                                                   _ptr(y), _stream(stream)))


def oal_decode_step_noalloc(dims: oal_dims, q, k, v, params_dev, state_dev, y, stream=None):
    """oal_decode_step with the library's static per-GPU workspace (no caller buffer)."""
    _check("oal_decode_step_noalloc", _lib.oal_decode_step_noalloc(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(params_dev), _ptr(state_dev), _ptr(y),
        _stream(stream)))


def oal_contribution_workspace_bytes(dims: oal_dims, T: int) -> int:
    return int(_lib.oal_contribution_workspace_bytes(ctypes.byref(dims), int(T)))


def oal_contribution(dims: oal_dims, T: int, q, k, workspace, chi, chi_mean=None, stream=None,
                     workspace_bytes=None):
    """Causal contribution scores chi [batch, n_q_heads, 64] and (unless chi_mean is None)
    their prompt mean [n_q_heads, 64], both fp32 device tensors written by the library."""
    _check("oal_contribution", _lib.oal_contribution(ctypes.byref(dims), int(T), _ptr(q), _ptr(k),
                                                     _ptr(workspace), _nbytes(workspace, workspace_bytes),
                                                     _ptr(chi), _ptr(chi_mean),
                                                     _stream(stream)))


def oal_prefill_backward_workspace_bytes(dims: oal_dims, T: int, chunk: int) -> int:
    return int(_lib.oal_prefill_backward_workspace_bytes(ctypes.byref(dims), int(T), int(chunk)))


def oal_prefill_backward(dims: oal_dims, T: int, chunk: int, q, k, v, dy, params_dev, workspace,
                         dq, dk, dv, dL=None, deps=None, stream=None, workspace_bytes=None,
                         state_in=None, dstate_in=None):
    """Gradients dq [batch, n_q_heads, T, 64], dk, dv [batch, n_kv_heads, T, 64] (fp32 device
    tensors written by the library) of sum(dy * y) for the prefill of T tokens continuing from
    state_in (None: an empty prefix); with dL [n_q_heads, 65, 65] and deps [n_q_heads] (fp32
    device tensors, or both None) also the coefficient gradients, and with dstate_in (a state
    buffer) the gradient of the incoming state."""
    _check("oal_prefill_backward", _lib.oal_prefill_backward(
        ctypes.byref(dims), int(T), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(dy),
        _ptr(params_dev), _ptr(state_in), _ptr(workspace), _nbytes(workspace, workspace_bytes), _ptr(dq),
        _ptr(dk), _ptr(dv), _ptr(dstate_in), _ptr(dL), _ptr(deps),
        _stream(stream)))


def oal_decode_step_indexed(dims: oal_dims, slots, pool_size: int, q, k, v, params_dev, state_pool,
                            workspace, y, stream=None, workspace_bytes=None):
    """Decode step on pool blocks: slots is a device int32 tensor [batch]."""
    _check("oal_decode_step_indexed", _lib.oal_decode_step_indexed(
        ctypes.byref(dims), _ptr(slots), int(pool_size), _ptr(q), _ptr(k), _ptr(v), _ptr(params_dev),
        _ptr(state_pool), _ptr(workspace), _nbytes(workspace, workspace_bytes), _ptr(y), _stream(stream)))


# ---- buffer helper (torch allocations sized by the library) ------------------------------

def state_view(state, batch: int, n_kv_heads: int):
    """[batch, n_kv_heads, 2145, 65] copy of the prefix states H in a state buffer: each
    block holds columns 0..63 as a [2145, 64] row-major matrix, then column 64 (2145 floats)."""
    import torch
    blk = state.view(batch, n_kv_heads, STATE_STRIDE)
    main = blk[:, :, : NFEAT * D].reshape(batch, n_kv_heads, NFEAT, D)
    den = blk[:, :, NFEAT * D: NFEAT * V1].reshape(batch, n_kv_heads, NFEAT, 1)
    return torch.cat([main, den], dim=3)


def state_index(f: int, c: int) -> int:
    """Offset of H[f][c] inside one state block (the C macro OAL_STATE_INDEX)."""
    return f * D + c if c < D else NFEAT * D + f


def alloc_buffers(dims: oal_dims, T: int = 0, chunk: int = 128, device: str = "cuda"):
    """Allocate params, state, prefill workspace and a zeroed decode workspace (uint8/fp32 tensors)."""
    import torch
    nb = lambda n: max(int(n), 16)
    params = torch.empty(nb(oal_params_bytes(dims)), dtype=torch.uint8, device=device)
    state = torch.empty(nb(oal_state_bytes(dims)) // 4, dtype=torch.float32, device=device)
    ws = torch.empty(nb(oal_prefill_workspace_bytes(dims, T, chunk)) if T else 16,
                     dtype=torch.uint8, device=device)
    dws = torch.zeros(nb(oal_decode_workspace_bytes(dims)), dtype=torch.uint8, device=device)
    return params, state, ws, dws
