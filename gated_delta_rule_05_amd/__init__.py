"""MI355X (gfx950) Kimi Delta Attention forward pass: Python binding.

Thin ctypes layer over ``libkda.so`` (the C ABI in ``include/kda.h``).  It
checks tensor dtypes, shapes, devices and contiguity, allocates outputs and
the workspace with torch, and passes raw pointers plus torch's current HIP
stream.  Every step of the computation runs in the library's HIP kernels;
there is no fallback: if the library is missing or the tensors are not on a
GPU, the calls raise.

    o, hT = prefill(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, scale=None)
    o = decode_step(q, k, v, log_alpha, beta, S, scale=None)   # S updated in place

Operation: the per-key-channel gated delta rule of "Kimi Delta Attention: la
atencion lineal detras de Kimi K2 y Qwen3", section "Cómo funciona Kimi
Delta Attention paso a paso"; the scale defaults to 1/sqrt(d_k) as there.
gate="head" takes log_alpha [.., H] (Gated DeltaNet: one scalar gate per
head, "Cos'è Kimi Delta Attention (KDA)?", section "Gating per canale: cosa
rende KDA diverso"); gate="none" takes no gate (DeltaNet, alpha = 1).
decode_step(state_index=...) updates states held in slots of a larger pool.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "KDAError", "STATUS", "DTYPE_BF16", "DTYPE_F32", "PATHS", "GATES", "FrontEnd",
    "PrefillOptions",
    "DecodeOptions", "library_path", "load_library",
    "abi_version", "status_string", "prefill_options", "prefill_workspace_bytes", "prefill",
    "decode_step", "DecodeMultiOptions", "decode_multi", "BwdOptions",
    "backward_workspace_bytes", "backward", "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda.so")

STATUS = {
    0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "MISALIGNED",
    4: "WORKSPACE_TOO_SMALL", 5: "HIP_ERROR",
}
DTYPE_BF16 = 0
DTYPE_F32 = 1
PATHS = {"auto": 0, "vector": 1, "matrix": 2, "two_pass": 3}
GATES = {"channel": 0, "head": 1, "none": 2}


class FrontEnd(ctypes.Structure):
    """Mirror of kda_front_end."""
    _fields_ = [("l2norm_qk", ctypes.c_int32), ("gate_scale", ctypes.c_float),
                ("gate_pre", ctypes.c_void_p), ("beta_pre", ctypes.c_void_p)]


class PrefillOptions(ctypes.Structure):
    """Mirror of kda_prefill_options."""
    _fields_ = [("path", ctypes.c_int32), ("value_tiles", ctypes.c_int32),
                ("block_chunks", ctypes.c_int32), ("gate", ctypes.c_int32),
                ("snapshot_tokens", ctypes.c_int32), ("snapshot_capacity", ctypes.c_int32),
                ("snapshots", ctypes.c_void_p), ("front", FrontEnd),
                ("chunk_states", ctypes.c_void_p), ("max_seqlen", ctypes.c_int64)]


class DecodeOptions(ctypes.Structure):
    """Mirror of kda_decode_options."""
    _fields_ = [("gate", ctypes.c_int32), ("num_states", ctypes.c_int32),
                ("state_index", ctypes.c_void_p), ("front", FrontEnd)]


class DecodeMultiOptions(ctypes.Structure):
    """Mirror of kda_decode_multi_options."""
    _fields_ = [("gate", ctypes.c_int32), ("num_states", ctypes.c_int32),
                ("state_index", ctypes.c_void_p), ("lengths", ctypes.c_void_p),
                ("write_state", ctypes.c_int32), ("front", FrontEnd)]

class BwdOptions(ctypes.Structure):
    """Mirror of kda_bwd_options."""
    _fields_ = [("gate", ctypes.c_int32), ("block_chunks", ctypes.c_int32),
                ("front", FrontEnd), ("chunk_states", ctypes.c_void_p),
                ("max_seqlen", ctypes.c_int64), ("aux_stream", ctypes.c_void_p)]

# Every function include/kda.h declares.
EXPORTED_SYMBOLS = ("kda_abi_version", "kda_status_string",
                    "kda_fwd_prefill_workspace_bytes", "kda_fwd_prefill_workspace_bytes_ex",
                    "kda_fwd_prefill", "kda_fwd_prefill_ex", "kda_decode_step",
                    "kda_decode_step_ex", "kda_decode_multi", "kda_bwd_workspace_bytes",
                    "kda_bwd", "kda_chunk_states_bytes", "kda_fwd_prefill_noalloc")


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (%d: %s)" % (
            where, STATUS.get(status, "?"), status, status_string(status)))


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            "libkda.so is not built at %s; build it with "
            "`python -m gated_delta_rule_05_amd.build` (hipcc, gfx950)" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_fwd_prefill_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32]
    lib.kda_fwd_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_fwd_prefill_workspace_bytes_ex.argtypes = [i64, i32, i32, i32, i32, i32,
                                                       ctypes.POINTER(PrefillOptions)]
    lib.kda_fwd_prefill_workspace_bytes_ex.restype = ctypes.c_size_t
    lib.kda_fwd_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32,
                                    i32, f32, vp, vp, vp, ctypes.c_size_t, vp]
    lib.kda_fwd_prefill.restype = ctypes.c_int
    lib.kda_fwd_prefill_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32,
                                       i32, f32, vp, vp, vp, ctypes.c_size_t,
                                       ctypes.POINTER(PrefillOptions), vp]
    lib.kda_fwd_prefill_ex.restype = ctypes.c_int
    lib.kda_fwd_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32,
                                            i32, f32, vp, vp, ctypes.POINTER(PrefillOptions), vp]
    lib.kda_fwd_prefill_noalloc.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                    vp, vp]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_step_ex.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                       vp, ctypes.POINTER(DecodeOptions), vp]
    lib.kda_decode_step_ex.restype = ctypes.c_int
    lib.kda_decode_multi.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                     vp, ctypes.POINTER(DecodeMultiOptions), vp]
    lib.kda_decode_multi.restype = ctypes.c_int
    lib.kda_bwd_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32,
                                            ctypes.POINTER(BwdOptions)]
    lib.kda_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, f32,
                            vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                            ctypes.POINTER(BwdOptions), vp]
    lib.kda_bwd.restype = ctypes.c_int
    lib.kda_chunk_states_bytes.argtypes = [i64, i32, i32, i32, i32]
    lib.kda_chunk_states_bytes.restype = ctypes.c_size_t
    _lib = lib
    return lib


def abi_version() -> int:
    return load_library().kda_abi_version()


def status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def _gate_code(gate):
    if gate not in GATES:
        raise ValueError("gate must be one of %s" % sorted(GATES))
    return GATES[gate]


def prefill_options(path="auto", value_tiles=0, block_chunks=0, gate="channel",
                    front=None, max_seqlen=0) -> PrefillOptions:
    if path not in PATHS:
        raise ValueError("path must be one of %s" % sorted(PATHS))
    opts = PrefillOptions(PATHS[path], int(value_tiles), int(block_chunks), _gate_code(gate))
    if front is not None:
        opts.front = front
    opts.max_seqlen = int(max_seqlen or 0)
    return opts


def front_end(l2norm_qk=False, gate_pre=None, gate_scale=1.0, beta_pre=None, shape=None,
              gate="channel", device=None):
    """A kda_front_end from torch tensors (None when every part is off).
    gate_pre: bf16 in log_alpha's layout; beta_pre: bf16 [tokens, H]."""
    if not l2norm_qk and gate_pre is None and beta_pre is None:
        return None
    torch = _torch()
    if gate_pre is not None:
        if gate == "none":
            raise ValueError("gate_pre needs a gate")
        _check(gate_pre, "gate_pre", tuple(shape) + ((gate_pre.shape[-1],) if gate == "channel" else ()),
               torch.bfloat16, device)
    if beta_pre is not None:
        _check(beta_pre, "beta_pre", tuple(shape), torch.bfloat16, device)
    return FrontEnd(1 if l2norm_qk else 0, float(gate_scale),
                    None if gate_pre is None else gate_pre.data_ptr(),
                    None if beta_pre is None else beta_pre.data_ptr())


def prefill_workspace_bytes(total_T: int, N: int, H: int, d_k: int, d_v: int,
                            dtype: int = DTYPE_BF16, path="auto", value_tiles=0,
                            block_chunks=0, gate="channel", front=False, max_seqlen=0) -> int:
    """``front``: True when the call will use the fused input front-end
    (it can change the automatic path, and with it the workspace)."""
    fe = FrontEnd(1, 0.0, None, None) if front else None
    opts = prefill_options(path, value_tiles, block_chunks, gate, fe, max_seqlen)
    return int(load_library().kda_fwd_prefill_workspace_bytes_ex(
        total_T, N, H, d_k, d_v, dtype, ctypes.byref(opts)))


# --------------------------------------------------------------------------
# torch-facing wrappers
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError("q, k, v must be bfloat16 or float32, got %s" % t.dtype)


def _check(t, name, shape, dtype, device):
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


_side_streams = {}


def _side_stream(device):
    """One extra torch stream per device (default priority) for the
    backward's operand and serial passes; the current stream is never
    returned."""
    torch = _torch()
    key = torch.device(device).index
    if key is None:
        key = torch.cuda.current_device()
    s = _side_streams.get(key)
    if s is None:
        s = _side_streams[key] = torch.cuda.Stream(device=torch.device("cuda", key))
    if s.cuda_stream == torch.cuda.current_stream(device).cuda_stream:
        return None
    return s


def _check_gate(log_alpha, gate, lead, dk, dev):
    """log_alpha for a gate layout: [*lead, d_k] (channel), [*lead] (head),
    ignored (none; may be None)."""
    torch = _torch()
    code = _gate_code(gate)
    if code == GATES["none"]:
        return None, code
    shape = tuple(lead) + ((dk,) if code == GATES["channel"] else ())
    _check(log_alpha, "log_alpha", shape, torch.float32, dev)
    return log_alpha, code


def prefill(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, scale=None,
            out=None, final_state=True, workspace=None, path="auto", value_tiles=0,
            block_chunks=0, gate="channel", snapshot_tokens=0, snapshots=None,
            l2norm_qk=False, gate_pre=None, gate_scale=1.0, beta_pre=None, chunk_states=None,
            max_seqlen=None, no_alloc=False):
    """Chunked prefill over a packed batch.

    q, k: [T, H, d_k]; v: [T, H, d_v] (bf16 or fp32, same dtype);
    log_alpha: [T, H, d_k] fp32 (gate="channel"), [T, H] fp32 (gate="head")
    or None (gate="none"); beta: [T, H] fp32; h0: [N, H, d_k, d_v] fp32
    or None (zeros); cu_seqlens: int32 [N+1] on the device, or None for one
    sequence of length T.  Returns (o [T, H, d_v] in the input dtype,
    hT [N, H, d_k, d_v] fp32 or None when final_state is False).
    ``final_state`` may also be a preallocated tensor (it may be h0 itself).
    ``path`` ("auto", "vector", "matrix" or "two_pass"), ``value_tiles`` and
    ``block_chunks`` (0 = automatic) are the kda_prefill_options tuning knobs.
    ``snapshot_tokens`` > 0 (a multiple of 64) also records the state after
    every snapshot_tokens tokens of each sequence into ``snapshots``
    [N, capacity, H, d_k, d_v] fp32 (allocated zeroed with capacity
    T // snapshot_tokens when None) and returns (o, hT, snapshots).
    The fused input front-end: ``l2norm_qk`` normalises q and k in the
    kernel; ``gate_pre`` (bf16, log_alpha's layout; log_alpha must be None)
    gives log_alpha = -gate_scale * softplus(gate_pre); ``beta_pre`` (bf16
    [T, H]; beta must be None) gives beta = sigmoid(beta_pre).
    ``chunk_states``: a uint8 device tensor of chunk_states_bytes(T, N, H)
    bytes that receives every chunk's start state, for a later backward()
    on the same inputs (which then skips recomputing this pass).
    ``max_seqlen``: at least the longest sequence (T when cu_seqlens is
    None); None leaves it unknown.  The two-pass path then launches blocks
    for that many tokens only, not for total_T.
    ``no_alloc``: call kda_fwd_prefill_noalloc, whose workspace is the
    library's static device array (``workspace`` must then be None); the
    outputs are still allocated here unless given.
    """
    torch = _torch()
    lib = load_library()
    if q.dim() != 3:
        raise ValueError("q must be [T, H, d_k]")
    T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU (HIP) device")
    dt = q.dtype
    code = _dtype_code(q)
    _check(q, "q", (T, H, dk), dt, dev)
    _check(k, "k", (T, H, dk), dt, dev)
    _check(v, "v", (T, H, dv), dt, dev)
    fe = front_end(l2norm_qk, gate_pre, gate_scale, beta_pre, (T, H), gate, dev)
    if gate_pre is None:
        log_alpha, _ = _check_gate(log_alpha, gate, (T, H), dk, dev)
    elif log_alpha is not None:
        raise ValueError("log_alpha must be None with gate_pre")
    if beta_pre is None:
        _check(beta, "beta", (T, H), torch.float32, dev)
    elif beta is not None:
        raise ValueError("beta must be None with beta_pre")
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, T], dtype=torch.int32, device=dev)
        max_seqlen = T
    if cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be 1-D")
    N = cu_seqlens.shape[0] - 1
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if h0 is not None:
        _check(h0, "h0", (N, H, dk, dv), torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    if out is None:
        out = torch.empty((T, H, dv), dtype=dt, device=dev)
    else:
        _check(out, "out", (T, H, dv), dt, dev)
    if final_state is True:
        hT = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is False or final_state is None:
        hT = None
    else:
        hT = final_state
        _check(hT, "final_state", (N, H, dk, dv), torch.float32, dev)
    opts = prefill_options(path, value_tiles, block_chunks, gate, fe, max_seqlen)
    if snapshot_tokens:
        if snapshots is None:
            cap = max(1, T // int(snapshot_tokens))
            snapshots = torch.zeros((N, cap, H, dk, dv), dtype=torch.float32, device=dev)
        if snapshots.dim() != 5:
            raise ValueError("snapshots must be [N, capacity, H, d_k, d_v]")
        _check(snapshots, "snapshots", (N, snapshots.shape[1], H, dk, dv), torch.float32, dev)
        opts.snapshot_tokens = int(snapshot_tokens)
        opts.snapshot_capacity = int(snapshots.shape[1])
        opts.snapshots = snapshots.data_ptr()
    if chunk_states is not None:
        _check_states(chunk_states, T, N, H, dk, dv, dev)
        opts.chunk_states = chunk_states.data_ptr()
    if no_alloc:
        if workspace is not None:
            raise ValueError("no_alloc takes no workspace")
        st = lib.kda_fwd_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                         _ptr(h0), _ptr(cu_seqlens), T, N, H, dk, dv, code,
                                         float(scale), _ptr(out), _ptr(hT), ctypes.byref(opts),
                                         _stream(dev))
        if st != 0:
            raise KDAError(st, "kda_fwd_prefill_noalloc")
        if snapshot_tokens:
            return out, hT, snapshots
        return out, hT
    need = lib.kda_fwd_prefill_workspace_bytes_ex(T, N, H, dk, dv, code, ctypes.byref(opts))
    if workspace is None:
        workspace = torch.empty((max(int(need), 1),), dtype=torch.uint8, device=dev)
    st = lib.kda_fwd_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                _ptr(h0), _ptr(cu_seqlens), T, N, H, dk, dv, code,
                                float(scale), _ptr(out), _ptr(hT), _ptr(workspace),
                                workspace.numel(), ctypes.byref(opts), _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_fwd_prefill_ex")
    if snapshot_tokens:
        return out, hT, snapshots
    return out, hT


def chunk_states_bytes(total_T: int, N: int, H: int, d_k: int = 128, d_v: int = 128) -> int:
    """Bytes of the per-chunk state record a prefill can write for the
    backward (0 for unsupported sizes)."""
    return int(load_library().kda_chunk_states_bytes(total_T, N, H, d_k, d_v))


def _check_states(chunk_states, T, N, H, dk, dv, dev):
    torch = _torch()
    need = chunk_states_bytes(T, N, H, dk, dv)
    if need == 0:
        raise ValueError("chunk_states needs d_k = d_v = 128")
    if (chunk_states.dtype != torch.uint8 or chunk_states.device != dev
            or not chunk_states.is_contiguous() or chunk_states.numel() < need):
        raise ValueError("chunk_states must be a contiguous uint8 tensor of at least %d bytes "
                         "on %s" % (need, dev))


def decode_step(q, k, v, log_alpha, beta, S, scale=None, out=None, gate="channel",
                state_index=None, l2norm_qk=False, gate_pre=None, gate_scale=1.0,
                beta_pre=None):
    """One decode step.  q, k: [N, H, d_k]; v: [N, H, d_v] (bf16 or fp32);
    log_alpha: [N, H, d_k] fp32 (gate="channel"), [N, H] (gate="head") or
    None (gate="none"); beta: [N, H] fp32; S: [N, H, d_k, d_v] fp32, updated
    in place.  With state_index (int32 [N] on the device) S is a pool
    [num_states, H, d_k, d_v] and sequence n updates S[state_index[n]];
    an index outside the pool skips that sequence (its o is not written).
    The front-end arguments are those of prefill(), over the N tokens.
    Returns o [N, H, d_v] in the input dtype."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 3:
        raise ValueError("q must be [N, H, d_k]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU (HIP) device")
    dt = q.dtype
    code = _dtype_code(q)
    _check(q, "q", (N, H, dk), dt, dev)
    _check(k, "k", (N, H, dk), dt, dev)
    _check(v, "v", (N, H, dv), dt, dev)
    fe = front_end(l2norm_qk, gate_pre, gate_scale, beta_pre, (N, H), gate, dev)
    gcode = _gate_code(gate)
    if gate_pre is None:
        log_alpha, gcode = _check_gate(log_alpha, gate, (N, H), dk, dev)
    elif log_alpha is not None:
        raise ValueError("log_alpha must be None with gate_pre")
    if beta_pre is None:
        _check(beta, "beta", (N, H), torch.float32, dev)
    elif beta is not None:
        raise ValueError("beta must be None with beta_pre")
    if state_index is None:
        _check(S, "S", (N, H, dk, dv), torch.float32, dev)
        nstates = N
    else:
        _check(state_index, "state_index", (N,), torch.int32, dev)
        if S.dim() != 4:
            raise ValueError("S must be [num_states, H, d_k, d_v]")
        nstates = S.shape[0]
        _check(S, "S", (nstates, H, dk, dv), torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    if out is None:
        out = torch.empty((N, H, dv), dtype=dt, device=dev)
    else:
        _check(out, "out", (N, H, dv), dt, dev)
    opts = DecodeOptions(gcode, nstates, None if state_index is None else state_index.data_ptr())
    if fe is not None:
        opts.front = fe
    st = lib.kda_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                _ptr(S), N, H, dk, dv, code, float(scale), _ptr(out),
                                ctypes.byref(opts), _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_decode_step_ex")
    return out


def decode_multi(q, k, v, log_alpha, beta, S, scale=None, out=None, outputs=True,
                 write_state=True, lengths=None, gate="channel", state_index=None,
                 l2norm_qk=False, gate_pre=None, gate_scale=1.0, beta_pre=None):
    """m decode tokens per sequence in one pass over the states.

    q, k: [N, m, H, d_k]; v: [N, m, H, d_v] (bf16 or fp32); log_alpha:
    [N, m, H, d_k] fp32 (gate="channel"), [N, m, H] (gate="head") or None
    (gate="none"); beta: [N, m, H] fp32; S: [N, H, d_k, d_v] fp32, or a pool
    [num_states, H, d_k, d_v] with state_index (int32 [N] on the device).
    Sequence n applies its first lengths[n] tokens (int32 [N] on the device,
    clamped to [0, m]; None = all m).  With ``outputs`` the outputs of the
    applied tokens are written into ``out`` (allocated when None) and
    returned; with ``write_state`` S is advanced in place past the applied
    tokens.  Verify draft tokens with write_state=False, commit an accepted
    prefix with outputs=False and lengths.  The fused input front-end per
    token as for decode_step() (gate_pre in log_alpha's layout, beta_pre
    [N, m, H] bf16)."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [N, m, H, d_k]")
    N, m, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU (HIP) device")
    dt = q.dtype
    code = _dtype_code(q)
    _check(q, "q", (N, m, H, dk), dt, dev)
    _check(k, "k", (N, m, H, dk), dt, dev)
    _check(v, "v", (N, m, H, dv), dt, dev)
    fe = front_end(l2norm_qk, gate_pre, gate_scale, beta_pre, (N, m, H), gate, dev)
    if gate_pre is None:
        log_alpha, gcode = _check_gate(log_alpha, gate, (N, m, H), dk, dev)
    elif log_alpha is not None:
        raise ValueError("log_alpha must be None with gate_pre")
    else:
        gcode = _gate_code(gate)
    if beta_pre is None:
        _check(beta, "beta", (N, m, H), torch.float32, dev)
    elif beta is not None:
        raise ValueError("beta must be None with beta_pre")
    if state_index is None:
        _check(S, "S", (N, H, dk, dv), torch.float32, dev)
        nstates = N
    else:
        _check(state_index, "state_index", (N,), torch.int32, dev)
        if S.dim() != 4:
            raise ValueError("S must be [num_states, H, d_k, d_v]")
        nstates = S.shape[0]
        _check(S, "S", (nstates, H, dk, dv), torch.float32, dev)
    if lengths is not None:
        _check(lengths, "lengths", (N,), torch.int32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    if not outputs:
        out = None
    elif out is None:
        out = torch.empty((N, m, H, dv), dtype=dt, device=dev)
    else:
        _check(out, "out", (N, m, H, dv), dt, dev)
    opts = DecodeMultiOptions(gcode, nstates,
                              None if state_index is None else state_index.data_ptr(),
                              None if lengths is None else lengths.data_ptr(),
                              1 if write_state else 0, fe if fe is not None else FrontEnd())
    st = lib.kda_decode_multi(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S),
                              N, m, H, dk, dv, code, float(scale), _ptr(out),
                              ctypes.byref(opts), _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_decode_multi")
    return out


def backward_workspace_bytes(total_T: int, N: int, H: int, d_k: int, d_v: int,
                             dtype: int = DTYPE_BF16, gate="channel", block_chunks=0,
                             l2norm_qk=False, gate_pre=False, beta_pre=False,
                             chunk_states=False, max_seqlen=0) -> int:
    """The front-end flags and chunk_states say which options the call will
    use (their tensors are not needed here)."""
    dummy = ctypes.c_void_p(16)
    fe = FrontEnd(1 if l2norm_qk else 0, 1.0, dummy if gate_pre else None,
                  dummy if beta_pre else None)
    opts = BwdOptions(_gate_code(gate), block_chunks, fe, dummy if chunk_states else None,
                      int(max_seqlen or 0))
    return int(load_library().kda_bwd_workspace_bytes(total_T, N, H, d_k, d_v, dtype,
                                                      ctypes.byref(opts)))


def backward(q, k, v, log_alpha, beta, do, h0=None, dhT=None, cu_seqlens=None, scale=None,
             gate="channel", want_dh0=True, block_chunks=0, workspace=None,
             l2norm_qk=False, gate_pre=None, gate_scale=1.0, beta_pre=None, chunk_states=None,
             max_seqlen=None, aux_stream="auto"):
    """Gradients of <o, do> + <hT, dhT> for the prefill on these inputs.

    Inputs as for prefill() (bf16 q, k, v with d_k = d_v = 128); do: [T, H,
    d_v] bf16, the adjoint of o; dhT: [N, H, d_k, d_v] fp32 or None (zeros).
    Returns a dict: dq, dk, dv (bf16, the shapes of q, k, v), dlog_alpha
    (fp32, the layout of log_alpha; None without a gate), dbeta [T, H]
    fp32, dh0 [N, H, d_k, d_v] fp32 (None when want_dh0 is False).

    The fused input front-end as for prefill(): with it, dq and dk are the
    gradients with respect to the raw q and k, dlog_alpha with respect to
    gate_pre (fp32, its layout) and dbeta with respect to beta_pre.
    ``chunk_states``: the record a prefill(..., chunk_states=...) call wrote
    on these same inputs (with the same front-end options); the forward
    pass is then not recomputed.
    ``max_seqlen`` as for prefill().  ``aux_stream``: a torch stream of the
    device for the per-block operand and serial passes, which then overlap
    the gradient pass on the current stream; "auto" takes one side stream
    per device kept by this module (default priority); None runs the whole
    call in order on the current stream.  The gradients are the same bits
    either way."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 3:
        raise ValueError("q must be [T, H, d_k]")
    T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU (HIP) device")
    dt = q.dtype
    code = _dtype_code(q)
    _check(q, "q", (T, H, dk), dt, dev)
    _check(k, "k", (T, H, dk), dt, dev)
    _check(v, "v", (T, H, dv), dt, dev)
    _check(do, "do", (T, H, dv), dt, dev)
    fe = front_end(l2norm_qk, gate_pre, gate_scale, beta_pre, (T, H), gate, dev)
    if gate_pre is None:
        log_alpha, gcode = _check_gate(log_alpha, gate, (T, H), dk, dev)
        la_like = log_alpha
    elif log_alpha is not None:
        raise ValueError("log_alpha must be None with gate_pre")
    else:
        gcode = _gate_code(gate)
        la_like = torch.empty(gate_pre.shape, dtype=torch.float32, device=dev)
    if beta_pre is None:
        _check(beta, "beta", (T, H), torch.float32, dev)
    elif beta is not None:
        raise ValueError("beta must be None with beta_pre")
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, T], dtype=torch.int32, device=dev)
        max_seqlen = T
    _check(cu_seqlens, "cu_seqlens", (cu_seqlens.shape[0],), torch.int32, dev)
    N = cu_seqlens.shape[0] - 1
    if h0 is not None:
        _check(h0, "h0", (N, H, dk, dv), torch.float32, dev)
    if dhT is not None:
        _check(dhT, "dhT", (N, H, dk, dv), torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dlog_alpha=None if la_like is None else torch.empty_like(la_like),
               dbeta=torch.empty((T, H), dtype=torch.float32, device=dev),
               dh0=torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if want_dh0 else None)
    opts = BwdOptions(gcode, block_chunks, fe if fe is not None else FrontEnd())
    opts.max_seqlen = int(max_seqlen or 0)
    if aux_stream == "auto":
        aux_stream = _side_stream(dev)
    if aux_stream is not None:
        if aux_stream.device != dev:
            raise ValueError("aux_stream must be a stream of %s" % dev)
        opts.aux_stream = aux_stream.cuda_stream
    if chunk_states is not None:
        _check_states(chunk_states, T, N, H, dk, dv, dev)
        opts.chunk_states = chunk_states.data_ptr()
    need = int(lib.kda_bwd_workspace_bytes(T, N, H, dk, dv, code, ctypes.byref(opts)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.kda_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0),
                     _ptr(cu_seqlens), T, N, H, dk, dv, code, float(scale), _ptr(do), _ptr(dhT),
                     _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]),
                     _ptr(out["dbeta"]), _ptr(out["dh0"]), _ptr(workspace), workspace.numel(),
                     ctypes.byref(opts), _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_bwd")
    return out
