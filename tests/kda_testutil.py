"""Helpers shared by the GPU parity tests: error metric, tolerances, host
copies and calls into the oracle."""
import numpy as np
import torch

import oracle

# Parity bars: max-relative error of each output tensor against the fp64
# oracle on identical stored inputs.
TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def tol_for(dtype):
    return TOL_F32 if dtype in ("f32", torch.float32) else TOL_BF16


def rel_err(x, ref):
    """max |x - ref| / max |ref| over the whole tensor."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    denom = max(float(np.max(np.abs(ref))), 1e-30)
    return float(np.max(np.abs(x - ref))) / denom


def rel_err_slices(x, ref, cu, states=False):
    """Worst max-relative error over the (sequence, head) slices of a packed
    tensor: o / gradients [T, H, .] sliced by cu_seqlens, or (states=True)
    [N, H, ...] per state.  Each slice is measured against its own largest
    magnitude, so a small-magnitude head cannot hide behind a large one."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    cu = np.asarray(cu, dtype=np.int64)
    worst = 0.0
    for n in range(len(cu) - 1):
        for h in range(ref.shape[1]):
            if states:
                a, b = x[n, h], ref[n, h]
            else:
                a, b = x[cu[n]:cu[n + 1], h], ref[cu[n]:cu[n + 1], h]
            if b.size == 0 or not np.any(b):
                # an empty slice, or an exactly-zero reference: must match exactly
                if b.size and np.any(a != b):
                    return float("inf")
                continue
            worst = max(worst, rel_err(a, b))
    return worst


def host(t):
    """Device tensor -> float64 numpy (bf16 and fp32 widen exactly)."""
    if t is None:
        return None
    return t.detach().to(torch.float64).cpu().numpy()


def oracle_prefill(inp, scale=None, threads=0):
    cu = inp["cu_seqlens"].cpu().numpy().astype(np.int64)
    return oracle.prefill(host(inp["q"]), host(inp["k"]), host(inp["v"]),
                          host(inp["log_alpha"]), host(inp["beta"]), h0=host(inp["h0"]),
                          cu_seqlens=cu, scale=scale, threads=threads)


def report(name, **errs):
    print("[parity] %s " % name + " ".join("%s=%.3e" % kv for kv in errs.items()), flush=True)
