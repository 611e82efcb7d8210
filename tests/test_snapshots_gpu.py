"""GPU checks of prefill state snapshots (prefix caching), through the C ABI.

With snapshot_tokens = 64 and a capacity of 4, snapshot j of sequence n is
the state after its first (j+1)*64 tokens.  On every prefill path:
  * bitwise equal to the final state of a prefill of that prefix alone
    (same path and value tiles; the prefixes are packed as their own batch);
  * within the parity bar of the fp64 oracle's final state of the prefix;
  * entries past a sequence's last snapshot are left untouched.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_05_amd as kda
import kda_inputs as gen
import oracle
from kda_testutil import host, rel_err, report, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda"
SNAP, CAP = 64, 4
LENS = [300, 64, 1, 129, 0, 256, 200]
PATHS = [("f32", "vector", 64, 0), ("bf16", "matrix", 128, 4), ("bf16", "matrix", 128, 1),
         ("bf16", "two_pass", 128, 8)]


@pytest.mark.parametrize("dtype,path,d,tiles", PATHS)
def test_snapshots_are_prefix_states(dtype, path, d, tiles):
    H = 2
    inp = gen.prefill_inputs(LENS, H, d, d, dtype, "softplus", state_std=0.05, seed=96,
                             device=DEV)
    N = len(LENS)
    sentinel = 5.0
    snaps = torch.full((N, CAP, H, d, d), sentinel, dtype=torch.float32, device=DEV)
    o, hT, snaps = kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                               h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], path=path,
                               value_tiles=tiles, snapshot_tokens=SNAP, snapshots=snaps)
    # the plain call gives the same o and hT
    o0, hT0 = kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                          h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], path=path,
                          value_tiles=tiles)
    assert torch.equal(o, o0) and torch.equal(hT, hT0)

    # every prefix that ends on a snapshot, packed as its own batch
    cu = np.concatenate([[0], np.cumsum(LENS)])
    pairs = [(n, j) for n in range(N) for j in range(CAP) if (j + 1) * SNAP <= LENS[n]]
    idx = np.concatenate([np.arange(cu[n], cu[n] + (j + 1) * SNAP) for n, j in pairs])
    sel = torch.tensor(idx, device=DEV)
    plens = [(j + 1) * SNAP for _, j in pairs]
    pcu = torch.tensor(np.concatenate([[0], np.cumsum(plens)]), dtype=torch.int32, device=DEV)
    ph0 = inp["h0"][torch.tensor([n for n, _ in pairs], device=DEV)].contiguous()
    sub = {kk: inp[kk][sel].contiguous() for kk in ("q", "k", "v", "log_alpha", "beta")}
    _, phT = kda.prefill(sub["q"], sub["k"], sub["v"], sub["log_alpha"], sub["beta"], h0=ph0,
                         cu_seqlens=pcu, path=path, value_tiles=tiles)
    got = torch.stack([snaps[n, j] for n, j in pairs])
    assert torch.equal(got, phT)

    # ... and the oracle's final state of each prefix
    _, h_ref = oracle.prefill(host(sub["q"]), host(sub["k"]), host(sub["v"]),
                              host(sub["log_alpha"]), host(sub["beta"]), h0=host(ph0),
                              cu_seqlens=np.asarray(pcu.cpu(), dtype=np.int64))
    err = rel_err(host(got), h_ref)
    report("snapshots %s %s (%d prefixes)" % (dtype, path, len(pairs)), snap=err)
    assert err <= tol_for(dtype)

    # entries no prefix reached are untouched
    taken = set(pairs)
    for n in range(N):
        for j in range(CAP):
            if (n, j) not in taken:
                assert bool((snaps[n, j] == sentinel).all()), (n, j)
