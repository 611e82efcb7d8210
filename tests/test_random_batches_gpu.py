"""GPU parity on seeded random batches that mix every form a chunk can take.

Each case draws (from its seed) the number of sequences, their lengths
(ragged, empty ones allowed), the number of heads, whether there is an
initial state, and for every 64-token chunk of every sequence one kind of
gate: the generator's own (inside the factored range), a strong constant
per-token decay whose 16-row blocks stay inside the range (the blocked
form), a stronger one that leaves it within a block (the pairwise form),
independent per-element gates in [-6, 0], or strong decay on one 16-row
block only.  The gate domain is the pages' (any per-channel alpha in
(0, 1], "Kimi Delta Attention: la atencion lineal detras de Kimi K2 y
Qwen3", section "Cómo funciona Kimi Delta Attention paso a paso"), and the
ragged batches are those of the varlen path.  Every prefill path and the
backward are compared with the fp64 oracle, including the worst single
(sequence, head) slice of o.
"""
import os

import numpy as np
import pytest
import torch

import gated_delta_rule_05_amd as kda
import kda_inputs as gen
import oracle
from kda_testutil import host, oracle_prefill, rel_err, rel_err_slices, report, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda"

PATHS = [("f32", "vector"), ("bf16", "matrix"), ("bf16", "two_pass")]
# KDA_RANDOM_SEEDS=n adds n more seeded prefill cases (and n // 5 backward
# cases) for a longer sweep; the default run keeps the fixed seeds only
EXTRA = int(os.environ.get("KDA_RANDOM_SEEDS", "0"))
PREFILL_SEEDS = [501, 502, 503, 504, 505, 506] + [10_000 + i for i in range(EXTRA)]
BACKWARD_SEEDS = [511, 512, 513, 514] + [20_000 + i for i in range(EXTRA // 5)]


def random_case(seed, dtype):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 6))
    lens = [int(x) for x in rng.integers(0, 260, size=N)]
    if sum(lens) == 0:
        lens[0] = 1
    H = int(rng.integers(1, 4))
    std = float(rng.choice([0.0, 0.1]))
    inp = gen.prefill_inputs(lens, H, 128, 128, dtype, "uniform", state_std=std, seed=seed,
                             device=DEV)
    la = inp["log_alpha"]
    cu = inp["cu_seqlens"].cpu().tolist()
    kinds = []
    for n in range(N):
        for c0 in range(cu[n], cu[n + 1], 64):
            c1 = min(c0 + 64, cu[n + 1])
            kind = int(rng.integers(0, 5))
            kinds.append(kind)
            if kind == 1:        # every 16-row block inside the range, the chunk not
                la[c0:c1] = -float(rng.uniform(1.5, 4.5))
            elif kind == 2:      # a 16-row block beyond the range
                la[c0:c1] = -float(rng.uniform(6.0, 12.0))
            elif kind == 3:      # independent per-element gates
                x = rng.uniform(0.0, 6.0, size=(c1 - c0, H, 128))
                la[c0:c1] = torch.from_numpy(-x).to(la.dtype).to(DEV)
            elif kind == 4:      # one strong 16-row block, mild elsewhere
                la[c0:c1] = -0.05
                b0 = c0 + 16 * int(rng.integers(0, 4))
                la[b0:min(b0 + 16, c1)] = -float(rng.uniform(6.0, 9.0))
    return inp, lens, kinds


@pytest.mark.parametrize("seed", PREFILL_SEEDS)
@pytest.mark.parametrize("dtype,path", PATHS)
def test_random_batch_prefill(dtype, path, seed):
    inp, lens, kinds = random_case(seed, dtype)
    o, hT = kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                        h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], path=path)
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()
    o_ref, h_ref = oracle_prefill(inp)
    cu = inp["cu_seqlens"].cpu().numpy()
    eo, eh = rel_err(host(o), o_ref), rel_err(host(hT), h_ref)
    ew = rel_err_slices(host(o), o_ref, cu)
    report("random %d %s (lengths %s, chunk kinds %s)" % (seed, path, lens, kinds),
           o=eo, hT=eh, o_worst_slice=ew)
    tol = tol_for(dtype)
    assert eo <= tol and eh <= tol and ew <= tol


@pytest.mark.parametrize("seed", BACKWARD_SEEDS)
def test_random_batch_backward(seed):
    inp, lens, kinds = random_case(seed, "bf16")
    T, H = inp["q"].shape[:2]
    N = len(lens)
    do = gen.normal((T, H, 128), seed, gen.DO, DEV, torch.bfloat16)
    dhT = gen.normal((N, H, 128, 128), seed, gen.DHT, DEV, torch.float32, std=0.1)
    g = kda.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], do,
                     h0=inp["h0"], dhT=dhT, cu_seqlens=inp["cu_seqlens"])
    for key, x in g.items():
        assert x is None or torch.isfinite(x).all(), key
    cu = inp["cu_seqlens"].cpu().numpy().astype(np.int64)
    r = oracle.backward(host(inp["q"]), host(inp["k"]), host(inp["v"]), host(inp["log_alpha"]),
                        host(inp["beta"]), host(do), h0=host(inp["h0"]), dhT=host(dhT),
                        cu_seqlens=cu)
    errs = {}
    for key in ("dq", "dk", "dv", "dbeta", "dh0"):
        if r[key] is not None:
            errs[key] = rel_err(host(g[key]), r[key])
    # dlog_alpha is a difference of terms of the size of q dq and k dk:
    # measured against the larger of its own magnitude and theirs
    terms = max(float(np.max(np.abs(r["dq"] * host(inp["q"])))),
                float(np.max(np.abs(r["dk"] * host(inp["k"])))))
    errs["dlog_alpha"] = float(np.max(np.abs(host(g["dlog_alpha"]) - r["dlog_alpha"]))) / max(
        float(np.max(np.abs(r["dlog_alpha"]))), terms)
    report("random backward %d (lengths %s, chunk kinds %s)" % (seed, lens, kinds), **errs)
    for key, e in errs.items():
        assert e <= tol_for("bf16"), (key, e)
