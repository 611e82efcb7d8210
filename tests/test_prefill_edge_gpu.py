"""GPU parity of kda_fwd_prefill on edge cases of the gates and the batch,
for every kernel path, against the fp64 oracle (through the C ABI).

Gates: no decay with beta = 1 (DeltaNet with full writes); beta = 0 (the
state only decays: outputs read the decayed initial state); per-token
gates of -1.2 on every channel, so the summed gate over a 64-token chunk
reaches -76.8, next to the -80 bound the library documents for its factored
exponentials; and a mix of undecayed and strongly decayed channels.

Batch: 200 short sequences (lengths 0..150, empty ones included, non-zero
initial states), through each path; on the two-pass path this also walks
many short blocks of chunks.

Bars: max-relative error <= 1e-5 (fp32 inputs) or 2e-2 (bf16 inputs) on o
and on the final states.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_05_amd as kda
import kda_inputs as gen
from kda_testutil import host, oracle_prefill, rel_err, report, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (dtype, path): the fp32 vector path and both bf16 matrix paths
PATHS = [("f32", "vector"), ("bf16", "matrix"), ("bf16", "two_pass")]


def run(inp, path):
    return kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                       h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], path=path)


def check(inp, path, dtype, name):
    o, hT = run(inp, path)
    o_ref, h_ref = oracle_prefill(inp)
    eo, eh = rel_err(host(o), o_ref), rel_err(host(hT), h_ref)
    report("%s %s" % (name, path), o=eo, hT=eh)
    tol = tol_for(dtype)
    assert eo <= tol and eh <= tol
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()


def gate_case(inp, case):
    la = inp["log_alpha"]
    if case == "no_decay_beta1":
        la.zero_()
        inp["beta"].fill_(1.0)
    elif case == "beta0":
        inp["beta"].zero_()
    elif case == "strong_decay":
        la.fill_(-1.2)
    elif case == "mixed":
        la[:, :, 0::2] = 0.0
        la[:, :, 1::2] = -1.2
    return inp


@pytest.mark.parametrize("dtype,path", PATHS)
@pytest.mark.parametrize("case", ["no_decay_beta1", "beta0", "strong_decay", "mixed"])
def test_degenerate_gates(dtype, path, case):
    inp = gen.prefill_inputs([300, 64, 1, 129], 2, 128, 128, dtype, "uniform", state_std=0.1,
                             seed=80, device=DEV)
    check(gate_case(inp, case), path, dtype, "gates %s" % case)


@pytest.mark.parametrize("dtype,path", PATHS)
def test_many_short_sequences(dtype, path):
    rng = np.random.default_rng(81)
    lens = rng.integers(0, 151, 200)
    lens[::17] = 0
    inp = gen.prefill_inputs(lens, 2, 128, 64, dtype, "softplus", state_std=0.05, seed=82,
                             device=DEV)
    check(inp, path, dtype, "200 short sequences")
