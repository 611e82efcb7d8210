"""GPU parity of the prefill gradients (kda_bwd), through the C ABI.

The gradients of L = <o, dO> + <hT, dhT> with respect to q, k, v,
log_alpha, beta and h0, against the fp64 gradient oracle (the reverse-mode
derivative of the token loop, pinned by finite differences of the forward
oracle) on the same stored inputs.  Cases: ragged packed batches with
empty and one-token sequences and partial last chunks, non-zero h0 and
dhT, all three gate layouts; zero h0 / dhT; sampled heads of the
4 x 4096 x 16 batch.  Properties: the block length of the backward walk
does not change a bit; two runs agree bitwise.

Bar: max-relative error <= 2e-2 per gradient tensor (bf16 inputs, fp32
states and adjoints), the bar of the forward pass.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_05_amd as kda
import kda_inputs as gen
import oracle
from kda_testutil import host, rel_err, report

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2
LENS = [300, 64, 1, 129, 0, 77]


def case(lens, H, seed, gate="channel", h0=True, dhT=True):
    inp = gen.prefill_inputs(lens, H, 128, 128, "bf16", "softplus", state_std=0.05 if h0 else 0.0,
                             seed=seed, device=DEV)
    T = inp["q"].shape[0]
    N = len(lens)
    if gate == "head":
        inp["log_alpha"] = gen.gates((T, H), seed + 1, DEV, "uniform").contiguous()
    elif gate == "none":
        inp["log_alpha"] = None
    if not h0:
        inp["h0"] = None
    inp["do"] = gen.normal((T, H, 128), seed, gen.DO, DEV, torch.bfloat16)
    inp["dhT"] = gen.normal((N, H, 128, 128), seed, gen.DHT, DEV, torch.float32, std=0.1) if dhT else None
    return inp


def gpu(inp, gate, **kw):
    return kda.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["do"],
                        h0=inp["h0"], dhT=inp["dhT"], cu_seqlens=inp["cu_seqlens"], gate=gate, **kw)


def ref(inp, heads=None):
    sel = (lambda x: x) if heads is None else (lambda x: x[:, heads])
    sel_s = (lambda x: x) if heads is None else (lambda x: x[:, heads])
    cu = inp["cu_seqlens"].cpu().numpy().astype(np.int64)
    la = inp["log_alpha"]
    return oracle.backward(sel(host(inp["q"])), sel(host(inp["k"])), sel(host(inp["v"])),
                           None if la is None else sel(host(la)), sel(host(inp["beta"])),
                           sel(host(inp["do"])),
                           h0=None if inp["h0"] is None else sel_s(host(inp["h0"])),
                           dhT=None if inp["dhT"] is None else sel_s(host(inp["dhT"])),
                           cu_seqlens=cu)


def compare(name, g, r, heads=None):
    sel = (lambda x: x) if heads is None else (lambda x: x[:, heads])
    errs = {}
    for key in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0"):
        if r[key] is None:
            assert g[key] is None
            continue
        errs[key] = rel_err(sel(host(g[key])), r[key])
    report(name, **errs)
    for key, e in errs.items():
        assert e <= TOL, (key, e)


@pytest.mark.parametrize("gate", ["channel", "head", "none"])
def test_backward_parity(gate):
    inp = case(LENS, 2, 300, gate)
    compare("backward %s" % gate, gpu(inp, gate), ref(inp))


def test_backward_zero_state_and_adjoint():
    inp = case([200, 64, 5], 2, 310, h0=False, dhT=False)
    compare("backward h0=0 dhT=0", gpu(inp, "channel"), ref(inp))


def test_backward_block_invariance_and_determinism():
    inp = case(LENS, 2, 320)
    base = gpu(inp, "channel")
    for blk in (1, 2, 3):
        other = gpu(inp, "channel", block_chunks=blk)
        for key, x in base.items():
            assert torch.equal(x, other[key]), (blk, key)
    again = gpu(inp, "channel")
    for key, x in base.items():
        assert torch.equal(x, again[key]), key


def test_backward_batch4_t4096_sampled_heads():
    w = gen.WORKLOADS["batch4_t4096"]
    inp = gen.workload_prefill_inputs(w, seed=330, device=DEV)
    T, H = inp["q"].shape[:2]
    N = inp["cu_seqlens"].shape[0] - 1
    inp["do"] = gen.normal((T, H, 128), 330, gen.DO, DEV, torch.bfloat16)
    inp["dhT"] = gen.normal((N, H, 128, 128), 330, gen.DHT, DEV, torch.float32, std=0.1)
    g = gpu(inp, "channel")
    heads = [0, 11]
    compare("backward batch4_t4096 heads %s" % heads, g, ref(inp, heads), heads)


def test_backward_long_t1m_last_window():
    """The 1M-token backward in the configuration bench.py times, checked on
    the last 8192 tokens of two heads: the oracle's backward over that
    window starts from the state the forward reaches at its first token (a
    snapshot of the same two-pass forward the backward recomputes, so the
    same bits) and takes the same dO and dhT; every gradient of a token in
    the window depends on nothing else."""
    w = gen.WORKLOADS["long_t1m"]
    inp = gen.workload_prefill_inputs(w, seed=340, device=DEV)
    T, H = inp["q"].shape[:2]
    W, heads = 8192, [3, 30]
    t0 = T - W
    do = gen.normal((T, H, 128), 340, gen.DO, DEV, torch.bfloat16)
    dhT = gen.normal((1, H, 128, 128), 340, gen.DHT, DEV, torch.float32, std=0.1)
    args = (inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"])
    g = kda.backward(*args, do, dhT=dhT, cu_seqlens=inp["cu_seqlens"], want_dh0=False)
    win = {key: host(x[t0:, heads]) for key, x in g.items() if x is not None}
    del g
    torch.cuda.empty_cache()
    _, _, snaps = kda.prefill(*args, cu_seqlens=inp["cu_seqlens"], final_state=False,
                              snapshot_tokens=t0)
    S0 = host(snaps[:, 0][:, heads])
    del snaps
    sel = lambda x: host(x[t0:, heads])
    ref = oracle.backward(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["log_alpha"]),
                          sel(inp["beta"]), sel(do), h0=S0, dhT=host(dhT[:, heads]))
    errs = {key: rel_err(win[key], ref[key]) for key in ("dq", "dk", "dv", "dlog_alpha", "dbeta")}
    report("backward long_t1m last %d tokens, heads %s" % (W, heads), **errs)
    for key, e in errs.items():
        assert e <= TOL, (key, e)


def test_backward_on_a_side_stream():
    """The call on a non-default stream (the library forks its serial pass
    onto a second stream of that stream's device and joins back): the same
    bits as on the default stream, complete once that stream is done."""
    inp = case(LENS, 2, 350)
    base = gpu(inp, "channel")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        other = gpu(inp, "channel")
    side.synchronize()
    for key, x in base.items():
        assert torch.equal(x, other[key]), key


@pytest.mark.parametrize("gate", ["channel", "head", "none"])
def test_backward_from_saved_chunk_states(gate):
    """A prefill that also writes the per-chunk state record gives the same
    o and hT as one that does not, and the backward that reads the record
    gives the same bits as the one that recomputes the forward pass."""
    inp = case(LENS, 2, 360, gate)
    T, N = inp["q"].shape[0], len(LENS)
    args = (inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"])
    kw = dict(h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], gate=gate)
    rec = torch.empty(kda.chunk_states_bytes(T, N, 2), dtype=torch.uint8, device=DEV)
    o0, hT0 = kda.prefill(*args, path="two_pass", **kw)
    o1, hT1 = kda.prefill(*args, chunk_states=rec, **kw)
    assert torch.equal(o0, o1) and torch.equal(hT0, hT1)
    base = gpu(inp, gate)
    other = gpu(inp, gate, chunk_states=rec)
    for key, x in base.items():
        assert (x is None) == (other[key] is None), key
        if x is not None:
            assert torch.equal(x, other[key]), key


def test_backward_from_saved_chunk_states_batch4_t4096():
    """The same on the 4 x 4096 x 16 batch, whose forward takes 32-column
    value tiles where the backward's own recompute takes 16-column ones:
    each state column is computed alone, so the record is the same bits."""
    w = gen.WORKLOADS["batch4_t4096"]
    inp = gen.workload_prefill_inputs(w, seed=370, device=DEV)
    T, H = inp["q"].shape[:2]
    N = inp["cu_seqlens"].shape[0] - 1
    inp["do"] = gen.normal((T, H, 128), 370, gen.DO, DEV, torch.bfloat16)
    inp["dhT"] = gen.normal((N, H, 128, 128), 370, gen.DHT, DEV, torch.float32, std=0.1)
    rec = torch.empty(kda.chunk_states_bytes(T, N, H), dtype=torch.uint8, device=DEV)
    kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=inp["h0"],
                cu_seqlens=inp["cu_seqlens"], chunk_states=rec)
    base = gpu(inp, "channel")
    other = gpu(inp, "channel", chunk_states=rec)
    for key, x in base.items():
        assert torch.equal(x, other[key]), key
