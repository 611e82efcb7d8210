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
    return make_case(lens, H, seed, gate, h0, dhT)


def make_case(lens, H, seed, gate="channel", h0=True, dhT=True):
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


def compare(name, g, r, heads=None, skip=()):
    sel = (lambda x: x) if heads is None else (lambda x: x[:, heads])
    errs = {}
    for key in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0"):
        if key in skip:
            continue
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


@pytest.mark.parametrize("case", ["decay_1", "decay_3", "decay_10", "mixed_0_10", "uniform_12", "tiers"])
def test_backward_gate_domain(case):
    """The whole gate domain the pages allow (any alpha in (0, 1]): -1 per
    token keeps a 64-token chunk inside the factored form's range (its gates
    sum to -64); -3 per token leaves it with every 16-row block inside (the
    blocked form); -10 per token, a mix of undecayed and -10 channels, and
    gates uniform in [-12, 0] leave it by 16-row blocks too (the pairwise
    form); "tiers" mixes the three forms chunk by chunk.  Every gradient must
    match the oracle and be finite."""
    inp = make_case(LENS, 2, 390)
    la = inp["log_alpha"]
    if case == "tiers":
        # by (chunk index + sequence) mod 4: -0.1 (factored), -3 (blocked),
        # -10 on rows 16..31 only (pairwise), channels alternating 0 and
        # -4.5 (blocked, with 16-row blocks spanning 72 nats)
        cu = inp["cu_seqlens"].cpu().tolist()
        for n in range(len(cu) - 1):
            for c0 in range(cu[n], cu[n + 1], 64):
                c1 = min(c0 + 64, cu[n + 1])
                kind = ((c0 - cu[n]) // 64 + n) % 4
                if kind == 0:
                    la[c0:c1] = -0.1
                elif kind == 1:
                    la[c0:c1] = -3.0
                elif kind == 2:
                    la[c0:c1] = -0.1
                    la[c0 + 16:min(c0 + 32, c1)] = -10.0
                else:
                    la[c0:c1, :, 0::2] = 0.0
                    la[c0:c1, :, 1::2] = -4.5
    elif case == "decay_1":
        la.fill_(-1.0)
    elif case == "decay_3":
        la.fill_(-3.0)
    elif case == "decay_10":
        la.fill_(-10.0)
    elif case == "mixed_0_10":
        la[..., 0::2] = 0.0
        la[..., 1::2] = -10.0
    else:
        g = torch.Generator(device="cpu").manual_seed(391)
        la.copy_(-12.0 * torch.rand(la.shape, generator=g))
    g = gpu(inp, "channel")
    for key, x in g.items():
        assert x is None or torch.isfinite(x).all(), key
    r = ref(inp)
    compare("backward gates %s" % case, g, r, skip=("dlog_alpha",))
    # dlog_alpha is a difference of products of the gradients of q and k
    # with q and k (the terms the gate's factors e^{+-g} multiply); under
    # strong decay the difference is many times smaller than its terms, and
    # the bf16 rounding of those terms bounds its error: measure it against
    # the larger of its own magnitude and theirs
    terms = max(float(np.max(np.abs(r["dq"] * host(inp["q"])))),
                float(np.max(np.abs(r["dk"] * host(inp["k"])))))
    dla, dla_ref = host(g["dlog_alpha"]), r["dlog_alpha"]
    err = float(np.max(np.abs(dla - dla_ref)))
    scale_ = max(float(np.max(np.abs(dla_ref))), terms)
    report("backward gates %s dlog_alpha (max |ref| %.3e, max |q dq|, |k dk| %.3e)"
           % (case, float(np.max(np.abs(dla_ref))), terms), dlog_alpha=err / scale_)
    assert err / scale_ <= TOL


@pytest.mark.parametrize("strength", [-3.0, -12.0])
def test_backward_head_gate_beyond_factored_range(strength):
    """Gated DeltaNet's one gate per (token, head) beyond the factored range:
    -3 per token keeps every 16-row block inside it (the blocked form), -12
    does not (the pairwise form).  The per-head gate's own kernels; every
    gradient matches the oracle and is finite (dlog_alpha against the
    magnitude of the terms it is a difference of, as for channel gates)."""
    inp = make_case(LENS, 2, 395, gate="head")
    inp["log_alpha"].fill_(strength)
    g = gpu(inp, "head")
    for key, x in g.items():
        assert x is None or torch.isfinite(x).all(), key
    r = ref(inp)
    compare("backward head gate %g" % strength, g, r, skip=("dlog_alpha",))
    # the head's gate sums its channels' terms: their per-row sums set the scale
    terms = max(float(np.max(np.sum(np.abs(r["dq"] * host(inp["q"])), axis=-1))),
                float(np.max(np.sum(np.abs(r["dk"] * host(inp["k"])), axis=-1))))
    dla, dla_ref = host(g["dlog_alpha"]), r["dlog_alpha"]
    err = float(np.max(np.abs(dla - dla_ref))) / max(float(np.max(np.abs(dla_ref))), terms)
    report("backward head gate %g dlog_alpha" % strength, dlog_alpha=err)
    assert err <= TOL


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
    window starts from the oracle's own forward state at the window's first
    token (the GPU forward's snapshot there is checked against it too) and
    takes the same dO and dhT; every gradient of a token in the window
    depends on nothing else.  dh0 of the whole sequence is checked against
    the oracle's backward over the first 8192 tokens with no adjoint
    entering at their end: whatever later tokens send back is decayed by
    the 8192 tokens' gates (about -0.04 per token and channel, so a factor
    near e^-300) before it reaches h0."""
    w = gen.WORKLOADS["long_t1m"]
    inp = gen.workload_prefill_inputs(w, seed=340, device=DEV)
    T, H = inp["q"].shape[:2]
    W, heads = 8192, [3, 30]
    t0 = T - W
    do = gen.normal((T, H, 128), 340, gen.DO, DEV, torch.bfloat16)
    dhT = gen.normal((1, H, 128, 128), 340, gen.DHT, DEV, torch.float32, std=0.1)
    args = (inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"])
    g = kda.backward(*args, do, dhT=dhT, cu_seqlens=inp["cu_seqlens"])
    win = {key: host(x[t0:, heads]) for key, x in g.items() if x is not None and key != "dh0"}
    dh0 = host(g["dh0"][:, heads])
    del g
    torch.cuda.empty_cache()
    _, _, snaps = kda.prefill(*args, cu_seqlens=inp["cu_seqlens"], final_state=False,
                              snapshot_tokens=t0)
    S0_gpu = host(snaps[:, 0][:, heads])
    del snaps
    head = lambda x: x[:t0, heads].to(torch.float32).cpu().numpy()
    _, S0 = oracle.prefill(head(inp["q"]), head(inp["k"]), head(inp["v"]),
                           head(inp["log_alpha"]), inp["beta"][:t0, heads].cpu().numpy(),
                           threads=len(heads))
    sel = lambda x: host(x[t0:, heads])
    ref = oracle.backward(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["log_alpha"]),
                          sel(inp["beta"]), sel(do), h0=S0, dhT=host(dhT[:, heads]))
    errs = {key: rel_err(win[key], ref[key]) for key in ("dq", "dk", "dv", "dlog_alpha", "dbeta")}
    errs["S0"] = rel_err(S0_gpu, S0)
    first = lambda x: host(x[:W, heads])
    ref0 = oracle.backward(first(inp["q"]), first(inp["k"]), first(inp["v"]),
                           first(inp["log_alpha"]), first(inp["beta"]), first(do))
    errs["dh0"] = rel_err(dh0, ref0["dh0"])
    report("backward long_t1m last %d tokens, heads %s" % (W, heads), **errs)
    for key, e in errs.items():
        assert e <= TOL, (key, e)


def test_backward_on_a_side_stream():
    """The call on a non-default stream (its serial pass forked onto the
    binding's second stream of that device and joined back): the same bits
    as on the default stream, complete once that stream is done."""
    inp = case(LENS, 2, 350)
    base = gpu(inp, "channel")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        other = gpu(inp, "channel")
    side.synchronize()
    for key, x in base.items():
        assert torch.equal(x, other[key]), key


def test_backward_second_stream_optional_same_bits():
    """The per-block operand and serial passes on a caller-supplied second
    stream, on the binding's side stream, or in order on the caller's
    stream alone: the same bits."""
    inp = case(LENS, 2, 355)
    alone = gpu(inp, "channel", aux_stream=None)
    auto = gpu(inp, "channel")
    mine = gpu(inp, "channel", aux_stream=torch.cuda.Stream())
    for key, x in alone.items():
        assert torch.equal(x, auto[key]), key
        assert torch.equal(x, mine[key]), key


@pytest.mark.parametrize("aux", [None, "auto"])
def test_backward_max_seqlen_same_bits(aux):
    """max_seqlen bounds the block walk (and the forward recompute's) to the
    longest sequence: the same bits as the walk over total_T; a sequence
    longer than it gets NaN in dh0."""
    inp = case(LENS, 2, 356)
    base = gpu(inp, "channel", block_chunks=1, aux_stream=aux)
    other = gpu(inp, "channel", block_chunks=1, aux_stream=aux, max_seqlen=max(LENS))
    for key, x in base.items():
        assert torch.equal(x, other[key]), key
    cut = gpu(inp, "channel", block_chunks=1, aux_stream=aux, max_seqlen=128)
    for n, L in enumerate(LENS):                     # 300 and 129 tokens exceed 128
        if L > 128:
            assert torch.isnan(cut["dh0"][n]).all(), n
        else:
            assert torch.equal(cut["dh0"][n], base["dh0"][n]), n


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
