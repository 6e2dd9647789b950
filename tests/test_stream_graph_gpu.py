"""Streams and HIP graphs: the library launches on the stream it is given and issues no
allocation, memset or synchronisation of its own, so its calls run on any stream and can
be captured into a HIP graph and replayed.

* side stream: the forward (bf16 d = 64 sweep, bf16 d = 128 half-split sweep, generic
  float32 sweep) and the chunked backward issued on a non-default stream (default
  priority) give bit-identical results to the same call on the current stream;
* graph: one call captured with `torch.cuda.graph` into fixed input, output and workspace
  buffers, then replayed three times after fresh inputs are copied into those buffers,
  with eager calls and synchronisations between the replays.  Every replay must be
  bit-identical to an eager call on the same inputs (the same kernels and plan run), and the
  first replay is also compared with the float64 oracle at the parity tolerances (2e-2
  bf16, 1e-4 float32; max-abs error relative to max |reference|);
* serving loop: several decode steps (state and ShortConv window updated in place) captured
  as one graph and replayed from a reset start, checked the same way.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

NAMES = ["q", "k", "v", "g", "beta", "u", "alpha", "gamma", "conv_w"]
TOL = {"f32": 1e-4, "bf16": 2e-2}

# (dtype, d, chunk, L, T): the three forward sweeps, each with a ragged last chunk
CASES = [("bf16", 64, 64, 4, 700), ("bf16", 128, 64, 4, 300), ("f32", 32, 32, 3, 200)]


@pytest.fixture(scope="module")
def prism():
    if not gpu_available():
        pytest.skip("no GPU")
    import delta_rule_sequence_amd as m
    m.load_library()
    return m


def log(msg):
    print(msg, flush=True)


def make(case, seed):
    dt, d, chunk, L, T = case
    w = workloads.Workload("graph", dt, B=1, H=2, T=T, dk=d, dv=d, L=L, chunk=chunk, seed=seed)
    x = workloads.generate(w)
    return w, x, workloads.to_torch(x, dt)


def fwd(prism, w, t, **kw):
    return prism.fwd(*(t[n] for n in NAMES), L=w.L, chunk=w.chunk, **kw)


def rel(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - b)) / max(1e-30, float(np.max(np.abs(b)))))


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_d{c[1]}_L{c[3]}_T{c[4]}")
def test_forward_side_stream(prism, case):
    import torch
    w, _, t = make(case, 600)
    o0, S0 = fwd(prism, w, t)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o1, S1 = fwd(prism, w, t)
    side.synchronize()
    log(f"[stream] fwd {case}: side stream bit-identical {torch.equal(o0, o1) and torch.equal(S0, S1)}")
    assert torch.equal(o0, o1) and torch.equal(S0, S1)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_d{c[1]}_L{c[3]}_T{c[4]}")
def test_forward_graph_replay(prism, case):
    import torch
    dt, d, chunk, L, T = case
    w, _, t = make(case, 610)
    static = {n: v.clone() for n, v in t.items()}
    o = torch.empty((w.B, w.H, T, d), dtype=t["q"].dtype, device="cuda")
    S = torch.empty((w.B, w.H, d, d), dtype=torch.float32, device="cuda")
    code = prism.PRISM_BF16 if dt == "bf16" else prism.PRISM_F32
    ws = torch.empty(max(1, prism.workspace_bytes(w.B, w.H, T, d, d, L, chunk, code)), dtype=torch.uint8,
                     device="cuda")
    # warm up on a side stream before capture, as torch's graph capture asks
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd(prism, w, static, out=(o, S), workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd(prism, w, static, out=(o, S), workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        w2, x2, t2 = make(case, 620 + rep)
        for n in NAMES:
            static[n].copy_(t2[n])
        graph.replay()
        torch.cuda.synchronize()
        oe, Se = fwd(prism, w2, t2)  # eager, fresh buffers
        torch.cuda.synchronize()
        same = torch.equal(o, oe) and torch.equal(S, Se)
        log(f"[graph] fwd {case} replay {rep}: bit-identical to eager {same}")
        assert same
        if rep == 0:
            ref = oracle.forward(*(x2[n] for n in NAMES), L)
            eo, es = rel(o.float().cpu().numpy(), ref[0]), rel(S.cpu().numpy(), ref[1])
            log(f"[graph] fwd {case} replay 0 vs oracle: o {eo:.2e} S_final {es:.2e}")
            assert eo <= TOL[dt] and es <= TOL[dt]


def _bwd_inputs(seed):
    from tests.test_bwd_gpu import _setup
    w, x, d_o, dS = _setup("bf16", 1, 2, 200, 64, 4, True, seed=seed)
    return w, x, d_o, dS


def _bwd(prism, t, L, d_o, dS, **kw):
    return prism.bwd(*(t[n] for n in NAMES), L=L, d_o=d_o, dS_final=dS, chunked=True, **kw)


GRADS = ["dq", "dk", "dv", "dg", "dbeta", "du", "dalpha", "dgamma", "dconv_w"]


def test_chunked_backward_side_stream_and_graph(prism):
    import torch
    from oracle import prism_grad
    w, x, d_o, dS = _bwd_inputs(630)
    t = workloads.to_torch(x, "bf16")
    t["d_o"] = torch.tensor(d_o, device="cuda").to(torch.bfloat16)
    t["dS"] = torch.tensor(dS, device="cuda")
    g0 = _bwd(prism, t, w.L, t["d_o"], t["dS"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g1 = _bwd(prism, t, w.L, t["d_o"], t["dS"])
    side.synchronize()
    same = all(torch.equal(g0[n], g1[n]) for n in GRADS)
    log(f"[stream] chunked bwd: side stream bit-identical {same}")
    assert same

    static = {n: v.clone() for n, v in t.items()}
    with torch.cuda.stream(side):  # warm-up before capture
        _bwd(prism, static, w.L, static["d_o"], static["dS"])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gs = _bwd(prism, static, w.L, static["d_o"], static["dS"])
    torch.cuda.synchronize()
    for rep in range(3):
        w2, x2, d_o2, dS2 = _bwd_inputs(640 + rep)
        t2 = workloads.to_torch(x2, "bf16")
        t2["d_o"] = torch.tensor(d_o2, device="cuda").to(torch.bfloat16)
        t2["dS"] = torch.tensor(dS2, device="cuda")
        for n in static:
            static[n].copy_(t2[n])
        graph.replay()
        torch.cuda.synchronize()
        ge = _bwd(prism, t2, w2.L, t2["d_o"], t2["dS"])
        torch.cuda.synchronize()
        same = all(torch.equal(gs[n], ge[n]) for n in GRADS)
        log(f"[graph] chunked bwd replay {rep}: bit-identical to eager {same}")
        assert same
        if rep == 0:
            ref = prism_grad.backward(*(x2[n] for n in NAMES), w2.L, d_o2, dS2)
            errs = {n: rel(gs[n].cpu().numpy(), ref[n]) for n in GRADS}
            log("[graph] chunked bwd replay 0 vs oracle: " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
            assert all(e <= 2e-2 for e in errs.values()), errs


# (dtype, d, L, steps): decode steps of the serving loop, one token for every pair per step
DECODE = [("bf16", 64, 4, 6), ("bf16", 128, 8, 5), ("f32", 32, 3, 6)]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: f"{c[0]}_d{c[1]}_L{c[2]}")
def test_decode_loop_graph_replay(prism, case):
    """A loop of decode steps captured as one graph (the state and the ShortConv window
    updated in place, step after step), replayed from a reset start on fresh tokens: every
    replay bit-identical to the same steps run eagerly, the first against the oracle over
    those tokens from the same start."""
    import torch
    dt, d, L, n = case
    seq = ["q", "k", "v", "g", "beta"] + (["u", "alpha", "gamma"] if L > 1 else [])

    def inputs(seed):
        w = workloads.Workload("decode_graph", dt, B=2, H=2, T=n, dk=d, dv=d, L=L, chunk=64, seed=seed)
        x = workloads.generate(w)
        st = workloads.generate_state(w)
        t = workloads.to_torch(x, dt)
        s = workloads.to_torch(st, dt)
        toks = [{m: t[m][:, :, i].contiguous() for m in seq} for i in range(n)]
        return w, x, st, toks, t["conv_w"], s["S0"], s["conv_in"]

    def steps(S, conv, toks, conv_w):
        return [prism.decode_step(S, conv, *(tk[m] for m in ["q", "k", "v", "g", "beta"]),
                                  tk.get("u"), tk.get("alpha"), tk.get("gamma"),
                                  conv_w if L > 1 else None, L=L) for tk in toks]

    w, x, st, toks, conv_w, S0, c0 = inputs(650)
    S, conv = S0.clone(), c0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up before capture
        steps(S, conv, toks, conv_w)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = steps(S, conv, toks, conv_w)
    torch.cuda.synchronize()
    for rep in range(3):
        w2, x2, st2, toks2, conv_w2, S02, c02 = inputs(660 + rep)
        for tk, tk2 in zip(toks, toks2):
            for m in seq:
                tk[m].copy_(tk2[m])
        conv_w.copy_(conv_w2)
        S.copy_(S02)
        conv.copy_(c02)
        graph.replay()
        torch.cuda.synchronize()
        Se, ce = S02.clone(), c02.clone()
        oe = steps(Se, ce, toks2, conv_w2)
        torch.cuda.synchronize()
        same = (all(torch.equal(a, b) for a, b in zip(outs, oe)) and torch.equal(S, Se) and torch.equal(conv, ce))
        log(f"[graph] decode {case} replay {rep}: bit-identical to eager {same}")
        assert same
        if rep == 0:
            ro, rS = oracle.forward(*(x2[m] for m in NAMES), L, S0=st2["S0"], conv_in=st2["conv_in"])[:2]
            o = np.stack([a.float().cpu().numpy() for a in outs], axis=2)
            eo, es = rel(o, ro), rel(S.cpu().numpy(), rS)
            log(f"[graph] decode {case} replay 0 vs oracle: o {eo:.2e} S_final {es:.2e}")
            assert eo <= TOL[dt] and es <= TOL[dt]
            assert np.array_equal(conv.float().cpu().numpy(), x2["v"][:, :, n - 3:])
