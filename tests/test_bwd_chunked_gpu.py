"""GPU parity of the chunked backward (prism_bwd_chunked through the C ABI) against the
float64 gradient oracle (oracle/prism_grad.py).

The chunked form rounds its matrix-product operands to bfloat16 as the forward does
(float32 sums, a float32 inverse), so every gradient is compared as
max |x - x_ref| / max |x_ref| <= 2e-2, the forward's bfloat16 bar.  A float64 replay of
the same algebra with every product operand rounded to bfloat16 lands at 2-3e-3 on the
16K workload's input recipe (d = 64, L = 4, 8 chunks), so the bar leaves a margin of
about 7 while a missing or wrong term (all of which are O(1) of some gradient) fails it.
Cases: L = 1 .. 8, one chunk and several, a ragged last chunk, sequences shorter than the
anchor window, with and without dS_final, several pairs."""
import numpy as np
import pytest

from tests.conftest import gpu_available
from tests.test_bwd_gpu import _setup

pytestmark = pytest.mark.gpu

TOL = 2e-2
CASES = [
    # name, B, H, T, L, with dS_final
    ("L4_T200_dS", 1, 2, 200, 4, True),
    ("L1_T100_dS", 1, 2, 100, 1, True),
    ("L2_T64", 2, 1, 64, 2, False),
    ("L3_T65_dS", 1, 1, 65, 3, True),
    ("L8_T130_dS", 1, 1, 130, 8, True),
    ("L5_T1_dS", 1, 2, 1, 5, True),
    ("L4_T3", 2, 1, 3, 4, False),
    ("L6_T256_dS", 1, 1, 256, 6, True),
    ("L7_T321", 1, 1, 321, 7, False),
    # twelve pairs: every pass indexes its workspace by pair (chunks, groups, conv shares)
    ("L4_T300_P12_dS", 4, 3, 300, 4, True),
]


def _check(name, B, H, T, L, with_dS):
    import torch
    import delta_rule_sequence_amd as prism
    import workloads
    from oracle import prism_grad
    print(f"[bwd-chunked] {name}", flush=True)
    w, x, d_o, dS = _setup("bf16", B, H, T, 64, L, with_dS, seed=len(name) + T)
    dev = workloads.to_torch(x, "bf16", "cuda")
    got = prism.bwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["u"], dev["alpha"], dev["gamma"],
                    dev["conv_w"], L=L, d_o=torch.tensor(d_o, device="cuda").to(torch.bfloat16),
                    dS_final=None if dS is None else torch.tensor(dS, device="cuda"), chunked=True)
    torch.cuda.synchronize()
    ref = prism_grad.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["gamma"],
                              x["conv_w"], L, d_o, dS)
    names = ["dq", "dk", "dv", "dg", "dbeta"] + (["du", "dalpha", "dgamma", "dconv_w"] if L > 1 else [])
    # A gradient that is identically zero (dg at T = 1: with a zero start the first state
    # does not depend on its gate) comes out of the chunked form as a sum of terms that
    # cancel; its error is measured against the largest entry of any gradient instead.
    scale = max(float(np.max(np.abs(ref[n]))) for n in names)
    errs = {}
    for n in names:
        g = got[n].cpu().numpy()
        r = ref[n]
        assert g.shape == r.shape, (n, g.shape, r.shape)
        assert np.all(np.isfinite(g)), n
        rmax = float(np.max(np.abs(r)))
        errs[n] = float(np.max(np.abs(g - r)) / (rmax if rmax > 0 else scale))
    print(f"[bwd-chunked] {name} rel errors " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()), flush=True)
    bad = {n: e for n, e in errs.items() if not e <= TOL}
    assert not bad, bad


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_chunked_matches_oracle(case):
    if not gpu_available():
        pytest.skip("no GPU")
    _check(*case)


def test_bwd_chunked_deterministic():
    """Two calls on the same inputs give bit-identical gradients (fixed reduction order)."""
    if not gpu_available():
        pytest.skip("no GPU")
    import torch
    import delta_rule_sequence_amd as prism
    import workloads
    w, x, d_o, dS = _setup("bf16", 2, 2, 300, 64, 4, True, seed=5)
    dev = workloads.to_torch(x, "bf16", "cuda")
    args = (dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["u"], dev["alpha"], dev["gamma"], dev["conv_w"])
    kw = dict(L=4, d_o=torch.tensor(d_o, device="cuda").to(torch.bfloat16), dS_final=torch.tensor(dS, device="cuda"),
              chunked=True)
    a = prism.bwd(*args, **kw)
    b = prism.bwd(*args, **kw)
    torch.cuda.synchronize()
    for n in a:
        assert torch.equal(a[n], b[n]), n


LONG_T, LONG_L = 4096, 4


@pytest.fixture(scope="module")
def long_pair():
    """One (b, h) pair of 4096 tokens (64 chunks, 16 groups of the two-level scan) and its
    float64 oracle gradients (~25 s on the host), shared by both forms' checks."""
    if not gpu_available():
        pytest.skip("no GPU")
    import time
    from oracle import prism_grad
    w, x, d_o, dS = _setup("bf16", 1, 1, LONG_T, 64, LONG_L, True, seed=31)
    t0 = time.perf_counter()
    ref = prism_grad.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["gamma"],
                              x["conv_w"], LONG_L, d_o, dS)
    print(f"[bwd] long pair oracle {time.perf_counter() - t0:.1f} s", flush=True)
    return x, d_o, dS, ref


@pytest.mark.parametrize("chunked", [True, False], ids=["chunked", "float32"])
def test_bwd_long_pair(long_pair, chunked):
    """Every gradient of the 4096-token pair against the oracle: the chunked form at its 2e-2
    bar, the float32 form at 1e-4 (the state and adjoint carried across 64 chunks)."""
    import torch
    import delta_rule_sequence_amd as prism
    import workloads
    x, d_o, dS, ref = long_pair
    print(f"[bwd] long pair chunked={chunked}", flush=True)
    dev = workloads.to_torch(x, "bf16", "cuda")
    got = prism.bwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["u"], dev["alpha"], dev["gamma"],
                    dev["conv_w"], L=LONG_L, d_o=torch.tensor(d_o, device="cuda").to(torch.bfloat16),
                    dS_final=torch.tensor(dS, device="cuda"), chunked=chunked)
    torch.cuda.synchronize()
    tol = TOL if chunked else 1e-4
    errs = {}
    for n in ["dq", "dk", "dv", "dg", "dbeta", "du", "dalpha", "dgamma", "dconv_w"]:
        g = got[n].cpu().numpy()
        r = ref[n]
        assert np.all(np.isfinite(g)), n
        errs[n] = float(np.max(np.abs(g - r)) / np.max(np.abs(r)))
    print("[bwd] long pair rel errors " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()), flush=True)
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad
