"""GPU parity of the backward pass (prism_bwd through the C ABI) against the float64
gradient oracle (oracle/prism_grad.py: autograd through the token recurrence, pinned
by finite differences of the numpy forward).

Every gradient is compared as max |x - x_ref| / max |x_ref| <= 1e-4: the kernels
compute in float32 from the same (bf16-rounded, for bf16 inputs) input values the
oracle reads, so the float32 bar applies to both input dtypes.  Both organisations are
covered: the segment-parallel default (prism_bwd; with prism_bwd_seg for chosen segment
lengths, ragged last segments and segments that span several 8-token sub-blocks) and the
sequential low-memory form (prism_bwd_lowmem).
"""
import numpy as np
import pytest

from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

TOL = 1e-4
CASES = [
    # name, dtype, B, H, T, d, L, with dS_final
    ("f32_d16_L1_T100", "f32", 1, 2, 100, 16, 1, True),
    ("f32_d32_L3_T130", "f32", 2, 2, 130, 32, 3, False),
    ("bf16_d64_L4_T200", "bf16", 1, 2, 200, 64, 4, True),
    ("f32_d64_L8_T65", "f32", 1, 1, 65, 64, 8, True),
    ("bf16_d128_L2_T70", "bf16", 1, 1, 70, 128, 2, True),
    ("f32_d16_L3_T1", "f32", 1, 2, 1, 16, 3, True),
    ("f32_d32_L2_T3", "f32", 2, 1, 3, 32, 2, False),
    ("bf16_d64_L4_T128", "bf16", 1, 1, 128, 64, 4, False),
    # d = 128 with L > 4: the inputs' LDS stages do not fit, so the kernel reads them from memory
    ("bf16_d128_L8_T70", "bf16", 1, 2, 70, 128, 8, True),
]


def _setup(dtype, B, H, T, d, L, with_dS, seed):
    import workloads
    w = workloads.Workload("bwd", dtype, B=B, H=H, T=T, dk=d, dv=d, L=L, chunk=64, seed=seed)
    x = workloads.generate(w)
    rng = np.random.default_rng(seed + 100)
    d_o = rng.standard_normal((B, H, T, d)).astype(np.float32)
    if dtype == "bf16":
        d_o = workloads.to_bf16_values(d_o)
    dS = rng.standard_normal((B, H, d, d)).astype(np.float32) if with_dS else None
    return w, x, d_o, dS


# segment-parallel cases with a chosen segment length: name, dtype, B, H, T, d, L, with
# dS_final, seg_len (several segments, a ragged last one, segments of 2-16 sub-blocks,
# rows split over workgroups at d = 128)
SEG_CASES = [
    ("bf16_d64_L4_T200_s16", "bf16", 1, 2, 200, 64, 4, True, 16),
    ("f32_d32_L3_T130_s24", "f32", 2, 2, 130, 32, 3, False, 24),
    ("f32_d16_L8_T97_s16", "f32", 1, 1, 97, 16, 8, True, 16),
    ("f32_d64_L1_T100_s32", "f32", 1, 2, 100, 64, 1, True, 32),
    ("bf16_d128_L8_T70_s16", "bf16", 1, 1, 70, 128, 8, True, 16),
    ("bf16_d128_L2_T300_s64", "bf16", 1, 1, 300, 128, 2, False, 64),
    ("bf16_d64_L4_T1000_s128", "bf16", 1, 1, 1000, 64, 4, True, 128),
    ("f32_d32_L5_T40_s40", "f32", 1, 1, 40, 32, 5, True, 40),
]


def _check_against_oracle(name, dtype, B, H, T, d, L, with_dS, **kw):
    import torch
    import delta_rule_sequence_amd as prism
    import workloads
    from oracle import prism_grad
    print(f"[bwd] {name} {kw}", flush=True)
    w, x, d_o, dS = _setup(dtype, B, H, T, d, L, with_dS, seed=len(name) + T)
    dev = workloads.to_torch(x, dtype, "cuda")
    vt = torch.bfloat16 if dtype == "bf16" else torch.float32
    got = prism.bwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["u"], dev["alpha"], dev["gamma"],
                    dev["conv_w"], L=L, d_o=torch.tensor(d_o, device="cuda").to(vt),
                    dS_final=None if dS is None else torch.tensor(dS, device="cuda"), **kw)
    torch.cuda.synchronize()
    ref = prism_grad.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["gamma"],
                              x["conv_w"], L, d_o, dS)
    names = ["dq", "dk", "dv", "dg", "dbeta"] + (["du", "dalpha", "dgamma", "dconv_w"] if L > 1 else [])
    errs = {}
    for n in names:
        g = got[n].cpu().numpy()
        r = ref[n]
        assert g.shape == r.shape, (n, g.shape, r.shape)
        assert np.all(np.isfinite(g)), n
        errs[n] = float(np.max(np.abs(g - r)) / max(1e-30, np.max(np.abs(r))))
    print(f"[bwd] {name} rel errors " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()), flush=True)
    bad = {n: e for n, e in errs.items() if not e <= TOL}
    assert not bad, bad


@pytest.mark.parametrize("low_memory", [False, True], ids=["segments", "lowmem"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_matches_oracle(case, low_memory):
    if not gpu_available():
        pytest.skip("no GPU")
    _check_against_oracle(*case, low_memory=low_memory)


@pytest.mark.parametrize("case", SEG_CASES, ids=[c[0] for c in SEG_CASES])
def test_bwd_seg_matches_oracle(case):
    if not gpu_available():
        pytest.skip("no GPU")
    _check_against_oracle(*case[:-1], seg_len=case[-1])


def test_bwd_deterministic():
    """Two calls on the same inputs give bit-identical gradients (fixed reduction order)."""
    if not gpu_available():
        pytest.skip("no GPU")
    import torch
    import delta_rule_sequence_amd as prism
    import workloads
    w, x, d_o, dS = _setup("bf16", 2, 2, 96, 32, 3, True, seed=5)
    dev = workloads.to_torch(x, "bf16", "cuda")
    args = (dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["u"], dev["alpha"], dev["gamma"], dev["conv_w"])
    kw = dict(L=3, d_o=torch.tensor(d_o, device="cuda").to(torch.bfloat16), dS_final=torch.tensor(dS, device="cuda"))
    a = prism.bwd(*args, **kw)
    b = prism.bwd(*args, **kw)
    torch.cuda.synchronize()
    for n in a:
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("chunked", [False, True], ids=["segments", "chunked"])
@pytest.mark.parametrize("which", ["v", "q"])
def test_bwd_full_size_linear_directions(which, chunked):
    """At the full 16K bf16 workload (B=2, H=4, T=16384, d=64, L=4): o and S_final are linear
    in v (A_t does not depend on v; B_t, the anchor and the residual chain are linear in it)
    and o is linear in q (S does not depend on q), so for any direction e
        <d_o, o(x := e)> + <dS_final, S_final(x := e)> = <dx, e>
    with the forward kernel on the left and the backward kernel on the right (dx does not
    depend on x).  Both sides carry bf16 rounding of their operands (a relative error of a
    few 2^-9 per element, with random signs), so the bound is 2^-6 sqrt(sum (d_o o)^2):
    about 23 here, against sums of a few hundred to a thousand that a wrong gradient would
    miss by their own size.  Run for the segment-parallel form and the chunked MFMA form
    (prism_bwd_chunked), whose gradients carry bf16 rounding of the same order."""
    if not gpu_available():
        pytest.skip("no GPU")
    import torch
    import delta_rule_sequence_amd as prism
    import workloads
    w = workloads.workload("rec16k_bf16")
    print(f"[bwd] full-size linear direction {which} on {w.name} chunked={chunked}", flush=True)
    x = workloads.generate(w)
    dev = workloads.to_torch(x, w.dtype, "cuda")
    gen = torch.Generator(device="cuda").manual_seed(17)
    d_o = torch.randn((w.B, w.H, w.T, w.dv), device="cuda", generator=gen).to(torch.bfloat16)
    dS = torch.randn((w.B, w.H, w.dk, w.dv), device="cuda", generator=gen)
    e = torch.randn(dev[which].shape, device="cuda", generator=gen).to(torch.bfloat16)
    if which == "q":
        e = e / e.float().norm(dim=-1, keepdim=True).to(torch.bfloat16)
    grads = prism.bwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["u"], dev["alpha"], dev["gamma"],
                      dev["conv_w"], L=w.L, d_o=d_o, dS_final=dS, chunked=chunked)
    args = dict(dev)
    args[which] = e
    o, S = prism.fwd(args["q"], args["k"], args["v"], args["g"], args["beta"], args["u"], args["alpha"],
                     args["gamma"], args["conv_w"], L=w.L, chunk=w.chunk)
    torch.cuda.synchronize()
    prod = d_o.double() * o.double()
    lhs = float(prod.sum())
    sq = float((prod * prod).sum())
    if which == "v":
        prodS = dS.double() * S.double()
        lhs += float(prodS.sum())
        sq += float((prodS * prodS).sum())
    rhs = float((grads["d" + which].double() * e.double()).sum())
    bound = 2.0 ** -6 * sq ** 0.5
    print(f"[bwd] <d_o, o(e)> = {lhs:.6e}, <d{which}, e> = {rhs:.6e}, bound {bound:.3e}", flush=True)
    assert abs(lhs - rhs) <= bound, (lhs, rhs, bound)
