"""RMSNorm in front of the LoRA linear on the GPU, against the oracle.

The frozen norm weight g is folded into W on the GPU (lora_fold_norm_weight),
then lora_norm_linear_fwd / _bwd run from the raw X.  H, U, the saved 1/rms,
dX (through the norm), dA and dB are compared element by element with
oracle.norm_forward / norm_backward on the float32 draws (graded bound), over
the kernels' forms: the rank-r product formed inside the GEMM tile (r <= 16,
whole contraction), the precomputed-Z form with a split contraction (r = 8 on
few tiles, r = 40, r = 128), the three forms of the row kernels (K up to 4096,
up to 8192, longer), the full 4096 x 4096 projection, and the call variants
(nothing saved, no dX, accumulated gradients, W folded in place).  Groups of
linears behind one norm (lora_norm_group_*) against the members' oracle
results, and a one-member group bit for bit against the plain norm layer.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import BF16_TOL, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

EPS = 1e-6
BF = torch.bfloat16

CASES = {
    # name: (M, K, N, r) -- which kernel form each one takes is in its comment
    "in_tile": (300, 192, 136, 16),        # both GEMMs form the rank-r product in the tile
    "r8_split": (300, 264, 520, 8),        # few tiles: split contraction, precomputed Z
    "r40": (1000, 1024, 768, 40),          # rank padded to 64, split contraction
    "r128": (2048, 512, 4096, 128),        # rank 128: forward whole tiles, dX split 16 ways
    "k6144": (260, 6144, 264, 16),         # row kernels: rows of 4097..8192 held in registers
    "k9224": (130, 9224, 136, 8),          # row kernels: rows longer than 8192, streamed, ragged last chunk
}


def _shape(name, M, K, N, r, seed=2100):
    return workloads.LinearShape(f"norm_{name}", M, K, N, r, 2.0 * r, seed)


def _run(sh, inp, *, save_u=True, save_inv=True, want_dx=True, flags=0, grads_init=None, fold_in_place=False,
         eps=EPS, X=None):
    import lora_linear_layer_amd as lla
    M, K, N, r = sh.M, sh.K, sh.N, sh.r
    dev = {k: to_dev(inp[k], BF) for k in ("X", "W", "A", "B", "dY", "g")}
    if X is not None:
        dev["X"] = X
    desc = lla.Desc(M, K, N, r, sh.alpha, lla.LORA_DTYPE_BF16, flags)
    Wg = dev["W"] if fold_in_place else torch.empty_like(dev["W"])
    lla.lora_fold_norm_weight(dev["W"], dev["g"], Wg)
    ws = torch.empty(lla.lora_norm_linear_workspace_size(desc), dtype=torch.uint8, device="cuda")
    H = torch.empty((M, N), dtype=BF, device="cuda")
    U = torch.empty((M, r), dtype=torch.float32, device="cuda") if save_u else None
    inv = torch.empty((M,), dtype=torch.float32, device="cuda") if save_inv else None
    lla.lora_norm_linear_fwd(desc, eps, dev["X"], dev["g"], Wg, dev["A"], dev["B"], H, U, inv, ws=ws)
    dX = torch.empty((M, K), dtype=BF, device="cuda") if want_dx else None
    if grads_init is not None:
        dA, dB = to_dev(grads_init[0], BF), to_dev(grads_init[1], BF)
    else:
        dA = torch.empty((r, K), dtype=BF, device="cuda")
        dB = torch.empty((N, r), dtype=BF, device="cuda")
    lla.lora_norm_linear_bwd(desc, eps, dev["dY"], dev["X"], dev["g"], Wg, dev["A"], dev["B"], U, inv, dX, dA, dB,
                             ws=ws)
    torch.cuda.synchronize()
    out = {"H": to_np(H), "dA": to_np(dA), "dB": to_np(dB), "Wg": Wg}
    if save_u:
        out["U"] = to_np(U)
    if save_inv:
        out["inv"] = inv.cpu().numpy()
    if want_dx:
        out["dX"] = to_np(dX)
    return out


def _expected(sh, inp):
    H, U, inv = oracle.norm_forward(inp["X"], inp["g"], EPS, inp["W"], inp["A"], inp["B"], sh.scale)
    dX, dA, dB = oracle.norm_backward(inp["dY"], inp["X"], inp["g"], EPS, inp["W"], inp["A"], inp["B"], sh.scale)
    return {"H": H, "U": U, "inv": inv, "dX": dX, "dA": dA, "dB": dB}


def _assert_close(name, got, ref, keys):
    errs = {k: rel_err(got[k], ref[k]) for k in keys}
    print(f"{name}: graded errors {errs}", flush=True)
    bad = {k: e for k, e in errs.items() if not e <= BF16_TOL}
    assert not bad, f"{name}: {bad} exceed {BF16_TOL}"


@pytest.mark.parametrize("case", list(CASES))
def test_norm_linear_matches_oracle(case):
    sh = _shape(case, *CASES[case])
    print(f"norm linear {case}: M={sh.M} K={sh.K} N={sh.N} r={sh.r}", flush=True)
    inp = workloads.make_norm_inputs(sh)
    got = _run(sh, inp)
    ref = _expected(sh, inp)
    _assert_close(case, got, ref, ("H", "U", "dX", "dA", "dB"))
    # 1/rms of the bf16 input the GPU reads, float32 sums over K
    _, inv16 = oracle.rms_norm(oracle.bf16_round(inp["X"]), np.ones(sh.K), EPS)
    np.testing.assert_allclose(got["inv"], inv16, rtol=2e-5)


def test_fold_norm_weight_is_the_rounded_product():
    """W_g = bf16(W g): the product of two bf16 numbers is exact in float32, so
    the folded weight must equal its round-to-nearest-even bit for bit (also
    when written over W itself)."""
    import lora_linear_layer_amd as lla
    sh = _shape("fold", 64, 520, 136, 8)
    inp = workloads.make_norm_inputs(sh)
    W, g = to_dev(inp["W"], BF), to_dev(inp["g"], BF)
    want = (W.float().cpu() * g.float().cpu()[None, :]).to(BF)
    out = torch.empty_like(W)
    lla.lora_fold_norm_weight(W, g, out)
    lla.lora_fold_norm_weight(W, g, W)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), want.view(torch.int16))
    assert torch.equal(W.cpu().view(torch.int16), want.view(torch.int16))


@pytest.mark.parametrize("case", ["in_tile", "r40"])
def test_norm_linear_recomputes_what_is_not_saved(case):
    """U and 1/rms not saved: the backward rebuilds them from X (same results
    as with them saved, to the bound); no dX: the adapter gradients alone."""
    sh = _shape(case, *CASES[case])
    inp = workloads.make_norm_inputs(sh)
    ref = _expected(sh, inp)
    got = _run(sh, inp, save_u=False, save_inv=False)
    _assert_close(f"{case} nothing saved", got, ref, ("H", "dX", "dA", "dB"))
    got = _run(sh, inp, want_dx=False, fold_in_place=True)
    _assert_close(f"{case} no dX, W folded in place", got, ref, ("H", "U", "dA", "dB"))


def test_norm_linear_accumulates_gradients():
    import lora_linear_layer_amd as lla
    sh = _shape("in_tile", *CASES["in_tile"])
    inp = workloads.make_norm_inputs(sh)
    ref = _expected(sh, inp)
    rng = np.random.Generator(np.random.PCG64(77))
    gA = rng.standard_normal((sh.r, sh.K), dtype=np.float32) * np.float32(0.1)
    gB = rng.standard_normal((sh.N, sh.r), dtype=np.float32) * np.float32(0.1)
    got = _run(sh, inp, flags=lla.LORA_FLAG_ACCUM_GRADS, grads_init=(gA, gB))
    ref = dict(ref, dA=ref["dA"] + oracle.bf16_round(gA), dB=ref["dB"] + oracle.bf16_round(gB))
    _assert_close("accumulated", got, ref, ("dA", "dB"))


def test_norm_linear_full_projection():
    """The 4096 x 4096 projection, M = 4096, r = 8, every element."""
    sh = workloads.LinearShape("norm_attn_proj", 4096, 4096, 4096, 8, 32.0, 2101)
    print("norm linear M=4096 K=4096 N=4096 r=8", flush=True)
    inp = workloads.make_norm_inputs(sh)
    got = _run(sh, inp)
    ref = _expected(sh, inp)
    _assert_close("attn_proj", got, ref, ("H", "U", "dX", "dA", "dB"))


def test_norm_linear_is_scale_invariant_bitwise():
    """At eps = 0, RMSNorm(2 X) = RMSNorm(X): with the input doubled (exact in
    bf16) 1/rms halves exactly and every product doubles exactly, so H, U and
    dA are bit-identical and dX is exactly half."""
    sh = _shape("r40", *CASES["r40"])
    inp = workloads.make_norm_inputs(sh)
    a = _run(sh, inp, eps=0.0)
    X2 = (to_dev(inp["X"], BF).float() * 2.0).to(BF)
    b = _run(sh, inp, eps=0.0, X=X2)
    for k in ("H", "U", "dA", "dB"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    np.testing.assert_array_equal(a["dX"], 2.0 * b["dX"])
    np.testing.assert_array_equal(a["inv"], 2.0 * b["inv"])


# ---------------------------------------------------------------- groups behind one norm
def _group_norm_inputs(M, K, Ns, r, seed):
    mem = [workloads.make_norm_inputs(workloads.LinearShape(f"gn{i}", M, K, n, r, 2.0 * r, seed + i))
           for i, n in enumerate(Ns)]
    return {"X": mem[0]["X"], "g": mem[0]["g"], "W": [m["W"] for m in mem], "A": [m["A"] for m in mem],
            "B": [m["B"] for m in mem], "dY": [m["dY"] for m in mem]}


def _run_group(gi, r, alpha, eps=EPS):
    import lora_linear_layer_amd as lla
    M, K = gi["X"].shape
    Ns = tuple(w.shape[0] for w in gi["W"])
    desc = lla.GroupDesc(M, K, Ns, r, alpha)
    X, g = to_dev(gi["X"], BF), to_dev(gi["g"], BF)
    W = to_dev(np.vstack(gi["W"]), BF)
    A = to_dev(np.vstack(gi["A"]), BF)
    B = to_dev(np.vstack(gi["B"]), BF)
    dY = to_dev(np.hstack(gi["dY"]), BF)
    N, R = sum(Ns), len(Ns) * r
    lla.lora_fold_norm_weight(W, g, W)
    H = torch.empty((M, N), dtype=BF, device="cuda")
    U = torch.empty((M, R), dtype=torch.float32, device="cuda")
    inv = torch.empty((M,), dtype=torch.float32, device="cuda")
    dX = torch.empty((M, K), dtype=BF, device="cuda")
    dA = torch.empty((R, K), dtype=BF, device="cuda")
    dB = torch.empty((N, r), dtype=BF, device="cuda")
    lla.lora_norm_group_fwd(desc, eps, X, g, W, A, B, H, U, inv)
    lla.lora_norm_group_bwd(desc, eps, dY, X, g, W, A, B, U, inv, dX, dA, dB)
    torch.cuda.synchronize()
    cols = np.cumsum((0,) + Ns)
    return {"H": [to_np(H)[:, cols[i]:cols[i + 1]] for i in range(len(Ns))],
            "U": [to_np(U)[:, i * r:(i + 1) * r] for i in range(len(Ns))],
            "dA": [to_np(dA)[i * r:(i + 1) * r] for i in range(len(Ns))],
            "dB": [to_np(dB)[cols[i]:cols[i + 1]] for i in range(len(Ns))],
            "dX": to_np(dX)}


NORM_GROUPS = [
    (300, 392, (264, 136, 520), 16),      # member boundaries inside output tiles
    (513, 256, (1024, 256, 256), 64),     # q / k / v proportions, group rank 192
    (257, 520, (1000, 1000), 24),         # gate / up
]


@pytest.mark.parametrize("M,K,Ns,r", NORM_GROUPS)
def test_norm_group_matches_oracle(M, K, Ns, r):
    """Each member against oracle.norm_forward / norm_backward with the shared
    X and g; dX against the sum of the members' input gradients (the norm's
    Jacobian is linear in the gradient it receives)."""
    print(f"norm group M={M} K={K} N={Ns} r={r}", flush=True)
    gi = _group_norm_inputs(M, K, Ns, r, seed=M + K)
    got = _run_group(gi, r, 2.0 * r)
    s = 2.0
    errs = {"dX": 0.0}
    dX = 0.0
    for i in range(len(Ns)):
        H, U, _ = oracle.norm_forward(gi["X"], gi["g"], EPS, gi["W"][i], gi["A"][i], gi["B"][i], s)
        dXi, dA, dB = oracle.norm_backward(gi["dY"][i], gi["X"], gi["g"], EPS, gi["W"][i], gi["A"][i], gi["B"][i], s)
        dX = dX + dXi
        for k, ref in (("H", H), ("U", U), ("dA", dA), ("dB", dB)):
            errs[f"{k}{i}"] = rel_err(got[k][i], ref)
    errs["dX"] = rel_err(got["dX"], dX)
    print(f"  graded errors {errs}", flush=True)
    bad = {k: e for k, e in errs.items() if not e <= BF16_TOL}
    assert not bad, f"{bad} exceed {BF16_TOL}"


@pytest.mark.parametrize("r", [8, 24])
def test_one_member_norm_group_is_the_norm_layer(r):
    """A norm group of one member takes the plain norm layer's kernels: every
    output bit-identical."""
    M, K, N = 300, 264, 520
    gi = _group_norm_inputs(M, K, (N,), r, seed=91)
    got = _run_group(gi, r, 2.0 * r)
    sh = workloads.LinearShape("gn0", M, K, N, r, 2.0 * r, 91)
    inp = {"X": gi["X"], "g": gi["g"], "W": gi["W"][0], "A": gi["A"][0], "B": gi["B"][0], "dY": gi["dY"][0]}
    plain = _run(sh, inp)
    for k in ("H", "U", "dA", "dB"):
        np.testing.assert_array_equal(got[k][0].view(np.uint32), plain[k].view(np.uint32), err_msg=k)
    np.testing.assert_array_equal(got["dX"].view(np.uint32), plain["dX"].view(np.uint32), err_msg="dX")
