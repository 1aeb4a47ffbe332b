"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: element-wise
brute force, exact finite differences, closed-form special cases, the merged
weight identity, permutation and additivity invariants, a library's inverse
normal CDF, torch's bfloat16 conversion and the golden codebook table.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(seed, M=5, K=7, N=6, r=3):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K))
    A = rng.standard_normal((r, K))
    B = rng.standard_normal((N, r))
    dY = rng.standard_normal((M, N))
    s = float(rng.uniform(0.25, 4.0))
    return X, W, A, B, dY, s


# ---------------------------------------------------------------- brute force
def brute_forward(X, W, A, B, s):
    """h_n = sum_k W[n,k] x_k + s * sum_j B[n,j] * (sum_k A[j,k] x_k), per token."""
    M, K = X.shape
    N, r = B.shape
    H = [[0.0] * N for _ in range(M)]
    for m in range(M):
        ax = [sum(A[j][k] * X[m][k] for k in range(K)) for j in range(r)]
        for n in range(N):
            H[m][n] = sum(W[n][k] * X[m][k] for k in range(K)) + s * sum(B[n][j] * ax[j] for j in range(r))
    return np.array(H)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_forward_matches_brute_force(seed):
    X, W, A, B, _, s = rand_case(seed)
    H, U = oracle.forward(X, W, A, B, s)
    np.testing.assert_allclose(H, brute_forward(X, W, A, B, s), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(U, [[sum(A[j][k] * X[m][k] for k in range(X.shape[1]))
                                    for j in range(A.shape[0])] for m in range(X.shape[0])],
                               rtol=1e-12, atol=1e-12)


def test_forward_merged_weight_identity():
    X, W, A, B, _, s = rand_case(3)
    H, _ = oracle.forward(X, W, A, B, s)
    Wm = oracle.merged_weight(W, A, B, s)
    np.testing.assert_allclose(H, X @ Wm.T, rtol=1e-12, atol=1e-12)
    # merged weight element-wise: W[n,k] + s * sum_j B[n,j] A[j,k]
    n, k = 2, 4
    assert math.isclose(Wm[n, k], W[n, k] + s * sum(B[n, j] * A[j, k] for j in range(A.shape[0])),
                        rel_tol=1e-13)


def test_merged_weight_unmerge_and_zero_b():
    """Unmerging with -s restores W (up to float64 rounding); B = 0 merges to W
    exactly; the merged weight is linear in s."""
    _, W, A, B, _, s = rand_case(5)
    Wm = oracle.merged_weight(W, A, B, s)
    np.testing.assert_allclose(oracle.merged_weight(Wm, A, B, -s), W, rtol=0, atol=1e-14)
    np.testing.assert_array_equal(oracle.merged_weight(W, A, np.zeros_like(B), s), W)
    np.testing.assert_allclose(oracle.merged_weight(W, A, B, 2 * s) - W, 2 * (Wm - W), rtol=1e-13, atol=1e-15)
    assert not np.allclose(Wm, W)


def test_forward_special_cases():
    X, W, A, B, _, s = rand_case(4)
    H0, _ = oracle.forward(X, W, A, np.zeros_like(B), s)            # B = 0 -> plain linear
    np.testing.assert_array_equal(H0, X @ W.T)
    Hw, U = oracle.forward(X, np.zeros_like(W), A, B, s)             # W = 0 -> pure adapter
    np.testing.assert_allclose(Hw, s * U @ B.T, rtol=1e-13)
    H1, _ = oracle.forward(X, W, A, B, 1.0)                          # linear in s
    Hs, _ = oracle.forward(X, W, A, B, s)
    np.testing.assert_allclose(Hs - X @ W.T, s * (H1 - X @ W.T), rtol=1e-11, atol=1e-12)


# -------------------------------------------------------------- backward pins
def loss(dY, X, W, A, B, s):
    H, _ = oracle.forward(X, W, A, B, s)
    return float(np.sum(dY * H))


def central_fd(f, P, h=0.5):
    """Central differences of a function that is linear in P (exact up to rounding)."""
    G = np.zeros_like(P)
    for idx in itertools.product(*map(range, P.shape)):
        Pp = P.copy(); Pp[idx] += h
        Pm = P.copy(); Pm[idx] -= h
        G[idx] = (f(Pp) - f(Pm)) / (2 * h)
    return G


@pytest.mark.parametrize("seed", [5, 6])
def test_backward_finite_differences(seed):
    X, W, A, B, dY, s = rand_case(seed)
    dX, dA, dB = oracle.backward(dY, X, W, A, B, s)
    # L is linear in each of X, A, B separately, so the central difference is exact
    np.testing.assert_allclose(dX, central_fd(lambda P: loss(dY, P, W, A, B, s), X), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(dA, central_fd(lambda P: loss(dY, X, W, P, B, s), A), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(dB, central_fd(lambda P: loss(dY, X, W, A, P, s), B), rtol=1e-9, atol=1e-10)


def test_backward_brute_force():
    X, W, A, B, dY, s = rand_case(7, M=4, K=5, N=6, r=2)
    M, K = X.shape; N, r = B.shape
    dX, dA, dB = oracle.backward(dY, X, W, A, B, s)
    for m, k in itertools.product(range(M), range(K)):
        want = sum(dY[m, n] * W[n, k] for n in range(N)) + \
            s * sum(sum(dY[m, n] * B[n, j] for n in range(N)) * A[j, k] for j in range(r))
        assert math.isclose(dX[m, k], want, rel_tol=1e-11, abs_tol=1e-12)
    for j, k in itertools.product(range(r), range(K)):
        want = s * sum(sum(dY[m, n] * B[n, j] for n in range(N)) * X[m, k] for m in range(M))
        assert math.isclose(dA[j, k], want, rel_tol=1e-11, abs_tol=1e-12)
    for n, j in itertools.product(range(N), range(r)):
        want = s * sum(dY[m, n] * sum(A[j, k] * X[m, k] for k in range(K)) for m in range(M))
        assert math.isclose(dB[n, j], want, rel_tol=1e-11, abs_tol=1e-12)


def test_backward_adjoint():
    """<dY, J d> = <J^T dY, d> for a random direction d over (X, A, B)."""
    X, W, A, B, dY, s = rand_case(8)
    rng = np.random.default_rng(80)
    dXd, dAd, dBd = (rng.standard_normal(t.shape) for t in (X, A, B))
    def cdiff(eps):
        H_p, _ = oracle.forward(X + eps * dXd, W, A + eps * dAd, B + eps * dBd, s)
        H_m, _ = oracle.forward(X - eps * dXd, W, A - eps * dAd, B - eps * dBd, s)
        return (H_p - H_m) / (2 * eps)
    # H is a cubic polynomial along the joint direction, so the central difference is
    # J d + c eps^2 exactly; Richardson extrapolation over eps and 2 eps removes c.
    jd = (4 * cdiff(0.5) - cdiff(1.0)) / 3
    dX, dA, dB = oracle.backward(dY, X, W, A, B, s)
    lhs = float(np.sum(dY * jd))
    rhs = float(np.sum(dX * dXd) + np.sum(dA * dAd) + np.sum(dB * dBd))
    assert math.isclose(lhs, rhs, rel_tol=1e-9)


def test_backward_special_cases():
    X, W, A, B, dY, s = rand_case(9)
    dX, dA, dB = oracle.backward(dY, X, W, A, np.zeros_like(B), s)    # B = 0: training start
    np.testing.assert_array_equal(dA, 0.0)
    np.testing.assert_array_equal(dX, dY @ W)
    assert np.abs(dB).max() > 0
    _, _, dB0 = oracle.backward(dY, X, W, np.zeros_like(A), B, s)      # A = 0
    np.testing.assert_array_equal(dB0, 0.0)
    _, dA0, dB0 = oracle.backward(dY, X, W, A, B, 0.0)                 # s = 0
    np.testing.assert_array_equal(dA0, 0.0)
    np.testing.assert_array_equal(dB0, 0.0)


def test_token_permutation_and_split_additivity():
    X, W, A, B, dY, s = rand_case(10, M=9)
    perm = np.random.default_rng(100).permutation(X.shape[0])
    H, _ = oracle.forward(X, W, A, B, s)
    Hp, _ = oracle.forward(X[perm], W, A, B, s)
    np.testing.assert_allclose(Hp, H[perm], rtol=1e-13)
    dX, dA, dB = oracle.backward(dY, X, W, A, B, s)
    dXp, dAp, dBp = oracle.backward(dY[perm], X[perm], W, A, B, s)
    np.testing.assert_allclose(dXp, dX[perm], rtol=1e-12)
    np.testing.assert_allclose(dAp, dA, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dBp, dB, rtol=1e-12, atol=1e-13)
    # split over tokens: gradients of the whole = sum over chunks
    parts = [oracle.backward_lora(dY[a:b], X[a:b], A, B, s) for a, b in ((0, 4), (4, 7), (7, 9))]
    np.testing.assert_allclose(sum(p[0] for p in parts), dA, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sum(p[1] for p in parts), dB, rtol=1e-12, atol=1e-13)


def test_torch_autograd_agrees():
    """Independent check of the gradient formulas with torch autograd (float64, CPU)."""
    X, W, A, B, dY, s = rand_case(11, M=6, K=8, N=5, r=4)
    Xt, At, Bt = (torch.tensor(t, requires_grad=True) for t in (X, A, B))
    Wt = torch.tensor(W)
    H = Xt @ Wt.T + s * (Xt @ At.T) @ Bt.T
    H.backward(torch.tensor(dY))
    dX, dA, dB = oracle.backward(dY, X, W, A, B, s)
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dA, At.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dB, Bt.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_lora_scale():
    assert oracle.lora_scale(32, 8) == 4.0
    assert oracle.lora_scale(16, 64) == 0.25


# --------------------------------------------------------------- number formats
def test_bf16_round_matches_torch():
    rng = np.random.default_rng(12)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),       # bf16 subnormals
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 3.0e38, -3.0e38, np.inf, -np.inf], np.float32),
    ])
    # exact ties: low 16 bits == 0x8000, both parities of the kept part
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x3F800000 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.bf16_round(x)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.isnan(oracle.bf16_round(np.array([np.nan], np.float32)))[0]


def test_f16_decode_matches_numpy():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.f16_to_f64(bits)
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(got[finite], ref[finite])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def load_golden_codebook():
    rows = []
    with open(os.path.join(GOLDEN, "codebook4_f32.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            i, bits, val = line.split()
            rows.append((int(i), int(bits, 16), float(val)))
    return rows


def test_codebook_golden_bits():
    cb = oracle.codebook4()
    rows = load_golden_codebook()
    assert [i for i, _, _ in rows] == list(range(16))
    np.testing.assert_array_equal(cb.view(np.uint32), np.array([b for _, b, _ in rows], np.uint32))


def test_codebook_closed_form_scipy():
    """Independent inverse normal CDF (scipy.special.ndtri)."""
    ref = np.array([scipy.special.ndtri((i + 0.5) / 16) for i in range(16)]) / scipy.special.ndtri(15.5 / 16)
    cb = oracle.codebook4()
    np.testing.assert_array_equal(cb, ref.astype(np.float32))
    assert cb[0] == -1.0 and cb[15] == 1.0
    np.testing.assert_array_equal(cb[::-1], -cb)          # symmetric
    assert np.all(np.diff(cb) > 0)
    assert not np.any(cb == 0)                             # no exact zero (not NF4)


def test_workload_codebook_equals_golden():
    np.testing.assert_array_equal(workloads.codebook4_f32(), oracle.codebook4())


def brute_dequant(codes, absmax, cb, k_total):
    N = codes.shape[0]
    out = np.zeros((N, k_total), np.float32)
    for n in range(N):
        for k in range(k_total):
            byte = int(codes[n, k // 2])
            code = byte & 0xF if k % 2 == 0 else byte >> 4
            a = np.float32(np.float16(absmax[n, k // 64]))
            out[n, k] = np.float32(cb[code]) * a                  # numpy float32 multiply (IEEE)
    return out


def test_dequant4_brute_force():
    rng = np.random.default_rng(13)
    N, K = 3, 128
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    absmax = rng.uniform(0.001, 0.1, size=(N, K // 64)).astype(np.float16)
    cb = oracle.codebook4()
    f32 = brute_dequant(codes, absmax, cb, K)
    np.testing.assert_array_equal(oracle.dequant4(codes, absmax, cb, out="f32").view(np.uint32),
                                  f32.view(np.uint32))
    want_bf16 = torch.from_numpy(f32).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(oracle.dequant4(codes, absmax, cb).view(np.uint32),
                                  want_bf16.view(np.uint32))


def test_dequant4_nibble_order():
    cb = oracle.codebook4()
    codes = np.zeros((1, 32), np.uint8)
    codes[0, 0] = 0x3A                      # k=0 -> 0xA (low nibble), k=1 -> 0x3 (high)
    absmax = np.ones((1, 1), np.float16)
    w = oracle.dequant4(codes, absmax, cb, out="f32")
    assert w[0, 0] == cb[10] and w[0, 1] == cb[3] and w[0, 2] == cb[0]


def test_quantize_roundtrip_bound():
    """|w - deq(q(w))| <= absmax * (largest codebook gap)/2 + rounding."""
    d = workloads.make_linear_inputs(workloads.LinearShape("q", 4, 256, 24, 4, 8.0, 77))
    W = d["W"]
    codes, absmax = workloads.quantize4(W)
    cb = oracle.codebook4()
    deq = oracle.dequant4(codes, absmax, cb, out="f32").astype(np.float64)
    am = np.repeat(oracle.f16_to_f64(absmax), 64, axis=1)
    gap = np.max(np.diff(cb.astype(np.float64))) / 2
    assert np.all(np.abs(W - deq) <= am * gap * (1 + 1e-3) + np.abs(W) * 2e-3 + 1e-7)
    # absmax is the fp16 image of the block max
    blk = np.abs(W.astype(np.float64)).reshape(24, 4, 64).max(axis=2)
    np.testing.assert_array_equal(absmax, blk.astype(np.float16))


# ----------------------------------------------------------------- generator
def test_generator_is_seeded():
    shape = workloads.LinearShape("t", 8, 32, 16, 4, 8.0, 99)
    a = workloads.make_linear_inputs(shape)
    b = workloads.make_linear_inputs(shape)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    c = workloads.make_linear_inputs(workloads.LinearShape("t", 8, 32, 16, 4, 8.0, 100))
    assert not np.array_equal(a["X"], c["X"])
    assert a["X"].dtype == np.float32 and a["A"].shape == (4, 32) and a["B"].shape == (16, 4)


def test_workload_flops():
    wl = workloads.workload("attn_proj_4096")
    assert wl.flops() == 4 * 4096 ** 3 + 6 * 4096 * 8 * 8192
    assert abs(wl.flops() / 1e9 - 276.49) < 0.01


# ---------------------------------------------------------------- linears sharing one input
def group_case(seed, M=4, K=6, Ns=(5, 3, 4), r=2):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    Ws = [rng.standard_normal((n, K)) for n in Ns]
    As = [rng.standard_normal((r, K)) for _ in Ns]
    Bs = [rng.standard_normal((n, r)) for n in Ns]
    dYs = [rng.standard_normal((M, n)) for n in Ns]
    return X, Ws, As, Bs, dYs, float(rng.uniform(0.25, 4.0))


def test_group_backward_finite_differences():
    """dX of a group is the gradient of L = sum_i <dY_i, H_i> with respect to
    the shared X (central differences; L is linear in X, so they are exact up
    to rounding), and each member's dA_i, dB_i that of its own parameters."""
    X, Ws, As, Bs, dYs, s = group_case(11)

    def loss(X_, As_, Bs_):
        outs = oracle.group_forward(X_, Ws, As_, Bs_, s)
        return sum(float(np.sum(dY * H)) for dY, (H, _) in zip(dYs, outs))

    dX, dAs, dBs = oracle.group_backward(dYs, X, Ws, As, Bs, s)
    h = 1e-3
    for idx in itertools.product(range(X.shape[0]), range(X.shape[1])):
        Xp, Xm = X.copy(), X.copy()
        Xp[idx] += h
        Xm[idx] -= h
        assert abs((loss(Xp, As, Bs) - loss(Xm, As, Bs)) / (2 * h) - dX[idx]) <= 1e-9 * max(1.0, abs(dX[idx]))
    for i in range(len(Ws)):
        for idx in itertools.product(range(As[i].shape[0]), range(As[i].shape[1])):
            Ap = [a.copy() for a in As]; Am = [a.copy() for a in As]
            Ap[i][idx] += h; Am[i][idx] -= h
            fd = (loss(X, Ap, Bs) - loss(X, Am, Bs)) / (2 * h)
            assert abs(fd - dAs[i][idx]) <= 1e-9 * max(1.0, abs(fd))
        for idx in itertools.product(range(Bs[i].shape[0]), range(Bs[i].shape[1])):
            Bp = [b.copy() for b in Bs]; Bm = [b.copy() for b in Bs]
            Bp[i][idx] += h; Bm[i][idx] -= h
            fd = (loss(X, As, Bp) - loss(X, As, Bm)) / (2 * h)
            assert abs(fd - dBs[i][idx]) <= 1e-9 * max(1.0, abs(fd))


def test_group_is_one_layer_with_block_diagonal_b():
    """A group equals one LoRA layer over the stacked weights: W = [W_1; ..; W_G],
    A = [A_1; ..; A_G] (rank G r), B block-diagonal diag(B_1, .., B_G).  Its
    output is the members' outputs side by side, its dX the group's dX, its
    dA the members' dA stacked, and the diagonal blocks of its dB the
    members' dB (the off-diagonal blocks belong to no parameter)."""
    X, Ws, As, Bs, dYs, s = group_case(12)
    Ns = [w.shape[0] for w in Ws]
    r = As[0].shape[0]
    Bbd = np.zeros((sum(Ns), r * len(Ns)))
    n0 = 0
    for i, B in enumerate(Bs):
        Bbd[n0:n0 + Ns[i], i * r:(i + 1) * r] = B
        n0 += Ns[i]
    Wst, Ast, dYst = np.vstack(Ws), np.vstack(As), np.hstack(dYs)
    H, U = oracle.forward(X, Wst, Ast, Bbd, s)
    outs = oracle.group_forward(X, Ws, As, Bs, s)
    np.testing.assert_allclose(H, np.hstack([h for h, _ in outs]), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(U, np.hstack([u for _, u in outs]), rtol=1e-12, atol=1e-12)
    dX, dA, dB = oracle.backward(dYst, X, Wst, Ast, Bbd, s)
    gdX, gdAs, gdBs = oracle.group_backward(dYs, X, Ws, As, Bs, s)
    np.testing.assert_allclose(dX, gdX, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dA, np.vstack(gdAs), rtol=1e-12, atol=1e-12)
    n0 = 0
    for i, g in enumerate(gdBs):
        np.testing.assert_allclose(dB[n0:n0 + Ns[i], i * r:(i + 1) * r], g, rtol=1e-12, atol=1e-12)
        n0 += Ns[i]


def test_group_of_one_is_the_layer():
    X, Ws, As, Bs, dYs, s = group_case(13, Ns=(5,))
    (H, U), = oracle.group_forward(X, Ws, As, Bs, s)
    H1, U1 = oracle.forward(X, Ws[0], As[0], Bs[0], s)
    np.testing.assert_array_equal(H, H1)
    dX, (dA,), (dB,) = oracle.group_backward(dYs, X, Ws, As, Bs, s)
    dX1, dA1, dB1 = oracle.backward(dYs[0], X, Ws[0], As[0], Bs[0], s)
    np.testing.assert_array_equal(dX, dX1)
    np.testing.assert_array_equal(dA, dA1)
    np.testing.assert_array_equal(dB, dB1)


# ---------------------------------------------------------------- RMSNorm in front of the layer
def norm_case(seed, M=4, K=6, N=5, r=2):
    X, W, A, B, dY, s = rand_case(seed, M, K, N, r)
    rng = np.random.default_rng(seed + 100)
    g = rng.uniform(0.5, 1.5, size=K)
    return X, g, 1e-3, W, A, B, dY, s


def test_rms_norm_brute_force():
    X, g, eps, *_ = norm_case(21)
    Xn, inv = oracle.rms_norm(X, g, eps)
    for m in range(X.shape[0]):
        ms = sum(float(v) * float(v) for v in X[m]) / X.shape[1]
        i = 1.0 / math.sqrt(ms + eps)
        assert abs(inv[m] - i) <= 1e-15 * i
        for k in range(X.shape[1]):
            assert abs(Xn[m, k] - X[m, k] * i * g[k]) <= 1e-14 * max(1.0, abs(Xn[m, k]))


def test_norm_backward_finite_differences():
    """dX of the norm + layer is the gradient of L = <dY, H> with respect to the
    raw X (central differences with h = 1e-6: the norm is not linear in X, so
    agreement is to ~1e-8), dA and dB those of the adapter."""
    X, g, eps, W, A, B, dY, s = norm_case(22)
    loss = lambda X_, A_, B_: float(np.sum(dY * oracle.norm_forward(X_, g, eps, W, A_, B_, s)[0]))
    dX, dA, dB = oracle.norm_backward(dY, X, g, eps, W, A, B, s)
    h = 1e-6
    for idx in itertools.product(range(X.shape[0]), range(X.shape[1])):
        Xp, Xm = X.copy(), X.copy()
        Xp[idx] += h
        Xm[idx] -= h
        fd = (loss(Xp, A, B) - loss(Xm, A, B)) / (2 * h)
        assert abs(fd - dX[idx]) <= 1e-6 * max(1.0, abs(dX[idx])), (idx, fd, dX[idx])
    for P, G, which in ((A, dA, "A"), (B, dB, "B")):
        for idx in itertools.product(*map(range, P.shape)):
            Pp, Pm = P.copy(), P.copy()
            Pp[idx] += h
            Pm[idx] -= h
            args_p = (Pp, B) if which == "A" else (A, Pp)
            args_m = (Pm, B) if which == "A" else (A, Pm)
            fd = (loss(X, *args_p) - loss(X, *args_m)) / (2 * h)
            assert abs(fd - G[idx]) <= 1e-6 * max(1.0, abs(G[idx]))


def test_norm_scale_invariance():
    """With eps = 0, RMSNorm(c X) = RMSNorm(X) for c > 0: H does not change and
    the input gradient scales by 1 / c (the adapter gradients do not change)."""
    X, g, _, W, A, B, dY, s = norm_case(23)
    c = 3.7
    H1, U1, _ = oracle.norm_forward(X, g, 0.0, W, A, B, s)
    H2, U2, _ = oracle.norm_forward(c * X, g, 0.0, W, A, B, s)
    np.testing.assert_allclose(H2, H1, rtol=1e-12, atol=1e-12)
    dX1, dA1, dB1 = oracle.norm_backward(dY, X, g, 0.0, W, A, B, s)
    dX2, dA2, dB2 = oracle.norm_backward(dY, c * X, g, 0.0, W, A, B, s)
    np.testing.assert_allclose(dX2, dX1 / c, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dA2, dA1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dB2, dB1, rtol=1e-11, atol=1e-12)


def test_norm_input_gradient_is_orthogonal_to_the_input():
    """With eps = 0 the rows of RMSNorm(X) do not change along X's own rows, so
    every row of dX is orthogonal to the same row of X (a property of the
    norm's Jacobian that the closed form must keep)."""
    X, g, _, W, A, B, dY, s = norm_case(24)
    dX, _, _ = oracle.norm_backward(dY, X, g, 0.0, W, A, B, s)
    dots = np.sum(dX * X, axis=1)
    assert np.all(np.abs(dots) <= 1e-11 * np.abs(dX).max() * np.abs(X).max() * X.shape[1])
