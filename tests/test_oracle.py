"""Pins for the CPU oracle (runs without a GPU).

Each test checks the oracle against something other than itself: numbers the
pages print, closed forms, invariants of the softmax-attention definition,
finite differences, a pure-Python brute force, or an independent torch CPU
float64 autograd evaluation.  They are chosen so that a plausible slip in the
oracle (a dropped scale, a wrong sign in dS, a transposed operand, a wrong GQA
head mapping, a causal off-by-one) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention_backward, attention_dq_rows, attention_forward, kv_head, softmax_probs, visible_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def qkv(B=1, Hq=2, Hkv=1, N=7, D=4, seed=0, scale=1.0):
    return (rnd((B, Hq, N, D), seed, scale), rnd((B, Hkv, N, D), seed + 1, scale),
            rnd((B, Hkv, N, D), seed + 2, scale))


# ---------------------------------------------------------------- pages' numbers

def test_page_softmax_table():
    """FlashStieltjes page, 'Why touch softmax' figure data table (softmax column)."""
    g = json.load(open(os.path.join(GOLDEN, "softmax_geometric_scores.json")))
    n = g["n_keys"]
    # one query, D=1, scale=1: q=1, k_j = step*j  ->  s_j = step*j
    q = np.ones((1, 1, n, 1))
    k = (g["score_step"] * np.arange(n, dtype=np.float64)).reshape(1, 1, n, 1)
    v = np.eye(n).reshape(1, 1, n, n)          # O row = the probability row itself
    q_full = np.zeros((1, 1, n, n)); q_full[..., 0] = 1.0
    k_full = np.zeros((1, 1, n, n)); k_full[..., 0] = k[..., 0]
    O, _ = attention_forward(q_full, k_full, v, 1.0, False, rows=[0])
    p = O[0, 0, 0]
    for row in g["rows"]:
        j = int(round(row["gap"] / -g["score_step"]))
        want, sig = row["softmax"], row["sig_digits"]
        got = float(f"{p[j]:.{sig}g}")
        assert got == pytest.approx(want, rel=1e-9), (row, p[j])


@pytest.mark.parametrize("causal", [False, True])
def test_hand_example(causal):
    g = json.load(open(os.path.join(GOLDEN, "hand_example_2x2.json")))
    q, k, v, do = (np.array(g[n], dtype=np.float64).reshape(1, 1, 2, 1) for n in ("q", "k", "v", "do"))
    exp = g["causal" if causal else "noncausal"]
    O, L = attention_forward(q, k, v, g["scale"], causal)
    np.testing.assert_allclose(O.reshape(2, 1), exp["o"], atol=1e-14)
    np.testing.assert_allclose(L.reshape(2), exp["lse"], atol=1e-14)
    dq, dk, dv = attention_backward(q, k, v, do, g["scale"], causal)
    np.testing.assert_allclose(dq.reshape(2, 1), exp["dq"], atol=1e-14)
    np.testing.assert_allclose(dk.reshape(2, 1), exp["dk"], atol=1e-14)
    np.testing.assert_allclose(dv.reshape(2, 1), exp["dv"], atol=1e-14)


# ------------------------------------------------------------ brute force, tiny

def brute_force(q, k, v, do, scale, causal):
    """Scalar pure-Python loops over the definition (float64 via math.exp)."""
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    O = np.zeros_like(q); L = np.zeros(q.shape[:3])
    dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kvh = h // grp
            P = [[0.0] * N for _ in range(N)]
            for i in range(N):
                s = [scale * sum(q[b, h, i, d] * k[b, kvh, j, d] for d in range(D)) for j in range(N)]
                vis = [j for j in range(N) if (j <= i or not causal)]
                z = sum(math.exp(s[j]) for j in vis)
                L[b, h, i] = math.log(z)
                for j in vis:
                    P[i][j] = math.exp(s[j]) / z
                for d in range(D):
                    O[b, h, i, d] = sum(P[i][j] * v[b, kvh, j, d] for j in range(N))
            for i in range(N):
                Di = sum(do[b, h, i, d] * O[b, h, i, d] for d in range(D))
                for j in range(N):
                    dPij = sum(do[b, h, i, d] * v[b, kvh, j, d] for d in range(D))
                    dSij = P[i][j] * (dPij - Di)
                    for d in range(D):
                        dq[b, h, i, d] += scale * dSij * k[b, kvh, j, d]
                        dk[b, kvh, j, d] += scale * dSij * q[b, h, i, d]
                        dv[b, kvh, j, d] += P[i][j] * do[b, h, i, d]
    return O, L, dq, dk, dv


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_gqa(causal):
    q, k, v = qkv(B=2, Hq=4, Hkv=2, N=5, D=3, seed=3, scale=0.8)
    do = rnd(q.shape, 9)
    O, L, dq, dk, dv = brute_force(q, k, v, do, 0.9, causal)
    O2, L2 = attention_forward(q, k, v, 0.9, causal, block=2)
    dq2, dk2, dv2 = attention_backward(q, k, v, do, 0.9, causal, block=2)
    for a, b_ in ((O, O2), (L, L2), (dq, dq2), (dk, dk2), (dv, dv2)):
        np.testing.assert_allclose(a, b_, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------- invariants

@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    q, k, _ = qkv(N=33, D=8, seed=5, scale=2.0)
    rows = np.arange(33)
    _, P, _ = softmax_probs(q[0, 0], k[0, 0], 0.5, rows, causal)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
    if causal:
        assert np.all(P[np.triu_indices(33, 1)] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_values(causal):
    N, D = 9, 6
    q, _, v = qkv(N=N, D=D, seed=11)
    k = np.broadcast_to(rnd((1, 1, 1, D), 12), (1, 1, N, D)).copy()
    O, L = attention_forward(q, k, v, 0.7, causal)
    for h in range(2):
        for i in range(N):
            n_vis = i + 1 if causal else N
            np.testing.assert_allclose(O[0, h, i], v[0, 0, :n_vis].mean(axis=0), atol=1e-13)
            s0 = 0.7 * q[0, h, i] @ k[0, 0, 0]
            assert L[0, h, i] == pytest.approx(s0 + math.log(n_vis), abs=1e-13)


def test_causal_row_zero_is_first_value():
    q, k, v = qkv(N=12, D=5, seed=13)
    O, L = attention_forward(q, k, v, 1.3, True)
    for h in range(2):
        np.testing.assert_allclose(O[0, h, 0], v[0, 0, 0], atol=1e-14)
        assert L[0, h, 0] == pytest.approx(1.3 * q[0, h, 0] @ k[0, 0, 0], abs=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_pass_through(causal):
    q, k, _ = qkv(N=10, D=4, seed=17, scale=3.0)
    c = rnd((4,), 18)
    v = np.broadcast_to(c, (1, 1, 10, 4)).copy()
    O, _ = attention_forward(q, k, v, 1.0, causal)
    np.testing.assert_allclose(O, np.broadcast_to(c, O.shape), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_is_uniform(causal):
    N = 8
    q, k, v = qkv(N=N, D=4, seed=19)
    O, L = attention_forward(q, k, v, 0.0, causal)
    for i in range(N):
        n_vis = i + 1 if causal else N
        np.testing.assert_allclose(O[0, :, i], np.broadcast_to(v[0, 0, :n_vis].mean(0), (2, 4)), atol=1e-14)
        np.testing.assert_allclose(L[0, :, i], math.log(n_vis), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_single_token(causal):
    q, k, v = qkv(N=1, D=4, seed=23)
    O, L = attention_forward(q, k, v, 0.6, causal)
    np.testing.assert_allclose(O[0, 0, 0], v[0, 0, 0], atol=1e-15)
    assert L[0, 0, 0] == pytest.approx(0.6 * q[0, 0, 0] @ k[0, 0, 0], abs=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift(causal):
    q, k, v = qkv(N=11, D=5, seed=29)
    c = rnd((5,), 30)
    O, L = attention_forward(q, k, v, 0.8, causal)
    O2, L2 = attention_forward(q, k + c, v, 0.8, causal)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(L2, L + 0.8 * np.einsum("bhnd,d->bhn", q, c), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_affine_values(causal):
    q, k, v = qkv(N=11, D=5, seed=31)
    O, _ = attention_forward(q, k, v, 0.8, causal)
    O2, _ = attention_forward(q, k, -2.5 * v + 0.75, 0.8, causal)
    np.testing.assert_allclose(O2, -2.5 * O + 0.75, atol=1e-12)


def test_key_permutation_noncausal():
    q, k, v = qkv(N=13, D=5, seed=37)
    perm = np.random.default_rng(38).permutation(13)
    O, L = attention_forward(q, k, v, 0.8, False)
    O2, L2 = attention_forward(q, k[:, :, perm], v[:, :, perm], 0.8, False)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(L2, L, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_repeated_mha(causal):
    q, k, v = qkv(B=2, Hq=6, Hkv=2, N=7, D=4, seed=41)
    do = rnd(q.shape, 42)
    k_rep = np.repeat(k, 3, axis=1)
    v_rep = np.repeat(v, 3, axis=1)
    O, L = attention_forward(q, k, v, 0.5, causal)
    O2, L2 = attention_forward(q, k_rep, v_rep, 0.5, causal)
    np.testing.assert_allclose(O, O2, atol=1e-13)
    np.testing.assert_allclose(L, L2, atol=1e-13)
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, causal)
    dq2, dk2, dv2 = attention_backward(q, k_rep, v_rep, do, 0.5, causal)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(2, 2, 3, 7, 4).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(2, 2, 3, 7, 4).sum(axis=2), atol=1e-13)
    assert [kv_head(h, 6, 2) for h in range(6)] == [0, 0, 0, 1, 1, 1]


def test_hard_attention_limit():
    q, k, v = qkv(N=9, D=4, seed=43)
    S = np.einsum("bhid,bkjd->bhij", q, k)
    O, _ = attention_forward(q, k, v, 1e3, False)
    arg = S.argmax(axis=-1)
    for h in range(2):
        np.testing.assert_allclose(O[0, h], v[0, 0, arg[0, h]], atol=1e-6)


def test_textbook_softmax_small_scores():
    q, k, v = qkv(N=6, D=3, seed=47, scale=0.3)
    S = 0.9 * np.einsum("bhid,bkjd->bhij", q, k)
    e = np.exp(S)                                   # no max subtraction: scores are small
    P = e / e.sum(-1, keepdims=True)
    O_ref = np.einsum("bhij,bkjd->bhid", P, v)
    O, L = attention_forward(q, k, v, 0.9, False)
    np.testing.assert_allclose(O, O_ref, atol=1e-14)
    np.testing.assert_allclose(L, np.log(e.sum(-1)), atol=1e-14)


def test_row_subset_matches_full():
    q, k, v = qkv(B=1, Hq=2, Hkv=2, N=40, D=4, seed=53)
    rows = np.array([0, 3, 17, 39])
    O, L = attention_forward(q, k, v, 0.5, True, block=7)
    O2, L2 = attention_forward(q, k, v, 0.5, True, rows=rows)
    np.testing.assert_allclose(O2, O[:, :, rows], atol=1e-14)
    np.testing.assert_allclose(L2, L[:, :, rows], atol=1e-14)
    do = rnd(q.shape, 54)
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, True, block=9)
    keys = np.array([1, 5, 38])
    dq2, dk2, dv2 = attention_backward(q, k, v, do, 0.5, True, rows=rows, keys=keys, block=2)
    np.testing.assert_allclose(dq2, dq[:, :, rows], atol=1e-13)
    np.testing.assert_allclose(dk2, dk[:, :, keys], atol=1e-13)
    np.testing.assert_allclose(dv2, dv[:, :, keys], atol=1e-13)


def test_visible_mask_top_left():
    m = visible_mask(np.arange(4), 4, True)
    assert m.tolist() == [[True, False, False, False], [True, True, False, False],
                          [True, True, True, False], [True, True, True, True]]


# ------------------------------------------------------------------ backward

@pytest.mark.parametrize("N", [1, 3, 7])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(N, causal):
    """Central differences of L = sum(O * dO) in float64."""
    q, k, v = qkv(B=1, Hq=2, Hkv=1, N=N, D=4, seed=100 + N)
    do = rnd(q.shape, 200 + N)
    scale, h = 0.7, 1e-6
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal)

    def loss(q_, k_, v_):
        O, _ = attention_forward(q_, k_, v_, scale, causal)
        return float((O * do).sum())

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        args = [q, k, v]
        num = np.zeros_like(args[which])
        for idx in np.ndindex(*args[which].shape):
            plus = [a.copy() for a in args]; minus = [a.copy() for a in args]
            plus[which][idx] += h; minus[which][idx] -= h
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        err = np.abs(num - grad).max() / max(np.abs(grad).max(), 1e-300)
        assert err < 1e-6 or np.abs(num - grad).max() < 1e-9, (which, err)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_row_identity_and_totals(causal):
    q, k, v = qkv(B=1, Hq=4, Hkv=2, N=19, D=6, seed=61)
    do = rnd(q.shape, 62)
    dq, dk, dv, delta = attention_backward(q, k, v, do, 0.6, causal, return_delta=True)
    # sum_j dS_ij = 0 for every row  =>  sum_j dK_j = 0 per (b, kv, d)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # sum_j dV_j = sum over the group of sum_i dO_i
    tot = do.reshape(1, 2, 2, 19, 6).sum(axis=(2, 3))
    np.testing.assert_allclose(dv.sum(axis=2), tot, atol=1e-12)
    O, _ = attention_forward(q, k, v, 0.6, causal)
    np.testing.assert_allclose(delta, (O * do).sum(-1), atol=1e-13)


def test_backward_constant_values():
    q, k, _ = qkv(N=8, D=4, seed=67)
    v = np.broadcast_to(rnd((4,), 68), (1, 1, 8, 4)).copy()
    do = rnd(q.shape, 69)
    dq, dk, dv = attention_backward(q, k, v, do, 0.9, True)
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)
    np.testing.assert_allclose(dk, 0.0, atol=1e-13)
    _, P0, _ = softmax_probs(q[0, 0], k[0, 0], 0.9, np.arange(8), True)
    _, P1, _ = softmax_probs(q[0, 1], k[0, 0], 0.9, np.arange(8), True)
    np.testing.assert_allclose(dv[0, 0], P0.T @ do[0, 0] + P1.T @ do[0, 1], atol=1e-13)


@pytest.mark.parametrize("scale", [0.4, -0.3])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_torch_cpu_autograd(causal, scale):
    """Second, independent CPU implementation: torch float64 autograd (a negative scale too)."""
    torch = pytest.importorskip("torch")
    q, k, v = qkv(B=1, Hq=4, Hkv=2, N=23, D=8, seed=71)
    do = rnd(q.shape, 72)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    kr = tk.repeat_interleave(2, dim=1); vr = tv.repeat_interleave(2, dim=1)
    S = scale * torch.matmul(tq, kr.transpose(-1, -2).contiguous())
    if causal:
        S = S.masked_fill(torch.ones(23, 23, dtype=torch.bool).triu(1), float("-inf"))
    O = torch.matmul(torch.softmax(S, dim=-1), vr)
    (O * torch.tensor(do)).sum().backward()
    O2, L2 = attention_forward(q, k, v, scale, causal)
    np.testing.assert_allclose(O2, O.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(L2, torch.logsumexp(S, -1).detach().numpy(), atol=1e-12)
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)
    rows = np.array([0, 5, 22])
    np.testing.assert_allclose(attention_dq_rows(q, k, v, do, scale, causal, rows), tq.grad.numpy()[:, :, rows],
                               atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_dq_rows_finite_differences(causal):
    """attention_dq_rows against central differences of L = sum(O * dO) in the listed rows of q."""
    q, k, v = qkv(B=1, Hq=2, Hkv=1, N=6, D=3, seed=91)
    do = rnd(q.shape, 92)
    rows = np.array([1, 5])
    g = attention_dq_rows(q, k, v, do, 0.8, causal, rows)
    h = 1e-6
    for hq in range(2):
        for ri, r in enumerate(rows):
            for d in range(3):
                qp, qm = q.copy(), q.copy()
                qp[0, hq, r, d] += h
                qm[0, hq, r, d] -= h
                lp = float((attention_forward(qp, k, v, 0.8, causal)[0] * do).sum())
                lm = float((attention_forward(qm, k, v, 0.8, causal)[0] * do).sum())
                assert abs((lp - lm) / (2 * h) - g[0, hq, ri, d]) < 1e-7


def test_rejects_bad_shapes():
    q, k, v = qkv(B=1, Hq=3, Hkv=2, N=4, D=4)
    with pytest.raises(ValueError):
        attention_forward(q, k, v, 1.0, False)
