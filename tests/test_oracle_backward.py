"""Pins for the fp64 backward oracle (oracle/backward.py).

The pages fix only what the backward pass consumes (page "FlashAttention/es", section "Paso hacia
atrás y recomputación": S and P recomputed from the saved L and dO); its result is the gradient
of the forward definition.  So the pins are the mathematics of a gradient, checked against code
that shares nothing with the backward oracle's formulas:
  * B1  central finite differences of the forward oracle (oracle.attention), every input element,
        every variant: a dropped term, a wrong sign, a transposed product or a missing soft-cap
        factor in the backward formulas fails here;
  * B2  torch autograd through torch's own fp64 scaled_dot_product_attention (masks as boolean
        masks, ALiBi as an additive bias);
  * B3  closed forms: N = 1; keys with one common value row; the key-gradient sum that the
        softmax Jacobian makes zero; D_i = dO_i . O_i;
  * B4  the error scales of backward_magnitudes, which set the GPU tolerance of the backward
        pass: they bound the gradients, are attained exactly by the worst-case rounding of the
        operands (formed by torch autograd with perturbed operands, not by restated formulas),
        and bound random roundings.
"""
import numpy as np
import pytest
import torch

import oracle


def rnd(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def variant_kwargs(mask, N, H, B=1, seed=0, alibi=False, softcap=0.0, window=4):
    kw = {"mask": mask, "softcap": softcap}
    if mask == "window":
        kw["window"] = window
    if mask == "document":
        rng = np.random.default_rng(seed + 7)
        offs = []
        for _ in range(B):
            cuts = np.sort(rng.choice(np.arange(1, N), size=min(2, N - 1), replace=False))
            offs.append(np.concatenate([[0], cuts, [N]]))
        kw["doc_offsets"] = np.array(offs)
    if alibi:
        kw["slopes"] = np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)])
    return kw


VARIANTS = [
    ("none", False, 0.0), ("causal", False, 0.0), ("window", False, 0.0),
    ("document", False, 0.0), ("causal", True, 0.0), ("none", False, 2.5),
    ("document", False, 1.5), ("window", True, 3.0),
]


@pytest.mark.parametrize("mask,alibi,cap", VARIANTS)
def test_b1_finite_differences(mask, alibi, cap):
    """B1: every element of dQ, dK, dV equals the central difference of sum(O * G)."""
    B, H, N, d, scale = 1, 2, 9, 4, 0.7
    q, k, v = rnd((B, H, N, d), 1), rnd((B, H, N, d), 2), rnd((B, H, N, d), 3)
    g = rnd((B, H, N, d), 4)
    kw = variant_kwargs(mask, N, H, B, alibi=alibi, softcap=cap)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, scale, **kw)

    def loss(q_, k_, v_):
        o, _ = oracle.attention(q_, k_, v_, scale, **kw)
        return float((o * g).sum())

    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            fd[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                       loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        err = np.abs(fd - grad).max()
        assert err <= 1e-7 * (1.0 + np.abs(grad).max()), (name, err)


@pytest.mark.parametrize("mask,alibi", [("none", False), ("causal", False), ("window", False),
                                        ("document", False), ("causal", True), ("none", True)])
def test_b2_torch_autograd(mask, alibi):
    """B2: torch autograd of torch's fp64 scaled_dot_product_attention."""
    B, H, N, d, scale = 1, 2, 40, 16, 0.3
    q, k, v, g = (rnd((B, H, N, d), s) for s in (11, 12, 13, 14))
    kw = variant_kwargs(mask, N, H, B, alibi=alibi, window=7)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, scale, **kw)
    rows = np.arange(N)
    ok = oracle.allowed(rows, rows, N, mask, kw.get("window", 0),
                        None if "doc_offsets" not in kw else kw["doc_offsets"][0])
    bias = np.where(ok, 0.0, -np.inf)[None, None].repeat(H, axis=1)
    if alibi:
        dist = (rows[:, None] - rows[None, :]).astype(np.float64)
        bias = bias - kw["slopes"][None, :, None, None] * dist[None, None]
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv,
                                                           attn_mask=torch.tensor(bias),
                                                           scale=scale)
    out.backward(torch.tensor(g))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(mine - ref.numpy()).max() <= 1e-10


def test_b3_single_key():
    """B3: N = 1 gives P = [[1]]: dV = dO and dQ = dK = 0."""
    q, k, v, g = (rnd((1, 3, 1, 8), s) for s in (1, 2, 3, 4))
    dq, dk, dv = oracle.attention_backward(q, k, v, g, 0.5, mask="causal")
    assert np.array_equal(dv, g)
    assert np.abs(dq).max() == 0.0 and np.abs(dk).max() == 0.0


@pytest.mark.parametrize("cap", [0.0, 2.0])
def test_b3_constant_values(cap):
    """B3: if every key carries the same value row, O does not depend on Q or K: dQ = dK = 0, and
    dV_j = sum_i P_ij dO_i still sums (over j) to sum_i dO_i."""
    B, H, N, d = 1, 2, 12, 6
    q, k = rnd((B, H, N, d), 5), rnd((B, H, N, d), 6)
    v = np.broadcast_to(rnd((B, H, 1, d), 7), (B, H, N, d)).copy()
    g = rnd((B, H, N, d), 8)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, 0.4, mask="causal", softcap=cap)
    assert np.abs(dq).max() <= 1e-12 and np.abs(dk).max() <= 1e-12
    assert np.abs(dv.sum(axis=2) - g.sum(axis=2)).max() <= 1e-12


def test_b3_key_gradient_sum():
    """B3: without soft-cap every row of dS sums to zero, so sum_j dK_j = scale * sum_i q_i *
    (sum_j dS_ij) = 0."""
    B, H, N, d = 1, 2, 15, 8
    q, k, v, g = (rnd((B, H, N, d), s) for s in (21, 22, 23, 24))
    for mask in ("none", "causal", "window"):
        _, dk, _ = oracle.attention_backward(q, k, v, g, 0.6, mask=mask, window=5)
        assert np.abs(dk.sum(axis=2)).max() <= 1e-12


def test_b3_row_dot_identity():
    """B3: D_i = sum_j P_ij dP_ij equals dO_i . O_i, the form the kernels use."""
    B, H, N, d = 1, 1, 20, 8
    q, k, v, g = (rnd((B, H, N, d), s) for s in (31, 32, 33, 34))
    o, _ = oracle.attention(q, k, v, 0.5, mask="causal")
    s = 0.5 * q[0, 0] @ k[0, 0].T
    s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    direct = (p * (g[0, 0] @ v[0, 0].T)).sum(axis=1)
    assert np.abs(oracle.backward_row_dot(o, g)[0, 0] - direct).max() <= 1e-12


# --- B4: the error scales M of backward_magnitudes ------------------------------------------
# M is defined as the largest change of a gradient element when one operand of every product
# term is rounded to a relative precision u (P in dV = P^T dO; dS in dQ, dK; D_i = dO_i . O_i
# formed from an O rounded the same way).  The pins below perturb those operands inside torch
# autograd (a hook on the gradient that flows into the scores, a factor on P in the forward) and
# let autograd form the perturbed gradients, so no backward formula is restated here:
#   * triangle inequality: |gradient| <= M element-wise;
#   * attainment: with Q, K >= 0 (dQ, dK) or dO >= 0 (dV) every term of a gradient element has
#     one sign, so the worst-case rounding (relative +u on |dS|, D moved by u sum|dO O| against
#     the terms, P scaled by 1 + u) moves every element by exactly u M;
#   * random roundings within u move every element by at most u M.
# A dropped scale, a dropped soft-cap factor, a |dS| counted twice, a transposed product or a
# missing D term in M each break the attainment equality.
U = 2.0 ** -8


def _autograd(q, k, v, g, scale, b, h, kw, ds_hook=None, p_factor=None):
    """Gradients of sum(O * g) for head (b, h) by torch autograd (fp64).  ds_hook(grad, P, O)
    replaces the gradient reaching the masked scores; p_factor multiplies P where it enters P V.
    Returns (dQ, dK, dV, P, O) as numpy arrays."""
    N = q.shape[2]
    rows = np.arange(N)
    off = None if kw.get("doc_offsets") is None else kw["doc_offsets"][b]
    ok = torch.tensor(oracle.allowed(rows, rows, N, kw["mask"], kw.get("window", 0), off))
    Q, K, V = (torch.tensor(x[b, h], requires_grad=True) for x in (q, k, v))
    t = scale * (Q @ K.T)
    cap = kw.get("softcap", 0.0)
    s = cap * torch.tanh(t / cap) if cap else t
    if kw.get("slopes") is not None:
        dist = torch.tensor((rows[:, None] - rows[None, :]).astype(np.float64))
        s = s - float(kw["slopes"][h]) * dist
    s = s.masked_fill(~ok, float("-inf"))
    P = torch.softmax(s, dim=-1)
    O = P @ V
    if ds_hook is not None:
        Pd, Od = P.detach(), O.detach()
        s.register_hook(lambda grad: ds_hook(grad, Pd, Od))
    Pv = P if p_factor is None else P * torch.tensor(p_factor)
    Ov = Pv @ V
    (Ov * torch.tensor(g[b, h])).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy(), P.detach().numpy(), O.detach().numpy()


B4_VARIANTS = [("none", False, 0.0), ("causal", False, 0.0), ("window", True, 0.0),
               ("document", False, 0.0), ("causal", False, 2.0), ("window", True, 1.5)]


def _b4_inputs(seed, positive_qk=False, positive_do=False):
    B, H, N, d = 1, 2, 24, 8
    q, k, v, g = (rnd((B, H, N, d), seed + i) for i in range(4))
    if positive_qk:
        q, k = np.abs(q), np.abs(k)
    if positive_do:
        g = np.abs(g)
    return q, k, v, g


@pytest.mark.parametrize("mask,alibi,cap", B4_VARIANTS)
def test_b4_magnitudes_bound_gradients(mask, alibi, cap):
    """Triangle inequality: every gradient element is at most its M."""
    q, k, v, g = _b4_inputs(40)
    kw = variant_kwargs(mask, q.shape[2], q.shape[1], alibi=alibi, softcap=cap, window=5)
    grads = oracle.attention_backward(q, k, v, g, 0.7, **kw)
    mags = oracle.backward_magnitudes(q, k, v, g, 0.7, **kw)
    for gr, m in zip(grads, mags):
        assert np.all(np.abs(gr) <= m * (1 + 1e-12) + 1e-300)


@pytest.mark.parametrize("mask,alibi,cap", B4_VARIANTS)
def test_b4_worst_case_rounding_attains_m(mask, alibi, cap):
    """Attainment: the worst-case operand rounding moves dQ, dK (Q, K >= 0) and dV (dO >= 0) by
    exactly u M, element by element."""
    scale = 0.7
    q, k, v, g = _b4_inputs(50, positive_qk=True)
    H, N = q.shape[1], q.shape[2]
    kw = variant_kwargs(mask, N, H, alibi=alibi, softcap=cap, window=5)
    mq, mk, _ = oracle.backward_magnitudes(q, k, v, g, scale, **kw)

    def worst(grad, P, O):
        # dS rounded up in magnitude by u, and D_i = dO_i . O_i off by u sum_c |dO_ic O_ic| in
        # the direction that adds P_ij times it to every dS_ij of the row
        dD = U * (torch.tensor(g[0, h]) * O).abs().sum(dim=1)
        return grad + U * grad.abs() + P * dD[:, None]

    for h in range(H):
        dq0, dk0, _, _, _ = _autograd(q, k, v, g, scale, 0, h, kw)
        dq1, dk1, _, _, _ = _autograd(q, k, v, g, scale, 0, h, kw, ds_hook=worst)
        np.testing.assert_allclose(dq1 - dq0, U * mq[0, h], rtol=1e-9, atol=1e-15)
        np.testing.assert_allclose(dk1 - dk0, U * mk[0, h], rtol=1e-9, atol=1e-15)

    q, k, v, g = _b4_inputs(60, positive_do=True)
    _, _, mv = oracle.backward_magnitudes(q, k, v, g, scale, **kw)
    for h in range(H):
        _, _, dv0, _, _ = _autograd(q, k, v, g, scale, 0, h, kw)
        _, _, dv1, _, _ = _autograd(q, k, v, g, scale, 0, h, kw,
                                    p_factor=np.full((N, N), 1.0 + U))
        np.testing.assert_allclose(dv1 - dv0, U * mv[0, h], rtol=1e-9, atol=1e-15)


@pytest.mark.parametrize("mask,alibi,cap", B4_VARIANTS[:4])
def test_b4_random_rounding_within_m(mask, alibi, cap):
    """Random roundings of the operands within relative u (signs of Q, K, dO arbitrary) move
    every gradient element by at most u M."""
    scale = 0.7
    q, k, v, g = _b4_inputs(70)
    H, N = q.shape[1], q.shape[2]
    kw = variant_kwargs(mask, N, H, alibi=alibi, softcap=cap, window=5)
    mq, mk, mv = oracle.backward_magnitudes(q, k, v, g, scale, **kw)
    rng = np.random.default_rng(3)
    for h in range(H):
        dq0, dk0, dv0, _, _ = _autograd(q, k, v, g, scale, 0, h, kw)
        for _ in range(3):
            dl = torch.tensor(rng.uniform(-U, U, (N, N)))
            eps = torch.tensor(rng.uniform(-U, U, (N, q.shape[3])))

            def rand_round(grad, P, O, dl=dl, eps=eps):
                dD = (torch.tensor(g[0, h]) * O * eps).sum(dim=1)  # D from O (1 + eps)
                return grad * (1 + dl) - P * dD[:, None]

            dq1, dk1, _, _, _ = _autograd(q, k, v, g, scale, 0, h, kw, ds_hook=rand_round)
            _, _, dv1, _, _ = _autograd(q, k, v, g, scale, 0, h, kw,
                                        p_factor=1 + rng.uniform(-U, U, (N, N)))
            for d1, d0, m in ((dq1, dq0, mq), (dk1, dk0, mk), (dv1, dv0, mv)):
                assert np.all(np.abs(d1 - d0) <= U * m[0, h] * (1 + 1e-9) + 1e-15)
