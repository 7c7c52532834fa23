"""Pins of the fp64 CPU oracle against things other than itself (CPU only).

The pages print no attention values for any input, so the oracle is pinned by
the mathematics of the definition it implements ("FlashAttention." plate:
standard attention is S = QK^T, a row softmax, then PV; the tiled method is
the same result up to rounding, section "Never write the scores"):

  * brute force in 40-digit decimal arithmetic on tiny inputs (no max shift,
    explicit sums), including arbitrary masks at tile size 1;
  * torch fp64 library routines: scaled_dot_product_attention, logsumexp, and
    autograd through an explicit softmax;
  * closed forms: equal scores give the mean of the visible V rows and
    LSE = ln(count); one-hot scores select a V row; causal row 0 is V_0;
  * invariants: rows of P sum to one, shift and permutation invariance, mask
    identities (all-ones tile mask == dense, lower-triangular tile mask with
    causal == causal);
  * backward: central finite differences of L = sum(dO * O), autograd, and
    the identities sum_j dV_j = sum_i dO_i, sum_j dK_j = 0,
    D_i = sum_j P_ij dP_ij = dO_i . O_i, causal dQ_0 = 0.
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(1234)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- brute force
def brute_decimal(q, k, v, scale, vis):
    """Attention of one head in 40-digit decimal: P = exp(S)/sum exp(S), O = PV."""
    getcontext().prec = 40
    N, d = q.shape
    sc = Decimal(float(scale))
    O = np.zeros((N, d))
    L = np.zeros(N)
    for i in range(N):
        z = Decimal(0)
        w = []
        for j in range(N):
            if vis(i, j):
                s = sc * sum(Decimal(float(q[i, c])) * Decimal(float(k[j, c])) for c in range(d))
                e = s.exp()
                w.append((j, e))
                z += e
        if not w:
            L[i] = -math.inf
            continue
        for c in range(d):
            O[i, c] = float(sum(e * Decimal(float(v[j, c])) for j, e in w) / z)
        L[i] = float(z.ln())
    return O, L


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 1), (3, 2), (5, 3), (8, 4)])
def test_forward_matches_decimal_brute_force(N, d, causal):
    q, k, v = rand(N, d), rand(N, d), rand(N, d)
    scale = 0.7
    o, lse = oracle.forward(q, k, v, scale, causal)
    vis = (lambda i, j: j <= i) if causal else (lambda i, j: True)
    ob, lb = brute_decimal(q, k, v, scale, vis)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_random_mask_at_tile_size_one_matches_brute_force(causal):
    N, d = 7, 3
    q, k, v = rand(N, d), rand(N, d), rand(N, d)
    mask = (RNG.random((N, N)) < 0.5).astype(np.uint8)
    mask[2, :] = 0  # one row fully masked: O = 0, LSE = -inf
    mask[5, :] = 0
    mask[5, 5] = 1
    o, lse = oracle.forward(q, k, v, 0.5, causal, block_mask=mask, mask_block=1)

    def vis(i, j):
        return bool(mask[i, j]) and (j <= i or not causal)

    ob, lb = brute_decimal(q, k, v, 0.5, vis)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    assert lse[2] == -math.inf and np.all(o[2] == 0.0)
    fin = np.isfinite(lb)
    assert np.array_equal(np.isfinite(lse), fin)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-13)


def test_rectangular_tile_mask_matches_brute_force():
    """Tiles of 3 over N=8 (a ragged last tile): mask[i//3][j//3]."""
    N, d, mb = 8, 2, 3
    q, k, v = rand(N, d), rand(N, d), rand(N, d)
    mask = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 0]], dtype=np.uint8)
    o, lse = oracle.forward(q, k, v, 1.1, False, block_mask=mask, mask_block=mb)
    ob, lb = brute_decimal(q, k, v, 1.1, lambda i, j: bool(mask[i // mb, j // mb]))
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


# ------------------------------------------------------------ library routine
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(17, 8), (130, 16), (257, 64)])
def test_forward_matches_torch_sdpa_fp64(N, d, causal):
    q, k, v = rand(2, N, d), rand(2, N, d), rand(2, N, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.forward(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    s = scale * tq @ tk.transpose(-1, -2)
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_block_mask_matches_torch_sdpa_with_explicit_mask():
    N, d, mb = 200, 16, 32
    nb = -(-N // mb)
    q, k, v = rand(3, N, d), rand(3, N, d), rand(3, N, d)
    mask = (RNG.random((nb, nb)) < 0.6).astype(np.uint8)
    np.fill_diagonal(mask, 1)
    o, _ = oracle.forward(q, k, v, 0.25, False, block_mask=mask, mask_block=mb)
    full = torch.from_numpy(mask.astype(bool)).repeat_interleave(mb, 0).repeat_interleave(mb, 1)
    full = full[:N, :N]
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(x) for x in (q, k, v)),
                                         attn_mask=full, scale=0.25)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_equal_scores_give_mean_of_v(causal):
    N, d = 37, 5
    q, k, v = np.zeros((N, d)), rand(N, d), rand(N, d)
    o, lse = oracle.forward(q, k, v, 0.3, causal)
    if causal:
        mean = np.cumsum(v, axis=0) / np.arange(1, N + 1)[:, None]
        np.testing.assert_allclose(lse, np.log(np.arange(1, N + 1)), rtol=0, atol=1e-14)
    else:
        mean = np.broadcast_to(v.mean(axis=0), (N, d))
        np.testing.assert_allclose(lse, np.full(N, math.log(N)), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o, mean, rtol=0, atol=1e-14)


def test_one_hot_scores_select_a_v_row():
    d = 6
    N = d
    c = 120.0
    scale = 0.5  # scale * c = 60: every other weight is e^-60 of the chosen one
    k = c * np.eye(d)
    v = rand(N, d)
    t = np.array([3, 0, 5, 1, 4, 2])
    q = np.eye(d)[t]
    o, lse = oracle.forward(q, k, v, scale, False)
    np.testing.assert_allclose(o, v[t], rtol=1e-20, atol=1e-20 * np.abs(v).max() + 1e-24)
    np.testing.assert_allclose(lse, np.full(N, 60.0), rtol=0, atol=1e-20 + 1e-14)


def test_causal_row_zero_is_v0_exactly():
    N, d = 50, 7
    q, k, v = rand(N, d), rand(N, d), rand(N, d)
    o, lse = oracle.forward(q, k, v, 0.9, True)
    assert np.array_equal(o[0], v[0])
    assert lse[0] == 0.9 * float(np.dot(q[0], k[0])) or abs(lse[0] - 0.9 * np.dot(q[0], k[0])) < 1e-15


def test_fully_masked_rows_give_zero_and_minus_inf():
    N, d = 20, 4
    q, k, v = rand(N, d), rand(N, d), rand(N, d)
    mask = np.ones((4, 4), dtype=np.uint8)
    mask[1, :] = 0  # rows 5..9 see nothing
    o, lse = oracle.forward(q, k, v, 1.0, False, block_mask=mask, mask_block=5)
    assert np.all(o[5:10] == 0.0) and np.all(np.isneginf(lse[5:10]))
    assert np.all(np.isfinite(lse[:5])) and np.all(np.isfinite(lse[10:]))


# ------------------------------------------------------------------ invariants
@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    N, d = 90, 16
    q, k, v = rand(N, d), rand(N, d), rand(N, d)
    scale = 0.25
    _, lse = oracle.forward(q, k, v, scale, causal)
    s = scale * q @ k.T
    if causal:
        s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    p = np.exp(s - lse[:, None])
    np.testing.assert_allclose(p.sum(axis=1), np.ones(N), rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_shift_of_keys(causal):
    N, d = 40, 8
    q, k, v = rand(N, d), rand(N, d), rand(N, d)
    c = rand(d)
    o1, l1 = oracle.forward(q, k, v, 0.4, causal)
    o2, l2 = oracle.forward(q, k + c, v, 0.4, causal)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + 0.4 * q @ c, rtol=0, atol=1e-12)


def test_permutation_equivariance():
    N, d = 33, 8
    q, k, v = rand(N, d), rand(N, d), rand(N, d)
    o, lse = oracle.forward(q, k, v, 0.35, False)
    pk = RNG.permutation(N)
    o2, l2 = oracle.forward(q, k[pk], v[pk], 0.35, False)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-12)
    pq = RNG.permutation(N)
    o3, l3 = oracle.forward(q[pq], k, v, 0.35, False)
    np.testing.assert_allclose(o3, o[pq], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l3, lse[pq], rtol=0, atol=1e-12)


def test_mask_identities():
    N, d, mb = 100, 8, 16
    nb = -(-N // mb)
    q, k, v = rand(2, N, d), rand(2, N, d), rand(2, N, d)
    od, ld = oracle.forward(q, k, v, 0.3, False)
    o1, l1 = oracle.forward(q, k, v, 0.3, False, block_mask=np.ones((nb, nb), np.uint8), mask_block=mb)
    np.testing.assert_array_equal(o1, od)
    np.testing.assert_array_equal(l1, ld)
    oc, lc = oracle.forward(q, k, v, 0.3, True)
    tri = np.tril(np.ones((nb, nb), np.uint8))
    o2, l2 = oracle.forward(q, k, v, 0.3, True, block_mask=tri, mask_block=mb)
    np.testing.assert_allclose(o2, oc, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, lc, rtol=0, atol=1e-14)


# -------------------------------------------------------------------- backward
def _loss(q, k, v, do, scale, causal, mask=None, mb=1):
    o, _ = oracle.forward(q, k, v, scale, causal, block_mask=mask, mask_block=mb)
    return float(np.sum(do * o))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(4, 3), (9, 4)])
def test_backward_matches_central_finite_differences(N, d, causal):
    q, k, v, do = rand(N, d), rand(N, d), rand(N, d), rand(N, d)
    scale = 0.6
    dq, dk, dv, _, _ = oracle.backward(q, k, v, do, scale, causal)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do, scale, causal)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], do, scale, causal)) / (2 * h)
        err = np.abs(num - g).max() / max(1.0, np.abs(g).max())
        assert err < 1e-6, (name, err)


def test_masked_backward_matches_finite_differences():
    N, d = 8, 3
    q, k, v, do = rand(N, d), rand(N, d), rand(N, d), rand(N, d)
    mask = (RNG.random((N, N)) < 0.6).astype(np.uint8)
    mask[3, :] = 0
    dq, dk, dv, _, _ = oracle.backward(q, k, v, do, 0.8, False, block_mask=mask, mask_block=1)
    h = 1e-6
    for which, g in ((0, dq), (1, dk), (2, dv)):
        for idx in np.ndindex(N, d):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            lp = _loss(*args, do, 0.8, False, mask, 1)
            args[which][idx] -= 2 * h
            lm = _loss(*args, do, 0.8, False, mask, 1)
            assert abs((lp - lm) / (2 * h) - g[idx]) < 1e-6
    assert np.all(dq[3] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd_fp64(causal):
    B, N, d = 3, 70, 16
    scale = 1 / math.sqrt(d)
    q, k, v, do = rand(B, N, d), rand(B, N, d), rand(B, N, d), rand(B, N, d)
    dq, dk, dv, lse, delta = oracle.backward(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    s = scale * tq @ tk.transpose(-1, -2)
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), -math.inf)
    o = torch.softmax(s, dim=-1) @ tv
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(s.detach(), -1).numpy(), rtol=0, atol=1e-12)
    # D_i = sum_j P_ij dP_ij equals dO_i . O_i
    np.testing.assert_allclose(delta, np.sum(do * o.detach().numpy(), -1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_identities(causal):
    N, d = 64, 8
    q, k, v, do = rand(N, d), rand(N, d), rand(N, d), rand(N, d)
    dq, dk, dv, _, delta = oracle.backward(q, k, v, do, 0.35, causal)
    o, _ = oracle.forward(q, k, v, 0.35, causal)
    np.testing.assert_allclose(dv.sum(0), do.sum(0), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk.sum(0), np.zeros(d), rtol=0, atol=1e-12)
    np.testing.assert_allclose(delta, np.sum(do * o, -1), rtol=0, atol=1e-12)
    if causal:
        assert np.all(np.abs(dq[0]) < 1e-15)


def test_backward_all_ones_mask_equals_dense():
    N, d, mb = 45, 4, 8
    nb = -(-N // mb)
    q, k, v, do = rand(N, d), rand(N, d), rand(N, d), rand(N, d)
    a = oracle.backward(q, k, v, do, 0.5, True)
    b = oracle.backward(q, k, v, do, 0.5, True, block_mask=np.ones((nb, nb), np.uint8), mask_block=mb)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_empty_and_argument_errors():
    o, lse = oracle.forward(np.zeros((0, 4)), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert o.shape == (0, 4) and lse.shape == (0,)
    with pytest.raises(ValueError):
        oracle.forward(np.zeros((3, 4)), np.zeros((3, 5)), np.zeros((3, 4)), 1.0)
    with pytest.raises(ValueError):
        oracle.forward(np.zeros((9, 4)), np.zeros((9, 4)), np.zeros((9, 4)), 1.0,
                       block_mask=np.ones((2, 2), np.uint8), mask_block=4)


# ------------------------------------------------- grouped K/V heads (MQA/GQA)
@pytest.mark.parametrize("H,Hkv", [(4, 2), (3, 1), (2, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_forward_matches_decimal_brute_force(H, Hkv, causal):
    """Query head h of a batch reads K/V head h // (H / Hkv) of that batch."""
    B, N, d = 2, 4, 2
    q, k, v = rand(B, H, N, d), rand(B, Hkv, N, d), rand(B, Hkv, N, d)
    o, lse = oracle.forward_gqa(q, k, v, 0.9, causal)
    assert o.shape == (B, H, N, d) and lse.shape == (B, H, N)
    vis = (lambda i, j: j <= i) if causal else (lambda i, j: True)
    for b in range(B):
        for h in range(H):
            kv = h // (H // Hkv)
            ob, lb = brute_decimal(q[b, h], k[b, kv], v[b, kv], 0.9, vis)
            np.testing.assert_allclose(o[b, h], ob, rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[b, h], lb, rtol=0, atol=1e-13)


@pytest.mark.parametrize("H,Hkv", [(4, 2), (3, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_backward_matches_finite_differences(H, Hkv, causal):
    """dK, dV of a shared head: derivative of L = sum(dO * O) over every query head."""
    B, N, d, scale = 1, 5, 2, 0.7
    q, k, v, do = rand(B, H, N, d), rand(B, Hkv, N, d), rand(B, Hkv, N, d), rand(B, H, N, d)
    dq, dk, dv, _, _ = oracle.backward_gqa(q, k, v, do, scale, causal)
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape

    def loss(q_, k_, v_):
        return float(np.sum(do * oracle.forward_gqa(q_, k_, v_, scale, causal)[0]))

    h = 1e-6
    for which, g in ((0, dq), (1, dk), (2, dv)):
        for idx in np.ndindex(*g.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            lp = loss(*args)
            args[which][idx] -= 2 * h
            lm = loss(*args)
            assert abs((lp - lm) / (2 * h) - g[idx]) < 1e-6, (which, idx)


def test_gqa_backward_matches_torch_autograd_fp64():
    B, H, Hkv, N, d = 2, 6, 2, 40, 8
    scale = 1 / math.sqrt(d)
    q, k, v, do = rand(B, H, N, d), rand(B, Hkv, N, d), rand(B, Hkv, N, d), rand(B, H, N, d)
    dq, dk, dv, _, _ = oracle.backward_gqa(q, k, v, do, scale, True)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    kk = tk.repeat_interleave(H // Hkv, dim=1)
    vv = tv.repeat_interleave(H // Hkv, dim=1)
    o = F.scaled_dot_product_attention(tq, kk, vv, is_causal=True, scale=scale)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


def test_mqa_with_identical_query_heads():
    """Hkv = 1 and every query head equal: equal outputs, and dK, dV are H times one head's."""
    H, N, d = 3, 12, 4
    q1, k, v, do1 = rand(1, 1, N, d), rand(1, 1, N, d), rand(1, 1, N, d), rand(1, 1, N, d)
    q, do = np.repeat(q1, H, axis=1), np.repeat(do1, H, axis=1)
    o, lse = oracle.forward_gqa(q, k, v, 0.5, True)
    o1, lse1 = oracle.forward(q1, k, v, 0.5, True)
    for h in range(H):
        np.testing.assert_array_equal(o[:, h], o1[:, 0])
        np.testing.assert_array_equal(lse[:, h], lse1[:, 0])
    _, dk, dv, _, _ = oracle.backward_gqa(q, k, v, do, 0.5, True)
    _, dk1, dv1, _, _ = oracle.backward(q1, k, v, do1, 0.5, True)
    np.testing.assert_allclose(dk, H * dk1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, H * dv1, rtol=0, atol=1e-13)


def test_gqa_shape_errors():
    with pytest.raises(ValueError):
        oracle.forward_gqa(rand(1, 4, 3, 2), rand(1, 3, 3, 2), rand(1, 3, 3, 2), 1.0)
    with pytest.raises(ValueError):
        oracle.forward_gqa(rand(1, 4, 3, 2), rand(1, 2, 5, 2), rand(1, 2, 5, 2), 1.0)
