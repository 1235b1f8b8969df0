"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a
closed form printed on the pages, a worked example, a library routine
that the definition reduces to in a special case, an invariance of
softmax attention, or finite differences.  A plausible slip anywhere in
the oracle (a wrong comparison in the mask, a dropped scale, natural vs
base-2 logarithm, a transposed operand) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import (WORKLOADS, cu_seqlens, make_fp8_inputs, make_fp8_integer_score_inputs, make_inputs,
                       make_varlen_inputs)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, mask=None, is_causal=False, scale=None):
    """torch's scaled_dot_product_attention on one head in float64."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    o = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, is_causal=is_causal, scale=scale)
    return o[0, 0].numpy()


def _blocks(n, b):
    """Consecutive runs of b positions from the start of a half."""
    return [list(range(s, min(s + b, n))) for s in range(0, n, b)]


# --------------------------------------------------------------------------
# Mask: cardinality (closed form on page 1) and brute force on tiny sizes
# --------------------------------------------------------------------------

def test_visible_pairs_closed_form_all_workloads():
    """Fast Diffusion Attention, 'The right yardstick': n^2 + n*b pairs."""
    with open(os.path.join(GOLDEN, "visible_pairs.json")) as f:
        gold = json.load(f)["workloads"]
    seen = set()
    for name, w in WORKLOADS.items():
        key = (w.n, w.b)
        if key in seen:
            continue
        seen.add(key)
        total = 0
        for r0 in range(0, 2 * w.n, 2048):  # row chunks keep memory small
            total += int(oracle.block_diffusion_mask(w.n, w.b, np.arange(r0, min(r0 + 2048, 2 * w.n))).sum())
        assert total == gold[name]["pairs"], name
        if w.n % w.b == 0:
            assert total == w.n * w.n + w.n * w.b


def _prose_mask(n, b):
    """The mask written from the prose of 'Block diffusion in one picture',
    one explicit list of blocks at a time."""
    blocks = _blocks(n, b)
    want = np.zeros((2 * n, 2 * n), dtype=bool)
    for i, blk in enumerate(blocks):
        for r in blk:
            # noisy row: its own noisy block, both directions
            for c in blk:
                want[r, c] = True
            # noisy row: every clean block strictly before block i
            for earlier in blocks[:i]:
                for c in earlier:
                    want[r, n + c] = True
            # clean row: its own clean block and the earlier clean blocks
            for earlier in blocks[: i + 1]:
                for c in earlier:
                    want[n + r, n + c] = True
    return want


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 11])
def test_mask_matches_block_description_bruteforce(n):
    """Tiny sizes: the mask equals the prose of 'Block diffusion in one picture'
    evaluated on explicit lists of blocks."""
    for b in range(1, n + 3):
        M = oracle.block_diffusion_mask(n, b)
        blocks = _blocks(n, b)
        want = _prose_mask(n, b)
        assert np.array_equal(M, want), (n, b)
        # staircase equivalence ('The right yardstick'): noisy row block i sees
        # i blocks in total, like a causal row over blocks
        for i, blk in enumerate(blocks):
            r = blk[0]
            assert M[r, n:].sum() == sum(len(x) for x in blocks[:i])


def test_causal_mask_is_lower_triangular():
    for S in (1, 2, 7, 33):
        assert np.array_equal(oracle.causal_mask(S), np.tril(np.ones((S, S), dtype=bool)))


# --------------------------------------------------------------------------
# Forward: sub-problems that reduce to textbook attention
# --------------------------------------------------------------------------

CASES = [(16, 4, 8), (13, 3, 8), (20, 1, 4), (9, 9, 6), (12, 20, 5), (32, 8, 16)]


@pytest.mark.parametrize("n,b,D", CASES)
def test_clean_half_is_block_causal_attention(n, b, D):
    """The clean half sees only clean keys, block-causally ('Block diffusion in
    one picture'); compare with SDPA over the clean tokens alone and an
    independently built block-causal mask (Kronecker product)."""
    q, k, v = (_rand((2 * n, D), s) for s in (1, 2, 3))
    scale = 1 / math.sqrt(D)
    O, lse = oracle.diffusion_forward(q, k, v, b, scale)
    nb = -(-n // b)
    bc = np.kron(np.tril(np.ones((nb, nb))), np.ones((b, b)))[:n, :n].astype(bool)
    want = _sdpa(q[n:], k[n:], v[n:], mask=bc, scale=scale)
    np.testing.assert_allclose(O[n:], want, rtol=0, atol=1e-12)
    # log-sum-exp of the clean rows, natural log, including the scale
    S = scale * q[n:] @ k[n:].T
    S = np.where(bc, S, -np.inf)
    want_lse = np.log(np.exp(S).sum(axis=1))
    np.testing.assert_allclose(lse[n:], want_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,b,D", CASES)
def test_noisy_block_attends_to_earlier_clean_plus_itself(n, b, D):
    """Noisy block i = plain (unmasked) attention over
    concat(clean blocks < i, noisy block i)."""
    q, k, v = (_rand((2 * n, D), s) for s in (4, 5, 6))
    scale = 0.37
    O, lse = oracle.diffusion_forward(q, k, v, b, scale)
    for i, blk in enumerate(_blocks(n, b)):
        ctx = [n + c for c in range(0, blk[0])] + blk
        want = _sdpa(q[blk], k[ctx], v[ctx], scale=scale)
        np.testing.assert_allclose(O[blk], want, rtol=0, atol=1e-12)
        S = scale * q[blk] @ k[ctx].T
        np.testing.assert_allclose(lse[blk], np.log(np.exp(S).sum(axis=1)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,D", [(7, 4), (64, 16), (100, 8)])
def test_block_size_one_clean_half_is_causal(n, D):
    """With block size 1 the clean half is causal attention on the clean tokens
    ('Accuracy' on page 1); torch's is_causal path in float64."""
    q, k, v = (_rand((2 * n, D), s) for s in (7, 8, 9))
    scale = 1 / math.sqrt(D)
    O, _ = oracle.diffusion_forward(q, k, v, 1, scale)
    want = _sdpa(q[n:], k[n:], v[n:], is_causal=True, scale=scale)
    np.testing.assert_allclose(O[n:], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,b", [(5, 5), (6, 9), (10, 64)])
def test_block_longer_than_half_is_bidirectional_per_half(n, b):
    """b >= n: one block per half.  The noisy half has no earlier clean block,
    so each half is full bidirectional attention over itself."""
    D = 4
    q, k, v = (_rand((2 * n, D), s) for s in (10, 11, 12))
    O, _ = oracle.diffusion_forward(q, k, v, b, 0.5)
    np.testing.assert_allclose(O[:n], _sdpa(q[:n], k[:n], v[:n], scale=0.5), atol=1e-12)
    np.testing.assert_allclose(O[n:], _sdpa(q[n:], k[n:], v[n:], scale=0.5), atol=1e-12)


@pytest.mark.parametrize("n,b", [(12, 4), (13, 5), (8, 1), (6, 8)])
def test_zero_queries_closed_form(n, b):
    """q = 0: every visible score is 0, so each row averages its visible values
    and LSE_i = ln(number of visible keys)."""
    D = 6
    q = np.zeros((2 * n, D))
    k, v = _rand((2 * n, D), 13), _rand((2 * n, D), 14)
    O, lse = oracle.diffusion_forward(q, k, v, b, 1.0)
    for i, blk in enumerate(_blocks(n, b)):
        noisy_ctx = [n + c for c in range(blk[0])] + blk
        clean_ctx = [n + c for c in range(blk[-1] + 1)]
        for r in blk:
            np.testing.assert_allclose(O[r], v[noisy_ctx].mean(axis=0), atol=1e-13)
            assert abs(lse[r] - math.log(len(noisy_ctx))) < 1e-13
            np.testing.assert_allclose(O[n + r], v[clean_ctx].mean(axis=0), atol=1e-13)
            assert abs(lse[n + r] - math.log(len(clean_ctx))) < 1e-13


def test_shift_invariances():
    """Adding c to every key leaves O unchanged and shifts LSE_i by
    scale*q_i.c; adding c to every value shifts O by c."""
    n, b, D, scale = 10, 3, 5, 0.7
    q, k, v = (_rand((2 * n, D), s) for s in (15, 16, 17))
    c = _rand((D,), 18)
    O, lse = oracle.diffusion_forward(q, k, v, b, scale)
    O2, lse2 = oracle.diffusion_forward(q, k + c, v, b, scale)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + scale * q @ c, atol=1e-12)
    O3, lse3 = oracle.diffusion_forward(q, k, v + c, b, scale)
    np.testing.assert_allclose(O3, O + c, atol=1e-12)
    np.testing.assert_allclose(lse3, lse, atol=1e-13)


def test_worked_example_of_online_softmax():
    """FlashAttention page, section 4.3: the row [1, 2 | 0, 3] in two blocks.
    (a) the oracle's softmax of the four scores equals the page's final
    weights; (b) the page's block-by-block recurrence (running max m,
    rescale e^(m - m'), new block weights) reproduces the same weights."""
    with open(os.path.join(GOLDEN, "online_softmax_worked_example.json")) as f:
        g = json.load(f)
    w = np.exp(np.array(g["final_weight_exponents"]))
    want = w / w.sum()
    # (a) one noisy row (n = 4, b = 4: the row sees the 4 noisy keys and
    # nothing else); q . k_j = score_j with scale 1; one-hot values read P.
    n, D = 4, 8
    q = np.zeros((2 * n, D))
    k = np.zeros((2 * n, D))
    q[0, 0] = 1.0
    k[:n, 0] = g["scores"]
    v = np.eye(2 * n, D)
    O, lse = oracle.diffusion_forward(q, k, v, 4, 1.0)
    np.testing.assert_allclose(O[0, :n], want, atol=1e-15)
    assert abs(lse[0] - (max(g["scores"]) + math.log(w.sum()))) < 1e-14
    # (b) the recurrence as the page states it, with its printed intermediates
    b1, b2 = (np.array(x) for x in g["blocks"])
    m = b1.max()
    assert m == g["block1_max"]
    np.testing.assert_allclose(b1 - m, g["block1_weight_exponents"])
    m2 = max(m, b2.max())
    assert m2 == g["block2_max"] and m - m2 == g["rescale_exponent"]
    np.testing.assert_allclose(b1 - m + (m - m2), g["block1_rescaled_exponents"])
    np.testing.assert_allclose(b2 - m2, g["block2_weight_exponents"])
    ell = np.exp(b1 - m).sum() * math.exp(m - m2) + np.exp(b2 - m2).sum()
    np.testing.assert_allclose(np.concatenate([np.exp(b1 - m2), np.exp(b2 - m2)]) / ell, want, atol=1e-15)


# --------------------------------------------------------------------------
# Backward: finite differences and gradient identities
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,b", [(4, 1), (5, 2), (6, 3), (3, 4), (8, 2)])
def test_gradients_match_central_differences(n, b):
    """Central differences of L = sum(dout * O) in float64; rel. error <= 1e-6."""
    D, scale, eps = 4, 0.8, 1e-6
    q, k, v, do = (_rand((2 * n, D), s) for s in (19, 20, 21, 22))
    dq, dk, dv = oracle.diffusion_backward(q, k, v, do, b, scale)

    def loss(qq, kk, vv):
        return float((oracle.diffusion_forward(qq, kk, vv, b, scale)[0] * do).sum())

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        err = np.abs(num - grad).max() / np.abs(grad).max()
        assert err <= 1e-6, (which, err)


def test_gradient_identities():
    """Shift invariance gives sum_j dK_j = 0 (every row of dS sums to zero) and
    sum_j dV_j = sum_i dO_i (every row of P sums to one); the score scale
    gives sum_i q_i.dQ_i = sum_j k_j.dK_j."""
    n, b, D, scale = 14, 4, 6, 0.45
    q, k, v, do = (_rand((2 * n, D), s) for s in (23, 24, 25, 26))
    dq, dk, dv = oracle.diffusion_backward(q, k, v, do, b, scale)
    np.testing.assert_allclose(dk.sum(axis=0), 0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
    assert abs((q * dq).sum() - (k * dk).sum()) < 1e-11
    # delta computed two ways: sum_j P_ij dP_ij == dO_i . O_i
    O, _ = oracle.diffusion_forward(q, k, v, b, scale)
    M = oracle.block_diffusion_mask(n, b)
    S = np.where(M, scale * q @ k.T, -np.inf)
    P = np.exp(S - S.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    np.testing.assert_allclose((P * (do @ v.T)).sum(1), (do * O).sum(1), atol=1e-12)


# --------------------------------------------------------------------------
# The causal yardstick and the sampled (row / column) forms
# --------------------------------------------------------------------------

def test_causal_oracle_matches_sdpa_and_finite_differences():
    S, D = 11, 4
    q, k, v, do = (_rand((S, D), s) for s in (27, 28, 29, 30))
    O, lse = oracle.causal_forward(q, k, v, 0.6)
    np.testing.assert_allclose(O, _sdpa(q, k, v, is_causal=True, scale=0.6), atol=1e-12)
    tq = torch.from_numpy(q).requires_grad_()
    tk = torch.from_numpy(k).requires_grad_()
    tv = torch.from_numpy(v).requires_grad_()
    o = F.scaled_dot_product_attention(tq[None], tk[None], tv[None], is_causal=True, scale=0.6)[0]
    (o * torch.from_numpy(do)).sum().backward()
    dq, dk, dv = oracle.causal_backward(q, k, v, do, 0.6)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("n,b", [(24, 5), (16, 16), (20, 1)])
def test_sampled_forms_equal_full(n, b):
    D, scale = 8, 0.3
    q, k, v, do = (_rand((2 * n, D), s) for s in (31, 32, 33, 34))
    O, lse = oracle.diffusion_forward(q, k, v, b, scale)
    dq, dk, dv = oracle.diffusion_backward(q, k, v, do, b, scale)
    rows = [0, 3, n - 1, n, n + 7, 2 * n - 1]
    Or, lr = oracle.diffusion_forward_rows(q, k, v, b, scale, rows)
    np.testing.assert_allclose(Or, O[rows], atol=1e-13)
    np.testing.assert_allclose(lr, lse[rows], atol=1e-13)
    np.testing.assert_allclose(oracle.diffusion_grad_q_rows(q, k, v, do, b, scale, rows), dq[rows], atol=1e-12)
    cols = [0, 1, n - 2, n, n + 3, 2 * n - 1]
    dkc, dvc = oracle.diffusion_grad_kv_cols(q, k, v, do, O, lse, b, scale, cols)
    np.testing.assert_allclose(dkc, dk[cols], atol=1e-12)
    np.testing.assert_allclose(dvc, dv[cols], atol=1e-12)


def test_batched_layout_against_sdpa():
    """(batch, 2n, heads, dim) handling: at block size 1 the clean half of every
    (sample, head) equals causal SDPA run in torch's (B, H, S, D) layout."""
    B, n, H, D = 2, 9, 3, 4
    q, k, v, _ = make_inputs(B, n, H, D, seed=7)
    O, lse = oracle.batched(oracle.diffusion_forward, oracle.to_f64(q), oracle.to_f64(k),
                            oracle.to_f64(v), b=1, scale=0.5)
    assert O.shape == (B, 2 * n, H, D) and lse.shape == (B, H, 2 * n)
    t = lambda x: x.to(torch.float64)[:, n:].permute(0, 2, 1, 3)
    want = F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True, scale=0.5)
    np.testing.assert_allclose(O[:, n:], want.permute(0, 2, 1, 3).numpy(), atol=1e-12)


def test_inputs_are_seeded_bf16():
    a = make_inputs(1, 8, 2, 4, seed=3)
    b = make_inputs(1, 8, 2, 4, seed=3)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.shape == (1, 16, 2, 4)
        assert torch.equal(x, y)
    c = make_inputs(1, 8, 2, 4, seed=4)
    assert not torch.equal(a[0], c[0])


# --------------------------------------------------------------------------
# Grouped-query attention (query heads sharing key/value heads)
# --------------------------------------------------------------------------

GQA_SHAPES = [(2, 7, 6, 2, 3), (1, 9, 4, 1, 4), (2, 5, 4, 4, 2)]  # B, n, H, H_kv, b


@pytest.mark.parametrize("B,n,H,H_kv,b", GQA_SHAPES)
def test_grouped_oracle_matches_sdpa_gqa(B, n, H, H_kv, b):
    """torch's scaled_dot_product_attention with enable_gqa (float64, CPU)
    under the prose mask: the grouped forward, and through autograd the
    grouped backward, whose dK / dV sum over each group's query heads."""
    D, scale = 5, 0.55
    q, k, v, do = make_inputs(B, n, H, D, seed=40 + H_kv, H_kv=H_kv)
    f = oracle.to_f64
    O, _ = oracle.grouped_forward(oracle.diffusion_forward, f(q), f(k), f(v), b=b, scale=scale)
    dq, dk, dv = oracle.grouped_backward(oracle.diffusion_backward, f(q), f(k), f(v), f(do),
                                         b=b, scale=scale)
    t = lambda x: x.to(torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_()
    tq, tk, tv = t(q), t(k), t(v)
    mask = torch.from_numpy(_prose_mask(n, b))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale, enable_gqa=True)
    (o * do.to(torch.float64).permute(0, 2, 1, 3)).sum().backward()
    back = lambda x: x.permute(0, 2, 1, 3).detach().numpy()
    np.testing.assert_allclose(O, back(o), atol=1e-12)
    np.testing.assert_allclose(dq, back(tq.grad), atol=1e-11)
    np.testing.assert_allclose(dk, back(tk.grad), atol=1e-11)
    np.testing.assert_allclose(dv, back(tv.grad), atol=1e-11)


def test_grouped_head_map_closed_forms():
    """q = 0 makes each row the mean of its visible values of the key/value
    head its group reads; shifting the keys of head j by c_j shifts the LSE
    of query head h by scale * q_h . c_{h // (H / H_kv)}.  Distinct values
    and shifts per key/value head fix the map for O and for LSE."""
    B, n, H, H_kv, b, D, scale = 1, 6, 6, 3, 2, 4, 0.9
    G = H // H_kv
    v = _rand((B, 2 * n, H_kv, D), 50) + 10.0 * np.arange(H_kv)[None, None, :, None]
    k = _rand((B, 2 * n, H_kv, D), 51)
    O, lse = oracle.grouped_forward(oracle.diffusion_forward, np.zeros((B, 2 * n, H, D)), k, v,
                                    b=b, scale=scale)
    M = _prose_mask(n, b)
    for h in range(H):
        for r in range(2 * n):
            np.testing.assert_allclose(O[0, r, h], v[0, M[r], h // G].mean(axis=0), atol=1e-12)
            assert abs(lse[0, h, r] - math.log(M[r].sum())) < 1e-12
    q = _rand((B, 2 * n, H, D), 52)
    c = _rand((H_kv, D), 53)
    _, l1 = oracle.grouped_forward(oracle.diffusion_forward, q, k, v, b=b, scale=scale)
    _, l2 = oracle.grouped_forward(oracle.diffusion_forward, q, k + c[None, None], v, b=b, scale=scale)
    for h in range(H):
        np.testing.assert_allclose(l2[0, h] - l1[0, h], scale * q[0, :, h] @ c[h // G], atol=1e-12)
    with pytest.raises(ValueError):
        oracle.kv_head_of(0, 6, 4)


def test_grouped_gradients_match_central_differences():
    """Central differences of L = sum(dout * O) over the grouped forward."""
    B, n, H, H_kv, b, D, scale, eps = 1, 3, 4, 2, 2, 3, 0.7, 1e-6
    q, do = _rand((B, 2 * n, H, D), 54), _rand((B, 2 * n, H, D), 55)
    k, v = _rand((B, 2 * n, H_kv, D), 56), _rand((B, 2 * n, H_kv, D), 57)
    grads = oracle.grouped_backward(oracle.diffusion_backward, q, k, v, do, b=b, scale=scale)

    def loss(qq, kk, vv):
        O, _ = oracle.grouped_forward(oracle.diffusion_forward, qq, kk, vv, b=b, scale=scale)
        return float((O * do).sum())

    for which, grad in enumerate(grads):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        err = np.abs(num - grad).max() / np.abs(grad).max()
        assert err <= 1e-6, (which, err)


def test_grouped_sampled_kv_columns_equal_full():
    B, n, H, H_kv, b, D, scale = 1, 10, 4, 2, 3, 6, 0.4
    G = H // H_kv
    q, do = _rand((B, 2 * n, H, D), 58), _rand((B, 2 * n, H, D), 59)
    k, v = _rand((B, 2 * n, H_kv, D), 60), _rand((B, 2 * n, H_kv, D), 61)
    O, L = oracle.grouped_forward(oracle.diffusion_forward, q, k, v, b=b, scale=scale)
    _, dk, dv = oracle.grouped_backward(oracle.diffusion_backward, q, k, v, do, b=b, scale=scale)
    cols = [0, 2, n - 1, n, 2 * n - 1]
    for j in range(H_kv):
        hs = range(j * G, (j + 1) * G)
        dkc, dvc = oracle.grouped_grad_kv_cols([q[0, :, h] for h in hs], k[0, :, j], v[0, :, j],
                                               [do[0, :, h] for h in hs], [O[0, :, h] for h in hs],
                                               [L[0, h] for h in hs], b, scale, cols)
        np.testing.assert_allclose(dkc, dk[0, cols, j], atol=1e-12)
        np.testing.assert_allclose(dvc, dv[0, cols, j], atol=1e-12)


def test_grouped_inputs_keep_the_mha_draws():
    """H_kv = H draws the same bits as the plain call; k and v take H_kv heads."""
    a = make_inputs(1, 8, 4, 4, seed=3)
    b = make_inputs(1, 8, 4, 4, seed=3, H_kv=4)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    q, k, v, do = make_inputs(1, 8, 4, 4, seed=3, H_kv=2)
    assert q.shape == do.shape == (1, 16, 4, 4) and k.shape == v.shape == (1, 16, 2, 4)


# --------------------------------------------------------------------------
# Variable-length (packed) batches
# --------------------------------------------------------------------------

@pytest.mark.parametrize("H,H_kv", [(3, 3), (4, 2)])
def test_varlen_with_equal_lengths_is_the_batched_oracle(H, H_kv):
    """Packing B samples of one length back to back is the (B, 2n, H, D)
    layout flattened: the packed oracle must reproduce the batched one."""
    B, n, D, b, scale = 3, 9, 4, 2, 0.6
    q, k, v, do = (oracle.to_f64(x) for x in make_inputs(B, n, H, D, seed=70 + H_kv, H_kv=H_kv))
    cu = cu_seqlens([n] * B)
    flat = lambda x: x.reshape(B * 2 * n, *x.shape[2:])
    O, L = oracle.varlen_forward(oracle.diffusion_forward, flat(q), flat(k), flat(v), cu, b=b, scale=scale)
    g = oracle.varlen_backward(oracle.diffusion_backward, flat(q), flat(k), flat(v), flat(do), cu,
                               b=b, scale=scale)
    Ob, Lb = oracle.grouped_forward(oracle.diffusion_forward, q, k, v, b=b, scale=scale)
    gb = oracle.grouped_backward(oracle.diffusion_backward, q, k, v, do, b=b, scale=scale)
    np.testing.assert_allclose(O, flat(Ob), atol=1e-13)
    np.testing.assert_allclose(L, Lb.transpose(1, 0, 2).reshape(H, B * 2 * n), atol=1e-13)
    for x, y in zip(g, gb):
        np.testing.assert_allclose(x, flat(y), atol=1e-12)


def test_varlen_each_sample_uses_its_own_length():
    """q = 0 with samples of lengths 5, 0, 1, 8, 3: every row averages the
    visible values of its own sample, LSE = ln(count) from that sample's
    own mask (an empty sample has no rows)."""
    ns, b, D = [5, 0, 1, 8, 3], 2, 3
    cu = cu_seqlens(ns)
    total = cu[-1]
    v = _rand((total, 2, D), 71)
    k = _rand((total, 2, D), 72)
    O, L = oracle.varlen_forward(oracle.diffusion_forward, np.zeros((total, 2, D)), k, v, cu, b=b, scale=1.0)
    for bi, nb in enumerate(ns):
        if nb == 0:
            continue
        M = _prose_mask(nb, b)
        s0 = cu[bi]
        for r in range(2 * nb):
            for h in range(2):
                np.testing.assert_allclose(O[s0 + r, h], v[s0:s0 + 2 * nb, h][M[r]].mean(axis=0), atol=1e-12)
                assert abs(L[h, s0 + r] - math.log(M[r].sum())) < 1e-12
    assert not np.isnan(O).any()


def test_varlen_samples_do_not_interact():
    """Changing one sample's keys and values leaves every other sample's
    outputs and gradients unchanged."""
    ns, b, D, scale = [4, 6, 0, 3], 3, 4, 0.8
    cu = cu_seqlens(ns)
    total = cu[-1]
    q, k, v, do = (_rand((total, 2, D), s) for s in (73, 74, 75, 76))
    k2, v2 = k.copy(), v.copy()
    k2[cu[1]:cu[2]] += 1.5
    v2[cu[1]:cu[2]] -= 2.0
    O, _ = oracle.varlen_forward(oracle.diffusion_forward, q, k, v, cu, b=b, scale=scale)
    O2, _ = oracle.varlen_forward(oracle.diffusion_forward, q, k2, v2, cu, b=b, scale=scale)
    g = oracle.varlen_backward(oracle.diffusion_backward, q, k, v, do, cu, b=b, scale=scale)
    g2 = oracle.varlen_backward(oracle.diffusion_backward, q, k2, v2, do, cu, b=b, scale=scale)
    other = np.r_[cu[0]:cu[1], cu[3]:cu[4]]
    np.testing.assert_array_equal(O[other], O2[other])
    for x, y in zip(g, g2):
        np.testing.assert_array_equal(x[other], y[other])
    assert not np.allclose(O[cu[1]:cu[2]], O2[cu[1]:cu[2]])


def test_varlen_inputs_are_seeded_and_packed():
    ns = [3, 0, 5]
    q, k, v, do, cu = make_varlen_inputs(ns, 4, 8, seed=9, H_kv=2)
    assert cu == [0, 6, 6, 16]
    assert q.shape == do.shape == (16, 4, 8) and k.shape == v.shape == (16, 2, 8)
    q2, *_ = make_varlen_inputs(ns, 4, 8, seed=9, H_kv=2)
    assert torch.equal(q, q2)
    assert cu_seqlens(ns, causal=True) == [0, 3, 3, 8]


@pytest.mark.parametrize("n,b", [(1000, 64), (130, 7), (64, 64), (16383, 64)])
def test_last_keys_are_seen_only_by_the_last_block(n, b):
    """When the last two keys of each half lie in its last block, they are
    seen by the rows of that block (in the same half) and no others; the
    full-size GPU test relies on this to need only those rows' statistics."""
    assert (n - 1) // b == (n - 2) // b
    if n > 2048:  # the two row blocks and key columns involved, not the whole mask
        rows = np.r_[0:4 * b, n - 4 * b:n + 4 * b, 2 * n - 4 * b:2 * n]
        M = oracle.block_diffusion_mask(n, b, rows)
        last = (n - 1) // b * b
        cols = np.array([n - 2, n - 1, 2 * n - 2, 2 * n - 1])
        got = rows[M[:, cols].any(axis=1)]
        assert np.array_equal(got, np.r_[last:n, n + last:2 * n])
        return
    cols = np.array([n - 2, n - 1, 2 * n - 2, 2 * n - 1])
    last = (n - 1) // b * b
    seen = np.r_[last:n, n + last:2 * n]
    M = _prose_mask(n, b)
    assert np.array_equal(np.flatnonzero(M[:, cols].any(axis=1)), seen)


# --------------------------------------------------------------------------
# FP8 forward: the E4M3 decoder, dequantized attention, the error bound
# --------------------------------------------------------------------------

def test_e4m3_decoder_matches_the_format():
    """Every code against torch's float8_e4m3fn (the same OCP format) and the
    format's landmarks: 1.0, the largest finite value, the smallest normal
    and subnormal values, the NaN patterns, signed zero."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    np.testing.assert_array_equal(got[~np.isnan(got)], want[~np.isnan(want)])
    assert oracle.e4m3_value(0x38) == 1.0 and oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6 and oracle.e4m3_value(0x01) == 2.0 ** -9
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    assert oracle.e4m3_value(0x80) == 0.0 and oracle.e4m3_value(0xC0) == -2.0


def test_fp8_forward_is_attention_on_dequantized_values():
    """The FP8 reference is exact attention over descale * value, with the
    dequantization done here by torch's own cast."""
    n, D, b, scale = 11, 16, 3, 0.3
    q8, k8, v8, qd, kd, vd = make_fp8_inputs(1, n, 1, D, seed=80)
    u8 = lambda t: t[0, :, 0].view(torch.uint8).numpy()
    deq = lambda t, d: t[0, :, 0].to(torch.float64).numpy() * float(d[0, 0])
    O, L = oracle.fp8_forward(u8(q8), u8(k8), u8(v8), float(qd[0, 0]), float(kd[0, 0]), float(vd[0, 0]), b, scale)
    Or, Lr = oracle.diffusion_forward(deq(q8, qd), deq(k8, kd), deq(v8, vd), b, scale)
    np.testing.assert_array_equal(O, Or)
    np.testing.assert_array_equal(L, Lr)


def _emulated_fp8_pv(q, k, v, b, scale, lag):
    """O with P~ = exp2(s log2 e - m) rounded to E4M3 by torch, for a
    reference m = row maximum - lag (lag < 8, as the lazy rescale allows)."""
    n = q.shape[0] // 2
    M = oracle.block_diffusion_mask(n, b)
    s2 = np.where(M, scale * (q @ k.T) * math.log2(math.e), -np.inf)
    m = s2.max(axis=1, keepdims=True) - lag
    pt = np.exp2(s2 - m)
    p8 = torch.from_numpy(pt).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    return (p8 @ v) / pt.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("lag", [0.0, 3.7, 7.9])
def test_fp8_output_bound_covers_the_rounding_of_p(lag):
    """The bound holds for P~ actually rounded to E4M3 (by torch), whatever
    the lazy reference's distance below the row maximum; and it is not
    vacuous (the rounding error reaches a sizeable part of it)."""
    n, D, b, scale = 40, 32, 5, 0.8
    q8, k8, v8, qd, kd, vd = make_fp8_inputs(1, n, 1, D, seed=81)
    deq = lambda t, d: t[0, :, 0].to(torch.float64).numpy() * float(d[0, 0])
    q, k, v = deq(q8, qd), deq(k8, kd), deq(v8, vd)
    O, _ = oracle.diffusion_forward(q, k, v, b, scale)
    err = np.abs(_emulated_fp8_pv(q, k, v, b, scale, lag) - O)
    bound = oracle.fp8_output_bound(q, k, v, b, scale)
    assert np.all(err <= bound)
    assert err.max() > 0.05 * bound.max()


def test_fp8_integer_scores_make_p_exact():
    """With integer base-2 scores (two +-1 entries per row of q and k,
    scale = ln 2) every P~ is a power of two within E4M3's range, so the
    rounded P.V equals exact attention up to float64 rounding."""
    n, D, b = 24, 64, 4
    q8, k8, v8, qd, kd, vd = make_fp8_integer_score_inputs(1, n, 1, D, seed=82)
    deq = lambda t, d: t[0, :, 0].to(torch.float64).numpy() * float(d[0, 0])
    q, k, v = deq(q8, qd), deq(k8, kd), deq(v8, vd)
    scale = math.log(2.0)
    s = q @ k.T
    assert np.array_equal(s, np.round(s)) and np.abs(s).max() <= 2
    O, _ = oracle.diffusion_forward(q, k, v, b, scale)
    for lag in (0.0, 3.0):  # integer lags keep the powers of two
        np.testing.assert_allclose(_emulated_fp8_pv(q, k, v, b, scale, lag), O, atol=1e-12)


def test_fp8_output_bound_needs_its_subnormal_term():
    """A row whose output comes from probabilities below E4M3's smallest
    normal value (2^-6): one key at score 0 with value 0, the others at a
    base-2 score of -7.3 with value 1.  Their rounding error (up to 2^-10
    absolute, about 16% relative) exceeds the 2^-4 relative term alone; the
    bound's second term covers it."""
    n, b = 40, 40                  # row 0 sees exactly the 40 noisy keys
    scale = 1.0 / math.log2(math.e)
    q = np.zeros((2 * n, 2))
    k = np.zeros((2 * n, 2))
    v = np.zeros((2 * n, 2))
    q[:, 0] = 1.0
    k[1:n, 0] = -7.3
    v[1:n, 0] = 1.0
    O, _ = oracle.diffusion_forward(q, k, v, b, scale)
    err = np.abs(_emulated_fp8_pv(q, k, v, b, scale, 0.0) - O)[0, 0]
    bound = oracle.fp8_output_bound(q, k, v, b, scale, rows=[0])[0, 0]
    M = oracle.block_diffusion_mask(n, b, [0])
    s = np.where(M, scale * (q[[0]] @ k.T), -np.inf)
    P = np.exp(s - s.max())
    P /= P.sum()
    assert err <= bound
    assert err > 2.0 ** -4 * (P @ np.abs(v))[0, 0]


def test_fp8_output_bound_with_an_explicit_mask():
    """Passing the block-diffusion mask explicitly gives the default bound;
    the causal mask bounds the causal pass."""
    n, D, b, scale = 30, 8, 4, 0.5
    q, k, v = (_rand((2 * n, D), s) for s in (90, 91, 92))
    rows = [0, 5, n, 2 * n - 1]
    np.testing.assert_array_equal(
        oracle.fp8_output_bound(q, k, v, b, scale, rows),
        oracle.fp8_output_bound(q, k, v, b, scale, rows, mask=oracle.block_diffusion_mask(n, b, rows)))
    O, _ = oracle.causal_forward(q, k, v, scale)
    # P rounded as the kernel would, with the row maximum as reference
    s2 = np.where(oracle.causal_mask(2 * n), scale * (q @ k.T) * math.log2(math.e), -np.inf)
    pt = np.exp2(s2 - s2.max(axis=1, keepdims=True))
    p8 = torch.from_numpy(pt).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    err = np.abs((p8 @ v) / pt.sum(axis=1, keepdims=True) - O)
    assert np.all(err <= oracle.fp8_output_bound(q, k, v, 1, scale, mask=oracle.causal_mask(2 * n)))


# --------------------------------------------------------------------------
# Softcapping: scores s -> cap * tanh(s / cap)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,b", [(4, 1), (6, 3), (5, 2)])
def test_softcap_gradients_match_central_differences(n, b):
    D, scale, cap, eps = 4, 0.9, 1.5, 1e-6
    q, k, v, do = (3.0 * _rand((2 * n, D), s) for s in (100, 101, 102, 103))
    dq, dk, dv = oracle.diffusion_backward(q, k, v, do, b, scale, softcap=cap)

    def loss(qq, kk, vv):
        return float((oracle.diffusion_forward(qq, kk, vv, b, scale, softcap=cap)[0] * do).sum())

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        err = np.abs(num - grad).max() / np.abs(grad).max()
        assert err <= 1e-6, (which, err)


def test_softcap_limits_and_bounds():
    """A very large cap is no cap; the capped scores lie in (-cap, cap), so
    within a row no probability exceeds another by more than e^(2 cap),
    however large the raw scores; q = 0 still gives uniform rows."""
    n, b, D, scale = 12, 4, 6, 0.7
    q, k, v, do = (_rand((2 * n, D), s) for s in (104, 105, 106, 107))
    O, L = oracle.diffusion_forward(q, k, v, b, scale)
    Oc, Lc = oracle.diffusion_forward(q, k, v, b, scale, softcap=1e7)
    np.testing.assert_allclose(Oc, O, atol=1e-9)
    np.testing.assert_allclose(Lc, L, atol=1e-9)
    for x, y in zip(oracle.diffusion_backward(q, k, v, do, b, scale, softcap=1e7),
                    oracle.diffusion_backward(q, k, v, do, b, scale)):
        np.testing.assert_allclose(x, y, atol=1e-9)
    cap = 2.0
    big_q = 50.0 * q
    M = oracle.block_diffusion_mask(n, b)
    onehot = np.eye(2 * n)[:, :2 * n]
    P, _ = oracle.diffusion_forward(big_q, k, onehot, b, scale, softcap=cap)  # O = P when v = I
    for r in range(2 * n):
        pr = P[r][M[r]]
        assert pr.max() / pr.min() <= math.exp(2 * cap) * (1 + 1e-9)
    Oz, _ = oracle.diffusion_forward(np.zeros_like(q), k, v, b, scale, softcap=cap)
    Ou, _ = oracle.diffusion_forward(np.zeros_like(q), k, v, b, scale)
    np.testing.assert_allclose(Oz, Ou, atol=1e-13)


def test_softcap_two_key_row_by_hand():
    """A clean row of the first block with b = 2 sees exactly two keys; its
    output is their average weighted by exp(cap tanh(s / cap))."""
    n, b, D, scale, cap = 4, 2, 3, 0.5, 0.8
    q, k, v = (_rand((2 * n, D), s) for s in (108, 109, 110))
    O, L = oracle.diffusion_forward(q, k, v, b, scale, softcap=cap)
    r = n + 1                         # clean row 1 sees clean keys 0 and 1
    s = [scale * float(q[r] @ k[n + j]) for j in (0, 1)]
    w = [math.exp(cap * math.tanh(x / cap)) for x in s]
    np.testing.assert_allclose(O[r], (w[0] * v[n] + w[1] * v[n + 1]) / (w[0] + w[1]), atol=1e-14)
    assert abs(L[r] - math.log(w[0] + w[1])) < 1e-14


def test_softcap_sampled_forms_equal_full():
    n, b, D, scale, cap = 20, 3, 8, 0.4, 1.2
    q, k, v, do = (2.0 * _rand((2 * n, D), s) for s in (111, 112, 113, 114))
    O, lse = oracle.diffusion_forward(q, k, v, b, scale, softcap=cap)
    dq, dk, dv = oracle.diffusion_backward(q, k, v, do, b, scale, softcap=cap)
    rows = [0, 4, n - 1, n, n + 9, 2 * n - 1]
    Or, lr = oracle.diffusion_forward_rows(q, k, v, b, scale, rows, softcap=cap)
    np.testing.assert_allclose(Or, O[rows], atol=1e-13)
    np.testing.assert_allclose(oracle.diffusion_grad_q_rows(q, k, v, do, b, scale, rows, softcap=cap),
                               dq[rows], atol=1e-12)
    dkc, dvc = oracle.diffusion_grad_kv_cols(q, k, v, do, O, lse, b, scale, rows, softcap=cap)
    np.testing.assert_allclose(dkc, dk[rows], atol=1e-12)
    np.testing.assert_allclose(dvc, dv[rows], atol=1e-12)
