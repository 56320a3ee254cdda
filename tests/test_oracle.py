"""Pins for the CPU float64 oracle, independent of the oracle itself.

Each test fixes the oracle against something the pages or the mathematics
determine: brute-force loops with math.fsum on tiny inputs, closed forms,
invariants, hand-derived worked examples (tests/golden) and torch's CPU float64
attention as a library special case.  The mutation tests at the end plant a
plausible mistake in one oracle step at a time and check that these pins catch
it.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.exact as oa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
REL = 1e-12


def brute_force(q, k, v, scale, causal):
    """softmax(s q k^T) v with scalar loops and math.fsum (exactly rounded sums)."""
    B, H, L, d = q.shape
    dv = v.shape[-1]
    out = np.zeros((B, H, L, dv))
    for b in range(B):
        for h in range(H):
            for i in range(L):
                keys = range(i + 1) if causal else range(L)
                z = [scale * math.fsum(q[b, h, i, c] * k[b, h, j, c] for c in range(d)) for j in keys]
                m = max(z)
                e = [math.exp(x - m) for x in z]
                tot = math.fsum(e)
                for c in range(dv):
                    out[b, h, i, c] = math.fsum(e[jj] * v[b, h, j, c] for jj, j in enumerate(keys)) / tot
    return out


def rnd(shape, seed, s=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * s


def close(a, b, rel=REL):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    return float(np.max(np.abs(a - b))) <= rel * scale


TINY = [
    (1, 1, 1, 1, 0.5, False),
    (1, 1, 5, 3, 0.7, False),
    (2, 2, 7, 4, 0.5, True),
    (1, 3, 9, 8, 1 / math.sqrt(8), False),
    (2, 1, 9, 8, 1 / math.sqrt(8), True),
    (1, 1, 6, 2, 0.0, True),
    (1, 2, 8, 5, -1.3, False),
    (1, 1, 9, 8, 3.0, True),
]


@pytest.mark.parametrize("B,H,L,d,scale,causal", TINY)
def test_brute_force_tiny(B, H, L, d, scale, causal):
    q, k, v = rnd((B, H, L, d), 1), rnd((B, H, L, d), 2), rnd((B, H, L, d), 3)
    assert close(oracle.attention(q, k, v, scale, causal), brute_force(q, k, v, scale, causal))


def test_brute_force_value_dim_differs():
    q, k, v = rnd((1, 2, 6, 4), 4), rnd((1, 2, 6, 4), 5), rnd((1, 2, 6, 3), 6)
    for causal in (False, True):
        assert close(oracle.attention(q, k, v, 0.4, causal), brute_force(q, k, v, 0.4, causal))


@pytest.mark.parametrize("causal", [False, True])
def test_rows_match_full(causal):
    q, k, v = rnd((2, 2, 13, 8), 7), rnd((2, 2, 13, 8), 8), rnd((2, 2, 13, 8), 9)
    full = oracle.attention(q, k, v, 0.3, causal)
    rows = [(0, 0, 0), (1, 1, 12), (0, 1, 6), (1, 0, 3)]
    got = oracle.attention_rows(q, k, v, 0.3, causal, rows)
    want = np.stack([full[b, h, i] for b, h, i in rows])
    assert close(got, want, 1e-14)
    # and against the brute force, independently of attention()
    bf = brute_force(q, k, v, 0.3, causal)
    assert close(got, np.stack([bf[b, h, i] for b, h, i in rows]))


def test_golden_worked_examples():
    doc = json.load(open(GOLDEN))
    assert len(doc["cases"]) >= 5
    for case in doc["cases"]:
        got = oracle.attention(np.array(case["q"]), np.array(case["k"]), np.array(case["v"]),
                               case["scale"], case["causal"])
        assert close(got, np.array(case["expected"]), 1e-14), case["name"]


@pytest.mark.parametrize("causal", [False, True])
def test_torch_cpu_float64_sdpa(causal):
    q, k, v = rnd((2, 3, 33, 16), 10), rnd((2, 3, 33, 16), 11), rnd((2, 3, 33, 16), 12)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=0.37, is_causal=causal
    ).numpy()
    assert close(oracle.attention(q, k, v, 0.37, causal), ref)


# ---- closed forms ---------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_v(causal):
    q, k = rnd((2, 2, 11, 6), 13, 3.0), rnd((2, 2, 11, 6), 14, 3.0)
    row = rnd((6,), 15)
    v = np.broadcast_to(row, (2, 2, 11, 6)).copy()
    assert close(oracle.attention(q, k, v, 0.5, causal), v)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_keys_give_mean_or_prefix_mean(causal):
    q = rnd((1, 2, 10, 5), 16)
    k = np.broadcast_to(rnd((5,), 17), (1, 2, 10, 5)).copy()
    v = rnd((1, 2, 10, 5), 18)
    o = oracle.attention(q, k, v, 0.9, causal)
    if causal:
        want = np.cumsum(v, axis=2) / np.arange(1, 11)[None, None, :, None]
    else:
        want = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    assert close(o, want)


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero_is_uniform(causal):
    q, k, v = rnd((1, 1, 12, 4), 19, 50.0), rnd((1, 1, 12, 4), 20, 50.0), rnd((1, 1, 12, 4), 21)
    o = oracle.attention(q, k, v, 0.0, causal)
    if causal:
        want = np.cumsum(v, axis=2) / np.arange(1, 13)[None, None, :, None]
    else:
        want = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    assert close(o, want)


def test_causal_row0_is_v0():
    q, k, v = rnd((2, 2, 9, 4), 22, 4.0), rnd((2, 2, 9, 4), 23, 4.0), rnd((2, 2, 9, 4), 24)
    o = oracle.attention(q, k, v, 1.0, True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])


def test_single_position_is_v():
    q, k, v = rnd((3, 2, 1, 8), 25), rnd((3, 2, 1, 8), 26), rnd((3, 2, 1, 8), 27)
    for causal in (False, True):
        assert np.array_equal(oracle.attention(q, k, v, 0.7, causal), v)


@pytest.mark.parametrize("causal", [False, True])
def test_huge_logits_select_argmax(causal):
    """Logit gaps of >= 1000 make the softmax one-hot in float64 (exp(-1000) == 0).

    A version that exponentiates before subtracting the row max overflows here.
    """
    L, d = 6, 6
    k = 40.0 * np.eye(L, d)[None, None]                      # k_j = 40 e_j
    target = np.array([0, 0, 2, 1, 4, 3])                    # the key each query aligns with
    q = (40.0 * np.eye(d)[target])[None, None]               # q_i = 40 e_target(i)
    v = rnd((1, 1, L, d), 28)
    o = oracle.attention(q, k, v, 1.0, causal)               # logits 1600 vs 0
    assert np.array_equal(o[0, 0], v[0, 0, target])


# ---- invariants -------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows(causal):
    q, k = rnd((2, 2, 17, 8), 29, 2.0), rnd((2, 2, 17, 8), 30, 2.0)
    P = oracle.probabilities(q, k, 0.6, causal)
    assert np.all(P >= 0)
    assert np.max(np.abs(P.sum(-1) - 1.0)) <= 1e-12
    if causal:
        assert np.all(np.triu(P[0, 0], 1) == 0)
        assert np.all(np.diagonal(P, axis1=2, axis2=3) > 0)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    """Adding one vector to every key adds a per-query constant to each logit row."""
    q, k, v = rnd((1, 2, 14, 6), 31), rnd((1, 2, 14, 6), 32), rnd((1, 2, 14, 6), 33)
    c = rnd((6,), 34, 3.0)
    assert close(oracle.attention(q, k + c, v, 0.8, causal), oracle.attention(q, k, v, 0.8, causal), 1e-11)


def test_permutation_equivariance():
    q, k, v = rnd((1, 1, 15, 7), 35), rnd((1, 1, 15, 7), 36), rnd((1, 1, 15, 7), 37)
    perm = np.random.default_rng(38).permutation(15)
    o = oracle.attention(q, k, v, 0.5)
    assert close(oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.5), o)
    assert close(oracle.attention(q[:, :, perm], k, v, 0.5), o[:, :, perm])


@pytest.mark.parametrize("causal", [False, True])
def test_linear_in_v(causal):
    q, k = rnd((1, 2, 10, 4), 39), rnd((1, 2, 10, 4), 40)
    v1, v2 = rnd((1, 2, 10, 4), 41), rnd((1, 2, 10, 4), 42)
    lhs = oracle.attention(q, k, 2.5 * v1 - 0.75 * v2, 0.5, causal)
    rhs = 2.5 * oracle.attention(q, k, v1, 0.5, causal) - 0.75 * oracle.attention(q, k, v2, 0.5, causal)
    assert close(lhs, rhs)


def test_dimension_errors():
    with pytest.raises(ValueError):
        oracle.attention(np.zeros((1, 1, 3, 2)), np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 3, 2)), 1.0)


# ---- planted mistakes: the pins above must catch each one -------------------

def _pins_pass():
    """A compact run of the pins; False if any fails or raises."""
    try:
        for B, H, L, d, scale, causal in [(1, 2, 7, 4, 0.5, True), (1, 1, 6, 3, 0.7, False)]:
            q, k, v = rnd((B, H, L, d), 50), rnd((B, H, L, d), 51), rnd((B, H, L, d), 52)
            if not close(oracle.attention(q, k, v, scale, causal), brute_force(q, k, v, scale, causal)):
                return False
        for case in json.load(open(GOLDEN))["cases"]:
            got = oracle.attention(np.array(case["q"]), np.array(case["k"]), np.array(case["v"]),
                                   case["scale"], case["causal"])
            if not close(got, np.array(case["expected"]), 1e-14):
                return False
        L = 6
        k = 40.0 * np.eye(L)[None, None]
        t = np.array([0, 0, 2, 1, 4, 3])
        q = (40.0 * np.eye(L)[t])[None, None]
        v = rnd((1, 1, L, L), 53)
        with np.errstate(all="ignore"):
            o = oracle.attention(q, k, v, 1.0, False)
        if not np.array_equal(o[0, 0], v[0, 0, t]):
            return False
        return True
    except (AssertionError, ValueError, FloatingPointError):
        return False


def test_pins_pass_unmutated():
    assert _pins_pass()


MUTANTS = {
    "transposed_logits": ("logits", lambda Q, K, s: float(s) * (K @ Q.T) if Q.shape == K.shape else float(s) * (Q @ K.T)),
    "scale_dropped": ("logits", lambda Q, K, s: Q @ K.T),
    "scale_squared": ("logits", lambda Q, K, s: float(s) ** 2 * (Q @ K.T)),
    "causal_excludes_diagonal": ("causal_mask", lambda Z, qi: _mask_ge(Z, qi)),
    "causal_one_late": ("causal_mask", lambda Z, qi: _mask_gt(Z, np.asarray(qi) + 1)),
    "softmax_over_queries": ("softmax_rows", lambda Z: np.exp(Z - Z.max(0, keepdims=True)) / np.exp(Z - Z.max(0, keepdims=True)).sum(0, keepdims=True)),
    "softmax_unnormalised": ("softmax_rows", lambda Z: np.exp(Z - Z.max(1, keepdims=True))),
    "softmax_no_max_shift": ("softmax_rows", lambda Z: np.exp(Z) / np.exp(Z).sum(1, keepdims=True)),
    "softmax_sign_flip": ("softmax_rows", lambda Z: np.exp(-(Z - Z.max(1, keepdims=True))) / np.exp(-(Z - Z.max(1, keepdims=True))).sum(1, keepdims=True)),
    "values_transposed_weights": ("weighted_values", lambda P, V: P.T @ V),
}


def _mask_gt(Z, qi):
    Z = Z.copy()
    Z[np.arange(Z.shape[1])[None, :] > np.asarray(qi)[:, None]] = -np.inf
    return Z


def _mask_ge(Z, qi):
    Z = Z.copy()
    Z[np.arange(Z.shape[1])[None, :] >= np.asarray(qi)[:, None]] = -np.inf
    return Z


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, bad = MUTANTS[name]
    monkeypatch.setattr(oa, attr, bad)
    assert not _pins_pass(), f"pins did not catch mutant {name}"


# ---- log-sum-exp output and grouped key/value heads --------------------------

def brute_force_lse(q, k, scale, causal):
    """log(sum_j exp(s q_i . k_j)) with scalar loops, math.fsum and no max shift
    (the tiny cases keep every logit small)."""
    B, H, L, d = q.shape
    g = H // k.shape[1]
    out = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            for i in range(L):
                keys = range(i + 1) if causal else range(L)
                z = [scale * math.fsum(q[b, h, i, c] * k[b, h // g, j, c] for c in range(d)) for j in keys]
                out[b, h, i] = math.log(math.fsum(math.exp(x) for x in z))
    return out


@pytest.mark.parametrize("B,H,L,d,scale,causal", TINY)
def test_lse_brute_force_tiny(B, H, L, d, scale, causal):
    q, k = rnd((B, H, L, d), 60 + L), rnd((B, H, L, d), 61 + d)
    assert close(oracle.log_sum_exp(q, k, scale, causal), brute_force_lse(q, k, scale, causal))


@pytest.mark.parametrize("causal", [False, True])
def test_lse_equal_keys_is_logit_plus_log_count(causal):
    # every key equal to k0: each allowed logit is s q_i . k0, so the sum is
    # (number of allowed keys) * exp(s q_i . k0)
    L, d, s = 11, 6, 0.4
    q = rnd((1, 1, L, d), 62)
    k0 = rnd((d,), 63)
    k = np.broadcast_to(k0, (1, 1, L, d)).copy()
    count = np.arange(1, L + 1) if causal else np.full(L, L)
    expected = s * (q[0, 0] @ k0) + np.log(count)
    assert close(oracle.log_sum_exp(q, k, s, causal)[0, 0], expected)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_scale_zero_is_log_count(causal):
    L = 9
    q, k = rnd((1, 2, L, 4), 64), rnd((1, 2, L, 4), 65)
    count = np.arange(1, L + 1) if causal else np.full(L, L)
    got = oracle.log_sum_exp(q, k, 0.0, causal)
    assert close(got, np.broadcast_to(np.log(count), got.shape))


@pytest.mark.parametrize("causal", [False, True])
def test_lse_shifts_with_a_common_key_offset(causal):
    # k_j -> k_j + c adds s q_i . c to every logit of row i, hence to its LSE
    L, d, s = 10, 5, 0.6
    q, k = rnd((1, 1, L, d), 66), rnd((1, 1, L, d), 67)
    c = rnd((d,), 68)
    base = oracle.log_sum_exp(q, k, s, causal)[0, 0]
    shifted = oracle.log_sum_exp(q, k + c, s, causal)[0, 0]
    assert close(shifted - base, s * (q[0, 0] @ c))


@pytest.mark.parametrize("causal", [False, True])
def test_lse_torch_logsumexp(causal):
    L, d, s = 17, 8, 0.9
    q, k = rnd((2, 3, L, d), 69), rnd((2, 3, L, d), 70)
    z = s * torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2).contiguous()
    if causal:
        z = z.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), float("-inf"))
    assert close(oracle.log_sum_exp(q, k, s, causal), torch.logsumexp(z, dim=-1).numpy())


def test_lse_ties_probabilities():
    # P_ij = exp(z_ij - lse_i) for the allowed keys
    L, d, s = 8, 4, 0.7
    q, k = rnd((1, 1, L, d), 71), rnd((1, 1, L, d), 72)
    P = oracle.probabilities(q, k, s, True)[0, 0]
    Z = oracle.causal_mask(oracle.logits(q[0, 0], k[0, 0], s), np.arange(L))
    with np.errstate(all="ignore"):
        assert close(np.exp(Z - oracle.log_sum_exp(q, k, s, True)[0, 0][:, None]), P)


@pytest.mark.parametrize("H,H_kv", [(4, 2), (6, 3), (6, 1), (3, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_heads_constant_values(H, H_kv, causal):
    # key/value head j holds the constant value j + 1: every output row of query
    # head h is then exactly h // (H / H_kv) + 1 (consecutive query heads share a
    # key/value head; an interleaved h % H_kv mapping would differ for H = 4, 6)
    L, d = 7, 4
    q, k = rnd((2, H, L, d), 73), rnd((2, H_kv, L, d), 74)
    v = np.broadcast_to((np.arange(H_kv) + 1.0)[None, :, None, None], (2, H_kv, L, 3)).copy()
    o = oracle.attention(q, k, v, 0.5, causal)
    want = (np.arange(H) // (H // H_kv) + 1.0)[None, :, None, None]
    assert np.allclose(o, np.broadcast_to(want, o.shape), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_heads_equal_repeated_heads(causal):
    # a grouped call equals the one-to-one call on key/value heads repeated
    # consecutively, which the brute force pins
    B, H, H_kv, L, d = 1, 4, 2, 6, 3
    q, k, v = rnd((B, H, L, d), 75), rnd((B, H_kv, L, d), 76), rnd((B, H_kv, L, d), 77)
    kr, vr = np.repeat(k, H // H_kv, axis=1), np.repeat(v, H // H_kv, axis=1)
    assert close(oracle.attention(q, k, v, 0.8, causal), brute_force(q, kr, vr, 0.8, causal))
    assert close(oracle.log_sum_exp(q, k, 0.8, causal), brute_force_lse(q, kr, 0.8, causal))
    rows = [(0, h, i) for h in range(H) for i in (0, L - 1)]
    assert close(oracle.attention_rows(q, k, v, 0.8, causal, rows),
                 np.stack([brute_force(q, kr, vr, 0.8, causal)[b, h, i] for b, h, i in rows]))


def test_grouped_heads_dimension_errors():
    with pytest.raises(ValueError):  # 3 query heads over 2 key/value heads
        oracle.attention(np.zeros((1, 3, 4, 2)), np.zeros((1, 2, 4, 2)), np.zeros((1, 2, 4, 2)), 1.0)
    with pytest.raises(ValueError):  # k and v head counts differ
        oracle.attention(np.zeros((1, 4, 4, 2)), np.zeros((1, 2, 4, 2)), np.zeros((1, 4, 4, 2)), 1.0)


def _lse_pins_pass():
    try:
        for B, H, L, d, scale, causal in [(1, 2, 7, 4, 0.5, True), (1, 1, 6, 3, 0.7, False)]:
            q, k = rnd((B, H, L, d), 80), rnd((B, H, L, d), 81)
            if not close(oracle.log_sum_exp(q, k, scale, causal), brute_force_lse(q, k, scale, causal)):
                return False
        L = 5
        q = rnd((1, 1, L, 3), 82)
        k = np.broadcast_to(rnd((3,), 83), (1, 1, L, 3)).copy()
        if not close(oracle.log_sum_exp(q, k, 0.0, True)[0, 0], np.log(np.arange(1, L + 1))):
            return False
        return True
    except (AssertionError, ValueError, FloatingPointError):
        return False


LSE_MUTANTS = {
    "lse_max_dropped": lambda Z: np.log(np.exp(Z - Z.max(1, keepdims=True)).sum(1)),
    "lse_log2": lambda Z: Z.max(1) + np.log2(np.exp(Z - Z.max(1, keepdims=True)).sum(1)),
    "lse_mean_not_sum": lambda Z: Z.max(1) + np.log(np.exp(Z - Z.max(1, keepdims=True)).mean(1)),
    "lse_max_only": lambda Z: Z.max(1),
}


def test_lse_pins_pass_unmutated():
    assert _lse_pins_pass()


@pytest.mark.parametrize("name", sorted(LSE_MUTANTS))
def test_lse_pins_catch_planted_mistake(name, monkeypatch):
    monkeypatch.setattr(oa, "row_log_sum_exp", LSE_MUTANTS[name])
    assert not _lse_pins_pass(), f"pins did not catch mutant {name}"


# ---- sliding windows -----------------------------------------------------------

def allowed_keys(i, L, causal, window):
    lo, hi = 0, L - 1
    if window is not None:
        if window[0] is not None:
            lo = max(lo, i - window[0])
        if window[1] is not None:
            hi = min(hi, i + window[1])
    if causal:
        hi = min(hi, i)
    return range(lo, hi + 1)


def brute_force_window(q, k, v, scale, causal, window):
    """softmax over the allowed keys only (scalar loops, math.fsum)."""
    B, H, L, d = q.shape
    out = np.zeros((B, H, L, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            for i in range(L):
                keys = allowed_keys(i, L, causal, window)
                z = [scale * math.fsum(q[b, h, i, c] * k[b, h, j, c] for c in range(d)) for j in keys]
                m = max(z)
                e = [math.exp(x - m) for x in z]
                tot = math.fsum(e)
                for c in range(v.shape[-1]):
                    out[b, h, i, c] = math.fsum(e[t] * v[b, h, j, c] for t, j in enumerate(keys)) / tot
    return out


WINDOWS = [(0, 0), (1, 0), (0, 2), (2, 3), (None, 1), (3, None), (None, None), (20, 20)]


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("causal", [False, True])
def test_window_brute_force(window, causal):
    B, H, L, d = 1, 2, 9, 4
    q, k, v = rnd((B, H, L, d), 90), rnd((B, H, L, d), 91), rnd((B, H, L, d), 92)
    assert close(oracle.attention(q, k, v, 0.6, causal, window),
                 brute_force_window(q, k, v, 0.6, causal, window))


@pytest.mark.parametrize("causal", [False, True])
def test_window_of_width_zero_returns_v(causal):
    # each query sees only its own key: the softmax of one logit is 1
    q, k, v = rnd((2, 2, 13, 5), 93), rnd((2, 2, 13, 5), 94), rnd((2, 2, 13, 5), 95)
    assert np.array_equal(oracle.attention(q, k, v, 0.7, causal, (0, 0)), v)


def test_window_limits_reduce_to_causal_and_full():
    L = 12
    q, k, v = rnd((1, 2, L, 4), 96), rnd((1, 2, L, 4), 97), rnd((1, 2, L, 4), 98)
    assert close(oracle.attention(q, k, v, 0.5, False, (None, 0)), oracle.attention(q, k, v, 0.5, True))
    assert close(oracle.attention(q, k, v, 0.5, False, (L, L)), oracle.attention(q, k, v, 0.5, False))
    assert close(oracle.attention(q, k, v, 0.5, True, (L, 5)), oracle.attention(q, k, v, 0.5, True))


@pytest.mark.parametrize("window", [(2, 1), (0, 3), (4, 0), (None, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_window_equal_keys_give_window_means(window, causal):
    L, d = 11, 3
    q, v = rnd((1, 1, L, d), 99), rnd((1, 1, L, d), 100)
    k = np.broadcast_to(rnd((d,), 101), (1, 1, L, d)).copy()
    want = np.stack([v[0, 0, list(allowed_keys(i, L, causal, window))].mean(axis=0) for i in range(L)])
    assert close(oracle.attention(q, k, v, 0.9, causal, window)[0, 0], want)


@pytest.mark.parametrize("window", [(2, 1), (0, 0), (None, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_window_lse_scale_zero_is_log_count(window, causal):
    L = 10
    q, k = rnd((1, 1, L, 3), 102), rnd((1, 1, L, 3), 103)
    want = np.log([len(allowed_keys(i, L, causal, window)) for i in range(L)])
    assert close(oracle.log_sum_exp(q, k, 0.0, causal, window)[0, 0], want)


def test_window_rows_match_full():
    L = 14
    q, k, v = rnd((1, 2, L, 4), 104), rnd((1, 2, L, 4), 105), rnd((1, 2, L, 4), 106)
    rows = [(0, h, i) for h in range(2) for i in (0, 5, L - 1)]
    full = oracle.attention(q, k, v, 0.4, True, (3, 2))
    assert close(oracle.attention_rows(q, k, v, 0.4, True, rows, (3, 2)),
                 np.stack([full[b, h, i] for b, h, i in rows]))


def _window_pins_pass():
    try:
        q, k, v = rnd((1, 1, 9, 4), 110), rnd((1, 1, 9, 4), 111), rnd((1, 1, 9, 4), 112)
        for window in [(2, 3), (1, 0), (0, 2)]:
            if not close(oracle.attention(q, k, v, 0.6, False, window),
                         brute_force_window(q, k, v, 0.6, False, window)):
                return False
        if not np.array_equal(oracle.attention(q, k, v, 0.7, False, (0, 0)), v):
            return False
        return True
    except (AssertionError, ValueError, FloatingPointError):
        return False


def _shifted_window(dl, dr, swap=False):
    def bad(Z, qi, left, right):
        if swap:
            left, right = right, left
        return oa_window_ref(Z, qi, None if left is None else left + dl,
                             None if right is None else right + dr)
    return bad


oa_window_ref = oa.window_mask
WINDOW_MUTANTS = {
    "window_left_one_short": _shifted_window(-1, 0),
    "window_left_one_long": _shifted_window(1, 0),
    "window_right_one_short": _shifted_window(0, -1),
    "window_right_one_long": _shifted_window(0, 1),
    "window_sides_swapped": _shifted_window(0, 0, swap=True),
}


def test_window_pins_pass_unmutated():
    assert _window_pins_pass()


@pytest.mark.parametrize("name", sorted(WINDOW_MUTANTS))
def test_window_pins_catch_planted_mistake(name, monkeypatch):
    monkeypatch.setattr(oa, "window_mask", WINDOW_MUTANTS[name])
    assert not _window_pins_pass(), f"pins did not catch mutant {name}"


# ---- query and key lengths that differ (bottom-right alignment) -----------------

def brute_force_qk(q, k, v, scale, causal, window):
    """Scalar loops for Lq != Lk: query i stands at key position i + Lk - Lq; a
    row with no allowed key is 0."""
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    out = np.zeros((B, H, Lq, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            for i in range(Lq):
                p = i + Lk - Lq
                lo, hi = 0, Lk - 1
                if window is not None and window[0] is not None:
                    lo = max(lo, p - window[0])
                if window is not None and window[1] is not None:
                    hi = min(hi, p + window[1])
                if causal:
                    hi = min(hi, p)
                keys = range(lo, hi + 1)
                if len(keys) == 0:
                    continue
                z = [scale * math.fsum(q[b, h, i, c] * k[b, h, j, c] for c in range(d)) for j in keys]
                m = max(z)
                e = [math.exp(x - m) for x in z]
                tot = math.fsum(e)
                for c in range(v.shape[-1]):
                    out[b, h, i, c] = math.fsum(e[t] * v[b, h, j, c] for t, j in enumerate(keys)) / tot
    return out


@pytest.mark.parametrize("Lq,Lk", [(3, 9), (1, 7), (9, 4), (6, 6)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [None, (2, 1)])
def test_qk_lengths_brute_force(Lq, Lk, causal, window):
    q, k, v = rnd((1, 2, Lq, 4), 120 + Lq), rnd((1, 2, Lk, 4), 121 + Lk), rnd((1, 2, Lk, 3), 122)
    assert close(oracle.attention(q, k, v, 0.7, causal, window),
                 brute_force_qk(q, k, v, 0.7, causal, window))


@pytest.mark.parametrize("window", [None, (3, 2)])
def test_qk_last_rows_of_square_problem(window):
    # bottom-right alignment: Lq queries against Lk keys are the last Lq rows of
    # the square problem over the same keys
    Lq, Lk = 5, 12
    qf, k, v = rnd((1, 2, Lk, 4), 123), rnd((1, 2, Lk, 4), 124), rnd((1, 2, Lk, 4), 125)
    full = oracle.attention(qf, k, v, 0.6, True, window)
    part = oracle.attention(qf[:, :, Lk - Lq:], k, v, 0.6, True, window)
    assert close(part, full[:, :, Lk - Lq:])
    lf = oracle.log_sum_exp(qf, k, 0.6, True, window)
    assert close(oracle.log_sum_exp(qf[:, :, Lk - Lq:], k, 0.6, True, window), lf[:, :, Lk - Lq:])


def test_single_query_sees_every_key_when_causal():
    q, k, v = rnd((2, 2, 1, 5), 126), rnd((2, 2, 17, 5), 127), rnd((2, 2, 17, 5), 128)
    assert close(oracle.attention(q, k, v, 0.4, True), oracle.attention(q, k, v, 0.4, False))


def test_rows_without_keys_are_zero_and_lse_minus_inf():
    Lq, Lk = 7, 3
    q, k, v = rnd((1, 1, Lq, 4), 129), rnd((1, 1, Lk, 4), 130), rnd((1, 1, Lk, 4), 131)
    o = oracle.attention(q, k, v, 0.5, True)
    lse = oracle.log_sum_exp(q, k, 0.5, True)
    assert np.array_equal(o[0, 0, : Lq - Lk], np.zeros((Lq - Lk, 4)))
    assert np.all(lse[0, 0, : Lq - Lk] == -np.inf) and np.all(np.isfinite(lse[0, 0, Lq - Lk:]))
    assert close(o[0, 0, Lq - Lk:], oracle.attention(q[:, :, Lq - Lk:], k, v, 0.5, True)[0, 0])


def test_qk_pins_catch_top_left_alignment(monkeypatch):
    def top_left(Lq, Lk, rows=None):
        return np.arange(Lq) if rows is None else np.asarray(rows)
    q, k, v = rnd((1, 1, 3, 4), 132), rnd((1, 1, 9, 4), 133), rnd((1, 1, 9, 3), 134)
    want = brute_force_qk(q, k, v, 0.7, True, None)
    assert close(oracle.attention(q, k, v, 0.7, True), want)
    monkeypatch.setattr(oa, "_query_positions", top_left)
    assert not close(oracle.attention(q, k, v, 0.7, True), want)


# ---- compressed causal mask (keys compress cf = Lq // Lk queries each) --------

def brute_force_compressed(q, k, v, scale):
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    cf = max(1, Lq // Lk)
    out = np.zeros((B, H, Lq, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            for i in range(Lq):
                keys = range(0, min(Lk, (i + 1) // cf))
                if len(keys) == 0:
                    continue
                z = [scale * math.fsum(q[b, h, i, c] * k[b, h, j, c] for c in range(d)) for j in keys]
                m = max(z)
                e = [math.exp(x - m) for x in z]
                tot = math.fsum(e)
                for c in range(v.shape[-1]):
                    out[b, h, i, c] = math.fsum(e[t] * v[b, h, j, c] for t, j in enumerate(keys)) / tot
    return out


@pytest.mark.parametrize("Lq,Lk", [(12, 4), (10, 3), (7, 7), (9, 2)])
def test_compressed_causal_brute_force(Lq, Lk):
    q, k, v = rnd((1, 2, Lq, 4), 140 + Lq), rnd((1, 2, Lk, 4), 141 + Lk), rnd((1, 2, Lk, 3), 142)
    assert close(oracle.attention(q, k, v, 0.6, "compressed"), brute_force_compressed(q, k, v, 0.6))


def test_compressed_causal_with_cf_one_is_causal():
    q, k, v = rnd((1, 2, 9, 4), 143), rnd((1, 2, 9, 4), 144), rnd((1, 2, 9, 4), 145)
    assert close(oracle.attention(q, k, v, 0.5, "compressed"), oracle.attention(q, k, v, 0.5, True))
    assert close(oracle.log_sum_exp(q, k, 0.5, "compressed"), oracle.log_sum_exp(q, k, 0.5, True))


def test_compressed_causal_closed_forms():
    # cf = 3: query i sees keys 0 .. (i + 1) // 3 - 1; rows 0 and 1 see none;
    # at scale 0 each other row is the mean of that prefix of V, its LSE the
    # log of the prefix length
    Lq, Lk = 12, 4
    q, k, v = rnd((1, 1, Lq, 4), 146), rnd((1, 1, Lk, 4), 147), rnd((1, 1, Lk, 4), 148)
    o = oracle.attention(q, k, v, 0.0, "compressed")[0, 0]
    lse = oracle.log_sum_exp(q, k, 0.0, "compressed")[0, 0]
    for i in range(Lq):
        n = (i + 1) // 3
        if n == 0:
            assert np.array_equal(o[i], np.zeros(4)) and lse[i] == -np.inf
        else:
            assert close(o[i], v[0, 0, :n].mean(axis=0)) and close(lse[i], np.log(n))


@pytest.mark.parametrize("shift", [-1, 1])
def test_compressed_causal_pins_catch_off_by_one(shift, monkeypatch):
    q, k, v = rnd((1, 1, 12, 4), 149), rnd((1, 1, 4, 4), 150), rnd((1, 1, 4, 3), 151)
    want = brute_force_compressed(q, k, v, 0.6)
    assert close(oracle.attention(q, k, v, 0.6, "compressed"), want)
    ref = oa.compressed_causal_mask

    def shifted(Z, qi, cf):
        return ref(Z, np.asarray(qi) + shift * cf, cf)
    monkeypatch.setattr(oa, "compressed_causal_mask", shifted)
    assert not close(oracle.attention(q, k, v, 0.6, "compressed"), want)
