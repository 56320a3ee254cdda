"""Exact softmax attention, O = softmax(s * Q K^T) V, in plain float64 NumPy.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU baseline leg, never by the library or its binding.

What it computes, and where the pages define it:
  * FastVideo wan22_vae_decode attn.cu, header comment: per latent frame one head
    of softmax(q k^T / 32) v over the H*W positions, C channels, no mask; and
    stage 3, the row softmax exp(S * scale - max) / sum.
  * same page, row_softmax_kernel: scale the row, take its max, exponentiate the
    difference, sum, multiply by the reciprocal of the sum.
  * cuDNN native_sparse_attention fmha.py (Blackwell FMHA example), module
    docstring and softmax_step: Q*K^T, a numerically stable softmax (row max
    subtracted before the exponential, then normalised by the row sum), times V,
    with an optional causal mask that removes keys after the query.

  * cuDNN native_sparse_attention fmha.py, __call__ and the epilogue: the query
    heads may be a multiple of the key/value heads, each key/value head serving
    a group of consecutive query heads (a zero stride over the group index
    broadcasts it); and the optional LSE output per query row, the log of the
    row sum plus the scaled row maximum, i.e. log(sum_j exp(z_ij)).
  * same page, __call__ parameters window_size_left / window_size_right: a
    sliding-window mask.  Its body is not on the page; the reading taken is
    key j allowed for query i iff i - left <= j <= i + right (None: that side
    unbounded), applied on top of the causal mask.
  * same page, __call__ problem_size (s_q, s_k) and cum_seqlen_q / cum_seqlen_k:
    the query and key lengths may differ.  Reading taken: bottom-right
    alignment, query i standing at key position i + (Lk - Lq) for the causal
    and window masks (the last query sees the last key, as in decoding against
    a cache); a row that then sees no key (Lq > Lk) outputs 0 and its LSE is
    -inf, as that page's softmax_step guard for an all -inf row gives.
  * same page, the compressed causal mask of its softmax: with the keys a
    compression of the queries by cf = Lq // Lk, query i (counted from 0)
    sees keys j <= (i + 1) // cf - 1; cf = 1 is the causal mask.

The method reaches exactly the plain definition (up to rounding order), so this
oracle is that definition written out, one step per function, in the pages'
order: logits, mask, row softmax, weighted sum of value rows; and for the LSE
output the row maximum plus the log of the shifted row sum.  Inputs are the
exact bf16 values as float64 arrays; the result is float64 and never rounded.

Readings where the pages leave a step open (each listed in the design notes):
  * the scale is the caller's, applied to the logits before the row max (the
    attn.cu softmax scales the row first); any finite value, including 0 and
    negative values, is allowed;
  * causal means key j is allowed for query i iff j <= i (square attention, so
    top-left and bottom-right alignment coincide);
  * a row with every key masked cannot occur (the diagonal is always allowed);
    the oracle asserts it rather than inventing an output.

Pins (tests/test_oracle.py): brute-force loops with math.fsum on tiny inputs
(with and without windows),
closed forms (constant V, equal keys, causal row 0, scale 0, L = 1, a one-hot
limit with huge logits, a hand-worked example in tests/golden, log L and
log(i + 1) for the LSE of equal keys, one constant value per key/value head
for the head groups, O = V for a window of width zero, window means of V for
equal keys, one query against all keys, zero rows when Lq > Lk), invariants
(the last Lq rows of a square causal problem equal the Lq < Lk one), (rows of P sum to 1, key-shift invariance,
permutation equivariance, linearity in V, the LSE's exact shift when every
key moves by the same vector) and a cross-check against torch's CPU float64
attention.  No function here is unpinned.
"""
from __future__ import annotations

import numpy as np


def logits(Q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """Z = s * Q K^T for one head: Q [n, d], K [L, d] -> Z [n, L]."""
    return float(scale) * (Q @ K.T)


def causal_mask(Z: np.ndarray, query_index: np.ndarray) -> np.ndarray:
    """Set Z[r, j] = -inf where key j comes after the query at position query_index[r]."""
    Z = Z.copy()
    keys = np.arange(Z.shape[1])
    Z[keys[None, :] > np.asarray(query_index)[:, None]] = -np.inf
    return Z


def window_mask(Z: np.ndarray, query_index: np.ndarray, left, right) -> np.ndarray:
    """Set Z[r, j] = -inf where key j lies more than `left` keys before or more
    than `right` keys after the query at position query_index[r] (None: no
    limit on that side)."""
    Z = Z.copy()
    keys = np.arange(Z.shape[1])[None, :]
    qi = np.asarray(query_index)[:, None]
    if left is not None:
        Z[keys < qi - left] = -np.inf
    if right is not None:
        Z[keys > qi + right] = -np.inf
    return Z


def compressed_causal_mask(Z: np.ndarray, query_index: np.ndarray, cf: int) -> np.ndarray:
    """Set Z[r, j] = -inf where j > (query_index[r] + 1) // cf - 1 (keys that
    compress cf queries each, none after the query's own block)."""
    Z = Z.copy()
    keys = np.arange(Z.shape[1])[None, :]
    last = (np.asarray(query_index)[:, None] + 1) // cf - 1
    Z[keys > last] = -np.inf
    return Z


def softmax_rows(Z: np.ndarray, allow_empty: bool = False) -> np.ndarray:
    """Numerically stable row softmax: exp(Z - rowmax) / rowsum.  A row with
    every key masked is an error unless allow_empty, when it becomes all 0."""
    m = Z.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m[:, 0])
    assert allow_empty or not empty.any(), "a row with every key masked"
    E = np.exp(Z - np.where(np.isfinite(m), m, 0.0))
    E[empty] = 0.0
    tot = E.sum(axis=1, keepdims=True)
    return E / np.where(tot > 0, tot, 1.0)


def weighted_values(P: np.ndarray, V: np.ndarray) -> np.ndarray:
    """O = P V: each output row is the P-weighted sum of the value rows."""
    return P @ V


def row_log_sum_exp(Z: np.ndarray, allow_empty: bool = False) -> np.ndarray:
    """log(sum_j exp(Z[r, j])) per row, as the row maximum plus the log of the
    row sum of exp(Z - max) (the LSE the FMHA epilogue stores); -inf for a row
    with every key masked (only with allow_empty)."""
    m = Z.max(axis=1)
    empty = ~np.isfinite(m)
    assert allow_empty or not empty.any(), "a row with every key masked"
    mm = np.where(empty, 0.0, m)
    with np.errstate(divide="ignore"):  # log(0) = -inf for the empty rows
        out = mm + np.log(np.exp(Z - mm[:, None]).sum(axis=1))
    out[empty] = -np.inf
    return out


def _head(x, b: int, h: int) -> np.ndarray:
    """One (batch, head) slice as float64 (exact for bf16 or float32 inputs)."""
    return np.asarray(x[b, h], dtype=np.float64)


def _dims(q, k, v):
    """(B, H, Lq, group): q is [B, H, Lq, d]; k and v are [B, H_kv, Lk, .] with
    H_kv dividing H, and query head h reads key/value head h // group."""
    sq, sk, sv = np.shape(q), np.shape(k), np.shape(v)
    if not (len(sq) == 4 and len(sk) == 4 and len(sv) == 4 and sq[0] == sk[0] == sv[0]
            and sk[2] == sv[2] and sq[3] == sk[3] and sk[1] == sv[1]
            and sk[1] >= 1 and sq[1] % sk[1] == 0):
        raise ValueError("q must be [B, H, Lq, d] and k, v [B, H_kv, Lk, .] with H_kv dividing H "
                         "(q, k share d)")
    return sq[0], sq[1], sq[2], sq[1] // sk[1]


def _query_positions(Lq: int, Lk: int, rows=None) -> np.ndarray:
    """Key position of each query row: bottom-right alignment, i + (Lk - Lq)."""
    i = np.arange(Lq) if rows is None else np.asarray(rows)
    return i + (Lk - Lq)


def _positions(causal, Lq: int, Lk: int, rows=None):
    """What _masked_logits needs to place the rows: key positions, or for the
    compressed causal mask the rows counted from 0 with the query count."""
    if isinstance(causal, str):
        return (np.arange(Lq) if rows is None else np.asarray(rows), Lq)
    return _query_positions(Lq, Lk, rows)


def _may_be_empty(causal, Lq: int, Lk: int) -> bool:
    """Whether a row can be left with no key (then it is 0, its LSE -inf)."""
    return Lq > Lk or isinstance(causal, str)


def _masked_logits(Q, K, scale, causal, window, query_index):
    """Logits of the rows at query_index with the causal and window masks.
    causal == "compressed": the compressed causal mask; query_index is then a
    pair (rows counted from 0, Lq) and cf = Lq // Lk."""
    Z = logits(Q, K, scale)
    if isinstance(causal, str):
        assert causal == "compressed" and window is None, "compressed causal takes no window"
        rows, Lq = query_index
        return compressed_causal_mask(Z, rows, max(1, Lq // max(1, K.shape[0])))
    if causal:
        Z = causal_mask(Z, query_index)
    if window is not None:
        Z = window_mask(Z, query_index, window[0], window[1])
    return Z


def probabilities(q, k, scale: float, causal: bool = False, window=None) -> np.ndarray:
    """P = softmax(s * Q K^T) (masked when causal / windowed), shape [B, H, Lq, Lk]."""
    B, H, L, g = _dims(q, k, k)
    Lk = np.shape(k)[2]
    P = np.empty((B, H, L, Lk), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            Z = _masked_logits(_head(q, b, h), _head(k, b, h // g), scale, causal, window,
                               _positions(causal, L, Lk))
            empty_ok = _may_be_empty(causal, L, Lk)
            P[b, h] = softmax_rows(Z, allow_empty=True) if empty_ok else softmax_rows(Z)
    return P


def attention(q, k, v, scale: float, causal: bool = False, window=None) -> np.ndarray:
    """O = softmax(s * Q K^T) V for every (batch, head); float64 [B, H, Lq, dv].

    k and v may have fewer heads than q (H_kv dividing H): query head h then
    reads key/value head h // (H / H_kv), and Lk keys (Lk may differ from Lq:
    query i stands at key position p = i + Lk - Lq).  window = (left, right)
    restricts query i to keys p - left .. p + right (None on a side:
    unbounded); causal to keys <= p; causal="compressed" to keys
    j <= (i + 1) // cf - 1, cf = Lq // Lk.  A query with no key left gives 0."""
    B, H, L, g = _dims(q, k, v)
    Lk = np.shape(k)[2]
    O = np.empty((B, H, L, np.shape(v)[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            Z = _masked_logits(_head(q, b, h), _head(k, b, h // g), scale, causal, window,
                               _positions(causal, L, Lk))
            P = softmax_rows(Z, allow_empty=True) if _may_be_empty(causal, L, Lk) else softmax_rows(Z)
            O[b, h] = weighted_values(P, _head(v, b, h // g))
    return O


def log_sum_exp(q, k, scale: float, causal: bool = False, window=None) -> np.ndarray:
    """lse[b, h, i] = log(sum over allowed keys j of exp(s * q_i . k_j)); float64
    [B, H, L].  Key heads and the window as in attention()."""
    B, H, L, g = _dims(q, k, k)
    Lk = np.shape(k)[2]
    out = np.empty((B, H, L), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            Z = _masked_logits(_head(q, b, h), _head(k, b, h // g), scale, causal, window,
                               _positions(causal, L, Lk))
            empty_ok = _may_be_empty(causal, L, Lk)
            out[b, h] = row_log_sum_exp(Z, allow_empty=True) if empty_ok else row_log_sum_exp(Z)
    return out


def attention_rows(q, k, v, scale: float, causal: bool, rows, window=None) -> np.ndarray:
    """The same definition evaluated only at the output rows listed in ``rows``.

    ``rows`` is a sequence of (b, h, i); returns float64 [len(rows), d].  Used to
    check full-size runs on a sample of rows the oracle can afford one by one.
    """
    g = _dims(q, k, v)[3]
    out = np.empty((len(rows), np.shape(v)[-1]), dtype=np.float64)
    cache = {}
    for r, (b, h, i) in enumerate(rows):
        if (b, h // g) not in cache:
            cache.clear()  # one head's K and V in float64 at a time
            cache[(b, h // g)] = (_head(k, b, h // g), _head(v, b, h // g))
        K, V = cache[(b, h // g)]
        Lq, Lk = np.shape(q)[2], np.shape(k)[2]
        Z = _masked_logits(np.asarray(q[b, h, i : i + 1], dtype=np.float64), K, scale, causal,
                           window, _positions(causal, Lq, Lk, [i]))
        P = softmax_rows(Z, allow_empty=True) if _may_be_empty(causal, Lq, Lk) else softmax_rows(Z)
        out[r] = weighted_values(P, V)[0]
    return out
