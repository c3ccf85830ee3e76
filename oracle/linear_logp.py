"""fp64 CPU oracle for the selected-token log-probability ("linear_logp").

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (``selected_token_lm_amd``) never does, and this module shares
no code with it: the only thing both sides use is the seeded input generator
in ``synth/``, which holds none of the operator's arithmetic.

What is computed is the plain definition.  "Announcing RL-Kernel for vime",
section "Key Capabilities", defines the operator as the log-softmax of the
logits ``hidden @ W^T`` evaluated at the target token, and section "Why the
Fused Path Wins" gives its boundary as hidden + lm_head_weight + target_ids
-> selected logprob.  For each token row t with target y_t:

    z[t, v]  = sum_k h[t, k] * W[v, k]
    lse[t]   = log(sum_v exp(z[t, v]))
    logp[t]  = z[t, y_t] - lse[t]

Rows whose target equals ``ignore_index`` are inactive: their logp, lse and
gradient rows are 0 and they contribute nothing to grad_W (the usual
ignore-index semantics; the pages do not spell this out).

Everything is evaluated in float64 on the exact values of the bf16 inputs.
The vocabulary is processed in blocks only to bound memory; inside a block
the logits are a plain float64 matrix product, and the log-sum-exp over
blocks uses the exact identity
    log(sum_a + sum_b) = M + log(sum_a e^{-M} + sum_b e^{-M}),  M = running max,
which changes nothing but float64 rounding.

Pins (tests/test_oracle_pins.py) tie every function here to something other
than itself: closed forms (zero and one-hot inputs), brute force over every
target on tiny inputs, a library log-softmax on materialised logits, central
finite differences for the gradients, the merge algebra, masking and row
permutation.  No function in this file is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

IGNORE_INDEX = -100


# -- input decoding --------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 numbers given as uint16 bit patterns, as float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _as_f64(x: np.ndarray) -> np.ndarray:
    """Accept either bf16 bit patterns (uint16) or real-valued arrays."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    return x.astype(np.float64)


def _active(y: np.ndarray, V: int, ignore_index: int) -> np.ndarray:
    y = np.asarray(y).astype(np.int64)
    act = y != ignore_index
    bad = act & ((y < 0) | (y >= V))
    if np.any(bad):
        raise ValueError(f"{int(bad.sum())} active targets outside [0, {V})")
    return act


# -- forward ------------------------------------------------------------------

def _logsumexp_rows(Ha: np.ndarray, W: np.ndarray, vocab_block: int):
    """Row-wise (max, sum exp(z - max)) of z = Ha @ W^T over all rows of W.

    Returns (m, s) with lse = m + log(s).  Blocks of the vocabulary are folded
    with the running-max identity (exact up to float64 rounding).
    """
    n = Ha.shape[0]
    m = np.full(n, -np.inf)
    s = np.zeros(n)
    for v0 in range(0, W.shape[0], vocab_block):
        Z = Ha @ W[v0:v0 + vocab_block].T
        m_new = np.maximum(m, Z.max(axis=1))
        s = s * np.exp(m - m_new) + np.exp(Z - m_new[:, None]).sum(axis=1)
        m = m_new
    return m, s


def forward(h, W, y, ignore_index: int = IGNORE_INDEX, vocab_block: int = 8192):
    """Selected-token log-probabilities and log-sum-exp, in float64.

    h: [T, H], W: [V, H] (uint16 bf16 bits or real arrays), y: [T] ints.
    Returns (logp [T], lse [T]); inactive rows hold 0 in both.
    """
    Hm = _as_f64(h)
    Wm = _as_f64(W)
    y = np.asarray(y).astype(np.int64)
    T, V = Hm.shape[0], Wm.shape[0]
    act = _active(y, V, ignore_index)
    logp = np.zeros(T)
    lse = np.zeros(T)
    if not act.any():
        return logp, lse
    Ha = Hm[act]
    ya = y[act]
    m, s = _logsumexp_rows(Ha, Wm, vocab_block)
    lse_a = m + np.log(s)
    # target logit as its own dot product h_t . W[y_t]
    z_t = np.einsum("tk,tk->t", Ha, Wm[ya])
    logp[act] = z_t - lse_a
    lse[act] = lse_a
    return logp, lse


# -- vocabulary-range partials and their merge ---------------------------------

def partial(h, W_shard, y, vocab_start: int, ignore_index: int = IGNORE_INDEX,
            vocab_block: int = 8192):
    """Statistics of one contiguous vocabulary range [vocab_start, vocab_start+len).

    Per row: m = max_v z, s = sum_v exp(z - m) over the range, owned = whether
    y_t lies in the range, z_t = z[t, y_t] when owned (else 0).  Inactive rows
    hold (m, s, z_t, owned) = (-inf, 0, 0, 0).  "Why the Fused Path Wins"
    (third reason) describes each rank reducing its local vocabulary shard and
    combining only these statistics.
    """
    Hm = _as_f64(h)
    Ws = _as_f64(W_shard)
    y = np.asarray(y).astype(np.int64)
    T, n = Hm.shape[0], Ws.shape[0]
    act = y != ignore_index
    m = np.full(T, -np.inf)
    s = np.zeros(T)
    z_t = np.zeros(T)
    local = y - vocab_start
    owned = act & (local >= 0) & (local < n)
    if act.any():
        m_a, s_a = _logsumexp_rows(Hm[act], Ws, vocab_block)
        m[act] = m_a
        s[act] = s_a
    if owned.any():
        z_t[owned] = np.einsum("tk,tk->t", Hm[owned], Ws[local[owned]])
    return {"m": m, "s": s, "z_t": z_t, "owned": owned}


def merge(parts, y, ignore_index: int = IGNORE_INDEX):
    """Combine range partials into (logp, lse), float64.

    m = max_r m_r;  s = sum_r s_r * exp(m_r - m);  lse = m + log s;
    logp = z_t(owner) - lse.  Exactly one part must own each active target.
    """
    y = np.asarray(y).astype(np.int64)
    act = y != ignore_index
    M = np.stack([p["m"] for p in parts])
    S = np.stack([p["s"] for p in parts])
    OWN = np.stack([p["owned"] for p in parts])
    ZT = np.stack([p["z_t"] for p in parts])
    T = y.shape[0]
    logp = np.zeros(T)
    lse = np.zeros(T)
    if not act.any():
        return logp, lse
    n_own = OWN[:, act].sum(axis=0)
    if np.any(n_own != 1):
        raise ValueError("every active target must be owned by exactly one part")
    m = M[:, act].max(axis=0)
    s = (S[:, act] * np.exp(M[:, act] - m)).sum(axis=0)
    lse_a = m + np.log(s)
    z_t = (ZT[:, act] * OWN[:, act]).sum(axis=0)
    logp[act] = z_t - lse_a
    lse[act] = lse_a
    return logp, lse


# -- backward ------------------------------------------------------------------

def backward(h, W, y, g, ignore_index: int = IGNORE_INDEX, vocab_block: int = 8192,
             want_grad_h: bool = True, want_grad_W: bool = True):
    """Gradients of L = sum_t g_t * logp_t with respect to h and W, float64.

    With p = softmax(z) per row and onehot(y):  dL/dz = g * (onehot(y) - p),
    grad_h = dL/dz @ W,  grad_W = (dL/dz)^T @ h.  Inactive rows contribute
    nothing and get zero grad_h rows.  "Announcing RL-Kernel for vime",
    "Key Capabilities", describes the full-gradient path (gradients reach both
    the hidden states and the weight).
    Returns (grad_h [T, H] or None, grad_W [V, H] or None).
    """
    Hm = _as_f64(h)
    Wm = _as_f64(W)
    y = np.asarray(y).astype(np.int64)
    gg = np.asarray(g, dtype=np.float64)
    T, Hd = Hm.shape
    V = Wm.shape[0]
    act = _active(y, V, ignore_index)
    grad_h = np.zeros((T, Hd)) if want_grad_h else None
    grad_W = np.zeros((V, Hd)) if want_grad_W else None
    if not act.any():
        return grad_h, grad_W
    Ha = Hm[act]
    ya = y[act]
    ga = gg[act]
    m, s = _logsumexp_rows(Ha, Wm, vocab_block)
    lse = m + np.log(s)
    gh_a = np.zeros_like(Ha) if want_grad_h else None
    rows = np.arange(Ha.shape[0])
    for v0 in range(0, V, vocab_block):
        v1 = min(V, v0 + vocab_block)
        Wb = Wm[v0:v1]
        P = np.exp(Ha @ Wb.T - lse[:, None])
        dZ = -ga[:, None] * P
        hit = (ya >= v0) & (ya < v1)
        dZ[rows[hit], ya[hit] - v0] += ga[hit]
        if want_grad_h:
            gh_a += dZ @ Wb
        if want_grad_W:
            grad_W[v0:v1] = dZ.T @ Ha
    if want_grad_h:
        grad_h[act] = gh_a
    return grad_h, grad_W


def backward_rows(h, W, y, g, rows, ignore_index: int = IGNORE_INDEX, vocab_block: int = 8192):
    """grad_h restricted to the given rows (each row's gradient depends only on
    that row), float64 [len(rows), H]."""
    rows = np.asarray(rows, dtype=np.int64)
    gh, _ = backward(np.asarray(h)[rows], W, np.asarray(y)[rows], np.asarray(g)[rows],
                     ignore_index, vocab_block, want_grad_h=True, want_grad_W=False)
    return gh


def grad_W_rows(h, W, y, g, vocab_rows, ignore_index: int = IGNORE_INDEX,
                vocab_block: int = 8192):
    """grad_W restricted to the given vocabulary rows, float64 [len(vocab_rows), H].

    Needs each active row's full log-sum-exp, computed here over all of W.
    """
    Hm = _as_f64(h)
    Wm = _as_f64(W)
    y = np.asarray(y).astype(np.int64)
    gg = np.asarray(g, dtype=np.float64)
    vr = np.asarray(vocab_rows, dtype=np.int64)
    act = _active(y, Wm.shape[0], ignore_index)
    out = np.zeros((vr.shape[0], Hm.shape[1]))
    if not act.any():
        return out
    Ha, ya, ga = Hm[act], y[act], gg[act]
    m, s = _logsumexp_rows(Ha, Wm, vocab_block)
    lse = m + np.log(s)
    P = np.exp(Ha @ Wm[vr].T - lse[:, None])          # [T_act, n]
    dZ = -ga[:, None] * P
    dZ += ga[:, None] * (ya[:, None] == vr[None, :])
    return dZ.T @ Ha
