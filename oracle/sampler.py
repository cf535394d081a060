"""Oracle rejection sampler (test infrastructure; see package docstring).

The steps, in the order of Algorithm 1 as printed on [P1 "What one iteration
actually does"] and the rule on [P3 "Why the output doesn't change"]:

1. p_i = softmax(logits_i / T) for the gamma+1 verify rows.
2. Accept test for i = 1..gamma in order: reject iff r_i > p_i(x_i)/q_i(x_i)
   [P1, Algorithm 1, the step that counts the accepted guesses].  Written
   division-free as: accept iff u_i * q_i(x_i) <= p_i(x_i), evaluated in
   float32 (the same precision on both sides, since it decides an integer).
   q(x) = 0 therefore accepts.
3. n = index of the first rejection (a rejection cuts the rest of the
   block [P1 "What one iteration actually does"]), or n_draft when all
   drafts pass.
4. Corrected distribution for row j = n (0-based): if n < n_draft,
   norm(max(0, p_j - q_j)) [P1, Algorithm 1, the corrected distribution;
   P3 residual]; otherwise p_j itself (the bonus token [P2 "The
   draft-then-verify loop", step 3]).  The subtraction is float32.  An
   all-zero residual (p == q up to rounding) falls back to p_j.
5. t ~ p' by a fixed-point inverse CDF: w_v = floor(r_v * 2**40) (exact),
   S = sum w (exact in uint64), T = floor(k * S / 2**24) with k = u * 2**24,
   t = smallest v whose inclusive prefix sum exceeds T.  The pages only say
   "t ~ p'"; the normalisation of step 4 is carried by S.
6. Emit [x_1 .. x_n, t]; the rest of the gamma+1 slots hold -1.

All steps are vectorised over the batch with NumPy; nothing else is reordered.
Valid for V < 2**23 (so that S < 2**63).
"""

from __future__ import annotations

import numpy as np

TWO40 = float(1 << 40)
TWO24 = 1 << 24


def softmax(logits: np.ndarray, temperature: float = 1.0) -> np.ndarray:
    """Row softmax in fp64 over the last axis of logits / T.

    T = 0 is the limit T -> 0: the distribution collapses onto the argmax
    [P3 "Exactness is a choice"], written as a one-hot row at the lowest
    index among equal maxima (the tie rule of ``argmax_rows``).
    """
    if float(temperature) == 0.0:
        a = argmax_rows(logits)
        out = np.zeros(np.shape(logits), dtype=np.float64)
        np.put_along_axis(out, a[..., None], 1.0, axis=-1)
        return out
    x = np.asarray(logits, dtype=np.float64) / float(temperature)
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def accept_flags(p_x, q_x, u) -> np.ndarray:
    """Per-draft accept decision, float32: u * q(x) <= p(x)."""
    p_x = np.asarray(p_x, dtype=np.float32)
    q_x = np.asarray(q_x, dtype=np.float32)
    u = np.asarray(u, dtype=np.float32)
    return (u * q_x) <= p_x


def accepted_length(ok: np.ndarray, n_draft: np.ndarray) -> np.ndarray:
    """n = index of the first failed test among the first n_draft, else n_draft."""
    B, g = ok.shape
    n_draft = np.asarray(n_draft, dtype=np.int64)
    valid = np.arange(g)[None, :] < n_draft[:, None]
    fail = valid & ~ok
    first = np.argmax(fail, axis=1) if g > 0 else np.zeros(B, dtype=np.int64)
    return np.where(fail.any(axis=1) if g > 0 else np.zeros(B, bool), first, n_draft).astype(np.int64)


def fixed_point_weights(r: np.ndarray) -> np.ndarray:
    """w = floor(r * 2**40) as uint64 (r float32 in [0, 1]; exact)."""
    r64 = np.asarray(r, dtype=np.float32).astype(np.float64)
    return np.floor(r64 * TWO40).astype(np.uint64)


def fixed_point_draw(r: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Inverse-CDF draw from unnormalised float32 rows r [N, V] with uniforms u [N]."""
    w = fixed_point_weights(r)
    S = w.sum(axis=-1, dtype=np.uint64)
    k = (np.asarray(u, dtype=np.float32).astype(np.float64) * TWO24).astype(np.uint64)
    mask = np.uint64(TWO24 - 1)
    T = (S >> np.uint64(24)) * k + (((S & mask) * k) >> np.uint64(24))
    C = np.cumsum(w, axis=-1, dtype=np.uint64)
    return (C <= T[..., None]).sum(axis=-1).astype(np.int64)


def reject_sample(p: np.ndarray, q, draft: np.ndarray, n_draft, u_acc: np.ndarray, u_res: np.ndarray):
    """One round's accept/resample given probability rows.

    p [B, g+1, V] float32 target rows; q [B, g, V] float32 draft rows, or None
    for a one-hot draft (q_i(x_i) = 1); draft [B, g] token ids; n_draft [B] or
    None (= g); u_acc [B, g], u_res [B] float32 uniforms.
    Returns (n [B] int64, emitted [B, g+1] int64, -1 padded).
    """
    p = np.asarray(p, dtype=np.float32)
    B, g1, V = p.shape
    g = g1 - 1
    draft = np.asarray(draft, dtype=np.int64).reshape(B, g)
    nd = np.full(B, g, dtype=np.int64) if n_draft is None else np.clip(np.asarray(n_draft, np.int64), 0, g)
    if g > 0:
        p_x = np.take_along_axis(p[:, :g, :], draft[:, :, None], axis=2)[..., 0]
        if q is None:
            q_x = np.ones((B, g), dtype=np.float32)
        else:
            q = np.asarray(q, dtype=np.float32)
            q_x = np.take_along_axis(q, draft[:, :, None], axis=2)[..., 0]
        ok = accept_flags(p_x, q_x, np.asarray(u_acc, np.float32).reshape(B, g))
    else:
        ok = np.zeros((B, 0), dtype=bool)
    n = accepted_length(ok, nd)
    r = corrected_rows(p, q, draft, n, nd)
    t = fixed_point_draw(r, np.asarray(u_res, np.float32).reshape(B))
    emitted = np.full((B, g + 1), -1, dtype=np.int64)
    for b in range(B):
        emitted[b, : n[b]] = draft[b, : n[b]]
        emitted[b, n[b]] = t[b]
    return n, emitted


def corrected_rows(p: np.ndarray, q, draft: np.ndarray, n: np.ndarray, nd: np.ndarray) -> np.ndarray:
    """Step 4: the row the round's last token is drawn from, per sequence.

    Row j = n of p; after a rejection (n < n_draft) the residual
    max(0, p_j - q_j) in float32 (a one-hot draft zeroes only the rejected
    token x_j), else p_j itself (the bonus).  A residual with no mass left on
    the fixed-point grid falls back to p_j.  p [B, g+1, V], q [B, g, V] or
    None, draft [B, g], n and nd [B].  Returns float32 [B, V]."""
    p = np.asarray(p, dtype=np.float32)
    B, _, V = p.shape
    n = np.asarray(n, np.int64)
    nd = np.asarray(nd, np.int64)
    draft = np.asarray(draft, np.int64).reshape(B, -1)
    pj = p[np.arange(B), n]  # [B, V]
    r = pj.copy()
    rej = n < nd
    if rej.any():
        idx = np.nonzero(rej)[0]
        if q is None:
            qj = np.zeros((len(idx), V), dtype=np.float32)
            qj[np.arange(len(idx)), draft[idx, n[idx]]] = 1.0
        else:
            qj = np.asarray(q, dtype=np.float32)[idx, n[idx]]
        r[idx] = np.maximum(np.float32(0.0), pj[idx] - qj)
    empty = fixed_point_weights(r).sum(axis=-1, dtype=np.uint64) == 0
    r[empty] = pj[empty]
    return r


def argmax_rows(logits: np.ndarray) -> np.ndarray:
    """Index of the largest entry of each row (last axis); among equal maxima
    the lowest index.  The comparison is made in the precision the logits
    arrive in, so a caller checking float32 logits passes float32."""
    return np.argmax(np.asarray(logits), axis=-1).astype(np.int64)


def greedy_verify(logits: np.ndarray, draft: np.ndarray, n_draft=None):
    """Greedy (T = 0) verification of one round.

    At temperature zero the target's distribution is its argmax [P3
    "Exactness is a choice"; P4 section 4.2 on acceptance measured under
    greedy decoding].  With a_i = argmax(logits_i) for the gamma + 1 rows: draft x_i
    is accepted while x_i == a_i; n = the first mismatch among the first
    n_draft drafts, else n_draft; the round emits x_1 .. x_n and then a_n
    (0-based row n): at a mismatch the target's own choice replaces the
    draft, and after a full pass a_gamma is the bonus token.

    logits [B, g+1, V]; draft [B, g]; n_draft [B] or None (= g).
    Returns (n [B] int64, emitted [B, g+1] int64, -1 padded).
    """
    logits = np.asarray(logits)
    B, g1, V = logits.shape
    g = g1 - 1
    draft = np.asarray(draft, dtype=np.int64).reshape(B, g)
    nd = np.full(B, g, dtype=np.int64) if n_draft is None else np.clip(np.asarray(n_draft, np.int64), 0, g)
    a = argmax_rows(logits)  # [B, g+1]
    n = accepted_length(draft == a[:, :g], nd)
    emitted = np.full((B, g + 1), -1, dtype=np.int64)
    for b in range(B):
        emitted[b, : n[b]] = draft[b, : n[b]]
        emitted[b, n[b]] = a[b, n[b]]
    return n, emitted


def sample(p: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Plain draw t ~ p (the gamma = 0 round): rows p [N, V], uniforms u [N]."""
    p = np.asarray(p, dtype=np.float32)
    N, V = p.shape
    n, em = reject_sample(p[:, None, :], None, np.zeros((N, 0), np.int64), None,
                          np.zeros((N, 0), np.float32), u)
    return em[:, 0]
