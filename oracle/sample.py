"""Speculative sampling at temperature T > 0 (TEST INFRASTRUCTURE ONLY; the product library
never imports this).

Quasar, Sec. 3.3 "Lossless Rejection Sampling": the target distribution p recovered in high
precision is compared with the draft distribution q (Eq. 2, whose formula is lost in the
text; Sec. 2.1 and the speculative-sampling abstract on the search-results page name the
modified rejection sampling of speculative decoding).  Reading taken: that standard scheme,
in float64 throughout.  Rows i < M-1 verify draft tokens, row M-1 gives the bonus token:

  p_i = softmax(target_logits[i] / T);
  q_i = softmax(draft_logits[i] / T), or, when no draft logits are given (a deterministic
        drafter such as n-gram lookup), the point mass at the draft token;
  for i = 0 .. M-2: the draft token x_i is accepted iff 0 <= x_i < V and u[i] * q_i(x_i) <
  p_i(x_i); at the first rejection i, the emitted token is drawn with u[M-1] from the
  residual weights max(0, p_i - q_i) (from p_i itself if those are all zero); if every draft
  is accepted, the bonus token is drawn from p_{M-1} with u[M-1].

Drawing from weights w with a uniform u in [0, 1) means the smallest v whose running sum of w
exceeds u * sum(w), or the last v with w > 0 if rounding leaves none.  Random numbers are
inputs, so every result is reproducible.  Returns (n_accept, token).
"""
from __future__ import annotations

import numpy as np


def softmax64(logits_row: np.ndarray, T: float) -> np.ndarray:
    """softmax(logits / T) in float64, shifted by the row maximum."""
    x = np.asarray(logits_row, dtype=np.float64)
    e = np.exp((x - x.max()) / T)
    return e / e.sum()


def draw(w: np.ndarray, u: float) -> int:
    """Inverse-CDF draw of an index from non-negative weights w (not necessarily normalised)."""
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    v = int(np.searchsorted(c, u * c[-1], side="right"))
    if v >= w.shape[0]:
        v = int(np.flatnonzero(w > 0)[-1])
    return v


def draft_distribution(draft_logits, i: int, x: int, V: int, T: float) -> np.ndarray:
    if draft_logits is not None:
        return softmax64(draft_logits[i], T)
    q = np.zeros(V)
    if 0 <= x < V:
        q[x] = 1.0
    return q


def speculative_sample(target_logits: np.ndarray, draft_logits, draft: np.ndarray,
                       u: np.ndarray, T: float):
    M, V = target_logits.shape
    for i in range(M - 1):
        x = int(draft[i])
        p = softmax64(target_logits[i], T)
        q = draft_distribution(draft_logits, i, x, V, T)
        if 0 <= x < V and u[i] * q[x] < p[x]:
            continue
        r = np.maximum(p - q, 0.0)
        return i, draw(r if r.sum() > 0 else p, float(u[M - 1]))
    return M - 1, draw(softmax64(target_logits[M - 1], T), float(u[M - 1]))


def decision_margins(target_logits: np.ndarray, draft_logits, draft: np.ndarray,
                     u: np.ndarray, T: float):
    """How far from a tie each decision the oracle takes lies, as relative gaps: one entry
    per examined draft (|p(x) - u q(x)| / max(p(x), u q(x))), then the final draw's distance
    from the running-sum boundaries around the drawn index (c[v] above it, the sum through
    the previous positive weight below it) over the total weight.  A GPU result computed in
    float64 in another summation order can only differ from the oracle where a gap is a few
    units in the last place."""
    M, V = target_logits.shape
    gaps = []
    n, _ = speculative_sample(target_logits, draft_logits, draft, u, T)
    for i in range(n + 1 if n < M - 1 else M - 1):
        x = int(draft[i])
        if not 0 <= x < V:
            gaps.append(np.inf)
            continue
        p = softmax64(target_logits[i], T)
        q = draft_distribution(draft_logits, i, x, V, T)
        a, b = p[x], u[i] * q[x]
        gaps.append(abs(a - b) / max(a, b) if max(a, b) > 0 else np.inf)
    if n < M - 1:
        x = int(draft[n])
        p = softmax64(target_logits[n], T)
        r = np.maximum(p - draft_distribution(draft_logits, n, x, V, T), 0.0)
        w = r if r.sum() > 0 else p
    else:
        w = softmax64(target_logits[M - 1], T)
    c = np.cumsum(w)
    t = float(u[M - 1]) * c[-1]
    v = draw(w, float(u[M - 1]))
    upper = c[v] - t if c[v] > t else 0.0            # 0: the fallback past the last sum
    before = np.flatnonzero(w[:v] > 0)
    lower = t - c[before[-1]] if before.size else np.inf  # no boundary below the first weight
    gaps.append(min(upper, lower) / c[-1])
    return gaps
