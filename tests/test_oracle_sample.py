"""Pins of the speculative-sampling oracle (oracle/sample.py).

The scheme is lossless: the first emitted token is distributed exactly as the target's p_0,
whatever the draft distribution q_0.  That is checked by simulation against p_0 (with the
draft token drawn from q_0), together with special cases that fix the answer: q = p always
accepts; a draft whose mass lies where p has none is always rejected and the emitted token
then follows p; and the inverse-CDF draw against a brute-force loop.
"""
import numpy as np
import pytest

from oracle.sample import decision_margins, draw, softmax64, speculative_sample


def test_draw_matches_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(300):
        w = rng.random(9) * (rng.random(9) < 0.7)
        if w.sum() == 0:
            continue
        u = float(rng.random())
        t, acc = u * w.sum(), 0.0
        expect = None
        for v in range(9):
            acc += w[v]
            if acc > t:
                expect = v
                break
        if expect is None:
            expect = int(np.flatnonzero(w > 0)[-1])
        assert draw(w, u) == expect


def test_softmax_is_a_distribution_and_shift_invariant():
    x = np.array([1.0, -2.0, 3.5, 0.0])
    p = softmax64(x, 0.7)
    assert abs(p.sum() - 1.0) < 1e-15 and (p > 0).all()
    assert np.allclose(softmax64(x + 40.0, 0.7), p, rtol=0, atol=1e-15)
    assert int(np.argmax(p)) == 2


def test_identical_distributions_always_accept():
    rng = np.random.default_rng(1)
    for _ in range(50):
        M, V = 5, 11
        lg = rng.standard_normal((M, V)) * 3
        draft = rng.integers(0, V, M - 1)
        u = rng.random(M)
        n, tok = speculative_sample(lg, lg[: M - 1], draft, u, 0.8)
        assert n == M - 1
        assert tok == draw(softmax64(lg[M - 1], 0.8), u[M - 1])


def test_disjoint_support_always_rejects_and_follows_p():
    V = 6
    target = np.array([[5.0, 5.0, 5.0, -1e4, -1e4, -1e4], [0.0] * V])
    drafter = np.array([[-1e4, -1e4, -1e4, 3.0, 3.0, 3.0]])
    for u0 in (0.0, 0.5, 0.999):
        for us in (0.1, 0.5, 0.9):
            n, tok = speculative_sample(target, drafter, np.array([4]), np.array([u0, us]), 1.0)
            assert n == 0 and tok == draw(softmax64(target[0], 1.0), us) and tok < 3


@pytest.mark.parametrize("seed", [3, 4])
def test_first_token_is_distributed_as_p(seed):
    """Draft token x ~ q_0; over 40000 draws the emitted first token has the frequencies of
    p_0 (each within 4.5 standard deviations)."""
    rng = np.random.default_rng(seed)
    V, T, n = 6, 0.9, 40000
    target = rng.standard_normal((2, V)) * 1.5
    drafter = rng.standard_normal((1, V)) * 1.5
    p0, q0 = softmax64(target[0], T), softmax64(drafter[0], T)
    counts = np.zeros(V)
    xs = rng.choice(V, size=n, p=q0)
    us = rng.random((n, 2))
    for k in range(n):
        nacc, tok = speculative_sample(target, drafter, xs[k:k + 1], us[k], T)
        first = int(xs[k]) if nacc >= 1 else tok
        counts[first] += 1
    sd = np.sqrt(n * p0 * (1 - p0))
    assert (np.abs(counts - n * p0) <= 4.5 * sd + 1).all(), (counts / n, p0)


def test_point_mass_drafter_equals_explicit_one_hot():
    """No draft logits means q is the point mass at the draft token: the same results as
    draft logits that put (numerically) all mass there."""
    rng = np.random.default_rng(5)
    M, V = 6, 9
    for _ in range(200):
        lg = rng.standard_normal((M, V)) * 2
        draft = rng.integers(0, V, M - 1)
        one_hot = np.full((M - 1, V), -1e6)
        one_hot[np.arange(M - 1), draft] = 0.0
        u = rng.random(M)
        assert speculative_sample(lg, None, draft, u, 0.7) == speculative_sample(lg, one_hot, draft, u, 0.7)


def test_point_mass_drafter_accepts_with_probability_p():
    """With a deterministic drafter, draft x is accepted iff u < p(x), and after a rejection
    the emitted token is drawn from p with x removed."""
    lg = np.array([[1.0, 2.0, 0.5, -1.0], [0.0, 0.0, 0.0, 0.0]])
    p = softmax64(lg[0], 1.0)
    for u0 in np.linspace(0.0, 0.99, 23):
        n, tok = speculative_sample(lg, None, np.array([1]), np.array([u0, 0.3]), 1.0)
        assert n == (1 if u0 < p[1] else 0)
        if n == 0:
            w = p.copy()
            w[1] = 0.0
            assert tok == draw(w, 0.3) and tok != 1


def test_out_of_range_draft_is_rejected():
    lg = np.zeros((3, 5))
    for bad in (-1, 5, 1 << 20):
        n, tok = speculative_sample(lg, None, np.array([bad, 0]), np.array([0.0, 0.0, 0.5]), 1.0)
        assert n == 0 and tok == 2          # residual is p itself: uniform over 5, u = 0.5
        n, _ = speculative_sample(lg, lg[:2], np.array([bad, 0]), np.array([0.0, 0.0, 0.5]), 1.0)
        assert n == 0


def test_low_temperature_reduces_to_greedy_verification():
    """As T -> 0, p and q become point masses at their argmax, and a draft drawn from q is
    the drafter's argmax: the accepted count is the greedy chain rule and the emitted token
    is the target's argmax at the stopping row."""
    from oracle import accept, argmax
    rng = np.random.default_rng(6)
    M, V = 8, 50
    for trial in range(100):
        lg = rng.permuted(np.tile(np.arange(V, dtype=np.float64), (M, 1)), axis=1)  # distinct
        am = argmax(lg.astype(np.float16))
        draft = am[:M - 1].copy()
        k = trial % M
        if k < M - 1:
            draft[k] = (draft[k] + 1 + trial) % V
        dl = lg[:M - 1] + rng.uniform(-0.1, 0.1, (M - 1, V))
        dl[np.arange(M - 1), draft] = V + 1.0     # the drafter's argmax is its draft
        u = rng.random(M) * 0.999
        for d in (None, dl):
            n, tok = speculative_sample(lg, d, draft, u, 0.02)
            assert n == accept(draft.astype(np.int32), am)
            assert tok == am[n]


def test_acceptance_rate_and_residual_on_a_grid():
    """One draft, V = 4: over a fine grid of u the acceptance fraction is min(1, p(x)/q(x))
    and, after rejection, the token frequencies are max(0, p - q) normalised (to within the
    grid spacing)."""
    rng = np.random.default_rng(7)
    target = rng.standard_normal((2, 4)) * 1.3
    drafter = rng.standard_normal((1, 4)) * 1.3
    p, q = softmax64(target[0], 1.0), softmax64(drafter[0], 1.0)
    G = 2000
    grid = (np.arange(G) + 0.5) / G
    for x in range(4):
        acc = sum(speculative_sample(target, drafter, np.array([x]), np.array([g, 0.5]), 1.0)[0]
                  for g in grid) / G
        assert abs(acc - min(1.0, p[x] / q[x])) <= 1.0 / G
    x = int(np.argmax(q / p))                  # the draft most likely to be rejected
    r = np.maximum(p - q, 0)
    freq = np.zeros(4)
    for g in grid:
        n, tok = speculative_sample(target, drafter, np.array([x]), np.array([0.9999999, g]), 1.0)
        assert n == 0
        freq[tok] += 1.0 / G
    assert np.abs(freq - r / r.sum()).max() <= 1.0 / G + 1e-12


def test_margins_cover_each_decision():
    rng = np.random.default_rng(8)
    M, V = 5, 30
    lg = rng.standard_normal((M, V))
    draft = rng.integers(0, V, M - 1)
    u = rng.random(M)
    n, _ = speculative_sample(lg, lg[:M - 1] * 0.9, draft, u, 0.8)
    gaps = decision_margins(lg, lg[:M - 1] * 0.9, draft, u, 0.8)
    assert len(gaps) == (n + 1 if n < M - 1 else M - 1) + 1 and min(gaps) > 0
