"""Checks that pin the verify step to what the pages and the mathematics fix.

Each check takes a *sampler* or an *attention* callable, so the same check runs
on the CPU oracle, on deliberately mutated oracle builds (which must fail it),
and on the GPU library.

Sampler callable: f(target_logits [B,K+1,V] f32, draft_logits [B,K,V] f32 | None,
draft_tokens [B,K] i32, u_accept [B,K] f32, u_sample [B] f32, temperature,
top_p, greedy) -> dict with "n_accepted" [B] and "out_tokens" [B,K+1].

Sources:
  * Theorem 1 of "Accelerating Large Language Model Decoding with Speculative
    Sampling" (appendix proof): the emitted token is distributed exactly as the
    target distribution q, and P(accept) = sum_x min(p(x), q(x)).
  * Same paper, "Modified rejection sampling": at least one token per round,
    at most K+1 (bonus token when all drafts are accepted); accept probability
    min(1, q/p) equals 1 when p = q; temperature / nucleus modify both
    distributions before the scheme.
"""
from __future__ import annotations

import numpy as np
from scipy import special, stats

ALPHA = 1e-4          # significance level of every statistical check
N_TRIALS = 1_000_000  # trials per statistical case


class Case:
    """A fixed (target rows, draft rows) pair with its modified distributions.

    ``q_mod``/``p_mod`` are the distributions the scheme must use after
    temperature and nucleus, derived by hand from the construction (not by
    re-running the method's code).
    """

    def __init__(self, name, zt, zd, q_mod, p_mod, temperature=1.0, top_p=1.0, top_k=0):
        self.name = name
        self.zt = np.asarray(zt, np.float32)   # [K+1, V]
        self.zd = np.asarray(zd, np.float32)   # [K, V]
        self.q_mod = np.asarray(q_mod, np.float64)  # [K+1, V]
        self.p_mod = np.asarray(p_mod, np.float64)  # [K, V]
        self.temperature = temperature
        self.top_p = top_p
        self.top_k = top_k

    @property
    def K(self):
        return self.zd.shape[0]

    @property
    def V(self):
        return self.zt.shape[1]

    def alpha(self):
        """Acceptance probability per position: sum_x min(p'(x), q'(x))."""
        return np.minimum(self.p_mod, self.q_mod[: self.K]).sum(axis=1)


def _softmax_rows(z):
    return special.softmax(np.asarray(z, np.float64), axis=-1)


def make_cases():
    rng = np.random.default_rng(20240424)
    cases = []
    # V=2, explicit probabilities.
    q = np.array([[0.6, 0.4], [0.25, 0.75]])
    p = np.array([[0.3, 0.7]])
    zt, zd = np.log(q).astype(np.float32), np.log(p).astype(np.float32)
    cases.append(Case("v2", zt, zd, _softmax_rows(zt), _softmax_rows(zd)))
    # V=4 and V=8 Dirichlet pairs, K=2, T=1, no nucleus.
    for V in (4, 8):
        q = rng.dirichlet(np.ones(V) * 2.0, size=3)
        p = rng.dirichlet(np.ones(V) * 2.0, size=2)
        zt, zd = np.log(q).astype(np.float32), np.log(p).astype(np.float32)
        cases.append(Case(f"dirichlet_v{V}", zt, zd, _softmax_rows(zt), _softmax_rows(zd)))
    # Temperature 0.5 on logits log(prob): exp(log(prob)/0.5) = prob^2, so the
    # tempered distribution is prob^2 / sum(prob^2).
    q = np.array([[0.4, 0.3, 0.2, 0.1], [0.1, 0.2, 0.3, 0.4]])
    p = np.array([[0.25, 0.25, 0.25, 0.25]])
    zt, zd = np.log(q).astype(np.float32), np.log(p).astype(np.float32)
    sq = _softmax_rows(zt) ** 2
    sp = _softmax_rows(zd) ** 2
    cases.append(Case("temp_half", zt, zd, sq / sq.sum(1, keepdims=True),
                      sp / sp.sum(1, keepdims=True), temperature=0.5))
    # Nucleus 0.79 on hand-picked rows.
    #   target [0.5, 0.3, 0.15, 0.05]: mass(>=0.5)=0.5 < 0.79, mass(>=0.3)=0.8 -> keep {0,1}
    #       q' = [0.625, 0.375, 0, 0]
    #   draft  [0.1, 0.6, 0.2, 0.1]:  mass(>=0.6)=0.6, mass(>=0.2)=0.8 -> keep {1,2}
    #       p' = [0, 0.75, 0.25, 0]
    #   bonus row [0.2, 0.2, 0.2, 0.4]: mass(>=0.4)=0.4, mass(>=0.2)=1.0 -> keep all
    #       (tie-closed: the three 0.2 tokens enter together)
    zt = np.log(np.array([[0.5, 0.3, 0.15, 0.05], [0.2, 0.2, 0.2, 0.4]])).astype(np.float32)
    zd = np.log(np.array([[0.1, 0.6, 0.2, 0.1]])).astype(np.float32)
    cases.append(Case("nucleus", zt, zd,
                      [[0.625, 0.375, 0.0, 0.0], [0.2, 0.2, 0.2, 0.4]],
                      [[0.0, 0.75, 0.25, 0.0]], top_p=0.79))
    # Top-k 2 ("Accelerating ... Speculative Sampling" names top-k among the
    # standard modifications), tie-closed at the k-th value:
    #   target [0.4, 0.3, 0.2, 0.1] -> keep {0,1}: q' = [4/7, 3/7, 0, 0]
    #   draft  [0.1, 0.5, 0.25, 0.15] -> keep {1,2}: p' = [0, 2/3, 1/3, 0]
    #   bonus  [0.25, 0.25, 0.3, 0.2]: the 2nd largest value 0.25 is a tie
    #       group of two -> keep {0,1,2}: q' = [0.25, 0.25, 0.3, 0] / 0.8
    zt = np.log(np.array([[0.4, 0.3, 0.2, 0.1], [0.25, 0.25, 0.3, 0.2]])).astype(np.float32)
    zd = np.log(np.array([[0.1, 0.5, 0.25, 0.15]])).astype(np.float32)
    cases.append(Case("topk2", zt, zd, [[4 / 7, 3 / 7, 0.0, 0.0], [0.3125, 0.3125, 0.375, 0.0]],
                      [[0.0, 2 / 3, 1 / 3, 0.0]], top_k=2))
    # Top-k 2, then nucleus 0.9 on the renormalised top set:
    #   target [0.5, 0.3, 0.15, 0.05] -> top-2 [0.625, 0.375] -> 0.625 < 0.9,
    #       1.0 >= 0.9: q' = [0.625, 0.375, 0, 0]   (nucleus alone keeps {0,1,2})
    #   draft  [0.1, 0.6, 0.2, 0.1] -> top-2 [0.75, 0.25] -> p' = [0, 0.75, 0.25, 0]
    #   bonus  [0.2, 0.2, 0.2, 0.4] -> the 0.2 tie group enters whole: all kept,
    #       and the nucleus needs all of them: q' = [0.2, 0.2, 0.2, 0.4]
    zt = np.log(np.array([[0.5, 0.3, 0.15, 0.05], [0.2, 0.2, 0.2, 0.4]])).astype(np.float32)
    zd = np.log(np.array([[0.1, 0.6, 0.2, 0.1]])).astype(np.float32)
    cases.append(Case("topk2_nucleus", zt, zd, [[0.625, 0.375, 0.0, 0.0], [0.2, 0.2, 0.2, 0.4]],
                      [[0.0, 0.75, 0.25, 0.0]], top_p=0.9, top_k=2))
    # Disjoint supports: logit -1e4 has exp(-1e4) == 0 in double.
    zt = np.array([[0.0, 0.0, -1e4, -1e4], [0.0, -1e4, -1e4, 0.0]], np.float32)
    zd = np.array([[-1e4, -1e4, 0.0, 0.0]], np.float32)
    cases.append(Case("disjoint", zt, zd, [[0.5, 0.5, 0, 0], [0.5, 0, 0, 0.5]],
                      [[0, 0, 0.5, 0.5]]))
    return cases


def make_trials(case: Case, n=N_TRIALS, seed=0):
    """Inputs of ``n`` independent verify rounds on the fixed rows of ``case``:
    each trial draws its own draft tokens x_j ~ p'_j and its own uniforms."""
    rng = np.random.default_rng(seed)
    K, V = case.K, case.V
    zt = np.ascontiguousarray(np.broadcast_to(case.zt, (n, K + 1, V)))
    zd = np.ascontiguousarray(np.broadcast_to(case.zd, (n, K, V)))
    tok = np.empty((n, K), np.int32)
    for j in range(K):
        tok[:, j] = rng.choice(V, size=n, p=case.p_mod[j] / case.p_mod[j].sum())
    ua = (rng.integers(0, 2 ** 24, size=(n, K)) * 2.0 ** -24).astype(np.float32)
    us = (rng.integers(0, 2 ** 24, size=n) * 2.0 ** -24).astype(np.float32)
    return zt, zd, tok, ua, us


def run_case(sampler, case: Case, n=N_TRIALS, seed=0):
    """Run ``n`` independent verify rounds of ``case`` through ``sampler``."""
    zt, zd, tok, ua, us = make_trials(case, n, seed)
    res = sampler(zt, zd, tok, ua, us, case.temperature, case.top_p, False, top_k=case.top_k)
    return tok, res


def chi2_pvalue(counts, probs):
    """Chi-square goodness of fit; categories of zero probability must be empty."""
    counts = np.asarray(counts, np.float64)
    probs = np.asarray(probs, np.float64)
    if counts[probs == 0].sum() > 0:
        return 0.0
    m = probs > 0
    if m.sum() < 2:
        return 1.0
    exp = probs[m] / probs[m].sum() * counts.sum()
    return float(stats.chisquare(counts[m], exp).pvalue)


def theorem1_pvalues(sampler, case: Case, n=N_TRIALS, seed=0):
    """Emitted token at position j, given the round reached j, is ~ q'_j.

    Returns (list of chi-square p-values for j = 0..K, result dict, tokens).
    """
    tok, res = run_case(sampler, case, n, seed)
    nacc, out = res["n_accepted"], res["out_tokens"]
    pv = []
    for j in range(case.K + 1):
        reached = nacc >= j
        if reached.sum() < 1000:
            continue
        counts = np.bincount(out[reached, j], minlength=case.V)
        pv.append(chi2_pvalue(counts, case.q_mod[j]))
    return pv, res, tok


def accept_rate_z(res, case: Case):
    """z-scores of the observed acceptance rate at each reached position vs
    sum_x min(p'(x), q'(x))."""
    nacc = res["n_accepted"]
    a = case.alpha()
    zs = []
    for j in range(case.K):
        reached = nacc >= j
        m = int(reached.sum())
        if m < 1000:
            continue
        k = int((nacc[reached] > j).sum())
        var = m * a[j] * (1 - a[j])
        zs.append(0.0 if var == 0 and k == m * a[j] else
                  (k - m * a[j]) / np.sqrt(var) if var > 0 else np.inf)
    return zs


def scan_length_pvalue(res, case: Case):
    """n_b distribution from the stopping rule: P(n >= k) = prod_{j<k} alpha_j."""
    a = case.alpha()
    K = case.K
    surv = np.concatenate([[1.0], np.cumprod(a)])  # P(n >= k), k = 0..K
    pk = np.empty(K + 1)
    pk[:K] = surv[:K] - surv[1:K + 1]
    pk[K] = surv[K]
    counts = np.bincount(res["n_accepted"], minlength=K + 1)
    return chi2_pvalue(counts, pk)


def check_counts(res, draft_tokens, K, V):
    """1 <= e_b <= K+1; accepted prefix equals the drafts; valid ids; -1 padding."""
    n, out = res["n_accepted"], res["out_tokens"]
    assert np.all((n >= 0) & (n <= K))
    B = n.shape[0]
    for b in range(B):
        e = int(n[b]) + 1
        assert 1 <= e <= K + 1
        assert np.array_equal(out[b, : n[b]], draft_tokens[b, : n[b]])
        assert 0 <= out[b, n[b]] < V
        assert np.all(out[b, e:] == -1)


# ---------------------------------------------------------------- fixed-value draw cases

def load_draw_cases(golden_dir):
    """Hand-derived verify rounds (tests/golden/draw_zero_weight_cases.json)
    whose emitted token is fixed by the inverse-CDF convention: ids of zero
    weight are never drawn, even at u = 0."""
    import json
    import os
    with open(os.path.join(golden_dir, "draw_zero_weight_cases.json")) as f:
        gold = json.load(f)
    out = []
    for c in gold["cases"]:
        zt = np.asarray(c["target_logits"], np.float32)
        K = zt.shape[0] - 1
        V = zt.shape[1]
        zd = np.asarray(c["draft_logits"], np.float32).reshape(K, V)
        out.append(dict(name=c["name"], zt=zt[None], zd=zd[None],
                        tok=np.asarray(c["draft_tokens"], np.int32).reshape(1, K),
                        ua=np.asarray(c["u_accept"], np.float32).reshape(1, K),
                        us=np.asarray([c["u_sample"]], np.float32),
                        T=c["temperature"], top_p=c["top_p"],
                        n=c["n_accepted"], out=np.asarray(c["out_tokens"], np.int32)))
    return out


def check_draw_cases(sampler, golden_dir):
    """Every case's n_accepted and out_tokens equal the hand-derived values."""
    for c in load_draw_cases(golden_dir):
        res = sampler(c["zt"], c["zd"], c["tok"], c["ua"], c["us"], c["T"], c["top_p"], False)
        assert int(res["n_accepted"][0]) == c["n"], (c["name"], res["n_accepted"])
        assert np.array_equal(np.asarray(res["out_tokens"][0]), c["out"]), \
            (c["name"], res["out_tokens"][0], c["out"])
