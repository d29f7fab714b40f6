"""Exact-rational enumeration of one speculative round's output distribution.

Pins the *reading* of the verification rules (token-level: "The rule that
makes it exact" on the speculative-decoding explainer; block-level: "Block
verification" on the luminal page) independently of the C oracle: for tiny
vocabularies and draft lengths it enumerates every draft sequence and every
verification outcome with Python ``fractions`` and returns the exact
distribution of the emitted tokens.  Tests then check that this distribution,
completed with target draws, equals the target's own joint distribution.

Tables are callables ``p(prefix) -> list[Fraction]`` (target conditional) and
``q(prefix) -> list[Fraction]`` (draft conditional), ``prefix`` a tuple.
"""
from __future__ import annotations

import itertools
from collections import defaultdict
from fractions import Fraction as F


def target_joint(p, length, V):
    """P_target(s) for every token sequence s of the given length."""
    out = {}
    for seq in itertools.product(range(V), repeat=length):
        pr = F(1)
        for i in range(length):
            pr *= p(seq[:i])[seq[i]]
        out[seq] = pr
    return out


def complete_with_target(dist, p, length, V):
    """Extends every emitted sequence to `length` tokens by target draws."""
    out = defaultdict(F)
    for s, pr in dist.items():
        for cont in itertools.product(range(V), repeat=length - len(s)):
            full = s + cont
            c = pr
            for i in range(len(s), length):
                c *= p(full[:i])[full[i]]
            if c:
                out[full] += c
    return dict(out)


def _draft_sequences(q, L, V):
    for xs in itertools.product(range(V), repeat=L):
        pq = F(1)
        for i in range(L):
            pq *= q(xs[:i])[xs[i]]
        if pq:
            yield xs, pq


def _normalise(weights):
    Z = sum(weights)
    return [w / Z for w in weights]


def token_round(p, q, L, V):
    """Exact output distribution of token-level verification over L drafts.

    Accept x_i with probability min(1, p/q); on the first rejection emit a
    draw from max(p - q, 0) normalised; if all pass, emit a draw from p."""
    out = defaultdict(F)
    expected_accepted = F(0)
    for xs, pq in _draft_sequences(q, L, V):
        alive = F(1)
        for i in range(L):
            pi = p(xs[:i])[xs[i]]
            qi = q(xs[:i])[xs[i]]
            a = min(F(1), pi / qi)
            rej = alive * (1 - a)
            if rej:
                pn, qn = p(xs[:i]), q(xs[:i])
                r = _normalise([max(pn[v] - qn[v], F(0)) for v in range(V)])
                for y in range(V):
                    if r[y]:
                        out[xs[:i] + (y,)] += pq * rej * r[y]
            expected_accepted += pq * rej * i
            alive *= a
        if alive:
            pn = p(xs)
            for y in range(V):
                if pn[y]:
                    out[xs + (y,)] += pq * alive * pn[y]
            expected_accepted += pq * alive * L
    return dict(out), expected_accepted


def block_round(p, q, L, V, degenerate_h=F(1)):
    """Exact output distribution of block verification over L drafts.

    Running ratio w_i = min(1, w_{i-1} p/q), w_0 = 1; thresholds
    h_i = m_i / (m_i + 1 - w_i) with m_i = sum_v max(w_i p_{i+1} - q_{i+1}, 0)
    for i < L and h_L = w_L; independent uniforms, tau = the largest passing i
    (else 0); correction from max(w_tau p_{tau+1} - q_{tau+1}, 0) or, for
    tau = L, the bonus from p_{L+1}."""
    out = defaultdict(F)
    expected_accepted = F(0)
    for xs, pq in _draft_sequences(q, L, V):
        w = [F(1)]
        for i in range(1, L + 1):
            pi, qi = p(xs[:i - 1])[xs[i - 1]], q(xs[:i - 1])[xs[i - 1]]
            w.append(min(F(1), w[-1] * pi / qi))
        h = [None] * (L + 1)
        for i in range(1, L):
            pn, qn = p(xs[:i]), q(xs[:i])
            m = sum(max(w[i] * pn[v] - qn[v], F(0)) for v in range(V))
            den = m + 1 - w[i]
            h[i] = m / den if den != 0 else degenerate_h
        if L >= 1:
            h[L] = w[L]
        for tau in range(0, L + 1):
            pt = F(1) if tau == 0 else h[tau]
            for j in range(tau + 1, L + 1):
                pt *= (1 - h[j])
            if not pt:
                continue
            pre = xs[:tau]
            pn, qn = p(pre), q(pre)
            if tau == L:
                r = list(pn)
            else:
                r = [max(w[tau] * pn[v] - qn[v], F(0)) for v in range(V)]
                if sum(r) == 0:
                    r = list(pn)
            r = _normalise(r)
            for y in range(V):
                if r[y]:
                    out[pre + (y,)] += pq * pt * r[y]
            expected_accepted += pq * pt * tau
    return dict(out), expected_accepted


def random_tables(rng, V, L, zero_prob=0.25, same_prob=0.0, context_free=False):
    """Random rational conditional tables for all prefixes up to length L.

    zero_prob: chance that an entry is 0 (disjoint supports arise);
    same_prob: chance that q equals p for a prefix (exercises degenerate
    thresholds)."""
    ptab, qtab = {}, {}

    def dist(zp):
        while True:
            w = [0 if rng.random() < zp else rng.randint(1, 7) for _ in range(V)]
            if sum(w):
                s = sum(w)
                return [F(x, s) for x in w]

    prefixes = [()] if context_free else [
        pre for n in range(L + 1) for pre in itertools.product(range(V), repeat=n)]
    for pre in prefixes:
        ptab[pre] = dist(zero_prob)
        qtab[pre] = list(ptab[pre]) if rng.random() < same_prob else dist(zero_prob)
    if context_free:
        return (lambda pre: ptab[()]), (lambda pre: qtab[()])
    return (lambda pre: ptab[pre]), (lambda pre: qtab[pre])


def tree_children(parents):
    """Children of every node (node 0 = root) in index order."""
    N = len(parents)
    ch = [[] for _ in range(N + 1)]
    for m in range(1, N + 1):
        ch[parents[m - 1]].append(m)
    return ch


def tree_round(p, q, parents, V):
    """Exact output distribution of tree verification (recursive rejection).

    The tree's children of a node are drawn independently from q(prefix of
    the node); at a node with residual r (initially p), each child's token x
    is accepted with probability min(1, r(x)/q(x)), continuing at that child;
    a rejection replaces r by max(r - q, 0) normalised; when every child is
    rejected the emitted token is drawn from r; at a leaf from p."""
    N = len(parents)
    ch = tree_children(parents)
    out = defaultdict(F)
    expected_accepted = F(0)
    for xs in itertools.product(range(V), repeat=N):
        # prefix of each node and the probability of this draft tree
        pre = {0: ()}
        pq = F(1)
        for m in range(1, N + 1):
            par = parents[m - 1]
            pq *= q(pre[par])[xs[m - 1]]
            pre[m] = pre[par] + (xs[m - 1],)
        if not pq:
            continue

        def walk(node, prob, depth):
            nonlocal expected_accepted
            s = pre[node]
            if not ch[node]:
                pn = p(s)
                for y in range(V):
                    if pn[y]:
                        out[s + (y,)] += pq * prob * pn[y]
                expected_accepted += pq * prob * depth
                return
            r = list(p(s))
            qn = q(s)
            alive = prob
            for c in ch[node]:
                x = xs[c - 1]
                a = F(1) if qn[x] == 0 else min(F(1), r[x] / qn[x])
                if a:
                    walk(c, alive * a, depth + 1)
                alive *= (1 - a)
                if not alive:
                    return
                resid = [max(r[v] - qn[v], F(0)) for v in range(V)]
                r = _normalise(resid) if sum(resid) else list(p(s))
            for y in range(V):
                if r[y]:
                    out[s + (y,)] += pq * alive * r[y]
            expected_accepted += pq * alive * depth

        walk(0, F(1), 0)
    return dict(out), expected_accepted
