"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test names what it pins and where that fact comes from:
  * exact-rational enumeration of the rules (losslessness: the round's output,
    completed with target draws, is distributed exactly as the target);
  * the target's own joint distribution, against which the oracle's Monte
    Carlo output is tested (chi-square) -- a dropped term, a wrong sign or a
    wrong row in the correction breaks it;
  * values the pages print (worked examples under tests/golden/);
  * closed forms, special cases and library routines (numpy searchsorted,
    scipy logsumexp, rocRAND's Philox engine, brute force).
"""
import itertools
import json
import math
import os
import random
import shutil
import subprocess
import tempfile
from fractions import Fraction as F

import numpy as np
import pytest
from scipy import special, stats

import exact_enum

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _log(prob):
    prob = np.asarray(prob, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(prob)


# ---------------------------------------------------------------- Philox ----

def test_philox_matches_rocrand_engine(orc):
    """Pins orc_philox4x32_10 / orc_uniform to rocRAND's Philox4x32-10 engine,
    an independent implementation of the SC'11 generator.  rocRAND's
    (seed, subsequence, 4*block) addresses counter (block lo, block hi,
    subsequence lo, subsequence hi) under key (seed lo, seed hi)."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND probe")
    src = os.path.join(os.path.dirname(__file__), "philox_rocrand_probe.cpp")
    rng = np.random.default_rng(7)
    cases = [(0, 0, 0), (1, 0, 0), (2**64 - 1, 2**64 - 1, 2**62 - 1)]
    for _ in range(200):
        cases.append((int(rng.integers(0, 2**63)), int(rng.integers(0, 2**63)),
                      int(rng.integers(0, 2**40))))
    with tempfile.TemporaryDirectory() as td:
        exe = os.path.join(td, "probe")
        subprocess.run([hipcc, "-O1", "--offload-arch=gfx950", src, "-o", exe], check=True,
                       capture_output=True)
        inp = "".join(f"{s} {sub} {blk}\n" for s, sub, blk in cases)
        res = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True)
    lines = res.stdout.strip().splitlines()
    assert len(lines) == len(cases)
    for (seed, sub, blk), line in zip(cases, lines):
        want = [int(t) for t in line.split()]
        ctr = [blk & 0xFFFFFFFF, blk >> 32, sub & 0xFFFFFFFF, sub >> 32]
        key = [seed & 0xFFFFFFFF, seed >> 32]
        got = orc.philox4x32_10(ctr, key).tolist()
        assert got == want, (seed, sub, blk)
    # the uniform is word 0's top 24 bits: check the counter layout end to end
    seed, req, pos, tag, off = 12345, 17, 3, 1, 2**33 + 5
    blk = req + (((pos & 0xFFFF) | (tag << 16)) << 32)
    w0 = orc.philox4x32_10([blk & 0xFFFFFFFF, blk >> 32, off & 0xFFFFFFFF, off >> 32],
                           [seed & 0xFFFFFFFF, seed >> 32])[0]
    assert orc.uniform(seed, off, req, pos, tag) == (int(w0) >> 8) / 2**24


def test_uniforms_chi_square(orc):
    """Uniformity of the 24-bit uniforms over 2e4 counters (64 bins)."""
    u = np.array([orc.uniform(1, 0, r, p, 0) for r in range(2000) for p in range(10)])
    assert u.min() >= 0.0 and u.max() <= 1.0 - 2**-24
    counts, _ = np.histogram(u, bins=64, range=(0, 1))
    chi2 = ((counts - len(u) / 64) ** 2 / (len(u) / 64)).sum()
    assert chi2 < stats.chi2.ppf(1 - 1e-6, 63)


# ------------------------------------------------------ row normaliser -----

def test_row_lse_closed_forms_and_library(orc):
    V = 1000
    lse, fl = orc.row_lse(np.full(V, 2.5), temperature=0.5)
    assert fl == 0 and abs(lse - (5.0 + math.log(V))) < 1e-12
    row = np.full(V, -np.inf)
    row[123] = 4.0
    lse, fl = orc.row_lse(row)
    assert fl == 0 and lse == 4.0
    rng = np.random.default_rng(0)
    for T in (1.0, 0.7, 2.0):
        x = rng.normal(0, 3, 5000).astype(np.float32).astype(np.float64)
        lse, _ = orc.row_lse(x, temperature=T)
        assert abs(lse - special.logsumexp(x / np.float64(np.float32(T)))) < 1e-10
    assert orc.row_lse(np.full(10, -np.inf))[1] == orc.FLAG_BAD_ROW
    bad = np.zeros(10)
    bad[3] = np.nan
    assert orc.row_lse(bad)[1] == orc.FLAG_BAD_ROW
    bad[3] = np.inf
    assert orc.row_lse(bad)[1] == orc.FLAG_BAD_ROW


# ---------------------------------------------------------- inverse CDF ----

def test_icdf_equals_searchsorted(orc):
    """Special case reducing to a library routine: the inverse-CDF draw equals
    numpy.searchsorted(cumsum(w), u*Z, side='right') (zero weights never win)."""
    rng = np.random.default_rng(1)
    for trial in range(300):
        V = int(rng.integers(1, 50))
        w = rng.random(V) * (rng.random(V) > 0.3)
        if w.sum() == 0:
            w[int(rng.integers(0, V))] = 0.5
        u = np.float32(rng.random()).item() if trial % 5 else 0.0
        y, Z, _ = orc.icdf(w, u)
        c = np.cumsum(w)
        t = u * c[-1]
        want = int(np.searchsorted(c, t, side="right"))
        gap = np.min(np.abs(c - t)) / c[-1]     # this test's own distance to a CDF step
        if gap > 1e-6:                 # away from a float tie the two must agree
            assert y == want, (trial, y, want)
        assert w[y] > 0
    assert orc.icdf(np.zeros(5), 0.3)[0] == -1
    # u at its largest value still returns the last positive-weight token
    w = np.array([0.2, 0.0, 0.3, 0.0])
    assert orc.icdf(w, 1.0 - 2**-24)[0] == 2


# ------------------------------------------------- exact enumeration -------

@pytest.mark.parametrize("seed", range(4))
def test_exact_enumeration_token_and_block_are_lossless(seed):
    """Reading pin: over random rational target/draft tables (context-dependent
    and context-free, V <= 3, L <= 3, with zero entries), the enumerated round
    output completed by target draws equals the target's joint distribution,
    for token verification and for the block completion; and block keeps at
    least as many draft tokens in expectation."""
    rng = random.Random(100 + seed)
    for trial in range(12):
        V = rng.randint(2, 3)
        L = rng.randint(1, 3 if V == 2 else 2)
        p, q = exact_enum.random_tables(rng, V, L, zero_prob=0.25, same_prob=0.3,
                                        context_free=(trial % 3 == 0))
        tj = exact_enum.target_joint(p, L + 1, V)
        dt, et = exact_enum.token_round(p, q, L, V)
        db, eb = exact_enum.block_round(p, q, L, V)
        assert exact_enum.complete_with_target(dt, p, L + 1, V) == {k: v for k, v in tj.items() if v}
        assert exact_enum.complete_with_target(db, p, L + 1, V) == {k: v for k, v in tj.items() if v}
        assert eb >= et


def test_exact_enumeration_block_toy_example():
    """Pin against the printed toy example (luminal page, "Block verification")."""
    g = _golden("block_toy_example.json")
    pr = g["printed"]
    p = [F(pr["p"]["A"]), F(pr["p"]["B"])]
    q = [F(pr["q"]["A"]), F(pr["q"]["B"])]
    assert p[0] / q[0] == F(pr["ratio_A"]) and p[1] / q[1] == F(pr["ratio_B"])
    assert p[0] * p[1] == F(pr["P_AB_under_p"]) and q[0] * q[1] == F(pr["P_AB_under_q"])
    P = lambda pre: p
    Q = lambda pre: q
    d = g["derived_exact"]

    def parse(m):
        return {tuple(int(t) for t in k.split(",")): F(v) for k, v in m.items()}

    for name, prop, fn in (("block_AB", (0, 1), exact_enum.block_round),
                           ("block_BA", (1, 0), exact_enum.block_round),
                           ("token_AB", (0, 1), exact_enum.token_round)):
        out = _round_given_proposal(fn, P, Q, prop)
        assert out == parse(d[name]), name


def _round_given_proposal(fn, P, Q, prop):
    """Outputs of one round conditioned on the draft being `prop` (exact)."""
    import exact_enum as ee
    orig = ee._draft_sequences
    try:
        ee._draft_sequences = lambda q, L, V: iter([(prop, F(1))])
        dist, _ = fn(P, Q, len(prop), 2)
    finally:
        ee._draft_sequences = orig
    return dist


# ---------------------------------------- oracle vs printed toy example ----

def test_oracle_block_toy_example_forced_uniforms(orc):
    g = _golden("block_toy_example.json")
    pA, pB = float(F(g["printed"]["p"]["A"])), float(F(g["printed"]["p"]["B"]))
    qA, qB = float(F(g["printed"]["q"]["A"])), float(F(g["printed"]["q"]["B"]))
    p = _log([[[pA, pB]] * 3])
    q = _log([[[qA, qB]] * 2])
    # AB: w = 1/2 then 1; h_1 = 0, h_2 = 1  -> tau = 2 whatever the uniforms
    for u in ([0.99, 0.99, 0.1], [0.0, 0.0, 0.9]):
        r = orc.block_verify(p, q, [[0, 1]], 2, uniforms=[u])
        assert r.accepted_len[0] == 2
        assert np.allclose(r.w[0], [0.5, 1.0]) and np.allclose(r.h[0], [0.0, 1.0])
        assert r.out_tokens[0, 2] == (0 if u[2] < pA else 1)
    # BA: w = 1 then 1/2; h_1 = 1, h_2 = 1/2
    r = orc.block_verify(p, q, [[1, 0]], 2, uniforms=[[0.3, 0.6, 0.2]])
    assert np.allclose(r.h[0], [1.0, 0.5], atol=1e-12)
    assert r.accepted_len[0] == 1 and r.out_tokens[0].tolist() == [1, 1, -1]
    r = orc.block_verify(p, q, [[1, 0]], 2, uniforms=[[0.3, 0.4, 0.2]])
    assert r.accepted_len[0] == 2 and r.out_tokens[0].tolist() == [1, 0, 0]
    # token verify AB: A accepted iff u_1 < 1/2; rejection emits B
    r = orc.token_verify(p, q, [[0, 1]], 2, uniforms=[[0.6, 0.0, 0.5]])
    assert r.accepted_len[0] == 0 and r.out_tokens[0].tolist() == [1, -1, -1]
    r = orc.token_verify(p, q, [[0, 1]], 2, uniforms=[[0.4, 0.99, 0.5]])
    assert r.accepted_len[0] == 2


def test_oracle_block_toy_example_monte_carlo(orc):
    """Frequencies of the oracle's outputs on the toy example vs the exact values."""
    g = _golden("block_toy_example.json")["derived_exact"]
    N = 60000
    p = np.broadcast_to(_log([[1 / 3, 2 / 3]] * 3), (N, 3, 2))
    q = np.broadcast_to(_log([[2 / 3, 1 / 3]] * 2), (N, 2, 2))
    for name, prop, fn in (("block_AB", (0, 1), orc.block_verify),
                           ("block_BA", (1, 0), orc.block_verify),
                           ("token_AB", (0, 1), orc.token_verify)):
        r = fn(p, q, np.tile(prop, (N, 1)), 2, seed=99)
        outs = [tuple(int(t) for t in row[:a + 1]) for row, a in zip(r.out_tokens, r.accepted_len)]
        want = {tuple(int(t) for t in k.split(",")): float(F(v)) for k, v in g[name].items()}
        cnt = {k: outs.count(k) for k in set(outs)}
        assert set(cnt) <= set(want)
        for k, pr in want.items():
            sd = math.sqrt(N * pr * (1 - pr))
            assert abs(cnt.get(k, 0) - N * pr) < 5 * sd + 1, (name, k)


# ------------------------------- Monte Carlo against the target's joint ----

def _mc_round(orc, fn, p_tab, q_tab, V, L, N, seed, temperature=1.0):
    """Samples N drafts from the draft tables, verifies them with the oracle,
    completes every output to L+1 tokens with target draws, and returns the
    counts per (L+1)-sequence.  Tables are dicts prefix-tuple -> prob array.
    Logits handed to the oracle are log-probabilities times T, so that
    softmax(logit / T) is the table."""
    rng = np.random.default_rng(seed)
    drafts = np.zeros((N, L), np.int64)
    for n in range(N):
        pre = ()
        for i in range(L):
            x = rng.choice(V, p=q_tab[pre])
            drafts[n, i] = x
            pre = pre + (int(x),)
    p = np.zeros((N, L + 1, V))
    q = np.zeros((N, L, V))
    for n in range(N):
        pre = tuple(int(t) for t in drafts[n])
        for i in range(L + 1):
            p[n, i] = _log(p_tab[pre[:i]]) * temperature
        for i in range(L):
            q[n, i] = _log(q_tab[pre[:i]]) * temperature
    r = fn(p, q, drafts, L, temperature=temperature, seed=seed + 1)
    counts = {}
    for n in range(N):
        a = int(r.accepted_len[n])
        seq = tuple(int(t) for t in r.out_tokens[n, :a + 1])
        while len(seq) < L + 1:
            seq = seq + (int(rng.choice(V, p=p_tab[seq])),)
        counts[seq] = counts.get(seq, 0) + 1
    return counts, r


def _tables_from_enum(p, q, V, L):
    pt, qt = {}, {}
    for n in range(L + 1):
        for pre in itertools.product(range(V), repeat=n):
            pt[pre] = np.array([float(x) for x in p(pre)])
            qt[pre] = np.array([float(x) for x in q(pre)])
    return pt, qt


@pytest.mark.parametrize("method,table_seed", [("token", 5), ("block", 6), ("block", 210)])
def test_oracle_output_distribution_equals_target(orc, method, table_seed):
    """The oracle's sampled outputs, completed with target draws, pass a
    chi-square test against the target's exact joint distribution (context-
    dependent tables, V=3, L=2, and a temperature != 1).  Table seed 210 is
    one where the block correction's w_tau factor moves the output
    distribution by 0.06 in total variation, so that factor is pinned too."""
    rng = random.Random(table_seed)
    V, L, N = 3, 2, 30000
    p, q = exact_enum.random_tables(rng, V, L, zero_prob=0.15)
    pt, qt = _tables_from_enum(p, q, V, L)
    fn = orc.token_verify if method == "token" else orc.block_verify
    counts, _ = _mc_round(orc, fn, pt, qt, V, L, N, seed=11, temperature=0.7)
    tj = exact_enum.target_joint(p, L + 1, V)
    cells = [s for s in tj if tj[s] > 0]
    assert set(counts) <= set(cells)
    obs = np.array([counts.get(s, 0) for s in cells], dtype=float)
    exp = np.array([float(tj[s]) * N for s in cells])
    chi2 = ((obs - exp) ** 2 / exp).sum()
    assert chi2 < stats.chi2.ppf(1 - 1e-6, len(cells) - 1), chi2


def test_oracle_acceptance_equals_overlap_mass(orc):
    """The chance that position 1 passes equals sum_v min(p, q) (the accepted
    mass is where p and q overlap), and the residual mass the oracle reports
    equals 1 - sum_v min(p, q) (luminal page, "On Speculative Sampling")."""
    rng = np.random.default_rng(3)
    V, N = 6, 40000
    pp = rng.dirichlet(np.ones(V))
    qq = rng.dirichlet(np.ones(V))
    x = rng.choice(V, size=(N, 1), p=qq)
    p = np.broadcast_to(_log(np.stack([pp, pp])), (N, 2, V))
    q = np.broadcast_to(_log(qq[None]), (N, 1, V))
    r = orc.token_verify(p, q, x, 1, seed=4)
    overlap = np.minimum(pp, qq).sum()
    rate = (r.accepted_len == 1).mean()
    assert abs(rate - overlap) < 5 * math.sqrt(overlap * (1 - overlap) / N)
    rej = r.accepted_len == 0
    assert np.allclose(r.resid_mass[rej], 1.0 - overlap, atol=1e-12)
    # and the correction is distributed as max(p - q, 0) / Z
    res = np.maximum(pp - qq, 0) / (1 - overlap)
    ys = r.out_tokens[rej, 0]
    for v in range(V):
        f = (ys == v).mean()
        assert abs(f - res[v]) < 5 * math.sqrt(max(res[v] * (1 - res[v]), 1e-9) / rej.sum()) + 1e-9


def test_printed_acceptance_ratio(orc):
    """p(x)=0.007, q(x)=0.025 -> accepted about 28% of the time (luminal page)."""
    g = _golden("worked_examples.json")["acceptance_ratio"]
    V, N = 3, 50000
    pp = np.array([g["p_x"], 0.5, 0.5 - g["p_x"]])
    qq = np.array([g["q_x"], 0.4, 0.6 - g["q_x"]])
    p = np.broadcast_to(_log(np.stack([pp, pp])), (N, 2, V))
    q = np.broadcast_to(_log(qq[None]), (N, 1, V))
    r = orc.token_verify(p, q, np.zeros((N, 1), np.int32), 1, seed=8)
    assert abs(r.ratio[0, 0] - g["p_x"] / g["q_x"]) < 1e-12
    assert abs(r.ratio[0, 0] - g["printed_acceptance"]) < 5e-3
    rate = (r.accepted_len == 1).mean()
    assert abs(rate - 0.28) < 5 * math.sqrt(0.28 * 0.72 / N)


def test_printed_expected_words(orc):
    """E[words] = (1 - a^(g+1)) / (1 - a): a=0.8, g=4 gives the printed 3.36
    (explainer sections 5-6); the oracle's mean emitted length over 4e4 rounds
    with per-position overlap 0.8 matches within 4 sigma."""
    g = _golden("worked_examples.json")["expected_words"]
    a, gam = g["alpha"], g["gamma"]
    closed = (1 - a ** (gam + 1)) / (1 - a)
    assert abs(closed - g["printed_value"]) <= g["printed_rounding"]
    V, N = 4, 40000
    # context-free tables with sum_v min(p, q) = 0.8
    pp = np.array([0.5, 0.3, 0.2, 0.0])
    qq = np.array([0.3, 0.3, 0.2, 0.2])
    assert abs(np.minimum(pp, qq).sum() - a) < 1e-12
    rng = np.random.default_rng(12)
    x = rng.choice(V, size=(N, gam), p=qq)
    p = np.broadcast_to(_log(np.tile(pp, (gam + 1, 1))), (N, gam + 1, V))
    q = np.broadcast_to(_log(np.tile(qq, (gam, 1))), (N, gam, V))
    r = orc.token_verify(p, q, x, gam, seed=13)
    emitted = r.accepted_len + 1
    sd = emitted.std() / math.sqrt(N)
    assert abs(emitted.mean() - closed) < 4 * sd


# ------------------------------------------------------- special cases -----

def test_special_cases(orc):
    rng = np.random.default_rng(21)
    B, gam, V = 64, 5, 50
    logits = rng.normal(0, 2, (B, gam + 1, V))
    x = rng.integers(0, V, (B, gam))
    # p == q: every draft token passes; the bonus is drawn from p_{gamma+1}
    r = orc.token_verify(logits, logits[:, :gam], x, gam, seed=3)
    assert (r.accepted_len == gam).all()
    assert (r.out_tokens[:, :gam] == x).all()
    # disjoint supports: first token always rejected, correction inside p's support
    p = np.full((B, gam + 1, V), -np.inf)
    q = np.full((B, gam, V), -np.inf)
    p[:, :, : V // 2] = rng.normal(0, 1, (B, gam + 1, V // 2))
    q[:, :, V // 2:] = rng.normal(0, 1, (B, gam, V - V // 2))
    xq = rng.integers(V // 2, V, (B, gam))
    for fn in (orc.token_verify, orc.block_verify):
        r = fn(p, q, xq, gam, seed=4)
        assert (r.accepted_len == 0).all()
        assert (r.out_tokens[:, 0] < V // 2).all() and (r.out_tokens[:, 1:] == -1).all()
    # gamma = 0: plain inverse-CDF sampling of p_1 (searchsorted of the cumsum)
    p0 = rng.normal(0, 2, (B, 1, V))
    r = orc.token_verify(p0, None, None, 0, seed=5)
    for b in range(B):
        pr = np.exp(p0[b, 0] - special.logsumexp(p0[b, 0]))
        u = orc.uniform(5, 0, b, 0, 1)
        want = int(np.searchsorted(np.cumsum(pr), u * pr.sum(), side="right"))
        assert r.out_tokens[b, 0] == want


def test_block_with_one_position_equals_token(orc):
    """Block verification with L = 1 takes token verification's decisions."""
    rng = np.random.default_rng(31)
    B, gam, V = 200, 4, 40
    p = rng.normal(0, 2, (B, gam + 1, V))
    q = p[:, :gam] + rng.normal(0, 1, (B, gam, V))
    x = rng.integers(0, V, (B, gam))
    vl = np.ones(B, np.int32)
    a = orc.token_verify(p, q, x, gam, verify_len=vl, seed=2)
    b = orc.block_verify(p, q, x, gam, verify_len=vl, seed=2)
    assert (a.accepted_len == b.accepted_len).all()
    assert (a.out_tokens == b.out_tokens).all()


def test_block_never_keeps_fewer_in_expectation(orc):
    rng = np.random.default_rng(41)
    B, gam, V = 3000, 4, 8
    pp = rng.dirichlet(np.ones(V) * 0.7, size=(1, gam + 1))
    qq = rng.dirichlet(np.ones(V) * 0.7, size=(1, gam))
    x = np.stack([rng.choice(V, size=B, p=qq[0, i]) for i in range(gam)], axis=1)
    p = np.broadcast_to(_log(pp), (B, gam + 1, V))
    q = np.broadcast_to(_log(qq), (B, gam, V))
    a = orc.token_verify(p, q, x, gam, seed=9).accepted_len.mean()
    b = orc.block_verify(p, q, x, gam, seed=9).accepted_len.mean()
    assert b >= a - 0.02


def test_temperature_is_division_of_logits(orc):
    """Verifying logits z at temperature T takes the same decisions as
    verifying z / T at T = 1 (up to the binary32 decision rounding)."""
    rng = np.random.default_rng(51)
    B, gam, V = 100, 3, 30
    p = rng.normal(0, 3, (B, gam + 1, V))
    q = p[:, :gam] + rng.normal(0, 1, (B, gam, V))
    x = rng.integers(0, V, (B, gam))
    T = np.float32(0.7)
    a = orc.token_verify(p, q, x, gam, temperature=float(T), seed=1)
    b = orc.token_verify(p / np.float64(T), q / np.float64(T), x, gam, temperature=1.0, seed=1)
    ok = np.abs(a.dec_margin - b.dec_margin) < 1e-9
    assert ok[~np.isnan(a.dec_margin)].all()
    assert (a.accepted_len == b.accepted_len).all() and (a.out_tokens == b.out_tokens).all()


def test_data_errors_flag_requests(orc):
    rng = np.random.default_rng(61)
    B, gam, V = 4, 3, 20
    p = rng.normal(0, 1, (B, gam + 1, V))
    q = rng.normal(0, 1, (B, gam, V))
    x = rng.integers(0, V, (B, gam))
    x[1, 2] = V            # out of range
    p[2, 1, 5] = np.nan    # bad row
    q[3, 0, :] = -np.inf   # all -inf row
    for fn in (orc.token_verify, orc.block_verify):
        r = fn(p, q, x, gam, seed=1)
        assert r.accepted_len.tolist()[1:] == [-1, -1, -1] and r.accepted_len[0] >= 0
        assert r.flags.tolist()[1:] == [orc.FLAG_BAD_TOKEN, orc.FLAG_BAD_ROW, orc.FLAG_BAD_ROW]
        assert (r.out_tokens[1:] == -1).all()
    # a verify_len that skips the bad rows leaves the request usable
    vl = np.array([3, 2, 1, 0], np.int32)
    r = orc.token_verify(p, q, x, gam, verify_len=vl, seed=1)
    assert r.accepted_len[1] >= 0 and r.accepted_len[3] == 0


# ------------------------------------------------------------ scheduler ----

def _brute_force_schedule(conf, a, K):
    B, gam = conf.shape
    S = np.cumprod(conf, axis=1)
    best, arg = -1.0, None
    for Ls in itertools.product(range(gam + 1), repeat=B):
        E = B + sum(S[b, :Ls[b]].sum() for b in range(B))
        n = B + sum(Ls)
        f = E * a / (1 + n / K)
        if f > best * (1 + 1e-12):
            best, arg = f, Ls
    return np.array(arg), best


def test_scheduler_equals_brute_force_optimum(orc):
    """Greedy admission with early stopping reaches the brute-force maximum of
    E[emitted] x SPS(rows) over every allocation (zskr.cn section 04: maximise
    expected accepted tokens x engine step rate)."""
    rng = np.random.default_rng(71)
    for trial in range(150):
        B = int(rng.integers(1, 4))
        gam = int(rng.integers(1, 4))
        K = float(rng.choice([1.0, 2.0, 5.0, 20.0]))
        conf = rng.random((B, gam)) ** 0.5
        vl, E, _ = orc.schedule(conf, sps_a=2000.0, sps_k=K)
        S = np.cumprod(conf, axis=1)
        f = lambda Ls: (B + sum(S[b, :Ls[b]].sum() for b in range(B))) * 2000.0 / (1 + (B + sum(Ls)) / K)
        _, best = _brute_force_schedule(conf, 2000.0, K)
        assert abs(f(vl) - best) <= 1e-9 * best, trial
        assert abs(E - (B + sum(S[b, :vl[b]].sum() for b in range(B)))) < 1e-9


def test_scheduler_admits_exactly_where_the_gain_test_passes(orc):
    """Along the order (survival descending, id ascending) the gain test
    g(k) = s_k (K + B + k) - (B + sum_{j<k} s_j) never rises, since
    g(k+1) - g(k) = (s_{k+1} - s_k)(K + B + k + 1) <= 0; so the early-stopping
    greedy scan admits exactly the candidates with g > 0, each decidable from
    its own rank and the survival mass ranked before it.  Checked on random
    and heavily tied confidences with a stable sort of the survivals."""
    rng = np.random.default_rng(97)
    for trial in range(300):
        B = int(rng.integers(1, 40))
        gam = int(rng.integers(1, 9))
        K = float(rng.choice([3.0, 50.0, 4096.0]))
        conf = rng.random((B, gam)) ** 0.3 if trial % 2 else rng.integers(1, 5, (B, gam)) / 4.0
        vl, _, _ = orc.schedule(conf, 2000.0, K)
        S = np.cumprod(conf, axis=1).reshape(-1)
        order = np.argsort(-S, kind="stable")           # ties keep id order
        s_sorted = S[order]
        before = np.concatenate([[0.0], np.cumsum(s_sorted)[:-1]])
        g = s_sorted * (K + B + np.arange(S.size)) - (B + before)
        assert (np.diff(g) <= 1e-9 * (1 + np.abs(g[:-1]))).all(), trial
        admitted = np.zeros(S.size, bool)
        admitted[order[g > 0]] = True
        assert (admitted.reshape(B, gam).sum(axis=1) == vl).all(), trial


def test_scheduler_budget_shrinks_with_load(orc):
    """Light load: long verify budgets; heavy load: the budget tightens
    (kongchang.com "The Third Ace"; zskr.cn Fig. 4)."""
    rng = np.random.default_rng(81)
    gam = 8
    means = []
    for B in (1, 64, 512, 4096):
        conf = np.clip(rng.normal(0.7, 0.15, (B, gam)), 0, 1)
        vl, _, _ = orc.schedule(conf, 2000.0, 4096.0)
        means.append(vl.mean())
    assert means[0] >= 4 and all(x >= y for x, y in zip(means, means[1:])) and means[-1] < 2


def test_scheduler_prefix_closed_and_ties(orc):
    conf = np.array([[1.0, 1.0, 0.5], [1.0, 0.0, 1.0]])
    vl, E, _ = orc.schedule(conf, 2000.0, 4096.0)
    assert vl.tolist() == [3, 1] and abs(E - (2 + 1 + 1 + 0.5 + 1)) < 1e-12


# ------------------------------------------- sequential temperature scaling ----

def test_sts_closed_forms(orc):
    """Temperature scaling divides the head's log-odds by the position's own
    temperature before the logistic (kongchang.com "The Second Ace"; zskr.cn
    section 04): log-odds T_i*ln(k) give exactly k/(1+k) at every position,
    0 gives 1/2 whatever T_i is, +-inf give 1 and 0."""
    temps = np.array([0.5, 1.0, 2.0, 3.7])
    ks = np.array([3.0, 9.0, 1.0 / 3.0, 19.0])
    logits = np.stack([temps * np.log(ks), -temps * np.log(ks), np.zeros(4),
                       np.array([np.inf, -np.inf, np.inf, -np.inf])])
    c = orc.sts_confidence(logits, temps)
    np.testing.assert_allclose(c[0], ks / (1 + ks), rtol=1e-14)
    np.testing.assert_allclose(c[1], 1 / (1 + ks), rtol=1e-14)
    assert (c[2] == 0.5).all()
    assert c[3].tolist() == [1.0, 0.0, 1.0, 0.0]


def test_sts_keeps_order_within_a_position(orc):
    """Scaling by a positive temperature never reorders the candidates of one
    position (it only changes their magnitudes); a larger temperature pulls
    every estimate toward 1/2, a smaller one pushes it away."""
    rng = np.random.default_rng(17)
    logits = rng.normal(0.8, 2.0, (200, 5))
    ones = orc.sts_confidence(logits, np.ones(5))
    for temps in (np.array([0.3, 0.7, 1.5, 2.0, 4.0]), np.full(5, 1e6)):
        c = orc.sts_confidence(logits, temps)
        for i in range(5):
            assert (np.argsort(c[:, i], kind="stable") == np.argsort(ones[:, i], kind="stable")).all()
            flatter = np.abs(c[:, i] - 0.5) <= np.abs(ones[:, i] - 0.5) + 1e-15
            assert flatter.all() if temps[i] >= 1 else (~flatter | (logits[:, i] == 0)).all()
    assert np.abs(orc.sts_confidence(logits, np.full(5, 1e6)) - 0.5).max() < 1e-5


def test_sts_equals_library_logistic(orc):
    """Against SciPy's logistic function (scipy.special.expit) of logit / T_i."""
    from scipy.special import expit
    rng = np.random.default_rng(23)
    logits = rng.normal(0.0, 6.0, (64, 7)).astype(np.float32)
    temps = rng.uniform(0.4, 3.0, 7).astype(np.float32)
    c = orc.sts_confidence(logits, temps)
    ref = expit(logits.astype(np.float64) / temps.astype(np.float64)[None, :])
    np.testing.assert_allclose(c, ref, rtol=1e-14, atol=1e-300)
    with pytest.raises(ValueError):
        orc.sts_confidence(logits, np.zeros(7))
    with pytest.raises(ValueError):
        orc.sts_confidence(np.full((2, 7), np.nan), temps)


# --------------------------------------------------------------- Markov ----

def test_markov_without_transition_is_independent_icdf(orc):
    """U = 0: each position is an independent inverse-CDF draw of softmax(base_k)."""
    rng = np.random.default_rng(91)
    B, gam, V, R = 5, 4, 64, 8
    base = rng.normal(0, 3, (B, gam, V))
    U = np.zeros((V, R))
    W = rng.normal(0, 1, (R, V))
    x0 = rng.integers(0, V, B)
    r = orc.markov_draft(base, U, W, x0, seed=3)
    for b in range(B):
        for k in range(gam):
            pr = np.exp(base[b, k] - special.logsumexp(base[b, k]))
            u = orc.uniform(3, 0, b, k + 1, 2)
            want = int(np.searchsorted(np.cumsum(pr), u * pr.sum(), side="right"))
            assert r.draft[b, k] == want
    assert np.array_equal(r.q_logits, base)


def test_markov_contraction_matches_matmul(orc):
    """q_k - base_k equals U[x_{k-1}] @ W (numpy matmul in float64), chained
    through the sampled tokens."""
    rng = np.random.default_rng(92)
    B, gam, V, R = 3, 5, 300, 16
    base = rng.normal(0, 3, (B, gam, V))
    U = rng.normal(0, 0.5, (V, R))
    W = rng.normal(0, 0.5, (R, V))
    x0 = rng.integers(0, V, B)
    r = orc.markov_draft(base, U, W, x0, temperature=0.8, seed=4)
    prev = x0.copy()
    for k in range(gam):
        d = U[prev] @ W
        assert np.allclose(r.q_logits[:, k] - base[:, k], d, rtol=0, atol=1e-10)
        for b in range(B):
            assert abs(r.lse_q[b, k] - special.logsumexp(r.q_logits[b, k] / np.float64(np.float32(0.8)))) < 1e-10
        prev = r.draft[:, k]


def test_markov_chain_distribution(orc):
    """Monte Carlo: (x_1, x_2) follows the Markov chain
    P(x1) P(x2 | x1) with P(. | prev) = softmax(base_k + U[prev] W)."""
    rng = np.random.default_rng(93)
    N, gam, V, R = 40000, 2, 3, 2
    base1 = rng.normal(0, 1, (gam, V))
    U = rng.normal(0, 1, (V, R))
    W = rng.normal(0, 1, (R, V))
    x0 = 1
    r = orc.markov_draft(np.broadcast_to(base1, (N, gam, V)), U, W, np.full(N, x0), seed=7,
                         want_q=False)
    sm = lambda z: np.exp(z - special.logsumexp(z))
    exp = {}
    P1 = sm(base1[0] + U[x0] @ W)
    for a in range(V):
        P2 = sm(base1[1] + U[a] @ W)
        for c in range(V):
            exp[(a, c)] = P1[a] * P2[c]
    obs = {}
    for row in r.draft:
        obs[(row[0], row[1])] = obs.get((row[0], row[1]), 0) + 1
    cells = sorted(exp)
    chi2 = sum((obs.get(c, 0) - N * exp[c]) ** 2 / (N * exp[c]) for c in cells)
    assert chi2 < stats.chi2.ppf(1 - 1e-6, len(cells) - 1)


# ------------------------------------------------------------------ RNN ----

def _torch_bf16(x):
    import torch
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _torch_tanh_bf16(a):
    """bf16(tanh(a)) for binary32 a, by torch on the CPU (its own tanh and
    bf16 conversion)."""
    import torch
    t = torch.tanh(torch.tensor(np.asarray(a, np.float32)))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_rounding_equals_torch(orc):
    """Round-to-nearest-even to bf16 against torch's float32 -> bfloat16
    conversion, on random values, exact halfway cases (both parities),
    subnormals, zeros and infinities."""
    rng = np.random.default_rng(101)
    xs = list(rng.normal(0, 1, 3000).astype(np.float32)) + list(rng.normal(0, 1e-38, 200).astype(np.float32))
    bits = rng.integers(0, 2 ** 31, 2000, dtype=np.int64).astype(np.uint32)
    halfway = (bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    xs += list(halfway.view(np.float32)) + list((halfway | np.uint32(0x80000000)).view(np.float32))
    xs += [0.0, -0.0, np.inf, -np.inf, 1.0, 3.0, 65504.0]
    xs = np.array([x for x in xs if np.isfinite(x) or np.isinf(x)], np.float32)
    got = np.array([orc.bf16(float(x)) for x in xs])
    want = _torch_bf16(xs)
    assert np.array_equal(got, want)


def test_rnn_without_recurrence_is_markov_on_tanh_embeddings(orc):
    """A = 0 removes the in-block memory: hb_k = bf16(tanh(U[x_{k-1}])), so
    the RNN head equals the Markov head run with U' = bf16(tanh(U)) (computed
    here by torch) -- same draws, same logits."""
    rng = np.random.default_rng(102)
    B, gam, V, R = 4, 5, 200, 16
    base = rng.normal(0, 3, (B, gam, V))
    U = _torch_bf16(rng.normal(0, 0.8, (V, R)))
    W = _torch_bf16(rng.normal(0, 0.5, (R, V)))
    x0 = rng.integers(0, V, B)
    r = orc.rnn_draft(base, U, W, np.zeros((R, R)), x0, temperature=0.9, seed=5)
    Ut = _torch_tanh_bf16(U)
    m = orc.markov_draft(base, Ut, W, x0, temperature=0.9, seed=5)
    assert (r.state_margin > 4).all()
    assert np.array_equal(r.draft, m.draft)
    assert np.allclose(r.q_logits, m.q_logits, rtol=0, atol=1e-12)
    prev = x0.copy()
    for k in range(gam):
        assert np.array_equal(r.states[:, k], Ut[prev])
        prev = r.draft[:, k]


def test_rnn_state_recurrence_against_numpy(orc):
    """The states chain through the sampled tokens: hb_k = bf16(tanh(U[x_{k-1}]
    + A hb_{k-1})) with hb_0 = 0 (A [out, in]) (numpy float64 matmul, torch tanh and bf16);
    entries the oracle reports within 64 binary32 ulps of a rounding midpoint
    may differ by rounding order and are skipped.  The logits are
    base_k + hb_k W."""
    rng = np.random.default_rng(103)
    B, gam, V, R = 3, 6, 120, 24
    base = rng.normal(0, 3, (B, gam, V))
    U = _torch_bf16(rng.normal(0, 0.7, (V, R)))
    W = _torch_bf16(rng.normal(0, 0.5, (R, V)))
    A = _torch_bf16(rng.normal(0, 0.4, (R, R)))
    x0 = rng.integers(0, V, B)
    r = orc.rnn_draft(base, U, W, A, x0, seed=6)
    hb = np.zeros((B, R))
    prev = x0.copy()
    checked = 0
    for k in range(gam):
        a = U[prev] + hb @ A.T          # A in linear-layer layout [out, in]
        want = _torch_tanh_bf16(a)
        ok = r.state_margin[:, k] > 64
        assert np.array_equal(r.states[ok, k], want[ok])
        checked += int(ok.sum())
        assert np.allclose(r.q_logits[:, k] - base[:, k], r.states[:, k] @ W, rtol=0, atol=1e-10)
        hb = r.states[:, k]
        prev = r.draft[:, k]
    assert checked >= B * gam - 2
    # the recurrence matters: a later state differs from the memoryless one
    assert not np.array_equal(r.states[:, -1], _torch_tanh_bf16(U[r.draft[:, -2]]))


def test_rnn_chain_distribution(orc):
    """Monte Carlo: (x_1, x_2) follows P(x1) P(x2 | x1) with
    P(x1) = softmax(base_1 + hb_1 W), hb_1 = bf16(tanh(U[x0])), and
    P(. | x1) = softmax(base_2 + hb_2 W), hb_2 = bf16(tanh(U[x1] + A hb_1))."""
    rng = np.random.default_rng(104)
    N, gam, V, R = 40000, 2, 3, 2
    base1 = rng.normal(0, 1, (gam, V))
    U = _torch_bf16(rng.normal(0, 1, (V, R)))
    W = _torch_bf16(rng.normal(0, 1.5, (R, V)))
    A = _torch_bf16(rng.normal(0, 1.5, (R, R)))
    x0 = 1
    r = orc.rnn_draft(np.broadcast_to(base1, (N, gam, V)), U, W, A, np.full(N, x0), seed=8, want_q=False)
    sm = lambda z: np.exp(z - special.logsumexp(z))
    h1 = _torch_tanh_bf16(U[x0])
    P1 = sm(base1[0] + h1 @ W)
    exp = {}
    for a in range(V):
        h2 = _torch_tanh_bf16(U[a] + A @ h1)
        P2 = sm(base1[1] + h2 @ W)
        for c in range(V):
            exp[(a, c)] = P1[a] * P2[c]
    obs = {}
    for row in r.draft:
        obs[(row[0], row[1])] = obs.get((row[0], row[1]), 0) + 1
    cells = sorted(exp)
    chi2 = sum((obs.get(c, 0) - N * exp[c]) ** 2 / (N * exp[c]) for c in cells)
    assert chi2 < stats.chi2.ppf(1 - 1e-6, len(cells) - 1)


# ----------------------------------------------------------------- trees ----

TREES = [[0], [0, 0], [0, 1], [0, 0, 1], [0, 0, 0], [0, 0, 1, 1], [0, 1, 0, 3], [0, 0, 0, 1, 2]]


@pytest.mark.parametrize("parents", TREES, ids=[str(t) for t in TREES])
def test_exact_enumeration_tree_is_lossless(parents):
    """Reading pin for tree verification (the explainer's section 7 names it,
    without a rule): recursive rejection over a tree whose children of a node
    are drawn independently from the draft at that node.  Enumerated exactly
    over random rational tables (context-dependent and context-free, zero
    entries, p = q at some prefixes), the round's output completed by target
    draws equals the target's joint distribution."""
    rng = random.Random(300 + len(parents) * 7 + sum(parents))
    D = exact_enum_depth(parents)
    for trial in range(6):
        V = rng.randint(2, 3)
        p, q = exact_enum.random_tables(rng, V, D + 1, zero_prob=0.25, same_prob=0.3,
                                        context_free=(trial % 3 == 0))
        tj = exact_enum.target_joint(p, D + 1, V)
        dist, _ = exact_enum.tree_round(p, q, parents, V)
        assert exact_enum.complete_with_target(dist, p, D + 1, V) == {k: v for k, v in tj.items() if v}


def exact_enum_depth(parents):
    dep = [0]
    for par in parents:
        dep.append(dep[par] + 1)
    return max(dep)


def test_tree_chain_equals_token_verification(orc):
    """A chain-shaped tree (node m's parent is m - 1) is token verification:
    same uniforms, same decisions, same emitted tokens and ratios."""
    rng = np.random.default_rng(111)
    for noise, gam in ((1.0, 5), (0.3, 6), (2.0, 3)):
        B, V = 40, 300
        p = rng.normal(0, 3, (B, gam + 1, V))
        q = p[:, :gam] + noise * rng.normal(0, 1, (B, gam, V))
        x = np.array([[int(np.argmax(q[b, i] + rng.gumbel(size=V))) for i in range(gam)] for b in range(B)])
        t = orc.token_verify(p, q, x, gam, seed=9, offset=4)
        r = orc.tree_verify(p, q, x, list(range(gam)), seed=9, offset=4)
        assert np.array_equal(r.accepted_len, t.accepted_len)
        assert np.array_equal(r.out_tokens, t.out_tokens)
        ok = ~np.isnan(t.ratio)
        assert np.array_equal(np.isnan(r.ratio), ~ok) and np.array_equal(r.ratio[ok], t.ratio[ok])
        nodes = np.where(np.arange(gam)[None, :] < r.accepted_len[:, None], np.arange(1, gam + 1)[None, :], -1)
        assert np.array_equal(r.accepted_nodes, nodes)


def _tree_logits(rng, parents, V, p_tab, q_tab, B):
    """Per request: draft tokens drawn independently from q at each node, and
    the logit rows (log of the tables) of every node / internal node."""
    N = len(parents)
    internal = sorted(set(parents))
    P = np.zeros((B, N + 1, V))
    Q = np.zeros((B, len(internal), V))
    X = np.zeros((B, N), np.int32)
    with np.errstate(divide="ignore"):
        for b in range(B):
            pre = {0: ()}
            for m in range(1, N + 1):
                qd = np.array([float(v) for v in q_tab(pre[parents[m - 1]])])
                X[b, m - 1] = rng.choice(V, p=qd / qd.sum())
                pre[m] = pre[parents[m - 1]] + (int(X[b, m - 1]),)
            for n in range(N + 1):
                P[b, n] = np.log([float(v) for v in p_tab(pre[n])])
            for j, n in enumerate(internal):
                Q[b, j] = np.log([float(v) for v in q_tab(pre[n])])
    return P, Q, X


@pytest.mark.parametrize("parents", [[0, 0, 0, 1], [0, 1, 0, 2, 0]], ids=["3 root children", "3 branches"])
def test_oracle_tree_output_distribution_equals_target(orc, parents):
    """Monte Carlo over the C oracle: the emitted tokens, completed by target
    draws to depth + 1 tokens, follow the target's joint distribution
    (chi-square over every sequence)."""
    rng = np.random.default_rng(112 + len(parents))
    prng = random.Random(7 + len(parents))
    V = 3
    D = exact_enum_depth(parents)
    p_tab, q_tab = exact_enum.random_tables(prng, V, D + 1, zero_prob=0.2)
    Nr = 30000
    P, Q, X = _tree_logits(rng, parents, V, p_tab, q_tab, Nr)
    r = orc.tree_verify(P, Q, X, parents, seed=13)
    assert (r.flags == 0).all()
    counts = {}
    for b in range(Nr):
        s = tuple(int(t) for t in r.out_tokens[b, :r.accepted_len[b] + 1])
        while len(s) < D + 1:
            pd = np.array([float(v) for v in p_tab(s)])
            s = s + (int(rng.choice(V, p=pd / pd.sum())),)
        counts[s] = counts.get(s, 0) + 1
    tj = {k: float(v) for k, v in exact_enum.target_joint(p_tab, D + 1, V).items() if v}
    assert set(counts) <= set(tj)
    chi2 = sum((counts.get(k, 0) - Nr * v) ** 2 / (Nr * v) for k, v in tj.items())
    assert chi2 < stats.chi2.ppf(1 - 1e-6, len(tj) - 1), chi2


def test_block_residual_masses_are_the_thresholds_numerators(orc):
    """The residual masses the oracle reports are the m_i of its thresholds:
    h_i = m_i / (m_i + 1 - w_i) (1 where that denominator is 0) for i < L,
    m_i >= 0, and each m_i is at most w_i (it sums w_i p - q over the tokens
    where that is positive, and p sums to 1); NaN at i = L and beyond."""
    rng = np.random.default_rng(31)
    B, gamma, V = 24, 6, 97
    p = rng.normal(size=(B, gamma + 1, V)) * 2.0
    q = p[:, :gamma] + rng.normal(size=(B, gamma, V)) * rng.choice([0.2, 1.0, 3.0], size=(B, 1, 1))
    draft = rng.integers(0, V, size=(B, gamma)).astype(np.int32)
    vl = rng.integers(0, gamma + 1, size=B).astype(np.int32)
    r = orc.block_verify(p, q, draft, gamma, verify_len=vl, seed=5)
    for b in range(B):
        L = int(vl[b])
        for i in range(gamma):
            m, w, h = r.m[b, i], r.w[b, i], r.h[b, i]
            if i + 1 >= L:
                assert np.isnan(m)
                continue
            assert 0.0 <= m <= w + 1e-12
            den = m + 1.0 - w
            assert h == (m / den if den > 0.0 else 1.0)
