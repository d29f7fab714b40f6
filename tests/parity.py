"""Decision-walk comparison of GPU results with the CPU oracle.

Integer outputs must match bit for bit on every decision whose oracle margin
exceeds MARGIN; the first disagreeing decision of a request whose margin is
at most MARGIN counts as a within-margin flip and ends that request's
comparison.  Probabilities (capped ratios, residual masses, w, h) must agree
within PROB_ATOL; log-sum-exps within LSE_ATOL + LSE_RTOL * |lse|.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

MARGIN = 1e-4
PROB_ATOL = 1e-5
LSE_ATOL, LSE_RTOL = 1e-5, 1e-6
# Absolute precision of the GPU's running ratios w_i and residual masses m_i:
# w is a product of ratios of fp32-normalised probabilities (~1e-7 relative
# each); m = sum max(w p - q, 0) carries the fp32 rounding of every weight it
# sums (~1e-7 of sum(w p + q) <= 2) plus its fp32 segment sums.  1e-6 bounds
# both with room to spare.
WM_ABS_EPS = 1e-6
# A block tau disagreement beyond MARGIN is accepted (and counted apart, as a
# widened flip) only where the threshold is that ill-conditioned:
# D = m + 1 - w at most WIDEN_MAX_D.
WIDEN_MAX_D = 1e-3

@dataclass
class Report:
    requests: int = 0
    flips: int = 0
    widened_flips: int = 0   # block tau flips beyond MARGIN at D <= WIDEN_MAX_D (included in flips)
    uniforms_checked: int = 0
    failures: list = field(default_factory=list)
    max_prob_err: float = 0.0
    max_lse_err: float = 0.0

    def ok(self) -> bool:
        return not self.failures

    def __str__(self):
        return (f"requests={self.requests} flips={self.flips} widened_flips={self.widened_flips} "
                f"failures={len(self.failures)} uniforms_checked={self.uniforms_checked} "
                f"max_prob_err={self.max_prob_err:.2e} max_lse_err={self.max_lse_err:.2e} "
                f"{self.failures[:5]}")

    def as_dict(self) -> dict:
        return {"requests": self.requests, "flips": self.flips, "widened_flips": self.widened_flips,
                "failures": len(self.failures), "uniforms_checked": self.uniforms_checked,
                "max_prob_err": self.max_prob_err, "max_lse_err": self.max_lse_err}


def threshold_tol(w, m, dw=None):
    """Bound on the GPU's block thresholds h = m / D, D = m + 1 - w (oracle
    values; m is NaN at i = L, where h_L = w_L).  dh/dm = (1 - h) / D and
    dh/dw = h / D, so absolute errors eps_m in m and eps_w in w move h by at
    most ((1 - h) eps_m + h eps_w) / D to first order -- more than the flat
    probability tolerance when D is small, and without bound at D = 0, where
    h is 1 by convention but the GPU's rounding of w and m can put it
    anywhere in [0, 1].  eps_m = WM_ABS_EPS; eps_w is the GPU's own w
    difference `dw` where it is known (w is a product of up to L ratios of
    fp32-normalised probabilities, each off by about 1e-7 to 1e-6, and is
    itself checked against PROB_ATOL), at least WM_ABS_EPS."""
    w = np.asarray(w, np.float64)
    m = np.asarray(m, np.float64)
    eps_w = np.full_like(w, WM_ABS_EPS) if dw is None else np.maximum(np.abs(np.asarray(dw, np.float64)), WM_ABS_EPS)
    den = m + 1.0 - w
    h = np.where(den > 0.0, m / np.where(den > 0.0, den, 1.0), 1.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        extra = np.where(np.isnan(m), 0.0,
                         np.where(den > 0.0, ((1.0 - h) * WM_ABS_EPS + h * eps_w) / np.maximum(den, 1e-300),
                                  np.inf))
    return PROB_ATOL + np.where(np.isnan(m), eps_w, 0.0) + extra


def _close_threshold(rep, g, o, w, mres, what, b, gw=None):
    """Block thresholds within threshold_tol of the oracle's.  A failure
    records the position, both thresholds, both running ratios (gw: the
    GPU's), the oracle's residual mass and the one the GPU's h and w imply."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    m = ~np.isnan(o)
    if not m.any():
        return
    if np.isnan(g[m]).any():
        rep.failures.append((b, what, "nan on the GPU"))
        return
    err = np.abs(g[m] - o[m])
    dw = None if gw is None else (np.asarray(gw, np.float64) - np.asarray(w, np.float64))[m]
    tol = threshold_tol(np.asarray(w, np.float64)[m], np.asarray(mres, np.float64)[m], dw)
    rep.max_prob_err = max(rep.max_prob_err, float(err.max()))
    if (err > tol).any():
        k = int(np.argmax(err - tol))
        i = int(np.flatnonzero(m)[k])
        ow, om = float(np.asarray(w)[i]), float(np.asarray(mres)[i])
        gwi = float(np.asarray(gw)[i]) if gw is not None else float("nan")
        gm = g[i] * (1.0 - gwi) / (1.0 - g[i]) if g[i] < 1.0 else float("nan")
        rep.failures.append((b, what, float(err[k]), float(tol[k]),
                             dict(pos=i + 1, h_gpu=float(g[i]), h_orc=float(o[i]), w_gpu=gwi, w_orc=ow,
                                  m_orc=om, m_gpu_implied=gm)))


def _close_prob(rep, g, o, what, b):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    m = ~np.isnan(o)
    if m.any():
        if np.isnan(g[m]).any():
            rep.failures.append((b, what, "nan on the GPU"))
            return
        err = float(np.abs(g[m] - o[m]).max())
        rep.max_prob_err = max(rep.max_prob_err, err)
        if err > PROB_ATOL:
            rep.failures.append((b, what, err))


def _close_lse(rep, g, o, what, b):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    m = ~np.isnan(o)
    if m.any():
        err = np.abs(g[m] - o[m])
        rep.max_lse_err = max(rep.max_lse_err, float(err.max()))
        if (err > LSE_ATOL + LSE_RTOL * np.abs(o[m])).any() or np.isnan(g[m]).any():
            rep.failures.append((b, what, float(np.nanmax(err))))


def _same_uniforms(rep, g, o, b):
    """Uniforms the oracle drew for request b (non-NaN entries) against the
    GPU's, bit for bit: both sides evaluate the same Philox4x32-10 counters."""
    g = np.asarray(g, np.float32)
    o = np.asarray(o, np.float32)
    m = ~np.isnan(o)
    rep.uniforms_checked += int(m.sum())
    if not np.array_equal(g[m].view(np.uint32), o[m].view(np.uint32)):
        i = int(np.flatnonzero(m)[np.argmax(g[m] != o[m])])
        rep.failures.append((b, "uniform", i, float(o[i]), float(g[i])))
        return False
    return True


def compare_verify(gpu: dict, orc, gamma: int, verify_len=None, block: bool = False,
                   draft=None, rep: Report | None = None) -> Report:
    """gpu: dict of numpy arrays accepted_len, out_tokens and diag entries
    (lse_p, lse_q, ratio, w, h, resid_mass, flags, uniform) for the same
    requests as the oracle result `orc` (oracle.VerifyResult)."""
    rep = rep or Report()
    B = len(orc.accepted_len)
    for b in range(B):
        rep.requests += 1
        L = gamma if verify_len is None else int(verify_len[b])
        oa, ga = int(orc.accepted_len[b]), int(gpu["accepted_len"][b])
        if "uniform" in gpu and oa >= 0 and ga >= 0:
            # the decisions below are only comparable on the same uniforms
            if not _same_uniforms(rep, gpu["uniform"][b], orc.uniform[b], b):
                continue
        if oa < 0 or ga < 0:
            if oa != ga:
                rep.failures.append((b, "error status", oa, ga))
            elif "flags" in gpu and int(gpu["flags"][b]) != int(orc.flags[b]):
                rep.failures.append((b, "flags", int(orc.flags[b]), int(gpu["flags"][b])))
            elif (gpu["out_tokens"][b] != -1).any():
                rep.failures.append((b, "error row not cleared"))
            continue
        flipped = False
        if not block:
            for i in range(1, L + 1):
                o_acc, g_acc = i <= oa, i <= ga
                if o_acc != g_acc:
                    if orc.dec_margin[b, i - 1] <= MARGIN:
                        rep.flips += 1
                        flipped = True
                    else:
                        rep.failures.append((b, "accept", i, oa, ga, float(orc.dec_margin[b, i - 1])))
                    break
                if not o_acc:
                    break
        elif oa != ga:
            # the decision at the larger tau: a flip where |eta_i - h_i| is
            # within the margin, or, where h_i is ill-conditioned (D small),
            # within h_i's own bound (counted apart)
            i = max(oa, ga)
            mi, wi = float(orc.m[b, i - 1]), float(orc.w[b, i - 1])
            marg = float(orc.dec_margin[b, i - 1])
            den = mi + 1.0 - wi   # NaN at i = L, where h_L = w_L
            dw = float(gpu["w"][b, i - 1]) - wi if "w" in gpu else None
            htol = float(threshold_tol([wi], [mi], None if dw is None else [dw])[0])
            if marg <= MARGIN:
                rep.flips += 1
                flipped = True
            elif den == den and den <= WIDEN_MAX_D and marg <= htol:
                rep.flips += 1
                rep.widened_flips += 1
                flipped = True
            else:
                rep.failures.append((b, "block tau", oa, ga, marg, den))
        if flipped or (rep.failures and rep.failures[-1][0] == b):
            continue
        # same tau: tokens x_1..x_tau, then the drawn token
        if not np.array_equal(orc.out_tokens[b, :oa], gpu["out_tokens"][b, :ga]):
            rep.failures.append((b, "prefix tokens"))
            continue
        if draft is not None and not np.array_equal(np.asarray(draft[b, :oa]), orc.out_tokens[b, :oa]):
            rep.failures.append((b, "prefix is not the draft"))
        if (gpu["out_tokens"][b, ga + 1:] != -1).any():
            rep.failures.append((b, "padding"))
        if int(orc.out_tokens[b, oa]) != int(gpu["out_tokens"][b, ga]):
            if orc.icdf_margin[b] <= MARGIN:
                rep.flips += 1
            else:
                rep.failures.append((b, "draw", int(orc.out_tokens[b, oa]), int(gpu["out_tokens"][b, ga]),
                                     float(orc.icdf_margin[b])))
            continue
        # probabilities of the evaluated positions
        if "lse_p" in gpu:
            _close_lse(rep, gpu["lse_p"][b, :L + 1], orc.lse_p[b, :L + 1], "lse_p", b)
        if "lse_q" in gpu and L > 0:
            _close_lse(rep, gpu["lse_q"][b, :L], orc.lse_q[b, :L], "lse_q", b)
        if "ratio" in gpu and L > 0:
            _close_prob(rep, gpu["ratio"][b, :L], orc.ratio[b, :L], "ratio", b)
        if block and "w" in gpu and L > 0:
            _close_prob(rep, gpu["w"][b, :L], orc.w[b, :L], "w", b)
        if block and "h" in gpu and L > 0:
            _close_threshold(rep, gpu["h"][b, :L], orc.h[b, :L], orc.w[b, :L], orc.m[b, :L], "h", b,
                             gw=gpu["w"][b, :L] if "w" in gpu else None)
        if "resid_mass" in gpu:
            _close_prob(rep, [gpu["resid_mass"][b]], [orc.resid_mass[b]], "resid_mass", b)
        if "flags" in gpu and int(gpu["flags"][b]) != int(orc.flags[b]):
            rep.failures.append((b, "flags", int(orc.flags[b]), int(gpu["flags"][b])))
    return rep


def compare_markov(g_draft, g_lse, g_q, orc, rep: Report | None = None, q_atol: float = 2e-5) -> Report:
    """Markov sampler: draws walked left to right per request; q logits and
    lse compared on positions before the first (flipped) disagreement."""
    rep = rep or Report()
    B, gamma = orc.draft.shape
    for b in range(B):
        rep.requests += 1
        for k in range(gamma):
            o, g = int(orc.draft[b, k]), int(g_draft[b, k])
            if g_q is not None and orc.q_logits is not None:
                err = float(np.abs(np.asarray(g_q[b, k], np.float64) - orc.q_logits[b, k]).max())
                rep.max_prob_err = max(rep.max_prob_err, err)
                if err > q_atol:
                    rep.failures.append((b, k, "q logits", err))
                    break
            if g_lse is not None:
                _close_lse(rep, [g_lse[b, k]], [orc.lse_q[b, k]], f"lse_q[{k}]", b)
            if o != g:
                if orc.margin[b, k] <= MARGIN:
                    rep.flips += 1
                else:
                    rep.failures.append((b, k, "draw", o, g, float(orc.margin[b, k])))
                break
    return rep


STATE_MARGIN_ULPS = 4.0   # bf16 state rounding: flips allowed this close (binary32 ulps) to a midpoint


def compare_rnn(g_draft, g_lse, g_q, g_states, orc, rep: Report | None = None, q_atol: float = 2e-5) -> Report:
    """RNN-head sampler, walked per request left to right: at each position the
    bf16 state (bit-exact unless the oracle puts an entry within
    STATE_MARGIN_ULPS of its rounding midpoint), then the logits, the
    normaliser and the draw as for the Markov head; a request stops at its
    first (flipped) disagreement."""
    rep = rep or Report()
    B, gamma = orc.draft.shape
    for b in range(B):
        rep.requests += 1
        for k in range(gamma):
            if g_states is not None:
                gs = np.asarray(g_states[b, k], np.float64)
                if not np.array_equal(gs, orc.states[b, k]):
                    if orc.state_margin[b, k] <= STATE_MARGIN_ULPS:
                        rep.flips += 1
                    else:
                        bad = int(np.argmax(gs != orc.states[b, k]))
                        rep.failures.append((b, k, "state", bad, float(gs[bad]), float(orc.states[b, k, bad]),
                                             float(orc.state_margin[b, k])))
                    break
            o, g = int(orc.draft[b, k]), int(g_draft[b, k])
            if g_q is not None and orc.q_logits is not None:
                err = float(np.abs(np.asarray(g_q[b, k], np.float64) - orc.q_logits[b, k]).max())
                rep.max_prob_err = max(rep.max_prob_err, err)
                if err > q_atol:
                    rep.failures.append((b, k, "q logits", err))
                    break
            if g_lse is not None:
                _close_lse(rep, [g_lse[b, k]], [orc.lse_q[b, k]], f"lse_q[{k}]", b)
            if o != g:
                if orc.margin[b, k] <= MARGIN:
                    rep.flips += 1
                else:
                    rep.failures.append((b, k, "draw", o, g, float(orc.margin[b, k])))
                break
    return rep


def tree_tested(parents, accepted_nodes, depth, N):
    """(node, accepted) decisions of a tree walk in the order they were taken,
    reconstructed from the accepted path: at each node on the path every child
    up to the accepted one (all children where none was)."""
    ch = [[] for _ in range(N + 1)]
    for m in range(1, N + 1):
        ch[parents[m - 1]].append(m)
    out, node = [], 0
    for level in range(depth + 1):
        nxt = int(accepted_nodes[level]) if level < depth else -1
        for c in ch[node]:
            out.append((c, c == nxt))
            if c == nxt:
                break
        if nxt < 0:
            break
        node = nxt
    return out


def compare_tree(gpu: dict, orc, parents, rep: Report | None = None) -> Report:
    """Tree verification, per request: the sequence of (node, decision) pairs
    must match the oracle's unless the first disagreement sits on a decision
    whose oracle margin is at most MARGIN (a within-margin flip); with the
    same path the drawn token must match unless its inverse-CDF margin is
    within MARGIN; ratios of the tested nodes within PROB_ATOL."""
    rep = rep or Report()
    N = len(parents)
    B = len(orc.accepted_len)
    for b in range(B):
        rep.requests += 1
        oa, ga = int(orc.accepted_len[b]), int(gpu["accepted_len"][b])
        if oa < 0 or ga < 0:
            if oa != ga:
                rep.failures.append((b, "error status", oa, ga))
            elif "flags" in gpu and int(gpu["flags"][b]) != int(orc.flags[b]):
                rep.failures.append((b, "flags", int(orc.flags[b]), int(gpu["flags"][b])))
            continue
        od = tree_tested(parents, orc.accepted_nodes[b], oa, N)
        gd = tree_tested(parents, gpu["accepted_nodes"][b], ga, N)
        diverged = False
        for i in range(max(len(od), len(gd))):
            if i < len(od) and i < len(gd) and od[i] == gd[i]:
                continue
            node = od[i][0] if i < len(od) else gd[i][0]
            if orc.dec_margin[b, node - 1] <= MARGIN:
                rep.flips += 1
            else:
                rep.failures.append((b, "decision", node, od[i:i + 1], gd[i:i + 1],
                                     float(orc.dec_margin[b, node - 1])))
            diverged = True
            break
        if diverged:
            continue
        if not np.array_equal(orc.out_tokens[b, :oa], gpu["out_tokens"][b, :ga]):
            rep.failures.append((b, "path tokens"))
            continue
        if (gpu["out_tokens"][b, ga + 1:] != -1).any():
            rep.failures.append((b, "padding"))
        if int(orc.out_tokens[b, oa]) != int(gpu["out_tokens"][b, ga]):
            if orc.icdf_margin[b] <= MARGIN:
                rep.flips += 1
            else:
                rep.failures.append((b, "draw", int(orc.out_tokens[b, oa]), int(gpu["out_tokens"][b, ga]),
                                     float(orc.icdf_margin[b])))
            continue
        if "ratio" in gpu:
            tested = [n for n, _ in od]
            g = np.asarray(gpu["ratio"][b], np.float64)
            if np.isnan(g[[n - 1 for n in tested]]).any():
                rep.failures.append((b, "ratio missing"))
            _close_prob(rep, g[[n - 1 for n in tested]], orc.ratio[b, [n - 1 for n in tested]], "ratio", b)
            untested = sorted(set(range(1, N + 1)) - set(tested))
            if untested and not np.isnan(g[[n - 1 for n in untested]]).all():
                rep.failures.append((b, "ratio of an untested node"))
        if "flags" in gpu and int(gpu["flags"][b]) != int(orc.flags[b]):
            rep.failures.append((b, "flags", int(orc.flags[b]), int(gpu["flags"][b])))
    return rep
