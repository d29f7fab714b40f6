"""Benchmark of the verification hot path on one MI355X.

One step = one token-level verification call (row statistics, acceptance
scan, correction / bonus draw) over the headline batch: B=256 requests,
gamma=7 draft tokens, V=129280, bf16 logits, inputs resident in HBM.  Two
input sets (each ~993 MB, above the 256 MB Infinity Cache) alternate between
steps.  Prints ONE JSON line:

  value     verified positions/s = B * gamma / step time
  roofline  the row-statistics kernel (the dominant one): algorithmic bytes
            (every verified logit read once) / its mean duration from HIP
            events recorded inside the library on the launch stream, against
            8 TB/s; `traffic` from rocprofv3 FETCH_SIZE / WRITE_SIZE when the
            committed counter summary matches the current kernel source
  call_roofline  the whole call (row statistics + tail): algorithmic bytes of
            the timed steps (every verified logit once, plus the one or two
            rows each request's correction / bonus draw reads) / step time
  cpu_baseline  the CPU oracle on the same batch and round as the last timed
            step: all 256 requests on a pool of host threads (`value`,
            `cores`), and one thread on a bounded sample
  parity    the last timed step's outputs (and, from one more call with the
            same inputs and round, its diagnostics) against that oracle run,
            walked decision by decision: requests, within-margin flips,
            failures, largest probability / log-sum-exp differences

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--no-cpu-baseline]
       [--copy-probe]   (other workloads: also run the copy probe, for the counter scale;
                         the headline line always carries it)
       [--fused-only]   (markov workload: time only the fused path)
       [--workload headline|tiny|batched|block|block_async|markov|rnn|tree|all]
The other workloads (one JSON line each, same fields) measure the tiny and
batched token-verification batches, scheduler + block verification
(B=512, gamma=8), the same with temperature-scaled confidences and the
scheduler two steps ahead on a second stream, and the Markov-head sampler
followed by verification (B=128, gamma=8, R=256; its roofline entry adds the
MFMA rate), the RNN-head draft on the same inputs, and tree verification
(B=64, 4 branches of 5 nodes).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified positions/s + HBM GB/s vs peak, B=256 gamma=7 V=129,280 bf16"
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "rowstats_headline_traffic.json")
ROWSTATS_SOURCES = [os.path.join(ROOT, "lossless_draft_verification_02_amd", "csrc", f)
                    for f in ("rowstats.hip", "sv_rowstats.h", "sv_device.h")]
MARKOV_COUNTERS_FILE = os.path.join(ROOT, "profiles", "markov_gemm_counters.json")
TAIL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tail_headline_traffic.json")
TAIL_SOURCES = [os.path.join(ROOT, "lossless_draft_verification_02_amd", "csrc", f)
                for f in ("verify.hip", "sv_rowstats.h", "sv_device.h")]
MARKOV_SOURCES = [os.path.join(ROOT, "lossless_draft_verification_02_amd", "csrc", f)
                  for f in ("markov.hip", "sv_device.h")]


def kernel_source_digest(sources=ROWSTATS_SOURCES) -> str:
    h = hashlib.sha256()
    for f in sources:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(bytes_per_launch_alg):
    """Counter-derived HBM bytes per launch, or None if absent / stale."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def tail_traffic():
    """The headline tail's committed counter bytes per launch, or None if
    absent or taken on other sources."""
    if not os.path.exists(TAIL_TRAFFIC_FILE):
        return None
    with open(TAIL_TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_digest(TAIL_SOURCES):
        return None
    return t.get("hbm_bytes_per_launch")


def markov_counters():
    """The Markov contraction's committed counter summary (HBM bytes, MFMA
    busy fraction per launch), or None if absent or taken on other sources."""
    if not os.path.exists(MARKOV_COUNTERS_FILE):
        return None
    with open(MARKOV_COUNTERS_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_digest(MARKOV_SOURCES):
        return None
    return t


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_pool(chunks, run, units_of, single_budget_s):
    """Times `run` over `chunks`: on one thread over a bounded sample (until
    `single_budget_s` of oracle time), then on a pool of host threads over
    all of them.  Returns (results in order, pool wall s, threads, units done
    by one thread, its seconds)."""
    import concurrent.futures
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle_pool import workers

    spent, done = 0.0, 0
    for c in chunks:
        t0 = time.perf_counter()
        run(c)
        spent += time.perf_counter() - t0
        done += units_of(c)
        if spent >= single_budget_s:
            break
    n = min(workers(), len(chunks))   # a single chunk runs on one thread
    t0 = time.perf_counter()
    if n == 1:
        parts = [run(c) for c in chunks]
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=n) as ex:
            parts = list(ex.map(run, chunks))
    return parts, time.perf_counter() - t0, n, done, spent


def _baseline_dict(units, wall, n, done, spent, unit, what):
    return {"value": round(units / wall, 1), "unit": unit, "cores": n, "kind": "oracle",
            "sample": f"{what} on {n} host threads, {wall:.2f} s wall; one thread: {done} positions in {spent:.2f} s",
            "single_thread_value": round(done / spent, 1), "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def cpu_baseline_and_parity(vi, offset, gpu, single_budget_s=3.0, chunk=4, block=False, verify_len=None):
    """The CPU oracle on every request of `vi` at round `offset` (token
    verification, or block verification with `verify_len`): timed on one host
    thread over a bounded sample, then on a pool of threads over the whole
    batch (logits converted to float64 beforehand, outside the timed region);
    that result is walked against the GPU's outputs `gpu`."""
    import numpy as np
    import oracle
    from lossless_draft_verification_02_amd import workloads as WL
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle_pool import merge
    from parity import compare_verify

    oracle.build(force=False)
    vl = None if verify_len is None else np.asarray(verify_len, np.int32)
    chunks = []
    for b0 in range(0, vi.B, chunk):
        b1 = min(vi.B, b0 + chunk)
        chunks.append((vi.p[b0:b1].float().cpu().double().numpy(), vi.q[b0:b1].float().cpu().double().numpy(),
                       vi.draft[b0:b1].cpu().numpy(), np.arange(b0, b1, dtype=np.int32),
                       None if vl is None else vl[b0:b1]))
    fn = oracle.block_verify if block else oracle.token_verify

    def run(c):
        p, q, x, rid, v = c
        return fn(p, q, x, vi.gamma, temperature=vi.T, seed=WL.VERIFY_SEED, offset=offset, req_ids=rid,
                  verify_len=v)

    def units(c):
        return int(c[4].sum()) if c[4] is not None else len(c[3]) * vi.gamma

    parts, wall, n, done, spent = _oracle_pool(chunks, run, units, single_budget_s)
    orc = merge(parts)
    rep = compare_verify(gpu, orc, vi.gamma, verify_len=vl, block=block, draft=vi.draft.cpu().numpy())
    total = int(vl.sum()) if vl is not None else vi.B * vi.gamma
    base = _baseline_dict(total, wall, n, done, spent, "verified positions/s",
                          f"all {vi.B} requests of the last timed step's batch and round "
                          f"(gamma={vi.gamma}, V={vi.V}{', block verification' if block else ''})")
    parity = rep.as_dict()
    parity["failure_examples"] = [str(f) for f in rep.failures[:3]]
    return base, parity


def cpu_baseline_and_parity_markov(mi, offset, draft, gpu, single_budget_s=3.0, chunk=2):
    """The CPU oracle on every request of the markov workload at round
    `offset`: the Markov-head draft (oracle sampler), then token verification
    of the oracle's own draft against p with the oracle's fp64 draft logits;
    timed as cpu_baseline_and_parity.  The GPU's drafts are walked against the
    oracle's; its verification outputs against the oracle's on the requests
    whose drafts agree."""
    import numpy as np
    import oracle
    from lossless_draft_verification_02_amd import workloads as WL
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle_pool import merge
    from parity import compare_markov, compare_verify

    oracle.build(force=False)
    U = mi.U.float().cpu().double().numpy()
    W = mi.W.float().cpu().double().numpy()
    chunks = []
    for b0 in range(0, mi.B, chunk):
        b1 = min(mi.B, b0 + chunk)
        chunks.append((mi.base[b0:b1].float().cpu().double().numpy(), mi.x0[b0:b1].cpu().numpy(),
                       mi.p[b0:b1].float().cpu().double().numpy(), np.arange(b0, b1, dtype=np.int32)))

    def run(c):
        base, x0, p, rid = c
        d = oracle.markov_draft(base, U, W, x0, temperature=mi.T, seed=WL.DRAFT_SEED, offset=offset, req_ids=rid)
        v = oracle.token_verify(p, d.q_logits, d.draft, mi.gamma, temperature=mi.T, seed=WL.VERIFY_SEED,
                                offset=offset, req_ids=rid)
        d.q_logits = None   # the logits were only needed for the verification
        return d, v

    parts, wall, n, done, spent = _oracle_pool(chunks, run, lambda c: len(c[3]) * mi.gamma, single_budget_s)
    od = merge([d for d, _ in parts])
    ov = merge([v for _, v in parts])
    rep = compare_markov(draft, None, None, od)
    same = np.array([np.array_equal(od.draft[b], draft[b]) for b in range(mi.B)])
    keep = np.flatnonzero(same)
    rep2 = compare_verify({k: v[keep] for k, v in gpu.items()},
                          type(ov)(*[getattr(ov, f)[keep] for f in ov.__dataclass_fields__]), mi.gamma)
    base = _baseline_dict(mi.B * mi.gamma, wall, n, done, spent, "verified positions/s",
                          f"all {mi.B} requests of the last timed step's round: Markov draft then verification "
                          f"(gamma={mi.gamma}, V={mi.V}, R={mi.R})")
    parity = {"draft": rep.as_dict(), "verify": rep2.as_dict(), "requests_with_equal_drafts": int(len(keep)),
              "failure_examples": [str(f) for f in (rep.failures + rep2.failures)[:3]]}
    return base, parity


def _acceptance_by_position(acc, gamma):
    """Per draft position i (0-based), the share of the requests with a valid
    result whose accepted length exceeds i, i.e. that accepted token i."""
    import numpy as np
    a = np.asarray(acc)
    a = a[a >= 0]
    return [round(float((a > i).mean()), 4) for i in range(gamma)] if a.size else []


def _gpu_outputs(acc, out):
    return {"accepted_len": acc.cpu().numpy().copy(), "out_tokens": out.cpu().numpy().copy()}


def _diag_call(L, call, B, gamma, acc, out, gpu):
    """One more call on the last timed step's inputs and round with every
    diagnostic; returns whether its outputs equal the timed step's."""
    import torch
    diag = dict(lse_p=torch.empty(B, gamma + 1, device="cuda"), lse_q=torch.empty(B, max(gamma, 1), device="cuda"),
                ratio=torch.empty(B, max(gamma, 1), device="cuda"), resid_mass=torch.empty(B, device="cuda"),
                flags=torch.zeros(B, dtype=torch.int32, device="cuda"),
                uniform=torch.empty(B, gamma + 1, device="cuda"))
    call(diag)
    torch.cuda.synchronize()
    same = bool((acc.cpu().numpy() == gpu["accepted_len"]).all() and (out.cpu().numpy() == gpu["out_tokens"]).all())
    gpu.update({k: v.cpu().numpy() for k, v in diag.items()})
    gpu["flags"] = gpu["flags"].astype("uint32")
    return same


def _time_steps(step, warmup, steps):
    """Mean ms per step over exactly `steps` steps, synchronised on both sides."""
    import torch
    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for k in range(steps):
        step(warmup + k)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1) / steps, wall / steps * 1e3


def _profile_steps(L, ctx, step, first, steps):
    """Per-kernel mean durations (HIP events recorded by the library)."""
    L.spec_verify_profile_enable(ctx, True)
    L.spec_verify_profile_read(ctx)
    for k in range(steps):
        step(first + k)
    prof = L.spec_verify_profile_read(ctx)
    L.spec_verify_profile_enable(ctx, False)
    return prof


def _mean_us(prof, name):
    ms, n = prof[name]
    return ms / max(n, 1) * 1e3


def _copy_probe():
    """A plain streaming kernel of known traffic (1 GiB read + 1 GiB written
    per dispatch): a reference for what this part sustains on a copy, and the
    kernel whose FETCH_SIZE / WRITE_SIZE readings scale the counters."""
    import torch
    n = (1 << 30) // 4
    src = torch.zeros(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        torch.bitwise_not(src, out=dst)
    e1.record()
    torch.cuda.synchronize()
    copy_us = e0.elapsed_time(e1) / 5 * 1e3
    del src, dst
    return {"kernel": "torch.bitwise_not over 1 GiB int32", "bytes_per_launch": 2 << 30,
            "mean_us": round(copy_us, 2), "gbps": round((2 << 30) / (copy_us * 1e-6) / 1e9, 1)}


def _hbm_roofline(kernel, alg_bytes, mean_us, traffic=None):
    achieved = alg_bytes / (mean_us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic, "kernel": kernel,
            "alg_bytes_per_launch": int(alg_bytes), "mean_us": round(mean_us, 2)}


def _line(metric, value, unit, args, ms, config, roofline, **extra):
    d = {"metric": metric, "value": round(value, 1), "unit": unit, "n_gpus": 1, "steps": args.steps,
         "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
         "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": config, "roofline": roofline}
    d.update(extra)
    return d


def bench_headline(args, L, WL):
    import numpy as np
    import torch
    cfg = WL.WORKLOADS["headline"]
    # two independent batches of the headline recipe (each above the 256 MB
    # Infinity Cache), alternated between steps
    sets = [WL.make_verify_inputs("headline", "cuda"), WL.make_verify_inputs("headline", "cuda", seed=1103)]
    vi = sets[0]
    B, gamma, V = vi.B, vi.gamma, vi.V
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, gamma + 1, dtype=torch.int32, device="cuda")
    ctx = L.Context(0, B, gamma, V)

    def step(k):
        s = sets[k % len(sets)]
        L.spec_verify_run(ctx, s.p, s.q, s.draft, acc, out, temperature=s.T, seed=WL.VERIFY_SEED, offset=k)

    ms, wall_ms = _time_steps(step, args.warmup, args.steps)
    # the last timed step's outputs, then one more call on the same inputs and
    # round with every diagnostic (its outputs must be the same)
    k_last = args.warmup + args.steps - 1
    gpu = _gpu_outputs(acc, out)
    s_last = sets[k_last % len(sets)]
    same = _diag_call(L, lambda d: L.spec_verify_run(ctx, s_last.p, s_last.q, s_last.draft, acc, out,
                                                     temperature=s_last.T, seed=WL.VERIFY_SEED, offset=k_last,
                                                     diag=d), B, gamma, acc, out, gpu)
    # bytes of the timed steps: every verified row once, plus the rows each
    # request's draw re-reads (p and q row tau+1 after a rejection, the bonus
    # row alone otherwise)
    row_bytes = V * vi.p.element_size()
    reread = 0
    a_all = []
    for k in range(args.warmup, args.warmup + args.steps):
        step(k)
        a = acc.cpu().numpy()
        a_all.append(a)
        reread += int(((a >= 0) & (a < gamma)).sum()) * 2 * row_bytes + int((a == gamma).sum()) * row_bytes
    a_all = np.concatenate(a_all)
    accepted = float(a_all[a_all >= 0].mean())
    call_bytes = WL.bytes_single_read(vi) + reread / args.steps + B * gamma * 4 + B * (gamma + 2) * 4
    prof = _profile_steps(L, ctx, step, args.warmup + args.steps, args.steps)
    alg = WL.bytes_single_read(vi)
    roofline = _hbm_roofline("k_rowstats", alg, _mean_us(prof, "rowstats"), measured_traffic(alg))
    call_gbps = call_bytes / (ms * 1e-3) / 1e9
    # the tail (acceptance, correction / bonus sums, draw): the rows the draws
    # re-read per call, over the tail's own time; with the committed counter
    # bytes when they were taken on the current sources
    # (the fused k_tail, or the split accept+sums / select pair where the
    # library routes the batch that way)
    tail_us = (_mean_us(prof, "tail") if prof["tail"][1]
               else sum(_mean_us(prof, k) for k in ("resid", "select") if prof[k][1]))
    tail_alg = reread / args.steps
    tail_hbm = tail_traffic()
    tail_roofline = {"bound": "hbm (re-read) + latency", "achieved": round(tail_alg / (tail_us * 1e-6) / 1e9, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(tail_alg / (tail_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                     "alg_bytes_per_launch": int(tail_alg), "mean_us": tail_us, "traffic": tail_hbm,
                     "traffic_gbps": (round(tail_hbm / (tail_us * 1e-6) / 1e9, 1) if tail_hbm else None),
                     "what": "k_tail: the rows each request's draw re-reads (2 after a rejection, 1 for a bonus)"}
    single_gbps = alg / (ms * 1e-3) / 1e9
    call_roofline = {"bound": "hbm", "achieved": round(call_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(call_gbps / PEAK_HBM_GBPS, 4), "alg_bytes_per_call": int(call_bytes),
                     "what": "whole verification call: every verified row once + the draw's re-read rows",
                     "single_read_achieved": round(single_gbps, 1),
                     "single_read_frac": round(single_gbps / PEAK_HBM_GBPS, 4),
                     "single_read_what": "the same call counting every verified row once and nothing else"}
    copy_probe = _copy_probe()
    ctx.close()
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline_and_parity(s_last, k_last, gpu)
        parity["diag_call_outputs_equal_timed"] = same
    return _line(METRIC, B * gamma / (ms / 1e3), "verified positions/s", args, ms,
                 {"workload": "token-level verification, headline batch", "B": B, "gamma": gamma, "V": V,
                  "logits": "bf16", "temperature": cfg["T"], "input_sets": len(sets)},
                 roofline, cpu_baseline=cpu, parity=parity, call_roofline=call_roofline, tail_roofline=tail_roofline,
                 kernels_mean_us={k: round(_mean_us(prof, k), 2) for k, v in prof.items() if v[1]},
                 emitted_tokens_per_s=round(B * (accepted + 1) / (ms / 1e3), 1),
                 mean_accepted=round(accepted, 4), acceptance_by_position=_acceptance_by_position(a_all, gamma),
                 wall_ms_per_step=round(wall_ms, 5), copy_probe=copy_probe,
                 env={"hip": torch.version.hip, "torch": torch.__version__,
                      "device": torch.cuda.get_device_name(0)})


def bench_token(args, L, WL, name, nsets):
    """Token verification of the tiny or the batched workload."""
    import torch
    seed0 = WL.WORKLOADS[name]["seed"]
    sets = [WL.make_verify_inputs(name, "cuda", seed=seed0 + 100 * k) for k in range(nsets)]
    vi = sets[0]
    B, gamma, V = vi.B, vi.gamma, vi.V
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, gamma + 1, dtype=torch.int32, device="cuda")
    ctx = L.Context(0, B, gamma, V)

    def step(k):
        s = sets[k % len(sets)]
        L.spec_verify_run(ctx, s.p, s.q, s.draft, acc, out, temperature=s.T, seed=WL.VERIFY_SEED, offset=k)

    ms, _ = _time_steps(step, args.warmup, args.steps)
    k_last = args.warmup + args.steps - 1
    gpu = _gpu_outputs(acc, out)
    s_last = sets[k_last % len(sets)]
    same = _diag_call(L, lambda d: L.spec_verify_run(ctx, s_last.p, s_last.q, s_last.draft, acc, out,
                                                     temperature=s_last.T, seed=WL.VERIFY_SEED, offset=k_last,
                                                     diag=d), B, gamma, acc, out, gpu)
    accepted = float(gpu["accepted_len"][gpu["accepted_len"] >= 0].mean())
    prof = _profile_steps(L, ctx, step, args.warmup + args.steps, args.steps)
    ctx.close()
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline_and_parity(s_last, k_last, gpu)
        parity["diag_call_outputs_equal_timed"] = same
    return _line(f"verified positions/s, {WL.describe(name)}", B * gamma / (ms / 1e3), "verified positions/s",
                 args, ms, {"workload": f"token-level verification, {name} batch", "B": B, "gamma": gamma, "V": V,
                            "logits": str(vi.p.dtype).split(".")[-1], "temperature": vi.T, "input_sets": nsets},
                 _token_roofline(prof, vi, WL), cpu_baseline=cpu, parity=parity,
                 mean_accepted_last_step=round(accepted, 4),
                 acceptance_by_position=_acceptance_by_position(gpu["accepted_len"], gamma),
                 emitted_tokens_per_s=round(B * (accepted + 1) / (ms / 1e3), 1),
                 us_per_call=round(ms * 1e3, 2),
                 kernels_mean_us={k: round(_mean_us(prof, k), 2) for k, v in prof.items() if v[1]})


def _token_roofline(prof, vi, WL):
    """Row statistics' roofline, or, when a small problem ran as one launch
    (no separate row-statistics kernel), that launch's."""
    if prof["rowstats"][1]:
        return _hbm_roofline("k_rowstats", WL.bytes_single_read(vi), _mean_us(prof, "rowstats"))
    r = _hbm_roofline("k_tail (row statistics + tail in one launch)", WL.bytes_single_read(vi),
                      _mean_us(prof, "tail"))
    r["bound"] = "latency"
    return r


def bench_block(args, L, WL):
    """The block workload: scheduler + block verification, B=512, gamma=8."""
    import torch
    sets = [WL.make_verify_inputs("block", "cuda"), WL.make_verify_inputs("block", "cuda", seed=1105)]
    vi = sets[0]
    B, gamma, V = vi.B, vi.gamma, vi.V
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, gamma + 1, dtype=torch.int32, device="cuda")
    vlen = torch.empty(B, dtype=torch.int32, device="cuda")
    ctx = L.Context(0, B, gamma, V)

    def step(k):
        s = sets[k % len(sets)]
        L.spec_blockverify_run(ctx, s.p, s.q, s.draft, acc, out, temperature=s.T, seed=WL.VERIFY_SEED, offset=k,
                               conf=s.conf, sps_a=2000.0, sps_k=4096.0, verify_len_out=vlen)

    ms, _ = _time_steps(step, args.warmup, args.steps)
    k_last = args.warmup + args.steps - 1
    gpu = _gpu_outputs(acc, out)
    vl_last = vlen.cpu().numpy().copy()
    s_last = sets[k_last % len(sets)]
    same = _diag_call(L, lambda d: L.spec_blockverify_run(ctx, s_last.p, s_last.q, s_last.draft, acc, out,
                                                          temperature=s_last.T, seed=WL.VERIFY_SEED, offset=k_last,
                                                          verify_len=vlen, diag=d), B, gamma, acc, out, gpu)
    accepted = float(gpu["accepted_len"][gpu["accepted_len"] >= 0].mean())
    prof = _profile_steps(L, ctx, step, args.warmup + args.steps, args.steps)
    # verified positions: what the scheduler admitted (the same for every step of a set)
    admitted = []
    for s in sets:
        L.spec_schedule_run(ctx, s.conf, vlen, sps_a=2000.0, sps_k=4096.0)
        torch.cuda.synchronize()
        admitted.append(vlen.cpu().numpy().astype("int64"))
    ctx.close()
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        import oracle
        ovl, _, _ = oracle.schedule(s_last.conf.double().cpu().numpy(), 2000.0, 4096.0)
        cpu, parity = cpu_baseline_and_parity(s_last, k_last, gpu, block=True, verify_len=ovl)
        parity["scheduler_lengths_equal_oracle"] = bool((ovl == vl_last).all())
        parity["diag_call_outputs_equal_timed"] = same
    positions = sum(float(x.sum()) for x in admitted) / len(admitted)
    rows = sum(float((2 * x + 1).sum()) for x in admitted) / len(admitted)
    alg = rows * V * vi.p.element_size()
    return _line("verified positions/s, B=512 gamma=8 V=129,280 bf16, scheduler + block verification",
                 positions / (ms / 1e3), "verified positions/s", args, ms,
                 {"workload": "block verification driven by the confidence scheduler", "B": B, "gamma": gamma,
                  "V": V, "logits": "bf16", "sps": "2000/(1+n/4096)", "input_sets": len(sets)},
                 _hbm_roofline("k_rowstats", alg, _mean_us(prof, "rowstats")), cpu_baseline=cpu, parity=parity,
                 mean_verify_len=round(positions / B, 4), mean_accepted_last_step=round(accepted, 4),
                 acceptance_by_position=_acceptance_by_position(gpu["accepted_len"], gamma),
                 emitted_tokens_per_s=round(B * (accepted + 1) / (ms / 1e3), 1),
                 kernels_mean_us={k: round(_mean_us(prof, k), 2) for k, v in prof.items() if v[1]})


def bench_markov(args, L, WL):
    """The markov workload: Markov-head draft sampling (gamma positions), then verification of
    that draft.  The timed step is the fused path (markov_verify_run: no fp32 draft
    logits materialised); the two-call path (markov_draft_run writing q, then
    spec_verify_run reading it) is timed alongside for comparison."""
    import torch
    mi = WL.make_markov_inputs("cuda")
    B, gamma, V, R = mi.B, mi.gamma, mi.V, mi.R
    draft = torch.empty(B, gamma, dtype=torch.int32, device="cuda")
    ql = torch.empty(B, gamma, V, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, gamma, dtype=torch.float32, device="cuda")
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, gamma + 1, dtype=torch.int32, device="cuda")
    ctx = L.Context(0, B, gamma, V, R)

    def step(k):
        L.markov_verify_run(ctx, mi.base, mi.U, mi.Wt, mi.x0, mi.p, draft, acc, out, lse_q=lse, temperature=mi.T,
                            draft_seed=WL.DRAFT_SEED, verify_seed=WL.VERIFY_SEED, offset=k)

    def step_two_calls(k):
        L.markov_draft_run(ctx, mi.base, mi.U, mi.Wt, mi.x0, draft, q_logits=ql, lse_q=lse, temperature=mi.T,
                           seed=WL.DRAFT_SEED, offset=k)
        L.spec_verify_run(ctx, mi.p, ql, draft, acc, out, temperature=mi.T, seed=WL.VERIFY_SEED, offset=k)

    ms, _ = _time_steps(step, args.warmup, args.steps)
    k_last = args.warmup + args.steps - 1
    gpu = _gpu_outputs(acc, out)
    draft_last = draft.cpu().numpy().copy()
    same = _diag_call(L, lambda d: L.markov_verify_run(ctx, mi.base, mi.U, mi.Wt, mi.x0, mi.p, draft, acc, out,
                                                       lse_q=lse, temperature=mi.T, draft_seed=WL.DRAFT_SEED,
                                                       verify_seed=WL.VERIFY_SEED, offset=k_last, diag=d),
                      B, gamma, acc, out, gpu)
    same = same and bool((draft.cpu().numpy() == draft_last).all())
    accepted = float(gpu["accepted_len"][gpu["accepted_len"] >= 0].mean())
    prof = _profile_steps(L, ctx, step, args.warmup + args.steps, args.steps)
    ms2 = None
    if not args.fused_only:
        ms2, _ = _time_steps(step_two_calls, args.warmup, args.steps)
    ctx.close()
    gemm_us = _mean_us(prof, "markov_gemm")
    # algorithmic bytes of the draft per call: the base logits once, W once
    # (its re-reads at every position are the kernel's, not the method's),
    # the gathered U rows; per launch = per call / gamma
    per_call = B * gamma * V * 2 + R * V * 2 + B * gamma * R * 2
    flops = 2.0 * B * R * V
    roof = _hbm_roofline("k_markov_gemm", per_call / gamma, gemm_us, None)
    roof["alg_bytes_what"] = "base logits + W once per call + U rows, per launch (per call / gamma)"
    per_launch_w_each = B * V * 2 + R * V * 2 + B * R * 2
    roof["frac_w_each_position"] = round(per_launch_w_each / (gemm_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)
    roof["mfma_tflops"] = round(flops / (gemm_us * 1e-6) / 1e12, 2)
    roof["mfma_frac_of_bf16_peak"] = round(flops / (gemm_us * 1e-6) / 2.5e15, 4)
    cnt = markov_counters()
    if cnt:
        roof["traffic"] = cnt.get("hbm_bytes_per_launch")
        roof["mfma_busy_frac_counters"] = cnt.get("mfma_busy_frac")
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline_and_parity_markov(mi, k_last, draft_last, gpu)
        parity["diag_call_outputs_equal_timed"] = same
    return _line("verified positions/s, B=128 gamma=8 V=129,280, Markov-head draft + verification",
                 B * gamma / (ms / 1e3), "verified positions/s", args, ms,
                 {"workload": "Markov-head draft sampling (R=256), then token verification of that draft "
                              "(p bf16; fused: no fp32 draft logits stored)",
                  "B": B, "gamma": gamma, "V": V, "R": R},
                 roof, cpu_baseline=cpu, parity=parity, mean_accepted_last_step=round(accepted, 4),
                 acceptance_by_position=_acceptance_by_position(gpu["accepted_len"], gamma),
                 emitted_tokens_per_s=round(B * (accepted + 1) / (ms / 1e3), 1),
                 kernels_mean_us={k: round(_mean_us(prof, k), 2) for k, v in prof.items() if v[1]},
                 markov_ms_per_call=round((prof["markov_gemm"][0] + prof["markov_select"][0]) / args.steps, 4),
                 two_call_ms_per_step=None if ms2 is None else round(ms2, 5),
                 two_call_verified_positions_per_s=None if ms2 is None else round(B * gamma / (ms2 / 1e3), 1))


def bench_tree(args, L, WL):
    """Tree verification: B=64 requests, 4 branches of 5 draft nodes from the
    root (N=20, 17 nodes with children), V=129,280, bf16.  A step is one
    tree_verify_run (row statistics of every node's rows, then the walk)."""
    import torch
    sets = [WL.make_tree_inputs("cuda"), WL.make_tree_inputs("cuda", seed=2007)]
    ti = sets[0]
    B, V, N = ti.B, ti.V, len(ti.parents)
    NQ = ti.q.shape[1]
    D = max(1, max(_tree_depths(ti.parents)))
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, D + 1, dtype=torch.int32, device="cuda")
    nodes = torch.empty(B, D, dtype=torch.int32, device="cuda")
    ctx = L.Context(0, B, N, V)
    accepted = []

    def step(k):
        s = sets[k % len(sets)]
        L.tree_verify_run(ctx, s.p, s.q, s.tokens, s.parents, acc, out, accepted_nodes=nodes, temperature=s.T,
                          seed=WL.VERIFY_SEED, offset=k)

    ms, _ = _time_steps(step, args.warmup, args.steps)
    prof = _profile_steps(L, ctx, step, args.warmup + args.steps, args.steps)
    for k in range(4):
        step(k)
        torch.cuda.synchronize()
        accepted.append(float(acc.float().mean().item()))
    ctx.close()
    alg = B * (N + 1 + NQ) * V * ti.p.element_size()
    mean_acc = sum(accepted) / len(accepted)
    return _line("verified tree nodes/s, B=64 tree 4x5 (N=20) V=129,280 bf16, tree verification",
                 B * N / (ms / 1e3), "verified tree nodes/s", args, ms,
                 {"workload": "tree verification (recursive rejection), 4 branches of 5 nodes from the root",
                  "B": B, "N": N, "depth": D, "V": V, "logits": "bf16", "input_sets": len(sets)},
                 _hbm_roofline("k_rowstats", alg, _mean_us(prof, "rowstats")),
                 mean_accepted_len=round(mean_acc, 4),
                 emitted_tokens_per_s=round(B * (mean_acc + 1) / (ms / 1e3), 1),
                 kernels_mean_us={k: round(_mean_us(prof, k), 2) for k, v in prof.items() if v[1]})


def _tree_depths(parents):
    dep = [0]
    for par in parents:
        dep.append(dep[par] + 1)
    return dep


def bench_rnn(args, L, WL):
    """RNN-head draft sampling on the markov workload's inputs plus a recurrent matrix:
    gamma positions, each the contraction with the bf16 state, the draw, and
    the next state (no logit rows stored).  Also timed: the Markov head's
    draft alone on the same inputs, the cost the recurrence adds to."""
    import torch
    mi = WL.make_markov_inputs("cuda")
    A = WL.make_rnn_recurrence(mi.R, "cuda")
    B, gamma, V, R = mi.B, mi.gamma, mi.V, mi.R
    draft = torch.empty(B, gamma, dtype=torch.int32, device="cuda")
    lse = torch.empty(B, gamma, dtype=torch.float32, device="cuda")
    ctx = L.Context(0, B, gamma, V, R)

    def step(k):
        L.rnn_draft_run(ctx, mi.base, mi.U, mi.Wt, A, mi.x0, draft, lse_q=lse, temperature=mi.T,
                        seed=WL.DRAFT_SEED, offset=k)

    ms, _ = _time_steps(step, args.warmup, args.steps)
    prof = _profile_steps(L, ctx, step, args.warmup + args.steps, args.steps)
    ctx.close()
    gemm_us = _mean_us(prof, "markov_gemm")
    # per call: the base logits once, W once, A once, the state rows; per
    # launch = per call / gamma (W's re-read at each position is the kernel's)
    per_call = B * gamma * V * 2 + R * V * 2 + R * R * 2 + B * gamma * R * 2
    flops = 2.0 * B * R * V
    roof = _hbm_roofline("k_markov_gemm", per_call / gamma, gemm_us)
    roof["alg_bytes_what"] = "base logits + W + A once per call + state rows, per launch (per call / gamma)"
    roof["frac_w_each_position"] = round((B * V * 2 + R * V * 2 + B * R * 2) / (gemm_us * 1e-6) / 1e9
                                         / PEAK_HBM_GBPS, 4)
    roof["mfma_tflops"] = round(flops / (gemm_us * 1e-6) / 1e12, 2)
    roof["mfma_frac_of_bf16_peak"] = round(flops / (gemm_us * 1e-6) / 2.5e15, 4)
    return _line("drafted positions/s, B=128 gamma=8 V=129,280 R=256, RNN-head draft",
                 B * gamma / (ms / 1e3), "drafted positions/s", args, ms,
                 {"workload": "RNN-head draft sampling (R=256, Elman state over the Markov factors; "
                              "no logit rows stored)", "B": B, "gamma": gamma, "V": V, "R": R},
                 roof, kernels_mean_us={k: round(_mean_us(prof, k), 2) for k, v in prof.items() if v[1]})


def bench_block_async(args, L, WL, side=None):
    """The block workload with temperature-scaled confidences and the scheduler run
    two steps ahead: at step k a second stream (own context) schedules from
    step k's head estimates the verify lengths that step k + 2 uses, while
    the verification stream works on step k with the lengths scheduled at
    step k - 2.  Three length buffers in a ring; events order the handovers
    (schedule done -> verify, verify done reading a slot -> its next
    schedule)."""
    import torch
    sets = [WL.make_verify_inputs("block", "cuda"), WL.make_verify_inputs("block", "cuda", seed=1105)]
    vi = sets[0]
    B, gamma, V = vi.B, vi.gamma, vi.V
    temps = WL.sts_temperatures(gamma)
    logits = [WL.sts_head_logits(s.conf, temps) for s in sets]
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, gamma + 1, dtype=torch.int32, device="cuda")
    ring = [torch.zeros(B, dtype=torch.int32, device="cuda") for _ in range(3)]
    sched_done = [torch.cuda.Event() for _ in range(3)]
    slot_free = [torch.cuda.Event() for _ in range(3)]
    ctx = L.Context(0, B, gamma, V)
    sctx = L.Context(0, B, gamma, 1)         # the scheduler needs no vocabulary workspace
    main_s = torch.cuda.current_stream()
    side = torch.cuda.Stream() if side is None else side

    def schedule(k):                          # lengths for step k + 2 from step k's estimates
        side.wait_event(slot_free[k % 3])
        L.spec_schedule_sts_run(sctx, logits[k % len(sets)], temps, ring[k % 3], sps_a=2000.0, sps_k=4096.0,
                                stream=side)
        sched_done[k % 3].record(side)

    def step(k):
        s = sets[k % len(sets)]
        main_s.wait_event(sched_done[(k - 2) % 3])
        L.spec_blockverify_run(ctx, s.p, s.q, s.draft, acc, out, temperature=s.T, seed=WL.VERIFY_SEED, offset=k,
                               verify_len=ring[(k - 2) % 3])
        slot_free[(k - 2) % 3].record(main_s)
        schedule(k)

    side.wait_stream(main_s)                  # inputs are written on the main stream
    schedule(-2)
    schedule(-1)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(main_s)
    for k in range(args.steps):
        step(args.warmup + k)
    main_s.wait_stream(side)                  # the timed region ends after the last schedule too
    ev1.record(main_s)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    first = args.warmup + args.steps
    L.spec_verify_profile_enable(sctx, True)
    L.spec_verify_profile_read(sctx)
    prof = _profile_steps(L, ctx, step, first, args.steps)
    sprof = L.spec_verify_profile_read(sctx)
    torch.cuda.synchronize()
    admitted = []
    for lg in logits:
        L.spec_schedule_sts_run(sctx, lg, temps, ring[0], sps_a=2000.0, sps_k=4096.0)
        torch.cuda.synchronize()
        admitted.append(ring[0].cpu().numpy().astype("int64"))
    ctx.close()
    sctx.close()
    positions = sum(float(x.sum()) for x in admitted) / len(admitted)
    rows = sum(float((2 * x + 1).sum()) for x in admitted) / len(admitted)
    alg = rows * V * vi.p.element_size()
    kernels = {k: round(_mean_us(prof, k), 2) for k, v in prof.items() if v[1]}
    kernels["schedule (second stream)"] = round(_mean_us(sprof, "schedule"), 2)
    return _line("verified positions/s, B=512 gamma=8 V=129,280 bf16, block verification with the "
                 "temperature-scaled scheduler two steps ahead",
                 positions / (ms / 1e3), "verified positions/s", args, ms,
                 {"workload": "block verification; scheduler on temperature-scaled confidences, two steps "
                              "ahead on a second stream", "B": B, "gamma": gamma, "V": V, "logits": "bf16",
                  "sps": "2000/(1+n/4096)", "temperatures": [round(t, 3) for t in temps],
                  "input_sets": len(sets)},
                 _hbm_roofline("k_rowstats", alg, _mean_us(prof, "rowstats")),
                 mean_verify_len=round(positions / B, 4), kernels_mean_us=kernels)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--fused-only", action="store_true",
                    help="markov workload: time only the fused path (for clean per-kernel profiles)")
    ap.add_argument("--workload", default="headline",
                    choices=["headline", "tiny", "batched", "block", "block_async", "markov", "rnn", "tree",
                             "all"],
                    help="headline (default: one JSON line for the headline workload) or another workload")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(batch sharding across GPUs needs no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import lossless_draft_verification_02_amd as L
    from lossless_draft_verification_02_amd import workloads as WL

    torch.cuda.set_device(0)
    runs = {"headline": lambda: bench_headline(args, L, WL),
            "tiny": lambda: bench_token(args, L, WL, "tiny", 1),
            "batched": lambda: bench_token(args, L, WL, "batched", 4),
            "block": lambda: bench_block(args, L, WL),
            "block_async": lambda: bench_block_async(args, L, WL),
            "markov": lambda: bench_markov(args, L, WL),
            "rnn": lambda: bench_rnn(args, L, WL),
            "tree": lambda: bench_tree(args, L, WL)}
    names = list(runs) if args.workload == "all" else [args.workload]
    for n in names:
        line = runs[n]()
        if args.copy_probe and "copy_probe" not in line:
            line["copy_probe"] = _copy_probe()
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
