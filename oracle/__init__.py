"""CPU oracle for lossless speculative-sampling verification.

TEST INFRASTRUCTURE ONLY.  The GPU library never imports or calls this
package; only the tests, the smoke check and the benchmark's CPU-baseline leg
do.  The arithmetic lives in ``oracle.c`` (plain C, binary64, sequential
sums); this module builds it with gcc and marshals numpy arrays into it.

Every function here takes logits as float arrays of any float dtype; they are
widened exactly to float64 before the call.  Definitions and sources of each
step are in ``oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FLAG_BAD_TOKEN = 1
FLAG_BAD_ROW = 2
FLAG_RESID_ZERO = 4


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (strict IEEE: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", _LIB, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def declare(lib):
    """Declares the C signatures on a loaded oracle library."""
    P = ctypes.c_void_p
    i32, i64, u64, f32, f64 = (ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                               ctypes.c_float, ctypes.c_double)
    lib.orc_philox4x32_10.argtypes = [P, P, P]
    lib.orc_philox4x32_10.restype = None
    lib.orc_uniform.argtypes = [u64, u64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
    lib.orc_uniform.restype = f32
    lib.orc_row_lse.argtypes = [P, i64, f32, P]
    lib.orc_row_lse.restype = ctypes.c_uint32
    lib.orc_icdf.argtypes = [P, i64, f32, P, P]
    lib.orc_icdf.restype = i64
    verify_args = [P, P, P, P, P, i32, i32, i64, f32, u64, u64, P, P, P, P, P]
    lib.orc_token_verify.argtypes = verify_args
    lib.orc_token_verify.restype = i32
    lib.orc_block_verify.argtypes = verify_args
    lib.orc_block_verify.restype = i32
    lib.orc_schedule.argtypes = [P, i32, i32, f64, f64, P, P, P]
    lib.orc_schedule.restype = i32
    lib.orc_bf16.argtypes = [f32]
    lib.orc_bf16.restype = f32
    lib.orc_rnn_draft.argtypes = [P, P, P, P, i32, P, P, i32, i32, i64, f32, u64, u64,
                                  P, P, P, P, P, P, P, P]
    lib.orc_rnn_draft.restype = i32
    lib.orc_tree_depth.argtypes = [P, i32]
    lib.orc_tree_depth.restype = i32
    lib.orc_tree_verify.argtypes = [P, P, P, P, i32, P, i32, i64, f32, u64, u64, P, P, P, P, P, P, P, P]
    lib.orc_tree_verify.restype = i32
    lib.orc_sts_confidence.argtypes = [P, P, i32, i32, P]
    lib.orc_sts_confidence.restype = i32
    lib.orc_markov_draft.argtypes = [P, P, P, i32, P, P, i32, i32, i64, f32, u64, u64,
                                     P, P, P, P, P, P]
    lib.orc_markov_draft.restype = i32
    return lib


def build_sanitized(path: str) -> str:
    """Compile the oracle with AddressSanitizer and UndefinedBehaviorSanitizer
    into `path` (same arithmetic flags; any undefined behaviour aborts).  A
    process loads it through ORACLE_LIB, with libasan preloaded."""
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-Wall", "-Wextra", "-o", path, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return path


def _load():
    global _lib
    if _lib is None:
        alt = os.environ.get("ORACLE_LIB")
        if alt:   # a separately built oracle (the sanitizer build)
            _lib = declare(ctypes.CDLL(alt))
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = declare(ctypes.CDLL(_LIB))
    return _lib


class _Diag(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("lse_p", "lse_q", "ratio", "w", "h", "dec_margin", "resid_mass",
                 "icdf_margin", "uniform", "m")]


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a) -> Optional[np.ndarray]:
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _f32(a) -> Optional[np.ndarray]:
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def philox4x32_10(counter, key) -> np.ndarray:
    """One Philox4x32-10 block: counter (4 x u32), key (2 x u32) -> 4 x u32."""
    c = np.ascontiguousarray(np.asarray(counter, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    _load().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed: int, offset: int, req: int, pos: int, tag: int) -> float:
    return float(_load().orc_uniform(seed, offset, req, pos, tag))


def row_lse(row, temperature: float = 1.0):
    r = _f64(row)
    out = ctypes.c_double(0.0)
    fl = _load().orc_row_lse(_ptr(r), r.size, temperature, ctypes.byref(out))
    return (None if fl else out.value), int(fl)


def icdf(weights, u: float):
    """Returns (index, Z, margin)."""
    w = _f64(weights)
    Z = ctypes.c_double(0.0)
    m = ctypes.c_double(0.0)
    y = _load().orc_icdf(_ptr(w), w.size, u, ctypes.byref(Z), ctypes.byref(m))
    return int(y), Z.value, m.value


@dataclass
class VerifyResult:
    accepted_len: np.ndarray      # [B] int32, -1 for a request with a data error
    out_tokens: np.ndarray        # [B, gamma+1] int32, -1 padded
    flags: np.ndarray             # [B] uint32
    lse_p: np.ndarray             # [B, gamma+1]
    lse_q: np.ndarray             # [B, gamma]
    ratio: np.ndarray             # [B, gamma] min(1, p/q)
    w: np.ndarray                 # [B, gamma] block running ratio (NaN for token verify)
    h: np.ndarray                 # [B, gamma] block thresholds (NaN for token verify)
    dec_margin: np.ndarray        # [B, gamma]
    resid_mass: np.ndarray        # [B]
    icdf_margin: np.ndarray       # [B]
    uniform: np.ndarray           # [B, gamma+1]
    m: np.ndarray                 # [B, gamma] block residual masses m_i, i < L (NaN elsewhere)


def _verify(fn_name, p, q, draft, gamma, temperature=1.0, seed=1, offset=0,
            verify_len=None, req_ids=None, uniforms=None) -> VerifyResult:
    p = _f64(p)
    B = p.shape[0]
    V = p.shape[-1]
    if p.shape != (B, gamma + 1, V):
        raise ValueError(f"p must be [B, gamma+1, V], got {p.shape}")
    q = _f64(q) if gamma > 0 else np.zeros((B, 0, V))
    draft = _i32(draft) if gamma > 0 else np.zeros((B, 0), np.int32)
    if q.shape != (B, gamma, V) or draft.shape != (B, gamma):
        raise ValueError("q must be [B, gamma, V] and draft [B, gamma]")
    vl = _i32(verify_len)
    rid = _i32(req_ids)
    un = _f32(uniforms)
    acc = np.zeros(B, np.int32)
    out = np.zeros((B, gamma + 1), np.int32)
    flags = np.zeros(B, np.uint32)
    arrs = dict(lse_p=np.zeros((B, gamma + 1)), lse_q=np.zeros((B, gamma)),
                ratio=np.zeros((B, gamma)), w=np.zeros((B, gamma)), h=np.zeros((B, gamma)),
                dec_margin=np.zeros((B, gamma)), resid_mass=np.zeros(B),
                icdf_margin=np.zeros(B), uniform=np.zeros((B, gamma + 1), np.float32),
                m=np.full((B, gamma), np.nan))
    diag = _Diag(**{k: _ptr(v).value if v.size else None for k, v in arrs.items()})
    rc = getattr(_load(), fn_name)(_ptr(p), _ptr(q), _ptr(draft), _ptr(vl), _ptr(rid), B, gamma,
                                   V, temperature, seed, offset, _ptr(un), _ptr(acc), _ptr(out),
                                   _ptr(flags), ctypes.byref(diag))
    if rc != 0:
        raise ValueError(f"{fn_name}: invalid arguments")
    return VerifyResult(acc, out, flags, **arrs)


def token_verify(p, q, draft, gamma, **kw) -> VerifyResult:
    """Token-level verification; see orc_token_verify in oracle.h."""
    return _verify("orc_token_verify", p, q, draft, gamma, **kw)


def block_verify(p, q, draft, gamma, **kw) -> VerifyResult:
    """Block verification; see orc_block_verify in oracle.h."""
    return _verify("orc_block_verify", p, q, draft, gamma, **kw)


def schedule(conf, sps_a: float = 2000.0, sps_k: float = 4096.0):
    """Prefix scheduler.  Returns (verify_len [B] int32, expected, stop_margin)."""
    c = _f64(conf)
    B, gamma = c.shape
    vl = np.zeros(B, np.int32)
    e = ctypes.c_double(0.0)
    m = ctypes.c_double(0.0)
    rc = _load().orc_schedule(_ptr(c), B, gamma, sps_a, sps_k, _ptr(vl), ctypes.byref(e),
                              ctypes.byref(m))
    if rc != 0:
        raise ValueError("orc_schedule: invalid arguments")
    return vl, e.value, m.value


def sts_confidence(logits, temps):
    """Sequentially temperature-scaled confidences [B, gamma] (float64); see
    orc_sts_confidence in oracle.h."""
    lg = _f64(logits)
    t = _f64(temps).reshape(-1)
    B, gamma = lg.shape
    if t.shape[0] != gamma:
        raise ValueError("sts_confidence: one temperature per position is required")
    out = np.zeros((B, gamma), np.float64)
    if _load().orc_sts_confidence(_ptr(lg), _ptr(t), B, gamma, _ptr(out)) != 0:
        raise ValueError("orc_sts_confidence: invalid arguments")
    return out


@dataclass
class MarkovResult:
    draft: np.ndarray       # [B, gamma] int32
    q_logits: np.ndarray    # [B, gamma, V] float64 (before 1/T)
    lse_q: np.ndarray       # [B, gamma]
    margin: np.ndarray      # [B, gamma]
    flags: np.ndarray       # [B]


def markov_draft(base, U, W, x0, temperature=1.0, seed=0, offset=0, req_ids=None,
                 uniforms=None, want_q=True) -> MarkovResult:
    """Markov-head sampler; see orc_markov_draft in oracle.h."""
    base = _f64(base)
    U = _f64(U)
    W = _f64(W)
    B, gamma, V = base.shape
    R = U.shape[1]
    if U.shape != (V, R) or W.shape != (R, V):
        raise ValueError("U must be [V, R] and W [R, V]")
    x0 = _i32(x0)
    draft = np.zeros((B, gamma), np.int32)
    ql = np.zeros((B, gamma, V)) if want_q else None
    lse = np.zeros((B, gamma))
    marg = np.zeros((B, gamma))
    flags = np.zeros(B, np.uint32)
    rc = _load().orc_markov_draft(_ptr(base), _ptr(U), _ptr(W), R, _ptr(x0), _ptr(_i32(req_ids)),
                                  B, gamma, V, temperature, seed, offset, _ptr(_f32(uniforms)),
                                  _ptr(draft), _ptr(ql), _ptr(lse), _ptr(marg), _ptr(flags))
    if rc != 0:
        raise ValueError("orc_markov_draft: invalid arguments")
    return MarkovResult(draft, ql, lse, marg, flags)


@dataclass
class RnnResult:
    draft: np.ndarray         # [B, gamma] int32
    q_logits: np.ndarray      # [B, gamma, V] float64 (before 1/T)
    lse_q: np.ndarray         # [B, gamma]
    margin: np.ndarray        # [B, gamma] inverse-CDF margins
    flags: np.ndarray         # [B]
    states: np.ndarray        # [B, gamma, R] the bf16 states hb_k (as float64)
    state_margin: np.ndarray  # [B, gamma] ulps from the nearest bf16 rounding midpoint


def bf16(x: float) -> float:
    """bf16 rounding of a binary32 value; see orc_bf16 in oracle.h."""
    return float(_load().orc_bf16(float(x)))


def rnn_draft(base, U, W, A, x0, temperature=1.0, seed=0, offset=0, req_ids=None,
              uniforms=None, want_q=True) -> RnnResult:
    """RNN-head sampler; see orc_rnn_draft in oracle.h."""
    base = _f64(base)
    U = _f64(U)
    W = _f64(W)
    A = _f64(A)
    B, gamma, V = base.shape
    R = U.shape[1]
    if U.shape != (V, R) or W.shape != (R, V) or A.shape != (R, R):
        raise ValueError("U must be [V, R], W [R, V] and A [R, R]")
    x0 = _i32(x0)
    draft = np.zeros((B, gamma), np.int32)
    ql = np.zeros((B, gamma, V)) if want_q else None
    lse = np.zeros((B, gamma))
    marg = np.zeros((B, gamma))
    flags = np.zeros(B, np.uint32)
    states = np.zeros((B, gamma, R))
    smarg = np.zeros((B, gamma))
    rc = _load().orc_rnn_draft(_ptr(base), _ptr(U), _ptr(W), _ptr(A), R, _ptr(x0), _ptr(_i32(req_ids)),
                               B, gamma, V, temperature, seed, offset, _ptr(_f32(uniforms)),
                               _ptr(draft), _ptr(ql), _ptr(lse), _ptr(marg), _ptr(flags), _ptr(states),
                               _ptr(smarg))
    if rc != 0:
        raise ValueError("orc_rnn_draft: invalid arguments")
    return RnnResult(draft, ql, lse, marg, flags, states, smarg)


@dataclass
class TreeResult:
    accepted_len: np.ndarray     # [B]
    out_tokens: np.ndarray       # [B, D+1]
    accepted_nodes: np.ndarray   # [B, D]
    flags: np.ndarray            # [B]
    ratio: np.ndarray            # [B, N]
    dec_margin: np.ndarray       # [B, N]
    icdf_margin: np.ndarray      # [B]


def tree_depth(parents) -> int:
    par = _i32(parents)
    d = _load().orc_tree_depth(_ptr(par), len(par))
    if d < 0:
        raise ValueError("invalid tree: parents[m-1] must lie in [0, m-1]")
    return d


def tree_verify(p, q, tokens, parents, temperature=1.0, seed=0, offset=0, req_ids=None,
                uniforms=None) -> TreeResult:
    """Tree verification; see orc_tree_verify in oracle.h."""
    p = _f64(p)
    B, N1, V = p.shape
    N = N1 - 1
    par = _i32(parents)
    if len(par) != N:
        raise ValueError("one parent per non-root node")
    D = tree_depth(par)
    NQ = len(set(int(x) for x in par))
    q = _f64(q) if NQ else np.zeros((B, 0, V))
    if q.shape != (B, NQ, V):
        raise ValueError(f"q must be [B, {NQ}, V]: one row per node with children")
    tok = _i32(tokens).reshape(B, N) if N else np.zeros((B, 0), np.int32)
    acc = np.zeros(B, np.int32)
    out = np.zeros((B, D + 1), np.int32)
    nodes = np.zeros((B, max(D, 1)), np.int32)
    flags = np.zeros(B, np.uint32)
    ratio = np.zeros((B, max(N, 1)))
    dm = np.zeros((B, max(N, 1)))
    im = np.zeros(B)
    rc = _load().orc_tree_verify(_ptr(p), _ptr(q), _ptr(tok), _ptr(par), N, _ptr(_i32(req_ids)), B, V,
                                 temperature, seed, offset, _ptr(_f32(uniforms)), _ptr(acc), _ptr(out),
                                 _ptr(nodes), _ptr(flags), _ptr(ratio), _ptr(dm), _ptr(im))
    if rc != 0:
        raise ValueError("orc_tree_verify: invalid arguments")
    return TreeResult(acc, out, nodes[:, :D], flags, ratio[:, :N], dm[:, :N], im)
