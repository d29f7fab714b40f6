"""ctypes binding of libspecverify.so (C ABI in include/spec_verify.h).

Argument marshalling only: every function takes torch tensors that already
live on the context's GPU, checks shapes / dtypes / contiguity, and passes
their device pointers and the current HIP stream to the C entry point of the
same name.  No computation happens here and there is no fallback: if the
library is not built or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SV_OK, SV_ERR_INVALID, SV_ERR_UNSUPPORTED, SV_ERR_HIP, SV_ERR_NOMEM = 0, 1, 2, 3, 4
SV_F32, SV_BF16 = 0, 1
SV_FLAG_BAD_TOKEN, SV_FLAG_BAD_ROW, SV_FLAG_RESID_ZERO, SV_FLAG_BAD_VERIFY_LEN = 1, 2, 4, 8

EXPORTED = ("spec_verify_create", "spec_verify_destroy", "spec_verify_last_error",
            "spec_verify_device_status", "spec_verify_run", "spec_verify_run_noalloc", "spec_schedule_run",
            "spec_schedule_sts_run",
            "spec_blockverify_run", "markov_draft_run", "markov_verify_run", "rnn_draft_run", "tree_verify_run",
            "spec_verify_profile_enable",
            "spec_verify_profile_read")
KERNELS = ("rowstats", "accept", "block_pass2", "resid", "select", "tail", "schedule", "markov_gemm",
           "markov_select", "markov_rebuild")


class SpecVerifyError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed (status {status}): {message}")
        self.status = status


class SvDiag(ctypes.Structure):
    _fields_ = [("lse_p", ctypes.c_void_p), ("lse_q", ctypes.c_void_p), ("ratio", ctypes.c_void_p),
                ("w", ctypes.c_void_p), ("h", ctypes.c_void_p), ("resid_mass", ctypes.c_void_p),
                ("flags", ctypes.c_void_p), ("uniform", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libspecverify.so and declares its signatures (raises if absent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run lossless_draft_verification_02_amd.build.build()")
    lib = ctypes.CDLL(path)
    P, I, I64, U64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
    lib.spec_verify_create.argtypes = [ctypes.POINTER(ctypes.c_void_p), I, I, I, I64, I]
    lib.spec_verify_create.restype = I
    lib.spec_verify_destroy.argtypes = [P]
    lib.spec_verify_destroy.restype = None
    lib.spec_verify_last_error.argtypes = []
    lib.spec_verify_last_error.restype = ctypes.c_char_p
    lib.spec_verify_device_status.argtypes = [P, P, ctypes.POINTER(ctypes.c_uint32)]
    lib.spec_verify_device_status.restype = I
    lib.spec_verify_run.argtypes = [P, P, P, I, P, I, P, P, I, I, I64, F, U64, U64, P, P, P, P]
    lib.spec_verify_run.restype = I
    lib.spec_verify_run_noalloc.argtypes = [P, P, I, P, I, P, P, I, I, I64, F, U64, U64, P, P, P, P]
    lib.spec_verify_run_noalloc.restype = I
    lib.spec_schedule_run.argtypes = [P, P, P, I, I, F, F, P, P]
    lib.spec_schedule_run.restype = I
    lib.spec_schedule_sts_run.argtypes = [P, P, P, P, I, I, F, F, P, P]
    lib.spec_schedule_sts_run.restype = I
    lib.spec_blockverify_run.argtypes = [P, P, P, I, P, I, P, P, P, F, F, P, I, I, I64, F, U64, U64, P,
                                         P, P, P]
    lib.spec_blockverify_run.restype = I
    lib.markov_draft_run.argtypes = [P, P, P, P, P, I, P, I, I, I64, F, U64, U64, P, P, P, P]
    lib.markov_verify_run.argtypes = [P, P, P, P, P, I, P, P, I, I, I, I64, F, U64, U64, U64, P, P, P, P, P]
    lib.markov_verify_run.restype = I
    lib.tree_verify_run.argtypes = [P, P, P, I, P, I, P, P, I, I, I64, F, U64, U64, P, P, P, P, P]
    lib.tree_verify_run.restype = I
    lib.rnn_draft_run.argtypes = [P, P, P, P, P, P, I, P, I, I, I64, F, U64, U64, P, P, P, P, P]
    lib.rnn_draft_run.restype = I
    lib.markov_draft_run.restype = I
    lib.spec_verify_profile_enable.argtypes = [P, I]
    lib.spec_verify_profile_enable.restype = I
    lib.spec_verify_profile_read.argtypes = [P, P, P]
    lib.spec_verify_profile_read.restype = I
    _lib = lib
    return lib


def spec_verify_last_error() -> str:
    return load_library().spec_verify_last_error().decode()


def _check(fn: str, status: int):
    if status != SV_OK:
        raise SpecVerifyError(fn, status, spec_verify_last_error())


# ----------------------------------------------------------- marshalling ---

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _need(t, name, dtype=None, shape=None, device=None):
    if t is None:
        return
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device.index != device:
        raise ValueError(f"{name} is on cuda:{t.device.index}, the context is on cuda:{device}")


def _stream(device: int, stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _diag_struct(diag: Optional[dict], device: int, shapes: dict):
    """sv_diag of the given tensors, each checked against `shapes` (entry name
    -> accepted shape, or a tuple of accepted shapes) before any launch: the
    kernels write every entry they are given."""
    if not diag:
        return None
    torch = _torch()
    unknown = sorted(set(diag) - set(shapes))
    if unknown:
        raise ValueError(f"unknown or unsupported diagnostics {unknown}; accepted: {sorted(shapes)}")
    for k, v in diag.items():
        if v is None:
            continue
        want = shapes[k]
        opts = want if isinstance(want[0], tuple) else (want,)
        dt = torch.int32 if k == "flags" else torch.float32
        _need(v, f"diag[{k!r}]", dtype=dt, device=device)
        if tuple(v.shape) not in [tuple(o) for o in opts]:
            raise ValueError(f"diag[{k!r}] must have shape {' or '.join(str(tuple(o)) for o in opts)}, "
                             f"got {tuple(v.shape)}")
    return SvDiag(**{k: _ptr(v) for k, v in diag.items()})


def _verify_diag_shapes(B: int, gamma: int) -> dict:
    """Diagnostic shapes of a draft verification call ([B, 0] or [B, 1] for
    the per-position entries when gamma = 0)."""
    g = ((B, gamma), (B, 1)) if gamma == 0 else (B, gamma)
    return dict(lse_p=(B, gamma + 1), lse_q=g, ratio=g, w=g, h=g, resid_mass=(B,), flags=(B,),
                uniform=(B, gamma + 1))


# ----------------------------------------------------------- entry points --

class Context:
    """Owns an sv_ctx handle (spec_verify_create / spec_verify_destroy)."""

    def __init__(self, device: int, max_batch: int, max_gamma: int, vocab: int, max_rank: int = 0):
        self.device = device
        self.max_batch, self.max_gamma, self.vocab, self.max_rank = max_batch, max_gamma, vocab, max_rank
        self._h = spec_verify_create(device, max_batch, max_gamma, vocab, max_rank)

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise ValueError("context is closed")
        return self._h

    def close(self):
        if self._h is not None:
            spec_verify_destroy(self._h)
            self._h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def spec_verify_create(device: int, max_batch: int, max_gamma: int, vocab: int, max_rank: int = 0):
    h = ctypes.c_void_p()
    _check("spec_verify_create",
           load_library().spec_verify_create(ctypes.byref(h), device, max_batch, max_gamma, vocab, max_rank))
    return h


def spec_verify_destroy(handle):
    load_library().spec_verify_destroy(handle)


def spec_verify_device_status(ctx: Context, stream=None) -> int:
    flags = ctypes.c_uint32(0)
    _check("spec_verify_device_status",
           load_library().spec_verify_device_status(ctx.handle, _stream(ctx.device, stream), ctypes.byref(flags)))
    return flags.value


def _verify_shapes(device: int, p, q, draft, accepted_len, out_tokens, verify_len, uniforms):
    torch = _torch()
    if p.dim() != 3:
        raise ValueError("p must be [B, gamma+1, V]")
    B, G1, V = p.shape
    gamma = G1 - 1
    _need(p, "p", device=device)
    if gamma > 0:
        _need(q, "q", shape=(B, gamma, V), device=device)
        _need(draft, "draft", dtype=torch.int32, shape=(B, gamma), device=device)
    _need(accepted_len, "accepted_len", dtype=torch.int32, shape=(B,), device=device)
    _need(out_tokens, "out_tokens", dtype=torch.int32, shape=(B, gamma + 1), device=device)
    _need(verify_len, "verify_len", dtype=torch.int32, shape=(B,), device=device)
    _need(uniforms, "uniforms", dtype=torch.float32, shape=(B, gamma + 1), device=device)
    return B, gamma, V


def spec_verify_run(ctx: Context, p, q, draft, accepted_len, out_tokens, *, temperature: float = 1.0,
                    seed: int = 1, offset: int = 0, verify_len=None, uniforms=None,
                    diag: Optional[dict] = None, stream=None):
    """Token-level verification into accepted_len [B] / out_tokens [B, gamma+1] (int32)."""
    B, gamma, V = _verify_shapes(ctx.device, p, q, draft, accepted_len, out_tokens, verify_len, uniforms)
    d = _diag_struct(diag, ctx.device, _verify_diag_shapes(B, gamma))
    qd = _dtype_code(q) if gamma > 0 else SV_BF16
    _check("spec_verify_run", load_library().spec_verify_run(
        ctx.handle, _stream(ctx.device, stream), _ptr(p), _dtype_code(p), _ptr(q) if gamma > 0 else None, qd,
        _ptr(draft) if gamma > 0 else None, _ptr(verify_len), B, gamma, V, temperature, seed, offset,
        _ptr(uniforms), _ptr(accepted_len), _ptr(out_tokens), ctypes.byref(d) if d else None))


def spec_verify_run_noalloc(p, q, draft, accepted_len, out_tokens, *, temperature: float = 1.0, seed: int = 1,
                            offset: int = 0, verify_len=None, uniforms=None, diag: Optional[dict] = None,
                            stream=None):
    """Token-level verification without a context or any allocation (the
    library's per-GPU scratch array), on p's device; calls that overlap on one
    GPU race."""
    torch = _torch()
    if p.dim() != 3 or not p.is_cuda:
        raise ValueError("p must be a GPU tensor [B, gamma+1, V]")
    dev = p.device.index
    B, gamma, V = _verify_shapes(dev, p, q, draft, accepted_len, out_tokens, verify_len, uniforms)
    d = _diag_struct(diag, dev, _verify_diag_shapes(B, gamma))
    qd = _dtype_code(q) if gamma > 0 else SV_BF16
    with torch.cuda.device(dev):
        _check("spec_verify_run_noalloc", load_library().spec_verify_run_noalloc(
            _stream(dev, stream), _ptr(p), _dtype_code(p), _ptr(q) if gamma > 0 else None, qd,
            _ptr(draft) if gamma > 0 else None, _ptr(verify_len), B, gamma, V, temperature, seed, offset,
            _ptr(uniforms), _ptr(accepted_len), _ptr(out_tokens), ctypes.byref(d) if d else None))


def spec_schedule_run(ctx: Context, conf, verify_len, *, sps_a: float = 2000.0, sps_k: float = 4096.0,
                      expected=None, stream=None):
    """Prefix scheduler: conf [B, gamma] fp32 -> verify_len [B] int32 (+ expected [1] fp64)."""
    torch = _torch()
    B, gamma = conf.shape
    _need(conf, "conf", dtype=torch.float32, device=ctx.device)
    _need(verify_len, "verify_len", dtype=torch.int32, shape=(B,), device=ctx.device)
    _need(expected, "expected", dtype=torch.float64, shape=(1,), device=ctx.device)
    _check("spec_schedule_run", load_library().spec_schedule_run(
        ctx.handle, _stream(ctx.device, stream), _ptr(conf), B, gamma, sps_a, sps_k, _ptr(verify_len),
        _ptr(expected)))


def spec_schedule_sts_run(ctx: Context, conf_logits, temperatures, verify_len, *, sps_a: float = 2000.0,
                          sps_k: float = 4096.0, expected=None, stream=None):
    """Prefix scheduler on temperature-scaled confidences: conf_logits [B, gamma]
    fp32 (device) and one temperature per position (host sequence of gamma
    floats) -> verify_len [B] int32 (+ expected [1] fp64)."""
    torch = _torch()
    B, gamma = conf_logits.shape
    _need(conf_logits, "conf_logits", dtype=torch.float32, device=ctx.device)
    _need(verify_len, "verify_len", dtype=torch.int32, shape=(B,), device=ctx.device)
    _need(expected, "expected", dtype=torch.float64, shape=(1,), device=ctx.device)
    temps = [float(t) for t in temperatures]
    if len(temps) != gamma:
        raise ValueError(f"spec_schedule_sts_run: {len(temps)} temperatures for gamma={gamma}")
    host = (ctypes.c_float * max(gamma, 1))(*temps)
    _check("spec_schedule_sts_run", load_library().spec_schedule_sts_run(
        ctx.handle, _stream(ctx.device, stream), _ptr(conf_logits), ctypes.cast(host, ctypes.c_void_p), B, gamma,
        sps_a, sps_k, _ptr(verify_len), _ptr(expected)))


def spec_blockverify_run(ctx: Context, p, q, draft, accepted_len, out_tokens, *, temperature: float = 1.0,
                         seed: int = 1, offset: int = 0, verify_len=None, conf=None, sps_a: float = 2000.0,
                         sps_k: float = 4096.0, verify_len_out=None, uniforms=None,
                         diag: Optional[dict] = None, stream=None):
    """Block verification (optionally scheduled by conf) into accepted_len / out_tokens."""
    torch = _torch()
    B, gamma, V = _verify_shapes(ctx.device, p, q, draft, accepted_len, out_tokens, verify_len, uniforms)
    _need(conf, "conf", dtype=torch.float32, shape=(B, gamma), device=ctx.device)
    _need(verify_len_out, "verify_len_out", dtype=torch.int32, shape=(B,), device=ctx.device)
    d = _diag_struct(diag, ctx.device, _verify_diag_shapes(B, gamma))
    qd = _dtype_code(q) if gamma > 0 else SV_BF16
    _check("spec_blockverify_run", load_library().spec_blockverify_run(
        ctx.handle, _stream(ctx.device, stream), _ptr(p), _dtype_code(p), _ptr(q) if gamma > 0 else None, qd,
        _ptr(draft) if gamma > 0 else None, _ptr(verify_len), _ptr(conf), sps_a, sps_k, _ptr(verify_len_out),
        B, gamma, V, temperature, seed, offset, _ptr(uniforms), _ptr(accepted_len), _ptr(out_tokens),
        ctypes.byref(d) if d else None))


def markov_draft_run(ctx: Context, base, U, Wt, x0, draft_out, *, q_logits=None, lse_q=None,
                     temperature: float = 1.0, seed: int = 0, offset: int = 0, uniforms=None, stream=None):
    """Markov-head sampler: base [B, gamma, V], U [V, R], Wt [V, R] (bf16; W stored vocabulary-major)
    -> draft_out [B, gamma]."""
    torch = _torch()
    B, gamma, V = base.shape
    R = U.shape[1]
    _need(base, "base", dtype=torch.bfloat16, device=ctx.device)
    _need(U, "U", dtype=torch.bfloat16, shape=(V, R), device=ctx.device)
    _need(Wt, "Wt", dtype=torch.bfloat16, shape=(V, R), device=ctx.device)
    _need(x0, "x0", dtype=torch.int32, shape=(B,), device=ctx.device)
    _need(draft_out, "draft_out", dtype=torch.int32, shape=(B, gamma), device=ctx.device)
    _need(q_logits, "q_logits", dtype=torch.float32, shape=(B, gamma, V), device=ctx.device)
    _need(lse_q, "lse_q", dtype=torch.float32, shape=(B, gamma), device=ctx.device)
    _need(uniforms, "uniforms", dtype=torch.float32, shape=(B, gamma), device=ctx.device)
    _check("markov_draft_run", load_library().markov_draft_run(
        ctx.handle, _stream(ctx.device, stream), _ptr(base), _ptr(U), _ptr(Wt), R, _ptr(x0), B, gamma, V,
        temperature, seed, offset, _ptr(uniforms), _ptr(draft_out), _ptr(q_logits), _ptr(lse_q)))


def tree_verify_run(ctx: Context, p, q, tokens, parents, accepted_len, out_tokens, *, accepted_nodes=None,
                    temperature: float = 1.0, seed: int = 1, offset: int = 0, uniforms=None,
                    diag: Optional[dict] = None, stream=None):
    """Tree verification: p [B, N+1, V], q [B, NQ, V] (rows of the nodes with
    children, node order), tokens [B, N], parents (host sequence of N ints,
    parents[m-1] in [0, m-1]) -> accepted_len [B], out_tokens [B, D+1]
    (+ accepted_nodes [B, D])."""
    torch = _torch()
    par = [int(x) for x in parents]
    N = len(par)
    if p.dim() != 3 or p.shape[1] != N + 1:
        raise ValueError("p must be [B, N+1, V]")
    B, _, V = p.shape
    NQ = len(set(par))
    depth = [0] * (N + 1)
    for m in range(1, N + 1):
        if not 0 <= par[m - 1] < m:
            raise ValueError(f"parents[{m - 1}]={par[m - 1]} must lie in [0, {m - 1}]")
        depth[m] = depth[par[m - 1]] + 1
    D = max(depth)
    _need(p, "p", shape=(B, N + 1, V), device=ctx.device)
    if N > 0:
        _need(q, "q", shape=(B, NQ, V), device=ctx.device)
        _need(tokens, "tokens", dtype=torch.int32, shape=(B, N), device=ctx.device)
    _need(accepted_len, "accepted_len", dtype=torch.int32, shape=(B,), device=ctx.device)
    _need(out_tokens, "out_tokens", dtype=torch.int32, shape=(B, D + 1), device=ctx.device)
    _need(accepted_nodes, "accepted_nodes", dtype=torch.int32, shape=(B, D), device=ctx.device)
    _need(uniforms, "uniforms", dtype=torch.float32, shape=(B, N + 1), device=ctx.device)
    nq = ((B, NQ), (B, 1)) if NQ == 0 else (B, NQ)
    nn = ((B, N), (B, 1)) if N == 0 else (B, N)
    d = _diag_struct(diag, ctx.device, dict(lse_p=(B, N + 1), lse_q=nq, ratio=nn, resid_mass=(B,), flags=(B,)))
    host = (ctypes.c_int32 * max(N, 1))(*par)
    _check("tree_verify_run", load_library().tree_verify_run(
        ctx.handle, _stream(ctx.device, stream), _ptr(p), _dtype_code(p), _ptr(q) if N > 0 else None,
        _dtype_code(q) if N > 0 else SV_F32, _ptr(tokens) if N > 0 else None, ctypes.cast(host, ctypes.c_void_p),
        N, B, V, temperature, seed, offset, _ptr(uniforms), _ptr(accepted_len), _ptr(out_tokens),
        _ptr(accepted_nodes), ctypes.byref(d) if d else None))


def rnn_draft_run(ctx: Context, base, U, Wt, A, x0, draft_out, *, q_logits=None, lse_q=None, states=None,
                  temperature: float = 1.0, seed: int = 0, offset: int = 0, uniforms=None, stream=None):
    """RNN-head sampler: as markov_draft_run plus the recurrent matrix A [R, R]
    (bf16); states [B, gamma, R] bf16 receives the state each position used."""
    torch = _torch()
    B, gamma, V = base.shape
    R = U.shape[1]
    _need(base, "base", dtype=torch.bfloat16, device=ctx.device)
    _need(U, "U", dtype=torch.bfloat16, shape=(V, R), device=ctx.device)
    _need(Wt, "Wt", dtype=torch.bfloat16, shape=(V, R), device=ctx.device)
    _need(A, "A", dtype=torch.bfloat16, shape=(R, R), device=ctx.device)
    _need(x0, "x0", dtype=torch.int32, shape=(B,), device=ctx.device)
    _need(draft_out, "draft_out", dtype=torch.int32, shape=(B, gamma), device=ctx.device)
    _need(q_logits, "q_logits", dtype=torch.float32, shape=(B, gamma, V), device=ctx.device)
    _need(lse_q, "lse_q", dtype=torch.float32, shape=(B, gamma), device=ctx.device)
    _need(states, "states", dtype=torch.bfloat16, shape=(B, gamma, R), device=ctx.device)
    _need(uniforms, "uniforms", dtype=torch.float32, shape=(B, gamma), device=ctx.device)
    _check("rnn_draft_run", load_library().rnn_draft_run(
        ctx.handle, _stream(ctx.device, stream), _ptr(base), _ptr(U), _ptr(Wt), _ptr(A), R, _ptr(x0), B, gamma,
        V, temperature, seed, offset, _ptr(uniforms), _ptr(draft_out), _ptr(q_logits), _ptr(lse_q),
        _ptr(states)))


def markov_verify_run(ctx: Context, base, U, Wt, x0, p, draft_out, accepted_len, out_tokens, *, lse_q=None,
                      temperature: float = 1.0, draft_seed: int = 0, verify_seed: int = 1, offset: int = 0,
                      diag: Optional[dict] = None, stream=None):
    """Markov-head draft, then token verification of it against p [B, gamma+1, V], without fp32 q."""
    torch = _torch()
    B, gamma, V = base.shape
    R = U.shape[1]
    _need(base, "base", dtype=torch.bfloat16, device=ctx.device)
    _need(U, "U", dtype=torch.bfloat16, shape=(V, R), device=ctx.device)
    _need(Wt, "Wt", dtype=torch.bfloat16, shape=(V, R), device=ctx.device)
    _need(x0, "x0", dtype=torch.int32, shape=(B,), device=ctx.device)
    _need(p, "p", shape=(B, gamma + 1, V), device=ctx.device)
    _need(draft_out, "draft_out", dtype=torch.int32, shape=(B, gamma), device=ctx.device)
    _need(accepted_len, "accepted_len", dtype=torch.int32, shape=(B,), device=ctx.device)
    _need(out_tokens, "out_tokens", dtype=torch.int32, shape=(B, gamma + 1), device=ctx.device)
    _need(lse_q, "lse_q", dtype=torch.float32, shape=(B, gamma), device=ctx.device)
    d = _diag_struct(diag, ctx.device, _verify_diag_shapes(B, gamma))
    _check("markov_verify_run", load_library().markov_verify_run(
        ctx.handle, _stream(ctx.device, stream), _ptr(base), _ptr(U), _ptr(Wt), R, _ptr(x0), _ptr(p),
        _dtype_code(p), B, gamma, V, temperature, draft_seed, verify_seed, offset, _ptr(draft_out),
        _ptr(accepted_len), _ptr(out_tokens), _ptr(lse_q), ctypes.byref(d) if d else None))


def spec_verify_profile_enable(ctx: Context, enable: bool = True):
    """Starts (or stops) per-kernel HIP-event timing inside the library."""
    _check("spec_verify_profile_enable", load_library().spec_verify_profile_enable(ctx.handle, int(enable)))


def spec_verify_profile_read(ctx: Context) -> dict:
    """{kernel name: (total_ms, launches)} since the last read (waits for the events)."""
    n = len(KERNELS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check("spec_verify_profile_read", load_library().spec_verify_profile_read(ctx.handle, ms, cnt))
    return {KERNELS[k]: (ms[k], cnt[k]) for k in range(n)}
