"""The allocation-free token verification (spec_verify_run_noalloc) against
spec_verify_run through the C ABI: the same kernels on the same inputs, so
every output and diagnostic must be identical, bit for bit.  Two calls in a
row, the second with a smaller input, so the second runs on scratch the
first left behind; then the size limit and argument errors."""
import numpy as np
import pytest
import torch

import lossless_draft_verification_02_amd as L
from lossless_draft_verification_02_amd import workloads as WL

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _outputs(B, gamma):
    dev = "cuda"
    return dict(acc=torch.full((B,), -7, dtype=torch.int32, device=dev),
                out=torch.full((B, gamma + 1), -7, dtype=torch.int32, device=dev),
                diag=dict(lse_p=torch.full((B, gamma + 1), -7.0, device=dev),
                          lse_q=torch.full((B, max(gamma, 1)), -7.0, device=dev),
                          ratio=torch.full((B, max(gamma, 1)), -7.0, device=dev),
                          resid_mass=torch.full((B,), -7.0, device=dev),
                          flags=torch.full((B,), -7, dtype=torch.int32, device=dev),
                          uniform=torch.full((B, gamma + 1), -7.0, device=dev)))


def _run_both(vi, offset, verify_len=None):
    B, gamma, V = vi.B, vi.gamma, vi.V
    ref, got = _outputs(B, gamma), _outputs(B, gamma)
    with L.Context(0, B, gamma, V) as ctx:
        L.spec_verify_run(ctx, vi.p, vi.q, vi.draft, ref["acc"], ref["out"], temperature=vi.T, seed=WL.VERIFY_SEED,
                          offset=offset, verify_len=verify_len, diag=ref["diag"])
        torch.cuda.synchronize()
    L.spec_verify_run_noalloc(vi.p, vi.q, vi.draft, got["acc"], got["out"], temperature=vi.T, seed=WL.VERIFY_SEED,
                              offset=offset, verify_len=verify_len, diag=got["diag"])
    torch.cuda.synchronize()
    assert torch.equal(ref["acc"], got["acc"]), "accepted_len differs"
    assert torch.equal(ref["out"], got["out"]), "out_tokens differs"
    for k in ref["diag"]:
        a, b = ref["diag"][k].cpu().numpy(), got["diag"][k].cpu().numpy()
        assert np.array_equal(a.view(np.int32), b.view(np.int32)), f"diag {k} differs"
    acc = got["acc"].cpu().numpy()
    return float(acc[acc >= 0].mean())


@pytest.mark.parametrize("first,second", [(("headline", 256, 7, 129280), ("headline", 40, 5, 40000)),
                                          (("batched", 32, 5, 151936), ("tiny", 1, 4, 1000))])
def test_noalloc_matches_context_call_twice(first, second):
    """The full headline (or batched) batch, then a smaller one on the same scratch."""
    for k, (wl, B, gamma, V) in enumerate((first, second)):
        _say(f"case: noalloc call {k + 1}: {wl} B={B} gamma={gamma} V={V}")
        vi = WL.make_verify_inputs(wl, "cuda", B=B, gamma=gamma, V=V)
        m = _run_both(vi, offset=3 + k)
        _say(f"  identical outputs; mean accepted {m:.3f}")


def test_noalloc_split_tail_and_verify_lengths():
    """A small batch over many segments takes the split tail (its segment
    sums in the scratch array); verify lengths take the compacted row pass."""
    B, gamma, V = 6, 4, 40000
    _say(f"case: noalloc split tail B={B} gamma={gamma} V={V}, with verify lengths")
    vi = WL.make_verify_inputs("headline", "cuda", B=B, gamma=gamma, V=V)
    _run_both(vi, offset=1)
    vl = torch.tensor([0, 4, 2, 1, 3, 4], dtype=torch.int32, device="cuda")
    _run_both(vi, offset=2, verify_len=vl)


def test_noalloc_rejects_a_call_beyond_its_scratch():
    """8 MiB of scratch: B=4096, gamma=16, V=129,280 needs more; nothing is launched."""
    B, gamma, V = 4096, 16, 129280
    _say(f"case: noalloc size limit B={B} gamma={gamma} V={V}")
    # the limit is checked on the host before anything is launched, so small
    # stand-in buffers are enough for the C call
    lib = L.load_library()
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, gamma + 1, dtype=torch.int32, device="cuda")
    d = torch.zeros(B, gamma, dtype=torch.int32, device="cuda")
    buf = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    st = lib.spec_verify_run_noalloc(torch.cuda.current_stream().cuda_stream, buf.data_ptr(), L.binding.SV_BF16,
                                     buf.data_ptr(), L.binding.SV_BF16, d.data_ptr(), None, B, gamma, V, 1.0, 1, 0,
                                     None, acc.data_ptr(), out.data_ptr(), None)
    assert st == L.binding.SV_ERR_UNSUPPORTED, st
    msg = L.spec_verify_last_error()
    assert "scratch" in msg and "maximum" in msg, msg
    st = lib.spec_verify_run_noalloc(torch.cuda.current_stream().cuda_stream, buf.data_ptr(), L.binding.SV_BF16,
                                     buf.data_ptr(), L.binding.SV_BF16, d.data_ptr(), None, 4, 65, 1000, 1.0, 1, 0,
                                     None, acc.data_ptr(), out.data_ptr(), None)
    assert st == L.binding.SV_ERR_INVALID, st
