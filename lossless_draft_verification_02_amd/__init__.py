"""Lossless speculative-sampling verification on AMD MI355X (gfx950).

The computation lives in libspecverify.so (hand-written HIP kernels behind the
C ABI declared in include/spec_verify.h); this package builds it
(``build.build()``), binds it (``binding``) and provides seeded synthetic
inputs (``workloads``).
"""
from .binding import (Context, SpecVerifyError, load_library, markov_draft_run, markov_verify_run, rnn_draft_run, tree_verify_run,
                      spec_blockverify_run,
                      spec_schedule_run, spec_schedule_sts_run, spec_verify_create, spec_verify_destroy,
                      spec_verify_device_status, spec_verify_last_error, spec_verify_profile_enable,
                      spec_verify_profile_read, spec_verify_run, spec_verify_run_noalloc)

__all__ = ["Context", "SpecVerifyError", "load_library", "spec_verify_create", "spec_verify_destroy",
           "markov_verify_run", "rnn_draft_run", "tree_verify_run", "spec_verify_last_error", "spec_verify_device_status", "spec_verify_run", "spec_verify_run_noalloc", "spec_schedule_run",
           "spec_schedule_sts_run",
           "spec_blockverify_run", "markov_draft_run", "spec_verify_profile_enable",
           "spec_verify_profile_read"]
