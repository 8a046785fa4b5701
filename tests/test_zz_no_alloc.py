"""flare_logprobs_run_noalloc (the library's static scratch, no workspace)
against flare_logprobs_run with a workspace, through the C ABI (needs an
MI355X).  Two calls in a row, the second with a smaller input, each equal bit
for bit to the workspace run (the same kernels), and a plan too large for the
scratch rejected before any launch."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import synth
import gpu_harness as H

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def noalloc_frame(w):
    import full_vocab_logprob_amd as flp
    s = w.spec
    plan = H.make_plan(s)
    d = H.to_device(w)
    out = plan.new_out(H.POISON)
    flp.flare_logprobs_run_noalloc(plan.raw, d["logits"], plan.torch_dtype, s.capacity * s.T, s.V,
                                   s.V_pad, d["requested"], d["id_counts"], d["ids"], d["emitted"],
                                   d["tokens"], s.K, out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), d, plan


def test_noalloc_matches_workspace_run_twice_then_smaller(oracle_handle):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    for spec in (synth.CONFIGS["C4"].with_(capacity=24, seed=71),
                 synth.CONFIGS["C3"].with_(capacity=3, T=5, V=50001, V_pad=50008, seed=72)):
        announce(f"noalloc {spec.name} cap={spec.capacity} T={spec.T} V={spec.V}")
        w = synth.make(spec)
        got, d, plan = noalloc_frame(w)
        assert plan.workspace_bytes <= 16 << 20
        ref, _ = H.run_gpu(w, dev_inputs=d)
        assert np.array_equal(got, ref), spec.name
        H.compare_words(got, H.oracle_frame(oracle_handle, w), f"noalloc {spec.name}")


def test_noalloc_rejects_a_plan_beyond_the_scratch():
    import full_vocab_logprob_amd as flp
    spec = synth.CONFIGS["C5"]  # 4,096 rows x 32 units of part records: 37 MB
    plan = H.make_plan(spec)
    assert plan.workspace_bytes > 16 << 20
    fake = 0x10000  # never dereferenced: the size check comes first
    rc = flp.lib().flare_logprobs_run_noalloc(
        plan.raw, fake, 0, spec.capacity * spec.T, spec.V, spec.V_pad, fake, fake, fake, fake,
        fake, spec.K, fake, None)
    assert rc == 7 and flp.flare_status_string(rc).startswith("the plan's workspace exceeds")
