"""The completion-records adapter on the GPU (needs an MI355X): emitted
counts and tokens read from int64 records [capacity, 16 + T], with and
without ID inputs (rows of 258 or 2 + 2K words), against the oracle and bit
for bit against the int32-input run."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import synth
import gpu_harness as H

pytestmark = pytest.mark.gpu
FIELD = 9  # the record field holding the emitted count in these tests


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import full_vocab_logprob_amd as flp
    flp.lib()
    torch.cuda.set_device(0)
    yield


def records_of(w: synth.Workload, seed=1):
    s = w.spec
    rng = np.random.default_rng(seed)
    rec = rng.integers(-2**40, 2**40, size=(s.capacity, 16 + s.T)).astype(np.int64)
    rec[:, FIELD] = w.emitted
    rec[:, 16:] = w.tokens.reshape(s.capacity, s.T)
    return rec


@pytest.mark.parametrize("name,kw,with_ids", [
    ("C3", dict(capacity=12), True), ("C4", dict(capacity=16), True),
    ("C3", dict(capacity=12), False), ("C2", dict(), False),
])
def test_records_adapter(oracle_handle, name, kw, with_ids):
    spec = synth.CONFIGS[name].with_(**kw)
    announce(f"records {name} {kw} ids={with_ids}")
    w = synth.make(spec)
    rec = records_of(w)
    # a few out-of-range fields: a huge count (slot inactive), a token beyond int32
    e = np.clip(w.emitted, 0, spec.T)
    act = [s for s in range(spec.capacity) if w.requested[s] and e[s] > 0]
    rec[act[0], FIELD] = 2**40 + 2
    rec[act[1], 16] = 2**33
    d = H.to_device(w)
    plan = H.make_plan(spec)
    words = 258 if with_ids else 2 + 2 * spec.K
    out = torch.full((spec.capacity * spec.T * words,), H.POISON, dtype=torch.int32,
                     device="cuda")
    plan.run_records(d["logits"], torch.from_numpy(rec).cuda(), d["requested"], out,
                     plan.workspace(), FIELD, id_counts=d["id_counts"] if with_ids else None,
                     ids=d["ids"] if with_ids else None)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(spec.capacity, spec.T, words)
    ref = np.full((spec.capacity, spec.T, words), H.POISON, dtype=np.int32)
    oracle_handle.frame_records(w.logits, spec.capacity, spec.T, spec.V, spec.V_pad, w.requested,
                                w.id_counts if with_ids else None, w.ids if with_ids else None,
                                rec, FIELD, spec.K, ref)
    H.compare_words(got, ref, f"records {name}")
    assert np.all(got[act[0]] == H.POISON)
    assert got[act[1], 0, 0] == -1
    # the int32-input run over the same values gives the same words
    w2 = synth.Workload(spec, w.logits, w.requested.copy(), w.emitted.copy(), w.tokens.copy(),
                        w.id_counts.copy() if with_ids else np.zeros_like(w.id_counts),
                        w.ids.copy())
    w2.emitted[act[0]] = 0
    w2.tokens[act[1] * spec.T] = -1
    rect, _ = H.run_gpu(w2)
    assert np.array_equal(got, rect[:, :, :words])
