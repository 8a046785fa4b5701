"""Packed target rows on the GPU (needs an MI355X): P < capacity * T logit
rows, slot s's committed row t at row_offsets[s] + t, each slot's rows
followed directly by another slot's, compared with the oracle and with the
rectangular run over the same rows (bit for bit: only addresses differ)."""
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import full_vocab_logprob_amd as flp
    flp.lib()
    torch.cuda.set_device(0)
    yield


def pack(w: synth.Workload, seed: int = 0):
    """The committed rows of w in a shuffled slot order: (packed [P, V_pad], offsets, P)."""
    s = w.spec
    rng = np.random.default_rng(seed)
    e = np.where(w.requested != 0, np.clip(w.emitted, 0, s.T), 0)
    offsets = np.zeros(s.capacity, dtype=np.int32)
    P = 0
    for sl in rng.permutation(s.capacity):
        offsets[sl] = P
        P += int(e[sl])
    packed = np.empty((max(P, 1), s.V_pad), dtype=w.logits.dtype)
    for sl in range(s.capacity):
        packed[offsets[sl]:offsets[sl] + e[sl]] = w.logits[sl * s.T:sl * s.T + e[sl]]
    return packed, offsets, max(P, 1)


def run_packed(w: synth.Workload, packed: np.ndarray, offsets: np.ndarray, P: int):
    import full_vocab_logprob_amd as flp
    s = w.spec
    bf16 = s.dtype == synth.BF16
    plan = flp.Plan(s.capacity, s.T, s.V, s.V_pad, dtype=torch.bfloat16 if bf16 else torch.float32,
                    K=s.K, packed_rows=P)
    lg = torch.from_numpy(packed.view(np.int16) if bf16 else packed).cuda()
    lg = (lg.view(torch.bfloat16) if bf16 else lg).reshape(-1)
    d = H.to_device(w)
    ws = plan.workspace()
    out = plan.new_out(H.POISON)
    plan.run(lg, d["tokens"], d["emitted"], d["requested"], d["id_counts"], d["ids"], out, ws,
             row_offsets=torch.from_numpy(offsets).cuda())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_packed(o, w, packed, offsets, P):
    s = w.spec
    ref = w.poisoned_out()
    o.frame_packed(packed, s.capacity, s.T, P, s.V, s.V_pad, w.requested, w.id_counts, w.ids,
                   w.emitted, w.tokens, offsets, s.K, ref)
    return ref


CASES = [
    ("C3", dict(capacity=16)),
    ("C4", dict(capacity=16)),
    ("C2", dict()),
    ("C3", dict(capacity=5, T=3, V=40000, V_pad=40008, dtype=synth.FP32, recipe=synth.NORMAL,
                p0=3.0)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(CASES)])
def test_packed_matches_oracle_and_rectangular(oracle_handle, name, kw):
    spec = synth.CONFIGS[name].with_(**kw)
    announce(f"packed {spec.name} cap={spec.capacity} T={spec.T} V={spec.V} dtype={spec.dtype}")
    w = synth.make(spec)
    packed, offsets, P = pack(w, seed=spec.capacity)
    assert P < spec.capacity * spec.T
    got = run_packed(w, packed, offsets, P)
    ref = oracle_packed(oracle_handle, w, packed, offsets, P)
    H.compare_words(got, ref, f"packed {name}")
    rect, _ = H.run_gpu(w)
    assert np.array_equal(got, rect)


def test_packed_full_size_c3(oracle_handle):
    """All 128 slots of the verify frame packed into P = 621 rows: the same
    bytes as the rectangular run, and sampled rows against the oracle."""
    spec = synth.CONFIGS["C3"]
    announce("packed full-size C3")
    w = synth.make(spec)
    packed, offsets, P = pack(w, seed=3)
    got = run_packed(w, packed, offsets, P)
    rect, _ = H.run_gpu(w)
    assert np.array_equal(got, rect)
    # the two launches called apart give the same frame
    import full_vocab_logprob_amd as flp
    plan = flp.Plan(spec.capacity, spec.T, spec.V, spec.V_pad, dtype=torch.bfloat16, K=spec.K,
                    packed_rows=P)
    lg = torch.from_numpy(packed.view(np.int16)).cuda().view(torch.bfloat16).reshape(-1)
    d = H.to_device(w)
    ws = plan.workspace()
    out = plan.new_out(H.POISON)
    offs = torch.from_numpy(offsets).cuda()
    for phase in ("reduce", "merge"):
        plan.run(lg, d["tokens"], d["emitted"], d["requested"], d["id_counts"], d["ids"], out, ws,
                 phase=phase, row_offsets=offs)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), got)
    o = oracle_handle
    act = np.argwhere(w.active_mask())
    for sl, t in act[:: max(1, len(act) // 8)][:8]:
        words, _ = o.row(packed[offsets[sl] + t], token=int(w.tokens[sl * spec.T + t]), K=spec.K,
                         V=spec.V)
        H.compare_words(got[sl, t, :len(words)][None], words[None], f"packed row {sl},{t}")


def test_packed_out_of_range_slots_write_nothing(oracle_handle):
    """Slots whose committed rows would leave [0, P) (negative offset, or
    running past P) read and write nothing; the other slots are unchanged."""
    spec = synth.CONFIGS["C3"].with_(capacity=12, V=30000, V_pad=30000)
    announce("packed out-of-range offsets")
    w = synth.make(spec)
    packed, offsets, P = pack(w, seed=5)
    e = np.where(w.requested != 0, np.clip(w.emitted, 0, spec.T), 0)
    bad = [int(sl) for sl in np.nonzero(e > 0)[0][:2]]
    offsets[bad[0]] = -1
    offsets[bad[1]] = P - int(e[bad[1]]) + 1
    got = run_packed(w, packed, offsets, P)
    ref = oracle_packed(oracle_handle, w, packed, offsets, P)
    H.compare_words(got, ref, "packed out of range")
    assert np.all(got[bad[0]] == H.POISON) and np.all(got[bad[1]] == H.POISON)
