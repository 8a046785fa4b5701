"""Vocabulary-sharded reduction on one GPU (shard passes, exchange records,
cross-shard merge) against the oracle (needs an MI355X).

The frame a sharded call writes is the frame the unsharded definition gives:
IDs, ordering, padding and layout bit-exact, values within 2e-5.  Only the
order in which L's FP32 partial sums are combined differs from the unsharded
kernels, so against the unsharded run the IDs are identical and the values
agree bit for bit wherever the two L agree.  Every test prints its case first.
"""
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


def sharded_plan(spec, shards):
    import full_vocab_logprob_amd as flp
    return flp.Plan(spec.capacity, spec.T, spec.V, spec.V_pad,
                    dtype=torch.bfloat16 if spec.dtype == synth.BF16 else torch.float32,
                    K=spec.K, device=torch.cuda.current_device(), shards=shards)


def run_sharded(w, shards, d=None, phase_by_phase=False):
    """One sharded frame; returns (out, lse, guard, plan, workspace)."""
    d = d if d is not None else H.to_device(w)
    plan = sharded_plan(w.spec, shards)
    ws = plan.workspace()
    out = plan.new_out(H.POISON)
    args = (d["logits"], d["tokens"], d["emitted"], d["requested"], d["id_counts"], d["ids"], out,
            ws)
    if phase_by_phase:
        for r in range(shards):
            plan.run(*args, phase=f"shard:{r}")
        plan.run(*args, phase="merge")
    else:
        plan.run(*args)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), plan.lse(ws).cpu().numpy().copy(),
            plan.guard(ws).cpu().numpy().copy(), plan, ws)


def compare_with_unsharded(w, got, lse, where):
    """IDs identical to the unsharded run; values bit-identical where L is."""
    ref, ref_lse = H.run_gpu(w)
    assert np.array_equal(got[..., 0::2], ref[..., 0::2]), f"{where}: IDs differ from unsharded"
    same_L = lse.view(np.int32) == ref_lse.view(np.int32)
    act = w.active_mask().reshape(-1)
    rows = np.nonzero(act & same_L)[0]
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    assert np.array_equal(g[rows], r[rows]), f"{where}: values differ although L agrees"
    return int((act & ~same_L).sum())


def test_sharded_c3_full_size_every_row(oracle_handle):
    spec = synth.CONFIGS["C3"]
    announce(f"sharded C3 full size, 8 shards of {spec.V // 8} lanes")
    w = synth.make(spec)
    got, lse, guard, _, _ = run_sharded(w, 8)
    act = np.nonzero(w.active_mask().reshape(-1))[0]
    worst, worst_L, L_differ = H.compare_rows_with_oracle(oracle_handle, w, got, lse, act,
                                                          "sharded C3")
    H.check_properties(w, got, lse)
    n_diff_L = compare_with_unsharded(w, got, lse, "sharded C3")
    announce(f"sharded C3: {act.size} rows exact; max |d logprob| {worst:.3g}, L bits differ "
             f"from the oracle on {L_differ} rows and from the unsharded run on {n_diff_L}; "
             f"guard rescans {int(guard[act].sum())} shards")


@pytest.mark.parametrize("name,shards,kw", [
    ("C1", 4, {}),
    ("C2", 8, {}),
    ("C4", 8, dict(capacity=16)),
    ("C4", 3, dict(capacity=12, seed=14)),
    ("C5", 8, dict(capacity=4)),
    ("C5", 5, dict(capacity=3, K=0)),
    ("C5", 8, dict(capacity=3, selected="all")),
    ("C3", 32, dict(capacity=4, T=8)),
], ids=["C1x4", "C2x8", "C4x8", "C4x3", "C5x8", "C5x5_K0", "C5x8_sel128", "C3x32"])
def test_sharded_configs(oracle_handle, name, shards, kw):
    spec = synth.CONFIGS[name].with_(**kw)
    announce(f"sharded {name} x{shards} cap={spec.capacity} T={spec.T} V={spec.V} K={spec.K} {kw}")
    w = synth.make(spec)
    got, lse, guard, _, _ = run_sharded(w, shards)
    H.compare_words(got, H.oracle_frame(oracle_handle, w), f"sharded {name}")
    H.check_properties(w, got, lse)
    compare_with_unsharded(w, got, lse, f"sharded {name}")


def test_one_shard_is_the_unsharded_frame():
    """With a single shard the records carry the unsharded partial sums in the
    same order, so the frame and L equal the unsharded run bit for bit."""
    spec = synth.CONFIGS["C4"].with_(capacity=10, seed=21)
    announce("one shard vs unsharded C4 cap=10")
    w = synth.make(spec)
    got, lse, _, _, _ = run_sharded(w, 1)
    ref, ref_lse = H.run_gpu(w)
    assert np.array_equal(got, ref)
    act = w.active_mask().reshape(-1)  # L is written for active rows only
    assert np.array_equal(lse[act].view(np.int32), ref_lse[act].view(np.int32))


def test_shard_passes_then_merge_equal_run(oracle_handle):
    """Each rank's pass called on its own, then the merge, gives run_sharded's
    frame bit for bit."""
    spec = synth.CONFIGS["C3"].with_(capacity=6, T=8, seed=33)
    announce("shard passes one by one, then merge, C3 cap=6 x8")
    w = synth.make(spec)
    d = H.to_device(w)
    a, la, _, _, _ = run_sharded(w, 8, d)
    b, lb, _, _, _ = run_sharded(w, 8, d, phase_by_phase=True)
    act = w.active_mask().reshape(-1)
    assert np.array_equal(a, b) and np.array_equal(la[act].view(np.int32), lb[act].view(np.int32))
    H.compare_words(a, H.oracle_frame(oracle_handle, w), "passes then merge")


def test_exchange_records_hold_what_a_rank_sends():
    """Each shard's record: its max exactly, its exponential sum relative to
    that max (float64 check within FP32 rounding), the chosen token's raw
    logit and ownership flag on its owner only, and best keys whose first K
    are the shard's exact top K by (raw value desc, global ID asc); selected
    rows carry the owned IDs' raw logits and their ownership bits."""
    import full_vocab_logprob_amd as flp
    spec = synth.CONFIGS["C4"].with_(capacity=8, T=2, seed=27)
    shards = 5
    announce(f"exchange records C4 cap=8 T=2 x{shards}")
    w = synth.make(spec)
    _, _, _, plan, ws = run_sharded(w, shards)
    rec = plan.exchange(ws).cpu().numpy()  # int32 [rows, shards, 138]
    b = flp.shard_bounds(spec.V, shards)
    act = np.nonzero(w.active_mask().reshape(-1))[0]
    checked = 0
    for r in act:
        sl = int(r) // spec.T
        n = int(np.clip(w.id_counts[sl], 0, 128))
        x = H.row_floats(w, int(r)).astype(np.float32)
        tok = int(w.tokens[r])
        for k in range(shards):
            lo, hi = b[k], b[k + 1]
            words = rec[r, k]
            m = words[0:1].view(np.float32)[0]
            ssum = words[1:2].view(np.float32)[0]
            seg = x[lo:hi].astype(np.float64)
            assert m == np.float32(seg.max()), (r, k)
            if np.isfinite(m):
                want = np.exp(seg - float(m)).sum()
                assert abs(float(ssum) - want) <= 1e-5 * want, (r, k, float(ssum), want)
            owns = lo <= tok < hi
            assert (words[3] & 1) == (1 if owns else 0)
            if owns:
                assert words[2:3].view(np.float32)[0] == x[tok]
            if n > 0:
                ids = w.ids[sl * 128: sl * 128 + n]
                mask = words[134:138].view(np.uint32)
                sel = words[6:134].view(np.float32)
                for j, i in enumerate(ids):
                    own = lo <= i < hi
                    assert bool((mask[j >> 5] >> (j & 31)) & 1) == own
                    if own:
                        assert sel[j] == x[i]
            elif spec.K > 0:
                keys = words[6:70].view(np.uint64)
                vals = seg.astype(np.float32)
                order = np.lexsort((np.arange(lo, hi), -vals))[:spec.K]
                kv = keys[:spec.K]
                ids_got = (~(kv & np.uint64(0xFFFFFFFF)).astype(np.uint32)).astype(np.int64)
                assert np.array_equal(ids_got, order + lo), (r, k)
            checked += 1
    announce(f"{checked} shard records checked")


@pytest.mark.parametrize("dtype", [synth.FP32, synth.BF16], ids=["fp32", "bf16"])
def test_sharded_guard_trips_inside_a_shard(oracle_handle, dtype):
    """Shard 1 holds 33 distinct logits that all report the same value after
    subtracting L (one dominant lane in shard 0 sets L).  The shard keeps the
    largest 32 raw keys and drops the smallest, which has the smallest ID and
    so belongs in the top K; its cut must fail the guard and the merge must
    stream shard 1 again."""
    V, shards = 4 * 16384, 4
    row = np.full(V, -np.inf, np.float32)
    lo = V // shards
    if dtype == synth.FP32:
        base = np.float32(1.0)
        for k in range(33):
            row[lo + k] = base  # the smallest logit at the smallest ID
            base = np.nextafter(base, np.float32(2.0))
        row[7] = 100.0
    else:
        for k in range(33):
            row[lo + k] = np.float32((k + 1) * 2.0 ** -30)
        row[7] = 10.0
    announce(f"sharded guard trip dtype={dtype}")
    from test_parity_gpu import _frame_from_rows
    w = _frame_from_rows(row[None, :], dtype, K=20)
    got, lse, guard, _, _ = run_sharded(w, shards)
    ref = H.oracle_frame(oracle_handle, w)
    H.compare_words(got, ref, "sharded guard")
    assert ref[0, 0, 2] == 7 and ref[0, 0, 4] == lo  # the smallest ID of the tie group second
    assert guard[0] >= 1


def test_sharded_invalid_ids_and_gating(oracle_handle):
    spec = synth.CONFIGS["C3"].with_(capacity=6, T=3, V=20000, V_pad=20000, seed=31)
    w = synth.make(spec)
    w.requested[:] = [1, 0, 1, 1, 1, 1]
    w.emitted[:] = [2, 3, 0, 9, -4, 3]
    w.id_counts[:] = [-5, 4, 3, 0, 0, 300]
    w.ids[5 * 128:6 * 128] = np.arange(128) * 150
    w.ids[5 * 128 + 3] = -1
    w.ids[5 * 128 + 4] = 20000
    w.ids[5 * 128 + 5] = 2**31 - 1
    w.tokens[3 * 3 + 1] = -7
    w.tokens[3 * 3 + 2] = 20000
    announce("sharded gating clamps and invalid ids x6")
    got, lse, _, _, _ = run_sharded(w, 6)
    H.compare_words(got, H.oracle_frame(oracle_handle, w), "sharded gating")
