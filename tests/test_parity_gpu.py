"""Parity of the HIP path with the CPU oracle (needs an MI355X).

Every test prints the case it runs before touching the GPU.  Inputs come from
the seeded generator; expected values come from the oracle only.
"""
from __future__ import annotations

import json
import glob
import os
import sys

import numpy as np
import pytest
import torch

import synth
import gpu_harness as H

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import full_vocab_logprob_amd as flp
    flp.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    yield


def full_compare(o, spec, **kw):
    announce(f"full compare {spec.name} cap={spec.capacity} T={spec.T} V={spec.V} "
             f"V_pad={spec.V_pad} dtype={spec.dtype} K={spec.K} {kw}")
    w = synth.make(spec)
    got, lse = H.run_gpu(w)
    ref = H.oracle_frame(o, w)
    H.compare_words(got, ref, spec.name)
    H.check_properties(w, got, lse)
    return w, got, ref, lse


# ------------------------------------------------------------ named workloads
def test_c1_decode_full(oracle_handle):
    full_compare(oracle_handle, synth.CONFIGS["C1"])
    full_size_all_rows(oracle_handle, synth.CONFIGS["C1"])


def test_c2_padded_half_requesting_full(oracle_handle):
    full_compare(oracle_handle, synth.CONFIGS["C2"])
    full_size_all_rows(oracle_handle, synth.CONFIGS["C2"])


@pytest.mark.parametrize("cap,T", [(8, 8), (3, 5)])
def test_c3_verify_reduced(oracle_handle, cap, T):
    full_compare(oracle_handle, synth.CONFIGS["C3"].with_(capacity=cap, T=T))


def test_c4_ties_and_selected_reduced(oracle_handle):
    w, got, ref, lse = full_compare(oracle_handle, synth.CONFIGS["C4"].with_(capacity=16))
    assert (w.id_counts > 0).sum() == 6


@pytest.mark.parametrize("variant", ["K20", "K0", "sel128"])
def test_c5_large_batch_reduced(oracle_handle, variant):
    spec = synth.CONFIGS["C5"].with_(capacity=4)
    if variant == "K0":
        spec = spec.with_(K=0)
    elif variant == "sel128":
        spec = spec.with_(selected="all")
    full_compare(oracle_handle, spec)


@pytest.mark.parametrize("K", [2, 5, 13])
@pytest.mark.parametrize("name", ["C3", "C4"])
def test_k_sweep_reduced(oracle_handle, name, K):
    # The admission bars and the parts' cuts rank by K; few rows spread each
    # row over several parts.
    full_compare(oracle_handle, synth.CONFIGS[name].with_(capacity=6, K=K, seed=60 + K))


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP32], ids=["bf16", "fp32"])
def test_many_ranges_per_row(oracle_handle, dtype):
    # About 1,150 active rows of 4 units each: several workgroup ranges start
    # inside most rows, at positions the merge recomputes from the partition.
    spec = synth.CONFIGS["C3"].with_(capacity=256, T=8, V=3 * 16384 + 5, V_pad=3 * 16384 + 8,
                                     dtype=dtype, seed=91)
    full_compare(oracle_handle, spec)


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP32], ids=["bf16", "fp32"])
def test_row_pieces_with_extra_pieces(oracle_handle, dtype):
    # About 500 active rows of 8 units: two pieces per row would leave about
    # 270 workgroups idle, so the partition cuts the last rows into three
    # pieces (the extra pieces go to the last workgroups).  Every row is
    # compared with the oracle.
    per = 16384 if dtype == synth.BF16 else 8192
    spec = synth.CONFIGS["C3"].with_(capacity=112, T=8, V=8 * per - 5, V_pad=8 * per,
                                     dtype=dtype, seed=93)
    w = synth.make(spec)
    rows = int(w.active_mask().sum())
    grid = int(H.make_plan(spec).raw.grid)
    p = grid // rows
    idle = grid - p * rows
    longest = -(-rows * 8 // grid)
    if not (rows * 8 >= 2 * grid and p >= 2 and -(-8 // p) <= longest + 1 and 16 * idle >= grid):
        pytest.skip(f"{rows} rows on a grid of {grid} do not take the extra-piece partition")
    full_compare(oracle_handle, spec)


@pytest.mark.parametrize("case", ["fp32_64_units", "bf16_33_units_selected"])
def test_four_wave_merge_many_parts(oracle_handle, case):
    # One-unit ranges, so every unit of a row is its own part: 64 parts per
    # row (eight pairs per merge wave, the most the layout holds) or 33 with
    # rows that select IDs among them.  Every row against the oracle.
    if case == "fp32_64_units":
        spec = synth.CONFIGS["C1"].with_(capacity=8, V=64 * 8192 - 3, V_pad=64 * 8192,
                                         emitted="one", seed=95)
    else:
        spec = synth.CONFIGS["C4"].with_(capacity=6, T=4, V=33 * 16384 - 9, V_pad=33 * 16384,
                                         emitted="uniform", selected="frac40", seed=96)
    full_compare(oracle_handle, spec)


def test_row_pieces_three_and_four(oracle_handle):
    # About 400 active rows of 12 units: three pieces per row leave about 80
    # workgroups idle, so the last rows get four pieces.
    spec = synth.CONFIGS["C3"].with_(capacity=400, T=1, emitted="one", V=12 * 16384 - 5,
                                     V_pad=12 * 16384, seed=97)
    w = synth.make(spec)
    rows = int(w.active_mask().sum())
    grid = int(H.make_plan(spec).raw.grid)
    p = grid // rows
    idle = grid - p * rows
    longest = -(-rows * 12 // grid)
    if not (rows * 12 >= 2 * grid and p == 3 and -(-12 // p) <= longest + 1 and 16 * idle >= grid):
        pytest.skip(f"{rows} rows on a grid of {grid} do not take three and four pieces")
    full_compare(oracle_handle, spec)


def full_size_all_rows(o, spec):
    """The configuration at its full size, in the launch configuration the
    bench times, every active row compared with the oracle."""
    announce(f"full size {spec.name} cap={spec.capacity} T={spec.T} V={spec.V} K={spec.K} "
             f"(every active row)")
    w = synth.make(spec)
    got, lse, guard = H.run_gpu(w, guard=True)
    act = np.nonzero(w.active_mask().reshape(-1))[0]
    worst, worst_L, L_differ = H.compare_rows_with_oracle(o, w, got, lse, act, spec.name)
    H.check_properties(w, got, lse)
    announce(f"{spec.name}: {act.size} rows exact; max |d logprob| = {worst:.3g}, "
             f"max |d L| = {worst_L:.3g}, L bits differ on {L_differ} rows, guard rescans "
             f"{int(guard[act].sum())} parts")


def test_c3_full_size_all_rows(oracle_handle):
    full_size_all_rows(oracle_handle, synth.CONFIGS["C3"])


def test_c4_full_size_all_rows(oracle_handle):
    full_size_all_rows(oracle_handle, synth.CONFIGS["C4"])


def test_c5_full_size_all_rows(oracle_handle):
    full_size_all_rows(oracle_handle, synth.CONFIGS["C5"])


def test_listing_at_the_last_bit_of_L(oracle_handle):
    """Two rows whose listing depends on the last bit of L (the golden
    fixtures last_bit_of_L_a/b): L is exact on both sides here (one lane
    dominates by e^99), so the GPU must give both listings bit for bit."""
    rows = []
    for name in ("last_bit_of_L_a_v64_fp32", "last_bit_of_L_b_v64_fp32"):
        fx = json.load(open(os.path.join(HERE, "golden", name + ".json")))
        rows.append(np.asarray(fx["row_bits"], np.uint32).view(np.float32))
    announce("last bit of L rows fp32")
    w = _frame_from_rows(np.stack(rows), synth.FP32, K=4)
    got, lse = H.run_gpu(w)
    assert lse[0] == np.float32(100.0) and lse[1] == np.float32(100 + 2.0**-17)
    H.compare_words(got, H.oracle_frame(oracle_handle, w), "last bit of L")
    assert got[0, 0, 2:8:2].tolist() == [2, 1, 0] and got[1, 0, 2:8:2].tolist() == [2, 0, 1]


# ----------------------------------------------------------------- edge cases
EDGE = [
    ("v1", dict(V=1, V_pad=1)),
    ("v5_vpad8", dict(V=5, V_pad=8)),
    ("v19", dict(V=19, V_pad=19)),
    ("v37_unaligned", dict(V=37, V_pad=41)),
    ("one_segment", dict(V=16384, V_pad=16384)),
    ("segment_plus_one", dict(V=16385, V_pad=16392)),
    ("ragged_chunk", dict(V=2 * 16384 + 3, V_pad=2 * 16384 + 8)),
    ("unaligned_stride", dict(V=50001, V_pad=50003)),
    ("k1", dict(V=30000, V_pad=30000, K=1)),
    ("k0", dict(V=30000, V_pad=30000, K=0)),
]


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("name,kw", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes(oracle_handle, dtype, name, kw):
    spec = synth.CONFIGS["C3"].with_(capacity=3, T=4, dtype=dtype, recipe=synth.GUMBEL,
                                     p1=10.0, seed=77, **kw)
    full_compare(oracle_handle, spec)


def _frame_from_rows(rows_f32: np.ndarray, dtype, T=1, K=20, V_pad=None):
    """A workload whose active rows are the given rows (one slot per row)."""
    nrow, V = rows_f32.shape
    V_pad = V if V_pad is None else V_pad
    spec = synth.Spec("designed", nrow, T, V, V_pad, dtype, synth.NORMAL, K=K, emitted="one",
                      seed=9)
    req, emi, tok, cnt, ids = synth.gating(spec)
    buf = np.zeros((nrow * T, V_pad), np.float32)
    buf[::T, :V] = rows_f32
    logits = synth.bf16_bits(buf) if dtype == synth.BF16 else buf
    return synth.Workload(spec, np.ascontiguousarray(logits), req, emi, tok, cnt, ids)


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP32], ids=["bf16", "fp32"])
def test_ties_all_equal_and_one_hot_rows(oracle_handle, dtype):
    """All-equal rows and one-hot rows take the tie fallback inside segments."""
    V = 40000
    rows = np.zeros((6, V), np.float32)
    rows[1, :] = -3.0
    rows[2, :] = -np.inf
    rows[2, 31337] = 2.0
    rows[3, :] = -np.inf
    rows[3, 7] = -0.0
    rows[4, :] = (np.arange(V) % 3).astype(np.float32)  # many ties at 2.0
    rows[5, :] = -np.inf
    rows[5, 39999] = 5.0
    rows[5, 16384] = 5.0
    announce(f"designed tie rows dtype={dtype}")
    w = _frame_from_rows(rows, dtype)
    got, lse = H.run_gpu(w)
    ref = H.oracle_frame(oracle_handle, w)
    H.compare_words(got, ref, "ties")
    H.check_properties(w, got, lse)
    # one finite lane: L is that lane's value and its logprob is exactly +0
    assert got[2, 0, 2] == 31337 and got[2, 0, 3] == 0
    assert got[3, 0, 2] == 7 and got[3, 0, 3] == 0


@pytest.mark.parametrize("dtype", [synth.FP32, synth.BF16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("background", ["neginf", "noise"])
def test_guard_trips_on_subtraction_ties(oracle_handle, dtype, background):
    """Segment 0 holds 32 distinct logits that all round to the same reported
    value after subtracting L.  Its best 32 raw keys keep the largest of them
    and drop the smallest, which have the smallest IDs and so belong in the
    top K.  The merge guard must catch this and rescan the segment.  With a
    -inf background the segment takes the in-segment tie fallback; with a
    noise background it takes the ordinary candidate path."""
    V = 3 * 16384
    rng = np.random.default_rng(5)
    if background == "neginf":
        row = np.full(V, -np.inf, np.float32)
    else:
        row = rng.uniform(-10.0, -5.0, size=V).astype(np.float32)
        if dtype == synth.BF16:
            row = synth.bf16_to_f32(synth.bf16_bits(row))
    if dtype == synth.FP32:
        base = np.float32(1.0)
        for k in range(33):
            row[k] = base
            base = np.nextafter(base, np.float32(2.0))
        row[50] = 100.0
    else:
        for k in range(33):
            row[k] = np.float32((k + 1) * 2.0 ** -30)  # exact in bf16
        row[50] = 10.0
    announce(f"guard trip row dtype={dtype} background={background}")
    w = _frame_from_rows(row[None, :], dtype)
    got, lse, guard = H.run_gpu(w, guard=True)
    ref = H.oracle_frame(oracle_handle, w)
    assert ref[0, 0, 2:8:2].tolist() == [50, 0, 1]
    H.compare_words(got, ref, "guard")
    assert guard[0] >= 1  # the diagnostic counts the rescanned part


def test_golden_fixtures_on_gpu(oracle_handle):
    for path in sorted(glob.glob(os.path.join(HERE, "golden", "*.json"))):
        fx = json.load(open(path))
        announce(f"golden {fx['name']}")
        if fx["dtype"] == "bf16":
            vals = synth.bf16_to_f32(np.asarray(fx["row_bits"], np.uint16))
            dt = synth.BF16
        else:
            vals = np.asarray(fx["row_bits"], np.uint32).view(np.float32)
            dt = synth.FP32
        w = _frame_from_rows(vals[None, :].astype(np.float32), dt, K=fx["K"])
        w.tokens[0] = fx["token"]
        if fx["sel"]:
            w.id_counts[0] = len(fx["sel"])
            w.ids[:len(fx["sel"])] = fx["sel"]
        got, _ = H.run_gpu(w)
        H.compare_words(got[0, 0, :len(fx["words"])], np.asarray(fx["words"], np.int32),
                        fx["name"])


def test_gating_clamps_and_invalid_ids(oracle_handle):
    spec = synth.CONFIGS["C3"].with_(capacity=6, T=3, V=20000, V_pad=20000, seed=31)
    w = synth.make(spec)
    w.requested[:] = [1, 0, 1, 1, 1, 1]
    w.emitted[:] = [2, 3, 0, 9, -4, 3]
    w.id_counts[:] = [-5, 4, 3, 0, 0, 300]
    w.ids[5 * 128:6 * 128] = np.arange(128) * 7
    w.ids[5 * 128 + 3] = -1
    w.ids[5 * 128 + 4] = 20000
    w.ids[5 * 128 + 5] = 2**31 - 1
    w.ids[1 * 128:1 * 128 + 4] = [1, 2, 3, 4]
    w.tokens[3 * 3 + 1] = -7
    w.tokens[3 * 3 + 2] = 20000
    announce("gating clamps and invalid ids")
    got, lse = H.run_gpu(w)
    ref = H.oracle_frame(oracle_handle, w)
    H.compare_words(got, ref, "gating")


def test_unaligned_base_pointer(oracle_handle):
    """A logits pointer 2 bytes past a 16-byte boundary takes the scalar path."""
    spec = synth.CONFIGS["C3"].with_(capacity=2, T=2, V=33000, V_pad=33000, seed=41)
    w = synth.make(spec)
    d = H.to_device(w)
    n = d["logits"].numel()
    big = torch.empty(n + 8, dtype=torch.bfloat16, device="cuda")
    big[1:1 + n].copy_(d["logits"])
    view = big[1:1 + n]
    assert view.data_ptr() % 16 == 2
    announce("unaligned base pointer bf16")
    got, lse = H.run_gpu(w, dev_inputs=d, logits=view)
    ref = H.oracle_frame(oracle_handle, w)
    H.compare_words(got, ref, "unaligned")


@pytest.mark.parametrize("name", ["C3", "C4", "C5"])
def test_workspace_needs_no_initialisation(oracle_handle, name):
    """A workspace full of garbage (every byte 0xFF, then a random fill)
    gives the oracle's frame: the library reads no workspace word before it
    writes it in the same call."""
    spec = synth.CONFIGS[name].with_(capacity={"C3": 6, "C4": 10, "C5": 3}[name])
    announce(f"garbage workspace {name} cap={spec.capacity}")
    w = synth.make(spec)
    d = H.to_device(w)
    plan = H.make_plan(spec)
    ref = H.oracle_frame(oracle_handle, w)
    ws = plan.workspace()
    ws.fill_(0xFF)
    got, _ = H.run_gpu(w, d, plan=plan, ws=ws)
    H.compare_words(got, ref, f"{name} 0xFF workspace")
    g = torch.Generator(device="cpu").manual_seed(11)
    ws.copy_(torch.randint(0, 256, (ws.numel(),), generator=g, dtype=torch.uint8))
    got2, _ = H.run_gpu(w, d, plan=plan, ws=ws)
    assert np.array_equal(got, got2)


# -------------------------------------------------- repeatability and graphs
def test_repeatable_bit_identical():
    spec = synth.CONFIGS["C3"].with_(capacity=16)
    w = synth.make(spec)
    d = H.to_device(w)
    plan = H.make_plan(spec)
    ws = plan.workspace()
    announce("repeatability C3 cap=16")
    a, la = H.run_gpu(w, d, plan, ws)
    b, lb = H.run_gpu(w, d, plan, ws)
    assert np.array_equal(a, b) and np.array_equal(la.view(np.int32), lb.view(np.int32))


def test_reduce_then_merge_equals_run(oracle_handle):
    """The two launches called apart, with other stream work between them,
    give run's frame bit for bit (and the oracle's)."""
    spec = synth.CONFIGS["C4"].with_(capacity=12, seed=45)
    w = synth.make(spec)
    d = H.to_device(w)
    plan = H.make_plan(spec)
    announce("reduce + merge vs run C4 cap=12")
    a, la = H.run_gpu(w, d, plan)
    ws = plan.workspace()
    out = plan.new_out(H.POISON)
    args = (d["logits"], d["tokens"], d["emitted"], d["requested"], d["id_counts"], d["ids"], out,
            ws)
    plan.run(*args, phase="reduce")
    scratch = torch.ones(1 << 20, device=out.device).neg_()  # unrelated work in between
    plan.run(*args, phase="merge")
    torch.cuda.synchronize()
    del scratch
    b = out.cpu().numpy()
    assert np.array_equal(a, b)
    assert np.array_equal(la.view(np.int32), plan.lse(ws).cpu().numpy().view(np.int32))
    H.compare_words(b, H.oracle_frame(oracle_handle, w), "reduce + merge")


def test_hip_graph_replay_matches_eager():
    spec = synth.CONFIGS["C4"].with_(capacity=8, seed=44)
    w = synth.make(spec)
    d = H.to_device(w)
    plan = H.make_plan(spec)
    ws = plan.workspace()
    announce("hip graph capture and replay C4 cap=8")
    eager, _ = H.run_gpu(w, d, plan, ws)
    out = plan.new_out(H.POISON)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            plan.run(d["logits"], d["tokens"], d["emitted"], d["requested"], d["id_counts"],
                     d["ids"], out, ws)
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(H.POISON)
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager), f"replay {i}"
        del junk


def test_bound_call_matches_run(oracle_handle):
    """A prepared call (Plan.bind) launches the same work as Plan.run."""
    import full_vocab_logprob_amd as flp
    spec = synth.CONFIGS["C3"].with_(capacity=6, T=4, V=50000, V_pad=50000)
    announce("bound call vs run")
    w = synth.make(spec)
    d = H.to_device(w)
    a, _ = H.run_gpu(w, dev_inputs=d)
    plan = H.make_plan(spec)
    ws = plan.workspace()
    out = plan.new_out(H.POISON)
    call = plan.bind(d["logits"], d["tokens"], d["emitted"], d["requested"], d["id_counts"],
                     d["ids"], out, ws)
    call()
    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), a)
    with pytest.raises(ValueError):
        plan.bind(d["logits"][:-1], d["tokens"], d["emitted"], d["requested"], d["id_counts"],
                  d["ids"], out, ws)
    with pytest.raises(flp.FlareError):
        bad = flp.BoundCall(call.name, (call._args[0], 0) + call._args[2:], ())
        bad()
