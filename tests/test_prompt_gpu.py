"""Parity of prompt scoring (scored prefill rows) with the CPU oracle (needs
an MI355X).

Each scored row is [target, bits, rank, twenty (id, bits) pairs].  IDs,
layout and invalid rows are compared bit for bit, values within the same
2e-5 as the generation path.  The rank is an integer that FP32 comparisons
decide: it must equal the count of strictly greater reported values taken
with the kernel's own L, and the oracle's rank whenever the two L agree
bit for bit (otherwise a lane whose comparison flips between the two L is
the only allowed difference).
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
    flp.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    yield


def run_prompt(w: synth.PromptWorkload, logits=None, plan=None, ws=None):
    import full_vocab_logprob_amd as flp
    s = w.spec
    if logits is None:
        if s.dtype == synth.BF16:
            logits = torch.from_numpy(w.logits.view(np.int16)).cuda().view(torch.bfloat16)
        else:
            logits = torch.from_numpy(w.logits).cuda()
        logits = logits.reshape(-1)
    plan = plan or flp.PromptPlan(w.rows, s.V, s.V_pad,
                                  dtype=torch.bfloat16 if s.dtype == synth.BF16 else torch.float32)
    ws = ws if ws is not None else plan.workspace()
    targets = torch.from_numpy(np.ascontiguousarray(w.targets, np.int32)).cuda()
    out = plan.new_out(H.POISON)
    plan.run(logits, targets, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), plan.lse(ws).cpu().numpy().copy()


def oracle_prompt(o, w: synth.PromptWorkload):
    s = w.spec
    ref = w.poisoned_out()
    _, lse = o.prompt(w.logits, w.rows, s.V, s.V_pad, w.targets, ref)
    return ref, lse


def row_floats(w, r):
    row = w.logits[r, :w.spec.V]
    return synth.bf16_to_f32(row) if w.spec.dtype == synth.BF16 else row.astype(np.float32)


def rank_with(x: np.ndarray, t: int, L) -> int:
    rep = (x - np.float32(L)).astype(np.float32)
    rep[rep == 0] = 0.0
    return 1 + int(np.count_nonzero(rep > rep[t]))


def compare_prompt(w, got, lse, ref, ref_lse, rows=None, where=""):
    rows = range(w.rows) if rows is None else rows
    rows = list(rows)
    g = got[rows]
    r = ref[rows]
    # pairs: words 0-1 and 3-42 (IDs and layout exact, values within 2e-5)
    H.compare_words(np.concatenate([g[:, :2], g[:, 3:]], axis=1),
                    np.concatenate([r[:, :2], r[:, 3:]], axis=1), where)
    for i, row in enumerate(rows):
        t = int(w.targets[row])
        if not (0 <= t < w.spec.V):
            assert g[i, 2] == 0 and r[i, 2] == 0, (where, row)
            continue
        x = row_floats(w, row)
        own = rank_with(x, t, lse[row])
        assert g[i, 2] == own, (where, row, int(g[i, 2]), own)
        if np.float32(lse[row]).view(np.int32) == np.float32(ref_lse[row]).view(np.int32):
            assert g[i, 2] == r[i, 2], (where, row, int(g[i, 2]), int(r[i, 2]))
        else:
            lo, hi = sorted((float(lse[row]), float(ref_lse[row])))
            # lanes whose comparison with the target can flip between the two L
            scale = abs(hi) + (abs(float(x[t])) if np.isfinite(x[t]) else 0.0)
            near = np.abs((x - x[t]).astype(np.float64)) <= 4 * np.spacing(np.float32(scale))
            assert abs(int(g[i, 2]) - int(r[i, 2])) <= int(near.sum()), (where, row)


def full_prompt_compare(o, spec):
    announce(f"prompt compare {spec.name} rows={spec.capacity} V={spec.V} V_pad={spec.V_pad} "
             f"dtype={spec.dtype}")
    w = synth.make_prompt(spec)
    got, lse = run_prompt(w)
    ref, ref_lse = oracle_prompt(o, w)
    compare_prompt(w, got, lse, ref, ref_lse, where=spec.name)
    return w, got, ref


# ------------------------------------------------------------ named chunks
def test_p1_bf16_full(oracle_handle):
    """The bench chunk itself: 128 rows x V=248,320 bf16, every row."""
    w, got, ref = full_prompt_compare(oracle_handle, synth.PROMPT_CONFIGS["P1"])
    assert w.valid_rows() < w.rows  # invalid rows are present
    ranks = got[:, 2][(w.targets >= 0)]
    assert (ranks == 1).any() and (ranks > 1000).any()  # peak targets and deep targets


def test_p2_fp32_padded_reduced(oracle_handle):
    full_prompt_compare(oracle_handle, synth.PROMPT_CONFIGS["P2"].with_(capacity=48))


def test_p2_fp32_full_size_all_rows(oracle_handle):
    """All 512 rows of the FP32 chunk on the GPU, every row against the
    oracle (rows on a thread pool), and the rank of every row recounted
    with the kernel's own L."""
    from concurrent.futures import ThreadPoolExecutor
    spec = synth.PROMPT_CONFIGS["P2"]
    announce(f"prompt full size {spec.name} rows={spec.capacity} (every row)")
    w = synth.make_prompt(spec)
    got, lse = run_prompt(w)
    o = oracle_handle
    ref = w.poisoned_out()
    ref_lse = np.full(w.rows, np.nan, np.float32)
    with ThreadPoolExecutor(16) as ex:
        res = list(ex.map(lambda r: o.prompt_row(w.logits[r], int(w.targets[r]), V=spec.V),
                          range(w.rows)))
    for r, (words, L) in enumerate(res):
        ref[r], ref_lse[r] = words, L
    compare_prompt(w, got, lse, ref, ref_lse, where="P2 full size")
    valid = (w.targets >= 0) & (w.targets < spec.V)
    same_L = np.float32(lse[valid]).view(np.int32) == np.float32(ref_lse[valid]).view(np.int32)
    announce(f"P2: {w.rows} rows compared; L bits differ on {int((~same_L).sum())} of "
             f"{int(valid.sum())} valid rows")
    for r in range(w.rows):
        t = int(w.targets[r])
        if 0 <= t < spec.V:
            assert got[r, 2] == rank_with(row_floats(w, r), t, lse[r]), r
        else:
            assert got[r, 0] == -1 and got[r, 2] == 0


EDGE = [
    ("v1", dict(V=1, V_pad=1)),
    ("v7_below_20", dict(V=7, V_pad=7)),
    ("v20", dict(V=20, V_pad=24)),
    ("one_unit_ragged", dict(V=16384 + 3, V_pad=16384 + 9)),
    ("many_units_ragged", dict(V=5 * 16384 + 4097, V_pad=5 * 16384 + 4101)),
    ("one_row", dict(capacity=1)),
    ("many_rows_small_v", dict(capacity=3000, V=300, V_pad=300)),
]


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("name,kw", EDGE, ids=[e[0] for e in EDGE])
def test_prompt_edge_shapes(oracle_handle, dtype, name, kw):
    base = dict(capacity=21, V=40000, V_pad=40000)
    base.update(kw)
    spec = synth.PROMPT_CONFIGS["P1"].with_(dtype=dtype, seed=31, **base)
    full_prompt_compare(oracle_handle, spec)


def test_prompt_all_rows_invalid():
    """No valid target: nothing is read, every row gets the invalid record."""
    spec = synth.PROMPT_CONFIGS["P1"].with_(capacity=16, V=5000, V_pad=5000)
    w = synth.make_prompt(spec)
    w.targets[:] = -1
    w.targets[3] = 5000
    w.targets[4] = -12345
    announce("prompt all rows invalid")
    got, _ = run_prompt(w)
    want = np.array([-1, 0x7FC00000, 0] + [-1, 0x7FC00000] * 20, dtype=np.int64).astype(np.int32)
    assert np.array_equal(got, np.broadcast_to(want, got.shape))


def _chunk_from_rows(rows_f32: np.ndarray, targets, dtype):
    n, V = rows_f32.shape
    spec = synth.Spec("designed", n, 1, V, V, dtype, synth.NORMAL, seed=9)
    logits = synth.bf16_bits(rows_f32) if dtype == synth.BF16 else rows_f32.astype(np.float32)
    return synth.PromptWorkload(spec, np.ascontiguousarray(logits),
                                np.asarray(targets, np.int32))


@pytest.mark.parametrize("dtype", [synth.FP32, synth.BF16], ids=["fp32", "bf16"])
def test_prompt_rank_subtraction_ties(oracle_handle, dtype):
    """33 distinct logits spread over several units all report the same value
    after subtracting L: none of them is strictly greater than another, so
    the raw count overcounts and the merge must recount those parts."""
    V = 6 * 16384 + 77
    rng = np.random.default_rng(8)
    rows = np.empty((6, V), np.float32)
    lanes = (np.arange(33) * 2999 + 11) % V  # spread over every unit
    targets = []
    for i in range(6):
        bg = rng.uniform(-30.0, -20.0, size=V).astype(np.float32)
        rows[i] = synth.bf16_to_f32(synth.bf16_bits(bg)) if dtype == synth.BF16 else bg
        if dtype == synth.FP32:
            base = np.float32(1.0)
            for k in range(33):
                rows[i, lanes[k]] = base
                base = np.nextafter(base, np.float32(2.0))
            rows[i, 5] = 200.0  # half an ulp of 199 exceeds the chain's spread
        else:
            for k in range(33):
                rows[i, lanes[k]] = np.float32((k + 1) * 2.0 ** -30)  # exact in bf16
            rows[i, 5] = 10.0
        targets.append(int(lanes[[0, 16, 32, 0, 7, 20][i]]))
    rows[3, 6] = rows[3, 5]  # a second peak: rank 3 for the tied group
    rows[4, lanes[7]] = rows[4, lanes[8]]  # an exact raw tie inside the group
    w = _chunk_from_rows(rows, targets, dtype)
    announce(f"prompt subtraction ties dtype={dtype}")
    got, lse = run_prompt(w)
    ref, ref_lse = oracle_prompt(oracle_handle, w)
    assert ref[:, 2].tolist() == [2, 2, 2, 3, 2, 2]
    compare_prompt(w, got, lse, ref, ref_lse, where="subtraction ties")


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP32], ids=["bf16", "fp32"])
def test_prompt_tie_heavy_rows(oracle_handle, dtype):
    """All-equal rows, one-hot rows, a -inf target and grid rows with ~2,000
    lanes per level."""
    V = 40000
    rows = np.zeros((6, V), np.float32)
    rows[1, :] = -3.0
    rows[2, :] = -np.inf
    rows[2, 31337] = 2.0
    rows[3, :] = (np.arange(V) % 3).astype(np.float32)
    rng = np.random.default_rng(4)
    rows[4, :] = (rng.integers(0, 129, size=V) / 8.0 - 8.0).astype(np.float32)
    rows[5, :] = rows[4, :]
    targets = [123, 39999, 5, 1, int(np.argmax(rows[4])), int(np.argmin(rows[5]))]
    w = _chunk_from_rows(rows, targets, dtype)
    announce(f"prompt tie-heavy rows dtype={dtype}")
    got, lse = run_prompt(w)
    ref, ref_lse = oracle_prompt(oracle_handle, w)
    compare_prompt(w, got, lse, ref, ref_lse, where="tie-heavy")
    assert got[0, 2] == 1 and got[1, 2] == 1 and got[2, 2] == 2


def test_prompt_repeatable_and_split_launches(oracle_handle):
    """Two runs give the same bytes, and reduce then merge equals run."""
    import full_vocab_logprob_amd as flp
    spec = synth.PROMPT_CONFIGS["P1"].with_(capacity=24, V=100000, V_pad=100000)
    w = synth.make_prompt(spec)
    announce("prompt repeatable / split")
    a, _ = run_prompt(w)
    b, _ = run_prompt(w)
    assert np.array_equal(a, b)
    plan = flp.PromptPlan(w.rows, spec.V, spec.V_pad, dtype=torch.bfloat16)
    ws = plan.workspace()
    logits = torch.from_numpy(w.logits.view(np.int16)).cuda().view(torch.bfloat16).reshape(-1)
    targets = torch.from_numpy(w.targets).cuda()
    out = plan.new_out(H.POISON)
    plan.run(logits, targets, out, ws, phase="reduce")
    plan.run(logits, targets, out, ws, phase="merge")
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), a)


def test_prompt_rank_fp32_value_tie_counts(oracle_handle):
    """FP32 rows where the logits just above the target tie with it after the
    subtraction: one value held by several lanes (taken off by its count, no
    recount), and two distinct tying values (recounted)."""
    V = 3 * 16384 + 5
    rng = np.random.default_rng(12)
    rows = rng.uniform(-30.0, -20.0, size=(3, V)).astype(np.float32)
    up = np.nextafter(np.float32(1.0), np.float32(2.0))
    for i in range(3):
        rows[i, 5] = 200.0            # L = 200: 1.0 and its neighbours report -199
        rows[i, 1000] = 1.0           # the target
        rows[i, 30000] = 1.5          # reports more than the target
    rows[0, [20000, 40000]] = up      # one tying value on two lanes, in one part or two
    rows[1, [1001, 1002, 1003]] = up  # three lanes beside the target
    rows[2, 20000] = up               # two distinct tying values
    rows[2, 40000] = np.nextafter(up, np.float32(2.0))
    w = _chunk_from_rows(rows, [1000, 1000, 1000], synth.FP32)
    announce("prompt fp32 value-tie counts")
    got, lse = run_prompt(w)
    ref, ref_lse = oracle_prompt(oracle_handle, w)
    assert ref[:, 2].tolist() == [3, 3, 3]
    compare_prompt(w, got, lse, ref, ref_lse, where="fp32 value ties")
