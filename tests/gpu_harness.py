"""Helpers for the GPU parity tests: upload a workload, run the HIP path
through the C ABI binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import full_vocab_logprob_amd as flp
import synth

TOL = 2e-5  # absolute, on FP32 logprobs and on L
POISON = int(synth.POISON)


def to_device(w: synth.Workload, dev="cuda"):
    s = w.spec
    if s.dtype == synth.BF16:
        lg = torch.from_numpy(w.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        lg = torch.from_numpy(w.logits).to(dev)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)  # noqa
    return dict(logits=lg.reshape(-1), tokens=g(w.tokens), emitted=g(w.emitted),
                requested=g(w.requested), id_counts=g(w.id_counts), ids=g(w.ids))


def make_plan(spec: synth.Spec, K: int | None = None):
    return flp.Plan(spec.capacity, spec.T, spec.V, spec.V_pad,
                    dtype=torch.bfloat16 if spec.dtype == synth.BF16 else torch.float32,
                    K=spec.K if K is None else K, device=torch.cuda.current_device())


def run_gpu(w: synth.Workload, dev_inputs=None, plan=None, ws=None, logits=None,
            guard=False):
    """Run the HIP path once; returns (out [cap, T, 258] int32, lse [cap*T]),
    plus the per-row guard rescan counts [cap*T] when `guard`."""
    d = dev_inputs if dev_inputs is not None else to_device(w)
    plan = plan or make_plan(w.spec)
    ws = ws if ws is not None else plan.workspace()
    out = plan.new_out(POISON)
    plan.run(d["logits"] if logits is None else logits, d["tokens"], d["emitted"],
             d["requested"], d["id_counts"], d["ids"], out, ws)
    torch.cuda.synchronize()
    res = (out.cpu().numpy(), plan.lse(ws).cpu().numpy().copy())
    if guard:
        res = res + (plan.guard(ws).cpu().numpy().copy(),)
    return res


def oracle_rows(o, w: synth.Workload, rows, threads: int = 16):
    """The oracle's (words, L) for each logit row in `rows`, one row per task
    on a thread pool (the oracle call releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    s = w.spec

    def one(r):
        sl = int(r) // s.T
        n = int(np.clip(w.id_counts[sl], 0, 128))
        sel = w.ids[sl * 128: sl * 128 + n] if n > 0 else None
        return o.row(w.logits[int(r)], token=int(w.tokens[int(r)]), K=s.K, sel=sel, V=s.V)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        return dict(zip((int(r) for r in rows), ex.map(one, rows)))


def compare_rows_with_oracle(o, w: synth.Workload, got: np.ndarray, lse: np.ndarray, rows,
                             where: str):
    """Every given active row against the oracle, element by element: IDs and
    layout bit-exact, values and L within TOL.  Returns (max |d logprob|,
    max |d L|, rows whose FP32 L differs from the oracle's in any bit).
    When IDs differ, the message says whether the oracle's listing at the
    kernel's own L (differing by a few units in the last place) would have
    matched, which names the cause; the test fails either way."""
    s = w.spec
    ref = oracle_rows(o, w, rows)
    worst = worst_L = 0.0
    L_bits_differ = 0
    for r in rows:
        r = int(r)
        sl, t = divmod(r, s.T)
        words, L = ref[r]
        g = got[sl, t, :len(words)]
        Lg = np.float32(lse[r])
        if np.float32(L).view(np.int32) != Lg.view(np.int32):
            L_bits_differ += 1
        if not np.array_equal(g[0::2], words[0::2]):
            n = int(np.clip(w.id_counts[sl], 0, 128))
            sel = w.ids[sl * 128: sl * 128 + n] if n > 0 else None
            at_own = o.row_at(w.logits[r], int(w.tokens[r]), s.K, Lg, sel=sel, V=s.V)
            raise AssertionError(
                f"{where} row {r}: IDs differ (GPU L {float(Lg)!r}, oracle L {L!r}); the "
                f"oracle listing at the GPU's L {'matches' if np.array_equal(at_own, g) else 'does not match'}")
        compare_words(g, words, f"{where} row {r}")
        assert abs(float(Lg) - L) <= TOL, (where, r, float(Lg), L)
        worst = max(worst, max_value_delta(g, words))
        worst_L = max(worst_L, abs(float(Lg) - L))
    return worst, worst_L, L_bits_differ


def oracle_frame(o, w: synth.Workload):
    s = w.spec
    ref = w.poisoned_out()
    o.frame(w.logits, s.capacity, s.T, s.V, s.V_pad, w.requested, w.id_counts, w.ids,
            w.emitted, w.tokens, s.K, ref)
    return ref


def compare_words(got: np.ndarray, ref: np.ndarray, where: str = ""):
    """IDs, layout and poison bit-exact; values within TOL (NaN bits exact)."""
    got = np.asarray(got, dtype=np.int32)
    ref = np.asarray(ref, dtype=np.int32)
    assert got.shape == ref.shape
    gi, ri = got[..., 0::2], ref[..., 0::2]
    bad = np.argwhere(gi != ri)
    assert bad.size == 0, f"{where}: id/layout mismatch at {bad[:5].tolist()} " \
                          f"got {gi[tuple(bad[0])]} want {ri[tuple(bad[0])]}"
    gb, rb = got[..., 1::2], ref[..., 1::2]
    gv, rv = gb.view(np.float32), rb.view(np.float32)
    same = gb == rb
    with np.errstate(invalid="ignore"):
        close = np.abs(gv.astype(np.float64) - rv.astype(np.float64)) <= TOL
    ok = same | (close & ~np.isnan(gv) & ~np.isnan(rv))
    bad = np.argwhere(~ok)
    assert bad.size == 0, f"{where}: value mismatch at {bad[:5].tolist()} " \
                          f"got {gv[tuple(bad[0])]!r} want {rv[tuple(bad[0])]!r}"


def max_value_delta(got: np.ndarray, ref: np.ndarray) -> float:
    gv = np.asarray(got, np.int32)[..., 1::2].view(np.float32).astype(np.float64)
    rv = np.asarray(ref, np.int32)[..., 1::2].view(np.float32).astype(np.float64)
    m = np.isfinite(gv) & np.isfinite(rv)
    return float(np.max(np.abs(gv[m] - rv[m]))) if m.any() else 0.0


def row_floats(w: synth.Workload, r: int) -> np.ndarray:
    row = w.logits[r, :w.spec.V]
    return synth.bf16_to_f32(row) if w.spec.dtype == synth.BF16 else row


def check_properties(w: synth.Workload, got: np.ndarray, lse: np.ndarray):
    """Facts that hold at any size, checked on every position: gating and
    poison, word 0 = chosen token, the chosen value is fl32(x - L) with the
    kernel's own L, natural pairs sorted by (value desc, ID asc), IDs in
    range and distinct, selected IDs echoed in caller order."""
    s = w.spec
    act = w.active_mask()
    n_sel = np.clip(w.id_counts, 0, 128)
    for sl in range(s.capacity):
        for t in range(s.T):
            cell = got[sl, t]
            r = sl * s.T + t
            if not act[sl, t]:
                assert np.all(cell == POISON), (sl, t)
                continue
            n = int(n_sel[sl])
            W = n if n > 0 else s.K
            assert np.all(cell[2 + 2 * W:] == POISON), (sl, t)
            assert cell[0] == w.tokens[r]
            L = np.float32(lse[r])
            x = row_floats(w, r)
            tok = int(w.tokens[r])
            if 0 <= tok < s.V:
                v = np.float32(x[tok] - L)
                v = np.float32(0.0) if v == 0 else v
                assert cell[1] == np.array([v], np.float32).view(np.int32)[0], (sl, t)
            if n > 0:
                assert np.array_equal(cell[2:2 + 2 * n:2], w.ids[sl * 128: sl * 128 + n])
                continue
            ids = cell[2:2 + 2 * W:2]
            vals = cell[3:3 + 2 * W:2].view(np.float32)
            k = min(W, s.V)
            assert np.all(ids[k:] == -1)
            ids, vals = ids[:k], vals[:k]
            if k == 0:
                continue
            assert len(set(ids.tolist())) == k and ids.min() >= 0 and ids.max() < s.V
            assert np.all(vals <= 0)
            assert np.all((vals[:-1] > vals[1:]) | ((vals[:-1] == vals[1:]) & (ids[:-1] < ids[1:])))
            want = (x[ids] - L).astype(np.float32)
            want[want == 0] = 0.0
            assert np.array_equal(want.view(np.int32), vals.view(np.int32)), (sl, t)
            # nothing outside the list beats its last entry
            last_v, last_id = vals[-1], ids[-1]
            allv = (x - L).astype(np.float32)
            better = (allv > last_v) | ((allv == last_v) & (np.arange(s.V) < last_id))
            assert int(better.sum()) == k - 1, (sl, t, int(better.sum()))
