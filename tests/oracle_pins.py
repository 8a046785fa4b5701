"""Pins for the CPU oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes an ``oracle.Oracle`` handle and raises
AssertionError when the oracle disagrees with something it must agree with.
None of them re-derives a result with the oracle's own recipe: they use
closed forms, brute-force ranks, a library logsumexp, designed tie rows and
poison invariants.  The same functions run against deliberately broken
builds of the oracle (test_oracle_mutants.py) to show that each plausible
mistake is caught.

Citations are to the Flare generation-logprobs design page (GLP) and the
Flare MTP design page.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import torch

import synth

NAN_BITS = 0x7FC00000
F32 = np.float32


def f32(x) -> np.float32:
    return np.float32(x)


def bits(x) -> int:
    return int(np.array([x], dtype=np.float32).view(np.int32)[0])


def from_bits(b) -> np.float32:
    return np.array([b], dtype=np.int32).view(np.float32)[0]


def ulp32(x: float) -> float:
    x = abs(float(x))
    return float(np.spacing(np.float32(x)))


def pairs(words):
    """words -> (ids, values) of the alternative pairs."""
    w = np.asarray(words, dtype=np.int32)
    return w[2::2].copy(), w[3::2].copy().view(np.float32)


# ---------------------------------------------------------------- closed forms
def pin_uniform_row(o):
    """A constant row x = c has L = c + ln V exactly, so every reported value
    is fl(c - fl(c + ln V)) (GLP definition paragraph)."""
    for V in (1, 7, 1000, 32000, 151936, 248320, 262144):
        for c in (0.0, 1.5, -3.25, 1000.0, -1000.0, 88.0):
            row = np.full(V, c, dtype=np.float32)
            words, L = o.row(row, token=V // 2, K=20)
            L_exact = f32(c + math.log(V))
            assert abs(float(L) - float(L_exact)) <= ulp32(L_exact), (V, c, L, L_exact)
            lp_tok = from_bits(words[1])
            want = f32(f32(c) - f32(L))
            assert lp_tok == want, (V, c, lp_tok, want)
            assert abs(float(lp_tok) - (c - (c + math.log(V)))) <= 2 * ulp32(L_exact) + 1e-7
    # The values printed for reference: -ln V rounded to FP32.
    for V, v in ((32000, -10.3734913), (151936, -11.9312143), (248320, -12.4224739),
                 (262144, -12.4766493)):
        words, _ = o.row(np.zeros(V, dtype=np.float32), token=0, K=1)
        assert abs(float(from_bits(words[1])) - v) < 2e-6, (V, from_bits(words[1]))


def pin_uniform_row_bf16(o):
    """Same closed form through the bf16 widening path."""
    for V in (3, 4096, 248320):
        for c in (0.0, 2.5, -7.75):
            row = synth.bf16_bits(np.full(V, c, dtype=np.float32))
            words, L = o.row(row, token=1 % V, K=20)
            L_exact = f32(c + math.log(V))
            assert abs(float(L) - float(L_exact)) <= ulp32(L_exact), (V, c, L)
            assert from_bits(words[1]) == f32(f32(c) - f32(L))


def pin_two_level_row(o):
    """a lanes at A and V - a lanes at B: L = A + ln(a + (V - a) e^(B - A))."""
    rng = np.random.default_rng(11)
    for V, a, A, B in ((10, 3, 2.0, -1.0), (5000, 17, 6.5, 0.25), (248320, 1, 12.0, 0.0),
                       (32000, 31999, 1.0, 3.0)):
        row = np.full(V, B, dtype=np.float32)
        hot = rng.choice(V, size=a, replace=False)
        row[hot] = A
        words, L = o.row(row, token=int(hot[0]), K=20)
        L_exact = A + math.log(a + (V - a) * math.exp(B - A))
        assert abs(float(L) - L_exact) <= ulp32(L_exact), (V, a, L, L_exact)
        assert from_bits(words[1]) == f32(f32(A) - f32(L))


def pin_probabilities_sum_to_one(o):
    """exp of the reported values over the whole vocabulary sums to 1.  All
    IDs are reported through selected-ID calls that cover [0, V)."""
    rng = np.random.default_rng(12)
    for V, scale in ((1, 1.0), (19, 3.0), (128, 4.0), (1000, 3.0), (5000, 8.0)):
        row = (rng.standard_normal(V) * scale).astype(np.float32)
        total = 0.0
        for start in range(0, V, 128):
            sel = np.arange(start, min(V, start + 128), dtype=np.int32)
            words, _ = o.row(row, token=0, K=20, sel=sel)
            ids, vals = pairs(words)
            assert np.array_equal(ids, sel)
            total += math.fsum(math.exp(float(v)) for v in vals)
        assert abs(total - 1.0) < 1e-5, (V, total)
    # Natural mode lists the whole vocabulary when V <= K.
    for V in range(1, 21):
        row = (rng.standard_normal(V) * 5).astype(np.float32)
        words, _ = o.row(row, token=0, K=20)
        ids, vals = pairs(words)
        assert sorted(ids[:V].tolist()) == list(range(V))
        assert abs(math.fsum(math.exp(float(v)) for v in vals[:V]) - 1.0) < 1e-5


def pin_one_hot(o):
    """One finite lane, the rest -inf: the hot lane's logprob is exactly +0
    and every other lane is -inf, listed by increasing ID."""
    for V, hot, v in ((64, 17, 3.5), (1000, 0, -2.0), (4096, 4095, 0.0), (257, 100, -0.0),
                      (248320, 123456, 7.0)):
        row = np.full(V, -np.inf, dtype=np.float32)
        row[hot] = v
        words, L = o.row(row, token=hot, K=20)
        assert words[0] == hot and words[1] == 0, (V, hot, words[:2])
        ids, vals = pairs(words)
        assert ids[0] == hot and bits(vals[0]) == 0
        rest = [i for i in range(V) if i != hot][:19]
        assert ids[1:1 + len(rest)].tolist() == rest
        assert np.all(np.isneginf(vals[1:1 + len(rest)]))


def pin_library_logsumexp(o):
    """L agrees with torch.logsumexp in float64 to within one FP32 ulp, and
    each reported value is one FP32 subtraction away from that L."""
    rng = np.random.default_rng(13)
    cases = []
    for V in (32000, 151936, 262144):
        cases.append((rng.standard_normal(V) * 3).astype(np.float32))
    g = rng.gumbel(size=248320)
    g[rng.integers(248320)] += 10
    cases.append(synth.bf16_bits(g.astype(np.float32)))
    cases.append((rng.standard_normal(50000) * 30 + 500).astype(np.float32))
    for row in cases:
        xs = synth.bf16_to_f32(row) if row.dtype == np.uint16 else row
        V = xs.size
        ref = float(torch.logsumexp(torch.from_numpy(xs.astype(np.float64)), 0))
        tok = int(rng.integers(V))
        words, L = o.row(row, token=tok, K=20)
        assert abs(float(L) - ref) <= ulp32(ref), (V, L, ref)
        assert from_bits(words[1]) == f32(xs[tok] - f32(L))
        assert abs(float(from_bits(words[1])) - (float(xs[tok]) - ref)) <= 2e-5


# ------------------------------------------------------------------ ordering
def _rank_order(vals: np.ndarray) -> list[int]:
    """The order given by pos(i) = #{j: v_j > v_i} + #{j: v_j == v_i, j < i}."""
    n = len(vals)
    pos = [sum(1 for j in range(n) if vals[j] > vals[i]) +
           sum(1 for j in range(i) if vals[j] == vals[i]) for i in range(n)]
    order = [0] * n
    for i, p in enumerate(pos):
        order[p] = i
    return order


def _check_full_listing(o, row_f32: np.ndarray):
    V = row_f32.size
    words, L = o.row(row_f32, token=0, K=20)
    ids, vals = pairs(words)
    expect_vals = (row_f32 - f32(L)).astype(np.float32)
    expect_vals[expect_vals == 0] = 0.0  # -0 is reported as +0
    order = _rank_order(expect_vals)
    assert ids[:V].tolist() == order, (row_f32, ids[:V], order)
    for k, i in enumerate(order):
        assert bits(vals[k]) == bits(expect_vals[i]), (row_f32, k, vals[k], expect_vals[i])
    t = torch.sort(torch.from_numpy(expect_vals), descending=True, stable=True)
    assert t.indices.tolist() == order
    assert np.all(ids[V:] == -1) and np.all(words[3 + 2 * V::2] == NAN_BITS)


def pin_brute_force_order(o):
    """Exhaustive small rows over {-inf, -2, -1, -0, +0, 1, 2}: the listed
    order is decreasing reported value, then increasing ID (GLP definition
    paragraph), equal to a stable library sort."""
    values = np.array([-np.inf, -2.0, -1.0, -0.0, 0.0, 1.0, 2.0], dtype=np.float32)
    for V in range(1, 5):
        for combo in itertools.product(range(len(values)), repeat=V):
            row = values[list(combo)]
            if np.all(np.isneginf(row)):
                continue  # an all -inf row is outside the contract
            _check_full_listing(o, row)
    rng = np.random.default_rng(14)
    for _ in range(1500):
        V = int(rng.integers(5, 11))
        row = values[rng.integers(0, len(values), size=V)]
        if np.all(np.isneginf(row)):
            continue
        _check_full_listing(o, row)


def pin_all_equal_row(o):
    """An all-equal row lists IDs 0..K-1."""
    for V, c in ((1000, 0.0), (248320, -3.0), (40, 1e-3)):
        words, _ = o.row(np.full(V, c, dtype=np.float32), token=5, K=20)
        assert pairs(words)[0].tolist() == list(range(20))


def pin_grid_row_by_counting(o):
    """Rows on a 1/8 grid: the top-K is the smallest IDs at the highest
    level, then at the next level, and so on (found here by counting)."""
    rng = np.random.default_rng(15)
    for V in (4096, 30000):
        k = rng.integers(0, 129, size=V)
        row = (k / 8.0 - 8.0).astype(np.float32)
        want = []
        for level in sorted(set(k.tolist()), reverse=True):
            want += np.nonzero(k == level)[0].tolist()
            if len(want) >= 20:
                break
        words, _ = o.row(synth.bf16_bits(row), token=0, K=20)
        assert pairs(words)[0].tolist() == want[:20]


def pin_subtraction_tie(o):
    """Designed row where two different logits round to the same reported
    value: x0 = nextafter(1, 0), x1 = 1, x2 = 100, the rest -inf.  L is
    exactly 100, both x0 - L and x1 - L round to -99, so the tie goes to the
    smaller ID and the order starts [2, 0, 1] (GLP tiled-reduction paragraph:
    ties created by the subtraction are ties)."""
    V = 64
    row = np.full(V, -np.inf, dtype=np.float32)
    row[0] = np.nextafter(np.float32(1.0), np.float32(0.0))
    row[1] = 1.0
    row[2] = 100.0
    words, L = o.row(row, token=1, K=20)
    assert L == f32(100.0)
    ids, vals = pairs(words)
    assert ids[:3].tolist() == [2, 0, 1]
    assert vals[1] == f32(-99.0) and vals[2] == f32(-99.0) and bits(vals[0]) == 0
    assert ids[3:20].tolist() == list(range(3, 20))


def pin_signed_zero(o):
    """A reported -0 is stored as +0 (GLP tiled-reduction paragraph; the
    stored bits are reading R4)."""
    row = np.full(32, -np.inf, dtype=np.float32)
    row[9] = -0.0
    words, L = o.row(row, token=9, K=3)
    assert words[0] == 9 and words[1] == 0
    ids, vals = pairs(words)
    assert ids[0] == 9 and bits(vals[0]) == 0
    row16 = synth.bf16_bits(row)
    assert row16[9] == 0x8000
    words, _ = o.row(row16, token=9, K=3, sel=[9, 9])
    assert words[1] == 0 and words[3] == 0 and words[5] == 0


def pin_v_below_k(o):
    """When V < K the unused alternative IDs are -1 (GLP packed-position
    paragraph) with NaN bits (reading R5)."""
    rng = np.random.default_rng(16)
    for V in range(1, 20):
        row = (rng.standard_normal(V) * 2).astype(np.float32)
        words, _ = o.row(row, token=0, K=20)
        assert len(words) == 42
        ids, _ = pairs(words)
        assert sorted(ids[:V].tolist()) == list(range(V))
        assert np.all(ids[V:] == -1)
        assert np.all(words[3 + 2 * V::2] == NAN_BITS)


def pin_selected_ids(o):
    """Selected IDs keep caller order, share the chosen token's value when
    equal to it, and IDs outside [0, V) get NaN bits (GLP definition
    paragraph; reading R7)."""
    rng = np.random.default_rng(17)
    V = 3000
    row = (rng.standard_normal(V) * 3).astype(np.float32)
    sel = rng.choice(V, size=128, replace=False).astype(np.int32)
    tok = int(sel[77])
    words, L = o.row(row, token=tok, K=20, sel=sel)
    assert len(words) == 2 + 2 * 128
    ids, vals = pairs(words)
    assert np.array_equal(ids, sel)
    assert bits(vals[77]) == words[1]
    assert np.array_equal(vals, (row[sel] - f32(L)).astype(np.float32))
    bad = np.array([-1, V, V + 5, 2**31 - 1, 5, 5], dtype=np.int32)
    words, _ = o.row(row, token=V, K=20, sel=bad)
    ids, vals = pairs(words)
    assert np.array_equal(ids, bad)
    assert words[1] == NAN_BITS
    assert np.all(words[3:3 + 8:2] == NAN_BITS)
    assert vals[4] == vals[5] == f32(row[5] - f32(L))
    words, _ = o.row(row, token=0, K=20, sel=np.arange(200, dtype=np.int32))
    assert len(words) == 2 + 2 * 128  # counts clamp to 128


# ------------------------------------------------------------- frame gating
def pin_frame_gating(o):
    """Only active positions are written and nothing else changes (GLP gating
    and zero-flag paragraphs; MTP round section); rows are s*T + t; padded
    lanes never enter; word 0 is the chosen token."""
    cap, T, V, V_pad = 6, 3, 50, 64
    rows = cap * T
    logits = np.full((rows, V_pad), np.inf, dtype=np.float32)  # +inf pads
    rng = np.random.default_rng(18)
    hot = [(r * 7 + 3) % V for r in range(rows)]
    for r in range(rows):
        logits[r, :V] = rng.standard_normal(V).astype(np.float32)
        logits[r, hot[r]] = 20.0
    requested = np.array([1, 0, 1, 1, 1, 1], dtype=np.int32)
    emitted = np.array([2, 3, 0, 7, -1, 3], dtype=np.int32)
    id_counts = np.array([-5, 4, 3, 0, 0, 300], dtype=np.int32)
    ids = np.full(cap * 128, -2, dtype=np.int32)
    ids[5 * 128:6 * 128] = np.arange(128) % V
    ids[1 * 128:1 * 128 + 4] = [1, 2, 3, 4]
    tokens = (np.arange(rows, dtype=np.int32) * 5) % V
    out = np.full((cap, T, 258), -559038737, dtype=np.int32)
    n, lse = o.frame(logits, cap, T, V, V_pad, requested, id_counts, ids, emitted, tokens,
                     20, out)
    active = {(0, 0), (0, 1), (3, 0), (3, 1), (3, 2), (5, 0), (5, 1), (5, 2)}
    assert n == len(active)
    for s in range(cap):
        for t in range(T):
            cell = out[s, t]
            if (s, t) not in active:
                assert np.all(cell == -559038737), (s, t)
                continue
            r = s * T + t
            W = 128 if s == 5 else 20
            assert np.all(cell[2 + 2 * W:] == -559038737), (s, t)
            assert cell[0] == tokens[r]
            assert np.isfinite(lse[r]) and float(lse[r]) >= 20.0
            if s == 5:
                assert np.array_equal(cell[2:2 + 256:2], np.arange(128) % V)
            else:
                assert cell[2] == hot[r], (s, t, cell[2], hot[r])
                assert float(from_bits(cell[3])) > -1e-3


# ------------------------------------------------------------ packed target rows
def packed_case(dtype=np.float32, seed=19):
    """A rectangular frame and the same rows packed into P < capacity * T
    physical rows in a shuffled slot order, each slot's committed rows
    followed directly by another slot's (MTP design page, graph catalog
    paragraph).  The packed buffer has capacity * T rows, those past P and
    the uncommitted ones NaN, so a reader of the wrong row sees NaN."""
    cap, T, V, V_pad = 7, 4, 90, 96
    rng = np.random.default_rng(seed)
    rect = np.full((cap * T, V_pad), np.nan, dtype=np.float32)
    rect[:, :V] = (rng.standard_normal((cap * T, V)) * 3).astype(np.float32)
    requested = np.array([1, 1, 0, 1, 1, 1, 1], dtype=np.int32)
    emitted = np.array([2, 4, 3, 0, 1, 3, 9], dtype=np.int32)  # slot 6 clamps to T
    id_counts = np.array([0, 5, 0, 0, 0, 0, 0], dtype=np.int32)
    ids = np.full(cap * 128, -2, dtype=np.int32)
    ids[128:133] = [3, 80, 3, 0, 89]
    tokens = (np.arange(cap * T, dtype=np.int32) * 7) % V
    order = rng.permutation(cap)
    offsets = np.zeros(cap, dtype=np.int32)
    P = 0
    for s in order:
        e = 0 if requested[s] == 0 else min(max(int(emitted[s]), 0), T)
        offsets[s] = P
        P += e
    packed = np.full((cap * T, V_pad), np.nan, dtype=np.float32)
    for s in range(cap):
        e = 0 if requested[s] == 0 else min(max(int(emitted[s]), 0), T)
        packed[offsets[s]:offsets[s] + e] = rect[s * T:s * T + e]
    if dtype == np.uint16:
        rect, packed = synth.bf16_bits(rect), synth.bf16_bits(packed)
    return dict(cap=cap, T=T, V=V, V_pad=V_pad, P=P, rect=rect, packed=packed,
                requested=requested, emitted=emitted, id_counts=id_counts, ids=ids,
                tokens=tokens, offsets=offsets)


def pin_packed_rows_equal_rectangular(o):
    """Packing the committed rows (any slot order, P < capacity * T) changes
    no output word; a slot whose committed rows would pass P writes nothing."""
    for dt in (np.float32, np.uint16):
        c = packed_case(dt)
        assert c["P"] < c["cap"] * c["T"]
        args = (c["requested"], c["id_counts"], c["ids"], c["emitted"], c["tokens"])
        ref = np.full((c["cap"], c["T"], 258), -559038737, dtype=np.int32)
        n_ref, lse_ref = o.frame(c["rect"], c["cap"], c["T"], c["V"], c["V_pad"], *args, 20, ref)
        got = np.full_like(ref, -559038737)
        n, lse = o.frame_packed(c["packed"], c["cap"], c["T"], c["P"], c["V"], c["V_pad"],
                                *args, c["offsets"], 20, got)
        assert n == n_ref and np.array_equal(got, ref)
        assert np.array_equal(np.isnan(lse), np.isnan(lse_ref))
        # slot 1's rows pushed past P: slot 1 becomes inactive, nothing else changes
        off = c["offsets"].copy()
        off[1] = c["P"] - 2  # 4 committed rows from P - 2
        got = np.full_like(ref, -559038737)
        n, _ = o.frame_packed(c["packed"], c["cap"], c["T"], c["P"], c["V"], c["V_pad"],
                              *args, off, 20, got)
        assert n == n_ref - 4
        assert np.all(got[1] == -559038737)
        keep = [s for s in range(c["cap"]) if s != 1]
        assert np.array_equal(got[keep], ref[keep])


# ------------------------------------------------------------ completion records
def pin_records_equal_int32_inputs(o):
    """Reading the emitted count from a record field and the tokens from
    fields 16 + t (GLP buffer table) gives the frame of the same values
    passed as int32 arrays; an out-of-range count reads as 0 and an
    out-of-range token as -1 (reading R14).  Without ID inputs each position
    holds exactly 2 + 2K words: the natural words of the 258-word frame."""
    cap, T, V = 6, 3, 50
    rng = np.random.default_rng(23)
    logits = (rng.standard_normal((cap * T, V)) * 3).astype(np.float32)
    requested = np.array([1, 1, 0, 1, 1, 1], dtype=np.int32)
    field = 5
    rec = rng.integers(-2**40, 2**40, size=(cap, 16 + T)).astype(np.int64)  # metadata noise
    counts = np.array([2, 3, 1, 2**40 + 2, -4, 7], dtype=np.int64)  # 2^40 + 2 would truncate to 2
    rec[:, field] = counts
    toks = rng.integers(0, V, size=(cap, T)).astype(np.int64)
    toks[1, 1] = 2**33  # outside int32: -1
    toks[5, 0] = -7
    rec[:, 16:] = toks
    emitted = np.array([2, 3, 1, 0, 0, 3], dtype=np.int32)  # R14 read by hand, clamped to T
    tokens = np.where((toks < -2**31) | (toks >= 2**31), -1, toks).astype(np.int32).reshape(-1)
    id_counts = np.array([0, 4, 0, 0, 0, 0], dtype=np.int32)
    ids = np.full(cap * 128, -2, dtype=np.int32)
    ids[128:132] = [7, 49, 0, 7]
    ref = np.full((cap, T, 258), -559038737, dtype=np.int32)
    n_ref, _ = o.frame(logits, cap, T, V, V, requested, id_counts, ids, emitted, tokens, 20, ref)
    got = np.full_like(ref, -559038737)
    n, _ = o.frame_records(logits, cap, T, V, V, requested, id_counts, ids, rec, field, 20, got)
    assert n == n_ref == 8 and np.array_equal(got, ref)
    assert ref[1, 1, 0] == -1 and ref[1, 1, 1] == NAN_BITS
    # no ID inputs: natural everywhere, 2 + 2K words per position
    ref0 = np.full((cap, T, 258), -559038737, dtype=np.int32)
    o.frame(logits, cap, T, V, V, requested, np.zeros(cap, np.int32), ids, emitted, tokens, 7, ref0)
    got0 = np.full((cap, T, 16), -559038737, dtype=np.int32)
    o.frame_records(logits, cap, T, V, V, requested, None, None, rec, field, 7, got0)
    assert np.array_equal(got0, ref0[:, :, :16])


# ------------------------------------------------------------ prompt scoring
def _prompt_words_check(o, row, target, V=None):
    """Check one scored row against facts derived without the oracle's rank
    loop: the count of strictly greater reported values (numpy), the first
    position of the target's value in a stable descending library sort, and
    the generation listing of the same row (GLP, prompt-logprobs paragraphs)."""
    V = row.shape[-1] if V is None else V
    words, L = o.prompt_row(row, target, V=V)
    xs = (synth.bf16_to_f32(row) if row.dtype == np.uint16 else row)[:V].astype(np.float32)
    rep = (xs - f32(L)).astype(np.float32)
    rep[rep == 0] = 0.0
    rt = rep[target]
    assert words[0] == target and words[1] == bits(rt), (words[:3], rt)
    greater = int(np.count_nonzero(rep > rt))
    assert words[2] == 1 + greater, (words[2], greater)
    t = torch.sort(torch.from_numpy(rep), descending=True, stable=True)
    first = int(np.nonzero(t.values.numpy() == rt)[0][0])
    assert words[2] == 1 + first
    gen, L2 = o.row(row, token=target, K=20, V=V)
    assert L2 == L and np.array_equal(words[3:], gen[2:]), (words[3:9], gen[2:8])
    return words


def pin_prompt_rank_by_counting(o):
    """Integer-valued logits (no subtraction can tie two of them): the rank is
    one plus the number of larger raw logits; checked for the top, middle and
    bottom targets, FP32 and bf16."""
    rng = np.random.default_rng(21)
    for V in (1, 5, 19, 20, 21, 1000, 30000):
        row = rng.integers(-8, 9, size=V).astype(np.float32)
        for target in {0, V // 2, V - 1, int(np.argmax(row)), int(np.argmin(row))}:
            w = _prompt_words_check(o, row, target)
            assert w[2] == 1 + int(np.count_nonzero(row > row[target]))
            w16 = _prompt_words_check(o, synth.bf16_bits(row), target)
            assert w16[2] == w[2]
    # Ranks of all targets of a permutation row are 1..V.
    V = 257
    row = rng.permutation(V).astype(np.float32) - 100.0
    ranks = sorted(int(o.prompt_row(row, t)[0][2]) for t in range(V))
    assert ranks == list(range(1, V + 1))


def pin_prompt_subtraction_tie(o):
    """x0 = nextafter(1, 0), x1 = 1, x2 = 100, the rest -inf: L = 100 and both
    x0 - L and x1 - L round to -99, so neither is strictly greater than the
    other (rank 2 for both), x2 ranks 1 and a -inf lane ranks 4."""
    V = 64
    row = np.full(V, -np.inf, dtype=np.float32)
    row[0] = np.nextafter(np.float32(1.0), np.float32(0.0))
    row[1] = 1.0
    row[2] = 100.0
    for target, rank in ((0, 2), (1, 2), (2, 1), (3, 4), (63, 4)):
        words, L = o.prompt_row(row, target)
        assert L == f32(100.0) and words[2] == rank, (target, words[2], rank)
        _prompt_words_check(o, row, target)
    assert o.prompt_row(row, 0)[0][1] == bits(f32(-99.0))


def pin_prompt_invalid_rows(o):
    """Targets outside [0, V) (-1 at the prompt end and in image spans) give
    ID -1, NaN bits, rank 0 and alternative IDs -1 (GLP, prompt-logprobs
    paragraphs; the alternatives' NaN bits are reading R12)."""
    row = np.arange(50, dtype=np.float32)
    want = np.array([-1, NAN_BITS, 0] + [-1, NAN_BITS] * 20, dtype=np.int64).astype(np.int32)
    for target in (-1, -7, 50, 51, 2**31 - 1):
        words, L = o.prompt_row(row, target)
        assert np.array_equal(words, want), (target, words[:5])
        assert math.isnan(L)


def pin_prompt_small_rows_exhaustive(o):
    """Every row of length 1..4 over {-inf, -2, -1, -0, +0, 1, 2} and every
    target: rank and listing against counting and a stable sort."""
    values = np.array([-np.inf, -2.0, -1.0, -0.0, 0.0, 1.0, 2.0], dtype=np.float32)
    for V in range(1, 5):
        for combo in itertools.product(range(len(values)), repeat=V):
            row = values[list(combo)]
            if np.all(np.isneginf(row)):
                continue
            for target in range(V):
                _prompt_words_check(o, row, target)


def pin_prompt_chunk(o):
    """A chunk of rows with V_pad > V (+inf pads that must not count), valid
    and invalid targets: row r uses logits row r and target r, and the valid
    count is returned."""
    rows, V, V_pad = 9, 300, 320
    rng = np.random.default_rng(22)
    logits = np.full((rows, V_pad), np.inf, dtype=np.float32)
    logits[:, :V] = (rng.standard_normal((rows, V)) * 3).astype(np.float32)
    targets = np.array([5, -1, 299, 0, 300, 17, -1, 150, 2], dtype=np.int32)
    out = np.full((rows, 43), -559038737, dtype=np.int32)
    n, lse = o.prompt(logits, rows, V, V_pad, targets, out)
    assert n == 6
    for r in range(rows):
        if 0 <= targets[r] < V:
            xs = logits[r, :V]
            assert out[r, 0] == targets[r]
            assert out[r, 2] == 1 + int(np.count_nonzero(xs > xs[targets[r]]))
            ref = float(torch.logsumexp(torch.from_numpy(xs.astype(np.float64)), 0))
            assert abs(float(lse[r]) - ref) <= ulp32(ref)
        else:
            assert out[r, 0] == -1 and out[r, 2] == 0 and math.isnan(lse[r])


ALL_PINS = [pin_uniform_row, pin_uniform_row_bf16, pin_two_level_row,
            pin_probabilities_sum_to_one, pin_one_hot, pin_library_logsumexp,
            pin_brute_force_order, pin_all_equal_row, pin_grid_row_by_counting,
            pin_subtraction_tie, pin_signed_zero, pin_v_below_k, pin_selected_ids,
            pin_frame_gating, pin_prompt_rank_by_counting, pin_prompt_subtraction_tie,
            pin_prompt_invalid_rows, pin_prompt_small_rows_exhaustive, pin_prompt_chunk,
            pin_packed_rows_equal_rectangular, pin_records_equal_int32_inputs]
