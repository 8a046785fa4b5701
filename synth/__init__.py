"""Seeded synthetic workloads for the generation-logprob reduction.

This package makes inputs and nothing else: it holds none of the reduction's
arithmetic.  The oracle's tests, the GPU parity tests and the benchmark all
draw from it, so both sides of every comparison see identical bytes.

The five named workloads follow the verify workloads the reduction serves
(decode rows, a padded decode batch, a speculative-verify frame, a tie-heavy
mixed frame and a large batch).  Every random choice is a pure function of
(seed, stream tag, row, lane) through SplitMix64 (see ``synth.c``), so each
row can be regenerated alone.

Stream tags: logits 1, chosen tokens 2, emitted counts 3, request flags 4,
selected IDs 5, spike lane 6, one-hot rows 7, prompt targets 8.

Prompt scoring (scored prefill) has its own chunk specs (``PROMPT_CONFIGS``):
one logit row per prompt position and one target per row.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "synth.c")
LIB = os.path.join(HERE, "libsynth.so")

FP32, BF16 = 0, 1
NORMAL, GUMBEL, GRID8 = 0, 1, 2
PAD_ZERO, PAD_PINF, PAD_NAN = 0, 1, 2
TAG_TOKENS, TAG_EMITTED, TAG_REQUESTED, TAG_IDS = 2, 3, 4, 5
TAG_SPIKE, TAG_TARGETS = 6, 8
PROMPT_WORDS = 43
MAX_IDS = 128
ROW_WORDS = 258
POISON = np.int32(-559038737)  # 0xDEADBEEF
UNUSED_ID = -2                 # filler for ID slots past a slot's count


def build(out: str = LIB) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", SRC, "-o", out,
           "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        c = ctypes
        L.synth_hash.restype = c.c_uint64
        L.synth_hash.argtypes = [c.c_uint64] * 4
        L.synth_hashes.restype = None
        L.synth_hashes.argtypes = [c.c_void_p, c.c_int64, c.c_uint64, c.c_uint64,
                                   c.c_uint64, c.c_uint64]
        L.synth_fill.restype = c.c_int
        L.synth_fill.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int64, c.c_int32,
                                 c.c_int32, c.c_int, c.c_double, c.c_double,
                                 c.c_uint64, c.c_void_p, c.c_int, c.c_int]
        _lib = L
    return _lib


def hash64(seed: int, tag: int, row: int, lane: int = 0) -> int:
    return int(lib().synth_hash(seed, tag, row, lane))


def hashes(n: int, seed: int, tag: int, row: int, lane0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    lib().synth_hashes(out.ctypes.data, n, seed, tag, row, lane0)
    return out


@dataclasses.dataclass
class Spec:
    """Shape, value recipe and gating of one workload."""
    name: str
    capacity: int
    T: int
    V: int
    V_pad: int
    dtype: int                 # FP32 or BF16
    recipe: int                # NORMAL, GUMBEL or GRID8
    p0: float = 0.0            # sigma (NORMAL) or one-hot period (GRID8)
    p1: float = 0.0            # spike added at one seeded lane per row
    pad: int = PAD_ZERO
    K: int = 20
    requesting: str = "all"    # "all" | "half"
    emitted: str = "all"       # "all" (=T) | "one" | "uniform" (1..T)
    selected: str = "none"     # "none" | "frac40" | "all"
    seed: int = 1
    description: str = ""

    def with_(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "C1": Spec("C1", 8, 1, 32000, 32000, FP32, NORMAL, p0=3.0, emitted="one", seed=1,
               description="plain decode: 8 rows x V=32,000 FP32 ~ N(0,3), K=20"),
    "C2": Spec("C2", 64, 1, 151936, 152064, FP32, NORMAL, p0=4.0, p1=15.0, pad=PAD_PINF,
               requesting="half", emitted="one", seed=2,
               description="decode batch: 64 slots x V=151,936 (V_pad 152,064, +inf pads) "
                           "FP32 ~ N(0,4) + 15 spike, half requesting, K=20"),
    "C3": Spec("C3", 128, 8, 248320, 248320, BF16, GUMBEL, p1=10.0, emitted="uniform",
               seed=3,
               description="speculative verify: 128 slots x T=8 x V=248,320 bf16 Gumbel + 10 "
                           "peak, emitted 1..8, K=20"),
    "C4": Spec("C4", 128, 8, 248320, 248320, BF16, GRID8, p0=8.0, emitted="uniform",
               selected="frac40", seed=4,
               description="tie stress: 128 slots x T=8 x V=248,320 bf16 on a 1/8 grid in "
                           "[-8,8], 1 in 8 rows one-hot, 40% of slots with 128 selected IDs"),
    "C5": Spec("C5", 1024, 4, 262144, 262144, FP32, NORMAL, p0=3.0, emitted="all", seed=5,
               description="large batch: 1,024 slots x T=4 x V=262,144 FP32 ~ N(0,3), K=20"),
}


@dataclasses.dataclass
class Workload:
    spec: Spec
    logits: np.ndarray         # [capacity*T, V_pad] float32, or uint16 bf16 bits
    requested: np.ndarray      # int32 [capacity]
    emitted: np.ndarray        # int32 [capacity]
    tokens: np.ndarray         # int32 [capacity*T]
    id_counts: np.ndarray      # int32 [capacity]
    ids: np.ndarray            # int32 [capacity*128]

    @property
    def K(self) -> int:
        return self.spec.K

    def active_mask(self) -> np.ndarray:
        """[capacity, T] bool: positions the reduction must reduce."""
        s = self.spec
        e = np.clip(self.emitted, 0, s.T)
        t = np.arange(s.T)[None, :]
        return (self.requested[:, None] != 0) & (t < e[:, None])

    def active_rows(self) -> int:
        return int(self.active_mask().sum())

    def algorithmic_bytes(self) -> int:
        """Bytes the reduction must move: each active row's V logits once, its
        chosen token, its output words and its selected IDs, plus per slot the
        flag, emitted count and ID count."""
        s = self.spec
        b = 2 if s.dtype == BF16 else 4
        m = self.active_mask()
        n = np.clip(self.id_counts, 0, MAX_IDS)
        n = np.where(self.requested != 0, n, 0)
        W = np.where(n > 0, n, s.K)
        per_row = s.V * b + 4 + 4 * (2 + 2 * W) + 4 * n
        return int((m.sum(axis=1) * per_row).sum() + 12 * s.capacity)

    def poisoned_out(self) -> np.ndarray:
        s = self.spec
        return np.full((s.capacity, s.T, ROW_WORDS), POISON, dtype=np.int32)


def _perm_first(n_total: int, n_take: int, seed: int, tag: int, row: int) -> np.ndarray:
    """The first n_take items of a seeded permutation of range(n_total)."""
    h = hashes(n_total, seed, tag, row)
    return np.argsort(h, kind="stable")[:n_take]


def _distinct_ids(V: int, n: int, seed: int, slot: int) -> np.ndarray:
    """n distinct IDs in [0, V) from a seeded partial Fisher-Yates shuffle."""
    n = min(n, V)
    h = hashes(n, seed, TAG_IDS, slot, 1)
    perm: dict[int, int] = {}
    out = np.empty(n, dtype=np.int32)
    for j in range(n):
        r = j + int(h[j] % np.uint64(V - j))
        pj, pr = perm.get(j, j), perm.get(r, r)
        perm[j], perm[r] = pr, pj
        out[j] = pr
    return out


def gating(spec: Spec):
    """(requested, emitted, tokens, id_counts, ids) for a spec."""
    s = spec
    requested = np.ones(s.capacity, dtype=np.int32)
    if s.requesting == "half":
        requested[:] = 0
        requested[_perm_first(s.capacity, s.capacity // 2, s.seed, TAG_REQUESTED, 0)] = 1
    if s.emitted == "all":
        emitted = np.full(s.capacity, s.T, dtype=np.int32)
    elif s.emitted == "one":
        emitted = np.ones(s.capacity, dtype=np.int32)
    elif s.emitted == "uniform":
        h = np.array([hash64(s.seed, TAG_EMITTED, i) for i in range(s.capacity)],
                     dtype=np.uint64)
        emitted = (1 + (h % np.uint64(s.T))).astype(np.int32)
    else:
        raise ValueError(s.emitted)
    tokens = np.empty(s.capacity * s.T, dtype=np.int32)
    for r in range(s.capacity * s.T):
        tokens[r] = hash64(s.seed, TAG_TOKENS, r) % s.V
    id_counts = np.zeros(s.capacity, dtype=np.int32)
    ids = np.full(s.capacity * MAX_IDS, UNUSED_ID, dtype=np.int32)
    if s.selected == "frac40":
        sel_slots = _perm_first(s.capacity, int(0.4 * s.capacity), s.seed, TAG_IDS, 1 << 40)
    elif s.selected == "all":
        sel_slots = np.arange(s.capacity)
    else:
        sel_slots = np.zeros(0, dtype=np.int64)
    for sl in sel_slots:
        d = _distinct_ids(s.V, MAX_IDS, s.seed, int(sl))
        id_counts[sl] = len(d)
        ids[sl * MAX_IDS: sl * MAX_IDS + len(d)] = d
    return requested, emitted, tokens, id_counts, ids


def garbage_rows(spec: Spec, requested: np.ndarray, emitted: np.ndarray) -> np.ndarray:
    """uint8 [capacity*T]: 1 for rows the reduction must never read."""
    t = np.arange(spec.T)[None, :]
    act = (requested[:, None] != 0) & (t < np.clip(emitted, 0, spec.T)[:, None])
    return (~act).reshape(-1).astype(np.uint8)


def fill_logits(spec: Spec, out: np.ndarray, garbage: np.ndarray | None,
                row_begin: int = 0, nthreads: int | None = None) -> np.ndarray:
    """Fill `out` ([rows, V_pad], float32 or uint16) with global rows
    [row_begin, row_begin + rows) of the workload."""
    s = spec
    want = np.uint16 if s.dtype == BF16 else np.float32
    assert out.dtype == want and out.flags.c_contiguous and out.shape[-1] == s.V_pad
    rows = out.shape[0]
    if nthreads is None:
        nthreads = min(16, os.cpu_count() or 1)
    g = None
    if garbage is not None:
        g = np.ascontiguousarray(garbage, dtype=np.uint8)
        assert g.size >= row_begin + rows
    rc = lib().synth_fill(out.ctypes.data, s.dtype, row_begin, row_begin + rows, s.V, s.V_pad,
                          s.recipe, float(s.p0), float(s.p1), s.seed,
                          None if g is None else g.ctypes.data, s.pad, nthreads)
    if rc != 0:
        raise RuntimeError("synth_fill failed")
    return out


def make(spec: Spec | str, logits_out: np.ndarray | None = None, **overrides) -> Workload:
    """Generate a whole workload.  `logits_out` may supply the destination
    buffer (e.g. a pinned host tensor's numpy view)."""
    if isinstance(spec, str):
        spec = CONFIGS[spec]
    if overrides:
        spec = spec.with_(**overrides)
    requested, emitted, tokens, id_counts, ids = gating(spec)
    garbage = garbage_rows(spec, requested, emitted)
    rows = spec.capacity * spec.T
    want = np.uint16 if spec.dtype == BF16 else np.float32
    if logits_out is None:
        logits_out = np.empty((rows, spec.V_pad), dtype=want)
    fill_logits(spec, logits_out, garbage)
    return Workload(spec, logits_out, requested, emitted, tokens, id_counts, ids)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (for hand-made rows)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + r) >> np.uint64(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------ prompt scoring
# A chunk spec reuses Spec with capacity = rows and T = 1 (the other gating
# fields are unused).  Targets: the row's last position and a span of image
# positions are -1; of the rest, half are the row's spike lane (the token the
# model favours, rank 1) and half a uniform ID (a deep rank: most of the
# vocabulary above it).
PROMPT_CONFIGS = {
    "P1": Spec("P1", 128, 1, 248320, 248320, BF16, GUMBEL, p1=10.0, seed=8,
               description="scored prefill chunk: 128 rows x V=248,320 bf16 Gumbel + 10 peak; "
                           "targets: 1/2 the peak lane, 1/2 uniform, an image span and the "
                           "prompt end -1"),
    "P2": Spec("P2", 512, 1, 151936, 152064, FP32, NORMAL, p0=4.0, p1=15.0, pad=PAD_PINF,
               seed=9,
               description="scored prefill chunk: 512 rows x V=151,936 (V_pad 152,064, +inf "
                           "pads) FP32 ~ N(0,4) + 15 peak; targets as P1"),
}


@dataclasses.dataclass
class PromptWorkload:
    spec: Spec
    logits: np.ndarray         # [rows, V_pad] float32, or uint16 bf16 bits
    targets: np.ndarray        # int32 [rows]; -1 marks an invalid row

    @property
    def rows(self) -> int:
        return self.spec.capacity

    def valid_rows(self) -> int:
        return int(((self.targets >= 0) & (self.targets < self.spec.V)).sum())

    def algorithmic_bytes(self) -> int:
        """Each valid row's V logits once plus its target; every row's target
        and 43 output words."""
        s = self.spec
        b = 2 if s.dtype == BF16 else 4
        return int(self.valid_rows() * s.V * b + self.rows * (4 + 4 * PROMPT_WORDS))

    def poisoned_out(self) -> np.ndarray:
        return np.full((self.rows, PROMPT_WORDS), POISON, dtype=np.int32)


def prompt_targets(spec: Spec) -> np.ndarray:
    """int32 [rows] targets for a chunk spec (recipe above)."""
    s = spec
    n = s.capacity
    t = np.empty(n, dtype=np.int32)
    for r in range(n):
        h = hash64(s.seed, TAG_TARGETS, r)
        if h & 1:
            t[r] = hash64(s.seed, TAG_SPIKE, r) % s.V if s.p1 != 0.0 else hash64(s.seed, TAG_TARGETS, r, 1) % s.V
        else:
            t[r] = hash64(s.seed, TAG_TARGETS, r, 1) % s.V
    if n >= 4:
        span0 = int(hash64(s.seed, TAG_TARGETS, 1 << 40) % np.uint64(n // 2))
        t[span0:span0 + max(1, n // 16)] = -1  # an image span
    t[n - 1] = -1  # the prompt end
    return t


def make_prompt(spec: Spec | str, logits_out: np.ndarray | None = None,
                **overrides) -> PromptWorkload:
    if isinstance(spec, str):
        spec = PROMPT_CONFIGS[spec]
    if overrides:
        spec = spec.with_(**overrides)
    targets = prompt_targets(spec)
    want = np.uint16 if spec.dtype == BF16 else np.float32
    if logits_out is None:
        logits_out = np.empty((spec.capacity, spec.V_pad), dtype=want)
    garbage = (targets < 0).astype(np.uint8)  # invalid rows are never read
    fill_logits(spec, logits_out, garbage)
    return PromptWorkload(spec, logits_out, targets)
