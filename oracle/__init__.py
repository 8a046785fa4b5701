"""CPU oracle for the generation-logprob reduction (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding)
never does.  The arithmetic lives in ``oracle_logprobs.c``; this module only
builds it with gcc and marshals numpy arrays through ctypes.

Every function is pinned by tests that do not reuse its arithmetic; none is
"parity unpinned" except the conventions listed in the C file's readings
(bit patterns for unused or invalid entries), which the pages do not fix.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_logprobs.c")
LIB = os.path.join(HERE, "liboracle_logprobs.so")

DTYPE_FP32 = 0
DTYPE_BF16 = 1
MAX_IDS = 128
ROW_WORDS = 258
MAX_K = 20
NAN_BITS = 0x7FC00000
PROMPT_WORDS = 43

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra: list[str] | None = None) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", *GCC_FLAGS, *(extra or []), src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class Oracle:
    """ctypes handle on one build of the oracle shared library."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            build(out=path)
        self.path = path
        self.lib = ctypes.CDLL(path)
        c = ctypes
        self.lib.oracle_row_lse.restype = c.c_float
        self.lib.oracle_row_lse.argtypes = [c.c_void_p, c.c_int, c.c_int32]
        self.lib.oracle_row.restype = c.c_int
        self.lib.oracle_row.argtypes = [c.c_void_p, c.c_int, c.c_int32, c.c_int32,
                                        c.c_int32, c.c_void_p, c.c_int32,
                                        c.c_void_p, c.c_void_p]
        self.lib.oracle_row_at_lse.restype = c.c_int
        self.lib.oracle_row_at_lse.argtypes = [c.c_void_p, c.c_int, c.c_int32, c.c_int32,
                                               c.c_int32, c.c_void_p, c.c_int32, c.c_float,
                                               c.c_void_p]
        self.lib.oracle_frame.restype = c.c_int64
        self.lib.oracle_frame.argtypes = [c.c_void_p, c.c_int, c.c_int32, c.c_int32,
                                          c.c_int32, c.c_int32, c.c_void_p,
                                          c.c_void_p, c.c_void_p, c.c_void_p,
                                          c.c_void_p, c.c_int32, c.c_void_p,
                                          c.c_void_p]
        self.lib.oracle_frame_packed.restype = c.c_int64
        self.lib.oracle_frame_packed.argtypes = [c.c_void_p, c.c_int, c.c_int32, c.c_int32,
                                                 c.c_int32, c.c_int32, c.c_int32, c.c_void_p,
                                                 c.c_void_p, c.c_void_p, c.c_void_p,
                                                 c.c_void_p, c.c_void_p, c.c_int32,
                                                 c.c_void_p, c.c_void_p]
        self.lib.oracle_frame_records.restype = c.c_int64
        self.lib.oracle_frame_records.argtypes = [c.c_void_p, c.c_int, c.c_int32, c.c_int32,
                                                  c.c_int32, c.c_int32, c.c_void_p, c.c_void_p,
                                                  c.c_void_p, c.c_void_p, c.c_int32, c.c_int32,
                                                  c.c_int32, c.c_void_p, c.c_void_p]
        self.lib.oracle_prompt_row.restype = c.c_int
        self.lib.oracle_prompt_row.argtypes = [c.c_void_p, c.c_int, c.c_int32, c.c_int32,
                                               c.c_void_p, c.c_void_p]
        self.lib.oracle_prompt.restype = c.c_int64
        self.lib.oracle_prompt.argtypes = [c.c_void_p, c.c_int, c.c_int32, c.c_int32,
                                           c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p]

    @staticmethod
    def _dtype_of(a: np.ndarray) -> int:
        if a.dtype == np.float32:
            return DTYPE_FP32
        if a.dtype == np.uint16:  # bf16 bit patterns
            return DTYPE_BF16
        raise TypeError(f"logits must be float32 or uint16 (bf16 bits), got {a.dtype}")

    def row_lse(self, row: np.ndarray, V: int | None = None) -> float:
        row = np.ascontiguousarray(row)
        V = row.shape[-1] if V is None else V
        return float(self.lib.oracle_row_lse(row.ctypes.data, self._dtype_of(row), V))

    def row(self, row: np.ndarray, token: int, K: int, sel=None, V: int | None = None):
        """One emitted position.  Returns (words[2 + 2W] as int32, L)."""
        row = np.ascontiguousarray(row)
        V = row.shape[-1] if V is None else V
        words = np.zeros(ROW_WORDS, dtype=np.int32)
        L = ctypes.c_float(0.0)
        if sel is None or len(sel) == 0:
            sel_arr, n = None, 0
        else:
            sel_arr = np.ascontiguousarray(sel, dtype=np.int32)
            n = len(sel_arr)
        rc = self.lib.oracle_row(row.ctypes.data, self._dtype_of(row), V, int(token), n,
                                 None if sel_arr is None else sel_arr.ctypes.data, K,
                                 words.ctypes.data, ctypes.byref(L))
        if rc < 0:
            raise ValueError("oracle_row rejected its arguments")
        return words[:rc].copy(), float(L.value)

    def row_at(self, row: np.ndarray, token: int, K: int, L: float, sel=None,
               V: int | None = None) -> np.ndarray:
        """The listing of one emitted position for a given FP32 normalization
        L (words[2 + 2W] as int32): what the row reports if its L is L."""
        row = np.ascontiguousarray(row)
        V = row.shape[-1] if V is None else V
        words = np.zeros(ROW_WORDS, dtype=np.int32)
        if sel is None or len(sel) == 0:
            sel_arr, n = None, 0
        else:
            sel_arr = np.ascontiguousarray(sel, dtype=np.int32)
            n = len(sel_arr)
        rc = self.lib.oracle_row_at_lse(row.ctypes.data, self._dtype_of(row), V, int(token), n,
                                        None if sel_arr is None else sel_arr.ctypes.data, K,
                                        float(np.float32(L)), words.ctypes.data)
        if rc < 0:
            raise ValueError("oracle_row_at_lse rejected its arguments")
        return words[:rc].copy()

    def frame(self, logits: np.ndarray, capacity: int, T: int, V: int, V_pad: int,
              requested, id_counts, ids, emitted, tokens, K: int, out: np.ndarray):
        """One frame.  `out` is [capacity, T, 258] int32 and is written in place
        (only active positions).  Returns (active rows, lse[capacity*T])."""
        logits = np.ascontiguousarray(logits)
        assert logits.size >= capacity * T * V_pad
        req = np.ascontiguousarray(requested, dtype=np.int32)
        cnt = np.ascontiguousarray(id_counts, dtype=np.int32)
        idv = np.ascontiguousarray(ids, dtype=np.int32)
        emi = np.ascontiguousarray(emitted, dtype=np.int32)
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        assert req.size == capacity and cnt.size == capacity and emi.size == capacity
        assert idv.size == capacity * MAX_IDS and tok.size == capacity * T
        assert out.dtype == np.int32 and out.size == capacity * T * ROW_WORDS
        assert out.flags.c_contiguous
        lse = np.full(capacity * T, np.nan, dtype=np.float32)
        n = self.lib.oracle_frame(logits.ctypes.data, self._dtype_of(logits), capacity, T,
                                  V, V_pad, req.ctypes.data, cnt.ctypes.data,
                                  idv.ctypes.data, emi.ctypes.data, tok.ctypes.data, K,
                                  out.ctypes.data, lse.ctypes.data)
        if n < 0:
            raise ValueError("oracle_frame rejected its arguments")
        return int(n), lse

    def frame_packed(self, logits: np.ndarray, capacity: int, T: int, P: int, V: int,
                     V_pad: int, requested, id_counts, ids, emitted, tokens, row_offsets,
                     K: int, out: np.ndarray):
        """One frame over P packed logit rows (slot s's row t at row_offsets[s] + t).
        `out` is [capacity, T, 258], written in place.  Returns (active rows, lse)."""
        logits = np.ascontiguousarray(logits)
        assert logits.size >= P * V_pad
        a = lambda x: np.ascontiguousarray(x, dtype=np.int32)  # noqa: E731
        req, cnt, idv, emi, tok, off = (a(requested), a(id_counts), a(ids), a(emitted),
                                        a(tokens), a(row_offsets))
        assert req.size == capacity and cnt.size == capacity and emi.size == capacity
        assert off.size == capacity and idv.size == capacity * MAX_IDS
        assert tok.size == capacity * T
        assert out.dtype == np.int32 and out.size == capacity * T * ROW_WORDS
        assert out.flags.c_contiguous
        lse = np.full(capacity * T, np.nan, dtype=np.float32)
        n = self.lib.oracle_frame_packed(logits.ctypes.data, self._dtype_of(logits), capacity,
                                         T, P, V, V_pad, req.ctypes.data, cnt.ctypes.data,
                                         idv.ctypes.data, emi.ctypes.data, tok.ctypes.data,
                                         off.ctypes.data, K, out.ctypes.data, lse.ctypes.data)
        if n < 0:
            raise ValueError("oracle_frame_packed rejected its arguments")
        return int(n), lse

    def frame_records(self, logits: np.ndarray, capacity: int, T: int, V: int, V_pad: int,
                      requested, id_counts, ids, records, emitted_field: int, K: int,
                      out: np.ndarray):
        """One frame reading counts and tokens from int64 records [capacity, 16 + T].
        id_counts/ids None: natural only, `out` [capacity, T, 2 + 2K]; else 258."""
        logits = np.ascontiguousarray(logits)
        req = np.ascontiguousarray(requested, dtype=np.int32)
        rec = np.ascontiguousarray(records, dtype=np.int64)
        assert rec.size == capacity * (16 + T) and req.size == capacity
        if id_counts is None:
            cnt = idv = None
            words = 2 + 2 * K
        else:
            cnt = np.ascontiguousarray(id_counts, dtype=np.int32)
            idv = np.ascontiguousarray(ids, dtype=np.int32)
            words = ROW_WORDS
        assert out.dtype == np.int32 and out.size == capacity * T * words
        assert out.flags.c_contiguous
        lse = np.full(capacity * T, np.nan, dtype=np.float32)
        n = self.lib.oracle_frame_records(logits.ctypes.data, self._dtype_of(logits), capacity, T,
                                          V, V_pad, req.ctypes.data,
                                          None if cnt is None else cnt.ctypes.data,
                                          None if idv is None else idv.ctypes.data,
                                          rec.ctypes.data, emitted_field, K, words,
                                          out.ctypes.data, lse.ctypes.data)
        if n < 0:
            raise ValueError("oracle_frame_records rejected its arguments")
        return int(n), lse

    def prompt_row(self, row: np.ndarray, target: int, V: int | None = None):
        """One scored prompt row.  Returns (words[43] as int32, L)."""
        row = np.ascontiguousarray(row)
        V = row.shape[-1] if V is None else V
        words = np.zeros(PROMPT_WORDS, dtype=np.int32)
        L = ctypes.c_float(0.0)
        rc = self.lib.oracle_prompt_row(row.ctypes.data, self._dtype_of(row), V, int(target),
                                        words.ctypes.data, ctypes.byref(L))
        if rc < 0:
            raise ValueError("oracle_prompt_row rejected its arguments")
        return words, float(L.value)

    def prompt(self, logits: np.ndarray, rows: int, V: int, V_pad: int, targets,
               out: np.ndarray):
        """A scored chunk.  `out` is [rows, 43] int32, written in place.
        Returns (valid rows, lse[rows])."""
        logits = np.ascontiguousarray(logits)
        assert logits.size >= rows * V_pad
        tg = np.ascontiguousarray(targets, dtype=np.int32)
        assert tg.size == rows
        assert out.dtype == np.int32 and out.size == rows * PROMPT_WORDS
        assert out.flags.c_contiguous
        lse = np.full(rows, np.nan, dtype=np.float32)
        n = self.lib.oracle_prompt(logits.ctypes.data, self._dtype_of(logits), rows, V, V_pad,
                                   tg.ctypes.data, out.ctypes.data, lse.ctypes.data)
        if n < 0:
            raise ValueError("oracle_prompt rejected its arguments")
        return int(n), lse


_DEFAULT: Oracle | None = None


def get() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
