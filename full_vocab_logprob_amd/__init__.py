"""MI355X generation-logprob reduction: Python binding of libflare_logprobs.

This module only marshals arguments.  Every step of the reduction runs in the
HIP kernels behind the C ABI declared in include/flare_logprobs.h; PyTorch
supplies device memory and the current stream.  There is no fallback: if the
shared library is missing the import of a binding function raises.

    plan = Plan(capacity, T, V, V_pad, dtype=torch.bfloat16, K=20)
    ws = plan.workspace()
    plan.run(logits, tokens, emitted_counts, requested, id_counts, ids, out, ws)

Prompt scoring (scored prefill rows: target logprob, rank, twenty
alternatives) has its own plan:

    pplan = PromptPlan(rows, V, V_pad, dtype=torch.bfloat16)
    pplan.run(logits, targets, out, pplan.workspace())

The functions ``flare_logprobs_plan``, ``flare_logprobs_run`` (and its two
launches ``flare_logprobs_reduce`` and ``flare_logprobs_merge``), the packed,
records and vocabulary-sharded variants, the ``flare_prompt_logprobs_*``
counterparts, ``flare_status_string`` and ``flare_logprobs_abi_version``
mirror the C entry points one to one.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libflare_logprobs.so")

ABI_VERSION = 6
MAX_K = 20
MAX_IDS = 128
ROW_WORDS = 258
NAN_BITS = 0x7FC00000
PROMPT_ROW_WORDS = 43
PROMPT_ALTERNATIVES = 20
MODE_GENERATION = 0
MODE_PROMPT = 1
DTYPE_FP32 = 0
DTYPE_BF16 = 1

STATUS = {0: "FLARE_OK", 1: "FLARE_ERR_INVALID_ARGUMENT", 2: "FLARE_ERR_UNSUPPORTED_DTYPE",
          3: "FLARE_ERR_PLAN_MISMATCH", 4: "FLARE_ERR_DEVICE", 5: "FLARE_ERR_LAUNCH",
          6: "FLARE_ERR_UNSUPPORTED_SIZE", 7: "FLARE_ERR_SCRATCH_TOO_SMALL"}


class PlanStruct(ctypes.Structure):
    """Mirror of flare_logprobs_plan_t."""
    _fields_ = [("abi_version", ctypes.c_uint32), ("capacity", ctypes.c_int32),
                ("T", ctypes.c_int32), ("V", ctypes.c_int32), ("V_pad", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("K", ctypes.c_int32), ("device", ctypes.c_int32),
                ("unit_elems", ctypes.c_int32), ("units", ctypes.c_int32),
                ("block", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("vector_rows", ctypes.c_int32), ("cu_count", ctypes.c_int32),
                ("ranges", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64), ("record_offset", ctypes.c_uint64),
                ("lse_offset", ctypes.c_uint64), ("slots_offset", ctypes.c_uint64),
                ("guard_offset", ctypes.c_uint64), ("packed_rows", ctypes.c_int32),
                ("shards", ctypes.c_int32), ("exchange_offset", ctypes.c_uint64),
                ("reserved", ctypes.c_uint32 * 2)]


class FlareError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({flare_status_string(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        c = ctypes
        L.flare_logprobs_plan.restype = c.c_int
        L.flare_logprobs_plan.argtypes = [c.POINTER(PlanStruct), c.c_int32, c.c_int32, c.c_int32,
                                          c.c_int32, c.c_int32, c.c_int32, c.c_int32]
        for name in ("flare_logprobs_run", "flare_logprobs_reduce", "flare_logprobs_merge"):
            f = getattr(L, name)
            f.restype = c.c_int
            f.argtypes = [c.POINTER(PlanStruct), c.c_void_p, c.c_int32, c.c_int64, c.c_int32,
                          c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                          c.c_void_p, c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p]
        L.flare_logprobs_plan_packed.restype = c.c_int
        L.flare_logprobs_plan_packed.argtypes = [c.POINTER(PlanStruct)] + [c.c_int32] * 8
        for name in ("flare_logprobs_run_packed", "flare_logprobs_reduce_packed",
                     "flare_logprobs_merge_packed"):
            f = getattr(L, name)
            f.restype = c.c_int
            f.argtypes = [c.POINTER(PlanStruct), c.c_void_p, c.c_int32, c.c_int64, c.c_int32,
                          c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                          c.c_void_p, c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p]
        L.flare_logprobs_run_records.restype = c.c_int
        L.flare_logprobs_run_records.argtypes = [c.POINTER(PlanStruct), c.c_void_p, c.c_int32,
                                                 c.c_int64, c.c_int32, c.c_int32, c.c_void_p,
                                                 c.c_void_p, c.c_void_p, c.c_void_p, c.c_int32,
                                                 c.c_int32, c.c_void_p, c.c_int32, c.c_void_p,
                                                 c.c_void_p]
        L.flare_prompt_logprobs_plan.restype = c.c_int
        L.flare_prompt_logprobs_plan.argtypes = [c.POINTER(PlanStruct), c.c_int32, c.c_int32,
                                                 c.c_int32, c.c_int32, c.c_int32]
        for name in ("flare_prompt_logprobs_run", "flare_prompt_logprobs_reduce",
                     "flare_prompt_logprobs_merge"):
            f = getattr(L, name)
            f.restype = c.c_int
            f.argtypes = [c.POINTER(PlanStruct), c.c_void_p, c.c_int32, c.c_int64, c.c_int32,
                          c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p]
        L.flare_logprobs_run_noalloc.restype = c.c_int
        L.flare_logprobs_run_noalloc.argtypes = [c.POINTER(PlanStruct), c.c_void_p, c.c_int32,
                                                 c.c_int64, c.c_int32, c.c_int32, c.c_void_p,
                                                 c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                                 c.c_int32, c.c_void_p, c.c_void_p]
        L.flare_logprobs_plan_sharded.restype = c.c_int
        L.flare_logprobs_plan_sharded.argtypes = [c.POINTER(PlanStruct)] + [c.c_int32] * 8
        for name in ("flare_logprobs_run_sharded", "flare_logprobs_shard_merge"):
            f = getattr(L, name)
            f.restype = c.c_int
            f.argtypes = [c.POINTER(PlanStruct), c.c_void_p, c.c_int32, c.c_int64, c.c_int32,
                          c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                          c.c_void_p, c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p]
        L.flare_logprobs_shard_pass.restype = c.c_int
        L.flare_logprobs_shard_pass.argtypes = [c.POINTER(PlanStruct), c.c_int32, c.c_void_p,
                                                c.c_int32, c.c_int64, c.c_int32, c.c_int32,
                                                c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                                c.c_void_p, c.c_int32, c.c_void_p, c.c_void_p,
                                                c.c_void_p]
        L.flare_status_string.restype = c.c_char_p
        L.flare_status_string.argtypes = [c.c_int]
        L.flare_logprobs_abi_version.restype = c.c_uint32
        L.flare_logprobs_abi_version.argtypes = []
        _lib = L
    return _lib


def flare_status_string(status: int) -> str:
    return lib().flare_status_string(int(status)).decode()


def flare_logprobs_abi_version() -> int:
    return int(lib().flare_logprobs_abi_version())


def dtype_code(dtype) -> int:
    if dtype in (torch.bfloat16, "bf16", DTYPE_BF16):
        return DTYPE_BF16
    if dtype in (torch.float32, "fp32", DTYPE_FP32):
        return DTYPE_FP32
    raise ValueError(f"unsupported logits dtype {dtype}")


def flare_logprobs_plan(capacity: int, T: int, V: int, V_pad: int, dtype, K: int,
                        device: int) -> PlanStruct:
    plan = PlanStruct()
    rc = lib().flare_logprobs_plan(ctypes.byref(plan), capacity, T, V, V_pad, dtype_code(dtype),
                                   K, device)
    if rc != 0:
        raise FlareError(rc, "flare_logprobs_plan")
    return plan


def flare_logprobs_plan_sharded(capacity: int, T: int, V: int, V_pad: int, dtype, K: int,
                                shards: int, device: int) -> PlanStruct:
    plan = PlanStruct()
    rc = lib().flare_logprobs_plan_sharded(ctypes.byref(plan), capacity, T, V, V_pad,
                                           dtype_code(dtype), K, shards, device)
    if rc != 0:
        raise FlareError(rc, "flare_logprobs_plan_sharded")
    return plan


def shard_bounds(V: int, shards: int) -> list[int]:
    """Vocabulary lanes of each shard: shard r owns [b[r], b[r + 1]) (the C
    library's rule: floor(r V / shards) rounded up to a multiple of 8)."""
    b = [min(V, -(-(r * V // shards) // 8) * 8) for r in range(shards)]
    return b + [V]


def flare_logprobs_plan_packed(capacity: int, T: int, packed_rows: int, V: int, V_pad: int,
                               dtype, K: int, device: int) -> PlanStruct:
    plan = PlanStruct()
    rc = lib().flare_logprobs_plan_packed(ctypes.byref(plan), capacity, T, packed_rows, V, V_pad,
                                          dtype_code(dtype), K, device)
    if rc != 0:
        raise FlareError(rc, "flare_logprobs_plan_packed")
    return plan


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr() if isinstance(t, torch.Tensor) else int(t)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _call(name: str, plan: PlanStruct, logits, dtype, rows: int, V: int, V_pad: int,
          requested, id_counts, ids, emitted_counts, tokens, K: int, out, workspace,
          stream) -> None:
    rc = getattr(lib(), name)(ctypes.byref(plan), _ptr(logits), dtype_code(dtype), rows, V,
                              V_pad, _ptr(requested), _ptr(id_counts), _ptr(ids),
                              _ptr(emitted_counts), _ptr(tokens), K, _ptr(out),
                              _ptr(workspace), _stream(stream))
    if rc != 0:
        raise FlareError(rc, name)


def flare_logprobs_run(plan: PlanStruct, logits, dtype, rows: int, V: int, V_pad: int,
                       requested, id_counts, ids, emitted_counts, tokens, K: int, out,
                       workspace, stream=None) -> None:
    """Launch one reduction on `stream` (default: torch's current stream).
    Tensor arguments are passed by device pointer; the C library checks the
    scalars against the plan before anything is launched."""
    _call("flare_logprobs_run", plan, logits, dtype, rows, V, V_pad, requested, id_counts, ids,
          emitted_counts, tokens, K, out, workspace, stream)


def _packed_call(name: str, plan: PlanStruct, logits, dtype, rows: int, V: int, V_pad: int,
                 requested, id_counts, ids, emitted_counts, tokens, row_offsets, K: int, out,
                 workspace, stream) -> None:
    rc = getattr(lib(), name)(ctypes.byref(plan), _ptr(logits), dtype_code(dtype), rows, V,
                              V_pad, _ptr(requested), _ptr(id_counts), _ptr(ids),
                              _ptr(emitted_counts), _ptr(tokens), _ptr(row_offsets), K,
                              _ptr(out), _ptr(workspace), _stream(stream))
    if rc != 0:
        raise FlareError(rc, name)


def flare_logprobs_run_packed(plan: PlanStruct, logits, dtype, rows: int, V: int, V_pad: int,
                              requested, id_counts, ids, emitted_counts, tokens, row_offsets,
                              K: int, out, workspace, stream=None) -> None:
    """One frame over packed target rows (rows = P, row_offsets int32 [capacity])."""
    _packed_call("flare_logprobs_run_packed", plan, logits, dtype, rows, V, V_pad, requested,
                 id_counts, ids, emitted_counts, tokens, row_offsets, K, out, workspace, stream)


def flare_logprobs_reduce_packed(plan: PlanStruct, logits, dtype, rows: int, V: int,
                                 V_pad: int, requested, id_counts, ids, emitted_counts, tokens,
                                 row_offsets, K: int, out, workspace, stream=None) -> None:
    """The first launch of flare_logprobs_run_packed (same arguments)."""
    _packed_call("flare_logprobs_reduce_packed", plan, logits, dtype, rows, V, V_pad, requested,
                 id_counts, ids, emitted_counts, tokens, row_offsets, K, out, workspace, stream)


def flare_logprobs_merge_packed(plan: PlanStruct, logits, dtype, rows: int, V: int,
                                V_pad: int, requested, id_counts, ids, emitted_counts, tokens,
                                row_offsets, K: int, out, workspace, stream=None) -> None:
    """The second launch of flare_logprobs_run_packed (same arguments, after reduce)."""
    _packed_call("flare_logprobs_merge_packed", plan, logits, dtype, rows, V, V_pad, requested,
                 id_counts, ids, emitted_counts, tokens, row_offsets, K, out, workspace, stream)


def flare_logprobs_run_records(plan: PlanStruct, logits, dtype, rows: int, V: int, V_pad: int,
                               requested, id_counts, ids, records, emitted_field: int, K: int,
                               out, out_row_words: int, workspace, stream=None) -> None:
    """One frame reading emitted counts and tokens from int64 completion
    records [capacity, 16 + T]; id_counts/ids may both be None (natural only,
    rows of 2 + 2K words)."""
    rc = lib().flare_logprobs_run_records(ctypes.byref(plan), _ptr(logits), dtype_code(dtype),
                                          rows, V, V_pad, _ptr(requested), _ptr(id_counts),
                                          _ptr(ids), _ptr(records), emitted_field, K, _ptr(out),
                                          out_row_words, _ptr(workspace), _stream(stream))
    if rc != 0:
        raise FlareError(rc, "flare_logprobs_run_records")


def flare_logprobs_run_noalloc(plan: PlanStruct, logits, dtype, rows: int, V: int, V_pad: int,
                               requested, id_counts, ids, emitted_counts, tokens, K: int, out,
                               stream=None) -> None:
    """flare_logprobs_run on the library's static 16 MiB scratch (no workspace,
    no allocation); calls that overlap on one GPU race."""
    rc = lib().flare_logprobs_run_noalloc(ctypes.byref(plan), _ptr(logits), dtype_code(dtype),
                                          rows, V, V_pad, _ptr(requested), _ptr(id_counts),
                                          _ptr(ids), _ptr(emitted_counts), _ptr(tokens), K,
                                          _ptr(out), _stream(stream))
    if rc != 0:
        raise FlareError(rc, "flare_logprobs_run_noalloc")


def flare_logprobs_run_sharded(plan: PlanStruct, logits, dtype, rows: int, V: int, V_pad: int,
                               requested, id_counts, ids, emitted_counts, tokens, K: int, out,
                               workspace, stream=None) -> None:
    """Every shard pass of a sharded plan, then the cross-shard merge."""
    _call("flare_logprobs_run_sharded", plan, logits, dtype, rows, V, V_pad, requested,
          id_counts, ids, emitted_counts, tokens, K, out, workspace, stream)


def flare_logprobs_shard_merge(plan: PlanStruct, logits, dtype, rows: int, V: int, V_pad: int,
                               requested, id_counts, ids, emitted_counts, tokens, K: int, out,
                               workspace, stream=None) -> None:
    """The cross-shard merge over the gathered shard records."""
    _call("flare_logprobs_shard_merge", plan, logits, dtype, rows, V, V_pad, requested,
          id_counts, ids, emitted_counts, tokens, K, out, workspace, stream)


def flare_logprobs_shard_pass(plan: PlanStruct, shard: int, logits, dtype, rows: int, V: int,
                              V_pad: int, requested, id_counts, ids, emitted_counts, tokens,
                              K: int, out, workspace, stream=None) -> None:
    """Shard `shard`'s pass: the reduction of its columns and its exchange records."""
    rc = lib().flare_logprobs_shard_pass(ctypes.byref(plan), shard, _ptr(logits),
                                         dtype_code(dtype), rows, V, V_pad, _ptr(requested),
                                         _ptr(id_counts), _ptr(ids), _ptr(emitted_counts),
                                         _ptr(tokens), K, _ptr(out), _ptr(workspace),
                                         _stream(stream))
    if rc != 0:
        raise FlareError(rc, "flare_logprobs_shard_pass")


def flare_logprobs_reduce(plan: PlanStruct, logits, dtype, rows: int, V: int, V_pad: int,
                          requested, id_counts, ids, emitted_counts, tokens, K: int, out,
                          workspace, stream=None) -> None:
    """The first launch of flare_logprobs_run (same arguments)."""
    _call("flare_logprobs_reduce", plan, logits, dtype, rows, V, V_pad, requested, id_counts,
          ids, emitted_counts, tokens, K, out, workspace, stream)


def flare_logprobs_merge(plan: PlanStruct, logits, dtype, rows: int, V: int, V_pad: int,
                         requested, id_counts, ids, emitted_counts, tokens, K: int, out,
                         workspace, stream=None) -> None:
    """The second launch of flare_logprobs_run (same arguments, after reduce)."""
    _call("flare_logprobs_merge", plan, logits, dtype, rows, V, V_pad, requested, id_counts,
          ids, emitted_counts, tokens, K, out, workspace, stream)


def _check(t: torch.Tensor, name: str, dtype, numel: int, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype or not t.is_contiguous() or t.numel() != numel or t.device != device:
        raise ValueError(f"{name}: expected contiguous {dtype} with {numel} elements on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


class Plan:
    """A validated geometry plus the shapes its tensors must have."""

    def __init__(self, capacity: int, T: int, V: int, V_pad: int | None = None,
                 dtype=torch.bfloat16, K: int = 20, device: int | None = None,
                 packed_rows: int | None = None, shards: int | None = None):
        """`packed_rows` = P selects packed target rows (logits [P, V_pad], slot s's
        row t at row_offsets[s] + t); None keeps the rectangular [capacity*T, V_pad].
        `shards` = N splits the vocabulary into N shards (a shard pass per shard,
        then the cross-shard merge)."""
        if device is None:
            device = torch.cuda.current_device()
        self.torch_dtype = torch.bfloat16 if dtype_code(dtype) == DTYPE_BF16 else torch.float32
        self.V_pad = V if V_pad is None else V_pad
        if packed_rows is not None and shards is not None:
            raise ValueError("a plan is either packed or sharded")
        if shards is not None:
            self.raw = flare_logprobs_plan_sharded(capacity, T, V, self.V_pad, dtype, K, shards,
                                                   device)
        elif packed_rows is None:
            self.raw = flare_logprobs_plan(capacity, T, V, self.V_pad, dtype, K, device)
        else:
            self.raw = flare_logprobs_plan_packed(capacity, T, packed_rows, V, self.V_pad, dtype,
                                                  K, device)
        self.packed_rows = packed_rows
        self.shards = shards
        self.capacity, self.T, self.V, self.K, self.device_index = capacity, T, V, K, device

    @property
    def device(self) -> torch.device:
        return torch.device("cuda", self.device_index)

    @property
    def workspace_bytes(self) -> int:
        return int(self.raw.workspace_bytes)

    def workspace(self) -> torch.Tensor:
        return torch.empty(self.workspace_bytes, dtype=torch.uint8, device=self.device)

    def lse(self, workspace: torch.Tensor) -> torch.Tensor:
        """Diagnostic view: the normalization L of every reduced row."""
        n = self.capacity * self.T
        off = int(self.raw.lse_offset)
        return workspace[off:off + 4 * n].view(torch.float32)

    def exchange(self, workspace: torch.Tensor) -> torch.Tensor:
        """Sharded plans: the gathered shard records, as int32 [capacity*T, shards, 138]."""
        n = self.capacity * self.T
        off = int(self.raw.exchange_offset)
        return workspace[off:off + n * self.shards * 552].view(torch.int32).view(n, self.shards, 138)

    def guard(self, workspace: torch.Tensor) -> torch.Tensor:
        """Diagnostic view: per reduced row, the parts (shards, for a sharded plan)
        that the merge's guard streamed again."""
        n = self.capacity * self.T
        off = int(self.raw.guard_offset)
        return workspace[off:off + 4 * n].view(torch.int32)

    def new_out(self, fill: int = 0) -> torch.Tensor:
        return torch.full((self.capacity, self.T, ROW_WORDS), fill, dtype=torch.int32,
                          device=self.device)

    def bind(self, logits, tokens, emitted_counts, requested, id_counts, ids, out, workspace,
             phase: str = "all", row_offsets=None) -> "BoundCall":
        """Validate one call's tensors once and marshal its C arguments: the
        returned BoundCall launches with a single C call each time (for
        serving loops and timing, where per-call Python checks would hold up
        the GPU).  It keeps the tensors alive."""
        dev = self.device
        rows = self.capacity * self.T
        packed = self.packed_rows is not None
        if packed and row_offsets is None:
            raise ValueError("a packed plan needs row_offsets")
        if not packed and row_offsets is not None:
            raise ValueError("row_offsets needs a packed plan")
        _check(logits, "logits", self.torch_dtype,
               (self.packed_rows if packed else rows) * self.V_pad, dev)
        if packed:
            _check(row_offsets, "row_offsets", torch.int32, self.capacity, dev)
        _check(tokens, "tokens", torch.int32, rows, dev)
        _check(emitted_counts, "emitted_counts", torch.int32, self.capacity, dev)
        _check(requested, "requested", torch.int32, self.capacity, dev)
        _check(id_counts, "id_counts", torch.int32, self.capacity, dev)
        _check(ids, "ids", torch.int32, self.capacity * MAX_IDS, dev)
        _check(out, "out", torch.int32, rows * ROW_WORDS, dev)
        _check(workspace, "workspace", torch.uint8, self.workspace_bytes, dev)
        head = (ctypes.byref(self.raw), _ptr(logits), DTYPE_BF16 if self.torch_dtype ==
                torch.bfloat16 else DTYPE_FP32, self.packed_rows if packed else rows, self.V,
                self.V_pad, _ptr(requested), _ptr(id_counts), _ptr(ids), _ptr(emitted_counts),
                _ptr(tokens))
        keep = (self, logits, tokens, emitted_counts, requested, id_counts, ids, out, workspace,
                row_offsets)
        if self.shards is not None:
            # "all": every shard pass, then the merge; "shard:r": rank r's pass;
            # "merge": the cross-shard merge of the gathered records.
            tail = (self.K, _ptr(out), _ptr(workspace))
            if phase == "all":
                return BoundCall("flare_logprobs_run_sharded", head + tail, keep)
            if phase == "merge":
                return BoundCall("flare_logprobs_shard_merge", head + tail, keep)
            if phase.startswith("shard:"):
                r = int(phase.split(":", 1)[1])
                return BoundCall("flare_logprobs_shard_pass", (head[0], r) + head[1:] + tail, keep)
            raise ValueError(f"sharded plans take phase 'all', 'shard:r' or 'merge', not {phase!r}")
        name = {"all": "flare_logprobs_run", "reduce": "flare_logprobs_reduce",
                "merge": "flare_logprobs_merge"}[phase] + ("_packed" if packed else "")
        args = head + ((_ptr(row_offsets),) if packed else ()) + (self.K, _ptr(out),
                                                                  _ptr(workspace))
        return BoundCall(name, args, keep)

    def bind_records(self, logits, records, requested, out, workspace, emitted_field: int,
                     id_counts=None, ids=None) -> "BoundCall":
        """A prepared frame whose emitted counts and tokens come from
        the int64 completion records [capacity, 16 + T] (emitted count at
        `emitted_field`).  Without ID inputs (both None) `out` holds 2 + 2K words
        per position, else 258."""
        if self.packed_rows is not None:
            raise ValueError("completion records take a rectangular plan")
        dev = self.device
        rows = self.capacity * self.T
        words = ROW_WORDS if id_counts is not None else 2 + 2 * self.K
        _check(logits, "logits", self.torch_dtype, rows * self.V_pad, dev)
        _check(records, "records", torch.int64, self.capacity * (16 + self.T), dev)
        _check(requested, "requested", torch.int32, self.capacity, dev)
        if id_counts is not None or ids is not None:
            _check(id_counts, "id_counts", torch.int32, self.capacity, dev)
            _check(ids, "ids", torch.int32, self.capacity * MAX_IDS, dev)
        _check(out, "out", torch.int32, rows * words, dev)
        _check(workspace, "workspace", torch.uint8, self.workspace_bytes, dev)
        args = (ctypes.byref(self.raw), _ptr(logits), dtype_code(self.torch_dtype), rows, self.V,
                self.V_pad, _ptr(requested), _ptr(id_counts), _ptr(ids), _ptr(records),
                emitted_field, self.K, _ptr(out), words, _ptr(workspace))
        return BoundCall("flare_logprobs_run_records", args,
                         (self, logits, records, requested, out, workspace, id_counts, ids))


    def run_records(self, logits, records, requested, out, workspace, emitted_field: int,
                    id_counts=None, ids=None, stream=None) -> torch.Tensor:
        """bind_records, then launch on `stream`."""
        self.bind_records(logits, records, requested, out, workspace, emitted_field, id_counts,
                          ids)(stream)
        return out

    def run(self, logits, tokens, emitted_counts, requested, id_counts, ids, out, workspace,
            stream=None, phase: str = "all", row_offsets=None) -> torch.Tensor:
        """One call: both launches (phase "all"), or only the first ("reduce")
        or the second ("merge") of them.  A packed plan takes `row_offsets`
        (int32 [capacity]) and the same phases."""
        self.bind(logits, tokens, emitted_counts, requested, id_counts, ids, out, workspace,
                  phase=phase, row_offsets=row_offsets)(stream)
        return out




class BoundCall:
    """One validated call of a C entry point with its arguments marshalled;
    calling it launches on `stream` (default: torch's current stream)."""

    def __init__(self, name: str, args: tuple, keep: tuple):
        self.name = name
        self._fn = getattr(lib(), name)
        self._args = args
        self._keep = keep  # the tensors whose pointers `args` holds

    def __call__(self, stream=None) -> None:
        rc = self._fn(*self._args, _stream(stream))
        if rc != 0:
            raise FlareError(rc, self.name)


# ------------------------------------------------------------ prompt scoring
def flare_prompt_logprobs_plan(rows: int, V: int, V_pad: int, dtype, device: int) -> PlanStruct:
    plan = PlanStruct()
    rc = lib().flare_prompt_logprobs_plan(ctypes.byref(plan), rows, V, V_pad, dtype_code(dtype),
                                          device)
    if rc != 0:
        raise FlareError(rc, "flare_prompt_logprobs_plan")
    return plan


def _prompt_call(name: str, plan: PlanStruct, logits, dtype, rows: int, V: int, V_pad: int,
                 targets, out, workspace, stream) -> None:
    rc = getattr(lib(), name)(ctypes.byref(plan), _ptr(logits), dtype_code(dtype), rows, V,
                              V_pad, _ptr(targets), _ptr(out), _ptr(workspace), _stream(stream))
    if rc != 0:
        raise FlareError(rc, name)


def flare_prompt_logprobs_run(plan: PlanStruct, logits, dtype, rows: int, V: int, V_pad: int,
                              targets, out, workspace, stream=None) -> None:
    """Score one prompt chunk on `stream` (default: torch's current stream)."""
    _prompt_call("flare_prompt_logprobs_run", plan, logits, dtype, rows, V, V_pad, targets, out,
                 workspace, stream)


def flare_prompt_logprobs_reduce(plan: PlanStruct, logits, dtype, rows: int, V: int, V_pad: int,
                                 targets, out, workspace, stream=None) -> None:
    """The first launch of flare_prompt_logprobs_run (same arguments)."""
    _prompt_call("flare_prompt_logprobs_reduce", plan, logits, dtype, rows, V, V_pad, targets,
                 out, workspace, stream)


def flare_prompt_logprobs_merge(plan: PlanStruct, logits, dtype, rows: int, V: int, V_pad: int,
                                targets, out, workspace, stream=None) -> None:
    """The second launch of flare_prompt_logprobs_run (same arguments, after reduce)."""
    _prompt_call("flare_prompt_logprobs_merge", plan, logits, dtype, rows, V, V_pad, targets,
                 out, workspace, stream)


class PromptPlan:
    """A validated prompt-scoring geometry plus the shapes its tensors must have."""

    def __init__(self, rows: int, V: int, V_pad: int | None = None, dtype=torch.bfloat16,
                 device: int | None = None):
        if device is None:
            device = torch.cuda.current_device()
        self.torch_dtype = torch.bfloat16 if dtype_code(dtype) == DTYPE_BF16 else torch.float32
        self.V_pad = V if V_pad is None else V_pad
        self.raw = flare_prompt_logprobs_plan(rows, V, self.V_pad, dtype, device)
        self.rows, self.V, self.device_index = rows, V, device

    @property
    def device(self) -> torch.device:
        return torch.device("cuda", self.device_index)

    @property
    def workspace_bytes(self) -> int:
        return int(self.raw.workspace_bytes)

    def workspace(self) -> torch.Tensor:
        return torch.empty(self.workspace_bytes, dtype=torch.uint8, device=self.device)

    def lse(self, workspace: torch.Tensor) -> torch.Tensor:
        """Diagnostic view: the normalization L of every scored row (valid rows only)."""
        off = int(self.raw.lse_offset)
        return workspace[off:off + 4 * self.rows].view(torch.float32)

    def guard(self, workspace: torch.Tensor) -> torch.Tensor:
        """Diagnostic view: per valid row, the parts whose lanes were counted again."""
        off = int(self.raw.guard_offset)
        return workspace[off:off + 4 * self.rows].view(torch.int32)

    def new_out(self, fill: int = 0) -> torch.Tensor:
        return torch.full((self.rows, PROMPT_ROW_WORDS), fill, dtype=torch.int32,
                          device=self.device)

    def bind(self, logits, targets, out, workspace, phase: str = "all") -> BoundCall:
        """Validate once and marshal the C arguments (see Plan.bind)."""
        dev = self.device
        _check(logits, "logits", self.torch_dtype, self.rows * self.V_pad, dev)
        _check(targets, "targets", torch.int32, self.rows, dev)
        _check(out, "out", torch.int32, self.rows * PROMPT_ROW_WORDS, dev)
        _check(workspace, "workspace", torch.uint8, self.workspace_bytes, dev)
        name = {"all": "flare_prompt_logprobs_run", "reduce": "flare_prompt_logprobs_reduce",
                "merge": "flare_prompt_logprobs_merge"}[phase]
        args = (ctypes.byref(self.raw), _ptr(logits), dtype_code(self.torch_dtype), self.rows,
                self.V, self.V_pad, _ptr(targets), _ptr(out), _ptr(workspace))
        return BoundCall(name, args, (self, logits, targets, out, workspace))

    def run(self, logits, targets, out, workspace, stream=None,
            phase: str = "all") -> torch.Tensor:
        """Both launches (phase "all"), or only "reduce" or "merge"."""
        self.bind(logits, targets, out, workspace, phase=phase)(stream)
        return out
