"""The C ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments with status codes before launching anything.  No call
here reaches a kernel launch."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def flp():
    import full_vocab_logprob_amd as m
    if not os.path.exists(m.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return m


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(flare_\w+)\s*\(", text,
                            flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert {"flare_logprobs_plan", "flare_logprobs_run", "flare_logprobs_reduce",
            "flare_logprobs_merge", "flare_status_string",
            "flare_logprobs_abi_version", "flare_prompt_logprobs_plan",
            "flare_prompt_logprobs_run", "flare_prompt_logprobs_reduce",
            "flare_prompt_logprobs_merge", "flare_logprobs_plan_packed",
            "flare_logprobs_run_packed", "flare_logprobs_run_records",
            "flare_logprobs_plan_sharded", "flare_logprobs_run_sharded",
            "flare_logprobs_shard_pass", "flare_logprobs_shard_merge"} <= set(names)


def test_library_exports_every_declared_symbol(flp):
    lib = ctypes.CDLL(flp.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(flp):
    assert flp.flare_logprobs_abi_version() == flp.ABI_VERSION
    for code in range(8):
        assert flp.flare_status_string(code) != "unknown status"
    assert flp.flare_status_string(99) == "unknown status"


def test_plan_struct_layout_matches_header(flp):
    # 16 int32-sized fields, 5 uint64, packed_rows, shards, exchange_offset, 2 reserved uint32
    assert ctypes.sizeof(flp.PlanStruct) == 16 * 4 + 5 * 8 + 2 * 4 + 8 + 2 * 4


def host_plan(flp, capacity=128, T=8, V=248320, V_pad=248320, dtype=1, K=20):
    plan = flp.PlanStruct()
    rc = flp.lib().flare_logprobs_plan(ctypes.byref(plan), capacity, T, V, V_pad, dtype, K, -1)
    return rc, plan


def test_plan_host_only_geometry(flp):
    rc, p = host_plan(flp)
    assert rc == 0
    assert p.units == 16 and p.unit_elems == 16384 and p.block == 256 and p.vector_rows == 1
    assert p.cu_count == 256 and p.abi_version == flp.ABI_VERSION and p.grid == 1024
    assert p.ranges == 1024 and p.mode == flp.MODE_GENERATION
    rows = 128 * 8
    assert p.lse_offset >= rows * 16 * 280 and p.slots_offset >= p.lse_offset + 4 * rows
    assert p.slots_offset % 16 == 0 and p.guard_offset >= p.slots_offset + 4 * (128 + 1)
    assert p.guard_offset % 16 == 0 and p.workspace_bytes >= p.guard_offset + 4 * rows
    rc, p = host_plan(flp, capacity=1024, T=4, V=262144, V_pad=262144, dtype=0)
    assert rc == 0 and p.units == 32 and p.unit_elems == 8192
    rc, p = host_plan(flp, V=37, V_pad=41)
    assert rc == 0 and p.vector_rows == 0


@pytest.mark.parametrize("kw,status", [
    (dict(capacity=0), 1), (dict(T=0), 1), (dict(V=0), 1), (dict(V_pad=100, V=200), 1),
    (dict(K=-1), 1), (dict(K=21), 1), (dict(dtype=2), 2), (dict(dtype=-1), 2),
    (dict(V=16384 * 64 + 1, V_pad=16384 * 64 + 1), 6), (dict(capacity=8193, T=1), 1),
])
def test_plan_rejects(flp, kw, status):
    rc, p = host_plan(flp, **kw)
    assert rc == status
    assert p.abi_version == 0  # left zeroed


def test_plan_null_pointer(flp):
    assert flp.lib().flare_logprobs_plan(None, 1, 1, 1, 1, 0, 0, -1) == 1


FAKE = 0x10000  # never dereferenced: every case below fails validation first


ENTRY = "flare_logprobs_run"


@pytest.fixture(params=["flare_logprobs_run", "flare_logprobs_reduce", "flare_logprobs_merge"],
                autouse=False)
def entry(request):
    """Every call taking run's arguments validates them the same way."""
    global ENTRY
    ENTRY = request.param
    yield request.param
    ENTRY = "flare_logprobs_run"


def run_status(flp, plan, **over):
    args = dict(logits=FAKE, dtype=plan.dtype, rows=plan.capacity * plan.T, V=plan.V,
                V_pad=plan.V_pad, requested=FAKE, id_counts=FAKE, ids=FAKE, emitted=FAKE,
                tokens=FAKE, K=plan.K, out=FAKE, workspace=FAKE, stream=None)
    args.update(over)
    return getattr(flp.lib(), ENTRY)(
        ctypes.byref(plan), args["logits"], args["dtype"], args["rows"], args["V"],
        args["V_pad"], args["requested"], args["id_counts"], args["ids"], args["emitted"],
        args["tokens"], args["K"], args["out"], args["workspace"], args["stream"])


@pytest.mark.parametrize("field", ["logits", "requested", "id_counts", "ids", "emitted",
                                   "tokens", "out", "workspace"])
def test_run_rejects_null_pointers(flp, entry, field):
    rc, plan = host_plan(flp)
    assert rc == 0
    assert run_status(flp, plan, **{field: None}) == 1


@pytest.mark.parametrize("over", [dict(dtype=0), dict(V=1000), dict(V_pad=248321), dict(K=5),
                                  dict(rows=1023)])
def test_run_rejects_plan_mismatch(flp, entry, over):
    rc, plan = host_plan(flp)
    assert run_status(flp, plan, **over) == 3


def test_run_rejects_bad_dtype_and_stale_plan(flp):
    rc, plan = host_plan(flp)
    assert run_status(flp, plan, dtype=7) == 2
    plan.abi_version = 99
    assert run_status(flp, plan) == 3
    assert flp.lib().flare_logprobs_run(None, FAKE, 1, 1, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        0, FAKE, FAKE, None) == 1


def test_run_rejects_corrupt_plan(flp, entry):
    rc, plan = host_plan(flp)
    plan.ranges = 3
    assert run_status(flp, plan) == 3
    rc, plan = host_plan(flp)
    plan.grid = 0
    assert run_status(flp, plan) == 3
    rc, plan = host_plan(flp)
    plan.block = 1024
    assert run_status(flp, plan) == 3


def test_run_rejects_misaligned_workspace(flp, entry):
    rc, plan = host_plan(flp)
    assert run_status(flp, plan, workspace=FAKE + 4) == 1


# ------------------------------------------------------------ prompt scoring
def prompt_plan(flp, rows=128, V=248320, V_pad=248320, dtype=1):
    plan = flp.PlanStruct()
    rc = flp.lib().flare_prompt_logprobs_plan(ctypes.byref(plan), rows, V, V_pad, dtype, -1)
    return rc, plan


def prompt_status(flp, plan, entry="flare_prompt_logprobs_run", **over):
    args = dict(logits=FAKE, dtype=plan.dtype, rows=plan.capacity, V=plan.V, V_pad=plan.V_pad,
                targets=FAKE, out=FAKE, workspace=FAKE, stream=None)
    args.update(over)
    return getattr(flp.lib(), entry)(ctypes.byref(plan), args["logits"], args["dtype"],
                                     args["rows"], args["V"], args["V_pad"], args["targets"],
                                     args["out"], args["workspace"], args["stream"])


def test_prompt_plan_geometry(flp):
    rc, p = prompt_plan(flp)
    assert rc == 0 and p.mode == flp.MODE_PROMPT and p.T == 1 and p.K == 20
    assert p.capacity == 128 and p.units == 16 and p.grid == 1024
    assert p.lse_offset >= 128 * 16 * 280 and p.slots_offset >= p.lse_offset + 4 * 128
    assert p.workspace_bytes >= p.slots_offset + 4 * 129
    rc, p = prompt_plan(flp, rows=8192, V=151936, V_pad=152064, dtype=0)
    assert rc == 0 and p.units == 19 and p.vector_rows == 1


@pytest.mark.parametrize("kw,status", [
    (dict(rows=0), 1), (dict(rows=8193), 1), (dict(V=0), 1), (dict(V_pad=5, V=6), 1),
    (dict(dtype=3), 2), (dict(V=16384 * 64 + 1, V_pad=16384 * 64 + 1), 6),
])
def test_prompt_plan_rejects(flp, kw, status):
    rc, p = prompt_plan(flp, **kw)
    assert rc == status and p.abi_version == 0
    assert flp.lib().flare_prompt_logprobs_plan(None, 1, 1, 1, 0, -1) == 1


@pytest.mark.parametrize("pentry", ["flare_prompt_logprobs_run", "flare_prompt_logprobs_reduce",
                                    "flare_prompt_logprobs_merge"])
def test_prompt_run_rejects(flp, pentry):
    rc, plan = prompt_plan(flp)
    assert rc == 0
    for field in ("logits", "targets", "out", "workspace"):
        assert prompt_status(flp, plan, pentry, **{field: None}) == 1
    for over in (dict(dtype=0), dict(V=1000), dict(V_pad=248328), dict(rows=127)):
        assert prompt_status(flp, plan, pentry, **over) == 3
    assert prompt_status(flp, plan, pentry, dtype=9) == 2
    assert prompt_status(flp, plan, pentry, workspace=FAKE + 8) == 1
    bad = flp.PlanStruct.from_buffer_copy(plan)
    bad.T = 2
    assert prompt_status(flp, bad, pentry) == 3
    bad = flp.PlanStruct.from_buffer_copy(plan)
    bad.abi_version = 2
    assert prompt_status(flp, bad, pentry) == 3


def test_plans_are_not_interchangeable(flp):
    """A generation plan is rejected by the prompt entry points and a prompt
    plan by the generation ones."""
    rc, gplan = host_plan(flp, capacity=128, T=1, K=20)
    assert rc == 0
    assert prompt_status(flp, gplan) == 3
    rc, pplan = prompt_plan(flp)
    assert rc == 0
    assert run_status(flp, pplan) == 3


# ------------------------------------------------------------ packed target rows
def packed_plan(flp, capacity=128, T=8, P=600, V=248320, V_pad=248320, dtype=1, K=20):
    plan = flp.PlanStruct()
    rc = flp.lib().flare_logprobs_plan_packed(ctypes.byref(plan), capacity, T, P, V, V_pad, dtype,
                                              K, -1)
    return rc, plan


def packed_status(flp, plan, **over):
    args = dict(logits=FAKE, dtype=plan.dtype, rows=plan.packed_rows, V=plan.V, V_pad=plan.V_pad,
                requested=FAKE, id_counts=FAKE, ids=FAKE, emitted=FAKE, tokens=FAKE,
                offsets=FAKE, K=plan.K, out=FAKE, workspace=FAKE, stream=None)
    args.update(over)
    return flp.lib().flare_logprobs_run_packed(
        ctypes.byref(plan), args["logits"], args["dtype"], args["rows"], args["V"], args["V_pad"],
        args["requested"], args["id_counts"], args["ids"], args["emitted"], args["tokens"],
        args["offsets"], args["K"], args["out"], args["workspace"], args["stream"])


def test_packed_plan(flp):
    rc, p = packed_plan(flp)
    assert rc == 0 and p.packed_rows == 600 and p.mode == flp.MODE_GENERATION
    rc0, p0 = host_plan(flp)
    assert p.workspace_bytes == p0.workspace_bytes and p0.packed_rows == 0
    for P in (0, -3, (1 << 30) + 1):
        rc, p = packed_plan(flp, P=P)
        assert rc == 1 and p.abi_version == 0


def test_packed_run_rejects(flp):
    rc, plan = packed_plan(flp)
    assert rc == 0
    for field in ("logits", "requested", "id_counts", "ids", "emitted", "tokens", "offsets",
                  "out", "workspace"):
        assert packed_status(flp, plan, **{field: None}) == 1, field
    for over in (dict(rows=1024), dict(rows=599), dict(V=1000), dict(K=3), dict(dtype=0)):
        assert packed_status(flp, plan, **over) == 3, over
    # plans of the other layout
    rc, rect = host_plan(flp)
    assert packed_status(flp, rect, rows=1024) == 3
    assert run_status(flp, plan, rows=600) == 3
    assert run_status(flp, plan, rows=1024) == 3


# ------------------------------------------------------------ completion records
def records_status(flp, plan, **over):
    args = dict(logits=FAKE, dtype=plan.dtype, rows=plan.capacity * plan.T, V=plan.V,
                V_pad=plan.V_pad, requested=FAKE, id_counts=FAKE, ids=FAKE, records=FAKE,
                field=3, K=plan.K, out=FAKE, words=258, workspace=FAKE, stream=None)
    args.update(over)
    return flp.lib().flare_logprobs_run_records(
        ctypes.byref(plan), args["logits"], args["dtype"], args["rows"], args["V"], args["V_pad"],
        args["requested"], args["id_counts"], args["ids"], args["records"], args["field"],
        args["K"], args["out"], args["words"], args["workspace"], args["stream"])


def test_records_run_rejects(flp):
    rc, plan = host_plan(flp)
    assert rc == 0
    for field in ("logits", "requested", "records", "out", "workspace"):
        assert records_status(flp, plan, **{field: None}) == 1, field
    assert records_status(flp, plan, id_counts=None) == 1  # one ID input without the other
    assert records_status(flp, plan, ids=None) == 1
    assert records_status(flp, plan, field=-1) == 1 and records_status(flp, plan, field=16) == 1
    assert records_status(flp, plan, words=42) == 1            # 2 + 2K needs no ID inputs
    assert records_status(flp, plan, id_counts=None, ids=None, words=41) == 1
    assert records_status(flp, plan, K=5) == 3                 # K differs from the plan
    rc, p0 = host_plan(flp, K=0)
    assert records_status(flp, p0, id_counts=None, ids=None, words=2) == 1  # K = 0
    rc, pk = packed_plan(flp)
    assert records_status(flp, pk, rows=600) == 3


def test_binding_names_mirror_the_abi(flp):
    for name in declared_functions():
        assert callable(getattr(flp, name)), name


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "full_vocab_logprob_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("oracle_handle", ""), f


# ------------------------------------------------------ vocabulary shards
def sharded_plan(flp, shards=8, capacity=128, T=8, V=248320, V_pad=248320, dtype=1, K=20):
    plan = flp.PlanStruct()
    rc = flp.lib().flare_logprobs_plan_sharded(ctypes.byref(plan), capacity, T, V, V_pad, dtype,
                                               K, shards, -1)
    return rc, plan


def test_sharded_plan_geometry(flp):
    rc, p = sharded_plan(flp)
    assert rc == 0 and p.shards == 8 and p.mode == flp.MODE_GENERATION
    b = flp.shard_bounds(248320, 8)
    assert b == [31040 * r for r in range(9)]
    assert p.units == 2  # each 31,040-lane shard needs two 16,384-lane units
    rows = 128 * 8
    assert p.exchange_offset >= p.guard_offset + 4 * rows and p.exchange_offset % 16 == 0
    assert p.workspace_bytes >= p.exchange_offset + rows * 8 * 552
    # boundaries: multiples of 8, nondecreasing, covering [0, V)
    for V, n in ((1000, 7), (50001, 32), (64, 8), (248320, 3)):
        b = flp.shard_bounds(V, n)
        assert b[0] == 0 and b[-1] == V and all(x % 8 == 0 for x in b[:-1])
        assert all(b[i] < b[i + 1] for i in range(n))
    # the unsharded plan of the same geometry has no shards
    rc, q = host_plan(flp)
    assert q.shards == 0 and q.exchange_offset == 0


@pytest.mark.parametrize("kw", [dict(shards=0), dict(shards=33), dict(V=40, V_pad=40, shards=8),
                                dict(V=50, V_pad=56, shards=8), dict(K=21)])
def test_sharded_plan_rejects(flp, kw):
    rc, p = sharded_plan(flp, **kw)
    assert rc == 1 and p.abi_version == 0


def test_sharded_and_unsharded_entry_points_reject_each_other(flp):
    rc, sp = sharded_plan(flp)
    rc2, up = host_plan(flp)
    assert rc == 0 and rc2 == 0
    L = flp.lib()
    args = (FAKE, 1, 128 * 8, 248320, 248320, FAKE, FAKE, FAKE, FAKE, FAKE, 20, FAKE, FAKE, None)
    assert L.flare_logprobs_run(ctypes.byref(sp), *args) == 3
    assert L.flare_logprobs_reduce(ctypes.byref(sp), *args) == 3
    assert L.flare_logprobs_run_sharded(ctypes.byref(up), *args) == 3
    assert L.flare_logprobs_shard_merge(ctypes.byref(up), *args) == 3
    assert L.flare_logprobs_shard_pass(ctypes.byref(up), 0, *args) == 1  # no shard 0
    assert L.flare_logprobs_shard_pass(ctypes.byref(sp), 8, *args) == 1
    assert L.flare_logprobs_shard_pass(ctypes.byref(sp), -1, *args) == 1
    assert L.flare_logprobs_run_sharded(ctypes.byref(sp), FAKE, 1, 128 * 8, 248320, 248320, FAKE,
                                        FAKE, FAKE, FAKE, FAKE, 5, FAKE, FAKE, None) == 3
