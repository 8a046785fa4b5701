"""Worked examples under tests/golden/: hand-checkable claims and oracle
regression (CPU only)."""
import glob
import json
import math
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
FILES = sorted(glob.glob(os.path.join(HERE, "golden", "*.json")))
NAN = 0x7FC00000


def load(name):
    with open(os.path.join(HERE, "golden", name + ".json")) as f:
        return json.load(f)


def fixture_row(fx):
    if fx["dtype"] == "bf16":
        return np.asarray(fx["row_bits"], dtype=np.uint16)
    return np.asarray(fx["row_bits"], dtype=np.uint32).view(np.float32)


def u32(w):
    return w & 0xFFFFFFFF


def test_fixture_set_present():
    names = {os.path.basename(f)[:-5] for f in FILES}
    assert {"uniform_v4_fp32", "subtraction_tie_v64_fp32", "signed_zero_v32_bf16",
            "v_below_k_v5_fp32", "selected_ids_v10_fp32", "grid_ties_v48_bf16"} <= names
    for f in FILES:
        fx = json.load(open(f))
        assert fx["cite"] and fx["note"]


@pytest.mark.parametrize("path", FILES, ids=lambda p: os.path.basename(p))
def test_oracle_reproduces_fixture(oracle_handle, path):
    fx = json.load(open(path))
    words, L = oracle_handle.row(fixture_row(fx), token=fx["token"], K=fx["K"],
                                 sel=fx["sel"] or None)
    assert [int(w) for w in words] == fx["words"]
    assert int(np.array([L], np.float32).view(np.uint32)[0]) == fx["L_bits"]


def test_hand_claims():
    fx = load("uniform_v4_fp32")
    assert fx["L_bits"] == 0x3FB17218 and np.float32(math.log(4)).view(np.uint32) == 0x3FB17218
    assert fx["words"][2::2][:4] == [0, 1, 2, 3] and fx["words"][2::2][4:] == [-1] * 16
    assert all(u32(b) == 0xBFB17218 for b in fx["words"][3:11:2])
    assert all(u32(b) == NAN for b in fx["words"][11::2])
    fx = load("subtraction_tie_v64_fp32")
    assert fx["words"][2::2][:5] == [2, 0, 1, 3, 4]
    assert u32(fx["words"][5]) == u32(fx["words"][7]) == 0xC2C60000  # -99.0
    fx = load("signed_zero_v32_bf16")
    assert fx["row_bits"][9] == 0x8000 and fx["words"][:4] == [9, 0, 9, 0]
    fx = load("v_below_k_v5_fp32")
    assert fx["words"][2::2][:5] == [1, 2, 0, 4, 3] and fx["words"][2::2][5:] == [-1] * 15
    fx = load("selected_ids_v10_fp32")
    assert fx["words"][2::2] == [9, -1, 10, 3, 3]
    assert [u32(b) == NAN for b in fx["words"][1::2]] == [True, False, True, True, False, False]
    assert fx["words"][9] == fx["words"][11]
    fx = load("grid_ties_v48_bf16")
    assert fx["words"][2::2] == [5, 17, 40, 0, 2, 3]
    a, b = load("last_bit_of_L_a_v64_fp32"), load("last_bit_of_L_b_v64_fp32")
    assert a["L_bits"] == 0x42C80000 and b["L_bits"] == 0x42C80001  # 100 and the next float
    assert a["words"][2::2][:3] == [2, 1, 0] and b["words"][2::2][:3] == [2, 0, 1]
    # -99 is 0xC2C60000; each step of 2^-17 near 99 is one unit in the last place
    assert [u32(x) for x in a["words"][3:9:2]] == [0, 0xC2C60000, 0xC2C60001]
    assert [u32(x) for x in b["words"][3:9:2]] == [0, 0xC2C60002, 0xC2C60002]


def test_listing_depends_on_the_last_bit_of_L(oracle_handle):
    """The two rows differ only in the dominant logit, so the listing of row
    a at row b's L is row b's listing of lanes 0 and 1: which of two logits
    one ulp apart ranks first depends on the last bit of L.  A GPU whose L is
    off by one unit would list them the other way."""
    a, b = load("last_bit_of_L_a_v64_fp32"), load("last_bit_of_L_b_v64_fp32")
    L_b = np.array([b["L_bits"]], np.uint32).view(np.float32)[0]
    at_b = oracle_handle.row_at(fixture_row(a), token=0, K=4, L=L_b)
    assert at_b[2::2].tolist()[:3] == [2, 0, 1]
    assert [u32(int(x)) for x in at_b[5:9:2]] == [0xC2C60002, 0xC2C60002]
    L_a = np.array([a["L_bits"]], np.uint32).view(np.float32)[0]
    assert oracle_handle.row_at(fixture_row(a), token=0, K=4, L=L_a).tolist() == a["words"]
