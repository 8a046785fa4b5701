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
