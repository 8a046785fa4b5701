"""The oracle against its pins (CPU only)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_handle, pin):
    pin(oracle_handle)


def test_packed_negative_offset_is_inactive(oracle_handle):
    """A negative packed row offset makes the slot inactive (reading R13).
    Kept out of the mutant pins: a mutant without the check would read
    before the buffer."""
    import numpy as np
    c = oracle_pins.packed_case()
    off = c["offsets"].copy()
    off[4] = -1
    out = np.full((c["cap"], c["T"], 258), -559038737, dtype=np.int32)
    n, _ = oracle_handle.frame_packed(c["packed"], c["cap"], c["T"], c["P"], c["V"], c["V_pad"],
                                      c["requested"], c["id_counts"], c["ids"], c["emitted"],
                                      c["tokens"], off, 20, out)
    assert np.all(out[4] == -559038737)
    assert n == 2 + 4 + 3 + 1 + 4 - 1  # every committed row but slot 4's one
