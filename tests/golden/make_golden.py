"""Write the small worked examples under tests/golden/ (calls only the oracle).

Each fixture is a designed row whose answer can be checked by hand from the
rule it exercises; the note in each file says how.  Run from the repository
root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def bf16(vals):
    u = np.asarray(vals, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)  # all values below are exact in bf16


FIXTURES = [
    dict(name="uniform_v4_fp32",
         cite="Generation-logprobs design page, definition paragraph (logit minus the "
              "full-vocabulary logsumexp)",
         note="Four equal logits: L = ln 4 = 1.3862944 (FP32 0x3FB17218); every lane "
              "reports -ln 4 (0xBFB17218); ties list IDs 0,1,2,3; the other 16 pairs are "
              "(-1, 0x7FC00000) because V < K.",
         dtype="fp32", row=[0.0, 0.0, 0.0, 0.0], token=2, K=20, sel=[]),
    dict(name="subtraction_tie_v64_fp32",
         cite="Generation-logprobs design page, tiled-reduction paragraph (keys rank the "
              "reported FP32 values; ties created by the subtraction are ties)",
         note="x0 = nextafter(1, 0), x1 = 1, x2 = 100, others -inf.  L = 100 exactly; "
              "x0 - L and x1 - L both round to -99, so ID 0 precedes ID 1 although its "
              "logit is smaller: order 2, 0, 1, then the -inf lanes by ID.",
         dtype="fp32",
         row=[float(np.nextafter(np.float32(1), np.float32(0))), 1.0, 100.0] + [-np.inf] * 61,
         token=1, K=20, sel=[]),
    dict(name="signed_zero_v32_bf16",
         cite="Generation-logprobs design page, tiled-reduction paragraph (signed zero is "
              "normalized)",
         note="Only lane 9 is finite and it is -0.0 (bf16 0x8000): L = 0 and the chosen "
              "value is -0 - 0 = -0, stored as +0 (bits 0).",
         dtype="bf16", row=[-np.inf] * 9 + [-0.0] + [-np.inf] * 22, token=9, K=3, sel=[]),
    dict(name="v_below_k_v5_fp32",
         cite="Generation-logprobs design page, definition paragraph (order) and "
              "packed-position paragraph (-1 IDs when the vocabulary has fewer than K "
              "entries)",
         note="Logits [1, 3, 3, -inf, 0.5]: order 1, 2 (tie -> smaller ID), 0, 4, 3; "
              "pairs 5..19 are (-1, 0x7FC00000).",
         dtype="fp32", row=[1.0, 3.0, 3.0, -np.inf, 0.5], token=3, K=20, sel=[]),
    dict(name="selected_ids_v10_fp32",
         cite="Generation-logprobs design page, definition paragraph (selected IDs in "
              "caller order, same normalization, chosen pair stored separately)",
         note="Selected [9, -1, 10, 3, 3] keep caller order; IDs outside [0, 10) carry "
              "NaN bits 0x7FC00000; the repeated ID 3 is reported twice; the chosen "
              "token 10 is outside the vocabulary and also gets NaN bits.",
         dtype="fp32", row=[0.5 * i for i in range(10)], token=10, K=20,
         sel=[9, -1, 10, 3, 3]),
    dict(name="grid_ties_v48_bf16",
         cite="Generation-logprobs design page, definition paragraph (equal values by "
              "increasing token ID)",
         note="Logits on a 1/8 grid with the top level 2.0 at IDs 5, 17, 40 and the next "
              "level 1.875 at IDs 0, 2, 3: the first six alternatives are 5, 17, 40, 0, 2, 3.",
         dtype="bf16",
         row=[1.875 if i in (0, 2, 3) else 2.0 if i in (5, 17, 40) else (i % 8) / 8.0 - 1.0
              for i in range(48)],
         token=17, K=6, sel=[]),
    dict(name="last_bit_of_L_a_v64_fp32",
         cite="Generation-logprobs design page, tiled-reduction paragraph (keys rank the "
              "reported FP32 values, one subtraction of the row's normalization)",
         note="x0 = 1 - 2^-18 - 2^-24, x1 = 1 - 2^-18, x2 = 100, others -inf.  L = 100 "
              "exactly.  x1 - L = -(99 + 2^-18) is halfway between -99 and -(99 + 2^-17) "
              "and rounds to the even -99; x0 - L lies past the halfway point and rounds "
              "to -(99 + 2^-17).  Order 2, 1, 0: the larger logit first.",
         dtype="fp32",
         row=[float(np.float32(1 - 2.0**-18 - 2.0**-24)), float(np.float32(1 - 2.0**-18)),
              100.0] + [-np.inf] * 61,
         token=0, K=4, sel=[]),
    dict(name="last_bit_of_L_b_v64_fp32",
         cite="Generation-logprobs design page, tiled-reduction paragraph (keys rank the "
              "reported FP32 values, one subtraction of the row's normalization)",
         note="The previous row with x2 = 100 + 2^-17, the next FP32 value: L = 100 + "
              "2^-17 exactly, one unit in the last place above the previous L.  Now x1 - L "
              "= -(99 + 3 * 2^-18) is halfway between -(99 + 2^-17) and -(99 + 2^-16) and "
              "rounds to the even -(99 + 2^-16), and x0 - L rounds there too: the two tie "
              "and the smaller ID leads.  Order 2, 0, 1.",
         dtype="fp32",
         row=[float(np.float32(1 - 2.0**-18 - 2.0**-24)), float(np.float32(1 - 2.0**-18)),
              float(np.float32(100 + 2.0**-17))] + [-np.inf] * 61,
         token=0, K=4, sel=[]),
]


def main():
    o = oracle.get()
    for fx in FIXTURES:
        vals = np.asarray(fx["row"], dtype=np.float32)
        row = bf16(vals) if fx["dtype"] == "bf16" else vals
        words, L = o.row(row, token=fx["token"], K=fx["K"], sel=fx["sel"] or None)
        rec = dict(name=fx["name"], cite=fx["cite"], note=fx["note"], dtype=fx["dtype"],
                   V=int(vals.size), K=fx["K"], token=fx["token"], sel=fx["sel"],
                   row_bits=[int(x) for x in (row.astype(np.uint32) if fx["dtype"] == "bf16"
                                              else row.view(np.uint32))],
                   L_bits=int(np.array([L], dtype=np.float32).view(np.uint32)[0]),
                   words=[int(w) for w in words])
        with open(os.path.join(HERE, fx["name"] + ".json"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print("wrote", fx["name"])


if __name__ == "__main__":
    main()
