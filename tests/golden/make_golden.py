"""Writes tests/golden/tiny_brute.json: tiny GQA decode cases and their 50-digit
decimal brute-force outputs (oracle/brute.py).  The expected values come from
the oracle package only; the inputs are stored alongside them so the fixture
stays valid if the input generator changes.

Definition pinned (kernbench2 page "_gqa_attention_decode_long.py", "Tile 0"
block over all keys + final normalise-and-store): o = softmax(scale * q K^T) V,
query head h reading kv head h // (h_q // h_kv).

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from gqa_split_kv_amd.inputs import host_case  # noqa: E402
from oracle.brute import brute_decode  # noqa: E402

CASES = [
    # name, dtype, batch, h_q, h_kv, d, seq_lens, scale, seed
    ("bf16_G2_ragged", "bf16", 2, 4, 2, 4, [3, 5], 0.5, 11),
    ("f32_G3_scale1", "f32", 1, 3, 1, 2, [4], 1.0, 12),
    ("bf16_mha_empty_and_one", "bf16", 3, 2, 2, 8, [0, 1, 7], 8 ** -0.5, 13),
    ("bf16_mqa_G4", "bf16", 1, 4, 1, 8, [16], 8 ** -0.5, 14),
]


def main():
    out = []
    for name, dtype, batch, h_q, h_kv, d, sl, scale, seed in CASES:
        c = host_case(batch, h_q, h_kv, d, sl, dtype, seed=seed, scale=scale)
        o = brute_decode(c.q, c.k, c.v, c.seq_lens, c.scale)
        out.append({
            "name": name, "dtype": dtype, "batch": batch, "h_q": h_q, "h_kv": h_kv, "d": d,
            "seq_lens": sl, "scale": scale,
            "q": c.q.reshape(-1).tolist(), "k": c.k.reshape(-1).tolist(), "v": c.v.reshape(-1).tolist(),
            "o": [[[format(x, ".30e") for x in row] for row in ob] for ob in o],
        })
    path = os.path.join(HERE, "tiny_brute.json")
    with open(path, "w") as f:
        json.dump({"source": "oracle/brute.py (50-digit decimal), definition: softmax(scale*qK^T)V, "
                             "kernbench2 page _gqa_attention_decode_long.py Tile 0 + final normalise",
                   "cases": out}, f, indent=0)
    print("wrote", path)


if __name__ == "__main__":
    main()
