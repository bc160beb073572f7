"""Draw and freeze the per-layer table of the 14B-shaped mixed 4x workload.

Workload: 48 layers, r = 512, d_R = 64.  Layer 0 is an anchor; every later
layer inherits from the nearest preceding anchor with probability 1/3,
otherwise it draws d from {128, 256, 384, 512} and b from {2, 4, 8, 16}
uniformly.  The whole table is redrawn until the stored bits per token are
within 1 % of one quarter of the uncompressed MLA cache (every layer an
anchor with d = r and b = 16: 48 * ((512 + 64) * 16 + 32) = 443,904 bits).

Bit accounting is the oracle's (per-token cost of an action from the
"Action Space and Cost Model" section of the KV-Kaizen summary page, plus one
32-bit scale per anchor).  Run:  python tests/golden/make_table_14b_mixed.py

It also freezes four tables drawn by the same rule (seeds 7, 8, 9, 10; the
first is the table above) for the heterogeneous-batch workload, where each
quarter of the batch uses one of them (a selector that adapts the table to
each prompt gives a batch of different tables).
"""

import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import kk_oracle as ko  # noqa: E402

L, R, DR, SEED = 48, 512, 64, 7
D_SET = (128, 256, 384, 512)
B_SET = (2, 4, 8, 16)


def draw(rng):
    table = [[0, int(rng.choice(D_SET)), int(rng.choice(B_SET))]]
    last_anchor = 0
    for l in range(1, L):
        if rng.random() < 1.0 / 3.0:
            table.append([last_anchor, 0, 0])
        else:
            table.append([l, int(rng.choice(D_SET)), int(rng.choice(B_SET))])
            last_anchor = l
    return table


def bits_of(table):
    layers = [ko.Layer(a, d, b, 1.0) for (a, d, b) in table]
    return ko.table_bits_per_token(layers, DR)


HETERO_SEEDS = (7, 8, 9, 10)


def freeze(seed):
    """(table, draws, bits) of the first draw of `seed` within 1 % of the target."""
    full = L * ((R + DR) * 16 + ko.SCALE_BITS)
    target = full / 4
    lo, hi = target * 0.99, target * 1.01
    rng = np.random.default_rng(seed)
    draws = 0
    while True:
        draws += 1
        t = draw(rng)
        bits = bits_of(t)
        if lo <= bits <= hi:
            return t, draws, bits


def main():
    full = L * ((R + DR) * 16 + ko.SCALE_BITS)
    t, draws, bits = freeze(SEED)
    out = {
        "description": "14B-shaped mixed 4x table: 48 layers, r=512, d_R=64, seed 7",
        "rule": "layer 0 anchor; later layers inherit nearest anchor w.p. 1/3, else d~U{128,256,384,512}, "
                "b~U{2,4,8,16}; redraw whole table until bits/token within 1% of 443904/4",
        "draws": draws,
        "bits_per_token": bits,
        "uncompressed_mla_bits_per_token": full,
        "ratio_vs_mla_uncompressed": full / bits,
        "ratio_vs_c0_non_mla": ko.c0_bits(48, 8, 128) / bits,
        "table": t,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "table_14b_mixed.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: v for k, v in out.items() if k != "table"}))
    tables = []
    for seed in HETERO_SEEDS:
        ts, ds, bs = freeze(seed)
        tables.append({"seed": seed, "draws": ds, "bits_per_token": bs, "table": ts})
    het = {
        "description": "four 14B-shaped mixed 4x tables (48 layers, r=512, d_R=64) drawn by the rule above, "
                       "seeds 7-10; the heterogeneous batch gives each a quarter of its sequences",
        "tables": tables,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tables_14b_hetero.json")
    with open(path, "w") as f:
        json.dump(het, f, indent=1)
    print(json.dumps([{k: v for k, v in x.items() if k != "table"} for x in tables]))


if __name__ == "__main__":
    main()
