"""Writes hash_v1.json: frozen index outputs of the oracle (hash version 1).

Calls only the oracle. The inputs are literal token IDs and identity
canonical maps, one case per layout shape used by the workloads. The stored
values are regression fixtures: they freeze the hash definition so that a
change to it is seen (the hash itself is pinned by the oracle's collision and
known-answer tests, not by this file).

    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))

TOKENS = [[0, 1, 2, 3, 1023, 7, 7, 7, 500, 12],
          [5, 5, 900, 0, 0, 1, 2, 3, 4, 1022]]

CASES = {
    "pagegram_K4_S4_r16_P64": dict(kind="pagegram", n_min=2, n_max=3, K=4,
                                   S=4, r=16, pages=[64, 64], head_rows=[],
                                   hash_seed=0x5EED0001, use_signs=1),
    "pagegram_K8_S4_r64_P48828": dict(kind="pagegram", n_min=2, n_max=3, K=8,
                                      S=4, r=64, pages=[48828, 48828],
                                      head_rows=[], hash_seed=0x5EED0001,
                                      use_signs=1),
    "engram_K8_r80_primes27b": dict(kind="engram", n_min=2, n_max=3, K=8, S=1,
                                    r=80, pages=[],
                                    head_rows=[4453129, 4453139, 4453147,
                                               4453159, 4453171, 4453177,
                                               4453187, 4453213, 4453223,
                                               4453231, 4453259, 4453271,
                                               4453291, 4453321, 4453331,
                                               4453349],
                                    hash_seed=0x5EED0001, use_signs=1),
}


def main():
    out = {"hash_version": oracle.HASH_VERSION, "vocab": 1024,
           "pad_id": 1024, "tokens": TOKENS, "cases": {}}
    for name, lay in CASES.items():
        res = oracle.index(lay, np.array(TOKENS), np.arange(1024), 1024)
        out["cases"][name] = dict(
            layout=lay,
            hashes=[[[str(int(v)) for v in o] for o in t] for t in res["hashes"]],
            rows=res["rows"].tolist(), pages=res["pages"].tolist(),
            signs=[[[[str(int(v)) for v in k] for k in o] for o in t]
                   for t in res["signs"]])
    with open(os.path.join(HERE, "hash_v1.json"), "w") as f:
        json.dump(out, f, indent=0)


if __name__ == "__main__":
    main()
