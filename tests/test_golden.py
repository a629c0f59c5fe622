"""Regression fixture: the oracle's hash version 1 outputs stay frozen.

tests/golden/hash_v1.json is written by tests/golden/make_golden.py, which
calls only the oracle."""
import json
import os

import numpy as np

import oracle

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_hash_v1_frozen():
    g = json.load(open(os.path.join(HERE, "hash_v1.json")))
    assert g["hash_version"] == oracle.HASH_VERSION == 1
    for name, case in g["cases"].items():
        res = oracle.index(case["layout"], np.array(g["tokens"]),
                           np.arange(g["vocab"]), g["pad_id"])
        hashes = np.array([[[int(v) for v in o] for o in t]
                           for t in case["hashes"]], dtype=np.uint64)
        signs = np.array([[[[int(v) for v in k] for k in o] for o in t]
                          for t in case["signs"]], dtype=np.uint64)
        assert np.array_equal(res["hashes"], hashes), name
        assert np.array_equal(res["rows"], np.array(case["rows"])), name
        assert np.array_equal(res["pages"], np.array(case["pages"])), name
        assert np.array_equal(res["signs"], signs), name
