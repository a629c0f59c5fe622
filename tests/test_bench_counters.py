"""Host logic of bench.py's counter processing (no GPU): which copies set the
FETCH_SIZE / WRITE_SIZE scale, and read bytes from requests counted by size."""
import csv
import importlib.util
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _bench():
    spec = importlib.util.spec_from_file_location("bench_for_tests", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    argv = sys.argv
    sys.argv = ["bench.py"]
    try:
        spec.loader.exec_module(mod)
    finally:
        sys.argv = argv
    return mod


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(COLS, r)))


def _dispatches(counter, copy_kib, gather_kib, big_copy_kib):
    """A set-up copy larger than the probe copies, two gather dispatches
    (counter values split over two instances), then the five probe copies."""
    rows = [(3, "__amd_rocclr_copyBuffer", counter, big_copy_kib)]
    for d in (10, 11):
        rows.append((d, "void pg::(anonymous namespace)::index_gather_kernel<1, false>(...)",
                     counter, gather_kib / 2))
        rows.append((d, "void pg::(anonymous namespace)::index_gather_kernel<1, false>(...)",
                     counter, gather_kib / 2))
    for d in range(20, 25):
        rows.append((d, "__amd_rocclr_copyBuffer", counter, copy_kib))
    return rows


def test_probe_copies_set_the_scale_and_request_sizes_give_bytes(tmp_path):
    b = _bench()
    gib_kib = (1 << 30) / 1024
    # FETCH_SIZE reads half of the probe copy (128-byte requests counted as
    # 64), WRITE_SIZE all of it; a 2.5 GiB set-up copy comes first
    _csv(tmp_path / "f.csv", _dispatches("FETCH_SIZE", gib_kib / 2, 100.0, 2.5 * gib_kib / 2))
    _csv(tmp_path / "w.csv", _dispatches("WRITE_SIZE", gib_kib, 50.0, 2.5 * gib_kib))
    req = []
    for name, n128 in (("__amd_rocclr_copyBuffer", (1 << 30) // 128),
                       ("void pg::(anonymous namespace)::index_gather_kernel<1, false>(...)", 1600)):
        for d in ((20, 21, 22, 23, 24) if "copy" in name else (10, 11)):
            req += [(d, name, "TCC_EA0_RDREQ_sum", n128 + 10), (d, name, "TCC_EA0_RDREQ_32B_sum", 0),
                    (d, name, "TCC_EA0_RDREQ_64B_sum", 10), (d, name, "TCC_EA0_RDREQ_128B_sum", n128)]
    req.append((3, "__amd_rocclr_copyBuffer", "TCC_EA0_RDREQ_sum", 5 * (1 << 30) // 128))
    _csv(tmp_path / "r.csv", req)
    out = tmp_path / "traffic.json"
    b.write_traffic("wl", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                    str(tmp_path / "r.csv"), path=str(out))
    ent = json.load(open(out))["wl"]
    assert ent["copy_scale"]["fetch"] == pytest.approx(2.0)
    assert ent["copy_scale"]["write"] == pytest.approx(1.0)
    g = ent["gather"]
    assert g["fetch_bytes"] == pytest.approx(100.0 * 1024 * 2.0)
    assert g["write_bytes"] == pytest.approx(50.0 * 1024)
    assert g["read_requests"]["bytes"] == 1600 * 128 + 10 * 64
    assert ent["copy_scale"]["copy_read_requests"]["bytes"] == (1 << 30) + 10 * 64
    assert g["source_digest"] == b.source_digest(b.KERNEL_SOURCES["gather"])


def test_source_digest_follows_code_not_comments(tmp_path, monkeypatch):
    # The digest that keeps counter figures attached to a kernel: an edit to
    # comments or blank lines keeps it, any edit to the code changes it.
    src = tmp_path / "k.hip"
    base = "// header\nint f(int x) {\n  return x + 1;  // one\n}\n"
    src.write_text(base)
    b = _bench()
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    d0 = b.source_digest(["k.hip"])
    src.write_text("// header, reworded\n\nint f(int x) {   \n  return x + 1;  // one more\n}\n")
    assert b.source_digest(["k.hip"]) == d0
    src.write_text(base.replace("x + 1", "x + 2"))
    assert b.source_digest(["k.hip"]) != d0
    src.write_text(base.replace("return", "return -"))
    assert b.source_digest(["k.hip"]) != d0
