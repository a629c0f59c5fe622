"""C ABI checks that need no GPU: the library loads and exports every symbol
include/*.h declares, the ctypes structs match the C compiler's layout, and
host-side validation returns the documented errors before anything is
enqueued (no call here reaches a kernel launch)."""
import ctypes
import glob
import os
import random
import re
import subprocess

import numpy as np
import pytest

import hashed_head_gram_amd as pg
import oracle
from synth import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    syms = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        txt = open(h).read()
        syms |= set(re.findall(r"PG_API\s+[\w\s\*]+?\b(pg_\w+)\s*\(", txt))
    return syms


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert {"pg_index", "pg_gather", "pg_index_gather", "pg_project_gate",
            "pg_forward", "pg_strerror", "pg_hash_version", "pg_layout_rows",
            "pg_workspace_size"} <= syms
    lib = pg.lib()
    for s in syms:
        assert hasattr(lib, s), s
    out = subprocess.run(["nm", "-D", "--defined-only", pg.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (pg_\w+)", out))
    assert syms <= exported


def test_struct_layout_matches_c_compiler(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "pagegram.h"
#define P(s, f) printf(#s "." #f " %zu\n", offsetof(s, f));
int main(void) {
  printf("pg_layout %zu\npg_table %zu\npg_fuse %zu\n", sizeof(pg_layout),
         sizeof(pg_table), sizeof(pg_fuse));
  P(pg_layout, pages) P(pg_layout, head_rows) P(pg_layout, hash_seed)
  P(pg_layout, use_signs) P(pg_layout, pad_id)
  P(pg_table, data) P(pg_table, scales) P(pg_table, n_rows)
  P(pg_fuse, g) P(pg_fuse, eps) P(pg_fuse, gamma_h) P(pg_fuse, conv_w)
  P(pg_fuse, conv_k) P(pg_fuse, increment_only)
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    vals = dict(line.split() for line in
                subprocess.run([str(exe)], capture_output=True, text=True,
                               check=True).stdout.splitlines())
    assert int(vals["pg_layout"]) == ctypes.sizeof(pg.PgLayout)
    assert int(vals["pg_table"]) == ctypes.sizeof(pg.PgTable)
    assert int(vals["pg_fuse"]) == ctypes.sizeof(pg.PgFuse)
    for key, v in vals.items():
        if "." in key:
            s, f = key.split(".")
            cls = {"pg_layout": pg.PgLayout, "pg_table": pg.PgTable,
                   "pg_fuse": pg.PgFuse}[s]
            assert getattr(cls, f).offset == int(v), key


def test_hash_version_and_strerror():
    assert pg.pg_hash_version() == oracle.HASH_VERSION == 1
    for st in (0, -1, -2, -3, -4):
        assert pg.lib().pg_strerror(st)
    assert pg.lib().pg_strerror(-99) == b"unknown status"


def layout_of(wl):
    d = wl["layout"]
    return pg.make_layout(d["kind"], d["K"], d["r"], S=d["S"], pages=d["pages"],
                          head_rows=d["head_rows"], hash_seed=d["hash_seed"],
                          use_signs=d["use_signs"], pad_id=wl["canon_vocab"])


@pytest.mark.parametrize("i", range(5))
def test_layout_rows_match_oracle(i):
    wl = configs.workload(i)
    assert pg.pg_layout_rows(layout_of(wl)) == oracle.layout_bases(wl["layout"])[1]


def expect(status, fn, *args):
    assert fn(*args) == status


def test_layout_validation():
    L = pg.lib()
    n = ctypes.c_int64()
    assert L.pg_layout_rows(None, ctypes.byref(n)) == pg.PG_EINVAL
    base = dict(kind="pagegram", K=8, r=64, S=4, pages=[10, 10], pad_id=5)
    for bad in (dict(K=0), dict(K=17), dict(r=0), dict(r=257), dict(S=0),
                dict(pages=[0, 10]), dict(pad_id=-1), dict(n_min=0),
                dict(n_min=3, n_max=2), dict(n_max=5), dict(kind=7),
                dict(use_signs=2)):
        lay = pg.make_layout(**{**base, **bad})
        assert L.pg_layout_rows(ctypes.byref(lay), ctypes.byref(n)) == pg.PG_EINVAL, bad
    lay = pg.make_layout(**{**base, "pages": [2**60, 2**60]})
    assert L.pg_layout_rows(ctypes.byref(lay), ctypes.byref(n)) == pg.PG_ERANGE
    en = pg.make_layout("engram", K=2, r=64, head_rows=[5, 7, 0, 11])
    assert L.pg_layout_rows(ctypes.byref(en), ctypes.byref(n)) == pg.PG_EINVAL
    en = pg.make_layout("engram", K=2, r=64, head_rows=[5, 7, 9, 11])
    assert L.pg_layout_rows(ctypes.byref(en), ctypes.byref(n)) == pg.PG_OK
    assert n.value == 32


FAKE = 1 << 40          # aligned, never dereferenced by these calls


def test_entry_points_validate_before_launch():
    L = pg.lib()
    wl = configs.workload(1)
    lay = layout_of(wl)
    R = pg.pg_layout_rows(lay)
    tab = pg.make_table(pg.PG_BF16, FAKE, R)
    by = ctypes.byref
    # pg_index: NULL layout, negative sizes, NULL required outputs
    assert L.pg_index(None, FAKE, 1, 1, FAKE, 10, None, None, FAKE, None, FAKE,
                      None, None) == pg.PG_EINVAL
    assert L.pg_index(by(lay), FAKE, -1, 1, FAKE, 10, None, None, FAKE, None, FAKE,
                      None, None) == pg.PG_EINVAL
    assert L.pg_index(by(lay), FAKE, 1, 4, FAKE, 10, None, None, None, None, FAKE,
                      None, None) == pg.PG_EINVAL
    assert L.pg_index(by(lay), FAKE, 1, 4, FAKE, 10, None, None, FAKE, None, None,
                      None, None) == pg.PG_EINVAL
    assert L.pg_index(by(lay), None, 1, 4, FAKE, 10, None, None, FAKE, None, FAKE,
                      None, None) == pg.PG_EINVAL
    assert L.pg_index(by(lay), FAKE, 1 << 20, 1 << 20, FAKE, 10, None, None, FAKE,
                      None, FAKE, None, None) == pg.PG_ERANGE
    # empty input: valid, nothing enqueued
    assert L.pg_index(by(lay), None, 0, 4, None, 0, None, None, None, None, None,
                      None, None) == pg.PG_OK
    # pg_gather: table rows mismatch, dtype mismatch, misaligned e, NULL signs
    bad_tab = pg.make_table(pg.PG_BF16, FAKE, R - 1)
    assert L.pg_gather(by(lay), by(bad_tab), FAKE, FAKE, 4, pg.PG_BF16, FAKE,
                       None) == pg.PG_EINVAL
    assert L.pg_gather(by(lay), by(tab), FAKE, FAKE, 4, pg.PG_F32, FAKE,
                       None) == pg.PG_EUNSUPPORTED
    assert L.pg_gather(by(lay), by(tab), FAKE, FAKE, 4, pg.PG_BF16, FAKE + 8,
                       None) == pg.PG_EINVAL
    assert L.pg_gather(by(lay), by(tab), FAKE, None, 4, pg.PG_BF16, FAKE,
                       None) == pg.PG_EINVAL
    assert L.pg_gather(by(lay), by(tab), None, None, 0, pg.PG_BF16, None,
                       None) == pg.PG_OK
    mis = pg.make_table(pg.PG_BF16, FAKE + 2, R)
    assert L.pg_gather(by(lay), by(mis), FAKE, FAKE, 4, pg.PG_BF16, FAKE,
                       None) == pg.PG_EINVAL
    nf4 = pg.make_table(pg.PG_NF4, FAKE, R)          # no scales
    assert L.pg_gather(by(lay), by(nf4), FAKE, FAKE, 4, pg.PG_BF16, FAKE,
                       None) == pg.PG_EINVAL
    # pg_index_gather: missing canon map
    assert L.pg_index_gather(by(lay), by(tab), FAKE, 1, 4, None, 10, pg.PG_BF16,
                             FAKE, None, None) == pg.PG_EINVAL
    # unsupported table widths
    lay12 = pg.make_layout("pagegram", 8, 12, S=4, pages=[3, 3], pad_id=5)
    t12 = pg.make_table(pg.PG_BF16, FAKE, pg.pg_layout_rows(lay12))
    assert L.pg_index_gather(by(lay12), by(t12), FAKE, 1, 4, FAKE, 10, pg.PG_BF16,
                             FAKE, None, None) == pg.PG_EUNSUPPORTED


def test_project_and_forward_validation():
    L = pg.lib()
    by = ctypes.byref
    f = pg.make_fuse(pg.PG_GATE_SCALAR, pg.PG_BF16, 768)
    assert L.pg_project_gate(None, FAKE, 1, 4, 1024, FAKE, None, FAKE, None, 0,
                             None) == pg.PG_EINVAL
    assert L.pg_project_gate(by(f), FAKE, 1, 4, 1020, FAKE, None, FAKE, None, 0,
                             None) == pg.PG_EUNSUPPORTED
    assert L.pg_project_gate(by(f), FAKE, 1, 4, 1024, None, None, FAKE, None, 0,
                             None) == pg.PG_EINVAL
    assert L.pg_project_gate(by(f), FAKE, 1, 4, 1024, FAKE, FAKE + 4, FAKE, None, 0,
                             None) == pg.PG_EINVAL
    assert L.pg_project_gate(by(f), None, 0, 4, 1024, None, None, None, None, 0,
                             None) == pg.PG_OK
    g = pg.make_fuse(pg.PG_GATE_ENGRAM, pg.PG_BF16, 2560, M=4, gamma_h=FAKE,
                     gamma_k=FAKE, gamma_u=FAKE, conv_w=FAKE)
    need = pg.pg_workspace_size(None, g, 2, 64)
    N = 128
    n_cb = 2560 // 256
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert need == (a(N * 2560 * 2) + a(n_cb * N * 4) + a(4 * 3 * n_cb * N * 4)
                    + a(4 * 2 * N * 4))
    assert L.pg_project_gate(by(g), FAKE, 2, 64, 1280, FAKE, FAKE, FAKE, FAKE,
                             need - 1, None) == pg.PG_EINVAL
    assert L.pg_project_gate(by(g), FAKE, 2, 64, 1280, FAKE, None, FAKE, FAKE,
                             need, None) == pg.PG_EINVAL           # h required
    g2 = pg.make_fuse(pg.PG_GATE_ENGRAM, pg.PG_BF16, 200, M=4, gamma_h=FAKE,
                      gamma_k=FAKE, gamma_u=FAKE, conv_w=FAKE)
    assert L.pg_project_gate(by(g2), FAKE, 2, 64, 1280, FAKE, FAKE, FAKE, FAKE,
                             1 << 30, None) == pg.PG_EUNSUPPORTED
    g3 = pg.make_fuse(pg.PG_GATE_ENGRAM, pg.PG_F32, 256, M=4, gamma_h=FAKE,
                      gamma_k=FAKE, gamma_u=FAKE, conv_w=FAKE)
    assert L.pg_project_gate(by(g3), FAKE, 2, 64, 1280, FAKE, FAKE, FAKE, FAKE,
                             1 << 30, None) == pg.PG_EUNSUPPORTED
    g4 = pg.make_fuse(pg.PG_GATE_ENGRAM, pg.PG_BF16, 256, M=9, gamma_h=FAKE,
                      gamma_k=FAKE, gamma_u=FAKE, conv_w=FAKE)
    assert L.pg_project_gate(by(g4), FAKE, 2, 64, 1280, FAKE, FAKE, FAKE, FAKE,
                             1 << 30, None) == pg.PG_EINVAL
    # pg_forward: workspace too small, dtype mismatch with the table
    wl = configs.workload(1)
    lay = layout_of(wl)
    R = pg.pg_layout_rows(lay)
    tab = pg.make_table(pg.PG_BF16, FAKE, R)
    need = pg.pg_workspace_size(lay, f, 8, 2048)
    assert need == 8 * 2048 * 1024 * 2
    assert L.pg_forward(by(lay), by(tab), by(f), FAKE, 8, 2048, FAKE, 50304, FAKE,
                        FAKE, FAKE, FAKE, need - 256, None, None) == pg.PG_EINVAL
    f32 = pg.make_fuse(pg.PG_GATE_SCALAR, pg.PG_F32, 768)
    assert L.pg_forward(by(lay), by(tab), by(f32), FAKE, 8, 2048, FAKE, 50304, FAKE,
                        FAKE, FAKE, FAKE, need, None, None) == pg.PG_EUNSUPPORTED
    assert L.pg_forward(by(lay), by(tab), by(f), None, 0, 2048, None, 0, None,
                        None, None, None, 0, None, None) == pg.PG_OK


def test_gathered_projection_validation():
    L = pg.lib()
    by = ctypes.byref
    wl = configs.workload(1)
    lay = layout_of(wl)
    R = pg.pg_layout_rows(lay)
    tab = pg.make_table(pg.PG_BF16, FAKE, R)
    f = pg.make_fuse(pg.PG_GATE_SCALAR, pg.PG_BF16, 768)
    assert pg.records_bytes(lay, 8 * 2048) == 16 * 8 * 2048 * 2 * 8
    # pg_index_records: NULL or misaligned output, rows other than 64 wide,
    # more than 2^28 tokens, empty input
    assert L.pg_index_records(by(lay), FAKE, 8, 2048, FAKE, 50304, None, None,
                              None) == pg.PG_EINVAL
    assert L.pg_index_records(by(lay), FAKE, 8, 2048, FAKE, 50304, FAKE + 8, None,
                              None) == pg.PG_EINVAL
    assert L.pg_index_records(by(lay), FAKE, 1 << 15, 1 << 14, FAKE, 50304, FAKE, None,
                              None) == pg.PG_ERANGE
    lay12 = pg.make_layout("pagegram", 8, 12, S=4, pages=[3, 3], pad_id=5)
    assert L.pg_index_records(by(lay12), FAKE, 1, 4, FAKE, 10, FAKE, None,
                              None) == pg.PG_EUNSUPPORTED
    assert L.pg_index_records(by(lay), None, 0, 4, None, 0, None, None, None) == pg.PG_OK
    # pg_project_gathered: NF4 table, Engram gate, fp32 operands, NULL records
    nf4 = pg.make_table(pg.PG_NF4, FAKE, R, scales=FAKE)
    assert L.pg_project_gathered(by(lay), by(nf4), by(f), FAKE, 8, 2048, FAKE, None, FAKE,
                                 None) == pg.PG_EUNSUPPORTED
    g = pg.make_fuse(pg.PG_GATE_ENGRAM, pg.PG_BF16, 768, M=4, gamma_h=FAKE,
                     gamma_k=FAKE, gamma_u=FAKE, conv_w=FAKE)
    assert L.pg_project_gathered(by(lay), by(tab), by(g), FAKE, 8, 2048, FAKE, FAKE, FAKE,
                                 None) == pg.PG_EUNSUPPORTED
    f32 = pg.make_fuse(pg.PG_GATE_SCALAR, pg.PG_F32, 768)
    assert L.pg_project_gathered(by(lay), by(tab), by(f32), FAKE, 8, 2048, FAKE, None, FAKE,
                                 None) == pg.PG_EUNSUPPORTED
    assert L.pg_project_gathered(by(lay), by(tab), by(f), None, 8, 2048, FAKE, None, FAKE,
                                 None) == pg.PG_EINVAL
    assert L.pg_project_gathered(by(lay), by(tab), by(f), FAKE, 8, 2048, FAKE, FAKE + 4,
                                 FAKE, None) == pg.PG_EINVAL
    assert L.pg_project_gathered(by(lay), by(tab), by(f), None, 0, 2048, None, None, None,
                                 None) == pg.PG_OK


def test_magic_remainder_needs_one_correction():
    # The kernels reduce 64-bit hashes with q = floor(x * floor((2^64-1)/P) /
    # 2^64) and one conditional subtraction. Check that q is the quotient or
    # one less, on edge cases and random values, with exact integers.
    M = 2**64 - 1
    rng = random.Random(1)
    Ps = [1, 2, 3, 4, 7, 15, 48828, 195319, 4453349, 4882812, 2**32 - 1, 2**32 + 15,
          2**40 + 3, 2**62 + 11] + [rng.randrange(1, 2**63) for _ in range(50)]
    xs = [0, 1, M, M - 1, 2**63, 2**32] + [rng.randrange(0, 2**64) for _ in range(200)]
    for P in Ps:
        m = M // P
        for x in xs + [P - 1, P, 2 * P - 1, (M // P) * P, (M // P) * P - 1]:
            if x > M or x < 0:
                continue
            q = (x * m) >> 64
            r = x - q * P
            assert 0 <= r < 2 * P
            if r >= P:
                r -= P
            assert r == x % P


def test_workspace_sizes_nonnegative_for_workloads():
    for i in range(5):
        wl = configs.workload(i)
        lay = layout_of(wl)
        dt = pg.PG_F32 if wl["act_dtype"] == "f32" else pg.PG_BF16
        if wl["gate"] == "engram":
            f = pg.make_fuse(pg.PG_GATE_ENGRAM, dt, wl["d"], M=wl["M"], gamma_h=FAKE,
                             gamma_k=FAKE, gamma_u=FAKE, conv_w=FAKE)
        else:
            f = pg.make_fuse(pg.PG_GATE_SCALAR, dt, wl["d"])
        n = pg.pg_workspace_size(lay, f, wl["B"], wl["T"])
        E = configs.e_dim(wl)
        assert n >= wl["B"] * wl["T"] * E * (4 if dt == pg.PG_F32 else 2)
        assert np.int64(n) > 0
