"""Pins of the oracle's index path: canonical IDs, n-grams, hashes, rows.

Everything here checks the oracle against what the pages or mathematics fix,
not against a retyped copy of its own formulas:
  * splitmix64 known answers (the published generator's reference outputs);
  * page locality and the exact two-pages-per-token count (PageGram §3.1,
    §9.4 check 2, Fig. 2);
  * the S=1 and single-page limits (PageGram §3.2);
  * per-head and cross-head collision statistics against the closed forms
    (PageGram §3.2 eq. E[extra shared heads] = (K-1)/S, §6.1 Table 3:
    7/15 = 0.467 and 38.3% at S=15, K=8);
  * causality (Engram explainer, validation section).
"""
import numpy as np
import pytest

import oracle
from oracle import pagegram as og
import synth
from synth import configs


def tiny_layout(kind="pagegram", K=8, S=4, r=64, P=7, primes=None, seed=123,
                use_signs=1):
    return dict(kind=kind, n_min=2, n_max=3, K=K, S=S, r=r,
                pages=[P, P], head_rows=list(primes or [P * S] * (2 * K)),
                hash_seed=seed, use_signs=use_signs)


def test_splitmix64_reference_outputs():
    # splitmix64 started at state 0: the reference generator's first outputs.
    assert oracle.splitmix64(0, 0) == 0xE220A8397B1DCDAF
    assert oracle.splitmix64(0, 1) == 0x6E789E6AA1B965F4
    assert oracle.splitmix64(0, 2) == 0x06C45D188009454F


def test_mix64_avalanche_and_bijection():
    # Flipping one input bit flips each output bit with probability ~1/2; a
    # dropped round or shift shows up as a biased bit. Bijection: the inverse
    # built from modular inverses of the two multipliers undoes it.
    rng = np.random.default_rng(0)
    x = rng.integers(0, 2**63, size=2000, dtype=np.int64).astype(np.uint64)
    hx = og.mix64(x)
    frac = np.zeros(64)
    for bit in range(64):
        y = og.mix64(x ^ np.uint64(1 << bit))
        d = hx ^ y
        frac += np.array([((d >> np.uint64(j)) & np.uint64(1)).mean()
                          for j in range(64)])
    frac /= 64
    assert np.all(np.abs(frac - 0.5) < 0.02)

    def unxorshift(z, s):
        out = z
        for _ in range(64 // s + 1):
            out = z ^ (out >> s)
        return out
    m1 = pow(0xBF58476D1CE4E5B9, -1, 2**64)
    m2 = pow(0x94D049BB133111EB, -1, 2**64)
    for v in [0, 1, 2**63, 0x123456789ABCDEF0, 2**64 - 1]:
        z = int(og.mix64(np.array([v], np.uint64))[0])
        z = unxorshift(z, 31)
        z = (z * m2) % 2**64
        z = unxorshift(z, 27)
        z = (z * m1) % 2**64
        z = unxorshift(z, 30)
        assert z == v


def test_ngram_hash_python_int_brute_force():
    # The numpy uint64 path agrees with exact Python integers (no silent
    # promotion to float, no lost carry).
    c, a = og.role_constants(0x5EED0001, 3, og.KIND_HEAD, 5)
    g = np.array([[7, 0, 98000], [2**31 - 1, 12345, 1], [0, 0, 0]], np.int64)
    got = og.ngram_hash(g, c, a)
    for row, h in zip(g, got):
        x = c
        for j in range(3):
            x ^= (int(row[j]) * a[j]) % 2**64
        x &= 2**64 - 1
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) % 2**64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) % 2**64
        z ^= z >> 31
        assert int(h) == z


def test_multipliers_odd_and_roles_distinct():
    seen = set()
    for n in (2, 3):
        for kind, ks, ws in ((og.KIND_PAGE, [0], [0]),
                             (og.KIND_HEAD, range(16), [0]),
                             (og.KIND_SIGN, range(16), range(2))):
            for k in ks:
                for w in ws:
                    c, a = og.role_constants(1, n, kind, k, w)
                    assert all(x & 1 for x in a) and len(a) == n
                    assert (c, tuple(a)) not in seen
                    seen.add((c, tuple(a)))


def test_suffix_ngrams_and_pad():
    c = np.array([[5, 6, 7, 8], [1, 2, 3, 4]])
    g = og.suffix_ngrams(c, 3, 99)
    assert g[0, 0].tolist() == [5, 99, 99]
    assert g[0, 1].tolist() == [6, 5, 99]
    assert g[0, 3].tolist() == [8, 7, 6]
    # no n-gram crosses a batch row
    assert g[1, 0].tolist() == [1, 99, 99]


def test_canonicalize_out_of_range_is_pad():
    cm = np.array([3, 2, 1, 0], np.int32)
    c, bad = og.canonicalize(np.array([[0, 3, 4, -1]]), cm, 4)
    assert c.tolist() == [[3, 0, 4, 4]] and bad
    c, bad = og.canonicalize(np.array([[0, 1]]), cm, 4)
    assert not bad


@pytest.mark.parametrize("S", [1, 4, 15])
def test_page_locality_and_two_pages_per_token(S):
    lay = tiny_layout(K=8, S=S, P=13)
    rng = np.random.default_rng(S)
    toks = rng.integers(0, 500, size=(4, 300))
    res = oracle.index(lay, toks, np.arange(500), 500)
    bases, R = oracle.layout_bases(lay)
    K = lay["K"]
    rows, pages = res["rows"], res["pages"]
    assert rows.min() >= 0 and rows.max() < R == 2 * 13 * K * S
    for i in range(2):
        p = pages[:, i]
        assert (p >= 0).all() and (p < 13).all()
        lo = bases[i] + p * K * S
        # every head of a token-order lies inside that order's page ...
        assert ((rows[:, i, :] >= lo[:, None]) &
                (rows[:, i, :] < lo[:, None] + K * S)).all()
        # ... and head k inside its own S-slot block
        blk = (rows[:, i, :] - lo[:, None]) // S
        assert (blk == np.arange(K)[None, :]).all()
    # exactly two distinct pages per token (one per order)
    page_ids = (rows - np.array(bases)[None, :, None]) // (K * S)
    page_ids = page_ids + np.array([0, 10**6])[None, :, None]
    assert all(len(set(r.reshape(-1).tolist())) == 2 for r in page_ids)


def test_engram_rows_in_own_subtable():
    lay = tiny_layout(kind="engram", K=8, primes=configs.ENGRAM_200M_PRIMES)
    toks = np.random.default_rng(1).integers(0, 50304, size=(2, 512))
    res = oracle.index(lay, toks, np.arange(50304), 50304)
    bases, R = oracle.layout_bases(lay)
    assert R == sum(configs.ENGRAM_200M_PRIMES)
    for i in range(2):
        for k in range(8):
            lo = bases[i][k]
            hi = lo + configs.ENGRAM_200M_PRIMES[i * 8 + k]
            col = res["rows"][:, i, k]
            assert ((col >= lo) & (col < hi)).all()
    assert (res["pages"] == -1).all()


def test_single_page_pagegram_equals_engram():
    # PageGram §3.2: with one page per order, PageGram is Engram-style
    # multi-head addressing with P_{n,k} = S rows per head.
    S = 37
    pg = tiny_layout(K=8, S=S, P=1)
    en = tiny_layout(kind="engram", K=8, primes=[S] * 16)
    toks = np.random.default_rng(2).integers(0, 1000, size=(3, 200))
    a = oracle.index(pg, toks, np.arange(1000), 1000)
    b = oracle.index(en, toks, np.arange(1000), 1000)
    assert np.array_equal(a["rows"], b["rows"])
    assert np.array_equal(a["signs"], b["signs"])
    assert np.array_equal(a["hashes"], b["hashes"])


def test_s1_full_co_collision():
    # PageGram §3.2: with S=1, two n-grams on the same page share all K heads.
    lay = tiny_layout(K=8, S=1, P=5)
    V = 64
    a, b = np.meshgrid(np.arange(V), np.arange(V), indexing="ij")
    toks = np.stack([a.reshape(-1), b.reshape(-1)], axis=1)  # all bigrams
    res = oracle.index(lay, toks, np.arange(V), V)
    rows = res["rows"][1::2, 0, :]   # order-2 row of position 1 = (a, b)
    pages = res["pages"][1::2, 0]
    for p in range(5):
        sel = rows[pages == p]
        assert (sel == sel[0]).all()


def _pair_stats(rows):
    """rows int [n_grams, K]. Returns (per-head pair collision rates,
    E[#other heads colliding | head 0 collides], P(>=1 | head 0))."""
    n, K = rows.shape
    pairs_total = n * (n - 1) / 2
    rates = []
    for k in range(K):
        _, cnt = np.unique(rows[:, k], return_counts=True)
        rates.append((cnt * (cnt - 1) / 2).sum() / pairs_total)
    order = np.argsort(rows[:, 0], kind="stable")
    r0 = rows[order]
    bounds = np.flatnonzero(np.diff(r0[:, 0])) + 1
    extra_sum, any_sum, npairs = 0.0, 0.0, 0
    for grp in np.split(r0, bounds):
        m = len(grp)
        if m < 2:
            continue
        iu = np.triu_indices(m, 1)
        eq = (grp[iu[0], 1:] == grp[iu[1], 1:])
        extra_sum += eq.sum()
        any_sum += eq.any(axis=1).sum()
        npairs += len(iu[0])
    return np.array(rates), extra_sum / npairs, any_sum / npairs, npairs


def _all_bigram_rows(lay, V):
    a, b = np.meshgrid(np.arange(V), np.arange(V), indexing="ij")
    toks = np.stack([a.reshape(-1), b.reshape(-1)], axis=1)
    res = oracle.index(lay, toks, np.arange(V), V)
    return res["rows"][1::2, 0, :]


@pytest.mark.parametrize("P,S", [(7, 4), (13, 4), (7, 15), (13, 1)])
def test_collision_statistics_match_closed_forms(P, S):
    K = 8
    V = 64                            # 4096 distinct bigrams
    pg = _all_bigram_rows(tiny_layout(K=K, S=S, P=P), V)
    en = _all_bigram_rows(tiny_layout(kind="engram", K=K, primes=[P * S] * 16), V)
    rates_pg, extra_pg, any_pg, n_pg = _pair_stats(pg)
    rates_en, extra_en, any_en, n_en = _pair_stats(en)
    p = 1.0 / (P * S)
    # PageGram §3.2: the per-head collision rate is the same in both layouts
    # (both give each head P*S rows): 1/(P*S) within binomial noise.
    npairs = 4096 * 4095 / 2
    for rates in (rates_pg, rates_en):
        se = np.sqrt(p * (1 - p) / npairs) * 8   # pairs are not independent
        assert np.all(np.abs(rates - p) < 6 * se + 0.02 * p)
    # Cross-head correlation: E[extra shared heads | head 0] = (K-1)/S.
    exp_extra = (K - 1) / S
    exp_any = 1 - (1 - 1 / S) ** (K - 1)
    assert abs(extra_pg - exp_extra) < 0.05 * max(exp_extra, 0.1) + 0.02
    assert abs(any_pg - exp_any) < 0.03
    # Engram-style heads are independent: E[extra] = (K-1)/(P*S).
    assert abs(extra_en - (K - 1) * p) < 0.02 + 0.3 * (K - 1) * p


def test_printed_table3_values_at_s15():
    # PageGram §6.1 (Table 3): at S=15, K=8, 38.3% of head-0 collisions share
    # another head and the mean number of extra shared heads is 0.467 = 7/15.
    rows = _all_bigram_rows(tiny_layout(K=8, S=15, P=5), 90)   # 8100 bigrams
    _, extra, anyp, _ = _pair_stats(rows)
    assert abs(extra - 0.467) < 0.02
    assert abs(anyp - 0.383) < 0.02


def test_per_row_load_vmr_near_one():
    # PageGram §6.1: per-row load variance-to-mean ratio about 1.0 (ideal
    # random hashing). 10,000 bigrams into 211 pages x 4 slots per head.
    lay = tiny_layout(K=8, S=4, P=211)
    V = 100
    a, b = np.meshgrid(np.arange(V), np.arange(V), indexing="ij")
    toks = np.stack([a.reshape(-1), b.reshape(-1)], axis=1)
    rows = oracle.index(lay, toks, np.arange(V), V)["rows"][1::2, 0, :]
    K, S = 8, 4
    for k in range(K):
        # head k's rows: page p, slot s -> p*S + s
        head_row = (rows[:, k] // (K * S)) * S + rows[:, k] % S
        per = np.bincount(head_row, minlength=211 * S)
        vmr = per.var() / per.mean()
        assert 0.85 < vmr < 1.15, vmr


def test_causality_of_index():
    # Editing later tokens leaves earlier canonical IDs, hashes, rows and
    # signs unchanged (Engram explainer, validation: causality).
    lay = tiny_layout(K=8, S=4, P=97)
    rng = np.random.default_rng(5)
    toks = rng.integers(0, 300, size=(2, 64))
    a = oracle.index(lay, toks, np.arange(300), 300)
    t_edit = 40
    toks2 = toks.copy()
    toks2[:, t_edit:] = rng.integers(0, 300, size=(2, 64 - t_edit))
    b = oracle.index(lay, toks2, np.arange(300), 300)
    keep = (np.arange(2 * 64) % 64) < t_edit
    for key in ("hashes", "rows", "pages", "signs"):
        assert np.array_equal(a[key][keep], b[key][keep])
    assert not np.array_equal(a["rows"][~keep], b["rows"][~keep])


def test_sign_bit_order_reading():
    # Element j of a head uses bit j%64 of word j//64; a set bit is -1.
    w = np.array([[1 | (1 << 63), 0b10]], dtype=np.uint64)
    s = og.sign_vectors(w, 80)[0]
    assert s[0] == -1 and s[63] == -1 and s[65] == -1
    assert (s[1:63] == 1).all() and s[64] == 1 and (s[66:] == 1).all()


def test_sign_bits_balanced():
    lay = tiny_layout(K=8, S=4, P=97, r=80)
    toks = np.random.default_rng(9).integers(0, 1000, size=(4, 256))
    s = oracle.index(lay, toks, np.arange(1000), 1000)["signs"]
    assert s.shape[-1] == 2
    bits = og.sign_vectors(s, 80)
    assert abs(bits.mean()) < 0.02


def test_prime_sizes_and_parameter_parity():
    # PageGram §4: all 200M tables within 0.1% of each other; per-head primes
    # near 195,300 (Engram-style). Trial division.
    def isprime(n):
        if n < 2:
            return False
        i = 2
        while i * i <= n:
            if n % i == 0:
                return False
            i += 1
        return True
    for plist, start in ((configs.ENGRAM_200M_PRIMES, 195313),
                         (configs.ENGRAM_27B_PRIMES, 4453125),
                         (configs.ENGRAM_20B_PRIMES, 312_500_000 // 16)):
        assert len(set(plist)) == 16 and all(isprime(p) for p in plist)
        assert plist == sorted(plist) and plist[0] >= start
        # the first 16 primes >= start: no prime is skipped
        assert sum(isprime(n) for n in range(start, plist[-1] + 1)) == 16
    flat = 520832 * 384
    assert flat == 199_999_488
    paper_pg = (48823 + 48821) * 32 * 64
    assert paper_pg == 199_974_912
    ours_pg = oracle.layout_bases(configs.workload(1)["layout"])[1] * 64
    ours_en = oracle.layout_bases(configs.workload(2)["layout"])[1] * 64
    for v in (paper_pg, ours_pg, ours_en):
        assert abs(v - flat) / flat < 1e-3
    # Engram-27B memory: 5.7B parameters at width 80.
    big = oracle.layout_bases(configs.workload(4)["layout"])[1] * 80
    assert abs(big - 5.7e9) / 5.7e9 < 1e-3
    # 20B NF4 table: 312.5M rows of 64.
    r4 = oracle.layout_bases(configs.workload(3)["layout"])[1]
    assert abs(r4 * 64 - 20e9) / 20e9 < 1e-6
    # The same table at S = 15 (PageGram §3.3): a page is K*S = 120 NF4 head
    # rows = 120 * 34 = 4080 bytes inside one 4096-byte block, and the row
    # count stays within 1e-6 of 20B parameters.
    # the Engram-style comparison layout of the same 20B table
    r_en = oracle.layout_bases(configs.workload("engram20b_nf4_16x4096")["layout"])[1]
    assert abs(r_en * 64 - 20e9) / 20e9 < 1e-4
    lay15 = configs.workload(5)["layout"]
    assert lay15["S"] == 15 and lay15["K"] * lay15["S"] == 120
    assert lay15["K"] * lay15["S"] * (lay15["r"] // 2 + 2) == 4080 <= 4096
    r15 = oracle.layout_bases(lay15)[1]
    assert abs(r15 * 64 - 20e9) / 20e9 < 1e-6


def test_canonical_maps():
    for i in range(len(configs.ORDER)):
        wl = configs.workload(i)
        m = synth.canon_map(wl)
        assert len(m) == wl["vocab"]
        assert len(np.unique(m)) == wl["canon_vocab"]      # surjective
        assert m.min() == 0 and m.max() == wl["canon_vocab"] - 1
        if wl["canon"] == "identity":
            assert np.array_equal(m, np.arange(wl["vocab"]))
    # Engram notes §3.2: 128k vocabulary shrinks by 23.43%.
    wl = configs.workload(3)
    assert abs(1 - wl["canon_vocab"] / wl["vocab"] - 0.2343) < 5e-4
