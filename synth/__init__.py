"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module generates inputs only; it holds none of the n-gram memory's
arithmetic (no canonicalisation, hashing, addressing, gathering, projection or
gating). Everything is reproducible from the seeds in ``synth.configs``:

* token streams: numpy PCG64; uniform IDs, or Zipf(s) IDs over [0, V) by
  inverse CDF (P(i) proportional to (i+1)^-s);
* canonical maps: identity, or a seeded surjection V -> V' built from a random
  permutation (the first V' permuted IDs take the canonical IDs 0..V'-1, the
  rest take random canonical IDs);
* float tensors (tables, projections, residual inputs, gains, conv weights):
  a counter-based generator, so that any element can be recomputed from its
  flat index without materialising the tensor. Element i of stream s under
  seed q is built from the 64-bit word

      base  = mix64(q XOR (s * 0xD1B54A32D192ED03))
      word  = mix64(base + (i + 1) * 0x9E3779B97F4A7C15)

  i.e. output i of a splitmix64 generator (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014) started at state
  ``base``. An approximately normal value takes the sum of the word's four
  16-bit fields (Irwin-Hall, n=4), subtracts the mean 131070 and multiplies
  once, in fp32 with round-to-nearest-even, by fp32(sigma*sqrt(3)/65536);
  bf16 tensors round that fp32 value to bf16 (nearest-even). NF4 tables take
  their 4-bit codes from the bytes of the words (row i, byte b comes from
  byte b%8, little-endian, of word i*(r/16) + b//8 of the table stream) and
  their scales as fp16(fp32(q16 + 49152) * fp32(0.05/65536)) from the low 16
  bits q16 of word i of the scale stream.

The GPU fills large tensors with a kernel implementing the same definition
(``synth/fill.hip``); tests check the two agree bit for bit on sampled indices.
"""
import math

import numpy as np

from . import configs  # noqa: F401

_M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
STREAM_MUL = 0xD1B54A32D192ED03


def _mix64_np(z):
    """splitmix64 output function on a uint64 array (wrapping arithmetic)."""
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= np.uint64(0xBF58476D1CE4E5B9)
    z ^= z >> np.uint64(27)
    z *= np.uint64(0x94D049BB133111EB)
    z ^= z >> np.uint64(31)
    return z


def _mix64_int(z):
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def stream_base(seed, stream):
    return _mix64_int((int(seed) ^ ((int(stream) * STREAM_MUL) & _M64)) & _M64)


def words(seed, stream, idx):
    """64-bit generator words for the flat indices ``idx`` (any int array)."""
    base = np.uint64(stream_base(seed, stream))
    i = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = base + (i + np.uint64(1)) * np.uint64(GOLDEN)
    return _mix64_np(state)


def normal_scale(sigma):
    """The fp32 multiplier that turns a centred Irwin-Hall sum into N(0,sigma)."""
    return np.float32(float(sigma) * math.sqrt(3.0) / 65536.0)


def normal_f32(seed, stream, idx, sigma):
    """Approximately N(0, sigma) fp32 values for the flat indices ``idx``."""
    w = words(seed, stream, idx)
    m = np.uint64(0xFFFF)
    s = ((w & m) + ((w >> np.uint64(16)) & m) + ((w >> np.uint64(32)) & m)
         + (w >> np.uint64(48))).astype(np.int64)
    return (s - 131070).astype(np.float32) * normal_scale(sigma)


def f32_to_bf16_bits(x):
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))
    return (b >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def normal_values(seed, stream, idx, sigma, dtype):
    """Values of a float tensor at flat indices, in its storage type.

    dtype "f32" gives float32; "bf16" gives uint16 bf16 bit patterns.
    """
    v = normal_f32(seed, stream, idx, sigma)
    if dtype == "f32":
        return v
    if dtype == "bf16":
        return f32_to_bf16_bits(v)
    raise ValueError(dtype)


def nf4_codes(seed, rows, r):
    """Packed 4-bit codes of the given rows: uint8 [len(rows), r/2]."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    nb = r // 2
    wpr = nb // 8
    widx = rows[:, None] * wpr + np.arange(wpr, dtype=np.int64)[None, :]
    w = words(seed, configs.STREAM_TABLE, widx)
    return w.view(np.uint8).reshape(len(rows), nb)


def nf4_scales(seed, rows):
    """fp16 per-row scales of the given rows."""
    w = words(seed, configs.STREAM_NF4_SCALE, np.asarray(rows, dtype=np.int64))
    q = (w & np.uint64(0xFFFF)).astype(np.float32)
    return ((q + np.float32(49152.0)) * np.float32(0.05 / 65536.0)).astype(
        np.float16)


# ----------------------------------------------------------------------------
# Tokens and canonical maps


def zipf_cdf(V, s):
    p = (np.arange(1, V + 1, dtype=np.float64)) ** (-float(s))
    c = np.cumsum(p)
    return c / c[-1]


def tokens(wl, batch=0):
    """int32 [B, T] token IDs of a workload; ``batch`` selects another draw."""
    B, T, V = wl["B"], wl["T"], wl["vocab"]
    rng = np.random.Generator(np.random.PCG64(wl["token_seed"] + 7919 * batch))
    if wl["token_dist"] == "uniform":
        t = rng.integers(0, V, size=(B, T))
    elif wl["token_dist"] == "zipf":
        u = rng.random(size=(B, T))
        t = np.searchsorted(zipf_cdf(V, wl["zipf_s"]), u, side="right")
        t = np.minimum(t, V - 1)
    else:
        raise ValueError(wl["token_dist"])
    return t.astype(np.int32)


def canon_map(wl):
    """int32 [V] canonical map of a workload (values in [0, V'))."""
    V, Vc = wl["vocab"], wl["canon_vocab"]
    if wl["canon"] == "identity":
        return np.arange(V, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(wl["map_seed"]))
    perm = rng.permutation(V)
    m = np.empty(V, dtype=np.int64)
    m[perm[:Vc]] = np.arange(Vc)
    m[perm[Vc:]] = rng.integers(0, Vc, size=V - Vc)
    return m.astype(np.int32)


# ----------------------------------------------------------------------------
# Workload tensors on the host (small ones whole, big ones by index)


def table_rows(wl, rows):
    """Stored values of table rows: f32 / bf16 bits, or (codes, scales)."""
    r = wl["layout"]["r"]
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    seed = wl["table_seed"]
    if wl["table_dtype"] == "nf4":
        return nf4_codes(seed, rows, r), nf4_scales(seed, rows)
    idx = rows[:, None] * r + np.arange(r, dtype=np.int64)[None, :]
    return normal_values(seed, configs.STREAM_TABLE, idx,
                         wl["table_sigma"], wl["table_dtype"])


def dense_rows(wl, stream, row_idx, width, sigma, dtype=None):
    """Rows of a row-major dense tensor of the given width."""
    row_idx = np.asarray(row_idx, dtype=np.int64).reshape(-1)
    idx = row_idx[:, None] * width + np.arange(width, dtype=np.int64)[None, :]
    return normal_values(wl["data_seed"], stream, idx, sigma,
                         dtype or wl["act_dtype"])


def weight(wl):
    """Projection W [d_out, E] in its storage type (d_out = (1+M)d if fused)."""
    E = configs.e_dim(wl)
    return dense_rows(wl, configs.STREAM_W, np.arange(configs.d_out(wl)), E,
                      wl["w_sigma"])


def resid_rows(wl, flat_rows):
    """Residual input rows (x, or h flattened as [M*N_tok]) by flat row."""
    return dense_rows(wl, configs.STREAM_RESID, flat_rows, wl["d"],
                      wl["resid_sigma"])


def engram_params(wl):
    """fp32 RMSNorm gains (h, k, u) [d] and conv weights [d, conv_k]."""
    d = wl["d"]
    if wl.get("gamma", "ones") == "ones":
        gh = np.ones(d, np.float32)
        gk = np.ones(d, np.float32)
        gu = np.ones(d, np.float32)
    else:
        s = wl["data_seed"]
        gh = 1.0 + normal_f32(s, configs.STREAM_GAMMA_H, np.arange(d), 0.2)
        gk = 1.0 + normal_f32(s, configs.STREAM_GAMMA_K, np.arange(d), 0.2)
        gu = 1.0 + normal_f32(s, configs.STREAM_GAMMA_U, np.arange(d), 0.2)
        gh, gk, gu = (np.float32(g) for g in (gh, gk, gu))
    cw = normal_f32(wl["data_seed"], configs.STREAM_CONV,
                    np.arange(d * wl["conv_k"]), wl["conv_sigma"])
    return (gh.astype(np.float32), gk.astype(np.float32),
            gu.astype(np.float32), cw.reshape(d, wl["conv_k"]))
