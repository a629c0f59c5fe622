"""Device inputs for a workload, and the matching host accessors the oracle
reads. Large tensors are filled on the GPU by the synth generator; the host
recomputes only the elements the oracle touches."""
import numpy as np
import torch

import hashed_head_gram_amd as pg
import synth
from synth import configs, device as sdev


def rel_err(got, want):
    """max_i |got_i - want_i| / max(|want_i|, rms(want)) (0 for empty)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if want.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(want * want))
    den = np.maximum(np.abs(want), rms)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(got - want) / den))


def bf16_to_np(t):
    """bfloat16 tensor -> float64 numpy."""
    return t.float().cpu().numpy().astype(np.float64)


def layout_of(wl):
    d = wl["layout"]
    return pg.make_layout(d["kind"], d["K"], d["r"], S=d["S"], pages=d["pages"],
                          head_rows=d["head_rows"], hash_seed=d["hash_seed"],
                          use_signs=d["use_signs"], n_min=d["n_min"],
                          n_max=d["n_max"], pad_id=wl["canon_vocab"])


def act_torch_dtype(wl):
    return torch.float32 if wl["act_dtype"] == "f32" else torch.bfloat16


class Case:
    """All device tensors of one workload plus oracle-side accessors."""

    def __init__(self, wl, dev="cuda:0", tokens=None, cmap=None, zero_table=False):
        self.wl = wl
        self.dev = torch.device(dev)
        lay = wl["layout"]
        self.lay_d = lay
        self.layout = layout_of(wl)
        self.R = pg.pg_layout_rows(self.layout)
        self.K, self.r = lay["K"], lay["r"]
        self.O = lay["n_max"] - lay["n_min"] + 1
        self.E = self.O * self.K * self.r
        self.W_words = (self.r + 63) // 64
        self.d = wl["d"]
        self.pad = wl["canon_vocab"]
        self.tokens_np = synth.tokens(wl) if tokens is None else np.asarray(tokens, np.int32)
        self.B, self.T = self.tokens_np.shape
        self.N = self.B * self.T
        self.cmap_np = synth.canon_map(wl) if cmap is None else np.asarray(cmap, np.int32)
        self.tokens = torch.from_numpy(self.tokens_np).to(self.dev)
        self.cmap = torch.from_numpy(self.cmap_np).to(self.dev)
        self.zero_table = zero_table
        self.act = act_torch_dtype(wl)
        self.e_dtype = pg.PG_F32 if wl["act_dtype"] == "f32" else pg.PG_BF16
        self._make_table()
        self._make_dense()

    # -- table
    def _make_table(self):
        wl, R, r = self.wl, self.R, self.r
        dt = wl["table_dtype"]
        if dt == "nf4":
            self.codes = torch.empty(R, r // 2, dtype=torch.uint8, device=self.dev)
            self.scales = torch.empty(R, dtype=torch.float16, device=self.dev)
            if self.zero_table:
                self.codes.zero_()
                self.scales.zero_()
            else:
                sdev.fill_nf4_table(self.codes, self.scales, wl["table_seed"])
            self.table = pg.make_table(pg.PG_NF4, self.codes, R, scales=self.scales)
        else:
            tdt = torch.float32 if dt == "f32" else torch.bfloat16
            self.tab = torch.empty(R, r, dtype=tdt, device=self.dev)
            if self.zero_table:
                self.tab.zero_()
            else:
                sdev.fill_normal(self.tab, wl["table_seed"], configs.STREAM_TABLE,
                                 wl["table_sigma"])
            self.table = pg.make_table(pg.PG_F32 if dt == "f32" else pg.PG_BF16,
                                       self.tab, R)

    def fetch(self, rows):
        """Stored values of table rows, for the oracle."""
        rows = np.asarray(rows, dtype=np.int64)
        if self.zero_table:
            n = len(rows)
            if self.wl["table_dtype"] == "nf4":
                return np.zeros((n, self.r // 2), np.uint8), np.zeros(n, np.float16)
            if self.wl["table_dtype"] == "f32":
                return np.zeros((n, self.r), np.float32)
            return np.zeros((n, self.r), np.uint16)
        return synth.table_rows(self.wl, rows)

    # -- projection weights, residual, Engram parameters
    def _make_dense(self):
        wl = self.wl
        d_out = configs.d_out(wl)
        self.W = torch.empty(d_out, self.E, dtype=self.act, device=self.dev)
        sdev.fill_normal(self.W, wl["data_seed"], configs.STREAM_W, wl["w_sigma"])
        self.M = wl.get("M", 1) if wl["gate"] == "engram" else 1
        nres = self.M * self.N if wl["gate"] == "engram" else self.N
        self.resid = torch.empty(nres, self.d, dtype=self.act, device=self.dev)
        sdev.fill_normal(self.resid, wl["data_seed"], configs.STREAM_RESID,
                         wl["resid_sigma"])
        if wl["gate"] == "engram":
            gh, gk, gu, cw = synth.engram_params(wl)
            self.eng_np = (gh, gk, gu, cw)
            self.gh, self.gk, self.gu, self.cw = (torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)
                                                  for a in (gh, gk, gu, cw))
        self._W_np = None

    def W_np(self):
        if self._W_np is None:
            self._W_np = synth.weight(self.wl)
            if self.act == torch.bfloat16:
                self._W_np = synth.bf16_bits_to_f32(self._W_np)
        return self._W_np

    def resid_rows(self, flat):
        v = synth.resid_rows(self.wl, flat)
        return synth.bf16_bits_to_f32(v) if self.act == torch.bfloat16 else v

    def fuse(self, increment_only=0):
        wl = self.wl
        if wl["gate"] == "engram":
            return pg.make_fuse(pg.PG_GATE_ENGRAM, self.e_dtype, self.d, M=self.M,
                                eps=wl["eps"], gamma_h=self.gh, gamma_k=self.gk,
                                gamma_u=self.gu, conv_w=self.cw, conv_k=wl["conv_k"],
                                conv_dil=wl["conv_dil"], increment_only=increment_only)
        return pg.make_fuse(pg.PG_GATE_SCALAR, self.e_dtype, self.d, g=wl["g"],
                            increment_only=increment_only)

    # -- running the library
    def run_index(self):
        N, O, K = self.N, self.O, self.K
        out = dict(
            canon=torch.full((N,), -7, dtype=torch.int32, device=self.dev),
            hashes=torch.zeros(N, O, 1 + K, dtype=torch.int64, device=self.dev),
            rows=torch.zeros(N, O, K, dtype=torch.int64, device=self.dev),
            pages=torch.zeros(N, O, dtype=torch.int64, device=self.dev),
            signs=torch.zeros(N, O, K, self.W_words, dtype=torch.int64, device=self.dev),
            status=torch.zeros(1, dtype=torch.int32, device=self.dev))
        pg.pg_index(self.layout, self.tokens, self.cmap, out["rows"], out["signs"],
                    canon_out=out["canon"], hash_out=out["hashes"],
                    pages_out=out["pages"], dev_status=out["status"])
        return out

    def e_buffer(self):
        return torch.empty(self.N, self.E, dtype=self.act, device=self.dev)

    def run_index_gather(self, status=None):
        e = self.e_buffer()
        pg.pg_index_gather(self.layout, self.table, self.tokens, self.cmap,
                           self.e_dtype, e, dev_status=status)
        return e

    def out_buffer(self):
        n = self.M * self.N if self.wl["gate"] == "engram" else self.N
        return torch.empty(n, self.d, dtype=self.act, device=self.dev)

    def run_forward(self, increment_only=0, resid=None):
        f = self.fuse(increment_only)
        ws = torch.empty(max(pg.pg_workspace_size(self.layout, f, self.B, self.T), 256),
                         dtype=torch.uint8, device=self.dev)
        out = self.out_buffer()
        pg.pg_forward(self.layout, self.table, f, self.tokens, self.cmap, self.W,
                      self.resid if resid is None else resid, out, ws)
        return out

    def run_project(self, e, increment_only=0):
        f = self.fuse(increment_only)
        ws = torch.empty(max(pg.pg_workspace_size(None, f, self.B, self.T), 256),
                         dtype=torch.uint8, device=self.dev)
        out = self.out_buffer()
        pg.pg_project_gate(f, e, self.B, self.T, self.W, self.resid, out, ws)
        return out

    # -- oracle side
    def oracle_scalar(self, positions, with_resid=True):
        import oracle
        x = (lambda p: self.resid_rows(p)) if with_resid else None
        return oracle.forward_scalar(self.lay_d, self.pad, self.tokens_np, self.cmap_np,
                                     self.wl["table_dtype"], self.fetch, self.W_np(),
                                     self.wl["g"], x, positions=positions)

    def oracle_engram(self, positions, with_resid=True):
        import oracle
        gh, gk, gu, cw = self.eng_np
        N = self.N
        cache = {}

        def h(m, flat):
            key = (m, flat)
            if key not in cache:
                cache[key] = self.resid_rows([m * N + flat])[0].astype(np.float64)
            return cache[key]
        return oracle.forward_engram(self.lay_d, self.pad, self.tokens_np, self.cmap_np,
                                     self.wl["table_dtype"], self.fetch, self.W_np(),
                                     self.d, self.M, gh, gk, gu, cw,
                                     self.wl["conv_dil"], self.wl["eps"], h,
                                     positions=positions, with_resid=with_resid)
