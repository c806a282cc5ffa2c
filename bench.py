#!/usr/bin/env python3
"""Decode-step benchmark of the compressed sparse KV attention path on one MI355X.

One step = one decode token for every sequence of the batch through one layer:
index_topk (indexer scores + exact top-512) and attend (gather attention over
the selected c4a entries + the 128-row window, inverse RoPE) for c4a layers;
attend alone (dense over every entry + window) for c128a layers; the 61-layer
workload also compresses each layer's 128 new states first. Inputs are
synthetic, generated on the device, and resident in HBM before timing starts;
caches are built by the library's own compress kernel. Timed steps rotate over
several disjoint input sets so that the 256 MB last-level cache cannot serve
them.

Prints one JSON line: decode tokens/s per layer (whole batch / step time), the
achieved HBM bandwidth of the dominant kernel call against the 8 TB/s peak, and
the CPU oracle's rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4a_128k_bf16",
                    choices=["c4a_128k_bf16", "c128a_1m_bf16", "c4a_1m_fp8_fp4", "mixed61_256k_bf16", "tiny_c4a_2k",
                             "stream_c4a_128k_bf16", "c128a_1m_mixed", "c128a_1m_fp4", "mixed61_256k_reuse"])
    ap.add_argument("--sets", type=int, default=0, help="input sets to rotate over (0 = automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--repeats", type=int, default=10,
                    help="repeats of the K timed steps after the main measurement, for the spread of the step time")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--chunk", type=int, default=0, help="index_topk chunk override")
    ap.add_argument("--splits", type=int, default=0, help="attend splits override")
    ap.add_argument("--graphs", action="store_true",
                    help="replay HIP graphs captured from each input set's calls in the timed steps "
                         "(slower than direct launches on this stack; kept for comparison)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.md from the counter_collection.csv files of a "
                         "FETCH_SIZE run and a WRITE_SIZE run of this bench (with --copy-calibration), then exit")
    return ap.parse_args()


# ------------------------------------------------------------------ workloads

class Workload:
    """Device inputs for one or more sets, a step function and byte accounting."""

    def __init__(self, cfg, args, torch, cskv, sd, synth):
        self.cfg, self.args, self.torch, self.cskv, self.sd, self.synth = cfg, args, torch, cskv, sd, synth
        self.dev = torch.device("cuda:0")

    def key(self, set_i, tensor, layer=0):
        return self.synth.stream_key(self.cfg.seed + 1000 * set_i, tensor, layer)


class C4aLayer(Workload):
    """One c4a layer: index_topk over every entry, then sparse attend."""

    def setup(self, n_sets):
        torch, cskv, sd, s = self.torch, self.cskv, self.sd, self.synth
        c = self.cfg
        B, L, D, H, Di, W = c.B, c.L, c.D, c.H, c.Di, c.W
        N = c.n_entries
        fp8 = c.cache_dtype == "fp8"
        fp4 = c.key_dtype == "fp4"
        self.sets = []
        for i in range(n_sets):
            log(f"setup: c4a input set {i + 1}/{n_sets}")
            st = {}
            cache = torch.empty((B, N, D), dtype=torch.uint8 if fp8 else torch.bfloat16, device=self.dev)
            cscale = torch.empty((B, N), dtype=torch.float32, device=self.dev) if fp8 else None
            win = torch.empty((B, W, D), dtype=torch.uint8 if fp8 else torch.bfloat16, device=self.dev)
            wscale = torch.empty((B, W), dtype=torch.float32, device=self.dev) if fp8 else None
            # the cache is compressed from the states, one sequence at a time (bounded scratch)
            for b in range(B):
                S = torch.empty((1, L, D), dtype=torch.bfloat16, device=self.dev)
                g = torch.empty((1, L), dtype=torch.float32, device=self.dev)
                sd.fill(S, s.KIND_NORMAL_BF16, self.key(i, s.T_S), offset=b * L * D)
                sd.fill(g, s.KIND_NORMAL_F32, self.key(i, s.T_GATE), offset=b * L)
                cskv.compress("c4a", S, g, cache[b:b + 1], None if cscale is None else cscale[b:b + 1])
                tail = S[0, L - W:].contiguous()
                if fp8:
                    wc, ws_ = cskv.encode_fp8_rows(tail)
                    win[b].copy_(wc)
                    wscale[b].copy_(ws_)
                else:
                    win[b].copy_(tail)
                del S, g
            if fp4:
                kidx = sd.new((B, N, Di // 2), s.KIND_BYTES, self.key(i, s.T_KIDX), device=self.dev)
                kscale = sd.new((B, N, Di // 16), s.KIND_POW2_E4M3, self.key(i, s.T_KIDX_SCALE), device=self.dev,
                                emin=-2, emax=2)
            else:
                kidx = sd.new((B, N, Di), s.KIND_INT_BF16, self.key(i, s.T_KIDX), device=self.dev, a=c.idx_range)
                kscale = None
            st.update(cache=cache, cscale=cscale, win=win, wscale=wscale, kidx=kidx, kscale=kscale,
                      qidx=sd.new((B, Di), s.KIND_INT_BF16, self.key(i, s.T_QIDX), device=self.dev, a=c.idx_range),
                      Q=sd.new((B, H, D), s.KIND_NORMAL_BF16, self.key(i, s.T_Q), device=self.dev),
                      ids=torch.empty((B, c.k), dtype=torch.int32, device=self.dev),
                      O=torch.empty((B, H, D), dtype=torch.float32, device=self.dev),
                      pos=torch.full((B,), c.q_pos, dtype=torch.int64, device=self.dev))
            self.sets.append(st)
        torch.cuda.synchronize()

    def dominant(self, st):
        self.cskv.index_topk(st["qidx"], st["kidx"], self.cfg.k, k_scale=st["kscale"], ids=st["ids"],
                             chunk=self.args.chunk)

    def rest(self, st):
        c = self.cfg
        self.cskv.attend(st["Q"], st["cache"], st["ids"], st["win"], cache_scale=st["cscale"],
                         window_scale=st["wscale"], softmax_scale=c.tau, rope_dims=c.R, rope_base=c.rope_base,
                         q_pos=st["pos"], out=st["O"], splits=self.args.splits)

    def bytes(self):
        c = self.cfg
        N = c.n_entries
        key_b = (c.Di // 2 + c.Di // 16) if c.key_dtype == "fp4" else c.Di * 2
        row_b = (c.D + 4) if c.cache_dtype == "fp8" else c.D * 2
        dom = c.B * (N * key_b + c.Di * 2 + c.k * 4)
        rest = c.B * ((c.k + c.W) * row_b + c.k * 4 + c.H * c.D * 2 + c.H * c.D * 4)
        return dom, rest

    def flops(self):
        c = self.cfg
        return c.B * (2 * c.n_entries * c.Di + 4 * c.H * c.D * (c.k + c.W))


class C128aLayer(Workload):
    """One c128a layer: dense attend over every entry plus the window."""

    def setup(self, n_sets):
        torch, cskv, sd, s = self.torch, self.cskv, self.sd, self.synth
        c = self.cfg
        B, L, D, H, W = c.B, c.L, c.D, c.H, c.W
        N = c.n_entries
        self.sets = []
        for i in range(n_sets):
            log(f"setup: c128a input set {i + 1}/{n_sets}")
            mixed = c.cache_dtype == "mixed"   # 448 fp8 codes + 64 bf16 rotary channels per row
            if mixed:
                cache = torch.empty((B, N, D + cskv.MIX_ROPE), dtype=torch.uint8, device=self.dev)
                cscale = torch.empty((B, N), dtype=torch.float32, device=self.dev)
            elif c.cache_dtype == "fp4":        # E2M1 codes + one E4M3 scale byte per 16 channels
                cache = torch.empty((B, N, D // 2 + D // 16), dtype=torch.uint8, device=self.dev)
                cscale = None
            else:
                cache = torch.empty((B, N, D), dtype=torch.bfloat16, device=self.dev)
                cscale = None
            win = torch.empty((B, W, D), dtype=torch.bfloat16, device=self.dev)
            for b in range(B):
                S = torch.empty((1, L, D), dtype=torch.bfloat16, device=self.dev)
                g = torch.empty((1, L), dtype=torch.float32, device=self.dev)
                sd.fill(S, s.KIND_NORMAL_BF16, self.key(i, s.T_S), offset=b * L * D)
                sd.fill(g, s.KIND_NORMAL_F32, self.key(i, s.T_GATE), offset=b * L)
                cskv.compress("c128a", S, g, cache[b:b + 1], None if cscale is None else cscale[b:b + 1])
                win[b].copy_(S[0, L - W:])
                del S, g
            self.sets.append(dict(cache=cache, cscale=cscale, win=win,
                                  Q=sd.new((B, H, D), s.KIND_NORMAL_BF16, self.key(i, s.T_Q), device=self.dev),
                                  O=torch.empty((B, H, D), dtype=torch.float32, device=self.dev),
                                  pos=torch.full((B,), c.q_pos, dtype=torch.int64, device=self.dev)))
        torch.cuda.synchronize()

    def dominant(self, st):
        c = self.cfg
        self.cskv.attend(st["Q"], st["cache"], None, st["win"], cache_scale=st["cscale"], softmax_scale=c.tau,
                         rope_dims=c.R, rope_base=c.rope_base, q_pos=st["pos"], out=st["O"], splits=self.args.splits)

    def rest(self, st):
        pass

    def bytes(self):
        c = self.cfg
        row = {"mixed": (c.D - 64) + 2 * 64 + 4, "fp4": c.D // 2 + c.D // 16}.get(c.cache_dtype, c.D * 2)
        return c.B * (c.n_entries * row + c.W * c.D * 2 + c.H * c.D * 2 + c.H * c.D * 4), 0

    def flops(self):
        c = self.cfg
        return c.B * 4 * c.H * c.D * (c.n_entries + c.W)


class Mixed61(Workload):
    """61 layers (c128a on even, c4a on odd): per layer compress 128 new states
    into the cache, then (c4a) index_topk, then attend."""

    def setup(self, n_sets):
        torch, cskv, sd, s = self.torch, self.cskv, self.sd, self.synth
        c = self.cfg
        B, L, D, H, W, Di = c.B, c.L, c.D, c.H, c.W, c.Di
        from synth.configs import c128a_entries, c4a_entries
        self.N4, self.N128 = c4a_entries(L), c128a_entries(L)
        self.layers = []
        i = 0
        for layer in range(c.layers):
            if layer % 10 == 0:
                log(f"setup: layer {layer + 1}/{c.layers}")
            kind = c.layer_kind(layer)
            lay = {"kind": kind}
            span_T = 132 if kind == "c4a" else 128
            lay["span"] = sd.new((B, span_T, D), s.KIND_NORMAL_BF16, self.key(i, s.T_S, layer), device=self.dev)
            lay["gate"] = sd.new((B, span_T), s.KIND_NORMAL_F32, self.key(i, s.T_GATE, layer), device=self.dev)
            lay["Q"] = sd.new((B, H, D), s.KIND_NORMAL_BF16, self.key(i, s.T_Q, layer), device=self.dev)
            lay["O"] = torch.empty((B, H, D), dtype=torch.float32, device=self.dev)
            if kind == "c4a":
                lay["cache"] = sd.new((B, self.N4, D), s.KIND_NORMAL_BF16, self.key(i, s.T_CACHE, layer), device=self.dev)
                lay["reuse"] = c.reuses(layer)
                if lay["reuse"] is None:   # a layer that reuses ids has no indexer of its own
                    lay["kidx"] = sd.new((B, self.N4, Di), s.KIND_INT_BF16, self.key(i, s.T_KIDX, layer),
                                         device=self.dev, a=c.idx_range)
                    lay["qidx"] = sd.new((B, Di), s.KIND_INT_BF16, self.key(i, s.T_QIDX, layer), device=self.dev,
                                         a=c.idx_range)
                    lay["ids"] = torch.empty((B, c.k), dtype=torch.int32, device=self.dev)
                lay["first"] = (L - 132) // 4
                lay["win"] = lay["span"][:, 4:, :]
            else:
                lay["cache"] = sd.new((B, self.N128, D), s.KIND_NORMAL_BF16, self.key(i, s.T_CACHE, layer),
                                      device=self.dev)
                lay["first"] = L // 128 - 1
                lay["win"] = lay["span"]
            self.layers.append(lay)
        self.pos = torch.full((B,), c.q_pos, dtype=torch.int64, device=self.dev)
        self.sets = [None]
        torch.cuda.synchronize()

    def step_layers(self):
        c, cskv = self.cfg, self.cskv
        for lay in self.layers:
            cskv.compress(lay["kind"], lay["span"], lay["gate"], lay["cache"], first_entry=lay["first"])
            if lay["kind"] == "c4a":
                if lay["reuse"] is None:
                    cskv.index_topk(lay["qidx"], lay["kidx"], c.k, ids=lay["ids"], chunk=self.args.chunk)
                    ids = lay["ids"]
                else:
                    ids = self.layers[lay["reuse"]]["ids"]   # computed earlier in this step
            else:
                ids = None
            cskv.attend(lay["Q"], lay["cache"], ids, lay["win"], softmax_scale=c.tau, rope_dims=c.R,
                        rope_base=c.rope_base, q_pos=self.pos, out=lay["O"], splits=self.args.splits)

    def dominant_layers(self):
        # the index calls of the c4a layers alone (the dominant call's timing pass)
        c = self.cfg
        for lay in self.layers:
            if lay["kind"] == "c4a" and lay["reuse"] is None:
                self.cskv.index_topk(lay["qidx"], lay["kidx"], c.k, ids=lay["ids"], chunk=self.args.chunk)

    def step(self, i, dominant_only=False):
        if dominant_only:
            self.dominant_layers()
        else:
            self.step_layers()

    def n_dominant(self):
        """Index calls per step (c4a layers that do not reuse another's ids)."""
        c = self.cfg
        return sum(1 for l in range(c.layers) if c.layer_kind(l) == "c4a" and c.reuses(l) is None)

    def bytes(self):
        c = self.cfg
        n4 = sum(1 for l in range(c.layers) if c.layer_kind(l) == "c4a")
        n128 = c.layers - n4
        dom = self.n_dominant() * c.B * (self.N4 * c.Di * 2 + c.Di * 2 + c.k * 4)
        qo = c.H * c.D * 6
        c4_rest = c.B * (132 * c.D * 2 + 132 * 4 + 32 * c.D * 2 + (c.k + c.W) * c.D * 2 + c.k * 4 + qo)
        c128 = c.B * (128 * c.D * 2 + 128 * 4 + c.D * 2 + (self.N128 + c.W) * c.D * 2 + qo)
        return dom, n4 * c4_rest + n128 * c128

    def flops(self):
        c = self.cfg
        n4 = sum(1 for l in range(c.layers) if c.layer_kind(l) == "c4a")
        n128 = c.layers - n4
        return c.B * (self.n_dominant() * 2 * self.N4 * c.Di + n4 * 4 * c.H * c.D * (c.k + c.W) +
                      n128 * 4 * c.H * c.D * (self.N128 + c.W))


class StreamC4a(Workload):
    """Streaming c4a decode of a ragged batch: every step appends one new state
    per sequence (cskv_append: ring write, an entry every 4 tokens), then
    index_topk over the per-sequence entry counts and attend over the selected
    entries plus the ring as window. The state carries over from step to step,
    so there is one input set; prefix caches, indexer keys and rings are drawn
    directly (their contents do not change the work)."""

    N_TOKENS = 8     # distinct new-state sets cycled through

    def setup(self, n_sets):
        torch, sd, s = self.torch, self.sd, self.synth
        c = self.cfg
        B, L, D, H, Di, W = c.B, c.L, c.D, c.H, c.Di, c.W
        from synth.configs import c4a_entries
        # warmup, the timed steps, then their repeats for the spread of the step time
        self.n_steps = self.args.warmup + self.args.steps * (1 + self.args.repeats)
        self.rows = c4a_entries(L + self.n_steps) + 1
        log(f"setup: stream caches ({B} x {self.rows} entries)")
        self.cache = sd.new((B, self.rows, D), s.KIND_NORMAL_BF16, self.key(0, s.T_CACHE), device=self.dev)
        self.kidx = sd.new((B, self.rows, Di), s.KIND_INT_BF16, self.key(0, s.T_KIDX), device=self.dev,
                           a=c.idx_range)
        self.qidx = sd.new((B, Di), s.KIND_INT_BF16, self.key(0, s.T_QIDX), device=self.dev, a=c.idx_range)
        self.Q = sd.new((B, H, D), s.KIND_NORMAL_BF16, self.key(0, s.T_Q), device=self.dev)
        self.ring = sd.new((B, W, D), s.KIND_NORMAL_BF16, self.key(0, s.T_WIN), device=self.dev)
        self.ring_gate = sd.new((B, W), s.KIND_NORMAL_F32, self.key(0, s.T_MISC), device=self.dev)
        self.s_new = sd.new((self.N_TOKENS, B, D), s.KIND_NORMAL_BF16, self.key(0, s.T_S), device=self.dev)
        self.g_new = sd.new((self.N_TOKENS, B), s.KIND_NORMAL_F32, self.key(0, s.T_GATE), device=self.dev)
        # step t appends token L - lag_b + t of sequence b
        lag = torch.tensor([c.stream_lag(b) for b in range(B)], dtype=torch.int64)
        self.pos = (L - lag[None, :] + torch.arange(self.n_steps, dtype=torch.int64)[:, None]).to(self.dev)
        self.n_entries = torch.zeros((B,), dtype=torch.int32, device=self.dev)
        self.n_window = torch.zeros((B,), dtype=torch.int32, device=self.dev)
        self.ids = torch.empty((B, c.k), dtype=torch.int32, device=self.dev)
        self.O = torch.empty((B, H, D), dtype=torch.float32, device=self.dev)
        self.sets = [None]
        self.t = 0
        torch.cuda.synchronize()

    def step(self, i, dominant_only=False):
        c, cskv = self.cfg, self.cskv
        if dominant_only:
            cskv.index_topk(self.qidx, self.kidx, c.k, n_entries=self.n_entries, ids=self.ids, chunk=self.args.chunk)
            return
        t = self.t
        if t >= self.n_steps:
            raise RuntimeError("stream workload: more steps than planned")
        self.t += 1
        j = t % self.N_TOKENS
        cskv.append("c4a", self.s_new[j], self.g_new[j], self.pos[t], self.ring, self.ring_gate, self.cache,
                    n_entries=self.n_entries, n_window=self.n_window)
        cskv.index_topk(self.qidx, self.kidx, c.k, n_entries=self.n_entries, ids=self.ids, chunk=self.args.chunk)
        cskv.attend(self.Q, self.cache, self.ids, self.ring, softmax_scale=c.tau, rope_dims=c.R,
                    rope_base=c.rope_base, q_pos=self.pos[t], n_window=self.n_window, out=self.O,
                    splits=self.args.splits)

    def bytes(self):
        c = self.cfg
        from synth.configs import c4a_entries
        # entries at the start of the timed steps (they grow by one per 4 steps)
        n = sum(c4a_entries(c.L - c.stream_lag(b)) for b in range(c.B))
        dom = n * c.Di * 2 + c.B * (c.Di * 2 + c.k * 4)
        # append: new state read + ring write (+ gate), and a quarter of the
        # 8-state folds and entry writes; attend: k + W rows, Q and O
        app = c.B * (2 * c.D * 2 + 8 + (8 * c.D * 2 + c.D * 2) // 4)
        att = c.B * ((c.k + c.W) * c.D * 2 + c.k * 4 + c.H * c.D * 6)
        return dom, app + att

    def flops(self):
        c = self.cfg
        return c.B * (2 * c.n_entries * c.Di + 4 * c.H * c.D * (c.k + c.W))


# ------------------------------------------------------------------ CPU oracle baseline

def cpu_baseline(cfg, seconds):
    """The oracle, as it is, on a bounded sample of the same workload: a few
    sequences of one layer (inputs regenerated on the host, outside the timed
    region), run repeatedly for about `seconds`. Returns a dict for the JSON."""
    import numpy as np
    import synth
    from oracle import formats as F
    from oracle import method as M
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    kind = cfg.layer_kind(1) if cfg.kind in ("mixed", "stream") else cfg.kind
    from synth.configs import c128a_entries, c4a_entries
    N = c4a_entries(cfg.L) if kind == "c4a" else c128a_entries(cfg.L)
    n_seq = 2
    seqs = []
    for b in range(n_seq):
        key = lambda t: synth.stream_key(cfg.seed, t, 1)  # noqa: E731
        Q = F.bf16_to_f64(synth.normal_bf16(key(synth.T_Q), b * cfg.H * cfg.D, cfg.H * cfg.D).reshape(cfg.H, cfg.D))
        win = F.bf16_to_f64(synth.normal_bf16(key(synth.T_WIN), b * cfg.W * cfg.D, cfg.W * cfg.D).reshape(cfg.W, cfg.D))
        # only the rows a query can read are filled: every row for c128a, the
        # rows the oracle's own top-k picks for c4a (filled after selection)
        cache = np.zeros((N, cfg.D), dtype=np.float64)
        st = {"Q": Q, "win": win, "cache": cache, "ring": win.copy(), "ring_gate": np.zeros(cfg.W)}
        if kind == "c4a":
            st["qidx"] = F.bf16_to_f64(synth.int_bf16(key(synth.T_QIDX), b * cfg.Di, cfg.Di, cfg.idx_range))
            if cfg.key_dtype == "fp4":
                codes = synth.random_bytes(key(synth.T_KIDX), b * N * cfg.Di // 2, N * cfg.Di // 2).reshape(N, cfg.Di // 2)
                sc = synth.pow2_e4m3(key(synth.T_KIDX_SCALE), b * N * cfg.Di // 16, N * cfg.Di // 16, -2, 2
                                     ).reshape(N, cfg.Di // 16)
                st["kidx_codes"], st["kidx_scales"] = codes, sc
            else:
                st["kidx"] = F.bf16_to_f64(synth.int_bf16(key(synth.T_KIDX), b * N * cfg.Di, N * cfg.Di,
                                                          cfg.idx_range).reshape(N, cfg.Di))
            ids = M.topk_ids(M.index_scores(st["qidx"], st["kidx"] if "kidx" in st else
                                            F.decode_fp4_g16(st["kidx_codes"], st["kidx_scales"])), cfg.k)
            rows = ids[ids >= 0]
        else:
            rows = np.arange(N)
        cache[rows] = F.bf16_to_f64(synth.normal_bf16(key(synth.T_CACHE), 0, rows.size * cfg.D)
                                    .reshape(rows.size, cfg.D))
        seqs.append(st)

    def one(st):
        if cfg.kind == "stream":
            # the step's append first (token L-1 completes an entry: the 8-state fold)
            M.append("c4a", st["ring"], st["ring_gate"], st["win"][0], 0.0, cfg.L - 1)
        if kind == "c4a":
            keys = st["kidx"] if "kidx" in st else F.decode_fp4_g16(st["kidx_codes"], st["kidx_scales"])
            M.c4a_decode(st["Q"], st["qidx"], keys, st["cache"], st["win"], cfg.k, cfg.tau, cfg.R,
                         cfg.rope_base, cfg.q_pos)
        else:
            M.c128a_decode(st["Q"], st["cache"], st["win"], cfg.tau, cfg.R, cfg.rope_base, cfg.q_pos)

    def timed(limit):
        done = 0
        t0 = time.perf_counter()
        while True:
            one(seqs[done % n_seq])
            done += 1
            el = time.perf_counter() - t0
            if el >= limit:
                return done, el

    done, el = timed(seconds)
    out = {"value": done / el, "unit": "decode tokens/s per layer", "cores": int(cores), "kind": "oracle",
           "sample": f"{done} single-sequence {kind} layer decodes ({n_seq} distinct sequences of the "
                     f"{cfg.name} workload, inputs generated before timing) in {el:.1f} s",
           "nproc": os.cpu_count(), "cpu_model": _cpu_model()}
    # a per-core rate: the same sample with the BLAS pool held to one thread
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            d1, e1 = timed(max(seconds / 4, 1.0))
        out["one_thread"] = {"value": d1 / e1, "sample": f"{d1} decodes in {e1:.1f} s"}
    except Exception as e:   # no thread control: report without it
        out["one_thread"] = {"value": None, "sample": f"not measured ({type(e).__name__})"}
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ------------------------------------------------------------------ HBM traffic from counters
#
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read for
# the 1 GiB device copy that --copy-calibration adds, so that the figure is in
# bytes that actually crossed the HBM interface. The summary records a digest of
# the kernel sources; the bench reports the figure only while that digest still
# matches, since a changed kernel makes old counters meaningless.

CSRC = os.path.join(ROOT, "compressed_sparse_kv_compress_amd", "csrc")
COPY_BYTES = 1 << 30


def dominant_kernels(kind):
    return ("k_index_score", "k_topk_final") if kind != "c128a" else ("k_attend", "k_attend_merge")


def kernel_source_digest():
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.md")


def summarize_traffic(cfg, fetch_csv, write_csv):
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        vals = defaultdict(list)
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    name = r["Kernel_Name"].split("(")[0].replace("void ", "").strip()
                    vals[name].append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    copy = "__amd_rocclr_copyBuffer"
    # the 1 GiB copy is the dispatch with the largest reading among copyBuffer dispatches
    f_scale = COPY_BYTES / (max(fetch[copy]) * 1024.0)
    w_scale = COPY_BYTES / (max(write[copy]) * 1024.0)
    dom = dominant_kernels(cfg.kind)
    rows, total = [], 0.0
    for name in sorted(set(fetch) | set(write)):
        if not name.startswith("cskv::"):
            continue
        fk = sum(fetch.get(name, [0])) / max(1, len(fetch.get(name, [])))
        wk = sum(write.get(name, [0])) / max(1, len(write.get(name, [])))
        fb, wb = fk * 1024 * f_scale, wk * 1024 * w_scale
        is_dom = name.split("<")[0].split("::")[-1] in dom
        if is_dom:
            total += fb + wb
        rows.append((name, len(fetch.get(name, [])), fk, wk, fb, wb, is_dom))
    lines = [
        f"# HBM traffic per dispatch: {cfg.name}",
        "",
        "Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged over the run's dispatches),",
        "each from its own rocprofv3 --pmc run of `python3 bench.py --workload "
        f"{cfg.name} --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration`, scaled by the",
        f"reading for the 1 GiB device copy: FETCH_SIZE x {f_scale:.4f}, WRITE_SIZE x {w_scale:.4f}.",
        "",
        "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | written bytes | dominant call |",
        "|---|---|---|---|---|---|---|",
    ]
    for name, n, fk, wk, fb, wb, d in rows:
        lines.append(f"| {name} | {n} | {fk:.1f} | {wk:.1f} | {fb:.4g} | {wb:.4g} | {'yes' if d else ''} |")
    lines += [
        "",
        f"traffic_bytes_per_dominant_call: {int(total)}",
        f"kernel_source_digest: {kernel_source_digest()}",
        "",
    ]
    with open(traffic_path(cfg.name), "w") as f:
        f.write("\n".join(lines))
    log(f"wrote {traffic_path(cfg.name)}: {int(total)} bytes per dominant call")


def recorded_traffic(workload):
    """Counter-measured bytes per dominant call, or None when absent or stale."""
    try:
        with open(traffic_path(workload)) as f:
            text = f.read()
    except OSError:
        return None
    kv = dict(l.split(": ", 1) for l in text.splitlines() if l.startswith(("traffic_bytes", "kernel_source")))
    if kv.get("kernel_source_digest") != kernel_source_digest():
        return None
    return int(kv["traffic_bytes_per_dominant_call"])


# ------------------------------------------------------------------ main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path shards by "
              "sequence with no communication, so N GPUs run N independent copies)", file=sys.stderr)
        sys.exit(2)
    from synth import configs
    cfg = configs.BY_NAME[args.workload]
    if args.summarize_traffic:
        summarize_traffic(cfg, *args.summarize_traffic)
        return

    import torch

    import compressed_sparse_kv_compress_amd as cskv
    import synth
    from synth import device as sd

    cls = {"c4a": C4aLayer, "c128a": C128aLayer, "mixed": Mixed61, "stream": StreamC4a}[cfg.kind]
    wl = cls(cfg, args, torch, cskv, sd, synth)
    stateful = cfg.kind in ("mixed", "stream")   # steps that carry state: no input-set rotation, no graphs
    n_sets = args.sets or (1 if stateful else 4)
    t_setup = time.perf_counter()
    wl.setup(n_sets)
    setup_s = time.perf_counter() - t_setup

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    mixed = cfg.kind == "mixed"
    n4 = wl.n_dominant() if mixed else 1
    for i in range(args.warmup):
        if stateful:
            wl.step(i)
        else:
            st = wl.sets[i % n_sets]
            wl.dominant(st)
            wl.rest(st)
    torch.cuda.synchronize()
    # Optionally the calls of each input set are captured once into HIP graphs
    # (the dominant call in a graph of its own, so that its duration is timed on
    # the launch stream) and replayed.
    graphs = None
    if not stateful and args.graphs:
        graphs = []
        for st in wl.sets:
            g_dom, g_rest = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_dom):
                wl.dominant(st)
            with torch.cuda.graph(g_rest):
                wl.rest(st)
            graphs.append((g_dom, g_rest))
        for i in range(max(1, args.warmup)):
            g_dom, g_rest = graphs[i % n_sets]
            g_dom.replay()
            g_rest.replay()
        torch.cuda.synchronize()
    log(f"setup {setup_s:.1f} s, warmup done; timing {args.steps} steps "
        f"({'eager launches' if graphs is None else 'HIP graph replays'})")

    def run_step(i, dominant_only=False):
        if stateful:
            wl.step(i, dominant_only)
            return
        if graphs is not None:
            g_dom, g_rest = graphs[i % n_sets]
            dom, rest = g_dom.replay, g_rest.replay
        else:
            st = wl.sets[i % n_sets]
            dom, rest = (lambda: wl.dominant(st)), (lambda: wl.rest(st))
        dom()
        if not dominant_only:
            rest()

    # the timed region: K steps bracketed by two events only (an event record
    # between kernels costs the stream several microseconds)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        run_step(i)
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    # the dominant call's duration: the dominant calls of K more steps issued
    # back to back (same input-set rotation), bracketed by two events on the
    # stream the kernels are launched on, so that no event record sits between
    # its kernels and the next call's
    start.record()
    for i in range(args.steps):
        run_step(i, dominant_only=True)
    end.record()
    torch.cuda.synchronize()
    dom_ms = start.elapsed_time(end) / (args.steps * n4)

    # spread of the step time: the K timed steps repeated, each repeat between
    # two events as above (a stateful workload continues its stream)
    rep_ms = []
    for r in range(args.repeats):
        start.record()
        for i in range(args.steps):
            run_step(args.steps * (1 + r) + i if stateful else i)
        end.record()
        torch.cuda.synchronize()
        rep_ms.append(start.elapsed_time(end) / args.steps)

    dom_bytes, rest_bytes = wl.bytes()
    dom_bytes_launch = dom_bytes / n4
    achieved = dom_bytes_launch / (dom_ms * 1e-3) / 1e9
    tokens = cfg.B / (ms_step * 1e-3)
    if mixed:
        metric = "decode tokens/s per 61-layer step"
    else:
        metric = "decode tokens/s per layer"
    out = {
        "metric": metric,
        "value": round(tokens, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if cfg.cache_dtype == "bf16" and cfg.key_dtype == "bf16" else
                  "fp8 + bf16 rotary (bf16 MFMA, fp32 accumulate)" if cfg.cache_dtype == "mixed" else
                  "fp4 E2M1 + E4M3/16 (bf16 MFMA, fp32 accumulate)" if cfg.cache_dtype == "fp4" else
                  "fp8+fp4 (bf16 MFMA, fp32 accumulate)"),
        "data": "synthetic (SplitMix64 streams; caches built by the library's compress kernel)" if not stateful
                else "synthetic (SplitMix64 streams; prefix caches drawn directly, new states compressed in the step)",
        "config": {"workload": cfg.name, "batch": cfg.B, "context": cfg.L, "heads": cfg.H, "D": cfg.D,
                   "rotary": cfg.R, "window": cfg.W, "top_k": cfg.k or None, "indexer_dim": cfg.Di or None,
                   "cache": cfg.cache_dtype, "indexer_keys": cfg.key_dtype if cfg.k else None,
                   "layers": cfg.layers, "input_sets_rotated": n_sets,
                   **({"ragged_context": f"{cfg.L} - (0..127)", "append": "one state per sequence per step"}
                      if cfg.kind == "stream" else {}),
                   "launch": "eager" if graphs is None else "hip_graph"},
        "roofline": {
            "bound": "hbm",
            "kernel": "index_topk (k_index_score + k_topk_final)" if (cfg.kind != "c128a") else
                      "attend (k_attend + k_attend_merge)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(cfg.name),
            "algorithmic_bytes_per_launch": int(dom_bytes_launch),
            "avg_launch_ms": round(dom_ms, 5),
        },
        "step_bandwidth_gbs": round((dom_bytes + rest_bytes) / (ms_step * 1e-3) / 1e9, 1),
        "algorithmic_bytes_per_step": int(dom_bytes + rest_bytes),
        "tflops_per_s": round(wl.flops() / (ms_step * 1e-3) / 1e12, 2),
        "setup_s": round(setup_s, 1),
    }
    if rep_ms:
        import numpy as np
        out["step_ms_spread"] = {
            "repeats": len(rep_ms),
            "median": round(float(np.percentile(rep_ms, 50)), 5),
            "p10": round(float(np.percentile(rep_ms, 10)), 5),
            "p90": round(float(np.percentile(rep_ms, 90)), 5),
            "of": f"ms per step of each repeat of the {args.steps} timed steps, after the timed region",
        }
    # what a plain read stream reaches on this machine: torch's max over 1 GiB viewed
    # as int64 (a reduction that only reads), after the timed steps, median of 5
    probe = torch.ones(1 << 27, dtype=torch.int64, device="cuda")
    probe.amax()
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        probe.amax()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del probe
    probe_gbs = (1 << 30) / (sorted(times)[2] * 1e-3) / 1e9
    out["hbm_probe"] = {"read_gbs": round(probe_gbs, 1),
                        "kind": "torch amax over 1 GiB of int64 (read-only stream), median of 5"}
    out["roofline"]["frac_of_probe"] = round(achieved / probe_gbs, 4)
    log(f"timed: {ms_step:.4f} ms/step")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
        if mixed:
            # the oracle sample is one c4a layer; a 61-layer step costs about 61 of them
            out["cpu_baseline"]["value"] /= cfg.layers
            if out["cpu_baseline"]["one_thread"]["value"]:
                out["cpu_baseline"]["one_thread"]["value"] /= cfg.layers
            out["cpu_baseline"]["unit"] = "decode tokens/s per 61-layer step (sampled c4a layer rate / 61)"
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
