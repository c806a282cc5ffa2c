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

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: at least 5; for workloads whose steps carry no state, "
                         "as many more as run 25 ms, so that the GPU clock has settled before the timed steps)")
    ap.add_argument("--workload", default=None,
                    choices=["c4a_128k_bf16", "c128a_1m_bf16", "c4a_1m_fp8_fp4", "mixed61_256k_bf16", "tiny_c4a_2k",
                             "stream_c4a_128k_bf16", "c128a_1m_mixed", "c128a_1m_fp4", "mixed61_256k_reuse"])
    ap.add_argument("--sets", type=int, default=0, help="input sets to rotate over (0 = automatic)")
    ap.add_argument("--no-extra", action="store_true",
                    help="without --workload: measure the headline workload only, not the 1M and 61-layer ones")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="parallel oracle time per workload (the one-thread rate takes a quarter of it more)")
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

def _host(t):
    """A device tensor's bytes on the host: bf16 as uint16 bit patterns."""
    if t is None:
        return None
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


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
                      pos=torch.full((B,), c.q_pos, dtype=torch.int64, device=self.dev),
                      part=torch.empty((cskv.partial_bytes(B, H, D) // 4,), dtype=torch.float32, device=self.dev))
            self.sets.append(st)
        # the overlapped step: the window partial on a second stream (default
        # priority) while the indexer runs on the launch stream
        self.side = torch.cuda.Stream()
        self.ev_ready, self.ev_done = torch.cuda.Event(), torch.cuda.Event()
        torch.cuda.synchronize()

    def dominant(self, st):
        self.cskv.index_topk(st["qidx"], st["kidx"], self.cfg.k, k_scale=st["kscale"], ids=st["ids"],
                             chunk=self.args.chunk)

    def overlapped(self, st):
        """One step with the window-only partial computed on the side stream
        during index_topk, merged by the attend over the selected entries."""
        torch, c = self.torch, self.cfg
        main = torch.cuda.current_stream()
        self.ev_ready.record(main)
        with torch.cuda.stream(self.side):
            self.side.wait_event(self.ev_ready)
            self.cskv.attend_window_partial(st["Q"], st["win"], window_scale=st["wscale"], softmax_scale=c.tau,
                                            out=st["part"])
            self.ev_done.record(self.side)
        self.dominant(st)
        main.wait_event(self.ev_done)
        self.cskv.attend(st["Q"], st["cache"], st["ids"], None, cache_scale=st["cscale"], softmax_scale=c.tau,
                         rope_dims=c.R, rope_base=c.rope_base, q_pos=st["pos"], out=st["O"],
                         splits=self.args.splits, partial=st["part"])

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


    def cpu_groups(self):
        c, st = self.cfg, self.sets[0]
        fp8, fp4 = c.cache_dtype == "fp8", c.key_dtype == "fp4"
        h = {"Q": _host(st["Q"]), "qidx": _host(st["qidx"]), "cache": _host(st["cache"]), "win": _host(st["win"]),
             "cache_fmt": "fp8" if fp8 else "bf16", "win_fmt": "fp8" if fp8 else "bf16",
             "cscale": _host(st["cscale"]), "wscale": _host(st["wscale"]),
             "key_fmt": "fp4" if fp4 else "bf16", "k": c.k, "D": c.D, "tau": c.tau, "R": c.R,
             "base": c.rope_base, "pos": c.q_pos}
        if fp4:
            h["kcodes"], h["kscale"] = _host(st["kidx"]), _host(st["kscale"])
        else:
            h["kidx"] = _host(st["kidx"])
        _CPU.clear()
        _CPU["main"] = h
        return [("c4a", [("c4a", b) for b in range(c.B)], 1)]

    def cpu_inputs_note(self):
        return (f"input set 0 as the GPU consumed it (indexer keys, {self.cfg.cache_dtype} cache built by the "
                f"library's compress, window, Q), all {self.cfg.B} sequences")


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


    def cpu_groups(self):
        c, st = self.cfg, self.sets[0]
        h = {"Q": _host(st["Q"]), "cache": _host(st["cache"]), "win": _host(st["win"]), "cscale": _host(st["cscale"]),
             "cache_fmt": c.cache_dtype, "win_fmt": "bf16", "N": c.n_entries, "D": c.D, "tau": c.tau, "R": c.R,
             "base": c.rope_base, "pos": c.q_pos}
        _CPU.clear()
        _CPU["main"] = h
        return [("c128a", [("c128a", b) for b in range(c.B)], 1)]

    def cpu_inputs_note(self):
        return (f"input set 0 as the GPU consumed it ({self.cfg.cache_dtype} cache built by the library's compress, "
                f"window, Q), all {self.cfg.B} sequences")


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
        for layer in (c.only_layers or range(c.layers)):
            if layer % 10 == 0:
                log(f"setup: layer {layer + 1}/{c.layers}")
            kind = c.layer_kind(layer)
            lay = {"kind": kind, "layer": layer}
            if c.only_layers and c.reuses(layer) is not None:
                raise ValueError("a subset of layers cannot include one that reuses another layer's ids")
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


    SAMPLE_LAYERS = (0, 1, 59, 60)

    def cpu_groups(self):
        c = self.cfg
        _CPU.clear()
        g128, g4 = [], []
        for layer in self.SAMPLE_LAYERS:
            lay = self.layers[layer]
            h = {"Q": _host(lay["Q"]), "span": _host(lay["span"]), "gate": _host(lay["gate"]),
                 "cache": _host(lay["cache"]), "first": lay["first"], "D": c.D, "k": c.k, "tau": c.tau, "R": c.R,
                 "base": c.rope_base, "pos": c.q_pos, "key_fmt": "bf16"}
            key = f"L{layer}"
            if lay["kind"] == "c4a":
                if lay.get("reuse") is None:
                    h["kidx"], h["qidx"] = _host(lay["kidx"]), _host(lay["qidx"])
                else:   # a layer that reuses another's ids attends over them
                    h["kidx"], h["ids"] = None, _host(self.layers[lay["reuse"]]["ids"])
                g4 += [("m4", b, key) for b in range(c.B)]
            else:
                g128 += [("m128", b, key) for b in range(c.B)]
            _CPU[key] = h
        n4 = sum(1 for l in range(c.layers) if c.layer_kind(l) == "c4a")
        return [("c128a layers 0, 60", g128, (c.layers - n4) / 2), ("c4a layers 1, 59", g4, n4 / 2)]

    def cpu_inputs_note(self):
        return (f"layers {', '.join(map(str, self.SAMPLE_LAYERS))} of the stack after the timed steps (spans, "
                f"gates, caches, indexer keys, Q as the GPU consumed them), all {self.cfg.B} sequences; the "
                f"step time scales the c128a sample by 31/2 and the c4a sample by 30/2")


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


    def cpu_groups(self):
        c = self.cfg
        h = {"Q": _host(self.Q), "qidx": _host(self.qidx), "kidx": _host(self.kidx), "cache": _host(self.cache),
             "win": _host(self.ring), "n_entries": _host(self.n_entries), "cache_fmt": "bf16", "win_fmt": "bf16",
             "key_fmt": "bf16", "k": c.k, "D": c.D, "tau": c.tau, "R": c.R, "base": c.rope_base, "pos": c.q_pos}
        _CPU.clear()
        _CPU["main"] = h
        return [("c4a", [("c4a", b) for b in range(c.B)], 1)]

    def cpu_inputs_note(self):
        return ("the stream's state after the timed steps (ragged entry counts, keys, cache, ring as window), all "
                f"{self.cfg.B} sequences; the append's ring write and occasional 8-state fold are not timed")


# ------------------------------------------------------------------ CPU oracle baseline
#
# The oracle as it stands, on the input bytes the GPU step consumed (input set
# 0, copied from the device after the GPU timing), run over the sequences in
# parallel on the host cores: a pool of worker processes forked after the
# inputs are on the host, each worker with one BLAS thread. A task is one
# sequence's decode step through one layer; it starts from the raw cache and
# key bytes (bf16 bits, fp8 / fp4 codes), so the oracle's own decoding of its
# inputs is part of the timed work. The one-thread rate is the same tasks run
# one after the other in the parent with its BLAS pool held to one thread.

_CPU = {}    # the host inputs of the workload being timed (inherited by the forked workers)


def _rows_f64(st, b, rows):
    """Decoded cache rows `rows` of sequence b (oracle decoders)."""
    from oracle import formats as F
    c = st["cache"][b]
    if st["cache_fmt"] == "fp8":
        return F.decode_fp8_rows(c[rows], st["cscale"][b][rows])
    if st["cache_fmt"] == "mixed":
        D = st["D"]
        raw = c[rows]
        codes = raw[:, :D - 64]
        rope = np.ascontiguousarray(raw[:, D - 64:]).view(np.uint16)
        return F.decode_mixed_rows(codes, rope, st["cscale"][b][rows])
    if st["cache_fmt"] == "fp4":
        return F.decode_fp4_rows(c[rows], st["D"])
    return F.bf16_to_f64(c[rows])


def _window_f64(st, b):
    from oracle import formats as F
    if st["win_fmt"] == "fp8":
        return F.decode_fp8_rows(st["win"][b], st["wscale"][b])
    return F.bf16_to_f64(st["win"][b])


def _c4a_ids(st, b):
    from oracle import formats as F
    from oracle import method as M
    q = F.bf16_to_f64(st["qidx"][b])
    if st["key_fmt"] == "fp4":
        keys = F.decode_fp4_g16(st["kcodes"][b], st["kscale"][b])
    else:
        keys = F.bf16_to_f64(st["kidx"][b])
    nv = None if st.get("n_entries") is None else int(st["n_entries"][b])
    return M.topk_ids(M.index_scores(q, keys), st["k"], nv)


def _cpu_task(task):
    """One sequence's decode step through one layer, from raw input bytes."""
    from oracle import formats as F
    from oracle import method as M
    kind, b = task[0], task[1]
    st = _CPU[task[2]] if len(task) > 2 else _CPU["main"]
    Q = F.bf16_to_f64(st["Q"][b])
    if kind == "c4a":
        ids = _c4a_ids(st, b)
        rows = _rows_f64(st, b, ids[ids >= 0])
        O = M.attend(Q, rows, None, _window_f64(st, b), st["tau"], st["R"], st["base"], st["pos"])
    elif kind == "c128a":
        O = M.attend(Q, _rows_f64(st, b, np.arange(st["N"])), None, _window_f64(st, b), st["tau"], st["R"],
                     st["base"], st["pos"])
    elif kind == "m4":
        # a c4a layer of the stack: 32 new entries from the 132-state span
        # (4 carried + 128 new), top-k over the keys, attention over the
        # selected rows and the 128 new states
        span = F.bf16_to_f64(st["span"][b])
        new = M.compress(M.C4A, span, st["gate"][b].astype(np.float64))
        ids = _c4a_ids(st, b) if st.get("kidx") is not None else st["ids"][b]
        sel = ids[ids >= 0]
        first = st["first"]
        fresh = (sel >= first) & (sel < first + new.shape[0])
        rows = np.empty((sel.size, st["D"]))
        rows[~fresh] = F.bf16_to_f64(st["cache"][b][sel[~fresh]])
        rows[fresh] = new[sel[fresh] - first]
        O = M.attend(Q, rows, None, span[4:], st["tau"], st["R"], st["base"], st["pos"])
    elif kind == "m128":
        # a c128a layer of the stack: one new entry from the 128 new states,
        # dense attention over every entry and the new states
        span = F.bf16_to_f64(st["span"][b])
        new = M.compress(M.C128A, span, st["gate"][b].astype(np.float64))
        first = st["first"]
        cache = np.concatenate([F.bf16_to_f64(st["cache"][b][:first]), new], axis=0)
        O = M.attend(Q, cache, None, span, st["tau"], st["R"], st["base"], st["pos"])
    else:
        raise ValueError(kind)
    return float(O[0, 0])


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:
        pass


def _run_pool(tasks, procs):
    import multiprocessing as mp
    ctx = mp.get_context("fork")
    with ctx.Pool(procs, initializer=_pool_init) as pool:
        pool.map(_cpu_task, tasks[:procs], chunksize=1)         # workers up and warm
        t0 = time.perf_counter()
        pool.map(_cpu_task, tasks, chunksize=1)
        return time.perf_counter() - t0


def _one_thread_rate(tasks, seconds):
    try:
        from threadpoolctl import threadpool_limits
        lim = threadpool_limits(limits=1)
    except Exception:
        lim = None
    done, t0 = 0, time.perf_counter()
    while True:
        _cpu_task(tasks[done % len(tasks)])
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    if lim is not None:
        lim.restore_original_limits()
    return done / el, done, el


def cpu_baseline(wl, cfg, seconds):
    """The oracle's decode rate on the host cores, for the JSON line: `value`
    in the workload's unit (decode tokens/s per layer, or per 61-layer step),
    with the one-thread rate beside it."""
    procs = max(1, min(15, os.cpu_count() or 1))
    groups = wl.cpu_groups()        # [(name, tasks, layers_per_step)], inputs in _CPU
    out = {"unit": None, "cores": procs, "kind": "oracle", "nproc": os.cpu_count(), "cpu_model": _cpu_model()}
    rates, rates1, parts = {}, {}, []
    for name, tasks, per_step in groups:
        r1, d1, e1 = _one_thread_rate(tasks, max(1.0, seconds / (4 * len(groups))))
        # enough tasks for about `seconds` of parallel work, whole batches
        est = r1 * procs * seconds / len(groups)
        reps = max(1, int(est // len(tasks)))
        wall = _run_pool(tasks * reps, procs)
        rates[name] = len(tasks) * reps / wall
        rates1[name] = r1
        parts.append(f"{name}: {len(tasks) * reps} tasks ({reps} x {len(tasks)}) in {wall:.1f} s on {procs} "
                     f"processes; one thread {d1} tasks in {e1:.1f} s")
    if len(groups) == 1:
        out["value"] = rates[groups[0][0]]
        out["one_thread"] = {"value": rates1[groups[0][0]]}
        out["unit"] = "decode tokens/s per layer"
    else:
        # a 61-layer step per sequence costs the sampled layers' times scaled
        # to 31 c128a and 30 c4a layers
        t = sum(per / rates[n] for n, _, per in groups)
        t1 = sum(per / rates1[n] for n, _, per in groups)
        out["value"] = 1.0 / t
        out["one_thread"] = {"value": 1.0 / t1}
        out["unit"] = "decode tokens/s per 61-layer step"
        out["layer_rates"] = {n: rates[n] for n, _, _ in groups}
    out["parallel_over_one_thread"] = out["value"] / out["one_thread"]["value"]
    out["sample"] = "; ".join(parts) + f". Inputs: {wl.cpu_inputs_note()}"
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
    return ("k_index_topk",) if kind != "c128a" else ("k_attend", "k_attend_merge")


def _code_only(text):
    """C++ source text without comments and blank space (what the compiler
    sees), so that a comment edit does not retire recorded counters."""
    import re
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif text[i] == '"':            # string literal, kept whole
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def kernel_source_digest():
    """Digest of the kernel sources' code (comments and spacing excluded)."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                h.update(_code_only(f.read()).encode())
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

# the default run: the headline workload, then these, each measured the same way
EXTRA_WORKLOADS = ("c128a_1m_bf16", "c4a_1m_fp8_fp4", "mixed61_256k_bf16")


def _roofline(bytes_per_launch, ms, kernel, traffic):
    achieved = bytes_per_launch / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": int(bytes_per_launch), "avg_launch_ms": round(ms, 5)}


def measure(cfg, args, with_cpu):
    """Times one workload (its own inputs, set up and freed here) and returns
    its part of the JSON line."""
    import torch

    import compressed_sparse_kv_compress_amd as cskv
    import synth
    from synth import device as sd

    cls = {"c4a": C4aLayer, "c128a": C128aLayer, "mixed": Mixed61, "stream": StreamC4a}[cfg.kind]
    stateful = cfg.kind in ("mixed", "stream")   # steps that carry state: no input-set rotation, no graphs
    # Warmup steps: --warmup exactly when given. By default at least 5, and
    # for stateless steps more until 25 ms of them have run: after only a few
    # short steps the GPU clock is still ramping (c128a 1M on one box: 44.7-45.2
    # us per timed step after 5 warmup steps, 39.5-40.5 us after 200). Steps
    # that carry state keep 5 (more would change the context they time; the
    # 61-layer steps are long, the streaming ones are not).
    auto_warm = args.warmup is None
    args = argparse.Namespace(**vars(args))
    if auto_warm:
        args.warmup = 5
    wl = cls(cfg, args, torch, cskv, sd, synth)
    n_sets = args.sets or (1 if stateful else 4)
    log(f"{cfg.name}: setup ({n_sets} input set{'s' if n_sets > 1 else ''})")
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
    def warm_step(i):
        if stateful:
            wl.step(i)
        else:
            st = wl.sets[i % n_sets]
            wl.dominant(st)
            wl.rest(st)

    for i in range(args.warmup):
        warm_step(i)
    torch.cuda.synchronize()
    if auto_warm and not stateful:
        t_warm = time.perf_counter()
        n_warm = args.warmup
        while time.perf_counter() - t_warm < 0.025 and n_warm < 20000:
            for _ in range(5):
                warm_step(n_warm)
                n_warm += 1
            torch.cuda.synchronize()
        args.warmup = n_warm
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
    log(f"{cfg.name}: setup {setup_s:.1f} s, warmup done; timing {args.steps} steps "
        f"({'eager launches' if graphs is None else 'HIP graph replays'})")

    def run_step(i, part="all"):
        if stateful:
            wl.step(i, part == "dominant")
            return
        if graphs is not None:
            g_dom, g_rest = graphs[i % n_sets]
            dom, rest = g_dom.replay, g_rest.replay
        else:
            st = wl.sets[i % n_sets]
            dom, rest = (lambda: wl.dominant(st)), (lambda: wl.rest(st))
        if part in ("all", "dominant"):
            dom()
        if part in ("all", "rest"):
            rest()

    def timed(part, first=0):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(args.steps):
            run_step(first + i, part)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    # the timed region: K steps bracketed by two events only (an event record
    # between kernels costs the stream several microseconds)
    ms_step = timed("all")
    # each call's duration: the calls of K more steps issued back to back
    # (same input-set rotation), bracketed by two events on the stream the
    # kernels are launched on
    dom_ms = timed("dominant") / n4
    rest_ms = timed("rest") if cfg.kind == "c4a" else None
    # spread of the step time: the K timed steps repeated, each repeat between
    # two events as above (a stateful workload continues its stream)
    rep_ms = [timed("all", args.steps * (1 + r) if stateful else 0) for r in range(args.repeats)]
    # c4a: the same steps with the window partial overlapping the indexer
    ovl_ms = None
    if cfg.kind == "c4a" and graphs is None:
        for i in range(args.warmup):
            wl.overlapped(wl.sets[i % n_sets])
        ovl = []
        for r in range(max(1, args.repeats)):
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record()
            for i in range(args.steps):
                wl.overlapped(wl.sets[i % n_sets])
            end.record()
            torch.cuda.synchronize()
            ovl.append(start.elapsed_time(end) / args.steps)
        ovl_ms = float(np.percentile(ovl, 50))

    dom_bytes, rest_bytes = wl.bytes()
    tokens = cfg.B / (ms_step * 1e-3)
    dom_kernel = ("index_topk (k_index_topk: scores, candidate lists, selection)" if cfg.kind != "c128a"
                  else "attend (k_attend + k_attend_merge)")
    out = {
        "metric": "decode tokens/s per 61-layer step" if mixed else "decode tokens/s per layer",
        "value": round(tokens, 1),
        "unit": "tokens/s",
        "ms_per_step": round(ms_step, 5),
        "warmup": args.warmup,
        "dtype": ("bf16" if cfg.cache_dtype == "bf16" and cfg.key_dtype == "bf16" else
                  "fp8 + bf16 rotary (bf16 MFMA, fp32 accumulate)" if cfg.cache_dtype == "mixed" else
                  "fp4 E2M1 + E4M3/16 (bf16 MFMA, fp32 accumulate)" if cfg.cache_dtype == "fp4" else
                  "fp8+fp4 (bf16 MFMA, fp32 accumulate)"),
        "config": {"workload": cfg.name, "batch": cfg.B, "context": cfg.L, "heads": cfg.H, "D": cfg.D,
                   "rotary": cfg.R, "window": cfg.W, "top_k": cfg.k or None, "indexer_dim": cfg.Di or None,
                   "cache": cfg.cache_dtype, "indexer_keys": cfg.key_dtype if cfg.k else None,
                   "layers": cfg.layers, "input_sets_rotated": n_sets,
                   **({"ragged_context": f"{cfg.L} - (0..127)", "append": "one state per sequence per step"}
                      if cfg.kind == "stream" else {}),
                   "launch": "eager" if graphs is None else "hip_graph"},
        "roofline": _roofline(dom_bytes / n4, dom_ms, dom_kernel, recorded_traffic(cfg.name)),
        "step_bandwidth_gbs": round((dom_bytes + rest_bytes) / (ms_step * 1e-3) / 1e9, 1),
        "step_frac": round((dom_bytes + rest_bytes) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": int(dom_bytes + rest_bytes),
        "tflops_per_s": round(wl.flops() / (ms_step * 1e-3) / 1e12, 2),
        "setup_s": round(setup_s, 1),
    }
    if rest_ms is not None:
        out["roofline_attend"] = _roofline(rest_bytes, rest_ms, "attend (sparse: k_attend + k_attend_merge)", None)
    if ovl_ms is not None:
        out["overlap"] = {
            "schedule": "window-only partial on a second stream during index_topk, merged by the attend over "
                        "the selected entries",
            "ms_per_step": round(ovl_ms, 5),
            "value": round(cfg.B / (ovl_ms * 1e-3), 1),
            "serial_ms_per_step": round(ms_step, 5),
            "of": f"median of {max(1, args.repeats)} repeats of {args.steps} steps, after the timed region",
        }
    if rep_ms:
        out["step_ms_spread"] = {
            "repeats": len(rep_ms),
            "median": round(float(np.percentile(rep_ms, 50)), 5),
            "p10": round(float(np.percentile(rep_ms, 10)), 5),
            "p90": round(float(np.percentile(rep_ms, 90)), 5),
            "of": f"ms per step of each repeat of the {args.steps} timed steps, after the timed region",
        }
    log(f"{cfg.name}: {ms_step * 1e3:.1f} us/step, dominant call {dom_ms * 1e3:.1f} us")
    if with_cpu:
        log(f"{cfg.name}: cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(wl, cfg, args.cpu_seconds)
        _CPU.clear()
    del wl, graphs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def hbm_probe():
    """What a plain read stream reaches on this machine: torch's max over 1 GiB
    viewed as int64 (a reduction that only reads), median of 5."""
    import torch
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
    return (1 << 30) / (sorted(times)[2] * 1e-3) / 1e9


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path shards by "
              "sequence with no communication, so N GPUs run N independent copies)", file=sys.stderr)
        sys.exit(2)
    from synth import configs
    name = args.workload or "c4a_128k_bf16"
    cfg = configs.BY_NAME[name]
    if args.summarize_traffic:
        summarize_traffic(cfg, *args.summarize_traffic)
        return
    with_cpu = not args.no_cpu_baseline
    head = measure(cfg, args, with_cpu)
    extras = {}
    if args.workload is None and not args.no_extra:
        for w in EXTRA_WORKLOADS:
            extras[w] = measure(configs.BY_NAME[w], args, with_cpu)
    probe_gbs = hbm_probe()
    out = {
        "metric": head["metric"], "value": head["value"], "unit": head["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": head["warmup"], "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"],
        "data": "synthetic (SplitMix64 streams; caches built by the library's compress kernel)"
                if cfg.kind not in ("mixed", "stream") else
                "synthetic (SplitMix64 streams; prefix caches drawn directly, new states compressed in the step)",
    }
    out.update({k: v for k, v in head.items() if k not in out})
    for part in [out] + list(extras.values()):
        part["roofline"]["frac_of_probe"] = round(part["roofline"]["achieved"] / probe_gbs, 4)
    out["hbm_probe"] = {"read_gbs": round(probe_gbs, 1),
                        "kind": "torch amax over 1 GiB of int64 (read-only stream), median of 5"}
    if extras:
        out["workloads"] = extras
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
