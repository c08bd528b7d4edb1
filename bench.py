"""Benchmark: sparse-FFN decode at batch 1 on the Llama-2-7B-shaped workload.

One step = one decode token through all 31 sparse layers (np_decode_step), with
the row stores in pinned host memory as the workload specifies. One launch
decodes the active sets, diffs them against the resident rows and assigns
slots for all layers. Then one token launch does the rest: a few workgroups
pull every layer's new [gate|up|down^T] bundles over the host link into their
slots, layer after layer. Each layer's fused sparse FFN runs on the other
compute units as soon as its bundles are in place and the previous layer's FFN
has finished.
Centroid IDs and x are resident in HBM before the timed region; the deltas
cross the host link inside it. `value` is that decode rate.

Beside it: the FFN kernel's own time per launch (the roofline: HBM bytes per
launch over launch time, against the 8 TB/s peak and a plain read of the same
bytes), the decode's and the scatter kernel's rates against the host link's
measured ceilings,
the same decode with the row stores moved into HBM ("hbm_store": the FFN then
reads the new bundles through and no scatter runs), and the CPU oracle.

--config N runs another built-in workload the same way (6-8: the paper's
Mistral-7B shape with SwiGLU and intersected masks).

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E peak, GB/s
DEFAULT_WORKLOAD = 2     # Llama-2-7B-shaped: 31 layers, d 4096, M 11008, K_max 4096


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--config", type=int, default=DEFAULT_WORKLOAD, help="built-in workload number")
    p.add_argument("--reduce", choices=["atomic", "ordered"], default="ordered",
                   help="FFN partial-sum reduction: fixed order without atomics (default, bit-reproducible) "
                        "or fp32 atomics")
    p.add_argument("--window", type=int, default=1,
                   help="residency window in tokens (1: the buffer holds exactly the active set)")
    p.add_argument("--layout", choices=["slots", "compact"], default="slots",
                   help="resident buffer layout: slot map (default) or compacted prefix with row moves")
    p.add_argument("--planar", action="store_true",
                   help="slot buffer as one plane per projection row instead of one bundle per slot")
    p.add_argument("--levels", type=int, default=0,
                   help="retention by frequency level: number of levels (0: off; exclusive with --window)")
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--ffn-steps", type=int, default=40,
                   help="tokens in each of the two per-kernel FFN timing passes")
    p.add_argument("--graphs", action="store_true",
                   help="replay each decode step as a captured HIP graph instead of launching one by one")
    p.add_argument("--pcie-steps", type=int, default=40, help="timed tokens of the staged delta I/O leg")
    p.add_argument("--hbm-steps", type=int, default=200, help="timed tokens with the row stores moved into HBM")
    p.add_argument("--no-hbm-store", action="store_true", help="skip the leg with the row stores in HBM")
    p.add_argument("--staging-mb", type=float, default=0.0,
                   help="also time the staged delta I/O (host gather + DMA copy + device scatter) with this "
                        "much pinned staging per buffer (two buffers), reported as staged_delta_io")
    p.add_argument("--staging-threads", type=int, default=0, help="host gather threads (0: library default)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work for the oracle sample")
    p.add_argument("--slots-per-wg", type=int, default=0)
    p.add_argument("--tile-cols", type=int, default=0)
    return p.parse_args()


def workload_text(c, mean_active: float) -> str:
    shape = {2: "Llama-2-7B-shaped", 3: "Llama-2-13B-shaped", 4: "OPT-6.7B-shaped", 5: "d7168 d_ff 28672",
             6: "Mistral-7B-shaped", 7: "Mistral-7B-shaped", 8: "Mistral-7B-shaped"}.get(c.num, c.name)
    ffn = ("SwiGLU (SiLU gate)" if c.act == "silu" else "gated ReLU") if c.R == 3 else "non-gated ReLU"
    rows = "[gate|up|down^T]" if c.R == 3 else "[up|down^T]"
    pers = f"{c.p_lo:.2f}-{c.p_hi:.2f}" if c.recipe == "trajectory" else "~0.84"
    masks = {"union": "union of gate and up centroid masks", "intersect": "intersection of gate and up centroid masks",
             "single": "one centroid mask"}[c.mode]
    return (f"{shape} sparse FFN decode: {c.L} layers, d_model {c.d}, d_ff {c.M}, K_max {c.K}, {ffn}, "
            f"bf16 {rows} bundles, {masks}, ~{100 * mean_active / c.M:.0f}% active, {pers} token-to-token "
            f"persistence, batch 1")


def token_ids(first: int, count: int, T: int) -> list[int]:
    """Token indices first, first+1, ... cycling over 1..T-1 (token 0 is the cold start)."""
    return [1 + ((first - 1 + i) % (T - 1)) for i in range(count)]


def _code_only(text: str) -> str:
    """C++ source without its comments and with whitespace runs collapsed: what the compiler
    sees, so that a comment edit does not count as a kernel change."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of what the sparse-FFN kernel is built from: the code (comments aside) of k_ffn.hip
    and of the launch structs (FfnShape, FfnArgs) of np_internal.hpp."""
    csrc = os.path.join(ROOT, "delta_prefetched_ffn_amd", "csrc")
    h = hashlib.sha256()
    h.update(_code_only(open(os.path.join(csrc, "k_ffn.hip")).read()).encode())
    hdr = open(os.path.join(csrc, "np_internal.hpp")).read()
    i = hdr.index("struct FfnShape")
    j = hdr.index("};", hdr.index("struct FfnArgs")) + 2
    h.update(_code_only(hdr[i:j]).encode())
    return h.hexdigest()[:16]


def stored_traffic(ffn_bytes_per_launch: float, config: int):
    """HBM traffic per FFN launch from the committed rocprofv3 counter summary, if it was taken on
    this kernel source and this workload."""
    path = os.path.join(ROOT, "profiles", "k_sparse_ffn_llama7b_traffic.json")
    if not os.path.exists(path):
        return None, "no counter summary"
    rec = json.load(open(path))
    if rec.get("config") != config:
        return None, f"counters taken on workload {rec.get('config')}, not this one"
    if rec.get("kernel_hash") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    return rec.get("traffic_bytes_per_launch"), rec.get("note", "")


def cpu_baseline(wl, stores, seconds: float, window: int = 1, n_levels: int = 0, threads: int = 0):
    """The CPU oracle, untouched, on a bounded sample of the same workload."""
    from oracle import oracle as O
    c = wl.cfg
    threads = threads or max(1, min(16, os.cpu_count() or 1))
    layers = [O.OracleLayer(c.M, c.K, c.R, c.d, window=window,
                            levels=wl.frequency_levels(l, n_levels) if n_levels else None, n_levels=n_levels)
              for l in range(c.L)]
    mode = O.MODES[c.mode]
    cids = wl.cids()
    tabs = [wl.masks(l) for l in range(c.L)]
    x_all = wl.x_all()

    def one(t, l):
        g, u = cids[t, l]
        S = O.active_set(tabs[l][0][g], tabs[l][-1][u], c.M, mode)
        res = layers[l].step(S)
        layers[l].copy_bundles(stores[l], res)
        O.sparse_ffn(stores[l], c.R, c.d, S, x_all[t, l], c.act)
        return S.size, res.d_in.size

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda l: one(0, l), range(c.L)))       # cold start, untimed
        t0 = time.perf_counter()
        tok, act, din = 0, 0, 0
        while True:  # tokens 1, 2, ..., T-1, 1, 2, ... until the time budget is spent
            t = 1 + tok % (c.T - 1)
            for a, b in ex.map(lambda l: one(t, l), range(c.L)):
                act += a
                din += b
            tok += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    eff = (act + din) * c.bundle_bytes
    return {"value": tok / dt, "unit": "tokens/s", "cores": threads, "host_cpu_count": os.cpu_count(),
            "threads_note": "threads = min(16, os.cpu_count()): the oracle's thread pool, capped at the "
                            "16 host CPUs that one GPU's host share provides", "kind": "oracle",
            "sample": f"{tok} tokens of the same workload (tokens 1..{c.T - 1} in order, repeating; all "
                      f"{c.L} layers; after an untimed cold start), fp64 oracle, "
                      + ("layers in parallel threads" if threads > 1 else "layers one after another on one thread"),
            "effective_gbps": eff / dt / 1e9, "seconds": dt}


def pinned_store(t, reuse: dict):
    """t (a CPU tensor) copied into pinned host memory, or an earlier pinned store when the
    host's pinned-memory limit is reached (reuse["distinct"] records how many could be pinned)."""
    import torch
    if reuse["distinct"] is None:
        try:
            p = torch.empty(t.numel(), dtype=torch.int16, pin_memory=True)
            p.copy_(t)
            reuse["pinned"].append(p)
            return p
        except (RuntimeError, torch.AcceleratorError) as e:  # the pinned-memory limit
            if not reuse["pinned"]:
                raise
            reuse["distinct"] = len(reuse["pinned"])
            log(f"pinning stopped after {len(reuse['pinned'])} row stores ({e.__class__.__name__}): "
                "later layers reuse them (same transfer sizes, other weight values)")
    return reuse["pinned"][reuse["n"] % len(reuse["pinned"])]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path runs on a single "
              "MI355X and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    import torch

    from delta_prefetched_ffn_amd import binding as B
    from workload.gen import CONFIGS, Workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    B.decode_use_graphs(args.graphs)
    wl = Workload(CONFIGS[args.config])
    c = wl.cfg
    t0 = time.time()
    stores = [wl.store(l) for l in range(c.L)]
    log(f"generated {c.L} row stores ({c.L * c.M * c.bundle_bytes / 1e9:.2f} GB) in {time.time() - t0:.1f}s")
    x_all = wl.x_all()
    cids = wl.cids()
    x = torch.from_numpy(x_all).cuda()
    y = torch.zeros_like(x)
    reuse = {"distinct": None, "pinned": [], "n": 0}

    def make_layers(where: str):
        out = []
        for l in range(c.L):
            t = torch.from_numpy(stores[l].reshape(-1).view(np.int16))
            if where == "device":
                dev = t.to("cuda")
            else:
                reuse["n"] = l
                dev = pinned_store(t, reuse)
            L = B.Layer(d_model=c.d, d_ff=c.M, k_max=c.K, n_rows=c.R, masks=wl.masks(l),
                        mask_mode=B.MODES[c.mode], act=B.ACTS[c.act], row_store=dev.data_ptr(), keepalive=dev)
            if args.slots_per_wg or args.tile_cols:
                L.set_ffn_shape(args.slots_per_wg, args.tile_cols)
            if args.window != 1:
                L.set_window(args.window)
            if args.levels:
                L.set_levels(wl.frequency_levels(l, args.levels), args.levels)
            if args.layout != "slots":
                L.set_layout(args.layout)
            if args.planar:
                L.set_planar(True)
            L.set_ffn_reduce(args.reduce)
            out.append(L)
        return out

    cs, ps = torch.cuda.Stream(), torch.cuda.Stream()

    def run_tokens(layers, toks, call_s=None):
        for t in toks:
            t0 = time.perf_counter()
            B.decode_step(layers, cids[t], x[t].data_ptr(), y[t].data_ptr(), cs.cuda_stream, ps.cuda_stream)
            if call_s is not None:
                call_s.append(time.perf_counter() - t0)

    def decode_leg(layers, steps, warmup):
        """Cold start (timed on its own), warm-up, then `steps` timed tokens."""
        torch.cuda.synchronize()
        tc = time.perf_counter()
        run_tokens(layers, [0])                               # cold start: whole active sets
        torch.cuda.synchronize()
        cold = (time.perf_counter() - tc) * 1e3
        run_tokens(layers, token_ids(1, warmup, c.T))
        torch.cuda.synchronize()
        before = np.array([L.counters() for L in layers], dtype=np.int64).sum(axis=0)
        toks = token_ids(1 + warmup, steps, c.T)
        torch.cuda.synchronize()
        call_s = []
        ts = time.perf_counter()
        run_tokens(layers, toks, call_s)
        enq = time.perf_counter() - ts
        torch.cuda.synchronize()
        el = time.perf_counter() - ts
        after = np.array([L.counters() for L in layers], dtype=np.int64).sum(axis=0)
        act_b, in_b = (after - before).tolist()
        return {"tokens_per_s": steps / el, "ms_per_step": el * 1e3 / steps, "cold_start_ms": cold,
                "host_call_ms": {"first_calls": float(np.mean(call_s[:4])) * 1e3, "mean": enq * 1e3 / steps,
                                 "note": "decode_step returns once the token is enqueued; it waits only to reuse "
                                         "what a token a few steps back used (the pinned argument copy of a direct "
                                         "token launch), so the first calls after an idle GPU give the host's own "
                                         "cost per token and the mean runs at the GPU's pace"},
                "effective_gbps": (act_b + in_b) * c.bundle_bytes / el / 1e9,
                "delta_gbps": in_b * c.bundle_bytes / el / 1e9,
                "mean_active_per_layer": act_b / (steps * c.L), "mean_delta_per_layer": in_b / (steps * c.L),
                "steps": steps, "warmup": warmup, "next_token": 1 + warmup + steps}

    def ffn_timing(layers, first_tok, n_tok, scatter: bool):
        """The FFN launches of one token back to back between two HIP events on their stream, after
        the token's assignments (and, for host-memory stores, its scatters) are done; on odd
        tokens each launch between its own events. scatter=False: each FFN reads its new bundles
        through from the (device) row store, as in a decode step with HBM stores. Algorithmic
        bytes of a launch: active bundles read (+ new bundles written when reading through) +
        x + y. Also times the scatter launches of the same tokens back to back."""
        s = cs
        # A 4 GiB streaming read (about 0.7 ms) ahead of each burst: the host queues the burst's
        # launches while it runs, so the launches follow each other on the GPU with no gap that
        # the host's per-call cost (ctypes and the library's checks) would leave.
        lead = torch.empty((4 << 30) // 2, dtype=torch.int16, device="cuda")
        lead_sink = torch.empty(65536, dtype=torch.float32, device="cuda")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(c.L)]
        burst = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        sc_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        acc = dict(burst_ms=0.0, event_ms=0.0, bytes=0, act_bytes=0, n=0, ev_n=0, sc_ms=0.0, sc_bytes=0, sc_n=0)
        for i, t in enumerate(token_ids(first_tok, 2 * n_tok, c.T)):
            ns = []
            for l, L in enumerate(layers):
                g, u = (int(v) for v in cids[t, l])
                L.delta_assign(g, u, s.cuda_stream)
                info = L.info()
                ns.append((info["n_active"], info["n_in"]))
            if scatter:
                sc_ev[0].record(s)
                for L in layers:
                    L.scatter_rows(s.cuda_stream)
                sc_ev[1].record(s)
            s.synchronize()
            if scatter:
                acc["sc_ms"] += sc_ev[0].elapsed_time(sc_ev[1])
                acc["sc_bytes"] += sum(ni for _, ni in ns) * c.bundle_bytes
                acc["sc_n"] += c.L
            if i % 2 == 0:
                B.probe_read(lead.data_ptr(), lead.numel() * 2, lead_sink.data_ptr(), s.cuda_stream)
                burst[0].record(s)
                for l, L in enumerate(layers):
                    L.sparse_ffn(x[t, l].data_ptr(), y[t, l].data_ptr(), s.cuda_stream)
                burst[1].record(s)
                s.synchronize()
                acc["burst_ms"] += burst[0].elapsed_time(burst[1])
                acc["bytes"] += sum((na + (0 if scatter else ni)) * c.bundle_bytes + 2 * c.d * 4 for na, ni in ns)
                acc["act_bytes"] += sum(na * c.bundle_bytes for na, _ in ns)
                acc["n"] += c.L
            else:
                for l, L in enumerate(layers):
                    ev[l][0].record(s)
                    L.sparse_ffn(x[t, l].data_ptr(), y[t, l].data_ptr(), s.cuda_stream)
                    ev[l][1].record(s)
                s.synchronize()
                acc["event_ms"] += sum(a.elapsed_time(b) for a, b in ev)
                acc["ev_n"] += c.L
        del lead, lead_sink
        us = acc["burst_ms"] * 1e3 / acc["n"]
        bpl = acc["bytes"] / acc["n"]
        apl = acc["act_bytes"] / acc["n"]
        out = {"bytes_per_launch": bpl, "active_row_bytes_per_launch": apl, "avg_launch_us": us,
               "avg_launch_us_own_events": acc["event_ms"] * 1e3 / max(acc["ev_n"], 1),
               "achieved_gbps": bpl / (us * 1e-6) / 1e9, "active_row_gbps": apl / (us * 1e-6) / 1e9,
               "launches": acc["n"]}
        if scatter:
            out["scatter"] = {"us_per_layer": acc["sc_ms"] * 1e3 / acc["sc_n"],
                              "bytes_per_layer": acc["sc_bytes"] / acc["sc_n"],
                              "gbps": acc["sc_bytes"] / (acc["sc_ms"] * 1e-3) / 1e9,
                              "timing": f"HIP events around the {c.L} layers' scatter launches of a token, back to back"}
        return out

    # ---------------- the workload as specified: row stores in pinned host memory ----------------
    # Per token: one assignment launch for all layers, then one token launch: a few workgroups
    # pull every layer's new bundles over the host link, and each layer's FFN runs on the other
    # compute units once its bundles are in place (and the previous layer's FFN has finished).
    hl = make_layers("host")
    log(f"pinned-host layers ready in {time.time() - t0:.1f}s")
    dec = decode_leg(hl, args.steps, args.warmup)
    log(f"decode (pinned-host stores): {dec['ms_per_step']:.3f} ms/token, {dec['tokens_per_s']:.1f} tok/s, "
        f"deltas {dec['delta_gbps']:.1f} GB/s over the host link")
    moves = None
    if args.layout == "compact":  # rows moved inside the buffer (read + written in HBM), untimed pass
        mv_toks = token_ids(dec["next_token"], 16, c.T)
        n_mv = 0
        for t in mv_toks:
            run_tokens(hl, [t])
            n_mv += sum(L.read_moves()[0].size for L in hl)
        moves = {"mean_moves_per_layer": n_mv / (len(mv_toks) * c.L),
                 "moved_bytes_per_token": 2 * n_mv / len(mv_toks) * c.bundle_bytes, "tokens": len(mv_toks)}
        log(f"compact layout: {moves['mean_moves_per_layer']:.1f} rows moved per layer")
    torch.cuda.synchronize()
    ffn = ffn_timing(hl, dec["next_token"] + 16, args.ffn_steps, scatter=True)
    log(f"k_sparse_ffn (rows resident): {ffn['bytes_per_launch'] / 1e6:.2f} MB/launch, {ffn['avg_launch_us']:.2f} "
        f"us/launch (back-to-back), {ffn['avg_launch_us_own_events']:.2f} us (own events) -> "
        f"{ffn['achieved_gbps']:.0f} GB/s; scatter {ffn['scatter']['us_per_layer']:.1f} us/layer, "
        f"{ffn['scatter']['gbps']:.1f} GB/s")
    staged = None
    if args.staging_mb > 0:
        B.decode_set_staging(int(args.staging_mb * (1 << 20)), args.staging_threads)
        for L in hl:
            L.reset()
        staged = decode_leg(hl, args.pcie_steps, 4)
        B.decode_set_staging(0)
        staged["staging_bytes"] = int(args.staging_mb * (1 << 20))
        staged["gather_threads"] = args.staging_threads or "library default (min(8, cores))"
        log(f"staged delta I/O: {staged['tokens_per_s']:.1f} tok/s, deltas {staged['delta_gbps']:.1f} GB/s")
    for L in hl:
        L.close()
    del hl

    # ---------------- host-link ceilings ----------------
    # Pull: the streaming-read kernel reading pinned host memory (what the scatter kernel does);
    # DMA: the copy engine moving pinned host memory to the device (hipMemcpyAsync).
    sink = torch.empty(65536, dtype=torch.float32, device="cuda")
    s = cs
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    link_bytes = 1 << 30
    hb = reuse["pinned"][0] if reuse["pinned"] else None
    if hb is None or hb.numel() * 2 < link_bytes:
        hb = torch.empty(link_bytes // 2, dtype=torch.int16, pin_memory=True)
    B.probe_read(hb.data_ptr(), link_bytes, sink.data_ptr(), s.cuda_stream)
    e0.record(s)
    for _ in range(3):
        B.probe_read(hb.data_ptr(), link_bytes, sink.data_ptr(), s.cuda_stream)
    e1.record(s)
    s.synchronize()
    pull_gbps = 3 * link_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    db = torch.empty(link_bytes // 2, dtype=torch.int16, device="cuda")
    with torch.cuda.stream(s):
        db.copy_(hb[: link_bytes // 2], non_blocking=True)
        e0.record(s)
        for _ in range(3):
            db.copy_(hb[: link_bytes // 2], non_blocking=True)
        e1.record(s)
    s.synchronize()
    dma_gbps = 3 * link_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del db, hb
    reuse["pinned"].clear()
    log(f"host link: pull {pull_gbps:.1f} GB/s, DMA {dma_gbps:.1f} GB/s")

    # ---------------- the same decode with the row stores moved into HBM ----------------
    # Not the specified workload (no host-link transfer): each FFN reads its new bundles from the
    # store in HBM and writes them into their slots (read-through), so no scatter runs.
    hbm = None
    if not args.no_hbm_store:
        dl = make_layers("device")
        hdec = decode_leg(dl, args.hbm_steps, args.warmup)
        hffn = ffn_timing(dl, hdec["next_token"], args.ffn_steps, scatter=False)
        for L in dl:
            L.close()
        del dl
        torch.cuda.empty_cache()
        hbm = {**{k: v for k, v in hdec.items() if k != "next_token"},
               "ffn_read_through": {**hffn, "frac_of_peak": hffn["achieved_gbps"] / HBM_PEAK_GBPS,
                                    "kernel": "k_sparse_ffn (read-through instantiation)"},
               "store": "HBM (device memory), new bundles read through by the FFN"}
        log(f"decode (HBM stores): {hdec['tokens_per_s']:.1f} tok/s; read-through FFN {hffn['avg_launch_us']:.2f} "
            f"us/launch, {hffn['achieved_gbps']:.0f} GB/s")

    # ---------------- plain read of the same bytes per launch ----------------
    # The streaming-read kernel on as many bytes as one FFN launch reads, launched back to back
    # by the library's own loop over rotating buffers (1.5 GB in all, more than the last-level
    # cache, so every launch reads HBM): what moving that many bytes costs in one launch, launch
    # gap and ramp included, with no dependent load, no exchange and no reduction.
    sb_bytes = int(ffn["bytes_per_launch"]) // 16 * 16
    n_sb = max(8, -(-1_500_000_000 // sb_bytes))
    sb_bufs = [torch.empty(sb_bytes // 2, dtype=torch.int16, device="cuda") for _ in range(n_sb)]
    sb_ptrs = [b.data_ptr() for b in sb_bufs]
    B.probe_read_set(sb_ptrs, sb_bytes, 1, sink.data_ptr(), s.cuda_stream)
    e0.record(s)
    B.probe_read_set(sb_ptrs, sb_bytes, 3, sink.data_ptr(), s.cuda_stream)
    e1.record(s)
    s.synchronize()
    sb_us = e0.elapsed_time(e1) * 1e3 / (3 * n_sb)
    del sb_bufs, sb_ptrs
    stream_bound = {"bytes_per_launch": sb_bytes, "us_per_launch": sb_us,
                    "gbps": sb_bytes / (sb_us * 1e-6) / 1e9,
                    "frac_of_peak": sb_bytes / (sb_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                    "ffn_launch_over_plain_read": ffn["avg_launch_us"] / sb_us,
                    "how": f"plain streaming read of the same bytes, {n_sb} rotating buffers, launched back to back "
                           "by the library (np_probe_read_set)"}
    log(f"plain read of {sb_bytes / 1e6:.2f} MB per launch: {sb_us:.2f} us/launch "
        f"({stream_bound['gbps']:.0f} GB/s); the FFN launch takes {ffn['avg_launch_us'] / sb_us:.2f}x that")

    # ---------------- streaming-read and copy probes (HBM) ----------------
    probe_bytes = 4 << 30
    buf = torch.empty(probe_bytes // 2, dtype=torch.int16, device="cuda")
    for _ in range(2):
        B.probe_read(buf.data_ptr(), probe_bytes, sink.data_ptr(), s.cuda_stream)
    e0.record(s)
    for _ in range(5):
        B.probe_read(buf.data_ptr(), probe_bytes, sink.data_ptr(), s.cuda_stream)
    e1.record(s)
    s.synchronize()
    probe_gbps = 5 * probe_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    # plain 128-bit copy of a known size: the reference that scales the HBM byte counters
    copy_bytes = 256 << 20
    cdst = torch.empty(copy_bytes // 2, dtype=torch.int16, device="cuda")
    B.probe_copy(cdst.data_ptr(), buf.data_ptr(), copy_bytes, s.cuda_stream)
    e0.record(s)
    for _ in range(3):
        B.probe_copy(cdst.data_ptr(), buf.data_ptr(), copy_bytes, s.cuda_stream)
    e1.record(s)
    s.synchronize()
    copy_gbps = 3 * 2 * copy_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, cdst
    log(f"HBM probes: streaming read {probe_gbps:.0f} GB/s, copy {copy_gbps:.0f} GB/s (read + write)")
    traffic, traffic_note = stored_traffic(ffn["bytes_per_launch"], args.config)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(wl, stores, args.cpu_seconds, args.window, args.levels)
        one = cpu_baseline(wl, stores, max(2.0, args.cpu_seconds / 3), args.window, args.levels, threads=1)
        cpu["single_thread"] = {"value": one["value"], "unit": "tokens/s", "cores": 1, "sample": one["sample"],
                                "seconds": one["seconds"]}
        log(f"cpu baseline, one thread: {one['value']:.3f} tok/s")
        log(f"cpu baseline: {cpu['value']:.3f} tok/s on {cpu['cores']} threads")

    store_text = "pinned host memory (hipHostMalloc via torch), the new bundles of every token pulled over the host link"
    if reuse["distinct"]:
        store_text += (f"; only {reuse['distinct']} of {c.L} row stores could be pinned, the other layers reuse them "
                       "(the host-link traffic is the same, the weights differ)")
    out = {
        "metric": "sparse-FFN decode tokens/s at batch 1; effective HBM GB/s vs peak",
        "value": dec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 weights / fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": workload_text(c, dec["mean_active_per_layer"]),
                   "global_batch": 1, "layers": c.L, "d_model": c.d, "d_ff": c.M, "k_max": c.K,
                   "weights": "bf16", "backing_store": store_text, "parallelism": "single GPU",
                   "residency_window": args.window, "frequency_levels": args.levels,
                   "buffer_layout": args.layout, "planar_buffers": args.planar,
                   "ffn_reduce": args.reduce},
        "effective_gbps": dec["effective_gbps"],
        "effective_frac_of_hbm_peak": dec["effective_gbps"] / HBM_PEAK_GBPS,
        "delta_gbps_over_host_link": dec["delta_gbps"],
        "mean_active_per_layer": dec["mean_active_per_layer"],
        "mean_delta_per_layer": dec["mean_delta_per_layer"],
        **({"compact_moves": moves} if moves else {}),
        "cold_start_ms": dec["cold_start_ms"],
        "host_call_ms": dec["host_call_ms"],
        "decode_launches": ("captured graph replay" if args.graphs else "direct launches") +
                           ": per token one assign launch and one token launch (every layer's delta scatter and FFN)",
        "roofline": {"bound": "hbm", "achieved": ffn["achieved_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": ffn["achieved_gbps"] / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "k_sparse_ffn", "bytes_per_launch": ffn["bytes_per_launch"],
                     "active_row_bytes_per_launch": ffn["active_row_bytes_per_launch"],
                     "active_row_gbps": ffn["active_row_gbps"],
                     "avg_launch_us": ffn["avg_launch_us"], "avg_launch_us_own_events": ffn["avg_launch_us_own_events"],
                     "timing": f"HIP events on the launch stream around the {c.L} FFN launches of a token back to back, "
                               "after that token's assignments and scatters (the FFN of the pinned-host decode: rows "
                               "resident, nothing written but y), queued behind a 4 GiB streaming read so that the "
                               "host's per-call cost leaves no gap between them",
                     "traffic_note": traffic_note,
                     "plain_read_same_bytes": stream_bound},
        "host_link": {"pull_probe_gbps": pull_gbps, "dma_probe_gbps": dma_gbps,
                      "pcie_gen5_x16_gbps_per_direction": 63.0,
                      "decode_delta_gbps": dec["delta_gbps"],
                      "decode_frac_of_pull_probe": dec["delta_gbps"] / pull_gbps,
                      "scatter_kernel": {**ffn["scatter"], "frac_of_pull_probe": ffn["scatter"]["gbps"] / pull_gbps},
                      "how": "pull: the streaming-read kernel on 1 GiB of pinned host memory; DMA: hipMemcpyAsync of "
                             "1 GiB pinned host -> device (torch copy_); both timed with HIP events"},
        "hbm_store": hbm,
        "hbm_read_probe_gbps": probe_gbps,
        "hbm_copy_probe_gbps": copy_gbps,
        **({"staged_delta_io": staged} if staged else {}),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
