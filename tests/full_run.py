"""Complete full-size parity run of one workload (GPU tests only; imports torch lazily).

One run covers a group of layers of a workload from a cold start over all its steps, with the
same layers built once per row-store placement ("device": the row store in HBM, the FFN reads
the new bundles through; "host": the row store in pinned host memory, the token launch pulls
them over the host link). Every placement runs np_decode_step as bench.py calls it (a compute
and a copy stream), and is compared with one oracle run:

  * at every (step, layer): the delta lists, slot map, owner table and active-slot list,
    bit-exact (NeuroPrefetcher section 3.4);
  * at steps 0, 1, T/2 and T-1: every layer's whole slot buffer, stale rows of freed slots
    included, bit-exact against the oracle's buffer (which copies each incoming bundle
    byte by byte into its slot);
  * y at every (step, layer) within max-abs 2e-2 and relative L2 5e-3 of the oracle's fp64
    sparse FFN, which the oracle evaluates from the row store over the active neuron IDs
    (never from its slot machinery);
  * with the ordered (atomics-free) reduction, y bit-identical between the placements;
  * a second pass that resets the layers and enqueues all T steps back to back without any
    synchronization in between: y of every step bit-identical to the first pass, and the
    final state and whole buffers bit-exact against the oracle's final ones.
"""
from __future__ import annotations

import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import oracle as O
from tests.harness import check_y, compare_state, torch_mod
from workload.gen import CONFIGS, Workload

POOL = 16  # host threads for the oracle (one GPU's share of the host CPUs)


def log(msg: str) -> None:
    print(f"[full] {msg}", flush=True)


def _same_bits(a, b) -> bool:
    return np.array_equal(np.ascontiguousarray(a).view(np.uint32), np.ascontiguousarray(b).view(np.uint32))


def run_complete(num: int, group: list[int] | None = None, wheres=("device", "host"), steps: int | None = None,
                 reduce: str | None = None, tag: str = "") -> dict:
    """reduce None keeps the library's default FFN reduction (the ordered one), so the bitwise
    repeat checks below test the default path."""
    from delta_prefetched_ffn_amd import binding as B
    torch = torch_mod()
    assert torch.cuda.is_available()
    B.decode_use_graphs(False)
    wl = Workload(CONFIGS[num])
    c = wl.cfg
    layers_idx = list(range(c.L)) if group is None else list(group)
    G = len(layers_idx)
    T = c.T if steps is None else steps
    bitwise = reduce in (None, "ordered")
    what = f"cfg{num}{tag} layers {layers_idx[0]}..{layers_idx[-1]}"
    t0 = time.time()

    # Row stores: one host copy per layer, which the oracle reads. With a pinned placement the
    # pinned buffer is that copy (no second one in host memory).
    host_views, keep = [], []
    dev_layers = {w: [] for w in wheres}
    for l in layers_idx:
        st = wl.store(l)
        flat = torch.from_numpy(st.reshape(-1).view(np.int16))
        pinned = None
        if "host" in wheres:
            pinned = torch.empty(flat.numel(), dtype=torch.int16, pin_memory=True)
            pinned.copy_(flat)
            keep.append(pinned)
            host_views.append(pinned.numpy().view(np.uint16).reshape(c.M, c.R, c.d))
            del st, flat
        else:
            host_views.append(st)
        for w in wheres:
            buf = pinned if w == "host" else (pinned if pinned is not None else flat).to("cuda")
            keep.append(buf)
            L = B.Layer(d_model=c.d, d_ff=c.M, k_max=c.K, n_rows=c.R, masks=wl.masks(l),
                        mask_mode=B.MODES[c.mode], act=B.ACTS[c.act], row_store=buf.data_ptr(), keepalive=buf)
            if reduce is not None:
                L.set_ffn_reduce(reduce)
            dev_layers[w].append(L)
    torch.cuda.synchronize()
    log(f"{what}: {G} layers x {list(wheres)} built in {time.time() - t0:.1f}s")

    cids_all = wl.cids()[:T, layers_idx]                       # [T][G][2]
    x_np = np.ascontiguousarray(wl.x_all()[:T, layers_idx])    # [T][G][d]
    x = torch.from_numpy(x_np).cuda()
    ys = {w: torch.full_like(x, float("nan")) for w in wheres}
    cs, ps = torch.cuda.Stream(), torch.cuda.Stream()
    orc = [O.OracleLayer(c.M, c.K, c.R, c.d, keep_buffer=True) for _ in layers_idx]
    tabs = [wl.masks(l) for l in layers_idx]
    mode = O.MODES[c.mode]

    def active(t, g):
        gc, uc = cids_all[t, g]
        return O.active_set(tabs[g][0][gc], tabs[g][-1][uc], c.M, mode)

    def oracle_step(t, g):
        S = active(t, g)
        res = orc[g].step(S)
        orc[g].copy_bundles(host_views[g], res)
        return S, res

    checkpoints = sorted({0, min(1, T - 1), T // 2, T - 1})
    pool = ThreadPoolExecutor(POOL)
    n_state = n_buf = 0
    for t in range(T):
        for w in wheres:
            B.decode_step(dev_layers[w], cids_all[t], x[t].data_ptr(), ys[w][t].data_ptr(), cs.cuda_stream,
                          ps.cuda_stream)
        results = list(pool.map(lambda g: oracle_step(t, g), range(G)))
        for w in wheres:
            for g in range(G):
                S, res = results[g]
                compare_state(dev_layers[w][g].read_state(), orc[g], res, S, f"{what} {w} t={t} l={layers_idx[g]}")
                n_state += 1
        if t in checkpoints:
            for w in wheres:
                for g in range(G):
                    got = dev_layers[w][g].read_rows()
                    assert np.array_equal(got, orc[g].buf), f"{what} {w} t={t} l={layers_idx[g]}: whole buffer"
                    n_buf += 1
        if t % 64 == 0:
            log(f"{what}: step {t}/{T} state ok ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    log(f"{what}: {n_state} (step, layer, placement) states and {n_buf} whole buffers bit-exact "
        f"({time.time() - t0:.1f}s)")

    # y at every (step, layer)
    yh = {w: ys[w].cpu().numpy() for w in wheres}

    def y_check(tg):
        t, g = tg
        ref = O.sparse_ffn(host_views[g], c.R, c.d, active(t, g), x_np[t, g], c.act)
        for w in wheres:
            check_y(yh[w][t, g], ref, f"{what} {w} t={t} l={layers_idx[g]}")
        return True

    n_y = sum(pool.map(y_check, [(t, g) for t in range(T) for g in range(G)]))
    log(f"{what}: y of {n_y} (step, layer) pairs x {len(wheres)} placements in tolerance ({time.time() - t0:.1f}s)")
    if bitwise and len(wheres) > 1:
        w0 = wheres[0]
        for w in wheres[1:]:
            assert _same_bits(yh[w], yh[w0]), f"{what}: y differs between {w0} and {w} stores"

    # back to back: reset, enqueue all steps with no synchronization in between
    for w in wheres:
        for L in dev_layers[w]:
            L.reset()
        y2 = torch.full_like(x, float("nan"))
        for t in range(T):
            B.decode_step(dev_layers[w], cids_all[t], x[t].data_ptr(), y2[t].data_ptr(), cs.cuda_stream,
                          ps.cuda_stream)
        torch.cuda.synchronize()
        y2h = y2.cpu().numpy()
        if bitwise:
            assert _same_bits(y2h, yh[w]), f"{what} {w}: back-to-back y differs from the synchronized run"
        else:
            for t in range(T):
                for g in range(G):
                    assert np.allclose(y2h[t, g], yh[w][t, g], rtol=1e-5, atol=1e-6)
        for g in range(G):
            st = dev_layers[w][g].read_state()
            assert st["err"] == 0
            assert np.array_equal(st["slot_map"], orc[g].slot_map), f"{what} {w} back-to-back l={layers_idx[g]}"
            assert np.array_equal(st["owner"], orc[g].owner), f"{what} {w} back-to-back l={layers_idx[g]}"
            assert np.array_equal(dev_layers[w][g].read_rows(), orc[g].buf), \
                f"{what} {w} back-to-back l={layers_idx[g]}: whole buffer"
    log(f"{what}: back-to-back pass reproduces y and the final state ({time.time() - t0:.1f}s)")
    pool.shutdown()
    for w in wheres:
        for L in dev_layers[w]:
            L.close()
    del dev_layers, keep, host_views, orc
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"states": n_state, "buffers": n_buf, "y": n_y}
