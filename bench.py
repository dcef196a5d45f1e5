#!/usr/bin/env python3
"""Draft-tree round throughput on one MI355X.

A step is one full speculative-decoding round of the hot path on the CAST
workload (B=8, V=128256, bf16 draft and target logits, depth 8, expand 10,
60 verify tokens, CAST width / depth / verify-count selection, greedy verify):
8 ddt_tree_expand layers, ddt_tree_select (rerank and flat layout in one
launch) and ddt_tree_verify.  Inputs are seeded synthetic logits resident in HBM before the
timed region, in a ring of rounds whose distinct logit bytes exceed 1 GB (more
than twice the 256 MB last-level cache).  Each ring slot's round is captured
once as a HIP graph (the kernels take every size from device memory, so no host
synchronisation is needed between layers) and the timed region replays them.

Prints one JSON line.  --gpus above 1 is refused: the bench measures one GPU.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time
from typing import Optional

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
SEED = 1002
PROFILES = os.path.join(ROOT, "profiles")


def pmc_file(workload: str) -> str:
    return os.path.join(PROFILES, f"k_expand_layer_traffic_{workload}.json")
CSRC = os.path.join(ROOT, "dynamic_draft_tree_row_amd", "csrc")
KERNEL_SRC = os.path.join(CSRC, "ddt_rowreduce.hpp")
LAYER_SRC = os.path.join(CSRC, "ddt_layer.hpp")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """The few HIP runtime calls the bench needs (events), via ctypes."""

    def __init__(self):
        self.h = C.CDLL("libamdhip64.so.7")
        self.h.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.h.hipEventDestroy.argtypes = [C.c_void_p]

    def events(self, n):
        out = []
        for _ in range(n):
            e = C.c_void_p()
            if self.h.hipEventCreate(C.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e)
        return out

    def elapsed_ms(self, a, b) -> float:
        ms = C.c_float()
        st = self.h.hipEventElapsedTime(C.byref(ms), a, b)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value


def flat_layout(run, B):
    """Per flat position: key, depth, expand slot, token, from the library's outputs."""
    t, f = run.tree, run.flat
    node = f.node.cpu().numpy()
    key, dep = t.key.cpu().numpy(), t.depth.cpu().numpy()
    esl, tok = t.eslot.cpu().numpy(), t.token.cpu().numpy()
    P = node.shape[1]
    fk = np.full((B, P), -1, np.int64)
    fd = np.zeros((B, P), np.int32)
    fs = np.full((B, P), -1, np.int32)
    ft = np.full((B, P), -1, np.int32)
    for b in range(B):
        ok = node[b] >= 0
        nv = node[b][ok]
        fk[b, ok], fd[b, ok], fs[b, ok], ft[b, ok] = key[b, nv], dep[b, nv], esl[b, nv], tok[b, nv]
    return fk, fd, fs, ft


def snapshot(run):
    return {k: v.clone() for k, v in (
        ("accept_len", run.accept_len), ("accept_path", run.accept_path),
        ("next_token", run.next_token), ("token", run.flat.token), ("mask", run.flat.mask),
        ("m", run.m_out), ("widths", run.tree.widths), ("argmax", run.row_argmax))}


def same(a, b) -> bool:
    import torch
    return all(torch.equal(a[k], b[k]) for k in a)


KERNEL_END = "#undef RR_ID\n}\n"   # the end of the chunk reduction in its source file


def kernel_hash() -> str:
    """Hash of the expand layer kernel's source: the chunk reduction's file up
    to the end of rr_chunk (the reduction and every helper it calls) and the
    layer kernel's own file."""
    text = open(KERNEL_SRC, "rb").read().decode()
    end = text.index(KERNEL_END) + len(KERNEL_END)
    layer = open(LAYER_SRC, "rb").read().decode()
    return hashlib.sha256((text[:end] + layer).encode()).hexdigest()[:16]


def traffic_per_launch(workload: str):
    """HBM bytes per expand-layer launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source for this workload."""
    try:
        d = json.load(open(pmc_file(workload)))
    except (OSError, ValueError):
        return None
    if d.get("kernel_sha") != kernel_hash() or d.get("workload") != workload:
        return None
    return d.get("expand_bytes_per_launch")


CAL_BYTES = 256 << 20          # the calibration copy: reads and writes this many bytes


def ingest_pmc(fetch_csv: str, write_csv: str, workload: str, ring: int) -> None:
    """Per-launch HBM bytes of the row reduction from two rocprofv3 --pmc passes
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Each counter is scaled by
    what it reads for the calibration copy of CAL_BYTES read + CAL_BYTES written."""
    import csv

    def per_dispatch(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        return vals

    f = per_dispatch(fetch_csv, "FETCH_SIZE")
    wr = per_dispatch(write_csv, "WRITE_SIZE")

    # the pmc run's two eager passes over the ring: per round D expand-layer
    # launches and one verify reduction launch
    def split(vals, name):
        ks = [v for (d, n), v in sorted(vals.items()) if name in n]
        cal = [v for (d, n), v in sorted(vals.items()) if "neg" in n.lower()]
        if not ks or not cal:
            raise SystemExit(f"counter CSV lacks {name} or the calibration dispatches")
        return ks, cal[-1]

    fe, fcal = split(f, "k_expand_layer")
    we, wcal = split(wr, "k_expand_layer")
    fv, _ = split(f, "k_row_partial")
    wv, _ = split(wr, "k_row_partial")
    ff = (CAL_BYTES / 1024.0) / fcal
    wf = (CAL_BYTES / 1024.0) / wcal
    fetch_b = float(np.mean(fe)) * 1024.0 * ff
    write_b = float(np.mean(we)) * 1024.0 * wf
    vfetch_b = float(np.mean(fv)) * 1024.0 * ff
    vwrite_b = float(np.mean(wv)) * 1024.0 * wf
    out = {"workload": workload, "kernel_sha": kernel_hash(),
           "expand_bytes_per_launch": round(fetch_b + write_b, 1),
           "expand_fetch_bytes_per_launch": round(fetch_b, 1),
           "expand_write_bytes_per_launch": round(write_b, 1),
           "verify_bytes_per_launch": round(vfetch_b + vwrite_b, 1),
           "fetch_scale": round(ff, 4), "write_scale": round(wf, 4),
           "dispatches": {"expand": [len(fe), len(we)], "verify": [len(fv), len(wv)]},
           "calibration": f"torch.neg over {CAL_BYTES >> 20} MiB fp32 (reads and writes {CAL_BYTES} bytes)"}
    os.makedirs(PROFILES, exist_ok=True)
    with open(pmc_file(workload), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def expand_b64_detail(api, lib, hip, dev, reps: int = 10) -> dict:
    """One draft layer at the B = 64 workload's shape through ddt_tree_expand:
    64 requests x 16 frontier rows of V = 128256 bf16 logits (262.7 MB),
    K_n = 16 children per row, frontier 16.  Each timed layer 2 follows an
    untimed layer 1 (64 rows) that sets the frontier.  Rows are N(0, 1)
    scaled per row by U(0.3, 3), generated on the device.  At this many rows the
    layer runs as the plain reduction and then one workgroup per request; the
    time spans both launches."""
    import torch
    B, R, V, K = 64, 16, 128256, 16
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    x = torch.randn(2, B, R, V, device=dev, generator=g)
    x.mul_(0.3 + 2.7 * torch.rand(2, B, R, 1, device=dev, generator=g))
    x = x.to(torch.bfloat16)
    tree = api.DeviceTree(B, 1 + K + K * K, 2, R, dev)
    ws = torch.empty(api.workspace_bytes(B * R, V, torch.bfloat16, K), dtype=torch.uint8, device=dev)
    roots = torch.zeros(B, dtype=torch.int32, device=dev)
    for _ in range(2):
        api.tree_expand(tree, 1, roots, x[0], K, R, ws)
        api.tree_expand(tree, 2, roots, x[1], K, R, ws)
    torch.cuda.synchronize()
    evs = hip.events(4 * reps)
    arr = (C.c_void_p * len(evs))(*[e.value for e in evs])
    lib.ddt_set_reduce_events(arr, 2 * reps)
    for _ in range(reps):
        api.tree_expand(tree, 1, roots, x[0], K, R, ws)
        api.tree_expand(tree, 2, roots, x[1], K, R, ws)
    used = lib.ddt_set_reduce_events(None, 0)
    torch.cuda.synchronize()
    assert used == 2 * reps
    us = np.array([hip.elapsed_ms(evs[4 * i + 2], evs[4 * i + 3]) * 1e3 for i in range(reps)])
    nbytes = B * R * V * 2
    gbs = nbytes / (us.mean() * 1e-6) / 1e9
    assert int(tree.n_nodes.min()) == 1 + K + R * K, "layer 2 did not expand every row"
    del x, tree, ws
    return {"kernel": "k_row_partial<bf16,8> + k_expand_finish", "rows": B * R, "V": V, "K_n": K,
            "mb": round(nbytes / 1e6, 1), "us": round(float(us.mean()), 2),
            "us_min": round(float(us.min()), 2), "gbs": round(float(gbs), 1),
            "frac": round(float(gbs / PEAK_HBM_GBS), 4)}


def tree_attention_detail(api, dev, seed: int = 7, launches: int = 10, B: int = 64, P: int = 129,
                          L: int = 4096, split_options=(None,)) -> dict:
    """The verify forward's tree attention, by default at the B=64 mixed
    shape: 129 flat positions per request over a 4096-token prefix, 32 query
    and 8 key/value heads of 128 (an 8B-class target).  Trees are random
    (every parent within the 16 positions before its child); q, k and v are
    seeded normal bf16.  Timed with events on the launch stream; algorithmic
    flops count the visible (query, key) pairs only: 4 * D per pair and query
    head.  split_options: None times ddt_tree_attention, an integer
    ddt_tree_attention_split with that many key splits (0: the library's
    choice); the first option gives the top-level figures."""
    import torch
    Hq, Hkv, D = 32, 8, 128
    rng = np.random.default_rng(seed)
    flat = api.DeviceFlat(B, P - 1, 10, dev)
    W = flat.W
    rows = np.arange(B)
    masks = np.zeros((B, P, W), np.uint32)
    vis = np.zeros((B, P), np.int64)                 # visible tree positions per query
    for i in range(P):
        if i > 0:
            par = rng.integers(max(0, i - 16), i, size=B)
            masks[:, i] = masks[rows, par]
            vis[:, i] = vis[rows, par]
        masks[:, i, i // 32] |= np.uint32(1 << (i % 32))
        vis[:, i] += 1
    flat.mask.copy_(torch.from_numpy(masks.view(np.int32)).to(dev))
    flat.m.fill_(P - 1)
    g = torch.Generator(device=dev).manual_seed(seed)
    mk = lambda *shape: torch.randn(*shape, device=dev, generator=g).to(torch.bfloat16)
    q, kt, vt = mk(B, P, Hq, D), mk(B, P, Hkv, D), mk(B, P, Hkv, D)
    kp, vp = mk(B, L, Hkv, D), mk(B, L, Hkv, D)
    out = torch.empty(B, P, Hq, D, dtype=torch.float32, device=dev)
    pairs = float(B * P * L + vis.sum())
    flops = 4.0 * D * Hq * pairs
    kv_bytes = (kp.numel() + vp.numel() + kt.numel() + vt.numel()) * 2
    res = {"kernel": "k_tree_attention (bf16 MFMA 32x32x16, fp32 accumulate)",
           "shape": {"B": B, "P": P, "prefix": L, "Hq": Hq, "Hkv": Hkv, "D": D},
           "flops_per_launch": flops, "launches": launches}
    for k, splits in enumerate(split_options):
        used, need = api.attention_splits(B, P, Hq, Hkv, L, splits or 0) if splits is not None else (1, 0)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        call = lambda: api.tree_attention(flat, q, kt, vt, out, k_pre=kp, v_pre=vp, splits=splits, ws=ws)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * launches)]
        for i in range(launches):
            ev[2 * i].record()
            call()
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        us = np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(launches)])
        tflops = flops / us.mean() / 1e6
        log(f"tree attention B={B} P={P} L={L} splits={splits} ({used}): {us.mean():.1f} us, "
            f"{tflops:.1f} TFLOP/s ({tflops / PEAK_BF16_TFLOPS:.3f} of peak)")
        one = {"splits": used, "avg_launch_us": round(float(us.mean()), 2), "tflops": round(float(tflops), 1),
               "roofline": {"bound": "mfma", "achieved": round(float(tflops), 1), "peak": PEAK_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(float(tflops / PEAK_BF16_TFLOPS), 4)},
               "kv_gbs": round(float(kv_bytes / us.mean() / 1e3), 1)}
        if k == 0:
            res.update(one)
        else:
            res.setdefault("variants", []).append(one)
        del ws
    del q, kt, vt, kp, vp, out
    torch.cuda.empty_cache()
    return res


def kv_commit_detail(api, dev, seed: int = 11, commits: int = 20) -> dict:
    """Committing the accepted path into a block-paged KV context at the B=64
    mixed shape: 16-token blocks, 8 key/value heads of 128, contexts of
    4096 + b % 16 tokens (so that tails are partly filled), accepted paths of
    0..10 draft tokens plus the root drawn at random from 129 flat positions.
    Commits (bookkeeping + copy kernels) are timed with events on the launch
    stream, eagerly one by one (host issue included) and as replays of a HIP
    graph that holds `commits` of them; bytes count each committed row read
    once and written once."""
    import torch
    B, P, Dp, Hkv, D, block = 64, 129, 10, 8, 128, 16
    per = 300                                        # blocks set aside per request
    kv = api.PagedKV(B, 320, B * per, block, Hkv, D, dev)
    base = 4096
    lens = torch.tensor([base + b % 16 for b in range(B)], dtype=torch.int32)
    used = (lens + block - 1) // block
    table = torch.full((B, 320), -1, dtype=torch.int32)
    ref = torch.zeros(B * per, dtype=torch.int32)
    taken = []
    for b in range(B):
        ids = torch.arange(b * per, b * per + int(used[b]), dtype=torch.int32)
        table[b, :len(ids)] = ids
        ref[ids.long()] = 1
        taken.append(ids)
    free = torch.tensor(sorted(set(range(B * per)) - set(torch.cat(taken).tolist()), reverse=True),
                        dtype=torch.int32)
    kv.table.copy_(table.to(dev)); kv.len.copy_(lens.to(dev)); kv.ref.copy_(ref.to(dev))
    kv.free_ids[:len(free)].copy_(free.to(dev)); kv.n_free.fill_(len(free))
    rng = np.random.default_rng(seed)
    g = torch.Generator(device=dev).manual_seed(seed)
    kt = torch.randn(B, P, Hkv, D, device=dev, generator=g).to(torch.bfloat16)
    vt = torch.randn(B, P, Hkv, D, device=dev, generator=g).to(torch.bfloat16)
    acc_all, path_all = [], []
    for _ in range(2 * commits + 3):
        acc = rng.integers(0, Dp + 1, size=B).astype(np.int32)
        path = np.full((B, Dp + 1), -1, np.int32)
        for b in range(B):
            path[b, :acc[b] + 1] = np.concatenate([[0], 1 + rng.permutation(P - 1)[:acc[b]]])
        acc_all.append(torch.from_numpy(acc).to(dev))
        path_all.append(torch.from_numpy(path).to(dev))
    status = torch.empty(B, dtype=torch.int32, device=dev)
    for i in range(3):
        kv.commit(acc_all[i], path_all[i], kt, vt, status)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * commits)]
    for i in range(commits):
        ev[2 * i].record()
        kv.commit(acc_all[3 + i], path_all[3 + i], kt, vt, status)
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    if not bool((status > 0).all()):
        raise RuntimeError("kv commit refused a request in the bench setup")
    us = np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(commits)])
    # the next `commits` commits captured once and replayed once
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(commits):
            kv.commit(acc_all[3 + commits + i], path_all[3 + commits + i], kt, vt, status)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    graph.replay()
    g1.record()
    torch.cuda.synchronize()
    if not bool((status > 0).all()):
        raise RuntimeError("kv commit refused a request in the bench setup")
    graph_us = g0.elapsed_time(g1) * 1e3 / commits
    tokens = float(np.mean([(a.cpu().numpy() + 1).sum() for a in acc_all[3:]]))
    nbytes = tokens * Hkv * D * 2 * 2 * 2            # k and v, read and written
    log(f"kv commit: {us.mean():.2f} us eager, {graph_us:.2f} us per commit in a graph, "
        f"{tokens:.0f} tokens")
    res = {"calls": "ddt_kv_commit (k_kv_plan + k_kv_copy)",
           "shape": {"B": B, "block": block, "Hkv": Hkv, "D": D, "context": "4096 + b % 16", "Dp": Dp},
           "eager_us": round(float(us.mean()), 2), "graph_us": round(float(graph_us), 2),
           "commits": commits, "tokens_per_commit": round(tokens, 1),
           "gbs_graph": round(float(nbytes / graph_us / 1e3), 2),
           "bound": "latency (two dependent launches; about 1.5 MB moved)"}
    del kv, kt, vt
    torch.cuda.empty_cache()
    return res


def cast_calibration_detail(w, run, ring, to_dev, dev, slots: int = 2, replays: int = 60,
                            save: Optional[str] = None) -> dict:
    """CAST cost tables measured on this GPU at the workload's batch and grid
    (proxy forwards of an 8B-class target and a one-layer draft head), then
    rounds of the same ring drafted and verified on those tables, replayed
    from HIP graphs like the headline rounds."""
    import torch
    from gen import configs, synth
    from dynamic_draft_tree_row_amd import api
    from dynamic_draft_tree_row_amd import cast_calibrate as CC
    cs = w.cast
    t0 = time.perf_counter()
    S_T, S_D = CC.measure_tables(w.B, cs.L, cs.M, cs.N, reps=3)
    cal_s = time.perf_counter() - t0
    log(f"cost tables measured in {cal_s:.1f} s: S_T[0][1] {S_T[0, 1]:.0f} us, S_D[0][1] {S_D[0, 1]:.0f} us")
    if save:
        CC.save_tables(save, S_T, S_D, B=w.B, L=cs.L, device=torch.cuda.get_device_name(dev))
    f = lambda a: torch.tensor(np.asarray(a, np.float32), device=dev)
    cast = api.CastParams(S_T=f(S_T), S_D=f(S_D), L=cs.L, C1=f([cs.C1] * w.D), C2=cs.C2,
                          C3=f([cs.C3] * w.B), R=cs.R, ctx_verify=w.prefix)
    ms, stats = [], []
    for r, slot in enumerate(ring[:slots]):
        run.draft(slot["draft"], slot["roots"], cast=cast)
        torch.cuda.synchronize()
        fk, fd, fs, ft = flat_layout(run, w.B)
        t_np = synth.target_arena(w, SEED, r, synth.draft_arena(w, SEED, r), fk, fd, fs, ft)
        m = dict(slot, target=to_dev(t_np))
        run.verify(m["target"], m["draft"], m["T"], m["U"])
        torch.cuda.synchronize()
        acc = run.accept_len.cpu().numpy()
        n_nodes, dep = run.tree.n_nodes.cpu().numpy(), run.tree.depth.cpu().numpy()
        depth = max(int(dep[b, :int(n_nodes[b])].max()) for b in range(w.B))
        stats.append(dict(widths=run.tree.widths.cpu().numpy().tolist(), m=run.m_out.cpu().numpy(),
                          accept=acc, depth=depth))
        ms.append(m)

    def one(m):
        run.draft(m["draft"], m["roots"], cast=cast)
        run.verify(m["target"], m["draft"], m["T"], m["U"])

    graphs = []
    for m in ms:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            one(m)
        graphs.append(g)
    for i in range(10):
        graphs[i % len(graphs)].replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(replays):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / replays
    cols = [n for n in (1, 2, 4, 8, 16, 32, 64, 128) if n <= cs.N]
    RT = synth.roofline_table(configs.PROXY_TARGET, w.B, cs.L, cs.M, cs.N)
    free = int(np.max(np.flatnonzero(S_T[0, 1:] <= 1.02 * S_T[0, 1]))) + 1
    return {
        "grid": {"B": w.B, "L": cs.L, "M": cs.M, "N": cs.N}, "calibration_s": round(cal_s, 1),
        "proxy": "target 32 x (d 4096, 32/8 heads of 128, FFN 14336) + LM head 128256; draft 1 layer of the same",
        "columns_n": cols,
        "S_T_us_ctx0": [round(float(S_T[0, n]), 1) for n in cols],
        "S_T_us_ctx_max": [round(float(S_T[-1, n]), 1) for n in cols],
        "S_D_us_ctx0": [round(float(S_D[0, n]), 1) for n in cols],
        "S_T_over_roofline_ctx0": [round(float(S_T[0, n] / RT[0, n]), 2) for n in cols],
        "target_tokens_within_2pct_of_one": free,
        "rounds_on_measured_tables": {
            "us_per_round_graph": round(us, 2),
            "widths": stats[0]["widths"][:stats[0]["depth"]], "depth": [s["depth"] for s in stats],
            "mean_m": round(float(np.mean([s["m"].mean() for s in stats])), 2),
            "mean_tau": round(float(np.mean([s["accept"].mean() + 1 for s in stats])), 3)},
    }


def graft_main(args, w, child) -> None:
    """The Graft workload: prune-then-graft rounds with the successor matrix.

    Checkpoint thresholds come from warm-up rounds drafted on the device
    without the gate (at each checkpoint depth, the 25th percentile of
    c_d = exp(max S at that depth) over the rows still active: the Graft
    review's warm-up calibration).  Every timed round starts from the initial
    successor matrix (reset outside the timed span, so that a replayed graph
    repeats its round and its target rows match its tree); rounds are
    graph-replayed and timed one by one with events, and `value` is
    1 / mean round time."""
    import torch
    from gen import configs, synth
    from dynamic_draft_tree_row_amd import _lib, api
    from dynamic_draft_tree_row_amd.round_driver import RoundRunner, RoundShape
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    lib = _lib.load()
    hip = Hip()
    gs = w.graft
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def to_dev(raw):
        if w.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(raw)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---- checkpoint thresholds from device warm-up rounds -------------------
    dck = max(gs.ck_depth)
    wck = configs.Workload(**{**w.__dict__, "D": dck, "graft": None})
    plain = RoundRunner(RoundShape(B=w.B, V=w.V, dtype=tdt, D=dck, K_e=w.K_e, K_n=w.K_n, m=w.m_max), dev)
    cds = []
    for r in range(args.tau_rounds):
        plain.draft(to_dev(synth.draft_arena(wck, SEED, 10_000 + r)),
                    torch.from_numpy(synth.root_tokens(w, SEED, 10_000 + r)).to(dev))
        torch.cuda.synchronize()
        S, dep, nn = plain.tree.S.cpu().numpy(), plain.tree.depth.cpu().numpy(), plain.tree.n_nodes.cpu().numpy()
        for b in range(w.B):
            n = int(nn[b])
            cds.append([float(np.exp(S[b, :n][dep[b, :n] == d].max())) for d in gs.ck_depth])
    del plain
    cds = np.array(cds)
    alive = np.ones(len(cds), bool)
    tau = []
    for k in range(len(gs.ck_depth)):
        tk = float(np.percentile(cds[alive, k], 25.0))
        tau.append(tk)
        alive &= cds[:, k] > tk
    gate = api.GraftGate(ck_depth=list(gs.ck_depth), tau=tau, k_draft=list(gs.k_draft), K_max=gs.K_max)
    log(f"checkpoint thresholds from {args.tau_rounds} warm-up rounds: {[round(x, 4) for x in tau]}")

    shape = RoundShape(B=w.B, V=w.V, dtype=tdt, D=w.D, K_e=w.K_e, K_n=w.K_n, m=w.m_max, prefix=w.prefix,
                       graft=True, tpl_depth=gs.tpl_depth, tpl_width=gs.tpl_width, k_succ=gs.k_succ)
    run = RoundRunner(shape, dev)
    M0_np = synth.succ_matrix0(w, SEED)
    M0 = torch.from_numpy(M0_np).to(dev)
    M = M0.clone()

    # ---- ring of rounds, inputs resident in HBM ------------------------------
    ring = []
    t0 = time.perf_counter()
    for r in range(args.ring):
        d_np = synth.draft_arena(w, SEED, r)
        slot = dict(draft=to_dev(d_np), roots=torch.from_numpy(synth.root_tokens(w, SEED, r)).to(dev),
                    T=torch.from_numpy(synth.temperatures(w, SEED, r)).to(dev),
                    U=torch.from_numpy(synth.uniforms(w, SEED, r)).to(dev))
        M.copy_(M0)
        run.draft(slot["draft"], slot["roots"], gate=gate, M=M)
        torch.cuda.synchronize()
        fk, fd, fs, ft = flat_layout(run, w.B)
        t_np = synth.target_arena(w, SEED, r, d_np, fk, fd, fs, ft, None, M0_np)
        slot["target"] = to_dev(t_np)
        if r == 0:
            slot.update(draft_np=d_np, target_np=t_np, roots_np=synth.root_tokens(w, SEED, r),
                        T_np=synth.temperatures(w, SEED, r), U_np=synth.uniforms(w, SEED, r))
        ring.append(slot)
    log(f"ring of {args.ring} Graft rounds generated in {time.perf_counter() - t0:.1f} s")

    def eager(slot):
        run.draft(slot["draft"], slot["roots"], gate=gate, M=M)
        run.verify(slot["target"], slot["draft"], slot["T"], slot["U"], M=M)

    ref, stats = [], []
    for slot in ring:
        M.copy_(M0)
        eager(slot)
        torch.cuda.synchronize()
        snap = snapshot(run)
        snap["M"] = M.clone()
        ref.append(snap)
        m = run.m_out.cpu().numpy()
        tree_esl, tree_dep = run.tree.eslot.cpu().numpy(), run.tree.depth.cpu().numpy()
        n_nodes = run.tree.n_nodes.cpu().numpy()
        rows_per_layer = [int(sum(((tree_esl[b, :int(n_nodes[b])] >= 0) &
                                   (tree_dep[b, :int(n_nodes[b])] == d - 1)).sum() for b in range(w.B)))
                          for d in range(1, w.D + 1)]
        stats.append(dict(rows_per_layer=rows_per_layer, verify_rows=int((m + 1).sum()),
                          k_draft=run.tree.k_draft.cpu().numpy().tolist(),
                          accept=run.accept_len.cpu().numpy().tolist()))
    graphs = []
    for slot in ring:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            eager(slot)
        graphs.append(g)
    for rep in range(3):
        for i, g in enumerate(graphs):
            M.copy_(M0)
            g.replay()
            torch.cuda.synchronize()
            snap = snapshot(run)
            snap["M"] = M.clone()
            if not same(snap, ref[i]):
                raise RuntimeError(f"graph replay {rep} of slot {i} differs from the eager round")
            M.copy_(M0)
            eager(ring[(i + 1) % len(ring)])
            torch.cuda.synchronize()
    log("graph replays match the eager rounds (successor matrix included)")

    K, W, R = args.steps, args.warmup, len(graphs)
    for i in range(W):
        M.copy_(M0)
        graphs[i % R].replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * K)]
    t0 = time.perf_counter()
    for i in range(K):
        M.copy_(M0)
        ev[2 * i].record()
        graphs[i % R].replay()
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    us = np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(K)])
    round_s = float(us.mean()) * 1e-6
    log(f"{K} Graft rounds: {us.mean():.1f} us/round (events per round; {wall_s * 1e6 / K:.1f} us wall "
        f"with the successor-matrix resets)")

    # ---- dominant kernel: the row reduction, kernel-stamped events -----------
    per_round = w.D + 1
    n_pairs = per_round * R * 4
    evs = hip.events(2 * n_pairs)
    arr = (C.c_void_p * len(evs))(*[e.value for e in evs])
    lib.ddt_set_reduce_events(arr, n_pairs)
    for slot in ring:
        M.copy_(M0)
        eager(slot)
    used = lib.ddt_set_reduce_events(None, 0)
    assert used == per_round * R, f"expected {per_round * R} timed launches, got {used}"
    torch.cuda.synchronize()
    ebytes = w.V * (2 if w.dtype == "bf16" else 4)
    durs, nbytes, vd, vb = [], [], [], []
    for k_s, st in enumerate(stats):
        for k in range(per_round):
            i = k_s * per_round + k
            d = hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) * 1e-3
            if k < w.D:
                durs.append(d); nbytes.append(st["rows_per_layer"][k] * ebytes)
            else:
                vd.append(d); vb.append(st["verify_rows"] * ebytes)
    durs, nbytes = np.array(durs), np.array(nbytes, dtype=np.float64)
    vd, vb = np.array(vd), np.array(vb, dtype=np.float64)
    achieved = nbytes.sum() / durs.sum() / 1e9
    log(f"expand layers: {len(durs)} launches, mean {durs.mean() * 1e6:.2f} us, {achieved:.0f} GB/s")
    expand_bytes = np.mean([sum(st["rows_per_layer"]) for st in stats]) * ebytes
    verify_bytes = np.mean([st["verify_rows"] for st in stats]) * ebytes
    out = {
        "metric": "draft-tree rounds/sec and logit HBM GB/s (% of roofline), Graft workload",
        "value": round(1.0 / round_s, 2), "unit": "rounds/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(round_s * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "V": w.V, "depth": w.D, "expand_topk": w.K_e,
                   "node_topk": w.K_n, "K_max": gs.K_max, "checkpoints": list(gs.ck_depth),
                   "k_draft": list(gs.k_draft), "tau": [round(x, 6) for x in tau],
                   "template": [gs.tpl_depth, gs.tpl_width], "k_succ": gs.k_succ,
                   "ring_rounds": R, "hip_graph": True,
                   "timing": "events around each replay; the successor matrix is reset before each"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "k_expand_layer<bf16,4> (one draft layer)",
                     "algorithmic_bytes_per_launch": round(float(nbytes.mean()), 1),
                     "avg_launch_us": round(float(durs.mean() * 1e6), 3), "launches": int(len(durs))},
        "logit_gbs": round((expand_bytes + verify_bytes) / round_s / 1e9, 1),
        "detail": {"round_us_p10_p50_p90": [round(float(np.percentile(us, q)), 2) for q in (10, 50, 90)],
                   "verify_reduction_launch": {
                       "kernel": "k_row_partial<bf16,8>, K = 8 (argmax and the refresh's top-8 of every verified row)",
                       "mb": round(float(vb.mean()) / 1e6, 3), "us": round(float(vd.mean() * 1e6), 3),
                       "gbs": round(float(vb.sum() / vd.sum() / 1e9), 1)},
                   "k_draft": stats[0]["k_draft"], "accept_len": stats[0]["accept"],
                   "mean_tau": round(float(np.mean([np.mean(st["accept"]) + 1 for st in stats])), 3)},
    }
    out["cpu_baseline"] = collect_oracle(child, {"tau": tau}) if child is not None else None
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle in a child process on one core
# ---------------------------------------------------------------------------

THREAD_ENV = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "NUMEXPR_NUM_THREADS",
              "BLIS_NUM_THREADS")


def resolve_workload(args):
    from gen import configs
    w = configs.C2
    if args.workload == "fixed":
        w = configs.Workload(**{**w.__dict__, "cast": None, "name": "eagle2_b8_v128256_bf16"})
    elif args.workload:
        w = configs.WORKLOADS[args.workload]
    if args.break_even and w.cast is not None:
        w = configs.Workload(**{**w.__dict__, "cast": configs.CastSpec(**configs.BREAK_EVEN)})
    return w


def spawn_oracle(args):
    """Start the CPU-baseline child before this process touches the GPU: a
    fresh interpreter with single-threaded BLAS, which builds ring slot 0's
    inputs itself, waits for one line on stdin (parameters the GPU side
    calibrated, e.g. Graft thresholds), pins itself to one core and times the
    oracle.  It never imports torch."""
    import subprocess
    env = dict(os.environ)
    for k in THREAD_ENV:
        env[k] = "1"
    cmd = [sys.executable, os.path.abspath(__file__), "--oracle-child", "--cpu-seconds", str(args.cpu_seconds)]
    if args.workload:
        cmd += ["--workload", args.workload]
    if args.break_even:
        cmd.append("--break-even")
    return subprocess.Popen(cmd, stdin=subprocess.PIPE, stdout=subprocess.PIPE, env=env, text=True)


def collect_oracle(child, params=None, timeout=900):
    """Send the go line (after every GPU measurement, so the child's timed
    span never overlaps this process's work) and read the child's JSON."""
    out, _ = child.communicate(json.dumps(params or {}) + "\n", timeout=timeout)
    lines = [l for l in out.splitlines() if l.startswith("{")]
    if child.returncode != 0 or not lines:
        raise RuntimeError(f"oracle baseline child failed (exit {child.returncode})")
    return json.loads(lines[-1])


def oracle_layout(trees, flats, P):
    """Per flat position of the oracle's own trees: key, depth, expand slot,
    token (how the synthetic target rows are laid out)."""
    B = len(flats)
    fk = np.full((B, P), -1, np.int64)
    fd = np.zeros((B, P), np.int32)
    fs = np.full((B, P), -1, np.int32)
    ft = np.full((B, P), -1, np.int32)
    for b, (t, f) in enumerate(zip(trees, flats)):
        for i, v in enumerate(f.node):
            if v >= 0:
                fk[b, i], fd[b, i], fs[b, i], ft[b, i] = t.key[v], t.depth[v], t.eslot[v], t.token[v]
    return fk, fd, fs, ft


def oracle_child(args) -> None:
    """The child's side of spawn_oracle: the oracle as it stands, single
    threaded, timed on ring slot 0 of the same workload for about
    args.cpu_seconds; input generation is outside the timed span."""
    from gen import synth
    from oracle import ddt_oracle as O
    w = resolve_workload(args)
    r = 0
    d_np = synth.draft_arena(w, SEED, r)
    roots = synth.root_tokens(w, SEED, r)
    T = synth.temperatures(w, SEED, r)
    U = synth.uniforms(w, SEED, r)
    cast = None
    if w.cast is not None:
        S_T, S_D = synth.cost_tables(w)
        cs = w.cast
        cast = dict(S_T=S_T, S_D=S_D, L=cs.L, M=cs.M, C1=[cs.C1] * w.D, C2=cs.C2, C3=[cs.C3] * w.B, R=cs.R)
    params = json.loads(sys.stdin.readline() or "{}")
    graft, M0, kw = None, None, {}
    if w.graft is not None:
        gs = w.graft
        graft = dict(ck_depth=tuple(gs.ck_depth), tau=list(params["tau"]), k_draft=tuple(gs.k_draft),
                     K_max=gs.K_max)
        M0 = synth.succ_matrix0(w, SEED)
        kw = dict(k_succ=gs.k_succ, tpl=(gs.tpl_depth, gs.tpl_width))
    held = {}

    def first_target(dr, flats):
        fk, fd, fs, ft = oracle_layout(dr.trees, flats, w.m_max + 1)
        held["t"] = synth.target_arena(w, SEED, r, d_np, fk, fd, fs, ft, None, M0)
        return held["t"]

    def one(tfn):
        O.run_round(B=w.B, V=w.V, dtype=w.dtype, D=w.D, K_e=w.K_e, K_n=w.K_n, m_max=w.m_max,
                    root_tok=roots, draft_raw=d_np, target_raw_fn=tfn, temperature=T, U=U,
                    prefix=w.prefix, cast=cast, graft=graft, M=None if M0 is None else M0.copy(),
                    proposal=w.proposal, **kw)

    one(first_target)
    core = min(os.sched_getaffinity(0))
    os.sched_setaffinity(0, {core})
    t0 = time.perf_counter()
    n = 0
    while True:
        one(lambda dr, flats: held["t"])
        n += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds:
            break
    cpu = "unknown cpu"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    print(json.dumps({
        "value": round(n / el, 3), "unit": "rounds/s", "cores": 1, "kind": "oracle",
        "core": core, "cpu": cpu, "host_cpus": os.cpu_count(),
        "threads_env": {k: os.environ.get(k) for k in THREAD_ENV[:3]},
        "sample": f"{n} rounds of {w.name} (ring slot 0, seed {SEED}; {el:.1f} s) in a child process "
                  f"pinned to core {core} with single-threaded BLAS, float64 numpy oracle; input "
                  f"generation excluded; started after every GPU measurement"}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--ring", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-attention", action="store_true",
                    help="only a few tree-attention launches and the calibration copy, for rocprofv3 --pmc")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the tree-attention measurement (the verify forward's MFMA kernel)")
    ap.add_argument("--tau-rounds", type=int, default=4,
                    help="Graft workload: warm-up rounds for the checkpoint thresholds")
    ap.add_argument("--save-tables", default=None, metavar="PATH",
                    help="write the measured CAST cost tables to PATH (.npz, cast_calibrate.load_tables)")
    ap.add_argument("--no-calibrate", action="store_true",
                    help="skip measuring the CAST cost tables on this GPU")
    ap.add_argument("--break-even", action="store_true",
                    help="CAST at the break-even thresholds C1=1, C2=0.1, C3=0.5")
    ap.add_argument("--pmc-run", action="store_true",
                    help="for rocprofv3 --pmc passes: eager rounds over the ring, then one "
                         "plain 256 MiB copy (torch.neg, fp32) whose counters scale the bytes")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn the two --pmc passes' counter CSVs into "
                         "profiles/k_expand_layer_traffic_<workload>.json")
    ap.add_argument("--oracle-child", action="store_true",
                    help="internal: the CPU-baseline child process (no GPU)")
    ap.add_argument("--workload", default=None,
                    help="profile another workload instead (e.g. eagle2_mixed_b64_v128256_bf16, "
                         "graft_b16_v152064_bf16; 'fixed' = the CAST shape with fixed EAGLE-2 widths)")
    args = ap.parse_args()
    if args.oracle_child:
        oracle_child(args)
        return
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.workload or "cast_b8_v128256_bf16", args.ring)
        return
    if args.gpus != 1:
        log("bench.py measures one GPU only: there is no multi-GPU path (batch rows "
            "would shard across GPUs, one process each; not built).")
        sys.exit(2)

    # the CPU baseline's child starts before this process touches the GPU
    child = None
    if not (args.no_cpu_baseline or args.pmc_run or args.pmc_attention):
        child = spawn_oracle(args)

    import torch
    from gen import configs, synth
    from dynamic_draft_tree_row_amd import _lib, api
    from dynamic_draft_tree_row_amd.round_driver import RoundRunner, RoundShape

    if args.pmc_attention:
        dev = torch.device("cuda", 0)
        torch.cuda.set_device(dev)
        _lib.load()
        tree_attention_detail(api, dev, launches=2)
        x = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        torch.neg(x, out=y)
        torch.cuda.synchronize()
        log(f"pmc attention run done: 5 launches, then a {CAL_BYTES >> 20} MiB copy (neg)")
        return

    w = resolve_workload(args)
    if w.graft is not None:
        return graft_main(args, w, child)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    lib = _lib.load()
    hip = Hip()
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def to_dev(raw):
        if w.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(raw)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).to(dev).view(torch.bfloat16)

    shape = RoundShape(B=w.B, V=w.V, dtype=tdt, D=w.D, K_e=w.K_e, K_n=w.K_n, m=w.m_max,
                       prefix=w.prefix)
    run = RoundRunner(shape, dev)
    cast_np, cast = None, None
    if w.cast is not None:
        S_T, S_D = synth.cost_tables(w)
        cs = w.cast
        cast_np = dict(S_T=S_T, S_D=S_D, L=cs.L, M=cs.M, C1=[cs.C1] * w.D, C2=cs.C2,
                       C3=[cs.C3] * w.B, R=cs.R)
        f = lambda a: torch.tensor(np.asarray(a, np.float32), device=dev)
        cast = api.CastParams(S_T=f(S_T), S_D=f(S_D), L=cs.L, C1=f(cast_np["C1"]), C2=cs.C2,
                              C3=f(cast_np["C3"]), R=cs.R, ctx_verify=w.prefix)

    # ---- inputs resident in HBM: a ring of rounds --------------------------
    ring = []
    t0 = time.perf_counter()
    for r in range(args.ring):
        d_np = synth.draft_arena(w, SEED, r)
        slot = dict(draft=to_dev(d_np), roots=torch.from_numpy(synth.root_tokens(w, SEED, r)).to(dev),
                    T=torch.from_numpy(synth.temperatures(w, SEED, r)).to(dev),
                    U=torch.from_numpy(synth.uniforms(w, SEED, r)).to(dev))
        run.draft(slot["draft"], slot["roots"], cast=cast)
        torch.cuda.synchronize()
        fk, fd, fs, ft = flat_layout(run, w.B)
        t_np = synth.target_arena(w, SEED, r, d_np, fk, fd, fs, ft)
        slot["target"] = to_dev(t_np)
        if r == 0:
            slot.update(draft_np=d_np, target_np=t_np, roots_np=synth.root_tokens(w, SEED, r),
                        T_np=synth.temperatures(w, SEED, r), U_np=synth.uniforms(w, SEED, r))
        ring.append(slot)
    ring_bytes = sum(s["draft"].numel() * s["draft"].element_size() +
                     s["target"].numel() * s["target"].element_size() for s in ring)
    log(f"ring of {args.ring} rounds, {ring_bytes / 1e9:.2f} GB of logits, "
        f"generated in {time.perf_counter() - t0:.1f} s")

    def eager(slot):
        run.draft(slot["draft"], slot["roots"], cast=cast)
        run.verify(slot["target"], slot["draft"], slot["T"], slot["U"])

    # eager reference outputs and per-round statistics
    ref, stats = [], []
    for slot in ring:
        eager(slot)
        torch.cuda.synchronize()
        ref.append(snapshot(run))
        tree_esl = run.tree.eslot.cpu().numpy()
        tree_dep = run.tree.depth.cpu().numpy()
        n_nodes = run.tree.n_nodes.cpu().numpy()
        rows_per_layer = []
        for d in range(1, w.D + 1):
            rows = 0
            for b in range(w.B):
                n = int(n_nodes[b])
                rows += int(((tree_esl[b, :n] >= 0) & (tree_dep[b, :n] == d - 1)).sum())
            rows_per_layer.append(rows)
        m = run.m_out.cpu().numpy()
        acc = run.accept_len.cpu().numpy()
        stats.append(dict(rows_per_layer=rows_per_layer, verify_rows=int((m + 1).sum()),
                          walk_rows=int((acc + 1).sum()), m=m.tolist(), accept=acc.tolist(),
                          widths=run.tree.widths.cpu().numpy().tolist(),
                          depth=int(max(d for d, r in enumerate(rows_per_layer, 1) if r > 0))))

    if args.pmc_run:
        for _ in range(2):
            for slot in ring:
                eager(slot)
        torch.cuda.synchronize()
        x = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        torch.neg(x, out=y)
        torch.cuda.synchronize()
        log(f"pmc run done: {2 * len(ring)} eager rounds, then a {CAL_BYTES >> 20} MiB copy (neg)")
        return

    # ---- capture one graph per ring slot -----------------------------------
    graphs = []
    for slot in ring:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            eager(slot)
        graphs.append(g)
    # every replay must reproduce the eager result, with eager work in between
    for rep in range(3):
        for i, g in enumerate(graphs):
            g.replay()
            torch.cuda.synchronize()
            if not same(snapshot(run), ref[i]):
                raise RuntimeError(f"graph replay {rep} of slot {i} differs from the eager round")
            eager(ring[(i + 1) % len(ring)])
            torch.cuda.synchronize()
    log("graph replays match the eager rounds")

    # ---- timed region ------------------------------------------------------
    K, W, R = args.steps, args.warmup, len(graphs)
    for i in range(W):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(K):
        graphs[i % R].replay()
    e1.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = wall_s * 1e3 / K
    log(f"{K} rounds: {ms_per_step * 1e3:.1f} us/round wall, {gpu_ms * 1e3 / K:.1f} us/round GPU events")

    # eager (no graph) rounds for reference
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ne = max(20, K // 4)
    for i in range(ne):
        eager(ring[i % R])
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t0) * 1e6 / ne

    # ---- dominant kernel: the expand layer ----------------------------------
    # Per round: D expand-layer launches (k_expand_layer: the vocabulary
    # reduction of the layer's draft rows, their merge and children, the
    # frontier and CAST's rule), then the verify reduction (k_row_partial,
    # K = 1 over every flat row).  The library launches them with start/stop
    # events that the runtime stamps at the kernel's own start and end
    # (ddt_set_reduce_events).  Events inside a captured graph are not valid
    # timing events on this runtime, so the launches are timed in eager
    # rounds of the same ring slots, on the same stream.
    per_round = w.D + 1
    n_pairs = per_round * R * 4
    evs = hip.events(2 * n_pairs)
    arr = (C.c_void_p * len(evs))(*[e.value for e in evs])
    lib.ddt_set_reduce_events(arr, n_pairs)
    for slot in ring:
        eager(slot)
    used = lib.ddt_set_reduce_events(None, 0)
    assert used == per_round * R, f"expected {per_round * R} timed launches, got {used}"
    torch.cuda.synchronize()
    ebytes = w.V * (2 if w.dtype == "bf16" else 4)
    exp_d, exp_b, ver_d, ver_b = [], [], [], []
    for s_i, st in enumerate(stats):
        for k in range(per_round):
            i = s_i * per_round + k
            d = hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) * 1e-3
            if k < w.D:
                exp_d.append(d); exp_b.append(st["rows_per_layer"][k] * ebytes)
            else:
                ver_d.append(d); ver_b.append(st["verify_rows"] * ebytes)
    exp_d, exp_b = np.array(exp_d), np.array(exp_b, dtype=np.float64)
    ver_d, ver_b = np.array(ver_d), np.array(ver_b, dtype=np.float64)
    achieved = exp_b.sum() / exp_d.sum() / 1e9
    log(f"expand layers: {len(exp_d)} launches, mean {exp_d.mean() * 1e6:.2f} us, "
        f"{exp_b.mean() / 1e6:.2f} MB/launch, {achieved:.0f} GB/s; verify reduction: "
        f"{ver_d.mean() * 1e6:.2f} us, {ver_b.mean() / 1e6:.2f} MB/launch")

    # ---- per-round spread: replays bracketed one by one ----------------------
    nspread = 100
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nspread)]
    for i in range(nspread):
        sev[2 * i].record()
        graphs[i % R].replay()
        sev[2 * i + 1].record()
    torch.cuda.synchronize()
    per_round_us = np.array([sev[2 * i].elapsed_time(sev[2 * i + 1]) * 1e3 for i in range(nspread)])

    # ---- the same reduction over all of a round's draft rows in one launch ----
    # (streaming efficiency without the layer-to-layer dependence)
    arena = ring[0]["draft"]
    flat_rows = arena.reshape(-1, arena.shape[-2], w.V)          # [D*B][R][V]
    nrows = flat_rows.shape[0] * flat_rows.shape[1]
    ws_b = torch.empty(api.workspace_bytes(nrows, w.V, tdt, w.K_n), dtype=torch.uint8, device=dev)
    nb = 10
    bev = hip.events(2 * nb)
    barr = (C.c_void_p * len(bev))(*[e.value for e in bev])
    api.row_topk(flat_rows, w.K_n, ws_b)
    torch.cuda.synchronize()
    lib.ddt_set_reduce_events(barr, nb)
    for _ in range(nb):
        api.row_topk(flat_rows, w.K_n, ws_b)
    lib.ddt_set_reduce_events(None, 0)
    torch.cuda.synchronize()
    bd = np.array([hip.elapsed_ms(bev[2 * i], bev[2 * i + 1]) * 1e-3 for i in range(nb)])
    batched_bytes = nrows * w.V * (2 if w.dtype == "bf16" else 4)
    batched_gbs = batched_bytes / bd.mean() / 1e9
    del ws_b

    # ---- algorithmic logit bytes per round ----------------------------------
    expand_bytes = np.mean([sum(s["rows_per_layer"]) for s in stats]) * ebytes
    walk_bytes = np.mean([s["walk_rows"] for s in stats]) * ebytes
    allrow_bytes = np.mean([s["verify_rows"] for s in stats]) * ebytes
    round_s = ms_per_step * 1e-3
    logit_gbs = (expand_bytes + walk_bytes) / round_s / 1e9

    out = {
        "metric": "draft-tree rounds/sec and logit HBM GB/s (% of roofline) at B=8, V=128256",
        "value": round(1.0 / round_s, 2),
        "unit": "rounds/s",
        "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "V": w.V, "depth": w.D, "expand_topk": w.K_e,
                   "node_topk": w.K_n, "m": w.m, "verify": w.verify,
                   "cast": ({"C1": w.cast.C1, "C2": w.cast.C2, "C3": w.cast.C3, "R": w.cast.R,
                             "cost": "c_k = 0.02k + 1.0"} if w.cast else None),
                   "prefix": w.prefix,
                   "ring_rounds": R, "ring_gb": round(ring_bytes / 1e9, 3), "hip_graph": True},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic_per_launch(w.name),
                     "kernel": "k_expand_layer<bf16,4> (one draft layer: vocabulary reduction of the "
                               "layer's draft rows, row merge and children, frontier, CAST rule)",
                     "algorithmic_bytes_per_launch": round(float(exp_b.mean()), 1),
                     "algorithmic_bytes": "the layer's live draft rows x V x 2 bytes (every draft row once)",
                     "avg_launch_us": round(float(exp_d.mean() * 1e6), 3),
                     "launches": int(len(exp_d)),
                     "timing": "kernel-stamped HIP start/stop events per launch (hipExtLaunchKernelGGL), "
                               "eager rounds; layers after CAST's depth stop are launched too and "
                               "count with 0 bytes"},
        "logit_gbs": round(logit_gbs, 1),
        "logit_frac_of_peak": round(logit_gbs / PEAK_HBM_GBS, 4),
        "detail": {
            "gpu_event_us_per_round": round(gpu_ms * 1e3 / K, 2),
            "round_us_p10_p50_p90": [round(float(np.percentile(per_round_us, q)), 2) for q in (10, 50, 90)],
            "verify_reduction_launch": {
                # short chunks below 512 flat rows, as the library launches them
                "kernel": f"k_row_partial<{w.dtype},{8 if w.B * (w.m_max + 1) >= 512 else 4}>, K = 1",
                "label": "greedy verify reduces every flat row (sum of m_b + 1 rows) to its argmax; "
                         "the accepted walk needs only sum of accept_len + 1 of them",
                "mb": round(float(ver_b.mean()) / 1e6, 3), "us": round(float(ver_d.mean() * 1e6), 3),
                "gbs": round(float(ver_b.sum() / ver_d.sum() / 1e9), 1),
                "frac": round(float(ver_b.sum() / ver_d.sum() / 1e9 / PEAK_HBM_GBS), 4)},
            "rows_batched_reduction": {"rows": int(nrows), "mb": round(batched_bytes / 1e6, 1),
                                       "us": round(float(bd.mean() * 1e6), 2),
                                       "gbs": round(float(batched_gbs), 1),
                                       "frac": round(float(batched_gbs / PEAK_HBM_GBS), 4)},
            "eager_us_per_round": round(eager_us, 2),
            "expand_mb_per_round": round(expand_bytes / 1e6, 3),
            "verify_walk_mb_per_round": round(walk_bytes / 1e6, 3),
            "verify_allrows_mb_per_round": round(allrow_bytes / 1e6, 3),
            "allrow_logit_gbs": round((expand_bytes + allrow_bytes) / round_s / 1e9, 1),
            "cast_widths": stats[0]["widths"][:stats[0]["depth"]],
            "depth": [s["depth"] for s in stats],
            "m_per_row": stats[0]["m"], "accept_len": stats[0]["accept"],
            "mean_tau": round(float(np.mean([np.mean(s["accept"]) + 1 for s in stats])), 3),
        },
    }
    out["detail"]["expand_layer_b64"] = expand_b64_detail(api, lib, hip, dev)
    if not args.no_attention:
        out["detail"]["tree_attention"] = tree_attention_detail(api, dev)
        # the CAST workload's verify shape (8 requests, 61 flat positions) over
        # a 4096-token context: too few tiles to fill the device on their own
        out["detail"]["tree_attention_b8"] = tree_attention_detail(api, dev, B=8, P=61, L=4096,
                                                                   split_options=(0, None))
        out["detail"]["kv_commit"] = kv_commit_detail(api, dev)
    if w.cast is not None and not args.no_calibrate:
        out["detail"]["cast_calibration"] = cast_calibration_detail(w, run, ring, to_dev, dev,
                                                                    save=args.save_tables)
    out["cpu_baseline"] = collect_oracle(child) if child is not None else None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
