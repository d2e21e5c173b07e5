#!/usr/bin/env python3
"""Throughput of the DeepSeek-V4 hybrid compressed attention layer on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:
  * chunked prefill: a 4096-token chunk appended to a 524288-token context,
    batch 2, through an interleaved CSA/HCA/CSA/HCA stack (compression of the
    chunk, window rows, indexer scores, top-k 1024, sparse / dense MQA
    attention with a 128-token window and sinks, 64 heads x 512);
  * decode at 1M context: one new token per sequence, batch 8, through one
    CSA layer (262144 cached entries, top-k 1024) and one HCA layer (8192).
value = query tokens per second = (2 * 4096 + 8) / step time; a query token
is counted once per layer stack. Inputs are seeded synthetic tensors already
resident in HBM when timing starts.

Prints one JSON line. `roofline` covers the dominant kernel, the bf16 MFMA
indexer scoring of the prefill CSA layers, timed with HIP events on its
stream over the timed region; `roofline_decode` does the same for the
HBM-bound decode scoring, `roofline_decode_step` for the whole decode step
and `decode_attention` for its two attention calls. `configs` times the
single-layer prefill configurations (HCA 16K, CSA 64K) outside the step.
`cpu_baseline` times the CPU oracle on a bounded sample of the same
workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "query-tokens/s for CSA/HCA layer at 1M ctx (prefill+decode); % HBM/MFMA peak"
PEAK_BF16_FLOPS = 2.5e15
PEAK_FP8_FLOPS = 5.0e15
PEAK_FP4_FLOPS = 10.1e15
PEAK_HBM_BYTES = 8.0e12
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# The stored counter figures describe the kernels built from these sources; a change to any of
# them makes the figures stale (reported as null).
CSRC = os.path.join("compressed_sparse_kv_02_amd", "csrc")
COPY_PROBE_BYTES = 1 << 30   # plain copy used to calibrate FETCH_SIZE / WRITE_SIZE
CU_COUNT, SIMD_PER_CU, XCD_COUNT = 256, 4, 8


def sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, CSRC)
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def load_traffic():
    """Stored per-kernel counter figures, or None when absent or stale."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        tr = json.load(f)
    if tr.get("sources_sha256") != sources_digest():
        return None
    return tr


def traffic_of(tr, kernel: str):
    """HBM bytes per launch of the stored kernel entry whose name starts with `kernel` (most dispatches)."""
    if not tr:
        return None
    ents = [e for e in tr.get("kernels", []) if e["kernel"].startswith(kernel)]
    if not ents:
        return None
    return max(ents, key=lambda e: e["dispatches"]).get("hbm_bytes_per_launch")


def write_traffic(fetch_csv: str, write_csv: str, mfma_csv=None) -> None:
    """Turn rocprofv3 --pmc counter_collection.csv files of `bench.py --copy-probe` into per-kernel
    figures: HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, KiB per dispatch) and, from a third
    run with SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE, the matrix cores' busy share.

    Each byte counter is scaled by bytes / counter of the calibration copy (a fp32 negation of
    COPY_PROBE_BYTES in, COPY_PROBE_BYTES out), so the figures are in the units the copy defines:
    bytes that crossed from HBM (or the memory-side cache) into L2 and back. GRBM_GUI_ACTIVE is
    summed over the XCDs and SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs, so the busy share is
    busy / (GUI / XCDs * CUs * SIMDs per CU); GUI / XCDs over the dispatch's duration is its clock.
    """
    import csv
    import re
    import statistics

    def short(n):
        return re.sub(r"\(.*$", "", re.sub(r"^void ", "", n)).replace("cskv::", "")

    def per_kernel(path):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                key = (short(r["Kernel_Name"]), int(r["Grid_Size"]))
                ent = vals.setdefault(key, {})
                ent.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                ent.setdefault("_dur_" + r["Counter_Name"], []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9)
        return vals

    out = {"sources_sha256": sources_digest(), "copy_probe_bytes": COPY_PROBE_BYTES}
    runs = {"FETCH_SIZE": per_kernel(fetch_csv), "WRITE_SIZE": per_kernel(write_csv)}
    for counter, vals in runs.items():
        copy = [v for (name, grid), cs in vals.items() if "neg_kernel" in name for v in cs.get(counter, [])]
        assert copy, f"no calibration copy dispatch for {counter}"
        out[f"{counter}_factor"] = COPY_PROBE_BYTES / (statistics.median(copy) * 1024.0)
    mf = per_kernel(mfma_csv) if mfma_csv else {}
    kernels = []
    ours = ("attn_", "indexer_", "topk_", "compress_", "gemm_", "quantize_")
    keys = sorted({k for run in runs.values() for k in run if k[0].startswith(ours)})
    for key in keys:
        ent = {"kernel": key[0], "grid": key[1]}
        for counter, vals in runs.items():
            vs = vals.get(key, {}).get(counter)
            if vs:
                ent[f"{counter}_bytes"] = statistics.mean(vs) * 1024.0 * out[f"{counter}_factor"]
                ent["dispatches"] = len(vs)
        if "FETCH_SIZE_bytes" in ent and "WRITE_SIZE_bytes" in ent:
            ent["hbm_bytes_per_launch"] = ent["FETCH_SIZE_bytes"] + ent["WRITE_SIZE_bytes"]
        m = mf.get(key, {})
        if m.get("SQ_VALU_MFMA_BUSY_CYCLES") and m.get("GRBM_GUI_ACTIVE"):
            gui = statistics.mean(m["GRBM_GUI_ACTIVE"]) / XCD_COUNT
            ent["mfma_busy"] = statistics.mean(m["SQ_VALU_MFMA_BUSY_CYCLES"]) / (gui * CU_COUNT * SIMD_PER_CU)
            ent["clock_ghz"] = gui / statistics.mean(m["_dur_GRBM_GUI_ACTIVE"]) / 1e9
            ent["duration_us_under_counters"] = statistics.mean(m["_dur_GRBM_GUI_ACTIVE"]) * 1e6
        kernels.append(ent)
    out["kernels"] = kernels
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def traffic_summary() -> None:
    """The stored counter figures as a markdown table (one line per kernel and grid)."""
    with open(TRAFFIC_FILE) as f:
        tr = json.load(f)
    print(f"FETCH_SIZE factor {tr['FETCH_SIZE_factor']:.3f}, WRITE_SIZE factor {tr['WRITE_SIZE_factor']:.3f} "
          f"(the {tr['copy_probe_bytes'] >> 20} MiB copy); sources sha256 {tr['sources_sha256'][:16]}")
    print()
    print("| kernel | grid | dispatches | HBM read MB | HBM write MB | MFMA busy | clock GHz |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for e in sorted(tr["kernels"], key=lambda e: -e.get("hbm_bytes_per_launch", 0)):
        # GRBM_GUI_ACTIVE also counts the dispatch's set-up and drain: below ~200 us that inflates
        # the clock and deflates the busy share, so those two are shown for long dispatches only
        long_run = e.get("duration_us_under_counters", 0) >= 200
        mb = f"{100 * e['mfma_busy']:.1f}%" if "mfma_busy" in e and (long_run or e["mfma_busy"] == 0) else "-"
        ck = f"{e['clock_ghz']:.2f}" if "clock_ghz" in e and long_run else "-"
        print(f"| `{e['kernel']}` | {e['grid']} | {e.get('dispatches', 0)} | {e.get('FETCH_SIZE_bytes', 0) / 1e6:.1f} "
              f"| {e.get('WRITE_SIZE_bytes', 0) / 1e6:.1f} | {mb} | {ck} |")


# what each (kernel, grid) of the profiled bench run is, for the kernel-time table
KERNEL_ROLES = {
    ("indexer_score_mfma<2, 8>", 524288): "chunk CSA scoring (2 x 4096 queries, 131072 keys)",
    ("attn_mfma<512, 4, 2, -1, 1>", 2097152): "chunk HCA attention (8192 queries, 64 heads)",
    ("attn_mfma<512, 4, 1, -1, 2>", 16777216): "64K CSA attention",
    ("attn_mfma<512, 4, 1, -1, 2>", 2097152): "chunk CSA attention (8192 queries, 64 heads)",
    ("indexer_score_mfma<2, 8>", 4194304): "64K CSA scoring",
    ("topk_select", 4194304): "chunk CSA top-k (8192 rows)",
    ("topk_select", 33554432): "64K CSA top-k (65536 rows)",
    ("attn_mfma<512, 2, 4, -1, 1>", 2097152): "16K HCA attention (32 heads, 4 queries per workgroup)",
    ("indexer_score_stream<2, 8>", 262144): "decode CSA scoring (8 x 262144 keys)",
    ("compress_block_kernel<bf16, 8, 1, 8>", 32768): "chunk HCA compression (2 x 32 entries of 128 rows)",
    ("compress_rows_kernel<bf16, 8, 1, 4>", 131072): "chunk window rows (2 x 4096)",
    ("compress_pool8_kernel<bf16, 8, 1>", 1048576): "64K CSA KV compression (16384 entries)",
    ("attn_mfma<512, 4, 1, -1, 1>", 65536): "decode HCA attention (32 splits)",
    ("compress_pool8_kernel<bf16, 8, 1>", 131072): "chunk CSA KV compression (2 x 1024 entries)",
    ("compress_rows_kernel<bf16, 8, 1, 4>", 1048576): "64K CSA window rows",
    ("topk_bm_select", 4096): "decode top-k: select",
    ("attn_mfma<512, 4, 1, -1, 1>", 36864): "decode CSA attention (18 splits)",
    ("compress_block_kernel<bf16, 8, 1, 8>", 65536): "16K HCA compression (128 entries)",
    ("compress_rows_kernel<bf16, 8, 1, 1>", 512): "decode window rows (8)",
    ("attn_merge<bf16>", 131072): "decode split merge",
    ("compress_pool8_kernel<bf16, 8, 1>", 32768): "chunk CSA indexer-key compression",
    ("compress_pool8_kernel<bf16, 8, 1>", 262144): "64K CSA indexer-key compression",
    ("compress_rows_kernel<bf16, 8, 1, 4>", 262144): "16K HCA window rows",
}


def kernel_table(trace_csv: str) -> None:
    """Per-dispatch kernel times of a rocprofv3 --kernel-trace csv as a markdown table, one line per
    library kernel and launch grid (work-items); other kernels (torch's input synthesis) are left out."""
    import collections
    import csv
    import re

    def short(name):
        name = re.sub(r"^void ", "", name).replace("cskv::", "")
        return re.sub(r"\(.*\)$", "", name).strip()

    times = collections.defaultdict(list)
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            n = short(r["Kernel_Name"])
            if not n.startswith(("indexer_", "attn_", "topk_", "compress_", "quantize_", "gemm_")):
                continue
            g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) if "Grid_Size_X" in r \
                else int(r["Grid_Size"])
            times[(n, g)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    total = sum(sum(v) for v in times.values())
    print("| kernel | grid (work-items) | what | dispatches | avg (us) | min (us) | max (us) | % of our kernels' time |")
    print("|---|---:|---|---:|---:|---:|---:|---:|")
    for (n, g), v in sorted(times.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{n}` | {g} | {KERNEL_ROLES.get((n, g), '-')} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} "
              f"| {max(v):.1f} | {100 * sum(v) / total:.2f} |")


def visible_pairs(L) -> int:
    """Sum over the call's queries of the visible compressed entries (indexer (t, s) pairs)."""
    tot = 0
    for j in range(L.T):
        tot += min(L.N, (L.pos0 + j + 1) // L.m)
    return tot * L.batch


def indexer_flops(L) -> float:
    return 2.0 * L.HI * L.dI * visible_pairs(L)


def decode_score_bytes(L) -> float:
    """The decode scoring's own bytes: indexer keys read once, queries and head weights (the
    fp32 score rows it hands to the top-k are a by-product of splitting the step, not counted)."""
    return L.batch * (L.N * L.dI * 2 + L.HI * L.dI * 2 + L.HI * 4)


def decode_step_bytes(decode) -> float:
    """Algorithmic HBM bytes of one decode step (every layer of `decode`), each byte once: queries
    and outputs, the new token's raw and prepared window row, the w window rows, lse; CSA: indexer
    keys, indexer queries and weights, the k selected entries and their indices; HCA: every
    visible entry."""
    tot = 0
    for L in decode:
        e, b = 2, L.batch
        tot += b * (2 * L.H * L.d * e + 2 * L.d * e + L.w * L.d * e + L.H * 4)
        if L.kind == "csa":
            tot += b * (L.N * L.dI * e + L.HI * L.dI * e + L.HI * 4 + L.k * L.d * e + 2 * L.k * 4)
        else:
            tot += b * min(L.N, (L.pos0 + 1) // L.m) * L.d * e
    return tot


def attn_pairs(L) -> int:
    """(query, key) pairs of the layer call's attention: selected (CSA, at most k) or visible (HCA)
    compressed entries plus the window rows, summed over queries."""
    tot = 0
    for j in range(L.T):
        t = L.pos0 + j
        V = min(L.N, (t + 1) // L.m)
        tot += (min(L.k, V) if L.kind == "csa" else V) + min(L.w, t + 1)
    return tot * L.batch


def attn_flops(L) -> float:
    return 4.0 * L.H * L.d * attn_pairs(L)   # S = Q K^T and O = P V, 2 H d each per pair


def prefill_layer_bytes(L) -> float:
    """Algorithmic HBM bytes of one prefill layer call read or written once: queries, outputs, lse,
    raw and prepared window rows, compressor streams and new entries; CSA adds the indexer streams,
    indexer queries and weights, the indexer keys and the selected indices. The gathered entry rows
    of the attention are counted once per distinct entry (the cache), not per gather."""
    e, b, T = 2, L.batch, L.T
    tot = b * T * (2 * L.H * L.d * e + L.H * 4 + 3 * L.d * e)
    if L.kind == "csa":
        tot += b * T * 4 * (L.d + L.dI) * e + b * (L.n_new + L.N) * (L.d + L.dI) * e
        tot += b * T * (L.HI * L.dI * e + L.HI * 4 + L.k * 4)
    else:
        tot += b * T * 2 * L.d * e + b * (L.n_new + L.N) * L.d * e
    return tot


def cpu_baseline(prefill, decode, tp, td, budget_s: float):
    """Time the CPU oracle on a bounded sample of the step's workload.

    Prefill: per layer, the whole chunk's compression and window rows for sequence 0 (amortised
    over the chunk's tokens), then query rows drawn from a seeded stratified order (the chunk's
    first rows, block and window edges, then a shuffle) until the layer's share of the budget is
    spent (at least 4 rows). Decode: every one of the 8 sequences' tokens through both layers.
    The rate weights the per-token times by the step's prefill and decode token counts.
    """
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import cskv_oracle as O

    def np64(t):
        return t.detach().float().cpu().numpy().astype(np.float64)

    def layer_inputs(L, t, b):
        kv = np64(t["cache.kv"][b])
        ik = np64(t["cache.ik"][b]) if L.kind == "csa" else None
        win = np64(t["win"][b])
        h = {k: np64(v[b]) for k, v in t.items() if k.split(".")[-1] in ("Ca", "Cb", "Za", "Zb", "C", "Z",
                                                                          "prevCb", "prevZb") and v.dim() == 3}
        hb = {k: np64(v) for k, v in t.items() if k.endswith(".B")}
        return kv, ik, win, h, hb

    def compress(L, t, b, kv, ik, win, h, hb):
        if L.n_new:
            if L.kind == "csa":
                kv[L.n_cached:] = O.csa_compress(h["kv.Ca"], h["kv.Cb"], h["kv.Za"], h["kv.Zb"], hb["kv.B"], L.m,
                                                 L.pos0, h.get("kv.prevCb"), h.get("kv.prevZb"), True,
                                                 rope_dims=L.rope_dims)
                ik[L.n_cached:] = O.csa_compress(h["ik.Ca"], h["ik.Cb"], h["ik.Za"], h["ik.Zb"], hb["ik.B"], L.m,
                                                 L.pos0, h.get("ik.prevCb"), h.get("ik.prevZb"))
            else:
                kv[L.n_cached:] = O.hca_compress(h["kv.C"], h["kv.Z"], hb["kv.B"], L.m, L.pos0, True,
                                                 rope_dims=L.rope_dims)
        win[L.win_cached:] = O.prepare_window(np64(t["win_raw"][b]), L.pos0, rope_dims=L.rope_dims)

    def row(L, t, b, r, kv, ik, win, sink):
        q = np64(t["q"][b, r:r + 1])
        idx = None
        if L.kind == "csa":
            I = O.indexer_scores(np64(t["qI"][b, r:r + 1]), np64(t["wI"][b, r:r + 1]), ik, L.pos0 + r, L.m)[0]
            idx = O.topk_row(I, O.visible(L.pos0 + r, L.m, L.N), L.k)[None]
        O.attention(q, kv, win, L.win_pos0, L.pos0 + r, L.m, L.w, idx=idx, sink=sink, rope_dims=L.rope_dims)

    share = budget_s * 0.8 / len(prefill)
    per_tok_pre, n_rows = 0.0, []
    for L, t in zip(prefill, tp):
        kv, ik, win, h, hb = layer_inputs(L, t, 0)
        sink = np64(t["sink"])
        t0 = time.perf_counter()
        compress(L, t, 0, kv, ik, win, h, hb)
        per_tok_pre += (time.perf_counter() - t0) / L.T
        order = [0, 1, 3, 4, L.m - 1, L.m, L.w - 1, L.w, L.T - 1]
        order += [int(r) for r in np.random.default_rng(5).permutation(L.T) if r not in order]
        spent, n = 0.0, 0
        for r in order:
            t0 = time.perf_counter()
            row(L, t, 0, r, kv, ik, win, sink)
            spent += time.perf_counter() - t0
            n += 1
            if n >= 4 and spent >= share:
                break
        per_tok_pre += spent / n
        n_rows.append(n)
    per_tok_dec, n_dec_rows = 0.0, 0
    for L, t in zip(decode, td):
        spent = 0.0
        for b in range(L.batch):
            kv, ik, win, h, hb = layer_inputs(L, t, b)
            t0 = time.perf_counter()
            compress(L, t, b, kv, ik, win, h, hb)     # the new token's window row
            row(L, t, b, 0, kv, ik, win, np64(t["sink"]))
            spent += time.perf_counter() - t0
        per_tok_dec += spent / L.batch
        n_dec_rows += L.batch
    n_pre_tok = prefill[0].batch * prefill[0].T
    n_dec_tok = decode[0].batch
    value = (n_pre_tok + n_dec_tok) / (n_pre_tok * per_tok_pre + n_dec_tok * per_tok_dec)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": value, "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"sequence 0 of the prefill chunk: whole-chunk compression and window rows of each of "
                       f"the 4 layers amortised over the chunk, plus {n_rows} query rows per layer (stratified, "
                       f"as many as a {budget_s:.0f} s budget allows); all {decode[0].batch} decode tokens "
                       f"through the CSA and HCA decode layers; per-token times weighted by the step's "
                       f"{n_pre_tok} prefill + {n_dec_tok} decode tokens"),
            "rows_timed": {"prefill_per_layer": n_rows, "decode": n_dec_rows},
            "seconds_per_prefill_token": per_tok_pre, "seconds_per_decode_token": per_tok_dec}


PHASES = ("compress", "score", "topk", "attend")


def run_phases(L, t, rec=None, ev=None):
    """One layer call, phase by phase (compression + window rows, indexer scores, top-k,
    attention); with `rec`, each phase is bracketed by HIP events on the launch stream."""
    from compressed_sparse_kv_02_amd import layer as LY
    for name, fn in zip(PHASES, (LY.compress_step, LY.score_step, LY.topk_step, LY.attend_step)):
        if rec is None:
            fn(L, t)
        else:
            a, b = ev(), ev()
            a.record()
            fn(L, t)
            b.record()
            rec.setdefault(name, []).append((a, b))


def mean_ms(pairs) -> float:
    return sum(a.elapsed_time(b) for a, b in pairs) / len(pairs) if pairs else 0.0


def prefill_config_rows(reps: int = 3):
    """The two single-layer prefill configurations, each a whole layer call (compression, window
    rows, scoring, top-k, attention), timed phase by phase with HIP events: HCA prefill of 16384
    tokens (32 heads, m' = 128; HBM-bound) and CSA prefill of 65536 tokens (64 heads, k = 1024,
    rank-256 indexer queries; the indexer and the attention against the bf16 matrix peak)."""
    import torch
    from compressed_sparse_kv_02_amd import layer as LY

    out = {}
    for name, L in (("hca_prefill_16k", LY.hca_prefill_16k()), ("csa_prefill_64k", LY.csa_prefill_64k())):
        t = LY.make_inputs(L)
        run_phases(L, t)
        torch.cuda.synchronize()
        pool, rec = [], {}

        def ev():
            e = torch.cuda.Event(enable_timing=True)
            pool.append(e)
            return e
        for _ in range(reps):
            run_phases(L, t, rec, ev)
        torch.cuda.synchronize()
        ph = {k: mean_ms(v) for k, v in rec.items()}
        total = sum(ph.values())
        by = prefill_layer_bytes(L)
        af, pairs = attn_flops(L), attn_pairs(L)
        ent = {"layer": f"{L.kind} batch {L.batch} x {L.T} tokens, {L.H} heads x {L.d}, m={L.m}, window {L.w}"
                        + (f", k={L.k}, indexer {L.HI} x {L.dI}" if L.kind == "csa" else ""),
               "ms_per_call": total, "query_tokens_per_s": L.batch * L.T / (total / 1e3), "phases_ms": ph,
               "hbm": {"algorithmic_bytes": by, "achieved_GBps": by / (total / 1e3) / 1e9,
                       "frac": by / (total / 1e3) / PEAK_HBM_BYTES},
               "attention": {"algorithmic_flops": af, "tflops": af / (ph["attend"] / 1e3) / 1e12,
                             "frac_mfma": af / (ph["attend"] / 1e3) / PEAK_BF16_FLOPS,
                             "gathered_rows_bytes": pairs * L.d * 2,
                             "gather_GBps": pairs * L.d * 2 / (ph["attend"] / 1e3) / 1e9}}
        if L.kind == "csa":
            fl = indexer_flops(L)
            ent["indexer"] = {"algorithmic_flops": fl, "tflops": fl / (ph["score"] / 1e3) / 1e12,
                              "frac_mfma": fl / (ph["score"] / 1e3) / PEAK_BF16_FLOPS}
        out[name] = ent
        del t
        torch.cuda.empty_cache()
    return out


def lowp_indexer_rows(prefill, tp, decode, td, reps: int = 3):
    """Low-precision indexer scoring (FP8 E4M3, FP4 E2M1 with row scales; MX-FP4 / MX-FP8: the same
    values with one E8M0 scale per 32) on the timed step's CSA inputs. Per key row the scales take 4 bytes
    in every format (one fp32, or four E8M0 bytes at dI = 128).

    The indexer keys and queries of prefill layer 0 and of the decode CSA layer
    are quantised once (outside the timing); the scoring entry point is then
    timed with HIP events on the launch stream, reps launches each.
    """
    import torch
    from compressed_sparse_kv_02_amd import binding as B

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    out = {}
    for fmt, quant, score, peak, bits in (("fp8", B.quantize_fp8, B.indexer_scores_fp8, PEAK_FP8_FLOPS, 8),
                                          ("fp4", B.quantize_fp4, B.indexer_scores_fp4, PEAK_FP4_FLOPS, 4),
                                          ("mxfp4", B.quantize_mxfp4, B.indexer_scores_mxfp4, PEAK_FP4_FLOPS, 4),
                                          ("mxfp8", B.quantize_mxfp8, B.indexer_scores_mxfp8, PEAK_FP8_FLOPS, 8)):
        res = {}
        for tag, L, t in (("prefill", prefill[0], tp[0]), ("decode", decode[0], td[0])):
            kc, ks = quant(t["cache.ik"])
            qc, qs = quant(t["qI"])
            # the keys a step appends (one per sequence at decode) are quantised as they arrive
            new_keys = (t["cache.ik"][:, L.n_cached:] if L.n_new else t["cache.ik"][:, :1]).contiguous()
            ms = timed(lambda: score(qc, qs, t["wI"], kc, ks, L.pos0, L.m, scores=t["ws.scores"]))
            q_ms = timed(lambda: quant(new_keys))
            kern = f"indexer_score_lowp_{'mfma' if tag == 'prefill' else 'stream'}<{fmt}>"
            if tag == "prefill":
                fl = indexer_flops(L)
                ent = {"kernel": kern, "bound": "mfma", "avg_launch_ms": ms, "achieved": fl / (ms / 1e3) / 1e12,
                       "peak": peak / 1e12, "unit": "TFLOP/s", "algorithmic_flops_per_launch": fl}
            else:
                by = L.batch * (L.N * (L.dI * bits // 8 + 4) + L.HI * L.dI * bits // 8 + 2 * L.HI * 4 + L.N * 4)
                ent = {"kernel": kern, "bound": "hbm", "avg_launch_ms": ms, "achieved": by / (ms / 1e3) / 1e9,
                       "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s", "algorithmic_bytes_per_launch": by}
            ent["frac"] = ent["achieved"] / ent["peak"]
            ent["quantize_new_keys_ms"] = q_ms
            res[tag] = ent
            del kc, ks, qc, qs
        out[f"indexer_{fmt}"] = res
    return out


def decode_step_lowp_rows(decode, td, bf16_ms: float, steps: int = 20):
    """The whole decode step with the CSA layer's indexer on MX-FP4 or MX-FP8 keys (the pages' V4
    and V3.2 indexer precisions): the key cache is stored quantised (quantised once, outside the
    timing, as a cache written in that format would be), and each step quantises its queries, then
    scores and selects with indexer_topk_mx*; everything else is the bf16 step's. Timed with
    events around `steps` whole steps."""
    import torch
    from compressed_sparse_kv_02_amd import binding as B
    from compressed_sparse_kv_02_amd import layer as LY

    out = {}
    Lc, tc = decode[0], td[0]
    for fmt, quant, topk, bits in (("mxfp4", B.quantize_mxfp4, B.indexer_topk_mxfp4, 4),
                                   ("mxfp8", B.quantize_mxfp8, B.indexer_topk_mxfp8, 8)):
        kc, ks = quant(tc["cache.ik"])
        ws = torch.empty(max(16, B.indexer_workspace_bytes(Lc.batch, Lc.T, Lc.N, Lc.HI, Lc.k,
                                                             B.MXFP4 if bits == 4 else B.MXFP8)),
                         dtype=torch.uint8, device=tc["q"].device)

        def step():
            LY.compress_step(Lc, tc)
            qc, qs = quant(tc["qI"])
            topk(qc, qs, tc["wI"], kc, ks, Lc.pos0, Lc.m, Lc.k, out=tc["idx"], workspace=ws)
            LY.attend_step(Lc, tc)
            for L, t in zip(decode[1:], td[1:]):
                LY.run_layer(L, t)

        for _ in range(3):
            step()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            step()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        # the bf16 step's bytes with the indexer keys and queries at the format's size (codes plus
        # one E8M0 scale byte per 32 values)
        per = lambda n: n * bits // 8 + n // 32
        by = decode_step_bytes(decode) - Lc.batch * (Lc.N + Lc.HI) * Lc.dI * 2 + \
            Lc.batch * (Lc.N + Lc.HI) * per(Lc.dI)
        out[f"decode_step_{fmt}_indexer"] = {
            "ms": ms, "query_tokens_per_s": Lc.batch / (ms / 1e3), "algorithmic_bytes": by,
            "achieved_GBps": by / (ms / 1e3) / 1e9, "frac_hbm": by / (ms / 1e3) / PEAK_HBM_BYTES,
            "bf16_step_ms": bf16_ms}
        del kc, ks, ws
    LY.select_step(Lc, tc)  # leave the bf16 selection in place
    return out


def kv_fp8_attention_rows(prefill, tp, decode, td, reps: int = 3):
    """Attention over FP8 + BF16 stored entries beside the bf16 cache, same inputs.

    Each layer's compressed cache is quantised once (outside the timing); both
    attention calls are timed with HIP events on the launch stream.
    """
    import torch
    from compressed_sparse_kv_02_amd import binding as B
    from compressed_sparse_kv_02_amd import layer as LY

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    res = {}
    for tag, L, t in (("prefill_csa", prefill[0], tp[0]), ("prefill_hca", prefill[1], tp[1]),
                      ("decode_csa", decode[0], td[0]), ("decode_hca", decode[1], td[1])):
        rows, sc = B.quantize_kv_fp8(t["cache.kv"], L.rope_dims)
        mode = B.CSA if L.kind == "csa" else B.HCA
        kw = dict(k=L.k, apply_q_norm=True, rope_dims=L.rope_dims, rope_on_output=True, out=t["out"], lse=t["lse"])
        idx = t.get("idx") if L.kind == "csa" else None
        if L.decode:
            kw.update(n_splits=L.n_splits, workspace=t["ws.dec"])
            call = lambda kv, s_: B.compressed_attn_decode(mode, t["q"], kv, idx, t["win"], L.win_pos0, t["sink"],
                                                           L.pos0, L.m, L.w, kv_scale=s_, **kw)
        else:
            # HCA: the entries are widened once per call into a workspace allocated here, outside the timing
            nws = int(B.lib().cskv_prefill_kv8_workspace_size(mode, L.batch, L.N, L.d))
            ws8 = torch.empty(nws, dtype=torch.uint8, device=t["q"].device) if nws else None
            call = lambda kv, s_: B.compressed_attn_prefill(mode, t["q"], kv, idx, t["win"], L.win_pos0, t["sink"],
                                                            L.pos0, L.m, L.w, kv_scale=s_,
                                                            **(dict(kw, workspace=ws8) if s_ is not None else kw))
        ms16 = timed(lambda: call(t["cache.kv"], None))
        ms8 = timed(lambda: call(rows, sc))
        res[tag] = {"bf16_cache_ms": ms16, "fp8_cache_ms": ms8,
                    "entry_bytes": {"bf16": 2 * L.d, "fp8": B.kv_fp8_row_bytes(L.d, L.rope_dims)}}
        del rows, sc
    LY.attend_step(prefill[0], tp[0])  # leave the step's own outputs in place
    return res


# Projection shapes. The pages give none: the latent rank follows the low-rank indexer-query
# reading (r = 256); the output groups G = 8 of 8 heads, d_g = 1024 and the model width
# D = 4096 are assumptions of this benchmark, named as such in its output.
PROJ_R, PROJ_G, PROJ_DG, PROJ_D = 256, 8, 1024, 4096


def projection_rows(prefill, reps: int = 3):
    """The projections around the attention for the prefill chunk's tokens (batch x chunk):
    attention queries c^Q W^Q, indexer queries c^Q W^QI, and the grouped output projection.
    Seeded synthetic latents and weights; each call timed with HIP events on the launch stream."""
    import torch
    from compressed_sparse_kv_02_amd import binding as B
    from compressed_sparse_kv_02_amd.synth import normal_device

    L = prefill[0]
    T = L.batch * L.T

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def row(ms, flops, nbytes):
        tf = flops / (ms / 1e3) / 1e12
        gb = nbytes / (ms / 1e3) / 1e9
        mfma_bound = flops / PEAK_BF16_FLOPS >= nbytes / PEAK_HBM_BYTES
        ent = {"avg_launch_ms": ms, "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes,
               "tflops": tf, "gbps": gb, "bound": "mfma" if mfma_bound else "hbm"}
        ent["frac"] = tf / (PEAK_BF16_FLOPS / 1e12) if mfma_bound else gb / (PEAK_HBM_BYTES / 1e9)
        return ent

    r, G, dg, D = PROJ_R, PROJ_G, PROJ_DG, PROJ_D
    cq = normal_device(61, "proj.cq", (T, r))
    out = {"shapes": {"tokens": T, "latent_rank": r, "groups": G, "group_dim": dg, "model_dim": D,
                      "assumed": "r, G, d_g and D are not on the pages"}}
    for tag, n_out in (("query_proj", L.H * L.d), ("indexer_query_proj", L.HI * L.dI)):
        W = normal_device(61, f"proj.{tag}", (r, n_out), r ** -0.5)
        dst = torch.empty(T, n_out, dtype=torch.bfloat16, device=cq.device)
        ms = timed(lambda: B.lowrank_proj(cq, W, out=dst))
        out[tag] = row(ms, 2 * T * r * n_out, 2 * (T * r + r * n_out + T * n_out))
        del W, dst
    kin = (L.H // G) * L.d
    o = normal_device(61, "proj.o", (T, L.H, L.d))
    Wg = normal_device(61, "proj.Wg", (G, kin, dg), kin ** -0.5)
    Wo = normal_device(61, "proj.Wo", (G * dg, D), (G * dg) ** -0.5)
    mid = torch.empty(T, G, dg, dtype=torch.bfloat16, device=o.device)
    y = torch.empty(T, D, dtype=torch.bfloat16, device=o.device)
    ms = timed(lambda: B.grouped_out_proj(o, Wg, Wo, mid=mid, out=y))
    fl = 2 * T * G * kin * dg + 2 * T * G * dg * D
    by = 2 * (T * L.H * L.d + G * kin * dg + 2 * T * G * dg + G * dg * D + T * D)
    out["grouped_out_proj"] = row(ms, fl, by)
    out["kernel"] = "gemm_bf16 (256 x 256 tiles, v_mfma_f32_32x32x16_bf16)"
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-configs", action="store_true", help="skip the 16K HCA and 64K CSA prefill lines")
    ap.add_argument("--no-next-rows", action="store_true", help="skip the low-precision / projection lines")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB copy (counter calibration for --write-traffic)")
    ap.add_argument("--write-traffic", nargs="+", metavar="CSV",
                    help="write profiles/traffic.json from rocprofv3 --pmc runs (FETCH_SIZE csv, WRITE_SIZE "
                         "csv[, SQ_VALU_MFMA_BUSY_CYCLES + GRBM_GUI_ACTIVE csv]) and exit")
    ap.add_argument("--traffic-summary", action="store_true", help="print profiles/traffic.json as a table and exit")
    ap.add_argument("--kernel-table", metavar="CSV",
                    help="print the kernel times of a rocprofv3 --kernel-trace csv as a table and exit")
    args = ap.parse_args()
    if args.kernel_table:
        kernel_table(args.kernel_table)
        return
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.traffic_summary:
        traffic_summary()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one MI355X; runs on more than one GPU are not supported "
              "(the layer has no sharded path here).", file=sys.stderr)
        sys.exit(2)

    import torch
    from compressed_sparse_kv_02_amd import layer as LY

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    prefill = LY.chunked_prefill_512k()
    decode = LY.decode_1m()
    tp = [LY.make_inputs(L) for L in prefill]
    td = [LY.make_inputs(L) for L in decode]
    torch.cuda.synchronize()

    ev_pool = []

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        ev_pool.append(e)
        return e

    def scored(L, t, rec, key):
        """One layer call; with rec, the scoring kernel is bracketed by events (rec[key])."""
        LY.compress_step(L, t)
        if rec is not None and L.kind == "csa":
            a, b = ev(), ev()
            a.record()
            LY.score_step(L, t)
            b.record()
            rec[key].append((a, b))
        else:
            LY.score_step(L, t)
        LY.topk_step(L, t)
        LY.attend_step(L, t)

    def step(rec=None):
        for L, t in zip(prefill, tp):
            scored(L, t, rec, "pre_score")
        if rec is not None:
            m = ev()
            m.record()
            rec["mid"].append(m)
        for L, t in zip(decode, td):
            scored(L, t, rec, "dec_score")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rec = {"pre_score": [], "dec_score": [], "mid": []}
    starts = []
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        s = ev()
        s.record()
        starts.append(s)
        step(rec)
    t_end.record()
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps
    if args.copy_probe:
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    pre_ms = sum(starts[i].elapsed_time(rec["mid"][i]) for i in range(args.steps)) / args.steps
    dec_ms = ms - pre_ms
    n_pre = prefill[0].batch * prefill[0].T
    n_dec = decode[0].batch
    value = (n_pre + n_dec) / (ms / 1e3)
    # phase breakdown from a separate pass (events around every phase add host gaps between the
    # short decode kernels, so the timed steps above bracket only the scoring kernels)
    prec = {"pre": [{} for _ in prefill], "dec": [{} for _ in decode]}
    for _ in range(3):
        for i, (L, t) in enumerate(zip(prefill, tp)):
            run_phases(L, t, prec["pre"][i], ev)
        for i, (L, t) in enumerate(zip(decode, td)):
            run_phases(L, t, prec["dec"][i], ev)
    torch.cuda.synchronize()
    phases = {
        "prefill": [dict(layer=f"{L.kind}{i}", **{k: mean_ms(v) for k, v in r.items()})
                    for i, (L, r) in enumerate(zip(prefill, prec["pre"]))],
        "decode": [dict(layer=L.kind, **{k: mean_ms(v) for k, v in r.items()}) for L, r in zip(decode, prec["dec"])],
        "note": "separate pass, every phase bracketed by events (the decode figures include launch gaps)",
    }

    score_ms = mean_ms(rec["pre_score"])
    fl = indexer_flops(prefill[0])
    achieved = fl / (score_ms / 1e3) / 1e12
    tr = load_traffic()
    traffic = traffic_of(tr, "indexer_score_mfma<2, 8>")
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                "frac": achieved * 1e12 / PEAK_BF16_FLOPS, "traffic": traffic,
                "kernel": "indexer_score_mfma<2,8> (prefill CSA layers)", "avg_launch_ms": score_ms,
                "algorithmic_flops_per_launch": fl}
    dscore_ms = mean_ms(rec["dec_score"])
    db = decode_score_bytes(decode[0])
    dach = db / (dscore_ms / 1e3) / 1e9
    dtraffic = traffic_of(tr, "indexer_score_stream<2, 8>")
    roofline_dec = {"bound": "hbm", "achieved": dach, "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                    "frac": dach * 1e9 / PEAK_HBM_BYTES, "traffic": dtraffic,
                    "kernel": "indexer_score_stream<2,8> (decode CSA layer)", "avg_launch_ms": dscore_ms,
                    "algorithmic_bytes_per_launch": db}
    sb = decode_step_bytes(decode)
    roofline_step = {"bound": "hbm", "achieved": sb / (dec_ms / 1e3) / 1e9, "peak": PEAK_HBM_BYTES / 1e9,
                     "unit": "GB/s", "frac": sb / (dec_ms / 1e3) / PEAK_HBM_BYTES, "ms": dec_ms,
                     "algorithmic_bytes": sb,
                     "what": "the whole decode step (window rows, scoring, top-k, CSA and HCA attention)"}
    dattn = {}
    for L, r in zip(decode, prec["dec"]):
        e = 2
        keys = min(L.k, L.N) if L.kind == "csa" else min(L.N, (L.pos0 + 1) // L.m)
        by = L.batch * ((keys + L.w) * L.d * e + 2 * L.H * L.d * e + L.H * 4)
        am = mean_ms(r["attend"])
        dattn[L.kind] = {"bound": "hbm", "ms": am, "algorithmic_bytes": by,
                         "achieved_GBps": by / (am / 1e3) / 1e9, "frac": by / (am / 1e3) / PEAK_HBM_BYTES}

    out = {
        "metric": METRIC, "value": value, "unit": "query-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "chunked_prefill_512k_b2_4layer+decode_1m_b8",
                   "prefill": "batch 2 x 4096-token chunk at pos 524288, layers CSA/HCA/CSA/HCA, "
                              "64 heads x 512 (RoPE 64), CSA m=4 k=1024, HCA m'=128, window 128, "
                              "indexer 64 x 128",
                   "decode": "batch 8 x 1 token at pos 1048576, CSA (262144 entries, k=1024) + HCA (8192)",
                   "query_tokens_per_step": n_pre + n_dec},
        "parts": {"prefill_ms": pre_ms, "prefill_query_tokens_per_s": n_pre / (pre_ms / 1e3),
                  "decode_ms": dec_ms, "decode_query_tokens_per_s": n_dec / (dec_ms / 1e3),
                  "phases_ms": phases},
        "roofline": roofline,
        "roofline_decode": roofline_dec,
        "roofline_decode_step": roofline_step,
        "decode_attention": dattn,
        "cpu_baseline": None,
    }
    if not args.no_configs:
        out["configs"] = prefill_config_rows()
    if not args.no_next_rows:
        out["next_rows"] = dict(lowp_indexer_rows(prefill, tp, decode, td), projections=projection_rows(prefill),
                                kv_fp8_attention=kv_fp8_attention_rows(prefill, tp, decode, td),
                                **decode_step_lowp_rows(decode, td, dec_ms))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(prefill, decode, tp, td, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
