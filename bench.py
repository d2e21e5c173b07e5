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
HBM-bound decode scoring. `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload on this host's cores.
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
# Sources whose kernels the stored counter figures describe; a change to any of
# them makes those figures stale (reported as null).
TRAFFIC_SOURCES = ("compressed_sparse_kv_02_amd/csrc/indexer.hip", "compressed_sparse_kv_02_amd/csrc/indexer.h",
                   "compressed_sparse_kv_02_amd/csrc/device_common.h")
COPY_PROBE_BYTES = 1 << 30   # plain copy used to calibrate FETCH_SIZE / WRITE_SIZE


def sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic():
    """Stored HBM bytes per launch of the scoring kernels, or None when absent or stale."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        tr = json.load(f)
    if tr.get("sources_sha256") != sources_digest():
        return None
    return tr


def write_traffic(fetch_csv: str, write_csv: str) -> None:
    """Turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, WRITE_SIZE, KiB per
    dispatch) of `bench.py --copy-probe` into HBM bytes per launch of the scoring kernels.

    Each counter is scaled by bytes / counter of the calibration copy (a fp32 negation of
    COPY_PROBE_BYTES in, COPY_PROBE_BYTES out), so the figures are in the units the copy
    defines: bytes that crossed from HBM (or the memory-side cache) into L2 and back.
    """
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault((r["Kernel_Name"], int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
        return vals

    out = {"sources_sha256": sources_digest(), "copy_probe_bytes": COPY_PROBE_BYTES}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_kernel(path, counter)
        copy = [v for (name, grid), vs in vals.items() if "neg_kernel" in name for v in vs]
        assert copy, f"no calibration copy dispatch in {path}"
        kib = statistics.median(copy)
        factor = COPY_PROBE_BYTES / (kib * 1024.0)
        out[f"{counter}_copy_kib"] = kib
        out[f"{counter}_factor"] = factor
        for tag, tmpl in (("prefill", "indexer_score_mfma<2, 8>"), ("decode", "indexer_score_stream<2, 8>")):
            vs = [v for (name, grid), xs in vals.items() if tmpl in name for v in xs]
            assert vs, f"no {tmpl} dispatch in {path}"
            ent = out.setdefault(f"indexer_score_mfma_{tag}", {})
            ent[f"{counter}_kib_mean"] = statistics.mean(vs)
            ent[f"{counter}_dispatches"] = len(vs)
            ent[f"{counter}_bytes"] = statistics.mean(vs) * 1024.0 * factor
    for tag in ("prefill", "decode"):
        ent = out[f"indexer_score_mfma_{tag}"]
        ent["hbm_bytes_per_launch"] = ent["FETCH_SIZE_bytes"] + ent["WRITE_SIZE_bytes"]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def visible_pairs(L) -> int:
    """Sum over the call's queries of the visible compressed entries (indexer (t, s) pairs)."""
    tot = 0
    for j in range(L.T):
        tot += min(L.N, (L.pos0 + j + 1) // L.m)
    return tot * L.batch


def indexer_flops(L) -> float:
    return 2.0 * L.HI * L.dI * visible_pairs(L)


def decode_score_bytes(L) -> float:
    # indexer keys read once, queries + weights, fp32 score rows written
    return L.batch * (L.N * L.dI * 2 + L.HI * L.dI * 2 + L.HI * 4 + L.N * 4)


def cpu_baseline(prefill, decode, tp, td, budget_s: float):
    """Time the CPU oracle on a bounded sample: whole-chunk compression plus a few query rows."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import cskv_oracle as O

    def np64(t):
        return t.detach().float().cpu().numpy().astype(np.float64)

    def layer_rows(L, t, rows, compress: bool):
        b = 0
        kv = np64(t["cache.kv"][b])
        ik = np64(t["cache.ik"][b]) if L.kind == "csa" else None
        win = np64(t["win"][b])
        h = {k: np64(v[b]) for k, v in t.items() if k.split(".")[-1] in ("Ca", "Cb", "Za", "Zb", "C", "Z",
                                                                          "prevCb", "prevZb") and v.dim() == 3}
        hb = {k: np64(v) for k, v in t.items() if k.endswith(".B")}
        q = {r: np64(t["q"][b, r:r + 1]) for r in rows}
        qI = {r: (np64(t["qI"][b, r:r + 1]), np64(t["wI"][b, r:r + 1])) for r in rows} if L.kind == "csa" else {}
        raw = np64(t["win_raw"][b])
        sink = np64(t["sink"])
        t0 = time.perf_counter()
        if compress and L.n_new:
            if L.kind == "csa":
                kv[L.n_cached:] = O.csa_compress(h["kv.Ca"], h["kv.Cb"], h["kv.Za"], h["kv.Zb"], hb["kv.B"], L.m,
                                                 L.pos0, h.get("kv.prevCb"), h.get("kv.prevZb"), True,
                                                 rope_dims=L.rope_dims)
                ik[L.n_cached:] = O.csa_compress(h["ik.Ca"], h["ik.Cb"], h["ik.Za"], h["ik.Zb"], hb["ik.B"], L.m,
                                                 L.pos0, h.get("ik.prevCb"), h.get("ik.prevZb"))
            else:
                kv[L.n_cached:] = O.hca_compress(h["kv.C"], h["kv.Z"], hb["kv.B"], L.m, L.pos0, True,
                                                 rope_dims=L.rope_dims)
            win[L.win_cached:] = O.prepare_window(raw, L.pos0, rope_dims=L.rope_dims)
        t_comp = time.perf_counter() - t0
        t0 = time.perf_counter()
        for r in rows:
            idx = None
            if L.kind == "csa":
                I = O.indexer_scores(qI[r][0], qI[r][1], ik, L.pos0 + r, L.m)[0]
                idx = O.topk_row(I, O.visible(L.pos0 + r, L.m, L.N), L.k)[None]
            O.attention(q[r], kv, win, L.win_pos0, L.pos0 + r, L.m, L.w, idx=idx, sink=sink,
                        rope_dims=L.rope_dims)
        return t_comp, time.perf_counter() - t0

    # prefill: per-sequence chunk compression amortised over the chunk's tokens, plus n rows
    n_pre = 4 if budget_s >= 10 else 2
    rows = [0, 1365, 2730, 4095][:n_pre]
    per_tok_pre = 0.0
    for L, t in zip(prefill, tp):
        tc, tr = layer_rows(L, t, rows, compress=True)
        per_tok_pre += tc / L.T + tr / len(rows)
    per_tok_dec = 0.0
    for L, t in zip(decode, td):
        tc, tr = layer_rows(L, t, [0], compress=True)  # decode: prepares the new token's window row
        per_tok_dec += tc + tr
    n_pre_tok = prefill[0].batch * prefill[0].T
    n_dec_tok = decode[0].batch
    value = (n_pre_tok + n_dec_tok) / (n_pre_tok * per_tok_pre + n_dec_tok * per_tok_dec)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": value, "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"sequence 0: whole-chunk compression of all 4 prefill layers amortised over the "
                       f"chunk, plus {len(rows)} query rows through the 4-layer stack and 1 decode token "
                       f"through the CSA+HCA decode layers; per-token times weighted by the step's "
                       f"{n_pre_tok} prefill + {n_dec_tok} decode tokens"),
            "seconds_per_prefill_token": per_tok_pre, "seconds_per_decode_token": per_tok_dec}


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
            call = lambda kv, s_: B.compressed_attn_prefill(mode, t["q"], kv, idx, t["win"], L.win_pos0, t["sink"],
                                                            L.pos0, L.m, L.w, kv_scale=s_, **kw)
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
    out["kernel"] = "gemm_bf16 (128 x 128 tiles, v_mfma_f32_32x32x16_bf16)"
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB copy (counter calibration for --write-traffic)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs and exit")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
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

    def step(rec=None):
        marks = {}
        for L, t in zip(prefill, tp):
            LY.compress_step(L, t)
            if L.kind == "csa" and rec is not None:
                a, b = ev(), ev()
                a.record()
                LY.score_step(L, t)
                b.record()
                rec["pre_score"].append((a, b))
            else:
                LY.score_step(L, t)
            LY.topk_step(L, t)
            LY.attend_step(L, t)
        if rec is not None:
            m = ev()
            m.record()
            rec["mid"].append(m)
        for L, t in zip(decode, td):
            LY.compress_step(L, t)
            if L.kind == "csa" and rec is not None:
                a, b = ev(), ev()
                a.record()
                LY.score_step(L, t)
                b.record()
                rec["dec_score"].append((a, b))
            else:
                LY.score_step(L, t)
            LY.topk_step(L, t)
            LY.attend_step(L, t)

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

    score_ms = sum(a.elapsed_time(b) for a, b in rec["pre_score"]) / len(rec["pre_score"])
    fl = indexer_flops(prefill[0])
    achieved = fl / (score_ms / 1e3) / 1e12
    tr = load_traffic() or {}
    traffic = tr.get("indexer_score_mfma_prefill", {}).get("hbm_bytes_per_launch")
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                "frac": achieved * 1e12 / PEAK_BF16_FLOPS, "traffic": traffic,
                "kernel": "indexer_score_mfma<2,8> (prefill CSA layers)", "avg_launch_ms": score_ms,
                "algorithmic_flops_per_launch": fl}
    dscore_ms = sum(a.elapsed_time(b) for a, b in rec["dec_score"]) / len(rec["dec_score"])
    db = decode_score_bytes(decode[0])
    dach = db / (dscore_ms / 1e3) / 1e9
    dtraffic = tr.get("indexer_score_mfma_decode", {}).get("hbm_bytes_per_launch")
    roofline_dec = {"bound": "hbm", "achieved": dach, "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                    "frac": dach * 1e9 / PEAK_HBM_BYTES, "traffic": dtraffic,
                    "kernel": "indexer_score_stream<2,8> (decode CSA layer)", "avg_launch_ms": dscore_ms,
                    "algorithmic_bytes_per_launch": db}

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
                  "decode_ms": dec_ms, "decode_query_tokens_per_s": n_dec / (dec_ms / 1e3)},
        "roofline": roofline,
        "roofline_decode": roofline_dec,
        "cpu_baseline": None,
        "next_rows": dict(lowp_indexer_rows(prefill, tp, decode, td), projections=projection_rows(prefill),
                          kv_fp8_attention=kv_fp8_attention_rows(prefill, tp, decode, td)),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(prefill, decode, tp, td, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
