"""Benchmark: compressed keys scored per second on the Llama-3.1-8B-shaped
decode-logits workload (batch 1, 32 query heads / 8 KV heads, head_dim 128,
32768-token context, 3-bit keys), one MI355X.

A step is one decode-step scoring pass: prepare the 32 queries (q' = R q,
p = S q' and the scoring operands), then score them against the resident
compressed K cache of that step.  Steps rotate over enough distinct
(cache, query, logits) buffer sets that the 256 MB Infinity Cache cannot hold
them, so every step streams its compressed keys from HBM.

Prints ONE JSON line (rank 0).  The dominant kernel is the logits kernel; its
roofline entry divides the algorithmic bytes of one launch (compressed
records read + prepared queries read + logits written) by the average launch
duration measured with HIP events on the stream the kernel runs on.

Other stages of the path (encode, 4-bit logits, fused decode attention at
128K context, search) are timed once each and reported under "stages".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed keys scored/sec + effective HBM GB/s (% of peak), 3-bit, 32K ctx"
PEAK_HBM_GBS = 8000.0
ROOFLINE_LAUNCHES = 200
INFINITY_CACHE = 256 * 2 ** 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--bits", type=int, default=3)
    ap.add_argument("--no-stages", action="store_true", help="skip the per-stage timings")
    ap.add_argument("--only-stages", action="store_true",
                    help="run only the per-stage timings (one JSON line of stages; for kernel-trace profiles)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-stage-sparse-v", action="store_true", help="skip the Sparse V decode stage")
    ap.add_argument("--no-stage-search", action="store_true", help="skip the 1M x 1536 encode and search stages")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run a short fixed workload for rocprofv3 --pmc (20 logits launches + calibration copies)")
    return ap.parse_args()


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "kv_cache_quantization_03_amd", "csrc"))):
        if f in ("kernels_logits_mfma.hip", "mfma_common.h", "kernels_common.h"):  # the fused logits kernel's sources
            h.update(open(os.path.join(ROOT, "kv_cache_quantization_03_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current logits kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "logits_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
    except Exception:
        return None
    if rec.get("kernel_sha") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode (the codec is data-oblivious, "
              "a sharded deployment would run one independent instance per GPU).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from kv_cache_quantization_03_amd import binding as B
    from kv_cache_quantization_03_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bits = args.bits
    w = I.llama8b_decode(bits=bits)
    d, hq, hkv, ctx, batch = w["d"], w["n_q_heads"], w["n_kv_heads"], w["ctx"], w["batch"]
    n_keys = batch * hkv * ctx
    codec = B.tq_codec_create(d, bits, 0, I.CODEC_SEED)
    if args.only_stages:
        print(json.dumps({"stages": time_stages(B, I, codec, dev, args)}))
        return

    t0 = time.time()
    k_host = w["keys"].rows()
    q_host = w["queries"].rows().reshape(batch, 1, hq, d)
    print(f"[bench] inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    k_dev = torch.from_numpy(k_host).to(dev).to(torch.bfloat16)
    q_dev = torch.from_numpy(q_host).to(dev).to(torch.bfloat16)

    # ---- encode the cache (timed as a stage)
    stream = torch.cuda.current_stream()
    kp = B.alloc_packed(codec, n_keys, dev)
    enc_ws = torch.empty(B.tq_encode_workspace(codec, n_keys), dtype=torch.uint8, device=dev)
    B.tq_encode_kv(codec, k_dev, k_out=kp, ws=enc_ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_enc = 5
    e0.record(stream)
    for _ in range(n_enc):
        B.tq_encode_kv(codec, k_dev, k_out=kp, ws=enc_ws)
    e1.record(stream)
    torch.cuda.synchronize()
    enc_ms = e0.elapsed_time(e1) / n_enc

    # ---- buffer sets: distinct memory for every step of a rotation
    rec_bytes = n_keys * codec.record_bytes
    logit_bytes = batch * hq * ctx * 4
    prep_bytes = B.tq_attn_logits_workspace(codec, batch, hq, hkv, 1)
    set_bytes = rec_bytes + logit_bytes + prep_bytes
    n_sets = max(4, math.ceil(2 * INFINITY_CACHE / set_bytes))
    sets = []
    for s in range(n_sets):
        pk = B.Packed(kp.codes.clone(), kp.signs.clone(), kp.norm.clone(), kp.rnorm.clone())
        sets.append({
            "k": pk,
            "q": q_dev.clone(),
            "prep": torch.empty(prep_bytes, dtype=torch.uint8, device=dev),
            "logits": torch.empty((batch, hq, 1, ctx), dtype=torch.float32, device=dev),
        })
    torch.cuda.synchronize()

    def step(i):
        # one decode step of scoring: query prep and logits in one launch
        S = sets[i % n_sets]
        B.tq_attn_logits(codec, S["q"], S["k"], ctx, hkv, logits=S["logits"], ws=S["prep"])

    def two_kernel_step(i):
        # the split form: query prep, then logits from the prepared operands
        S = sets[i % n_sets]
        B.tq_attn_query_prep(codec, S["q"], hkv, prep=S["prep"])
        B.tq_attn_logits_prepped(codec, S["prep"], (batch, 1, hq), S["k"], ctx, hkv, logits=S["logits"])

    for i in range(max(args.warmup, n_sets)):
        step(i)
    torch.cuda.synchronize()
    eager = [S["logits"].clone() for S in sets]

    if args.pmc_pass:
        # short fixed workload for rocprofv3 --pmc: 20 step launches, then plain
        # 64 MiB device copies that calibrate the byte counters
        for i in range(20):
            step(i)
        src = torch.empty(64 * 2 ** 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        # then 5 decode-attention calls on the 128K-context shape (3-bit K and
        # V) and 3 encodes of its keys, for the per-kernel instruction counters
        cdc = B.tq_codec_create(d, 3, 0, I.CODEC_SEED)
        g = torch.Generator(device=dev)
        g.manual_seed(11)
        kd = torch.randn((8 * 131072, d), generator=g, device=dev).to(torch.bfloat16)
        qd = torch.randn((1, 32, d), generator=g, device=dev).to(torch.bfloat16)
        kpd = B.alloc_packed(cdc, kd.shape[0], dev)
        for _ in range(3):
            B.tq_encode_kv(cdc, kd, k_out=kpd)
        outd = torch.empty((1, 32, d), dtype=torch.bfloat16, device=dev)
        for _ in range(5):
            B.tq_decode_attn(cdc, cdc, qd, kpd, kpd, 131072, 8, 1 / math.sqrt(d), out=outd)
        # and 5 with the same keys as a V cache in 32-row blocks
        cvb = B.tq_codec_create_vblock(d, 3, False, I.CODEC_SEED)
        vbd = B.tq_encode_kv(cvb, kd)[0]
        for _ in range(5):
            B.tq_decode_attn(cdc, cvb, qd, kpd, vbd, 131072, 8, 1 / math.sqrt(d), out=outd)
        del vbd
        # and 5 with PolarQuant K and V records of the same keys (the polar scorer, then the value kernel)
        cpo = B.tq_codec_create_polar(d, 3, 0, I.CODEC_SEED)
        kpo = B.tq_encode_kv(cpo, kd)[0]
        for _ in range(5):
            B.tq_decode_attn(cpo, cpo, qd, kpo, kpo, 131072, 8, 1 / math.sqrt(d), out=outd)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_pass": True, "logits_launches": 20, "copy_bytes": 64 * 2 ** 20, "copies": 5,
                          "decode_launches": 15, "encode_launches": 5}))
        return

    # ---- the timed steps run as one HIP graph (no host launch cost per step)
    K = args.steps
    g_steps = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_steps):
        for i in range(K):
            step(i)
    # every replay must reproduce the eager results
    g_steps.replay()
    torch.cuda.synchronize()
    for s_i, S in enumerate(sets[:min(n_sets, K)]):
        if not torch.equal(S["logits"], eager[s_i]):
            raise RuntimeError(f"graph replay differs from the eager step on buffer set {s_i}")

    # timed region: K steps; HIP events on the launch stream bracket the same
    # replay, so the kernel's average duration comes from the timed run itself
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    e0.record(stream)
    g_steps.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / K
    logits_ms = e0.elapsed_time(e1) / K
    roof_launches = K
    scores_per_step = batch * hq * ctx
    value = scores_per_step / (ms_per_step * 1e-3)
    for s_i, S in enumerate(sets[:min(n_sets, K)]):
        if not torch.equal(S["logits"], eager[s_i]):
            raise RuntimeError(f"timed replay differs from the eager step on buffer set {s_i}")
    del g_steps
    if K < ROOFLINE_LAUNCHES:
        # a short timed region is dominated by the graph's launch and drain; the
        # kernel's per-launch duration for the roofline comes from a replay of
        # ROOFLINE_LAUNCHES back-to-back steps right after it (value stays the
        # K-step wall-clock rate)
        g_r = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_r):
            for i in range(ROOFLINE_LAUNCHES):
                step(i)
        g_r.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g_r.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        logits_ms = e0.elapsed_time(e1) / ROOFLINE_LAUNCHES
        roof_launches = ROOFLINE_LAUNCHES
        del g_r

    # the split two-launch form on the same buffers, for comparison
    g_two = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_two):
        for i in range(K):
            two_kernel_step(i)
    g_two.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    g_two.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    two_ms = e0.elapsed_time(e1) / K
    two_diff = max(float(((S["logits"] - eager[s_i]).abs().amax(dim=-1) / eager[s_i].abs().amax(dim=-1)).max())
                   for s_i, S in enumerate(sets[:min(n_sets, K)]))
    del g_two

    q_bytes = batch * hq * d * 2
    alg_bytes = rec_bytes + logit_bytes + q_bytes
    achieved = alg_bytes / (logits_ms * 1e-3) / 1e9
    workload = w["name"]
    traffic = measured_traffic(workload)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8xfp4",
        "data": "synthetic",
        "config": {"workload": workload, "batch": batch, "n_q_heads": hq, "n_kv_heads": hkv, "head_dim": d,
                   "ctx_len": ctx, "bits": bits, "key_dtype": "bf16", "buffer_sets": n_sets,
                   "record_bytes_per_key": codec.record_bytes},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "logits_fused_kernel", "kernel_ms": logits_ms, "kernel_ms_launches": roof_launches,
                     "kernel_ms_method": "HIP events around a graph replay of back-to-back launches on the "
                                         "kernel's stream (per-launch time, the gap between launches included)",
                     "algorithmic_bytes": alg_bytes,
                     "keys_per_s_kernel": scores_per_step / (logits_ms * 1e-3),
                     "k_only_GBs": rec_bytes / (logits_ms * 1e-3) / 1e9},
        "stages": {"encode_k_ms": enc_ms, "encode_vectors_per_s": n_keys / (enc_ms * 1e-3),
                   "two_kernel_step_ms": two_ms, "two_kernel_vs_fused_max_row_rel": two_diff},
    }
    print(f"[bench] step {ms_per_step * 1e3:.2f} us, fused kernel {logits_ms * 1e3:.2f} us, "
          f"{achieved:.0f} GB/s; two-kernel step {two_ms * 1e3:.2f} us (max row rel diff {two_diff:.1e})",
          file=sys.stderr, flush=True)

    if not args.no_stages:
        out["stages"].update(time_stages(B, I, codec, dev, args))
        ceil = out["stages"].get("stream_ceiling_c2_traffic")
        if ceil:  # the same byte count read by a plain streaming kernel, on this machine
            out["roofline"]["stream_ceiling_GBs"] = ceil["achieved_GBs"]
            out["roofline"]["frac_of_stream_ceiling"] = achieved / ceil["achieved_GBs"]

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, k_host, q_host, bits)
    print(json.dumps(out))


def _time(fn, n=5, graph=False):
    """Average ms per call of fn on the current stream (HIP events); with
    graph=True the n calls are captured once and replayed as one graph."""
    import torch
    s = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        a.record(s)
        g.replay()
        b.record(s)
    else:
        a.record(s)
        for _ in range(n):
            fn()
        b.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


PEAK_FP16_TFLOPS = 2500.0      # dense fp16 / bf16 matrix ops
PEAK_FP8_TFLOPS = 5000.0       # dense fp8 matrix ops (the f8f6f4 op with an fp8 operand runs at this rate)


def _hbm(ms, nbytes):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "algorithmic_bytes": nbytes, "achieved_GBs": gbs, "frac": gbs / PEAK_HBM_GBS}


def sparse_v_stage(B, codec3, dev, g, k, vp, dsets, qd, out, ws, ctx, d, tag="c4", vblock=None):
    """Sparse V on a decode shape (32 query heads, 8 KV heads, ctx keys).
    Needle cache: the same haystack keys plus, with probability 1/512 per (KV
    head, position), a key z + 64·u, u the unit sum of that KV head's four
    queries (peaked attention, as in long-context decoding); values unchanged.
    Times plain decode and the gate 1e-6 on the needle cache, and the gate on
    the Gaussian cache (where it drops nothing: its cost); with `vblock` =
    (V codec in 32-row blocks, its V sets), plain and gated decode on the
    needle cache again with that V.  The dropped fraction of 128-key blocks
    comes from the cache's own logits (tq_attn_logits)."""
    import torch
    gate, scale, hkv, hq = 1e-6, 1 / math.sqrt(d), 8, 32
    u = qd.float().view(hkv, hq // hkv, d).sum(1)
    u = u / u.norm(dim=1, keepdim=True)
    mask = torch.rand(hkv * ctx, generator=g, device=dev) < 1.0 / 512
    kn = k.float()
    kn[mask] += 64.0 * u.repeat_interleave(ctx, dim=0)[mask]
    kpn = B.tq_encode_kv(codec3, kn.to(torch.bfloat16))[0]
    del kn
    lg = B.tq_attn_logits(codec3, qd.view(1, 1, hq, d), kpn, ctx, hkv).view(hkv, hq // hkv, ctx // 1024, 1024)
    sc = lg * scale
    e = torch.exp(sc - sc.amax(dim=-1, keepdim=True))
    keep = e >= gate * e.sum(dim=-1, keepdim=True)
    dropped = float((~keep.view(hkv, hq // hkv, ctx // 128, 128).any(dim=3).any(dim=1)).float().mean())
    del lg, sc, e, keep
    ns = max(4, len(dsets))
    nsets = [(kpn if i == 0 else B.Packed(kpn.codes.clone(), kpn.signs.clone(), kpn.norm.clone(), kpn.rnorm.clone()),
              dsets[i % len(dsets)][1]) for i in range(ns)]
    runs = [(f"decode_attn_{tag}_needles_plain", nsets, False, codec3),
            (f"decode_attn_{tag}_needles_sparse_v", nsets, True, codec3),
            (f"decode_attn_{tag}_gaussian_sparse_v", dsets, True, codec3)]
    if vblock is not None:
        cvb, vbsets = vblock
        bsets = [(kk, vbsets[i % len(vbsets)]) for i, (kk, _) in enumerate(nsets)]
        runs += [(f"decode_attn_{tag}_needles_plain_vblock", bsets, False, cvb),
                 (f"decode_attn_{tag}_needles_sparse_v_vblock", bsets, True, cvb)]
    res = {}
    for name, sets, gated, cv in runs:
        it = iter(range(10 ** 9))

        def step():
            kk, vv = sets[next(it) % len(sets)]
            if gated:
                B.tq_decode_attn_sparse_v(codec3, cv, qd, kk, vv, ctx, hkv, scale, gate, out=out, ws=ws)
            else:
                B.tq_decode_attn(codec3, cv, qd, kk, vv, ctx, hkv, scale, out=out, ws=ws)
        ms = _time(step, 30, graph=True)
        res[name] = {"ms": ms, "buffer_sets": len(sets), "gate": gate if gated else None}
        print(f"[bench] {name} {ms * 1e3:.1f} us", file=sys.stderr, flush=True)
    needle_v = 8 * ctx * codec3.record_bytes * (1 - dropped)
    for suffix in ("", "_vblock") if vblock is not None else ("",):
        r = res[f"decode_attn_{tag}_needles_sparse_v{suffix}"]
        r["dropped_block_fraction"] = dropped
        r["speedup_vs_plain"] = res[f"decode_attn_{tag}_needles_plain{suffix}"]["ms"] / r["ms"]
        r.update(_hbm(r["ms"], 8 * ctx * codec3.record_bytes + needle_v + 2 * hq * d * 2))
    del kpn, nsets
    return res


def polar_stage(B, I, dev, k, q, ctx, d):
    """The PolarQuant first stage (3-bit: 2-bit angles + 1 QJL bit) on the
    Llama-8B decode shape: encode of the 262144 keys, then one decode step of
    logits (prep launch + the polar scorer), 24 rotating buffer sets."""
    import torch
    pc = B.tq_codec_create_polar(d, 3, 0, I.CODEC_SEED)
    kp = B.alloc_packed(pc, k.shape[0], dev)
    ms_e = _time(lambda: B.tq_encode_kv(pc, k, k_out=kp), 20, graph=True)
    ns = 24
    sets = [(B.Packed(kp.codes.clone(), kp.signs.clone(), kp.norm.clone(), kp.rnorm.clone()), q.clone(),
             torch.empty((1, 32, 1, ctx), device=dev),
             torch.empty(B.tq_attn_logits_workspace(pc, 1, 32, 8, 1), dtype=torch.uint8, device=dev))
            for _ in range(ns)]
    it = iter(range(10 ** 9))

    def step():
        kk, qq, ll, ww = sets[next(it) % ns]
        B.tq_attn_logits(pc, qq, kk, ctx, 8, logits=ll, ws=ww)
    ms = _time(step, 240, graph=True)
    print(f"[bench] polar 3-bit: encode {ms_e * 1e3:.1f} us, logits {ms * 1e3:.1f} us", file=sys.stderr, flush=True)
    return {"polar_encode_c2": {"ms": ms_e, "vectors_per_s": k.shape[0] / (ms_e * 1e-3), "bound": "alu"},
            "polar_logits_c2_3bit": {"ms": ms, "keys_per_s": 32 * ctx / (ms * 1e-3), "buffer_sets": ns,
                                     **_hbm(ms, 8 * ctx * pc.record_bytes + 32 * ctx * 4 + 32 * d * 2),
                                     "note": "VALU-bound: y-hat rebuilt per key from the angle codes"}}


def mse_v_stage(B, codec3, dev, g, dsets, qd, out, ctx, d):
    """Decode attention on the long-context shape with 3-bit K and an MSE-only
    V codec (3 and 2 code bits, no QJL stage; records of 52 and 36 bytes), and
    the encode of that V cache."""
    import torch
    hkv, hq, scale = 8, 32, 1 / math.sqrt(d)
    v = torch.randn((hkv * ctx, d), generator=g, device=dev).to(torch.bfloat16)
    res = {}
    for bits in (3, 2):
        cv = B.tq_codec_create_mse(d, bits)
        vp = B.alloc_packed(cv, hkv * ctx, dev)
        ms_e = _time(lambda: B.tq_encode_kv(cv, v, k_out=vp), 10, graph=True)
        sets = [(kk, vp if i == 0 else B.Packed(vp.codes.clone(), None, vp.norm.clone(), None))
                for i, (kk, _) in enumerate(dsets)]
        ws = torch.empty(B.tq_decode_attn_workspace(codec3, cv, 1, hq, hkv, ctx), dtype=torch.uint8, device=dev)
        it = iter(range(10 ** 9))

        def step():
            kk, vv = sets[next(it) % len(sets)]
            B.tq_decode_attn(codec3, cv, qd, kk, vv, ctx, hkv, scale, out=out, ws=ws)
        ms = _time(step, 30, graph=True)
        name = f"decode_attn_c4_mse_v{bits}"
        res[name] = {"ms": ms, "buffer_sets": len(sets), "v_record_bytes": cv.record_bytes,
                     **_hbm(ms, hkv * ctx * (codec3.record_bytes + cv.record_bytes) + 2 * hq * d * 2)}
        res[f"encode_mse_v{bits}_c4"] = {"ms": ms_e, "vectors_per_s": hkv * ctx / (ms_e * 1e-3)}
        print(f"[bench] {name} {ms * 1e3:.1f} us (V encode {ms_e * 1e3:.1f} us)", file=sys.stderr, flush=True)
        del sets, vp, ws, cv
    del v
    return res


def polar_decode_stage(B, I, codec3, dev, g, dsets, qd, out, ctx, d):
    """Decode attention on the long-context shape with the recursive polar
    first stage: polar K and V (3-bit, 56-byte records), and per-coordinate K
    with polar V.  Three K/V sets."""
    import torch
    hkv, hq, scale = 8, 32, 1 / math.sqrt(d)
    cp = B.tq_codec_create_polar(d, 3, 0, I.CODEC_SEED)
    k = torch.randn((hkv * ctx, d), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((hkv * ctx, d), generator=g, device=dev).to(torch.bfloat16)
    kp, vp = B.tq_encode_kv(cp, k, v)
    del k, v
    sets = [(kp, vp)] + [(B.Packed(kp.codes.clone(), kp.signs.clone(), kp.norm.clone(), kp.rnorm.clone()),
                          B.Packed(vp.codes.clone(), vp.signs.clone(), vp.norm.clone(), vp.rnorm.clone()))
                         for _ in range(len(dsets) - 1)]
    res = {}
    for name, ck, ksets in (("decode_attn_c4_polar_kv", cp, [s[0] for s in sets]),
                            ("decode_attn_c4_polar_v", codec3, [s[0] for s in dsets])):
        ws = torch.empty(B.tq_decode_attn_workspace(ck, cp, 1, hq, hkv, ctx), dtype=torch.uint8, device=dev)
        it = iter(range(10 ** 9))

        def step():
            i = next(it) % len(sets)
            B.tq_decode_attn(ck, cp, qd, ksets[i], sets[i][1], ctx, hkv, scale, out=out, ws=ws)
        ms = _time(step, 30, graph=True)
        res[name] = {"ms": ms, "buffer_sets": len(sets),
                     **_hbm(ms, hkv * ctx * (ck.record_bytes + cp.record_bytes) + 2 * hq * d * 2)}
        print(f"[bench] {name} {ms * 1e3:.1f} us", file=sys.stderr, flush=True)
        del ws
    del sets, kp, vp, cp
    return res


def paged_stage(B, codec3, dev, g, dsets, qd, out, ws, ctx, d):
    """Paged cache on the long-context decode shape.  (1) The same caches
    copied into 256-position pages in shuffled order, read through the page
    table, against the contiguous call.  (2) Eight sequences of 128K, 64K, ...,
    1K positions in one paged pool (one decode step for all).  (3) Appending
    one token per KV head to K and V of those eight sequences."""
    import torch
    hkv, hq, P = 8, 32, 256
    scale = 1 / math.sqrt(d)
    res = {}
    npg = ctx // P

    def to_pages(src, perm):  # rows [kv_head][position] -> [page][kv_head][slot]
        idx = torch.empty(hkv * ctx, dtype=torch.int64, device=dev)
        pos = torch.arange(ctx, device=dev)
        for kh in range(hkv):
            idx[(perm[pos // P] * hkv + kh) * P + pos % P] = kh * ctx + pos
        return B.Packed(src.codes[idx].contiguous(), src.signs[idx].contiguous(), src.norm[idx].contiguous(),
                        src.rnorm[idx].contiguous())
    perm = torch.randperm(npg, generator=g, device=dev)
    psets = [(to_pages(kk, perm), to_pages(vv, perm)) for kk, vv in dsets]
    pt = perm.to(torch.int32).view(1, npg).contiguous()  # position block i sits in page perm[i]
    cl = torch.tensor([ctx], dtype=torch.int32, device=dev)
    it = iter(range(10 ** 9))

    def paged():
        kk, vv = psets[next(it) % len(psets)]
        B.tq_decode_attn_paged(codec3, codec3, qd, kk, vv, cl, pt, P, ctx, hkv, scale, out=out, ws=ws)
    ms_dec = _time(paged, 30, graph=True)
    res["decode_attn_c4_paged256"] = {"ms": ms_dec, "page_size": P, "buffer_sets": len(psets),
                                      **_hbm(ms_dec, 2 * hkv * ctx * codec3.record_bytes + 2 * hq * d * 2)}
    print(f"[bench] C4 decode attention, 256-position pages {ms_dec * 1e3:.1f} us", file=sys.stderr, flush=True)
    del psets
    # logits of one decode step over paged K caches and over contiguous ones.
    # Only K and the logits move, so the rotation holds enough K caches (each
    # with its own logits buffer) to cover twice the Infinity Cache.
    ql = qd.view(1, 1, hq, d)
    kbytes, lbytes = hkv * ctx * codec3.record_bytes, hq * ctx * 4
    n_l = max(len(dsets), math.ceil(2 * INFINITY_CACHE / (kbytes + lbytes)))
    kc_sets = [dsets[i][0] if i < len(dsets) else
               B.Packed(*(t.clone() for t in (dsets[i % len(dsets)][0].codes, dsets[i % len(dsets)][0].signs,
                                             dsets[i % len(dsets)][0].norm, dsets[i % len(dsets)][0].rnorm)))
               for i in range(n_l)]
    kp_sets = [to_pages(kk, perm) for kk in kc_sets]
    lgs = [torch.empty((1, hq, 1, ctx), dtype=torch.float32, device=dev) for _ in range(n_l)]
    wsl = torch.empty(max(B.lib.tq_attn_logits_paged_workspace(codec3.handle, 1, hq, hkv, 1),
                          B.tq_attn_logits_workspace(codec3, 1, hq, hkv, 1), 1), dtype=torch.uint8, device=dev)
    it2 = iter(range(10 ** 9))

    def logits_paged():
        i = next(it2) % n_l
        B.tq_attn_logits_paged(codec3, ql, kp_sets[i], cl, pt, P, ctx, hkv, logits=lgs[i], ws=wsl)

    def logits_contig():
        i = next(it2) % n_l
        B.tq_attn_logits(codec3, ql, kc_sets[i], ctx, hkv, logits=lgs[i], ws=wsl)
    for name, fn in (("logits_c4_paged256", logits_paged), ("logits_c4_contiguous", logits_contig)):
        ms = _time(fn, 2 * n_l, graph=True)
        res[name] = {"ms": ms, "page_size": P if "paged" in name else None, "buffer_sets": n_l,
                     "scores_per_s": hq * ctx / (ms * 1e-3), **_hbm(ms, kbytes + lbytes + hq * d * 2)}
        print(f"[bench] {name} (one decode step, 128K keys) {ms * 1e3:.1f} us", file=sys.stderr, flush=True)
    del kp_sets, kc_sets, lgs
    # eight sequences of different lengths in one pool
    lens = [ctx >> i for i in range(8)]
    bsz, mp = len(lens), ctx // P
    n_pages = sum(n // P for n in lens)
    pool_k = B.alloc_packed(codec3, n_pages * hkv * P, dev)
    pool_v = B.alloc_packed(codec3, n_pages * hkv * P, dev)
    for t in (pool_k.codes, pool_k.signs, pool_v.codes, pool_v.signs):
        t.copy_(torch.randint(-2 ** 31, 2 ** 31 - 1, t.shape, generator=g, device=dev, dtype=torch.int32))
    for t in (pool_k.norm, pool_v.norm):
        t.copy_(torch.rand(t.shape, generator=g, device=dev) + 0.5)
    for t in (pool_k.rnorm, pool_v.rnorm):
        t.copy_(torch.rand(t.shape, generator=g, device=dev) * 0.3)
    order = torch.randperm(n_pages, generator=g, device=dev).to(torch.int32)
    ptab = torch.zeros((bsz, mp), dtype=torch.int32, device=dev)
    o = 0
    for b, n in enumerate(lens):
        ptab[b, :n // P] = order[o:o + n // P]
        o += n // P
    cls = torch.tensor(lens, dtype=torch.int32, device=dev)
    qb = torch.randn((bsz, hq, d), generator=g, device=dev).to(torch.bfloat16)
    outb = torch.empty((bsz, hq, d), dtype=torch.bfloat16, device=dev)
    wsb = torch.empty(B.lib.tq_decode_attn_paged_workspace(codec3.handle, codec3.handle, bsz, hq, hkv, ctx),
                      dtype=torch.uint8, device=dev)
    ms = _time(lambda: B.tq_decode_attn_paged(codec3, codec3, qb, pool_k, pool_v, cls, ptab, P, ctx, hkv, scale,
                                              out=outb, ws=wsb), 30, graph=True)
    tot = sum(lens)
    res["decode_attn_paged_8seq"] = {"ms": ms, "ctx_lens": lens, "page_size": P,
                                     "keys_per_s": hq // hkv * hkv * tot / (ms * 1e-3),
                                     **_hbm(ms, 2 * hkv * tot * codec3.record_bytes + 2 * bsz * hq * d * 2)}
    print(f"[bench] paged decode, 8 sequences 1K..128K {ms * 1e3:.1f} us", file=sys.stderr, flush=True)
    # append one token per (sequence, KV head) to K and V: the step before decode
    xk = torch.randn((bsz, hkv, 1, d), generator=g, device=dev).to(torch.bfloat16)
    xv = torch.randn((bsz, hkv, 1, d), generator=g, device=dev).to(torch.bfloat16)
    cla = (cls - 1).contiguous()      # rewrite each sequence's last position
    wsa = torch.empty(max(B.lib.tq_encode_append_paged_workspace(codec3.handle, bsz, hkv, 1), 16), dtype=torch.uint8,
                      device=dev)

    def append():
        B.tq_encode_append_paged(codec3, xk, cla, ptab, P, n_pages, pool_k, ws=wsa)
        B.tq_encode_append_paged(codec3, xv, cla, ptab, P, n_pages, pool_v, ws=wsa)
    ms = _time(append, 50, graph=True)
    res["append_paged_8seq"] = {"ms": ms, "tokens": 2 * bsz * hkv, "bound": "latency"}
    print(f"[bench] paged append of K and V, 8 x 8 tokens {ms * 1e3:.1f} us", file=sys.stderr, flush=True)
    del pool_k, pool_v
    return res


def time_stages(B, I, codec3, dev, args):
    """The other rows of the path, each timed on its own configuration with
    synthetic data drawn on the GPU (torch, seeded), with the roofline that
    bounds it: algorithmic bytes (or flops) per call over the measured time."""
    import torch
    res = {}
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    d = 128
    # C1: the tiny reference (1 fp32 query, 4096 fp32 keys, 3-bit): latency only
    w1 = I.tiny_ref()
    k1 = torch.from_numpy(w1["keys"].rows()).to(dev)
    q1 = torch.from_numpy(w1["queries"].rows().reshape(1, 1, 1, d)).to(dev)
    kp1 = B.alloc_packed(codec3, k1.shape[0], dev)
    ws1 = torch.empty(max(B.tq_encode_workspace(codec3, k1.shape[0]), 1), dtype=torch.uint8, device=dev)
    ms_e = _time(lambda: B.tq_encode_kv(codec3, k1, k_out=kp1, ws=ws1), 50, graph=True)
    lg1 = torch.empty((1, 1, 1, k1.shape[0]), device=dev)
    wl1 = torch.empty(B.tq_attn_logits_workspace(codec3, 1, 1, 1, 1), dtype=torch.uint8, device=dev)
    ms_l = _time(lambda: B.tq_attn_logits(codec3, q1, kp1, k1.shape[0], 1, logits=lg1, ws=wl1), 50, graph=True)
    res["c1_tiny"] = {"encode_ms": ms_e, "logits_ms": ms_l, "bound": "latency"}
    print(f"[bench] C1 encode {ms_e * 1e3:.1f} us, logits {ms_l * 1e3:.1f} us", file=sys.stderr, flush=True)
    del k1, q1, kp1, ws1, lg1, wl1
    # Every HBM-bound stage rotates over enough buffer sets that the 256 MB
    # Infinity Cache cannot hold them, so its data streams from HBM.
    # C2 4-bit: 4-bit logits on the Llama-8B decode shape
    c4 = B.tq_codec_create(d, 4, 0, I.CODEC_SEED)
    ctx = 32768
    k = torch.randn((8 * ctx, d), generator=g, device=dev).to(torch.bfloat16)
    q = torch.randn((1, 1, 32, d), generator=g, device=dev).to(torch.bfloat16)
    kp4, _ = B.tq_encode_kv(c4, k)
    ns = 24
    sets = [(B.Packed(kp4.codes.clone(), kp4.signs.clone(), kp4.norm.clone(), kp4.rnorm.clone()), q.clone(),
             torch.empty((1, 32, 1, ctx), device=dev),
             torch.empty(B.tq_attn_logits_workspace(c4, 1, 32, 8, 1), dtype=torch.uint8, device=dev))
            for _ in range(ns)]
    it = iter(range(10 ** 9))

    def c2():
        kk, qq, ll, ww = sets[next(it) % ns]
        B.tq_attn_logits(c4, qq, kk, ctx, 8, logits=ll, ws=ww)
    ms = _time(c2, 240, graph=True)
    res["logits_c2_4bit"] = {"ms": ms, "keys_per_s": 32 * ctx / (ms * 1e-3), "buffer_sets": ns,
                             **_hbm(ms, 8 * ctx * c4.record_bytes + 32 * ctx * 4 + 32 * d * 2)}
    print(f"[bench] C2 4-bit logits {ms * 1e3:.1f} us", file=sys.stderr, flush=True)
    del kp4, sets
    res.update(polar_stage(B, I, dev, k, q, ctx, d))
    del k
    # Streaming ceiling at the C2 step's algorithmic traffic: one launch that
    # reads the records' bytes and writes the logits' bytes (tq_diag_stream:
    # four independent 16-byte loads per thread), rotating buffers, timed the
    # same way; and a plain read of the whole byte count
    rbytes = (8 * 32768 * codec3.record_bytes + 32 * d * 2) // 16 * 16
    wbytes = 32 * 32768 * 4
    ns = 29
    bufs = [torch.randint(0, 1 << 30, (rbytes // 4,), generator=g, device=dev, dtype=torch.int32) for _ in range(ns)]
    outs = [torch.empty(wbytes // 4, dtype=torch.int32, device=dev) for _ in range(ns)]
    sink = torch.empty(B.lib.tq_diag_stream_sink_words(rbytes + wbytes), dtype=torch.int32, device=dev)
    it = iter(range(10 ** 9))

    def rw():
        i = next(it) % ns
        B.tq_diag_stream(bufs[i], outs[i], sink)
    ms = _time(rw, 240, graph=True)
    res["stream_ceiling_c2_traffic"] = {"ms": ms, **_hbm(ms, rbytes + wbytes), "read_bytes": rbytes,
                                        "write_bytes": wbytes, "buffer_sets": ns}
    print(f"[bench] streaming read {rbytes / 1e6:.1f} MB + write {wbytes / 1e6:.1f} MB: {ms * 1e3:.2f} us",
          file=sys.stderr, flush=True)
    del bufs, outs, sink
    # the same at the batch-16 step's traffic (16x; two buffer sets of 302 MB)
    bufs = [torch.randint(0, 1 << 30, (16 * rbytes // 4,), generator=g, device=dev, dtype=torch.int32)
            for _ in range(2)]
    outs = [torch.empty(16 * wbytes // 4, dtype=torch.int32, device=dev) for _ in range(2)]
    sink = torch.empty(B.lib.tq_diag_stream_sink_words(16 * rbytes), dtype=torch.int32, device=dev)
    it = iter(range(10 ** 9))

    def rw16():
        i = next(it) % 2
        B.tq_diag_stream(bufs[i], outs[i], sink)
    ms = _time(rw16, 40, graph=True)
    res["stream_ceiling_c2_traffic_batch16"] = {"ms": ms, **_hbm(ms, 16 * (rbytes + wbytes)),
                                                "read_bytes": 16 * rbytes, "write_bytes": 16 * wbytes,
                                                "buffer_sets": 2}
    print(f"[bench] streaming ceiling at batch 16: {ms * 1e3:.2f} us", file=sys.stderr, flush=True)
    del bufs, outs, sink
    # C2 at batch 16: the same decode step, 16 sequences (the streaming asymptote)
    bsz = 16
    k = torch.randn((bsz * 8 * ctx, d), generator=g, device=dev).to(torch.bfloat16)
    kb = B.tq_encode_kv(codec3, k)[0]
    del k
    qb = torch.randn((bsz, 1, 32, d), generator=g, device=dev).to(torch.bfloat16)
    ns = 2
    bsets = [(kb if i == 0 else B.Packed(kb.codes.clone(), kb.signs.clone(), kb.norm.clone(), kb.rnorm.clone()),
              qb.clone(), torch.empty((bsz, 32, 1, ctx), device=dev),
              torch.empty(B.tq_attn_logits_workspace(codec3, bsz, 32, 8, 1), dtype=torch.uint8, device=dev))
             for i in range(ns)]
    it = iter(range(10 ** 9))

    def c2b():
        kk, qq, ll, ww = bsets[next(it) % ns]
        B.tq_attn_logits(codec3, qq, kk, ctx, 8, logits=ll, ws=ww)
    ms = _time(c2b, 40, graph=True)
    res["logits_c2_3bit_batch16"] = {"ms": ms, "keys_per_s": bsz * 32 * ctx / (ms * 1e-3), "buffer_sets": ns,
                                     **_hbm(ms, bsz * (8 * ctx * codec3.record_bytes + 32 * ctx * 4 + 32 * d * 2))}
    print(f"[bench] C2 3-bit logits at batch 16 {ms * 1e3:.1f} us", file=sys.stderr, flush=True)
    del kb, qb, bsets
    # C4: fused decode attention, 128K context, K and V 3-bit
    ctx = 131072
    k = torch.randn((8 * ctx, d), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((8 * ctx, d), generator=g, device=dev).to(torch.bfloat16)
    qd = torch.randn((1, 32, d), generator=g, device=dev).to(torch.bfloat16)
    kp, vp = B.tq_encode_kv(codec3, k, v)
    # the same V in 32-row blocks (a codec with codec3's tables)
    cvb = B.tq_codec_create_vblock(d, 3, False, I.CODEC_SEED)
    vbp = B.alloc_packed(cvb, 8 * ctx, dev)
    wse = torch.empty(max(B.tq_encode_workspace(cvb, 8 * ctx), 1), dtype=torch.uint8, device=dev)
    ms_vbe = _time(lambda: B.tq_encode_kv(cvb, v, k_out=vbp, ws=wse), 10, graph=True)
    ms_vre = _time(lambda: B.tq_encode_kv(codec3, v, k_out=vp, ws=wse), 10, graph=True)
    k_c4 = k
    del k, v, wse
    ns = 3
    dsets = [(kp, vp)] + [(B.Packed(kp.codes.clone(), kp.signs.clone(), kp.norm.clone(), kp.rnorm.clone()),
                           B.Packed(vp.codes.clone(), vp.signs.clone(), vp.norm.clone(), vp.rnorm.clone()))
                          for _ in range(ns - 1)]
    vbsets = [vbp] + [B.Packed(vbp.codes.clone(), vbp.signs.clone(), vbp.norm.clone(), vbp.rnorm.clone())
                      for _ in range(ns - 1)]
    out = torch.empty((1, 32, d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(B.tq_decode_attn_workspace(codec3, codec3, 1, 32, 8, ctx), dtype=torch.uint8, device=dev)
    it = iter(range(10 ** 9))

    def c4():
        kk, vv = dsets[next(it) % ns]
        B.tq_decode_attn(codec3, codec3, qd, kk, vv, ctx, 8, 1 / math.sqrt(d), out=out, ws=ws)
    ms = _time(c4, 30, graph=True)
    res["decode_attn_c4"] = {"ms": ms, "buffer_sets": ns,
                             **_hbm(ms, 2 * 8 * ctx * codec3.record_bytes + 2 * 32 * d * 2)}
    print(f"[bench] C4 decode attention {ms * 1e3:.1f} us", file=sys.stderr, flush=True)
    it = iter(range(10 ** 9))

    def c4b():
        i = next(it) % ns
        B.tq_decode_attn(codec3, cvb, qd, dsets[i][0], vbsets[i], ctx, 8, 1 / math.sqrt(d), out=out, ws=ws)
    ms_b = _time(c4b, 30, graph=True)
    o_row = B.tq_decode_attn(codec3, codec3, qd, kp, vp, ctx, 8, 1 / math.sqrt(d), out_dtype=torch.float32)
    o_blk = B.tq_decode_attn(codec3, cvb, qd, kp, vbp, ctx, 8, 1 / math.sqrt(d), out_dtype=torch.float32)
    res["decode_attn_c4_vblock"] = {"ms": ms_b, "buffer_sets": ns, "speedup_vs_row_v": ms / ms_b,
                                    "equal_to_row_v": bool(torch.equal(o_row, o_blk)),
                                    "v_encode_ms": ms_vbe, "v_encode_row_ms": ms_vre,
                                    **_hbm(ms_b, 2 * 8 * ctx * codec3.record_bytes + 2 * 32 * d * 2)}
    del o_row, o_blk
    print(f"[bench] C4 decode attention, V in 32-row blocks {ms_b * 1e3:.1f} us "
          f"(V encode {ms_vbe * 1e3:.1f} us, rows {ms_vre * 1e3:.1f} us)", file=sys.stderr, flush=True)
    if not args.no_stage_sparse_v:
        res.update(sparse_v_stage(B, codec3, dev, g, k_c4, vp, dsets, qd, out, ws, ctx, d, vblock=(cvb, vbsets)))
    res.update(paged_stage(B, codec3, dev, g, dsets, qd, out, ws, ctx, d))
    res.update(mse_v_stage(B, codec3, dev, g, dsets, qd, out, ctx, d))
    res.update(polar_decode_stage(B, I, codec3, dev, g, dsets, qd, out, ctx, d))
    del kp, vp, dsets, ws, k_c4, vbp, vbsets
    if not args.no_stage_sparse_v:
        # Sparse V on the 32K decode shape: 12 K/V sets (about 2.6x the Infinity Cache)
        ctx = 32768
        k = torch.randn((8 * ctx, d), generator=g, device=dev).to(torch.bfloat16)
        v = torch.randn((8 * ctx, d), generator=g, device=dev).to(torch.bfloat16)
        kp, vp = B.tq_encode_kv(codec3, k, v)
        vbp = B.alloc_packed(cvb, 8 * ctx, dev)
        B.tq_encode_kv(cvb, v, k_out=vbp)
        del v
        ns = 12
        dsets = [(kp, vp)] + [(B.Packed(kp.codes.clone(), kp.signs.clone(), kp.norm.clone(), kp.rnorm.clone()),
                               B.Packed(vp.codes.clone(), vp.signs.clone(), vp.norm.clone(), vp.rnorm.clone()))
                              for _ in range(ns - 1)]
        vbsets = [vbp] + [B.Packed(vbp.codes.clone(), vbp.signs.clone(), vbp.norm.clone(), vbp.rnorm.clone())
                          for _ in range(ns - 1)]
        ws = torch.empty(B.tq_decode_attn_workspace(codec3, codec3, 1, 32, 8, ctx), dtype=torch.uint8, device=dev)
        res.update(sparse_v_stage(B, codec3, dev, g, k, vp, dsets, qd, out, ws, ctx, d, tag="c2",
                                  vblock=(cvb, vbsets)))
        del k, kp, vp, vbp, dsets, vbsets, ws
    del cvb
    # C3: prefill encode of K and V [16][8][8192][128] bf16, then 16 queries per sequence
    bsz, hkv, ctx, nq = 16, 8, 8192, 16
    n = bsz * hkv * ctx
    k = torch.randn((n, d), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((n, d), generator=g, device=dev).to(torch.bfloat16)
    kp, vp = B.alloc_packed(codec3, n, dev), B.alloc_packed(codec3, n, dev)
    ws = torch.empty(max(B.tq_encode_workspace(codec3, n), 1), dtype=torch.uint8, device=dev)
    ms = _time(lambda: B.tq_encode_kv(codec3, k, v, k_out=kp, v_out=vp, ws=ws), 5, graph=True)
    res["encode_c3"] = {"ms": ms, "vectors_per_s": 2 * n / (ms * 1e-3),
                        **_hbm(ms, 2 * n * (d * 2 + codec3.record_bytes))}
    print(f"[bench] C3 prefill encode {ms:.3f} ms", file=sys.stderr, flush=True)
    del k, v, vp, ws
    qp = torch.randn((bsz, nq, hkv, d), generator=g, device=dev).to(torch.bfloat16)
    ns = 3
    lsets = [(kp if i == 0 else B.Packed(kp.codes.clone(), kp.signs.clone(), kp.norm.clone(), kp.rnorm.clone()),
              qp.clone(), torch.empty((bsz, hkv, nq, ctx), device=dev),
              torch.empty(B.tq_attn_logits_workspace(codec3, bsz, hkv, hkv, nq), dtype=torch.uint8, device=dev))
             for i in range(ns)]
    it = iter(range(10 ** 9))

    def c3():
        kk, qq, ll, ww = lsets[next(it) % ns]
        B.tq_attn_logits(codec3, qq, kk, ctx, hkv, logits=ll, ws=ww)
    ms = _time(c3, 30, graph=True)
    res["logits_c3"] = {"ms": ms, "scores_per_s": bsz * hkv * nq * ctx / (ms * 1e-3), "buffer_sets": ns,
                        **_hbm(ms, n * codec3.record_bytes + bsz * hkv * nq * ctx * 4 + bsz * nq * hkv * d * 2)}
    print(f"[bench] C3 logits {ms:.3f} ms", file=sys.stderr, flush=True)
    del kp, qp, lsets
    if not args.no_stage_search:
        # C5: encode the 10^6 x 1536 database (4-bit), then 1024 queries top-10
        c16 = B.tq_codec_create(1536, 4, 0, I.CODEC_SEED)
        db, qs = I.vector_search_torch(dev)
        n_db, nqs, ds = db.shape[0], qs.shape[0], db.shape[1]
        dbp = B.alloc_packed(c16, n_db, dev)
        ws = torch.empty(max(B.tq_encode_workspace(c16, n_db), 1), dtype=torch.uint8, device=dev)
        ms = _time(lambda: B.tq_encode_kv(c16, db, k_out=dbp, ws=ws), 3)
        flops = 2.0 * ds * ds * n_db  # the QJL projection z = S r
        executed = 3 * flops          # on the fp16 matrix cores as S_hi r_hi + S_hi r_lo + S_lo r_hi
        res["encode_c5"] = {"ms": ms, "vectors_per_s": n_db / (ms * 1e-3), "bound": "mfma (fp16)",
                            "algorithmic_tflop": flops / 1e12, "algorithmic_TFLOPs": flops / (ms * 1e-3) / 1e12,
                            "matrix_TFLOPs": executed / (ms * 1e-3) / 1e12,
                            "frac": flops / (ms * 1e-3) / 1e12 / PEAK_FP16_TFLOPS,
                            "frac_executed": executed / (ms * 1e-3) / 1e12 / PEAK_FP16_TFLOPS}
        print(f"[bench] C5 encode {ms:.2f} ms", file=sys.stderr, flush=True)
        del db, ws
        ws = torch.empty(B.tq_search_workspace(c16, n_db, nqs, 10), dtype=torch.uint8, device=dev)
        idx = torch.empty((nqs, 10), dtype=torch.int64, device=dev)
        sc = torch.empty((nqs, 10), dtype=torch.float32, device=dev)
        ms = _time(lambda: B.tq_search_topk(c16, dbp, qs, 10, out_idx=idx, out_score=sc, ws=ws), 3)
        alg = 2.0 * (ds + ds) * nqs * n_db  # the estimator's multiply-adds, fp32-grade
        # matrix ops issued: per (16 queries, 16 records, 128 coordinates) 15 (MSE, 4 planes) + 3 (QJL)
        ops = (nqs // 16) * (n_db // 16) * (ds // 128) * 18
        executed = ops * 16 * 16 * 128 * 2
        res["search_c5"] = {"ms": ms, "scores_per_s": nqs * n_db / (ms * 1e-3), "bound": "mfma (fp8 x fp4)",
                            "algorithmic_tflop": alg / 1e12, "algorithmic_TFLOPs": alg / (ms * 1e-3) / 1e12,
                            "matrix_TFLOPs": executed / (ms * 1e-3) / 1e12,
                            "frac": alg / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
                            "frac_executed": executed / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS}
        print(f"[bench] C5 search {ms:.2f} ms", file=sys.stderr, flush=True)
    return res


def _timed(fn, budget_s, max_reps=20):
    """Median seconds of fn over repetitions that fit about budget_s (at least one)."""
    ts = []
    while not ts or (sum(ts) < budget_s and len(ts) < max_reps):
        t = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t)
    ts.sort()
    return ts[len(ts) // 2], len(ts)


def cpu_baseline(w, k_host, q_host, bits):
    """The fp64 NumPy oracle (oracle/, unmodified) timed on this host, beside
    the GPU: the headline decode-logits workload in full, and a bounded sample
    of every other configuration (sizes stated in each entry, scaled to the
    whole workload linearly in the number of vectors or scores).  Input
    generation is outside the timed regions."""
    import numpy as np
    import oracle as O
    from kv_cache_quantization_03_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas_threads = max((x.get("num_threads", 1) for x in threadpool_info()), default=1)
    except Exception:
        threadpool_limits = None
        blas_threads = os.cpu_count()
    one_thread = (lambda: threadpool_limits(limits=1)) if threadpool_limits else None
    cfg = {}

    # C2, the headline: one decode step's scores over the full 32K context
    oc = O.make_codec(w["d"], bits, seed=1234)
    k64 = k_host.astype(np.float64)
    n_enc = 32768
    enc_s, _ = _timed(lambda: O.encode(oc, k64[:n_enc]), 3.0, 3)
    rec = O.encode(oc, k64)
    qh = q_host.astype(np.float64)
    score = lambda: O.attn_logits(oc, qh, rec, w["batch"], w["n_q_heads"], w["n_kv_heads"], 1, w["ctx"])
    score_s, reps = _timed(score, 8.0)
    n_scores = w["batch"] * w["n_q_heads"] * w["ctx"]
    one_core = None
    if one_thread:
        with one_thread():
            s1, _ = _timed(score, 2.0, 1)
        one_core = n_scores / s1
    headline = {"value": n_scores / score_s, "unit": "keys/s", "cores": blas_threads, "kind": "oracle",
                "sample": f"the full workload ({n_scores} scores per step), median of {reps} runs; the step's "
                          f"encode timed on {n_enc} of its {k_host.shape[0]} keys",
                "encode_vectors_per_s": n_enc / enc_s, "value_one_thread": one_core,
                "os_cpu_count": os.cpu_count(), "cpu_model": _cpu_model()}

    # C1: the whole tiny reference (4096 fp32 keys, one query)
    t1 = I.tiny_ref()
    kt = t1["keys"].rows().astype(np.float64)
    qt = t1["queries"].rows().reshape(1, 1, 1, 128).astype(np.float64)
    e1, _ = _timed(lambda: O.encode(oc, kt), 2.0, 5)
    rt = O.encode(oc, kt)
    s1, _ = _timed(lambda: O.attn_logits(oc, qt, rt, 1, 1, 1, 1, 4096), 1.0, 5)
    c1 = {"encode_vectors_per_s": 4096 / e1, "scores_per_s": 4096 / s1, "sample": "whole workload"}
    if one_thread:
        with one_thread():
            e1s, _ = _timed(lambda: O.encode(oc, kt), 1.0, 1)
            s1s, _ = _timed(lambda: O.attn_logits(oc, qt, rt, 1, 1, 1, 1, 4096), 0.5, 1)
        c1.update({"encode_vectors_per_s_one_thread": 4096 / e1s, "scores_per_s_one_thread": 4096 / s1s})
    cfg["tiny_ref_4096x128_f32"] = c1
    if one_thread:
        with one_thread():
            e2s, _ = _timed(lambda: O.encode(oc, k64[:8192]), 1.0, 1)
        headline["encode_vectors_per_s_one_thread"] = 8192 / e2s

    # C3: encode 16384 of the 2^21 K and V rows; score one (sequence, KV head):
    # 16 queries x 8192 keys (of 16 x 8 such pairs)
    p3 = I.prefill_encode()
    k3 = p3["keys"].rows(0, 16384).astype(np.float64)
    e3, _ = _timed(lambda: O.encode(oc, k3), 2.0, 2)
    r3 = O.encode(oc, p3["keys"].rows(0, 8192).astype(np.float64))
    q3 = p3["queries"].rows().reshape(16, 16, 8, 128)[0:1, :, 0:1].astype(np.float64)
    s3, _ = _timed(lambda: O.attn_logits(oc, q3, r3, 1, 1, 1, 16, 8192), 2.0, 3)
    cfg[p3["name"]] = {"encode_vectors_per_s": 16384 / e3, "scores_per_s": 16 * 8192 / s3,
                       "encode_s_full": 2 * 16 * 8 * 8192 / (16384 / e3), "score_s_full": 128 * s3,
                       "sample": "encode of 16384 K rows; scores of one (sequence, KV head): 16 queries x 8192 keys"}

    # C4: decode attention of one KV head (4 query heads) over 32768 of the
    # 131072 positions, scaled x4 (context) x8 (KV heads)
    w4 = I.long_decode()
    k4 = O.encode(oc, w4["keys"].rows(0, 32768).astype(np.float64))
    v4 = O.encode(oc, w4["values"].rows(0, 32768).astype(np.float64))
    q4 = w4["queries"].rows()[:4].reshape(1, 4, 128).astype(np.float64)
    s4, _ = _timed(lambda: O.decode_attn_accumulated(oc, oc, q4, k4, v4, 1, 4, 1, 32768, w4["scale"]), 2.0, 3)
    full4 = s4 * 4 * 8
    cfg[w4["name"]] = {"step_s_full": full4, "keys_per_s": 4 * 32768 / s4,
                       "sample": "one KV head (4 query heads) x 32768 positions, scaled x32 to the step"}

    # C5: encode 2048 database rows; score 64 queries against them (scaled to
    # 1024 queries x 10^6 rows)
    w5 = I.vector_search()
    c16 = O.make_codec(1536, 4, seed=1234)
    x5 = w5["db"].rows(0, 2048).astype(np.float64)
    e5, _ = _timed(lambda: O.encode(c16, x5), 2.0, 2)
    r5 = O.encode(c16, x5)
    q5 = w5["queries"].rows(0, 64).astype(np.float64)
    s5, _ = _timed(lambda: O.score(c16, q5, r5), 2.0, 3)
    sps = 64 * 2048 / s5
    cfg[w5["name"]] = {"encode_vectors_per_s": 2048 / e5, "scores_per_s": sps,
                       "encode_s_full": 1e6 / (2048 / e5), "search_s_full": 1024 * 1e6 / sps,
                       "sample": "encode of 2048 rows; 64 queries x 2048 rows scored (linear in both)"}
    headline["configs"] = cfg
    return headline


if __name__ == "__main__":
    main()
