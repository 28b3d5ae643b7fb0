#!/usr/bin/env python3
"""libmla benchmark: one MI355X, synthetic DeepSeek-V3-shaped MLA layer.

A step is one mla_decode call on the DeepSeek-V3 decode workload (batch 32,
one new token per sequence, cache length 4096 after the append, bf16): query
and KV down-projections with RoPE and the cache append, the query
up-projection, W_UK absorption, split-KV latent attention, the split combine,
W_UV and W_O.  ``value`` is decode tokens/s (batch / step time) with every
input resident in HBM.  Input sets (weights, cache, h) are rotated over
several copies so consecutive steps do not find their operands in the 256 MB
Infinity Cache.

Also reported: per-kernel times from HIP events recorded by the library on
the launch stream, the roofline of the dominant kernel, a causal prefill of
4096 tokens (TFLOPS against the bf16 MFMA peak), the ragged paged batch-128
and 128K two-token decode workloads, the three decode workloads again with
the FP8 (E4M3 + per-128-column scale) latent cache, a sampled parity check,
and the CPU oracle's throughput on a bounded sample (cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense fp8 MFMA


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_kernel_bytes(d, B, n_q, sum_len, e=2, row_bytes=None, fp8_weights=False):
    """Algorithmic HBM bytes per launch of each decode kernel (weights and
    cache read once, activations read/written once); row_bytes is the size
    of a cached row (e * (d_c + d_R) for a cache in the layer dtype, 656 for
    the FP8 cache).  fp8_weights: W_DQ, W_DKV, W_KR and W_O are one byte per
    element plus a 4-byte scale per 128x128 block, and their products read
    the quantised activations (a byte per element, a byte per 128)."""
    T = B * n_q
    nh = d.n_heads
    D = d.d_c + d.d_rope
    rb = e * D if row_bytes is None else row_bytes
    if fp8_weights:
        w_down = (d.d_cq + D) * d.d_model * (1 + 4 / 16384)
        w_o = d.d_model * nh * d.d_v * (1 + 4 / 16384)
        return {
            "quant_fp8": int(e * T * (d.d_model + nh * d.d_v) + T * (d.d_model + nh * d.d_v) * (1 + 1 / 128)),
            "q_kv_down": int(w_down + T * d.d_model * (1 + 1 / 128) + e * (T * d.d_cq + T * D)),
            "o_proj": int(w_o + T * nh * d.d_v * (1 + 1 / 128) + e * T * d.d_model),
        } | {k: v for k, v in decode_kernel_bytes(d, B, n_q, sum_len, e, row_bytes).items()
             if k not in ("q_kv_down", "o_proj")}
    return {
        "q_kv_down": e * ((d.d_cq + D) * d.d_model + T * d.d_model + T * d.d_cq + T * D),
        "q_up": e * (nh * (d.d_nope + d.d_rope) * d.d_cq + T * d.d_cq + T * nh * (d.d_nope + d.d_rope)),
        "absorb": e * (nh * d.d_nope * d.d_c + T * nh * d.d_nope + T * nh * d.d_c),
        "decode_attn": sum_len * rb + e * T * nh * D,
        "decode_combine": e * T * nh * d.d_c,
        "unabsorb": e * (nh * d.d_v * d.d_c + T * nh * d.d_c + T * nh * d.d_v),
        "decode_combine_uv": e * (nh * d.d_v * d.d_c + T * nh * d.d_c + T * nh * d.d_v),
        "q_up_absorb": e * (nh * (d.d_nope + d.d_rope) * d.d_cq + nh * d.d_nope * d.d_c + T * d.d_cq
                            + T * nh * (d.d_c + d.d_rope)),
        "o_proj": e * (d.d_model * nh * d.d_v + T * nh * d.d_v + T * d.d_model),
    }


def decode_step_bytes(d, B, n_q, sum_len, e=2, row_bytes=None, fp8_weights=False):
    """Whole decode step: every weight once, every cached row once, h in, u
    out.  fp8_weights: W_DQ, W_DKV, W_KR and W_O at one byte per element
    plus their block scales."""
    nfp8 = (d.d_cq + d.d_c + d.d_rope) * d.d_model + d.d_model * d.n_heads * d.d_v
    nparams = (d.d_cq * d.d_model + d.n_heads * (d.d_nope + d.d_rope) * d.d_cq + (d.d_c + d.d_rope) * d.d_model
               + d.n_heads * (d.d_nope + d.d_v) * d.d_c + d.d_model * d.n_heads * d.d_v)
    rb = e * (d.d_c + d.d_rope) if row_bytes is None else row_bytes
    wbytes = e * nparams if not fp8_weights else e * (nparams - nfp8) + int(nfp8 * (1 + 4 / 16384))
    return wbytes + e * 2 * B * n_q * d.d_model + sum_len * rb


def prefill_fp8_flops(d, B, L):
    """The part of prefill_flops done by the FP8 projections (W_DQ, W_DKV,
    W_KR, W_O)."""
    T = B * L
    return 2 * T * d.d_model * (d.d_cq + d.d_c + d.d_rope) + 2 * T * d.n_heads * d.d_v * d.d_model


def prefill_flops(d, B, L):
    T = B * L
    pairs = B * L * (L + 1) // 2
    return (2 * T * d.d_model * (d.d_cq + d.d_c + d.d_rope)
            + 2 * T * d.d_cq * d.n_heads * (d.d_nope + d.d_rope)
            + 2 * T * d.d_c * d.n_heads * (d.d_nope + d.d_v)
            + pairs * d.n_heads * 2 * (d.d_nope + d.d_rope + d.d_v)
            + 2 * T * d.n_heads * d.d_v * d.d_model)


def measured_traffic(kernel_label):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE summary, scaled by the copy-kernel
    calibration; None when no summary covers this kernel or its source has
    changed since the counters were taken."""
    import hashlib
    files = {"decode_attn": ("profiles/decode_attn_b32_len4096_traffic.txt",
                             "head_latent_attention_18_amd/csrc/attn_decode.hip"),
             "o_proj": ("profiles/o_proj_b32_traffic.txt",
                        "head_latent_attention_18_amd/csrc/gemm_stream.hip")}
    if kernel_label not in files:
        return None
    summ, src = (os.path.join(ROOT, f) for f in files[kernel_label])
    try:
        kv = {}
        for line in open(summ):
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if kv.get("source_sha256") != sha:
            return None
        return int(float(kv["traffic_bytes"]))
    except (OSError, KeyError, ValueError):
        return None


def kernel_times(run, steps):
    """Run `steps` calls with library kernel timing on; average ms per launch."""
    import torch
    from head_latent_attention_18_amd import libmla as L
    torch.cuda.synchronize()
    L.mla_timing_enable(True)
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    t = L.mla_timing_read()
    L.mla_timing_enable(False)
    return {k: {"avg_ms": ms / max(n, 1), "launches_per_step": n / steps} for k, (ms, n) in t.items()}


def event_times(run, calls):
    """Per-call durations (ms) from torch events on the current stream (every
    kernel of a call is launched on that stream)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for i in range(calls):
        ev[i][0].record()
        run(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def spread(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"ms_median": round(float(np.median(a)), 5), "ms_p10": round(float(np.percentile(a, 10)), 5),
            "ms_p90": round(float(np.percentile(a, 90)), 5), "calls": int(a.size)}


def event_kernels(ktimes):
    return {k: {"avg_us_event_timed": round(v["avg_ms"] * 1e3, 2), "launches_per_step": v["launches_per_step"]}
            for k, v in ktimes.items()}


def run_prefill(args, dev, weights_kind="layer"):
    """Causal prefill of the DeepSeek-V3 layer, batch 1 x 4096 tokens, bf16
    (weights_kind "fp8": block-scaled FP8 projections): per-call event times
    of at least 20 calls (median, p10, p90)."""
    import torch
    from head_latent_attention_18_amd.layer import MlaLayer, upload
    from mla_inputs import make_workload
    f8 = weights_kind == "fp8"
    wp = make_workload(3, weights_fp8=f8)
    lp = MlaLayer.from_host(wp.dims, "bf16", wp.weights_f32, wp.weights_bits, weights_fp8=wp.weights_fp8)
    hp = upload(wp.h_f32, wp.h_bits, True)
    cp = lp.new_cache(wp.batch, wp.seq_len)
    for _ in range(3):
        lp.prefill(hp, cp)
    torch.cuda.synchronize()
    pk = max(20, args.steps // 10)
    st = spread(event_times(lambda i: lp.prefill(hp, cp), pk))
    pdt = st["ms_median"] * 1e-3
    pk_times = kernel_times(lambda i: lp.prefill(hp, cp), pk)
    fl = prefill_flops(wp.dims, wp.batch, wp.seq_len)
    log(f"prefill{' (FP8 projections)' if f8 else ''}: median {pdt * 1e3:.3f} ms (p10 {st['ms_p10']:.3f}, "
        f"p90 {st['ms_p90']:.3f}), {fl / pdt / 1e12:.1f} TFLOPS")
    out = {"workload": wp.name + ("-fp8weights" if f8 else ""), "ms": st["ms_median"], **st,
           "TFLOPS": round(fl / pdt / 1e12, 1), "mfma_frac": round(fl / pdt / 1e12 / BF16_PEAK_TFLOPS, 4),
           "alg_flops": fl, "kernels": event_kernels(pk_times)}
    if f8:
        # the FP8 projections' flops at the FP8 MFMA peak, the rest at bf16
        f8fl = prefill_fp8_flops(wp.dims, wp.batch, wp.seq_len)
        bound = f8fl / (FP8_PEAK_TFLOPS * 1e12) + (fl - f8fl) / (BF16_PEAK_TFLOPS * 1e12)
        out.update({"fp8_flops": f8fl, "mfma_bound_ms": round(bound * 1e3, 4),
                    "mfma_frac": round(bound / pdt, 4)})
    return out


def decode_attn_flops(d, lens, n_q):
    """Absorbed attention flops: 2*(d_c + d_R) for the score and 2*d_c for
    P.V per (query, visible key, head)."""
    import numpy as np
    L = np.asarray(lens, dtype=np.int64)
    vis = int(np.sum(n_q * (L - n_q) + n_q * (n_q + 1) // 2))
    return vis * d.n_heads * 2 * ((d.d_c + d.d_rope) + d.d_c)


def device_cache_rows(d, n, gen, dev, fp8):
    """n cached rows drawn on the device from a seeded generator: bf16
    N(0,1) rows, or FP8 rows by the recipe of mla_inputs.fp8_cache_rows
    (scales 2^-7, 2^-6 or 2^-5 per row and 128-column group, codes of N(0,1)
    draws divided by the scale, clamped to +-448; k_R N(0,1) in bf16)."""
    import torch
    if not fp8:
        out = torch.empty(n, d.d_row, dtype=torch.bfloat16, device=dev)
        for s in range(0, n, 1 << 18):
            e = min(n, s + (1 << 18))
            out[s:e] = torch.empty(e - s, d.d_row, device=dev).normal_(generator=gen).to(torch.bfloat16)
        return out
    G = d.d_c // 128
    out = torch.empty(n, d.d_c + 2 * d.d_rope + 4 * G, dtype=torch.uint8, device=dev)
    for s in range(0, n, 1 << 18):
        e = min(n, s + (1 << 18))
        m = e - s
        x = torch.empty(m, G, 128, device=dev).normal_(generator=gen)
        sc = torch.ldexp(torch.ones(m, G, device=dev),
                         torch.randint(-7, -4, (m, G), generator=gen, device=dev)).contiguous()
        q = (x / sc[:, :, None]).clamp_(-448.0, 448.0).reshape(m, d.d_c)
        out[s:e, :d.d_c] = q.to(torch.float8_e4m3fn).view(torch.uint8)
        kr = torch.empty(m, d.d_rope, device=dev).normal_(generator=gen).to(torch.bfloat16).contiguous()
        out[s:e, d.d_c:d.d_c + 2 * d.d_rope] = kr.view(torch.uint8)
        out[s:e, d.d_c + 2 * d.d_rope:] = sc.view(torch.uint8)
    return out


def run_decode_workload(args, dev, wid, cache_kind="layer", weights_kind="layer"):
    """Decode step of workload 2 (batch 32, cache 4096), 4 (batch 128,
    lengths U{1..32768}, paged 64-row blocks in a permuted order) or 5
    (batch 4, 128K cache, two query tokens), with a bf16 or an FP8 latent
    cache.  Lengths, block order, weights and h come from the workload's
    seed; the cached rows (workload 4: 2.5 GB bf16, 1.4 GB FP8) are drawn on
    the device from a seeded torch generator (device_cache_rows).  Workload 2
    rotates --sets copies of weights and cache so that neither stays in the
    Infinity Cache."""
    import numpy as np
    import torch
    from head_latent_attention_18_amd import libmla as L
    from head_latent_attention_18_amd.layer import CacheBuf, MlaLayer, upload
    from mla_inputs import make_workload
    t0 = time.perf_counter()
    fp8 = cache_kind == "fp8"
    w8 = weights_kind == "fp8"
    wl = make_workload(wid, cache_rows=False, weights_fp8=w8)
    d = wl.dims
    B, nq = wl.batch, wl.n_q
    lens_np = wl.lens.astype(np.int32)
    layer = MlaLayer.from_host(d, "bf16", wl.weights_f32, wl.weights_bits, cache=cache_kind,
                               weights_fp8=wl.weights_fp8)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 + wid + (500 if fp8 else 0))

    def new_cache():
        if wl.paged:
            bs = wl.block_size
            nblk = int(sum((int(l) + bs - 1) // bs for l in lens_np))
            maxb = int(max((int(l) + bs - 1) // bs for l in lens_np))
            table = np.full((B, maxb), -1, dtype=np.int32)
            off = 0
            for b in range(B):
                n = (int(lens_np[b]) + bs - 1) // bs
                table[b, :n] = wl.block_perm[off:off + n]
                off += n
            return CacheBuf.paged(device_cache_rows(d, nblk * bs, gen, dev, fp8), bs, table)
        ml = int(lens_np.max())
        c = CacheBuf(device_cache_rows(d, B * ml, gen, dev, fp8), None, max_len=ml)
        c.desc = L.make_cache(c.pool, max_len=ml)
        return c

    h = upload(wl.h_f32, wl.h_bits, True)
    sets = [(layer, new_cache(), h)]
    for _ in range((args.sets if wid == 2 else 1) - 1):
        lw = MlaLayer(d, "bf16", {k: v.clone() for k, v in layer.weights.items()}, cache=cache_kind,
                      scales={k: v.clone() for k, v in layer.scales.items()} if layer.scales else None)
        sets.append((lw, new_cache(), h.clone()))
    lens = torch.from_numpy(lens_np).to(dev)
    Lmax = int(lens_np.max())
    u = torch.empty(B, nq, d.d_model, dtype=torch.bfloat16, device=dev)

    def run(i):
        lw, c, hh = sets[i % len(sets)]
        lw.decode(hh, lens, Lmax, c, u=u, lens_host=lens_np)

    torch.cuda.synchronize()
    name = wl.name + ("-fp8cache" if fp8 else "") + ("-fp8weights" if w8 else "")
    log(f"workload {name}: set up in {time.perf_counter() - t0:.1f}s, sum of lengths {int(lens_np.sum())}")
    for i in range(5):
        run(i)
    torch.cuda.synchronize()
    k = max(20, args.steps // 10)
    st = spread(event_times(run, k))
    dt = st["ms_median"] * 1e-3
    kt = kernel_times(run, k)
    sum_len = int(lens_np.sum())
    rb = layer.row_width * (1 if fp8 else 2)
    step_bytes = decode_step_bytes(d, B, nq, sum_len, row_bytes=rb, fp8_weights=w8)
    kb = decode_kernel_bytes(d, B, nq, sum_len, row_bytes=rb)["decode_attn"]
    attn_fl = decode_attn_flops(d, lens_np, nq)
    attn_ms = kt["decode_attn"]["avg_ms"]
    t_hbm = kb / (HBM_PEAK_GBS * 1e9)
    t_mfma = attn_fl / (BF16_PEAK_TFLOPS * 1e12)
    bound = "mfma" if t_mfma > t_hbm else "hbm"
    log(f"{name}: median {dt * 1e6:.1f} us/step, attention {attn_ms * 1e3:.1f} us (event-timed), "
        f"bound {bound} {max(t_hbm, t_mfma) * 1e6:.1f} us")
    del sets, layer
    torch.cuda.empty_cache()
    return {"workload": name, "batch": B, "n_q": nq, "sum_len": sum_len, "max_len": Lmax, "paged": wl.paged,
            "cache": cache_kind, "cache_row_bytes": rb, "weights": weights_kind,
            **st, "tokens_per_s": round(B * nq / dt, 1),
            "step_hbm": {"alg_bytes": step_bytes, "GBps": round(step_bytes / dt / 1e9, 1),
                         "frac": round(step_bytes / dt / 1e9 / HBM_PEAK_GBS, 4)},
            "attention": {"alg_bytes": kb, "alg_flops": attn_fl, "us_event_timed": round(attn_ms * 1e3, 2),
                          "hbm_frac": round(kb / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "mfma_frac": round(attn_fl / (attn_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                          "bound": bound, "bound_us": round(max(t_hbm, t_mfma) * 1e6, 2),
                          "frac_of_bound": round(max(t_hbm, t_mfma) / (attn_ms * 1e-3), 4)},
            "kernels": event_kernels(kt)}


def chunk_flops(d, C, P):
    """Algorithmic flops of a chunk of C new tokens against P cached ones in
    the pages' (non-absorbed) form: projections of the chunk, K/V
    up-projection of all P + C keys, causal attention, W_O."""
    pairs = C * P + C * (C + 1) // 2
    return (2 * C * d.d_model * (d.d_cq + d.d_c + d.d_rope)
            + 2 * C * d.d_cq * d.n_heads * (d.d_nope + d.d_rope)
            + 2 * (P + C) * d.d_c * d.n_heads * (d.d_nope + d.d_v)
            + pairs * d.n_heads * 2 * (d.d_nope + d.d_rope + d.d_v)
            + 2 * C * d.n_heads * d.d_v * d.d_model)


def run_chunk(args, dev, C=512, P=4096):
    """Chunked prefill: 512 new tokens of one sequence against a 4096-token
    cached prefix (mla_decode with n_q = 512, causal among the chunk)."""
    import numpy as np
    import torch
    from head_latent_attention_18_amd.layer import MlaLayer, cache_from_rows, upload
    from mla_inputs import make_workload
    wc = make_workload(2, batch=1, uniform_len=P + C, n_q=C)
    lc = MlaLayer.from_host(wc.dims, "bf16", wc.weights_f32, wc.weights_bits)
    cc = cache_from_rows(wc.cache_bits, wc.lens, wc.dims.d_row, True)
    hc = upload(wc.h_f32, wc.h_bits, True)
    lens = torch.from_numpy(wc.lens.astype(np.int32)).to(dev)
    run = lambda i: lc.decode(hc, lens, P + C, cc)
    for i in range(3):
        run(i)
    torch.cuda.synchronize()
    k = max(3, args.steps // 5)
    t0 = time.perf_counter()
    for i in range(k):
        run(i)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / k
    times = kernel_times(run, k)
    fl = chunk_flops(wc.dims, C, P)
    log(f"chunk: {dt * 1e3:.3f} ms, {C / dt:.0f} tokens/s, {fl / dt / 1e12:.1f} TFLOPS (non-absorbed flops)")
    return {"workload": f"dsv3-chunk{C}-prefix{P}", "ms": round(dt * 1e3, 4), "tokens_per_s": round(C / dt, 1),
            "TFLOPS_nonabsorbed": round(fl / dt / 1e12, 1), "alg_flops": fl,
            "kernels": {k2: {"avg_us_event_timed": round(v["avg_ms"] * 1e3, 2),
                             "launches_per_step": v["launches_per_step"]} for k2, v in times.items()}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=3, help="rotated input copies (defeat the Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the ragged and 128K decode workloads")
    ap.add_argument("--cpu-seqs", type=int, default=32, help="sequences in the oracle's first (parity) pass")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="least CPU time of the timed oracle sample")
    ap.add_argument("--only", choices=["all", "decode", "prefill", "chunk", "ragged", "long"], default="all",
                    help="profiling runs: time one path only (the JSON line is printed for 'all' and 'decode')")
    ap.add_argument("--cache", choices=["layer", "fp8"], default="layer",
                    help="latent cache of the --only decode/ragged/long runs (fp8: E4M3 codes + group scales)")
    ap.add_argument("--weights", choices=["layer", "fp8"], default="layer",
                    help="projections of the --only runs (fp8: W_DQ, W_DKV, W_KR, W_O block-scaled E4M3)")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-cache and FP8-weight workloads")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only copy a buffer of this many MB three times (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from head_latent_attention_18_amd import libmla as L
    from head_latent_attention_18_amd.layer import MlaLayer, cache_from_rows, upload
    from mla_inputs import make_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: 3 copies of {args.copy_probe_mb} MiB")
        return
    if args.only == "prefill":
        args.no_cpu_baseline = True

    if args.only == "prefill":
        print(json.dumps(run_prefill(args, dev, args.weights)), flush=True)
        return
    if args.only == "chunk":
        print(json.dumps(run_chunk(args, dev)), flush=True)
        return
    if args.only in ("ragged", "long") or (args.only == "decode" and (args.cache == "fp8" or args.weights == "fp8")):
        wid = {"decode": 2, "ragged": 4, "long": 5}[args.only]
        print(json.dumps(run_decode_workload(args, dev, wid, args.cache, args.weights)), flush=True)
        return

    # ------------------------------------------------------------ decode
    t0 = time.perf_counter()
    wl = make_workload(2)
    d = wl.dims
    B, nq = wl.batch, wl.n_q
    Lmax = int(wl.lens.max())
    log(f"workload {wl.name}: inputs drawn in {time.perf_counter() - t0:.1f}s")
    layer0 = MlaLayer.from_host(d, "bf16", wl.weights_f32, wl.weights_bits)
    cache0 = cache_from_rows(wl.cache_bits, wl.lens, d.d_row, True)
    h0 = upload(wl.h_f32, wl.h_bits, True)
    lens_np = wl.lens.astype(np.int32)
    lens = torch.from_numpy(lens_np).to(dev)
    sets = [(layer0, cache0, h0)]
    for _ in range(args.sets - 1):
        lw = MlaLayer(d, "bf16", {k: v.clone() for k, v in layer0.weights.items()})
        c = type(cache0)(cache0.pool.clone(), None, max_len=cache0.max_len)
        c.desc = L.make_cache(c.pool, max_len=cache0.max_len)
        sets.append((lw, c, h0.clone()))
    outs = [torch.empty(B, nq, d.d_model, dtype=torch.bfloat16, device=dev) for _ in sets]

    def step(i):
        lw, c, h = sets[i % len(sets)]
        lw.decode(h, lens, Lmax, c, u=outs[i % len(sets)], lens_host=lens_np)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    log(f"decode: {dt * 1e6:.1f} us/step")
    ktimes = kernel_times(step, args.steps)
    sum_len = int(wl.lens.sum())
    kbytes = decode_kernel_bytes(d, B, nq, sum_len)
    kernels = {}
    for name, v in ktimes.items():
        ent = {"avg_us_event_timed": round(v["avg_ms"] * 1e3, 2), "launches_per_step": v["launches_per_step"]}
        if name in kbytes:
            gbs = kbytes[name] / (v["avg_ms"] * 1e-3) / 1e9
            ent["alg_bytes"] = kbytes[name]
            ent["alg_GBps"] = round(gbs, 1)
            ent["hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
        kernels[name] = ent
    dom = max((k for k in kernels if k in kbytes), key=lambda k: kernels[k]["avg_us_event_timed"] * kernels[k]["launches_per_step"])
    dom_gbs = kernels[dom]["alg_GBps"]
    step_bytes = decode_step_bytes(d, B, nq, sum_len)

    # sampled parity of the timed output against the oracle (sequences 0 and B-1)
    from oracle import mla_oracle as O
    W = {k: v.astype(np.float64) for k, v in wl.weights_f32.items()}
    u_gpu = outs[(args.steps - 1) % len(sets)].float().cpu().numpy()
    parity = {}
    cpu = None
    t_or = 0.0
    n_or = 0
    for b in ([0, B - 1] + list(range(1, max(0, args.cpu_seqs - 2) + 1))):
        t1 = time.perf_counter()
        ref = O.decode(d, W, wl.h_f32[b].astype(np.float64), wl.cache_f32[b].astype(np.float64))["u"]
        t_or += time.perf_counter() - t1
        n_or += nq
        diff = u_gpu[b] - ref
        parity[f"seq{b}"] = {"max_abs": float(np.max(np.abs(diff))),
                             "rel_frob": float(np.linalg.norm(diff) / np.linalg.norm(ref))}
        if args.no_cpu_baseline and len(parity) >= 2:
            break
    # the timed oracle sample runs for at least --cpu-seconds (whole sequences,
    # cycling over the batch again if one pass is shorter)
    passes = 1
    while not args.no_cpu_baseline and t_or < args.cpu_seconds and passes < 8:
        passes += 1
        for b in range(B):
            t1 = time.perf_counter()
            O.decode(d, W, wl.h_f32[b].astype(np.float64), wl.cache_f32[b].astype(np.float64))
            t_or += time.perf_counter() - t1
            n_or += nq
            if t_or >= args.cpu_seconds:
                break
    if not args.no_cpu_baseline:
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            blas_threads = None
        cores = len(os.sched_getaffinity(0))
        cpu = {"value": round(n_or / t_or, 3), "unit": "tokens/s", "cores": int(blas_threads or cores),
               "kind": "oracle",
               "sample": f"fp64 numpy oracle decode of {n_or} sequence-tokens drawn from the {B} sequences "
                         f"(one token each, cache length {Lmax}), {t_or:.1f}s; host has {cores} cores"}

    del sets, outs
    torch.cuda.empty_cache()

    prefill = None if (args.no_prefill or args.only == "decode") else run_prefill(args, dev)
    ragged = long_ctx = None
    fp8 = None
    if args.only == "all" and not args.no_extra:
        ragged = run_decode_workload(args, dev, 4)
        long_ctx = run_decode_workload(args, dev, 5)
    fp8w = None
    if args.only == "all" and not args.no_fp8:
        fp8 = {"b32_len4096": run_decode_workload(args, dev, 2, "fp8")}
        if not args.no_extra:
            fp8["ragged"] = run_decode_workload(args, dev, 4, "fp8")
            fp8["long"] = run_decode_workload(args, dev, 5, "fp8")
        fp8w = {"decode_b32_len4096": run_decode_workload(args, dev, 2, "layer", "fp8"),
                "decode_b32_len4096_fp8cache": run_decode_workload(args, dev, 2, "fp8", "fp8")}
        if not args.no_prefill:
            fp8w["prefill_len4096"] = run_prefill(args, dev, "fp8")

    out = {
        "metric": "MLA decode tokens/s (DeepSeek-V3 layer, batch 32, cache 4096)",
        "value": round(B * nq / dt, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "n_q": nq, "cache_len": Lmax, "d_model": d.d_model,
                   "n_heads": d.n_heads, "d_c": d.d_c, "d_rope": d.d_rope, "paged": False},
        "step_hbm": {"alg_bytes": step_bytes, "GBps": round(step_bytes / dt / 1e9, 1),
                     "frac": round(step_bytes / dt / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": dom_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dom),
                     "alg_bytes": kbytes[dom]},
        "kernels": kernels,
        "kernel_timing": "HIP events recorded around each launch on its stream (about 2 us per launch above the "
                         "kernel's own duration; rocprofv3 kernel traces under profiles/ give the durations alone)",
        "parity": parity,
        "prefill": prefill,
        "decode_ragged": ragged,
        "decode_long": long_ctx,
        "decode_fp8_cache": fp8,
        "fp8_weights": fp8w,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
