#!/usr/bin/env python3
"""Benchmark of the KV4-RL hybrid decode-attention path on one MI355X.

Workload (qwen8b-shaped decode step): B=256 sequences, Hq/Hkv = 32/8, head_dim
128, page 16, 36 layers, contexts = U[128,512] prompt + a length-biased
lognormal(mean 3000, sd 2250) response position (+ this step's token).  One
step = for each of the 36 layers: the append of one token per sequence and
the decode attention, in one launch (kv4_append_decode_attention).  Every layer has its own cache, so the step streams
~28 GB of INT4 pages and never hits the 256 MB last-level cache.

Prints one JSON line: decode-attention tokens/s (whole step), achieved HBM
GB/s of the decode against the 8 TB/s peak, the roofline of the dominant
kernel (timed with HIP events on its own stream), the in-build BF16 paged
decode for the speed ratio, the re-prefill timing, and the CPU oracle timed on
a bounded sample on the host cores.
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

METRIC = "decode-attn tokens/s + achieved HBM GB/s (% of peak), B=256 mixed ctx, 1 GPU"
PEAK_GBS = 8000.0
WORKLOAD = 4
LAYERS = 36
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "main_kernel_traffic_qwen8b.json")
MAIN_SOURCES = [os.path.join(ROOT, "int8_mixed_precision_kv4_amd", "csrc", f)
                for f in ("kv4_decode.hip", "kv4_device.hpp")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the main kernel's sources with comments and whitespace removed,
    so that only a change of code invalidates the stored traffic figure."""
    import re
    h = hashlib.sha256()
    for f in MAIN_SOURCES:
        text = open(f, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(re.sub(r"\s+", "", text).encode())
    return h.hexdigest()[:16]


def metric_bytes(ctx, Hkv):
    """Bytes per layer by the metric's formula: sum ctx*Hkv*128*2*4.25/8 plus
    the side rows read (min(ctx,144) rows of 2x(128+2) bytes per kv-head)."""
    import numpy as np
    ctx = np.asarray(ctx, dtype=np.int64)
    return int((ctx * Hkv * 136).sum() + (np.minimum(ctx, 144) * Hkv * 260).sum())


def main_kernel_bytes(ctx, Hkv):
    """Algorithmic bytes of the main kernel per launch: 136 B (64 B K codes +
    64 B V codes + 4 B + 4 B FP16 metadata) per main (position, kv-head), plus
    the protected region its last workgroups read: 260 B (2 x 128 B INT8
    codes + 2 x 2 B FP16 scales) per side (position, kv-head), plus this
    step's append done by those workgroups: 512 B of BF16 K and V read, 136 B
    of page entry and 260 B of side row written per (sequence, kv-head)."""
    import numpy as np
    ctx = np.asarray(ctx, dtype=np.int64)
    return int((np.maximum(ctx - 144, 0) * Hkv * 136).sum() + (np.minimum(ctx, 144) * Hkv * 260).sum()
               + len(ctx) * Hkv * (512 + 136 + 260))


class HipEvents:
    """Raw hipEvent_t pairs (hipEventCreate / hipEventElapsedTime) so the
    library can record them on the stream the kernel is launched on."""

    def __init__(self, n):
        import ctypes
        self.C = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e)

    def pair(self, i):
        return self.ev[2 * i], self.ev[2 * i + 1]

    def elapsed_ms(self, i):
        ms = self.C.c_float()
        e0, e1 = self.pair(i)
        assert self.hip.hipEventSynchronize(e1) == 0
        assert self.hip.hipEventElapsedTime(self.C.byref(ms), e0, e1) == 0
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def build_layers(wl, dev, with_bf16=True):
    import numpy as np
    import torch

    import int8_mixed_precision_kv4_amd as kv4
    from synth import draw_values

    n_tok = int(wl.ctx.sum())
    off = np.zeros(wl.B + 1, np.int64)
    off[1:] = np.cumsum(wl.ctx)
    lead = wl.ctx - 1
    rows_lead = torch.from_numpy(np.concatenate(
        [np.arange(off[b], off[b] + lead[b]) for b in range(wl.B)])).to(dev)
    rows_last = torch.from_numpy(off[:-1] + lead).to(dev)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lead)]).astype(np.int32)).to(dev)
    zeros = torch.zeros(wl.B, dtype=torch.int32, device=dev)
    table = torch.from_numpy(wl.page_table).to(dev)
    slots = torch.from_numpy(wl.slots).to(dev)
    # physical page and in-page slot of every position (for the BF16 pools)
    pos_all = np.concatenate([np.arange(n) for n in wl.ctx])
    seq_all = np.repeat(np.arange(wl.B), wl.ctx)
    page_all = torch.from_numpy(wl.page_table[seq_all, pos_all // 16].astype(np.int64)).to(dev)
    t_all = torch.from_numpy((pos_all % 16).astype(np.int64)).to(dev)
    layers = []
    for layer in range(wl.layers):
        k, v, q = draw_values(wl.seed, layer, n_tok, wl.B, wl.Hq, wl.Hkv, device=dev)
        cache = kv4.Kv4Cache.zeros(wl.num_pages, wl.Hkv, wl.max_slots, dev)
        kv4.prefill_quantize(cache, k[rows_lead].contiguous(), v[rows_lead].contiguous(), cu, zeros,
                             slots, table, int(lead.max()))
        L = dict(cache=cache, q=q, k_app=k[rows_last].contiguous(), v_app=v[rows_last].contiguous())
        if with_bf16:
            pool = torch.empty((wl.num_pages, wl.Hkv, 2, 16, 128), dtype=torch.bfloat16, device=dev)
            pool[page_all, :, 0, t_all, :] = k
            vview = pool.view(wl.num_pages, wl.Hkv, 2, 2048)[:, :, 1].view(wl.num_pages, wl.Hkv, 128, 16)
            vview[page_all, :, :, t_all] = v
            L["bf16"] = pool
        if layer == 0:
            L["k_all"], L["v_all"] = k, v
        else:
            del k, v
        layers.append(L)
        if layer % 6 == 5:
            log(f"built {layer + 1}/{wl.layers} layers")
    torch.cuda.synchronize()
    return layers, dict(table=table, slots=slots, offsets=off)


def fp64_attention(q, k, v, ctx, off, sample, scale):
    """Exact attention of the sampled sequences in FP64 on the unquantized BF16
    keys and values (the reference the variants' error is measured against):
    out[b, h] = softmax(scale * q[b, h] . K_b^T) V_b over positions [0, ctx_b)."""
    import torch
    outs = []
    Hq, Hkv = q.shape[1], k.shape[1]
    for b in sample:
        n = int(ctx[b])
        K = k[int(off[b]):int(off[b]) + n].double()  # [n][Hkv][128]
        V = v[int(off[b]):int(off[b]) + n].double()
        Q = q[int(b)].double().view(Hkv, Hq // Hkv, 128)              # [Hkv][G][128]
        Kt = K.permute(1, 2, 0).contiguous()                             # [Hkv][128][n]
        Vg = V.permute(1, 0, 2).contiguous()                             # [Hkv][n][128]
        p = torch.softmax(torch.matmul(Q, Kt) * scale, dim=-1)          # [Hkv][G][n]
        outs.append(torch.matmul(p, Vg).reshape(Hq, 128))
    return torch.stack(outs)


def variant_leg(wl, layers, sh, ctx, scale, steps, t_bf16):
    """Protection-budget variants through the same kernels (unprotected KV4,
    all-sink, all-recent, and the default split): the side rows of every layer
    are rebuilt for each budget (the INT4 pages do not depend on it), then the
    36-layer decode is timed, the main kernel is timed with HIP events, and the
    output of layer 0 on sampled sequences is compared with exact FP64
    attention."""
    import numpy as np
    import torch

    import int8_mixed_precision_kv4_amd as kv4
    from synth import draw_values

    dev = ctx.device
    table, slots, off = sh["table"], sh["slots"], sh["offsets"]
    B, Hq = wl.B, wl.Hq
    lead = wl.ctx - 1
    n_tok = int(wl.ctx.sum())
    rows_lead = torch.from_numpy(np.concatenate(
        [np.arange(off[b], off[b] + lead[b]) for b in range(B)])).to(dev)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lead)]).astype(np.int32)).to(dev)
    zeros = torch.zeros(B, dtype=torch.int32, device=dev)
    pos = (ctx - 1).contiguous()
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(kv4.decode_workspace_bytes(layers[0]["cache"], B, Hq, wl.max_ctx),
                     dtype=torch.uint8, device=dev)
    order = np.argsort(wl.ctx, kind="stable")
    sample = np.unique(np.concatenate([order[:2], order[-2:], order[::max(1, B // 8)][:8]]))
    k0, v0 = layers[0]["k_all"], layers[0]["v_all"]
    ref = fp64_attention(layers[0]["q"], k0, v0, wl.ctx, off, sample, scale)
    sel = torch.from_numpy(sample).to(dev)
    res = {}
    for s, w in ((0, 0), (144, 0), (0, 144), (16, 128)):
        name = "kv4" if s + w == 0 else f"kv4rl_s{s}_w{w}"
        log(f"variant {name}: rebuilding side rows of {wl.layers} layers")
        caches = []
        for li, L in enumerate(layers):
            c = L["cache"]
            vc = kv4.Kv4Cache(c.pages, c.side_codes, c.side_scales, sink=s, window=w)
            if li == 0:
                k, v = k0, v0
            else:
                k, v, _ = draw_values(wl.seed, li, n_tok, B, Hq, wl.Hkv, device=dev)
            c.side_codes.zero_()
            c.side_scales.zero_()
            kv4.prefill_quantize(vc, k[rows_lead].contiguous(), v[rows_lead].contiguous(), cu, zeros,
                                 slots, table, int(lead.max()))
            kv4.append(vc, L["k_app"], L["v_app"], pos, slots, table)
            del k, v
            caches.append(vc)
        torch.cuda.synchronize()

        def dstep():
            for vc, L in zip(caches, layers):
                kv4.decode_attention(vc, L["q"], ctx, slots, table, wl.max_ctx, scale, out, lse, ws)

        for _ in range(2):
            dstep()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            dstep()
        torch.cuda.synchronize()
        t = (time.perf_counter() - t0) / steps
        evs = HipEvents(len(caches))
        for i, (vc, L) in enumerate(zip(caches, layers)):
            e0, e1 = evs.pair(i)
            kv4.decode_attention_timed(vc, L["q"], ctx, slots, table, wl.max_ctx, scale, out, lse,
                                       ws, e0, e1)
        torch.cuda.synchronize()
        main_us = float(np.mean([evs.elapsed_ms(i) for i in range(len(caches))])) * 1e3
        evs.close()
        kv4.decode_attention(caches[0], layers[0]["q"], ctx, slots, table, wl.max_ctx, scale, out,
                             lse, ws)
        torch.cuda.synchronize()
        err = (out[sel].double() - ref).abs()
        res[name] = dict(sink=s, window=w, decode_ms_per_step=round(t * 1e3, 3),
                         decode_tokens_per_s=round(B / t, 1), main_kernel_us=round(main_us, 2),
                         speedup_vs_bf16=round(t_bf16 / t, 3) if t_bf16 else None,
                         err_vs_fp64_maxabs=float(err.max()), err_vs_fp64_meanabs=float(err.mean()))
        log(f"variant {name}: {t * 1e3:.3f} ms/step, main {main_us:.1f} us, "
            f"max err vs FP64 {float(err.max()):.3e}")
    # MXFP4 main region (OCP MXFP4 pages, the same side rows and budget):
    # the layers' caches are rewritten in that format in place
    log(f"variant mxfp4: rewriting the pages of {wl.layers} layers in MXFP4")
    rows_last = torch.from_numpy(off[:-1] + lead).to(dev)
    for li, L in enumerate(layers):
        if li == 0:
            k, v = k0, v0
        else:
            k, v, _ = draw_values(wl.seed, li, n_tok, B, Hq, wl.Hkv, device=dev)
        c = L["cache"]
        mc = kv4.Kv4Cache(c.pages, c.side_codes, c.side_scales)
        kv4.mx_prefill_quantize(mc, k[rows_lead].contiguous(), v[rows_lead].contiguous(), cu, zeros,
                                slots, table, int(lead.max()))
        kv4.mx_append(mc, L["k_app"], L["v_app"], pos, slots, table)
        del k, v
    torch.cuda.synchronize()

    def mx_step():
        for L in layers:
            kv4.mx_decode_attention(L["cache"], L["q"], ctx, slots, table, wl.max_ctx, scale, out, lse, ws)

    for _ in range(2):
        mx_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        mx_step()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / steps
    kv4.mx_decode_attention(layers[0]["cache"], layers[0]["q"], ctx, slots, table, wl.max_ctx, scale, out,
                            lse, ws)
    torch.cuda.synchronize()
    err = (out[sel].double() - ref).abs()
    res["mxfp4_rl"] = dict(sink=16, window=128, decode_ms_per_step=round(t * 1e3, 3),
                           decode_tokens_per_s=round(B / t, 1),
                           speedup_vs_bf16=round(t_bf16 / t, 3) if t_bf16 else None,
                           err_vs_fp64_maxabs=float(err.max()), err_vs_fp64_meanabs=float(err.mean()))
    log(f"variant mxfp4: {t * 1e3:.3f} ms/step, max err vs FP64 {float(err.max()):.3e}")

    # KV8 everywhere: every position in the side rows' INT8 representation,
    # attended with the protected path's arithmetic (its own pool per layer)
    for L in layers:
        L.pop("bf16", None)
    torch.cuda.empty_cache()
    log(f"variant kv8: building the INT8 pools of {wl.layers} layers")
    pools = []
    for li, L in enumerate(layers):
        if li == 0:
            k, v = k0, v0
        else:
            k, v, _ = draw_values(wl.seed, li, n_tok, B, Hq, wl.Hkv, device=dev)
        c8 = kv4.Kv8Cache.zeros(wl.num_pages, wl.Hkv, dev)
        kv4.kv8_prefill_quantize(c8, k[rows_lead].contiguous(), v[rows_lead].contiguous(), cu, zeros,
                                 table, int(lead.max()))
        kv4.kv8_append(c8, k[rows_last].contiguous(), v[rows_last].contiguous(), pos, table)
        del k, v
        pools.append(c8)
    torch.cuda.synchronize()
    ws8 = torch.empty(kv4.kv8_decode_workspace_bytes(pools[0], B, Hq, wl.max_ctx), dtype=torch.uint8,
                      device=dev)

    def kv8_step():
        for c8, L in zip(pools, layers):
            kv4.kv8_decode_attention(c8, L["q"], ctx, table, wl.max_ctx, scale, out, lse, ws8)

    for _ in range(2):
        kv8_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        kv8_step()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / steps
    kv4.kv8_decode_attention(pools[0], layers[0]["q"], ctx, table, wl.max_ctx, scale, out, lse, ws8)
    torch.cuda.synchronize()
    err = (out[sel].double() - ref).abs()
    kv8_bytes = int((wl.ctx.astype(np.int64) * wl.Hkv * 260).sum())
    res["kv8"] = dict(decode_ms_per_step=round(t * 1e3, 3), decode_tokens_per_s=round(B / t, 1),
                      hbm_gbps=round(kv8_bytes * len(pools) / t / 1e9, 1),
                      speedup_vs_bf16=round(t_bf16 / t, 3) if t_bf16 else None,
                      err_vs_fp64_maxabs=float(err.max()), err_vs_fp64_meanabs=float(err.mean()))
    log(f"variant kv8: {t * 1e3:.3f} ms/step, max err vs FP64 {float(err.max()):.3e}")
    del pools, ws8
    torch.cuda.empty_cache()
    for name in res:
        res[name]["throughput_vs_kv4"] = round(res["kv4"]["decode_ms_per_step"] /
                                               res[name]["decode_ms_per_step"], 4)
    return dict(workload="qwen8b decode step, 36 layers, decode only",
                error_sample=(f"layer 0, sequences {sample.tolist()}, all {Hq} heads, vs exact FP64 "
                              "attention on the unquantized BF16 K/V"),
                budgets=res)


def prefill_leg(wl, dev, scale, steps):
    """The benchmark's re-prefill of 8 sequences x 16384 tokens (one layer,
    Hkv = 8): the quantize kernel (kv4_prefill_quantize) timed over several
    calls, then the attention half (kv4_prefill_attention) of the same chunks."""
    import numpy as np
    import torch

    import int8_mixed_precision_kv4_amd as kv4
    from synth import draw_values

    log("timing the 8 x 16384-token re-prefill")
    nseq, n = wl.prefill_nseq, wl.prefill_len
    pk, pv, _ = draw_values(wl.seed, 1000, nseq * n, 1, 4, wl.Hkv, device=dev)
    ppages = nseq * n // 16
    pcache = kv4.Kv4Cache.zeros(ppages, wl.Hkv, nseq, dev)
    ptable = torch.arange(ppages, dtype=torch.int32, device=dev).view(nseq, n // 16)
    pcu = torch.arange(0, nseq * n + 1, n, dtype=torch.int32, device=dev)
    pstart = torch.zeros(nseq, dtype=torch.int32, device=dev)
    pslot = torch.arange(nseq, dtype=torch.int32, device=dev)
    t_pre = _timed(lambda: kv4.prefill_quantize(pcache, pk, pv, pcu, pstart, pslot, ptable, n),
                   max(3, steps // 2), 2)
    pbytes = nseq * n * wl.Hkv * (512 + 136)
    res = dict(prefill_ms_per_layer=round(t_pre * 1e3, 3), prefill_gbps=round(pbytes / t_pre / 1e9, 1),
               prefill_frac_of_peak=round(pbytes / t_pre / 1e9 / PEAK_GBS, 4))
    del pk, pv
    # the attention half: every token of each 16384-token chunk attends its prefix
    log("timing the re-prefill attention of the 8 x 16384 tokens")
    pq = draw_values(wl.seed, 1001, 1, nseq * n, wl.Hq, wl.Hkv, device=dev)[2]
    pws = torch.empty(kv4.prefill_attention_workspace_bytes(pcache, nseq * n, wl.Hq, n),
                      dtype=torch.uint8, device=dev)
    pout = torch.empty((nseq * n, wl.Hq, 128), dtype=torch.float32, device=dev)
    plse = torch.empty((nseq * n, wl.Hq), dtype=torch.float32, device=dev)
    t_att = _timed(lambda: kv4.prefill_attention(pcache, pq, pcu, pstart, pslot, ptable, n, scale, pout,
                                                 plse, pws), 2, 1)
    pos = np.arange(n, dtype=np.int64)
    per_seq = (np.maximum(pos + 1 - 144, 0) * 136 + np.minimum(pos + 1, 144) * 260).sum()
    # bytes of cache the tokens attend (each tile is served to 8 tokens from
    # one load, so this is attended bytes per second, not HBM traffic)
    res.update(prefill_attention_ms_per_layer=round(t_att * 1e3, 3),
               prefill_attention_attended_gb_per_s=round(per_seq * nseq * wl.Hkv / t_att / 1e9, 1),
               prefill_attention_finite=bool(torch.isfinite(pout).all()))
    del pq, pws, pout, plse, pcache
    torch.cuda.empty_cache()
    return res


def _timed(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def cpu_baseline(wl, layer0, shared, budget_s):
    """The oracle as it stands, on the host cores, on layer 0 of the step (all
    256 sequences): one append + one 32-head decode, repeated until about
    budget_s seconds; extrapolated to the 36-layer step."""
    import numpy as np
    import torch

    import oracle

    def bf16_bits(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    sample = np.arange(wl.B)
    ctx = wl.ctx[sample]
    off = shared["offsets"]
    need = (ctx + 15) // 16
    table = np.zeros((len(sample), int(need.max())), np.int32)
    table_flat = np.arange(int(need.sum()), dtype=np.int32)
    o = 0
    for i, n in enumerate(need):
        table[i, :n] = table_flat[o:o + n]
        o += n
    k_all, v_all = layer0["k_all"], layer0["v_all"]
    rows = np.concatenate([np.arange(off[b], off[b] + wl.ctx[b] - 1) for b in sample])
    k = bf16_bits(k_all[rows].cpu())
    v = bf16_bits(v_all[rows].cpu())
    cu = np.concatenate([[0], np.cumsum(ctx - 1)]).astype(np.int32)
    q = bf16_bits(layer0["q"][sample].cpu())
    ka = bf16_bits(layer0["k_app"][sample].cpu())
    va = bf16_bits(layer0["v_app"][sample].cpu())
    threads = oracle.default_threads()
    cache = oracle.Cache(int(need.sum()), wl.Hkv, len(sample))
    slots = np.arange(len(sample), dtype=np.int32)
    oracle.prefill(cache, k, v, cu, np.zeros(len(sample), np.int32), slots, table, threads)
    reps, t_total = 0, 0.0
    while t_total < budget_s and reps < 50:
        t0 = time.perf_counter()
        oracle.append(cache, ka, va, (ctx - 1).astype(np.int32), slots, table)
        out, lse, _ = oracle.decode(cache, q, ctx.astype(np.int32), slots, table, wl.Hq,
                                    1.0 / math.sqrt(128), nthreads=threads)
        t_total += time.perf_counter() - t0
        reps += 1
    t_layer_sample = t_total / reps
    t_step = t_layer_sample * (wl.ctx.sum() / ctx.sum()) * wl.layers
    # the same layer once on one thread
    t0 = time.perf_counter()
    oracle.append(cache, ka, va, (ctx - 1).astype(np.int32), slots, table)
    oracle.decode(cache, q, ctx.astype(np.int32), slots, table, wl.Hq, 1.0 / math.sqrt(128), nthreads=1)
    t_single = time.perf_counter() - t0
    cpu = open("/proc/cpuinfo").read().split("model name")[1].split("\n")[0].strip(" :\t") \
        if os.path.exists("/proc/cpuinfo") else "unknown"
    return dict(value=round(wl.B / t_step, 3), unit="tokens/s", cores=threads, kind="oracle",
                sample=(f"layer 0 of 36 (all {len(sample)} sequences, mean ctx {ctx.mean():.0f}): "
                        f"append + 32-head decode, {reps} reps in {t_total:.1f}s; x36 layers"),
                cpu=cpu, single_thread_layer_s=round(t_single, 3)), (sample, out, lse, cache, table, need)


def traffic_from_counters(fetch_db, write_db, command):
    """Write TRAFFIC_FILE from two rocprofv3 --pmc runs of this script (one
    with FETCH_SIZE, one with WRITE_SIZE; KiB per dispatch).  Each counter is
    scaled by what it reads for the 2 GiB device copy the script also runs,
    whose true traffic is 2 GiB read and 2 GiB written."""
    import re
    import sqlite3

    def per_kernel(db, counter):
        con = sqlite3.connect(db)
        rows = con.execute("select name, counter_name, counter_value from pmc_events").fetchall()
        out = {}
        for name, cn, val in rows:
            if cn != counter:
                continue
            out.setdefault(name, []).append(float(val))
        return out

    def pick(d, pattern):
        hits = [k for k in d if re.search(pattern, k)]
        assert hits, (pattern, list(d)[:10])
        return hits

    fetch = per_kernel(fetch_db, "FETCH_SIZE")
    write = per_kernel(write_db, "WRITE_SIZE")
    main_k = pick(fetch, r"main_kernel<.*Kv4Format, false>")[0]
    # the 2 GiB device copy: the largest dispatch of the runtime's copy kernel
    copy_f = max(v for k in pick(fetch, r"copyBuffer") for v in fetch[k])
    copy_w = max(v for k in pick(write, r"copyBuffer") for v in write[k])
    f_scale = 2 ** 31 / (copy_f * 1024)
    w_scale = 2 ** 31 / (copy_w * 1024)
    import numpy as np
    f_main = float(np.mean(fetch[main_k])) * 1024 * f_scale
    w_main = float(np.mean(write[main_k])) * 1024 * w_scale
    rec = {"kernel": main_k, "workload": "qwen8b decode step, one layer",
           "source_hash": source_hash(),
           "fetch_bytes_per_launch": round(f_main), "write_bytes_per_launch": round(w_main),
           "bytes_per_launch": round(f_main + w_main),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "copy_counter_kib": {"FETCH_SIZE": copy_f, "WRITE_SIZE": copy_w},
           "launches": len(fetch[main_k]), "command": command}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(rec))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--traffic-from":
        traffic_from_counters(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle CPU work")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--library", default=None,
                    help="another build of libkv4 to load instead of the package's (for A/B measurements of "
                         "build variants made with int8_mixed_precision_kv4_amd/build.py --define/--out)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the 8 x 16384-token re-prefill leg (quantize + attention) and "
                         "print its figures (for profiling those kernels)")
    ap.add_argument("--no-copy", action="store_true", help="skip the 2 GiB device copy probe")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay of the step")
    ap.add_argument("--workload", choices=("qwen8b", "refill"), default="qwen8b",
                    help="qwen8b: contexts from the length-biased sampler; refill: the B=256 batch "
                         "of one steady-state step of a simulated continuous-refill run, same law")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the protection-budget variants (run last; they rebuild the side rows)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path has no multi-GPU part "
              "(sequences and kv-heads shard with no exchange).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import int8_mixed_precision_kv4_amd as kv4
    from synth import make_workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.library:
        kv4.LIB_PATH = os.path.abspath(args.library)
    kv4.lib()
    wl = make_workload(WORKLOAD)
    if args.prefill_only:
        print(json.dumps(dict(workload="re-prefill of 8 x 16384 tokens, one layer, Hq/Hkv = 32/8",
                              **prefill_leg(wl, dev, 1.0 / math.sqrt(128), args.steps))), flush=True)
        return
    if args.workload == "refill":
        from synth.concentration import LengthLaw, refill_snapshot
        wl = make_workload(WORKLOAD, ctx=refill_snapshot(LengthLaw.lognormal(3000, 2250), wl.B, wl.seed))
    scale = 1.0 / math.sqrt(128)
    log(f"workload qwen8b: B={wl.B} Hq/Hkv={wl.Hq}/{wl.Hkv} mean ctx {wl.ctx.mean():.0f} "
        f"max {wl.max_ctx} pages/layer {wl.num_pages}")
    layers, sh = build_layers(wl, dev, with_bf16=not args.no_bf16)
    table, slots = sh["table"], sh["slots"]
    ctx = torch.from_numpy(wl.ctx.astype(np.int32)).to(dev)
    pos = (ctx - 1).contiguous()
    B, Hq = wl.B, wl.Hq
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(kv4.decode_workspace_bytes(layers[0]["cache"], B, Hq, wl.max_ctx),
                     dtype=torch.uint8, device=dev)

    def step(decode_only=False):
        for L in layers:
            if decode_only:
                kv4.decode_attention(L["cache"], L["q"], ctx, slots, table, wl.max_ctx, scale,
                                     out, lse, ws)
            else:  # this step's append and the decode in one launch
                kv4.append_decode_attention(L["cache"], L["k_app"], L["v_app"], pos, L["q"], ctx, slots,
                                            table, wl.max_ctx, scale, out, lse, ws)

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    log("timing the 36-layer step (append + decode)")
    t_step = timed(step, args.steps, args.warmup)
    t_decode = timed(lambda: step(True), args.steps, 2)

    extra = {}
    if not args.no_graph:
        # the same 36-layer step captured once in a HIP graph and replayed
        log("timing the step replayed from a HIP graph")
        step()
        torch.cuda.synchronize()
        eager_out, eager_lse = out.clone(), lse.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        t_graph = timed(graph.replay, args.steps, 2)
        torch.cuda.synchronize()
        same = bool(torch.equal(out, eager_out) and torch.equal(lse, eager_lse))
        extra.update(graph_ms_per_step=round(t_graph * 1e3, 4),
                     graph_tokens_per_s=round(B / t_graph, 1), graph_output_bit_identical=same)
        del graph

    # dominant kernel: main-region decode kernel, HIP events on its stream
    log("timing the main-region kernel with HIP events")
    evs = HipEvents(LAYERS * args.steps)
    for r in range(args.steps):
        for li, L in enumerate(layers):
            e0, e1 = evs.pair(r * LAYERS + li)
            kv4.decode_attention_timed(L["cache"], L["q"], ctx, slots, table, wl.max_ctx, scale,
                                       out, lse, ws, e0, e1, k=L["k_app"], v=L["v_app"], pos=pos)
    torch.cuda.synchronize()
    main_ms = float(np.mean([evs.elapsed_ms(i) for i in range(LAYERS * args.steps)]))
    evs.close()
    main_bytes = main_kernel_bytes(wl.ctx, wl.Hkv)
    achieved = main_bytes / (main_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE) and args.workload == "qwen8b":
        # the stored counters were taken on the qwen8b contexts: another
        # context mix moves other bytes, so the figure applies to this one only
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("source_hash") == source_hash():
            traffic = rec.get("bytes_per_launch")

    t_bf16 = None
    if not args.no_bf16:
        log("timing the BF16 paged decode comparator")
        bws = torch.empty(kv4.bf16_workspace_bytes(B, Hq, wl.Hkv, wl.max_ctx), dtype=torch.uint8,
                          device=dev)
        bout = torch.empty_like(out)
        blse = torch.empty_like(lse)

        def bstep():
            for L in layers:
                kv4.bf16_paged_decode(L["bf16"], L["q"], ctx, table, wl.max_ctx, scale, bout, blse, bws)

        t_bf16 = timed(bstep, args.steps, 2)
        bf16_bytes = int((wl.ctx.astype(np.int64) * wl.Hkv * 512).sum())
        # agreement of the two paths on the last layer (quantization error, information only)
        kv4.decode_attention(layers[-1]["cache"], layers[-1]["q"], ctx, slots, table, wl.max_ctx,
                             scale, out, lse, ws)
        kv4.bf16_paged_decode(layers[-1]["bf16"], layers[-1]["q"], ctx, table, wl.max_ctx, scale,
                              bout, blse, bws)
        torch.cuda.synchronize()
        extra.update(bf16_decode_ms_per_step=round(t_bf16 * 1e3, 3),
                     bf16_hbm_gbps=round(bf16_bytes * LAYERS / t_bf16 / 1e9, 1),
                     speedup_decode_vs_bf16=round(t_bf16 / t_decode, 3),
                     kv4_vs_bf16_out_maxabs=float((out - bout).abs().max()))
    if not args.no_prefill:
        extra.update(prefill_leg(wl, dev, scale, args.steps))

    if not args.no_copy:
        # plain device-to-device copy of a known size: the box's practical HBM
        # rate, and the scale of the FETCH_SIZE / WRITE_SIZE counters
        src = torch.empty(2 ** 31, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        t_copy = timed(lambda: dst.copy_(src), 10, 2)
        extra["copy_2GiB_gbps"] = round(2 * 2 ** 31 / t_copy / 1e9, 1)
        del src, dst

    cpu = None
    if not args.no_cpu:
        log("oracle CPU baseline")
        cpu, (sample, ref_out, ref_lse, ref_cache, ref_table, need) = cpu_baseline(wl, layers[0], sh,
                                                                                   args.cpu_budget)
        # parity of the timed launch itself (the one-launch step; re-appending
        # this step's token rewrites the same bytes) on layer 0, every sequence
        L0 = layers[0]
        kv4.append_decode_attention(L0["cache"], L0["k_app"], L0["v_app"], pos, L0["q"], ctx, slots, table,
                                    wl.max_ctx, scale, out, lse, ws)
        torch.cuda.synchronize()
        sel = torch.from_numpy(sample).to(dev)
        extra["sample_parity_out_maxabs"] = float(np.abs(out[sel].cpu().numpy() - ref_out).max())
        extra["sample_parity_lse_maxabs"] = float(np.abs(lse[sel].cpu().numpy() - ref_lse).max())
        gpu_ids = np.concatenate([wl.page_table[b, :need[i]] for i, b in enumerate(sample)]).astype(np.int64)
        ref_ids = np.concatenate([ref_table[i, :need[i]] for i in range(len(sample))]).astype(np.int64)
        slot_ids = torch.from_numpy(wl.slots[sample].astype(np.int64)).to(dev)
        extra["sample_parity_pages_equal"] = bool(
            np.array_equal(L0["cache"].pages[torch.from_numpy(gpu_ids).to(dev)].cpu().numpy(),
                           ref_cache.pages[ref_ids])
            and np.array_equal(L0["cache"].side_codes[slot_ids].cpu().numpy(), ref_cache.side_codes)
            and np.array_equal(L0["cache"].side_scales[slot_ids].cpu().numpy().view(np.uint16),
                               ref_cache.side_scales))
        extra["sample_parity_launch"] = "kv4_append_decode_attention (the timed launch), layer 0, all sequences"

    if not args.no_variants:
        extra["variants"] = variant_leg(wl, layers, sh, ctx, scale, max(3, args.steps // 2), t_bf16)

    mb = metric_bytes(wl.ctx, wl.Hkv)
    rec = {
        "metric": METRIC,
        "value": round(B / t_step, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": ("qwen8b decode step: B=256, Hq/Hkv=32/8, head_dim 128, page 16, "
                                "36 layers, ctx = U[128,512] + length-biased lognormal(3000, 2250) "
                                "position + 1; per layer kv4_append_decode_attention (this step's "
                                "append and the decode in one launch)"
                                + ("; contexts replayed from one steady-state step of a simulated "
                                   "continuous-refill run" if args.workload == "refill" else "")),
                   "B": B, "layers": LAYERS, "mean_ctx": round(float(wl.ctx.mean()), 1),
                   "max_ctx": wl.max_ctx, "parallelism": "single GPU"},
        "decode_tokens_per_s": round(B / t_decode, 1),
        "decode_ms_per_step": round(t_decode * 1e3, 4),
        "append_ms_per_step": round((t_step - t_decode) * 1e3, 4),
        # the metric's byte formula over the decode-only step, and over the
        # timed step (this step's appends included, same bytes)
        "hbm_gbps": round(mb * LAYERS / t_decode / 1e9, 1),
        "hbm_frac_of_peak": round(mb * LAYERS / t_decode / 1e9 / PEAK_GBS, 4),
        "hbm_gbps_with_append": round(mb * LAYERS / t_step / 1e9, 1),
        "hbm_frac_of_peak_with_append": round(mb * LAYERS / t_step / 1e9 / PEAK_GBS, 4),
        "metric_bytes_per_layer": mb,
        "roofline": {"bound": "hbm", "kernel": ("main_kernel (INT4 main region + INT8 protected region "
                                                "+ this step's append)"),
                     "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic,
                     "avg_launch_us": round(main_ms * 1e3, 2), "alg_bytes_per_launch": main_bytes},
        "cpu_baseline": cpu,
    }
    rec.update(extra)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
