"""Benchmark of the MI355X FlashAttention forward pass.

One step = one fa_fwd call on the large bf16 causal batch (B=8, Hq=32, Hkv=8, Tq=Tk=8192,
d=128, scale 1/sqrt(128), inputs N(0,1) already resident in HBM).  `value` is attention
TFLOP/s counted over causal-visible pairs (4 d flops per visible (query, key) pair: 2d for
the scores, 2d for P V; exp, max and sum not counted) over the wall time of the timed steps.

The same JSON line also reports
  * roofline: the kernel's average duration from HIP events on its stream, against the
    MI355X dense bf16 MFMA peak; hbm_from_counters: the HBM bytes per launch that the committed
    rocprofv3 counter summary measured (FETCH_SIZE, WRITE_SIZE, scaled by a plain copy), over
    this run's launch time, when that summary was taken on the current kernel source;
  * prefill_ms: 28 back-to-back calls (one per layer, fresh seeded inputs per layer) at
    16 query / 8 KV heads, d 128: 511 tokens fp32, 2044 tokens fp32 and bf16; and
    prefill_ms_splitkv: the same through split-KV at the default split size (results within
    tolerance of the plain call, still invariant to query chunking at that split size);
  * single_head_128: the 1 x 128 x 64 fp32 causal call (launch-latency bound);
  * extra workloads: the 32/8-head d 64 sliding-window (512) prefill with sinks, chunked
    (1000, 1000, 1000, 1096) and whole, the non-causal run with a broadcast additive mask, and
    decode (one query row, split-KV and unsplit) at 8 x 32/8 heads x 8,192 keys bf16 and at
    9/3 heads d 64 fp32 with 1,024 and 4,096 keys; a packed varlen batch of 8 mixed-length
    prefills against one call per sequence; the softcap / ALiBi score variants at 32/8 heads,
    8,192 tokens;
  * cpu_baseline: the fp64 oracle timed on the host cores over a bounded row sample of the
    headline workload;
  * cpu_oracle_prefill: the same oracle over one layer of each prefill shape, on one host thread
    and on all of them (context beside the pages' CPU prefill figures, not a target);
  * sclk_during_headline: the shader clock rocm-smi reports while the headline kernel runs;
  * inputs_sha256_16 (and mask_sha256_16 of the mask run): digests of the seeded host inputs,
    the same on every run and box.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk/CU x 2.4 GHz, dense
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd TFLOP/s (causal-visible) + % MFMA peak; prefill ms @511/2044"


KERNEL_SRC = os.path.join(ROOT, "flashattention_forward_flash_amd", "csrc", "fa_fwd.hip")
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "fa_fwd_all_workloads.md")
TRACE_SUMMARY = os.path.join(ROOT, "profiles", "fa_fwd_bf16_d128_causal_B8_H32_T8192.md")


def kernel_source_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counter_traffic():
    """{workload: figures} from the committed rocprofv3 counter summary (profiles/
    fa_fwd_all_workloads.md: HBM bytes per step from FETCH_SIZE + WRITE_SIZE scaled by a plain
    copy, the kernels' time per step), or {} when it is missing or was taken on a different
    kernel source."""
    try:
        text = open(PROFILE_SUMMARY).read()
    except OSError:
        return {}
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return {}
    data = json.loads(m.group(1))
    return data["workloads"] if data.get("kernel_source_sha256_16") == kernel_source_hash() else {}


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size: the reference that scales the memory
    counters (FETCH_SIZE, WRITE_SIZE) into bytes."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": reps}), flush=True)


def visible_pairs(Tq, Tk, q_offset=0, causal=True, window=0):
    """sum over rows of |V_i| from the interval form of the visible set."""
    p = np.arange(Tq, dtype=np.int64) + q_offset
    hi = np.minimum(Tk, p + 1) if causal else np.full(Tq, Tk, np.int64)
    lo = np.maximum(0, p - window + 1) if window > 0 else np.zeros(Tq, np.int64)
    return int(np.maximum(0, hi - lo).sum())


def _dev(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _digest(a):
    """sha256[:16] of a host array's bytes (the seeded inputs are the same on every run)."""
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()[:16]


def _inputs(tag, B, Hq, Hkv, Tq, Tk, d, dtype, layout="bhsd", digests=None):
    """Seeded N(0, 1) q, k, v on the GPU; `digests` (a dict) receives their sha256[:16]."""
    import synth
    if layout == "bshd":
        shapes = ((B, Tq, Hq, d), (B, Tk, Hkv, d), (B, Tk, Hkv, d))
    else:
        shapes = ((B, Hq, Tq, d), (B, Hkv, Tk, d), (B, Hkv, Tk, d))
    arrs = [synth.normal(synth.seed_of(tag, n), sh, dtype) for n, sh in zip("qkv", shapes)]
    if digests is not None:
        digests.update({n: _digest(a) for n, a in zip("qkv", arrs)})
    if layout == "bshd":
        return tuple(_dev(a).transpose(1, 2) for a in arrs)
    return tuple(_dev(a) for a in arrs)


def _timed(fn, steps, warmup):
    """Returns (wall ms per step, mean event ms per call) for `steps` calls after `warmup`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in evs:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ev = float(np.mean([s.elapsed_time(e) for s, e in evs]))
    return wall, ev


def bench_headline(steps, warmup):
    import torch
    import flashattention_forward_flash_amd as fa
    B, Hq, Hkv, T, d = 8, 32, 8, 8192, 128
    digests = {}
    q, k, v = _inputs("c5", B, Hq, Hkv, T, T, d, "bf16", digests=digests)
    scale = float(np.float32(1 / math.sqrt(d)))
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    print(f"[bench] headline B={B} Hq={Hq} Hkv={Hkv} T={T} d={d} bf16 causal", file=sys.stderr, flush=True)
    wall, ev = _timed(lambda: fa.forward(q, k, v, scale=scale, causal=True, out=out, lse=lse), steps, warmup)
    flops = 4.0 * d * B * Hq * visible_pairs(T, T)
    algo_bytes = 2 * (q.numel() + k.numel() + v.numel() + out.numel()) + 4 * lse.numel()
    return dict(B=B, Hq=Hq, Hkv=Hkv, T=T, d=d, flops=flops, bytes=algo_bytes, wall_ms=wall, event_ms=ev,
                q=q, k=k, v=v, scale=scale, digests=digests)


def bench_mask_run(h, steps, warmup):
    """Same inputs, non-causal, fp32 additive mask [8192, 8192] broadcast over b and h (stride 0):
    10 % of entries -inf, 16 fully masked rows."""
    import torch
    import synth
    import flashattention_forward_flash_amd as fa
    T = h["T"]
    m = synth.neg_inf_mask(synth.seed_of("c5", "mask"), (T, T), 0.1)
    for r in (0, 1, 63, 64, 65, 127, 128, 1023, 1024, 2047, 4095, 4096, 6000, 8127, 8128, 8191):
        m[r] = -np.inf
    digest = _digest(m)
    mask = torch.from_numpy(m).cuda()
    out = torch.empty_like(h["q"])
    print("[bench] headline inputs, non-causal, broadcast additive mask", file=sys.stderr, flush=True)
    wall, ev = _timed(lambda: fa.forward(h["q"], h["k"], h["v"], scale=h["scale"], causal=False, mask=mask,
                                         out=out), steps, warmup)
    flops = 4.0 * h["d"] * h["B"] * h["Hq"] * T * T
    return dict(ms=ev, tflops=flops / (ev * 1e-3) / 1e12, mask_sha256_16=digest)


def bench_prefill(T, dtype, layers=28, reps=5, split=False):
    """28 calls (one per layer) at 16/8 heads, d 128, in the concatenated-heads layout; with
    `split`, through split-KV at the default split size (one workspace for all layers)."""
    import torch
    import flashattention_forward_flash_amd as fa
    Hq, Hkv, d = 16, 8, 128
    per_layer = [_inputs(f"prefill{T}/{dtype}/{layer}", 1, Hq, Hkv, T, T, d, dtype, layout="bshd")
                 for layer in range(layers)]
    outs = [torch.empty((1, T, Hq, d), dtype=per_layer[0][0].dtype, device="cuda").transpose(1, 2)
            for _ in range(layers)]
    scale = float(np.float32(1 / math.sqrt(d)))

    sk = fa.fa_splitkv_default_keys(1, Hq, Hkv, T, T, 0, True, 0, fa.FA_BF16 if dtype == "bf16" else fa.FA_F32)
    ws = torch.empty(fa.fa_splitkv_workspace_bytes(1, Hq, T, T, d, sk), dtype=torch.uint8, device="cuda")

    def run_all():
        for (q, k, v), o in zip(per_layer, outs):
            if split:
                fa.forward_splitkv(q, k, v, split_keys=sk, workspace=ws, scale=scale, causal=True, out=o,
                                   return_lse=False)
            else:
                fa.forward(q, k, v, scale=scale, causal=True, out=o, return_lse=False)

    print(f"[bench] prefill T={T} {dtype} x{layers} layers{' split-KV' if split else ''}", file=sys.stderr, flush=True)
    wall, ev = _timed(run_all, reps, 2)
    flops = 4.0 * d * Hq * visible_pairs(T, T) * layers
    peak = PEAK_F32_TFLOPS if dtype == "f32" else PEAK_BF16_TFLOPS
    res = dict(ms=round(ev, 4), per_call_ms=round(ev / layers, 5), tflops=round(flops / (ev * 1e-3) / 1e12, 2),
               frac_peak=round(flops / (ev * 1e-3) / 1e12 / peak, 4))
    if split:
        res["split_keys"] = int(sk)
    return res


def bench_single_head(steps=20, warmup=5):
    """The single-head case: B 1, H 1, Tq = Tk = 128, d 64, fp32, causal, with LSE (launch
    latency bound: the call's duration, and the wall time per call back to back)."""
    import torch
    import flashattention_forward_flash_amd as fa
    q, k, v = _inputs("c1", 1, 1, 1, 128, 128, 64, "f32")
    out = torch.empty_like(q)
    lse = torch.empty((1, 1, 128), dtype=torch.float32, device="cuda")
    scale = float(np.float32(1 / math.sqrt(64)))
    print("[bench] single head 1x128 d64 f32", file=sys.stderr, flush=True)
    wall, ev = _timed(lambda: fa.forward(q, k, v, scale=scale, causal=True, out=out, lse=lse), steps, warmup)
    return dict(event_us=round(ev * 1e3, 2), wall_us_per_call=round(wall * 1e3, 2),
                tflops=round(4.0 * 64 * visible_pairs(128, 128) / (ev * 1e-3) / 1e12, 4))


def bench_window_chunks(steps=10, warmup=3):
    """32/8 heads, d 64, Tk 4096, window 512, sinks, causal, fp32: one call and 4 chunks."""
    import torch
    import synth
    import flashattention_forward_flash_amd as fa
    Hq, Hkv, T, d = 32, 8, 4096, 64
    q, k, v = _inputs("c4", 1, Hq, Hkv, T, T, d, "f32")
    z = torch.from_numpy(synth.normal_f32(synth.seed_of("c4", "z"), (Hq,))).cuda()
    scale = float(np.float32(1 / math.sqrt(d)))
    out = torch.empty_like(q)
    lse = torch.empty((1, Hq, T), dtype=torch.float32, device="cuda")
    print("[bench] sliding window with sinks, whole and chunked", file=sys.stderr, flush=True)
    _, ev_full = _timed(lambda: fa.forward(q, k, v, scale=scale, causal=True, window=512, sinks=z, out=out, lse=lse),
                        steps, warmup)
    chunks = [(0, 1000), (1000, 1000), (2000, 1000), (3000, 1096)]

    def run_chunks():
        for s, n in chunks:
            fa.forward(q[:, :, s:s + n], k, v, scale=scale, q_offset=s, causal=True, window=512, sinks=z,
                       out=out[:, :, s:s + n], lse=lse[:, :, s:s + n])

    _, ev_chunks = _timed(run_chunks, steps, warmup)
    flops = 4.0 * d * Hq * visible_pairs(T, T, 0, True, 512)
    return dict(ms=round(ev_full, 4), chunked_ms=round(ev_chunks, 4),
                tflops=round(flops / (ev_full * 1e-3) / 1e12, 2))


def _timed_batch(fn, steps, warmup):
    """Mean ms per call of `steps` back-to-back calls between one pair of events (for calls
    short enough that an event pair per call would time the launch path rather than the work)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def bench_decode(steps=50, warmup=10):
    """Decode (one query row per sequence at q_offset = Tk - 1) through split-KV (default split)
    and through the unsplit call: the 32/8-head d 128 bf16 model at 8,192 cached keys, B = 8,
    and the 9/3-head d 64 fp32 shape at 1,024 and 4,096 keys.  HBM-bound: rate = algorithmic
    bytes (K, V, Q, O, LSE once) / time per call (both kernels for split-KV), calls back to
    back between one pair of events."""
    import torch
    import flashattention_forward_flash_amd as fa
    res = {}
    for name, B, Hq, Hkv, Tk, d, dtype in (("8x32x8192_bf16_d128", 8, 32, 8, 8192, 128, "bf16"),
                                            ("1x9x1024_f32_d64", 1, 9, 3, 1024, 64, "f32"),
                                            ("1x9x4096_f32_d64", 1, 9, 3, 4096, 64, "f32")):
        q, k, v = _inputs(f"decode/{name}", B, Hq, Hkv, 1, Tk, d, dtype)
        scale = float(np.float32(1 / math.sqrt(d)))
        out = torch.empty_like(q)
        lse = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
        split = fa.fa_splitkv_default_keys(B, Hq, Hkv, 1, Tk, Tk - 1, True, 0,
                                           fa.FA_BF16 if dtype == "bf16" else fa.FA_F32)
        ws = torch.empty(fa.fa_splitkv_workspace_bytes(B, Hq, 1, Tk, d, split), dtype=torch.uint8, device="cuda")
        print(f"[bench] decode {name} split_keys={split}", file=sys.stderr, flush=True)
        kw = dict(scale=scale, q_offset=Tk - 1, causal=True, out=out, lse=lse)
        ev_split = _timed_batch(lambda: fa.forward_splitkv(q, k, v, split_keys=split, workspace=ws, **kw), steps, warmup)
        ev_plain = _timed_batch(lambda: fa.forward(q, k, v, **kw), steps, warmup)
        es = q.element_size()
        nbytes = es * (q.numel() + k.numel() + v.numel() + out.numel()) + 4 * lse.numel()
        gbs = nbytes / (ev_split * 1e-3) / 1e9
        res[name] = dict(split_keys=split, splitkv_us=round(ev_split * 1e3, 2), unsplit_us=round(ev_plain * 1e3, 2),
                         algorithmic_bytes=nbytes, splitkv_GBs=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4))
        if B == 8:  # the same keys in pages of 256 keys, blocks in shuffled order, split-KV
            bs = 256
            nbs = Tk // bs
            perm = torch.from_numpy(np.random.default_rng(1).permutation(B * nbs).astype(np.int32)).cuda()
            table = perm.view(B, nbs)
            kp = torch.empty((B * nbs, Hkv, bs, d), dtype=k.dtype, device="cuda")
            vp = torch.empty_like(kp)
            kp[table.long()] = k.view(B, Hkv, nbs, bs, d).transpose(1, 2)
            vp[table.long()] = v.view(B, Hkv, nbs, bs, d).transpose(1, 2)
            ev_paged = _timed_batch(lambda: fa.forward_paged(q, kp, vp, table, split_keys=split, workspace=ws, **kw),
                                    steps, warmup)
            res[name]["paged256_splitkv_us"] = round(ev_paged * 1e3, 2)
            del kp, vp
    return res


def bench_varlen(steps=10, warmup=3):
    """Packed batch of 8 causal self-attention prefills of mixed lengths (16/8 heads, d 128,
    bf16) in one call, against one call per sequence."""
    import torch
    import synth
    import flashattention_forward_flash_amd as fa
    lens = [2044, 511, 1024, 100, 2044, 300, 1500, 777]
    Hq, Hkv, d = 16, 8, 128
    tot = sum(lens)
    q = _dev(synth.normal(synth.seed_of("varlen", "q"), (tot, Hq, d), "bf16"))
    k = _dev(synth.normal(synth.seed_of("varlen", "k"), (tot, Hkv, d), "bf16"))
    v = _dev(synth.normal(synth.seed_of("varlen", "v"), (tot, Hkv, d), "bf16"))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((Hq, tot), dtype=torch.float32, device="cuda")
    scale = float(np.float32(1 / math.sqrt(d)))
    print("[bench] varlen packed batch", file=sys.stderr, flush=True)
    packed = _timed_batch(lambda: fa.forward_varlen(q, k, v, cu, cu, max(lens), max(lens), scale=scale, causal=True,
                                                   out=out, lse=lse), steps, warmup)
    views = []
    s0 = 0
    for n in lens:
        views.append(tuple(t[s0:s0 + n].transpose(0, 1)[None] for t in (q, k, v, out)))
        s0 += n

    def per_seq():
        for qs, ks, vs, os_ in views:
            fa.forward(qs, ks, vs, scale=scale, causal=True, out=os_, return_lse=False)

    separate = _timed_batch(per_seq, steps, warmup)
    flops = 4.0 * d * Hq * sum(visible_pairs(n, n) for n in lens)
    return dict(lengths=lens, packed_ms=round(packed, 4), per_sequence_calls_ms=round(separate, 4),
                packed_tflops=round(flops / (packed * 1e-3) / 1e12, 2))


def bench_variants(steps=10, warmup=3):
    """Score variants at B=1, 32/8 heads, T=8192, d 128, bf16, causal: the plain call, softcap
    30, ALiBi (slopes 2^(-8(h+1)/32)) and both; TFLOP/s over causal-visible pairs."""
    import torch
    import flashattention_forward_flash_amd as fa
    B, Hq, Hkv, T, d = 1, 32, 8, 8192, 128
    q, k, v = _inputs("variants", B, Hq, Hkv, T, T, d, "bf16")
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    scale = float(np.float32(1 / math.sqrt(d)))
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)], dtype=torch.float32, device="cuda")
    flops = 4.0 * d * B * Hq * visible_pairs(T, T)
    res = {}
    for name, kw in (("plain", {}), ("softcap30", dict(softcap=30.0)), ("alibi", dict(alibi_slopes=slopes)),
                     ("softcap30_alibi", dict(softcap=30.0, alibi_slopes=slopes))):
        print(f"[bench] variants {name}", file=sys.stderr, flush=True)
        ms = _timed_batch(lambda: fa.forward(q, k, v, scale=scale, causal=True, out=out, lse=lse, **kw), steps, warmup)
        res[name] = dict(ms=round(ms, 4), tflops=round(flops / (ms * 1e-3) / 1e12, 2))
    return res


def sample_sclk(h, seconds=2.0):
    """The shader clock while the headline kernel runs back to back: `rocm-smi --showclocks`
    polled from a host thread (MHz values seen; None where rocm-smi is unavailable, and under
    a profiler whose preloaded library would start the GPU in every child process)."""
    import subprocess
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return None
    import threading
    import torch
    import flashattention_forward_flash_amd as fa
    seen, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                                     timeout=10).stdout
                m = re.search(r'"sclk clock speed:": "\((\d+)Mhz\)"', out)
                if m:
                    seen.append(int(m.group(1)))
            except (OSError, subprocess.SubprocessError):
                return
            stop.wait(0.3)

    out = torch.empty_like(h["q"])
    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fa.forward(h["q"], h["k"], h["v"], scale=h["scale"], causal=True, out=out, return_lse=False)
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    if not seen:
        return None
    return dict(mhz_samples=seen, mhz_median=float(np.median(seen)))


def cpu_baseline(h, target_s=15.0):
    """The fp64 oracle on the host cores over a seeded row sample of the headline workload,
    scaled to the metric's unit (TFLOP/s over the sampled rows' visible pairs)."""
    import oracle
    B, Hq, T, d = h["B"], h["Hq"], h["T"], h["d"]
    q = h["q"].view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    k = h["k"].view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    v = h["v"].view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    cores = len(os.sched_getaffinity(0))
    oracle.attention(q[:1, :1, :1], k[:1, :1, :1], v[:1, :1, :1], scale=h["scale"], threads=cores)
    cores = oracle.threads()
    rng = np.random.default_rng(5)
    n = 256
    while True:
        rows = np.stack([rng.integers(0, B, n), rng.integers(0, Hq, n), rng.integers(0, T, n)], 1)
        t0 = time.perf_counter()
        oracle.attention(q, k, v, scale=h["scale"], causal=True, rows=rows, threads=cores)
        dt = time.perf_counter() - t0
        if dt >= target_s / 4 or n >= (1 << 20):
            break
        n = int(n * min(16.0, max(2.0, target_s / max(dt, 1e-3))))
    pairs = int(np.sum(rows[:, 2] + 1))
    flops = 4.0 * d * pairs
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=cores, kind="oracle",
                sample=f"{n} seeded (b, h, i) rows of the headline workload ({pairs} visible pairs, fp64), "
                       f"{dt:.1f} s wall",
                seconds=round(dt, 2))


def cpu_oracle_prefill():
    """The fp64 oracle on the host, one layer of each prefill shape (16/8 heads, d 128, causal,
    fp32 inputs; and the 1 x 128 x 64 single head), on one thread and on all host threads, to sit
    beside the pages' CPU prefill figures.  28-layer figures are these times x 28."""
    import oracle
    import synth
    cores = len(os.sched_getaffinity(0))
    res = {"cores": cores}
    for name, (Hq, Hkv, T, d, one_thread) in (("1x128_d64", (1, 1, 128, 64, True)),
                                                ("511_f32_layer", (16, 8, 511, 128, True)),
                                                ("2044_f32_layer", (16, 8, 2044, 128, False))):
        q = synth.normal(synth.seed_of("cpu-prefill", name, "q"), (1, Hq, T, d), "f32")
        k = synth.normal(synth.seed_of("cpu-prefill", name, "k"), (1, Hkv, T, d), "f32")
        v = synth.normal(synth.seed_of("cpu-prefill", name, "v"), (1, Hkv, T, d), "f32")
        scale = float(np.float32(1 / math.sqrt(d)))
        row = {}
        for label, thr in (("threads1_ms", 1), ("threads_all_ms", cores)):
            if thr == 1 and not one_thread:
                continue
            t0 = time.perf_counter()
            oracle.attention(q, k, v, scale=scale, causal=True, threads=thr)
            row[label] = round((time.perf_counter() - t0) * 1e3, 2)
        if Hq == 16:
            row.update({key.replace("_ms", "_x28_ms"): round(ms * 28, 1) for key, ms in list(row.items())})
        res[name] = row
    return res


# ---- single workloads for the profiler (``--leg``): the same seeded inputs and calls as the legs
# above, run `warmup + steps` times with nothing else on the GPU.  Each returns a callable that
# performs one step and the step's algorithmic bytes and flops.
def _leg_headline():
    import torch
    import flashattention_forward_flash_amd as fa
    B, Hq, Hkv, T, d = 8, 32, 8, 8192, 128
    q, k, v = _inputs("c5", B, Hq, Hkv, T, T, d, "bf16")
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    scale = float(np.float32(1 / math.sqrt(d)))
    nbytes = 2 * (q.numel() + k.numel() + v.numel() + out.numel()) + 4 * lse.numel()
    return (lambda: fa.forward(q, k, v, scale=scale, causal=True, out=out, lse=lse)), nbytes, \
        4.0 * d * B * Hq * visible_pairs(T, T)


def _leg_mask():
    import torch
    import synth
    import flashattention_forward_flash_amd as fa
    B, Hq, Hkv, T, d = 8, 32, 8, 8192, 128
    q, k, v = _inputs("c5", B, Hq, Hkv, T, T, d, "bf16")
    m = synth.neg_inf_mask(synth.seed_of("c5", "mask"), (T, T), 0.1)
    for r in (0, 1, 63, 64, 65, 127, 128, 1023, 1024, 2047, 4095, 4096, 6000, 8127, 8128, 8191):
        m[r] = -np.inf
    mask = torch.from_numpy(m).cuda()
    out = torch.empty_like(q)
    scale = float(np.float32(1 / math.sqrt(d)))
    nbytes = 2 * (q.numel() + k.numel() + v.numel() + out.numel()) + 4 * mask.numel()
    return (lambda: fa.forward(q, k, v, scale=scale, causal=False, mask=mask, out=out, return_lse=False)), \
        nbytes, 4.0 * d * B * Hq * T * T


def _leg_prefill(T, dtype):
    import torch
    import flashattention_forward_flash_amd as fa
    Hq, Hkv, d, layers = 16, 8, 128, 28
    per_layer = [_inputs(f"prefill{T}/{dtype}/{layer}", 1, Hq, Hkv, T, T, d, dtype, layout="bshd")
                 for layer in range(layers)]
    outs = [torch.empty((1, T, Hq, d), dtype=per_layer[0][0].dtype, device="cuda").transpose(1, 2)
            for _ in range(layers)]
    scale = float(np.float32(1 / math.sqrt(d)))
    es = 4 if dtype == "f32" else 2

    def run_all():
        for (q, k, v), o in zip(per_layer, outs):
            fa.forward(q, k, v, scale=scale, causal=True, out=o, return_lse=False)

    nbytes = layers * es * (2 * T * Hq * d + 2 * T * Hkv * d)
    return run_all, nbytes, 4.0 * d * Hq * visible_pairs(T, T) * layers


def _leg_single_head():
    import torch
    import flashattention_forward_flash_amd as fa
    q, k, v = _inputs("c1", 1, 1, 1, 128, 128, 64, "f32")
    out = torch.empty_like(q)
    lse = torch.empty((1, 1, 128), dtype=torch.float32, device="cuda")
    scale = float(np.float32(1 / math.sqrt(64)))
    return (lambda: fa.forward(q, k, v, scale=scale, causal=True, out=out, lse=lse)), \
        4 * (4 * 128 * 64) + 4 * 128, 4.0 * 64 * visible_pairs(128, 128)


def _leg_window(chunked):
    import torch
    import synth
    import flashattention_forward_flash_amd as fa
    Hq, Hkv, T, d = 32, 8, 4096, 64
    q, k, v = _inputs("c4", 1, Hq, Hkv, T, T, d, "f32")
    z = torch.from_numpy(synth.normal_f32(synth.seed_of("c4", "z"), (Hq,))).cuda()
    scale = float(np.float32(1 / math.sqrt(d)))
    out = torch.empty_like(q)
    lse = torch.empty((1, Hq, T), dtype=torch.float32, device="cuda")
    chunks = [(0, 1000), (1000, 1000), (2000, 1000), (3000, 1096)] if chunked else [(0, T)]

    def run():
        for s0, n in chunks:
            fa.forward(q[:, :, s0:s0 + n], k, v, scale=scale, q_offset=s0, causal=True, window=512, sinks=z,
                       out=out[:, :, s0:s0 + n], lse=lse[:, :, s0:s0 + n])

    nbytes = 4 * (q.numel() + k.numel() + v.numel() + out.numel() + lse.numel() + Hq)
    return run, nbytes, 4.0 * d * Hq * visible_pairs(T, T, 0, True, 512)


def _leg_decode(B, Hq, Hkv, Tk, d, dtype):
    import torch
    import flashattention_forward_flash_amd as fa
    name = {8: "8x32x8192_bf16_d128"}.get(B, f"1x9x{Tk}_f32_d64")
    q, k, v = _inputs(f"decode/{name}", B, Hq, Hkv, 1, Tk, d, dtype)
    scale = float(np.float32(1 / math.sqrt(d)))
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
    split = fa.fa_splitkv_default_keys(B, Hq, Hkv, 1, Tk, Tk - 1, True, 0, fa.FA_BF16 if dtype == "bf16" else fa.FA_F32)
    ws = torch.empty(fa.fa_splitkv_workspace_bytes(B, Hq, 1, Tk, d, split), dtype=torch.uint8, device="cuda")
    es = q.element_size()
    nbytes = es * (q.numel() + k.numel() + v.numel() + out.numel()) + 4 * lse.numel()
    return (lambda: fa.forward_splitkv(q, k, v, split_keys=split, workspace=ws, scale=scale, q_offset=Tk - 1,
                                       causal=True, out=out, lse=lse)), nbytes, 4.0 * d * B * Hq * Tk


def _leg_noncausal():
    """The mask run's inputs without the mask (non-causal): the HBM bytes the mask adds are the
    difference between the two legs' counters."""
    import torch
    import flashattention_forward_flash_amd as fa
    B, Hq, Hkv, T, d = 8, 32, 8, 8192, 128
    q, k, v = _inputs("c5", B, Hq, Hkv, T, T, d, "bf16")
    out = torch.empty_like(q)
    scale = float(np.float32(1 / math.sqrt(d)))
    nbytes = 2 * (q.numel() + k.numel() + v.numel() + out.numel())
    return (lambda: fa.forward(q, k, v, scale=scale, causal=False, out=out, return_lse=False)), \
        nbytes, 4.0 * d * B * Hq * T * T


LEGS = {
    "headline": _leg_headline,
    "mask": _leg_mask,
    "noncausal": _leg_noncausal,
    "prefill511_f32": lambda: _leg_prefill(511, "f32"),
    "prefill2044_f32": lambda: _leg_prefill(2044, "f32"),
    "prefill2044_bf16": lambda: _leg_prefill(2044, "bf16"),
    "single_head": _leg_single_head,
    "window_sinks": lambda: _leg_window(False),
    "window_sinks_chunked": lambda: _leg_window(True),
    "decode_bf16": lambda: _leg_decode(8, 32, 8, 8192, 128, "bf16"),
    "decode_f32_1024": lambda: _leg_decode(1, 9, 3, 1024, 64, "f32"),
    "decode_f32_4096": lambda: _leg_decode(1, 9, 3, 4096, 64, "f32"),
}


def run_leg(name, steps, warmup):
    """One workload, `warmup + steps` steps back to back (for rocprofv3)."""
    import torch
    import flashattention_forward_flash_amd as fa
    fa.load_library()
    fn, nbytes, flops = LEGS[name]()
    for _ in range(warmup + steps):
        fn()
    torch.cuda.synchronize()
    print(json.dumps({"leg": name, "steps": steps, "warmup": warmup, "algorithmic_bytes": nbytes,
                      "flops": flops}), flush=True)


SQ_SUMMARY = os.path.join(ROOT, "profiles", "fa_fwd_bf16_d128_causal_B8_H32_T8192_sq.md")
SQ_COUNTERS = (("SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
                "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM"),
               ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY",
                "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY"),
               ("SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_VALU_TRANS_F32", "SQ_BUSY_CU_CYCLES"))


def profile_commands(leg, steps=10, warmup=2):
    """The rocprofv3 commands whose CSV output write_profile_summaries() reads (DIR: any output directory)."""
    b = f"python3 <repo>/bench.py --leg {leg} --steps {steps} --warmup {warmup}"
    return [f"rocprofv3 --kernel-trace --stats --output-format csv -d DIR/{leg}_trace -o run -- {b}",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/{leg}_FETCH_SIZE -o run -- {b}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/{leg}_WRITE_SIZE -o run -- {b}"]


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _ours(name):
    """A kernel of the library (the forward kernels and the split-KV merge)."""
    return any(k in name for k in ("fa_fwd_kernel", "fa_fwd_so_kernel", "fa_merge_kernel"))


def _short(name):
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0]


def _write_trace_summary(d, leg, src):
    """The headline's kernel trace: every call's duration, the average after the warm-up steps
    (what bench.py's per-launch timing compares to) and rocprofv3's own --stats line."""
    meta = json.loads(open(os.path.join(d, f"{leg}_trace", "leg.json")).read().strip().splitlines()[-1])
    trace = sorted((r for r in _csv_rows(os.path.join(d, f"{leg}_trace", "run_kernel_trace.csv"))
                    if _ours(r["Kernel_Name"])), key=lambda r: int(r["Start_Timestamp"]))
    us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace]
    timed = us[meta["warmup"]:]
    stats = [r for r in _csv_rows(os.path.join(d, f"{leg}_trace", "run_kernel_stats.csv"))
             if _ours(r["Name"])]
    flops = meta["flops"]
    lines = ["# fa_fwd kernel, bf16, d = 128, causal, B = 8, Hq = 32, Hkv = 8, Tq = Tk = 8192", "",
             "Kernel trace of the headline workload (one call = one step of `bench.py`).", "",
             "Command (repository root on one MI355X, `cd /tmp && export TMPDIR=/tmp` first; DIR is",
             "any output directory):", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d DIR/{leg}_trace -o run -- python3 "
             f"<repo>/bench.py --leg {leg} --steps {meta['steps']} --warmup {meta['warmup']}",
             "python3 bench.py --profile-summary DIR   # writes this file", "```", "",
             f"kernel source sha256[:16]: {src}", "",
             "| kernel | calls | average us (all) | average us (after the warm-up call) | min us | max us |",
             "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(np.mean(timed)):.1f} | {float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    lines += ["", "Per call (us): " + ", ".join(f"{u:.1f}" for u in us), "",
              f"The first {meta['warmup']} call(s) are the warm-up.  Causal-visible work per call: {flops:.4e} flop; "
              f"the average after the warm-up, {np.mean(timed):.1f} us, is {flops / (np.mean(timed) * 1e-6) / 1e12:.0f} "
              f"TFLOP/s under the profiler ({flops / (np.mean(timed) * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.3f} of the "
              f"{PEAK_BF16_TFLOPS} TFLOP/s dense bf16 peak).", ""]
    with open(TRACE_SUMMARY, "w") as f:
        f.write("\n".join(lines))


def write_profile_summaries(d):
    """Turns rocprofv3 CSV output under `d` into the profiles/ summaries: per workload, the kernels'
    average time per step after the warm-up steps (kernel trace), and the HBM bytes per step from
    FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter reads for a plain 1 GiB copy;
    for the headline workload also the SQ counters.  Expects DIR/<leg>_trace/, DIR/<leg>_FETCH_SIZE/,
    DIR/<leg>_WRITE_SIZE/ (each with leg.json, the leg's own output line), DIR/copy_FETCH_SIZE/,
    DIR/copy_WRITE_SIZE/ and DIR/headline_sq<n>/."""
    def counter_kib(sub):
        rows = _csv_rows(os.path.join(d, sub, "run_counter_collection.csv"))
        per = {}  # (dispatch, kernel) -> counter -> value summed over the rows (instances) of the dispatch
        for r in rows:
            c = per.setdefault((int(r["Dispatch_Id"]), r["Kernel_Name"]), {})
            c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        return per

    scale = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        vals = [v[c] for (_, name), v in counter_kib(f"copy_{c}").items() if "copy" in name.lower()]
        scale[c] = (1 << 20) / float(np.mean(vals))  # KiB the counter reads for 1 GiB moved
    legs = sorted({n[:-len("_trace")] for n in os.listdir(d) if n.endswith("_trace")})
    src = kernel_source_hash()
    lines = ["# HBM traffic and kernel time of every bench workload",
             "",
             "Per workload (one step = what `bench.py` times for it: one call, or the 28 calls of a",
             "28-layer prefill, or the 4 calls of the chunked window run; decode runs split-KV: the",
             "streaming kernel and the merge): the kernels' time per step averaged over the steps after",
             "the warm-up (kernel trace), and the HBM bytes per step from the FETCH_SIZE and WRITE_SIZE",
             "counters (KiB per dispatch, each pass a run of its own), scaled by what the same counter",
             "reads for a plain 1 GiB device copy: FETCH_SIZE x %.4f, WRITE_SIZE x %.4f." % (
                 scale["FETCH_SIZE"], scale["WRITE_SIZE"]),
             "Algorithmic bytes read Q, K, V (and the mask, sinks) once and write O (and LSE) once.",
             "",
             "Commands (repository root on one MI355X, `cd /tmp && export TMPDIR=/tmp` first; DIR is",
             "any output directory; the calibration copy is `python3 <repo>/bench.py --copy-calibration`",
             "under the same two counter passes, into DIR/copy_FETCH_SIZE and DIR/copy_WRITE_SIZE); for",
             "each workload LEG below:",
             "",
             "```"] + profile_commands("LEG") + [
             "python3 bench.py --profile-summary DIR   # writes this file",
             "```",
             "",
             f"kernel source sha256[:16]: {src}",
             "",
             "| workload | kernels | us per step | TFLOP/s | algorithmic bytes | counter bytes (read + write) | read / algorithmic read | GB/s (counters) |",
             "|---|---|---|---|---|---|---|---|"]
    machine = {}
    for leg in legs:
        meta = json.loads(open(os.path.join(d, f"{leg}_trace", "leg.json")).read().strip().splitlines()[-1])
        steps, warmup = meta["steps"], meta["warmup"]
        # the library's kernels only (torch's setup copies of the inputs are not part of a step)
        trace = [r for r in _csv_rows(os.path.join(d, f"{leg}_trace", "run_kernel_trace.csv"))
                 if _ours(r["Kernel_Name"])]
        trace.sort(key=lambda r: int(r["Start_Timestamp"]))
        per_step = len(trace) // (steps + warmup)
        timed = trace[warmup * per_step:]
        us = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in timed) / 1e3 / steps
        names = sorted({_short(r["Kernel_Name"]) for r in trace})
        byts = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            per = {key: v for key, v in counter_kib(f"{leg}_{c}").items()
                   if _ours(key[1])}
            ids = sorted(per)[warmup * per_step:]
            byts[c] = sum(per[i][c] for i in ids) * 1024 * scale[c] / steps
        total = byts["FETCH_SIZE"] + byts["WRITE_SIZE"]
        algo = meta["algorithmic_bytes"]
        gbs = total / (us * 1e-6) / 1e9
        tfl = meta["flops"] / (us * 1e-6) / 1e12
        # the algorithmic reads: every input once (the bench's count minus the outputs)
        machine[leg] = dict(us_per_step=round(us, 2), counter_bytes_per_step=int(total),
                            read_bytes_per_step=int(byts["FETCH_SIZE"]), write_bytes_per_step=int(byts["WRITE_SIZE"]),
                            algorithmic_bytes=algo, GBs=round(gbs, 1), kernels=names,
                            dispatches_per_step=per_step)
        lines.append(f"| {leg} | {', '.join('`' + n + '`' for n in names)} ({per_step} per step) | {us:.1f} | "
                     f"{tfl:.2f} | {algo:,} | {int(total):,} | {byts['FETCH_SIZE'] / max(1, algo - byts['WRITE_SIZE']):.2f} "
                     f"| {gbs:.1f} |")
    lines += ["", "Machine-readable (bench.py reports these while the kernel source hash matches):", "",
              "```json", json.dumps({"kernel_source_sha256_16": src, "workloads": machine}, indent=1), "```", ""]
    with open(PROFILE_SUMMARY, "w") as f:
        f.write("\n".join(lines))
    _write_trace_summary(d, "headline", src)
    # SQ counters of the headline kernel
    sq = {}
    for n in range(len(SQ_COUNTERS)):
        sub = os.path.join(d, f"headline_sq{n}")
        if not os.path.isdir(sub):
            continue
        rows = _csv_rows(os.path.join(sub, "run_counter_collection.csv"))
        meta = json.loads(open(os.path.join(sub, "leg.json")).read().strip().splitlines()[-1])
        ids = set(sorted({int(r["Dispatch_Id"]) for r in rows})[meta["warmup"]:])
        per = {}
        for r in rows:
            if int(r["Dispatch_Id"]) in ids:
                key = (int(r["Dispatch_Id"]), r["Counter_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (_, name), val in per.items():
            sq.setdefault(name, []).append(val)
    if sq:
        mean = {k: float(np.mean(v)) for k, v in sq.items()}
        waves = mean.get("SQ_WAVES", 1.0)
        tiles = 8 * 32 * 8192 // 32 * (8192 // 64 + 1) / 2  # wave-tiles per call (32-row waves, causal)
        cmd = [f"rocprofv3 --pmc {' '.join(g)} --output-format csv -d DIR/headline_sq{n} -o run -- "
               f"python3 <repo>/bench.py --leg headline --steps 3 --warmup 1" for n, g in enumerate(SQ_COUNTERS)]
        out = ["# SQ counters of the headline kernel (bf16, d 128, causal, B 8, Hq 32, Hkv 8, T 8192)", "",
               "Per dispatch after the warm-up, summed over the device (one rocprofv3 pass per group of",
               "at most 8 SQ counters).  Commands (`cd /tmp && export TMPDIR=/tmp` first, DIR as in",
               "`fa_fwd_all_workloads.md`):", "", "```"] + cmd + ["```", "",
               f"kernel source sha256[:16]: {src}", "",
               "| counter | per dispatch | per wave | per wave-tile (32 rows x 64 keys) |", "|---|---|---|---|"]
        for k in sorted(mean):
            out.append(f"| {k} | {mean[k]:.4g} | {mean[k] / waves:.4g} | {mean[k] / tiles:.4g} |")
        busy = mean.get("SQ_BUSY_CYCLES")
        mfma = mean.get("SQ_VALU_MFMA_BUSY_CYCLES")
        if busy and mfma:
            # SQ_BUSY_CYCLES counts per shader engine (32 instances); SQ_VALU_MFMA_BUSY_CYCLES per SIMD
            out += ["", f"MFMA-busy fraction: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x SQ_BUSY_CYCLES / 32) = "
                        f"{mfma / (1024 * busy / 32):.3f}"]
        with open(SQ_SUMMARY, "w") as f:
            f.write("\n".join(out) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)  # the shader clock is still rising over the first calls
    ap.add_argument("--headline-only", action="store_true", help="skip the prefill / window / mask / CPU legs")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (reference for the memory counters)")
    ap.add_argument("--leg", choices=sorted(LEGS), help="only run this workload warmup + steps times (profiling)")
    ap.add_argument("--profile-summary", metavar="DIR",
                    help="write the profiles/ summaries from the rocprofv3 CSV output under DIR (no GPU)")
    args = ap.parse_args()
    if args.profile_summary:
        write_profile_summaries(args.profile_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only (the pass would shard over (b, head group) or query "
              "tiles with no exchange between GPUs; runs on several GPUs are not supported). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.leg:
        run_leg(args.leg, args.steps, args.warmup)
        return
    import torch
    import flashattention_forward_flash_amd as fa
    fa.load_library()
    torch.cuda.init()

    counters = counter_traffic()
    h = bench_headline(args.steps, args.warmup)
    tflops = h["flops"] / (h["wall_ms"] * 1e-3) / 1e12
    achieved = h["flops"] / (h["event_ms"] * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["wall_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal bf16 batch: B=8, Hq=32, Hkv=8, Tq=Tk=8192, d=128, scale 1/sqrt(128), "
                               "N(0,1) inputs, fp32 accumulate, bf16 O + fp32 LSE",
                   "global_batch": 8, "seq_len": 8192, "parallelism": "none (1 GPU)"},
        "frac_mfma_peak": round(achieved / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": counters.get("headline", {}).get("counter_bytes_per_step")},
        "kernel_source_sha256_16": kernel_source_hash(),
        "kernel_ms": round(h["event_ms"], 4),
        "algorithmic_bytes": h["bytes"],
        "inputs_sha256_16": h["digests"],
    }
    leg_ms = {"headline": h["event_ms"]}
    clk = sample_sclk(h)
    result["sclk_during_headline"] = clk
    if clk:  # the published peak assumes 2.4 GHz; the same fraction at the clock the box ran at
        result["frac_mfma_peak_at_measured_sclk"] = round(achieved / (PEAK_BF16_TFLOPS * clk["mhz_median"] / 2400.0), 4)
    if not args.headline_only:
        m = bench_mask_run(h, max(3, args.steps // 4), 2)
        result["mask_run"] = {"ms": round(m["ms"], 4), "tflops": round(m["tflops"], 2),
                              "frac_mfma_peak": round(m["tflops"] / PEAK_BF16_TFLOPS, 4),
                              "mask_sha256_16": m["mask_sha256_16"]}
        torch.cuda.empty_cache()
        result["prefill_ms"] = {
            "511_f32_28L": bench_prefill(511, "f32"),
            "2044_f32_28L": bench_prefill(2044, "f32"),
            "2044_bf16_28L": bench_prefill(2044, "bf16"),
        }
        result["prefill_ms_splitkv"] = {
            "511_f32_28L": bench_prefill(511, "f32", split=True),
            "2044_f32_28L": bench_prefill(2044, "f32", split=True),
            "2044_bf16_28L": bench_prefill(2044, "bf16", split=True),
        }
        result["single_head_128"] = bench_single_head()
        result["window_sinks_4096"] = bench_window_chunks()
        result["decode"] = bench_decode()
        result["varlen_batch"] = bench_varlen()
        result["score_variants"] = bench_variants()
    if not args.headline_only:
        pf, dec = result["prefill_ms"], result["decode"]
        leg_ms.update({"mask": result["mask_run"]["ms"], "prefill511_f32": pf["511_f32_28L"]["ms"],
                       "prefill2044_f32": pf["2044_f32_28L"]["ms"], "prefill2044_bf16": pf["2044_bf16_28L"]["ms"],
                       "single_head": result["single_head_128"]["event_us"] / 1e3,
                       "window_sinks": result["window_sinks_4096"]["ms"],
                       "window_sinks_chunked": result["window_sinks_4096"]["chunked_ms"],
                       "decode_bf16": dec["8x32x8192_bf16_d128"]["splitkv_us"] / 1e3,
                       "decode_f32_1024": dec["1x9x1024_f32_d64"]["splitkv_us"] / 1e3,
                       "decode_f32_4096": dec["1x9x4096_f32_d64"]["splitkv_us"] / 1e3})
    if counters:
        # HBM bytes per step from the committed rocprofv3 counters, over this run's time per step
        result["hbm_from_counters"] = {
            leg: {"bytes_per_step": c["counter_bytes_per_step"], "algorithmic_bytes": c["algorithmic_bytes"],
                  "GBs": round(c["counter_bytes_per_step"] / (leg_ms[leg] * 1e-3) / 1e9, 1),
                  "frac_hbm_peak": round(c["counter_bytes_per_step"] / (leg_ms[leg] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            for leg, c in counters.items() if leg in leg_ms}
    if not args.no_cpu and not args.headline_only:
        result["cpu_baseline"] = cpu_baseline(h)
        result["cpu_oracle_prefill"] = cpu_oracle_prefill()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
