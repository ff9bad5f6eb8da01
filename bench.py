#!/usr/bin/env python3
"""Benchmark of the lightning-indexer hot path on one MI355X.

One step = one decode step of the indexer for the headline workload: B = 32
requests, each with a 131072-token fp8 (E4M3FN) key cache plus fp32 per-token
scales, 64 heads x 128 dims, bf16 queries: the scan over every cached key and
the top-2048 selection per request (li_index_decode).  `value` is keys scored
per second over the K timed steps (inputs resident in HBM before timing).

The timed steps run without instrumentation; the per-kernel times come from
a repetition of the same steps with HIP events recorded by the library on its
own stream (each event adds a few microseconds to a step).  The same run also
reports, under "components": per-kernel times of that step, the prefill chunk
(T = 4096 against a causal 65536-token cache: TFLOP/s), the LatentIndex group
(G = 4 over a [16 x 131072, 256] bf16 latent: GB/s and MFMA share), the HS
decode (anchor top-8192 + three followers) against four native decodes, and
the ragged batched decode (B = 32, L ~ U{8K..32K}); and under "cpu_baseline"
the CPU oracle timed on a sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0    # dense fp8 MFMA
BF16_PEAK_TFLOPS = 2500.0   # dense bf16 / fp16 MFMA
FP8_KEY_BYTES = 128 + 4     # one fp8 key row + its fp32 scale
APPEND_COPIES = 6           # hidden-state / encoder copies the append rotates over
RAGGED_COPIES = 6           # key-cache copies the ragged decode rotates over (MALL is 256 MB)
METRIC = "decode indexer keys scored/s + HBM GB/s at 128K; prefill TFLOP/s; top-2048 µs"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Trace:
    """Per-kernel HIP events: the library launches kernel i of a call with
    events 2i and 2i+1 as the launch's start and stop events, which the
    runtime sets to that kernel's own start and end (no event marker sits
    between two kernels, so the kernels run back to back as they do
    untraced).  The events are created through the HIP runtime this process
    already runs (torch's), with hipEventDisableSystemFence, since they serve
    only for timing."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, torch, li, per_call, calls):
        self.torch, self.li, self.per = torch, li, per_call
        torch.cuda.synchronize()
        path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
        self.hip = hip = ctypes.CDLL(path)
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(per_call * calls):
            e = ctypes.c_void_p()
            if hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e.value)
        self.handles = (ctypes.c_void_p * len(self.ev))(*self.ev)

    def arm(self, i):
        addr = ctypes.addressof(self.handles) + i * self.per * ctypes.sizeof(ctypes.c_void_p)
        self.li.li_trace_events(ctypes.c_void_p(addr), self.per)

    def off(self):
        self.li.li_trace_events(None, 0)

    def spans(self, i):
        """Milliseconds of each kernel of call i (its start/stop event pair)."""
        e = self.ev[i * self.per:(i + 1) * self.per]
        out = []
        for j in range(0, self.per, 2):
            ms = ctypes.c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), e[j], e[j + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return out

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def traced(torch, li, fn, kernels, iters, check_count=True):
    """Per-kernel milliseconds (averages over `iters` calls of fn, which
    launches `kernels` kernels), from the start/stop events the library
    attaches to its kernel launches."""
    per_call = 2 * kernels
    tr = Trace(torch, li, per_call, iters)
    for i in range(iters):
        tr.arm(i)
        fn()
        if check_count and li.li_trace_count() != per_call:
            raise RuntimeError(f"expected {per_call} trace events, got {li.li_trace_count()}")
    torch.cuda.synchronize()
    tr.off()
    spans = [tr.spans(i) for i in range(iters)]
    tr.close()
    return [sum(s[j] for s in spans) / iters for j in range(kernels)]


def timed(torch, li, fn, kernels, iters, warmup, check_count=True):
    """Wall-clock milliseconds per call over `iters` calls (no events), then the
    per-kernel split from a traced repetition of the same calls."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(iters):
        fn()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / iters * 1e3
    return wall, traced(torch, li, fn, kernels, iters, check_count)


def dev(torch, a, dt=None):
    import numpy as np
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dt == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    elif dt == "fp8_e4m3":
        t = t.view(torch.float8_e4m3fn)
    return t.cuda()


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_attention_token_lightning_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, src_hash, launches_keys):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they
    were taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p)).get(kernel)
    except (ValueError, OSError):
        return None
    if not d or d.get("source_hash") != src_hash:
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(x, sample, min_s=10.0):
    """The CPU oracle on the first `sample` requests of the headline workload."""
    import numpy as np
    import oracle

    b = min(sample, x.B)
    off = x.kv_off[:b + 1].copy()
    n = int(off[-1])
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    # Repeated until about min_s seconds of CPU work have been timed.
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.index_decode(x.q[:b], x.q_dt, x.w[:b], x.kc[:n], x.k_dt, x.k_scale[:n], off, x.H, x.D, x.k,
                            want_scores=False)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            break
    return {"value": n * runs / dt, "unit": "keys/s", "cores": min(threads, b), "kind": "oracle",
            "sample": f"{b} of {x.B} requests x {int(x.kv_off[1] - x.kv_off[0])} keys "
                      f"(scan + top-{x.k}, fp64, OpenMP over requests), {runs} runs in {dt:.1f} s",
            "host_cpu": host_cpu(), "host_logical_cpus": os.cpu_count()}


def host_cpu():
    """The host's CPU model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


MFMA_PROBE_FLOP = {0: 16384.0, 1: 32768.0, 2: 65536.0}  # per product: f16 16x16x32, bf16 32x32x16, fp8 16x16x128


def mfma_ceiling(torch, li, form, iters, reps=3):
    """The matrix-core rate and shader clock of li_mfma_probe's product form
    on constant (1.0) and on random operands, timed like the scans."""
    sink = torch.empty(li.LI_MFMA_PROBE_SINK_WORDS, dtype=torch.float32, device="cuda")
    clk = torch.empty(li.LI_MFMA_PROBE_CLOCK_WORDS, dtype=torch.int32, device="cuda")
    flop = li.LI_MFMA_PROBE_WAVES * iters * li.LI_MFMA_PROBE_PRODUCTS_PER_ITER * MFMA_PROBE_FLOP[form]
    res = {}
    for name, rnd in (("constant", False), ("random", True)):
        for _ in range(2):
            li.li_mfma_probe(form, rnd, iters, sink, clk)
        (ms,) = traced(torch, li, lambda: li.li_mfma_probe(form, rnd, iters, sink, clk), 1, reps)
        c = clk.cpu().numpy().view("uint32").astype("float64").reshape(-1, 2)
        res[name] = {"tflops": flop / (ms * 1e-3) / 1e12, "avg_launch_ms": ms,
                     "shader_clock_mhz": float(c[:, 0].sum() / max(c[:, 1].sum(), 1.0) * 100.0)}
    del sink, clk
    return res


def components(torch, li, inputs, args):
    import numpy as np
    out = {}
    # ---- prefill chunk: T = 4096 against a causal L = 65536 cache (fp8) --------
    x = inputs.cfg3()
    q, qs, w, kc, ks = dev(torch, x.q, "fp8_e4m3"), dev(torch, x.q_scale), dev(torch, x.w), \
        dev(torch, x.kc, "fp8_e4m3"), dev(torch, x.k_scale)
    idx = torch.empty((x.T, x.k), dtype=torch.int32, device="cuda")
    ws = torch.empty(li.lib().li_index_prefill_ws(x.T, x.L, x.k, 0), dtype=torch.uint8, device="cuda")
    fn = lambda: li.li_index_prefill(q, qs, w, kc, ks, x.qpos0, x.k, out_idx=idx, ws=ws)
    # u-row preparation, scan (+ thresholds), select; the first prefill calls
    # in a process run slower than the settled ones, so three warm-up calls
    wall, (prep, scan, topk) = timed(torch, li, fn, 3, args.comp_iters, 3)
    pairs = sum(x.qpos0 + t + 1 for t in range(x.T))
    flop = 2.0 * x.H * x.D * pairs
    out["prefill_fp8_T4096_L65536"] = {
        "prep_ms": prep, "scan_ms": scan, "topk_ms": topk, "step_ms": prep + scan + topk, "total_ms": wall,
        "visible_pairs": pairs,
        "tflops": flop / (scan * 1e-3) / 1e12, "mfma_frac_fp8": flop / (scan * 1e-3) / 1e12 / FP8_PEAK_TFLOPS,
        "mfma_frac_fp8_incl_prep": flop / ((scan + prep) * 1e-3) / 1e12 / FP8_PEAK_TFLOPS,
        "topk_us_per_row": topk * 1e3 / x.T}
    # the fp8 product's rate on this GPU (li_mfma_probe), constant and random operands
    ceil = mfma_ceiling(torch, li, li.LI_MFMA_PROBE_FP8, 400)
    ceil["kernel"] = "mfma_probe_kernel<fp8> (li_mfma_probe): v_mfma_f32_16x16x128_f8f6f4 chains, 8 waves per SIMD"
    out["prefill_fp8_T4096_L65536"]["measured_mfma_ceiling"] = ceil
    out["prefill_fp8_T4096_L65536"]["mfma_frac_of_measured_random"] = \
        flop / (scan * 1e-3) / 1e12 / ceil["random"]["tflops"]
    del q, qs, w, kc, ks, idx, ws, x
    # ---- LatentIndex group: G = 4, B = 16, L = 131072, Dc = 256 (bf16) ----------
    x = inputs.cfg4()
    q, w, wd, lat, off = dev(torch, x.q, "bf16"), dev(torch, x.w), dev(torch, x.w_dec, "bf16"), \
        dev(torch, x.latent, "bf16"), dev(torch, x.kv_off)
    idx = torch.empty((x.B, x.G, x.k), dtype=torch.int32, device="cuda")
    ws = torch.empty(li.lib().li_latent_score_group_ws(x.B, x.n_tok, 131072, x.G, x.H, x.Dc, x.k, 0),
                     dtype=torch.uint8, device="cuda")
    fn = lambda: li.li_latent_score_group(q, w, wd, lat, None, off, 131072, x.k, out_idx=idx, ws=ws)
    wall, (absorb, scan, topk) = timed(torch, li, fn, 3, args.comp_iters, 2)
    lat_bytes = x.n_tok * x.Dc * 2
    flop = 2.0 * x.G * x.H * x.Dc * x.n_tok
    out["latent_G4_B16_L131072"] = {
        "absorb_ms": absorb, "scan_ms": scan, "topk_ms": topk, "total_ms": wall,
        "scan_gbs": lat_bytes / (scan * 1e-3) / 1e9, "scan_hbm_frac": lat_bytes / (scan * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "scan_mfma_frac_fp16": flop / (scan * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    # the fp16 product's rate on this GPU (li_mfma_probe), constant and random operands
    ceil = mfma_ceiling(torch, li, li.LI_MFMA_PROBE_F16, 800)
    ceil["kernel"] = "mfma_probe_kernel<f16> (li_mfma_probe): v_mfma_f32_16x16x32_f16 chains, 6 waves per SIMD"
    out["latent_G4_B16_L131072"]["measured_mfma_ceiling"] = ceil
    out["latent_G4_B16_L131072"]["scan_mfma_frac_of_measured_random"] = \
        flop / (scan * 1e-3) / 1e12 / ceil["random"]["tflops"]
    # the same step with LI_LATENT_SPLIT_BF16 (two bf16 products per element)
    fn = lambda: li.li_latent_score_group(q, w, wd, lat, None, off, 131072, x.k, out_idx=idx, ws=ws,
                                          flags=li.LI_LATENT_SPLIT_BF16)
    wall, (absorb, scan, topk) = timed(torch, li, fn, 3, args.comp_iters, 2)
    out["latent_split_bf16_G4_B16_L131072"] = {
        "absorb_ms": absorb, "scan_ms": scan, "topk_ms": topk, "total_ms": wall,
        "scan_gbs": lat_bytes / (scan * 1e-3) / 1e9, "scan_hbm_frac": lat_bytes / (scan * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "scan_mfma_frac_bf16": 2 * flop / (scan * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    # the same group over an fp8 latent with one scale per 128 values (264 B per token)
    inputs.latent_to_fp8(x)
    lat8, bsc = dev(torch, x.latent, "fp8_e4m3"), dev(torch, x.c_scale)
    fn = lambda: li.li_latent_score_group(q, w, wd, lat8, bsc, off, 131072, x.k, out_idx=idx, ws=ws)
    wall, (absorb, scan, topk) = timed(torch, li, fn, 3, args.comp_iters, 2)
    lat8_bytes = x.n_tok * (x.Dc + 4 * (x.Dc // 128))
    out["latent_fp8_G4_B16_L131072"] = {
        "absorb_ms": absorb, "scan_ms": scan, "topk_ms": topk, "total_ms": wall, "bytes_per_token": x.Dc + 4 * (x.Dc // 128),
        "scan_gbs": lat8_bytes / (scan * 1e-3) / 1e9, "scan_hbm_frac": lat8_bytes / (scan * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "scan_mfma_frac_fp16": flop / (scan * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    del q, w, wd, lat, lat8, bsc, off, idx, ws, x
    # ---- HS decode: fp8 anchor top-8192 + 3 latent followers, B = 16, L = 131072 --
    h = inputs.cfg5()
    a, f = h.anchor, h.followers
    aq, aw, akc, aks, off = dev(torch, a.q, "bf16"), dev(torch, a.w), dev(torch, a.kc, "fp8_e4m3"), \
        dev(torch, a.k_scale), dev(torch, a.kv_off)
    fq, fw, fwd, lat = dev(torch, f.q, "bf16"), dev(torch, f.w), dev(torch, f.w_dec, "bf16"), \
        dev(torch, f.latent, "bf16")
    cand = torch.empty((a.B, h.C), dtype=torch.int32, device="cuda")
    fidx = torch.empty((a.B, f.G, f.k), dtype=torch.int32, device="cuda")
    nidx = torch.empty((a.B, 2048), dtype=torch.int32, device="cuda")
    L = li.lib()
    ws_a = torch.empty(L.li_index_decode_ws(a.B, a.n_tok, 131072, h.C, 0), dtype=torch.uint8, device="cuda")
    ws_f = torch.empty(L.li_hs_refine_ws(a.B, h.C, f.G, f.H, f.Dc, f.k, 0), dtype=torch.uint8, device="cuda")
    fa = lambda: li.li_index_decode(aq, aw, akc, aks, off, 131072, h.C, out_idx=cand, ws=ws_a)
    ff = lambda: li.li_hs_refine(cand, fq, fw, fwd, lat, None, off, f.k, out_idx=fidx, ws=ws_f)
    fn_native = lambda: li.li_index_decode(aq, aw, akc, aks, off, 131072, 2048, out_idx=nidx, ws=ws_a)
    _, (a_scan, a_topk) = timed(torch, li, fa, 2, args.comp_iters, 2)
    _, (f_abs, f_scan, f_topk) = timed(torch, li, ff, 3, args.comp_iters, 2)
    _, (n_scan, n_topk) = timed(torch, li, fn_native, 2, args.comp_iters, 2)
    hs_ms = a_scan + a_topk + f_abs + f_scan + f_topk
    native = n_scan + n_topk
    out["hs_B16_L131072_C8192_F3"] = {
        "anchor_scan_ms": a_scan, "anchor_top8192_ms": a_topk, "follower_absorb_ms": f_abs,
        "follower_gather_scan_ms": f_scan, "follower_top2048_ms": f_topk, "hs_total_ms": hs_ms,
        "native_decode_ms": native, "four_native_layers_over_hs": 4 * native / hs_ms}
    del aq, aw, akc, aks, off, fq, fw, fwd, lat, cand, fidx, nidx, ws_a, ws_f, h, a, f
    # ---- ragged batched decode: B = 32, L_b ~ U{8192..32768} (fp8) --------------
    # Its 86.5 MB of keys would fit in the 256 MB MALL, so the calls rotate over
    # six copies of the cache (519 MB): each call reads keys last touched five
    # calls earlier, after more than the MALL's size of other traffic.
    x = inputs.cfg2()
    q, w, off = dev(torch, x.q, "bf16"), dev(torch, x.w), dev(torch, x.kv_off)
    copies = [(dev(torch, x.kc, "fp8_e4m3"), dev(torch, x.k_scale)) for _ in range(RAGGED_COPIES)]
    idx = torch.empty((x.B, x.k), dtype=torch.int32, device="cuda")
    ws = torch.empty(L.li_index_decode_ws(x.B, x.n_tok, int(x.lens.max()), x.k, 0), dtype=torch.uint8, device="cuda")
    turn = [0]

    def fn():
        kc, ks = copies[turn[0] % RAGGED_COPIES]
        turn[0] += 1
        li.li_index_decode(q, w, kc, ks, off, int(x.lens.max()), x.k, out_idx=idx, ws=ws)
    wall, (scan, topk) = timed(torch, li, fn, 2, max(args.comp_iters, 2 * RAGGED_COPIES), 2)
    out["decode_fp8_B32_ragged8K-32K"] = {
        "scan_ms": scan, "topk_ms": topk, "total_ms": wall, "keys": x.n_tok,
        "scan_gbs": x.n_tok * FP8_KEY_BYTES / (scan * 1e-3) / 1e9,
        "scan_hbm_frac": x.n_tok * FP8_KEY_BYTES / (scan * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "note": f"calls rotate over {RAGGED_COPIES} copies of the 86.5 MB cache so the keys come from HBM, "
                "not the 256 MB MALL"}
    del q, w, off, copies, idx, ws, x
    # ---- decode at shorter contexts: B = 32 x L for L = 8K, 32K (the 128K point
    # is the headline); each cache fits the 256 MB MALL, so the calls rotate over
    # copies holding more than 512 MB together
    sweep = {}
    for Ls in (8192, 32768):
        x = inputs.decode_sweep(Ls)
        q, w, off = dev(torch, x.q, "bf16"), dev(torch, x.w), dev(torch, x.kv_off)
        ncp = -(-(512 << 20) // (x.n_tok * FP8_KEY_BYTES))
        copies = [(dev(torch, x.kc, "fp8_e4m3"), dev(torch, x.k_scale)) for _ in range(ncp)]
        idx = torch.empty((x.B, x.k), dtype=torch.int32, device="cuda")
        ws = torch.empty(L.li_index_decode_ws(x.B, x.n_tok, Ls, x.k, 0), dtype=torch.uint8, device="cuda")
        turn = [0]

        def fn():
            kc, ks = copies[turn[0] % ncp]
            turn[0] += 1
            li.li_index_decode(q, w, kc, ks, off, Ls, x.k, out_idx=idx, ws=ws)
        wall, (scan, topk) = timed(torch, li, fn, 2, max(args.comp_iters, 2 * ncp), 2)
        sweep[f"L{Ls}"] = {"scan_ms": scan, "topk_ms": topk, "total_ms": wall, "copies": ncp,
                           "keys_per_s": x.n_tok / (wall * 1e-3),
                           "scan_gbs": x.n_tok * FP8_KEY_BYTES / (scan * 1e-3) / 1e9,
                           "scan_hbm_frac": x.n_tok * FP8_KEY_BYTES / (scan * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del q, w, off, copies, idx, ws, x
    out["decode_fp8_B32_sweep"] = sweep
    # ---- latent-cache append: prefill chunk (T = 4096) and decode step (B = 16) ---
    # h and W_enc rotate over copies (the chunk's 59 MB would otherwise be served
    # from the 256 MB MALL), as a model step streams other weights in between.
    for x in (inputs.append_prefill(), inputs.append_decode()):
        srcs = [(dev(torch, x.h, "bf16"), dev(torch, x.w_enc, "bf16")) for _ in range(APPEND_COPIES)]
        dst = dev(torch, x.dst_row)
        lat = torch.zeros((x.n_tok, x.Dc), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(L.li_latent_append_ws(x.M, x.d_model, x.Dc, li.LI_BF16), dtype=torch.uint8, device="cuda")
        turn = [0]

        def fn():
            h, wenc = srcs[turn[0] % APPEND_COPIES]
            turn[0] += 1
            li.li_latent_append(h, wenc, dst, lat, ws=ws)
        wall, (gemm, red) = timed(torch, li, fn, 2, max(args.comp_iters, 2 * APPEND_COPIES), 2)
        nbytes = 2 * (x.M * x.d_model + x.Dc * x.d_model + x.M * x.Dc) + 8 * x.M
        flop = 2.0 * x.M * x.Dc * x.d_model
        t = (gemm + red) * 1e-3
        out[x.name] = {
            "gemm_ms": gemm, "reduce_ms": red, "total_ms": wall, "splits": L.li_latent_append_ws(x.M, x.d_model, x.Dc, li.LI_BF16)
            // max(1, x.M * x.Dc * 4), "algorithmic_bytes": nbytes,
            "gbs": nbytes / t / 1e9, "hbm_frac": nbytes / t / 1e9 / HBM_PEAK_GBS,
            "tflops": flop / t / 1e12, "mfma_frac_bf16": flop / t / 1e12 / BF16_PEAK_TFLOPS}
        if x.M > 16:  # the chunk again with fp8 output (codes + one scale per 128 values)
            lat8 = torch.zeros((x.n_tok, x.Dc), dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
            sc8 = torch.zeros((x.n_tok, x.Dc // 128), dtype=torch.float32, device="cuda")
            ws8 = torch.empty(L.li_latent_append_ws(x.M, x.d_model, x.Dc, li.LI_FP8_E4M3), dtype=torch.uint8,
                              device="cuda")

            def fn8():
                h, wenc = srcs[turn[0] % APPEND_COPIES]
                turn[0] += 1
                li.li_latent_append(h, wenc, dst, lat8, c_scale=sc8, ws=ws8)
            wall8, (gemm8, red8) = timed(torch, li, fn8, 2, max(args.comp_iters, 2 * APPEND_COPIES), 2)
            out[x.name.replace("append_", "append_fp8_")] = {"gemm_ms": gemm8, "reduce_ms": red8, "total_ms": wall8}
            del lat8, sc8, ws8
        del srcs, dst, lat, ws
    out.update(stack_component(torch, li, args))
    out.update(attention_component(torch, li, inputs, args))
    out.update(mli_component(torch, li, args))
    return out


def attention_component(torch, li, inputs, args):
    """The selection's consumer on its own: 16 requests x 128 heads attend k =
    2048 of 131072 cached rows (576 bf16 values each)."""
    x = inputs.attention_decode()
    kv = inputs.device_kv_cache(x)
    q, idx, off = dev(torch, x.q, "bf16"), dev(torch, x.idx), dev(torch, x.kv_off)
    o = torch.empty((x.B, x.H, 512), dtype=torch.float32, device="cuda")
    ws = torch.empty(li.lib().li_sparse_attention_ws(x.B, x.H, x.k), dtype=torch.uint8, device="cuda")
    fn = lambda: li.li_sparse_attention(q, kv, idx, off, x.scale, out=o, ws=ws)
    wall, (attn, comb) = timed(torch, li, fn, 2, max(args.comp_iters, 10), 2)
    nbytes = x.B * x.k * 576 * 2 + q.numel() * 2 + o.numel() * 4 + idx.numel() * 4
    flop = 2.0 * x.B * x.H * x.k * (576 + 512)
    t = (attn + comb) * 1e-3
    res = {x.name: {"attn_ms": attn, "combine_ms": comb, "total_ms": wall, "algorithmic_bytes": nbytes,
                    "gbs": nbytes / t / 1e9, "hbm_frac": nbytes / t / 1e9 / HBM_PEAK_GBS,
                    "tflops": flop / t / 1e12, "mfma_frac_bf16": flop / t / 1e12 / BF16_PEAK_TFLOPS}}
    del kv, q, idx, off, o, ws
    return res


def mli_component(torch, li, args, n_layers=8, B=16, L=131072, H_idx=64, H_attn=128, k=2048):
    """Multi-layer Indexer overlap on an n_layers decode stack (each layer with
    its own fp8 indexer cache and bf16 attention cache).  Serial: every layer
    scans, then attends its own selection.  MLI (lag 1): layer 0 is serial;
    layer l attends layer l-1's selection on the main stream while its own
    indexer runs on a second stream, started once the layer's input exists and
    joined before the next layer's attention.  Each schedule is captured once
    into a HIP graph and replayed."""
    g = torch.Generator(device="cuda")
    g.manual_seed(4343)
    n_tok = B * L
    off = torch.arange(0, (B + 1) * L, L, dtype=torch.int64, device="cuda")
    layers = []
    for _ in range(n_layers):
        q = torch.randn((B, H_idx, 128), generator=g, device="cuda").to(torch.bfloat16)
        w = torch.randn((B, H_idx), generator=g, device="cuda") / 8
        kc = torch.randn((n_tok, 128), generator=g, device="cuda").clamp_(-448, 448).to(torch.float8_e4m3fn)
        ks = torch.rand((n_tok,), generator=g, device="cuda") * 1.5 + 0.5
        qa = torch.randn((B, H_attn, 576), generator=g, device="cuda").to(torch.bfloat16)
        kv = torch.randn((n_tok, 576), generator=g, device="cuda").to(torch.bfloat16)
        layers.append((q, w, kc, ks, qa, kv))
    L_ = li.lib()
    sel = [torch.empty((B, k), dtype=torch.int32, device="cuda") for _ in range(n_layers)]
    outs = [torch.empty((B, H_attn, 512), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    ws_i = torch.empty(L_.li_index_decode_ws(B, n_tok, L, k, 0), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(L_.li_sparse_attention_ws(B, H_attn, k), dtype=torch.uint8, device="cuda")
    scale = 1.0 / 192 ** 0.5

    def indexer(l):
        q, w, kc, ks, _, _ = layers[l]
        li.li_index_decode(q, w, kc, ks, off, L, k, out_idx=sel[l], ws=ws_i)

    def attention(l, s):
        qa, kv = layers[l][4], layers[l][5]
        li.li_sparse_attention(qa, kv, sel[s], off, scale, out=outs[l], ws=ws_a)

    side = torch.cuda.Stream()

    def serial():
        for l in range(n_layers):
            indexer(l)
            attention(l, l)

    def mli():
        cur = torch.cuda.current_stream()
        indexer(0)
        attention(0, 0)
        for l in range(1, n_layers):
            side.wait_stream(cur)  # the layer's input exists
            with torch.cuda.stream(side):
                indexer(l)
            attention(l, l - 1)
            cur.wait_stream(side)  # the next layer attends this selection

    def graph_ms(fn, reps=10):
        main = torch.cuda.Stream()
        with torch.cuda.stream(main):
            fn()  # eager warm-up
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=main):
            fn()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            gr.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / reps * 1e3
        del gr
        return ms

    _, (i_scan, i_topk) = timed(torch, li, lambda: indexer(1), 2, 10, 2)
    _, (a_attn, a_comb) = timed(torch, li, lambda: attention(1, 1), 2, 10, 2)
    t_serial = graph_ms(serial)
    t_mli = graph_ms(mli)
    idx_ms = i_scan + i_topk
    attn_ms = a_attn + a_comb
    res = {"serial_ms": t_serial, "mli_ms": t_mli, "speedup": t_serial / t_mli,
           "indexer_ms_per_layer": idx_ms, "attention_ms_per_layer": attn_ms,
           "hidden_ms": t_serial - t_mli,
           "hidden_frac_of_overlappable_attention": (t_serial - t_mli) / ((n_layers - 1) * min(idx_ms, attn_ms)),
           "note": f"{n_layers} layers, B = {B}, L = {L}: per layer an fp8 indexer scan + top-{k} ({H_idx} heads) and "
                   f"a {H_attn}-head attention over {k} selected rows of a 576-value bf16 cache; graph replays, "
                   "wall clock; layer 0 stays serial"}
    del layers, sel, outs, ws_i, ws_a
    torch.cuda.empty_cache()
    return {f"mli_{n_layers}L_B{B}_L{L}": res}


def stack_component(torch, li, args, n_layers=61, B=16, L=131072, G=4, C=8192):
    """Decode-indexer time per step over a 61-layer stack (DeepSeek-V3.2's indexer
    count), every layer with its own cache: native DSA (every layer scans),
    IndexCache at 1/2 and 1/4 retention (li_indexcache_plan: F layers scan into
    the index buffer, S layers reuse it), and LatentIndex + HS (groups of G: an
    fp8 anchor proposing C candidates, G - 1 latent followers refining them).
    Inputs are drawn on the GPU from a seeded generator in the distributions of
    the decode and latent workloads (about 33 GB: too large for host drawing)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    H, D, Dc, k = 64, 128, 256, 2048
    n_tok = B * L
    off = torch.arange(0, (B + 1) * L, L, dtype=torch.int64, device="cuda")
    layers = []
    for _ in range(n_layers):
        q = torch.randn((B, H, D), generator=g, device="cuda").to(torch.bfloat16)
        w = torch.randn((B, H), generator=g, device="cuda") / 8
        kc = torch.randn((n_tok, D), generator=g, device="cuda").clamp_(-448, 448).to(torch.float8_e4m3fn)
        ks = torch.rand((n_tok,), generator=g, device="cuda") * 1.5 + 0.5
        layers.append((q, w, kc, ks))
    n_groups = n_layers // G
    groups = []
    for _ in range(n_groups):
        fq = torch.randn((B, G - 1, H, D), generator=g, device="cuda").to(torch.bfloat16)
        fw = torch.randn((B, G - 1, H), generator=g, device="cuda") / 8
        wd = (torch.randn((G - 1, Dc, H * D), generator=g, device="cuda") / Dc ** 0.5).to(torch.bfloat16)
        lat = torch.randn((n_tok, Dc), generator=g, device="cuda").to(torch.bfloat16)
        groups.append((fq, fw, wd, lat))
    L_ = li.lib()
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    cand = torch.empty((B, C), dtype=torch.int32, device="cuda")
    fidx = torch.empty((B, G - 1, k), dtype=torch.int32, device="cuda")
    ws_d = torch.empty(L_.li_index_decode_ws(B, n_tok, L, C, 0), dtype=torch.uint8, device="cuda")
    ws_f = torch.empty(L_.li_hs_refine_ws(B, C, G - 1, H, Dc, k, 0), dtype=torch.uint8, device="cuda")

    def indexcache(retain_every):
        n_f, src = li.li_indexcache_plan(n_layers, retain_every)
        full = [l for l in range(n_layers) if src[l] == l]
        assert len(full) == n_f

        def step():
            for l in full:  # S layers attend idx as the last F layer left it
                q, w, kc, ks = layers[l]
                li.li_index_decode(q, w, kc, ks, off, L, k, out_idx=idx, ws=ws_d)
        return step, n_f

    def hs_step():
        for gi in range(n_groups):
            q, w, kc, ks = layers[gi * G]
            fq, fw, wd, lat = groups[gi]
            li.li_index_decode(q, w, kc, ks, off, L, C, out_idx=cand, ws=ws_d)
            li.li_hs_refine(cand, fq, fw, wd, lat, None, off, k, out_idx=fidx, ws=ws_f)
        for l in range(n_groups * G, n_layers):  # layers past the last whole group scan natively
            q, w, kc, ks = layers[l]
            li.li_index_decode(q, w, kc, ks, off, L, k, out_idx=idx, ws=ws_d)

    def wall(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps * 1e3

    res = {}
    for name, r in (("dsa", 1), ("indexcache_half", 2), ("indexcache_quarter", 4)):
        fn, n_f = indexcache(r)
        res[name + "_ms"] = wall(fn)
        res[name + "_scans"] = n_f
    res["latentindex_hs_ms"] = wall(hs_step)
    res["latentindex_hs_anchor_scans"] = n_groups + (n_layers - n_groups * G)
    for name in ("indexcache_half", "indexcache_quarter", "latentindex_hs"):
        res[name + "_speedup"] = res["dsa_ms"] / res[name + "_ms"]
    res["note"] = (f"decode-indexer ms per step (B = {B} tokens) summed over {n_layers} indexer layers, each with its "
                   f"own fp8 key cache at L = {L}; HS groups of {G} share a bf16 latent (Dc = {Dc}), C = {C}")
    del layers, groups, idx, cand, fidx, ws_d, ws_f
    torch.cuda.empty_cache()
    return {f"stack{n_layers}_B{B}_L{L}": res}


def ab_compare(torch, li, inputs, args):
    """Two builds of the library on one workload, alternating in one process
    (same inputs, same GPU state drift for both): per round and build, a few
    warm-up calls and then traced calls; prints the median per-kernel
    microseconds of each build and whether their indices agree."""
    import statistics
    builds = {}
    for name, path in (("package", li.LIB_PATH), ("other", os.path.abspath(args.ab_lib))):
        li._lib = None
        li.LIB_PATH = path
        builds[name] = li.lib()
    if args.ab_workload in ("decode", "decode16", "anchor"):
        # the headline; B = 16 at k = 2048; the HS anchor (B = 16, k = 8192)
        x = inputs.decode_sweep(131072, B=32 if args.ab_workload == "decode" else 16)
        kk = 8192 if args.ab_workload == "anchor" else x.k
        q, w, kc, ks, off = dev(torch, x.q, "bf16"), dev(torch, x.w), dev(torch, x.kc, "fp8_e4m3"), \
            dev(torch, x.k_scale), dev(torch, x.kv_off)
        kernels, iters = ("scan", "top-k"), 20
        def setup(L):
            ws = torch.empty(L.li_index_decode_ws(x.B, x.n_tok, 131072, kk, 0), dtype=torch.uint8, device="cuda")
            idx = torch.empty((x.B, kk), dtype=torch.int32, device="cuda")
            return idx, lambda: li.li_index_decode(q, w, kc, ks, off, 131072, kk, out_idx=idx, ws=ws)
    elif args.ab_workload in ("ragged", "decode8k"):
        # as the ragged and sweep components: calls rotate over copies of the cache so the keys come from HBM
        x = inputs.cfg2() if args.ab_workload == "ragged" else inputs.decode_sweep(8192)
        q, w, off = dev(torch, x.q, "bf16"), dev(torch, x.w), dev(torch, x.kv_off)
        ncp = max(RAGGED_COPIES, -(-(512 << 20) // (x.n_tok * FP8_KEY_BYTES)))
        copies = [(dev(torch, x.kc, "fp8_e4m3"), dev(torch, x.k_scale)) for _ in range(ncp)]
        ml = int(x.lens.max())
        kernels, iters = ("scan", "top-k"), 2 * ncp
        def setup(L):
            ws = torch.empty(L.li_index_decode_ws(x.B, x.n_tok, ml, x.k, 0), dtype=torch.uint8, device="cuda")
            idx = torch.empty((x.B, x.k), dtype=torch.int32, device="cuda")
            turn = [0]
            def fn():
                kc, ks = copies[turn[0] % ncp]
                turn[0] += 1
                li.li_index_decode(q, w, kc, ks, off, ml, x.k, out_idx=idx, ws=ws)
            return idx, fn
    elif args.ab_workload == "prefill":
        x = inputs.cfg3()
        q, qs, w, kc, ks = dev(torch, x.q, "fp8_e4m3"), dev(torch, x.q_scale), dev(torch, x.w), \
            dev(torch, x.kc, "fp8_e4m3"), dev(torch, x.k_scale)
        kernels, iters = ("prep", "scan", "top-k"), 5
        def setup(L):
            ws = torch.empty(L.li_index_prefill_ws(x.T, x.L, x.k, 0), dtype=torch.uint8, device="cuda")
            idx = torch.empty((x.T, x.k), dtype=torch.int32, device="cuda")
            return idx, lambda: li.li_index_prefill(q, qs, w, kc, ks, x.qpos0, x.k, out_idx=idx, ws=ws)
    else:
        x = inputs.cfg4()
        q, w, wd, lat, off = dev(torch, x.q, "bf16"), dev(torch, x.w), dev(torch, x.w_dec, "bf16"), \
            dev(torch, x.latent, "bf16"), dev(torch, x.kv_off)
        B = len(x.kv_off) - 1
        kernels, iters = ("absorb", "scan", "top-k"), 10
        def setup(L):
            ws = torch.empty(L.li_latent_score_group_ws(B, x.n_tok, 131072, x.G, x.H, x.Dc, x.k, 0),
                             dtype=torch.uint8, device="cuda")
            idx = torch.empty((B, x.G, x.k), dtype=torch.int32, device="cuda")
            return idx, lambda: li.li_latent_score_group(q, w, wd, lat, None, off, 131072, x.k, out_idx=idx, ws=ws)
    times, outs = {n: [] for n in builds}, {}
    for rnd in range(args.ab_rounds):
        for name, L in builds.items():
            li._lib = L
            idx, fn = setup(L)
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            t = traced(torch, li, fn, len(kernels), iters)
            times[name].append([v * 1e3 for v in t])
            outs[name] = idx.clone()
            log(f"[ab] round {rnd} {name}: " + ", ".join(f"{k} {v * 1e3:.1f} us" for k, v in zip(kernels, t)))
            del idx, fn
    res = {"workload": args.ab_workload, "other": args.ab_lib, "rounds": args.ab_rounds, "traced_calls": iters,
           "median_us": {n: {k: statistics.median(r[j] for r in v) for j, k in enumerate(kernels)}
                         for n, v in times.items()},
           "indices_identical": bool(torch.equal(outs["package"], outs["other"]))}
    print(json.dumps(res), flush=True)


def phase_stamps(torch, li, inputs, args, calls=20):
    """The bucket top-k's phases at the headline shape, from the stamps build:
    after each call, thread 0 of every row's workgroup has recorded the
    100 MHz real-time counter after each phase's barrier.  Prints, per phase,
    the median over rows and calls of the time from the row's start, and the
    median over calls of the slowest row."""
    import statistics
    li._lib = None
    li.LIB_PATH = os.path.abspath(args.stamps_lib)
    L = li.lib()
    L.li_read_stamps.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    L.li_read_stamps.restype = ctypes.c_int32
    x = inputs.decode_sweep(131072, B=32 if args.stamps_workload == "decode" else 16)
    k = 2048 if args.stamps_workload == "decode" else 8192
    q, w, kc, ks, off = dev(torch, x.q, "bf16"), dev(torch, x.w), dev(torch, x.kc, "fp8_e4m3"), \
        dev(torch, x.k_scale), dev(torch, x.kv_off)
    ws = torch.empty(L.li_index_decode_ws(x.B, x.n_tok, 131072, k, 0), dtype=torch.uint8, device="cuda")
    idx = torch.empty((x.B, k), dtype=torch.int32, device="cuda")
    phases = {1: "partials and list prefixes loaded, Q summed", 2: "b* and the list starts",
              3: "candidates in LDS", 5: "radix levels", 6: "bitmaps marked", 7: "word prefixes",
              8: "slots placed", 9: "output row written"}
    buf = (ctypes.c_ulonglong * (64 * 10))()
    per, slow = {p: [] for p in phases}, {p: [] for p in phases}
    for c in range(calls + 3):
        li.li_index_decode(q, w, kc, ks, off, 131072, k, out_idx=idx, ws=ws)
        torch.cuda.synchronize()
        if c < 3:
            continue
        if L.li_read_stamps(ctypes.addressof(buf), 64 * 10) != 0:
            raise RuntimeError("li_read_stamps failed")
        t0 = min(buf[r * 10] for r in range(x.B))
        for p in phases:
            v = [(buf[r * 10 + p] - buf[r * 10]) / 100.0 for r in range(x.B)]
            per[p] += v
            slow[p].append(max((buf[r * 10 + p] - t0) / 100.0 for r in range(x.B)))
    res = {"workload": f"decode fp8 B={x.B} L=131072 top-{k}", "calls": calls, "unit": "us",
           "phases": {phases[p]: {"median_row": statistics.median(per[p]), "slowest_row": statistics.median(slow[p])}
                      for p in phases}}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--comp-iters", type=int, default=5, help="timed iterations per component")
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=32, help="requests in the oracle's timed sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counter scaling)")
    ap.add_argument("--ab-lib", default=None,
                    help="A/B mode: path of another build of libli.so; alternate it with the package's build on "
                         "--ab-workload in one process and print the per-kernel medians (no bench line)")
    ap.add_argument("--ab-workload", default="decode",
                    choices=["decode", "decode16", "anchor", "decode8k", "ragged", "prefill", "latent"])
    ap.add_argument("--ab-rounds", type=int, default=4)
    ap.add_argument("--stamps-workload", default="decode", choices=["decode", "anchor"],
                    help="decode: B = 32 x 131072, k = 2048; anchor: the HS anchor, B = 16 x 131072, k = 8192")
    ap.add_argument("--stamps-lib", default=None,
                    help="phase mode: path of the stamps build (build.py --stamps); run the headline decode and "
                         "print the bucket top-k's per-phase times (no bench line)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}, WORLD_SIZE {world}): the indexer "
              f"path here is single-GPU; sharding across GPUs is a design note, not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_token_lightning_amd as li
    from sparse_attention_token_lightning_amd import inputs

    torch.cuda.set_device(0)
    if args.ab_lib:
        ab_compare(torch, li, inputs, args)
        return
    if args.stamps_lib:
        phase_stamps(torch, li, inputs, args)
        return
    log("[bench] generating decode B=32 L=131072 fp8 inputs")
    x = inputs.decode_sweep(131072)
    B, Lk = x.B, 131072
    q, w, kc, ks, off = dev(torch, x.q, "bf16"), dev(torch, x.w), dev(torch, x.kc, "fp8_e4m3"), \
        dev(torch, x.k_scale), dev(torch, x.kv_off)
    idx = torch.empty((B, x.k), dtype=torch.int32, device="cuda")
    ws = torch.empty(li.lib().li_index_decode_ws(B, x.n_tok, Lk, x.k, 0), dtype=torch.uint8, device="cuda")
    step = lambda: li.li_index_decode(q, w, kc, ks, off, Lk, x.k, out_idx=idx, ws=ws)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    log(f"[bench] warmup {args.warmup}, timing {args.steps} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    # The same steps again with the library's HIP events on its stream:
    # start | after scan | after top-k.
    scan_ms, topk_ms = traced(torch, li, step, 2, args.steps)
    keys = B * Lk
    achieved = keys * FP8_KEY_BYTES / (scan_ms * 1e-3) / 1e9
    # The read rate this GPU reaches for a plain stream of the same key bytes
    # with the scan's load pattern (li_read_probe), timed the same way.
    sink = torch.empty(li.LI_READ_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    for _ in range(3):
        li.li_read_probe(kc, sink)
    (probe_ms,) = traced(torch, li, lambda: li.li_read_probe(kc, sink), 1, args.steps)
    probe_bytes = kc.numel() * kc.element_size()
    probe_gbs = probe_bytes / (probe_ms * 1e-3) / 1e9
    del sink
    traffic = load_traffic("decode_score", source_hash("decode.hip", "li_device.h", "li_select.h"), keys)
    log(f"[bench] step {ms_per_step:.3f} ms, scan {scan_ms * 1e3:.1f} us ({achieved:.0f} GB/s), "
        f"top-2048 {topk_ms * 1e3:.1f} us; read probe {probe_ms * 1e3:.1f} us ({probe_gbs:.0f} GB/s)")

    result = {
        "metric": METRIC,
        "value": keys / (ms_per_step * 1e-3),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_fp8_B32_L131072", "B": B, "L": Lk, "H": x.H, "D": x.D, "k": x.k,
                   "k_cache": "fp8_e4m3 + fp32 per-token scale", "q": "bf16", "mfma": "bf16 x bf16 -> fp32",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "decode_score", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": keys * FP8_KEY_BYTES, "avg_launch_ms": scan_ms,
                     "measured_read_ceiling": {
                         "gbs": probe_gbs, "bytes": probe_bytes, "avg_launch_ms": probe_ms,
                         "frac_of_ceiling": achieved / probe_gbs, "ceiling_frac_of_peak": probe_gbs / HBM_PEAK_GBS,
                         "kernel": "read_probe_kernel (li_read_probe): the key bytes streamed with the scan's "
                                   "load pattern, back to back, same timing method"},
                     "timing": "HIP start/stop events of the kernel's own launch (hipExtLaunchKernel), on "
                               "the library's stream, averaged over a repetition of the timed steps"},
        "components": {"decode_fp8_B32_L131072": {"scan_ms": scan_ms, "top2048_ms": topk_ms,
                                                  "top2048_us": topk_ms * 1e3,
                                                  "scan_gbs": achieved}},
    }
    if not args.no_components:
        log("[bench] components: prefill, latent, HS, ragged decode, latent append")
        del ws
        result["components"].update(components(torch, li, inputs, args))
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle on {args.cpu_sample} requests")
        result["cpu_baseline"] = cpu_baseline(x, args.cpu_sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
