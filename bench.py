"""Benchmark of the fused attention hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  1. fa_fwd      bf16 causal prefill, B=1 H=32 N=16384 d=128   (headline)
  2. fa_quantize_fp8_qkv  rotation + E4M3 block quantiser of Q, K (with R)
                 and V (without) of the fp8 workload's shape, one launch,
                 timed before the fp8 forward as a caller runs them
  3. fa_fwd_fp8  E4M3 causal prefill, B=2 H=16 N=8192 d=128
  4. fa_paged_decode  64 sequences, H=32, d=128, contexts 512..32768
  5. fa_bwd      backward of (1) given its O, L and a seeded dO (the first
                 of the next rows; TFLOP/s on the 5-product count, 2.5x the
                 forward's)
  6. fa_paged_prefill  chunked prefill through the block table: the last
                 2048 tokens of 16 sequences (contexts 2048..16384), H=32, d=128
  7. fa_fwd_block_sparse  the inputs of (1) with a seeded block mask keeping
                 half of the causal 128 x 128 blocks (the diagonal always),
                 without and with dropout p = 0.1
  8. fa_fwd      bf16 non-causal MHA, B=4 H=16 N=2048 d=64
Each launch is bracketed by HIP events on the stream it runs on. `value` is
the prefill's TFLOP/s (4*B*H*N^2*d, halved for causal, per the kernel's mean
event time); decode GB/s and fp8 TFLOP/s are reported beside it. The CPU
baselines are the fp64 oracle, timed on bounded samples of the prefill and
decode workloads on this host's cores. After the timed steps the headline
prefill runs back to back for about a second while the GPU's gfx clock is
sampled (amdsmi), for a clock-adjusted fraction of peak beside the spec one,
and then the same launch on all-zero Q, K, V is timed and clocked the same
way (roofline.zero_inputs): identical instructions and traffic, so the gap
shows how far the chip's clock drops under MFMAs on random operands.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd TFLOP/s & % MFMA peak (N=16k,d=128 causal); decode HBM GB/s"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def measured_traffic(summary):
    """HBM bytes per launch from a committed rocprofv3 counter summary
    (profiles/<summary>), or None when the kernel sources it names (and the
    build script with their compile flags) have changed since the counters
    were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path, encoding="utf-8"):
        if " = " in line and not line.startswith("|"):
            key, val = line.strip().split(" = ", 1)
            kv[key] = val
    try:
        h = hashlib.sha256()
        for src in kv["sources"].split():
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != kv["source_sha256"]:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def decode_bytes(p):
    """Algorithmic HBM bytes of one decode: every unique (page, head) slot of a
    valid token read once for K and once for V, plus q, O, L and the table
    entries read. Also returns the logical (per-sequence) count."""
    import numpy as np
    ctx = p.ctx_lens.cpu().numpy().astype(np.int64)
    bt = p.block_table.cpu().numpy()
    S, H, d = p.q.shape
    per_tok = 2 * H * d * 2                      # K and V, all heads, bf16
    logical_tok = int(ctx.sum())
    seen = {}
    for s in range(S):
        nb = (int(ctx[s]) + 15) // 16
        for b in range(nb):
            valid = min(16, int(ctx[s]) - 16 * b)
            pg = int(bt[s, b])
            seen[pg] = max(seen.get(pg, 0), valid)
    unique_tok = sum(seen.values())
    fixed = S * H * d * 2 * 2 + S * H * 4 + int(((ctx + 15) // 16).sum()) * 4 + S * 4
    return unique_tok * per_tok + fixed, logical_tok * per_tok + fixed


def cpu_baseline(x, budget_s=20.0):
    """Time the fp64 oracle on a bounded sample of the causal prefill: query rows
    i = stride-1 mod stride of the first h heads. A first head at stride 64,
    timed after one untimed run of it, sets the pace; the stride and head count
    are then chosen so that the whole sample takes about budget_s."""
    import numpy as np
    import oracle
    B, H, N, d = x.q.shape
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    stride = 64
    rows = np.arange(stride - 1, N, stride)

    def head_f64(t, h):
        return oracle.bf16_bits_to_f64(t[0, h].contiguous().view(__import__("torch").int16).numpy().view(np.uint16))

    def run(heads):
        flops = 0.0
        t = 0.0
        for h in heads:
            q, k, v = head_f64(x.q, h), head_f64(x.k, h), head_f64(x.v, h)
            t0 = time.perf_counter()
            oracle.attention_rows(q[rows], rows, k, v, x.scale, True)
            t += time.perf_counter() - t0
            flops += float(np.sum(4.0 * d * (rows + 1)))
        return flops, t

    run([0])                                 # warm: threads, page faults, caches
    f1, t1 = run([0])
    per_head = max(t1, 1e-3)                 # seconds per head at stride 64
    n_heads = H - 1
    while stride > 1 and per_head * 2 * n_heads <= budget_s:
        stride //= 2
        per_head *= 2
    n_heads = max(1, min(H - 1, int(budget_s / per_head)))
    rows = np.arange(stride - 1, N, stride)
    f, t = run(list(range(1, n_heads + 1)))
    return {"value": f / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "fp64 oracle on causal B1 H32 N16384 d128 query rows i %% %d == %d of heads "
                      "1..%d (%d rows, %.3g flop, %.1f s)" % (stride, stride - 1, n_heads,
                                                            n_heads * len(rows), f, t)}


def device_info(dev):
    """GPU name, ROCm / HIP versions and host CPU of this run."""
    import torch
    info = {"gpu": torch.cuda.get_device_name(dev),
            "arch": torch.cuda.get_device_properties(dev).gcnArchName,
            "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count,
            "hip": torch.version.hip}
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        info["rocm"] = None
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        try:
            h = amdsmi.amdsmi_get_processor_handles()[0]
            info["market_name"] = amdsmi.amdsmi_get_gpu_asic_info(h).get("market_name")
            try:
                info["product_name"] = amdsmi.amdsmi_get_gpu_board_info(h).get("product_name")
            except Exception:
                info["product_name"] = None
        finally:
            amdsmi.amdsmi_shut_down()
    except Exception:          # the tool library is optional: report what is known
        info["market_name"] = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["host_cpu"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return info


def clock_window(fn, seconds=2.0):
    """Run fn back to back for about `seconds` while another thread samples the
    current gfx clock of every XCD (amdsmi GPU metrics); returns the median
    over the samples of the second half of the window of the mean XCD clock in
    MHz, or None without amdsmi. The metrics table lags the activity (a window
    right after a heavier one still reads that one's clock), so the first half
    is not used."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception:
        return None
    samples, stop = [], threading.Event()

    def poll():
        t_start = time.perf_counter()
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                clk = [c for c in m.get("current_gfxclks", []) if isinstance(c, (int, float)) and 0 < c < 10000]
                if clk and time.perf_counter() - t_start >= seconds / 2:
                    samples.append(sum(clk) / len(clk))
            except Exception:
                pass
            time.sleep(0.01)
    try:
        fn()
        torch.cuda.synchronize()
        t = threading.Thread(target=poll)
        t.start()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                fn()
            torch.cuda.synchronize()
        stop.set()
        t.join()
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass
    if not samples:
        return None
    samples.sort()
    return samples[len(samples) // 2]


def digest(*tensors):
    """SHA-256 (first 16 hex digits) of the raw bytes of host or device tensors."""
    import hashlib
    import torch
    h = hashlib.sha256()
    for t in tensors:
        t = t.detach().contiguous()
        if t.dtype in (torch.bfloat16, torch.float8_e4m3fn):
            t = t.view(torch.uint8)
        h.update(t.cpu().numpy().tobytes())
    return h.hexdigest()[:16]


def pool_digest(p):
    """Digest of a paged pool: q, block table, contexts, and one int64 sum of
    the raw 16-bit words of every page of each cache (computed on the device;
    hashing 17 GB of pages byte by byte on the host would take minutes)."""
    import torch
    sums = [c.view(torch.int16).sum(dim=(1, 2, 3), dtype=torch.int64) for c in (p.kcache, p.vcache)]
    return digest(p.q, p.block_table, p.ctx_lens, *sums)


def decode_cpu_baseline(p, budget_s=10.0):
    """Time the fp64 oracle's paged decode on whole sequences of the decode
    workload (all heads), taken in sequence order until about budget_s of
    oracle time; GB/s = K and V bytes of their contexts / time (the gather of
    each sequence's pages to the host is not timed)."""
    import numpy as np
    import torch
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    ctx = p.ctx_lens.cpu().numpy()
    bt = p.block_table.cpu().numpy()
    S, H, d = p.q.shape
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    seconds, nbytes, done = 0.0, 0, []
    for s in range(S):
        nb = (int(ctx[s]) + 15) // 16
        pages = torch.from_numpy(bt[s, :nb].astype(np.int64)).to(p.kcache.device)
        kc, vc = bits(p.kcache.index_select(0, pages)), bits(p.vcache.index_select(0, pages))
        qf = oracle.bf16_bits_to_f64(bits(p.q[s:s + 1]))
        table = np.arange(nb, dtype=np.int32)[None, :]
        t0 = time.perf_counter()
        oracle.paged_decode(qf, kc, vc, table, ctx[s:s + 1], p.scale)
        seconds += time.perf_counter() - t0
        nbytes += int(ctx[s]) * H * d * 2 * 2
        done.append(int(s))
        if seconds >= budget_s:
            break
    return {"value": nbytes / seconds / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "fp64 oracle paged decode of %d whole sequences (all %d heads; contexts %d..%d, "
                      "%.3g B of K and V, %.1f s)" % (len(done), H, int(ctx[done].min()), int(ctx[done].max()),
                                                      nbytes, seconds)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--only", default="",
                    help="comma list of prefill,fp8,decode,backward,paged_prefill,block_sparse,"
                         "fp8_quantize,mha (default all)")
    ap.add_argument("--no-clock", action="store_true", help="skip the clock-sampling window")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the path would shard heads / sequences across GPUs with no communication)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_106_amd as fa
    from exact_attention_106_amd import inputs

    only = set(filter(None, args.only.split(","))) or {"prefill", "fp8", "decode", "backward", "paged_prefill",
                                                         "block_sparse", "fp8_quantize", "mha"}
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fa.fa_version()

    log("generating inputs")
    parts = []
    digests = {}
    if "prefill" in only:
        x3 = inputs.config3()
        digests["causal_bf16_B1H32N16384d128"] = digest(x3.q, x3.k, x3.v)
        q3, k3, v3 = x3.q.to(dev), x3.k.to(dev), x3.v.to(dev)
        o3 = torch.empty_like(q3)
        l3 = torch.empty(q3.shape[:3], dtype=torch.float32, device=dev)
        parts.append(("prefill", lambda: fa.fa_fwd(q3, k3, v3, scale=x3.scale, causal=True, out=o3, lse=l3)))
    if "fp8_quantize" in only:
        # Q and K of the fp8 workload's shape with the incoherent rotation, V
        # without; timed right before the FP8 forward, the order a caller runs them
        qz = [inputs.quant_inputs(2, 16, 8192, 128, seed=40 + i) for i in range(3)]
        digests["fp8_quantize_B2H16N8192d128"] = digest(*[x for x, _ in qz], qz[0][1])
        xz = [x.to(dev) for x, _ in qz]
        rz = qz[0][1].to(dev)
        oz = [(torch.empty(x.shape, dtype=torch.uint8, device=dev),
               torch.empty((2, 16, 64), dtype=torch.float32, device=dev)) for x in xz]
        parts.append(("fp8_quantize", lambda: fa.fa_quantize_fp8_qkv(*xz, rz, out=oz)))
    if "fp8" in only:
        x4 = inputs.config4()
        digests["causal_fp8_B2H16N8192d128"] = digest(x4.q8, x4.k8, x4.v8, x4.q_scale, x4.k_scale, x4.v_scale)
        t4 = [t.to(dev) for t in (x4.q8, x4.k8, x4.v8, x4.q_scale, x4.k_scale, x4.v_scale)]
        o4 = torch.empty(x4.q8.shape, dtype=torch.bfloat16, device=dev)
        l4 = torch.empty(x4.q8.shape[:3], dtype=torch.float32, device=dev)
        parts.append(("fp8", lambda: fa.fa_fwd_fp8(*t4, scale=x4.scale, causal=True, out=o4, lse=l4)))
    if "decode" in only:
        p5 = inputs.config5(device=dev)
        digests["paged_decode_S64H32d128"] = pool_digest(p5)
        ws = torch.empty(fa.fa_paged_decode_workspace_bytes(64, 32, 128, 16, p5.block_table.shape[1]),
                         dtype=torch.uint8, device=dev)
        o5 = torch.empty(p5.q.shape, dtype=torch.bfloat16, device=dev)
        l5 = torch.empty(p5.q.shape[:2], dtype=torch.float32, device=dev)
        parts.append(("decode", lambda: fa.fa_paged_decode(p5.q, p5.kcache, p5.vcache, p5.block_table,
                                                           p5.ctx_lens, scale=p5.scale, workspace=ws,
                                                           out=o5, lse=l5)))
    if "backward" in only:
        if "prefill" not in only:
            x3 = inputs.config3()
            q3, k3, v3 = x3.q.to(dev), x3.k.to(dev), x3.v.to(dev)
            o3 = torch.empty_like(q3)
            l3 = torch.empty(q3.shape[:3], dtype=torch.float32, device=dev)
        fa.fa_fwd(q3, k3, v3, scale=x3.scale, causal=True, out=o3, lse=l3)
        g3 = inputs.grad_out(1, 32, 16384, 128, seed=6).to(dev)
        wsb = torch.empty(fa.fa_bwd_workspace_bytes(1, 32, 16384, 128), dtype=torch.uint8, device=dev)
        dq3, dk3, dv3 = (torch.empty_like(q3) for _ in range(3))
        parts.append(("backward", lambda: fa.fa_bwd(q3, k3, v3, o3, l3, g3, scale=x3.scale, causal=True,
                                                    workspace=wsb, dq=dq3, dk=dk3, dv=dv3)))
    if "paged_prefill" in only:
        p6 = inputs.paged_prefill_workload(device=dev)
        o6 = torch.empty(p6.q.shape, dtype=torch.bfloat16, device=dev)
        l6 = torch.empty(p6.q.shape[:3], dtype=torch.float32, device=dev)
        parts.append(("paged_prefill", lambda: fa.fa_paged_prefill(p6.q, p6.kcache, p6.vcache, p6.block_table,
                                                                   p6.ctx_lens, scale=p6.scale, out=o6, lse=l6)))
    if "block_sparse" in only:
        if "prefill" not in only and "backward" not in only:
            x3 = inputs.config3()
            q3, k3, v3 = x3.q.to(dev), x3.k.to(dev), x3.v.to(dev)
        bmask = inputs.block_mask(16384, density=0.5, seed=9, causal=True)
        bmask_d = bmask.to(dev)
        o7 = torch.empty_like(q3)
        l7 = torch.empty(q3.shape[:3], dtype=torch.float32, device=dev)
        parts.append(("block_sparse", lambda: fa.fa_fwd_block_sparse(q3, k3, v3, bmask_d, scale=x3.scale, causal=True,
                                                                     out=o7, lse=l7)))
        parts.append(("block_sparse_dropout", lambda: fa.fa_fwd_block_sparse(q3, k3, v3, bmask_d, scale=x3.scale,
                                                                             causal=True, dropout_p=0.1, seed=11,
                                                                             out=o7, lse=l7)))
    if "mha" in only:
        x2 = inputs.config2()
        digests["mha_bf16_B4H16N2048d64"] = digest(x2.q, x2.k, x2.v)
        q2, k2, v2 = x2.q.to(dev), x2.k.to(dev), x2.v.to(dev)
        o2 = torch.empty_like(q2)
        l2 = torch.empty(q2.shape[:3], dtype=torch.float32, device=dev)
        parts.append(("mha", lambda: fa.fa_fwd(q2, k2, v2, scale=x2.scale, causal=False, out=o2, lse=l2)))
    torch.cuda.synchronize()

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        for _, fn in parts:
            fn()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)] for name, _ in parts}
    log("timing %d steps" % args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for name, fn in parts:
            a, b = ev[name][i]
            a.record(stream)
            fn()
            b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {name: sum(a.elapsed_time(b) for a, b in ev[name]) / args.steps for name, _ in parts}
    log("mean ms per launch: %s" % ms)

    def spread(name, launches=1):
        t = sorted(a.elapsed_time(b) / launches for a, b in ev[name])
        q = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]
        return {"p10": q(0.1), "median": q(0.5), "p90": q(0.9)}
    sclk = None
    zero_inputs = None
    if not args.no_clock and "prefill" in only:
        log("clock window")
        sclk = clock_window(lambda: fa.fa_fwd(q3, k3, v3, scale=x3.scale, causal=True, out=o3, lse=l3))
        # The same kernel, shape and launch on all-zero Q, K, V: the same
        # instructions and memory traffic, far less switching in the matrix
        # cores. The gap between the two is the chip lowering its clock under
        # the power drawn by MFMAs on random operands (context, not a result).
        zq, zk, zv = (torch.zeros_like(t) for t in (q3, k3, v3))
        zrun = lambda: fa.fa_fwd(zq, zk, zv, scale=x3.scale, causal=True, out=o3, lse=l3)
        zclk = clock_window(zrun)
        za, zb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        za.record(stream)
        for _ in range(20):
            zrun()
        zb.record(stream)
        torch.cuda.synchronize()
        zms = za.elapsed_time(zb) / 20
        ztf = prefill_flops(1, 32, 16384, 128, True) / (zms * 1e-3) / 1e12
        zero_inputs = {"workload": "causal bf16 prefill B1 H32 N16384 d128 on all-zero Q, K, V",
                       "launch_ms": zms, "tflops": ztf, "frac": ztf / PEAK_BF16_TFLOPS, "sclk_mhz": zclk}
        del zq, zk, zv
    # A plain streaming read on the same GPU (the library's fa_read_probe over
    # 8 GiB, far beyond every cache), best of 5: the practical ceiling beside
    # the spec peak for the decode, whose only significant traffic is
    # reading each needed page once.
    read_probe = None
    if "decode" in only and not args.no_clock:
        big = torch.ones(8 << 30, dtype=torch.uint8, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        fa.fa_read_probe(big, sink)
        torch.cuda.synchronize()
        best = None
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fa.fa_read_probe(big, sink)
            b.record(stream)
            torch.cuda.synchronize()
            t = a.elapsed_time(b)
            best = t if best is None else min(best, t)
        read_probe = {"kernel": "fa_read_probe over 8 GiB", "ms": best, "GBps": big.numel() / (best * 1e-3) / 1e9}
        del big, sink
    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy of %d MiB done" % args.calib_copy_mib)

    result = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic (seeded N(0,1); fp8 with outliers, Haar rotation, block E4M3; "
                      "paged pool with shared prefixes)",
              "config": {"workload": "causal bf16 prefill B1 H32 N16384 d128 + fp8 causal prefill "
                                     "B2 H16 N8192 d128 + paged decode S64 H32 d128 ctx 512..32768",
                         "global_batch": 1, "seq_len": 16384, "parallelism": "single GPU"},
              "device": device_info(dev), "sclk_mhz": sclk, "input_sha256": digests}
    if "prefill" in ms:
        f = prefill_flops(1, 32, 16384, 128, True)
        tf = f / (ms["prefill"] * 1e-3) / 1e12
        result["value"] = tf
        result["roofline"] = {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                              "traffic": measured_traffic("pmc_fwd_prefill_bf16_causal_B1H32N16384d128.md"),
                              "kernel": "fwd_kernel3<128,causal,bf16>", "launch_ms": ms["prefill"],
                              "launch_ms_spread": spread("prefill"), "flop_per_launch": f}
        if sclk:
            # the same fraction against the peak at the gfx clock measured while the kernel ran
            result["roofline"]["frac_at_sclk"] = tf / (PEAK_BF16_TFLOPS * sclk / 2400.0)
        if zero_inputs:
            result["roofline"]["zero_inputs"] = zero_inputs
    if "fp8" in ms:
        f = prefill_flops(2, 16, 8192, 128, True)
        tf = f / (ms["fp8"] * 1e-3) / 1e12
        result["fp8"] = {"value": tf, "unit": "TFLOP/s", "launch_ms": ms["fp8"],
                         "launch_ms_spread": spread("fp8"),
                         "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP8_TFLOPS,
                                      "unit": "TFLOP/s", "frac": tf / PEAK_FP8_TFLOPS,
                                      "traffic": measured_traffic("pmc_fwd_prefill_fp8_causal_B2H16N8192d128.md"),
                                      "kernel": "fwd_kernel3<128,causal,fp8>"}}
    if "decode" in ms:
        ub, lb = decode_bytes(p5)
        gbs = ub / (ms["decode"] * 1e-3) / 1e9
        result["decode"] = {"value": gbs, "unit": "GB/s", "launch_ms": ms["decode"],
                            "launch_ms_spread": spread("decode"),
                            "bytes_unique": ub, "bytes_logical": lb,
                            "logical_GBps": lb / (ms["decode"] * 1e-3) / 1e9,
                            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                         "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                         "traffic": measured_traffic("pmc_paged_decode_S64H32d128.md"),
                                         "kernel": "decode_plan/pair + decode_split + decode_pair_split "
                                                   "+ decode_merge kernels"}}
        if read_probe:
            result["decode"]["roofline"]["read_probe"] = read_probe
            result["decode"]["roofline"]["frac_of_read_probe"] = gbs / read_probe["GBps"]
    if "backward" in ms:
        f = 2.5 * prefill_flops(1, 32, 16384, 128, True)
        tf = f / (ms["backward"] * 1e-3) / 1e12
        result["backward"] = {"value": tf, "unit": "TFLOP/s", "launch_ms": ms["backward"],
                              "launch_ms_spread": spread("backward"), "flop_per_launch": f,
                              "workload": "causal bf16 backward B1 H32 N16384 d128",
                              "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                                           "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                                           "traffic": measured_traffic("pmc_bwd_causal_B1H32N16384d128.md"),
                                           "kernel": "bwd_dot + bwd_dkdv + bwd_dq kernels"}}
    if "paged_prefill" in ms:
        n_new = p6.q.shape[2]
        ctx = p6.ctx_lens.cpu().double()
        # sum over sequences and new tokens of 4 d (position + 1), times heads
        keys = (n_new * (ctx - n_new) + n_new * (n_new + 1) / 2).sum().item()
        f = 4.0 * 128 * 32 * keys
        tf = f / (ms["paged_prefill"] * 1e-3) / 1e12
        result["paged_prefill"] = {"value": tf, "unit": "TFLOP/s", "launch_ms": ms["paged_prefill"],
                                   "launch_ms_spread": spread("paged_prefill"), "flop_per_launch": f,
                                   "workload": "paged chunked prefill S16 H32 d128, last 2048 tokens of "
                                               "contexts 2048..16384",
                                   "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                                                "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                                                "traffic": measured_traffic("pmc_paged_prefill_S16H32d128.md"),
                                                "kernel": "fwd_kernel3<128,causal,bf16,paged>"}}
    if "block_sparse" in ms:
        nb = bmask.shape[0]
        keep = bmask.numpy().astype(bool)
        # visible (query, key) pairs: full off-diagonal kept blocks + causal diagonal blocks
        i, j = np.nonzero(keep)
        pairs = float(((i > j).sum()) * 128 * 128 + (i == j).sum() * 128 * 129 / 2)
        f = 4.0 * 128 * 32 * pairs
        for name in ("block_sparse", "block_sparse_dropout"):
            tf = f / (ms[name] * 1e-3) / 1e12
            result[name] = {"value": tf, "unit": "TFLOP/s", "launch_ms": ms[name],
                            "launch_ms_spread": spread(name), "flop_per_launch": f,
                            "workload": "block-sparse causal B1 H32 N16384 d128, %d of %d causal blocks kept%s"
                                        % (int(keep.sum()), nb * (nb + 1) // 2,
                                           ", dropout 0.1" if name.endswith("dropout") else ""),
                            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                                         "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                                         "traffic": measured_traffic("pmc_block_sparse_B1H32N16384d128.md"),
                                         "kernel": "sparse_fwd_kernel"}}
    if "fp8_quantize" in ms:
        tokens = 3 * 2 * 16 * 8192                              # Q, K and V
        nbytes = tokens * 128 * (2 + 1) + 3 * 2 * 16 * 64 * 4  # bf16 in, E4M3 out, scales
        per_launch = ms["fp8_quantize"]
        gbs = nbytes / (per_launch * 1e-3) / 1e9
        result["fp8_quantize"] = {"value": tokens / (per_launch * 1e-3), "unit": "tokens/s",
                                  "launch_ms": per_launch, "launch_ms_spread": spread("fp8_quantize"),
                                  "bytes_per_launch": nbytes,
                                  "workload": "rotate + E4M3 block quantise Q, K (Haar R) and V (no R), "
                                              "B2 H16 N8192 d128 each, one launch (fa_quantize_fp8_qkv)",
                                  "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                               "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                               "traffic": measured_traffic("pmc_fp8_quantize_B2H16N8192d128.md"),
                                               "kernel": "fp8_quant_kernel"}}
    if "mha" in ms:
        f = prefill_flops(4, 16, 2048, 64, False)
        tf = f / (ms["mha"] * 1e-3) / 1e12
        result["mha"] = {"value": tf, "unit": "TFLOP/s", "launch_ms": ms["mha"], "launch_ms_spread": spread("mha"),
                         "flop_per_launch": f, "workload": "non-causal bf16 MHA B4 H16 N2048 d64",
                         "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                      "frac": tf / PEAK_BF16_TFLOPS,
                                      "traffic": measured_traffic("pmc_fwd_mha_bf16_B4H16N2048d64.md"),
                                      "kernel": "fwd_kernel3<64,non-causal,bf16>"}}
    if result["value"] is None and "decode" in result:
        result["value"], result["unit"] = result["decode"]["value"], "GB/s"
    if not args.no_cpu_baseline and "prefill" in only:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(x3, args.cpu_budget)
    if not args.no_cpu_baseline and "decode" in only:
        log("cpu baseline (oracle paged decode)")
        result["decode"]["cpu_baseline"] = decode_cpu_baseline(p5, args.cpu_budget / 2)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
