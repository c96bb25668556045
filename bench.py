"""Paged-attention benchmark on one MI355X.

Headline workload: Llama-style GQA decode -- batch 64, 32 query / 8 KV heads,
head_dim 128, bf16 K/V, block size 16, contexts uniform in [1, 8192]
(seeded), random block tables over a 40000-block pool.  One step is the whole
hot path for one new token per sequence: slot mapping and the K/V write of
the new token (one fused launch), and the partitioned decode kernel (whose last partition of each
sequence and KV head does the log-sum-exp merge), all through libpa.so on torch's current stream, with every input already
resident in HBM.  Before the warm-up steps, 50 ms of a read stream over a
buffer of its own brings the GPU to its steady clocks, and between the
synchronisation that opens the timed region and its start event one more
untimed read (~80 us) lets the host queue the first timed step before the GPU
reaches it (both reported in the line).

Printed: one JSON line with whole-step throughput (K/V bytes read per
second), the decode call's roofline (K/V bytes / decode kernel time against
8 TB/s, timed with events over the timed region), the split the decode ran
(workgroups, slice length, pieces per pair), the CPU oracle timed on one
whole step of the same workload, and secondary measurements of the
batched causal prefill (TFLOP/s against 2.5 PFLOP/s bf16), of the
long-context shared-prefix decode, of the copy-on-write block copy and of
the block swap between the device pool and a pinned host pool, the fp32
prefill on GPT-2 shapes (against the fp32 matrix peak), and the decode step
in one launch (pa_decode_step) against the two-launch step.

    python bench.py [--gpus 1] [--steps 200] [--warmup 200]
    python bench.py --calibrate-copy     # plain 1 GiB copies, for counter scaling
    python bench.py --prefill-only       # the batched prefill alone, for its counters
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PCIE5_X16_GBPS = 63.0   # 32 GT/s x 16 lanes, 128b/130b coding, one direction
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
F32_MFMA_PEAK_TFLOPS = 157.3
METRIC = "paged-attn decode μs/step + KV-read HBM GB/s (% of peak), batch 64 ctx 4096"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--partition-size", type=int, default=1024)
    p.add_argument("--layout", default="token",
                   help="pool layout of the headline decode (token, head, unified_token, "
                        "unified_head, layers_token, layers_head)")
    p.add_argument("--cpu-runs", type=int, default=3,
                   help="timed runs of the CPU oracle step (the median is reported)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    p.add_argument("--no-secondary", action="store_true",
                   help="skip the prefill and long-context measurements")
    p.add_argument("--fixed-context", type=int, default=None,
                   help="every context at this length instead of uniform [1, 8192]")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run plain device copies of 1 GiB (HBM counter calibration)")
    p.add_argument("--prefill-only", action="store_true",
                   help="only run the batched prefill (for its matrix-core counters)")
    return p.parse_args()


DECODE_SOURCES = ("decode.hip", "pa_device.h", "pa_internal.h")


def code_text(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed: what the
    compiler sees, so an edit of a comment keeps the decode's hash."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(read=None) -> str:
    """Hash of the decode kernel's sources (the kernel, the device helpers
    and the plan it shares with the host), comments and layout ignored."""
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        if read is None:
            with open(os.path.join(ROOT, "paged_kv_cache_87_amd", "csrc", name)) as f:
                text = f.read()
        else:
            text = read(name)
        h.update(code_text(text).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload_name: str, partition_size: int):
    """HBM bytes per decode call from committed rocprofv3 counter runs, if
    they were taken on the current decode source; else None."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    if rec.get("workload") != workload_name or rec.get("partition_size") != partition_size:
        return None
    return rec.get("bytes_per_call")


def cpu_baseline(w, runs: int = 3):
    """The oracle as it stands, on the host cores: one whole step of the
    headline workload -- the K/V write of the 64 new tokens, then the decode
    of every sequence -- with the sequences spread over a thread pool (one
    sequence per task, longest first, numpy's own BLAS held to one thread per
    worker).  The pre-step history is written into the pools untimed; the
    step is timed `runs` times and the median taken."""
    import concurrent.futures as cf
    import statistics

    from oracle import run as orun
    import oracle.paged_attention as orc

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # threadpoolctl absent: BLAS keeps its own thread count
        threadpool_limits = None
    k_cache, v_cache = orun.build_pools(w)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    order = sorted(range(w.num_seqs), key=lambda s: -int(w.context_lens[s]))

    def one(s):
        return orc.decode(w.q[s:s + 1], k_cache, v_cache, w.block_tables[s:s + 1],
                          w.context_lens[s:s + 1], w.scale, w.dtype)

    times = []
    limit = threadpool_limits(1) if threadpool_limits is not None else None
    try:
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            for _ in range(runs):
                t0 = time.perf_counter()
                orun.write_step(w, k_cache, v_cache)
                list(ex.map(one, order))
                times.append(time.perf_counter() - t0)
    finally:
        if limit is not None:
            limit.unregister()
    step_s = statistics.median(times)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    kv_bytes = w.kv_bytes_read()
    return {
        "value": kv_bytes / step_s / 1e9,
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"the whole step of this workload (write of {w.num_seqs} new tokens, decode of "
                  f"{w.num_seqs} sequences, {kv_bytes / 1e9:.3f} GB of K/V), median of {runs} runs "
                  f"({', '.join(f'{t:.2f}' for t in times)} s), numpy float64 over a pool of "
                  f"{workers} threads, BLAS at 1 thread each; host CPU {model!r}, "
                  f"{len(os.sched_getaffinity(0))} cores visible",
        "us_per_step": step_s * 1e6,
    }


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """Timing-only HIP events on a stream, created with
    hipEventDisableSystemFence: recording one does not write back and
    invalidate the caches, so bracketing every call costs ~1.5 us per event
    less than torch's events (which use the system-scope fence) and does not
    slow the next kernel.  The HIP runtime is the one torch already loaded."""

    def __init__(self, torch):
        torch.cuda.init()
        path = next(line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line)
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.live = []

    def _check(self, rc, what):
        if rc != 0:
            self.hip.hipGetLastError()
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def new(self):
        ev = ctypes.c_void_p()
        self._check(self.hip.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE),
                    "hipEventCreateWithFlags")
        self.live.append(ev)
        return ev

    def record(self, ev, stream):
        self._check(self.hip.hipEventRecord(ev, ctypes.c_void_p(stream.cuda_stream)), "hipEventRecord")

    def ms(self, a, b):
        out = ctypes.c_float()
        self._check(self.hip.hipEventElapsedTime(ctypes.byref(out), a, b), "hipEventElapsedTime")
        return out.value

    def free(self):
        for ev in self.live:
            self.hip.hipEventDestroy(ev)
        self.live = []


_EVENTS = None


LEAD_BYTES = 512 << 20
_LEAD = None


def gpu_lead(torch, stream):
    """One untimed read of LEAD_BYTES of a buffer of its own (the library's
    read probe, ~80 us), enqueued after the synchronisation that opens a timed
    region and before its start event.  While it runs, the host queues the
    first timed iteration, so that the GPU does not reach that iteration's
    body before the host has launched it: without the lead, the first timed
    decode call's events also hold the ~20 us the host takes to launch it.
    Nothing of the timed workload is touched."""
    global _LEAD
    from paged_kv_cache_87_amd import binding
    if _LEAD is None:
        _LEAD = (torch.ones(LEAD_BYTES // 4, dtype=torch.float32, device="cuda"),
                 torch.zeros(4096, dtype=torch.int32, device="cuda"))
    binding.pa_read_checksum(_LEAD[0], _LEAD[1], stream)


# Timing-only events bracket the body of every EVENT_STRIDE-th timed
# iteration (0, 2, 4, ...): a bracketed step costs ~4 us more than a bare one
# on the batch-64 decode (two event packets between its kernels), so
# bracketing every step would slow the very steps whose rate is reported.
EVENT_STRIDE = 2


def timed(torch, stream, K, W, prefix, body, suffix=None, settle=False):
    """Run W untimed then K timed iterations; each iteration is prefix(),
    body(), suffix(), the body of every EVENT_STRIDE-th one bracketed by
    timing-only events.  With settle, the GPU first runs gpu_settle (steady
    clocks).  The timed region opens with a synchronisation and the untimed
    gpu_lead, then the start event.  Returns (total ms / K, [ms of each
    bracketed body])."""
    global _EVENTS
    if _EVENTS is None:
        _EVENTS = HipEvents(torch)
    E = _EVENTS
    # the timed region's events exist before the warm-up, so that no host work
    # sits between the synchronisation and the first timed step
    ev = [[E.new() for _ in range(2)] for _ in range(0, K, EVENT_STRIDE)]
    start, stop = E.new(), E.new()
    if settle:
        gpu_settle(torch, stream)
    for _ in range(W):
        prefix()
        body()
        if suffix:
            suffix()
    gpu_lead(torch, stream)          # allocates its buffer on first use, outside the region
    torch.cuda.synchronize()
    gpu_lead(torch, stream)
    E.record(start, stream)
    for i in range(K):
        prefix()
        if i % EVENT_STRIDE == 0:
            E.record(ev[i // EVENT_STRIDE][0], stream)
            body()
            E.record(ev[i // EVENT_STRIDE][1], stream)
        else:
            body()
        if suffix:
            suffix()
    E.record(stop, stream)
    torch.cuda.synchronize()
    res = E.ms(start, stop) / K, [E.ms(a, b) for a, b in ev]
    E.free()
    return res


SETTLE_MS = 50.0


def gpu_settle(torch, stream, ms: float = SETTLE_MS) -> int:
    """Bring the GPU to its steady clocks before a timed region: `ms` of an
    unrelated read stream (the library's read probe over a 256 MiB buffer of
    its own, so none of the timed workload's data is touched or left in a
    cache).  From idle the clocks need a few tens of milliseconds of load to
    ramp: without this, a warm-up of a few steps leaves the first ~50 decode
    calls ~3 % slower than the steady state.  Returns the probe calls run."""
    from paged_kv_cache_87_amd import binding
    buf = torch.ones(1 << 26, dtype=torch.float32, device="cuda")
    words = torch.zeros(4096, dtype=torch.int32, device="cuda")
    calls = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            binding.pa_read_checksum(buf, words, stream)
        torch.cuda.synchronize()
        calls += 10
    del buf, words
    return calls


def secondary(torch, np, stream, K, W, partition_size):
    from paged_kv_cache_87_amd import runner
    from paged_kv_cache_87_amd import workloads as wl

    out = {}
    # the headline decode on each block layout of the pool, same timing
    out["decode_layouts"] = {}
    for layout in ("token", "head", "unified_head"):
        w = wl.llama_gqa_decode(pool_fill="zero", partition_size=partition_size)
        g = runner.GpuStep(w, layout=layout)
        g.write_history()
        _, dec_ms = timed(torch, stream, K, W, g.append, g.attend, settle=True)
        dec = float(np.mean(dec_ms))
        out["decode_layouts"][layout] = {
            "decode_us": dec * 1e3, "kv_GBps": w.kv_bytes_read() / (dec * 1e-3) / 1e9,
            "frac_hbm_peak": w.kv_bytes_read() / (dec * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        del g
        torch.cuda.empty_cache()
    # the decode step in one launch (pa_decode_step) against the two-launch
    # step (pa_append_kv, then pa_decode), on the headline batch and on one
    # sequence of 4096 tokens (partition 256), where launches weigh most
    out["decode_step_fused"] = {}
    for name, w in (("batch64", wl.llama_gqa_decode(pool_fill="zero",
                                                    partition_size=partition_size)),
                    ("batch1_ctx4096", wl.decode_workload(
                        "gqa_b1", 87006, dtype=wl.BF16, num_q_heads=32, num_kv_heads=8,
                        head_dim=128, block_size=16, num_blocks=400, context_lens=[4096],
                        partition_size=256, pool_fill="zero"))):
        g = runner.GpuStep(w)
        g.write_history()
        two_ms, _ = timed(torch, stream, K, W, g.append, g.attend, settle=True)
        one_ms, _ = timed(torch, stream, K, W, lambda: None, g.decode_step, settle=True)
        out["decode_step_fused"][name] = {"two_launches_us_per_step": two_ms * 1e3,
                                          "one_launch_us_per_step": one_ms * 1e3}
        del g
        torch.cuda.empty_cache()
    # batched causal prefill: slot mapping + write of every prompt token + prefill
    w = wl.batched_prefill(pool_fill="zero")
    g = runner.GpuStep(w)
    g.write_history()
    step_ms, pre_ms = timed(torch, stream, K, W, lambda: (g.slot_mapping(), g.write()), g.attend,
                            settle=True)
    lens = w.context_lens.astype(np.int64)
    flops = 2.0 * w.num_q_heads * w.head_dim * float(np.sum(lens * (lens + 1)))
    pre = float(np.mean(pre_ms))
    out["batched_prefill"] = {
        "config": {"batch": w.num_seqs, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "prompt_lens": "uniform [256, 2048], seed 87004",
                   "total_tokens": int(lens.sum())},
        "us_per_step": step_ms * 1e3, "prefill_us": pre * 1e3,
        "flops": flops, "tflops": flops / (pre * 1e-3) / 1e12,
        "frac_bf16_peak": flops / (pre * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
    }
    del g
    torch.cuda.empty_cache()
    # the fp32 prefill on GPT-2-shaped prompts: 12 heads of 64 (MHA), 16 prompts
    # U[256, 2048], on the fp32 matrix cores
    rng = np.random.default_rng(87007)
    plens = [int(x) for x in rng.integers(256, 2049, size=16)]
    w = wl.prefill_workload("gpt2_prefill_f32", 87007, dtype=wl.F32, num_q_heads=12,
                            num_kv_heads=12, head_dim=64, block_size=16,
                            num_blocks=sum((x + 15) // 16 for x in plens) + 16,
                            context_lens=plens, pool_fill="zero")
    g = runner.GpuStep(w)
    g.write_history()
    step_ms, pre_ms = timed(torch, stream, K, W, lambda: (g.slot_mapping(), g.write()), g.attend,
                            settle=True)
    lens = w.context_lens.astype(np.int64)
    flops = 2.0 * w.num_q_heads * w.head_dim * float(np.sum(lens * (lens + 1)))
    pre = float(np.mean(pre_ms))
    out["batched_prefill_f32"] = {
        "config": {"batch": w.num_seqs, "num_q_heads": 12, "num_kv_heads": 12, "head_dim": 64,
                   "prompt_lens": "uniform [256, 2048], seed 87007",
                   "total_tokens": int(lens.sum())},
        "us_per_step": step_ms * 1e3, "prefill_us": pre * 1e3, "flops": flops,
        "tflops": flops / (pre * 1e-3) / 1e12,
        "frac_f32_mfma_peak": flops / (pre * 1e-3) / 1e12 / F32_MFMA_PEAK_TFLOPS,
    }
    del g
    torch.cuda.empty_cache()
    # long-context decode over a copy-on-write shared prefix, partition 512
    w = wl.long_context_cow(pool_fill="zero")
    g = runner.GpuStep(w)
    g.write_history()
    from paged_kv_cache_87_amd import binding as _b
    lc_split = _b.pa_decode_split_info(g.pool, g.seqs, w.num_q_heads, w.partition_size)
    step_ms, dec_ms = timed(torch, stream, K, W, g.append, g.attend, settle=True)
    dec = float(np.mean(dec_ms))
    logical = w.kv_bytes_read()
    prefix = w.meta["shared_prefix_tokens"]
    unique = logical - (w.num_seqs - 1) * prefix * 2 * w.num_kv_heads * w.head_dim * 2
    out["long_context_cow"] = {
        "config": {"batch": w.num_seqs, "context": int(w.context_lens[0]), "shared_prefix": prefix,
                   "partition_size": w.partition_size, "decode_split": lc_split},
        "us_per_step": step_ms * 1e3, "decode_us": dec * 1e3,
        "logical_kv_GBps": logical / (dec * 1e-3) / 1e9,
        "unique_kv_GBps": unique / (dec * 1e-3) / 1e9,
        "frac_hbm_peak_unique": unique / (dec * 1e-3) / 1e9 / HBM_PEAK_GBPS,
    }
    del g
    torch.cuda.empty_cache()
    # copy-on-write data move: 2048 disjoint block pairs of a 40000-block
    # 8 x 128 bf16 pool (32 KiB per block and pool), K and V
    from paged_kv_cache_87_amd import binding
    nb, pairs = 40000, 2048
    kc = torch.zeros((nb, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    pool = binding.KVPool(kc, vc)
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(87005))
    src = perm[:pairs].to(torch.int32).cuda()
    dst = perm[pairs:2 * pairs].to(torch.int32).cuda()
    _, cp_ms = timed(torch, stream, K, W, lambda: None,
                     lambda: binding.pa_copy_blocks(pool, src, dst), settle=True)
    cp = float(np.mean(cp_ms))
    moved = 2 * 2 * pairs * 16 * 8 * 128 * 2          # read + write, K and V
    out["cow_copy_blocks"] = {
        "config": {"pairs": pairs, "block_bytes_per_pool": 16 * 8 * 128 * 2},
        "copy_us": cp * 1e3, "hbm_GBps": moved / (cp * 1e-3) / 1e9,
        "frac_hbm_peak": moved / (cp * 1e-3) / 1e9 / HBM_PEAK_GBPS,
    }
    # offload tier: the same 2048 blocks swapped out to a pinned host pool and
    # back, against a plain contiguous host<->device copy of the same bytes
    hk = torch.zeros((4096, 16, 8, 128), dtype=torch.bfloat16).pin_memory()
    hv = torch.zeros_like(hk).pin_memory()
    hsl = torch.randperm(4096, generator=torch.Generator().manual_seed(87006))[:pairs]
    hsl = hsl.to(torch.int32).cuda()
    _, out_ms = timed(torch, stream, K, W, lambda: None, lambda: binding.pa_swap_blocks(
        pool, hk, hv, src, hsl, binding.PA_SWAP_OUT))
    _, in_ms = timed(torch, stream, K, W, lambda: None, lambda: binding.pa_swap_blocks(
        pool, hk, hv, dst, hsl, binding.PA_SWAP_IN))
    link = 2 * pairs * 16 * 8 * 128 * 2                # K and V, one way
    flat_h = hk.view(-1)[:link // 2]
    flat_d = kc.view(-1)[:link // 2]
    _, d2h_ms = timed(torch, stream, K, W, lambda: None,
                      lambda: flat_h.copy_(flat_d, non_blocking=True))
    _, h2d_ms = timed(torch, stream, K, W, lambda: None,
                      lambda: flat_d.copy_(flat_h, non_blocking=True))
    gbps = lambda ms, b: b / (float(np.mean(ms)) * 1e-3) / 1e9  # noqa: E731
    out["swap_blocks"] = {
        "config": {"pairs": pairs, "bytes_each_way": link, "host_pool_blocks": 4096},
        "swap_out_us": float(np.mean(out_ms)) * 1e3, "swap_in_us": float(np.mean(in_ms)) * 1e3,
        "swap_out_GBps": gbps(out_ms, link), "swap_in_GBps": gbps(in_ms, link),
        "contiguous_d2h_GBps": gbps(d2h_ms, link // 2),
        "contiguous_h2d_GBps": gbps(h2d_ms, link // 2),
        "pcie5_x16_peak_GBps": PCIE5_X16_GBPS,
    }
    del hk, hv
    # context for the HBM fraction: a plain 1 GiB device copy (1 GiB read + 1 GiB
    # written) through Tensor.copy_, the ceiling a streaming kernel meets here
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    _, cp_ms = timed(torch, stream, K, W, lambda: None, lambda: b.copy_(a), settle=True)
    out["hbm_copy_ceiling"] = {"bytes_moved": 2 << 30,
                               "GBps": (2 << 30) / (float(np.mean(cp_ms)) * 1e-3) / 1e9}
    out["hbm_copy_ceiling"]["frac_hbm_peak"] = out["hbm_copy_ceiling"]["GBps"] / HBM_PEAK_GBPS
    del b
    # and a plain read stream over the same 1 GiB: the library's read probe
    # (non-temporal 16-byte loads, the decode's load kind; one checksum word per
    # workgroup), the practical ceiling of a read-once kernel such as the decode
    words = torch.zeros(8192, dtype=torch.int32, device="cuda")
    _, rd_ms = timed(torch, stream, K, W, lambda: None,
                     lambda: binding.pa_read_checksum(a, words, stream), settle=True)
    out["hbm_read_ceiling"] = {"bytes_read": 1 << 30, "kernel": "pa_read_checksum, 8192 workgroups",
                               "GBps": (1 << 30) / (float(np.mean(rd_ms)) * 1e-3) / 1e9}
    out["hbm_read_ceiling"]["frac_hbm_peak"] = out["hbm_read_ceiling"]["GBps"] / HBM_PEAK_GBPS
    del a, words
    return out


def calibrate_copy(torch):
    """Plain device-to-device copies of 1 GiB: 1 GiB read and 1 GiB written per
    copy kernel, the reference for scaling the HBM byte counters."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode path shards by sequence or KV head with no exchange; "
              "this benchmark runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from paged_kv_cache_87_amd import binding, runner
    from paged_kv_cache_87_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.load_library()
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    if args.prefill_only:
        w = wl.batched_prefill(pool_fill="zero")
        g = runner.GpuStep(w)
        g.write_history()
        g.slot_mapping()
        g.write()
        _, pre_ms = timed(torch, torch.cuda.current_stream(), args.steps, args.warmup,
                          lambda: None, g.attend)
        lens = w.context_lens.astype(np.int64)
        flops = 2.0 * w.num_q_heads * w.head_dim * float(np.sum(lens * (lens + 1)))
        print(json.dumps({"prefill_us": float(np.mean(pre_ms)) * 1e3, "flops": flops,
                          "tflops": flops / (float(np.mean(pre_ms)) * 1e-3) / 1e12}), flush=True)
        return

    w = wl.llama_gqa_decode(pool_fill="zero", partition_size=args.partition_size,
                            fixed_context=args.fixed_context)
    g = runner.GpuStep(w, layout=args.layout)
    g.write_history()
    kv_bytes = w.kv_bytes_read()
    stream = torch.cuda.current_stream()

    split = binding.pa_decode_split_info(g.pool, g.seqs, w.num_q_heads, args.partition_size)
    K = args.steps
    settle_calls = gpu_settle(torch, stream)
    step_ms, decode_ms = timed(torch, stream, K, args.warmup, g.append, g.attend)
    dec_avg_ms = float(np.mean(decode_ms))
    achieved = kv_bytes / (dec_avg_ms * 1e-3) / 1e9
    sum_ctx = int(w.context_lens.astype(np.int64).sum())
    del g
    torch.cuda.empty_cache()

    sec = None if args.no_secondary else secondary(torch, np, stream, max(10, K // 5), 30,
                                                       args.partition_size)
    cpu = None if args.no_cpu else cpu_baseline(w, args.cpu_runs)

    traffic = measured_traffic(w.name, args.partition_size) if args.layout == "token" else None
    rec = {
        "metric": METRIC,
        "value": kv_bytes / (step_ms * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "us_per_step": step_ms * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": w.num_seqs,
            "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "num_blocks": w.num_blocks,
            "context_lens": ("fixed %d" % args.fixed_context) if args.fixed_context
            else "uniform [1, 8192], seed 87003",
            "sum_context_tokens": sum_ctx,
            "kv_bytes_per_step": kv_bytes,
            "partition_size": args.partition_size,
            "decode_split": split,
            "pool_layout": args.layout,
        },
        "decode_us": {"mean": dec_avg_ms * 1e3, "p10": float(np.percentile(decode_ms, 10)) * 1e3,
                      "p50": float(np.percentile(decode_ms, 50)) * 1e3,
                      "p90": float(np.percentile(decode_ms, 90)) * 1e3,
                      "calls_bracketed": len(decode_ms),
                      "bracketing": f"timing-only HIP events around timed calls 0, {EVENT_STRIDE}, "
                                    f"{2 * EVENT_STRIDE}, ... on the launch stream"},
        "roofline": {
            "kernel": "pa_decode (persistent partition kernel, log-sum-exp merge fused)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
        },
        "gpu_settle": {"ms": SETTLE_MS, "kernel": "pa_read_checksum over 256 MiB of its own",
                       "calls": settle_calls, "why": "steady clocks before the W warm-up steps"},
        "gpu_lead": {"kernel": f"pa_read_checksum over {LEAD_BYTES >> 20} MiB of its own, once",
                     "where": "after the synchronisation that opens the timed region, before its "
                              "start event (untimed)",
                     "why": "the host queues the first timed step while it runs, so the first "
                            "decode call's events do not hold the host's launch latency"},
        "cpu_baseline": cpu,
        "secondary": sec,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
