"""Benchmark of the paged-KV-cache attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

Default workload (the headline): the Llama-3-8B-shaped decode step -- 40
sequences, 32 query and 8 kv heads of 128, bf16 cache in 16-token blocks
behind shuffled block tables, context lengths uniform in [512, 4096].  One
step is one pass of the decode hot path over that batch: grow every sequence
by one token and append its new K/V rows (kvc_seq_grow_append: the host
allocator places each row, one launch writes the rows and the table and
length updates), then kvc_attn_decode (work-list partials and their (m, l)
merge).  The headline `value` is the decode's algorithmic HBM bytes per step
(K/V rows read through the tables, queries, outputs, table entries) divided
by the wall-clock time per step.

The same JSON line carries one object per other workload, each with its own
`roofline` (and, where the oracle is timed, `cpu_baseline`):
  prefill               causal prefill, 4 x 8,192 tokens, 32/8 heads of 128,
                        bf16, K/V appended to the cache (TFLOP/s)
  decode_llama70b_bf16  8 x 32,768-token contexts, 64/8 heads, bf16 cache
  decode_llama70b_fp8   the same rows on an fp8-e4m3 cache with block scales
  decode_long_mha       one 128,000-token context, 32/32 heads, fp16 cache
  decode_int4           the 70B-shaped rows on an int4 cache
  extend                chunked prefill: the last 512-token chunk of the
                        prefill prompts against the 7,680 rows cached before
  decode_window         the headline batch under a 1,024-row window + 4 sinks
  prefix_share          40 sequences sharing a 600-token prompt

`roofline` is the dominant kernel of each workload: its algorithmic bytes
(or FLOPs) over its duration, timed by HIP dispatch events attached to that
kernel (kvc_set_dispatch_events), as a kernel trace times it.  Decode: the
work-list kernel of the same call repeated K times after the timed steps,
each launch preceded by a read of a separate 1 GiB buffer that evicts the
Infinity Cache.  Prefill and extend: the attention kernel.  Beside it,
`roofline.call` gives the whole library call: for decode the work-list
kernel, the merge and the gap between them (first kernel start to last
kernel end) and the same calls timed by stream markers; for prefill and
extend the stream-marker time of up to 10 single calls after the timed ones.
The K timed steps carry no markers of their own (a marker in the stream
leaves a gap beside the kernels it brackets).  `traffic` is the HBM
bytes per launch of the dominant kernel (in `call`: of every kernel of the
call) that rocprofv3's
FETCH_SIZE / WRITE_SIZE counters recorded (profiles/counters.json, scaled by
a copy-kernel calibration), reported only while the kernel sources are
unchanged since that measurement.  `cpu_baseline` times the float64 oracle
on a bounded sample of the same workload on this host's cores.  Inputs are
synthetic and seeded.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
METRIC = "decode attn HBM GB/s (% of peak) + prefill attn TFLOP/s (% MFMA peak)"


def cpu_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count()


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 0) for p in threadpool_info()] or [0])
    except Exception:
        return None


# ---------------------------------------------------------------- counters
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SOURCES = ["mfma_decode.hip", "decode.hip", "mfma_prefill.hip", "prefill.hip",
                  "cache_kernels.hip", "common.h", "fp8_e4m3.h", "kvfa_internal.h"]


def kernel_source_digest():
    """sha256 over the device sources, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "kv_cache_flashattention_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def counter_traffic(key, kernel=None):
    """HBM bytes per call from rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded
    in profiles/counters.json, scaled by the copy-kernel calibration factors
    (with `kernel`: only the kernels whose names start with it); None unless
    the kernels are byte-identical in source to those measured."""
    try:
        with open(COUNTERS) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    e = rec.get("workloads", {}).get(key)
    if e is None or rec.get("kernel_source_sha256") != kernel_source_digest():
        return None
    cal = rec["calibration"]
    if kernel is None:
        fetch, write = e["fetch_kib_per_call"], e["write_kib_per_call"]
    else:
        ks = [v for n, v in e["kernels"].items() if n.startswith(kernel)]
        if not ks:
            return None
        fetch, write = sum(v["fetch_kib"] for v in ks), sum(v["write_kib"] for v in ks)
    return fetch * 1024 * cal["fetch_factor"] + write * 1024 * cal["write_factor"]


_T0 = time.perf_counter()


def log(msg):
    """Progress line on stderr (the JSON result goes alone to stdout)."""
    print(f"[bench {time.perf_counter() - _T0:6.1f} s] {msg}", file=sys.stderr, flush=True)


def warm_up_clocks(call, torch, seconds=0.05):
    """Repeat `call` (untimed) for at least `seconds` of GPU time.  From idle
    the GPU needs some tens of milliseconds of load before its clocks settle:
    the 4 x 8,192 prefill takes ~3.4 ms on its first call and ~2.3 ms from
    about the tenth on, so timing right after a short warm-up measures the
    ramp rather than the kernel."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            call()
        torch.cuda.synchronize()


# ---------------------------------------------------------------- decode
# Source rows of the decode workloads, rounded to the io type on the host,
# kept for the run: the three 70B-shaped legs (bf16, fp8 and int4 caches)
# read the same rows, and the CPU baseline takes its float64 inputs from them.
_ROWS = {}


def source_rows(w, b, torch, io):
    """All L_b rows of sequence b of workload w, as host tensors of the io
    type [L, n_kv, d] (drawn once per (rows tag, sequence))."""
    key = (w.tag, w.seed, b, str(io))
    if key not in _ROWS:
        L = int(w.lengths[b])
        ks, vs = [], []
        for s0 in range(0, L, 8192):
            k, v = w.kv_rows(b, s0, min(8192, L - s0))
            ks.append(torch.from_numpy(k).to(io))
            vs.append(torch.from_numpy(v).to(io))
        _ROWS[key] = (torch.cat(ks), torch.cat(vs))
    return _ROWS[key]


def drop_rows(tag):
    for key in [k for k in _ROWS if k[0] == tag]:
        del _ROWS[key]


def build_decode(name, torch, kv, grow=112):
    """The workload's cache, with room for every sequence to grow by `grow`
    more tokens."""
    from workloads import decode_workload
    w = decode_workload(name)
    dt = {"bf16": "bf16", "fp16": "f16", "fp8": "fp8", "int4": "int4"}[w.kv_dtype]
    io = kv.IO_TORCH[dt]
    room = -(-grow // 16) + 1                              # blocks per sequence to grow into
    spare = w.batch * room
    max_bps = int(w.blocks_per_seq.max()) + room
    c = kv.KvCache(1, w.n_q, w.n_kv, w.d, w.n_blocks + spare, w.batch, max_bps, dt)
    tables = w.block_tables()
    for b in range(w.batch):
        c.set_block_table(b, tables[b], int(w.lengths[b]))
    for b in range(w.batch):
        K, V = source_rows(w, b, torch, io)
        sel = torch.tensor([b], dtype=torch.int32, device="cuda")
        for s0 in range(0, K.shape[0], 8192):
            n = min(8192, K.shape[0] - s0)
            c.write(0, sel, s0, K[s0:s0 + n].cuda()[None], V[s0:s0 + n].cuda()[None])
    torch.cuda.synchronize()
    return w, c, io


KV_ELEM_BYTES = {"bf16": 2, "fp16": 2, "fp8": 1, "int4": 0.5}


def decode_bytes(w, lengths, kv_elem):
    """Algorithmic HBM bytes of one decode call: every valid K and V row once
    (per kv head), the query and output rows, one table entry per block, and
    for fp8 and int4 the two scales per block and kv head.  kv_elem: bytes per
    stored element (0.5 for int4)."""
    rows = int(np.sum(lengths))
    kvb = int(2 * rows * w.n_kv * w.d * kv_elem)
    qo = 2 * w.batch * w.n_q * w.d * 2
    blocks = int(np.sum(-(-np.asarray(lengths) // 16)))
    tab = blocks * 4
    sc = 2 * blocks * w.n_kv * 4 if kv_elem < 2 else 0
    return kvb + qo + tab + sc


def window_rows(L, window, sinks):
    """Rows a decode query at position L-1 sees under a sliding window of
    `window` rows plus `sinks` sink rows, and the blocks holding them."""
    if window <= 0 or L <= window:
        pos = np.arange(L)
    else:
        pos = np.r_[0:min(sinks, L - window), L - window:L]
    return len(pos), len(np.unique(pos // 16))


def evict_and_time(call, steps, torch, cache):
    """Mean times (s) of `call`, a decode on `cache`, over `steps` launches on
    the current stream, each launch preceded by a full read of a separate
    1 GiB buffer: the read evicts the 256 MB Infinity Cache without leaving
    dirty lines, so the call's K/V bytes all come from HBM.  Three passes:
    dispatch events on the call's main kernel (the work-list kernel), dispatch
    events from the call's first kernel's start to its last kernel's end
    (kvc_set_dispatch_events), and stream markers recorded before and after
    the call with the hook unset (its events add packets of their own to the
    stream).  Returns (kernel, call, markers)."""
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for e in ev:
        for x in e[:4]:
            x.record(stream)                          # creates the events the hook takes
    torch.cuda.synchronize()
    for main, (i0, i1) in ((True, (0, 1)), (False, (2, 3))):
        for i in range(steps):
            torch.sum(flush, dim=0, out=sink)
            cache.set_dispatch_events(ev[i][i0], ev[i][i1], main_kernel=main)
            call()
    for i in range(steps):
        torch.sum(flush, dim=0, out=sink)
        ev[i][4].record(stream)
        call()
        ev[i][5].record(stream)
    torch.cuda.synchronize()
    return tuple(float(np.mean([e[i0].elapsed_time(e[i0 + 1]) for e in ev])) / 1e3
                 for i0 in (0, 2, 4))


def dispatch_time(call, steps, torch, cache):
    """Mean time (s) of the main kernel of `call` (an attention call on
    `cache`) over `steps` launches, by dispatch events on that kernel."""
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        for x in e:
            x.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        cache.set_dispatch_events(ev[i][0], ev[i][1], main_kernel=True)
        call()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3


def decode_roofline(per_call, kern_s, call_s, mark_s, key, extra=None):
    """The decode `roofline` object: algorithmic bytes over the work-list
    kernel's time (the dominant kernel, as a kernel trace times it), with the
    whole call (work list, merge and the gap between them) beside it."""
    r = {"bound": "hbm", "achieved": per_call / kern_s / 1e9, "peak": HBM_PEAK_GBS,
         "unit": "GB/s", "frac": per_call / kern_s / 1e9 / HBM_PEAK_GBS,
         "traffic": counter_traffic(key, "k_decode_work<") if key else None,
         "kernel": "k_decode_work (the work-list kernel; dispatch events on it)",
         "avg_kernel_us": kern_s * 1e6, "bytes_per_call": per_call,
         "cache_evicted_before_each_call": True,
         "call": {"what": "kvc_attn_decode: work-list kernel, merge kernel and the gap "
                          "between them (first kernel start to last kernel end)",
                  "avg_us": call_s * 1e6, "achieved": per_call / call_s / 1e9,
                  "frac": per_call / call_s / 1e9 / HBM_PEAK_GBS,
                  "avg_us_stream_markers": mark_s * 1e6,
                  "traffic": counter_traffic(key) if key else None}}
    r.update(extra or {})
    return r


def bench_decode_window(steps, torch, kv, window=1024, sinks=4):
    """The Llama-8B decode batch with a 1,024-row sliding window and 4 sink
    rows: only the visible rows are read.  Algorithmic bytes count the
    visible K/V rows, their table entries, Q and O; every call is preceded
    by the Infinity-Cache eviction used for the decode roofline."""
    w, c, io = build_decode("llama8b_decode", torch, kv)
    seqs = torch.arange(w.batch, dtype=torch.int32, device="cuda")
    q = torch.from_numpy(w.q()).to(io).cuda()
    out = torch.empty((w.batch, w.n_q, w.d), dtype=io, device="cuda")
    ws = torch.empty((max(c.decode_workspace_bytes(w.batch), 16),), dtype=torch.uint8,
                     device="cuda")
    vis = [window_rows(int(L), window, sinks) for L in w.lengths]
    rows, blocks = sum(r for r, _ in vis), sum(b for _, b in vis)
    per_call = 2 * rows * w.n_kv * w.d * 2 + 2 * w.batch * w.n_q * w.d * 2 + 4 * blocks

    def call():
        c.attn_decode(0, seqs, q, out=out, ws=ws, window=window, sinks=sinks)
    warm_up_clocks(call, torch)
    kern_s, call_s, mark_s = evict_and_time(call, steps, torch, c)
    return {"workload": f"llama8b_decode, window {window} + {sinks} sink rows",
            "roofline": decode_roofline(per_call, kern_s, call_s, mark_s, None),
            "visible_rows": rows, "all_rows": int(np.sum(w.lengths))}


def bench_decode(name, steps, warmup, torch, kv, with_cpu):
    """One workload of the decode path.  A step grows every sequence by one
    token and appends its new rows (kvc_seq_grow_append), then runs
    kvc_attn_decode; `value` is the decode's algorithmic bytes per step over
    the wall-clock time of the K steps.  The roofline times kvc_attn_decode
    alone after an Infinity-Cache eviction."""
    diag = min(steps, 10)                                  # steps timed one by one, after
    w, c, io = build_decode(name, torch, kv, grow=warmup + steps + diag)
    kv_elem = KV_ELEM_BYTES[w.kv_dtype]
    seqs_host = list(range(w.batch))
    seqs = torch.arange(w.batch, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(123)
    q = torch.from_numpy(w.q()).to(io).cuda()
    knew = torch.from_numpy(rng.standard_normal((w.batch, w.n_kv, w.d), dtype=np.float32)).to(io).cuda()
    vnew = torch.from_numpy(rng.standard_normal((w.batch, w.n_kv, w.d), dtype=np.float32)).to(io).cuda()
    out = torch.empty((w.batch, w.n_q, w.d), dtype=io, device="cuda")
    # the library's own figure; the work-list plan does not depend on the
    # lengths, so it covers every step of the run
    ws_bytes = c.decode_workspace_bytes(w.batch)
    ws = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        c.seq_grow_append(0, seqs_host, knew, vnew)
        c.attn_decode(0, seqs, q, out=out, ws=ws)
        if ev is not None:
            ev[1].record(stream)

    def call():
        c.attn_decode(0, seqs, q, out=out, ws=ws)

    # pre-heat: the same decode call, which changes no state, until the clocks
    # have left their idle level (the first launches also load the kernels)
    warm_up_clocks(call, torch)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    lens0 = np.array([c.seq_len(b) for b in range(w.batch)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # algorithmic bytes of each timed decode: lengths lens0+1 .. lens0+steps
    total_bytes = sum(decode_bytes(w, lens0 + i + 1, kv_elem) for i in range(steps))
    # device time of single steps, outside the timed region: event records in
    # the stream leave gaps of their own between the steps they bracket
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(diag)]
    for i in range(diag):
        step(events[i])
    torch.cuda.synchronize()
    warm_avg_s = float(np.mean([a.elapsed_time(b) for a, b in events])) / 1e3
    # roofline: the same decode call (state after those steps), cold
    lens1 = lens0 + steps + diag
    per_call = decode_bytes(w, lens1, kv_elem)
    kern_s, call_s, mark_s = evict_and_time(call, steps, torch, c)
    res = {
        "workload": name,
        "value": total_bytes / wall / 1e9,
        "unit": "GB/s",
        "ms_per_step": wall / steps * 1e3,
        "roofline": decode_roofline(per_call, kern_s, call_s, mark_s, "decode_" + name,
                                    {"avg_step_us_warm": warm_avg_s * 1e6}),
        "shape": {"batch": w.batch, "n_q": w.n_q, "n_kv": w.n_kv, "d": w.d,
                  "kv_dtype": w.kv_dtype, "mean_len": float(np.mean(lens0 + 1))},
    }
    if with_cpu:
        res["cpu_baseline"] = cpu_decode(w, q, kv_elem, torch, io)
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_fields():
    return {"cores": cpu_cores(), "blas_threads": blas_threads(), "cpu_model": cpu_model(),
            "kind": "oracle"}


def cpu_decode(w, q, kv_elem, torch, io, budget_s=10.0, prep_budget_s=15.0):
    """Time the float64 oracle's decode on the workload, one (sequence, kv
    head) unit at a time: the G query rows of that kv head against all L_b
    cached rows.  Passes run over the units in order (sequence-major) until
    `budget_s` of oracle time is spent; each unit's inputs (the source rows
    rounded to the io type, widened to float64) are prepared outside the timed
    region, at most `prep_budget_s` worth of them.  Reported in the same
    algorithmic bytes per second as the GPU: a unit carries 2 L_b d element
    bytes of K/V, its query and output rows, and its share of the table
    entries and block scales."""
    from oracle import attention as A
    scale = 1.0 / math.sqrt(w.d)
    G = w.n_q // w.n_kv
    qd = q.detach().cpu().double().numpy()
    units, t_prep = [], time.perf_counter()
    for b in range(w.batch):
        if time.perf_counter() - t_prep >= prep_budget_s:
            break
        K, V = source_rows(w, b, torch, io)
        K32, V32 = K.float().numpy(), V.float().numpy()        # contiguous, exact widening
        for g in range(w.n_kv):
            units.append((b, g, K32[:, g:g + 1].astype(np.float64),
                          V32[:, g:g + 1].astype(np.float64)))
        del K32, V32
    prep = time.perf_counter() - t_prep
    done_bytes, spent, n_done = 0.0, 0.0, 0
    while spent < budget_s:
        for b, g, Kd, Vd in units:
            t0 = time.perf_counter()
            A.decode_attention(qd[b, g * G:(g + 1) * G], Kd, Vd, scale)
            spent += time.perf_counter() - t0
            L = Kd.shape[0]
            nblk = -(-L // 16)
            done_bytes += (2 * L * w.d * kv_elem + 2 * G * w.d * 2 + nblk * 4 / w.n_kv
                           + (2 * nblk * 4 if kv_elem < 2 else 0))
            n_done += 1
            if spent >= budget_s:
                break
    src = "bf16-rounded source rows (the oracle's cost does not depend on the values)" \
        if w.kv_dtype in ("fp8", "int4") else "the cached rows"
    return dict(value=done_bytes / spent / 1e9, unit="GB/s", **cpu_fields(),
                sample=f"float64 oracle decode of {n_done} (sequence, kv head) units of "
                       f"{w.batch} x {w.n_kv}, passes over the first {len(units)} units, "
                       f"on {src} ({spent:.1f} s; inputs prepared in {prep:.1f} s)")


# ---------------------------------------------------------------- prefill
def prefill_flops(batch, T, n_q, d):
    """Causal attention FLOPs: per (sequence, head) 2*d multiply-adds for QK^T
    and 2*d for PV over the T(T+1)/2 visible (query, key) pairs."""
    return batch * n_q * 4 * d * T * (T + 1) // 2


def bench_prefill(steps, warmup, torch, kv, with_cpu, small=False):
    from workloads import prefill_workload
    w = prefill_workload(small=small)
    qn, kn, vn = w.qkv()
    q, k, v = (torch.from_numpy(a).to(torch.bfloat16).cuda() for a in (qn, kn, vn))
    del qn, kn, vn
    nb = -(-w.T // 16)
    c = kv.KvCache(1, w.n_q, w.n_kv, w.d, w.batch * nb, w.batch, nb, "bf16")
    seqs = torch.arange(w.batch, dtype=torch.int32, device="cuda")
    for b in range(w.batch):
        c.seq_alloc(b, w.T)
    out = torch.empty((w.batch, w.T, w.n_q, w.d), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        c.attn_prefill(0, q, k, v, seqs=seqs, out=out)
    warm_up_clocks(lambda: c.attn_prefill(0, q, k, v, seqs=seqs, out=out), torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        c.attn_prefill(0, q, k, v, seqs=seqs, out=out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    flops = prefill_flops(w.batch, w.T, w.n_q, w.d)
    # stream markers around single calls, outside the timed region
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(min(steps, 10))]
    for e0, e1 in events:
        e0.record(stream)
        c.attn_prefill(0, q, k, v, seqs=seqs, out=out)
        e1.record(stream)
    torch.cuda.synchronize()
    call_s = float(np.mean([a.elapsed_time(b) for a, b in events])) / 1e3
    kern_s = dispatch_time(lambda: c.attn_prefill(0, q, k, v, seqs=seqs, out=out), steps, torch, c)
    achieved = flops / kern_s / 1e12
    res = {
        "workload": "llama8b_prefill" if not small else "llama8b_prefill_small",
        "value": flops * steps / wall / 1e12, "unit": "TFLOP/s",
        "ms_per_step": wall / steps * 1e3,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
                     "traffic": counter_traffic("prefill_llama8b_prefill", "k_prefill_mfma<"),
                     "kernel": "k_prefill_mfma (the attention kernel; dispatch events on it)",
                     "avg_kernel_us": kern_s * 1e6, "flops_per_call": flops,
                     "call": {"what": "kvc_attn_prefill: attention kernel with the K/V cache "
                                      "write beside it on the side stream (stream markers)",
                              "avg_us_stream_markers": call_s * 1e6,
                              "achieved": flops / call_s / 1e12,
                              "frac": flops / call_s / 1e12 / BF16_PEAK_TFLOPS,
                              "traffic": counter_traffic("prefill_llama8b_prefill")}},
        "shape": {"batch": w.batch, "T": w.T, "n_q": w.n_q, "n_kv": w.n_kv, "d": w.d},
    }
    if with_cpu:
        res["cpu_baseline"] = cpu_prefill(w, q, k, v, torch)
    return res


def cpu_prefill(w, q, k, v, torch, budget_s=12.0):
    """The float64 oracle's causal attention, one (sequence, query head) at a
    time, until the budget is used; reported as algorithmic TFLOP/s."""
    from oracle import attention as A
    scale = 1.0 / math.sqrt(w.d)
    G = w.n_q // w.n_kv
    spent, heads = 0.0, 0
    for b in range(w.batch):
        for h in range(w.n_q):
            qh = q[b, :, h].double().cpu().numpy()
            kh = k[b, :, h // G].double().cpu().numpy()
            vh = v[b, :, h // G].double().cpu().numpy()
            t0 = time.perf_counter()
            A.attention(qh, kh, vh, scale, q_pos=np.arange(w.T))
            spent += time.perf_counter() - t0
            heads += 1
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    flops = heads * 4 * w.d * w.T * (w.T + 1) // 2
    return dict(value=flops / spent / 1e12, unit="TFLOP/s", **cpu_fields(),
                sample=f"float64 oracle causal attention of {heads} of {w.batch * w.n_q} "
                       f"(sequence, head) pairs ({spent:.1f} s)")


# ---------------------------------------------------------------- extend
EXTEND_CHUNK = 512


def extend_flops(batch, ctx, chunk, n_q, d):
    """4*d per visible (query, key) pair: query t of the chunk sees ctx + t + 1 keys."""
    pairs = chunk * ctx + chunk * (chunk + 1) // 2
    return 4 * d * pairs * batch * n_q


def bench_extend(steps, warmup, torch, kv, with_cpu):
    """Chunked prefill: the last 512-token chunk of the four 8,192-token
    prompts of the prefill workload, against the 7,680 cached rows before it.
    A step writes the chunk's K/V into the paged cache (kvc_write at 7,680)
    and runs kvc_attn_extend on its queries; the roofline times the
    attention call."""
    from workloads import prefill_workload
    w = prefill_workload()
    ctx = w.T - EXTEND_CHUNK
    qn, kn, vn = w.qkv()
    q = torch.from_numpy(qn[:, ctx:]).to(torch.bfloat16).cuda().contiguous()
    k, v = (torch.from_numpy(a).to(torch.bfloat16).cuda() for a in (kn, vn))
    del qn, kn, vn
    nb = -(-w.T // 16)
    c = kv.KvCache(1, w.n_q, w.n_kv, w.d, w.batch * nb, w.batch, nb, "bf16")
    perm = np.random.default_rng(5).permutation(w.batch * nb).astype(np.int32)
    for b in range(w.batch):
        c.set_block_table(b, perm[b * nb:(b + 1) * nb], w.T)
    seqs = torch.arange(w.batch, dtype=torch.int32, device="cuda")
    c.write(0, seqs, 0, k[:, :ctx].contiguous(), v[:, :ctx].contiguous())
    kc, vc = k[:, ctx:].contiguous(), v[:, ctx:].contiguous()
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        c.write(0, seqs, ctx, kc, vc)
        if ev is not None:
            ev[0].record(stream)
        c.attn_extend(0, seqs, q, out=out)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(warmup):
        step()
    warm_up_clocks(step, torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    flops = extend_flops(w.batch, ctx, EXTEND_CHUNK, w.n_q, w.d)
    # stream markers around single calls, outside the timed region
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(min(steps, 10))]
    for ev in events:
        step(ev)
    torch.cuda.synchronize()
    call_s = float(np.mean([a.elapsed_time(b) for a, b in events])) / 1e3

    def step_timed():
        c.write(0, seqs, ctx, kc, vc)
        c.attn_extend(0, seqs, q, out=out)
    kern_s = dispatch_time(step_timed, steps, torch, c)
    achieved = flops / kern_s / 1e12
    res = {
        "workload": "llama8b_extend",
        "value": flops * steps / wall / 1e12, "unit": "TFLOP/s",
        "ms_per_step": wall / steps * 1e3,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
                     "traffic": counter_traffic("extend_llama8b_extend", "k_prefill_mfma<"),
                     "kernel": "k_prefill_mfma, paged (dispatch events on it)",
                     "avg_kernel_us": kern_s * 1e6, "flops_per_call": flops,
                     "call": {"what": "kvc_attn_extend (stream markers)",
                              "avg_us_stream_markers": call_s * 1e6,
                              "achieved": flops / call_s / 1e12,
                              "frac": flops / call_s / 1e12 / BF16_PEAK_TFLOPS}},
        "shape": {"batch": w.batch, "context": ctx, "chunk": EXTEND_CHUNK, "n_q": w.n_q,
                  "n_kv": w.n_kv, "d": w.d},
    }
    if with_cpu:
        res["cpu_baseline"] = cpu_extend(w, ctx, q, k, v)
    return res


def cpu_extend(w, ctx, q, k, v, budget_s=12.0):
    """The float64 oracle on the same chunk, one (sequence, query head) at a
    time, pass after pass over the pairs, until the budget is used; reported
    as algorithmic TFLOP/s."""
    from oracle import attention as A
    scale = 1.0 / math.sqrt(w.d)
    G = w.n_q // w.n_kv
    pairs = [(q[b, :, h].double().cpu().numpy(), k[b, :, h // G].double().cpu().numpy(),
              v[b, :, h // G].double().cpu().numpy())
             for b in range(w.batch) for h in range(w.n_q)]
    spent, heads = 0.0, 0
    while spent < budget_s:
        for qh, kh, vh in pairs:
            t0 = time.perf_counter()
            A.attention(qh, kh, vh, scale, q_pos=np.arange(ctx, w.T))
            spent += time.perf_counter() - t0
            heads += 1
            if spent >= budget_s:
                break
    flops = extend_flops(1, ctx, EXTEND_CHUNK, 1, w.d) * heads
    return dict(value=flops / spent / 1e12, unit="TFLOP/s", **cpu_fields(),
                sample=f"float64 oracle chunk attention of {heads} (sequence, head) pairs, "
                       f"passes over the {w.batch * w.n_q} pairs ({spent:.1f} s)")


# ---------------------------------------------------------------- prefix sharing
def bench_prefix_share(torch, kv, n_seq=40, prompt=600, n_layers=32):
    """Forty conversations sharing one 600-token system prompt (Llama-8B
    cache shape: 32 layers, 8 kv heads of 128, bf16).  Sharing holds the
    prompt's 38 blocks once; the first grow of every sequence copies the
    shared, partly filled last block (copy-on-write).  Reports the blocks
    held and the copy kernel's rate (bytes copied / GPU time of the grow,
    median of 7 repetitions after 3 untimed ones)."""
    n_kv, d = 8, 128
    nb_prompt = -(-prompt // 16)
    c = kv.KvCache(n_layers, 32, n_kv, d, nb_prompt + 2 * n_seq + 8, n_seq + 1, nb_prompt + 4,
                   "bf16")
    c.seq_alloc(0, prompt)
    stream = torch.cuda.current_stream()
    held = None

    def share_grow_release():
        """Share the prompt with every sequence, time their first grow (the
        block copies), release them again."""
        nonlocal held
        for s in range(1, n_seq + 1):
            c.seq_share_prefix(0, s, prompt)
        held = c.cfg.n_blocks - c.free_blocks()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        c.seq_grow(list(range(1, n_seq + 1)))
        b.record(stream)
        torch.cuda.synchronize()
        for s in range(1, n_seq + 1):
            c.seq_release(s)
        return a.elapsed_time(b) * 1e3

    for _ in range(3):                                         # kernels loaded, clocks up
        share_grow_release()
    us = float(np.median([share_grow_release() for _ in range(7)]))
    copied = n_seq * n_layers * 2 * n_kv * 16 * d * 2          # K and V of each copied block
    return {"workload": f"{n_seq} sequences sharing a {prompt}-token prompt, Llama-8B cache shape "
                        f"({n_layers} layers, {n_kv} kv heads of {d}, bf16)",
            "blocks_held_shared": held, "blocks_held_unshared": (n_seq + 1) * nb_prompt,
            "first_grow_us": us, "copy_on_write_bytes": copied,
            "copy_on_write_GBps": copied / (us * 1e-6) / 1e9}


DECODE_WORKLOADS = {
    "llama8b_decode": "40 sequences, 32 q / 8 kv heads, d 128, bf16 cache, 16-token blocks, "
                      "shuffled tables, lengths uniform in [512, 4096]; step = grow + "
                      "kvc_attn_decode_append (kv_append and the decode in one call)",
    "llama70b_decode_bf16": "8 x 32,768-token contexts, 64 q / 8 kv heads, d 128, bf16 cache, "
                            "1% outliers x8",
    "llama70b_decode_fp8": "8 x 32,768-token contexts, 64 q / 8 kv heads, d 128, fp8-e4m3 cache "
                           "with per-block scales, 1% outliers x8",
    "llama70b_decode_int4": "8 x 32,768-token contexts, 64 q / 8 kv heads, d 128, int4 cache "
                            "with per-block scales, 1% outliers x8",
    "long_mha_decode": "1 x 128,000-token context, 32 / 32 heads, d 128, fp16 cache, "
                       "split-context decode",
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_decode",
                    choices=sorted(DECODE_WORKLOADS) + ["llama8b_prefill", "llama8b_extend"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-prefill", action="store_true",
                    help="headline decode only (no prefill section)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 5 times (calibrates the HBM "
                         "byte counters read by rocprofv3 --pmc) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the work shards into independent per-GPU units; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        nbytes = args.copy_probe << 20
        x = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes,
                          "repeats": 5}))
        return
    import kv_cache_flashattention_amd as kv
    kv.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    with_cpu = not args.no_cpu

    if args.workload == "llama8b_extend":
        log("llama8b_extend")
        ex = bench_extend(args.steps, args.warmup, torch, kv, with_cpu)
        line = {"metric": METRIC, "value": ex["value"], "unit": "TFLOP/s", "n_gpus": 1,
                "steps": args.steps, "warmup": args.warmup, "ms_per_step": ex["ms_per_step"],
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                "dtype": "bf16", "data": "synthetic (seeded N(0,1))",
                "config": {"workload": "llama8b_extend: last 512-token chunk of 4 x 8,192-token "
                                       "prompts against 7,680 cached rows, 32 q / 8 kv heads, "
                                       "d 128, bf16 paged cache"},
                "roofline": ex["roofline"], "cpu_baseline": ex.get("cpu_baseline")}
        print(json.dumps(line))
        return
    if args.workload == "llama8b_prefill":
        log("llama8b_prefill")
        pf = bench_prefill(args.steps, args.warmup, torch, kv, with_cpu)
        line = {"metric": METRIC, "value": pf["value"], "unit": "TFLOP/s", "n_gpus": 1,
                "steps": args.steps, "warmup": args.warmup, "ms_per_step": pf["ms_per_step"],
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                "dtype": "bf16", "data": "synthetic (seeded N(0,1))",
                "config": {"workload": "llama8b_prefill: 4 x 8,192 tokens, 32 q / 8 kv heads, "
                                       "d 128, bf16, causal, K/V appended to the paged cache"},
                "roofline": pf["roofline"], "cpu_baseline": pf.get("cpu_baseline")}
        print(json.dumps(line))
        return

    log(f"{args.workload}: building the cache")
    dec = bench_decode(args.workload, args.steps, args.warmup, torch, kv, with_cpu)
    log(f"{args.workload}: {dec['roofline']['avg_kernel_us']:.1f} us per work kernel, "
        f"frac {dec['roofline']['frac']:.3f}")
    dtype = {"bf16": "bf16", "fp16": "f16", "fp8": "fp8-e4m3 (bf16 q/o)",
             "int4": "int4 (bf16 q/o)"}[dec["shape"]["kv_dtype"]]
    line = {"metric": METRIC, "value": dec["value"], "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": dec["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": dtype, "data": "synthetic (seeded N(0,1))",
            "config": {"workload": f"{args.workload}: {DECODE_WORKLOADS[args.workload]}",
                       "mean_context": dec["shape"]["mean_len"]},
            "roofline": dec["roofline"], "cpu_baseline": dec.get("cpu_baseline")}
    if args.workload == "llama8b_decode" and not args.no_prefill:
        k2 = max(5, args.steps // 2)
        line["decode_window"] = bench_decode_window(k2, torch, kv)
        log(f"decode_window: frac {line['decode_window']['roofline']['frac']:.3f}")
        drop_rows("llama8b_decode")
        line["prefill"] = bench_prefill(k2, 2, torch, kv, with_cpu)
        log(f"prefill: frac {line['prefill']['roofline']['frac']:.3f}")
        for key, name in (("decode_llama70b_bf16", "llama70b_decode_bf16"),
                          ("decode_llama70b_fp8", "llama70b_decode_fp8"),
                          ("decode_int4", "llama70b_decode_int4"),
                          ("decode_long_mha", "long_mha_decode")):
            line[key] = bench_decode(name, k2, 2, torch, kv, with_cpu and "int4" not in name)
            line[key]["config"] = DECODE_WORKLOADS[name]
            log(f"{key}: {line[key]['roofline']['avg_kernel_us']:.1f} us per work kernel, "
                f"frac {line[key]['roofline']['frac']:.3f}")
            if name == "llama70b_decode_int4":
                drop_rows("llama70b_decode")
        drop_rows("long_mha_decode")
        line["extend"] = bench_extend(k2, 2, torch, kv, with_cpu)
        log(f"extend: frac {line['extend']['roofline']['frac']:.3f}")
        line["prefix_share"] = bench_prefix_share(torch, kv)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
