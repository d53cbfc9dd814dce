"""Benchmark: GatedDeltaNet speculative verify + commit on one MI355X.

A step is one pass of the whole path over one batch: the verify of every
request's k+1 rows and the commit of its accepted rows. The default
workload is the saturated batch: 64 requests, 9 verify rows (k = 8), a
Qwen3-Next-shaped layer (16 key / 32 value heads, d = 128, conv width 4 over
8192 channels, bf16 inputs, fp32 state), a 256-slot pool and geometric(0.3)
accept lengths capped at 9.

Steps rotate over 16 independent copies of the workload (as the layers of a
hybrid stack would), verifying a group of copies and then committing them, as
a model verifies every layer before it commits any. Between two uses of a
copy the other copies move several GB, so nothing of it (state, inputs, or
the stash the commit reads back) is still in the 256 MB Infinity Cache: every
kernel runs cold. All inputs are resident in HBM before the timed region.

Schedule (--schedule, reported in the line): fused (the default on the layers
it serves: bf16 storage, d = 128, an even number of value heads per key head,
eager launches) makes each step one gdn_spec_commit_verify launch, which
commits the copy's previous step into the state on its way into this step's
verify; every step still verifies one batch and commits one. serial issues
gdn_spec_verify then gdn_spec_commit on one stream (the default elsewhere).
overlap issues a group's commits on a second stream
once the whole group is verified, and a copy's next verify waits for that
copy's commit, as a serving loop that starts the next step's layers while the
last step's states are committed would; every data dependency of the serial
order holds. It pays in long runs of large replay batches (one kernel's ramp
and tail take the other's work); over a few steps the pipeline's fill and
drain and the per-launch stream waits cost more than it gains. Per-kernel
durations are always timed serially, each kernel's launches back to back.

Prints one JSON line. value = verify rows per second (batch x rows per step);
gbps = algorithmic HBM bytes per second: per request, verify reads the state,
the conv history, x and the gates and writes o and a stash of the rows' raw
inputs; commit reads and writes the state and the conv history and reads the
accepted rows' stash. A fused step reads the state and the history once for
both (gbps counts them once); its line adds serial_equivalent, the serial
pair's bytes over the same step time: the rate at which a verify then a
commit would have to run to match the step (not an HBM measurement).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "GDN verify+commit rows/s and achieved HBM GB/s (% of MI355X peak)"
HBM_PEAK_GBPS = 8000.0
COPY_BYTES = 256 << 20
KERNEL_SOURCE = os.path.join(ROOT, "linear_attention_verify_amd", "csrc", "gdn_spec.hip")
ATTN_SOURCE = os.path.join(ROOT, "linear_attention_verify_amd", "csrc", "spec_attention.hip")
SAMPLE_SOURCE = os.path.join(ROOT, "linear_attention_verify_amd", "csrc", "spec_sample.hip")

# HBM bytes per launch read from rocprofv3 counters: FETCH_SIZE and WRITE_SIZE
# (KiB per dispatch, one run each) of every launch of the kernel, averaged,
# each scaled by known bytes / counter bytes of a plain 256 MiB device copy
# in the same run. They hold only for the kernel code they were taken on
# (kernel_source_digest of the source file); for any other code the bench
# reports null.
MEASURED_TRAFFIC = [
    {"source": KERNEL_SOURCE,
     "source_sha256": "20972e0f456647e2e7bccd4b0e45b0b3bbf201907f65ff6507239ea2b36bbc95",
     "bytes": {   # (workload, mode, kernel) -> bytes per launch
         ("saturated-b64", "replay", "commit_verify"): 322533434,
         ("saturated-b64", "replay", "verify"): 179223169,
         ("saturated-b64", "replay", "commit"): 282701289,
         ("saturated-b64", "snapshot", "commit_verify"): 1525092159,
         ("saturated-b64", "snapshot", "verify"): 1387496722,
         ("saturated-b64", "snapshot", "commit"): 274768731,
     }},
    {"source": ATTN_SOURCE,
     "source_sha256": "f254bc77bc855d9281a6304db619d063533d81c6e4ed714c46000f8b555346f6",
     "bytes": {   # one call: split kernel + combine kernel
         ("attn-b64", "-", "attn_verify"): 681347947,
     }},
    {"source": SAMPLE_SOURCE,
     "source_sha256": "efe9de2a538f6b01887b342eff1afa6650fcceddd1d855fb42a42a7e920bffab",
     "bytes": {   # one call: stats kernel + draw kernel
         ("sample-b64", "-", "accept_sample"): 275209893,
     }},
]


def kernel_source_digest(path=KERNEL_SOURCE):
    """SHA-256 of the kernel source with comments and whitespace removed, so
    that only a change to the code itself invalidates measured figures."""
    import hashlib
    import re
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


def measured_traffic(workload, mode, kernel):
    for entry in MEASURED_TRAFFIC:
        key = (workload, mode, kernel)
        if key in entry["bytes"] and kernel_source_digest(entry["source"]) == entry["source_sha256"]:
            return entry["bytes"][key]
    return None


def calibration_copy():
    """A plain 256 MiB device copy: the reference dispatch that scales the
    rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()


def algorithmic_bytes(w, accept, mode="replay"):
    """(verify bytes, commit bytes) per launch for workload w and accept lengths.

    Per request, verify reads the state (HV*D*D fp32), the conv history
    ((W-1)*C), the rows' inputs (R*C) and gates (2*R*HV) and writes o (R*HV*D)
    and a stash of each row's raw inputs and gates (R*(C+2*HV)); snapshot mode
    also writes the R states S_1..S_R. Per request with n > 0 accepted rows,
    commit reads and writes the state and the conv history and reads the n
    stashed rows (replay), or reads the selected snapshot instead of the
    state (snapshot). Element sizes: E for inputs, 4 for the state.
    """
    s = w.shape
    E, HV, D, C, W, R = s.elem_bytes, s.num_v_heads, s.d_k, s.conv_channels, s.conv_width, w.rows
    state = HV * D * D * 4
    hist = (W - 1) * C * E
    row_stash = (C + 2 * HV) * E
    per_verify = state + hist + R * C * E + 2 * R * HV * E + R * HV * D * E + R * row_stash
    if mode == "snapshot":
        per_verify += R * state
    verify = w.batch * per_verify
    commit = 0
    for n in accept:
        if n > 0:
            commit += 2 * state + 2 * hist + int(n) * row_stash
    return verify, commit


def fused_bytes(w, accept, mode="replay"):
    """Bytes per commit-verify launch: one step's verify and the previous
    step's commit of the same requests, less what the two share. The state
    (replay) or the saved S_n (snapshot) and the conv history are read once
    for both, so a request with n > 0 pending rows reads its state once and
    writes it once."""
    vbytes, cbytes = algorithmic_bytes(w, accept, mode)
    s = w.shape
    state = s.num_v_heads * s.d_k * s.d_v * 4
    hist = (s.conv_width - 1) * s.conv_channels * s.elem_bytes
    shared = sum(state + hist for n in accept if n > 0)
    return vbytes + cbytes - shared


# Worker threads for the oracle leg: a host serving one GPU gives this process
# a share of 16 cores, whatever the affinity mask shows, so the oracle uses at
# most 16 threads; the affinity count is reported beside it.
CPU_SHARE_THREADS = 16


def _oracle_passes(orc, w, d, accept, threads, budget_s):
    """Verify + commit passes of the whole batch for budget_s seconds;
    returns (passes, seconds)."""
    import numpy as np

    from linear_attention_verify_amd import workloads as wl

    # compact pool: request b in slot b (the oracle's cost does not depend on slot ids)
    compact = wl.Workload(name=w.name, shape=w.shape, batch=w.batch, rows=w.rows, num_slots=w.batch)
    slot_ids = np.arange(w.batch, dtype=np.int32)
    ssm, conv = wl.build_pools(compact, d, slot_ids)
    s = w.shape
    reps = 0
    t0 = time.perf_counter()
    while True:
        # verify, then commit in place: the state moves on as in a decode loop
        orc.verify(s, ssm, conv, d["conv_w"], d["x"], d["alpha"], d["beta"], slot_ids, w.rows,
                   nthreads=threads)
        orc.commit(s, ssm, conv, d["conv_w"], d["x"], d["alpha"], d["beta"], slot_ids, accept,
                   w.rows, nthreads=threads)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return reps, time.perf_counter() - t0


def cpu_baseline(w, budget_s=12.0, single_s=6.0):
    """The oracle (as it stands) on the same workload on this host: with one
    OpenMP thread per core of the process's CPU share, and with one thread."""
    import oracle
    from linear_attention_verify_amd import workloads as wl

    affinity = len(os.sched_getaffinity(0))
    threads = min(affinity, CPU_SHARE_THREADS)
    orc = oracle.Oracle()
    _, accept = wl.draw_requests(w)
    d = wl.draw_layer(w)
    rows = w.batch * w.rows
    reps, dt = _oracle_passes(orc, w, d, accept, threads, budget_s)
    reps1, dt1 = _oracle_passes(orc, w, d, accept, 1, single_s)
    return {"value": reps * rows / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "threads": threads, "affinity_cores": affinity,
            "threads_note": "one OpenMP thread per core of the %d-core share of a host serving one GPU "
                            "(min of the affinity mask and %d)" % (CPU_SHARE_THREADS, CPU_SHARE_THREADS),
            "sample": "%d full verify+commit passes of the %s batch (%d requests x %d rows), fp64, %.1f s"
                      % (reps, w.name, w.batch, w.rows, dt),
            "single_thread": {"value": reps1 * rows / dt1, "unit": "rows/s", "cores": 1,
                              "sample": "%d full passes of the same batch on one thread, %.1f s" % (reps1, dt1)}}


ATTN_METRIC = "verification attention rows/s and achieved HBM GB/s (% of MI355X peak)"


def attention_bytes(w, seq_lens):
    """Algorithmic bytes of one verification-attention call: every key and value
    of each request's seq_len positions (Hkv heads of D bf16 values each) read
    once, the queries read and the outputs written once. The split partial
    results are scratch traffic of this implementation and are not counted."""
    s = w.shape
    kv = sum(2 * int(L) * s.num_kv_heads * s.head_dim * 2 for L in seq_lens)
    qo = 2 * w.batch * w.rows * s.num_q_heads * s.head_dim * 2
    return kv + qo


def attention_cpu_baseline(w, d, budget_s=12.0):
    """The attention oracle (NumPy fp64, as it stands) on a sample of requests."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention
    from linear_attention_verify_amd import workloads as wl

    f = wl.bf16_bits_to_f32
    k, v = f(d["k_cache"]), f(d["v_cache"])
    n = min(4, w.batch)
    q = f(d["q"][:n])
    reps = 0
    t0 = time.perf_counter()
    while True:
        attention.verify_attention(q, k, v, d["block_table"][:n], d["seq_lens"][:n], w.shape.page_size,
                                   w.shape.scale)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": reps * n * w.rows / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": "%d passes over requests 0..%d of the %s batch (%d rows each, seq_len %s), fp64"
                      % (reps, n - 1, w.name, w.rows, d["seq_lens"][:n].tolist())}


def run_attention(args, w):
    """Verification attention over the paged KV cache: a step is one
    gdn_spec_attn_verify call (split kernel + combine kernel) over the batch.
    Steps alternate between two copies of the cache so that no call finds the
    previous call's keys and values in the 256 MB memory-side cache."""
    import numpy as np
    import torch

    from linear_attention_verify_amd import binding as bd
    from linear_attention_verify_amd import workloads as wl

    if args.graph or args.accept != "given" or args.mode != "replay":
        raise SystemExit("--graph, --accept and --mode apply to GDN workloads")
    if args.calibrate_copy:
        calibration_copy()
    d = wl.draw_attention(w)
    s = w.shape
    dev = "cuda"

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    desc = bd.attn_desc(s)
    q = bits(d["q"])
    bt = torch.from_numpy(d["block_table"]).to(dev)
    sl = torch.from_numpy(d["seq_lens"]).to(dev)
    nbytes = bd.gdn_spec_attn_scratch_bytes(desc, w.batch, w.rows, bt.shape[1])
    stream = torch.cuda.current_stream()
    M = 2
    calls, keep = [], []
    for _ in range(M):
        kc, vc = bits(d["k_cache"]), bits(d["v_cache"])
        scratch = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        calls.append(bd.PreparedAttn(desc, q, kc, vc, bt, sl, scratch, out, err, stream))
        keep.append(err)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        calls[i % M]()
    torch.cuda.synchronize()
    if any(int(e.item()) for e in keep):
        raise SystemExit("device error flags set")
    t0 = time.perf_counter()
    for i in range(args.steps):
        calls[i % M]()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-call durations: HIP events on the launch stream around each call
    ev = []
    for i in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        calls[i % M]()
        b.record(stream)
        ev.append((a, b))
    torch.cuda.synchronize()
    tcall = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    nb = attention_bytes(w, d["seq_lens"])
    rows = w.batch * w.rows
    ach = nb / tcall / 1e9
    line = {
        "metric": ATTN_METRIC, "value": rows * args.steps / wall, "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "rows": w.rows, "q_heads": s.num_q_heads,
                   "kv_heads": s.num_kv_heads, "head_dim": s.head_dim, "page_size": s.page_size,
                   "seq_len_mean": float(np.mean(d["seq_lens"])), "seq_len_range": [w.min_len, w.max_len],
                   "rotating_copies": M},
        "gbps": nb * args.steps / wall / 1e9, "hbm_frac": nb * args.steps / wall / 1e9 / HBM_PEAK_GBPS,
        "kernels": {"attn_verify": {"avg_us": tcall * 1e6, "bytes": nb, "gbps": ach}},
        "roofline": {"bound": "hbm", "kernel": "attn_verify (split + combine)", "achieved": ach,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(w.name, "-", "attn_verify")},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = attention_cpu_baseline(w, d, args.cpu_seconds)
    print(json.dumps(line), flush=True)


SAMPLE_METRIC = "speculative sampling rows/s and achieved HBM GB/s (% of MI355X peak)"


def sample_bytes(w, d):
    """Algorithmic bytes of one sampling call: every logit of every row read
    once (each row's softmax needs its whole row), the prior counts once, and
    the small per-request inputs and outputs."""
    B, R, V = w.batch, w.rows, w.vocab
    logits = B * R * V * 2
    counts = B * V * 4 if "prior_counts" in d else 0
    probs = B * (R - 1) * V * 4 if w.draft_probs else 0
    small = B * (R - 1) * 4 + B * 4 * 6
    return logits + counts + probs + small


def sample_cpu_baseline(w, d, budget_s=12.0):
    """The sampling oracle (NumPy fp64, as it stands) on a sample of requests."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import sampling
    from linear_attention_verify_amd import workloads as wl

    n = min(2, w.batch)
    lg = wl.bf16_bits_to_f32(d["logits"][:n])
    opt = {k: d[k][:n] for k in ("pending", "prior_counts", "presence", "frequency") if k in d}
    reps = 0
    t0 = time.perf_counter()
    while True:
        sampling.speculative_sample(lg, d["draft"][:n], 1 + reps, d["temperature"][:n], **opt)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": reps * n * w.rows / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": "%d passes over requests 0..%d of the %s batch (%d rows x %d vocabulary), fp64"
                      % (reps, n - 1, w.name, w.rows, w.vocab)}


def run_sample(args, w):
    """Speculative sampling of the verify rows' logits: a step is one
    gdn_spec_accept_sample call (stats, residual and final kernels) over the
    batch, with a new seed per step. Steps alternate between two copies of the
    logits so that no call finds the previous call's in the memory-side cache."""
    import numpy as np
    import torch

    from linear_attention_verify_amd import binding as bd
    from linear_attention_verify_amd import workloads as wl

    if args.graph or args.accept != "given" or args.mode != "replay":
        raise SystemExit("--graph, --accept and --mode apply to GDN workloads")
    if args.calibrate_copy:
        calibration_copy()
    d = wl.draw_sample(w)
    dev = "cuda"
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    B, R, V = w.batch, w.rows, w.vocab
    M = 2
    calls, keep = [], []
    for _ in range(M):
        lg = torch.from_numpy(np.ascontiguousarray(d["logits"]).view(np.int16)).to(dev).view(torch.bfloat16)
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        nxt = torch.empty(B, dtype=torch.int32, device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        scratch = torch.empty(bd.gdn_spec_sample_scratch_bytes(B, R, V), dtype=torch.uint8, device=dev)
        calls.append(bd.PreparedSample(lg, t(d["draft"]), t(d["temperature"]), acc, nxt, scratch,
                                       pending=t(d.get("pending")), prior_counts=t(d.get("prior_counts")),
                                       presence=t(d.get("presence")), frequency=t(d.get("frequency")),
                                       err_flag=err, stream=torch.cuda.current_stream()))
        keep.append((acc, err))
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    for i in range(args.warmup):
        calls[i % M](1000 + i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        calls[i % M](i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    a, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(args.steps):
        calls[i % M](i)
    b2.record(stream)
    torch.cuda.synchronize()
    tcall = a.elapsed_time(b2) * 1e-3 / args.steps
    if any(int(e.item()) for _, e in keep):
        raise SystemExit("device error flags set")
    acc_mean = float(np.mean(keep[0][0].cpu().numpy()))
    nb = sample_bytes(w, d)
    ach = nb / tcall / 1e9
    line = {
        "metric": SAMPLE_METRIC, "value": B * R * args.steps / wall, "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "rows": R, "vocab": V, "logits": "bf16",
                   "drafter": "probabilities" if w.draft_probs else "greedy", "penalties": w.penalties,
                   "accept_mean": acc_mean, "rotating_copies": M},
        "gbps": nb * args.steps / wall / 1e9, "hbm_frac": nb * args.steps / wall / 1e9 / HBM_PEAK_GBPS,
        "kernels": {"accept_sample": {"avg_us": tcall * 1e6, "bytes": nb, "gbps": ach}},
        "roofline": {"bound": "hbm", "kernel": "accept_sample (stats + draw kernels)", "achieved": ach,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(w.name, "-", "accept_sample")},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = sample_cpu_baseline(w, d, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def run_stack(args, w):
    """A hybrid stack slice: every step verifies the batch through each of the
    w.layers GDN layers (one pool per layer) and then commits all layers, one
    launch per layer or all in one launch (--stack-commit fused); with the
    fused schedule, each layer's commit of the previous step runs inside its
    verify of this one (one gdn_spec_commit_verify launch per layer)."""
    import numpy as np
    import torch

    import gpu_harness as gh
    from linear_attention_verify_amd import binding as bd
    from linear_attention_verify_amd import workloads as wl

    if args.graph or args.accept != "given" or args.calibrate_copy:
        raise SystemExit("--graph, --accept and --calibrate-copy apply to single-layer workloads")
    sid, acc = wl.draw_requests(w)
    stream = torch.cuda.current_stream()
    layers = [gh.make_device_case(w, l, sid, acc, mode=args.mode) for l in range(w.layers)]
    prepared = [bd.Prepared(c.desc, c.ssm, c.conv, c.conv_w, c.x, c.alpha, c.beta, c.slot_ids, c.accept,
                            w.rows, c.mode, c.scratch, c.out, c.err, stream) for c in layers]
    c0 = layers[0]
    fused = bd.PreparedCommitLayers(c0.desc, [(c.ssm, c.conv, c.scratch) for c in layers], c0.slot_ids,
                                    c0.accept, w.rows, args.mode, c0.err, stream)
    cv = args.schedule == "fused"
    csteps = []
    if cv:
        ident = torch.arange(w.batch, dtype=torch.int32, device="cuda")
        for c, p in zip(layers, prepared):
            alt = torch.empty_like(c.scratch)
            csteps.append([[bd.PreparedCommitVerify(c.desc, c.ssm, c.conv, c.conv_w, c.x, c.alpha, c.beta,
                                                    c.slot_ids, w.rows, dst, ident, src, c.slot_ids, c.accept,
                                                    c.out, c.err, stream, mode=args.mode)
                            for dst, src in ((alt, c.scratch), (c.scratch, alt))], 0])
            p.verify()   # the step before the first: its commit is pending
    torch.cuda.synchronize()

    def verifies():
        for k, p in enumerate(prepared):
            if cv:
                pair, i = csteps[k]
                pair[i]()
                csteps[k][1] = 1 - i
            else:
                p.verify()

    def commits():
        if cv:
            return
        if args.stack_commit == "fused":
            fused()
        else:
            for p in prepared:
                p.commit()

    def step():
        verifies()
        commits()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if any(int(c.err.item()) for c in layers):
        raise SystemExit("device error flags set")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-phase durations in a second pass with HIP events on the launch stream:
    # around each step's L verifies, and around its commits
    ev_v, ev_c = [], []
    for _ in range(args.steps):
        a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record(stream)
        verifies()
        b.record(stream)
        commits()
        c.record(stream)
        ev_v.append((a, b))
        ev_c.append((b, c))
    torch.cuda.synchronize()
    tv = np.array([a.elapsed_time(b) for a, b in ev_v]) * 1e-3 / w.layers
    tc = np.array([a.elapsed_time(b) for a, b in ev_c]) * 1e-3
    vb, cb = algorithmic_bytes(w, acc, args.mode)
    L = w.layers
    rows_per_step = w.batch * w.rows * L
    if cv:
        fb = fused_bytes(w, acc, args.mode)
        gbps = fb * L * args.steps / wall / 1e9
        kernels = {"commit_verify": {"avg_us": float(tv.mean() * 1e6), "bytes": fb,
                                     "gbps": float(fb / tv.mean() / 1e9)}}
        dom = "commit_verify"
    else:
        gbps = (vb + cb) * L * args.steps / wall / 1e9
        kernels = {"verify": {"avg_us": float(tv.mean() * 1e6), "bytes": vb, "gbps": float(vb / tv.mean() / 1e9)},
                   "commit_all_layers": {"avg_us": float(tc.mean() * 1e6), "bytes": cb * L,
                                         "gbps": float(cb * L / tc.mean() / 1e9)}}
        dom = "commit_all_layers" if tc.mean() >= tv.mean() * L else "verify"
    line = {
        "metric": METRIC, "value": rows_per_step * args.steps / wall, "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "rows": w.rows, "layers": L,
                   "key_heads": w.shape.num_k_heads, "value_heads": w.shape.num_v_heads,
                   "head_dim": w.shape.d_k, "conv_width": w.shape.conv_width, "storage": w.shape.dtype,
                   "state": "f32", "pool_slots": w.num_slots, "commit_mode": args.mode,
                   "commit_launch": "with each verify" if cv else args.stack_commit,
                   "schedule": args.schedule, "accept_mean": float(np.mean(acc))},
        "gbps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS, "kernels": kernels,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["gbps"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": kernels[dom]["gbps"] / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(w.name, args.mode, dom)},
    }
    if cv:
        sb = (vb + cb) * L
        line["serial_equivalent"] = {
            "bytes": sb, "gbps": sb * args.steps / wall / 1e9, "frac": sb * args.steps / wall / 1e9 / HBM_PEAK_GBPS,
            "note": "the serial verify + commit pairs' algorithmic bytes over this step's time: the rate the "
                    "serial schedule would need to match it; the fused launches move fewer bytes (gbps, roofline)"}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="saturated-b64")
    ap.add_argument("--mode", default="replay", choices=["replay", "snapshot"])
    ap.add_argument("--copies", type=int, default=16,
                    help="independent copies of the workload the steps rotate over; with 16, a "
                         "copy's inputs, state and scratch have left every cache when it comes round")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--stack-commit", default="per-layer", choices=["fused", "per-layer"],
                    help="multi-layer workloads: commit all layers in one launch or one per layer")
    ap.add_argument("--accept", default="given", choices=["given", "greedy"],
                    help="given: the commit reads the workload's drawn accept lengths; greedy: each "
                         "step runs device-side greedy acceptance on draft/target tokens that realise "
                         "them, and the commit reads its output")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a captured HIP graph of each group of steps instead of "
                         "eager launches (steps and warmup must be multiples of --copies)")
    ap.add_argument("--schedule", default=None, choices=["serial", "overlap", "fused"],
                    help="serial: every launch on one stream; overlap: a group's commits on a second "
                         "stream, each copy's next verify waiting for its own commit, so one group's "
                         "commits run beside the next group's verifies (pays in long runs of large "
                         "replay batches; the pipeline's fill and drain cost more over a few steps); "
                         "fused: each step is one gdn_spec_commit_verify launch that commits the copy's "
                         "previous step into the state on its way into this step's verify ("
                         "every step still commits one batch and verifies one). Default: fused with eager "
                         "launches on the layers it serves (bf16, d = 128, an even number of value heads "
                         "per key head), serial otherwise")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 256 MiB device copy (the reference dispatch for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py runs on one GPU: the verify/commit path has no cross-GPU step "
              "(requests and value heads shard with no exchange); --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gpu_harness as gh
    from linear_attention_verify_amd import binding as bd
    from linear_attention_verify_amd import workloads as wl

    torch.cuda.init()
    if args.workload in wl.ATTN_WORKLOADS:
        return run_attention(args, wl.ATTN_WORKLOADS[args.workload])
    if args.workload in wl.SAMPLE_WORKLOADS:
        return run_sample(args, wl.SAMPLE_WORKLOADS[args.workload])
    w = wl.WORKLOADS[args.workload]
    if args.schedule is None:
        s = w.shape
        fits = s.dtype == "bf16" and s.d_k == 128 and (s.num_v_heads // s.num_k_heads) % 2 == 0
        args.schedule = "fused" if not args.graph and fits else "serial"
    if w.layers != 1:
        return run_stack(args, w)
    if args.calibrate_copy:
        calibration_copy()
    M = max(1, args.copies)
    base = gh.make_case(w, mode=args.mode)
    cases = [base]
    for _ in range(M - 1):
        c = gh.make_case(w, mode=args.mode, draw=base.draw)
        cases.append(c)
    stream = torch.cuda.current_stream()
    prepared = [bd.Prepared(c.desc, c.ssm, c.conv, c.conv_w, c.x, c.alpha, c.beta, c.slot_ids,
                            c.accept, w.rows, c.mode, c.scratch, c.out, c.err, stream)
                for c in cases]
    overlap = args.schedule == "overlap"
    fused = args.schedule == "fused"
    if overlap and args.graph:
        raise SystemExit("--graph captures one stream: use --schedule serial")
    if fused and args.graph:
        raise SystemExit("--schedule fused: eager launches")
    vstream, cstream = (torch.cuda.Stream(), torch.cuda.Stream()) if overlap else (stream, stream)
    pv = [bd.Prepared(c.desc, c.ssm, c.conv, c.conv_w, c.x, c.alpha, c.beta, c.slot_ids, c.accept, w.rows,
                      c.mode, c.scratch, c.out, c.err, vstream) for c in cases] if overlap else prepared
    pc = [bd.Prepared(c.desc, c.ssm, c.conv, c.conv_w, c.x, c.alpha, c.beta, c.slot_ids, c.accept, w.rows,
                      c.mode, c.scratch, c.out, c.err, cstream) for c in cases] if overlap else prepared
    committed = [torch.cuda.Event() for _ in range(M)]
    accepts = [None] * M
    if args.accept == "greedy":
        draft, target = wl.draw_tokens(w, base.accept_np)
        for k, c in enumerate(cases):
            dt = torch.from_numpy(draft).cuda()
            tt = torch.from_numpy(target).cuda()
            nxt = torch.empty(w.batch, dtype=torch.int32, device="cuda")
            c.accept.zero_()
            accepts[k] = bd.PreparedAccept(dt, tt, c.slot_ids, w.rows, c.accept, nxt, cstream)
    accepts_serial = [None if a is None or not overlap else
                      bd.PreparedAccept(*a._keep[:3], w.rows, *a._keep[3:], stream) for a in accepts]
    # fused schedule: two scratch buffers per copy, alternating between the
    # step that is verified and the step whose commit is pending; each
    # copy's first verify (untimed, before the warmup) leaves a pending commit
    fsteps = []
    if fused:
        ident = torch.arange(w.batch, dtype=torch.int32, device="cuda")
        for c, p in zip(cases, prepared):
            alt = torch.empty_like(c.scratch)
            pair = [bd.PreparedCommitVerify(c.desc, c.ssm, c.conv, c.conv_w, c.x, c.alpha, c.beta, c.slot_ids,
                                            w.rows, dst, ident, src, c.slot_ids, c.accept, c.out, c.err, stream,
                                            mode=args.mode)
                    for dst, src in ((alt, c.scratch), (c.scratch, alt))]
            fsteps.append([pair, 0])
            p.verify()
    torch.cuda.synchronize()

    def fused_step(k):
        pair, i = fsteps[k]
        pair[i]()
        fsteps[k][1] = 1 - i

    graph = None
    if args.graph:
        if args.steps % M or args.warmup % M:
            raise SystemExit("--graph: --steps and --warmup must be multiples of --copies")
        cap = torch.cuda.Stream()
        on_cap = [bd.Prepared(c.desc, c.ssm, c.conv, c.conv_w, c.x, c.alpha, c.beta, c.slot_ids,
                              c.accept, w.rows, c.mode, c.scratch, c.out, c.err, cap)
                  for c in cases]
        acc_cap = [None if a is None else bd.PreparedAccept(*a._keep[:3], w.rows, *a._keep[3:], cap)
                   for a in accepts]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            for p in on_cap:
                p.verify()
            for a in acc_cap:
                if a is not None:
                    a()
            for p in on_cap:
                p.commit()
        torch.cuda.synchronize()

    def run_overlapped(nsteps):
        """nsteps steps in groups of M copies on two streams: the group's
        verifies on one, then (once every verify of the group is done, as
        sampling needs the last layer) its acceptances and commits on the
        other; a copy's next verify waits for that copy's commit. So one
        group's commits run beside the next group's verifies, and every data
        dependency of the serial order is kept."""
        s = 0
        while s < nsteps:
            group = list(range(s, min(s + M, nsteps)))
            for k in group:
                vstream.wait_event(committed[k % M])
                pv[k % M].verify()
            verified = torch.cuda.Event()
            verified.record(vstream)
            cstream.wait_event(verified)
            for k in group:
                if accepts[k % M] is not None:
                    accepts[k % M]()
            for k in group:
                pc[k % M].commit()
                committed[k % M].record(cstream)
            s += len(group)

    def run(nsteps, marks=None):
        """nsteps steps in groups of M copies: the group's verifies, then its
        acceptances (if any), then its commits. With `marks`, HIP events on the
        launch stream bracket each of the three phases of every group (always
        one stream: each kernel's launches back to back)."""
        if graph is not None and marks is None:
            for _ in range(nsteps // M):
                graph.replay()
            return
        if overlap and marks is None:
            return run_overlapped(nsteps)
        s = 0
        while s < nsteps:
            group = list(range(s, min(s + M, nsteps)))
            ev = []

            def mark():
                if marks is not None:
                    e = torch.cuda.Event(enable_timing=True)
                    e.record(stream)
                    ev.append(e)
            mark()
            for k in group:
                if fused:
                    fused_step(k % M)
                else:
                    prepared[k % M].verify()
            mark()
            for k in group:
                if accepts[k % M] is not None:
                    (accepts_serial[k % M] or accepts[k % M])()
            mark()
            for k in group:
                if not fused:
                    prepared[k % M].commit()
            mark()
            if marks is not None:
                marks.append((len(group), ev))
            s += len(group)

    run(args.warmup)
    torch.cuda.synchronize()

    # timed region: exactly K steps, wall clock bracketed by synchronisation.
    # The device error flags are read after the timed passes (they are
    # sticky), so that no host reads sit between the warmup and the region.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the same K steps again, eagerly, with HIP events on the launch stream around
    # each phase of each group: a kernel's average duration is its phase time
    # over the launches in it (back-to-back launches, as in the timed region)
    marks = []
    run(args.steps, marks)
    torch.cuda.synchronize()
    launches = sum(n for n, _ in marks)
    phase = [sum(ev[i].elapsed_time(ev[i + 1]) for _, ev in marks) * 1e-3 / launches for i in range(3)]
    tv, ta, tc = (np.array(x) for x in phase)
    errs = torch.stack([c.err for c in cases]).cpu().numpy().ravel().tolist()
    if any(errs):
        raise SystemExit("device error flags set: %s" % errs)

    vbytes, cbytes = algorithmic_bytes(w, base.accept_np, args.mode)
    rows_per_step = w.batch * w.rows
    value = rows_per_step * args.steps / wall
    if fused:
        fbytes = fused_bytes(w, base.accept_np, args.mode)
        gbps = fbytes * args.steps / wall / 1e9
        kernels = {"commit_verify": {"avg_us": float(tv.mean() * 1e6), "bytes": fbytes,
                                     "gbps": float(fbytes / tv.mean() / 1e9)}}
        dom = "commit_verify"
    else:
        gbps = (vbytes + cbytes) * args.steps / wall / 1e9
        kernels = {
            "verify": {"avg_us": float(tv.mean() * 1e6), "bytes": vbytes,
                       "gbps": float(vbytes / tv.mean() / 1e9)},
            "commit": {"avg_us": float(tc.mean() * 1e6), "bytes": cbytes,
                       "gbps": float(cbytes / tc.mean() / 1e9)},
        }
        dom = "verify" if tv.mean() >= tc.mean() else "commit"
    if args.accept == "greedy":
        kernels["accept_greedy"] = {"avg_us": float(ta * 1e6)}
    ach = kernels[dom]["gbps"]
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "rows": w.rows,
                   "key_heads": w.shape.num_k_heads, "value_heads": w.shape.num_v_heads,
                   "head_dim": w.shape.d_k, "conv_width": w.shape.conv_width,
                   "storage": w.shape.dtype, "state": "f32", "pool_slots": w.num_slots,
                   "commit_mode": args.mode, "accept_mean": float(np.mean(base.accept_np)),
                   "rotating_copies": M, "launch": "hip graph" if args.graph else "eager",
                   "schedule": args.schedule, "accept": args.accept},
        "gbps": gbps,
        "hbm_frac": gbps / HBM_PEAK_GBPS,
        "kernels": kernels,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(w.name, args.mode, dom)},
    }
    if fused:
        sb = vbytes + cbytes
        line["serial_equivalent"] = {
            "bytes": sb, "gbps": sb * args.steps / wall / 1e9, "frac": sb * args.steps / wall / 1e9 / HBM_PEAK_GBPS,
            "note": "the serial verify + commit pair's algorithmic bytes over this step's time: the rate a verify "
                    "then a commit would need to match it; the fused launch moves fewer bytes (gbps, roofline)"}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
