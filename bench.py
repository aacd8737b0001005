"""Benchmark: one rank's sharded mixed-precision AdamW step on one MI355X.

Workload (the 10B-parameter FlatParameter over N=8 ranks, rank 7's shard of
1.25e9 parameters, slot offset 8.75e9): a pre-reduced fp16 gradient shard
~N(0,1e-3) is unscaled (static scale 2^16), checked for overflow and reduced
to the global L2 norm, clipped at 1.0, and the fused AdamW step updates the
fp32 master/m/v shard and writes the fp16 parameters into the rank's slot of a
full 20 GB All-Gather buffer.  Inputs are synthetic (seeded, generated on the
GPU before timing) and resident in HBM when the timed region starts.

A "step" is the whole path: statistics kernel + fold, the AdamW update, and
the loss-scaler finalize.  The AdamW update is the dominant kernel (for this
shard one launch of the counter-scheduled kernel); its duration is taken with
HIP events on the launch stream around every call.  Where the
step's arrays land in physical memory moves every streaming kernel on them,
so the arrays are allocated afresh three times, each allocation running the
warm-up and the timed steps; `value` and `roofline` cover all of them and
`allocations` lists each with the median and minimum.  The same process
measures the practical ceilings: read-only, write-only and copy streams over
4 GiB, and on the step's own arrays the update's byte mix and a plain copy,
each in three launch forms (one launch, launch slices, slices with two blocks
per compute unit) with the fastest kept; `roofline` gives the AdamW rate
against 8 TB/s, against each of these, and against the fastest read-only and
write-only rates taken back to back for its 14 B read and 14 B written per
parameter.

Also timed, each as whole steps: the other workloads (8- and 64-way reduces,
the 70B INT8 shard, the 7B block, the Tiny MLP, gradient accumulation over 2
micro-steps, INT8-quantised rank gradients; for the 16-bit reduces also the
reduce call alone, against its bytes at the read-only and write-only ceilings
back to back), the ZeRO-Offload step (the
update on host cores), and the INT8 All-Gather consumer (gathered slots
dequantised into the full flat parameter) on the 7B block and the whole 70B
flat parameter.  The oracle is timed on one host core beside the headline and
beside every other workload (the full shard for the Tiny MLP, the 1.5B/64
shard and the 7B block; a window of the shard for the others).

Prints ONE JSON line.  --gpus N with N > 1 exits: the library runs one rank's
step on one GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
ADAM_BYTES_PER_PARAM = {        # algorithmic bytes of one AdamW-kernel launch per parameter
    "f16": 2 + 12 + 12 + 2,     # grad read, master/m/v read+write, 16-bit slot write
    "f32": 4 + 12 + 12 + 2,
}
KERNEL_SOURCE = os.path.join(ROOT, "fsdp_sharded_mixed_flatparameter_amd", "csrc",
                             "zeroflat_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "adamw_10b_n8_hbm_traffic.txt")
N_ALLOC = 3                     # fresh allocations of the headline step's arrays
VARIANTS = (   # the other workloads, whole steps each (parity cases in tests/ as well)
    ("10b_n8_reduce8", "10B/8 rank-7 shard with the 8 raw fp16 rank slices reduced (AVG) in the step"),
    ("70b_n64_int8", "70B/64 rank-63 shard (1.09e9), pre-reduced bf16, clipping active, bf16 "
                     "write-back + INT8 blocks of 256"),
    ("gpt1p5b_n64", "1.5B/64 rank-0 shard (2.34e7), 64 fp16 rank slices reduced (AVG), dynamic scale"),
    ("llama7b_block_n8", "Llama-7B block (2.02e8 params)/8 rank-3 shard, 8 bf16 rank slices (AVG)"),
    ("tiny_mlp_n4", "2-layer MLP (1.05e6 params)/4 rank-0 shard, 4 fp16 rank slices (AVG); "
                    "launch-bound"),
    ("10b_n8_accum2", "10B/8 rank-7 shard, gradient accumulation over 2 micro-steps: each "
                      "reduces 8 fp16 rank slices (AVG) into the fp32 shard, then the step"),
    ("10b_n8_qg", "10B/8 rank-7 shard, the 8 ranks' gradient slices arriving INT8-quantised "
                  "(blocks of 256, quantised before timing) and reduced (AVG), then the step"),
    ("gpt1p5b_n64_qg", "1.5B/64 rank-0 shard, 64 INT8-quantised rank gradient slices reduced "
                       "(AVG), dynamic scale"),
)
GATHER_VARIANTS = (   # the INT8 All-Gather consumer: gathered slots -> full flat parameter
    ("llama7b_block_n8_gather", "Llama-7B block flat parameter (2.02e8) from 8 INT8 slots "
                                "(block 256) to bf16"),
    ("70b_n64_gather", "the whole 70B flat parameter (7e10) from 64 INT8 slots (block 256) "
                       "to bf16"),
)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the other workloads")
    ap.add_argument("--no-reduce-call", action="store_true",
                    help="skip timing the 16-bit reduces alone (keeps a profiled run's launches "
                         "to the steps)")
    ap.add_argument("--only", default="",
                    help="comma-separated workloads to run alone (10b_n8 for the headline, a "
                         "variant, 10b_n8_reduce8_shift1, tiny_mlp_n4_graph, offload or a "
                         "gather), for per-workload profiles; the line then holds just those")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="accepted for older command lines: the calibration kernels (the "
                         "counters' copy reference and the ceilings) now always run")
    return ap.parse_args()


def kernel_source_hash():
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def read_traffic():
    """HBM bytes per AdamW launch from the committed rocprofv3 counter runs,
    or None if they were taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, window=1 << 26, steps=5):
    """The oracle as it stands, single-threaded, on a window of the same
    shard (same generator, same hyper-parameters), generation untimed."""
    import numpy as np

    from oracle import oracle as orc
    from synth import synth
    from synth.workloads import key_grad_reduced, key_master
    start = w.start
    p = synth.normal_f32(key_master(w), start, window, w.master_sigma, threads=8)
    m = np.zeros(window, np.float32)
    v = np.zeros(window, np.float32)
    grads = [synth.normal(key_grad_reduced(w, s), start, window, w.grad_sigma, w.grad_dtype,
                          threads=8) for s in range(steps)]
    sc = orc.make_scaler(w.loss_scale, w.dynamic, w.window)
    hp = orc.Hparams(**w.hp)
    # the oracle is single-threaded; pin the process to one core while it runs
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    try:
        t0 = time.perf_counter()
        for s in range(steps):
            orc.shard_step(grad=grads[s], grad_dtype=w.grad_dtype, master=p, exp_avg=m,
                           exp_avg_sq=v, scaler=sc, hp=hp, param_dtype=w.param_dtype)
        dt = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, allowed)
    return {"value": window * steps / dt, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": "%d-parameter window of the rank-7 shard (elements %d..), %d steps of "
                      "the oracle's statistics + AdamW + fp16 write-back, one thread pinned to "
                      "core %d; %.1f s" % (window, start, steps, core, dt),
            "host": {"cpu_model": cpu_model(), "cores_available": len(allowed)}}


# The oracle on every other workload: the full shard where the oracle finishes
# in seconds (the Tiny MLP, the 1.5B/64 shard, the 7B block), else a window of
# the same shard; (window or None, steps).
CPU_SAMPLES = {
    "tiny_mlp_n4": (None, 10),
    "gpt1p5b_n64": (None, 1),
    "llama7b_block_n8": (None, 2),
    "10b_n8_reduce8": (1 << 24, 2),
    "70b_n64_int8": (1 << 24, 3),
    "10b_n8_accum2": (1 << 24, 1),
    "10b_n8_qg": (1 << 24, 2),
    "gpt1p5b_n64_qg": (1 << 22, 2),
}


def _host_normal(torch, key, start, n, sigma, dtype):
    """Host array of the seeded generator's values (filled by the generator's
    device implementation, which is bit-identical to its host one, then
    copied down: input generation is not timed)."""
    import numpy as np
    from synth import synth
    tdt = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}[dtype]
    t = torch.empty(n, dtype=tdt, device="cuda")
    synth.fill_normal(t, key, start, sigma)
    if dtype == 0:
        return t.cpu().numpy()
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def cpu_baseline_workload(torch, w, window, steps):
    """The oracle as it stands on one workload's step (the same inputs as the
    GPU variant: the step-0 gradients, reused every step), one thread pinned
    to one core; inputs generated first, untimed."""
    import numpy as np

    from oracle import oracle as orc
    from synth.workloads import key_grad, key_grad_micro, key_grad_reduced, key_master
    n = w.shard if window is None else min(window, w.shard)
    start = w.start
    p = _host_normal(torch, key_master(w), start, n, w.master_sigma, 0)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    sc = orc.make_scaler(w.loss_scale, w.dynamic, w.window)
    hp = orc.Hparams(**w.hp)
    gd = w.grad_dtype
    if w.grad_int8:   # the senders' quantisation of their slices (not timed)
        qs, ss = [], []
        for k in range(w.n_ranks):
            q, s_ = orc.quant_int8(_host_normal(torch, key_grad(w, 0, k), start, n, w.grad_sigma,
                                                gd), gd, 256)
            qs.append(q)
            ss.append(s_)
    elif w.micro_steps > 1:
        micro = [[_host_normal(torch, key_grad_micro(w, 0, mi, k), start, n, w.grad_sigma, gd)
                  for k in range(w.n_ranks)] for mi in range(w.micro_steps)]
    elif w.reduce:
        bufs = [_host_normal(torch, key_grad(w, 0, k), start, n, w.grad_sigma, gd)
                for k in range(w.n_ranks)]
    else:
        g = _host_normal(torch, key_grad_reduced(w, 0), start, n, w.grad_sigma, gd)
    torch.cuda.empty_cache()

    def one():
        if w.grad_int8:
            grad, gdt = orc.reduce_q8(qs, ss, n, 256, w.op), orc.F32
        elif w.micro_steps > 1:
            grad, gdt = orc.reduce(micro[0], gd, 0, n, w.op), orc.F32
            for mi in range(1, w.micro_steps):
                orc.reduce_accumulate(micro[mi], gd, 0, n, w.op, grad)
        elif w.reduce:
            grad, gdt = orc.reduce(bufs, gd, 0, n, w.op), orc.F32
        else:
            grad, gdt = g, gd
        orc.shard_step(grad=grad, grad_dtype=gdt, master=p, exp_avg=m, exp_avg_sq=v, scaler=sc,
                       hp=hp, param_dtype=w.param_dtype, quant_block=w.quant_block or None)

    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    try:
        t0 = time.perf_counter()
        for _ in range(steps):
            one()
        dt = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, allowed)
    what = "full %d-parameter shard" % n if window is None or n == w.shard else \
        "%d-parameter window of the %d-parameter shard" % (n, w.shard)
    return {"value": n * steps / dt, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": "%s, %d step(s) of the oracle's whole step, one thread pinned to core %d; "
                      "%.1f s" % (what, steps, core, dt)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def run_prereduced(zf, torch, w, steps, warmup):
    """The headline workload: pre-reduced fp16 shard -> statistics -> AdamW."""
    from synth import synth
    from synth.workloads import key_grad_reduced, key_master
    S, dev = w.shard, torch.device("cuda:0")
    f16 = torch.float16
    master = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_normal(master, key_master(w), w.start, w.master_sigma)
    opt = zf.ShardOptimizer(master, w.hp, loss_scale=w.loss_scale, dynamic=w.dynamic)
    grads = []
    for s in range(2):   # two distinct pre-reduced gradient shards, alternated
        g = torch.empty(S, dtype=f16, device=dev)
        synth.fill_normal(g, key_grad_reduced(w, s), w.start, w.grad_sigma)
        grads.append(g)
    ag = torch.zeros(w.padded, dtype=f16, device=dev)      # full 20 GB All-Gather buffer
    torch.cuda.synchronize()

    ev = []

    def one_step(i, timed):
        g = grads[i % 2]
        zf.zero_unscale_norm(g, opt.state)
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        zf.zero_adamw_shard_step(g, opt.master, opt.exp_avg, opt.exp_avg_sq, ag, w.start,
                                 w.hp, opt.state, finalize=False)
        if timed:
            e1.record()
            ev.append((e0, e1))
        zf.zero_adamw_shard_step(g[:0], opt.master[:0], opt.exp_avg[:0], opt.exp_avg_sq[:0],
                                 ag, 0, w.hp, opt.state, finalize=True)   # scaler/counters

    for i in range(warmup):
        one_step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one_step(warmup + i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    adam_ms = [a.elapsed_time(b) for a, b in ev]
    st = opt.state.read()
    assert st.last_skipped == 0 and st.step == warmup + steps, "unexpected skipped step"
    res = dict(wall=wall, adam_ms=adam_ms, norm=st.last_norm)
    # after the timed steps: the update's byte mix with trivial arithmetic on
    # these same arrays (same physical placement), the kernel's own ceiling
    n = S // 1024 * 1024
    slot = ag[w.start:w.start + n]
    from synth import synth as _s
    mix_ms, mix_forms = _best_form(torch, lambda: _s.mix28(grads[0][:n], opt.master[:n],
                                                           opt.exp_avg[:n], opt.exp_avg_sq[:n],
                                                           slot), 5)
    res["mix"] = dict(bytes_per_launch=28 * n, ms_per_launch=mix_ms,
                      GBps=28 * n / (mix_ms * 1e-3) / 1e9,
                      GBps_by_form={k: 28 * n / (v * 1e-3) / 1e9 for k, v in mix_forms.items()},
                      what="the update's byte mix (fp16 g, fp32 p/m/v, fp16 copy of p; trivial "
                           "arithmetic, same lane layout) on the step's own arrays, after the "
                           "timed steps, fastest launch form")
    # and a plain copy between two of them (master into exp_avg; the state is
    # not used again): every streaming kernel on these arrays moves with their
    # physical placement, so this is the ceiling the update is compared with
    copy_ms, copy_forms = _best_form(torch, lambda: _s.copy(opt.master, opt.exp_avg), 5)
    res["copy"] = dict(bytes_per_launch=8 * S, ms_per_launch=copy_ms,
                       GBps=8 * S / (copy_ms * 1e-3) / 1e9,
                       GBps_by_form={k: 8 * S / (v * 1e-3) / 1e9 for k, v in copy_forms.items()},
                       what="plain non-temporal 16-byte copy of the fp32 master into exp_avg "
                            "(the step's own arrays), after the timed steps, fastest launch form")
    del opt, grads, ag, master
    torch.cuda.empty_cache()
    return res


def step_bytes_per_param(w):
    """Algorithmic HBM bytes of one whole step per shard parameter."""
    g16 = 2
    if w.grad_int8:
        stats_and_reduce = (1 + 4.0 / 256) * w.n_ranks + 4   # N INT8 payloads, fp32 shard written
        adam_grad = 4
    elif w.reduce:
        stats_and_reduce = g16 * w.n_ranks + 4          # N reads, fp32 reduced shard written
        # later micro-steps also read the accumulated fp32 shard back
        stats_and_reduce += (w.micro_steps - 1) * (g16 * w.n_ranks + 8)
        adam_grad = 4                                   # the fp32 reduced shard read back
    else:
        stats_and_reduce = g16                          # statistics pass over the 16-bit shard
        adam_grad = g16
    b = stats_and_reduce + adam_grad + 12 + 12 + 2      # master/m/v read+write, 16-bit slot
    if w.quant_block:
        b += 1 + 4.0 / w.quant_block                    # INT8 codes + one fp32 scale per block
    return b


FLUSHED = ("tiny_mlp_n4", "llama7b_block_n8")   # working sets within a few times the 256 MB cache


def run_workload(zf, torch, w, steps, warmup, flush=False, shift=0, time_reduce=True):
    """Whole steps of any workload (inputs generated on the GPU first).  With
    `flush`, a 512 MB scratch buffer is streamed before each timed step, so the
    step starts with none of its data in the 256 MB Infinity Cache, and each
    step is timed with HIP events around it; the back-to-back rate is kept
    beside it.  With `shift` > 0 the rank slices (reduce workloads) start that
    many elements into their buffers and the slot that many elements past its
    place in the All-Gather buffer: the layout of a shard size that is not a
    multiple of the vector width."""
    from synth import synth
    from synth.workloads import key_grad, key_grad_micro, key_grad_reduced, key_master
    S, dev = w.shard, torch.device("cuda:0")
    gdt = torch.float16 if w.grad_dtype == 1 else torch.bfloat16
    pdt = torch.float16 if w.param_dtype == 1 else torch.bfloat16
    master = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_normal(master, key_master(w), w.start, w.master_sigma)
    opt = zf.ShardOptimizer(master, w.hp, loss_scale=w.loss_scale, dynamic=w.dynamic,
                            window=w.window, quant_block=w.quant_block)
    if w.grad_int8:
        # each rank's fp16 slice quantised by the library (the sender's side,
        # outside the timed step): codes + one scale per 256 elements
        grads = ([], [])
        tmp = torch.empty(S, dtype=gdt, device=dev)
        for k in range(w.n_ranks):
            synth.fill_normal(tmp, key_grad(w, 0, k), w.start, w.grad_sigma)
            q_k = torch.empty(S, dtype=torch.int8, device=dev)
            s_k = torch.empty(-(-S // 256), dtype=torch.float32, device=dev)
            zf.zero_quant_allgather_slot(tmp, q_k, s_k)
            grads[0].append(q_k)
            grads[1].append(s_k)
        del tmp
    elif w.micro_steps > 1:
        # per micro-step, the rank-r slices of the N ranks' gradient buffers
        grads = []
        for mi in range(w.micro_steps):
            grads.append([])
            for k in range(w.n_ranks):
                b = torch.empty(S, dtype=gdt, device=dev)
                synth.fill_normal(b, key_grad_micro(w, 0, mi, k), w.start, w.grad_sigma)
                grads[mi].append(b)
    elif w.reduce:
        # rank-r slices of the N ranks' gradient buffers (slot-sized, offset 0,
        # or `shift` elements in)
        grads = []
        for k in range(w.n_ranks):
            b = torch.empty(S + shift, dtype=gdt, device=dev)
            synth.fill_normal(b[shift:], key_grad(w, 0, k), w.start, w.grad_sigma)
            grads.append(b)
    else:
        grads = torch.empty(S, dtype=gdt, device=dev)
        synth.fill_normal(grads, key_grad_reduced(w, 0), w.start, w.grad_sigma)
    if w.full_allgather:
        ag, off = torch.zeros(w.padded + shift, dtype=pdt, device=dev), w.start + shift
    else:
        ag, off = torch.zeros(S + shift, dtype=pdt, device=dev), shift
    q = qs = None
    if w.quant_block:
        q = torch.zeros(S, dtype=torch.int8, device=dev)
        qs = torch.zeros(-(-S // w.quant_block), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def one():
        if w.grad_int8:
            opt.step_from_int8_grads(grads[0], grads[1], ag, off, op=w.op, q_buf=q, q_scales=qs)
        elif w.micro_steps > 1:
            for mi in range(w.micro_steps):
                opt.micro_step(grads[mi], 0, op=w.op, first=mi == 0, last=mi == w.micro_steps - 1)
            opt.step_from_accumulated(ag, off, q_buf=q, q_scales=qs)
        elif w.reduce:
            opt.step_from_rank_buffers(grads, shift, ag, off, op=w.op, q_buf=q, q_scales=qs)
        else:
            opt.step_from_reduced(grads, ag, off, q_buf=q, q_scales=qs)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall / steps * 1e3
    flushed_ms = None
    if flush:
        scratch = torch.empty(512 << 18, dtype=torch.float32, device=dev)   # 512 MB
        evs = []
        for _ in range(steps):
            synth.write_stream(scratch)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            one()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        flushed_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
        del scratch
    st = opt.state.read()
    assert st.last_skipped == 0, "unexpected skipped step"
    reduce_call = None
    if time_reduce and w.reduce and not w.grad_int8 and w.micro_steps <= 1 and not flush:
        # the reduce with its statistics alone (its launches and the fold),
        # timed by HIP events on the stream it runs on, into the optimizer's
        # reduce buffer with a state of its own
        red, st2 = opt.reduced_buffer(), zf.StepState(w.loss_scale, False)
        rms = _event_ms_back_to_back(
            torch, lambda: zf.zero_grad_reduce_shard(grads, shift, S, w.op, red, st2),
            max(10, steps))
        nbytes = (w.n_ranks * grads[0].element_size() + 4) * S
        reduce_call = {"ms": rms, "bytes": nbytes,
                       "read_bytes": w.n_ranks * grads[0].element_size() * S,
                       "write_bytes": 4 * S, "GBps": nbytes / (rms * 1e-3) / 1e9,
                       "what": "zero_grad_reduce_shard with statistics alone (reduce_kernel "
                               "launches + fold), median of HIP-event-timed calls issued back to back"}
        if shift == 0:
            # the same N buffers read at once by a read-only calibration kernel
            # (N concurrent streams, the fastest launch form)
            sink = torch.zeros(1, dtype=torch.int32, device=dev)
            rbytes = grads[0].element_size() * S
            best, forms = _best_form(torch, lambda: synth.read_streams(grads, rbytes, sink),
                                     max(5, steps))
            reduce_call["read_same_buffers_GBps"] = w.n_ranks * rbytes / (best * 1e-3) / 1e9
            reduce_call["read_same_buffers_GBps_by_form"] = {
                k: w.n_ranks * rbytes / (v * 1e-3) / 1e9 for k, v in forms.items()}
            del sink
        del red, st2
    del opt, grads, ag, master, q, qs
    torch.cuda.empty_cache()
    bpp = step_bytes_per_param(w)
    res = {}
    if flush:
        res["ms_per_step_back_to_back"] = ms
        ms = flushed_ms
        res["cache"] = "flushed: 512 MB streamed before each timed step, the step timed by HIP events"
    res.update({"ms_per_step": ms, "params_per_s": S / (ms * 1e-3), "bytes_per_param": bpp,
                "step_GBps": bpp * S / (ms * 1e-3) / 1e9,
                "step_frac_of_peak": bpp * S / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS})
    if reduce_call:
        res["reduce_call"] = reduce_call
    return res


def add_reduce_bounds(variants, ceilings):
    """Each timed reduce against its bytes read and written at the same
    process's read-only and write-only ceilings, back to back."""
    for r in variants.values():
        rc = r.get("reduce_call")
        if not rc:
            continue
        t = (rc["read_bytes"] / (ceilings["read"]["GBps"] * 1e9) +
             rc["write_bytes"] / (ceilings["write"]["GBps"] * 1e9)) * 1e3
        rc["additive_read_write_ms"] = t
        rc["frac_of_additive_read_write"] = t / rc["ms"]
        if "read_same_buffers_GBps" in rc:
            # the same with the read side at the rate of these N buffers read at once
            t2 = (rc["read_bytes"] / (rc["read_same_buffers_GBps"] * 1e9) +
                  rc["write_bytes"] / (ceilings["write"]["GBps"] * 1e9)) * 1e3
            rc["additive_same_buffers_ms"] = t2
            rc["frac_of_additive_same_buffers"] = t2 / rc["ms"]


def run_graph(zf, torch, w, steps, warmup):
    """A whole step (reduce with statistics, AdamW, write-back, finalize)
    captured once as a HIP graph and replayed: for launch-bound shards."""
    from synth import synth
    from synth.workloads import key_grad, key_master
    S, dev = w.shard, torch.device("cuda:0")
    master = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_normal(master, key_master(w), w.start, w.master_sigma)
    opt = zf.ShardOptimizer(master, w.hp, loss_scale=w.loss_scale, dynamic=w.dynamic)
    grads = []
    for k in range(w.n_ranks):
        b = torch.empty(S, dtype=torch.float16, device=dev)
        synth.fill_normal(b, key_grad(w, 0, k), w.start, w.grad_sigma)
        grads.append(b)
    ag = torch.zeros(w.padded, dtype=torch.float16, device=dev)
    opt.step_from_rank_buffers(grads, 0, ag, w.start, op=w.op)      # warm-up, outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            opt.step_from_rank_buffers(grads, 0, ag, w.start, op=w.op)
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = opt.state.read()
    assert st.last_skipped == 0 and st.step == 1 + warmup + steps
    del graph, opt, grads, ag, master
    torch.cuda.empty_cache()
    ms = wall / steps * 1e3
    return {"ms_per_step": ms, "params_per_s": S / (ms * 1e-3),
            "what": "the same step captured once as a HIP graph and replayed"}


def run_gather(zf, torch, g, steps, warmup):
    """The INT8 All-Gather consumer on a gathered payload resident in HBM:
    every launch dequantises all n_ranks slots into the full flat buffer."""
    from synth import synth
    from synth.workloads import key_codes, key_scales
    out_dt = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}[g.out_dtype]
    es = torch.empty(0, dtype=out_dt).element_size()
    n_sc = g.n_ranks * g.n_blocks
    need = g.padded * (1 + es) + 4 * n_sc
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < need + (2 << 30):
        return {"skipped": "needs %.1f GB of device memory, %.1f GB free" % (need / 1e9, free / 1e9)}
    q = torch.empty(g.padded, dtype=torch.int8, device="cuda")
    synth.fill_codes(q, key_codes(g))
    sc = torch.empty(n_sc, device="cuda")
    synth.fill_normal(sc, key_scales(g), 0, g.scale_sigma)
    sc.abs_()
    out = torch.empty(g.padded, dtype=out_dt, device="cuda")
    torch.cuda.synchronize()
    for _ in range(warmup):
        zf.zero_dequant_allgather(q, sc, g.n_ranks, g.shard, out, block=g.block)
    ev = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        zf.zero_dequant_allgather(q, sc, g.n_ranks, g.shard, out, block=g.block)
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    del q, sc, out
    torch.cuda.empty_cache()
    gbps = need / (ms * 1e-3) / 1e9
    return {"ms_per_launch": ms, "wall_ms_per_launch": wall / steps * 1e3,
            "params_per_s": g.padded / (ms * 1e-3), "bytes_per_launch": need,
            "bytes_per_param": need / g.padded, "GBps": gbps, "frac_of_peak": gbps / PEAK_HBM_GBPS}


def run_offload(zf, torch, w, steps, warmup):
    """ZeRO-Offload on the same shard (the median of `steps` steps): statistics
    on the GPU, the fp16 gradient to pinned host memory in chunks, the update
    on host cores over host-resident fp32 master/m/v, the fp16 parameters back
    into the All-Gather slot.  Also the host link's own rates (pinned 2.5 GB
    copies each way) and the host threads' streaming rate, the two ceilings of
    this step."""
    from synth import synth
    from synth.workloads import key_grad_reduced, key_master
    S = w.shard
    # the update's threads leave two of the cores this process may use to the
    # HIP runtime's copy threads and this (Python) thread
    cores = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS", "0")) or cores
    threads = max(1, min(cap, cores) - 2)
    master = torch.empty(S, dtype=torch.float32)
    tmp = torch.empty(S, dtype=torch.float32, device="cuda")
    synth.fill_normal(tmp, key_master(w), w.start, w.master_sigma)
    master.copy_(tmp.cpu())
    del tmp
    opt = zf.OffloadShardOptimizer(master, w.hp, loss_scale=w.loss_scale, dynamic=w.dynamic,
                                   n_threads=threads)
    g = torch.empty(S, dtype=torch.float16, device="cuda")
    synth.fill_normal(g, key_grad_reduced(w, 0), w.start, w.grad_sigma)
    ag = torch.zeros(w.padded, dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()
    for _ in range(warmup):
        opt.step_from_reduced(g, ag, w.start)
    # each step returns when its copies and the device finalize are done
    per_step = []
    for _ in range(steps):
        t0 = time.perf_counter()
        opt.step_from_reduced(g, ag, w.start)
        per_step.append(time.perf_counter() - t0)
    wall = sorted(per_step)[len(per_step) // 2]       # the median step
    st = opt.state.read()
    assert st.last_skipped == 0 and st.step == warmup + steps
    # the host update alone (no copies), same threads, same arrays
    stage = opt._staging("grad", torch.float16)
    lp_out = torch.empty(S, dtype=torch.float16)
    best = 1e30
    for _ in range(2):
        t1 = time.perf_counter()
        zf.zero_offload_adamw_host(stage, opt.master, opt.exp_avg, opt.exp_avg_sq, lp_out, w.hp,
                                   st, threads)
        best = min(best, time.perf_counter() - t1)
    host_only = best
    # host link: pinned <-> device copies of the same 2.5 GB
    rates = {}
    for name, dst, src in (("d2h", stage, g), ("h2d", g, stage)):
        best = 1e30
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            dst.copy_(src, non_blocking=True)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        rates[name] = 2 * S / (best * 1e-3) / 1e9
    # host memory: a threaded streaming copy of the master array
    torch.set_num_threads(threads)
    buf = torch.empty_like(master)
    best = 1e30
    for _ in range(3):
        t1 = time.perf_counter()
        buf.copy_(master)
        best = min(best, time.perf_counter() - t1)
    host_copy = 2 * 4 * S / best / 1e9
    del opt, g, ag, master, buf, stage, lp_out
    torch.cuda.empty_cache()
    host_bytes = 2 + 12 + 12 + 2                  # grad read, master/m/v read+write, fp16 write
    return {"ms_per_step": wall * 1e3, "ms_each_step": [t * 1e3 for t in per_step],
            "params_per_s": S / wall, "host_threads": threads,
            "host_link_bytes_per_param": 4, "host_link_GBps": 4 * S / wall / 1e9,
            "host_link_ceiling_GBps": rates, "host_bytes_per_param": host_bytes,
            "host_GBps": host_bytes * S / wall / 1e9, "host_copy_ceiling_GBps": host_copy,
            "host_update_only_ms": host_only * 1e3,
            "host_update_only_GBps": host_bytes * S / host_only / 1e9,
            # the link's copies read and write the same host memory: 2 B of
            # gradient written and 2 B of parameters read per parameter on top
            # of the update's 28 B, at the update's own host-memory rate
            "host_memory_bound_ms": host_only * 1e3 * (host_bytes + 4) / host_bytes,
            "frac_of_host_memory_bound": host_only * (host_bytes + 4) / host_bytes / wall,
            "what": "10B/8 rank-7 shard offloaded: fp32 state in host memory, AdamW on %d host "
                    "threads, fp16 gradient down and fp16 parameters up over the host link"
                    % threads}


def _event_ms_back_to_back(torch, fn, reps):
    """Median ms of fn by HIP events around each call, the calls issued back
    to back (no host wait between them, so the launches' host time stays off
    the device's timeline); the first call is a warm-up."""
    fn()
    evs = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    return ms[len(ms) // 2]


# launch forms of the calibration streams: one launch, the library's launch
# slices of 32,768 blocks, and those slices with two resident blocks per
# compute unit (56 KiB of dynamic LDS reserved); a stream's ceiling is the
# fastest form
SLICE_BLOCKS, LDS_TWO_BLOCKS = 32768, 56 * 1024
LAUNCH_FORMS = (("one_launch", 0, 0), ("slices", SLICE_BLOCKS, 0),
                ("slices_two_blocks_per_cu", SLICE_BLOCKS, LDS_TWO_BLOCKS))


def _best_form(torch, fn, reps):
    """ms of fn in each launch form; (best ms, {form: ms})."""
    from synth import synth
    forms = {}
    for name, sl, lds in LAUNCH_FORMS:
        with synth.launch_form(sl, lds):
            forms[name] = _event_ms_back_to_back(torch, fn, reps)
    return min(forms.values()), forms


def run_ceilings(torch, nbytes=4 << 30, reps=5):
    """The practical HBM ceilings of this machine, measured in the same process as
    the step with the streaming calibration kernels of synth (non-temporal
    16-byte accesses, HIP events on the launch stream): read-only, write-only
    and copy, each in every launch form, the fastest kept (the one-launch
    copy's dispatches also calibrate the rocprofv3 byte counters).  The fused
    update's own byte mix is measured by run_prereduced on its arrays."""
    from synth import synth
    out = {}
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    for name, fn, moved in (("read", lambda: synth.read_stream(a, sink), nbytes),
                            ("write", lambda: synth.write_stream(b), nbytes),
                            ("copy", lambda: synth.copy(a, b), 2 * nbytes)):
        ms, forms = _best_form(torch, fn, reps)
        out[name] = dict(bytes_per_launch=moved, ms_per_launch=ms, GBps=moved / (ms * 1e-3) / 1e9,
                         GBps_by_form={k: moved / (v * 1e-3) / 1e9 for k, v in forms.items()})
    del a, b
    torch.cuda.empty_cache()
    out["what"] = ("synth calibration kernels, same process, read/write/copy over %d MiB, the "
                   "fastest of: one launch, launches of %d blocks, those with two blocks per "
                   "compute unit; adamw_mix runs on the step's own arrays"
                   % (nbytes >> 20, SLICE_BLOCKS))
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs one rank's step on a single MI355X "
              "(the other ranks are buffers in the same HBM); --gpus %d is not supported."
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import fsdp_sharded_mixed_flatparameter_amd as zf
    from synth.workloads import WORKLOADS
    w = WORKLOADS["10b_n8"]
    S = w.shard
    only = [x for x in args.only.split(",") if x]

    def sel(name):
        return not only or name in only

    if sel("10b_n8"):
        out = run_headline(zf, torch, w, args)
    else:
        out = {"only": only}
    if not args.no_variants:
        out["variants"] = {}
        for name, what in VARIANTS:
            if not sel(name):
                continue
            r = run_workload(zf, torch, WORKLOADS[name], max(3, args.steps // 2), 2,
                             flush=name in FLUSHED, time_reduce=not args.no_reduce_call)
            r["what"] = what
            if not args.no_cpu_baseline:
                r["cpu_baseline"] = cpu_baseline_workload(torch, WORKLOADS[name],
                                                          *CPU_SAMPLES[name])
                r["cpu_baseline"]["gpu_over_oracle"] = r["params_per_s"] / r["cpu_baseline"]["value"]
            out["variants"][name] = r
        # the same steps with every rank slice and the slot one element off
        # the vector boundary (rank r's slice starts at r*S for any S)
        for name, base in (("10b_n8_reduce8_shift1", "10b_n8_reduce8"),):
            if not sel(name):
                continue
            r = run_workload(zf, torch, WORKLOADS[base], max(3, args.steps // 2), 2, shift=1,
                             time_reduce=not args.no_reduce_call)
            r["what"] = ("as %s, with every rank slice starting 1 element into its buffer and "
                         "the slot 1 element past its place: the reduce's shifted vector path "
                         "and the update's joined slot words" % base)
            if base in out["variants"]:
                r["vs_aligned"] = out["variants"][base]["ms_per_step"] / r["ms_per_step"]
            out["variants"][name] = r
        if "ceilings" in out:
            add_reduce_bounds(out["variants"], out["ceilings"])
        if sel("tiny_mlp_n4_graph"):
            out["variants"]["tiny_mlp_n4_graph"] = run_graph(
                zf, torch, WORKLOADS["tiny_mlp_n4"], max(20, args.steps), 5)
        if sel("offload"):
            out["offload"] = run_offload(zf, torch, w, 5, 2)
        from synth.workloads import GATHERS
        out["allgather_consumer"] = {}
        for name, what in GATHER_VARIANTS:
            if not sel(name):
                continue
            r = run_gather(zf, torch, GATHERS[name], max(3, args.steps // 4), 1)
            r["what"] = what
            out["allgather_consumer"][name] = r
    if not args.no_cpu_baseline and sel("10b_n8"):
        out["cpu_baseline"] = cpu_baseline(w)
        out["cpu_baseline"]["gpu_over_oracle"] = out["value"] / out["cpu_baseline"]["value"]
    print(json.dumps(out), flush=True)


def run_headline(zf, torch, w, args):
    """The headline line: the 10B/8 step over N_ALLOC fresh allocations, with
    the ceilings measured in the same process."""
    S = w.shard
    ceilings = run_ceilings(torch)
    # the headline over N_ALLOC fresh allocations of the step's arrays: where
    # they land in physical memory moves every streaming kernel on them
    allocs = [run_prereduced(zf, torch, w, args.steps, args.warmup) for _ in range(N_ALLOC)]
    adam_bytes = ADAM_BYTES_PER_PARAM["f16"] * S
    step_bytes = (2 + ADAM_BYTES_PER_PARAM["f16"]) * S           # + the statistics pass
    each = []
    for r in allocs:
        ms = r["wall"] / args.steps * 1e3
        am = sum(r["adam_ms"]) / len(r["adam_ms"])
        each.append({"ms_per_step": ms, "params_per_s": S / (ms * 1e-3),
                     "adam_avg_launch_ms": am, "adam_GBps": adam_bytes / (am * 1e-3) / 1e9,
                     "adam_frac_of_peak": adam_bytes / (am * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                     "copy_step_arrays_GBps": r["copy"]["GBps"], "adamw_mix_GBps": r["mix"]["GBps"]})
    all_adam = [x for r in allocs for x in r["adam_ms"]]
    ms_step = sum(r["wall"] for r in allocs) / (N_ALLOC * args.steps) * 1e3
    adam_ms = sum(all_adam) / len(all_adam)
    achieved = adam_bytes / (adam_ms * 1e-3) / 1e9
    mean = lambda xs: sum(xs) / len(xs)
    ceilings["adamw_mix"] = dict(allocs[0]["mix"], GBps=mean([e["adamw_mix_GBps"] for e in each]),
                                 what=allocs[0]["mix"]["what"] + "; mean over the allocations")
    ceilings["copy_step_arrays"] = dict(allocs[0]["copy"],
                                        GBps=mean([e["copy_step_arrays_GBps"] for e in each]),
                                        what=allocs[0]["copy"]["what"] +
                                        "; mean over the allocations")
    # reads and writes share the HBM: the update's 14 B read and 14 B written
    # per parameter at the read-only and write-only rates, back to back
    rd = wr = 14 * S
    t_add = rd / (ceilings["read"]["GBps"] * 1e9) + wr / (ceilings["write"]["GBps"] * 1e9)
    additive = (rd + wr) / t_add / 1e9
    pps = sorted(e["params_per_s"] for e in each)
    agb = sorted(e["adam_GBps"] for e in each)
    out = {
        "metric": "sharded AdamW step: params updated/s and achieved HBM GB/s (% of peak) at 1 GPU",
        "value": S / (ms_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "10b_n8: 10B-param FlatParameter over 8 ranks, rank 7 shard "
                               "(1.25e9 params), pre-reduced fp16 grads, static loss scale 2^16, "
                               "clip 1.0, AdamW lr 3e-5 betas (0.9,0.999) eps 1e-8 wd 0.01, fp16 "
                               "write-back into the full All-Gather buffer at offset 8.75e9",
                   "shard_params": S, "n_ranks": w.n_ranks, "rank": w.rank,
                   "parallelism": "one rank's shard on 1 GPU"},
        "allocations": {"n": N_ALLOC, "each": each,
                        "params_per_s_median": pps[len(pps) // 2], "params_per_s_min": pps[0],
                        "adam_GBps_median": agb[len(agb) // 2], "adam_GBps_min": agb[0],
                        "what": "the step's arrays allocated afresh %d times, each running the "
                                "warm-up and the %d timed steps; value, ms_per_step and roofline "
                                "are over all of them" % (N_ALLOC, args.steps)},
        "step_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
        "step_frac_of_peak": step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "roofline": {"bound": "hbm",
                     "kernel": "adamw_sched_kernel<1, 1> (fused AdamW + fp16 write-back, one "
                               "counter-scheduled launch)",
                     "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": read_traffic(),
                     "algorithmic_bytes_per_launch": adam_bytes,
                     "avg_launch_ms": adam_ms,
                     "median_launch_ms": sorted(all_adam)[len(all_adam) // 2],
                     "min_launch_ms": min(all_adam),
                     "additive_read_write_GBps": additive,
                     "frac_of_additive_read_write": achieved / additive,
                     "frac_of_copy_ceiling": achieved / ceilings["copy"]["GBps"],
                     "frac_of_mix_ceiling": achieved / ceilings["adamw_mix"]["GBps"],
                     "frac_of_step_array_copy": achieved / ceilings["copy_step_arrays"]["GBps"]},
        "ceilings": ceilings,
    }
    return out


if __name__ == "__main__":
    main()
