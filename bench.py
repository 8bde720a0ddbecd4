"""Throughput of the segment-masked flash-attention forward on one MI355X.

One step = one vdx_attn_fwd_ws call (the forward with a resident workspace;
the whole hot path: tile scheduling, segment classification, QK^T, masking,
online softmax, PV, epilogue, and the merge of split items' parts) over one
batch of seeded synthetic input already resident in HBM; with --plain, one
vdx_attn_fwd call (no workspace: unmasked launches run a static persistent
grid and never split, masked ones run one workgroup per query block).  Steps call the C ABI through the binding with their
arguments prepared once (the tensor-level wrappers check them on a first,
untimed call), and the warm-up runs until the clock has settled (at least 3
steps and 1 s unless --warmup is given).  The default
workload is the 720p large-DiT layer (B=1, S=75,600 = 21x45x80 latent
patches, H=40, D=128, bf16, unmasked), the shape the throughput target is
quoted on.

Prints ONE JSON line:
  value        valid-pair TFLOP/s = 4*D*H*sum_b #valid(i,j) / (wall time per step)
  roofline     the attention kernel against the MI355X dense bf16 MFMA peak,
               with its average launch time from HIP events on its stream and
               the HBM traffic from rocprofv3 counters when they are current
  cpu_baseline the fp64 oracle timed on a bounded row sample on the host cores

With --pass bwd the step is one vdx_attn_bwd call (the gradient: delta/lse
prep, the key-major dK/dV kernel and the query-major dQ kernel) on the same
workload, given resident q, k, v, out, lse and a seeded dout; the FLOP count
is the algorithmic 10*D per valid pair and head (five products of 2*D:
scores, dP, dV, dK, dQ), of which the two-kernel split executes 14*D.

With --workload natten_vae_decoder (or natten_tiny) the step is one
vdx_natten3d_fwd call instead (3D neighbourhood attention over a t x h x w
grid), and the FLOP count is that of the window pairs: 4*D*H*B*S*|window|.

With --rope the step is one vdx_rope3d_attn_fwd_ws call on the workload: the 3D
rotary position embedding of the keys (a pre-pass into a resident buffer) and
of the queries (in the attention kernel's prologue), then the same attention;
the FLOP count is the attention's.

Every line also carries the graphics clock and socket power sampled with
amdsmi while the same step runs back to back for a few seconds after the
timed ones (null where amdsmi cannot read them), and the
CPU baseline's row rate with the extrapolated time of the whole workload on
the oracle (labelled as an extrapolation).

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME] [--pass fwd|bwd]
       [--rope] [--plain] [--no-cpu-baseline] [--copy-calib]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
METRIC = "attention TFLOP/s and % of bf16 MFMA peak at S=75,600 H=40 D=128 (1 GPU)"
BWD_METRIC = ("attention backward TFLOP/s (dq, dk, dv; 10*D flop per valid pair) and % of "
              "bf16 MFMA peak (1 GPU)")
NATTEN_METRIC = "3D neighbourhood attention TFLOP/s (window pairs) and % of bf16 MFMA peak (1 GPU)"
# The device code and launch configuration of each path (the C-ABI file only
# validates arguments and calls the launchers, so it is not part of them).
KERNEL_SOURCES = [os.path.join(ROOT, "spatiotemporal_attention_amd", "csrc", f)
                  for f in ("attn_fwd_kernel.hip", "attn_common.h", "attn_fwd_launch.h")]
BWD_KERNEL_SOURCES = [os.path.join(ROOT, "spatiotemporal_attention_amd", "csrc", f)
                      for f in ("attn_bwd_kernel.hip", "attn_common.h", "attn_fwd_launch.h")]
NATTEN_KERNEL_SOURCES = [os.path.join(ROOT, "spatiotemporal_attention_amd", "csrc", f)
                         for f in ("natten_fwd_kernel.hip", "attn_common.h", "attn_fwd_launch.h")]
COUNTERS_DIR = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def valid_pairs(w: W.Workload) -> int:
    """Number of (query, key) pairs that take part, summed over the batch."""
    if w.seg_runs is None:
        return w.B * w.S * w.S
    per_id = {}
    for a, b, sid in w.seg_runs:
        if sid != 0:
            per_id[sid] = per_id.get(sid, 0) + (b - a)
    return w.B * sum(n * n for n in per_id.values())


def algorithmic_bytes(w: W.Workload) -> int:
    """Bytes one call must move at least: read q, k, v (+ segs), write out and lse."""
    n = w.B * w.S * w.H * w.D
    b = 4 * 2 * n + 4 * w.B * w.H * w.S
    if w.seg_runs is not None:
        b += 2 * 4 * w.B * w.S
    return b


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload: str, pass_: str = "fwd"):
    """HBM bytes per launch (forward, neighbourhood forward) or per call
    (backward: its three kernels) from the committed rocprofv3 counter
    summary, or None when the summary is missing or was taken on different
    kernel source.  pass_ is "fwd", "bwd" or "natten"."""
    prefix, sources, key = {
        "fwd": ("attn_fwd", KERNEL_SOURCES, "traffic_bytes_per_launch"),
        "bwd": ("attn_bwd", BWD_KERNEL_SOURCES, "traffic_bytes_per_call"),
        "natten": ("natten_fwd", NATTEN_KERNEL_SOURCES, "traffic_bytes_per_launch"),
    }[pass_]
    name = workload.removeprefix("natten_") if pass_ == "natten" else workload
    path = os.path.join(COUNTERS_DIR, f"{prefix}_{name}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    if doc.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    return doc.get(key)


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5) -> None:
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {nbytes} bytes")


def cpu_baseline(w: W.Workload, x, target_s: float = 15.0):
    import oracle
    cores = oracle.default_threads()
    qb, kb, vb = W.bf16_bits(x["q"]), W.bf16_bits(x["k"]), W.bf16_bits(x["v"])
    sq = None if x["seg_q"] is None else x["seg_q"].numpy()
    sk = None if x["seg_kv"] is None else x["seg_kv"].numpy()
    rng = np.random.default_rng(7)

    def rows_for(n):
        b = rng.integers(0, w.B, n)
        h = rng.integers(0, w.H, n)
        i = rng.integers(0, w.S, n)
        return np.stack([b, h, i], 1).astype(np.int64)

    def flops(rows):
        if sq is None:
            return 4.0 * w.D * w.S * len(rows)
        tot = 0.0
        for b, _, i in rows:
            c = sq[b, i]
            if c != 0:
                tot += 4.0 * w.D * float(np.count_nonzero(sk[b] == c))
        return tot

    probe = rows_for(cores)
    t0 = time.perf_counter()
    oracle.attn_fwd(qb, kb, vb, sq, sk, float(np.float32(w.scale)), rows=probe, n_threads=cores)
    dt = time.perf_counter() - t0
    n = max(cores, int(cores * target_s / max(dt, 1e-3)))
    rows = rows_for(n)
    t0 = time.perf_counter()
    oracle.attn_fwd(qb, kb, vb, sq, sk, float(np.float32(w.scale)), rows=rows, n_threads=cores)
    dt = time.perf_counter() - t0
    rate = flops(rows) / dt / 1e12
    full = 4.0 * w.D * w.H * valid_pairs(w)
    return {"value": rate, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} random (b,h,i) rows of {w.name}, each over its full key set, "
                      f"{dt:.1f} s on {cores} threads",
            "rows_per_s": round(n / dt, 2),
            "extrapolated_full_workload_s": round(full / (rate * 1e12), 1),
            "extrapolation": "whole-workload oracle time = the workload's valid-pair FLOP / the sampled rate"}


def natten_window_volume(w) -> int:
    return math.prod(min(k, n) for k, n in zip(w.window, w.grid))


def natten_brick_frames(NT, NH, KT, KH) -> int:
    """Frames per query brick the kernel picks (its brick is BT x 8/BT x 32):
    the fewest window-union key rows per query row, ties to more frames."""
    kt, kh = min(KT, NT), min(KH, NH)
    best, best_rows, best_q = 1, 0, 1
    for bt in (1, 2, 4, 8):
        by = 8 // bt
        rows = min(bt + kt - 1, NT) * min(by + kh - 1, NH)
        q = min(bt, NT) * min(by, NH)
        if bt == 1 or rows * best_q <= best_rows * q:
            best, best_rows, best_q = bt, rows, q
    return best


def natten_executed_flop(w) -> float:
    """MFMA flops the kernel issues: per workgroup (a BT x 8/BT x 32 (t, y, x)
    query brick) one step per two key rows of its window union (an odd row
    count adds a masked row), each row 8 waves x 32 queries x 16 keys x 2
    products x 2*D."""
    NT, NH, NW = w.grid
    KT, KH, KW = w.window
    bt, by = natten_brick_frames(NT, NH, KT, KH), 8 // natten_brick_frames(NT, NH, KT, KH)

    def start(c, k, n):
        ke = min(k, n)
        return min(max(c - k // 2, 0), n - ke)

    def span(c0, brick, k, n):  # window-union length of a brick starting at c0
        return start(min(c0 + brick - 1, n - 1), k, n) + min(k, n) - start(c0, k, n)

    rows = 0
    for t0 in range(0, NT, bt):
        nt = span(t0, bt, KT, NT)
        for y0 in range(0, NH, by):
            rows += 2 * ((nt * span(y0, by, KH, NH) + 1) // 2)
    rows *= (NW + 31) // 32
    return float(rows) * w.B * w.H * 8 * 32 * 16 * 4 * w.D


def natten_cpu_baseline(w, x, target_s: float = 15.0):
    import oracle
    cores = oracle.default_threads()
    qb, kb, vb = W.bf16_bits(x["q"]), W.bf16_bits(x["k"]), W.bf16_bits(x["v"])
    rng = np.random.default_rng(7)

    def rows_for(n):
        return np.stack([rng.integers(0, w.B, n), rng.integers(0, w.H, n),
                         rng.integers(0, w.S, n)], 1).astype(np.int64)

    probe = rows_for(cores * 16)
    t0 = time.perf_counter()
    oracle.natten3d_fwd(qb, kb, vb, w.grid, w.window, float(np.float32(w.scale)), rows=probe,
                        n_threads=cores)
    dt = time.perf_counter() - t0
    n = max(cores, int(len(probe) * target_s / max(dt, 1e-3)))
    rows = rows_for(n)
    t0 = time.perf_counter()
    oracle.natten3d_fwd(qb, kb, vb, w.grid, w.window, float(np.float32(w.scale)), rows=rows,
                        n_threads=cores)
    dt = time.perf_counter() - t0
    rate = 4.0 * w.D * natten_window_volume(w) * n / dt / 1e12
    full = 4.0 * w.D * w.H * w.B * w.S * natten_window_volume(w)
    return {"value": rate, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} random (b,h,i) rows of {w.name}, each over its full window, "
                      f"{dt:.1f} s on {cores} threads",
            "rows_per_s": round(n / dt, 2),
            "extrapolated_full_workload_s": round(full / (rate * 1e12), 1),
            "extrapolation": "whole-workload oracle time = the workload's window-pair FLOP / the sampled rate"}


class ClockSampler:
    """Reads the GPU's current graphics clock (MHz) and socket power (W) with
    amdsmi every `period` seconds from a background thread while the timed
    steps run.  Any amdsmi failure leaves the summary null."""

    def __init__(self, period: float = 0.05):
        self.period = period
        self.clk, self.pwr = [], []
        self.err = None
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            bus = None
            props = torch.cuda.get_device_properties(torch.cuda.current_device())
            if hasattr(props, "pci_bus_id"):
                bus = int(props.pci_bus_id)
            for h in handles:
                try:
                    bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                    if bus is not None and int(bdf.split(":")[1], 16) == bus:
                        self._handle = h
                except Exception:  # pragma: no cover
                    pass
            if self._handle is None and len(handles) == 1:
                self._handle = handles[0]
            self._smi = amdsmi
        except Exception as e:  # pragma: no cover - no driver here
            self.err = f"{type(e).__name__}: {e}"

    def _run(self):
        smi = self._smi
        while not self._stop.is_set():
            try:
                c = smi.amdsmi_get_clock_info(self._handle, smi.AmdSmiClkType.GFX)
                self.clk.append(float(c["clk"]))
                p = smi.amdsmi_get_power_info(self._handle)
                w = p.get("current_socket_power", p.get("average_socket_power"))
                if isinstance(w, (int, float)):
                    self.pwr.append(float(w))
            except Exception as e:  # pragma: no cover
                self.err = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period)

    def __enter__(self):
        if self._handle is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def summary(self, skip: float = 0.5):
        """Median over the samples after the first `skip` fraction (the
        readings lag the load by a few hundred ms)."""
        if not self.clk:
            return {"gfx_clock_mhz_median": None, "source": "amdsmi", "error": self.err or "no handle"}
        k = int(len(self.clk) * skip)
        clk, pwr = self.clk[k:], self.pwr[k:]
        return {"gfx_clock_mhz_median": float(np.median(clk)),
                "socket_power_w_median": float(np.median(pwr)) if pwr else None,
                "samples": len(clk),
                "source": f"amdsmi current GFX clock and socket power every {self.period * 1e3:.0f} ms, "
                          f"over the second half of {CLOCK_WINDOW_S:.0f} s of back-to-back steps after "
                          f"the timed ones"}


CLOCK = {"summary": None}
CLOCK_WINDOW_S = 3.0


def clock_window(step, seconds: float = CLOCK_WINDOW_S):
    """Runs steps back to back for about `seconds` while sampling the clock
    (outside the timed region, so the sampling thread cannot disturb it)."""
    sampler = ClockSampler()
    with sampler:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(4):
                step()
            torch.cuda.synchronize()
    CLOCK["summary"] = sampler.summary()


def c_step(fn, *args):
    """One timed step: a direct call of a C-ABI entry point through the binding
    with every argument prepared beforehand (device addresses, sizes, the
    stream handle), so that the host issues launches faster than the GPU runs
    them and the events around a step time the launch, not the Python
    argument checks of the tensor-level wrappers."""
    def step():
        rc = fn(*args)
        if rc != 0:
            raise RuntimeError(f"{fn.__name__}: {status_str(rc)}")
    return step


WARMUP_SECONDS = 1.0


def warm_up(step, warmup):
    """Runs the untimed warm-up steps and returns how many ran: exactly
    `warmup` when given, else at least 3 and at least WARMUP_SECONDS of
    back-to-back steps, so that the shader clock and power have settled to
    their sustained values before the timed region (a short kernel's first
    launches run at a lower clock; a long power-limited one's at a higher)."""
    if warmup is not None:
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        return warmup
    n, t0 = 0, time.perf_counter()
    while n < 3 or time.perf_counter() - t0 < WARMUP_SECONDS:
        for _ in range(max(1, n)):
            step()
            n += 1
        torch.cuda.synchronize()
    return n


def time_steps(step, stream, steps, warmup, sample_clock=True):
    """(wall ms per step, mean kernel ms per step, warm-up steps run)."""
    warmup = warm_up(step, warmup)
    log(f"warmup done ({warmup} steps)")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if sample_clock:
        clock_window(step)
    kernel_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    ms_per_step = wall * 1e3 / steps
    log(f"timed {steps} steps: {ms_per_step:.3f} ms/step wall, "
        f"kernel mean {np.mean(kernel_ms):.3f} ms (min {np.min(kernel_ms):.3f}, "
        f"median {np.median(kernel_ms):.3f})")
    return ms_per_step, float(np.mean(kernel_ms)), warmup


def bwd_cpu_baseline(w: W.Workload, x, dout, target_s: float = 15.0):
    import oracle
    cores = oracle.default_threads()
    qb, kb, vb, db = (W.bf16_bits(t) for t in (x["q"], x["k"], x["v"], dout))
    sq = None if x["seg_q"] is None else x["seg_q"].numpy()
    sk = None if x["seg_kv"] is None else x["seg_kv"].numpy()
    rng = np.random.default_rng(11)

    def rows_for(n):
        return np.stack([rng.integers(0, w.B, n), rng.integers(0, w.H, n),
                         rng.integers(0, w.S, n)], 1).astype(np.int64)

    def flops(rows):
        # scores, dP and dq: 6*D per valid key of the row
        if sq is None:
            return 6.0 * w.D * w.S * len(rows)
        return sum(6.0 * w.D * float(np.count_nonzero(sk[b] == sq[b, i]))
                   for b, _, i in rows if sq[b, i] != 0)

    probe = rows_for(cores)
    t0 = time.perf_counter()
    oracle.attn_bwd_dq_rows(qb, kb, vb, db, sq, sk, float(np.float32(w.scale)), probe,
                            n_threads=cores)
    dt = time.perf_counter() - t0
    n = max(cores, int(cores * target_s / max(dt, 1e-3)))
    rows = rows_for(n)
    t0 = time.perf_counter()
    oracle.attn_bwd_dq_rows(qb, kb, vb, db, sq, sk, float(np.float32(w.scale)), rows,
                            n_threads=cores)
    dt = time.perf_counter() - t0
    rate = flops(rows) / dt / 1e12
    full = 6.0 * w.D * w.H * valid_pairs(w)
    return {"value": rate, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"dq of {n} random (b,h,i) rows of {w.name} (scores, dP and dq over the "
                      f"row's full key set), {dt:.1f} s on {cores} threads",
            "rows_per_s": round(n / dt, 2),
            "extrapolated_full_workload_s": round(full / (rate * 1e12), 1),
            "extrapolation": "dq of every row (6*D FLOP per valid pair) at the sampled rate"}


def bwd_main(args, vdx):
    w = W.WORKLOADS[args.workload]
    log(f"workload {w.name} backward: B={w.B} S={w.S} H={w.H} D={w.D} masked={w.masked}")
    x = W.make_inputs(w)
    dout = W.randn_bf16((w.B, w.S, w.H, w.D), w.seeds[2] + 1)
    dev = torch.device("cuda:0")
    d = {n: (None if t is None else t.to(dev)) for n, t in x.items()}
    ddo = dout.to(dev)
    stream = torch.cuda.current_stream(dev)
    out, lse = vdx.attn_fwd(d["q"], d["k"], d["v"], d["seg_q"], d["seg_kv"], scale=w.scale,
                            stream=stream)
    dq, dk, dv = (torch.empty_like(d["q"]) for _ in range(3))
    ws = torch.empty(vdx.attn_bwd_workspace_size(w.B, w.S, w.H), dtype=torch.uint8, device=dev)

    # the first call through the tensor-level wrapper checks the arguments
    vdx.attn_bwd(d["q"], d["k"], d["v"], out, lse, ddo, d["seg_q"], d["seg_kv"],
                 scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws, stream=stream)
    sp = lambda t: 0 if t is None else t.data_ptr()
    step = c_step(_native.attn_bwd_raw, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                  sp(d["seg_q"]), sp(d["seg_kv"]), out.data_ptr(), lse.data_ptr(), ddo.data_ptr(),
                  dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(),
                  w.B, w.S, w.H, w.D, w.scale, stream.cuda_stream)

    ms_per_step, call_ms, n_warm = time_steps(step, stream, args.steps, args.warmup)
    pairs = valid_pairs(w)
    flop = 10.0 * w.D * w.H * pairs
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (call_ms * 1e-3) / 1e12
    n = w.B * w.S * w.H * w.D
    line = {
        "metric": BWD_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": n_warm, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "bwd", "B": w.B, "S": w.S, "H": w.H, "D": w.D,
                   "segments": "none" if w.seg_runs is None else w.seg_runs,
                   "flop_per_step": flop, "executed_mfma_flop_per_step": 14.0 * w.D * w.H * pairs,
                   "peak_frac": round(value / PEAK_BF16_TFLOPS, 4)},
        # The three kernels of one call, timed together with HIP events on
        # their stream; per-kernel durations come from rocprofv3.
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "scope": "vdx_attn_bwd call (prep + dK/dV + dQ kernels)",
                     "traffic": load_traffic(w.name, "bwd"),
                     # reads q, k, v, out, dout, lse; writes dq, dk, dv
                     "algorithmic_bytes": 2 * 8 * n + 4 * w.B * w.H * w.S,
                     "kernel_ms_mean": round(call_ms, 4)},
        "clock": CLOCK["summary"],
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a row sample")
        line["cpu_baseline"] = bwd_cpu_baseline(w, x, dout, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def natten_main(args, vdx):
    w = W.NATTEN_WORKLOADS[args.workload]
    log(f"workload {w.name}: B={w.B} grid={w.grid} window={w.window} H={w.H} D={w.D}")
    x = W.make_natten_inputs(w)
    dev = torch.device("cuda:0")
    d = {n: t.to(dev) for n, t in x.items()}
    out = torch.empty_like(d["q"])
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    vdx.natten3d_fwd(d["q"], d["k"], d["v"], w.grid, w.window, scale=w.scale, out=out, lse=lse,
                     stream=stream)
    step = c_step(_native.natten3d_fwd_raw, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                  out.data_ptr(), lse.data_ptr(), w.B, *w.grid, w.H, w.D, *w.window, w.scale,
                  stream.cuda_stream)

    ms_per_step, kernel_ms, n_warm = time_steps(step, stream, args.steps, args.warmup)
    flop = 4.0 * w.D * w.H * w.B * w.S * natten_window_volume(w)
    executed = natten_executed_flop(w)
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (kernel_ms * 1e-3) / 1e12
    n = w.B * w.S * w.H * w.D
    line = {
        "metric": NATTEN_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": n_warm, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "grid": list(w.grid), "window": list(w.window),
                   "H": w.H, "D": w.D, "flop_per_step": flop,
                   "executed_mfma_flop_per_step": executed,
                   "window_pair_fraction_of_executed": round(flop / executed, 4),
                   "peak_frac": round(value / PEAK_BF16_TFLOPS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "executed_achieved": round(executed / (kernel_ms * 1e-3) / 1e12, 2),
                     "traffic": load_traffic(w.name, "natten"),
                     "algorithmic_bytes": 4 * 2 * n + 4 * w.B * w.H * w.S,
                     "kernel_ms_mean": round(kernel_ms, 4)},
        "clock": CLOCK["summary"],
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a row sample")
        line["cpu_baseline"] = natten_cpu_baseline(w, x, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 3 and at least 1 s of steps)")
    ap.add_argument("--workload", default=W.HEADLINE,
                    choices=sorted(W.WORKLOADS) + sorted(W.NATTEN_WORKLOADS))
    ap.add_argument("--pass", dest="pass_", choices=("fwd", "bwd"), default="fwd")
    ap.add_argument("--rope", action="store_true",
                    help="time vdx_rope3d_attn_fwd_ws (3D rotary embedding of q and k, then attention)")
    ap.add_argument("--plain", action="store_true",
                    help="time vdx_attn_fwd (no workspace) instead of vdx_attn_fwd_ws")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calib", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py measures one GPU only: the attention kernel runs on one GPU's share "
              "with every head local; the library has no multi-GPU execution path", file=sys.stderr)
        sys.exit(2)

    import spatiotemporal_attention_amd as vdx
    global _native, status_str
    from spatiotemporal_attention_amd import _native
    from spatiotemporal_attention_amd import status_str

    if args.copy_calib:
        copy_calibration()
        return
    if args.rope and (args.workload in W.NATTEN_WORKLOADS or args.pass_ != "fwd"):
        ap.error("--rope applies to the forward of the segment-masked workloads")
    if args.plain and (args.rope or args.workload in W.NATTEN_WORKLOADS or args.pass_ != "fwd"):
        ap.error("--plain applies to the attention forward without --rope")
    if args.workload in W.NATTEN_WORKLOADS:
        if args.pass_ != "fwd":
            ap.error("the neighbourhood-attention workloads have a forward pass only")
        natten_main(args, vdx)
        return
    if args.pass_ == "bwd":
        bwd_main(args, vdx)
        return

    w = W.WORKLOADS[args.workload]
    log(f"workload {w.name}: B={w.B} S={w.S} H={w.H} D={w.D} masked={w.masked} rope={args.rope}")
    x = W.make_inputs(w)
    dev = torch.device("cuda:0")
    d = {n: (None if t is None else t.to(dev)) for n, t in x.items()}
    out = torch.empty_like(d["q"])
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    rope_cfg = None
    sp = lambda t: 0 if t is None else t.data_ptr()
    if args.rope:
        r = W.workload_rope3d(w)
        rr = dict(pos=r.pos.to(dev), cos=[c.to(dev) for c in r.cos], sin=[t.to(dev) for t in r.sin],
                  dims=r.dims, interleaved=r.interleaved)
        k_rot = torch.empty_like(d["k"])
        rope_cfg = {"dims": list(r.dims), "interleaved": r.interleaved, "grids": W.ROPE_GRIDS[w.name],
                    "theta": W.ROPE_THETA}

        vdx.rope3d_attn_fwd(d["q"], d["k"], d["v"], **rr, seg_q=d["seg_q"], seg_kv=d["seg_kv"],
                            scale=w.scale, k_rot=k_rot, out=out, lse=lse, stream=stream)
        desc = vdx._rope_desc(d["q"], rr["pos"], rr["cos"], rr["sin"], rr["dims"], rr["interleaved"])
        ws = torch.empty(vdx.attn_fwd_workspace_size(w.B, w.S, w.H), dtype=torch.uint8, device=dev)
        step = c_step(_native.rope3d_attn_fwd_ws_raw, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                      sp(d["seg_q"]), sp(d["seg_kv"]), desc, k_rot.data_ptr(), out.data_ptr(),
                      lse.data_ptr(), ws.data_ptr(), ws.numel(), w.B, w.S, w.H, w.D, w.scale,
                      stream.cuda_stream)
    elif not args.plain:
        ws = torch.empty(vdx.attn_fwd_workspace_size(w.B, w.S, w.H), dtype=torch.uint8, device=dev)
        vdx.attn_fwd(d["q"], d["k"], d["v"], d["seg_q"], d["seg_kv"], scale=w.scale, out=out, lse=lse,
                     stream=stream, workspace=ws)
        step = c_step(_native.attn_fwd_ws_raw, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                      sp(d["seg_q"]), sp(d["seg_kv"]), out.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                      ws.numel(), w.B, w.S, w.H, w.D, w.scale, stream.cuda_stream)
    else:
        vdx.attn_fwd(d["q"], d["k"], d["v"], d["seg_q"], d["seg_kv"], scale=w.scale, out=out, lse=lse,
                     stream=stream, scheduled=False)
        step = c_step(_native.attn_fwd_raw, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                      sp(d["seg_q"]), sp(d["seg_kv"]), out.data_ptr(), lse.data_ptr(), w.B, w.S, w.H, w.D, w.scale,
                      stream.cuda_stream)

    ms_per_step, kernel_ms, n_warm = time_steps(step, stream, args.steps, args.warmup)
    clock = CLOCK["summary"]
    prepass_ms = None
    if args.rope:
        # the key pre-pass alone, timed the same way
        prepass_ms = time_steps(c_step(_native.rope3d_apply_raw, d["k"].data_ptr(), k_rot.data_ptr(), desc,
                                       w.B, w.S, w.H, w.D, stream.cuda_stream), stream,
                                max(3, args.steps), 1, sample_clock=False)[1]

    flop = 4.0 * w.D * w.H * valid_pairs(w)
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (kernel_ms * 1e-3) / 1e12
    entry = "vdx_rope3d_attn_fwd_ws" if args.rope else ("vdx_attn_fwd" if args.plain else "vdx_attn_fwd_ws")
    config = {"workload": w.name, "entry": entry, "B": w.B, "S": w.S, "H": w.H, "D": w.D,
              "segments": "none" if w.seg_runs is None else w.seg_runs,
              "flop_per_step": flop, "peak_frac": round(value / PEAK_BF16_TFLOPS, 4)}
    if rope_cfg is not None:
        config["rope3d"] = rope_cfg
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None if args.rope else load_traffic(w.name),
                     "algorithmic_bytes": algorithmic_bytes(w),
                     "kernel_ms_mean": round(kernel_ms, 4)},
        "clock": clock,
    }
    if args.rope:
        line["roofline"]["scope"] = "vdx_rope3d_attn_fwd_ws call (key pre-pass + attention kernels)"
        line["roofline"]["rope_key_prepass_ms"] = round(prepass_ms, 4)
    elif not args.plain:
        line["roofline"]["scope"] = ("vdx_attn_fwd_ws call (" + ("tile summaries, block counts and order, "
                                     if w.masked else "the work counters' reset, ") + "the forward, the merge of "
                                     "split items)")
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a row sample")
        line["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
