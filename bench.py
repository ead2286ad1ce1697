"""Throughput of the row pipeline on one MI355X, in achieved HBM GB/s.

One step is one pass of the whole hot path at both model widths: for level 1
([131040, 192], grid 8x182x90) and level 2 ([32760, 384], grid 8x91x45):
ln_fixed, add_ln, window_index_build (window (2,6,12), shift (1,3,6)),
window_gather and the fused norm_gather. Inputs are seeded synthetic tensors
(workloads.py) already resident in HBM. Every op of a step reads its own copy
of the inputs, and R sets of buffers rotate across steps, so no timed launch
finds its data in the 256 MB Infinity Cache from an earlier launch.

Output: one JSON line (see the keys below). ``value`` is the algorithmic bytes
of a step / the device time of a step: HIP events on the launch stream around
exactly --steps steps, queued behind a spin kernel so that host launch latency
never idles the GPU inside the region, median of several such regions; the
host wall clock of --steps steps launched from an idle GPU is reported beside
it as ``config.wall_us_per_step``. ``kernels`` times every op alone on its own
cold buffer pool, in rounds interleaved across the ops, and ``roofline`` is the
dominant kernel (add_ln at level 1) from that table; ``targets`` holds the
fraction of peak of add_ln and norm_gather at both widths. ``cpu_baseline``
times the CPU oracle on the same workload, on one core and on all cores of the
affinity set, before the GPU is touched.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from workloads import LEVEL1, LEVEL2, PATCH_MERGE, WINDOW, SHIFT  # noqa: E402

METRIC = "achieved HBM GB/s (% of peak) + Mtokens/s, fused add_ln/norm_gather C=192/384"
PEAK_GBS = 8000.0          # MI355X HBM3E, AMD's published peak
TARGET_PCT = 70.0          # share of peak HBM bandwidth the fused add_ln and norm_gather aim for
HALF = 2                   # bytes per binary16
INDEX = 4                  # bytes per int32 table entry
PMC_FILE = os.path.join(ROOT, "profiles", "add_ln_level1_pmc.json")
KERNEL_SOURCE = os.path.join(ROOT, "layernorm_window_gather_amd", "csrc", "lwg_kernels.hip")
BUILD_SCRIPT = os.path.join(ROOT, "layernorm_window_gather_amd", "build.py")


def algorithmic_bytes(op: str, n: int, m: int, c: int) -> int:
    """Bytes the operation itself must move (fp16 = 2 B, index = 4 B). Gathers
    read each source row once (the table is a bijection onto the tokens plus
    padding rows, which read nothing), write every output row, read the table."""
    if op == "ln_fixed":
        return 2 * n * c * HALF
    if op == "add_ln":
        return 4 * n * c * HALF
    if op == "window_index_build":
        return INDEX * m
    if op in ("window_gather", "norm_gather"):
        return n * c * HALF + m * c * HALF + INDEX * m
    if op == "window_inverse_build":
        return INDEX * n
    if op == "window_reverse_add_ln":
        # reads the n window rows that hold tokens, the residual and the inverse
        # table; writes residual_out and y
        return 4 * n * c * HALF + INDEX * n
    if op == "add_norm_gather":
        # reads branch and residual, writes residual_out and the m gathered rows
        return 3 * n * c * HALF + m * c * HALF + INDEX * m
    if op == "ln_affine":
        return 2 * n * c * HALF + 2 * c * HALF       # + gamma and beta
    if op == "add_ln_affine":
        return 4 * n * c * HALF + 2 * c * HALF
    raise ValueError(op)


OPS = ("ln_fixed", "add_ln", "window_index_build", "window_gather", "norm_gather")
# the fused rows around the gather, reported per kernel (not part of the step)
NEXT_OPS = ("window_inverse_build", "window_reverse_add_ln", "add_norm_gather", "ln_affine", "add_ln_affine")
# the patch-merge LayerNorm (C = 768 on the level-2 grid), reported per kernel
MERGE_OPS = ("ln_fixed", "ln_affine")
# the float32 bias + tanh-GELU at the shapes of the HIP extension tutorial
GELU_SHAPES = ((1024, 768), (4096, 1024), (8192, 2048))


def level_inputs(level):
    if level is LEVEL1:
        x, residual = workloads.level1_inputs()
    else:
        x, residual, _ = workloads.level2_inputs()
    return x, residual


class LevelBuffers:
    """One rotation set of device buffers for one level."""

    def __init__(self, lwg, torch, dev, level, x_dev, res_dev, m):
        n, c = level.tokens, level.channels
        e = lambda rows: torch.empty(rows, c, dtype=torch.float16, device=dev)  # noqa: E731
        self.x = {op: x_dev.clone() for op in ("ln_fixed", "add_ln", "window_gather", "norm_gather")}
        self.res = res_dev.clone()
        self.y_ln, self.r_out, self.y_add = e(n), e(n), e(n)
        self.g_out, self.ng_out = e(m), e(m)
        self.table = torch.empty(m, dtype=torch.int32, device=dev)
        self.calls = {
            "ln_fixed": lwg.prepare("ln_fixed", self.x["ln_fixed"], self.y_ln),
            "add_ln": lwg.prepare("add_ln", self.x["add_ln"], self.res, self.r_out, self.y_add),
            "window_index_build": lwg.prepare("window_index_build", self.table, grid=level.grid,
                                              window=WINDOW, shift=SHIFT),
            "window_gather": lwg.prepare("window_gather", self.x["window_gather"], self.table, self.g_out),
            "norm_gather": lwg.prepare("norm_gather", self.x["norm_gather"], self.table, self.ng_out),
        }


SPIN_CYCLES = 5_000_000    # a few ms of GPU spin ahead of each timed region
STEP_REGIONS = 5           # timed regions of --steps steps; the step time is their median
KERNEL_ROUNDS = 7          # rounds of the per-kernel table; each op's time is the median
COLD_BYTES = 5 << 28   # 1.25 GiB: reuse distance of any buffer in a timed run (MALL is 256 MB)


def op_pool(lwg, torch, dev, level, op, x_dev, res_dev, table, m, nbytes):
    """Enough independent buffer sets for `op` that consecutive reuses of one
    buffer are at least COLD_BYTES of traffic apart; returns prepared calls."""
    count = min(64, max(3, -(-COLD_BYTES // nbytes) + 1))   # the 64 cap only binds for the table build
    n, c = level.tokens, level.channels
    calls = []
    for _ in range(count):
        if op == "ln_fixed":
            x = x_dev.clone()
            calls.append(lwg.prepare(op, x, torch.empty_like(x)))
        elif op == "add_ln":
            b, r = x_dev.clone(), res_dev.clone()
            calls.append(lwg.prepare(op, b, r, torch.empty_like(r), torch.empty_like(r)))
        elif op == "window_index_build":
            t = torch.empty(m, dtype=torch.int32, device=dev)
            calls.append(lwg.prepare(op, t, grid=level.grid, window=WINDOW, shift=SHIFT))
        elif op == "window_inverse_build":
            t = torch.empty(n, dtype=torch.int32, device=dev)
            calls.append(lwg.prepare(op, t, grid=level.grid, window=WINDOW, shift=SHIFT))
        elif op == "window_reverse_add_ln":
            rows = lwg.window_gather(x_dev, table)            # window-ordered rows, padding = 0
            inv = lwg.window_inverse_table(level.grid, WINDOW, SHIFT, device=dev)
            r = res_dev.clone()
            calls.append(lwg.prepare(op, rows, inv, r, torch.empty_like(r), torch.empty_like(r)))
        elif op == "add_norm_gather":
            b, r = x_dev.clone(), res_dev.clone()
            calls.append(lwg.prepare(op, b, r, torch.empty_like(r), table,
                                     torch.empty(m, c, dtype=torch.float16, device=dev)))
        elif op in ("ln_affine", "add_ln_affine"):
            g = torch.linspace(0.5, 1.5, c, device=dev).to(torch.float16)
            bt = torch.linspace(-0.25, 0.25, c, device=dev).to(torch.float16)
            if op == "ln_affine":
                x = x_dev.clone()
                calls.append(lwg.prepare(op, x, g, bt, torch.empty_like(x)))
            else:
                b, r = x_dev.clone(), res_dev.clone()
                calls.append(lwg.prepare(op, b, r, g, bt, torch.empty_like(r), torch.empty_like(r)))
        else:
            x = x_dev.clone()
            calls.append(lwg.prepare(op, x, table, torch.empty(m, c, dtype=torch.float16, device=dev)))
    return calls


def replay_calls(lwg, torch, dev, m_of):
    """The 66-call block-stack replay (workloads.replay_schedule) prepared on
    device-resident inputs: per level a residual stream updated in place by
    add_ln, norm_gather reading it through shifted or unshifted tables.
    Returns (prepared calls in order, algorithmic bytes of one replay)."""
    streams = workloads.replay_streams()
    dev_streams = {k: torch.from_numpy(v[0]).to(dev) for k, v in streams.items()}
    outs, calls, total = {}, [], 0
    for call in workloads.replay_schedule():
        lv = call.level
        st = dev_streams[lv.name]
        m = m_of[lv.name]
        key = (lv.name, call.op)
        if key not in outs:
            rows = m if call.op == "norm_gather" else lv.tokens
            outs[key] = torch.empty(rows, lv.channels, dtype=torch.float16, device=dev)
        if call.op == "ln_fixed":
            calls.append(lwg.prepare("ln_fixed", st, outs[key]))
        elif call.op == "norm_gather":
            table = lwg.window_table(lv.grid, WINDOW, call.shift, device=dev)
            calls.append(lwg.prepare("norm_gather", st, table, outs[key]))
        else:
            _, nc, off = streams[lv.name]
            br = torch.from_numpy(workloads.replay_branch(call, nc, off)).to(dev)
            calls.append(lwg.prepare("add_ln", br, st, st, outs[key]))
        total += algorithmic_bytes(call.op, lv.tokens, m, lv.channels)
    return calls, total


def parity_gate(lwg, torch, sets, host, levels, m_of):
    """Sampled parity of every op on the bench buffers before any timing."""
    import oracle
    rng = np.random.default_rng(123)
    for lv in levels:
        b = sets[0][lv.name]
        for op in OPS:
            b.calls[op]()
        torch.cuda.synchronize()
        x, residual = host[lv.name]
        table = oracle.window_index_table(lv.grid, WINDOW, SHIFT)
        if not np.array_equal(b.table.cpu().numpy(), table):
            raise SystemExit(f"parity gate: window table differs at {lv.name}")
        rows = np.unique(np.concatenate([rng.choice(lv.tokens, 1024, replace=False), [0, lv.tokens - 1]]))
        jrows = np.unique(np.concatenate([rng.choice(m_of[lv.name], 1024, replace=False), [m_of[lv.name] - 1]]))
        r_ref, y_ref = oracle.add_ln(x[rows], residual[rows])
        checks = [
            ("ln_fixed", b.y_ln.cpu().numpy()[rows], oracle.layer_norm(x[rows]), False),
            ("add_ln residual", b.r_out.cpu().numpy()[rows], r_ref, True),
            ("add_ln", b.y_add.cpu().numpy()[rows], y_ref, False),
            ("window_gather", b.g_out.cpu().numpy()[jrows], oracle.window_gather(x, table[jrows]), True),
            ("norm_gather", b.ng_out.cpu().numpy()[jrows], oracle.norm_gather_rows(x, table, jrows), False),
        ]
        for name, got, ref, exact in checks:
            if exact:
                ok = np.array_equal(got.view(np.uint16), ref.view(np.uint16))
            else:
                d = np.abs(got.astype(np.float64) - ref.astype(np.float64))
                ok = d.max() <= 2e-3 and d.mean() <= 1e-4
            if not ok:
                raise SystemExit(f"parity gate failed: {name} at {lv.name}")
    return True


def next_ops_gate(lwg, torch, dev, host, levels):
    """Sampled parity of the ops reported per kernel but not in the step (the
    table inverse, the fused residual kernels, the affine LayerNorms, width 768
    and bias_gelu), one call each on seeded inputs, before any timing. Inputs
    come from workloads or the oracle, never from a HIP output."""
    import oracle
    rng = np.random.default_rng(321)

    def close(name, got, ref):
        d = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        if not (d.max() <= 2e-3 and d.mean() <= 1e-4):
            raise SystemExit(f"parity gate failed: {name}")

    def exact(name, got, ref):
        if not np.array_equal(np.asarray(got).view(np.uint16), np.asarray(ref).view(np.uint16)):
            raise SystemExit(f"parity gate failed: {name}")

    for lv in levels:
        x, residual = host[lv.name]
        n, c = lv.tokens, lv.channels
        table = oracle.window_index_table(lv.grid, WINDOW, SHIFT)
        inv = oracle.window_inverse_table(lv.grid, WINDOW, SHIFT)
        m = table.shape[0]
        rows = np.unique(np.concatenate([rng.choice(n, 1024, replace=False), [0, n - 1]]))
        jrows = np.unique(np.concatenate([rng.choice(m, 1024, replace=False), [m - 1]]))
        tx, tr = torch.from_numpy(x).to(dev), torch.from_numpy(residual).to(dev)
        tinv = lwg.window_inverse_build(lv.grid, WINDOW, SHIFT, device=dev)
        if not np.array_equal(tinv.cpu().numpy(), inv):
            raise SystemExit(f"parity gate: inverse table differs at {lv.name}")
        win = workloads.normal_rows(700 + c, m, c)
        r, y = lwg.window_reverse_add_ln(torch.from_numpy(win).to(dev), tinv, tr)
        r_ref, y_ref = oracle.add_ln(win[inv[rows]], residual[rows])
        exact(f"window_reverse_add_ln residual at {lv.name}", r.cpu().numpy()[rows], r_ref)
        close(f"window_reverse_add_ln at {lv.name}", y.cpu().numpy()[rows], y_ref)
        ttab = lwg.window_table(lv.grid, WINDOW, SHIFT, device=dev)
        r, g = lwg.add_norm_gather(tx, tr, ttab)
        exact(f"add_norm_gather residual at {lv.name}", r.cpu().numpy()[rows], oracle.residual_sum(residual[rows], x[rows]))
        t = table[jrows]
        ref = np.zeros((jrows.size, c), np.float16)
        ref[t >= 0] = oracle.layer_norm(oracle.residual_sum(residual[t[t >= 0]], x[t[t >= 0]]))
        close(f"add_norm_gather at {lv.name}", g.cpu().numpy()[jrows], ref)
        gamma = np.linspace(0.5, 1.5, c).astype(np.float16)
        beta = np.linspace(-0.25, 0.25, c).astype(np.float16)
        tg, tb = torch.from_numpy(gamma).to(dev), torch.from_numpy(beta).to(dev)
        close(f"ln_affine at {lv.name}", lwg.ln_affine(tx, tg, tb).cpu().numpy()[rows],
              oracle.layer_norm_affine(x[rows], gamma, beta))
        r, y = lwg.add_ln_affine(tx, tr, tg, tb)
        r_ref, y_ref = oracle.add_ln_affine(x[rows], residual[rows], gamma, beta)
        exact(f"add_ln_affine residual at {lv.name}", r.cpu().numpy()[rows], r_ref)
        close(f"add_ln_affine at {lv.name}", y.cpu().numpy()[rows], y_ref)
    # width 768 (patch merge) and the float32 bias + GELU
    nc, off = workloads.stress_row_classes(11, PATCH_MERGE.tokens)
    xm = workloads.mixed_rows(12, PATCH_MERGE.tokens, PATCH_MERGE.channels, nc, off)
    rows = np.unique(np.concatenate([rng.choice(PATCH_MERGE.tokens, 1024, replace=False), nc[:64], off[:64]]))
    txm = torch.from_numpy(xm).to(dev)
    close("ln_fixed at width 768", lwg.ln_fixed(txm).cpu().numpy()[rows], oracle.layer_norm(xm[rows]))
    gamma = np.linspace(0.5, 1.5, 768).astype(np.float16)
    beta = np.linspace(-0.25, 0.25, 768).astype(np.float16)
    close("ln_affine at width 768",
          lwg.ln_affine(txm, torch.from_numpy(gamma).to(dev), torch.from_numpy(beta).to(dev)).cpu().numpy()[rows],
          oracle.layer_norm_affine(xm[rows], gamma, beta))
    xg, bg = workloads.gelu_inputs(20260716, *GELU_SHAPES[-1])
    grows = rng.choice(xg.shape[0], 256, replace=False)
    got = lwg.bias_gelu(torch.from_numpy(xg).to(dev), torch.from_numpy(bg).to(dev)).cpu().numpy()[grows]
    ref = oracle.bias_gelu(xg[grows], bg).astype(np.float64)
    if not np.all(np.abs(got.astype(np.float64) - ref) <= 2e-5 + 2e-5 * np.abs(ref)):
        raise SystemExit("parity gate failed: bias_gelu")
    torch.cuda.synchronize()
    return True


SWEEP_ROWS = (16384, 32768, 65536, 131040, 262144, 524288)
# grids of the C = 384 gather sweep: level 2's 8 x _ x 45 with the grid height varied
# (32760 tokens at height 91), cut by the (2, 6, 12) window with shift (1, 3, 6)
GATHER_SWEEP_GRIDS = ((8, 12, 45), (8, 24, 45), (8, 48, 45), (8, 91, 45), (8, 182, 45), (8, 364, 45))
# the same at C = 192 on grids 8 x h x 90 (level 1 is h = 182)
GATHER_SWEEP_GRIDS_192 = ((8, 23, 90), (8, 46, 90), (8, 91, 90), (8, 182, 90), (8, 364, 90), (8, 728, 90))


def size_sweep(lwg, torch, dev, reps):
    """add_ln and ln_fixed at C = 192 over SWEEP_ROWS, and norm_gather,
    window_gather and ln_fixed at C = 384 over GATHER_SWEEP_GRIDS and at C = 192
    over GATHER_SWEEP_GRIDS_192, each on a cold
    buffer pool, timed like the per-kernel table; a least-squares fit of time =
    fixed + bytes / rate separates the per-launch fixed cost from the streaming
    rate."""
    c = 192
    base = workloads.normal_rows(9, 1 << 16, c)
    out = {"C": c, "rows": list(SWEEP_ROWS), "add_ln_us": [], "ln_fixed_us": [], "torch_copy_us": []}

    def timed(pool):
        for f in pool:
            f()
        torch.cuda.synchronize()
        runs = []
        for _ in range(5):
            torch.cuda._sleep(SPIN_CYCLES)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(reps):
                pool[i % len(pool)]()
            b.record()
            b.synchronize()
            runs.append(a.elapsed_time(b) * 1e3 / reps)
        return float(np.median(runs))

    for rows in SWEEP_ROWS:
        x0 = torch.from_numpy(np.resize(base, (rows, c))).to(dev)
        for op, nbytes in (("add_ln", 4 * rows * c * HALF), ("ln_fixed", 2 * rows * c * HALF),
                           ("torch_copy", 2 * rows * c * HALF)):
            count = max(3, -(-COLD_BYTES // nbytes) + 1)
            pool = []
            for _ in range(count):
                if op == "add_ln":
                    b, r = x0.clone(), x0.clone()
                    pool.append(lwg.prepare(op, b, r, torch.empty_like(r), torch.empty_like(r)))
                elif op == "ln_fixed":
                    xx = x0.clone()
                    pool.append(lwg.prepare(op, xx, torch.empty_like(xx)))
                else:   # the platform's own device copy, for reference
                    src, dst = x0.clone(), torch.empty_like(x0)
                    pool.append(lambda src=src, dst=dst: dst.copy_(src))
            out[f"{op}_us"].append(round(timed(pool), 3))
            del pool
            torch.cuda.empty_cache()
    def fit_of(nbytes, us):
        nb = np.array(nbytes, dtype=np.float64)
        us = np.array(us)
        (fixed, slope), *_ = np.linalg.lstsq(np.vstack([np.ones_like(nb), nb]).T, us, rcond=None)
        return {"fixed_us": round(float(fixed), 2), "marginal_GBps": round(1e-3 / float(slope), 1),
                "pct_of_peak_at_sizes": [round(100 * b / (t * 1e3) / PEAK_GBS, 1) for b, t in zip(nb, us)]}

    out["fit"] = {op: fit_of([r * per_row for r in SWEEP_ROWS], out[f"{op}_us"])
                  for op, per_row in (("add_ln", 4 * c * HALF), ("ln_fixed", 2 * c * HALF),
                                      ("torch_copy", 2 * c * HALF))}

    def gathers(c, grids, seed):
        """norm_gather, window_gather and ln_fixed at width c over `grids`, in
        the launch configuration each size takes; their extra per-launch cost
        is the fixed term of the fit."""
        base = workloads.normal_rows(seed, 1 << 15, c)
        g = {"C": c, "grids": [list(gr) for gr in grids], "tokens": [], "rows_out": [],
             "norm_gather_us": [], "window_gather_us": [], "ln_fixed_us": [], "bytes": {}}
        nbytes = {"norm_gather": [], "window_gather": [], "ln_fixed": []}
        for grid in grids:
            n = int(np.prod(grid))
            m = lwg.window_token_count(grid, WINDOW)
            g["tokens"].append(n)
            g["rows_out"].append(m)
            x0 = torch.from_numpy(np.resize(base, (n, c))).to(dev)
            table = lwg.window_index_build(grid, WINDOW, SHIFT, device=dev)
            for op in ("norm_gather", "window_gather", "ln_fixed"):
                nb = algorithmic_bytes(op, n, m, c)
                nbytes[op].append(nb)
                count = max(3, -(-COLD_BYTES // nb) + 1)
                if op == "ln_fixed":
                    pool = [lwg.prepare(op, xx, torch.empty_like(xx)) for xx in (x0.clone() for _ in range(count))]
                else:
                    pool = [lwg.prepare(op, x0.clone(), table, torch.empty(m, c, dtype=torch.float16, device=dev))
                            for _ in range(count)]
                g[f"{op}_us"].append(round(timed(pool), 3))
                del pool
                torch.cuda.empty_cache()
            del x0, table
        g["bytes"] = nbytes
        g["fit"] = {op: fit_of(nbytes[op], g[f"{op}_us"]) for op in nbytes}
        return g

    out["gathers_c384"] = gathers(384, GATHER_SWEEP_GRIDS, 10)
    out["gathers_c192"] = gathers(192, GATHER_SWEEP_GRIDS_192, 11)
    return out


def memory_attributes(dev_index: int):
    """The device's reported memory clock (kHz) and bus width (bits), read with
    hipDeviceGetAttribute, and the figure clock x bus width x 2 transfers per
    clock. HBM3E moves more than two transfers per reported clock, so that
    figure sits below the published peak; the fractions use the published
    8 TB/s."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return None
    bus, clk = ctypes.c_int(0), ctypes.c_int(0)
    # hipDeviceAttributeMemoryBusWidth = 59, hipDeviceAttributeMemoryClockRate = 60
    if hip.hipDeviceGetAttribute(ctypes.byref(bus), 59, dev_index) != 0 or \
            hip.hipDeviceGetAttribute(ctypes.byref(clk), 60, dev_index) != 0:
        return None
    return {"memory_clock_khz": clk.value, "memory_bus_bits": bus.value,
            "clock_x_bus_x2_GBps": round(clk.value * 1e3 * 2 * bus.value / 8 / 1e9, 1),
            "published_peak_GBps": PEAK_GBS}


def kernel_source_hash() -> str:
    """Hash of what the kernel binary is built from: the kernel source and the
    build script (compiler flags)."""
    h = hashlib.sha256()
    for path in (KERNEL_SOURCE, BUILD_SCRIPT):
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(dominant_bytes):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 PMC
    counters (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel calibration), or
    None when absent or taken on a different kernel source."""
    try:
        rec = json.load(open(PMC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


_CPU = {}     # inputs the all-cores workers read (inherited by fork, never pickled)


def _oracle_step_ops(x, residual, grid, rows):
    """The five ops of one step on the source rows ``rows`` (a slice) of one
    level, with the oracle; the gathers run on the table entries that read
    those rows plus their share of the padding entries."""
    import oracle
    xs, rs = x[rows], residual[rows]
    oracle.layer_norm(xs)
    oracle.add_ln(xs, rs)
    table = oracle.window_index_table(grid, WINDOW, SHIFT)
    n = x.shape[0]
    part = np.flatnonzero(((table >= rows.start) & (table < rows.stop)) |
                          ((table < 0) & (np.arange(table.size) * n // table.size >= rows.start) &
                           (np.arange(table.size) * n // table.size < rows.stop)))
    oracle.window_gather(x, table[part])
    oracle.norm_gather_rows(x, table, part)


def _cpu_worker(task):
    name, lo, hi = task
    x, residual, grid = _CPU[name]
    t = time.perf_counter()
    _oracle_step_ops(x, residual, grid, slice(lo, hi))
    return time.perf_counter() - t


def cpu_baseline(step_bytes, host, levels, min_seconds):
    """The oracle (float64 numpy, unchanged) on the host cores, on the same
    workload, in two legs:
      * one core: full steps repeated until at least ``min_seconds`` have passed
        (at most 30), ops timed one by one (numpy ufuncs run on one thread);
      * all cores: the rows of each level split into one contiguous chunk per
        core of this process's affinity set, each chunk run by its own worker
        process (forked before the GPU is touched); a step is the wall time of
        all workers finishing both levels, median of 3.
    Reported in GB/s of the step's algorithmic bytes."""
    import oracle
    per_op = {}

    def timed(key, fn, *a):
        t = time.perf_counter()
        out = fn(*a)
        per_op.setdefault(key, []).append(time.perf_counter() - t)
        return out

    t0 = time.perf_counter()
    repeats = 0
    while repeats < 30 and (repeats == 0 or time.perf_counter() - t0 < min_seconds):
        repeats += 1
        for lv in levels:
            x, residual = host[lv.name]
            timed(("ln_fixed", lv), oracle.layer_norm, x)
            timed(("add_ln", lv), oracle.add_ln, x, residual)
            table = timed(("window_index_build", lv), oracle.window_index_table, lv.grid, WINDOW, SHIFT)
            timed(("window_gather", lv), oracle.window_gather, x, table)
            timed(("norm_gather", lv), oracle.norm_gather, x, table)
    dt = time.perf_counter() - t0
    ops = {}
    for (op, lv), times in per_op.items():
        med = float(np.median(times))
        m = oracle.window_token_count(lv.grid, WINDOW)
        ops[f"{op}@{lv.name}"] = {
            "median_s": round(med, 4), "runs": len(times),
            "GBps": round(algorithmic_bytes(op, lv.tokens, m, lv.channels) / med / 1e9, 4),
            "Mtokens_per_s": round(lv.tokens / med / 1e6, 3),
        }
    one_core = round(step_bytes * repeats / dt / 1e9, 4)

    # all cores of the affinity set, one forked worker per core
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    for lv in levels:
        _CPU[lv.name] = (*host[lv.name], lv.grid)
    tasks = []
    for lv in levels:
        n = lv.tokens
        bounds = [n * i // cores for i in range(cores + 1)]
        tasks += [(lv.name, bounds[i], bounds[i + 1]) for i in range(cores) if bounds[i + 1] > bounds[i]]
    walls = []
    with mp.get_context("fork").Pool(cores) as pool:
        pool.map(_cpu_worker, tasks[:cores])      # start-up
        for _ in range(3):
            t = time.perf_counter()
            pool.map(_cpu_worker, tasks, chunksize=1)
            walls.append(time.perf_counter() - t)
    all_wall = float(np.median(walls))
    return {
        "value": one_core,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{repeats} full step(s) of the same workload (both levels, all five ops) "
                  f"in {dt:.1f} s; numpy ufuncs run on one thread; host has {os.cpu_count()} logical CPUs, "
                  f"{cores} in this process's affinity set",
        "per_op": ops,
        "all_cores": {
            "value": round(step_bytes / all_wall / 1e9, 4), "unit": "GB/s", "cores": cores,
            "step_s": round(all_wall, 4),
            "sample": f"one full step, rows of each level split into {cores} contiguous chunks, one forked "
                      "worker process per core running the oracle's five ops on its chunk (the gathers on "
                      "the table entries reading those rows); wall time until every worker is done, median "
                      "of 3 steps",
        },
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sets", type=int, default=3, help="rotating buffer sets")
    ap.add_argument("--kernel-reps", type=int, default=40, help="back-to-back launches per timed run")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="minimum oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=OPS + NEXT_OPS + ("all",), default=None,
                    help="launch only this op (or every op), --steps times per level (profiling runs)")
    ap.add_argument("--size-sweep", action="store_true",
                    help="time add_ln and ln_fixed at C=192, and the gathers against ln_fixed at C=384, "
                         "over a range of sizes and fit fixed cost + rate")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run an elementwise copy of this many MiB (PMC calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the row pipeline is sharded by rows/windows across GPUs; only the one-GPU shard is built)",
              file=sys.stderr)
        return 2

    levels = (LEVEL1, LEVEL2)
    host = {lv.name: level_inputs(lv) for lv in levels}
    cpu = None
    if not args.no_cpu_baseline and args.only is None and not args.size_sweep:
        # before anything touches the GPU: the all-cores leg forks worker processes
        import oracle
        m_cpu = {lv.name: oracle.window_token_count(lv.grid, WINDOW) for lv in levels}
        step_bytes_cpu = sum(algorithmic_bytes(op, lv.tokens, m_cpu[lv.name], lv.channels)
                             for lv in levels for op in OPS)
        cpu = cpu_baseline(step_bytes_cpu, host, levels, args.cpu_seconds)

    import torch
    import layernorm_window_gather_amd as lwg

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda", 0)
    lwg.library()
    props = torch.cuda.get_device_properties(dev)
    m_of = {lv.name: lwg.window_token_count(lv.grid, WINDOW) for lv in levels}

    sets = []
    for s in range(args.sets):
        per = {}
        for lv in levels:
            x, residual = host[lv.name]
            xd = torch.from_numpy(x).to(dev)
            rd = torch.from_numpy(residual).to(dev)
            per[lv.name] = LevelBuffers(lwg, torch, dev, lv, xd, rd, m_of[lv.name])
            del xd, rd
        sets.append(per)
    torch.cuda.synchronize()

    parity_gate(lwg, torch, sets, host, levels, m_of)
    if args.size_sweep:
        print(json.dumps({"size_sweep": size_sweep(lwg, torch, dev, args.kernel_reps)}), flush=True)
        return 0
    if args.only is None:
        next_ops_gate(lwg, torch, dev, host, levels)

    bytes_of = {(lv.name, op): algorithmic_bytes(op, lv.tokens, m_of[lv.name], lv.channels)
                for lv in levels for op in OPS + NEXT_OPS}
    step_bytes = sum(bytes_of[(lv.name, op)] for lv in levels for op in OPS)
    stream = torch.cuda.current_stream(dev)

    if args.only:
        only = OPS + NEXT_OPS if args.only == "all" else (args.only,)
        for lv in levels:
            xd, rd = (torch.from_numpy(a).to(dev) for a in host[lv.name])
            table = sets[0][lv.name].table
            for op in only:
                calls = [sets[i][lv.name].calls[op] for i in range(args.sets)] if op in OPS else \
                    op_pool(lwg, torch, dev, lv, op, xd, rd, table, m_of[lv.name], 1 << 40)
                for i in range(args.warmup + args.steps):
                    calls[i % len(calls)]()
        if args.only == "all":
            for rows, cols in GELU_SHAPES[-1:]:
                xh, bh = workloads.gelu_inputs(20260716, rows, cols)
                xg, bg = torch.from_numpy(xh).to(dev), torch.from_numpy(bh).to(dev)
                call = lwg.prepare("bias_gelu", xg, bg, torch.empty_like(xg))
                for _ in range(args.warmup + args.steps):
                    call()
        torch.cuda.synchronize()
        if args.calibration_copy_mib:
            n = args.calibration_copy_mib * (1 << 20) // 2
            a = torch.ones(n, dtype=torch.float16, device=dev)
            b = torch.empty_like(a)
            for _ in range(3):
                torch.mul(a, 1, out=b)
            torch.cuda.synchronize()
        print(json.dumps({"profiling_run": args.only, "launches_per_level": args.warmup + args.steps}))
        return 0

    def step(i):
        per = sets[i % args.sets]
        for lv in levels:
            calls = per[lv.name].calls
            for op in OPS:
                calls[op]()

    def wall_single(launch, count=20):
        """Median host wall time of one launch bracketed by two synchronisations
        (the way the pages time an operator); includes launch latency."""
        times = []
        for i in range(count):
            torch.cuda.synchronize()
            t = time.perf_counter()
            launch(i)
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t)
        return float(np.median(times)) * 1e6

    def run_timed(launch, count, spin=True):
        """HIP events on the launch stream around `count` back-to-back launches;
        returns the average microseconds per launch. A spin kernel queued first
        keeps the GPU busy while the launches are enqueued, so host launch
        latency never leaves the GPU idle inside the timed region."""
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if spin:
            torch.cuda._sleep(SPIN_CYCLES)
        a.record(stream)
        for i in range(count):
            launch(i)
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / count

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed regions 1: exactly --steps steps each, STEP_REGIONS times, each behind
    # a spin kernel and bracketed by synchronisations; the step time is the median
    # of the regions' event times (device calibre). The host wall clock of one
    # more region of --steps steps launched from an idle GPU is reported beside
    # it (host calibre: includes launch latency and the final synchronisation).
    step_runs = []
    for r in range(STEP_REGIONS):
        torch.cuda.synchronize()
        step_runs.append(run_timed(lambda i, r=r: step(args.warmup + r * args.steps + i), args.steps))
        torch.cuda.synchronize()
    step_us = float(np.median(step_runs))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall_us_per_step = (time.perf_counter() - t0) * 1e6 / args.steps
    ms_per_step = step_us * 1e-3

    # device copies of the inputs, for the per-op pools
    dev_in = {}
    for lv in levels:
        x, residual = host[lv.name]
        dev_in[lv.name] = (torch.from_numpy(x).to(dev), torch.from_numpy(residual).to(dev),
                           sets[0][lv.name].table)

    def pool_for(lv, op):
        xd, rd, table = dev_in[lv.name]
        return op_pool(lwg, torch, dev, lv, op, xd, rd, table, m_of[lv.name], bytes_of[(lv.name, op)])

    # timed regions 2: every op on its own cold buffer pool (all pools built
    # first), KERNEL_ROUNDS rounds that each time every op once (spin kernel, then
    # --kernel-reps back-to-back launches between HIP events), so that drift in
    # the device's state affects all ops alike; median over the rounds
    nc, off = workloads.stress_row_classes(11, PATCH_MERGE.tokens)
    merge_x = torch.from_numpy(workloads.mixed_rows(12, PATCH_MERGE.tokens, PATCH_MERGE.channels, nc, off)).to(dev)
    dev_in[PATCH_MERGE.name] = (merge_x, merge_x, None)
    m_of[PATCH_MERGE.name] = PATCH_MERGE.tokens
    for op in MERGE_OPS:
        bytes_of[(PATCH_MERGE.name, op)] = algorithmic_bytes(op, PATCH_MERGE.tokens, PATCH_MERGE.tokens,
                                                             PATCH_MERGE.channels)
    entries = {}      # name -> (pool, bytes, description)
    for rows, cols in GELU_SHAPES:
        nb = 2 * rows * cols * 4 + cols * 4
        count = min(64, max(3, -(-COLD_BYTES // nb) + 1))
        xh, bh = workloads.gelu_inputs(20260716, rows, cols)
        x0 = torch.from_numpy(xh).to(dev)
        bias = torch.from_numpy(bh).to(dev)
        pool = []
        for _ in range(count):
            xi = x0.clone()
            pool.append(lwg.prepare("bias_gelu", xi, bias, torch.empty_like(xi)))
        entries[f"bias_gelu@{rows}x{cols}"] = (pool, nb, {"dtype": "f32", "rows_in": rows, "cols": cols,
                                                           "in_step": False})
    for lv, ops in ((LEVEL1, OPS + NEXT_OPS), (LEVEL2, OPS + NEXT_OPS), (PATCH_MERGE, MERGE_OPS)):
        for op in ops:
            entries[f"{op}@{lv.name}"] = (pool_for(lv, op), bytes_of[(lv.name, op)], {
                "C": lv.channels, "rows_in": lv.tokens, "in_step": op in OPS and lv is not PATCH_MERGE,
                "rows_out": m_of[lv.name] if op in ("window_gather", "norm_gather", "window_index_build",
                                                    "add_norm_gather") else lv.tokens})
    next_i = {}
    for name, (pool, _, _) in entries.items():
        for f in pool:
            f()
        next_i[name] = 0
    torch.cuda.synchronize()
    runs = {name: [] for name in entries}
    for _ in range(KERNEL_ROUNDS):
        for name, (pool, _, _) in entries.items():
            base = next_i[name]
            runs[name].append(run_timed(lambda i, pool=pool, base=base: pool[(base + i) % len(pool)](),
                                        args.kernel_reps))
            next_i[name] = (base + args.kernel_reps) % len(pool)
    kernels = {}
    for name, (pool, nb, info) in entries.items():
        r = np.array(runs[name])
        med = float(np.median(r))
        gbs = nb / (med * 1e-6) / 1e9
        rec = dict(info)
        rec.update({"bytes": nb, "avg_us": round(med, 2), "min_run_us": round(float(r.min()), 2),
                    "max_run_us": round(float(r.max()), 2), "GBps": round(gbs, 1),
                    "pct_of_peak": round(100 * gbs / PEAK_GBS, 1)})
        if "rows_in" in info and "C" in info:
            rec["Mtokens_per_s"] = round(info["rows_in"] / (med * 1e-6) / 1e6, 1)
        rec["wall_us_sync"] = round(wall_single(lambda i, pool=pool: pool[i % len(pool)]()), 2)
        kernels[name] = rec
    del entries
    torch.cuda.empty_cache()
    dom_us = kernels["add_ln@level1"]["avg_us"]
    dom_bytes = bytes_of[(LEVEL1.name, "add_ln")]

    # block-stack replay: 66 dependent calls on resident residual streams
    rcalls, rbytes = replay_calls(lwg, torch, dev, m_of)
    for c in rcalls:
        c()
    torch.cuda.synchronize()
    rep_runs = []
    for _ in range(5):
        rep_runs.append(run_timed(lambda i: [c() for c in rcalls], 3))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for c in rcalls:
        c()
    torch.cuda.synchronize()
    rep_wall_ms = (time.perf_counter() - t0) * 1e3
    rep_us = float(np.median(rep_runs))
    replay = {
        "calls": len(rcalls), "bytes": rbytes, "avg_us": round(rep_us, 1),
        "GBps": round(rbytes / (rep_us * 1e-6) / 1e9, 1),
        "pct_of_peak": round(100 * rbytes / (rep_us * 1e-6) / 1e9 / PEAK_GBS, 1),
        "wall_ms_single_replay": round(rep_wall_ms, 3),
        "note": "34 LayerNorm-family + 32 norm_gather calls alternating level 1 and level 2; the residual "
                "streams are re-read from call to call as in a block stack, so part of the traffic is "
                "served by the Infinity Cache (unlike the cold per-kernel figures)",
    }
    del rcalls

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {
            "workload": "row pipeline at both widths per step: ln_fixed, add_ln, window_index_build, "
                        "window_gather, norm_gather on [131040,192] (grid 8x182x90) and [32760,384] "
                        "(grid 8x91x45), window (2,6,12), shift (1,3,6)",
            "io_dtype": "fp16", "statistics": "f64",
            "step_bytes": step_bytes, "pct_of_peak": round(100 * value / PEAK_GBS, 1),
            "step_timing": f"HIP events on the launch stream around exactly {args.steps} steps behind a spin "
                           f"kernel, {STEP_REGIONS} such regions, median (ms_per_step); the host wall clock of "
                           f"{args.steps} more steps launched from an idle GPU, bracketed by synchronisations, "
                           "is wall_us_per_step (a separate calibre: launch latency and final sync included)",
            "step_region_us": [round(u, 2) for u in step_runs],
            "wall_us_per_step": round(wall_us_per_step, 2),
            "buffer_sets": args.sets, "device": props.name,
            "arch": getattr(props, "gcnArchName", "?"), "cus": props.multi_processor_count,
            "memory": memory_attributes(dev.index or 0),
            "versions": {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
                         "python": sys.version.split()[0], "numpy": np.__version__},
            "seeds": {"level1": 1, "level2": 2, "patch_merge_rows": 11, "patch_merge_values": 12,
                      "replay_streams": 4, "replay_branch_of_block_b": "4 + b",
                      "bias_gelu": 20260716},
        },
        "roofline": {
            "kernel": "add_ln@level1",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4),
            "traffic": traffic_from_profile(dom_bytes),
            "avg_launch_us": round(dom_us, 3),
            "bytes_per_launch": dom_bytes,
            "timing": f"HIP events around {args.kernel_reps} back-to-back launches on the launch stream behind "
                      f"a spin kernel, median of {KERNEL_ROUNDS} rounds interleaved with every other op, buffers "
                      "rotated so each is reused >= 1.25 GiB of traffic later",
        },
        "targets": {
            name: {"pct_of_peak": kernels[name]["pct_of_peak"], "GBps": kernels[name]["GBps"],
                   "avg_us": kernels[name]["avg_us"], "Mtokens_per_s": kernels[name]["Mtokens_per_s"],
                   "target_pct_of_peak": TARGET_PCT, "met": kernels[name]["pct_of_peak"] >= TARGET_PCT}
            for name in ("add_ln@level1", "add_ln@level2", "norm_gather@level1", "norm_gather@level2")
        },
        "parity_gate": "passed: sampled outputs of every reported op against the oracle, before timing",
        "kernels": kernels,
        "replay": replay,
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
