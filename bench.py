"""Benchmark: batch-invariant RMSNorm forward + backward on one MI355X.

One step = the whole hot path over one batch: rmsnorm_fwd (y, rstd), then
rmsnorm_bwd_dx with the canonical dweight accumulator (dx and dweight
contributions in one pass), then rmsnorm_dw_finalize (dweight), then the
accumulator reset.  Workload: hidden 4096, 8 samples x 4096 tokens = 32768
rows, bf16, one B=N call (the identity layout).  Inputs are resident in HBM
before timing; buffer sets rotate so consecutive steps never reuse data.

value = algorithmic HBM bytes of fwd + bwd per step / step time, in GB/s:
  fwd = rows*(2H + 4) + rows*2H + 2H        (x, rstd, y, w)
  bwd = rows*(4H + 4) + rows*2H + 2H + 4H   (x, dy, rstd, dx, w, dweight)
The roofline entry is the backward kernel alone: its algorithmic bytes over
its average duration, measured with HIP events around K back-to-back
launches on the stream it runs on; `traffic` is the HBM bytes per launch
from rocprofv3 FETCH_SIZE/WRITE_SIZE (calibrated on a 1 GiB copy) when the
committed counters were taken on the current kernel sources, else null.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "RMSNorm fwd+bwd achieved HBM GB/s (% of peak) with bitwise B1/BN/chunk invariance"
PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_traffic_rmsnorm_h4096_t32768.json")
EMB_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_traffic_det_embedding_v32000_d4096_t32768.json")


def algorithmic_bytes(rows_real: int, rows_phys: int, H: int):
    fwd = rows_real * (2 * H + 4) + rows_phys * 2 * H + 2 * H
    bwd = rows_real * (4 * H + 4) + rows_phys * 2 * H + 2 * H + 4 * H
    return fwd, bwd


# Sources that define the RMSNorm kernels (the linear-layer kernels and the
# C-ABI glue do not change them).
NORM_KERNEL_SOURCES = ("kernels.hip", "kernels.h", "device_math.h", "plan.h")
GEMM_KERNEL_SOURCES = ("linear.hip", "linear.h", "tile_map.h")


def kernel_source_hash(names=NORM_KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "invariant_rmsnorm_backward_amd", "csrc")
    for name in sorted(names):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(bwd_bytes: int, path: str = TRAFFIC_FILE, sources=None):
    """HBM bytes per backward launch (or per backward call, summed over its
    launches) from committed rocprofv3 counters, or None when the kernels
    changed since they were taken."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    h = kernel_source_hash() if sources is None else kernel_source_hash(sources)
    if t.get("kernel_source_hash") != h:
        return None
    return t.get("bytes_per_launch")


def _oracle_pieces(wl, n_pieces: int, chunk: int = 1024):
    """Inputs of the first n_pieces 1024-row pieces of the workload (bf16 bits)."""
    from invariant_rmsnorm_backward_amd import inputs
    import numpy as np
    out = []
    for k in range(n_pieces):
        a = (k * chunk) % wl.n_logical
        rows = np.arange(a, min(a + chunk, wl.n_logical))
        out.append((inputs.bf16_bits(inputs.gen_x(wl, rows)), inputs.bf16_bits(inputs.gen_dy(wl, rows))))
    return out


def cpu_baseline(wl, single_s: float = 6.0, parallel_s: float = 1.5):
    """The FP64 oracle as it stands over 1024-row pieces of the same workload
    (inputs generated before timing; a pass over the workload repeats its
    pieces): first on one thread for about single_s seconds, then on every
    host core the process may use (at most 16, one thread each, the oracle's
    C calls running outside Python's lock) for about parallel_s seconds of
    wall time.  Reported: the all-cores rate, with the one-core rate beside it."""
    import threading
    import oracle
    from invariant_rmsnorm_backward_amd import inputs
    H = wl.hidden
    wb = inputs.bf16_bits(inputs.gen_w(wl))
    pieces = _oracle_pieces(wl, min(32, (wl.n_logical + 1023) // 1024))
    oracle.rmsnorm_fwd_bf16(pieces[0][0][:1], wb, wl.eps)      # load the library once

    def work(k0, step, stop_at, tally, idx):
        rows, k = 0, k0
        while time.perf_counter() < stop_at:
            xb, dyb = pieces[k % len(pieces)]
            oracle.rmsnorm_fwd_bf16(xb, wb, wl.eps)
            oracle.rmsnorm_bwd_bf16(xb, wb, dyb, wl.eps)
            rows += xb.shape[0]
            k += step
        tally[idx] = rows

    def run(n_threads, seconds):
        tally = [0] * n_threads
        t0 = time.perf_counter()
        ts = [threading.Thread(target=work, args=(i, n_threads, t0 + seconds, tally, i))
              for i in range(n_threads)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        spent = time.perf_counter() - t0
        done = sum(tally)
        f, b = algorithmic_bytes(done, done, H)
        return done, spent, (f + b) / spent / 1e9

    d1, s1, g1 = run(1, single_s)
    cores = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 1))
    dn, sn, gn = run(cores, parallel_s)
    return {"value": round(gn, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{dn} rows of {wl.name} in 1024-row pieces on {cores} threads ({sn:.1f} s wall), "
                      f"fwd+bwd in FP64 (the plain C oracle, one call per piece), input generation "
                      f"excluded",
            "rows_per_s": round(dn / sn, 1),
            "single_core": {"value": round(g1, 4), "unit": "GB/s", "cores": 1,
                            "sample": f"{d1} rows, {s1:.1f} s", "rows_per_s": round(d1 / s1, 1)}}


def copy_ceiling(torch, nbytes: int, iters: int = 20):
    """Device-to-device copy bandwidth (read + write bytes / time), GB/s:
    (the library's streaming copy, torch's copy).  The first is the practical
    ceiling the step is compared with; the second (hipMemcpy's copy kernel)
    is also the calibration run of the rocprofv3 traffic counters."""
    from invariant_rmsnorm_backward_amd import binding
    n = nbytes // 2
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    sh = binding.current_stream()

    def rate(f):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            f()
        e1.record()
        torch.cuda.synchronize()
        return 2.0 * nbytes * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9

    ours = rate(lambda: binding.rmsnorm_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes, sh))
    theirs = rate(lambda: dst.copy_(src))
    del src, dst
    return ours, theirs


def stream_2to1(torch, nbytes: int, iters: int = 20):
    """Two reads for each write, the backward's traffic mix: torch's bf16
    elementwise add c = a + b over three nbytes tensors, GB/s of the three
    (a library kernel, so the ceiling is not one of ours)."""
    n = nbytes // 2
    a = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    b = torch.ones_like(a)
    c = torch.empty_like(a)
    for _ in range(3):
        torch.add(a, b, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        torch.add(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    gbps = 3.0 * nbytes * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b, c
    return gbps


def stream_2r1w(binding, torch, nbytes: int, iters: int = 20):
    """The same mix with the library's two-read probe (c = a XOR b, 16-byte
    non-temporal accesses, four units per thread per pass), GB/s of the
    three nbytes buffers: the practical ceiling for the backward's traffic."""
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.int32, device="cuda")
    b = torch.ones_like(a)
    c = torch.empty_like(a)
    sh = binding.current_stream()
    for _ in range(3):
        binding.rmsnorm_stream_2r1w(a.data_ptr(), b.data_ptr(), c.data_ptr(), nbytes, sh)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        binding.rmsnorm_stream_2r1w(a.data_ptr(), b.data_ptr(), c.data_ptr(), nbytes, sh)
    e1.record()
    torch.cuda.synchronize()
    gbps = 3.0 * nbytes * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b, c
    return gbps


QK_PAIR = "qknorm_d128_t16384"


def launch_floor(torch, np, binding, stream, sizes, steps: int):
    """The cell's call pattern with every kernel replaced by the library's
    streaming copy moving the same algorithmic bytes: per call one copy of
    its forward bytes, then per call one copy of its backward bytes, each at
    fresh addresses in a 1 GiB pool (so no launch finds its data in the
    caches).  sizes: (fwd_bytes, bwd_bytes) of each call in order.  Returns
    the median fwd and bwd phase times (ms) over `steps` steps: what a plain
    stream achieves in the same number of launches of the same sizes."""
    pool = 1 << 30
    src = torch.empty(pool, dtype=torch.uint8, device="cuda")
    dst = torch.empty(pool, dtype=torch.uint8, device="cuda")
    sh = stream.cuda_stream
    off = [0]

    def copy(nbytes):
        n = max(16, (nbytes // 2 + 15) // 16 * 16)     # a copy of n bytes moves 2n
        if off[0] + n > pool:
            off[0] = 0
        binding.rmsnorm_stream_copy(src.data_ptr() + off[0], dst.data_ptr() + off[0], n, sh)
        off[0] += (n + 255) // 256 * 256

    for _ in range(2):
        for f, _ in sizes:
            copy(f)
        for _, b in sizes:
            copy(b)
    times = {"fwd": [], "bwd": []}
    ev = []
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        for f, _ in sizes:
            copy(f)
        e[1].record(stream)
        for _, b in sizes:
            copy(b)
        e[2].record(stream)
        ev.append(e)
    torch.cuda.synchronize()
    for e in ev:
        times["fwd"].append(e[0].elapsed_time(e[1]))
        times["bwd"].append(e[1].elapsed_time(e[2]))
    del src, dst
    return {k: float(np.median(v)) for k, v in times.items()}


def measure_cell(args, torch, np, binding, inputs, layouts):
    """Info measurement of one workload on one layout cell: a step runs every
    call of the cell (rmsnorm_fwd, then rmsnorm_bwd_dx into the accumulator),
    then rmsnorm_dw_finalize, for each norm of the workload (Q and K for the
    per-head pair).  Physical inputs are gathered before timing; padding rows
    hold a NaN pattern that the kernels never read.  The cell's dweight is
    also checked bitwise against one B=N call on the same logical rows."""
    from invariant_rmsnorm_backward_amd import adapters
    if args.workload == QK_PAIR:
        wls = [inputs.ALL_WORKLOADS[QK_PAIR + "_q"](), inputs.ALL_WORKLOADS[QK_PAIR + "_k"]()]
    else:
        wls = [inputs.ALL_WORKLOADS[args.workload]()]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    norms = []
    for wl in wls:
        T, H = wl.n_logical, wl.hidden
        chunk = 7 if wl.hidden <= 8 else 512
        cells = {c.name: c for c in layouts.standard_matrix(wl, chunk)}
        if args.cell not in cells:
            print(f"unknown cell {args.cell!r}; cells: {sorted(cells)}", file=sys.stderr)
            sys.exit(2)
        cell = cells[args.cell]
        print(f"[bench] generating {wl.name} ({T} x {H}), cell {cell.name}: "
              f"{len(cell.calls)} call(s)", file=sys.stderr, flush=True)
        x = inputs.gen_x(wl, device="cuda")
        dy = inputs.gen_dy(wl, device="cuda")
        w = inputs.gen_w(wl, device="cuda")
        calls = []
        for call in cell.calls:
            if call.row_logical is None:
                calls.append(dict(rows=call.rows, real=call.rows, layout=None, x=x, dy=dy))
                continue
            rl = torch.from_numpy(call.row_logical.astype(np.int64)).cuda()
            real = rl >= 0
            xc = torch.full((call.rows, H), 0x7FC1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
            dyc = xc.clone()
            xc[real] = x[rl[real]]
            dyc[real] = dy[rl[real]]
            calls.append(dict(rows=call.rows, real=int(real.sum()),
                              layout=binding.Layout(call.row_logical, T), x=xc, dy=dyc))
        sets = []
        for k in range(args.sets):
            sets.append([dict(x=c["x"] if k == 0 else c["x"].clone(),
                              dy=c["dy"] if k == 0 else c["dy"].clone(),
                              y=torch.empty_like(c["x"]), dx=torch.empty_like(c["x"]),
                              rstd=torch.empty(c["rows"], dtype=torch.float32, device="cuda"))
                         for c in calls])
        # bounded spill area: 64 rows per block a call holds in part
        acc = binding.DwAccumulator(T, H, max_spill_rows=adapters.spill_bound(cell, T))
        # B=N reference dweight on the logical rows (identity layout)
        acc_ref = binding.DwAccumulator(T, H)
        _, r_ref = binding.fwd(x, w, wl.eps)
        binding.bwd(x, w, dy, r_ref, None, acc_ref)
        dw_ref = acc_ref.finalize()
        norms.append(dict(wl=wl, T=T, H=H, w=w, calls=calls, sets=sets, acc=acc,
                          dw=torch.empty(H, dtype=torch.float32, device="cuda"),
                          dw_ref=dw_ref, acc_ref=acc_ref, cell=cell))

    def run_fwd(n, s, st=sh):
        for c, b in zip(n["calls"], s):
            binding.rmsnorm_fwd(b["x"].data_ptr(), n["w"].data_ptr(), b["y"].data_ptr(),
                                b["rstd"].data_ptr(), c["rows"], n["H"], n["wl"].eps,
                                None if c["layout"] is None else c["layout"].handle, st)

    def run_bwd(n, s, st=sh):
        for c, b in zip(n["calls"], s):
            binding.rmsnorm_bwd_dx(b["x"].data_ptr(), n["w"].data_ptr(), b["dy"].data_ptr(),
                                   b["rstd"].data_ptr(), b["dx"].data_ptr(), c["rows"], n["H"],
                                   None if c["layout"] is None else c["layout"].handle,
                                   n["acc"].handle, st)

    def run_fin(n, st=sh):
        binding.rmsnorm_dw_finalize(n["acc"].handle, n["dw"].data_ptr(), st)
        binding.rmsnorm_dw_acc_reset(n["acc"].handle, st)

    def step(i, st=sh):
        for n in norms:
            s = n["sets"][i % len(n["sets"])]
            run_fwd(n, s, st)
            run_bwd(n, s, st)
            run_fin(n, st)

    step(0)
    torch.cuda.synchronize()
    inv_ok = all(torch.equal(n["dw"].view(torch.int32), n["dw_ref"].view(torch.int32)) for n in norms)
    for i in range(args.warmup):
        step(i)
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / K * 1e3

    # per-phase times: events around each phase of each norm
    ph = {"fwd": [], "bwd": [], "finalize": []}
    for i in range(K):
        tot = {"fwd": [], "bwd": [], "finalize": []}
        for n in norms:
            s = n["sets"][i % len(n["sets"])]
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record(stream)
            run_fwd(n, s)
            e[1].record(stream)
            run_bwd(n, s)
            e[2].record(stream)
            run_fin(n)
            e[3].record(stream)
            tot["fwd"].append((e[0], e[1]))
            tot["bwd"].append((e[1], e[2]))
            tot["finalize"].append((e[2], e[3]))
        for k in ph:
            ph[k].append(tot[k])
    torch.cuda.synchronize()
    med = {k: float(np.median([sum(a.elapsed_time(b) for a, b in step_ev) for step_ev in v]))
           for k, v in ph.items()}

    # The same steps captured once in a HIP graph and replayed (launch-bound
    # cells); only when no block is split across calls, since the finalize
    # then enqueues kernels alone (with split blocks it uploads a spill list).
    graph = None
    if args.graph:
        split = sum(binding.rmsnorm_layout_check(c.row_logical, n["T"])["partial_blocks"]
                    for n in norms for c in n["cell"].calls if c.row_logical is not None)
        if split:
            graph = {"skipped": f"{split} block(s) split across calls: the finalize uploads a spill list"}
        else:
            nsets = len(norms[0]["sets"])
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cs = torch.cuda.current_stream().cuda_stream
                for i in range(nsets):
                    step(i, cs)
            for _ in range(2):
                g.replay()
            reps = max(1, K // nsets)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            graph = {"ms_per_step": round((time.perf_counter() - t0) / (reps * nsets) * 1e3, 4),
                     "steps": reps * nsets}
            del g

    fb = bb = 0
    for n in norms:
        for c in n["calls"]:
            f1, b1 = algorithmic_bytes(c["real"], c["rows"], n["H"])
            fb += f1
            bb += b1 - 4 * n["H"]          # dweight is written once per norm, not per call
        bb += 4 * n["H"]
    rows_real = sum(c["real"] for n in norms for c in n["calls"])
    rows_phys = sum(c["rows"] for n in norms for c in n["calls"])
    value = (fb + bb) / (ms_step * 1e-3) / 1e9
    achieved = bb / (med["bwd"] * 1e-3) / 1e9
    n_calls = sum(len(n["calls"]) for n in norms)
    # The per-head pair: the same calls with Q and K of each call in one launch
    # per phase (rmsnorm_fwd_packed_pair / rmsnorm_bwd_dx_packed_pair), when
    # every call holds whole tokens of both.
    pair = None
    if args.workload == QK_PAIR:
        nq, nk = norms
        hq, hk, d = nq["wl"].heads, nk["wl"].heads, nq["H"]
        if all(cq["rows"] % hq == 0 and ck["rows"] % hk == 0 and cq["rows"] // hq == ck["rows"] // hk
               for cq, ck in zip(nq["calls"], nk["calls"])):
            lay = lambda c: None if c["layout"] is None else c["layout"].handle

            def pair_fwd(i):
                sq, sk = nq["sets"][i % len(nq["sets"])], nk["sets"][i % len(nk["sets"])]
                for cq, ck, bq, bk in zip(nq["calls"], nk["calls"], sq, sk):
                    binding.rmsnorm_fwd_packed_pair(
                        (bq["x"].data_ptr(), nq["w"].data_ptr(), bq["y"].data_ptr(), bq["rstd"].data_ptr(),
                         hq, hq * d, lay(cq)),
                        (bk["x"].data_ptr(), nk["w"].data_ptr(), bk["y"].data_ptr(), bk["rstd"].data_ptr(),
                         hk, hk * d, lay(ck)), cq["rows"] // hq, d, nq["wl"].eps, sh)

            def pair_bwd(i):
                sq, sk = nq["sets"][i % len(nq["sets"])], nk["sets"][i % len(nk["sets"])]
                for cq, ck, bq, bk in zip(nq["calls"], nk["calls"], sq, sk):
                    binding.rmsnorm_bwd_dx_packed_pair(
                        (bq["x"].data_ptr(), nq["w"].data_ptr(), bq["dy"].data_ptr(), bq["rstd"].data_ptr(),
                         bq["dx"].data_ptr(), hq, hq * d, lay(cq), nq["acc"].handle),
                        (bk["x"].data_ptr(), nk["w"].data_ptr(), bk["dy"].data_ptr(), bk["rstd"].data_ptr(),
                         bk["dx"].data_ptr(), hk, hk * d, lay(ck), nk["acc"].handle), cq["rows"] // hq, d, sh)

            def pair_step(i):
                pair_fwd(i)
                pair_bwd(i)
                run_fin(nq)
                run_fin(nk)

            pair_step(0)
            torch.cuda.synchronize()
            pair_ok = all(torch.equal(n["dw"].view(torch.int32), n["dw_ref"].view(torch.int32)) for n in norms)
            for i in range(args.warmup):
                pair_step(i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(K):
                pair_step(i)
            torch.cuda.synchronize()
            pair_ms = (time.perf_counter() - t0) / K * 1e3
            pev = []
            for i in range(K):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
                e[0].record(stream)
                pair_fwd(i)
                e[1].record(stream)
                pair_bwd(i)
                e[2].record(stream)
                run_fin(nq)
                run_fin(nk)
                e[3].record(stream)
                pev.append(e)
            torch.cuda.synchronize()
            pm = {k: float(np.median([e[j].elapsed_time(e[j + 1]) for e in pev]))
                  for j, k in enumerate(("fwd", "bwd", "finalize"))}
            pair = {"ms_per_step": round(pair_ms, 4), "phases_ms": {k: round(v, 5) for k, v in pm.items()},
                    "dweight_bitwise_equal_to_bn_full": pair_ok,
                    "launches": "one rmsnorm_fwd_packed_pair and one rmsnorm_bwd_dx_packed_pair per call"}

    # One call over every row (BN/full): the rstd-recompute backward on the
    # same rows, back to back, checked bit for bit against the saved-rstd one.
    recompute = None
    if n_calls == 1 and norms[0]["calls"][0]["layout"] is None and norms[0]["H"] > 256:
        n = norms[0]
        c = n["calls"][0]
        b0 = n["sets"][0][0]
        T1, H1 = c["rows"], n["H"]
        dx_rc = torch.empty_like(b0["dx"])
        dw_rc = torch.empty_like(n["dw"])
        run_fwd(n, n["sets"][0])
        run_bwd(n, n["sets"][0])
        run_fin(n)
        binding.rmsnorm_bwd_dx_recompute(b0["x"].data_ptr(), n["w"].data_ptr(), b0["dy"].data_ptr(),
                                         n["wl"].eps, dx_rc.data_ptr(), T1, H1, None,
                                         n["acc"].handle, sh)
        binding.rmsnorm_dw_finalize(n["acc"].handle, dw_rc.data_ptr(), sh)
        binding.rmsnorm_dw_acc_reset(n["acc"].handle, sh)
        torch.cuda.synchronize()
        same = bool(torch.equal(dx_rc.view(torch.int16), b0["dx"].view(torch.int16)) and
                    torch.equal(dw_rc.view(torch.int32), n["dw"].view(torch.int32)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(K):
            b = n["sets"][i % len(n["sets"])][0]
            binding.rmsnorm_bwd_dx_recompute(b["x"].data_ptr(), n["w"].data_ptr(), b["dy"].data_ptr(),
                                             n["wl"].eps, b["dx"].data_ptr(), T1, H1, None,
                                             n["acc"].handle, sh)
            binding.rmsnorm_dw_acc_reset(n["acc"].handle, sh)
        e1.record(stream)
        torch.cuda.synchronize()
        rc_ms = e0.elapsed_time(e1) / K
        _, bb1 = algorithmic_bytes(c["real"], c["rows"], H1)
        rc_bytes = bb1 - 4 * c["real"]          # no rstd read
        recompute = {"avg_launch_ms": round(rc_ms, 5),
                     "gbps": round(rc_bytes / (rc_ms * 1e-3) / 1e9, 1),
                     "frac": round(rc_bytes / (rc_ms * 1e-3) / 1e9 / PEAK_GBPS, 4),
                     "bitwise_equal_to_saved_rstd": same}
    floor = None
    if n_calls > 1:
        sizes = [algorithmic_bytes(c["real"], c["rows"], n["H"]) for n in norms for c in n["calls"]]
        fl = launch_floor(torch, np, binding, stream, sizes, K)
        fl_gbps = (fb + bb) / ((fl["fwd"] + fl["bwd"]) * 1e-3) / 1e9
        floor = {"fwd_ms": round(fl["fwd"], 5), "bwd_ms": round(fl["bwd"], 5),
                 "gbps": round(fl_gbps, 1), "frac": round(fl_gbps / PEAK_GBPS, 4),
                 "value_over_floor": round(value / fl_gbps, 4),
                 "kernel": "rmsnorm_stream_copy, one launch per call and phase, same bytes"}
    # the oracle on a bounded sample of the (first) norm's logical rows
    cpu = None if args.no_cpu_baseline else cpu_baseline(norms[0]["wl"])
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "cell": args.cell, "hidden": norms[0]["H"],
                   "rows_real": rows_real, "rows_physical": rows_phys, "calls_per_step": n_calls,
                   "norms": [n["wl"].name for n in norms], "io_dtype": "bf16",
                   "buffer_sets": args.sets},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4), "traffic": None,
                     "kernel": "backward phase (all bwd launches of the step)",
                     "algorithmic_bytes_per_step": bb, "bwd_ms": round(med["bwd"], 5)},
        "cpu_baseline": cpu,
        "phases_ms": {k: round(v, 5) for k, v in med.items()},
        "phases_gbps": {"fwd": round(fb / (med["fwd"] * 1e-3) / 1e9, 1),
                        "bwd": round(achieved, 1)},
        "rows_per_s": round(rows_real / (ms_step * 1e-3), 1),
        "frac_of_peak": round(value / PEAK_GBPS, 4),
        "dweight_bitwise_equal_to_bn_full": inv_ok,
        "kernel_source_hash": kernel_source_hash(),
    }
    if floor is not None:
        out["launch_floor"] = floor
    if recompute is not None:
        out["bwd_rstd_recompute"] = recompute
    if pair is not None:
        pair["value"] = round((fb + bb) / (pair["ms_per_step"] * 1e-3) / 1e9, 2)
        pair["frac_of_peak"] = round(pair["value"] / PEAK_GBPS, 4)
        pair["bwd_gbps"] = round(bb / (pair["phases_ms"]["bwd"] * 1e-3) / 1e9, 1)
        out["qk_pair_launch"] = pair
    if graph is not None:
        if "ms_per_step" in graph:
            graph["value"] = round((fb + bb) / (graph["ms_per_step"] * 1e-3) / 1e9, 2)
        out["graph_replay"] = graph
    for n in norms:
        for c in n["calls"]:
            if c["layout"] is not None:
                c["layout"].close()
        n["acc"].close()
        n["acc_ref"].close()
    print(json.dumps(out))


GEMM_METRIC = "det_gemm fwd+bwd achieved TFLOP/s (% of bf16 MFMA peak) with bitwise B1/BN/chunk invariant dW"
BF16_PEAK_TFLOPS = 2500.0


def gemm_cpu_baseline(x_bits, w_bits, dy_bits, budget_rows=24):
    """The FP64 oracle (single-threaded C) on the first rows of the workload:
    dX of those rows and their dW contribution (2 x rows x N x K multiply-adds)."""
    import oracle
    t0 = time.perf_counter()
    oracle.linear_bwd_bf16(x_bits[:budget_rows], w_bits, dy_bits[:budget_rows])
    dt = time.perf_counter() - t0
    n, k = w_bits.shape
    flops = 2.0 * 2 * budget_rows * n * k
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"dX and dW of the first {budget_rows} rows ({n} x {k} weight), FP64 C, "
                      f"{dt:.1f} s timed"}


def measure_det_gemm(args, torch, np, binding, inputs, layouts):
    """One step = y = x W^T, dX = dY W and dW = dY^T X (one B=N call into the
    canonical accumulator, then finalize) on the linear workload (--op
    det_gemm) or the LM head (--op lm_head: N = the 32,000-token vocabulary);
    inputs resident in HBM.  torch.matmul (hipBLASLt, not batch invariant) on
    the same three products is timed beside it as a reference point, and the
    dW of the chunked-512 cell (64 calls with layouts, staged rows) beside the
    one-call dW."""
    wl = inputs.workload_lmhead() if args.op == "lm_head" else inputs.workload_linear()
    T, K, N = wl.n_logical, wl.hidden, wl.out_features
    st = torch.cuda.current_stream()
    sh = st.cuda_stream
    print(f"[bench] generating {wl.name} on the GPU", file=sys.stderr, flush=True)
    x = inputs.gen_x(wl, device="cuda")
    w = inputs.gen_wmat(wl, device="cuda")
    dy = inputs.gen_dy(wl, device="cuda")
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((N, K), dtype=torch.float32, device="cuda")
    acc = binding.GemmDwAccumulator(T, N, K)
    G = (T + 16383) // 16384
    acc_bytes = {"q": 4 * G * N * K, "staging": 2 * T * (N + K)}

    def fwd():
        binding.det_gemm_fwd(x.data_ptr(), w.data_ptr(), y.data_ptr(), T, N, K, None, sh)

    def bdx():
        binding.det_gemm_bwd_dx(dy.data_ptr(), w.data_ptr(), dx.data_ptr(), T, N, K, None, sh)

    def bdw():
        binding.det_gemm_dw_contrib(x.data_ptr(), dy.data_ptr(), T, N, K, None, acc.handle, sh)
        binding.det_gemm_dw_finalize(acc.handle, dw.data_ptr(), sh)
        binding.det_gemm_dw_acc_reset(acc.handle, sh)

    def step():
        fwd()
        bdx()
        bdw()

    def timed(f, iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(iters):
            f()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    for _ in range(args.warmup):
        step()
    K_ = max(1, args.steps // 5)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K_):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / K_ * 1e3
    # the chunked-512 cell's dW: every call's rows staged by logical index
    # (no call holds a whole 16384-row group), the group chains at finalize
    chunk_cell = layouts.chunked_packed(wl, chunk=512, name="BN/chunked_512")
    chunk_lays = [(binding.Layout(c.row_logical, T), int(c.row_logical[0]), c.rows)
                  for c in chunk_cell.calls]

    def bdw_chunked():
        for lay, a0, n_rows in chunk_lays:
            binding.det_gemm_dw_contrib(x[a0:a0 + n_rows].data_ptr(), dy[a0:a0 + n_rows].data_ptr(),
                                        n_rows, N, K, lay.handle, acc.handle, sh)
        binding.det_gemm_dw_finalize(acc.handle, dw.data_ptr(), sh)
        binding.det_gemm_dw_acc_reset(acc.handle, sh)

    ph = {"fwd": timed(fwd, K_), "dx": timed(bdx, K_), "dw": timed(bdw, K_)}
    dw_one = dw.clone()
    bdw_chunked()
    torch.cuda.synchronize()
    chunk_same = bool(torch.equal(dw.view(torch.int32), dw_one.view(torch.int32)))
    ph["dw_chunked512"] = timed(bdw_chunked, max(1, K_ // 2))
    for lay, _, _ in chunk_lays:
        lay.close()
    lib_ops = {"fwd": lambda: torch.matmul(x, w.t()), "dx": lambda: torch.matmul(dy, w),
               "dw": lambda: torch.matmul(dy.t(), x)}
    lib = {}
    for name, f in lib_ops.items():
        timed(f, 3)                      # first calls select and load the library kernels
        lib[name] = timed(f, K_)
    gf = 2.0 * T * N * K
    value = 3 * gf / (ms_step * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        cpu = gemm_cpu_baseline(inputs.bf16_bits(x[:32]), inputs.bf16_bits(w), inputs.bf16_bits(dy[:32]),
                                budget_rows=24 if N <= 8192 else 6)
    out = {
        "metric": GEMM_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K_, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "rows": T, "in_features": K, "out_features": N,
                   "layout": "BN/full (one call)", "step": "fwd + bwd_dx + dw_contrib + dw_finalize"},
        "roofline": {"bound": "mfma", "achieved": round(gf / (ph["dw"] * 1e-3) / 1e12, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gf / (ph["dw"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "dw_group_kernel<256x256, 64-deep stages, 8 wavefronts> + group tree (dW)",
                     "algorithmic_flops_per_launch": gf, "avg_launch_ms": round(ph["dw"], 5)},
        "cpu_baseline": cpu,
        "phases_ms": {k: round(v, 5) for k, v in ph.items()},
        "phases_tflops": {k: round(gf / (v * 1e-3) / 1e12, 1) for k, v in ph.items()},
        "dw_chunked512_bitwise_equal_to_one_call": chunk_same,
        "dw_accumulator_bytes": {"group_results": int(acc_bytes["q"]), "staging": int(acc_bytes["staging"])},
        "hipblaslt_torch_matmul_ms": {k: round(v, 5) for k, v in lib.items()},
        "kernel_source_hash": kernel_source_hash(GEMM_KERNEL_SOURCES),
    }
    acc.close()
    print(json.dumps(out))


EMB_METRIC = "det_embedding fwd+bwd achieved HBM GB/s (% of peak) with bitwise B1/BN/chunk invariant dE"
EMB_KERNEL_SOURCES = ("embedding.hip", "embedding.h")


def emb_cpu_baseline(ids, dy_bits, vocab, budget_rows=4096):
    """The FP64 oracle (single-threaded C) on the first rows of the batch."""
    import oracle
    t0 = time.perf_counter()
    oracle.embedding_bwd_bf16(ids[:budget_rows], dy_bits[:budget_rows], vocab)
    dt = time.perf_counter() - t0
    dim = dy_bits.shape[1]
    nbytes = budget_rows * dim * 2 + vocab * dim * 4
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"dE of the first {budget_rows} rows ({vocab} x {dim} table), FP64 C, "
                      f"{dt:.1f} s timed, same byte formula as value"}


def measure_det_embedding(args, torch, np, binding, inputs):
    """One step = y = E[ids] (gather) and dE (det_embedding_bwd: the whole
    B=N batch in one call, every table row written) on the embedding
    workload; ids, table and dY resident in HBM.  Algorithmic bytes: gather
    T*4 + 2*T*dim (table rows read) + 2*T*dim (y); gradient 2*T*dim (dY) +
    4*vocab*dim (dE).  Block partials are not counted.  The accumulator path
    (contrib + finalize) is timed beside it and checked bit for bit."""
    wl = inputs.workload_embedding()
    T, D, V = wl.n_logical, wl.hidden, wl.vocab
    st = torch.cuda.current_stream()
    sh = st.cuda_stream
    print(f"[bench] generating {wl.name}", file=sys.stderr, flush=True)
    ids_h = inputs.gen_ids(wl)
    ids = torch.from_numpy(ids_h).cuda()
    table = inputs.gen_table(wl, device="cuda")
    dy = inputs.gen_dy(wl, device="cuda")
    y = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    dE = torch.empty((V, D), dtype=torch.float32, device="cuda")
    acc = binding.EmbeddingDwAccumulator(ids_h, V, D)

    def fwd():
        binding.det_embedding_fwd(ids.data_ptr(), table.data_ptr(), y.data_ptr(), T, V, D, None, sh)

    dE_acc = torch.empty((V, D), dtype=torch.float32, device="cuda")

    def bwd():
        binding.det_embedding_bwd(dy.data_ptr(), T, D, acc.handle, dE.data_ptr(), sh)
        binding.det_embedding_dw_acc_reset(acc.handle, sh)

    def bwd_acc():
        binding.det_embedding_dw_contrib(dy.data_ptr(), T, D, None, acc.handle, sh)
        binding.det_embedding_dw_finalize(acc.handle, dE_acc.data_ptr(), sh)
        binding.det_embedding_dw_acc_reset(acc.handle, sh)

    def timed(f, iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(iters):
            f()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    for _ in range(args.warmup):
        fwd()
        bwd()
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / K * 1e3
    ph = {"fwd": timed(fwd, K), "bwd": timed(bwd, K), "bwd_accumulator": timed(bwd_acc, K)}
    same = bool(torch.equal(dE.view(torch.int32), dE_acc.view(torch.int32)))
    fb = T * 4 + 4 * T * D
    bb = 2 * T * D + 4 * V * D
    cpu = None
    if not args.no_cpu_baseline:
        cpu = emb_cpu_baseline(ids_h, inputs.bf16_bits(dy), V)
    out = {
        "metric": EMB_METRIC, "value": round((fb + bb) / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "rows": T, "vocab": V, "dim": D,
                   "distinct_tokens": int((np.bincount(ids_h, minlength=V) > 0).sum()),
                   "layout": "BN/full (one call)", "step": "fwd + det_embedding_bwd"},
        "roofline": {"bound": "hbm", "achieved": round(bb / (ph["bwd"] * 1e-3) / 1e9, 2),
                     "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(bb / (ph["bwd"] * 1e-3) / 1e9 / PEAK_GBPS, 4),
                     "traffic": measured_traffic(bb, EMB_TRAFFIC_FILE, EMB_KERNEL_SOURCES),
                     "kernel": "bwd_head_kernel (multi-block token folds, zero rows) + bwd_tail_kernel (trees, single-block tokens)",
                     "algorithmic_bytes_per_launch": bb, "avg_launch_ms": round(ph["bwd"], 5)},
        "cpu_baseline": cpu,
        "phases_ms": {k: round(v, 5) for k, v in ph.items()},
        "phases_gbps": {"fwd": round(fb / (ph["fwd"] * 1e-3) / 1e9, 1),
                        "bwd": round(bb / (ph["bwd"] * 1e-3) / 1e9, 1),
                        "bwd_accumulator": round(bb / (ph["bwd_accumulator"] * 1e-3) / 1e9, 1)},
        "one_call_equals_accumulator_bitwise": same,
        "kernel_source_hash": kernel_source_hash(EMB_KERNEL_SOURCES),
    }
    acc.close()
    print(json.dumps(out))


def measure_qk_packed(args, torch, np, binding, inputs):
    """The QK-norm workload with Q (32 heads) and K (8 heads) inside one packed
    QKV tensor [16384, 48 x 128] (V heads untouched): per step, for Q then K,
    rmsnorm_fwd_packed, rmsnorm_bwd_dx_packed with the accumulator, finalize.
    The same two norms on contiguous Q and K are timed beside it."""
    wq, wk = inputs.workload_qk("q"), inputs.workload_qk("k")
    T, d = wq.n_tokens, wq.hidden
    hq, hk = wq.heads, wk.heads
    ts = (hq + 2 * hk) * d
    st = torch.cuda.current_stream()
    sh = st.cuda_stream
    sides = []
    for wl, heads, col0 in ((wq, hq, 0), (wk, hk, hq * d)):
        x = inputs.gen_x(wl, device="cuda")
        dy = inputs.gen_dy(wl, device="cuda")
        w = inputs.gen_w(wl, device="cuda")
        sides.append(dict(wl=wl, heads=heads, col0=col0, x=x, dy=dy, w=w, rows=T * heads,
                          acc=binding.DwAccumulator(T * heads, d),
                          rstd=torch.empty(T * heads, dtype=torch.float32, device="cuda"),
                          y=torch.empty_like(x), dx=torch.empty_like(x),
                          dw=torch.empty(d, dtype=torch.float32, device="cuda")))
    qkv = torch.zeros((T, ts), dtype=torch.bfloat16, device="cuda")
    dqkv = torch.zeros_like(qkv)
    yqkv = torch.zeros_like(qkv)
    gqkv = torch.zeros_like(qkv)
    for s_ in sides:
        sl = slice(s_["col0"], s_["col0"] + s_["heads"] * d)
        qkv[:, sl] = s_["x"].view(T, -1)
        dqkv[:, sl] = s_["dy"].view(T, -1)

    def base(t, s_):
        return t.data_ptr() + 2 * s_["col0"]

    def packed_step():
        for s_ in sides:
            binding.rmsnorm_fwd_packed(base(qkv, s_), s_["w"].data_ptr(), base(yqkv, s_),
                                       s_["rstd"].data_ptr(), T, s_["heads"], d, ts, wq.eps, None, sh)
            binding.rmsnorm_bwd_dx_packed(base(qkv, s_), s_["w"].data_ptr(), base(dqkv, s_),
                                          s_["rstd"].data_ptr(), base(gqkv, s_), T, s_["heads"], d,
                                          ts, None, s_["acc"].handle, sh)
            binding.rmsnorm_dw_finalize(s_["acc"].handle, s_["dw"].data_ptr(), sh)
            binding.rmsnorm_dw_acc_reset(s_["acc"].handle, sh)

    def contiguous_step():
        for s_ in sides:
            binding.rmsnorm_fwd(s_["x"].data_ptr(), s_["w"].data_ptr(), s_["y"].data_ptr(),
                                s_["rstd"].data_ptr(), s_["rows"], d, wq.eps, None, sh)
            binding.rmsnorm_bwd_dx(s_["x"].data_ptr(), s_["w"].data_ptr(), s_["dy"].data_ptr(),
                                   s_["rstd"].data_ptr(), s_["dx"].data_ptr(), s_["rows"], d, None,
                                   s_["acc"].handle, sh)
            binding.rmsnorm_dw_finalize(s_["acc"].handle, s_["dw"].data_ptr(), sh)
            binding.rmsnorm_dw_acc_reset(s_["acc"].handle, sh)

    def timed(f, iters):
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(iters):
            f()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / iters * 1e3

    ms_p = timed(packed_step, args.steps)
    ms_c = timed(contiguous_step, args.steps)
    nbytes = 0
    for s_ in sides:
        f, b = algorithmic_bytes(s_["rows"], s_["rows"], d)
        nbytes += f + b
    out = {
        "metric": METRIC + " (per-head norm inside a packed QKV tensor)",
        "value": round(nbytes / (ms_p * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_p, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "qknorm_d128_t16384 packed", "tokens": T, "q_heads": hq, "k_heads": hk,
                   "head_dim": d, "token_stride": ts},
        "roofline": None, "cpu_baseline": None,
        "contiguous_ms_per_step": round(ms_c, 4),
        "contiguous_gbps": round(nbytes / (ms_c * 1e-3) / 1e9, 2),
        "kernel_source_hash": kernel_source_hash(),
    }
    for s_ in sides:
        s_["acc"].close()
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=3, help="rotating input/output buffer sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy", action="store_true")
    ap.add_argument("--workload", default=None,
                    help="measure another workload (info line; the default run is the headline)")
    ap.add_argument("--cell", default="BN/full", help="layout cell for --workload")
    ap.add_argument("--graph", action="store_true",
                    help="with --workload: also time the cell's steps captured in one HIP graph and replayed")
    ap.add_argument("--op", default="rms_norm",
                    choices=["rms_norm", "det_gemm", "lm_head", "det_embedding", "qk_packed"],
                    help="det_gemm: the linear layer 4096 -> 4096 on 32768 rows; lm_head: the "
                         "4096 -> 32000 vocabulary projection on 32768 rows; det_embedding: "
                         "a 32000 x 4096 table on 32768 rows (info lines)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(rows would shard across GPUs, with an all-gather of the block partials before the "
              "same finalize on every GPU).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from invariant_rmsnorm_backward_amd import binding, inputs, layouts

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    binding.load()
    torch.cuda.set_device(0)
    if args.op in ("det_gemm", "lm_head"):
        measure_det_gemm(args, torch, np, binding, inputs, layouts)
        return
    if args.op == "det_embedding":
        measure_det_embedding(args, torch, np, binding, inputs)
        return
    if args.op == "qk_packed":
        measure_qk_packed(args, torch, np, binding, inputs)
        return
    if args.workload is not None:
        measure_cell(args, torch, np, binding, inputs, layouts)
        return
    wl = inputs.workload_h4096()
    T, H = wl.n_logical, wl.hidden
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    print(f"[bench] generating {wl.name} on the GPU", file=sys.stderr, flush=True)
    x0 = inputs.gen_x(wl, device="cuda")
    dy0 = inputs.gen_dy(wl, device="cuda")
    w = inputs.gen_w(wl, device="cuda")
    sets = []
    for _ in range(args.sets):
        sets.append(dict(x=x0.clone(), dy=dy0.clone(), y=torch.empty_like(x0),
                         dx=torch.empty_like(x0),
                         rstd=torch.empty(T, dtype=torch.float32, device="cuda"),
                         dw=torch.empty(H, dtype=torch.float32, device="cuda")))
    del x0, dy0
    acc = binding.DwAccumulator(T, H)

    def step(s):
        binding.rmsnorm_fwd(s["x"].data_ptr(), w.data_ptr(), s["y"].data_ptr(), s["rstd"].data_ptr(),
                            T, H, wl.eps, None, sh)
        binding.rmsnorm_bwd_dx(s["x"].data_ptr(), w.data_ptr(), s["dy"].data_ptr(),
                               s["rstd"].data_ptr(), s["dx"].data_ptr(), T, H, None, acc.handle, sh)
        binding.rmsnorm_dw_finalize(acc.handle, s["dw"].data_ptr(), sh)
        binding.rmsnorm_dw_acc_reset(acc.handle, sh)

    # Invariance check on the benchmark data: B=N vs 8 x B=1 aggregate, bitwise.
    # The singleton calls use the dx-only and dweight-only kernel instances, so
    # the fused backward kernel only ever runs at full size in this process.
    s0 = sets[0]
    step(s0)
    ref_dw = s0["dw"].clone()
    ref_dx = s0["dx"].clone()
    acc8 = binding.DwAccumulator(T, H)
    cell = layouts.singleton_aggregate(wl)
    dx8 = torch.empty_like(s0["dx"])
    lays = []
    for call in cell.calls:
        a, b = int(call.row_logical[0]), int(call.row_logical[-1]) + 1
        lay = binding.Layout(call.row_logical, T)
        lays.append(lay)
        xs, dys = s0["x"][a:b], s0["dy"][a:b]
        y8, r8 = binding.fwd(xs, w, wl.eps, lay)
        binding.bwd(xs, w, dys, r8, lay, None, dx=dx8[a:b])
        binding.dw_contrib(xs, dys, r8, acc8, lay)
    dw8 = acc8.finalize()
    torch.cuda.synchronize()
    inv_ok = bool(torch.equal(dw8.view(torch.int32), ref_dw.view(torch.int32))
                  and torch.equal(dx8.view(torch.int16), ref_dx.view(torch.int16)))
    for lay in lays:
        lay.close()
    acc8.close()

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    K = args.steps
    # The timed region: K whole steps, nothing else on the stream.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Phase split (separate loop: events between kernels add small gaps).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        s = sets[i % len(sets)]
        e = ev[i]
        e[0].record(stream)
        binding.rmsnorm_fwd(s["x"].data_ptr(), w.data_ptr(), s["y"].data_ptr(), s["rstd"].data_ptr(),
                            T, H, wl.eps, None, sh)
        e[1].record(stream)
        binding.rmsnorm_bwd_dx(s["x"].data_ptr(), w.data_ptr(), s["dy"].data_ptr(),
                               s["rstd"].data_ptr(), s["dx"].data_ptr(), T, H, None, acc.handle, sh)
        e[2].record(stream)
        binding.rmsnorm_dw_finalize(acc.handle, s["dw"].data_ptr(), sh)
        e[3].record(stream)
        binding.rmsnorm_dw_acc_reset(acc.handle, sh)
    torch.cuda.synchronize()

    # The backward kernel alone, back to back on the same stream (the
    # accumulator reset between launches is host bookkeeping and enqueues
    # nothing), for the roofline entry.
    eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    eb0.record(stream)
    for i in range(K):
        s = sets[i % len(sets)]
        binding.rmsnorm_bwd_dx(s["x"].data_ptr(), w.data_ptr(), s["dy"].data_ptr(),
                               s["rstd"].data_ptr(), s["dx"].data_ptr(), T, H, None, acc.handle, sh)
        binding.rmsnorm_dw_acc_reset(acc.handle, sh)
    eb1.record(stream)
    torch.cuda.synchronize()
    bwd_only_ms = eb0.elapsed_time(eb1) / K

    # The rstd-recompute backward on the same rows (no rstd read; rstd rebuilt
    # in the forward's order): timed the same way, and checked bit for bit
    # against the saved-rstd backward (dx and dweight).
    s0 = sets[0]
    dx_rc = torch.empty_like(s0["dx"])
    dw_rc = torch.empty_like(s0["dw"])
    binding.rmsnorm_bwd_dx_recompute(s0["x"].data_ptr(), w.data_ptr(), s0["dy"].data_ptr(),
                                     wl.eps, dx_rc.data_ptr(), T, H, None, acc.handle, sh)
    binding.rmsnorm_dw_finalize(acc.handle, dw_rc.data_ptr(), sh)
    binding.rmsnorm_dw_acc_reset(acc.handle, sh)
    torch.cuda.synchronize()
    rc_same = bool(torch.equal(dx_rc.view(torch.int16), ref_dx.view(torch.int16))
                   and torch.equal(dw_rc.view(torch.int32), ref_dw.view(torch.int32)))
    eb0.record(stream)
    for i in range(K):
        s = sets[i % len(sets)]
        binding.rmsnorm_bwd_dx_recompute(s["x"].data_ptr(), w.data_ptr(), s["dy"].data_ptr(),
                                         wl.eps, s["dx"].data_ptr(), T, H, None, acc.handle, sh)
        binding.rmsnorm_dw_acc_reset(acc.handle, sh)
    eb1.record(stream)
    torch.cuda.synchronize()
    rc_ms = eb0.elapsed_time(eb1) / K

    fwd_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    bwd_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    fin_ms = np.array([e[2].elapsed_time(e[3]) for e in ev])
    ms_step = wall / K * 1e3
    fb, bb = algorithmic_bytes(T, T, H)
    value = (fb + bb) / (ms_step * 1e-3) / 1e9
    bwd_avg = bwd_only_ms
    achieved = bb / (bwd_avg * 1e-3) / 1e9
    traffic = measured_traffic(bb)

    copy_gbps, torch_copy_gbps = (None, None) if args.no_copy else copy_ceiling(torch, 1 << 30)
    s21_gbps = None if args.no_copy else stream_2to1(torch, 1 << 29)
    # the probe on buffers of the backward's tensor size (x, dy, dx: 32768 x 4096 bf16)
    s2p_gbps = None if args.no_copy else stream_2r1w(binding, torch, 1 << 28)
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl)

    # host-side setup, timed on its own: a layout plan for the packed, padded,
    # permuted map of the same rows, and an accumulator
    rl = layouts.packed_with_padding(inputs.scaled(wl, wl.name, pad_rows=4096)).calls[0].row_logical
    t0 = time.perf_counter()
    lay = binding.Layout(rl, T)
    setup_layout_ms = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    acc2 = binding.DwAccumulator(T, H)
    setup_acc_ms = (time.perf_counter() - t0) * 1e3
    lay.close()
    acc2.close()

    def pct(a, q):
        return round(float(np.percentile(a, q)), 5)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "hidden": H, "rows": T, "samples": "8 x 4096 tokens",
                   "layout": "BN/full (one call)", "io_dtype": "bf16", "eps": wl.eps,
                   "step": "fwd + bwd_dx(fused dweight contributions) + dw_finalize",
                   "buffer_sets": args.sets},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "bwd_team_kernel<V=2,TW=4,TEAMS=2,PD=1,FULL,identity,DX,DW> (two rows in flight per "
                               "workgroup, 4 wavefronts per row, 64-row block walked in two passes)",
                     "algorithmic_bytes_per_launch": bb, "avg_launch_ms": round(bwd_avg, 5)},
        "cpu_baseline": cpu,
        "phases_ms": {"fwd": round(float(np.median(fwd_ms)), 5),
                      "bwd": round(float(np.median(bwd_ms)), 5),
                      "finalize": round(float(np.median(fin_ms)), 5)},
        "phases_ms_p10_p90": {"fwd": [pct(fwd_ms, 10), pct(fwd_ms, 90)],
                              "bwd": [pct(bwd_ms, 10), pct(bwd_ms, 90)],
                              "finalize": [pct(fin_ms, 10), pct(fin_ms, 90)]},
        "phases_gbps": {"fwd": round(fb / (float(np.median(fwd_ms)) * 1e-3) / 1e9, 1),
                        "bwd": round(bb / (float(np.median(bwd_ms)) * 1e-3) / 1e9, 1)},
        "setup_ms": {"layout_create_36864_rows": round(setup_layout_ms, 3),
                     "dw_acc_create": round(setup_acc_ms, 3)},
        "rows_per_s": round(T / (ms_step * 1e-3), 1),
        "frac_of_peak": round(value / PEAK_GBPS, 4),
        "copy_ceiling_gbps": None if copy_gbps is None else round(copy_gbps, 1),
        "frac_of_copy_ceiling": None if copy_gbps is None else round(value / copy_gbps, 4),
        "torch_copy_gbps": None if torch_copy_gbps is None else round(torch_copy_gbps, 1),
        "stream_2to1_gbps": None if s21_gbps is None else round(s21_gbps, 1),
        "bwd_frac_of_stream_2to1": None if s21_gbps is None else round(achieved / s21_gbps, 4),
        "stream_2r1w_gbps": None if s2p_gbps is None else round(s2p_gbps, 1),
        "bwd_frac_of_stream_2r1w": None if s2p_gbps is None else round(achieved / s2p_gbps, 4),
        "invariance_bn_vs_8xb1_bitwise": inv_ok,
        "bwd_rstd_recompute": {"avg_launch_ms": round(rc_ms, 5),
                               "gbps": round((bb - 4 * T) / (rc_ms * 1e-3) / 1e9, 1),
                               "bitwise_equal_to_saved_rstd": rc_same},
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
