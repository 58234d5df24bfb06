#!/usr/bin/env python3
"""Benchmark of the fused Echo rank pipeline on one MI355X.

Workload (default): a 1 GB message -- one rank's bf16 vector of 2^29
elements, N(0,1) with 0.1% of elements x20, P = 8 logical ranks, this rank 0,
group 128; the 7 incoming stage-1 shards of this rank's 2^26-element chunk
and the 7 gathered stage-2 chunks are seeded int4 messages resident in HBM.
The averages are carried across calls.  A step is one call: the entry phase
(K_entry), the own-chunk reduce phase (K_reduce) and the exit phase
(K_exit) -- exactly the launches echo_call makes -- on one stream.

Prints one JSON line: payload GB/s (2 bytes per element per call), the
roofline of the dominant kernel (K_entry) from HIP events recorded on the
launch stream inside the timed region, and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GB/s of bf16 payload through fused Echo rank pipeline @1GB msg; % HBM peak"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD's published peak


def bytes_per_element(P: int, bits: int = 4) -> dict:
    """Algorithmic HBM bytes per element of each kernel's range."""
    code = bits / 8.0 + 4.0 / 128.0  # code + share of the fp32 group scale
    return {
        "entry": 2 + 8 + 8 + code,             # x, 2 averages in, 2 out, send message
        "reduce": 2 + 8 + 8 + 2 + code * P,    # x, averages in/out, y, P-1 shards in + codes2 out
        "exit": code + 2,                      # gathered message in, y out
    }


def rs_bytes(N: int, P: int) -> float:
    """Algorithmic bytes of the reduce-scatter call: the entry pass plus the
    own chunk's x, averages, P-1 incoming shards and bf16 output."""
    code = 0.5 + 4.0 / 128.0
    C = N // P
    return (N - C) * bytes_per_element(P)["entry"] + C * (2 + 16 + code * (P - 1) + 2)


def step_bytes(N: int, P: int, bits: int = 4) -> float:
    b = bytes_per_element(P, bits)
    C = N // P
    return (N - C) * b["entry"] + C * b["reduce"] + (N - C) * b["exit"]


def source_hash() -> str:
    """Hash of the kernel and launch sources with comments and whitespace
    removed (a comment edit does not change the kernels)."""
    import re

    h = hashlib.sha256()
    for rel in ("error_compensated_bit_echo_amd/csrc/echo_device.h",
                "error_compensated_bit_echo_amd/csrc/launch_shape.h",
                "error_compensated_bit_echo_amd/csrc/echo_api.hip",
                "error_compensated_bit_echo_amd/build.py"):
        with open(os.path.join(ROOT, rel)) as f:
            src = f.read()
        if rel.endswith(".py"):
            src = re.sub(r'""".*?"""', "", src, flags=re.S)
            src = re.sub(r"#[^\n]*", "", src)
        else:
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            src = re.sub(r"//[^\n]*", "", src)
        h.update("".join(src.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; None otherwise."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload, {}).get(kernel)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_launch")


def make_messages(N: int, P: int, rank: int, seed: int = 0):
    """The seeded incoming stage-1 shards and gathered stage-2 chunks of the
    workload's own call."""
    import numpy as np

    from error_compensated_bit_echo_amd import inputs as I

    C = N // P
    tag = ("echo-1gb", seed)
    recv = [None if q == rank else I.int4_message(C, I.stream_key(*tag, "recv", q))
            for q in range(P)]
    # gathered stage-2 chunks carry sums of P contributions: larger scales
    gath = [None if j == rank else
            I.int4_message(C, I.stream_key(*tag, "gath", j),
                           scale_lo=0.05 * np.sqrt(P), scale_hi=0.55 * np.sqrt(P))
            for j in range(P)]
    return recv, gath


def make_workload(N: int, P: int, rank: int, seed: int = 0):
    from error_compensated_bit_echo_amd import inputs as I

    x = I.vector_with_outliers(N, I.stream_key("echo-1gb", seed, "x"), outlier_mult=20.0)
    recv, gath = make_messages(N, P, rank, seed)
    return x, recv, gath


def host_cpu() -> str:
    """CPU model and logical CPU count of the host the oracle ran on."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return (f"{model}, {os.cpu_count()} logical CPUs visible, "
            f"{len(os.sched_getaffinity(0))} usable by this process")


def oracle_threads() -> int:
    """Host threads for the oracle's all-core leg: the CPUs this process may
    run on, at most 16 (one GPU's share of the host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(x, recv, gath, P: int, rank: int, n_sample: int, calls: int):
    """The CPU oracle as it stands, rank-mode calls on the first n_sample
    elements of the workload (the whole workload by default; a smaller
    sample's chunks are prefixes of the workload's shards), from zero state:
    one call on one thread, then `calls` calls on all host cores through the
    oracle's threaded driver (the single-thread step functions over disjoint
    runs of groups), state carried.  The first all-core call must give the
    single-thread call's bytes.  Payload GB/s of each."""
    import numpy as np

    from oracle import oracle as orc

    Cs = n_sample // P
    xs = np.ascontiguousarray(x[:n_sample])
    rc = [None if m is None else np.ascontiguousarray(m[0][:Cs // 2]) for m in recv]
    rs = [None if m is None else np.ascontiguousarray(m[1][:Cs // 128]) for m in recv]
    gc = [None if m is None else np.ascontiguousarray(m[0][:Cs // 2]) for m in gath]
    gs = [None if m is None else np.ascontiguousarray(m[1][:Cs // 128]) for m in gath]
    T = oracle_threads()
    mf, ms = np.zeros(n_sample, np.float32), np.zeros(n_sample, np.float32)
    t0 = time.perf_counter()
    one = orc.call(P, rank, xs, mf, ms, rc, rs, gc, gs, threads=1)
    dt1 = time.perf_counter() - t0
    mf[:] = 0.0
    ms[:] = 0.0
    out, dtT = None, []
    for k in range(max(1, calls)):
        t0 = time.perf_counter()
        out = orc.call(P, rank, xs, mf, ms, rc, rs, gc, gs, threads=T, out=out)
        dtT.append(time.perf_counter() - t0)
        if k == 0:
            same = all(np.array_equal(out[key], one[key]) for key in one)
            del one
    gbps = lambda dt: round(2.0 * n_sample / dt / 1e9, 4)  # noqa: E731
    alg = lambda dt: round(step_bytes(n_sample, P) / dt / 1e9, 3)  # noqa: E731
    mean_T = float(np.mean(dtT))
    return {
        "value": gbps(mean_T),
        "unit": "GB/s",
        "cores": T,
        "kind": "oracle",
        "sample": (f"rank-mode calls (P={P}, rank {rank}) on {n_sample} elements"
                   f"{' (the whole workload)' if n_sample == x.size else ''} from zero state: "
                   f"1 call on 1 thread ({dt1:.2f} s), then {len(dtT)} calls on {T} threads, "
                   f"state carried ({sum(dtT):.2f} s)"),
        "single_thread": {"GBps": gbps(dt1), "algorithmic_GBps": alg(dt1), "s_per_call": round(dt1, 3)},
        "all_cores": {"GBps": gbps(mean_T), "algorithmic_GBps": alg(mean_T), "s_per_call": round(mean_T, 3),
                      "threads": T},
        "all_core_output_equals_single_thread": bool(same),
        "host": host_cpu(),
    }


def cu_partition_streams(torch, frac):
    """Two streams over disjoint sets of compute units, made before any other
    stream (a CU-masked stream needs a hardware queue of its own): in every
    32-CU word of the mask, the low `frac` of the CUs for the update and the
    rest for the matmul.  The runtime on MI355X accepts masks whose set bits
    come in whole runs of 8 within each word (measured: 0xFF, 0xFFFF,
    0x00FF00FF, 0xFFFFFF00 per word work; 0x0F, 0x0F0F0F0F, 0x33333333,
    0x55555555 are refused with hipErrorOutOfMemory), so frac is rounded to a
    multiple of 1/4."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    k = min(24, max(8, 8 * round(frac * 4)))  # CUs of each 32 for the update
    upd = [c for c in range(ncu) if c % 32 < k]
    rest = [c for c in range(ncu) if c % 32 >= k]
    return cu_masked_stream(torch, upd), cu_masked_stream(torch, rest), len(upd), len(rest)


def cu_masked_stream(torch, cus):
    """A stream whose kernels may run only on the compute units listed (HIP's
    hipExtStreamCreateWithCUMask, default priority), wrapped for torch."""
    import ctypes
    import re

    with open("/proc/self/maps") as f:
        path = sorted(set(re.findall(r"(/\S*libamdhip64\.so\S*)", f.read())))[0]
    hip = ctypes.CDLL(path)
    words = (ctypes.c_uint32 * 32)()
    for c in cus:
        words[c // 32] |= 1 << (c % 32)
    nwords = (max(cus) // 32) + 1
    handle = ctypes.c_void_p()
    rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), ctypes.c_uint32(nwords), words)
    if rc != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask failed ({rc})")
    return torch.cuda.ExternalStream(handle.value)


def schedules(B, torch, st, xd, rc_, rs_, gc_, gs_, send_c, send_s, own_c, own_s, y, e2,
              N, P, rank, steps, cu_streams=()):
    """The compensation's cost on the critical path (in the pages' schedule
    the averages' update overlaps the following matrix multiplication).  Times, per
    call: the fused call; the uncompensated call; the split schedule's
    critical path (entry pass with the averages read-only, reduce, exit)
    with the update on a side stream; and each followed by a matmul that
    consumes y -- one TP=8 shard of a Llama-3-8B MLP up-projection,
    [N/4096 x 4096] @ [4096 x 1792] in bf16."""
    C = N // P
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    w = torch.randn(4096, 1792, device=y.device, dtype=torch.bfloat16) * 0.02
    yb = y.view(torch.bfloat16).reshape(-1, 4096)
    sh_c = [send_c[rank * C // 2:(rank + 1) * C // 2] if q == rank else rc_[q] for q in range(P)]
    sh_s = [send_s[rank * C // 128:(rank + 1) * C // 128] if q == rank else rs_[q] for q in range(P)]

    def fused():
        B.echo_call(st, xd, rc_, rs_, gc_, gs_, send_c, send_s, own_c, own_s, y, main)

    def plain():
        B.echo_call_plain(P, rank, xd, rc_, rs_, gc_, gs_, send_c, send_s, own_c, own_s, y,
                          stream=main)

    state = {"updated": None}

    def wait_update():
        if state["updated"] is not None:
            main.wait_event(state["updated"])

    def split_critical():
        B.echo_encode(st, xd, send_c, send_s, main)
        B.echo_reduce_shard(sh_c, sh_s, own_c, own_s, y[rank * C:(rank + 1) * C], e2, chunk_n=C,
                            stream=main)
        B.echo_call_exit(st, gc_, gs_, y, main)
        done = torch.cuda.Event()  # the update starts once the critical path is done
        done.record(main)
        return done

    def split_update(reduced):
        side.wait_event(reduced)
        B.echo_update(st, xd, send_c, send_s, e2, side)
        ev = torch.cuda.Event()
        ev.record(side)
        state["updated"] = ev

    def gemm():
        return yb @ w

    def timed(body, k=steps):
        body()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                torch.cuda.Event(enable_timing=True)) for _ in range(k)]
        t0 = time.perf_counter()
        for e in evs:
            body(e)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / k
        first = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        return wall, first

    import numpy as np

    def b_fused(e=None):
        if e: e[0].record(main)
        fused()
        if e: e[1].record(main)
        gemm()

    def b_plain(e=None):
        if e: e[0].record(main)
        plain()
        if e: e[1].record(main)
        gemm()

    def b_split(e=None):
        wait_update()  # the entry pass reads the averages the previous update wrote
        if e: e[0].record(main)
        reduced = split_critical()
        if e: e[1].record(main)
        gemm()
        split_update(reduced)

    corr = torch.empty(N, dtype=torch.float32, device=y.device)
    B.echo_correction(st, corr, main)

    def split_corr_critical():
        B.echo_encode_corr(st, xd, corr, send_c, send_s, main)
        B.echo_reduce_shard(sh_c, sh_s, own_c, own_s, y[rank * C:(rank + 1) * C], e2, chunk_n=C,
                            stream=main)
        B.echo_call_exit(st, gc_, gs_, y, main)
        done = torch.cuda.Event()
        done.record(main)
        return done

    def split_corr_update(reduced):
        side.wait_event(reduced)
        B.echo_update_corr(st, xd, send_c, send_s, e2, corr, side)
        ev = torch.cuda.Event()
        ev.record(side)
        state["updated"] = ev

    def b_split_corr(e=None):
        wait_update()  # the entry pass reads the correction the previous update wrote
        if e: e[0].record(main)
        reduced = split_corr_critical()
        if e: e[1].record(main)
        gemm()
        split_corr_update(reduced)

    def b_update_corr(e=None):
        if e: e[0].record(main)
        B.echo_update_corr(st, xd, send_c, send_s, e2, corr, main)
        if e: e[1].record(main)

    def b_gemm(e=None):
        if e: e[0].record(main)
        gemm()
        if e: e[1].record(main)

    def b_update(e=None):
        if e: e[0].record(main)
        B.echo_update(st, xd, send_c, send_s, e2, main)
        if e: e[1].record(main)

    y_own = torch.empty(C, dtype=torch.int16, device=y.device)
    # The reduce-scatter call has no exit pass, whose loads would push the
    # incoming shards out of the 256 MB Infinity Cache between calls, and its
    # entry pass is non-temporal: calls on one message set would find the
    # previous call's shards (238 MB) cached.  Three copies, cycled, keep
    # every call's shards coming from HBM, as a fresh message's would.
    NSETS = 3
    rs_sets = [(rc_, rs_)] + [([None if t is None else t.clone() for t in rc_],
                               [None if t is None else t.clone() for t in rs_]) for _ in range(NSETS - 1)]
    turn = {"rs": 0, "call8": 0}

    def b_rs(e=None):
        rc_k, rs_k = rs_sets[turn["rs"] % NSETS]
        turn["rs"] += 1
        if e: e[0].record(main)
        B.echo_rs_call(st, xd, rc_k, rs_k, send_c, send_s, y_own, main)
        if e: e[1].record(main)

    # the 8-bit promotion of a call: the same call with one byte per code
    # (seeded random 8-bit messages drawn on the device: only the bytes moved
    # matter for the timing)
    g8 = torch.Generator(device=y.device)
    g8.manual_seed(8)

    def msg8():
        c = torch.randint(0, 256, (C,), device=y.device, generator=g8, dtype=torch.uint8)
        c[c == 0x80] = 0x7F
        sc = torch.rand(C // 128, device=y.device, generator=g8) * 0.01 + 0.001
        return c, sc

    def set8():
        # incoming shards and gathered chunks of one 8-bit call, distinct buffers
        m8 = [None if q == rank else msg8() for q in range(P)]
        g8m = [None if q == rank else msg8() for q in range(P)]
        return ([None if m is None else m[0] for m in m8], [None if m is None else m[1] for m in m8],
                [None if m is None else m[0] for m in g8m], [None if m is None else m[1] for m in g8m])

    sets8 = [set8() for _ in range(NSETS)]
    send_c8 = torch.empty(N, dtype=torch.uint8, device=y.device)
    own_c8 = torch.empty(C, dtype=torch.uint8, device=y.device)

    def b_call8(e=None):
        rc8, rs8, gc8, gs8 = sets8[turn["call8"] % NSETS]
        turn["call8"] += 1
        st.bits = 8
        if e: e[0].record(main)
        B.echo_call(st, xd, rc8, rs8, gc8, gs8, send_c8, send_s, own_c8, own_s, y, main)
        if e: e[1].record(main)
        st.bits = 4

    out = {}
    for name, body in (("gemm", b_gemm), ("fused", b_fused), ("plain", b_plain), ("split", b_split),
                       ("update_alone", b_update), ("rs", b_rs), ("call8", b_call8)):
        wall, first = timed(body)
        out[name] = (wall, first)
        if name == "split":
            main.wait_event(state["updated"])
            state["updated"] = None
    # the correction array must come from the averages the other schedules left
    B.echo_correction(st, corr, main)
    for name, body in (("split_corr", b_split_corr), ("update_corr_alone", b_update_corr)):
        wall, first = timed(body)
        out[name] = (wall, first)
        if name == "split_corr":
            main.wait_event(state["updated"])
            state["updated"] = None
    torch.cuda.synchronize()

    # The split schedule with the compute units partitioned: the matmul on a
    # stream limited to one part, the update on a stream limited to the other.
    cu_rows = []
    for s_upd, s_mm, n_upd, n_mm in cu_streams:

        def b_cu(e=None, s_upd=s_upd, s_mm=s_mm):
            wait_update()
            if e: e[0].record(main)
            reduced = split_corr_critical()
            if e: e[1].record(main)
            s_mm.wait_event(reduced)
            with torch.cuda.stream(s_mm):
                gemm()
            s_upd.wait_event(reduced)
            B.echo_update_corr(st, xd, send_c, send_s, e2, corr, s_upd)
            ev = torch.cuda.Event()
            ev.record(s_upd)
            state["updated"] = ev
            main.wait_stream(s_mm)

        def b_upd_only(e=None, s_upd=s_upd):
            s_upd.wait_stream(main)
            if e: e[0].record(s_upd)
            B.echo_update_corr(st, xd, send_c, send_s, e2, corr, s_upd)
            if e: e[1].record(s_upd)
            main.wait_stream(s_upd)

        def b_mm_only(e=None, s_mm=s_mm):
            s_mm.wait_stream(main)
            if e: e[0].record(s_mm)
            with torch.cuda.stream(s_mm):
                gemm()
            if e: e[1].record(s_mm)
            main.wait_stream(s_mm)

        wall, _ = timed(b_cu)
        main.wait_event(state["updated"])
        state["updated"] = None
        _, upd_ms = timed(b_upd_only)
        _, mm_ms = timed(b_mm_only)
        torch.cuda.synchronize()
        cu_rows.append({"update_cus": n_upd, "matmul_cus": n_mm,
                        "split_corr+matmul_ms": round(wall, 4), "update_corr_alone_ms": round(upd_ms, 4),
                        "matmul_alone_ms": round(mm_ms, 4)})
    torch.cuda.synchronize()
    return {
        "matmul": "[%d x 4096] @ [4096 x 1792] bf16" % (N // 4096),
        "matmul_ms": round(out["gemm"][1], 4),
        "fused_call_ms": round(out["fused"][1], 4),
        "plain_call_ms": round(out["plain"][1], 4),
        "split_critical_ms": round(out["split"][1], 4),
        "update_alone_ms": round(out["update_alone"][1], 4),
        "split_corr_critical_ms": round(out["split_corr"][1], 4),
        "update_corr_alone_ms": round(out["update_corr_alone"][1], 4),
        "layer_ms": {"fused+matmul": round(out["fused"][0], 4), "plain+matmul": round(out["plain"][0], 4),
                     "split+matmul(update beside it)": round(out["split"][0], 4),
                     "split_corr+matmul(update beside it)": round(out["split_corr"][0], 4)},
        "call_8bit_ms": round(out["call8"][1], 4),
        "call_8bit_GBps": round(step_bytes(N, P, bits=8) / (out["call8"][1] * 1e-3) / 1e9, 1),
        "reduce_scatter_call_ms": round(out["rs"][1], 4),
        "reduce_scatter_GBps": round(rs_bytes(N, P) / (out["rs"][1] * 1e-3) / 1e9, 1),
        "cu_partitioned": cu_rows,
        "compensation_on_critical_path_ms": {
            "fused": round(out["fused"][1] - out["plain"][1], 4),
            "split": round(out["split"][1] - out["plain"][1], 4),
            "split_corr": round(out["split_corr"][1] - out["plain"][1], 4)},
    }


# message sets cycled by the smaller workloads (see run_workload)
MESSAGE_POOL = 16

WORKLOADS = {
    # name: (elements per rank, calls per step, description)
    "tiny": (16 * 4096, 4, "bf16 [16 x 4096] per rank, N(0,1), 0.1% of channels x20; 4 calls per step"),
    "decode": (256 * 4096, 64, "Llama-3-8B TP=8 decode site: bf16 [256 x 4096] per rank, 0.5 z lambda_c, "
                               "0.1% of channels x30; 64 calls (32 layers x 2 sites) per step"),
    "prefill": (8192 * 4096, 1, "Llama-3-8B TP=8 prefill site: bf16 [8192 x 4096] per rank; one call "
                                "on warm state per step"),
    "train": (8 * 4096 * 1024, 112, "Qwen3-0.6B TP=8 training step: bf16 [8 x 4096 x 1024]; 56 forward "
                                    "calls on one state, 56 backward calls (1e-3 Student-t(3)) on another"),
}


def practical_ceiling(B, torch, stream, nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """The library's plain streaming copy (16 bytes per lane, non-temporal,
    a grid covering the range) over nbytes: the bandwidth a kernel with no
    arithmetic reaches on this GPU, read + write bytes per second."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        B.echo_stream_copy(src, dst, nbytes, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        B.echo_stream_copy(src, dst, nbytes, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"kernel": "echo_stream_copy (16 B per lane, non-temporal)", "bytes_per_launch": 2 * nbytes,
            "GBps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def run_sweep(args) -> int:
    """Time per fused call (rank 0 of P = 8) over message sizes from 2^16 to
    2^29 elements; small sizes replay a captured graph of 64 calls so the
    figure is the GPU's, not the host's.  Calls cycle a pool of message
    sets."""
    import torch

    from error_compensated_bit_echo_amd import binding as B

    dev = torch.device("cuda:0")
    P, rank = 8, 0
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    rows = []
    for log2n in range(16, 30):
        n = 1 << log2n
        C = n // P
        print(f"bench: sweep n=2^{log2n}", file=sys.stderr, flush=True)
        x = torch.randn(n, device=dev, generator=gen).to(torch.bfloat16).view(torch.int16)

        def msg():
            c = torch.randint(0, 256, (C // 2,), device=dev, generator=gen, dtype=torch.uint8)
            c = torch.where((c & 15) == 8, c ^ 1, c)
            c = torch.where((c >> 4) == 8, c ^ 16, c)
            return c, torch.rand(C // 128, device=dev, generator=gen) * 0.5 + 0.05

        # a pool of message sets, cycled call by call: 2^29 bytes or more
        # (twice the Infinity Cache) where 16 sets reach it, so the larger
        # sizes read every call's messages from HBM
        set_bytes = 2 * (P - 1) * (C // 2 + C // 32)
        nsets = max(2, min(16, -(-(1 << 29) // set_bytes)))
        sl = lambda arr, k: [None if m is None else m[k] for m in arr]  # noqa: E731
        pool = []
        for _ in range(nsets):
            recv = [None if q == rank else msg() for q in range(P)]
            gath = [None if j == rank else msg() for j in range(P)]
            pool.append((sl(recv, 0), sl(recv, 1), sl(gath, 0), sl(gath, 1)))
        mf, ms = torch.empty(n, device=dev), torch.empty(n, device=dev)
        st = B.echo_state_init(mf, ms, n, P, rank)
        send_c = torch.empty(n // 2, dtype=torch.uint8, device=dev)
        send_s = torch.empty(n // 128, device=dev)
        own_c = torch.empty(C // 2, dtype=torch.uint8, device=dev)
        own_s = torch.empty(C // 128, device=dev)
        y = torch.empty(n, dtype=torch.int16, device=dev)
        calls = [B.echo_call_prepare(st, x, *m, send_c, send_s, own_c, own_s, y) for m in pool]
        reps = 64 if log2n < 24 else 8 * nsets
        if log2n < 24:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for i in range(reps):
                    calls[i % nsets](side)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(reps):
                    calls[i % nsets]()
            run = g.replay
        else:
            def run():
                for i in range(reps):
                    calls[i % nsets]()
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            run()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (5 * reps)
        rows.append({"elements": n, "us_per_call": round(us, 2),
                     "payload_GBps": round(2.0 * n / (us * 1e-6) / 1e9, 1),
                     "pct_hbm_peak": round(100.0 * step_bytes(n, P) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)})
        del x, recv, gath, pool, mf, ms, send_c, send_s, own_c, own_s, y, calls, st
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "fused Echo call time vs message size (rank 0 of 8)", "unit": "us",
                      "dtype": "f32", "data": "synthetic", "n_gpus": 1, "sweep": rows}), flush=True)
    return 0


def calibration_copy(dev) -> None:
    """A plain device copy of known size (reads 1 GiB, writes 1 GiB): the
    reference that scales HBM counter readings to bytes."""
    import torch

    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def run_workload(args) -> int:
    """Per-rank timing of the smaller workloads (rank 0 of P = 8): a step is
    the workload's whole call sequence; inputs differ call to call, and the
    messages come from a pool of sets cycled call by call.  With --graph each
    of the pool's step variants is also captured in a HIP graph and the
    graphs are replayed in turn."""
    import numpy as np
    import torch

    from error_compensated_bit_echo_amd import binding as B
    from error_compensated_bit_echo_amd import inputs as I

    n, calls, desc = WORKLOADS[args.workload]
    P, rank = 8, 0
    C = n // P
    dev = torch.device("cuda:0")
    print(f"bench: workload {args.workload}: n={n}, {calls} calls per step", file=sys.stderr, flush=True)

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    # inputs, one per call of a step
    if args.workload == "tiny":
        ck = I.stream_key("tiny", "channels")
        xs = [d(I.gaussian_outlier_channels(16, 4096, I.stream_key("tiny", c), channel_key=ck))
              for c in range(calls)]
    elif args.workload in ("decode", "prefill"):
        ck = I.stream_key(args.workload, "channels")
        rows = n // 4096
        xs = [d(I.lognormal_channel_activations(rows, 4096, I.stream_key(args.workload, c), ck))
              for c in range(calls)]
    else:
        lam = I.channel_scales(1024, I.stream_key("train", "channels"))
        xs = [I.device_lognormal_channel_activations(n // 1024, 1024, 1000 + c, lam, dev)
              for c in range(calls // 2)]
        xs += [I.device_student_t3(n, 2000 + c, dev) for c in range(calls // 2)]
    # the serving policy of the pages: the first half of the layers' calls
    # carry 8-bit codes, the rest 4-bit codes
    bits_of = [8 if args.serving_policy and c < calls // 2 else 4 for c in range(calls)]
    # Incoming shards and gathered chunks: K seeded sets drawn on the device;
    # call g of the run (counted over steps) takes set g % K.  A set is read
    # again only after K - 1 others, and at the prefill and training sizes the
    # K sets hold about twice the 256 MB Infinity Cache, so their calls read
    # every message from HBM as fresh messages would be (one set re-read call
    # after call would stay cached: 5% faster there).  At the decode and tiny
    # sizes all K sets fit the cache, as the messages of a whole step do.
    K = MESSAGE_POOL
    sl = lambda arr, k: [None if m is None else m[k] for m in arr]  # noqa: E731
    msgs_d = {}
    for bits in sorted(set(bits_of)):
        pool = []
        for k in range(K):
            recv = [None if q == rank else I.device_message(C, I.stream_key("w-recv", k, q, bits), dev, bits=bits)
                    for q in range(P)]
            gath = [None if j == rank else I.device_message(C, I.stream_key("w-gath", k, j, bits), dev,
                                                            scale_lo=0.15, scale_hi=1.5, bits=bits)
                    for j in range(P)]
            pool.append((sl(recv, 0), sl(recv, 1), sl(gath, 0), sl(gath, 1)))
        msgs_d[bits] = pool
    nstates = 2 if args.workload == "train" else 1
    mem = [(torch.empty(n, device=dev), torch.empty(n, device=dev)) for _ in range(nstates)]
    stream = torch.cuda.current_stream()
    states = [B.echo_state_init(a, b, n, P, rank, stream) for a, b in mem]
    # the same averages seen by 8-bit calls
    states8 = [B.EchoState(a, b, n, P, rank, bits=8) for a, b in mem]
    send_c = torch.empty(n, dtype=torch.uint8, device=dev)  # room for 8-bit codes
    send_s = torch.empty(n // 128, dtype=torch.float32, device=dev)
    own_c = torch.empty(C, dtype=torch.uint8, device=dev)
    own_s = torch.empty(C // 128, dtype=torch.float32, device=dev)
    ys = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(calls)]

    # one prepared call per call of the step (arguments marshalled once)
    def state_of(c):
        k = 0 if c < calls // nstates or nstates == 1 else 1
        return states8[k] if bits_of[c] == 8 else states[k]

    # step variant v: call c takes message set (v * calls + c) % K
    L = K // math.gcd(K, calls)
    prepared = [[B.echo_call_prepare(state_of(c), xs[c], *msgs_d[bits_of[c]][(v * calls + c) % K], send_c,
                                     send_s, own_c, own_s, ys[c])
                 for c in range(calls)] for v in range(L)]

    def step(v):
        s = torch.cuda.current_stream()
        for pc in prepared[v % L]:
            pc(s)

    if args.calibrate:
        calibration_copy(dev)

    for w in range(max(1, args.warmup)):
        step(w)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    graph_ms = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)  # warm the side stream before capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for v in range(L):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(v)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            graphs[k % L].replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    best = min(eager_ms, graph_ms) if graph_ms else eager_ms
    per_call = sum(step_bytes(n, P, bits=b) for b in bits_of) / calls
    policy = " (serving policy: first half of the calls 8-bit)" if args.serving_policy else ""
    out = {
        "metric": f"GB/s of bf16 payload through fused Echo rank pipeline @{args.workload} workload{policy}; "
                  "% HBM peak",
        "value": round(2.0 * n * calls / (best * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(best, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {desc}{policy}", "elements": n, "nranks": P, "rank": rank,
                   "calls_per_step": calls, "calls_8bit": bits_of.count(8), "message_sets": K},
        "us_per_call": round(best * 1e3 / calls, 2),
        "eager_ms_per_step": round(eager_ms, 4),
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
        "pct_hbm_peak": round(100.0 * per_call * calls / (best * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "algorithmic_bytes_per_call": int(per_call),
    }
    def host_msgs(c):
        """host copies of the messages of call c of the first step"""
        return tuple([None if t is None else t.cpu().numpy() for t in ts]
                     for ts in msgs_d[bits_of[c]][c % K])

    out["cpu_baseline"] = None if args.no_cpu else workload_cpu_baseline(
        xs, host_msgs, bits_of, P, rank, nstates, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def workload_cpu_baseline(xs, msgs_of, bits_of, P: int, rank: int, nstates: int, budget_s: float):
    """The CPU oracle as it stands on the workload's own call sequence, from
    zero state (one state per direction for the training step): the first
    call on one thread, then the step's calls in order on all host cores
    (the oracle's threaded driver) until the step ends or about budget_s
    seconds have passed; payload GB/s of each."""
    import numpy as np

    from oracle import oracle as orc

    n = int(xs[0].numel())
    calls = len(xs)
    T = oracle_threads()
    x0 = xs[0].cpu().numpy().view(np.uint16)
    mf, ms = np.zeros(n, np.float32), np.zeros(n, np.float32)
    m0 = msgs_of(0)
    t0 = time.perf_counter()
    orc.call(P, rank, x0, mf, ms, *m0, threads=1, bits=bits_of[0])
    dt1 = time.perf_counter() - t0
    states = [(np.zeros(n, np.float32), np.zeros(n, np.float32)) for _ in range(nstates)]
    done, spent, outs = 0, 0.0, {}
    while done < calls and (done == 0 or spent < budget_s):
        x = xs[done].cpu().numpy().view(np.uint16)
        mf, ms = states[0] if nstates == 1 or done < calls // nstates else states[1]
        b = bits_of[done]
        m = msgs_of(done)
        t0 = time.perf_counter()
        outs[b] = orc.call(P, rank, x, mf, ms, *m, threads=T, out=outs.get(b), bits=b)
        spent += time.perf_counter() - t0
        done += 1
    return {
        "value": round(2.0 * n * done / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": T,
        "kind": "oracle",
        "sample": f"the step's first call on 1 thread ({dt1:.3f} s), then its first {done} of "
                  f"{calls} rank-mode calls (P={P}, rank {rank}), {n} elements each, state carried, "
                  f"on {T} threads ({spent:.2f} s)",
        "single_thread": {"GBps": round(2.0 * n / dt1 / 1e9, 4), "s_per_call": round(dt1, 4)},
        "host": host_cpu(),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--log2n", type=int, default=29, help="elements per rank = 2^log2n")
    ap.add_argument("--nranks", type=int, default=8)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-log2n", type=int, default=29,
                    help="oracle leg: elements of the sample = 2^cpu_log2n (capped at the workload)")
    ap.add_argument("--cpu-calls", type=int, default=3, help="oracle leg: calls on all host cores")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="smaller workloads: CPU time budget of the oracle leg")
    ap.add_argument("--no-schedules", action="store_true",
                    help="skip the critical-path comparison (fused / split / uncompensated)")
    ap.add_argument("--message-sets", type=int, default=3,
                    help="distinct sets of incoming and gathered messages, cycled call by call")
    ap.add_argument("--cu-split", type=float, default=None,
                    help="also time the split schedule with the compute units partitioned: the "
                         "update's stream gets this fraction of the CUs and the matmul's the rest")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain 1 GiB device copy (torch) before the warmup, as "
                         "the known-size reference for HBM counter runs")
    ap.add_argument("--workload", default="1gb", choices=["1gb", *WORKLOADS],
                    help="1gb (the headline, default) or one of the smaller workloads")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline: time per fused call for 2^16 .. 2^29 elements")
    ap.add_argument("--graph", action="store_true",
                    help="smaller workloads: also time the step captured in a HIP graph")
    ap.add_argument("--serving-policy", action="store_true",
                    help="tiny/decode workloads: the first half of the calls (layers) with 8-bit codes, "
                         "as the pages serve Llama-3-8B")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures the per-rank pipeline on one GPU; the library has no "
              "multi-GPU transport, so --gpus must be 1", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0 or args.message_sets < 1:
        print("--steps and --message-sets must be at least 1 and --warmup at least 0", file=sys.stderr)
        return 2
    if args.serving_policy and args.workload not in ("tiny", "decode"):
        print("--serving-policy applies to the serving workloads (tiny, decode)", file=sys.stderr)
        return 2
    if args.sweep:
        return run_sweep(args)
    if args.workload != "1gb":
        return run_workload(args)

    import numpy as np
    import torch

    from error_compensated_bit_echo_amd import binding as B
    from error_compensated_bit_echo_amd import inputs as I

    N, P, rank = 1 << args.log2n, args.nranks, 0
    C = N // P
    dev = torch.device("cuda:0")
    cu_streams = [] if args.cu_split is None else [cu_partition_streams(torch, args.cu_split)]
    print(f"bench: generating workload N={N} P={P}", file=sys.stderr, flush=True)
    x, recv, gath = make_workload(N, P, rank)

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    xd = d(x)
    # message sets cycled call by call (set 0 is the workload's own)
    # set 0 is the workload's own (the oracle leg's); the others are drawn on
    # the device with the same distributions
    dsets = []
    for k in range(args.message_sets):
        if k == 0:
            rd = [None if m is None else (d(m[0]), d(m[1])) for m in recv]
            gd = [None if m is None else (d(m[0]), d(m[1])) for m in gath]
        else:
            rd = [None if q == rank else I.device_message(C, I.stream_key("echo-1gb", "set", k, "recv", q), dev)
                  for q in range(P)]
            gd = [None if j == rank else I.device_message(C, I.stream_key("echo-1gb", "set", k, "gath", j), dev,
                                                          scale_lo=0.05 * np.sqrt(P), scale_hi=0.55 * np.sqrt(P))
                  for j in range(P)]
        dsets.append(([None if m is None else m[0] for m in rd], [None if m is None else m[1] for m in rd],
                      [None if m is None else m[0] for m in gd], [None if m is None else m[1] for m in gd]))
    mf = torch.empty(N, dtype=torch.float32, device=dev)
    ms = torch.empty(N, dtype=torch.float32, device=dev)
    send_c = torch.empty(N // 2, dtype=torch.uint8, device=dev)
    send_s = torch.empty(N // 128, dtype=torch.float32, device=dev)
    own_c = torch.empty(C // 2, dtype=torch.uint8, device=dev)
    own_s = torch.empty(C // 128, dtype=torch.float32, device=dev)
    y = torch.empty(N, dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    st = B.echo_state_init(mf, ms, N, P, rank, stream)
    rc_, rs_, gc_, gs_ = dsets[0]
    calls = [0]

    def step(ev=None):
        # ev: events before and after the entry pass, and (4 of them) after
        # the reduce and after the exit pass
        rc_k, rs_k, gc_k, gs_k = dsets[calls[0] % len(dsets)]
        calls[0] += 1
        if ev is not None:
            ev[0].record(stream)
        B.echo_call_entry(st, xd, send_c, send_s, stream)
        if ev is not None:
            ev[1].record(stream)
        B.echo_call_reduce(st, xd, rc_k, rs_k, own_c, own_s, y, stream)
        if ev is not None and len(ev) > 2:
            ev[2].record(stream)
        B.echo_call_exit(st, gc_k, gs_k, y, stream)
        if ev is not None and len(ev) > 3:
            ev[3].record(stream)

    def new_events(k, per_step):
        return [[torch.cuda.Event(enable_timing=True) for _ in range(per_step)] for _ in range(k)]

    if args.calibrate:
        calibration_copy(dev)
    print(f"bench: {args.warmup} warmup + {args.steps} timed steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed steps: events only around the entry pass, the roofline's kernel
    # (each event is one more packet on the stream)
    events = new_events(args.steps, 2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # the same number of steps again with an event between every two kernels
    events4 = new_events(args.steps, 4)
    for k in range(args.steps):
        step(events4[k])
    torch.cuda.synchronize()
    k_each = {"entry": [e[0].elapsed_time(e[1]) for e in events]}
    k_each.update({name: [e[i].elapsed_time(e[i + 1]) for e in events4]
                   for i, name in ((1, "reduce"), (2, "exit"))})
    k_ms = {name: float(np.mean(v)) for name, v in k_each.items()}
    call_event_ms = [e[0].elapsed_time(e[3]) for e in events4]

    # the fused entry point itself, same stream, for reference
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for k in range(args.steps):
        B.echo_call(st, xd, *dsets[k % len(dsets)], send_c, send_s, own_c, own_s, y, stream)
    torch.cuda.synchronize()
    call_ms = (time.perf_counter() - t2) * 1e3 / args.steps

    ceiling = practical_ceiling(B, torch, stream)

    bpe = bytes_per_element(P)
    entry_bytes = (N - C) * bpe["entry"]
    achieved = entry_bytes / (k_ms["entry"] * 1e-3) / 1e9
    total_bytes = step_bytes(N, P)
    workload = f"1GB message: bf16[2^{args.log2n}] per rank, P={P}, rank {rank}, group 128"
    out = {
        "metric": METRIC,
        "value": round(2.0 * N / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": workload, "elements": N, "nranks": P, "rank": rank, "group": 128,
                   "message_sets": args.message_sets,
                   "input": "N(0,1), 0.1% of elements x20; seeded int4 shards in HBM"},
        "pct_hbm_peak": round(100.0 * total_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "algorithmic_bytes_per_step": int(total_bytes),
        "kernel_ms": {k: round(v, 4) for k, v in k_ms.items()},
        "kernel_ms_from": "entry: HIP events in the timed steps; reduce, exit and call_ms_events: "
                          "the same number of steps right after, with an event between every two kernels",
        "kernel_ms_min_max": {k: [round(float(min(v)), 4), round(float(max(v)), 4)]
                              for k, v in k_each.items()},
        "call_ms_events": {"mean": round(float(np.mean(call_event_ms)), 4),
                           "median": round(float(np.median(call_event_ms)), 4)},
        "echo_call_ms": round(call_ms, 4),
        "roofline": {
            "kernel": "K_entry (k_stage1<entry>)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile("entry", "1gb") if args.log2n == 29 and P == 8 else None,
            "bytes_per_launch": int(entry_bytes),
        },
        "cpu_baseline": None,
    }
    out["practical_ceiling"] = dict(
        ceiling, entry_frac=round(achieved / ceiling["GBps"], 4),
        call_frac=round(total_bytes / (ms_step * 1e-3) / 1e9 / ceiling["GBps"], 4))
    if not args.no_schedules:
        print("bench: critical-path schedules", file=sys.stderr, flush=True)
        e2 = torch.empty(C, dtype=torch.float32, device=dev)
        out["schedules"] = schedules(B, torch, st, xd, rc_, rs_, gc_, gs_, send_c, send_s, own_c,
                                     own_s, y, e2, N, P, rank, args.steps, cu_streams)
    if not args.no_cpu:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        n_s = min(N, 1 << args.cpu_log2n)
        out["cpu_baseline"] = cpu_baseline(x, recv, gath, P, rank, n_s, args.cpu_calls)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
