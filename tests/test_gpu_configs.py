"""GPU parity at the full sizes of the five workloads, through the C ABI, in
the launch configuration bench.py times.

  tiny     P=8 ranks simulated on one GPU, bf16 [16 x 4096] per rank, 4 calls
           from zero state: every output of every rank against the oracle's
           full simulation.
  decode   P=8 simulated, [256 x 4096] per rank, 64 calls with the averages
           carried: every output, every call; also under the serving policy
           (first half of the layers with 8-bit codes).
  prefill  rank mode, [8192 x 4096] (32M elements), 4 warm-up calls then the
           measured call; sampled windows of every chunk checked after every
           call (the oracle follows each window through the whole sequence),
           and every output byte of the measured call against the oracle's
           own run of the whole sequence.
  train    rank mode, [8 x 4096 x 1024], 56 forward calls on one state then 56
           backward calls on another, inputs drawn on the GPU each call;
           sampled windows after every call, every output byte of the last
           forward and the last backward call.
  1gb      rank mode, bf16[2^29], 23 calls on the same input (the bench's 3
           warm-up + 20 timed); sampled windows after every call, every
           output byte of calls 0 and 22.
The whole-tensor oracle runs are the oracle's threaded driver (the
single-thread step functions over disjoint runs of groups, pinned
bit-identical to the single-thread call on the CPU), from zero state, on the
same inputs: no oracle input comes from the GPU.
"""
import os

import numpy as np
import pytest
import torch

import gpu_util as g
from error_compensated_bit_echo_amd import binding as B
from error_compensated_bit_echo_amd import inputs as I
from oracle import oracle as orc

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


# ---- full simulation ------------------------------------------------------------------

def _simulate_sequence(P, n, calls, make_x, label, bits_of=lambda call: 4):
    mf = [np.zeros(n, np.float32) for _ in range(P)]
    ms = [np.zeros(n, np.float32) for _ in range(P)]
    ranks = [g.GpuRank(np.zeros(n, np.uint16), mf[p], ms[p], P, p) for p in range(P)]
    for call in range(calls):
        xs = [make_x(call, p) for p in range(P)]
        bits = bits_of(call)
        codes2, scales2, _, _ = g.gpu_simulate_call(ranks, xs, bits=bits)
        want = orc.simulate(xs, mf, ms, bits=bits)
        g.eq(g.host(codes2, np.uint8), want["codes2"], f"{label} call {call} codes2")
        g.eq(g.host(scales2, np.float32), want["scales2"], f"{label} call {call} scales2")
        for p, r in enumerate(ranks):
            g.eq(g.host(r.y, np.uint16), want["y"], f"{label} call {call} y rank {p}")
            g.eq(g.host(r.mf, np.float32), mf[p], f"{label} call {call} m_fast rank {p}")
            g.eq(g.host(r.ms, np.float32), ms[p], f"{label} call {call} m_slow rank {p}")
        if call % 16 == 0:
            say(f"{label}: call {call} ok")


def test_config_tiny_full_simulation():
    P, tokens, hidden = 8, 16, 4096
    ck = I.stream_key("tiny", 0, "channels")

    def make_x(call, p):
        return I.gaussian_outlier_channels(tokens, hidden, I.stream_key("tiny", 0, call, p),
                                           outlier_mult=20.0, channel_key=ck)
    _simulate_sequence(P, tokens * hidden, 4, make_x, "tiny")


@pytest.mark.timeout(600)
def test_config_decode_full_simulation():
    P, tokens, hidden = 8, 256, 4096
    ck = I.stream_key("decode", 0, "channels")

    def make_x(call, p):
        return I.lognormal_channel_activations(tokens, hidden, I.stream_key("decode", 0, call, p), ck)
    _simulate_sequence(P, tokens * hidden, 64, make_x, "decode")


@pytest.mark.timeout(600)
def test_config_decode_serving_policy():
    """The decode workload under the pages' serving policy: the first half of
    the layers (calls 0-31) with 8-bit codes, the rest with 4-bit codes, one
    state carried through all 64 calls; every output of every rank, every
    call, against the oracle's full simulation."""
    P, tokens, hidden = 8, 256, 4096
    ck = I.stream_key("decode", 1, "channels")

    def make_x(call, p):
        return I.lognormal_channel_activations(tokens, hidden, I.stream_key("decode", 1, call, p), ck)
    _simulate_sequence(P, tokens * hidden, 64, make_x, "decode 8/4-bit",
                       bits_of=lambda call: 8 if call < 32 else 4)


# ---- rank mode --------------------------------------------------------------------------

# host threads for the whole-tensor oracle runs (the CPU share of one GPU)
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


class FullOracle:
    """The oracle's run of a rank-mode call sequence on the whole tensor, from
    zero state, with the sequence's own seeded messages and inputs."""

    def __init__(self, run):
        self.run = run
        self.mf = np.zeros(run.n, np.float32)
        self.ms = np.zeros(run.n, np.float32)
        sl = lambda arr, k: [None if m is None else m[k] for m in arr]  # noqa: E731
        self.msgs = (sl(run.recv, 0), sl(run.recv, 1), sl(run.gath, 0), sl(run.gath, 1))
        self.out = None

    def call(self, x_host):
        r = self.run
        self.out = orc.call(r.P, r.rank, x_host, self.mf, self.ms, *self.msgs, comp=r.comp,
                            bits=r.bits, threads=ORACLE_THREADS, out=self.out)

    def compare(self, tag):
        """every byte of the GPU's outputs and averages against this run's"""
        torch.cuda.synchronize()
        r, want = self.run, self.out
        C, p, f = r.C, r.rank, r.f
        what = f"{r.label} {tag} (whole tensor)"
        g.eq(g.host(r.y, np.uint16), want["y"], what + " y")
        g.eq(g.host(r.own_c, np.uint8), want["own_codes2"], what + " own codes2")
        g.eq(g.host(r.own_s, np.float32), want["own_scales2"], what + " own scales2")
        sc, ss = g.host(r.send_c, np.uint8), g.host(r.send_s, np.float32)
        for j in range(r.P):
            if j == p:
                continue  # the own chunk of the send message is not written
            cs, gs = slice(j * C // f, (j + 1) * C // f), slice(j * C // 128, (j + 1) * C // 128)
            g.eq(sc[cs], want["send_codes"][cs], what + f" send codes chunk {j}")
            g.eq(ss[gs], want["send_scales"][gs], what + f" send scales chunk {j}")
        del sc, ss
        if r.comp:
            g.eq(g.host(r.mf, np.float32), self.mf, what + " m_fast")
            g.eq(g.host(r.ms, np.float32), self.ms, what + " m_slow")
        say(f"{what}: every byte equal")


class RankRun:
    """Device buffers of one rank-mode sequence plus the oracle's windows."""

    def __init__(self, P, rank, n, seed, windows_per_chunk=2, W=4, label="", bits=4, comp=True,
                 full=False):
        self.P, self.rank, self.n, self.C = P, rank, n, n // P
        self.label = label
        self.bits = bits
        self.comp = comp
        self.f = 1 if bits == 8 else 2  # elements per code byte
        C = self.C
        self.recv = [None if q == rank else I.int4_message(C, I.stream_key(label, seed, "recv", q),
                                                           zero_group_frac=1e-3, bits=bits)
                     for q in range(P)]
        self.gath = [None if j == rank else
                     I.int4_message(C, I.stream_key(label, seed, "gath", j), scale_lo=0.15,
                                    scale_hi=1.5, zero_group_frac=1e-3, bits=bits)
                     for j in range(P)]
        self.recv_d = [None if m is None else (g.dev(m[0]), g.dev(m[1])) for m in self.recv]
        self.gath_d = [None if m is None else (g.dev(m[0]), g.dev(m[1])) for m in self.gath]
        self.mf = g.empty_f32(n)
        self.ms = g.empty_f32(n)
        self.st = B.echo_state_init(self.mf, self.ms, n, P, rank)
        self.st.bits = bits
        self.send_c = g.empty_u8(n // self.f)
        self.send_s = g.empty_f32(n // 128)
        self.own_c = g.empty_u8(C // self.f)
        self.own_s = g.empty_f32(C // 128)
        self.y = g.empty_bf16(n)
        rng = np.random.default_rng(seed)
        self.wins = [g.WindowOracle(P, rank, j, off, W, bits=bits, comp=comp)
                     for j, off in g.pick_windows(P, C, W, rng, windows_per_chunk)]
        self.full = FullOracle(self) if full else None

    def oracle_call(self, x_host):
        """advance the whole-tensor oracle by one call on the same input"""
        self.full.call(x_host)

    def call(self, xd):
        sl = lambda arr, k: [None if m is None else m[k] for m in arr]  # noqa: E731
        B.echo_call(self.st, xd, sl(self.recv_d, 0), sl(self.recv_d, 1), sl(self.gath_d, 0),
                    sl(self.gath_d, 1), self.send_c, self.send_s, self.own_c, self.own_s, self.y)

    def call_plain(self, xd):
        sl = lambda arr, k: [None if m is None else m[k] for m in arr]  # noqa: E731
        B.echo_call_plain(self.P, self.rank, xd, sl(self.recv_d, 0), sl(self.recv_d, 1),
                          sl(self.gath_d, 0), sl(self.gath_d, 1), self.send_c, self.send_s,
                          self.own_c, self.own_s, self.y, bits=self.bits)

    def call_split(self, xd, e2, side):
        """The pages' schedule: the critical path (entry pass with the
        averages read-only, reduce of the own chunk with e2 kept, exit) on
        the current stream, then the update on a side stream."""
        P, r, C, f = self.P, self.rank, self.C, self.f
        main = torch.cuda.current_stream()
        sl = lambda arr, k: [None if m is None else m[k] for m in arr]  # noqa: E731
        sh_c = [self.send_c[r * C // f:(r + 1) * C // f] if q == r else self.recv_d[q][0] for q in range(P)]
        sh_s = [self.send_s[r * C // 128:(r + 1) * C // 128] if q == r else self.recv_d[q][1] for q in range(P)]
        B.echo_encode(self.st, xd, self.send_c, self.send_s, main)
        B.echo_reduce_shard(sh_c, sh_s, self.own_c, self.own_s, self.y[r * C:(r + 1) * C], e2, chunk_n=C,
                            stream=main, bits=self.bits)
        B.echo_call_exit(self.st, sl(self.gath_d, 0), sl(self.gath_d, 1), self.y, main)
        side.wait_stream(main)
        B.echo_update(self.st, xd, self.send_c, self.send_s, e2, side)
        main.wait_stream(side)

    def call_split_corr(self, xd, e2, corr, side):
        """The same schedule with the correction kept as one array: the entry
        pass reads corr, the side-stream update refreshes the averages and
        writes the next call's corr."""
        P, r, C, f = self.P, self.rank, self.C, self.f
        main = torch.cuda.current_stream()
        sl = lambda arr, k: [None if m is None else m[k] for m in arr]  # noqa: E731
        sh_c = [self.send_c[r * C // f:(r + 1) * C // f] if q == r else self.recv_d[q][0] for q in range(P)]
        sh_s = [self.send_s[r * C // 128:(r + 1) * C // 128] if q == r else self.recv_d[q][1] for q in range(P)]
        B.echo_encode_corr(self.st, xd, corr, self.send_c, self.send_s, main)
        B.echo_reduce_shard(sh_c, sh_s, self.own_c, self.own_s, self.y[r * C:(r + 1) * C], e2, chunk_n=C,
                            stream=main, bits=self.bits)
        B.echo_call_exit(self.st, sl(self.gath_d, 0), sl(self.gath_d, 1), self.y, main)
        side.wait_stream(main)
        B.echo_update_corr(self.st, xd, self.send_c, self.send_s, e2, corr, side)
        main.wait_stream(side)

    def check_windows(self, xd, tag):
        """Run every window's oracle one call further and compare."""
        torch.cuda.synchronize()
        C, r = self.C, self.rank
        for w in self.wins:
            es = w.elems(C)
            ce = w.chunk_elems()
            x_win = g.host(xd[es], np.uint16)
            if w.j == r:
                msg = [None if q == r else (self.recv[q][0][w.code_slice(ce)],
                                            self.recv[q][1][ce.start // 128:ce.stop // 128])
                       for q in range(self.P)]
            else:
                m = self.gath[w.j]
                msg = (m[0][w.code_slice(ce)], m[1][ce.start // 128:ce.stop // 128])
            want = w.call(x_win, msg)
            what = f"{self.label} {tag} window (chunk {w.j}, group {w.off})"
            g.eq(g.host(self.y[es], np.uint16), want["y"], what + " y")
            g.eq(g.host(self.mf[es], np.float32), want["m_fast"], what + " m_fast")
            g.eq(g.host(self.ms[es], np.float32), want["m_slow"], what + " m_slow")
            if w.j == r:
                g.eq(g.host(self.own_c[w.code_slice(ce)], np.uint8), want["codes"], what + " codes2")
                g.eq(g.host(self.own_s[ce.start // 128:ce.stop // 128], np.float32), want["scales"],
                     what + " scales2")
            else:
                g.eq(g.host(self.send_c[w.code_slice(es)], np.uint8), want["codes"], what + " send codes")
                g.eq(g.host(self.send_s[es.start // 128:es.stop // 128], np.float32), want["scales"],
                     what + " send scales")

    def check_message_properties(self, tag):
        """Send and own stage-2 messages never hold the code -8 and their scales
        are finite and non-negative."""
        torch.cuda.synchronize()
        C, r = self.C, self.rank
        sc = g.host(self.send_c, np.uint8)
        ss = g.host(self.send_s, np.float32)
        f = self.f
        keep = np.ones(self.n // f, bool)
        keep[r * C // f:(r + 1) * C // f] = False
        keep_s = np.ones(self.n // 128, bool)
        keep_s[r * C // 128:(r + 1) * C // 128] = False
        for codes, scales in ((sc[keep], ss[keep_s]),
                              (g.host(self.own_c, np.uint8), g.host(self.own_s, np.float32))):
            if self.bits == 8:
                assert not np.any(codes == 0x80), tag
            else:
                assert not np.any((codes & 0xF) == 8) and not np.any((codes >> 4) == 8), tag
            assert np.all(np.isfinite(scales)) and np.all(scales >= 0), tag


@pytest.mark.timeout(600)
def test_config_prefill_rank_mode():
    P, rank, tokens, hidden = 8, 0, 8192, 4096
    n = tokens * hidden
    run = RankRun(P, rank, n, seed=3, label="prefill", full=True)
    ck = I.stream_key("prefill", "channels")
    for call in range(5):  # 4 warm-up calls, then the measured call on warm state
        x = I.lognormal_channel_activations(tokens, hidden, I.stream_key("prefill", call), ck)
        xd = g.dev(x)
        run.call(xd)
        run.oracle_call(x)
        run.check_windows(xd, f"call {call}")
        say(f"prefill: call {call} windows ok")
    run.full.compare("measured call 4")
    run.check_message_properties("final call")


@pytest.mark.timeout(900)
def test_config_train_rank_mode():
    """56 forward calls (activations) on one state, then 56 backward calls
    (1e-3 Student-t(3) gradients) in reverse site order on another."""
    P, rank = 8, 5
    b, s, hidden = 8, 4096, 1024
    n = b * s * hidden
    dev = torch.device(g.DEV)
    lam = I.channel_scales(hidden, I.stream_key("train", "channels"))
    fwd = RankRun(P, rank, n, seed=41, windows_per_chunk=1, label="train-fwd", full=True)
    bwd = RankRun(P, rank, n, seed=43, windows_per_chunk=1, label="train-bwd", full=True)
    for site in range(56):
        xd = I.device_lognormal_channel_activations(b * s, hidden, 1000 + site, lam, dev)
        fwd.call(xd)
        fwd.oracle_call(g.host(xd, np.uint16))
        fwd.check_windows(xd, f"forward site {site}")
        if site % 14 == 0:
            say(f"train: forward site {site} ok")
    fwd.full.compare("last forward call")
    for site in reversed(range(56)):
        xd = I.device_student_t3(n, 2000 + site, dev)
        bwd.call(xd)
        bwd.oracle_call(g.host(xd, np.uint16))
        bwd.check_windows(xd, f"backward site {site}")
        if site % 14 == 0:
            say(f"train: backward site {site} ok")
    bwd.full.compare("last backward call")
    fwd.check_message_properties("last forward call")
    bwd.check_message_properties("last backward call")


@pytest.mark.timeout(900)
def test_config_1gb_rank_mode():
    """The bench's workload and call sequence: bf16[2^29], P = 8, rank 0,
    3 warm-up + 20 timed calls on the same input, the averages carried."""
    P, rank, n = 8, 0, 1 << 29
    C = n // P
    say("1gb: generating inputs")
    x = I.vector_with_outliers(n, I.stream_key("echo-1gb", 0, "x"), outlier_mult=20.0)
    xd = g.dev(x)
    run = RankRun(P, rank, n, seed=0, windows_per_chunk=3, label="1gb", full=True)
    for call in range(23):
        run.call(xd)
        run.oracle_call(x)
        if call in (0, 22):
            run.full.compare(f"call {call}")
        run.check_windows(xd, f"call {call}")
        if call % 5 == 0:
            say(f"1gb: call {call} windows ok")
    run.check_message_properties("call 22")


@pytest.mark.timeout(900)
def test_1gb_message_sixteen_ranks():
    """The 1 GB message at the largest rank count (P = 16, rank 11): 15
    incoming shards per chunk element, four calls with the averages carried,
    windows of every chunk after each call, every output byte of the last."""
    P, rank, n = 16, 11, 1 << 29
    say("1gb P=16: generating inputs")
    x = I.vector_with_outliers(n, I.stream_key("echo-1gb", 16, "x"), outlier_mult=20.0)
    xd = g.dev(x)
    run = RankRun(P, rank, n, seed=16, windows_per_chunk=2, label="1gb P=16", full=True)
    for call in range(4):
        run.call(xd)
        run.oracle_call(x)
        run.check_windows(xd, f"call {call}")
        say(f"1gb P=16: call {call} windows ok")
    run.full.compare("call 3")
    run.check_message_properties("call 3")


@pytest.mark.timeout(900)
def test_1gb_message_8bit_promoted_call():
    """The 1 GB message with 8-bit codes (the promoted width), as the bench
    times it: P = 8, rank 0, four calls with the averages carried, windows
    of every chunk after each call, every output byte of the last, no -128
    code in any message."""
    P, rank, n = 8, 0, 1 << 29
    say("1gb 8-bit: generating inputs")
    x = I.vector_with_outliers(n, I.stream_key("echo-1gb", 8, "x"), outlier_mult=20.0)
    xd = g.dev(x)
    run = RankRun(P, rank, n, seed=8, windows_per_chunk=2, label="1gb 8-bit", bits=8, full=True)
    for call in range(4):
        run.call(xd)
        run.oracle_call(x)
        run.check_windows(xd, f"call {call}")
        say(f"1gb 8-bit: call {call} windows ok")
    run.full.compare("call 3")
    run.check_message_properties("call 3")


@pytest.mark.timeout(900)
def test_1gb_message_reduce_scatter():
    """The reduce-scatter call at the bench's size (bf16[2^29], P = 8, rank
    0): four calls with the averages carried, windows of every chunk (send
    codes or y_own, and the averages) after each call and every output byte
    of the last against the oracle."""
    P, rank, n = 8, 0, 1 << 29
    C = n // P
    say("1gb reduce-scatter: generating inputs")
    x = I.vector_with_outliers(n, I.stream_key("echo-1gb", 0, "x"), outlier_mult=20.0)
    xd = g.dev(x)
    recv = [None if q == rank else I.int4_message(C, I.stream_key("1gb rs", q), zero_group_frac=1e-3)
            for q in range(P)]
    rc = [None if m is None else g.dev(m[0]) for m in recv]
    rs = [None if m is None else g.dev(m[1]) for m in recv]
    mf, ms = g.empty_f32(n), g.empty_f32(n)
    st = B.echo_state_init(mf, ms, n, P, rank)
    send_c, send_s, y_own = g.empty_u8(n // 2), g.empty_f32(n // 128), g.empty_bf16(C)
    rng = np.random.default_rng(12)
    wins = [g.RSWindowOracle(P, rank, j, off, 4) for j, off in g.pick_windows(P, C, 4, rng, 2)]
    hmf, hms = np.zeros(n, np.float32), np.zeros(n, np.float32)  # the oracle's whole-tensor run
    for call in range(4):
        B.echo_rs_call(st, xd, rc, rs, send_c, send_s, y_own)
        want_all = orc.rs_call(P, rank, x, hmf, hms, [None if m is None else m[0] for m in recv],
                               [None if m is None else m[1] for m in recv], threads=ORACLE_THREADS)
        torch.cuda.synchronize()
        for w in wins:
            es, ce = w.elems(C), w.chunk_elems()
            msg = ([None if q == rank else (recv[q][0][w.code_slice(ce)], recv[q][1][ce.start // 128:ce.stop // 128])
                    for q in range(P)] if w.j == rank else None)
            want = w.call(g.host(xd[es], np.uint16), msg)
            what = f"1gb rs call {call} window (chunk {w.j}, group {w.off})"
            g.eq(g.host(mf[es], np.float32), want["m_fast"], what + " m_fast")
            g.eq(g.host(ms[es], np.float32), want["m_slow"], what + " m_slow")
            if w.j == rank:
                g.eq(g.host(y_own[ce], np.uint16), want["y_own"], what + " y_own")
            else:
                g.eq(g.host(send_c[w.code_slice(es)], np.uint8), want["codes"], what + " send codes")
                g.eq(g.host(send_s[es.start // 128:es.stop // 128], np.float32), want["scales"],
                     what + " send scales")
        say(f"1gb reduce-scatter: call {call} windows ok")
    what = "1gb rs call 3 (whole tensor)"
    g.eq(g.host(y_own, np.uint16), want_all["y_own"], what + " y_own")
    keep = np.ones(n // 2, bool)
    keep[rank * C // 2:(rank + 1) * C // 2] = False
    g.eq(g.host(send_c, np.uint8)[keep], want_all["send_codes"][keep], what + " send codes")
    keep_s = np.ones(n // 128, bool)
    keep_s[rank * C // 128:(rank + 1) * C // 128] = False
    g.eq(g.host(send_s, np.float32)[keep_s], want_all["send_scales"][keep_s], what + " send scales")
    g.eq(g.host(mf, np.float32), hmf, what + " m_fast")
    g.eq(g.host(ms, np.float32), hms, what + " m_slow")
    say(f"{what}: every byte equal")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("schedule", ["uncompensated", "split", "split_corr"])
def test_1gb_message_other_schedules(schedule):
    """The bench's other 1 GB schedules: the uncompensated call, the split
    schedule (averages read-only on the critical path, the update on a side
    stream), and the split schedule with the correction kept as one array;
    four calls, windows of every chunk after each call and every output byte
    of the last against the oracle."""
    P, rank, n = 8, 0, 1 << 29
    say(f"1gb {schedule}: generating inputs")
    x = I.vector_with_outliers(n, I.stream_key("echo-1gb", 0, "x"), outlier_mult=20.0)
    xd = g.dev(x)
    run = RankRun(P, rank, n, seed=21, windows_per_chunk=2, label=f"1gb {schedule}",
                  comp=schedule != "uncompensated", full=True)
    e2 = g.empty_f32(n // P)
    side = torch.cuda.Stream()
    corr = None
    if schedule == "split_corr":
        corr = g.empty_f32(n)
        B.echo_correction(run.st, corr)
    for call in range(4):
        if schedule == "uncompensated":
            run.call_plain(xd)
        elif schedule == "split":
            run.call_split(xd, e2, side)
        else:
            run.call_split_corr(xd, e2, corr, side)
        run.oracle_call(x)
        run.check_windows(xd, f"call {call}")
        say(f"1gb {schedule}: call {call} windows ok")
    run.full.compare("call 3")
    if corr is not None:
        g.eq(g.host(corr, np.float32), orc.correction(run.full.mf, run.full.ms),
             "1gb split_corr call 3 correction array")


@pytest.mark.parametrize("a", [1.0, 1.1])
def test_deep_chain_on_the_gpu(a):
    """The deep chain h <- a h + y run through the GPU (P = 8 ranks simulated),
    every call bit-identical to the oracle: bounded at sqrt(2.289) times one
    call's injected error for the identity map, geometric growth for a = 1.1."""
    P, n, L = 8, 8 * 128 * 4, 48
    rng = np.random.default_rng(17)
    mf = [np.zeros(n, np.float32) for _ in range(P)]
    ms = [np.zeros(n, np.float32) for _ in range(P)]
    ranks = [g.GpuRank(np.zeros(n, np.uint16), mf[p], ms[p], P, p) for p in range(P)]
    h = np.zeros(n)
    H = np.zeros(n)
    dev, inj = [], []
    for call in range(L):
        xs = [I.to_bf16_bits(rng.standard_normal(n)) for _ in range(P)]
        g.gpu_simulate_call(ranks, xs)
        want = orc.simulate(xs, mf, ms, want_detail=True)
        y_gpu = g.host(ranks[0].y, np.uint16)
        g.eq(y_gpu, want["y"], f"chain call {call} y")
        g.eq(g.host(ranks[3].mf, np.float32), mf[3], f"chain call {call} m_fast")
        y = (y_gpu.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        xsum = np.sum([(x.astype(np.uint32) << 16).view(np.float32).astype(np.float64) for x in xs], axis=0)
        inj.append(np.sqrt(np.mean((y - np.sum(want["xp"], axis=0, dtype=np.float64)) ** 2)))
        h = a * h + y
        H = a * H + xsum
        dev.append(np.sqrt(np.mean((h - H) ** 2)))
    dev = np.array(dev) / np.mean(inj)
    if a == 1.0:
        assert abs(dev[-8:].mean() - np.sqrt(2.2889)) < 0.2, dev[-8:]
    else:
        rate = np.polyfit(np.arange(24, L), np.log(dev[24:]), 1)[0]
        assert abs(rate - np.log(a)) < 0.03, rate
