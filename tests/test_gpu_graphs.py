"""The library's calls inside a captured HIP graph.

Every entry point only launches kernels on the caller's stream (no
allocation, no memset, no synchronization), so a sequence of calls can be
captured once and replayed -- the way a serving loop amortizes the launch
cost of a small decode-time all-reduce.  The graph is replayed several times,
the state restored eagerly between replays, and every replay is checked
against the eager run bit for bit."""
import numpy as np
import pytest
import torch

import gpu_util as g
from error_compensated_bit_echo_amd import binding as B
from error_compensated_bit_echo_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits", [4, 8])
def test_captured_call_sequence_replays_bit_exact(bits):
    P, rank, n, L = 8, 3, 8 * 128 * 8, 6
    C = n // P
    cb = n if bits == 8 else n // 2
    ccb = C if bits == 8 else C // 2
    xs = [g.dev(I.gaussian_outlier_channels(n // 1024, 1024, I.stream_key("graph", l))) for l in range(L)]
    recv = [None if q == rank else tuple(g.dev(t) for t in I.int4_message(C, I.stream_key("gr", q), bits=bits))
            for q in range(P)]
    gath = [None if j == rank else tuple(g.dev(t) for t in I.int4_message(C, I.stream_key("gg", j), bits=bits))
            for j in range(P)]
    sl = lambda arr, k: [None if m is None else m[k] for m in arr]  # noqa: E731
    mf = g.empty_f32(n, 0.0)
    ms = g.empty_f32(n, 0.0)
    st = B.EchoState(mf, ms, n, P, rank, bits=bits)
    send_c, send_s = g.empty_u8(cb), g.empty_f32(n // 128)
    own_c, own_s = g.empty_u8(ccb), g.empty_f32(C // 128)
    ys = [g.empty_bf16(n) for _ in range(L)]

    def sequence():
        for l in range(L):
            B.echo_call(st, xs[l], sl(recv, 0), sl(recv, 1), sl(gath, 0), sl(gath, 1), send_c, send_s,
                        own_c, own_s, ys[l])

    # eager reference
    sequence()
    torch.cuda.synchronize()
    want_y = [y.clone() for y in ys]
    want_mf, want_ms = mf.clone(), ms.clone()
    want_c = own_c.clone()

    # capture (warm the capture stream first), then replay from the zero state
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mf.zero_()
        ms.zero_()
        sequence()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sequence()
    for replay in range(3):
        mf.zero_()   # eager work between replays: restore the state, scribble on outputs
        ms.zero_()
        for y in ys:
            y.fill_(0x7F)
        own_c.fill_(0x55)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(L):
            g.eq(g.host(ys[l], np.uint16), g.host(want_y[l], np.uint16), f"replay {replay} call {l} y")
        g.eq(g.host(mf, np.float32), g.host(want_mf, np.float32), f"replay {replay} m_fast")
        g.eq(g.host(ms, np.float32), g.host(want_ms, np.float32), f"replay {replay} m_slow")
        g.eq(g.host(own_c, np.uint8), g.host(want_c, np.uint8), f"replay {replay} codes2")


def test_captured_mixed_schedules_with_a_side_stream():
    """One captured sequence mixing the entry points: a fused call, the
    uncompensated call, a reduce-scatter call, the split schedule whose
    update runs on a second stream forked and joined inside the capture, and
    the same schedule with the correction kept as one array.  Every replay
    equals the eager run bit for bit."""
    P, rank, n = 8, 5, 8 * 128 * 6
    C = n // P
    xs = [g.dev(I.gaussian_outlier_channels(n // 1024, 1024, I.stream_key("mixed", l))) for l in range(4)]
    recv = [None if q == rank else tuple(g.dev(t) for t in I.int4_message(C, I.stream_key("mr", q)))
            for q in range(P)]
    gath = [None if j == rank else tuple(g.dev(t) for t in I.int4_message(C, I.stream_key("mg", j)))
            for j in range(P)]
    sl = lambda arr, k: [None if m is None else m[k] for m in arr]  # noqa: E731
    mf, ms = g.empty_f32(n, 0.0), g.empty_f32(n, 0.0)
    st = B.EchoState(mf, ms, n, P, rank)
    send_c, send_s = g.empty_u8(n // 2), g.empty_f32(n // 128)
    own_c, own_s = g.empty_u8(C // 2), g.empty_f32(C // 128)
    e2 = g.empty_f32(C, 0.0)
    ys = [g.empty_bf16(n) for _ in range(4)]
    corr = g.empty_f32(n, 0.0)
    y_rs = g.empty_bf16(C)
    side = torch.cuda.Stream()
    sh_c = [send_c[rank * C // 2:(rank + 1) * C // 2] if q == rank else recv[q][0] for q in range(P)]
    sh_s = [send_s[rank * C // 128:(rank + 1) * C // 128] if q == rank else recv[q][1] for q in range(P)]

    def sequence():
        main = torch.cuda.current_stream()
        B.echo_call(st, xs[0], sl(recv, 0), sl(recv, 1), sl(gath, 0), sl(gath, 1), send_c, send_s,
                    own_c, own_s, ys[0], main)
        B.echo_call_plain(P, rank, xs[1], sl(recv, 0), sl(recv, 1), sl(gath, 0), sl(gath, 1), send_c,
                          send_s, own_c, own_s, ys[1], stream=main)
        B.echo_rs_call(st, xs[2], sl(recv, 0), sl(recv, 1), send_c, send_s, y_rs, main)
        # split schedule: critical path on main, the update on the side stream
        B.echo_encode(st, xs[3], send_c, send_s, main)
        B.echo_reduce_shard(sh_c, sh_s, own_c, own_s, ys[2][rank * C:(rank + 1) * C], e2, chunk_n=C,
                            stream=main)
        B.echo_call_exit(st, sl(gath, 0), sl(gath, 1), ys[2], main)
        side.wait_stream(main)
        B.echo_update(st, xs[3], send_c, send_s, e2, side)
        main.wait_stream(side)
        # the same with the correction array: set up, then one call
        B.echo_correction(st, corr, main)
        B.echo_encode_corr(st, xs[0], corr, send_c, send_s, main)
        B.echo_reduce_shard(sh_c, sh_s, own_c, own_s, ys[3][rank * C:(rank + 1) * C], e2, chunk_n=C,
                            stream=main)
        B.echo_call_exit(st, sl(gath, 0), sl(gath, 1), ys[3], main)
        side.wait_stream(main)
        B.echo_update_corr(st, xs[0], send_c, send_s, e2, corr, side)
        main.wait_stream(side)

    outs = lambda: [mf, ms, own_c, own_s, send_c, send_s, e2, y_rs, corr, *ys]  # noqa: E731
    sequence()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs()]

    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        sequence()
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sequence()
    for replay in range(3):
        mf.zero_()
        ms.zero_()
        for t in outs()[2:]:
            t.view(torch.uint8).fill_(0x3C)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs(), want)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {replay} output {i}"
