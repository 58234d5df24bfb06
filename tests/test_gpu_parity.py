"""GPU parity: every libecho entry point against the CPU oracle, element by
element, on seeded inputs that span many workgroups and end in ragged tails
(odd group counts, chunks that are not a multiple of a wave's two groups).

The bar: int4 codes, scales, bf16 outputs, e2 and the averages bit-exact
(the method's binary32 steps are reproduced operation for operation; the
stated tolerances -- 1 bf16 ulp for y, 1e-6 relative for the averages --
are not needed and a bitwise comparison is made instead)."""
import zlib

import numpy as np
import pytest
import torch

from error_compensated_bit_echo_amd import inputs as I
from oracle import oracle as orc

import gpu_util
from error_compensated_bit_echo_amd import binding as B

pytestmark = pytest.mark.gpu


def gu():
    return gpu_util


def eq(a, b, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    bad = np.nonzero(a != b)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: {a[bad[:5]]} vs {b[bad[:5]]}"


def x_of(n, seed, scale=1.0, hidden=4096):
    if n % hidden:
        hidden = 128
    v = I.normal(n, I.stream_key("px", seed)).reshape(-1, hidden) * scale
    v[:, I.outlier_channels(hidden, 0.01, I.stream_key("pc", seed))] *= 20
    return I.to_bf16_bits(v.ravel())


def state_of(n, seed, scale=0.05):
    mf = (I.normal(n, I.stream_key("mf", seed)) * scale).astype(np.float32)
    ms = (I.normal(n, I.stream_key("ms", seed)) * scale).astype(np.float32)
    return mf, ms


SHAPES = [(1, 1), (1, 7), (2, 3), (3, 5), (4, 1), (8, 33), (8, 257), (16, 3), (5, 2049)]


def cb(n, bits):
    return n if bits == 8 else n // 2


@pytest.mark.parametrize("P,k", SHAPES)
@pytest.mark.parametrize("warm", [False, True])
@pytest.mark.parametrize("bits", [4, 8])
def test_encode(P, k, warm, bits):
    g = gu()
    n = P * 128 * k
    x = x_of(n, 1000 * P + k)
    mf, ms = state_of(n, k) if warm else (np.zeros(n, np.float32), np.zeros(n, np.float32))
    mfd, msd = g.dev(mf), g.dev(ms)
    st = B.EchoState(mfd, msd, n, P, P - 1, bits=bits)
    codes, scales = g.empty_u8(cb(n, bits), 0xAB), g.empty_f32(n // 128, -1.0)
    B.echo_encode(st, g.dev(x), codes, scales)
    want_c, want_s = orc.encode(x, mf, ms, bits=bits)
    eq(g.host(codes, np.uint8), want_c, "codes")
    eq(g.host(scales, np.float32), want_s, "scales")
    eq(g.host(mfd, np.float32), mf, "m_fast untouched")
    eq(g.host(msd, np.float32), ms, "m_slow untouched")


@pytest.mark.parametrize("P", [1, 2, 3, 7, 8, 16])
@pytest.mark.parametrize("k", [1, 6, 129])
@pytest.mark.parametrize("any_byte", [False, True])
@pytest.mark.parametrize("bits", [4, 8])
def test_reduce_shard(P, k, any_byte, bits):
    g = gu()
    cn = 128 * k
    msgs = [I.int4_message(cn, I.stream_key("rs", P, k, q), zero_group_frac=0.05, any_byte=any_byte,
                           bits=bits) for q in range(P)]
    out_c, out_s = g.empty_u8(cb(cn, bits)), g.empty_f32(cn // 128)
    out_y, out_e2 = g.empty_bf16(cn), g.empty_f32(cn)
    B.echo_reduce_shard([g.dev(c) for c, _ in msgs], [g.dev(s) for _, s in msgs], out_c, out_s,
                        out_y, out_e2, chunk_n=cn, bits=bits)
    wc, ws, wy, we = orc.reduce_chunk([c for c, _ in msgs], [s for _, s in msgs], cn, bits=bits)
    eq(g.host(out_c, np.uint8), wc, "codes2")
    eq(g.host(out_s, np.float32), ws, "scales2")
    eq(g.host(out_y, np.uint16), wy, "y")
    eq(g.host(out_e2, np.float32), we, "e2")
    # optional outputs may be skipped
    c2, s2 = g.empty_u8(cb(cn, bits)), g.empty_f32(cn // 128)
    B.echo_reduce_shard([g.dev(c) for c, _ in msgs], [g.dev(s) for _, s in msgs], c2, s2, chunk_n=cn,
                        bits=bits)
    eq(g.host(c2, np.uint8), wc, "codes2 without y/e2")


@pytest.mark.parametrize("dq, s_want", [((2.0 ** 24, 1.0, 1.0), 2.0 ** 24),
                                         ((1.0, 1.0, 2.0 ** 24), 2.0 ** 24 + 2.0)])
def test_reduce_sums_in_rank_order_from_rank_0(dq, s_want):
    """The GPU's chunk sums are the binary32 left fold from rank 0: with
    dequantized values (2^24, 1, 1) the ones are absorbed, with (1, 1, 2^24)
    they are kept.  S is read back exactly as f32(y) - e (y is within a
    factor of two of S), for both the requantizing and the bf16 sum."""
    g = gu()
    P, n = 3, 128
    codes = [np.zeros(n, np.uint8) for _ in range(P)]
    for c in codes:
        c[0] = 1
    scales = [np.array([v], np.float32) for v in dq]
    oc, os_, y, e = g.empty_u8(n), g.empty_f32(1), g.empty_bf16(n), g.empty_f32(n)
    B.echo_reduce_shard([g.dev(c) for c in codes], [g.dev(s) for s in scales], oc, os_, y, e,
                        chunk_n=n, bits=8)
    yh, eh = g.host(y, np.uint16), g.host(e, np.float32)
    assert float(orc.bf16_to_f32(yh[:1])[0]) - float(eh[0]) == s_want
    wc, ws, wy, we = orc.reduce_chunk(codes, scales, n, bits=8)
    eq(yh, wy, "y")
    eq(eh, we, "e2")
    y2, e2 = g.empty_bf16(n), g.empty_f32(n)
    B.echo_reduce_shard_sum([g.dev(c) for c in codes], [g.dev(s) for s in scales], y2, e2, chunk_n=n,
                            bits=8)
    assert float(orc.bf16_to_f32(g.host(y2, np.uint16)[:1])[0]) - float(g.host(e2, np.float32)[0]) == s_want


@pytest.mark.parametrize("k", [1, 3, 4, 5, 1023, 4099])
@pytest.mark.parametrize("bits", [4, 8])
def test_decode(k, bits):
    g = gu()
    n = 128 * k
    c, s = I.int4_message(n, I.stream_key("dec", k), zero_group_frac=0.1, any_byte=True, bits=bits)
    y = g.empty_bf16(n)
    B.echo_decode(g.dev(c), g.dev(s), y, bits=bits)
    eq(g.host(y, np.uint16), orc.decode(c, s, n, bits=bits), "y")


@pytest.mark.parametrize("bits", [4, 8])
def test_decode_bf16_narrowing_every_upper_half(bits):
    """The exit pass's binary32 -> bf16 narrowing on every finite upper half
    (sign, exponent, 7 kept mantissa bits), each with exact, tie, near-tie and
    other lower halves: with every code 1 each group's products are its scale
    itself, so y = bf16(scale) (ties to even, overflow to inf, denormals)."""
    g = gu()
    hi = np.arange(1 << 16, dtype=np.uint32)
    hi = hi[(hi & 0x7F80) != 0x7F80]
    lows = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xC000], np.uint32)
    s = ((hi[:, None] << 16) | lows[None, :]).ravel().view(np.float32)
    n = 128 * s.size
    c = np.full(n if bits == 8 else n // 2, 0x01 if bits == 8 else 0x11, np.uint8)
    y = g.empty_bf16(n)
    B.echo_decode(g.dev(c), g.dev(s), y, bits=bits)
    want = orc.decode(c, s, n, bits=bits)
    got = g.host(y, np.uint16)
    eq(got, want, "y")
    eq(got[::128], orc.f32_to_bf16(s), "y of each group vs bf16(scale)")


def _loaded_hip_runtime():
    """The HIP runtime this process already loaded (torch's, which libecho
    shares), opened by its path so both handles are the same library."""
    import ctypes
    import re

    with open("/proc/self/maps") as f:
        paths = sorted(set(re.findall(r"(/\S*libamdhip64\.so\S*)", f.read())))
    assert paths, "no HIP runtime mapped"
    hip = ctypes.CDLL(paths[0])
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    hip.hipSetDevice.restype = ctypes.c_int
    return hip


def test_stale_hip_error_is_not_reported_as_the_calls():
    """An error an earlier, unrelated HIP call left behind (here: selecting a
    device that does not exist, which the runtime rejects on the host) does
    not make a valid call return ECHO_ERR_HIP: each call reports its own
    launches' status."""
    g = gu()
    n = 128 * 37
    c, s = I.int4_message(n, I.stream_key("stale", 0), bits=4)
    cd, sd = g.dev(c), g.dev(s)
    y = g.empty_bf16(n)
    torch.cuda.synchronize()
    hip = _loaded_hip_runtime()
    assert hip.hipSetDevice(9999) != 0
    try:
        B.echo_decode(cd, sd, y, bits=4)  # raises EchoError on a non-zero status
    finally:
        hip.hipGetLastError()  # clear the planted error before torch launches anything
    torch.cuda.synchronize()
    eq(g.host(y, np.uint16), orc.decode(c, s, n, bits=4), "y after a stale error")


@pytest.mark.parametrize("P,k", SHAPES)
@pytest.mark.parametrize("bits", [4, 8])
def test_update(P, k, bits):
    g = gu()
    n = P * 128 * k
    rank = (k * 7) % P
    x = x_of(n, 7 * k + P)
    mf, ms = state_of(n, 3 * k, scale=0.2)
    codes1, scales1 = orc.encode(x, mf, ms, bits=bits)
    e2 = (I.normal(n // P, I.stream_key("e2", k)) * 0.01).astype(np.float32)
    mfd, msd = g.dev(mf), g.dev(ms)
    st = B.EchoState(mfd, msd, n, P, rank, bits=bits)
    B.echo_update(st, g.dev(x), g.dev(codes1), g.dev(scales1), g.dev(e2))
    orc.update(x, mf, ms, codes1, scales1, e2, P, rank, bits=bits)
    eq(g.host(mfd, np.float32), mf, "m_fast")
    eq(g.host(msd, np.float32), ms, "m_slow")


def _rank_inputs(P, n, seed, zero_frac=0.02, bits=4):
    Cn = n // P
    recv = [I.int4_message(Cn, I.stream_key("recv", seed, q), zero_group_frac=zero_frac, bits=bits)
            for q in range(P)]
    gath = [I.int4_message(Cn, I.stream_key("gath", seed, j), scale_lo=0.2, scale_hi=1.5,
                           zero_group_frac=zero_frac, bits=bits) for j in range(P)]
    return recv, gath


class RankCase:
    """Device and host copies of one rank-mode problem."""

    def __init__(self, P, rank, k, seed, bits=4):
        g = gu()
        self.P, self.rank, self.bits = P, rank, bits
        self.n = n = P * 128 * k
        self.Cn = n // P
        self.recv, self.gath = _rank_inputs(P, n, seed, bits=bits)
        self.mf = np.zeros(n, np.float32)
        self.ms = np.zeros(n, np.float32)
        self.mfd, self.msd = g.dev(self.mf), g.dev(self.ms)
        self.st = B.EchoState(self.mfd, self.msd, n, P, rank, bits=bits)
        self.recv_d = [(g.dev(c), g.dev(s)) for c, s in self.recv]
        self.gath_d = [(g.dev(c), g.dev(s)) for c, s in self.gath]
        self.send_c = g.empty_u8(cb(n, bits), 0xAB)
        self.send_s = g.empty_f32(n // 128, -3.0)
        self.own_c = g.empty_u8(cb(self.Cn, bits))
        self.own_s = g.empty_f32(self.Cn // 128)
        self.y = g.empty_bf16(n)

    def slot(self, arrs, which):
        return [None if q == self.rank else a[which] for q, a in enumerate(arrs)]

    def gpu_call(self, xd, y=None):
        B.echo_call(self.st, xd, self.slot(self.recv_d, 0), self.slot(self.recv_d, 1),
                    self.slot(self.gath_d, 0), self.slot(self.gath_d, 1), self.send_c, self.send_s,
                    self.own_c, self.own_s, self.y if y is None else y)

    def oracle_call(self, x):
        return orc.call(self.P, self.rank, x, self.mf, self.ms, self.slot(self.recv, 0),
                        self.slot(self.recv, 1), self.slot(self.gath, 0), self.slot(self.gath, 1),
                        bits=self.bits)

    def check(self, want, y=None):
        g = gu()
        P, r, Cn = self.P, self.rank, self.Cn
        sc = g.host(self.send_c, np.uint8)
        ss = g.host(self.send_s, np.float32)
        cbc = cb(Cn, self.bits)
        for j in range(P):
            cs = slice(j * cbc, (j + 1) * cbc)
            gs = slice(j * Cn // 128, (j + 1) * Cn // 128)
            if j == r:  # the own chunk of the send buffers is never written
                assert np.all(sc[cs] == 0xAB) and np.all(ss[gs] == -3.0)
            else:
                eq(sc[cs], want["send_codes"][cs], f"send codes chunk {j}")
                eq(ss[gs], want["send_scales"][gs], f"send scales chunk {j}")
        eq(g.host(self.own_c, np.uint8), want["own_codes2"], "own codes2")
        eq(g.host(self.own_s, np.float32), want["own_scales2"], "own scales2")
        eq(g.host(self.y if y is None else y, np.uint16), want["y"], "y")
        eq(g.host(self.mfd, np.float32), self.mf, "m_fast")
        eq(g.host(self.msd, np.float32), self.ms, "m_slow")


CALL_SHAPES = [(1, 0, 3), (2, 1, 1), (3, 0, 5), (3, 2, 2), (4, 1, 9), (8, 0, 16), (8, 5, 33),
               (8, 7, 3), (16, 15, 2), (16, 6, 5)]


@pytest.mark.parametrize("P,rank,k", CALL_SHAPES)
@pytest.mark.parametrize("bits", [4, 8])
def test_call_rank_mode(P, rank, k, bits):
    """Fused echo_call over 3 consecutive calls (fresh input each call, the
    averages carried) against the oracle's rank mode."""
    g = gu()
    case = RankCase(P, rank, k, seed=P * 100 + rank * 10 + k, bits=bits)
    for call in range(3):
        x = x_of(case.n, 31 * call + k + P)
        case.gpu_call(g.dev(x))
        want = case.oracle_call(x)
        case.check(want)


@pytest.mark.parametrize("bits", [4, 8])
def test_call_every_rank_count_and_slot(bits):
    """Every P from 1 to 16 and every rank p < P (the own slot at every
    position of the rank-order sum), an odd number of groups per chunk (a
    half-empty last wave), two calls each: fused call and reduce-scatter call
    against the oracle."""
    g = gu()
    for P in range(1, 17):
        for rank in range(P):
            k = 3
            print(f"every-slot: P={P} rank={rank} bits={bits}", flush=True)
            case = RankCase(P, rank, k, seed=1000 + 17 * P + rank, bits=bits)
            for call in range(2):
                x = x_of(case.n, 7 * call + 3 * P + rank)
                case.gpu_call(g.dev(x))
                case.check(case.oracle_call(x))
            # uncompensated call: the own slot quantized from x alone
            xp = x_of(case.n, 55 + P + rank)
            B.echo_call_plain(P, rank, g.dev(xp), case.slot(case.recv_d, 0), case.slot(case.recv_d, 1),
                              case.slot(case.gath_d, 0), case.slot(case.gath_d, 1), case.send_c,
                              case.send_s, case.own_c, case.own_s, case.y, bits=bits)
            want = orc.call(P, rank, xp, None, None, case.slot(case.recv, 0), case.slot(case.recv, 1),
                            case.slot(case.gath, 0), case.slot(case.gath, 1), comp=False, bits=bits)
            eq(g.host(case.own_c, np.uint8), want["own_codes2"], f"P={P} rank={rank} plain codes2")
            eq(g.host(case.y, np.uint16), want["y"], f"P={P} rank={rank} plain y")
            # reduce-scatter: the same own-slot position in its rank-order sum
            mf, ms = state_of(case.n, P + rank, scale=0.1)
            mfd, msd = g.dev(mf), g.dev(ms)
            st = B.EchoState(mfd, msd, case.n, P, rank, bits=bits)
            x = x_of(case.n, 99 + P + rank)
            y_own = g.empty_bf16(case.Cn)
            B.echo_rs_call(st, g.dev(x), case.slot(case.recv_d, 0), case.slot(case.recv_d, 1),
                           case.send_c, case.send_s, y_own)
            want = orc.rs_call(P, rank, x, mf, ms, case.slot(case.recv, 0), case.slot(case.recv, 1),
                               bits=bits)
            eq(g.host(y_own, np.uint16), want["y_own"], f"P={P} rank={rank} rs y_own")
            eq(g.host(mfd, np.float32), mf, f"P={P} rank={rank} rs m_fast")
            eq(g.host(msd, np.float32), ms, f"P={P} rank={rank} rs m_slow")


@pytest.mark.parametrize("P,rank,k", [(8, 3, 5), (3, 1, 7), (1, 0, 2)])
def test_phases_equal_fused_call_and_in_place(P, rank, k):
    g = gu()
    fused = RankCase(P, rank, k, seed=77)
    phased = RankCase(P, rank, k, seed=77)
    inplace = RankCase(P, rank, k, seed=77)
    for call in range(3):
        x = x_of(fused.n, 500 + call)
        xd = g.dev(x)
        fused.gpu_call(xd)
        B.echo_call_entry(phased.st, xd, phased.send_c, phased.send_s)
        B.echo_call_reduce(phased.st, xd, phased.slot(phased.recv_d, 0), phased.slot(phased.recv_d, 1),
                           phased.own_c, phased.own_s, phased.y)
        B.echo_call_exit(phased.st, phased.slot(phased.gath_d, 0), phased.slot(phased.gath_d, 1),
                         phased.y)
        xi = g.dev(x)
        inplace.gpu_call(xi, y=xi)  # y == x: every element is read before it is written
        want = fused.oracle_call(x)
        fused.check(want)
        phased.mf, phased.ms = fused.mf, fused.ms
        phased.check(want)
        inplace.mf, inplace.ms = fused.mf, fused.ms
        inplace.check(want, y=xi)


@pytest.mark.parametrize("P,rank,k,bits", [(8, 2, 9, 4), (4, 3, 3, 4), (2, 0, 1, 4), (8, 6, 5, 8),
                                           (3, 1, 2, 8)])
def test_fused_equals_unfused_sequence(P, rank, k, bits):
    """echo_call == echo_encode + echo_reduce_shard (own slot = own encode)
    + echo_decode + echo_update, bit for bit."""
    g = gu()
    a = RankCase(P, rank, k, seed=5, bits=bits)
    b = RankCase(P, rank, k, seed=5, bits=bits)
    n, Cn = a.n, a.Cn
    cc = cb(Cn, bits)
    for call in range(3):
        x = x_of(n, 900 + call)
        xd = g.dev(x)
        a.gpu_call(xd)
        codes1, scales1 = g.empty_u8(cb(n, bits)), g.empty_f32(n // 128)
        B.echo_encode(b.st, xd, codes1, scales1)
        sh_c = [codes1[rank * cc:(rank + 1) * cc] if q == rank else b.recv_d[q][0] for q in range(P)]
        sh_s = [scales1[rank * Cn // 128:(rank + 1) * Cn // 128] if q == rank else b.recv_d[q][1]
                for q in range(P)]
        e2 = g.empty_f32(Cn)
        codes2 = torch.cat([b.gath_d[j][0] for j in range(P)])
        scales2 = torch.cat([b.gath_d[j][1] for j in range(P)])
        B.echo_reduce_shard(sh_c, sh_s, codes2[rank * cc:(rank + 1) * cc],
                            scales2[rank * Cn // 128:(rank + 1) * Cn // 128], None, e2, chunk_n=Cn,
                            bits=bits)
        y = g.empty_bf16(n)
        B.echo_decode(codes2, scales2, y, bits=bits)
        B.echo_update(b.st, xd, codes1, scales1, e2)
        eq(g.host(a.y, np.uint16), g.host(y, np.uint16), "y")
        eq(g.host(a.own_c, np.uint8), g.host(codes2, np.uint8)[rank * cc:(rank + 1) * cc], "codes2")
        eq(g.host(a.mfd, np.float32), g.host(b.mfd, np.float32), "m_fast")
        eq(g.host(a.msd, np.float32), g.host(b.msd, np.float32), "m_slow")
        sc = g.host(a.send_c, np.uint8)
        c1 = g.host(codes1, np.uint8)
        for j in range(P):
            if j != rank:
                eq(sc[j * cc:(j + 1) * cc], c1[j * cc:(j + 1) * cc], "send")


def test_state_init_zero_fills():
    g = gu()
    n = 8 * 128 * 5
    mf, ms = g.empty_f32(n, 3.0), g.empty_f32(n, -2.0)
    st = B.echo_state_init(mf, ms, n, 8, 3)
    torch.cuda.synchronize()
    assert st.n == n and st.nranks == 8 and st.rank == 3
    assert torch.count_nonzero(mf).item() == 0 and torch.count_nonzero(ms).item() == 0


@pytest.mark.parametrize("kind", ["zeros", "neg_zeros", "denormal", "huge", "mixed_tiny"])
def test_edge_inputs(kind):
    """Degenerate groups: all-zero input, signed zeros, bf16 denormals whose
    scale is itself denormal or underflows to zero, values near the top of
    the bf16 range, and groups mixing tiny and zero values."""
    g = gu()
    P, k = 4, 6
    n = P * 128 * k
    rng = np.random.default_rng(zlib.crc32(kind.encode()))
    if kind == "zeros":
        x = np.zeros(n, np.uint16)
    elif kind == "neg_zeros":
        x = np.full(n, 0x8000, np.uint16)
    elif kind == "denormal":
        x = (rng.integers(0, 128, n) | (rng.integers(0, 2, n) << 15)).astype(np.uint16)
    elif kind == "huge":
        x = I.to_bf16_bits(rng.standard_normal(n) * 1e36)
    else:
        v = rng.standard_normal(n) * 2.0 ** -133
        v[rng.random(n) < 0.5] = 0.0
        x = I.to_bf16_bits(v)
    case = RankCase(P, 1, k, seed=11)
    for call in range(2):
        case.gpu_call(g.dev(x))
        case.check(case.oracle_call(x))


def test_deterministic():
    g = gu()
    P, rank, k = 8, 4, 17
    x = x_of(P * 128 * k, 3)
    outs = []
    for _ in range(2):
        case = RankCase(P, rank, k, seed=9)
        case.gpu_call(g.dev(x))
        case.gpu_call(g.dev(x))
        torch.cuda.synchronize()
        outs.append([g.host(t, np.uint8) for t in (case.send_c, case.own_c, case.y, case.mfd, case.msd)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("P,k,calls", [(2, 1, 3), (3, 2, 3), (8, 4, 4)])
@pytest.mark.parametrize("bits", [4, 8])
def test_full_simulation_small(P, k, calls, bits):
    """P logical ranks on one GPU (each rank's encode, every chunk's reduce,
    each rank's fused call) against the oracle's full simulation."""
    g = gu()
    n = P * 128 * k
    ranks_np = [(np.zeros(n, np.float32), np.zeros(n, np.float32)) for _ in range(P)]
    mf = [a for a, _ in ranks_np]
    ms = [b for _, b in ranks_np]
    ranks = [g.GpuRank(np.zeros(n, np.uint16), mf[p], ms[p], P, p) for p in range(P)]
    for call in range(calls):
        xs = [x_of(n, 1000 * call + p) for p in range(P)]
        codes2, scales2, own2, own2s = g.gpu_simulate_call(ranks, xs, bits=bits)
        want = orc.simulate(xs, mf, ms, bits=bits)
        eq(g.host(codes2, np.uint8), want["codes2"], "codes2")
        eq(g.host(scales2, np.float32), want["scales2"], "scales2")
        for p, r in enumerate(ranks):
            eq(g.host(r.y, np.uint16), want["y"], f"y rank {p}")
            eq(g.host(r.mf, np.float32), mf[p], f"m_fast rank {p}")
            eq(g.host(r.ms, np.float32), ms[p], f"m_slow rank {p}")


def test_zero_padded_tail_full_simulation():
    """A tensor padded with zeros to whole groups per chunk (the tail spans
    the last chunk and part of the one before): the GPU matches the oracle's
    simulation, and the tail's outputs and averages stay zero."""
    g = gu()
    P, n, real = 4, 1536, 1036
    mf = [np.zeros(n, np.float32) for _ in range(P)]
    ms = [np.zeros(n, np.float32) for _ in range(P)]
    ranks = [g.GpuRank(np.zeros(n, np.uint16), mf[p], ms[p], P, p) for p in range(P)]
    for call in range(3):
        xs = [np.concatenate([I.to_bf16_bits(I.normal(real, I.stream_key("pad", call, p)) * (1 + p)),
                              np.zeros(n - real, np.uint16)]) for p in range(P)]
        codes2, scales2, _, _ = g.gpu_simulate_call(ranks, xs)
        want = orc.simulate(xs, mf, ms)
        eq(g.host(codes2, np.uint8), want["codes2"], f"call {call} codes2")
        for p, r in enumerate(ranks):
            eq(g.host(r.y, np.uint16), want["y"], f"call {call} y rank {p}")
            eq(g.host(r.mf, np.float32), mf[p], f"call {call} m_fast rank {p}")
            eq(g.host(r.ms, np.float32), ms[p], f"call {call} m_slow rank {p}")
            assert not g.host(r.y, np.uint16)[real:].any()
            assert not g.host(r.mf, np.float32)[real:].view(np.uint32).any()


def test_empty_calls_touch_nothing():
    """n == 0: every entry point returns success and writes nothing, with
    empty tensors (NULL pointers) or with real buffers passed in."""
    g = gu()
    P, rank = 8, 2
    empty = torch.empty(0, dtype=torch.uint8, device=g.DEV)
    st = B.echo_state_init(empty, empty, 0, P, rank)
    assert st.n == 0
    sent_u8 = g.empty_u8(4096, 0x5A)
    sent_f = g.empty_f32(1024, -7.0)
    sent_y = g.empty_u8(8192, 0xC3)
    lst = [None if q == rank else sent_u8 for q in range(P)]
    lsf = [None if q == rank else sent_f for q in range(P)]
    B.echo_encode(st, sent_y, sent_u8, sent_f)
    B.echo_call(st, sent_y, lst, lsf, lst, lsf, sent_u8, sent_f, sent_u8, sent_f, sent_y)
    B.echo_call_plain(P, rank, sent_y, lst, lsf, lst, lsf, sent_u8, sent_f, sent_u8, sent_f, sent_y, 0)
    B.echo_rs_call(st, sent_y, lst, lsf, sent_u8, sent_f, sent_y)
    B.echo_update(st, sent_y, sent_u8, sent_f, sent_f)
    B.echo_reduce_shard([sent_u8] * P, [sent_f] * P, sent_u8, sent_f, sent_y, sent_f, 0)
    B.echo_reduce_shard_sum([sent_u8] * P, [sent_f] * P, sent_y, sent_f, 0)
    B.echo_decode(sent_u8, sent_f, sent_y, 0, bits=8)
    torch.cuda.synchronize()
    assert (g.host(sent_u8, np.uint8) == 0x5A).all()
    assert (g.host(sent_f, np.float32) == -7.0).all()
    assert (g.host(sent_y, np.uint8) == 0xC3).all()


@pytest.mark.parametrize("P,rank,k", [(1, 0, 3), (2, 1, 5), (3, 2, 4), (8, 0, 9), (8, 6, 33), (16, 9, 2)])
@pytest.mark.parametrize("bits", [4, 8])
def test_call_plain_uncompensated(P, rank, k, bits):
    """The uncompensated call against the oracle with compensation off."""
    g = gu()
    case = RankCase(P, rank, k, seed=300 + P + k, bits=bits)
    n = case.n
    for call in range(2):
        x = x_of(n, 700 + call + k)
        B.echo_call_plain(P, rank, g.dev(x), case.slot(case.recv_d, 0), case.slot(case.recv_d, 1),
                          case.slot(case.gath_d, 0), case.slot(case.gath_d, 1), case.send_c,
                          case.send_s, case.own_c, case.own_s, case.y, bits=bits)
        want = orc.call(P, rank, x, None, None, case.slot(case.recv, 0), case.slot(case.recv, 1),
                        case.slot(case.gath, 0), case.slot(case.gath, 1), comp=False,
                        bits=bits)
        case.check(want)  # the averages stay untouched (zero), as the oracle's


@pytest.mark.parametrize("P,rank,k", [(8, 3, 9), (4, 0, 5)])
def test_deferred_update_on_side_stream_equals_fused(P, rank, k):
    """The critical-path split: encode + reduce_shard + exit on the main
    stream, the averages' update on a side stream (beside a matmul that
    consumes y), ordered by events; bit-identical to the fused call."""
    g = gu()
    fused = RankCase(P, rank, k, seed=61)
    split = RankCase(P, rank, k, seed=61)
    n, Cn = fused.n, fused.Cn
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    codes1, scales1 = g.empty_u8(n // 2), g.empty_f32(n // 128)
    e2 = g.empty_f32(Cn)
    updated = None
    w = torch.randn(128, 64, device=g.DEV, dtype=torch.bfloat16)
    for call in range(4):
        x = x_of(n, 40 + call)
        xd = g.dev(x)
        fused.gpu_call(xd)
        if updated is not None:
            main.wait_event(updated)  # the next entry pass reads the averages
        B.echo_encode(split.st, xd, codes1, scales1, stream=main)
        sh_c = [codes1[rank * Cn // 2:(rank + 1) * Cn // 2] if q == rank else split.recv_d[q][0]
                for q in range(P)]
        sh_s = [scales1[rank * Cn // 128:(rank + 1) * Cn // 128] if q == rank else split.recv_d[q][1]
                for q in range(P)]
        B.echo_reduce_shard(sh_c, sh_s, split.own_c, split.own_s, split.y[rank * Cn:(rank + 1) * Cn],
                            e2, chunk_n=Cn, stream=main)
        reduced = torch.cuda.Event()
        reduced.record(main)
        B.echo_call_exit(split.st, split.slot(split.gath_d, 0), split.slot(split.gath_d, 1), split.y,
                         stream=main)
        # the next layer's matmul on the critical stream consumes y
        h = split.y.view(torch.bfloat16).reshape(-1, 128) @ w
        side.wait_event(reduced)
        B.echo_update(split.st, xd, codes1, scales1, e2, stream=side)
        updated = torch.cuda.Event()
        updated.record(side)
        xd.record_stream(side)
        torch.cuda.synchronize()
        assert torch.isfinite(h.float()).all()
        g.eq(g.host(split.y, np.uint16), g.host(fused.y, np.uint16), f"call {call} y")
        g.eq(g.host(split.own_c, np.uint8), g.host(fused.own_c, np.uint8), f"call {call} codes2")
        g.eq(g.host(split.mfd, np.float32), g.host(fused.mfd, np.float32), f"call {call} m_fast")
        g.eq(g.host(split.msd, np.float32), g.host(fused.msd, np.float32), f"call {call} m_slow")
        c1 = g.host(codes1, np.uint8)
        fc = g.host(fused.send_c, np.uint8)
        for j in range(P):
            if j != rank:
                g.eq(c1[j * Cn // 2:(j + 1) * Cn // 2], fc[j * Cn // 2:(j + 1) * Cn // 2], "send")


@pytest.mark.parametrize("P,rank,k", [(1, 0, 3), (4, 0, 5), (8, 3, 9), (16, 11, 2)])
@pytest.mark.parametrize("bits", [4, 8])
def test_deferred_update_with_correction_array(P, rank, k, bits):
    """The deferred-update schedule with the correction kept as one array:
    echo_encode_corr + echo_reduce_shard + echo_call_exit on the main stream,
    echo_update_corr on a side stream; 4 calls against the oracle's fused
    call, and the array against the oracle's correction of its averages."""
    g = gu()
    case = RankCase(P, rank, k, seed=67, bits=bits)
    n, Cn, f = case.n, case.Cn, (1 if bits == 8 else 2)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    codes1, scales1 = g.empty_u8(n // f), g.empty_f32(n // 128)
    e2 = g.empty_f32(Cn)
    corr = g.empty_f32(n, 7.0)
    B.echo_correction(case.st, corr, stream=main)  # from the zero averages
    updated = None
    for call in range(4):
        x = x_of(n, 70 + call)
        xd = g.dev(x)
        if updated is not None:
            main.wait_event(updated)  # the entry pass reads the correction the update wrote
        B.echo_encode_corr(case.st, xd, corr, codes1, scales1, stream=main)
        sh_c = [codes1[rank * Cn // f:(rank + 1) * Cn // f] if q == rank else case.recv_d[q][0]
                for q in range(P)]
        sh_s = [scales1[rank * Cn // 128:(rank + 1) * Cn // 128] if q == rank else case.recv_d[q][1]
                for q in range(P)]
        B.echo_reduce_shard(sh_c, sh_s, case.own_c, case.own_s, case.y[rank * Cn:(rank + 1) * Cn],
                            e2, chunk_n=Cn, stream=main, bits=bits)
        reduced = torch.cuda.Event()
        reduced.record(main)
        B.echo_call_exit(case.st, case.slot(case.gath_d, 0), case.slot(case.gath_d, 1), case.y,
                         stream=main)
        side.wait_event(reduced)
        B.echo_update_corr(case.st, xd, codes1, scales1, e2, corr, stream=side)
        updated = torch.cuda.Event()
        updated.record(side)
        xd.record_stream(side)
        torch.cuda.synchronize()
        want = case.oracle_call(x)
        c1 = g.host(codes1, np.uint8)
        s1 = g.host(scales1, np.float32)
        for j in range(P):
            if j != rank:
                cs, gs = slice(j * Cn // f, (j + 1) * Cn // f), slice(j * Cn // 128, (j + 1) * Cn // 128)
                eq(c1[cs], want["send_codes"][cs], f"call {call} send codes chunk {j}")
                eq(s1[gs], want["send_scales"][gs], f"call {call} send scales chunk {j}")
        eq(g.host(case.own_c, np.uint8), want["own_codes2"], f"call {call} own codes2")
        eq(g.host(case.own_s, np.float32), want["own_scales2"], f"call {call} own scales2")
        eq(g.host(case.y, np.uint16), want["y"], f"call {call} y")
        eq(g.host(case.mfd, np.float32), case.mf, f"call {call} m_fast")
        eq(g.host(case.msd, np.float32), case.ms, f"call {call} m_slow")
        eq(g.host(corr, np.float32), orc.correction(case.mf, case.ms), f"call {call} correction")


def test_correction_of_given_averages():
    """echo_correction against the oracle's correction on averages spanning
    large, tiny, subnormal and cancelling values."""
    g = gu()
    rng = np.random.default_rng(71)
    n = 8 * 128 * 37
    mf = (rng.standard_normal(n) * np.exp2(rng.integers(-140, 120, n))).astype(np.float32)
    ms = (rng.standard_normal(n) * np.exp2(rng.integers(-140, 120, n))).astype(np.float32)
    ms[::5] = -mf[::5]
    mf[1::9] = np.finfo(np.float32).max
    ms[1::9] = np.finfo(np.float32).max
    mfd, msd = g.dev(mf), g.dev(ms)
    st = B.EchoState(mfd, msd, n, 8, 2)
    corr = g.empty_f32(n, 3.0)
    B.echo_correction(st, corr)
    torch.cuda.synchronize()
    eq(g.host(corr, np.float32), orc.correction(mf, ms), "correction")


def _adversarial_groups(rng, ngroups):
    """x' values placed on the quantizer's decision boundaries.  Each group:
    element 0 is the absmax A, s = fl(A / 7), and the rest are fl((k + 1/2) s)
    for k in -7..6 together with their 1-3 ulp neighbours, in random order;
    scales range over normal, denormal and near-overflow magnitudes."""
    vals = np.zeros((ngroups, 128), np.float32)
    for gi in range(ngroups):
        kind = gi % 6
        if kind == 0:
            A = np.float32(rng.uniform(0.5, 8.0))
        elif kind == 1:
            A = np.float32(7.0 * 2.0 ** rng.integers(-20, 20))  # s a power of two: exact ties
        elif kind == 2:
            A = np.float32(rng.uniform(1.0, 1000.0) * 2.0 ** -135)  # denormal scale
        elif kind == 3:
            A = np.float32(rng.uniform(1.0, 6.0) * 2.0 ** 124)  # scale near 2^126
        elif kind == 4:
            A = np.float32(rng.uniform(1e-30, 1e-20))
        else:
            A = np.float32(rng.uniform(1e20, 1e30))
        s = np.float32(A / np.float32(7.0))
        cand = []
        for k in range(-7, 7):
            t = np.float32(np.float32(k + 0.5) * s)
            cand.append(t)
            up, dn = t, t
            for _ in range(3):
                up = np.nextafter(up, np.float32(np.inf))
                dn = np.nextafter(dn, np.float32(-np.inf))
                cand += [up, dn]
        cand = np.array(cand, np.float32)
        cand = cand[np.abs(cand) <= A]
        rng.shuffle(cand)
        row = np.zeros(128, np.float32)
        row[0] = A if rng.random() < 0.5 else -A
        m = min(127, cand.size)
        row[1:1 + m] = cand[:m]
        vals[gi] = row
    return vals.ravel()


def test_quantizer_decision_boundaries():
    """Codes for quotients exactly on, and a few ulps beside, every rounding
    boundary -- the cases where a reciprocal-multiply could disagree with the
    correctly rounded division -- match the oracle bit for bit."""
    g = gu()
    rng = np.random.default_rng(123)
    t = _adversarial_groups(rng, 6 * 200)
    n = t.size
    x = np.zeros(n, np.uint16)                 # x' = 0 - (0.5 * (-2t) + 0.5 * 0) = t exactly
    mf = (np.float32(-2.0) * t).astype(np.float32)
    ms = np.zeros(n, np.float32)
    assert np.all(np.isfinite(mf))
    st = B.EchoState(g.dev(mf), g.dev(ms), n, 1, 0)
    codes, scales = g.empty_u8(n // 2), g.empty_f32(n // 128)
    B.echo_encode(st, g.dev(x), codes, scales)
    want_c, want_s, xp = orc.encode(x, mf, ms, want_xp=True)
    assert np.array_equal(xp.view(np.uint32), t.view(np.uint32))  # the construction holds
    eq(g.host(scales, np.float32), want_s, "scales")
    eq(g.host(codes, np.uint8), want_c, "codes")


@pytest.mark.parametrize("ulps", [0, 1, -1, 3])
def test_requantizer_decision_boundaries(ulps):
    """The reduce stage's quantizer on sums that sit on half-integers of the
    stage-2 scale: shard 0 carries codes with scale s0 (one code 7 per group
    fixes amax = 7 s0), shard 1 odd codes with scale s0/2 moved by `ulps`, so
    S / s2 = c0 + c1/2 (+ a few ulps)."""
    g = gu()
    rng = np.random.default_rng(77 + ulps)
    groups = 512
    cn = 128 * groups
    q0 = rng.integers(-4, 5, cn).astype(np.int8)  # |c0 + c1/2| <= 6.5 < 7: amax stays 7 s0
    q0[::128] = 7
    q1 = (rng.integers(-3, 3, cn) * 2 + 1).astype(np.int8)
    q1[::128] = 0
    s0 = rng.uniform(0.01, 100.0, groups).astype(np.float32)
    s0[::2] = (2.0 ** rng.integers(-30, 30, groups // 2)).astype(np.float32)  # s2 == s0: exact ties
    s1 = (s0 / np.float32(2.0)).astype(np.float32)
    for _ in range(abs(ulps)):
        s1 = np.nextafter(s1, np.float32(np.inf if ulps > 0 else -np.inf)).astype(np.float32)
    msgs = [(orc.pack(q0), s0), (orc.pack(q1), s1)]
    out_c, out_s = g.empty_u8(cn // 2), g.empty_f32(cn // 128)
    out_y, out_e2 = g.empty_bf16(cn), g.empty_f32(cn)
    B.echo_reduce_shard([g.dev(c) for c, _ in msgs], [g.dev(sc) for _, sc in msgs], out_c, out_s,
                        out_y, out_e2, chunk_n=cn)
    wc, ws, wy, we = orc.reduce_chunk([c for c, _ in msgs], [sc for _, sc in msgs], cn)
    eq(g.host(out_s, np.float32), ws, "scales2")
    eq(g.host(out_c, np.uint8), wc, "codes2")
    eq(g.host(out_y, np.uint16), wy, "y")
    eq(g.host(out_e2, np.float32), we, "e2")


# ---- reduce-scatter only ----------------------------------------------------------------

@pytest.mark.parametrize("P", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("k", [1, 5, 129])
@pytest.mark.parametrize("bits", [4, 8])
def test_reduce_shard_sum(P, k, bits):
    g = gu()
    cn = 128 * k
    msgs = [I.int4_message(cn, I.stream_key("rss", P, k, q), zero_group_frac=0.05, any_byte=(q % 2 == 1),
                           bits=bits) for q in range(P)]
    y, e = g.empty_bf16(cn), g.empty_f32(cn)
    B.echo_reduce_shard_sum([g.dev(c) for c, _ in msgs], [g.dev(s) for _, s in msgs], y, e, chunk_n=cn,
                            bits=bits)
    wy, we = orc.reduce_chunk_sum([c for c, _ in msgs], [s for _, s in msgs], cn, bits=bits)
    eq(g.host(y, np.uint16), wy, "y")
    eq(g.host(e, np.float32), we, "e")


class RsCase(RankCase):
    def __init__(self, P, rank, k, seed, bits=4):
        super().__init__(P, rank, k, seed, bits=bits)
        self.y_own = gu().empty_bf16(self.Cn)

    def gpu_rs(self, xd):
        B.echo_rs_call(self.st, xd, self.slot(self.recv_d, 0), self.slot(self.recv_d, 1),
                       self.send_c, self.send_s, self.y_own)

    def oracle_rs(self, x):
        return orc.rs_call(self.P, self.rank, x, self.mf, self.ms, self.slot(self.recv, 0),
                           self.slot(self.recv, 1), bits=self.bits)

    def check_rs(self, want):
        g = gu()
        P, r, Cn = self.P, self.rank, self.Cn
        sc = g.host(self.send_c, np.uint8)
        ss = g.host(self.send_s, np.float32)
        cbc = cb(Cn, self.bits)
        for j in range(P):
            cs = slice(j * cbc, (j + 1) * cbc)
            gs = slice(j * Cn // 128, (j + 1) * Cn // 128)
            if j == r:
                assert np.all(sc[cs] == 0xAB) and np.all(ss[gs] == -3.0)
            else:
                eq(sc[cs], want["send_codes"][cs], f"send codes chunk {j}")
                eq(ss[gs], want["send_scales"][gs], f"send scales chunk {j}")
        eq(g.host(self.y_own, np.uint16), want["y_own"], "y_own")
        eq(g.host(self.mfd, np.float32), self.mf, "m_fast")
        eq(g.host(self.msd, np.float32), self.ms, "m_slow")


@pytest.mark.parametrize("P,rank,k", [(1, 0, 2), (2, 1, 3), (3, 0, 5), (8, 0, 16), (8, 7, 33), (16, 4, 3)])
@pytest.mark.parametrize("bits", [4, 8])
def test_rs_call_rank_mode(P, rank, k, bits):
    g = gu()
    case = RsCase(P, rank, k, seed=400 + P * 10 + rank, bits=bits)
    for call in range(3):
        x = x_of(case.n, 800 + call + k)
        case.gpu_rs(g.dev(x))
        case.check_rs(case.oracle_rs(x))


@pytest.mark.parametrize("P,rank,k,bits", [(8, 5, 9, 4), (4, 0, 3, 4), (8, 2, 3, 8)])
def test_rs_fused_equals_unfused(P, rank, k, bits):
    """echo_rs_call == echo_encode + echo_reduce_shard_sum (own slot = own
    stage-1 chunk) + echo_update, bit for bit, and the phased form too."""
    g = gu()
    a = RsCase(P, rank, k, seed=9, bits=bits)
    b = RsCase(P, rank, k, seed=9, bits=bits)
    c = RsCase(P, rank, k, seed=9, bits=bits)
    n, Cn = a.n, a.Cn
    cc = cb(Cn, bits)
    for call in range(3):
        xd = g.dev(x_of(n, 60 + call))
        a.gpu_rs(xd)
        codes1, scales1 = g.empty_u8(cb(n, bits)), g.empty_f32(n // 128)
        B.echo_encode(b.st, xd, codes1, scales1)
        sh_c = [codes1[rank * cc:(rank + 1) * cc] if q == rank else b.recv_d[q][0] for q in range(P)]
        sh_s = [scales1[rank * Cn // 128:(rank + 1) * Cn // 128] if q == rank else b.recv_d[q][1]
                for q in range(P)]
        e = g.empty_f32(Cn)
        B.echo_reduce_shard_sum(sh_c, sh_s, b.y_own, e, chunk_n=Cn, bits=bits)
        B.echo_update(b.st, xd, codes1, scales1, e)
        B.echo_call_entry(c.st, xd, c.send_c, c.send_s)
        B.echo_rs_reduce(c.st, xd, c.slot(c.recv_d, 0), c.slot(c.recv_d, 1), c.y_own)
        for other in (b, c):
            eq(g.host(a.y_own, np.uint16), g.host(other.y_own, np.uint16), "y_own")
            eq(g.host(a.mfd, np.float32), g.host(other.mfd, np.float32), "m_fast")
            eq(g.host(a.msd, np.float32), g.host(other.msd, np.float32), "m_slow")


@pytest.mark.parametrize("P,k,calls", [(3, 2, 3), (8, 4, 4)])
def test_rs_full_simulation(P, k, calls):
    """P logical ranks, each running echo_rs_call on the others' stage-1
    chunks of its own chunk, against the oracle's reduce-scatter simulation."""
    g = gu()
    n = P * 128 * k
    Cn = n // P
    mf = [np.zeros(n, np.float32) for _ in range(P)]
    ms = [np.zeros(n, np.float32) for _ in range(P)]
    ranks = [g.GpuRank(np.zeros(n, np.uint16), mf[p], ms[p], P, p) for p in range(P)]
    y_own = [g.empty_bf16(Cn) for _ in range(P)]
    for call in range(calls):
        xs = [x_of(n, 3000 + 10 * call + p) for p in range(P)]
        for r, x in zip(ranks, xs):
            r.x.copy_(g.dev(x))
            B.echo_encode(r.st, r.x, r.codes1, r.scales1)
        for p, r in enumerate(ranks):
            recv_c = [None if q == p else ranks[q].codes1[p * Cn // 2:(p + 1) * Cn // 2] for q in range(P)]
            recv_s = [None if q == p else ranks[q].scales1[p * Cn // 128:(p + 1) * Cn // 128] for q in range(P)]
            B.echo_rs_call(r.st, r.x, recv_c, recv_s, r.send_codes, r.send_scales, y_own[p])
        torch.cuda.synchronize()
        want = orc.rs_simulate(xs, mf, ms)
        for p, r in enumerate(ranks):
            eq(g.host(y_own[p], np.uint16), want["y"][p * Cn:(p + 1) * Cn], f"call {call} y rank {p}")
            eq(g.host(r.mf, np.float32), mf[p], f"call {call} m_fast rank {p}")
            eq(g.host(r.ms, np.float32), ms[p], f"call {call} m_slow rank {p}")



@pytest.mark.parametrize("P,rank,k", [(8, 3, 6), (4, 0, 5)])
def test_mixed_code_width_sequence(P, rank, k):
    """The serving policy: one state carried through 8 calls, the first half
    with 8-bit messages and the second half with 4-bit ones (the width is set
    on the state before each call), against the oracle call by call."""
    g = gu()
    c4 = RankCase(P, rank, k, seed=77, bits=4)
    c8 = RankCase(P, rank, k, seed=77, bits=8)
    mfd, msd = c4.mfd, c4.msd
    mf, ms = c4.mf, c4.ms
    for call in range(8):
        bits = 8 if call < 4 else 4
        c = c8 if bits == 8 else c4
        st = B.EchoState(mfd, msd, c.n, P, rank, bits=bits)
        x = x_of(c.n, 5000 + call)
        B.echo_call(st, g.dev(x), c.slot(c.recv_d, 0), c.slot(c.recv_d, 1), c.slot(c.gath_d, 0),
                    c.slot(c.gath_d, 1), c.send_c, c.send_s, c.own_c, c.own_s, c.y)
        want = orc.call(P, rank, x, mf, ms, c.slot(c.recv, 0), c.slot(c.recv, 1), c.slot(c.gath, 0),
                        c.slot(c.gath, 1), bits=bits)
        eq(g.host(c.y, np.uint16), want["y"], f"call {call} ({bits}-bit) y")
        eq(g.host(c.own_c, np.uint8), want["own_codes2"], f"call {call} codes2")
        eq(g.host(mfd, np.float32), mf, f"call {call} m_fast")
        eq(g.host(msd, np.float32), ms, f"call {call} m_slow")


def test_checkpoint_resume_is_bit_identical():
    """The averages are the only state carried between calls: saving them
    after k calls and continuing from the saved copy in fresh buffers (as a
    checkpoint restore would) gives exactly the uninterrupted run."""
    g = gu()
    P, rank, k = 8, 2, 7
    whole = RankCase(P, rank, k, seed=91)
    xs = [x_of(whole.n, 9100 + c) for c in range(6)]
    for c in range(3):
        whole.gpu_call(g.dev(xs[c]))
    torch.cuda.synchronize()
    saved_mf = g.host(whole.mfd, np.float32).copy()  # the checkpoint, on the host
    saved_ms = g.host(whole.msd, np.float32).copy()
    for c in range(3, 6):
        whole.gpu_call(g.dev(xs[c]))
    resumed = RankCase(P, rank, k, seed=91)
    resumed.mfd.copy_(g.dev(saved_mf))
    resumed.msd.copy_(g.dev(saved_ms))
    for c in range(3, 6):
        resumed.gpu_call(g.dev(xs[c]))
    torch.cuda.synchronize()
    eq(g.host(resumed.y, np.uint16), g.host(whole.y, np.uint16), "y after resume")
    eq(g.host(resumed.mfd, np.float32), g.host(whole.mfd, np.float32), "m_fast after resume")
    eq(g.host(resumed.msd, np.float32), g.host(whole.msd, np.float32), "m_slow after resume")


def test_prepared_call_matches_echo_call():
    """echo_call_prepare marshals the arguments once; each call of it is the
    same echo_call on the buffers' current contents."""
    g = gu()
    P, rank, k = 8, 4, 5
    a = RankCase(P, rank, k, seed=33)
    b = RankCase(P, rank, k, seed=33)
    xb = g.dev(np.zeros(b.n, np.uint16))
    prepared = B.echo_call_prepare(b.st, xb, b.slot(b.recv_d, 0), b.slot(b.recv_d, 1),
                                   b.slot(b.gath_d, 0), b.slot(b.gath_d, 1), b.send_c, b.send_s,
                                   b.own_c, b.own_s, b.y)
    side = torch.cuda.Stream()
    for call in range(4):
        x = x_of(a.n, 3300 + call)
        a.gpu_call(g.dev(x))
        xb.copy_(g.dev(x))
        if call % 2:
            prepared()
        else:  # an explicit stream, ordered after the input copy
            side.wait_stream(torch.cuda.current_stream())
            prepared(side)
            torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        eq(g.host(b.y, np.uint16), g.host(a.y, np.uint16), f"call {call} y")
        eq(g.host(b.mfd, np.float32), g.host(a.mfd, np.float32), f"call {call} m_fast")
        eq(g.host(b.own_c, np.uint8), g.host(a.own_c, np.uint8), f"call {call} codes2")


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 257 + 16 * 256 * 3, (1 << 20) + 48])
def test_stream_copy_copies_exactly(nbytes):
    """The measurement copy moves every byte and touches nothing beyond."""
    g = gu()
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=g.DEV)
    dst = g.empty_u8(nbytes + 64, 0xEE)
    B.echo_stream_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert (g.host(dst[nbytes:], np.uint8) == 0xEE).all()


def test_binding_checks_tensor_arguments():
    """Non-contiguous or undersized tensors are refused on the host with the
    argument named; the same call with proper buffers runs."""
    g = gu()
    P, rank, k = 4, 1, 3
    case = RankCase(P, rank, k, seed=3)
    xd = g.dev(x_of(case.n, 1))
    short_y = g.empty_bf16(case.n - 128)
    with pytest.raises(ValueError, match="y: holds"):
        B.echo_call(case.st, xd, case.slot(case.recv_d, 0), case.slot(case.recv_d, 1),
                    case.slot(case.gath_d, 0), case.slot(case.gath_d, 1), case.send_c, case.send_s,
                    case.own_c, case.own_s, short_y)
    strided = torch.empty(2 * case.n, dtype=torch.int16, device=g.DEV)[::2]
    with pytest.raises(ValueError, match="x: the tensor must be contiguous"):
        B.echo_call_entry(case.st, strided, case.send_c, case.send_s)
    bad = case.slot(case.recv_d, 0)
    bad[(rank + 1) % P] = bad[(rank + 1) % P][:-1]
    with pytest.raises(ValueError, match=r"recv_codes\[\d+\]: holds"):
        B.echo_call_reduce(case.st, xd, bad, case.slot(case.recv_d, 1), case.own_c, case.own_s, case.y)
    torch.cuda.synchronize()
    case.gpu_call(xd)
    case.check(case.oracle_call(g.host(xd, np.uint16)))


@pytest.mark.parametrize("P,rank,k,bits", [(1, 0, 3, 4), (3, 1, 5, 4), (8, 0, 4, 4), (8, 5, 3, 8),
                                           (16, 7, 2, 4), (16, 0, 3, 8)])
def test_entry_in_chunk_ranges_then_per_chunk_exit(P, rank, k, bits):
    """The pipelined form of a call: the entry pass in chunk ranges (shuffled,
    half of them on a second stream), the reduce, then the exit one gathered
    chunk at a time with echo_decode -- against the oracle's call, twice in a
    row (the averages carried)."""
    g = gu()
    rng = np.random.default_rng(1000 * P + 10 * rank + bits)
    case = RankCase(P, rank, k, seed=4000 + P, bits=bits)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    C = case.Cn
    for call in range(2):
        x = x_of(case.n, 77 + call)
        xd = g.dev(x)
        cuts = sorted(set(rng.integers(0, P + 1, size=3).tolist()) | {0, P})
        ranges = list(zip(cuts[:-1], cuts[1:]))
        rng.shuffle(ranges)
        side.wait_stream(main)
        for i, (j0, j1) in enumerate(ranges):
            B.echo_call_entry_range(case.st, xd, j0, j1, case.send_c, case.send_s, side if i % 2 else main)
        main.wait_stream(side)
        B.echo_call_reduce(case.st, xd, case.slot(case.recv_d, 0), case.slot(case.recv_d, 1),
                           case.own_c, case.own_s, case.y)
        for j in range(P):
            if j == rank:
                continue
            B.echo_decode(case.gath_d[j][0], case.gath_d[j][1], case.y[j * C:(j + 1) * C], n=C, bits=bits)
        case.check(case.oracle_call(x))


def test_concurrent_sequences_on_two_streams_from_two_threads():
    """No global state: two independent call sequences (different P, rank,
    width and state), each issued from its own host thread on its own stream
    with no synchronization between them, both equal the oracle."""
    import threading

    g = gu()
    cases = [RankCase(8, 3, 6, seed=61, bits=4), RankCase(5, 0, 9, seed=62, bits=8)]
    inputs = [[x_of(c.n, 6100 + 10 * i + k) for k in range(4)] for i, c in enumerate(cases)]
    devs = [[g.dev(x) for x in xs] for xs in inputs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []

    def run(i):
        try:
            c, s = cases[i], streams[i]
            for xd in devs[i]:
                B.echo_call(c.st, xd, c.slot(c.recv_d, 0), c.slot(c.recv_d, 1), c.slot(c.gath_d, 0),
                            c.slot(c.gath_d, 1), c.send_c, c.send_s, c.own_c, c.own_s, c.y, s)
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for c, xs in zip(cases, inputs):
        for x in xs:
            want = c.oracle_call(x)
        c.check(want)  # the last call's outputs and the state after all four
