"""The oracle's threaded driver (orc_call_mt, orc_rs_call_mt) against the
single-thread call it parallelizes: for every thread count, rank count, rank, code width and
with or without compensation, a sequence of rank-mode calls gives the same
bytes -- send message, own stage-2 chunk, y and both averages.  Group counts
are chosen so that the runs of groups are ragged and some threads get none."""
import numpy as np
import pytest

from error_compensated_bit_echo_amd import inputs as I
from oracle import oracle as orc


def _messages(P, rank, C, key, bits):
    recv = [None if q == rank else I.int4_message(C, I.stream_key(*key, "r", q), zero_group_frac=0.1,
                                                   bits=bits) for q in range(P)]
    gath = [None if j == rank else I.int4_message(C, I.stream_key(*key, "g", j), scale_lo=0.15,
                                                   scale_hi=1.5, bits=bits) for j in range(P)]
    sl = lambda arr, k: [None if m is None else m[k] for m in arr]  # noqa: E731
    return sl(recv, 0), sl(recv, 1), sl(gath, 0), sl(gath, 1)


def _bits_of(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("threads", [1, 2, 3, 16])
@pytest.mark.parametrize("P,rank,k", [(1, 0, 5), (3, 2, 7), (8, 0, 3), (8, 5, 1), (16, 11, 2)])
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("comp", [True, False])
def test_threaded_call_equals_single_thread(threads, P, rank, k, bits, comp):
    C = 128 * k
    n = P * C
    key = ("mt", P, rank, k, bits)
    rc, rs, gc, gs = _messages(P, rank, C, key, bits)
    mf1, ms1 = np.zeros(n, np.float32), np.zeros(n, np.float32)
    mfT, msT = np.zeros(n, np.float32), np.zeros(n, np.float32)
    for call in range(3):
        x = I.to_bf16_bits(3.0 * I.normal(n, I.stream_key(*key, "x", call)))
        want = orc.call(P, rank, x, mf1, ms1, rc, rs, gc, gs, comp=comp, bits=bits)
        got = orc.call(P, rank, x, mfT, msT, rc, rs, gc, gs, comp=comp, bits=bits, threads=threads)
        for name in ("own_codes2", "own_scales2", "y"):
            assert np.array_equal(_bits_of(got[name]), _bits_of(want[name])), (name, call)
        f = 1 if bits == 8 else 2
        for j in range(P):
            if j == rank:
                continue
            cs, ss = slice(j * C // f, (j + 1) * C // f), slice(j * C // 128, (j + 1) * C // 128)
            assert np.array_equal(got["send_codes"][cs], want["send_codes"][cs]), ("send codes", j, call)
            assert np.array_equal(_bits_of(got["send_scales"][ss]), _bits_of(want["send_scales"][ss]))
        assert np.array_equal(mfT.view(np.uint32), mf1.view(np.uint32)), ("m_fast", call)
        assert np.array_equal(msT.view(np.uint32), ms1.view(np.uint32)), ("m_slow", call)


def test_threaded_call_rejects_what_the_call_rejects():
    x = np.zeros(8 * 128, np.uint16)
    mf, ms = np.zeros(x.size, np.float32), np.zeros(x.size, np.float32)
    none = [None] * 8
    for kw in (dict(bits=5), dict(bits=4)):
        with pytest.raises(ValueError):
            # P = 8 with 1024 elements has one group per chunk; rank 8 is out of range
            orc.call(8, 8, x, mf, ms, none, none, none, none, threads=4, **kw)


@pytest.mark.parametrize("threads", [2, 3, 16])
@pytest.mark.parametrize("P,rank,k", [(1, 0, 5), (3, 2, 7), (8, 5, 1), (16, 11, 2)])
@pytest.mark.parametrize("bits", [4, 8])
def test_threaded_reduce_scatter_equals_single_thread(threads, P, rank, k, bits):
    C = 128 * k
    n = P * C
    key = ("mt-rs", P, rank, k, bits)
    rc, rs, _, _ = _messages(P, rank, C, key, bits)
    mf1, ms1 = np.zeros(n, np.float32), np.zeros(n, np.float32)
    mfT, msT = np.zeros(n, np.float32), np.zeros(n, np.float32)
    for call in range(3):
        x = I.to_bf16_bits(3.0 * I.normal(n, I.stream_key(*key, "x", call)))
        want = orc.rs_call(P, rank, x, mf1, ms1, rc, rs, bits=bits)
        got = orc.rs_call(P, rank, x, mfT, msT, rc, rs, bits=bits, threads=threads)
        assert np.array_equal(got["y_own"], want["y_own"]), call
        f = 1 if bits == 8 else 2
        keep = np.ones(n // f, bool)
        keep[rank * C // f:(rank + 1) * C // f] = False
        assert np.array_equal(got["send_codes"][keep], want["send_codes"][keep]), call
        assert np.array_equal(mfT.view(np.uint32), mf1.view(np.uint32)), ("m_fast", call)
        assert np.array_equal(msT.view(np.uint32), ms1.view(np.uint32)), ("m_slow", call)
