"""numpy front end of the CPU oracle (oracle/echo_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark; the product path never imports it.

Every function takes and returns numpy arrays on the host:
bf16 tensors as uint16 bit patterns, packed int4 codes as uint8, scales and
averages as float32.  The C side does all the arithmetic.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_DEFAULT_LIB = os.path.join(_HERE, "liborc.so")
# ECHO_ORACLE_LIB names another build of the same sources; the mutation test
# uses it to run the pins against copies with planted mistakes
_LIB_PATH = os.environ.get("ECHO_ORACLE_LIB") or _DEFAULT_LIB

GROUP = 128
QMAX = 7
QMAX8 = 127
W_FAST = 0.5
W_SLOW = 0.5
BETA_FAST = 0.5
ALPHA_FAST = 0.5
BETA_SLOW = 0.875
ALPHA_SLOW = 0.125
MAX_RANKS = 16

_u8p = C.POINTER(C.c_uint8)
_u16p = C.POINTER(C.c_uint16)
_i8p = C.POINTER(C.c_int8)
_f32p = C.POINTER(C.c_float)
_vp = C.c_void_p


def _load():
    if _LIB_PATH == _DEFAULT_LIB and not os.path.exists(_LIB_PATH):
        from oracle import build as _b  # noqa: WPS433 (build on first use)

        _b.build()
    lib = C.CDLL(_LIB_PATH)
    sig = {
        "orc_counters_reset": (None, []),
        "orc_counter": (C.c_longlong, [C.c_int]),
        "orc_f32_to_bf16": (C.c_uint16, [C.c_float]),
        "orc_bf16_to_f32": (C.c_float, [C.c_uint16]),
        "orc_quantize_group": (None, [_vp, C.c_int, _vp, _vp, C.c_int]),
        "orc_quantize_group_q": (None, [_vp, C.c_int, C.c_int, _vp, _vp, C.c_int]),
        "orc_pack_codes": (None, [_vp, C.c_int64, _vp, C.c_int]),
        "orc_unpack_codes": (None, [_vp, C.c_int64, _vp, C.c_int]),
        "orc_pack": (None, [_vp, C.c_int64, _vp]),
        "orc_unpack": (None, [_vp, C.c_int64, _vp]),
        "orc_ema_refresh": (None, [C.c_int64, _vp, _vp, _vp]),
        "orc_encode": (None, [C.c_int64, _vp, _vp, _vp, _vp, _vp, _vp, C.c_int, C.c_int]),
        "orc_reduce_chunk": (None, [C.c_int, C.c_int64, _vp, _vp, _vp, _vp, _vp, _vp, C.c_int]),
        "orc_decode": (None, [C.c_int64, _vp, _vp, _vp, C.c_int]),
        "orc_update": (None, [C.c_int64, C.c_int, C.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                              C.c_int]),
        "orc_call": (C.c_int, [C.c_int, C.c_int, C.c_int64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, _vp, _vp, C.c_int, C.c_int]),
        "orc_call_mt": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int64, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _vp, C.c_int, C.c_int]),
        "orc_rs_call_mt": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int64, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _vp, C.c_int, C.c_int]),
        "orc_correction": (None, [C.c_int64, _vp, _vp, _vp]),
        "orc_encode_corr": (None, [C.c_int64, _vp, _vp, _vp, _vp, C.c_int]),
        "orc_update_corr": (None, [C.c_int64, C.c_int, C.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   C.c_int]),
        "orc_update_span": (None, [C.c_int64, C.c_int64, C.c_int64, C.c_int64, _vp, _vp, _vp, _vp,
                                   _vp, _vp, _vp, C.c_int]),
        "orc_simulate": (C.c_int, [C.c_int, C.c_int64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _vp, C.c_int, C.c_int]),
        "orc_reduce_chunk_sum": (None, [C.c_int, C.c_int64, _vp, _vp, _vp, _vp, C.c_int]),
        "orc_rs_call": (C.c_int, [C.c_int, C.c_int, C.c_int64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, C.c_int, C.c_int]),
        "orc_rs_simulate": (C.c_int, [C.c_int, C.c_int64, _vp, _vp, _vp, _vp, _vp, _vp,
                                      C.c_int, C.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def _p(a):
    """Address of a C-contiguous numpy array (None -> NULL)."""
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _ptr_array(arrs):
    """void*[len(arrs)] holding the addresses of the arrays (None -> NULL)."""
    out = (C.c_void_p * max(1, len(arrs)))()
    for i, a in enumerate(arrs):
        out[i] = _p(a)
    return out


# ---- element helpers --------------------------------------------------------

def f32_to_bf16(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    f = lib().orc_f32_to_bf16
    return np.array([f(float(t)) for t in v], dtype=np.uint16)


def bf16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def quantize_group(v, stage: int = 0):
    v = np.ascontiguousarray(v, dtype=np.float32)
    q = np.zeros(v.size, dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    lib().orc_quantize_group(_p(v), v.size, _p(q), _p(s), stage)
    return q, float(s[0])


def code_bytes(n: int, bits: int = 4) -> int:
    return n if bits == 8 else n // 2


def quantize_group_q(v, qmax: int, stage: int = 0):
    v = np.ascontiguousarray(v, dtype=np.float32)
    q = np.zeros(v.size, dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    lib().orc_quantize_group_q(_p(v), v.size, int(qmax), _p(q), _p(s), stage)
    return q, float(s[0])


def pack_codes(q, bits: int = 4) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    out = np.zeros(code_bytes(q.size, bits), dtype=np.uint8)
    lib().orc_pack_codes(_p(q), q.size, _p(out), bits)
    return out


def unpack_codes(codes, n: int, bits: int = 4) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    q = np.zeros(n, dtype=np.int8)
    lib().orc_unpack_codes(_p(codes), n, _p(q), bits)
    return q


def pack(q) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    out = np.zeros(q.size // 2, dtype=np.uint8)
    lib().orc_pack(_p(q), q.size, _p(out))
    return out


def unpack(codes, n: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    q = np.zeros(n, dtype=np.int8)
    lib().orc_unpack(_p(codes), n, _p(q))
    return q


def ema_refresh(m_fast, m_slow, r) -> None:
    lib().orc_ema_refresh(r.size, _p(m_fast), _p(m_slow), _p(np.ascontiguousarray(r, np.float32)))


def counters_reset() -> None:
    lib().orc_counters_reset()


def counter(stage: int) -> int:
    return int(lib().orc_counter(stage))


# ---- pipeline steps -----------------------------------------------------------

def encode(x, m_fast=None, m_slow=None, comp: bool = True, want_xp: bool = False, bits: int = 4):
    """Entry pass. Returns (codes u8[n/2 or n], scales f32[n/128]) (+ x' if want_xp)."""
    n = x.size
    codes = np.zeros(code_bytes(n, bits), np.uint8)
    scales = np.zeros(n // GROUP, np.float32)
    xp = np.zeros(n, np.float32) if want_xp else None
    lib().orc_encode(n, _p(x), _p(m_fast) if comp else None, _p(m_slow) if comp else None,
                     _p(codes), _p(scales), _p(xp), int(bool(comp)), bits)
    return (codes, scales, xp) if want_xp else (codes, scales)


def reduce_chunk(shard_codes, shard_scales, chunk_n: int, bits: int = 4):
    """Reduce stage for one chunk. Returns (codes2, scales2, y_bf16, e2)."""
    P = len(shard_codes)
    codes2 = np.zeros(code_bytes(chunk_n, bits), np.uint8)
    scales2 = np.zeros(chunk_n // GROUP, np.float32)
    y = np.zeros(chunk_n, np.uint16)
    e2 = np.zeros(chunk_n, np.float32)
    lib().orc_reduce_chunk(P, chunk_n, _ptr_array(shard_codes), _ptr_array(shard_scales),
                           _p(codes2), _p(scales2), _p(y), _p(e2), bits)
    return codes2, scales2, y, e2


def decode(codes, scales, n: int, bits: int = 4) -> np.ndarray:
    y = np.zeros(n, np.uint16)
    lib().orc_decode(n, _p(codes), _p(scales), _p(y), bits)
    return y


def update(x, m_fast, m_slow, codes1, scales1, e2_own, nranks: int, rank: int,
           want_r: bool = False, bits: int = 4):
    """Refresh the averages in place; optionally return r."""
    r = np.zeros(x.size, np.float32) if want_r else None
    lib().orc_update(x.size, nranks, rank, _p(x), _p(m_fast), _p(m_slow), _p(codes1),
                     _p(scales1), _p(e2_own), _p(r), bits)
    return r


def correction(m_fast, m_slow) -> np.ndarray:
    """corr = (W_F m_fast) + (W_S m_slow), elementwise in binary32."""
    corr = np.zeros(m_fast.size, np.float32)
    lib().orc_correction(m_fast.size, _p(m_fast), _p(m_slow), _p(corr))
    return corr


def encode_corr(x, corr, bits: int = 4):
    """Entry pass from a correction array. Returns (codes, scales)."""
    n = x.size
    codes = np.zeros(code_bytes(n, bits), np.uint8)
    scales = np.zeros(n // GROUP, np.float32)
    lib().orc_encode_corr(n, _p(x), _p(np.ascontiguousarray(corr, np.float32)), _p(codes),
                          _p(scales), bits)
    return codes, scales


def update_corr(x, m_fast, m_slow, codes1, scales1, e2_own, corr, nranks: int, rank: int,
                bits: int = 4) -> None:
    """Refresh the averages in place, then write the next call's correction into corr."""
    lib().orc_update_corr(x.size, nranks, rank, _p(x), _p(m_fast), _p(m_slow), _p(codes1),
                          _p(scales1), _p(e2_own), _p(corr), bits)


def call(nranks: int, rank: int, x, m_fast, m_slow, recv_codes, recv_scales,
         gath_codes, gath_scales, comp: bool = True, bits: int = 4, threads: int = 1, out=None):
    """Rank-mode call. recv_*/gath_* are lists of P arrays (slot `rank` may be
    None).  Updates m_fast/m_slow in place.  Returns a dict of outputs.

    threads > 1 runs the threaded driver (orc_call_mt: the same step
    functions on disjoint runs of groups, bit-identical outputs).  `out`, a
    dict returned by an earlier call of the same shape, is reused for the
    outputs instead of fresh arrays."""
    n = x.size
    Cn = n // nranks
    if out is None:
        out = dict(send_codes=np.zeros(code_bytes(n, bits), np.uint8),
                   send_scales=np.zeros(n // GROUP, np.float32),
                   own_codes2=np.zeros(code_bytes(Cn, bits), np.uint8),
                   own_scales2=np.zeros(Cn // GROUP, np.float32),
                   y=np.zeros(n, np.uint16))
    send_codes, send_scales = out["send_codes"], out["send_scales"]
    own_codes2, own_scales2, y = out["own_codes2"], out["own_scales2"], out["y"]
    args = (nranks, rank, n, _p(x), _p(m_fast), _p(m_slow),
            _ptr_array(recv_codes), _ptr_array(recv_scales),
            _ptr_array(gath_codes), _ptr_array(gath_scales),
            _p(send_codes), _p(send_scales), _p(own_codes2), _p(own_scales2),
            _p(y), int(bool(comp)), bits)
    rc = lib().orc_call_mt(int(threads), *args) if threads > 1 else lib().orc_call(*args)
    if rc != 0:
        raise ValueError("orc_call rejected its arguments")
    return out


def simulate(xs, m_fast=None, m_slow=None, comp: bool = True, want_detail: bool = False,
             bits: int = 4):
    """One call with all P ranks simulated.  xs: list of P uint16 arrays;
    m_fast/m_slow: lists of P float32 arrays updated in place (ignored when
    comp is False).  Returns dict(codes2, scales2, y[, codes1, scales1, xp, r])."""
    P = len(xs)
    n = xs[0].size
    codes2 = np.zeros(code_bytes(n, bits), np.uint8)
    scales2 = np.zeros(n // GROUP, np.float32)
    y = np.zeros(n, np.uint16)
    det = None
    if want_detail:
        det = dict(codes1=[np.zeros(code_bytes(n, bits), np.uint8) for _ in range(P)],
                   scales1=[np.zeros(n // GROUP, np.float32) for _ in range(P)],
                   xp=[np.zeros(n, np.float32) for _ in range(P)],
                   r=[np.zeros(n, np.float32) for _ in range(P)])
    rc = lib().orc_simulate(
        P, n, _ptr_array(xs),
        _ptr_array(m_fast) if comp else None, _ptr_array(m_slow) if comp else None,
        _p(codes2), _p(scales2), _p(y),
        _ptr_array(det["codes1"]) if det else None, _ptr_array(det["scales1"]) if det else None,
        _ptr_array(det["xp"]) if det else None, _ptr_array(det["r"]) if det else None,
        int(bool(comp)), bits)
    if rc != 0:
        raise ValueError("orc_simulate rejected its arguments")
    out = dict(codes2=codes2, scales2=scales2, y=y)
    if det:
        out.update(det)
    return out


# ---- reduce-scatter only ----------------------------------------------------------

def reduce_chunk_sum(shard_codes, shard_scales, chunk_n: int, bits: int = 4):
    """Rank-order sum of P shards output as bf16. Returns (y_bf16, e)."""
    y = np.zeros(chunk_n, np.uint16)
    e = np.zeros(chunk_n, np.float32)
    lib().orc_reduce_chunk_sum(len(shard_codes), chunk_n, _ptr_array(shard_codes),
                               _ptr_array(shard_scales), _p(y), _p(e), bits)
    return y, e


def rs_call(nranks: int, rank: int, x, m_fast, m_slow, recv_codes, recv_scales, comp: bool = True,
            bits: int = 4, threads: int = 1):
    """Rank-mode reduce-scatter call.  Returns dict(send_codes, send_scales, y_own).
    threads > 1 runs the threaded driver (bit-identical outputs)."""
    n = x.size
    Cn = n // nranks
    send_codes = np.zeros(code_bytes(n, bits), np.uint8)
    send_scales = np.zeros(n // GROUP, np.float32)
    y_own = np.zeros(Cn, np.uint16)
    args = (nranks, rank, n, _p(x), _p(m_fast), _p(m_slow), _ptr_array(recv_codes),
            _ptr_array(recv_scales), _p(send_codes), _p(send_scales), _p(y_own),
            int(bool(comp)), bits)
    rc = lib().orc_rs_call_mt(int(threads), *args) if threads > 1 else lib().orc_rs_call(*args)
    if rc != 0:
        raise ValueError("orc_rs_call rejected its arguments")
    return dict(send_codes=send_codes, send_scales=send_scales, y_own=y_own)


def rs_simulate(xs, m_fast=None, m_slow=None, comp: bool = True, want_detail: bool = False,
                bits: int = 4):
    """All P ranks' reduce-scatter call: y[n] holds chunk j as reduced by rank j."""
    P = len(xs)
    n = xs[0].size
    y = np.zeros(n, np.uint16)
    det = None
    if want_detail:
        det = dict(xp=[np.zeros(n, np.float32) for _ in range(P)],
                   r=[np.zeros(n, np.float32) for _ in range(P)])
    rc = lib().orc_rs_simulate(P, n, _ptr_array(xs), _ptr_array(m_fast) if comp else None,
                               _ptr_array(m_slow) if comp else None, _p(y),
                               _ptr_array(det["xp"]) if det else None,
                               _ptr_array(det["r"]) if det else None, int(bool(comp)), bits)
    if rc != 0:
        raise ValueError("orc_rs_simulate rejected its arguments")
    out = dict(y=y)
    if det:
        out.update(det)
    return out
