"""Thin Python binding of libecho (include/echo.h).

Argument marshalling only: every step of the pipeline runs in the HIP
kernels of libecho.so.  PyTorch provides device memory and streams: tensors
are passed by address, the stream defaults to torch's current stream.
Tensor arguments are checked on the host before the call (on the GPU,
contiguous, at least the bytes the call reads or writes); plain integer
addresses are passed through unchecked.

Functions keep the C names (echo_state_init, echo_encode, ...) and raise
EchoError on a non-zero status.  There is no fallback: if libecho.so is
missing the import fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os

import torch  # load torch's HIP runtime first: libecho binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libecho.so")

GROUP = 128
MAX_RANKS = 16


class EchoError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


class EchoStateC(C.Structure):
    _fields_ = [("m_fast", C.c_void_p), ("m_slow", C.c_void_p), ("n", C.c_int64),
                ("nranks", C.c_int32), ("rank", C.c_int32), ("bits", C.c_int32),
                ("reserved", C.c_int32)]


class EchoConfigC(C.Structure):
    _fields_ = [("abi_version", C.c_int32), ("group", C.c_int32), ("qmax", C.c_int32),
                ("qmax8", C.c_int32), ("max_ranks", C.c_int32), ("w_fast", C.c_float), ("w_slow", C.c_float),
                ("beta_fast", C.c_float), ("alpha_fast", C.c_float), ("beta_slow", C.c_float),
                ("alpha_slow", C.c_float), ("max_elements", C.c_int64)]


_vp = C.c_void_p
_pp = C.POINTER(C.c_void_p)
_SIGNATURES = {
    "echo_state_init": [C.POINTER(EchoStateC), _vp, _vp, C.c_int64, C.c_int32, C.c_int32, _vp],
    "echo_encode": [C.POINTER(EchoStateC), _vp, _vp, _vp, _vp],
    "echo_reduce_shard": [C.c_int32, C.c_int64, C.c_int32, _pp, _pp, _vp, _vp, _vp, _vp, _vp],
    "echo_decode": [C.c_int64, C.c_int32, _vp, _vp, _vp, _vp],
    "echo_update": [C.POINTER(EchoStateC), _vp, _vp, _vp, _vp, _vp],
    "echo_correction": [C.POINTER(EchoStateC), _vp, _vp],
    "echo_encode_corr": [C.POINTER(EchoStateC), _vp, _vp, _vp, _vp, _vp],
    "echo_update_corr": [C.POINTER(EchoStateC), _vp, _vp, _vp, _vp, _vp, _vp],
    "echo_call_entry": [C.POINTER(EchoStateC), _vp, _vp, _vp, _vp],
    "echo_call_entry_range": [C.POINTER(EchoStateC), _vp, C.c_int32, C.c_int32, _vp, _vp, _vp],
    "echo_call_reduce": [C.POINTER(EchoStateC), _vp, _pp, _pp, _vp, _vp, _vp, _vp],
    "echo_call_exit": [C.POINTER(EchoStateC), _pp, _pp, _vp, _vp],
    "echo_call": [C.POINTER(EchoStateC), _vp, _pp, _pp, _pp, _pp, _vp, _vp, _vp, _vp, _vp, _vp],
    "echo_call_plain": [C.c_int32, C.c_int32, C.c_int64, C.c_int32, _vp, _pp, _pp, _pp, _pp, _vp,
                        _vp, _vp, _vp, _vp, _vp],
    "echo_reduce_shard_sum": [C.c_int32, C.c_int64, C.c_int32, _pp, _pp, _vp, _vp, _vp],
    "echo_rs_reduce": [C.POINTER(EchoStateC), _vp, _pp, _pp, _vp, _vp],
    "echo_rs_call": [C.POINTER(EchoStateC), _vp, _pp, _pp, _vp, _vp, _vp, _vp],
    "echo_stream_copy": [_vp, _vp, C.c_int64, _vp],
    "echo_get_config": [C.POINTER(EchoConfigC)],
    "echo_status_string": [C.c_int],
    "echo_version": [],
}
EXPORTED = tuple(_SIGNATURES)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libecho.so not built at {LIB_PATH}; run __graft_entry__.build()")
    lib = C.CDLL(LIB_PATH)
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = C.c_char_p if name == "echo_status_string" else C.c_int
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.echo_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise EchoError(status, where)


def _cb(n: int, bits: int) -> int:
    """bytes of the codes of n elements"""
    return n if bits == 8 else n // 2


def _sb(n: int) -> int:
    """bytes of the scales of n elements"""
    return (n // GROUP) * 4


def _ptr(t, nbytes: int = 0, what: str = "buffer"):
    """Device address of a tensor (None -> NULL; plain ints pass through
    unchecked).  A tensor must live on the GPU, be contiguous and hold at
    least nbytes: the library cannot see a host pointer or the end of a
    buffer, and a kernel given either would fault."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{what}: a GPU tensor is required (got one on {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{what}: the tensor must be contiguous")
    if t.nbytes < nbytes:
        raise ValueError(f"{what}: holds {t.nbytes} bytes, the call needs {nbytes}")
    return t.data_ptr()


_PTR16 = C.c_void_p * MAX_RANKS


def _ptrs(ts, nbytes: int = 0, what: str = "buffers"):
    """void*[>= MAX_RANKS] of device addresses: entries past the list are NULL,
    which the library rejects instead of reading past the array."""
    vals = [_ptr(t, nbytes, f"{what}[{i}]") for i, t in enumerate(ts)]
    if len(vals) <= MAX_RANKS:
        return _PTR16(*vals)
    return (C.c_void_p * len(vals))(*vals)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class EchoState:
    """Compensator state of one call sequence: two float32 averages of n
    elements (caller-owned tensors), P ranks, this rank, and the code width of
    the next call's messages (`bits`, 4 or 8; may change from call to call)."""

    def __init__(self, m_fast: torch.Tensor, m_slow: torch.Tensor, n: int, nranks: int, rank: int,
                 bits: int = 4):
        self.m_fast, self.m_slow = m_fast, m_slow  # keep the buffers alive
        self.c = EchoStateC(_ptr(m_fast, 4 * int(n), "m_fast"), _ptr(m_slow, 4 * int(n), "m_slow"),
                            int(n), int(nranks), int(rank), int(bits), 0)

    @property
    def bits(self) -> int:
        return self.c.bits

    @bits.setter
    def bits(self, value: int) -> None:
        self.c.bits = int(value)

    @property
    def n(self) -> int:
        return self.c.n

    @property
    def nranks(self) -> int:
        return self.c.nranks

    @property
    def rank(self) -> int:
        return self.c.rank

    def sizes(self):
        """(n, chunk, bits) of this state's calls"""
        n, P = self.c.n, self.c.nranks
        return n, (n // P if P > 0 else 0), self.c.bits


def echo_state_init(m_fast, m_slow, n, nranks, rank, stream=None, bits: int = 4) -> EchoState:
    st = EchoState(m_fast, m_slow, n, nranks, rank)
    _check(lib.echo_state_init(C.byref(st.c), st.c.m_fast, st.c.m_slow, int(n), int(nranks),
                               int(rank), _stream(stream)), "echo_state_init")
    st.bits = bits
    return st


def echo_encode(st: EchoState, x, codes, scales, stream=None) -> None:
    n, _, bits = st.sizes()
    _check(lib.echo_encode(C.byref(st.c), _ptr(x, 2 * n, "x"), _ptr(codes, _cb(n, bits), "codes"),
                           _ptr(scales, _sb(n), "scales"), _stream(stream)), "echo_encode")


def echo_reduce_shard(shard_codes, shard_scales, out_codes, out_scales, out_y=None, out_e2=None,
                      chunk_n=None, stream=None, bits: int = 4) -> None:
    P = len(shard_codes)
    if chunk_n is None:
        chunk_n = out_codes.numel() * (1 if bits == 8 else 2)
    cn = int(chunk_n)
    _check(lib.echo_reduce_shard(P, cn, int(bits), _ptrs(shard_codes, _cb(cn, bits), "shard_codes"),
                                 _ptrs(shard_scales, _sb(cn), "shard_scales"),
                                 _ptr(out_codes, _cb(cn, bits), "out_codes"),
                                 _ptr(out_scales, _sb(cn), "out_scales"), _ptr(out_y, 2 * cn, "out_y"),
                                 _ptr(out_e2, 4 * cn, "out_e2"), _stream(stream)), "echo_reduce_shard")


def echo_decode(codes, scales, y, n=None, stream=None, bits: int = 4) -> None:
    if n is None:
        n = y.numel()
    n = int(n)
    _check(lib.echo_decode(n, int(bits), _ptr(codes, _cb(n, bits), "codes"), _ptr(scales, _sb(n), "scales"),
                           _ptr(y, 2 * n, "y"), _stream(stream)), "echo_decode")


def echo_stream_copy(src, dst, nbytes=None, stream=None) -> None:
    """Plain streaming copy (the bandwidth ceiling the kernels are measured
    against); nbytes defaults to dst's size in bytes."""
    if nbytes is None:
        nbytes = dst.numel() * dst.element_size()
    nb = int(nbytes)
    _check(lib.echo_stream_copy(_ptr(src, nb, "src"), _ptr(dst, nb, "dst"), nb, _stream(stream)),
           "echo_stream_copy")


def echo_update(st: EchoState, x, codes1, scales1, e2_own, stream=None) -> None:
    n, cn, bits = st.sizes()
    _check(lib.echo_update(C.byref(st.c), _ptr(x, 2 * n, "x"), _ptr(codes1, _cb(n, bits), "codes1"),
                           _ptr(scales1, _sb(n), "scales1"), _ptr(e2_own, 4 * cn, "e2_own"),
                           _stream(stream)), "echo_update")


def echo_correction(st: EchoState, corr, stream=None) -> None:
    n, _, _ = st.sizes()
    _check(lib.echo_correction(C.byref(st.c), _ptr(corr, 4 * n, "corr"), _stream(stream)),
           "echo_correction")


def echo_encode_corr(st: EchoState, x, corr, codes, scales, stream=None) -> None:
    n, _, bits = st.sizes()
    _check(lib.echo_encode_corr(C.byref(st.c), _ptr(x, 2 * n, "x"), _ptr(corr, 4 * n, "corr"),
                                _ptr(codes, _cb(n, bits), "codes"), _ptr(scales, _sb(n), "scales"),
                                _stream(stream)), "echo_encode_corr")


def echo_update_corr(st: EchoState, x, codes1, scales1, e2_own, corr, stream=None) -> None:
    n, cn, bits = st.sizes()
    _check(lib.echo_update_corr(C.byref(st.c), _ptr(x, 2 * n, "x"), _ptr(codes1, _cb(n, bits), "codes1"),
                                _ptr(scales1, _sb(n), "scales1"), _ptr(e2_own, 4 * cn, "e2_own"),
                                _ptr(corr, 4 * n, "corr"), _stream(stream)), "echo_update_corr")


def echo_call_entry(st: EchoState, x, send_codes, send_scales, stream=None) -> None:
    n, _, bits = st.sizes()
    _check(lib.echo_call_entry(C.byref(st.c), _ptr(x, 2 * n, "x"), _ptr(send_codes, _cb(n, bits), "send_codes"),
                               _ptr(send_scales, _sb(n), "send_scales"), _stream(stream)), "echo_call_entry")


def echo_call_entry_range(st: EchoState, x, chunk_begin, chunk_end, send_codes, send_scales,
                          stream=None) -> None:
    n, _, bits = st.sizes()
    _check(lib.echo_call_entry_range(C.byref(st.c), _ptr(x, 2 * n, "x"), int(chunk_begin), int(chunk_end),
                                     _ptr(send_codes, _cb(n, bits), "send_codes"),
                                     _ptr(send_scales, _sb(n), "send_scales"), _stream(stream)),
           "echo_call_entry_range")


def echo_call_reduce(st: EchoState, x, recv_codes, recv_scales, own_codes2, own_scales2, y,
                     stream=None) -> None:
    n, cn, bits = st.sizes()
    _check(lib.echo_call_reduce(C.byref(st.c), _ptr(x, 2 * n, "x"),
                                _ptrs(recv_codes, _cb(cn, bits), "recv_codes"),
                                _ptrs(recv_scales, _sb(cn), "recv_scales"),
                                _ptr(own_codes2, _cb(cn, bits), "own_codes2"),
                                _ptr(own_scales2, _sb(cn), "own_scales2"), _ptr(y, 2 * n, "y"),
                                _stream(stream)), "echo_call_reduce")


def echo_call_exit(st: EchoState, gath_codes, gath_scales, y, stream=None) -> None:
    n, cn, bits = st.sizes()
    _check(lib.echo_call_exit(C.byref(st.c), _ptrs(gath_codes, _cb(cn, bits), "gath_codes"),
                              _ptrs(gath_scales, _sb(cn), "gath_scales"), _ptr(y, 2 * n, "y"),
                              _stream(stream)), "echo_call_exit")


def _call_args(n, cn, bits, x, recv_codes, recv_scales, gath_codes, gath_scales, send_codes,
               send_scales, own_codes2, own_scales2, y):
    """checked addresses of one call's buffers (n elements, chunk cn, bits)"""
    return (_ptr(x, 2 * n, "x"), _ptrs(recv_codes, _cb(cn, bits), "recv_codes"),
            _ptrs(recv_scales, _sb(cn), "recv_scales"), _ptrs(gath_codes, _cb(cn, bits), "gath_codes"),
            _ptrs(gath_scales, _sb(cn), "gath_scales"), _ptr(send_codes, _cb(n, bits), "send_codes"),
            _ptr(send_scales, _sb(n), "send_scales"), _ptr(own_codes2, _cb(cn, bits), "own_codes2"),
            _ptr(own_scales2, _sb(cn), "own_scales2"), _ptr(y, 2 * n, "y"))


def echo_call(st: EchoState, x, recv_codes, recv_scales, gath_codes, gath_scales, send_codes,
              send_scales, own_codes2, own_scales2, y, stream=None) -> None:
    _check(lib.echo_call(C.byref(st.c), *_call_args(*st.sizes(), x, recv_codes, recv_scales, gath_codes,
                                                    gath_scales, send_codes, send_scales, own_codes2,
                                                    own_scales2, y), _stream(stream)), "echo_call")


def echo_call_plain(nranks, rank, x, recv_codes, recv_scales, gath_codes, gath_scales,
                    send_codes, send_scales, own_codes2, own_scales2, y, n=None,
                    stream=None, bits: int = 4) -> None:
    if n is None:
        n = x.numel()
    n, P = int(n), int(nranks)
    cn = n // P if P > 0 else 0
    _check(lib.echo_call_plain(P, int(rank), n, int(bits),
                               *_call_args(n, cn, int(bits), x, recv_codes, recv_scales, gath_codes,
                                           gath_scales, send_codes, send_scales, own_codes2,
                                           own_scales2, y), _stream(stream)), "echo_call_plain")


def echo_reduce_shard_sum(shard_codes, shard_scales, out_y, out_e2=None, chunk_n=None,
                          stream=None, bits: int = 4) -> None:
    if chunk_n is None:
        chunk_n = out_y.numel()
    cn = int(chunk_n)
    _check(lib.echo_reduce_shard_sum(len(shard_codes), cn, int(bits),
                                     _ptrs(shard_codes, _cb(cn, bits), "shard_codes"),
                                     _ptrs(shard_scales, _sb(cn), "shard_scales"),
                                     _ptr(out_y, 2 * cn, "out_y"), _ptr(out_e2, 4 * cn, "out_e2"),
                                     _stream(stream)), "echo_reduce_shard_sum")


def echo_rs_reduce(st: EchoState, x, recv_codes, recv_scales, y_own, stream=None) -> None:
    n, cn, bits = st.sizes()
    _check(lib.echo_rs_reduce(C.byref(st.c), _ptr(x, 2 * n, "x"),
                              _ptrs(recv_codes, _cb(cn, bits), "recv_codes"),
                              _ptrs(recv_scales, _sb(cn), "recv_scales"), _ptr(y_own, 2 * cn, "y_own"),
                              _stream(stream)), "echo_rs_reduce")


def echo_rs_call(st: EchoState, x, recv_codes, recv_scales, send_codes, send_scales, y_own,
                 stream=None) -> None:
    n, cn, bits = st.sizes()
    _check(lib.echo_rs_call(C.byref(st.c), _ptr(x, 2 * n, "x"),
                            _ptrs(recv_codes, _cb(cn, bits), "recv_codes"),
                            _ptrs(recv_scales, _sb(cn), "recv_scales"),
                            _ptr(send_codes, _cb(n, bits), "send_codes"),
                            _ptr(send_scales, _sb(n), "send_scales"), _ptr(y_own, 2 * cn, "y_own"),
                            _stream(stream)), "echo_rs_call")


class PreparedCall:
    """echo_call with every argument marshalled once: for loops that call the
    pipeline again and again on the same buffers (a serving loop's per-layer
    buffers).  Calling it enqueues the call on `stream` (default: torch's
    current stream).  The tensors are kept alive by this object; their
    contents may change between calls, their storage may not.

    The buffer sizes were checked for the state as it was when the call was
    prepared (its n, P, rank and code width).  The library is handed a copy
    of that state, and a call made after the EchoState changed (say, its
    `bits` set from 4 to 8) raises instead of launching: the buffers may be
    too small for the new width."""

    def __init__(self, st: EchoState, x, recv_codes, recv_scales, gath_codes, gath_scales,
                 send_codes, send_scales, own_codes2, own_scales2, y):
        self._keep = (st, x, recv_codes, recv_scales, gath_codes, gath_scales, send_codes,
                      send_scales, own_codes2, own_scales2, y)
        self._st = st
        self._snap = EchoStateC.from_buffer_copy(st.c)
        self._args = (C.byref(self._snap), *_call_args(*st.sizes(), x, recv_codes, recv_scales,
                                                       gath_codes, gath_scales, send_codes, send_scales,
                                                       own_codes2, own_scales2, y))
        self._fn = lib.echo_call

    def __call__(self, stream=None) -> None:
        if bytes(self._st.c) != bytes(self._snap):
            raise ValueError("echo_call: the state changed since the call was prepared "
                             f"(bits {self._snap.bits} -> {self._st.c.bits}); prepare it again")
        rc = self._fn(*self._args, _stream(stream))
        if rc != 0:
            raise EchoError(rc, "echo_call")


def echo_call_prepare(st: EchoState, x, recv_codes, recv_scales, gath_codes, gath_scales,
                      send_codes, send_scales, own_codes2, own_scales2, y) -> PreparedCall:
    """A reusable echo_call on fixed buffers (see PreparedCall)."""
    return PreparedCall(st, x, recv_codes, recv_scales, gath_codes, gath_scales, send_codes,
                        send_scales, own_codes2, own_scales2, y)


def echo_get_config() -> dict:
    cfg = EchoConfigC()
    _check(lib.echo_get_config(C.byref(cfg)), "echo_get_config")
    return {name: getattr(cfg, name) for name, _ in EchoConfigC._fields_}


def echo_version() -> int:
    return int(lib.echo_version())
