"""C-ABI checks that need no GPU: the library loads, exports every function
include/echo.h declares, reports the same named parameters the oracle
restates independently, and rejects bad arguments before launching anything
(every call below fails validation, so no kernel is enqueued)."""
import ctypes as C
import os
import re

import pytest

from error_compensated_bit_echo_amd import binding as B
from oracle import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "echo.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(echo_\w+)\s*\(", src, re.M)))


def test_header_declares_the_calls():
    names = declared_functions()
    for want in ("echo_state_init", "echo_encode", "echo_reduce_shard", "echo_decode",
                 "echo_update", "echo_call", "echo_call_entry", "echo_call_reduce",
                 "echo_call_exit", "echo_call_entry_range", "echo_call_plain", "echo_reduce_shard_sum",
                 "echo_rs_reduce",
                 "echo_rs_call", "echo_stream_copy", "echo_get_config", "echo_status_string",
                 "echo_version", "echo_correction", "echo_encode_corr", "echo_update_corr"):
        assert want in names


def test_library_exports_every_declared_symbol():
    raw = C.CDLL(B.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert set(declared_functions()) == set(B.EXPORTED)


def test_config_matches_oracle_constants():
    cfg = B.echo_get_config()
    assert cfg["abi_version"] == B.echo_version() == 3
    assert cfg["qmax8"] == orc.QMAX8 == 127
    assert cfg["group"] == orc.GROUP == 128
    assert cfg["qmax"] == orc.QMAX
    assert cfg["max_ranks"] == orc.MAX_RANKS
    assert cfg["w_fast"] == orc.W_FAST and cfg["w_slow"] == orc.W_SLOW
    assert cfg["beta_fast"] == orc.BETA_FAST and cfg["alpha_fast"] == orc.ALPHA_FAST
    assert cfg["beta_slow"] == orc.BETA_SLOW and cfg["alpha_slow"] == orc.ALPHA_SLOW
    # the averages are normalized: B + A = 1, and the correction weights sum to 1
    assert cfg["beta_fast"] + cfg["alpha_fast"] == 1.0
    assert cfg["beta_slow"] + cfg["alpha_slow"] == 1.0
    assert cfg["w_fast"] + cfg["w_slow"] == 1.0


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert B.status_string(code) and B.status_string(code) != "unknown status"
    assert B.status_string(-99) == "unknown status"


# Fake, well-aligned device addresses: never dereferenced, because every call
# below is rejected by the host-side checks.
A = 1 << 32


def st(n=1024, P=2, rank=0, mf=A, ms=2 * A):
    return B.EchoState(mf, ms, n, P, rank)


def rc(fn, *args, **kw):
    with pytest.raises(B.EchoError) as e:
        fn(*args, stream=0, **kw)  # an explicit null stream: no GPU is touched
    return e.value.status


def test_state_init_rejections():
    L = B.lib
    s = B.EchoStateC()
    assert L.echo_state_init(None, A, 2 * A, 1024, 2, 0, None) == -1
    assert L.echo_state_init(C.byref(s), None, 2 * A, 1024, 2, 0, None) == -1
    assert L.echo_state_init(C.byref(s), A, 2 * A, 1000, 2, 0, None) == -2
    assert L.echo_state_init(C.byref(s), A, 2 * A, -1024, 2, 0, None) == -2
    assert L.echo_state_init(C.byref(s), A, 2 * A, 128, 2, 0, None) == -2   # n % (P*128)
    assert L.echo_state_init(C.byref(s), A, 2 * A, 1024, 0, 0, None) == -4
    assert L.echo_state_init(C.byref(s), A, 2 * A, 1024 * 17, 17, 0, None) == -4
    assert L.echo_state_init(C.byref(s), A, 2 * A, 1024, 2, 2, None) == -4
    assert L.echo_state_init(C.byref(s), A, 2 * A, 1024, 2, -1, None) == -4
    assert L.echo_state_init(C.byref(s), A + 4, 2 * A, 1024, 2, 0, None) == -3
    assert L.echo_state_init(C.byref(s), A, A + 1024, 1024, 2, 0, None) == -6  # overlap
    assert L.echo_state_init(C.byref(s), A, 2 * A, (1 << 37) + 256, 2, 0, None) == -2


def test_encode_rejections():
    assert rc(B.echo_encode, st(), None, 3 * A, 4 * A) == -1
    assert rc(B.echo_encode, st(), 3 * A + 2, 4 * A, 5 * A) == -3
    assert rc(B.echo_encode, st(), 3 * A, 4 * A + 8, 5 * A) == -3
    assert rc(B.echo_encode, st(), 3 * A, 4 * A, 5 * A + 2) == -3
    assert rc(B.echo_encode, st(n=1000), 3 * A, 4 * A, 5 * A) == -2
    assert rc(B.echo_encode, st(rank=5), 3 * A, 4 * A, 5 * A) == -4
    # codes overlapping x, scales overlapping the averages
    assert rc(B.echo_encode, st(), 3 * A, 3 * A + 16, 5 * A) == -6
    assert rc(B.echo_encode, st(), 3 * A, 4 * A, A + 64) == -6


def test_reduce_shard_rejections():
    c = [3 * A, 4 * A]
    s = [5 * A, 6 * A]
    assert rc(B.echo_reduce_shard, c, s, 7 * A, 8 * A, None, None, 100) == -2
    assert rc(B.echo_reduce_shard, [3 * A, None], s, 7 * A, 8 * A, None, None, 256) == -1
    assert rc(B.echo_reduce_shard, [3 * A, 4 * A + 2], s, 7 * A, 8 * A, None, None, 256) == -3
    assert rc(B.echo_reduce_shard, c, s, 7 * A, 8 * A, 9 * A + 2, None, 256) == -3
    assert rc(B.echo_reduce_shard, c, s, 3 * A, 8 * A, None, None, 256) == -6  # out over shard
    assert rc(B.echo_reduce_shard, c, s, 7 * A, 7 * A + 64, None, None, 256) == -6
    assert rc(B.echo_reduce_shard, [3 * A] * 17, [5 * A] * 17, 7 * A, 8 * A, None, None, 256) == -4


def test_decode_update_rejections():
    assert rc(B.echo_decode, 3 * A, 4 * A, 5 * A, 100) == -2
    assert rc(B.echo_decode, 3 * A, 4 * A, None, 128) == -1
    assert rc(B.echo_decode, 3 * A, 4 * A, 3 * A, 128) == -6
    assert rc(B.echo_update, st(), 3 * A, 4 * A, 5 * A, None) == -1
    assert rc(B.echo_update, st(), 3 * A, 4 * A, 5 * A, 6 * A + 4) == -3
    assert rc(B.echo_update, st(), A + 64, 4 * A, 5 * A, 6 * A) == -6  # x over m_fast


def test_call_rejections():
    P, n = 4, 4096
    s4 = st(n=n, P=P, rank=1)
    recv_c = [10 * A + k * A for k in range(P)]
    recv_s = [20 * A + k * A for k in range(P)]
    gath_c = [30 * A + k * A for k in range(P)]
    gath_s = [40 * A + k * A for k in range(P)]
    outs = [50 * A, 51 * A, 52 * A, 53 * A, 54 * A]
    # slot `rank` may be NULL, the others may not
    bad = list(recv_c)
    bad[2] = None
    assert rc(B.echo_call, s4, 3 * A, bad, recv_s, gath_c, gath_s, *outs) == -1
    bad = list(gath_s)
    bad[0] = 40 * A + 2
    assert rc(B.echo_call, s4, 3 * A, recv_c, recv_s, gath_c, bad, *outs) == -3
    # y may alias x exactly, but not partially; send may not overlap a gathered chunk
    assert rc(B.echo_call, s4, 3 * A, recv_c, recv_s, gath_c, gath_s, 50 * A, 51 * A, 52 * A,
              53 * A, 3 * A + 16) == -6
    assert rc(B.echo_call, s4, 3 * A, recv_c, recv_s, gath_c, gath_s, 30 * A, 51 * A, 52 * A,
              53 * A, 54 * A) == -6
    assert rc(B.echo_call_reduce, s4, 3 * A, recv_c, recv_s, 52 * A, 53 * A, None) == -1
    assert rc(B.echo_call_exit, s4, gath_c, gath_s, A) == -6  # y over m_fast
    assert rc(B.echo_call_entry, st(n=n, P=P, rank=4), 3 * A, 50 * A, 51 * A) == -4


def test_call_plain_rejections():
    P, n = 4, 4096
    recv_c = [10 * A + k * A for k in range(P)]
    recv_s = [20 * A + k * A for k in range(P)]
    gath_c = [30 * A + k * A for k in range(P)]
    gath_s = [40 * A + k * A for k in range(P)]
    outs = [50 * A, 51 * A, 52 * A, 53 * A, 54 * A]
    assert rc(B.echo_call_plain, P, 4, 3 * A, recv_c, recv_s, gath_c, gath_s, *outs, n) == -4
    assert rc(B.echo_call_plain, 0, 0, 3 * A, recv_c, recv_s, gath_c, gath_s, *outs, n) == -4
    assert rc(B.echo_call_plain, P, 1, 3 * A, recv_c, recv_s, gath_c, gath_s, *outs, 1000) == -2
    assert rc(B.echo_call_plain, P, 1, 3 * A + 8, recv_c, recv_s, gath_c, gath_s, *outs, n) == -3
    bad = list(recv_c)
    bad[3] = None
    assert rc(B.echo_call_plain, P, 1, 3 * A, bad, recv_s, gath_c, gath_s, *outs, n) == -1
    assert rc(B.echo_call_plain, P, 1, 3 * A, recv_c, recv_s, gath_c, gath_s, 50 * A, 51 * A,
              52 * A, 53 * A, 3 * A + 32, n) == -6


def test_reduce_scatter_rejections():
    P, n = 4, 4096
    s4 = st(n=n, P=P, rank=2)
    recv_c = [10 * A + k * A for k in range(P)]
    recv_s = [20 * A + k * A for k in range(P)]
    assert rc(B.echo_reduce_shard_sum, [3 * A, 4 * A], [5 * A, 6 * A], 7 * A, None, 100) == -2
    assert rc(B.echo_reduce_shard_sum, [3 * A, 4 * A], [5 * A, 6 * A], 4 * A, None, 256) == -6
    assert rc(B.echo_rs_reduce, s4, 3 * A, recv_c, recv_s, None) == -1
    assert rc(B.echo_rs_reduce, s4, 3 * A, recv_c, recv_s, 3 * A + 4096) == -6  # y_own inside x
    assert rc(B.echo_rs_call, s4, 3 * A, recv_c, recv_s, 50 * A, 51 * A, 52 * A + 2) == -3
    assert rc(B.echo_rs_call, s4, 3 * A, recv_c, recv_s, 50 * A, 51 * A, A) == -6  # y_own over m_fast


def test_code_width_rejections():
    s8 = st()
    s8.bits = 5
    assert rc(B.echo_encode, s8, 3 * A, 4 * A, 5 * A) == -7
    assert rc(B.echo_decode, 3 * A, 4 * A, 5 * A, 128, bits=6) == -7
    assert rc(B.echo_reduce_shard, [3 * A], [5 * A], 7 * A, 8 * A, None, None, 256, bits=2) == -7
    assert rc(B.echo_reduce_shard_sum, [3 * A], [5 * A], 7 * A, None, 256, bits=16) == -7
    # 8-bit codes take n bytes: codes ending 496 bytes before x in 4-bit form
    # (n/2 = 512 bytes from x - 1008) reach 16 bytes into x in 8-bit form
    s8.bits = 8
    assert rc(B.echo_encode, s8, 3 * A, 3 * A - 1008, 5 * A) == -6


def test_empty_calls_are_noops():
    """n == 0 (chunk_n == 0): scalar arguments are checked, pointers are not
    looked at, nothing is launched (so no GPU is touched here), success."""
    L = B.lib
    s = B.EchoStateC()
    assert L.echo_state_init(C.byref(s), None, None, 0, 8, 3, None) == 0
    assert (s.n, s.nranks, s.rank, s.bits) == (0, 8, 3, 4)
    assert L.echo_state_init(C.byref(s), None, None, 0, 8, 8, None) == -4
    assert L.echo_state_init(C.byref(s), None, None, 0, 17, 0, None) == -4
    assert L.echo_state_init(None, None, None, 0, 8, 0, None) == -1
    e = B.EchoState(None, None, 0, 8, 3)
    nulls = [None] * 8
    B.echo_encode(e, None, None, None, stream=0)
    B.echo_update(e, None, None, None, None, stream=0)
    B.echo_call_entry(e, None, None, None, stream=0)
    B.echo_call_reduce(e, None, nulls, nulls, None, None, None, stream=0)
    B.echo_call_exit(e, nulls, nulls, None, stream=0)
    B.echo_call(e, None, nulls, nulls, nulls, nulls, None, None, None, None, None, stream=0)
    B.echo_rs_reduce(e, None, nulls, nulls, None, stream=0)
    B.echo_rs_call(e, None, nulls, nulls, None, None, None, stream=0)
    B.echo_call_plain(8, 3, None, nulls, nulls, nulls, nulls, None, None, None, None, None, 0, stream=0)
    B.echo_reduce_shard(nulls, nulls, None, None, None, None, 0, stream=0)
    B.echo_reduce_shard_sum(nulls, nulls, None, None, 0, stream=0)
    B.echo_decode(None, None, None, 0, stream=0)
    B.echo_decode(None, None, None, 0, bits=8, stream=0)
    # the scalar checks still apply to an empty call
    e.bits = 5
    assert rc(B.echo_call, e, None, nulls, nulls, nulls, nulls, None, None, None, None, None) == -7
    assert rc(B.echo_call, B.EchoState(None, None, 0, 8, 9), None, nulls, nulls, nulls, nulls,
              None, None, None, None, None) == -4
    assert rc(B.echo_call_plain, 0, 0, None, [], [], [], [], None, None, None, None, None, 0) == -4
    assert rc(B.echo_decode, None, None, None, 0, bits=3) == -7
    assert rc(B.echo_decode, None, None, None, -128) == -2
    assert rc(B.echo_reduce_shard, nulls * 3, nulls * 3, None, None, None, None, 0) == -4
    assert rc(B.echo_reduce_shard_sum, nulls, nulls, None, None, 0, bits=2) == -7


def test_entry_range_rejections():
    s4 = st(n=4096, P=4, rank=1)
    assert rc(B.echo_call_entry_range, s4, 3 * A, -1, 2, 50 * A, 51 * A) == -4
    assert rc(B.echo_call_entry_range, s4, 3 * A, 0, 5, 50 * A, 51 * A) == -4
    assert rc(B.echo_call_entry_range, s4, 3 * A, 3, 2, 50 * A, 51 * A) == -4
    assert rc(B.echo_call_entry_range, s4, None, 0, 4, 50 * A, 51 * A) == -1
    assert rc(B.echo_call_entry_range, s4, 3 * A, 0, 4, 3 * A + 16, 51 * A) == -6  # codes over x
    s4.bits = 6
    assert rc(B.echo_call_entry_range, s4, 3 * A, 0, 4, 50 * A, 51 * A) == -7


def test_stream_copy_rejections():
    assert rc(B.echo_stream_copy, 3 * A, 4 * A, 100) == -2
    assert rc(B.echo_stream_copy, 3 * A, 4 * A, -16) == -2
    assert rc(B.echo_stream_copy, None, 4 * A, 256) == -1
    assert rc(B.echo_stream_copy, 3 * A + 8, 4 * A, 256) == -3
    assert rc(B.echo_stream_copy, 3 * A, 3 * A + 128, 256) == -6
    B.echo_stream_copy(None, None, 0, stream=0)  # empty: a no-op


def test_build_entry_check_matches_header():
    import __graft_entry__ as ge
    ge.check_loaded()


def test_binding_refuses_host_tensors_before_calling():
    """A host tensor would reach a kernel as a bad address: the binding stops
    it on the host (no library call, so no GPU is touched)."""
    import torch
    codes = torch.zeros(64, dtype=torch.uint8)
    scales = torch.zeros(1)
    y = torch.zeros(128, dtype=torch.int16)
    with pytest.raises(ValueError, match="GPU tensor"):
        B.echo_decode(codes, scales, y, stream=0)
    with pytest.raises(ValueError, match="GPU tensor"):
        B.EchoState(torch.zeros(1024), torch.zeros(1024), 1024, 2, 0)
    with pytest.raises(ValueError, match="GPU tensor"):
        B.echo_stream_copy(codes, codes.clone(), 64, stream=0)


# Page titles and the sections of them that the header may cite.
PAGES = {
    "Echo: Error-Compensated 4-Bit Tensor-Parallel Communication": ("Abstract",),
    "Tensor-parallel traffic drops to 4 bits": ("Synopsis", "Interpretation", "Perspective"),
    "How Echo lets big AI models train faster": ("How Echo keeps errors from snowballing",
                                                 "What the benchmarks show", "Key facts"),
}
# calls that are not steps of the method (measurement and bookkeeping)
NOT_METHOD = {"echo_stream_copy", "echo_get_config", "echo_status_string", "echo_version"}


def declaration_comments():
    """{function: the comment text between the previous declaration and it}"""
    src = open(HEADER).read()
    src = src[src.index("typedef struct echo_config"):]
    out, last = {}, 0
    for m in re.finditer(r"^\s*(?:const\s+)?\w+\**\s+\**(echo_\w+)\s*\([^;]*\);", src, re.M):
        between = src[last:m.start()]
        out[m.group(1)] = " ".join(re.findall(r"/\*(.*?)\*/", between, flags=re.S))
        last = m.end()
    return out


def test_every_method_call_cites_a_page_section():
    comments = declaration_comments()
    assert set(comments) == set(declared_functions())
    for name, text in comments.items():
        if name in NOT_METHOD:
            continue
        flat = " ".join(text.replace("*", " ").split())
        cited = [(t, sec) for t, secs in PAGES.items() for sec in secs
                 if t.replace("-", "") in flat.replace("- ", "").replace("-", "") and sec in flat]
        assert cited, f"{name}: its comment cites no page section"


def test_prepared_call_refuses_a_changed_state():
    """A prepared call checked its buffers for the state's width at prepare
    time; after st.bits changes it raises before reaching the library (the
    fake addresses below are never handed to a kernel)."""
    P, n = 4, 4096
    s4 = st(n=n, P=P, rank=1)
    cn = n // P
    recv_c = [None if k == 1 else 10 * A + k * A for k in range(P)]
    recv_s = [None if k == 1 else 20 * A + k * A for k in range(P)]
    gath_c = [None if k == 1 else 30 * A + k * A for k in range(P)]
    gath_s = [None if k == 1 else 40 * A + k * A for k in range(P)]
    call = B.echo_call_prepare(s4, 3 * A, recv_c, recv_s, gath_c, gath_s, 50 * A, 51 * A, 52 * A,
                               53 * A, 54 * A)
    assert call._snap.bits == 4 and cn == 1024
    s4.bits = 8
    with pytest.raises(ValueError, match="changed since the call was prepared"):
        call(stream=0)
    # the copy the library would read keeps the prepared width
    assert call._snap.bits == 4


def test_library_reports_only_its_own_launch_status():
    """The library launches through hipLaunchKernel, whose return value is that
    launch's status, and never reads the thread's last-error slot
    (hipGetLastError / hipPeekAtLastError are not even imported), so an error
    an earlier, unrelated HIP call left behind can neither be reported as an
    echo_* call's ECHO_ERR_HIP nor be cleared by it."""
    import shutil
    import subprocess

    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--undefined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    imported = {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}
    assert "hipLaunchKernel" in imported
    assert not imported & {"hipGetLastError", "hipPeekAtLastError", "hipExtGetLastError"}


def test_correction_array_rejections():
    """echo_correction / echo_encode_corr / echo_update_corr check their
    arguments before launching (every call below is rejected)."""
    s = st()  # n = 1024, P = 2: averages at A and 2A
    assert rc(B.echo_correction, s, None) == -1
    assert rc(B.echo_correction, s, 3 * A + 4) == -3
    assert rc(B.echo_correction, s, A + 512) == -6          # corr over m_fast
    assert rc(B.echo_encode_corr, s, 3 * A, None, 4 * A, 5 * A) == -1
    assert rc(B.echo_encode_corr, s, 3 * A, 6 * A + 8, 4 * A, 5 * A) == -3
    assert rc(B.echo_encode_corr, s, 3 * A, 6 * A, 6 * A + 64, 5 * A) == -6  # codes over corr
    assert rc(B.echo_encode_corr, st(n=1000), 3 * A, 6 * A, 4 * A, 5 * A) == -2
    assert rc(B.echo_update_corr, s, 3 * A, 4 * A, 5 * A, 6 * A, None) == -1
    assert rc(B.echo_update_corr, s, 3 * A, 4 * A, 5 * A, 6 * A, 7 * A + 4) == -3
    assert rc(B.echo_update_corr, s, 3 * A, 4 * A, 5 * A, 6 * A, 2 * A + 256) == -6  # corr over m_slow
    assert rc(B.echo_update_corr, s, 3 * A, 4 * A, 5 * A, 6 * A, 3 * A) == -6        # corr over x
