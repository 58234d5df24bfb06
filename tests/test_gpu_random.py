"""Seeded random sweep (1500 cases) of the GPU path against the oracle: drawn rank counts,
ranks, chunk lengths (1 to 40 groups: every parity of the last wave's slice),
code widths, input magnitudes and entry points (fused call, in place, the
phased calls, the uncompensated call, the reduce-scatter call, the
deferred-update schedule with and without the correction array), two calls
each with the averages carried.  Bit-exact."""
import numpy as np
import pytest

import gpu_util as g
from error_compensated_bit_echo_amd import binding as B
from error_compensated_bit_echo_amd import inputs as I
from oracle import oracle as orc
from test_gpu_parity import RankCase, eq

pytestmark = pytest.mark.gpu

MODES = ("call", "in_place", "phased", "plain", "rs", "split", "split_corr")


def _cases(count=1500, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        P = int(rng.integers(1, 17))
        out.append(dict(i=i, P=P, rank=int(rng.integers(0, P)), k=int(rng.integers(1, 41)),
                        bits=int(rng.choice([4, 8])), mode=MODES[i % len(MODES)],
                        log2_scale=int(rng.integers(-12, 13))))
    return out


def _x(n, case, call):
    v = I.normal(n, I.stream_key("random-sweep", case["i"], call)) * 2.0 ** case["log2_scale"]
    v[: n // 7] *= 0.0 if case["i"] % 3 == 0 else 1.0  # some cases start with all-zero groups
    return I.to_bf16_bits(v)


@pytest.mark.timeout(600)
def test_random_sweep_bit_exact():
    for case in _cases():
        P, rank, k, bits, mode = case["P"], case["rank"], case["k"], case["bits"], case["mode"]
        print(f"random sweep: case {case}", flush=True)
        rc = RankCase(P, rank, k, seed=5000 + case["i"], bits=bits)
        what = f"case {case['i']} ({mode}, P={P}, rank={rank}, k={k}, bits={bits})"
        f = 1 if bits == 8 else 2
        if mode.startswith("split"):
            codes1, scales1 = g.empty_u8(rc.n // f), g.empty_f32(rc.n // 128)
            e2 = g.empty_f32(rc.Cn)
            corr = g.empty_f32(rc.n, 5.0)
            if mode == "split_corr":
                B.echo_correction(rc.st, corr)
        for call in range(2):
            x = _x(rc.n, case, call)
            xd = g.dev(x)
            if mode in ("call", "in_place", "phased"):
                if mode == "call":
                    rc.gpu_call(xd)
                    y = rc.y
                elif mode == "in_place":
                    rc.gpu_call(xd, y=xd)
                    y = xd
                else:
                    B.echo_call_entry(rc.st, xd, rc.send_c, rc.send_s)
                    B.echo_call_reduce(rc.st, xd, rc.slot(rc.recv_d, 0), rc.slot(rc.recv_d, 1),
                                       rc.own_c, rc.own_s, rc.y)
                    B.echo_call_exit(rc.st, rc.slot(rc.gath_d, 0), rc.slot(rc.gath_d, 1), rc.y)
                    y = rc.y
                rc.check(rc.oracle_call(x), y=y)
            elif mode.startswith("split"):
                Cn = rc.Cn
                if mode == "split":
                    B.echo_encode(rc.st, xd, codes1, scales1)
                else:
                    B.echo_encode_corr(rc.st, xd, corr, codes1, scales1)
                sh_c = [codes1[rank * Cn // f:(rank + 1) * Cn // f] if q == rank else rc.recv_d[q][0]
                        for q in range(P)]
                sh_s = [scales1[rank * Cn // 128:(rank + 1) * Cn // 128] if q == rank else rc.recv_d[q][1]
                        for q in range(P)]
                B.echo_reduce_shard(sh_c, sh_s, rc.own_c, rc.own_s, rc.y[rank * Cn:(rank + 1) * Cn], e2,
                                    chunk_n=Cn, bits=bits)
                B.echo_call_exit(rc.st, rc.slot(rc.gath_d, 0), rc.slot(rc.gath_d, 1), rc.y)
                if mode == "split":
                    B.echo_update(rc.st, xd, codes1, scales1, e2)
                else:
                    B.echo_update_corr(rc.st, xd, codes1, scales1, e2, corr)
                want = rc.oracle_call(x)
                eq(g.host(rc.y, np.uint16), want["y"], what + " y")
                eq(g.host(rc.own_c, np.uint8), want["own_codes2"], what + " own codes2")
                eq(g.host(rc.own_s, np.float32), want["own_scales2"], what + " own scales2")
                eq(g.host(rc.mfd, np.float32), rc.mf, what + " m_fast")
                eq(g.host(rc.msd, np.float32), rc.ms, what + " m_slow")
                c1 = g.host(codes1, np.uint8)
                for j in range(P):
                    if j != rank:
                        cs = slice(j * Cn // f, (j + 1) * Cn // f)
                        eq(c1[cs], want["send_codes"][cs], what + f" send chunk {j}")
                if mode == "split_corr":
                    eq(g.host(corr, np.float32), orc.correction(rc.mf, rc.ms), what + " correction")
            elif mode == "plain":
                B.echo_call_plain(P, rank, xd, rc.slot(rc.recv_d, 0), rc.slot(rc.recv_d, 1),
                                  rc.slot(rc.gath_d, 0), rc.slot(rc.gath_d, 1), rc.send_c, rc.send_s,
                                  rc.own_c, rc.own_s, rc.y, bits=bits)
                want = orc.call(P, rank, x, None, None, rc.slot(rc.recv, 0), rc.slot(rc.recv, 1),
                                rc.slot(rc.gath, 0), rc.slot(rc.gath, 1), comp=False, bits=bits)
                rc.check(want)
            else:
                y_own = g.empty_bf16(rc.Cn)
                B.echo_rs_call(rc.st, xd, rc.slot(rc.recv_d, 0), rc.slot(rc.recv_d, 1), rc.send_c,
                               rc.send_s, y_own)
                want = orc.rs_call(P, rank, x, rc.mf, rc.ms, rc.slot(rc.recv, 0), rc.slot(rc.recv, 1),
                                   bits=bits)
                eq(g.host(y_own, np.uint16), want["y_own"], what + " y_own")
                eq(g.host(rc.mfd, np.float32), rc.mf, what + " m_fast")
                eq(g.host(rc.msd, np.float32), rc.ms, what + " m_slow")
                cb = rc.Cn if bits == 8 else rc.Cn // 2
                sc = g.host(rc.send_c, np.uint8)
                for j in range(P):
                    if j != rank:
                        eq(sc[j * cb:(j + 1) * cb], want["send_codes"][j * cb:(j + 1) * cb],
                           what + f" send chunk {j}")
