"""Randomized properties of the oracle (CPU only): what the pages fix, checked
over drawn rank counts, tensor sizes, code widths, magnitudes and states.

  * every value is quantized exactly twice per all-reduce call and once per
    reduce-scatter call ("Echo: Error-Compensated 4-Bit Tensor-Parallel
    Communication", Abstract);
  * the residuals the ranks fold into their averages add up to the error the
    call injected ("Tensor-parallel traffic drops to 4 bits",
    Interpretation), up to binary32 rounding;
  * a rank fed the other ranks' messages reproduces the full simulation
    (the two exchanges carry everything a rank needs);
  * messages never hold the most negative code, scales are finite and
    non-negative, and every output is the group's dequantized code.
"""
import numpy as np
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import oracle as orc

G = orc.GROUP

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def bf16_bits(v):
    t = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_vals(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


problems = st.fixed_dictionaries({
    "P": st.integers(1, 16),
    "k": st.integers(1, 3),
    "bits": st.sampled_from([4, 8]),
    "log2_scale": st.integers(-20, 20),
    "state_scale": st.sampled_from([0.0, 0.01, 0.3]),
    "zero_groups": st.booleans(),
    "seed": st.integers(0, 2**31 - 1),
})


def draw_ranks(pr):
    rng = np.random.default_rng(pr["seed"])
    P, n = pr["P"], pr["P"] * G * pr["k"]
    scale = 2.0 ** pr["log2_scale"]
    xs = []
    for _ in range(P):
        v = rng.standard_normal(n) * scale
        if pr["zero_groups"]:
            v.reshape(-1, G)[rng.random(n // G) < 0.3] = 0.0
        xs.append(bf16_bits(v))
    mf = [(rng.standard_normal(n) * pr["state_scale"] * scale).astype(np.float32) for _ in range(P)]
    ms = [(rng.standard_normal(n) * pr["state_scale"] * scale).astype(np.float32) for _ in range(P)]
    return xs, mf, ms


def check_message(codes, scales, bits):
    if bits == 8:
        assert not np.any(codes == 0x80)
    else:
        assert not np.any((codes & 0xF) == 8) and not np.any((codes >> 4) == 8)
    assert np.all(np.isfinite(scales)) and np.all(scales >= 0)


@SETTINGS
@given(problems, st.booleans())
def test_all_reduce_properties(pr, comp):
    P, bits = pr["P"], pr["bits"]
    xs, mf, ms = draw_ranks(pr)
    n = xs[0].size
    Cn = n // P
    mf0, ms0 = [a.copy() for a in mf], [a.copy() for a in ms]
    orc.counters_reset()
    sim = orc.simulate(xs, mf, ms, comp=comp, want_detail=True, bits=bits)
    assert orc.counter(1) == P * n and orc.counter(2) == n

    # messages and the output: y is the bf16 of each stage-2 code times its scale
    for p in range(P):
        check_message(sim["codes1"][p], sim["scales1"][p], bits)
    check_message(sim["codes2"], sim["scales2"], bits)
    q2 = orc.unpack_codes(sim["codes2"], n, bits).astype(np.float32)
    d2 = q2 * np.repeat(sim["scales2"], G)
    assert np.array_equal(sim["y"], bf16_bits(d2))

    # residual identity: sum_p r_p = f32(y) - sum_p x'_p (binary32 rounding aside)
    if comp:
        y = bf16_vals(sim["y"]).astype(np.float64)
        xp = np.array(sim["xp"], dtype=np.float64)
        r = np.array(sim["r"], dtype=np.float64)
        u = 2.0 ** -24
        bound = 4 * P * u * (np.abs(xp).sum(axis=0) + np.abs(r).sum(axis=0) + np.abs(y)
                             + np.abs(y - xp.sum(axis=0))) + 4 * 2.0 ** -149 * P
        assert np.all(np.abs(r.sum(axis=0) - (y - xp.sum(axis=0))) <= bound)

    # rank mode reproduces the simulation for one drawn rank
    p = pr["seed"] % P
    cb = Cn if bits == 8 else Cn // 2
    cs, ss = slice(p * cb, (p + 1) * cb), slice(p * Cn // G, (p + 1) * Cn // G)
    recv_c = [None if q == p else sim["codes1"][q][cs].copy() for q in range(P)]
    recv_s = [None if q == p else sim["scales1"][q][ss].copy() for q in range(P)]
    gath_c = [None if j == p else sim["codes2"][j * cb:(j + 1) * cb].copy() for j in range(P)]
    gath_s = [None if j == p else sim["scales2"][j * Cn // G:(j + 1) * Cn // G].copy() for j in range(P)]
    mfp, msp = mf0[p].copy(), ms0[p].copy()
    out = orc.call(P, p, xs[p], mfp, msp, recv_c, recv_s, gath_c, gath_s, comp=comp, bits=bits)
    assert np.array_equal(out["y"], sim["y"])
    assert np.array_equal(out["own_codes2"], sim["codes2"][cs])
    assert np.array_equal(out["own_scales2"], sim["scales2"][ss])
    for j in range(P):
        if j != p:
            js = slice(j * cb, (j + 1) * cb)
            assert np.array_equal(out["send_codes"][js], sim["codes1"][p][js])
    if comp:
        assert np.array_equal(mfp.view(np.uint32), mf[p].view(np.uint32))
        assert np.array_equal(msp.view(np.uint32), ms[p].view(np.uint32))
    else:
        assert np.array_equal(mfp, mf0[p]) and np.array_equal(msp, ms0[p])


@SETTINGS
@given(problems)
def test_reduce_scatter_properties(pr):
    P, bits = pr["P"], pr["bits"]
    xs, mf, ms = draw_ranks(pr)
    n = xs[0].size
    Cn = n // P
    mf0, ms0 = [a.copy() for a in mf], [a.copy() for a in ms]
    # each rank's stage-1 message, from the entry pass on the state before the call
    msgs = [orc.encode(xs[p], mf0[p], ms0[p], bits=bits) for p in range(P)]
    orc.counters_reset()
    sim = orc.rs_simulate(xs, mf, ms, bits=bits)
    assert orc.counter(1) == P * n and orc.counter(2) == 0
    # the chunk owner's output is the bf16 of the exact rank-order binary32 sum
    d1 = []
    for p in range(P):
        check_message(*msgs[p], bits)
        q = orc.unpack_codes(msgs[p][0], n, bits).astype(np.float32)
        d1.append(q * np.repeat(msgs[p][1], G))
    S = d1[0].copy()
    for p in range(1, P):
        S = (S + d1[p]).astype(np.float32)
    assert np.array_equal(sim["y"], bf16_bits(S))
    # rank mode reproduces the simulation
    p = pr["seed"] % P
    cb = Cn if bits == 8 else Cn // 2
    cs, ss = slice(p * cb, (p + 1) * cb), slice(p * Cn // G, (p + 1) * Cn // G)
    recv_c = [None if q == p else msgs[q][0][cs].copy() for q in range(P)]
    recv_s = [None if q == p else msgs[q][1][ss].copy() for q in range(P)]
    mfp, msp = mf0[p].copy(), ms0[p].copy()
    out = orc.rs_call(P, p, xs[p], mfp, msp, recv_c, recv_s, bits=bits)
    assert np.array_equal(out["y_own"], sim["y"][p * Cn:(p + 1) * Cn])
    assert np.array_equal(mfp.view(np.uint32), mf[p].view(np.uint32))
    assert np.array_equal(msp.view(np.uint32), ms[p].view(np.uint32))
