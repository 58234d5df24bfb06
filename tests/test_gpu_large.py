"""Beyond 32-bit offsets: a rank tensor of 2^31 + 3072 elements (x 4 GiB, each
average 8 GiB, byte offsets up to 2^33, a group count that is not a multiple
of a wavefront's two groups), with 4-bit and 8-bit codes (the 8-bit send
message alone exceeds 2^31 bytes), checked on windows of every chunk -- the
last groups of the tensor among them -- over two calls with the averages
carried.
Inputs are drawn on the device; the oracle reads the windows' bytes back."""
import numpy as np
import pytest
import torch

import gpu_util as g
from error_compensated_bit_echo_amd import binding as B

pytestmark = pytest.mark.gpu


def _device_message(C, gen, bits=4):
    """Seeded message drawn on the device: bytes with no -8 field (4-bit) or
    any byte but -128 (8-bit), scales in [0.05, 0.55)."""
    if bits == 8:
        table = torch.tensor([b for b in range(256) if b != 0x80], dtype=torch.uint8, device=g.DEV)
    else:
        table = torch.tensor([b for b in range(256) if (b & 0xF) != 8 and (b >> 4) != 8],
                             dtype=torch.uint8, device=g.DEV)
    idx = torch.randint(0, table.numel(), (C if bits == 8 else C // 2,), generator=gen, device=g.DEV)
    codes = table[idx]
    scales = torch.rand(C // 128, generator=gen, device=g.DEV) * 0.5 + 0.05
    return codes, scales


@pytest.mark.timeout(600)
@pytest.mark.parametrize("bits", [4, 8])
def test_tensor_beyond_2_to_the_31_elements(bits):
    P, rank = 8, 6
    n = (1 << 31) + P * 128 * 3
    C = n // P
    gen = torch.Generator(device=g.DEV)
    gen.manual_seed(31)
    print("large: allocating and drawing inputs", flush=True)
    recv = [None if q == rank else _device_message(C, gen, bits) for q in range(P)]
    gath = [None if j == rank else _device_message(C, gen, bits) for j in range(P)]
    mf = g.empty_f32(n)
    ms = g.empty_f32(n)
    st = B.echo_state_init(mf, ms, n, P, rank, bits=bits)
    f = 1 if bits == 8 else 2  # elements per code byte
    send_c, send_s = g.empty_u8(n // f), g.empty_f32(n // 128)
    own_c, own_s = g.empty_u8(C // f), g.empty_f32(C // 128)
    y = g.empty_bf16(n)
    sl = lambda arr, k: [None if m is None else m[k] for m in arr]  # noqa: E731
    W = 3
    rng = np.random.default_rng(7)
    wins = [g.WindowOracle(P, rank, j, off, W, bits=bits) for j, off in g.pick_windows(P, C, W, rng, 2)]
    x = torch.empty(n, dtype=torch.int16, device=g.DEV)
    for call in range(2):
        x.copy_((torch.randn(n, generator=gen, device=g.DEV) * (1 + call)).to(torch.bfloat16).view(torch.int16))
        B.echo_call(st, x, sl(recv, 0), sl(recv, 1), sl(gath, 0), sl(gath, 1), send_c, send_s,
                    own_c, own_s, y)
        torch.cuda.synchronize()
        for w in wins:
            es, ce = w.elems(C), w.chunk_elems()
            if w.j == rank:
                msg = [None if q == rank else (g.host(recv[q][0][w.code_slice(ce)], np.uint8),
                                               g.host(recv[q][1][ce.start // 128:ce.stop // 128], np.float32))
                       for q in range(P)]
            else:
                msg = (g.host(gath[w.j][0][w.code_slice(ce)], np.uint8),
                       g.host(gath[w.j][1][ce.start // 128:ce.stop // 128], np.float32))
            want = w.call(g.host(x[es], np.uint16), msg)
            what = f"call {call} window (chunk {w.j}, group {w.off})"
            g.eq(g.host(y[es], np.uint16), want["y"], what + " y")
            g.eq(g.host(mf[es], np.float32), want["m_fast"], what + " m_fast")
            g.eq(g.host(ms[es], np.float32), want["m_slow"], what + " m_slow")
            if w.j == rank:
                g.eq(g.host(own_c[w.code_slice(ce)], np.uint8), want["codes"], what + " codes2")
            else:
                g.eq(g.host(send_c[w.code_slice(es)], np.uint8), want["codes"], what + " send")
                g.eq(g.host(send_s[es.start // 128:es.stop // 128], np.float32), want["scales"],
                     what + " send scales")
        print(f"large ({bits}-bit): call {call} windows ok (last window ends at element {wins[-1].elems(C).stop})",
              flush=True)
    assert wins[-1].elems(C).stop == n  # the tensor's last group was checked
