"""Helpers shared by the GPU parity tests: host <-> device copies of raw
bytes, and a GPU harness that simulates P ranks on one device through the C
ABI.  Nothing here computes any step of the method."""
from __future__ import annotations

import numpy as np
import torch

from error_compensated_bit_echo_amd import binding as B

DEV = "cuda:0"


def eq(a, b, what):
    """bitwise equality of two arrays, with the first mismatches in the message"""
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    bad = np.nonzero(a.ravel() != b.ravel())[0]
    assert bad.size == 0, (f"{what}: {bad.size} mismatches, first at {bad[:5]}: "
                           f"{a.ravel()[bad[:5]]} vs {b.ravel()[bad[:5]]}")


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy array -> device tensor holding the same bytes."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV)
    return torch.from_numpy(a.copy()).to(DEV)


def host(t: torch.Tensor, dtype) -> np.ndarray:
    """device tensor -> numpy array of `dtype` over the same bytes."""
    a = t.detach().cpu().contiguous().numpy()
    return a.view(dtype)


def empty_u8(n, fill=None):
    t = torch.empty(n, dtype=torch.uint8, device=DEV)
    if fill is not None:
        t.fill_(fill)
    return t


def empty_f32(n, fill=None):
    t = torch.empty(n, dtype=torch.float32, device=DEV)
    if fill is not None:
        t.fill_(fill)
    return t


def empty_bf16(n):
    return torch.empty(n, dtype=torch.int16, device=DEV)


class GpuRank:
    """Device buffers of one logical rank in full-simulation mode."""

    def __init__(self, x: np.ndarray, mf: np.ndarray, ms: np.ndarray, nranks: int, rank: int):
        n = x.size
        self.n = n
        self.x = dev(x)
        self.mf = dev(mf.astype(np.float32))
        self.ms = dev(ms.astype(np.float32))
        self.st = B.EchoState(self.mf, self.ms, n, nranks, rank)
        # room for either code width (one byte per element at 8 bits)
        self.codes1 = empty_u8(n)
        self.scales1 = empty_f32(n // 128)
        self.send_codes = empty_u8(n)
        self.send_scales = empty_f32(n // 128)
        self.y = empty_bf16(n)


def gpu_simulate_call(ranks, xs_np, bits=4):
    """One call of P logical ranks on the GPU: every rank's entry pass
    (echo_encode, state read-only), the reduce of every chunk from the
    ranks' stage-1 chunks (echo_reduce_shard), then each rank's fused
    echo_call fed with those chunks, which re-derives its own chunk, writes
    y and refreshes its state.  `bits` is the call's code width.  Returns
    (codes2, scales2, own codes2 per rank, own scales2 per rank)."""
    P = len(ranks)
    n = ranks[0].n
    Cn = n // P
    f = 1 if bits == 8 else 2  # elements per code byte
    cb = Cn // f
    for r, x in zip(ranks, xs_np):
        r.st.bits = bits
        r.x.copy_(dev(x))
        B.echo_encode(r.st, r.x, r.codes1[:n // f], r.scales1)
    codes2 = empty_u8(n // f)
    scales2 = empty_f32(n // 128)
    for j in range(P):
        B.echo_reduce_shard([r.codes1[j * cb:(j + 1) * cb] for r in ranks],
                            [r.scales1[j * Cn // 128:(j + 1) * Cn // 128] for r in ranks],
                            codes2[j * cb:(j + 1) * cb],
                            scales2[j * Cn // 128:(j + 1) * Cn // 128], chunk_n=Cn, bits=bits)
    own2 = [empty_u8(cb) for _ in range(P)]
    own2s = [empty_f32(Cn // 128) for _ in range(P)]
    for p, r in enumerate(ranks):
        recv_c = [None if q == p else ranks[q].codes1[p * cb:(p + 1) * cb] for q in range(P)]
        recv_s = [None if q == p else ranks[q].scales1[p * Cn // 128:(p + 1) * Cn // 128]
                  for q in range(P)]
        gath_c = [None if j == p else codes2[j * cb:(j + 1) * cb] for j in range(P)]
        gath_s = [None if j == p else scales2[j * Cn // 128:(j + 1) * Cn // 128] for j in range(P)]
        B.echo_call(r.st, r.x, recv_c, recv_s, gath_c, gath_s, r.send_codes[:n // f], r.send_scales,
                    own2[p], own2s[p], r.y)
    torch.cuda.synchronize()
    return codes2, scales2, own2, own2s


from windows import RSWindowOracle, WindowOracle, pick_windows  # noqa: E402,F401
