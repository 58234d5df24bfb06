"""Windows of a rank-mode call sequence, recomputed by the oracle (test
infrastructure; imports only numpy and the oracle)."""
import numpy as np


class WindowOracle:
    """The oracle's view of a window of W groups at group offset `off` of
    chunk j, in a rank-mode problem of P ranks seen from rank p.

    Every output of a group depends only on that group's own inputs (x, the
    averages, the incoming shards or the gathered chunk of that group), so a
    small rank-mode problem of P chunks of W groups whose chunk j holds the
    window's inputs (the other chunks zero) computes exactly the window's
    outputs; its chunk-j averages are carried from call to call."""

    def __init__(self, P, rank, j, off, W, mf0=None, ms0=None, bits=4, comp=True):
        from oracle import oracle as orc

        self.orc = orc
        self.P, self.rank, self.j, self.off, self.W = P, rank, j, off, W
        self.bits = bits
        self.comp = comp  # False: the uncompensated call (the averages stay zero)
        self.Cm = W * 128
        self.cbm = self.Cm if bits == 8 else self.Cm // 2  # code bytes of the window
        self.nm = P * self.Cm
        self.mf = np.zeros(self.nm, np.float32)
        self.ms = np.zeros(self.nm, np.float32)
        sl = slice(j * self.Cm, (j + 1) * self.Cm)
        if mf0 is not None:
            self.mf[sl] = mf0
            self.ms[sl] = ms0

    def elems(self, C):
        """element slice of the window in the big tensor (chunk size C)"""
        e0 = self.j * C + self.off * 128
        return slice(e0, e0 + self.Cm)

    def chunk_elems(self):
        """element slice of the window inside its chunk"""
        return slice(self.off * 128, self.off * 128 + self.Cm)

    def code_slice(self, elems):
        """byte slice of the codes of an element slice (both code widths)"""
        f = 1 if self.bits == 8 else 2
        return slice(elems.start // f, elems.stop // f)

    def call(self, x_win, msg_win):
        """x_win: bf16 bits of the window; msg_win: the window's incoming
        shards [(codes, scales) per q, slot rank None] when j == rank, else
        the gathered chunk's window (codes, scales).  Returns the window's
        outputs."""
        P, r, j, Cm = self.P, self.rank, self.j, self.Cm
        x = np.zeros(self.nm, np.uint16)
        x[j * Cm:(j + 1) * Cm] = x_win
        zc, zs = np.zeros(self.cbm, np.uint8), np.zeros(Cm // 128, np.float32)
        recv_c = [None if q == r else (msg_win[q][0] if j == r else zc) for q in range(P)]
        recv_s = [None if q == r else (msg_win[q][1] if j == r else zs) for q in range(P)]
        gath_c = [None if q == r else (msg_win[0] if q == j else zc) for q in range(P)]
        gath_s = [None if q == r else (msg_win[1] if q == j else zs) for q in range(P)]
        out = self.orc.call(P, r, x, self.mf, self.ms, recv_c, recv_s, gath_c, gath_s, comp=self.comp,
                            bits=self.bits)
        cs = slice(j * self.cbm, (j + 1) * self.cbm)
        gs = slice(j * Cm // 128, (j + 1) * Cm // 128)
        es = slice(j * Cm, (j + 1) * Cm)
        res = dict(y=out["y"][es], m_fast=self.mf[es].copy(), m_slow=self.ms[es].copy())
        if j == r:
            res.update(codes=out["own_codes2"], scales=out["own_scales2"])
        else:
            res.update(codes=out["send_codes"][cs], scales=out["send_scales"][gs])
        return res


class RSWindowOracle(WindowOracle):
    """The same window argument for the reduce-scatter call: the window's
    send codes (chunk j != p) or its slice of y_own (j == p), and its
    averages."""

    def call(self, x_win, msg_win):
        P, r, j, Cm = self.P, self.rank, self.j, self.Cm
        x = np.zeros(self.nm, np.uint16)
        x[j * Cm:(j + 1) * Cm] = x_win
        zc, zs = np.zeros(self.cbm, np.uint8), np.zeros(Cm // 128, np.float32)
        recv_c = [None if q == r else (msg_win[q][0] if j == r else zc) for q in range(P)]
        recv_s = [None if q == r else (msg_win[q][1] if j == r else zs) for q in range(P)]
        out = self.orc.rs_call(P, r, x, self.mf, self.ms, recv_c, recv_s, bits=self.bits)
        es = slice(j * Cm, (j + 1) * Cm)
        res = dict(m_fast=self.mf[es].copy(), m_slow=self.ms[es].copy())
        if j == r:
            res["y_own"] = out["y_own"]
        else:
            res.update(codes=out["send_codes"][j * self.cbm:(j + 1) * self.cbm],
                       scales=out["send_scales"][j * Cm // 128:(j + 1) * Cm // 128])
        return res


def pick_windows(P, C, W, rng, per_chunk=2):
    """(j, off) windows of W groups: the first and last groups of every
    chunk plus `per_chunk` seeded random offsets per chunk."""
    Gc = C // 128
    out = []
    for j in range(P):
        offs = {0, max(0, Gc - W)}
        for _ in range(per_chunk):
            offs.add(int(rng.integers(0, max(1, Gc - W + 1))))
        out += [(j, o) for o in sorted(offs)]
    return out
