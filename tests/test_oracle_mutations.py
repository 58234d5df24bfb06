"""Planted mistakes in the CPU oracle are caught by its pins.

Each case copies the oracle's C sources, plants one plausible mistake (a
flipped sign, a dropped term, a wrong index or slot, a wrong rounding rule,
decay, code range or nibble order), builds the copy with the oracle's own
flags and runs the oracle's CPU pins against it (the numpy front end loads
the copy named by ECHO_ORACLE_LIB).  The pins must fail for every planted
mistake, and must pass for an unmodified copy built the same way.  Only the
oracle is mutated, on the CPU; no GPU is involved.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
PINS = [os.path.join(ROOT, "tests", f) for f in (
    "test_oracle_units.py", "test_oracle_pipeline.py", "test_oracle_correction.py",
    "test_oracle_threaded.py", "test_oracle_properties.py")]

C1, MT = "echo_oracle.c", "echo_oracle_mt.c"

# (name, file, text to replace (first occurrence), replacement)
MUTANTS = [
    ("bf16 ties always round up", C1,
     "round_up = (int)(kept & 1u);", "round_up = 1;"),
    ("bf16 exact ties counted as above", C1,
     "if (dropped > 0x8000u) {", "if (dropped >= 0x8000u) {"),
    ("codes round half away from zero", C1,
     "float t = rintf(v[i] / s);", "float t = roundf(v[i] / s);"),
    ("codes by a reciprocal multiply", C1,
     "float t = rintf(v[i] / s);", "float t = rintf(v[i] * (1.0f / s));"),
    ("input corrected one average at a time", C1,
     "return xf - corr;", "return (xf - (ORC_W_FAST * mf)) - (ORC_W_SLOW * ms);"),
    ("scale by a reciprocal multiply", C1,
     "float s = amax / (float)qmax;", "float s = amax * (1.0f / (float)qmax);"),
    ("group absmax taken over signed values", C1,
     "float a = fabsf(v[i]);", "float a = v[i];"),
    ("zero-group rule dropped", C1,
     "if (s == 0.0f) {", "if (s != s) {"),
    ("odd groups dequantized with the even neighbour's scale", C1,
     "return (float)code_at(codes, i, bits) * scales[i / ORC_GROUP];",
     "return (float)code_at(codes, i, bits) * scales[(i / ORC_GROUP) & ~(int64_t)1];"),
    ("rank-order sum started from the last rank", C1,
     """      float acc = dequant(shard_codes[0], shard_scales[0], e, bits);
      for (int r = 1; r < nranks; ++r) acc = acc + dequant(shard_codes[r], shard_scales[r], e, bits);""",
     """      float acc = dequant(shard_codes[nranks - 1], shard_scales[nranks - 1], e, bits);
      for (int r = nranks - 2; r >= 0; --r) acc = acc + dequant(shard_codes[r], shard_scales[r], e, bits);"""),
    ("reduce-scatter sum started from the last rank", C1,
     """    float acc = dequant(shard_codes[0], shard_scales[0], i, bits);
    for (int r = 1; r < nranks; ++r) acc = acc + dequant(shard_codes[r], shard_scales[r], i, bits);""",
     """    float acc = dequant(shard_codes[nranks - 1], shard_scales[nranks - 1], i, bits);
    for (int r = nranks - 2; r >= 0; --r) acc = acc + dequant(shard_codes[r], shard_scales[r], i, bits);"""),
    ("stage-2 requantized to 4-bit levels at 8 bits", C1,
     "orc_quantize_group_q(S, ORC_GROUP, qmax_of(bits), q, &scales2[g], 2);",
     "orc_quantize_group_q(S, ORC_GROUP, ORC_QMAX, q, &scales2[g], 2);"),
    ("every rank sent the own chunk's message", C1,
     "memcpy(send_codes + j * cb, codes1 + j * cb, (size_t)cb);",
     "memcpy(send_codes + j * cb, codes1 + rank * cb, (size_t)cb);"),
    ("bf16 widened with a stray low bit", C1,
     "uint32_t u = (uint32_t)h << 16;", "uint32_t u = ((uint32_t)h << 16) | 0x8000u;"),
    ("nibbles swapped in a byte", C1,
     "codes[k] = (uint8_t)(lo | (hi << 4));", "codes[k] = (uint8_t)(hi | (lo << 4));"),
    ("wrong sign extension of a nibble", C1,
     "(int)nib - 16);", "(int)nib - 15);"),
    ("8-bit codes read unsigned", C1,
     "if (bits == 8) return (int)(int8_t)codes[i];", "if (bits == 8) return (int)codes[i];"),
    ("8-bit code range one short", C1,
     "return bits == 8 ? ORC_QMAX8 : ORC_QMAX;", "return bits == 8 ? ORC_QMAX8 - 1 : ORC_QMAX;"),
    ("correction subtracts the slow average", C1,
     "return (ORC_W_FAST * mf) + (ORC_W_SLOW * ms);", "return (ORC_W_FAST * mf) - (ORC_W_SLOW * ms);"),
    ("correction halves the summed averages", C1,
     "return (ORC_W_FAST * mf) + (ORC_W_SLOW * ms);", "return ORC_W_FAST * (mf + ms);"),
    ("slow average refreshed in increment form", C1,
     "m_slow[i] = (ORC_BETA_SLOW * m_slow[i]) + (ORC_ALPHA_SLOW * r);",
     "m_slow[i] = m_slow[i] + (ORC_ALPHA_SLOW * (r - m_slow[i]));"),
    ("exit pass truncates to bf16", C1,
     "for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_bf16(dequant(codes, scales, i, bits));",
     "for (int64_t i = 0; i < n; ++i) { float f = dequant(codes, scales, i, bits); uint32_t u; "
     "memcpy(&u, &f, sizeof u); y[i] = (uint16_t)(u >> 16); }"),
    ("correction added to the input", C1,
     "return xf - corr;", "return xf + corr;"),
    ("stage-1 residual with the wrong sign", C1,
     "float e1 = dequant(codes1, scales1, i, bits) - xp;",
     "float e1 = xp - dequant(codes1, scales1, i, bits);"),
    ("own chunk's stage-2 error dropped", C1,
     "if (i >= own0 && i < own1) r = e1 + e2_own[i - own0];",
     "if (i >= own0 && i < own1) r = e1 + 0.0f * e2_own[i - own0];"),
    ("slow average refreshed with the fast weight", C1,
     "m_slow[i] = (ORC_BETA_SLOW * m_slow[i]) + (ORC_ALPHA_SLOW * r);",
     "m_slow[i] = (ORC_BETA_SLOW * m_slow[i]) + (ORC_ALPHA_FAST * r);"),
    ("fast average decays at the slow rate", C1,
     "m_fast[i] = (ORC_BETA_FAST * m_fast[i]) + (ORC_ALPHA_FAST * r);",
     "m_fast[i] = (ORC_BETA_SLOW * m_fast[i]) + (ORC_ALPHA_FAST * r);"),
    ("last rank's shard left out of the sum", C1,
     "for (int r = 1; r < nranks; ++r) acc = acc + dequant(shard_codes[r], shard_scales[r], e, bits);",
     "for (int r = 1; r < nranks - 1; ++r) acc = acc + dequant(shard_codes[r], shard_scales[r], e, bits);"),
    ("stage-2 error with the wrong sign", C1,
     "if (e2) e2[base + i] = orc_bf16_to_f32(yi) - S[i];",
     "if (e2) e2[base + i] = S[i] - orc_bf16_to_f32(yi);"),
    ("own output is the sum, not its requantized value", C1,
     "uint16_t yi = orc_f32_to_bf16((float)q[i] * scales2[g]);",
     "uint16_t yi = orc_f32_to_bf16(S[i]);"),
    ("own slot reads chunk 0 of the stage-1 message", C1,
     "sc[q] = (q == rank) ? codes1 + rank * cb : recv_codes[q];",
     "sc[q] = (q == rank) ? codes1 : recv_codes[q];"),
    ("gathered chunk decoded into the wrong place", C1,
     "orc_decode(C, gath_codes[j], gath_scales[j], y + j * C, bits);",
     "orc_decode(C, gath_codes[j], gath_scales[j], y + (nranks - 1 - j) * C, bits);"),
    ("update adds stage-2 error on chunk 0", C1,
     "if (comp) orc_update(n, nranks, rank, x, m_fast, m_slow, codes1, scales1, e2, NULL, bits);",
     "if (comp) orc_update(n, nranks, 0, x, m_fast, m_slow, codes1, scales1, e2, NULL, bits);"),
    ("correction array from the slow average twice", C1,
     "corr[i] = correction_of(m_fast[i], m_slow[i]);", "corr[i] = correction_of(m_slow[i], m_slow[i]);"),
    ("entry pass adds the correction array", C1,
     "v[i] = orc_bf16_to_f32(x[base + i]) - corr[base + i];",
     "v[i] = orc_bf16_to_f32(x[base + i]) + corr[base + i];"),
    ("reduce-scatter error with the wrong sign", C1,
     "if (e) e[i] = orc_bf16_to_f32(yi) - acc;", "if (e) e[i] = acc - orc_bf16_to_f32(yi);"),
    ("reduce-scatter sums one rank too few", C1,
     "orc_reduce_chunk_sum(nranks, C, sc, ss, y_own, e, bits);",
     "orc_reduce_chunk_sum(nranks - 1, C, sc, ss, y_own, e, bits);"),
    ("threaded driver drops a group at each run boundary", MT,
     "task[t].g1 = groups * (t + 1) / threads;",
     "task[t].g1 = groups * (t + 1) / threads - (t + 1 < threads ? 1 : 0);"),
    ("threaded reduce reads chunk 0 as its own slot", MT,
     "sc[q] = j->codes1 + code_bytes_of(own, j->bits) + cb0;", "sc[q] = j->codes1 + cb0;"),
]


def _build_copy(dest, mutant=None):
    """Copy the oracle's C sources to dest, plant the mutation, build."""
    from oracle import build as ob

    os.makedirs(dest)
    for f in ("echo_oracle.h", C1, MT):
        shutil.copy(os.path.join(ORACLE, f), dest)
    if mutant is not None:
        _, fname, old, new = mutant
        path = os.path.join(dest, fname)
        with open(path) as fh:
            src = fh.read()
        assert src.count(old) >= 1, f"mutation site not found in {fname}: {old}"
        with open(path, "w") as fh:
            fh.write(src.replace(old, new, 1))
    lib = os.path.join(dest, "liborc.so")
    # the oracle's flags, less -Werror: a planted mistake may leave an
    # argument unused
    flags = [f for f in ob.CFLAGS if f != "-Werror"]
    subprocess.run(["gcc", *flags, "-pthread", os.path.join(dest, C1), os.path.join(dest, MT),
                    "-o", lib, "-lm"], check=True, capture_output=True)
    return lib


def _run_pins(lib, cwd):
    env = dict(os.environ, ECHO_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PINS], cwd=cwd, env=env, capture_output=True, text=True,
                       timeout=900)
    return r.returncode, (r.stdout + r.stderr)[-1500:]


def _case(tmp, k, mutant):
    d = os.path.join(tmp, f"m{k:02d}")
    lib = _build_copy(d, mutant)
    rc, tail = _run_pins(lib, d)
    return mutant, rc, tail


@pytest.mark.timeout(1800)
def test_pins_catch_every_planted_mistake(tmp_path):
    tmp = str(tmp_path)
    lib = _build_copy(os.path.join(tmp, "pristine"))
    rc, tail = _run_pins(lib, os.path.join(tmp, "pristine"))
    assert rc == 0, "the pins fail on an unmodified copy of the oracle:\n" + tail
    workers = max(1, min(4, (os.cpu_count() or 2) // 2))
    with cf.ThreadPoolExecutor(max_workers=workers) as pool:
        results = list(pool.map(lambda km: _case(tmp, *km), enumerate(MUTANTS)))
    survivors = [(m[0], tail) for m, rc, tail in results if rc == 0]
    assert not survivors, "planted mistakes the pins did not catch: " + "; ".join(s[0] for s in survivors)
    # a crash is not a catch: every mutant must fail by a failed assertion
    crashed = [m[0] for m, rc, tail in results if rc not in (1,)]
    assert not crashed, f"mutants that ended the pin run abnormally: {crashed}"
