"""Write tests/golden/quantizer_hand_cases.json.

The expected values here are derived by hand (see each case's "why"); this
script only lays them out, with every float stored as float.hex() so the
fixture is exact.  It imports nothing from the library or the oracle.
Sources: the pages fix a transport of 4-bit integer codes ("Tensor-parallel
traffic drops to 4 bits", Interpretation; "Echo: Error-Compensated 4-Bit
Tensor-Parallel Communication", Abstract); per-group scaling, the group size
128, the code range [-7, 7], s = amax / 7 and round-half-to-even are the
stated readings.
"""
import json
import os

TINY = 2.0 ** -149  # smallest positive binary32 (denormal)


def pad(v, n=128):
    return list(v) + [0.0] * (n - len(v))


CASES = [
    dict(name="unit scale, ties to even",
         why="amax = 7 so s = 7/7 = 1 exactly and v/s = v; rint sends 2.5->2, "
             "3.5->4, -2.5->-2, 0.5->0, 1.5->2, -0.5->0, 6.5->6, -6.5->-6",
         v=pad([7.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 6.5, -6.5, 0.0, 1.0, -3.0]),
         scale=1.0,
         codes=pad([7, 2, 4, -2, 0, 2, 0, 6, -6, 0, 1, -3])),
    dict(name="negative amax lane",
         why="amax = |-7| = 7, s = 1; the -7 lane maps to -7, 3.5 -> 4",
         v=pad([-7.0, 3.5, -4.5]), scale=1.0, codes=pad([-7, 4, -4])),
    dict(name="scale 2",
         why="amax = 14, s = 2; 14/2 = 7, -3/2 = -1.5 -> -2, 5/2 = 2.5 -> 2, "
             "1/2 = 0.5 -> 0, 3/2 = 1.5 -> 2, -13/2 = -6.5 -> -6",
         v=pad([14.0, -3.0, 5.0, 1.0, 3.0, -13.0]), scale=2.0,
         codes=pad([7, -2, 2, 0, 2, -6])),
    dict(name="all-zero group",
         why="amax = 0 so s = 0 and every code is 0 (no 0/0)",
         v=pad([]), scale=0.0, codes=pad([])),
    dict(name="amax/7 underflows to zero",
         why="amax = 3 * 2^-149; 3/7 of the smallest denormal rounds to 0, so "
             "the group is treated as all-zero",
         v=pad([3 * TINY, -TINY]), scale=0.0, codes=pad([])),
    dict(name="denormal scale, clamp at 7",
         why="amax = 8 * 2^-149; 8/7 = 1.14 rounds to s = 2^-149, so v/s = 8 "
             "clamps to 7, 4 * 2^-149 -> 4, -2^-149 -> -1",
         v=pad([8 * TINY, 4 * TINY, -TINY]), scale=TINY, codes=pad([7, 4, -1])),
    dict(name="denormal scale, clamp at -7",
         why="mirror of the previous case: -8 * 2^-149 / 2^-149 = -8 clamps to -7",
         v=pad([-8 * TINY, 4 * TINY, TINY]), scale=TINY, codes=pad([-7, 4, 1])),
]

CASES8 = [
    dict(name="8-bit: unit scale, ties to even",
         why="amax = 127 so s = 127/127 = 1 exactly and v/s = v; rint sends 2.5->2, "
             "3.5->4, 126.5->126, -126.5->-126, -0.5->0, 64.5->64",
         v=pad([127.0, 2.5, 3.5, 126.5, -126.5, -0.5, 64.5, -100.0]),
         scale=1.0, codes=pad([127, 2, 4, 126, -126, 0, 64, -100])),
    dict(name="8-bit: scale 2",
         why="amax = 254, s = 2; -254/2 = -127, 3/2 = 1.5 -> 2, 5/2 = 2.5 -> 2, 253/2 = 126.5 -> 126",
         v=pad([-254.0, 3.0, 5.0, 253.0]), scale=2.0, codes=pad([-127, 2, 2, 126])),
    dict(name="8-bit: amax/127 underflows to zero",
         why="amax = 63 * 2^-149; 63/127 < 1/2 of the smallest denormal rounds to 0",
         v=pad([63 * TINY, -TINY]), scale=0.0, codes=pad([])),
    dict(name="8-bit: denormal scale, clamp at -127",
         why="amax = 128 * 2^-149; 128/127 rounds to s = 2^-149, so -128 clamps to -127",
         v=pad([-128 * TINY, 5 * TINY]), scale=TINY, codes=pad([-127, 5])),
]

PACK8 = [
    dict(q=[-1, 127, -127, 0], bytes=[0xFF, 0x7F, 0x81, 0x00],
         why="one two's-complement byte per code"),
]

PACK = [
    dict(q=[1, -1], byte=0xF1, why="low nibble 0x1, high nibble -1 = 0xF"),
    dict(q=[-7, 7], byte=0x79, why="-7 = 0x9 low, 7 high"),
    dict(q=[-1, 0], byte=0x0F, why="-1 = 0xF low, 0 high"),
    dict(q=[0, -1], byte=0xF0, why="0 low, 0xF high"),
    dict(q=[7, -7], byte=0x97, why="7 low, -7 = 0x9 high"),
    dict(q=[0, 0], byte=0x00, why="zero"),
]

BF16 = [
    dict(f32=0x3F800000, bf16=0x3F80, why="1.0 is exact"),
    dict(f32=0x3F808000, bf16=0x3F80, why="1 + 2^-8 is a tie; 0x3F80 is even"),
    dict(f32=0x3F818000, bf16=0x3F82, why="tie with odd kept part rounds up"),
    dict(f32=0x3F808001, bf16=0x3F81, why="just above the tie rounds up"),
    dict(f32=0x3F807FFF, bf16=0x3F80, why="just below the tie rounds down"),
    dict(f32=0xBF818000, bf16=0xBF82, why="negative tie, odd kept part: away from zero"),
    dict(f32=0x3F7FFFFF, bf16=0x3F80, why="rounding up carries into the exponent"),
    dict(f32=0x7F7FFFFF, bf16=0x7F80, why="FLT_MAX is past the last bf16 midpoint: +inf"),
    dict(f32=0x00018000, bf16=0x0002, why="denormal tie with odd kept part rounds up"),
    dict(f32=0x00008000, bf16=0x0000, why="denormal tie with even kept part rounds down"),
    dict(f32=0x80000000, bf16=0x8000, why="-0 stays -0"),
]


def main():
    out = dict(
        source="hand-derived; readings of the pages' 4-bit group quantization "
               "('Tensor-parallel traffic drops to 4 bits', Interpretation; "
               "'Echo: Error-Compensated 4-Bit Tensor-Parallel Communication', Abstract)",
        quantizer=[dict(name=c["name"], why=c["why"], v=[float(t).hex() for t in c["v"]],
                        scale=float(c["scale"]).hex(), codes=c["codes"]) for c in CASES],
        quantizer8=[dict(name=c["name"], why=c["why"], v=[float(t).hex() for t in c["v"]],
                         scale=float(c["scale"]).hex(), codes=c["codes"]) for c in CASES8],
        pack=PACK, pack8=PACK8, bf16=BF16)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quantizer_hand_cases.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path)


if __name__ == "__main__":
    main()
