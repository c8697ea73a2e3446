"""Prints the constants of csrc/rtp_exp.h: 2^(j/256) for j = 0..255, each
rounded to the nearest double, and the range-reduction constants 256/ln 2
and ln2/256 split into a 34-bit head (so that n * head is exact for every
|n| < 2^19) and a tail.  Exact decimal arithmetic at 60 digits; Python's
float() of a decimal string rounds correctly.

    python gen_exp2_table.py
"""
from decimal import Decimal, getcontext

getcontext().prec = 60
LN2 = Decimal(2).ln()


def dbl(x: Decimal) -> float:
    return float(format(x, "e"))


def main() -> None:
    vals = [dbl((Decimal(j) / 256 * LN2).exp()) for j in range(256)]
    print("#define RTP_EXP2_TABLE" + " " * 66 + "\\")
    print("    {" + " " * 79 + "\\")
    for i in range(0, 256, 4):
        row = ", ".join(v.hex() for v in vals[i:i + 4])
        print(f"        {row}, \\")
    print("    }")
    step = LN2 / 256
    head = float((step * (Decimal(2) ** 42)).to_integral_value()) / 2.0 ** 42  # 34 bits
    tail = dbl(step - Decimal(head))
    print(f"kExpInvStep = {dbl(256 / LN2).hex()}")
    print(f"kExpStepHi  = {head.hex()}")
    print(f"kExpStepLo  = {tail.hex()}")


if __name__ == "__main__":
    main()
