"""Print the constants used by sad_crmath.h.

Each Taylor coefficient c is stored as (hi, lo): hi = c rounded to double,
lo = c - hi rounded to double, computed here in 300-bit arithmetic (mpmath).
The split constants of the double-precision argument reductions are printed
after the tables: ln 2 and pi/2 cut into leading parts with few significant
bits (so that k times them is exact for the multiples k that occur) and a
rounded remainder.  Run from the repository root and paste the output into
sad_crmath.h:

    python3 voronoi_rendering_amd/csrc/gen_crmath_coeffs.py
"""
import mpmath

mpmath.mp.prec = 300


def dd(c) -> str:
    hi = float(c)
    lo = float(c - mpmath.mpf(hi))
    return "{%s, %s}" % (hi.hex(), lo.hex())


def table(name: str, values, what: str) -> str:
    rows = ",\n".join("    " + dd(v) for v in values)
    return f"// {what}\nconstexpr dd {name}[{len(values)}] = {{\n{rows}}};\n"


print(table("EXP_C", [1 / mpmath.factorial(n) for n in range(21)], "1/n!, n = 0..20"))
print(table("SIN_C", [(-1) ** n / mpmath.factorial(2 * n + 1) for n in range(15)], "(-1)^n/(2n+1)!, n = 0..14"))
print(table("COS_C", [(-1) ** n / mpmath.factorial(2 * n) for n in range(15)], "(-1)^n/(2n)!, n = 0..14"))


def split(c, bits: int) -> tuple:
    """c rounded down to a double with at most `bits` significant bits, and the rest."""
    e = int(mpmath.floor(mpmath.log(abs(c), 2)))
    q = mpmath.floor(c * mpmath.mpf(2) ** (bits - 1 - e))
    head = q * mpmath.mpf(2) ** (e - bits + 1)
    assert float(head) == head
    return head, c - head


ln2 = mpmath.log(2)
l1, l_rest = split(ln2, 32)
print("// ln 2 = SAD_LN2_A + SAD_LN2_B + O(2^-85); SAD_LN2_A has 32 significant bits")
print(f"#define SAD_LN2_A {float(l1).hex()}")
print(f"#define SAD_LN2_B {float(l_rest).hex()}")
pio2 = mpmath.pi / 2
p1, rest = split(pio2, 33)
p2, rest = split(rest, 33)
print("// pi/2 = SAD_PIO2_A + SAD_PIO2_B + SAD_PIO2_C + O(2^-118); A and B have 33 significant bits")
print(f"#define SAD_PIO2_A {float(p1).hex()}")
print(f"#define SAD_PIO2_B {float(p2).hex()}")
print(f"#define SAD_PIO2_C {float(rest).hex()}")
print(f"// remainders: ln2 {float(l_rest - mpmath.mpf(float(l_rest)))!r}, pi/2 {float(rest - mpmath.mpf(float(rest)))!r}")
