"""Print the double-double Taylor coefficients used by sad_crmath.h.

Each coefficient c is stored as (hi, lo): hi = c rounded to double, lo = c - hi
rounded to double, computed here in 300-bit arithmetic (mpmath).  Run from the
repository root and paste the output into sad_crmath.h:

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
