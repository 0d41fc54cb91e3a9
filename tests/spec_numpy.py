"""A second, independent implementation of the Fused-Softmax forward pass for
tiny inputs, written from the method description ("Fused-Softmax shifts an AI
attention bottleneck onto faster GPU hardware", paragraphs 5-6) with exact
rational arithmetic (``fractions.Fraction``).  It shares no code with the C
oracle: its number formats are built by enumerating the representable grid and
rounding by nearest-neighbour search, its scores are exact rationals, and every
binary32 rounding is done from the rational value directly.  Used only to pin
the oracle on tiny cases (every key, every element checked).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

# (exponent bits, mantissa bits, bias, top-binade mantissa fields usable)
_FORMATS = {
    0: (4, 3, 7, "e4m3"),
    1: (5, 2, 15, "e5m2"),
    2: (2, 3, 1, "e2m3"),
    3: (3, 2, 3, "e3m2"),
    4: (2, 1, 1, "e2m1"),
}


def grid(elem: int) -> list[tuple[Fraction, int]]:
    """All finite non-negative values of the format with their codes, sorted."""
    eb, mb, bias, name = _FORMATS[elem]
    out = []
    for E in range(1 << eb):
        for M in range(1 << mb):
            code = (E << mb) | M
            if name == "e4m3" and E == (1 << eb) - 1 and M == (1 << mb) - 1:
                continue  # NaN
            if name == "e5m2" and E == (1 << eb) - 1:
                continue  # Inf/NaN
            if E == 0:
                v = Fraction(M, 1 << mb) * Fraction(2) ** (1 - bias)
            else:
                v = (1 + Fraction(M, 1 << mb)) * Fraction(2) ** (E - bias)
            out.append((v, code))
    out.sort()
    return out


_GRIDS = {e: grid(e) for e in _FORMATS}


def value(elem: int, code: int) -> Fraction:
    eb, mb, _, _ = _FORMATS[elem]
    sign = (code >> (eb + mb)) & 1
    mag = code & ((1 << (eb + mb)) - 1)
    for v, c in _GRIDS[elem]:
        if c == mag:
            return -v if sign else v
    raise ValueError("NaN/Inf code")


def encode(elem: int, x: Fraction, neg_zero: bool = False) -> int:
    """Nearest grid value, ties to the even code; beyond the largest value -> largest."""
    eb, mb, _, _ = _FORMATS[elem]
    g = _GRIDS[elem]
    a = abs(x)
    sign = 1 if (x < 0 or (x == 0 and neg_zero)) else 0
    if a >= g[-1][0]:
        c = g[-1][1]
    else:
        # locate bracketing pair
        lo = max(i for i, (v, _) in enumerate(g) if v <= a)
        vlo, clo = g[lo]
        vhi, chi = g[lo + 1]
        if a - vlo < vhi - a:
            c = clo
        elif a - vlo > vhi - a:
            c = chi
        else:
            c = clo if clo % 2 == 0 else chi
    return (sign << (eb + mb)) | c


def scale_code(elem: int, amax: Fraction) -> int:
    """Smallest power of two X = 2^(code-127) with amax / X <= largest value."""
    if amax == 0:
        return 0
    top = _GRIDS[elem][-1][0]
    k = -200
    while amax / Fraction(2) ** k > top:
        k += 1
    while k > -200 and amax / Fraction(2) ** (k - 1) <= top:
        k -= 1
    return min(max(k + 127, 0), 254)


def mx_block(elem: int, xs: list[Fraction]) -> tuple[list[int], int]:
    amax = max(abs(x) for x in xs)
    sc = scale_code(elem, amax)
    X = Fraction(2) ** (sc - 127)
    return [encode(elem, x / X) for x in xs], sc


def fl32(x: Fraction) -> Fraction:
    """Round a rational to the nearest binary32 value, ties to even."""
    if x == 0:
        return Fraction(0)
    s = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 23)
    n = a / q
    f = math.floor(n)
    r = n - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return s * f * q


def bf16_value(pattern: int) -> Fraction:
    E = (pattern >> 7) & 0xFF
    M = pattern & 0x7F
    if E == 0:
        return Fraction(M, 128) * Fraction(2) ** (-126)
    return (1 + Fraction(M, 128)) * Fraction(2) ** (E - 127)


def bf16_bits_to_fraction(u16: np.ndarray) -> list[Fraction]:
    f32 = (u16.astype(np.uint32) << 16).view(np.float32)
    return [Fraction(float(v)) for v in f32.ravel()]


def operands(qb, kb, vb, sigma: float, qk_elem: int, v_elem: int):
    """Exact values of the quantized operands of one head: Q' = fl32(alpha q)
    quantized along D, K along D, V along keys (zero padded to a multiple of
    32 keys).  Returns (Qh [Sq][D], Kh [Skv][D], Vh [S32][D]) as Fractions."""
    Sq, D = qb.shape
    Skv = kb.shape[0]
    S32 = (Skv + 31) // 32 * 32
    alpha = fl32(Fraction(128.0 * math.log2(math.e) * sigma))
    Q = [bf16_bits_to_fraction(qb[i]) for i in range(Sq)]
    K = [bf16_bits_to_fraction(kb[i]) for i in range(Skv)]
    V = [bf16_bits_to_fraction(vb[i]) for i in range(Skv)]

    def quant_rows(rows):
        out = []
        for r in rows:
            vals = []
            for g in range(D // 32):
                codes, sc = mx_block(qk_elem, r[g * 32:(g + 1) * 32])
                X = Fraction(2) ** (sc - 127)
                vals += [value(qk_elem, cc) * X for cc in codes]
            out.append(vals)
        return out
    Qh = quant_rows([[fl32(alpha * x) for x in r] for r in Q])
    Kh = quant_rows(K)
    Vh = [[Fraction(0)] * D for _ in range(S32)]
    for d in range(D):
        col = [V[k][d] if k < Skv else Fraction(0) for k in range(S32)]
        for g in range(S32 // 32):
            codes, sc = mx_block(v_elem, col[g * 32:(g + 1) * 32])
            X = Fraction(2) ** (sc - 127)
            for j in range(32):
                Vh[g * 32 + j][d] = value(v_elem, codes[j]) * X
    return Qh, Kh, Vh


def references(qb, kb, vb, sigma: float, qk_elem: int, v_elem: int, p_elem: int):
    """Conventional softmax on the same quantized operands, one head, every
    query row ("conventional softmax on the same quantized operands" of the
    pages' error claim).  The exact scores s = sum_d Qh Kh / 128 are in log2
    units (Q carries 128 log2(e) sigma); p = 2^(s - max s) is evaluated in
    binary64 from the exactly rounded exponent.  Returns three [Sq][D] arrays:
      R1   sum p V / sum p                   (P unquantized)
      R2   sum MX(p) V / sum p               (numerator with P quantized like the
                                              method's P: 32 consecutive keys per
                                              block, fit-max E8M0, keys past Skv 0)
      R2'  sum MX(p) V / sum MX(p)
    with numerators and denominators accumulated exactly."""
    Sq, D = qb.shape
    Skv = kb.shape[0]
    S32 = (Skv + 31) // 32 * 32
    Qh, Kh, Vh = operands(qb, kb, vb, sigma, qk_elem, v_elem)
    out = {name: np.zeros((Sq, D)) for name in ("R1", "R2", "R2'")}
    for i in range(Sq):
        s = [sum(a * b for a, b in zip(Qh[i], Kh[k])) / 128 for k in range(Skv)]
        m = max(s)
        p = [Fraction(2.0 ** float(x - m)) for x in s] + [Fraction(0)] * (S32 - Skv)
        ph = []
        for g in range(S32 // 32):
            codes, sc = mx_block(p_elem, p[g * 32:(g + 1) * 32])
            X = Fraction(2) ** (sc - 127)
            ph += [value(p_elem, cc) * X for cc in codes]
        num_p = [sum(p[k] * Vh[k][d] for k in range(S32)) for d in range(D)]
        num_q = [sum(ph[k] * Vh[k][d] for k in range(S32)) for d in range(D)]
        den_p, den_q = sum(p), sum(ph)
        out["R1"][i] = [float(x / den_p) for x in num_p]
        out["R2"][i] = [float(x / den_p) for x in num_q]
        out["R2'"][i] = [float(x / den_q) for x in num_q]
    return out


def forward(qb, kb, vb, sigma: float, qk_elem: int, v_elem: int, p_elem: int, tau: float = 8.0,
            kv_tile: int = 64, c: float = 0.0, visible=None, t_out=None):
    """Tiny forward for one head.  qb [Sq,D], kb/vb [Skv,D] uint16 bf16 bit patterns.
    visible: optional [Sq] number of keys row i sees (keys 0 .. visible[i]-1);
    the others are absent (no part in any maximum, P = 0); a row that sees no
    key gives O = 0.  t_out: optional [Sq, Skv] array receiving the folded
    scores stage 1 sees (after each tile's gate shift).
    Returns (O [Sq,D] float, counts [Sq], P codes [Sq,Skv32], P scales [Sq,Skv32/32])."""
    Sq, D = qb.shape
    Skv = kb.shape[0]
    S32 = (Skv + 31) // 32 * 32
    Qh, Kh, Vh = operands(qb, kb, vb, sigma, qk_elem, v_elem)
    T0 = fl32(Fraction(128 * 127) - Fraction(c))
    Tg = fl32(Fraction(128) * (127 + Fraction(tau)) - Fraction(c))
    O = np.zeros((Sq, D))
    counts = np.zeros(Sq, np.int32)
    pcodes = np.zeros((Sq, S32), np.int64)
    pscales = np.zeros((Sq, S32 // 32), np.int64)
    for i in range(Sq):
        n_i = Skv if visible is None else max(0, min(Skv, int(visible[i])))
        if n_i == 0:
            continue
        ntiles = (n_i + kv_tile - 1) // kv_tile
        sig = [sum(a * b for a, b in zip(Qh[i], Kh[k])) for k in range(n_i)]
        num = [Fraction(0)] * D
        den = Fraction(0)
        C = Fraction(0)
        for j in range(ntiles):
            ks = list(range(j * kv_tile, min((j + 1) * kv_tile, n_i)))
            if j == 0:
                t = {k: fl32(sig[k]) for k in ks}
                C = fl32(T0 - max(t.values()))
                t = {k: fl32(t[k] + C) for k in ks}
            else:
                t = {k: fl32(C + sig[k]) for k in ks}
                mx = max(t.values())
                if mx > Tg:
                    delta = fl32(mx - T0)
                    t = {k: fl32(t[k] - delta) for k in ks}
                    C = fl32(C - delta)
                    rho = 2.0 ** (-float(delta) / 128.0)
                    num = [x * Fraction(rho) for x in num]
                    den = den * Fraction(rho)
                    counts[i] += 1
            if t_out is not None:
                for k in ks:
                    t_out[i, k] = float(t[k])
            # stage 1 (integer part of the folded score as a BF16 pattern) and stage 2 (MX)
            hi = min((j + 1) * kv_tile, S32)
            pvals = {}
            for k in range(j * kv_tile, hi):
                if k < n_i and t[k] >= 128:
                    pvals[k] = bf16_value(min(math.floor(t[k]), 0x7F7F))
                else:
                    pvals[k] = Fraction(0)
            for g in range(j * kv_tile // 32, hi // 32):
                blk = [pvals[k] for k in range(g * 32, g * 32 + 32)]
                codes, sc = mx_block(p_elem, blk)
                pscales[i, g] = sc
                X = Fraction(2) ** (sc - 127)
                for jj in range(32):
                    k = g * 32 + jj
                    pcodes[i, k] = codes[jj]
                    ph = value(p_elem, codes[jj]) * X
                    if ph:
                        for d in range(D):
                            num[d] += ph * Vh[k][d]
                        den += ph
        O[i] = [float(x / den) for x in num]
    return O, counts, pcodes, pscales
