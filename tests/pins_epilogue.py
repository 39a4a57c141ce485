"""Pins of the oracle's multi-step epilogue ("The Graph IR", op table:
ContractionEpilogue; the activation compositions of "Tracing a Model").

Nothing here re-types the oracle's chains.  The primitives are checked against
independent high-precision evaluations over every element-type input: exp from
Python's decimal module, erf from its Taylor series in decimal arithmetic with
pi from Machin's formula, and the rounding to the element type done in exact
rational arithmetic.  The activation chains are held to the exact mathematical
function (SiLU, the tanh-form GeLU, the erf GeLU) within a rounding-error bound
derived from the chain, and where exp overflows in the element type the
composition's IEEE result (a signed zero) is required.  The binary steps are
compared with the exact operation rounded once.
"""
from __future__ import annotations

import concurrent.futures
import math
import multiprocessing
from decimal import Decimal, getcontext, localcontext
from fractions import Fraction

import numpy as np

import oracle
from oracle import tolerance

ELEMS = (tolerance.F16, tolerance.BF16)
P_BITS = {tolerance.F16: 11, tolerance.BF16: 8}
EMIN = {tolerance.F16: -14, tolerance.BF16: -126}
MAXV = {tolerance.F16: Fraction(65504), tolerance.BF16: Fraction(2 ** 8 - 1, 2 ** 7) * Fraction(2) ** 127}


def all_words() -> np.ndarray:
    return np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)


def values(words, elem) -> np.ndarray:
    return tolerance.words_to_f64(words, elem)


def encode(v: float, elem) -> int:
    """Word of an exactly representable element-type value (or +-inf)."""
    if elem == tolerance.F16:
        return int(np.array([v], np.float64).astype(np.float16).view(np.uint16)[0])
    return int(np.array([v], np.float32).view(np.uint32)[0] >> 16)


def round_exact(q: Fraction, elem) -> int:
    """Round an exact rational to the element type, ties to even (gradual underflow,
    overflow to infinity)."""
    if q == 0:
        return 0
    neg = q < 0
    a = -q if neg else q
    p = P_BITS[elem]
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, EMIN[elem])
    quantum = Fraction(2) ** (e - (p - 1))
    n = a / quantum
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    r = k * quantum
    if r > MAXV[elem]:
        w = encode(math.inf, elem)
    else:
        w = encode(float(r), elem)
    return w | 0x8000 if neg else w


def _pi(prec: int) -> Decimal:
    """pi by Machin's formula: 16 atan(1/5) - 4 atan(1/239)."""
    with localcontext() as ctx:
        ctx.prec = prec + 10

        def atan_inv(n):
            x = Decimal(1) / n
            x2 = x * x
            total, term, k, sign = Decimal(0), x, 1, 1
            while True:
                t = term / k
                if t == 0 or abs(t) < Decimal(10) ** (-(prec + 8)):
                    break
                total += sign * t
                term *= x2
                k += 2
                sign = -sign
            return total

        return +(16 * atan_inv(5) - 4 * atan_inv(239))


def erf_decimal(x: Decimal, prec: int = 90) -> Decimal:
    """erf by its Maclaurin series 2/sqrt(pi) sum (-1)^n x^(2n+1) / (n! (2n+1)) (|x| <= 6)."""
    with localcontext() as ctx:
        ctx.prec = prec
        x2 = x * x
        term = x            # (-1)^n x^(2n+1) / n!
        total = Decimal(0)
        n = 0
        while True:
            t = term / (2 * n + 1)
            total += t
            if t == 0 or abs(t) < abs(total) * Decimal(10) ** (-(prec - 5)):
                break
            n += 1
            term = -term * x2 / n
        return total * 2 / _pi(prec).sqrt()


def exp_rounded_reference(word: int, elem) -> int:
    v = float(values(np.array([word], np.uint16), elem)[0])
    if math.isnan(v):
        return -1
    if v > 100:
        return encode(math.inf, elem)
    if v < -120:
        return 0
    with localcontext() as ctx:
        ctx.prec = 60
        return round_exact(Fraction(Decimal(v).exp()), elem)


def erf_rounded_reference(word: int, elem) -> int:
    v = float(values(np.array([word], np.uint16), elem)[0])
    if math.isnan(v):
        return -1
    if abs(v) > 6:
        return encode(1.0 if v > 0 else -1.0, elem)
    if v == 0:
        return word                      # erf(+-0) = +-0
    return round_exact(Fraction(erf_decimal(Decimal(v))), elem)


def _refs(ref_fn, words, elem):
    return [ref_fn(int(x), elem) for x in words]


def _pool_map(fn, chunks):
    """fn over chunks in 8 spawned processes (the references are pure-Python
    decimal arithmetic; spawn, because the test process runs torch's threads)."""
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(8, mp_context=ctx) as ex:
        return list(ex.map(fn, *zip(*chunks)))


def _compare_unary(orc, op, ref_fn, elem):
    w = all_words()
    got = orc.unary(op, w, elem)
    parts = np.array_split(w, 64)
    wants = [x for part in _pool_map(_refs, [(ref_fn, part, elem) for part in parts]) for x in part]
    bad = []
    for i in range(w.size):
        want = wants[i]
        if want < 0:                     # NaN input
            assert np.isnan(values(got[i:i + 1], elem)[0]), hex(int(w[i]))
            continue
        g = int(got[i])
        if g != want and not (g & 0x7FFF == 0 and want & 0x7FFF == 0 and g == want):
            bad.append((hex(int(w[i])), hex(g), hex(want)))
    assert not bad, "%d mismatches, first %s" % (len(bad), bad[:5])


def pin_exp_every_input(orc):
    """exp rounded to the element type, every binary16 and bfloat16 word, against decimal exp."""
    for elem in ELEMS:
        _compare_unary(orc, oracle.UNARY_EXP, exp_rounded_reference, elem)


def pin_erf_every_input(orc):
    """erf rounded to the element type, every word, against the decimal Maclaurin series."""
    for elem in ELEMS:
        _compare_unary(orc, oracle.UNARY_ERF, erf_rounded_reference, elem)


def pin_f64_to_elem(orc, count: int = 20000, seed: int = 31):
    """Rounding doubles to the element type: random values over the whole range,
    exact midpoints between neighbours (ties), the subnormal range and the overflow
    threshold, against exact rational rounding."""
    rng = np.random.default_rng(seed)
    for elem in ELEMS:
        emin = EMIN[elem]
        emax = 16 if elem == tolerance.F16 else 128
        e = rng.integers(emin - 12, emax + 1, count)
        v = (rng.random(count) + 1.0) * np.ldexp(1.0, e) * np.where(rng.random(count) < 0.5, -1, 1)
        w = all_words()[rng.integers(0, 1 << 16, 2000)]
        vals = values(w, elem)
        nxt = values((w.astype(np.uint32) + 1).astype(np.uint16), elem)
        ok = np.isfinite(vals) & np.isfinite(nxt) & (np.sign(vals) == np.sign(nxt))
        with np.errstate(invalid="ignore"):
            mids = ((vals + nxt) / 2)[ok]        # exact in double (one extra bit)
        edge = [float(MAXV[elem]), float(MAXV[elem]) * (1 + 2.0 ** -(P_BITS[elem] + 1)),
                math.ldexp(1.0, emin - P_BITS[elem]), math.ldexp(1.0, emin - P_BITS[elem] + 1) * 0.75,
                0.0, -0.0]
        allv = np.concatenate([v, mids, np.array(edge)])
        got = orc.f64_to_elem(allv, elem)
        for i, x in enumerate(allv):
            want = round_exact(Fraction(float(x)), elem)
            if x == 0 and math.copysign(1, x) < 0:
                want = 0x8000
            assert int(got[i]) == want, (elem, float(x), hex(int(got[i])), hex(want))


def _bound_check(got_w, exact, bound, elem, what):
    g = values(got_w, elem)
    err = np.abs(g - exact)
    bad = ~(err <= bound)
    assert not bad.any(), "%s: %d outside the bound, e.g. got %r want %r (bound %r)" % (
        what, bad.sum(), g[bad][:3], exact[bad][:3], bound[bad][:3])


def _decimal_map(fn, xs, prec=40):
    out = np.empty(xs.size, np.float64)
    with localcontext() as ctx:
        ctx.prec = prec
        for i, x in enumerate(xs):
            out[i] = float(fn(Decimal(float(x))))
    return out


def pin_silu_chain_vs_math(orc):
    """SiLU composition against x / (1 + e^-x) over every finite input: within
    3 unit roundoffs plus half a subnormal quantum, except where e^-x overflows the
    element type, where the composition gives a signed zero."""
    for elem in ELEMS:
        w = all_words()
        x = values(w, elem)
        fin = np.isfinite(x)
        w, x = w[fin], x[fin]
        got = orc.unary(oracle.EPI_SILU, w, elem)
        e_w = orc.unary(oracle.UNARY_EXP, (w ^ 0x8000).astype(np.uint16), elem)   # exp(-x)
        over = np.isinf(values(e_w, elem))
        gv = values(got, elem)
        assert (gv[over] == 0).all(), "overflowed exp must give a signed zero"
        keep = ~over & (np.abs(x) < 1e30)
        exact = _decimal_map(lambda d: d / (1 + (-d).exp()), x[keep])
        u = 2.0 ** -P_BITS[elem]
        q = math.ldexp(1.0, EMIN[elem] - P_BITS[elem] + 1)
        _bound_check(got[keep], exact, 3.01 * u * np.abs(exact) + q, elem, "silu")


def pin_gelu_tanh_chain_vs_math(orc):
    """tanh-form GeLU composition against x / (1 + exp(-2 sqrt(2/pi) (x + 0.044715 x^3)))
    over every finite input with |x| <= 64: within (8 |z| + 4) unit roundoffs of the
    value plus a subnormal quantum (z the exponent), or a signed zero where the
    composition's exp overflows."""
    k = Decimal(2) / _pi(50)
    for elem in ELEMS:
        w = all_words()
        x = values(w, elem)
        keep = np.isfinite(x) & (np.abs(x) <= 64)
        w, x = w[keep], x[keep]
        got = orc.unary(oracle.EPI_GELU_TANH, w, elem)
        zs = _decimal_map(lambda d: -2 * k.sqrt() * (d + Decimal("0.044715") * d * d * d), x)
        exact = _decimal_map(lambda d: d / (1 + (-2 * k.sqrt() * (d + Decimal("0.044715") * d * d * d)).exp()), x)
        gv = values(got, elem)
        u = 2.0 ** -P_BITS[elem]
        q = math.ldexp(1.0, EMIN[elem] - P_BITS[elem] + 1)
        # where exp(z) is beyond the element type's range (exp(z) >= the overflow
        # threshold of rounding) the composition yields +-0; z itself carries up
        # to 8 |z| u of rounding error, so values that close to the threshold are
        # held to neither form
        thr = math.log(65520.0) if elem == tolerance.F16 else math.log(float(MAXV[elem]) * (1 + 2.0 ** -9))
        big = zs * (1 - 8 * u) > thr
        near = ~big & (zs * (1 + 8 * u) > thr)
        assert (gv[big] == 0).all(), "overflowed exp must give a signed zero"
        m = ~big & ~near
        _bound_check(got[m], exact[m], (8 * np.abs(zs[m]) + 4) * u * np.abs(exact[m]) + q, elem, "gelu_tanh")


def _gelu_erf_exact(xs):
    """x (1 + erf(x / sqrt 2)) / 2 in decimal, rounded to double, for each x."""
    s2 = Decimal(2).sqrt()
    out = []
    for xv in xs:
        d = Decimal(float(xv))
        s = d / s2
        ef = erf_decimal(s, 50) if abs(s) <= 6 else Decimal(1 if s > 0 else -1)
        out.append(float(d * (1 + ef) / 2))
    return out


def pin_gelu_erf_chain_vs_math(orc):
    """erf GeLU composition against x (1 + erf(x / sqrt 2)) / 2 over every finite input
    with |x| <= 64: absolute error within |x| u (0.8 |x| + 2.5) + a subnormal quantum."""
    for elem in ELEMS:
        w = all_words()
        x = values(w, elem)
        keep = np.isfinite(x) & (np.abs(x) <= 64)
        w, x = w[keep], x[keep]
        got = orc.unary(oracle.EPI_GELU_ERF, w, elem)
        parts = np.array_split(x, 64)
        ex = np.array([v for part in _pool_map(_gelu_erf_exact, [(part,) for part in parts]) for v in part])
        u = 2.0 ** -P_BITS[elem]
        q = math.ldexp(1.0, EMIN[elem] - P_BITS[elem] + 1)
        _bound_check(got, ex, np.abs(x) * u * (0.8 * np.abs(x) + 2.5) + q, elem, "gelu_erf")


def pin_binary_steps_vs_exact(orc, count: int = 1 << 14, seed: int = 32):
    """Bias and residual add and the multiply step: the exact sum or product of two
    element-type values rounded once (random words, all finite)."""
    rng = np.random.default_rng(seed)
    for elem in ELEMS:
        a = rng.integers(0, 1 << 16, count).astype(np.uint16)
        b = rng.integers(0, 1 << 16, count).astype(np.uint16)
        av, bv = values(a, elem), values(b, elem)
        ok = np.isfinite(av) & np.isfinite(bv)
        a, b, av, bv = a[ok], b[ok], av[ok], bv[ok]
        for op, fn in ((oracle.EPI_BIAS, lambda p, q: p + q), (oracle.EPI_RESIDUAL, lambda p, q: p + q),
                       (oracle.EPI_MUL, lambda p, q: p * q)):
            kw = {oracle.EPI_BIAS: "bias", oracle.EPI_RESIDUAL: "res", oracle.EPI_MUL: "mul"}[op]
            got = orc.epilogue([op], a, elem=elem, **{kw: b})
            for i in range(0, a.size, 7):
                want = round_exact(fn(Fraction(float(av[i])), Fraction(float(bv[i]))), elem)
                g = int(got[i])
                if want & 0x7FFF == 0 and g & 0x7FFF == 0:
                    continue                   # +0 / -0 of an exact zero sum
                assert g == want, (elem, op, float(av[i]), float(bv[i]), hex(g), hex(want))


def pin_step_order_and_composition(orc, seed: int = 33):
    """A program of several steps equals the steps applied one at a time, in order
    (bias, activation, residual, multiply), and the empty program is the identity."""
    rng = np.random.default_rng(seed)
    for elem in ELEMS:
        n = 4096
        t = rng.integers(0, 1 << 16, n).astype(np.uint16)
        b = rng.integers(0, 1 << 16, n).astype(np.uint16)
        r = rng.integers(0, 1 << 16, n).astype(np.uint16)
        u = rng.integers(0, 1 << 16, n).astype(np.uint16)
        fin = np.isfinite(values(t, elem)) & np.isfinite(values(b, elem)) & np.isfinite(values(r, elem)) \
            & np.isfinite(values(u, elem))
        t, b, r, u = t[fin], b[fin], r[fin], u[fin]
        assert np.array_equal(orc.epilogue([], t, elem=elem), t)
        for act in (oracle.EPI_SILU, oracle.EPI_GELU_TANH, oracle.EPI_GELU_ERF):
            prog = [oracle.EPI_BIAS, act, oracle.EPI_RESIDUAL, oracle.EPI_MUL]
            got = orc.epilogue(prog, t, bias=b, res=r, mul=u, elem=elem)
            s1 = orc.epilogue([oracle.EPI_BIAS], t, bias=b, elem=elem)
            s2 = orc.unary(act, s1, elem)
            s3 = orc.epilogue([oracle.EPI_RESIDUAL], s2, res=r, elem=elem)
            s4 = orc.epilogue([oracle.EPI_MUL], s3, mul=u, elem=elem)
            ok = (got == s4) | (np.isnan(values(got, elem)) & np.isnan(values(s4, elem)))
            assert ok.all()
            # a different order gives a different function (the order is observable)
            other = orc.epilogue([oracle.EPI_RESIDUAL, act, oracle.EPI_BIAS, oracle.EPI_MUL], t, bias=b, res=r,
                                 mul=u, elem=elem)
            assert (other != got).any()


def pin_special_values(orc):
    """Closed forms of the compositions at special inputs: silu(0) = 0, silu(+inf) =
    +inf, silu(-inf) is NaN (-inf / inf), gelu(0) = 0, gelu_erf(+inf) = +inf, NaN
    propagates through every step."""
    for elem in ELEMS:
        inf = encode(math.inf, elem)
        ninf = inf | 0x8000
        nan = 0x7E00 if elem == tolerance.F16 else 0x7FC0
        w = np.array([0, inf, ninf, nan], np.uint16)
        s = values(orc.unary(oracle.EPI_SILU, w, elem), elem)
        assert s[0] == 0 and s[1] == np.inf and np.isnan(s[2]) and np.isnan(s[3])
        g = values(orc.unary(oracle.EPI_GELU_TANH, w, elem), elem)
        assert g[0] == 0 and g[1] == np.inf and np.isnan(g[3])
        e = values(orc.unary(oracle.EPI_GELU_ERF, w, elem), elem)
        assert e[0] == 0 and e[1] == np.inf and np.isnan(e[3])
        one = encode(1.0, elem)
        for op in (oracle.EPI_BIAS, oracle.EPI_RESIDUAL, oracle.EPI_MUL):
            kw = {oracle.EPI_BIAS: "bias", oracle.EPI_RESIDUAL: "res", oracle.EPI_MUL: "mul"}[op]
            got = orc.epilogue([op], np.array([nan, one], np.uint16), elem=elem,
                               **{kw: np.array([one, nan], np.uint16)})
            assert np.isnan(values(got, elem)).all()


GOLDEN_DIR = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


def _golden_chains(orc, name, elem):
    """The hand-derived composition results of tests/golden/<name>: every line is
    `op x y`, x an element-type value, y the composition with every primitive
    rounded to the element type (derivations in the file)."""
    ops = {"silu": oracle.EPI_SILU, "gelu_tanh": oracle.EPI_GELU_TANH, "gelu_erf": oracle.EPI_GELU_ERF}
    n = 0
    for line in open(__import__("os").path.join(GOLDEN_DIR, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        op, x, y = line.split()
        w = np.array([encode(float(x), elem)], np.uint16)
        assert round_exact(Fraction(float(x)), elem) == int(w[0]), "fixture input not of the element type"
        assert round_exact(Fraction(float(y)), elem) == int(encode(float(y), elem)), "fixture result not of the element type"
        got = float(values(orc.unary(ops[op], w, elem), elem)[0])
        assert got == float(y), (op, x, got, y)
        n += 1
    return n


def pin_golden_chains_bf16(orc):
    """Hand-derived bfloat16 composition results (tests/golden/epilogue_chains_bf16.txt)
    where rounding every primitive changes the answer."""
    assert _golden_chains(orc, "epilogue_chains_bf16.txt", tolerance.BF16) == 6


def pin_golden_chains_f16(orc):
    """Hand-derived binary16 composition results (tests/golden/epilogue_chains_f16.txt)
    where rounding every primitive changes the answer; four of them turn on a tie
    at an intermediate step."""
    assert _golden_chains(orc, "epilogue_chains_f16.txt", tolerance.F16) == 6


# cheapest first: the mutation check stops at the first pin that fails
EPILOGUE_PINS = [
    pin_golden_chains_f16,
    pin_golden_chains_bf16,
    pin_f64_to_elem,
    pin_binary_steps_vs_exact,
    pin_step_order_and_composition,
    pin_special_values,
    pin_silu_chain_vs_math,
    pin_gelu_tanh_chain_vs_math,
    pin_exp_every_input,
    pin_gelu_erf_chain_vs_math,
    pin_erf_every_input,
]
