"""Shared helpers of the GPU parity tests: moving bit patterns to and from the device, and the
acceptance rules.

Acceptance (every floating-point output, element by element):

* ``max |gpu - oracle| <= TOL * rms(oracle)`` (TOL = 2e-2, float32 accumulation), and
* a bf16 output equals the oracle's bits, or is a *rounding straddle*: the float32 sum the GPU
  rounds and the exact sum the oracle rounds lie on either side of a bf16 rounding boundary.
  Such an output is accepted only if it is the bf16 rounding of some value within the stated
  accumulation-error bound of the oracle's exact (pre-rounding) value; every other output must
  match bit for bit.
* float32 outputs are also held, element by element, to that accumulation-error bound.

Accumulation-error bound (``acc_bound``): ``|a - v| <= c * sum_k |x_k w_k| + 2^-23 |v|`` between
the GPU's float32 sum ``a`` and the exact sum ``v`` (bias included in both sums). The worst case
of float32 summation, ``K * 2^-24 * sum|x w|``, is wider than a bf16 unit at these K and would
accept anything; the kernels add the products in increasing K, 16 (bf16) or 64 (E4M3) per
matrix instruction into one float32 accumulator, whose running sums stay far below
``sum|x w|``. ``c = 2^-20`` for the bf16 matrix instructions and ``C_FP8`` for the E4M3 ones
(their 64 products are summed at reduced precision inside the instruction).
"""
import numpy as np
import torch

import oracle

TOL = 2e-2  # max |gpu - oracle| <= TOL * rms(oracle) for floating-point outputs (fp32 accumulation)
U32 = 2.0 ** -24   # unit roundoff of float32
C_BF16 = 2.0 ** -20
C_FP8 = 2.0 ** -16
GELU_SLOPE = 1.13  # max |GELU'(a)| = 1.1289 at a = 2.2
STRADDLE_SHARE = 1e-2  # sanity cap on the share of outputs that straddle (expected: ~1e-4)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes)).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def as_f64(a) -> np.ndarray:
    a = np.asarray(a)
    return oracle.bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def err_ratio(gpu, ref) -> float:
    """max |gpu - ref| / rms(ref), both given as bf16 bits or float arrays."""
    g, r = as_f64(gpu), as_f64(ref)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    return float(np.max(np.abs(g - r), initial=0.0)) / (rms if rms > 0 else 1.0)


def assert_close(gpu, ref, tol=TOL, what=""):
    """max |gpu - ref| <= tol * rms(ref) (the float tolerance alone)."""
    e = err_ratio(gpu, ref)
    assert e <= tol, f"{what}: max|err|/rms = {e:.3e} > {tol}"
    return e


# --- sums of |x w| for the accumulation bound --------------------------------------------------

class AbsSums:
    """``sum_k |x[m,k] w[n,k]| (+ |b[n]|)`` of a linear layer, computed for given (row, column)
    pairs on demand (``pairs``) or for whole row blocks (``block``)."""

    def __init__(self, x, w, bias=None, x_scale=None, w_scale=None):
        self.x, self.w = np.abs(x), np.abs(w)
        self.b = None if bias is None else np.abs(bias)
        self.xs = None if x_scale is None else np.abs(np.asarray(x_scale, np.float64))
        self.ws = None if w_scale is None else np.abs(np.asarray(w_scale, np.float64))

    @classmethod
    def bf16(cls, x_bits, w_bits, bias_bits=None):
        b = None if bias_bits is None else oracle.bf16_to_f64(bias_bits)
        return cls(oracle.bf16_to_f64(x_bits), oracle.bf16_to_f64(w_bits), b)

    @classmethod
    def fp8(cls, xq, x_scale, wq, w_scale, bias_bits=None):
        b = None if bias_bits is None else oracle.bf16_to_f64(bias_bits)
        return cls(oracle.e4m3_to_f64(xq), oracle.e4m3_to_f64(wq), b, x_scale, w_scale)

    def pairs(self, rows, cols, row0=0):
        rows, cols = np.asarray(rows) + row0, np.asarray(cols)
        s = np.zeros(rows.size)
        for i in range(0, rows.size, 4096):
            r, c = rows[i:i + 4096], cols[i:i + 4096]
            t = np.einsum("ik,ik->i", self.x[r], self.w[c])
            if self.xs is not None:
                t = t * self.xs[r] * self.ws[c]
            s[i:i + 4096] = t
        return s + (0.0 if self.b is None else self.b[cols])

    def block(self, r0, r1):
        s = self.x[r0:r1] @ self.w.T
        if self.xs is not None:
            s = s * self.xs[r0:r1, None] * self.ws[None, :]
        return s + (0.0 if self.b is None else self.b[None, :])


def acc_bound(abs_sums, v, c=C_BF16):
    """The stated bound on |GPU float32 sum - exact sum|."""
    return c * abs_sums + 2.0 ** -23 * np.abs(v)


def _bf16_value(v64):
    """Value of the bf16 rounding (float32 first, as the method rounds) of float64 values."""
    return oracle.bf16_to_f64(oracle.bf16_round(oracle.f32(v64)))


def check_bf16(gpu_bits, ref_bits, exact, abs_sums, c=C_BF16, gelu=False, extra=None, what="", tol=TOL,
               row0=0, share=STRADDLE_SHARE):
    """Element-wise acceptance of bf16 outputs of a linear layer (``gpu_bits``, ``ref_bits``
    ``[rows, cols]``), given the oracle's exact sums ``exact`` (float64, same shape, bias
    included) and an ``AbsSums`` for the bound. With ``gelu`` the output is GELU of the sum: the
    bound is carried through GELU's slope, plus 8 float32 units for its evaluation. ``extra``
    (same shape, optional) widens the window where an input of the GPU differs from the
    oracle's by a known amount. Returns the number of straddles.

    Every other output equals the oracle's bits, so it meets the float tolerance; a validated
    straddle is a correct rounding of an admissible sum and is accepted even where one unit of a
    large output exceeds ``tol * rms`` (heavy-tailed GELU and SwiGLU outputs)."""
    g, r = np.asarray(gpu_bits), np.asarray(ref_bits)
    assert g.shape == r.shape == np.shape(exact), what
    diff = np.argwhere(g != r)
    assert diff.shape[0] <= max(4, share * g.size), f"{what}: {diff.shape[0]} of {g.size} outputs differ"
    if diff.shape[0]:
        ri, ci = diff[:, 0], diff[:, 1]
        v = np.asarray(exact)[ri, ci]
        e = acc_bound(abs_sums.pairs(ri, ci, row0), v, c)
        if gelu:
            p = oracle.gelu_erf(oracle.f32(v))
            e = GELU_SLOPE * (e + U32 * np.abs(v)) + 8 * U32 * np.abs(p)
        else:
            p = v
        if extra is not None:
            e = e + np.abs(np.asarray(extra)[ri, ci])
        lo, hi = _bf16_value(p - e), _bf16_value(p + e)
        got = oracle.bf16_to_f64(g[ri, ci])
        bad = ~((got >= lo) & (got <= hi))
        if bad.any():
            k = int(np.argmax(bad))
            raise AssertionError(
                f"{what}: {int(bad.sum())} of {diff.shape[0]} differing outputs are not rounding straddles; first at "
                f"({ri[k] + row0}, {ci[k]}): gpu {got[k]!r}, oracle {oracle.bf16_to_f64(r[ri[k], ci[k]])!r}, exact "
                f"{p[k]!r}, window {e[k]:.3g}")
    same = g == r
    assert_close(np.where(same, g, r), r, tol, what)
    return int(diff.shape[0])


def check_f32(gpu, exact, abs_sums_block, c=C_BF16, what="", tol=TOL, ref=None, extra=None):
    """Element-wise acceptance of float32 outputs: within the accumulation bound of the exact
    sums everywhere (``abs_sums_block`` is the full ``sum|x w|`` array of the block), and the
    float tolerance against the oracle's float32 output ``ref`` (default: f32(exact)).
    ``extra`` widens the bound where the GPU's input differed from the oracle's by accepted
    straddles (``sum_k |d_k w_k|`` of those differences). Returns the largest
    ``|gpu - exact| / sum|x w|`` (the measured accumulation error against the bound's scale)."""
    g = np.asarray(gpu, dtype=np.float64)
    v = np.asarray(exact, dtype=np.float64)
    e = acc_bound(np.asarray(abs_sums_block), v, c)
    if extra is not None:
        e = e + np.asarray(extra)
    over = np.abs(g - v) > e
    if over.any():
        k = np.unravel_index(int(np.argmax(over)), g.shape)
        raise AssertionError(f"{what}: {int(over.sum())} float32 outputs beyond the accumulation bound; first at "
                             f"{k}: gpu {g[k]!r}, exact {v[k]!r}, bound {e[k]:.3g}")
    assert_close(g, oracle.f32(v) if ref is None else ref, tol, what)
    a = np.asarray(abs_sums_block, dtype=np.float64)
    return float(np.max(np.abs(g - v) / np.where(a > 0, a, 1.0), initial=0.0))


def argmax_ok(gpu_idx, ref_logits, tol=TOL):
    """Exact argmax, except rows whose top-2 oracle logits are closer than tol*rms: there any
    index whose oracle logit is within that tolerance of the maximum is accepted."""
    ref = np.asarray(ref_logits, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    want = np.argmax(ref, axis=1)
    bad = []
    for b, i in enumerate(np.asarray(gpu_idx)):
        if i == want[b]:
            continue
        top = ref[b, want[b]]
        if not (0 <= i < ref.shape[1]) or top - ref[b, i] > tol * rms:
            bad.append((b, int(i), int(want[b])))
    return bad


SWISH_ARGMIN = -1.2784645427610737  # swish(v) = v / (1 + e^-v) is smallest here (value -0.2784645)


def swish_range(lo, hi):
    """[min, max] of the Swish over the real intervals [lo, hi] (element-wise)."""
    a, b = oracle.swish(lo), oracle.swish(hi)
    mn = np.where((lo <= SWISH_ARGMIN) & (hi >= SWISH_ARGMIN), oracle.swish(np.float64(SWISH_ARGMIN)), np.minimum(a, b))
    return mn, np.maximum(a, b)


def check_swiglu(gpu_bits, ref_bits, gate_v, value_v, gate_sums, value_sums, c=C_BF16, what="", tol=TOL, row0=0,
                 share=STRADDLE_SHARE):
    """Element-wise acceptance of SwiGLU outputs ``y = bf16(swish(bf16(gate)) * bf16(value))``
    (evaluated in float32) ``[rows, cols]``: the oracle's bits, or the rounding (within 8 float32
    units of evaluation error) of ``swish(g) * u`` for some bf16 gate ``g`` and value ``u`` that are
    roundings of values within the accumulation bound of the exact sums ``gate_v``, ``value_v``
    (``AbsSums`` ``gate_sums``, ``value_sums`` over the gate and value weight rows); the set of
    such products is enclosed by interval arithmetic over [bf16(v - e), bf16(v + e)] for both.
    Returns the number of outputs that differ from the oracle's."""
    g, r = np.asarray(gpu_bits), np.asarray(ref_bits)
    assert g.shape == r.shape == np.shape(gate_v) == np.shape(value_v), what
    diff = np.argwhere(g != r)
    assert diff.shape[0] <= max(4, share * g.size), f"{what}: {diff.shape[0]} of {g.size} outputs differ"
    if diff.shape[0]:
        ri, ci = diff[:, 0], diff[:, 1]
        got = oracle.bf16_to_f64(g[ri, ci])

        def rounding_range(v, e):
            # the bf16 values the GPU may hold lie in [bf16(v - e), bf16(v + e)]
            return _bf16_value(v - e), _bf16_value(v + e)

        gv, uv = np.asarray(gate_v)[ri, ci], np.asarray(value_v)[ri, ci]
        g_lo, g_hi = rounding_range(gv, acc_bound(gate_sums.pairs(ri, ci, row0), gv, c))
        u_lo, u_hi = rounding_range(uv, acc_bound(value_sums.pairs(ri, ci, row0), uv, c))
        s_lo, s_hi = swish_range(g_lo, g_hi)
        prods = np.stack([s_lo * u_lo, s_lo * u_hi, s_hi * u_lo, s_hi * u_hi])
        p_lo, p_hi = prods.min(axis=0), prods.max(axis=0)
        e = 8 * U32 * np.maximum(np.abs(p_lo), np.abs(p_hi)) + 2.0 ** -140
        ok = (got >= _bf16_value(p_lo - e)) & (got <= _bf16_value(p_hi + e))
        if not ok.all():
            k = int(np.argmin(ok))
            raise AssertionError(f"{what}: {int((~ok).sum())} of {ri.size} differing SwiGLU outputs are not roundings "
                                 f"of admissible gate/value pairs; first at ({ri[k] + row0}, {ci[k]}): gpu {got[k]!r}, "
                                 f"oracle {oracle.bf16_to_f64(r[ri[k], ci[k]])!r}, gate {gv[k]!r}, value {uv[k]!r}")
    same = g == r
    assert_close(np.where(same, g, r), r, tol, what)
    return int(diff.shape[0])


def check_rmsnorm_rows(xn_gpu, x, s, r0=0):
    """The GPU's normalised rows equal the oracle's, except rows whose factor r took the other
    float32 rounding where that is admissible. The GPU sums the exact squares in float64 (K / 256
    values per thread, then a tree), then divides, adds eps, takes the square root and the
    reciprocal in float64: its unrounded factor is within (K / 512 + 8) 2^-53 of the exact one
    (relative), and the oracle's float64 factor within (log2 K + 4) 2^-53. So the other rounding
    is admissible only when the oracle's factor lies within (K / 256 + 32) 2^-53 of the midpoint
    between the two float32 values. Returns ``(oracle rows, {row: r})`` for the rows that took it."""
    ref, r_o = oracle.rmsnorm(x, s)
    err = (x.shape[1] / 256 + 32) * 2.0 ** -53
    bad = np.nonzero(np.any(xn_gpu != ref, axis=1))[0]
    other = {}
    if bad.size:
        rho = oracle.rmsnorm_factor(x[bad])
        for i, b in enumerate(bad):
            found = None
            for dr in (-1, 1):
                cand = np.array([np.nextafter(r_o[b], np.float32(np.inf) if dr > 0 else np.float32(-np.inf))],
                                dtype=np.float32)
                mid = (float(cand[0]) + float(r_o[b])) / 2.0
                if abs(mid - rho[i]) > err * rho[i]:
                    continue
                y, _ = oracle.rmsnorm(x[b:b + 1], s, r=cand)
                if np.array_equal(y[0], xn_gpu[b]):
                    found = cand
            assert found is not None, f"normalised row {r0 + b} is not the oracle's for any admissible factor"
            other[int(b)] = found
    return ref, other


def admissible_rows(xn_ref, other, x, s):
    """The oracle's normalised rows, with the rows in ``other`` (``check_rmsnorm_rows``) taken
    with their other admissible factor."""
    a = xn_ref.copy()
    for b, r in other.items():
        a[b] = oracle.rmsnorm(x[b:b + 1], s, r=r)[0][0]
    return a
