"""Shared helpers of the GPU parity tests: moving bit patterns to and from the device, tolerances."""
import numpy as np
import torch

import oracle

TOL = 2e-2  # max |gpu - oracle| <= TOL * rms(oracle) for floating-point outputs (fp32 accumulation)


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
    rms = float(np.sqrt(np.mean(r * r)))
    return float(np.max(np.abs(g - r))) / (rms if rms > 0 else 1.0)


STRADDLE = 1e-3  # largest share of bf16 outputs allowed to sit one ulp from the oracle's


def assert_close(gpu, ref, tol=TOL, what="", straddle=STRADDLE, ulps=1):
    """max |gpu - ref| <= tol * rms(ref). For bf16 outputs (uint16 bits on both sides), an
    output exactly one unit in the last place from the oracle's is a second correct result:
    the float32 sum and the exact sum fell on either side of a bf16 rounding boundary. Such
    outputs may make up at most ``straddle`` of the elements; the bound applies to all others
    (one ulp of a large output can exceed tol * rms when the outputs are heavy-tailed).
    ``ulps`` > 1 widens that allowance where the method rounds to bf16 more than once on the
    way to an output, so that one straddled intermediate can move it by several ulps."""
    g, r = np.asarray(gpu), np.asarray(ref)
    if g.dtype == np.uint16 and r.dtype == np.uint16:
        same_sign = (g & 0x8000) == (r & 0x8000)
        d_bits = np.abs(g.astype(np.int32) - r.astype(np.int32))
        one_ulp = same_sign & (d_bits >= 1) & (d_bits <= ulps)
        n = int(np.count_nonzero(one_ulp))
        assert n <= straddle * g.size, f"{what}: {n} outputs 1..{ulps} ulp off (> {straddle} of {g.size})"
        rf = oracle.bf16_to_f64(r)
        rms = float(np.sqrt(np.mean(rf * rf)))
        d = np.abs(oracle.bf16_to_f64(g) - rf)
        e = float(np.max(np.where(one_ulp, 0.0, d), initial=0.0)) / (rms if rms > 0 else 1.0)
    else:
        e = err_ratio(gpu, ref)
    assert e <= tol, f"{what}: max|err|/rms = {e:.3e} > {tol}"
    return e


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
