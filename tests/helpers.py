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


def assert_close(gpu, ref, tol=TOL, what=""):
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
