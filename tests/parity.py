"""Host-side comparison rules for the GPU parity tests.

Tolerances (checked per output tensor):
  * integer and byte results (hash indices, gathered rows): bit-exact;
  * float32 path: max|gpu - ref| / max|ref| <= 1e-5 for kv, alpha and Y;
  * bfloat16 path: |d alpha| <= 2e-3 and max|dY| <= 1e-2 * RMS(Y_ref) on the
    float32 Y output; H_out, stored in bf16, must lie within half a bf16 ulp
    (of |H + Y_ref| + tol) plus the Y tolerance of H + Y_ref, since it is
    round(H + Y_gpu);
  * projections kv stored in bf16: within one bf16 half-ulp of the exact
    product plus float32 accumulation error.
"""
import sys

import numpy as np
import torch

F32_REL = 1e-5
BF16_ALPHA_ABS = 2e-3
BF16_Y_REL_RMS = 1e-2


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits_equal(gpu: np.ndarray, ref: np.ndarray) -> bool:
    """Value and sign equality (so -0.0 differs from +0.0)."""
    return bool(np.array_equal(gpu, ref) and np.array_equal(np.signbit(gpu), np.signbit(ref)))


def rel_max(gpu: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(gpu - ref))) / (den if den > 0 else 1.0)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def check_f32(name: str, gpu: np.ndarray, ref: np.ndarray, tol: float = F32_REL):
    r = rel_max(gpu, ref)
    assert r <= tol, f"{name}: max rel err {r:.3e} > {tol:.1e}"
    return r


def check_bf16_layer(alpha_gpu, alpha_ref, y_gpu, y_ref, h_gpu, h_in, tag=""):
    da = float(np.max(np.abs(alpha_gpu - alpha_ref)))
    assert da <= BF16_ALPHA_ABS, f"{tag} alpha err {da:.3e}"
    tol_y = BF16_Y_REL_RMS * float(np.sqrt(np.mean(y_ref ** 2)))
    dy = float(np.max(np.abs(y_gpu - y_ref)))
    assert dy <= tol_y, f"{tag} Y err {dy:.3e} > {tol_y:.3e}"
    target = h_in + y_ref
    bound = 0.5 * bf16_ulp(np.abs(target) + tol_y) + tol_y
    dh = np.abs(h_gpu - target)
    assert np.all(dh <= bound), f"{tag} H_out err {float(np.max(dh - bound)):.3e} over bound"
    log(f"{tag} margins: alpha {da / BF16_ALPHA_ABS:.3f}, Y {dy / max(tol_y, 1e-30):.3f} of the tolerance")
    return da, dy / max(tol_y, 1e-30)


def check_f32_layer(alpha_gpu, alpha_ref, y_gpu, y_ref, h_gpu, h_in, tag=""):
    check_f32(f"{tag} alpha", alpha_gpu, alpha_ref)
    check_f32(f"{tag} Y", y_gpu, y_ref)
    target = h_in + y_ref
    bound = F32_REL * float(np.max(np.abs(y_ref))) + np.abs(target) * 2.0 ** -23
    assert np.all(np.abs(h_gpu - target) <= bound), f"{tag} H_out"


def check_kv_bf16(gpu: np.ndarray, ref: np.ndarray, K: int, tag=""):
    """bf16 output of a float32-accumulated product: half a bf16 ulp plus a
    float32 accumulation allowance."""
    scale = float(np.sqrt(np.mean(ref ** 2)))
    acc = K * 2.0 ** -24 * scale
    bound = 0.5 * bf16_ulp(np.abs(ref) + acc) + acc
    err = np.abs(gpu - ref)
    assert np.all(err <= bound), f"{tag} kv err {float(np.max(err - bound)):.3e} over bound"
