"""Shared test helpers: the parity tolerance, tensor conversions, the oracle's
view of a device layer."""
import numpy as np

# Tolerance for fp16 outputs (layer outputs, attention outputs, logits):
# max |err| <= 1e-2 * max |ref| + 1e-3.
REL, ABS = 1e-2, 1e-3


def np16(t) -> np.ndarray:
    """torch fp16 tensor -> numpy uint16 bit patterns (host copy)."""
    import torch
    assert t.dtype == torch.float16
    return t.detach().cpu().contiguous().numpy().view(np.uint16)


def f32(u16) -> np.ndarray:
    return np.asarray(u16).view(np.float16).astype(np.float32)


def max_err(got_u16, ref_u16):
    g, r = f32(got_u16), f32(ref_u16)
    return float(np.abs(g - r).max()), float(REL * np.abs(r).max() + ABS)


def assert_close(got_u16, ref_u16, what=""):
    err, tol = max_err(got_u16, ref_u16)
    assert np.all(np.isfinite(f32(got_u16))), f"{what}: non-finite output"
    assert err <= tol, f"{what}: max|err| {err:.3e} > tol {tol:.3e}"
    return err, tol


def dev16(a, device="cuda"):
    """numpy fp16 / uint16 bit patterns -> torch fp16 device tensor (same bits)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.float16).to(device)


def ranked_kv(q, P: int, seed: int):
    """Keys and values of P cached positions whose scores against q are
    evenly spread: per (sequence, head) the keys are c_p sign(q_h) r_h with
    c_p a random permutation of evenly spaced values in [-1.5, 1.5) and
    r_h = sqrt(hd) / |q_h|_1, so the head's scores are c_p (spaced 3 / P).
    The key rows are two-level, which the 4-bit codec keeps exactly, and a
    Top-K selection does not hinge on either side's rounding of q.
    q: float [bls, nh, hd].  Returns (k, v) fp16 [bls, P, nh * hd]."""
    bls, nh, hd = q.shape
    h1 = nh * hd
    rng = np.random.default_rng(seed)
    c = np.stack([rng.permutation(P) for _ in range(bls * nh)]).reshape(bls, nh, P) * (3.0 / P) - 1.5
    sg = np.where(q >= 0, 1.0, -1.0) * (np.sqrt(hd) / np.abs(q).sum(-1))[..., None]
    k = c[..., None] * sg[:, :, None, :]
    kx = k.transpose(0, 2, 1, 3).reshape(bls, P, h1).astype(np.float16)
    vx = (rng.standard_normal((bls, P, h1)) * 2).astype(np.float16)
    return kx, vx
