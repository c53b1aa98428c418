"""Shared helpers for the GPU parity tests (no method arithmetic here)."""

import numpy as np

REL_L2_TOL = 5e-3
MAX_ABS_TOL = 3e-2


def to_dev(x, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def bf16_half_ulp(x):
    """Half a bfloat16 ulp at |x| (the most the final round-to-nearest store can move a value)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def compare(gpu, ref, what, bf16_out=True, rel_tol=REL_L2_TOL, abs_tol=MAX_ABS_TOL):
    """Parity bar: rel-L2 <= rel_tol and, element-wise, |gpu - ref| <= abs_tol (+ the half-ulp of
    the bf16 store when the GPU output is bf16).  Returns a dict of the measured errors."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), what + ": non-finite GPU output"
    err = gpu - ref
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    bound = abs_tol + (bf16_half_ulp(gpu) if bf16_out else 0.0)
    excess = np.abs(err) - bound
    worst = int(np.argmax(excess))
    info = {"rel_l2": rel, "max_abs": float(np.abs(err).max()), "max_excess": float(excess.flat[worst])}
    assert rel <= rel_tol, "%s: rel-L2 %.3e > %.1e" % (what, rel, rel_tol)
    assert excess.flat[worst] <= 0, "%s: |err| %.3e at %s exceeds %.3e (ref %.4f gpu %.4f)" % (
        what, abs(err.flat[worst]), np.unravel_index(worst, err.shape), bound if np.isscalar(bound)
        else bound.flat[worst], ref.flat[worst], gpu.flat[worst])
    return info


L_REL_TOL = 1e-4


def compare_l(gpu, ref, what, rel_tol=L_REL_TOL):
    """Row sums of P~: element-wise |gpu - ref| <= rel_tol * ref (the GPU sums the same quantized
    codes in fp32; rows with ref = 0, which see no key, must be exactly 0).  Returns the largest
    relative error."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), what + ": non-finite l"
    empty = ref == 0
    assert np.all(gpu[empty] == 0), what + ": l of a row that sees no key is not 0"
    r = np.abs(gpu - ref)[~empty] / ref[~empty]
    worst = float(r.max(initial=0.0))
    print("%s: largest relative l error %.2e" % (what, worst))
    assert worst <= rel_tol, "%s: relative l error %.3e > %.1e" % (what, worst, rel_tol)
    return worst


def cosine(a, b):
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
