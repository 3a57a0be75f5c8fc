"""Helpers shared by the GPU parity tests: uploads, the error bar, and the near-tie
protocol for routing.

Error bar (the layer's stated tolerance, bf16 I/O with fp32 accumulation):
  * fp32 output:  max |y - ref| <= 1e-2 * RMS(ref)
  * bf16 output:  |y - ref| <= 1e-2 * RMS(ref) + 2^-8 * |ref| per element (the second
    term is the bf16 rounding of the output itself, |fl(v) - v| <= 2^-8 |v|)
where ref is the fp64 oracle and RMS(ref) is taken over the whole compared output.

Near ties: the GPU ranks fp32 logits, the oracle fp64 ones.  A token whose oracle gap
between the k-th and (k+1)-th logit is below TAU is "ambiguous": either selection is
correct, and its output is compared with the oracle evaluated on the GPU's own routing.
Elsewhere the selected experts must match exactly.
"""
import numpy as np

TAU = 1e-5
W_TOL = 1e-6          # |w_gpu - w_ref| at unambiguous tokens (the stated routing-weight bound)


def to_dev(a, torch):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def y_to_np(y, torch):
    if y.dtype == torch.bfloat16:
        return y.float().cpu().numpy().astype(np.float64)
    return y.cpu().numpy().astype(np.float64)


def check_output(y, ref, bf16_out: bool, what: str = ""):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(y - ref)
    if bf16_out:
        excess = err - (1e-2 * rms + 2.0 ** -8 * np.abs(ref))
        ok = bool((excess <= 0).all())
    else:
        ok = bool(err.max() <= 1e-2 * rms)
    rel = float(err.max() / rms)
    assert ok, f"{what}: max|err|/RMS = {rel:.3e} (bf16_out={bf16_out})"
    return rel


def check_routing(idx_gpu, w_gpu, idx_ref, w_ref, gap, w_tol=None):
    """Exact expert sets at unambiguous tokens; returns (the ambiguous-token mask, the
    largest |w_gpu - w_ref| at unambiguous tokens)."""
    w_tol = W_TOL if w_tol is None else w_tol
    idx_gpu = np.asarray(idx_gpu)
    amb = np.asarray(gap) < TAU
    ok = ~amb
    assert (np.diff(idx_gpu, axis=1) > 0).all(), "indices not strictly ascending"
    bad = np.nonzero((idx_gpu[ok] != idx_ref[ok]).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} unambiguous tokens route differently"
    werr = np.abs(np.asarray(w_gpu, np.float64)[ok] - w_ref[ok])
    wmax = float(werr.max()) if werr.size else 0.0
    assert wmax <= w_tol, f"max |w err| = {wmax:.3e}"
    assert np.allclose(np.asarray(w_gpu, np.float64).sum(axis=1), 1.0, atol=1e-5)
    return amb, wmax


def report(what: str, **kv):
    """One line per parity case (shown with pytest -s / -rP): the error, the ambiguous
    tokens, the largest routing-weight error."""
    print(f"[parity] {what}: " + ", ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}"
                                         for k, v in kv.items()), flush=True)


def sample_tokens(T: int, n: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    pick |= {0, T - 1}
    return np.array(sorted(pick))
