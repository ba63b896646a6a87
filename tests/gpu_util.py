"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

from oracle import spatten_ref as R


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype=dtype).cuda()


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_err_over_rms(got, ref):
    """max |got - ref| / rms(ref): the largest element error in units of
    the reference's root mean square."""
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / max(rms, 1e-30))


def bf16_ulp(v):
    """Spacing of bf16 values at |v|."""
    _, e = np.frexp(np.abs(np.asarray(v, np.float64)))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def check_bf16_output(got, ref, tol=2e-2, what="", allow=0.0):
    """bf16 outputs: RMS error within `tol` of the output RMS, and no
    element off by more than tol * RMS beyond one bf16 spacing of its own
    value (an fp32 and an fp64 evaluation of the same value can round to
    neighbouring bf16 values when it lies near a rounding boundary).
    `allow` (per element, or scalar) widens the element bound where a
    decision the two sides take in different precision (a value-pruning
    threshold) may differ; the RMS check then excludes it too.
    Returns (normalised RMS error, max |error| / RMS)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    rms = max(np.sqrt(np.mean(ref * ref)), 1e-30)
    d_rms = np.sign(d) * np.maximum(np.abs(d) - allow, 0.0)
    nrmse = np.sqrt(np.mean(d_rms * d_rms)) / rms
    excess = np.abs(d) - bf16_ulp(ref) - allow
    i = int(np.argmax(excess))
    assert nrmse <= tol, "%s: normalised RMS error %.3g > %g" % (what, nrmse, tol)
    assert excess.flat[i] <= tol * rms, (
        "%s: element %d got %.6g want %.6g (rms %.3g)" % (what, i, got.flat[i], ref.flat[i], rms))
    return nrmse, float(np.max(np.abs(d)) / rms)


def check_selection(gpu_idx, oracle_scores, k, band=1e-5):
    """The GPU's selected set must equal the oracle's top-k apart from
    elements whose oracle score lies within `band` (relative) of the
    oracle's k-th score. Returns the number of differing elements."""
    s32 = np.asarray(oracle_scores, np.float64).astype(np.float32)
    ref = R.topk(s32, k)
    kth = float(R.kth_value(s32, k))
    diff = np.setxor1d(np.asarray(gpu_idx), ref)
    for j in diff:
        assert abs(float(oracle_scores[j]) - kth) <= band * abs(kth) + 1e-30, (
            "selection differs outside the tie band: idx %d score %.9g kth %.9g" %
            (j, oracle_scores[j], kth))
    assert len(np.unique(gpu_idx)) == k and np.all(np.diff(gpu_idx) > 0)
    return len(diff)


class PrefillWs:
    """Byte offsets of the prefill scratch arrays (mirrors the library's
    workspace layout) so tests can read the head outputs O."""

    def __init__(self, B, n, h, dh, es, bf16):
        def a256(v):
            return (v + 255) // 256 * 256
        n_pad = (n + 255) // 256 * 256
        off = 0
        self.n_pad = n_pad
        sizes = [("q", B * h * n_pad * dh * es), ("k", B * h * n_pad * dh * es),
                 ("vt", B * h * n_pad * dh * es), ("o", B * n * h * dh * es)]
        for name, sz in sizes:
            setattr(self, name, off)
            off += a256(sz)
