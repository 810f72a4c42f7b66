"""Comparison helpers shared by the GPU parity tests."""
from __future__ import annotations

import numpy as np

import oracle


def log(msg: str):
    print(msg, flush=True)


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def assert_close(got, ref, *, atol=0.0, rtol=0.0, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} out of tolerance; worst at "
                             f"{i}: got {got[i]!r} ref {ref[i]!r} err {err[i]:.3g} bound {bound[i]:.3g}")


def assert_attn_close(got, ref, *, atol, rel_rms, rtol=0.0, what=""):
    """Attention outputs: every element within `atol` (the element-wise gate), and every
    output row (one query, one head: the last axis) within `rel_rms` of the row's RMS in RMS
    error, plus atol / 16 for rows that are nearly zero.

    The second bound is what catches structural mistakes: attention outputs of unit-RMS rows
    averaged over hundreds of candidates are only ~0.05 in size, so a row that loses or
    double-counts a tenth of its softmax mass can stay within an absolute 2e-2.  The bf16
    path rounds the normalised query, the probabilities and the output to 8 significant
    bits (2^-9 relative each), which puts its RMS error near 0.5 % of the row's RMS.
    `rtol` widens the element gate by a multiple of |ref| where one or two candidates carry
    the whole softmax (see the callers)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert_close(got, ref, atol=atol, rtol=rtol, what=what)
    n = ref.shape[-1]
    e = np.sqrt(np.mean((got - ref) ** 2, axis=-1))
    r = np.sqrt(np.mean(ref ** 2, axis=-1))
    bound = rel_rms * r + atol / 16.0
    bad = ~(e <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, e / np.maximum(r, 1e-30), -np.inf)), e.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {e.size} rows (of {n}) beyond RMS bound; "
                             f"worst at {i}: rms err {e[i]:.3g}, row rms {r[i]:.3g}")


def assert_bf16_close(got, ref, ulps=1.0, atol=4e-6, what=""):
    """|got - ref| <= ulps * ulp_bf16(ref) + atol.  The float32 result rounded to bf16 may land
    on either neighbour of the exact value (1 ulp); atol covers float32 accumulation over up to
    128 pooled positions of unit-RMS rows, which dominates where the exact value is tiny."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bound = ulps * bf16_ulp(ref) + atol
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} beyond {ulps} bf16 ulp; "
                             f"worst at {i}: got {got[i]!r} ref {ref[i]!r}")


def check_topk(idx, cnt, ref_scores, *, t0, m, k, rel=1e-4, gpu_scores=None, what=""):
    """Compare GPU top-k against float64 oracle scores.

    idx [T][k] (ascending, -1 padded), cnt [T]; ref_scores [T][>=E] float64.
    Exact set equality where the relative gap between the k-th and (k+1)-th oracle
    scores exceeds `rel`; otherwise the selection must be a valid top-k within `rel`.
    Returns the number of queries that needed the tolerant rule.
    """
    T = idx.shape[0]
    tolerant = 0
    for j in range(T):
        t = t0 + j
        E = (t + 1) // m
        n = min(k, E)
        assert cnt[j] == n, f"{what} row {j}: cnt {cnt[j]} != {n}"
        sel = idx[j, :n]
        assert np.all(idx[j, n:] == -1), f"{what} row {j}: padding"
        if n == 0:
            continue
        assert np.all(np.diff(sel) > 0), f"{what} row {j}: not ascending/unique"
        assert sel[0] >= 0 and sel[-1] < E, f"{what} row {j}: index outside visible entries"
        s = ref_scores[j, :E]
        if gpu_scores is not None:
            g = gpu_scores[j, :n]
            assert np.allclose(g, s[sel], rtol=2e-5, atol=1e-5 * max(1.0, np.abs(s).max())), \
                f"{what} row {j}: returned scores differ from the oracle's"
        if n == E:
            continue
        order = np.lexsort((np.arange(E), -s))
        vk, vn = s[order[n - 1]], s[order[n]]
        scale = max(abs(vk), 1e-30)
        if (vk - vn) / scale > rel:
            assert set(sel.tolist()) == set(order[:n].tolist()), f"{what} row {j}: set differs"
        else:
            tolerant += 1
            mask = np.zeros(E, bool)
            mask[sel] = True
            assert np.all(s[mask] >= vk - rel * scale), f"{what} row {j}: selected too small"
            assert np.all(s[~mask] <= vk + rel * scale), f"{what} row {j}: left out too large"
    return tolerant


def fp8_step(v):
    """Spacing of E4M3 values at |v| (v already divided by the row scale)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    return 2.0 ** (e - 3)


def e2m1_step(v):
    a = np.abs(v)
    return np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))


def decode_stored(t, dt, scale=None):
    """Device tensor in a stored format -> float64 numpy via the oracle's decoders."""
    import torch
    if dt == "f32":
        return t.detach().cpu().numpy().astype(np.float64)
    if dt == "bf16":
        return oracle.decode_bf16(t.detach().view(torch.int16).cpu().numpy().view(np.uint16))
    if dt == "fp8":
        return oracle.decode_fp8_rows(t.detach().cpu().numpy(), scale.detach().cpu().numpy())
    if dt == "mxfp4":
        return oracle.decode_mxfp4_rows(t.detach().cpu().numpy(), scale.detach().cpu().numpy())
    raise ValueError(dt)
