"""The attention parity gates against mistakes planted in oracle outputs (CPU only).

A kernel that computes the softmax over a slightly wrong candidate set (one entry counted
twice) produces outputs that stay within the absolute 2e-2 gate, because outputs averaged
over hundreds of unit-RMS rows are only ~0.08 in size.  The per-row RMS
gate of `assert_attn_close` must reject those, and must accept bf16 rounding of the exact
result.  The workload follows the 8K CSA prefill: c = 512, k = 512 selected entries of
~1000 visible ones, w = 128, normalised and rotated query and rows.
"""
import numpy as np
import pytest

import oracle
from _helpers import assert_attn_close, assert_close

ATOL = 2e-2
REL_RMS = 0.03


def _bf16(x):
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


@pytest.fixture(scope="module")
def case():
    rng = np.random.default_rng(2024)
    c, n_h, k, w, T, t0 = 512, 16, 512, 128, 2, 4000
    E = (t0 + T) // 4
    q = rng.standard_normal((T, n_h, c)) / np.sqrt(c)
    kv = rng.standard_normal((E, c))
    local = rng.standard_normal((t0 + T, c)) / np.sqrt(c)
    idx = np.stack([np.sort(rng.choice((t0 + j + 1) // 4, k, replace=False)) for j in range(T)])
    cnt = np.full(T, k, np.int32)
    kw = dict(loc_base=0, t0=t0, w=w, q_norm=True, kv_norm=True, rope_dims=64)
    ref = oracle.attend_csa(q, kv, local, idx.astype(np.int32), cnt, **kw)
    return dict(q=q, kv=kv, local=local, idx=idx.astype(np.int32), cnt=cnt, kw=kw, ref=ref)


def test_bf16_rounding_passes(case):
    assert_attn_close(_bf16(case["ref"]), case["ref"], atol=ATOL, rel_rms=REL_RMS, what="bf16")


def test_missing_chunk_fails(case):
    """64 of the 640 candidates left out (one chunk never gathered)."""
    c2 = case["cnt"] - 64
    got = oracle.attend_csa(case["q"], case["kv"], case["local"], case["idx"], c2, **case["kw"])
    with pytest.raises(AssertionError):
        assert_attn_close(got, case["ref"], atol=ATOL, rel_rms=REL_RMS, what="missing chunk")


def test_one_duplicated_candidate_fails_only_the_rms_gate(case):
    """One selected entry counted twice: within the absolute gate everywhere, but the rows
    whose softmax it shifts fail the per-row RMS bound."""
    idx, k = case["idx"], case["idx"].shape[1]
    dup = np.concatenate([idx, idx[:, :1]], axis=1).astype(np.int32)
    got = oracle.attend_csa(case["q"], case["kv"], case["local"], dup,
                            np.full(len(dup), k + 1, np.int32), **case["kw"])
    assert_close(got, case["ref"], atol=ATOL, what="absolute gate alone")
    with pytest.raises(AssertionError, match="RMS bound"):
        assert_attn_close(got, case["ref"], atol=ATOL, rel_rms=REL_RMS, what="duplicated entry")


def test_swapped_heads_fail(case):
    got = case["ref"].copy()
    got[:, [0, 1]] = got[:, [1, 0]]
    with pytest.raises(AssertionError):
        assert_attn_close(got, case["ref"], atol=ATOL, rel_rms=REL_RMS, what="swapped heads")
