"""Pins for the oracle's decode step and its stored-format decoders.

Decode order: page "CSA And HCA: Definition, State, And Cost Model", section 7
(ring insert, compressor updates, emission when (t+1) is a multiple of m, then
selection and attention).  A decode step at t must reproduce prefill row t.

Decoders: OCP OFP8 v1.0 (E4M3) and OCP MX v1.0 (E2M1 elements, E8M0 scales);
expected values are the specifications' code points.
"""
import math

import numpy as np
import pytest

import oracle


def _prefill(n=40, c=16, cI=8, n_h=3, n_hI=2, m=4, k=3, w=5, rd=8, seed=0):
    rng = np.random.default_rng(seed)
    P = dict(n=n, c=c, cI=cI, n_h=n_h, n_hI=n_hI, m=m, k=k, w=w, rd=rd)
    P["C"], P["Z"] = rng.standard_normal((n, 2 * c)), rng.standard_normal((n, 2 * c))
    P["CI"], P["ZI"] = rng.standard_normal((n, 2 * cI)), rng.standard_normal((n, 2 * cI))
    P["B"], P["BI"] = rng.standard_normal((2 * m, c)), rng.standard_normal((2 * m, cI))
    P["local"] = rng.standard_normal((n, c))
    P["q"] = rng.standard_normal((n, n_h, c))
    P["qI"] = rng.standard_normal((n, n_hI, cI))
    P["wI"] = rng.random((n, n_hI))
    E = n // m
    P["kv"] = oracle.compress(P["C"], P["Z"], P["B"], tok_base=0, i_begin=0, i_end=E, c=c, m=m,
                              overlap=True, gamma=np.ones(c), rope_dims=rd)
    P["KI"] = oracle.compress(P["CI"], P["ZI"], P["BI"], tok_base=0, i_begin=0, i_end=E, c=cI,
                              m=m, overlap=True, gamma=np.ones(cI))
    sc = oracle.index_scores(P["qI"], P["KI"], P["wI"], t0=0, m=m, ld=E)
    P["idx"], P["cnt"] = oracle.topk(sc, t0=0, m=m, k=k)
    P["out"] = oracle.attend_csa(P["q"], P["kv"], P["local"], P["idx"], P["cnt"], loc_base=0,
                                 t0=0, w=w, q_norm=True, kv_norm=True, rope_dims=rd)
    return P


@pytest.mark.parametrize("t", [39, 37, 3, 2, 0])
def test_decode_step_equals_prefill_row(t):
    P = _prefill()
    m, w, c, cI = P["m"], P["w"], P["c"], P["cI"]
    E_before = t // m
    st = {
        "kv_comp": np.zeros((P["n"] // m, c)), "KI": np.zeros((P["n"] // m, cI)),
        "ring": np.full((w, c), np.nan),
    }
    st["kv_comp"][:E_before] = P["kv"][:E_before]
    st["KI"][:E_before] = P["KI"][:E_before]
    for j in range(max(0, t - w), t):
        st["ring"][j % w] = P["local"][j]
    i = t // m
    base = max(0, m * (i - 1))
    for nm, src in (("tail_C", "C"), ("tail_Z", "Z"), ("tail_CI", "CI"), ("tail_ZI", "ZI")):
        st[nm] = P[src][base:m * (i + 1)]
    st["tail_base"] = base
    st["B"], st["BI"] = P["B"], P["BI"]
    st["kv_new"] = P["local"][t]
    st["q"], st["qI"], st["wI"] = P["q"][t], P["qI"][t], P["wI"][t]
    r = oracle.decode_step(st, t=t, c=c, cI=cI, m=m, k=P["k"], w=w, rope_dims=P["rd"],
                           gamma=np.ones(c), gammaI=np.ones(cI))
    assert r["emitted"] == ((t + 1) % m == 0)
    if r["emitted"]:
        assert np.array_equal(st["kv_comp"][i], P["kv"][i])
        assert np.array_equal(st["KI"][i], P["KI"][i])
    assert r["cnt"] == P["cnt"][t]
    assert np.array_equal(r["idx"], P["idx"][t])
    assert np.allclose(r["out"], P["out"][t], rtol=1e-13, atol=1e-14)
    assert np.array_equal(st["ring"][t % w], P["local"][t])


# --------------------------------------------------------------- formats --- #

def test_bf16_decoder():
    bits = np.array([0x3F80, 0xC020, 0x0000, 0x8000, 0x7F80, 0x3F81, 0x0001], np.uint16)
    v = oracle.decode_bf16(bits)
    assert v[0] == 1.0 and v[1] == -2.5 and v[2] == 0.0 and math.copysign(1, v[3]) < 0
    assert math.isinf(v[4]) and v[5] == 1.0 + 2.0 ** -7 and v[6] == 2.0 ** -133


def test_fp8_e4m3_decoder_code_points():
    codes = np.array([[0x00, 0x01, 0x07, 0x08, 0x38, 0x3F, 0x7E, 0xB8, 0xFE, 0x80]], np.uint8)
    v = oracle.decode_fp8_rows(codes)[0]
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.875, 448.0, -1.0, -448.0, -0.0]
    assert v.tolist() == want
    assert math.isnan(oracle.decode_fp8_rows(np.array([[0x7F]], np.uint8))[0, 0])
    sc = oracle.decode_fp8_rows(np.array([[0x38, 0x40], [0x38, 0x40]], np.uint8),
                                np.array([0.5, 3.0], np.float32))
    assert sc.tolist() == [[0.5, 1.0], [3.0, 6.0]]


def test_mxfp4_decoder_code_points():
    # nibbles 0..15 -> E2M1 values; element 2j is the low nibble of byte j
    packed = np.array([[0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE] + [0] * 8], np.uint8)
    e8 = np.array([[127]], np.uint8)
    v = oracle.decode_mxfp4_rows(packed, e8)[0, :16]
    want = [0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    assert v.tolist() == want
    for code, scale in ((128, 2.0), (126, 0.5), (0, 2.0 ** -127), (254, 2.0 ** 127)):
        s = oracle.decode_mxfp4_rows(np.array([[0x02] + [0] * 15], np.uint8),
                                     np.array([[code]], np.uint8))
        assert s[0, 0] == scale  # code 2 is 1.0
    assert math.isnan(oracle.decode_mxfp4_rows(np.zeros((1, 16), np.uint8),
                                               np.array([[255]], np.uint8))[0, 0])
    # one scale per 32 elements
    two = oracle.decode_mxfp4_rows(np.full((1, 32), 0x22, np.uint8), np.array([[127, 130]], np.uint8))
    assert np.all(two[0, :32] == 1.0) and np.all(two[0, 32:] == 8.0)


def test_kv576_row_decoder():
    """A production cache row: E4M3 codes (times the row scale) for the leading channels,
    bf16 for the rotated ones; code points from the OCP FP8 and bfloat16 definitions."""
    c, rd = 16, 4
    row = np.zeros(c + rd, np.uint8)
    row[0] = 0x7E        # E4M3 448 (exponent 15, mantissa 6)
    row[1] = 0x38        # 1.0
    row[2] = 0xB8        # -1.0
    row[3] = 0x01        # smallest subnormal 2^-9
    bf = np.array([0x3F80, 0xC000, 0x3E80, 0x0000], np.uint16)  # 1, -2, 0.25, 0
    row[c - rd:] = bf.view(np.uint8)
    got = oracle.decode_kv576_rows(row[None], np.array([0.5], np.float32), c=c, rope_dims=rd)[0]
    assert got[0] == 224.0 and got[1] == 0.5 and got[2] == -0.5 and got[3] == 2.0 ** -10
    assert np.all(got[4:c - rd] == 0.0)
    assert list(got[c - rd:]) == [1.0, -2.0, 0.25, 0.0]
