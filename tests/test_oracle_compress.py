"""Pins for the oracle's visibility sets and learned compressor.

Sources (page "CSA And HCA: Definition, State, And Cost Model"):
  section 1      completed entries E_t = {s < floor((t+1)/r)}
  section 2.1    CSA two-stream overlapping compression and its entry-composition listing
  section 2.2    HCA one-stream compression
  section 5.1    window L_t
  section 6      worked-example table (golden file)
Page "transformers PR 45892 discussion": a padded incomplete block must never
contribute to a compressed entry.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ sets --- #

def test_worked_example_table():
    g = _gold("p3_worked_example.json")
    for row in g["rows"]:
        t = row["t"]
        csa = list(range(oracle.visible_count(t, g["m"])))
        hca = list(range(oracle.visible_count(t, g["m_prime"])))
        s = oracle.sets(t, 1, g["m"], 0, g["w"])
        local = list(range(int(s["win_lo"][0]), int(s["win_lo"][0]) + int(s["win_len"][0])))
        assert csa == row["csa"], t
        assert hca == row["hca"], t
        assert local == row["local"], t


@pytest.mark.parametrize("m,k,w", [(4, 16, 16), (4, 512, 128), (128, 0, 128), (3, 5, 1)])
def test_sets_closed_forms(m, k, w):
    T = 3000
    s = oracle.sets(0, T, m, k, w)
    t = np.arange(T)
    E = (t + 1) // m
    assert np.array_equal(s["E"], E)
    assert np.array_equal(s["cnt"], np.minimum(E, k) if k > 0 else E)
    assert np.array_equal(s["win_len"], np.minimum(w, t + 1))
    assert np.array_equal(s["win_lo"] + s["win_len"] - 1, t)  # window ends at t itself


def test_block_final_token_sees_its_entry():
    # the last token of a block (t = m*i + m - 1) already sees entry i; earlier ones do not
    m = 4
    for i in range(5):
        assert oracle.visible_count(m * i + m - 1, m) == i + 1
        for j in range(m - 1):
            assert oracle.visible_count(m * i + j, m) == i


# ------------------------------------------------------------ compressor --- #

def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_overlap_composition_one_hot():
    """One-hot values reproduce the printed composition: entry i pools a(block i) + b(block i-1)."""
    g = _gold("p3_overlap_example.json")
    m = g["m"]
    n = 12
    c = 2 * n  # channel p marks stream a of token p, channel n+p marks stream b of token p
    C = np.zeros((n, 2 * c))
    for p in range(n):
        C[p, p] = 1.0             # stream a value of token p (a-half, channel p)
        C[p, c + n + p] = 1.0     # stream b value of token p (b-half, channel n+p)
    Z = np.zeros((n, 2 * c))
    B = np.zeros((2 * m, c))
    out = oracle.compress(C, Z, B, tok_base=0, i_begin=0, i_end=n // m, c=c, m=m, overlap=True)
    for ent in g["entries"]:
        i = ent["i"]
        nz = set(np.nonzero(out[i])[0].tolist())
        expect = set(ent["a"]) | {n + p for p in ent["b"]}
        assert nz == expect, (i, nz, expect)
        npos = len(ent["a"]) + len(ent["b"])
        assert np.allclose(out[i][sorted(expect)], 1.0 / npos, rtol=0, atol=1e-15)


@pytest.mark.parametrize("overlap", [False, True])
def test_equal_logits_give_block_mean(overlap):
    m, c, n = 4, 8, 24
    width = 2 * c if overlap else c
    C = _rand(1, n, width)
    Z = np.full((n, width), 0.7)
    B = np.zeros((2 * m if overlap else m, c))
    out = oracle.compress(C, Z, B, tok_base=0, i_begin=0, i_end=n // m, c=c, m=m, overlap=overlap)
    for i in range(n // m):
        a = C[m * i:m * (i + 1), :c]
        if overlap and i > 0:
            b = C[m * (i - 1):m * i, c:]
            expect = np.concatenate([a, b]).mean(axis=0)
        else:
            expect = a.mean(axis=0)
        assert np.allclose(out[i], expect, rtol=1e-14, atol=1e-15)


def test_softmax_weights_and_bias_rows_by_hand():
    """m=1, c=1: entry 1 pools a(token 1) with bias B^a and b(token 0) with bias B^b."""
    C = np.array([[100.0, 0.0],    # token 0: a-value 100 (must not enter entry 1), b-value 0
                  [1.0, -50.0]])   # token 1: a-value 1, b-value -50 (must not enter entry 1)
    Z = np.zeros((2, 2))
    B = np.array([[math.log(3.0)], [0.0]])  # B^a row then B^b row
    out = oracle.compress(C, Z, B, tok_base=0, i_begin=0, i_end=2, c=1, m=1, overlap=True)
    assert out[0, 0] == pytest.approx(100.0, abs=1e-13)           # i = 0: stream a only
    assert out[1, 0] == pytest.approx(0.75 * 1.0 + 0.25 * 0.0, abs=1e-15)
    B2 = B[::-1].copy()  # swapped bias rows give the other weighting
    out2 = oracle.compress(C, Z, B2, tok_base=0, i_begin=0, i_end=2, c=1, m=1, overlap=True)
    assert out2[1, 0] == pytest.approx(0.25, abs=1e-15)
    # logits come from the Z column of the same stream
    Z3 = np.array([[0.0, math.log(3.0)], [0.0, 0.0]])  # token 0, stream b logit ln3
    out3 = oracle.compress(C, Z3, np.zeros((2, 1)), tok_base=0, i_begin=1, i_end=2, c=1, m=1,
                           overlap=True)
    assert out3[0, 0] == pytest.approx(0.25 * 1.0 + 0.75 * 0.0, abs=1e-15)


@pytest.mark.parametrize("overlap", [False, True])
def test_shift_invariance_and_dominant_logit(overlap):
    m, c, n = 4, 16, 32
    width = 2 * c if overlap else c
    C, Z = _rand(2, n, width), _rand(3, n, width)
    B = _rand(4, 2 * m if overlap else m, c) * math.sqrt(0.1)
    ref = oracle.compress(C, Z, B, tok_base=0, i_begin=0, i_end=n // m, c=c, m=m, overlap=overlap)
    shift = _rand(5, width)
    if overlap:  # the same per-channel constant must be added to both halves
        shift[c:] = shift[:c]
    out = oracle.compress(C, Z + 80.0 + shift, B, tok_base=0, i_begin=0, i_end=n // m, c=c, m=m,
                          overlap=overlap)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)
    Zd = Z.copy()
    Zd[9, 3] += 1000.0  # token 9 dominates channel 3 of every entry that pools it (a-stream)
    out = oracle.compress(C, Zd, B, tok_base=0, i_begin=0, i_end=n // m, c=c, m=m, overlap=overlap)
    assert out[9 // m, 3] == pytest.approx(C[9, 3], abs=1e-12)


def test_incomplete_block_never_visible():
    """n = 254, 255: floor(n/m) entries; the partial tail block changes nothing emitted."""
    m, c = 4, 8
    for n in (254, 255):
        C, Z = _rand(6, n, 2 * c), _rand(7, n, 2 * c)
        B = _rand(8, 2 * m, c)
        E = oracle.visible_count(n - 1, m)
        assert E == n // m
        ref = oracle.compress(C, Z, B, tok_base=0, i_begin=0, i_end=E, c=c, m=m, overlap=True)
        C2, Z2 = C.copy(), Z.copy()
        C2[m * E:] = 1e6
        Z2[m * E:] = 50.0
        out = oracle.compress(C2, Z2, B, tok_base=0, i_begin=0, i_end=E, c=c, m=m, overlap=True)
        assert np.array_equal(out, ref)
        with pytest.raises(ValueError):  # the incomplete block cannot be emitted
            oracle.compress(C, Z, B, tok_base=0, i_begin=E, i_end=E + 1, c=c, m=m, overlap=True)


@pytest.mark.parametrize("overlap,m", [(True, 4), (False, 128)])
def test_buffer_offset_and_chunking(overlap, m):
    """Emitting from a buffer that starts at tok_base equals emitting from the full sequence."""
    c, n = 8, 6 * m
    width = 2 * c if overlap else c
    C, Z = _rand(9, n, width), _rand(10, n, width)
    B = _rand(11, 2 * m if overlap else m, c)
    g = np.abs(_rand(12, c)) + 0.5
    kw = dict(c=c, m=m, overlap=overlap, gamma=g, eps=1e-6, rope_dims=4)
    full = oracle.compress(C, Z, B, tok_base=0, i_begin=0, i_end=n // m, **kw)
    for i in range(n // m):
        base = m * (i - 1) if (overlap and i > 0) else m * i
        part = oracle.compress(C[base:m * (i + 1)], Z[base:m * (i + 1)], B, tok_base=base,
                               i_begin=i, i_end=i + 1, **kw)
        assert np.array_equal(part[0], full[i])


def test_norm_and_rope_epilogue_order():
    """Entry i = RoPE_{m*i}(RMSNorm(pooled)); checked against pooled values from a norm/rope-free call."""
    m, c, n = 4, 16, 16
    C, Z = _rand(13, n, 2 * c), _rand(14, n, 2 * c)
    B = _rand(15, 2 * m, c)
    g = np.abs(_rand(16, c)) + 0.5
    raw = oracle.compress(C, Z, B, tok_base=0, i_begin=0, i_end=4, c=c, m=m, overlap=True)
    out = oracle.compress(C, Z, B, tok_base=0, i_begin=0, i_end=4, c=c, m=m, overlap=True,
                          gamma=g, eps=0.0, rope_dims=8, rope_base=10000.0)
    for i in range(4):
        y = raw[i] / np.sqrt(np.mean(raw[i] ** 2)) * g
        # first c-8 channels: only the norm applies
        assert np.allclose(out[i, :c - 8], y[:c - 8], rtol=1e-13)
        # rotated channels keep each pair's norm
        pr = out[i, c - 8:].reshape(4, 2)
        py = y[c - 8:].reshape(4, 2)
        assert np.allclose(np.hypot(pr[:, 0], pr[:, 1]), np.hypot(py[:, 0], py[:, 1]), rtol=1e-13)
        # pair 0 turns by exactly m*i radians (theta_0 = 1)
        ang = math.atan2(pr[0, 1], pr[0, 0]) - math.atan2(py[0, 1], py[0, 0])
        assert math.remainder(ang - m * i, 2 * math.pi) == pytest.approx(0.0, abs=1e-12)


@pytest.mark.parametrize("overlap,m", [(True, 4), (False, 4), (False, 8)])
def test_bias_rows_follow_position_in_block(overlap, m):
    """Bias row j belongs to position j of its block ("CSA And HCA" section 2.1: B^a with
    block i, B^b with block i-1; section 2.2: B with the one stream).  Zero gate logits and
    one large bias per channel make the softmax one-hot, so channel ch of entry i must equal
    the value row m*i + tgt[ch] (stream a) or m*(i-1) + tgt[ch] (stream b); a reversed or
    shifted row order picks another row."""
    c, n = 8, 6 * m
    rng = np.random.default_rng(31 + m + overlap)
    width = 2 * c if overlap else c
    C = rng.standard_normal((n, width))
    Z = np.zeros((n, width))
    tgt = rng.integers(0, m, c)
    if m == 4:
        tgt[:4] = [0, 1, 2, 3]  # every row of the block is somebody's target
    use_b = np.array([overlap and ch % 2 == 1 for ch in range(c)])
    B = np.zeros(((2 if overlap else 1) * m, c))
    for ch in range(c):
        B[(m if use_b[ch] else 0) + tgt[ch], ch] = 60.0
    out = oracle.compress(C, Z, B, tok_base=0, i_begin=0, i_end=n // m, c=c, m=m,
                          overlap=overlap)
    for i in range(n // m):
        for ch in range(c):
            if use_b[ch]:
                if i == 0:  # no preceding block: plain mean of the a-stream rows
                    expect = C[0:m, ch].mean()
                else:
                    expect = C[m * (i - 1) + tgt[ch], c + ch]
            else:
                expect = C[m * i + tgt[ch], ch]
            assert out[i, ch] == pytest.approx(expect, rel=1e-12, abs=1e-12), (i, ch)
    # sensitivity: the bias rows reversed inside the block select other rows
    Brev = B.copy()
    Brev[:m] = B[:m][::-1]
    if overlap:
        Brev[m:] = B[m:][::-1]
    out_rev = oracle.compress(C, Z, Brev, tok_base=0, i_begin=0, i_end=n // m, c=c, m=m,
                              overlap=overlap)
    assert np.abs(out_rev - out).max() > 1e-2
