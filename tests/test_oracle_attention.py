"""Pins for the oracle's shared-KV MQA attention, RMSNorm and RoPE.

Sources:
  page "CSA And HCA: Definition, State, And Cost Model"
    section 3.2   each selected compressed entry is both key and value for all heads
    section 4     HCA attends over every completed entry
    section 5.1   one candidate list (compressed || window), one softmax per head
    section 5.2   RMSNorm, partial RoPE on the last 64 channels, inverse RoPE at t
    section 5.3   sink logit in the denominator only
  page "transformers PR 45892 discussion": the gathered [S, S*top_k] mask form and the
    scattered [S, compressed_len] mask form give the same attention.
"""
import math

import numpy as np
import pytest

import oracle


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------- RMSNorm/RoPE --- #

def test_rmsnorm_closed_forms():
    x = _rand(0, 5, 64)
    y = oracle.rmsnorm(x, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y ** 2, axis=1)), 1.0, rtol=1e-14)
    assert np.allclose(oracle.rmsnorm(3.5 * x, eps=0.0), y, rtol=1e-14)
    g = np.linspace(0.5, 2.0, 64)
    assert np.allclose(oracle.rmsnorm(x, gamma=g, eps=0.0), y * g, rtol=1e-14)
    # eps enters under the root: a constant row c gives c / sqrt(c^2 + eps)
    c = np.full((1, 8), 0.01)
    assert oracle.rmsnorm(c, eps=1e-4)[0, 0] == pytest.approx(0.01 / math.sqrt(1e-4 + 1e-4))


def test_rope_closed_forms():
    c, rd, base = 16, 8, 10000.0
    e = np.zeros(c)
    e[c - rd] = 1.0  # pair 0 of the rotated slice, theta_0 = 1
    for p in (0.0, 1.0, 2.5, 1000.0):
        r = oracle.rope(e, p, rd, base)
        assert r[c - rd] == pytest.approx(math.cos(p), abs=1e-15)
        assert r[c - rd + 1] == pytest.approx(math.sin(p), abs=1e-15)
    # pair i = rd/4 has theta = base^(-1/2) = 0.01: position 100 turns it by 1 radian
    f = np.zeros(c)
    f[c - rd + 2 * (rd // 4)] = 1.0
    r = oracle.rope(f, 100.0, rd, base)
    assert r[c - rd + 2 * (rd // 4)] == pytest.approx(math.cos(1.0), abs=1e-14)
    assert r[c - rd + 2 * (rd // 4) + 1] == pytest.approx(math.sin(1.0), abs=1e-14)
    x = _rand(1, c)
    assert np.array_equal(oracle.rope(x, 0.0, rd), x)                        # identity at 0
    assert np.array_equal(oracle.rope(x, 37.0, rd)[:c - rd], x[:c - rd])     # leading channels kept
    assert np.linalg.norm(oracle.rope(x, 37.0, rd)) == pytest.approx(np.linalg.norm(x))
    assert np.allclose(oracle.rope(oracle.rope(x, 13.0, rd), 29.0, rd), oracle.rope(x, 42.0, rd),
                       atol=1e-13)                                          # composition
    assert np.allclose(oracle.rope(oracle.rope(x, 77.0, rd), -77.0, rd), x, atol=1e-13)  # inverse
    # logits depend on relative position only
    q, k = _rand(2, c), _rand(3, c)
    a = oracle.rope(q, 50.0, rd) @ oracle.rope(k, 20.0, rd)
    b = oracle.rope(q, 1050.0, rd) @ oracle.rope(k, 1020.0, rd)
    assert a == pytest.approx(b, abs=1e-11)


# ------------------------------------------------------------- attention --- #

def _problem(seed, n=40, c=16, n_h=3, m=4, k=3, w=5, cI=8, n_hI=2):
    q = _rand(seed, n, n_h, c)
    local = _rand(seed + 1, n, c)
    E = n // m
    kv = _rand(seed + 2, E, c)
    qI = _rand(seed + 3, n, n_hI, cI)
    KI = _rand(seed + 4, E, cI)
    wI = np.random.default_rng(seed + 5).random((n, n_hI))
    sc = oracle.index_scores(qI, KI, wI, t0=0, m=m, ld=E)
    idx, cnt = oracle.topk(sc, t0=0, m=m, k=k)
    return dict(q=q, local=local, kv=kv, idx=idx, cnt=cnt, n=n, c=c, n_h=n_h, m=m, k=k, w=w, E=E)


def test_single_candidate_returns_its_row():
    """t = 0: the only candidate is local row 0; softmax of one logit is 1."""
    c = 16
    q = _rand(0, 1, 2, c)
    local = _rand(1, 1, c)
    idx = -np.ones((1, 4), np.int32)
    cnt = np.zeros(1, np.int32)
    out = oracle.attend_csa(q, np.zeros((1, c)), local, idx, cnt, loc_base=0, t0=0, w=8,
                            q_norm=True, kv_norm=True, eps=0.0, rope_dims=8)
    y = local[0] / np.sqrt(np.mean(local[0] ** 2))  # RoPE at 0 and inverse at 0 are identities
    assert np.allclose(out[0], np.tile(y, (2, 1)), atol=1e-14)
    # with w = 1 at t > 0 the only candidate is token t itself: RoPE_t then RoPE_-t cancel
    qq = _rand(2, 10, 2, c)
    ll = _rand(3, 10, c)
    out = oracle.attend_csa(qq, np.zeros((1, c)), ll, -np.ones((10, 4), np.int32),
                            np.zeros(10, np.int32), loc_base=0, t0=0, w=1, q_norm=True,
                            kv_norm=True, eps=0.0, rope_dims=8)
    for t in range(10):
        y = ll[t] / np.sqrt(np.mean(ll[t] ** 2))
        assert np.allclose(out[t], np.tile(y, (2, 1)), atol=1e-13)


def test_sink_closed_form():
    """All N candidates equal u: a = 1/(N + exp(z' - z)) and o = u * N/(N + exp(z' - z))."""
    c, n_h, w, m = 8, 4, 6, 4
    n = 20
    u = _rand(0, c)
    q = _rand(1, n, n_h, c)
    local = np.tile(u, (n, 1))
    E = n // m
    kv = np.tile(u, (E, 1))
    k = 3
    idx = np.full((n, k), -1, np.int32)
    cnt = np.zeros(n, np.int32)
    for t in range(n):
        e = min(k, (t + 1) // m)
        idx[t, :e] = np.arange(e)
        cnt[t] = e
    sink = np.array([-1.0, 0.0, 0.5, 3.0])
    scale = 1.0 / math.sqrt(c)
    out = oracle.attend_csa(q, kv, local, idx, cnt, loc_base=0, t0=0, w=w, sink=sink, scale=scale)
    for t in range(n):
        N = cnt[t] + min(w, t + 1)
        for h in range(n_h):
            z = scale * q[t, h] @ u
            assert np.allclose(out[t, h], u * N / (N + math.exp(sink[h] - z)), rtol=1e-13)
    none = oracle.attend_csa(q, kv, local, idx, cnt, loc_base=0, t0=0, w=w)
    minf = oracle.attend_csa(q, kv, local, idx, cnt, loc_base=0, t0=0, w=w,
                             sink=np.full(n_h, -np.inf))
    assert np.array_equal(none, minf)
    assert np.allclose(none, np.tile(u, (n, n_h, 1)), rtol=1e-14)


def _dense_attention(logits, values):
    """Textbook masked softmax attention; -inf entries carry zero weight."""
    mx = logits.max(axis=-1, keepdims=True)
    p = np.exp(logits - mx)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ values


def test_two_mask_forms_equal_index_form():
    P = _problem(10)
    q, local, kv, idx, cnt = P["q"], P["local"], P["kv"], P["idx"], P["cnt"]
    n, c, n_h, k, w, E = P["n"], P["c"], P["n_h"], P["k"], P["w"], P["E"]
    scale = 1.0 / math.sqrt(c)
    ref = oracle.attend_csa(q, kv, local, idx, cnt, loc_base=0, t0=0, w=w)
    valid = np.arange(k)[None, :] < cnt[:, None]
    # window mask [S, S]: 0 where j in L_t
    t = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    win = np.where((j <= t) & (j > t - w), 0.0, -np.inf)
    # gather form: flat KV [S*k, c], mask [S, S*k] is 0 only on the query's own valid slots
    flat = kv[np.where(valid, idx, 0).reshape(-1)]
    gmask = np.full((n, n, k), -np.inf)
    gmask[np.arange(n), np.arange(n), :] = np.where(valid, 0.0, -np.inf)
    gmask = gmask.reshape(n, n * k)
    # scatter form: mask [S, E+1], invalid slots redirected to a dummy column then dropped
    safe = np.where(valid, idx, E)
    smask = np.full((n, E + 1), -np.inf)
    np.put_along_axis(smask, safe, 0.0, axis=1)
    smask = smask[:, :E]
    for h in range(n_h):
        qh = q[:, h, :]
        lg = np.concatenate([qh @ flat.T * scale + gmask, qh @ local.T * scale + win], axis=1)
        og = _dense_attention(lg, np.concatenate([flat, local]))
        ls = np.concatenate([qh @ kv.T * scale + smask, qh @ local.T * scale + win], axis=1)
        os_ = _dense_attention(ls, np.concatenate([kv, local]))
        assert np.allclose(og, ref[:, h], rtol=1e-12, atol=1e-13)
        assert np.allclose(os_, ref[:, h], rtol=1e-12, atol=1e-13)


def test_full_topk_equals_dense_hca_routine():
    """k >= visible entries: CSA over top-k equals attention over every completed entry (HCA routine, m' := m)."""
    P = _problem(20, k=64)
    kw = dict(loc_base=0, t0=0, w=P["w"], q_norm=True, kv_norm=True, rope_dims=8,
              sink=np.array([0.3, -0.2, 1.0]))
    csa = oracle.attend_csa(P["q"], P["kv"], P["local"], P["idx"], P["cnt"], **kw)
    hca = oracle.attend_hca(P["q"], P["kv"], P["local"], m_prime=P["m"], **kw)
    assert np.allclose(csa, hca, rtol=1e-13, atol=1e-14)


def test_candidate_order_does_not_matter_and_rows_subset():
    P = _problem(30)
    kw = dict(loc_base=0, t0=0, w=P["w"], q_norm=True, kv_norm=True, rope_dims=8)
    ref = oracle.attend_csa(P["q"], P["kv"], P["local"], P["idx"], P["cnt"], **kw)
    idx2 = P["idx"].copy()
    for t in range(P["n"]):
        idx2[t, :P["cnt"][t]] = idx2[t, :P["cnt"][t]][::-1]
    out = oracle.attend_csa(P["q"], P["kv"], P["local"], idx2, P["cnt"], **kw)
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-14)
    rows = np.array([3, 17, 39])
    sub = oracle.attend_csa(P["q"], P["kv"], P["local"], P["idx"], P["cnt"], rows=rows, **kw)
    assert np.array_equal(sub, ref[rows])


def test_chunked_prefill_equals_unchunked():
    """Scores, top-k and attention of the chunk [t0, t0+T) equal rows t0.. of the full prefill."""
    P = _problem(40, n=64)
    rng = np.random.default_rng(41)
    qI = rng.standard_normal((64, 2, 8))
    KI = rng.standard_normal((16, 8))
    wI = rng.random((64, 2))
    kw = dict(w=P["w"], q_norm=True, kv_norm=True, rope_dims=8)
    sc = oracle.index_scores(qI, KI, wI, t0=0, m=4, ld=16)
    idx, cnt = oracle.topk(sc, t0=0, m=4, k=3)
    full = oracle.attend_csa(P["q"], P["kv"], P["local"], idx, cnt, loc_base=0, t0=0, **kw)
    for t0, T in ((0, 24), (24, 17), (41, 23)):
        s2 = oracle.index_scores(qI[t0:t0 + T], KI, wI[t0:t0 + T], t0=t0, m=4, ld=16)
        i2, c2 = oracle.topk(s2, t0=t0, m=4, k=3)
        assert np.array_equal(i2, idx[t0:t0 + T]) and np.array_equal(c2, cnt[t0:t0 + T])
        lb = max(0, t0 - P["w"] + 1)  # the chunk only brings the local rows it needs
        out = oracle.attend_csa(P["q"][t0:t0 + T], P["kv"], P["local"][lb:t0 + T], i2, c2,
                                loc_base=lb, t0=t0, **kw)
        assert np.array_equal(out, full[t0:t0 + T])


def test_scale_and_query_norm_invariance():
    """With q normalised, scaling q changes nothing; doubling scale equals squaring weights' temperature."""
    P = _problem(50)
    kw = dict(loc_base=0, t0=0, w=P["w"], kv_norm=True, rope_dims=8)
    a = oracle.attend_csa(P["q"], P["kv"], P["local"], P["idx"], P["cnt"], q_norm=True, eps=0.0, **kw)
    b = oracle.attend_csa(5.0 * P["q"], P["kv"], P["local"], P["idx"], P["cnt"], q_norm=True,
                          eps=0.0, **kw)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-14)
    c1 = oracle.attend_csa(2.0 * P["q"], P["kv"], P["local"], P["idx"], P["cnt"], scale=0.25, **kw)
    c2 = oracle.attend_csa(P["q"], P["kv"], P["local"], P["idx"], P["cnt"], scale=0.5, **kw)
    assert np.allclose(c1, c2, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------ RoPE positions --- #

def _rot_complex(x, pos, rd, base=10000.0):
    """Partial RoPE written in complex form: the pair (x[c-rd+2i], x[c-rd+2i+1]) is the
    complex number a + ib, multiplied by exp(i * pos * base^(-2i/rd))."""
    y = np.array(x, dtype=np.float64, copy=True)
    c = y.shape[-1]
    z = y[..., c - rd::2] + 1j * y[..., c - rd + 1::2]
    z = z * np.exp(1j * pos * base ** (-2.0 * np.arange(rd // 2) / rd))
    y[..., c - rd::2], y[..., c - rd + 1::2] = z.real, z.imag
    return y


def _norm(x):
    return x / np.sqrt(np.mean(x ** 2, axis=-1, keepdims=True))


def _attention_by_positions(q_t, t, comp_rows, local_rows, local_pos, sink, rd, c):
    """Dense softmax over [compressed rows as stored || window rows rotated at their own
    position], query rotated at t, output rotated back at t ("CSA And HCA" section 5.2)."""
    cands = np.concatenate([comp_rows.reshape(-1, c),
                            _rot_complex(_norm(local_rows), np.asarray(local_pos)[:, None], rd)])
    out = np.empty_like(q_t)
    for h in range(q_t.shape[0]):
        qh = _rot_complex(_norm(q_t[h]), t, rd)
        z = cands @ qh / math.sqrt(c)
        mx = max(z.max(), sink[h]) if sink is not None else z.max()
        e = np.exp(z - mx)
        den = e.sum() + (math.exp(sink[h] - mx) if sink is not None else 0.0)
        out[h] = _rot_complex((e / den) @ cands, -t, rd)
    return out


@pytest.mark.parametrize("kind", ["csa", "hca", "decode"])
def test_rope_positions_in_attention(kind):
    """Several candidates, w >= 3, RoPE on: the query turns at t, window row j at j, stored
    compressed rows are not turned again, and the output turns back at t.  Rotating a
    window row at t, or leaving the query unrotated, changes the result (checked)."""
    c, rd, n_h, m, w, k, n = 16, 8, 2, 4, 4, 3, 28
    rng = np.random.default_rng(123)
    q = rng.standard_normal((n, n_h, c))
    local = rng.standard_normal((n, c))
    E = n // m
    # stored entries: already normalised and turned at their anchor m*s
    kv = _rot_complex(_norm(rng.standard_normal((E, c))), (m * np.arange(E))[:, None], rd)
    sink = np.array([0.4, -0.7])
    idx = -np.ones((n, k), np.int32)
    cnt = np.zeros(n, np.int32)
    for t in range(n):
        e = min(k, (t + 1) // m)
        idx[t, :e] = np.sort(rng.choice((t + 1) // m, e, replace=False)) if e else []
        cnt[t] = e
    kw = dict(q_norm=True, kv_norm=True, eps=0.0, rope_dims=rd, sink=sink)
    if kind == "csa":
        got = oracle.attend_csa(q, kv, local, idx, cnt, loc_base=0, t0=0, w=w, **kw)
    elif kind == "hca":
        got = oracle.attend_hca(q, kv, local, loc_base=0, t0=0, m_prime=m, w=w, **kw)
    else:
        got = np.empty((n, n_h, c))
        for t in range(n):
            ring = np.full((w, c), np.nan)
            for j in range(max(0, t - w + 1), t + 1):
                ring[j % w] = local[j]
            got[t] = oracle.attend_decode(q[t], kv, ring, idx[t], int(cnt[t]), t=t, w=w, **kw)
    sens_win = sens_q = 0.0
    for t in range(n):
        lo = max(0, t - w + 1)
        pos = np.arange(lo, t + 1)
        comp = kv[: (t + 1) // m] if kind == "hca" else kv[idx[t, :cnt[t]]]
        ref = _attention_by_positions(q[t], t, comp, local[lo:t + 1], pos, sink, rd, c)
        assert np.allclose(got[t], ref, rtol=1e-12, atol=1e-13), (kind, t)
        # the two plausible mistakes move the result far beyond that tolerance
        wrong_win = _attention_by_positions(q[t], t, comp, local[lo:t + 1], np.full(pos.size, t),
                                            sink, rd, c)
        sens_win = max(sens_win, np.abs(wrong_win - ref).max())
        wrong_q = _attention_by_positions(_rot_complex(q[t], -t, rd), t, comp, local[lo:t + 1],
                                          pos, sink, rd, c)
        sens_q = max(sens_q, np.abs(wrong_q - ref).max())
    assert sens_win > 1e-3 and sens_q > 1e-3
