"""The float64 oracle against an independent pure-Python brute force of the whole
chain on tiny inputs (n <= 64): CSA (both compressors, indexer, top-k, attention
with window, RMSNorm, RoPE and sink) and HCA (one-stream compressor, dense
attention).  The brute force lives in tests/bruteforce.py and shares no code
with the oracle.
"""
import numpy as np
import pytest

import bruteforce as bf
import oracle


def _csa_problem(seed, n=64, c=16, cI=8, n_h=3, n_hI=2, m=4, k=5, w=6, rd=8):
    rng = np.random.default_rng(seed)
    P = dict(n=n, c=c, cI=cI, n_h=n_h, n_hI=n_hI, m=m, k=k, w=w, rd=rd, eps=1e-6)
    P["C"], P["Z"] = rng.standard_normal((n, 2 * c)), rng.standard_normal((n, 2 * c))
    P["CI"], P["ZI"] = rng.standard_normal((n, 2 * cI)), rng.standard_normal((n, 2 * cI))
    P["B"] = np.sqrt(0.1) * rng.standard_normal((2 * m, c))
    P["BI"] = np.sqrt(0.1) * rng.standard_normal((2 * m, cI))
    P["local"] = rng.standard_normal((n, c))
    P["q"] = rng.standard_normal((n, n_h, c))
    P["qI"] = rng.standard_normal((n, n_hI, cI))
    P["wI"] = rng.random((n, n_hI))
    P["gamma"] = 1.0 + 0.2 * rng.standard_normal(c)
    P["gammaI"] = 1.0 + 0.2 * rng.standard_normal(cI)
    P["sink"] = rng.standard_normal(n_h)
    return P


def _lists(P):
    """numpy arrays -> nested Python lists for the brute force."""
    return {k: (v.tolist() if isinstance(v, np.ndarray) else v) for k, v in P.items()}


@pytest.mark.parametrize("seed", [0, 1])
def test_csa_chain_matches_bruteforce(seed):
    P = _csa_problem(seed)
    n, c, cI, m, k, w, rd = (P[x] for x in ("n", "c", "cI", "m", "k", "w", "rd"))
    E = n // m
    ref = bf.csa_chain(_lists(P))
    kv = oracle.compress(P["C"], P["Z"], P["B"], tok_base=0, i_begin=0, i_end=E, c=c, m=m,
                         overlap=True, gamma=P["gamma"], rope_dims=rd)
    KI = oracle.compress(P["CI"], P["ZI"], P["BI"], tok_base=0, i_begin=0, i_end=E, c=cI, m=m,
                         overlap=True, gamma=P["gammaI"])
    assert np.allclose(kv, ref["kv"], rtol=1e-12, atol=1e-13)
    assert np.allclose(KI, ref["KI"], rtol=1e-12, atol=1e-13)
    sc = oracle.index_scores(P["qI"], KI, P["wI"], t0=0, m=m, ld=E)
    for t in range(n):
        Et = (t + 1) // m
        assert np.allclose(sc[t, :Et], ref["scores"][t], rtol=1e-12, atol=1e-12), t
    idx, cnt = oracle.topk(sc, t0=0, m=m, k=k)
    for t in range(n):
        assert idx[t, :cnt[t]].tolist() == ref["idx"][t], t
        assert np.all(idx[t, cnt[t]:] == -1)
    out = oracle.attend_csa(P["q"], kv, P["local"], idx, cnt, loc_base=0, t0=0, w=w,
                            sink=P["sink"], q_gamma=P["gamma"], kv_gamma=P["gamma"], q_norm=True,
                            kv_norm=True, rope_dims=rd)
    assert np.allclose(out, np.array(ref["out"]), rtol=1e-11, atol=1e-12)


def test_csa_decode_steps_match_bruteforce():
    """The oracle's decode step (ring, tail emission, selection, attention) at every position
    of a 40-token sequence equals brute-force prefill row t."""
    P = _csa_problem(7, n=40)
    n, c, cI, m, k, w, rd = (P[x] for x in ("n", "c", "cI", "m", "k", "w", "rd"))
    ref = bf.csa_chain(_lists(P))
    st = {"kv_comp": np.zeros((n // m, c)), "KI": np.zeros((n // m, cI)),
          "ring": np.full((w, c), np.nan), "B": P["B"], "BI": P["BI"]}
    for t in range(n):
        i = t // m
        base = max(0, m * (i - 1))
        for nm, src in (("tail_C", "C"), ("tail_Z", "Z"), ("tail_CI", "CI"), ("tail_ZI", "ZI")):
            st[nm] = P[src][base:m * (i + 1)]
        st["tail_base"] = base
        st["kv_new"], st["q"], st["qI"], st["wI"] = P["local"][t], P["q"][t], P["qI"][t], P["wI"][t]
        r = oracle.decode_step(st, t=t, c=c, cI=cI, m=m, k=k, w=w, rope_dims=rd,
                               gamma=P["gamma"], gammaI=P["gammaI"], q_gamma=P["gamma"],
                               kv_gamma=P["gamma"], sink=P["sink"])
        assert r["idx"][:r["cnt"]].tolist() == ref["idx"][t], t
        assert np.allclose(r["out"], np.array(ref["out"][t]), rtol=1e-11, atol=1e-12), t


def test_hca_chain_matches_bruteforce():
    rng = np.random.default_rng(3)
    n, c, n_h, mp, w, rd = 64, 16, 2, 8, 5, 8
    P = dict(n=n, c=c, mp=mp, w=w, rd=rd, eps=1e-6)
    P["C"], P["Z"] = rng.standard_normal((n, c)), rng.standard_normal((n, c))
    P["B"] = np.sqrt(0.1) * rng.standard_normal((mp, c))
    P["local"] = rng.standard_normal((n, c))
    P["q"] = rng.standard_normal((n, n_h, c))
    P["gamma"] = 1.0 + 0.2 * rng.standard_normal(c)
    P["sink"] = rng.standard_normal(n_h)
    ref = bf.hca_chain(_lists(P))
    kv = oracle.compress(P["C"], P["Z"], P["B"], tok_base=0, i_begin=0, i_end=n // mp, c=c, m=mp,
                         overlap=False, gamma=P["gamma"], rope_dims=rd)
    assert np.allclose(kv, ref["kv"], rtol=1e-12, atol=1e-13)
    out = oracle.attend_hca(P["q"], kv, P["local"], loc_base=0, t0=0, m_prime=mp, w=w,
                            sink=P["sink"], q_gamma=P["gamma"], kv_gamma=P["gamma"], q_norm=True,
                            kv_norm=True, rope_dims=rd)
    assert np.allclose(out, np.array(ref["out"]), rtol=1e-11, atol=1e-12)
