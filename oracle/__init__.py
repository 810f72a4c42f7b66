"""CPU oracle for the CSA/HCA hot path (float64).  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It is independent of the GPU library: it loads its own C
library (liboracle.so, built from v4a_oracle.c by oracle/build.py) and decodes
stored tensors with its own decoders.

Functions follow "CSA And HCA: Definition, State, And Cost Model" ([Def]):
  sets           -- section 1 (completed entries) and 5.1 (window)
  compress       -- sections 2.1 / 2.2 (+ 5.2 RMSNorm and RoPE on the entry)
  index_scores   -- section 3.1 (lightning-indexer score)
  topk           -- section 3.1 (TopK over completed entries)
  attend_csa     -- sections 3.2, 5.1-5.3 (one softmax over top-k entries + window)
  attend_hca     -- sections 4, 5.1-5.3 (all completed entries + window)
  decode_step    -- section 7 (incremental decode order)
  linear         -- the projections around the path (sections 2.1, 3.1, 3.2, 5.1)
  grouped_out_proj -- section 5.4 (grouped output projection)

Parity pins for every function live in tests/test_oracle_*.py.
"""
from __future__ import annotations

import ctypes as ct
import math
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_d = ct.POINTER(ct.c_double)
_i32 = ct.POINTER(ct.c_int32)
_i64 = ct.POINTER(ct.c_int64)


def lib():
    global _lib
    if _lib is None:
        # V4A_ORACLE_LIB names another build of the oracle (the sanitizer checking build)
        path = os.environ.get("V4A_ORACLE_LIB") or _build.library_path()
        if not os.environ.get("V4A_ORACLE_LIB") and (not os.path.exists(path) or _build.is_stale()):
            _build.build()
        L = ct.CDLL(path)
        I64, INT, DBL = ct.c_int64, ct.c_int, ct.c_double
        L.v4o_visible_count.restype = I64
        L.v4o_visible_count.argtypes = [I64, I64]
        L.v4o_sets.argtypes = [I64, I64, I64, I64, I64, _i32, _i32, _i32, _i32]
        L.v4o_rmsnorm.argtypes = [_d, I64, _d, DBL, _d]
        L.v4o_rope.argtypes = [_d, I64, I64, DBL, DBL]
        L.v4o_compress.restype = INT
        L.v4o_compress.argtypes = [_d, _d, I64, I64, I64, I64, I64, I64, INT, _d, _d, DBL, I64,
                                   DBL, _d]
        L.v4o_index_scores.argtypes = [_d, _d, _d, I64, I64, I64, I64, I64, I64, _d]
        L.v4o_topk.argtypes = [_d, I64, I64, I64, I64, I64, _i32, _i32]
        L.v4o_attend_csa.argtypes = [_d, _d, _d, I64, _i32, _i32, I64, _d, _d, _d, INT, INT, DBL,
                                     I64, DBL, DBL, I64, I64, I64, I64, _i64, I64, _d]
        L.v4o_attend_hca.argtypes = [_d, _d, _d, I64, _d, _d, _d, INT, INT, DBL, I64, DBL, DBL,
                                     I64, I64, I64, I64, I64, _i64, I64, _d]
        L.v4o_attend_decode.argtypes = [_d, _d, _d, I64, _i32, I64, _d, _d, _d, INT, INT, DBL,
                                        I64, DBL, DBL, I64, I64, I64, _d]
        L.v4o_decode_bf16.argtypes = [ct.POINTER(ct.c_uint16), I64, _d]
        L.v4o_decode_fp8_rows.argtypes = [ct.POINTER(ct.c_uint8), ct.POINTER(ct.c_float), I64, I64,
                                          _d]
        L.v4o_decode_mxfp4_rows.argtypes = [ct.POINTER(ct.c_uint8), ct.POINTER(ct.c_uint8), I64,
                                            I64, _d]
        L.v4o_num_threads.restype = INT
        _lib = L
    return _lib


def _pd(a):
    return None if a is None else a.ctypes.data_as(_d)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    return lib().v4o_num_threads()


# --------------------------------------------------------------------------- #
# decoders of stored formats
# --------------------------------------------------------------------------- #

def decode_bf16(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().v4o_decode_bf16(b.ctypes.data_as(ct.POINTER(ct.c_uint16)), b.size, _pd(out))
    return out


def decode_fp8_rows(codes, scale=None) -> np.ndarray:
    cd = np.ascontiguousarray(codes, dtype=np.uint8)
    cols = cd.shape[-1]
    rows = cd.size // cols
    sc = None if scale is None else np.ascontiguousarray(scale, dtype=np.float32)
    out = np.empty(cd.shape, np.float64)
    lib().v4o_decode_fp8_rows(cd.ctypes.data_as(ct.POINTER(ct.c_uint8)),
                              None if sc is None else sc.ctypes.data_as(ct.POINTER(ct.c_float)),
                              rows, cols, _pd(out))
    return out


def decode_mxfp4_rows(packed, e8m0) -> np.ndarray:
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    s = np.ascontiguousarray(e8m0, dtype=np.uint8)
    cols = p.shape[-1] * 2
    rows = p.size // p.shape[-1]
    out = np.empty(p.shape[:-1] + (cols,), np.float64)
    lib().v4o_decode_mxfp4_rows(p.ctypes.data_as(ct.POINTER(ct.c_uint8)),
                                s.ctypes.data_as(ct.POINTER(ct.c_uint8)), rows, cols, _pd(out))
    return out


def decode_kv576_rows(rows, scale, c=512, rope_dims=64) -> np.ndarray:
    """Production main-cache rows ("CSA And HCA: Definition, State, And Cost Model",
    section 8: FP8 for the c - rope_dims leading channels, BF16 for the RoPE channels):
    bytes [..][c + rope_dims] = E4M3 codes times the row's float32 scale, then the
    little-endian bf16 channels."""
    r = np.ascontiguousarray(rows, dtype=np.uint8)
    nq = c - rope_dims
    lead = decode_fp8_rows(r[..., :nq].reshape(-1, nq), np.asarray(scale, np.float32).reshape(-1))
    tail = decode_bf16(np.ascontiguousarray(r[..., nq:]).view(np.uint16).reshape(-1, rope_dims))
    return np.concatenate([lead, tail], axis=1).reshape(r.shape[:-1] + (c,))


def decode(x, dt: str, scale=None) -> np.ndarray:
    """Stored array -> float64 for dt in {'f32', 'bf16', 'fp8', 'mxfp4'}."""
    if dt == "f32":
        return np.asarray(x, dtype=np.float64)
    if dt == "bf16":
        return decode_bf16(x)
    if dt == "fp8":
        return decode_fp8_rows(x, scale)
    if dt == "mxfp4":
        return decode_mxfp4_rows(x, scale)
    if dt == "kv576":
        return decode_kv576_rows(x, scale)
    raise ValueError(dt)


# --------------------------------------------------------------------------- #
# method
# --------------------------------------------------------------------------- #

def visible_count(t: int, r: int) -> int:
    return int(lib().v4o_visible_count(t, r))


def sets(t0: int, T: int, m: int, k: int, w: int) -> dict:
    out = {n: np.empty(T, np.int32) for n in ("E", "cnt", "win_lo", "win_len")}
    lib().v4o_sets(t0, T, m, k, w, *(out[n].ctypes.data_as(_i32)
                                     for n in ("E", "cnt", "win_lo", "win_len")))
    return out


def rmsnorm(x, gamma=None, eps=1e-6) -> np.ndarray:
    x = _f64(x)
    y = np.empty_like(x)
    g = _f64(gamma)
    for r in range(x.shape[0] if x.ndim > 1 else 1):
        xr = x[r] if x.ndim > 1 else x
        yr = y[r] if x.ndim > 1 else y
        lib().v4o_rmsnorm(_pd(xr), xr.size, _pd(g), eps, _pd(yr))
    return y


def rope(x, pos, rope_dims, base=10000.0) -> np.ndarray:
    """Rotate the last rope_dims channels of each row of x by position pos (scalar or per row)."""
    y = np.array(x, dtype=np.float64, copy=True)
    rows = y.reshape(-1, y.shape[-1])
    pos = np.broadcast_to(np.asarray(pos, dtype=np.float64), (rows.shape[0],))
    for r in range(rows.shape[0]):
        row = np.ascontiguousarray(rows[r])
        lib().v4o_rope(_pd(row), row.size, rope_dims, base, float(pos[r]))
        rows[r] = row
    return rows.reshape(y.shape)


def compress(C, Z, B, *, tok_base, i_begin, i_end, c, m, overlap, gamma=None, eps=1e-6,
             rope_dims=0, rope_base=10000.0) -> np.ndarray:
    C, Z, B, g = _f64(C), _f64(Z), _f64(B), _f64(gamma)
    n_buf = C.shape[0]
    out = np.empty((max(i_end - i_begin, 0), c), np.float64)
    rc = lib().v4o_compress(_pd(C), _pd(Z), n_buf, tok_base, i_begin, i_end, c, m, int(overlap),
                            _pd(B), _pd(g), eps, rope_dims, rope_base, _pd(out))
    if rc != 0:
        raise ValueError("compress: rows needed for the requested entries are not in the buffer")
    return out


def index_scores(qI, KI, wI, *, t0, m, ld=None) -> np.ndarray:
    qI, KI, wI = _f64(qI), _f64(KI), _f64(wI)
    T, n_hI, cI = qI.shape
    ld = ld if ld is not None else max(visible_count(t0 + T - 1, m), 1)
    out = np.empty((T, ld), np.float64)
    lib().v4o_index_scores(_pd(qI), _pd(KI), _pd(wI), T, t0, n_hI, cI, m, ld, _pd(out))
    return out


def topk(scores, *, t0, m, k):
    s = _f64(scores)
    T, ld = s.shape
    idx = np.empty((T, k), np.int32)
    cnt = np.empty(T, np.int32)
    lib().v4o_topk(_pd(s), T, t0, m, k, ld, idx.ctypes.data_as(_i32), cnt.ctypes.data_as(_i32))
    return idx, cnt


def _rows_arg(rows, T):
    if rows is None:
        return None, T
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, r.size


def attend_csa(q, kv_comp, kv_local, idx, cnt, *, loc_base, t0, w, sink=None, q_gamma=None,
               kv_gamma=None, q_norm=False, kv_norm=False, eps=1e-6, rope_dims=0,
               rope_base=10000.0, scale=None, rows=None) -> np.ndarray:
    q, kc, kl, sk = _f64(q), _f64(kv_comp), _f64(kv_local), _f64(sink)
    T, n_h, c = q.shape
    k = idx.shape[1]
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    idx = np.ascontiguousarray(idx, np.int32)
    cnt = np.ascontiguousarray(cnt, np.int32)
    r, nr = _rows_arg(rows, T)
    out = np.empty((nr, n_h, c), np.float64)
    lib().v4o_attend_csa(_pd(q), _pd(kc), _pd(kl), loc_base, idx.ctypes.data_as(_i32),
                         cnt.ctypes.data_as(_i32), k, _pd(sk), _pd(_f64(q_gamma)),
                         _pd(_f64(kv_gamma)), int(q_norm), int(kv_norm), eps, rope_dims,
                         rope_base, scale, t0, n_h, c, w,
                         None if r is None else r.ctypes.data_as(_i64), nr, _pd(out))
    return out


def attend_hca(q, kv_comp, kv_local, *, loc_base, t0, m_prime, w, sink=None, q_gamma=None,
               kv_gamma=None, q_norm=False, kv_norm=False, eps=1e-6, rope_dims=0,
               rope_base=10000.0, scale=None, rows=None) -> np.ndarray:
    q, kc, kl, sk = _f64(q), _f64(kv_comp), _f64(kv_local), _f64(sink)
    T, n_h, c = q.shape
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    r, nr = _rows_arg(rows, T)
    out = np.empty((nr, n_h, c), np.float64)
    lib().v4o_attend_hca(_pd(q), _pd(kc), _pd(kl), loc_base, _pd(sk), _pd(_f64(q_gamma)),
                         _pd(_f64(kv_gamma)), int(q_norm), int(kv_norm), eps, rope_dims,
                         rope_base, scale, t0, n_h, c, m_prime, w,
                         None if r is None else r.ctypes.data_as(_i64), nr, _pd(out))
    return out


def attend_decode(q, kv_comp, ring, idx, cnt, *, t, w, sink=None, q_gamma=None, kv_gamma=None,
                  q_norm=False, kv_norm=False, eps=1e-6, rope_dims=0, rope_base=10000.0,
                  scale=None) -> np.ndarray:
    """One sequence: q [n_h][c], ring [w][c] already holding token t in slot t % w."""
    q, kc, rg, sk = _f64(q), _f64(kv_comp), _f64(ring), _f64(sink)
    n_h, c = q.shape
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    idx = np.ascontiguousarray(idx, np.int32)
    out = np.empty((n_h, c), np.float64)
    lib().v4o_attend_decode(_pd(q), _pd(kc), _pd(rg), t, idx.ctypes.data_as(_i32), int(cnt),
                            _pd(sk), _pd(_f64(q_gamma)), _pd(_f64(kv_gamma)), int(q_norm),
                            int(kv_norm), eps, rope_dims, rope_base, scale, n_h, c, w, _pd(out))
    return out


def linear(X, W) -> np.ndarray:
    """A projection of the layer around the path (sections 2.1, 3.1, 3.2, 5.1):
    Y[t][n] = sum_k X[t][k] W[n][k] in float64."""
    return _f64(X) @ _f64(W).T


def grouped_out_proj(o, W_A, W_B) -> np.ndarray:
    """Section 5.4: out_t = W^{O,B} [W^{O,A}_1 o^G_{t,1}; ...; W^{O,A}_g o^G_{t,g}] in float64.
    o [T][n_h][c]; W_A [g][d_g][c n_h/g]; W_B [d][g d_g]; group i is heads
    i n_h/g .. (i+1) n_h/g - 1, concatenated in head order."""
    o, W_A, W_B = _f64(o), _f64(W_A), _f64(W_B)
    T, n_h, c = o.shape
    g, d_g, Kg = W_A.shape
    assert n_h % g == 0 and Kg == c * (n_h // g)
    mid = np.empty((T, g, d_g))
    for i in range(g):
        oG = o[:, i * (n_h // g):(i + 1) * (n_h // g), :].reshape(T, Kg)
        mid[:, i, :] = oG @ W_A[i].T
    return mid.reshape(T, g * d_g) @ W_B.T


def decode_step(state: dict, *, t, c, cI, m, k, w, rope_dims, rope_base=10000.0, eps=1e-6,
                gamma=None, gammaI=None, q_gamma=None, kv_gamma=None, q_norm=True,
                kv_norm=True, sink=None, scale=None):
    """One CSA decode step for one sequence, in the order of [Def] section 7.

    state (float64 arrays, modified in place):
      kv_comp [E_cap][c], KI [E_cap][cI]   -- entries 0 .. floor(t/m)-1 valid
      ring [w][c]                          -- token j at slot j % w, j < t
      tail_C, tail_Z [rows][2c], tail_CI, tail_ZI [rows][2cI], tail_base  -- raw rows
      B [2m][c], BI [2m][cI]
      kv_new [c], q [n_h][c], qI [n_hI][cI], wI [n_hI]
    Returns dict(out=[n_h][c], idx=[k], cnt=int, emitted=bool, scores=[E]).
    """
    # 1. the new token's local entry goes into the w-slot ring
    state["ring"][t % w] = state["kv_new"]
    emitted = (t + 1) % m == 0
    if emitted:
        i = (t + 1) // m - 1
        # 2.-4. completed block: emit one main and one indexer entry
        state["kv_comp"][i] = compress(state["tail_C"], state["tail_Z"], state["B"],
                                       tok_base=state["tail_base"], i_begin=i, i_end=i + 1, c=c,
                                       m=m, overlap=True, gamma=gamma, eps=eps,
                                       rope_dims=rope_dims, rope_base=rope_base)[0]
        state["KI"][i] = compress(state["tail_CI"], state["tail_ZI"], state["BI"],
                                  tok_base=state["tail_base"], i_begin=i, i_end=i + 1, c=cI, m=m,
                                  overlap=True, gamma=gammaI, eps=eps)[0]
    # 5. eligible set, top-k, window, shared-KV MQA
    E = visible_count(t, m)
    sc = index_scores(state["qI"][None], state["KI"][:max(E, 1)], state["wI"][None], t0=t, m=m,
                      ld=max(E, 1))
    idx, cnt = topk(sc, t0=t, m=m, k=k)
    out = attend_decode(state["q"], state["kv_comp"], state["ring"], idx[0], cnt[0], t=t, w=w,
                        sink=sink, q_gamma=q_gamma, kv_gamma=kv_gamma, q_norm=q_norm,
                        kv_norm=kv_norm, eps=eps, rope_dims=rope_dims, rope_base=rope_base,
                        scale=scale)
    return dict(out=out, idx=idx[0], cnt=int(cnt[0]), emitted=emitted, scores=sc[0, :E])
