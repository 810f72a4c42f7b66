"""Torch-side plumbing around the C ABI: device uploads, output and workspace
allocation, and the call sequences of a CSA prefill, an HCA prefill and a CSA
decode step.  Every arithmetic step runs in libv4a.so.

Call order follows "CSA And HCA: Definition, State, And Cost Model": section 3
(compression -> indexing -> shared-KV MQA) for prefill and section 7 (ring
insert, compressor updates, emission, selection, attention) for decode.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}
_NP_DT = {"f32": B.F32, "bf16": B.BF16, "fp8": B.FP8_E4M3, "mxfp4": B.MXFP4, "kv576": B.KV576}


def upload(x: np.ndarray, dt: str | None = None, device="cuda") -> torch.Tensor:
    """Stored numpy array -> device tensor (bf16 bit patterns become torch.bfloat16)."""
    x = np.ascontiguousarray(x)
    if dt == "bf16" or (dt is None and x.dtype == np.uint16):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(x).to(device)


def download_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def workspace(nbytes: int, device="cuda") -> torch.Tensor | None:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def dtcode(dt: str) -> int:
    return _NP_DT[dt]


# --------------------------------------------------------------------------- #

def compress(C, Z, B_, *, c, m, overlap, in_dt, out_dt="bf16", t0=0, T=None, tok_base=0,
             gamma=None, eps=1e-6, rope_dims=0, rope_base=10000.0, E_cap=None, out=None,
             out_scale=None, stream=None):
    """C, Z: [batch][n_buf][width] device tensors; returns (out, out_scale)."""
    if C.dim() == 2:
        C, Z = C.unsqueeze(0), Z.unsqueeze(0)
    batch, n_buf = C.shape[0], C.shape[1]
    T = (n_buf + tok_base - t0) if T is None else T
    if E_cap is None:  # rows per sequence of the output cache
        E_cap = out.shape[1] if out is not None else (t0 + T) // m
    dev = C.device
    if out is None:
        if out_dt in ("f32", "bf16"):
            out = torch.empty(batch, E_cap, c, dtype=_TORCH[out_dt], device=dev)
        elif out_dt == "fp8":
            out = torch.empty(batch, E_cap, c, dtype=torch.uint8, device=dev)
            out_scale = torch.empty(batch, E_cap, dtype=torch.float32, device=dev)
        elif out_dt == "kv576":
            out = torch.empty(batch, E_cap, c + rope_dims, dtype=torch.uint8, device=dev)
            out_scale = torch.empty(batch, E_cap, dtype=torch.float32, device=dev)
        else:
            out = torch.empty(batch, E_cap, c // 2, dtype=torch.uint8, device=dev)
            out_scale = torch.empty(batch, E_cap, c // 32, dtype=torch.uint8, device=dev)
    B.v4a_compress(C, Z, _NP_DT[in_dt], B_, batch, n_buf, tok_base, t0, T, c, m, int(overlap),
                   gamma, eps, rope_dims, rope_base, out, out_scale, _NP_DT[out_dt], E_cap, stream)
    return out, out_scale


def indexer_topk(qI, KI, wI, *, dt, m, k, t0=0, qI_scale=None, KI_scale=None, E_cap=None,
                 with_scores=True, stream=None, ws=None):
    """qI [batch][T][n_hI][cI] (MXFP4: [..][cI/2]), KI [batch][E_cap][..]; returns (idx, cnt, score)."""
    if qI.dim() == 3:
        qI, wI = qI.unsqueeze(0), wI.unsqueeze(0)
        KI = KI.unsqueeze(0)
        if KI_scale is not None:
            KI_scale = KI_scale.unsqueeze(0)
            qI_scale = qI_scale.unsqueeze(0)
    batch, T, n_hI = qI.shape[0], qI.shape[1], qI.shape[2]
    cI = qI.shape[3] * (2 if dt == "mxfp4" else 1)
    E_cap = KI.shape[1] if E_cap is None else E_cap
    dev = qI.device
    idx = torch.empty(batch, T, k, dtype=torch.int32, device=dev)
    cnt = torch.empty(batch, T, dtype=torch.int32, device=dev)
    sc = torch.empty(batch, T, k, dtype=torch.float32, device=dev) if with_scores else None
    nbytes = B.v4a_indexer_topk_workspace(batch, T, t0, n_hI, cI, m, k, _NP_DT[dt])
    if ws is None or ws.numel() < nbytes:
        ws = workspace(nbytes, dev)
    B.v4a_indexer_topk(qI, qI_scale, KI, KI_scale, _NP_DT[dt], wI, batch, T, t0, n_hI, cI, m, k,
                       E_cap, idx, cnt, sc, ws, nbytes, stream)
    return idx, cnt, sc


def sparse_mqa_prefill(q, kv_comp, kv_local, idx, cnt, *, t0, w, dt, loc_base=0, sink=None,
                       q_gamma=None, kv_gamma=None, eps=1e-6, rope_dims=0, rope_base=10000.0,
                       scale=0.0, out=None, stream=None):
    if q.dim() == 3:
        q, kv_comp, kv_local = q.unsqueeze(0), kv_comp.unsqueeze(0), kv_local.unsqueeze(0)
        idx, cnt = idx.reshape(1, *idx.shape[-2:]), cnt.reshape(1, -1)
    batch, T, n_h, c = q.shape
    k = idx.shape[-1]
    n_loc = kv_local.shape[1]
    E_cap = kv_comp.shape[1]
    if out is None:
        out = torch.empty_like(q)
    nbytes = B.v4a_sparse_mqa_prefill_workspace(batch, t0, T, loc_base, n_loc, n_h, c, k, w,
                                                _NP_DT[dt])
    ws = workspace(nbytes, q.device)
    B.v4a_sparse_mqa_prefill(q, kv_comp, kv_local, loc_base, n_loc, idx, cnt, sink, q_gamma,
                             kv_gamma, eps, rope_dims, rope_base, scale, batch, t0, T, n_h, c, k,
                             w, E_cap, out, _NP_DT[dt], ws, nbytes, stream)
    return out


def sparse_mqa_decode(q, kv_comp, kv_ring, kv_new, idx, cnt, *, t, w, dt, sink=None,
                      q_gamma=None, kv_gamma=None, eps=1e-6, rope_dims=0, rope_base=10000.0,
                      scale=0.0, num_splits=0, out=None, stream=None, ws=None):
    batch, n_h, c = q.shape
    k = idx.shape[-1]
    E_cap = kv_comp.shape[1]
    if out is None:
        out = torch.empty_like(q)
    nbytes = B.v4a_sparse_mqa_decode_workspace(batch, n_h, c, k, w, num_splits, _NP_DT[dt])
    if ws is None or ws.numel() < nbytes:
        ws = workspace(nbytes, q.device)
    B.v4a_sparse_mqa_decode(q, kv_comp, kv_ring, kv_new, t, idx.reshape(batch, k),
                            cnt.reshape(batch), sink, q_gamma, kv_gamma, eps, rope_dims,
                            rope_base, scale, batch, n_h, c, k, w, E_cap, num_splits, out,
                            _NP_DT[dt], ws, nbytes, stream)
    return out


def csa_decode_step(*, t, m, k, w, tail_base, C, Z, B_, CI, ZI, BI, kv_comp, KI, KI_scale, qI,
                    qI_scale, wI, q, kv_ring, kv_new, index_dt, gamma=None, gammaI=None, sink=None,
                    q_gamma=None, kv_gamma=None, rope_dims=0, rope_dims_I=0, rope_base=10000.0,
                    eps=1e-6, scale=0.0, num_splits=0, out=None, with_scores=True, stream=None,
                    ws=None, noalloc=False, t_seq=None, page_table=None, page_entries=0,
                    pool_rows=0, kv576=False, kv_scale=None):
    """One CSA decode step (tail compression of both instances, index top-k, ring insert and
    attention) through v4a_csa_decode_step.  C, Z: [batch][n_buf][2c] bf16; CI, ZI likewise
    with cI; qI [batch][n_hI][cI or cI/2]; q [batch][n_h][c].  Caches are updated in place.
    noalloc=True calls v4a_csa_decode_step_noalloc (the library's fixed scratch, no
    workspace).  Serving state: t_seq (int64 [batch], per-sequence positions; t is then
    their maximum and the tails are [batch][2m][2c]), page_table (int32
    [batch][max_pages]) with page_entries and pool_rows (kv_comp / KI are then pools).
    Returns (out, idx, cnt, score)."""
    batch, n_h, c = q.shape
    n_hI = qI.shape[1]
    cI = CI.shape[2] // 2
    dev = q.device
    out = torch.empty_like(q) if out is None else out
    idx = torch.empty(batch, k, dtype=torch.int32, device=dev)
    cnt = torch.empty(batch, dtype=torch.int32, device=dev)
    sc = torch.empty(batch, k, dtype=torch.float32, device=dev) if with_scores else None
    paged = page_table is not None
    E_cap = page_table.shape[1] * page_entries if paged else kv_comp.shape[1]
    step = B.decode_step(
        t=t, E_cap=E_cap, n_buf=C.shape[1], tok_base=tail_base, batch=batch, n_h=n_h,
        c=c, n_hI=n_hI, cI=cI, m=m, k=k, w=w, num_splits=num_splits, rope_dims=rope_dims,
        rope_dims_I=rope_dims_I, rope_base=rope_base, eps=eps, scale=scale, tail_dt=B.BF16,
        index_dt=_NP_DT[index_dt], attn_dt=B.BF16, C=C, Z=Z, B=B_, gamma=gamma, CI=CI, ZI=ZI,
        BI=BI, gammaI=gammaI, kv_comp=kv_comp, KI=KI, KI_scale=KI_scale, qI=qI,
        qI_scale=qI_scale, wI=wI, q=q, sink=sink, q_gamma=q_gamma, kv_gamma=kv_gamma,
        kv_ring=kv_ring, kv_new=kv_new, topk_idx=idx, topk_cnt=cnt, topk_score=sc, out=out,
        t_seq=t_seq, page_table=page_table, max_pages=page_table.shape[1] if paged else 0,
        pool_rows=pool_rows, page_entries=page_entries, kv576=int(kv576), kv_scale=kv_scale)
    if noalloc:
        B.v4a_csa_decode_step_noalloc(step, stream)
        return out, idx, cnt, sc
    nbytes = B.v4a_csa_decode_step_workspace(step)
    if ws is None or ws.numel() < nbytes:
        ws = workspace(nbytes, dev)
    B.v4a_csa_decode_step(step, ws, nbytes, stream)
    return out, idx, cnt, sc


def hca_attn(q, kv_comp, kv_local, *, t0, m_prime, w, dt, loc_base=0, sink=None, q_gamma=None,
             kv_gamma=None, eps=1e-6, rope_dims=0, rope_base=10000.0, scale=0.0, out=None,
             stream=None):
    if q.dim() == 3:
        q, kv_comp, kv_local = q.unsqueeze(0), kv_comp.unsqueeze(0), kv_local.unsqueeze(0)
    batch, T, n_h, c = q.shape
    n_loc = kv_local.shape[1]
    E_cap = kv_comp.shape[1]
    if out is None:
        out = torch.empty_like(q)
    nbytes = B.v4a_hca_attn_workspace(batch, t0, T, loc_base, n_loc, n_h, c, m_prime, w,
                                      _NP_DT[dt])
    ws = workspace(nbytes, q.device)
    B.v4a_hca_attn(q, kv_comp, kv_local, loc_base, n_loc, sink, q_gamma, kv_gamma, eps,
                   rope_dims, rope_base, scale, batch, t0, T, n_h, c, m_prime, w, E_cap, out,
                   _NP_DT[dt], ws, nbytes, stream)
    return out


def csa_prefill_chunked(C, Z, B_, CI, ZI, BI, q, qI, wI, local, *, chunk, m, k, w, gamma=None,
                        gammaI=None, q_gamma=None, kv_gamma=None, sink=None, rope_dims=0,
                        rope_dims_I=0, rope_base=10000.0, eps=1e-6, bufs=None, stream=None,
                        events=None):
    """CSA prefill of one sequence of n tokens in chunks of `chunk` queries, in the order of
    "CSA And HCA: Definition, State, And Cost Model" section 3 per chunk [t0, t0 + T):
    emit the main and indexer entries completed inside the chunk (from the C/Z rows of the
    whole sequence, row r = position r), index top-k of the chunk's queries over every entry
    visible to them, then sparse attention.  The long-context chunks take the streaming
    indexer, so no score matrix reaches HBM.

    C, Z [n][2c]; CI, ZI [n][2cI]; q [n][n_h][c]; qI [n][n_hI][cI]; wI [n][n_hI];
    local [n][c]; all bf16 (wI float32).  bufs: optional dict of preallocated outputs and
    workspaces (from a previous call with the same shapes).  events: optional list that
    receives (stage, start, end) CUDA events per stage and chunk.
    Returns dict(kv [1][E][c], KI [1][E][cI], idx [1][n][k], cnt [1][n], out [1][n][n_h][c],
    bufs)."""
    n, n_h, c = q.shape
    n_hI, cI = qI.shape[1], qI.shape[2]
    E = n // m
    dev = q.device
    if bufs is None:
        bufs = dict(
            kv=torch.empty(1, E, c, dtype=torch.bfloat16, device=dev),
            KI=torch.empty(1, E, cI, dtype=torch.bfloat16, device=dev),
            idx=torch.empty(1, n, k, dtype=torch.int32, device=dev),
            cnt=torch.empty(1, n, dtype=torch.int32, device=dev),
            out=torch.empty(1, n, n_h, c, dtype=torch.bfloat16, device=dev))
        wi = max(B.v4a_indexer_topk_workspace(1, min(chunk, n - t0), t0, n_hI, cI, m, k, B.BF16)
                 for t0 in range(0, n, chunk))
        wa = max(B.v4a_sparse_mqa_prefill_workspace(1, t0, min(chunk, n - t0), 0, n, n_h, c, k, w,
                                                    B.BF16) for t0 in range(0, n, chunk))
        bufs["ws_i"], bufs["ws_i_bytes"] = workspace(wi, dev), wi
        bufs["ws_a"], bufs["ws_a_bytes"] = workspace(wa, dev), wa
    kv, KI, idx, cnt, out = (bufs[x] for x in ("kv", "KI", "idx", "cnt", "out"))
    s = stream if stream is not None else torch.cuda.current_stream()
    C3, Z3, CI3, ZI3 = C.view(1, n, 2 * c), Z.view(1, n, 2 * c), CI.view(1, n, 2 * cI), ZI.view(1, n, 2 * cI)
    loc3 = local.view(1, n, c)

    def mark(name, fn):
        if events is None:
            fn()
            return
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        fn()
        b.record(s)
        events.append((name, a, b))

    for t0 in range(0, n, chunk):
        T = min(chunk, n - t0)
        mark("compress_main", lambda: B.v4a_compress(
            C3, Z3, B.BF16, B_, 1, n, 0, t0, T, c, m, 1, gamma, eps, rope_dims, rope_base, kv,
            None, B.BF16, E, s))
        mark("compress_index", lambda: B.v4a_compress(
            CI3, ZI3, B.BF16, BI, 1, n, 0, t0, T, cI, m, 1, gammaI, eps, rope_dims_I, rope_base,
            KI, None, B.BF16, E, s))
        mark("indexer_topk", lambda: B.v4a_indexer_topk(
            qI[t0:t0 + T].unsqueeze(0), None, KI, None, B.BF16, wI[t0:t0 + T].unsqueeze(0), 1, T,
            t0, n_hI, cI, m, k, E, idx[:, t0:t0 + T], cnt[:, t0:t0 + T], None, bufs["ws_i"],
            bufs["ws_i_bytes"], s))
        mark("sparse_mqa", lambda: B.v4a_sparse_mqa_prefill(
            q[t0:t0 + T].unsqueeze(0), kv, loc3, 0, n, idx[:, t0:t0 + T], cnt[:, t0:t0 + T], sink,
            q_gamma, kv_gamma, eps, rope_dims, rope_base, 0.0, 1, t0, T, n_h, c, k, w, E,
            out[:, t0:t0 + T], B.BF16, bufs["ws_a"], bufs["ws_a_bytes"], s))
    return dict(kv=kv, KI=KI, idx=idx, cnt=cnt, out=out, bufs=bufs)


def linear(X, W, *, out_dt="bf16", out=None, ws=None, stream=None):
    """Y = X W^T through v4a_linear: X [T][K] bf16, W [N][K] bf16 -> Y [T][N] (bf16 or f32)."""
    T, K = X.shape
    N = W.shape[0]
    if out is None:
        out = torch.empty(T, N, dtype=_TORCH[out_dt], device=X.device)
    nbytes = B.v4a_linear_workspace(T, K, N)
    if ws is None or ws.numel() < nbytes:
        ws = workspace(nbytes, X.device)
    B.v4a_linear(X, W, T, K, N, out, _NP_DT[out_dt], ws, nbytes, stream)
    return out


def grouped_out_proj(o, W_A, W_B, *, out=None, ws=None, stream=None):
    """o [T][n_h][c], W_A [g][d_g][c n_h/g], W_B [d][g d_g] (bf16) -> [T][d] bf16."""
    T, n_h, c = o.shape
    g, d_g = W_A.shape[0], W_A.shape[1]
    d = W_B.shape[0]
    if out is None:
        out = torch.empty(T, d, dtype=torch.bfloat16, device=o.device)
    nbytes = B.v4a_grouped_out_proj_workspace(T, n_h, c, g, d_g, d)
    if ws is None or ws.numel() < nbytes:
        ws = workspace(nbytes, o.device)
    B.v4a_grouped_out_proj(o, W_A, W_B, T, n_h, c, g, d_g, d, out, ws, nbytes, stream)
    return out


def csa_layer_prefill(H, Wt, *, m, k, w, chunk=None, rope_dims=64, gamma=None, gammaI=None,
                      stream=None, keep=False):
    """One CSA attention layer over a prefill of n tokens (H [n][d] bf16), "CSA And HCA:
    Definition, State, And Cost Model": the projections of sections 2.1, 3.1, 3.2 and
    5.1 (v4a_linear), the hot path (compressors, indexer top-k, sparse attention;
    chunked when chunk is given) and the grouped output projection of section 5.4.
    Wt: bf16 weights W_dq [d_c][d], W_uq [n_h c][d_c], W_iuq [n_hI cI][d_c], W_w [n_hI][d],
    W_loc [c][d], W_kv, W_z [2c][d], W_ikv, W_iz [2cI][d], W_oa [g][d_g][c n_h/g],
    W_ob [d][g d_g]; float32 B [2m][c], BI [2m][cI].  Returns the [n][d] output (and the
    intermediates when keep=True)."""
    n = H.shape[0]
    c = Wt["W_loc"].shape[0]
    n_h = Wt["W_uq"].shape[0] // c
    cI = Wt["W_ikv"].shape[0] // 2
    n_hI = Wt["W_w"].shape[0]
    ws = workspace(B.v4a_linear_workspace(n, 8, 8), H.device)
    lin = lambda X, W_, dt="bf16": linear(X, W_, out_dt=dt, ws=ws, stream=stream)
    cq = lin(H, Wt["W_dq"])
    q = lin(cq, Wt["W_uq"]).view(n, n_h, c)
    qI = lin(cq, Wt["W_iuq"]).view(n, n_hI, cI)
    wI = lin(H, Wt["W_w"], "f32")
    local = lin(H, Wt["W_loc"])
    C, Z = lin(H, Wt["W_kv"]), lin(H, Wt["W_z"])
    CI, ZI = lin(H, Wt["W_ikv"]), lin(H, Wt["W_iz"])
    r = csa_prefill_chunked(C, Z, Wt["B"], CI, ZI, Wt["BI"], q, qI, wI, local,
                            chunk=chunk or n, m=m, k=k, w=w, gamma=gamma, gammaI=gammaI,
                            q_gamma=gamma, kv_gamma=gamma, rope_dims=rope_dims, stream=stream)
    out = grouped_out_proj(r["out"][0], Wt["W_oa"], Wt["W_ob"], stream=stream)
    if keep:
        return out, dict(cq=cq, q=q, qI=qI, wI=wI, local=local, C=C, Z=Z, CI=CI, ZI=ZI, **r)
    return out


def hca_decode_step(*, t, m_prime, w, tail_base, C, Z, B_, kv_comp, q, kv_ring, kv_new=None,
                    gamma=None, sink=None, q_gamma=None, kv_gamma=None, rope_dims=0,
                    rope_base=10000.0, eps=1e-6, scale=0.0, num_splits=0, out=None, stream=None,
                    t_seq=None, page_table=None, page_entries=0, pool_rows=0):
    """One HCA decode step (ring insert, tail emission every m' tokens, dense attention over
    every completed entry and the window) through v4a_hca_decode_step.  C, Z: [batch][n_buf][c]
    bf16 tails; kv_comp [batch][E_cap][c] (or the pool); q [batch][n_h][c].  Returns out."""
    batch, n_h, c = q.shape
    out = torch.empty_like(q) if out is None else out
    paged = page_table is not None
    E_cap = page_table.shape[1] * page_entries if paged else kv_comp.shape[1]
    step = B.hca_step(
        t=t, E_cap=E_cap, n_buf=C.shape[1], tok_base=tail_base, batch=batch, n_h=n_h, c=c,
        m_prime=m_prime, w=w, num_splits=num_splits, rope_dims=rope_dims, rope_base=rope_base,
        eps=eps, scale=scale, tail_dt=B.BF16, attn_dt=B.BF16, C=C, Z=Z, B=B_, gamma=gamma,
        kv_comp=kv_comp, q=q, sink=sink, q_gamma=q_gamma, kv_gamma=kv_gamma, kv_ring=kv_ring,
        kv_new=kv_new, out=out, t_seq=t_seq, page_table=page_table,
        max_pages=page_table.shape[1] if paged else 0, pool_rows=pool_rows,
        page_entries=page_entries)
    nbytes = B.v4a_hca_decode_step_workspace(step)
    ws = workspace(nbytes, q.device)
    B.v4a_hca_decode_step(step, ws, nbytes, stream)
    return out
