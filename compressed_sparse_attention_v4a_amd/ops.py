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
_NP_DT = {"f32": B.F32, "bf16": B.BF16, "fp8": B.FP8_E4M3, "mxfp4": B.MXFP4}


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
    E_cap = (t0 + T) // m if E_cap is None else E_cap
    dev = C.device
    if out is None:
        if out_dt in ("f32", "bf16"):
            out = torch.empty(batch, E_cap, c, dtype=_TORCH[out_dt], device=dev)
        elif out_dt == "fp8":
            out = torch.empty(batch, E_cap, c, dtype=torch.uint8, device=dev)
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
                    ws=None):
    """One CSA decode step (tail compression of both instances, index top-k, ring insert and
    attention) through v4a_csa_decode_step.  C, Z: [batch][n_buf][2c] bf16; CI, ZI likewise
    with cI; qI [batch][n_hI][cI or cI/2]; q [batch][n_h][c].  Caches are updated in place.
    Returns (out, idx, cnt, score)."""
    batch, n_h, c = q.shape
    n_hI = qI.shape[1]
    cI = CI.shape[2] // 2
    dev = q.device
    out = torch.empty_like(q) if out is None else out
    idx = torch.empty(batch, k, dtype=torch.int32, device=dev)
    cnt = torch.empty(batch, dtype=torch.int32, device=dev)
    sc = torch.empty(batch, k, dtype=torch.float32, device=dev) if with_scores else None
    step = B.decode_step(
        t=t, E_cap=kv_comp.shape[1], n_buf=C.shape[1], tok_base=tail_base, batch=batch, n_h=n_h,
        c=c, n_hI=n_hI, cI=cI, m=m, k=k, w=w, num_splits=num_splits, rope_dims=rope_dims,
        rope_dims_I=rope_dims_I, rope_base=rope_base, eps=eps, scale=scale, tail_dt=B.BF16,
        index_dt=_NP_DT[index_dt], attn_dt=B.BF16, C=C, Z=Z, B=B_, gamma=gamma, CI=CI, ZI=ZI,
        BI=BI, gammaI=gammaI, kv_comp=kv_comp, KI=KI, KI_scale=KI_scale, qI=qI,
        qI_scale=qI_scale, wI=wI, q=q, sink=sink, q_gamma=q_gamma, kv_gamma=kv_gamma,
        kv_ring=kv_ring, kv_new=kv_new, topk_idx=idx, topk_cnt=cnt, topk_score=sc, out=out)
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
