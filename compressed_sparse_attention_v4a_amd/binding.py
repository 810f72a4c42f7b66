"""Thin ctypes binding of libv4a.so (declarations in include/v4a.h).

Each function has the C name and argument order; device buffers are passed as
torch tensors (or None for NULL) and the stream defaults to torch's current
stream.  This module only marshals arguments: every step runs in the HIP
library, and a missing library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes as ct
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# V4A_LIB names another build of the same library (the host-sanitizer checking build)
LIB_PATH = os.environ.get("V4A_LIB") or os.path.join(_HERE, "libv4a.so")

F32, BF16, FP8_E4M3, MXFP4, KV576 = 0, 1, 2, 3, 4
DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "mxfp4": MXFP4, "kv576": KV576}

_lib = None


class V4AError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


def lib() -> ct.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libv4a.so is not built ({LIB_PATH}); run "
                               "python -m compressed_sparse_attention_v4a_amd.build")
        L = ct.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ct.c_void_p, ct.c_int, ct.c_int64, ct.c_float, ct.c_size_t
        L.v4a_last_error.restype = ct.c_char_p
        L.v4a_version.restype = ct.c_char_p
        L.v4a_set_kernel_policy.argtypes = [i32]
        L.v4a_visibility.argtypes = [i64, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.v4a_compress.argtypes = [vp, vp, i32, vp, i32, i64, i64, i64, i32, i32, i32, i32, vp, f32,
                                   i32, f32, vp, vp, i32, i64, vp]
        L.v4a_indexer_topk_workspace.restype = sz
        L.v4a_indexer_topk_workspace.argtypes = [i32, i32, i64, i32, i32, i32, i32, i32]
        L.v4a_indexer_topk.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, i64, i32, i32, i32, i32,
                                       i64, vp, vp, vp, vp, sz, vp]
        L.v4a_sparse_mqa_prefill_workspace.restype = sz
        L.v4a_sparse_mqa_prefill_workspace.argtypes = [i32, i64, i32, i64, i64, i32, i32, i32, i32,
                                                       i32]
        L.v4a_sparse_mqa_prefill.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, f32, i32,
                                             f32, f32, i32, i64, i32, i32, i32, i32, i32, i64, vp,
                                             i32, vp, sz, vp]
        L.v4a_sparse_mqa_decode_workspace.restype = sz
        L.v4a_sparse_mqa_decode_workspace.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.v4a_sparse_mqa_decode.argtypes = [vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, f32, i32, f32,
                                            f32, i32, i32, i32, i32, i32, i64, i32, vp, i32, vp,
                                            sz, vp]
        L.v4a_hca_attn_workspace.restype = sz
        L.v4a_hca_attn_workspace.argtypes = [i32, i64, i32, i64, i64, i32, i32, i32, i32, i32]
        L.v4a_hca_attn.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp, f32, i32, f32, f32, i32, i64,
                                   i32, i32, i32, i32, i32, i64, vp, i32, vp, sz, vp]
        L.v4a_decode_step_layout.restype = i32
        L.v4a_decode_step_layout.argtypes = [vp, i32, vp]
        L.v4a_csa_decode_step_workspace.restype = sz
        L.v4a_csa_decode_step_workspace.argtypes = [vp]
        L.v4a_csa_decode_step.argtypes = [vp, vp, sz, vp]
        L.v4a_csa_decode_step_noalloc.argtypes = [vp, vp]
        L.v4a_hca_decode_step_layout.restype = i32
        L.v4a_hca_decode_step_layout.argtypes = [vp, i32, vp]
        L.v4a_hca_decode_step_workspace.restype = sz
        L.v4a_hca_decode_step_workspace.argtypes = [vp]
        L.v4a_hca_decode_step.argtypes = [vp, vp, sz, vp]
        L.v4a_linear_workspace.restype = sz
        L.v4a_linear_workspace.argtypes = [i32, i32, i32]
        L.v4a_linear.argtypes = [vp, vp, i32, i32, i32, vp, i32, vp, sz, vp]
        L.v4a_grouped_out_proj_workspace.restype = sz
        L.v4a_grouped_out_proj_workspace.argtypes = [i32, i32, i32, i32, i32, i32]
        L.v4a_grouped_out_proj.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, sz, vp]
        _check_step_layout(L)
        _lib = L
    return _lib


class DecodeStep(ct.Structure):
    """Mirror of v4a_decode_step (field order and types as declared in include/v4a.h;
    checked against the library's own offsets when the library loads)."""
    _fields_ = (
        [(n, ct.c_int64) for n in ("t", "E_cap", "n_buf", "tok_base")]
        + [(n, ct.c_int) for n in ("batch", "n_h", "c", "n_hI", "cI", "m", "k", "w", "num_splits",
                                   "rope_dims", "rope_dims_I")]
        + [(n, ct.c_float) for n in ("rope_base", "eps", "scale")]
        + [(n, ct.c_int) for n in ("tail_dt", "index_dt", "attn_dt")]
        + [(n, ct.c_void_p) for n in ("C", "Z", "B", "gamma", "CI", "ZI", "BI", "gammaI", "kv_comp",
                                      "KI", "KI_scale", "qI", "qI_scale", "wI", "q", "sink",
                                      "q_gamma", "kv_gamma", "kv_ring", "kv_new", "topk_idx",
                                      "topk_cnt", "topk_score", "out")]
        + [("t_seq", ct.c_void_p), ("page_table", ct.c_void_p), ("max_pages", ct.c_int64),
           ("pool_rows", ct.c_int64), ("page_entries", ct.c_int), ("kv576", ct.c_int),
           ("kv_scale", ct.c_void_p)])


class HcaStep(ct.Structure):
    """Mirror of v4a_hca_step (checked against the library's offsets when it loads)."""
    _fields_ = (
        [(n, ct.c_int64) for n in ("t", "E_cap", "n_buf", "tok_base")]
        + [(n, ct.c_int) for n in ("batch", "n_h", "c", "m_prime", "w", "num_splits", "rope_dims")]
        + [(n, ct.c_float) for n in ("rope_base", "eps", "scale")]
        + [(n, ct.c_int) for n in ("tail_dt", "attn_dt")]
        + [(n, ct.c_void_p) for n in ("C", "Z", "B", "gamma", "kv_comp", "q", "sink", "q_gamma",
                                      "kv_gamma", "kv_ring", "kv_new", "out", "t_seq",
                                      "page_table")]
        + [("max_pages", ct.c_int64), ("pool_rows", ct.c_int64), ("page_entries", ct.c_int)])


def _check_layout(fn, cls, name):
    n = len(cls._fields_)
    off = (ct.c_size_t * n)()
    size = ct.c_size_t()
    nf = fn(ct.cast(off, ct.c_void_p), n, ct.cast(ct.byref(size), ct.c_void_p))
    mine = [getattr(cls, f).offset for f, _ in cls._fields_]
    if nf != n or list(off) != mine or size.value != ct.sizeof(cls):
        raise RuntimeError(f"{name} layout of the library does not match the binding")


def _check_step_layout(L):
    _check_layout(L.v4a_decode_step_layout, DecodeStep, "v4a_decode_step")
    _check_layout(L.v4a_hca_decode_step_layout, HcaStep, "v4a_hca_step")


def _fill(cls, fields, what):
    d = cls()
    names = {f for f, _ in cls._fields_}
    ptrs = {f for f, t in cls._fields_ if t is ct.c_void_p}
    for key, val in fields.items():
        if key not in names:
            raise TypeError(f"unknown {what} field {key!r}")
        setattr(d, key, (None if val is None else val.data_ptr()) if key in ptrs else val)
    return d


def decode_step(**fields) -> DecodeStep:
    """A DecodeStep from keyword arguments: tensors (or None) for the pointer fields,
    numbers for the rest (unset fields are 0 / NULL)."""
    return _fill(DecodeStep, fields, "decode-step")


def hca_step(**fields) -> HcaStep:
    """An HcaStep from keyword arguments (as decode_step)."""
    return _fill(HcaStep, fields, "HCA-step")


def v4a_hca_decode_step_workspace(step: HcaStep) -> int:
    return lib().v4a_hca_decode_step_workspace(ct.c_void_p(ct.addressof(step)))


def v4a_hca_decode_step(step: HcaStep, ws, ws_bytes, stream=None):
    _check("v4a_hca_decode_step", lib().v4a_hca_decode_step(
        ct.c_void_p(ct.addressof(step)), _p(ws), ws_bytes, _s(stream)))


def v4a_csa_decode_step_workspace(step: DecodeStep) -> int:
    return lib().v4a_csa_decode_step_workspace(ct.c_void_p(ct.addressof(step)))


def v4a_csa_decode_step(step: DecodeStep, ws, ws_bytes, stream=None):
    _check("v4a_csa_decode_step", lib().v4a_csa_decode_step(
        ct.c_void_p(ct.addressof(step)), _p(ws), ws_bytes, _s(stream)))


def v4a_csa_decode_step_noalloc(step: DecodeStep, stream=None):
    _check("v4a_csa_decode_step_noalloc", lib().v4a_csa_decode_step_noalloc(
        ct.c_void_p(ct.addressof(step)), _s(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20  # V4A_NOALLOC_SCRATCH_BYTES


def _p(t):
    if t is None:
        return None
    return ct.c_void_p(t.data_ptr())


def _s(stream):
    if stream is None:
        import torch
        return ct.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ct.c_void_p(stream)
    return ct.c_void_p(stream.cuda_stream)


def _check(fn: str, rc: int):
    if rc != 0:
        raise V4AError(fn, rc, lib().v4a_last_error().decode())


def v4a_last_error() -> str:
    return lib().v4a_last_error().decode()


def v4a_version() -> str:
    return lib().v4a_version().decode()


def v4a_set_kernel_policy(policy: int) -> int:
    return lib().v4a_set_kernel_policy(policy)


def v4a_visibility(t0, T, m, k, w, E=None, cnt=None, win_lo=None, win_len=None, stream=None):
    _check("v4a_visibility", lib().v4a_visibility(t0, T, m, k, w, _p(E), _p(cnt), _p(win_lo),
                                                   _p(win_len), _s(stream)))


def v4a_compress(C, Z, in_dt, B, batch, n_buf, tok_base, t0, T, c, m, overlap, gamma, eps,
                 rope_dims, rope_base, out, out_scale, out_dt, E_cap, stream=None):
    _check("v4a_compress", lib().v4a_compress(
        _p(C), _p(Z), in_dt, _p(B), batch, n_buf, tok_base, t0, T, c, m, overlap, _p(gamma), eps,
        rope_dims, rope_base, _p(out), _p(out_scale), out_dt, E_cap, _s(stream)))


def v4a_indexer_topk_workspace(batch, T, t0, n_hI, cI, m, k, dt) -> int:
    return lib().v4a_indexer_topk_workspace(batch, T, t0, n_hI, cI, m, k, dt)


def v4a_indexer_topk(qI, qI_scale, KI, KI_scale, dt, wI, batch, T, t0, n_hI, cI, m, k, E_cap,
                     topk_idx, topk_cnt, topk_score, ws, ws_bytes, stream=None):
    _check("v4a_indexer_topk", lib().v4a_indexer_topk(
        _p(qI), _p(qI_scale), _p(KI), _p(KI_scale), dt, _p(wI), batch, T, t0, n_hI, cI, m, k,
        E_cap, _p(topk_idx), _p(topk_cnt), _p(topk_score), _p(ws), ws_bytes, _s(stream)))


def v4a_sparse_mqa_prefill_workspace(batch, t0, T, loc_base, n_loc, n_h, c, k, w, dt) -> int:
    return lib().v4a_sparse_mqa_prefill_workspace(batch, t0, T, loc_base, n_loc, n_h, c, k, w, dt)


def v4a_sparse_mqa_prefill(q, kv_comp, kv_local, loc_base, n_loc, topk_idx, topk_cnt, sink,
                           q_gamma, kv_gamma, eps, rope_dims, rope_base, scale, batch, t0, T, n_h,
                           c, k, w, E_cap, out, dt, ws, ws_bytes, stream=None):
    _check("v4a_sparse_mqa_prefill", lib().v4a_sparse_mqa_prefill(
        _p(q), _p(kv_comp), _p(kv_local), loc_base, n_loc, _p(topk_idx), _p(topk_cnt), _p(sink),
        _p(q_gamma), _p(kv_gamma), eps, rope_dims, rope_base, scale, batch, t0, T, n_h, c, k, w,
        E_cap, _p(out), dt, _p(ws), ws_bytes, _s(stream)))


def v4a_sparse_mqa_decode_workspace(batch, n_h, c, k, w, num_splits, dt) -> int:
    return lib().v4a_sparse_mqa_decode_workspace(batch, n_h, c, k, w, num_splits, dt)


def v4a_sparse_mqa_decode(q, kv_comp, kv_ring, kv_new, t, topk_idx, topk_cnt, sink, q_gamma,
                          kv_gamma, eps, rope_dims, rope_base, scale, batch, n_h, c, k, w, E_cap,
                          num_splits, out, dt, ws, ws_bytes, stream=None):
    _check("v4a_sparse_mqa_decode", lib().v4a_sparse_mqa_decode(
        _p(q), _p(kv_comp), _p(kv_ring), _p(kv_new), t, _p(topk_idx), _p(topk_cnt), _p(sink),
        _p(q_gamma), _p(kv_gamma), eps, rope_dims, rope_base, scale, batch, n_h, c, k, w, E_cap,
        num_splits, _p(out), dt, _p(ws), ws_bytes, _s(stream)))


def v4a_hca_attn_workspace(batch, t0, T, loc_base, n_loc, n_h, c, m_prime, w, dt) -> int:
    return lib().v4a_hca_attn_workspace(batch, t0, T, loc_base, n_loc, n_h, c, m_prime, w, dt)


def v4a_hca_attn(q, kv_comp, kv_local, loc_base, n_loc, sink, q_gamma, kv_gamma, eps, rope_dims,
                 rope_base, scale, batch, t0, T, n_h, c, m_prime, w, E_cap, out, dt, ws, ws_bytes,
                 stream=None):
    _check("v4a_hca_attn", lib().v4a_hca_attn(
        _p(q), _p(kv_comp), _p(kv_local), loc_base, n_loc, _p(sink), _p(q_gamma), _p(kv_gamma),
        eps, rope_dims, rope_base, scale, batch, t0, T, n_h, c, m_prime, w, E_cap, _p(out), dt,
        _p(ws), ws_bytes, _s(stream)))


def v4a_linear_workspace(T, K, N) -> int:
    return lib().v4a_linear_workspace(T, K, N)


def v4a_linear(X, W, T, K, N, Y, out_dt, ws, ws_bytes, stream=None):
    _check("v4a_linear", lib().v4a_linear(_p(X), _p(W), T, K, N, _p(Y), out_dt, _p(ws), ws_bytes,
                                          _s(stream)))


def v4a_grouped_out_proj_workspace(T, n_h, c, g, d_g, d) -> int:
    return lib().v4a_grouped_out_proj_workspace(T, n_h, c, g, d_g, d)


def v4a_grouped_out_proj(o, W_A, W_B, T, n_h, c, g, d_g, d, out, ws, ws_bytes, stream=None):
    _check("v4a_grouped_out_proj", lib().v4a_grouped_out_proj(
        _p(o), _p(W_A), _p(W_B), T, n_h, c, g, d_g, d, _p(out), _p(ws), ws_bytes, _s(stream)))
