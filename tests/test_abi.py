"""The C ABI library loads, exports every symbol include/v4a.h declares, and
rejects invalid arguments on the host before any device work (no GPU needed)."""
import ctypes as ct
import os
import re
import subprocess

import pytest

from compressed_sparse_attention_v4a_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "v4a.h")

EINVAL, ENOTSUP, ENOSPC = -22, -95, -28
P = ct.c_void_p(4096)  # a non-null, aligned fake device address: validation never dereferences it


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"V4A_API\s+[\w\s\*]*?\b(v4a_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libv4a.so is not built")
    return B.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared()
    assert len(names) == 24, names
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (v4a_\w+)", out))
    assert set(names) == exported
    for n in names:
        assert hasattr(lib, n)


def test_version_and_policy(lib):
    assert "gfx950" in B.v4a_version()
    prev = B.v4a_set_kernel_policy(1)
    assert B.v4a_set_kernel_policy(prev) == 1
    assert B.v4a_set_kernel_policy(7) == prev  # invalid policy: unchanged


def test_visibility_validation(lib):
    assert lib.v4a_visibility(-1, 4, 4, 2, 3, None, None, None, None, None) == EINVAL
    assert lib.v4a_visibility(0, 4, 0, 2, 3, None, None, None, None, None) == EINVAL
    assert lib.v4a_visibility(0, 4, 4, 2, 0, None, None, None, None, None) == EINVAL
    assert "m and w" in B.v4a_last_error()


def _compress(lib, **kw):
    a = dict(C=P, Z=P, in_dt=1, B=P, batch=1, n_buf=16, tok_base=0, t0=0, T=16, c=64, m=4,
             overlap=1, gamma=None, eps=1e-6, rope_dims=0, rope_base=10000.0, out=P,
             out_scale=None, out_dt=1, E_cap=4, stream=None)
    a.update(kw)
    return lib.v4a_compress(*a.values())


def test_compress_validation(lib):
    assert _compress(lib, C=None) == EINVAL
    assert _compress(lib, overlap=2) == EINVAL
    assert _compress(lib, m=0) == EINVAL
    assert _compress(lib, c=63) == EINVAL
    assert _compress(lib, rope_dims=3) == EINVAL
    assert _compress(lib, rope_dims=66) == EINVAL
    assert _compress(lib, E_cap=3) == EINVAL                    # entries 0..3 need E_cap 4
    assert _compress(lib, n_buf=15) == EINVAL                   # last block not in the buffer
    assert _compress(lib, tok_base=5, n_buf=11, t0=8, T=8) == EINVAL  # entry 2 pools block 1 (pos 4..7)
    assert _compress(lib, in_dt=2) == ENOTSUP                   # fp8 input
    assert _compress(lib, out_dt=9) == ENOTSUP
    assert _compress(lib, out_dt=2) == EINVAL                   # fp8 output needs out_scale
    assert _compress(lib, c=48, out_dt=3, out_scale=P) == EINVAL  # MXFP4 needs c % 32
    assert _compress(lib, C=ct.c_void_p(4098)) == EINVAL        # misaligned
    assert _compress(lib, c=4096) == ENOTSUP
    assert "E_cap" in B.v4a_last_error() or B.v4a_last_error() != ""


def _indexer(lib, **kw):
    a = dict(qI=P, qI_scale=None, KI=P, KI_scale=None, dt=1, wI=P, batch=1, T=8, t0=0, n_hI=4,
             cI=32, m=4, k=2, E_cap=2, idx=P, cnt=P, score=None, ws=P, ws_bytes=1 << 30,
             stream=None)
    a.update(kw)
    return lib.v4a_indexer_topk(*a.values())


def test_indexer_validation(lib):
    assert _indexer(lib, qI=None) == EINVAL
    assert _indexer(lib, T=0) == EINVAL
    assert _indexer(lib, k=0) == EINVAL
    assert _indexer(lib, E_cap=1) == EINVAL
    assert _indexer(lib, dt=2) == EINVAL          # FP8 needs scales
    assert _indexer(lib, dt=3, cI=48, qI_scale=P, KI_scale=P) == EINVAL
    assert _indexer(lib, dt=7) == ENOTSUP
    assert _indexer(lib, ws_bytes=16) == ENOSPC
    assert _indexer(lib, ws=ct.c_void_p(4096 + 64)) == EINVAL  # workspace alignment
    # the fused bf16 prefill path keeps scores on chip; the general path needs a score buffer
    assert lib.v4a_indexer_topk_workspace(1, 8192, 0, 64, 128, 4, 512, 1) == 0
    prev = B.v4a_set_kernel_policy(1)
    try:
        assert lib.v4a_indexer_topk_workspace(1, 8192, 0, 64, 128, 4, 512, 1) >= 8192 * 2048 * 4
    finally:
        B.v4a_set_kernel_policy(prev)
    # decode scan (fp8 keys, 32768 entries): scores plus stage-A candidates
    assert lib.v4a_indexer_topk_workspace(32, 1, 131071, 64, 128, 4, 512, 2) >= 32 * 32768 * 4


def test_attention_validation(lib):
    def pre(**kw):
        a = dict(q=P, kv_comp=P, kv_local=P, loc_base=0, n_loc=16, idx=P, cnt=P, sink=None,
                 q_gamma=None, kv_gamma=None, eps=1e-6, rope_dims=0, rope_base=1e4, scale=0.0,
                 batch=1, t0=0, T=16, n_h=4, c=64, k=4, w=4, E_cap=4, out=P, dt=1, ws=P,
                 ws_bytes=1 << 30, stream=None)
        a.update(kw)
        return lib.v4a_sparse_mqa_prefill(*a.values())
    assert pre(q=None) == EINVAL
    assert pre(c=63) == EINVAL
    assert pre(c=2048) == ENOTSUP
    assert pre(dt=2) == ENOTSUP
    assert pre(rope_dims=66) == EINVAL
    assert pre(w=0) == EINVAL
    assert pre(n_loc=15) == EINVAL                      # local rows miss the last query
    assert pre(t0=20, loc_base=18, n_loc=16) == EINVAL  # window of t0=20 starts at 17
    assert pre(eps=-1.0) == EINVAL

    def dec(**kw):
        a = dict(q=P, kv_comp=P, ring=P, kv_new=None, t=100, idx=P, cnt=P, sink=None,
                 q_gamma=None, kv_gamma=None, eps=1e-6, rope_dims=0, rope_base=1e4, scale=0.0,
                 batch=2, n_h=4, c=64, k=4, w=4, E_cap=32, num_splits=0, out=P, dt=1, ws=P,
                 ws_bytes=1 << 30, stream=None)
        a.update(kw)
        return lib.v4a_sparse_mqa_decode(*a.values())
    assert dec(ring=None) == EINVAL
    assert dec(t=-1) == EINVAL
    assert dec(num_splits=65) == EINVAL
    assert dec(num_splits=4, ws_bytes=8) == ENOSPC

    def hca(**kw):
        a = dict(q=P, kv_comp=P, kv_local=P, loc_base=0, n_loc=256, sink=None, q_gamma=None,
                 kv_gamma=None, eps=1e-6, rope_dims=0, rope_base=1e4, scale=0.0, batch=1, t0=0,
                 T=256, n_h=4, c=64, m_prime=128, w=16, E_cap=2, out=P, dt=1, ws=P,
                 ws_bytes=1 << 30, stream=None)
        a.update(kw)
        return lib.v4a_hca_attn(*a.values())
    assert hca(E_cap=1) == EINVAL
    assert hca(m_prime=0) == EINVAL
    assert hca(kv_local=None) == EINVAL


def test_decode_step_layout_and_validation(lib):
    """The binding's mirror of v4a_decode_step matches the library's offsets (checked when
    the library loads), and the one-call decode step validates like the separate calls."""
    n = len(B.DecodeStep._fields_)
    off = (ct.c_size_t * n)()
    size = ct.c_size_t()
    assert lib.v4a_decode_step_layout(ct.cast(off, ct.c_void_p), n,
                                      ct.cast(ct.byref(size), ct.c_void_p)) == n
    assert list(off) == [getattr(B.DecodeStep, f).offset for f, _ in B.DecodeStep._fields_]
    assert size.value == ct.sizeof(B.DecodeStep)

    class Fake:  # a non-null, aligned fake device address with the tensor interface
        def __init__(self, addr=4096):
            self.addr = addr

        def data_ptr(self):
            return self.addr

    F = Fake()

    def step(**kw):
        a = dict(t=131071, E_cap=32768, n_buf=8, tok_base=131064, batch=2, n_h=64, c=512,
                 n_hI=64, cI=128, m=4, k=512, w=128, num_splits=0, rope_dims=64, rope_dims_I=0,
                 rope_base=1e4, eps=1e-6, scale=0.0, tail_dt=B.BF16, index_dt=B.FP8_E4M3,
                 attn_dt=B.BF16, C=F, Z=F, B=F, gamma=F, CI=F, ZI=F, BI=F, gammaI=None,
                 kv_comp=F, KI=F, KI_scale=F, qI=F, qI_scale=F, wI=F, q=F, sink=None, q_gamma=F,
                 kv_gamma=F, kv_ring=F, kv_new=F, topk_idx=F, topk_cnt=F, topk_score=None, out=F)
        a.update(kw)
        return B.decode_step(**a)

    def run(d, ws_bytes=1 << 34, ws=F):
        return lib.v4a_csa_decode_step(ct.c_void_p(ct.addressof(d)), ct.c_void_p(ws.data_ptr()),
                                       ws_bytes, None)

    need = B.v4a_csa_decode_step_workspace(step())
    # indexer workspace (scores of 2 x 32768 entries) plus the attention workspace
    assert need >= 2 * 32768 * 4 + 2 * 128 * 512 * 2
    assert run(step(q=None)) == EINVAL                  # attention inputs
    assert run(step(kv_ring=None)) == EINVAL
    assert run(step(CI=None)) == EINVAL                 # index compressor inputs
    assert run(step(KI_scale=None)) == EINVAL           # FP8 keys need their scales
    assert run(step(tok_base=131065)) == EINVAL         # tail buffer misses position 131064
    assert run(step(E_cap=32767)) == EINVAL             # entry 32767 does not fit
    assert run(step(attn_dt=B.FP8_E4M3)) == ENOTSUP
    assert run(step(num_splits=65)) == EINVAL
    assert run(step(t=-1)) == EINVAL
    assert run(step(), ws_bytes=need - 1) == ENOSPC
    assert run(step(), ws=Fake(4096 + 64)) == EINVAL    # workspace alignment
    assert lib.v4a_csa_decode_step(None, ct.c_void_p(4096), 1 << 30, None) == EINVAL


def test_decode_step_noalloc_validation(lib):
    """The no-allocation decode step rejects a step whose scratch need exceeds its fixed
    64 MiB array (batch 128 at 128K context needs ~97 MiB) before any device call."""
    class Fake:
        def data_ptr(self):
            return 4096

    F = Fake()
    big = B.decode_step(t=131071, E_cap=32768, n_buf=8, tok_base=131064, batch=128, n_h=64,
                        c=512, n_hI=64, cI=128, m=4, k=512, w=128, rope_dims=64, rope_base=1e4,
                        eps=1e-6, tail_dt=B.BF16, index_dt=B.FP8_E4M3, attn_dt=B.BF16, C=F, Z=F,
                        B=F, CI=F, ZI=F, BI=F, kv_comp=F, KI=F, KI_scale=F, qI=F, qI_scale=F, wI=F,
                        q=F, kv_ring=F, topk_idx=F, topk_cnt=F, out=F)
    assert B.v4a_csa_decode_step_workspace(big) > B.NOALLOC_SCRATCH_BYTES
    assert lib.v4a_csa_decode_step_noalloc(ct.c_void_p(ct.addressof(big)), None) == ENOSPC
    msg = B.v4a_last_error()
    assert "67108864" in msg and str(B.v4a_csa_decode_step_workspace(big)) in msg
    assert lib.v4a_csa_decode_step_noalloc(None, None) == EINVAL
    hdr = open(HEADER).read()
    assert f"#define V4A_NOALLOC_SCRATCH_BYTES (64u << 20)" in hdr


def test_projection_validation(lib):
    """v4a_linear / v4a_grouped_out_proj validate on the host before any device work."""
    assert lib.v4a_linear_workspace(0, 8, 8) == 0
    ws = B.v4a_linear_workspace(16, 64, 64)
    assert ws > 0
    run = lambda **kw: lib.v4a_linear(*[kw.get(n, d) for n, d in (
        ("X", P), ("W", P), ("T", 16), ("K", 64), ("N", 64), ("Y", P), ("dt", 1), ("ws", P),
        ("wsb", ws), ("s", None))])
    assert run(X=None) == EINVAL
    assert run(T=0) == EINVAL
    assert run(K=60) == ENOTSUP
    assert run(dt=2) == ENOTSUP
    assert run(wsb=ws - 1) == ENOSPC
    assert B.v4a_grouped_out_proj_workspace(16, 64, 512, 7, 64, 64) == 0   # n_h % g
    need = B.v4a_grouped_out_proj_workspace(16, 64, 512, 8, 64, 64)
    assert need >= 16 * 8 * 64 * 2
    gp = lambda **kw: lib.v4a_grouped_out_proj(*[kw.get(n, d) for n, d in (
        ("o", P), ("A", P), ("B", P), ("T", 16), ("n_h", 64), ("c", 512), ("g", 8), ("d_g", 64),
        ("d", 64), ("out", P), ("ws", P), ("wsb", need), ("s", None))])
    assert gp(o=None) == EINVAL
    assert gp(g=7) == EINVAL
    assert gp(d=60) == ENOTSUP
    assert gp(wsb=need - 1) == ENOSPC


def test_serving_state_validation(lib):
    """Per-sequence positions and paged caches are checked on the host: the tail layout of
    a ragged step, the page geometry, and the shapes the matrix-core kernels take."""
    class Fake:
        def __init__(self, addr=4096):
            self.addr = addr

        def data_ptr(self):
            return self.addr

    F = Fake()

    def step(**kw):
        a = dict(t=131071, E_cap=32768, n_buf=8, tok_base=131064, batch=2, n_h=64, c=512,
                 n_hI=64, cI=128, m=4, k=512, w=128, rope_dims=64, rope_base=1e4, eps=1e-6,
                 tail_dt=B.BF16, index_dt=B.FP8_E4M3, attn_dt=B.BF16, C=F, Z=F, B=F, CI=F, ZI=F,
                 BI=F, kv_comp=F, KI=F, KI_scale=F, qI=F, qI_scale=F, wI=F, q=F, kv_ring=F,
                 topk_idx=F, topk_cnt=F, out=F)
        a.update(kw)
        return B.decode_step(**a)

    def run(d):
        return lib.v4a_csa_decode_step(ct.c_void_p(ct.addressof(d)), ct.c_void_p(4096), 1 << 34, None)

    assert run(step(t_seq=F, n_buf=16)) == EINVAL                     # ragged tails are 2m rows
    pg = dict(page_table=F, max_pages=1024, page_entries=32, pool_rows=65536)
    assert run(step(**dict(pg, page_entries=24))) == EINVAL           # not a power of two
    assert run(step(**dict(pg, max_pages=512))) == EINVAL             # E_cap != pages * entries
    assert run(step(**dict(pg, pool_rows=100))) == EINVAL             # not whole pages
    assert run(step(t_seq=F, c=256, n_buf=8)) == ENOTSUP              # general-kernel shape
    need = B.v4a_csa_decode_step_workspace(step(**pg))
    assert need >= B.v4a_csa_decode_step_workspace(step()) + 2 * 512 * 4  # pool rows of the selection

    def hstep(**kw):
        a = dict(t=65535, E_cap=512, n_buf=128, tok_base=65408, batch=2, n_h=64, c=512,
                 m_prime=128, w=128, rope_dims=64, rope_base=1e4, eps=1e-6, tail_dt=B.BF16,
                 attn_dt=B.BF16, C=F, Z=F, B=F, kv_comp=F, q=F, kv_ring=F, out=F)
        a.update(kw)
        return B.hca_step(**a)

    def hrun(d):
        return lib.v4a_hca_decode_step(ct.c_void_p(ct.addressof(d)), ct.c_void_p(4096), 1 << 34, None)

    assert B.v4a_hca_decode_step_workspace(hstep()) > 0
    assert hrun(hstep(m_prime=0)) == EINVAL
    assert hrun(hstep(E_cap=511)) == EINVAL
    assert hrun(hstep(c=256)) == ENOTSUP
    assert hrun(hstep(t_seq=F, n_buf=64)) == EINVAL
    assert hrun(hstep(tok_base=65409)) == EINVAL                      # tail misses 65408
