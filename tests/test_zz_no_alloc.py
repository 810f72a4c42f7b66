"""v4a_csa_decode_step_noalloc (fixed device scratch, no workspace argument) against
v4a_csa_decode_step with a caller workspace: bit for bit on two calls in a row, the
second with a smaller step, both through the C ABI."""
import numpy as np
import pytest
import torch

import synth
from compressed_sparse_attention_v4a_amd import ops

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _up(x):
    return None if x is None else ops.upload(x, None, DEV)


def _step(cfg, d, noalloc):
    g, gI = _up(d["gamma"]), _up(d["gammaI"])
    kv, KI, KIs, ring = _up(d["kv_comp"]), _up(d["KI"]), _up(d["KI_scale"]), _up(d["ring"])
    out, idx, cnt, sc = ops.csa_decode_step(
        t=d["t"], m=cfg["m"], k=cfg["k"], w=cfg["w"], tail_base=d["tail_base"], C=_up(d["C"]),
        Z=_up(d["Z"]), B_=_up(d["B"]), CI=_up(d["CI"]), ZI=_up(d["ZI"]), BI=_up(d["BI"]),
        kv_comp=kv, KI=KI, KI_scale=KIs, qI=_up(d["qI"]), qI_scale=_up(d["qI_scale"]),
        wI=_up(d["wI"]), q=_up(d["q"]), kv_ring=ring, kv_new=_up(d["kv_new"]),
        index_dt=cfg["idt"], gamma=g, gammaI=gI, q_gamma=g, kv_gamma=g,
        rope_dims=cfg["rope_dims"], noalloc=noalloc)
    torch.cuda.synchronize()
    return dict(kv=kv, KI=KI, KIs=KIs, ring=ring, idx=idx, cnt=cnt, sc=sc, out=out)


def _bits(x):
    return x.view(torch.uint8) if x.dtype == torch.bfloat16 else x


@pytest.mark.parametrize("name", ["csa_decode_flash_128k", "csa_decode_pro_1m"])
def test_noalloc_decode_step_matches_workspace_call(name):
    big = dict(csa_decode_flash_128k=(8, 131072), csa_decode_pro_1m=(4, 262144))[name]
    for batch, L in (big, (2, 8188)):  # the second call is smaller
        cfg = synth.configs.workload(name, batch=batch, L=L)
        cfg["id"] = 13
        d = synth.configs.gen_csa_decode(cfg)
        print(f"noalloc decode step {name} batch={batch} L={L}", flush=True)
        ref = _step(cfg, d, noalloc=False)
        got = _step(cfg, d, noalloc=True)
        for key in ("kv", "KI", "KIs", "ring", "idx", "cnt", "sc", "out"):
            assert torch.equal(_bits(ref[key]), _bits(got[key])), (name, batch, L, key)
