"""Synthetic workloads: shapes, value distributions and seeded generation.

Each workload is a dict of named arrays in their *stored* format:
  * float32 arrays for fp32 tensors,
  * uint16 bf16 bit patterns for bf16 tensors,
  * uint8 codes + float32 per-row scales for FP8 E4M3,
  * uint8 packed nibbles + uint8 E8M0 scales for MXFP4.
The GPU path uploads these bytes; the oracle decodes them with its own code.

Shapes follow the published V4-Flash / V4-Pro table in "CSA And HCA:
Definition, State, And Cost Model" (section 1, configuration table).  Value
distributions (N(0,1)/sqrt(c) for q and K=V rows, N(0,1) gate logits,
N(0,0.1) positional bias as a variance, U(0,1) indexer head weights) are the
project's synthetic recipe; no dataset is involved.

Tensor seeds: seed = base + tensor_id, base = 0x5EED0000 + workload * 256.
"""
from __future__ import annotations

import math

import numpy as np

from . import formats, rng

TID = {  # tensor ids
    "H": 1, "W_kv": 2, "W_z": 3, "W_ikv": 4, "W_iz": 5, "W_loc": 6, "W_q": 7, "W_qi": 8,
    "C": 10, "Z": 11, "B": 12, "CI": 13, "ZI": 14, "BI": 15, "local": 16, "q": 17,
    "qI": 18, "wI": 19, "kv_comp": 20, "KI": 21, "ring": 22, "kv_new": 23, "sink": 24,
}


def seed_of(workload: int, name: str) -> int:
    return 0x5EED0000 + workload * 256 + TID[name]


def store(x: np.ndarray, dt: str):
    """float64 -> stored representation for dtype dt ('f32' or 'bf16')."""
    if dt == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dt == "bf16":
        return formats.bf16_bits(np.asarray(x, dtype=np.float32))
    raise ValueError(dt)


# --------------------------------------------------------------------------- #
# Workload table
# --------------------------------------------------------------------------- #

WORKLOADS = {
    # tiny CSA layer, fp32, host projections from H
    "csa_tiny_f32": dict(id=0, kind="csa_prefill", dt="f32", n=256, d=128, c=64, n_h=8,
                         n_hI=4, cI=32, m=4, k=16, w=16, rope_dims=0, norm=False,
                         inorm=False, host_proj=True),
    # CSA prefill, V4-Flash shapes
    "csa_prefill_flash_8k": dict(id=1, kind="csa_prefill", dt="bf16", n=8192, c=512, n_h=64,
                                 n_hI=64, cI=128, m=4, k=512, w=128, rope_dims=64, norm=True,
                                 inorm=True, host_proj=False),
    # HCA prefill, V4-Flash shapes
    "hca_prefill_flash_64k": dict(id=2, kind="hca_prefill", dt="bf16", n=65536, c=512, n_h=64,
                                  m_prime=128, w=128, rope_dims=64, norm=True),
    # CSA decode, V4-Flash shapes, fp8 indexer keys
    "csa_decode_flash_128k": dict(id=3, kind="csa_decode", dt="bf16", idt="fp8", batch=32,
                                  L=131072, c=512, n_h=64, n_hI=64, cI=128, m=4, k=512, w=128,
                                  rope_dims=64, norm=True, inorm=True),
    # CSA decode, V4-Pro shapes at 1M, MXFP4 indexer
    "csa_decode_pro_1m": dict(id=4, kind="csa_decode", dt="bf16", idt="mxfp4", batch=4,
                              L=1048576, c=512, n_h=128, n_hI=64, cI=128, m=4, k=1024, w=128,
                              rope_dims=64, norm=True, inorm=True),
}


def workload(name: str, **over) -> dict:
    cfg = dict(WORKLOADS[name])
    cfg.update(over)
    cfg["name"] = name
    return cfg


# --------------------------------------------------------------------------- #
# Generators
# --------------------------------------------------------------------------- #

def _nrm(cfg, name, shape, std, r0=0, r1=None):
    return rng.normal_rows(seed_of(cfg["id"], name), shape, r0, r1, std)


def _uni(cfg, name, shape, r0=0, r1=None):
    return rng.uniform_rows(seed_of(cfg["id"], name), shape, r0, r1)


def gen_csa_prefill(cfg: dict) -> dict:
    """Inputs for a CSA prefill of n tokens (t0 = 0).

    Returns stored arrays: C, Z [n, 2c]; B [2m, c] f32; CI, ZI [n, 2cI]; BI [2m, cI] f32;
    local [n, c]; q [n, n_h, c]; qI [n, n_hI, cI]; wI [n, n_hI] f32; gamma vectors.
    """
    n, c, n_h, n_hI, cI, m = (cfg[k] for k in ("n", "c", "n_h", "n_hI", "cI", "m"))
    dt = cfg["dt"]
    out = {}
    if cfg.get("host_proj"):
        d = cfg["d"]
        H = _nrm(cfg, "H", (n, d), 1.0)
        sw = 1.0 / math.sqrt(d)
        proj = lambda nm, cols: H @ _nrm(cfg, nm, (d, cols), sw)
        C = proj("W_kv", 2 * c)
        Z = proj("W_z", 2 * c)
        CI = proj("W_ikv", 2 * cI)
        ZI = proj("W_iz", 2 * cI)
        local = proj("W_loc", c)
        q = proj("W_q", n_h * c).reshape(n, n_h, c)
        qI = proj("W_qi", n_hI * cI).reshape(n, n_hI, cI)
    else:
        sc = 1.0 / math.sqrt(c)
        C = _nrm(cfg, "C", (n, 2 * c), sc)
        Z = _nrm(cfg, "Z", (n, 2 * c), 1.0)
        CI = _nrm(cfg, "CI", (n, 2 * cI), 1.0)
        ZI = _nrm(cfg, "ZI", (n, 2 * cI), 1.0)
        local = _nrm(cfg, "local", (n, c), sc)
        q = _nrm(cfg, "q", (n, n_h, c), sc)
        qI = _nrm(cfg, "qI", (n, n_hI, cI), 1.0)
    out["C"], out["Z"] = store(C, dt), store(Z, dt)
    out["CI"], out["ZI"] = store(CI, dt), store(ZI, dt)
    out["local"], out["q"], out["qI"] = store(local, dt), store(q, dt), store(qI, dt)
    sb = math.sqrt(0.1)
    out["B"] = _nrm(cfg, "B", (2 * m, c), sb).astype(np.float32)
    out["BI"] = _nrm(cfg, "BI", (2 * m, cI), sb).astype(np.float32)
    out["wI"] = _uni(cfg, "wI", (n, n_hI)).astype(np.float32)
    out["gamma"] = np.ones(c, np.float32)
    out["gammaI"] = np.ones(cI, np.float32)
    if cfg.get("sink"):
        out["sink"] = _nrm(cfg, "sink", (n_h,), 1.0).astype(np.float32)
    return out


def gen_hca_prefill(cfg: dict, q_rows=None) -> dict:
    """Inputs for an HCA prefill of n tokens.  q_rows=(r0, r1) limits q to those rows."""
    n, c, n_h, mp = cfg["n"], cfg["c"], cfg["n_h"], cfg["m_prime"]
    dt = cfg["dt"]
    sc = 1.0 / math.sqrt(c)
    out = {
        "C": store(_nrm(cfg, "C", (n, c), sc), dt),
        "Z": store(_nrm(cfg, "Z", (n, c), 1.0), dt),
        "B": _nrm(cfg, "B", (mp, c), math.sqrt(0.1)).astype(np.float32),
        "local": store(_nrm(cfg, "local", (n, c), sc), dt),
        "gamma": np.ones(c, np.float32),
    }
    r0, r1 = q_rows if q_rows else (0, n)
    out["q"] = store(_nrm(cfg, "q", (n, n_h, c), sc, r0, r1), dt)
    if cfg.get("sink"):
        out["sink"] = _nrm(cfg, "sink", (n_h,), 1.0).astype(np.float32)
    return out


def gen_csa_decode(cfg: dict, seqs=None) -> dict:
    """Cache state and new-token inputs for one CSA decode step at t = L - 1.

    Before the step a sequence holds entries 0 .. E-2 (E = L // m) in both caches,
    the ring holds tokens t-w .. t-1 at slot j % w, and the tail buffers hold the
    raw C/Z rows of the last two blocks (positions m*(E-2) .. m*E - 1).
    seqs: optional list of sequence indices to generate (default all).
    """
    B, L, c, n_h, n_hI, cI, m, w = (cfg[k] for k in ("batch", "L", "c", "n_h", "n_hI", "cI", "m", "w"))
    E = L // m
    seqs = list(range(B)) if seqs is None else list(seqs)
    nb = len(seqs)
    sc = 1.0 / math.sqrt(c)
    idt = cfg["idt"]
    out = {"seqs": seqs}

    def per_seq(name, shape, std, uni=False):
        # sequence b uses rows [b*shape0, (b+1)*shape0) of one tall tensor
        rows = []
        for b in seqs:
            full = (B * shape[0],) + tuple(shape[1:])
            if uni:
                rows.append(_uni(cfg, name, full, b * shape[0], (b + 1) * shape[0]))
            else:
                rows.append(_nrm(cfg, name, full, std, b * shape[0], (b + 1) * shape[0]))
        return np.stack(rows)

    kv = per_seq("kv_comp", (E, c), 1.0)
    kv[:, E - 1, :] = 0.0  # emitted by this step
    out["kv_comp"] = store(kv, "bf16")
    ki = per_seq("KI", (E, cI), 1.0)
    ki[:, E - 1, :] = 0.0
    if idt == "fp8":
        out["KI"], out["KI_scale"] = formats.fp8_e4m3_rows(ki)
        qi = per_seq("qI", (n_hI, cI), 1.0)
        out["qI"], out["qI_scale"] = formats.fp8_e4m3_rows(qi)
    elif idt == "mxfp4":
        out["KI"], out["KI_scale"] = formats.mxfp4_rows(ki)
        qi = per_seq("qI", (n_hI, cI), 1.0)
        out["qI"], out["qI_scale"] = formats.mxfp4_rows(qi)
    else:
        out["KI"], out["KI_scale"] = store(ki, idt), None
        out["qI"], out["qI_scale"] = store(per_seq("qI", (n_hI, cI), 1.0), idt), None
    out["ring"] = store(per_seq("ring", (w, c), sc), "bf16")
    out["kv_new"] = store(per_seq("kv_new", (1, c), sc)[:, 0], "bf16")
    out["C"] = store(per_seq("C", (2 * m, 2 * c), sc), "bf16")
    out["Z"] = store(per_seq("Z", (2 * m, 2 * c), 1.0), "bf16")
    out["CI"] = store(per_seq("CI", (2 * m, 2 * cI), 1.0), "bf16")
    out["ZI"] = store(per_seq("ZI", (2 * m, 2 * cI), 1.0), "bf16")
    out["B"] = _nrm(cfg, "B", (2 * m, c), math.sqrt(0.1)).astype(np.float32)
    out["BI"] = _nrm(cfg, "BI", (2 * m, cI), math.sqrt(0.1)).astype(np.float32)
    out["q"] = store(per_seq("q", (n_h, c), sc), "bf16")
    out["wI"] = per_seq("wI", (n_hI,), 0, uni=True).astype(np.float32)
    out["gamma"] = np.ones(c, np.float32)
    out["gammaI"] = np.ones(cI, np.float32)
    out["t"] = L - 1
    out["tail_base"] = m * (E - 2)
    if cfg.get("sink"):
        out["sink"] = _nrm(cfg, "sink", (n_h,), 1.0).astype(np.float32)
    return out
