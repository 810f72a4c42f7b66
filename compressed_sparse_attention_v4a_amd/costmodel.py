"""Algorithmic byte and FLOP counts for the CSA/HCA hot path.

The analytical model is the one in "CSA And HCA: Definition, State, And Cost
Model", section 8 (persistent state M(L), per-token decode reads B, attention
and indexer FLOPs F) and 8.2 (fixed projection FLOPs).  The workload counts
below apply the same per-unit figures to whole calls: they count causal
visible pairs only and one multiply-add as two FLOPs, and exclude score
matrices, intermediates and any padding.
"""
from __future__ import annotations

MIB = 1024.0 * 1024.0


# ------------------------------------------------------------------------- #
# The page's model (section 8)
# ------------------------------------------------------------------------- #

def main_entry_bytes(c=512, rope_dims=64) -> int:
    """Production main/local entry payload: BF16 RoPE channels + FP8 for the rest."""
    return rope_dims * 2 + (c - rope_dims) * 1


def fp4_index_key_bytes(cI=128) -> int:
    """MXFP4 indexer key payload (scales excluded)."""
    return cI // 2


def csa_state_bytes(L, m=4, w=128, b_C=576, b_I=64) -> dict:
    E = L // m
    return {"entries": E, "main": E * b_C, "index": E * b_I, "local": w * b_C,
            "total": w * b_C + E * (b_C + b_I)}


def hca_state_bytes(L, m_prime=128, w=128, b_C=576) -> int:
    return w * b_C + (L // m_prime) * b_C


def csa_decode_reads(L, m=4, k=512, w=128, b_C=576, b_I=64) -> dict:
    return {"index": (L // m) * b_I, "main": (k + w) * b_C}


def main_attention_flops(N, n_h=64, c=512) -> int:
    """F_main(N) = 4 n_h c N: QK and AV multiply-adds for N candidates, all heads."""
    return 4 * n_h * c * N


def index_flops(E, n_hI=64, cI=128) -> int:
    """F_index = 2 n_h^I c^I E: the indexer dot products over E entries."""
    return 2 * n_hI * cI * E


def fixed_flops(d=4096, d_c=1024, n_h=64, c=512, n_hI=64, cI=128, g=8, d_g=1024) -> dict:
    rows = {
        "q_down": 2 * d * d_c,
        "q_up": 2 * d_c * n_h * c,
        "index_q_up": 2 * d_c * n_hI * cI,
        "index_w": 2 * d * n_hI,
        "local_kv": 2 * d * c,
        "csa_main_comp": 8 * d * c,
        "csa_index_comp": 8 * d * cI,
        "grouped_out": 2 * n_h * c * d_g + 2 * g * d_g * d,
    }
    rows["total"] = sum(rows.values())
    return rows


def amortized_write_bytes(m=4, b_C=576, b_I=64) -> float:
    return b_C + (b_C + b_I) / m


def hca_decode_flops(L, m_prime=128, w=128, n_h=64, c=512) -> int:
    return main_attention_flops(L // m_prime + w, n_h, c)


# ------------------------------------------------------------------------- #
# Whole-call counts for this library's entry points
# ------------------------------------------------------------------------- #

def _sum_floor(a, b, r):
    """sum_{u=a}^{b} floor(u / r) for 0 <= a <= b (closed form)."""
    def S(x):  # sum_{u=0}^{x} floor(u/r)
        if x < 0:
            return 0
        q, rem = divmod(x + 1, r)
        return r * q * (q - 1) // 2 + q * rem
    return S(b) - S(a - 1)


def prefill_sets(t0, T, m, k, w) -> dict:
    """Sum over queries t0..t0+T-1 of visible entries E_t, selected cnt_t, window |L_t|."""
    sumE = _sum_floor(t0 + 1, t0 + T, m)
    if k and k > 0:
        # cnt = min(k, E_t); E_t >= k once t+1 >= m*k
        t_full = m * k - 1
        lo, hi = t0, t0 + T - 1
        part_hi = min(hi, t_full - 1)
        sumC = _sum_floor(lo + 1, part_hi + 1, m) if part_hi >= lo else 0
        n_full = hi - max(lo, t_full) + 1
        sumC += k * max(n_full, 0)
    else:
        sumC = sumE
    sumL = 0
    # |L_t| = min(w, t+1)
    lo, hi = t0, t0 + T - 1
    ramp_hi = min(hi, w - 2)
    if ramp_hi >= lo:
        sumL += (lo + 1 + ramp_hi + 1) * (ramp_hi - lo + 1) // 2
    sumL += w * max(0, hi - max(lo, w - 1) + 1)
    return {"sumE": sumE, "sumC": sumC, "sumL": sumL}


def csa_prefill_counts(n, m=4, k=512, w=128, n_h=64, c=512, n_hI=64, cI=128, t0=0, elem=2) -> dict:
    s = prefill_sets(t0, n, m, k, w)
    E_out = (t0 + n) // m - t0 // m
    return {
        **s,
        "index_flops": index_flops(s["sumE"], n_hI, cI),
        "attn_flops": main_attention_flops(s["sumC"] + s["sumL"], n_h, c),
        # compressor: reads C and Z (2c wide each) once, writes one row per entry
        "compress_main_bytes": 2 * n * 2 * c * elem + E_out * c * elem,
        "compress_index_bytes": 2 * n * 2 * cI * elem + E_out * cI * elem,
        # attention: q read + out write dominate; candidates come from the L2-resident caches
        "attn_min_bytes": 2 * n * n_h * c * elem,
    }


def hca_prefill_counts(n, m_prime=128, w=128, n_h=64, c=512, t0=0, elem=2) -> dict:
    s = prefill_sets(t0, n, m_prime, 0, w)
    E_out = (t0 + n) // m_prime - t0 // m_prime
    return {
        **s,
        "attn_flops": main_attention_flops(s["sumE"] + s["sumL"], n_h, c),
        "compress_bytes": 2 * n * c * elem + E_out * c * elem,
        "attn_min_bytes": 2 * n * n_h * c * elem,
    }


def csa_decode_counts(batch, L, m=4, k=512, w=128, n_h=64, c=512, n_hI=64, cI=128,
                      idt="fp8", elem=2, main_row_bytes=None) -> dict:
    """Bytes and FLOPs one decode call must move and do (batch sequences at L - 1).
    main_row_bytes: bytes of one stored compressed entry (default c * elem; the production
    row of section 8 is 576 + a 4-byte scale); window rows are read as bf16."""
    mrb = c * elem if main_row_bytes is None else main_row_bytes
    t = L - 1
    E = (t + 1) // m
    cnt = min(k, E)
    nl = min(w, t + 1)
    if idt == "fp8":
        key_b = cI + 4            # e4m3 codes + one fp32 scale per row
        q_b = n_hI * (cI + 4)
    elif idt == "mxfp4":
        key_b = cI // 2 + cI // 32
        q_b = n_hI * (cI // 2 + cI // 32)
    else:
        key_b = cI * elem
        q_b = n_hI * cI * elem
    per_seq = {
        "index_read": E * key_b + q_b + n_hI * 4,
        "gather_read": cnt * mrb + nl * c * elem,
        "q_out": 2 * n_h * c * elem,
        "tail": 2 * m * (2 * c + 2 * cI) * elem * 2,
    }
    tot = {kk: v * batch for kk, v in per_seq.items()}
    tot["total_bytes"] = sum(tot.values())
    tot["index_flops"] = batch * index_flops(E, n_hI, cI)
    tot["attn_flops"] = batch * main_attention_flops(cnt + nl, n_h, c)
    tot["E"], tot["cnt"], tot["nl"] = E, cnt, nl
    return tot
