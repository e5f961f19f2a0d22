"""Shapes of the five synthetic workloads of the CSA/HCA attention core.

Each preset names its sizes only; the arithmetic lives in the HIP library and,
separately, in the oracle.  Sizes follow the DeepSeek-V4 summaries: m = 4 for
CSA and m' = 128 for HCA, top-k 512 (Flash) / 1024 (Pro), a 128-token window,
partial RoPE on the last 64 dims (DeepSeek-V4 abstract page, section 3.3; full
technical-report digest, "hybrid attention: CSA + HCA").
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

# tensor ids (seed namespaces) shared by every consumer of a workload
T_CA, T_ZA, T_CB, T_ZB = 1, 2, 3, 4          # KV compressor candidates / logits
T_ICA, T_IZA, T_ICB, T_IZB = 5, 6, 7, 8      # indexer-key compressor candidates / logits
T_QI, T_WI, T_KI = 9, 10, 11                 # indexer query, head weights, key cache
T_Q, T_SINK = 12, 13                         # attention query, sink logits
T_KVRAW, T_WINRAW = 14, 15                   # pre-norm entry rows / per-token window rows
T_SCORES = 16                                # score rows for stand-alone top-k cases
T_GAMMA = 17                                 # RMSNorm weight of the KV rows (when not 1)


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    kind: str            # "csa" (top-k sparse) or "hca" (dense)
    dtype: str           # storage of q, entries, window rows, outputs: "f32" | "bf16"
    k_dtype: str         # indexer key storage: "f32" | "bf16" | "e4m3" | "mxfp4"
    B: int
    ctx: int             # tokens present before the first query (decode) / total (prefill)
    Tq: int              # queries per sequence
    q_pos0: int          # absolute position of the first query
    m: int               # compression rate
    N_cap: int           # entry-cache capacity
    d: int               # entry / head width c = d
    rope_dim: int
    n_h: int
    H_I: int = 0
    d_I: int = 0
    k: int = 0
    n_win: int = 128
    W_cap: int = 128
    sink: str = "normal"  # "normal" (N(0,1) per head) | "zero"
    rope_base: float = 10000.0
    eps: float = 1e-6
    kv_store: str = ""   # storage of the entries and window rows if not dtype: "mixed"
    kv_gamma: str = "ones"   # RMSNorm weight of the KV rows: "ones" | "normal" (1 + N(0, 1/16))
    notes: str = field(default="", compare=False)

    @property
    def kv_dtype(self) -> str:
        """Storage of the compressed entries and window rows: dtype, or "mixed"
        (e4m3 codes with a row scale for the first d - rope_dim dims, bf16 for
        the rotated ones)."""
        return self.kv_store or self.dtype

    @property
    def overlap(self) -> int:
        return 1 if self.kind == "csa" else 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def q_positions(self):
        return [self.q_pos0 + t for t in range(self.Tq)]

    def n_vis(self, i: int) -> int:
        return min(self.N_cap, (i + 1) // self.m)

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload(
    name="tiny_csa_fp32_T256", wid=1, kind="csa", dtype="f32", k_dtype="f32",
    B=1, ctx=256, Tq=256, q_pos0=0, m=4, N_cap=64, d=64, rope_dim=16, n_h=4,
    H_I=2, d_I=32, k=16, n_win=16, W_cap=256, sink="zero",
    notes="causal prefill of all 256 tokens; entries and indexer keys built by the compressor")

CSA_DECODE_FLASH = Workload(
    name="csa_decode_flash_b8_ctx65536", wid=2, kind="csa", dtype="bf16", k_dtype="bf16",
    B=8, ctx=65536, Tq=1, q_pos0=65536, m=4, N_cap=16384, d=512, rope_dim=64, n_h=64,
    H_I=64, d_I=128, k=512, n_win=128, W_cap=128)

HCA_DECODE = Workload(
    name="hca_decode_b4_ctx1M", wid=3, kind="hca", dtype="bf16", k_dtype="bf16",
    B=4, ctx=1048576, Tq=1, q_pos0=1048576, m=128, N_cap=8192, d=512, rope_dim=64, n_h=64,
    n_win=128, W_cap=128, notes="the step recompresses the just-completed block (entry 8191)")

CSA_PREFILL_PRO = Workload(
    name="csa_prefill_pro_chunk16384_ctx131072", wid=4, kind="csa", dtype="bf16", k_dtype="bf16",
    B=1, ctx=131072, Tq=16384, q_pos0=131072 - 16384, m=4, N_cap=32768, d=512, rope_dim=64,
    n_h=128, H_I=64, d_I=128, k=1024, n_win=128, W_cap=131072)

CSA_DECODE_1M = Workload(
    name="csa_decode_pro_b16_ctx1M_fp8keys", wid=5, kind="csa", dtype="bf16", k_dtype="e4m3",
    B=16, ctx=1048576, Tq=1, q_pos0=1048576, m=4, N_cap=262144, d=512, rope_dim=64, n_h=128,
    H_I=64, d_I=128, k=1024, n_win=128, W_cap=128)

# the same workload with the indexer keys in MXFP4 (the FP4 query-key path); same
# seeds as the fp8-key workload, so the two selections can be compared
CSA_DECODE_1M_MX4 = CSA_DECODE_1M.scaled(name="csa_decode_pro_b16_ctx1M_mxfp4keys", k_dtype="mxfp4",
                                         notes="fp32 N(0,1) keys stored as OCP MXFP4")

# Mixed KV rows take a non-unit RMSNorm weight, as a trained model has: with a
# unit weight and bf16 rows, 448 x / amax is often exactly an e4m3 rounding
# midpoint, where the order of fp32 operations alone decides the code.
HCA_DECODE_MIXED = HCA_DECODE.scaled(name="hca_decode_b4_ctx1M_mixedkv", kv_store="mixed", kv_gamma="normal",
                                     notes="entries and window rows stored as mixed rows")
CSA_DECODE_1M_MIXED = CSA_DECODE_1M.scaled(name="csa_decode_pro_b16_ctx1M_fp8keys_mixedkv", kv_store="mixed",
                                           kv_gamma="normal",
                                           notes="entries and window rows stored as mixed rows")

WORKLOADS = {w.name: w for w in (TINY, CSA_DECODE_FLASH, HCA_DECODE, CSA_PREFILL_PRO, CSA_DECODE_1M,
                                 CSA_DECODE_1M_MX4, HCA_DECODE_MIXED, CSA_DECODE_1M_MIXED)}
