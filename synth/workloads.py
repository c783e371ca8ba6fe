"""The five named CSA workloads: shapes, precisions and input distributions.

Shapes follow the pages' production layer where they give it ("Anatomy of a Frontier Model",
section "The attention: compress, then select": m=4 tokens per entry, 512-dim single shared K=V
entry, indexer of 64 heads x 128 dims, top-1024 (512 in Flash), 128-token window) and the
lab-scale toy for the tiny case ("The Exchange Rates of a Million Tokens", section 3).
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "prefill" (x is projected and compressed) or "decode" (caches are given)
    B: int             # sequences
    L: int             # context tokens before the first query
    T: int             # query tokens per sequence
    m: int             # tokens per compressed entry
    d: int             # d_model (0 for decode: no projection)
    D: int             # entry dim = query head dim (K = V)
    H: int             # query heads sharing the one KV head
    H_I: int           # indexer heads
    D_I: int           # indexer head dim
    k: int             # top-k
    W: int             # sliding window of raw tokens
    dtype: str         # activation / cache storage: "f32" or "bf16"
    idx_dtype: str     # indexer q/k storage: same as dtype, or "mxfp4"
    seed: int = 0

    @property
    def n_cap(self) -> int:
        """Compressed entries that exist once the last query's block is complete."""
        return (self.L + self.T) // self.m

    @property
    def n_tot(self) -> int:
        """Columns of the fused projection [Ca Za Cb Zb | Ca' Za' Cb' Zb' | q | q_I | kv_raw]."""
        return 4 * self.D + 4 * self.D_I + self.H * self.D + self.H_I * self.D_I + self.D

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Tiny fp32 forward; the CPU oracle finishes in milliseconds.
    "tiny": Workload("tiny", "prefill", B=1, L=0, T=256, m=4, d=64, D=32, H=4, H_I=4, D_I=16,
                     k=16, W=16, dtype="f32", idx_dtype="f32"),
    # Single-layer causal prefill, bf16 storage, fp32 accumulation.
    "prefill8k": Workload("prefill8k", "prefill", B=1, L=0, T=8192, m=4, d=4096, D=512, H=64,
                          H_I=64, D_I=128, k=512, W=128, dtype="bf16", idx_dtype="bf16"),
    # Batched decode: 64 sequences at 131072 tokens of context, one new token each.
    "decode128k": Workload("decode128k", "decode", B=64, L=131072, T=1, m=4, d=0, D=512, H=128,
                           H_I=64, D_I=128, k=1024, W=128, dtype="bf16", idx_dtype="bf16"),
    # 4096-token query chunk at the end of a 1M-token context.
    "chunk1m": Workload("chunk1m", "prefill", B=1, L=1_044_480, T=4096, m=4, d=4096, D=512,
                        H=128, H_I=64, D_I=128, k=1024, W=128, dtype="bf16", idx_dtype="bf16"),
    # 1M-token decode with the indexer q/k in MXFP4.
    "decode1m_fp4": Workload("decode1m_fp4", "decode", B=4, L=1_048_576, T=1, m=4, d=0, D=512,
                             H=128, H_I=64, D_I=128, k=1024, W=128, dtype="bf16",
                             idx_dtype="mxfp4"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]
