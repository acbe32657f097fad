"""The five synthetic workloads, shaped like the HySparse2 pages' settings.

HySparse2 (onedev.kr/papers/146, section "어떻게 쓰나") fixes MQA (one KV head),
NoPE, 128 forced local tokens and 1,024 global tokens; 32k is its pre-training
context and 256k its post-training context; its efficiency figures use an FP8
KV cache up to 1M tokens (section "전제와 한계"). Head counts, head dim and
batch sizes are not on the pages; the values below are this build's choices.
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int          # seed namespace
    B: int               # sequences
    n_q: int             # query tokens per sequence
    q_pos0: int          # position of the first query token
    n_ctx: int           # KV length (includes the query tokens themselves)
    H: int               # query heads (MQA: one KV head)
    d: int               # head dim
    q_dtype: str         # "f32" | "bf16"
    kv_dtype: str        # "f32" | "bf16" | "fp8"
    window: int          # forced recent tokens
    k_global: int        # top-k outside the window
    n_sparse: int        # sparse layers reusing the indices
    needles: str         # "rows" | "decode" | "clusters" | "depth" | "none"
    n_needles: int       # needles per sequence (clusters: number of clusters)
    cluster_len: int = 8
    decode: bool = False

    @property
    def n_sel(self) -> int:
        return self.window + self.k_global

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    1: Workload("tiny_prefill_2k_f32", 1, B=1, n_q=2048, q_pos0=0, n_ctx=2048, H=4, d=64,
                q_dtype="f32", kv_dtype="f32", window=128, k_global=256, n_sparse=1,
                needles="rows", n_needles=16),
    2: Workload("prefill_32k_bf16", 2, B=1, n_q=32768, q_pos0=0, n_ctx=32768, H=16, d=128,
                q_dtype="bf16", kv_dtype="bf16", window=128, k_global=1024, n_sparse=2,
                needles="rows", n_needles=256),
    3: Workload("decode_b64_128k_bf16", 3, B=64, n_q=1, q_pos0=131071, n_ctx=131072, H=16, d=128,
                q_dtype="bf16", kv_dtype="bf16", window=128, k_global=1024, n_sparse=4,
                needles="decode", n_needles=32, decode=True),
    4: Workload("chunked_prefill_8k_at_256k_fp8", 4, B=1, n_q=8192, q_pos0=253952, n_ctx=262144,
                H=16, d=128, q_dtype="bf16", kv_dtype="fp8", window=128, k_global=1024,
                n_sparse=3, needles="clusters", n_needles=32, cluster_len=8),
    5: Workload("decode_b4_1m_fp8", 5, B=4, n_q=1, q_pos0=1048575, n_ctx=1048576, H=16, d=128,
                q_dtype="bf16", kv_dtype="fp8", window=128, k_global=1024, n_sparse=5,
                needles="depth", n_needles=64, decode=True),
}


def workload(cfg: int) -> Workload:
    return WORKLOADS[cfg]
