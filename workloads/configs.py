"""The five attention workloads, named by what they are.

Shapes are ``[B, H, N, D]`` (batch, heads, sequence length, head dimension),
one layout for Q, K, V and O.  Values are iid draws from a seeded generator
(see ``inputs.py``); the softmax scale is ``1/sqrt(D)``, the factor used in
"Flash Attention on Android: tiled SGEMM with RenderScript", section
"Architecture: tiled attention with RenderScript BLAS".

The first page ("Android Transformer Optimization: Attention and Mobile GPU
Bottlenecks", opening paragraph and section "Pitfalls I Hit") measures the
prefill attention of a 1B-parameter LLM at 2048 tokens; the second page's
section "Benchmark results: Snapdragon vs. Dimensity" measures 32-head
attention at head dimension 128.  The workloads below stand in for those with
synthetic data of that shape.
"""

from dataclasses import dataclass, replace
import math


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str  # "f32" | "f16" | "bf16": storage type of Q, K, V and O
    causal: bool
    seed: int
    qk_sigma: float = 1.0  # Q and K ~ N(0, qk_sigma^2)
    v_dist: str = "normal"  # "normal": V ~ N(0,1); "uniform": V ~ U[-1, 1)
    uniform_head: bool = False  # head (b=0, h=0): every K row equals its row 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.D)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


_LIST = [
    Workload("single_head_b1h1n128d64_f32", 1, 1, 128, 64, "f32", False, 1001),
    Workload("prefill_b1h32n2048d64_f16", 1, 32, 2048, 64, "f16", False, 1002),
    Workload("prefill_causal_b4h32n2048d64_bf16", 4, 32, 2048, 64, "bf16", True, 1003),
    Workload("long_prefill_causal_b1h16n8192d128_f16_sigma3", 1, 16, 8192, 128, "f16", True, 1004,
             qk_sigma=3.0, v_dist="uniform"),
    Workload("ragged_b2h8n1000d96_f16_uniform_head", 2, 8, 1000, 96, "f16", False, 1005,
             uniform_head=True),
]

# The shapes of the second page's comparison of the tiled pass with naive
# attention ("Flash Attention on Android: tiled SGEMM with RenderScript",
# section "Benchmark results: Snapdragon vs. Dimensity": 32 heads, head
# dimension 128, sequence lengths 512 and 1024), at fp16 storage.  They are
# benchmark cases for that comparison, not among the five parity workloads.
_PAGE_TABLE = [
    Workload("page_table_b1h32n512d128_f16", 1, 32, 512, 128, "f16", False, 1006),
    Workload("page_table_b1h32n1024d128_f16", 1, 32, 1024, 128, "f16", False, 1007),
]

CONFIGS = {w.name: w for w in _LIST + _PAGE_TABLE}
ORDER = [w.name for w in _LIST]
PAGE_TABLE = [w.name for w in _PAGE_TABLE]
# The workload the throughput figure is quoted on: 1B-LLM prefill, fp16.
HEADLINE = "prefill_b1h32n2048d64_f16"


def get(name: str) -> Workload:
    return CONFIGS[name]


def flops(w: Workload) -> float:
    """Algorithmic FLOPs of one forward pass: two N x N x D products per head
    (QK^T and PV, 2 FLOP per multiply-add), halved under the causal mask."""
    f = 4.0 * w.B * w.H * w.N * w.N * w.D
    return f / 2 if w.causal else f


def min_bytes(w: Workload) -> int:
    """The least HBM traffic any implementation needs: read Q, K, V once and
    write O once."""
    item = 4 if w.dtype == "f32" else 2
    return 4 * w.B * w.H * w.N * w.D * item


def score_matrix_bytes(n: int, itemsize: int) -> int:
    """Bytes of one head's n x n score matrix, the intermediate that the
    tiled pass never writes out."""
    return n * n * itemsize


def naive_bytes(w: Workload) -> int:
    """HBM traffic a three-pass attention needs at the least, as built here:
    min_bytes, plus the fp32 score matrix written once and read once, plus
    the probabilities written once and read once (2 bytes per entry; 4 for
    bf16 storage, which keeps P as a rounded value and its remainder), over
    the visible entries of each head (N^2, or N(N+1)/2 under the causal
    mask).  The pages count the same round trips of the n x n matrix
    ("Android Transformer Optimization: Attention and Mobile GPU
    Bottlenecks", section "The Self-Attention Bottleneck Is Memory Traffic,
    Not Compute")."""
    if w.dtype == "f32":
        raise ValueError("the three-pass path takes 16-bit storage only")
    p_item = 4 if w.dtype == "bf16" else 2
    vis = w.N * (w.N + 1) // 2 if w.causal else w.N * w.N
    return min_bytes(w) + w.B * w.H * vis * (4 + 4 + 2 * p_item)
