"""Workload shapes for the Focus group-gated attention forward pass.

Each workload fixes the shapes of one layer's inference-time forward:
hidden states h (B x n x d_model) are projected by P (d_model x d_proj) and
compared with K centroids C (K x d_proj) to pick each token's group (Focus,
"Focus: Learning Which Attention Pairs Matter", technical summary §2.1 and the
hard top-k assignment of §2.2); attention then runs over the causal local
window of width w plus same-group long-range pairs (§2.1-§2.2, pair count
O(n^2/K + n*w)).

Pure data: no arithmetic of the method lives here.
"""
from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class Workload:
    name: str
    B: int            # batch
    Hq: int           # query heads
    Hkv: int          # key/value heads (GQA when Hkv < Hq)
    n: int            # sequence length
    d: int            # head dim
    d_model: int      # hidden width
    d_proj: int       # width of the centroid space (projection output)
    K: int            # number of groups / centroids
    w: int            # local window: pairs with 0 <= i-j <= w are always kept
    m: int = 1        # groups per token (top-m membership; far pairs sharing any group are kept)
    # how P and C are drawn: "gauss" = P ~ N(0, 1/d_model), C = row-normalised
    # N(0,1); "orthonormal" = P with orthonormal columns and C with orthonormal
    # rows, which makes the K centroid logits i.i.d. N(0,1) per token so that a
    # per-group logit bias sets the expected group sizes exactly.
    pc_kind: str = "gauss"
    # target group-size distribution for the logit bias ("zipf" / None)
    bias_target: Optional[str] = None
    zipf_s: float = 1.1
    # q is drawn N(0,1) and multiplied by q_prescale before bf16 rounding
    q_prescale: float = 1.0
    # softmax scale passed to the attention call; None = 1/sqrt(d)
    scale: Optional[float] = None
    seed: int = 0

    @property
    def softmax_scale(self) -> float:
        return (1.0 / self.d ** 0.5) if self.scale is None else float(self.scale)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five layer shapes this library is measured and checked on.
TINY = Workload("tiny_n256", B=1, Hq=2, Hkv=2, n=256, d=32, d_model=64, d_proj=32,
                K=4, w=32, seed=1000)
GPT2 = Workload("gpt2_small_n1024", B=8, Hq=12, Hkv=12, n=1024, d=64, d_model=768,
                d_proj=64, K=16, w=128, seed=1001)
ZIPF7B = Workload("7b_zipf_n8192", B=1, Hq=32, Hkv=32, n=8192, d=128, d_model=4096,
                  d_proj=128, K=32, w=512, pc_kind="orthonormal", bias_target="zipf",
                  seed=1002)
LONG64K = Workload("long_n65536", B=1, Hq=8, Hkv=8, n=65536, d=128, d_model=1024,
                   d_proj=128, K=64, w=1024, pc_kind="orthonormal",
                   q_prescale=1.0 / 128 ** 0.5, scale=1.0, seed=1003)
GQA70B = Workload("70b_gqa_n32768", B=1, Hq=64, Hkv=8, n=32768, d=128, d_model=8192,
                  d_proj=128, K=32, w=1024, seed=1004)

# The pages' one-million-token regime (Korean page §3.4, Japanese page §3.3;
# K, w and the model are not stated there): the 64K layer shape at n = 2^20.
LONG1M = Workload("long_n1048576", B=1, Hq=8, Hkv=8, n=1 << 20, d=128, d_model=1024,
                  d_proj=128, K=64, w=1024, pc_kind="orthonormal",
                  q_prescale=1.0 / 128 ** 0.5, scale=1.0, seed=1005)

# Top-2 membership at K = 4, the pages' top-k setting (Korean page §3.4,
# Japanese page §3.3), on the 70B attention layer shape; and the same rule at
# K = 32, where it is much sparser.
TOP2_K4 = Workload("70b_gqa_top2_k4_n32768", B=1, Hq=64, Hkv=8, n=32768, d=128, d_model=8192,
                   d_proj=128, K=4, w=1024, m=2, seed=1006)
TOP2_K32 = Workload("70b_gqa_top2_k32_n32768", B=1, Hq=64, Hkv=8, n=32768, d=128,
                    d_model=8192, d_proj=128, K=32, w=1024, m=2, seed=1007)

ALL = [TINY, GPT2, ZIPF7B, LONG64K, GQA70B, LONG1M, TOP2_K4, TOP2_K32]
BY_NAME = {w.name: w for w in ALL}
