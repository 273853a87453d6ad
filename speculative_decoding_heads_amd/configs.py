"""The five synthetic workloads of the verify step, as data.

Shapes follow the problem statement: a tiny fp32 case, a Llama-7B-shaped
case at batch 1 and 16, a Llama-70B-layer shape with grouped-query attention,
and a 128k-vocabulary, 32k-context stress case.  Weights ~ N(0, 0.02^2) and
hidden states, queries and cache ~ N(0, 1) (see ``synth``).
"""

from dataclasses import dataclass, field
from fractions import Fraction


@dataclass(frozen=True)
class Config:
    name: str
    index: int                 # 1-based workload number, used in input seeds
    b: int                     # sequences per step
    H: int                     # hidden size
    V: int                     # vocabulary
    k: tuple                   # shortlist size per Medusa head (K = len(k))
    N: object                  # candidates kept (None = full tree)
    nq: int                    # query heads
    nkv: int                   # key/value heads
    d: int                     # head dim
    P: int                     # prefix length per sequence
    dtype: str                 # "f32" or "bf16" (logits are always fp32)
    mode: str                  # "greedy", "typical" or "reject"
    temperature: float = 0.7
    eps: float = 0.3
    delta: float = 0.09
    decay: Fraction = Fraction(4, 5)

    @property
    def K(self):
        return len(self.k)

    @property
    def kmax(self):
        return max(self.k)

    @property
    def n_candidates(self):
        if self.N is not None:
            return self.N
        total, p = 0, 1
        for s in self.k:
            p *= s
            total += p
        return total

    @property
    def T(self):
        return self.n_candidates + 1

    @property
    def Pmax(self):
        return self.P + self.T

    @property
    def seed(self):
        return 0x5EED + self.index

    def with_(self, **kw):
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


TINY = Config("tiny_fp32", 1, b=1, H=256, V=4096, k=(2, 2, 1), N=None,
              nq=4, nkv=4, d=64, P=128, dtype="f32", mode="greedy", temperature=1.0)
LLAMA7B_BS1 = Config("llama7b_bs1", 2, b=1, H=4096, V=32000, k=(10, 10, 10, 10), N=64,
                     nq=32, nkv=32, d=128, P=2048, dtype="bf16", mode="greedy", temperature=1.0)
LLAMA7B_BS16 = Config("llama7b_bs16", 3, b=16, H=4096, V=32000, k=(10, 10, 10, 10), N=64,
                      nq=32, nkv=32, d=128, P=4096, dtype="bf16", mode="typical")
LLAMA70B_BS8 = Config("llama70b_layer_bs8", 4, b=8, H=8192, V=32000, k=(10, 10, 10, 10, 10),
                      N=128, nq=64, nkv=8, d=128, P=8192, dtype="bf16", mode="greedy",
                      temperature=1.0)
LONGCTX_BS32 = Config("vocab128k_ctx32k_bs32", 5, b=32, H=4096, V=128256, k=(10, 10, 10, 10),
                      N=64, nq=32, nkv=8, d=128, P=32768, dtype="bf16", mode="typical")

CONFIGS = [TINY, LLAMA7B_BS1, LLAMA7B_BS16, LLAMA70B_BS8, LONGCTX_BS32]
BY_NAME = {c.name: c for c in CONFIGS}
