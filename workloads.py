"""Seeded synthetic router workloads — inputs only.

This module draws the random inputs that the HIP path and the CPU oracle are
both fed; it holds none of the routing arithmetic. Every array is drawn on
the CPU with ``torch.Generator().manual_seed(seed)`` in the order W_g, bias,
x, then rounded to the input dtype (bf16 by round-to-nearest-even), so the
same seed gives the same bits on every machine.

The five workloads are the router shapes the method is described on: a tiny
four-expert softmax router, a Mixtral-like top-2 router, the DeepSeek-V3
group-limited sigmoid router (256 experts, 8 groups of 32, keep 4, top-8),
the same router under collapse (four "celebrity" experts with a +3.0 logit
offset) driven by the sign bias update, and a decode-shaped batch of 64
independent router layers with a shared-expert slot.
"""
from dataclasses import dataclass, field, replace

import torch

SOFTMAX, SIGMOID = 0, 1
BF16, F32 = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens per layer
    d: int                 # hidden size
    N: int                 # routed experts
    K: int                 # routed experts per token
    score_fn: int
    dtype: int             # dtype of x and W_g
    n_groups: int = 1
    topk_groups: int = 1
    n_shared: int = 0
    n_layers: int = 1
    bias_range: float = 0.0          # bias ~ U(-r, r); 0 -> zeros
    celebrities: tuple = ()          # experts given a logit offset
    celebrity_offset: float = 0.0
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def Kt(self):
        return self.K + self.n_shared

    @property
    def Nb(self):
        return self.N + self.n_shared


WORKLOADS = {
    "tiny_softmax": Workload("tiny_softmax", T=64, d=128, N=4, K=1, score_fn=SOFTMAX, dtype=F32,
                             notes="64 assignments over 4 experts, fp32"),
    "mixtral_top2": Workload("mixtral_top2", T=4096, d=4096, N=8, K=2, score_fn=SOFTMAX, dtype=BF16),
    "dsv3_group": Workload("dsv3_group", T=16384, d=7168, N=256, K=8, score_fn=SIGMOID, dtype=BF16,
                           n_groups=8, topk_groups=4, bias_range=0.01),
    "collapse_balance": Workload("collapse_balance", T=16384, d=7168, N=256, K=8, score_fn=SIGMOID,
                                 dtype=BF16, n_groups=8, topk_groups=4, bias_range=0.01,
                                 celebrities=(2, 4, 7, 12), celebrity_offset=3.0),
    "decode_layers": Workload("decode_layers", T=128, d=7168, N=256, K=8, score_fn=SIGMOID,
                              dtype=BF16, n_shared=1, n_layers=64, bias_range=0.01),
}


def scaled(wl: Workload, **kw) -> Workload:
    """The same router recipe at other sizes (for tests the oracle finishes fast)."""
    return replace(wl, **kw)


def _round(t, dtype):
    return t.to(torch.bfloat16) if dtype == BF16 else t.contiguous()


def make_router(wl: Workload):
    """W_g [L,N,d] (~N(0, 1/d)), bias [L,N] fp32, logit offset [N] or None."""
    g = torch.Generator().manual_seed(wl.seed)
    L, N, d = wl.n_layers, wl.N, wl.d
    W = torch.randn(L, N, d, generator=g) * (1.0 / d ** 0.5)
    if wl.bias_range > 0:
        b = (torch.rand(L, N, generator=g) * 2.0 - 1.0) * wl.bias_range
    else:
        b = torch.zeros(L, N)
    off = None
    if wl.celebrities:
        off = torch.zeros(N)
        off[list(wl.celebrities)] = wl.celebrity_offset
    return _round(W, wl.dtype), b.float().contiguous(), off, g


def make_hidden(wl: Workload, gen=None, seed=None):
    """x [L,T,d] ~ N(0,1). Drawn after W_g and b from the router's generator,
    or from its own generator when ``seed`` is given (per-iteration batches)."""
    if seed is not None:
        gen = torch.Generator().manual_seed(seed)
    x = torch.randn(wl.n_layers, wl.T, wl.d, generator=gen)
    return _round(x, wl.dtype)


def make_inputs(wl: Workload):
    W, b, off, g = make_router(wl)
    x = make_hidden(wl, gen=g)
    return {"x": x, "W": W, "bias": b, "offset": off}


def make_logits(T, N, seed, n_layers=1):
    """Standard-normal logits [L,T,N] fp32 — the distribution of h = x·W_g
    under the recipe above — for score-level tests that skip the GEMM."""
    g = torch.Generator().manual_seed(seed)
    return torch.randn(n_layers, T, N, generator=g)


def make_bias(N, seed, r=0.01, n_layers=1):
    g = torch.Generator().manual_seed(seed)
    return ((torch.rand(n_layers, N, generator=g) * 2.0 - 1.0) * r).float()


def make_indices(T, Kt, Nb, seed, n_layers=1):
    """Random distinct expert ids per token [L,T,Kt] int32."""
    g = torch.Generator().manual_seed(seed)
    r = torch.rand(n_layers, T, Nb, generator=g)
    return torch.argsort(r, dim=-1)[..., :Kt].to(torch.int32).contiguous()


def make_expert_rows(n_rows, d, seed, dtype=BF16, n_layers=1):
    """Stand-in expert outputs [L,n_rows,d] ~ N(0,1), one row per layout
    position (the experts themselves are outside the router)."""
    g = torch.Generator().manual_seed(seed)
    return _round(torch.randn(n_layers, n_rows, d, generator=g), dtype)


def make_weights(T, Kt, seed, n_layers=1):
    """Positive fp32 weights [L,T,Kt] in (0, 1) for combine-only tests."""
    g = torch.Generator().manual_seed(seed)
    return torch.rand(n_layers, T, Kt, generator=g).float().contiguous()
