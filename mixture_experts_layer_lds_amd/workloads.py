"""Seeded synthetic MoE-layer workloads: shapes, value distributions and input generation.

This module holds no arithmetic of the layer itself (no routing, no expert math, no combine):
it only draws the inputs, so that the HIP library's tests and the CPU oracle's checks can be fed
the very same tensors.  It imports neither the HIP binding nor the oracle.

Shapes follow the layers the SonicMoE summary page discusses (background table of activation
ratio K/E and granularity d/n: Mixtral-like coarse layers, DeepSeek-V3 8 of 256 with d/n = 3.5,
Kimi K2 8 of 384, and the "fine-grained 7B MoE at microbatch 32768" kernel benchmark).  The
pages publish no dataset or weights for these, so every tensor is drawn from a seeded normal:

* X, dY ~ N(0, 1);  router W_r ~ N(0, 0.02);  W_gate, W_up ~ N(0, 1/sqrt(d));
  W_down ~ N(0, 1/sqrt(n))   (second argument = standard deviation);
* DeepSeek-V3-shaped layer: per-expert logit bias ~ N(0, 1) (moderate load imbalance);
* Kimi-K2-shaped layer: Zipf(s = 1.1) per-expert bias  b_e = -1.1 ln(pi_e)  with pi a seeded
  random permutation of 1..E, i.e. log-probabilities proportional to rank^-1.1 (skewed loads
  without always making expert 0 the hot one).

Tensors are drawn in float32 from ``torch.Generator`` (on the device they are made for), seeded
per tensor with ``seed = 1000 * config_index + tensor_id``, then rounded to the layer's dtype.
"""

from dataclasses import dataclass, replace
import math

import torch

TENSOR_IDS = dict(X=0, W_r=1, W_gate=2, W_up=3, W_down=4, dY=5, bias=6, perm=7, round_rand=8)


@dataclass(frozen=True)
class LayerShape:
    name: str
    T: int
    d: int
    E: int
    K: int
    n: int
    dtype: str            # "f32" or "bf16"
    bias: str = "none"    # "none" | "normal" | "zipf"
    backward: bool = False
    round_mode: int = 0   # 0 none, 1 nearest, 2 up, 3 down, 4 stochastic
    tile_m: int = 128
    index: int = 0        # seed namespace

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw):
        return replace(self, **kw)


# The five layer shapes (index 0..4).
CONFIGS = [
    LayerShape("tiny_fp32", 256, 128, 8, 2, 256, "f32", index=0),
    LayerShape("mixtral_coarse", 8192, 4096, 8, 2, 14336, "bf16", index=1),
    LayerShape("fine_grained_7b", 32768, 1536, 128, 8, 256, "bf16", backward=True, index=2),
    LayerShape("deepseek_v3", 16384, 7168, 256, 8, 2048, "bf16", bias="normal", index=3),
    LayerShape("kimi_k2", 32768, 7168, 384, 8, 2048, "bf16", bias="zipf", backward=True, index=4),
]
BY_NAME = {c.name: c for c in CONFIGS}


def _gen(shape_cfg, tensor, device):
    g = torch.Generator(device=device)
    g.manual_seed(1000 * shape_cfg.index + TENSOR_IDS[tensor])
    return g


def _normal(cfg, tensor, size, std, device, chunk_rows=None):
    """float32 N(0, std) draw rounded to the layer dtype; drawn in chunks along dim 0."""
    g = _gen(cfg, tensor, device)
    out = torch.empty(size, dtype=cfg.torch_dtype, device=device)
    rows = size[0]
    step = chunk_rows or rows
    for lo in range(0, rows, step):
        hi = min(rows, lo + step)
        part = torch.randn((hi - lo,) + tuple(size[1:]), generator=g, device=device,
                           dtype=torch.float32)
        out[lo:hi].copy_(part.mul_(std))
        del part
    return out


def make_bias(cfg, device="cpu"):
    """Per-expert logit bias (float32) or None."""
    if cfg.bias == "none":
        return None
    if cfg.bias == "normal":
        g = _gen(cfg, "bias", device)
        return torch.randn(cfg.E, generator=g, device=device, dtype=torch.float32)
    if cfg.bias == "zipf":
        g = _gen(cfg, "perm", "cpu")
        ranks = torch.randperm(cfg.E, generator=g).to(torch.float64) + 1.0
        return (-1.1 * torch.log(ranks)).to(torch.float32).to(device)
    raise ValueError(cfg.bias)


def make_inputs(cfg, device="cpu", with_grad_out=None):
    """All inputs of one layer: X, W_r, bias, W_gate, W_up, W_down and (backward) dY."""
    T, d, E, n = cfg.T, cfg.d, cfg.E, cfg.n
    big = T * d > (1 << 26) or E * n * d > (1 << 28)
    chunk_e = max(1, (1 << 26) // (n * d)) if big else None
    chunk_t = max(1, (1 << 26) // d) if big else None
    inp = dict(
        X=_normal(cfg, "X", (T, d), 1.0, device, chunk_t),
        W_r=_normal(cfg, "W_r", (E, d), 0.02, device),
        bias=make_bias(cfg, device),
        W_gate=_normal(cfg, "W_gate", (E, n, d), 1.0 / math.sqrt(d), device, chunk_e),
        W_up=_normal(cfg, "W_up", (E, n, d), 1.0 / math.sqrt(d), device, chunk_e),
        W_down=_normal(cfg, "W_down", (E, d, n), 1.0 / math.sqrt(n), device, chunk_e),
    )
    if with_grad_out if with_grad_out is not None else cfg.backward:
        inp["dY"] = _normal(cfg, "dY", (T, d), 1.0, device, chunk_t)
    inp["round_rand"] = make_round_rand(cfg, device)
    return inp


def make_round_rand(cfg, device="cpu"):
    """[E] uniform 32-bit random words (stored as int32 bit patterns) for stochastic token
    rounding; drawn like every other input, from the layer's seed namespace."""
    g = _gen(cfg, "round_rand", device)
    w = torch.randint(0, 1 << 32, (cfg.E,), generator=g, device=device, dtype=torch.int64)
    return (w - (w >= (1 << 31)).to(torch.int64) * (1 << 32)).to(torch.int32)


def round_rand_words(t):
    """The words of a make_round_rand tensor as numpy uint32 (for the CPU side)."""
    return t.cpu().numpy().view("uint32")


def small_shape(T, d, E, K, n, dtype="bf16", bias="none", backward=True, round_mode=0,
                tile_m=128, seed=17):
    """A custom shape in its own seed namespace (for tests)."""
    return LayerShape("custom", T, d, E, K, n, dtype, bias=bias, backward=backward,
                      round_mode=round_mode, tile_m=tile_m, index=seed)
