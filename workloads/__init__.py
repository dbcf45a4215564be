"""Seeded synthetic inputs for the MoE layer forward pass.

This module is shared by the CPU oracle, the tests, ``bench.py`` and the smoke
entry point.  It draws random tensors and casts them to their storage dtypes;
it performs none of the layer's own arithmetic (no projection, ranking, gating,
capacity, alignment, expert FFN or combine).

Workload shapes follow the layer families named in "Mixture-of-Experts Routing
at Inference Time" (section "Who this is for": Mixtral, DeepSeek and Qwen MoE
families); the per-config recipes are stated on each ``Workload`` below.

Every tensor gets its own generator stream derived from ``(seed, name, index)``
so that any one expert's weights can be regenerated alone, and the same bytes
come out on every call.  Large weight stacks may be drawn on a GPU (torch's
Philox generator) with ``device="cuda"``; the bytes are then the source of
truth and are copied back to the host for the oracle.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import torch

F32, BF16, FP8 = "f32", "bf16", "fp8_e4m3"
FP8_MAX = 448.0  # largest finite OCP E4M3FN magnitude


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int              # tokens
    H: int              # hidden
    N: int              # routed experts
    k: int              # experts per token
    I: int              # expert FFN intermediate
    B: int              # padded row-block size of the alignment
    act_dtype: str      # h, residual, out, router weight, act, y_route
    expert_dtype: str   # f32 / bf16 / fp8_e4m3
    cap_num: int = 0    # capacity factor as a rational; 0/0 = dropless
    cap_den: int = 0
    n_shared: int = 0
    renormalize: int = 1
    scale_block: int = 0       # fp8 block scale size (128) or 0
    reroute_depth: int = 0     # overflow policy under capacity: 0 drop, d > 0 reroute rounds
    zipf_s: float = 0.0        # additive per-expert logit bias -s*ln(e+1)
    near_tie_frac: float = 0.0 # fraction of tokens given a k-th/(k+1)-th margin < 1e-3
    routing: str = "token_choice"  # or "expert_choice" (each expert picks its tokens)
    seed: int = 0

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five layer shapes.  c0 is small enough for pure-Python checks, c2 is the
# Mixtral-shaped layer the throughput line is quoted on.
TOY_FP32 = Workload("toy_fp32", T=64, H=128, N=8, k=2, I=256, B=8,
                    act_dtype=F32, expert_dtype=F32)
SWITCH_BF16 = Workload("switch_capacity_bf16", T=2048, H=1024, N=16, k=1, I=4096, B=64,
                       act_dtype=BF16, expert_dtype=BF16, cap_num=5, cap_den=4, zipf_s=1.1)
MIXTRAL_BF16 = Workload("mixtral_bf16", T=4096, H=4096, N=8, k=2, I=14336, B=64,
                        act_dtype=BF16, expert_dtype=BF16)
QWEN3MOE_BF16 = Workload("qwen3moe_bf16", T=8192, H=2048, N=128, k=8, I=768, B=16,
                         act_dtype=BF16, expert_dtype=BF16, near_tie_frac=0.05)
DEEPSEEKV3_FP8 = Workload("deepseekv3_fp8", T=16384, H=7168, N=256, k=8, I=2048, B=64,
                          act_dtype=BF16, expert_dtype=FP8, n_shared=1, scale_block=128)

# the capacity workload with the reroute overflow policy walking each token's whole ranking
SWITCH_REROUTE_BF16 = SWITCH_BF16.with_(name="switch_reroute_bf16", reroute_depth=15)
# Expert-choice routing on the same inputs ("Mixture-of-experts routing & LLM repeatability",
# paragraph on expert-choice routing): k is the mean number of experts per token, so each
# expert takes T*k/N tokens (capacity factor 1) -- as many expert rows as token choice.
TOY_EC_FP32 = TOY_FP32.with_(name="toy_ec_fp32", routing="expert_choice")
MIXTRAL_EC_BF16 = MIXTRAL_BF16.with_(name="mixtral_ec_bf16", routing="expert_choice")
QWEN3MOE_EC_BF16 = QWEN3MOE_BF16.with_(name="qwen3moe_ec_bf16", routing="expert_choice", near_tie_frac=0.0)
DEEPSEEKV3_EC_FP8 = DEEPSEEKV3_FP8.with_(name="deepseekv3_ec_fp8", routing="expert_choice")
ALL = {w.name: w for w in (TOY_FP32, SWITCH_BF16, SWITCH_REROUTE_BF16, MIXTRAL_BF16, QWEN3MOE_BF16, DEEPSEEKV3_FP8,
                           TOY_EC_FP32, MIXTRAL_EC_BF16, QWEN3MOE_EC_BF16, DEEPSEEKV3_EC_FP8)}


def _stream_seed(seed: int, name: str, index: int = 0) -> int:
    digest = hashlib.sha256(f"{seed}/{name}/{index}".encode()).digest()
    return int.from_bytes(digest[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, name: str, index: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_stream_seed(seed, name, index))
    return g


def _normal(shape, std: float, seed: int, name: str, index: int = 0, device: str = "cpu") -> torch.Tensor:
    g = _gen(seed, name, index, device)
    return torch.randn(shape, generator=g, dtype=torch.float32, device=device) * std


def torch_dtype(tag: str) -> torch.dtype:
    return {F32: torch.float32, BF16: torch.bfloat16, FP8: torch.float8_e4m3fn}[tag]


def hidden_states(w: Workload, T: Optional[int] = None, device: str = "cpu") -> torch.Tensor:
    """h [T, H]: x ~ N(0,1), then each row RMS-normalised (eps 1e-6), cast to the act dtype.

    Rows are drawn one stream per 256-token slab so that a prefix of a longer
    pool is the same bytes as a shorter draw.
    """
    T = w.T if T is None else T
    slab = 256
    parts = []
    for s in range(0, T, slab):
        n = min(slab, T - s)
        x = _normal((slab, w.H), 1.0, w.seed, "x", s // slab, device)[:n].double()
        x = x / torch.sqrt((x * x).mean(dim=1, keepdim=True) + 1e-6)
        parts.append(x.to(torch_dtype(w.act_dtype)))
    return torch.cat(parts, 0).contiguous()


def router_weight(w: Workload, device: str = "cpu") -> torch.Tensor:
    """W_g stored [N, H] (the nn.Linear layout), entries ~ N(0, 0.02), act dtype."""
    return _normal((w.N, w.H), 0.02, w.seed, "w_gate", 0, device).to(torch_dtype(w.act_dtype)).contiguous()


def logit_bias(w: Workload) -> Optional[torch.Tensor]:
    """Zipf-shaped additive router bias, fp32 [N]: bias[e] = -s * ln(e + 1); None if s == 0."""
    if w.zipf_s == 0.0:
        return None
    return torch.tensor([-w.zipf_s * math.log(e + 1) for e in range(w.N)], dtype=torch.float32)


def _expert_f32(w: Workload, which: str, e: int, device: str) -> torch.Tensor:
    if which == "w13":
        return _normal((2 * w.I, w.H), 1.0 / math.sqrt(w.H), w.seed, "w13", e, device)
    if which == "w2":
        return _normal((w.H, w.I), 1.0 / math.sqrt(w.I), w.seed, "w2", e, device)
    if which == "shared_w13":
        return _normal((2 * w.I, w.H), 1.0 / math.sqrt(w.H), w.seed, "shared_w13", e, device)
    if which == "shared_w2":
        return _normal((w.H, w.I), 1.0 / math.sqrt(w.I), w.seed, "shared_w2", e, device)
    raise ValueError(which)


def quantize_fp8_blocks(wf: torch.Tensor, block: int):
    """Encode an fp32 matrix [R, C] as OCP E4M3FN codes with one bf16 scale per block x block tile.

    scale = bf16(max|W| / 448) over the tile; code = e4m3(clamp(W / scale, +-448)).
    Returns (codes uint8 [R, C], scales bf16 [R/block, C/block]).
    """
    R, C = wf.shape
    t = wf.reshape(R // block, block, C // block, block)
    amax = t.abs().amax(dim=(1, 3))
    scale = (amax / FP8_MAX).clamp(min=2.0 ** -126).to(torch.bfloat16)
    s = scale.float()[:, None, :, None]
    q = (t / s).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q.reshape(R, C).view(torch.uint8).contiguous(), scale.contiguous()


def expert_weight(w: Workload, which: str, e: int, device: str = "cpu"):
    """One expert's weight in storage form.

    which: "w13" -> [2I, H] (rows 0..I-1 gate projection, I..2I-1 up projection),
           "w2"  -> [H, I]; "shared_w13"/"shared_w2" likewise for the always-on expert.
    Returns the tensor (and for fp8 a (codes, scales) pair).
    """
    wf = _expert_f32(w, which, e, device)
    if w.expert_dtype == FP8:
        return quantize_fp8_blocks(wf, w.scale_block)
    return wf.to(torch_dtype(w.expert_dtype)).contiguous()


def expert_stack(w: Workload, which: str, device: str = "cpu"):
    """All N experts' weights stacked: w13 [N, 2I, H], w2 [N, H, I] (and scales for fp8)."""
    parts = [expert_weight(w, which, e, device) for e in range(w.N)]
    if w.expert_dtype == FP8:
        return torch.stack([p[0] for p in parts]).contiguous(), torch.stack([p[1] for p in parts]).contiguous()
    return torch.stack(parts).contiguous()


def drawn_logits(w: Workload, T: Optional[int] = None) -> torch.Tensor:
    """Router logits drawn directly (fp32 [T, N]) for routing-only stress.

    Entries ~ N(0, 0.905^2), the spread h.W_g has under this recipe.  Then a seeded
    permutation of tokens is walked and, until round(near_tie_frac * T) tokens have a
    gap below 1e-3 between their k-th and (k+1)-th largest logit, the (k+1)-th
    largest is moved to (k-th largest - delta), with delta = 0 for a quarter of the
    injected tokens (exact ties) and U(0, 1e-3) otherwise.
    """
    T = w.T if T is None else T
    g = _gen(w.seed, "drawn_logits", 0, "cpu")
    lg = torch.randn((T, w.N), generator=g, dtype=torch.float32) * 0.905
    if w.near_tie_frac <= 0 or w.k >= w.N:
        return lg.contiguous()
    target = int(round(w.near_tie_frac * T))
    vals, order = torch.sort(lg, dim=1, descending=True, stable=True)
    gap = vals[:, w.k - 1] - vals[:, w.k]
    have = int((gap < 1e-3).sum())
    perm = torch.randperm(T, generator=g)
    u = torch.rand((T,), generator=g, dtype=torch.float32)
    n_inj = 0
    for t in perm.tolist():
        if have >= target:
            break
        if gap[t] < 1e-3:
            continue
        delta = 0.0 if n_inj % 4 == 0 else float(u[t]) * 1e-3
        kth = float(vals[t, w.k - 1])
        new = torch.tensor(kth, dtype=torch.float32) - torch.tensor(delta, dtype=torch.float32)
        if float(kth - new) >= 1e-3:  # keep the injected gap strictly below 1e-3 after rounding
            new = torch.tensor(kth, dtype=torch.float32)
        lg[t, order[t, w.k]] = new
        n_inj += 1
        have += 1
    return lg.contiguous()


def layer_inputs(w: Workload, device: str = "cpu", weights_device: Optional[str] = None) -> dict:
    """Every input of one layer pass, in storage dtypes.

    h, residual (= h, so a fully dropped token passes h through), w_gate, bias,
    w13/w2 (+ scales), shared expert (if any).
    """
    wdev = weights_device or device
    d = {
        "h": hidden_states(w, device=device),
        "w_gate": router_weight(w, device=device),
        "bias": logit_bias(w),
    }
    d["residual"] = d["h"]
    if w.expert_dtype == FP8:
        d["w13"], d["w13_scale"] = expert_stack(w, "w13", wdev)
        d["w2"], d["w2_scale"] = expert_stack(w, "w2", wdev)
    else:
        d["w13"] = expert_stack(w, "w13", wdev)
        d["w2"] = expert_stack(w, "w2", wdev)
        d["w13_scale"] = d["w2_scale"] = None
    if w.n_shared:
        sw13 = expert_weight(w, "shared_w13", 0, wdev)
        sw2 = expert_weight(w, "shared_w2", 0, wdev)
        if w.expert_dtype == FP8:
            d["shared_w13"], d["shared_w13_scale"] = sw13
            d["shared_w2"], d["shared_w2_scale"] = sw2
        else:
            d["shared_w13"], d["shared_w2"] = sw13, sw2
            d["shared_w13_scale"] = d["shared_w2_scale"] = None
    return d


def random_routes(T: int, N: int, k: int, seed: int, skew: float = 0.0) -> torch.Tensor:
    """Synthetic expert ids [T, k] int32 (distinct per token), optionally Zipf-skewed.

    Used to drive the alignment and capacity stages directly.  Each token draws k
    distinct experts without replacement from weights (e+1)^-skew.
    """
    g = _gen(seed, "routes", 0, "cpu")
    wts = torch.tensor([(e + 1.0) ** (-skew) for e in range(N)], dtype=torch.float64)
    ids = torch.multinomial(wts.expand(T, N), k, replacement=False, generator=g)
    return ids.to(torch.int32).contiguous()


def random_gates(T: int, k: int, seed: int) -> torch.Tensor:
    """Positive fp32 gates [T, k] in (0.05, 1) for driving the combine stage directly."""
    g = _gen(seed, "gates", 0, "cpu")
    return (torch.rand((T, k), generator=g, dtype=torch.float32) * 0.95 + 0.05).contiguous()


def random_rows(R: int, H: int, dtype: str, seed: int, name: str = "rows") -> torch.Tensor:
    """Standard-normal rows [R, H] in a storage dtype (expert outputs for driving combine)."""
    return _normal((R, H), 1.0, seed, name, 0).to(torch_dtype(dtype)).contiguous()
