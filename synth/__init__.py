"""Seeded synthetic inputs shared by the tests, the benchmark and the CPU baseline.

This module only draws random numbers and casts them to storage types.  It holds
none of the expert-FFN arithmetic: no quantisation, no routing, no products.
Both the fp64 oracle (``oracle/``) and the HIP path receive what is drawn here.

Workload shapes and distributions follow the five expert configurations the
library is exercised on (SwiGLU experts with INT2 up weights, FloE review page,
"MoE 专家前向计算" and "混合压缩策略" sections):

=====  ====================================================================
name   shape / distribution
=====  ====================================================================
tiny   one expert, d=256, f=704, T=1; weights N(0, 0.02); x N(0,1)/16
mixtral one Mixtral-8x7B expert, d=4096, f=14336, T in {1, 4}; x N(0,1)/64
stack  32 layers x 8 experts of the Mixtral shape, top-2, x carried across
       layers as x_{l+1} = unit(x_l + 0.2 n_l), n_l ~ N(0,1)/64
wide   Mixtral-8x22B shape, 8 experts, d=6144, f=16384, top-2, 256 tokens, bf16
fine   DeepSeek-V2-Lite shape, 64 routed (top-6) + 2 shared, d=2048, f=1408,
       router bias -1.1 ln(rank) (Zipf, s=1.1), x N(0,1)
=====  ====================================================================

Request-level expert activation matrices (MoE-Infinity review, "4.3"-"4.4":
L x E token counts per request that fall into 10-30 groups of similar
matrices, each skewed within the request) are drawn by ``eam_collection``.

Seeds: ``seed = 1_000_000*cfg + 10_000*layer + 100*expert + tensor_id``.
"""
from __future__ import annotations

import numpy as np

T_GATE, T_UP, T_DOWN, T_ROUTER, T_X, T_CALIB, T_NOISE, T_RANK, T_EAM = range(9)

CFG_TINY, CFG_MIXTRAL, CFG_STACK, CFG_WIDE, CFG_FINE = 1, 2, 3, 4, 5

CONFIGS = {
    CFG_TINY: dict(name="tiny", d=256, f=704, E=1, k=1, S=0, L=1, wdt="f16",
                   x_scale=1.0 / 16, w_std=0.02),
    CFG_MIXTRAL: dict(name="mixtral", d=4096, f=14336, E=1, k=1, S=0, L=1, wdt="f16",
                      x_scale=1.0 / 64, w_std=0.02),
    CFG_STACK: dict(name="stack", d=4096, f=14336, E=8, k=2, S=0, L=32, wdt="f16",
                    x_scale=1.0 / 64, w_std=0.02, sparsity=0.8),
    CFG_WIDE: dict(name="wide", d=6144, f=16384, E=8, k=2, S=0, L=1, wdt="bf16",
                   x_scale=1.0 / 64, w_std=0.02, sparsity=0.7, T=256),
    CFG_FINE: dict(name="fine", d=2048, f=1408, E=64, k=6, S=2, L=1, wdt="f16",
                   x_scale=1.0, w_std=0.02, sparsity=0.7, zipf_s=1.1),
}


def seed_of(cfg: int, layer: int = 0, expert: int = 0, tensor_id: int = 0) -> int:
    return 1_000_000 * cfg + 10_000 * layer + 100 * expert + tensor_id


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_f32(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """Standard normal draws (PCG64) scaled by ``std``, float32."""
    a = rng(seed).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def to_f16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 (round to nearest even) as uint16 bit patterns."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (round to nearest even) as uint16 bit patterns.

    Finite inputs only (the generators here never produce NaN)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def to_bits(a: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f16":
        return to_f16_bits(a)
    if dt == "bf16":
        return to_bf16_bits(a)
    raise ValueError(dt)


def expert_weights_f32(cfg: int, layer: int, expert: int, d: int, f: int, std: float = 0.02):
    """fp32 draws for one expert: (gate_t [f][d], up_t [f][d], down [f][d]).

    Row j of ``gate_t`` is column j of W^gate, row j of ``up_t`` is column j
    of W^up and row j of ``down`` is row j of W^down."""
    g = normal_f32(seed_of(cfg, layer, expert, T_GATE), (f, d), std)
    u = normal_f32(seed_of(cfg, layer, expert, T_UP), (f, d), std)
    dn = normal_f32(seed_of(cfg, layer, expert, T_DOWN), (f, d), std)
    return g, u, dn


def tokens_f32(cfg: int, T: int, d: int, scale: float, layer: int = 0, tensor_id: int = T_X):
    return normal_f32(seed_of(cfg, layer, 0, tensor_id), (T, d), scale)


def calibration_f32(cfg: int, d: int, scale: float, layer: int = 0, expert: int = 0, n: int = 64):
    """The 64 seeded calibration vectors used to place an expert's threshold."""
    return normal_f32(seed_of(cfg, layer, expert, T_CALIB), (n, d), scale)


def router_f32(cfg: int, layer: int, E: int, d: int, std: float = 0.02):
    return normal_f32(seed_of(cfg, layer, 0, T_ROUTER), (E, d), std)


def zipf_bias(cfg: int, layer: int, E: int, s: float) -> np.ndarray:
    """Router bias skewed like a Zipf law: b_e = -s * ln(r_e), r a seeded
    permutation of the ranks 1..E (float32)."""
    ranks = rng(seed_of(cfg, layer, 0, T_RANK)).permutation(E) + 1
    return (-s * np.log(ranks.astype(np.float64))).astype(np.float32)


def eam_collection(cfg: int, n: int, L: int, E: int, k: int, groups: int = 20,
                   max_tokens: int = 512, alpha: float = 0.3):
    """n + 1 flattened request-level EAMs [n + 1][L * E] int32 (the last row a
    query).  Every group has, per layer, expert preferences ~ Dirichlet(alpha)
    (small alpha: few experts take most tokens); a request picks a group and a
    token count uniform in [1, max_tokens], and each layer's k * tokens choices
    are drawn multinomially from the group's preferences."""
    r = rng(seed_of(cfg, 0, 0, T_EAM))
    pref = r.dirichlet(np.full(E, alpha), size=(groups, L))
    g = r.integers(0, groups, size=n + 1)
    tok = r.integers(1, max_tokens + 1, size=n + 1)
    out = np.empty((n + 1, L, E), dtype=np.int32)
    for i in range(n + 1):
        for l in range(L):
            out[i, l] = r.multinomial(int(tok[i]) * k, pref[g[i], l])
    return out.reshape(n + 1, L * E)


def hidden_stream_f32(cfg: int, L: int, T: int, d: int, scale: float = 1.0 / 64, mix: float = 0.2):
    """Per-layer hidden states [L][T][d] with consecutive-layer cosine ~0.98:
    x_0 ~ N(0,1)*scale, x_{l+1} = unit(x_l + mix * n_l), n_l ~ N(0,1)*scale.

    FloE observes cosine similarity above 0.95 between the hidden states of
    consecutive MoE layers (FloE review page, "双稀疏预测器", observation 3)."""
    out = np.empty((L, T, d), dtype=np.float32)
    x = normal_f32(seed_of(cfg, 0, 0, T_X), (T, d), scale).astype(np.float64)
    for l in range(L):
        out[l] = x.astype(np.float32)
        n = normal_f32(seed_of(cfg, l, 0, T_NOISE), (T, d), scale).astype(np.float64)
        x = x + mix * n
        x /= np.linalg.norm(x, axis=1, keepdims=True)
    return out


# ---------------------------------------------------------------------------
# Device-side draws (large configurations).  torch is used as a random-number
# source only; nothing of the method is computed here.
# ---------------------------------------------------------------------------

def device_normal(seed: int, shape, std: float, device, dtype=None):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    a = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        a.mul_(std)
    if dtype is not None:
        a = a.to(dtype)
    return a
