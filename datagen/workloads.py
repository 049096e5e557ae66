"""The synthetic workloads: shapes, seeds and the keyed slices of every tensor.

Shapes follow the Ling-3.0-flash model table ("Ling-3.0-flash on 4 Blackwell
GPUs", section "The model"): hidden 2560, 512 routed experts + 1 shared,
top-8, expert intermediate 768, vocabulary about 157k (157184 here), with the
tensor-parallel shard taking a quarter of the intermediate size.  All weights
are ~N(0, 0.02^2) and inputs ~N(0, 1) (Irwin-Hall(12) approximation, see
dg_core.h).  Nothing here computes any part of the MoE layer.
"""
from dataclasses import dataclass

from . import (FAMILY_LING, FAMILY_TINY, FP8_BLOCK, FP8_MUL, SIGMA_W, SIGMA_X, TENSOR_BIAS,
               TENSOR_DOWN, TENSOR_DOWN_FP8, TENSOR_GAIN, TENSOR_GATE_UP, TENSOR_GATE_UP_FP8,
               TENSOR_LMHEAD, TENSOR_ROUTER, TENSOR_SCALE_D, TENSOR_SCALE_GU, TENSOR_X, fill_host,
               fill_host_fp8, fill_scales, key, round_bf16_bits)

WEIGHT_SEED = 0x5EED0001


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    family: int
    H: int
    E: int
    K: int
    I: int          # intermediate size of this call (the shard's share under TP)
    S: int          # shared experts (0 or 1)
    M: int          # token rows
    x_seed: int
    n_layers: int = 1
    V: int = 0      # lm_head vocabulary (0 = no lm_head)
    n_shards: int = 1
    shard: int = 0
    out_f32: bool = False
    residual: bool = False
    prenorm: bool = False   # each layer's MoE sees bf16(RMSNorm(h_l) * gain)
    bias_sigma: float = 0.0     # router selection bias ~N(0, bias_sigma^2) per expert (0: none)
    gain_sigma: float = 0.0     # norm gain ~1 + N(0, gain_sigma^2) per channel (0: unit gain)
    routed_scale: float = 1.0   # routed scaling factor of the combine
    fp8: bool = False           # expert weights as fp8 e4m3 codes with 128x128 block scales

    @property
    def I_full(self):
        return self.I * self.n_shards

    def expert_bytes(self):
        """HBM bytes of one expert (weights, plus block scales for fp8)."""
        if self.fp8:
            nb = (2 * self.I // FP8_BLOCK) * (self.H // FP8_BLOCK) + \
                (self.H // FP8_BLOCK) * (self.I // FP8_BLOCK)
            return 3 * self.H * self.I + 4 * nb
        return 3 * self.H * self.I * 2

    def router_bytes(self):
        return self.E * self.H * 2

    def layer_bytes(self):
        return self.router_bytes() + (self.E + self.S) * self.expert_bytes()

    def front_bytes(self):
        """Bytes of the router front's small vectors: fp32 bias [E], bf16 gain [H]."""
        return (4 * self.E if self.bias_sigma else 0) + (2 * self.H if self.gain_sigma else 0)


C1 = Workload("tiny_moe_layer_m1", 1, FAMILY_TINY, H=256, E=16, K=2, I=64, S=1, M=1, x_seed=101)
C2 = Workload("ling_moe_layer_m1", 2, FAMILY_LING, H=2560, E=512, K=8, I=768, S=1, M=1,
              x_seed=202)
C3 = Workload("ling_moe_layer_m6", 3, FAMILY_LING, H=2560, E=512, K=8, I=768, S=1, M=6,
              x_seed=303)
C4 = Workload("ling_tp4_shard_moe_layer_m6", 4, FAMILY_LING, H=2560, E=512, K=8, I=192, S=1,
              M=6, x_seed=404, n_shards=4, shard=0, out_f32=True)
C5 = Workload("ling_chain16_lmhead_m6", 5, FAMILY_LING, H=2560, E=512, K=8, I=768, S=1, M=6,
              x_seed=505, n_layers=16, V=157184, residual=True, prenorm=True)

# The router front on a single layer: RMSNorm with a gain vector, a per-expert
# selection bias and a routed scaling factor (2.5: not a power of two, so the
# scaling is a real rounding step).  Bias sigma 0.25 moves about a third of the
# selections at E = 512 (the logits have std ~1 and the K-th gap ~0.05).
C6 = Workload("tiny_moe_layer_front_m3", 6, FAMILY_TINY, H=256, E=16, K=2, I=64, S=1, M=3,
              x_seed=606, prenorm=True, bias_sigma=0.25, gain_sigma=0.1, routed_scale=2.5)
C7 = Workload("ling_moe_layer_front_m6", 7, FAMILY_LING, H=2560, E=512, K=8, I=768, S=1, M=6,
              x_seed=707, prenorm=True, bias_sigma=0.25, gain_sigma=0.1, routed_scale=2.5)

# fp8 e4m3 expert weights with 128x128 block scales (the router stays bf16).  The
# block-128 format needs I % 128 == 0, so there is no TP4 shard of I = 768.
C8 = Workload("tiny_fp8_moe_layer_m3", 8, FAMILY_TINY, H=256, E=16, K=2, I=128, S=1, M=3,
              x_seed=808, fp8=True)
C9 = Workload("ling_fp8_moe_layer_m1", 9, FAMILY_LING, H=2560, E=512, K=8, I=768, S=1, M=1,
              x_seed=909, fp8=True)
C10 = Workload("ling_fp8_moe_layer_m6", 10, FAMILY_LING, H=2560, E=512, K=8, I=768, S=1, M=6,
               x_seed=1010, fp8=True)
# A 16-token verify ("Muse Spark Open Ultrafast", "Speculative decoding": the
# target checks 16 tokens per step), bf16 and fp8 experts.
C12 = Workload("ling_moe_layer_m16", 12, FAMILY_LING, H=2560, E=512, K=8, I=768, S=1, M=16,
               x_seed=1313)
C13 = Workload("ling_fp8_moe_layer_m16", 13, FAMILY_LING, H=2560, E=512, K=8, I=768, S=1, M=16,
               x_seed=1414, fp8=True)
C11 = Workload("ling_fp8_chain16_lmhead_m6", 11, FAMILY_LING, H=2560, E=512, K=8, I=768, S=1,
               M=6, x_seed=1111, n_layers=16, V=157184, residual=True, prenorm=True, fp8=True)

ALL = (C1, C2, C3, C4, C5)
FRONT = (C6, C7)
FP8 = (C8, C9, C10, C11)
WIDE = (C12, C13)


# ---- host slices ------------------------------------------------------------

def x_row(wl, m, attempt=0):
    k = key(wl.x_seed, wl.family, wl.cfg_id, TENSOR_X, m, attempt)
    return fill_host(k, 1, wl.H, SIGMA_X)[0]


def x_rows(wl, attempts):
    import numpy as np
    return np.stack([x_row(wl, m, a) for m, a in enumerate(attempts)])


def router(wl, layer=0):
    k = key(WEIGHT_SEED, wl.family, layer, TENSOR_ROUTER)
    return fill_host(k, wl.E, wl.H, SIGMA_W)


def expert_gate_up(wl, layer, e):
    """[2I][H]: this shard's gate rows, then its up rows, of the full [2*I_full][H] tensor."""
    import numpy as np
    k = key(WEIGHT_SEED, wl.family, layer, TENSOR_GATE_UP, e)
    g = fill_host(k, wl.I, wl.H, SIGMA_W, row0=wl.shard * wl.I, ld_full=wl.H)
    u = fill_host(k, wl.I, wl.H, SIGMA_W, row0=wl.I_full + wl.shard * wl.I, ld_full=wl.H)
    return np.concatenate([g, u], axis=0)


def expert_down(wl, layer, e):
    """[H][I]: this shard's columns of the full [H][I_full] tensor."""
    k = key(WEIGHT_SEED, wl.family, layer, TENSOR_DOWN, e)
    return fill_host(k, wl.H, wl.I, SIGMA_W, col0=wl.shard * wl.I, ld_full=wl.I_full)


def expert_gate_up_scales(wl, layer, e):
    ks = key(WEIGHT_SEED, wl.family, layer, TENSOR_SCALE_GU, e)
    return fill_scales(ks, (2 * wl.I // FP8_BLOCK, wl.H // FP8_BLOCK), SIGMA_W / FP8_MUL)


def expert_down_scales(wl, layer, e):
    ks = key(WEIGHT_SEED, wl.family, layer, TENSOR_SCALE_D, e)
    return fill_scales(ks, (wl.H // FP8_BLOCK, wl.I // FP8_BLOCK), SIGMA_W / FP8_MUL)


def expert_gate_up_fp8(wl, layer, e):
    """(codes uint8 [2I][H], block scales fp32 [2I/128][H/128]) of one expert."""
    k = key(WEIGHT_SEED, wl.family, layer, TENSOR_GATE_UP_FP8, e)
    return fill_host_fp8(k, 2 * wl.I, wl.H), expert_gate_up_scales(wl, layer, e)


def expert_down_fp8(wl, layer, e):
    """(codes uint8 [H][I], block scales fp32 [H/128][I/128]) of one expert."""
    k = key(WEIGHT_SEED, wl.family, layer, TENSOR_DOWN_FP8, e)
    return fill_host_fp8(k, wl.H, wl.I), expert_down_scales(wl, layer, e)


def router_bias(wl, layer=0):
    """fp32 [E] selection bias (bf16-representable values), or None."""
    if not wl.bias_sigma:
        return None
    import numpy as np
    k = key(WEIGHT_SEED, wl.family, layer, TENSOR_BIAS)
    b = fill_host(k, 1, wl.E, wl.bias_sigma)[0]
    return (b.astype(np.uint32) << 16).view(np.float32)


def norm_gain(wl, layer=0):
    """bf16 bits [H] of 1 + N(0, gain_sigma^2), or None (unit gain)."""
    if not wl.gain_sigma:
        return None
    import numpy as np
    k = key(WEIGHT_SEED, wl.family, layer, TENSOR_GAIN)
    v = (fill_host(k, 1, wl.H, wl.gain_sigma)[0].astype(np.uint32) << 16).view(np.float32)
    return round_bf16_bits(v + np.float32(1.0))


def lmhead(wl):
    k = key(WEIGHT_SEED, wl.family, 0, TENSOR_LMHEAD)
    return fill_host(k, wl.V, wl.H, SIGMA_W)


def lmhead_rows(wl, v0, n):
    k = key(WEIGHT_SEED, wl.family, 0, TENSOR_LMHEAD)
    return fill_host(k, n, wl.H, SIGMA_W, row0=v0, ld_full=wl.H)


# ---- correlated inputs -------------------------------------------------------
# The rows above are independent, which makes routing ~uniform and unrelated from
# one call to the next: the worst case for bytes and for any guess of the next
# routing.  Real decode is correlated in time and within a batch.  These two
# generators mix a base row with fresh N(0, 1) rows, x = bf16(rho * base +
# sqrt(1 - rho^2) * z), which keeps every row ~N(0, 1); they draw on attempts
# far above any used by x_rows.

_WALK_ATTEMPT = 1 << 20
_BATCH_ATTEMPT = 1 << 21


def _mix(base_bits, z_bits, rho):
    import numpy as np
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)  # noqa: E731
    return round_bf16_bits(np.float32(rho) * f(base_bits)
                           + np.float32(np.sqrt(1.0 - rho * rho)) * f(z_bits))


def x_walk(wl, n_steps, rho, walk=0):
    """[n_steps][H] bf16 bits: a decode-like sequence of single rows whose step s is
    the mix of step s-1 with a fresh row (correlation rho between consecutive steps)."""
    import numpy as np
    base = _WALK_ATTEMPT + walk * 4096
    rows = [x_row(wl, 0, base)]
    for s in range(1, n_steps):
        rows.append(_mix(rows[-1], x_row(wl, 0, base + s), rho))
    return np.stack(rows)


def x_perturbed(wl, M, rho, batch=0):
    """[M][H] bf16 bits: one base row and M perturbed copies of it (correlation rho
    with the base, rho^2 between two rows)."""
    import numpy as np
    base_attempt = _BATCH_ATTEMPT + batch * 64
    base = x_row(wl, 0, base_attempt)
    return np.stack([_mix(base, x_row(wl, m + 1, base_attempt), rho) for m in range(M)])
