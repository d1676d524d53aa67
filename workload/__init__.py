"""Seeded synthetic inputs for the weight-delta codec.

This module is shared by the HIP path's tests/bench and by the oracle side, so
it holds none of the codec's arithmetic: no cast, no compare, no compaction, no
encoding.  It only draws FP32 "master weights" and applies a synthetic trainer
step to them, standing in for the optimizer (which is not part of the codec).

Workloads (model shapes and learning rate):
  c1  one 4096x1024 FP32 tensor, numpy default_rng(0); w ~ N(0, 0.02); one step
  c2  Qwen2.5-32B-shaped set: 64 layers, hidden 5120, 40 q / 8 kv heads x 128,
      MLP 27648, vocab 152064, untied embeddings, q/k/v biases
  c3  Llama-3-8B-shaped set: 32 layers, hidden 4096, 32 / 8 heads x 128,
      MLP 14336, vocab 128256, untied embeddings; 20 chained steps
  c4  the first 16e9 elements of c2's tensor order (XOR-mask path)
  c5  Kimi-K2-shaped MoE layer share: 384 experts x {gate, up [2048, 7168],
      down [7168, 2048]} plus q, k, v [8192, 7168]
  6   trainer-to-trainer rounds on a Qwen2.5-7B-shaped set: FP32 checkpoint
      drawn like the others, and per round a pseudo-gradient, the sum of H
      synthetic local steps -lr * clip(u, -3, 3)
The step is w' = fl32(w - fl32(lr * clip(u, -3, 3))), u ~ N(0, 1) per step,
lr = 3e-6 (the RL learning rate the PULSE technical summary quotes, section
"Osservazione Centrale").  Matrices and biases start N(0, 0.02); norm weights
start N(1, 0.01).  Device tensors use one torch generator per (workload,
tensor, step) with seed (workload << 40) | (tensor << 20) | step, step 0 being
the initial weights.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

LR = 3e-6
INIT_STD = 0.02
NORM_MEAN, NORM_STD = 1.0, 0.01


@dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: tuple
    kind: str  # "matrix" | "bias" | "norm"

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n


def _decoder_specs(layers, hidden, n_q, n_kv, head, mlp, vocab, qkv_bias):
    specs = [TensorSpec("embed", (vocab, hidden), "matrix")]
    for l in range(layers):
        p = f"l{l}."
        specs.append(TensorSpec(p + "in_ln", (hidden,), "norm"))
        specs.append(TensorSpec(p + "q", (n_q * head, hidden), "matrix"))
        specs.append(TensorSpec(p + "k", (n_kv * head, hidden), "matrix"))
        specs.append(TensorSpec(p + "v", (n_kv * head, hidden), "matrix"))
        if qkv_bias:
            specs.append(TensorSpec(p + "q_b", (n_q * head,), "bias"))
            specs.append(TensorSpec(p + "k_b", (n_kv * head,), "bias"))
            specs.append(TensorSpec(p + "v_b", (n_kv * head,), "bias"))
        specs.append(TensorSpec(p + "o", (hidden, n_q * head), "matrix"))
        specs.append(TensorSpec(p + "post_ln", (hidden,), "norm"))
        specs.append(TensorSpec(p + "gate", (mlp, hidden), "matrix"))
        specs.append(TensorSpec(p + "up", (mlp, hidden), "matrix"))
        specs.append(TensorSpec(p + "down", (hidden, mlp), "matrix"))
    specs.append(TensorSpec("norm", (hidden,), "norm"))
    specs.append(TensorSpec("lm_head", (vocab, hidden), "matrix"))
    return specs


def qwen25_32b_specs(layers=64):
    return _decoder_specs(layers, 5120, 40, 8, 128, 27648, 152064, True)


def llama3_8b_specs(layers=32):
    return _decoder_specs(layers, 4096, 32, 8, 128, 14336, 128256, False)


def qwen25_7b_specs(layers=28):
    """Qwen2.5-7B shape (one of the models the pages' PULSELoCo runs use): hidden
    3584, 28 q / 4 kv heads x 128, MLP 18944, vocab 152064, q/k/v biases."""
    return _decoder_specs(layers, 3584, 28, 4, 128, 18944, 152064, True)


def kimi_k2_layer_specs(experts=384):
    specs = []
    for e in range(experts):
        specs.append(TensorSpec(f"e{e}.gate", (2048, 7168), "matrix"))
        specs.append(TensorSpec(f"e{e}.up", (2048, 7168), "matrix"))
        specs.append(TensorSpec(f"e{e}.down", (7168, 2048), "matrix"))
    for nm in ("q", "k", "v"):
        specs.append(TensorSpec(nm, (64 * 128, 7168), "matrix"))
    return specs


C4_NUMEL = 16_000_000_000


def total_numel(specs) -> int:
    return sum(s.numel for s in specs)


def seed_of(workload: int, tensor: int, step: int) -> int:
    return (workload << 40) | (tensor << 20) | step


# --------------------------------------------------------------------------
# c1: numpy, fully on the host
# --------------------------------------------------------------------------
def c1_masters(rows=4096, cols=1024, seed=0):
    """(w0, w1) float32 [rows, cols]: w0 ~ N(0, 0.02); w1 = w0 - lr * clip(u)."""
    rng = np.random.default_rng(seed)
    n = rows * cols
    w0 = rng.standard_normal(n, dtype=np.float32) * np.float32(INIT_STD)
    u = np.clip(rng.standard_normal(n, dtype=np.float32), np.float32(-3), np.float32(3))
    w1 = w0 - np.float32(LR) * u
    return w0.reshape(rows, cols), w1.reshape(rows, cols)


def host_masters(n, seed, kind="matrix", steps=1, lr=LR):
    """Host-side (numpy) stand-in of the device generator for CPU-only tests:
    returns [w0, w1, ..., w_steps] float32 arrays of n elements."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(n, dtype=np.float32)
    if kind == "norm":
        w = np.float32(NORM_MEAN) + np.float32(NORM_STD) * z
    else:
        w = np.float32(INIT_STD) * z
    out = [w]
    for _ in range(steps):
        u = np.clip(rng.standard_normal(n, dtype=np.float32), np.float32(-3), np.float32(3))
        w = w - np.float32(lr) * u
        out.append(w)
    return out


# --------------------------------------------------------------------------
# device generation (torch) for the large workloads
# --------------------------------------------------------------------------
def fill_init(out, workload: int, tensor: int, kind: str):
    """Write the initial FP32 weights of one tensor into `out` (a float32 torch
    tensor, any device)."""
    import torch

    g = torch.Generator(device=out.device)
    g.manual_seed(seed_of(workload, tensor, 0))
    torch.randn(out.shape, generator=g, device=out.device, dtype=torch.float32, out=out)
    if kind == "norm":
        out.mul_(NORM_STD).add_(NORM_MEAN)
    else:
        out.mul_(INIT_STD)
    return out


def apply_step(w, workload: int, tensor: int, step: int, lr: float = LR, tmp=None):
    """In place: w <- fl32(w - fl32(lr * clip(u, -3, 3))), u drawn for `step`.
    `tmp` (float32, >= w.numel()) avoids an allocation when given."""
    import torch

    g = torch.Generator(device=w.device)
    g.manual_seed(seed_of(workload, tensor, step))
    if tmp is None:
        u = torch.empty(w.shape, device=w.device, dtype=torch.float32)
    else:
        u = tmp.view(-1)[: w.numel()].view(w.shape)
    torch.randn(w.shape, generator=g, device=w.device, dtype=torch.float32, out=u)
    u.clamp_(-3.0, 3.0).mul_(lr)
    w.sub_(u)
    return w


def pseudo_gradient(out, workload: int, tensor: int, rnd: int, local_steps: int = 8, lr: float = LR,
                    tmp=None):
    """Write into `out` (float32 torch tensor) the synthetic pseudo-gradient of
    round `rnd` >= 1: the sum, in float32 and in order, of `local_steps` updates
    -lr * clip(u, -3, 3), u ~ N(0, 1) drawn with step numbers
    (rnd - 1) * local_steps + 1 ... rnd * local_steps."""
    import torch

    out.zero_()
    for h in range(local_steps):
        g = torch.Generator(device=out.device)
        g.manual_seed(seed_of(workload, tensor, (rnd - 1) * local_steps + h + 1))
        u = torch.empty(out.shape, device=out.device, dtype=torch.float32) if tmp is None else \
            tmp.view(-1)[: out.numel()].view(out.shape)
        torch.randn(out.shape, generator=g, device=out.device, dtype=torch.float32, out=u)
        u.clamp_(-3.0, 3.0).mul_(lr)
        out.sub_(u)
    return out

