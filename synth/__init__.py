"""Seeded synthetic inputs shaped like the pages' workloads.

Shared by the tests (for both the oracle and the HIP library) and by the
bench.  This module holds no codec arithmetic: it only draws random numbers
and casts float32 to bf16 through torch's CPU cast.

Recipes (shape, distribution, seed):
  weight_block  N(0, 0.02^2) with round(0.001 N) elements x50 (outliers);
                stand-in for the weight blocks of "weight precision part 2"
                and fp4-train; 256 x 2048 at seed 1.
  moe_dispatch  Student-t(4) * 0.5 with 8 hidden channels x30; stand-in for
                the MoE dispatch activation (hidden 7168); 4096 x 7168 at seed 2.
  tp_tensor     N(0,1) with 1% of columns x20; stand-in for the tensor-parallel
                communication tensor (2 x 4096 tokens x 4096); seed 3.
  ef_weight / ef_update
                W0 ~ N(0, 0.02^2) bf16 and per-step updates fl32(1e-4 * g),
                g ~ N(0,1) fp32; 8192 x 8192 at seed 4.
  expert_counts Multinomial(T, p_k ~ k^-1.1, k = 1..E) token counts in expert
                order and their exclusive prefix sum; 65536 tokens, 256
                experts, seed 5.
  expert_activations  N(0,1) activations [T, H] (bf16), seed 5.
  random_mxfp4  uniformly random E2M1 code bytes and UE8M0 scale bytes in a
                chosen band: raw MXFP4 rows with no quantizer involved.
"""
import numpy as np
import torch


def to_bf16_bits(x32):
    """float32 numpy -> bf16 bit patterns (uint16) via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def weight_block(rows=256, cols=2048, seed=1):
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, 0.02, size=(rows, cols)).astype(np.float32)
    n_out = int(round(0.001 * rows * cols))
    idx = rng.choice(rows * cols, size=n_out, replace=False)
    x.reshape(-1)[idx] *= np.float32(50.0)
    return to_bf16_bits(x)


def moe_dispatch(rows=4096, cols=7168, seed=2, n_hot=8):
    rng = np.random.default_rng(seed)
    x = (rng.standard_t(4.0, size=(rows, cols)) * 0.5).astype(np.float32)
    hot = rng.choice(cols, size=min(n_hot, cols), replace=False)
    x[:, hot] *= np.float32(30.0)
    return to_bf16_bits(x)


def tp_tensor(rows=8192, cols=4096, seed=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=(rows, cols), dtype=np.float32)
    hot = rng.choice(cols, size=int(round(0.01 * cols)), replace=False)
    x[:, hot] *= np.float32(20.0)
    return to_bf16_bits(x)


def ef_weight(rows=8192, cols=8192, seed=4):
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.normal(0.0, 0.02, size=(rows, cols)).astype(np.float32))


def ef_update(rows=8192, cols=8192, seed=4, step=0, lr=1e-4):
    """u_t = fl32(lr * g_t), g_t ~ N(0,1) fp32, one independent stream per step."""
    rng = np.random.default_rng([seed, 1000 + step])
    g = rng.standard_normal(size=(rows, cols), dtype=np.float32)
    return (np.float32(lr) * g).astype(np.float32)


def expert_counts(tokens=65536, experts=256, seed=5, s=1.1):
    rng = np.random.default_rng(seed)
    p = np.arange(1, experts + 1, dtype=np.float64) ** (-s)
    counts = rng.multinomial(tokens, p / p.sum())
    offsets = np.zeros(experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return counts.astype(np.int64), offsets


def expert_activations(tokens=65536, hidden=7168, seed=5):
    rng = np.random.default_rng([seed, 1])
    return to_bf16_bits(rng.standard_normal(size=(tokens, hidden), dtype=np.float32))


def random_mxfp4(tokens, hidden, seed=5, scale_lo=118, scale_hi=130):
    """Random packed E2M1 bytes [T, H/2] and UE8M0 bytes [T, H/32] with
    scale bytes uniform in [scale_lo, scale_hi]."""
    rng = np.random.default_rng([seed, 2])
    packed = rng.integers(0, 256, size=(tokens, hidden // 2), dtype=np.uint8)
    sb = rng.integers(scale_lo, scale_hi + 1, size=(tokens, hidden // 32), dtype=np.uint8)
    return packed, sb
