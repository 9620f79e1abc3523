"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds none of the method's arithmetic: only random draws, the
rounding of those draws to bf16 (that *is* the input format), and the shape
tables of the workloads.  It imports neither the oracle nor the GPU library.

Recipe: every (workload, layer, matrix, role) gets its own seed, derived with
numpy's SeedSequence from the workload seed; values are drawn as fp32 standard
normals by torch's generator on the target device, scaled by the standard
deviation and rounded to bf16 (round to nearest even).  Weights use std 0.02,
activations std 1.  Draws on the CPU and on the GPU come from different
generators, so a test that compares the two sides always copies the device
tensor to the host rather than redrawing it.
"""
import numpy as np
import torch

W_STD = 0.02
X_STD = 1.0

ROLE_W = 0
ROLE_X = 1

# Matrix order inside one decoder layer (rows N = outputs, K = inputs).
LAYER_MATS = ("q", "k", "v", "o", "gate", "up", "down")


def _layer(d, kv, ff):
    return [("q", d, d), ("k", kv, d), ("v", kv, d), ("o", d, d),
            ("gate", ff, d), ("up", ff, d), ("down", d, ff)]


# TinyLlama-1.1B: hidden 2048, 4 KV heads x 64 = 256, MLP 5632, vocab 32000, 22 layers.
TINYLLAMA = dict(name="tinyllama-1.1b", seed=1002, layers=22,
                 layer=_layer(2048, 256, 5632), head=("head", 32000, 2048))
# Qwen2.5-7B: hidden 3584, 4 KV heads x 128 = 512, MLP 18944, vocab 152064, 28 layers.
QWEN7B = dict(name="qwen2.5-7b", seed=1003, layers=28,
              layer=_layer(3584, 512, 18944), head=("head", 152064, 3584))
# Mistral-7B projection shapes for the batched (skinny) product.
MISTRAL_SHAPES = [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336), (32000, 4096)]
MISTRAL_M = (8, 64, 256)
MISTRAL_SEED = 1005
SINGLE_SEED = 1001
SINGLE_SHAPE = (2048, 2048)


def decode_matrices(model):
    """[(layer, mat_idx, name, N, K)] for one decode step, in model order; the
    output head is layer == model['layers'], mat_idx 0."""
    out = []
    for layer in range(model["layers"]):
        for i, (name, n, k) in enumerate(model["layer"]):
            out.append((layer, i, name, n, k))
    name, n, k = model["head"]
    out.append((model["layers"], 0, name, n, k))
    return out


def decode_groups(model, fused=True):
    """Launch groups of one decode step, in model order: [(layer, [(mat_idx, name,
    N, K), ...])].  Fused: matrices that read the same input are concatenated
    along N at load time (q|k|v and gate|up), as an engine does to cut launches;
    unfused: one group per matrix."""
    groups = []
    for layer in range(model["layers"]):
        mats = [(i, name, n, k) for i, (name, n, k) in enumerate(model["layer"])]
        if fused:
            by = {m[1]: m for m in mats}
            for names in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
                groups.append((layer, [by[nm] for nm in names]))
        else:
            groups += [(layer, [m]) for m in mats]
    name, n, k = model["head"]
    groups.append((model["layers"], [(0, name, n, k)]))
    return groups


def seed_for(cfg_seed, layer, mat_idx, role):
    """A 63-bit seed unique to (workload, layer, matrix, role)."""
    ss = np.random.SeedSequence([int(cfg_seed), int(layer), int(mat_idx), int(role)])
    return int(ss.generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1)


def normal_bf16(shape, std, seed, device="cpu"):
    """bf16 tensor of N(0, std^2) draws, seeded; drawn in fp32, rounded once."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & ((1 << 63) - 1))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def weight(cfg_seed, layer, mat_idx, n, k, device="cpu"):
    return normal_bf16((n, k), W_STD, seed_for(cfg_seed, layer, mat_idx, ROLE_W), device)


def activation(cfg_seed, layer, mat_idx, m, k, device="cpu"):
    return normal_bf16((m, k), X_STD, seed_for(cfg_seed, layer, mat_idx, ROLE_X), device)


def bits(t):
    """Raw bit patterns of a bf16/fp16 tensor as a host numpy uint16 array."""
    if t.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("expected a 16-bit float tensor")
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def from_bits(a, dtype=torch.bfloat16, device="cpu"):
    """Tensor of the given 16-bit float dtype holding the uint16 bit patterns a."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(dtype).to(device)


def outlier_weight(seed, n, k, lo=30.0, hi=50.0, shared=False, group=64):
    """bf16 [n, k] weights dominated by one outlier per group of `group`
    consecutive k: N(0, W_STD^2) draws, with one entry per group replaced by
    +-U(lo, hi) * W_STD.  Quantised with one scale per group, such a group has
    a single code of magnitude 7 and almost every other code 0.  shared: the
    outlier sits at the same position of a group in every row.  Returns the
    tensor (CPU) and the outlier positions, an int64 [n, k / group] array of k
    indices."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) & ((1 << 63) - 1))
    t = torch.randn((n, k), generator=g, dtype=torch.float32) * W_STD
    G = k // group
    rows = 1 if shared else n
    pos = torch.randint(0, group, (rows, G), generator=g) + torch.arange(G) * group
    mag = (torch.rand((rows, G), generator=g) * (hi - lo) + lo) * W_STD
    sign = torch.where(torch.rand((rows, G), generator=g) < 0.5, -1.0, 1.0)
    pos, val = pos.expand(n, G), (mag * sign).expand(n, G)
    t.scatter_(1, pos, val)
    return t.to(torch.bfloat16), pos.numpy().astype(np.int64)
