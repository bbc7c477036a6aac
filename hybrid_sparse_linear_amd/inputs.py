"""Seeded synthetic inputs for the SALA layer group.

This module only draws random tensors; it holds none of the attention
arithmetic.  Both the HIP path (tests, bench) and the float64 oracle (via the
tests) consume exactly the tensors produced here, so they see identical bits.

Recipe (every draw is fp32 from ``torch.randn`` with a seeded
``torch.Generator`` on the requested device, scaled in fp32, then rounded
once to the target dtype with round-to-nearest-even):

  seed = 1000 * workload + 100 * layer + tensor id
         tensor ids: q 0, k 1, v 2, shift direction 3, shifted-block set 4, state 5,
                     gamma_q 6, gamma_k 7, gate 8

  workload 1  tiny group, fp32, B=1, H=4, d=64, N=2048, q/k/v ~ N(0,1)/8.
              Linear decay per head [1.0, 0.99, 1.0, 0.99], chunk 64.
              Sparse layer: Hq = Hkv = 4, block 64, top-k 4 + 1 initial + 2 local.
  workload 2  linear prefill, bf16, B=1, H=32, d=128, N=32768, chunk 128,
              q/k/v ~ N(0,1)/sqrt(128), lam_h = exp(-2**(-(h+1)/4)).
  workload 3  sparse prefill, bf16, B=1, Hq=32, Hkv=2, d=128, N=131072, block 64,
              top-k 64 + 1 + 2.  q, k, v ~ N(0,1); floor(5% of the key blocks)
              (drawn without replacement, shared by every batch row and KV head)
              get +2.0 * u added to every key, u a seeded unit vector.
  workload 4  the 3:1 group at N=262144: three linear layers shaped as workload 2
              (layers 0, 1, 2) and one sparse layer shaped as workload 3 (layer 3).
  workload 5  decode at a 1,048,576-token context, bf16, B=4: linear q/k/v [4,32,128]
              ~ N(0,1)/sqrt(128), fp32 state ~ N(0,1)/128, lam as workload 2;
              sparse q [4,32,128] ~ N(0,1), K/V cache [4,2,1048576,128] ~ N(0,1).

Small test cases generate on the CPU and copy to the GPU; full-size cases
generate on the GPU (``device='cuda'``) and copy back only what the oracle
needs.  The CPU and GPU generators give different streams for one seed, so a
case is always generated on exactly one device.
"""

import math

import torch

F32 = torch.float32
BF16 = torch.bfloat16


def seed_of(workload, layer, tensor_id):
    return 1000 * workload + 100 * layer + tensor_id


def normal(shape, seed, std=1.0, dtype=F32, device="cpu"):
    """fp32 N(0, 1) draws scaled by std in fp32, rounded once to dtype."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=F32)
    if std != 1.0:
        x.mul_(float(std))
    return x if dtype == F32 else x.to(dtype)


def slope_decay(h):
    """Per-head decay lam_h = exp(-2**(-(i+1)/4)), i = 0..h-1, as fp32."""
    return torch.tensor([math.exp(-2.0 ** (-(i + 1) / 4.0)) for i in range(h)], dtype=F32)


def alternating_decay(h, values=(1.0, 0.99)):
    """Per-head decay cycling through ``values`` (head 0 -> values[0], ...)."""
    return torch.tensor([values[i % len(values)] for i in range(h)], dtype=F32)


def linear_inputs(B, H, N, d, dtype, workload, layer, std, device="cpu", decay=None):
    """q, k, v [B, H, N, d] for one linear-attention layer."""
    q = normal((B, H, N, d), seed_of(workload, layer, 0), std, dtype, device)
    k = normal((B, H, N, d), seed_of(workload, layer, 1), std, dtype, device)
    v = normal((B, H, N, d), seed_of(workload, layer, 2), std, dtype, device)
    return {"q": q, "k": k, "v": v, "decay": decay}


def neighbour_inputs(B, H, N, d, workload, layer, device="cpu"):
    """The linear layer's neighbour tensors: RMS-norm weights gamma_q, gamma_k [d]
    (fp32, 1/sqrt(d) * (1 + 0.25 z), so normalised rows keep the workloads' input
    scale) and a gate pre-activation [B, H, N, d] ~ N(0, 1) in bf16."""
    gq = normal((d,), seed_of(workload, layer, 6), 0.25, F32, device).add_(1.0).mul_(1.0 / math.sqrt(d))
    gk = normal((d,), seed_of(workload, layer, 7), 0.25, F32, device).add_(1.0).mul_(1.0 / math.sqrt(d))
    gate = normal((B, H, N, d), seed_of(workload, layer, 8), 1.0, BF16, device)
    return {"gamma_q": gq, "gamma_k": gk, "gate": gate}


def sparse_inputs(B, Hq, Hkv, N, d, dtype, workload, layer, std=1.0, device="cpu",
                  shift_frac=0.0, shift=2.0, block=64):
    """q [B, Hq, N, d], k/v [B, Hkv, N, d] for one sparse layer.

    With shift_frac > 0, floor(shift_frac * n_complete_blocks) key blocks get
    ``shift * u`` added (fp32, before rounding), u a seeded unit vector.
    """
    q = normal((B, Hq, N, d), seed_of(workload, layer, 0), std, dtype, device)
    k = normal((B, Hkv, N, d), seed_of(workload, layer, 1), std, F32, device)
    v = normal((B, Hkv, N, d), seed_of(workload, layer, 2), std, dtype, device)
    shifted = torch.empty(0, dtype=torch.int64)
    if shift_frac > 0.0:
        n_full = N // block
        n_shift = int(math.floor(shift_frac * n_full))
        gd = torch.Generator().manual_seed(seed_of(workload, layer, 3))
        u = torch.randn(d, generator=gd, dtype=torch.float64)
        u = (u / u.norm()).to(F32)
        gs = torch.Generator().manual_seed(seed_of(workload, layer, 4))
        shifted = torch.randperm(n_full, generator=gs)[:n_shift].sort().values
        su = (shift * u).to(k.device)
        for j in shifted.tolist():
            k[:, :, j * block:(j + 1) * block] += su
    k = k if dtype == F32 else k.to(dtype)
    return {"q": q, "k": k, "v": v, "shifted_blocks": shifted}


# ---------------------------------------------------------------- named workloads

def workload1_linear(layer, device="cpu"):
    return linear_inputs(1, 4, 2048, 64, F32, 1, layer, 1.0 / 8.0, device, alternating_decay(4))


def workload1_sparse(device="cpu"):
    return sparse_inputs(1, 4, 4, 2048, 64, F32, 1, 3, 1.0 / 8.0, device)


def workload2_linear(layer=0, device="cpu", N=32768, workload=2):
    return linear_inputs(1, 32, N, 128, BF16, workload, layer, 1.0 / math.sqrt(128.0), device,
                         slope_decay(32))


def workload3_sparse(layer=0, device="cpu", N=131072, workload=3):
    return sparse_inputs(1, 32, 2, N, 128, BF16, workload, layer, 1.0, device, shift_frac=0.05)


def workload4_group(device="cuda", N=262144):
    """Three linear layers (layers 0..2) and one sparse layer (layer 3) at N tokens."""
    lin = [workload2_linear(layer, device, N, workload=4) for layer in range(3)]
    sp = workload3_sparse(3, device, N, workload=4)
    return lin, sp


def workload5_decode(device="cuda", B=4, L=1048576, H=32, Hkv=2, d=128):
    """Decode step inputs: three linear layers (0..2) and one sparse layer (3)."""
    lin = []
    for layer in range(3):
        x = linear_inputs(B, H, 1, d, BF16, 5, layer, 1.0 / math.sqrt(d), device, slope_decay(H))
        x = {kk: (vv[:, :, 0] if kk in ("q", "k", "v") else vv) for kk, vv in x.items()}
        x["state"] = normal((B, H, d, d), seed_of(5, layer, 5), 1.0 / d, F32, device)
        lin.append(x)
    q = normal((B, H, d), seed_of(5, 3, 0), 1.0, BF16, device)
    kc = normal((B, Hkv, L, d), seed_of(5, 3, 1), 1.0, BF16, device)
    vc = normal((B, Hkv, L, d), seed_of(5, 3, 2), 1.0, BF16, device)
    return lin, {"q": q, "k_cache": kc, "v_cache": vc, "L": L}


def to_f64(t):
    """Widen a tensor's exact values to a float64 NumPy array on the host (for the oracle)."""
    return t.detach().to("cpu", torch.float64).numpy()
