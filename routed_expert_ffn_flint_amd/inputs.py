"""Seeded synthetic inputs for the Flint MoE layer.

This module only draws random numbers.  It holds none of the layer's
arithmetic: the GPU path and the CPU oracle both take what it returns as input.

Workloads (sizes from the Flint pages' layer shape: hidden 2048, 256 routed
experts, top-6, expert width 512, shared width 1024; no trained weights exist
here, so every tensor is drawn):

  toy          T=64,    H=256,  E=16,  K=2, I=64,  Is=128,  float32,  seed 0
  decode32     T=32,    H=2048, E=256, K=6, I=512, Is=1024, bf16,     seed 0
  prefill4096  T=4096,  same layer, no router bias,                   seed 0
  skew16384    T=16384, same layer, Zipf(1.1) per-expert router bias, seed 0
  stack47      T=256,   47 distinct layers, RMSNorm between layers,   seed 1
  decode32_mx4 decode32 with every expert matrix stored as MXFP4 (block-scaled
               4-bit, see mx4_quantize, in the tiled order of mx4_tile); router bf16
  dense32      a dense gated MLP layer (the model's first two layers), T=32,
               H=2048, width 6144, bf16, seed 0
  dense4096    the same at T=4096

Weights ~ N(0, 0.02^2), hidden states ~ N(0, 1), drawn in float32 and rounded
to bf16 (round-to-nearest-even, torch's conversion) for the bf16 workloads.

The 4-bit workloads store the drawn expert matrices in the block-scaled 4-bit
format the kernels read (mx4_quantize: a storage encoding of the drawn
values, done once when the weights are made; the layer's arithmetic starts
from the stored codes, which the GPU path and the oracle each decode).

Each tensor has its own generator, seeded from (seed, layer, tensor id), so a
layer can be drawn without drawing the ones before it, and a tensor can be
drawn on the CPU or directly on the GPU (the two devices' generators give
different, equally valid, streams; a test always hands the same drawn values
to both sides).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    bf16: bool
    seed: int
    zipf_bias: bool = False
    layers: int = 1
    mx4: bool = False  # expert matrices stored as MXFP4 (router stays bf16)
    dense: bool = False  # a dense gated MLP layer of width `inter` (no router, no experts)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.bf16 else torch.float32


WORKLOADS = {
    "toy": Workload("toy", 64, 256, 16, 2, 64, 128, False, 0),
    "decode32": Workload("decode32", 32, 2048, 256, 6, 512, 1024, True, 0),
    "prefill4096": Workload("prefill4096", 4096, 2048, 256, 6, 512, 1024, True, 0),
    "skew16384": Workload("skew16384", 16384, 2048, 256, 6, 512, 1024, True, 0, zipf_bias=True),
    "stack47": Workload("stack47", 256, 2048, 256, 6, 512, 1024, True, 1, layers=47),
    "decode32_mx4": Workload("decode32_mx4", 32, 2048, 256, 6, 512, 1024, True, 0, mx4=True),
    "dense32": Workload("dense32", 32, 2048, 0, 0, 6144, 0, True, 0, dense=True),
    "dense4096": Workload("dense4096", 4096, 2048, 0, 0, 6144, 0, True, 0, dense=True),
}

EXPERT_MATRICES = ("gate", "up", "down", "shared_gate", "shared_up", "shared_down")

WEIGHT_STD = 0.02
ZIPF_S = 1.1
ZIPF_SCALE = 0.5

_TENSOR_IDS = {"router": 1, "bias": 2, "gate": 3, "up": 4, "down": 5,
               "shared_gate": 6, "shared_up": 7, "shared_down": 8, "x": 9,
               "dense_gate": 10, "dense_up": 11, "dense_down": 12}


def _gen(seed: int, layer: int, tensor: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + layer * 7919 + _TENSOR_IDS[tensor] * 104_729) % (2**62))
    return g


def _normal(shape, std, dtype, seed, layer, tensor, device):
    dev = torch.device(device)
    g = _gen(seed, layer, tensor, dev)
    if dtype == torch.float32:
        t = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
        return t.mul_(std) if std != 1.0 else t
    # Draw in float32 chunks and round, to bound the float32 temporary.
    out = torch.empty(shape, device=dev, dtype=dtype)
    flat = out.view(-1)
    chunk = 1 << 26
    for s in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - s)
        t = torch.randn((n,), generator=g, device=dev, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        flat[s:s + n].copy_(t)
    return out


def zipf_bias(n_experts: int, seed: int) -> np.ndarray:
    """Per-expert router bias that skews the load: expert e gets rank r(e) from a
    seeded permutation of 1..E and bias 0.5 * ln(E * p_r), p_r = r^-1.1 / sum_j j^-1.1."""
    g = torch.Generator().manual_seed(seed * 31 + 7)
    ranks = torch.randperm(n_experts, generator=g).numpy() + 1
    j = np.arange(1, n_experts + 1, dtype=np.float64)
    p = ranks.astype(np.float64) ** (-ZIPF_S) / np.sum(j ** (-ZIPF_S))
    return (ZIPF_SCALE * np.log(n_experts * p)).astype(np.float32)


def mx4_quantize(w: torch.Tensor):
    """Store a weight matrix in OCP Microscaling MXFP4, blocks of 32 along the
    last (reduction) dimension.  Returns (codes uint8 [..., n/2], scales uint8
    [..., n/32]).

    Per block: shared exponent X = floor(log2(max |w|)) - 2 (2 is the largest
    exponent of an E2M1 element), scale byte X + 127 (an all-zero block gets
    byte 0); elements w / 2^X go to the nearest E2M1 magnitude
    (0, 0.5, 1, 1.5, 2, 3, 4, 6; halfway cases to the code with a zero
    mantissa bit, i.e. the even code), saturating at 6; the sign goes to bit 3.
    Two elements per byte, the lower-indexed one in the low nibble."""
    n = w.shape[-1]
    if n % 32:
        raise ValueError("mx4_quantize: the last dimension must be a multiple of 32")
    lead = w.shape[:-1]
    codes = torch.empty(lead + (n // 2,), dtype=torch.uint8, device=w.device)
    scales = torch.empty(lead + (n // 32,), dtype=torch.uint8, device=w.device)
    wf_all = w.reshape(-1, n)
    cf, sf = codes.view(-1, n // 2), scales.view(-1, n // 32)
    rows = max(1, (1 << 24) // n)
    for r0 in range(0, wf_all.shape[0], rows):
        wf = wf_all[r0:r0 + rows].float().view(-1, n // 32, 32)
        amax = wf.abs().amax(-1)
        X = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 2, torch.full_like(amax, -127.0))
        X = X.clamp(-127, 127)
        q = wf / torch.exp2(X).unsqueeze(-1)
        m = q.abs()
        idx = ((m > 0.25).to(torch.uint8) + (m >= 0.75) + (m > 1.25) + (m >= 1.75) + (m > 2.5) + (m >= 3.5)
               + (m > 5.0))
        code = idx | ((q < 0).to(torch.uint8) << 3)
        code = code.view(code.shape[0], n)
        cf[r0:r0 + rows] = code[:, 0::2] | (code[:, 1::2] << 4)
        sf[r0:r0 + rows] = (X + 127).to(torch.uint8)
    return codes, scales


def mx4_tile(codes: torch.Tensor, scales: torch.Tensor):
    """Row-major MXFP4 arrays (codes [..., R, n/2], scales [..., R, n/32], as
    mx4_quantize returns them) in the tiled byte order the kernels read: a tile
    is 16 rows x one 32-element block; codes [..., R/16, n/32, 16, 16] (per
    tile, each row's 16 bytes, rows in order), scales [..., R/16, n/32, 16]."""
    R, nb = codes.shape[-2], scales.shape[-1]
    if R % 16:
        raise ValueError("mx4_tile: the row count must be a multiple of 16")
    lead = tuple(codes.shape[:-2])
    c = codes.reshape(lead + (R // 16, 16, nb, 16)).transpose(-3, -2).contiguous()
    s = scales.reshape(lead + (R // 16, 16, nb)).transpose(-2, -1).contiguous()
    return c, s


def make_dense(wl: Workload, layer: int = 0, device="cpu") -> dict:
    """Weights of a dense MLP layer: gate, up [I,H], down [H,I], N(0, 0.02^2)."""
    H, I, dt, s = wl.hidden, wl.inter, wl.torch_dtype, wl.seed
    return {"gate": _normal((I, H), WEIGHT_STD, dt, s, layer, "dense_gate", device),
            "up": _normal((I, H), WEIGHT_STD, dt, s, layer, "dense_up", device),
            "down": _normal((H, I), WEIGHT_STD, dt, s, layer, "dense_down", device)}


def make_layer(wl: Workload, layer: int = 0, device="cpu", with_shared: bool = True) -> dict:
    """Weights of one layer as torch tensors on ``device``.

    Layouts (row-major, reduction dimension contiguous):
      router [E,H], bias [E] float32 or None, gate/up [E,I,H], down [E,H,I],
      shared_gate/shared_up [Is,H], shared_down [H,Is].
    """
    E, H, I, Is = wl.n_experts, wl.hidden, wl.inter, wl.shared_inter
    dt, s = wl.torch_dtype, wl.seed
    w = {
        "router": _normal((E, H), WEIGHT_STD, dt, s, layer, "router", device),
        "gate": _normal((E, I, H), WEIGHT_STD, dt, s, layer, "gate", device),
        "up": _normal((E, I, H), WEIGHT_STD, dt, s, layer, "up", device),
        "down": _normal((E, H, I), WEIGHT_STD, dt, s, layer, "down", device),
        "bias": None,
    }
    if wl.zipf_bias:
        w["bias"] = torch.from_numpy(zipf_bias(E, s)).to(device)
    if with_shared and Is > 0:
        w["shared_gate"] = _normal((Is, H), WEIGHT_STD, dt, s, layer, "shared_gate", device)
        w["shared_up"] = _normal((Is, H), WEIGHT_STD, dt, s, layer, "shared_up", device)
        w["shared_down"] = _normal((H, Is), WEIGHT_STD, dt, s, layer, "shared_down", device)
    if wl.mx4:
        # stored as MXFP4 in tiled order: <name>_q codes and <name>_s scales replace <name>
        for name in EXPERT_MATRICES:
            if name in w:
                w[name + "_q"], w[name + "_s"] = mx4_tile(*mx4_quantize(w.pop(name)))
    return w


def make_tokens(wl: Workload, T: int | None = None, device="cpu", stream: int = 0) -> torch.Tensor:
    """Hidden states x [T,H] ~ N(0,1) in the workload's dtype."""
    T = wl.T if T is None else T
    return _normal((T, wl.hidden), 1.0, wl.torch_dtype, wl.seed, 10**6 + stream, "x", device)


def custom(name="custom", T=8, hidden=64, n_experts=8, top_k=2, inter=64, shared_inter=64,
           bf16=True, seed=0, zipf=False, layers=1, mx4=False, dense=False) -> Workload:
    return Workload(name, T, hidden, n_experts, top_k, inter, shared_inter, bf16, seed, zipf, layers, mx4, dense)


def expected_distinct_experts(T: int, E: int = 256, K: int = 6) -> float:
    """Expected number of experts hit by T tokens under uniform routing (a sizing
    aid for the roofline figures; the benchmark uses the measured count)."""
    return E * (1.0 - (1.0 - K / E) ** T) if T > 0 else 0.0


def to_numpy_f32(t: torch.Tensor | None):
    """Exact float32 copy of a (bf16 or float32) tensor, on the host."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float32).numpy()


__all__ = ["Workload", "WORKLOADS", "make_layer", "make_tokens", "zipf_bias", "custom",
           "expected_distinct_experts", "to_numpy_f32", "mx4_quantize", "EXPERT_MATRICES"]
