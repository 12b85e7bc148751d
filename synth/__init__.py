"""Seeded synthetic inputs for the MapFlow attention-retrieval path.

This module holds input recipes only: sender attention maps, the receiver's head
map W and the receiver's value tensor V, at the shapes of the workloads the path
is measured on.  None of the method's own arithmetic (block mass, Top-p
selection, BSR build, head mixing, retrieval) lives here; the oracle and the
HIP path both take what this module produces and compute independently.

MapFlow ("Accelerating Cross-Model LLM Inference via Attention Map Reuse",
montaan.com/papers/2610.14688) caches the sender's causal attention maps
(section "Attention Maps as Reuse States") and mixes its heads into the
receiver's heads with a learned linear map (section "MapFlow System Design",
item 3).  The maps, weights and datasets of the pages' model pairs are not
available, so every input here is drawn from a seeded recipe:

* ``gaussian``: A = causal softmax(Q K^T / sqrt(d) / tau_h) with Q, K ~ N(0, 1);
  tau_h = 1 for the tiny workload, tau_h ~ U(0.5, 2) for the 8B->3B-like pair.
* ``structured``: causal softmax of Gaussian noise (sigma = 1) plus an attention
  sink on key 0, a local band of width 512 and four random vertical stripes per
  head -- the sparsity the block Top-p compressor is designed for.
* W ~ N(0, 1/H_s) in fp32, V ~ N(0, 1) stored in the workload dtype.

Seeds: layer ``l`` of workload ``k`` uses ``s = 1000*k + l``.  The map stream
(seed ``s``) draws, in this order, tau, Q, K (gaussian recipes) or the stripe
columns (structured recipe); V and W come from their own CPU streams (seeds
``s + 9_000_000`` and ``s + 7_000_000``).  The N^2 score noise of the
structured maps uses a generator on the target device, so a map drawn on the
GPU differs from one drawn on the CPU with the same seed.  Whatever the device,
the generated tensor is the single source of truth: the oracle always receives
a host copy.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

__all__ = [
    "Workload", "WORKLOADS", "workload", "layer_seed", "gen_layer", "gen_maps",
    "gen_W", "gen_V", "varlen_lengths", "torch_dtype", "DTYPE_BYTES",
]

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "f64": 8}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
            "f64": torch.float64}[name]


@dataclass(frozen=True)
class Workload:
    """Shape and recipe of one workload (one sender layer unless ``layers`` > 1)."""
    name: str
    index: int          # seed family: layer seed = 1000 * index + layer
    N: int
    B: int
    H_s: int
    H_r: int
    H_kv: int
    d: int
    dtype: str
    p: float
    maps: str           # "gaussian" | "gaussian-temp" | "structured"
    layers: int = 1
    softmax_dtype: str = "f32"   # precision the generator's softmax runs in
    band: int = 512
    sink_bonus: float = 8.0
    band_bonus: float = 6.0
    stripe_bonus: float = 5.0
    n_stripes: int = 4
    noise_sigma: float = 1.0
    extra: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return -(-self.N // self.B)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # tiny fp32 single layer; the oracle finishes in well under a second
    "tiny-f32": Workload("tiny-f32", 1, N=256, B=16, H_s=4, H_r=4, H_kv=4, d=64,
                         dtype="f32", p=0.9, maps="gaussian", softmax_dtype="f64"),
    # 8B->3B-like pair, one reuse layer
    "pair8b3b-f16": Workload("pair8b3b-f16", 2, N=4096, B=64, H_s=32, H_r=24, H_kv=8,
                             d=128, dtype="f16", p=0.95, maps="gaussian-temp"),
    # 14B->8B-like pair, 24 reuse layers back to back (the measured workload)
    "pair14b8b-bf16": Workload("pair14b8b-bf16", 3, N=8192, B=64, H_s=40, H_r=32, H_kv=8,
                               d=128, dtype="bf16", p=0.9, maps="structured", layers=24),
    # long context single layer
    "long32k-f16": Workload("long32k-f16", 4, N=32768, B=128, H_s=32, H_r=32, H_kv=8,
                            d=128, dtype="f16", p=0.9, maps="structured"),
    # varlen packed batch: one Workload per sequence is derived by varlen_workloads()
    "varlen-bf16": Workload("varlen-bf16", 5, N=16384, B=64, H_s=32, H_r=24, H_kv=8,
                            d=128, dtype="bf16", p=0.9, maps="structured",
                            extra={"n_seq": 16, "len_lo": 1024, "len_hi": 16384,
                                   "ps": (0.8, 0.9, 0.95)}),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.with_(**overrides) if overrides else w


def layer_seed(w: Workload, layer: int = 0) -> int:
    return 1000 * w.index + layer


def varlen_lengths(w: Workload, seed: int | None = None) -> list[int]:
    """Sequence lengths U[len_lo, len_hi] (inclusive) of the packed varlen batch."""
    ex = w.extra
    g = torch.Generator().manual_seed(5000 if seed is None else seed)
    return [int(x) for x in torch.randint(ex["len_lo"], ex["len_hi"] + 1, (ex["n_seq"],),
                                          generator=g)]


def _cpu_gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed)


def _causal_softmax_rows(scores: torch.Tensor) -> torch.Tensor:
    """Row softmax over keys j <= i of an [N][N] score matrix (input recipe)."""
    N = scores.shape[-1]
    mask = torch.ones(N, N, dtype=torch.bool, device=scores.device).triu_(1)
    scores = scores.masked_fill(mask, float("-inf"))
    return torch.softmax(scores, dim=-1)


def gen_maps(w: Workload, seed: int, device="cpu", out_dtype: str | None = None,
             return_qk: bool = False):
    """Sender causal attention maps A[H_s][N][N] in ``out_dtype`` (default: the
    workload dtype), drawn on ``device``.  With ``return_qk`` the gaussian recipes
    also return the Q and K they were built from (fp64, CPU)."""
    out_dtype = out_dtype or w.dtype
    H, N, d = w.H_s, w.N, w.d
    g = _cpu_gen(seed)
    sm = torch_dtype(w.softmax_dtype)
    A = torch.empty(H, N, N, dtype=torch_dtype(out_dtype), device=device)
    if w.maps in ("gaussian", "gaussian-temp"):
        if w.maps == "gaussian-temp":
            tau = torch.rand(H, generator=g, dtype=torch.float64) * 1.5 + 0.5
        else:
            tau = torch.ones(H, dtype=torch.float64)
        Q = torch.randn(H, N, d, generator=g, dtype=torch.float64)
        K = torch.randn(H, N, d, generator=g, dtype=torch.float64)
        for h in range(H):
            q = Q[h].to(device=device, dtype=sm)
            k = K[h].to(device=device, dtype=sm)
            s = (q @ k.T) / (math.sqrt(d) * float(tau[h]))
            A[h] = _causal_softmax_rows(s).to(A.dtype)
        if return_qk:
            return A, Q, K, tau
        return A
    if w.maps == "structured":
        # fixed draw order: (no tau), (no Q/K), then V and W are drawn by gen_layer
        # from their own seeds; stripes and noise come from this map seed.
        stripes = torch.randint(0, N, (H, w.n_stripes), generator=g)
        dev = torch.device(device)
        gd = torch.Generator(device=dev).manual_seed(seed)
        i = torch.arange(N, device=dev).view(N, 1)
        j = torch.arange(N, device=dev).view(1, N)
        bonus = (w.sink_bonus * (j == 0).to(sm)
                 + w.band_bonus * ((j > i - w.band) & (j <= i)).to(sm))
        for h in range(H):
            s = torch.randn(N, N, generator=gd, device=dev, dtype=sm) * w.noise_sigma
            s += bonus
            s[:, stripes[h].to(dev)] += w.stripe_bonus
            A[h] = _causal_softmax_rows(s).to(A.dtype)
            del s
        return A
    raise ValueError(f"unknown map recipe {w.maps!r}")


def gen_W(w: Workload, seed: int) -> torch.Tensor:
    """Head map W[H_r][H_s] ~ N(0, 1/H_s), fp32, CPU."""
    g = _cpu_gen(seed + 7_000_000)
    return (torch.randn(w.H_r, w.H_s, generator=g, dtype=torch.float64)
            / math.sqrt(w.H_s)).to(torch.float32)


def gen_V(w: Workload, seed: int, out_dtype: str | None = None) -> torch.Tensor:
    """Receiver values V[N][H_kv][d] ~ N(0, 1), CPU, in the workload dtype."""
    g = _cpu_gen(seed + 9_000_000)
    return torch.randn(w.N, w.H_kv, w.d, generator=g, dtype=torch.float64).to(
        torch_dtype(out_dtype or w.dtype))


def gen_layer(w: Workload, layer: int = 0, device="cpu", seed: int | None = None,
              map_dtype: str | None = None, return_qk: bool = False) -> dict:
    """One reuse layer's inputs: sender maps A (on ``device``), W and V (CPU)."""
    s = layer_seed(w, layer) if seed is None else seed
    out = {"seed": s}
    r = gen_maps(w, s, device=device, out_dtype=map_dtype, return_qk=return_qk)
    if return_qk:
        out["A"], out["Q"], out["K"], out["tau"] = r
    else:
        out["A"] = r
    out["V"] = gen_V(w, s)
    out["W"] = gen_W(w, s)
    return out
