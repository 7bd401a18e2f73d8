"""Seeded synthetic inputs for the GDN-2 chunked prefill forward.

This module only draws random tensors. It holds none of the method's
arithmetic and imports neither the GPU binding nor the oracle, so both sides
can be fed the exact same bytes.

Distributions follow the Flash-GDN-2 README "Quick start" (q, k drawn from a
normal, L2-normalised per head and cast to bf16; v normal; g = -0.1 * U(0, 1)
as float32 log-decay; erase/write gates U(0, 1)), and the shapes follow the
FlashRT card's validated Hv/Hk/D profiles. The five named workloads are:

  tiny        1 x 256 tokens, H = HV = 2, K = V = 64, zero initial state,
              scale 1/8
  single      1 x 4096 tokens, H = HV = 16, K = V = 128, initial state
              N(0, 0.02^2)
  varlen      8 sequences with lengths uniform in [256, 8192] packed end to
              end, H = HV = 32, K = V = 128, per-sequence initial state
              N(0, 0.02^2)
  gva         4 x 16384 tokens, H = 16, HV = 48 (each q/k head shared by three
              value heads), K = V = 128, zero initial state
  long_decay  2 x 65536 tokens, H = HV = 16, K = V = 128; per value head, 13 of
              128 key channels (a seeded choice) draw g = -U(0, 8) and the rest
              g = -U(0, 0.1); beta = U(0, 2); zero initial state

Draw order from one ``torch.Generator`` seeded with ``seed``: lengths (varlen
only), q, k, v, g, beta, w, initial state, extreme-channel choice (long_decay
only).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    lengths: tuple | None          # fixed lengths, or None for drawn lengths
    n_seqs: int
    H: int
    HV: int
    K: int
    V: int
    init_std: float | None         # None: zero initial state (argument omitted)
    g_max: float = 0.1             # g = -U(0, g_max) on ordinary channels
    g_extreme_max: float = 0.0     # g = -U(0, g_extreme_max) on extreme channels
    extreme_frac: float = 0.0      # share of key channels that are extreme
    beta_max: float = 1.0          # beta = U(0, beta_max)
    len_range: tuple = field(default=(256, 8192))
    scale: float | None = None     # None: 1/sqrt(K)


WORKLOADS = {
    0: Workload("tiny", (256,), 1, 2, 2, 64, 64, None, scale=1.0 / 8.0),
    1: Workload("single", (4096,), 1, 16, 16, 128, 128, 0.02),
    2: Workload("varlen", None, 8, 32, 32, 128, 128, 0.02),
    3: Workload("gva", (16384,) * 4, 4, 16, 48, 128, 128, None),
    4: Workload("long_decay", (65536,) * 2, 2, 16, 16, 128, 128, None,
                g_extreme_max=8.0, extreme_frac=0.1, beta_max=2.0),
}


def describe(config_id: int) -> str:
    w = WORKLOADS[config_id]
    lens = "U[%d,%d]x%d" % (w.len_range[0], w.len_range[1], w.n_seqs) if w.lengths is None \
        else "x".join(str(x) for x in (len(w.lengths), w.lengths[0]))
    return f"{w.name}: seqs {lens}, H={w.H}, HV={w.HV}, K={w.K}, V={w.V}"


def synth(lengths, H, HV, K, V, seed, *, init_std=None, g_max=0.1,
          g_extreme_max=0.0, extreme_frac=0.0, beta_max=1.0, scale=None,
          draw_lengths=None):
    """Draw one packed batch.

    ``lengths``: list of sequence lengths (may contain 0), or None together with
    ``draw_lengths=(n, lo, hi)`` to draw n integer lengths uniform in [lo, hi].

    Returns a dict of CPU tensors:
      q, k [T, H, K] bf16; v, w [T, HV, V] bf16; g [T, HV, K] float32;
      beta [T, HV, K] bf16; initial_state [N, HV, K, V] float32 or None;
      cu_seqlens [N + 1] int32; plus ``scale`` (float or None) and ``lengths``.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    if lengths is None:
        n, lo, hi = draw_lengths
        lengths = torch.randint(lo, hi + 1, (n,), generator=gen).tolist()
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if lengths:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)

    def unit_rows(shape):
        x = torch.randn(shape, generator=gen, dtype=torch.float32)
        n = x.norm(dim=-1, keepdim=True).clamp_min(1e-12)
        return (x / n).to(torch.bfloat16)

    q = unit_rows((T, H, K))
    k = unit_rows((T, H, K))
    v = torch.randn((T, HV, V), generator=gen, dtype=torch.float32).to(torch.bfloat16)
    u = torch.rand((T, HV, K), generator=gen, dtype=torch.float32)
    beta = (torch.rand((T, HV, K), generator=gen, dtype=torch.float32) * beta_max).to(torch.bfloat16)
    w = torch.rand((T, HV, V), generator=gen, dtype=torch.float32).to(torch.bfloat16)
    S0 = None
    if init_std is not None:
        S0 = torch.randn((len(lengths), HV, K, V), generator=gen, dtype=torch.float32) * init_std
    span = torch.full((HV, K), float(g_max), dtype=torch.float32)
    n_ext = int(round(extreme_frac * K))
    if n_ext > 0:
        for hv in range(HV):
            idx = torch.randperm(K, generator=gen)[:n_ext]
            span[hv, idx] = float(g_extreme_max)
    g = -(u * span)
    return dict(q=q, k=k, v=v, g=g, beta=beta, w=w, initial_state=S0,
                cu_seqlens=cu, scale=scale, lengths=lengths)


def make_inputs(config_id: int, seed: int | None = None):
    """Inputs of one named workload (seed defaults to the workload id)."""
    wl = WORKLOADS[config_id]
    seed = config_id if seed is None else seed
    draw = None
    if wl.lengths is None:
        draw = (wl.n_seqs, wl.len_range[0], wl.len_range[1])
    d = synth(wl.lengths, wl.H, wl.HV, wl.K, wl.V, seed, init_std=wl.init_std,
              g_max=wl.g_max, g_extreme_max=wl.g_extreme_max,
              extreme_frac=wl.extreme_frac, beta_max=wl.beta_max,
              scale=wl.scale, draw_lengths=draw)
    d["workload"] = wl
    return d


def lengths_of(config_id: int, seed: int | None = None) -> list:
    """Sequence lengths of a workload without drawing the tensors (the
    lengths are the generator's first draw)."""
    wl = WORKLOADS[config_id]
    if wl.lengths is not None:
        return [int(x) for x in wl.lengths]
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(config_id if seed is None else seed))
    return torch.randint(wl.len_range[0], wl.len_range[1] + 1, (wl.n_seqs,), generator=gen).tolist()


def total_tokens(config_id: int, seed: int | None = None) -> int:
    """Total packed length of a workload without drawing the tensors."""
    return int(sum(lengths_of(config_id, seed)))



def synth_cotangents(T, N, HV, K, V, seed, *, d_final=True):
    """Incoming gradients for a backward call: d_out [T, HV, V] ~ N(0, 1) as
    bf16 and d_final_state [N, HV, K, V] ~ N(0, 1) as float32 (None when
    ``d_final`` is false), from their own generator seeded with ``seed``."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed) + 7919)
    d_out = torch.randn((T, HV, V), generator=gen).to(torch.bfloat16)
    dht = torch.randn((N, HV, K, V), generator=gen) if d_final else None
    return d_out, dht
