"""GPU parity on seeded random configurations against the FP64 oracles:
the chunked forward, the backward and the token-by-token entry; and the
allocation-free entry against the allocating one, bit for bit.

The hand-picked tests elsewhere each exercise one option at a time; here
every configuration draws all of them together from a seeded generator:
ragged lengths with empty and one-token sequences, (K, V) in {64, 128}^2
(the backward: K = V), grouped value heads (HV = m H, m up to 3), bf16 or
fp16 io, float32, bf16 or fp16 g, beta up to 1 or 2, strong-decay channels
(a tenth of the key channels at g = -U(0, 8) or -U(0, 40)), an initial
state (float32, bf16 or none, K- or V-major), in-kernel L2 normalisation of
q and k rows of arbitrary length, the default scale or the inputs' own,
and whole, split or automatically planned sequences. The bars are those of
the other parity tests: the forward's output and final state within 5e-3
relative L2 and 2e-2 max-abs of the oracle's, the backward's gradients
within its own bar (1e-2 relative L2, 5e-2 max-abs over the tensor's
largest reference magnitude).
"""

import random

import pytest
import torch

from linear_attention_rnn_gdn2_amd.workloads import synth, synth_cotangents
from tests.test_bwd_gpu import GRADS
from tests.test_bwd_gpu import assert_parity as assert_bwd_parity
from tests.test_parity_gpu import NAMES, assert_parity, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
IO = (torch.bfloat16, torch.float16)
GT = (torch.float32, torch.bfloat16, torch.float16)


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from linear_attention_rnn_gdn2_amd import gdn2
    gdn2.load_library()
    return gdn2


def draw_lengths(r):
    n = r.randint(1, 6)
    out = []
    for _ in range(n):
        u = r.random()
        out.append(0 if u < 0.15 else 1 if u < 0.25 else r.randint(2, 700))
    return out


def draw_case(seed, square):
    """One configuration: the drawn options and the seeded inputs (CPU),
    already in the drawn types (the oracle sees the same quantised values).
    square: K = V and no in-kernel L2 normalisation (the backward's range).
    Rows of q and k are scaled away from unit length only where the kernel
    normalises them: the transition I - k (beta * k)^T has the eigenvalue
    1 - sum_c beta_c k_c^2, below -1 (expansive) once that sum exceeds 2,
    which keys longer than 1 reach at beta near 2; the recurrence then
    amplifies every rounding on both sides."""
    r = random.Random(seed)
    lengths = draw_lengths(r)
    K = r.choice((64, 128))
    V = K if square else r.choice((64, 128))
    H = r.choice((1, 2))
    HV = H * r.choice((1, 2, 3))
    io, gt = r.choice(IO), r.choice(GT)
    strong = r.random() < 0.4
    opts = dict(lengths=lengths, K=K, V=V, H=H, HV=HV, io=io, gt=gt, beta_max=r.choice((1.0, 2.0)),
                strong=strong, g_ext=r.choice((8.0, 40.0)) if strong else 0.0,
                init=r.choice(("f32", "bf16", None)), default_scale=r.random() < 0.5,
                l2norm=r.random() < 0.4 and not square, layout=r.choice(("kv", "vk")),
                split=r.choice((None, -1, 2, 3)))
    d = synth(lengths, H, HV, K, V, seed=1000 + seed, init_std=0.02 if opts["init"] else None,
              beta_max=opts["beta_max"], g_extreme_max=opts["g_ext"], extreme_frac=0.1 if strong else 0.0)
    if opts["l2norm"]:  # rows of any length: the kernel normalises them
        gen = torch.Generator().manual_seed(seed)
        for n in ("q", "k"):
            d[n] = d[n].float() * (0.2 + 4.8 * torch.rand(d[n].shape[:2] + (1,), generator=gen))
    for n in ("q", "k", "v", "beta", "w"):
        d[n] = d[n].float().to(io)
    d["g"] = d["g"].to(gt)
    if opts["init"] == "bf16":
        d["initial_state"] = d["initial_state"].to(torch.bfloat16)
    if opts["default_scale"]:
        d["scale"] = None
    return opts, d


@pytest.mark.parametrize("seed", range(12))
def test_random_forward(lib, seed):
    from oracle.c_oracle import gdn2_recurrence_c
    o, d = draw_case(seed, square=False)
    tag = f"forward seed {seed}: " + ", ".join(f"{k}={v}" for k, v in o.items())
    say(f"[random] {tag}")
    s0 = d["initial_state"]
    if s0 is not None:
        s0 = (s0.transpose(-1, -2).contiguous() if o["layout"] == "vk" else s0).to(DEV)
    out, fin = lib.chunk_fwd(*[d[n].to(DEV) for n in NAMES], scale=d["scale"], initial_state=s0,
                             cu_seqlens=d["cu_seqlens"].to(DEV), seq_split=o["split"], state_layout=o["layout"],
                             qk_l2norm=o["l2norm"])
    torch.cuda.synchronize()
    assert out.dtype == o["io"]
    fin = fin.transpose(-1, -2) if o["layout"] == "vk" else fin
    ro, rs = gdn2_recurrence_c(*[d[n] for n in NAMES], d["scale"], d["initial_state"], d["cu_seqlens"],
                               qk_l2norm=o["l2norm"])
    assert_parity(tag, out.float(), fin.float(), ro, rs)


@pytest.mark.parametrize("seed", range(8))
def test_random_backward(lib, seed):
    from oracle.build import LIB, build_c_oracle
    import os
    if not os.path.exists(LIB):
        build_c_oracle()
    from oracle.c_oracle import gdn2_recurrence_bwd_c
    o, d = draw_case(100 + seed, square=True)
    if o["init"] == "bf16":  # the backward takes a float32 initial state
        d["initial_state"] = d["initial_state"].float()
    T, N = sum(o["lengths"]), len(o["lengths"])
    d_out, dht = synth_cotangents(T, N, o["HV"], o["K"], o["V"], 2000 + seed, d_final=seed % 3 != 0)
    d_out = d_out.float().to(o["io"])
    keys = ("lengths", "K", "H", "HV", "io", "gt", "beta_max", "strong", "g_ext", "init", "default_scale")
    tag = f"backward seed {seed}: " + ", ".join(f"{k}={o[k]}" for k in keys) + f", d_final={dht is not None}"
    say(f"[random] {tag}")
    got = lib.chunk_bwd(*[d[n].to(DEV) for n in NAMES], d_out.to(DEV), scale=d["scale"],
                        initial_state=None if d["initial_state"] is None else d["initial_state"].to(DEV),
                        cu_seqlens=d["cu_seqlens"].to(DEV), d_final_state=None if dht is None else dht.to(DEV))
    torch.cuda.synchronize()
    ref = gdn2_recurrence_bwd_c(*[d[n] for n in NAMES], d["scale"], d["initial_state"], d["cu_seqlens"].numpy(),
                                d_out, dht)
    assert_bwd_parity({n: got[n].float().cpu().double().numpy() for n in GRADS}, ref, tag)


NOALLOC_BYTES = 64 << 20  # GDN2_NOALLOC_SCRATCH_BYTES in include/gdn2.h


def split_bytes(o, split):
    """The split run's workspace at segments of `split` chunks, as the
    header states it: N * HV * nseg * (2 K V + K K) * 4 bytes."""
    T, N = sum(o["lengths"]), len(o["lengths"])
    nseg = (-(-T // 64) + split - 1) // split
    return N * o["HV"] * nseg * (2 * o["K"] * o["V"] + o["K"] * o["K"]) * 4


@pytest.mark.parametrize("seed", range(8))
def test_random_recurrent(lib, seed):
    """The token-by-token entry on the same kind of configurations."""
    from oracle.c_oracle import gdn2_recurrence_c
    o, d = draw_case(300 + seed, square=False)
    keys = ("lengths", "K", "V", "H", "HV", "io", "gt", "strong", "init", "l2norm", "layout", "default_scale")
    tag = f"recurrent seed {seed}: " + ", ".join(f"{k}={o[k]}" for k in keys)
    say(f"[random] {tag}")
    s0 = d["initial_state"]
    if s0 is not None:
        s0 = (s0.transpose(-1, -2).contiguous() if o["layout"] == "vk" else s0).to(DEV)
    out, fin = lib.recurrent_fwd(*[d[n].to(DEV) for n in NAMES], scale=d["scale"], initial_state=s0,
                                 cu_seqlens=d["cu_seqlens"].to(DEV), state_layout=o["layout"], qk_l2norm=o["l2norm"])
    torch.cuda.synchronize()
    fin = fin.transpose(-1, -2) if o["layout"] == "vk" else fin
    ro, rs = gdn2_recurrence_c(*[d[n] for n in NAMES], d["scale"], d["initial_state"], d["cu_seqlens"],
                               qk_l2norm=o["l2norm"])
    assert_parity(tag, out.float(), fin.float(), ro, rs)


@pytest.mark.parametrize("seed", range(6))
def test_random_noalloc_equals_allocating(lib, seed):
    """The allocation-free entry against the allocating one, bit for bit
    (an explicit split whose workspace would exceed the scratch array is
    drawn again as the automatic plan, which the entry fits to the array)."""
    o, d = draw_case(200 + seed, square=False)
    split = o["split"]
    if split is not None and split > 0 and split_bytes(o, split) > NOALLOC_BYTES:
        split = None
    say(f"[random] noalloc seed {seed}: lengths {o['lengths']}, K {o['K']} V {o['V']} HV {o['HV']}, split {split}")
    s0 = d["initial_state"]
    if s0 is not None:
        s0 = (s0.transpose(-1, -2).contiguous() if o["layout"] == "vk" else s0).to(DEV)
    args = [d[n].to(DEV) for n in NAMES]
    kw = dict(scale=d["scale"], initial_state=s0, cu_seqlens=d["cu_seqlens"].to(DEV), seq_split=split,
              state_layout=o["layout"], qk_l2norm=o["l2norm"])
    o1, f1 = lib.chunk_fwd(*args, **kw)
    o2, f2 = torch.empty_like(o1), torch.empty_like(f1)
    lib.chunk_fwd_noalloc(*args, out=o2, final_state=f2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
