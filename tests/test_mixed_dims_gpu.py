"""GPU parity at unequal head dimensions, (K, V) = (128, 64) and (64, 128)
(the Flash-GDN-2 README's training paragraph: both head dimensions in
{64, 128}), against the FP64 oracle: ragged lengths with grouped value
heads and the default scale 1/sqrt(K); the split path, whose transition
maps are K x K (walked by the square kernel) while the end states are
K x V; the automatic plan on one long sequence; fp16 io, fp16 g, in-kernel
L2 normalisation and V-major bf16 states together; strong decay on both of
its paths; the token-by-token entry; and the allocation-free entry against
the allocating one, bit for bit.
"""

import numpy as np
import pytest
import torch

from linear_attention_rnn_gdn2_amd.workloads import synth
from tests.test_parity_gpu import NAMES, assert_parity, assert_slices, c_oracle, lib, ref, run_gpu, say  # noqa: F401

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
DIMS = [(128, 64), (64, 128)]
LENS = [1, 63, 64, 65, 0, 127, 129, 300, 17]


@pytest.mark.parametrize("K,V", DIMS)
def test_mixed_ragged_default_scale(lib, c_oracle, K, V):
    """Ragged lengths, grouped heads (HV = 2H), beta up to 2, scale None:
    the kernel's default must be 1/sqrt(K), the oracle's pinned reading."""
    say(f"[mixed ragged] K={K} V={V}")
    d = synth(LENS, 2, 4, K, V, seed=300 + K, init_std=0.02, beta_max=2.0)
    out, fin = run_gpu(lib, d, scale=None)
    assert out.shape == (sum(LENS), 4, V) and fin.shape == (len(LENS), 4, K, V)
    ro, rs = ref(c_oracle, d, scale=None)
    assert_parity(f"mixed ragged K={K} V={V}", out, fin, ro, rs)
    assert_slices(f"mixed ragged K={K} V={V}", out, fin, ro, rs, d["cu_seqlens"].tolist(), min_len=64)


@pytest.mark.parametrize("K,V", DIMS)
@pytest.mark.parametrize("seg", [1, 3])
def test_mixed_forced_split(lib, c_oracle, K, V, seg):
    """Segments of 1 and 3 chunks: end states K x V and transition maps
    K x K in separate launches, chained by the combine."""
    say(f"[mixed split] K={K} V={V} segment {seg}")
    d = synth([700, 65, 1, 0, 300], 2, 4, K, V, seed=310 + seg, init_std=0.02, beta_max=2.0)
    ro, rs = ref(c_oracle, d)
    out, fin = lib.chunk_fwd(*[d[n].to(DEV) for n in NAMES], scale=d["scale"],
                             initial_state=d["initial_state"].to(DEV), cu_seqlens=d["cu_seqlens"].to(DEV),
                             seq_split=seg)
    torch.cuda.synchronize()
    assert_parity(f"mixed split K={K} V={V} seg={seg}", out, fin, ro, rs)
    assert_slices(f"mixed split K={K} V={V} seg={seg}", out, fin, ro, rs, d["cu_seqlens"].tolist(), min_len=64)


@pytest.mark.parametrize("K,V", DIMS)
def test_mixed_single_sequence_auto_plan(lib, c_oracle, K, V):
    """One 4096-token sequence over 16 heads: few chains, so the automatic
    plan splits it."""
    plan = lib.split_plan(4096, 1, 16, torch.cuda.get_device_properties(0).multi_processor_count)
    say(f"[mixed single] K={K} V={V} automatic segment length {plan}")
    d = synth([4096], 16, 16, K, V, seed=320, init_std=0.02)
    out, fin = run_gpu(lib, d)
    ro, rs = ref(c_oracle, d)
    assert_parity(f"mixed single K={K} V={V}", out, fin, ro, rs)
    assert_slices(f"mixed single K={K} V={V}", out, fin, ro, rs, d["cu_seqlens"].tolist())


@pytest.mark.parametrize("K,V", DIMS)
@pytest.mark.parametrize("path", ["chunk", "split", "rec"])
def test_mixed_options_together(lib, c_oracle, K, V, path):
    """fp16 io and g, rows that are not unit length normalised in the kernel,
    bf16 initial state stored V-major, float32 final state V-major."""
    from oracle.c_oracle import gdn2_recurrence_c
    gen = torch.Generator().manual_seed(K + 2 * V)
    lens = [300, 64, 1, 0, 129, 17] if path != "rec" else [1, 5, 0, 33]
    d = synth(lens, 2, 4, K, V, seed=330 + K, init_std=0.02, g_extreme_max=8.0, extreme_frac=0.1, beta_max=2.0)
    for n in ("q", "k"):
        f = 0.2 + 4.8 * torch.rand(d[n].shape[:2] + (1,), generator=gen)
        d[n] = (d[n].float() * f).half()
    for n in ("v", "beta", "w"):
        d[n] = d[n].float().half()
    d["g"] = d["g"].half()
    d["initial_state"] = d["initial_state"].to(torch.bfloat16)
    say(f"[mixed options] K={K} V={V} {path}")
    args = {n: d[n].to(DEV) for n in NAMES}
    s0 = d["initial_state"].transpose(-1, -2).contiguous().to(DEV)
    cu = d["cu_seqlens"].long().to(DEV)
    if path == "rec":
        out, fin = lib.recurrent_fwd(**args, scale=None, initial_state=s0, cu_seqlens=cu, state_layout="vk",
                                     qk_l2norm=True)
    else:
        out, fin = lib.chunk_fwd(**args, scale=None, initial_state=s0, cu_seqlens=cu, state_layout="vk",
                                 qk_l2norm=True, seq_split=2 if path == "split" else -1)
    torch.cuda.synchronize()
    ro, rs = gdn2_recurrence_c(*[d[n] for n in NAMES], None, d["initial_state"], d["cu_seqlens"], qk_l2norm=True)
    assert_parity(f"mixed options K={K} V={V} {path}", out.float(), fin.transpose(-1, -2), ro, rs)


@pytest.mark.parametrize("K,V", DIMS)
@pytest.mark.parametrize("g_ext", [8.0, 300.0])
def test_mixed_strong_decay(lib, c_oracle, K, V, g_ext):
    """10% of the key channels at g = -U(0, g_ext): flagged channels on MFMA
    (8), or the scalar per-pair path (300), whole and split."""
    say(f"[mixed strong decay] K={K} V={V} g_ext={g_ext}")
    d = synth([500, 64, 130], 2, 2, K, V, seed=340, init_std=0.02, g_extreme_max=g_ext, extreme_frac=0.1,
              beta_max=2.0)
    ro, rs = ref(c_oracle, d)
    for split in (-1, 2):
        out, fin = lib.chunk_fwd(*[d[n].to(DEV) for n in NAMES], scale=d["scale"],
                                 initial_state=d["initial_state"].to(DEV), cu_seqlens=d["cu_seqlens"].to(DEV),
                                 seq_split=split)
        torch.cuda.synchronize()
        assert_parity(f"mixed strong decay K={K} V={V} g_ext={g_ext} split={split}", out, fin, ro, rs)


@pytest.mark.parametrize("K,V", DIMS)
def test_mixed_prefill_then_decode(lib, c_oracle, K, V):
    """Chunked prefill of 300 tokens, then 64 tokens decoded one call per
    token from the carried state, against one oracle pass over all 364."""
    say(f"[mixed decode] K={K} V={V}")
    d = synth([364], 2, 4, K, V, seed=350, init_std=0.02, beta_max=2.0)
    ro, rs = ref(c_oracle, d)
    P = 300
    args = {n: d[n].to(DEV) for n in NAMES}
    out, fin = lib.chunk_fwd(**{n: a[:P] for n, a in args.items()}, scale=d["scale"],
                             initial_state=d["initial_state"].to(DEV))
    outs = [out]
    for t in range(P, 364):
        o, fin = lib.recurrent_fwd(**{n: a[t:t + 1] for n, a in args.items()}, scale=d["scale"],
                                   initial_state=fin, final_state=fin)
        outs.append(o)
    torch.cuda.synchronize()
    assert_parity(f"mixed prefill+decode K={K} V={V}", torch.cat(outs), fin, ro, rs)
    o_dec = torch.cat(outs[1:]).float().cpu().double().numpy()
    rel = np.linalg.norm(o_dec - ro[P:]) / np.linalg.norm(ro[P:])
    say(f"mixed decoded tokens alone: rel-L2 {rel:.3e}")
    assert rel <= 5e-3


@pytest.mark.parametrize("K,V", DIMS)
def test_mixed_noalloc_matches(lib, K, V):
    """The allocation-free entry equals the allocating one bit for bit on a
    split run, twice in a row (the second call smaller)."""
    for lens, seg in (([900, 70, 5], 2), ([200, 3], 1)):
        say(f"[mixed noalloc] K={K} V={V} lengths {lens} segment {seg}")
        d = synth(lens, 2, 4, K, V, seed=360 + seg, init_std=0.02)
        args = [d[n].to(DEV) for n in NAMES]
        s0, cu = d["initial_state"].to(DEV), d["cu_seqlens"].to(DEV)
        o1, f1 = lib.chunk_fwd(*args, scale=d["scale"], initial_state=s0, cu_seqlens=cu, seq_split=seg)
        o2 = torch.empty_like(o1)
        f2 = torch.empty_like(f1)
        lib.chunk_fwd_noalloc(*args, scale=d["scale"], initial_state=s0, cu_seqlens=cu, out=o2, final_state=f2,
                              seq_split=seg)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(f1, f2)
