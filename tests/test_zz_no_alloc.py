"""GPU test of gdn2_chunk_fwd_noalloc (the entry point for callers that cannot
allocate): through the C ABI, its output and final state match
gdn2_chunk_fwd_opts' on the same inputs and options, on consecutive calls
that share the fixed scratch array, the second with a smaller input, and the
automatic plan fits its segments to the array.

Bar: the parity tolerance (rel-L2 <= 5e-3, max-abs <= 2e-2 on output and
final state); with the same segment length the two entry points run the same
kernels on the same plan, so the bits are expected to agree as well.
"""

import sys

import numpy as np
import pytest
import torch

from linear_attention_rnn_gdn2_amd.workloads import synth

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "beta", "w")
REL_L2 = 5e-3
MAX_ABS = 2e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from linear_attention_rnn_gdn2_amd import gdn2
    gdn2.load_library()
    return gdn2


def close(tag, x, r):
    x = x.double().cpu().numpy()
    r = r.double().cpu().numpy()
    nr = np.linalg.norm(r)
    rel = float(np.linalg.norm(x - r) / nr) if nr > 0 else 0.0
    mx = float(np.abs(x - r).max()) if x.size else 0.0
    say(f"{tag}: rel-L2 {rel:.3e} max-abs {mx:.3e}")
    assert np.isfinite(x).all() and rel <= REL_L2 and mx <= MAX_ABS, tag


def both(lib, d, split):
    dev = torch.device("cuda:0")
    a = {n: d[n].to(dev) for n in NAMES}
    s0 = d["initial_state"].to(dev)
    cu = d["cu_seqlens"].to(dev)
    T, HV, V = d["v"].shape
    N, K = cu.shape[0] - 1, d["q"].shape[2]
    ref_o, ref_s = lib.chunk_fwd(**a, scale=None, initial_state=s0, cu_seqlens=cu, seq_split=split)
    # the no-alloc call writes into buffers that hold stale values
    out = torch.full((T, HV, V), 3.0, dtype=torch.bfloat16, device=dev)
    fin = torch.full((N, HV, K, V), -5.0, dtype=torch.float32, device=dev)
    o, s = lib.chunk_fwd_noalloc(**a, scale=None, initial_state=s0, cu_seqlens=cu, out=out, final_state=fin,
                                 seq_split=split)
    torch.cuda.synchronize()
    return ref_o, ref_s, o, s


@pytest.mark.parametrize("split", [4, 0])
def test_noalloc_matches_allocating_entry(lib, split):
    """Two calls in a row on the shared scratch array: a long varlen batch,
    then a smaller one (fewer segments, other lengths)."""
    cases = [([1500, 900, 0, 2100], 2, 4, 128, 200), ([700, 130, 65], 1, 2, 64, 201)]
    for i, (lens, H, HV, D, seed) in enumerate(cases):
        say(f"[noalloc split={split}] call {i}: lengths {lens} H={H} HV={HV} K=V={D}")
        d = synth(lens, H, HV, D, D, seed=seed, init_std=0.02, beta_max=2.0)
        ro, rs, o, s = both(lib, d, split)
        close(f"call {i} out", o, ro)
        close(f"call {i} state", s, rs)
        assert torch.equal(o, ro) and torch.equal(s, rs), "same plan, same kernels: bits differ"


def test_noalloc_auto_plan_fits_scratch(lib):
    """Few long chains: the automatic plan splits; its segments are
    lengthened until the workspace fits the fixed array, and the result
    stays within the bar of the allocating entry."""
    # 2 x 8 chains x 512 chunks: the allocating plan (L = 23) would need
    # 3 x 16 x 45 x 64 KiB = 135 MiB
    lens = [32768, 32768]
    say(f"[noalloc auto] lengths {lens} H=HV=8 K=V=128")
    d = synth(lens, 8, 8, 128, 128, seed=202, init_std=0.02)
    ro, rs, o, s = both(lib, d, None)
    close("auto out", o, ro)
    close("auto state", s, rs)
