"""GPU tests of the boundary's breadth (FlashInfer chunk_gated_delta_rule2
parameter list): strided inputs and output, V-major states, fp16 io, bf16 /
fp16 g, int64 cu_seqlens and the in-kernel q/k L2 normalisation, on the
chunked path (whole sequences and split) and the token-by-token path.

Layout options change only where the kernels read and write, not what they
compute, so strided views, V-major states and int64 cu_seqlens must give the
same bits as the dense, K-major, int32 call. Type options and the L2
normalisation change the arithmetic and are held to the oracle bar
(relative L2 <= 5e-3, max abs <= 2e-2) on the same quantised inputs.
"""

import pytest
import torch

from linear_attention_rnn_gdn2_amd.workloads import synth
from tests.test_parity_gpu import NAMES, assert_parity, c_oracle, lib, say  # noqa: F401

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
LENS = [300, 64, 1, 0, 129, 17]


def dev(d):
    return {n: (None if d[n] is None else d[n].to(DEV)) for n in NAMES}


def call(lib, path, args, d, **kw):
    """One forward on `path` ("chunk", "split": segments of 2 chunks, or
    "rec"), synchronised."""
    s0 = kw.pop("initial_state", d["initial_state"])
    s0 = None if s0 is None else s0.to(DEV)
    cu = kw.pop("cu_seqlens", d["cu_seqlens"]).to(DEV)
    if path == "rec":
        out, fin = lib.recurrent_fwd(**args, scale=d["scale"], initial_state=s0, cu_seqlens=cu, **kw)
    else:
        out, fin = lib.chunk_fwd(**args, scale=d["scale"], initial_state=s0, cu_seqlens=cu,
                                 seq_split=2 if path == "split" else -1, **kw)
    torch.cuda.synchronize()
    return out, fin


def oracle(c_oracle, d, **kw):
    return c_oracle(*[d[n] for n in NAMES], d["scale"], d["initial_state"], d["cu_seqlens"], **kw)


def strided_copies(d, H, HV, D):
    """The inputs as strided device views: q, k, v from one fused
    [T, 3, H, D] buffer (H = HV), g with padded heads, beta and w stored
    head-major ([HV, T, D] seen as [T, HV, D])."""
    T = d["q"].shape[0]
    qkv = torch.empty((T, 3, H, D), dtype=d["q"].dtype, device=DEV)
    qkv[:, 0], qkv[:, 1], qkv[:, 2] = d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV)
    pad = 16 // d["g"].element_size()  # one 16-byte step of padding per head
    gp = torch.full((T, HV, D + pad), float("nan"), dtype=d["g"].dtype, device=DEV)
    gp[:, :, :D] = d["g"].to(DEV)
    bh = d["beta"].to(DEV).transpose(0, 1).contiguous().transpose(0, 1)
    wh = d["w"].to(DEV).transpose(0, 1).contiguous().transpose(0, 1)
    return dict(q=qkv[:, 0], k=qkv[:, 1], v=qkv[:, 2], g=gp[:, :, :D], beta=bh, w=wh)


@pytest.mark.parametrize("path", ["chunk", "split", "rec"])
def test_strided_views_bitwise(lib, path):
    """Strided inputs and a strided output (padded rows: the padding keeps its
    sentinel) give the bits of the dense call."""
    H = HV = 4
    D = 128
    d = synth(LENS if path != "rec" else [1, 5, 0, 33], H, HV, D, D, seed=200, init_std=0.02, beta_max=2.0)
    say(f"[strided {path}]")
    o_ref, f_ref = call(lib, path, dev(d), d)
    args = strided_copies(d, H, HV, D)
    T = d["q"].shape[0]
    big = torch.full((T, HV, D + 8), 5.0, dtype=torch.bfloat16, device=DEV)
    out, fin = call(lib, path, args, d, out=big[:, :, :D])
    assert torch.equal(out, o_ref), "strided output differs"
    assert torch.equal(fin, f_ref), "strided final state differs"
    assert torch.all(big[:, :, D:] == 5.0), "padding of the output was written"
    # head-major output [HV, T, V] seen as [T, HV, V]
    oh = torch.empty((HV, T, D), dtype=torch.bfloat16, device=DEV)
    out2, _ = call(lib, path, args, d, out=oh.transpose(0, 1))
    assert torch.equal(out2, o_ref)


@pytest.mark.parametrize("path", ["chunk", "split", "rec"])
def test_state_layout_vk_bitwise(lib, path):
    """V-major states ([N, HV, V, K]) in and out give the bits of the
    K-major call, transposed."""
    K = 128
    d = synth(LENS if path != "rec" else [1, 5, 0, 33], 2, 4, K, K, seed=201, init_std=0.05)
    say(f"[state vk {path}]")
    o_ref, f_ref = call(lib, path, dev(d), d)
    s0t = d["initial_state"].transpose(-1, -2).contiguous()
    out, fin = call(lib, path, dev(d), d, initial_state=s0t, state_layout="vk")
    assert torch.equal(out, o_ref)
    assert torch.equal(fin, f_ref.transpose(-1, -2))
    if path == "rec":  # in place, V-major
        s = s0t.to(DEV)
        out3, fin3 = lib.recurrent_fwd(**dev(d), scale=d["scale"], initial_state=s,
                                       cu_seqlens=d["cu_seqlens"].to(DEV), final_state=s, state_layout="vk")
        torch.cuda.synchronize()
        assert torch.equal(out3, o_ref) and torch.equal(s, f_ref.transpose(-1, -2))


@pytest.mark.parametrize("path", ["chunk", "split", "rec"])
def test_int64_cu_seqlens_bitwise(lib, path):
    d = synth(LENS if path != "rec" else [1, 5, 0, 33], 1, 2, 64, 64, seed=202, init_std=0.02)
    o_ref, f_ref = call(lib, path, dev(d), d)
    out, fin = call(lib, path, dev(d), d, cu_seqlens=d["cu_seqlens"].long())
    assert torch.equal(out, o_ref) and torch.equal(fin, f_ref)


@pytest.mark.parametrize("path", ["chunk", "split", "rec"])
@pytest.mark.parametrize("K,H,HV", [(128, 2, 4), (64, 1, 3)])
def test_fp16_io(lib, c_oracle, path, K, H, HV):
    """q, k, v, beta, w and out in float16; the oracle reads the same fp16
    values."""
    d = synth(LENS if path != "rec" else [1, 5, 0, 33, 2], H, HV, K, K, seed=203 + K, init_std=0.02,
              beta_max=2.0)
    for n in ("q", "k", "v", "beta", "w"):
        d[n] = d[n].float().half()
    say(f"[fp16 io {path}] K={K} H={H} HV={HV}")
    out, fin = call(lib, path, dev(d), d)
    assert out.dtype == torch.float16
    ro, rs = oracle(c_oracle, d)
    assert_parity(f"fp16 io {path}", out, fin, ro, rs)


@pytest.mark.parametrize("path", ["chunk", "split", "rec"])
@pytest.mark.parametrize("gt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("g_ext", [0.0, 8.0, 300.0])
def test_16bit_decay(lib, c_oracle, path, gt, g_ext):
    """g in bf16 or fp16, with and without extreme-decay channels (8: their
    share of A and P on MFMA from the staged decay sums; 300: the scalar
    per-pair path, which reads g again); the oracle reads the rounded g."""
    d = synth(LENS if path != "rec" else [1, 5, 0, 33], 2, 2, 128, 128, seed=204, init_std=0.02,
              g_extreme_max=g_ext, extreme_frac=0.1 if g_ext else 0.0, beta_max=2.0)
    d["g"] = d["g"].to(gt)
    say(f"[g {gt} {path}] g_ext={g_ext}")
    out, fin = call(lib, path, dev(d), d)
    ro, rs = oracle(c_oracle, d)
    assert_parity(f"g {gt} {path} ext {g_ext}", out, fin, ro, rs)


def unnormalised(d, seed):
    """q and k rows rescaled by factors in [0.2, 5] (then rounded to the io
    type again): inputs that are not unit rows."""
    gen = torch.Generator().manual_seed(seed)
    for n in ("q", "k"):
        f = 0.2 + 4.8 * torch.rand(d[n].shape[:2] + (1,), generator=gen)
        d[n] = (d[n].float() * f).to(d[n].dtype)
    return d


@pytest.mark.parametrize("path", ["chunk", "split", "rec"])
@pytest.mark.parametrize("K,H,HV", [(128, 2, 4), (64, 1, 3)])
def test_qk_l2norm(lib, c_oracle, path, K, H, HV):
    """In-kernel q/k L2 normalisation on rows that are not unit length."""
    d = unnormalised(synth(LENS if path != "rec" else [1, 5, 0, 33, 2], H, HV, K, K, seed=205 + K,
                           init_std=0.02, beta_max=2.0), 7)
    say(f"[l2norm {path}] K={K} H={H} HV={HV}")
    out, fin = call(lib, path, dev(d), d, qk_l2norm=True)
    ro, rs = oracle(c_oracle, d, qk_l2norm=True)
    assert_parity(f"l2norm {path}", out, fin, ro, rs)


@pytest.mark.parametrize("g_ext", [8.0, 300.0])
def test_qk_l2norm_extreme_decay(lib, c_oracle, g_ext):
    """L2 normalisation together with both extreme-decay paths (the flagged
    channels' operands take the normalised q and k)."""
    d = unnormalised(synth([500, 64, 130], 2, 2, 128, 128, seed=206, init_std=0.02, g_extreme_max=g_ext,
                           extreme_frac=0.1, beta_max=2.0), 8)
    for path in ("chunk", "split"):
        out, fin = call(lib, path, dev(d), d, qk_l2norm=True)
        ro, rs = oracle(c_oracle, d, qk_l2norm=True)
        assert_parity(f"l2norm extreme {path}", out, fin, ro, rs)


def test_l2norm_of_unit_rows_is_close(lib):
    """On unit rows the option changes only rounding."""
    d = synth(LENS, 2, 4, 128, 128, seed=207, init_std=0.02)
    o1, f1 = call(lib, "chunk", dev(d), d)
    o2, f2 = call(lib, "chunk", dev(d), d, qk_l2norm=True)
    assert (o1.float() - o2.float()).abs().max().item() < 1e-2
    assert (f1 - f2).abs().max().item() < 1e-2


@pytest.mark.parametrize("path", ["chunk", "split", "rec"])
def test_everything_together(lib, c_oracle, path):
    """fp16 io, fp16 g, strided views, V-major state, int64 cu_seqlens and
    L2 normalisation in one call."""
    H = HV = 2
    D = 128
    d = unnormalised(synth(LENS if path != "rec" else [1, 5, 0, 33], H, HV, D, D, seed=208, init_std=0.02,
                           g_extreme_max=40.0, extreme_frac=0.1, beta_max=2.0), 9)
    for n in ("q", "k", "v", "beta", "w"):
        d[n] = d[n].float().half()
    d["g"] = d["g"].half()
    args = strided_copies(d, H, HV, D)
    T = d["q"].shape[0]
    big = torch.full((T, HV, D + 8), 5.0, dtype=torch.float16, device=DEV)
    out, fin = call(lib, path, args, d, out=big[:, :, :D], initial_state=d["initial_state"].transpose(-1, -2).contiguous(),
                    cu_seqlens=d["cu_seqlens"].long(), state_layout="vk", qk_l2norm=True)
    ro, rs = oracle(c_oracle, d, qk_l2norm=True)
    assert_parity(f"everything {path}", out, fin.transpose(-1, -2), ro, rs)
    assert torch.all(big[:, :, D:] == 5.0)


@pytest.mark.parametrize("path", ["chunk", "split", "rec"])
@pytest.mark.parametrize("h0_t,ht_t", [(torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float32),
                                       (torch.float32, torch.bfloat16)])
def test_bf16_states(lib, c_oracle, path, h0_t, ht_t):
    """Initial and final states in bf16 (FlashInfer parameter list: float32
    or bfloat16), K-major and V-major; the oracle starts from the same
    rounded state, and a bf16 final state is the float32 one rounded."""
    d = synth(LENS if path != "rec" else [1, 5, 0, 33], 2, 4, 128, 128, seed=209, init_std=0.05, beta_max=2.0)
    d["initial_state"] = d["initial_state"].to(h0_t)
    ro, rs = oracle(c_oracle, d)
    N, HV, K, V = d["initial_state"].shape
    for layout in ("kv", "vk"):
        s0 = d["initial_state"] if layout == "kv" else d["initial_state"].transpose(-1, -2).contiguous()
        fin = torch.empty((N, HV, K, V), dtype=ht_t, device=DEV)
        out, fin = call(lib, path, dev(d), d, initial_state=s0, final_state=fin, state_layout=layout)
        f = fin if layout == "kv" else fin.transpose(-1, -2)
        assert_parity(f"states {h0_t}->{ht_t} {layout} {path}", out, f.float(), ro, rs)
        if ht_t == torch.bfloat16:
            # the float32 final state of the same call, rounded once
            f32 = torch.empty((N, HV, K, V), dtype=torch.float32, device=DEV)
            _, f32 = call(lib, path, dev(d), d, initial_state=s0, final_state=f32, state_layout=layout)
            assert torch.equal(fin, f32.to(torch.bfloat16))
    if path == "rec" and h0_t == ht_t:  # in place, bf16
        s = d["initial_state"].to(DEV)
        out3, _ = lib.recurrent_fwd(**dev(d), scale=d["scale"], initial_state=s, cu_seqlens=d["cu_seqlens"].to(DEV),
                                    final_state=s)
        torch.cuda.synchronize()
        assert_parity("states in place bf16", out3, s.float(), ro, rs)
