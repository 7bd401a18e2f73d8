"""CPU tests of the C-ABI library: it loads, exports every symbol the public
header declares, and its host-side validation rejects each malformed call
with the documented status. No GPU is touched: ``gdn2_chunk_fwd_check``
runs the validation alone and descriptors may point at host memory.
"""

import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn2.h")


@pytest.fixture(scope="module")
def gdn2():
    from linear_attention_rnn_gdn2_amd import gdn2 as mod
    if not os.path.exists(mod.LIB_PATH):
        from linear_attention_rnn_gdn2_amd._build import build_library
        build_library()
    mod.load_library()
    return mod


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn2_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(gdn2):
    import ctypes
    lib = ctypes.CDLL(gdn2.LIB_PATH)
    names = declared_functions()
    assert set(names) == set(gdn2.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_abi_version_matches_header(gdn2):
    m = re.search(r"#define GDN2_ABI_VERSION (\d+)", open(HEADER).read())
    assert gdn2.load_library().gdn2_abi_version() == int(m.group(1))


def test_status_codes_match_header(gdn2):
    src = open(HEADER).read()
    codes = dict((int(v), k) for k, ok, v in re.findall(r"GDN2_(?:ERR_(\w+)|(OK)) = (-?\d+)", src)
                 for k in [k or ok])
    assert codes == gdn2.STATUS


def case(T=70, H=2, HV=4, K=64, V=64, N=2):
    t = dict(q=torch.zeros(T, H, K, dtype=torch.bfloat16), k=torch.zeros(T, H, K, dtype=torch.bfloat16),
             v=torch.zeros(T, HV, V, dtype=torch.bfloat16), g=torch.zeros(T, HV, K),
             beta=torch.zeros(T, HV, K, dtype=torch.bfloat16), w=torch.zeros(T, HV, V, dtype=torch.bfloat16),
             initial_state=torch.zeros(N, HV, K, V), cu_seqlens=torch.tensor([0, 30, T], dtype=torch.int32),
             out=torch.zeros(T, HV, V, dtype=torch.bfloat16), final_state=torch.zeros(N, HV, K, V))
    return t


def status(gdn2, **kw):
    rc = gdn2.check(**kw)
    return gdn2.STATUS[rc], gdn2.last_error()


def test_valid_calls(gdn2):
    assert status(gdn2, **case()) == ("OK", "")
    assert status(gdn2, **case(K=128, V=128))[0] == "OK"
    # unequal head dimensions (K and V each 64 or 128)
    assert status(gdn2, **case(K=128, V=64))[0] == "OK"
    assert status(gdn2, **case(K=64, V=128))[0] == "OK"
    c = case()
    for opt in ("g", "beta", "w", "initial_state", "final_state"):
        c2 = dict(c)
        c2[opt] = None
        assert status(gdn2, **c2)[0] == "OK", opt
    c2 = dict(c)
    c2["cu_seqlens"] = None
    c2["initial_state"] = torch.zeros(1, 4, 64, 64)
    c2["final_state"] = torch.zeros(1, 4, 64, 64)
    assert status(gdn2, **c2)[0] == "OK"
    assert status(gdn2, **case(T=0))[0] == "OK"


@pytest.mark.parametrize("mutate,expect", [
    (lambda c: c.update(q=None), "NULL_ARG"),
    (lambda c: c.update(v=None), "NULL_ARG"),
    (lambda c: c.update(out=None), "NULL_ARG"),
    (lambda c: c.update(q=c["q"].float()), "DTYPE"),
    (lambda c: c.update(g=c["g"].double()), "DTYPE"),
    (lambda c: c.update(g=c["g"].int()), "DTYPE"),
    (lambda c: c.update(k=c["k"].half()), "DTYPE"),                     # io types disagree
    (lambda c: c.update(beta=c["beta"].half()), "DTYPE"),
    (lambda c: c.update(out=c["out"].half()), "DTYPE"),
    (lambda c: c.update(q=c["q"].half(), k=c["k"].half(), v=c["v"].half(), beta=c["beta"].half(),
                        w=c["w"].half()), "DTYPE"),                       # out left bf16
    (lambda c: c.update(initial_state=c["initial_state"].half()), "DTYPE"),
    (lambda c: c.update(final_state=c["final_state"].double()), "DTYPE"),
    (lambda c: c.update(cu_seqlens=c["cu_seqlens"].float()), "DTYPE"),
    (lambda c: c.update(cu_seqlens=c["cu_seqlens"].short()), "DTYPE"),
    (lambda c: c.update(out=c["out"].float()), "DTYPE"),
    (lambda c: c.update(k=c["k"][:60]), "SHAPE"),
    (lambda c: c.update(beta=c["beta"][:, :2]), "SHAPE"),
    (lambda c: c.update(q=c["q"][None]), "SHAPE"),
    (lambda c: c.update(final_state=torch.zeros(3, 4, 64, 64)), "SHAPE"),
    (lambda c: c.update(cu_seqlens=torch.tensor([0], dtype=torch.int32)), "SHAPE"),
    (lambda c: c.update(v=torch.zeros(70, 3, 64, dtype=torch.bfloat16)), "HEADS"),
    (lambda c: c.update(v=torch.zeros(70, 1, 64, dtype=torch.bfloat16)), "HEADS"),
    (lambda c: c.update(q=torch.zeros(70, 2, 96, dtype=torch.bfloat16), k=torch.zeros(70, 2, 96, dtype=torch.bfloat16)),
     "UNSUPPORTED"),
    (lambda c: c.update(v=torch.zeros(70, 4, 96, dtype=torch.bfloat16)), "UNSUPPORTED"),
    (lambda c: c.update(v=torch.zeros(70, 4, 32, dtype=torch.bfloat16)), "UNSUPPORTED"),
    (lambda c: c.update(v=torch.zeros(70, 4, 128, dtype=torch.bfloat16)), "SHAPE"),   # w, out stay V = 64
    (lambda c: c.update(v=torch.zeros(70, 64, 4, dtype=torch.bfloat16).transpose(1, 2)), "LAYOUT"),
    (lambda c: c.update(q=torch.zeros(70 * 2 * 64 + 1, dtype=torch.bfloat16)[1:].view(70, 2, 64)), "LAYOUT"),
    # head stride of 68 elements: rows not 16-byte aligned
    (lambda c: c.update(q=torch.zeros(70, 2, 68, dtype=torch.bfloat16)[:, :, :64]), "LAYOUT"),
    # token stride shorter than a row (rows of one head overlap)
    (lambda c: c.update(k=torch.zeros(2 * 70 * 64, dtype=torch.bfloat16).as_strided((70, 2, 64), (8, 64 * 70, 1))),
     "LAYOUT"),
    # a broadcast (stride 0) token dimension: shorter than a row
    (lambda c: c.update(v=torch.zeros(1, 4, 64, dtype=torch.bfloat16).expand(70, 4, 64)), "LAYOUT"),
    # out rows overlapping each other (two heads at one address)
    (lambda c: c.update(out=torch.zeros(70, 1, 64, dtype=torch.bfloat16).expand(70, 4, 64)), "LAYOUT"),
    (lambda c: c.update(initial_state=c["initial_state"].transpose(2, 3)), "LAYOUT"),
])
def test_rejections(gdn2, mutate, expect):
    c = case()
    mutate(c)
    code, msg = status(gdn2, **c)
    assert code == expect, (code, msg)
    assert msg


def test_accepted_types_and_strides(gdn2):
    """fp16 io, 16-bit g, int64 cu_seqlens, and strided views whose rows are
    contiguous (FlashInfer parameter list: strides honoured, innermost
    dimension contiguous) pass validation."""
    c = case()
    for n in ("q", "k", "v", "beta", "w", "out"):
        c[n] = c[n].half()
    assert status(gdn2, **c) == ("OK", "")
    for gt in (torch.bfloat16, torch.float16):
        c = case()
        c["g"] = c["g"].to(gt)
        assert status(gdn2, **c)[0] == "OK"
    c = case()
    c["cu_seqlens"] = c["cu_seqlens"].long()
    assert status(gdn2, **c)[0] == "OK"
    c = case()
    c["initial_state"] = c["initial_state"].bfloat16()
    c["final_state"] = c["final_state"].bfloat16()
    assert status(gdn2, **c)[0] == "OK"
    # q, k, v as views of one fused [T, 3, H, D] projection (H = HV here)
    c = case(H=4)
    qkv = torch.zeros(70, 3, 4, 64, dtype=torch.bfloat16)
    c["q"], c["k"], c["v"] = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    assert status(gdn2, **c) == ("OK", "")
    # head-major storage [H, T, D] seen as [T, H, D]; padded token rows
    c = case()
    c["q"] = torch.zeros(2, 70, 64, dtype=torch.bfloat16).transpose(0, 1)
    c["g"] = torch.zeros(70, 4, 72)[:, :, :64]
    c["out"] = torch.zeros(4, 70, 64, dtype=torch.bfloat16).transpose(0, 1)
    assert status(gdn2, **c) == ("OK", "")
    # one token: its token stride is never used
    c = case(T=1)
    c["cu_seqlens"] = torch.tensor([0, 1, 1], dtype=torch.int32)
    c["q"] = torch.zeros(1, 2, 64, dtype=torch.bfloat16).as_strided((1, 2, 64), (3, 64, 1))
    assert status(gdn2, **c) == ("OK", "")


def test_alias_rules(gdn2):
    c = case()
    c["final_state"] = c["initial_state"]
    assert status(gdn2, **c)[0] == "ALIAS"
    c = case()
    buf = torch.zeros(70, 4, 64, dtype=torch.bfloat16)
    c["v"], c["out"] = buf, buf
    assert status(gdn2, **c)[0] == "ALIAS"
    c = case()
    big = torch.zeros(2 * 70 * 4 * 64, dtype=torch.bfloat16)
    c["w"] = big[: 70 * 4 * 64].view(70, 4, 64)
    c["out"] = big[70 * 4 * 64 - 8: 2 * 70 * 4 * 64 - 8].view(70, 4, 64)  # overlaps the tail of w
    assert status(gdn2, **c)[0] == "ALIAS"
    c = case()
    c["out"] = torch.zeros(70, 4, 64, dtype=torch.bfloat16)
    assert status(gdn2, **c)[0] == "OK"


def test_no_cpu_path(gdn2):
    c = case()
    with pytest.raises(ValueError):
        gdn2.chunk_fwd(c["q"], c["k"], c["v"])


def test_options_rejected_before_any_device_work(gdn2):
    """A bad options struct is rejected (SHAPE) after the tensor checks pass
    and before anything touches a device (host tensors here)."""
    import ctypes
    lib = gdn2.load_library()
    t = case()
    P = lambda x: None if x is None else ctypes.byref(x)
    for size, split in ((4, 0), (ctypes.sizeof(gdn2.Gdn2FwdOptions), -2)):
        opts = gdn2.Gdn2FwdOptions(size, split)
        descs = [gdn2.describe(t[n]) for n in ("q", "k", "v", "g", "beta", "w")]
        rest = [gdn2.describe(t[n]) for n in ("initial_state", "cu_seqlens", "out", "final_state")]
        rc = lib.gdn2_chunk_fwd_opts(*[P(x) for x in descs], 0.0, *[P(x) for x in rest],
                                     ctypes.byref(opts), None)
        assert rc == -3, (size, split, rc)
        assert "options" in gdn2.last_error()


def test_split_plan(gdn2):
    """The automatic split: whole sequences when the chains fill at least
    half the CUs or are short (under 32 chunks); otherwise segments of about
    sqrt(chunks per sequence), at least 8 chunks."""
    plan = gdn2.split_plan
    assert plan(4096, 1, 16, 256) == 8          # 16 chains x 64 chunks
    assert plan(131072, 2, 16, 256) == 32       # 32 chains x 1024 chunks
    assert plan(65536, 4, 48, 256) == 0         # 192 chains: no split
    assert plan(37517, 8, 32, 256) == 0         # 256 chains
    assert plan(256, 1, 2, 256) == 0            # 4 chunks per chain
    assert plan(31 * 64, 1, 1, 256) == 0 and plan(32 * 64, 1, 1, 256) == 8
    assert plan(0, 1, 1, 256) == 0 and plan(4096, 1, 1, 0) == 0
    for T, N, HV in ((8192, 1, 1), (65536, 1, 4), (1 << 20, 2, 8), (50000, 3, 7)):
        L = plan(T, N, HV, 256)
        avg = -(-(-(-T // 64)) // N)
        assert L >= 8 and abs(L - avg ** 0.5) <= max(1.0, 8 - avg ** 0.5)


def test_recurrent_allows_in_place_state_only(gdn2):
    """gdn2_recurrent_fwd accepts final_state == initial_state (same
    buffer); a partial overlap, and the in-place pair on the chunked entry,
    are ALIAS."""
    import ctypes
    lib = gdn2.load_library()
    t = case()
    P = lambda x: None if x is None else ctypes.byref(x)

    def call(fn, init, final):
        descs = [gdn2.describe(t[n]) for n in ("q", "k", "v", "g", "beta", "w")]
        rest = [gdn2.describe(x) for x in (init, t["cu_seqlens"], t["out"], final)]
        return fn(*[P(x) for x in descs], 0.0, *[P(x) for x in rest])

    s0 = t["initial_state"]
    assert call(lib.gdn2_recurrent_fwd_check, s0, s0) == 0
    assert call(lib.gdn2_chunk_fwd_check, s0, s0) == -7
    big = torch.zeros(2 * s0.numel() + 64)
    a = big[:s0.numel()].view(s0.shape)
    b = big[16:16 + s0.numel()].view(s0.shape)  # shifted by 64 bytes: overlaps a
    assert call(lib.gdn2_recurrent_fwd_check, a, b) == -7
    assert "final_state overlaps initial_state" in gdn2.last_error()


# ------------------------------------------------------------------ backward --
def bwd_case(T=70, N=2, H=2, HV=4, D=64):
    bf = torch.bfloat16
    c = dict(q=torch.zeros(T, H, D, dtype=bf), k=torch.zeros(T, H, D, dtype=bf),
             v=torch.zeros(T, HV, D, dtype=bf), g=torch.zeros(T, HV, D), beta=torch.zeros(T, HV, D, dtype=bf),
             w=torch.zeros(T, HV, D, dtype=bf), d_out=torch.zeros(T, HV, D, dtype=bf),
             initial_state=torch.zeros(N, HV, D, D), d_final_state=torch.zeros(N, HV, D, D),
             cu_seqlens=torch.tensor([0, 30, T][: N + 1] if N == 2 else [0, T], dtype=torch.int32))
    grads = dict(dq=torch.zeros(T, H, D, dtype=bf), dk=torch.zeros(T, H, D, dtype=bf),
                 dv=torch.zeros(T, HV, D, dtype=bf), dw=torch.zeros(T, HV, D, dtype=bf),
                 dbeta=torch.zeros(T, HV, D, dtype=bf), dg=torch.zeros(T, HV, D),
                 d_initial_state=torch.zeros(N, HV, D, D))
    return c, grads


def bwd_status(gdn2, c, grads):
    rc = gdn2.check_bwd(c["q"], c["k"], c["v"], c["g"], c["beta"], c["w"], c["d_out"],
                        initial_state=c["initial_state"], cu_seqlens=c["cu_seqlens"],
                        d_final_state=c["d_final_state"], grads=grads)
    return gdn2.STATUS[rc], gdn2.last_error()


def test_bwd_valid_calls(gdn2):
    c, gr = bwd_case()
    assert bwd_status(gdn2, c, gr) == ("OK", "")
    c, gr = bwd_case(D=128)
    assert bwd_status(gdn2, c, gr)[0] == "OK"
    # fp16 io and 16-bit g (the gradients in the inputs' types)
    for io, gt in ((torch.float16, torch.float32), (torch.bfloat16, torch.bfloat16), (torch.float16, torch.float16)):
        c, gr = bwd_case()
        for n in ("q", "k", "v", "beta", "w", "d_out"):
            c[n] = c[n].to(io)
        for n in ("dq", "dk", "dv", "dw", "dbeta"):
            gr[n] = gr[n].to(io)
        c["g"], gr["dg"] = c["g"].to(gt), gr["dg"].to(gt)
        assert bwd_status(gdn2, c, gr) == ("OK", ""), (io, gt)
    for opt in ("initial_state", "d_final_state"):
        c, gr = bwd_case()
        c[opt] = None
        assert bwd_status(gdn2, c, gr)[0] == "OK", opt
    c, gr = bwd_case()
    gr["d_initial_state"] = None
    assert bwd_status(gdn2, c, gr)[0] == "OK"
    c, gr = bwd_case(T=0)
    assert bwd_status(gdn2, c, gr)[0] == "OK"


@pytest.mark.parametrize("mutate,expect", [
    (lambda c, g: c.update(g=None), "NULL_ARG"),          # the backward needs every gate
    (lambda c, g: c.update(beta=None), "NULL_ARG"),
    (lambda c, g: c.update(w=None), "NULL_ARG"),
    (lambda c, g: c.update(d_out=None), "NULL_ARG"),
    (lambda c, g: g.update(dq=None), "NULL_ARG"),
    (lambda c, g: g.update(dg=None), "NULL_ARG"),
    (lambda c, g: c.update(q=c["q"].half()), "DTYPE"),     # q's type differs from k's
    (lambda c, g: c.update(q=c["q"].float(), k=c["k"].float()), "DTYPE"),  # 16-bit io only
    (lambda c, g: c.update(g=c["g"].double()), "DTYPE"),
    (lambda c, g: c.update(g=c["g"].bfloat16()), "DTYPE"),  # dg must take g's type
    (lambda c, g: c.update(d_out=c["d_out"].float()), "DTYPE"),
    (lambda c, g: g.update(dg=g["dg"].bfloat16()), "DTYPE"),
    (lambda c, g: g.update(dq=g["dq"].half()), "DTYPE"),
    (lambda c, g: g.update(dbeta=g["dbeta"].float()), "DTYPE"),
    (lambda c, g: c.update(initial_state=c["initial_state"].bfloat16()), "DTYPE"),
    (lambda c, g: c.update(d_out=c["d_out"][:60]), "SHAPE"),
    (lambda c, g: g.update(dq=torch.zeros(70, 4, 64, dtype=torch.bfloat16)), "SHAPE"),
    (lambda c, g: g.update(d_initial_state=torch.zeros(3, 4, 64, 64)), "SHAPE"),
    (lambda c, g: c.update(v=torch.zeros(70, 3, 64, dtype=torch.bfloat16)), "HEADS"),
    (lambda c, g: c.update(q=torch.zeros(70, 2, 96, dtype=torch.bfloat16)), "UNSUPPORTED"),
    # the backward takes K == V only (the forward also K != V)
    (lambda c, g: c.update(v=torch.zeros(70, 4, 128, dtype=torch.bfloat16)), "UNSUPPORTED"),
    # strided views are forward-only: the backward takes dense tensors
    (lambda c, g: c.update(q=torch.zeros(70, 2, 128, dtype=torch.bfloat16)[:, :, :64]), "LAYOUT"),
    (lambda c, g: g.update(dv=torch.zeros(70, 64, 4, dtype=torch.bfloat16).transpose(1, 2)), "LAYOUT"),
])
def test_bwd_rejections(gdn2, mutate, expect):
    c, gr = bwd_case()
    mutate(c, gr)
    code, msg = bwd_status(gdn2, c, gr)
    assert code == expect, (code, msg)
    assert msg


def test_bwd_alias_rules(gdn2):
    c, gr = bwd_case()
    gr["dv"] = c["d_out"]
    assert bwd_status(gdn2, c, gr)[0] == "ALIAS"
    c, gr = bwd_case()
    gr["dw"] = gr["dv"]
    assert bwd_status(gdn2, c, gr)[0] == "ALIAS"
    c, gr = bwd_case()
    gr["d_initial_state"] = c["initial_state"]
    assert bwd_status(gdn2, c, gr)[0] == "ALIAS"


def test_bwd_no_cpu_path(gdn2):
    c, _ = bwd_case()
    with pytest.raises(ValueError):
        gdn2.chunk_bwd(c["q"], c["k"], c["v"], c["g"], c["beta"], c["w"], c["d_out"])


def test_noalloc_rejects_oversized_split_before_device_work(gdn2):
    """gdn2_chunk_fwd_noalloc: an explicit segment length whose workspace
    exceeds the fixed scratch array is UNSUPPORTED, with both sizes in the
    message, before any device query (host tensors here)."""
    import ctypes
    lib = gdn2.load_library()
    cap = int(re.search(r"#define GDN2_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
              .group(1)) << 20
    P = lambda x: None if x is None else ctypes.byref(x)
    # 100 one-chunk segments x 16 heads x 3 x 16 KiB = 75 MiB > 64 MiB
    T, H, K = 6400, 16, 64
    t = dict(q=torch.zeros(T, H, K, dtype=torch.bfloat16), k=torch.zeros(T, H, K, dtype=torch.bfloat16),
             v=torch.zeros(T, H, K, dtype=torch.bfloat16), out=torch.zeros(T, H, K, dtype=torch.bfloat16))
    descs = [gdn2.describe(t.get(n)) for n in ("q", "k", "v", "g", "beta", "w")]
    rest = [gdn2.describe(t.get(n)) for n in ("initial_state", "cu_seqlens", "out", "final_state")]
    need = 3 * 1 * H * 100 * K * K * 4
    assert need > cap
    opts = gdn2.make_options(seq_split=1)
    rc = lib.gdn2_chunk_fwd_noalloc(*[P(x) for x in descs], 0.0, *[P(x) for x in rest], ctypes.byref(opts), None)
    assert gdn2.STATUS[rc] == "UNSUPPORTED"
    msg = gdn2.last_error()
    assert str(need) in msg and str(cap) in msg, msg
    # argument errors come first, as for gdn2_chunk_fwd_opts
    bad = gdn2.Gdn2FwdOptions(4, 0)
    rc = lib.gdn2_chunk_fwd_noalloc(*[P(x) for x in descs], 0.0, *[P(x) for x in rest], ctypes.byref(bad), None)
    assert rc == -3 and "options" in gdn2.last_error()
