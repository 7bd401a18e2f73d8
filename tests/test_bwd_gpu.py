"""GPU parity of the backward (gdn2_chunk_bwd through the C ABI) against the
plain-C FP64 backward oracle, on identical bf16-quantised seeded inputs.

Bar, per gradient tensor: relative L2 error <= BWD_REL_L2 and max abs error
<= BWD_MAX_ABS times the tensor's largest reference magnitude. The bound is
looser than the forward's 5e-3 because a gradient passes through up to four
chained bf16-operand products (the forward's output through two) and the
bf16-rounded dq, dk, dv, dw, dbeta themselves carry 2^-9 relative rounding;
errors of independent bf16 roundings add in quadrature, so four products at
the forward's measured ~2.5e-3 each give ~5e-3, doubled for margin.
"""

import sys

import numpy as np
import pytest
import torch

from linear_attention_rnn_gdn2_amd.workloads import synth, synth_cotangents

pytestmark = pytest.mark.gpu

BWD_REL_L2 = 1e-2
BWD_MAX_ABS = 5e-2
GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dw", "d_initial_state")


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


@pytest.fixture(scope="module")
def c_oracle():
    import os
    from oracle.build import LIB, build_c_oracle
    if not os.path.exists(LIB):
        build_c_oracle()
    from oracle.c_oracle import gdn2_recurrence_bwd_c
    return gdn2_recurrence_bwd_c


def case(lengths, H, HV, D, seed, init_std=0.02, g_max=0.1, beta_max=1.0, d_final=True, g_extreme_max=0.0,
         extreme_frac=0.0):
    d = synth(list(lengths), H, HV, D, D, seed, init_std=init_std, g_max=g_max, beta_max=beta_max,
              g_extreme_max=g_extreme_max, extreme_frac=extreme_frac)
    T, N = sum(lengths), len(lengths)
    d["d_out"], d["d_final_state"] = synth_cotangents(T, N, HV, D, D, seed, d_final=d_final)
    return d


def run_both(gdn2, c_oracle, d, tag):
    dev = torch.device("cuda:0")
    g = {n: d[n].to(dev) for n in ("q", "k", "v", "g", "beta", "w", "d_out")}
    s0 = None if d["initial_state"] is None else d["initial_state"].to(dev)
    dht = None if d["d_final_state"] is None else d["d_final_state"].to(dev)
    say(f"[bwd] {tag}: GPU")
    got = gdn2.chunk_bwd(g["q"], g["k"], g["v"], g["g"], g["beta"], g["w"], g["d_out"], scale=d["scale"],
                         initial_state=s0, cu_seqlens=d["cu_seqlens"].to(dev), d_final_state=dht)
    torch.cuda.synchronize()
    say(f"[bwd] {tag}: oracle")
    ref = c_oracle(d["q"], d["k"], d["v"], d["g"], d["beta"], d["w"], d["scale"], d["initial_state"],
                   d["cu_seqlens"].numpy(), d["d_out"], d["d_final_state"])
    return {n: got[n].float().cpu().double().numpy() for n in GRADS}, ref


def errors(got, ref):
    """Per gradient: relative L2 error and max-abs error over the largest
    reference magnitude. A reference that is identically zero (dg and dbeta
    of one-token sequences entered from a zero state vanish exactly: every
    term meets the zero state) has no scale of its own; the GPU's float32
    rounding residue there is measured against the largest reference
    magnitude of any gradient of the case (as RMS for the first figure)."""
    res = {}
    scale = max((float(np.max(np.abs(ref[n]))) for n in GRADS if ref[n].size), default=0.0) or 1.0
    for n in GRADS:
        a, b = got[n], ref[n]
        nb = np.linalg.norm(b)
        rel = np.linalg.norm(a - b) / nb if nb > 0 else np.linalg.norm(a - b) / (scale * np.sqrt(max(b.size, 1)))
        bm = float(np.max(np.abs(b))) if b.size else 0.0
        mx = np.max(np.abs(a - b)) / (bm if bm > 0 else scale) if b.size else 0.0
        res[n] = (rel, mx)
    return res


def assert_parity(got, ref, tag):
    errs = errors(got, ref)
    say(f"[bwd] {tag}: " + ", ".join(f"{n} rel-L2 {r:.2e} max {m:.2e}" for n, (r, m) in errs.items()))
    for n, (r, m) in errs.items():
        assert np.isfinite(got[n]).all(), f"{tag}: {n} not finite"
        assert r <= BWD_REL_L2, f"{tag}: {n} rel-L2 {r:.3e}"
        assert m <= BWD_MAX_ABS, f"{tag}: {n} max-abs/ref-max {m:.3e}"


@pytest.mark.parametrize("lengths,H,HV,D", [
    ((256,), 2, 2, 64),                          # one sequence, whole chunks
    ((65, 0, 1, 130, 64, 63), 2, 4, 128),        # ragged varlen, empty and 1-token sequences, grouped heads
    ((200, 77), 1, 3, 64),                       # three value heads per q/k head
    ((1000,), 4, 4, 128),                        # 16 chunks with a ragged tail
    ((4096,), 2, 2, 64),                         # few long chains: the recompute runs split
    ((3000, 2100), 1, 2, 128),                   # split recompute, ragged segments
])
def test_bwd_matches_oracle(lib, c_oracle, lengths, H, HV, D):
    d = case(lengths, H, HV, D, seed=sum(lengths) + D)
    got, ref = run_both(lib, c_oracle, d, f"lengths {lengths} H {H} HV {HV} D {D}")
    assert_parity(got, ref, f"{lengths}")


def test_bwd_defaults_and_strong_gates(lib, c_oracle):
    """Zero initial state and no final-state gradient; beta up to 2 and
    stronger decay (g = -U(0, 1) per token)."""
    d = case((190, 70), 2, 2, 128, seed=5, init_std=None, g_max=1.0, beta_max=2.0, d_final=False)
    got, ref = run_both(lib, c_oracle, d, "defaults, strong gates")
    assert_parity(got, ref, "defaults, strong gates")


def test_bwd_one_token_sequences_from_zero_state(lib, c_oracle):
    """One-token sequences entered from a zero state, fp16 io, bf16 g, beta
    up to 2 and strong-decay channels: the exact dg and dbeta vanish (every
    term meets the zero state), and the GPU's are zero or float32 rounding
    residue; the other gradients meet the bar as usual."""
    d = case((1, 0, 1, 0), 1, 1, 64, seed=132, init_std=None, beta_max=2.0, g_extreme_max=8.0, extreme_frac=0.1)
    for n in ("q", "k", "v", "beta", "w", "d_out"):
        d[n] = d[n].float().half()
    d["g"] = d["g"].to(torch.bfloat16)
    got, ref = run_both(lib, c_oracle, d, "one-token sequences from a zero state")
    assert np.max(np.abs(ref["dg"])) == 0.0 and np.max(np.abs(ref["dbeta"])) == 0.0
    assert np.max(np.abs(got["dg"])) <= 1e-5 and np.max(np.abs(got["dbeta"])) <= 1e-5
    assert_parity(got, ref, "one-token sequences from a zero state")


def test_bwd_deterministic(lib):
    d = case((300,), 2, 2, 64, seed=9)
    dev = torch.device("cuda:0")
    args = [d[n].to(dev) for n in ("q", "k", "v", "g", "beta", "w", "d_out")]
    kw = dict(scale=d["scale"], initial_state=d["initial_state"].to(dev), cu_seqlens=d["cu_seqlens"].to(dev),
              d_final_state=d["d_final_state"].to(dev))
    a = lib.chunk_bwd(*args, **kw)
    b = lib.chunk_bwd(*args, **kw)
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_strong_decay_every_channel(lib, c_oracle, D):
    """g = -3 per token on every channel of the first sequence: every
    channel of its chunks leaves the single-reference range (|G| up to 192
    nats), so every channel takes the exact per-pair path, in batches; the
    gradients are finite and match the oracle, and the second sequence
    (ordinary decay) is unaffected."""
    d = case((64, 150, 64), 1, 2, D, seed=13 + D, beta_max=2.0)
    d["g"][:64] = -3.0
    d["g"][214:] = -3.0
    got, ref = run_both(lib, c_oracle, d, f"g = -3 on every channel, D {D}")
    assert_parity(got, ref, f"strong decay D {D}")


@pytest.mark.parametrize("g_ext,frac,D", [(8.0, 0.1, 128), (8.0, 0.5, 128), (40.0, 0.1, 128), (300.0, 0.1, 128),
                                          (8.0, 0.1, 64)])
def test_bwd_extreme_channels(lib, c_oracle, g_ext, frac, D):
    """Per-channel extreme decay (a fraction of the channels draw
    g = -U(0, g_ext) per token) with beta up to 2, ragged lengths and grouped
    heads: the flagged channels' exact share and the ordinary channels'
    products meet in the same chunk."""
    d = case((500, 0, 64, 130), 2, 4, D, seed=int(g_ext) + D + int(100 * frac), beta_max=2.0, g_extreme_max=g_ext,
             extreme_frac=frac)
    got, ref = run_both(lib, c_oracle, d, f"extreme channels g_ext {g_ext} frac {frac} D {D}")
    assert_parity(got, ref, f"extreme channels {g_ext} {frac} {D}")


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_bwd_full_size_workloads(lib, c_oracle, wid):
    """The single-sequence (H16), varlen (H32, the headline shape),
    grouped-value-head (HV48) and long-context extreme-decay workloads at
    full size, every element against the plain-C oracle."""
    from linear_attention_rnn_gdn2_amd.workloads import make_inputs
    d = make_inputs(wid)
    T, N = int(d["cu_seqlens"][-1]), len(d["lengths"])
    wl = d["workload"]
    d["d_out"], d["d_final_state"] = synth_cotangents(T, N, wl.HV, wl.K, wl.V, wid)
    got, ref = run_both(lib, c_oracle, d, f"workload {wl.name}")
    assert_parity(got, ref, wl.name)


def test_bwd_empty_batch_passes_state_gradient_through(lib):
    """Every sequence empty (T = 0): no chunk anywhere, so the initial state's
    gradient is the final state's."""
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    N, H, HV, D = 3, 2, 2, 64
    z3 = lambda *s, dt=bf: torch.zeros(*s, dtype=dt, device=dev)
    dht = torch.randn(N, HV, D, D, device=dev)
    cu = torch.zeros(N + 1, dtype=torch.int32, device=dev)
    got = lib.chunk_bwd(z3(0, H, D), z3(0, H, D), z3(0, HV, D), z3(0, HV, D, dt=torch.float32), z3(0, HV, D),
                        z3(0, HV, D), z3(0, HV, D), initial_state=torch.zeros(N, HV, D, D, device=dev),
                        cu_seqlens=cu, d_final_state=dht)
    torch.cuda.synchronize()
    assert torch.equal(got["d_initial_state"], dht)


def test_bwd_int64_cu_default_scale_no_initial_gradient(lib, c_oracle):
    """int64 cu_seqlens, scale left to its default 1/sqrt(K), no initial
    state and d_initial_state not requested; one sequence without
    cu_seqlens."""
    d = case((70, 150), 1, 2, 64, seed=21, init_std=None)
    dev = torch.device("cuda:0")
    g = [d[n].to(dev) for n in ("q", "k", "v", "g", "beta", "w", "d_out")]
    got = lib.chunk_bwd(*g, scale=None, cu_seqlens=d["cu_seqlens"].to(torch.int64).to(dev),
                        d_final_state=d["d_final_state"].to(dev), need_d_initial_state=False)
    torch.cuda.synchronize()
    assert got["d_initial_state"] is None
    ref = c_oracle(d["q"], d["k"], d["v"], d["g"], d["beta"], d["w"], None, None, d["cu_seqlens"].numpy(),
                   d["d_out"], d["d_final_state"])
    gotn = {n: got[n].float().cpu().double().numpy() for n in GRADS if n != "d_initial_state"}
    gotn["d_initial_state"] = ref["d_initial_state"]  # not produced; compared by the others
    assert_parity(gotn, ref, "int64 cu, default scale")
    # one sequence, no cu_seqlens
    d1 = case((190,), 2, 2, 64, seed=22)
    got1 = lib.chunk_bwd(*[d1[n].to(dev) for n in ("q", "k", "v", "g", "beta", "w", "d_out")], scale=d1["scale"],
                         initial_state=d1["initial_state"].to(dev), d_final_state=d1["d_final_state"].to(dev))
    torch.cuda.synchronize()
    ref1 = c_oracle(d1["q"], d1["k"], d1["v"], d1["g"], d1["beta"], d1["w"], d1["scale"], d1["initial_state"], None,
                    d1["d_out"], d1["d_final_state"])
    assert_parity({n: got1[n].float().cpu().double().numpy() for n in GRADS}, ref1, "no cu_seqlens")


@pytest.mark.parametrize("io,gt", [(torch.float16, torch.float32), (torch.bfloat16, torch.bfloat16),
                                   (torch.float16, torch.float16), (torch.bfloat16, torch.float16)])
@pytest.mark.parametrize("D", [64, 128])
def test_bwd_input_types(lib, c_oracle, io, gt, D):
    """fp16 or bf16 q, k, v, beta, w, d_out with float32, bf16 or fp16 g
    (the Flash-GDN-2 README's training paragraph: FP16/BF16 Q/K/V,
    half/FP32 gates), ragged lengths, grouped heads, beta up to 2, and a
    tenth of the channels at strong decay: the oracle differentiates the
    same quantised values, and the gradients come back in the inputs' types
    (dg in g's)."""
    d = case((65, 0, 1, 300, 64), 2, 4, D, seed=31 + D, beta_max=2.0, g_extreme_max=8.0, extreme_frac=0.1)
    for n in ("q", "k", "v", "beta", "w", "d_out"):
        d[n] = d[n].float().to(io)
    d["g"] = d["g"].to(gt)
    dev = torch.device("cuda:0")
    args = [d[n].to(dev) for n in ("q", "k", "v", "g", "beta", "w", "d_out")]
    tag = f"io {io} g {gt} D {D}"
    say(f"[bwd] {tag}: GPU")
    got = lib.chunk_bwd(*args, scale=d["scale"], initial_state=d["initial_state"].to(dev),
                        cu_seqlens=d["cu_seqlens"].to(dev), d_final_state=d["d_final_state"].to(dev))
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv", "dw", "dbeta"):
        assert got[n].dtype == io, (n, got[n].dtype)
    assert got["dg"].dtype == gt and got["d_initial_state"].dtype == torch.float32
    say(f"[bwd] {tag}: oracle")
    ref = c_oracle(d["q"], d["k"], d["v"], d["g"], d["beta"], d["w"], d["scale"], d["initial_state"],
                   d["cu_seqlens"].numpy(), d["d_out"], d["d_final_state"])
    assert_parity({n: got[n].float().cpu().double().numpy() for n in GRADS}, ref, tag)


@pytest.mark.parametrize("lengths", [(700, 0, 65, 1, 300, 129),
                                     (0, 513, 0, 0, 64, 0)])  # the shorter half: empty sequences only
def test_bwd_two_groups_match_per_sequence_calls(lib, c_oracle, lengths):
    """With whole sequences and between half of the compute units and all of
    them in (sequence, value head) chains, the backward runs the longer half
    of the sequences on the call's stream and the shorter half on a second
    one. Every chain's arithmetic is its own either way, so each sequence's
    gradients equal those of a call with that sequence alone, bit for bit
    (ragged, 1-token and empty sequences, grouped heads, a tenth of the
    channels at strong decay; a batch whose shorter half holds no chunk at
    all); and the batch matches the oracle."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    N, T = len(lengths), sum(lengths)
    HV = 2 * max(1, ncu // (2 * N))
    H = HV // 2
    if not (2 * N * HV > ncu and N * HV <= ncu and lib.split_plan(T, N, HV, ncu) == 0):
        pytest.skip(f"{ncu} compute units: no shape of {N} sequences runs as two groups")
    say(f"[bwd two groups] {ncu} CUs, lengths {lengths}, H {H}, HV {HV}")
    d = case(lengths, H, HV, 64, seed=77 + lengths[0], beta_max=2.0, g_extreme_max=8.0, extreme_frac=0.1)
    dev = torch.device("cuda:0")
    names = ("q", "k", "v", "g", "beta", "w", "d_out")
    got = lib.chunk_bwd(*[d[n].to(dev) for n in names], scale=d["scale"], initial_state=d["initial_state"].to(dev),
                        cu_seqlens=d["cu_seqlens"].to(dev), d_final_state=d["d_final_state"].to(dev))
    torch.cuda.synchronize()
    cu = d["cu_seqlens"].tolist()
    for i in range(N):
        b, e = cu[i], cu[i + 1]
        if e == b:  # no chunk: the state gradient passes through
            assert torch.equal(got["d_initial_state"][i].cpu(), d["d_final_state"][i])
            continue
        one = lib.chunk_bwd(*[d[n][b:e].to(dev) for n in names], scale=d["scale"],
                            initial_state=d["initial_state"][i:i + 1].to(dev),
                            d_final_state=d["d_final_state"][i:i + 1].to(dev))
        torch.cuda.synchronize()
        for n in GRADS:
            part = got[n][i:i + 1] if n == "d_initial_state" else got[n][b:e]
            assert torch.equal(part, one[n]), f"sequence {i} ({e - b} tokens): {n} differs"
    say("[bwd two groups] oracle")
    ref = c_oracle(d["q"], d["k"], d["v"], d["g"], d["beta"], d["w"], d["scale"], d["initial_state"],
                   d["cu_seqlens"].numpy(), d["d_out"], d["d_final_state"])
    assert_parity({n: got[n].float().cpu().double().numpy() for n in GRADS}, ref, "two groups")


def test_bwd_two_groups_from_two_host_threads(lib):
    """Two host threads, each on its own stream, enqueue backward calls in
    the two-group regime at the same time: both share the device's second
    stream, whose fork and join each call enqueues under a lock. Every
    result equals the same call's result made alone, bit for bit."""
    import threading
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    lengths = (300, 65, 0, 200, 1, 129)
    N, T = len(lengths), sum(lengths)
    HV = 2 * max(1, ncu // (2 * N))
    if not (2 * N * HV > ncu and N * HV <= ncu and lib.split_plan(T, N, HV, ncu) == 0):
        pytest.skip(f"{ncu} compute units: no shape of {N} sequences runs as two groups")
    dev = torch.device("cuda:0")
    names = ("q", "k", "v", "g", "beta", "w", "d_out")
    cases = []
    for seed in (41, 42):
        d = case(lengths, HV // 2, HV, 64, seed=seed)
        cases.append(([d[n].to(dev) for n in names],
                      dict(scale=d["scale"], initial_state=d["initial_state"].to(dev),
                           cu_seqlens=d["cu_seqlens"].to(dev), d_final_state=d["d_final_state"].to(dev))))
    alone = [lib.chunk_bwd(*a, **kw) for a, kw in cases]
    torch.cuda.synchronize()
    results, errors_seen = [[None] * 3, [None] * 3], []

    def worker(i):
        try:
            s = torch.cuda.Stream(device=dev)
            a, kw = cases[i]
            with torch.cuda.stream(s):
                for r in range(3):
                    results[i][r] = lib.chunk_bwd(*a, **kw)
            s.synchronize()
        except Exception as e:  # reported below, in the test's thread
            errors_seen.append(repr(e))

    say(f"[bwd two threads] N {N}, HV {HV}: two threads, three calls each")
    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join(timeout=120)
    torch.cuda.synchronize()
    assert not errors_seen, errors_seen
    for i in range(2):
        for r in range(3):
            for n in GRADS:
                assert torch.equal(results[i][r][n], alone[i][n]), f"thread {i} call {r}: {n} differs"
