"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Bit-exact: top-k ids, the permutation (expert offsets, sorted routes, inverse
positions) and dequantized weight values. Routing weights: within 4 fp32 ulps
of the oracle's softmax. Outputs: the G1-or-G2 tolerance of tests/tolerance.py.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import qmoe_inputs as qi
from tests.gpu_util import DEV, fp32_ulps, layer_for, oracle_acc, run, sample_rows, say
from tests.tolerance import compare

pytestmark = pytest.mark.gpu

FORMATS = [(b, bs) for b in (4, 3, 2) for bs in (32, 64, 128)]


def small_spec(bits, bs, act="bf16", **kw):
    d = dict(hidden=256, inter=128, num_experts=8, top_k=2, bits=bits, block_size=bs,
             zero_point=1 << (bits - 1), scale_c=0.03, act_dtype=act)
    d.update(kw)
    return qi.LayerSpec(**d)


# ------------------------------------------------------------------ dequant

@pytest.mark.parametrize("bits,bs", FORMATS)
def test_dequant_bit_exact_small(bits, bs):
    wl = qi.make_layer(small_spec(bits, bs), T=1, seed=bits * 100 + bs)
    layer = layer_for(wl, 16)
    s = wl.spec
    for fc, e in ((1, 0), (2, 7), (1, 5)):
        f32, b16 = layer.dequant(fc, e)
        torch.cuda.synchronize()
        K = s.hidden if fc == 1 else s.inter
        codes = wl.weights.fc1_codes[e] if fc == 1 else wl.weights.fc2_codes[e]
        scales = wl.weights.fc1_scales[e] if fc == 1 else wl.weights.fc2_scales[e]
        ref = oracle.dequant(codes, scales, bits, bs, s.zero_point, K)
        assert np.array_equal(f32.cpu().numpy().astype(np.float64), ref)
        got = b16.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, oracle.dequant_f16(codes, scales, bits, bs, s.zero_point, K))


@pytest.mark.parametrize("name", ["decode", "int3", "stack"])
def test_dequant_bit_exact_full_shape(name):
    wl = qi.make_workload(name, T=1)
    layer = layer_for(wl, 16)
    s = wl.spec
    for fc, e in ((1, 3), (2, 127)):
        f32, b16 = layer.dequant(fc, e)
        torch.cuda.synchronize()
        K = s.hidden if fc == 1 else s.inter
        codes = wl.weights.fc1_codes[e] if fc == 1 else wl.weights.fc2_codes[e]
        scales = wl.weights.fc1_scales[e] if fc == 1 else wl.weights.fc2_scales[e]
        ref = oracle.dequant(codes, scales, s.bits, s.block_size, s.zero_point, K)
        assert np.array_equal(f32.cpu().numpy().astype(np.float64), ref)
        got = b16.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, oracle.dequant_f16(codes, scales, s.bits, s.block_size,
                                                      s.zero_point, K))


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_dequant_f16_every_scale_pattern(bits):
    """The prefill GEMM's fp16 weight operand (the routine its staging calls,
    exported) against the oracle's fp16((q - zp) * s) for all 65,536 fp16
    scale patterns (subnormals, infinities and NaN included), every code,
    and per-block zero points covering every code: bit for bit (NaN
    position for NaN)."""
    spec = small_spec(bits, 32, hidden=256, inter=4096, num_experts=2)
    wl = qi.make_layer(spec, T=1, seed=bits)
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    sc1 = allh.reshape(1, 2 * 4096, 8)
    sc1 = np.concatenate([sc1, sc1[:, ::-1]], axis=0).copy()       # [2, 8192, 8]
    rng = np.random.default_rng(bits)
    z1 = rng.integers(0, 1 << bits, size=sc1.shape).astype(np.uint8)
    w = qi.LayerWeights(wl.weights.fc1_codes, sc1, wl.weights.fc2_codes, wl.weights.fc2_scales)
    wl2 = qi.Workload("scales", spec, wl.tokens, w)
    for zps in (None, z1):
        layer = layer_for(wl2, 4, fc1_zero_points=zps,
                          fc2_zero_points=None if zps is None else random_zero_points(wl2, 1)[1])
        for e in (0, 1):
            _, b16 = layer.dequant(1, e)
            torch.cuda.synchronize()
            got = b16.view(torch.int16).cpu().numpy().view(np.uint16)
            ref = oracle.dequant_f16(w.fc1_codes[e], sc1[e], bits, 32, spec.zero_point, 256,
                                     zero_points=None if zps is None else zps[e])
            nan = np.isnan(ref.view(np.float16))
            assert np.array_equal(np.isnan(got.view(np.float16)), nan)
            assert np.array_equal(got[~nan], ref[~nan])


def random_zero_points(wl, seed):
    rng = np.random.default_rng(seed)
    hi = 1 << wl.spec.bits
    return (rng.integers(0, hi, size=wl.weights.fc1_scales.shape).astype(np.uint8),
            rng.integers(0, hi, size=wl.weights.fc2_scales.shape).astype(np.uint8))


@pytest.mark.parametrize("bits,bs", FORMATS)
def test_dequant_zero_point_tensor_bit_exact(bits, bs):
    """With per-block zero-point tensors the exported dequantized weights are
    (q - zp[n][k/bs]) * s exactly in fp32, and fp16 of it as the prefill's
    operand."""
    wl = qi.make_layer(small_spec(bits, bs), T=1, seed=bits * 10 + bs)
    z1, z2 = random_zero_points(wl, bits + bs)
    layer = layer_for(wl, 16, fc1_zero_points=z1, fc2_zero_points=z2)
    s = wl.spec
    for fc, e in ((1, 0), (2, 7), (1, 5)):
        f32, b16 = layer.dequant(fc, e)
        torch.cuda.synchronize()
        K = s.hidden if fc == 1 else s.inter
        codes = wl.weights.fc1_codes[e] if fc == 1 else wl.weights.fc2_codes[e]
        scales = wl.weights.fc1_scales[e] if fc == 1 else wl.weights.fc2_scales[e]
        z = z1[e] if fc == 1 else z2[e]
        ref = oracle.dequant(codes, scales, bits, bs, s.zero_point, K, zero_points=z)
        assert np.array_equal(f32.cpu().numpy().astype(np.float64), ref)
        got = b16.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, oracle.dequant_f16(codes, scales, bits, bs, s.zero_point, K,
                                                      zero_points=z))


# ------------------------------------------------------------------ routing

def check_routing(wl, layer):
    T, k, E = wl.tokens.x.shape[0], wl.spec.top_k, wl.spec.num_experts
    ids, w, offs, srt, inv = layer.route(wl.tokens.logits.to(DEV))
    torch.cuda.synchronize()
    rid, rw = oracle.route(wl.tokens.logits, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    ulps = fp32_ulps(w.cpu().numpy(), rw.astype(np.float32))
    assert ulps.max() <= 4, ulps.max()
    counts, roffs, rsrt, rinv = oracle.permute(rid, E)
    assert np.array_equal(offs.cpu().numpy(), roffs)
    assert np.array_equal(srt.cpu().numpy(), rsrt)
    assert np.array_equal(inv.cpu().numpy(), rinv)
    return counts


@pytest.mark.parametrize("name,T", [("tiny", 4), ("decode", 1), ("decode", 4), ("prefill", 8192),
                                    ("int3", 2048), ("stack", 32768), ("prefill", 777),
                                    ("decode", 13), ("decode", 32), ("prefill", 256), ("stack", 100)])
def test_routing_bit_exact(name, T):
    """qmoe_route runs the routing a forward of T tokens would run: the
    chunked launches of the grouped GEMMs, or (13 to 256 tokens here) the
    small-batch path's one-launch routing."""
    say(f"routing {name} T={T}")
    wl = qi.make_workload(name, T=T)
    layer = layer_for(wl, max(T, 8))
    counts = check_routing(wl, layer)
    assert counts.sum() == T * wl.spec.top_k


@pytest.mark.parametrize("kw,T", [
    (dict(act="f16"), 40), (dict(act="f32"), 8), (dict(num_experts=1024, top_k=8), 40),
    (dict(num_experts=1024, top_k=8), 100), (dict(num_experts=128, top_k=32), 100),
    (dict(num_experts=64, top_k=1), 256), (dict(num_experts=300, top_k=5), 77)])
def test_small_routing_bit_exact(kw, T):
    """The small-batch path's one-launch routing (and, where the route list
    outgrows it, E = 1024 at 100 tokens, the chunked routing) for fp16 and
    fp32 logits, up to 1024 experts and top-32: ids, offsets, sorted routes
    and inverse positions bit-exact, weights within 4 ulp; the layer's output
    matches the oracle on sampled rows."""
    d = dict(num_experts=8, top_k=2)
    d.update(kw)
    act = d.pop("act", "bf16")
    spec = small_spec(4, 32, act=act, **d)
    wl = qi.make_layer(spec, T=T, seed=1000 + T + spec.num_experts + spec.top_k)
    say(f"small routing E={spec.num_experts} k={spec.top_k} act={act} T={T}")
    with _env(QMOE_FORCE_PATH="small"):
        layer = layer_for(wl, 256)
    check_routing(wl, layer)
    rows = sample_rows(T, 12, seed=T)
    out, _ = run(layer, wl.tokens.x, wl.tokens.logits)
    rep = compare(out[torch.as_tensor(rows, device=DEV)], oracle_acc(wl, rows))
    say(f"  output on {len(rows)} rows: {rep}")
    assert rep.ok, rep


@pytest.mark.parametrize("E,k", [(1, 1), (8, 8), (2, 1)])
@pytest.mark.parametrize("T", [1, 4, 9, 40, 300])
def test_degenerate_expert_counts(E, k, T):
    """One expert for every token (E = k = 1), every expert for every token
    (k = E, whose routing weights are the plain softmax of all logits) and
    top-1 of two, on each path the default dispatch takes (fused decode,
    grouped decode, small-batch path, grouped GEMMs): routing bit-exact and
    the output matches the oracle."""
    spec = small_spec(4, 32, num_experts=E, top_k=k)
    wl = qi.make_layer(spec, T=T, seed=500 + 10 * E + k + T)
    layer = layer_for(wl, 300)
    out, ws = run(layer, wl.tokens.x, wl.tokens.logits)
    ids, _ = layer.routing_from_workspace(T, ws)
    rid, _ = oracle.route(wl.tokens.logits, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    rep = compare(out, oracle_acc(wl))
    say(f"E={E} k={k} T={T}: {rep}")
    assert rep.ok, rep


def test_routing_constructed_ties():
    wl = qi.make_workload("decode", T=64)
    l = wl.tokens.logits.clone()
    l[0, :] = 0.5                       # every logit equal: experts 0..7 in order
    l[1, ::2] = 1.0                     # even experts tie at the top
    l[2, :] = -0.0
    l[2, 5] = 0.0                       # -0 and +0 compare equal: lowest indices win
    l[3, :] = torch.arange(128).flip(0).to(l.dtype) * 0   # zeros
    wl.tokens.logits = l
    layer = layer_for(wl, 64)
    check_routing(wl, layer)


# ------------------------------------------------------------------ decode path

# The decode paths compute in fp32 and differ from the oracle's double sums by
# reordering; h enters FC2 with 16 significant bits (bf16 hi + lo) in the
# fused decode. An element of y sums I terms W2[m,n] h[n]: a relative error
# 2^-17 per h value moves it by about 2^-17 * sqrt(I) (about 2^-12.2 at
# I = 768) of the row's root mean square. Elements beyond 2 bf16 ulps must
# therefore stay within 2^-11 of their row's rms (they are the near-zero
# outputs, where 2 ulps is a tiny absolute error).
DECODE_OUTLIER_BOUND = 2.0 ** -11


def check_decode(wl, layer):
    T = wl.tokens.x.shape[0]
    out, ws = run(layer, wl.tokens.x, wl.tokens.logits)
    ids, w = layer.routing_from_workspace(T, ws)
    rid, rw = oracle.route(wl.tokens.logits, wl.spec.top_k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert fp32_ulps(w.cpu().numpy(), rw.astype(np.float32)).max() <= 4
    rep = compare(out, oracle_acc(wl))
    say(f"decode {wl.name} T={T}: {rep}")
    assert rep.ok, rep
    assert rep.outlier_rel <= DECODE_OUTLIER_BOUND, rep
    return out


@pytest.mark.parametrize("name,T", [("tiny", 4), ("tiny", 1), ("decode", 1), ("decode", 2),
                                    ("decode", 4), ("int3", 4), ("stack", 1), ("stack", 4)])
def test_decode_parity(name, T):
    wl = qi.make_workload(name, T=T)
    check_decode(wl, layer_for(wl, 16))


@pytest.mark.parametrize("bits,bs", FORMATS)
def test_decode_parity_formats(bits, bs):
    wl = qi.make_layer(small_spec(bits, bs), T=3, seed=7 + bits + bs)
    check_decode(wl, layer_for(wl, 16))


def test_decode_fp32_activations_formats():
    for bits, bs in ((3, 64), (2, 128)):
        wl = qi.make_layer(small_spec(bits, bs, act="f32"), T=4, seed=3 + bits)
        check_decode(wl, layer_for(wl, 16))


@pytest.mark.parametrize("name,T", [("decode", 1), ("decode", 4), ("int3", 4), ("stack", 1)])
def test_fused_decode_matches_split_decode(name, T):
    """The single-launch decode and the two-kernel decode compute the same
    layer in fp32 with different summation orders."""
    wl = qi.make_workload(name, T=T)
    a = check_decode(wl, layer_for(wl, 16))
    os.environ["QMOE_FORCE_PATH"] = "decode_split"
    try:
        ls = layer_for(wl, 16)
    finally:
        del os.environ["QMOE_FORCE_PATH"]
    b = check_decode(wl, ls)
    d = (a.float() - b.float()).abs().max().item()
    scale = a.float().abs().max().item()
    assert d <= 2 ** -7 * scale, (d, scale)


def test_decode_back_to_back_calls_reuse_sync_state():
    """The fused decode's exchange entries carry a per-call epoch and all data
    crossing workgroups goes through coherent loads and stores. One handle
    alternates three different inputs (different x, logits and token
    counts), so an entry left over from the previous call would hold a value
    of another input; every call must equal that input's own first result
    bit for bit. The same sequence runs again on a handle whose epoch
    counter wraps in the middle of it."""
    wl = qi.make_workload("decode", T=4)
    inputs = []
    for T, seed in ((4, 201), (1, 202), (3, 203)):
        t = qi.draw_tokens(wl.spec, T, np.random.default_rng(seed))
        inputs.append((t.x.to(DEV), t.logits.to(DEV)))
    ref_layer = layer_for(wl, 16)
    refs = []
    for x, g in inputs:
        refs.append(ref_layer(x, g).clone())
        torch.cuda.synchronize()
    assert not torch.equal(refs[0][:1], refs[1])
    with _env(QMOE_FUSED_EPOCH_START=2 ** 32 - 30):
        wrapping = layer_for(wl, 16)
    for L in (layer_for(wl, 16), wrapping):
        outs = []
        for r in range(60):
            i = r % 3
            outs.append((i, L(inputs[i][0], inputs[i][1])))
        torch.cuda.synchronize()
        for i, o in outs:
            assert torch.equal(o.view(torch.int16), refs[i].view(torch.int16)), i
        # no bounded wait of the fused decode ran out in any of these calls
        assert L.decode_errors() == 0


@pytest.mark.parametrize("T,force", [(4, "decode_split"), (12, "small"), (300, "prefill")])
def test_graph_capture_replays(T, force):
    """A forward captured in a HIP graph (torch.cuda.CUDAGraph) on a layer
    whose eager calls of up to four tokens take the fused decode: under
    capture the call takes the paths without cross-workgroup exchange (split
    decode up to four tokens; the grouped paths above), so every replay, with new inputs copied in
    between and eager work and synchronizations between the replays, equals
    an eager run of that path on the same inputs bit for bit, and meets the
    tolerance against the oracle."""
    wl = qi.make_workload("decode", T=T)
    L = layer_for(wl, max(T, 16))
    with _env(QMOE_FORCE_PATH=force):
        Lref = layer_for(wl, max(T, 16))
    x_in = torch.empty((T, wl.spec.hidden), dtype=torch.bfloat16, device=DEV)
    g_in = torch.empty((T, wl.spec.num_experts), dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(x_in)
    ws = torch.empty(L.workspace_size(T), dtype=torch.uint8, device=DEV)
    x_in.copy_(wl.tokens.x.to(DEV))
    g_in.copy_(wl.tokens.logits.to(DEV))
    L(x_in, g_in, out=out, workspace=ws)            # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        L(x_in, g_in, out=out, workspace=ws)
    torch.cuda.synchronize()
    say(f"graph capture T={T}: replays")
    for rep in range(4):
        t = qi.draw_tokens(wl.spec, T, np.random.default_rng(300 + rep), nseq=max(1, T // 50))
        x_in.copy_(t.x.to(DEV))
        g_in.copy_(t.logits.to(DEV))
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = Lref(t.x.to(DEV), t.logits.to(DEV))
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), rep
        if rep % 2 == 0:
            sub = qi.Workload("graph", wl.spec, t, wl.weights)
            rows = None if T <= 12 else sample_rows(T, 12, seed=rep)
            acc = oracle_acc(sub, rows)
            rep_ = compare(got if rows is None else got[torch.as_tensor(rows, device=DEV)], acc)
            assert rep_.ok, rep_


class _env:
    """Set environment variables while a layer is created (the library reads
    them once, at create)."""

    def __init__(self, **kv):
        self.kv = kv

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kv}
        os.environ.update({k: str(v) for k, v in self.kv.items()})

    def __exit__(self, *exc):
        for k, v in self.old.items():
            if v is None:
                del os.environ[k]
            else:
                os.environ[k] = v


@pytest.mark.parametrize("name,T", [("decode", 4), ("int3", 4), ("stack", 1)])
def test_fused_decode_schedule_independent(name, T):
    """Every output element of the fused decode is computed by the same
    arithmetic whatever the grid: with 1, 7, 16 or 40 workgroups (more
    experts than workgroups, whole experts per workgroup, many FC1/FC2 chunks
    per wave) the output equals the full-grid output bit for bit, twice in a
    row on the same layer."""
    wl = qi.make_workload(name, T=T)
    ref = check_decode(wl, layer_for(wl, 16))
    x, g = wl.tokens.x.to(DEV), wl.tokens.logits.to(DEV)
    for grid in (1, 7, 16, 40):
        with _env(QMOE_FUSED_GRID=grid):
            L = layer_for(wl, 16)
        for rep in range(2):
            out = L(x, g)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (grid, rep)
        assert L.decode_errors() == 0, grid


def test_fused_decode_epoch_wrap():
    """The fused decode tags every exchanged value with the call's epoch. A
    handle whose epoch counter starts just below the 32-bit wrap takes the
    wrap path on its second call (the exchange buffer is zeroed again and
    the epochs restart at 1); every call still equals the reference bit for
    bit."""
    wl = qi.make_workload("decode", T=4)
    ref = check_decode(wl, layer_for(wl, 16))
    x, g = wl.tokens.x.to(DEV), wl.tokens.logits.to(DEV)
    with _env(QMOE_FUSED_EPOCH_START=2 ** 32 - 2):
        L = layer_for(wl, 16)
    for rep in range(4):
        out = L(x, g)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
    assert L.decode_errors() == 0


def test_fused_decode_reports_waits_that_run_out():
    """The fused decode's waits for another workgroup's h or y are bounded.
    With the bound set from the host to one poll, consumers give up on
    results that have not arrived yet: every kernel still finishes, and the
    handle reports the waits that ran out in its error bits (bit 0: h,
    bit 1: y), which the query clears. The outputs of such calls are not
    checked (they read values that were not ready)."""
    wl = qi.make_workload("decode", T=4)
    x, g = wl.tokens.x.to(DEV), wl.tokens.logits.to(DEV)
    with _env(QMOE_FUSED_SPIN_LIMIT=1):
        L = layer_for(wl, 16)
    for _ in range(3):
        L(x, g)
    bits = L.decode_errors()
    assert bits != 0 and bits & ~3 == 0, bits
    assert L.decode_errors() == 0
    # a handle with the default bound, on the same inputs, meets every wait
    check_decode(wl, layer_for(wl, 16))


def test_decode_many_experts_uses_split_path():
    """More experts than the fused kernel's routing holds (E = 320 > 256):
    the forward takes the two-kernel decode and still matches the oracle. A
    handle without the fused decode reports no wait errors."""
    spec = small_spec(4, 32, num_experts=320, top_k=6)
    wl = qi.make_layer(spec, T=4, seed=91)
    L = layer_for(wl, 16)
    check_decode(wl, L)
    assert L.decode_errors() == 0


def test_decode_repeated_experts_across_tokens():
    """Four tokens with identical logits share all k experts: each expert is
    streamed once and serves every token."""
    wl = qi.make_workload("decode", T=4)
    wl.tokens.logits = wl.tokens.logits[:1].repeat(4, 1).contiguous()
    check_decode(wl, layer_for(wl, 16))


# ------------------------------------------------------------------ prefill path

# The prefill's fp16 operands move the result by fp16 rounding of x (fp32
# layers only), of the weights and of h: a per-token relative L2 of about
# 1.8e-3 against the plain oracle at the Qwen3-30B-A3B shape, nearly all of
# it the bf16 output rounding. Those layers must keep a 4x margin to the
# 1e-2 bound.
PREFILL_QWEN_REL_L2 = 2.5e-3
# Against the oracle run with the same rounding points, an output differs
# only by fp32 summation order and the rare fp16 h value rounded the other
# way. One such flip of a large h value (a few times the rms of h) moves an
# element of y by about 2^-11 * 15 / sqrt(I) of its row's rms (y sums I
# terms). Elements beyond 2 bf16 ulps are near-zero outputs; each must stay
# within two such flips, 2^-6 / sqrt(I) of its row's rms. (Measured at most
# 3.4e-4 at I = 768 against a bound of 5.6e-4, 9.9e-4 at I = 128 against
# 1.4e-3; about 0.05-0.1% of the elements are beyond 2 ulps.)
def prefill_emu_outlier_bound(I):
    return 2.0 ** -6 / np.sqrt(I)


def emulated_acc(wl, x=None, rows=None):
    """The oracle with the fp16 datapath's rounding points (x as fp16 with a
    per-token exponent only where the layer's activations are not fp16)."""
    x = wl.tokens.x if x is None else x
    l = wl.tokens.logits
    if rows is not None:
        idx = torch.as_tensor(rows, dtype=torch.long)
        x, l = x[idx], l[idx]
    emu = oracle.EMU_W_F16 | oracle.EMU_H_F16
    if wl.spec.act_dtype != "f16":
        emu |= oracle.EMU_X_F16
    return oracle.forward(oracle.Layer.from_spec(wl.spec), x, l, wl.weights, emulate=emu)


def check_against_emulation(wl, out, rows=None, x=None):
    emu = emulated_acc(wl, x=x, rows=rows)
    got = out if rows is None else out[torch.as_tensor(rows, device=DEV)]
    rep = compare(got, emu)
    say(f"  vs fp16-datapath emulation: {rep}")
    assert rep.outlier_rel <= prefill_emu_outlier_bound(wl.spec.inter), rep
    assert rep.frac_within_ulp >= 0.995, rep
    return rep


def check_prefill(wl, layer, rows=None, emulation=False):
    T = wl.tokens.x.shape[0]
    out, ws = run(layer, wl.tokens.x, wl.tokens.logits)
    ids, w = layer.routing_from_workspace(T, ws)
    rid, _ = oracle.route(wl.tokens.logits, wl.spec.top_k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    if rows is None:
        rep = compare(out, oracle_acc(wl))
    else:
        rep = compare(out[torch.as_tensor(rows, device=DEV)], oracle_acc(wl, rows))
    say(f"prefill {wl.name} T={T} rows={'all' if rows is None else len(rows)}: {rep}")
    assert rep.ok, rep
    if wl.spec.hidden == 2048:
        assert rep.max_rel_l2 <= PREFILL_QWEN_REL_L2, rep
    if emulation:
        check_against_emulation(wl, out, rows)
    return out


def prefill_layer(wl, max_tokens):
    """A layer whose calls all take the grouped-GEMM path (small batches of a
    bf16 layer would otherwise run the fused decode per group of four)."""
    with _env(QMOE_FORCE_PATH="prefill"):
        return layer_for(wl, max_tokens)


@pytest.mark.parametrize("name,T", [("tiny", 5), ("tiny", 37), ("decode", 5), ("decode", 150),
                                    ("int3", 67), ("stack", 129)])
def test_prefill_parity_full(name, T):
    """Every row against the plain oracle (the stated tolerance; the Qwen3
    shapes with a 4x margin) and against the fp16-datapath emulation
    (per element)."""
    wl = qi.make_workload(name, T=T)
    check_prefill(wl, prefill_layer(wl, max(T, 8)), emulation=True)


@pytest.mark.parametrize("name,T,n", [("prefill", 8192, 256), ("int3", 2048, 256), ("stack", 4096, 32),
                                      ("stack", 32768, 256)])
def test_prefill_parity_sampled(name, T, n):
    """Full-size workloads in the launch configuration bench.py times, on
    sampled rows (first and last included): the plain oracle's tolerance
    with the 4x margin, and per element against the emulation."""
    say(f"prefill sampled {name} T={T}")
    wl = qi.make_workload(name, T=T)
    check_prefill(wl, layer_for(wl, T), rows=sample_rows(T, n, seed=T), emulation=n >= 256)


@pytest.mark.parametrize("bits,bs", FORMATS)
def test_prefill_parity_formats(bits, bs):
    wl = qi.make_layer(small_spec(bits, bs), T=300, seed=11 + bits + bs, nseq=3)
    check_prefill(wl, prefill_layer(wl, 300))


@pytest.mark.parametrize("name,T,xscale", [("decode", 40, 2.0 ** 9), ("decode", 33, 2.0 ** -16),
                                           ("int3", 24, 2.0 ** 12), ("tiny", 29, 2.0 ** 20),
                                           ("tiny", 30, 2.0 ** -30)])
def test_prefill_operand_ranges(name, T, xscale):
    """Activations far outside the fp16 range on the prefill path: scaled up
    so that h leaves it too (h chunks get exponents that differ within a
    route, so FC2 rescales them while staging), or down so that x and h
    would sink into the fp16 subnormals without their exponents. The output
    keeps the fp16 datapath's accuracy: per-token relative L2 (no floor)
    against the plain oracle within 2.5e-3, and per element against the
    emulation."""
    wl = qi.make_workload(name, T=T)
    x = (wl.tokens.x.to(torch.float64) * xscale).to(wl.tokens.x.dtype)
    say(f"prefill operand ranges {name} T={T} x*{xscale:g}")
    out, _ = run(prefill_layer(wl, max(T, 8)), x, wl.tokens.logits)
    assert torch.isfinite(out.float()).all()
    ref = oracle.forward(oracle.Layer.from_spec(wl.spec), x, wl.tokens.logits, wl.weights)
    d = out.double().cpu().numpy() - ref
    rel = np.linalg.norm(d, axis=1) / np.linalg.norm(ref, axis=1)
    say(f"  rel-L2 no floor: max {rel.max():.3e}")
    assert rel.max() <= 2.5e-3, rel.max()
    check_against_emulation(wl, out, x=x)


def test_prefill_fp32_activations():
    wl = qi.make_layer(small_spec(4, 32, act="f32", hidden=192, inter=96), T=45, seed=5)
    check_prefill(wl, layer_for(wl, 64))


def grouped_layer(wl, max_tokens, **kw):
    """A layer whose batches of 5..24 tokens run the fused decode once per
    group of up to four tokens (QMOE_FORCE_PATH=grouped)."""
    with _env(QMOE_FORCE_PATH="grouped"):
        return layer_for(wl, max_tokens, **kw)


@pytest.mark.parametrize("name,T", [("decode", 5), ("decode", 8), ("decode", 13), ("int3", 24),
                                    ("stack", 7)])
def test_grouped_decode_parity(name, T):
    """Batches of 5..24 tokens of a bf16 layer on the fused decode, once per
    group of up to four tokens: the routing of every token (read back from
    the workspace) is bit-exact and every output row matches the oracle."""
    wl = qi.make_workload(name, T=T)
    check_decode(wl, grouped_layer(wl, 32))


@pytest.mark.parametrize("T,k", [(8, 10), (8, 16), (3, 10)])
def test_speculative_decode_shape(T, k):
    """Eight draft tokens with top-10 routing (80 routes), the speculative
    decode shape the pages measure, and the largest top-k (16): on the grouped
    fused decode (the default up to 8 tokens) and on the small-batch path,
    the routing is bit-exact and the output matches the oracle (and the
    small-batch path the fp16-datapath emulation)."""
    spec = qi.spec_with(qi.QWEN3_INT4, top_k=k)
    wl = qi.make_layer(spec, T=T, seed=91 + T + k)
    say(f"speculative decode shape T={T} k={k}")
    check_decode(wl, grouped_layer(wl, 32))
    if T > 4:
        check_prefill(wl, small_layer(wl, 32), emulation=True)


@pytest.mark.parametrize("T,f16,extras", [(9, True, False), (7, False, True), (13, True, True)])
def test_grouped_decode_fp16_and_extras(T, f16, extras):
    """Batches of 5..24 tokens of fp16 layers or layers with biases and
    zero-point tensors run the fused decode's matching instance once per group
    of up to four tokens: every output row matches the oracle."""
    spec = qi.QWEN3_INT4 if not f16 else qi.spec_with(qi.QWEN3_INT4, act_dtype="f16")
    wl = qi.make_layer(spec, T=T, seed=71 + T)
    dt = torch.float16 if f16 else torch.bfloat16
    b1 = b2 = z1 = z2 = None
    if extras:
        rng = np.random.default_rng(T + 5)
        b1 = torch.from_numpy(rng.standard_normal((spec.num_experts, 2 * spec.inter)) * 0.25).to(dt)
        b2 = torch.from_numpy(rng.standard_normal((spec.num_experts, spec.hidden)) * 0.1).to(dt)
        z1, z2 = random_zero_points(wl, T)
    say(f"grouped fused decode T={T} f16={f16} extras={extras}")
    out, _ = run(grouped_layer(wl, 32, fc1_bias=b1, fc2_bias=b2, fc1_zero_points=z1, fc2_zero_points=z2),
                 wl.tokens.x, wl.tokens.logits)
    assert out.dtype == dt
    ref = oracle.forward(oracle.Layer.from_spec(spec), wl.tokens.x, wl.tokens.logits, wl.weights,
                         fc1_bias=b1, fc2_bias=b2, fc1_zero_points=z1, fc2_zero_points=z2)
    rep = compare(out, ref)
    assert rep.ok, rep


@pytest.mark.parametrize("f16", [False, True])
def test_wide_inter_with_extras_takes_split_decode(f16):
    """With inter > 768, layers with fp16 activations or biases take the split
    decode (the fused instances for them would spill); the result still
    matches the oracle."""
    spec = small_spec(4, 32, act="f16" if f16 else "bf16", hidden=512, inter=1024, num_experts=16,
                      top_k=4)
    wl = qi.make_layer(spec, T=4, seed=83)
    dt = torch.float16 if f16 else torch.bfloat16
    rng = np.random.default_rng(9)
    b1 = torch.from_numpy(rng.standard_normal((spec.num_experts, 2 * spec.inter)) * 0.25).to(dt)
    b2 = torch.from_numpy(rng.standard_normal((spec.num_experts, spec.hidden)) * 0.1).to(dt)
    out, _ = run(layer_for(wl, 8, fc1_bias=b1, fc2_bias=b2), wl.tokens.x, wl.tokens.logits)
    ref = oracle.forward(oracle.Layer.from_spec(spec), wl.tokens.x, wl.tokens.logits, wl.weights,
                         fc1_bias=b1, fc2_bias=b2)
    rep = compare(out, ref)
    say(f"wide inter with biases f16={f16}: {rep}")
    assert rep.ok, rep


def test_grouped_decode_matches_prefill():
    """The grouped decode and the grouped GEMMs compute the same 11-token
    layer (fp32 h against fp16 h): both meet the tolerance and agree per
    token to rel-L2 < 1e-2."""
    wl = qi.make_workload("decode", T=11)
    a = check_decode(wl, grouped_layer(wl, 16))
    b = check_prefill(wl, prefill_layer(wl, 16))
    d = (a.float() - b.float()).norm(dim=1) / a.float().norm(dim=1)
    assert d.max().item() < 1e-2


@pytest.mark.parametrize("name,T,force", [("decode", 4, None), ("decode", 8, None),
                                          ("decode", 1, "decode_split"), ("tiny", 4, None),
                                          ("prefill", 300, None), ("f32", 45, None),
                                          ("stack", 129, "prefill")])
def test_unnormalized_routing_parity(name, T, force):
    """normalize_routing = 0 on every routing implementation (fused, grouped
    and split decode, prefill routing; bf16 and fp32 logits): the same top-k
    bit for bit, each weight the selected expert's softmax probability over
    all experts (within 8 fp32 ulp: the denominator is a tree sum over all E
    terms instead of k), and the layer output within the tolerance. "f32" is
    the small fp32-activation layer of the fp32 prefill test."""
    if name == "f32":
        wl = qi.make_layer(small_spec(4, 32, act="f32", hidden=192, inter=96), T=T, seed=5)
    else:
        wl = qi.make_workload(name, T=T)
    with _env(**({"QMOE_FORCE_PATH": force} if force else {})):
        layer = layer_for(wl, max(T, 8), normalize=False)
    out, ws = run(layer, wl.tokens.x, wl.tokens.logits)
    ids, w = layer.routing_from_workspace(T, ws)
    rid, rw = oracle.route(wl.tokens.logits, wl.spec.top_k, normalize=False)
    assert np.array_equal(ids.cpu().numpy(), rid)
    ulp = fp32_ulps(w.cpu().numpy(), rw.astype(np.float32)).max()
    ref = oracle.forward(oracle.Layer.from_spec(wl.spec, normalize=False), wl.tokens.x,
                         wl.tokens.logits, wl.weights)
    rep = compare(out, ref)
    say(f"unnormalized {name} T={T} path={force or 'default'}: weight ulp {ulp}, {rep}")
    assert ulp <= 8
    assert rep.ok, rep


def interleave_fc1(wl):
    """The same layer with its FC1 rows (and scale rows) stored interleaved."""
    w, I = wl.weights, wl.spec.inter

    def il(a):
        out = np.empty_like(a)
        out[:, 0::2], out[:, 1::2] = a[:, :I], a[:, I:]
        return out

    return qi.Workload(wl.name, wl.spec, wl.tokens,
                       qi.LayerWeights(il(w.fc1_codes), il(w.fc1_scales), w.fc2_codes, w.fc2_scales))


@pytest.mark.parametrize("name,T,force", [("decode", 4, None), ("decode", 8, None),
                                          ("decode", 2, "decode_split"), ("int3", 300, None),
                                          ("tiny", 4, None), ("f32", 45, None)])
def test_interleaved_fc1_rows(name, T, force):
    """FC1 stored interleaved (row 2n gate n, row 2n+1 up n) on every FC1 path
    (fused, grouped and split decode, prefill; bf16 and fp32): the output
    equals, bit for bit, the block-layout run of the same rows (only the rows'
    addresses differ), and matches the oracle on the interleaved layout."""
    if name == "f32":
        wl = qi.make_layer(small_spec(4, 32, act="f32", hidden=192, inter=96), T=T, seed=5)
    else:
        wl = qi.make_workload(name, T=T)
    wi = interleave_fc1(wl)
    with _env(**({"QMOE_FORCE_PATH": force} if force else {})):
        lb = layer_for(wl, max(T, 8))
        li = layer_for(wi, max(T, 8), fc1_interleaved=True)
    a, _ = run(lb, wl.tokens.x, wl.tokens.logits)
    b, _ = run(li, wl.tokens.x, wl.tokens.logits)
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    ref = oracle.forward(oracle.Layer.from_spec(wl.spec, fc1_interleaved=True), wl.tokens.x,
                         wl.tokens.logits, wi.weights)
    rep = compare(b, ref)
    say(f"interleaved FC1 {name} T={T} path={force or 'default'}: {rep}")
    assert rep.ok, rep


def test_three_dimensional_input():
    """x [batch, seq, hidden] is the packed token-major layout with a leading
    dimension: the output (shaped like x) equals the 2-D run bit for bit, with
    3-D and with flattened logits, on the decode and the prefill path."""
    for T, B in ((4, 2), (40, 4)):
        wl = qi.make_workload("decode", T=T)
        layer = layer_for(wl, T)
        x, l = wl.tokens.x.to(DEV), wl.tokens.logits.to(DEV)
        ref = layer(x, l)
        a = layer(x.view(B, T // B, -1), l.view(B, T // B, -1))
        b = layer(x.view(B, T // B, -1), l)
        torch.cuda.synchronize()
        assert a.shape == (B, T // B, x.shape[1]) and b.shape == a.shape
        assert torch.equal(a.view(T, -1).view(torch.int16), ref.view(torch.int16))
        assert torch.equal(b.view(T, -1).view(torch.int16), ref.view(torch.int16))
        with pytest.raises(ValueError):
            layer(x.view(B, T // B, -1), l.view(1, T, -1))


@pytest.mark.parametrize("name,T,il", [("decode", 4, False), ("decode", 2, True),
                                       ("decode", 12, False), ("int3", 300, False),
                                       ("prefill", 300, True), ("tiny", 4, False), ("f32", 45, False)])
def test_biases_parity(name, T, il):
    """Optional FC1/FC2 biases in the activation dtype, on the decode (the
    fused kernel for bf16 layers, the split decode otherwise) and on the
    prefill path, with
    block and interleaved FC1 rows: the output matches the oracle given the
    same biases, and differs from the run without them."""
    if name == "f32":
        wl = qi.make_layer(small_spec(4, 32, act="f32", hidden=192, inter=96), T=T, seed=5)
    else:
        wl = qi.make_workload(name, T=T)
    if il:
        wl = interleave_fc1(wl)
    spec = wl.spec
    rng = np.random.default_rng(T + 7)
    dt = torch.float32 if spec.act_dtype == "f32" else torch.bfloat16
    b1 = torch.from_numpy(rng.standard_normal((spec.num_experts, 2 * spec.inter)) * 0.25).to(dt)
    b2 = torch.from_numpy(rng.standard_normal((spec.num_experts, spec.hidden)) * 0.1).to(dt)
    layer = layer_for(wl, max(T, 8), fc1_interleaved=il, fc1_bias=b1, fc2_bias=b2)
    out, _ = run(layer, wl.tokens.x, wl.tokens.logits)
    ref = oracle.forward(oracle.Layer.from_spec(spec, fc1_interleaved=il), wl.tokens.x,
                         wl.tokens.logits, wl.weights, fc1_bias=b1, fc2_bias=b2)
    rep = compare(out, ref)
    say(f"biases {name} T={T} interleaved={il}: {rep}")
    assert rep.ok, rep
    nob, _ = run(layer_for(wl, max(T, 8), fc1_interleaved=il), wl.tokens.x, wl.tokens.logits)
    assert not torch.equal(out, nob)


@pytest.mark.parametrize("name,T", [("decode", 4), ("decode", 300), ("int3", 67), ("stack", 129),
                                    ("tiny", 4), ("f32", 45)])
def test_zero_point_tensors_parity(name, T):
    """Per-block zero-point tensors in FC1 and FC2, on the decode (the fused
    kernel for bf16 layers, the split decode otherwise) and the prefill path,
    every format and both activation dtypes: the output matches the oracle
    given the same tensors."""
    if name == "f32":
        wl = qi.make_layer(small_spec(4, 32, act="f32", hidden=192, inter=96), T=T, seed=5)
    else:
        wl = qi.make_workload(name, T=T)
    z1, z2 = random_zero_points(wl, T)
    out, _ = run(layer_for(wl, max(T, 8), fc1_zero_points=z1, fc2_zero_points=z2),
                 wl.tokens.x, wl.tokens.logits)
    ref = oracle.forward(oracle.Layer.from_spec(wl.spec), wl.tokens.x, wl.tokens.logits,
                         wl.weights, fc1_zero_points=z1, fc2_zero_points=z2)
    rep = compare(out, ref)
    say(f"zero-point tensors {name} T={T}: {rep}")
    assert rep.ok, rep


@pytest.mark.parametrize("name,T,bias,zps", [("decode", 4, True, True), ("decode", 1, True, False),
                                             ("int3", 4, False, True), ("stack", 2, True, True)])
def test_fused_decode_with_extras_matches_split(name, T, bias, zps):
    """Layers with biases or zero-point tensors run the fused decode's instance
    that loads them; it computes the same layer as the two-kernel decode (fp32
    throughout, different summation orders), and both match the oracle."""
    wl = qi.make_workload(name, T=T)
    spec = wl.spec
    rng = np.random.default_rng(T + 11)
    b1 = b2 = z1 = z2 = None
    if bias:
        b1 = torch.from_numpy(rng.standard_normal((spec.num_experts, 2 * spec.inter)) * 0.25).to(torch.bfloat16)
        b2 = torch.from_numpy(rng.standard_normal((spec.num_experts, spec.hidden)) * 0.1).to(torch.bfloat16)
    if zps:
        z1, z2 = random_zero_points(wl, T)
    kw = dict(fc1_bias=b1, fc2_bias=b2, fc1_zero_points=z1, fc2_zero_points=z2)
    say(f"fused decode with extras {name} T={T} bias={bias} zps={zps}")
    a, _ = run(layer_for(wl, 16, **kw), wl.tokens.x, wl.tokens.logits)
    with _env(QMOE_FORCE_PATH="decode_split"):
        ls = layer_for(wl, 16, **kw)
    b, _ = run(ls, wl.tokens.x, wl.tokens.logits)
    ref = oracle.forward(oracle.Layer.from_spec(spec), wl.tokens.x, wl.tokens.logits, wl.weights,
                         fc1_bias=b1, fc2_bias=b2, fc1_zero_points=z1, fc2_zero_points=z2)
    for out in (a, b):
        rep = compare(out, ref)
        assert rep.ok, rep
    d = (a.float() - b.float()).abs().max().item()
    scale = a.float().abs().max().item()
    assert d <= 2 ** -7 * scale, (d, scale)


@pytest.mark.parametrize("T", [3, 200])
def test_zero_point_tensor_of_the_scalar_is_bitwise_same(T):
    """A zero-point tensor filled with the layer's scalar zero point gives the
    output of the scalar zero point bit for bit, on each path: the fused and
    the split decode (T <= 4) and the prefill."""
    wl = qi.make_workload("decode", T=T)
    z1 = np.full(wl.weights.fc1_scales.shape, wl.spec.zero_point, np.uint8)
    z2 = np.full(wl.weights.fc2_scales.shape, wl.spec.zero_point, np.uint8)
    for force in ((None, "decode_split") if T <= 4 else (None,)):
        with _env(**({"QMOE_FORCE_PATH": force} if force else {})):
            la = layer_for(wl, max(T, 8))
            lb = layer_for(wl, max(T, 8), fc1_zero_points=z1, fc2_zero_points=z2)
        a, _ = run(la, wl.tokens.x, wl.tokens.logits)
        b, _ = run(lb, wl.tokens.x, wl.tokens.logits)
        say(f"scalar zero point vs tensor T={T} path={force or 'default'}")
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), force


@pytest.mark.parametrize("T,extras", [(1, False), (4, False), (4, True), (37, False), (300, True)])
def test_fp16_activations_parity(T, extras):
    """fp16 x, logits and out on the Qwen3-shaped INT4 layer: T <= 4 runs the
    fused decode on fp16 operands, larger T the prefill path (fp16 x straight
    into the matrix cores). The routing of the fp16 logits is bit-exact and the
    output (rounded once to fp16) matches the oracle; with extras, fp16
    biases and unnormalized routing too."""
    spec = qi.spec_with(qi.QWEN3_INT4, act_dtype="f16")
    wl = qi.make_layer(spec, T=T, seed=41 + T, nseq=max(1, T // 40))
    b1 = b2 = None
    if extras:
        rng = np.random.default_rng(T)
        b1 = torch.from_numpy(rng.standard_normal((spec.num_experts, 2 * spec.inter)) * 0.25).half()
        b2 = torch.from_numpy(rng.standard_normal((spec.num_experts, spec.hidden)) * 0.1).half()
    layer = layer_for(wl, max(T, 8), normalize=not extras, fc1_bias=b1, fc2_bias=b2)
    out, ws = run(layer, wl.tokens.x, wl.tokens.logits)
    assert out.dtype == torch.float16
    ids, _ = layer.routing_from_workspace(T, ws)
    rid, _ = oracle.route(wl.tokens.logits, spec.top_k, normalize=not extras)
    assert np.array_equal(ids.cpu().numpy(), rid)
    ref = oracle.forward(oracle.Layer.from_spec(spec, normalize=not extras), wl.tokens.x,
                         wl.tokens.logits, wl.weights, fc1_bias=b1, fc2_bias=b2)
    rep = compare(out, ref)
    say(f"fp16 activations T={T} extras={extras}: {rep}")
    assert rep.ok, rep


@pytest.mark.parametrize("name,T,extras", [("decode", 4, False), ("decode", 1, True), ("int3", 3, False),
                                            ("stack", 4, True)])
def test_fused_decode_fp16_matches_split(name, T, extras):
    """fp16 layers run the fused decode's fp16 instance (FC1 on fp16 operands);
    it computes the same layer as the two-kernel decode, which widens x to
    fp32, and both match the oracle. With extras: fp16 biases and zero-point
    tensors as well."""
    spec = qi.spec_with(qi.make_workload(name, T=1).spec, act_dtype="f16")
    wl = qi.make_layer(spec, T=T, seed=61 + T)
    b1 = b2 = z1 = z2 = None
    if extras:
        rng = np.random.default_rng(T + 3)
        b1 = torch.from_numpy(rng.standard_normal((spec.num_experts, 2 * spec.inter)) * 0.25).half()
        b2 = torch.from_numpy(rng.standard_normal((spec.num_experts, spec.hidden)) * 0.1).half()
        z1, z2 = random_zero_points(wl, T)
    kw = dict(fc1_bias=b1, fc2_bias=b2, fc1_zero_points=z1, fc2_zero_points=z2)
    say(f"fused fp16 decode {name} T={T} extras={extras}")
    a, _ = run(layer_for(wl, 16, **kw), wl.tokens.x, wl.tokens.logits)
    with _env(QMOE_FORCE_PATH="decode_split"):
        ls = layer_for(wl, 16, **kw)
    b, _ = run(ls, wl.tokens.x, wl.tokens.logits)
    assert a.dtype == torch.float16 and b.dtype == torch.float16
    ref = oracle.forward(oracle.Layer.from_spec(spec), wl.tokens.x, wl.tokens.logits, wl.weights,
                         fc1_bias=b1, fc2_bias=b2, fc1_zero_points=z1, fc2_zero_points=z2)
    for out in (a, b):
        rep = compare(out, ref)
        assert rep.ok, rep
    d = (a.float() - b.float()).abs().max().item()
    scale = a.float().abs().max().item()
    assert d <= 2 ** -9 * scale, (d, scale)


@pytest.mark.parametrize("name,T,force", [("decode", 4, None), ("decode", 9, None), ("decode", 300, None),
                                           ("tiny", 4, None), ("decode", 4, "decode_split")])
def test_nan_and_inf_inputs_stay_local(name, T, force):
    """NaN and infinite values in x or the logits of some tokens (the pages
    leave their result open): the call completes, every token still gets k
    distinct valid experts, and the tokens with clean inputs match the oracle
    (each token's output depends on its own inputs only)."""
    wl = qi.make_workload(name, T=T)
    E, k = wl.spec.num_experts, wl.spec.top_k
    x, lg = wl.tokens.x.clone(), wl.tokens.logits.clone()
    x[1, 5] = float("nan")
    lg[2, 3 % E] = float("inf")
    lg[0, 1 % E] = float("nan")
    dirty = [0, 1, 2]
    say(f"nan/inf inputs {name} T={T} path={force or 'default'}")
    with _env(**({"QMOE_FORCE_PATH": force} if force else {})):
        layer = layer_for(wl, max(T, 16))
    out, ws = run(layer, x, lg)
    ids, _ = layer.routing_from_workspace(T, ws)
    ids = ids.cpu().numpy()
    assert ids.min() >= 0 and ids.max() < E
    assert all(len(set(row)) == k for row in ids.tolist())
    clean = [t for t in range(T) if t not in dirty]
    ref = oracle.forward(oracle.Layer.from_spec(wl.spec), x[clean], lg[clean], wl.weights)
    rep = compare(out[torch.as_tensor(clean, device=DEV)], ref)
    assert rep.ok, rep


# ------------------------------------------------------------------ small-batch path

def small_layer(wl, max_tokens, **kw):
    """A layer whose calls of any size take the small-batch path."""
    with _env(QMOE_FORCE_PATH="small"):
        return layer_for(wl, max_tokens, **kw)


@pytest.mark.parametrize("name,T", [("decode", 5), ("decode", 25), ("decode", 32), ("decode", 48),
                                    ("decode", 64), ("decode", 128), ("int3", 40), ("stack", 64),
                                    ("prefill", 100)])
def test_small_path_parity(name, T):
    """The small-batch path (the default from 9 to 256 tokens; forced here for
    every size): routing bit-exact, every row against the plain oracle (4x
    margin) and per element against the fp16-datapath emulation."""
    wl = qi.make_workload(name, T=T)
    check_prefill(wl, small_layer(wl, max(T, 8)), emulation=True)


@pytest.mark.parametrize("T,path", [(4, "decode"), (8, "decode"), (9, "small"), (256, "small"),
                                    (257, "prefill")])
def test_default_dispatch(T, path):
    """The default dispatch of the Qwen3-shaped bf16 layer: the fused decode up
    to 8 tokens (groups of four above four), the small-batch path up to 256,
    the grouped GEMMs above; each call's stage names show the path taken, and
    the output matches the oracle on sampled rows."""
    wl = qi.make_workload("decode", T=T)
    L = layer_for(wl, T)
    names = []
    L.set_stage_hook(lambda stage, name: names.append(name))
    out, _ = run(L, wl.tokens.x, wl.tokens.logits)
    L.set_stage_hook(None)
    taken = ("decode" if any(n.startswith("decode") for n in names)
             else "small" if any(n.startswith("small") for n in names) else "prefill")
    assert taken == path, names
    rows = sample_rows(T, 16, seed=T)
    assert compare(out[torch.as_tensor(rows, device=DEV)], oracle_acc(wl, rows)).ok


@pytest.mark.parametrize("bits,bs", FORMATS)
def test_small_path_formats(bits, bs):
    wl = qi.make_layer(small_spec(bits, bs), T=40, seed=21 + bits + bs, nseq=2)
    check_prefill(wl, small_layer(wl, 64), emulation=True)


@pytest.mark.parametrize("kw,T", [
    (dict(hidden=640, inter=640, block_size=128, num_experts=6, top_k=3), 23),
    (dict(hidden=640, inter=640, block_size=64, num_experts=6, top_k=3, bits=2), 17),
    (dict(hidden=384, inter=896, block_size=128, num_experts=4, top_k=2, bits=3), 11),
    (dict(hidden=4096, inter=4096, block_size=128, num_experts=4, top_k=2), 9)])
def test_small_path_ragged_and_largest_shapes(kw, T):
    """Shapes whose K is not a multiple of the 256-K weight blocks (a tail
    block with a sub-block past K), whose h columns and output rows end
    inside a workgroup's groups (groups past I or H computed on clamped rows
    and not stored), and the largest shape the small-batch path takes
    (H = I = 4096: 144 KB of LDS per workgroup): against the plain oracle and
    per element against the emulation."""
    d = dict(kw)
    bits = d.pop("bits", 4)
    spec = small_spec(bits, d.pop("block_size"), **d)
    wl = qi.make_layer(spec, T=T, seed=300 + T + spec.hidden)
    say(f"small path H={spec.hidden} I={spec.inter} bits={bits} bs={spec.block_size} T={T}")
    check_prefill(wl, small_layer(wl, 32), emulation=True)


@pytest.mark.parametrize("T", [1, 3, 4])
def test_small_path_few_tokens(T):
    """The small-batch path also computes 1..4 tokens (forced): the same
    tolerance as every grouped path."""
    wl = qi.make_workload("decode", T=T)
    check_prefill(wl, small_layer(wl, 8), emulation=True)


@pytest.mark.parametrize("case", ["biases_interleaved", "zero_points", "fp16", "fp32", "unnormalized"])
def test_small_path_variants(case):
    """Biases with interleaved FC1 rows, zero-point tensors, fp16 and fp32
    activations and unnormalized routing on the small-batch path, against
    the oracle given the same inputs."""
    T = 30
    il = case == "biases_interleaved"
    if case == "fp32":
        wl = qi.make_layer(small_spec(4, 32, act="f32", hidden=256, inter=128), T=T, seed=5)
    elif case == "fp16":
        wl = qi.make_layer(qi.spec_with(qi.QWEN3_INT4, act_dtype="f16"), T=T, seed=6)
    else:
        wl = qi.make_workload("decode", T=T)
    if il:
        wl = interleave_fc1(wl)
    spec = wl.spec
    dt = qi.TORCH_DTYPE[spec.act_dtype]
    rng = np.random.default_rng(17)
    b1 = b2 = z1 = z2 = None
    if il:
        b1 = torch.from_numpy(rng.standard_normal((spec.num_experts, 2 * spec.inter)) * 0.25).to(dt)
        b2 = torch.from_numpy(rng.standard_normal((spec.num_experts, spec.hidden)) * 0.1).to(dt)
    if case == "zero_points":
        z1, z2 = random_zero_points(wl, 3)
    norm = case != "unnormalized"
    layer = small_layer(wl, 64, normalize=norm, fc1_interleaved=il, fc1_bias=b1, fc2_bias=b2,
                        fc1_zero_points=z1, fc2_zero_points=z2)
    out, _ = run(layer, wl.tokens.x, wl.tokens.logits)
    ref = oracle.forward(oracle.Layer.from_spec(spec, normalize=norm, fc1_interleaved=il), wl.tokens.x,
                         wl.tokens.logits, wl.weights, fc1_bias=b1, fc2_bias=b2, fc1_zero_points=z1,
                         fc2_zero_points=z2)
    rep_ = compare(out, ref)
    say(f"small path {case}: {rep_}")
    assert rep_.ok, rep_


@pytest.mark.parametrize("xscale", [2.0 ** 9, 2.0 ** -16])
def test_small_path_operand_ranges(xscale):
    """Activations far outside the fp16 range on the small-batch path: the
    per-token activation exponent and the per-route h exponent keep the
    fp16 datapath's accuracy (rel-L2 without floor within 2.5e-3)."""
    wl = qi.make_workload("decode", T=24)
    x = (wl.tokens.x.to(torch.float64) * xscale).to(wl.tokens.x.dtype)
    out, _ = run(small_layer(wl, 32), x, wl.tokens.logits)
    assert torch.isfinite(out.float()).all()
    ref = oracle.forward(oracle.Layer.from_spec(wl.spec), x, wl.tokens.logits, wl.weights)
    d = out.double().cpu().numpy() - ref
    rel = np.linalg.norm(d, axis=1) / np.linalg.norm(ref, axis=1)
    say(f"small path ranges x*{xscale:g}: rel-L2 no floor max {rel.max():.3e}")
    assert rel.max() <= 2.5e-3, rel.max()


def test_small_path_batch_invariant():
    """Each token's rows of the small-batch path depend on its own routes
    only: sequences run alone reproduce their rows of the packed run bit for
    bit."""
    wl = qi.make_workload("prefill", T=120)
    L = small_layer(wl, 128)
    packed, _ = run(L, wl.tokens.x, wl.tokens.logits)
    s0 = 0
    for n in wl.tokens.seq_lens:
        part, _ = run(L, wl.tokens.x[s0:s0 + n].contiguous(), wl.tokens.logits[s0:s0 + n].contiguous())
        assert torch.equal(part.view(torch.int16), packed[s0:s0 + n].view(torch.int16)), (s0, n)
        s0 += n


# ------------------------------------------------------------------ properties

def test_decode_and_prefill_agree():
    wl = qi.make_workload("decode", T=4)
    a, _ = run(layer_for(wl, 16), wl.tokens.x, wl.tokens.logits)
    os.environ["QMOE_FORCE_PATH"] = "prefill"
    try:
        lp = layer_for(wl, 16)
    finally:
        del os.environ["QMOE_FORCE_PATH"]
    b, _ = run(lp, wl.tokens.x, wl.tokens.logits)
    ref = oracle_acc(wl)
    ra, rb = compare(a, ref), compare(b, ref)
    assert ra.ok and rb.ok, (ra, rb)
    d = (a.float() - b.float()).norm(dim=1) / a.float().norm(dim=1)
    assert d.max().item() < 1e-2


def test_packed_equals_per_sequence():
    """Prefill rows are batch-invariant: with every call on the grouped-GEMM
    path, each sequence run alone reproduces its rows of the packed run bit
    for bit. With the default dispatch, sequences of up to 24 tokens take the
    fused decode (per group of four tokens) and must meet the tolerance."""
    wl = qi.make_workload("prefill", T=160)
    lp = prefill_layer(wl, 160)
    ld = layer_for(wl, 160)
    packed, _ = run(lp, wl.tokens.x, wl.tokens.logits)
    s = 0
    for n in wl.tokens.seq_lens:
        xs, ls = wl.tokens.x[s:s + n].contiguous(), wl.tokens.logits[s:s + n].contiguous()
        part, _ = run(lp, xs, ls)
        assert torch.equal(part, packed[s:s + n]), (s, n)
        dpart, _ = run(ld, xs, ls)
        sub = qi.Workload("seq", wl.spec, qi.Tokens(xs, ls), wl.weights)
        assert compare(dpart, oracle_acc(sub)).ok, (s, n)
        s += n


@pytest.mark.parametrize("name,T", [("decode", 4), ("prefill", 1024)])
def test_run_to_run_bitwise_deterministic(name, T):
    wl = qi.make_workload(name, T=T)
    layer = layer_for(wl, T)
    a, _ = run(layer, wl.tokens.x, wl.tokens.logits)
    b, _ = run(layer, wl.tokens.x, wl.tokens.logits)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_empty_input_is_a_noop():
    wl = qi.make_workload("decode", T=4)
    layer = layer_for(wl, 16)
    out = torch.full((0, 2048), 7.0, dtype=torch.bfloat16, device=DEV)
    res = layer(torch.empty((0, 2048), dtype=torch.bfloat16, device=DEV),
                torch.empty((0, 128), dtype=torch.bfloat16, device=DEV), out=out)
    torch.cuda.synchronize()
    assert res.shape == (0, 2048)


def test_forward_rejects_small_workspace_and_too_many_tokens():
    import quantized_mixture_experts_qmoe_amd as q
    wl = qi.make_workload("decode", T=4)
    layer = layer_for(wl, 4)
    x, l = wl.tokens.x.to(DEV), wl.tokens.logits.to(DEV)
    ws = torch.empty(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(q.QMoEError) as ei:
        layer(x, l, workspace=ws)
    assert ei.value.status == 3
    x5 = torch.zeros((5, 2048), dtype=torch.bfloat16, device=DEV)
    l5 = torch.zeros((5, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(q.QMoEError) as ei:
        layer(x5, l5, workspace=layer.workspace(4))
    assert ei.value.status == 1
