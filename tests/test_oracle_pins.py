"""Pins for the CPU oracle: each check ties it to something other than itself.

The pages print no worked numeric example for the QMoE layer, so the pins are
closed forms, library routines, brute force on small inputs, invariants and
the hand-written packing vectors in ``tests/golden/packing.json``.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import qmoe_inputs as qi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "packing.json")


# ---------------------------------------------------------------- conversions

def test_half_decode_all_patterns():
    """All 65,536 fp16 patterns against numpy's float16 -> float64 conversion."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.half_to_double(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros and infinities keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("chunk", range(16))
def test_bf16_rounding_all_floats(chunk):
    """fp32 -> bf16 round-to-nearest-even over all 2^32 patterns (16 slices)
    against torch's conversion; NaN must stay NaN."""
    n = 1 << 28
    step = 1 << 24
    base = chunk * n
    for off in range(0, n, step):
        u = np.arange(base + off, base + off + step, dtype=np.uint64).astype(np.uint32)
        f = u.view(np.float32)
        got = oracle.f32_to_bf16_bits(f)
        ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        isnan = np.isnan(f)
        got_nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
        assert np.array_equal(got_nan, isnan)
        assert np.array_equal(got[~isnan], ref[~isnan])


# ---------------------------------------------------------------- packing / dequant

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["packing"], ids=lambda c: f"int{c['bits']}-{c['bytes']}")
def test_packing_golden(case):
    bits, codes, want = case["bits"], case["codes"], np.array(case["bytes"], dtype=np.uint8)
    K = len(codes)
    assert np.array_equal(brute.pack_codes(np.array([codes]), bits)[0], want)
    assert np.array_equal(brute.unpack_codes(want[None], bits, K)[0], codes)
    # oracle reads the same codes: scale 1.0 (fp16 0x3C00), zero point 0.
    # K may be shorter than a block, so use block size = K (the oracle only
    # requires K % 8 == 0 and K % bs == 0).
    if K % 8 == 0:
        s = np.full((1, 1), 0x3C00, dtype=np.uint16).view(np.float16)
        got = oracle.dequant(want[None], s, bits, K, 0, K)[0]
        assert np.array_equal(got, np.array(codes, dtype=np.float64))


@pytest.mark.parametrize("case", _golden()["dequant"], ids=lambda c: f"int{c['bits']}")
def test_dequant_golden(case):
    bits, zp, codes = case["bits"], case["zero_point"], case["codes"]
    K = 8 * ((len(codes) + 7) // 8)
    q = np.zeros(K, dtype=np.int64)
    q[: len(codes)] = codes
    packed = brute.pack_codes(q[None], bits)
    s = np.full((1, 1), case["scale_fp16_bits"], dtype=np.uint16).view(np.float16)
    assert float(s[0, 0]) == case["scale"]
    got = oracle.dequant(packed, s, bits, K, zp, K)[0][: len(codes)]
    assert np.array_equal(got, np.array(case["values"], dtype=np.float64))


@pytest.mark.parametrize("bits,bs,K", [(4, 32, 64), (4, 64, 256), (4, 128, 2048),
                                       (3, 32, 64), (3, 64, 768), (3, 128, 256),
                                       (2, 32, 96), (2, 64, 128), (2, 128, 2048)])
def test_dequant_matches_bitstream_reading(bits, bs, K):
    """C per-format shifts vs the numpy bit-stream reading, random rows and scales."""
    rng = np.random.default_rng(bits * 1000 + bs + K)
    N = 37
    codes = rng.integers(0, 256, size=(N, K * bits // 8), dtype=np.uint8)
    scales = (rng.standard_normal((N, K // bs)) * 3).astype(np.float16)
    zp = 1 << (bits - 1)
    got = oracle.dequant(codes, scales, bits, bs, zp, K)
    ref = brute.dequant_dense(codes, scales, bits, bs, zp, K)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_dequant_exhaustive_codes_times_scales(bits):
    """Every code times every finite fp16 scale: (q - zp) * s is exact in
    float64 and equals the integer multiple of the decoded scale."""
    zp = 1 << (bits - 1)
    ncodes = 1 << bits
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = np.isfinite(allh.view(np.float16))
    hs = allh[finite]
    # one row per scale, K = 8*ncodes codes cycling through all codes
    K = 8 * ncodes
    q = np.tile(np.arange(ncodes), K // ncodes)
    packed = np.broadcast_to(brute.pack_codes(q[None], bits), (hs.size, K * bits // 8)).copy()
    scales = np.repeat(hs.view(np.float16)[:, None], K // K, axis=1)       # block = K
    got = oracle.dequant(packed, scales, bits, K, zp, K)
    s64 = hs.view(np.float16).astype(np.float64)
    ref = (q[None, :] - zp).astype(np.float64) * s64[:, None]
    assert np.array_equal(got, ref)
    # exact in fp32 as well: at most 11 + 3 significant bits
    assert np.array_equal(got.astype(np.float32).astype(np.float64), got)


# ---------------------------------------------------------------- routing

def _logits_with_ties(T, E, rng):
    l = rng.standard_normal((T, E))
    # quantize hard so that many logits tie
    l = np.round(l * 2) / 2
    return l


@pytest.mark.parametrize("E,k", [(4, 2), (8, 8), (16, 1), (128, 8), (64, 6)])
def test_topk_against_stable_sort(E, k):
    rng = np.random.default_rng(E * 31 + k)
    T = 300
    for logits in (rng.standard_normal((T, E)), _logits_with_ties(T, E, rng),
                   np.zeros((T, E))):
        ids, w = oracle.route(logits, k)
        assert np.array_equal(ids, brute.topk_brute(logits, k))
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15 * k)


def test_topk_bf16_logits_ties():
    """bf16 logits tie often; the lower expert index must win."""
    rng = np.random.default_rng(7)
    l = torch.from_numpy(rng.standard_normal((2000, 128))).to(torch.bfloat16)
    l64 = l.to(torch.float64).numpy()
    ids, _ = oracle.route(l, 8)
    assert np.array_equal(ids, brute.topk_brute(l64, 8))
    # the draw really exercises ties among the selected/next experts
    srt = -np.sort(-l64, axis=1)
    assert (srt[:, 7] == srt[:, 8]).mean() > 0.01


def test_topk_constructed_ties():
    logits = np.array([[1.0, 3.0, 3.0, 0.5, 3.0],
                       [2.0, 2.0, 2.0, 2.0, 2.0],
                       [-1.0, 0.0, -1.0, 0.0, 5.0]])
    ids, w = oracle.route(logits, 3)
    assert ids.tolist() == [[1, 2, 4], [0, 1, 2], [4, 1, 3]]
    np.testing.assert_allclose(w[0], [1 / 3] * 3, rtol=0, atol=1e-16)
    np.testing.assert_allclose(w[1], [1 / 3] * 3, rtol=0, atol=1e-16)


def test_softmax_full_k_is_softmax():
    """With k = E the routing weights are the textbook softmax (torch, fp64)."""
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((64, 16)) * 4
    ids, w = oracle.route(logits, 16)
    ref = torch.softmax(torch.from_numpy(logits), dim=1).numpy()
    got = np.zeros_like(ref)
    np.put_along_axis(got, ids.astype(np.int64), w, axis=1)
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-300)


def test_softmax_k1_is_one():
    rng = np.random.default_rng(12)
    ids, w = oracle.route(rng.standard_normal((50, 32)), 1)
    assert np.all(w == 1.0)


def test_softmax_selected_closed_form():
    logits = np.array([[0.0, np.log(3.0), -50.0, np.log(2.0)]])
    ids, w = oracle.route(logits, 3)
    assert ids.tolist() == [[1, 3, 0]]
    np.testing.assert_allclose(w[0], [0.5, 1 / 3, 1 / 6], rtol=1e-15)


def test_unnormalized_weights_are_full_softmax_at_selected():
    """Without normalization a selected expert's weight is its probability
    under the softmax over all experts (torch, fp64); the selection is the
    same top-k as with normalization, and k = E gives identical weights."""
    rng = np.random.default_rng(13)
    logits = rng.standard_normal((200, 32)) * 3
    ids0, w0 = oracle.route(logits, 6, normalize=False)
    ids1, w1 = oracle.route(logits, 6)
    assert np.array_equal(ids0, ids1)
    ref = torch.softmax(torch.from_numpy(logits), dim=1).numpy()
    np.testing.assert_allclose(w0, np.take_along_axis(ref, ids0.astype(np.int64), axis=1),
                               rtol=1e-14, atol=0)
    # the ratios between slots do not depend on the denominator
    np.testing.assert_allclose(w0 / w0[:, :1], w1 / w1[:, :1], rtol=1e-14)
    assert np.all(w0.sum(axis=1) < 1.0)
    idsf, wf0 = oracle.route(logits, 32, normalize=False)
    _, wf1 = oracle.route(logits, 32)
    np.testing.assert_allclose(wf0, wf1, rtol=1e-14)


def test_unnormalized_closed_form():
    logits = np.array([[0.0, np.log(3.0), np.log(0.5), np.log(2.0)]])
    ids, w = oracle.route(logits, 2, normalize=False)
    assert ids.tolist() == [[1, 3]]
    np.testing.assert_allclose(w[0], [3 / 6.5, 2 / 6.5], rtol=1e-15)


def test_unnormalized_forward_scales_each_token():
    """The layer output without normalization is, per token, the normalized
    output times (sum over the selected of exp) / (sum over all of exp)."""
    wl = qi.make_workload("tiny")
    L1 = oracle.Layer.from_spec(wl.spec)
    L0 = oracle.Layer.from_spec(wl.spec, normalize=False)
    a1 = oracle.forward(L1, wl.tokens.x, wl.tokens.logits, wl.weights)
    a0 = oracle.forward(L0, wl.tokens.x, wl.tokens.logits, wl.weights)
    l = wl.tokens.logits.to(torch.float64).numpy()
    ids, _ = oracle.route(l, wl.spec.top_k)
    e = np.exp(l - l.max(axis=1, keepdims=True))
    frac = np.take_along_axis(e, ids.astype(np.int64), axis=1).sum(axis=1) / e.sum(axis=1)
    np.testing.assert_allclose(a0, a1 * frac[:, None], rtol=1e-12, atol=1e-300)
    assert np.all(frac < 1.0)


def test_interleaved_fc1_rows_equal_block_layout():
    """FC1 stored interleaved (row 2n = gate n, row 2n+1 = up n, scale rows in
    the same order) gives exactly the layer of the block layout (gate rows,
    then up rows) holding the same rows."""
    wl = qi.make_workload("tiny")
    w = wl.weights
    I = wl.spec.inter

    def interleave(a):
        out = np.empty_like(a)
        out[:, 0::2], out[:, 1::2] = a[:, :I], a[:, I:]
        return out

    wi = qi.LayerWeights(interleave(w.fc1_codes), interleave(w.fc1_scales), w.fc2_codes,
                         w.fc2_scales)
    a = oracle.forward(oracle.Layer.from_spec(wl.spec), wl.tokens.x, wl.tokens.logits, w)
    b = oracle.forward(oracle.Layer.from_spec(wl.spec, fc1_interleaved=True), wl.tokens.x,
                       wl.tokens.logits, wi)
    assert np.array_equal(a, b)
    # and reading the interleaved rows as blocks is a different layer
    c = oracle.forward(oracle.Layer.from_spec(wl.spec), wl.tokens.x, wl.tokens.logits, wi)
    assert not np.allclose(a, c)


# ---------------------------------------------------------------- permutation

@pytest.mark.parametrize("T,E,k,skew", [(0, 8, 2, False), (1, 128, 8, False), (4, 4, 2, False),
                                        (513, 128, 8, True), (2000, 64, 4, False)])
def test_permutation_against_stable_argsort(T, E, k, skew):
    rng = np.random.default_rng(T + E + k)
    logits = rng.standard_normal((T, E))
    if skew:
        logits += qi.zipf_bias(E, 1.1, rng)[None, :]
    ids, _ = oracle.route(logits, k) if T else (np.zeros((0, k), np.int32), None)
    counts, offsets, sorted_routes, inv_pos = oracle.permute(ids, E)
    flat = ids.reshape(-1)
    R = flat.size
    assert np.array_equal(sorted_routes, np.argsort(flat, kind="stable"))
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == R and np.all(np.diff(offsets) == counts)
    assert np.array_equal(np.sort(sorted_routes), np.arange(R))
    assert np.all(np.diff(flat[sorted_routes]) >= 0)
    assert np.array_equal(inv_pos[sorted_routes], np.arange(R))


# ---------------------------------------------------------------- whole layer

def _small_spec(**kw):
    return qi.spec_with(qi.TINY, **kw)


def _run(wl, nthreads=4, emulate=0):
    return oracle.forward(oracle.Layer.from_spec(wl.spec), wl.tokens.x, wl.tokens.logits,
                          wl.weights, nthreads=nthreads, emulate=emulate)


def _brute(wl, **kw):
    return brute.dense_masked_forward(oracle.as_f64(wl.tokens.x), oracle.as_f64(wl.tokens.logits),
                                      wl.weights, wl.spec, **kw)


def _close(a, b, rtol=1e-12):
    scale = np.abs(b).max() + 1e-300
    return np.abs(a - b).max() <= rtol * scale


def test_biases_against_dense_masked():
    """Optional FC1/FC2 biases: the oracle equals the dense masked mixture with
    the FC1 bias added to the gate/up projections before SwiGLU and the FC2
    bias to y before the routing weights; placing the FC1 bias after the
    activation, or dropping either bias, would be noticed."""
    wl = qi.make_workload("tiny")
    rng = np.random.default_rng(21)
    E, H, I = wl.spec.num_experts, wl.spec.hidden, wl.spec.inter
    b1 = rng.standard_normal((E, 2 * I)) * 0.5
    b2 = rng.standard_normal((E, H)) * 0.5
    got = oracle.forward(oracle.Layer.from_spec(wl.spec), wl.tokens.x, wl.tokens.logits,
                         wl.weights, fc1_bias=b1, fc2_bias=b2)
    x64, l64 = oracle.as_f64(wl.tokens.x), oracle.as_f64(wl.tokens.logits)
    ref = brute.dense_masked_forward(x64, l64, wl.weights, wl.spec, fc1_bias=b1, fc2_bias=b2)
    assert _close(got, ref)
    for kw in ({"fc1_bias": b1, "fc2_bias": b2, "bias_after_silu": True},
               {"fc2_bias": b2}, {"fc1_bias": b1}):
        assert not _close(got, brute.dense_masked_forward(x64, l64, wl.weights, wl.spec, **kw))
    # the FC2 bias enters linearly: out(b2) - out(0) = sum_j w_j b2[e_j]
    nob = oracle.forward(oracle.Layer.from_spec(wl.spec), wl.tokens.x, wl.tokens.logits,
                         wl.weights, fc1_bias=b1)
    ids, w = oracle.route(wl.tokens.logits, wl.spec.top_k)
    lin = np.einsum("tj,tjm->tm", w, b2[ids])
    assert _close(got - nob, lin)


@pytest.mark.parametrize("bits,bs", [(4, 32), (3, 64), (2, 128)])
def test_dequant_zero_point_tensor(bits, bs):
    """A zero-point tensor (one code per row and quant block) gives, exactly,
    (q - zp[n][k/bs]) * s; filled with the scalar zero point it reproduces the
    scalar-zero-point dequant bit for bit."""
    rng = np.random.default_rng(bits * 100 + bs)
    N, K = 24, 4 * bs
    q = rng.integers(0, 1 << bits, size=(N, K))
    codes = brute.pack_codes(q, bits)
    scales = (np.abs(rng.standard_normal((N, K // bs))) * 0.05 + 1e-3).astype(np.float16)
    zps = rng.integers(0, 1 << bits, size=(N, K // bs)).astype(np.uint8)
    got = oracle.dequant(codes, scales, bits, bs, 0, K, zero_points=zps)
    ref = (q - np.repeat(zps.astype(np.int64), bs, axis=1)) * np.repeat(
        scales.astype(np.float64), bs, axis=1)
    assert np.array_equal(got, ref)
    assert np.array_equal(got, brute.dequant_dense(codes, scales, bits, bs, zps, K))
    zc = 1 << (bits - 1)
    full = np.full_like(zps, zc)
    assert np.array_equal(oracle.dequant(codes, scales, bits, bs, 0, K, zero_points=full),
                          oracle.dequant(codes, scales, bits, bs, zc, K))


def test_zero_point_tensors_against_dense_masked():
    """Per-block zero points in both FC1 and FC2: the oracle equals the dense
    masked mixture; an off-by-one zero point would be noticed."""
    wl = qi.make_workload("tiny")
    rng = np.random.default_rng(31)
    z1 = rng.integers(0, 16, size=wl.weights.fc1_scales.shape).astype(np.uint8)
    z2 = rng.integers(0, 16, size=wl.weights.fc2_scales.shape).astype(np.uint8)
    got = oracle.forward(oracle.Layer.from_spec(wl.spec), wl.tokens.x, wl.tokens.logits,
                         wl.weights, fc1_zero_points=z1, fc2_zero_points=z2)
    x64, l64 = oracle.as_f64(wl.tokens.x), oracle.as_f64(wl.tokens.logits)
    ref = brute.dense_masked_forward(x64, l64, wl.weights, wl.spec, fc1_zero_points=z1,
                                     fc2_zero_points=z2)
    assert _close(got, ref)
    assert not _close(got, brute.dense_masked_forward(x64, l64, wl.weights, wl.spec,
                                                      fc1_zero_points=z1, fc2_zero_points=z2,
                                                      zp_delta=1))


def test_tiny_layer_against_dense_masked():
    wl = qi.make_workload("tiny")
    acc = _run(wl)
    ref = _brute(wl)
    assert _close(acc, ref)
    f32, _ = oracle.round_output(acc)
    f32_ref = ref.astype(np.float32)
    ulps = np.abs(f32.view(np.int32).astype(np.int64) - f32_ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1


@pytest.mark.parametrize("name,T", [("decode", 4), ("int3", 3), ("stack", 2), ("prefill", 3)])
def test_qwen_shaped_slices_against_dense_masked(name, T):
    wl = qi.make_workload(name, T=T)
    acc = _run(wl, nthreads=4)
    ref = _brute(wl)
    assert _close(acc, ref)


@pytest.mark.parametrize("bits,bs", [(4, 64), (4, 128), (3, 32), (3, 128), (2, 64), (2, 128)])
def test_formats_against_dense_masked(bits, bs):
    spec = _small_spec(hidden=256, inter=128, num_experts=6, top_k=3, bits=bits,
                       block_size=bs, zero_point=1 << (bits - 1), act_dtype="bf16")
    wl = qi.make_layer(spec, T=9, seed=100 + bits * 10 + bs)
    assert _close(_run(wl), _brute(wl))


def test_planted_mistakes_are_visible():
    """Each plausible slip in the layer definition moves the result far beyond
    rounding noise, so the dense-masked pin would catch it."""
    wl = qi.make_workload("tiny")
    acc = _run(wl)
    for kw in ({"swap_gate_up": True}, {"zp_delta": 1}, {"softmax_all": True}):
        bad = _brute(wl, **kw)
        assert not _close(acc, bad, rtol=1e-3), kw


def test_single_expert_is_dense_swiglu_mlp():
    """E=1, k=1 reduces to a dense SwiGLU MLP on the dequantized weights."""
    spec = _small_spec(num_experts=1, top_k=1, hidden=128, inter=64, act_dtype="bf16")
    wl = qi.make_layer(spec, T=7, seed=5)
    acc = _run(wl)
    W1 = brute.dequant_dense(wl.weights.fc1_codes[0], wl.weights.fc1_scales[0], 4, 32, 8, 128)
    W2 = brute.dequant_dense(wl.weights.fc2_codes[0], wl.weights.fc2_scales[0], 4, 32, 8, 64)
    x = torch.from_numpy(oracle.as_f64(wl.tokens.x))
    gu = x @ torch.from_numpy(W1).T
    h = torch.nn.functional.silu(gu[:, :64]) * gu[:, 64:]
    ref = (h @ torch.from_numpy(W2).T).numpy()
    assert _close(acc, ref)


def test_zero_point_codes_give_zero_output():
    spec = _small_spec(act_dtype="bf16")
    wl = qi.make_layer(spec, T=5, seed=9)
    q1 = np.full((spec.num_experts, 2 * spec.inter, spec.hidden), spec.zero_point)
    wl.weights.fc1_codes = np.ascontiguousarray(brute.pack_codes(q1, 4))
    acc = _run(wl)
    assert np.all(acc == 0.0)


def test_identical_experts_reduce_to_one():
    """All experts equal: the routing weights sum to one, so the output is the
    single-expert FFN whatever the routing."""
    spec = _small_spec(num_experts=5, top_k=3, act_dtype="bf16")
    wl = qi.make_layer(spec, T=6, seed=21)
    w = wl.weights
    for arr_name in ("fc1_codes", "fc1_scales", "fc2_codes", "fc2_scales"):
        a = getattr(w, arr_name)
        setattr(w, arr_name, np.ascontiguousarray(np.broadcast_to(a[:1], a.shape)))
    acc = _run(wl)
    one = qi.Workload("one", qi.spec_with(spec, num_experts=1, top_k=1), wl.tokens, qi.LayerWeights(
        w.fc1_codes[:1].copy(), w.fc1_scales[:1].copy(), w.fc2_codes[:1].copy(), w.fc2_scales[:1].copy()))
    one.tokens = qi.Tokens(wl.tokens.x, wl.tokens.logits[:, :1].contiguous())
    ref = _run(one)
    assert _close(acc, ref, rtol=1e-13)


def test_packed_equals_per_sequence_runs():
    """Token-local routing: concatenating per-sequence runs reproduces the
    packed run bit for bit."""
    wl = qi.make_workload("prefill", T=24)
    assert len(wl.tokens.seq_lens) == 16 and sum(wl.tokens.seq_lens) == 24
    packed = _run(wl, nthreads=3)
    parts, s = [], 0
    for n in wl.tokens.seq_lens:
        sub = qi.Workload("seq", wl.spec, qi.Tokens(wl.tokens.x[s:s + n], wl.tokens.logits[s:s + n]),
                          wl.weights)
        parts.append(_run(sub, nthreads=2))
        s += n
    assert np.array_equal(np.concatenate(parts), packed)


def test_thread_count_does_not_change_result():
    wl = qi.make_workload("decode", T=4)
    assert np.array_equal(_run(wl, nthreads=1), _run(wl, nthreads=4))


def test_empty_input():
    wl = qi.make_workload("tiny", T=0)
    assert _run(wl).shape == (0, 64)


def test_routing_weights_sum_to_one_on_workloads():
    for name, T in (("decode", 4), ("prefill", 512), ("stack", 256)):
        wl = qi.make_workload(name, T=T)
        _, w = oracle.route(wl.tokens.logits, wl.spec.top_k)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_zipf_skew_present():
    wl = qi.make_workload("prefill", T=2048)
    ids, _ = oracle.route(wl.tokens.logits, 8)
    counts = np.bincount(ids.reshape(-1), minlength=128)
    assert counts.max() > 0.8 * 2048          # top experts take nearly every token
    assert (counts == 0).sum() > 10           # a long tail of idle experts


# ---------------------------------------------------------------- fp16 datapath emulation
#
# The grouped (prefill) path feeds fp16 operands to the matrix cores. The
# oracle's emulation of those rounding points (EMU_*) is pinned against
# numpy's own float16 conversion and an independent vectorized twin in
# oracle/brute.py, and each plausible slip in it is shown to be visible.

def _half_bits_numpy(v):
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def test_double_to_half_against_numpy():
    """Nearest fp16 of float64 values against numpy's conversion: every fp16
    value, every exact tie between neighbours (and a hair either side of
    it), the overflow and underflow edges, and random values over the whole
    range, both signs."""
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = allh[np.isfinite(allh.view(np.float16))].view(np.float16).astype(np.float64)
    pos = np.unique(fin[fin >= 0])
    mids = (pos[:-1] + pos[1:]) / 2                       # exact ties (float64 holds them)
    hair = np.concatenate([np.nextafter(mids, 0), np.nextafter(mids, np.inf)])
    edges = np.array([65504.0, 65519.99, 65520.0, 65535.0, 1e6, 2.0 ** -24, 2.0 ** -25,
                      3 * 2.0 ** -26, 2.0 ** -26, 2.0 ** -14 - 2.0 ** -25, 0.0, np.inf])
    rng = np.random.default_rng(3)
    rnd = np.ldexp(rng.random(200000) + 0.5, rng.integers(-30, 18, 200000))
    v = np.concatenate([fin, mids, hair, edges, rnd])
    v = np.concatenate([v, -v])
    got = oracle.double_to_half_bits(v)
    assert np.array_equal(got, _half_bits_numpy(v))
    nan = oracle.double_to_half_bits(np.array([np.nan, -np.nan]))
    assert all((b & 0x7C00) == 0x7C00 and (b & 0x3FF) != 0 for b in nan)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_dequant_f16_exhaustive_codes_times_scales(bits):
    """Every code times every fp16 scale (infinities and NaN included), for
    every zero point: the fp16 operand is numpy's float16 of the exact
    product (q - zp) * s."""
    ncodes = 1 << bits
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    K = 8 * ncodes
    q = np.tile(np.arange(ncodes), K // ncodes)
    packed = np.broadcast_to(brute.pack_codes(q[None], bits), (allh.size, K * bits // 8)).copy()
    scales = allh.view(np.float16)[:, None]
    s64 = scales.astype(np.float64)
    for zp in range(ncodes):
        got = oracle.dequant_f16(packed, scales, bits, K, zp, K)
        with np.errstate(invalid="ignore"):
            exact = (q[None, :] - zp).astype(np.float64) * s64
        ref = _half_bits_numpy(exact)
        nan = np.isnan(exact)
        assert np.array_equal(np.isnan(got.view(np.float16)), nan)
        assert np.array_equal(got[~nan], ref[~nan])


def _emu_rows():
    """Rows that exercise every branch of the range scaling: ordinary values,
    rows far above and far below the fp16 range, zero rows, a row with an
    infinity, and rows whose 32-wide chunks differ by many binades (so the
    common exponent pushes some chunks into the fp16 subnormals)."""
    rng = np.random.default_rng(11)
    rows = [rng.standard_normal(256), rng.standard_normal(256) * 2.0 ** 20,
            rng.standard_normal(256) * 2.0 ** -20, np.zeros(256),
            np.r_[rng.standard_normal(255), np.inf]]
    mixed = rng.standard_normal(256) * 3
    mixed[:32] *= 2.0 ** 30
    mixed[64:96] *= 2.0 ** -14
    rows.append(mixed)
    for shift in (12, 16, 17, 24, 40):
        r = rng.standard_normal(256)
        r[32:64] *= 2.0 ** shift
        rows.append(r)
    return np.stack(rows)


def test_emulated_activation_rounding_matches_numpy_twin():
    rows = _emu_rows()
    got = oracle.emulate_x_rows(rows)
    ref = brute.f16_rows_scaled(rows)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # ordinary bf16 activations pass through exactly
    x = torch.randn(16, 256).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.emulate_x_rows(x), x)
    # without the scaling, large rows would overflow fp16 and tiny ones lose bits
    plant = brute.f16(rows[1:3])
    assert not np.array_equal(plant, ref[1:3])


def test_emulated_h_rounding_matches_numpy_twin():
    rows = _emu_rows()
    got = oracle.emulate_h_rows(rows)
    ref = brute.f16_chunks_scaled(rows)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # ordinary values: plain fp16 rounding, no exponent anywhere
    assert np.array_equal(got[0], brute.f16(rows[0]))
    # each slip in the chunk logic changes some row
    for kw in ({"plant_no_chunk_exponent": True}, {"plant_no_common_exponent": True}):
        bad = brute.f16_chunks_scaled(rows, **kw)
        assert not np.array_equal(bad[ok], ref[ok]), kw


def _emu_forward(wl, x=None):
    x = wl.tokens.x if x is None else x
    return oracle.forward(oracle.Layer.from_spec(wl.spec), x, wl.tokens.logits, wl.weights,
                          nthreads=4, emulate=oracle.EMU_F16_DATAPATH)


def _emu_brute(wl, x=None, **kw):
    x = wl.tokens.x if x is None else x
    return brute.dense_masked_forward(oracle.as_f64(x), oracle.as_f64(wl.tokens.logits),
                                      wl.weights, wl.spec, emu_x=True, emu_w=True, emu_h=True, **kw)


@pytest.mark.parametrize("name,T,xscale", [("tiny", 9, 1.0), ("decode", 2, 1.0), ("int3", 2, 1.0),
                                           ("stack", 2, 1.0), ("decode", 2, 2.0 ** 9),
                                           ("tiny", 6, 2.0 ** -16)])
def test_emulated_datapath_against_dense_masked(name, T, xscale):
    """The whole layer with the fp16 datapath's rounding points, against the
    dense masked twin with the same points: fp32 activations (tiny), bf16
    activations at every format, activations large enough that h leaves the
    fp16 range (its chunk exponents engage) and activations so small that
    they would fall into the fp16 subnormals without the per-token scaling."""
    wl = qi.make_workload(name, T=T)
    x = (wl.tokens.x.to(torch.float64) * xscale).to(wl.tokens.x.dtype)
    acc = _emu_forward(wl, x)
    ref = _emu_brute(wl, x)
    assert np.isfinite(ref).all()
    assert _close(acc, ref, rtol=1e-10)
    plain = _brute(qi.Workload(wl.name, wl.spec, qi.Tokens(x, wl.tokens.logits), wl.weights))
    # the rounding points move the result, but only by fp16 rounding noise
    rel = np.linalg.norm(acc - plain, axis=1) / np.linalg.norm(plain, axis=1)
    assert 1e-6 < rel.max() < 5e-3, rel.max()


def test_emulated_datapath_planted_mistakes_are_visible():
    """Each slip in the emulated rounding points moves the layer output far
    beyond the agreement of the two emulations (1e-10 relative)."""
    wl = qi.make_workload("decode", T=2)
    acc = _emu_forward(wl)
    for kw in ({"plant_h_unrounded": True},):
        assert not _close(acc, _emu_brute(wl, **kw), rtol=1e-8), kw
    w_plain = brute.dense_masked_forward(oracle.as_f64(wl.tokens.x), oracle.as_f64(wl.tokens.logits),
                                         wl.weights, wl.spec, emu_x=True, emu_h=True)
    assert not _close(acc, w_plain, rtol=1e-8)
    big = (wl.tokens.x.to(torch.float64) * 2.0 ** 9).to(torch.bfloat16)
    acc_big = _emu_forward(wl, big)
    bad = _emu_brute(wl, big, plant_h_no_chunk_exponent=True)
    assert not np.isfinite(bad).all() or not _close(acc_big, bad, rtol=1e-8)
    wt = qi.make_workload("tiny", T=6)      # fp32 activations: x rounding matters
    x_plain = brute.dense_masked_forward(oracle.as_f64(wt.tokens.x), oracle.as_f64(wt.tokens.logits),
                                         wt.weights, wt.spec, emu_w=True, emu_h=True)
    assert not _close(_emu_forward(wt), x_plain, rtol=1e-8)
    huge = (wt.tokens.x.to(torch.float64) * 2.0 ** 20).to(torch.float32)
    acc_h = _emu_forward(wt, huge)
    bad = _emu_brute(wt, huge, plant_x_unscaled=True)
    assert not np.isfinite(bad).all() or not _close(acc_h, bad, rtol=1e-8)
