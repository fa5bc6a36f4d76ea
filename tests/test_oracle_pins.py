"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test compares the oracle with a library routine (torch / numpy / scipy casts and
matmuls), a brute-force full sort, or a closed form, on inputs chosen so that a plausible
mistake (a dropped term, a wrong index or sign, a transposed operand, a swapped half)
fails at least one of them.
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle

rng = np.random.default_rng(12345)


# ---------------------------------------------------------------------------------------
# codecs
# ---------------------------------------------------------------------------------------

def test_bf16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = oracle.bf16_to_f32(bits)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_encode_round_to_nearest_even():
    # random values, exact halfway cases with even and odd kept parts, and near-halfway ones
    kept = rng.integers(0, 0x7F7F, 4000, dtype=np.uint32)
    half = (kept << 16) | 0x8000
    vals = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 7,
                           half.view(np.float32), (half + 1).view(np.float32), (half - 1).view(np.float32),
                           np.array([0.0, -0.0, 1e-40, 3.4e38, -3.4e38], np.float32)])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (oracle.f32_to_bf16(vals) == ref).all()


def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = oracle.f16_to_f32(bits)
    assert ((got == ref) | (np.isnan(got) & np.isnan(ref))).all()


def _torch_e4m3_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def test_e4m3_decode_exhaustive():
    codes = np.arange(256, dtype=np.uint8)
    ref = _torch_e4m3_decode(codes)
    got = oracle.e4m3_to_f32(codes)
    assert ((got == ref) | (np.isnan(got) & np.isnan(ref))).all()
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0x7E] == 448.0
    assert np.isfinite(got[[c for c in range(256) if c not in (0x7F, 0xFF)]]).all()


def test_e4m3_encode_rne_and_saturation():
    vals = _torch_e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)   # 0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2                       # exact ties: must go to the even code
    probe = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000)]).astype(np.float32)
    probe = np.concatenate([probe, -probe, rng.uniform(-460, 460, 3000).astype(np.float32),
                            np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e30, -1e30], np.float32)])
    ref = torch.from_numpy(np.clip(probe, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.f32_to_e4m3(probe)
    # -0.0 may legitimately encode as 0x80; compare decoded values for zeros
    same = (got == ref) | ((_torch_e4m3_decode(got) == 0) & (_torch_e4m3_decode(ref) == 0))
    assert same.all()
    tie_codes = oracle.f32_to_e4m3(mids.astype(np.float32))
    assert (tie_codes % 2 == 0).all()


def test_sigmoid_exhaustive_over_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    x = x[np.isfinite(x)]
    ref = scipy.special.expit(x.astype(np.float64)).astype(np.float32)
    got = oracle.sigmoid(x)
    assert (got.view(np.uint32) == ref.view(np.uint32)).all()


# ---------------------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------------------

def _brute_topk(keys, k, allowed=None):
    cand = [e for e in range(len(keys)) if allowed is None or allowed[e]]
    return sorted(cand, key=lambda e: (-float(keys[e]), e))[:k]


def _bf16_bits(a32):
    return torch.from_numpy(np.asarray(a32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("E,k", [(4, 1), (8, 2), (16, 4), (16, 16), (64, 8)])
@pytest.mark.parametrize("ties", [False, True])
def test_softmax_topk_matches_full_sort(E, k, ties):
    T = 40
    x = rng.integers(-1, 2, (T, E)).astype(np.float32) if ties else rng.standard_normal((T, E)).astype(np.float32)
    bits = _bf16_bits(x)
    xf = oracle.bf16_to_f32(bits)
    for renorm in (True, False):
        ids, w = oracle.route(oracle.ROUTE_SOFTMAX, E, k, bits, renormalize=renorm)
        p = torch.softmax(torch.from_numpy(xf.astype(np.float64)), dim=1).numpy()
        for t in range(T):
            exp = _brute_topk(xf[t], k)
            assert list(ids[t]) == exp
            ref = p[t, exp] / p[t, exp].sum() if renorm else p[t, exp]
            np.testing.assert_allclose(w[t], ref, rtol=1e-6)
        if renorm:
            np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, rtol=0, atol=k * 2e-7)
    if k == E:   # every expert chosen and renormalised: the full softmax in rank order
        ids, w = oracle.route(oracle.ROUTE_SOFTMAX, E, k, bits, renormalize=True)
        np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-6)


def test_route_fp32_logits_and_scaling():
    x = rng.standard_normal((9, 8)).astype(np.float32)
    ids, w = oracle.route(oracle.ROUTE_SOFTMAX, 8, 3, x, renormalize=True, routed_scaling=2.0)
    for t in range(9):
        assert list(ids[t]) == _brute_topk(x[t], 3)
    np.testing.assert_allclose(w.sum(1), 2.0, rtol=1e-6)


@pytest.mark.parametrize("with_bias", [False, True])
def test_sigmoid_topk_matches_full_sort(with_bias):
    T, E, k = 50, 16, 2
    x = rng.standard_normal((T, E)).astype(np.float32) * 3
    x[:10] = rng.integers(-1, 2, (10, E))                      # forced ties
    bits = _bf16_bits(x)
    xf = oracle.bf16_to_f32(bits)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32) if with_bias else None
    ids, w = oracle.route(oracle.ROUTE_SIGMOID, E, k, bits, renormalize=False, bias=bias)
    s = scipy.special.expit(xf.astype(np.float64)).astype(np.float32)
    key = s + bias if with_bias else s
    for t in range(T):
        exp = _brute_topk(key[t], k)
        assert list(ids[t]) == exp
        np.testing.assert_allclose(w[t], s[t, exp], rtol=1e-7)


def _brute_grouped(xf, bias, E, k, ng, tg, scale, renorm):
    s = scipy.special.expit(xf.astype(np.float64)).astype(np.float32)
    key = (s + bias).astype(np.float32)
    G = E // ng
    score = []
    for g in range(ng):
        top = sorted(key[g * G:(g + 1) * G].tolist(), reverse=True)[:2]
        score.append(np.float32(top[0]) + np.float32(top[1]) if len(top) == 2 else np.float32(top[0]))
    kept = sorted(range(ng), key=lambda g: (-float(score[g]), g))[:tg]
    allowed = np.zeros(E, bool)
    for g in kept:
        allowed[g * G:(g + 1) * G] = True
    ids = _brute_topk(key, k, allowed)
    sel = s[ids].astype(np.float64)
    w = (sel / sel.sum() if renorm else sel) * scale
    return ids, w


@pytest.mark.parametrize("E,ng,tg,k", [(256, 8, 4, 8), (64, 8, 3, 6), (16, 4, 2, 3), (32, 16, 16, 4)])
def test_grouped_gate_matches_full_sort(E, ng, tg, k):
    T = 30
    x = rng.standard_normal((T, E)).astype(np.float32)
    x[:6] = rng.integers(-1, 2, (6, E))                        # forced ties
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    bias[: E // 4] = 0.0                                        # equal biases: more ties
    bits = _bf16_bits(x)
    xf = oracle.bf16_to_f32(bits)
    for renorm in (True, False):
        ids, w = oracle.route(oracle.ROUTE_GROUPED_SIGMOID_BIAS, E, k, bits, renormalize=renorm,
                              n_group=ng, topk_group=tg, routed_scaling=2.5, bias=bias)
        for t in range(T):
            eids, ew = _brute_grouped(xf[t], bias, E, k, ng, tg, 2.5, renorm)
            assert list(ids[t]) == eids
            np.testing.assert_allclose(w[t], ew, rtol=1e-6)
        if renorm:
            np.testing.assert_allclose(w.astype(np.float64).sum(1), 2.5, rtol=2e-6)


def test_grouped_gate_special_cases():
    T, E, k = 40, 32, 4
    x = rng.standard_normal((T, E)).astype(np.float32)
    bits = _bf16_bits(x)
    xf = oracle.bf16_to_f32(bits)
    zero = np.zeros(E, np.float32)
    # one group, no bias: plain sigmoid top-k, i.e. top-k of the logits themselves
    ids, w = oracle.route(oracle.ROUTE_GROUPED_SIGMOID_BIAS, E, k, bits, renormalize=False,
                          n_group=1, topk_group=1, bias=zero)
    ids2, w2 = oracle.route(oracle.ROUTE_SIGMOID, E, k, bits, renormalize=False)
    assert (ids == ids2).all() and (w == w2).all()
    for t in range(T):
        assert list(ids[t]) == _brute_topk(xf[t], k)   # no sigmoid ties at these magnitudes
    # all groups kept: the ungrouped biased top-k
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    ids, _ = oracle.route(oracle.ROUTE_GROUPED_SIGMOID_BIAS, E, k, bits, n_group=8, topk_group=8, bias=bias)
    ids2, _ = oracle.route(oracle.ROUTE_SIGMOID, E, k, bits, bias=bias)
    assert (ids == ids2).all()


def test_route_rejects_bad_arguments():
    x = np.zeros((2, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.route(oracle.ROUTE_SOFTMAX, 8, 9, x)
    with pytest.raises(ValueError):
        oracle.route(oracle.ROUTE_GROUPED_SIGMOID_BIAS, 8, 2, x, n_group=3, topk_group=1)
    with pytest.raises(ValueError):
        oracle.route(oracle.ROUTE_GROUPED_SIGMOID_BIAS, 8, 5, x, n_group=4, topk_group=2)


# ---------------------------------------------------------------------------------------
# align
# ---------------------------------------------------------------------------------------

def _check_align(ids, T, k, E, BM):
    flat = ids.reshape(-1)
    a = oracle.align(ids, T, k, E, BM)
    P = T * k
    cap = oracle.align_capacity(T, k, E, BM)
    counts = np.bincount(flat, minlength=E)
    padded = -(-counts // BM) * BM
    off = np.concatenate([[0], np.cumsum(padded)[:-1]]).astype(np.int64)
    exp_sorted = np.full(cap, P, np.int32)
    exp_eids = np.full(cap // BM, -1, np.int32)
    order = np.argsort(flat, kind="stable")                # brute force: a stable sort by expert
    pos = 0
    for e in range(E):
        exp_sorted[off[e]:off[e] + counts[e]] = order[pos:pos + counts[e]]
        exp_eids[off[e] // BM:(off[e] + padded[e]) // BM] = e
        pos += counts[e]
    assert (a["expert_counts"] == counts).all() and counts.sum() == P
    assert (a["sorted_token_ids"] == exp_sorted).all()
    assert (a["expert_ids"] == exp_eids).all()
    npp = int(a["num_tokens_post_padded"][0])
    assert npp == padded.sum() and npp % BM == 0 and npp <= cap and cap % BM == 0
    # each pair appears exactly once; the rest are fillers; permute then unpermute is the identity
    valid = a["sorted_token_ids"] < P
    assert np.sort(a["sorted_token_ids"][valid]).tolist() == list(range(P))
    assert (~valid).sum() == cap - P
    assert (a["sorted_token_ids"][a["inv_pos"]] == np.arange(P)).all()
    # each block's rows belong to the block's expert
    blk = a["inv_pos"] // BM
    assert (a["expert_ids"][blk] == flat).all()
    return a


@pytest.mark.parametrize("BM", [1, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("T,k,E", [(1, 1, 8), (3, 2, 8), (37, 2, 8), (100, 8, 64), (64, 8, 256), (257, 1, 16)])
def test_align_matches_stable_sort(T, k, E, BM):
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _check_align(ids, T, k, E, BM)


def test_align_zero_token_experts_and_skew():
    T, k, E, BM = 200, 1, 16, 16
    ids = np.where(rng.random((T, k)) < 0.8, 3, 11).astype(np.int32)    # only two experts used
    a = _check_align(ids, T, k, E, BM)
    assert (a["expert_counts"][[e for e in range(E) if e not in (3, 11)]] == 0).all()


def test_align_capacity_is_tight():
    # worst case: every used expert ends with a lone pair in its last block
    T, k, E, BM = 8 * 17, 1, 8, 16
    ids = np.repeat(np.arange(8), 17).astype(np.int32).reshape(T, k)
    a = _check_align(ids, T, k, E, BM)
    assert int(a["num_tokens_post_padded"][0]) == oracle.align_capacity(T, k, E, BM)


def test_align_empty():
    a = oracle.align(np.zeros((0, 2), np.int32), 0, 2, 8, 16)
    assert a["sorted_token_ids"].size == 0 and int(a["num_tokens_post_padded"][0]) == 0


# ---------------------------------------------------------------------------------------
# the layer (FFN and slot combination)
# ---------------------------------------------------------------------------------------

def _dense_ffn(x, W1, W3, W2):
    """SiLU-gated FFN with torch fp64 matmuls: W2 (SiLU(W1 x) * (W3 x))."""
    x, W1, W3, W2 = (torch.as_tensor(np.asarray(a, np.float64)) for a in (x, W1, W3, W2))
    return (torch.nn.functional.silu(x @ W1.T) * (x @ W3.T) @ W2.T).numpy()


def _bf16_weights(E, H, I):
    w13 = (rng.standard_normal((E, 2 * I, H)) / np.sqrt(H)).astype(np.float32)
    w2 = (rng.standard_normal((E, H, I)) / np.sqrt(I)).astype(np.float32)
    b13, b2 = _bf16_bits(w13), _bf16_bits(w2)
    return oracle.Weights(oracle.BF16, E, H, I, b13, b2), oracle.bf16_to_f32(b13), oracle.bf16_to_f32(b2)


def test_forward_single_expert_is_dense_ffn():
    T, H, I = 12, 48, 80
    W, w13, w2 = _bf16_weights(1, H, I)
    xb = _bf16_bits(rng.standard_normal((T, H)))
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    out = oracle.forward(W, xb, ids, w)
    ref = _dense_ffn(oracle.bf16_to_f32(xb), w13[0, :I], w13[0, I:], w2[0])
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_forward_slots_pick_their_experts():
    T, E, k, H, I = 10, 4, 2, 32, 64
    W, w13, w2 = _bf16_weights(E, H, I)
    xb = _bf16_bits(rng.standard_normal((T, H)))
    xf = oracle.bf16_to_f32(xb)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    for j in range(k):                     # one-hot slot weights: the output is that slot's expert
        w = np.zeros((T, k), np.float32)
        w[:, j] = 1.0
        out = oracle.forward(W, xb, ids, w)
        for t in range(T):
            e = ids[t, j]
            np.testing.assert_allclose(out[t], _dense_ffn(xf[t], w13[e, :I], w13[e, I:], w2[e]),
                                       rtol=1e-10, atol=1e-12)
    # identical experts: out = (sum of slot weights) * FFN(x)
    Wsame = oracle.Weights(oracle.BF16, E, H, I, np.repeat(W.arrays["w13"][:1], E, 0),
                           np.repeat(W.arrays["w2"][:1], E, 0))
    w = rng.random((T, k)).astype(np.float32)
    out = oracle.forward(Wsame, xb, ids, w)
    ref = _dense_ffn(xf, w13[0, :I], w13[0, I:], w2[0]) * w.astype(np.float64).sum(1, keepdims=True)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    # token subset equals the matching rows of the full output
    full = oracle.forward(W, xb, ids, w)
    sub = oracle.forward(W, xb, ids, w, tokens=[7, 2])
    np.testing.assert_array_equal(sub, full[[7, 2]])


def test_forward_int4_dequantises_groups():
    E, k, T, H, I = 3, 2, 6, 256, 128
    def make(N, K):
        q = rng.integers(0, 16, (E, N, K)).astype(np.uint8)
        z = rng.integers(0, 16, (E, N, K // 128)).astype(np.float16)
        s = (rng.random((E, N, K // 128)) * 0.02 + 0.001).astype(np.float16)
        packed = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
        deq = (q.astype(np.float64) - np.repeat(z.astype(np.float64), 128, -1)) * np.repeat(s.astype(np.float64), 128, -1)
        # scales and zero points are stored group-major: [E, K/128, N]
        gm = lambda a: np.ascontiguousarray(a.transpose(0, 2, 1)).view(np.uint16)  # noqa: E731
        return packed, gm(s), gm(z), deq
    p13, s13, z13, d13 = make(2 * I, H)
    p2, s2, z2, d2 = make(H, I)
    W = oracle.Weights(oracle.INT4_G128, E, H, I, p13, p2, w13_s=s13, w13_z=z13, w2_s=s2, w2_z=z2)
    assert W.value(0, 1, 5, 129) == d13[1, 5, 129] and W.value(1, 2, 7, 6) == d2[2, 7, 6]
    xb = _bf16_bits(rng.standard_normal((T, H)))
    xf = oracle.bf16_to_f32(xb)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    out = oracle.forward(W, xb, ids, w)
    for t in range(T):
        ref = sum(float(w[t, j]) * _dense_ffn(xf[t], d13[e, :I], d13[e, I:], d2[e]) for j, e in enumerate(ids[t]))
        np.testing.assert_allclose(out[t], ref, rtol=1e-9, atol=1e-9)


def _e4m3_grid_weights(E, N, K):
    codes = rng.integers(0, 0x7F, (E, N, K)).astype(np.uint8) | (rng.integers(0, 2, (E, N, K)).astype(np.uint8) << 7)
    codes[codes == 0xFF] = 0xFE
    return codes


def test_forward_fp8_exact_case():
    """Hidden on the E4M3 grid (so the first quantisation is exact) and an identity down
    projection (so the output is the quantised intermediate itself): the w8a8 result then
    equals sum_j w_j * dq(q(h_j)) with h from torch matmuls and the codes from torch's cast."""
    E, k, T, H = 3, 2, 8, 64
    I = H
    c13 = _e4m3_grid_weights(E, 2 * I, H)
    s13 = (rng.random(E) * 0.01 + 0.001).astype(np.float32)
    c2 = np.zeros((E, H, I), np.uint8)
    c2[:, np.arange(H), np.arange(H)] = 0x38                   # 1.0
    s2w = np.ones(E, np.float32)
    W = oracle.Weights(oracle.FP8_E4M3, E, H, I, c13, c2, w13_scale=s13, w2_scale=s2w)
    xc = _e4m3_grid_weights(1, T, H)[0]
    xc[0, 0] = 0x7E                                            # the largest magnitude: 448
    xs = np.float32(2.0 ** -6)
    x = _torch_e4m3_decode(xc) * xs                            # exact in bf16
    xb = _bf16_bits(x)
    assert (oracle.bf16_to_f32(xb) == x).all()
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    out, sc = oracle.forward(W, xb, ids, w, return_scales=True)
    assert sc[0] == xs
    w13 = _torch_e4m3_decode(c13).astype(np.float64) * s13[:, None, None]
    h = np.stack([[ _dense_ffn(x[t], w13[e, :I], w13[e, I:], np.eye(H))  # identity: h itself
                    for e in ids[t]] for t in range(T)]).astype(np.float32)
    amax = np.abs(h).max()
    s2, inv2 = np.float32(amax / np.float32(448)), np.float32(np.float32(448) / amax)
    codes = torch.from_numpy(np.clip(h * inv2, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    hq = _torch_e4m3_decode(codes).astype(np.float64) * np.float64(s2)
    ref = (hq * w[..., None].astype(np.float64)).sum(1)
    assert sc[1] == s2
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-15)
    # the intermediate's largest magnitude lands on the largest code
    _, oq, _ = oracle.fp8_intermediate(W, xb, ids)
    assert np.abs(_torch_e4m3_decode(oq)).max() == 448.0
    assert (oq == codes.reshape(T * k, I)).all()


def test_forward_fp8_close_to_unquantised():
    """w8a8 with random data stays within E4M3's rounding error of the same layer computed on
    the dequantised weights without activation quantisation."""
    E, k, T, H, I = 4, 2, 16, 128, 64
    c13 = _e4m3_grid_weights(E, 2 * I, H)
    c2 = _e4m3_grid_weights(E, H, I)
    s13 = np.full(E, 1.0 / (448 * np.sqrt(H)), np.float32)
    s2 = np.full(E, 1.0 / (448 * np.sqrt(I)), np.float32)
    W = oracle.Weights(oracle.FP8_E4M3, E, H, I, c13, c2, w13_scale=s13, w2_scale=s2)
    xb = _bf16_bits(rng.standard_normal((T, H)))
    xf = oracle.bf16_to_f32(xb)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    out = oracle.forward(W, xb, ids, w)
    d13 = _torch_e4m3_decode(c13).astype(np.float64) * s13[:, None, None]
    d2 = _torch_e4m3_decode(c2).astype(np.float64) * s2[:, None, None]
    ref = np.stack([sum(float(w[t, j]) * _dense_ffn(xf[t], d13[e, :I], d13[e, I:], d2[e])
                        for j, e in enumerate(ids[t])) for t in range(T)])
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 0.1


def test_forward_fp8_all_zero_hidden():
    E, k, T, H, I = 2, 1, 4, 32, 32
    W = oracle.Weights(oracle.FP8_E4M3, E, H, I, _e4m3_grid_weights(E, 2 * I, H), _e4m3_grid_weights(E, H, I),
                       w13_scale=np.ones(E, np.float32), w2_scale=np.ones(E, np.float32))
    out, sc = oracle.forward(W, np.zeros((T, H), np.uint16), np.zeros((T, k), np.int32),
                             np.ones((T, k), np.float32), return_scales=True)
    assert (out == 0).all() and sc[0] == 1.0 and sc[1] == 1.0


def test_forward_empty_batch():
    W, _, _ = _bf16_weights(2, 16, 32)
    out = oracle.forward(W, np.zeros((0, 16), np.uint16), np.zeros((0, 1), np.int32), np.zeros((0, 1), np.float32))
    assert out.shape == (0, 16)


# ---- grouped GEMM over contiguous per-expert segments (EP-MoE) --------------------------

def _bits_bf16(rng, shape):
    """Random bf16 bit patterns of normal values (the top half of fp32 normals)."""
    return (rng.standard_normal(shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _e4m3_to_f64(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.mark.parametrize("sizes", [[3, 0, 5, 1, 7], [0, 0, 16, 0, 0], [1, 1, 1, 1, 1]])
def test_grouped_gemm_bf16_is_segment_matmuls(sizes):
    """bf16: each segment's rows times its expert's transposed weight (numpy fp64 matmul on
    numpy's own bf16 decode); rows past the last segment stay zero."""
    rng = np.random.default_rng(11)
    E, N, K = 5, 24, 40
    M = sum(sizes) + 3
    x, w = _bits_bf16(rng, (M, K)), _bits_bf16(rng, (E, N, K))
    y = oracle.grouped_gemm(oracle.BF16, E, N, K, x, w, sizes)
    ref = np.zeros((M, N))
    r = 0
    for e, m in enumerate(sizes):
        ref[r:r + m] = _bf16_to_f64(x[r:r + m]) @ _bf16_to_f64(w[e]).T
        r += m
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    assert (y[sum(sizes):] == 0).all()


def test_grouped_gemm_fp8_applies_per_tensor_scales():
    """E4M3 codes (decoded by torch) with the activation scale and each expert's own
    weight scale."""
    rng = np.random.default_rng(12)
    E, N, K = 4, 16, 48
    sizes = [6, 2, 0, 9]
    M = sum(sizes)
    codes = lambda shape: np.where(((v := rng.integers(0, 256, shape, dtype=np.uint8)) & 0x7F) == 0x7F, 0, v).astype(np.uint8)  # noqa: E731
    x, w = codes((M, K)), codes((E, N, K))
    ws = np.array([0.5, 0.125, 3.0, 0.01], np.float32)
    y = oracle.grouped_gemm(oracle.FP8_E4M3, E, N, K, x, w, sizes, x_scale=0.37, w_scale=ws)
    ref = np.zeros((M, N))
    r = 0
    for e, m in enumerate(sizes):
        ref[r:r + m] = np.float64(np.float32(0.37)) * np.float64(ws[e]) * (_e4m3_to_f64(x[r:r + m]) @ _e4m3_to_f64(w[e]).T)
        r += m
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_grouped_gemm_rejects_bad_sizes():
    E, N, K = 2, 8, 8
    x, w = np.zeros((4, K), np.uint16), np.zeros((E, N, K), np.uint16)
    for sizes in ([3, 2], [-1, 2]):   # past M; negative
        with pytest.raises(ValueError):
            oracle.grouped_gemm(oracle.BF16, E, N, K, x, w, sizes)
