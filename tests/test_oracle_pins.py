"""Pins of the fp64 oracle to facts fixed outside itself (no GPU needed).

Each test checks the oracle against something other than its own code: the
worked example of the aclnnIncreFlashAttention guide (section 7) in closed
form, a whole-matrix brute force, torch's float64 scaled_dot_product_attention
(a third-party library routine), closed forms, and invariants the pages fix
(rows sum to one through the LSE, lossless split-and-merge, GQA sharing,
length truncation ignoring whatever the padding holds).
"""
import math
import os

import numpy as np
import pytest

import fa_synth
import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ifa_worked_example.txt")


def tiny(layout="BNSD", B=2, QN=4, KVN=2, QS=5, KVS=17, D=16, dtype="bf16", std=1.0,
         scale=None, mask="none", lens=None, seed=3):
    spec = fa_synth.Spec("tiny", layout, B, QN, KVN, QS, KVS, D, dtype, std=std, scale=scale,
                         mask=mask, lens=lens, seed=seed)
    return fa_synth.make(spec)


def prob_of(inp, mode=None, lens="inp"):
    p = oracle.Problem.from_inputs(inp, mode)
    return p


def dec(bits, dtype):
    return oracle.decode16(bits, dtype)


# ---------------------------------------------------------------- worked example

def read_golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = rest
    return vals


def test_worked_example_closed_form():
    g = read_golden()
    B, QN, KVN, QS, KVS, D = (int(g[k][0]) for k in ("B", "QN", "KVN", "QS", "KVS", "D"))
    one = fa_synth.round_bits(np.ones(1, np.float32), g["dtype"][0])[0]
    q = np.full((B, QN, QS, D), one, np.uint16)
    k = np.full((B, KVN, KVS, D), one, np.uint16)
    v = np.full((B, KVN, KVS, D), one, np.uint16)
    mask = np.zeros([int(x) for x in g["mask_shape"]], np.uint8)
    strides = (KVS, 0, 0, 1)  # (B, 1, 1, S) broadcast over heads and the query row
    lens = np.array([int(g["actual_seq_lengths"][0])], np.int64)
    p = oracle.Problem(B, QN, KVN, QS, KVS, D, g["layout"][0], g["dtype"][0],
                       float(g["scale"][0]), lens, "bool", mask, strides)
    out, lse = oracle.attention(p, q, k, v)
    assert np.all(out == float(g["expect_out"][0]))
    assert np.allclose(lse, float(g["expect_lse"][0]), rtol=0, atol=1e-13)
    # Split into chunks of 5 (uneven, last chunk shorter) and merged: same result.
    o, m, l = oracle.split_partials(p, q, k, v, splits=4, chunk=5)
    out2, lse2 = oracle.merge(o, m, l)
    assert np.allclose(out2, 1.0, atol=1e-14)
    assert np.allclose(lse2, float(g["expect_lse"][0]), atol=1e-13)


# ---------------------------------------------------------------- brute force

BRUTE_CASES = [
    dict(layout="BNSD", B=1, QN=1, KVN=1, QS=1, KVS=1, D=8),
    dict(layout="BNSD", B=2, QN=2, KVN=1, QS=3, KVS=17, D=8),
    dict(layout="BSND", B=2, QN=4, KVN=2, QS=17, KVS=33, D=16, mask="causal"),
    dict(layout="BNSD", B=1, QN=8, KVN=2, QS=33, KVS=33, D=16, mask="bool_causal"),
    dict(layout="BSND", B=2, QN=4, KVN=4, QS=2, KVS=64, D=64, lens=(0, 64), seed=11),
    dict(layout="BNSD", B=2, QN=8, KVN=2, QS=64, KVS=17, D=16, mask="causal", lens=(0, 17),
         dtype="f16", std=0.5, seed=12),
    dict(layout="BSND", B=2, QN=2, KVN=2, QS=3, KVS=2, D=8, dtype="f16", seed=13),
]


@pytest.mark.parametrize("case", BRUTE_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_brute_matches_oracle(case):
    inp = tiny(**case)
    p = prob_of(inp)
    o1, l1 = oracle.attention(p, inp.q, inp.k, inp.v)
    o2, l2 = brute.attention(p, inp.q, inp.k, inp.v)
    assert np.array_equal(np.isinf(l1), np.isinf(l2))
    fin = np.isfinite(l1)
    assert np.allclose(l1[fin], l2[fin], rtol=1e-12, atol=1e-12)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)


def test_brute_random_bool_mask_with_empty_rows():
    inp = tiny(layout="BNSD", B=2, QN=4, KVN=2, QS=9, KVS=13, D=8, seed=5)
    rng = np.random.default_rng(9)
    mask = (rng.random((2, 4, 9, 13)) < 0.6).astype(np.uint8)
    mask[0, 1, 3, :] = 1  # a fully masked row
    p = oracle.Problem(2, 4, 2, 9, 13, 8, "BNSD", "bf16", 0.3, None, "bool", mask,
                       (4 * 9 * 13, 9 * 13, 13, 1))
    o1, l1 = oracle.attention(p, inp.q, inp.k, inp.v)
    o2, l2 = brute.attention(p, inp.q, inp.k, inp.v)
    assert l1[0, 1, 3] == np.inf and np.all(o1[0, 1, 3] == 0.0)
    assert np.array_equal(np.isinf(l1), np.isinf(l2))
    fin = np.isfinite(l1)
    assert np.allclose(l1[fin], l2[fin], rtol=1e-12, atol=1e-12)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- library routine

def _sdpa(Q, K, V, scale, g, attn_mask=None, is_causal=False):
    torch = pytest.importorskip("torch")
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (Q, K, V))
    if g > 1:
        tk = tk.repeat_interleave(g, dim=1)
        tv = tv.repeat_interleave(g, dim=1)
    am = None if attn_mask is None else torch.from_numpy(attn_mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am,
                                                         is_causal=is_causal, scale=scale)
    return o.numpy()


@pytest.mark.parametrize("layout", ["BNSD", "BSND"])
@pytest.mark.parametrize("kind", ["none", "causal", "bool", "lens"])
def test_sdpa_pin(layout, kind):
    QS, KVS = (24, 24) if kind == "causal" else (7, 40)
    inp = tiny(layout=layout, B=2, QN=6, KVN=2, QS=QS, KVS=KVS, D=16, scale=0.21,
               mask="causal" if kind == "causal" else "none",
               lens=(5, 40) if kind == "lens" else None, seed=21)
    s = inp.spec
    Q, K, V = (dec(x, s.dtype) for x in (inp.q, inp.k, inp.v))
    if layout == "BSND":
        Q, K, V = (x.transpose(0, 2, 1, 3) for x in (Q, K, V))
    if kind == "bool":
        rng = np.random.default_rng(4)
        mask = (rng.random((s.B, s.QN, QS, KVS)) < 0.5).astype(np.uint8)
        mask[..., 0] = 0  # keep every row non-empty (SDPA gives NaN on empty rows)
        p = oracle.Problem(s.B, s.QN, s.KVN, QS, KVS, s.D, layout, s.dtype, 0.21, None, "bool",
                           mask, (s.QN * QS * KVS, QS * KVS, KVS, 1))
        ref = _sdpa(Q, K, V, 0.21, s.g, attn_mask=(mask == 0))
    elif kind == "lens":
        p = prob_of(inp)
        ref = np.empty_like(Q)
        for b in range(s.B):
            L = int(inp.lens[b])
            ref[b:b + 1] = _sdpa(Q[b:b + 1], K[b:b + 1, :, :L], V[b:b + 1, :, :L], 0.21, s.g)
    else:
        p = prob_of(inp)
        ref = _sdpa(Q, K, V, 0.21, s.g, is_causal=(kind == "causal"))
    out, lse = oracle.attention(p, inp.q, inp.k, inp.v)
    if layout == "BSND":
        out = out.transpose(0, 2, 1, 3)
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------- closed forms

def test_single_valid_key_and_causal_first_row():
    inp = tiny(layout="BNSD", B=1, QN=2, KVN=1, QS=4, KVS=6, D=8, mask="causal", seed=31)
    p = prob_of(inp)
    out, lse = oracle.attention(p, inp.q, inp.k, inp.v)
    Q, K, V = (dec(x, "bf16") for x in (inp.q, inp.k, inp.v))
    for n1 in range(2):
        s0 = p.scale * float(Q[0, n1, 0] @ K[0, 0, 0])
        assert np.array_equal(out[0, n1, 0], V[0, 0, 0])      # row 0 sees key 0 only
        assert lse[0, n1, 0] == pytest.approx(s0, abs=1e-14)
    # length 1: every row sees only key 0
    p1 = oracle.Problem(1, 2, 1, 4, 6, 8, "BNSD", "bf16", p.scale, np.array([1]), "none")
    out1, _ = oracle.attention(p1, inp.q, inp.k, inp.v)
    assert np.all(out1 == V[0, 0, 0])


def test_zero_query_gives_mean_and_log_length():
    inp = tiny(layout="BSND", B=2, QN=2, KVN=2, QS=3, KVS=9, D=8, lens=(1, 9), seed=32)
    q0 = np.zeros_like(inp.q)
    p = prob_of(inp)
    out, lse = oracle.attention(p, q0, inp.k, inp.v)
    V = dec(inp.v, "bf16")
    for b in range(2):
        L = int(inp.lens[b])
        for n in range(2):
            mean = V[b, :L, n].mean(axis=0)
            assert np.allclose(out[b, :, n], mean, atol=1e-14)
            assert np.allclose(lse[b, n], math.log(L), atol=1e-14)


def test_two_keys_sigmoid_weights():
    inp = tiny(layout="BNSD", B=1, QN=1, KVN=1, QS=2, KVS=2, D=8, scale=0.7, seed=33)
    p = prob_of(inp)
    out, lse = oracle.attention(p, inp.q, inp.k, inp.v)
    Q, K, V = (dec(x, "bf16") for x in (inp.q, inp.k, inp.v))
    for i in range(2):
        s0, s1 = (0.7 * float(Q[0, 0, i] @ K[0, 0, j]) for j in (0, 1))
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        assert np.allclose(out[0, 0, i], w0 * V[0, 0, 0] + (1 - w0) * V[0, 0, 1], atol=1e-14)
        assert lse[0, 0, i] == pytest.approx(max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))),
                                             abs=1e-13)


# ---------------------------------------------------------------- invariants

def test_rows_sum_to_one_through_lse():
    inp = tiny(layout="BSND", B=2, QN=4, KVN=2, QS=6, KVS=21, D=16, mask="causal",
               lens=(3, 21), seed=41)
    p = prob_of(inp)
    _, lse = oracle.attention(p, inp.q, inp.k, inp.v)
    Q, K = dec(inp.q, "bf16"), dec(inp.k, "bf16")
    for b in range(2):
        L = int(inp.lens[b])
        for n1 in range(4):
            for i in range(6):
                js = [j for j in range(L) if j <= i]
                s = [p.scale * float(Q[b, i, n1] @ K[b, j, n1 // 2]) for j in js]
                assert sum(math.exp(x - lse[b, n1, i]) for x in s) == pytest.approx(1.0, abs=1e-13)


def test_constant_value_rows_come_back():
    inp = tiny(layout="BNSD", B=2, QN=4, KVN=4, QS=5, KVS=19, D=8, lens=(2, 19), seed=42)
    c = fa_synth.round_bits(np.array([0.8125], np.float32), "bf16")[0]
    v = np.full_like(inp.v, c)
    out, _ = oracle.attention(prob_of(inp), inp.q, inp.k, v)
    assert np.allclose(out, 0.8125, atol=1e-14)


@pytest.mark.parametrize("splits,chunk", [(1, 40), (3, 7), (40, 1), (5, 16), (8, 3)])
def test_split_then_merge_equals_unsplit(splits, chunk):
    inp = tiny(layout="BSND", B=2, QN=4, KVN=2, QS=3, KVS=21, D=16, mask="causal",
               lens=(0, 21), seed=43)
    p = prob_of(inp)
    if splits * chunk < p.KVS:
        pytest.skip("chunks must cover the cache")
    out, lse = oracle.attention_rows(p, inp.q, inp.k, inp.v)
    o, m, l = oracle.split_partials(p, inp.q, inp.k, inp.v, splits, chunk)
    out2, lse2 = oracle.merge(o, m, l)
    assert np.array_equal(np.isinf(lse), np.isinf(lse2))
    fin = np.isfinite(lse)
    assert np.allclose(lse[fin], lse2[fin], atol=1e-12)
    assert np.allclose(out, out2, atol=1e-12)


def test_partials_of_single_token_chunks():
    inp = tiny(layout="BNSD", B=1, QN=2, KVN=1, QS=1, KVS=6, D=8, lens=(4, 4), seed=44)
    p = prob_of(inp)
    o, m, l = oracle.split_partials(p, inp.q, inp.k, inp.v, splits=6, chunk=1)
    Q, K, V = (dec(x, "bf16") for x in (inp.q, inp.k, inp.v))
    for n1 in range(2):
        r = n1
        for c in range(6):
            if c < 4:
                assert m[r, c] == pytest.approx(p.scale * float(Q[0, n1, 0] @ K[0, 0, c]), abs=1e-14)
                assert l[r, c] == 1.0
                assert np.array_equal(o[r, c], V[0, 0, c])
            else:  # beyond the length: empty chunk
                assert m[r, c] == -np.inf and l[r, c] == 0.0 and np.all(o[r, c] == 0.0)


def test_merge_agrees_with_lse_weight_form_and_is_order_free():
    """Page 2 (IFA guide 8.3) weights normalised split results by exp(lse_i)/sum exp(lse_j):
    that form must give the oracle's merge.  The merge is also a reduction that does not
    depend on how the splits are grouped (FlashAttn developer guide 10, FD block; the
    tutorial, section 2): any order of the splits, and merging each half first and then
    the two halves' results (each as a one-key partial m = lse, l = 1, O = out), give
    the same output."""
    inp = tiny(layout="BNSD", B=2, QN=4, KVN=2, QS=1, KVS=50, D=16, lens=(10, 50), seed=45)
    p = prob_of(inp)
    o, m, l = oracle.split_partials(p, inp.q, inp.k, inp.v, splits=7, chunk=8)
    out, lse = oracle.merge(o, m, l)
    for r in range(o.shape[0]):
        live = np.isfinite(m[r])
        lse_i = m[r, live] + np.log(l[r, live])
        res_i = o[r, live] / l[r, live][:, None]
        scale_i = np.exp(lse_i) / np.exp(lse_i).sum()
        assert np.allclose((res_i * scale_i[:, None]).sum(axis=0), out[r], atol=1e-12)
    rng = np.random.default_rng(7)
    perm = rng.permutation(7)
    out_p, lse_p = oracle.merge(o[:, perm], m[:, perm], l[:, perm])
    assert np.allclose(out_p, out, atol=1e-12) and np.allclose(lse_p, lse, atol=1e-12)

    def as_partial(o_h, lse_h):  # a merged result as one partial: empty rows stay empty
        empty = np.isinf(lse_h)
        return (np.where(empty[:, None], 0.0, o_h), np.where(empty, -np.inf, lse_h),
                np.where(empty, 0.0, 1.0))
    for cut in (1, 3, 6):
        oa, la = oracle.merge(o[:, :cut], m[:, :cut], l[:, :cut])
        ob, lb = oracle.merge(o[:, cut:], m[:, cut:], l[:, cut:])
        pa, pb = as_partial(oa, la), as_partial(ob, lb)
        o2 = np.stack([pa[0], pb[0]], axis=1)
        m2 = np.stack([pa[1], pb[1]], axis=1)
        l2 = np.stack([pa[2], pb[2]], axis=1)
        out2, lse2 = oracle.merge(o2, m2, l2)
        assert np.allclose(out2, out, atol=1e-12) and np.allclose(lse2, lse, atol=1e-12)


def test_gqa_equals_repeated_kv_mha():
    inp = tiny(layout="BSND", B=2, QN=8, KVN=2, QS=4, KVS=11, D=8, mask="causal", lens=(1, 11),
               seed=46)
    p = prob_of(inp)
    out, lse = oracle.attention(p, inp.q, inp.k, inp.v)
    k_rep = np.repeat(inp.k, 4, axis=2)  # BSND head axis; head n2 repeated for n1 = 4*n2..4*n2+3
    v_rep = np.repeat(inp.v, 4, axis=2)
    p2 = oracle.Problem(2, 8, 8, 4, 11, 8, "BSND", "bf16", p.scale, inp.lens, "causal")
    out2, lse2 = oracle.attention(p2, inp.q, k_rep, v_rep)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_padding_contents_do_not_matter():
    inp = tiny(layout="BNSD", B=3, QN=4, KVN=2, QS=3, KVS=20, D=8, mask="causal", lens=(0, 20),
               seed=47)
    p = prob_of(inp)
    out, lse = oracle.attention(p, inp.q, inp.k, inp.v)
    for bits in (fa_synth.NAN_BITS["bf16"], 0x7F80, 0x461C):  # NaN, +inf, 1e4
        pad = fa_synth.fill_padding(inp, bits)
        o2, l2 = oracle.attention(p, pad.q, pad.k, pad.v)
        assert np.array_equal(out, o2) and np.array_equal(lse, l2)


def test_bsnd_is_transposed_bnsd():
    inp = tiny(layout="BNSD", B=2, QN=4, KVN=2, QS=6, KVS=13, D=8, mask="causal", seed=48)
    p = prob_of(inp)
    out, lse = oracle.attention(p, inp.q, inp.k, inp.v)
    t = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3))
    p2 = oracle.Problem(2, 4, 2, 6, 13, 8, "BSND", "bf16", p.scale, None, "causal")
    out2, lse2 = oracle.attention(p2, t(inp.q), t(inp.k), t(inp.v))
    assert np.array_equal(t(out), out2) and np.array_equal(lse, lse2)


def test_key_permutation_invariance():
    inp = tiny(layout="BNSD", B=1, QN=2, KVN=2, QS=3, KVS=15, D=8, seed=49)
    p = prob_of(inp)
    out, lse = oracle.attention(p, inp.q, inp.k, inp.v)
    perm = np.random.default_rng(1).permutation(15)
    out2, lse2 = oracle.attention(p, inp.q, inp.k[:, :, perm], inp.v[:, :, perm])
    assert np.allclose(out, out2, atol=1e-14) and np.allclose(lse, lse2, atol=1e-14)


def test_fp16_decoding_covers_subnormals_and_limits():
    bits = np.array([0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0xFBFF, 0x8001], np.uint16)
    want = [2.0 ** -24, 1023 * 2.0 ** -24, 2.0 ** -14, 1.0, 65504.0, -65504.0, -(2.0 ** -24)]
    # through the oracle: one key, D=1, the output is that value row exactly
    for b, w in zip(bits, want):
        p = oracle.Problem(1, 1, 1, 1, 1, 1, "BNSD", "f16", 1.0)
        one = np.array([[[[0x3C00]]]], np.uint16)
        out, _ = oracle.attention(p, one, one, np.array([[[[b]]]], np.uint16))
        assert out[0, 0, 0, 0] == w


def test_generator_is_deterministic_and_rounds_to_nearest_even():
    a = fa_synth.make(fa_synth.WORKLOADS["prefill_small"])
    b = fa_synth.make(fa_synth.WORKLOADS["prefill_small"])
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    got = fa_synth.f32_to_bf16_bits(x)
    # ties go to even: 1+2^-8 -> 1.0 (0x3F80); 1+3*2^-8 -> 1+2^-6 (0x3F82); above tie rounds up
    assert list(got) == [0x3F80, 0x3F82, 0x3F81]


# ---------------------------------------------------------------- paged KV cache

@pytest.mark.parametrize("kv_layout", ["PA_BBND", "PA_BNBD"])
@pytest.mark.parametrize("layout", ["BNSD", "BSND"])
def test_paged_cache_equals_contiguous(kv_layout, layout):
    """A paged cache (FlashAttn guide 1.2) holds the same logical K/V: the oracle must give
    the contiguous result, and never touch the NaN-filled spare blocks or padding."""
    inp = tiny(layout=layout, B=3, QN=8, KVN=2, QS=1, KVS=70, D=16, lens=(0, 70), seed=61)
    p = prob_of(inp)
    out, lse = oracle.attention(p, inp.q, inp.k, inp.v)
    kp, vp, table, _ = fa_synth.to_paged(inp, 16, kv_layout, seed=3)
    pp = oracle.Problem(3, 8, 2, 1, 70, 16, layout, "bf16", p.scale, inp.lens, "none",
                        kv_layout=kv_layout, block_table=table, block_size=16)
    out2, lse2 = oracle.attention(pp, inp.q, kp, vp)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    o, m, l = oracle.split_partials(pp, inp.q, kp, vp, splits=3, chunk=32)
    o0, m0, l0 = oracle.split_partials(p, inp.q, inp.k, inp.v, splits=3, chunk=32)
    assert np.array_equal(o, o0) and np.array_equal(m, m0) and np.array_equal(l, l0)


def test_paged_block_gather_by_hand():
    """Closed check of the indirection: with one-row-per-block paging (block_size 1 is not a
    legal GPU block size, but the oracle's indexing is general) the value rows seen by a
    query with Q=0 are exactly the rows the table points to, so out = their mean."""
    inp = tiny(layout="BNSD", B=1, QN=1, KVN=1, QS=1, KVS=4, D=8, seed=62)
    table = np.array([[2, 0, 3, 1]], np.int32)
    vp = np.zeros((4, 1, 1, 8), np.uint16)      # PA_BBND with block_size 1
    kp = np.zeros((4, 1, 1, 8), np.uint16)
    for j in range(4):
        vp[table[0, j], 0, 0] = inp.v[0, 0, j]
        kp[table[0, j], 0, 0] = inp.k[0, 0, j]
    pp = oracle.Problem(1, 1, 1, 1, 4, 8, "BNSD", "bf16", 0.5, None, "none",
                        kv_layout="PA_BBND", block_table=table, block_size=1)
    out, _ = oracle.attention(pp, np.zeros_like(inp.q), kp, vp)
    assert np.allclose(out[0, 0, 0], dec(inp.v, "bf16")[0, 0].mean(axis=0), atol=1e-14)


# ---------------------------------------------------------------- window mask

def _band(QS, KVS, wl, wr):
    """Keep-matrix of the window band built from numpy's triangle routines."""
    keep = np.ones((QS, KVS), dtype=bool)
    if wr >= 0:
        keep &= np.tril(np.ones((QS, KVS), dtype=bool), k=wr)
    if wl >= 0:
        keep &= np.triu(np.ones((QS, KVS), dtype=bool), k=-wl)
    return keep


@pytest.mark.parametrize("wl,wr", [(3, 0), (0, 2), (5, 7), (-1, 4), (6, -1), (0, 0), (40, 40)])
@pytest.mark.parametrize("layout", ["BNSD", "BSND"])
def test_window_equals_band_bool_mask(wl, wr, layout):
    """Window mode (FlashAttn guide 1.5, mode 4) against the same band given as a boolean
    tensor, through the whole-matrix brute force (a separate route)."""
    inp = tiny(layout=layout, B=2, QN=4, KVN=2, QS=21, KVS=26, D=16, lens=(9, 26), seed=81)
    s = inp.spec
    pw = oracle.Problem(s.B, s.QN, s.KVN, s.QS, s.KVS, s.D, layout, "bf16", s.softmax_scale,
                        inp.lens, "window", window=(wl, wr))
    mask = (~_band(s.QS, s.KVS, wl, wr)).astype(np.uint8)
    pb = oracle.Problem(s.B, s.QN, s.KVN, s.QS, s.KVS, s.D, layout, "bf16", s.softmax_scale,
                        inp.lens, "bool", mask, (0, 0, s.KVS, 1))
    o1, l1 = oracle.attention(pw, inp.q, inp.k, inp.v)
    o2, l2 = brute.attention(pb, inp.q, inp.k, inp.v)
    assert np.array_equal(np.isinf(l1), np.isinf(l2))
    fin = np.isfinite(l1)
    assert np.allclose(l1[fin], l2[fin], rtol=1e-12, atol=1e-12)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)


def test_window_special_cases():
    """(-1, 0) is the causal mask, (-1, -1) no mask, (0, 0) the diagonal alone:
    out_i = v_i and lse_i = scale * q_i . k_i in closed form."""
    inp = tiny(layout="BNSD", B=1, QN=2, KVN=1, QS=12, KVS=12, D=16, seed=82)
    s = inp.spec
    mk = lambda mode, w=(-1, -1): oracle.Problem(1, 2, 1, 12, 12, 16, "BNSD", "bf16",
                                                 s.softmax_scale, None, mode, window=w)
    oc, lc = oracle.attention(mk("causal"), inp.q, inp.k, inp.v)
    ow, lw = oracle.attention(mk("window", (-1, 0)), inp.q, inp.k, inp.v)
    assert np.array_equal(oc, ow) and np.array_equal(lc, lw)
    on, ln_ = oracle.attention(mk("none"), inp.q, inp.k, inp.v)
    ow, lw = oracle.attention(mk("window", (-1, -1)), inp.q, inp.k, inp.v)
    assert np.array_equal(on, ow) and np.array_equal(ln_, lw)
    od, ld = oracle.attention(mk("window", (0, 0)), inp.q, inp.k, inp.v)
    Q, K, V = (dec(x, "bf16") for x in (inp.q, inp.k, inp.v))
    for n1 in range(2):
        assert np.array_equal(od[0, n1], V[0, 0])
        assert np.allclose(ld[0, n1], s.softmax_scale * np.einsum("id,id->i", Q[0, n1], K[0, 0]),
                           atol=1e-13)


def test_window_sdpa_pin():
    """Window band as an attention mask of torch's float64 SDPA (a library routine)."""
    inp = tiny(layout="BNSD", B=1, QN=3, KVN=3, QS=30, KVS=30, D=16, scale=0.3, seed=83)
    s = inp.spec
    keep = _band(30, 30, 4, 2)
    Q, K, V = (dec(x, "bf16") for x in (inp.q, inp.k, inp.v))
    ref = _sdpa(Q, K, V, 0.3, 1, attn_mask=keep)
    p = oracle.Problem(1, 3, 3, 30, 30, 16, "BNSD", "bf16", 0.3, None, "window", window=(4, 2))
    out, _ = oracle.attention(p, inp.q, inp.k, inp.v)
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------- packed variable length (TND)

def _tnd_prob(x, mode="none", lens=None, seqused_q=None, window=(-1, -1)):
    B = len(x.cu_q) - 1
    return oracle.Problem(B, x.QN, x.KVN, int(x.cu_q[-1]), int(x.cu_kv[-1]), x.D, "TND", x.dtype,
                          x.scale, lens, mode, window=window, cu_seqlens_q=x.cu_q,
                          cu_seqlens_kv=x.cu_kv, seqused_q=seqused_q)


@pytest.mark.parametrize("mode", ["none", "causal"])
def test_tnd_equals_brute_force_per_sequence(mode):
    """The packed layout (FlashAttn guide 1.3) is the padded one without padding: every
    sequence of a TND batch must give the whole-matrix brute force of that sequence alone."""
    x = fa_synth.make_packed(4, 4, 2, 16, q_lens=(1, 23), kv_lens=(1, 31), seed=101)
    out, lse = oracle.attention(_tnd_prob(x, mode), x.q, x.k, x.v)
    for b in range(4):
        q0, q1, k0, k1 = x.cu_q[b], x.cu_q[b + 1], x.cu_kv[b], x.cu_kv[b + 1]
        pb = oracle.Problem(1, 4, 2, int(q1 - q0), int(k1 - k0), 16, "BSND", "bf16", x.scale,
                            None, mode)
        ro, rl = brute.attention(pb, x.q[None, q0:q1], x.k[None, k0:k1], x.v[None, k0:k1])
        assert np.allclose(out[q0:q1], ro[0], rtol=1e-12, atol=1e-12)
        fin = np.isfinite(rl[0].T)
        assert np.array_equal(np.isinf(lse[q0:q1]), np.isinf(rl[0].T))
        assert np.allclose(lse[q0:q1][fin], rl[0].T[fin], rtol=1e-12, atol=1e-12)


def test_tnd_truncation_and_unused_rows():
    """seqused_q leaves the rows past it at the initial output (0, lse +inf); the KV
    lengths truncate each sequence's keys (the shorter of the two takes effect)."""
    x = fa_synth.make_packed(3, 2, 1, 16, q_lens=(5, 12), seed=102)
    used = np.array([3, 0, 100], np.int32)
    kv_lens = np.array([2, 5, 1000], np.int64)
    out, lse = oracle.attention(_tnd_prob(x, "none", kv_lens, used), x.q, x.k, x.v)
    for b in range(3):
        q0, q1, k0 = x.cu_q[b], x.cu_q[b + 1], x.cu_kv[b]
        nq = min(int(used[b]), int(q1 - q0))
        L = min(int(kv_lens[b]), int(x.cu_kv[b + 1] - k0))
        assert np.all(out[q0 + nq:q1] == 0) and np.all(np.isposinf(lse[q0 + nq:q1]))
        if nq:
            pb = oracle.Problem(1, 2, 1, nq, L, 16, "BSND", "bf16", x.scale, None, "none")
            ro, rl = brute.attention(pb, x.q[None, q0:q0 + nq], x.k[None, k0:k0 + L],
                                     x.v[None, k0:k0 + L])
            assert np.allclose(out[q0:q0 + nq], ro[0], rtol=1e-12, atol=1e-12)
            assert np.allclose(lse[q0:q0 + nq], rl[0].T, rtol=1e-12, atol=1e-12)


def test_tnd_rejects_malformed_offsets():
    x = fa_synth.make_packed(2, 2, 2, 16, q_lens=(3, 5), seed=103)
    bad = x.cu_q.copy(); bad[1] = bad[2] + 1
    p = oracle.Problem(2, 2, 2, int(x.cu_q[-1]), int(x.cu_kv[-1]), 16, "TND", "bf16", 1.0, None,
                       "none", cu_seqlens_q=bad, cu_seqlens_kv=x.cu_kv)
    with pytest.raises(ValueError):
        oracle.attention(p, x.q, x.k, x.v)


@pytest.mark.parametrize("layout", ["BNSD", "BSND"])
def test_seqused_q_on_padded_layouts(layout):
    """seqused_q (developer guide 1.4, any layout) truncates each batch's query rows:
    rows below it equal the untruncated result (pinned against the whole-matrix brute
    force), rows at or past it are 0 with lse = +inf; values above Q_S change nothing."""
    spec = fa_synth.Spec("su", layout, 3, 4, 2, 9, 13, 16, "bf16", lens=(2, 13), seed=131)
    inp = fa_synth.make(spec)
    used = np.array([4, 0, 100], np.int32)
    full = oracle.Problem.from_inputs(inp)
    trunc = oracle.Problem(3, 4, 2, 9, 13, 16, layout, "bf16", spec.softmax_scale, inp.lens, "none",
                           seqused_q=used)
    out, lse = oracle.attention(trunc, inp.q, inp.k, inp.v)
    ref, ref_lse = brute.attention(full, inp.q, inp.k, inp.v)
    for b in range(3):
        nq = min(int(used[b]), 9)
        o_b = out[b] if layout == "BNSD" else out[b].transpose(1, 0, 2)   # [QN, QS, D]
        r_b = ref[b] if layout == "BNSD" else ref[b].transpose(1, 0, 2)
        assert np.allclose(o_b[:, :nq], r_b[:, :nq], rtol=1e-12, atol=1e-12)
        assert np.allclose(lse[b][:, :nq], ref_lse[b][:, :nq], rtol=1e-12, atol=1e-12)
        assert np.all(o_b[:, nq:] == 0) and np.all(np.isposinf(lse[b][:, nq:]))
