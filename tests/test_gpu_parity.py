"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bar (from the benchmark spec): on 16-bit outputs max |err| <= 2e-2 and mean |err| <=
2e-3 against the oracle; |lse - lse_oracle| <= 1e-3; rows with no valid key are
exactly 0 with lse = +inf; no NaN anywhere.  Stage-1 partials of the split-KV
decode: m within 1e-3 absolute, l and O within 2e-3 of the oracle's partials
relative to the partial's own scale.
"""
import dataclasses
import functools
import math

import numpy as np
import pytest

import fa_synth
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

import split_kv_decode_amd as fa  # noqa: E402

DEV = torch.device("cuda:0")
OUT_MAX, OUT_MEAN, LSE_TOL = 2e-2, 2e-3, 1e-3


def dev16(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def check(out, lse, ref, ref_lse, what=""):
    """out/ref: same shape; lse/ref_lse: same shape (or lse None)."""
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out - ref)
    assert err.max() <= OUT_MAX, f"{what}: max abs err {err.max():.3e}"
    assert err.mean() <= OUT_MEAN, f"{what}: mean abs err {err.mean():.3e}"
    if lse is not None:
        inv = np.isinf(ref_lse)
        assert np.array_equal(np.isinf(lse), inv) and np.all(lse[inv] > 0), f"{what}: invalid-row lse"
        if (~inv).any():
            le = np.abs(lse[~inv] - ref_lse[~inv]).max()
            assert le <= LSE_TOL, f"{what}: lse err {le:.3e}"
        # invalid rows exactly zero
        inv_rows = inv.reshape(-1)
        if inv_rows.any():
            flat = out.reshape(-1, out.shape[-1]) if out.ndim == 2 else None
            if flat is not None:
                assert np.all(flat[inv_rows] == 0.0)
    return float(err.max())


def run_fwd(inp, mask_mode=None, return_lse=True):
    s = inp.spec
    q, k, v = (dev16(x, s.dtype) for x in (inp.q, inp.k, inp.v))
    lens = None if inp.lens is None else torch.from_numpy(inp.lens).to(DEV)
    mode = mask_mode or {"none": "none", "causal": "causal", "bool_causal": "bool"}[s.mask]
    mask = None
    if mode == "bool":
        mask = torch.from_numpy(inp.mask).to(DEV)
    out, lse = fa.fwd(q, k, v, layout=s.layout, scale=s.softmax_scale, actual_seq_lengths=lens,
                      mask=mask, mask_stride=inp.mask_strides, causal=(mode == "causal"),
                      return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def rows_of(out_t, s, rows):
    """GPU output rows (flat ids (b*QN+n1)*QS+i) as [nrows, D] fp64."""
    o = out_t
    if s.layout == "BSND":
        o = o.permute(0, 2, 1, 3)
    o = o.reshape(-1, s.D)
    idx = torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(DEV)
    return to_np(o.index_select(0, idx))


def full_check(inp, mask_mode=None, what=""):
    out, lse = run_fwd(inp, mask_mode)
    prob = oracle.Problem.from_inputs(inp, {"bool": "bool", "causal": "causal", None: None,
                                            "none": "none"}[mask_mode])
    ref, ref_lse = oracle.attention(prob, inp.q, inp.k, inp.v)
    s = inp.spec
    o_rows = rows_of(out, s, np.arange(s.B * s.QN * s.QS))
    r_rows = ref if s.layout == "BNSD" else ref.transpose(0, 2, 1, 3)
    r_rows = np.ascontiguousarray(r_rows).reshape(-1, s.D)
    return check(o_rows, to_np(lse).reshape(-1), r_rows, ref_lse.reshape(-1), what)


@functools.lru_cache(maxsize=2)
def workload(name):
    return fa_synth.make(fa_synth.WORKLOADS[name])


def spec(layout="BNSD", B=1, QN=2, KVN=2, QS=1, KVS=64, D=128, dtype="bf16", std=1.0, mask="none",
         lens=None, seed=1, scale=None):
    return fa_synth.Spec("t", layout, B, QN, KVN, QS, KVS, D, dtype, std=std, mask=mask, lens=lens,
                         seed=seed, scale=scale)


# ------------------------------------------------------------------ decode (q_seq == 1)

DECODE_CASES = [
    dict(B=1, QN=1, KVN=1, KVS=1, D=128),
    dict(B=1, QN=32, KVN=32, KVS=4096, D=128),
    dict(B=2, QN=8, KVN=2, KVS=1000, D=128, layout="BSND", lens=(0, 1000)),
    dict(B=3, QN=16, KVN=2, KVS=777, D=64, lens=(1, 777)),
    dict(B=2, QN=6, KVN=2, KVS=333, D=128, dtype="f16", layout="BSND"),    # g = 3
    dict(B=1, QN=4, KVN=4, KVS=70000, D=64, dtype="f16", std=0.5),
    dict(B=4, QN=64, KVN=4, KVS=2048, D=128, lens=(1, 2048)),             # g = 16
    dict(B=5, QN=2, KVN=1, KVS=300, D=128, lens=(0, 3)),
    dict(B=2, QN=4, KVN=2, KVS=500, D=128, scale=-0.09),
    dict(B=2, QN=8, KVN=2, KVS=3000, D=256, lens=(0, 3000)),               # D = 256
    dict(B=1, QN=16, KVN=16, KVS=20000, D=256, dtype="f16", layout="BSND"),
    dict(B=3, QN=8, KVN=1, KVS=333, D=256, lens=(1, 333)),                  # g = 8
    dict(B=1, QN=1, KVN=1, KVS=131072, D=128),   # 512 splits: stage 1 + combine kernels
    dict(B=2, QN=1, KVN=1, KVS=60000, D=64, lens=(0, 60000)),   # fused, one unit empty or not
    # grouped heads 4..32 on a contiguous cache run the matrix-core stage 1
    dict(B=1, QN=32, KVN=1, KVS=3000, D=128, lens=(1, 3000)),              # g = 32
    dict(B=3, QN=8, KVN=2, KVS=200, D=128, dtype="f16", lens=(0, 200)),    # g = 4, one split
    dict(B=2, QN=16, KVN=4, KVS=1500, D=64, scale=-0.07, layout="BSND"),   # g = 4, negative scale
    dict(B=6, QN=24, KVN=3, KVS=777, D=128, lens=(1, 40)),                  # g = 8, short lengths
    dict(B=70, QN=8, KVN=2, KVS=1300, D=64, lens=(0, 1300)),   # balanced plan over > 64 batches
    # chunks above 512 tokens (on 256 CUs) take the two-wave, 64-key-tile stage 1;
    # the cases above run one wave on 32-key tiles
    dict(B=1, QN=32, KVN=8, KVS=40000, D=128),                       # g = 4, fixed chunks
    dict(B=2, QN=16, KVN=4, KVS=40000, D=64, lens=(1, 40000)),       # g = 4, balanced pieces
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_decode_fwd_matches_oracle(case):
    inp = fa_synth.make(spec(**case))
    full_check(inp, what=str(case))


def test_decode_ignores_nan_padding():
    inp = fa_synth.make(spec(layout="BSND", B=4, QN=8, KVN=2, KVS=600, lens=(0, 600), seed=5))
    base, base_lse = run_fwd(inp)
    pad = fa_synth.fill_padding(inp, fa_synth.NAN_BITS["bf16"])
    out, lse = run_fwd(pad)
    assert torch.equal(out, base) and torch.equal(torch.isinf(lse), torch.isinf(base_lse))
    assert torch.equal(lse[~torch.isinf(lse)], base_lse[~torch.isinf(base_lse)])


FUSED_CASES = [
    (dict(B=1, QN=32, KVN=32, KVS=131072, D=128), 32, 4096),     # the 128K decode plan
    (dict(layout="BSND", B=8, QN=32, KVN=8, KVS=4096, D=128, lens=(1, 4096)), 16, 256),
    (dict(B=3, QN=16, KVN=2, KVS=777, D=64, lens=(0, 777)), 13, 64),          # empty units
    (dict(B=2, QN=8, KVN=2, KVS=3000, D=256, dtype="f16", lens=(1, 3000)), 5, 640),
    (dict(B=1, QN=2, KVN=1, KVS=300, D=128), 1, 320),                         # one split
    (dict(B=1, QN=4, KVN=4, KVS=32768, D=128), 256, 128),                     # the most splits
]


def _fused_setup(inp, splits, chunk):
    s = inp.spec
    q, k, v = (dev16(x, s.dtype) for x in (inp.q, inp.k, inp.v))
    lens = None if inp.lens is None else torch.from_numpy(inp.lens).to(DEV)
    p = fa.params_for(q, k, layout=s.layout, scale=s.softmax_scale, actual_seq_lengths=lens)
    _, _, nbytes = fa.fa_splitkv_plan(p, chunk_hint=chunk)
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device=DEV)  # zero once: the counter contract
    return q, k, v, lens, p, ws, nbytes


@pytest.mark.parametrize("case,splits,chunk", FUSED_CASES,
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()) if isinstance(c, dict) else str(c))
def test_decode_fused_matches_oracle(case, splits, chunk):
    """The single-launch split-KV: the workgroup that completes a unit merges it.
    Two calls in a row on one workspace agree bit for bit (the counters come back to 0)."""
    inp = fa_synth.make(spec(seed=43, **case))
    s = inp.spec
    q, k, v, lens, p, ws, nbytes = _fused_setup(inp, splits, chunk)
    outs = []
    for _ in range(2):
        out = torch.empty_like(q)
        lse = torch.empty((s.B, s.QN, 1), dtype=torch.float32, device=DEV)
        fa.fa_decode_fused(p, splits, chunk, q, k, v, ws, nbytes, out, lse, torch.cuda.current_stream())
        torch.cuda.synchronize()
        outs.append((out, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    if splits > 1:
        units = s.B * s.KVN * (s.g // max(h for h in (8, 4, 2, 1) if s.g % h == 0))
        n_counter_words = -(-(units * 4) // 256) * 64   # the trailing 256-byte-aligned region
        assert torch.count_nonzero(ws.view(torch.int32)[-n_counter_words:]) == 0
    out, lse = outs[0]
    prob = oracle.Problem.from_inputs(inp)
    ref, ref_lse = oracle.attention_rows(prob, inp.q, inp.k, inp.v)
    check(rows_of(out, s, np.arange(s.B * s.QN)), to_np(lse).reshape(-1), ref, ref_lse, f"fused {case}")


def test_decode_fused_graph_replays():
    """The fused decode captured in a HIP graph: every replay (with new q and eager work in
    between, the workspace never cleared again) must equal the eager two-kernel result."""
    inp = fa_synth.make(spec(layout="BSND", B=4, QN=16, KVN=4, KVS=3000, lens=(1, 3000), seed=41))
    s = inp.spec
    splits, chunk = 12, 256
    q, k, v, lens, p, ws, nbytes = _fused_setup(inp, splits, chunk)
    out = torch.empty_like(q)
    lse = torch.empty((s.B, s.QN, 1), dtype=torch.float32, device=DEV)
    qg = q.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up off the capture
        fa.fa_decode_fused(p, splits, chunk, qg, k, v, ws, nbytes, out, lse, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.fa_decode_fused(p, splits, chunk, qg, k, v, ws, nbytes, out, lse,
                           torch.cuda.current_stream())
    for rep in range(4):
        qn = torch.randn(q.shape, device=DEV).to(q.dtype)
        qg.copy_(qn)
        graph.replay()
        torch.cuda.synchronize()
        ref_out, ref_lse = fa.fwd(qn, k, v, layout=s.layout, scale=s.softmax_scale,
                                  actual_seq_lengths=lens, return_lse=True)
        torch.cuda.synchronize()
        err = (out.float() - ref_out.float()).abs().max().item()
        assert err <= OUT_MAX, f"replay {rep}: {err}"
        assert (lse - ref_lse).abs().max().item() <= 1e-5, f"replay {rep}"


def _partials(inp, splits, chunk):
    s = inp.spec
    p = fa.params_for(dev16(inp.q, s.dtype), dev16(inp.k, s.dtype), layout=s.layout,
                      scale=s.softmax_scale,
                      actual_seq_lengths=None)
    lens_t = None
    if inp.lens is not None:
        lens_t = torch.from_numpy(inp.lens).to(DEV)
        p.actual_seq_lengths = lens_t.data_ptr()
    q, k, v = (dev16(x, s.dtype) for x in (inp.q, inp.k, inp.v))
    rows = s.B * s.QN
    o = torch.full((rows * splits * s.D,), float("nan"), device=DEV)
    m = torch.full((rows * splits,), float("nan"), device=DEV)
    l = torch.full((rows * splits,), float("nan"), device=DEV)
    fa.fa_decode_splitkv(p, splits, chunk, q, k, v, o, m, l, torch.cuda.current_stream())
    out = torch.empty_like(q)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    fa.fa_combine(p, splits, o, m, l, out, lse, torch.cuda.current_stream())
    torch.cuda.synchronize()
    return (o.view(rows, splits, s.D), m.view(rows, splits), l.view(rows, splits), out, lse,
            lens_t)


@pytest.mark.parametrize("splits,chunk", [(1, 1024), (3, 384), (16, 64), (40, 64), (2, 4096)])
def test_stage1_partials_and_combine(splits, chunk):
    inp = fa_synth.make(spec(layout="BNSD", B=2, QN=8, KVN=2, KVS=1000, lens=(1, 1000), seed=9))
    if splits * chunk < 1000:
        pytest.skip("plan must cover the cache")
    o, m, l, out, lse, _ = _partials(inp, splits, chunk)
    prob = oracle.Problem.from_inputs(inp)
    ro, rm, rl = oracle.split_partials(prob, inp.q, inp.k, inp.v, splits, chunk)
    go, gm, gl = to_np(o), to_np(m), to_np(l)
    empty = np.isinf(rm)
    assert np.array_equal(np.isinf(gm) & (gm < 0), empty), "empty-split flags"
    assert np.all(gl[empty] == 0.0) and np.all(go[empty] == 0.0)
    live = ~empty
    assert np.abs(gm[live] - rm[live]).max() <= 1e-3
    assert np.all(np.abs(gl[live] - rl[live]) <= 2e-3 * rl[live])
    # The matrix-core stage 1 (grouped heads) rounds P to the 16-bit input type
    # before the PV product, as the pages' FlashAttention design casts P: each
    # term may move by 2^-8 of |p v| (bf16 unit roundoff 2^-9, doubled).  The
    # bound needs sum_j p_j |v_j|, the partial of the same scores with |V|.
    vabs = np.ascontiguousarray(inp.v) & np.uint16(0x7FFF)
    ro_abs, _, _ = oracle.split_partials(prob, inp.q, inp.k, vabs, splits, chunk)
    tol = 2e-3 * np.abs(ro).max(axis=2, keepdims=True) + 2.0 ** -8 * ro_abs + 1e-6
    assert np.all((np.abs(go - ro) <= tol)[live]), "stage-1 O partials"
    # combine of the GPU partials against the oracle's unsplit result
    ref, ref_lse = oracle.attention_rows(prob, inp.q, inp.k, inp.v)
    check(to_np(out).reshape(-1, 128), to_np(lse), ref, ref_lse, f"combine {splits}x{chunk}")


def test_combine_alone_matches_oracle_merge():
    """fa_combine on oracle partials (cast to fp32) against the oracle's own merge."""
    rng = np.random.default_rng(3)
    rows, splits, D = 12, 9, 128
    m = rng.normal(0, 3, (rows, splits))
    l = rng.uniform(0.5, 40, (rows, splits))
    o = rng.normal(0, 1, (rows, splits, D)) * l[..., None]
    m[0, :] = -np.inf; l[0, :] = 0; o[0] = 0          # all splits empty
    m[1, 3:] = -np.inf; l[1, 3:] = 0; o[1, 3:] = 0     # some empty
    ref, ref_lse = oracle.merge(o, m, l)
    p = fa.make_params(rows, 1, 1, 4096, D, layout="BNSD", dtype="bf16", scale=1.0)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    out = torch.empty((rows, 1, 1, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    fa.fa_combine(p, splits, t(o), t(m), t(l), out, lse, torch.cuda.current_stream())
    torch.cuda.synchronize()
    got = to_np(out).reshape(rows, D)
    assert np.all(got[0] == 0) and math.isinf(float(lse[0])) and float(lse[0]) > 0
    check(got, to_np(lse), ref, ref_lse, "combine")


# ------------------------------------------------------------------ paged KV cache (decode)

def _paged_params(inp, kv_layout, table, bs, nb, lens_t):
    s = inp.spec
    return fa.make_params(s.B, s.QN, 1, s.KVS, s.D, num_kv_heads=s.KVN, layout=s.layout,
                          dtype=s.dtype, scale=s.softmax_scale, actual_seq_lengths=lens_t,
                          kv_layout=kv_layout, block_table=table, block_size=bs,
                          max_blocks_per_seq=table.shape[1], num_blocks=nb)


def run_paged(inp, kv_layout, bs, seed=0, table_tail=None):
    """fa_fwd on the paged copy of inp's cache (spare blocks and padding hold NaN).

    table_tail: value written into the block-table entries past each batch's last
    used block (they must never be read)."""
    s = inp.spec
    kp, vp, table, nb = fa_synth.to_paged(inp, bs, kv_layout, seed=seed)
    if table_tail is not None:
        for b in range(s.B):
            table[b, -(-int(inp.lens[b]) // bs):] = table_tail
    q, k, v = dev16(inp.q, s.dtype), dev16(kp, s.dtype), dev16(vp, s.dtype)
    lens_t = torch.from_numpy(inp.lens).to(DEV)
    tab_t = torch.from_numpy(table).to(DEV)
    p = _paged_params(inp, kv_layout, tab_t, bs, nb, lens_t)
    out = torch.empty_like(q)
    lse = torch.empty((s.B, s.QN, 1), dtype=torch.float32, device=DEV)
    nbytes = fa.fa_workspace_size(p)
    ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=DEV)
    fa.fa_fwd(p, q, k, v, out, lse, ws, nbytes, torch.cuda.current_stream())
    torch.cuda.synchronize()
    return out, lse, table


PAGED_CASES = [
    dict(kv_layout="PA_BBND", bs=16, B=3, QN=8, KVN=2, KVS=1000, D=128, layout="BSND", lens=(0, 1000)),
    dict(kv_layout="PA_BNBD", bs=128, B=2, QN=32, KVN=8, KVS=4096, D=128, lens=(1, 4096)),
    dict(kv_layout="PA_BBND", bs=48, B=4, QN=16, KVN=2, KVS=700, D=64, dtype="f16", std=0.5,
         lens=(1, 700)),
    dict(kv_layout="PA_BNBD", bs=1024, B=1, QN=4, KVN=4, KVS=20000, D=128, lens=(19000, 20000)),
    dict(kv_layout="PA_BNBD", bs=16, B=2, QN=6, KVN=2, KVS=333, D=128, layout="BSND", lens=(1, 333)),
    dict(kv_layout="PA_BBND", bs=64, B=2, QN=8, KVN=2, KVS=1500, D=256, lens=(1, 1500)),
    # matrix-core stage 1 on paged caches: blocks smaller than a 64-key tile
    dict(kv_layout="PA_BNBD", bs=16, B=3, QN=32, KVN=4, KVS=900, D=64, lens=(0, 900)),
    dict(kv_layout="PA_BBND", bs=32, B=2, QN=64, KVN=4, KVS=2100, D=128, lens=(1, 2100)),
    dict(kv_layout="PA_BBND", bs=64, B=1, QN=32, KVN=8, KVS=40000, D=128, lens=(30000, 40000)),  # two waves
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_paged_decode_matches_oracle_and_contiguous(case):
    case = dict(case)
    kv_layout, bs = case.pop("kv_layout"), case.pop("bs")
    inp = fa_synth.make(spec(seed=71, **case))
    out, lse, table = run_paged(inp, kv_layout, bs, seed=5)
    s = inp.spec
    kp, vp, _, _ = fa_synth.to_paged(inp, bs, kv_layout, seed=5)
    prob = oracle.Problem(s.B, s.QN, s.KVN, 1, s.KVS, s.D, s.layout, s.dtype, s.softmax_scale,
                          inp.lens, "none", kv_layout=kv_layout, block_table=table, block_size=bs)
    ref, ref_lse = oracle.attention(prob, inp.q, kp, vp)
    r_rows = np.ascontiguousarray(ref if s.layout == "BNSD" else ref.transpose(0, 2, 1, 3))
    check(rows_of(out, s, np.arange(s.B * s.QN)), to_np(lse).reshape(-1),
          r_rows.reshape(-1, s.D), ref_lse.reshape(-1), f"paged {case}")
    # Same split plan and the same per-token arithmetic as the contiguous cache
    # (both take the vector or both the matrix-core stage 1).
    c_out, c_lse = run_fwd(inp)
    assert torch.equal(out, c_out)
    assert torch.equal(lse.reshape(-1), c_lse.reshape(-1))


def test_paged_decode_never_reads_unused_table_entries():
    inp = fa_synth.make(spec(layout="BNSD", B=4, QN=8, KVN=2, KVS=900, lens=(0, 900), seed=72))
    base, base_lse, _ = run_paged(inp, "PA_BBND", 32, seed=6)
    for tail in (-1, 1 << 30):
        out, lse, _ = run_paged(inp, "PA_BBND", 32, seed=6, table_tail=tail)
        assert torch.equal(out, base) and torch.equal(torch.isinf(lse), torch.isinf(base_lse))


@pytest.mark.parametrize("bs,chunk,splits,qn", [
    (48, 64, 19, 4), (16, 16256, 2, 4), (64, 320, 63, 4),
    # grouped heads (g = 4) on the matrix cores: the longest one-wave chunk over
    # 16-token blocks (32 block ids in the per-lane register table), a one-wave
    # chunk that cuts 48-token blocks, a two-wave chunk, and short chunks
    (16, 512, 2, 8), (48, 512, 2, 8), (16, 576, 2, 8), (48, 64, 19, 8)])
def test_paged_stage1_partials(bs, chunk, splits, qn):
    """Chunks that cut blocks (48 vs 64), a chunk whose 1016 block ids fill the LDS
    table, and a chunk that is a multiple of the block size."""
    KVS = 20000 if chunk == 16256 else 900
    inp = fa_synth.make(spec(layout="BSND", B=2, QN=qn, KVN=2, KVS=KVS,
                             lens=(KVS // 2, KVS), seed=73))
    if splits * chunk < KVS:
        splits = -(-KVS // chunk)
    s = inp.spec
    kp, vp, table, nb = fa_synth.to_paged(inp, bs, "PA_BNBD", seed=8)
    q, k, v = dev16(inp.q, s.dtype), dev16(kp, s.dtype), dev16(vp, s.dtype)
    lens_t = torch.from_numpy(inp.lens).to(DEV)
    tab_t = torch.from_numpy(table).to(DEV)
    p = _paged_params(inp, "PA_BNBD", tab_t, bs, nb, lens_t)
    rows = s.B * s.QN
    o = torch.full((rows * splits * s.D,), float("nan"), device=DEV)
    m = torch.full((rows * splits,), float("nan"), device=DEV)
    l = torch.full((rows * splits,), float("nan"), device=DEV)
    fa.fa_decode_splitkv(p, splits, chunk, q, k, v, o, m, l, torch.cuda.current_stream())
    torch.cuda.synchronize()
    prob = oracle.Problem(s.B, s.QN, s.KVN, 1, s.KVS, s.D, s.layout, s.dtype, s.softmax_scale,
                          inp.lens, "none", kv_layout="PA_BNBD", block_table=table, block_size=bs)
    ro, rm, rl = oracle.split_partials(prob, inp.q, kp, vp, splits, chunk)
    go, gm, gl = (to_np(x) for x in (o.view(rows, splits, s.D), m.view(rows, splits),
                                     l.view(rows, splits)))
    empty = np.isinf(rm)
    assert np.array_equal(np.isinf(gm) & (gm < 0), empty)
    assert np.all(gl[empty] == 0.0) and np.all(go[empty] == 0.0)
    live = ~empty
    assert np.abs(gm[live] - rm[live]).max() <= 1e-3
    assert np.all(np.abs(gl[live] - rl[live]) <= 2e-3 * rl[live])
    tol = 2e-3 * np.abs(ro).max(axis=2, keepdims=True) + 1e-6
    if qn // 2 >= 4:  # matrix-core stage 1: P rounded to 16 bits (bound as in the contiguous test)
        ro_abs, _, _ = oracle.split_partials(prob, inp.q, kp, np.ascontiguousarray(vp) & np.uint16(0x7FFF),
                                             splits, chunk)
        tol = tol + 2.0 ** -8 * ro_abs
    assert np.all((np.abs(go - ro) <= tol)[live])


# ------------------------------------------------------------------ prefill

PREFILL_CASES = [
    dict(QS=1, KVS=1, D=64, mask="causal"),
    dict(B=2, QN=4, KVN=2, QS=17, KVS=33, D=64, mask="causal"),
    dict(B=1, QN=2, KVN=2, QS=200, KVS=200, D=128, mask="causal", layout="BSND"),
    dict(B=2, QN=8, KVN=2, QS=129, KVS=300, D=128, lens=(0, 300)),
    dict(B=2, QN=4, KVN=4, QS=333, KVS=333, D=64, dtype="f16", std=0.5, mask="causal",
         lens=(100, 333)),
    dict(B=1, QN=2, KVN=1, QS=64, KVS=64, D=128, mask="bool_causal", layout="BSND"),
    dict(B=2, QN=8, KVN=1, QS=256, KVS=512, D=128, dtype="f16"),
    dict(B=1, QN=3, KVN=3, QS=5, KVS=1000, D=128, lens=(1, 1000)),
    dict(B=1, QN=2, KVN=1, QS=150, KVS=150, D=128, mask="causal", scale=-0.09),
    dict(B=1, QN=2, KVN=2, QS=96, KVS=200, D=64, scale=-0.125, layout="BSND"),
    dict(B=1, QN=2, KVN=2, QS=300, KVS=77, D=128, scale=-0.07, layout="BSND"),  # 256-row tiles, ragged
    dict(B=2, QN=4, KVN=2, QS=513, KVS=640, D=128, lens=(0, 640)),
    dict(B=2, QN=4, KVN=2, QS=300, KVS=300, D=256, mask="causal"),          # D = 256
    dict(B=1, QN=2, KVN=1, QS=129, KVS=700, D=256, dtype="f16", layout="BSND", lens=(1, 700)),
    dict(B=1, QN=2, KVN=2, QS=64, KVS=64, D=256, mask="bool_causal"),
    # scale 1: scores spread over tens of units, so a row's running max moves
    # by more than 2^8 well after its first tile and the rescale of a
    # non-zero output runs often
    dict(B=1, QN=2, KVN=2, QS=300, KVS=700, D=256, scale=1.0),
    dict(B=1, QN=2, KVN=1, QS=300, KVS=700, D=256, scale=1.0, mask="causal", layout="BSND"),
    dict(B=1, QN=2, KVN=1, QS=300, KVS=700, D=128, scale=1.0, mask="causal"),
    dict(B=1, QN=2, KVN=2, QS=200, KVS=500, D=64, scale=0.7),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_prefill_matches_oracle(case):
    inp = fa_synth.make(spec(**case))
    full_check(inp, what=str(case))


def test_prefill_causal_mode_equals_bool_mask():
    inp = fa_synth.make(spec(layout="BSND", B=1, QN=4, KVN=4, QS=300, KVS=300, mask="bool_causal",
                             seed=17))
    o1, l1 = run_fwd(inp, "bool")
    o2, l2 = run_fwd(inp, "causal")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_prefill_random_bool_mask_with_empty_rows():
    s = spec(layout="BNSD", B=2, QN=4, KVN=2, QS=70, KVS=150, D=64, seed=19)
    inp = fa_synth.make(s)
    rng = np.random.default_rng(2)
    mask = (rng.random((2, 4, 70, 150)) < 0.7).astype(np.uint8)
    mask[1, 2, 5, :] = 1
    inp.mask = mask
    inp.mask_strides = (4 * 70 * 150, 70 * 150, 150, 1)
    e = full_check(inp, "bool", "random bool mask")
    out, lse = run_fwd(inp, "bool")
    assert math.isinf(float(lse[1, 2, 5])) and torch.all(out[1, 2, 5] == 0)


def _bool_mask_run(inp, mask_np, strides, byte_offset=0, summary=False):
    """fa_fwd with a boolean mask given as a (possibly offset) device byte buffer;
    with summary=True the workspace fa_workspace_size asks for is passed, so a
    staged mask is summarised per tile first."""
    s = inp.spec
    q, k, v = (dev16(x, s.dtype) for x in (inp.q, inp.k, inp.v))
    lens = None if inp.lens is None else torch.from_numpy(inp.lens).to(DEV)
    flat = np.zeros(mask_np.size + 64, np.uint8)
    flat[byte_offset:byte_offset + mask_np.size] = mask_np.reshape(-1)
    buf = torch.from_numpy(flat).to(DEV)
    p = fa.params_for(q, k, layout=s.layout, scale=s.softmax_scale, actual_seq_lengths=lens,
                      mask=buf.data_ptr() + byte_offset, mask_stride=strides)
    out = torch.empty_like(q)
    lse = torch.empty((s.B, s.QN, s.QS), dtype=torch.float32, device=DEV)
    nbytes = fa.fa_workspace_size(p) if summary else 0
    ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV) if nbytes else None
    fa.fa_fwd(p, q, k, v, out, lse, ws, nbytes, torch.cuda.current_stream())
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("byte_offset", [0, 4, 1], ids=["lds_staged", "dword_staged", "elementwise"])
def test_prefill_bool_mask_both_paths(byte_offset, D):
    """Rows of 16-byte aligned keys go through LDS in 16-byte loads (with per-wave
    tile skipping), rows of 4-byte aligned keys in 4-byte loads; a misaligned mask
    pointer takes the element-wise path.  All match the oracle."""
    s = spec(layout="BNSD", B=2, QN=4, KVN=2, QS=200, KVS=320, D=D, lens=(150, 320), seed=29)
    inp = fa_synth.make(s)
    rng = np.random.default_rng(5)
    mask = (rng.random((2, 4, 200, 320)) < 0.5).astype(np.uint8)
    mask[:, :, :, 256:] = 1          # a fully masked key tile
    mask[1, 3, :128, :] = 1          # a fully masked query tile of one head
    mask[0, 2, 77, :] = 1            # an empty row
    strides = (4 * 200 * 320, 200 * 320, 320, 1)
    out, lse = _bool_mask_run(inp, mask, strides, byte_offset)
    inp.mask, inp.mask_strides = mask, strides
    prob = oracle.Problem.from_inputs(inp, "bool")
    ref, ref_lse = oracle.attention(prob, inp.q, inp.k, inp.v)
    o_rows = rows_of(out, s, np.arange(s.B * s.QN * s.QS))
    check(o_rows, to_np(lse).reshape(-1), ref.reshape(-1, s.D), ref_lse.reshape(-1), "bool mask")
    assert math.isinf(float(lse[0, 2, 77])) and torch.all(out[0, 2, 77] == 0)


def test_prefill_broadcast_bool_mask_matches_oracle():
    """A (B,1,1,S) mask (one key mask per batch, as in the IFA example) broadcast over heads and rows."""
    s = spec(layout="BSND", B=3, QN=4, KVN=4, QS=130, KVS=256, D=64, seed=31)
    inp = fa_synth.make(s)
    rng = np.random.default_rng(8)
    mask = (rng.random((3, 1, 1, 256)) < 0.3).astype(np.uint8)
    strides = (256, 0, 0, 1)
    out, lse = _bool_mask_run(inp, mask, strides)
    inp.mask, inp.mask_strides = mask, strides
    prob = oracle.Problem.from_inputs(inp, "bool")
    ref, ref_lse = oracle.attention(prob, inp.q, inp.k, inp.v)
    o_rows = rows_of(out, s, np.arange(s.B * s.QN * s.QS))
    r_rows = np.ascontiguousarray(ref.transpose(0, 2, 1, 3)).reshape(-1, s.D)
    check(o_rows, to_np(lse).reshape(-1), r_rows, ref_lse.reshape(-1), "broadcast bool mask")


def _block_mask(rng, shape, p_dead, p_full, blk=(64, 64)):
    """Random mask built from blocks that are fully masked, fully visible or random."""
    m = (rng.random(shape) < 0.5).astype(np.uint8)
    nb_i = -(-shape[-2] // blk[0])
    nb_j = -(-shape[-1] // blk[1])
    kind = rng.random(shape[:-2] + (nb_i, nb_j))
    for idx in np.ndindex(*kind.shape):
        *lead, bi, bj = idx
        sl = tuple(lead) + (slice(bi * blk[0], (bi + 1) * blk[0]), slice(bj * blk[1], (bj + 1) * blk[1]))
        if kind[idx] < p_dead:
            m[sl] = 1
        elif kind[idx] < p_dead + p_full:
            m[sl] = 0
    return m


SUMMARY_CASES = [
    # per-(b, n) block-sparse mask, ragged lengths, interior dead tiles
    dict(s=dict(layout="BNSD", B=2, QN=4, KVN=2, QS=300, KVS=1024, D=128, lens=(700, 1024), seed=41),
         shape=(2, 4, 300, 1024), bcast=(False, False), blk=(64, 64)),
    # broadcast causal pattern, sizes that are not tile multiples
    dict(s=dict(layout="BSND", B=2, QN=4, KVN=4, QS=464, KVS=464, D=64, seed=43),
         shape=(1, 1, 464, 464), bcast=(True, True), blk=None),
    # per-batch mask broadcast over heads, D = 256, 32-key blocks
    dict(s=dict(layout="BNSD", B=2, QN=4, KVN=1, QS=200, KVS=640, D=256, dtype="f16", seed=47),
         shape=(2, 1, 200, 640), bcast=(False, True), blk=(32, 32)),
    # more KV tiles (1040) than the lanes keep classes for (1024): tiles past
    # them run as partly masked, the loop bounds still come from the summary
    # (four query heads on one KV head, the mask broadcast over them: 520 rows
    # per KV head, past what the split path takes, so this stays a prefill)
    dict(s=dict(layout="BNSD", B=1, QN=4, KVN=1, QS=130, KVS=66560, D=64, seed=53),
         shape=(1, 1, 130, 66560), bcast=(False, True), blk=(128, 1024)),
]


@pytest.mark.parametrize("case", SUMMARY_CASES, ids=lambda c: "{layout}-QS{QS}-KVS{KVS}-D{D}".format(**c["s"]))
def test_prefill_mask_summary_changes_nothing(case):
    """The per-tile summary of a staged mask only removes work: outputs with and
    without it are identical, and match the oracle."""
    s = spec(**case["s"])
    inp = fa_synth.make(s)
    rng = np.random.default_rng(case["s"]["seed"])
    shape = case["shape"]
    if case["blk"] is None:
        mask = np.triu(np.ones(shape[-2:], np.uint8), 1).reshape(shape)
    else:
        mask = _block_mask(rng, shape, 0.4, 0.3, case["blk"])
    if shape[-1] > 60000:   # first and last visible tiles far apart, past tile 1024
        mask[..., :, :] = 1
        mask[..., :, 64 * 3:64 * 5] = (rng.random((shape[-2], 128)) < 0.5)
        mask[..., :, 64 * 1030:64 * 1031] = 0
        mask[..., :, 64 * 1033:64 * 1034 - 5] = (rng.random((shape[-2], 59)) < 0.5)
    mask[tuple(0 for _ in shape[:-2]) + (3,)] = 1      # an empty row
    st_i, st_j = shape[-1], 1
    st_n = 0 if case["bcast"][1] else shape[-2] * shape[-1]
    st_b = 0 if case["bcast"][0] else shape[1] * shape[-2] * shape[-1]
    strides = (st_b, st_n, st_i, st_j)
    o0, l0 = _bool_mask_run(inp, mask, strides, summary=False)
    o1, l1 = _bool_mask_run(inp, mask, strides, summary=True)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    inp.mask, inp.mask_strides = mask, strides
    prob = oracle.Problem.from_inputs(inp, "bool")
    ref, ref_lse = oracle.attention(prob, inp.q, inp.k, inp.v)
    o_rows = rows_of(o1, s, np.arange(s.B * s.QN * s.QS))
    r_rows = ref if s.layout == "BNSD" else ref.transpose(0, 2, 1, 3)
    r_rows = np.ascontiguousarray(r_rows).reshape(-1, s.D)
    check(o_rows, to_np(l1).reshape(-1), r_rows, ref_lse.reshape(-1), "mask summary")


def _expected_summary(mask, strides, B, QN, QS, KVS):
    """The per-tile classes fa_fwd writes to its workspace for a staged mask:
    per (slice, 128-row q tile) a row of 32-bit words, 16 KV tiles of 64 keys
    per word, bit 0 = some key visible, bit 1 = some key masked."""
    flat = mask.reshape(-1)
    sb = B if strides[0] else 1
    sn = QN if strides[1] else 1
    qt_n = -(-QS // 128)
    words = -(-(-(-KVS // 64)) // 16)
    out = np.zeros((sb, sn, qt_n, words), np.uint32)
    for b in range(sb):
        for n in range(sn):
            base = b * strides[0] + n * strides[1]
            rows = np.arange(QS)[:, None] * strides[2] + np.arange(KVS)[None, :] * strides[3]
            m = flat[base + rows]
            for qt in range(qt_n):
                for jt in range(-(-KVS // 64)):
                    sub = m[qt * 128:(qt + 1) * 128, jt * 64:(jt + 1) * 64]
                    c = int((sub == 0).any()) | (int((sub != 0).any()) << 1)
                    out[b, n, qt, jt // 16] |= np.uint32(c << (2 * (jt % 16)))
    return out.reshape(-1)


@pytest.mark.parametrize("case", [0, 1], ids=["causal_broadcast", "per_head_blocks"])
def test_mask_summary_words(case):
    """The summary kernel's words, read back from the caller's workspace, equal
    the classes computed from the mask on the host."""
    if case == 0:
        s = spec(layout="BSND", B=2, QN=4, KVN=1, QS=464, KVS=1200, D=64, seed=59)  # 1856 rows per KV head: a prefill
        mask = np.triu(np.ones((464, 1200), np.uint8), 1)[None, None]
        strides = (0, 0, 1200, 1)
    else:
        s = spec(layout="BNSD", B=1, QN=3, KVN=1, QS=200, KVS=1104, D=128, seed=61)
        mask = _block_mask(np.random.default_rng(61), (1, 3, 200, 1104), 0.4, 0.3, (64, 64))
        strides = (0, 200 * 1104, 1104, 1)
    inp = fa_synth.make(s)
    q, k, v = (dev16(x, s.dtype) for x in (inp.q, inp.k, inp.v))
    buf = torch.from_numpy(np.ascontiguousarray(mask).reshape(-1)).to(DEV)
    p = fa.params_for(q, k, layout=s.layout, scale=s.softmax_scale, mask=buf, mask_stride=strides)
    nbytes = fa.fa_workspace_size(p)
    ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(q)
    fa.fa_fwd(p, q, k, v, out, None, ws, nbytes, torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = _expected_summary(mask, strides, s.B, s.QN, s.QS, s.KVS)
    got = ws.cpu().numpy()[:want.size * 4].view(np.uint32)
    assert np.array_equal(got, want)


def test_prefill_staged_causal_mask_equals_causal_mode():
    inp = fa_synth.make(spec(layout="BSND", B=1, QN=4, KVN=2, QS=320, KVS=320, mask="bool_causal",
                             seed=37))
    o1, l1 = run_fwd(inp, "bool")
    o2, l2 = run_fwd(inp, "causal")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_prefill_ignores_nan_padding():
    inp = fa_synth.make(spec(layout="BNSD", B=3, QN=2, KVN=2, QS=100, KVS=300, D=128, lens=(0, 300),
                             mask="causal", seed=23))
    base, bl = run_fwd(inp)
    pad = fa_synth.fill_padding(inp, fa_synth.NAN_BITS["bf16"])
    out, lse = run_fwd(pad)
    assert torch.equal(out, base) and torch.equal(lse, bl)


# ------------------------------------------------------------------ window mask

def run_window(inp, window):
    s = inp.spec
    q, k, v = (dev16(x, s.dtype) for x in (inp.q, inp.k, inp.v))
    lens = None if inp.lens is None else torch.from_numpy(inp.lens).to(DEV)
    out, lse = fa.fwd(q, k, v, layout=s.layout, scale=s.softmax_scale, actual_seq_lengths=lens,
                      window=window, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def window_prob(inp, window):
    s = inp.spec
    return oracle.Problem(s.B, s.QN, s.KVN, s.QS, s.KVS, s.D, s.layout, s.dtype, s.softmax_scale,
                          inp.lens, "window", window=window)


WINDOW_CASES = [
    (dict(layout="BSND", B=2, QN=4, KVN=2, QS=300, KVS=300, D=128), (64, 0)),
    (dict(B=1, QN=4, KVN=4, QS=200, KVS=500, D=64, dtype="f16", std=0.5, lens=(100, 500)), (10, 30)),
    (dict(B=1, QN=2, KVN=1, QS=130, KVS=130, D=128), (0, 0)),
    (dict(B=2, QN=2, KVN=2, QS=300, KVS=300, D=128, lens=(50, 60)), (20, 0)),   # rows with no key
    (dict(B=1, QN=8, KVN=2, QS=1, KVS=700, D=128, lens=(300, 700)), (0, 200)),  # decode row
    (dict(B=1, QN=2, KVN=2, QS=257, KVS=1000, D=64, layout="BSND"), (-1, 100)),
    (dict(B=1, QN=2, KVN=2, QS=400, KVS=400, D=128, scale=-0.09), (150, -1)),
    (dict(B=1, QN=2, KVN=1, QS=300, KVS=300, D=256), (70, 5)),
]


@pytest.mark.parametrize("case,window", WINDOW_CASES,
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()) if isinstance(c, dict) else str(c))
def test_window_matches_oracle(case, window):
    inp = fa_synth.make(spec(seed=91, **case))
    s = inp.spec
    out, lse = run_window(inp, window)
    ref, ref_lse = oracle.attention_rows(window_prob(inp, window), inp.q, inp.k, inp.v)
    check(rows_of(out, s, np.arange(s.B * s.QN * s.QS)), to_np(lse).reshape(-1), ref, ref_lse,
          f"window {window} {case}")


def test_window_special_cases_equal_causal_and_none():
    """(-1, 0) reproduces the causal mode bit for bit (the same tiled kernel); (-1, -1)
    agrees with the unmasked path, which at D = 128 runs another kernel (the interleaved
    one, whose sums round in another order), within the parity bar, and both match the
    oracle."""
    inp = fa_synth.make(spec(layout="BNSD", B=1, QN=4, KVN=2, QS=333, KVS=333, lens=(200, 333),
                             seed=92))
    o1, l1 = run_window(inp, (-1, 0))
    o2, l2 = run_fwd(inp, "causal")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o1, l1 = run_window(inp, (-1, -1))
    o2, l2 = run_fwd(inp, "none")
    check(to_np(o1), to_np(l1), to_np(o2), to_np(l2), "window (-1, -1) vs no mask")
    ref, ref_lse = oracle.attention(oracle.Problem.from_inputs(inp, "none"), inp.q, inp.k, inp.v)
    check(to_np(o1), to_np(l1), ref, ref_lse, "window (-1, -1) vs oracle")
    check(to_np(o2), to_np(l2), ref, ref_lse, "no mask vs oracle")


def test_window_4k_sampled():
    """Sliding window of 1024 keys on the 4096-token prefill shape (sampled rows)."""
    inp = workload("prefill_4k")
    s = inp.spec
    out, lse = run_window(inp, (1024, 0))
    rows = fa_synth.sample_rows(s, 2000, seed=12, lens=inp.lens)
    ref, ref_lse = oracle.attention_rows(window_prob(inp, (1024, 0)), inp.q, inp.k, inp.v, rows)
    check(rows_of(out, s, rows), to_np(lse).reshape(-1)[rows], ref, ref_lse, "window 4k")


# ------------------------------------------------------------------ packed variable length (TND)

def run_packed(x, mode="none", window=None, seqused_q=None, kv_lens=None, extra_rows=0):
    """fa_fwd on packed inputs; extra_rows appends q rows owned by no sequence."""
    q_bits = x.q
    if extra_rows:
        pad = fa_synth.round_bits(np.ones((extra_rows, x.QN, x.D), np.float32), x.dtype)
        q_bits = np.concatenate([x.q, pad])
    q, k, v = dev16(q_bits, x.dtype), dev16(x.k, x.dtype), dev16(x.v, x.dtype)
    t32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)
    lens_t = None if kv_lens is None else torch.from_numpy(np.asarray(kv_lens, np.int64)).to(DEV)
    out, lse = fa.fwd(q, k, v, layout="TND", scale=x.scale, causal=(mode == "causal"),
                      window=window, actual_seq_lengths=lens_t, cu_seqlens_q=t32(x.cu_q),
                      cu_seqlens_kv=t32(x.cu_kv), seqused_q=t32(seqused_q), return_lse=True)
    torch.cuda.synchronize()
    return out, lse, q_bits


def packed_prob(x, q_total, mode="none", window=(-1, -1), seqused_q=None, kv_lens=None):
    return oracle.Problem(len(x.cu_q) - 1, x.QN, x.KVN, q_total, int(x.cu_kv[-1]), x.D, "TND",
                          x.dtype, x.scale, kv_lens, mode, window=window, cu_seqlens_q=x.cu_q,
                          cu_seqlens_kv=x.cu_kv, seqused_q=seqused_q)


PACKED_CASES = [
    (dict(B=5, QN=4, KVN=2, D=128, q_lens=(1, 300)), "none", None),
    (dict(B=5, QN=4, KVN=2, D=128, q_lens=(1, 300)), "causal", None),
    (dict(B=4, QN=8, KVN=2, D=128, q_lens=(1, 200), kv_lens=(0, 500)), "causal", None),
    (dict(B=3, QN=2, KVN=2, D=64, dtype="f16", std=0.5, q_lens=(100, 400)), "window", (50, 10)),
    (dict(B=7, QN=2, KVN=1, D=128, q_lens=(0, 3)), "none", None),                 # tiny and empty
    (dict(B=2, QN=2, KVN=2, D=64, q_lens=(129, 260), scale=-0.1), "causal", None),
    (dict(B=3, QN=4, KVN=2, D=256, q_lens=(1, 300)), "causal", None),
    (dict(B=4, QN=4, KVN=1, D=128, q_lens=(1, 600), kv_lens=(100, 700)), "window", (200, 0)),
    (dict(B=3, QN=2, KVN=2, D=256, dtype="f16", q_lens=(50, 400)), "window", (100, 30)),
]


@pytest.mark.parametrize("case,mode,window", PACKED_CASES,
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()) if isinstance(c, dict) else str(c))
def test_packed_matches_oracle(case, mode, window):
    x = fa_synth.make_packed(seed=111, **case)
    out, lse, q_bits = run_packed(x, mode, window)
    prob = packed_prob(x, int(x.cu_q[-1]), mode, window or (-1, -1))
    ref, ref_lse = oracle.attention(prob, q_bits, x.k, x.v)
    check(to_np(out).reshape(-1, x.D), to_np(lse).reshape(-1), ref.reshape(-1, x.D),
          ref_lse.reshape(-1), f"packed {case} {mode}")


def test_packed_truncation_and_unowned_rows():
    """seqused_q, KV lengths, an empty sequence and q rows past the last sequence
    (written as 0 with lse +inf)."""
    x = fa_synth.make_packed(4, 4, 2, 128, q_lens=(0, 300), seed=112)
    used = np.array([5, 0, 1000, 130], np.int32)
    kv_lens = np.array([300, 7, 0, 64], np.int64)
    out, lse, q_bits = run_packed(x, "causal", seqused_q=used, kv_lens=kv_lens, extra_rows=77)
    prob = packed_prob(x, q_bits.shape[0], "causal", seqused_q=used, kv_lens=kv_lens)
    ref, ref_lse = oracle.attention(prob, q_bits, x.k, x.v)
    got = to_np(out).reshape(-1, x.D)
    check(got, to_np(lse).reshape(-1), ref.reshape(-1, x.D), ref_lse.reshape(-1), "packed trunc")
    tail = got.reshape(-1, x.QN, x.D)[int(x.cu_q[-1]):]
    assert np.all(tail == 0) and torch.all(torch.isposinf(lse[int(x.cu_q[-1]):]))


def test_packed_equals_each_sequence_alone():
    """Every sequence of the packed batch gives, bit for bit, the BSND kernel on that
    sequence alone: same tiles, same order, same arithmetic."""
    x = fa_synth.make_packed(5, 8, 2, 128, q_lens=(1, 400), seed=113)
    out, lse, _ = run_packed(x, "causal")
    for b in range(5):
        q0, q1, k0, k1 = (int(v) for v in (x.cu_q[b], x.cu_q[b + 1], x.cu_kv[b], x.cu_kv[b + 1]))
        if q1 == q0:
            continue
        q = dev16(x.q[None, q0:q1], x.dtype)
        k, v = dev16(x.k[None, k0:k1], x.dtype), dev16(x.v[None, k0:k1], x.dtype)
        o1, l1 = fa.fwd(q, k, v, layout="BSND", scale=x.scale, causal=True, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out[q0:q1], o1[0])
        assert torch.equal(lse[q0:q1], l1[0].transpose(0, 1))


@pytest.mark.parametrize("mode,window", [("causal", None), ("none", None), ("window", (150, 20))])
def test_packed_persistent_matches_oracle_and_each_sequence(mode, window):
    """More work-list entries x heads than CUs: the packed prefill runs one persistent
    workgroup per CU over the entries (padding entries included, which it skips).  Checked
    against the oracle, and bit for bit against sequences computed alone (a
    one-workgroup-per-tile launch)."""
    x = fa_synth.make_packed(40, 8, 2, 128, q_lens=(0, 300), seed=114)
    T = int(x.cu_q[-1])
    entries = -(-T // 128) + 40 + 1
    assert -(-entries // 8) * 8 * 8 > 256
    out, lse, q_bits = run_packed(x, mode, window)
    prob = packed_prob(x, T, mode, window or (-1, -1))
    ref, ref_lse = oracle.attention(prob, q_bits, x.k, x.v)
    check(to_np(out).reshape(-1, x.D), to_np(lse).reshape(-1), ref.reshape(-1, x.D), ref_lse.reshape(-1),
          f"packed persistent {mode}")
    seen = 0
    for b in range(40):
        q0, q1, k0, k1 = (int(v) for v in (x.cu_q[b], x.cu_q[b + 1], x.cu_kv[b], x.cu_kv[b + 1]))
        if q1 == q0 or k1 == k0:
            continue
        q = dev16(x.q[None, q0:q1], x.dtype)
        k, v = dev16(x.k[None, k0:k1], x.dtype), dev16(x.v[None, k0:k1], x.dtype)
        o1, l1 = fa.fwd(q, k, v, layout="BSND", scale=x.scale, causal=(mode == "causal"), window=window,
                        return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out[q0:q1], o1[0]), f"sequence {b}"
        assert torch.equal(lse[q0:q1], l1[0].transpose(0, 1)), f"sequence {b}"
        seen += 1
        if seen == 6:
            break


def test_workload_prefill_varlen_sampled():
    x = fa_synth.make_packed(**fa_synth.PACKED_WORKLOADS["prefill_varlen"])
    out, lse, _ = run_packed(x, "causal")
    T = int(x.cu_q[-1])
    rng = np.random.default_rng(13)
    # rows t*QN + n1: every sequence's first and last row plus a random sample
    ts = np.concatenate([x.cu_q[:-1], x.cu_q[1:] - 1, rng.integers(0, T, 1500)])
    rows = np.unique(ts.astype(np.int64) * x.QN + rng.integers(0, x.QN, ts.size))
    ref, ref_lse = oracle.attention_rows(packed_prob(x, T, "causal"), x.q, x.k, x.v, rows)
    got = to_np(out).reshape(-1, x.D)[rows]
    check(got, to_np(lse).reshape(-1)[rows], ref, ref_lse, "prefill_varlen")


# ------------------------------------------------------------------ the five workloads

def test_workload_prefill_small_full():
    full_check(workload("prefill_small"), what="prefill_small")


def test_workload_decode_gqa_full():
    full_check(workload("decode_gqa"), what="decode_gqa")


def test_workload_decode_128k_full():
    full_check(workload("decode_128k"), what="decode_128k")


@pytest.mark.parametrize("chunk", [1024, 2048, 4096])
def test_workload_decode_128k_chunks(chunk):
    inp = workload("decode_128k")
    splits = 131072 // chunk
    _, _, _, out, lse, _ = _partials(inp, splits, chunk)
    rows = np.arange(32)
    ref, ref_lse = oracle.attention_rows(oracle.Problem.from_inputs(inp), inp.q, inp.k, inp.v, rows)
    check(to_np(out).reshape(-1, 128), to_np(lse), ref, ref_lse, f"128k chunk {chunk}")


def sampled_check(name, mask_mode=None, n=3000):
    inp = workload(name)
    s = inp.spec
    out, lse = run_fwd(inp, mask_mode)
    rows = fa_synth.sample_rows(s, n, seed=11, lens=inp.lens)
    prob = oracle.Problem.from_inputs(inp, mask_mode)
    ref, ref_lse = oracle.attention_rows(prob, inp.q, inp.k, inp.v, rows)
    got = rows_of(out, s, rows)
    got_lse = to_np(lse).reshape(-1)[rows]
    return check(got, got_lse, ref, ref_lse, name)


def test_workload_prefill_causal_bool_sampled():
    sampled_check("prefill_causal")


def test_workload_prefill_causal_mode_sampled():
    sampled_check("prefill_causal", "causal")


def test_workload_prefill_4k_sampled():
    sampled_check("prefill_4k")


def test_workload_prefill_gqa_long_sampled():
    sampled_check("prefill_gqa_long", n=2000)


# ------------------------------------------------------------------ seeded shape sweep

def _sweep_case(seed):
    """A seeded draw over the parameter space the fixed cases sample by hand:
    decode (contiguous or paged) or prefill (no mask, causal, or the causal
    pattern as a boolean tensor), layout, head dim, dtype, GQA group, lengths,
    scale sign; sized so the oracle stays fast."""
    r = np.random.default_rng(1000 + seed)
    D = int(r.choice([64, 128, 128, 256]))
    KVN = int(r.choice([1, 2, 4, 8]))
    g = int(r.choice([1, 2, 3, 4, 6, 8, 16, 32]))
    while g * KVN > 64:
        g //= 2
    c = dict(layout=str(r.choice(["BNSD", "BSND"])), B=int(r.integers(1, 5)), QN=g * KVN, KVN=KVN,
             D=D, dtype=str(r.choice(["bf16", "f16"])), seed=seed)
    if r.random() < 0.3:
        c["scale"] = float(-r.uniform(0.03, 0.12))
    decode = r.random() < 0.5
    if decode:
        c.update(QS=1, KVS=int(r.integers(1, 6000)))
    else:
        c.update(QS=int(r.integers(1, 400)), KVS=int(r.integers(1, 700)),
                 mask=str(r.choice(["none", "causal", "bool_causal"])))
    if r.random() < 0.6:
        lo = int(r.integers(0, c["KVS"] + 1))
        c["lens"] = (lo, int(r.integers(lo, c["KVS"] + 1)))
    paged = None
    if decode and "lens" in c and r.random() < 0.5:
        paged = (str(r.choice(["PA_BBND", "PA_BNBD"])), 16 * int(r.integers(1, 9)))
    return c, paged


@pytest.mark.parametrize("seed", range(64))
def test_seeded_shape_sweep(seed):
    case, paged = _sweep_case(seed)
    inp = fa_synth.make(spec(**case))
    if paged is None:
        full_check(inp, what=f"sweep {seed}: {case}")
        return
    kv_layout, bs = paged
    s = inp.spec
    out, lse, table = run_paged(inp, kv_layout, bs, seed=seed)
    kp, vp, _, _ = fa_synth.to_paged(inp, bs, kv_layout, seed=seed)
    prob = oracle.Problem(s.B, s.QN, s.KVN, 1, s.KVS, s.D, s.layout, s.dtype, s.softmax_scale,
                          inp.lens, "none", kv_layout=kv_layout, block_table=table, block_size=bs)
    ref, ref_lse = oracle.attention(prob, inp.q, kp, vp)
    r_rows = np.ascontiguousarray(ref if s.layout == "BNSD" else ref.transpose(0, 2, 1, 3))
    check(rows_of(out, s, np.arange(s.B * s.QN)), to_np(lse).reshape(-1),
          r_rows.reshape(-1, s.D), ref_lse.reshape(-1), f"sweep {seed} paged {paged}: {case}")


# ------------------------------------------------------------------ split-KV, general rows
# Masked decode (IFA guide 4: attenMask (B,N,1,S) or (1,N,1,S) / (B,1,1,S)), used query
# lengths, and a few query positions against a long cache run stage 1 on the matrix
# cores with the rows (query head, position) of a KV head in 32-row tiles, then the
# combine (FlashAttn developer guide 1.9 and 4).

def _mask_for(s, kind, seed, all_masked=None):
    """A uint8 mask (nonzero = excluded) and its (b, n, i, j) strides.
    kind: "b11s" (B,1,1,S) broadcast over heads and positions, "bn1s" (B,N,1,S),
    "bnqs" (B,N,Q_S,S), "bqs_odd" (B,1,Q_S,S+3) rows with an odd pitch (byte reads)."""
    rng = np.random.default_rng(seed)
    if kind == "b11s":
        m = (rng.random((s.B, 1, 1, s.KVS)) < 0.4).astype(np.uint8)
        st = (s.KVS, 0, 0, 1)
    elif kind == "bn1s":
        m = (rng.random((s.B, s.QN, 1, s.KVS)) < 0.5).astype(np.uint8)
        st = (s.QN * s.KVS, s.KVS, 0, 1)
    elif kind == "bnqs":
        m = (rng.random((s.B, s.QN, s.QS, s.KVS)) < 0.3).astype(np.uint8)
        st = (s.QN * s.QS * s.KVS, s.QS * s.KVS, s.KVS, 1)
    else:
        pitch = s.KVS + 3
        m = (rng.random((s.B, 1, s.QS, pitch)) < 0.3).astype(np.uint8)
        st = (s.QS * pitch, 0, pitch, 1)
    if all_masked is not None:  # one batch masks every key of every row
        m[all_masked] = 1
    return np.ascontiguousarray(m), st


def run_general(inp, *, mask=None, mask_strides=(0, 0, 0, 0), causal=False, window=None,
                seqused=None, paging=None, scale=None):
    """fa.fwd on the inputs; returns (out rows [nrows, D] fp64, lse rows, oracle Problem)."""
    s = inp.spec
    sc = s.softmax_scale if scale is None else scale
    q = dev16(inp.q, s.dtype)
    lens_np = inp.lens
    if paging is not None and lens_np is None:
        lens_np = np.full(s.B, s.KVS, dtype=np.int64)
    lens = None if lens_np is None else torch.from_numpy(lens_np).to(DEV)
    kw = {}
    if paging is None:
        k, v = dev16(inp.k, s.dtype), dev16(inp.v, s.dtype)
    else:
        inp2 = dataclasses.replace(inp, lens=lens_np)
        kp, vp, table, nblocks = fa_synth.to_paged(inp2, paging[1], paging[0], seed=3)
        k, v = dev16(kp, s.dtype), dev16(vp, s.dtype)
        kw = dict(kv_layout=paging[0], block_table=torch.from_numpy(table).to(DEV))
    mask_t = None if mask is None else torch.from_numpy(mask).to(DEV)
    su = None if seqused is None else torch.from_numpy(np.asarray(seqused, np.int32)).to(DEV)
    out, lse = fa.fwd(q, k, v, layout=s.layout, scale=sc, actual_seq_lengths=lens, mask=mask_t,
                      mask_stride=mask_strides, causal=causal, window=window, seqused_q=su,
                      return_lse=True, **kw)
    torch.cuda.synchronize()
    mode = "bool" if mask is not None else ("causal" if causal else ("window" if window else "none"))
    prob = oracle.Problem(s.B, s.QN, s.KVN, s.QS, s.KVS, s.D, s.layout, s.dtype, sc, lens_np, mode,
                          mask, mask_strides, window=window if window else (-1, -1), seqused_q=seqused)
    return rows_of(out, s, np.arange(s.B * s.QN * s.QS)), to_np(lse).reshape(-1), prob


GENERAL_CASES = [
    # one query position with a boolean mask: broadcast over heads, and per head, with
    # one batch fully masked (its rows are 0 / +inf); g = 1 and g = 4; both layouts
    (dict(B=3, QN=8, KVN=2, QS=1, KVS=5000, D=128, lens=(1, 5000)), dict(mask="b11s", all_masked=1)),
    (dict(B=2, QN=4, KVN=4, QS=1, KVS=3000, D=64, layout="BSND"), dict(mask="bn1s", all_masked=0)),
    (dict(B=2, QN=32, KVN=1, QS=1, KVS=2000, D=128, dtype="f16", lens=(100, 2000)), dict(mask="bn1s")),
    (dict(B=1, QN=2, KVN=2, QS=1, KVS=777, D=128), dict(mask="bqs_odd")),          # byte-wise mask reads
    # the vector stage 1 with the mask (shapes without a matrix-core stage 1): g = 2
    # with a fully masked batch, D = 256 per head, g = 48 (eight heads per workgroup)
    (dict(B=2, QN=4, KVN=2, QS=1, KVS=3000, D=128, lens=(1, 3000)), dict(mask="b11s", all_masked=1)),
    (dict(B=2, QN=4, KVN=4, QS=1, KVS=2000, D=256, layout="BSND"), dict(mask="bn1s", all_masked=0)),
    (dict(B=1, QN=48, KVN=1, QS=1, KVS=1500, D=128, dtype="f16"), dict(mask="b11s")),
    # one query position, causal (top-left: key 0 only) and window
    (dict(B=2, QN=8, KVN=2, QS=1, KVS=3000, D=128, lens=(1, 3000)), dict(causal=True)),
    (dict(B=2, QN=8, KVN=8, QS=1, KVS=3000, D=128, layout="BSND"), dict(window=(0, 700))),
    # used query lengths with one position: batch 1 uses none
    (dict(B=3, QN=8, KVN=2, QS=1, KVS=2500, D=128, lens=(1, 2500)), dict(seqused=[1, 0, 5])),
    # a few positions against a long cache: no mask, a window reaching far right, boolean (B,N,Q_S,S); a top-left causal row sees at most Q_S keys, so fa_fwd runs such calls as a prefill (the split of that mask is tested through fa_decode_splitkv)
    (dict(B=1, QN=32, KVN=8, QS=8, KVS=65536, D=128), dict()),
    (dict(B=1, QN=32, KVN=8, QS=8, KVS=65536, D=128, layout="BSND"), dict(window=(-1, 30000))),
    (dict(B=2, QN=8, KVN=2, QS=5, KVS=9000, D=64, lens=(3000, 9000)), dict(mask="bnqs")),
    # four row groups (g * Q_S = 128), three (g * Q_S = 72) and odd counts
    (dict(B=1, QN=16, KVN=2, QS=16, KVS=20000, D=128, layout="BSND"), dict()),
    # 256 and 512 (query head, position) rows per KV head: 8 and 16 row groups
    (dict(B=1, QN=16, KVN=4, QS=64, KVS=6000, D=128), dict()),
    (dict(B=2, QN=16, KVN=4, QS=128, KVS=5000, D=64, layout="BSND", lens=(1000, 5000)), dict(mask="bnqs")),
    (dict(B=2, QN=24, KVN=3, QS=9, KVS=7000, D=64, dtype="f16", lens=(1, 7000)), dict(window=(40, 2000))),
    (dict(B=1, QN=3, KVN=1, QS=3, KVS=4000, D=128), dict(seqused=[2])),
    # negative scale
    (dict(B=1, QN=8, KVN=2, QS=4, KVS=6000, D=128, scale=-0.07), dict(mask="b11s")),
]


@pytest.mark.parametrize("case,opts", GENERAL_CASES,
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()) if isinstance(c, dict) else str(c))
def test_general_split_matches_oracle(case, opts):
    inp = fa_synth.make(spec(seed=151, **case))
    s = inp.spec
    o = dict(opts)
    mask, strides = None, (0, 0, 0, 0)
    if "mask" in o:
        mask, strides = _mask_for(s, o.pop("mask"), 152, o.pop("all_masked", None))
    p = fa.params_for(dev16(inp.q, s.dtype), dev16(inp.k, s.dtype), layout=s.layout,
                      scale=s.softmax_scale, causal=o.get("causal", False), window=o.get("window"),
                      mask=None if mask is None else torch.zeros(1, dtype=torch.uint8, device=DEV),
                      mask_stride=strides,
                      seqused_q=None if "seqused" not in o else torch.zeros(s.B, dtype=torch.int32, device=DEV))
    assert fa.fa_workspace_size(p) > 0, "expected the split-KV path"
    got, got_lse, prob = run_general(inp, mask=mask, mask_strides=strides, **o)
    ref, ref_lse = oracle.attention_rows(prob, inp.q, inp.k, inp.v)
    check(got, got_lse, ref, ref_lse, f"general split {case} {opts}")


def test_general_split_ignores_nan_padding():
    """Keys past each batch's length hold NaN: outputs are bit-identical (masked decode)."""
    inp = fa_synth.make(spec(layout="BSND", B=3, QN=8, KVN=2, QS=1, KVS=3000, lens=(0, 3000), seed=153))
    mask, st = _mask_for(inp.spec, "b11s", 154)
    base = run_general(inp, mask=mask, mask_strides=st)
    pad = fa_synth.fill_padding(inp, fa_synth.NAN_BITS["bf16"])
    again = run_general(pad, mask=mask, mask_strides=st)
    assert np.array_equal(base[0], again[0]) and np.array_equal(base[1], again[1])


@pytest.mark.parametrize("paging", [("PA_BBND", 64), ("PA_BNBD", 16)])
def test_general_split_on_paged_cache(paging):
    """A boolean mask and several positions on a paged cache: equal to the oracle, and bit
    for bit to the same call on the contiguous cache."""
    inp = fa_synth.make(spec(B=2, QN=8, KVN=2, QS=3, KVS=4100, D=128, lens=(1000, 4100), seed=155))
    mask, st = _mask_for(inp.spec, "bnqs", 156)
    got, got_lse, prob = run_general(inp, mask=mask, mask_strides=st, paging=paging)
    ref, ref_lse = oracle.attention_rows(prob, inp.q, inp.k, inp.v)
    check(got, got_lse, ref, ref_lse, f"paged general {paging}")
    base, base_lse, _ = run_general(inp, mask=mask, mask_strides=st)
    assert np.array_equal(got, base) and np.array_equal(got_lse, base_lse)


def test_general_stage1_partials_match_oracle_partials():
    """fa_decode_splitkv on several positions with a boolean mask: m, l and the unnormalised
    O of every (row, chunk) against the oracle's partials; fa_combine then gives the
    oracle's output."""
    inp = fa_synth.make(spec(B=2, QN=8, KVN=2, QS=4, KVS=3000, D=128, lens=(500, 3000), seed=157))
    s = inp.spec
    mask, st = _mask_for(s, "bnqs", 158)
    q, k, v = (dev16(x, s.dtype) for x in (inp.q, inp.k, inp.v))
    lens = torch.from_numpy(inp.lens).to(DEV)
    mt = torch.from_numpy(mask).to(DEV)
    p = fa.params_for(q, k, layout=s.layout, scale=s.softmax_scale, actual_seq_lengths=lens, mask=mt,
                      mask_stride=st)
    splits, chunk = 12, 256
    rows = s.B * s.QN * s.QS
    o_part = torch.empty((rows * splits * s.D,), dtype=torch.float32, device=DEV)
    m_part = torch.empty((rows * splits,), dtype=torch.float32, device=DEV)
    l_part = torch.empty((rows * splits,), dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream()
    fa.fa_decode_splitkv(p, splits, chunk, q, k, v, o_part, m_part, l_part, stream)
    out = torch.empty_like(q)
    lse = torch.empty((s.B, s.QN, s.QS), dtype=torch.float32, device=DEV)
    fa.fa_combine(p, splits, o_part, m_part, l_part, out, lse, stream)
    torch.cuda.synchronize()
    prob = oracle.Problem(s.B, s.QN, s.KVN, s.QS, s.KVS, s.D, s.layout, s.dtype, s.softmax_scale, inp.lens,
                          "bool", mask, st)
    ro, rm, rl = oracle.split_partials(prob, inp.q, inp.k, inp.v, splits, chunk)
    gm = m_part.cpu().numpy().reshape(rows, splits).astype(np.float64)
    gl = l_part.cpu().numpy().reshape(rows, splits).astype(np.float64)
    go = o_part.cpu().numpy().reshape(rows, splits, s.D).astype(np.float64)
    empty = np.isinf(rm)
    assert np.array_equal(np.isinf(gm) & (gm < 0), empty), "empty-chunk flags"
    assert np.all(gl[empty] == 0) and np.all(go[empty] == 0)
    live = ~empty
    assert np.abs(gm[live] - rm[live]).max() <= 1e-3
    # l and O: relative to the partial's own scale, plus the 16-bit rounding of P, whose
    # bound needs sum_j p_j |v_j|, the partial of the same scores with |V|
    assert np.all(np.abs(gl[live] - rl[live]) <= 2e-3 * rl[live] + 1e-6)
    vabs = np.ascontiguousarray(inp.v) & np.uint16(0x7FFF)
    ro_abs, _, _ = oracle.split_partials(prob, inp.q, inp.k, vabs, splits, chunk)
    tol = 2e-3 * np.abs(ro).max(axis=2, keepdims=True) + 2.0 ** -8 * ro_abs + 1e-6
    assert np.all((np.abs(go - ro) <= tol)[live]), "general stage-1 O partials"
    ref, ref_lse = oracle.attention_rows(prob, inp.q, inp.k, inp.v)
    check(rows_of(out, s, np.arange(rows)), to_np(lse).reshape(-1), ref, ref_lse, "general combine")


@pytest.mark.parametrize("mode,window", [("causal", None), ("window", (40, 2)), ("window", (-1, 300))])
def test_general_split_causal_and_window_explicit(mode, window):
    """fa_decode_splitkv + fa_combine on several positions under the causal flag or a
    window.  fa_fwd sends shapes whose rows see so few keys to the prefill; the split
    stage 1 still takes them.  The result matches the oracle's output."""
    inp = fa_synth.make(spec(B=2, QN=8, KVN=2, QS=6, KVS=3000, D=128, lens=(500, 3000), seed=161))
    s = inp.spec
    q, k, v = (dev16(x, s.dtype) for x in (inp.q, inp.k, inp.v))
    lens = torch.from_numpy(inp.lens).to(DEV)
    p = fa.params_for(q, k, layout=s.layout, scale=s.softmax_scale, actual_seq_lengths=lens,
                      causal=(mode == "causal"), window=window)
    assert "path=prefill" in fa.fa_describe(p)
    splits, chunk = 12, 256
    rows = s.B * s.QN * s.QS
    o_part = torch.empty((rows * splits * s.D,), dtype=torch.float32, device=DEV)
    m_part = torch.empty((rows * splits,), dtype=torch.float32, device=DEV)
    l_part = torch.empty((rows * splits,), dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream()
    fa.fa_decode_splitkv(p, splits, chunk, q, k, v, o_part, m_part, l_part, stream)
    out = torch.empty_like(q)
    lse = torch.empty((s.B, s.QN, s.QS), dtype=torch.float32, device=DEV)
    fa.fa_combine(p, splits, o_part, m_part, l_part, out, lse, stream)
    torch.cuda.synchronize()
    prob = oracle.Problem(s.B, s.QN, s.KVN, s.QS, s.KVS, s.D, s.layout, s.dtype, s.softmax_scale, inp.lens,
                          mode, window=window or (-1, -1))
    ref, ref_lse = oracle.attention_rows(prob, inp.q, inp.k, inp.v)
    check(rows_of(out, s, np.arange(rows)), to_np(lse).reshape(-1), ref, ref_lse, f"explicit split {mode} {window}")


@pytest.mark.parametrize("layout,causal", [("BNSD", True), ("BSND", False), ("BNSD", False)])
def test_prefill_seqused_q_padded_layouts(layout, causal):
    """seqused_q on BNSD/BSND prefill (developer guide 1.4): rows past each batch's used
    length are 0 / +inf, the rest match the oracle (tiled kernel when causal, the
    interleaved kernel for mask-free D = 128, whole query tiles unused included)."""
    inp = fa_synth.make(spec(layout=layout, B=3, QN=4, KVN=2, QS=600, KVS=700, D=128, lens=(300, 700),
                             seed=159))
    got, got_lse, prob = run_general(inp, causal=causal, seqused=[599, 0, 130])
    ref, ref_lse = oracle.attention_rows(prob, inp.q, inp.k, inp.v)
    check(got, got_lse, ref, ref_lse, f"prefill seqused {layout} causal={causal}")


@pytest.mark.parametrize("case,opts", [
    (dict(B=1, QN=2, KVN=2, QS=300, KVS=333, D=128), dict()),                       # interleaved prefill
    (dict(B=2, QN=2, KVN=1, QS=200, KVS=250, D=64, lens=(7, 250)), dict(causal=True)),  # tiled prefill
    (dict(B=2, QN=4, KVN=4, QS=1, KVS=1000, D=128, lens=(1, 1000)), dict()),        # vector decode
    (dict(B=2, QN=16, KVN=4, QS=1, KVS=1500, D=128, lens=(1, 1500)), dict()),       # matrix-core decode
    (dict(B=1, QN=8, KVN=2, QS=3, KVS=900, D=128), dict(mask="b11s")),              # general split
])
def test_scale_zero_gives_the_mean_of_visible_values(case, opts):
    """scale = 0: every score is 0, so each row is the plain mean of the values it sees and
    lse = ln(count); masked keys and keys past the length must still be excluded."""
    inp = fa_synth.make(spec(seed=160, **case))
    s = inp.spec
    o = dict(opts)
    mask, st = None, (0, 0, 0, 0)
    if "mask" in o:
        mask, st = _mask_for(s, o.pop("mask"), 161)
    got, got_lse, prob = run_general(inp, mask=mask, mask_strides=st, scale=0.0, **o)
    assert np.all(np.isfinite(got))
    ref, ref_lse = oracle.attention_rows(prob, inp.q, inp.k, inp.v)
    check(got, got_lse, ref, ref_lse, f"scale 0 {case}")


# More query tiles of 256 rows than the device has CUs: the mask-free, the
# window and the causal prefill at head dim 128 then run one persistent
# workgroup per CU that takes the tiles in turn, fetching the next tile's Q and
# first K tile during the current one's last slot; causal rounds alternate
# direction.  (The packed layout's persistent launch is tested with the packed
# cases.)
PERSISTENT_CASES = [
    (dict(B=3, QN=44, KVN=11, QS=300, KVS=300, D=128), (300, 0, 131), None, None),
    (dict(layout="BSND", B=3, QN=44, KVN=4, QS=300, KVS=333, D=128, dtype="f16"), (333, 77, 1),
     None, [300, 0, 257]),
    (dict(B=3, QN=44, KVN=44, QS=300, KVS=700, D=128), (700, 5, 400), (100, 20), None),
    (dict(layout="BSND", B=2, QN=64, KVN=8, QS=520, KVS=520, D=128), None, (300, 0), [520, 400]),
    (dict(B=3, QN=44, KVN=4, QS=300, KVS=600, D=128, scale=1.0), None, (-1, 40), [300, 299, 1]),
    (dict(B=3, QN=44, KVN=4, QS=300, KVS=300, D=128), None, "causal", None),
    (dict(layout="BSND", B=1, QN=52, KVN=4, QS=1300, KVS=1400, D=128, dtype="f16"), None, "causal", None),
    (dict(B=3, QN=44, KVN=4, QS=520, KVS=600, D=128, dtype="f16"), (600, 3, 311), "causal", [520, 520, 100]),
]


@pytest.mark.parametrize("case,lens,mode,seqused", PERSISTENT_CASES,
                         ids=["none", "none_f16_bsnd_used", "window_back", "window_causal_used",
                              "window_forward_rescale", "causal_partial_round", "causal_six_ranks",
                              "causal_ragged_used"])
def test_persistent_prefill_matches_oracle_and_per_batch_launches(case, lens, mode, seqused):
    """The persistent launch against the oracle, and bit for bit against each batch
    computed alone (fewer tiles than CUs: one workgroup per tile).  KV lengths include
    0 and 1, used query rows include 0 and a partial last tile."""
    inp = fa_synth.make(spec(seed=170, **case))
    if lens is not None:
        inp = dataclasses.replace(inp, lens=np.asarray(lens, dtype=np.int64))
    s = inp.spec
    units = s.B * s.QN * -(-s.QS // 256)
    assert units > 256, "the case must have more tiles than the CUs of the device"
    causal = mode == "causal"
    window = None if (mode is None or causal) else mode
    p = fa.params_for(dev16(inp.q, s.dtype), dev16(inp.k, s.dtype), layout=s.layout,
                      scale=s.softmax_scale, window=window, causal=causal)
    assert "persistent" in fa.fa_describe(p), fa.fa_describe(p)
    got, got_lse, prob = run_general(inp, window=window, causal=causal, seqused=seqused)
    ref, ref_lse = oracle.attention_rows(prob, inp.q, inp.k, inp.v)
    check(got, got_lse, ref, ref_lse, f"persistent {case} {mode}")
    per_row = s.QN * s.QS
    for b in range(s.B if s.B > 1 else 0):
        one = dataclasses.replace(
            inp, spec=dataclasses.replace(s, B=1), q=inp.q[b:b + 1], k=inp.k[b:b + 1], v=inp.v[b:b + 1],
            lens=None if inp.lens is None else inp.lens[b:b + 1])
        o1, l1, _ = run_general(one, window=window, causal=causal,
                                seqused=None if seqused is None else seqused[b:b + 1])
        assert np.array_equal(o1, got[b * per_row:(b + 1) * per_row]), f"batch {b} output"
        assert np.array_equal(l1, got_lse[b * per_row:(b + 1) * per_row]), f"batch {b} lse"


def test_persistent_prefill_graph_replays():
    """The persistent causal prefill captured in a HIP graph: every replay, with new q and
    eager work in between, equals the eager call bit for bit (the launch keeps no state
    between calls)."""
    inp = fa_synth.make(spec(layout="BSND", B=3, QN=44, KVN=4, QS=300, KVS=300, D=128, seed=171))
    s = inp.spec
    q, k, v = (dev16(x, s.dtype) for x in (inp.q, inp.k, inp.v))
    p = fa.params_for(q, k, layout=s.layout, scale=s.softmax_scale, causal=True)
    assert "persistent" in fa.fa_describe(p), fa.fa_describe(p)
    out = torch.empty_like(q)
    lse = torch.empty((s.B, s.QN, s.QS), dtype=torch.float32, device=DEV)
    qg = q.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up off the capture
        fa.fa_fwd(p, qg, k, v, out, lse, None, 0, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.fa_fwd(p, qg, k, v, out, lse, None, 0, torch.cuda.current_stream())
    for rep in range(3):
        qn = torch.randn(q.shape, device=DEV).to(q.dtype)
        qg.copy_(qn)
        graph.replay()
        torch.cuda.synchronize()
        ref_out, ref_lse = fa.fwd(qn, k, v, layout=s.layout, scale=s.softmax_scale, causal=True,
                                  return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {rep}"
        assert torch.equal(lse, ref_lse), f"replay {rep}"


@pytest.mark.parametrize("paging,g", [(("PA_BBND", 128), 4), (("PA_BNBD", 48), 4), (("PA_BBND", 128), 2),
                                      (("PA_BBND", 128), 1), (("PA_BNBD", 64), 8)])
def test_decode_fused_on_paged_cache(paging, g):
    """The single-launch split-KV on a paged cache, with the fused plan: equal to the oracle."""
    inp = fa_synth.make(spec(layout="BSND", B=3, QN=2 * g, KVN=2, QS=1, KVS=5000, lens=(1, 5000), seed=162))
    s = inp.spec
    kp, vp, table, nblocks = fa_synth.to_paged(inp, paging[1], paging[0], seed=4)
    q, k, v = dev16(inp.q, s.dtype), dev16(kp, s.dtype), dev16(vp, s.dtype)
    lens = torch.from_numpy(inp.lens).to(DEV)
    p = fa.params_for(q, k, layout=s.layout, scale=s.softmax_scale, actual_seq_lengths=lens,
                      kv_layout=paging[0], block_table=torch.from_numpy(table).to(DEV))
    sp, ch, nbytes = fa.fa_decode_fused_plan(p)
    assert sp > 1
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty((s.B, s.QN, 1), dtype=torch.float32, device=DEV)
    fa.fa_decode_fused(p, sp, ch, q, k, v, ws, nbytes, out, lse, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(oracle.Problem.from_inputs(inp), inp.q, inp.k, inp.v)
    check(to_np(out), to_np(lse), ref, ref_lse, f"fused paged {paging}")


# ------------------------------------------------------------------ offsets past 2^31 elements

@pytest.mark.parametrize("QN", [8, 32], ids=["vector_stage1", "matrix_core_stage1"])
def test_decode_offsets_past_2_31_elements(QN):
    """Decode whose last batch's K and V start at element 2^31 (4 GiB of bf16 in):
    17 batches of 131072 keys x 8 KV heads x 128.  The far batch holds random data
    at full length; the others random data in a short prefix (their used lengths)
    and zeros beyond.  Each part is checked against the oracle on that part alone."""
    B, KVN, S, D = 17, 8, 131072, 128
    rng = np.random.default_rng(2031)
    far = fa_synth.make(spec(layout="BSND", B=1, QN=QN, KVN=KVN, QS=1, KVS=S, D=D, seed=2032))
    near_lens = rng.integers(1, 65, size=B - 1).astype(np.int64)
    near = fa_synth.make(spec(layout="BSND", B=B - 1, QN=QN, KVN=KVN, QS=1, KVS=64, D=D, seed=2033))
    near.lens = near_lens
    k = torch.zeros((B, S, KVN, D), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    assert 16 * k.stride(0) == 2 ** 31
    k[B - 1] = dev16(far.k, "bf16")[0]
    v[B - 1] = dev16(far.v, "bf16")[0]
    k[: B - 1, :64] = dev16(near.k, "bf16")
    v[: B - 1, :64] = dev16(near.v, "bf16")
    q = torch.cat([dev16(near.q, "bf16"), dev16(far.q, "bf16")])
    lens = torch.from_numpy(np.concatenate([near_lens, [S]])).to(DEV)
    out, lse = fa.fwd(q, k, v, layout="BSND", scale=far.spec.softmax_scale, actual_seq_lengths=lens,
                      return_lse=True)
    torch.cuda.synchronize()
    del k, v
    for part, sl in ((far, slice(B - 1, B)), (near, slice(0, B - 1))):
        ref, ref_lse = oracle.attention(oracle.Problem.from_inputs(part, "none"), part.q, part.k, part.v)
        s = part.spec
        got = to_np(out[sl].permute(0, 2, 1, 3)).reshape(-1, D)
        r_rows = np.ascontiguousarray(ref.transpose(0, 2, 1, 3)).reshape(-1, D)
        check(got, to_np(lse[sl]).reshape(-1), r_rows, ref_lse.reshape(-1), f"decode past 2^31, {s.B} batches")


def test_packed_prefill_offsets_past_2_31_elements():
    """Packed causal prefill of 4097 sequences of 128 tokens, 32/8 heads, D = 128: the
    last sequence's q rows start at element 2^31.  That sequence holds random data and
    is checked against the oracle; the others are all zeros, where every row's output
    is exactly 0 and its lse is ln(visible keys)."""
    NS, L, QN, KVN, D = 4097, 128, 32, 8, 128
    T = NS * L
    last = fa_synth.make(spec(layout="BSND", B=1, QN=QN, KVN=KVN, QS=L, KVS=L, D=D, mask="causal", seed=2034))
    q = torch.zeros((T, QN, D), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((T, KVN, D), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    assert (T - L) * q.stride(0) == 2 ** 31
    q[T - L:] = dev16(last.q, "bf16")[0]
    k[T - L:] = dev16(last.k, "bf16")[0]
    v[T - L:] = dev16(last.v, "bf16")[0]
    cu = torch.arange(0, T + 1, L, dtype=torch.int32, device=DEV)
    out, lse = fa.fwd(q, k, v, layout="TND", scale=last.spec.softmax_scale, causal=True,
                      cu_seqlens_q=cu, cu_seqlens_kv=cu, return_lse=True)
    torch.cuda.synchronize()
    del q, k, v
    ref, ref_lse = oracle.attention(oracle.Problem.from_inputs(last), last.q, last.k, last.v)
    got = to_np(out[T - L:].permute(1, 0, 2)).reshape(-1, D)
    r_rows = np.ascontiguousarray(ref.transpose(0, 2, 1, 3)).reshape(-1, D)
    check(got, to_np(lse[T - L:].t()).reshape(-1), r_rows, ref_lse.reshape(-1), "packed prefill past 2^31")
    for seq in (0, NS // 2, NS - 2):
        rows = slice(seq * L, (seq + 1) * L)
        assert torch.count_nonzero(out[rows]).item() == 0, f"sequence {seq}: non-zero output"
        want = np.log(np.arange(1, L + 1, dtype=np.float64))[:, None]
        err = np.abs(to_np(lse[rows]) - want).max()
        assert err <= LSE_TOL, f"sequence {seq}: lse err {err:.3e}"
