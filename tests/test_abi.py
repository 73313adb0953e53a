"""The C-ABI library loads, exports every entry point include/fa.h declares, and
rejects invalid calls before touching the GPU (these tests make no compute call)."""
import ctypes
import os
import re

import pytest

import split_kv_decode_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:fa_status|const char \*)\s*(fa_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return fa.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(fa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def params(**kw):
    base = dict(batch=1, num_heads=32, q_seq=1, kv_seq=131072, head_dim=128, layout="BNSD",
                dtype="bf16", scale=0.088)
    base.update(kw)
    b = base.pop("batch"); n = base.pop("num_heads"); qs = base.pop("q_seq")
    kvs = base.pop("kv_seq"); d = base.pop("head_dim")
    return fa.make_params(b, n, qs, kvs, d, **base)


FAKE = 1 << 20  # a 16-byte-aligned non-null address; never dereferenced (validation fails first)


@pytest.mark.parametrize("kw,status,text", [
    (dict(num_heads=6, num_kv_heads=4), fa.FA_ERR_PARAM_INVALID, "multiple"),
    (dict(head_dim=192), fa.FA_ERR_UNSUPPORTED, "not built"),
    (dict(head_dim=100), fa.FA_ERR_PARAM_INVALID, "head_dim"),
    (dict(batch=0), fa.FA_ERR_PARAM_INVALID, "batch"),
    (dict(q_seq=0), fa.FA_ERR_PARAM_INVALID, "q_seq"),
    (dict(kv_seq=0), fa.FA_ERR_PARAM_INVALID, "kv_seq"),
    (dict(scale=float("nan")), fa.FA_ERR_PARAM_INVALID, "scale"),
    (dict(mask_mode="bool"), fa.FA_ERR_NULLPTR, "mask"),
    (dict(mask=FAKE), fa.FA_ERR_PARAM_INVALID, "not BOOL"),
    (dict(layout=7), fa.FA_ERR_PARAM_INVALID, "layout"),
    (dict(dtype=5), fa.FA_ERR_PARAM_INVALID, "dtype"),
    (dict(mask_mode="window", win_left=-2), fa.FA_ERR_PARAM_INVALID, "win_left"),
    (dict(mask_mode="window", win_right=-7), fa.FA_ERR_PARAM_INVALID, "win_right"),
    (dict(mask_mode=9), fa.FA_ERR_PARAM_INVALID, "mask_mode"),
])
def test_fwd_rejects_invalid_parameters(lib, kw, status, text):
    p = params(**kw)
    st = lib.fa_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, 0, None)
    assert st == status
    assert text in fa.fa_last_error()


def test_fwd_rejects_null_and_misaligned_tensors(lib):
    p = params(q_seq=16)
    assert lib.fa_fwd(ctypes.byref(p), None, FAKE, FAKE, FAKE, None, None, 0, None) == fa.FA_ERR_NULLPTR
    assert lib.fa_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, None, 0, None) == fa.FA_ERR_NULLPTR
    assert lib.fa_fwd(ctypes.byref(p), FAKE + 2, FAKE, FAKE, FAKE, None, None, 0, None) == fa.FA_ERR_PARAM_INVALID
    assert lib.fa_fwd(None, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == fa.FA_ERR_NULLPTR


def test_decode_entry_points_validate(lib):
    # several query positions: built for head_dim 64 / 128 (head_dim 256 is refused
    # before anything is launched)
    p = params(q_seq=2, head_dim=256)
    st = lib.fa_decode_splitkv(ctypes.byref(p), 32, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == fa.FA_ERR_UNSUPPORTED and "several query positions" in fa.fa_last_error()
    # more than 512 (query head, position) rows per KV head
    p = params(q_seq=17, num_heads=32, num_kv_heads=1)
    st = lib.fa_decode_splitkv(ctypes.byref(p), 32, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == fa.FA_ERR_UNSUPPORTED
    p = params()
    st = lib.fa_decode_splitkv(ctypes.byref(p), 31, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == fa.FA_ERR_PARAM_INVALID and "cover" in fa.fa_last_error()
    st = lib.fa_decode_splitkv(ctypes.byref(p), 32, 4000, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == fa.FA_ERR_PARAM_INVALID and "multiple of 64" in fa.fa_last_error()
    st = lib.fa_decode_splitkv(ctypes.byref(p), 32, 4096, FAKE, FAKE, FAKE, None, FAKE, FAKE, None)
    assert st == fa.FA_ERR_NULLPTR
    pm = params(mask_mode="causal", head_dim=256)
    st = lib.fa_decode_splitkv(ctypes.byref(pm), 32, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == fa.FA_ERR_UNSUPPORTED
    # o_part is read and written as 16-byte vectors
    st = lib.fa_decode_splitkv(ctypes.byref(p), 32, 4096, FAKE, FAKE, FAKE, FAKE + 4, FAKE, FAKE, None)
    assert st == fa.FA_ERR_PARAM_INVALID and "16-byte" in fa.fa_last_error()
    st = lib.fa_combine(ctypes.byref(p), 32, FAKE + 4, FAKE, FAKE, FAKE, None, None)
    assert st == fa.FA_ERR_PARAM_INVALID and "16-byte" in fa.fa_last_error()
    st = lib.fa_combine(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == fa.FA_ERR_PARAM_INVALID
    st = lib.fa_combine(ctypes.byref(p), 4, FAKE, FAKE, FAKE, None, None, None)
    assert st == fa.FA_ERR_NULLPTR


@pytest.mark.parametrize("kw,cus,splits,chunk", [
    (dict(), 256, 32, 4096),                                               # 128K decode, B=1, N=32
    (dict(batch=8, num_heads=32, num_kv_heads=8, kv_seq=4096, layout="BSND"), 256, 16, 256),
    (dict(kv_seq=100), 256, 1, 128),                                       # tiny cache: one split
    (dict(batch=64, num_heads=32, kv_seq=1024), 256, 1, 1024),             # plenty of units
    (dict(kv_seq=131072), 80, 10, 13120),                                  # fewer CUs
])
def test_split_plan(lib, kw, cus, splits, chunk):
    p = params(**kw)
    sp, ch, ws = fa.fa_splitkv_plan(p, num_cus=cus)
    assert (sp, ch) == (splits, chunk)
    assert ch % 64 == 0 and sp * ch >= p.kv_seq
    rows = p.batch * p.num_heads * sp
    assert ws >= rows * (p.head_dim + 2) * 4


def test_split_plan_honours_chunk_hint(lib):
    p = params()
    assert fa.fa_splitkv_plan(p, num_cus=256, chunk_hint=1024)[:2] == (128, 1024)
    with pytest.raises(fa.FaError):
        fa.fa_splitkv_plan(p, num_cus=256, chunk_hint=1000)


def test_prefill_needs_no_workspace(lib):
    assert fa.fa_workspace_size(params(q_seq=128, batch=8)) == 0
    # head_dim 256 with a mask: the prefill kernel, no workspace
    assert fa.fa_workspace_size(params(q_seq=1, mask_mode="causal", head_dim=256)) == 0


def test_split_path_routing_and_workspace(lib):
    # masked decode, decode with used lengths, and a few query positions against a
    # long cache take the split-KV path: partials for every (b, n1, i) row
    for kw in (dict(q_seq=1, mask_mode="causal"), dict(q_seq=1, seqused_q=FAKE),
               dict(q_seq=8, num_heads=32, num_kv_heads=8, kv_seq=65536),
               dict(q_seq=1, mask_mode="window", win_left=100, win_right=0)):
        p = params(**kw)
        sp, ch, ws = fa.fa_splitkv_plan(p, num_cus=256)
        assert sp > 1 and sp * ch >= p.kv_seq
        rows = p.batch * p.num_heads * p.q_seq
        assert ws >= rows * sp * (p.head_dim + 2) * 4
        assert fa.fa_workspace_size(p) > 0
    # row groups count as units of the plan: 8 heads x 4 positions of one KV head
    # fill one 32-row tile, x 8 positions two tiles, which need half the splits
    one = fa.fa_splitkv_plan(params(q_seq=4, num_heads=8, num_kv_heads=1, kv_seq=1 << 20), num_cus=256)
    two = fa.fa_splitkv_plan(params(q_seq=8, num_heads=8, num_kv_heads=1, kv_seq=1 << 20), num_cus=256)
    assert two[0] < one[0] and two[0] * 2 >= one[0] - 2
    # enough query tiles to fill the CUs: the prefill kernel (no workspace)
    assert fa.fa_workspace_size(params(q_seq=8, batch=64, num_heads=32, kv_seq=65536)) == 0


def test_window_bounds_and_scale_validated(lib):
    # developer guide 1.5: without the window mode both bounds are -1
    for kw in (dict(win_left=0), dict(win_right=5), dict(mask_mode="causal", win_left=3)):
        p = params(**kw)
        assert lib.fa_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == fa.FA_ERR_PARAM_INVALID
        assert "-1 outside the window mode" in fa.fa_last_error()
    # scale * log2(e) must stay finite in fp32
    p = params(scale=1e39)
    assert lib.fa_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == fa.FA_ERR_PARAM_INVALID
    assert "scale" in fa.fa_last_error()
    # cu_seqlens stay TND-only; seqused_q is accepted in every layout
    p = params(cu_seqlens_q=FAKE)
    assert lib.fa_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == fa.FA_ERR_PARAM_INVALID
    assert fa.fa_workspace_size(params(q_seq=64, batch=64, seqused_q=FAKE)) == 0


def test_fused_plan_stays_within_the_fused_merge(lib):
    # one batch, one KV head: the matrix-core plan asks for hundreds of splits, the
    # fused launch takes at most 256 (its chunk grows instead)
    p = params(num_heads=8, num_kv_heads=1, kv_seq=131072)
    assert fa.fa_splitkv_plan(p, num_cus=256)[0] > 256
    sp, ch, ws = fa.fa_decode_fused_plan(p, num_cus=256)
    assert 1 <= sp <= 256 and sp * ch >= p.kv_seq and ch % 64 == 0
    assert ws >= p.batch * p.num_heads * sp * (p.head_dim + 2) * 4
    sp, ch, _ = fa.fa_decode_fused_plan(params(), num_cus=256)
    assert sp <= 256 and sp * ch >= 131072
    with pytest.raises(fa.FaError):
        fa.fa_decode_fused_plan(params(mask_mode="causal"), num_cus=256)


# ---------------------------------------------------------------- paged KV cache

def paged(**kw):
    base = dict(kv_layout="PA_BBND", block_table=FAKE, block_size=128, max_blocks_per_seq=1024,
                num_blocks=1024, actual_seq_lengths=FAKE)
    base.update(kw)
    return params(**base)


@pytest.mark.parametrize("kw,status,text", [
    (dict(kv_layout=9), fa.FA_ERR_PARAM_INVALID, "kv_layout"),
    (dict(block_table=None), fa.FA_ERR_NULLPTR, "block_table"),
    (dict(actual_seq_lengths=None), fa.FA_ERR_NULLPTR, "actual_seq_lengths"),
    (dict(block_size=8), fa.FA_ERR_PARAM_INVALID, "block_size"),
    (dict(block_size=40), fa.FA_ERR_PARAM_INVALID, "block_size"),
    (dict(block_size=2048), fa.FA_ERR_PARAM_INVALID, "block_size"),
    (dict(max_blocks_per_seq=0), fa.FA_ERR_PARAM_INVALID, "max_blocks_per_seq"),
    (dict(num_blocks=0), fa.FA_ERR_PARAM_INVALID, "num_blocks"),
    (dict(max_blocks_per_seq=1023), fa.FA_ERR_PARAM_INVALID, "exceeds"),    # 1023*128 < 131072
    (dict(q_seq=16, head_dim=256), fa.FA_ERR_UNSUPPORTED, "split-KV paths"),
    (dict(mask_mode="causal", head_dim=256), fa.FA_ERR_UNSUPPORTED, "split-KV paths"),
    (dict(q_seq=600), fa.FA_ERR_UNSUPPORTED, "split-KV paths"),
    (dict(kv_layout="contiguous"), fa.FA_ERR_PARAM_INVALID, "contiguous"),  # table without paging
])
def test_paged_params_validated(lib, kw, status, text):
    p = paged(**kw)
    st = lib.fa_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert st == status
    assert text in fa.fa_last_error()


def test_paged_plan_caps_chunk_to_the_lds_table(lib):
    # 64 batches x 16 KV heads fill the chip without splitting, so the contiguous
    # plan takes the whole cache as one chunk; with 16-token blocks a chunk may
    # span at most 1016 blocks.
    kw = dict(batch=64, num_heads=16, kv_seq=40000)
    assert fa.fa_splitkv_plan(params(**kw), num_cus=256)[:2] == (1, 40000)
    sp, ch, _ = fa.fa_splitkv_plan(paged(block_size=16, max_blocks_per_seq=2500, **kw), num_cus=256)
    assert (sp, ch) == (3, 1016 * 16)
    p = paged(block_size=16, max_blocks_per_seq=2500, **kw)
    with pytest.raises(fa.FaError, match="exceeds"):
        fa.fa_splitkv_plan(p, num_cus=256, chunk_hint=1024 * 16)
    st = lib.fa_decode_splitkv(ctypes.byref(p), 2, 1024 * 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == fa.FA_ERR_PARAM_INVALID and "exceeds" in fa.fa_last_error()


# ---------------------------------------------------------------- packed layout (TND)

def tnd(**kw):
    base = dict(batch=4, q_seq=1000, kv_seq=1200, layout="TND", cu_seqlens_q=FAKE,
                cu_seqlens_kv=FAKE, mask_mode="causal")
    base.update(kw)
    return params(**base)


@pytest.mark.parametrize("kw,status,text", [
    (dict(cu_seqlens_q=None), fa.FA_ERR_NULLPTR, "cu_seqlens"),
    (dict(cu_seqlens_kv=None), fa.FA_ERR_NULLPTR, "cu_seqlens"),
    (dict(batch=16384), fa.FA_ERR_PARAM_INVALID, "at most"),
    (dict(mask_mode="bool", mask=FAKE, mask_stride=(0, 0, 1, 1)), fa.FA_ERR_UNSUPPORTED, "boolean"),
    (dict(kv_layout="PA_BBND", block_table=FAKE, block_size=16, max_blocks_per_seq=100,
          num_blocks=100, actual_seq_lengths=FAKE), fa.FA_ERR_UNSUPPORTED, "paged"),
    (dict(layout="BSND"), fa.FA_ERR_PARAM_INVALID, "TND layout only"),
])
def test_tnd_params_validated(lib, kw, status, text):
    p = tnd(**kw)
    st = lib.fa_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert st == status
    assert text in fa.fa_last_error()


def test_bool_mask_summary_workspace(lib):
    # A staged boolean mask (unit key stride, 16-byte multiples) asks for its
    # per-tile summary: one 32-bit word per 16 KV tiles of 64 keys, per mask
    # slice (broadcast axes count once) and 128-row query tile.
    bcast = params(batch=2, q_seq=4096, kv_seq=4096, mask_mode="bool", mask=FAKE,
                   mask_stride=(0, 0, 4096, 1))
    assert fa.fa_workspace_size(bcast) == 256 * (((32 * 4 * 4) + 255) // 256)
    per_bn = params(batch=2, num_heads=4, q_seq=1000, kv_seq=1040, mask_mode="bool", mask=FAKE,
                    mask_stride=(4 * 1000 * 1040, 1000 * 1040, 1040, 1))
    # 8 slices x ceil(1000/128) = 8 q tiles x ceil(ceil(1040/64)/16) = 2 words
    assert fa.fa_workspace_size(per_bn) == ((8 * 8 * 2 * 4) + 255) // 256 * 256
    # element-wise masks (key stride != 1) take no workspace
    assert fa.fa_workspace_size(params(q_seq=256, kv_seq=256, mask_mode="bool", mask=FAKE,
                                       mask_stride=(0, 0, 1, 256))) == 0
    # a misaligned or short workspace is refused before anything runs
    st = lib.fa_fwd(ctypes.byref(bcast), FAKE, FAKE, FAKE, FAKE, None, FAKE + 16, 1 << 20, None)
    assert st == fa.FA_ERR_PARAM_INVALID and "aligned" in fa.fa_last_error()
    st = lib.fa_fwd(ctypes.byref(bcast), FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, None)
    assert st == fa.FA_ERR_PARAM_INVALID and "too small" in fa.fa_last_error()


def _partial_bytes(rows, splits, D, units):
    r256 = lambda x: (x + 255) // 256 * 256
    return r256(rows * splits * D * 4) + 2 * r256(rows * splits * 4) + r256(units * 4)


def test_decode_workspace_fixed_and_balanced_plans(lib):
    """Host planning without a device (the planner falls back to 256 CUs and no
    occupancy answer): grouped heads with per-batch lengths take the
    length-balanced plan, whose slots per row are min(ceil(kv_seq/64),
    ceil(target/KV_N) + 1) with target = 2 workgroups x 256 CUs - B*KV_N (so the
    grid of target + B*KV_N workgroups is one resident round)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("the expected sizes assume the planner's no-device fallbacks")
    base = dict(batch=1, num_heads=32, num_kv_heads=8, q_seq=1, kv_seq=4096)
    fixed = fa.fa_workspace_size(params(**base))
    # fixed plan: 8 units, 4 x 256 target -> 128 splits wanted -> 256-token chunks -> 16 splits
    assert fixed == _partial_bytes(32, 16, 128, 8)
    bal = fa.fa_workspace_size(params(actual_seq_lengths=FAKE, **base))
    assert bal == _partial_bytes(32, min(4096 // 64, -(-(512 - 8) // 8) + 1), 128, 8)
    # B = 8: target 512 - 64 = 448 -> 57 slots per row
    b8 = dict(base, batch=8)
    assert fa.fa_workspace_size(params(actual_seq_lengths=FAKE, **b8)) == _partial_bytes(8 * 32, 448 // 8 + 1, 128, 64)
    # vector path (g = 2) keeps the fixed plan with or without lengths
    g2 = dict(base, num_kv_heads=16)
    assert fa.fa_workspace_size(params(actual_seq_lengths=FAKE, **g2)) == fa.fa_workspace_size(params(**g2))


def test_tnd_workspace(lib):
    p = tnd()
    # one (sequence, tile) pair per 128-row tile: ceil(1000/128) + 4 + 1 entries of 8 bytes
    assert fa.fa_workspace_size(p) == 256
    assert fa.fa_workspace_size(tnd(q_seq=1 << 20, batch=1000)) == ((8192 + 1001) * 8 + 255) // 256 * 256
    st = lib.fa_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, 0, None)
    assert st == fa.FA_ERR_NULLPTR and "workspace" in fa.fa_last_error()
    st = lib.fa_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, None)
    assert st == fa.FA_ERR_PARAM_INVALID and "too small" in fa.fa_last_error()
    pd = tnd(q_seq=4, mask_mode="none")
    st = lib.fa_decode_splitkv(ctypes.byref(pd), 1, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == fa.FA_ERR_UNSUPPORTED


def test_fused_decode_validates(lib):
    p = params()
    st = lib.fa_decode_fused(ctypes.byref(p), 512, 256, FAKE, FAKE, FAKE, FAKE, 1 << 30, FAKE, None, None)
    assert st == fa.FA_ERR_PARAM_INVALID and "1 to 256" in fa.fa_last_error()
    st = lib.fa_decode_fused(ctypes.byref(p), 32, 4096, FAKE, FAKE, FAKE, None, 0, FAKE, None, None)
    assert st == fa.FA_ERR_NULLPTR and "workspace" in fa.fa_last_error()
    st = lib.fa_decode_fused(ctypes.byref(p), 32, 4096, FAKE, FAKE, FAKE, FAKE, 1024, FAKE, None, None)
    assert st == fa.FA_ERR_PARAM_INVALID and "too small" in fa.fa_last_error()
    st = lib.fa_decode_fused(ctypes.byref(p), 16, 4096, FAKE, FAKE, FAKE, FAKE, 1 << 30, FAKE, None, None)
    assert st == fa.FA_ERR_PARAM_INVALID and "cover" in fa.fa_last_error()
    pq = params(q_seq=4)
    st = lib.fa_decode_fused(ctypes.byref(pq), 32, 4096, FAKE, FAKE, FAKE, FAKE, 1 << 30, FAKE, None, None)
    assert st == fa.FA_ERR_UNSUPPORTED


def test_noalloc_rejects_calls_beyond_its_scratch(lib):
    # the work list of a packed batch of 2^29 query tokens needs far more than the
    # 16 MiB of scratch fa_fwd_noalloc holds: rejected before any launch (the
    # pointers are fake and never read)
    p = params(batch=4, num_heads=2, q_seq=1 << 29, kv_seq=1 << 29, head_dim=64, layout="TND",
               cu_seqlens_q=FAKE, cu_seqlens_kv=FAKE)
    assert fa.fa_workspace_size(p) > (16 << 20)
    st = lib.fa_fwd_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == fa.FA_ERR_PARAM_INVALID
    assert "scratch" in fa.fa_last_error()
    # validation errors come first, as for fa_fwd
    bad = params(head_dim=100)
    assert lib.fa_fwd_noalloc(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, None, None) == fa.FA_ERR_PARAM_INVALID


def test_params_keep_the_tensors_they_point_to_alive():
    """FaParams holds raw addresses; the tensors behind them must outlive a
    temporary passed straight into params_for (else the allocator hands their
    memory to the next tensor and the kernels read that instead)."""
    import gc
    import weakref
    torch = pytest.importorskip("torch")
    q = torch.zeros((2, 1, 4, 64), dtype=torch.bfloat16)
    k = torch.zeros((8, 16, 2, 64), dtype=torch.bfloat16)
    refs = []

    def tmp(*shape):
        t = torch.zeros(shape, dtype=torch.int32)
        refs.append(weakref.ref(t))
        return t

    p = fa.params_for(q, k, layout="BSND", actual_seq_lengths=tmp(2), kv_layout="PA_BBND",
                      block_table=tmp(2, 4), seqused_q=tmp(2))
    gc.collect()
    assert all(r() is not None for r in refs)
    assert p.block_table == refs[1]().data_ptr()
    del p
    gc.collect()
    assert all(r() is None for r in refs)


def test_describe_names_path_kernels_and_plan(lib):
    """fa_describe: the line FA_LOG prints, for one shape of each path; its
    workspace figure is fa_workspace_size's."""
    F = 1 << 20  # fake device address: nothing is read
    cases = [
        (dict(batch=2, num_heads=32, q_seq=4096, kv_seq=4096, head_dim=128, layout="BSND"),
         ["path=prefill", "prefill_il_kernel<BF16,128,0>", "rows=256",
          "workgroups=256 (persistent, over 1024 units)"]),
        (dict(batch=2, num_heads=32, q_seq=4096, kv_seq=4096, head_dim=128, layout="BSND", mask_mode="window",
              win_left=1024, win_right=0),
         ["prefill_il_kernel<BF16,128,4>", "workgroups=256 (persistent, over 1024 units)"]),
        (dict(batch=2, num_heads=32, q_seq=4096, kv_seq=4096, head_dim=128, layout="BSND", mask_mode="causal"),
         ["prefill_il_kernel<BF16,128,1>", "workgroups=256 (persistent, over 1024 units)"]),
        (dict(batch=2, num_heads=32, q_seq=4096, kv_seq=4096, head_dim=128, layout="BSND", mask_mode="causal",
              actual_seq_lengths=F),
         ["prefill_il_kernel<BF16,128,1>", "workgroups=256 (persistent, over 1024 units)"]),
        (dict(batch=2, num_heads=16, q_seq=4096, kv_seq=4096, head_dim=256),
         ["prefill_il_kernel<BF16,256,0>", "workgroups=1024 "]),
        (dict(batch=1, num_heads=32, q_seq=2048, kv_seq=2048, head_dim=128),
         ["prefill_il_kernel<BF16,128,0>", "workgroups=256 "]),
        (dict(batch=2, num_heads=16, q_seq=4096, kv_seq=4096, head_dim=256, mask_mode="causal", dtype="f16"),
         ["prefill_il_kernel<F16,256,1>", "rows=128", "workgroups=1024"]),
        (dict(batch=2, num_heads=4, q_seq=300, kv_seq=320, head_dim=128, mask_mode="bool", mask=F,
              mask_stride=(4 * 300 * 320, 300 * 320, 320, 1)),
         ["pre=mask_summary_kernel", "prefill_il_kernel<BF16,128,3>"]),
        (dict(batch=2, num_heads=4, q_seq=300, kv_seq=320, head_dim=128, mask_mode="bool", mask=F + 1,
              mask_stride=(4 * 300 * 320, 300 * 320, 320, 1)),
         ["prefill_kernel<BF16,128,2>", "mask=element-wise", "rows=128"]),
        (dict(batch=2, num_heads=4, q_seq=300, kv_seq=320, head_dim=128, mask_mode="bool", mask=F + 4,
              mask_stride=(4 * 300 * 320, 300 * 320, 320, 1)),
         ["prefill_il_kernel<BF16,128,2>", "mask=4-byte runs", "rows=256"]),
        (dict(batch=1, num_heads=32, q_seq=1, kv_seq=131072, head_dim=128),
         ["path=decode", "stage1=decode_stage1_kernel", "then combine_kernel"]),
        (dict(batch=8, num_heads=32, num_kv_heads=8, q_seq=1, kv_seq=4096, head_dim=128, layout="BSND",
              actual_seq_lengths=F),
         ["path=decode", "stage1=decode_mfma_kernel", "length-balanced", "then combine_kernel"]),
        (dict(batch=1, num_heads=32, num_kv_heads=8, q_seq=8, kv_seq=65536, head_dim=128, layout="BSND"),
         ["path=general-split", "stage1=decode_mfma_kernel", "then combine_kernel"]),
        (dict(batch=16, num_heads=32, num_kv_heads=8, q_seq=55635, kv_seq=55635, head_dim=128, layout="TND",
              mask_mode="causal", cu_seqlens_q=F, cu_seqlens_kv=F),
         ["path=prefill", "pre=varlen_schedule_kernel", "prefill_il_kernel<BF16,128,1>", "32 heads",
          "workgroups=256 (persistent, over the work list of <= "]),
        (dict(batch=2, num_heads=4, q_seq=300, kv_seq=300, head_dim=128, layout="TND", mask_mode="causal",
              cu_seqlens_q=F, cu_seqlens_kv=F),
         ["prefill_il_kernel<BF16,128,1>", "workgroups=(work list of <= 6 items) x 4 heads"]),
    ]
    for kw, want in cases:
        p = fa.make_params(**kw)
        d = fa.fa_describe(p)
        for w in want:
            assert w in d, (w, d)
        assert d.endswith(f"workspace={fa.fa_workspace_size(p)}"), d
    with pytest.raises(fa.FaError) as e:
        fa.fa_describe(fa.make_params(1, 3, 1, 64, 128, num_kv_heads=2))
    assert e.value.status == fa.FA_ERR_PARAM_INVALID
    p = fa.make_params(1, 2, 1, 64, 128)
    assert lib.fa_describe(ctypes.byref(p), None, 16) == fa.FA_ERR_NULLPTR
    buf = ctypes.create_string_buffer(12)  # longer text is cut, NUL-terminated
    assert lib.fa_describe(ctypes.byref(p), buf, 12) == fa.FA_OK and len(buf.value) == 11


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="launches with fake addresses: CPU-only hosts")
def test_fa_log_prints_the_plan_before_launching():
    """FA_LOG=1: fa_fwd prints fa_describe's line to stderr before it launches (here the
    launch then fails: no GPU); without FA_LOG it prints nothing."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import split_kv_decode_amd as fa\n"
            "p = fa.make_params(2, 32, 256, 256, 128, layout='BSND')\n"
            "try:\n    fa.fa_fwd(p, 1 << 20, 1 << 20, 1 << 20, 1 << 20)\n"
            "except fa.FaError as e:\n    print(e.status)\n") % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for env_val, expect in (("1", True), ("0", False), (None, False)):
        env = dict(os.environ)
        env.pop("FA_LOG", None)
        if env_val is not None:
            env["FA_LOG"] = env_val
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
        logged = [ln for ln in r.stderr.splitlines() if ln.startswith("fa_fwd: ")]
        assert bool(logged) == expect, (env_val, r.stderr)
        if expect:
            assert "path=prefill kernel=prefill_il_kernel<BF16,128,0>" in logged[0]


def test_short_query_routing_by_visible_keys(lib):
    """A few query positions split the KV axis only when the prefill would leave CUs idle
    and a row sees enough keys (640 at head_dim 128, 1024 at 64; the causal mask is
    top-left)."""
    def path(**kw):
        return fa.fa_describe(fa.make_params(**kw)).split(" -> ")[1].split()[0]
    assert path(batch=1, num_heads=2, q_seq=128, kv_seq=128, head_dim=64) == "path=prefill"
    assert path(batch=1, num_heads=8, q_seq=64, kv_seq=4096, head_dim=128) == "path=general-split"
    assert path(batch=4, num_heads=8, q_seq=32, kv_seq=2048, head_dim=64, mask_mode="causal") == "path=prefill"
    assert path(batch=2, num_heads=16, num_kv_heads=4, q_seq=128, kv_seq=16384, head_dim=128,
                layout="BSND") == "path=general-split"                       # 512 rows per KV head
    assert path(batch=1, num_heads=8, q_seq=64, kv_seq=8192, head_dim=128, mask_mode="window",
                win_left=4000, win_right=0) == "path=prefill"               # rows see <= 64 keys
    assert path(batch=1, num_heads=8, q_seq=64, kv_seq=8192, head_dim=128, mask_mode="window",
                win_left=-1, win_right=2000) == "path=general-split"
    assert path(batch=1, num_heads=8, q_seq=64, kv_seq=8192, head_dim=128,
                num_kv_heads=1, mask_mode="causal") == "path=prefill"
    assert path(batch=1, num_heads=32, num_kv_heads=1, q_seq=17, kv_seq=8192, head_dim=128) == "path=prefill"  # 544 rows
    # a window bound near the int64 limit counts as unbounded reach (no overflow)
    assert path(batch=1, num_heads=8, q_seq=64, kv_seq=4096, head_dim=128, mask_mode="window",
                win_left=-1, win_right=(1 << 63) - 1) == "path=general-split"
    # the threshold: 640 visible keys at head_dim 128, 1024 at 64
    assert path(batch=1, num_heads=8, q_seq=64, kv_seq=768, head_dim=128) == "path=general-split"
    assert path(batch=1, num_heads=8, q_seq=64, kv_seq=512, head_dim=128) == "path=prefill"
    assert path(batch=2, num_heads=16, q_seq=100, kv_seq=768, head_dim=64) == "path=prefill"
    assert path(batch=2, num_heads=16, q_seq=100, kv_seq=1024, head_dim=64) == "path=general-split"
