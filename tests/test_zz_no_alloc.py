"""fa_fwd_noalloc (the entry point that allocates nothing) against fa_fwd.

Both run the same kernels with the same plan, so their outputs must be
bit-identical: fa_fwd with a torch workspace, fa_fwd_noalloc with the scratch
array the library holds per GPU.  Every case makes two calls in a row, the
second on a smaller input, so the second call reads a scratch that still holds
the first call's contents.
"""
import numpy as np
import pytest

import fa_synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

import split_kv_decode_amd as fa  # noqa: E402

DEV = torch.device("cuda:0")


def dev16(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def both(spec, causal=False):
    inp = fa_synth.make(spec)
    s = inp.spec
    q, k, v = (dev16(x, s.dtype) for x in (inp.q, inp.k, inp.v))
    lens = None if inp.lens is None else torch.from_numpy(inp.lens).to(DEV)
    p = fa.params_for(q, k, layout=s.layout, scale=s.softmax_scale, actual_seq_lengths=lens, causal=causal)
    nbytes = fa.fa_workspace_size(p)
    ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=DEV)
    out_a, lse_a = torch.empty_like(q), torch.empty((s.B, s.QN, s.QS), dtype=torch.float32, device=DEV)
    out_b, lse_b = torch.full_like(q, float("nan")), torch.full_like(lse_a, float("nan"))
    stream = torch.cuda.current_stream()
    fa.fa_fwd(p, q, k, v, out_a, lse_a, ws if nbytes else None, nbytes, stream)
    fa.fa_fwd_noalloc(p, q, k, v, out_b, lse_b, stream)
    torch.cuda.synchronize()
    return nbytes, out_a, lse_a, out_b, lse_b


def assert_same(a, b, what):
    ta, tb = a.view(torch.int16) if a.dtype != torch.float32 else a.view(torch.int32), \
        b.view(torch.int16) if b.dtype != torch.float32 else b.view(torch.int32)
    assert torch.equal(ta, tb), f"{what}: fa_fwd_noalloc differs from fa_fwd"


def spec(**kw):
    base = dict(layout="BNSD", B=1, QN=2, KVN=2, QS=1, KVS=64, D=128, dtype="bf16", seed=1)
    base.update(kw)
    return fa_synth.Spec("noalloc", base.pop("layout"), base.pop("B"), base.pop("QN"), base.pop("KVN"),
                         base.pop("QS"), base.pop("KVS"), base.pop("D"), base.pop("dtype"), **base)


@pytest.mark.parametrize("first,second", [
    # split-KV decode (partials in the scratch): the long cache, then a short ragged batch
    (dict(B=1, QN=32, KVN=32, KVS=131072, seed=11),
     dict(B=3, QN=8, KVN=2, KVS=1000, lens=(1, 1000), seed=12, layout="BSND")),
    # matrix-core decode with the length-balanced plan, then a smaller one
    (dict(B=8, QN=32, KVN=8, KVS=4096, lens=(1, 4096), seed=13, layout="BSND"),
     dict(B=2, QN=16, KVN=4, KVS=3000, lens=(1, 3000), D=64, dtype="f16", seed=14)),
])
def test_noalloc_decode_matches_fa_fwd_twice(first, second):
    for i, kw in enumerate((first, second)):
        nbytes, out_a, lse_a, out_b, lse_b = both(spec(**kw))
        assert nbytes > 0, "the case should need scratch"
        assert_same(out_a, out_b, f"call {i} out")
        assert_same(lse_a, lse_b, f"call {i} lse")


def test_noalloc_prefill_matches_fa_fwd_twice():
    for i, kw in enumerate((dict(B=1, QN=4, KVN=2, QS=700, KVS=900, seed=15),
                            dict(B=1, QN=2, KVN=1, QS=130, KVS=200, seed=16))):
        nbytes, out_a, lse_a, out_b, lse_b = both(spec(**kw), causal=True)
        assert_same(out_a, out_b, f"call {i} out")
        assert_same(lse_a, lse_b, f"call {i} lse")
