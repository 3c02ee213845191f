"""kv_decode_attention_noalloc (the entry point for callers that cannot
allocate) against kv_decode_attention with a caller workspace: the same
kernels on the same inputs, so the outputs must agree bit for bit. Two calls
in a row, the second smaller, show that the shared scratch keeps nothing
that changes a later call; an oversized call is refused before launch."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DeviceCache, bits_tensor, i32, oracle_threads, tensor_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_quantization_paged_amd as K
    return K


def make_case(orc, seed, B, H, G, ps, layout, max_len, D=128):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, max_len + 1, size=B).astype(np.int32)
    lens[0] = max_len
    maxp = max(1, (max_len + ps - 1) // ps)
    P = B * maxp + 2
    shape = (P, ps, H, D) if layout == W.NHD else (P, H, ps, D)
    k = W.f32_to_bits(W.normal_rows(rng, shape), True)
    v = W.f32_to_bits(W.normal_rows(rng, shape), True)
    gk, gv = orc.global_scale(k, True), orc.global_scale(v, True)
    cache = W.make_cache(rng, P, ps, H, D, layout, fill="zero")
    orc.quantize_paged_cache(cache, k, v, True, gk, gv, v_sf_interleaved=False, threads=oracle_threads())
    bt = rng.permutation(P)[:B * maxp].reshape(B, maxp).astype(np.int32)
    q = W.f32_to_bits(W.normal_rows(rng, (B, H * G, D)), True)
    return dict(dev=DeviceCache(cache), bt=i32(bt), lens=i32(lens), q=bits_tensor(q, True),
                gk=torch.tensor([gk], device="cuda"), gv=torch.tensor([gv], device="cuda"), B=B, H=H, G=G, ps=ps,
                maxp=maxp, D=D)


def both(K, c, sm):
    Hq = c["H"] * c["G"]
    ref = torch.full((c["B"], Hq, c["D"]), float("nan"), dtype=torch.bfloat16, device="cuda")
    got = torch.full_like(ref, float("nan"))
    ws = torch.full((K.kv_decode_attention_workspace_size(c["B"], c["H"], Hq, c["maxp"], c["ps"], c["D"]),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    K.kv_decode_attention(c["dev"].cache, c["q"], c["bt"], c["lens"], c["gk"], c["gv"], sm, ref, ws)
    K.kv_decode_attention_noalloc(c["dev"].cache, c["q"], c["bt"], c["lens"], c["gk"], c["gv"], sm, got)
    torch.cuda.synchronize()
    return tensor_bits(ref), tensor_bits(got)


def test_noalloc_matches_workspace_call_twice(K, orc):
    sm = float(np.float32(1.0 / np.sqrt(128)))
    big = make_case(orc, 900, B=24, H=4, G=4, ps=16, layout=W.NHD, max_len=1500)
    small = make_case(orc, 901, B=5, H=2, G=8, ps=16, layout=W.HND, max_len=300)
    for name, case in (("first, larger", big), ("second, smaller", small)):
        print(f"noalloc attention: {name} call, B={case['B']} H={case['H']} G={case['G']}", flush=True)
        ref, got = both(K, case, sm)
        assert np.array_equal(ref, got), name


@pytest.mark.parametrize("D,G,layout", [(64, 20, W.NHD), (256, 4, W.HND), (128, 33, W.HND)])
def test_noalloc_head_dims_and_query_head_passes(K, orc, D, G, layout):
    """head_dim 64 and 256, and more than 16 query heads per kv head (passes
    of 16 over the one scratch array), against the workspace call"""
    sm = float(np.float32(1.0 / np.sqrt(D)))
    case = make_case(orc, 910 + D + G, B=7, H=2, G=G, ps=16, layout=layout, max_len=700, D=D)
    print(f"noalloc attention: D={D} G={G} layout={layout}", flush=True)
    ref, got = both(K, case, sm)
    assert np.array_equal(ref, got)


def test_noalloc_refuses_calls_beyond_its_scratch(K, orc):
    """partials beyond the fixed scratch give KVFP4_ESCRATCH before anything
    is queued: `out` keeps its contents (every length is 0, so even a launch
    would read no page)"""
    c = make_case(orc, 902, B=2, H=8, G=1, ps=16, layout=W.HND, max_len=40)
    B, G, cols = 4096, 16, 64
    Hq = 8 * G
    need = K.kv_decode_attention_workspace_size(B, 8, Hq, cols, 16)
    assert need > K._binding.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 3.0)
    bt = torch.zeros((B, cols), dtype=torch.int32, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(K.KVFP4Error) as err:
        K.kv_decode_attention_noalloc(c["dev"].cache, q, bt, lens, c["gk"], c["gv"], 0.1, out)
    assert err.value.status == K._binding.KVFP4_ESCRATCH
    torch.cuda.synchronize()
    assert bool(torch.all(out == 3.0))
