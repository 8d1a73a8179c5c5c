"""GPU check of ra_splitkv_decode_noalloc (the decode entry point that allocates
nothing: its partials live in the library's per-device scratch array) against
ra_splitkv_decode, which takes the partials from caller buffers. Both run the same
kernels on the same inputs, so the outputs must agree bit for bit; they are also
held to the fp64 oracle at the bf16 gates. Two calls in a row, the second smaller,
show that one call's scratch contents do not leak into the next."""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import randn_np
from gpu_util import assert_close, np64, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ra():
    import blockwise_exact_attention_block_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return m


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(torch.bfloat16).contiguous()


def one_case(ra, B, Hq, Hkv, L, D, n, seed):
    say(f"splitkv_decode_noalloc B{B} Hq{Hq} Hkv{Hkv} L{L} D{D} n{n} seed {seed}")
    q = randn_np((B, Hq, D), seed, "bf16")
    k = randn_np((B, Hkv, L, D), seed + 1, "bf16")
    v = randn_np((B, Hkv, L, D), seed + 2, "bf16")
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    ra.splitkv_decode_noalloc(dq, dk, dv, n_splits=n, out=out, lse=lse)
    _, _, o_ref_gpu, l_ref_gpu = ra.splitkv_decode(dq, dk, dv, n_splits=n)
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref_gpu), "output differs from ra_splitkv_decode"
    assert torch.equal(lse, l_ref_gpu), "LSE differs from ra_splitkv_decode"
    _, _, o_r, l_r = oracle.splitkv_decode(q, k, v, n_splits=n, scale=1 / math.sqrt(D))
    assert_close(np64(out), np64(lse), o_r, l_r, "bf16", "splitkv_decode_noalloc")


def test_noalloc_decode_two_calls_second_smaller(ra):
    one_case(ra, B=4, Hq=32, Hkv=4, L=4096, D=128, n=8, seed=7100)
    one_case(ra, B=2, Hq=16, Hkv=2, L=1000, D=64, n=4, seed=7200)


def test_noalloc_decode_rejects_partials_beyond_the_scratch(ra):
    B, Hq, Hkv, L, D, n = 32, 64, 8, 64, 128, 32      # 32*64*32*129*4 bytes = 33.8 MB > 16 MiB
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((B, Hkv, L, D), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ra.RingAttnError, match="scratch"):
        ra.splitkv_decode_noalloc(q, k, k, n_splits=n)
