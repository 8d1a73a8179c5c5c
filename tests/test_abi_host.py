"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports every
entry point include/ringattn.h declares, reports its ABI version, computes the ring
schedule on the host, and rejects invalid arguments before touching a device."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ringattn.h")


@pytest.fixture(scope="module")
def ra():
    import blockwise_exact_attention_block_amd as ra_mod
    if not os.path.exists(ra_mod.library_path()):
        from blockwise_exact_attention_block_amd import build
        build.build()
    ra_mod.load_library()
    return ra_mod


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for name in ("ra_ring_attn_fwd", "ra_ring_attn_fwd_striped", "ra_block_attn_step", "ra_lse_merge",
                 "ra_splitkv_decode"):
        assert name in syms


def test_library_exports_every_declared_symbol(ra):
    lib = ctypes.CDLL(ra.library_path())
    missing = [s for s in declared_symbols() if not hasattr(lib, s)]
    assert not missing, missing


def test_abi_version(ra):
    assert ra.abi_version() == 4


@pytest.mark.parametrize("P", [1, 2, 4, 8, 13])
@pytest.mark.parametrize("causal", [False, True])
def test_schedule_matches_oracle(ra, P, causal):
    for i in range(P):
        assert ra.ring_schedule(P, i, causal) == oracle.ring_schedule(P, i, causal)


@pytest.mark.parametrize("P", [1, 2, 4, 8, 13])
@pytest.mark.parametrize("causal", [False, True])
def test_striped_schedule_matches_oracle(ra, P, causal):
    for i in range(P):
        assert ra.ring_schedule(P, i, causal, "striped") == oracle.ring_schedule(P, i, causal, "striped")


def test_schedule_rejects_bad_arguments(ra):
    lib = ra.load_library()
    kv = (ctypes.c_int * 4)()
    kind = (ctypes.c_int * 4)()
    assert lib.ra_ring_schedule(0, 0, 1, kv, kind) == -1
    assert lib.ra_ring_schedule(4, 4, 1, kv, kind) == -1
    assert lib.ra_ring_schedule(4, -1, 1, kv, kind) == -1
    assert lib.ra_ring_schedule(4, 0, 1, None, kind) == -1
    assert b"ra_ring_schedule" in lib.ra_last_error()
    assert lib.ra_ring_schedule_striped(4, 4, 1, kv, kind) == -1
    assert b"ra_ring_schedule_striped" in lib.ra_last_error()
    with pytest.raises(ra.RingAttnError):
        ra.ring_schedule(4, 0, True, "zigzag")


FAKE = 1 << 20   # non-null, 16-byte aligned; never dereferenced: validation fails first


def test_ring_fwd_validation(ra):
    lib = ra.load_library()
    args = dict(dtype=1, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=8, Hkv=8, Sp=64, P=4, q_part0=0,
                nq=4, Dqk=128, Dv=128, scale=0.088, causal=1, stream=None)

    for fn in (lib.ra_ring_attn_fwd, lib.ra_ring_attn_fwd_striped):
        def call(**kw):
            a = dict(args, **kw)
            return fn(*a.values())
        check_ring_validation(lib, call)


def check_ring_validation(lib, call):

    assert call(q=None) == 1
    assert call(B=0) == 1
    assert call(Hkv=3) == 1                      # 8 % 3 != 0
    assert call(q_part0=2, nq=3) == 1           # partitions 2..4 outside a ring of 4
    assert call(scale=float("nan")) == 1
    assert call(scale=0.0) == 1
    assert call(q=FAKE + 2) == 1                # misaligned
    assert call(dtype=7) == 1
    assert call(Dqk=96, Dv=96) == 2             # no kernel for that head dim
    assert call(dtype=0, Dqk=192, Dv=128) == 2  # fp32 path has no 192
    assert call(Sp=1 << 24, P=8) == 2           # per-head slab past 2^31 bytes
    assert b"" != lib.ra_last_error()


def test_step_merge_decode_validation(ra):
    lib = ra.load_library()
    # block step: Sq <= 0, negative positions
    assert lib.ra_block_attn_step(1, FAKE, 0, 0, FAKE, FAKE, 0, 64, 1, 2, 2, 64, 64, 0.1, 1, FAKE, FAKE, None) == 1
    assert lib.ra_block_attn_step(1, FAKE, -1, 8, FAKE, FAKE, 0, 64, 1, 2, 2, 64, 64, 0.1, 1, FAKE, FAKE, None) == 1
    assert lib.ra_block_attn_step(1, None, 0, 8, FAKE, FAKE, 0, 64, 1, 2, 2, 64, 64, 0.1, 1, FAKE, FAKE, None) == 1
    # fp8 decode: bad scales, bf16 shapes rules still apply
    assert lib.ra_splitkv_decode_fp8(FAKE, FAKE, FAKE, 0.0, 1.0, 1, 8, 2, 64, 128, 128, 2, 0.1, FAKE, FAKE,
                                     FAKE, FAKE, None) == 1
    assert lib.ra_splitkv_partial_fp8(FAKE, FAKE, FAKE, 1.0, float("inf"), 1, 8, 2, 64, 128, 128, 2, 0.1,
                                      FAKE, FAKE, None) == 1
    assert lib.ra_splitkv_partial_fp8(FAKE, FAKE, FAKE, 1.0, 1.0, 1, 8, 2, 64, 96, 96, 2, 0.1, FAKE, FAKE,
                                      None) == 2
    assert lib.ra_splitkv_partial_fp8(FAKE, FAKE, FAKE, 1e30, 1.0, 1, 8, 2, 64, 128, 128, 2, 1e10, FAKE, FAKE,
                                      None) == 1
    # backward: unsupported dims and dtypes, bad sizes
    bw = lambda **kw: lib.ra_block_attn_bwd_step(*dict(dict(
        dtype=1, q=FAKE, dout=FAKE, lse=FAKE, delta=FAKE, q_pos0=0, Sq=64, k=FAKE, v=FAKE, k_pos0=0, Sk=64, B=1,
        Hq=2, Hkv=2, Dqk=128, Dv=128, scale=0.1, causal=1, dq=FAKE, dk=FAKE, dv=FAKE, stream=None), **kw).values())
    assert bw(Dqk=192, Dv=128) == 2
    assert bw(dtype=0) == 2
    assert bw(Sq=0) == 1
    assert bw(q=None) == 1
    assert bw(Hkv=3) == 1
    assert lib.ra_attn_bwd_preprocess(0, FAKE, FAKE, 10, 128, FAKE, None) == 2
    assert lib.ra_attn_bwd_preprocess(1, FAKE, FAKE, 10, 12, FAKE, None) == 1
    assert lib.ra_attn_bwd_preprocess(1, FAKE, FAKE, 0, 128, FAKE, None) == 0
    # merges: zero rows is a no-op; bad Dv rejected
    assert lib.ra_lse_merge(0, 128, None, None, None, None, None, None, None) == 0
    assert lib.ra_lse_merge(10, 6, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.ra_lse_merge(-1, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.ra_lse_merge_n(1, 0, 8, 128, None, None, None, None, None) == 0
    assert lib.ra_lse_merge_n(1, 4, 0, 128, FAKE, FAKE, FAKE, FAKE, None) == 1
    # decode: L not divisible by n_splits; unsupported dtype / dims / group
    dec = lambda **kw: lib.ra_splitkv_decode(*dict(
        dict(dtype=1, q=FAKE, k=FAKE, v=FAKE, B=2, Hq=16, Hkv=2, L=1024, Dqk=128, Dv=128, n=8, scale=0.1,
             op=FAKE, lp=FAKE, o=FAKE, l=FAKE, st=None), **kw).values())
    assert dec(L=1000, n=3) == 1
    assert dec(dtype=0) == 2
    assert dec(Dqk=192, Dv=128) == 2
    assert dec(Hq=64, Hkv=2) == 2   # group of 32 heads is more than one MFMA tile
    assert dec(k=None) == 1
