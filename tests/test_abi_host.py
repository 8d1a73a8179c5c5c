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
    assert ra.abi_version() == 5


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
    assert call(Sp=1 << 30, P=1 << 30, nq=1) == 2   # rows * d * 2 would wrap 64 bits
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
    assert bw(Dqk=96, Dv=96) == 2
    assert bw(dtype=0, Dqk=192, Dv=128) == 2   # no fp32 kernel at D_qk 192
    assert bw(dtype=2) == 1
    assert bw(dtype=0, Dqk=64, Dv=96) == 2
    assert bw(Sq=0) == 1
    assert bw(q=None) == 1
    assert bw(Hkv=3) == 1
    assert lib.ra_attn_bwd_preprocess(2, FAKE, FAKE, 10, 128, FAKE, None) == 1
    assert lib.ra_attn_bwd_preprocess(0, FAKE, FAKE, 10, 12, FAKE, None) == 1
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


def test_alignment_of_every_pointer(ra):
    """Every pointer, the LSE-like fp32 vectors included, must be 16-byte aligned."""
    lib = ra.load_library()
    bad = FAKE + 4
    # two-way merge: each of the six pointers in turn
    for pos in range(6):
        ptrs = [FAKE] * 6
        ptrs[pos] = bad
        assert lib.ra_lse_merge(10, 128, *ptrs, None) == 1, pos
    # n-way merge
    for pos in range(4):
        ptrs = [FAKE] * 4
        ptrs[pos] = bad
        assert lib.ra_lse_merge_n(1, 4, 8, 128, *ptrs, None) == 1, pos
    # decode partials and outputs
    dec = lambda **kw: lib.ra_splitkv_decode(*dict(
        dict(dtype=1, q=FAKE, k=FAKE, v=FAKE, B=2, Hq=16, Hkv=2, L=1024, Dqk=128, Dv=128, n=8, scale=0.1,
             op=FAKE, lp=FAKE, o=FAKE, l=FAKE, st=None), **kw).values())
    assert dec(lp=bad) == 1
    assert dec(l=bad) == 1
    assert dec(op=bad) == 1
    assert lib.ra_splitkv_partial(1, FAKE, FAKE, FAKE, 2, 16, 2, 1024, 128, 128, 8, 0.1, FAKE, bad, None) == 1
    assert lib.ra_splitkv_partial_fp8(FAKE, FAKE, FAKE, 1.0, 1.0, 2, 16, 2, 1024, 128, 128, 8, 0.1, FAKE, bad,
                                      None) == 1
    # backward: delta of the preprocess; lse and delta of the step
    assert lib.ra_attn_bwd_preprocess(1, FAKE, FAKE, 10, 128, bad, None) == 1
    bw = lambda **kw: lib.ra_block_attn_bwd_step(*dict(dict(
        dtype=1, q=FAKE, dout=FAKE, lse=FAKE, delta=FAKE, q_pos0=0, Sq=64, k=FAKE, v=FAKE, k_pos0=0, Sk=64, B=1,
        Hq=2, Hkv=2, Dqk=128, Dv=128, scale=0.1, causal=1, dq=FAKE, dk=FAKE, dv=FAKE, stream=None), **kw).values())
    assert bw(lse=bad) == 1
    assert bw(delta=bad) == 1
    assert b"aligned" in lib.ra_last_error()


def _cpu(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def _raises_shape(ra, fn, *a, **kw):
    with pytest.raises(ra.RingAttnError) as e:
        fn(*a, **kw)
    msg = str(e.value)
    assert "shape" in msg or "dimensions" in msg or "dtype" in msg, msg
    return msg


def test_binding_checks_shapes_before_the_abi(ra):
    """The Python wrappers compare every tensor's shape with q's before any pointer
    crosses the C ABI (CPU tensors here: a shape error must come first; tensors of
    the right shapes then fail only because they are not on the device)."""
    import torch
    f32 = torch.float32
    q, k, v = _cpu(1, 4, 64, 128), _cpu(1, 2, 128, 128), _cpu(1, 2, 128, 128)
    # ring prefill: k / v against q, and user-supplied outputs
    _raises_shape(ra, ra.ring_attn_fwd, q, _cpu(1, 2, 128, 64), v, P=2, causal=True)
    _raises_shape(ra, ra.ring_attn_fwd, q, k, _cpu(1, 2, 64, 128), P=2, causal=True)
    _raises_shape(ra, ra.ring_attn_fwd, q, k, v, P=2, causal=True, out=_cpu(1, 4, 32, 128))
    _raises_shape(ra, ra.ring_attn_fwd, q, k, v, P=2, causal=True, lse=_cpu(1, 4, 65, dtype=f32))
    _raises_shape(ra, ra.ring_attn_fwd, q[0], k, v, P=2, causal=True)
    with pytest.raises(ra.RingAttnError, match="device"):
        ra.ring_attn_fwd(q, k, v, P=2, causal=True)
    # block step: k_blk / v_blk against q, state shapes
    o_acc, l_acc = _cpu(1, 4, 64, 128, dtype=f32), _cpu(1, 4, 64, dtype=f32)
    _raises_shape(ra, ra.block_attn_step, q, _cpu(1, 2, 100, 64), v, o_acc, l_acc, q_pos0=0, k_pos0=0, causal=True)
    _raises_shape(ra, ra.block_attn_step, q, k, v, _cpu(1, 4, 63, 128, dtype=f32), l_acc, q_pos0=0, k_pos0=0,
                  causal=True)
    # merges
    oa, la = _cpu(8, 128, dtype=f32), _cpu(8, dtype=f32)
    _raises_shape(ra, ra.lse_merge, oa, la, oa, la, out=_cpu(4, 128, dtype=f32))
    _raises_shape(ra, ra.lse_merge, oa, la, oa, la, lse_out=_cpu(7, dtype=f32))
    _raises_shape(ra, ra.lse_merge_n, _cpu(8, 4, 128, dtype=f32), _cpu(8, 3, dtype=f32))
    # decode: caches against q, user partial buffers
    qd, kc, vc = _cpu(2, 16, 128), _cpu(2, 2, 1024, 128), _cpu(2, 2, 1024, 128)
    _raises_shape(ra, ra.splitkv_decode, qd, _cpu(2, 2, 1024, 64), vc, n_splits=8)
    _raises_shape(ra, ra.splitkv_decode, qd, kc, _cpu(2, 3, 1024, 128), n_splits=8)
    _raises_shape(ra, ra.splitkv_partial, qd, kc, vc, n_splits=8, o_part=_cpu(2, 16, 4, 128, dtype=f32))
    _raises_shape(ra, ra.splitkv_partial, qd, kc, vc, n_splits=8, lse_part=_cpu(2, 16, 4, dtype=f32))
    _raises_shape(ra, ra.splitkv_partial, qd, kc, vc, n_splits=8, lse_part=_cpu(2, 16, 8))   # bf16, not fp32
    with pytest.raises(ra.RingAttnError, match="device"):
        ra.splitkv_partial(qd, kc, vc, n_splits=8)
    # backward: every accumulator, dout, lse and delta
    dq, dk, dv = _cpu(1, 4, 64, 128, dtype=f32), _cpu(1, 2, 128, 128, dtype=f32), _cpu(1, 2, 128, 128, dtype=f32)
    lse, dl, do = _cpu(1, 4, 64, dtype=f32), _cpu(1, 4, 64, dtype=f32), _cpu(1, 4, 64, 128)
    kw = dict(q_pos0=0, k_pos0=0, causal=True)
    _raises_shape(ra, ra.block_attn_bwd_step, q, do, lse, dl, k, v, _cpu(1, 4, 64, 64, dtype=f32), dk, dv, **kw)
    _raises_shape(ra, ra.block_attn_bwd_step, q, do, lse, dl, k, v, dq, _cpu(1, 4, 128, 128, dtype=f32), dv, **kw)
    _raises_shape(ra, ra.block_attn_bwd_step, q, do, lse, dl, k, v, dq, dk, _cpu(1, 2, 127, 128, dtype=f32), **kw)
    _raises_shape(ra, ra.block_attn_bwd_step, q, _cpu(1, 4, 64, 64), lse, dl, k, v, dq, dk, dv, **kw)
    _raises_shape(ra, ra.block_attn_bwd_step, q, do, _cpu(1, 4, 32, dtype=f32), dl, k, v, dq, dk, dv, **kw)
    _raises_shape(ra, ra.block_attn_bwd_step, q, do, lse, _cpu(1, 4, 65, dtype=f32), k, v, dq, dk, dv, **kw)
    with pytest.raises(ra.RingAttnError, match="device"):
        ra.block_attn_bwd_step(q, do, lse, dl, k, v, dq, dk, dv, **kw)
    _raises_shape(ra, ra.attn_bwd_preprocess, do, do, _cpu(1, 4, 63, dtype=f32))


def test_noalloc_decode_validation(ra):
    """The no-allocation decode rejects partials beyond its 16 MiB scratch, and bad
    arguments, before it looks the scratch up or launches anything."""
    lib = ra.load_library()
    call = lambda **kw: lib.ra_splitkv_decode_noalloc(*dict(
        dict(dtype=1, q=FAKE, k=FAKE, v=FAKE, B=16, Hq=64, Hkv=8, L=131072, Dqk=128, Dv=128, n=8, scale=0.1,
             o=FAKE, l=FAKE, st=None), **kw).values())
    assert call(B=64, n=64) == 1                  # 64*64*64*129*4 bytes of partials > 16 MiB
    assert b"scratch" in lib.ra_last_error()
    assert call(B=16, Hq=64, n=64) == 1           # 33.8 MB
    # products of the sizes that wrap 64 bits must not slip under the limit
    assert call(B=1 << 30, Hq=1 << 30, Hkv=1 << 30, n=1 << 30, L=1 << 30) == 1
    assert call(B=1 << 21, Hq=1 << 21, Hkv=1 << 21, n=1 << 21, L=1 << 21) == 1
    assert call(o=None) == 1
    assert call(l=FAKE + 4) == 1
    assert call(q=None) == 1
    assert call(B=0) == 1


def test_largest_slab_boundary(ra):
    """One row past the largest per-head slab (2^31 - 1 bytes) is refused with
    RA_EUNSUPPORTED before any launch; tests/test_gpu_limits.py runs the largest
    accepted sizes on the GPU."""
    lib = ra.load_library()
    D = 128
    max_bf16, max_fp8 = (2**31 - 1) // (2 * D), (2**31 - 1) // D
    # block step: K / V slab of Sk rows
    assert lib.ra_block_attn_step(1, FAKE, 0, 64, FAKE, FAKE, 0, max_bf16 + 1, 1, 16, 1, D, D, 0.1, 1, FAKE, FAKE,
                                  None) == 2
    # decode: cache slab of L rows (bf16, then one-byte fp8 values)
    L = (max_bf16 // 8 + 1) * 8
    assert lib.ra_splitkv_partial(1, FAKE, FAKE, FAKE, 1, 8, 1, L, D, D, 8, 0.1, FAKE, FAKE, None) == 2
    L8 = (max_fp8 // 8 + 1) * 8
    assert lib.ra_splitkv_partial_fp8(FAKE, FAKE, FAKE, 1.0, 1.0, 1, 8, 1, L8, D, D, 8, 0.1, FAKE, FAKE, None) == 2
    assert b"exceeds 2^31 bytes" in lib.ra_last_error()
