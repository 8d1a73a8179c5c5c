"""The entry points under HIP graph capture: they enqueue kernels on the given stream
and nothing else (no allocation, no synchronisation, no memset), so a captured ring
of block steps, a captured no-allocation decode and a captured backward ring replay
like the eager calls.

Each graph is replayed several times, with other eager work and synchronisations
between the replays, and every replay is compared bit for bit with the eager result
of the same calls. The running state is reset inside the graph with fill kernels
(torch's zero_ and fill_), not memsets."""
import math

import numpy as np
import pytest
import torch

from workloads import prefill_inputs_np, randn_np
from gpu_util import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ra():
    import blockwise_exact_attention_block_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return m


def to_dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype).contiguous()


def capture(fn):
    """fn once on a side stream (warm-up, as torch's graph capture expects), then
    captured into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ring_of_block_steps_in_a_graph(ra, dtype):
    """Partition 2 of a causal ring of 4 (GQA 4:1, D 128): its three visible block
    steps in ring order, captured with the state reset (bf16 and fp32 kernels)."""
    B, Hq, Hkv, Sp, P, D = 1, 8, 2, 384, 4, 128
    S, i = Sp * P, 2
    q, k, v = (to_dev(x, dtype) for x in prefill_inputs_np(B, Hq, Hkv, S, S, D, D, seed=181, dtype="f32"))
    qi = q[:, :, i * Sp:(i + 1) * Sp].contiguous()
    blocks = [(j, k[:, :, j * Sp:(j + 1) * Sp].contiguous(), v[:, :, j * Sp:(j + 1) * Sp].contiguous())
              for j, kind in ra.ring_schedule(P, i, True) if kind != "skip"]
    o_acc, l_acc = ra.init_state(qi, D)

    def chain():
        o_acc.zero_()
        l_acc.fill_(-math.inf)
        for j, kj, vj in blocks:
            ra.block_attn_step(qi, kj, vj, o_acc, l_acc, q_pos0=i * Sp, k_pos0=j * Sp, causal=True)

    chain()
    torch.cuda.synchronize()
    o_ref, l_ref = o_acc.clone(), l_acc.clone()
    g = capture(chain)
    for rep in range(3):
        o_acc.normal_()                      # garbage the graph must overwrite
        l_acc.normal_()
        g.replay()
        torch.cuda.synchronize()
        say(f"replay {rep}")
        assert torch.equal(o_acc, o_ref) and torch.equal(l_acc, l_ref), rep
        other, _ = ra.ring_attn_fwd(q, k, v, P=P, causal=True)   # eager work between replays
        torch.cuda.synchronize()
        del other


def test_noalloc_decode_in_a_graph(ra):
    """ra_splitkv_decode_noalloc captured with caller-owned outputs: its partials
    live in the library's device array, so the graph holds no allocation."""
    B, Hq, Hkv, L, D, n = 4, 16, 2, 4096, 128, 4
    q = to_dev(randn_np((B, Hq, D), 191, "bf16"))
    kc = to_dev(randn_np((B, Hkv, L, D), 192, "bf16"))
    vc = to_dev(randn_np((B, Hkv, L, D), 193, "bf16"))
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    _, _, o_ref, l_ref = ra.splitkv_decode(q, kc, vc, n_splits=n)
    torch.cuda.synchronize()
    g = capture(lambda: ra.splitkv_decode_noalloc(q, kc, vc, n_splits=n, out=out, lse=lse))
    for rep in range(3):
        out.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        say(f"replay {rep}")
        assert torch.equal(out, o_ref) and torch.equal(lse, l_ref), rep
        # an eager call on a smaller problem between replays overwrites the shared partials
        ra.splitkv_decode_noalloc(q[:1].contiguous(), kc[:1].contiguous(), vc[:1].contiguous(), n_splits=2)
        torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_backward_ring_in_a_graph(ra, dtype):
    """The backward ring protocol (delta, then every visible (query partition, KV
    block) step, accumulators zeroed by fill kernels) captured and replayed: bf16
    and fp32 kernels."""
    B, Hq, Hkv, Sp, P, D = 1, 4, 2, 160, 3, 128
    S = Sp * P
    q, k, v = (to_dev(x, dtype) for x in prefill_inputs_np(B, Hq, Hkv, S, S, D, D, seed=195, dtype="f32"))
    dout = to_dev(randn_np((B, Hq, S, D), 196, "f32"), dtype)
    o, lse = ra.ring_attn_fwd(q, k, v, P=P, causal=True)
    delta = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    part = lambda t, i: t[:, :, i * Sp:(i + 1) * Sp]
    qs, ks, vs, ds, ls = ([part(t, i).contiguous() for i in range(P)] for t in (q, k, v, dout, lse))
    dqs = [torch.empty((B, Hq, Sp, D), dtype=torch.float32, device=DEV) for _ in range(P)]
    dks = [torch.empty((B, Hkv, Sp, D), dtype=torch.float32, device=DEV) for _ in range(P)]
    dvs = [torch.empty((B, Hkv, Sp, D), dtype=torch.float32, device=DEV) for _ in range(P)]
    deltas = [torch.empty((B, Hq, Sp), dtype=torch.float32, device=DEV) for _ in range(P)]
    os_ = [part(o, i).contiguous() for i in range(P)]

    def chain():
        for t in dqs + dks + dvs:
            t.zero_()
        for i in range(P):
            ra.attn_bwd_preprocess(os_[i], ds[i], deltas[i])
        for i in range(P):
            for j, kind in ra.ring_schedule(P, i, True):
                if kind != "skip":
                    ra.block_attn_bwd_step(qs[i], ds[i], ls[i], deltas[i], ks[j], vs[j], dqs[i], dks[j], dvs[j],
                                           q_pos0=i * Sp, k_pos0=j * Sp, causal=True)

    chain()
    torch.cuda.synchronize()
    ref = [t.clone() for t in dqs + dks + dvs + deltas]
    g = capture(chain)
    for rep in range(3):
        for t in dqs + dks + dvs + deltas:
            t.normal_()                        # garbage the graph must overwrite
        g.replay()
        torch.cuda.synchronize()
        say(f"backward replay {rep} ({dtype})")
        for a, b in zip(dqs + dks + dvs + deltas, ref):
            assert torch.equal(a, b), rep
        other = ra.attn_bwd(q, k, v, o, lse, dout, causal=True)   # eager work between replays
        torch.cuda.synchronize()
        del other
    del delta
