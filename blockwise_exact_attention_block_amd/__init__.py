"""Ring-ordered blockwise exact attention on MI355X (gfx950).

Thin Python binding of libringattn.so (declared in include/ringattn.h). Every call
only checks and marshals arguments; all arithmetic runs in the library's HIP
kernels on the current torch stream. PyTorch provides device memory and streams.
There is no fallback: if the library is missing, every call raises.

Entry points (same names as the C ABI without the ``ra_`` prefix):
  ring_schedule    ring visiting order of one query partition (host only)
  ring_attn_fwd    ring prefill over P KV blocks, running state in registers
                   (layout="contiguous" or "striped": ra_ring_attn_fwd /
                   ra_ring_attn_fwd_striped, ra_ring_schedule / _striped)
  block_attn_step  merge one KV block into a running fp32 (O, LSE) state
  lse_merge        two-way merge of normalised partials
  lse_merge_n      n-way merge of normalised partials
  splitkv_partial  split-KV partial attention per chunk (no reduction)
  splitkv_decode   split-KV (pass-Q) decode: partials per chunk + reduction
  splitkv_partial_fp8 / splitkv_decode_fp8   the same over an fp8 e4m3 KV cache
  splitkv_decode_noalloc  splitkv_decode with its partials in library-held device
                   scratch, for callers that cannot allocate
  attn_bwd_preprocess  delta = rowsum(dO o O) for the backward pass
  block_attn_bwd_step  one (query block, KV block) pair's dQ, dK, dV contributions
  attn_bwd         whole-sequence backward (preprocess + one step over all pairs)
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import List, Optional, Tuple

import torch

__all__ = [
    "RingAttnError", "library_path", "load_library", "abi_version", "ring_schedule",
    "ring_attn_fwd", "block_attn_step", "init_state", "lse_merge", "lse_merge_n",
    "splitkv_partial", "splitkv_decode", "splitkv_partial_fp8", "splitkv_decode_fp8", "splitkv_decode_noalloc",
    "attn_bwd_preprocess", "block_attn_bwd_step", "attn_bwd",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libringattn.so"
_ABI_VERSION = 5
RA_F32, RA_BF16 = 0, 1
_STATUS = {0: "RA_OK", 1: "RA_EINVAL", 2: "RA_EUNSUPPORTED", 3: "RA_EHIP"}
_KIND = {0: "skip", 1: "diag", 2: "full"}

_lib = None


class RingAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def _hip_runtimes_mapped() -> List[str]:
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
        return sorted(os.path.realpath(p) for p in paths)
    except OSError:
        return []


def load_library() -> ctypes.CDLL:
    """Load libringattn.so (after torch, so it binds to the HIP runtime torch
    already mapped). Raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RingAttnError(3, f"{path} is missing: build it with "
                               "`python -m blockwise_exact_attention_block_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, ll, f, ip = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float, ctypes.POINTER(ctypes.c_int)
    sig = {
        "ra_abi_version": ([], i),
        "ra_last_error": ([], ctypes.c_char_p),
        "ra_ring_schedule": ([i, i, i, ip, ip], i),
        "ra_ring_attn_fwd": ([i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, vp], i),
        "ra_ring_schedule_striped": ([i, i, i, ip, ip], i),
        "ra_ring_attn_fwd_striped": ([i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, vp], i),
        "ra_block_attn_step": ([i, vp, ll, i, vp, vp, ll, i, i, i, i, i, i, f, i, vp, vp, vp], i),
        "ra_lse_merge": ([ll, i, vp, vp, vp, vp, vp, vp, vp], i),
        "ra_lse_merge_n": ([i, ll, i, i, vp, vp, vp, vp, vp], i),
        "ra_splitkv_decode": ([i, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, vp, vp, vp], i),
        "ra_splitkv_partial": ([i, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, vp], i),
        "ra_splitkv_decode_fp8": ([vp, vp, vp, f, f, i, i, i, i, i, i, i, f, vp, vp, vp, vp, vp], i),
        "ra_splitkv_partial_fp8": ([vp, vp, vp, f, f, i, i, i, i, i, i, i, f, vp, vp, vp], i),
        "ra_splitkv_decode_noalloc": ([i, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, vp], i),
        "ra_attn_bwd_preprocess": ([i, vp, vp, ll, i, vp, vp], i),
        "ra_block_attn_bwd_step": ([i, vp, vp, vp, vp, ll, i, vp, vp, ll, i, i, i, i, i, i, f, i, vp, vp, vp, vp], i),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if lib.ra_abi_version() != _ABI_VERSION:
        raise RingAttnError(2, f"library ABI {lib.ra_abi_version()} != binding ABI {_ABI_VERSION}")
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RingAttnError(3, "two HIP runtimes are mapped in this process: " + ", ".join(runtimes))
    _lib = lib
    return lib


def abi_version() -> int:
    return load_library().ra_abi_version()


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().ra_last_error().decode(errors="replace")
        raise RingAttnError(status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float32:
        return RA_F32
    raise RingAttnError(2, f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise RingAttnError(1, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise RingAttnError(1, f"{name} must be contiguous")
    return t.data_ptr()


def _expect(t: torch.Tensor, shape, name: str, dtype=None) -> None:
    """Raise RingAttnError unless t is a tensor of exactly `shape` (and `dtype`).
    The C ABI sees only pointers, so a tensor smaller than the sizes passed with it
    would be read or written past its end; every wrapper checks every tensor here
    before any pointer crosses the boundary."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise RingAttnError(1, f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if dtype is not None and t.dtype != dtype:
        raise RingAttnError(1, f"{name} has dtype {t.dtype}, expected {dtype}")


def _ndim(t: torch.Tensor, n: int, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != n:
        raise RingAttnError(1, f"{name} must have {n} dimensions, not {t.dim()}")


def _same_device(ref: torch.Tensor, *named) -> None:
    for t, name in named:
        if t.device != ref.device:
            raise RingAttnError(1, f"{name} is on {t.device}, not on {ref.device} with the others")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


_LAYOUTS = ("contiguous", "striped")


def _layout(layout: str) -> bool:
    if layout not in _LAYOUTS:
        raise RingAttnError(1, f"layout must be one of {_LAYOUTS}, not {layout!r}")
    return layout == "striped"


def ring_schedule(P: int, i: int, causal: bool, layout: str = "contiguous") -> List[Tuple[int, str]]:
    """[(kv_block, kind)] for the P ring steps of query partition i (host only)."""
    lib = load_library()
    fn = lib.ra_ring_schedule_striped if _layout(layout) else lib.ra_ring_schedule
    n = max(int(P), 1)
    kv = (ctypes.c_int * n)()
    kind = (ctypes.c_int * n)()
    r = fn(int(P), int(i), int(bool(causal)), kv, kind)
    if r < 0:
        _check(-r)
    return [(kv[s], _KIND[kind[s]]) for s in range(r)]


def ring_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, P: int, causal: bool,
                  scale: Optional[float] = None, q_part0: int = 0,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  layout: str = "contiguous"):
    """Ring prefill. q [B,Hq,nq*Sp,Dqk] holds query partitions q_part0..q_part0+nq-1;
    k [B,Hkv,P*Sp,Dqk] and v [B,Hkv,P*Sp,Dv] hold all P KV blocks. Partition p is
    tokens p*Sp.. (layout "contiguous") or tokens p, p+P, p+2P, ... ("striped").
    Returns (o [B,Hq,nq*Sp,Dv] in q's dtype, lse [B,Hq,nq*Sp] fp32)."""
    lib = load_library()
    fn = lib.ra_ring_attn_fwd_striped if _layout(layout) else lib.ra_ring_attn_fwd
    _ndim(q, 4, "q")
    _ndim(k, 4, "k")
    _ndim(v, 4, "v")
    B, Hq, Sq, Dqk = q.shape
    Hkv, Skv, Dv = k.shape[1], k.shape[2], v.shape[3]
    _expect(k, (B, Hkv, Skv, Dqk), "k")
    _expect(v, (B, Hkv, Skv, Dv), "v")
    if P <= 0:
        raise RingAttnError(1, f"P must be positive, not {P}")
    if Skv % P:
        raise RingAttnError(1, f"KV length {Skv} is not P={P} equal blocks")
    Sp = Skv // P
    if Sq % Sp:
        raise RingAttnError(1, f"query length {Sq} is not a whole number of partitions of {Sp}")
    nq = Sq // Sp
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    if out is None:
        out = torch.empty((B, Hq, Sq, Dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if k.dtype != q.dtype or v.dtype != q.dtype or out.dtype != q.dtype or lse.dtype != torch.float32:
        raise RingAttnError(1, "q, k, v, out must share one dtype and lse must be fp32")
    _expect(out, (B, Hq, Sq, Dv), "out")
    _expect(lse, (B, Hq, Sq), "lse")
    _same_device(q, (k, "k"), (v, "v"), (out, "out"), (lse, "lse"))
    _check(fn(_dtype_code(q), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
              _dev(lse, "lse"), B, Hq, Hkv, Sp, int(P), int(q_part0), nq, Dqk, Dv,
              float(scale), int(bool(causal)), _stream(q)))
    return out, lse


def init_state(q: torch.Tensor, Dv: int):
    """Empty running state for block_attn_step: O = 0 (fp32), LSE = -inf."""
    B, Hq, Sq, _ = q.shape
    o = torch.zeros((B, Hq, Sq, Dv), dtype=torch.float32, device=q.device)
    lse = torch.full((B, Hq, Sq), float("-inf"), dtype=torch.float32, device=q.device)
    return o, lse


def block_attn_step(q: torch.Tensor, k_blk: torch.Tensor, v_blk: torch.Tensor, o_acc: torch.Tensor,
                    lse_acc: torch.Tensor, *, q_pos0: int, k_pos0: int, causal: bool,
                    scale: Optional[float] = None) -> None:
    """Merge one KV block (keys at k_pos0..) into the running fp32 state of the
    queries at q_pos0.., in place."""
    lib = load_library()
    _ndim(q, 4, "q")
    _ndim(k_blk, 4, "k_blk")
    _ndim(v_blk, 4, "v_blk")
    B, Hq, Sq, Dqk = q.shape
    Hkv, Sk, Dv = k_blk.shape[1], k_blk.shape[2], v_blk.shape[3]
    _expect(k_blk, (B, Hkv, Sk, Dqk), "k_blk")
    _expect(v_blk, (B, Hkv, Sk, Dv), "v_blk")
    _same_device(q, (k_blk, "k_blk"), (v_blk, "v_blk"), (o_acc, "o_acc"), (lse_acc, "lse_acc"))
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    if o_acc.dtype != torch.float32 or lse_acc.dtype != torch.float32:
        raise RingAttnError(1, "running state must be fp32")
    if k_blk.dtype != q.dtype or v_blk.dtype != q.dtype:
        raise RingAttnError(1, "q, k_blk, v_blk must share one dtype")
    if tuple(o_acc.shape) != (B, Hq, Sq, Dv) or tuple(lse_acc.shape) != (B, Hq, Sq):
        raise RingAttnError(1, "running state shape does not match q / v_blk")
    _check(lib.ra_block_attn_step(_dtype_code(q), _dev(q, "q"), int(q_pos0), Sq, _dev(k_blk, "k_blk"),
                                  _dev(v_blk, "v_blk"), int(k_pos0), Sk, B, Hq, Hkv, Dqk, Dv, float(scale),
                                  int(bool(causal)), _dev(o_acc, "o_acc"), _dev(lse_acc, "lse_acc"),
                                  _stream(q)))


def lse_merge(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor, lse_b: torch.Tensor,
              out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None):
    """Two-way merge of normalised fp32 partials; o_* [..., Dv], lse_* [...]."""
    lib = load_library()
    Dv = o_a.shape[-1]
    rows = lse_a.numel()
    if out is None:
        out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    for t in (o_a, lse_a, o_b, lse_b, out, lse_out):
        if t.dtype != torch.float32:
            raise RingAttnError(1, "lse_merge works on fp32 tensors")
    if o_b.shape != o_a.shape or lse_b.shape != lse_a.shape or o_a.numel() != rows * Dv:
        raise RingAttnError(1, "shape mismatch")
    _expect(out, o_a.shape, "out")
    _expect(lse_out, lse_a.shape, "lse_out")
    _same_device(o_a, (lse_a, "lse_a"), (o_b, "o_b"), (lse_b, "lse_b"), (out, "out"), (lse_out, "lse_out"))
    _check(lib.ra_lse_merge(rows, Dv, _dev(o_a, "o_a"), _dev(lse_a, "lse_a"), _dev(o_b, "o_b"),
                            _dev(lse_b, "lse_b"), _dev(out, "out"), _dev(lse_out, "lse_out"), _stream(o_a)))
    return out, lse_out


def lse_merge_n(o_parts: torch.Tensor, lse_parts: torch.Tensor, out_dtype=torch.float32):
    """n-way merge along the partial axis: o_parts [..., n, Dv], lse_parts [..., n]."""
    lib = load_library()
    n, Dv = o_parts.shape[-2], o_parts.shape[-1]
    lead = tuple(o_parts.shape[:-2])
    rows = int(math.prod(lead))
    if tuple(lse_parts.shape) != lead + (n,):
        raise RingAttnError(1, "lse_parts shape must be o_parts.shape[:-1]")
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise RingAttnError(1, "o_parts and lse_parts must be fp32")
    _same_device(o_parts, (lse_parts, "lse_parts"))
    o = torch.empty(lead + (Dv,), dtype=out_dtype, device=o_parts.device)
    lse = torch.empty(lead, dtype=torch.float32, device=o_parts.device)
    _check(lib.ra_lse_merge_n(_dtype_code(o), rows, n, Dv, _dev(o_parts, "o_parts"),
                              _dev(lse_parts, "lse_parts"), _dev(o, "o"), _dev(lse, "lse"), _stream(o_parts)))
    return o, lse


def _decode_shapes(q, k_cache, v_cache, n_splits, o_part=None, lse_part=None):
    """Checks the decode tensors against each other; returns (B, Hq, Dqk, Hkv, L, Dv)."""
    _ndim(q, 3, "q")
    _ndim(k_cache, 4, "k_cache")
    _ndim(v_cache, 4, "v_cache")
    B, Hq, Dqk = q.shape
    Hkv, L, Dv = k_cache.shape[1], k_cache.shape[2], v_cache.shape[3]
    _expect(k_cache, (B, Hkv, L, Dqk), "k_cache")
    _expect(v_cache, (B, Hkv, L, Dv), "v_cache")
    if int(n_splits) <= 0:
        raise RingAttnError(1, f"n_splits must be positive, not {n_splits}")
    if o_part is not None:
        _expect(o_part, (B, Hq, n_splits, Dv), "o_part", torch.float32)
    if lse_part is not None:
        _expect(lse_part, (B, Hq, n_splits), "lse_part", torch.float32)
    named = [(k_cache, "k_cache"), (v_cache, "v_cache")]
    named += [(t, n) for t, n in ((o_part, "o_part"), (lse_part, "lse_part")) if t is not None]
    _same_device(q, *named)
    return B, Hq, Dqk, Hkv, L, Dv


def splitkv_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, *, n_splits: int,
                   scale: Optional[float] = None):
    """One query token per sequence: q [B,Hq,D], caches [B,Hkv,L,D]. Returns
    (o_part [B,Hq,n,D] fp32, lse_part [B,Hq,n] fp32, o [B,Hq,D] q.dtype, lse [B,Hq] fp32)."""
    lib = load_library()
    B, Hq, Dqk, Hkv, L, Dv = _decode_shapes(q, k_cache, v_cache, n_splits)
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    dev = q.device
    o_part = torch.empty((B, Hq, n_splits, Dv), dtype=torch.float32, device=dev)
    lse_part = torch.empty((B, Hq, n_splits), dtype=torch.float32, device=dev)
    o = torch.empty((B, Hq, Dv), dtype=q.dtype, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise RingAttnError(1, "q and the caches must share one dtype")
    _check(lib.ra_splitkv_decode(_dtype_code(q), _dev(q, "q"), _dev(k_cache, "k_cache"),
                                 _dev(v_cache, "v_cache"), B, Hq, Hkv, L, Dqk, Dv, int(n_splits), float(scale),
                                 _dev(o_part, "o_part"), _dev(lse_part, "lse_part"), _dev(o, "o"),
                                 _dev(lse, "lse"), _stream(q)))
    return o_part, lse_part, o, lse


def splitkv_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, *, n_splits: int,
                           scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None):
    """splitkv_decode whose partials live in the library's per-device scratch (no
    device allocation inside the call; pass `out` [B,Hq,D] and `lse` [B,Hq] to
    allocate nothing at all). Calls overlapping on one GPU race on that scratch.
    Returns (o, lse)."""
    lib = load_library()
    B, Hq, Dqk, Hkv, L, Dv = _decode_shapes(q, k_cache, v_cache, n_splits)
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    if out is None:
        out = torch.empty((B, Hq, Dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _expect(out, (B, Hq, Dv), "out", q.dtype)
    _expect(lse, (B, Hq), "lse", torch.float32)
    _same_device(q, (out, "out"), (lse, "lse"))
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise RingAttnError(1, "q and the caches must share one dtype")
    _check(lib.ra_splitkv_decode_noalloc(_dtype_code(q), _dev(q, "q"), _dev(k_cache, "k_cache"),
                                         _dev(v_cache, "v_cache"), B, Hq, Hkv, L, Dqk, Dv, int(n_splits),
                                         float(scale), _dev(out, "out"), _dev(lse, "lse"), _stream(q)))
    return out, lse


def splitkv_partial(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, *, n_splits: int,
                    scale: Optional[float] = None, o_part: Optional[torch.Tensor] = None,
                    lse_part: Optional[torch.Tensor] = None):
    """Partial attention of each of the n_splits chunks: returns (o_part [B,Hq,n,D]
    fp32, lse_part [B,Hq,n] fp32); reduce them with lse_merge_n."""
    lib = load_library()
    B, Hq, Dqk, Hkv, L, Dv = _decode_shapes(q, k_cache, v_cache, n_splits, o_part, lse_part)
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    if o_part is None:
        o_part = torch.empty((B, Hq, n_splits, Dv), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Hq, n_splits), dtype=torch.float32, device=q.device)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise RingAttnError(1, "q and the caches must share one dtype")
    _check(lib.ra_splitkv_partial(_dtype_code(q), _dev(q, "q"), _dev(k_cache, "k_cache"),
                                  _dev(v_cache, "v_cache"), B, Hq, Hkv, L, Dqk, Dv, int(n_splits), float(scale),
                                  _dev(o_part, "o_part"), _dev(lse_part, "lse_part"), _stream(q)))
    return o_part, lse_part


def _fp8_args(q, k_cache, v_cache, k_scale, v_scale):
    if q.dtype != torch.bfloat16:
        raise RingAttnError(1, "q must be bf16 for the fp8 cache path")
    if k_cache.dtype != torch.float8_e4m3fn or v_cache.dtype != torch.float8_e4m3fn:
        raise RingAttnError(1, "k_cache and v_cache must be torch.float8_e4m3fn")
    return float(k_scale), float(v_scale)


def splitkv_partial_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, *, k_scale: float,
                        v_scale: float, n_splits: int, scale: Optional[float] = None,
                        o_part: Optional[torch.Tensor] = None, lse_part: Optional[torch.Tensor] = None):
    """splitkv_partial over an fp8 e4m3 cache: keys are k_scale * k_cache, values
    v_scale * v_cache; q is bf16. Returns (o_part, lse_part) fp32."""
    lib = load_library()
    ks, vs = _fp8_args(q, k_cache, v_cache, k_scale, v_scale)
    B, Hq, Dqk, Hkv, L, Dv = _decode_shapes(q, k_cache, v_cache, n_splits, o_part, lse_part)
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    if o_part is None:
        o_part = torch.empty((B, Hq, n_splits, Dv), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Hq, n_splits), dtype=torch.float32, device=q.device)
    _check(lib.ra_splitkv_partial_fp8(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), ks, vs,
                                      B, Hq, Hkv, L, Dqk, Dv, int(n_splits), float(scale),
                                      _dev(o_part, "o_part"), _dev(lse_part, "lse_part"), _stream(q)))
    return o_part, lse_part


def splitkv_decode_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, *, k_scale: float,
                       v_scale: float, n_splits: int, scale: Optional[float] = None):
    """splitkv_decode over an fp8 e4m3 cache (see splitkv_partial_fp8). Returns
    (o_part, lse_part, o [B,Hq,D] bf16, lse [B,Hq] fp32)."""
    lib = load_library()
    ks, vs = _fp8_args(q, k_cache, v_cache, k_scale, v_scale)
    B, Hq, Dqk, Hkv, L, Dv = _decode_shapes(q, k_cache, v_cache, n_splits)
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    dev = q.device
    o_part = torch.empty((B, Hq, n_splits, Dv), dtype=torch.float32, device=dev)
    lse_part = torch.empty((B, Hq, n_splits), dtype=torch.float32, device=dev)
    o = torch.empty((B, Hq, Dv), dtype=q.dtype, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    _check(lib.ra_splitkv_decode_fp8(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), ks, vs,
                                     B, Hq, Hkv, L, Dqk, Dv, int(n_splits), float(scale),
                                     _dev(o_part, "o_part"), _dev(lse_part, "lse_part"), _dev(o, "o"),
                                     _dev(lse, "lse"), _stream(q)))
    return o_part, lse_part, o, lse


def attn_bwd_preprocess(o: torch.Tensor, dout: torch.Tensor, delta: Optional[torch.Tensor] = None):
    """delta [B,H,S] fp32 = rowsum(dout * o) for o, dout [B,H,S,Dv] (both bf16 or both fp32)."""
    lib = load_library()
    if o.shape != dout.shape or o.dtype != dout.dtype:
        raise RingAttnError(1, "o and dout must have one shape and dtype")
    Dv = o.shape[-1]
    rows = o.numel() // Dv
    if delta is None:
        delta = torch.empty(o.shape[:-1], dtype=torch.float32, device=o.device)
    _expect(delta, o.shape[:-1], "delta", torch.float32)
    _same_device(o, (dout, "dout"), (delta, "delta"))
    _check(lib.ra_attn_bwd_preprocess(_dtype_code(o), _dev(o, "o"), _dev(dout, "dout"), rows, Dv,
                                      _dev(delta, "delta"), _stream(o)))
    return delta


def block_attn_bwd_step(q: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor, delta: torch.Tensor,
                        k_blk: torch.Tensor, v_blk: torch.Tensor, dq_acc: torch.Tensor, dk_acc: torch.Tensor,
                        dv_acc: torch.Tensor, *, q_pos0: int, k_pos0: int, causal: bool,
                        scale: Optional[float] = None) -> None:
    """Adds one (query block, KV block) pair's gradient contributions into the fp32
    accumulators dq_acc [B,Hq,Sq,Dqk], dk_acc [B,Hkv,Sk,Dqk], dv_acc [B,Hkv,Sk,Dv].
    lse / delta are the queries' full-row values."""
    lib = load_library()
    _ndim(q, 4, "q")
    _ndim(k_blk, 4, "k_blk")
    _ndim(v_blk, 4, "v_blk")
    B, Hq, Sq, Dqk = q.shape
    Hkv, Sk, Dv = k_blk.shape[1], k_blk.shape[2], v_blk.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    for t, name in ((dq_acc, "dq_acc"), (dk_acc, "dk_acc"), (dv_acc, "dv_acc"), (lse, "lse"), (delta, "delta")):
        if t.dtype != torch.float32:
            raise RingAttnError(1, f"{name} must be fp32")
    _expect(k_blk, (B, Hkv, Sk, Dqk), "k_blk")
    _expect(v_blk, (B, Hkv, Sk, Dv), "v_blk")
    _expect(dout, (B, Hq, Sq, Dv), "dout", q.dtype)
    _expect(lse, (B, Hq, Sq), "lse")
    _expect(delta, (B, Hq, Sq), "delta")
    _expect(dq_acc, (B, Hq, Sq, Dqk), "dq_acc")
    _expect(dk_acc, (B, Hkv, Sk, Dqk), "dk_acc")
    _expect(dv_acc, (B, Hkv, Sk, Dv), "dv_acc")
    if k_blk.dtype != q.dtype or v_blk.dtype != q.dtype:
        raise RingAttnError(1, "q, k_blk, v_blk must share one dtype")
    _same_device(q, (dout, "dout"), (lse, "lse"), (delta, "delta"), (k_blk, "k_blk"), (v_blk, "v_blk"),
                 (dq_acc, "dq_acc"), (dk_acc, "dk_acc"), (dv_acc, "dv_acc"))
    _check(lib.ra_block_attn_bwd_step(_dtype_code(q), _dev(q, "q"), _dev(dout, "dout"), _dev(lse, "lse"),
                                      _dev(delta, "delta"), int(q_pos0), Sq, _dev(k_blk, "k_blk"),
                                      _dev(v_blk, "v_blk"), int(k_pos0), Sk, B, Hq, Hkv, Dqk, Dv, float(scale),
                                      int(bool(causal)), _dev(dq_acc, "dq_acc"), _dev(dk_acc, "dk_acc"),
                                      _dev(dv_acc, "dv_acc"), _stream(q)))


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
             dout: torch.Tensor, *, causal: bool, scale: Optional[float] = None):
    """Backward of ring_attn_fwd over a whole contiguous sequence on one device:
    returns fp32 (dq, dk, dv). Every (query partition, KV block) pair of the ring
    is covered by one step over the full sequence (positions 0..S-1)."""
    delta = attn_bwd_preprocess(o, dout)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=q.device)
    block_attn_bwd_step(q, dout, lse, delta, k, v, dq, dk, dv, q_pos0=0, k_pos0=0, causal=causal, scale=scale)
    return dq, dk, dv
