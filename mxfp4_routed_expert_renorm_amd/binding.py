"""ctypes binding of libmoe_mi355x.so: argument marshalling only.

Every function here forwards to the C entry point of the same name in
include/moe.h.  Tensors are torch tensors on the GPU (torch supplies device
memory and streams); their data pointers, sizes and the current HIP stream are
passed through unchanged.  Nothing is computed in Python, and there is no
fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_F32, MOE_BF16 = 0, 1
FP4, INT2, DROPPED = 0, 1, -1

c_int, c_size_t, c_void_p, c_char_p = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_char_p


class MoeError(RuntimeError):
    def __init__(self, name, status, msg):
        super().__init__(f"{name} failed with status {status}: {msg}")
        self.status = status


class moe_layer(ctypes.Structure):
    _fields_ = [
        ("H", c_int), ("I", c_int),
        ("fp4_base", c_void_p), ("fp4_stride", c_size_t), ("num_slots", c_int),
        ("int2_base", c_void_p), ("int2_stride", c_size_t), ("num_int2", c_int),
        ("shared", c_void_p), ("flags", c_int),
    ]


MOE_LAYER_SINGLE_LAUNCH = 1


class moe_cache_desc(ctypes.Structure):
    _fields_ = [
        ("L", c_int), ("E", c_int), ("H", c_int), ("I", c_int),
        ("num_slots", c_int), ("k", c_int), ("ladder_a", c_int), ("ladder_b", c_int),
        ("max_tokens", c_int),
        ("fp4_host", c_void_p), ("int2_host", c_void_p),
        ("fp4_arena", c_void_p), ("int2_staging", c_void_p),
        ("int2_slots", c_int), ("policy", c_int), ("lfu_decay", ctypes.c_double), ("lfu_seed", c_void_p),
        ("prefetch_slots", c_int), ("poll_us", ctypes.c_longlong),
    ]


MOE_CACHE_LRU, MOE_CACHE_LFU = 0, 1


class moe_cache_stats(ctypes.Structure):
    _fields_ = [
        ("calls", ctypes.c_int64), ("hits", ctypes.c_int64), ("misses", ctypes.c_int64),
        ("int2_uses", ctypes.c_int64), ("drops", ctypes.c_int64),
        ("bytes_h2d", ctypes.c_int64), ("evictions", ctypes.c_int64), ("int2_hits", ctypes.c_int64),
        ("prefetches", ctypes.c_int64), ("ring_hits", ctypes.c_int64), ("streamed", ctypes.c_int64),
    ]


_SIGS = {
    "moe_last_error": (c_char_p, []),
    "moe_version": (c_char_p, []),
    "moe_fp4_expert_bytes": (c_size_t, [c_int, c_int]),
    "moe_int2_expert_bytes": (c_size_t, [c_int, c_int]),
    "moe_router_logits": (c_int, [c_void_p, c_int, c_void_p, c_int, c_int, c_int, c_void_p, c_void_p]),
    "moe_route": (c_int, [c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "moe_group": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_group_scratch_bytes": (c_size_t, [c_int, c_int]),
    "moe_group_wide": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_expert_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
    "moe_expert_workspace_sync_offset": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
    "moe_expert_forward": (c_int, [ctypes.POINTER(moe_layer), c_void_p, c_int, c_int, c_int, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_int, c_void_p, c_size_t, c_void_p]),
    "moe_layer_decode": (c_int, [ctypes.POINTER(moe_layer), c_void_p, c_int, c_void_p, c_int, c_int, c_void_p,
                                 c_void_p, c_void_p, c_int, c_void_p, c_size_t, c_void_p]),
    "moe_layer_decode_noalloc": (c_int, [ctypes.POINTER(moe_layer), c_void_p, c_int, c_void_p, c_int, c_int,
                                         c_void_p, c_void_p, c_void_p, c_int, c_void_p]),
    "moe_noalloc_scratch_bytes": (c_size_t, []),
    "moe_combine": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_int, c_void_p]),
    "moe_debug_dequant": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p]),
    "moe_debug_stream_read": (c_int, [c_void_p, c_size_t, c_void_p, c_void_p]),
    "moe_tp_slice": (c_int, [c_void_p, c_size_t, c_int, c_int, c_int, c_int, c_int, c_void_p, c_size_t, c_void_p]),
    "moe_quant_mxfp8": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "moe_int2_from_fp4": (c_int, [c_void_p, c_size_t, c_int, c_int, c_int, c_void_p, c_size_t, c_void_p]),
    "moe_prefill_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
    "moe_prefill_forward": (c_int, [ctypes.POINTER(moe_layer), c_void_p, c_int, c_int, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_pinned_alloc": (c_int, [c_size_t, ctypes.POINTER(c_void_p)]),
    "moe_pinned_free": (c_int, [c_void_p]),
    "moe_cache_create": (c_int, [ctypes.POINTER(moe_cache_desc), ctypes.POINTER(c_void_p)]),
    "moe_cache_destroy": (c_int, [c_void_p]),
    "moe_cache_reset": (c_int, [c_void_p]),
    "moe_cache_plan": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_cache_ensure": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_cache_prefetch": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p]),
    "moe_prefill_streams": (c_int, [c_int, c_int, c_int]),
    "moe_cache_stream_layer": (c_int, [c_void_p, c_int, ctypes.POINTER(c_int), c_void_p, c_void_p]),
    "moe_cache_layer_buffer": (c_int, [c_void_p, c_int, c_void_p, ctypes.POINTER(moe_layer)]),
    "moe_cache_slot_map": (c_int, [c_void_p, c_void_p]),
    "moe_cache_get_stats": (c_int, [c_void_p, ctypes.POINTER(moe_cache_stats)]),
    "moe_cache_layer": (c_int, [c_void_p, ctypes.POINTER(moe_layer)]),
    "moe_profile_begin": (c_int, [c_int]),
    "moe_profile_end": (c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_int), c_int]),
}

_lib = None


def load():
    """Load the built library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(or python -m mxfp4_routed_expert_renorm_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(name, st):
    if st != 0:
        raise MoeError(name, st, load().moe_last_error().decode())


def _p(t):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    import torch
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t):
    import torch
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# ---------------------------------------------------------------------- sizes

def moe_version() -> str:
    return load().moe_version().decode()


def moe_fp4_expert_bytes(H, I) -> int:
    return load().moe_fp4_expert_bytes(H, I)


def moe_int2_expert_bytes(H, I) -> int:
    return load().moe_int2_expert_bytes(H, I)


def moe_expert_workspace_bytes(H, I, T, k, has_shared) -> int:
    return load().moe_expert_workspace_bytes(H, I, T, k, int(bool(has_shared)))


def moe_expert_workspace_sync_offset(H, I, T, k, has_shared) -> int:
    return load().moe_expert_workspace_sync_offset(H, I, T, k, int(bool(has_shared)))


def moe_noalloc_scratch_bytes() -> int:
    return load().moe_noalloc_scratch_bytes()


def expert_workspace(H, I, T, k, has_shared, device="cuda"):
    """A device workspace for moe_expert_forward / moe_layer_decode, zeroed
    (the single-launch batch-1 step keeps call tags in it from call to call)."""
    import torch
    return torch.zeros(moe_expert_workspace_bytes(H, I, T, k, has_shared), dtype=torch.uint8, device=device)


# -------------------------------------------------------------------- routing

def moe_router_logits(x, w_router, logits, stream=None):
    T, H = x.shape
    E = w_router.shape[0]
    _check("moe_router_logits", load().moe_router_logits(_p(x), _dt(x), _p(w_router), T, E, H, _p(logits),
                                                         _stream(stream)))
    return logits


def moe_prefill_streams(T, k, E) -> bool:
    """The prefill crossover: stream whole expert layers when T * k >= E."""
    return bool(load().moe_prefill_streams(T, k, E))


def moe_route(logits, k, ids, w, stream=None):
    T, E = logits.shape
    _check("moe_route", load().moe_route(_p(logits), T, E, k, _p(ids), _p(w), _stream(stream)))
    return ids, w


def moe_group(keys, nkeys, counts, offsets, perm, stream=None):
    n = keys.numel()
    _check("moe_group", load().moe_group(_p(keys), n, nkeys, _p(counts), _p(offsets), _p(perm), _stream(stream)))
    return counts, offsets, perm


def moe_group_scratch_bytes(n, nkeys):
    return load().moe_group_scratch_bytes(n, nkeys)


def moe_group_wide(keys, nkeys, counts, offsets, perm, scratch, stream=None):
    n = keys.numel()
    _check("moe_group_wide", load().moe_group_wide(_p(keys), n, nkeys, _p(counts), _p(offsets), _p(perm),
                                                   _p(scratch), _stream(stream)))
    return counts, offsets, perm


# ----------------------------------------------------------------- expert MLP

def make_layer(H, I, fp4_base=None, fp4_stride=0, num_slots=0, int2_base=None, int2_stride=0, num_int2=0,
               shared=None, flags=0) -> moe_layer:
    """A moe_layer descriptor from device tensors (uint8 records).  The
    descriptor holds raw device pointers, so it keeps references to the tensors:
    they cannot be freed (and their memory unmapped) while it is alive."""
    lay = moe_layer(H, I, _p(fp4_base), fp4_stride, num_slots, _p(int2_base), int2_stride, num_int2, _p(shared),
                    flags)
    lay._tensors = (fp4_base, int2_base, shared)
    return lay


def moe_expert_forward(layer: moe_layer, x, T, k, slot_ids, prec, w, out, workspace, stream=None):
    ot = _dt(out)
    st = load().moe_expert_forward(ctypes.byref(layer), _p(x), _dt(x), T, k, _p(slot_ids), _p(prec), _p(w),
                                   _p(out), ot, _p(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream))
    _check("moe_expert_forward", st)
    return out


def moe_layer_decode(layer: moe_layer, logits, x, k, ids, w, out, workspace, stream=None):
    """One token: route logits [E] (or [1, E]) and run the resident layer; ids/w [k] out."""
    E = logits.shape[-1]
    st = load().moe_layer_decode(ctypes.byref(layer), _p(logits), E, _p(x), _dt(x), k, _p(ids), _p(w), _p(out),
                                 _dt(out), _p(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream))
    _check("moe_layer_decode", st)
    return out


def moe_layer_decode_noalloc(layer: moe_layer, logits, x, k, ids, w, out, stream=None):
    """moe_layer_decode with the library's static per-device scratch as its
    workspace (no allocation in the call)."""
    E = logits.shape[-1]
    st = load().moe_layer_decode_noalloc(ctypes.byref(layer), _p(logits), E, _p(x), _dt(x), k, _p(ids), _p(w),
                                         _p(out), _dt(out), _stream(stream))
    _check("moe_layer_decode_noalloc", st)
    return out


def moe_combine(y, w, prec, T, k, H, has_shared, out, stream=None):
    st = load().moe_combine(_p(y), _p(w), _p(prec), T, k, H, int(bool(has_shared)), _p(out), _dt(out),
                            _stream(stream))
    _check("moe_combine", st)
    return out


def moe_debug_dequant(record, H, I, prec, matrix, out, stream=None):
    _check("moe_debug_dequant", load().moe_debug_dequant(_p(record), H, I, prec, matrix, _p(out), _stream(stream)))
    return out


def moe_tp_slice(src, H, I, G, g, dst, stream=None):
    """Rank g of G's share of a bank: src uint8 [n, stride] (H, I) -> dst uint8 [n, stride'] (H, I/G)."""
    def row_stride(t):  # a size-1 leading dimension may carry any stride
        return t.stride(0) if t.shape[0] > 1 else t.shape[1]
    _check("moe_tp_slice", load().moe_tp_slice(_p(src), row_stride(src), src.shape[0], H, I, G, g, _p(dst),
                                               row_stride(dst), _stream(stream)))
    return dst


def moe_int2_from_fp4(src, H, I, dst, stream=None):
    """2-bit copies of FP4 records: src uint8 [n, stride] -> dst uint8 [n, stride'] (clip search)."""
    def row_stride(t):
        return t.stride(0) if t.shape[0] > 1 else t.shape[1]
    _check("moe_int2_from_fp4", load().moe_int2_from_fp4(_p(src), row_stride(src), src.shape[0], H, I, _p(dst),
                                                         row_stride(dst), _stream(stream)))
    return dst


def moe_debug_stream_read(buf, sink, stream=None):
    """Read every byte of the uint8 device tensor `buf` once (measurement reference)."""
    _check("moe_debug_stream_read", load().moe_debug_stream_read(_p(buf), buf.numel(), _p(sink), _stream(stream)))


# -------------------------------------------------------------------- prefill

def moe_quant_mxfp8(x, codes, scales, stream=None):
    rows, K = x.shape
    _check("moe_quant_mxfp8", load().moe_quant_mxfp8(_p(x), rows, K, _p(codes), _p(scales), _stream(stream)))
    return codes, scales


def moe_prefill_workspace_bytes(H, I, T, k, has_shared) -> int:
    return load().moe_prefill_workspace_bytes(H, I, T, k, int(bool(has_shared)))


def moe_prefill_forward(layer: moe_layer, x, k, ids, w, out, workspace, stream=None):
    T = x.shape[0]
    st = load().moe_prefill_forward(ctypes.byref(layer), _p(x), T, k, _p(ids), _p(w), _p(out), _p(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream))
    _check("moe_prefill_forward", st)
    return out


# ----------------------------------------------------------------- slot cache

class PinnedBuffer:
    """Exact-size pinned host memory from moe_pinned_alloc, viewed as uint8."""

    def __init__(self, nbytes: int):
        import numpy as np
        p = c_void_p()
        _check("moe_pinned_alloc", load().moe_pinned_alloc(nbytes, ctypes.byref(p)))
        self.ptr, self.nbytes = p.value, nbytes
        self.array = np.ctypeslib.as_array((ctypes.c_uint8 * nbytes).from_address(self.ptr))

    def free(self):
        if self.ptr:
            self.array = None
            _check("moe_pinned_free", load().moe_pinned_free(c_void_p(self.ptr)))
            self.ptr = None


def _np_p(a):
    return None if a is None else c_void_p(a.ctypes.data)


def _addr(x):
    """Address of a torch tensor, a PinnedBuffer, an int, or None."""
    if x is None:
        return None
    if isinstance(x, PinnedBuffer):
        return c_void_p(x.ptr)
    if isinstance(x, int):
        return c_void_p(x)
    return c_void_p(x.data_ptr())


class Cache:
    """moe_cache handle.  Host banks and device buffers are supplied by the
    caller; the handle keeps references to them, so they outlive it."""

    def __init__(self, L, E, H, I, num_slots, k, a, b, max_tokens=1, fp4_host=None, int2_host=None,
                 fp4_arena=None, int2_staging=None, int2_slots=0, policy="lru", lfu_decay=1.0, lfu_seed=None,
                 prefetch_slots=0, poll_us=0):
        """lfu_seed: host float32 array [L*E] of initial use counts (copied), or None.
        prefetch_slots: staging-ring entries after the slots (fp4_arena then holds
        num_slots + prefetch_slots records).  poll_us: the host's polling budget for
        each call's picks (0: the default, < 0: no poll)."""
        import numpy as np
        seed = None if lfu_seed is None else np.ascontiguousarray(lfu_seed, dtype=np.float32).reshape(-1)
        d = moe_cache_desc(L, E, H, I, num_slots, k, a, b, max_tokens, _addr(fp4_host), _addr(int2_host),
                           _addr(fp4_arena), _addr(int2_staging), int2_slots,
                           {"lru": MOE_CACHE_LRU, "lfu": MOE_CACHE_LFU}[policy], lfu_decay,
                           None if seed is None else seed.ctypes.data, prefetch_slots, poll_us)
        h = c_void_p()
        _check("moe_cache_create", load().moe_cache_create(ctypes.byref(d), ctypes.byref(h)))
        self.h, self.L, self.E, self.k = h, L, E, k
        self._buffers = (fp4_host, int2_host, fp4_arena, int2_staging)

    def destroy(self):
        if self.h:
            _check("moe_cache_destroy", load().moe_cache_destroy(self.h))
            self.h = None

    def reset(self):
        _check("moe_cache_reset", load().moe_cache_reset(self.h))

    def plan(self, layer, ids, w):
        """Host-only policy step: ids int32 [T,k], w float32 [T,k] numpy."""
        import numpy as np
        ids = np.ascontiguousarray(ids, np.int32)
        w = np.ascontiguousarray(w, np.float32)
        T = ids.shape[0]
        slots = np.empty_like(ids)
        prec = np.empty(ids.shape, np.int8)
        wo = np.empty_like(w)
        _check("moe_cache_plan", load().moe_cache_plan(self.h, layer, T, _np_p(ids), _np_p(w), _np_p(slots),
                                                       _np_p(prec), _np_p(wo)))
        return slots, prec, wo

    def ensure(self, layer, T, ids_inout, w_inout, prec_out, compute=None, copy=None):
        st = load().moe_cache_ensure(self.h, layer, T, _p(ids_inout), _p(w_inout), _p(prec_out),
                                     _stream(compute), None if copy is None else _stream(copy))
        _check("moe_cache_ensure", st)

    def prefetch(self, layer, experts, copy=None):
        """Stage predicted experts (host int sequence, most likely first) of
        `layer` into the ring; copies go on `copy` (a torch stream; None is the
        null stream, and a cache without a device arena copies nothing)."""
        import numpy as np
        e = np.ascontiguousarray(np.asarray(experts, np.int32).reshape(-1))
        st = load().moe_cache_prefetch(self.h, layer, int(e.size), _np_p(e) if e.size else None,
                                       None if copy is None else _stream(copy))
        _check("moe_cache_prefetch", st)

    def stream_layer(self, layer, compute=None, copy=None, device=True):
        """Stream every expert of `layer` into the next layer buffer; returns
        the buffer (0 or 1).  device=False: a cache without a device arena
        (policy only, no streams touched)."""
        b = c_int(-1)
        st = load().moe_cache_stream_layer(self.h, layer, ctypes.byref(b),
                                           _stream(compute) if device else None,
                                           (None if copy is None else _stream(copy)) if device else None)
        _check("moe_cache_stream_layer", st)
        return b.value

    def layer_buffer(self, layer, compute=None) -> moe_layer:
        lay = moe_layer()
        _check("moe_cache_layer_buffer", load().moe_cache_layer_buffer(self.h, layer, _stream(compute),
                                                                       ctypes.byref(lay)))
        lay._tensors = self._buffers
        return lay

    def slot_map(self):
        import numpy as np
        m = np.empty(self.L * self.E, np.int32)
        _check("moe_cache_slot_map", load().moe_cache_slot_map(self.h, _np_p(m)))
        return m

    def stats(self) -> dict:
        s = moe_cache_stats()
        _check("moe_cache_get_stats", load().moe_cache_get_stats(self.h, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in moe_cache_stats._fields_}

    def layer(self) -> moe_layer:
        lay = moe_layer()
        _check("moe_cache_layer", load().moe_cache_layer(self.h, ctypes.byref(lay)))
        lay._tensors = self._buffers
        return lay


# --------------------------------------------------------------------- timing

PROF_KINDS = ("route", "router_logits", "gateup", "down", "combine", "group", "plan", "quant",
              "gemm_gateup", "gemm_down", "dequant", "read", "cache", "fused", "scratch")
MOE_PROF_KINDS = 16


def moe_profile_begin(max_launches: int):
    _check("moe_profile_begin", load().moe_profile_begin(max_launches))


def moe_profile_end() -> dict:
    """{kind: (total_ms, launches)} for every kind that ran."""
    tot = (ctypes.c_double * MOE_PROF_KINDS)()
    cnt = (c_int * MOE_PROF_KINDS)()
    _check("moe_profile_end", load().moe_profile_end(tot, cnt, MOE_PROF_KINDS))
    return {PROF_KINDS[i]: (tot[i], cnt[i]) for i in range(len(PROF_KINDS)) if cnt[i] > 0}
