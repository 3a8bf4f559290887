"""ctypes binding of libzs.so: argument marshalling only.

Each function has the name of the C entry point it calls (include/zs.h) and
takes torch tensors for device buffers; it checks that they are contiguous
device tensors of the right dtype and length, turns them into raw pointers
and the current stream, and raises ZsError on a nonzero status. All work of
the shard step runs in the library's HIP kernels. There is no fallback: if
the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import threading
from typing import List, Sequence, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzs.so")

ZS_OK, ZS_EINVAL, ZS_EALIAS, ZS_EHIP, ZS_EUNSUPPORTED, ZS_EIO = 0, 1, 2, 3, 4, 5
ZS_BF16, ZS_F32 = 1, 2
ZS_MAX_D = 64


class ZsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libzs status {status}: {message}")
        self.status = status


class zs_tensor_ref(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("numel", ctypes.c_int64),
                ("flat_offset", ctypes.c_int64)]


class zs_bucket(ctypes.Structure):
    _fields_ = [("p", ctypes.c_void_p), ("m", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("w_out", ctypes.c_void_p), ("S", ctypes.c_int64),
                ("sources", ctypes.POINTER(ctypes.c_void_p))]


ZS_W_STREAM, ZS_W_KEEP = 0, 1


class zs_reduce_opts(ctypes.Structure):
    _fields_ = [("replicas", ctypes.c_int32), ("round_to_reduce_dtype", ctypes.c_int32),
                ("scale", ctypes.c_double), ("working_shard_hint", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class zs_shard_info(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("D", ctypes.c_int32), ("N", ctypes.c_int64),
                ("S", ctypes.c_int64), ("step", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return dict(rank=self.rank, D=self.D, N=self.N, S=self.S, step=self.step)


class zs_adamw_hp(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("step", ctypes.c_int64)]


@dataclasses.dataclass(frozen=True)
class AdamWHP:
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    step: int


_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """Load libzs.so (once). Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m fsdp_sharded_optimizer_zs_amd.build` (needs hipcc)")
            lib = ctypes.CDLL(LIB_PATH)
            i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
            P = ctypes.POINTER
            sig = {
                "zs_unit_layout": (i32, [P(i64), i32, i32, P(i64), P(i64), P(i64), P(i64)]),
                "zs_pack_flat": (i32, [P(zs_tensor_ref), vp, i32, i32, i32, P(vp), i64, vp]),
                "zs_reduce_shard": (i32, [P(vp), i32, i32, i64, vp, vp]),
                "zs_adamw_step": (i32, [vp, vp, vp, vp, i64, P(vp), i32, i32,
                                        P(zs_adamw_hp), vp]),
                "zs_reduce_shard_ex": (i32, [P(vp), i32, P(zs_reduce_opts), i32, i64, vp, vp]),
                "zs_adamw_step_ex": (i32, [vp, vp, vp, vp, i64, P(vp), i32, P(zs_reduce_opts),
                                           i32, P(zs_adamw_hp), vp]),
                "zs_adamw_step_timed": (i32, [vp, vp, vp, vp, i64, P(vp), i32,
                                              P(zs_reduce_opts), i32, P(zs_adamw_hp), vp, vp,
                                              vp]),
                "zs_gather_unit": (i32, [P(vp), i32, i64, i32, vp, vp]),
                "zs_reshard": (i32, [P(vp), i32, i64, i64, i32, P(vp), i32, i64, vp]),
                "zs_adamw_step_host": (i32, [vp, vp, vp, vp, i64, vp, P(zs_adamw_hp), i32]),
                "zs_stream_ceiling": (i32, [vp, vp, vp, vp, i64, P(vp), i32, i32, vp]),
                "zs_stream_ceiling_timed": (i32, [vp, vp, vp, vp, i64, P(vp), i32, i32, vp, vp,
                                                  vp]),
                "zs_hbm_probe": (i32, [i32, vp, vp, i64, i32, vp]),
                "zs_offload_step": (i32, [P(vp), i32, i32, i64, vp, vp, vp, vp, vp, vp, vp,
                                          P(zs_adamw_hp), i32, i64, vp, vp]),
                "zs_shard_save": (i32, [ctypes.c_char_p, P(zs_shard_info), vp, vp, vp, vp, vp]),
                "zs_shard_info_read": (i32, [ctypes.c_char_p, P(zs_shard_info)]),
                "zs_shard_load": (i32, [ctypes.c_char_p, vp, vp, vp, vp, i64, P(zs_shard_info),
                                        vp]),
                "zs_shard_load_resharded": (i32, [P(ctypes.c_char_p), i32, i32, i32, vp, vp, vp,
                                                  vp, i64, P(zs_shard_info), vp]),
                "zs_step_pipelined": (i32, [P(zs_bucket), i32, i32, i32, vp, vp, i64,
                                            P(zs_adamw_hp), vp, vp]),
                "zs_step_pipelined_static": (i32, [P(zs_bucket), i32, i32, i32,
                                                   P(zs_adamw_hp), vp, vp]),
                "zs_last_error": (ctypes.c_char_p, []),
                "zs_abi_version": (i32, []),
            }
            for name, (res, args) in sig.items():
                f = getattr(lib, name)
                f.restype = res
                f.argtypes = args
            _lib = lib
    return _lib


def _check(status: int) -> None:
    if status != ZS_OK:
        raise ZsError(status, load().zs_last_error().decode())


def zs_last_error() -> str:
    return load().zs_last_error().decode()


def zs_abi_version() -> int:
    return int(load().zs_abi_version())


# ------------------------------------------------------------------ helpers
def _torch():
    import torch
    return torch


def _dtype_code_of(dtype) -> int:
    torch = _torch()
    if dtype in (torch.bfloat16, torch.int16) or dtype == getattr(torch, "uint16", None):
        return ZS_BF16
    if dtype == torch.float32:
        return ZS_F32
    raise TypeError(f"unsupported dtype {dtype}: use bf16 (bfloat16/int16 bits) or float32")


def _dtype_code(t) -> int:
    return _dtype_code_of(t.dtype)


def _dev(t, what: str):
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device (cuda/HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _stream(t, stream):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    return ctypes.c_void_p(_torch().cuda.current_stream(t.device).cuda_stream)


def _ptr_array(ts: Sequence) -> ctypes.Array:
    arr = (ctypes.c_void_p * max(1, len(ts)))()
    for i, t in enumerate(ts):
        arr[i] = t.data_ptr()
    return arr


def _hp(hp) -> zs_adamw_hp:
    if isinstance(hp, dict):
        hp = AdamWHP(**hp)
    return zs_adamw_hp(float(hp.lr), float(hp.beta1), float(hp.beta2), float(hp.eps),
                       float(hp.weight_decay), int(hp.step))


# --------------------------------------------------------------- entry points
def zs_unit_layout(numels: Sequence[int], D: int) -> Tuple[List[int], int, int, int]:
    """(offsets[T+1], N, N_pad, S) of a unit; host arithmetic in the library."""
    lib = load()
    T = len(numels)
    arr = (ctypes.c_int64 * max(1, T))(*[int(n) for n in numels])
    off = (ctypes.c_int64 * (T + 1))()
    n, npad, s = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib.zs_unit_layout(arr, T, int(D), off, ctypes.byref(n), ctypes.byref(npad),
                              ctypes.byref(s)))
    return list(off), n.value, npad.value, s.value


class PackTable:
    """The tensor table of one unit for zs_pack_flat: a host copy (checked
    by the library) and a device copy (read by the kernel), built once from
    the unit's tensors so that a unit packed again (a re-wrap, a repeated
    pack into fresh shards) does not rebuild it. It holds the tensors'
    pointers: valid while those tensors live."""

    def __init__(self, tensors: Sequence, D: int, device):
        import numpy as np
        torch = _torch()
        tensors = list(tensors)
        self.T = len(tensors)
        self.D = int(D)
        numels = [t.numel() for t in tensors]
        offsets, self.N, _, self.S = zs_unit_layout(numels, D)
        # rows are zs_tensor_ref: (ptr, numel, flat_offset), 3 x 8 bytes
        self._host = np.empty((max(1, self.T), 3), dtype=np.int64)
        if self.T:
            self._host[:self.T, 0] = np.array([t.data_ptr() for t in tensors],
                                              dtype=np.uint64).view(np.int64)
            self._host[:self.T, 1] = numels
            self._host[:self.T, 2] = offsets[:self.T]
        self.device = (torch.from_numpy(self._host[:self.T]).to(device) if self.T
                       else torch.zeros((0, 3), dtype=torch.int64, device=device))

    def host_ptr(self):
        return self._host.ctypes.data_as(ctypes.POINTER(zs_tensor_ref))

    def device_ptr(self):
        return ctypes.c_void_p(self.device.data_ptr() if self.T else None)


def _check_pack_operands(tensors, shards, D):
    if len(shards) != D:
        raise ValueError("need exactly D shard tensors")
    ref = shards[0]
    code = _dtype_code(ref)
    everything = list(tensors) + list(shards)
    # one pass per property, then the failing index for the message
    same = {t.dtype for t in everything}
    if not all(t.is_cuda and t.is_contiguous() for t in everything) or any(
            _dtype_code_of(d) != code for d in same) or len(
            {t.element_size() for t in everything}) != 1:
        for i, t in enumerate(everything):
            _dev(t, f"tensor {i}")
            if _dtype_code(t) != code or t.element_size() != ref.element_size():
                raise TypeError("tensors and shards must share one element type")
    return code


def zs_pack_flat(tensors: Sequence, D: int, shards: Sequence, stream=None,
                 table: "PackTable" = None) -> "PackTable":
    """Pack tensors (all bf16 or all fp32, contiguous, on the device) into D
    shard tensors of S elements each. Returns the unit's PackTable, whose
    device copy the enqueued kernel reads (stream-ordered; keep it, or let
    torch's caching allocator recycle it on the same stream); pass it back
    as `table` to pack the same tensors again without rebuilding it."""
    torch = _torch()
    tensors = list(tensors)
    ref = shards[0] if shards else None
    if table is None:
        code = _check_pack_operands(tensors, shards, D)
        table = PackTable(tensors, D, ref.device)
    else:
        # the tensors were checked when the table was built (the library
        # checks the table itself on every call); only the shards are new
        if table.T != len(tensors) or table.D != D or len(shards) != D:
            raise ValueError("table was built for another unit")
        code = _check_pack_operands([], shards, D)
        if table.T and ref.element_size() != tensors[0].element_size():
            raise TypeError("tensors and shards must share one element type")
    if any(s.numel() != table.S for s in shards):
        raise ValueError(f"every shard must hold S = {table.S} elements")
    if isinstance(stream, torch.cuda.Stream):
        # the kernel reads the table on `stream`: tell the caching allocator
        table.device.record_stream(stream)
    _check(load().zs_pack_flat(table.host_ptr(), table.device_ptr(), table.T, code, int(D),
                               _ptr_array(shards), table.S, _stream(ref, stream)))
    return table


def zs_reduce_shard(contribs: Sequence, grad_out, stream=None) -> None:
    """grad_out (fp32, S) = mean of the contributions, folded in rank order."""
    S = grad_out.numel()
    _dev(grad_out, "grad_out")
    if grad_out.dtype != _torch().float32:
        raise TypeError("grad_out must be float32")
    code = _dtype_code(contribs[0]) if contribs else ZS_F32
    for i, c in enumerate(contribs):
        _dev(c, f"contribs[{i}]")
        if c.numel() != S or _dtype_code(c) != code:
            raise ValueError("contributions must share one dtype and hold S elements")
    _check(load().zs_reduce_shard(_ptr_array(contribs), len(contribs), code, S,
                                  ctypes.c_void_p(grad_out.data_ptr()),
                                  _stream(grad_out, stream)))


def zs_adamw_step(p, m, v, w_out, contribs: Sequence, hp, stream=None) -> None:
    """Fused reduce + AdamW on one shard: p, m, v in place, w_out (bf16) written."""
    torch = _torch()
    S = p.numel()
    for name, t in (("p", p), ("m", m), ("v", v)):
        _dev(t, name)
        if t.dtype != torch.float32 or t.numel() != S:
            raise ValueError(f"{name} must be float32 with S = {S} elements")
    _dev(w_out, "w_out")
    if _dtype_code(w_out) != ZS_BF16 or w_out.numel() != S:
        raise ValueError("w_out must be bf16 bits with S elements")
    code = _dtype_code(contribs[0]) if contribs else ZS_F32
    for i, c in enumerate(contribs):
        _dev(c, f"contribs[{i}]")
        if c.numel() != S or _dtype_code(c) != code:
            raise ValueError("contributions must share one dtype and hold S elements")
    h = _hp(hp)
    _check(load().zs_adamw_step(ctypes.c_void_p(p.data_ptr()), ctypes.c_void_p(m.data_ptr()),
                                ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(w_out.data_ptr()),
                                S, _ptr_array(contribs), len(contribs), code,
                                ctypes.byref(h), _stream(p, stream)))


def _groups(contribs: Sequence, replicas: int) -> int:
    if replicas < 1 or len(contribs) % replicas:
        raise ValueError("contributions must form `replicas` equal groups")
    return len(contribs) // replicas


def zs_reduce_shard_ex(contribs: Sequence, grad_out, replicas: int = 1,
                       round_to_reduce_dtype: bool = False, stream=None,
                       scale: float = 0.0) -> None:
    """grad_out (fp32, S) = HYBRID_SHARD reduce of replicas groups of
    contributions (replica-major), optionally rounding each level's output to
    the reduce dtype; scale (0 = 1 / #contributions) is the one multiplier."""
    S = grad_out.numel()
    _dev(grad_out, "grad_out")
    if grad_out.dtype != _torch().float32:
        raise TypeError("grad_out must be float32")
    code = _dtype_code(contribs[0]) if contribs else ZS_F32
    for i, c in enumerate(contribs):
        _dev(c, f"contribs[{i}]")
        if c.numel() != S or _dtype_code(c) != code:
            raise ValueError("contributions must share one dtype and hold S elements")
    D = _groups(contribs, replicas)
    opts = zs_reduce_opts(int(replicas), 1 if round_to_reduce_dtype else 0, float(scale))
    _check(load().zs_reduce_shard_ex(_ptr_array(contribs), D, ctypes.byref(opts), code, S,
                                     ctypes.c_void_p(grad_out.data_ptr()),
                                     _stream(grad_out, stream)))


def _adamw_ex_args(p, m, v, w_out, contribs, hp, replicas, round_to_reduce_dtype, scale,
                   keep_working_shard):
    """Checked arguments of zs_adamw_step_ex / _timed, up to opts and hp
    (kept alive by the returned tuple)."""
    torch = _torch()
    S = p.numel()
    for name, t in (("p", p), ("m", m), ("v", v)):
        _dev(t, name)
        if t.dtype != torch.float32 or t.numel() != S:
            raise ValueError(f"{name} must be float32 with S = {S} elements")
    _dev(w_out, "w_out")
    if _dtype_code(w_out) != ZS_BF16 or w_out.numel() != S:
        raise ValueError("w_out must be bf16 bits with S elements")
    code = _dtype_code(contribs[0]) if contribs else ZS_F32
    for i, c in enumerate(contribs):
        _dev(c, f"contribs[{i}]")
        if c.numel() != S or _dtype_code(c) != code:
            raise ValueError("contributions must share one dtype and hold S elements")
    D = _groups(contribs, replicas)
    opts = zs_reduce_opts(int(replicas), 1 if round_to_reduce_dtype else 0, float(scale),
                          ZS_W_KEEP if keep_working_shard else ZS_W_STREAM, 0)
    h = _hp(hp)
    return (ctypes.c_void_p(p.data_ptr()), ctypes.c_void_p(m.data_ptr()),
            ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(w_out.data_ptr()), S,
            _ptr_array(contribs), D, opts, code, h)


def zs_adamw_step_ex(p, m, v, w_out, contribs: Sequence, hp, replicas: int = 1,
                     round_to_reduce_dtype: bool = False, stream=None,
                     scale: float = 0.0, keep_working_shard: bool = False) -> None:
    """zs_adamw_step with the reduce of zs_reduce_shard_ex; keep_working_shard
    stores the bf16 working shard with cache-allocating stores, for a caller
    that reads it right after (the unit's all-gather)."""
    pp, mp, vp_, wp, S, arr, D, opts, code, h = _adamw_ex_args(
        p, m, v, w_out, contribs, hp, replicas, round_to_reduce_dtype, scale, keep_working_shard)
    _check(load().zs_adamw_step_ex(pp, mp, vp_, wp, S, arr, D, ctypes.byref(opts), code,
                                   ctypes.byref(h), _stream(p, stream)))


def _event_handle(e, name):
    if isinstance(e, int):
        handle = e
    else:
        handle = int(getattr(e, "cuda_event", 0) or 0)   # torch.cuda.Event
    if not handle:
        raise ValueError(f"{name}: a created event is needed (a torch.cuda.Event with "
                         "enable_timing=True exists once it has been recorded)")
    return ctypes.c_void_p(handle)


def zs_adamw_step_timed(p, m, v, w_out, contribs: Sequence, hp, start, stop, replicas: int = 1,
                        round_to_reduce_dtype: bool = False, stream=None, scale: float = 0.0,
                        keep_working_shard: bool = False) -> None:
    """zs_adamw_step_ex whose kernel records `start` and `stop` (timing events:
    torch.cuda.Event(enable_timing=True), recorded once beforehand so that
    they exist, or raw hipEvent_t handles) at its own start and end; then
    start.elapsed_time(stop) is the kernel's execution time."""
    pp, mp, vp_, wp, S, arr, D, opts, code, h = _adamw_ex_args(
        p, m, v, w_out, contribs, hp, replicas, round_to_reduce_dtype, scale, keep_working_shard)
    _check(load().zs_adamw_step_timed(pp, mp, vp_, wp, S, arr, D, ctypes.byref(opts), code,
                                      ctypes.byref(h), _event_handle(start, "start"),
                                      _event_handle(stop, "stop"), _stream(p, stream)))


def zs_gather_unit(shards: Sequence, flat_out, stream=None) -> None:
    """flat_out[r*S + i] = shards[r][i]."""
    D = len(shards)
    _dev(flat_out, "flat_out")
    S = shards[0].numel() if shards else 0
    code = _dtype_code(flat_out)
    for i, s in enumerate(shards):
        _dev(s, f"shards[{i}]")
        if s.numel() != S or _dtype_code(s) != code:
            raise ValueError("shards must share one dtype and length")
    if flat_out.numel() != D * S:
        raise ValueError(f"flat_out must hold D*S = {D * S} elements")
    _check(load().zs_gather_unit(_ptr_array(shards), D, S, code,
                                 ctypes.c_void_p(flat_out.data_ptr()), _stream(flat_out, stream)))


def _bucket_array(buckets: Sequence, n_contrib: int, code: int):
    """zs_bucket descriptors for [(p, m, v, w_out, sources), ...], checked;
    returns (array, pointer arrays to keep alive)."""
    torch = _torch()
    arr = (zs_bucket * max(1, len(buckets)))()
    keep = []
    for b, (p, m, v, w, srcs) in enumerate(buckets):
        S = p.numel()
        for name, t in (("p", p), ("m", m), ("v", v)):
            _dev(t, f"bucket {b} {name}")
            if t.dtype != torch.float32 or t.numel() != S:
                raise ValueError(f"bucket {b}: {name} must be float32 with S = {S} elements")
        _dev(w, f"bucket {b} w_out")
        if _dtype_code(w) != ZS_BF16 or w.numel() != S:
            raise ValueError(f"bucket {b}: w_out must be bf16 bits with S elements")
        if len(srcs) != n_contrib:
            raise ValueError(f"bucket {b}: need {n_contrib} sources")
        for q, c in enumerate(srcs):
            if not c.is_contiguous() or c.numel() != S or _dtype_code(c) != code:
                raise ValueError(f"bucket {b} source {q}: contiguous, S elements, one dtype")
            if not c.is_cuda and c.numel() > 0 and not c.is_pinned():
                raise ValueError(f"bucket {b} source {q}: host sources must be pinned memory")
        ptrs = _ptr_array(srcs)
        keep.append(ptrs)
        arr[b] = zs_bucket(p.data_ptr(), m.data_ptr(), v.data_ptr(), w.data_ptr(), S,
                           ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)))
    return arr, keep


def zs_step_pipelined(buckets: Sequence, staging: Sequence, hp, compute=None,
                      transfer=None) -> None:
    """The shard step over buckets [(p, m, v, w_out, sources), ...], each
    bucket's sources (device tensors or pinned host tensors, one dtype)
    copied into alternating staging slots on `transfer` while the previous
    bucket steps on `compute`. staging = (slot0, slot1): device tensors of
    the sources' dtype, shape [n_contrib, staging_len]."""
    if len(staging) != 2:
        raise ValueError("staging must be two slot tensors")
    s0, s1 = staging
    for i, t in enumerate((s0, s1)):
        _dev(t, f"staging[{i}]")
        if t.dim() != 2 or t.shape != s0.shape or t.dtype != s0.dtype:
            raise ValueError("staging slots must be equal [n_contrib, staging_len] tensors")
    n_contrib, staging_len = int(s0.shape[0]), int(s0.shape[1])
    code = _dtype_code(s0)
    arr, keep = _bucket_array(buckets, n_contrib, code)
    h = _hp(hp)
    _check(load().zs_step_pipelined(arr, len(buckets), n_contrib, code,
                                    ctypes.c_void_p(s0.data_ptr()), ctypes.c_void_p(s1.data_ptr()),
                                    staging_len, ctypes.byref(h), _stream(s0, compute),
                                    _stream(s0, transfer)))


def zs_step_pipelined_static(buckets: Sequence, hp, compute=None, transfer=None) -> None:
    """zs_step_pipelined with the library's own staging array (no staging
    argument, no device allocation): buckets [(p, m, v, w_out, sources), ...]
    with sources of one dtype, as many per bucket."""
    if not buckets:
        raise ValueError("need at least one bucket")
    srcs0 = buckets[0][4]
    n_contrib = len(srcs0)
    code = _dtype_code(srcs0[0]) if srcs0 else ZS_F32
    arr, keep = _bucket_array(buckets, n_contrib, code)
    h = _hp(hp)
    ref = buckets[0][0]
    _check(load().zs_step_pipelined_static(arr, len(buckets), n_contrib, code, ctypes.byref(h),
                                           _stream(ref, compute), _stream(ref, transfer)))


def zs_reshard(src: Sequence, N: int, dst: Sequence, stream=None) -> None:
    """Re-shard a unit of N elements from shards src (D tensors of ceil(N/D))
    to shards dst (D2 tensors of ceil(N/D2)), bits copied, new pad +0."""
    if not src or not dst:
        raise ValueError("need at least one source and one destination shard")
    S, S2 = src[0].numel(), dst[0].numel()
    code = _dtype_code(src[0])
    for i, t in enumerate(list(src) + list(dst)):
        _dev(t, f"shard {i}")
        if _dtype_code(t) != code or t.element_size() != src[0].element_size():
            raise TypeError("all shards must share one element type")
    if any(t.numel() != S for t in src) or any(t.numel() != S2 for t in dst):
        raise ValueError("shards of one side must have equal lengths")
    _check(load().zs_reshard(_ptr_array(src), len(src), S, int(N), code, _ptr_array(dst),
                             len(dst), S2, _stream(dst[0], stream)))


def _state(p, m, v, w, S=None):
    torch = _torch()
    S = p.numel() if S is None else S
    for name, t in (("p", p), ("m", m), ("v", v)):
        _dev(t, name)
        if t.dtype != torch.float32 or t.numel() != S:
            raise ValueError(f"{name} must be float32 with S = {S} elements")
    _dev(w, "w")
    if _dtype_code(w) != ZS_BF16 or w.numel() != S:
        raise ValueError("w must be bf16 bits with S elements")
    return [ctypes.c_void_p(t.data_ptr()) for t in (p, m, v, w)]


def zs_shard_save(path: str, rank: int, D: int, N: int, step: int, p, m, v, w,
                  stream=None) -> None:
    """Save rank `rank`'s shard (of D over N elements) after `step` steps.
    Synchronizes the stream and writes the file."""
    S = zs_unit_layout([int(N)], int(D))[3]        # the layout's S = ceil(N / D)
    info = zs_shard_info(int(rank), int(D), int(N), S, int(step))
    ptrs = _state(p, m, v, w, S)
    _check(load().zs_shard_save(os.fsencode(path), ctypes.byref(info), *ptrs,
                                _stream(p, stream)))


def zs_shard_info_read(path: str) -> dict:
    info = zs_shard_info()
    _check(load().zs_shard_info_read(os.fsencode(path), ctypes.byref(info)))
    return info.as_dict()


def zs_shard_load(path: str, p, m, v, w, stream=None) -> dict:
    """Load a shard file saved at the same D into p, m, v, w; returns its info."""
    ptrs = _state(p, m, v, w)
    info = zs_shard_info()
    _check(load().zs_shard_load(os.fsencode(path), *ptrs, p.numel(), ctypes.byref(info),
                                _stream(p, stream)))
    return info.as_dict()


def zs_shard_load_resharded(paths: Sequence[str], rank: int, D2: int, p, m, v, w,
                            stream=None) -> dict:
    """Load rank `rank` of a D2-way sharding from the len(paths) files of one
    checkpoint (paths[r] = rank r's file); returns the new rank's info."""
    ptrs = _state(p, m, v, w)
    arr = (ctypes.c_char_p * max(1, len(paths)))(*[os.fsencode(x) for x in paths])
    info = zs_shard_info()
    _check(load().zs_shard_load_resharded(arr, len(paths), int(rank), int(D2), *ptrs, p.numel(),
                                          ctypes.byref(info), _stream(p, stream)))
    return info.as_dict()


def _host_f32(t, name, S):
    torch = _torch()
    if t.is_cuda or t.dtype != torch.float32 or t.numel() != S or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous host float32 tensor of {S} elements")
    return ctypes.c_void_p(t.data_ptr())


def _host_bf16(t, name, S):
    if t.is_cuda or _dtype_code(t) != ZS_BF16 or t.numel() != S or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous host bf16-bits tensor of {S} elements")
    return ctypes.c_void_p(t.data_ptr())


def zs_adamw_step_host(p, m, v, w_out, grad, hp, threads: int = 16) -> None:
    """AdamW on host tensors (p, m, v in place, w_out written) from the
    reduced fp32 gradient, on `threads` host threads."""
    S = p.numel()
    args = [_host_f32(p, "p", S), _host_f32(m, "m", S), _host_f32(v, "v", S),
            _host_bf16(w_out, "w_out", S)]
    h = _hp(hp)
    _check(load().zs_adamw_step_host(*args, S, _host_f32(grad, "grad", S), ctypes.byref(h),
                                     int(threads)))


def zs_offload_step(contribs: Sequence, grad_dev, grad_host, p, m, v, w_host, w_dev, hp,
                    threads: int = 16, chunk: int = 1 << 24, stream=None, h2d_stream=None) -> None:
    """One ZeRO-Offload shard step: device reduce, gradient down in chunks,
    host AdamW per chunk, working shard up on h2d_stream."""
    S = p.numel()
    code = _dtype_code(contribs[0]) if contribs else ZS_F32
    for i, c in enumerate(contribs):
        _dev(c, f"contribs[{i}]")
        if c.numel() != S or _dtype_code(c) != code:
            raise ValueError("contributions must share one dtype and hold S elements")
    _dev(grad_dev, "grad_dev")
    _dev(w_dev, "w_dev")
    if grad_dev.dtype != _torch().float32 or grad_dev.numel() != S:
        raise ValueError("grad_dev must be float32 with S elements")
    if _dtype_code(w_dev) != ZS_BF16 or w_dev.numel() != S:
        raise ValueError("w_dev must be bf16 bits with S elements")
    h = _hp(hp)
    _check(load().zs_offload_step(
        _ptr_array(contribs), len(contribs), code, S, ctypes.c_void_p(grad_dev.data_ptr()),
        _host_f32(grad_host, "grad_host", S), _host_f32(p, "p", S), _host_f32(m, "m", S),
        _host_f32(v, "v", S), _host_bf16(w_host, "w_host", S), ctypes.c_void_p(w_dev.data_ptr()),
        ctypes.byref(h), int(threads), int(chunk), _stream(grad_dev, stream),
        _stream(grad_dev, h2d_stream)))


def _ceiling_args(p, m, v, w, contribs):
    S = p.numel()
    ptrs = _state(p, m, v, w)
    code = _dtype_code(contribs[0])
    for i, c in enumerate(contribs):
        _dev(c, f"contribs[{i}]")
        if c.numel() != S or _dtype_code(c) != code:
            raise ValueError("contributions must share one dtype and hold S elements")
    return ptrs, S, _ptr_array(contribs), len(contribs), code


def zs_stream_ceiling(p, m, v, w, contribs: Sequence, stream=None) -> None:
    """Measurement aid: the fused step's streams without its arithmetic
    (p, m, v, w are overwritten with placeholders)."""
    ptrs, S, arr, n, code = _ceiling_args(p, m, v, w, contribs)
    _check(load().zs_stream_ceiling(*ptrs, S, arr, n, code, _stream(p, stream)))


def zs_stream_ceiling_timed(p, m, v, w, contribs: Sequence, start, stop, stream=None) -> None:
    """zs_stream_ceiling whose kernel records `start` and `stop` (as for
    zs_adamw_step_timed) at its own start and end."""
    ptrs, S, arr, n, code = _ceiling_args(p, m, v, w, contribs)
    _check(load().zs_stream_ceiling_timed(*ptrs, S, arr, n, code, _event_handle(start, "start"),
                                          _event_handle(stop, "stop"), _stream(p, stream)))


ZS_PROBE_READ, ZS_PROBE_WRITE, ZS_PROBE_COPY, ZS_PROBE_TRIAD = 0, 1, 2, 3


def zs_hbm_probe(kind: int, buf, buf2=None, blocks_per_cu: int = 1, stream=None) -> None:
    """Measurement aid: read, write or copy all of buf (any dtype; its byte
    size a multiple of 16) with the library's streaming access pattern, or a
    triad: buf2 = first half of buf XOR second half (buf's byte size a
    multiple of 32). buf2: the copy's or triad's destination (at least as
    large as what it receives), or a 16-byte sink for a read."""
    _dev(buf, "buf")
    nbytes = buf.numel() * buf.element_size()
    if kind == ZS_PROBE_TRIAD:
        if nbytes % 32:
            raise ValueError("a triad's buf must hold a multiple of 32 bytes")
        nbytes //= 2
    if buf2 is not None:
        _dev(buf2, "buf2")
        need = 16 if kind == ZS_PROBE_READ else nbytes
        if buf2.numel() * buf2.element_size() < need:
            raise ValueError(f"buf2 must hold at least {need} bytes")
    elif kind != ZS_PROBE_WRITE:
        raise ValueError("buf2 is required for read, copy and triad")
    _check(load().zs_hbm_probe(int(kind), buf.data_ptr(),
                               buf2.data_ptr() if buf2 is not None else None, nbytes,
                               int(blocks_per_cu), _stream(buf, stream)))


# Raw-pointer forms, for callers that manage device memory themselves.
def raw_adamw_step(p: int, m: int, v: int, w: int, S: int, contribs: Sequence[int],
                   dtype: int, hp, stream: int) -> None:
    arr = (ctypes.c_void_p * max(1, len(contribs)))(*contribs)
    h = _hp(hp)
    _check(load().zs_adamw_step(ctypes.c_void_p(p), ctypes.c_void_p(m), ctypes.c_void_p(v),
                                ctypes.c_void_p(w), int(S), arr, len(contribs), int(dtype),
                                ctypes.byref(h), ctypes.c_void_p(stream)))
