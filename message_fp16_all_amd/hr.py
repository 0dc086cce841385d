"""Python binding of libhr (``include/hr.h``): argument marshalling only.

Every function named ``hr_*`` here calls the C entry point of the same name
with the same arguments; every step of the combine runs in libhr's HIP
kernels.  The torch helpers at the bottom only turn tensors and streams into
the device pointers and ``hipStream_t`` handles those entry points take:
PyTorch is used for device memory and streams, nothing else.

The library is loaded from this package's directory on first use.  If it is
missing, loading raises ``ImportError``: there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhr.so")

HR_OK = 0
HR_ERR_INVALID_ARG = 1
HR_ERR_ALIGNMENT = 2
HR_ERR_TOO_LARGE = 3
HR_ERR_UNSUPPORTED = 4
HR_ERR_HIP = 5
HR_ERR_TIMEOUT = 6
HR_ERR_ABORTED = 7

HR_MAX_G = 16
HR_MAX_WORLD = 8
HR_DEFAULT_MAX_NUMEL = 131072
HR_MAX_NUMEL_LIMIT = 1 << 29
HR_NOALLOC_MAX_NUMEL = 131072
HR_NOALLOC_SCRATCH_BYTES = 8 << 20
HR_DEFAULT_TIMEOUT_US = 1_000_000
HR_DEFAULT_LINK_MBPS = 50_000
HR_LINK_UNPACED = 0xFFFFFFFF
HR_LINK_CALIBRATE = 0xFFFFFFFE
HR_MIN_LINK_MBPS = 100
HR_ALGO_AUTO = 0
HR_ALGO_ONE_SHOT = 1
HR_ALGO_TWO_SHOT = 2
HR_ALGO_LL = 3

# Every symbol include/hr.h declares.
EXPORTS = ("hr_create_channel", "hr_allreduce_f16", "hr_reduce_f16", "hr_channel_status",
           "hr_channel_abort", "hr_channel_get_info", "hr_destroy", "hr_status_str",
           "hr_loopback_stream_create", "hr_loopback_stream_destroy",
           "hr_reduce_bf16", "hr_allreduce_bf16", "hr_admit", "hr_route_str", "hr_decode_numel",
           "hr_workspace_stride", "hr_exchange_algorithm", "hr_allreduce_group_f16",
           "hr_allreduce_group_bf16", "hr_allreduce_group_noalloc_f16", "hr_channel_timeout_info")

HR_ROUTE_HOST = 0
HR_DECLINE_DISABLED = 1
HR_DECLINE_DTYPE = 2
HR_DECLINE_WORLD_SIZE = 3
HR_DECLINE_PEER_ACCESS = 4
HR_DECLINE_TOO_LARGE = 5
HR_DTYPE_F16 = 0
HR_DTYPE_BF16 = 1
HR_DTYPE_OTHER = 2


class hr_channel_config(ctypes.Structure):
    _fields_ = [("device", ctypes.c_int),
                ("world_size", ctypes.c_int),
                ("max_numel", ctypes.c_size_t),
                ("num_blocks", ctypes.c_int),
                ("timeout_us", ctypes.c_uint32),
                ("algorithm", ctypes.c_int),
                ("link_mbps", ctypes.c_uint32)]


class hr_admit_policy(ctypes.Structure):
    _fields_ = [("enabled", ctypes.c_int),
                ("max_bytes", ctypes.c_size_t),
                ("allow_bf16", ctypes.c_int),
                ("max_world", ctypes.c_int)]


class hr_channel_info(ctypes.Structure):
    _fields_ = [("device", ctypes.c_int),
                ("world_size", ctypes.c_int),
                ("max_numel", ctypes.c_size_t),
                ("num_blocks", ctypes.c_int),
                ("block_threads", ctypes.c_int),
                ("timeout_us", ctypes.c_uint32),
                ("host_slots", ctypes.c_void_p),
                ("slot_stride", ctypes.c_size_t),
                ("host_flags", ctypes.POINTER(ctypes.c_uint64)),
                ("flag_stride", ctypes.c_size_t),
                ("host_error", ctypes.POINTER(ctypes.c_uint32)),
                ("host_abort", ctypes.POINTER(ctypes.c_uint32)),
                ("algorithm", ctypes.c_int),
                ("host_reduced", ctypes.c_void_p),
                ("host_flags2", ctypes.POINTER(ctypes.c_uint64)),
                ("host_ll", ctypes.c_void_p),
                ("ll_stride", ctypes.c_size_t),
                ("link_mbps", ctypes.c_uint32),
                ("dev_epochs", ctypes.c_void_p)]


class HrError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {hr_status_str(status)} ({status})")


_lib = None


def load() -> ctypes.CDLL:
    """Load libhr.so from this package (raises ImportError if it is absent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m message_fp16_all_amd.build")
    # torch ships its own HIP runtime under the same soname as the system one;
    # whichever loads first serves the process.  Load torch's first (when
    # torch is installed), so that the library and torch share one runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    lib.hr_create_channel.argtypes = [ctypes.POINTER(hr_channel_config), ctypes.POINTER(vp)]
    lib.hr_allreduce_f16.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_size_t, vp]
    lib.hr_reduce_f16.argtypes = [ctypes.POINTER(vp), ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.hr_allreduce_bf16.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_size_t, vp]
    lib.hr_allreduce_group_f16.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_size_t, vp]
    lib.hr_allreduce_group_bf16.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_size_t, vp]
    lib.hr_allreduce_group_noalloc_f16.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int,
                                                   ctypes.c_size_t, vp, vp]
    lib.hr_reduce_bf16.argtypes = [ctypes.POINTER(vp), ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.hr_channel_status.argtypes = [vp]
    lib.hr_exchange_algorithm.argtypes = [vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int)]
    lib.hr_channel_abort.argtypes = [vp]
    lib.hr_channel_timeout_info.argtypes = [vp, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_uint32),
                                            ctypes.POINTER(ctypes.c_uint64)]
    lib.hr_channel_get_info.argtypes = [vp, ctypes.POINTER(hr_channel_info)]
    lib.hr_destroy.argtypes = [vp]
    lib.hr_loopback_stream_create.argtypes = [ctypes.c_int, ctypes.POINTER(vp)]
    lib.hr_loopback_stream_destroy.argtypes = [vp]
    lib.hr_status_str.argtypes = [ctypes.c_int]
    lib.hr_status_str.restype = ctypes.c_char_p
    lib.hr_admit.argtypes = [ctypes.POINTER(hr_admit_policy), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                             ctypes.c_size_t]
    lib.hr_route_str.argtypes = [ctypes.c_int]
    lib.hr_route_str.restype = ctypes.c_char_p
    lib.hr_decode_numel.argtypes = [ctypes.c_size_t, ctypes.c_size_t, ctypes.c_size_t]
    lib.hr_decode_numel.restype = ctypes.c_size_t
    lib.hr_workspace_stride.argtypes = [ctypes.c_size_t]
    lib.hr_workspace_stride.restype = ctypes.c_size_t
    for name in EXPORTS:
        if name not in ("hr_status_str", "hr_route_str", "hr_decode_numel", "hr_workspace_stride"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


# ------------------------------------------------------- the C entry points

def hr_status_str(status: int) -> str:
    return load().hr_status_str(int(status)).decode()


def hr_create_channel(device: int = 0, world_size: int = 2, max_numel: int = 0,
                      num_blocks: int = 0, timeout_us: int = 0, algorithm: int = 0,
                      link_mbps: int = 0) -> int:
    """Returns the channel handle (an integer address) or raises HrError."""
    cfg = hr_channel_config(device, world_size, max_numel, num_blocks, timeout_us, algorithm, link_mbps)
    h = ctypes.c_void_p()
    st = load().hr_create_channel(ctypes.byref(cfg), ctypes.byref(h))
    if st != HR_OK:
        raise HrError(st, "hr_create_channel")
    return h.value


def hr_allreduce_f16(ch: int, rank: int, in_ptr: int, out_ptr: int, numel: int,
                     stream: int) -> int:
    """Raw call; returns the hr_status code."""
    return load().hr_allreduce_f16(ch, rank, in_ptr, out_ptr, numel, stream)


def hr_reduce_f16(ptrs, G: int, out_ptr: int, numel: int, stream: int) -> int:
    """Raw call; ``ptrs`` is a sequence of G device addresses.  Returns hr_status."""
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    return load().hr_reduce_f16(arr, G, out_ptr, numel, stream)


def hr_allreduce_bf16(ch: int, rank: int, in_ptr: int, out_ptr: int, numel: int,
                      stream: int) -> int:
    """Raw call; returns the hr_status code."""
    return load().hr_allreduce_bf16(ch, rank, in_ptr, out_ptr, numel, stream)


def hr_allreduce_group_f16(ch: int, in_ptrs, out_ptrs, numel: int, stream: int) -> int:
    """Raw call; ``in_ptrs``/``out_ptrs`` are sequences of world_size device
    addresses (None for a null pointer).  Returns the hr_status code."""
    ins = (ctypes.c_void_p * max(1, len(in_ptrs)))(*in_ptrs)
    outs = (ctypes.c_void_p * max(1, len(out_ptrs)))(*out_ptrs)
    return load().hr_allreduce_group_f16(ch, ins, outs, numel, stream)


def hr_allreduce_group_bf16(ch: int, in_ptrs, out_ptrs, numel: int, stream: int) -> int:
    """As hr_allreduce_group_f16 for bfloat16 buffers."""
    ins = (ctypes.c_void_p * max(1, len(in_ptrs)))(*in_ptrs)
    outs = (ctypes.c_void_p * max(1, len(out_ptrs)))(*out_ptrs)
    return load().hr_allreduce_group_bf16(ch, ins, outs, numel, stream)


def hr_allreduce_group_noalloc_f16(in_ptrs, out_ptrs, world_size: int, numel: int, status_ptr,
                                   stream: int) -> int:
    """Raw call of the channel-free group all-reduce; ``status_ptr`` is a
    device address or None.  Returns the hr_status code."""
    ins = (ctypes.c_void_p * max(1, len(in_ptrs)))(*in_ptrs)
    outs = (ctypes.c_void_p * max(1, len(out_ptrs)))(*out_ptrs)
    return load().hr_allreduce_group_noalloc_f16(ins, outs, world_size, numel, status_ptr, stream)


def hr_reduce_bf16(ptrs, G: int, out_ptr: int, numel: int, stream: int) -> int:
    """Raw call; ``ptrs`` is a sequence of G device addresses.  Returns hr_status."""
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    return load().hr_reduce_bf16(arr, G, out_ptr, numel, stream)


def hr_channel_status(ch: int) -> int:
    return load().hr_channel_status(ch)


def hr_exchange_algorithm(ch: int, numel: int) -> int:
    """The HR_ALGO_* a call of numel values takes (raises HrError)."""
    algo = ctypes.c_int(-1)
    st = load().hr_exchange_algorithm(ch, numel, ctypes.byref(algo))
    if st != HR_OK:
        raise HrError(st, "hr_exchange_algorithm")
    return algo.value


def hr_channel_abort(ch: int) -> int:
    return load().hr_channel_abort(ch)


def hr_channel_timeout_info(ch: int):
    """(rank, peer_mask, call) of the channel's timeout record; rank is -1
    when nothing is recorded (raises HrError)."""
    rank, mask, call = ctypes.c_int(-1), ctypes.c_uint32(0), ctypes.c_uint64(0)
    st = load().hr_channel_timeout_info(ch, ctypes.byref(rank), ctypes.byref(mask), ctypes.byref(call))
    if st != HR_OK:
        raise HrError(st, "hr_channel_timeout_info")
    return rank.value, mask.value, call.value


def hr_channel_get_info(ch: int) -> hr_channel_info:
    info = hr_channel_info()
    st = load().hr_channel_get_info(ch, ctypes.byref(info))
    if st != HR_OK:
        raise HrError(st, "hr_channel_get_info")
    return info


def hr_destroy(ch: int) -> int:
    return load().hr_destroy(ch)


def hr_loopback_stream_create(device: int = 0) -> int:
    """Returns a hipStream_t (integer) that owns its hardware queue."""
    h = ctypes.c_void_p()
    st = load().hr_loopback_stream_create(device, ctypes.byref(h))
    if st != HR_OK:
        raise HrError(st, "hr_loopback_stream_create")
    return h.value


def hr_loopback_stream_destroy(stream: int) -> int:
    return load().hr_loopback_stream_destroy(stream)


def hr_admit(policy, dtype: int, world_size: int, peer_access: bool, numel: int) -> int:
    """Route code for one reduction; ``policy`` is an hr_admit_policy or None."""
    ref = ctypes.byref(policy) if policy is not None else None
    return load().hr_admit(ref, dtype, world_size, int(bool(peer_access)), numel)


def hr_route_str(route: int) -> str:
    return load().hr_route_str(int(route)).decode()


def hr_decode_numel(max_batch: int, tokens_per_request: int, hidden: int) -> int:
    return load().hr_decode_numel(max_batch, tokens_per_request, hidden)


def hr_workspace_stride(numel: int) -> int:
    """Values between consecutive contributions in one fold workspace."""
    return load().hr_workspace_stride(numel)


def workspace(G: int, numel: int, dtype=None, device=0):
    """A device buffer holding G contributions in the hr_workspace_stride
    layout; returns (buffer, [view of contribution g])."""
    import torch
    dtype = torch.float16 if dtype is None else dtype
    stride = hr_workspace_stride(numel)
    buf = torch.empty(G * stride, dtype=dtype, device=torch.device("cuda", device))
    return buf, [buf[g * stride:g * stride + numel] for g in range(G)]


# ----------------------------------------------------- torch marshalling
#
# An eager call's host time is HIP's kernel launch (about 3 us) plus this
# marshalling, so the per-call helpers keep to attribute reads: torch and its
# two element types are looked up once, dtypes are compared by identity
# (torch dtypes are singletons), and a Channel binds its entry points once.
# Measured on MI355X, host time per enqueued Channel.allreduce: 4.62-4.76 us
# with an import and equality compares per call, 4.22-4.33 us as here, and
# 3.28-3.76 us for the bare ctypes call.

_torch = None
_F16 = None
_BF16 = None


def _tm():
    """The torch module, imported on first use (with its two dtypes)."""
    global _torch, _F16, _BF16
    if _torch is None:
        import torch
        _F16, _BF16 = torch.float16, torch.bfloat16
        _torch = torch
    return _torch


def _check(st: int, where: str):
    if st != HR_OK:
        raise HrError(st, where)


def _f16_ptr(t, name: str, dtype=None) -> int:
    if _torch is None:
        _tm()
    want = _F16 if dtype is None else dtype
    if t.dtype is not want:
        raise TypeError(f"{name}: expected {want}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return t.data_ptr()


def _stream_handle(stream, tensor=None) -> int:
    """The hipStream_t of ``stream``; for None, torch's current stream on the
    device of ``tensor`` (or the current device).  torch's raw query returns
    the handle without building a Stream object, which costs more than the
    library call itself; the public call is the fallback."""
    if stream is not None:
        return stream.cuda_stream
    torch = _tm()
    dev = tensor.get_device() if tensor is not None else torch.cuda.current_device()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return int(raw(dev))
    return int(torch.cuda.current_stream(dev).cuda_stream)


def reduce(tensors, out, stream=None):
    """out = left fold of ``tensors`` (all torch.float16, or all
    torch.bfloat16, same numel) on ``stream``."""
    _tm()
    n = out.numel()
    bf = out.dtype is _BF16
    dt = _BF16 if bf else _F16
    ptrs = []
    for i, t in enumerate(tensors):
        if t.numel() != n:
            raise ValueError(f"tensors[{i}] has {t.numel()} values, out has {n}")
        ptrs.append(_f16_ptr(t, f"tensors[{i}]", dt))
    fn, name = (hr_reduce_bf16, "hr_reduce_bf16") if bf else (hr_reduce_f16, "hr_reduce_f16")
    _check(fn(ptrs, len(ptrs), _f16_ptr(out, "out", dt), n, _stream_handle(stream, out)), name)
    return out


def allreduce_group_noalloc(ins, outs, status=None, stream=None):
    """Every rank's call in one launch without a channel
    (hr_allreduce_group_noalloc_f16): ``ins[r]``/``outs[r]`` are rank r's
    torch.float16 tensors; ``status``, if given, a one-element torch.int32
    (or uint32) device tensor that receives the call's status."""
    W = len(ins)
    if len(outs) != W:
        raise ValueError("ins and outs differ in length")
    n = ins[0].numel()
    for r in range(W):
        if ins[r].numel() != n or outs[r].numel() != n:
            raise ValueError(f"rank {r}: every input and output must hold {n} values")
    ip = [_f16_ptr(t, f"ins[{r}]") for r, t in enumerate(ins)]
    op = [_f16_ptr(t, f"outs[{r}]") for r, t in enumerate(outs)]
    sp = None
    if status is not None:
        if status.numel() < 1 or status.element_size() != 4 or not status.is_cuda:
            raise TypeError("status: expected a 4-byte device tensor")
        sp = status.data_ptr()
    _check(hr_allreduce_group_noalloc_f16(ip, op, W, n, sp, _stream_handle(stream, outs[0])),
           "hr_allreduce_group_noalloc_f16")
    return outs


class Channel:
    """An owned channel of ``world_size`` ranks; ``allreduce`` enqueues one
    rank's call."""

    def __init__(self, device: int = 0, max_numel: int = 0, num_blocks: int = 0,
                 timeout_us: int = 0, world_size: int = 2, algorithm: int = 0, link_mbps: int = 0):
        self.world_size = world_size
        self.handle = hr_create_channel(device, world_size, max_numel, num_blocks, timeout_us,
                                        algorithm, link_mbps)
        lib = load()
        _tm()
        # the per-rank entry point of each element type, bound once
        self._per_rank = {_F16: (lib.hr_allreduce_f16, "hr_allreduce_f16"),
                          _BF16: (lib.hr_allreduce_bf16, "hr_allreduce_bf16")}

    def allreduce(self, rank: int, inp, out, stream=None):
        """One rank's call; torch.float16 or torch.bfloat16 tensors.

        In loopback every rank's call must be in flight at once, on streams
        from ``LoopbackStreams``.  Those streams are ordered with the null
        stream (they are not non-blocking), so work on the null stream --
        torch's default stream included -- enqueued between the ranks'
        calls of one all-reduce holds back the ranks launched after it while
        the others spin: the call ends at the channel's watchdog with the
        sticky HR_ERR_TIMEOUT.  Enqueue nothing on the null stream between
        the ranks' calls, or use ``allreduce_group``."""
        n = inp.numel()
        if out.numel() != n:
            raise ValueError("in and out differ in numel")
        dt = inp.dtype
        fn, name = self._per_rank.get(dt, self._per_rank[_F16])
        if dt is not _BF16:
            dt = _F16                     # anything else is refused as not float16
        st = fn(self.handle, rank, _f16_ptr(inp, "in", dt), _f16_ptr(out, "out", dt), n,
                _stream_handle(stream, out))
        if st != HR_OK:
            raise HrError(st, self._where(name, st))
        return out

    def _where(self, name: str, st: int) -> str:
        """The call's name, with the timeout record when the channel holds one."""
        if st != HR_ERR_TIMEOUT:
            return name
        info = self.timeout_info()
        if info is None:
            return name
        rank, missing, call = info
        return f"{name} (rank {rank} waited at call {call} for ranks {missing})"

    def allreduce_group(self, ins, outs, stream=None):
        """Every rank's call in one launch (loopback): ``ins[r]``/``outs[r]``
        are rank r's torch.float16 or torch.bfloat16 tensors."""
        if len(ins) != self.world_size or len(outs) != self.world_size:
            raise ValueError(f"expected {self.world_size} inputs and outputs")
        n = ins[0].numel()
        bf = ins[0].dtype is _BF16
        dt = _BF16 if bf else _F16
        for r in range(self.world_size):
            if ins[r].numel() != n or outs[r].numel() != n:
                raise ValueError(f"rank {r}: every input and output must hold {n} values")
        ip = [_f16_ptr(t, f"ins[{r}]", dt) for r, t in enumerate(ins)]
        op = [_f16_ptr(t, f"outs[{r}]", dt) for r, t in enumerate(outs)]
        fn, name = ((hr_allreduce_group_bf16, "hr_allreduce_group_bf16") if bf
                    else (hr_allreduce_group_f16, "hr_allreduce_group_f16"))
        st = fn(self.handle, ip, op, n, _stream_handle(stream, outs[0]))
        if st != HR_OK:
            raise HrError(st, self._where(name, st))
        return outs

    def status(self) -> int:
        return hr_channel_status(self.handle)

    def abort(self):
        _check(hr_channel_abort(self.handle), "hr_channel_abort")

    def timeout_info(self):
        """After HR_ERR_TIMEOUT: (rank whose wait expired, [ranks whose
        publish never arrived], call number), or None if nothing is
        recorded."""
        rank, mask, call = hr_channel_timeout_info(self.handle)
        if rank < 0:
            return None
        return rank, [q for q in range(self.world_size) if (mask >> q) & 1], call

    def info(self) -> hr_channel_info:
        return hr_channel_get_info(self.handle)

    def algorithm_for(self, numel: int) -> int:
        """The HR_ALGO_* a call of numel values on this channel takes."""
        return hr_exchange_algorithm(self.handle, numel)

    def destroy(self):
        if self.handle:
            st = hr_destroy(self.handle)
            self.handle = None
            _check(st, "hr_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.destroy()


class LoopbackStreams:
    """One stream per rank of a loopback channel, each owning its hardware
    queue (see hr_loopback_stream_create), wrapped as torch streams."""

    def __init__(self, device: int = 0, n: int = 2):
        import torch
        self.handles = [hr_loopback_stream_create(device) for _ in range(n)]
        self.streams = tuple(torch.cuda.ExternalStream(h, device=torch.device("cuda", device))
                             for h in self.handles)

    def __getitem__(self, i):
        return self.streams[i]

    def __iter__(self):
        return iter(self.streams)

    def __len__(self):
        return len(self.streams)

    def destroy(self):
        for s in self.streams:
            s.synchronize()
        for h in self.handles:
            _check(hr_loopback_stream_destroy(h), "hr_loopback_stream_destroy")
        self.handles = []
