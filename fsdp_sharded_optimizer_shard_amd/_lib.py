"""ctypes binding of libzeroshard (include/zero_shard.h).  Argument
marshalling only: every step of the path runs in the HIP library.

Buffers may be given as torch tensors (their data_ptr() is passed) or as raw
integer device addresses.  A tensor is checked before the call: its dtype,
that it is contiguous, and that it holds every element the call touches (from
the layout's unit range), so that an undersized buffer raises ValueError here
instead of being read or written past its end by a kernel.  Raw addresses are
passed as they are.  `stream` defaults to torch's current stream on the
current device.  Errors of the library raise ZeroShardError with its message.
There is no fallback: if the library is missing this module fails to import.
"""
import ctypes
import os
from typing import Optional, Sequence

# torch first: its ROCm build ships its own HIP runtime (same soname,
# libamdhip64.so.7).  Loading torch before the library makes the library bind
# to that runtime, so device pointers and streams from torch are valid in it;
# loading the library first would put a second HIP runtime in the process.
import torch  # noqa: E402,F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzeroshard.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run __graft_entry__.build() or "
        "python -m fsdp_sharded_optimizer_shard_amd.build")

_lib = ctypes.CDLL(LIB_PATH)

# enums (zero_shard.h)
OK, ERR_INVALID_ARG, ERR_ALIGNMENT, ERR_OOM, ERR_HIP, ERR_UNSUPPORTED = range(6)
DDP, STAGE1, STAGE2, STAGE3, FSDP, MEGATRON_DO = range(6)
BF16, FP32 = 0, 1
INDEX_FULL, INDEX_SHARD = 0, 1
K_INNER, K_OUTER = 0, 1
MIX_STEP_STREAMS, MIX_READS, MIX_WRITES = 0, 1, 2
MAX_RANKS_PER_CALL = 64
NOALLOC_MAX_PARTIALS = 524288
STATE_CHUNK_MIN, STATE_CHUNK_MAX = 4, 1 << 24     # zero_layout_chunk_state bounds
STATE_CHUNK_DEFAULT = 8192                         # the measured best on MI355X
GRAD_CHUNK_DEFAULT = 16384                         # chunked gradients, likewise

STRATEGY = {"ddp": DDP, "zero1": STAGE1, "zero1_allreduce": STAGE1, "zero2": STAGE2,
            "zero3": STAGE3, "fsdp": FSDP, "fsdp2": FSDP, "megatron_do": MEGATRON_DO}

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


class _Grads(ctypes.Structure):
    _fields_ = [("ptrs", ctypes.POINTER(ctypes.c_void_p)), ("index", ctypes.POINTER(ctypes.c_uint8)),
                ("n", _I32), ("dtype", _I32), ("index_all", _I32), ("chunk", _I32)]


class AdamCfg(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("decoupled", _I32), ("step", _I64)]


def adam_cfg(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, decoupled=False,
             step=1) -> AdamCfg:
    return AdamCfg(lr, beta1, beta2, eps, weight_decay, int(bool(decoupled)), int(step))


class AdamTableEntry(ctypes.Structure):
    _fields_ = [(k, ctypes.c_float) for k in ("lr", "beta1", "beta2", "eps", "weight_decay",
                                               "one_minus_beta1", "one_minus_beta2", "bias1",
                                               "bias2", "decay")] + \
               [("has_decay", _I32), ("decoupled", _I32)]


_lib.zero_shard_init.argtypes = [ctypes.POINTER(_P), _I32, _I32, _I32, _I32, ctypes.POINTER(_I64)]
_lib.zero_shard_init.restype = _I32
_lib.zero_shard_init_rows.argtypes = [ctypes.POINTER(_P), _I32, _I32, _I32, _I32,
                                      ctypes.POINTER(_I64), ctypes.POINTER(_I64)]
_lib.zero_shard_init_rows.restype = _I32
_lib.zero_layout_rows.argtypes = [_P, _I32] + [ctypes.POINTER(_I64)] * 3
_lib.zero_layout_rows.restype = _I32
_lib.zero_shard_destroy.argtypes = [_P]
_lib.zero_shard_destroy.restype = None
_lib.zero_layout_info.argtypes = [_P] + [ctypes.POINTER(_I64)] * 2 + [ctypes.POINTER(_I32)] * 4
_lib.zero_layout_info.restype = _I32
_lib.zero_layout_query.argtypes = [_P, _I32] + [ctypes.POINTER(_I64)] * 6
_lib.zero_layout_query.restype = _I32
_lib.zero_layout_chunk_state.argtypes = [_P, _I64, ctypes.POINTER(_P)]
_lib.zero_layout_chunk_state.restype = _I32
_lib.zero_layout_state.argtypes = [_P, ctypes.POINTER(_I64), ctypes.POINTER(_I64)]
_lib.zero_layout_state.restype = _I32
_lib.zero_reduce_shard.argtypes = [_P, _I32, _I32, ctypes.POINTER(_Grads), _P, _I32, _P, _I64,
                                   _P]
_lib.zero_reduce_shard.restype = _I32
_lib.zero_reduce_partials_count.argtypes = [_P, _I32, _I32]
_lib.zero_reduce_partials_count.restype = _I64
_lib.zero_clip_coef.argtypes = [_P, _I64, ctypes.c_float, _P, _P, _P]
_lib.zero_clip_coef.restype = _I32
_lib.zero_adam_step.argtypes = [_P, _I32, _I32, ctypes.POINTER(AdamCfg), _P, _I32, _P,
                                ctypes.POINTER(_Grads), _P, _P, _P, _P, _I32, _P]
_lib.zero_adam_step.restype = _I32
_lib.zero_adam_step_clip_noalloc.argtypes = [_P, _I32, _I32, ctypes.POINTER(AdamCfg),
                                             ctypes.c_float, ctypes.POINTER(_Grads), _P, _P, _P,
                                             _P, _P, _I32, _P, _P]
_lib.zero_adam_step_clip_noalloc.restype = _I32
_lib.zero_adam_table_fill.argtypes = [ctypes.POINTER(AdamCfg), _I64, _P]
_lib.zero_adam_table_fill.restype = _I32
_lib.zero_adam_step_table.argtypes = [_P, _I32, _I32, _P, _I64, _P, _P, _I32, _P,
                                      ctypes.POINTER(_Grads), _P, _P, _P, _P, _I32, _P]
_lib.zero_adam_step_table.restype = _I32
_lib.zero_step_advance.argtypes = [_P, _P]
_lib.zero_step_advance.restype = _I32
_lib.zero_gather_params.argtypes = [_P, _I32, _I32, ctypes.POINTER(ctypes.c_void_p), _I32, _P, _P]
_lib.zero_gather_params.restype = _I32


class _UnitIO(ctypes.Structure):
    _fields_ = [("rank_grads", ctypes.POINTER(ctypes.c_void_p)),
                ("peer_shards", ctypes.POINTER(ctypes.c_void_p)), ("unit_full", _P)]


_lib.zero_fsdp_sweep.argtypes = [_P, _I32, _I32, ctypes.POINTER(AdamCfg), _I32, _I32,
                                 ctypes.POINTER(_UnitIO), _P, _P, _P, _I32, _P, _P]
_lib.zero_fsdp_sweep.restype = _I32
_lib.zero_fsdp_sweep_table.argtypes = [_P, _I32, _I32, _P, _I64, _P, _I32, _I32,
                                       ctypes.POINTER(_UnitIO), _P, _P, _P, _I32, _P, _P]
_lib.zero_fsdp_sweep_table.restype = _I32
_lib.zero_gemm_bf16.argtypes = [_I64, _I64, _I64, _P, _I64, _I32, _P, _I64, _I32, _P, _I64, _I32,
                                _P]
_lib.zero_gemm_bf16.restype = _I32
_lib.zero_gemm_bf16_nt.argtypes = [_I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _I32, _P]
_lib.zero_gemm_bf16_nt.restype = _I32
_lib.zero_transpose_bf16.argtypes = [_I64, _I64, _P, _I64, _P, _I64, _P]
_lib.zero_transpose_bf16.restype = _I32
_lib.zero_fsdp_linear_forward.argtypes = [_P, _I32, ctypes.POINTER(ctypes.c_void_p), _I64, _P, _P,
                                          _P, _I32, _P]
_lib.zero_fsdp_linear_forward.restype = _I32
_lib.zero_fsdp_linear_backward.argtypes = [_P, _I32, ctypes.POINTER(ctypes.c_void_p), _I64, _P,
                                           _P, _P, _P, _I32, _P, _P]
_lib.zero_fsdp_linear_backward.restype = _I32
_lib.zero_stream_mix.argtypes = [_I32, ctypes.POINTER(ctypes.c_void_p), _I32, _P, _P, _P, _P,
                                 _I64, _I64, _I64, _P]
_lib.zero_stream_mix.restype = _I32
_lib.zero_grad_accumulate.argtypes = [_P, _P, _I64, _P]
_lib.zero_grad_accumulate.restype = _I32
_lib.zero_status_str.argtypes = [_I32]
_lib.zero_status_str.restype = ctypes.c_char_p
_lib.zero_last_error.argtypes = []
_lib.zero_last_error.restype = ctypes.c_char_p

EXPORTS = ("zero_shard_init", "zero_shard_init_rows", "zero_layout_rows", "zero_shard_destroy",
           "zero_layout_info", "zero_layout_query", "zero_layout_chunk_state", "zero_layout_state",
           "zero_reduce_shard",
           "zero_reduce_partials_count", "zero_clip_coef", "zero_adam_step",
           "zero_adam_step_clip_noalloc",
           "zero_adam_table_fill", "zero_adam_step_table", "zero_step_advance", "zero_gather_params",
           "zero_grad_accumulate", "zero_stream_mix", "zero_fsdp_sweep", "zero_fsdp_sweep_table", "zero_gemm_bf16",
           "zero_gemm_bf16_nt",
           "zero_transpose_bf16", "zero_fsdp_linear_forward", "zero_fsdp_linear_backward",
           "zero_status_str", "zero_last_error")


class ZeroShardError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        msg = _lib.zero_last_error().decode(errors="replace")
        super().__init__(f"{fn}: {_lib.zero_status_str(status).decode()} ({status}): {msg}")


def _check(status: int, fn: str) -> None:
    if status != OK:
        raise ZeroShardError(status, fn)


def _addr(x) -> Optional[int]:
    """Device address of a buffer: None, a raw int address, or a tensor that
    lives on the GPU (a host tensor's pointer would fault inside a kernel,
    so it is refused here)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if getattr(x, "is_cuda", True) is False:
        raise ValueError("buffers passed to libzeroshard must be GPU tensors (got one on "
                         f"{getattr(x, 'device', 'the host')})")
    return x.data_ptr()


_DTYPES = {
    "fp32": (torch.float32,),
    "fp64": (torch.float64,),
    "bf16": (torch.int16, torch.uint16, torch.bfloat16),   # bf16 bit patterns
    "int64": (torch.int64,),
}


def _need(x, what: str, count: Optional[int], kind: str) -> None:
    """A tensor argument must be of `kind`, contiguous, and hold at least
    `count` elements (bytes for kind "bytes").  None, raw addresses and an
    unknown count (an invalid range, reported by the library) pass."""
    if x is None or x.__class__ is int or not hasattr(x, "numel"):
        return
    if x.is_cuda is False:
        raise ValueError(f"{what}: buffers passed to libzeroshard must be GPU tensors (got one "
                         f"on {x.device})")
    if count is None:
        return
    if kind == "bytes":
        have = x.numel() * x.element_size()
    else:
        if x.dtype not in _DTYPES[kind]:
            raise ValueError(f"{what}: dtype {x.dtype}, expected one of "
                             f"{', '.join(str(d) for d in _DTYPES[kind])}")
        have = x.numel()
    if have < count:
        raise ValueError(f"{what} holds {have} {'bytes' if kind == 'bytes' else 'elements'}, "
                         f"the call touches {count}")
    if not x.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _kind(dtype: int) -> str:
    return "fp32" if dtype == FP32 else "bf16"


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Layout:
    """An owned zero_layout (host memory).  Use shard_init() to make one."""

    def __init__(self, handle: int, units: Sequence[int]):
        self._h = handle
        self.units = list(units)
        self._uq = None
        self._lens = {}
        self._state = None

    def _unit_table(self):
        """Every unit's query(), read once (a layout never changes)."""
        if self._uq is None:
            self._uq = [self.query(u) for u in range(self.info()["n_units"])]
        return self._uq

    def range_lens(self, unit_begin: int, unit_end: int):
        """(shard-indexed, full-indexed) element counts of a unit range, or
        (None, None) for a range the library will refuse."""
        key = (unit_begin, unit_end)
        r = self._lens.get(key)
        if r is None:
            r = self._lens[key] = self._range_lens(unit_begin, unit_end)
        return r

    def _range_lens(self, unit_begin, unit_end):
        q = self._unit_table()
        if not (0 <= unit_begin <= unit_end <= len(q)):
            return None, None
        if unit_begin == unit_end:
            return 0, 0
        a, b = q[unit_begin], q[unit_end - 1]
        return (b["shard_off"] + b["shard_len"] - a["shard_off"],
                b["flat_off"] + b["padded_len"] - a["flat_off"])

    @property
    def handle(self) -> int:
        if not self._h:
            raise ValueError("layout is destroyed")
        return self._h

    def destroy(self) -> None:
        if self._h and _lib is not None:   # _lib may already be gone at exit
            _lib.zero_shard_destroy(self._h)
        self._h = None

    __del__ = destroy

    def info(self) -> dict:
        f, s = _I64(), _I64()
        nu, wn, r, st = _I32(), _I32(), _I32(), _I32()
        _check(_lib.zero_layout_info(self.handle, ctypes.byref(f), ctypes.byref(s), ctypes.byref(nu),
                                     ctypes.byref(wn), ctypes.byref(r), ctypes.byref(st)),
               "zero_layout_info")
        return {"flat_len": f.value, "shard_len": s.value, "n_units": nu.value,
                "world_n": wn.value, "rank": r.value, "strategy": st.value}

    def query(self, unit: int) -> dict:
        v = [_I64() for _ in range(6)]
        _check(_lib.zero_layout_query(self.handle, unit, *[ctypes.byref(x) for x in v]),
               "zero_layout_query")
        keys = ("numel", "padded_len", "flat_off", "shard_len", "shard_off", "rank_flat_off")
        return dict(zip(keys, (x.value for x in v)))

    def rows(self, unit: int) -> dict:
        v = [_I64() for _ in range(3)]
        _check(_lib.zero_layout_rows(self.handle, unit, *[ctypes.byref(x) for x in v]),
               "zero_layout_rows")
        return dict(zip(("cols", "first_row", "row_count"), (x.value for x in v)))

    def chunk_state(self, chunk: int) -> "Layout":
        """A copy of this layout whose master, m and v form one buffer in
        chunks of `chunk` elements (0: three arrays); see state_views()."""
        h = _P()
        _check(_lib.zero_layout_chunk_state(self.handle, chunk, ctypes.byref(h)),
               "zero_layout_chunk_state")
        return Layout(h.value, self.units)

    def _state_format(self):
        if self._state is None:
            e, n = _I64(), _I64()
            _check(_lib.zero_layout_state(self.handle, ctypes.byref(e), ctypes.byref(n)),
                   "zero_layout_state")
            self._state = (e.value, n.value)
        return self._state

    @property
    def state_chunk(self) -> int:
        """0 for three state arrays, else the chunk E of the one state buffer."""
        return self._state_format()[0]

    @property
    def state_len(self) -> int:
        """Floats of the state: shard_len per array, or the chunked buffer's length."""
        return self._state_format()[1]

    def state_views(self, state):
        """(master, m, v) for a chunked layout: views of one state tensor of
        state_len floats starting at 0, E and 2E, as the library expects."""
        E = self.state_chunk
        if E == 0:
            raise ValueError("this layout keeps master, m and v as three arrays")
        if state.numel() != self.state_len:
            raise ValueError(f"state: expected {self.state_len} floats, got {state.numel()}")
        return state[0:], state[E:], state[2 * E:]

    def state_count(self, unit_begin: int, unit_end: int):
        """Floats each of master, m and v must hold from its pointer for a
        call over [unit_begin, unit_end), or None for a range the library
        will refuse.  A chunked state is addressed by absolute shard index."""
        shard, _ = self.range_lens(unit_begin, unit_end)
        E = self.state_chunk
        if shard is None or E == 0 or shard == 0:
            return shard
        last = self._unit_table()[unit_end - 1]
        i = last["shard_off"] + last["shard_len"] - 1     # highest shard index touched
        return (i // E) * 3 * E + i % E + 1

    def grad_count(self, unit_begin: int, unit_end: int, chunk: int):
        """Elements each rank's pointer into chunked gradients (chunk E) must
        reach for a call over [unit_begin, unit_end): the range's last
        element i sits at (i // E) N E + i % E (None as above)."""
        shard, _ = self.range_lens(unit_begin, unit_end)
        if shard is None or chunk == 0 or shard == 0:
            return shard
        i, E = shard - 1, chunk
        return (i // E) * self.info()["world_n"] * E + i % E + 1

    def grad_len(self, chunk: int, unit_begin: int = 0, unit_end: Optional[int] = None) -> int:
        """Elements of one buffer holding all N ranks' gradients for the
        range's part of this shard (the whole shard by default) in chunks of
        `chunk`: ceil(S / E) rows of N chunks."""
        if chunk <= 0:
            raise ValueError(f"chunk must be positive (got {chunk})")
        ue = self.info()["n_units"] if unit_end is None else unit_end
        shard, _ = self.range_lens(unit_begin, ue)
        if shard is None:
            raise ValueError(f"unit range [{unit_begin}, {ue}) is outside the layout")
        return -(-shard // chunk) * self.info()["world_n"] * chunk

    @property
    def flat_len(self) -> int:
        return self.info()["flat_len"]

    @property
    def shard_len(self) -> int:
        return self.info()["shard_len"]


def shard_init(strategy, world_n: int, rank: int, unit_numel: Sequence[int]) -> Layout:
    s = STRATEGY[strategy] if isinstance(strategy, str) else int(strategy)
    arr = (_I64 * len(unit_numel))(*[int(u) for u in unit_numel]) if len(unit_numel) else None
    h = _P()
    _check(_lib.zero_shard_init(ctypes.byref(h), s, world_n, rank, len(unit_numel), arr),
           "zero_shard_init")
    return Layout(h.value, unit_numel)


def shard_init_rows(strategy, world_n: int, rank: int, shapes) -> Layout:
    """FSDP2-style layout: one unit per (rows, cols) parameter."""
    s = STRATEGY[strategy] if isinstance(strategy, str) else int(strategy)
    n = len(shapes)
    rows = (_I64 * max(1, n))(*[int(r) for r, _ in shapes])
    cols = (_I64 * max(1, n))(*[int(c) for _, c in shapes])
    h = _P()
    _check(_lib.zero_shard_init_rows(ctypes.byref(h), s, world_n, rank, n, rows, cols),
           "zero_shard_init_rows")
    return Layout(h.value, [int(r) * int(c) for r, c in shapes])


class Grads:
    """Marshalled zero_grads; keeps its ctypes arrays alive."""

    def __init__(self, bufs, dtype: int = BF16, index=INDEX_FULL, chunk: int = 0):
        self._keep = list(bufs)              # keeps tensors alive; sliceable by callers
        ptrs = [_addr(b) for b in bufs]
        self._ptrs = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
        self._index = None
        idx_all = INDEX_FULL
        if isinstance(index, int):
            idx_all = index
        else:
            self._index = (ctypes.c_uint8 * len(index))(*[int(i) for i in index])
        self.s = _Grads(self._ptrs, self._index, len(ptrs), dtype, idx_all, chunk)
        self._checked = None

    @classmethod
    def chunked(cls, buf, n: int, chunk: int, dtype: int = BF16, full=None):
        """N ranks' shard-indexed gradients interleaved in one buffer in
        chunks of `chunk` elements (Layout.grad_len long): rank q's pointer
        is the buffer's start + q * chunk.  `full` maps ranks whose
        gradient is a full-indexed buffer of its own (a rank's own main
        gradient) to that buffer; their slots in `buf` are not read."""
        full = full or {}
        bufs = [full[q] if q in full else buf[q * chunk:] for q in range(n)]
        index = ([INDEX_FULL if q in full else INDEX_SHARD for q in range(n)] if full
                 else INDEX_SHARD)
        return cls(bufs, dtype, index, chunk)

    @property
    def chunk(self) -> int:
        return self.s.chunk

    def ref(self):
        return ctypes.byref(self.s)

    def check(self, layout, unit_begin: int, unit_end: int) -> None:
        """Each rank buffer holds what a call over [unit_begin, unit_end)
        reads from it.  The buffers of a Grads never change, so a range
        checked once is not checked again."""
        shard, full = layout.range_lens(unit_begin, unit_end)
        if self.chunk and shard is not None:
            shard = layout.grad_count(unit_begin, unit_end, self.chunk)
        lens = (shard, full)
        if lens == self._checked:
            return
        for q, b in enumerate(self._keep):
            mode = self.s.index_all if self._index is None else self._index[q]
            _need(b, f"gradient buffer of rank {q}", full if mode == INDEX_FULL else shard,
                  _kind(self.s.dtype))
        if None not in lens:
            self._checked = lens


def reduce_partials_count(layout: Layout, unit_begin: int, unit_end: int) -> int:
    return _lib.zero_reduce_partials_count(layout.handle, unit_begin, unit_end)


def reduce_shard(layout: Layout, unit_begin: int, unit_end: int, grads: Grads, out,
                 sumsq_partials=None, n_partials: int = 0, stream=None,
                 out_index: int = INDEX_SHARD) -> None:
    shard, full = layout.range_lens(unit_begin, unit_end)
    if grads is not None:
        grads.check(layout, unit_begin, unit_end)
    _need(out, "out", full if out_index == INDEX_FULL else shard, "fp32")
    _need(sumsq_partials, "sumsq_partials", n_partials, "fp64")
    _check(_lib.zero_reduce_shard(layout.handle, unit_begin, unit_end, grads.ref() if grads else None,
                                  _addr(out), out_index, _addr(sumsq_partials), n_partials,
                                  _stream(stream)),
           "zero_reduce_shard")


def clip_coef(partials, n: int, max_norm: float, coef_out, norm_out=None, stream=None) -> None:
    _need(partials, "partials", n, "fp64")
    _need(coef_out, "coef_out", 1, "fp32")
    _need(norm_out, "norm_out", 1, "fp64")
    _check(_lib.zero_clip_coef(_addr(partials), n, max_norm, _addr(coef_out), _addr(norm_out),
                               _stream(stream)), "zero_clip_coef")


def _check_step(layout, unit_begin, unit_end, master, m, v, param_out, param_index,
                grad_fp32=None, grad_index=INDEX_SHARD, clip_coef=None, grads=None):
    lens = layout.range_lens(unit_begin, unit_end)
    shard, full = lens
    sc = layout.state_count(unit_begin, unit_end)
    _need(master, "master", sc, "fp32")
    _need(m, "m", sc, "fp32")
    _need(v, "v", sc, "fp32")
    _need(param_out, "param_out", full if param_index == INDEX_FULL else shard, "bf16")
    if grad_fp32 is not None:
        _need(grad_fp32, "grad_fp32", full if grad_index == INDEX_FULL else shard, "fp32")
    if clip_coef is not None:
        _need(clip_coef, "clip_coef", 1, "fp32")
    if grads is not None:
        grads.check(layout, unit_begin, unit_end)


def adam_step(layout: Layout, unit_begin: int, unit_end: int, cfg: AdamCfg, master, m, v,
              param_out, param_index: int = INDEX_FULL, grad_fp32=None, clip_coef=None,
              grads: Optional[Grads] = None, stream=None, grad_index: int = INDEX_SHARD) -> None:
    _check_step(layout, unit_begin, unit_end, master, m, v, param_out, param_index, grad_fp32,
                grad_index, clip_coef, grads)
    _check(_lib.zero_adam_step(layout.handle, unit_begin, unit_end, ctypes.byref(cfg),
                               _addr(grad_fp32), grad_index, _addr(clip_coef),
                               grads.ref() if grads else None,
                               _addr(master), _addr(m), _addr(v), _addr(param_out), param_index,
                               _stream(stream)), "zero_adam_step")


def adam_step_clip_noalloc(layout: Layout, unit_begin: int, unit_end: int, cfg: AdamCfg,
                           max_norm: float, grads: Grads, grad_out, master, m, v, param_out,
                           param_index: int = INDEX_FULL, norm_out=None, stream=None) -> None:
    """The clipped two-pass step with the library's static scratch (no
    device allocation): reduce with partials, clip coefficient, Adam."""
    _check_step(layout, unit_begin, unit_end, master, m, v, param_out, param_index,
                grad_fp32=grad_out, grads=grads)
    _need(norm_out, "norm_out", 1, "fp64")
    _check(_lib.zero_adam_step_clip_noalloc(layout.handle, unit_begin, unit_end,
                                            ctypes.byref(cfg), max_norm,
                                            grads.ref() if grads else None, _addr(grad_out),
                                            _addr(master), _addr(m), _addr(v), _addr(param_out),
                                            param_index, _addr(norm_out), _stream(stream)),
           "zero_adam_step_clip_noalloc")


def adam_table(cfgs):
    """Host table of step scalars, one entry per configuration (entry k is
    used when the device step counter holds k + 1): an array of
    AdamTableEntry; bytes(table) is what goes to the device."""
    n = len(cfgs)
    arr = (AdamCfg * max(1, n))(*cfgs)
    out = (AdamTableEntry * max(1, n))()
    _check(_lib.zero_adam_table_fill(arr, n, out), "zero_adam_table_fill")
    return out


def adam_table_device(cfgs, device="cuda"):
    """adam_table(cfgs) copied into a device uint8 tensor."""
    import torch
    t = adam_table(cfgs)
    return torch.frombuffer(bytearray(bytes(t)), dtype=torch.uint8).to(device)


def adam_step_table(layout: Layout, unit_begin: int, unit_end: int, table, n_entries: int,
                    step_counter, master, m, v, param_out, param_index: int = INDEX_FULL,
                    grad_fp32=None, clip_coef=None, grads: Optional[Grads] = None, stream=None,
                    grad_index: int = INDEX_SHARD) -> None:
    _check_step(layout, unit_begin, unit_end, master, m, v, param_out, param_index, grad_fp32,
                grad_index, clip_coef, grads)
    _need(table, "table", n_entries * ctypes.sizeof(AdamTableEntry), "bytes")
    _need(step_counter, "step_counter", 1, "int64")
    _check(_lib.zero_adam_step_table(layout.handle, unit_begin, unit_end, _addr(table), n_entries,
                                     _addr(step_counter), _addr(grad_fp32), grad_index,
                                     _addr(clip_coef), grads.ref() if grads else None,
                                     _addr(master), _addr(m), _addr(v), _addr(param_out),
                                     param_index, _stream(stream)), "zero_adam_step_table")


def step_advance(step_counter, stream=None) -> None:
    _need(step_counter, "step_counter", 1, "int64")
    _check(_lib.zero_step_advance(_addr(step_counter), _stream(stream)), "zero_step_advance")


def gather_params(layout: Layout, unit_begin: int, unit_end: int, shards, param_full,
                  stream=None) -> None:
    shard, full = layout.range_lens(unit_begin, unit_end)
    for q, x in enumerate(shards):
        _need(x, f"shard of rank {q}", shard, "bf16")
    _need(param_full, "param_full", full, "bf16")
    ptrs = [_addr(s) for s in shards]
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    _check(_lib.zero_gather_params(layout.handle, unit_begin, unit_end, arr, len(ptrs),
                                   _addr(param_full), _stream(stream)), "zero_gather_params")


def _parts(layout: Layout) -> int:
    """Slices per unit: world_n, or 1 for a DDP layout."""
    i = layout.info()
    return 1 if i["strategy"] == DDP else i["world_n"]


def _need_len(what: str, seq, n: int) -> None:
    # The library reads exactly n entries of these host arrays; a shorter
    # list would have it read past the ctypes array.
    if len(seq) != n:
        raise ValueError(f"{what}: expected {n} entries, got {len(seq)}")


def _unit_ios(layout: Layout, unit_begin: int, unit_end: int, units, grad_dtype=BF16,
              grad_chunk=0):
    if 0 <= unit_begin <= unit_end:
        _need_len("units", units, unit_end - unit_begin)
        n, parts = layout.info()["world_n"], _parts(layout)
        table = layout._unit_table()
        for i, (grads, peers, full) in enumerate(units):
            _need_len("rank_grads", grads, n)
            _need_len("peer_shards", peers, parts)
            if unit_begin + i < len(table):
                u = unit_begin + i
                q = table[u]
                count = (layout.grad_count(u, u + 1, grad_chunk) if grad_chunk else
                         q["shard_len"])
                for k, x in enumerate(grads):
                    _need(x, f"unit {u} gradient of rank {k}", count, _kind(grad_dtype))
                for k, x in enumerate(peers):
                    _need(x, f"unit {unit_begin + i} shard of rank {k}", q["shard_len"], "bf16")
                _need(full, f"unit {unit_begin + i} buffer", q["padded_len"], "bf16")
    keep = []
    arr = (_UnitIO * max(1, len(units)))()
    for i, (grads, peers, full) in enumerate(units):
        g = (ctypes.c_void_p * max(1, len(grads)))(*[_addr(x) for x in grads])
        p = (ctypes.c_void_p * max(1, len(peers)))(*[_addr(x) for x in peers])
        keep += [g, p]
        arr[i] = _UnitIO(g, p, _addr(full))
    return arr, keep


def fsdp_sweep(layout: Layout, unit_begin: int, unit_end: int, cfg: AdamCfg, grad_dtype: int,
               units, master, m, v, max_inflight: int = 2, step_stream=None,
               gather_stream=None, grad_chunk: int = 0) -> None:
    """units: one (rank_grads, peer_shards, unit_full) per unit of the range;
    rank_grads are world_n buffers and peer_shards one per slice (world_n,
    or 1 under DDP; None allowed).  gather_stream defaults to step_stream
    (sequential).  grad_chunk E > 0: every unit's rank_grads are the
    pointers of one chunked receive buffer over the shard (Grads.chunked)."""
    arr, keep = _unit_ios(layout, unit_begin, unit_end, units, grad_dtype, grad_chunk)
    sc = layout.state_count(unit_begin, unit_end)
    for name, x in (("master", master), ("m", m), ("v", v)):
        _need(x, name, sc, "fp32")
    ss = _stream(step_stream)
    gs = ss if gather_stream is None else _stream(gather_stream)
    _check(_lib.zero_fsdp_sweep(layout.handle, unit_begin, unit_end, ctypes.byref(cfg), grad_dtype,
                                grad_chunk, arr, _addr(master), _addr(m), _addr(v), max_inflight,
                                ss, gs),
           "zero_fsdp_sweep")


def fsdp_sweep_table(layout: Layout, unit_begin: int, unit_end: int, table, n_entries: int,
                     step_counter, grad_dtype: int, units, master, m, v, max_inflight: int = 2,
                     step_stream=None, gather_stream=None, grad_chunk: int = 0) -> None:
    """fsdp_sweep with the step scalars of table[*step_counter - 1] (device
    table and counter); advances the counter once, after the last unit."""
    arr, keep = _unit_ios(layout, unit_begin, unit_end, units, grad_dtype, grad_chunk)
    sc = layout.state_count(unit_begin, unit_end)
    for name, x in (("master", master), ("m", m), ("v", v)):
        _need(x, name, sc, "fp32")
    _need(table, "table", n_entries * ctypes.sizeof(AdamTableEntry), "bytes")
    _need(step_counter, "step_counter", 1, "int64")
    ss = _stream(step_stream)
    gs = ss if gather_stream is None else _stream(gather_stream)
    _check(_lib.zero_fsdp_sweep_table(layout.handle, unit_begin, unit_end, _addr(table),
                                      n_entries, _addr(step_counter), grad_dtype, grad_chunk,
                                      arr,
                                      _addr(master), _addr(m), _addr(v), max_inflight, ss, gs),
           "zero_fsdp_sweep_table")


def _operand_extent(rows: int, K: int, ld: int, order: int) -> int:
    """Elements from an operand's start to its last one read."""
    if rows <= 0 or K <= 0:
        return 0
    return (rows - 1) * ld + K if order == K_INNER else (K - 1) * ld + rows


def gemm_bf16(M: int, N: int, K: int, A, lda: int, a_order: int, B, ldb: int, b_order: int, C,
              ldc: int, c_dtype: int = FP32, stream=None) -> None:
    if M > 0 and N > 0 and K >= 0:
        _need(A, "A", _operand_extent(M, K, lda, a_order), "bf16")
        _need(B, "B", _operand_extent(N, K, ldb, b_order), "bf16")
        _need(C, "C", (M - 1) * ldc + N, _kind(c_dtype))
    _check(_lib.zero_gemm_bf16(M, N, K, _addr(A), lda, a_order, _addr(B), ldb, b_order, _addr(C),
                               ldc, c_dtype, _stream(stream)), "zero_gemm_bf16")


def gemm_bf16_nt(M: int, N: int, K: int, A, lda: int, B, ldb: int, C, ldc: int,
                 c_dtype: int = FP32, stream=None) -> None:
    if M > 0 and N > 0 and K >= 0:
        _need(A, "A", _operand_extent(M, K, lda, K_INNER), "bf16")
        _need(B, "B", _operand_extent(N, K, ldb, K_INNER), "bf16")
        _need(C, "C", (M - 1) * ldc + N, _kind(c_dtype))
    _check(_lib.zero_gemm_bf16_nt(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc, c_dtype,
                                  _stream(stream)), "zero_gemm_bf16_nt")


def transpose_bf16(rows: int, cols: int, src, lds: int, dst, ldd: int, stream=None) -> None:
    if rows > 0 and cols > 0:
        _need(src, "src", (rows - 1) * lds + cols, "bf16")
        _need(dst, "dst", (cols - 1) * ldd + rows, "bf16")
    _check(_lib.zero_transpose_bf16(rows, cols, _addr(src), lds, _addr(dst), ldd, _stream(stream)),
           "zero_transpose_bf16")


def _ptrs(bufs):
    return (ctypes.c_void_p * max(1, len(bufs)))(*[_addr(b) for b in bufs])


def _layer_dims(layout: Layout, unit: int):
    """(in, out, shard, padded) of a linear layer's unit, or None if the unit
    does not exist (the library reports that)."""
    table = layout._unit_table()
    if not 0 <= unit < len(table):
        return None
    q = table[unit]
    cols = layout.rows(unit)["cols"]
    return q["numel"] // cols, cols, q["shard_len"], q["padded_len"]


def _check_layer(layout, unit, w_shards, w_full, batch):
    d = _layer_dims(layout, unit)
    if d is None or batch < 0:
        return None
    for q, x in enumerate(w_shards):
        _need(x, f"W shard of rank {q}", d[2], "bf16")
    _need(w_full, "w_full", d[3], "bf16")
    return d


def fsdp_linear_forward(layout: Layout, unit: int, w_shards, batch: int, x, w_full, y,
                        y_dtype: int = BF16, stream=None) -> None:
    _need_len("w_shards", w_shards, _parts(layout))
    d = _check_layer(layout, unit, w_shards, w_full, batch)
    if d is not None:
        _need(x, "x", batch * d[0], "bf16")
        _need(y, "y", batch * d[1], _kind(y_dtype))
    _check(_lib.zero_fsdp_linear_forward(layout.handle, unit, _ptrs(w_shards), batch, _addr(x),
                                         _addr(w_full), _addr(y), y_dtype, _stream(stream)),
           "zero_fsdp_linear_forward")


def fsdp_linear_backward(layout: Layout, unit: int, w_shards, batch: int, x, dy, w_full, dx,
                         dw_full, dx_dtype: int = BF16, stream=None) -> None:
    _need_len("w_shards", w_shards, _parts(layout))
    d = _check_layer(layout, unit, w_shards, w_full, batch)
    if d is not None:
        _need(x, "x", batch * d[0], "bf16")
        _need(dy, "dy", batch * d[1], "bf16")
        _need(dx, "dx", batch * d[0], _kind(dx_dtype))
        _need(dw_full, "dw_full", d[3], "fp32")
    _check(_lib.zero_fsdp_linear_backward(layout.handle, unit, _ptrs(w_shards), batch, _addr(x),
                                          _addr(dy), _addr(w_full), _addr(dx), dx_dtype,
                                          _addr(dw_full), _stream(stream)),
           "zero_fsdp_linear_backward")


def stream_mix(kind: int, grads, master, m, v, param, n: int, stream=None,
               state_chunk: int = 0, grad_chunk: int = 0) -> None:
    """zero_stream_mix: the fused step's memory traffic without its
    arithmetic (kind MIX_STEP_STREAMS), its reads alone (MIX_READS) or its
    writes alone (MIX_WRITES), over n elements; state_chunk E > 0 takes
    master, m, v in the chunked format (m = master + E, v = master + 2E),
    grad_chunk G > 0 the rank gradients chunked (grads[q] = grads[0] + qG)."""

    def count(E, k):
        return n if E <= 0 or n <= 0 else ((n - 1) // E) * k * E + (n - 1) % E + 1

    for q, x in enumerate(grads):
        _need(x, f"gradient buffer of rank {q}", count(grad_chunk, len(grads)), "bf16")
    sc = count(state_chunk, 3)
    for name, x in (("master", master), ("m", m), ("v", v)):
        _need(x, name, sc, "fp32")
    _need(param, "param", n, "bf16")
    _check(_lib.zero_stream_mix(kind, _ptrs(grads), len(grads), _addr(master), _addr(m), _addr(v),
                                _addr(param), n, state_chunk, grad_chunk, _stream(stream)),
           "zero_stream_mix")


def grad_accumulate(main_grad, micro_bf16, n: int, stream=None) -> None:
    _need(main_grad, "main_grad", n, "fp32")
    _need(micro_bf16, "micro_bf16", n, "bf16")
    _check(_lib.zero_grad_accumulate(_addr(main_grad), _addr(micro_bf16), n, _stream(stream)),
           "zero_grad_accumulate")


def raw():
    """The ctypes library object (for tests of the exported symbols)."""
    return _lib
