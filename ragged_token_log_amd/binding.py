"""Thin ctypes binding over liblogprob (argument marshalling only).

Every step of the computation runs in the library: the host plan in its C++
code and everything per logit in its HIP kernels.  PyTorch is used here for
device memory and the stream, nothing else.  If the library is not built,
loading raises immediately; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblogprob.so")

STATUS_NAMES = {
    0: "LP_OK", 1: "LP_ERR_NULL_ARG", 2: "LP_ERR_OFFSETS", 3: "LP_ERR_SHAPE",
    4: "LP_ERR_TOP_N_NEGATIVE", 5: "LP_ERR_TOP_N_TOO_LARGE", 6: "LP_ERR_ECHO_NEEDS_LOGITS",
    7: "LP_ERR_TOKEN_RANGE", 8: "LP_ERR_UNSUPPORTED", 9: "LP_ERR_WORKSPACE",
    10: "LP_ERR_HIP", 11: "LP_ERR_NOMEM", 12: "LP_ERR_TEMPERATURE", 13: "LP_ERR_TOP_K",
}

# every symbol include/liblogprob.h declares
EXPORTED = (
    "lp_plan_ragged", "lp_plan_get_info", "lp_plan_set_split", "lp_plan_set_waves",
    "lp_plan_set_depth", "lp_plan_set_deterministic", "lp_plan_set_temperature",
    "lp_plan_set_top_k", "lp_plan_descriptors",
    "lp_assemble_ragged",
    "lp_stage_ragged", "lp_launch_ragged", "lp_compute_ragged", "lp_compute_ragged_noalloc",
    "lp_shard_records",
    "lp_merge_shards", "lp_plan_destroy",
    "lp_status_string", "lp_last_hip_error", "lp_bench_stream_read",
    "lp_bench_stream_read_shape",
)

LEVELS = 3          # default heap depth: 8 columns, top_n <= 7
MAX_LEVELS = 6      # 64 columns
COLUMNS = 8         # columns at the default levels
MAX_TOP_N = 7
PAD_ID = 0xFFFFFFFF


class LogprobError(RuntimeError):
    """A non-OK lp_status from the library."""

    def __init__(self, code: int, where: str, hip_error: int = 0):
        self.code = code
        self.name = STATUS_NAMES.get(code, f"status {code}")
        extra = f" (hipError {hip_error})" if hip_error else ""
        super().__init__(f"{where}: {self.name}{extra}")


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_uint32), ("vocab", ctypes.c_uint32),
        ("levels", ctypes.c_uint32), ("columns", ctypes.c_uint32),
        ("out_rows", ctypes.c_uint64), ("read_rows", ctypes.c_uint64),
        ("split", ctypes.c_uint32), ("has_logits", ctypes.c_uint32),
        ("waves", ctypes.c_uint32), ("depth", ctypes.c_uint32),
        ("workspace_bytes", ctypes.c_uint64),
        ("direct_rows", ctypes.c_uint32), ("record_words", ctypes.c_uint32),
        ("deterministic", ctypes.c_uint32),
    ]


_lib = None


def load():
    """Loads liblogprob.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m ragged_token_log_amd.build` "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    vp, u32, u64, i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32
    P = ctypes.POINTER
    # host arrays go in as plain addresses (numpy's .ctypes.data)
    lib.lp_plan_ragged.argtypes = [u32, u32, u32, vp, vp, vp, ctypes.c_int, u64, P(vp), vp,
                                   P(u64), P(u64)]
    lib.lp_plan_get_info.argtypes = [vp, P(PlanInfo)]
    lib.lp_plan_set_split.argtypes = [vp, u32]
    lib.lp_plan_set_waves.argtypes = [vp, u32]
    lib.lp_plan_set_depth.argtypes = [vp, u32]
    lib.lp_plan_set_deterministic.argtypes = [vp, ctypes.c_int]
    lib.lp_plan_set_temperature.argtypes = [vp, vp]
    lib.lp_plan_set_top_k.argtypes = [vp, vp]
    lib.lp_plan_descriptors.argtypes = [vp, vp, vp, vp]
    lib.lp_assemble_ragged.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.lp_stage_ragged.argtypes = [vp, vp, vp, vp, u64, vp]
    lib.lp_launch_ragged.argtypes = [vp, vp, vp, vp, vp, vp, u64, vp]
    lib.lp_compute_ragged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, u64, vp]
    lib.lp_compute_ragged_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
    lib.lp_shard_records.argtypes = [vp, u32, u32, vp, vp, vp, vp, u64, vp]
    lib.lp_merge_shards.argtypes = [vp, u32, vp, vp, vp, vp, u64, vp]
    lib.lp_plan_destroy.argtypes = [vp]
    lib.lp_plan_destroy.restype = None
    lib.lp_status_string.argtypes = [ctypes.c_int]
    lib.lp_status_string.restype = ctypes.c_char_p
    lib.lp_last_hip_error.argtypes = []
    lib.lp_bench_stream_read.argtypes = [vp, u32, u32, vp, vp]
    lib.lp_bench_stream_read_shape.argtypes = [vp, u32, u32, u32, u32, u32, vp, vp]
    for name in ("lp_plan_ragged", "lp_plan_get_info", "lp_plan_set_split",
                 "lp_plan_set_waves", "lp_plan_set_depth", "lp_plan_set_deterministic",
                 "lp_plan_set_temperature",
                 "lp_plan_set_top_k",
                 "lp_plan_descriptors", "lp_assemble_ragged",
                 "lp_stage_ragged", "lp_launch_ragged", "lp_shard_records", "lp_merge_shards",
                 "lp_compute_ragged", "lp_compute_ragged_noalloc", "lp_bench_stream_read",
                 "lp_bench_stream_read_shape", "lp_last_hip_error"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        hip = load().lp_last_hip_error() if status == 10 else 0
        raise LogprobError(status, where, hip)


def _ints(a, dtype, lo, hi, code, what):
    """``a`` as a contiguous array of ``dtype``.  Raises LogprobError(code)
    when an entry lies outside [lo, hi], and LP_ERR_SHAPE when one is not a
    whole number: a plain cast would wrap or truncate it into a different,
    valid-looking value."""
    arr = np.asarray(a)
    if arr.size:
        if arr.dtype.kind == "f":
            if not np.all(np.isfinite(arr)) or not np.all(np.floor(arr) == arr):
                raise LogprobError(3, f"{what} must hold whole numbers")
        elif arr.dtype.kind not in "iub":
            raise LogprobError(3, f"{what} must hold integers")
        if arr.min() < lo or arr.max() > hi:
            raise LogprobError(code, f"{what} outside [{lo}, {hi}]")
    return np.ascontiguousarray(arr, dtype=dtype)


def _u32(a, n=None, what="tokens"):
    """A 1-D uint32 copy of the host id array ``a`` (None stays None); with
    ``n`` given it must hold exactly n entries, because the library reads
    that many (LP_ERR_SHAPE otherwise)."""
    if a is None:
        return None
    ndim = np.ndim(a)   # before the copy, which makes a scalar 1-D
    arr = _ints(a, np.uint32, 0, 0xFFFFFFFF, 7, what)
    if n is not None and (ndim != 1 or arr.shape[0] != n):
        raise LogprobError(3, f"{what} must be 1-D with {n} entries, got shape {arr.shape}")
    return arr


def _ptr(arr, ctype=None):
    """The address of a contiguous host array (None for NULL); ``ctype``
    only names the element type the C side expects.  Read from the array
    interface: ``arr.ctypes`` builds a helper object per call."""
    return None if arr is None else arr.__array_interface__["data"][0]


def _dev_ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream):
    return ctypes.c_void_p(stream.cuda_stream) if stream is not None else None


class Plan:
    """lp_plan_ragged: host planning for one ragged batch (no GPU needed)."""

    def __init__(self, input_row_offsets, batch_echo, batch_top_n, vocab: int,
                 has_logits: bool, logits_rows: int | None = None, levels: int = LEVELS):
        lib = load()
        off = _ints(input_row_offsets, np.uint32, 0, 0xFFFFFFFF, 2, "input_row_offsets")
        if off.ndim != 1 or off.shape[0] < 1:
            raise LogprobError(3, "input_row_offsets must be 1-D with batch+1 entries")
        batch = off.shape[0] - 1
        echo = np.ascontiguousarray(np.asarray(batch_echo, dtype=bool).astype(np.uint8))
        # clipped, not wrapped: the library still names a negative or too large top_n
        top_n = _ints(np.clip(np.asarray(batch_top_n), -1, 1 << 20) if np.size(batch_top_n)
                      else batch_top_n, np.int32, -1, 1 << 20, 3, "batch_top_n")
        if echo.shape[0] != batch or top_n.shape[0] != batch:
            raise LogprobError(3, "batch_echo / batch_top_n length != batch")
        if logits_rows is None:
            logits_rows = int(off[-1]) if has_logits else batch
        self._lib = lib
        self._h = ctypes.c_void_p()
        out_off = np.zeros(batch + 1, dtype=np.uint32)
        rows = ctypes.c_uint64()
        ws = ctypes.c_uint64()
        _check(lib.lp_plan_ragged(batch, int(vocab), int(levels), _ptr(off, ctypes.c_uint32),
                                  _ptr(echo, ctypes.c_uint8), _ptr(top_n, ctypes.c_int32),
                                  1 if has_logits else 0, int(logits_rows),
                                  ctypes.byref(self._h), _ptr(out_off, ctypes.c_uint32),
                                  ctypes.byref(rows), ctypes.byref(ws)), "lp_plan_ragged")
        self.batch = batch
        self.vocab = int(vocab)
        self.levels = int(levels)
        self.has_logits = bool(has_logits)
        self.out_off = out_off
        self.out_rows = int(rows.value)
        self.logits_rows = int(logits_rows)
        self.input_row_offsets = off
        self._columns = None
        self.record_words = int(self.info()["record_words"])   # fixed by the levels

    def _token_arrays(self, tokens, sampled_tokens):
        """The host id arrays as the library reads them: tokens (T =
        input_row_offsets[-1] entries, or None when no request echoes) and
        sampled_tokens (batch entries)."""
        tok = _u32(tokens, int(self.input_row_offsets[-1]), "tokens")
        smp = _u32(sampled_tokens, self.batch, "sampled_tokens")
        return tok, smp

    # ---------------------------------------------------------------- facts
    @property
    def columns(self) -> int:
        """Output columns per row (2^levels, one slot per lane)."""
        if self._columns is None:
            self._columns = int(self.info()["columns"])
        return self._columns

    def info(self) -> dict:
        inf = PlanInfo()
        _check(self._lib.lp_plan_get_info(self._h, ctypes.byref(inf)), "lp_plan_get_info")
        return {f: getattr(inf, f) for f, _ in PlanInfo._fields_}

    @property
    def workspace_bytes(self) -> int:
        return int(self.info()["workspace_bytes"])

    @property
    def split(self) -> int:
        return int(self.info()["split"])

    def set_split(self, split: int):
        _check(self._lib.lp_plan_set_split(self._h, int(split)), "lp_plan_set_split")

    def set_waves(self, waves: int):
        _check(self._lib.lp_plan_set_waves(self._h, int(waves)), "lp_plan_set_waves")

    def set_depth(self, depth: int):
        _check(self._lib.lp_plan_set_depth(self._h, int(depth)), "lp_plan_set_depth")

    def set_deterministic(self, deterministic: bool = True):
        """Bit-reproducible log-probabilities (a fixed chunk assignment) when
        true; by default the chunks go to whichever wave is free, which is
        faster and may change the last bits of a value between runs (ids,
        offsets and padding are exact either way)."""
        _check(self._lib.lp_plan_set_deterministic(self._h, 1 if deterministic else 0),
               "lp_plan_set_deterministic")

    def set_temperature(self, temperature):
        """Per-request temperatures (a scalar for all, a length-batch
        sequence, or None for 1)."""
        if temperature is None:
            _check(self._lib.lp_plan_set_temperature(self._h, None), "lp_plan_set_temperature")
            return
        t = np.asarray(temperature, dtype=np.float32)
        if t.ndim == 0:
            t = np.full(self.batch, t, dtype=np.float32)
        t = np.ascontiguousarray(t)
        if t.shape != (self.batch,):
            raise LogprobError(3, "temperature must be a scalar or one value per request")
        _check(self._lib.lp_plan_set_temperature(self._h, _ptr(t, ctypes.c_float)),
               "lp_plan_set_temperature")

    def set_top_k(self, top_k):
        """Per-request top-k front end (a scalar for all, a length-batch
        sequence, or None for none; 0 = none)."""
        if top_k is None:
            _check(self._lib.lp_plan_set_top_k(self._h, None), "lp_plan_set_top_k")
            return
        k = np.asarray(top_k, dtype=np.int64)
        if k.ndim == 0:
            k = np.full(self.batch, k)
        if k.shape != (self.batch,):
            raise LogprobError(3, "top_k must be a scalar or one value per request")
        k = np.ascontiguousarray(np.clip(k, -1, 1 << 20).astype(np.int32))
        _check(self._lib.lp_plan_set_top_k(self._h, _ptr(k, ctypes.c_int32)), "lp_plan_set_top_k")

    def descriptors(self, tokens, sampled_tokens) -> np.ndarray:
        """(R, 4) uint32, as the device reads them: logits row read, chosen
        token, top_n | k << 16 (k the top-k front end), fp32 bits of the
        temperature."""
        tok, smp = self._token_arrays(tokens, sampled_tokens)
        out = np.zeros((self.out_rows, 4), dtype=np.uint32)
        _check(self._lib.lp_plan_descriptors(self._h, _ptr(tok, ctypes.c_uint32),
                                             _ptr(smp, ctypes.c_uint32),
                                             _ptr(out, ctypes.c_uint32)), "lp_plan_descriptors")
        return out

    def assemble(self, lp, ids):
        """lp_assemble_ragged on host (R, C) outputs: per output row the
        (token, logprob) entries of its top dict in insertion order, as
        ``(tokens (R, C) uint32, logprobs (R, C) float32, counts (R,) uint32)``."""
        C = self.columns
        lp = np.ascontiguousarray(lp, dtype=np.float32)
        ids = np.ascontiguousarray(ids, dtype=np.uint32)
        if lp.shape != (self.out_rows, C) or ids.shape != (self.out_rows, C):
            raise LogprobError(3, "assemble: outputs must be (out_rows, columns)")
        toks = np.zeros((self.out_rows, C), dtype=np.uint32)
        vals = np.zeros((self.out_rows, C), dtype=np.float32)
        counts = np.zeros(self.out_rows, dtype=np.uint32)
        _check(self._lib.lp_assemble_ragged(self._h, _ptr(lp, ctypes.c_float), _ptr(ids, ctypes.c_uint32),
                                            _ptr(toks, ctypes.c_uint32), _ptr(vals, ctypes.c_float),
                                            _ptr(counts, ctypes.c_uint32)), "lp_assemble_ragged")
        return toks, vals, counts

    # ---------------------------------------------------------------- device work
    def _check_buffers(self, logits, next_token_logits, out_logprobs, out_token_ids):
        """The kernels read and write these tensors through bare pointers, so
        each given one must be a contiguous GPU tensor of the right element
        type holding at least what the plan reads or writes (LP_ERR_SHAPE
        otherwise); a missing one is left to the library (LP_ERR_NULL_ARG)."""
        src = logits if self.has_logits else next_token_logits
        rows = self.logits_rows if self.has_logits else self.batch
        _check_device_tensor(src, "logits" if self.has_logits else "next_token_logits",
                             (4,), rows * self.vocab)
        if self.out_rows > 0:
            n = self.out_rows * self.columns
            _check_device_tensor(out_logprobs, "out_logprobs", (4,), n, floating=True)
            _check_device_tensor(out_token_ids, "out_token_ids", (4,), n, floating=False)

    def stage(self, tokens, sampled_tokens, workspace, stream=None):
        tok, smp = self._token_arrays(tokens, sampled_tokens)
        _check(self._lib.lp_stage_ragged(self._h, _ptr(tok, ctypes.c_uint32),
                                         _ptr(smp, ctypes.c_uint32), _dev_ptr(workspace),
                                         _nbytes(workspace), _stream_ptr(stream)),
               "lp_stage_ragged")

    def launch(self, logits, next_token_logits, out_logprobs, out_token_ids, workspace,
               stream=None):
        self._check_buffers(logits, next_token_logits, out_logprobs, out_token_ids)
        _check(self._lib.lp_launch_ragged(self._h, _dev_ptr(logits), _dev_ptr(next_token_logits),
                                          _dev_ptr(out_logprobs), _dev_ptr(out_token_ids),
                                          _dev_ptr(workspace), _nbytes(workspace),
                                          _stream_ptr(stream)), "lp_launch_ragged")

    def launcher(self, logits, next_token_logits, out_logprobs, out_token_ids, workspace,
                 stream=None):
        """A zero-argument callable doing lp_launch_ragged with these buffers,
        its ctypes arguments converted once (for tight launch loops).  It
        holds references to the tensors, so their memory cannot go back to
        the caching allocator while the callable exists."""
        self._check_buffers(logits, next_token_logits, out_logprobs, out_token_ids)
        fn = self._lib.lp_launch_ragged
        args = (self._h, _dev_ptr(logits), _dev_ptr(next_token_logits), _dev_ptr(out_logprobs),
                _dev_ptr(out_token_ids), _dev_ptr(workspace), ctypes.c_uint64(_nbytes(workspace)),
                _stream_ptr(stream))
        keep = (logits, next_token_logits, out_logprobs, out_token_ids, workspace, self)

        def launch():
            st = fn(*args)
            if st != 0:
                _check(st, "lp_launch_ragged")
            return keep
        return launch

    def computer(self, logits, next_token_logits, tokens, sampled_tokens, out_logprobs,
                 out_token_ids, workspace, stream=None):
        """A zero-argument callable doing lp_compute_ragged (descriptor build
        and upload, then the launch) with these buffers, its arguments
        checked and converted once; it keeps the host id arrays and the
        tensors alive."""
        tok, smp = self._token_arrays(tokens, sampled_tokens)
        self._check_buffers(logits, next_token_logits, out_logprobs, out_token_ids)
        fn = self._lib.lp_compute_ragged
        args = (self._h, _dev_ptr(logits), _dev_ptr(next_token_logits), _ptr(tok), _ptr(smp),
                _dev_ptr(out_logprobs), _dev_ptr(out_token_ids), _dev_ptr(workspace),
                ctypes.c_uint64(_nbytes(workspace)), _stream_ptr(stream))
        keep = (tok, smp, logits, next_token_logits, out_logprobs, out_token_ids, workspace, self)

        def compute():
            st = fn(*args)
            if st != 0:
                _check(st, "lp_compute_ragged")
            return keep
        return compute

    def compute(self, logits, next_token_logits, tokens, sampled_tokens, out_logprobs,
                out_token_ids, workspace, stream=None):
        tok, smp = self._token_arrays(tokens, sampled_tokens)
        self._check_buffers(logits, next_token_logits, out_logprobs, out_token_ids)
        _check(self._lib.lp_compute_ragged(self._h, _dev_ptr(logits), _dev_ptr(next_token_logits),
                                           _ptr(tok, ctypes.c_uint32), _ptr(smp, ctypes.c_uint32),
                                           _dev_ptr(out_logprobs), _dev_ptr(out_token_ids),
                                           _dev_ptr(workspace), _nbytes(workspace),
                                           _stream_ptr(stream)), "lp_compute_ragged")

    def compute_noalloc(self, logits, next_token_logits, tokens, sampled_tokens, out_logprobs,
                        out_token_ids, stream=None):
        """lp_compute_ragged_noalloc: the same computation with the library's
        fixed device workspace (at most 4 MiB of workspace; no allocation).
        Up to 1984 output rows the descriptors go in launch arguments and the
        call waits for nothing; larger plans return after a synchronous
        descriptor copy.  The kernels run on ``stream``."""
        tok, smp = self._token_arrays(tokens, sampled_tokens)
        self._check_buffers(logits, next_token_logits, out_logprobs, out_token_ids)
        _check(self._lib.lp_compute_ragged_noalloc(self._h, _dev_ptr(logits),
                                                   _dev_ptr(next_token_logits),
                                                   _ptr(tok, ctypes.c_uint32),
                                                   _ptr(smp, ctypes.c_uint32),
                                                   _dev_ptr(out_logprobs), _dev_ptr(out_token_ids),
                                                   _stream_ptr(stream)),
               "lp_compute_ragged_noalloc")

    def noalloc_computer(self, logits, next_token_logits, tokens, sampled_tokens, out_logprobs,
                         out_token_ids, stream=None):
        """A zero-argument callable doing lp_compute_ragged_noalloc with these
        buffers, its arguments checked and converted once (for timing loops);
        it keeps the host id arrays and the tensors alive."""
        tok, smp = self._token_arrays(tokens, sampled_tokens)
        self._check_buffers(logits, next_token_logits, out_logprobs, out_token_ids)
        fn = self._lib.lp_compute_ragged_noalloc
        args = (self._h, _dev_ptr(logits), _dev_ptr(next_token_logits), _ptr(tok), _ptr(smp),
                _dev_ptr(out_logprobs), _dev_ptr(out_token_ids), _stream_ptr(stream))
        keep = (tok, smp, logits, next_token_logits, out_logprobs, out_token_ids, self)

        def compute():
            st = fn(*args)
            if st != 0:
                _check(st, "lp_compute_ragged_noalloc")
            return keep
        return compute

    def _shard_args(self, vocab_begin, shard_logits, shard_next_token_logits, records, workspace,
                    stream):
        t = shard_logits if self.has_logits else shard_next_token_logits
        if t is None or t.dim() != 2:
            raise LogprobError(3, "the shard's logits must be a 2-D tensor")
        width = int(t.shape[1])
        rows = self.logits_rows if self.has_logits else self.batch
        _check_device_tensor(t, "shard logits", (4,), rows * width, floating=True)
        if self.out_rows > 0:
            _check_device_tensor(records, "records", (8, 4, 2, 1),
                                 self.out_rows * self.record_words * 8, as_bytes=True)
        return (self._h, int(vocab_begin), width, _dev_ptr(shard_logits),
                _dev_ptr(shard_next_token_logits), _dev_ptr(records), _dev_ptr(workspace),
                ctypes.c_uint64(_nbytes(workspace)), _stream_ptr(stream))

    def shard_records(self, vocab_begin: int, shard_logits, shard_next_token_logits, records,
                      workspace, stream=None):
        """lp_shard_records: one record per output row for the vocabulary
        shard [vocab_begin, vocab_begin + width) whose logits (rows of
        ``width`` fp32, the shard's columns only) are given; ``records`` is a
        device tensor of out_rows * record_words 8-byte words."""
        _check(self._lib.lp_shard_records(*self._shard_args(vocab_begin, shard_logits,
                                                            shard_next_token_logits, records,
                                                            workspace, stream)),
               "lp_shard_records")

    def shard_records_launcher(self, vocab_begin: int, shard_logits, shard_next_token_logits,
                               records, workspace, stream=None):
        """A zero-argument callable doing lp_shard_records with these buffers,
        checked and converted once (for tight launch loops)."""
        fn = self._lib.lp_shard_records
        args = self._shard_args(vocab_begin, shard_logits, shard_next_token_logits, records,
                                workspace, stream)
        keep = (shard_logits, shard_next_token_logits, records, workspace, self)

        def launch():
            st = fn(*args)
            if st != 0:
                _check(st, "lp_shard_records")
            return keep
        return launch

    def _merge_args(self, num_shards, records, out_logprobs, out_token_ids, workspace, stream):
        if self.out_rows > 0:
            _check_device_tensor(records, "records", (8, 4, 2, 1),
                                 int(num_shards) * self.out_rows * self.record_words * 8,
                                 as_bytes=True)
        self._check_buffers(None, None, out_logprobs, out_token_ids)
        return (self._h, int(num_shards), _dev_ptr(records), _dev_ptr(out_logprobs),
                _dev_ptr(out_token_ids), _dev_ptr(workspace), ctypes.c_uint64(_nbytes(workspace)),
                _stream_ptr(stream))

    def merge_shards(self, num_shards: int, records, out_logprobs, out_token_ids, workspace,
                     stream=None):
        """lp_merge_shards over records laid out (num_shards, out_rows,
        record_words) in a device tensor."""
        _check(self._lib.lp_merge_shards(*self._merge_args(num_shards, records, out_logprobs,
                                                           out_token_ids, workspace, stream)),
               "lp_merge_shards")

    def merge_launcher(self, num_shards: int, records, out_logprobs, out_token_ids, workspace,
                       stream=None):
        """A zero-argument callable doing lp_merge_shards with these buffers,
        checked and converted once."""
        fn = self._lib.lp_merge_shards
        args = self._merge_args(num_shards, records, out_logprobs, out_token_ids, workspace, stream)
        keep = (records, out_logprobs, out_token_ids, workspace, self)

        def launch():
            st = fn(*args)
            if st != 0:
                _check(st, "lp_merge_shards")
            return keep
        return launch

    def close(self):
        if self._h is not None and self._h.value:
            self._lib.lp_plan_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def _check_device_tensor(t, name, itemsizes, need, floating=None, as_bytes=False):
    """A contiguous GPU tensor whose element size is in ``itemsizes`` (and
    floating point or not, when ``floating`` says) holding at least ``need``
    elements (bytes with ``as_bytes``); None passes (the library reports
    it).  LP_ERR_SHAPE otherwise."""
    if t is None:
        return
    if getattr(t, "device", None) is None or t.device.type != "cuda":
        raise LogprobError(3, f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise LogprobError(3, f"{name} must be contiguous")
    if t.element_size() not in itemsizes:
        raise LogprobError(3, f"{name} has {t.element_size()}-byte elements")
    if floating is not None and t.is_floating_point() != floating:
        raise LogprobError(3, f"{name} must be {'float32' if floating else 'an integer type'}")
    have = t.numel() * t.element_size() if as_bytes else t.numel()
    if have < need:
        raise LogprobError(3, f"{name} holds {have} {'bytes' if as_bytes else 'elements'}, "
                              f"the plan needs {need}")


def _nbytes(t) -> int:
    return 0 if t is None else int(t.numel() * t.element_size())


def stream_read_launcher(x, rows: int, row_len: int, partial, stream=None):
    """A zero-argument callable running the plain-read probe
    (lp_bench_stream_read) over ``rows`` rows of ``row_len`` floats of x."""
    lib = load()
    if x.numel() < rows * row_len or partial.numel() < rows:
        raise LogprobError(3, "x must hold rows * row_len floats and partial rows floats")
    args = (_dev_ptr(x), ctypes.c_uint32(rows), ctypes.c_uint32(row_len), _dev_ptr(partial),
            _stream_ptr(stream))
    keep = (x, partial)

    def launch():
        _check(lib.lp_bench_stream_read(*args), "lp_bench_stream_read")
        return keep
    return launch


def stream_read_shape_launcher(x, rows: int, row_len: int, segments: int, threads: int,
                               loads: int, partial, stream=None):
    """A zero-argument callable running the plain-read probe in another launch
    shape (lp_bench_stream_read_shape): ``segments`` workgroups of
    ``threads`` per row, ``loads`` 16-byte loads in flight per thread;
    ``partial`` holds rows * segments floats."""
    lib = load()
    if x.numel() < rows * row_len or partial.numel() < rows * segments:
        raise LogprobError(3, "x must hold rows * row_len floats and partial rows * segments")
    args = (_dev_ptr(x), ctypes.c_uint32(rows), ctypes.c_uint32(row_len),
            ctypes.c_uint32(segments), ctypes.c_uint32(threads), ctypes.c_uint32(loads),
            _dev_ptr(partial), _stream_ptr(stream))
    keep = (x, partial)

    def launch():
        _check(lib.lp_bench_stream_read_shape(*args), "lp_bench_stream_read_shape")
        return keep
    return launch


def status_string(code: int) -> str:
    return load().lp_status_string(int(code)).decode()


# -------------------------------------------------------------------- torch front end

def _check_logits(t, rows, vocab, name, torch):
    if t.dim() != 2:
        raise LogprobError(3, f"{name} must be 2-D")
    if t.dtype != torch.float32:
        raise LogprobError(3, f"{name} must be float32")
    if t.device.type != "cuda":
        raise LogprobError(3, f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise LogprobError(3, f"{name} must be contiguous")
    if rows is not None and t.shape[0] != rows:
        raise LogprobError(3, f"{name} has {t.shape[0]} rows, expected {rows}")
    if vocab is not None and t.shape[1] != vocab:
        raise LogprobError(3, f"{name} vocab {t.shape[1]} != {vocab}")


def alloc_outputs(plan: Plan, device, torch):
    lp = torch.empty((plan.out_rows, plan.columns), dtype=torch.float32, device=device)
    ids = torch.empty((plan.out_rows, plan.columns), dtype=torch.uint32, device=device)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=device)
    return lp, ids, ws


@dataclass
class LogProbabilities:
    """One request's result, with the fields of the MAX page's
    ``LogProbabilities`` (section "数据结构：可序列化的 LogProbabilities"):
    per output row, the chosen token's log-probability and the dict of top
    token ids to log-probabilities."""

    token_log_probabilities: list
    top_log_probabilities: list


def compute_log_probabilities_ragged(input_row_offsets, logits, next_token_logits, tokens,
                                     sampled_tokens, batch_top_n, batch_echo, *,
                                     split: int | None = None, waves: int | None = None,
                                     depth: int | None = None, stream=None,
                                     levels: int = LEVELS, temperature=None, top_k=None,
                                     deterministic: bool = False):
    """Ragged batched token log-probabilities on the GPU.

    Arguments follow the MAX page's ``compute_log_probabilities_ragged``
    (section "compute_log_probabilities_ragged：执行计算并组装结果"):
    ``logits`` (tokens, vocab) float32 on the GPU, or None when no request
    echoes; ``next_token_logits`` (batch, vocab) float32 on the GPU;
    ``input_row_offsets``, ``tokens``, ``sampled_tokens``, ``batch_top_n`` and
    ``batch_echo`` are host sequences.

    ``levels`` is the heap depth of the MAX page's graph (section
    "log_probabilities_ragged_graph"): C = 2**levels output columns (one at
    levels 0), top_n <= C - 1.  ``temperature`` (a scalar or one per
    request, each in [2^-126, 2^120]) gives log_softmax(logits /
    temperature); None means 1.
    ``top_k`` (a scalar or one per request, 0 or None = none, at most C - 1)
    adds the FlashInfer page's TopK-then-Softmax front end: the k best tokens
    are kept and the log-probabilities renormalised over them.
    ``deterministic`` makes the log-probability values bit-reproducible from
    run to run (lp_plan_set_deterministic); ids and offsets always are.

    Returns ``(logprobs (R, C) float32, token_ids (R, C) uint32,
    output_row_offsets (batch+1,) uint32 numpy)``, the tensors on the GPU.
    """
    import torch

    plan = _checked_plan(input_row_offsets, logits, next_token_logits, batch_top_n, batch_echo,
                         levels, temperature, top_k, torch, deterministic)
    try:
        lp, ids = _run(plan, logits, next_token_logits, tokens, sampled_tokens, split, waves,
                       depth, stream, torch)
        out_off = plan.out_off.copy()
    finally:
        plan.close()   # host memory only: the enqueued work does not depend on the plan
    return lp, ids, out_off


def _checked_plan(input_row_offsets, logits, next_token_logits, batch_top_n, batch_echo, levels,
                  temperature, top_k, torch, deterministic=False) -> Plan:
    """Checks the device tensors (2-D fp32 contiguous on one GPU, matching
    rows and vocabulary) and plans the batch with its options."""
    off = np.asarray(input_row_offsets)
    if off.ndim != 1:
        raise LogprobError(3, "input_row_offsets must be 1-D")
    batch = off.shape[0] - 1
    _check_logits(next_token_logits, batch, None, "next_token_logits", torch)
    vocab = int(next_token_logits.shape[1])
    if logits is not None:
        _check_logits(logits, None, vocab, "logits", torch)
        if logits.device != next_token_logits.device:
            raise LogprobError(3, "logits and next_token_logits on different devices")
    plan = Plan(off, batch_echo, batch_top_n, vocab, logits is not None,
                None if logits is None else int(logits.shape[0]), levels=levels)
    try:
        if temperature is not None:
            plan.set_temperature(temperature)
        if top_k is not None:
            plan.set_top_k(top_k)
        if deterministic:
            plan.set_deterministic(True)
    except BaseException:
        plan.close()
        raise
    return plan


def _run(plan, logits, next_token_logits, tokens, sampled_tokens, split, waves, depth, stream,
         torch):
    if split is not None:
        plan.set_split(split)
    if waves is not None:
        plan.set_waves(waves)
    if depth is not None:
        plan.set_depth(depth)
    device = next_token_logits.device
    if stream is None:
        stream = torch.cuda.current_stream(device)
    # Allocated on the launch stream: the caching allocator hands a freed
    # block (the workspace, dropped on return) only to later work on that
    # same stream, which runs after these kernels.
    with torch.cuda.stream(stream):
        lp, ids, ws = alloc_outputs(plan, device, torch)
    plan.compute(logits, next_token_logits, tokens, sampled_tokens, lp, ids, ws, stream)
    return lp, ids


def log_probabilities_ragged(input_row_offsets, logits, next_token_logits, tokens, sampled_tokens,
                             batch_top_n, batch_echo, *, levels: int = LEVELS, temperature=None,
                             top_k=None, stream=None, deterministic: bool = False):
    """The whole call of the MAX page's ``compute_log_probabilities_ragged``:
    the device computation, the copy back, and the host assembly
    (lp_assemble_ragged).  Returns one entry per request: None when its
    top_n is 0, else a LogProbabilities whose lists hold one item per output
    row of the request."""
    import torch

    plan = _checked_plan(input_row_offsets, logits, next_token_logits, batch_top_n, batch_echo,
                         levels, temperature, top_k, torch, deterministic)
    try:
        if stream is None:
            stream = torch.cuda.current_stream(next_token_logits.device)
        lp, ids = _run(plan, logits, next_token_logits, tokens, sampled_tokens, None, None, None,
                       stream, torch)
        stream.synchronize()
        lp_h, ids_h = lp.cpu().numpy(), ids.cpu().numpy()
        toks, vals, counts = plan.assemble(lp_h, ids_h)
        out_off = plan.out_off.copy()
    finally:
        plan.close()
    C = lp_h.shape[1]
    out = []
    for n, top_n in enumerate(np.asarray(batch_top_n)):
        if int(top_n) == 0:
            out.append(None)
            continue
        rows = range(int(out_off[n]), int(out_off[n + 1]))
        out.append(LogProbabilities(
            token_log_probabilities=[float(lp_h[o, C - 1]) for o in rows],
            top_log_probabilities=[{int(toks[o, k]): float(vals[o, k]) for k in range(int(counts[o]))}
                                   for o in rows]))
    return out
