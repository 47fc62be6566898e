"""Thin ctypes binding of libfg.so (include/fg.h). Argument marshalling only:
every step of the path runs in the HIP library. torch is used for device
memory and streams. Importing this module does not need a GPU; creating a
Context does, and it fails loudly when the library is not built."""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libfg.so")

CHUNK_ROWS = 64
ROW_BLOCK = 128
MAX_SHARDS = 64
MAX_GROUPS = 64

OK, EINVAL, ENOMEM, EHIP, ERESIDENCY, ETIMEOUT, EPROTOCOL, ESTATE = 0, -1, -2, -3, -4, -5, -6, -7
CALL_COMM_ONLY = 1 << 0
CALL_GEMM_ONLY = 1 << 1
CALL_VERIFY = 1 << 2
CALL_STRICT = 1 << 3
CALL_SAME_ROUTE = 1 << 4
CALL_TRACE = 1 << 5
CALL_LAYOUT_TWO_PASS = 1 << 6
CALL_GATE_WATERMARK = 1 << 7
COUNTER_STRIDE = 64      # int32 per arrival counter in the control plane (FG_COUNTER_STRIDE)
FAULT_SEED_LOW = 1 << 8
FAULT_SEED_HIGH = 1 << 9
FAULT_DROP_PUBLISH = 1 << 10

ROUTE_CONTIG, ROUTE_EXPLICIT, ROUTE_TOPK = 0, 1, 2

EXPORTS = ("fg_init", "fg_gather_gemm", "fg_gather_gemm_staged", "fg_gather_gemm_ring", "fg_ring_bytes", "fg_barrier",
           "fg_pingpong", "fg_stress", "fg_combine", "fg_litmus", "fg_stats", "fg_views", "fg_capacity",
           "fg_gather_gemm_noalloc", "fg_destroy", "fg_strerror")


class FgConfig(C.Structure):
    _fields_ = [("n_shards", C.c_int32), ("max_rows_per_shard", C.c_int32), ("K", C.c_int32),
                ("N", C.c_int32), ("n_groups", C.c_int32), ("n_comm_wg", C.c_int32),
                ("n_gemm_wg", C.c_int32), ("tile_n", C.c_int32), ("timeout_ns", C.c_int64),
                ("stress_producers", C.c_int32), ("stress_consumers", C.c_int32),
                ("stress_max_chunks", C.c_int32), ("split_parts", C.c_int32), ("split_tiles", C.c_int32),
                ("tile_order", C.c_int32), ("copy_rows", C.c_int32), ("combine_wg", C.c_int32),
                ("copy_mode", C.c_int32)]


class FgRoute(C.Structure):
    _fields_ = [("mode", C.c_int32), ("rows_per_shard", C.c_int32),
                ("stream_len", C.POINTER(C.c_int32)), ("src_row", C.c_void_p), ("dst_row", C.c_void_p),
                ("m_pad", C.c_int32), ("group_off", C.POINTER(C.c_int32)),
                ("topk", C.c_void_p), ("topk_k", C.c_int32), ("expert_base", C.c_int32)]


class FgStats(C.Structure):
    _fields_ = [("seq", C.c_int32), ("bseq", C.c_int32), ("stress_seq", C.c_int32), ("m_pad", C.c_int32),
                ("error_code", C.c_int32), ("error_id", C.c_int32),
                ("publishes", C.c_int64), ("gate_polls", C.c_int64), ("slot_polls", C.c_int64),
                ("gate_passes", C.c_int64), ("stale", C.c_int64),
                ("t_kernel_us", C.c_double), ("t_comm_span_us", C.c_double), ("t_gemm_span_us", C.c_double),
                ("t_gemm_busy_us", C.c_double), ("t_gate_wait_us", C.c_double),
                ("t_barrier_us", C.c_double), ("t_rtt_us", C.c_double),
                ("n_comm_wg", C.c_int32), ("n_gemm_wg", C.c_int32), ("cu_count", C.c_int32),
                ("m_pad_cap", C.c_int32), ("tiles_whole", C.c_int32), ("tiles_split", C.c_int32),
                ("split_parts", C.c_int32), ("combine_seq", C.c_int32), ("clock_mhz", C.c_double),
                ("litmus_stale", C.c_int64), ("litmus_words", C.c_int64),
                ("expected_publishes", C.c_int64), ("timeouts", C.c_int64), ("max_wait_ns", C.c_int64),
                ("first_timeout_id", C.c_int32), ("copy_in_tiles", C.c_int32), ("lead_rows", C.c_int32),
                ("reserved4", C.c_int32)]


class FgViews(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("slot", "counter", "elect", "pub_count", "seed", "inv_row",
                                          "group_of_rb", "src_row", "dst_row", "stream_len", "group_off",
                                          "bslot", "stress_slot", "stress_pub")] + [
        ("chunk_cap", C.c_int32), ("rb_cap", C.c_int32), ("m_pad_cap", C.c_int32), ("route_ver", C.c_uint32),
        ("wg_time", C.c_void_p), ("trace", C.c_void_p), ("rb_time", C.c_void_p), ("grid", C.c_int32),
        ("trace_cap", C.c_int32), ("wall_khz", C.c_int64), ("desc", C.c_void_p), ("slab", C.c_void_p),
        ("group_slab", C.c_void_p), ("combine_slot", C.c_void_p), ("combine_elect", C.c_void_p),
        ("combine_pub", C.c_void_p), ("src_k", C.c_void_p), ("tok_first", C.c_void_p),
        ("ring_tail", C.c_void_p), ("ring_head", C.c_void_p), ("ring_cap", C.c_int32), ("reserved2", C.c_int32),
        ("src_of", C.c_void_p)]


class FgError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


_lib = None


def load_library() -> C.CDLL:
    """Load libfg.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(f"{LIB_PATH} is missing: build it with `python -m sync_protocols_amd.build`")
    lib = C.CDLL(LIB_PATH)
    vp = C.c_void_p
    lib.fg_init.argtypes = [C.POINTER(FgConfig), C.c_int, C.POINTER(vp)]
    lib.fg_gather_gemm.argtypes = [vp, C.POINTER(vp), C.POINTER(FgRoute), vp, vp, vp, C.c_uint32, vp]
    lib.fg_gather_gemm_staged.argtypes = [vp, C.POINTER(vp), C.POINTER(FgRoute), vp, C.POINTER(vp), C.c_int32,
                                          vp, vp, C.c_uint32, vp]
    lib.fg_gather_gemm_ring.argtypes = [vp, C.POINTER(vp), C.POINTER(FgRoute), vp, vp, C.c_int32, C.c_int32,
                                        C.c_int32, vp, vp, C.c_uint32, vp]
    lib.fg_ring_bytes.argtypes = [C.POINTER(FgConfig), C.c_int32, C.c_int32, C.POINTER(C.c_int64)]
    lib.fg_barrier.argtypes = [vp, C.c_int32, vp]
    lib.fg_pingpong.argtypes = [vp, C.c_int32, C.c_int32, vp]
    lib.fg_stress.argtypes = [vp, vp, vp, vp, C.c_uint32, vp]
    lib.fg_combine.argtypes = [vp, vp, vp, C.POINTER(vp), C.POINTER(vp), C.c_uint32, vp]
    lib.fg_litmus.argtypes = [vp, C.c_int32, C.c_int32, vp]
    lib.fg_stats.argtypes = [vp, C.POINTER(FgStats), C.c_int]
    lib.fg_views.argtypes = [vp, C.POINTER(FgViews)]
    lib.fg_capacity.argtypes = [C.POINTER(FgConfig), C.POINTER(C.c_int32)]
    lib.fg_gather_gemm_noalloc.argtypes = [C.POINTER(FgConfig), C.c_int, C.POINTER(vp), C.POINTER(FgRoute), vp,
                                           vp, vp, vp, C.c_uint32, vp]
    lib.fg_destroy.argtypes = [vp]
    lib.fg_strerror.argtypes = [C.c_int]
    lib.fg_strerror.restype = C.c_char_p
    for f in EXPORTS[:-1]:
        getattr(lib, f).restype = C.c_int
    _lib = lib
    return lib


def strerror(code: int) -> str:
    try:
        return load_library().fg_strerror(code).decode()
    except OSError:
        return str(code)


def _check(code: int, what: str) -> None:
    if code != OK:
        raise FgError(code, what)


def _stream_ptr(stream) -> C.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _ptr(t: torch.Tensor) -> C.c_void_p:
    return C.c_void_p(t.data_ptr())


COPY_WORKGROUPS, COPY_IN_TILES = 0, 1


def make_config(n_shards, max_rows_per_shard, K, N, n_groups=1, n_comm_wg=0, n_gemm_wg=0, tile_n=0,
                timeout_ns=0, stress=(0, 0, 0), split_parts=0, split_tiles=0, tile_order=0,
                copy_rows=0, combine_wg=0, copy_mode=COPY_WORKGROUPS) -> FgConfig:
    return FgConfig(n_shards, max_rows_per_shard, K, N, n_groups, n_comm_wg, n_gemm_wg, tile_n, timeout_ns,
                    stress[0], stress[1], stress[2], split_parts, split_tiles, tile_order, copy_rows, combine_wg,
                    copy_mode)


def ring_bytes(cfg: FgConfig, n_channels: int, ring_chunks: int) -> int:
    out = C.c_int64(0)
    _check(load_library().fg_ring_bytes(C.byref(cfg), n_channels, ring_chunks, C.byref(out)), "fg_ring_bytes")
    return out.value


def gather_gemm_noalloc(cfg: FgConfig, shards, w, gathered, out, status, *, route: FgRoute | None = None,
                        flags: int = 0, device: int = 0, stream=None) -> int:
    """fg_gather_gemm_noalloc: one iteration with no context and no allocation
    (status: a device int32 tensor the call clears and the kernels set on a
    device-side error). Returns the fg_status code of the launch."""
    arr = (C.c_void_p * len(shards))(*[s.data_ptr() for s in shards])
    return load_library().fg_gather_gemm_noalloc(C.byref(cfg), device, arr,
                                                 C.byref(route) if route is not None else None, _ptr(w),
                                                 _ptr(gathered), _ptr(out), _ptr(status), flags, _stream_ptr(stream))


def capacity(cfg: FgConfig) -> int:
    out = C.c_int32(0)
    _check(load_library().fg_capacity(C.byref(cfg), C.byref(out)), "fg_capacity")
    return out.value


class Context:
    """One fg context on one device (owns the control plane)."""

    def __init__(self, cfg: FgConfig, device: int = 0):
        lib = load_library()
        self.cfg = cfg
        self.device = device
        h = C.c_void_p()
        _check(lib.fg_init(C.byref(cfg), device, C.byref(h)), "fg_init")
        self._h = h
        self._lib = lib
        self._keep = []

    def close(self):
        if getattr(self, "_h", None):
            self._lib.fg_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ calls
    def gather_gemm(self, shards, w, gathered, out, *, route: FgRoute | None = None, flags: int = 0,
                    stream=None) -> int:
        """Returns the fg_status code (0 = launched)."""
        arr = (C.c_void_p * len(shards))(*[s.data_ptr() for s in shards])
        self._keep = [arr, route]
        return self._lib.fg_gather_gemm(self._h, arr, C.byref(route) if route is not None else None,
                                        _ptr(w), _ptr(gathered), _ptr(out), flags, _stream_ptr(stream))

    def gather_gemm_staged(self, shards, w, staging, gathered, out, *, self_shard: int = -1,
                           route: FgRoute | None = None, flags: int = 0, stream=None) -> int:
        """Two-stage dispatch; staging is a list of per-shard device tensors (None
        allowed for self_shard). Returns the fg_status code."""
        arr = (C.c_void_p * len(shards))(*[s.data_ptr() for s in shards])
        st = (C.c_void_p * len(staging))(*[0 if t is None else t.data_ptr() for t in staging])
        self._keep = [arr, st, route]
        return self._lib.fg_gather_gemm_staged(self._h, arr, C.byref(route) if route is not None else None,
                                               _ptr(w), st, self_shard, _ptr(gathered), _ptr(out), flags,
                                               _stream_ptr(stream))

    def gather_gemm_ring(self, shards, w, ring, gathered, out, *, n_channels: int, ring_chunks: int,
                         self_shard: int = -1, route: FgRoute | None = None, flags: int = 0, stream=None) -> int:
        """Dispatch through bounded FIFO rings (ring: a device tensor of at least
        ring_bytes(...) bytes). Returns the fg_status code."""
        arr = (C.c_void_p * len(shards))(*[s.data_ptr() for s in shards])
        self._keep = [arr, route]
        return self._lib.fg_gather_gemm_ring(self._h, arr, C.byref(route) if route is not None else None,
                                             _ptr(w), _ptr(ring), n_channels, ring_chunks, self_shard,
                                             _ptr(gathered), _ptr(out), flags, _stream_ptr(stream))

    def barrier(self, rounds: int = 1, stream=None) -> int:
        return self._lib.fg_barrier(self._h, rounds, _stream_ptr(stream))

    def pingpong(self, round_trips: int, sys_scope: bool = False, stream=None) -> int:
        return self._lib.fg_pingpong(self._h, round_trips, int(sys_scope), _stream_ptr(stream))

    def stress(self, chunk_rows, delays_ns, payload, flags: int = 0, stream=None) -> int:
        return self._lib.fg_stress(self._h, _ptr(chunk_rows), _ptr(delays_ns), _ptr(payload), flags,
                                   _stream_ptr(stream))

    def combine(self, out, weights, staging, y, flags: int = 0, stream=None) -> int:
        """fg_combine on the TOPK route of the last gather_gemm; staging and y are
        lists of per-shard device tensors. Returns the fg_status code."""
        st = (C.c_void_p * len(staging))(*[t.data_ptr() for t in staging])
        ys = (C.c_void_p * len(y))(*[t.data_ptr() for t in y])
        self._keep_c = [st, ys]
        return self._lib.fg_combine(self._h, _ptr(out), _ptr(weights), st, ys, flags, _stream_ptr(stream))

    def prepare_combine(self, out, weights, staging, y, stream=None):
        """fg_combine with its arguments marshalled once: returns f(flags=0) ->
        fg_status. The tensors must stay alive (and in place) while f is used."""
        st = (C.c_void_p * len(staging))(*[t.data_ptr() for t in staging])
        ys = (C.c_void_p * len(y))(*[t.data_ptr() for t in y])
        args = (self._h, _ptr(out), _ptr(weights), st, ys)
        sp = _stream_ptr(stream)
        fn = self._lib.fg_combine

        def call(flags: int = 0) -> int:
            return fn(*args, flags, sp)
        call._keep = (st, ys, out, weights, staging, y)
        return call

    def litmus(self, rounds: int, mode: int = 0, stream=None) -> int:
        return self._lib.fg_litmus(self._h, rounds, mode, _stream_ptr(stream))

    def stats(self, wait: bool = True) -> FgStats:
        st = FgStats()
        _check(self._lib.fg_stats(self._h, C.byref(st), int(wait)), "fg_stats")
        return st

    def views(self) -> FgViews:
        v = FgViews()
        _check(self._lib.fg_views(self._h, C.byref(v)), "fg_views")
        return v

    # ------------------------------------------------ control-plane snapshots
    def read_i32(self, ptr: int, count: int) -> torch.Tensor:
        """Copy `count` int32 of library-owned device memory to a CPU tensor."""
        torch.cuda.synchronize(self.device)
        return _as_device_tensor(ptr, count, self.device).clone().cpu()

    def read_timeline(self) -> dict:
        """Timing records of the last fused kernel, in microseconds from the
        earliest workgroup start: per workgroup (fg_views wg_time) and, after a
        call with CALL_TRACE, per compute item and per row block."""
        v = self.views()
        us = 1000.0 / v.wall_khz
        wg = self.read_i32(v.wg_time, 2 * 12 * v.grid).view(torch.int64).reshape(v.grid, 12).numpy().copy()
        t0 = wg[:, 0].min()
        out = dict(wg=wg, t0=t0, us_per_tick=us)
        if v.trace_cap:
            tr = self.read_i32(v.trace, 2 * 8 * v.trace_cap).view(torch.int64).reshape(v.trace_cap, 8).numpy().copy()
            out["trace"] = tr
            out["rb_time"] = self.read_i32(v.rb_time, 2 * v.rb_cap).view(torch.int64).numpy().copy()
        return out

    def read_inverse_map(self) -> torch.Tensor:
        """The inverse map of the route in use: gathered row -> (shard << 24 |
        stream index), -1 for a padding row."""
        v = self.views()
        raw = self.read_i32(v.inv_row, 2 * v.m_pad_cap).view(torch.int64)
        ver = raw.bitwise_right_shift(32).bitwise_and(0xFFFFFFFF)
        val = raw.bitwise_and(0xFFFFFFFF)
        return torch.where(ver == int(v.route_ver), val, torch.full_like(val, -1)).to(torch.int32)


class _DevArray:
    def __init__(self, ptr, count):
        self.__cuda_array_interface__ = {"shape": (count,), "typestr": "<i4", "data": (ptr, False),
                                         "version": 3, "strides": None}


def _as_device_tensor(ptr: int, count: int, device: int) -> torch.Tensor:
    with torch.cuda.device(device):
        return torch.as_tensor(_DevArray(ptr, count), device=f"cuda:{device}")


def route_contig(rows_per_shard: int) -> FgRoute:
    r = FgRoute()
    r.mode = ROUTE_CONTIG
    r.rows_per_shard = rows_per_shard
    return r


def route_explicit(stream_len, src_row: torch.Tensor, dst_row: torch.Tensor, m_pad: int, rows_per_shard: int,
                   group_off=None) -> FgRoute:
    r = FgRoute()
    r.mode = ROUTE_EXPLICIT
    r.rows_per_shard = rows_per_shard
    sl = (C.c_int32 * len(stream_len))(*[int(x) for x in stream_len])
    r.stream_len = C.cast(sl, C.POINTER(C.c_int32))
    r.src_row = src_row.data_ptr()
    r.dst_row = dst_row.data_ptr()
    r.m_pad = m_pad
    r._keep = [sl, src_row, dst_row]
    if group_off is not None:
        go = (C.c_int32 * len(group_off))(*[int(x) for x in group_off])
        r.group_off = C.cast(go, C.POINTER(C.c_int32))
        r._keep.append(go)
    return r


def route_topk(topk: torch.Tensor, tokens_per_shard: int, expert_base: int) -> FgRoute:
    r = FgRoute()
    r.mode = ROUTE_TOPK
    r.rows_per_shard = tokens_per_shard
    r.topk = topk.data_ptr()
    r.topk_k = topk.shape[-1]
    r.expert_base = expert_base
    r._keep = [topk]
    return r
