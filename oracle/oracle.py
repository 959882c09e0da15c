"""ctypes wrapper of the CPU oracle (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this module.  It loads ``libks_oracle.so`` (built by ``oracle/build.py``) and
returns numpy arrays in the same binary layouts the GPU path writes: 80-byte
per-warp counter records and per-warp trace slots of 16 + 8 * trace_cap bytes.
"""
import ctypes
import os

import numpy as np

from . import build as _build

NLAT = 18
LAT_NAMES = ["int32", "int64", "fp32", "setp", "selp", "mov", "ld_param", "ld_global",
             "ld_shared", "st_global", "st_shared", "bra", "bar", "ret", "l1_hit", "l2_hit", "dram"]

ST_FINISHED, ST_BUDGET, ST_FAULT, ST_TRACE_DROP, ST_BARDIV, ST_CYCLE_OVF = 1, 2, 4, 8, 16, 32

COUNTER_DTYPE = np.dtype([
    ("thread_instrs", "<u8"), ("status", "<u4"), ("cycles", "<u4"), ("warp_instrs", "<u4"),
    ("stall_cycles", "<u4"), ("gld_n", "<u4"), ("gld_sectors", "<u4"), ("gld_lines", "<u4"),
    ("gst_n", "<u4"), ("gst_sectors", "<u4"), ("gst_lines", "<u4"), ("sh_n", "<u4"),
    ("sh_degree_sum", "<u4"), ("sh_degree_max", "<u4"), ("diverge_n", "<u4"),
    ("barrier_n", "<u4"), ("fault_n", "<u4"), ("max_stack_depth", "<u4"), ("reserved", "<u4"),
])
assert COUNTER_DTYPE.itemsize == 80

TRACE_HEADER_DTYPE = np.dtype([("records_written", "<u4"), ("version", "u1"), ("flags", "u1"),
                               ("warp_in_block", "<u2"), ("records_dropped", "<u8")])
# the 16-byte records of the extended trace format
EXT_RECORD_DTYPE = np.dtype([("cycle", "<u4"), ("pc", "<u2"), ("kind", "u1"), ("reserved", "u1"),
                             ("active", "<u4"), ("payload", "<u4")])
TRACE_BASIC, TRACE_EXTENDED = 0, 1
FLAG_EXT_TRACE = 2
FLAG_CACHE = 4
# cache-latency model: per warp {u32 l1_hits, l2_hits, misses, 0}, L1 tags, L2 tags
CACHE_L1_LINES, CACHE_L2_LINES = 1024, 49152
CACHE_WARP_BYTES = 16 + 4 * (CACHE_L1_LINES + CACHE_L2_LINES)

E_RACE = -7


class OracleError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("oracle error %d: %s" % (code, msg))
        self.code = code
        self.msg = msg


class _Cfg(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_uint32 * 3), ("block", ctypes.c_uint32 * 3),
                ("gmem_bytes", ctypes.c_uint64), ("trace_cap", ctypes.c_uint32),
                ("max_warp_instrs", ctypes.c_uint32), ("latency", ctypes.c_uint16 * NLAT),
                ("n_threads", ctypes.c_uint32), ("flags", ctypes.c_uint32),
                ("block_list", ctypes.POINTER(ctypes.c_uint32)), ("n_block_list", ctypes.c_uint64),
                ("cache", ctypes.c_void_p)]


class _Info(ctypes.Structure):
    _fields_ = [("n_instrs", ctypes.c_uint32), ("n_params", ctypes.c_uint32),
                ("param_bytes", ctypes.c_uint32), ("shared_bytes", ctypes.c_uint32),
                ("reg_words", ctypes.c_uint32), ("n_preds", ctypes.c_uint32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_run.restype = ctypes.c_int
        L.oracle_run.argtypes = [ctypes.c_char_p, ctypes.c_size_t, ctypes.c_char_p, ctypes.POINTER(_Cfg),
                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_char_p, ctypes.c_size_t]
        L.oracle_program_info.restype = ctypes.c_int
        L.oracle_program_info.argtypes = [ctypes.c_char_p, ctypes.c_size_t, ctypes.c_char_p,
                                          ctypes.POINTER(_Info), ctypes.c_char_p, ctypes.c_size_t]
        L.oracle_param.restype = ctypes.c_int
        L.oracle_param.argtypes = [ctypes.c_char_p, ctypes.c_size_t, ctypes.c_char_p, ctypes.c_uint32,
                                   ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32),
                                   ctypes.c_char_p, ctypes.c_size_t, ctypes.c_char_p, ctypes.c_size_t]
        L.oracle_ipdom_table.restype = ctypes.c_int
        L.oracle_ipdom_table.argtypes = [ctypes.c_char_p, ctypes.c_size_t, ctypes.c_char_p,
                                         ctypes.POINTER(ctypes.c_uint32), ctypes.c_uint32,
                                         ctypes.c_char_p, ctypes.c_size_t]
        L.oracle_default_latency.restype = None
        L.oracle_default_latency.argtypes = [ctypes.POINTER(ctypes.c_uint16)]
        _lib = L
    return _lib


def _enc(s):
    return s.encode() if isinstance(s, str) else s


def default_latency():
    arr = (ctypes.c_uint16 * NLAT)()
    lib().oracle_default_latency(arr)
    return [int(x) for x in arr]


def program_info(ptx, entry=None):
    info = _Info()
    err = ctypes.create_string_buffer(512)
    b = _enc(ptx)
    rc = lib().oracle_program_info(b, len(b), _enc(entry) if entry else None, ctypes.byref(info), err, 512)
    if rc != 0:
        raise OracleError(rc, err.value.decode())
    return {k: getattr(info, k) for k, _ in _Info._fields_}


def params(ptx, entry=None):
    """[(name, offset, size)] in declaration order."""
    n = program_info(ptx, entry)["n_params"]
    out = []
    b = _enc(ptx)
    for i in range(n):
        off, size = ctypes.c_uint32(), ctypes.c_uint32()
        name = ctypes.create_string_buffer(256)
        err = ctypes.create_string_buffer(512)
        rc = lib().oracle_param(b, len(b), _enc(entry) if entry else None, i, ctypes.byref(off),
                                ctypes.byref(size), name, 256, err, 512)
        if rc != 0:
            raise OracleError(rc, err.value.decode())
        out.append((name.value.decode(), off.value, size.value))
    return out


def ipdom_table(ptx, entry=None):
    n = program_info(ptx, entry)["n_instrs"]
    arr = (ctypes.c_uint32 * max(n, 1))()
    err = ctypes.create_string_buffer(512)
    b = _enc(ptx)
    rc = lib().oracle_ipdom_table(b, len(b), _enc(entry) if entry else None, arr, n, err, 512)
    if rc != 0:
        raise OracleError(rc, err.value.decode())
    return [int(arr[i]) for i in range(n)]


def _dim3(d):
    if isinstance(d, int):
        return (d, 1, 1)
    d = tuple(d) + (1,) * (3 - len(d))
    return d


def run(ptx, grid, block, params_bytes, gmem, trace_cap=0, max_warp_instrs=0xFFFFFFFF, latency=None,
        threads=0, blocks=None, check_races=False, entry=None, trace_format=TRACE_BASIC, cache=None):
    """Simulate.  `gmem` is a writable uint8 numpy array, updated in place.

    Returns (counters, trace, rc): counters is a COUNTER_DTYPE array with one record
    per simulated warp, trace a uint8 array of (16 + R * trace_cap) bytes per warp
    (R = 8, or 16 with trace_format TRACE_EXTENDED), rc 0 or E_RACE (race checking
    only).  `blocks` optionally lists the linear block ids to simulate; outputs
    follow that order.  `cache`, a writable uint8 array of CACHE_WARP_BYTES per
    simulated warp, turns the cache-latency model on and receives its per-warp
    state."""
    assert gmem.dtype == np.uint8 and gmem.flags.c_contiguous and gmem.flags.writeable
    grid, block = _dim3(grid), _dim3(block)
    cfg = _Cfg()
    cfg.grid[:] = grid
    cfg.block[:] = block
    cfg.gmem_bytes = gmem.size
    cfg.trace_cap = trace_cap
    cfg.max_warp_instrs = max_warp_instrs
    lat = default_latency() if latency is None else list(latency)
    lat = lat + [0] * (NLAT - len(lat))
    cfg.latency[:] = lat
    cfg.n_threads = threads
    cfg.flags = (1 if check_races else 0) | (FLAG_EXT_TRACE if trace_format == TRACE_EXTENDED else 0)
    if cache is not None:
        cfg.flags |= FLAG_CACHE
    rec = 16 if trace_format == TRACE_EXTENDED else 8
    tpb = block[0] * block[1] * block[2]
    wpb = (tpb + 31) // 32
    if blocks is None:
        nb = grid[0] * grid[1] * grid[2]
        bl = None
        cfg.n_block_list = 0
    else:
        bl = np.ascontiguousarray(np.asarray(blocks, dtype=np.uint32))
        nb = bl.size
        cfg.block_list = bl.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))
        cfg.n_block_list = nb
    counters = np.zeros(nb * wpb, dtype=COUNTER_DTYPE)
    if cache is not None:
        assert cache.dtype == np.uint8 and cache.flags.c_contiguous and cache.flags.writeable
        assert cache.size >= nb * wpb * CACHE_WARP_BYTES
        cfg.cache = cache.ctypes.data
    trace = np.zeros(nb * wpb * (16 + rec * trace_cap), dtype=np.uint8)
    pb = bytes(params_bytes)
    pbuf = ctypes.create_string_buffer(pb, max(len(pb), 1))
    err = ctypes.create_string_buffer(1024)
    b = _enc(ptx)
    rc = lib().oracle_run(b, len(b), _enc(entry) if entry else None, ctypes.byref(cfg), pbuf, len(pb),
                          gmem.ctypes.data, counters.ctypes.data, trace.ctypes.data, err, 1024)
    if rc != 0 and rc != E_RACE:
        raise OracleError(rc, err.value.decode())
    return counters, trace, rc


def trace_slots(trace, trace_cap, trace_format=TRACE_BASIC):
    """Split a trace buffer into (headers, records): records[warp, cap, 2] u32 for
    the basic format, records[warp, cap] of EXT_RECORD_DTYPE for the extended one."""
    rec = 16 if trace_format == TRACE_EXTENDED else 8
    slot = 16 + rec * trace_cap
    t = trace.reshape(-1, slot)
    hdr = t[:, :16].copy().view(TRACE_HEADER_DTYPE).reshape(-1)
    body = t[:, 16:].copy()
    if trace_format == TRACE_EXTENDED:
        return hdr, body.view(EXT_RECORD_DTYPE).reshape(t.shape[0], trace_cap)
    return hdr, body.view("<u4").reshape(t.shape[0], trace_cap, 2)


CACHE_HEADER_DTYPE = np.dtype([("l1_hits", "<u4"), ("l2_hits", "<u4"), ("misses", "<u4"), ("reserved", "<u4")])


def cache_state(cache, n_warps):
    """Split a cache-model buffer into (headers, l1 tags, l2 tags) per warp; a tag is
    the line number + 1, 0 for an empty set."""
    c = cache[:n_warps * CACHE_WARP_BYTES].reshape(n_warps, CACHE_WARP_BYTES)
    hdr = c[:, :16].copy().view(CACHE_HEADER_DTYPE).reshape(-1)
    tags = c[:, 16:].copy().view("<u4")
    return hdr, tags[:, :CACHE_L1_LINES], tags[:, CACHE_L1_LINES:]
