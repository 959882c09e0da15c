"""Thin Python binding of libkscope (include/ks.h).

Argument marshalling only: every step of the simulation runs in the library's
gfx950 kernels.  PyTorch provides device memory and streams (plumbing).  If the
compiled library is missing or no gfx950 device is usable, calls raise; there
is no CPU fallback.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkscope.so")

KS_OK = 0
KS_NLAT = 18
ST_FINISHED, ST_BUDGET, ST_FAULT, ST_TRACE_DROP, ST_BARDIV, ST_CYCLE_OVF = 1, 2, 4, 8, 16, 32
LAT_LD_GLOBAL, LAT_BAR = 7, 12

COUNTER_DTYPE = np.dtype([
    ("thread_instrs", "<u8"), ("status", "<u4"), ("cycles", "<u4"), ("warp_instrs", "<u4"),
    ("stall_cycles", "<u4"), ("gld_n", "<u4"), ("gld_sectors", "<u4"), ("gld_lines", "<u4"),
    ("gst_n", "<u4"), ("gst_sectors", "<u4"), ("gst_lines", "<u4"), ("sh_n", "<u4"),
    ("sh_degree_sum", "<u4"), ("sh_degree_max", "<u4"), ("diverge_n", "<u4"),
    ("barrier_n", "<u4"), ("fault_n", "<u4"), ("max_stack_depth", "<u4"), ("reserved", "<u4"),
])
TRACE_HEADER_DTYPE = np.dtype([("records_written", "<u4"), ("version", "u1"), ("flags", "u1"),
                               ("warp_in_block", "<u2"), ("records_dropped", "<u8")])
# program and launch limits (include/ks.h)
KS_MAX_REG_SLOTS, KS_MAX_PREDS, KS_MAX_INSTRS = 64, 32, 65535
KS_MAX_PARAM_BYTES, KS_MAX_SHARED_BYTES, KS_MAX_BLOCK_THREADS = 512, 65536, 1024
# trace formats (ks_config.trace_format) and the 16-byte extended record
KS_TRACE_BASIC, KS_TRACE_EXTENDED = 0, 1
KS_EXT_MAX_BLOCKS = 32  # blocks per launch of an extended-record run (ks_run chunks larger grids)
KS_STATIC_MAX_INSTRS = 8187  # largest program a ks_alloc_state_static binding holds
KS_EXT_MAX_BLOCK_THREADS, KS_EXT64_MAX_BLOCK_THREADS = 1024, 768  # largest block of an extended-record run (> 32 slots)
# cache-latency model (ks_config.cache_model) and its per-warp state in d_cache
KS_CACHE_NONE, KS_CACHE_WARP = 0, 1
KS_LAT_L1_HIT, KS_LAT_L2_HIT, KS_LAT_DRAM = 14, 15, 16
KS_CACHE_L1_LINES, KS_CACHE_L2_LINES = 1024, 49152
KS_CACHE_WARP_BYTES = 16 + 4 * (KS_CACHE_L1_LINES + KS_CACHE_L2_LINES)
CACHE_HEADER_DTYPE = np.dtype([("l1_hits", "<u4"), ("l2_hits", "<u4"), ("misses", "<u4"), ("reserved", "<u4")])
EXT_RECORD_DTYPE = np.dtype([("cycle", "<u4"), ("pc", "<u2"), ("kind", "u1"), ("reserved", "u1"),
                             ("active", "<u4"), ("payload", "<u4")])
EV_NAMES = ["other", "ld.global", "st.global", "ld.shared", "st.shared", "branch", "diverge", "barrier", "ret"]
(KS_EV_OTHER, KS_EV_LD_GLOBAL, KS_EV_ST_GLOBAL, KS_EV_LD_SHARED, KS_EV_ST_SHARED, KS_EV_BRANCH, KS_EV_DIVERGE,
 KS_EV_BARRIER, KS_EV_RET) = range(9)


class KsError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("libkscope error %d: %s" % (code, msg))
        self.code = code
        self.msg = msg


class ks_dim3(ctypes.Structure):
    _fields_ = [("x", ctypes.c_uint32), ("y", ctypes.c_uint32), ("z", ctypes.c_uint32)]


class ks_config(ctypes.Structure):
    _fields_ = [("max_grid", ks_dim3), ("max_block", ks_dim3), ("gmem_bytes", ctypes.c_uint64),
                ("trace_cap", ctypes.c_uint32), ("max_warp_instrs", ctypes.c_uint32),
                ("latency", ctypes.c_uint16 * KS_NLAT), ("trace_format", ctypes.c_uint32),
                ("cache_model", ctypes.c_uint32)]


class ks_program_desc(ctypes.Structure):
    _fields_ = [("n_instrs", ctypes.c_uint32), ("n_params", ctypes.c_uint32), ("param_bytes", ctypes.c_uint32),
                ("shared_bytes", ctypes.c_uint32), ("reg_slots", ctypes.c_uint32), ("n_preds", ctypes.c_uint32)]


class ks_instr_desc(ctypes.Structure):
    _fields_ = [("line", ctypes.c_uint32), ("kind", ctypes.c_uint32), ("access_bytes", ctypes.c_uint32),
                ("lat_class", ctypes.c_uint32)]


class ks_layout(ctypes.Structure):
    _fields_ = [("warps_per_block", ctypes.c_uint32), ("reserved", ctypes.c_uint32), ("n_warps", ctypes.c_uint64),
                ("counters_bytes", ctypes.c_uint64), ("slot_bytes", ctypes.c_uint64), ("trace_bytes", ctypes.c_uint64),
                ("cache_bytes", ctypes.c_uint64)]


_P = ctypes.c_void_p
_EXPORTS = {
    "ks_load_program": ([ctypes.c_char_p, ctypes.c_size_t, ctypes.c_char_p, ctypes.POINTER(_P)], ctypes.c_int32),
    "ks_program_info": ([_P, ctypes.POINTER(ks_program_desc)], ctypes.c_int32),
    "ks_param_info": ([_P, ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32),
                       ctypes.POINTER(ctypes.c_char_p)], ctypes.c_int32),
    "ks_param_offset": ([_P, ctypes.c_char_p, ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32)],
                        ctypes.c_int32),
    "ks_ipdom_table": ([_P, ctypes.POINTER(ctypes.c_uint32), ctypes.c_uint32], ctypes.c_int32),
    "ks_instr_info": ([_P, ctypes.c_uint32, ctypes.POINTER(ks_instr_desc)], ctypes.c_int32),
    "ks_default_config": ([ctypes.POINTER(ks_config)], ctypes.c_int32),
    "ks_query_layout": ([_P, ctypes.POINTER(ks_config), ctypes.POINTER(ks_layout)], ctypes.c_int32),
    "ks_alloc_state": ([_P, ctypes.POINTER(ks_config), _P, _P, _P, _P, ctypes.POINTER(_P)], ctypes.c_int32),
    "ks_alloc_state_static": ([_P, ctypes.POINTER(ks_config), _P, _P, _P, _P, ctypes.POINTER(_P)], ctypes.c_int32),
    "ks_run": ([_P, ks_dim3, ks_dim3, ctypes.c_void_p, ctypes.c_size_t, _P], ctypes.c_int32),
    "ks_interp_kernel": ([_P, ks_dim3, ctypes.POINTER(ctypes.c_char_p)], ctypes.c_int32),
    "ks_read_outputs": ([_P, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_size_t, _P], ctypes.c_int32),
    "ks_read_counters": ([_P, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_size_t, _P], ctypes.c_int32),
    "ks_read_trace": ([_P, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_size_t, _P], ctypes.c_int32),
    "ks_run_status": ([_P, ctypes.POINTER(ctypes.c_uint32), _P], ctypes.c_int32),
    "ks_write_trace_events": ([ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64,
                               ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(ctypes.c_char_p),
                               ctypes.POINTER(ctypes.c_char_p), ctypes.c_char_p, ctypes.POINTER(ctypes.c_uint64)],
                              ctypes.c_int32),
    "ks_state_free": ([_P], None),
    "ks_program_free": ([_P], None),
    "ks_last_error": ([], ctypes.c_char_p),
}

_lib = None


def lib():
    """Load libkscope.so (built by analysis_ptxsimulator_amd/build.py).  Raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkscope.so is not built (run __graft_entry__.build()); there is no fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _EXPORTS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(rc):
    if rc != KS_OK:
        raise KsError(rc, lib().ks_last_error().decode(errors="replace"))


def _dim3(d):
    if isinstance(d, int):
        d = (d,)
    d = tuple(int(x) for x in d) + (1,) * (3 - len(d))
    return ks_dim3(*d)


# ---------------------------------------------------------------- entry points (same names as the C ABI)

def ks_load_program(ptx, entry=None):
    b = ptx.encode() if isinstance(ptx, str) else bytes(ptx)
    out = _P()
    _check(lib().ks_load_program(b, len(b), entry.encode() if entry else None, ctypes.byref(out)))
    return out


def ks_program_info(prog):
    d = ks_program_desc()
    _check(lib().ks_program_info(prog, ctypes.byref(d)))
    return {k: getattr(d, k) for k, _ in ks_program_desc._fields_}


def ks_param_info(prog, index):
    off, size, name = ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_char_p()
    _check(lib().ks_param_info(prog, index, ctypes.byref(off), ctypes.byref(size), ctypes.byref(name)))
    return off.value, size.value, name.value.decode()


def ks_param_offset(prog, name):
    off, size = ctypes.c_uint32(), ctypes.c_uint32()
    _check(lib().ks_param_offset(prog, name.encode(), ctypes.byref(off), ctypes.byref(size)))
    return off.value, size.value


def ks_instr_info(prog, pc):
    d = ks_instr_desc()
    _check(lib().ks_instr_info(prog, pc, ctypes.byref(d)))
    return {k: getattr(d, k) for k, _ in ks_instr_desc._fields_}


def ks_ipdom_table(prog):
    n = ks_program_info(prog)["n_instrs"]
    arr = (ctypes.c_uint32 * max(n, 1))()
    _check(lib().ks_ipdom_table(prog, arr, n))
    return [int(arr[i]) for i in range(n)]


def ks_interp_kernel(prog, block):
    name = ctypes.c_char_p()
    _check(lib().ks_interp_kernel(prog, _dim3(block), ctypes.byref(name)))
    return name.value.decode()


def ks_default_config():
    c = ks_config()
    _check(lib().ks_default_config(ctypes.byref(c)))
    return c


def ks_query_layout(prog, cfg):
    lay = ks_layout()
    _check(lib().ks_query_layout(prog, ctypes.byref(cfg), ctypes.byref(lay)))
    return lay


def ks_alloc_state(prog, cfg, d_gmem, d_counters, d_trace, d_cache=0):
    out = _P()
    _check(lib().ks_alloc_state(prog, ctypes.byref(cfg), _P(d_gmem), _P(d_counters), _P(d_trace), _P(d_cache),
                                ctypes.byref(out)))
    return out


def ks_alloc_state_static(prog, cfg, d_gmem, d_counters, d_trace, d_cache=0):
    out = _P()
    _check(lib().ks_alloc_state_static(prog, ctypes.byref(cfg), _P(d_gmem), _P(d_counters), _P(d_trace),
                                       _P(d_cache), ctypes.byref(out)))
    return out


def ks_run(state, grid, block, params, stream=0):
    pb = bytes(params)
    buf = ctypes.create_string_buffer(pb, max(len(pb), 1))
    _check(lib().ks_run(state, _dim3(grid), _dim3(block), buf, len(pb), _P(stream)))


def ks_read_outputs(state, sim_addr, nbytes, stream=0):
    out = np.empty(nbytes, dtype=np.uint8)
    _check(lib().ks_read_outputs(state, sim_addr, out.ctypes.data, nbytes, _P(stream)))
    return out


def ks_read_counters(state, first_warp, n_warps, stream=0):
    out = np.empty(n_warps, dtype=COUNTER_DTYPE)
    _check(lib().ks_read_counters(state, first_warp, n_warps, out.ctypes.data, out.nbytes, _P(stream)))
    return out


def ks_read_trace(state, first_warp, n_warps, slot_bytes, stream=0):
    out = np.empty(n_warps * slot_bytes, dtype=np.uint8)
    _check(lib().ks_read_trace(state, first_warp, n_warps, out.ctypes.data, out.nbytes, _P(stream)))
    return out


def ks_run_status(state, stream=0):
    v = ctypes.c_uint32()
    _check(lib().ks_run_status(state, ctypes.byref(v), _P(stream)))
    return v.value


def ks_write_trace_events(trace, n_warps, slot_bytes, trace_format, first_warp, warps_per_block, pc_names,
                          pc_args, path):
    """trace: a C-contiguous host buffer (numpy) of n_warps slots; pc_names / pc_args:
    lists of str (JSON fragments).  Returns the number of instruction events."""
    t = np.ascontiguousarray(trace)
    assert t.nbytes >= n_warps * slot_bytes, "trace buffer smaller than its slots"
    n = len(pc_names)
    assert len(pc_args) == n
    names = (ctypes.c_char_p * max(n, 1))(*[x.encode() for x in pc_names])
    args = (ctypes.c_char_p * max(n, 1))(*[x.encode() for x in pc_args])
    out = ctypes.c_uint64()
    _check(lib().ks_write_trace_events(t.ctypes.data_as(ctypes.c_void_p), n_warps, slot_bytes, trace_format,
                                       first_warp, warps_per_block, n, names, args, os.fsencode(path),
                                       ctypes.byref(out)))
    return out.value


def ks_state_free(state):
    lib().ks_state_free(state)


def ks_program_free(prog):
    lib().ks_program_free(prog)


def ks_last_error():
    return lib().ks_last_error().decode(errors="replace")


def trace_slots(trace, trace_cap, trace_format=KS_TRACE_BASIC):
    """Split trace slot bytes into (headers, records): records[warp, cap, 2] u32 for
    the basic format, records[warp, cap] of EXT_RECORD_DTYPE for the extended one."""
    rec = 16 if trace_format == KS_TRACE_EXTENDED else 8
    slot = 16 + rec * trace_cap
    t = trace.reshape(-1, slot)
    hdr = t[:, :16].copy().view(TRACE_HEADER_DTYPE).reshape(-1)
    body = t[:, 16:].copy()
    if trace_format == KS_TRACE_EXTENDED:
        return hdr, body.view(EXT_RECORD_DTYPE).reshape(t.shape[0], trace_cap)
    return hdr, body.view("<u4").reshape(t.shape[0], trace_cap, 2)


# ---------------------------------------------------------------- device-memory plumbing

class Session:
    """Owns the torch device buffers of one program: simulated global memory,
    counters and trace slots sized by ks_query_layout, plus the library state.

    Memory management only; all simulation work happens in ks_run."""

    def __init__(self, ptx, grid, block, gmem_bytes, trace_cap=0, max_warp_instrs=0xFFFFFFFF, latency=None,
                 device="cuda:0", entry=None, trace_format=KS_TRACE_BASIC, cache_model=KS_CACHE_NONE):
        import torch
        self.torch = torch
        self.device = torch.device(device)
        self.prog = ks_load_program(ptx, entry)
        cfg = ks_default_config()
        g, b = _dim3(grid), _dim3(block)
        cfg.max_grid = g
        cfg.max_block = b
        cfg.gmem_bytes = int(gmem_bytes)
        cfg.trace_cap = int(trace_cap)
        cfg.max_warp_instrs = int(max_warp_instrs)
        cfg.trace_format = int(trace_format)
        cfg.cache_model = int(cache_model)
        self.trace_format = int(trace_format)
        self.cache_model = int(cache_model)
        self.trace_cap = int(trace_cap)
        if latency is not None:
            lat = list(latency) + [0] * (KS_NLAT - len(latency))
            cfg.latency[:] = lat
        self.cfg = cfg
        self.grid, self.block = (g.x, g.y, g.z), (b.x, b.y, b.z)
        self.layout = ks_query_layout(self.prog, cfg)
        self.last_warps = 0
        self.gmem = torch.empty(max(int(gmem_bytes), 1), dtype=torch.uint8, device=self.device)
        self.counters = torch.empty(max(int(self.layout.counters_bytes), 1), dtype=torch.uint8, device=self.device)
        self.trace = torch.empty(max(int(self.layout.trace_bytes), 1), dtype=torch.uint8, device=self.device)
        self.cache = (torch.empty(int(self.layout.cache_bytes), dtype=torch.uint8, device=self.device)
                      if self.layout.cache_bytes else None)
        with torch.cuda.device(self.device):
            self.state = ks_alloc_state(self.prog, cfg, self.gmem.data_ptr(), self.counters.data_ptr(),
                                        self.trace.data_ptr(), self.cache.data_ptr() if self.cache is not None else 0)

    @property
    def n_warps(self):
        return int(self.layout.n_warps)

    def load_gmem(self, image):
        src = self.torch.from_numpy(np.ascontiguousarray(image, dtype=np.uint8))
        self.gmem[: src.numel()].copy_(src.to(self.device))

    def stream_ptr(self, stream=None):
        s = stream if stream is not None else self.torch.cuda.current_stream(self.device)
        return s.cuda_stream

    def run(self, params, stream=None, grid=None, block=None):
        g, b = _dim3(grid or self.grid), _dim3(block or self.block)
        ks_run(self.state, (g.x, g.y, g.z), (b.x, b.y, b.z), params, self.stream_ptr(stream))
        self.last_warps = g.x * g.y * g.z * ((b.x * b.y * b.z + 31) // 32)

    def read_gmem(self, offset=0, nbytes=None):
        n = int(self.cfg.gmem_bytes) - offset if nbytes is None else nbytes
        return ks_read_outputs(self.state, offset, n, self.stream_ptr())

    def read_counters(self, first=0, n=None):
        return ks_read_counters(self.state, first, self.last_warps - first if n is None else n, self.stream_ptr())

    def read_trace(self, first=0, n=None):
        n = self.last_warps - first if n is None else n
        return ks_read_trace(self.state, first, n, int(self.layout.slot_bytes), self.stream_ptr())

    def status(self):
        return ks_run_status(self.state, self.stream_ptr())

    def trace_records(self, first=0, n=None):
        """(headers, records) of the last run's trace slots (see trace_slots)."""
        return trace_slots(self.read_trace(first, n), self.trace_cap, self.trace_format)

    def kernel_name(self):
        """Name of the interpreter kernel ks_run launches for this session."""
        name = ks_interp_kernel(self.prog, self.block)
        if self.trace_format == KS_TRACE_EXTENDED:
            return name + "_ext"
        return name + ("_cache" if self.cache_model == KS_CACHE_WARP else "")

    def read_cache_headers(self, first=0, n=None):
        """Only the 16-byte headers (outcome counts) of warps [first, first + n)."""
        assert self.cache is not None, "the session has no cache model"
        n = self.last_warps - first if n is None else n
        v = self.cache[first * KS_CACHE_WARP_BYTES:(first + n) * KS_CACHE_WARP_BYTES].view(n, KS_CACHE_WARP_BYTES)
        raw = v[:, :16].contiguous().cpu().numpy()
        return raw.reshape(-1).view(CACHE_HEADER_DTYPE)

    def read_cache(self, first=0, n=None):
        """The cache model's state of warps [first, first + n) after the last run:
        (headers of CACHE_HEADER_DTYPE, L1 tags [n, 1024], L2 tags [n, 49152]) as u32,
        a tag being the line number + 1 (0: empty)."""
        assert self.cache is not None, "the session has no cache model"
        n = self.last_warps - first if n is None else n
        self.torch.cuda.synchronize(self.device)
        raw = self.cache[first * KS_CACHE_WARP_BYTES:(first + n) * KS_CACHE_WARP_BYTES].cpu().numpy()
        c = raw.reshape(n, KS_CACHE_WARP_BYTES)
        hdr = c[:, :16].copy().view(CACHE_HEADER_DTYPE).reshape(-1)
        tags = c[:, 16:].copy().view("<u4")
        return hdr, tags[:, :KS_CACHE_L1_LINES], tags[:, KS_CACHE_L1_LINES:]

    def close(self):
        if getattr(self, "state", None):
            ks_state_free(self.state)
            self.state = None
        if getattr(self, "prog", None):
            ks_program_free(self.prog)
            self.prog = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
