"""The no-allocation binding, ks_alloc_state_static, against ks_alloc_state.

Both bindings run the same program on the same inputs through the C ABI
(ks_run, ks_read_*, ks_run_status); the static one keeps its decoded program in
the library's per-GPU static scratch instead of device memory of its own.  Every
byte of simulated memory, every counter record and every trace slot must agree.
Two static bindings in a row, the second on a smaller input, check that the
scratch is rewritten correctly and that the older static state is refused.
"""
import sys

import numpy as np
import pytest

from workloads import configs as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from analysis_ptxsimulator_amd import ks
    ks.lib()
    return ks


class Bound:
    """A program bound to fresh caller-owned buffers by one of the two calls."""

    def __init__(self, K, w, static):
        import torch
        self.K, self.w = K, w
        dev = torch.device("cuda:0")
        self.prog = K.ks_load_program(w.ptx)
        cfg = K.ks_default_config()
        cfg.max_grid = K._dim3(w.grid)
        cfg.max_block = K._dim3(w.block)
        cfg.gmem_bytes = w.gmem.size
        cfg.trace_cap = w.trace_cap
        lay = K.ks_query_layout(self.prog, cfg)
        self.slot = int(lay.slot_bytes)
        self.gmem = torch.from_numpy(w.gmem.copy()).to(dev)
        self.counters = torch.zeros(int(lay.counters_bytes), dtype=torch.uint8, device=dev)
        self.trace = torch.zeros(int(lay.trace_bytes), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize(dev)
        bind = K.ks_alloc_state_static if static else K.ks_alloc_state
        self.state = bind(self.prog, cfg, self.gmem.data_ptr(), self.counters.data_ptr(), self.trace.data_ptr())
        self.stream = torch.cuda.current_stream(dev).cuda_stream

    def run(self):
        self.K.ks_run(self.state, self.w.grid, self.w.block, self.w.params_bytes, self.stream)

    def results(self):
        K, w = self.K, self.w
        nw = w.n_blocks * w.warps_per_block
        return (K.ks_read_outputs(self.state, 0, w.gmem.size, self.stream),
                K.ks_read_counters(self.state, 0, nw, self.stream),
                K.ks_read_trace(self.state, 0, nw, self.slot, self.stream),
                K.ks_run_status(self.state, self.stream))

    def close(self):
        self.K.ks_state_free(self.state)
        self.K.ks_program_free(self.prog)


def _same(K, w, static_res, ref_res):
    names = ("memory", "counters", "trace slots")
    for name, a, b in zip(names, static_res[:3], ref_res[:3]):
        assert a.shape == b.shape and np.array_equal(a, b), "%s: %s differ" % (w.name, name)
    assert static_res[3] == ref_res[3], "%s: run status %#x vs %#x" % (w.name, static_res[3], ref_res[3])


def test_static_binding_matches_allocating_binding(K):
    # first call: a 64-slot random program over 40 blocks; second call: a smaller
    # input (the 19-instruction vector_add over 4 blocks)
    big = W.random_stress(prog_seed=1, grid=40, block=256, gmem_bytes=1 << 24, trace_cap=512)
    small = W.vector_add()
    first = None
    for w in (big, small):
        _say("static binding vs ks_alloc_state: %s grid=%s block=%s cap=%d" % (w.name, w.grid, w.block, w.trace_cap))
        ref = Bound(K, w, static=False)
        ref.run()
        ref_res = ref.results()
        st = Bound(K, w, static=True)
        st.run()
        st_res = st.results()
        _same(K, w, st_res, ref_res)
        # a second run of the same static state: the scratch still holds its program
        st.run()
        _same(K, w, st.results(), ref_res)
        assert int(ref_res[1]["thread_instrs"].sum()) > 0
        ref.close()
        if first is None:
            first = st
        else:
            # the first static state's program was replaced by this binding
            with pytest.raises(K.KsError) as e:
                first.run()
            assert e.value.code == -6  # KS_E_STATE
            first.close()
            st.close()
    _say("static binding: both calls bit-exact, the replaced state refused")
