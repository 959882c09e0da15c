"""CPU-side tests of libkscope's host half: exports, parser, reconvergence table,
layouts and error paths (no GPU needed; no compute call is made)."""
import ctypes
import os
import re

import numpy as np
import pytest

from workloads import configs as W
from workloads import small as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="session")
def ks():
    from analysis_ptxsimulator_amd import build, ks as K
    build.build(force=False)
    return K


def test_library_exports_every_declared_symbol(ks):
    with open(os.path.join(ROOT, "include", "ks.h")) as f:
        header = f.read()
    names = set(re.findall(r"^(?:ks_status|void|const char\*)\s+(ks_\w+)\s*\(", header, re.M))
    assert len(names) >= 15
    L = ctypes.CDLL(ks.LIB_PATH)
    for n in sorted(names):
        assert hasattr(L, n), n
    assert names == set(ks._EXPORTS)


def _all_programs():
    progs = [W.VECTOR_ADD_PTX, W.STRIDED_PTX, W.ffma_probe_ptx(1), W.ffma_probe_ptx(8), W.bank_probe_ptx(),
             S.F32_OPS_PTX, S.ADDR_PROBE_PTX, S.staircase_ptx(31), S.fma_chain_ptx(9, 3)]
    from workloads.randprog import random_program
    for seed in range(3):
        progs.append(random_program(seed)[0])
    for seed in range(20):
        progs.append(S.random_cfg_ptx(seed))
    return progs


def test_binding_constants_match_the_header(ks):
    """Every integer constant include/ks.h defines that the Python binding mirrors
    has the header's value."""
    src = open(os.path.join(ROOT, "include", "ks.h")).read()
    seen = 0
    for name, val in re.findall(r"^#define (KS_\w+)\s+\(?(-?(?:0x[0-9A-Fa-f]+|\d+))u?\)?\s*(?:/\*.*)?$", src, re.M):
        if hasattr(ks, name):
            assert getattr(ks, name) == int(val, 0), name
            seen += 1
    assert ks.KS_CACHE_WARP_BYTES == 16 + 4 * (ks.KS_CACHE_L1_LINES + ks.KS_CACHE_L2_LINES)
    assert seen >= 15


def test_program_shape_matches_oracle(ks, oracle_mod):
    for ptx in _all_programs():
        p = ks.ks_load_program(ptx)
        info = ks.ks_program_info(p)
        o = oracle_mod.program_info(ptx)
        assert info["n_instrs"] == o["n_instrs"]
        assert info["param_bytes"] == o["param_bytes"]
        assert info["shared_bytes"] == o["shared_bytes"]
        assert info["reg_slots"] == o["reg_words"]
        assert info["n_preds"] == o["n_preds"]
        for i, (name, off, size) in enumerate(oracle_mod.params(ptx)):
            assert ks.ks_param_info(p, i) == (off, size, name)
            assert ks.ks_param_offset(p, name) == (off, size)
        ks.ks_program_free(p)


def test_param_offset_unknown_name_is_an_error(ks):
    p = ks.ks_load_program(W.VECTOR_ADD_PTX)
    with pytest.raises(ks.KsError) as e:
        ks.ks_param_offset(p, "no_such_param")
    assert e.value.code == -3 and "no_such_param" in e.value.msg
    ks.ks_program_free(p)


def test_random_stress_uses_64_slots(ks):
    from workloads.randprog import random_program
    p = ks.ks_load_program(random_program(0)[0])
    assert ks.ks_program_info(p)["reg_slots"] == 64
    ks.ks_program_free(p)


@pytest.mark.parametrize("seed", range(300))
def test_reconvergence_table_matches_oracle(ks, oracle_mod, seed):
    """Cooper-Harvey-Kennedy on basic blocks (library) versus post-dominator sets
    by fixed point on instructions (oracle), loops included."""
    ptx = S.random_cfg_ptx(5000 + seed, n_instr=10 + seed % 40, loops=(seed % 3 == 0))
    p = ks.ks_load_program(ptx)
    assert ks.ks_ipdom_table(p) == oracle_mod.ipdom_table(ptx)
    ks.ks_program_free(p)


def test_reconvergence_on_workloads(ks, oracle_mod):
    for ptx in _all_programs():
        p = ks.ks_load_program(ptx)
        assert ks.ks_ipdom_table(p) == oracle_mod.ipdom_table(ptx)
        ks.ks_program_free(p)


BAD = [
    ("add.f32 %f3, %f1, %f2;", "add.f32 %f3, %f1, %f9;", -1, "undeclared register %f9"),
    ("add.f32 %f3, %f1, %f2;", "div.rn.f32 %f3, %f1, %f2;", -2, "unsupported instruction"),
    ("@%p1 bra $L__exit;", "@%p1 bra $L__nowhere;", -1, "unknown label"),
    ("mov.u32 %r2, %tid.x;", "mov.u32 %r2, 1.5;", -1, None),
    ("add.f32 %f3, %f1, %f2;", "add.f32 %f3, %f1, 1;", -2, "0fXXXXXXXX"),
    ("add.s64 %rd5, %rd1, %rd4;", "add.s64 %rd5, %rd1, %r4;", -1, "is 32-bit"),
    # token spacing the subset's grammar fixes (the oracle splits on the same places)
    (".param .u64 param_b,", ".param .u64 param_b", -1, "expected ','"),
    ("    ret;", "    L.x:\n    ret;", -1, "bad label name"),
    ("$L__exit:", "$L__exit :", -1, "space between label"),
    (".reg .b32 %r<6>;", ".reg .b32 %r <6>;", -1, "space between register name"),
    ("@%p1 bra $L__exit;", "@ %p1 bra $L__exit;", -1, "space inside the guard"),
    ("@%p1 bra $L__exit;", "@! %p1 bra $L__exit;", -1, "space inside the guard"),
    ("ld.global.f32 %f1, [%rd5];", "ld.global.f32 %f1, [%rd5+- 4];", -1, "space between '-'"),
    ("mul.wide.s32 %rd4, %r5, 4;", "mul.wide.s32 %rd4, %r5, - 4;", -1, "space between '-'"),
    ("st.global.f32 [%rd7], %f3;", "st.global.f32[%rd7], %f3;", -1, "expected a space after"),
]


@pytest.mark.parametrize("old,new,code,msg", BAD)
def test_parse_errors(ks, old, new, code, msg):
    ptx = W.VECTOR_ADD_PTX.replace(old, new)
    assert ptx != W.VECTOR_ADD_PTX
    with pytest.raises(ks.KsError) as e:
        ks.ks_load_program(ptx)
    assert e.value.code == code
    line = 1 + W.VECTOR_ADD_PTX.split(old)[0].count("\n")
    if code == -1 or msg:
        assert ("line %d:" % line) in e.value.msg
    if msg:
        assert msg in e.value.msg


SPACING_OK = [
    (".address_size 64", ".address_size 64 // pointer size", 19),
    (".address_size 64", ".address_size 64 /* pointer\n size */", 19),
    ("    mov.u32 %r2, %tid.x;", "    .loc 1 2 0 /* source */\n    mov.u32 %r2, %tid.x;", 19),
    # a line-scoped directive runs to the end of its line, comments removed
    ("    mov.u32 %r2, %tid.x;", "    .loc 1 2 0 /* source */ mov.u32 %r2, %tid.x;", 18),
    ("    mov.u32 %r2, %tid.x;", "    .loc 1 2 0 /* source\n */ mov.u32 %r2, %tid.x;", 19),
    ("    mov.u32 %r2, %tid.x;", "    /* a\n */ .loc 1 2 0\n    mov.u32 %r2, %tid.x;", 19),
    ("ld.global.f32 %f1, [%rd5];", "ld.global.f32 %f1, [%rd5 + 4];", 19),
    ("ld.global.f32 %f1, [%rd5];", "ld.global.f32 %f1, [%rd5+-4];", 19),
    ("@%p1 bra $L__exit;", "@!%p1 bra $L__exit;", 19),
    (".param .u64 param_b,", ".param .u64 param_b ,", 19),
]


@pytest.mark.parametrize("old,new,n", SPACING_OK)
def test_spacing_forms_both_sides_accept(ks, oracle_mod, old, new, n):
    """Comments around header and .loc directives, spaces around an address's '+',
    a negative offset and a spaced comma: the library and the oracle read the same
    program."""
    ptx = W.VECTOR_ADD_PTX.replace(old, new)
    assert ptx != W.VECTOR_ADD_PTX
    p = ks.ks_load_program(ptx)
    info = ks.ks_program_info(p)
    o = oracle_mod.program_info(ptx)
    assert (info["n_instrs"], info["param_bytes"]) == (o["n_instrs"], o["param_bytes"]) == (n, 28)
    assert ks.ks_ipdom_table(p) == oracle_mod.ipdom_table(ptx)
    ks.ks_program_free(p)


def _mutate(rnd, t):
    toks = ["%r1", "%rd1", "%p1", "[", "]", "+", "-", ",", ";", "{", "}", ".reg", ".b32", ".u64", "0x", "0f",
            "99999999999999999999", "-2147483649", "@%p1", "@!", "bra", "$L", ":", ".shared", ".align", "<", ">",
            "<0>", "<100000>", "ld.global.u32", "st.shared.b64", "setp.lt.f32", "mul.wide.s32", ".param", "(", ")",
            "\n", " ", "\t", "//", "/*", "*/"]
    for _ in range(rnd.randint(1, 4)):
        k = rnd.randrange(len(t) + 1)
        op = rnd.randrange(4)
        if op == 0:
            t = t[:k] + t[k + rnd.randint(1, 20):]
        elif op == 1:
            t = t[:k] + rnd.choice(toks) + t[k:]
        elif op == 2:
            j = rnd.randrange(len(t) + 1)
            t = t[:k] + t[min(k, j):max(k, j)] + t[k:]
        else:
            t = t[:k]
    return t


def test_parser_differential_on_mutated_programs(ks, oracle_mod):
    """6000 seeded mutations of valid programs (deleted, inserted, duplicated and
    truncated text): the library never accepts a text the oracle rejects, and
    where both accept they read the same program (instructions, parameters,
    shared window, reconvergence table).  The oracle is the more lenient reader
    of malformed text; the library rejects what the subset's grammar does not
    define."""
    import random
    rnd = random.Random(20261202)
    seeds = [W.VECTOR_ADD_PTX, W.STRIDED_PTX, W.bank_probe_ptx(), S.random_cfg_ptx(5, 40), S.block_reduce_ptx(64),
             S.tile_transpose_ptx(1), S.setp_forms_ptx(), S.lcg64_ptx(), S.stencil3_ptx()]
    both = 0
    for _ in range(6000):
        t = _mutate(rnd, rnd.choice(seeds))
        try:
            p = ks.ks_load_program(t)
        except ks.KsError as e:
            assert e.code in (-1, -2), e
            continue
        li = ks.ks_program_info(p)
        lt = ks.ks_ipdom_table(p)
        ks.ks_program_free(p)
        o = oracle_mod.program_info(t)  # raises if the oracle rejects what the library took
        assert (li["n_instrs"], li["n_params"], li["param_bytes"], li["shared_bytes"]) == \
            (o["n_instrs"], o["n_params"], o["param_bytes"], o["shared_bytes"]), t
        assert lt == oracle_mod.ipdom_table(t), t
        both += 1
    assert both > 20


def test_layout_and_default_config(ks):
    p = ks.ks_load_program(W.VECTOR_ADD_PTX)
    cfg = ks.ks_default_config()
    assert list(cfg.latency)[:14] == [4, 4, 4, 4, 4, 4, 4, 200, 23, 200, 23, 4, 20, 4]
    cfg.max_grid = ks.ks_dim3(4, 1, 1)
    cfg.max_block = ks.ks_dim3(256, 1, 1)
    cfg.trace_cap = 32
    lay = ks.ks_query_layout(p, cfg)
    assert lay.warps_per_block == 8 and lay.n_warps == 32
    assert lay.slot_bytes == 16 + 8 * 32 and lay.trace_bytes == 32 * lay.slot_bytes
    assert lay.counters_bytes == 32 * 80
    # oracle and library agree on the default latency table
    ks.ks_program_free(p)


def test_zero_or_oversized_shapes_are_invalid(ks):
    """A grid or block with a zero dimension, or a block of more than 1024 threads,
    is an invalid argument when the buffers are sized (an empty launch is refused,
    not run as a no-op)."""
    p = ks.ks_load_program(W.VECTOR_ADD_PTX)
    cfg = ks.ks_default_config()
    cfg.gmem_bytes = 1 << 16
    for g, b in (((0, 1, 1), (32, 1, 1)), ((1, 0, 1), (32, 1, 1)), ((1, 1, 0), (32, 1, 1)),
                 ((1, 1, 1), (0, 1, 1)), ((1, 1, 1), (32, 0, 1)), ((1, 1, 1), (32, 1, 0)),
                 ((1, 1, 1), (1025, 1, 1)), ((1, 1, 1), (32, 32, 2))):
        cfg.max_grid = ks.ks_dim3(*g)
        cfg.max_block = ks.ks_dim3(*b)
        with pytest.raises(ks.KsError) as e:
            ks.ks_query_layout(p, cfg)
        assert e.value.code == -3, (g, b)
    cfg.max_grid = ks.ks_dim3(1, 1, 1)
    cfg.max_block = ks.ks_dim3(1024, 1, 1)
    assert ks.ks_query_layout(p, cfg).warps_per_block == 32
    ks.ks_program_free(p)


def test_extended_layout_any_grid(ks):
    """Extended slots hold 16-byte records, for a grid of any size (ks_run launches
    it KS_EXT_MAX_BLOCKS blocks at a time); the basic format likewise."""
    p = ks.ks_load_program(W.VECTOR_ADD_PTX)
    cfg = ks.ks_default_config()
    cfg.max_block = ks.ks_dim3(256, 1, 1)
    cfg.trace_cap = 32
    cfg.trace_format = ks.KS_TRACE_EXTENDED
    cfg.max_grid = ks.ks_dim3(ks.KS_EXT_MAX_BLOCKS // 2, 2, 1)
    lay = ks.ks_query_layout(p, cfg)
    assert lay.slot_bytes == 16 + 16 * 32 and lay.n_warps == 8 * ks.KS_EXT_MAX_BLOCKS
    cfg.max_grid = ks.ks_dim3(65536, 1, 1)
    lay = ks.ks_query_layout(p, cfg)
    assert lay.n_warps == 8 * 65536 and lay.trace_bytes == 8 * 65536 * (16 + 16 * 32)
    cfg.trace_format = ks.KS_TRACE_BASIC
    assert ks.ks_query_layout(p, cfg).n_warps == 8 * 65536
    ks.ks_program_free(p)


def test_extended_block_limit(ks):
    """Extended records run blocks up to the extended kernels' register budgets:
    KS_EXT64_MAX_BLOCK_THREADS for a program of more than 32 register slots,
    KS_EXT_MAX_BLOCK_THREADS (the block maximum) otherwise; the basic format runs
    every block size."""
    from workloads.randprog import random_program
    p = ks.ks_load_program(random_program(0, n_threads=1024)[0])
    cfg = ks.ks_default_config()
    cfg.trace_format = ks.KS_TRACE_EXTENDED
    cfg.max_block = ks.ks_dim3(ks.KS_EXT64_MAX_BLOCK_THREADS, 1, 1)
    ks.ks_query_layout(p, cfg)
    cfg.max_block = ks.ks_dim3(ks.KS_EXT64_MAX_BLOCK_THREADS + 1, 1, 1)
    with pytest.raises(ks.KsError) as e:
        ks.ks_query_layout(p, cfg)
    assert e.value.code == -2 and "%d threads" % ks.KS_EXT64_MAX_BLOCK_THREADS in e.value.msg
    cfg.trace_format = ks.KS_TRACE_BASIC
    cfg.max_block = ks.ks_dim3(1024, 1, 1)
    ks.ks_query_layout(p, cfg)
    ks.ks_program_free(p)
    q = ks.ks_load_program(W.bank_probe_ptx())
    cfg.trace_format = ks.KS_TRACE_EXTENDED
    cfg.max_block = ks.ks_dim3(ks.KS_EXT_MAX_BLOCK_THREADS, 1, 1)
    ks.ks_query_layout(q, cfg)
    ks.ks_program_free(q)
    assert ks.KS_EXT_MAX_BLOCK_THREADS == ks.KS_MAX_BLOCK_THREADS


def test_static_binding_refuses_programs_beyond_its_scratch(ks):
    """ks_alloc_state_static holds at most KS_STATIC_MAX_INSTRS decoded
    instructions; a longer program is refused before any device work."""
    from workloads.randprog import random_program
    ptx = random_program(0, n_instr=ks.KS_STATIC_MAX_INSTRS + 100, n_threads=256)[0]
    p = ks.ks_load_program(ptx)
    assert ks.ks_program_info(p)["n_instrs"] > ks.KS_STATIC_MAX_INSTRS
    cfg = ks.ks_default_config()
    cfg.max_block = ks.ks_dim3(256, 1, 1)
    cfg.gmem_bytes = 1 << 20
    with pytest.raises(ks.KsError) as e:
        ks.ks_alloc_state_static(p, cfg, 1, 2, 3)  # dummy buffers: refused before they are used
    assert e.value.code == -2 and "%d instructions" % ks.KS_STATIC_MAX_INSTRS in e.value.msg
    ks.ks_program_free(p)


def test_cache_model_layout_and_limits(ks, oracle_mod):
    """The cache model adds KS_CACHE_WARP_BYTES of state per warp (the oracle's
    layout), refuses extended records and memories above 2^38 bytes, and needs
    its 16-byte aligned buffer at allocation; an unknown model is an invalid argument."""
    p = ks.ks_load_program(W.VECTOR_ADD_PTX)
    cfg = ks.ks_default_config()
    assert list(cfg.latency)[14:17] == [28, 150, 400] and cfg.cache_model == ks.KS_CACHE_NONE
    cfg.max_grid = ks.ks_dim3(4, 1, 1)
    cfg.max_block = ks.ks_dim3(256, 1, 1)
    cfg.gmem_bytes = 1 << 20
    assert ks.ks_query_layout(p, cfg).cache_bytes == 0
    cfg.cache_model = ks.KS_CACHE_WARP
    lay = ks.ks_query_layout(p, cfg)
    assert ks.KS_CACHE_WARP_BYTES == oracle_mod.CACHE_WARP_BYTES == 200720
    assert lay.cache_bytes == 32 * ks.KS_CACHE_WARP_BYTES
    with pytest.raises(ks.KsError) as e:
        ks.ks_alloc_state(p, cfg, 1, 1, 1, 0)
    assert e.value.code == -3 and "cache buffer" in e.value.msg
    with pytest.raises(ks.KsError) as e:  # the kernel clears the state with 16-byte stores
        ks.ks_alloc_state(p, cfg, 1, 1, 1, 4104)
    assert e.value.code == -3 and "16-byte aligned" in e.value.msg
    cfg.gmem_bytes = (1 << 38) + 4096
    with pytest.raises(ks.KsError) as e:
        ks.ks_query_layout(p, cfg)
    assert e.value.code == -2
    cfg.gmem_bytes = 1 << 20
    cfg.trace_format = ks.KS_TRACE_EXTENDED
    with pytest.raises(ks.KsError) as e:
        ks.ks_query_layout(p, cfg)
    assert e.value.code == -2 and "basic trace" in e.value.msg
    cfg.trace_format = ks.KS_TRACE_BASIC
    cfg.cache_model = 7
    with pytest.raises(ks.KsError) as e:
        ks.ks_query_layout(p, cfg)
    assert e.value.code == -3
    ks.ks_program_free(p)


def test_default_latency_matches_oracle(ks, oracle_mod):
    assert list(ks.ks_default_config().latency) == oracle_mod.default_latency()


def test_alloc_rejects_null_buffers(ks):
    p = ks.ks_load_program(W.VECTOR_ADD_PTX)
    cfg = ks.ks_default_config()
    with pytest.raises(ks.KsError) as e:
        ks.ks_alloc_state(p, cfg, 0, 0, 0)
    assert e.value.code == -3
    ks.ks_program_free(p)


def test_program_limits(ks):
    too_many = S.HEADER + ".visible .entry k()\n{\n    .reg .b32 %r<65>;\n    mov.u32 %r64, 1;\n    ret;\n}\n"
    p = ks.ks_load_program(too_many)
    assert ks.ks_program_info(p)["reg_slots"] == 65
    cfg = ks.ks_default_config()
    with pytest.raises(ks.KsError) as e:
        ks.ks_alloc_state(p, cfg, 1, 1, 1)
    assert e.value.code == -2 and "register slots" in e.value.msg
    ks.ks_program_free(p)
    # pcs are 16-bit in the stack entries and extended records: at most KS_MAX_INSTRS
    body = lambda n: S.HEADER + ".visible .entry k()\n{\n    .reg .b32 %r<2>;\n" + "    mov.u32 %r1, 1;\n" * (n - 1) + \
        "    ret;\n}\n"
    p = ks.ks_load_program(body(ks.KS_MAX_INSTRS))
    assert ks.ks_program_info(p)["n_instrs"] == ks.KS_MAX_INSTRS
    ks.ks_program_free(p)
    with pytest.raises(ks.KsError) as e:
        ks.ks_load_program(body(ks.KS_MAX_INSTRS + 1))
    assert e.value.code == -2 and "instructions" in e.value.msg


def test_interp_kernel_choice(ks):
    """Register-file variant: 40 reserved VGPRs when the program needs at most 32
    slots (six more hold immediates, two the f32 constants), else 72; blocks of up
    to 1024 threads."""
    small = ks.ks_load_program(W.vector_add().ptx)
    big = ks.ks_load_program(W.random_stress(prog_seed=0, grid=4, gmem_bytes=1 << 20).ptx)
    edge = {n: ks.ks_load_program(S.HEADER + ".visible .entry k()\n{\n    .reg .b32 %%r<%d>;\n"
                                   "    mov.u32 %%r%d, 1;\n    ret;\n}\n" % (n, n - 1)) for n in (32, 33, 64)}
    try:
        assert ks.ks_program_info(small)["reg_slots"] <= 32
        assert ks.ks_interp_kernel(edge[32], (32,)) == "ks_interp_v32"
        assert ks.ks_interp_kernel(edge[33], (32,)) == "ks_interp_v64"
        assert ks.ks_interp_kernel(edge[64], (32,)) == "ks_interp_v64"
        assert ks.ks_program_info(big)["reg_slots"] == 64
        for block in ((32,), (256,), (1024,), (32, 32)):
            assert ks.ks_interp_kernel(small, block) == "ks_interp_v32"
            assert ks.ks_interp_kernel(big, block) == "ks_interp_v64"
        for bad in ((0,), (1025,), (64, 32)):
            with pytest.raises(ks.KsError):
                ks.ks_interp_kernel(small, bad)
    finally:
        ks.ks_program_free(small)
        ks.ks_program_free(big)
        for p in edge.values():
            ks.ks_program_free(p)


def test_instr_info_maps_pcs_to_source_lines(ks):
    """ks_instr_info: each decoded instruction's PTX line, record kind and access width."""
    import re as _re
    ptx = W.VECTOR_ADD_PTX
    lines = ptx.split("\n")
    p = ks.ks_load_program(ptx)
    try:
        n = ks.ks_program_info(p)["n_instrs"]
        d = [ks.ks_instr_info(p, pc) for pc in range(n)]
        with pytest.raises(ks.KsError):
            ks.ks_instr_info(p, n)
    finally:
        ks.ks_program_free(p)
    texts = [_re.sub(r"^@!?%\w+\s+", "", lines[x["line"] - 1].strip()) for x in d]
    assert [t.split()[0] for t in texts] == (["ld.param.u64"] * 3 + ["ld.param.u32"] + ["mov.u32"] * 3 +
                                             ["mad.lo.s32", "setp.ge.s32", "bra", "mul.wide.s32", "add.s64",
                                              "ld.global.f32", "add.s64", "ld.global.f32", "add.f32", "add.s64",
                                              "st.global.f32", "ret;"])
    assert [x["kind"] for x in d] == [0] * 9 + [5, 0, 0, 1, 0, 1, 0, 0, 2, 8]
    assert [x["access_bytes"] for x in d] == [0] * 12 + [4, 0, 4, 0, 0, 4, 0]
    assert d[15]["lat_class"] == 2 and d[12]["lat_class"] == 7  # add.f32: FP32; ld.global


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with status 2 and says why,
    before touching any device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
