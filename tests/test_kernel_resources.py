"""Resource checks of the gfx950 interpreter kernels (CPU: compile to assembly only).

The VGPR register-file kernels keep simulated registers in VGPRs from a reserved
base (v56, or v64 for the extended-trace and cache-model variants) up, outside the compiler's
allocation; if compiler-written code ever touched them, simulated
register values (and the compiler's own) would be silently corrupted, and if the
kernel's VGPR count did not cover the file, indexed accesses would reach past
the wave's allocation.  These tests compile the kernels and check that no
compiler-allocated instruction names a VGPR at or above the base, that the VGPR
count covers the file and that no kernel spills to scratch, and that the checker
itself rejects assembly that breaks any of these.
"""
import os
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "..", "analysis_ptxsimulator_amd"))
import build as kbuild  # noqa: E402


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(kbuild.HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "k.s")
    return open(kbuild.device_asm(out)).read()


def test_interpreters_leave_reserved_vgprs_alone(asm):
    info = kbuild.check_device_asm(asm)
    for k in kbuild.RESERVED_VGPR_KERNELS:
        assert info[k]["max_compiler_vgpr"] < kbuild.RESERVED_BASE[k]
    for k in kbuild.INTERP_KERNELS:
        assert info[k]["scratch"] == 0


def _fake(kernel, body, scratch=0, vgprs=None):
    name = "_Z%d%sN2ks6KsArgsE" % (len(kernel), kernel)
    text = ""
    for k in kbuild.INTERP_KERNELS:
        n = "_Z%d%sN2ks6KsArgsE" % (len(k), k)
        b = body if k == kernel else "\ts_endpgm\n"
        text += "%s:  ; @%s\n%s.Lfunc_end_%s:\n" % (n, n, b, k)
    for k in kbuild.INTERP_KERNELS:
        n = "_Z%d%sN2ks6KsArgsE" % (len(k), k)
        v = vgprs if (vgprs is not None and n == name) else 200
        text += "  - .name: %s\n    .private_segment_fixed_size: %d\n    .sgpr_count: 90\n    .vgpr_count: %d\n" % (
            n, scratch if n == name else 0, v)
    return text


def test_checker_rejects_compiler_use_of_reserved_vgprs():
    for k in ("ks_interp_v32", "ks_interp_v64", "ks_interp_v64_ext"):
        b = kbuild.RESERVED_BASE[k]
        ok = "\t;;#ASMSTART\n\tv_mov_b32 v3, v%d\n\t;;#ASMEND\n\tv_add_u32_e32 v%d, v1, v2\n" % (b, b - 1)
        kbuild.check_device_asm(_fake(k, ok + "\ts_endpgm\n"))
        for bad in ("\tv_add_u32_e32 v%d, v1, v2\n" % b, "\tv_mov_b64_e32 v[%d:%d], 0\n" % (b - 1, b),
                    "\tglobal_load_dwordx4 v[%d:%d], v[0:1], off\n" % (b + 4, b + 7)):
            with pytest.raises(RuntimeError, match="compiler-allocated code uses v"):
                kbuild.check_device_asm(_fake(k, ok + bad + "\ts_endpgm\n"))


def test_checker_rejects_index_mode_with_a_load_in_flight():
    """VGPR index mode must not be switched on while a vector-memory or LDS load
    may still return into a VGPR; a wait for the counter in between, on every path,
    makes it legal."""
    on = ("\t;;#ASMSTART\n\ts_set_gpr_idx_on s2, gpr_idx(SRC0)\n\tv_mov_b32 v3, v%d\n\ts_set_gpr_idx_off\n"
          "\t;;#ASMEND\n" % kbuild.RESERVED_BASE["ks_interp_v64"])
    vm = "\tglobal_load_dword v4, v[0:1], off\n"
    ds = "\tds_read_b32 v5, v6\n"
    good = [vm + "\ts_waitcnt vmcnt(0)\n" + on, ds + "\ts_waitcnt lgkmcnt(0)\n" + on,
            on + vm + "\ts_waitcnt vmcnt(0)\n",
            # the load is only on the branch that also waits
            "\ts_cbranch_scc1 .LB_1\n" + vm + "\ts_waitcnt vmcnt(0)\n.LB_1:\n" + on]
    bad = [vm + on, ds + on, vm + "\ts_waitcnt lgkmcnt(0)\n" + on,
           "\tscratch_load_dword v7, off, off\n" + on,
           # waits on one path only
           vm + "\ts_cbranch_scc1 .LB_1\n\ts_waitcnt vmcnt(0)\n.LB_1:\n" + on,
           # a load late in a loop body reaches the index mode at its head
           ".LB_0:\n" + on + vm + "\ts_cbranch_scc1 .LB_0\n\ts_waitcnt vmcnt(0)\n"]
    # a flag pair set to a constant decides a vcc branch: the edge it never takes is not followed
    skip = "\ts_mov_b64 s[26:27], 0\n\ts_and_b64 vcc, exec, s[26:27]\n\ts_cbranch_vccz .LB_9\n" + on + ".LB_9:\n"
    good.append(vm + skip)
    skip2 = "\ts_mov_b64 s[26:27], -1\n\ts_andn2_b64 vcc, exec, s[26:27]\n\ts_cbranch_vccnz .LB_9\n\ts_waitcnt vmcnt(0)\n.LB_9:\n" + on
    good.append(vm + skip2)
    # ... but not when the pair is not known to be that constant, or was overwritten
    bad.append(vm + "\ts_mov_b64 s[26:27], -1\n\ts_and_b64 vcc, exec, s[26:27]\n\ts_cbranch_vccz .LB_9\n" + on + ".LB_9:\n")
    bad.append(vm + "\ts_mov_b64 s[26:27], 0\n\ts_and_b64 s[26:27], s[26:27], s[4:5]\n"
               "\ts_or_b64 s[26:27], s[4:5], s[6:7]\n\ts_and_b64 vcc, exec, s[26:27]\n\ts_cbranch_vccz .LB_9\n" + on + ".LB_9:\n")
    bad.append(vm + "\ts_cbranch_scc0 .LB_8\n\ts_mov_b64 s[26:27], 0\n.LB_8:\n\ts_and_b64 vcc, exec, s[26:27]\n"
               "\ts_cbranch_vccz .LB_9\n" + on + ".LB_9:\n")
    for b in good:
        kbuild.check_device_asm(_fake("ks_interp_v64", b + "\ts_endpgm\n"))
    for b in bad:
        with pytest.raises(RuntimeError, match="index mode"):
            kbuild.check_device_asm(_fake("ks_interp_v64", b + "\ts_endpgm\n"))


def test_checker_rejects_a_store_just_before_index_mode():
    """A vector-memory store must be STORE_INDEX_GAP instructions or more ahead of
    the next `s_set_gpr_idx_on` on every path, unless `s_waitcnt vmcnt(0)` comes
    between them; the gap counts instructions, not labels, and a flag-steered
    branch the compiler never takes does not shorten it."""
    on = ("\t;;#ASMSTART\n\ts_set_gpr_idx_on s2, gpr_idx(SRC0)\n\tv_mov_b32 v3, v%d\n\ts_set_gpr_idx_off\n"
          "\t;;#ASMEND\n" % kbuild.RESERVED_BASE["ks_interp_v64"])
    st = "\tglobal_store_dwordx4 v[0:1], v[4:7], off offset:16\n"
    gap = kbuild.STORE_INDEX_GAP

    def pad(n):
        return "".join("\tv_add_u32_e32 v10, v10, v11\n" + (".LB_p%d:\n" % i) for i in range(n))

    good = [st + pad(gap) + on, st + "\ts_waitcnt vmcnt(0)\n" + on, on + st,
            st + pad(3) + "\ts_waitcnt vmcnt(0)\n" + on,
            # the short branch is never taken: the pair is 0, so vcc is 0
            st + "\ts_mov_b64 s[26:27], 0\n\ts_and_b64 vcc, exec, s[26:27]\n\ts_cbranch_vccnz .LB_9\n" + pad(gap)
            + on + "\ts_endpgm\n.LB_9:\n" + on]
    bad = [st + pad(gap - 2) + on, st + pad(3) + "\ts_waitcnt lgkmcnt(0)\n" + on,
           "\tbuffer_store_dword v1, v2, s[4:7], 0 offen\n" + on,
           # waits on one path only
           st + "\ts_cbranch_scc1 .LB_1\n\ts_waitcnt vmcnt(0)\n.LB_1:\n" + on,
           # a store late in a loop reaches the index mode at its head
           ".LB_0:\n" + on + st + "\ts_cbranch_scc1 .LB_0\n"]
    for b in good:
        kbuild.check_device_asm(_fake("ks_interp_v64", b + "\ts_endpgm\n"))
    for b in bad:
        with pytest.raises(RuntimeError, match="store within"):
            kbuild.check_device_asm(_fake("ks_interp_v64", b + "\ts_endpgm\n"))


def test_interpreter_stores_keep_their_gap(asm):
    """Every vector-memory store of the four interpreters is far enough ahead of
    index mode, or followed by a wait for it."""
    import re
    for k in kbuild.INTERP_KERNELS:
        body = re.search(r"^_Z\d+%sN2ks6KsArgsE:[^\n]*\n(.*?)^\.Lfunc_end" % k, asm, re.S | re.M).group(1)
        gaps = kbuild.store_index_gaps(body)
        assert gaps, k
        assert all(g is None or g >= kbuild.STORE_INDEX_GAP for g, _, _ in gaps), (k, gaps)


def test_checker_rejects_short_vgpr_count():
    for k, n in kbuild.RF_VGPRS.items():
        kbuild.check_device_asm(_fake(k, "\ts_endpgm\n", vgprs=kbuild.RESERVED_BASE[k] + n))
        with pytest.raises(RuntimeError, match="does not cover"):
            kbuild.check_device_asm(_fake(k, "\ts_endpgm\n", vgprs=kbuild.RESERVED_BASE[k] + n - 8))


def test_checker_rejects_scratch():
    with pytest.raises(RuntimeError, match="scratch"):
        kbuild.check_device_asm(_fake("ks_interp_v32", "\ts_endpgm\n", scratch=16))
    with pytest.raises(RuntimeError, match="scratch"):
        kbuild.check_device_asm(_fake("ks_interp_v64_ext", "\ts_endpgm\n", scratch=8))


def test_register_file_names_match_the_reserved_base():
    """The interpreter's inline assembly names the register file's first six VGPRs
    (slot 0 onward, offset by the index mode); for every register file they must
    start at the reserved base of the kernels that use it and be consecutive, and
    every VGPR its zeroing names must lie inside the file."""
    import re
    src = open(os.path.join(kbuild.CSRC, "ks_kernel.hip")).read()
    access = src[src.index("#define KS_RF_ASM_ACCESS"):src.index("template <>\nstruct RegFile<40, 56>")]
    assert not re.findall(r'"[^"]*\bv\d+', access.replace('"v_mov_b32 "', '')), "literal VGPR in the accessors"
    specs = re.findall(r"struct RegFile<(\d+), (\d+)> \{\n  KS_RF_ASM_ACCESS\(([^)]*)\)", src)
    assert sorted((int(n), int(b)) for n, b, _ in specs) == [(40, 56), (40, 64), (72, 56), (72, 64)]
    for n, b, names in specs:
        n, b = int(n), int(b)
        assert [int(x) for x in re.findall(r'"v(\d+)"', names)] == list(range(b, b + 6))
        body = src[src.index("struct RegFile<%d, %d>" % (n, b)):]
        body = body[:body.index("};")]
        zero = body[body.index("zero()"):]
        regs = sorted({int(r) for r in re.findall(r'\bv(\d+)\b', zero)})
        assert regs == list(range(b, b + n)), (n, b)
    for k, base in kbuild.RESERVED_BASE.items():
        assert base == (64 if k.endswith("_ext") else 56)
    # each kernel's register file is the one its VGPR budget reserves: amdgpu_num_vgpr(base / 2)
    for k, base in kbuild.RESERVED_BASE.items():
        m = re.search(r"amdgpu_num_vgpr\((\d+)\)\)\) %s\(" % k, src)
        assert m and int(m.group(1)) * 2 == base, k
