"""Seeded random programs of the PTX subset (the 16.8M-thread stress workload).

Construction rules (inputs only; the pages give no generator):

* 64 32-bit register slots in total: 2 scratch words, seven 64-bit registers
  (up to four read bases, the two write bases, one scratch), 24 s32 and 24 f32
  data registers; 8 predicates on top.
* Prologue: gtid = ctaid * ntid + tid; read base k = R + 4 * a_k * gtid with
  a_k in 0..7 (0 makes every lane load the same word); write bases
  W1 + 4 * gtid (stride 1) and W4 + 16 * gtid (stride 4).
* Body mix: 50 % ALU (half s32 add/sub/mul.lo/mad.lo, half f32
  add/sub/mul/fma.rn), 20 % global memory (half loads from R at
  [base_k + 4 b], half stores to the thread's own words of W1 or W4),
  10 % control (setp on data registers, then a guarded forward bra 2..32
  instructions ahead that never passes the final ret), 5 % bar.sync placed
  only where no earlier branch jumps past it (so the warp is converged), the
  rest mov/selp.
* Race freedom: loads only touch R, stores only touch words owned by the
  storing thread, so no thread reads or overwrites another thread's data.
"""
import numpy as np

N_SCRATCH = 2           # 32-bit scratch registers (%t)
N_B64 = 7               # read bases rd0..rd3, write bases rd4 (W1) and rd5 (W4), scratch rd6
N_RBASE_MAX = 4
N_INT = 24              # s32 data registers
N_FLT = 24              # f32 data registers: 2 + 7 * 2 + 24 + 24 = 64 slots
N_PRED = 8
B_WORDS = 4096          # load offsets b are drawn from [0, B_WORDS)


def random_program(seed: int, n_instr: int = 2000, n_threads: int = 1 << 24, r_bytes: int = 1 << 29,
                   w1_bytes: int = 1 << 28, w4_bytes: int = 1 << 28):
    rng = np.random.default_rng(seed)
    assert 4 * n_threads * 4 <= w1_bytes, "W1 too small for 4 words per thread"
    assert 16 * n_threads <= w4_bytes, "W4 too small for 4 words per thread"
    n_rb = int(rng.integers(2, N_RBASE_MAX + 1))
    a_k = [int(x) for x in rng.integers(0, 8, size=n_rb)]
    # every load stays inside R
    assert 4 * max(a_k + [0]) * (n_threads - 1) + 4 * B_WORDS <= r_bytes

    body = []   # list of (kind, text) with branch targets resolved later

    # gtid in %t0; %rd6 is a scratch 64-bit register for the bases
    pro = [
        "ld.param.u64 %rd6, [param_r];",
        "mov.u32 %t1, %ctaid.x;",
        "mov.u32 %t0, %ntid.x;",
        "mul.lo.s32 %t0, %t0, %t1;",
        "mov.u32 %t1, %tid.x;",
        "add.s32 %t0, %t0, %t1;",
    ]
    for k in range(n_rb):
        pro.append("mul.wide.u32 %%rd%d, %%t0, %d;" % (k, 4 * a_k[k]))
        pro.append("add.s64 %%rd%d, %%rd%d, %%rd6;" % (k, k))
    pro += [
        "ld.param.u64 %rd6, [param_w1];",
        "mul.wide.u32 %rd4, %t0, 4;",
        "add.s64 %rd4, %rd4, %rd6;",
        "ld.param.u64 %rd6, [param_w4];",
        "mul.wide.u32 %rd5, %t0, 16;",
        "add.s64 %rd5, %rd5, %rd6;",
    ]

    n_body = n_instr - len(pro) - 1  # final ret
    assert n_body > 100
    kinds = rng.choice(["alu_i", "alu_f", "ld", "st", "setp", "bra", "bar", "mov"],
                       size=n_body, p=[0.25, 0.25, 0.10, 0.10, 0.05, 0.05, 0.05, 0.15])
    ret_index = len(pro) + n_body
    preds_set = []
    pending_bar = 0
    max_target = 0            # largest branch target seen so far (absolute index)
    int_regs = ["%%r%d" % i for i in range(N_INT)]
    flt_regs = ["%%f%d" % i for i in range(N_FLT)]

    def pick(lst):
        return lst[int(rng.integers(0, len(lst)))]

    def f32_imm():
        return "0f%08X" % int(rng.integers(0, 1 << 32))

    for i in range(n_body):
        pos = len(pro) + i
        kind = str(kinds[i])
        converged = max_target <= pos
        if kind == "bar" and not converged:
            pending_bar += 1
            kind = "alu_i"
        elif pending_bar and converged and kind in ("alu_i", "alu_f", "mov"):
            pending_bar -= 1
            kind = "bar"
        if kind == "alu_i":
            op = pick(["add.s32", "sub.s32", "mul.lo.s32", "mad.lo.s32"])
            d, a, b = pick(int_regs), pick(int_regs), pick(int_regs)
            if rng.random() < 0.15:
                b = str(int(rng.integers(-1000, 1000)))
            if op == "mad.lo.s32":
                body.append("%s %s, %s, %s, %s;" % (op, d, a, b, pick(int_regs)))
            else:
                body.append("%s %s, %s, %s;" % (op, d, a, b))
        elif kind == "alu_f":
            op = pick(["add.f32", "sub.f32", "mul.f32", "fma.rn.f32"])
            d, a, b = pick(flt_regs), pick(flt_regs), pick(flt_regs)
            if rng.random() < 0.1:
                b = f32_imm()
            if op == "fma.rn.f32":
                body.append("%s %s, %s, %s, %s;" % (op, d, a, b, pick(flt_regs)))
            else:
                body.append("%s %s, %s, %s;" % (op, d, a, b))
        elif kind == "ld":
            k = int(rng.integers(0, n_rb))
            b = int(rng.integers(0, B_WORDS))
            off = "" if b == 0 else "+%d" % (4 * b)
            if rng.random() < 0.5:
                body.append("ld.global.u32 %s, [%%rd%d%s];" % (pick(int_regs), k, off))
            else:
                body.append("ld.global.f32 %s, [%%rd%d%s];" % (pick(flt_regs), k, off))
        elif kind == "st":
            j = int(rng.integers(0, 4))
            if rng.random() < 0.5:
                addr = "[%%rd4%s]" % ("" if j == 0 else "+%d" % (4 * j * n_threads))
            else:
                addr = "[%%rd5%s]" % ("" if j == 0 else "+%d" % (4 * j))
            if rng.random() < 0.5:
                body.append("st.global.u32 %s, %s;" % (addr, pick(int_regs)))
            else:
                body.append("st.global.f32 %s, %s;" % (addr, pick(flt_regs)))
        elif kind == "setp":
            p = int(rng.integers(0, N_PRED))
            cmp = pick(["lt", "le", "gt", "ge", "eq", "ne"])
            if rng.random() < 0.5:
                typ = pick(["s32", "u32"])
                body.append("setp.%s.%s %%p%d, %s, %s;" % (cmp, typ, p, pick(int_regs), pick(int_regs)))
            else:
                body.append("setp.%s.f32 %%p%d, %s, %s;" % (cmp, p, pick(flt_regs), pick(flt_regs)))
            if p not in preds_set:
                preds_set.append(p)
        elif kind == "bra":
            if not preds_set:
                body.append("mov.b32 %s, %s;" % (pick(int_regs), pick(int_regs)))
                continue
            p = pick(preds_set)
            dist = int(rng.integers(2, 33))
            target = min(pos + dist, ret_index)
            max_target = max(max_target, target)
            neg = "!" if rng.random() < 0.5 else ""
            body.append(("BRA", "@%s%%p%d bra $L__t%d;" % (neg, p, target), target))
        elif kind == "bar":
            body.append("bar.sync 0;")
        else:
            r = rng.random()
            if r < 0.35:
                body.append("mov.b32 %s, %s;" % (pick(int_regs), pick(int_regs)))
            elif r < 0.5:
                body.append("mov.f32 %s, %s;" % (pick(flt_regs), f32_imm()))
            elif r < 0.6:
                body.append("mov.u32 %s, %d;" % (pick(int_regs), int(rng.integers(0, 1 << 31))))
            elif preds_set and r < 0.8:
                body.append("selp.b32 %s, %s, %s, %%p%d;" % (pick(int_regs), pick(int_regs), pick(int_regs),
                                                             pick(preds_set)))
            elif preds_set:
                body.append("selp.f32 %s, %s, %s, %%p%d;" % (pick(flt_regs), pick(flt_regs), pick(flt_regs),
                                                             pick(preds_set)))
            else:
                body.append("mov.b32 %s, %s;" % (pick(int_regs), pick(int_regs)))

    code = pro + body + ["ret;"]
    targets = set()
    for c in code:
        if isinstance(c, tuple):
            targets.add(c[2])
    lines = [".version 7.5", ".target sm_80", ".address_size 64", "",
             ".visible .entry random_stress(",
             "    .param .u64 param_r,", "    .param .u64 param_w1,", "    .param .u64 param_w4", ")", "{",
             "    .reg .pred %%p<%d>;" % N_PRED,
             "    .reg .b32 %%t<%d>;" % N_SCRATCH,
             "    .reg .b64 %%rd<%d>;" % N_B64,
             "    .reg .s32 %%r<%d>;" % N_INT,
             "    .reg .f32 %%f<%d>;" % N_FLT,
             ]
    out_lines = []
    for idx, c in enumerate(code):
        if idx in targets:
            out_lines.append("$L__t%d:" % idx)
        text = c[1] if isinstance(c, tuple) else c
        out_lines.append("    " + text)
    if len(code) in targets:
        out_lines.append("$L__t%d:" % len(code))
    src = "\n".join(lines + out_lines + ["}"]) + "\n"
    meta = {"n_instr": len(code), "a_k": a_k, "n_read_bases": n_rb, "reg_slots": 64}
    return src, meta
