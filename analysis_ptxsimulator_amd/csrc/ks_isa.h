// ks_isa.h -- decoded-instruction records and launch arguments of libkscope.
//
// Internal to the library.  The front end (ks_host.cpp) parses PTX into KsInst
// records (one per instruction, operand kinds kept as written); when a state is
// allocated they are lowered to DInst records, the form the gfx950 interpreter
// (ks_kernel.hip) executes: every field the per-instruction path reads is a
// whole dword, so the interpreter reads it with a scalar load and no bit
// extraction, and operations are grouped into classes whose variants differ
// only in per-instruction constants.
#pragma once
#include <stdint.h>

namespace ks {

// Kernel opcodes: one per (operation, width/type class) so that the interpreter
// dispatches once per instruction.
enum KOp : uint8_t {
  KO_ADD32, KO_SUB32, KO_MUL32, KO_MAD32,
  KO_ADD64, KO_SUB64, KO_MUL64, KO_MAD64,
  KO_MULWIDE_S, KO_MULWIDE_U,
  KO_FADD, KO_FSUB, KO_FMUL, KO_FFMA,
  KO_SETP_S32, KO_SETP_U32, KO_SETP_S64, KO_SETP_U64, KO_SETP_F32,
  KO_SELP32, KO_SELP64, KO_MOV32, KO_MOV64,
  KO_LDP32, KO_LDP64,
  KO_LDG32, KO_LDG64, KO_STG32, KO_STG64,
  KO_LDS32, KO_LDS64, KO_STS32, KO_STS64,
  KO_BRA, KO_BAR, KO_RET,
  KO_COUNT
};

// Operand kinds (2 bits per source in KsInst::kinds).
enum : uint8_t { KK_NONE = 0, KK_REG = 1, KK_IMM = 2, KK_SPECIAL = 3 };

// Special register ids (KK_SPECIAL sources).
enum : uint8_t {
  KSP_TID_X, KSP_TID_Y, KSP_TID_Z, KSP_NTID_X, KSP_NTID_Y, KSP_NTID_Z,
  KSP_CTAID_X, KSP_CTAID_Y, KSP_CTAID_Z, KSP_NCTAID_X, KSP_NCTAID_Y, KSP_NCTAID_Z, KSP_LANEID
};

// setp comparison codes.
enum : uint8_t { KC_EQ, KC_NE, KC_LT, KC_LE, KC_GT, KC_GE };

// flags
enum : uint8_t { KF_GUARD = 1, KF_GUARD_NEG = 2 };

constexpr uint8_t KS_NO_SB = 0xFF;      // no scoreboard entry
constexpr uint16_t KS_RPC_EXIT = 0xFFFF;
constexpr uint32_t KS_SB_PRED_BASE = 64; // scoreboard index of predicate p = 64 + p
constexpr uint8_t KS_SB_DUMP = 126;      // scoreboard entry written by instructions without a destination
constexpr uint8_t KS_SB_ZERO = 127;      // scoreboard entry that always reads 0 (no source)
// Two scoreboard words no instruction names (registers use 0-63, predicates 64-95):
// at each barrier release a warp keeps its issue count and its next issue cycle
// from before the release there, so that a warp whose last issue was the bar.sync
// reports cycles = that issue + 1 however late the release.
constexpr uint8_t KS_SB_BAR_WI = 124;
constexpr uint8_t KS_SB_BAR_NEXT = 125;
constexpr uint32_t KS_SB_ENTRIES = 129;  // scoreboard words per warp in LDS (odd: warps start in different banks)
// LDS words per warp of the basic-record interpreters: the 129 scoreboard words, a
// pad word, then a ring of 32 staged {issue cycle, pc} trace records (record k in
// slot k % 32) from word KS_SB_RING on; 194 is not a multiple of the 32 banks.
constexpr uint32_t KS_SB_STRIDE = 194;
constexpr uint32_t KS_SB_RING = 130;
constexpr uint32_t KS_IMM_SLOTS = 6;     // register slots after the program's that hold an instruction's immediates
constexpr uint32_t KS_CONST_SLOTS = 2;   // then two slots holding 1.0f and -0.0f (f32 add/sub and mul operands)
constexpr uint32_t KS_PREFETCH_PAD = 4;  // zero records after the end sentinel: reads ahead stay in bounds

struct KsInst {            // 64 bytes
  uint8_t op;              // KOp
  uint8_t flags;           // KF_*
  uint8_t dst;             // destination slot (low slot of a 64-bit register) or predicate
  uint8_t guard;           // guard predicate index
  uint8_t src[3];          // register slot, special id or (selp's third) predicate index
  uint8_t kinds;           // 2 bits per source, KK_*
  uint8_t sb[4];           // scoreboard index of src0, src1, src2, guard (host: KS_NO_SB; device table: KS_SB_ZERO)
  uint8_t sb_dst;          // scoreboard index of the destination (KS_NO_SB = none)
  uint8_t cmp;             // KC_* for setp
  uint16_t lat;            // latency of the destination (cycles)
  uint16_t target;         // branch target index
  uint16_t rpc;            // reconvergence index of a divergent branch, KS_RPC_EXIT = exit
  uint16_t aux;            // ld.param: byte offset in the parameter block
  uint16_t pad0;
  uint64_t imm[3];         // immediate value of each KK_IMM source
  int64_t off;             // ld/st: byte offset added to the address register
  uint64_t pad1;
};
static_assert(sizeof(KsInst) == 64, "KsInst must be 64 bytes");

// ---------------------------------------------------------------- device records
//
// Interpreter classes.  Register-writing classes first (their issue ends with
// pc + 1), then memory, then control.
enum DClass : uint32_t {
  DC_FMA,      // f32 add/sub/mul/fma as one rounding: r = fma(x0, x1, x2 ^ a2) (1.0 / -0.0 from the constant slots)
  DC_IADD,     // add/sub.{s,u}32: r = x0 + (x1 ^ a0) + a1
  DC_IMAD,     // mul.lo/mad.lo.{s,u}32: r = x0 * x1 + (x2 & a0)
  DC_MOV,      // mov (register or immediate); a0 = 1: 64-bit
  DC_SETP,     // setp; a0 = DS_* operand type, a1 = relation mask (bit0 lt, bit1 eq, bit2 gt)
  DC_SELP,     // selp; s2 = predicate index; a0 = 1: 64-bit
  DC_I64,      // 64-bit integer ops and mul.wide; a0 = DI_*
  DC_MOVSP,    // mov from a special register; a0 = KSP_*
  DC_LDP,      // ld.param; a0 = byte offset in the parameter block, a1 = 1: 64-bit
  DC_LDG,      // ld.global 32-bit through a 64-bit address register; (a0, a1) = byte offset
  DC_STG,      // st.global 32-bit through a 64-bit address register; (a0, a1) = byte offset
  DC_MEMG,     // other ld/st.global; XF_LOAD, XF_W64, XF_A64; (a0, a1) = byte offset (signed 64-bit)
  DC_MEMS,     // ld/st.shared; as DC_MEMG
  DC_BRA,      // bra; a0 = target, a1 = reconvergence index (0xFFFFFFFF = exit)
  DC_BAR,      // bar.sync 0
  DC_RET,      // ret / exit
  DC_END,      // sentinel after the last instruction: lanes that get here exit at no cost
  DC_COUNT
};
constexpr uint32_t CB(uint32_t c) { return 1u << c; }  // class bit in DInst::ctl
// classes that write a register (or predicate) and continue at pc + 1
constexpr uint32_t CB_REG = CB(DC_FMA) | CB(DC_IADD) | CB(DC_IMAD) | CB(DC_MOV) | CB(DC_SETP) | CB(DC_SELP) |
                            CB(DC_I64) | CB(DC_MOVSP) | CB(DC_LDP);
constexpr uint32_t CB_MEM = CB(DC_MEMG) | CB(DC_MEMS);  // the general memory classes
constexpr uint32_t CB_CTRL = CB(DC_BRA) | CB(DC_BAR) | CB(DC_RET);  // classes that set the next pc

enum : uint32_t { DS_S32, DS_U32, DS_F32, DS_S64, DS_U64 };                 // DC_SETP operand types
enum : uint32_t { DI_ADD, DI_SUB, DI_MUL, DI_MAD, DI_WIDE_S, DI_WIDE_U };  // DC_I64 operations

// DInst::ctl flags (above the class bits)
constexpr uint32_t XF_SHIFT = 20;
static_assert(DC_COUNT <= XF_SHIFT, "class bits overlap the flags");
enum : uint32_t {
  XF_IMM = 1u << XF_SHIFT,        // some source is an immediate: imm[] goes into the immediate slots first
  XF_FIX = 1u << (XF_SHIFT + 1),  // the end sentinel, or a divergent branch reconverges here
  XF_LOAD = 1u << (XF_SHIFT + 2), // memory: load (else store)
  XF_W64 = 1u << (XF_SHIFT + 3),  // memory: 8-byte access
  XF_A64 = 1u << (XF_SHIFT + 4),  // memory: 64-bit address register
};
// DInst::ctl bits 25-31: length of the straight run that starts here (1..127):
// the instructions from here on that the interpreter may issue back to back
// without rescheduling.  None is a control class (a control instruction has run
// length 1 and is issued on its own), and only the first may be a reconvergence
// point.
constexpr uint32_t RUN_SHIFT = 25, RUN_MAX = 127;

struct DInst {         // 128 bytes; dwords 0-15 are read for every instruction
  uint32_t ctl;        // CB(class) | XF_* flags
  uint32_t a2;         // class-specific
  uint32_t s0, s1, s2; // source register slots (immediates: the immediate slots)
  uint32_t dst;        // destination slot (low slot of a 64-bit register) or predicate index
  uint32_t sbo[4];     // byte offsets in the warp's scoreboard of src0, src1, src2 and the guard
  uint32_t sbod;       // byte offset of the destination's scoreboard word (the dump word if none)
  uint32_t lat;        // cycles until the destination is ready
  uint32_t gp;         // guard predicate index
  uint32_t gmode;      // 0: @p, 1: @!p, 2: unguarded (compared with the predicate bit: on = bit != gmode)
  uint32_t a0, a1;     // class-specific
  uint32_t imm[6];     // immediate slot values: source k at imm[2k] (low) and imm[2k+1] (high)
  uint32_t nsbo[4];    // sbo[] of the next record: its issue cycle is read without waiting for it
  uint32_t pad[6];
};
static_assert(sizeof(DInst) == 128, "DInst must be 128 bytes");

constexpr int KS_PARAM_MAX = 512;

struct KsArgs {
  const DInst* prog;
  uint8_t* gmem;
  uint8_t* counters;
  uint8_t* trace;
  uint64_t gmem_bytes;
  uint64_t slot_bytes;
  uint32_t n_instrs;       // instructions (the device table holds n_instrs + 1 records: DC_END last)
  uint32_t trace_cap;
  uint32_t max_warp_instrs;
  uint32_t shared_bytes;
  uint32_t grid[3];
  uint32_t block[3];
  uint32_t threads_per_block;
  uint32_t warps_per_block;
  uint32_t lat_bar;
  uint32_t rf_slots;       // register slots per simulated thread, immediate and constant slots included
  uint32_t cyc_safe;       // a run may continue past its first instruction when that one issues
                           // at most at this cycle: RUN_MAX issues cannot then pass the cycle limit
  uint32_t ext;            // 1: extended 16-byte trace records (KS_TRACE_EXTENDED)
  uint8_t* cache;          // cache model (KS_CACHE_WARP): KS_CACHE_WARP_BYTES of state per warp
  uint32_t cache_on;       // 1: the cache model is on
  uint32_t lat_l1, lat_l2, lat_dram;  // its latencies
  uint32_t div_bx, div_by, div_bxy;  // ceil(2^22 / d) for d = block x, y and x * y (special registers)
  uint32_t block_base;     // block id of the launch's first workgroup (launches over part of a grid)
  uint8_t params[KS_PARAM_MAX];
};

}  // namespace ks
