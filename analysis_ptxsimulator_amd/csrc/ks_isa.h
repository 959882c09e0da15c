// ks_isa.h -- decoded-instruction records and launch arguments of libkscope.
//
// Internal to the library: the host encoder (ks_host.cpp) writes these records
// and the gfx950 interpreter (ks_kernel.hip) reads them with scalar loads, one
// 64-byte record per instruction, so that one s_load_dwordx16 fetches it.
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
constexpr uint8_t KS_SB_ZERO = 127;      // scoreboard entry that always reads 0 (no source)
constexpr uint32_t KS_SB_ENTRIES = 129;  // scoreboard words per warp in LDS (odd: warps start in different banks)

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

constexpr int KS_PARAM_MAX = 512;

struct KsArgs {
  const KsInst* prog;
  uint8_t* gmem;
  uint8_t* counters;
  uint8_t* trace;
  uint64_t gmem_bytes;
  uint64_t slot_bytes;
  uint32_t n_instrs;
  uint32_t trace_cap;
  uint32_t max_warp_instrs;
  uint32_t shared_bytes;
  uint32_t grid[3];
  uint32_t block[3];
  uint32_t threads_per_block;
  uint32_t warps_per_block;
  uint32_t lat_bar;
  uint32_t rf_slots;       // 32-bit register slots per simulated thread (LDS register file)
  uint8_t params[KS_PARAM_MAX];
};

}  // namespace ks
