// ks_kernel.hip -- the gfx950 SIMT interpreter of libkscope.
//
// Mapping (CDNA4, wave64):
//   * one workgroup = one simulated block; wave w runs simulated warps 2w
//     (lanes 0-31) and 2w+1 (lanes 32-63), one GPU lane per simulated thread;
//   * each wave step executes ONE decoded instruction: the one at the smaller pc
//     of the two warps (both warps run it when they share that pc), so fetch
//     (scalar loads), dispatch and register slot indices are wave-uniform;
//   * simulated registers live in a register file of 32-bit slots per lane in
//     physical VGPRs reserved for it (v56 upward, reached through the VGPR
//     index mode of s_set_gpr_idx_on: exec-masked, no memory traffic).  Six
//     slots after the program's hold the current instruction's immediates, so
//     every source operand is a register read;
//   * lane masks of the two warps are 64-bit scalars (warp 2w in the low half),
//     so one scalar operation updates both; per-warp values that the lanes use
//     (next issue cycle, instruction count, trace state) are VGPRs that are
//     uniform over each warp's 32 lanes; the divergence stack, counters and a
//     32-record trace staging buffer live in VGPR lanes (16-byte extended
//     records: a 32-record ring per warp in LDS); the register scoreboard of
//     each warp is an LDS array;
//   * trace flushes, the issue budget and the cycle limit are one per-lane
//     comparison per step against a precomputed event threshold;
//   * the analyser counts distinct sectors/lines of monotone addresses with a
//     DPP prefix-max within each 32-lane half (any active mask) and the bank
//     degree of affine shared accesses in closed form; other patterns take an
//     exact ballot loop over distinct values;
//   * simulated bar.sync maps onto epochs: each wave runs its two warps until
//     both wait or finish, then the workgroup meets at a real barrier and the
//     release cycle is an LDS max-reduction of the arrival cycles.
//
// Semantics (the same written specification the CPU oracle implements):
//   KernelScope backend documentation (github.com/briefgaming/kernelscope):
//   the execution-simulator part (warp of 32, active mask, SIMT stack of
//   (pc, mask, reconvergence pc), if/else executed serially then reconverged),
//   the memory-analysis part (32 banks of 4 bytes, broadcast, 128-byte lines,
//   32-byte sectors) and the latency-model part (per-opcode latencies).  The
//   trace slot follows "CuTeDSL IKET 浅析" (zhen8838.github.io/posts/iket.html),
//   section 2: one slot per warp, a 16-byte header, fixed-size records, records
//   past the cap counted as dropped.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ks.h"
#include "ks_isa.h"
#include "ks_launch.h"

using namespace ks;

namespace {

constexpr uint32_t INF = 0xFFFFFFFFu;
constexpr uint32_t CYCLE_LIMIT = 0x7FFFFFFFu;
constexpr uint64_t LO = 0x00000000FFFFFFFFull, HI = 0xFFFFFFFF00000000ull;
// per-warp run state bits (one scalar for both warps of a wave)
constexpr uint32_t WAIT0 = 1, WAIT1 = 2, DONE0 = 4, DONE1 = 8;

// dword index of each field in the 80-byte counter record; the counter VGPR keeps
// counter d of half h in lane 32 h + d
enum {
  C_TI_LO = 0, C_TI_HI, C_STATUS, C_CYCLES, C_WARP_INSTRS, C_STALL, C_GLD_N, C_GLD_SEC, C_GLD_LINES,
  C_GST_N, C_GST_SEC, C_GST_LINES, C_SH_N, C_SH_SUM, C_SH_MAX, C_DIV, C_BAR, C_FAULT, C_MAXDEPTH, C_RES
};

typedef const __attribute__((address_space(4))) DInst* cdinst;
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));  // the 16 dwords every instruction reads
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t rl(uint32_t v, uint32_t l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, (int)l);
}
// Write the wave-uniform `val` into lane `l` of `old`.
__device__ __forceinline__ uint32_t wl(uint32_t old, uint32_t val, uint32_t l, uint32_t lane) {
  return lane == l ? val : old;
}
__device__ __forceinline__ uint64_t rl64(uint64_t v, uint32_t l) {
  return (uint64_t)rl((uint32_t)v, l) | ((uint64_t)rl((uint32_t)(v >> 32), l) << 32);
}
__device__ __forceinline__ uint64_t ballot(bool c) { return __builtin_amdgcn_ballot_w64(c); }
__device__ __forceinline__ bool lanes(uint64_t m) { return __builtin_amdgcn_inverse_ballot_w64(m); }
__device__ __forceinline__ uint32_t uni(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint32_t popc(uint32_t m) { return (uint32_t)__builtin_popcount(m); }
// a == b ? ~0 : 0 for wave-uniform a, b, as a scalar word.  Written as scalar
// assembly so that the result stays an integer: the optimiser turns the plain
// expression into a boolean, which it keeps as a lane mask across blocks.
__device__ __forceinline__ uint32_t s_eq_mask(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("s_cmp_eq_u32 %1, %2\n\ts_cselect_b32 %0, -1, 0" : "=s"(r) : "s"(a), "s"(b) : "scc");
  return r;
}
// a == 0 ? ~0 : 0, the same way.
__device__ __forceinline__ uint32_t s_zero_mask(uint32_t a) {
  uint32_t r;
  asm("s_cmp_eq_u32 %1, 0\n\ts_cselect_b32 %0, -1, 0" : "=s"(r) : "s"(a) : "scc");
  return r;
}

// ---------------------------------------------------------------------------- register files
//
// RFN = 40 / 72 physical VGPRs vBASE .. vBASE+RFN-1, outside the compiler's
// allocation, hold the register file: slot s of a lane is VGPR v[BASE + s] of
// that lane.  The kernels carry amdgpu_num_vgpr(BASE / 2): on targets with the
// unified VGPR/AGPR file the compiler doubles that figure, so vBASE and up are
// reserved (never allocated).  BASE is 56, except for the extended-trace
// variants (64), whose record payloads need more compiler registers.  A figure
// the launch bound cannot honour is silently ignored, which would hand vBASE+
// back to the allocator; the build checks the assembly for any compiler-written
// use of them and that the kernel's VGPR count covers the file (the zero()
// clobber lists make the compiler count it).

template <int RFN, int BASE>
struct RegFile;

// VGPR index mode: between s_set_gpr_idx_on and s_set_gpr_idx_off the SRC0 (or
// DST) VGPR operand of each VALU instruction is offset by the index held in M0;
// s_set_gpr_idx_idx changes the index without leaving the mode.  V0 .. V5 name
// the first six VGPRs of the register file (V0 = slot 0 before indexing); the
// build's reserved base of each kernel must name the same register.
#define KS_RF_ASM_ACCESS(V0, V1, V2, V3, V4, V5)                                                                           \
  __device__ __forceinline__ uint32_t get(uint32_t s) const {                                      \
    uint32_t r;                                                                                    \
    asm volatile("s_set_gpr_idx_on %1, gpr_idx(SRC0)\n\tv_mov_b32 %0, " V0                  \
                 "\n\ts_set_gpr_idx_off"                                                          \
                 : "=v"(r) : "s"(s) : "m0");                                                      \
    return r;                                                                                      \
  }                                                                                                \
  __device__ __forceinline__ void get2(uint32_t i0, uint32_t i1, uint32_t& a, uint32_t& b) const {  \
    asm volatile("s_set_gpr_idx_on %2, gpr_idx(SRC0)\n\tv_mov_b32 %0, " V0 "\n\t"          \
                 "s_set_gpr_idx_idx %3\n\tv_mov_b32 %1, " V0 "\n\ts_set_gpr_idx_off"         \
                 : "=&v"(a), "=v"(b) : "s"(i0), "s"(i1) : "m0");                                  \
  }                                                                                                \
  __device__ __forceinline__ void get3(uint32_t i0, uint32_t i1, uint32_t i2, uint32_t& a, uint32_t& b, \
                                       uint32_t& c) const {                                        \
    asm volatile("s_set_gpr_idx_on %3, gpr_idx(SRC0)\n\tv_mov_b32 %0, " V0 "\n\t"          \
                 "s_set_gpr_idx_idx %4\n\tv_mov_b32 %1, " V0 "\n\t"                          \
                 "s_set_gpr_idx_idx %5\n\tv_mov_b32 %2, " V0 "\n\ts_set_gpr_idx_off"         \
                 : "=&v"(a), "=&v"(b), "=v"(c) : "s"(i0), "s"(i1), "s"(i2) : "m0");               \
  }                                                                                                \
  __device__ __forceinline__ void put(uint32_t s, uint32_t v) const {                              \
    asm volatile("s_set_gpr_idx_on %0, gpr_idx(DST)\n\tv_mov_b32 " V0 ", %1"                 \
                 "\n\ts_set_gpr_idx_off"                                                          \
                 : : "s"(s), "v"(v) : "m0");                                                      \
  }                                                                                                \
  __device__ __forceinline__ void put2(uint32_t s, uint32_t lo, uint32_t hi) const {               \
    asm volatile("s_set_gpr_idx_on %0, gpr_idx(DST)\n\tv_mov_b32 " V0 ", %1\n\t"           \
                 "v_mov_b32 " V1 ", %2\n\ts_set_gpr_idx_off"                                 \
                 : : "s"(s), "v"(lo), "v"(hi) : "m0");                                            \
  }                                                                                                \
  /* slot s of the lanes in m takes v, the other lanes keep their value: SRC0 and DST */          \
  /* are both indexed, so v_cndmask reads the old value and writes the slot under full exec */    \
  __device__ __forceinline__ void put_m(uint32_t s, uint32_t v, uint64_t m) const {                \
    asm volatile("s_set_gpr_idx_on %0, gpr_idx(SRC0,DST)\n\tv_cndmask_b32_e64 " V0 ", "      \
                 V0 ", %1, %2\n\ts_set_gpr_idx_off"                                          \
                 : : "s"(s), "v"(v), "s"(m) : "m0");                                              \
  }                                                                                                \
  __device__ __forceinline__ void put2_m(uint32_t s, uint32_t lo, uint32_t hi, uint64_t m) const { \
    asm volatile("s_set_gpr_idx_on %0, gpr_idx(SRC0,DST)\n\tv_cndmask_b32_e64 " V0 ", "      \
                 V0 ", %1, %3\n\tv_cndmask_b32_e64 " V1 ", " V1 ", %2, %3\n\t"    \
                 "s_set_gpr_idx_off"                                                               \
                 : : "s"(s), "v"(lo), "v"(hi), "s"(m) : "m0");                                    \
  }                                                                                                \
  __device__ __forceinline__ void put_imm(uint32_t ib, const uint32_t* v) const {                  \
    asm volatile("s_set_gpr_idx_on %0, gpr_idx(DST)\n\t"                                           \
                 "v_mov_b32 " V0 ", %1\n\tv_mov_b32 " V1 ", %2\n\t"                     \
                 "v_mov_b32 " V2 ", %3\n\tv_mov_b32 " V3 ", %4\n\t"                     \
                 "v_mov_b32 " V4 ", %5\n\tv_mov_b32 " V5 ", %6\n\t"                     \
                 "s_set_gpr_idx_off"                                                               \
                 : : "s"(ib), "s"(v[0]), "s"(v[1]), "s"(v[2]), "s"(v[3]), "s"(v[4]), "s"(v[5])     \
                 : "m0");                                                                          \
  }

template <>
struct RegFile<40, 56> {
  KS_RF_ASM_ACCESS("v56", "v57", "v58", "v59", "v60", "v61")
  __device__ __forceinline__ static void zero() {
    asm volatile(
                 "v_mov_b32 v56, 0\n\t""v_mov_b32 v57, 0\n\t""v_mov_b32 v58, 0\n\t""v_mov_b32 v59, 0\n\t"
                 "v_mov_b32 v60, 0\n\t""v_mov_b32 v61, 0\n\t""v_mov_b32 v62, 0\n\t""v_mov_b32 v63, 0\n\t"
                 "v_mov_b32 v64, 0\n\t""v_mov_b32 v65, 0\n\t""v_mov_b32 v66, 0\n\t""v_mov_b32 v67, 0\n\t"
                 "v_mov_b32 v68, 0\n\t""v_mov_b32 v69, 0\n\t""v_mov_b32 v70, 0\n\t""v_mov_b32 v71, 0\n\t"
                 "v_mov_b32 v72, 0\n\t""v_mov_b32 v73, 0\n\t""v_mov_b32 v74, 0\n\t""v_mov_b32 v75, 0\n\t"
                 "v_mov_b32 v76, 0\n\t""v_mov_b32 v77, 0\n\t""v_mov_b32 v78, 0\n\t""v_mov_b32 v79, 0\n\t"
                 "v_mov_b32 v80, 0\n\t""v_mov_b32 v81, 0\n\t""v_mov_b32 v82, 0\n\t""v_mov_b32 v83, 0\n\t"
                 "v_mov_b32 v84, 0\n\t""v_mov_b32 v85, 0\n\t""v_mov_b32 v86, 0\n\t""v_mov_b32 v87, 0\n\t"
                 "v_mov_b32 v88, 0\n\t""v_mov_b32 v89, 0\n\t""v_mov_b32 v90, 0\n\t""v_mov_b32 v91, 0\n\t"
                 "v_mov_b32 v92, 0\n\t""v_mov_b32 v93, 0\n\t""v_mov_b32 v94, 0\n\t""v_mov_b32 v95, 0\n\t"
                 :::
                 "v56", "v57", "v58", "v59", "v60", "v61", "v62", "v63",
                 "v64", "v65", "v66", "v67", "v68", "v69", "v70", "v71",
                 "v72", "v73", "v74", "v75", "v76", "v77", "v78", "v79",
                 "v80", "v81", "v82", "v83", "v84", "v85", "v86", "v87",
                 "v88", "v89", "v90", "v91", "v92", "v93", "v94", "v95");
  }
};

template <>
struct RegFile<72, 56> {
  KS_RF_ASM_ACCESS("v56", "v57", "v58", "v59", "v60", "v61")
  __device__ __forceinline__ static void zero() {
    asm volatile(
                 "v_mov_b32 v56, 0\n\t""v_mov_b32 v57, 0\n\t""v_mov_b32 v58, 0\n\t""v_mov_b32 v59, 0\n\t"
                 "v_mov_b32 v60, 0\n\t""v_mov_b32 v61, 0\n\t""v_mov_b32 v62, 0\n\t""v_mov_b32 v63, 0\n\t"
                 "v_mov_b32 v64, 0\n\t""v_mov_b32 v65, 0\n\t""v_mov_b32 v66, 0\n\t""v_mov_b32 v67, 0\n\t"
                 "v_mov_b32 v68, 0\n\t""v_mov_b32 v69, 0\n\t""v_mov_b32 v70, 0\n\t""v_mov_b32 v71, 0\n\t"
                 "v_mov_b32 v72, 0\n\t""v_mov_b32 v73, 0\n\t""v_mov_b32 v74, 0\n\t""v_mov_b32 v75, 0\n\t"
                 "v_mov_b32 v76, 0\n\t""v_mov_b32 v77, 0\n\t""v_mov_b32 v78, 0\n\t""v_mov_b32 v79, 0\n\t"
                 "v_mov_b32 v80, 0\n\t""v_mov_b32 v81, 0\n\t""v_mov_b32 v82, 0\n\t""v_mov_b32 v83, 0\n\t"
                 "v_mov_b32 v84, 0\n\t""v_mov_b32 v85, 0\n\t""v_mov_b32 v86, 0\n\t""v_mov_b32 v87, 0\n\t"
                 "v_mov_b32 v88, 0\n\t""v_mov_b32 v89, 0\n\t""v_mov_b32 v90, 0\n\t""v_mov_b32 v91, 0\n\t"
                 "v_mov_b32 v92, 0\n\t""v_mov_b32 v93, 0\n\t""v_mov_b32 v94, 0\n\t""v_mov_b32 v95, 0\n\t"
                 "v_mov_b32 v96, 0\n\t""v_mov_b32 v97, 0\n\t""v_mov_b32 v98, 0\n\t""v_mov_b32 v99, 0\n\t"
                 "v_mov_b32 v100, 0\n\t""v_mov_b32 v101, 0\n\t""v_mov_b32 v102, 0\n\t""v_mov_b32 v103, 0\n\t"
                 "v_mov_b32 v104, 0\n\t""v_mov_b32 v105, 0\n\t""v_mov_b32 v106, 0\n\t""v_mov_b32 v107, 0\n\t"
                 "v_mov_b32 v108, 0\n\t""v_mov_b32 v109, 0\n\t""v_mov_b32 v110, 0\n\t""v_mov_b32 v111, 0\n\t"
                 "v_mov_b32 v112, 0\n\t""v_mov_b32 v113, 0\n\t""v_mov_b32 v114, 0\n\t""v_mov_b32 v115, 0\n\t"
                 "v_mov_b32 v116, 0\n\t""v_mov_b32 v117, 0\n\t""v_mov_b32 v118, 0\n\t""v_mov_b32 v119, 0\n\t"
                 "v_mov_b32 v120, 0\n\t""v_mov_b32 v121, 0\n\t""v_mov_b32 v122, 0\n\t""v_mov_b32 v123, 0\n\t"
                 "v_mov_b32 v124, 0\n\t""v_mov_b32 v125, 0\n\t""v_mov_b32 v126, 0\n\t""v_mov_b32 v127, 0\n\t"
                 :::
                 "v56", "v57", "v58", "v59", "v60", "v61", "v62", "v63",
                 "v64", "v65", "v66", "v67", "v68", "v69", "v70", "v71",
                 "v72", "v73", "v74", "v75", "v76", "v77", "v78", "v79",
                 "v80", "v81", "v82", "v83", "v84", "v85", "v86", "v87",
                 "v88", "v89", "v90", "v91", "v92", "v93", "v94", "v95",
                 "v96", "v97", "v98", "v99", "v100", "v101", "v102", "v103",
                 "v104", "v105", "v106", "v107", "v108", "v109", "v110", "v111",
                 "v112", "v113", "v114", "v115", "v116", "v117", "v118", "v119",
                 "v120", "v121", "v122", "v123", "v124", "v125", "v126", "v127");
  }
};

template <>
struct RegFile<40, 64> {
  KS_RF_ASM_ACCESS("v64", "v65", "v66", "v67", "v68", "v69")
  __device__ __forceinline__ static void zero() {
    asm volatile(
                 "v_mov_b32 v64, 0\n\t""v_mov_b32 v65, 0\n\t""v_mov_b32 v66, 0\n\t""v_mov_b32 v67, 0\n\t"
                 "v_mov_b32 v68, 0\n\t""v_mov_b32 v69, 0\n\t""v_mov_b32 v70, 0\n\t""v_mov_b32 v71, 0\n\t"
                 "v_mov_b32 v72, 0\n\t""v_mov_b32 v73, 0\n\t""v_mov_b32 v74, 0\n\t""v_mov_b32 v75, 0\n\t"
                 "v_mov_b32 v76, 0\n\t""v_mov_b32 v77, 0\n\t""v_mov_b32 v78, 0\n\t""v_mov_b32 v79, 0\n\t"
                 "v_mov_b32 v80, 0\n\t""v_mov_b32 v81, 0\n\t""v_mov_b32 v82, 0\n\t""v_mov_b32 v83, 0\n\t"
                 "v_mov_b32 v84, 0\n\t""v_mov_b32 v85, 0\n\t""v_mov_b32 v86, 0\n\t""v_mov_b32 v87, 0\n\t"
                 "v_mov_b32 v88, 0\n\t""v_mov_b32 v89, 0\n\t""v_mov_b32 v90, 0\n\t""v_mov_b32 v91, 0\n\t"
                 "v_mov_b32 v92, 0\n\t""v_mov_b32 v93, 0\n\t""v_mov_b32 v94, 0\n\t""v_mov_b32 v95, 0\n\t"
                 "v_mov_b32 v96, 0\n\t""v_mov_b32 v97, 0\n\t""v_mov_b32 v98, 0\n\t""v_mov_b32 v99, 0\n\t"
                 "v_mov_b32 v100, 0\n\t""v_mov_b32 v101, 0\n\t""v_mov_b32 v102, 0\n\t""v_mov_b32 v103, 0\n\t"
                 :::
                 "v64", "v65", "v66", "v67", "v68", "v69", "v70", "v71",
                 "v72", "v73", "v74", "v75", "v76", "v77", "v78", "v79",
                 "v80", "v81", "v82", "v83", "v84", "v85", "v86", "v87",
                 "v88", "v89", "v90", "v91", "v92", "v93", "v94", "v95",
                 "v96", "v97", "v98", "v99", "v100", "v101", "v102", "v103");
  }
};

template <>
struct RegFile<72, 64> {
  KS_RF_ASM_ACCESS("v64", "v65", "v66", "v67", "v68", "v69")
  __device__ __forceinline__ static void zero() {
    asm volatile(
                 "v_mov_b32 v64, 0\n\t""v_mov_b32 v65, 0\n\t""v_mov_b32 v66, 0\n\t""v_mov_b32 v67, 0\n\t"
                 "v_mov_b32 v68, 0\n\t""v_mov_b32 v69, 0\n\t""v_mov_b32 v70, 0\n\t""v_mov_b32 v71, 0\n\t"
                 "v_mov_b32 v72, 0\n\t""v_mov_b32 v73, 0\n\t""v_mov_b32 v74, 0\n\t""v_mov_b32 v75, 0\n\t"
                 "v_mov_b32 v76, 0\n\t""v_mov_b32 v77, 0\n\t""v_mov_b32 v78, 0\n\t""v_mov_b32 v79, 0\n\t"
                 "v_mov_b32 v80, 0\n\t""v_mov_b32 v81, 0\n\t""v_mov_b32 v82, 0\n\t""v_mov_b32 v83, 0\n\t"
                 "v_mov_b32 v84, 0\n\t""v_mov_b32 v85, 0\n\t""v_mov_b32 v86, 0\n\t""v_mov_b32 v87, 0\n\t"
                 "v_mov_b32 v88, 0\n\t""v_mov_b32 v89, 0\n\t""v_mov_b32 v90, 0\n\t""v_mov_b32 v91, 0\n\t"
                 "v_mov_b32 v92, 0\n\t""v_mov_b32 v93, 0\n\t""v_mov_b32 v94, 0\n\t""v_mov_b32 v95, 0\n\t"
                 "v_mov_b32 v96, 0\n\t""v_mov_b32 v97, 0\n\t""v_mov_b32 v98, 0\n\t""v_mov_b32 v99, 0\n\t"
                 "v_mov_b32 v100, 0\n\t""v_mov_b32 v101, 0\n\t""v_mov_b32 v102, 0\n\t""v_mov_b32 v103, 0\n\t"
                 "v_mov_b32 v104, 0\n\t""v_mov_b32 v105, 0\n\t""v_mov_b32 v106, 0\n\t""v_mov_b32 v107, 0\n\t"
                 "v_mov_b32 v108, 0\n\t""v_mov_b32 v109, 0\n\t""v_mov_b32 v110, 0\n\t""v_mov_b32 v111, 0\n\t"
                 "v_mov_b32 v112, 0\n\t""v_mov_b32 v113, 0\n\t""v_mov_b32 v114, 0\n\t""v_mov_b32 v115, 0\n\t"
                 "v_mov_b32 v116, 0\n\t""v_mov_b32 v117, 0\n\t""v_mov_b32 v118, 0\n\t""v_mov_b32 v119, 0\n\t"
                 "v_mov_b32 v120, 0\n\t""v_mov_b32 v121, 0\n\t""v_mov_b32 v122, 0\n\t""v_mov_b32 v123, 0\n\t"
                 "v_mov_b32 v124, 0\n\t""v_mov_b32 v125, 0\n\t""v_mov_b32 v126, 0\n\t""v_mov_b32 v127, 0\n\t"
                 "v_mov_b32 v128, 0\n\t""v_mov_b32 v129, 0\n\t""v_mov_b32 v130, 0\n\t""v_mov_b32 v131, 0\n\t"
                 "v_mov_b32 v132, 0\n\t""v_mov_b32 v133, 0\n\t""v_mov_b32 v134, 0\n\t""v_mov_b32 v135, 0\n\t"
                 :::
                 "v64", "v65", "v66", "v67", "v68", "v69", "v70", "v71",
                 "v72", "v73", "v74", "v75", "v76", "v77", "v78", "v79",
                 "v80", "v81", "v82", "v83", "v84", "v85", "v86", "v87",
                 "v88", "v89", "v90", "v91", "v92", "v93", "v94", "v95",
                 "v96", "v97", "v98", "v99", "v100", "v101", "v102", "v103",
                 "v104", "v105", "v106", "v107", "v108", "v109", "v110", "v111",
                 "v112", "v113", "v114", "v115", "v116", "v117", "v118", "v119",
                 "v120", "v121", "v122", "v123", "v124", "v125", "v126", "v127",
                 "v128", "v129", "v130", "v131", "v132", "v133", "v134", "v135");
  }
};

// ---------------------------------------------------------------------------- analyser

// Inclusive prefix maximum within each 32-lane half (rows 0-1 and rows 2-3).
__device__ __forceinline__ uint32_t half_prefix_max(uint32_t x) {
  x = umax(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true));  // row_shr:1
  x = umax(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true));  // row_shr:2
  x = umax(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true));  // row_shr:4
  x = umax(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true));  // row_shr:8
  x = umax(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false)); // row_bcast:15 -> rows 1, 3
  return x;
}
// Inclusive prefix sum within each 32-lane half (lanes 31 and 63 hold the totals).
__device__ __forceinline__ uint32_t half_sum(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false); // row_bcast:15 -> rows 1, 3
  return x;
}
// Value of the previous lane in the same half (0 for the first lane of each half).
__device__ __forceinline__ uint32_t prev_in_half(uint32_t x, uint32_t lane) {
  const uint32_t p = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x138, 0xF, 0xF, true);  // wave_shr:1
  return lane == 32u ? 0u : p;
}

// Number of distinct values in {k1[l], k2[l] : l in lanes}.  Full exec required.
__device__ uint32_t distinct2(uint64_t k1, uint64_t k2, uint64_t lanes) {
  uint64_t rem1 = lanes;
  uint64_t rem2 = lanes & ballot(k2 != k1);
  uint32_t n = 0;
  while (rem1 | rem2) {
    const uint64_t key = rem1 ? rl64(k1, (uint32_t)__builtin_ctzll(rem1)) : rl64(k2, (uint32_t)__builtin_ctzll(rem2));
    rem1 &= ~ballot(k1 == key);
    rem2 &= ~ballot(k2 == key);
    ++n;
  }
  return n;
}

// Bank-conflict degree of a shared warp access over `lanes` (full exec required):
// group lanes by bank = (A / 4) mod 32; a bank whose lanes do not all use one
// address contributes its lane count; the degree is the largest, at least 1.
__device__ uint32_t bank_degree(uint64_t A, uint64_t lanes) {
  const uint32_t bank = (uint32_t)(A >> 2) & 31u;
  uint64_t rem = lanes;
  uint32_t deg = 1;
  while (rem) {
    const uint32_t f = (uint32_t)__builtin_ctzll(rem);
    const uint32_t b = rl(bank, f);
    const uint64_t af = rl64(A, f);
    const uint64_t inb = ballot(bank == b) & rem;
    const uint64_t same = ballot(bank == b && A == af) & rem;
    const uint32_t nb = (uint32_t)__builtin_popcountll(inb);
    if (nb >= 2 && same != inb && nb > deg) deg = nb;
    rem &= ~inb;
  }
  return deg;
}

__device__ __forceinline__ uint32_t canon_bits(float r) {
  return __builtin_isnan(r) ? 0x7FFFFFFFu : __float_as_uint(r);
}

// Add v to counter d of the warps in `hm` (bit 0: warp 2w, bit 1: warp 2w+1).
__device__ __forceinline__ uint32_t cnt_add2(uint32_t cnt, uint32_t sl, uint32_t hl, uint32_t d, uint32_t hm, uint32_t v) {
  return cnt + ((sl == d && ((hm >> hl) & 1u)) ? v : 0u);
}

// ---------------------------------------------------------------------------- divergence stack
//
// The top entry of each warp's stack is scalar state: mask (in the 64-bit mask
// pair), reconvergence pc, depth, and pc.  While the warp runs its top pc is its
// scheduled pc; Stk::pc holds it across a barrier wait and inside stack updates.
// Entries below it live in lanes 0..depth-2 of two VGPRs per warp: pc | rpc << 16
// (0xFFFF = exit) and mask.

struct Stk {
  uint32_t pc, rpc, sp, md;   // top pc (see above), top reconvergence pc (INF = exit), depth, maximum depth
  uint32_t pr, m;             // VGPRs: saved entries
};

__device__ __forceinline__ uint32_t enc_rpc(uint32_t r) { return r == INF ? 0xFFFFu : r; }

// Pop: the entry below becomes the top (returns its mask).
__device__ __forceinline__ uint32_t stk_pop(Stk& S) {
  S.sp -= 1;
  uint32_t mask = 0;
  if (S.sp) {
    const uint32_t pr = rl(S.pr, S.sp - 1);
    S.pc = pr & 0xFFFFu;
    S.rpc = (pr >> 16) == 0xFFFFu ? INF : (pr >> 16);
    mask = rl(S.m, S.sp - 1);
  }
  return mask;
}

// Push (pc, rpc) with `mask` over the current top (whose mask is `top_mask`).
__device__ __forceinline__ void stk_push(Stk& S, uint32_t top_mask, uint32_t pc, uint32_t rpc, uint32_t lane) {
  S.pr = wl(S.pr, (S.pc & 0xFFFFu) | (enc_rpc(S.rpc) << 16), S.sp - 1, lane);
  S.m = wl(S.m, top_mask, S.sp - 1, lane);
  S.pc = pc;
  S.rpc = rpc;
  S.sp += 1;
  S.md = umax(S.md, S.sp);
}

// ---------------------------------------------------------------------------- the interpreter

// EXT: extended 16-byte trace records (kind, active mask, payload) written from
// each step, instead of the staged 8-byte {issue cycle, pc} records.
// CACHE: the cache-latency model (per-warp direct-mapped L1 and L2 in a.cache).
template <int RFN, bool EXT, bool CACHE>
__device__ __forceinline__ void interp(const KsArgs& a) {
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ uint32_t ep_max[3], ep_alive[3];

  const uint32_t WG = blockDim.x;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = uni(tid >> 6);  // wave-uniform: keeps every per-warp value scalar
  const uint32_t hl = lane >> 5;
  const uint32_t sl = lane & 31u;
  const uint32_t blk = blockIdx.x + (EXT ? a.block_base : 0u);  // extended-record grids run in parts
  const uint32_t W = a.warps_per_block;
  const uint32_t T = a.threads_per_block;
  const uint32_t n_instr = a.n_instrs;
  const cdinst prog = (cdinst)(uintptr_t)a.prog;
  const __attribute__((address_space(4))) uint8_t* const prog_b = (const __attribute__((address_space(4))) uint8_t*)prog;
  const uint32_t ib = a.rf_slots - KS_IMM_SLOTS - KS_CONST_SLOTS;  // first immediate slot

  // LDS: [scoreboard, 129 words per warp] [scratch scoreboard, 129 words] (to 16 bytes)
  //      [EXT: record ring, 32 x 16 bytes per warp] [shared window]
  RegFile<RFN, EXT ? 64 : 56> R;
  RegFile<RFN, EXT ? 64 : 56>::zero();
  // the constant slots after the immediates: 1.0f and -0.0f
  R.put(ib + KS_IMM_SLOTS, 0x3F800000u);
  R.put(ib + KS_IMM_SLOTS + 1u, 0x80000000u);
  uint32_t* const sbw = lds;
  // words per warp: the scoreboard, and with basic records the staging ring after it
  constexpr uint32_t SBS = EXT ? KS_SB_ENTRIES : KS_SB_STRIDE;
  uint8_t* const dump_sb = reinterpret_cast<uint8_t*>(sbw + (WG / 32u) * SBS);
  const uint32_t sb_words = (WG / 32u + 1u) * SBS;
  uint8_t* const ring = reinterpret_cast<uint8_t*>(lds) + ((4u * sb_words + 15u) & ~15u);
  uint8_t* const win = ring + (EXT ? 16u * WG : 0u);
  {
    for (uint32_t i = tid; i < sb_words; i += WG) lds[i] = 0;
    uint32_t* const win_w = reinterpret_cast<uint32_t*>(win);
    for (uint32_t i = tid, n = (a.shared_bytes + 3u) >> 2; i < n; i += WG) win_w[i] = 0;
    if (tid < 3) {
      ep_max[tid] = 0;
      ep_alive[tid] = 0;
    }
  }
  __syncthreads();

  const uint32_t my_w = 2u * wave + hl;
  // sector ids + 1 of valid accesses fit 32 bits (and stay non-zero)
  const uint32_t small_gmem = a.gmem_bytes <= (1ull << 37) - 64u ? 1u : 0u;
  const uint64_t glim4 = a.gmem_bytes >= 4 ? a.gmem_bytes - 3u : 0u;   // a 4-byte access at A is inside iff A < glim4
  uint8_t* const my_sb = reinterpret_cast<uint8_t*>(sbw + my_w * SBS);  // this lane's warp's scoreboard
  auto sb_at = [&](uint32_t off) -> uint32_t& { return *reinterpret_cast<uint32_t*>(my_sb + off); };

  // per-warp scalar state (warp 2w = half 0, warp 2w+1 = half 1)
  const uint32_t w0 = 2u * wave, w1 = w0 + 1u;
  auto live_mask = [&](uint32_t w) -> uint32_t {
    if (w >= W) return 0u;
    const uint32_t live = T - w * 32u;
    return live >= 32u ? 0xFFFFFFFFu : ((1u << live) - 1u);
  };
  const uint64_t init64 = (uint64_t)live_mask(w0) | ((uint64_t)live_mask(w1) << 32);
  uint64_t mask64 = init64;   // masks of the two top entries
  uint64_t ex64 = 0;          // exited lanes
  uint64_t m64 = init64;      // mask64 & ~ex64
  Stk S0, S1;
  S0.pc = 0; S0.rpc = INF; S0.sp = w0 < W ? 1u : 0u; S0.md = 1; S0.pr = 0; S0.m = 0;
  S1.pc = 0; S1.rpc = INF; S1.sp = w1 < W ? 1u : 0u; S1.md = 1; S1.pr = 0; S1.m = 0;
  uint32_t spc0 = w0 < W ? 0u : INF, spc1 = w1 < W ? 0u : INF;  // scheduled pc: top pc while running, else INF
  uint32_t hst = (w0 < W ? 0u : DONE0) | (w1 < W ? 0u : DONE1);
  uint32_t status = 0;        // KS_ST_* of warp 2w in bits 0-7, of warp 2w+1 in bits 8-15

  // per-lane state (uniform over each warp's lanes where noted)
  const uint32_t cap = a.trace_cap;
  const uint32_t budget = a.max_warp_instrs;
  uint32_t v_next = 0;        // warp: previous issue cycle + 1
  uint32_t wi = 0;            // warp: issued warp-instructions
  uint32_t fl = 0;            // warp: trace records written to memory
  // warp: record count at which the next chunk is written (from the records written so far)
  auto next_flush = [&](uint32_t written) -> uint32_t { return written < cap ? umin(cap, written + 32u) : INF; };
  uint32_t ev = umin(next_flush(0), budget);      // warp: next event (chunk write or budget)
  uint32_t act = 0;           // instructions issued with this lane's thread active (see KS_SET_LIVE)
  uint32_t cnt = 0;           // counter d of the lane's warp in lane 32 h + d
  uint32_t pbits = 0;         // predicate p of this lane's thread in bit p
  // basic records: record k of a warp is staged in slot k % 32 of the ring after its
  // scoreboard; lane l of the warp writes slot l to memory (chunks start at multiples of 32)
  auto staged = [&]() -> uint2 {
    return *reinterpret_cast<const uint2*>(my_sb + 4u * KS_SB_RING + 8u * sl);
  };
  // EXT: record k of this lane's warp is staged in slot k % 32 of the warp's LDS ring
  uint8_t* const my_ring = ring + 512u * my_w;
  // global loads / stores: per-lane shares of the access, sector and line counters of
  // the fast analyser path (summed over each warp's lanes at the end)
  uint32_t q_ln = 0, q_ls = 0, q_ll = 0, q_sn = 0, q_ss = 0, q_sl = 0;
  const uint64_t gw0 = (uint64_t)blk * W + 2u * wave;  // global warp id of half 0
  uint8_t* const slot_base = a.trace + (gw0 + hl) * a.slot_bytes + 16u;  // this lane's warp's records

  // Every instruction a warp issues between two changes of its live mask runs with
  // the same mask, so thread-instructions are counted per lane only when the live
  // masks change: a lane that becomes live subtracts its warp's issue count, one
  // that stops being live adds it (and so does every live lane at the end).
#define KS_SET_LIVE(newm)                         \
  {                                               \
    const uint64_t nm_ = (newm);                  \
    act += lanes(m64 & ~nm_) ? wi : 0u;           \
    act -= lanes(nm_ & ~m64) ? wi : 0u;           \
    m64 = nm_;                                    \
  }

  // Pop entries of warp h that cannot issue (no live lane, reconverged); lanes past
  // the end exit at no cost; an empty stack finishes the warp.  Leaves spc_h.
#define KS_SETTLE(h, S, spc)                                                   \
  {                                                                            \
    while (true) {                                                             \
      if (S.sp == 0) {                                                         \
        spc = INF;                                                             \
        hst |= DONE0 << (h);                                                   \
        status |= KS_ST_FINISHED << (8 * (h));                                 \
        break;                                                                 \
      }                                                                        \
      const uint32_t mk = (uint32_t)(mask64 >> (32 * (h)));                    \
      const uint32_t lv = mk & ~(uint32_t)(ex64 >> (32 * (h)));                \
      if (lv == 0 || S.pc == S.rpc) {                                          \
        const uint32_t nm = stk_pop(S);                                        \
        mask64 = (mask64 & ~((uint64_t)0xFFFFFFFFu << (32 * (h)))) | ((uint64_t)nm << (32 * (h))); \
        continue;                                                              \
      }                                                                        \
      if (S.pc >= n_instr) {                                                   \
        ex64 |= (uint64_t)lv << (32 * (h));                                    \
        continue;                                                              \
      }                                                                        \
      spc = S.pc;                                                              \
      break;                                                                   \
    }                                                                          \
    KS_SET_LIVE(mask64 & ~ex64);                                               \
  }

  // Faulting lanes (invalid address or alignment): status FAULT and the fault counter.
#define KS_COUNT_FAULTS(faults)                                                      \
  if (faults) {                                                                     \
    const uint32_t f0 = popc((uint32_t)(faults)), f1 = popc((uint32_t)((faults) >> 32)); \
    if (f0) status |= KS_ST_FAULT;                                                   \
    if (f1) status |= KS_ST_FAULT << 8;                                              \
    cnt += sl == C_FAULT ? (hl ? f1 : f0) : 0u;                                      \
  }

  // Distinct 32-byte sectors and 128-byte lines of a global warp access of S bytes
  // per lane at A over the guard lanes on64, added to the access / sector / line
  // counters of the load or store.  Where a warp's sector ids do not decrease over
  // its guard lanes in lane order, a lane opens a new sector exactly when its id
  // exceeds the largest id of the guard lanes before it (and a new line likewise),
  // so each lane adds its own 0/1 flags to per-lane counters that are summed per
  // warp at the end; other warps (and any access with a faulting lane) count the
  // distinct values exactly.  Full exec.
#define KS_GLOBAL_ACCOUNT(A, S, faults, is_load)                                     \
  {                                                                                 \
    uint64_t exact = on64;                                                          \
    if (!(faults) && small_gmem) {                                                  \
      const bool on_ = lanes(on64);                                                 \
      /* sector id + 1 on guard lanes, 0 elsewhere; prev: the largest over the earlier lanes of the half */ \
      const uint32_t sid1 = on_ ? (uint32_t)((A) >> 5) + 1u : 0u;                   \
      /* with every lane on, the previous lane's id is that largest id wherever */  \
      /* the ids do not decrease, and the other halves are found by the same test */ \
      uint32_t pm_ = sid1;                                                          \
      if (on64 != ~0ull) {                                                          \
        pm_ = half_prefix_max(sid1);                                                \
        asm volatile("" : "+v"(pm_)); /* a branch, not a select of both arms */     \
      }                                                                             \
      const uint32_t prev = prev_in_half(pm_, lane);                                \
      uint64_t fast = on64;                                                         \
      const uint64_t nonmono = ballot(sid1 < prev) & on64;                          \
      if (nonmono) {                                                                \
        if ((uint32_t)nonmono) fast &= HI;                                          \
        if (nonmono >> 32) fast &= LO;                                              \
      }                                                                             \
      exact = on64 & ~fast;                                                         \
      const bool f_ = lanes(fast);                                                  \
      const uint32_t fn_ = (f_ && prev == 0u) ? 1u : 0u;                            \
      const uint32_t fs_ = (f_ && sid1 != prev) ? 1u : 0u;                          \
      const uint32_t fl_ = (f_ && (prev == 0u || ((sid1 - 1u) >> 2) != ((prev - 1u) >> 2))) ? 1u : 0u; \
      if constexpr (EXT) {                                                          \
        /* the per-warp counts of this access go into the record and the counters */ \
        const uint64_t bs_ = ballot(fs_ != 0u), bl_ = ballot(fl_ != 0u);            \
        const uint32_t s0_ = popc((uint32_t)bs_), s1_ = popc((uint32_t)(bs_ >> 32)); \
        const uint32_t l0_ = popc((uint32_t)bl_), l1_ = popc((uint32_t)(bl_ >> 32)); \
        x_sl0 = s0_ | (l0_ << 8);                                                   \
        x_sl1 = s1_ | (l1_ << 8);                                                   \
        /* counters n, sectors, lines of the lane's warp when its half took this path */ \
        const uint32_t d_ = sl - ((is_load) ? C_GLD_N : C_GST_N);                   \
        const bool fh_ = hl ? (fast >> 32) != 0 : (uint32_t)fast != 0;              \
        if (fh_ && d_ < 3u) cnt += d_ == 0 ? 1u : (d_ == 1 ? (hl ? s1_ : s0_) : (hl ? l1_ : l0_)); \
      } else if (is_load) {                                                         \
        q_ln += fn_;                                                                \
        q_ls += fs_;                                                                \
        q_ll += fl_;                                                                \
      } else {                                                                      \
        q_sn += fn_;                                                                \
        q_ss += fs_;                                                                \
        q_sl += fl_;                                                                \
      }                                                                             \
    }                                                                               \
    if (exact) {                                                                    \
      const uint32_t e0 = (uint32_t)exact, e1 = (uint32_t)(exact >> 32);            \
      const uint64_t last = (A) + ((S) - 1u);                                       \
      uint32_t sec0 = 0, lin0 = 0, sec1 = 0, lin1 = 0;                              \
      if (e0) {                                                                     \
        sec0 = distinct2((A) >> 5, last >> 5, (uint64_t)e0);                        \
        lin0 = distinct2((A) >> 7, last >> 7, (uint64_t)e0);                        \
      }                                                                             \
      if (e1) {                                                                     \
        sec1 = distinct2((A) >> 5, last >> 5, (uint64_t)e1 << 32);                  \
        lin1 = distinct2((A) >> 7, last >> 7, (uint64_t)e1 << 32);                  \
      }                                                                             \
      /* counters n, sectors, lines of the lane's warp: lanes 32 h + {cn, cn+1, cn+2} */ \
      const uint32_t cn = (is_load) ? C_GLD_N : C_GST_N;                            \
      const uint32_t d = sl - cn;                                                   \
      const uint32_t eh = hl ? e1 : e0;                                             \
      if (eh && d < 3u) cnt += d == 0 ? 1u : (d == 1 ? (hl ? sec1 : sec0) : (hl ? lin1 : lin0)); \
      if constexpr (EXT) {                                                          \
        if (e0) x_sl0 = sec0 | (lin0 << 8);                                         \
        if (e1) x_sl1 = sec1 | (lin1 << 8);                                         \
      }                                                                             \
    }                                                                               \
  }

  // Issue of one instruction by the warps of gm, written as per-lane selects so
  // that exec stays full: the trace record (issue cycle, pc) goes into slot wi % 32
  // of each issuing warp's staging ring; the issue count and the next issue cycle
  // advance; the destination's scoreboard entry gets its ready cycle (the other
  // warp's lanes write a scratch scoreboard and ring instead).
#define KS_ISSUE(is_, p_, sbod_, lat_)                                               \
  {                                                                                 \
    if constexpr (!EXT) {                                                           \
      uint32_t* const tq_ = reinterpret_cast<uint32_t*>(sb_sel + 4u * KS_SB_RING + ((wi & 31u) << 3)); \
      tq_[0] = (is_);                                                               \
      tq_[1] = (p_);                                                                \
    }                                                                               \
    wi += ginc;                                                                     \
    v_next = gl ? (is_) + 1u : v_next;                                              \
    *reinterpret_cast<uint32_t*>(sb_sel + (sbod_)) = (is_) + (lat_);                 \
  }

  // Extended trace record of the instruction just issued by the warps of gm (after
  // KS_ISSUE: it is the warp's record wi - 1), written by the first lane of each
  // issuing half: issue cycle, pc | kind << 16, the warp's live lanes, payload.
  // Four 32-bit LDS stores, not one 16-byte store: a 16-byte LDS store whose data
  // registers the next instructions overwrite (the compiler inserts no wait there)
  // now and then stored a word of the new value once three or more waves shared a
  // SIMD; 32-bit stores read their data at issue.
#define KS_EXT_REC(is_, pc_, kind_, pay_)                                            \
  if constexpr (EXT) {                                                              \
    const uint32_t k_ = wi - 1u;                                                    \
    if (gl && sl == 0u && k_ < cap) {                                               \
      volatile uint32_t* const rp_ = reinterpret_cast<volatile uint32_t*>(my_ring + 16u * (k_ & 31u)); \
      rp_[0] = (is_);                                                               \
      rp_[1] = (pc_) | ((uint32_t)(kind_) << 16);                                   \
      rp_[2] = hl ? (uint32_t)(mm >> 32) : (uint32_t)mm;                            \
      rp_[3] = (pay_);                                                              \
    }                                                                               \
  }

  // A global store whose next index-mode register access may come within a few
  // instructions (the extended variants' general memory path) waits until the store
  // has completed, so that it no longer reads its address or data registers then.
#define KS_EXT_STORE_WAIT()                                                          \
  if constexpr (EXT) asm volatile("s_waitcnt vmcnt(0)" ::: "memory")

  // Cache-latency model (KernelScope memory analysis: direct-mapped L1 and L2 of
  // 128-byte lines): the line of the lowest valid guard lane of each warp (okm)
  // is looked up in that warp's L1, on a miss in its L2, installing it where it
  // missed; lane 0 of each half does its warp's lookup.  The outcome (0 L1 hit,
  // 1 L2 hit, 2 miss) is counted in lanes 32 h + 20 + outcome of cnt, and a load's
  // destination becomes ready after that level's latency (a warp with no valid
  // lane keeps the ld.global latency its issue wrote).  Valid addresses are below
  // 2^38 bytes, so line numbers fit 32 bits.
#define KS_CACHE_ISSUE(A, okm)                                                        \
  [[maybe_unused]] uint32_t cline_ = 0, co1_ = 0, co2_ = 0, cvalid_ = 0;            \
  if constexpr (CACHE) {                                                            \
    const uint32_t v0_ = (uint32_t)(okm), v1_ = (uint32_t)((okm) >> 32);            \
    const uint32_t lnl_ = (uint32_t)((A) >> 7);                                     \
    const uint32_t line0_ = rl(lnl_, v0_ ? (uint32_t)__builtin_ctz(v0_) : 0u);       \
    const uint32_t line1_ = rl(lnl_, v1_ ? 32u + (uint32_t)__builtin_ctz(v1_) : 32u); \
    cline_ = hl ? line1_ : line0_;                                                  \
    cvalid_ = (sl == 0u && (hl ? v1_ : v0_) != 0u) ? 1u : 0u;                        \
    if (cvalid_) {                                                                  \
      const uint32_t* const cw_ =                                                   \
          reinterpret_cast<const uint32_t*>(a.cache + (gw0 + hl) * (uint64_t)KS_CACHE_WARP_BYTES); \
      /* both tags in one memory round trip (the two arrays never overlap) */        \
      co1_ = cw_[4u + (cline_ & (KS_CACHE_L1_LINES - 1u))];                         \
      co2_ = cw_[4u + KS_CACHE_L1_LINES + cline_ % KS_CACHE_L2_LINES];              \
    }                                                                               \
  }

  // The lookup itself, once the tags of KS_CACHE_ISSUE are needed: a hit in L1, else
  // install there and look in L2, else install there too.
#define KS_CACHE_FINISH(is_load, sbod_)                                               \
  if constexpr (CACHE) {                                                            \
    uint32_t lvl_ = 3u;                                                             \
    if (cvalid_) {                                                                  \
      uint32_t* const cw_ = reinterpret_cast<uint32_t*>(a.cache + (gw0 + hl) * (uint64_t)KS_CACHE_WARP_BYTES); \
      const uint32_t t_ = cline_ + 1u;                                              \
      if (co1_ == t_) {                                                             \
        lvl_ = 0u;                                                                  \
      } else {                                                                      \
        cw_[4u + (cline_ & (KS_CACHE_L1_LINES - 1u))] = t_;                         \
        if (co2_ == t_) {                                                           \
          lvl_ = 1u;                                                                \
        } else {                                                                    \
          cw_[4u + KS_CACHE_L1_LINES + cline_ % KS_CACHE_L2_LINES] = t_;            \
          lvl_ = 2u;                                                                \
        }                                                                           \
      }                                                                             \
    }                                                                               \
    /* index mode follows soon: the tag stores must be done with their registers */ \
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                                \
    const uint32_t my_lv_ = hl ? rl(lvl_, 32) : rl(lvl_, 0);                         \
    cnt += (my_lv_ < 3u && sl == 20u + my_lv_) ? 1u : 0u;                            \
    /* the three latencies as values (a select of their fields would address the */ \
    /* kernel arguments dynamically and copy them to scratch) */                    \
    const uint32_t c1_ = uni(a.lat_l1), c2_ = uni(a.lat_l2), c3_ = uni(a.lat_dram);  \
    if ((is_load) && my_lv_ < 3u)                                                   \
      *reinterpret_cast<uint32_t*>(sb_sel + (sbod_)) = is + (my_lv_ == 0u ? c1_ : (my_lv_ == 1u ? c2_ : c3_)); \
  }

  // Issue cycle of the instruction whose hot words are h: the later of the warp's
  // previous issue + 1 and the ready cycle of every register source (absent
  // sources read a zero entry).
#define KS_ISSUE_CYCLE(h)                                                            \
  umax(umax(v_next, sb_at((h)[6])), umax(umax(sb_at((h)[7]), sb_at((h)[8])), sb_at((h)[9])))

  uint32_t epoch = 0;
  // kept in a register (the compiler would reload the kernel argument on every pass)
  uint32_t cyc_safe = a.cyc_safe;
  asm volatile("" : "+v"(cyc_safe));
  while (true) {
    // ------------------------------------------------------------------ run both warps until blocked
    while (true) {
      const uint32_t pc = umin(spc0, spc1);
      if (pc == INF) break;
      // issuing warps, as all-ones / zero words (integers, not bools: a bool that lives
      // across blocks becomes a lane mask, and turning it back into a value costs VALU work)
      const uint32_t go0 = s_eq_mask(spc0, pc), go1 = s_eq_mask(spc1, pc);
      const uint64_t gm = ((uint64_t)go1 << 32) | go0;  // lanes of the issuing warps
      const u32x16 hot = *reinterpret_cast<const __attribute__((address_space(4))) u32x16*>(prog + pc);
      const uint32_t ctl = hot[0];  // class bit | flags | run length
      const uint32_t iss = KS_ISSUE_CYCLE(hot);

      uint32_t need = 0;  // warps whose top stack entry must be settled (bit h)
      if (ctl & XF_FIX) {  // the end sentinel, or a reconvergence point: warps whose top entry ends here pop
        if (ctl & CB(DC_END)) {
          need = (go0 & 1u) | (go1 & 2u);
          ex64 |= m64 & gm;  // lanes that get past the last instruction exit, at no cost
        } else {
          need = (s_eq_mask(uni(S0.rpc), pc) & go0 & 1u) | (s_eq_mask(uni(S1.rpc), pc) & go1 & 2u);
        }
        if (need & 1u) S0.pc = pc;
        if (need & 2u) S1.pc = pc;
      }
      const uint64_t evm = (ballot(wi == ev) | ballot(iss > CYCLE_LIMIT)) & gm;
      // per-step selects of the issuing lanes
      const bool gl = lanes(gm);
      const uint32_t ginc = gl ? 1u : 0u;   // issue count step
      uint8_t* const sb_sel = gl ? my_sb : dump_sb;
      const uint64_t mm = m64 & gm;        // live lanes of the issuing warps
      if (need) {
        // no issue this step
      } else if (evm) {
        // events: trace chunk complete, issue budget reached (checked first), cycle limit passed
        const uint64_t bm = ballot(wi == budget) & gm;
        const uint64_t om = ballot(iss > CYCLE_LIMIT) & gm & ~bm;
        const uint64_t fm = ballot(wi == next_flush(fl)) & gm & ~om;  // a full chunk (or the cap) to write
        if (lanes(fm)) {
          if constexpr (EXT) {
            if (sl < wi - fl)
              *reinterpret_cast<uint4*>(slot_base + 16ull * (fl + sl)) = *reinterpret_cast<const uint4*>(my_ring + 16u * sl);
            KS_EXT_STORE_WAIT();  // the next step's index mode follows soon
          } else {
            if (sl < wi - fl) *reinterpret_cast<uint2*>(slot_base + 8ull * (fl + sl)) = staged();
          }
          fl = wi;
        }
        if (gl) ev = umin(next_flush(fl), budget);
        const uint64_t stop = bm | om;
        if (stop & LO) {
          spc0 = INF;
          hst |= DONE0;
          status |= (bm & LO) ? KS_ST_BUDGET : KS_ST_CYCLE_OVF;
        }
        if (stop & HI) {
          spc1 = INF;
          hst |= DONE1;
          status |= ((bm & HI) ? KS_ST_BUDGET : KS_ST_CYCLE_OVF) << 8;
        }
      } else if (ctl & CB_CTRL) {
        // ---------------------------------------------------------------- control instructions
        const uint64_t on64 = mm & ballot(((pbits >> hot[12]) & 1u) != hot[13]);  // guard
        KS_ISSUE(iss, pc, hot[10], hot[11]);
        const uint32_t g0 = (uint32_t)on64, g1 = (uint32_t)(on64 >> 32);
        if (ctl & CB(DC_BRA)) {
          const uint32_t target = hot[14], rpc = hot[15];
          const uint32_t mm0 = (uint32_t)mm, mm1 = (uint32_t)(mm >> 32);
          uint32_t divm = 0;
          if (go0) {
            const uint32_t nt = mm0 & ~g0;
            if (nt == 0) {
              spc0 = target;
            } else if (g0 == 0) {
              spc0 = pc + 1u;
            } else {
              divm |= 1u;
              const uint32_t mk = (uint32_t)mask64;
              S0.pc = rpc;
              if (target != rpc) stk_push(S0, mk, target, rpc, lane);
              uint32_t top = target != rpc ? g0 : mk;
              if (pc + 1u != rpc) {
                stk_push(S0, top, pc + 1u, rpc, lane);
                top = nt;
              }
              mask64 = (mask64 & HI) | top;
              spc0 = S0.pc;
            }
          }
          if (go1) {
            const uint32_t nt = mm1 & ~g1;
            if (nt == 0) {
              spc1 = target;
            } else if (g1 == 0) {
              spc1 = pc + 1u;
            } else {
              divm |= 2u;
              const uint32_t mk = (uint32_t)(mask64 >> 32);
              S1.pc = rpc;
              if (target != rpc) stk_push(S1, mk, target, rpc, lane);
              uint32_t top = target != rpc ? g1 : mk;
              if (pc + 1u != rpc) {
                stk_push(S1, top, pc + 1u, rpc, lane);
                top = nt;
              }
              mask64 = (mask64 & LO) | ((uint64_t)top << 32);
              spc1 = S1.pc;
            }
          }
          if (divm) {
            KS_SET_LIVE(mask64 & ~ex64);
            cnt = cnt_add2(cnt, sl, hl, C_DIV, divm, 1u);
          }
          KS_EXT_REC(iss, pc, ((divm >> hl) & 1u) ? KS_EV_DIVERGE : KS_EV_BRANCH, (hl ? (uint32_t)(on64 >> 32) : (uint32_t)on64));
        } else if (ctl & CB(DC_RET)) {
          KS_EXT_REC(iss, pc, KS_EV_RET, (hl ? (uint32_t)(on64 >> 32) : (uint32_t)on64));
          ex64 |= on64;
          KS_SET_LIVE(mask64 & ~ex64);
          if (go0) {
            spc0 = pc + 1u;
            S0.pc = pc + 1u;
            need |= s_zero_mask((uint32_t)m64) & 1u;  // every lane has exited: pop
          }
          if (go1) {
            spc1 = pc + 1u;
            S1.pc = pc + 1u;
            need |= s_zero_mask((uint32_t)(m64 >> 32)) & 2u;
          }
        } else {  // DC_BAR: the issuing warps wait for the block
          KS_EXT_REC(iss, pc, KS_EV_BARRIER, 0u);
          const uint64_t conv = init64 & ~ex64;
          const uint32_t hm = (go0 & 1u) | (go1 & 2u);
          cnt = cnt_add2(cnt, sl, hl, C_BAR, hm, 1u);
          if (go0 && (uint32_t)mm != (uint32_t)conv) status |= KS_ST_BARDIV;
          if (go1 && (uint32_t)(mm >> 32) != (uint32_t)(conv >> 32)) status |= KS_ST_BARDIV << 8;
          if ((go0 | (0u - ((hst >> 2) & 1u))) & (go1 | (0u - ((hst >> 3) & 1u)))) {
            // Every unfinished warp of the wave arrives here together: the wave takes
            // part in the block's epoch right away (the protocol of the epoch below,
            // arrival = this issue cycle) and its warps go on after the barrier.
            const uint32_t slot = epoch % 3u;
            if (lane == 0) {
              atomicAdd(&ep_alive[slot], hm == 3u ? 2u : 1u);
              atomicMax(&ep_max[slot], umax(go0 ? rl(iss, 0) : 0u, go1 ? rl(iss, 32) : 0u));
            }
            if (tid == 0) {
              ep_alive[(epoch + 1u) % 3u] = 0;
              ep_max[(epoch + 1u) % 3u] = 0;
            }
            // the issue count and next issue cycle from before the release
            *reinterpret_cast<uint32_t*>(sb_sel + 4u * KS_SB_BAR_WI) = wi;
            *reinterpret_cast<uint32_t*>(sb_sel + 4u * KS_SB_BAR_NEXT) = v_next;
            __syncthreads();
            const uint32_t release = uni(ep_max[slot]) + a.lat_bar;
            v_next = gl ? umax(v_next, release) : v_next;
            ++epoch;
            if (go0) spc0 = pc + 1u;
            if (go1) spc1 = pc + 1u;
          } else {
            if (go0) {
              S0.pc = pc + 1u;
              spc0 = INF;
              hst |= WAIT0;
            }
            if (go1) {
              S1.pc = pc + 1u;
              spc1 = INF;
              hst |= WAIT1;
            }
          }
        }
      } else {
        // ---------------------------------------------------------------- a straight run
        // This instruction and the ones after it up to the next control instruction or
        // reconvergence point (the host's run length) issue back to back by the same
        // warps, without rescheduling: none of them may reach an event (chunk write,
        // budget) and none may pass the cycle limit.
        uint32_t n = ctl >> RUN_SHIFT;  // at least 1
        {
          const uint32_t room = ev - wi;  // per warp: issues before its next event (at least 1 here)
          n = umin(n, umin(rl(room, 0) | ~go0, rl(room, 32) | ~go1));
          if (ballot(iss > cyc_safe) & gm) n = 1u;
        }
        uint32_t off = pc * (uint32_t)sizeof(DInst);  // byte offset of the current record
        uint32_t is = iss;
        u32x16 h = hot;
        while (true) {
          const uint32_t c = h[0];
          // touch the record two ahead, so that its line is in the scalar cache by then
          // (the value is consumed only after the next record arrives)
          const uint32_t pf = *reinterpret_cast<const __attribute__((address_space(4))) uint32_t*>(
              prog_b + off + 2u * (uint32_t)sizeof(DInst));
          // the next record's scoreboard offsets, carried by this one
          const u32x4 nsbo = *reinterpret_cast<const __attribute__((address_space(4))) u32x4*>(
              prog_b + off + offsetof(DInst, nsbo));
          KS_ISSUE(is, off / (uint32_t)sizeof(DInst), h[10], h[11]);
          const uint64_t on64 = mm & ballot(((pbits >> h[12]) & 1u) != h[13]);  // guard
          // extended record of a non-memory instruction: the lanes passing the guard
          // (memory instructions write theirs after the access is analysed)
          if constexpr (EXT)
            if (!(c & (CB(DC_LDG) | CB(DC_STG) | CB_MEM)))
              KS_EXT_REC(is, off / (uint32_t)sizeof(DInst), KS_EV_OTHER, (hl ? (uint32_t)(on64 >> 32) : (uint32_t)on64));
          if (c & XF_IMM) {
            uint32_t iv[6];
            for (int k = 0; k < 6; ++k) iv[k] = *reinterpret_cast<const __attribute__((address_space(4))) uint32_t*>(
                prog_b + off + offsetof(DInst, imm) + 4u * k);
            R.put_imm(ib, iv);
          }
          const uint32_t s0 = h[2], s1 = h[3], s2 = h[4], dst = h[5];
          const uint32_t a0 = h[14], a1 = h[15], a2 = h[1];
          if (c & CB(DC_FMA)) {
            uint32_t x0, x1, x2;
            R.get3(s0, s1, s2, x0, x1, x2);
            R.put_m(dst, canon_bits(__builtin_fmaf(__uint_as_float(x0), __uint_as_float(x1), __uint_as_float(x2 ^ a2))),
                    on64);
          } else if (c & CB(DC_IADD)) {
            uint32_t x0, x1;
            R.get2(s0, s1, x0, x1);
            R.put_m(dst, x0 + (x1 ^ a0) + a1, on64);
          } else if (c & CB(DC_IMAD)) {
            uint32_t x0, x1, x2;
            R.get3(s0, s1, s2, x0, x1, x2);
            R.put_m(dst, x0 * x1 + (x2 & a0), on64);
          } else if (c & (CB(DC_LDG) | CB(DC_STG))) {
            // 32-bit global load or store through a 64-bit address register
            uint32_t blo, bhi;
            R.get2(s0, s0 + 1u, blo, bhi);
            const uint64_t A = (((uint64_t)bhi << 32) | blo) + (((uint64_t)a1 << 32) | a0);
            const uint64_t okm = ballot(((uint32_t)A & 3u) == 0u) & ballot(A < glim4) & on64;
            const uint64_t faults = on64 & ~okm;
            [[maybe_unused]] uint32_t x_sl0 = 0, x_sl1 = 0;  // sectors | lines << 8 of each warp (extended records)
            if (c & CB(DC_LDG)) {
              if (faults) R.put_m(dst, 0u, faults);  // lanes without a valid access read 0
              // the loaded value; lanes outside okm are never written to the register,
              // so the register starts with whatever it holds (no write that the load
              // would have to wait for)
              uint32_t ld_v;
              asm volatile("" : "=v"(ld_v));
              if (lanes(okm)) ld_v = *reinterpret_cast<const uint32_t*>(a.gmem + A);
              // The accounting needs only the addresses: it runs while the load (and
              // the cache model's tag loads) are in flight.  Nothing in it uses VGPR
              // index mode, which must stay off while a load that returns into a VGPR
              // is outstanding (a loaded value then lands in the wrong register).
              KS_CACHE_ISSUE(A, okm);
              KS_COUNT_FAULTS(faults);
              KS_GLOBAL_ACCOUNT(A, 4u, faults, true);
              KS_CACHE_FINISH(true, h[10]);
              R.put_m(dst, ld_v, okm);
            } else {
              if (lanes(okm)) *reinterpret_cast<uint32_t*>(a.gmem + A) = R.get(s1);
              KS_CACHE_ISSUE(A, okm);
              KS_COUNT_FAULTS(faults);
              KS_GLOBAL_ACCOUNT(A, 4u, faults, false);
              KS_CACHE_FINISH(false, h[10]);
            }
            if constexpr (EXT) {
              const uint32_t p0 = x_sl0 | (popc((uint32_t)on64) << 16) | (popc((uint32_t)faults) << 24);
              const uint32_t p1 = x_sl1 | (popc((uint32_t)(on64 >> 32)) << 16) | (popc((uint32_t)(faults >> 32)) << 24);
              KS_EXT_REC(is, off / (uint32_t)sizeof(DInst), (c & CB(DC_LDG)) ? KS_EV_LD_GLOBAL : KS_EV_ST_GLOBAL,
                         hl ? p1 : p0);
            }
          } else if (c & CB(DC_MOV)) {
            if (a0) {
              uint32_t lo, hi;
              R.get2(s0, s0 + 1u, lo, hi);
              R.put2_m(dst, lo, hi, on64);
            } else {
              R.put_m(dst, R.get(s0), on64);
            }
          } else if (c & CB(DC_SELP)) {
            const bool pr = (pbits >> s2) & 1u;
            if (a0) {
              uint32_t xl, xh, yl, yh;
              R.get2(s0, s0 + 1u, xl, xh);
              R.get2(s1, s1 + 1u, yl, yh);
              R.put2_m(dst, pr ? xl : yl, pr ? xh : yh, on64);
            } else {
              uint32_t x0, x1;
              R.get2(s0, s1, x0, x1);
              R.put_m(dst, pr ? x0 : x1, on64);
            }
          } else if (c & CB(DC_SETP)) {
            bool lt, eq, gt;
            if (a0 == DS_F32) {
              uint32_t x0, x1;
              R.get2(s0, s1, x0, x1);
              const float x = __uint_as_float(x0), y = __uint_as_float(x1);
              lt = x < y;
              eq = x == y;
              gt = x > y;  // all false when an input is NaN
            } else if (a0 <= DS_U32) {
              uint32_t x0, x1;
              R.get2(s0, s1, x0, x1);
              lt = a0 == DS_S32 ? (int32_t)x0 < (int32_t)x1 : x0 < x1;
              eq = x0 == x1;
              gt = !lt && !eq;
            } else {
              uint32_t xl, xh, yl, yh;
              R.get2(s0, s0 + 1u, xl, xh);
              R.get2(s1, s1 + 1u, yl, yh);
              const uint64_t x = (uint64_t)xl | ((uint64_t)xh << 32), y = (uint64_t)yl | ((uint64_t)yh << 32);
              lt = a0 == DS_S64 ? (int64_t)x < (int64_t)y : x < y;
              eq = x == y;
              gt = !lt && !eq;
            }
            const bool cv = (lt && (a1 & 1u)) || (eq && (a1 & 2u)) || (gt && (a1 & 4u));
            const uint32_t nb = (pbits & ~(1u << dst)) | ((cv ? 1u : 0u) << dst);
            pbits = lanes(on64) ? nb : pbits;
          } else if (c & CB(DC_I64)) {
            uint64_t r;
            if (a0 >= DI_WIDE_S) {
              uint32_t x0, x1;
              R.get2(s0, s1, x0, x1);
              r = a0 == DI_WIDE_S ? (uint64_t)((int64_t)(int32_t)x0 * (int64_t)(int32_t)x1)
                                  : (uint64_t)x0 * (uint64_t)x1;
            } else {
              uint32_t xl, xh, yl, yh;
              R.get2(s0, s0 + 1u, xl, xh);
              R.get2(s1, s1 + 1u, yl, yh);
              const uint64_t x = (uint64_t)xl | ((uint64_t)xh << 32), y = (uint64_t)yl | ((uint64_t)yh << 32);
              if (a0 == DI_ADD) r = x + y;
              else if (a0 == DI_SUB) r = x - y;
              else if (a0 == DI_MUL) r = x * y;
              else {
                uint32_t zl, zh;
                R.get2(s2, s2 + 1u, zl, zh);
                r = x * y + ((uint64_t)zl | ((uint64_t)zh << 32));
              }
            }
            R.put2_m(dst, (uint32_t)r, (uint32_t)(r >> 32), on64);
          } else if (c & CB_MEM) {
            const uint32_t is_global = c & CB(DC_MEMG);
            const uint32_t is_load = c & XF_LOAD;
            const uint32_t w64 = c & XF_W64;
            const uint32_t S = w64 ? 8u : 4u;
            const uint64_t size = is_global ? a.gmem_bytes : (uint64_t)a.shared_bytes;
            const uint64_t aoff = (uint64_t)a0 | ((uint64_t)a1 << 32);  // byte offset of the address
            uint64_t base;
            if (c & XF_A64) {
              uint32_t lo, hi;
              R.get2(s0, s0 + 1u, lo, hi);
              base = (uint64_t)lo | ((uint64_t)hi << 32);
            } else {
              base = R.get(s0);
            }
            const uint64_t A = base + aoff;
            const uint64_t okm = ballot((A & (S - 1u)) == 0 && A <= size && size - A >= S) & on64;
            if (is_load) {
              uint32_t lo = 0, hi = 0;
              if (lanes(okm)) {
                if (is_global) {
                  if (w64) {
                    const uint2 v = *reinterpret_cast<const uint2*>(a.gmem + A);
                    lo = v.x;
                    hi = v.y;
                  } else {
                    lo = *reinterpret_cast<const uint32_t*>(a.gmem + A);
                  }
                } else {
                  lo = *reinterpret_cast<const uint32_t*>(win + A);
                  if (w64) hi = *reinterpret_cast<const uint32_t*>(win + A + 4);
                }
              }
              if (w64) R.put2_m(dst, lo, hi, on64);
              else R.put_m(dst, lo, on64);
            } else if (lanes(okm)) {
              if (w64) {
                uint32_t lo, hi;
                R.get2(s1, s1 + 1u, lo, hi);
                if (is_global) {
                  *reinterpret_cast<uint2*>(a.gmem + A) = make_uint2(lo, hi);
                  KS_EXT_STORE_WAIT();
                } else {
                  *reinterpret_cast<uint32_t*>(win + A) = lo;
                  *reinterpret_cast<uint32_t*>(win + A + 4) = hi;
                }
              } else {
                const uint32_t lo = R.get(s1);
                if (is_global) {
                  *reinterpret_cast<uint32_t*>(a.gmem + A) = lo;
                  KS_EXT_STORE_WAIT();
                } else {
                  *reinterpret_cast<uint32_t*>(win + A) = lo;
                }
              }
            }
            const uint64_t faults = on64 & ~okm;
            KS_COUNT_FAULTS(faults);
            [[maybe_unused]] uint32_t x_sl0 = 0, x_sl1 = 0;
            if (is_global) {
              KS_CACHE_ISSUE(A, okm);
              KS_GLOBAL_ACCOUNT(A, S, faults, is_load);
              KS_CACHE_FINISH(is_load, h[10]);
              if constexpr (EXT) {
                const uint32_t p0 = x_sl0 | (popc((uint32_t)on64) << 16) | (popc((uint32_t)faults) << 24);
                const uint32_t p1 = x_sl1 | (popc((uint32_t)(on64 >> 32)) << 16) | (popc((uint32_t)(faults >> 32)) << 24);
                KS_EXT_REC(is, off / (uint32_t)sizeof(DInst), is_load ? KS_EV_LD_GLOBAL : KS_EV_ST_GLOBAL, hl ? p1 : p0);
              }
            } else {
              const uint32_t g0 = (uint32_t)on64, g1 = (uint32_t)(on64 >> 32);
              const uint32_t hm = (g0 ? 1u : 0u) | (g1 ? 2u : 0u);  // warps with participating lanes
              uint32_t d0 = 1, d1 = 1;
              bool slow0 = g0 != 0, slow1 = g1 != 0;
              if (!faults) {
                // affine fast path for full halves: lanes at A0 + l * d
                const uint32_t a32 = (uint32_t)A;
                const uint32_t diff = a32 - prev_in_half(a32, lane);
                const uint32_t dA = rl(diff, 1), dB = rl(diff, 33);
                const uint64_t same = ballot(diff == (hl ? dB : dA));
                if (g0 == 0xFFFFFFFFu && ((uint32_t)same | 1u) == 0xFFFFFFFFu && (dA & 3u) == 0) {
                  const uint32_t ws = (dA >> 2) & 31u;
                  d0 = dA == 0 ? 1u : (ws == 0 ? 32u : (1u << __builtin_ctz(ws)));
                  slow0 = false;
                }
                if (g1 == 0xFFFFFFFFu && ((uint32_t)(same >> 32) | 1u) == 0xFFFFFFFFu && (dB & 3u) == 0) {
                  const uint32_t ws = (dB >> 2) & 31u;
                  d1 = dB == 0 ? 1u : (ws == 0 ? 32u : (1u << __builtin_ctz(ws)));
                  slow1 = false;
                }
              }
              if (slow0) d0 = bank_degree(A, (uint64_t)g0);
              if (slow1) d1 = bank_degree(A, (uint64_t)g1 << 32);
              const uint32_t dh = hl ? d1 : d0;
              if ((hm >> hl) & 1u) {
                if (sl == C_SH_N) cnt += 1;
                if (sl == C_SH_SUM) cnt += dh;
                if (sl == C_SH_MAX) cnt = umax(cnt, dh);
              }
              if constexpr (EXT) {
                const uint32_t p0 = ((hm & 1u) ? d0 : 0u) | (popc((uint32_t)on64) << 16) | (popc((uint32_t)faults) << 24);
                const uint32_t p1 = ((hm & 2u) ? d1 : 0u) | (popc((uint32_t)(on64 >> 32)) << 16) |
                                    (popc((uint32_t)(faults >> 32)) << 24);
                KS_EXT_REC(is, off / (uint32_t)sizeof(DInst), is_load ? KS_EV_LD_SHARED : KS_EV_ST_SHARED, hl ? p1 : p0);
              }
            }
          } else if (c & CB(DC_MOVSP)) {
            // t / bx and t / (bx by) as (t * m) >> 22 with m = ceil(2^22 / d) from the
            // host: exact for t < 1024 and d <= 1024, and cheaper than a division.  The
            // empty asm keeps these per-lane values here: hoisted out of the loop they
            // would hold registers for the whole run.
            uint32_t t_lin = my_w * 32u + sl;
            asm volatile("" : "+v"(t_lin));
            const uint32_t bx = a.block[0], by = a.block[1];
            const uint32_t gx = a.grid[0], gy = a.grid[1];
            const uint32_t qx = (t_lin * a.div_bx) >> 22;  // t / bx
            uint32_t v;
            switch (a0) {
              case KSP_TID_X: v = t_lin - qx * bx; break;
              case KSP_TID_Y: v = qx - ((qx * a.div_by) >> 22) * by; break;
              case KSP_TID_Z: v = (t_lin * a.div_bxy) >> 22; break;
              case KSP_NTID_X: v = a.block[0]; break;
              case KSP_NTID_Y: v = a.block[1]; break;
              case KSP_NTID_Z: v = a.block[2]; break;
              case KSP_CTAID_X: v = blk % gx; break;
              case KSP_CTAID_Y: v = (blk / gx) % gy; break;
              case KSP_CTAID_Z: v = blk / (gx * gy); break;
              case KSP_NCTAID_X: v = a.grid[0]; break;
              case KSP_NCTAID_Y: v = a.grid[1]; break;
              case KSP_NCTAID_Z: v = a.grid[2]; break;
              default: v = sl; break;
            }
            R.put_m(dst, v, on64);
          } else {  // DC_LDP: a uniform value from the launch arguments (scalar loads)
            typedef const __attribute__((address_space(4))) uint32_t* cword;
            const uint32_t lo = *(cword)(a.params + a0);
            if (a1) R.put2_m(dst, lo, *(cword)(a.params + a0 + 4u), on64);
            else R.put_m(dst, lo, on64);
          }
          // the next record (the end sentinel at the latest: a run never includes it),
          // and its issue cycle: its scoreboard reads go out with the record's load
          off += (uint32_t)sizeof(DInst);
          const u32x16 hn = *reinterpret_cast<const __attribute__((address_space(4))) u32x16*>(prog_b + off);
          asm volatile("" :: "s"(off));  // the record's load goes out ahead of the scoreboard reads
          const uint32_t r0 = sb_at(nsbo[0]), r1 = sb_at(nsbo[1]), r2 = sb_at(nsbo[2]), r3 = sb_at(nsbo[3]);
          h = hn;
          asm volatile("; prefetched %0" : : "s"(pf));
          is = umax(umax(v_next, r0), umax(umax(r1, r2), r3));
          if (--n == 0) break;
        }
        const uint32_t p = off / (uint32_t)sizeof(DInst);
        spc0 = go0 ? p : spc0;
        spc1 = go1 ? p : spc1;
        if constexpr (!EXT) {
          // a run that stopped for a full trace chunk writes it here
          const uint64_t fm = ballot(wi == ev) & ballot(wi == next_flush(fl)) & gm;
          if (fm) {
            if (lanes(fm) && sl < wi - fl) *reinterpret_cast<uint2*>(slot_base + 8ull * (fl + sl)) = staged();
            if (lanes(fm)) {
              fl = wi;
              ev = umin(next_flush(fl), budget);
            }
          }
        }
      }
      if (need & 1u) KS_SETTLE(0, S0, spc0);
      if (need & 2u) KS_SETTLE(1, S1, spc1);
    }

    // ------------------------------------------------------------------ barrier epoch
    const uint32_t slot = epoch % 3u;
    if (lane == 0) {
      const uint32_t alive = ((hst & DONE0) ? 0u : 1u) + ((hst & DONE1) ? 0u : 1u);
      // a waiting warp arrived at its last issue cycle: v_next - 1
      const uint32_t a0 = (hst & WAIT0) ? rl(v_next, 0) - 1u : 0u;
      const uint32_t a1 = (hst & WAIT1) ? rl(v_next, 32) - 1u : 0u;
      if (alive) {
        atomicAdd(&ep_alive[slot], alive);
        atomicMax(&ep_max[slot], umax(a0, a1));
      }
    }
    if (tid == 0) {  // clear the slot of the next epoch (last read two epochs ago)
      ep_alive[(epoch + 1u) % 3u] = 0;
      ep_max[(epoch + 1u) % 3u] = 0;
    }
    {
      // a waiting warp's issue count and next issue cycle from before the release
      uint8_t* const sbr = ((hst >> hl) & 1u) ? my_sb : dump_sb;
      *reinterpret_cast<uint32_t*>(sbr + 4u * KS_SB_BAR_WI) = wi;
      *reinterpret_cast<uint32_t*>(sbr + 4u * KS_SB_BAR_NEXT) = v_next;
    }
    __syncthreads();
    const uint32_t alive_all = uni(ep_alive[slot]);
    if (alive_all == 0) break;
    // release: every waiting warp's next issue waits for max(arrival) + lat(bar.sync)
    const uint32_t release = uni(ep_max[slot]) + a.lat_bar;
    const bool waiting = (hst >> hl) & 1u;
    if (waiting) v_next = umax(v_next, release);
    if (hst & WAIT0) spc0 = S0.pc;
    if (hst & WAIT1) spc1 = S1.pc;
    hst &= ~(WAIT0 | WAIT1);
    ++epoch;
  }
#undef KS_SETTLE
#undef KS_COUNT_FAULTS
#undef KS_GLOBAL_ACCOUNT
#undef KS_CACHE_ISSUE
#undef KS_CACHE_FINISH
  act += lanes(m64) ? wi : 0u;
#undef KS_SET_LIVE

  // -------------------------------------------------------------------- counters, trace tail, headers
  {
    const uint32_t w = my_w;
    // thread-instructions: the sum over the warp's lanes of their active counts
    uint64_t ti0 = 0, ti1 = 0;
    for (uint32_t l = 0; l < 32u; ++l) {
      ti0 += rl(act, l);
      ti1 += rl(act, 32u + l);
    }
    // per-lane analyser shares: lane 32 h + d of cnt holds counter d of warp h
    {
      const uint32_t qs[6] = {q_ln, q_ls, q_ll, q_sn, q_ss, q_sl};
      const uint32_t qd[6] = {C_GLD_N, C_GLD_SEC, C_GLD_LINES, C_GST_N, C_GST_SEC, C_GST_LINES};
      for (int k = 0; k < 6; ++k) {
        // read both totals here, with every lane active: a cross-lane read under a
        // lane condition may see lanes where the sum was never computed
        const uint32_t t = half_sum(qs[k]);
        const uint32_t t0 = rl(t, 31), t1 = rl(t, 63);
        cnt += sl == qd[k] ? (hl ? t1 : t0) : 0u;
      }
    }
    if (w < W) {
      const uint32_t m_status = (status >> (8u * hl)) & 0xFFu;
      const uint32_t m_depth = hl ? S1.md : S0.md;
      const uint64_t m_ti = hl ? ti1 : ti0;
      // last issue + 1: a release after the warp's last issue (a bar.sync) does not count
      const uint32_t cycles = wi == sb_at(4u * KS_SB_BAR_WI) ? sb_at(4u * KS_SB_BAR_NEXT) : v_next;
      const uint32_t written = umin(wi, cap);
      const uint32_t dropped = wi - written;
      const uint32_t st = m_status | (dropped ? KS_ST_TRACE_DROP : 0u);
      // this lane's warp, recomputed here (kept from the start it would hold two
      // registers through the whole run)
      uint32_t hl_e = hl;
      asm volatile("" : "+v"(hl_e));
      const uint64_t gw = gw0 + hl_e;
      // records staged since the last chunk write
      if (sl < written - fl) {
        if constexpr (EXT)
          *reinterpret_cast<uint4*>(slot_base + 16ull * (fl + sl)) = *reinterpret_cast<const uint4*>(my_ring + 16u * sl);
        else
          *reinterpret_cast<uint2*>(slot_base + 8ull * (fl + sl)) = staged();
      }
      if (sl < 20) {
        uint32_t v;
        switch (sl) {
          case C_TI_LO: v = (uint32_t)m_ti; break;
          case C_TI_HI: v = (uint32_t)(m_ti >> 32); break;
          case C_STATUS: v = st; break;
          case C_CYCLES: v = cycles; break;
          case C_WARP_INSTRS: v = wi; break;
          case C_STALL: v = cycles - wi; break;
          case C_MAXDEPTH: v = m_depth; break;
          case C_RES: v = 0; break;
          default: v = cnt; break;
        }
        reinterpret_cast<uint32_t*>(a.counters + gw * 80u)[sl] = v;
      }
      if constexpr (CACHE)  // the warp's cache outcome counts: L1 hits, L2 hits, misses
        if (sl >= 20u && sl < 23u) reinterpret_cast<uint32_t*>(a.cache + gw * (uint64_t)KS_CACHE_WARP_BYTES)[sl - 20u] = cnt;
      if (sl < 4) {
        const uint32_t flags = (dropped ? 1u : 0u) | ((st & KS_ST_FAULT) ? 2u : 0u) |
                               ((st & KS_ST_BUDGET) ? 4u : 0u) | ((st & KS_ST_FINISHED) ? 8u : 0u);
        uint32_t v;
        switch (sl) {
          case 0: v = written; break;
          case 1: v = (EXT ? 2u : 1u) | (flags << 8) | ((w & 0xFFFFu) << 16); break;  // version: record format
          case 2: v = dropped; break;
          default: v = 0; break;
        }
        reinterpret_cast<uint32_t*>(a.trace + gw * a.slot_bytes)[sl] = v;
      }
    }
  }
}

}  // namespace

// Register file in 40 reserved VGPRs (v56..v95): 96 VGPRs, 5 waves per SIMD,
// blocks up to 1024 threads.
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_num_vgpr(28))) ks_interp_v32(const KsArgs a) {
  interp<40, false, false>(a);
}

// Register file in 72 reserved VGPRs (v56..v127): 128 VGPRs, 4 waves per SIMD,
// blocks up to 1024 threads.
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_num_vgpr(28))) ks_interp_v64(const KsArgs a) {
  interp<72, false, false>(a);
}

// The same interpreters writing extended 16-byte trace records, with 64 compiler
// VGPRs and the register file from v64: 104 VGPRs (4 waves per SIMD, blocks up to
// 1024 threads) and 136 (3 waves per SIMD, so blocks up to 768 threads).
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_num_vgpr(32))) ks_interp_v32_ext(const KsArgs a) {
  interp<40, true, false>(a);
}
__global__ void __launch_bounds__(768) __attribute__((amdgpu_num_vgpr(32))) ks_interp_v64_ext(const KsArgs a) {
  interp<72, true, false>(a);
}
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_num_vgpr(28))) ks_interp_v32_cache(const KsArgs a) {
  interp<40, false, true>(a);
}
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_num_vgpr(28))) ks_interp_v64_cache(const KsArgs a) {
  interp<72, false, true>(a);
}

__global__ void ks_zero_word(uint32_t* out) { *out = 0; }

__global__ void ks_status_or_kernel(const uint8_t* counters, uint64_t n, uint32_t* out) {
  uint32_t acc = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    acc |= reinterpret_cast<const uint32_t*>(counters + i * 80u)[C_STATUS];
  for (int o = 32; o > 0; o >>= 1) acc |= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63u) == 0 && acc) atomicOr(out, acc);
}

size_t ks_lds_limit() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 65536;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 65536;
  return (size_t)v;
}

// Register-file variant for a program of `slots` slots (plus the immediate slots):
// 32 (40-VGPR file) or 64 (72-VGPR file); 0 if it fits neither.
int ks_choose_variant(uint32_t slots, uint32_t block_threads) {
  (void)block_threads;  // both variants run blocks of up to 1024 threads
  const uint32_t total = slots + KS_IMM_SLOTS + KS_CONST_SLOTS;
  if (total <= 40) return 32;
  if (total <= 72) return 64;
  return 0;
}

uint32_t ks_max_block_threads(int variant, bool ext) { return (ext && variant == 64) ? 768u : 1024u; }

size_t ks_lds_bytes(uint32_t wg, uint32_t shared_bytes, bool ext) {
  // scoreboards (+ staging rings) of the warps and a scratch one
  const size_t sb = ((size_t)(wg / 32u + 1u) * (ext ? KS_SB_ENTRIES : KS_SB_STRIDE) * 4u + 15u) & ~(size_t)15u;
  const size_t ring = ext ? (size_t)wg * 16u : 0u;  // 32 staged 16-byte records per warp
  return sb + ring + (((size_t)shared_bytes + 15u) & ~(size_t)15u);
}

hipError_t ks_launch_interp(const KsArgs& a, uint32_t n_blocks, uint32_t slots, hipStream_t s) {
  const uint32_t waves = (a.warps_per_block + 1u) / 2u;
  const uint32_t wg = 64u * waves;
  const int variant = ks_choose_variant(slots, a.threads_per_block);
  const size_t lds = ks_lds_bytes(wg, a.shared_bytes, a.ext != 0);
  if (variant == 0 || lds + 64 > ks_lds_limit() || wg > ks_max_block_threads(variant, a.ext != 0))
    return hipErrorInvalidValue;
  if (a.rf_slots != slots + KS_IMM_SLOTS + KS_CONST_SLOTS) return hipErrorInvalidValue;
  if (a.ext && a.cache_on) return hipErrorInvalidValue;
  const int vi = (variant == 32 ? 0 : 1) + (a.ext ? 2 : 0) + (a.cache_on ? 4 : 0);
  const void* const fns[6] = {(const void*)ks_interp_v32,     (const void*)ks_interp_v64,
                              (const void*)ks_interp_v32_ext, (const void*)ks_interp_v64_ext,
                              (const void*)ks_interp_v32_cache, (const void*)ks_interp_v64_cache};
  static bool attr_set[6] = {false, false, false, false, false, false};
  if (!attr_set[vi]) {
    hipError_t e = hipFuncSetAttribute(fns[vi], hipFuncAttributeMaxDynamicSharedMemorySize, (int)(ks_lds_limit() - 64));
    if (e != hipSuccess) return e;
    attr_set[vi] = true;
  }
  switch (vi) {
    case 0: hipLaunchKernelGGL(ks_interp_v32, dim3(n_blocks), dim3(wg), lds, s, a); break;
    case 1: hipLaunchKernelGGL(ks_interp_v64, dim3(n_blocks), dim3(wg), lds, s, a); break;
    case 2: hipLaunchKernelGGL(ks_interp_v32_ext, dim3(n_blocks), dim3(wg), lds, s, a); break;
    case 3: hipLaunchKernelGGL(ks_interp_v64_ext, dim3(n_blocks), dim3(wg), lds, s, a); break;
    case 4: hipLaunchKernelGGL(ks_interp_v32_cache, dim3(n_blocks), dim3(wg), lds, s, a); break;
    default: hipLaunchKernelGGL(ks_interp_v64_cache, dim3(n_blocks), dim3(wg), lds, s, a); break;
  }
  return hipGetLastError();
}

hipError_t ks_launch_status_or(const void* counters, uint64_t n_warps, uint32_t* d_out, hipStream_t s) {
  hipLaunchKernelGGL(ks_zero_word, dim3(1), dim3(1), 0, s, d_out);
  uint64_t blocks = (n_warps + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(ks_status_or_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, (const uint8_t*)counters, n_warps,
                     d_out);
  return hipGetLastError();
}
