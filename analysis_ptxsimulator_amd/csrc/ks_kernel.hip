// ks_kernel.hip -- the gfx950 SIMT interpreter of libkscope.
//
// Mapping (CDNA4, wave64):
//   * one workgroup = one simulated block; wave w runs simulated warps 2w
//     (lanes 0-31) and 2w+1 (lanes 32-63), one GPU lane per simulated thread;
//   * each wave-step executes ONE decoded instruction: the one at the smaller pc
//     of the two warps (both warps run it when they share that pc), so fetch
//     (s_load), decode, dispatch and register slot indices are wave-uniform;
//   * simulated registers live in a register file of 32-bit slots per lane,
//     either in physical VGPRs reserved for it (v96 upward, indexed in the
//     VGPR index mode of s_set_gpr_idx_on: zero latency, exec-masked writes) or,
//     for programs or blocks that do not fit, in LDS as [slot][thread];
//   * per-warp control state (stack top, masks, cycle counters) is scalar; the
//     divergence stack, scoreboard, counters and a 32-record trace staging
//     buffer live in VGPR lanes;
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

constexpr uint32_t H_RUN = 0, H_WAIT = 1, H_DONE = 2;
constexpr uint32_t RPC_EXIT = 0xFFFFFFFFu;
constexpr uint32_t CYCLE_LIMIT = 0x7FFFFFFFu;

// dword index of each field in the 80-byte counter record; the counter VGPR keeps
// counter d of half h in lane 32 h + d
enum {
  C_TI_LO = 0, C_TI_HI, C_STATUS, C_CYCLES, C_WARP_INSTRS, C_STALL, C_GLD_N, C_GLD_SEC, C_GLD_LINES,
  C_GST_N, C_GST_SEC, C_GST_LINES, C_SH_N, C_SH_SUM, C_SH_MAX, C_DIV, C_BAR, C_FAULT, C_MAXDEPTH, C_RES
};


typedef const __attribute__((address_space(4))) uint32_t* cu32p;

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
__device__ __forceinline__ uint32_t uni(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// ---------------------------------------------------------------------------- register files
//
// RF = 0: LDS, [slot][thread of the workgroup].  RF = 32 / 64: physical VGPRs
// v96 .. v96+RF-1, outside the compiler's allocation; slot s of a lane is VGPR
// v[96 + s] of that lane.  The kernels carry amdgpu_num_vgpr(48): on targets with
// the unified VGPR/AGPR file the compiler doubles that figure, so v96 and up are
// reserved (never allocated).  A larger figure that exceeds what the launch bound
// allows is silently ignored, which would hand v96+ back to the allocator; the
// build checks the assembly for any compiler-written use of them.
template <int RF>
struct RegFile;

template <>
struct RegFile<0> {
  uint32_t* base;
  uint32_t stride;
  uint32_t tid;
  __device__ __forceinline__ uint32_t get(uint32_t s) const { return base[s * stride + tid]; }
  __device__ __forceinline__ void get2(uint32_t i0, uint32_t i1, uint32_t& a, uint32_t& b) const {
    a = get(i0);
    b = get(i1);
  }
  __device__ __forceinline__ void get3(uint32_t i0, uint32_t i1, uint32_t i2, uint32_t& a, uint32_t& b,
                                       uint32_t& c) const {
    a = get(i0);
    b = get(i1);
    c = get(i2);
  }
  __device__ __forceinline__ void put(uint32_t s, uint32_t v) const { base[s * stride + tid] = v; }
  __device__ __forceinline__ void put2(uint32_t s, uint32_t lo, uint32_t hi) const {
    put(s, lo);
    put(s + 1, hi);
  }
};

// VGPR index mode: between s_set_gpr_idx_on and s_set_gpr_idx_off the SRC0 (or
// DST) VGPR operand of each VALU instruction is offset by the index held in M0;
// s_set_gpr_idx_idx changes the index without leaving the mode.
#define KS_RF_ASM_ACCESS                                                                          \
  __device__ __forceinline__ uint32_t get(uint32_t s) const {                                     \
    uint32_t r;                                                                                   \
    asm volatile("s_set_gpr_idx_on %1, gpr_idx(SRC0)\n\tv_mov_b32 %0, v96\n\ts_set_gpr_idx_off"  \
                 : "=v"(r) : "s"(s) : "m0");                                                     \
    return r;                                                                                     \
  }                                                                                               \
  __device__ __forceinline__ void get2(uint32_t i0, uint32_t i1, uint32_t& a, uint32_t& b) const { \
    asm volatile("s_set_gpr_idx_on %2, gpr_idx(SRC0)\n\tv_mov_b32 %0, v96\n\t"                    \
                 "s_set_gpr_idx_idx %3\n\tv_mov_b32 %1, v96\n\ts_set_gpr_idx_off"                 \
                 : "=&v"(a), "=v"(b) : "s"(i0), "s"(i1) : "m0");                                 \
  }                                                                                               \
  __device__ __forceinline__ void get3(uint32_t i0, uint32_t i1, uint32_t i2, uint32_t& a, uint32_t& b, \
                                       uint32_t& c) const {                                       \
    asm volatile("s_set_gpr_idx_on %3, gpr_idx(SRC0)\n\tv_mov_b32 %0, v96\n\t"                    \
                 "s_set_gpr_idx_idx %4\n\tv_mov_b32 %1, v96\n\t"                                  \
                 "s_set_gpr_idx_idx %5\n\tv_mov_b32 %2, v96\n\ts_set_gpr_idx_off"                 \
                 : "=&v"(a), "=&v"(b), "=v"(c) : "s"(i0), "s"(i1), "s"(i2) : "m0");              \
  }                                                                                               \
  __device__ __forceinline__ void put(uint32_t s, uint32_t v) const {                             \
    asm volatile("s_set_gpr_idx_on %0, gpr_idx(DST)\n\tv_mov_b32 v96, %1\n\ts_set_gpr_idx_off"   \
                 : : "s"(s), "v"(v) : "m0");                                                     \
  }                                                                                               \
  __device__ __forceinline__ void put2(uint32_t s, uint32_t lo, uint32_t hi) const {              \
    asm volatile("s_set_gpr_idx_on %0, gpr_idx(DST)\n\tv_mov_b32 v96, %1\n\t"                     \
                 "s_set_gpr_idx_idx %3\n\tv_mov_b32 v96, %2\n\ts_set_gpr_idx_off"                 \
                 : : "s"(s), "v"(lo), "v"(hi), "s"(s + 1) : "m0");                               \
  }

#define KS_Z(i) "v_mov_b32 v" #i ", 0\n\t"
#define KS_Z8(a, b, c, d, e, f, g, h) KS_Z(a) KS_Z(b) KS_Z(c) KS_Z(d) KS_Z(e) KS_Z(f) KS_Z(g) KS_Z(h)
#define KS_C8(a, b, c, d, e, f, g, h) "v" #a, "v" #b, "v" #c, "v" #d, "v" #e, "v" #f, "v" #g, "v" #h

template <>
struct RegFile<32> {
  KS_RF_ASM_ACCESS
  __device__ __forceinline__ static void zero() {
    asm volatile(KS_Z8(96, 97, 98, 99, 100, 101, 102, 103) KS_Z8(104, 105, 106, 107, 108, 109, 110, 111)
                     KS_Z8(112, 113, 114, 115, 116, 117, 118, 119) KS_Z8(120, 121, 122, 123, 124, 125, 126, 127)
                 ::: KS_C8(96, 97, 98, 99, 100, 101, 102, 103), KS_C8(104, 105, 106, 107, 108, 109, 110, 111),
                     KS_C8(112, 113, 114, 115, 116, 117, 118, 119), KS_C8(120, 121, 122, 123, 124, 125, 126, 127));
  }
};

template <>
struct RegFile<64> {
  KS_RF_ASM_ACCESS
  __device__ __forceinline__ static void zero() {
    asm volatile(KS_Z8(96, 97, 98, 99, 100, 101, 102, 103) KS_Z8(104, 105, 106, 107, 108, 109, 110, 111)
                     KS_Z8(112, 113, 114, 115, 116, 117, 118, 119) KS_Z8(120, 121, 122, 123, 124, 125, 126, 127)
                         KS_Z8(128, 129, 130, 131, 132, 133, 134, 135) KS_Z8(136, 137, 138, 139, 140, 141, 142, 143)
                             KS_Z8(144, 145, 146, 147, 148, 149, 150, 151) KS_Z8(152, 153, 154, 155, 156, 157, 158, 159)
                 ::: KS_C8(96, 97, 98, 99, 100, 101, 102, 103), KS_C8(104, 105, 106, 107, 108, 109, 110, 111),
                     KS_C8(112, 113, 114, 115, 116, 117, 118, 119), KS_C8(120, 121, 122, 123, 124, 125, 126, 127),
                     KS_C8(128, 129, 130, 131, 132, 133, 134, 135), KS_C8(136, 137, 138, 139, 140, 141, 142, 143),
                     KS_C8(144, 145, 146, 147, 148, 149, 150, 151), KS_C8(152, 153, 154, 155, 156, 157, 158, 159));
  }
};

// ---------------------------------------------------------------------------- divergence stack

// Per-warp control state, wave-uniform (SGPRs).  The next-issue cycle of a warp
// lives in a VGPR, uniform over the warp's 32 lanes.
struct Half {
  uint32_t pc, mask, rpc, sp;  // top of the divergence stack and its depth
  uint32_t m;                  // mask & ~exited of the top entry
  uint32_t exited, init_mask;
  uint32_t state, status, max_depth, arrival;
  uint32_t wi;                 // issued warp-instructions
};

__device__ __forceinline__ void hs_pop(Half& H, uint32_t spc, uint32_t sm, uint32_t sr) {
  H.sp -= 1;
  if (H.sp) {
    H.pc = rl(spc, H.sp - 1);
    H.mask = rl(sm, H.sp - 1);
    H.rpc = rl(sr, H.sp - 1);
  }
}

__device__ __forceinline__ void hs_push(Half& H, uint32_t& spc, uint32_t& sm, uint32_t& sr, uint32_t pc, uint32_t mask,
                                        uint32_t rpc, uint32_t lane) {
  spc = wl(spc, H.pc, H.sp - 1, lane);
  sm = wl(sm, H.mask, H.sp - 1, lane);
  sr = wl(sr, H.rpc, H.sp - 1, lane);
  H.pc = pc;
  H.mask = mask;
  H.m = mask & ~H.exited;
  H.rpc = rpc;
  H.sp += 1;
  H.max_depth = umax(H.max_depth, H.sp);
}

// The top entry cannot issue: no live lane, reconverged, or past the end.
__device__ __forceinline__ bool hs_blocked(const Half& H, uint32_t n) {
  return H.state == H_RUN && (H.m == 0 || H.pc == H.rpc || H.pc >= n);
}

// Pop finished or reconverged entries; lanes that ran off the end exit at no cost.
__device__ __forceinline__ void hs_settle(Half& H, uint32_t spc, uint32_t sm, uint32_t sr, uint32_t n) {
  while (H.sp) {
    H.m = H.mask & ~H.exited;
    if (H.m == 0 || H.pc == H.rpc) {
      hs_pop(H, spc, sm, sr);
      continue;
    }
    if (H.pc >= n) {
      H.exited |= H.m;
      continue;
    }
    return;
  }
  H.state = H_DONE;
  H.status |= KS_ST_FINISHED;
}

__device__ __forceinline__ void half_init(Half& H, uint32_t w, uint32_t W, uint32_t T) {
  const bool exists = w < W;
  const uint32_t live = T > w * 32u ? (T - w * 32u > 32u ? 32u : T - w * 32u) : 0u;
  H.init_mask = live >= 32u ? 0xFFFFFFFFu : ((1u << live) - 1u);
  H.pc = 0;
  H.mask = H.init_mask;
  H.m = H.init_mask;
  H.rpc = RPC_EXIT;
  H.sp = exists ? 1u : 0u;
  H.exited = 0;
  H.state = exists ? H_RUN : H_DONE;
  H.status = 0;
  H.max_depth = 1;
  H.arrival = 0;
  H.wi = 0;
}

__device__ __forceinline__ uint32_t cnt_add(uint32_t cnt, uint32_t lane, uint32_t idx, uint32_t v) {
  return cnt + (lane == idx ? v : 0u);
}


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

// ---------------------------------------------------------------------------- the interpreter

template <int RF>
__device__ __forceinline__ void interp(const KsArgs& a) {
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ uint32_t ep_max[3], ep_alive[3];

  const uint32_t WG = blockDim.x;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = uni(tid >> 6);  // wave-uniform: keeps every per-warp value scalar
  const uint32_t hl = lane >> 5;
  const uint32_t sl = lane & 31u;
  const uint32_t blk = blockIdx.x;
  const uint32_t W = a.warps_per_block;
  const uint32_t T = a.threads_per_block;
  const uint32_t n_instr = a.n_instrs;

  // LDS: [register file (LDS variant)] [scoreboard, 129 words per warp] [shared window]
  RegFile<RF> R;
  const uint32_t rf_words = RF == 0 ? (a.rf_slots ? a.rf_slots : 1u) * WG : 0u;
  if constexpr (RF == 0) {
    R.base = lds;
    R.stride = WG;
    R.tid = tid;
  } else {
    RegFile<RF>::zero();
  }
  uint32_t* const sbw = lds + rf_words;
  uint8_t* const win = reinterpret_cast<uint8_t*>(sbw + (WG / 32u) * KS_SB_ENTRIES);
  {
    const uint32_t words = rf_words + (WG / 32u) * KS_SB_ENTRIES + ((a.shared_bytes + 3u) >> 2);
    for (uint32_t i = tid; i < words; i += WG) lds[i] = 0;
    if (tid < 3) {
      ep_max[tid] = 0;
      ep_alive[tid] = 0;
    }
  }
  __syncthreads();

  // special registers of this lane's simulated thread
  const uint32_t my_w = 2u * wave + hl;
  const uint32_t t_lin = my_w * 32u + sl;
  const uint32_t bx = a.block[0], by = a.block[1];
  const uint32_t tid_x = t_lin % bx, tid_y = (t_lin / bx) % by, tid_z = t_lin / (bx * by);
  const uint32_t gx = a.grid[0], gy = a.grid[1];
  const uint32_t cta_x = blk % gx, cta_y = (blk / gx) % gy, cta_z = blk / (gx * gy);
  const bool small_gmem = a.gmem_bytes <= (1ull << 37);  // sector ids of valid accesses fit 32 bits
  uint32_t* const my_sb = sbw + my_w * KS_SB_ENTRIES;    // this lane's warp's scoreboard

  Half H0, H1;
  half_init(H0, 2u * wave, W, T);
  half_init(H1, 2u * wave + 1u, W, T);
  uint32_t stk_pc0 = 0, stk_m0 = 0, stk_r0 = 0, stk_pc1 = 0, stk_m1 = 0, stk_r1 = 0;
  uint32_t v_next = 0;      // previous issue cycle + 1 of the lane's warp (uniform over the warp)
  uint32_t cnt = 0;         // counter d of the lane's warp in lane 32 h + d
  uint32_t pbits = 0;       // predicate p of this lane's thread in bit p
  uint32_t tr_c = 0, tr_p = 0;  // trace staging: record k of a warp in its lane k % 32
  uint32_t act = 0;         // instructions issued with this lane's thread active

  const uint32_t cap = a.trace_cap;
  const uint32_t budget = a.max_warp_instrs;
  const uint64_t gw0 = (uint64_t)blk * W + 2u * wave;  // global warp id of half 0
  uint8_t* const slot_base = a.trace + (gw0 + hl) * a.slot_bytes + 16u;  // this lane's warp's records

  uint32_t epoch = 0;
  while (true) {
    // ------------------------------------------------------------------ run both warps until blocked
    while (true) {
      if (hs_blocked(H0, n_instr)) hs_settle(H0, stk_pc0, stk_m0, stk_r0, n_instr);
      if (hs_blocked(H1, n_instr)) hs_settle(H1, stk_pc1, stk_m1, stk_r1, n_instr);
      const bool r0 = H0.state == H_RUN, r1 = H1.state == H_RUN;
      if (!r0 && !r1) break;
      const uint32_t pc = uni((r0 && r1) ? (H0.pc < H1.pc ? H0.pc : H1.pc) : (r0 ? H0.pc : H1.pc));
      bool go0 = r0 && H0.pc == pc, go1 = r1 && H1.pc == pc;
      if ((go0 && H0.wi >= budget) || (go1 && H1.wi >= budget)) {  // issue budget
        if (go0 && H0.wi >= budget) {
          H0.state = H_DONE;
          H0.status |= KS_ST_BUDGET;
        }
        if (go1 && H1.wi >= budget) {
          H1.state = H_DONE;
          H1.status |= KS_ST_BUDGET;
        }
        continue;
      }

      const cu32p I = (cu32p)(uintptr_t)(a.prog + pc);
      const uint32_t w0 = I[0], w1 = I[1], wsb = I[2], w3 = I[3];
      const uint32_t op = w0 & 0xFFu, flags = (w0 >> 8) & 0xFFu, dst = (w0 >> 16) & 0xFFu, guard = w0 >> 24;
      const uint32_t kinds = w1 >> 24;
      const uint32_t sb_dst = w3 & 0xFFu, cmp = (w3 >> 8) & 0xFFu, lat = w3 >> 16;

      // lanes of the warps that issue this instruction
      const uint64_t gm = (go0 ? 0xFFFFFFFFull : 0ull) | (go1 ? 0xFFFFFFFF00000000ull : 0ull);

      // issue cycle (per warp, uniform over its lanes): the later of the previous issue
      // + 1 and the ready cycle of every register source (absent sources read entry 127 = 0)
      const uint32_t iss = umax(v_next, umax(umax(my_sb[wsb & 0xFFu], my_sb[(wsb >> 8) & 0xFFu]),
                                             umax(my_sb[(wsb >> 16) & 0xFFu], my_sb[wsb >> 24])));
      {
        const uint64_t ovf = ballot(iss > CYCLE_LIMIT) & gm;
        if (ovf) {
          if (ovf & 1u) {
            H0.state = H_DONE;
            H0.status |= KS_ST_CYCLE_OVF;
          }
          if (ovf >> 32) {
            H1.state = H_DONE;
            H1.status |= KS_ST_CYCLE_OVF;
          }
          continue;
        }
      }
      const uint32_t m0 = go0 ? H0.m : 0u;
      const uint32_t m1 = go1 ? H1.m : 0u;

      // trace: stage the record in lane k % 32 of the warp; write 32 records at once
      {
        const bool rec0 = go0 && H0.wi < cap, rec1 = go1 && H1.wi < cap;
        const uint32_t k0 = H0.wi & 31u, k1 = H1.wi & 31u;
        const uint64_t smask = (rec0 ? (1ull << k0) : 0ull) | (rec1 ? (1ull << (32 + k1)) : 0ull);
        if (__builtin_amdgcn_inverse_ballot_w64(smask)) {
          tr_c = iss;
          tr_p = pc;
        }
        const bool fl0 = rec0 && (k0 == 31u || H0.wi + 1u == cap);
        const bool fl1 = rec1 && (k1 == 31u || H1.wi + 1u == cap);
        if (fl0 || fl1) {
          const uint64_t fmask = (fl0 ? (0xFFFFFFFFull >> (31u - k0)) : 0ull) |
                                 (fl1 ? ((0xFFFFFFFFull >> (31u - k1)) << 32) : 0ull);
          const uint32_t chunk = (hl ? H1.wi : H0.wi) & ~31u;
          if (__builtin_amdgcn_inverse_ballot_w64(fmask))
            *reinterpret_cast<uint2*>(slot_base + 8ull * (chunk + sl)) = make_uint2(tr_c, tr_p);
        }
      }
      H0.wi += go0 ? 1u : 0u;
      H1.wi += go1 ? 1u : 0u;
      act += __builtin_amdgcn_inverse_ballot_w64((uint64_t)m0 | ((uint64_t)m1 << 32)) ? 1u : 0u;
      if (__builtin_amdgcn_inverse_ballot_w64(gm)) {
        v_next = iss + 1;
        if (sb_dst != 0xFFu) my_sb[sb_dst] = iss + lat;
      }

      // guard: lanes that execute
      uint64_t on64 = (uint64_t)m0 | ((uint64_t)m1 << 32);
      if (flags & KF_GUARD) on64 &= ballot((((pbits >> guard) & 1u) != 0) != ((flags & KF_GUARD_NEG) != 0));
      const bool on = __builtin_amdgcn_inverse_ballot_w64(on64);
      const uint32_t g0 = (uint32_t)on64, g1 = (uint32_t)(on64 >> 32);

      // ---------------------------------------------------------------- execute
      if (op < KO_LDP32) {
        if (on) {
          const uint32_t s0 = w1 & 0xFFu, s1 = (w1 >> 8) & 0xFFu, s2 = (w1 >> 16) & 0xFFu;
          const uint32_t k0 = kinds & 3u, k1 = (kinds >> 2) & 3u, k2 = (kinds >> 4) & 3u;
          // register or immediate operands: the three slots are read in one go (slot 0 stands
          // in for an immediate), then immediates replace the values read
          uint32_t x0, x1, x2;
          R.get3(s0, s1, s2, x0, x1, x2);
          x0 = k0 == KK_REG ? x0 : I[6];
          x1 = k1 == KK_REG ? x1 : I[8];
          x2 = k2 == KK_REG ? x2 : I[10];
          auto rd64 = [&](uint32_t kind, uint32_t s, uint32_t imm_lo, uint32_t imm_hi) -> uint64_t {
            if (kind == KK_REG) {
              uint32_t lo, hi;
              R.get2(s, s + 1, lo, hi);
              return (uint64_t)lo | ((uint64_t)hi << 32);
            }
            return (uint64_t)imm_lo | ((uint64_t)imm_hi << 32);
          };
          uint32_t rlo = 0, rhi = 0;
          bool wide = false, wr = true;
          switch (op) {
            case KO_ADD32: rlo = x0 + x1; break;
            case KO_SUB32: rlo = x0 - x1; break;
            case KO_MUL32: rlo = x0 * x1; break;
            case KO_MAD32: rlo = x0 * x1 + x2; break;
            case KO_ADD64:
            case KO_SUB64:
            case KO_MUL64:
            case KO_MAD64: {
              const uint64_t x = rd64(k0, s0, I[6], I[7]), y = rd64(k1, s1, I[8], I[9]);
              uint64_t r;
              if (op == KO_ADD64) r = x + y;
              else if (op == KO_SUB64) r = x - y;
              else if (op == KO_MUL64) r = x * y;
              else r = x * y + rd64(k2, s2, I[10], I[11]);
              rlo = (uint32_t)r;
              rhi = (uint32_t)(r >> 32);
              wide = true;
              break;
            }
            case KO_MULWIDE_S: {
              const int64_t r = (int64_t)(int32_t)x0 * (int64_t)(int32_t)x1;
              rlo = (uint32_t)r;
              rhi = (uint32_t)((uint64_t)r >> 32);
              wide = true;
              break;
            }
            case KO_MULWIDE_U: {
              const uint64_t r = (uint64_t)x0 * (uint64_t)x1;
              rlo = (uint32_t)r;
              rhi = (uint32_t)(r >> 32);
              wide = true;
              break;
            }
            case KO_FADD:
              rlo = canon_bits(__uint_as_float(x0) + __uint_as_float(x1));
              break;
            case KO_FSUB:
              rlo = canon_bits(__uint_as_float(x0) - __uint_as_float(x1));
              break;
            case KO_FMUL:
              rlo = canon_bits(__uint_as_float(x0) * __uint_as_float(x1));
              break;
            case KO_FFMA:
              rlo = canon_bits(__builtin_fmaf(__uint_as_float(x0), __uint_as_float(x1),
                                              __uint_as_float(x2)));
              break;
            case KO_SETP_S32:
            case KO_SETP_U32:
            case KO_SETP_S64:
            case KO_SETP_U64:
            case KO_SETP_F32: {
              bool c;
              if (op == KO_SETP_F32) {
                const float x = __uint_as_float(x0), y = __uint_as_float(x1);
                // ordered comparisons: false whenever an input is NaN
                switch (cmp) {
                  case KC_EQ: c = x == y; break;
                  case KC_NE: c = x < y || x > y; break;
                  case KC_LT: c = x < y; break;
                  case KC_LE: c = x <= y; break;
                  case KC_GT: c = x > y; break;
                  default: c = x >= y; break;
                }
              } else if (op == KO_SETP_S32 || op == KO_SETP_U32) {
                const uint32_t x = x0, y = x1;
                const bool lt = op == KO_SETP_S32 ? (int32_t)x < (int32_t)y : x < y;
                switch (cmp) {
                  case KC_EQ: c = x == y; break;
                  case KC_NE: c = x != y; break;
                  case KC_LT: c = lt; break;
                  case KC_LE: c = lt || x == y; break;
                  case KC_GT: c = !lt && x != y; break;
                  default: c = !lt; break;
                }
              } else {
                const uint64_t x = rd64(k0, s0, I[6], I[7]), y = rd64(k1, s1, I[8], I[9]);
                const bool lt = op == KO_SETP_S64 ? (int64_t)x < (int64_t)y : x < y;
                switch (cmp) {
                  case KC_EQ: c = x == y; break;
                  case KC_NE: c = x != y; break;
                  case KC_LT: c = lt; break;
                  case KC_LE: c = lt || x == y; break;
                  case KC_GT: c = !lt && x != y; break;
                  default: c = !lt; break;
                }
              }
              pbits = (pbits & ~(1u << dst)) | ((c ? 1u : 0u) << dst);
              wr = false;
              break;
            }
            case KO_SELP32:
            case KO_SELP64: {
              const bool p = (pbits >> s2) & 1u;
              if (op == KO_SELP32) {
                const uint32_t x = x0, y = x1;
                rlo = p ? x : y;
              } else {
                const uint64_t x = rd64(k0, s0, I[6], I[7]), y = rd64(k1, s1, I[8], I[9]);
                const uint64_t r = p ? x : y;
                rlo = (uint32_t)r;
                rhi = (uint32_t)(r >> 32);
                wide = true;
              }
              break;
            }
            case KO_MOV32:
              if (k0 == KK_SPECIAL) {
                switch (s0) {
                  case KSP_TID_X: rlo = tid_x; break;
                  case KSP_TID_Y: rlo = tid_y; break;
                  case KSP_TID_Z: rlo = tid_z; break;
                  case KSP_NTID_X: rlo = a.block[0]; break;
                  case KSP_NTID_Y: rlo = a.block[1]; break;
                  case KSP_NTID_Z: rlo = a.block[2]; break;
                  case KSP_CTAID_X: rlo = cta_x; break;
                  case KSP_CTAID_Y: rlo = cta_y; break;
                  case KSP_CTAID_Z: rlo = cta_z; break;
                  case KSP_NCTAID_X: rlo = a.grid[0]; break;
                  case KSP_NCTAID_Y: rlo = a.grid[1]; break;
                  case KSP_NCTAID_Z: rlo = a.grid[2]; break;
                  default: rlo = sl; break;
                }
              } else {
                rlo = x0;
              }
              break;
            default: {  // KO_MOV64
              const uint64_t r = rd64(k0, s0, I[6], I[7]);
              rlo = (uint32_t)r;
              rhi = (uint32_t)(r >> 32);
              wide = true;
              break;
            }
          }
          if (wr) {
            R.put(dst, rlo);
            if (wide) R.put(dst + 1, rhi);
          }
        }
      } else if (op <= KO_LDP64) {
        // parameter load: uniform value from the launch arguments
        const uint32_t aux = I[5] & 0xFFFFu;
        const uint32_t lo = *reinterpret_cast<const uint32_t*>(a.params + aux);
        const uint32_t hi = op == KO_LDP64 ? *reinterpret_cast<const uint32_t*>(a.params + aux + 4) : 0u;
        if (on) {
          R.put(dst, lo);
          if (op == KO_LDP64) R.put(dst + 1, hi);
        }
      } else if (op <= KO_STS64) {
        const bool is_global = op <= KO_STG64;
        const bool is_load = op == KO_LDG32 || op == KO_LDG64 || op == KO_LDS32 || op == KO_LDS64;
        const bool w64 = op == KO_LDG64 || op == KO_STG64 || op == KO_LDS64 || op == KO_STS64;
        const uint32_t S = w64 ? 8u : 4u;
        const uint64_t size = is_global ? a.gmem_bytes : (uint64_t)a.shared_bytes;
        const uint32_t s0 = w1 & 0xFFu, s1 = (w1 >> 8) & 0xFFu;
        const uint32_t addr_w = I[6];
        const uint64_t off = (uint64_t)I[12] | ((uint64_t)I[13] << 32);
        uint64_t A = 0;
        bool ok = false;
        if (on) {
          uint64_t base = R.get(s0);
          if (addr_w == 64u) base |= (uint64_t)R.get(s0 + 1) << 32;
          A = base + off;
          ok = (A & (S - 1u)) == 0 && A <= size && size - A >= S;
          if (is_load) {
            uint32_t lo = 0, hi = 0;
            if (ok) {
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
            R.put(dst, lo);
            if (w64) R.put(dst + 1, hi);
          } else if (ok) {
            const uint32_t lo = R.get(s1);
            if (is_global) {
              if (w64) {
                *reinterpret_cast<uint2*>(a.gmem + A) = make_uint2(lo, R.get(s1 + 1));
              } else {
                *reinterpret_cast<uint32_t*>(a.gmem + A) = lo;
              }
            } else {
              *reinterpret_cast<uint32_t*>(win + A) = lo;
              if (w64) *reinterpret_cast<uint32_t*>(win + A + 4) = R.get(s1 + 1);
            }
          }
        }
        // fault counting and analysis (full exec)
        const uint64_t faults = ballot(on && !ok);
        if (faults) {
          const uint32_t f0 = (uint32_t)__builtin_popcountll(faults & 0xFFFFFFFFull);
          const uint32_t f1 = (uint32_t)__builtin_popcountll(faults >> 32);
          if (f0) {
            H0.status |= KS_ST_FAULT;
            cnt = cnt_add(cnt, lane, C_FAULT, f0);
          }
          if (f1) {
            H1.status |= KS_ST_FAULT;
            cnt = cnt_add(cnt, lane, 32 + C_FAULT, f1);
          }
        }
        if (is_global) {
          uint32_t sec0 = 0, lin0 = 0, sec1 = 0, lin1 = 0;
          bool slow0 = g0 != 0, slow1 = g1 != 0;
          if (!faults && small_gmem) {
            // monotone fast path: prefix max of sector ids over the active lanes of each half
            const uint32_t s = on ? (uint32_t)(A >> 5) : 0u;
            const uint32_t prev = prev_in_half(half_prefix_max(s), lane);
            const uint64_t nonmono = ballot(on && s < prev);
            const uint64_t news = ballot(on && s != prev);
            const uint64_t newl = ballot(on && (s >> 2) != (prev >> 2));
            if (g0 && !(uint32_t)nonmono) {
              const uint32_t first = g0 & (0u - g0);
              sec0 = (uint32_t)__builtin_popcount((uint32_t)news | first);
              lin0 = (uint32_t)__builtin_popcount((uint32_t)newl | first);
              slow0 = false;
            }
            if (g1 && !(uint32_t)(nonmono >> 32)) {
              const uint32_t first = g1 & (0u - g1);
              sec1 = (uint32_t)__builtin_popcount((uint32_t)(news >> 32) | first);
              lin1 = (uint32_t)__builtin_popcount((uint32_t)(newl >> 32) | first);
              slow1 = false;
            }
          }
          if (slow0 || slow1) {
            const uint64_t last = A + (S - 1u);
            if (slow0) {
              sec0 = distinct2(A >> 5, last >> 5, (uint64_t)g0);
              lin0 = distinct2(A >> 7, last >> 7, (uint64_t)g0);
            }
            if (slow1) {
              sec1 = distinct2(A >> 5, last >> 5, (uint64_t)g1 << 32);
              lin1 = distinct2(A >> 7, last >> 7, (uint64_t)g1 << 32);
            }
          }
          // counters n, sectors, lines of the lane's warp: lanes 32 h + {cn, cn+1, cn+2}
          const uint32_t cn = is_load ? C_GLD_N : C_GST_N;
          const uint32_t gh = hl ? g1 : g0;
          const uint32_t d = sl - cn;
          if (gh && d < 3u) cnt += d == 0 ? 1u : (d == 1 ? (hl ? sec1 : sec0) : (hl ? lin1 : lin0));
        } else {
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
          const uint32_t gh = hl ? g1 : g0;
          const uint32_t dh = hl ? d1 : d0;
          if (gh) {
            if (sl == C_SH_N) cnt += 1;
            if (sl == C_SH_SUM) cnt += dh;
            if (sl == C_SH_MAX) cnt = umax(cnt, dh);
          }
        }
      }

      // ---------------------------------------------------------------- control (scalar)
      if (op == KO_BRA) {
        const uint32_t w4 = I[4];
        const uint32_t target = w4 & 0xFFFFu, rpc_raw = w4 >> 16;
        const uint32_t rpc = rpc_raw == KS_RPC_EXIT ? RPC_EXIT : rpc_raw;
        if (go0) {
          const uint32_t nt = m0 & ~g0;
          if (nt == 0) {
            H0.pc = target;
          } else if (g0 == 0) {
            H0.pc = pc + 1;
          } else {
            H0.pc = rpc;
            cnt = cnt_add(cnt, lane, C_DIV, 1);
            if (target != rpc) hs_push(H0, stk_pc0, stk_m0, stk_r0, target, g0, rpc, lane);
            if (pc + 1 != rpc) hs_push(H0, stk_pc0, stk_m0, stk_r0, pc + 1, nt, rpc, lane);
          }
        }
        if (go1) {
          const uint32_t nt = m1 & ~g1;
          if (nt == 0) {
            H1.pc = target;
          } else if (g1 == 0) {
            H1.pc = pc + 1;
          } else {
            H1.pc = rpc;
            cnt = cnt_add(cnt, lane, 32 + C_DIV, 1);
            if (target != rpc) hs_push(H1, stk_pc1, stk_m1, stk_r1, target, g1, rpc, lane);
            if (pc + 1 != rpc) hs_push(H1, stk_pc1, stk_m1, stk_r1, pc + 1, nt, rpc, lane);
          }
        }
      } else if (op == KO_RET) {
        if (go0) {
          H0.exited |= g0;
          H0.m = H0.mask & ~H0.exited;
          H0.pc = pc + 1;
        }
        if (go1) {
          H1.exited |= g1;
          H1.m = H1.mask & ~H1.exited;
          H1.pc = pc + 1;
        }
      } else if (op == KO_BAR) {
        if (go0) {
          cnt = cnt_add(cnt, lane, C_BAR, 1);
          if (m0 != (H0.init_mask & ~H0.exited)) H0.status |= KS_ST_BARDIV;
          H0.state = H_WAIT;
          H0.arrival = rl(iss, 0);
          H0.pc = pc + 1;
        }
        if (go1) {
          cnt = cnt_add(cnt, lane, 32 + C_BAR, 1);
          if (m1 != (H1.init_mask & ~H1.exited)) H1.status |= KS_ST_BARDIV;
          H1.state = H_WAIT;
          H1.arrival = rl(iss, 32);
          H1.pc = pc + 1;
        }
      } else {
        H0.pc += go0 ? 1u : 0u;
        H1.pc += go1 ? 1u : 0u;
      }
    }

    // ------------------------------------------------------------------ barrier epoch
    const uint32_t slot = epoch % 3u;
    if (lane == 0) {
      const uint32_t alive = (H0.state != H_DONE ? 1u : 0u) + (H1.state != H_DONE ? 1u : 0u);
      uint32_t mx = H0.state == H_WAIT ? H0.arrival : 0u;
      if (H1.state == H_WAIT && H1.arrival > mx) mx = H1.arrival;
      if (alive) {
        atomicAdd(&ep_alive[slot], alive);
        atomicMax(&ep_max[slot], mx);
      }
    }
    if (tid == 0) {  // clear the slot of the next epoch (last read two epochs ago)
      ep_alive[(epoch + 1u) % 3u] = 0;
      ep_max[(epoch + 1u) % 3u] = 0;
    }
    __syncthreads();
    const uint32_t alive_all = uni(ep_alive[slot]);
    if (alive_all == 0) break;
    // release: every waiting warp's next issue waits for max(arrival) + lat(bar.sync)
    const uint32_t release = uni(ep_max[slot]) + a.lat_bar;
    const bool waiting = hl ? H1.state == H_WAIT : H0.state == H_WAIT;
    if (waiting) v_next = umax(v_next, release);
    if (H0.state == H_WAIT) H0.state = H_RUN;
    if (H1.state == H_WAIT) H1.state = H_RUN;
    ++epoch;
  }

  // -------------------------------------------------------------------- counters, trace tail, headers
  {
    const uint32_t w = my_w;
    if (w < W) {
      const uint32_t m_status = hl ? H1.status : H0.status;
      const uint32_t m_depth = hl ? H1.max_depth : H0.max_depth;
      const uint32_t m_wi = hl ? H1.wi : H0.wi;
      // thread-instructions: the sum over the warp's lanes of their active counts
      uint64_t ti0 = 0, ti1 = 0;
      for (uint32_t l = 0; l < 32u; ++l) {
        ti0 += rl(act, l);
        ti1 += rl(act, 32u + l);
      }
      const uint64_t m_ti = hl ? ti1 : ti0;
      const uint32_t cycles = v_next;
      const uint32_t written = m_wi < cap ? m_wi : cap;
      const uint32_t dropped = m_wi - written;
      const uint32_t status = m_status | (dropped ? KS_ST_TRACE_DROP : 0u);
      const uint64_t gw = gw0 + hl;
      // staged records of a last, partly filled chunk (a full chunk was written when it filled)
      if (sl < (written & 31u))
        *reinterpret_cast<uint2*>(slot_base + 8ull * ((written & ~31u) + sl)) = make_uint2(tr_c, tr_p);
      if (sl < 20) {
        uint32_t v;
        switch (sl) {
          case C_TI_LO: v = (uint32_t)m_ti; break;
          case C_TI_HI: v = (uint32_t)(m_ti >> 32); break;
          case C_STATUS: v = status; break;
          case C_CYCLES: v = cycles; break;
          case C_WARP_INSTRS: v = m_wi; break;
          case C_STALL: v = cycles - m_wi; break;
          case C_MAXDEPTH: v = m_depth; break;
          case C_RES: v = 0; break;
          default: v = cnt; break;
        }
        reinterpret_cast<uint32_t*>(a.counters + gw * 80u)[sl] = v;
      }
      if (sl < 4) {
        const uint32_t flags = (dropped ? 1u : 0u) | ((status & KS_ST_FAULT) ? 2u : 0u) |
                               ((status & KS_ST_BUDGET) ? 4u : 0u) | ((status & KS_ST_FINISHED) ? 8u : 0u);
        uint32_t v;
        switch (sl) {
          case 0: v = written; break;
          case 1: v = 1u | (flags << 8) | ((w & 0xFFFFu) << 16); break;
          case 2: v = dropped; break;
          default: v = 0; break;
        }
        reinterpret_cast<uint32_t*>(a.trace + gw * a.slot_bytes)[sl] = v;
      }
    }
  }
}


}  // namespace

// Register file in LDS: any slot count that fits, blocks up to 1024 threads.
__global__ void __launch_bounds__(1024) ks_interp_lds(const KsArgs a) { interp<0>(a); }

// Register file in 32 reserved VGPRs (v96..v127): 128 VGPRs, blocks up to 1024 threads.
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_num_vgpr(48))) ks_interp_v32(const KsArgs a) {
  interp<32>(a);
}

// Register file in 64 reserved VGPRs (v96..v159): 160 VGPRs, blocks up to 768 threads.
__global__ void __launch_bounds__(768) __attribute__((amdgpu_num_vgpr(48))) ks_interp_v64(const KsArgs a) {
  interp<64>(a);
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

int ks_choose_variant(uint32_t slots, uint32_t block_threads) {
  const uint32_t waves = ((block_threads + 31u) / 32u + 1u) / 2u;
  if (slots <= 32) return 32;
  if (slots <= 64 && waves <= 12) return 64;
  return 0;
}

size_t ks_lds_bytes(int variant, uint32_t slots, uint32_t wg, uint32_t shared_bytes) {
  const size_t rf = variant == 0 ? (size_t)(slots ? slots : 1u) * wg * 4u : 0u;
  const size_t sb = (size_t)(wg / 32u) * KS_SB_ENTRIES * 4u;
  return rf + sb + (((size_t)shared_bytes + 15u) & ~(size_t)15u);
}

hipError_t ks_launch_interp(const KsArgs& a, uint32_t n_blocks, uint32_t slots, hipStream_t s) {
  const uint32_t waves = (a.warps_per_block + 1u) / 2u;
  const uint32_t wg = 64u * waves;
  const int variant = ks_choose_variant(slots, a.threads_per_block);
  const size_t lds = ks_lds_bytes(variant, slots, wg, a.shared_bytes);
  if (lds + 64 > ks_lds_limit()) return hipErrorInvalidValue;
  const void* fn = variant == 32 ? (const void*)ks_interp_v32
                   : variant == 64 ? (const void*)ks_interp_v64
                                   : (const void*)ks_interp_lds;
  static bool attr_set[3] = {false, false, false};
  const int vi = variant == 0 ? 0 : (variant == 32 ? 1 : 2);
  if (!attr_set[vi]) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(ks_lds_limit() - 64));
    if (e != hipSuccess) return e;
    attr_set[vi] = true;
  }
  if (variant == 32) hipLaunchKernelGGL(ks_interp_v32, dim3(n_blocks), dim3(wg), lds, s, a);
  else if (variant == 64) hipLaunchKernelGGL(ks_interp_v64, dim3(n_blocks), dim3(wg), lds, s, a);
  else hipLaunchKernelGGL(ks_interp_lds, dim3(n_blocks), dim3(wg), lds, s, a);
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
