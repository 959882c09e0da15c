// ks_kernel.hip -- the gfx950 SIMT interpreter of libkscope.
//
// Mapping (CDNA4, wave64):
//   * one workgroup = one simulated block; wave w runs simulated warps 2w
//     (lanes 0-31) and 2w+1 (lanes 32-63), one GPU lane per simulated thread;
//   * each wave-step executes ONE decoded instruction: the one at the smaller pc
//     of the two warps (both warps run it when they share that pc), so the
//     instruction fetch (s_load), decode, dispatch and operand slot indices are
//     wave-uniform and live in SGPRs;
//   * simulated registers live in LDS, structure-of-arrays [slot][thread], so a
//     register read or write is one conflict-free ds_read/ds_write of 64 lanes;
//   * per-warp control state (stack top, masks, cycle counters) is scalar; the
//     divergence stack, the scoreboard and the counters live in VGPR lanes and
//     are accessed with v_readlane / v_writelane;
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

// Per-warp control state, wave-uniform (SGPRs).
struct Half {
  uint32_t pc, mask, rpc, sp;  // top of the divergence stack and its depth
  uint32_t exited, init_mask;
  uint32_t next;               // previous issue cycle + 1
  uint32_t bar_ready, arrival;
  uint32_t state, status, warp_instrs, max_depth;
  uint64_t thread_instrs;
};

typedef const __attribute__((address_space(4))) uint32_t* cu32p;

__device__ __forceinline__ uint32_t rl(uint32_t v, uint32_t l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, (int)l);
}
// Write the wave-uniform `val` into lane `l` of `old`.
__device__ __forceinline__ uint32_t wl(uint32_t old, uint32_t val, uint32_t l) {
  return __lane_id() == l ? val : old;
}
__device__ __forceinline__ uint64_t rl64(uint64_t v, uint32_t l) {
  return (uint64_t)rl((uint32_t)v, l) | ((uint64_t)rl((uint32_t)(v >> 32), l) << 32);
}
__device__ __forceinline__ uint64_t ballot(bool c) { return __builtin_amdgcn_ballot_w64(c); }
__device__ __forceinline__ uint32_t uni(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }

__device__ __forceinline__ void hs_pop(Half& H, uint32_t spc, uint32_t sm, uint32_t sr) {
  H.sp -= 1;
  if (H.sp) {
    H.pc = rl(spc, H.sp - 1);
    H.mask = rl(sm, H.sp - 1);
    H.rpc = rl(sr, H.sp - 1);
  }
}

__device__ __forceinline__ void hs_push(Half& H, uint32_t& spc, uint32_t& sm, uint32_t& sr, uint32_t pc, uint32_t mask,
                                        uint32_t rpc) {
  spc = wl(spc, H.pc, H.sp - 1);
  sm = wl(sm, H.mask, H.sp - 1);
  sr = wl(sr, H.rpc, H.sp - 1);
  H.pc = pc;
  H.mask = mask;
  H.rpc = rpc;
  H.sp += 1;
  H.max_depth = H.sp > H.max_depth ? H.sp : H.max_depth;
}

// Pop finished or reconverged entries; lanes that ran off the end exit at no cost.
__device__ __forceinline__ void hs_resolve(Half& H, uint32_t spc, uint32_t sm, uint32_t sr, uint32_t n, uint32_t budget) {
  if (H.state != H_RUN) return;
  while (H.sp) {
    uint32_t m = H.mask & ~H.exited;
    if (m == 0 || H.pc == H.rpc) {
      hs_pop(H, spc, sm, sr);
      continue;
    }
    if (H.pc >= n) {
      H.exited |= m;
      continue;
    }
    break;
  }
  if (!H.sp) {
    H.state = H_DONE;
    H.status |= KS_ST_FINISHED;
    return;
  }
  if (H.warp_instrs >= budget) {
    H.state = H_DONE;
    H.status |= KS_ST_BUDGET;
  }
}

__device__ __forceinline__ uint32_t sb_get(uint32_t lo, uint32_t hi, uint32_t j) {
  return j < 64 ? rl(lo, j) : rl(hi, j - 64);
}
__device__ __forceinline__ void sb_set(uint32_t& lo, uint32_t& hi, uint32_t j, uint32_t v) {
  if (j < 64) lo = wl(lo, v, j);
  else hi = wl(hi, v, j - 64);
}

// Issue cycle: the later of previous issue + 1, the barrier release and the ready
// cycle of every register source (sb holds four scoreboard indices, 0xFF = none).
__device__ __forceinline__ uint32_t issue_cycle(const Half& H, uint32_t lo, uint32_t hi, uint32_t sb) {
  uint32_t t = H.next > H.bar_ready ? H.next : H.bar_ready;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t j = (sb >> (8 * k)) & 0xFF;
    if (j != 0xFF) {
      uint32_t r = sb_get(lo, hi, j);
      t = r > t ? r : t;
    }
  }
  return t;
}

__device__ __forceinline__ uint32_t cnt_add(uint32_t cnt, uint32_t lane, uint32_t idx, uint32_t v) {
  return cnt + (lane == idx ? v : 0u);
}
__device__ __forceinline__ uint32_t cnt_max(uint32_t cnt, uint32_t lane, uint32_t idx, uint32_t v) {
  return (lane == idx && v > cnt) ? v : cnt;
}

// Number of distinct values in {k1[l], k2[l] : l in lanes}.  Full exec required.
__device__ uint32_t distinct2(uint64_t k1, uint64_t k2, uint64_t lanes) {
  uint64_t rem1 = lanes;
  uint64_t rem2 = lanes & ballot(k2 != k1);
  uint32_t n = 0;
  while (rem1 | rem2) {
    uint64_t key = rem1 ? rl64(k1, (uint32_t)__builtin_ctzll(rem1)) : rl64(k2, (uint32_t)__builtin_ctzll(rem2));
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

}  // namespace

__global__ void __launch_bounds__(1024) ks_interp_kernel(const KsArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ uint32_t ep_max[3], ep_alive[3];

  const uint32_t WG = blockDim.x;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = tid >> 6;
  const uint32_t hl = lane >> 5;
  const uint32_t sl = lane & 31u;
  const uint32_t blk = blockIdx.x;
  const uint32_t W = a.warps_per_block;
  const uint32_t T = a.threads_per_block;
  const uint32_t n_instr = a.n_instrs;

  uint32_t* rf = lds;                                          // [slot][WG]
  uint8_t* win = reinterpret_cast<uint8_t*>(lds + a.rf_slots * WG);  // simulated shared window

  {  // zero the register file and the shared window
    const uint32_t words = a.rf_slots * WG + ((a.shared_bytes + 3u) >> 2);
    for (uint32_t i = tid; i < words; i += WG) lds[i] = 0;
    if (tid < 3) {
      ep_max[tid] = 0;
      ep_alive[tid] = 0;
    }
  }
  __syncthreads();

  // special registers of this lane's simulated thread
  const uint32_t t_lin = (2u * wave + hl) * 32u + sl;
  const uint32_t bx = a.block[0], by = a.block[1];
  const uint32_t tid_x = t_lin % bx, tid_y = (t_lin / bx) % by, tid_z = t_lin / (bx * by);
  const uint32_t gx = a.grid[0], gy = a.grid[1];
  const uint32_t cta_x = blk % gx, cta_y = (blk / gx) % gy, cta_z = blk / (gx * gy);

  Half H0, H1;
  {
    Half* hs[2] = {&H0, &H1};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      Half& H = *hs[hh];
      const uint32_t w = 2u * wave + (uint32_t)hh;
      const bool exists = w < W;
      const uint32_t live = T > w * 32u ? (T - w * 32u > 32u ? 32u : T - w * 32u) : 0u;
      H.init_mask = live >= 32u ? 0xFFFFFFFFu : ((1u << live) - 1u);
      H.pc = 0;
      H.mask = H.init_mask;
      H.rpc = RPC_EXIT;
      H.sp = exists ? 1u : 0u;
      H.exited = 0;
      H.next = 0;
      H.bar_ready = 0;
      H.arrival = 0;
      H.state = exists ? H_RUN : H_DONE;
      H.status = 0;
      H.warp_instrs = 0;
      H.max_depth = 1;
      H.thread_instrs = 0;
    }
  }
  uint32_t stk_pc0 = 0, stk_m0 = 0, stk_r0 = 0, stk_pc1 = 0, stk_m1 = 0, stk_r1 = 0;
  uint32_t sb_lo0 = 0, sb_hi0 = 0, sb_lo1 = 0, sb_hi1 = 0;
  uint32_t cnt = 0;    // counter d of half h in lane 32 h + d
  uint32_t pbits = 0;  // predicate p of this lane's thread in bit p

  const uint32_t cap = a.trace_cap;
  const uint64_t gw0 = (uint64_t)blk * W + 2u * wave;  // global warp id of half 0

  uint32_t epoch = 0;
  while (true) {
    // ------------------------------------------------------------------ run both warps until blocked
    while (true) {
      hs_resolve(H0, stk_pc0, stk_m0, stk_r0, n_instr, a.max_warp_instrs);
      hs_resolve(H1, stk_pc1, stk_m1, stk_r1, n_instr, a.max_warp_instrs);
      const bool r0 = H0.state == H_RUN, r1 = H1.state == H_RUN;
      if (!r0 && !r1) break;
      const uint32_t pc = (r0 && r1) ? (H0.pc < H1.pc ? H0.pc : H1.pc) : (r0 ? H0.pc : H1.pc);
      bool go0 = r0 && H0.pc == pc, go1 = r1 && H1.pc == pc;

      const cu32p I = (cu32p)(uintptr_t)(a.prog + pc);
      const uint32_t w0 = I[0], w1 = I[1], wsb = I[2], w3 = I[3], w4 = I[4], w5 = I[5];
      const uint32_t op = w0 & 0xFFu, flags = (w0 >> 8) & 0xFFu, dst = (w0 >> 16) & 0xFFu, guard = w0 >> 24;
      const uint32_t kinds = w1 >> 24;
      const uint32_t sb_dst = w3 & 0xFFu, cmp = (w3 >> 8) & 0xFFu, lat = w3 >> 16;
      const uint32_t target = w4 & 0xFFFFu, rpc_raw = w4 >> 16;
      const uint32_t rpc = rpc_raw == KS_RPC_EXIT ? RPC_EXIT : rpc_raw;

      uint32_t iss0 = 0, iss1 = 0;
      if (go0) {
        iss0 = issue_cycle(H0, sb_lo0, sb_hi0, wsb);
        if (iss0 > CYCLE_LIMIT) {
          H0.state = H_DONE;
          H0.status |= KS_ST_CYCLE_OVF;
          go0 = false;
        }
      }
      if (go1) {
        iss1 = issue_cycle(H1, sb_lo1, sb_hi1, wsb);
        if (iss1 > CYCLE_LIMIT) {
          H1.state = H_DONE;
          H1.status |= KS_ST_CYCLE_OVF;
          go1 = false;
        }
      }
      if (!go0 && !go1) continue;
      const uint32_t m0 = go0 ? (H0.mask & ~H0.exited) : 0u;
      const uint32_t m1 = go1 ? (H1.mask & ~H1.exited) : 0u;

      // trace records, one lane per warp
      {
        const bool rec0 = go0 && H0.warp_instrs < cap, rec1 = go1 && H1.warp_instrs < cap;
        if ((lane == 0 && rec0) || (lane == 32 && rec1)) {
          const uint32_t wi = hl ? H1.warp_instrs : H0.warp_instrs;
          const uint32_t cyc = hl ? iss1 : iss0;
          uint8_t* p = a.trace + (gw0 + hl) * a.slot_bytes + 16u + 8ull * wi;
          *reinterpret_cast<uint2*>(p) = make_uint2(cyc, pc);
        }
      }
      if (go0) {
        H0.warp_instrs += 1;
        H0.thread_instrs += (uint32_t)__builtin_popcount(m0);
        H0.next = iss0 + 1;
      }
      if (go1) {
        H1.warp_instrs += 1;
        H1.thread_instrs += (uint32_t)__builtin_popcount(m1);
        H1.next = iss1 + 1;
      }

      // guard
      const uint64_t m64 = (uint64_t)m0 | ((uint64_t)m1 << 32);
      const bool act = (m64 >> lane) & 1u;
      bool pass = true;
      if (flags & KF_GUARD) pass = (((pbits >> guard) & 1u) != 0) != ((flags & KF_GUARD_NEG) != 0);
      const bool on = act && pass;
      const uint64_t g64 = ballot(on);
      const uint32_t g0 = (uint32_t)g64, g1 = (uint32_t)(g64 >> 32);

      // ---------------------------------------------------------------- execute
      if (op < KO_LDP32) {
        if (on) {
          const uint32_t s0 = w1 & 0xFFu, s1 = (w1 >> 8) & 0xFFu, s2 = (w1 >> 16) & 0xFFu;
          const uint32_t k0 = kinds & 3u, k1 = (kinds >> 2) & 3u, k2 = (kinds >> 4) & 3u;
          auto special = [&](uint32_t id) -> uint32_t {
            switch (id) {
              case KSP_TID_X: return tid_x;
              case KSP_TID_Y: return tid_y;
              case KSP_TID_Z: return tid_z;
              case KSP_NTID_X: return a.block[0];
              case KSP_NTID_Y: return a.block[1];
              case KSP_NTID_Z: return a.block[2];
              case KSP_CTAID_X: return cta_x;
              case KSP_CTAID_Y: return cta_y;
              case KSP_CTAID_Z: return cta_z;
              case KSP_NCTAID_X: return a.grid[0];
              case KSP_NCTAID_Y: return a.grid[1];
              case KSP_NCTAID_Z: return a.grid[2];
              default: return sl;
            }
          };
          auto rd32 = [&](uint32_t kind, uint32_t s, uint32_t imm) -> uint32_t {
            if (kind == KK_REG) return rf[s * WG + tid];
            if (kind == KK_IMM) return imm;
            return special(s);
          };
          auto rd64 = [&](uint32_t kind, uint32_t s, uint32_t imm_lo, uint32_t imm_hi) -> uint64_t {
            if (kind == KK_REG) return (uint64_t)rf[s * WG + tid] | ((uint64_t)rf[(s + 1) * WG + tid] << 32);
            return (uint64_t)imm_lo | ((uint64_t)imm_hi << 32);
          };
          uint32_t rlo = 0, rhi = 0;
          bool wide = false, wr = true;
          switch (op) {
            case KO_ADD32: rlo = rd32(k0, s0, I[6]) + rd32(k1, s1, I[8]); break;
            case KO_SUB32: rlo = rd32(k0, s0, I[6]) - rd32(k1, s1, I[8]); break;
            case KO_MUL32: rlo = rd32(k0, s0, I[6]) * rd32(k1, s1, I[8]); break;
            case KO_MAD32: rlo = rd32(k0, s0, I[6]) * rd32(k1, s1, I[8]) + rd32(k2, s2, I[10]); break;
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
              const int64_t r = (int64_t)(int32_t)rd32(k0, s0, I[6]) * (int64_t)(int32_t)rd32(k1, s1, I[8]);
              rlo = (uint32_t)r;
              rhi = (uint32_t)((uint64_t)r >> 32);
              wide = true;
              break;
            }
            case KO_MULWIDE_U: {
              const uint64_t r = (uint64_t)rd32(k0, s0, I[6]) * (uint64_t)rd32(k1, s1, I[8]);
              rlo = (uint32_t)r;
              rhi = (uint32_t)(r >> 32);
              wide = true;
              break;
            }
            case KO_FADD:
              rlo = canon_bits(__uint_as_float(rd32(k0, s0, I[6])) + __uint_as_float(rd32(k1, s1, I[8])));
              break;
            case KO_FSUB:
              rlo = canon_bits(__uint_as_float(rd32(k0, s0, I[6])) - __uint_as_float(rd32(k1, s1, I[8])));
              break;
            case KO_FMUL:
              rlo = canon_bits(__uint_as_float(rd32(k0, s0, I[6])) * __uint_as_float(rd32(k1, s1, I[8])));
              break;
            case KO_FFMA:
              rlo = canon_bits(__builtin_fmaf(__uint_as_float(rd32(k0, s0, I[6])), __uint_as_float(rd32(k1, s1, I[8])),
                                              __uint_as_float(rd32(k2, s2, I[10]))));
              break;
            case KO_SETP_S32:
            case KO_SETP_U32:
            case KO_SETP_S64:
            case KO_SETP_U64:
            case KO_SETP_F32: {
              bool c;
              if (op == KO_SETP_F32) {
                const float x = __uint_as_float(rd32(k0, s0, I[6])), y = __uint_as_float(rd32(k1, s1, I[8]));
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
                const uint32_t x = rd32(k0, s0, I[6]), y = rd32(k1, s1, I[8]);
                const bool sg = op == KO_SETP_S32;
                const bool lt = sg ? (int32_t)x < (int32_t)y : x < y;
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
                const bool sg = op == KO_SETP_S64;
                const bool lt = sg ? (int64_t)x < (int64_t)y : x < y;
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
                rlo = p ? rd32(k0, s0, I[6]) : rd32(k1, s1, I[8]);
              } else {
                const uint64_t r = p ? rd64(k0, s0, I[6], I[7]) : rd64(k1, s1, I[8], I[9]);
                rlo = (uint32_t)r;
                rhi = (uint32_t)(r >> 32);
                wide = true;
              }
              break;
            }
            case KO_MOV32: rlo = rd32(k0, s0, I[6]); break;
            default: {  // KO_MOV64
              const uint64_t r = rd64(k0, s0, I[6], I[7]);
              rlo = (uint32_t)r;
              rhi = (uint32_t)(r >> 32);
              wide = true;
              break;
            }
          }
          if (wr) {
            rf[dst * WG + tid] = rlo;
            if (wide) rf[(dst + 1) * WG + tid] = rhi;
          }
        }
      } else if (op <= KO_LDP64) {
        // parameter load: uniform value from the launch arguments
        const uint32_t aux = w5 & 0xFFFFu;
        const uint32_t lo = *reinterpret_cast<const uint32_t*>(a.params + aux);
        const uint32_t hi = op == KO_LDP64 ? *reinterpret_cast<const uint32_t*>(a.params + aux + 4) : 0u;
        if (on) {
          rf[dst * WG + tid] = lo;
          if (op == KO_LDP64) rf[(dst + 1) * WG + tid] = hi;
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
          uint64_t base = rf[s0 * WG + tid];
          if (addr_w == 64u) base |= (uint64_t)rf[(s0 + 1) * WG + tid] << 32;
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
            rf[dst * WG + tid] = lo;
            if (w64) rf[(dst + 1) * WG + tid] = hi;
          } else if (ok) {
            const uint32_t lo = rf[s1 * WG + tid];
            if (is_global) {
              if (w64) {
                *reinterpret_cast<uint2*>(a.gmem + A) = make_uint2(lo, rf[(s1 + 1) * WG + tid]);
              } else {
                *reinterpret_cast<uint32_t*>(a.gmem + A) = lo;
              }
            } else {
              *reinterpret_cast<uint32_t*>(win + A) = lo;
              if (w64) *reinterpret_cast<uint32_t*>(win + A + 4) = rf[(s1 + 1) * WG + tid];
            }
          }
        }
        // analysis and fault counting (full exec)
        const uint64_t faults = ballot(on && !ok);
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
        if (is_global) {
          const uint64_t last = A + (S - 1u);
          const uint32_t cn = is_load ? C_GLD_N : C_GST_N;
          if (g0) {
            const uint32_t sec = distinct2(A >> 5, last >> 5, (uint64_t)g0);
            const uint32_t lin = distinct2(A >> 7, last >> 7, (uint64_t)g0);
            cnt = cnt_add(cnt, lane, cn, 1);
            cnt = cnt_add(cnt, lane, cn + 1, sec);
            cnt = cnt_add(cnt, lane, cn + 2, lin);
          }
          if (g1) {
            const uint32_t sec = distinct2(A >> 5, last >> 5, (uint64_t)g1 << 32);
            const uint32_t lin = distinct2(A >> 7, last >> 7, (uint64_t)g1 << 32);
            cnt = cnt_add(cnt, lane, 32 + cn, 1);
            cnt = cnt_add(cnt, lane, 32 + cn + 1, sec);
            cnt = cnt_add(cnt, lane, 32 + cn + 2, lin);
          }
        } else {
          if (g0) {
            const uint32_t d = bank_degree(A, (uint64_t)g0);
            cnt = cnt_add(cnt, lane, C_SH_N, 1);
            cnt = cnt_add(cnt, lane, C_SH_SUM, d);
            cnt = cnt_max(cnt, lane, C_SH_MAX, d);
          }
          if (g1) {
            const uint32_t d = bank_degree(A, (uint64_t)g1 << 32);
            cnt = cnt_add(cnt, lane, 32 + C_SH_N, 1);
            cnt = cnt_add(cnt, lane, 32 + C_SH_SUM, d);
            cnt = cnt_max(cnt, lane, 32 + C_SH_MAX, d);
          }
        }
      }

      // ---------------------------------------------------------------- scoreboard and control
      if (sb_dst != 0xFFu) {
        if (go0) sb_set(sb_lo0, sb_hi0, sb_dst, iss0 + lat);
        if (go1) sb_set(sb_lo1, sb_hi1, sb_dst, iss1 + lat);
      }
      if (op == KO_BRA) {
        if (go0) {
          const uint32_t nt = m0 & ~g0;
          if (nt == 0) {
            H0.pc = target;
          } else if (g0 == 0) {
            H0.pc = pc + 1;
          } else {
            H0.pc = rpc;
            cnt = cnt_add(cnt, lane, C_DIV, 1);
            if (target != rpc) hs_push(H0, stk_pc0, stk_m0, stk_r0, target, g0, rpc);
            if (pc + 1 != rpc) hs_push(H0, stk_pc0, stk_m0, stk_r0, pc + 1, nt, rpc);
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
            if (target != rpc) hs_push(H1, stk_pc1, stk_m1, stk_r1, target, g1, rpc);
            if (pc + 1 != rpc) hs_push(H1, stk_pc1, stk_m1, stk_r1, pc + 1, nt, rpc);
          }
        }
      } else if (op == KO_RET) {
        if (go0) {
          H0.exited |= g0;
          H0.pc = pc + 1;
        }
        if (go1) {
          H1.exited |= g1;
          H1.pc = pc + 1;
        }
      } else if (op == KO_BAR) {
        if (go0) {
          cnt = cnt_add(cnt, lane, C_BAR, 1);
          if (m0 != (H0.init_mask & ~H0.exited)) H0.status |= KS_ST_BARDIV;
          H0.state = H_WAIT;
          H0.arrival = iss0;
          H0.pc = pc + 1;
        }
        if (go1) {
          cnt = cnt_add(cnt, lane, 32 + C_BAR, 1);
          if (m1 != (H1.init_mask & ~H1.exited)) H1.status |= KS_ST_BARDIV;
          H1.state = H_WAIT;
          H1.arrival = iss1;
          H1.pc = pc + 1;
        }
      } else {
        if (go0) H0.pc = pc + 1;
        if (go1) H1.pc = pc + 1;
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
    const uint32_t release = uni(ep_max[slot]) + a.lat_bar;
    if (H0.state == H_WAIT) {
      H0.state = H_RUN;
      H0.bar_ready = release;
    }
    if (H1.state == H_WAIT) {
      H1.state = H_RUN;
      H1.bar_ready = release;
    }
    ++epoch;
  }

  // -------------------------------------------------------------------- counters and trace headers
  {
    const Half& M = hl ? H1 : H0;
    const uint32_t w = 2u * wave + hl;
    if (w < W) {
      const uint32_t cycles = M.next;
      const uint32_t written = M.warp_instrs < cap ? M.warp_instrs : cap;
      const uint32_t dropped = M.warp_instrs - written;
      const uint32_t status = M.status | (dropped ? KS_ST_TRACE_DROP : 0u);
      const uint64_t gw = gw0 + hl;
      if (sl < 20) {
        uint32_t v;
        switch (sl) {
          case C_TI_LO: v = (uint32_t)M.thread_instrs; break;
          case C_TI_HI: v = (uint32_t)(M.thread_instrs >> 32); break;
          case C_STATUS: v = status; break;
          case C_CYCLES: v = cycles; break;
          case C_WARP_INSTRS: v = M.warp_instrs; break;
          case C_STALL: v = cycles - M.warp_instrs; break;
          case C_MAXDEPTH: v = M.max_depth; break;
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

__global__ void ks_zero_word(uint32_t* out) { *out = 0; }

__global__ void ks_status_or_kernel(const uint8_t* counters, uint64_t n, uint32_t* out) {
  uint32_t acc = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    acc |= reinterpret_cast<const uint32_t*>(counters + i * 80u)[C_STATUS];
  // wave-level OR, then one atomic per wave
  for (int o = 32; o > 0; o >>= 1) acc |= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63u) == 0 && acc) atomicOr(out, acc);
}

size_t ks_lds_limit() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 65536;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 65536;
  return (size_t)v;
}

hipError_t ks_launch_interp(const KsArgs& a, uint32_t n_blocks, uint32_t slots, hipStream_t s) {
  (void)slots;
  const uint32_t waves = (a.warps_per_block + 1u) / 2u;
  const uint32_t wg = 64u * waves;
  const size_t lds = (size_t)a.rf_slots * wg * 4u + (((size_t)a.shared_bytes + 15u) & ~(size_t)15u);
  if (lds + 64 > ks_lds_limit()) return hipErrorInvalidValue;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)ks_interp_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(ks_lds_limit() - 64));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(ks_interp_kernel, dim3(n_blocks), dim3(wg), lds, s, a);
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
