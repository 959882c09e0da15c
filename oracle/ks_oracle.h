/*
 * ks_oracle.h -- C interface of the CPU oracle for the PTX-subset SIMT simulator.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, plainly written reference
 * that the GPU simulator is checked against.  Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load it.  The product path never
 * links, imports or calls it.  It shares no source with the GPU path: it has its
 * own parser, its own post-dominator computation and its own copy of the output
 * layouts, all written from the written specification of the method.
 *
 * Output layouts (little-endian, identical in meaning to the GPU path's):
 *   per-warp counters: 80 bytes, see struct oracle_counters below;
 *   per-warp trace slot: 16-byte header {u32 records_written, u8 version,
 *   u8 flags, u16 warp_in_block, u64 records_dropped} followed by trace_cap
 *   records.  Version 1: 8-byte records {u32 issue_cycle, u32 pc}.  Version 2
 *   (ORACLE_FLAG_EXT_TRACE): 16-byte records {u32 issue_cycle, u16 pc, u8 kind,
 *   u8 0, u32 active lanes, u32 payload}, kinds and payloads as listed at
 *   ORACLE_EV_* below.  The slot shape (a fixed header, then fixed-size records,
 *   one slot per warp, overflow counted rather than dropped silently; events of
 *   4/8 bytes without a payload and 16 bytes with one) follows the per-warp buffer
 *   described in "CuTeDSL IKET 浅析" (zhen8838.github.io/posts/iket.html),
 *   section 2, "buffer 是怎么定形的".
 */
#ifndef KS_ORACLE_H
#define KS_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_NLAT 18

/* Latency classes: index into oracle_cfg.latency[]. */
enum {
  ORACLE_LAT_INT32 = 0, ORACLE_LAT_INT64 = 1, ORACLE_LAT_FP32 = 2, ORACLE_LAT_SETP = 3,
  ORACLE_LAT_SELP = 4, ORACLE_LAT_MOV = 5, ORACLE_LAT_LD_PARAM = 6, ORACLE_LAT_LD_GLOBAL = 7,
  ORACLE_LAT_LD_SHARED = 8, ORACLE_LAT_ST_GLOBAL = 9, ORACLE_LAT_ST_SHARED = 10,
  ORACLE_LAT_BRA = 11, ORACLE_LAT_BAR = 12, ORACLE_LAT_RET = 13,
  /* ld.global under ORACLE_FLAG_CACHE: L1 hit, L2 hit, miss in both */
  ORACLE_LAT_L1_HIT = 14, ORACLE_LAT_L2_HIT = 15, ORACLE_LAT_DRAM = 16
};

/* Per-warp status bits. */
#define ORACLE_ST_FINISHED  0x01u
#define ORACLE_ST_BUDGET    0x02u
#define ORACLE_ST_FAULT     0x04u
#define ORACLE_ST_TRACE_DROP 0x08u
#define ORACLE_ST_BARDIV    0x10u
#define ORACLE_ST_CYCLE_OVF 0x20u

/* Return codes. */
#define ORACLE_OK 0
#define ORACLE_E_PARSE (-1)
#define ORACLE_E_UNSUPPORTED (-2)
#define ORACLE_E_INVALID_ARG (-3)
#define ORACLE_E_RACE (-7)

#define ORACLE_FLAG_CHECK_RACES 0x1u
#define ORACLE_FLAG_EXT_TRACE 0x2u   /* 16-byte trace records (version 2) */
#define ORACLE_FLAG_CACHE 0x4u       /* cache-latency model: per-warp L1 and L2 */

/* Cache-latency model (KernelScope simulator page, memory-analysis part: the cache
 * parameters and the direct-mapped SimpleCache).  Each warp owns an L1 of 1024 and
 * an L2 of 49152 direct-mapped 128-byte lines, both empty at the start of a run.
 * A global warp access with at least one valid guard lane looks up the line of its
 * lowest such lane: the L1 first, on a miss the L2; a miss installs the line.  A
 * load's destination is then ready after the L1-hit, L2-hit or DRAM latency; a
 * load with no valid guard lane takes the ld.global latency and touches no cache.
 * Output, per warp, ORACLE_CACHE_WARP_BYTES: {u32 l1_hits, u32 l2_hits, u32
 * misses, u32 0}, then the L1 and the L2 tags as u32 (line number + 1, 0 = empty). */
#define ORACLE_CACHE_L1_LINES 1024u
#define ORACLE_CACHE_L2_LINES 49152u
#define ORACLE_CACHE_WARP_BYTES (16u + 4u * (ORACLE_CACHE_L1_LINES + ORACLE_CACHE_L2_LINES))

/* Record kinds of the 16-byte trace records, and their payloads:
 *   LD/ST_GLOBAL: sectors | lines << 8 | guard lanes << 16 | faulting lanes << 24
 *                 (counts; all 0 when no lane passes the guard);
 *   LD/ST_SHARED: bank-conflict degree (0 when no lane passes) | guard lanes << 16 |
 *                 faulting lanes << 24;
 *   BRANCH, DIVERGE (the warp split): mask of the lanes taking the branch;
 *   BARRIER: 0;  OTHER, RET: mask of the lanes passing the guard. */
enum {
  ORACLE_EV_OTHER = 0, ORACLE_EV_LD_GLOBAL = 1, ORACLE_EV_ST_GLOBAL = 2, ORACLE_EV_LD_SHARED = 3,
  ORACLE_EV_ST_SHARED = 4, ORACLE_EV_BRANCH = 5, ORACLE_EV_DIVERGE = 6, ORACLE_EV_BARRIER = 7, ORACLE_EV_RET = 8
};

typedef struct {
  uint64_t thread_instrs;   /* sum over issued warp-instructions of popcount(active mask) */
  uint32_t status;          /* ORACLE_ST_* bits */
  uint32_t cycles;          /* last issue cycle + 1 (0 if nothing issued) */
  uint32_t warp_instrs;     /* issued warp-instructions */
  uint32_t stall_cycles;    /* cycles - warp_instrs */
  uint32_t gld_n, gld_sectors, gld_lines;
  uint32_t gst_n, gst_sectors, gst_lines;
  uint32_t sh_n, sh_degree_sum, sh_degree_max;
  uint32_t diverge_n, barrier_n, fault_n;
  uint32_t max_stack_depth; /* deepest divergence stack seen */
  uint32_t reserved;
} oracle_counters;          /* 80 bytes */

typedef struct {
  uint32_t grid[3];
  uint32_t block[3];
  uint64_t gmem_bytes;
  uint32_t trace_cap;        /* records per warp slot */
  uint32_t max_warp_instrs;  /* per-warp issue budget */
  uint16_t latency[ORACLE_NLAT];
  uint32_t n_threads;        /* CPU worker threads; 0 = all hardware threads */
  uint32_t flags;            /* ORACLE_FLAG_* */
  const uint32_t* block_list; /* optional: linear ids of the blocks to simulate */
  uint64_t n_block_list;      /* 0 = simulate every block of the grid */
  uint8_t* cache;             /* ORACLE_FLAG_CACHE: n_out_warps * ORACLE_CACHE_WARP_BYTES out */
} oracle_cfg;

typedef struct {
  uint32_t n_instrs;
  uint32_t n_params;
  uint32_t param_bytes;
  uint32_t shared_bytes;
  uint32_t reg_words;    /* 32-bit words of declared registers (64-bit ones count 2) */
  uint32_t n_preds;
} oracle_info;

/* Parse `ptx` (NUL-free, `len` bytes) and report its shape.  entry == NULL or ""
 * selects the first .entry.  Returns ORACLE_OK or an error code; `err` receives a
 * message ("line N: ..." for parse errors). */
int oracle_program_info(const char* ptx, size_t len, const char* entry, oracle_info* out,
                        char* err, size_t err_len);

/* Byte offset and size of parameter number `index` (declaration order). */
int oracle_param(const char* ptx, size_t len, const char* entry, uint32_t index,
                 uint32_t* offset, uint32_t* size, char* name, size_t name_len,
                 char* err, size_t err_len);

/* Default latency table (sm_80 model of the KernelScope latency page). */
void oracle_default_latency(uint16_t out[ORACLE_NLAT]);

/* Simulate.  `gmem` (gmem_bytes) is read and updated in place.  `counters` receives
 * n_out_warps * 80 bytes and `trace` n_out_warps * (16 + R * trace_cap) bytes (R = 8, or 16
 * with ORACLE_FLAG_EXT_TRACE), where
 * n_out_warps = (n_block_list ? n_block_list : total blocks) * warps_per_block, in
 * block-list (or linear block) order.  Returns ORACLE_OK, an error code, or
 * ORACLE_E_RACE when race checking is on and a race was seen (outputs still written). */
int oracle_run(const char* ptx, size_t len, const char* entry, const oracle_cfg* cfg,
               const void* params, size_t params_len, uint8_t* gmem,
               uint8_t* counters, uint8_t* trace, char* err, size_t err_len);

/* Debug: the reconvergence index the oracle computes for the instruction at `pc`
 * (n_instrs means "exit"; 0xFFFFFFFF when pc is not a conditional branch). */
int oracle_ipdom_table(const char* ptx, size_t len, const char* entry, uint32_t* out,
                       uint32_t out_len, char* err, size_t err_len);

#ifdef __cplusplus
}
#endif
#endif
