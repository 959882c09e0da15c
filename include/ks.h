/*
 * ks.h -- C ABI of libkscope, a PTX-subset SIMT simulator that runs on one
 * AMD Instinct MI355X (gfx950).
 *
 * The library simulates NVIDIA-style 32-thread warps executing a small PTX
 * subset.  It models three things:
 *   - per-warp active masks and a divergence stack that reconverges at immediate
 *     post-dominators computed on the host;
 *   - a register-scoreboard cycle model with a per-opcode latency table;
 *   - a memory analyser (32-byte sectors and 128-byte lines per global warp
 *     access, the bank-conflict degree over 32 four-byte banks per shared warp
 *     access).
 * It also writes a per-warp trace: {issue cycle, pc} records, or (extended
 * format) 16-byte records that add the instruction kind, the active mask and a
 * per-kind payload (sectors and lines of a global access, bank-conflict degree of
 * a shared access, the lanes taking a branch).  Extended records support blocks
 * of up to KS_EXT_MAX_BLOCK_THREADS threads (KS_EXT64_MAX_BLOCK_THREADS for
 * programs of more than 32 register slots), and ks_run covers an extended-record
 * grid with launches of at most KS_EXT_MAX_BLOCKS blocks each.
 *
 * Sources of the semantics, by page and section:
 *   - KernelScope backend documentation (github.com/briefgaming/kernelscope).
 *     The PTX-parser part gives the grammar.  The execution-simulator part gives
 *     warps, the active mask and the SIMT stack of (pc, mask, reconvergence pc).
 *     The memory-analysis part gives banks, broadcast, lines and sectors.  The
 *     latency-model part gives the sm_80 latencies.
 *   - "CuTeDSL IKET 浅析" (zhen8838.github.io/posts/iket.html), section 2
 *     ("buffer 是怎么定形的"): the trace slot shape.
 *   - The SASS-probe method page (teach-meaning.tistory.com/1954), sections 2
 *     and 14: the dependent versus independent FMA contrast that the scoreboard
 *     model reproduces.
 *
 * Conventions
 *   - Every entry point returns ks_status: 0 (KS_OK) or a negative error code.
 *     No C++ exception crosses the ABI.
 *   - ks_last_error() returns the message of the last failing call on this
 *     thread.  It is valid until the next call on the same thread.
 *   - Host pointers are plain CPU memory.  Device pointers ("d_") are HIP device
 *     allocations, owned by the caller.
 *   - The library owns only what it creates: program and state descriptors, and
 *     a small device copy of the decoded program (freed by ks_state_free).
 *   - `stream` is a hipStream_t (NULL = the default stream).  ks_run and
 *     ks_read_* are ordered on that stream; ks_read_* wait for their copy.
 *   - All multi-byte data are little-endian.
 *   - The library computes every result on the GPU.  There is no CPU fallback:
 *     if no gfx950 device is usable, ks_alloc_state fails with KS_E_HIP.
 */
#ifndef KS_H
#define KS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ks_status;
#define KS_OK 0
#define KS_E_PARSE (-1)        /* malformed PTX; message "line N: ..." */
#define KS_E_UNSUPPORTED (-2)  /* valid PTX outside the subset, or beyond a size limit */
#define KS_E_INVALID_ARG (-3)  /* bad pointer, size, shape or configuration */
#define KS_E_HIP (-4)          /* a HIP runtime call failed, or no gfx950 device */
#define KS_E_NOMEM (-5)        /* a host or device allocation failed */
#define KS_E_STATE (-6)        /* call out of order (for example a read before any run) */

/* Per-warp status bits (counter field `status`, OR-ed by ks_run_status). */
#define KS_ST_FINISHED 0x01u   /* every lane exited normally */
#define KS_ST_BUDGET 0x02u     /* stopped at max_warp_instrs */
#define KS_ST_FAULT 0x04u      /* at least one lane access out of range or misaligned */
#define KS_ST_TRACE_DROP 0x08u /* trace records past trace_cap were dropped (and counted) */
#define KS_ST_BARDIV 0x10u     /* bar.sync reached with a partial (divergent) mask */
#define KS_ST_CYCLE_OVF 0x20u  /* an issue cycle would exceed 2^31 - 1; warp stopped */

/* Latency classes, the indices of ks_config.latency[]. */
#define KS_NLAT 18
enum {
  KS_LAT_INT32 = 0, KS_LAT_INT64 = 1, KS_LAT_FP32 = 2, KS_LAT_SETP = 3, KS_LAT_SELP = 4,
  KS_LAT_MOV = 5, KS_LAT_LD_PARAM = 6, KS_LAT_LD_GLOBAL = 7, KS_LAT_LD_SHARED = 8,
  KS_LAT_ST_GLOBAL = 9, KS_LAT_ST_SHARED = 10, KS_LAT_BRA = 11, KS_LAT_BAR = 12, KS_LAT_RET = 13,
  /* ld.global under the cache-latency model: L1 hit, L2 hit, miss in both */
  KS_LAT_L1_HIT = 14, KS_LAT_L2_HIT = 15, KS_LAT_DRAM = 16
};

/* Cache-latency model (ks_config.cache_model), after the KernelScope simulator
 * page's memory-analysis part (its cache parameters and direct-mapped SimpleCache):
 *   KS_CACHE_NONE  ld.global takes latency[KS_LAT_LD_GLOBAL];
 *   KS_CACHE_WARP  each warp owns a direct-mapped L1 of KS_CACHE_L1_LINES and L2 of
 *                  KS_CACHE_L2_LINES 128-byte lines, empty at the start of every
 *                  run.  A global warp access with at least one valid guard lane
 *                  looks up the line of its lowest such lane in the L1, on a miss in
 *                  the L2, installing it where it missed; a load's destination is
 *                  then ready after latency[KS_LAT_L1_HIT], [KS_LAT_L2_HIT] or
 *                  [KS_LAT_DRAM].  A load with no valid guard lane touches no cache
 *                  and takes latency[KS_LAT_LD_GLOBAL].  The caches are private to
 *                  each warp so that the result does not depend on how the
 *                  simulated warps interleave (the page has one cache for all).
 * The state lives in a caller-owned buffer d_cache of KS_CACHE_WARP_BYTES per warp:
 * {u32 l1_hits, u32 l2_hits, u32 misses, u32 0}, the L1 tags, then the L2 tags, a
 * tag being the line number + 1 (0: empty set).  Runs with the cache model use the
 * basic trace format and at most 2^38 bytes of simulated memory. */
#define KS_CACHE_NONE 0u
#define KS_CACHE_WARP 1u
#define KS_CACHE_L1_LINES 1024u
#define KS_CACHE_L2_LINES 49152u
#define KS_CACHE_WARP_BYTES (16u + 4u * (KS_CACHE_L1_LINES + KS_CACHE_L2_LINES))

/* Trace record formats (ks_config.trace_format).  Both follow the IKET page's
 * per-warp slot: a 16-byte header {u32 records_written, u8 version, u8 flags,
 * u16 warp_in_block, u64 records_dropped}, then trace_cap fixed-size records;
 * the header's version byte names the format (1 or 2).
 *   KS_TRACE_BASIC     8-byte records {u32 issue_cycle, u32 pc}.
 *   KS_TRACE_EXTENDED  16-byte records {u32 issue_cycle, u16 pc, u8 kind,
 *                      u8 reserved (0), u32 active, u32 payload}: `active` is the
 *                      warp's live-lane mask at issue (bit l = lane l), `kind` a
 *                      KS_EV_* value, and `payload` depends on the kind:
 *     KS_EV_LD_GLOBAL / KS_EV_ST_GLOBAL: bits 0-7 distinct 32-byte sectors,
 *         bits 8-15 distinct 128-byte lines, bits 16-23 lanes passing the guard,
 *         bits 24-31 lanes whose access faulted (all 0 when no lane passes);
 *     KS_EV_LD_SHARED / KS_EV_ST_SHARED: bits 0-7 bank-conflict degree (0 when
 *         no lane passes), bits 16-23 lanes passing the guard, bits 24-31 faults;
 *     KS_EV_BRANCH / KS_EV_DIVERGE: the lanes taking the branch (DIVERGE when the
 *         warp split: some but not all live lanes take it);
 *     KS_EV_BARRIER: 0;
 *     KS_EV_OTHER / KS_EV_RET: the lanes passing the guard.
 *   Stall cycles are the gaps between consecutive records' issue cycles. */
#define KS_TRACE_BASIC 0u
#define KS_TRACE_EXTENDED 1u
enum {
  KS_EV_OTHER = 0, KS_EV_LD_GLOBAL = 1, KS_EV_ST_GLOBAL = 2, KS_EV_LD_SHARED = 3, KS_EV_ST_SHARED = 4,
  KS_EV_BRANCH = 5, KS_EV_DIVERGE = 6, KS_EV_BARRIER = 7, KS_EV_RET = 8
};

/* Limits of this build. */
#define KS_MAX_REG_SLOTS 64      /* 32-bit register slots per thread (a 64-bit register takes 2) */
#define KS_MAX_PREDS 32          /* predicate registers */
#define KS_MAX_INSTRS 65535      /* decoded instructions per program */
#define KS_MAX_PARAM_BYTES 512   /* parameter block */
#define KS_MAX_SHARED_BYTES 65536 /* simulated shared window per block */
#define KS_MAX_BLOCK_THREADS 1024
/* Blocks per launch of a KS_TRACE_EXTENDED run: ks_run covers a larger grid with
 * consecutive launches of this many blocks on the caller's stream (the last one
 * shorter), each of a size the extended-record interpreter has been checked at on
 * the GPU.  A single 65536-block extended launch faulted, with the cause not yet
 * found, and is never made.  Basic and cache-model runs are one launch. */
#define KS_EXT_MAX_BLOCKS 32
/* Largest block (threads) of a KS_TRACE_EXTENDED allocation or run: 1024, and 768
 * for programs of more than 32 register slots (their extended kernel's 136 VGPRs
 * leave room for three waves per SIMD).  Larger blocks are refused
 * (KS_E_UNSUPPORTED). */
#define KS_EXT_MAX_BLOCK_THREADS 1024
#define KS_EXT64_MAX_BLOCK_THREADS 768
/* Largest program (decoded instructions) a state bound by ks_alloc_state_static can
 * hold: the library's static device scratch is (KS_STATIC_MAX_INSTRS + 5) 128-byte
 * records plus 256 bytes, 1 MiB + 256 bytes per GPU. */
#define KS_STATIC_MAX_INSTRS 8187

typedef struct ks_program ks_program; /* opaque; created by ks_load_program */
typedef struct ks_state ks_state;     /* opaque; created by ks_alloc_state */
typedef struct { uint32_t x, y, z; } ks_dim3;

typedef struct {
  ks_dim3 max_grid;          /* largest grid ks_run will accept */
  ks_dim3 max_block;         /* largest block ks_run will accept (<= 1024 threads) */
  uint64_t gmem_bytes;       /* size of the simulated global memory d_gmem */
  uint32_t trace_cap;        /* trace records per warp slot; 0 = headers only */
  uint32_t max_warp_instrs;  /* per-warp issue budget; a warp reaching it stops with KS_ST_BUDGET */
  uint16_t latency[KS_NLAT]; /* cycles per latency class (ks_default_config fills sm_80 values) */
  uint32_t trace_format;     /* KS_TRACE_BASIC (default) or KS_TRACE_EXTENDED */
  uint32_t cache_model;      /* KS_CACHE_NONE (default) or KS_CACHE_WARP */
} ks_config;

typedef struct {
  uint32_t n_instrs;         /* decoded instructions */
  uint32_t n_params;
  uint32_t param_bytes;      /* size of the parameter block ks_run expects */
  uint32_t shared_bytes;     /* simulated shared window per block */
  uint32_t reg_slots;        /* 32-bit register slots per thread */
  uint32_t n_preds;          /* predicate registers */
} ks_program_desc;

typedef struct {
  uint32_t warps_per_block;  /* ceil(threads per block / 32) for max_block */
  uint32_t reserved;
  uint64_t n_warps;          /* warps of the largest grid: max blocks * warps_per_block */
  uint64_t counters_bytes;   /* n_warps * 80: size of d_counters */
  uint64_t slot_bytes;       /* 16 + 8 * trace_cap (basic) or 16 + 16 * trace_cap (extended): one slot */
  uint64_t trace_bytes;      /* n_warps * slot_bytes: size of d_trace */
  uint64_t cache_bytes;      /* n_warps * KS_CACHE_WARP_BYTES with the cache model, else 0: size of d_cache */
} ks_layout;

/* Parse a PTX module and decode the entry `entry` (NULL or "" = the first .entry).
 * `ptx` holds `len` bytes of text (not necessarily NUL-terminated; the library
 * keeps no pointer to it).  On success *out owns the decoded program, to be
 * released with ks_program_free.
 * Defined by: the KernelScope page's "ptx/parser.py, ptx/models.py" part (the
 * module, kernel, parameter and instruction grammar, predicate guards) and its
 * "simulator/engine.py" part, load_kernel (the first kernel is taken, directives
 * are dropped, and instructions are numbered in listing order: the pc).  Branch
 * reconvergence points are computed here too (the SIMT stack entry of that part
 * holds one); they are immediate post-dominators.
 * Text outside the grammar is an error, never skipped: parameters are separated
 * by commas; a label is an identifier without dots written against its ':';
 * "%r<N>", "@%p", "@!%p" and negative numbers take no inner spaces; an opcode is
 * followed by a space; .loc/.file/.section and the module header directives end
 * at the end of their line, comments removed.
 * Errors: KS_E_PARSE (message "line N: ..."), KS_E_UNSUPPORTED (an instruction,
 * type or directive outside the subset, or a size limit), KS_E_INVALID_ARG. */
ks_status ks_load_program(const char* ptx, size_t len, const char* entry, ks_program** out);

/* Shape of a decoded program: instruction count, parameter block, shared window,
 * register slots and predicates.  Writes *out; no ownership changes.
 * Defined by: the KernelScope page's "ptx/parser.py, ptx/models.py" part (a
 * parsed kernel's params, registers and instructions).  KS_E_INVALID_ARG for NULL. */
ks_status ks_program_info(const ks_program* prog, ks_program_desc* out);

/* Parameter `index` (declaration order): byte offset in the parameter block, size
 * in bytes, and its name (points into `prog`, valid while prog lives).  Parameters
 * are laid out in declaration order, each at its natural alignment (the pages give
 * no layout; this is the reading the oracle uses too).  Any output pointer may be
 * NULL.  Defined by: the KernelScope page's "ptx/parser.py, ptx/models.py" part
 * (the kernel's .param list).  KS_E_INVALID_ARG for an index out of range. */
ks_status ks_param_info(const ks_program* prog, uint32_t index, uint32_t* offset, uint32_t* size,
                        const char** name);

/* The parameter named `name` (a NUL-terminated string, as declared in the .entry's
 * parameter list): its byte offset in the parameter block ks_run takes, and its
 * size in bytes.  `offset` or `size` may be NULL.  The same layout as
 * ks_param_info.  Defined by: the KernelScope page's "ptx/parser.py,
 * ptx/models.py" part (parameters by name, as ld.param [name] reads them).
 * Errors: KS_E_INVALID_ARG for NULL prog/name or no parameter of that name. */
ks_status ks_param_offset(const ks_program* prog, const char* name, uint32_t* offset, uint32_t* size);

typedef struct {
  uint32_t line;          /* 1-based line of the instruction in the PTX text */
  uint32_t kind;          /* KS_EV_* kind of its extended trace records (a bra: KS_EV_BRANCH) */
  uint32_t access_bytes;  /* bytes per lane of a ld/st.global or ld/st.shared (4 or 8), else 0 */
  uint32_t lat_class;     /* KS_LAT_* class whose latency its destination takes */
} ks_instr_desc;

/* Host-side description of decoded instruction `pc` (0 <= pc < n_instrs): what the
 * tools that read trace records (pc -> source line, access width) need.  Writes
 * *out.  Defined by: the KernelScope page's "ptx/parser.py, ptx/models.py" part
 * (each instruction keeps its source line, used to place hints and highlight
 * code) and its "simulator/models.py" part (the trace event names the
 * instruction it comes from).  KS_E_INVALID_ARG for NULL or a pc out of range. */
ks_status ks_instr_info(const ks_program* prog, uint32_t pc, ks_instr_desc* out);

/* Debug: for each instruction, the reconvergence index of a guarded bra (n_instrs
 * meaning "exit"), 0xFFFFFFFF for every other instruction.  `out` (host memory)
 * holds `n` entries; the first min(n, n_instrs) are written.  Defined by: the
 * KernelScope page's "simulator/engine.py, simulator/models.py" part (the SIMT
 * stack entry's reconvergence point), read as the immediate post-dominator.
 * KS_E_INVALID_ARG for NULL arguments. */
ks_status ks_ipdom_table(const ks_program* prog, uint32_t* out, uint32_t n);

/* Fill `cfg` with defaults: the sm_80 latency table of the KernelScope page's
 * "latency/model.py" part (int/fp32 4, ld.global 200, ld.shared 23, ld.param as
 * ld.const 4, bar.sync 20) and the cache latencies of its memory-analysis part
 * (L1 hit 28, L2 hit 150, DRAM 400), trace_cap 0, max_warp_instrs 0xFFFFFFFF
 * (the simulator's run(max_steps) cap, per warp), max grid/block 1, basic trace
 * format, no cache model.  KS_E_INVALID_ARG for NULL. */
ks_status ks_default_config(ks_config* cfg);

/* Sizes of the caller-owned device buffers for runs up to cfg->max_grid x
 * cfg->max_block, written to *out.  Defined by: the IKET page, section 2 ("buffer
 * 是怎么定形的"): the buffer is sized once the launch's grid and block are known,
 * one slot per warp (warps per block = ceil(threads / 32)), a slot being a
 * 16-byte header plus the per-warp record cap times the record size (8 bytes, or
 * 16 with a payload); the 1.15 margin is dropped because records past the cap are
 * counted, not stored.  KS_E_INVALID_ARG for an unknown trace_format or
 * cache_model; KS_E_UNSUPPORTED for the cache model with extended records or over
 * more than 2^38 bytes. */
ks_status ks_query_layout(const ks_program* prog, const ks_config* cfg, ks_layout* out);

/* Bind a program to caller-owned device buffers on the current HIP device.
 * Defined by: the KernelScope page's "simulator/engine.py" part (PtxSimulator(config)
 * with load_kernel: a simulator instance holds one program and its launch
 * configuration) and the IKET page, section 2 (the trace buffer is allocated per
 * launch shape and handed to the kernel by its base address).  Buffers:
 *   d_gmem      cfg->gmem_bytes of simulated global memory (inputs are written here by
 *               the caller; ks_run updates it in place and it persists across runs),
 *   d_counters  layout.counters_bytes: 80-byte per-warp counter records,
 *   d_trace     layout.trace_bytes: per-warp trace slots,
 *   d_cache     layout.cache_bytes: the cache model's per-warp state, 16-byte
 *               aligned (NULL without the cache model; each ks_run first clears
 *               the state of its grid's warps with a kernel of its own).
 * Uploads the decoded program (latencies baked in from cfg) to a small device
 * buffer owned by the state.  Errors: KS_E_INVALID_ARG (NULL buffers, limits),
 * KS_E_UNSUPPORTED (program beyond this build's limits), KS_E_HIP, KS_E_NOMEM. */
ks_status ks_alloc_state(const ks_program* prog, const ks_config* cfg, void* d_gmem, void* d_counters,
                         void* d_trace, void* d_cache, ks_state** out);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): ks_alloc_state without
 * any device allocation.  The decoded program and the status word of
 * ks_run_status go into a static scratch array the library holds on each GPU
 * (1 MiB + 256 bytes, kept until the process ends) instead of memory of the
 * state's own; the caller-owned buffers are as for ks_alloc_state.  The program is
 * copied in synchronously (hipMemcpy) by this call; nothing else is allocated on
 * the device, and ks_run, ks_run_status, ks_read_* and ks_state_free work on the
 * returned state as on any other (ks_state_free releases no device memory).
 * Sharing: every static state on a GPU shares that GPU's scratch, which holds the
 * program of the latest binding.  A ks_run of a static state bound before the
 * latest one on its device fails with KS_E_STATE; work of two static states that
 * overlaps on one GPU (other streams, other host threads) races.
 * Errors: KS_E_UNSUPPORTED for a program of more than KS_STATIC_MAX_INSTRS
 * instructions, otherwise those of ks_alloc_state (never KS_E_NOMEM). */
ks_status ks_alloc_state_static(const ks_program* prog, const ks_config* cfg, void* d_gmem, void* d_counters,
                                void* d_trace, void* d_cache, ks_state** out);

/* Launch one simulation of grid x block threads on `stream` (asynchronous).
 * Defined by: the KernelScope page's "simulator/engine.py" part, run() (step every
 * warp of every block until all have finished or the step cap is reached; here
 * the cap is cfg->max_warp_instrs per warp) and its "simulator/models.py" part
 * (warps, active masks, the SIMT stack, barriers); the trace base pointer is a
 * launch argument as on the IKET page, section 2.
 * `params` holds `params_len` >= param_bytes bytes of the parameter block (host
 * memory; copied into the launch arguments).  Each run re-initialises registers,
 * predicates, stacks, scoreboards, shared windows and (with the cache model) the
 * caches, and rewrites every counter record and trace header of the grid's
 * warps.  Warps are numbered linear block id * warps_per_block + warp in block.  With extended records the
 * grid is launched KS_EXT_MAX_BLOCKS blocks at a time (blocks share nothing but
 * simulated global memory, whose accesses by different blocks must not race).
 * Errors: KS_E_INVALID_ARG (shape beyond the allocation, short params),
 * KS_E_UNSUPPORTED (a block too large for the interpreter variant), KS_E_HIP. */
ks_status ks_run(ks_state* st, ks_dim3 grid, ks_dim3 block, const void* params, size_t params_len,
                 void* stream);

/* Name of the interpreter kernel ks_run launches for this program and block shape,
 * as profilers list it: "ks_interp_v32" (programs of up to 32 register slots: a
 * 40-VGPR register file per lane, six slots of it for immediates and two for the
 * constants 1.0f and -0.0f) or "ks_interp_v64" (up to 64 slots: a 72-VGPR
 * file); runs with the extended trace
 * format launch the same kernel with the suffix "_ext", runs with the cache model
 * the one with the suffix "_cache".  *name points to a static
 * string.  Errors: KS_E_INVALID_ARG (NULL arguments, empty or oversized block). */
ks_status ks_interp_kernel(const ks_program* prog, ks_dim3 block, const char** name);

/* Copy n bytes of simulated global memory at byte offset sim_addr to host memory
 * `host` (caller-owned, >= n bytes), after the work queued on `stream`; returns
 * when the copy is done.  Defined by: the KernelScope page's "simulator/models.py"
 * part (the simulated global memory the kernel's st.global writes).
 * KS_E_INVALID_ARG if out of range or NULL, KS_E_HIP if the copy fails. */
ks_status ks_read_outputs(ks_state* st, uint64_t sim_addr, void* host, size_t n, void* stream);

/* Copy the counter records of warps [first_warp, first_warp + n_warps) of the last
 * run to `host` (caller-owned, n >= 80 * n_warps bytes); returns when done.
 * Defined by: the KernelScope page's "simulator/models.py" part (per-warp
 * statistics: instructions, cycles, stalls) and its memory-analysis part (per
 * access transactions, sectors and bank-conflict degree), summed per warp.
 * KS_E_STATE before any run; KS_E_INVALID_ARG for a range outside the last run. */
ks_status ks_read_counters(ks_state* st, uint64_t first_warp, uint64_t n_warps, void* host, size_t n,
                           void* stream);

/* Copy the trace slots of warps [first_warp, first_warp + n_warps) of the last run
 * to `host` (caller-owned, n >= slot_bytes * n_warps); returns when done.  Record
 * bytes past a slot's records_written are unspecified.  Defined by: the IKET
 * page, section 2 (per-warp slots) and section 3 (after the kernel finishes the
 * buffer is copied back to the host for post-processing).  KS_E_STATE before any
 * run; KS_E_INVALID_ARG for a range outside the last run. */
ks_status ks_read_trace(ks_state* st, uint64_t first_warp, uint64_t n_warps, void* host, size_t n,
                        void* stream);

/* OR of the status bits of every warp of the last run (reduced on the GPU into a
 * small device word the state owns), written to *or_bits.  Defined by: the IKET
 * page, section 2 (overflow is reported, never silently dropped) and the
 * KernelScope page's "simulator/engine.py" part (a run ends when every warp has
 * finished or the step cap is reached).  KS_E_STATE before any run. */
ks_status ks_run_status(ks_state* st, uint32_t* or_bits, void* stream);

/* Host-side export (no device work): write the trace slots of warps [first_warp,
 * first_warp + n_warps) -- `trace` holds them as ks_read_trace returns them,
 * slot_bytes each, in trace_format -- as a Chrome / Perfetto trace-event JSON file
 * at `path`: one process per block, one thread per warp (warps_per_block warps per
 * block), one complete event per record from its issue cycle to the warp's next
 * issue (1 cycle for the last), time unit one simulated cycle.  Extended records
 * add the record's active mask and its payload fields (sectors, lines, lanes and
 * faults; degree; taken; guard_lanes) to the event's args.  pc_names[pc] and
 * pc_args[pc] (pc < n_pcs) are inserted verbatim: a JSON string for the event name
 * and the leading JSON members of its args (for example "pc":4,"line":12).
 * *n_events (may be NULL) receives the number of instruction events.  Defined by:
 * the IKET page, sections 3 and 5 (post-processing of the per-warp buffer into a
 * Perfetto timeline).  Errors: KS_E_INVALID_ARG for NULL arguments (a NULL
 * fragment included), a slot size
 * that does not fit the format, a record whose pc or kind is outside the program,
 * or a file that cannot be written (a file opened before the error is left
 * partly written). */
ks_status ks_write_trace_events(const void* trace, uint64_t n_warps, uint64_t slot_bytes, uint32_t trace_format,
                                uint64_t first_warp, uint32_t warps_per_block, uint32_t n_pcs,
                                const char* const* pc_names, const char* const* pc_args, const char* path,
                                uint64_t* n_events);

/* Release a state (and its device copy of the program) or a program.  NULL is a no-op. */
void ks_state_free(ks_state* st);
void ks_program_free(ks_program* prog);

/* Message of the last error on this thread ("" if none). */
const char* ks_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KS_H */
