// ks_launch.h -- host-side launch wrappers of the gfx950 kernels (internal).
#pragma once
#include <hip/hip_runtime.h>

#include "ks_isa.h"

// Interpreter: one workgroup per simulated block, ceil(warps/2) wave64s per
// workgroup.  `slots` is the program's register-slot count.
hipError_t ks_launch_interp(const ks::KsArgs& a, uint32_t n_blocks, uint32_t slots, hipStream_t s);

// OR of the status words of `n_warps` counter records into *d_out.
hipError_t ks_launch_status_or(const void* counters, uint64_t n_warps, uint32_t* d_out, hipStream_t s);

// Largest dynamic LDS a workgroup of the interpreter may use on the current device.
size_t ks_lds_limit();

// Register-file variant for a program and block size: 32 or 64 (reserved VGPRs)
// or 0 (LDS).
int ks_choose_variant(uint32_t slots, uint32_t block_threads);

// Dynamic LDS bytes of one workgroup of `wg` lanes for that variant.
size_t ks_lds_bytes(int variant, uint32_t slots, uint32_t wg, uint32_t shared_bytes);
