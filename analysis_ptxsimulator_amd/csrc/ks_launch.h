// ks_launch.h -- host-side launch wrappers of the gfx950 kernels (internal).
#pragma once
#include <hip/hip_runtime.h>

#include "ks_isa.h"

// Interpreter: one workgroup per simulated block, ceil(warps/2) wave64s per
// workgroup.  `slots` is the program's register-slot count (a.rf_slots must be
// slots plus the immediate slots).
hipError_t ks_launch_interp(const ks::KsArgs& a, uint32_t n_blocks, uint32_t slots, hipStream_t s);

// Zeroes `bytes` (a multiple of 16) at the 16-byte aligned device address p.
hipError_t ks_launch_clear(void* p, uint64_t bytes, hipStream_t s);

// OR of the status words of `n_warps` counter records into *d_out.
hipError_t ks_launch_status_or(const void* counters, uint64_t n_warps, uint32_t* d_out, hipStream_t s);

// Largest dynamic LDS a workgroup of the interpreter may use on the current device.
size_t ks_lds_limit();

// Register-file variant for a program of `slots` register slots: 32 (40 reserved
// VGPRs) or 64 (72 reserved VGPRs), immediate slots included; 0 if neither fits.
int ks_choose_variant(uint32_t slots, uint32_t block_threads);

// Largest block the interpreter variant can run: 1024 threads, except the
// extended-trace variant with the 72-VGPR file (136 VGPRs: 768 threads); `ext`
// selects the extended-trace variants.
uint32_t ks_max_block_threads(int variant, bool ext);

// Dynamic LDS bytes of one workgroup of `wg` lanes (scoreboards, with `ext` the
// staging ring of extended trace records, and the shared window).
size_t ks_lds_bytes(uint32_t wg, uint32_t shared_bytes, bool ext);

// The library's static scratch on device `dev` (the current device), for states
// that must not allocate: where the decoded program and the status word go.  The
// first call on a device looks the array's address up (hipGetSymbolAddress); each
// call starts a new binding generation on that device, returned in *generation.
hipError_t ks_static_scratch(int dev, ks::DInst** prog, uint32_t** status, uint64_t* generation);

// The latest binding generation of device `dev` (0 before any static binding).
uint64_t ks_static_generation(int dev);
