// ks_scratch.hip -- the library's static device scratch (states bound by
// ks_alloc_state_static, for callers that cannot allocate device memory).
//
// It holds the decoded program (up to KS_STATIC_MAX_INSTRS instructions plus the
// end sentinel and the prefetch padding) and the status word of ks_run_status.
// There is one copy per GPU, held until the process ends.  In host code the
// array's name is a host-side stand-in, not a device address: its address on each
// device is looked up once with hipGetSymbolAddress (with that device current) and
// only that address is used afterwards (kernel arguments, copies).  The
// interpreter kernels take it as their program pointer like any other.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/ks.h"
#include "ks_isa.h"
#include "ks_launch.h"

using ks::DInst;

constexpr size_t KS_STATIC_PROG_BYTES = (size_t)(KS_STATIC_MAX_INSTRS + 1 + ks::KS_PREFETCH_PAD) * sizeof(DInst);
constexpr size_t KS_STATIC_SCRATCH_BYTES = KS_STATIC_PROG_BYTES + 256;
static_assert(KS_STATIC_PROG_BYTES % 256 == 0, "the status word starts on a 256-byte boundary");

static __device__ __align__(256) uint8_t scratch[KS_STATIC_SCRATCH_BYTES];

namespace {
constexpr int KS_MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[KS_MAX_DEVICES];      // device address of `scratch` on each device (null: not looked up yet)
uint64_t g_gen[KS_MAX_DEVICES];   // static bindings made on each device so far
}  // namespace

hipError_t ks_static_scratch(int dev, DInst** prog, uint32_t** status, uint64_t* generation) {
  if (dev < 0 || dev >= KS_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = ptr;
  }
  *prog = reinterpret_cast<DInst*>(g_ptr[dev]);
  *status = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(g_ptr[dev]) + KS_STATIC_PROG_BYTES);
  *generation = ++g_gen[dev];
  return hipSuccess;
}

uint64_t ks_static_generation(int dev) {
  if (dev < 0 || dev >= KS_MAX_DEVICES) return 0;
  std::lock_guard<std::mutex> lock(g_mu);
  return g_gen[dev];
}
