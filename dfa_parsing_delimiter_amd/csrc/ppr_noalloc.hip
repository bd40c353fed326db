// ppr_parse_noalloc: the parse of ppr_parse for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc). Its workspace is `scratch`, a fixed array in the
// library's own device memory, so the call brings in no workspace argument and
// allocates nothing.
//
// In host code `scratch` names a host-side stand-in, not the device array: its
// device address is taken once per device with hipGetSymbolAddress (with that
// device current) and kept in scratch_ptr[device]; only that pointer is ever
// handed to kernels. Each GPU holds its own copy of the array, at its own
// address, until the process ends.
#include <mutex>

#include "ppr_csv_common.h"

// the scratch of every ppr_parse_noalloc call on a GPU (its device address:
// ppr::device_scratch)
static __device__ __align__(256) uint8_t scratch[PPR_NOALLOC_SCRATCH_BYTES];

namespace ppr {
namespace {

// 16 MiB: the fused kernel's statuses for the largest input of one call
// (131,070 tiles x 72 bytes) plus the header and step tables; the generic
// kernel's for up to 233,000 tiles of 1024 chunks.
constexpr size_t kScratchBytes = PPR_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

uint8_t* scratch_ptr[kMaxDevices];
std::mutex scratch_mu;

// The current device's scratch (its address from hipGetSymbolAddress, taken
// at the first call on the device). Nothing in it needs to start at zero: a
// parse resets its header and clears its look-back statuses itself. NULL on a
// HIP error.
uint8_t* device_scratch()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        scratch_ptr[dev] = (uint8_t*)ptr;
    }
    return scratch_ptr[dev];
}

}  // namespace
}  // namespace ppr

namespace ppr {
int parse_results(const void* d_ws, ppr_parse_out_t* out, hipStream_t s, bool may_alloc);  // ppr_csv.hip
}  // namespace ppr

using namespace ppr;

extern "C" PPR_API int ppr_parse_noalloc(const uint8_t* d_bytes, uint64_t n, const ppr_dfa_t* dfa,
                                         const uint8_t class_map[256], ppr_parse_out_t* out,
                                         const ppr_parse_opts_t* opts, void* stream)
{
    if (!out) return PPR_EINVAL;
    uint8_t* ws = device_scratch();
    if (!ws) return PPR_EHIP;
    // an input whose statuses exceed the scratch is refused before anything is enqueued
    const int rc = parse_enqueue(d_bytes, n, dfa, class_map, out, ws, kScratchBytes, opts, stream, true);
    if (rc == PPR_EWORKSPACE) return PPR_ETOOBIG;
    if (rc) return rc;
    return parse_results(ws, out, (hipStream_t)stream, false);  // (no pinned header buffer: it allocates)
}
