// Allocation-free variant of the backward call (flamia_attn_bwd_noalloc).
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the
// backward's workspace -- quantized dO, D, 2^-8/l, G, the fp16 dQ
// accumulator, the per-row planes and, by mode, the dQ partial slots or fp32
// staging -- lives in a file-scope device array instead of a caller buffer.
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  Its device address is looked up once per device, with that
// device current, on the entry point's first call there; host code only ever
// uses that address (the array's name on the host is a stand-in, not a
// device address).  Every call on one GPU uses the same array: calls that
// overlap on one GPU (two streams, two threads) race.  What must start at
// zero is cleared by the call itself (the prep stage zeroes the fp16 dQ
// accumulator; every other region is written before it is read), so the
// previous call's contents never leak into the next.
#include <mutex>

#include "../../include/flamia.h"
#include "flamia_internal.hpp"

constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(32) << 20;   // per GPU

static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;

std::once_flag g_once[NOALLOC_MAX_DEVICES];
void* g_scratch[NOALLOC_MAX_DEVICES];
hipError_t g_status[NOALLOC_MAX_DEVICES];

// Device address of `scratch` on device `dev`, which must be current.
hipError_t scratch_address(int dev, void** out) {
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_status[dev] == hipSuccess ? p : nullptr;
  });
  *out = g_scratch[dev];
  return g_status[dev];
}

}  // namespace

extern "C" flamia_status flamia_attn_bwd_noalloc(const flamia_attn_desc* desc, const flamia_qtensors* qt,
                                                 const void* o, const int32_t* row_max, const float* row_sum,
                                                 const void* dout, void* dq, void* dk, void* dv,
                                                 hipStream_t stream) {
  size_t ws_bytes = 0;
  const flamia_status s = flamia_buffer_sizes(desc, nullptr, nullptr, &ws_bytes);
  if (s != FLAMIA_OK) return s;
  if (ws_bytes > NOALLOC_SCRATCH_BYTES) return FLAMIA_ERR_WORKSPACE;
  int cur = 0, on = 0;
  if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &on) != hipSuccess) return FLAMIA_ERR_HIP;
  if (on != cur || cur < 0 || cur >= NOALLOC_MAX_DEVICES) return FLAMIA_ERR_INVALID_ARG;
  void* ws = nullptr;
  if (scratch_address(cur, &ws) != hipSuccess || ws == nullptr) return FLAMIA_ERR_HIP;
  return flamia_attn_bwd(desc, qt, o, row_max, row_sum, dout, dq, dk, dv, ws, stream);
}
