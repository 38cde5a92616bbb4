// pa_decode_scratch: pa_decode whose workspace is a file-scope device array,
// so that a call allocates nothing (for callers that cannot: code under graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array is the library's: each device the library runs on holds its own
// copy for the life of the process.  Its address on a device comes from
// hipGetSymbolAddress, taken once per device with that device current; host
// code passes only that address on (the array's name in host code is a
// host-side stand-in, not a device address).  Every call on a device shares
// the device's array and it keeps the last call's contents: the error word is
// cleared by a one-thread kernel on the call's stream at the start of each
// call (a kernel, not a memset, so a captured graph replays it), and the chunk
// partials and plan header are written before they are read.  Calls that
// overlap on one device race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(PA_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};       // device address of `scratch` on each device, once taken

__global__ void clear_error_word(uint32_t* w) {
  if (threadIdx.x == 0) *w = 0u;
}

}  // namespace

namespace pa {

// Device address of the scratch array on the current device (nullptr with an
// error status when it cannot be taken).
void* scratch_buffer(pa_status* st) {
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= kMaxDevices) {
    *st = PA_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[device]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      *st = PA_ERR_HIP;
      return nullptr;
    }
    g_ptr[device] = ptr;
  }
  *st = PA_OK;
  return g_ptr[device];
}

}  // namespace pa

extern "C" pa_status pa_decode_scratch(const float* q, const void* k_pool, const void* v_pool,
                                       const int32_t* block_table, const int32_t* seq_lens, int32_t n_seq,
                                       int32_t n_qtok, int32_t kv_type, int32_t page_size, float* out,
                                       hipStream_t stream, const pa_decode_ext* ext) {
  if (!ext || ext->workspace || ext->workspace_bytes) return PA_ERR_INVALID;
  if (n_seq < 0 || n_qtok < 1 || n_qtok > PA_MAX_QTOK) return PA_ERR_INVALID;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return PA_ERR_HIP;
  size_t need = 0;
  const pa_status ws = pa_decode_workspace_size(n_seq, n_qtok, device, &need);
  if (ws != PA_OK) return ws;
  if (need > kScratchBytes) return PA_ERR_UNSUPPORTED;   // beyond the array: use pa_decode with a workspace
  pa_status st = PA_OK;
  void* ptr = pa::scratch_buffer(&st);
  if (st != PA_OK) return st;
  pa_decode_ext e = *ext;
  e.workspace = ptr;
  e.workspace_bytes = kScratchBytes;
  if (n_seq > 0) {
    hipLaunchKernelGGL(clear_error_word, dim3(1), dim3(64), 0, stream, static_cast<uint32_t*>(ptr));
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
  return pa_decode(q, k_pool, v_pool, block_table, seq_lens, n_seq, n_qtok, kv_type, page_size, out, stream, &e);
}
