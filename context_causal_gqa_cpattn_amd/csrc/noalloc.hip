// The backward for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): cpattn_bwd with its
// workspace in a file-scope device array instead of a caller-provided buffer.
//
// The array is part of the library's code object, so each GPU that runs the library holds
// one copy (CPATTN_NOALLOC_SCRATCH_BYTES) from the time the code object is loaded on it
// until the process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the device symbol): on the first call on a device the
// device address is looked up once with hipGetSymbolAddress, with that device current,
// and kept per device.
//
// No part of the workspace has to start at zero: the pre-pass writes Delta, the transposed
// tiles and their row statistics before dK/dV reads them, the chunks' dS offsets are
// written before dK/dV, dQ reads only the dS blocks that dK/dV wrote in the same call, and
// the dBias kernel writes its partial sums before they are added.  So the array needs no
// clearing between calls, and whatever an earlier call left in it is never read.  Calls that overlap in time on one GPU (different streams, or different host
// threads) share the one array and race; serialize them.
#include <mutex>

#include "../../include/cpattn.h"
#include "common.h"

static __device__ __align__(256) unsigned char scratch[CPATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per device).
int scratch_address(void** out, int* dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return CPATTN_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return CPATTN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return CPATTN_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  *dev_out = dev;
  return CPATTN_OK;
}

}  // namespace

extern "C" {

// Implemented next to the other entry points; sets the message cpattn_last_error returns.
__attribute__((visibility("hidden"))) int cpattn_internal_fail(int status, const char* msg);

int cpattn_bwd_noalloc(const cpattn_problem* p, const void* q, const void* k, const void* v,
                       const int32_t* seq_offsets, const int32_t* seq_lens,
                       const int32_t* q_chunk_map, const float* bias, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       float* dbias, int dkv_accumulate, int32_t* dev_err,
                       cpattn_stream_t stream) {
  // The workspace this problem needs: the stored-dS backward when it fits, else the one
  // that forms dS again for dQ (the same choice cpattn_bwd makes by workspace size).
  const size_t need_ds = cpattn_workspace_size(p, CPATTN_OP_BWD_DS);
  size_t need_rc = cpattn_workspace_size(p, CPATTN_OP_BWD);
  if (need_rc == 0 && need_ds == 0)  // the problem itself is invalid: let cpattn_bwd say why
    return cpattn_bwd(p, q, k, v, seq_offsets, seq_lens, q_chunk_map, bias, o, lse, dout, dq, dk,
                      dv, dbias, dkv_accumulate, nullptr, 0, dev_err, stream);
  size_t use;
  if (need_ds > 0 && need_ds <= (size_t)CPATTN_NOALLOC_SCRATCH_BYTES) {
    use = need_ds;
  } else if (need_rc <= (size_t)CPATTN_NOALLOC_SCRATCH_BYTES) {
    use = need_rc;
  } else {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "cpattn_bwd_noalloc: the problem needs %zu bytes of workspace, more than the %zu "
             "bytes of its static scratch (use cpattn_bwd with a caller-provided workspace)",
             need_rc, (size_t)CPATTN_NOALLOC_SCRATCH_BYTES);
    return cpattn_internal_fail(CPATTN_EUNSUPPORTED, msg);
  }
  void* ws = nullptr;
  int dev = -1;
  const int r = scratch_address(&ws, &dev);
  if (r != CPATTN_OK)
    return cpattn_internal_fail(r, "cpattn_bwd_noalloc: no device address for the static scratch "
                                   "on the current device");
  return cpattn_bwd(p, q, k, v, seq_offsets, seq_lens, q_chunk_map, bias, o, lse, dout, dq, dk, dv,
                    dbias, dkv_accumulate, ws, use, dev_err, stream);
}

}  // extern "C"
