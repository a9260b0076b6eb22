// noalloc.hip -- blasst_attn_decode_noalloc: the decode call with its split partials in a
// scratch array the library owns, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ object: every GPU the library runs on holds its own copy
// for the life of the process. Host code never passes the array's name to a kernel (on the host
// that name is only a stand-in, not a device address): the first call on a device looks up that
// device's address with hipGetSymbolAddress and keeps it, and every launch takes that address.
// The kernels write every partial row they later read (O and LSE of each (sequence, head,
// split), empty splits included), so nothing in the array has to start at zero and no call
// clears it. Calls that overlap on one GPU share the array and race.
#include <mutex>

#include "blasst.h"
#include "internal.h"

namespace {

static __device__ __attribute__((aligned(256))) unsigned char scratch[BLASST_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices];  // per device: the device address of `scratch`, once looked up

// The device address of this device's copy of the scratch array (looked up once per device).
blasst_status scratch_for_current_device(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return BLASST_ERR_HIP;
  if (dev >= kMaxDevices) return BLASST_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BLASST_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return BLASST_OK;
}

}  // namespace

extern "C" blasst_status blasst_attn_decode_noalloc(const blasst_decode_args *a, void *stream) {
  // Host checks first (no HIP call): a bad argument or a plan whose partials do not fit the
  // array is refused before the device is touched.
  const blasst_status st = blasst::decode_check(a);
  if (st != BLASST_OK) return st;
  const size_t need = blasst_decode_workspace_size(a);
  if (need > (size_t)BLASST_NOALLOC_SCRATCH_BYTES) return BLASST_ERR_WORKSPACE;
  void *ws = nullptr;
  if (need > 0) {
    const blasst_status sp = scratch_for_current_device(&ws);
    if (sp != BLASST_OK) return sp;
  }
  return blasst::decode_with_workspace(a, ws, need > 0 ? (size_t)BLASST_NOALLOC_SCRATCH_BYTES : 0,
                                       stream);
}
