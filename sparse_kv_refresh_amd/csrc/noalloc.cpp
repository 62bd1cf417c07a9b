// wamc_prefill_chunk_noalloc: the refresh chunk with its workspace in a
// static device array, for callers that cannot allocate device memory.
#include "../../include/wamc.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <map>
#include <mutex>

namespace wamc {
int api_fail(int code, const char* msg);
}

// The chunk's workspace.  One copy per GPU the library runs on, held until
// the process ends.  In host code this name stands for the host-side shadow
// of the array, not a device address: kernels and copies get the address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[WAMC_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_mu;
std::map<int, void*> g_scratch;   // device -> address of its copy of `scratch`

int scratch_ptr(void** out) {
  char msg[160];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess)
    return wamc::api_fail(WAMC_ERR_DEVICE, "wamc_prefill_chunk_noalloc: no HIP device");
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      std::snprintf(msg, sizeof(msg), "wamc_prefill_chunk_noalloc: scratch address on device %d: %s", dev,
                    hipGetErrorString(e));
      return wamc::api_fail(WAMC_ERR_DEVICE, msg);
    }
    it = g_scratch.emplace(dev, p).first;
  }
  *out = it->second;
  return WAMC_OK;
}

}  // namespace

extern "C" int wamc_prefill_chunk_noalloc(const wamc_dims* dims, const wamc_layer_w* layers, const void* z,
                                          void* zref, const void* q_act, const float* mass_in, void* k_cache,
                                          void* v_cache, int32_t* age, int32_t k, const int32_t* idx_override,
                                          const int32_t* k_eff_override, int32_t* idx_out, int32_t* k_eff_out,
                                          float* score_out, float* layer_out, int32_t rows_cap, void* stream) {
  size_t need = 0;
  if (dims && wamc_workspace_bytes(dims, rows_cap, &need) == WAMC_OK && need > WAMC_NOALLOC_SCRATCH_BYTES) {
    char msg[200];
    std::snprintf(msg, sizeof(msg),
                  "wamc_prefill_chunk_noalloc: this chunk needs %zu bytes of scratch, the static scratch holds %zu "
                  "(pass a workspace to wamc_prefill_chunk instead)",
                  need, static_cast<size_t>(WAMC_NOALLOC_SCRATCH_BYTES));
    return wamc::api_fail(WAMC_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  if (int st = scratch_ptr(&ws)) return st;
  return wamc_prefill_chunk(dims, layers, z, zref, q_act, mass_in, k_cache, v_cache, age, k, idx_override,
                            k_eff_override, idx_out, k_eff_out, score_out, layer_out, rows_cap, ws,
                            WAMC_NOALLOC_SCRATCH_BYTES, stream);
}
