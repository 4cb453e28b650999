// rp_sgmm_step_noalloc: rp_sgmm_step for callers that cannot allocate device
// memory.  Its workspace is `scratch`, a file-scope device array of
// kScratchBytes that every GPU the library runs on holds until the process
// ends.  Host code never passes the array's name to a kernel or a copy: it
// uses the device address hipGetSymbolAddress returns for the current device,
// looked up once per device on the first call there.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/rank_pregate.h"
#include "kernels.h"

namespace rp {  // api.cpp
rp_status record_error(rp_status st, const char* msg);  // sets rp_last_error()
rp_status validate_step(const char* fn, const rp_group* groups, int32_t n_groups, int64_t T, int64_t E, int64_t r,
                        int32_t k, const void* Wg_or_null, int32_t* topk_idx, float* topk_gate, int32_t* seg_offsets,
                        int32_t* pair_perm, rp_dtype dt);  // rp_sgmm_step's checks but the workspace's
}

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Zero n 16-byte words (the control region must start at zero; no memset node
// is recorded, so the call stays capturable once a device is set up).
__global__ void zero16(uint4* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {nullptr};  // device address of `scratch`, per device

// Device address of this device's scratch; on the first call on a device it is
// looked up and its control region cleared on `stream` (ordered before the
// step the caller queues next on the same stream).
rp_status scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return rp::record_error(RP_ERR_HIP, "rp_sgmm_step_noalloc: cannot query the current device");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev]) {
    *out = g_ptr[dev];
    return RP_OK;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return rp::record_error(RP_ERR_INVALID_ARG,
                            "rp_sgmm_step_noalloc: the first call on a device sets up its static workspace and "
                            "must not be recorded into a graph");
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr) {
    char msg[256];
    snprintf(msg, sizeof msg, "rp_sgmm_step_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    return rp::record_error(RP_ERR_HIP, msg);
  }
  const int words = (int)(rp::kWorkspaceCounterBytes / 16);
  zero16<<<(words + 255) / 256, 256, 0, stream>>>(static_cast<uint4*>(p), words);
  e = hipGetLastError();
  if (e != hipSuccess) {
    char msg[256];
    snprintf(msg, sizeof msg, "rp_sgmm_step_noalloc: clearing the workspace: %s", hipGetErrorString(e));
    return rp::record_error(RP_ERR_HIP, msg);
  }
  g_ptr[dev] = p;
  *out = p;
  return RP_OK;
}

}  // namespace

extern "C" rp_status rp_sgmm_step_noalloc(const rp_group* groups, int32_t n_groups, int64_t T, int64_t E, int64_t r,
                                          int32_t k, const void* Wg_or_null, int32_t* topk_idx, float* topk_gate,
                                          int32_t* seg_offsets, int32_t* pair_perm, rp_dtype dt,
                                          hipStream_t stream) {
  rp_status st = rp::validate_step("rp_sgmm_step_noalloc", groups, n_groups, T, E, r, k, Wg_or_null, topk_idx,
                                   topk_gate, seg_offsets, pair_perm, dt);
  if (st != RP_OK || T == 0) return st;
  // the workspace the call needs on this device
  const size_t need = rp_sgmm_step_workspace_size(groups, n_groups, T, E, r, k, dt);
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "rp_sgmm_step_noalloc: the call needs a %zu-byte workspace, beyond the %zu-byte static one "
             "(use rp_sgmm_step with a workspace of its own)",
             need, kScratchBytes);
    return rp::record_error(RP_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  st = scratch_for_current_device(stream, &ws);
  if (st != RP_OK) return st;
  return rp_sgmm_step(groups, n_groups, T, E, r, k, Wg_or_null, topk_idx, topk_gate, seg_offsets, pair_perm, dt, ws,
                      kScratchBytes, stream);
}
