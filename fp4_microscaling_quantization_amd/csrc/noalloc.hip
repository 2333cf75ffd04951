// noalloc.hip -- fp4_quantize without a caller workspace, for callers that
// cannot allocate device memory: code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc.
//
// The NVFP4 / NVINT4 scratch that fp4_quantize takes as its workspace (the
// partial maxima of the tensor-maximum pass and the single-pass exchange
// region) is a file-scope device array here: one copy per GPU, loaded with
// the library's code object and held until the process ends.  Host code never
// passes the array's name to a kernel (in host code it is only a stand-in for
// the symbol): the device address of each GPU's copy is looked up once per
// device with hipGetSymbolAddress and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fp4.h"
#include "launch.h"

namespace {

// fp4_workspace_bytes() of every NV configuration (MX formats need none).
constexpr size_t kScratchBytes = 8192;
// The single-pass exchange region inside it, which must start at zero.
constexpr size_t kExchangeOffset = 4096;
constexpr int kMaxScratchDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// Zeroes the single-pass exchange region when its give-up flag (word 1) is
// set.  A launch whose grid-wide wait gave up can leave a slot tagged with the
// next call's number (a workgroup that started after workgroup 0 advanced the
// call number), which the next single-pass call would otherwise read as one of
// its own maxima; a caller workspace is re-zeroed with fp4_workspace_init, the
// static scratch by this kernel, queued before every single-pass call.  One
// workgroup: every thread reads the flag before any thread clears it.
__global__ __launch_bounds__(256) void exchange_repair_kernel(uint32_t* __restrict__ region,
                                                              uint32_t nwords) {
  __shared__ uint32_t flag;
  if (threadIdx.x == 0) flag = region[1];
  __syncthreads();
  if (flag == 0) return;
  for (uint32_t i = threadIdx.x; i < nwords; i += blockDim.x) region[i] = 0u;
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

// Device address of the current device's copy of `scratch`; on the first call
// on a device the exchange region is also zeroed (a fill kernel on `st`, so
// the call may run under graph capture).  FP4_OK or a negative status.
int scratch_of_current_device(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return FP4_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return FP4_ERR_HIP;
    uint32_t* xchg = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(p) + kExchangeOffset);
    if (fp4lib::launch_zero_words(xchg, (int64_t)((kScratchBytes - kExchangeOffset) / 4), st) !=
        hipSuccess)
      return FP4_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FP4_OK;
}

}  // namespace

extern "C" int fp4_quantize_noalloc(const fp4_qconfig* cfg, const void* x, int32_t xdt,
                                    int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes,
                                    uint8_t* scales, float* global_scale, int32_t gs_mode,
                                    void* stream) {
  const size_t need = fp4_workspace_bytes(cfg, rows, cols);
  if (need > kScratchBytes) return FP4_ERR_WORKSPACE;
  if (need == 0)  // MX formats, or a configuration fp4_quantize will reject
    return fp4_quantize(cfg, x, xdt, rows, cols, ldx, codes, scales, global_scale, gs_mode,
                        nullptr, 0, stream);
  void* ws = nullptr;
  const int rc = scratch_of_current_device(static_cast<hipStream_t>(stream), &ws);
  if (rc != FP4_OK) return rc;
  if (gs_mode == FP4_GS_COMPUTE_ONE_PASS) {
    uint32_t* xchg = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + kExchangeOffset);
    exchange_repair_kernel<<<1, 256, 0, static_cast<hipStream_t>(stream)>>>(
        xchg, (uint32_t)((kScratchBytes - kExchangeOffset) / 4));
    if (hipGetLastError() != hipSuccess) return FP4_ERR_HIP;
  }
  return fp4_quantize(cfg, x, xdt, rows, cols, ldx, codes, scales, global_scale, gs_mode, ws,
                      kScratchBytes, stream);
}
