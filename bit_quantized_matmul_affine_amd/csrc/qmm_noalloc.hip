// qmm_noalloc.hip -- qmm_run_noalloc: qmm_run for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops and
// harnesses that forbid hipMalloc).  The split-K workspace (ticket words,
// then partial tiles) comes from `scratch`, a fixed device array of the
// library, instead of from the caller.
//
// Each device holds its own copy of `scratch` (at its own address) from the
// moment the code object is loaded on it until the process ends.  Host code
// never uses the array's name as an address: on the first call on a device,
// with that device current, hipGetSymbolAddress gives the device address,
// which is kept per device and passed to the kernels like any workspace.
// The array is zero when loaded; the same first call also clears its ticket
// words with a small kernel on the caller's stream (a kernel, not a memset,
// so the clearing may itself be captured into a graph); every completed
// call leaves the ticket words at zero again.  Calls that overlap in time on
// one device share the array and race: the caller orders them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/qmm.h"
#include "qmm_internal.h"

namespace qmm {
qmm_status set_error(qmm_status st, const char* msg);
}

namespace {

constexpr size_t kScratchBytes = QMM_NOALLOC_MAX_WORKSPACE;
constexpr size_t kTicketClearBytes = 256 * 1024;  // ticket words of up to 2^20 output columns
static_assert(kTicketClearBytes <= kScratchBytes, "ticket area inside the array");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchAddr {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchAddr g_scratch[kMaxDevices];

__global__ void __launch_bounds__(256) clear_words(uint32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace

extern "C" qmm_status qmm_run_noalloc(const qmm_plan* plan, const void* x, const void* codes,
                                      const void* sb, void* y, int32_t rows, void* stream) {
  if (!plan) return qmm::set_error(QMM_ERR_INVALID_ARG, "plan is NULL");
  // what qmm_run needs for the family it picks (0 for rows outside the
  // plan's range: qmm_run reports that below)
  const size_t need = qmm_workspace_bytes_ex(plan, QMM_VARIANT_AUTO, 0, 0, 0, rows);
  if (need > kScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof msg,
             "this call needs %zu bytes of workspace; qmm_run_noalloc holds %zu (use qmm_run)",
             need, kScratchBytes);
    return qmm::set_error(QMM_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  if (need > 0) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
      return qmm::set_error(e == hipErrorNoDevice ? QMM_ERR_NO_DEVICE : QMM_ERR_HIP,
                            "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices)
      return qmm::set_error(QMM_ERR_UNSUPPORTED, "device index beyond the library's table");
    ScratchAddr& s = g_scratch[dev];
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    std::call_once(s.once, [&] {
      void* p = nullptr;
      s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (s.err == hipSuccess && p) {
        const int words = (int)(kTicketClearBytes / 4);
        clear_words<<<words / 256 / 16, 256, 0, st>>>(static_cast<uint32_t*>(p), words);
        s.err = hipGetLastError();
      }
      if (s.err == hipSuccess) s.ptr = p;
    });
    if (s.err != hipSuccess || !s.ptr)
      return qmm::set_error(QMM_ERR_HIP, "the workspace array's device address is unavailable");
    ws = s.ptr;
  }
  return qmm_run(plan, x, codes, sb, y, rows, ws, need > 0 ? kScratchBytes : 0, stream);
}
