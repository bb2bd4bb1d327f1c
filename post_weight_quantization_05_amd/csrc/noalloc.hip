// gptq_hessian_accumulate_noalloc: the Hessian accumulation with its scratch in a static device array,
// for callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The scratch holds the split-K partials of gptq_hessian_accumulate (fp32 tile sums of each row slice and
// fp64 column sums of squares). Every partial is written before it is read within one call, so nothing
// needs clearing. The array lives in this file's device code; each GPU the library runs on holds its own
// copy from the first use until the process ends. Host code never passes the array's name to a kernel:
// it looks up the device address once per device with hipGetSymbolAddress and uses that pointer.
#include <mutex>

#include "common.h"

namespace {

constexpr size_t SCRATCH_BYTES = (size_t)80 << 20;  // 80 MiB: in <= 4096 (bf16) with two row slices
constexpr int MAX_DEVICES = 64;

static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

std::mutex g_lock;
void* g_scratch[MAX_DEVICES] = {};  // device address of `scratch` on each device, once looked up

// The calling thread's current device's copy of the array, or nullptr on failure.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> hold(g_lock);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int gptq_hessian_accumulate_noalloc(const void* X, int x_dtype, int64_t n_rows, int64_t in, int64_t ld_x,
                                    double* S, double* colsq, int64_t* n_total, void* stream) {
  using namespace gptq;
  if (!X || !S || !colsq || !n_total) return GPTQ_ERR_INVALID_ARG;
  if (x_dtype != GPTQ_F32 && x_dtype != GPTQ_BF16) return GPTQ_ERR_INVALID_ARG;
  if (n_rows < 1 || in < 1 || in > 65536 || ld_x < in || *n_total < 0) return GPTQ_ERR_INVALID_ARG;
  HessianPlan p = hessian_plan(n_rows, in, x_dtype, SCRATCH_BYTES);
  if (p.total_bytes > SCRATCH_BYTES) return GPTQ_ERR_UNSUPPORTED;  // even one row slice does not fit
  p.ld = ld_x;
  void* ws = scratch_on_current_device();
  if (!ws) return GPTQ_ERR_HIP;
  const hipError_t e = hessian_launch(p, X, S, colsq, ws, reinterpret_cast<hipStream_t>(stream), *n_total == 0);
  if (e != hipSuccess) return GPTQ_ERR_HIP;
  *n_total += n_rows;
  return GPTQ_OK;
}

}  // extern "C"
