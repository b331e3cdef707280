// The transpose's entry point for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the same kernels as spgemm_transpose, with their temporaries
// carved from one fixed device array instead of a hipMallocAsync block.
//
// The array is a file-scope __device__ object, so every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  In
// host code the array's name is only a stand-in: its device address is
// looked up once per device with hipGetSymbolAddress, and only that address
// is handed to kernels.  Calls on one device share the array and keep the
// last call's contents; everything that must start at zero is cleared by a
// kernel on the caller's stream, so calls in stream order are safe, and
// calls that overlap on one device (different streams, or host threads)
// race on it.
#include <mutex>

#include "../../include/spgemm.h"
#include "internal.hpp"

namespace {

constexpr int64_t kScratchBytes = int64_t(64) << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's `scratch`, looked up on first use with the
// device current; null if the lookup failed.
char* scratch_address(int device) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[device] = (char*)p;
  }
  return g_scratch_ptr[device];
}

}  // namespace

extern "C" spgemm_status spgemm_transpose_noalloc(int64_t m, int64_t n, int64_t nnz,
                                                  const void* dA_row_ptr, int32_t a_rowptr64,
                                                  const int32_t* dA_col, const void* dA_val,
                                                  spgemm_dtype dtype, void* dT_row_ptr,
                                                  int32_t t_rowptr64, int32_t* dT_col,
                                                  void* dT_val, void* stream) {
  spgemm_status st = sg::transpose_check_args(m, n, nnz, dA_row_ptr, dA_col, dA_val, dtype,
                                              dT_row_ptr, t_rowptr64, dT_col, dT_val);
  if (st != SPGEMM_OK) return st;
  const int64_t need = sg::transpose_workspace_bytes(n, nnz, dtype, dA_val != nullptr);
  if (need > kScratchBytes) {
    sg::set_thread_error(
        "the transpose needs more workspace than the 64 MiB scratch array of "
        "spgemm_transpose_noalloc holds; call spgemm_transpose");
    return SPGEMM_ERR_INVALID_ARG;
  }
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= kMaxDevices) {
    (void)hipGetLastError();
    sg::set_thread_error("no usable current device");
    return SPGEMM_ERR_HIP;
  }
  char* ws = scratch_address(device);
  if (!ws) {
    sg::set_thread_error("hipGetSymbolAddress of the scratch array failed");
    return SPGEMM_ERR_HIP;
  }
  return sg::transpose_run(m, n, nnz, dA_row_ptr, a_rowptr64, dA_col, dA_val, dtype,
                           dT_row_ptr, t_rowptr64, dT_col, dT_val, ws, (hipStream_t)stream);
}

