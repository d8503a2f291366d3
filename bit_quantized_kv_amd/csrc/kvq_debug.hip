// kvq_debug.hip -- the optional checks of device index arrays (environment
// variable KVQ_DEBUG=1).  Without them an out-of-range slot, page id or
// sequence length is undefined behaviour, as an out-of-bounds index would be;
// with them the entry point first runs one of the kernels below over the
// array, waits for the stream, and returns an error instead of launching its
// kernels when any entry is out of range.
#include <algorithm>
#include <mutex>

#include "kvq_debug.h"
#include "kvq_device.h"

namespace kvq {

// The result word: one copy per device, held until the process ends.  Host
// code never passes the word's name to a kernel (on the host it is a
// stand-in for the symbol) but the device address hipGetSymbolAddress
// returns, looked up once per device.  Calls that overlap on one device share
// the word; debug mode serialises each call on its stream, so calls from one
// thread on one device are ordered.
static __device__ __align__(16) uint32_t debug_word;

__global__ void debug_clear_kernel(uint32_t* w) {
  if (threadIdx.x == 0 && blockIdx.x == 0) w[0] = 0u;
}

// A write slot must address a row of the pool: slot < num_pages * page_size
// (a negative slot skips its token and is valid).
__global__ __launch_bounds__(256) void debug_slots_kernel(const int32_t* __restrict__ slots, int64_t n,
                                                          int64_t limit, uint32_t* w) {
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    bad |= slots[i] >= limit;
  if (bad) atomicOr(w, kDebugBadSlot);
}

// One workgroup per page-table row b: the row's sequence length (lens[b], or
// len for every row when lens is null) must lie in [0, max_len], and the page
// ids the length uses -- the row's first ceil(length / page_size) entries --
// in [0, num_pages).  A length past max_len is scanned up to max_len only,
// the entries the host's shape checks guarantee to exist.
__global__ __launch_bounds__(256) void debug_pages_kernel(const int32_t* __restrict__ table, int64_t row_stride,
                                                          const int32_t* __restrict__ lens, int32_t len,
                                                          int32_t max_len, int32_t page_size, int32_t num_pages,
                                                          uint32_t* w) {
  const int64_t b = blockIdx.x;
  int32_t L = lens != nullptr ? lens[b] : len;
  uint32_t bad = 0u;
  if (L < 0 || L > max_len) {
    bad |= kDebugBadLength;
    L = L < 0 ? 0 : max_len;
  }
  const int32_t np = (int32_t)(((int64_t)L + page_size - 1) / page_size);
  for (int32_t i = threadIdx.x; i < np; i += 256) {
    const int32_t pg = table[b * row_stride + i];
    if (pg < 0 || pg >= num_pages) bad |= kDebugBadPage;
  }
  if (bad != 0u) atomicOr(w, bad);
}

static hipError_t debug_word_ptr(uint32_t** ptr) {
  constexpr int kDevices = 64;
  static std::mutex mu;
  static void* addr[kDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(debug_word));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = (uint32_t*)addr[dev];
  return hipSuccess;
}

// clear the word, run the check, copy the word back and wait for it
template <typename Launch>
static hipError_t debug_run(hipStream_t stream, uint32_t* bits, Launch launch) {
  *bits = 0u;
  uint32_t* w = nullptr;
  hipError_t e = debug_word_ptr(&w);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(debug_clear_kernel, dim3(1), dim3(64), 0, stream, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  launch(w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  uint32_t host = 0u;
  if ((e = hipMemcpyAsync(&host, w, sizeof(host), hipMemcpyDeviceToHost, stream)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
  *bits = host;
  return hipSuccess;
}

hipError_t debug_check_slots(const int32_t* slots, int64_t n, int64_t limit, hipStream_t stream, uint32_t* bits) {
  const int64_t blocks = std::min((n + 255) / 256, (int64_t)4096);
  return debug_run(stream, bits, [&](uint32_t* w) {
    hipLaunchKernelGGL(debug_slots_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, slots, n, limit, w);
  });
}

hipError_t debug_check_pages(const int32_t* table, int64_t row_stride, int32_t rows, const int32_t* lens,
                             int32_t len, int32_t max_len, int32_t page_size, int32_t num_pages, hipStream_t stream,
                             uint32_t* bits) {
  return debug_run(stream, bits, [&](uint32_t* w) {
    hipLaunchKernelGGL(debug_pages_kernel, dim3((unsigned)rows), dim3(256), 0, stream, table, row_stride, lens, len,
                       max_len, page_size, num_pages, w);
  });
}

}  // namespace kvq
