// abi_sanitize_stubs.cpp -- host stand-ins for everything kvq_api.cpp calls
// below the C ABI (the kernel launchers, the static-scratch lookup, the
// debug-mode checks and the three HIP runtime queries), so that the argument
// validation can be built
// for the host alone with AddressSanitizer and UndefinedBehaviorSanitizer and
// run without a GPU (test infrastructure: tests/test_abi_sanitized.py).
// Each launcher records which kernel family was asked for; nothing runs.  The
// debug-mode checks record how often they ran and report the fault bits the
// driver sets in g_debug_bits.
#include <hip/hip_runtime.h>

#include "kvq_debug.h"
#include "kvq_launch.h"

int g_launch_count = 0;
int g_last_launch = 0;  // 1 store, 2 dequant, 3 amax, 4 global scale, 5 hadamard, 6 decode, 7 extend, 8 read,
                        // 9 write, 10 copy, 11 mfma rate

uint32_t g_debug_bits = 0;  // what the debug checks report
int g_debug_checks = 0;      // how many ran

namespace {
hipError_t record(int kind) {
  g_launch_count++;
  g_last_launch = kind;
  return hipSuccess;
}
}  // namespace

namespace kvq {
hipError_t launch_quantize_store(const StoreParams&, int, int, int, hipStream_t) { return record(1); }
hipError_t launch_dequant_prefix(const DequantParams&, int, int, hipStream_t) { return record(2); }
hipError_t launch_calibrate_amax(const StoreParams&, int, int, float*, hipStream_t) { return record(3); }
hipError_t launch_global_scale(const float*, float*, hipStream_t) { return record(4); }
hipError_t launch_hadamard(const RotateParams&, int, int, int, hipStream_t) { return record(5); }
hipError_t launch_decode(const DecodeParams& p, int, int, hipStream_t) {
  // the partials must lie inside the workspace the entry point was given
  return p.part_o != nullptr && p.part_ml != nullptr ? record(6) : hipErrorInvalidValue;
}
hipError_t launch_extend(const ExtendParams&, int, int, hipStream_t) { return record(7); }
hipError_t launch_stream_read(const void*, int64_t, uint32_t*, int, hipStream_t) { return record(8); }
hipError_t launch_stream_write(void*, int64_t, uint32_t, int, hipStream_t) { return record(9); }
hipError_t launch_stream_copy(const void*, void*, int64_t, int, hipStream_t) { return record(10); }
hipError_t launch_mfma_rate(int, int, int, uint32_t*, hipStream_t) { return record(11); }
hipError_t debug_check_slots(const int32_t* slots, int64_t n, int64_t limit, hipStream_t, uint32_t* bits) {
  g_debug_checks++;
  *bits = slots != nullptr && n > 0 && limit > 0 ? g_debug_bits : 0xFFFFFFFFu;
  return hipSuccess;
}
hipError_t debug_check_pages(const int32_t* table, int64_t, int32_t rows, const int32_t*, int32_t, int32_t max_len,
                             int32_t page_size, int32_t num_pages, hipStream_t, uint32_t* bits) {
  g_debug_checks++;
  *bits = table != nullptr && rows > 0 && max_len >= 0 && page_size > 0 && num_pages > 0 ? g_debug_bits : 0xFFFFFFFFu;
  return hipSuccess;
}
hipError_t decode_scratch(void** ptr) {
  *ptr = (void*)(uintptr_t)0x200000;  // a stand-in device address, never dereferenced
  return hipSuccess;
}
}  // namespace kvq

extern "C" {
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  *value = 256;  // MI355X compute units
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
}
