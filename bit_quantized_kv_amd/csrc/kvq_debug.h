// kvq_debug.h -- the KVQ_DEBUG checks of device index arrays (kvq_debug.hip).
// Each check runs one kernel over the array on `stream`, waits for the stream
// and returns in *bits the union of the faults it found (0: none).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr uint32_t kDebugBadSlot = 1u;    // a write slot at or past num_pages * page_size
constexpr uint32_t kDebugBadPage = 2u;    // a page id the call reads outside [0, num_pages)
constexpr uint32_t kDebugBadLength = 4u;  // a sequence length outside [0, max_seq_len]

// slots[0 .. n): each below limit (negative: skipped, valid)
hipError_t debug_check_slots(const int32_t* slots, int64_t n, int64_t limit, hipStream_t stream, uint32_t* bits);

// rows page-table rows of row_stride entries: row b's length lens[b] (or len
// when lens is null) in [0, max_len], its first ceil(length / page_size)
// entries in [0, num_pages)
hipError_t debug_check_pages(const int32_t* table, int64_t row_stride, int32_t rows, const int32_t* lens,
                             int32_t len, int32_t max_len, int32_t page_size, int32_t num_pages, hipStream_t stream,
                             uint32_t* bits);

}  // namespace kvq
