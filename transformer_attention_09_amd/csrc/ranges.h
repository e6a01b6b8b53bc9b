// Byte ranges of raw buffer resources (plain arithmetic, usable on the host).
//
// A buffer resource carries a 32-bit byte range: loads at or past it return
// zeros and stores there are dropped, which is how the kernels mask rows past
// the end of a tensor without branches.  Every per-lane byte offset inside
// one resource stays below 2^31 (a tile or a 128-row block of one head), so a
// range of 2^31 bytes or more is saturated to 2^31 - 1: the clamp hides
// nothing a lane can address.  Narrowing such a range to 32 bits instead
// would wrap it (a 4 GiB range becomes 0) and turn real rows into zeros.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace attn {

constexpr uint32_t kMaxRange = 0x7fffffffu;

// A byte count saturated to what the resource's range field is used for.
constexpr uint32_t rsrc_range(size_t bytes) { return bytes > kMaxRange ? kMaxRange : (uint32_t)bytes; }

// Range of a resource based at the first element of one row of a strided
// [rows][stride] layout, covering n_rows rows of row_elems elements each (the
// last row ends after its own elements, not after the stride).  n_rows <= 0
// gives an empty range.
constexpr uint32_t rows_range(long long n_rows, size_t stride_elems, size_t row_elems, size_t elem_bytes) {
  return n_rows <= 0 ? 0u : rsrc_range((((size_t)n_rows - 1) * stride_elems + row_elems) * elem_bytes);
}

}  // namespace attn
