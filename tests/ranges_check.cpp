// Host check of the buffer-resource range arithmetic (csrc/ranges.h).
// Prints one line per case: "ok <name>" or "FAIL <name> ...", exit status 0
// only if every case holds.
#include <cstdio>
#include <cstdint>

#include "ranges.h"

static int fails = 0;
static void expect(const char* name, bool ok, unsigned long long got, unsigned long long want) {
  if (ok) std::printf("ok %s\n", name);
  else { std::printf("FAIL %s got %llu want %llu\n", name, got, want); ++fails; }
}

int main() {
  using attn::rows_range;
  using attn::rsrc_range;
  // 3 rows of 128 bf16 elements at a stride of 4 heads: (2 * 512 + 128) * 2 bytes
  expect("small", rows_range(3, 512, 128, 2) == 2304u, rows_range(3, 512, 128, 2), 2304u);
  expect("one row", rows_range(1, 4096, 64, 2) == 128u, rows_range(1, 4096, 64, 2), 128u);
  expect("no rows", rows_range(0, 4096, 64, 2) == 0u, rows_range(0, 4096, 64, 2), 0u);
  expect("negative rows", rows_range(-5, 4096, 64, 2) == 0u, rows_range(-5, 4096, 64, 2), 0u);
  expect("saturate exact", rsrc_range(0x7fffffffull) == 0x7fffffffu, rsrc_range(0x7fffffffull), 0x7fffffffu);
  expect("saturate above", rsrc_range(0x80000000ull) == 0x7fffffffu, rsrc_range(0x80000000ull), 0x7fffffffu);
  // A query block whose remaining rows span 2^32 + 256 bytes (Lq = 131073,
  // Hq = 128, D = 128, 16-bit): narrowing would give 256 bytes and zero every
  // row after the first; the saturated range keeps all 128 rows of the block
  // (the farthest byte a lane of the block reads lies below 4 MiB).
  const long long Lq = 131073, Hq = 128, D = 128;
  const unsigned long long raw = ((unsigned long long)(Lq - 1) * Hq * D + D) * 2;
  expect("wide raw value", raw == (1ull << 32) + 256, raw, (1ull << 32) + 256);
  expect("wide narrowing wraps", (uint32_t)raw == 256u, (uint32_t)raw, 256u);
  const uint32_t r = rows_range(Lq, (size_t)(Hq * D), (size_t)D, 2);
  expect("wide saturates", r == 0x7fffffffu, r, 0x7fffffffu);
  const unsigned long long last_byte = ((127ull * Hq * D) + D) * 2;  // end of row 127 of the block
  expect("block rows inside range", last_byte <= r, last_byte, r);
  // The last q-block of that tensor (q0 = 131072: one row left) is exact.
  const uint32_t t = rows_range(Lq - 131072, (size_t)(Hq * D), (size_t)D, 2);
  expect("tail block exact", t == 256u, t, 256u);
  return fails == 0 ? 0 : 1;
}
