// Clamps for the caller's tables that kernels read on the device (packed-sequence
// offsets, paged-cache lengths and page numbers).  A table that breaks its documented
// form cannot be rejected on the host without a copy back, so every kernel maps each
// value it reads into the range the buffers allow: a malformed table then gives
// meaningless results but no access outside the caller's buffers.  A well-formed
// table passes through unchanged.
//
// Plain constexpr functions, so device code (where clang treats constexpr functions
// as host-and-device) and host-side tests use the same definitions.
#pragma once
#include <stdint.h>

namespace msa {

constexpr int64_t clamp_i64(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Sequence s of a packed batch of T tokens, read as a = cu[s], b = cu[s + 1]: the
// start is clamped into [0, T] and the end into [start, T], so the span's rows are
// rows of the buffers.
struct PackedSpan {
  int64_t start, len;
};
constexpr PackedSpan packed_span(int64_t a, int64_t b, int64_t T) {
  return PackedSpan{clamp_i64(a, 0, T), clamp_i64(b, clamp_i64(a, 0, T), T) - clamp_i64(a, 0, T)};
}

// Entry s (0 <= s <= batch) of a sanitised offset table, given pmax = max(cu[0..s]):
// 0 at s = 0, T at s = batch, else the running maximum clamped into [0, T].  The
// result is non-decreasing, and its sequences partition [0, T) (every token belongs to
// exactly one sequence), whatever the raw table holds.
constexpr int64_t sanitized_offset(int64_t pmax, int64_t s, int64_t batch, int64_t T) {
  return s == 0 ? 0 : (s == batch ? T : clamp_i64(pmax, 0, T));
}

// Paged cache: a length clamped into [0, max_blocks * page_tokens] (the table row
// holds max_blocks pages), and a page number clamped into [0, num_pages - 1].
constexpr int64_t paged_len(int64_t raw, int64_t max_blocks, int64_t page_tokens) {
  return clamp_i64(raw, 0, max_blocks * page_tokens);
}
constexpr int64_t page_number(int64_t raw, int64_t num_pages) { return clamp_i64(raw, 0, num_pages - 1); }

}  // namespace msa
