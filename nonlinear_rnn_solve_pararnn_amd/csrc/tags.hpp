// tags.hpp -- arithmetic of the launch epochs and tags that the look-back
// records carry (common.hpp), host- and device-callable so that a host
// program can check it.
//
// A workspace's ticket header holds two 64-bit words:
//   word 0: tickets drawn in the current launch (low half) and the launch
//           epoch (high half), 0 <= epoch < kTagPeriod;
//   word 1: in the last launch of a period, the workgroups that have
//           finished (zero otherwise).
// Each launch that draws tickets tags its records with launch_tag(epoch).
// The launch that uses the last tag of a period clears the whole workspace
// (but the header and the range the call still needs) when its last
// workgroup finishes, and the next launch starts the next period at epoch 0.
// So every tagged word in a workspace was written in the current period, in
// which no two launches share a tag: a record can only match the tag of the
// launch that wrote it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prn {

// Tags are signalling-NaN bit patterns (exponent all ones, quiet bit clear,
// non-zero mantissa; both signs), which arithmetic never produces, so a
// float that another entry point left in the workspace cannot look like one.
constexpr uint32_t kTagHalf = 0x3fffffu;
constexpr uint32_t kTagPeriod = 2u * kTagHalf;
// Words of the ticket header.
constexpr uint64_t kHeaderWords = 2;

__host__ __device__ constexpr uint32_t launch_tag(uint32_t epoch) {
    return epoch < kTagHalf ? 0x7f800001u + epoch : 0xff800001u + (epoch - kTagHalf);
}

// Epoch of the launch after one at `epoch` (0 after the last of a period).
__host__ __device__ constexpr uint32_t next_epoch(uint32_t epoch, uint32_t period = kTagPeriod) {
    return epoch + 1u >= period ? 0u : epoch + 1u;
}

// Whether the launch at `epoch` is the last of its period: its workgroups
// count themselves out and the last one clears the workspace.
__host__ __device__ constexpr bool is_wrap_launch(uint32_t epoch, uint32_t period = kTagPeriod) {
    return next_epoch(epoch, period) == 0u;
}

// Header word 0 after a draw that returned count `idx` of a launch of
// `draws` tickets at `epoch`: the last draw resets the count and advances
// the epoch; any other draw leaves the incremented word.
__host__ __device__ constexpr uint64_t header_after_draw(uint32_t idx, uint32_t epoch, uint32_t draws,
                                                         uint32_t period = kTagPeriod) {
    return idx + 1u == draws ? (uint64_t)next_epoch(epoch, period) << 32
                             : ((uint64_t)epoch << 32) | (uint64_t)(idx + 1u);
}

// The two word ranges [lo0, hi0) and [lo1, hi1) that the clear of a
// workspace of `words` 64-bit words writes: everything past the header
// except [keep_lo, keep_hi) (an empty keep range when keep_lo >= keep_hi).
struct ClearRanges {
    uint64_t lo0, hi0, lo1, hi1;
};
__host__ __device__ constexpr uint64_t clamp_words(uint64_t x, uint64_t lo, uint64_t hi) {
    return x < lo ? lo : (x > hi ? hi : x);
}
__host__ __device__ constexpr ClearRanges clear_ranges(uint64_t words, uint64_t keep_lo, uint64_t keep_hi) {
    const uint64_t start = words < kHeaderWords ? words : kHeaderWords;
    if (keep_lo >= keep_hi) return {start, words, words, words};
    const uint64_t a = clamp_words(keep_lo, start, words), b = clamp_words(keep_hi, start, words);
    return {start, a, b, words};
}

}  // namespace prn
