// sv_host.h -- host-side argument checks shared by the library's entry
// points.
#pragma once

#include <stdint.h>

namespace sv {
// Whether every byte offset of a strided array,
// sum of (count_i - 1) * stride_i over three dimensions plus `len` bytes of
// the last item (strides and len in bytes, non-negative), stays below 2^62,
// so that device address arithmetic in 64-bit integers never overflows.
// An empty dimension (count 0) makes the array empty and always fits.
inline bool span_fits(int64_t n0, int64_t s0, int64_t n1, int64_t s1, int64_t n2, int64_t s2, int64_t len)
{
    if (n0 <= 0 || n1 <= 0 || n2 <= 0 || len <= 0) return true;
    const __int128 end = (__int128)(n0 - 1) * s0 + (__int128)(n1 - 1) * s1 + (__int128)(n2 - 1) * s2 + len;
    return s0 >= 0 && s1 >= 0 && s2 >= 0 && end < ((__int128)1 << 62);
}

}  // namespace sv
