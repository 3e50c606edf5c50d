// split.hpp -- key-range split arithmetic shared by the scan kernels and
// their host launchers.  Plain C++ with no HIP dependency: constexpr
// functions are callable from device code as well, and a host-only unit
// check compiles this header with g++.
#pragma once

#include <stdint.h>

namespace ltk {

struct KeyRange {
    int32_t lo, hi;   // [lo, hi): empty when lo == hi
};

// Range of split s of n over the keys [0, end), each split a whole number
// of `tile` keys (the last one ragged, trailing splits possibly empty).
// Computed in 64 bits: with end close to 2^31 and up to 4,096 splits of
// 512-key tiles, the int32 forms of split * per or end + n - 1 would wrap.
constexpr KeyRange split_range(int64_t end, int64_t n, int64_t s, int64_t tile) {
    const int64_t per = ((end + n - 1) / n + tile - 1) / tile * tile;
    const int64_t lo = s * per < end ? s * per : end;
    const int64_t hi = lo + per < end ? lo + per : end;
    return KeyRange{(int32_t)lo, (int32_t)hi};
}

// Whole tiles of `tile` keys starting at key0 lie inside [0, L): the 64-bit
// form of key0 + tile <= L.
constexpr bool tile_inside(int64_t key0, int64_t tile, int64_t L) { return key0 + tile <= L; }

}  // namespace ltk
