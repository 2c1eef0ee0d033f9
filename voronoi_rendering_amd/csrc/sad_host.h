// sad_host.h -- argument checks and launch helpers of the C ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sad.h"

namespace sad {

constexpr int64_t MAX_SITES = int64_t(1) << 30;
constexpr int32_t MAX_SIDE = 1 << 15;
constexpr int64_t MAX_TILES = int64_t(1) << 26;
constexpr int64_t MAX_QUERIES = int64_t(1) << 40;
constexpr int64_t QUERY_CHUNK = int64_t(1) << 30;  // points per query launch

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// p must be non-NULL and a-aligned unless the array is empty.
inline bool array_ok(const void* p, int64_t count, uintptr_t a) {
    if (count == 0) return true;
    return p != nullptr && aligned(p, a);
}

inline bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    if (!a || !b || abytes == 0 || bbytes == 0) return false;
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

inline bool sites_ok(int32_t n) { return n >= 0 && n <= MAX_SITES; }
inline bool image_ok(int32_t h, int32_t w) { return h >= 0 && w >= 0 && h <= MAX_SIDE && w <= MAX_SIDE; }

inline int tiles_x(int32_t w) { return (w + SAD_TILE - 1) / SAD_TILE; }
inline int tiles_y(int32_t h) { return (h + SAD_TILE - 1) / SAD_TILE; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Clear a stale error left by earlier, unrelated runtime calls so that a
// failed launch is reported by the call that made it.
inline void clear_error() { (void)hipGetLastError(); }

inline int launch_status() { return hipGetLastError() == hipSuccess ? SAD_OK : SAD_EHIP; }

}  // namespace sad
