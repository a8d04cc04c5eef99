// Range limits of the attention kernel's direct-to-LDS tile loads. Plain C++
// (no HIP types), so host code and host-only tests can evaluate them too.
#pragma once

#include <stdint.h>

namespace dflash {

// A direct-to-LDS V^T load adds a 32-bit byte offset to a wave-uniform base.
// The largest offset a lane forms is that of swizzle row 15, chunk 15 of the
// transposed cache [D][ctx_total]:
//     (15 * ctx_total + 15 * elems_per_chunk) * elem_bytes,
// computed in uint32 arithmetic, so it must not exceed 2^32 - 1. This returns
// the largest ctx_total for which it does not; longer caches take the
// register-staged tile path.
constexpr int64_t vt_dma_max_ctx(int elem_bytes, int elems_per_chunk) {
    return ((int64_t)0xFFFFFFFF / elem_bytes - 15 * (int64_t)elems_per_chunk) / 15;
}

}  // namespace dflash
