// Host-side helpers shared by the entry points: argument checks that run before
// any HIP call, and launch-status mapping.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mxfp4.h"

namespace mxh {

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // M, N, K limit: 32-bit index math with headroom

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int launch_status(hipError_t e) { return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP; }

// Packed-B geometry (see mxfp4_pack_B in include/mxfp4.h): 1 KB units of
// 32 columns x 64 k, NT = ceil(N/32) column tiles, KU = ceil(K/64) k units,
// KG = ceil(KU/4) scale groups.
struct PackedGeom {
  int64_t NT, KU, KG;
  size_t code_bytes, scale_bytes;
  PackedGeom(int64_t N, int64_t K)
      : NT(cdiv(N, 32)), KU(cdiv(K, 64)), KG(cdiv(cdiv(K, 64), 4)),
        code_bytes((size_t)(cdiv(N, 32) * cdiv(K, 64)) * 1024u),
        scale_bytes((size_t)(cdiv(N, 32) * cdiv(cdiv(K, 64), 4)) * 256u) {}
  size_t total() const { return code_bytes + scale_bytes; }
};

}  // namespace mxh
