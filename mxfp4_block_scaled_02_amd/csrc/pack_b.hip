// mxfp4_pack_B: offline repacking of a quantised weight B[N, K] (fp4x2 codes +
// E8M0 scales, row-major) into MFMA-fragment order. The idea follows kernelbot
// amd-mxfp4-mm submission 683203 (docstring trick 1 and ``_quant_shuffled``:
// scales stored at permuted offsets so each wave's lanes fetch theirs with one
// coalesced load; byte 127 as the neutral pad) and kernelbot nvfp4-group-gemm
// submission 496271 (``_prepare_scale_for_tma``: scales pre-arranged in the
// matrix instruction's order). The layout itself is this library's: every 32x64
// block of B is the exact 1 KB operand of one scaled 32x32x64 FP4 MFMA, in lane
// order (lane l: column l%32, k-chunk l/32), and the scale bytes of four
// consecutive k units of a lane share one dword. The same units serve the
// 16x16x128 instruction: its operand for 16 columns x 128 k is four 256-byte
// runs of two consecutive units.
#include "host_common.hpp"
#include "mx_device.hpp"

namespace {

struct PackArgs {
  const uint8_t* bq;
  const uint8_t* bs;
  uint8_t* out;
  int64_t N, K, NT, KU, KG;
};

// One thread per 16-byte lane slot of a code unit: unit (t, u), lane l holds
// row 32t + l%32 of B, elements k = 64u + 32(l/32) .. +31.
__global__ __launch_bounds__(256) void pack_codes_kernel(PackArgs a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.NT * a.KU * 64) return;
  const int l = (int)(t & 63);
  const int64_t f = t >> 6, u = f % a.KU, tt = f / a.KU;
  const int64_t n = 32 * tt + (l & 31), k0 = 64 * u + 32 * (l >> 5);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (n < a.N && k0 < a.K) v = mx::ldg16(a.bq + n * (a.K / 2) + k0 / 2);
  *reinterpret_cast<uint4*>(a.out + t * 16) = v;
}

// One thread per scale dword (t, g, l): byte i = scale of row 32t + l%32,
// 32-element chunk 2(4g+i) + l/32.
__global__ __launch_bounds__(256) void pack_scales_kernel(PackArgs a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.NT * a.KG * 64) return;
  const int l = (int)(t & 63);
  const int64_t f = t >> 6, g = f % a.KG, tt = f / a.KG;
  const int64_t n = 32 * tt + (l & 31), nchunk = a.K / 32;
  uint32_t d = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t kc = 2 * (4 * g + i) + (l >> 5);
    const uint32_t b = (n < a.N && kc < nchunk) ? a.bs[n * nchunk + kc] : mx::kScaleOne;
    d |= b << (8 * i);
  }
  reinterpret_cast<uint32_t*>(a.out + a.NT * a.KU * 1024)[t] = d;
}

}  // namespace

extern "C" size_t mxfp4_pack_B_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 32 || K % 32 != 0 || N > mxh::kMaxDim || K > mxh::kMaxDim) return 0;
  return mxh::PackedGeom(N, K).total();
}

extern "C" int mxfp4_pack_B(const void* bq, const void* bs, int64_t N, int64_t K, void* out, size_t out_bytes,
                            void* stream) {
  if (!bq || !bs || !out) return MXFP4_ERR_NULL;
  if (N < 1 || K < 32 || K % 32 != 0 || N > mxh::kMaxDim || K > mxh::kMaxDim) return MXFP4_ERR_SHAPE;
  if (!mxh::aligned(bq, 16) || !mxh::aligned(out, 16)) return MXFP4_ERR_ALIGN;
  const mxh::PackedGeom g(N, K);
  if (out_bytes < g.total()) return MXFP4_ERR_BUFFER;
  PackArgs a{(const uint8_t*)bq, (const uint8_t*)bs, (uint8_t*)out, N, K, g.NT, g.KU, g.KG};
  void* args[] = {&a};
  const int64_t n1 = g.NT * g.KU * 64, n2 = g.NT * g.KG * 64;
  if (mxh::cdiv(n1, 256) > INT32_MAX) return MXFP4_ERR_SHAPE;  // grid size limit (n2 <= n1)
  hipError_t e = hipLaunchKernel((const void*)pack_codes_kernel, dim3((unsigned)mxh::cdiv(n1, 256)), dim3(256), args,
                                 0, (hipStream_t)stream);
  if (e != hipSuccess) return MXFP4_ERR_HIP;
  e = hipLaunchKernel((const void*)pack_scales_kernel, dim3((unsigned)mxh::cdiv(n2, 256)), dim3(256), args, 0,
                      (hipStream_t)stream);
  return mxh::launch_status(e);
}
