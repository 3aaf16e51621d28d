// mxfp4_quant: standalone per-1x32 MXFP4 quantisation of a bf16 matrix
// (kernelbot amd-mxfp4-mm submission 683203, ``_quant_shuffled``: a tile of A
// in, fp4x2 codes and E8M0 bytes out, with row tails masked; here scales are
// stored row-major). A lane quad quantises one 32-element block with the
// register routine the fused GEMM uses (quant8_quad, with the full zero-block
// rule): lane 4b + p holds elements 8p .. 8p+7 of block b, so a wave reads 16
// consecutive blocks, 1 KB, with one 16-byte load per lane.
#include "host_common.hpp"
#include "mx_device.hpp"

namespace {

struct QuantArgs {
  const uint16_t* x;
  int64_t ldx;
  uint8_t* q;
  int64_t ldq;
  uint8_t* s;
  int64_t lds;
  int64_t M;
  int64_t G;  // blocks per row, K/32
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void quant_kernel(QuantArgs a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = t >> 2;  // block; whole quads leave together (256 % 4 == 0)
  if (b >= a.M * a.G) return;
  const int part = (int)(t & 3);
  const int64_t r = b / a.G, g = b - r * a.G;
  // Read once and written once: non-temporal (streaming) loads and stores.
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.x + r * a.ldx + 32 * g + 8 * part));
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t sb;
  const uint32_t codes = mx::quant8_quad<true>(w, sb);
  __builtin_nontemporal_store(codes, reinterpret_cast<uint32_t*>(a.q + r * a.ldq + 16 * g + 4 * part));
  if (part == 0) __builtin_nontemporal_store((uint8_t)sb, a.s + r * a.lds + g);
}


// The same with 32-bit indices (M * K/8 < 2^31) and two units per thread, 256
// threads apart: both 16-byte loads are issued before either block is
// quantised, so each wave keeps 2 KB in flight. Past the end the load index is
// clamped to the last unit (read, never stored). Measured at M4096 K7168:
// 14.4-14.5 us against 16.1-16.2 us for one unit per thread with 64-bit indices.
constexpr int kQuantUnits = 2;
__global__ __launch_bounds__(256) void quant_kernel_u32(QuantArgs a) {
  const uint32_t n = (uint32_t)(a.M * a.G * 4), G = (uint32_t)a.G;
  const uint32_t t0 = blockIdx.x * (256u * kQuantUnits) + threadIdx.x;
  u32x4 v[kQuantUnits];
  uint32_t rr[kQuantUnits], gg[kQuantUnits];
#pragma unroll
  for (int i = 0; i < kQuantUnits; ++i) {
    const uint32_t t = min(t0 + 256u * i, n - 1);
    const uint32_t b = t >> 2, part = t & 3;
    rr[i] = b / G;
    gg[i] = b - rr[i] * G;
    v[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(a.x + (int64_t)rr[i] * a.ldx + 32 * gg[i] + 8 * part));
  }
#pragma unroll
  for (int i = 0; i < kQuantUnits; ++i) {
    // Every lane of a quad runs the quantisation (it exchanges values within
    // the quad); whole quads are past the end together, since n % 4 == 0.
    const uint32_t t = t0 + 256u * i, part = t & 3;
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    uint32_t sb;
    const uint32_t codes = mx::quant8_quad<true>(w, sb);
    if (t < n) {
      __builtin_nontemporal_store(codes,
                                  reinterpret_cast<uint32_t*>(a.q + (int64_t)rr[i] * a.ldq + 16 * gg[i] + 4 * part));
      if (part == 0) __builtin_nontemporal_store((uint8_t)sb, a.s + (int64_t)rr[i] * a.lds + gg[i]);
    }
  }
}

}  // namespace

extern "C" const char* mxfp4_status_str(int status) {
  switch (status) {
    case MXFP4_OK: return "MXFP4_OK";
    case MXFP4_ERR_NULL: return "MXFP4_ERR_NULL: a required pointer is NULL";
    case MXFP4_ERR_SHAPE: return "MXFP4_ERR_SHAPE: bad M/N/K or row stride";
    case MXFP4_ERR_ALIGN: return "MXFP4_ERR_ALIGN: pointer or row stride not suitably aligned";
    case MXFP4_ERR_WORKSPACE: return "MXFP4_ERR_WORKSPACE: workspace missing or too small";
    case MXFP4_ERR_TOO_MANY_GROUPS: return "MXFP4_ERR_TOO_MANY_GROUPS: G outside [1, MXFP4_MAX_GROUPS]";
    case MXFP4_ERR_HIP: return "MXFP4_ERR_HIP: the HIP runtime rejected a launch";
    case MXFP4_ERR_BUFFER: return "MXFP4_ERR_BUFFER: output buffer too small";
    case MXFP4_ERR_ARG: return "MXFP4_ERR_ARG: a scalar argument is out of range";
    default: return "unknown mxfp4 status";
  }
}

extern "C" int mxfp4_quant(const void* x, int64_t ldx, void* q, int64_t ldq, void* s, int64_t lds, int64_t M,
                           int64_t K, void* stream) {
  if (!x || !q || !s) return MXFP4_ERR_NULL;
  if (M < 1 || K < 32 || K % 32 != 0 || M > mxh::kMaxDim || K > mxh::kMaxDim) return MXFP4_ERR_SHAPE;
  if (ldx < K || ldq < K / 2 || lds < K / 32) return MXFP4_ERR_SHAPE;
  if (!mxh::aligned(x, 16) || (ldx * 2) % 16 != 0 || !mxh::aligned(q, 16) || ldq % 16 != 0) return MXFP4_ERR_ALIGN;
  QuantArgs a{(const uint16_t*)x, ldx, (uint8_t*)q, ldq, (uint8_t*)s, lds, M, K / 32};
  const int64_t n = M * (K / 32) * 4;  // four lanes per block
  if (mxh::cdiv(n, 256) > INT32_MAX) return MXFP4_ERR_SHAPE;  // grid size limit
  void* args[] = {&a};
  if (n < ((int64_t)1 << 31))
    return mxh::launch_status(hipLaunchKernel((const void*)quant_kernel_u32,
                                              dim3((unsigned)mxh::cdiv(n, 256 * kQuantUnits)), dim3(256), args, 0,
                                              (hipStream_t)stream));
  return mxh::launch_status(hipLaunchKernel((const void*)quant_kernel, dim3((unsigned)mxh::cdiv(n, 256)), dim3(256),
                                            args, 0, (hipStream_t)stream));
}
