// mxfp4_rmsnorm_quant: RMSNorm of each bf16 row, y = x / sqrt(mean(x^2) + eps) * w,
// followed by per-1x32 MXFP4 quantisation of y, in one launch (the fusion that
// kernelbot amd-mxfp4-mm submission 683203 names in its docstring, trick 1,
// without printing its arithmetic; the norm is the standard root-mean-square
// normalisation).
//
// One wave per row. Lane l takes the 8 elements k = 512c + 8l .. +7 of pass c,
// so a lane quad holds one 32-element block and one 16-byte load per lane per
// pass covers 1 KB of the row. Pass one sums the squares in float64, each lane
// in pass-then-element order, and the 64 lane sums meet in a halving tree
// (S[t] += S[t+s], s = 32 .. 1): a fixed order, so the result, and with it
// every quantised code, is the same on every run. inv = fp32(1 / sqrt(ss/K +
// eps)) with float64 steps; pass two forms y = bf16((x * inv) * w) in fp32 and
// quantises it with the lane-quad routine of the GEMM, storing codes and scale
// bytes row-major as mxfp4_quant does.
#include "host_common.hpp"
#include "mx_device.hpp"

namespace {

struct RmsArgs {
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* w;
  uint8_t* q;
  int64_t ldq;
  uint8_t* s;
  int64_t lds;
  int64_t M;
  int K;
  float eps;
};

constexpr int kRowsPerBlock = 4;  // waves per 256-thread workgroup, one row each
constexpr int kBatch = 8;         // passes whose loads are in flight together

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__global__ __launch_bounds__(256) void rmsnorm_quant_kernel(RmsArgs a) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + wave;
  if (r >= a.M) return;  // whole waves only; the kernel has no barrier
  const uint16_t* const xr = a.x + r * a.ldx;
  const int passes = (a.K + 511) / 512;

  // Pass one: lane sum of squares, pass by pass and element by element. K is a
  // multiple of 32, so a lane's 8 elements lie wholly inside or outside the row.
  // Loads past the row read its last 16 bytes (they stay in bounds and are
  // issued unconditionally, kBatch at a time) and count as zeros, which leaves
  // every sum unchanged.
  double acc = 0.0;
  for (int c0 = 0; c0 < passes; c0 += kBatch) {
    uint4 v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int k0 = 512 * (c0 + b) + 8 * l;
      v[b] = mx::ldg16(xr + (k0 < a.K ? k0 : a.K - 8));
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const bool in = 512 * (c0 + b) + 8 * l < a.K;
      const uint32_t wd[4] = {in ? v[b].x : 0u, in ? v[b].y : 0u, in ? v[b].z : 0u, in ? v[b].w : 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double f = (double)((e & 1) ? bf16_hi(wd[e >> 1]) : bf16_lo(wd[e >> 1]));
        acc = __builtin_fma(f, f, acc);  // f*f is exact in float64: this is acc + f^2, rounded once
      }
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const double o = __shfl_down(acc, (unsigned)s, 64);
    if (l < s) acc = acc + o;
  }
  const double ss = __shfl(acc, 0, 64);
  const double ms = ss / (double)a.K + (double)a.eps;
  const float inv = (float)(1.0 / __builtin_sqrt(ms));

  // Pass two: y = bf16((x * inv) * w), then MXFP4 per lane quad. Every lane
  // computes (clamped loads as above); only lanes inside the row store.
  for (int c0 = 0; c0 < passes; c0 += kBatch) {
    uint4 xv[kBatch], wv[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int k0 = 512 * (c0 + b) + 8 * l, kc = k0 < a.K ? k0 : a.K - 8;
      xv[b] = mx::ldg16(xr + kc);
      wv[b] = mx::ldg16(a.w + kc);
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int k0 = 512 * (c0 + b) + 8 * l;
      const uint32_t xw[4] = {xv[b].x, xv[b].y, xv[b].z, xv[b].w}, ww[4] = {wv[b].x, wv[b].y, wv[b].z, wv[b].w};
      uint32_t y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float t0 = bf16_lo(xw[i]) * inv, t1 = bf16_hi(xw[i]) * inv;
        const float y0 = t0 * bf16_lo(ww[i]), y1 = t1 * bf16_hi(ww[i]);
        y[i] = (uint32_t)mx::f32_to_bf16(y0) | ((uint32_t)mx::f32_to_bf16(y1) << 16);
      }
      uint32_t sb;
      const uint32_t codes = mx::quant8_quad<true>(y, sb);  // all four lanes of a quad agree on `in`
      if (k0 < a.K) {
        *reinterpret_cast<uint32_t*>(a.q + r * a.ldq + k0 / 2) = codes;
        if ((l & 3) == 0) a.s[r * a.lds + k0 / 32] = (uint8_t)sb;
      }
    }
  }
}

}  // namespace

extern "C" int mxfp4_rmsnorm_quant(const void* x, int64_t ldx, const void* w, float eps, void* q, int64_t ldq,
                                   void* s, int64_t lds, int64_t M, int64_t K, void* stream) {
  if (!x || !w || !q || !s) return MXFP4_ERR_NULL;
  if (M < 1 || K < 32 || K % 32 != 0 || M > mxh::kMaxDim || K > mxh::kMaxDim) return MXFP4_ERR_SHAPE;
  if (ldx < K || ldq < K / 2 || lds < K / 32) return MXFP4_ERR_SHAPE;
  if (!(eps > 0.0f) || !(eps <= 3.4028235e38f)) return MXFP4_ERR_ARG;  // also rejects NaN
  if (!mxh::aligned(x, 16) || (ldx * 2) % 16 != 0 || !mxh::aligned(w, 16) || !mxh::aligned(q, 4) || ldq % 4 != 0)
    return MXFP4_ERR_ALIGN;
  RmsArgs a{(const uint16_t*)x, ldx, (const uint16_t*)w, (uint8_t*)q, ldq, (uint8_t*)s, lds, M, (int)K, eps};
  void* args[] = {&a};
  return mxh::launch_status(hipLaunchKernel((const void*)rmsnorm_quant_kernel,
                                            dim3((unsigned)mxh::cdiv(M, kRowsPerBlock)), dim3(256), args, 0,
                                            (hipStream_t)stream));
}
