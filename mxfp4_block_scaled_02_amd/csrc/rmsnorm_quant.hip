// mxfp4_rmsnorm_quant: RMSNorm of each bf16 row, y = x / sqrt(mean(x^2) + eps) * w,
// followed by per-1x32 MXFP4 quantisation of y, in one launch (the fusion that
// kernelbot amd-mxfp4-mm submission 683203 names in its docstring, trick 1,
// without printing its arithmetic; the norm is the standard root-mean-square
// normalisation).
//
// A row is read in passes of 512 elements: lane l of a wave takes the 8
// elements k = 512c + 8l .. +7 of pass c, so a lane quad holds one 32-element
// block and one 16-byte load per lane covers 1 KB of the row. Rows of up to 16
// passes (K <= 8192) take one 256-thread workgroup each: wave v of its four
// takes passes [P*v/4, P*(v+1)/4) and keeps them in registers (x is read once).
// Longer rows take one wave each and read x again for the second phase.
//
// Phase one sums the squares in float64, each lane over its passes in
// pass-then-element order; the 64 lane sums meet in a halving tree
// (S[t] += S[t+s], s = 32 .. 1), and a row split over four waves adds the
// waves' sums in wave order. The order is fixed, so the result, and with it
// every quantised code, is the same on every run. The squares are exact; the
// sum is within (K-1)*2^-53 relative of the exact sum of squares, which is
// what the norm's definition asks for (an fp32 inv that this moves across a
// rounding boundary would differ from the exact one). inv = fp32(1 / sqrt(ss/K +
// eps)) with float64 steps; phase two forms y = bf16((x * inv) * w) in fp32 and
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

constexpr int kRowWaves = 4;      // waves per row (and per 256-thread workgroup), rows of <= kRowPasses passes
constexpr int kRowPasses = 16;    // 4 passes per wave
constexpr int kLongRows = 4;      // rows per 256-thread workgroup of the long-row kernel, one wave each
constexpr int kBatch = 8;         // passes whose loads are in flight together (long rows)

// Row loads go through a buffer resource over the row's 2K bytes: a lane whose
// 16 bytes lie past the row reads zeros by the range check on its own offset,
// which leaves the sums unchanged and needs no clamp or select.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 row_load16(__amdgpu_buffer_rsrc_t r, int k) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, 2 * k, 0, 0));
}
// x is read by one wave, once: a streaming (non-temporal) load, measured ~10 %
// faster for this kernel. (w, read by every row, keeps the default policy.)
__device__ __forceinline__ uint4 row_load16_nt(__amdgpu_buffer_rsrc_t r, int k) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, 2 * k, 0, 2));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Lane quad quantisation of y = bf16((x * inv) * w) for one pass: 8 elements
// of x and w per lane (zeros past the row); only lanes inside the row store.
__device__ __forceinline__ void norm_quant_pass(const RmsArgs& a, int64_t r, int k0, const uint4& xv, const uint4& wv,
                                                float inv, int l) {
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, ww[4] = {wv.x, wv.y, wv.z, wv.w};
  uint32_t y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float t0 = bf16_lo(xw[i]) * inv, t1 = bf16_hi(xw[i]) * inv;
    const float y0 = t0 * bf16_lo(ww[i]), y1 = t1 * bf16_hi(ww[i]);
    y[i] = mx::pack_bf16x2(y0, y1);  // one packed convert, round to nearest even
  }
  uint32_t sb;
  const uint32_t codes = mx::quant8_quad<true>(y, sb);  // all four lanes of a quad agree on k0 < K
  if (k0 < a.K) {  // written once, not read here: non-temporal stores
    __builtin_nontemporal_store(codes, reinterpret_cast<uint32_t*>(a.q + r * a.ldq + k0 / 2));
    if ((l & 3) == 0) __builtin_nontemporal_store((uint8_t)sb, a.s + r * a.lds + k0 / 32);
  }
}

// Adds the squares of one pass's 8 elements to acc in element order.
__device__ __forceinline__ double add_squares(double acc, const uint4& v) {
  const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double f = (double)((e & 1) ? bf16_hi(wd[e >> 1]) : bf16_lo(wd[e >> 1]));
    acc = __builtin_fma(f, f, acc);  // f*f is exact in float64: this is acc + f^2, rounded once
  }
  return acc;
}

// The 64 lane sums of a wave in the halving tree; lane 0 ends with the total.
__device__ __forceinline__ double wave_sum(double acc, int l) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const double o = __shfl_down(acc, (unsigned)s, 64);
    if (l < s) acc = acc + o;
  }
  return acc;
}

__device__ __forceinline__ float inv_of(double ss, int K, float eps) {
  const double ms = ss / (double)K + (double)eps;
  return (float)(1.0 / __builtin_sqrt(ms));
}

// Rows of at most kRowPasses passes: workgroup = row, wave v = passes
// [P*v/4, P*(v+1)/4) (at most 4; none for some waves when P < 4). Its x and w
// stay in registers between the phases; the four wave sums meet in LDS.
__global__ __launch_bounds__(64 * kRowWaves) void rmsnorm_quant_rows_kernel(RmsArgs a) {
  constexpr int KP = kRowPasses / kRowWaves;
  __shared__ double part[kRowWaves];
  const int v = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t r = blockIdx.x;
  const __amdgpu_buffer_rsrc_t xr = row_rsrc(a.x + r * a.ldx, 2 * a.K), wr = row_rsrc(a.w, 2 * a.K);
  const int P = (a.K + 511) / 512;
  const int c0 = P * v / kRowWaves, c1 = P * (v + 1) / kRowWaves;
  // Passes past this wave's range read offset K: past the row, zeros.
  uint4 xv[KP], wv[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) xv[i] = row_load16_nt(xr, c0 + i < c1 ? 512 * (c0 + i) + 8 * l : a.K);
#pragma unroll
  for (int i = 0; i < KP; ++i) wv[i] = row_load16(wr, c0 + i < c1 ? 512 * (c0 + i) + 8 * l : a.K);
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < KP; ++i) acc = add_squares(acc, xv[i]);  // zeros past the range add nothing
  acc = wave_sum(acc, l);
  if (l == 0) part[v] = acc;
  __syncthreads();
  double ss = part[0];
#pragma unroll
  for (int u = 1; u < kRowWaves; ++u) ss = ss + part[u];
  const float inv = inv_of(ss, a.K, a.eps);
#pragma unroll
  for (int i = 0; i < KP; ++i)
    if (c0 + i < c1) norm_quant_pass(a, r, 512 * (c0 + i) + 8 * l, xv[i], wv[i], inv, l);
}

// Longer rows: one wave per row, x read again in phase two, kBatch passes at a
// time.
__global__ __launch_bounds__(64 * kLongRows) void rmsnorm_quant_long_kernel(RmsArgs a) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kLongRows + wave;
  if (r >= a.M) return;  // whole waves only; the kernel has no barrier
  const __amdgpu_buffer_rsrc_t xr = row_rsrc(a.x + r * a.ldx, 2 * a.K), wr = row_rsrc(a.w, 2 * a.K);
  const int passes = (a.K + 511) / 512;
  double acc = 0.0;
  for (int c0 = 0; c0 < passes; c0 += kBatch) {
    uint4 v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) v[b] = row_load16_nt(xr, 512 * (c0 + b) + 8 * l);
#pragma unroll
    for (int b = 0; b < kBatch; ++b) acc = add_squares(acc, v[b]);
  }
  const float inv = inv_of(__shfl(wave_sum(acc, l), 0, 64), a.K, a.eps);
  for (int c0 = 0; c0 < passes; c0 += kBatch) {
    uint4 xv[kBatch], wv[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      xv[b] = row_load16_nt(xr, 512 * (c0 + b) + 8 * l);
      wv[b] = row_load16(wr, 512 * (c0 + b) + 8 * l);
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) norm_quant_pass(a, r, 512 * (c0 + b) + 8 * l, xv[b], wv[b], inv, l);
  }
}

}  // namespace

extern "C" int mxfp4_rmsnorm_quant(const void* x, int64_t ldx, const void* w, float eps, void* q, int64_t ldq,
                                   void* s, int64_t lds, int64_t M, int64_t K, void* stream) {
  if (!x || !w || !q || !s) return MXFP4_ERR_NULL;
  // K <= 2^29: a row's byte offsets (2k) then stay inside a buffer resource's 31-bit range.
  if (M < 1 || K < 32 || K % 32 != 0 || M > mxh::kMaxDim || K > ((int64_t)1 << 29)) return MXFP4_ERR_SHAPE;
  if (ldx < K || ldq < K / 2 || lds < K / 32) return MXFP4_ERR_SHAPE;
  if (!(eps > 0.0f) || !(eps <= 3.4028235e38f)) return MXFP4_ERR_ARG;  // also rejects NaN
  if (!mxh::aligned(x, 16) || (ldx * 2) % 16 != 0 || !mxh::aligned(w, 16) || !mxh::aligned(q, 4) || ldq % 4 != 0)
    return MXFP4_ERR_ALIGN;
  RmsArgs a{(const uint16_t*)x, ldx, (const uint16_t*)w, (uint8_t*)q, ldq, (uint8_t*)s, lds, M, (int)K, eps};
  void* args[] = {&a};
  const int64_t passes = (K + 511) / 512;
  if (passes <= kRowPasses)  // one workgroup per row (M <= 2^30)
    return mxh::launch_status(hipLaunchKernel((const void*)rmsnorm_quant_rows_kernel, dim3((unsigned)M),
                                              dim3(64 * kRowWaves), args, 0, (hipStream_t)stream));
  return mxh::launch_status(hipLaunchKernel((const void*)rmsnorm_quant_long_kernel,
                                            dim3((unsigned)mxh::cdiv(M, kLongRows)), dim3(64 * kLongRows), args, 0,
                                            (hipStream_t)stream));
}
