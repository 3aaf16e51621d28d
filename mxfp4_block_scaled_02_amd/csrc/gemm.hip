// gemm_a4w4_fused / grouped_gemm_a4w4: C = Q(A) . B^T with the MXFP4
// quantisation of A done in registers inside the GEMM, so the quantised A never
// reaches global memory (kernelbot amd-mxfp4-mm submission 517169, module
// docstring: the two-kernel pipeline writes A_q to HBM and reads it back; the
// fix loads a bf16 tile, quantises on chip, feeds the block-scaled dot,
// accumulates in fp32 and stores bf16).
//
// Work decomposition. A wave owns a (16*MW) x (16*NW) block of C and a range of
// 128-wide K steps. Per K step every lane loads the 32 bf16 of its own MFMA A
// slot (row l%16, k-chunk l/16) -- exactly one MXFP4 block -- so amax, the E8M0
// byte and the E2M1 codes are computed by that lane alone with no cross-lane
// traffic, and the lane's scale byte is the matrix instruction's A scale. B
// comes pre-packed in fragment order: one 16-byte load per lane per 16x128 block.
// Four waves per workgroup either split the workgroup's K range (WK = 4, skinny
// M; partial sums reduced through LDS) or tile M x N (WK = 1). Across
// workgroups K may be split S ways (split-K as in page 683203's call of the
// assembly GEMM with a k-split argument); the partial tiles go to the caller's
// workspace and the last workgroup to arrive on a tile (an atomic counter) adds
// them in fixed order 0..S-1, writes bf16 and resets the counter, all in the
// same launch.
#include "host_common.hpp"
#include "mx_device.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;

struct Operand {
  const uint16_t* A;
  int64_t lda;
  const uint8_t* Bfrag;    // packed codes, fragment (t, j) at (t*KT + j)*1024
  const uint32_t* Bscale;  // packed scale dwords, (t, g, lane) at (t*KG + g)*64 + lane
  uint16_t* C;
  int64_t ldc;
  int M;
  int pad_;
};

struct Dims {
  int N, K, KT, NT16, KG;
};

template <int MW, int NW>
__device__ __forceinline__ void wave_mainloop(const Operand& p, const Dims& d, int m0, int n0, int jb, int je,
                                              mx::v4f (&acc)[MW][NW]) {
  const int l = threadIdx.x & 63, r = l & 15, c = l >> 4;
  for (int j = jb; j < je; ++j) {
    uint4 bq[NW];
    uint32_t bsc[NW];
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const int n16 = (n0 >> 4) + t;
      if (n16 < d.NT16) {
        bq[t] = mx::ldg16(p.Bfrag + (((int64_t)n16 * d.KT + j) * 64 + l) * 16);
        bsc[t] = p.Bscale[((int64_t)n16 * d.KG + (j >> 2)) * 64 + l] >> (8 * (j & 3));
      } else {
        bq[t] = make_uint4(0u, 0u, 0u, 0u);
        bsc[t] = mx::kScaleOne;
      }
    }
    const int kk = 128 * j + 32 * c;
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const int row = m0 + 16 * i + r;
      uint32_t w[16];
      if (row < p.M && kk < d.K) {
        const uint16_t* src = p.A + (int64_t)row * p.lda + kk;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = mx::ldg16(src + 8 * q);
          w[4 * q + 0] = v.x;
          w[4 * q + 1] = v.y;
          w[4 * q + 2] = v.z;
          w[4 * q + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) w[q] = 0u;
      }
      uint32_t qa[4], sa;
      mx::quant32(w, qa, sa);
      const uint4 a4 = make_uint4(qa[0], qa[1], qa[2], qa[3]);
#pragma unroll
      for (int t = 0; t < NW; ++t) acc[i][t] = mx::mfma_fp4(a4, bq[t], acc[i][t], sa, bsc[t]);
    }
  }
}

// Store a wave's accumulators as bf16 with M/N masks.
template <int MW, int NW>
__device__ __forceinline__ void store_c(const Operand& p, int N, int m0, int n0, const mx::v4f (&acc)[MW][NW]) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const int col = n0 + 16 * t + (l & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + 16 * i + 4 * (l >> 4) + e;
        if (row < p.M && col < N) p.C[(int64_t)row * p.ldc + col] = mx::f32_to_bf16(acc[i][t][e]);
      }
    }
}

// One workgroup's tile: main loop, intra-workgroup K reduction, split-K
// reduction across workgroups, bf16 store.
template <int MW, int NW, int WM, int WN, int WK>
__device__ __forceinline__ void gemm_tile(const Operand& p, const Dims& d, int mtile, int ntile, int s, int S,
                                          int64_t tile_id, float* partial, uint32_t* counters) {
  static_assert(WM * WN * WK == kWaves, "four waves per workgroup");
  constexpr int BM = 16 * MW * WM, BN = 16 * NW * WN, NACC = MW * NW * 4;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int wk = wave % WK, wn = (wave / WK) % WN, wm = wave / (WK * WN);
  const int m0 = mtile * BM + wm * 16 * MW, n0 = ntile * BN + wn * 16 * NW;
  const int parts = S * WK, part = s * WK + wk;
  const int jb = (int)((int64_t)d.KT * part / parts), je = (int)((int64_t)d.KT * (part + 1) / parts);

  mx::v4f acc[MW][NW];
#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int t = 0; t < NW; ++t) acc[i][t] = mx::v4f{0.f, 0.f, 0.f, 0.f};
  wave_mainloop<MW, NW>(p, d, m0, n0, jb, je, acc);

  if constexpr (WK > 1) {
    __shared__ float red[(WK - 1) * WM * WN][NACC][64];
    const int slot = (wk - 1) * WM * WN + wm * WN + wn;
    if (wk > 0) {
#pragma unroll
      for (int i = 0; i < MW; ++i)
#pragma unroll
        for (int t = 0; t < NW; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) red[slot][(i * NW + t) * 4 + e][l] = acc[i][t][e];
    }
    __syncthreads();
    if (wk == 0) {
      for (int k2 = 1; k2 < WK; ++k2) {
        const int sl = (k2 - 1) * WM * WN + wm * WN + wn;
#pragma unroll
        for (int i = 0; i < MW; ++i)
#pragma unroll
          for (int t = 0; t < NW; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][t][e] += red[sl][(i * NW + t) * 4 + e][l];
      }
    }
  }

  if (S == 1) {
    if (wk == 0) store_c<MW, NW>(p, d.N, m0, n0, acc);
    return;
  }

  // Split-K across workgroups: publish this split's partial tile, then the last
  // arriver sums all S partials in order and writes C.
  constexpr int TILE = BM * BN;
  const int64_t wslot = (int64_t)((wm * WN + wn) * NACC) * 64;
  if (wk == 0) {
    float* dst = partial + (tile_id * S + s) * TILE + wslot;
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
      for (int t = 0; t < NW; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[((i * NW + t) * 4 + e) * 64 + l] = acc[i][t][e];
  }
  __threadfence();
  __syncthreads();
  __shared__ int is_last;
  if (threadIdx.x == 0) is_last = (atomicAdd(&counters[tile_id], 1u) == (uint32_t)(S - 1));
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  if (wk == 0) {
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
      for (int t = 0; t < NW; ++t) acc[i][t] = mx::v4f{0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < S; ++s2) {
      const float* src = partial + (tile_id * S + s2) * TILE + wslot;
#pragma unroll
      for (int i = 0; i < MW; ++i)
#pragma unroll
        for (int t = 0; t < NW; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][t][e] += src[((i * NW + t) * 4 + e) * 64 + l];
    }
    store_c<MW, NW>(p, d.N, m0, n0, acc);
  }
  if (threadIdx.x == 0) counters[tile_id] = 0u;
}

template <int MW, int NW, int WM, int WN, int WK>
__global__ __launch_bounds__(kThreads) void gemm_fused_kernel(Operand p, Dims d, int S, float* partial,
                                                               uint32_t* counters) {
  const int64_t tile_id = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  gemm_tile<MW, NW, WM, WN, WK>(p, d, blockIdx.y, blockIdx.x, blockIdx.z, S, tile_id, partial, counters);
}

struct GroupedArgs {
  Operand g[MXFP4_MAX_GROUPS];
  int tile_start[MXFP4_MAX_GROUPS + 1];  // prefix sums of per-group tile counts
  int G;
  int ntiles_n;
};

template <int MW, int NW, int WM, int WN, int WK>
__global__ __launch_bounds__(kThreads) void gemm_grouped_kernel(GroupedArgs a, Dims d) {
  const int id = blockIdx.x;
  int g = 0;
  while (g + 1 < a.G && a.tile_start[g + 1] <= id) ++g;
  const int local = id - a.tile_start[g];
  gemm_tile<MW, NW, WM, WN, WK>(a.g[g], d, local / a.ntiles_n, local % a.ntiles_n, 0, 1, 0, nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// Host side: plan, workspace size, launch.
// ---------------------------------------------------------------------------
enum Variant { kSkinny1, kSkinny2, kSkinny4, kTiled };

struct Plan {
  Variant v;
  int BM, BN, S;
  int64_t mtiles, ntiles;
  size_t ws_bytes;
};

constexpr int kMaxSplit = 16;

Plan make_plan(int64_t M, int64_t N, int64_t K) {
  Plan pl{};
  const int64_t KT = mxh::cdiv(K, 128);
  if (M <= 64) {
    pl.v = M <= 16 ? kSkinny1 : (M <= 32 ? kSkinny2 : kSkinny4);
    pl.BM = M <= 16 ? 16 : (M <= 32 ? 32 : 64);
    pl.BN = 64;
  } else {
    pl.v = kTiled;
    pl.BM = 128;
    pl.BN = 128;
  }
  pl.mtiles = mxh::cdiv(M, pl.BM);
  pl.ntiles = mxh::cdiv(N, pl.BN);
  pl.S = 1;
  if (pl.v != kTiled) {
    const int64_t tiles = pl.mtiles * pl.ntiles;
    int64_t S = mxh::cdiv(256, tiles);
    S = S > KT / 4 ? KT / 4 : S;
    S = S > kMaxSplit ? kMaxSplit : S;
    pl.S = S < 1 ? 1 : (int)S;
  }
  pl.ws_bytes = 0;
  if (pl.S > 1) {
    const size_t tiles = (size_t)(pl.mtiles * pl.ntiles);
    const size_t counter_bytes = (tiles * 4 + 255) / 256 * 256;
    pl.ws_bytes = counter_bytes + tiles * (size_t)pl.S * pl.BM * pl.BN * 4;
  }
  return pl;
}

Dims make_dims(int64_t N, int64_t K) {
  const mxh::PackedGeom g(N, K);
  return Dims{(int)N, (int)K, (int)g.KT, (int)g.NT, (int)g.KG};
}

Operand make_operand(const void* A, int64_t lda, const void* Bp, void* C, int64_t ldc, int64_t M, int64_t N,
                     int64_t K) {
  const mxh::PackedGeom g(N, K);
  Operand o{};
  o.A = (const uint16_t*)A;
  o.lda = lda;
  o.Bfrag = (const uint8_t*)Bp;
  o.Bscale = (const uint32_t*)((const uint8_t*)Bp + g.code_bytes);
  o.C = (uint16_t*)C;
  o.ldc = ldc;
  o.M = (int)M;
  return o;
}

int check_problem(const void* A, int64_t lda, const void* Bp, const void* C, int64_t ldc, int64_t M, int64_t N,
                  int64_t K) {
  if (!A || !Bp || !C) return MXFP4_ERR_NULL;
  if (M < 1 || N < 1 || K < 32 || K % 32 != 0 || M > mxh::kMaxDim || N > mxh::kMaxDim || K > mxh::kMaxDim)
    return MXFP4_ERR_SHAPE;
  if (lda < K || ldc < N) return MXFP4_ERR_SHAPE;
  if (!mxh::aligned(A, 16) || (lda * 2) % 16 != 0 || !mxh::aligned(Bp, 16) || !mxh::aligned(C, 2))
    return MXFP4_ERR_ALIGN;
  return MXFP4_OK;
}

template <int MW, int NW, int WM, int WN, int WK>
hipError_t launch_fused(const Plan& pl, const Operand& o, const Dims& d, void* ws, hipStream_t st) {
  uint32_t* counters = (uint32_t*)ws;
  float* partial = nullptr;
  if (pl.S > 1) {
    const size_t tiles = (size_t)(pl.mtiles * pl.ntiles);
    partial = (float*)((uint8_t*)ws + (tiles * 4 + 255) / 256 * 256);
  }
  Operand op = o;
  Dims dd = d;
  int S = pl.S;
  void* args[] = {&op, &dd, &S, &partial, &counters};
  return hipLaunchKernel((const void*)gemm_fused_kernel<MW, NW, WM, WN, WK>,
                         dim3((unsigned)pl.ntiles, (unsigned)pl.mtiles, (unsigned)pl.S), dim3(kThreads), args, 0, st);
}

}  // namespace

extern "C" size_t gemm_a4w4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 32 || K % 32 != 0 || M > mxh::kMaxDim || N > mxh::kMaxDim || K > mxh::kMaxDim) return 0;
  return make_plan(M, N, K).ws_bytes;
}

extern "C" int gemm_a4w4_fused(const void* A, int64_t lda, const void* Bp, void* C, int64_t ldc, int64_t M, int64_t N,
                               int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_problem(A, lda, Bp, C, ldc, M, N, K);
  if (st != MXFP4_OK) return st;
  const Plan pl = make_plan(M, N, K);
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes || !mxh::aligned(workspace, 256)))
    return MXFP4_ERR_WORKSPACE;
  const Operand o = make_operand(A, lda, Bp, C, ldc, M, N, K);
  const Dims d = make_dims(N, K);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (pl.v) {
    case kSkinny1: e = launch_fused<1, 4, 1, 1, 4>(pl, o, d, workspace, s); break;
    case kSkinny2: e = launch_fused<2, 4, 1, 1, 4>(pl, o, d, workspace, s); break;
    case kSkinny4: e = launch_fused<4, 4, 1, 1, 4>(pl, o, d, workspace, s); break;
    default: e = launch_fused<4, 4, 2, 2, 1>(pl, o, d, workspace, s); break;
  }
  return mxh::launch_status(e);
}

extern "C" size_t grouped_gemm_a4w4_workspace_bytes(const mxfp4_group* groups, int G, int64_t N, int64_t K) {
  (void)groups;
  (void)G;
  (void)N;
  (void)K;
  return 0;  // one tile per workgroup over the full K: no split-K partials
}

extern "C" int grouped_gemm_a4w4(const mxfp4_group* groups, int G, int64_t N, int64_t K, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!groups) return MXFP4_ERR_NULL;
  if (G < 1 || G > MXFP4_MAX_GROUPS) return MXFP4_ERR_TOO_MANY_GROUPS;
  GroupedArgs a{};
  constexpr int BM = 128, BN = 128;
  const int64_t ntn = mxh::cdiv(N, BN);
  int64_t total = 0;
  for (int g = 0; g < G; ++g) {
    const mxfp4_group& q = groups[g];
    const int st = check_problem(q.A, q.lda, q.Bp, q.C, q.ldc, q.M, N, K);
    if (st != MXFP4_OK) return st;
    a.g[g] = make_operand(q.A, q.lda, q.Bp, q.C, q.ldc, q.M, N, K);
    a.tile_start[g] = (int)total;
    total += mxh::cdiv(q.M, BM) * ntn;
    if (total > INT32_MAX) return MXFP4_ERR_SHAPE;
  }
  a.tile_start[G] = (int)total;
  a.G = G;
  a.ntiles_n = (int)ntn;
  Dims d = make_dims(N, K);
  void* args[] = {&a, &d};
  return mxh::launch_status(hipLaunchKernel((const void*)gemm_grouped_kernel<4, 4, 2, 2, 1>, dim3((unsigned)total),
                                            dim3(kThreads), args, 0, (hipStream_t)stream));
}
