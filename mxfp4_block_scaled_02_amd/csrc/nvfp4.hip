// grouped_gemm_nvfp4: the NVFP4 block-scaled GEMM of kernelbot nvfp4-group-gemm,
// submission 496271 (module docstring, constants block, ``nvfp4_gemm_kernel``,
// ``custom_kernel``): C = A B^T for a list of problems with their own (m, n, k, l),
// E2M1 elements on both sides with one E4M3 scale per 16 along K, fp32
// accumulation, float16 C. One launch covers every problem's output tiles.
//
// The gfx950 scaled matrix instructions take one power-of-two (E8M0) scale per
// lane's 32-element chunk, and their fp4 conversions likewise use only the
// exponent of the scale they are given; an E4M3 scale has three mantissa bits
// and covers 16 elements. An E2M1 value (2 significant bits) times an E4M3 scale
// (4 significant bits) has at most 6 significant bits and lies in [2^-10, 2688]
// in magnitude (or is zero), so it is exact in fp16. Each workgroup
// therefore expands its operand tiles to fp16 in LDS, exactly, and runs the
// dense fp16 32x32x16 instruction: the sum is then that of the exact products,
// in fp32.
//
// Workgroup: 256 threads own a 128 x 128 tile of C; a K step is 64. Thread t
// expands 32 elements of row t/2 (K half t%2) of each operand per step: two
// 8-byte code loads and its two scale bytes (from one 16-byte load of the row's
// scale bytes of four steps, one dword per step, or two byte loads, whichever
// the scale rows' layout allows),
// then per pair of elements one convert (two fp4 to two fp16, times 2^8, exact)
// and one packed fp16 multiply by 2^-8 times the scale (exact). Wave w computes
// rows 64(w/2).. and columns 64(w%2).. as 2 x 2 32x32 accumulators. LDS holds
// two fp16 tiles per operand (double buffer), rows padded to 144 bytes so that
// the 16-byte operand reads of 8 consecutive rows cover all banks once. The problems' tiles are laid out longest K first, so
// that the workgroups dispatched last (when the GPU is already full) are the
// shortest ones.
#include <algorithm>

#include "host_common.hpp"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kNvBM = 128, kNvBN = 128, kNvBK = 64, kNvThreads = 256;
constexpr int kNvRow = kNvBK + 8;        // fp16 per LDS row: 64 + 8 padding (144 bytes)
constexpr int kNvTile = kNvBM * kNvRow;  // fp16 per operand tile (kNvBM == kNvBN)
constexpr int kNvDepth = 4;              // K steps of code loads in flight (the loop runs 8 steps a turn)

struct NvProblem {
  const uint8_t* Aq;  // codes [M, K/2], row stride lda bytes
  const uint8_t* As;  // E4M3 [M, K/16], row stride ldas bytes
  const uint8_t* Bq;
  const uint8_t* Bs;
  uint16_t* C;  // fp16 [M, N], row stride ldc elements
  int64_t lda, ldas, ldb, ldbs, ldc;
  int M, N, K, pad_;
};
struct NvArgs {
  NvProblem p[MXFP4_MAX_GROUPS];
  int tile_start[MXFP4_MAX_GROUPS + 1];
  int P;
};

// Buffer resource over [base, base + bytes): loads past the end read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t nv_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// E4M3 byte (OCP 8-bit floating point, E4M3: bias 7, subnormals m/8 * 2^-6,
// S.1111.111 is NaN) as an fp16 pair (both halves) holding 2^-8 times its value:
// the byte's exponent and mantissa fields shifted into fp16's (E4M3 field e is
// 2^(e-7), fp16 field e is 2^(e-15); the subnormals line up likewise), the sign
// into fp16's, and a NaN for S.1111.111. Exact.
__device__ __forceinline__ uint32_t e4m3_f16x2_div256(uint32_t b) {
  uint32_t h = ((b & 0x7fu) << 7) | ((b & 0x80u) << 8);
  if ((b & 0x7fu) == 0x7fu) h |= 0x7e00u;  // exponent field all ones, mantissa non-zero
  return h | (h << 16);
}

// One operand row piece of a K step: 32 elements (16 code bytes, loaded as two
// 8-byte halves so that rows need only 8-byte alignment) and their two scale
// bytes. A thread reads 32 bytes of one row per step, so a wave's code load
// touches 32 cache lines; the scale loads are what the mode SM trims:
//   SM 2: one 16-byte load per row and four K steps (the row's 16 scale bytes of
//         those steps, carried in registers; bytes 4s + 2h and 4s + 2h + 1 of step
//         s's dword are K half h's): K % 256 == 0 and scale rows on 16-byte
//         boundaries, so no load straddles the end of a row. The kernel places
//         the step's dword in s0 and s1 before expanding.
//   SM 1: one dword load per row and step (K % 64 == 0, 4-byte boundaries).
//   SM 0: two byte loads (any layout). A byte load's value is widened where it
//         is used, and with the load ring that widening lands at the loop head,
//         where it waits for the newest loads; dword loads need no widening.
// One wave's scale load touches 32 lines in every mode, so SM 2 issues a quarter
// of SM 1's L1 requests for scales (measured 15 % faster on the grouped shapes).
struct Piece {
  u32x2 q0, q1;
  uint32_t s0, s1;
};

template <int SM>
__device__ __forceinline__ Piece load_piece(__amdgpu_buffer_rsrc_t qr, __amdgpu_buffer_rsrc_t sr, uint32_t row_q,
                                            uint32_t row_s, int kk) {
  Piece p;
  p.q0 = __builtin_amdgcn_raw_buffer_load_b64(qr, row_q + (uint32_t)(kk / 2), 0, 0);
  p.q1 = __builtin_amdgcn_raw_buffer_load_b64(qr, row_q + (uint32_t)(kk / 2) + 8u, 0, 0);
  if constexpr (SM == 2) {
    p.s0 = p.s1 = 0u;  // from the row's scale quads
  } else if constexpr (SM == 1) {
    p.s0 = __builtin_amdgcn_raw_buffer_load_b32(sr, row_s + (uint32_t)((kk / 16) & ~3), 0, 0);
    p.s1 = p.s0;
  } else {
    p.s0 = __builtin_amdgcn_raw_buffer_load_b8(sr, row_s + (uint32_t)(kk / 16), 0, 0);
    p.s1 = __builtin_amdgcn_raw_buffer_load_b8(sr, row_s + (uint32_t)(kk / 16) + 1u, 0, 0);
  }
  return p;
}

// Expands one piece to 32 fp16 in LDS at dst (16-byte aligned). Blocks at or past
// K get scale 0: their products are zero whatever bytes the loads returned.
template <int SM>
__device__ __forceinline__ void expand_piece(const Piece& pin, int kk, int K, _Float16* dst) {
  Piece p = pin;
  // Ties the piece's registers to this point: left free, the compiler hoists the
  // scale decoding of every ring slot to the loop head, which then waits for the
  // loads issued last.
  asm volatile("" : "+v"(p.q0), "+v"(p.q1), "+v"(p.s0), "+v"(p.s1));
  const int sh = SM ? 16 * ((kk >> 5) & 1) : 0;  // byte 2*(K half) of the step's scale dword
  // The decode masks every field it reads, so the bytes above need no clearing.
  f16x2 s0 = __builtin_bit_cast(f16x2, e4m3_f16x2_div256(p.s0 >> sh));
  f16x2 s1 = __builtin_bit_cast(f16x2, e4m3_f16x2_div256(p.s1 >> (SM ? sh + 8 : 0)));
  if (kk >= K) s0 = f16x2{(_Float16)0.0f, (_Float16)0.0f};
  if (kk + 16 >= K) s1 = f16x2{(_Float16)0.0f, (_Float16)0.0f};
  const uint32_t qw[4] = {p.q0.x, p.q0.y, p.q1.x, p.q1.y};
  uint32_t out[16];
  // Each element: E2M1 * 2^8 from the convert (at most 1536: exact), times the
  // scale's 2^-8 multiple: the exact product E2M1 * E4M3, which has at most 6
  // significant bits and lies in [2^-10, 2688] (or is zero): exact in fp16.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 sc = i < 2 ? s0 : s1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f16x2 v;
      switch (j) {  // the byte select must be a constant
        case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw[i], 256.0f, 0); break;
        case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw[i], 256.0f, 1); break;
        case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw[i], 256.0f, 2); break;
        default: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qw[i], 256.0f, 3); break;
      }
      out[4 * i + j] = __builtin_bit_cast(uint32_t, v * sc);  // element 2(4i+j) in the low half
    }
  }
  u32x4* d = reinterpret_cast<u32x4*>(dst);
#pragma unroll
  for (int c = 0; c < 4; ++c) d[c] = u32x4{out[4 * c], out[4 * c + 1], out[4 * c + 2], out[4 * c + 3]};
}

template <int SM>
__global__ __launch_bounds__(kNvThreads) void gemm_nvfp4_kernel(NvArgs a) {
  __shared__ __align__(16) _Float16 sA[2][kNvTile];
  __shared__ __align__(16) _Float16 sB[2][kNvTile];

  int g = 0;
  while (g + 1 < a.P && a.tile_start[g + 1] <= (int)blockIdx.x) ++g;
  const NvProblem& q = a.p[g];
  const int local = (int)blockIdx.x - a.tile_start[g];
  const int ntn = (q.N + kNvBN - 1) / kNvBN;
  const int m0 = (local / ntn) * kNvBM, n0 = (local % ntn) * kNvBN;

  const int tid = threadIdx.x, l = tid & 63, wave = tid >> 6;
  const int prow = tid >> 1, ph = tid & 1;  // this thread's piece: row and K half
  // Rows past M (N) start past the end of the resource and read zeros, and so
  // do the last row's loads past K (K/2 is a whole number of 8-byte loads).
  const __amdgpu_buffer_rsrc_t aq = nv_rsrc(q.Aq, (int64_t)(q.M - 1) * q.lda + q.K / 2);
  const __amdgpu_buffer_rsrc_t as = nv_rsrc(q.As, (int64_t)(q.M - 1) * q.ldas + q.K / 16);
  const __amdgpu_buffer_rsrc_t bq = nv_rsrc(q.Bq, (int64_t)(q.N - 1) * q.ldb + q.K / 2);
  const __amdgpu_buffer_rsrc_t bs = nv_rsrc(q.Bs, (int64_t)(q.N - 1) * q.ldbs + q.K / 16);
  const uint32_t arq = (uint32_t)((m0 + prow) * q.lda), ars = (uint32_t)((m0 + prow) * q.ldas);
  const uint32_t brq = (uint32_t)((n0 + prow) * q.ldb), brs = (uint32_t)((n0 + prow) * q.ldbs);
  const int KT = (q.K + kNvBK - 1) / kNvBK;
  const int dst = prow * kNvRow + 32 * ph;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // The pieces of the next kNvDepth steps are in flight in a register ring
  // (slot = step mod kNvDepth): one K step's matrix work is far shorter than a
  // load's latency. The loop runs 8 steps a turn (the SM 2 scale quads cover 4
  // steps each and alternate), so the step count is padded to a multiple of 8;
  // the padding steps lie past K, so they expand to zeros (zero scales) and add
  // nothing, and every load is unconditional (past the end, a load reads zeros).
  const int KTp = (KT + 7) / 8 * 8;
  Piece ra[kNvDepth], rb[kNvDepth];
#pragma unroll
  for (int u = 0; u < kNvDepth; ++u) {
    const int kk = kNvBK * u + 32 * ph;
    ra[u] = load_piece<SM>(aq, as, arq, ars, kk);
    rb[u] = load_piece<SM>(bq, bs, brq, brs, kk);
  }
  // SM 2: qa[c] / qb[c] hold the row's scale bytes of steps 4g .. 4g+3 for the
  // two groups g of a turn's 8 steps (c = g % 2); each is reloaded after its last
  // use. The step's dword is written into the piece before it is expanded.
  u32x4 qa[2], qb[2];
  if constexpr (SM == 2) {
    qa[0] = __builtin_amdgcn_raw_buffer_load_b128(as, (int)ars, 0, 0);
    qb[0] = __builtin_amdgcn_raw_buffer_load_b128(bs, (int)brs, 0, 0);
    qa[1] = __builtin_amdgcn_raw_buffer_load_b128(as, (int)(ars + 16u), 0, 0);
    qb[1] = __builtin_amdgcn_raw_buffer_load_b128(bs, (int)(brs + 16u), 0, 0);
    ra[0].s0 = ra[0].s1 = qa[0].x;
    rb[0].s0 = rb[0].s1 = qb[0].x;
  }
  expand_piece<SM>(ra[0], 32 * ph, q.K, &sA[0][dst]);
  expand_piece<SM>(rb[0], 32 * ph, q.K, &sB[0][dst]);
  ra[0] = load_piece<SM>(aq, as, arq, ars, kNvBK * kNvDepth + 32 * ph);
  rb[0] = load_piece<SM>(bq, bs, brq, brs, kNvBK * kNvDepth + 32 * ph);
  __syncthreads();

  const int wm = 64 * (wave >> 1), wn = 64 * (wave & 1);
  const int orow = (l & 31) * kNvRow + 8 * (l >> 5);  // operand element of this lane within a 32-row block
  for (int j0 = 0; j0 < KTp; j0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      const _Float16* A = sA[u & 1];  // j & 1
      const _Float16* B = sB[u & 1];
      // All operand reads of the step first, then its 16 matrix instructions.
      f16x8 fa[kNvBK / 16][2], fb[kNvBK / 16][2];
#pragma unroll
      for (int ks = 0; ks < kNvBK / 16; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          fa[ks][i] = *reinterpret_cast<const f16x8*>(&A[(wm + 32 * i) * kNvRow + orow + 16 * ks]);
          fb[ks][i] = *reinterpret_cast<const f16x8*>(&B[(wn + 32 * i) * kNvRow + orow + 16 * ks]);
        }
#pragma unroll
      for (int ks = 0; ks < kNvBK / 16; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
            acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[ks][i], fb[ks][jj], acc[i][jj], 0, 0, 0);
      // Step j+1 into the other buffer (last read in step j-1, before the barrier
      // that ended it), then its ring slot takes step j+1+kNvDepth. The
      // scheduling barriers keep the three phases in this order.
      const int un = (u + 1) % kNvDepth;
      const int kn = kNvBK * (j + 1) + 32 * ph;
      __builtin_amdgcn_sched_barrier(0);
      {
        Piece pa = ra[un], pb = rb[un];
        if constexpr (SM == 2) {
          const int sn = (u + 1) & 7;  // step j+1 within the turn: quad sn / 4, dword sn % 4
          const u32x4 xa = qa[sn >> 2], xb = qb[sn >> 2];
          pa.s0 = pa.s1 = (sn & 3) == 0 ? xa.x : (sn & 3) == 1 ? xa.y : (sn & 3) == 2 ? xa.z : xa.w;
          pb.s0 = pb.s1 = (sn & 3) == 0 ? xb.x : (sn & 3) == 1 ? xb.y : (sn & 3) == 2 ? xb.z : xb.w;
        }
        expand_piece<SM>(pa, kn, q.K, &sA[(u + 1) & 1][dst]);
        expand_piece<SM>(pb, kn, q.K, &sB[(u + 1) & 1][dst]);
      }
      __builtin_amdgcn_sched_barrier(0);
      ra[un] = load_piece<SM>(aq, as, arq, ars, kn + kNvBK * kNvDepth);
      rb[un] = load_piece<SM>(bq, bs, brq, brs, kn + kNvBK * kNvDepth);
      // Quad 0 (steps j0 .. j0+3) was last used at u = 2 and is next needed at
      // u = 7 (step j0+8); quad 1 (steps j0+4 .. j0+7) last at u = 6, next at u = 3
      // of the following turn.
      if constexpr (SM == 2) {
        if (u == 3) {
          qa[0] = __builtin_amdgcn_raw_buffer_load_b128(as, (int)(ars + 16u * (uint32_t)(j0 / 4 + 2)), 0, 0);
          qb[0] = __builtin_amdgcn_raw_buffer_load_b128(bs, (int)(brs + 16u * (uint32_t)(j0 / 4 + 2)), 0, 0);
        }
        if (u == 7) {
          qa[1] = __builtin_amdgcn_raw_buffer_load_b128(as, (int)(ars + 16u * (uint32_t)(j0 / 4 + 3)), 0, 0);
          qb[1] = __builtin_amdgcn_raw_buffer_load_b128(bs, (int)(brs + 16u * (uint32_t)(j0 / 4 + 3)), 0, 0);
        }
      }
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // acc[i][jj] register r of lane l: row 8(r/4) + 4(l/32) + r%4, column l%32 of its 32x32 block.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int col = n0 + wn + 32 * jj + (l & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        if (row < q.M && col < q.N)
          q.C[(int64_t)row * q.ldc + col] = __builtin_bit_cast(uint16_t, (_Float16)acc[i][jj][r]);
      }
    }
}

}  // namespace

extern "C" int grouped_gemm_nvfp4(const nvfp4_group* groups, int G, void* stream) {
  if (!groups) return MXFP4_ERR_NULL;
  if (G < 1) return MXFP4_ERR_TOO_MANY_GROUPS;
  NvArgs a{};
  int P = 0;
  int64_t total = 0;
  int sm = 2;  // the widest scale loads every problem's scale rows allow
  const int64_t lim = (int64_t)1 << 31;  // 32-bit buffer offsets, with a tile of rows to spare
  for (int g = 0; g < G; ++g) {
    const nvfp4_group& q = groups[g];
    if (!q.Aq || !q.As || !q.Bq || !q.Bs || !q.C) return MXFP4_ERR_NULL;
    if (q.M < 1 || q.N < 1 || q.K < 16 || q.K % 16 != 0 || q.M > mxh::kMaxDim || q.N > mxh::kMaxDim ||
        q.K > mxh::kMaxDim || q.L < 1)
      return MXFP4_ERR_SHAPE;
    if (q.lda < q.K / 2 || q.ldas < q.K / 16 || q.ldb < q.K / 2 || q.ldbs < q.K / 16 || q.ldc < q.N)
      return MXFP4_ERR_SHAPE;
    if ((q.M + kNvBM) * q.lda >= lim || (q.M + kNvBM) * q.ldas >= lim || (q.N + kNvBN) * q.ldb >= lim ||
        (q.N + kNvBN) * q.ldbs >= lim)
      return MXFP4_ERR_SHAPE;
    if (!mxh::aligned(q.Aq, 8) || !mxh::aligned(q.Bq, 8) || q.lda % 8 != 0 || q.ldb % 8 != 0 ||
        !mxh::aligned(q.C, 2))
      return MXFP4_ERR_ALIGN;
    if (q.L > MXFP4_MAX_GROUPS - P) return MXFP4_ERR_TOO_MANY_GROUPS;
    if (q.L > 1) {  // batches: C slices must not overlap; every slice keeps the alignment rules
      if (q.strideA < 0 || q.strideAs < 0 || q.strideB < 0 || q.strideBs < 0 || q.strideC < q.M * q.ldc)
        return MXFP4_ERR_SHAPE;
      if (q.strideA % 8 != 0 || q.strideB % 8 != 0) return MXFP4_ERR_ALIGN;
    }
    const int64_t tiles = mxh::cdiv(q.M, kNvBM) * mxh::cdiv(q.N, kNvBN);
    auto rows_on = [&](int64_t k_mult, int64_t bytes) {  // scale rows of every batch on `bytes` boundaries
      return q.K % k_mult == 0 && q.ldas % bytes == 0 && q.ldbs % bytes == 0 &&
             (q.L == 1 || (q.strideAs % bytes == 0 && q.strideBs % bytes == 0)) && mxh::aligned(q.As, bytes) &&
             mxh::aligned(q.Bs, bytes);
    };
    if (!rows_on(256, 16)) sm = std::min(sm, rows_on(64, 4) ? 1 : 0);
    for (int64_t l = 0; l < q.L; ++l) {
      NvProblem& o = a.p[P];
      o.Aq = (const uint8_t*)q.Aq + l * q.strideA;
      o.As = (const uint8_t*)q.As + l * q.strideAs;
      o.Bq = (const uint8_t*)q.Bq + l * q.strideB;
      o.Bs = (const uint8_t*)q.Bs + l * q.strideBs;
      o.C = (uint16_t*)q.C + l * q.strideC;
      o.lda = q.lda;
      o.ldas = q.ldas;
      o.ldb = q.ldb;
      o.ldbs = q.ldbs;
      o.ldc = q.ldc;
      o.M = (int)q.M;
      o.N = (int)q.N;
      o.K = (int)q.K;
      total += tiles;
      if (total > INT32_MAX) return MXFP4_ERR_SHAPE;
      ++P;
    }
  }
  // Longest K first (a stable order): the hardware hands out workgroups in id
  // order, so the tiles that start last, once the GPU is full, are the shortest.
  int order[MXFP4_MAX_GROUPS];
  for (int i = 0; i < P; ++i) order[i] = i;
  std::stable_sort(order, order + P, [&](int x, int y) { return a.p[x].K > a.p[y].K; });
  NvArgs b{};
  int64_t start = 0;
  for (int i = 0; i < P; ++i) {
    const NvProblem& o = a.p[order[i]];
    b.p[i] = o;
    b.tile_start[i] = (int)start;
    start += mxh::cdiv(o.M, kNvBM) * mxh::cdiv(o.N, kNvBN);
  }
  b.tile_start[P] = (int)start;
  b.P = P;
  void* args[] = {&b};
  const void* kern = sm == 2 ? (const void*)gemm_nvfp4_kernel<2>
                     : sm == 1 ? (const void*)gemm_nvfp4_kernel<1>
                               : (const void*)gemm_nvfp4_kernel<0>;
  return mxh::launch_status(
      hipLaunchKernel(kern, dim3((unsigned)total), dim3(kNvThreads), args, 0, (hipStream_t)stream));
}
