// gemm_a4w4_fused / grouped_gemm_a4w4: C = Q(A) . B^T with the MXFP4
// quantisation of A done on chip inside the GEMM, so the quantised A never
// reaches global memory (kernelbot amd-mxfp4-mm submission 517169, module
// docstring: the two-kernel pipeline writes A_q to HBM and reads it back; the
// fix loads a bf16 tile, quantises on chip, feeds the block-scaled dot,
// accumulates in fp32 and stores bf16).
//
// Both kernels load A with fully coalesced 16-byte accesses: a 32-element
// MXFP4 block then lies in the four lanes of a lane quad, which combine their
// partial maxima with two DPP steps and each convert their 8 elements
// (mx::quant8_quad). The codes are written to LDS in the lane order of the
// scaled matrix instruction, with an XOR swizzle that keeps both the quad
// writes and the operand reads free of bank conflicts. B arrives pre-packed in
// 32x64 operand units (mxfp4_pack_B), one 16-byte load per lane per unit.
//
// Three kernels:
//  * split-K (M <= 16): the grid is 64-column tiles x K splits. Each workgroup
//    issues all of its loads at once, quantises its A block once into LDS and
//    runs the 16x16x128 instruction; the splits of a tile hand their fp32
//    partials to the tile's last split (the owner) through the workspace,
//    which sums them in split order and stores bf16 C.
//  * skinny (16 < M <= 64; M <= 16 where a time model rates it faster than
//    split-K; a few hundred rows where the mid-M model does): a 1024-thread
//    workgroup owns MS rows x 16*NB columns of C over the whole K; its 16
//    waves split K, each quantises its own A slice into a private LDS operand
//    tile and runs the 16x16x128 instruction, and the 16 partial tiles are
//    summed in LDS. The same tile, on 8 waves and with up to four 16-row
//    sub-tiles, serves the grouped calls' small groups (and, by a launch
//    model, groups of up to 512 rows); a launch of small groups only takes it
//    on 16 waves. gemm_a4w4 runs its pre-quantised form (operands loaded
//    straight from A_q).
//  * tiled (larger M, and the grouped calls' larger groups): a 512-thread
//    workgroup (8 waves, one per CU) owns a 128 x 512 tile of C. Per 128-wide
//    K step the workgroup quantises the 128x128 bf16 A block once into a
//    double-buffered LDS tile; wave w computes all 128 rows x columns
//    [64w, 64w+64) with the 32x32x64 instruction from that shared A and its
//    own B units, which arrive by buffer-to-LDS loads in a three-stage
//    per-wave LDS ring two K steps ahead. The two waves sharing a SIMD run
//    their matrix and quantisation phases in opposite orders so the two
//    overlap. The C tile leaves through a per-wave LDS staging block as 16-byte
//    row stores. Workgroups are ordered so that the ones sharing an XCD (and
//    its L2) share A rows and B columns.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "host_common.hpp"
#include "mx_device.hpp"

namespace {

struct Operand {
  const uint16_t* A;       // bf16 A (fused path)
  int64_t lda;
  const uint8_t* Aq;       // pre-quantised A (gemm_a4w4): fp4x2 [M, K/2], row stride ldaq bytes
  int64_t ldaq;
  const uint8_t* As;       // and its E8M0 scales [M, K/32], row stride ldas bytes
  int64_t ldas;
  const uint8_t* Bunit;    // packed codes: unit (t, u) at (t*KU + u)*1024
  const uint32_t* Bscale;  // packed scale dwords: (t, g, lane) at (t*KG + g)*64 + lane
  uint16_t* C;
  int64_t ldc;
  int M;
  int pad_;
  // Verification instances only (DUMP): the quantised A each workgroup computes
  // on chip, codes [copy][M][K/2] at dq and E8M0 bytes [copy][M][K/32] at ds,
  // one copy per N-tile (every N-tile quantises the same A again).
  uint8_t* dq;
  uint8_t* ds;
};

// Writes one lane's share of an on-chip quantised block into the dump: the 8
// codes (4 bytes) of elements k0 .. k0+7 of row `row`, and, from the first lane
// of the quad, the block's scale byte as the matrix instruction receives it.
__device__ __forceinline__ void dump_piece(const Operand& p, int K, int copy, int row, int k0, uint32_t code,
                                           uint32_t sb, bool quad_lead) {
  if (row >= p.M || k0 >= K) return;
  const int64_t r = (int64_t)copy * p.M + row;
  *reinterpret_cast<uint32_t*>(p.dq + r * (K / 2) + k0 / 2) = code;
  if (quad_lead) p.ds[r * (K / 32) + k0 / 32] = (uint8_t)sb;
}

struct Dims {
  int N, K;
  int KT;    // 128-wide K steps, ceil(K/128)
  int KU;    // 64-wide packed units, ceil(K/64)
  int NT32;  // 32-column packed tiles, ceil(N/32)
  int KG;    // scale dword groups, ceil(KU/4)
};

// Buffer resource over [base, base + bytes): raw buffer loads outside it return
// zeros, which implements the M and N tails without branches. Each resource is
// built once per tile; the K position moves through the scalar offset of the
// load. The layouts below are chosen so that correctness does not depend on
// whether the range check includes that scalar offset: out-of-range rows and
// tiles are out of range by their per-lane offset alone, and elements past K are
// either zeroed explicitly (A) or never loaded (B).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// Cache-policy operand of the buffer intrinsics: device scope (the access is
// performed where every CU of the device observes it).
constexpr int kCpolDevice = 16;
constexpr int kCpolNonTemporal = 2;  // the nt bit of the buffer instructions
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// Streaming (non-temporal) 16-byte load, for B bytes that pass through once: a
// cold stream read this way runs ~10 % faster (measured). Operands that several
// CUs of an XCD keep re-reading through L2 (A everywhere, B of the tiled kernel)
// were measured slower with it and keep the default policy.
__device__ __forceinline__ uint4 bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kCpolNonTemporal);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t bload1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void to_words(const uint4& v, uint32_t (&w)[4]) {
  w[0] = v.x;
  w[1] = v.y;
  w[2] = v.z;
  w[3] = v.w;
}

// Window of A for 128-wide K step j of the row tile starting at m0: in-range
// bytes run to the end of row M-1's K elements. Elements k >= K of rows below
// the last are in range but are not A (next row or caller padding); the K-tail
// step zeroes them explicitly.
struct AWindow {
  const uint8_t* base;  // A + m0*lda
  int64_t bytes;        // extent from base
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t at(int j) const {
    return make_rsrc(base + (int64_t)j * 256, bytes - (int64_t)j * 256);
  }
};
// Rows m0.. of a byte matrix with row stride ld and rowlen meaningful bytes
// (pre-quantised A codes or scales): in range up to the end of row M-1.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_window(const uint8_t* base, int64_t ld, int64_t rowlen, int M,
                                                             int m0) {
  return make_rsrc(base + (int64_t)m0 * ld, m0 < M ? (int64_t)(M - 1 - m0) * ld + rowlen : 0);
}
__device__ __forceinline__ AWindow a_window(const Operand& p, int K, int m0) {
  AWindow w;
  w.base = reinterpret_cast<const uint8_t*>(p.A) + (int64_t)m0 * p.lda * 2;
  w.bytes = m0 < p.M ? ((int64_t)(p.M - 1 - m0) * p.lda + K) * 2 : 0;
  return w;
}

// A bijection on [0, G) giving each of the 8 XCDs (workgroup id mod 8) a
// contiguous run of tiles, so the tiles sharing an L2 share A rows / B columns.
__device__ __forceinline__ int xcd_remap(int id, int G) {
  const int full = G & ~7;
  if (id >= full) return id;
  return (id & 7) * (full >> 3) + (id >> 3);
}

// ---------------------------------------------------------------------------
// Skinny kernel
// ---------------------------------------------------------------------------
constexpr int kSkWaves = 16;

// 16-byte LDS slot of the 16x16x128 A operand element (row < 16, 32-k chunk < 4).
// The MFMA lane for it is chunk*16 + row; the XOR keeps a quad write pass (4
// rows x 4 chunks x 4 dwords) and each 16-lane operand read conflict-free.
__device__ __forceinline__ int slot16(int row, int chunk) { return chunk * 16 + (row ^ (chunk << 2)); }

// LDS of one skinny tile: per-wave A operand codes and scales of its MT 16-row
// sub-tiles, and the waves' partial C tiles of one sub-tile.
template <int WAVES, int NB, int MT = 1>
struct SkinnySmem {
  uint32_t aq[WAVES][MT][64 * 4];
  uint8_t as[WAVES][MT][64];
  float red[WAVES][NB * 4][64];
};

// Rows m0 .. m0+MS-1 x 16-column tiles T0 .. T0+NB-1 of C over the whole K, by
// the WAVES waves of the calling workgroup (all of its threads), each taking a
// contiguous share of the K steps; the partial tiles are summed in LDS. MS of
// 32, 48 or 64 is two to four 16-row sub-tiles that share each B operand the
// wave loads. `copy` is the verification dump's copy index of this tile's quantised A.
// PREQ: A arrives pre-quantised (gemm_a4w4): each lane loads its operand (row
// l%16 of a sub-tile, 32-element chunk l/16: 16 code bytes and one scale byte)
// and the quantisation and its LDS stage are skipped.
template <int WAVES, int MS, int NB, int PF, bool DUMP, bool PREQ = false>
__device__ __forceinline__ void skinny_tile(const Operand& p, const Dims& d, int m0, int T0, int copy,
                                            SkinnySmem<WAVES, NB, (MS + 15) / 16>& sm) {
  static_assert(MS == 4 || MS == 8 || MS == 16 || MS == 32 || MS == 48 || MS == 64, "rows per workgroup");
  constexpr int MT = (MS + 15) / 16;  // 16-row sub-tiles
  constexpr int PIECES = MS / 4;      // 16-byte A pieces per lane per K step (piece h: sub-tile h/4)
  auto& sAq = sm.aq;
  auto& sAs = sm.as;
  auto& red = sm.red;

  const int l = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
  const int jb = d.KT * wave / WAVES, je = d.KT * (wave + 1) / WAVES;

  // Rows MS..15 of the operand are never written: zero codes, neutral scales.
  if constexpr (MS < 16 && !PREQ) {
#pragma unroll
    for (int x = 0; x < 4; ++x) sAq[wave][0][x * 64 + l] = 0u;
    sAs[wave][0][l] = (uint8_t)mx::kScaleOne;
  }

  mx::v4f acc[MT][NB];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NB; ++t) acc[mt][t] = mx::v4f{0.f, 0.f, 0.f, 0.f};

  // Per-lane constants. A piece h: row 4h + l/16 of the tile, 8 elements at
  // 8*(l%16) of the K step (a wave pass covers 4 whole rows: coalesced).
  // Piece h's offset is aoff0 + h * arow4 (arow4: 4 rows of A, uniform). Up to
  // 48 rows the offsets are kept per piece; at 64 rows they are formed at each
  // load instead (15 fewer VGPRs, which keeps the 64-row tile within 256), and
  // the B offsets below are kept per column parity rather than per column.
  constexpr bool kStepOffsets = PIECES > 12;
  const AWindow aw = a_window(p, d.K, m0);
  const uint32_t aoff0 = (uint32_t)(((l >> 4) * p.lda + 8 * (l & 15)) * 2);
  const uint32_t arow4 = (uint32_t)(p.lda * 8);
  uint32_t aoff[kStepOffsets ? 1 : PIECES];
#pragma unroll
  for (int h = 0; h < (kStepOffsets ? 1 : PIECES); ++h) aoff[h] = aoff0 + (uint32_t)h * arow4;
  // LDS dword this lane writes for piece h, and the operand slot it reads.
  const int chunk = (l & 15) >> 2, sub = l & 3;
  int wslot[PIECES];
#pragma unroll
  for (int h = 0; h < PIECES; ++h) wslot[h] = slot16((4 * h + (l >> 4)) & 15, chunk);
  const int aslot = slot16(l & 15, l >> 4);
  // B operand of 16-column tile T at step j: lane l reads unit 2j + (l/16)/2 of
  // packed tile T/2 at unit lane ((l/16)%2)*32 + 16*(T%2) + l%16.
  // The unit lane depends on t only through the parity of T0 + t: at 64 rows
  // boff[0] and boff[1] hold the offsets of even and odd t (likewise soff for
  // the scales); otherwise one per column tile t.
  const int s16 = l >> 4;
  constexpr int kNBoff = kStepOffsets ? 2 : NB;
  uint32_t boff[kNBoff], soff[kNBoff];
#pragma unroll
  for (int q = 0; q < kNBoff; ++q) {
    const int odd = (T0 + q) & 1;
    boff[q] = (uint32_t)((s16 >> 1) * 1024 + (((s16 & 1) * 32 + odd * 16 + (l & 15)) * 16));
    soff[q] = (uint32_t)(((s16 & 1) * 32 + odd * 16 + (l & 15)) * 4);
  }
  const int tail_k = d.K - 128 * (d.KT - 1);  // valid elements in the last K step

  // Resources built once: A rows of the tile, and per 16-column tile its packed
  // 32-column tile's code units and scale dwords (empty past the packed N).
  const __amdgpu_buffer_rsrc_t ar = aw.at(0);
  __amdgpu_buffer_rsrc_t brs[NB], bss[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const int t32 = (T0 + t) >> 1;
    const bool ok = t32 < d.NT32;
    brs[t] = make_rsrc(p.Bunit + (int64_t)t32 * d.KU * 1024, ok ? (int64_t)d.KU * 1024 : 0);
    bss[t] = make_rsrc(p.Bscale + (int64_t)t32 * d.KG * 64, ok ? (int64_t)d.KG * 256 : 0);
  }
  const bool hi_unit = (s16 >> 1) != 0;  // lanes 32..63 read the step's second unit
  // Pre-quantised A: rows m0.. of the codes and scale bytes (rows past M read zeros).
  const __amdgpu_buffer_rsrc_t qr = PREQ ? row_window(p.Aq, p.ldaq, d.K / 2, p.M, m0) : ar;
  const __amdgpu_buffer_rsrc_t sr = PREQ ? row_window(p.As, p.ldas, d.K / 32, p.M, m0) : ar;
  const uint32_t qoff = PREQ ? (uint32_t)((l & 15) * p.ldaq + 16 * (l >> 4)) : 0u;
  const uint32_t qsoff = PREQ ? (uint32_t)((l & 15) * p.ldas + (l >> 4)) : 0u;

  for (int j0 = jb; j0 < je; j0 += PF) {
    uint32_t w[PF][PREQ ? 1 : PIECES][4];
    uint4 aop[PF][PREQ ? MT : 1];
    uint32_t asb[PF][PREQ ? MT : 1];
    uint4 bq[PF][NB];
    uint32_t bs[PF][NB];
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int j = j0 + s;
      if (j < je) {
        const bool last_odd = 2 * j + 1 >= d.KU;  // odd K/64: the second unit does not exist
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          if (!last_odd) {
            // read by the M/16 row-block workgroups
            bq[s][t] = bload16_nt(brs[t], boff[t % kNBoff], (uint32_t)j * 2048);
          } else {
            bq[s][t] = make_uint4(0u, 0u, 0u, 0u);
            if (!hi_unit) bq[s][t] = bload16_nt(brs[t], boff[t % kNBoff], (uint32_t)j * 2048);
          }
          bs[s][t] = bload4(bss[t], soff[t % kNBoff], (uint32_t)(j >> 1) * 256);
        }
        if constexpr (PREQ) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            aop[s][mt] = bload16(qr, qoff + (uint32_t)(16 * mt) * (uint32_t)p.ldaq, (uint32_t)j * 64);
            asb[s][mt] = bload1(sr, qsoff + (uint32_t)(16 * mt) * (uint32_t)p.ldas, (uint32_t)j * 4);
          }
        } else if constexpr (kStepOffsets) {
          uint32_t ao = aoff0;
          asm volatile("" : "+v"(ao));  // per step: the compiler does not keep PIECES offsets live
#pragma unroll
          for (int h = 0; h < PIECES; ++h)
            to_words(bload16(ar, ao + (uint32_t)h * arow4, (uint32_t)j * 256), w[s][h]);
        } else {
#pragma unroll
          for (int h = 0; h < PIECES; ++h) to_words(bload16(ar, aoff[h], (uint32_t)j * 256), w[s][h]);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int j = j0 + s;
      if (j < je) {
        const int bsh = 8 * ((2 * j + (l >> 5)) & 3);
        if constexpr (PREQ) {
          // K tail: chunks past K are not A (and their scale bytes are not scales).
          if (j == d.KT - 1 && 32 * (l >> 4) >= tail_k) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              aop[s][mt] = make_uint4(0u, 0u, 0u, 0u);
              asb[s][mt] = mx::kScaleOne;
            }
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < NB; ++t)
              acc[mt][t] = mx::mfma_fp4(aop[s][mt], bq[s][t], acc[mt][t], asb[s][mt], bs[s][t] >> bsh);
        } else {
          if (j == d.KT - 1 && tail_k < 128) {  // K tail: elements past K are not A
#pragma unroll
            for (int h = 0; h < PIECES; ++h)
              if (8 * (l & 15) >= tail_k) w[s][h][0] = w[s][h][1] = w[s][h][2] = w[s][h][3] = 0u;
          }
#pragma unroll
          for (int h = 0; h < PIECES; ++h) {
            uint32_t sb;
            const uint32_t code = mx::quant8_quad(w[s][h], sb);
            if constexpr (DUMP)
              dump_piece(p, d.K, copy, m0 + 4 * h + (l >> 4), 128 * j + 8 * (l & 15), code, sb, sub == 0);
            sAq[wave][h >> 2][wslot[h] * 4 + sub] = code;
            sAs[wave][h >> 2][wslot[h]] = (uint8_t)sb;  // the quad's four lanes store the same byte
          }
          // LDS operations of one wave complete in order: the reads see the writes.
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const uint4 a = *reinterpret_cast<const uint4*>(&sAq[wave][mt][aslot * 4]);
            const uint32_t sa = sAs[wave][mt][aslot];
#pragma unroll
            for (int t = 0; t < NB; ++t) acc[mt][t] = mx::mfma_fp4(a, bq[s][t], acc[mt][t], sa, bs[s][t] >> bsh);
          }
        }
      }
    }
  }

  // Sum the waves' partial tiles in LDS and store bf16, one 16-row sub-tile at a time.
  constexpr int OUT = NB * 256;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt > 0) __syncthreads();  // every thread is done reading the previous sub-tile
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][t * 4 + e][l] = acc[mt][t][e];
    __syncthreads();
    for (int o = threadIdx.x; o < OUT; o += WAVES * 64) {
      const int slot = o >> 6, ll = o & 63, t = slot >> 2, e = slot & 3;
      const int r = 16 * mt + 4 * (ll >> 4) + e;
      if (r >= MS) continue;
      float sum = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < WAVES; ++w2) sum += red[w2][slot][ll];
      const int row = m0 + r, col = (T0 + t) * 16 + (ll & 15);
      if (row < p.M && col < d.N) p.C[(int64_t)row * p.ldc + col] = mx::f32_to_bf16(sum);
    }
  }
}

// A 1-D grid of column tiles x `rows` row tiles: workgroup id v (after the XCD
// remap) is column tile v / rows and row tile v % rows, so the row tiles of a
// column tile are adjacent and read its B through one XCD's L2.
template <int MS, int NB, int PF, bool DUMP, bool PREQ = false>
__global__ __launch_bounds__(kSkWaves * 64) void gemm_skinny_kernel(Operand p, Dims d, int rows) {
  __shared__ __align__(16) SkinnySmem<kSkWaves, NB> sm;
  const int v = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int c = v / rows, r = v - c * rows;
  skinny_tile<kSkWaves, MS, NB, PF, DUMP, PREQ>(p, d, r * MS, c * NB, c, sm);
}

// ---------------------------------------------------------------------------
// Split-K kernel (M <= 16*MT, small)
// ---------------------------------------------------------------------------
// Grid: T tiles x S splits, workgroup id = tile * S + split. Tile t owns the
// 16-column groups 4t .. 4t+3 (wave w computes group 4t+w) for all rows; split q
// owns K steps [KT*q/S, KT*(q+1)/S). Each workgroup issues all of its loads at
// once, quantises its A block once into LDS and runs the 16x16x128 instruction.
// The splits of a tile are summed by its last split (the owner). Every other
// split stores the bitwise complement of its fp32 partial with device scope and
// exits; a workspace slot that still reads zero has not been written yet. The
// owner polls its tile's slots (eight splits per round trip), adds the partials
// in split order to its own, stores bf16 C and zeroes the slots again, so the
// workspace is all zero between calls. No read-modify-write is shared between
// workgroups (same-address atomics serialise at the memory side), and no
// workgroup waits for one dispatched after it: the owner has the highest id of
// its tile, so with in-order dispatch its producers have all started when it
// starts, and they never wait. A partial whose bits are all ones (a NaN, from
// non-finite input only) reads as unwritten; the poll bound then ends the wait.
constexpr int kSpW = 4;           // waves per workgroup = column groups per tile
constexpr int kSpT = kSpW * 64;
constexpr int kSpMaxSteps = 8;    // K steps per split, at most (LDS size)
constexpr int kSpMaxSplits = 64;
constexpr int kSpBatch = 8;       // partial slots polled per round trip
constexpr uint32_t kSpSpinCap = 1u << 22;  // owner's poll bound (never reached with finite input)

struct SplitArgs {
  uint32_t* part;  // [tile][split < S-1][wave][row tile][lane] x 4 words, complemented fp32; zero = empty
  int S;
};

// PREQ: A arrives pre-quantised (gemm_a4w4); each lane then loads its operand and
// scale byte directly, and the quantisation and LDS stages are skipped.
template <int MT, bool PREQ, bool DUMP>
__global__ __launch_bounds__(kSpT) void gemm_splitk_kernel(Operand p, Dims d, SplitArgs sk) {
  __shared__ __align__(16) uint32_t sAq[PREQ ? 1 : kSpMaxSteps][MT][64 * 4];  // A operand codes per step, row tile
  __shared__ uint8_t sAs[PREQ ? 1 : kSpMaxSteps][MT][64];                    // A operand scales

  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = sk.S;
  const int tile = blockIdx.x / S, q = blockIdx.x - tile * S;
  const int jb = d.KT * q / S, ns = d.KT * (q + 1) / S - jb;
  const int cg = tile * kSpW + wave;  // this wave's 16-column group
  const int tail_k = d.K - 128 * (d.KT - 1);

  // Every load is issued unconditionally, before any of them is used: steps past
  // this split's range repeat its last step (cache hits, never used). A guard
  // per load would let the compiler pair each load with its use and wait for it.
  // Fused: piece i = s*MT + rt is row 16rt + tid/16, elements 8*(tid%16) of step
  // jb+s (a wave pass covers 4 whole rows; each lane quad holds one 32-element
  // block). Pre-quantised: lane l's operand of row tile rt at step jb+s is row
  // 16rt + l%16, 32-element chunk l/16: 16 code bytes and one scale byte.
  uint32_t w[PREQ ? 1 : kSpMaxSteps * MT][4];
  uint4 aop[PREQ ? kSpMaxSteps * MT : 1];
  uint32_t asb[PREQ ? kSpMaxSteps * MT : 1];
  if constexpr (!PREQ) {
    const __amdgpu_buffer_rsrc_t ar = a_window(p, d.K, 0).at(0);
    const uint32_t aoff = (uint32_t)(((tid >> 4) * p.lda + 8 * (tid & 15)) * 2);
    const uint32_t arow16 = (uint32_t)(16 * p.lda * 2);
#pragma unroll
    for (int i = 0; i < kSpMaxSteps * MT; ++i) {
      const int s = min(i / MT, ns - 1);
      to_words(bload16(ar, aoff + (uint32_t)(i % MT) * arow16, (uint32_t)(jb + s) * 256), w[i]);
    }
  } else {
    const __amdgpu_buffer_rsrc_t qr = row_window(p.Aq, p.ldaq, d.K / 2, p.M, 0);
    const __amdgpu_buffer_rsrc_t sr = row_window(p.As, p.ldas, d.K / 32, p.M, 0);
    const int row = l & 15, ch = l >> 4;
#pragma unroll
    for (int i = 0; i < kSpMaxSteps * MT; ++i) {
      const int s = min(i / MT, ns - 1), rt = i % MT, j = jb + s;
      const int r = 16 * rt + row;
      aop[i] = bload16(qr, (uint32_t)(r * p.ldaq + 16 * ch), (uint32_t)j * 64);
      asb[i] = bload1(sr, (uint32_t)(r * p.ldas + ch), (uint32_t)j * 4);
      if (j == d.KT - 1 && 32 * ch >= tail_k) {  // K tail: not A (and not a scale that could be NaN)
        aop[i] = make_uint4(0u, 0u, 0u, 0u);
        asb[i] = mx::kScaleOne;
      }
    }
  }

  // B of column group cg (half of packed 32-column tile cg/2): as in the skinny
  // kernel. Requested after A, so that the quantisation can start while B streams.
  const int s16 = l >> 4;
  const int t32 = cg >> 1;
  const bool okB = t32 < d.NT32;
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(p.Bunit + (int64_t)t32 * d.KU * 1024, okB ? (int64_t)d.KU * 1024 : 0);
  const __amdgpu_buffer_rsrc_t bss = make_rsrc(p.Bscale + (int64_t)t32 * d.KG * 64, okB ? (int64_t)d.KG * 256 : 0);
  const uint32_t boff = (uint32_t)((s16 >> 1) * 1024 + (((s16 & 1) * 32 + (cg & 1) * 16 + (l & 15)) * 16));
  const uint32_t soff = (uint32_t)(((s16 & 1) * 32 + (cg & 1) * 16 + (l & 15)) * 4);
  const bool hi_unit = (s16 >> 1) != 0;
  uint4 bq[kSpMaxSteps];
  uint32_t bs[kSpMaxSteps];
  // A scale dword covers two K steps (four 64-k units): one load per pair of
  // steps, kSpMaxSteps/2 + 1 of them for a range that may start on an odd step.
  constexpr int kSg = kSpMaxSteps / 2 + 1;
  uint32_t bsg[kSg];
  const int g0 = jb >> 1, glast = (jb + ns - 1) >> 1;
#pragma unroll
  for (int g = 0; g < kSg; ++g) bsg[g] = bload4(bss, soff, (uint32_t)min(g0 + g, glast) * 256);
#pragma unroll
  for (int s = 0; s < kSpMaxSteps; ++s) {
    const int j = jb + min(s, ns - 1);
    // Odd K/64: the last step has no second unit; its lanes read the first one
    // (in range) and are zeroed below.
    const bool no_unit = 2 * j + 1 >= d.KU && hi_unit;
    bq[s] = bload16_nt(brs, no_unit ? boff - 1024 : boff, (uint32_t)j * 2048);  // read by this workgroup only
    if (no_unit) bq[s] = make_uint4(0u, 0u, 0u, 0u);
  }
  // Step s (< ns) lies in scale group ((jb + s) >> 1) - g0 = (s + jb % 2) >> 1.
  const bool jodd = (jb & 1) != 0;  // uniform
#pragma unroll
  for (int s = 0; s < kSpMaxSteps; ++s) bs[s] = jodd ? bsg[(s + 1) >> 1] : bsg[s >> 1];

  // Quantise A into the operand layout of the 16x16x128 instruction.
  if constexpr (!PREQ) {
    const int chunk = (tid & 15) >> 2, sub = tid & 3;
    const int wslot = slot16(tid >> 4, chunk);
#pragma unroll
    for (int i = 0; i < kSpMaxSteps * MT; ++i) {
      if (i < ns * MT) {
        const int s = i / MT, rt = i % MT;
        if (jb + s == d.KT - 1 && tail_k < 128 && 8 * (tid & 15) >= tail_k) w[i][0] = w[i][1] = w[i][2] = w[i][3] = 0u;
        uint32_t sb;
        const uint32_t code = mx::quant8_quad(w[i], sb);
        if constexpr (DUMP) dump_piece(p, d.K, tile, 16 * rt + (tid >> 4), 128 * (jb + s) + 8 * (tid & 15), code, sb, sub == 0);
        sAq[s][rt][wslot * 4 + sub] = code;
        sAs[s][rt][wslot] = (uint8_t)sb;  // the quad's four lanes store the same byte
      }
    }
    __syncthreads();
  }

  mx::v4f acc[MT];
#pragma unroll
  for (int rt = 0; rt < MT; ++rt) acc[rt] = mx::v4f{0.f, 0.f, 0.f, 0.f};
  const int aslot = slot16(l & 15, l >> 4);
#pragma unroll
  for (int s = 0; s < kSpMaxSteps; ++s) {
    if (s < ns) {
      const int bsh = 8 * ((2 * (jb + s) + (l >> 5)) & 3);
#pragma unroll
      for (int rt = 0; rt < MT; ++rt) {
        if constexpr (PREQ) {
          acc[rt] = mx::mfma_fp4(aop[s * MT + rt], bq[s], acc[rt], asb[s * MT + rt], bs[s] >> bsh);
        } else {
          const uint4 a = *reinterpret_cast<const uint4*>(&sAq[s][rt][aslot * 4]);
          acc[rt] = mx::mfma_fp4(a, bq[s], acc[rt], sAs[s][rt][aslot], bs[s] >> bsh);
        }
      }
    }
  }

  if (S > 1) {
    const int64_t tile_part = (int64_t)tile * (S - 1) * kSpW * MT * 64 * 16;  // bytes
    const __amdgpu_buffer_rsrc_t pr =
        make_rsrc(reinterpret_cast<uint8_t*>(sk.part) + tile_part, (int64_t)(S - 1) * kSpW * MT * 64 * 16);
    auto part_off = [&](int qq, int rt) { return (int)((((qq * kSpW + wave) * MT + rt) * 64 + l) * 16); };
    // Whole-vector casts only: with this compiler a bit cast of one element of a
    // vector value reads element 0 whatever the index.
    if (q < S - 1) {
#pragma unroll
      for (int rt = 0; rt < MT; ++rt)
        __builtin_amdgcn_raw_buffer_store_b128(~__builtin_bit_cast(u32x4, acc[rt]), pr, part_off(q, rt), 0,
                                               kCpolDevice);
      return;
    }
    // Owner: each wave collects its own column group's partials.
    mx::v4f sum[MT];
#pragma unroll
    for (int rt = 0; rt < MT; ++rt) sum[rt] = mx::v4f{0.f, 0.f, 0.f, 0.f};
    for (int q0 = 0; q0 < S - 1; q0 += kSpBatch) {
      const int nb = min(kSpBatch, S - 1 - q0);
      u32x4 v[kSpBatch][MT];
      for (uint32_t it = 0;; ++it) {
        // All loads first (slots past the batch repeat its last one), then the test.
#pragma unroll
        for (int b = 0; b < kSpBatch; ++b)
#pragma unroll
          for (int rt = 0; rt < MT; ++rt)
            v[b][rt] = __builtin_amdgcn_raw_buffer_load_b128(pr, part_off(q0 + min(b, nb - 1), rt), 0, kCpolDevice);
        bool ready = true;
#pragma unroll
        for (int b = 0; b < kSpBatch; ++b)
#pragma unroll
          for (int rt = 0; rt < MT; ++rt) {
            const u32x4 x = v[b][rt];
            ready = ready && x.x != 0u && x.y != 0u && x.z != 0u && x.w != 0u;
          }
        if (__builtin_amdgcn_ballot_w64(!ready) == 0 || it >= kSpSpinCap) break;
        __builtin_amdgcn_s_sleep(1);
      }
#pragma unroll
      for (int b = 0; b < kSpBatch; ++b)
        if (b < nb)
#pragma unroll
          for (int rt = 0; rt < MT; ++rt) {
            sum[rt] += __builtin_bit_cast(mx::v4f, ~v[b][rt]);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, pr, part_off(q0 + b, rt), 0, kCpolDevice);
          }
    }
#pragma unroll
    for (int rt = 0; rt < MT; ++rt) acc[rt] = sum[rt] + acc[rt];
  }

  // acc[rt] register e of lane l: row 16rt + 4(l/16) + e, column 16cg + l%16.
  const int col = cg * 16 + (l & 15);
  if (col < d.N) {
#pragma unroll
    for (int rt = 0; rt < MT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * rt + 4 * (l >> 4) + e;
        if (row < p.M) p.C[(int64_t)row * p.ldc + col] = mx::f32_to_bf16(acc[rt][e]);
      }
  }
}

// ---------------------------------------------------------------------------
// Tiled kernel
// ---------------------------------------------------------------------------
// 512 threads (8 waves, two per SIMD so one wave's quantisation overlaps the
// other's matrix instructions) own a 128 x 512 tile of C; wave w computes all
// 128 rows x columns [64w, 64w+64) with 4 x 2 32x32x64 accumulators.
constexpr int kTBM = 128, kTBN = 512, kTThreads = 512, kTWaves = kTThreads / 64;


// 16-byte LDS slot, within one 32x64 operand block, of unit lane `lane`
// (row lane%32, chunk lane/32) at 64-k half `ks` of a 128-k step; the XOR with the
// 32-element chunk index (2*ks + lane/32) keeps quad writes and operand reads
// conflict-free.
__device__ __forceinline__ int slot32(int lane, int ks) { return lane ^ ((((ks << 1) | (lane >> 5)) & 3) << 2); }

// Epilogue C staging block of one wave: 32 rows x 64 bf16 (32 dwords per row).
// The 16-dword halves of rows with bit 2 set are swapped, which puts the 4 rows
// of one packed write (rows a, a+1, a+4, a+5) and the 2 rows of one 16-lane read
// phase on disjoint banks.
constexpr int kCPitch = 32;
__device__ __forceinline__ int cst_at(int row, int dword) { return row * kCPitch + (dword ^ (((row >> 2) & 1) << 4)); }

// LDS of the tiled kernel (dwords): A operand codes [buffer][64-k half][32-row
// tile][64 lanes x 4], A scales [buffer][64-k half][lane] (byte = 32-row tile),
// and a per-wave staging block for the C epilogue.
struct TiledSmem {
  uint32_t a[2][2][4][256];
  uint32_t as[2][2][64];
  uint32_t cst[kTWaves][32 * kCPitch];  // per-wave C staging, 32 rows x 64 bf16
};

// One stage of the per-wave B ring: the wave's 2 packed tiles x 2 units of a K
// step (4 KB, unit (t, ks) at (2t + ks) * 1024, lane l's 16 bytes at l * 16) and
// the tiles' scale dwords (t * 256 + l * 4). Three stages, filled by
// buffer-to-LDS loads two steps ahead; each wave reads only its own part, so no
// barrier guards it. The ring is read with ds instructions written as inline
// assembly and explicit waits: the buffer loads into a stage are waited for by
// count (vmcnt) and the reads by an lgkmcnt wait bound to their results. The
// compiler sees neither, so it adds no wait of its own for the ring (which
// would drain every outstanding ring load, the next step's included).
constexpr int kRingWave = 4096 + 512;
constexpr int kRingStage = kTWaves * kRingWave;
constexpr int kRingBytes = 3 * kRingStage;
typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_addr(const void* ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ptr;
}
template <int OFF>
__device__ __forceinline__ u32x4v ring_read16(uint32_t addr) {
  u32x4v r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ uint32_t ring_read4(uint32_t addr) {
  uint32_t r;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
// Wait until at most N vector-memory operations of this wave are outstanding.
// The builtin (rather than assembly) lets the compiler's own wait analysis
// account for it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  // s_waitcnt fields: vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8]; the
  // latter two at their maximum (no wait).
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the LDS written with ds instructions (the A tiles): wait
// for this wave's LDS operations, then meet. Unlike __syncthreads() it does not
// wait for outstanding buffer loads, which would drain the B ring.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The A tiles' LDS stores, also written as inline assembly: the compiler waits
// for every outstanding buffer-to-LDS load before an LDS store it emits itself.
// The lds_barrier that follows them waits for their completion.
template <int OFF>
__device__ __forceinline__ void lds_st8(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b8 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF) : "memory");
}
__device__ __forceinline__ void lds_st32(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
// Two dwords at addr + 256 * O0 and addr + 256 * O1.
template <int O0, int O1>
__device__ __forceinline__ void lds_st2x32_st64(uint32_t addr, uint32_t v0, uint32_t v1) {
  asm volatile("ds_write2st64_b32 %0, %1, %2 offset0:%3 offset1:%4" ::"v"(addr), "v"(v0), "v"(v1), "i"(O0),
               "i"(O1)
               : "memory");
}
__device__ __forceinline__ void lds_st128(uint32_t addr, const uint4& v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(__builtin_bit_cast(u32x4v, v)) : "memory");
}

// PREQ: A arrives pre-quantised (gemm_a4w4). Thread tid then loads the 16 code
// bytes of row tid/4, 32-element chunk tid%4 of each K step (and row tid%128's
// 4 scale bytes) and stores them into the same LDS operand layout; everything
// else is shared with the fused path.
template <bool PREQ, bool DUMP = false>
__device__ __forceinline__ void tiled_tile(const Operand& p, const Dims& d, int mt, int nt, TiledSmem& sm,
                                           uint8_t* ring) {
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar addressing
  const int m0 = mt * kTBM;
  const int t0 = nt * (kTBN / 32) + wave * 2;  // this wave's first 32-column packed tile

  mx::v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][t][e] = 0.f;

  // Thread tid owns pieces P = 512h + tid (h < 4) of the 128 x 16 pieces of a K
  // step: row 32h + tid/16, elements 8*(tid%16) .. +7. Piece h lies in 32-row
  // tile h; a wave's pass covers 4 whole rows (coalesced) and each lane quad
  // holds one 32-element block.
  // One resource per piece h, over the window of rows m0 + 32h onwards, so the
  // four loads share one per-lane offset and each stays range-checked by it.
  __amdgpu_buffer_rsrc_t ar[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) ar[h] = a_window(p, d.K, m0 + 32 * h).at(0);
  const uint32_t aoff0 = (uint32_t)(((tid >> 4) * p.lda + 8 * (tid & 15)) * 2);
  const int chunk = (tid & 15) >> 2, sub = tid & 3, qks = chunk >> 1;
  // LDS dword written for piece h: block (buf, ks, i = h), slot of unit lane
  // (chunk%2)*32 + tid/16 (its XOR term is chunk << 2).
  const int wbase = (qks * 4) * 256 + ((chunk & 1) * 32 + ((tid >> 4) ^ (chunk << 2))) * 4 + sub;
  // Scale dword of this lane's 4 pieces: byte h is the scale of piece h (32-row
  // tile h), so one lane per quad stores all four as one dword.
  const int sdw = qks * 64 + (chunk & 1) * 32 + (tid >> 4);
  const int tail_k = d.K - 128 * (d.KT - 1);

  // A registers in flight. Fused: the bf16 pieces of one K step; two sets
  // alternate, the A of step j+1 is quantised at step j while the A of step j+2
  // is arriving. Pre-quantised: the codes and scale bytes of a PAIR of K steps
  // (2p, 2p+1) for two rows of this thread; a wave's load then covers 8 rows x
  // 128 bytes, whole cache lines (one step's 64 code bytes per row are half a
  // line), and its scale-byte load 8 rows x 8 bytes. Set p%2 holds pair p.
  struct AStage {
    uint32_t raw[PREQ ? 1 : 4][4];
    uint4 q[2];
    uint32_t qb[2];
  };
  AStage s0, s1;
  // Pre-quantised A: thread tid holds, of a step pair, rows qr0 = tid/8 and
  // qr0 + 64, 16-byte chunk qcc = tid%8 of the pair's 128 bytes, which is step
  // 2p + qcc/4 and 32-element chunk qc = qcc%4 of that step; in the operand
  // layout that is 64-k half qc/2, 32-row tile qr/32, unit lane (qc%2)*32 + qr%32.
  const int qr0 = tid >> 3, qcc = tid & 7, qc = qcc & 3, qhalf = qcc >> 2;
  const __amdgpu_buffer_rsrc_t aqr = row_window(p.Aq, p.ldaq, d.K / 2, p.M, m0);
  const __amdgpu_buffer_rsrc_t asr = row_window(p.As, p.ldas, d.K / 32, p.M, m0);
  // Step j's A (clamped to the last step: the loads run ahead of K and must stay
  // inside A, whose K offset is not range-checked; the extra copies go unused).
  auto load_a_piece = [&](int j, AStage& S, int h) {
    const uint32_t jo = (uint32_t)(j < d.KT ? j : d.KT - 1);
    to_words(bload16(ar[h], aoff0, jo * 256), S.raw[h]);
  };
  auto load_a = [&](int j, AStage& S) {
    const uint32_t jo = (uint32_t)(j < d.KT ? j : d.KT - 1);
    if constexpr (!PREQ) {
#pragma unroll
      for (int h = 0; h < 4; ++h) load_a_piece(j, S, h);
    } else {
      (void)jo;
      (void)S;
    }
  };
  // Pre-quantised: step pair p (clamped to the last pair that starts inside K;
  // a pair's second step may lie past K, in row padding or the next row, and is
  // never used) into set S: the codes and, from the same (row, step, chunk), the
  // scale byte; a wave's scale-byte load covers 8 rows x 8 consecutive bytes.
  auto load_pair = [&](int pr, AStage& S) {
    const int last = (d.KT - 1) >> 1;
    const uint32_t po = (uint32_t)(pr < last ? pr : last);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = qr0 + 64 * i;
      S.q[i] = bload16(aqr, (uint32_t)(r * p.ldaq + 16 * qcc), po * 128);
      S.qb[i] = bload1(asr, (uint32_t)(r * p.ldas + qcc), po * 8);
    }
  };
  // LDS byte addresses of this thread's A stores in buffer 0 (buffer 1 follows).
  constexpr uint32_t kABuf = sizeof(sm.a[0]), kSBuf = sizeof(sm.as[0]);
  const uint32_t qa = lds_addr(&sm.a[0][0][0][0]) + (uint32_t)wbase * 4;
  const uint32_t qs = lds_addr(&sm.as[0][0][0]) + (uint32_t)sdw * 4;
  uint32_t pa[2], ps[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int qr = qr0 + 64 * i;
    pa[i] = lds_addr(&sm.a[0][qc >> 1][qr >> 5][slot32((qc & 1) * 32 + (qr & 31), qc >> 1) * 4]);
    // Scale byte of (row qr, chunk qc): half qc/2, unit lane (qc%2)*32 + qr%32,
    // byte = 32-row tile qr/32.
    ps[i] = lds_addr(&sm.as[0][qc >> 1][(qc & 1) * 32 + (qr & 31)]) + (uint32_t)(qr >> 5);
  }
  // Pre-quantised: step j's codes and scale bytes from set S into LDS buffer
  // `buf`, by the threads whose half of the pair is step j (j%2). The other
  // threads store too, into their own wave's C staging block (idle until the
  // epilogue, which this wave alone writes after these stores): a select of
  // the address rather than a branch, which would make the compiler keep the
  // whole register set live across divergent code (it spilled). A chunk past K
  // gets zero codes and the neutral scale (never a NaN byte).
  const uint32_t sink = lds_addr(&sm.cst[wave][0]) + (uint32_t)l * 16;
  const uint32_t sink_sc = lds_addr(&sm.cst[wave][0]) + 1024u + (uint32_t)l;
  auto store_preq = [&](int j, int buf, AStage& S) {
    const bool mine = qhalf == (j & 1);
    const bool tl = j == d.KT - 1 && 32 * qc >= tail_k;  // K tail: not A
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lds_st128(mine ? pa[i] + buf * kABuf : sink, tl ? make_uint4(0u, 0u, 0u, 0u) : S.q[i]);
      lds_st8<0>(mine ? ps[i] + buf * kSBuf : sink_sc, tl ? mx::kScaleOne : S.qb[i]);
    }
  };
  // Quantise the bf16 A of step j held in S into LDS buffer j&1. The lanes of a
  // quad hold the same four scales and all store that dword. A 32-element block
  // past K (last step only) is stored as zero codes with the neutral scale,
  // whatever the registers held. after_piece(h) runs once piece h's registers
  // are consumed (the caller refills them there).
  const bool ktail_lane = 8 * (tid & 15) >= tail_k;
  auto quant_write = [&](int j, AStage& S, auto&& after_piece) {
    // The quantisation phase at raised wave priority: the SIMD's other wave is
    // in its matrix phase, whose instructions run on regardless (measured ~1 %).
    __builtin_amdgcn_s_setprio(1);
    uint32_t c[4], sw = 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      uint32_t sb;
      c[h] = mx::quant8_quad(S.raw[h], sb);
      if constexpr (DUMP)
        if (j < d.KT) dump_piece(p, d.K, nt, m0 + 32 * h + (tid >> 4), 128 * j + 8 * (tid & 15), c[h], sb, sub == 0);
      sw |= sb << (8 * h);
      __builtin_amdgcn_sched_barrier(0);
      after_piece(h);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (j == d.KT - 1 && ktail_lane) {  // selects, not a branch
#pragma unroll
      for (int h = 0; h < 4; ++h) c[h] = 0u;
      sw = mx::kScaleOne * 0x01010101u;
    }
    const int buf = j & 1;
    const uint32_t aa = qa + buf * kABuf;  // piece h at + 1024h bytes
    lds_st2x32_st64<0, 4>(aa, c[0], c[1]);
    lds_st2x32_st64<8, 12>(aa, c[2], c[3]);
    lds_st32(qs + buf * kSBuf, sw);
    __builtin_amdgcn_s_setprio(0);
  };
  // Step j's A into LDS buffer j&1 (K tail included).
  auto quant_store = [&](int j, AStage& S) {
    if constexpr (PREQ)
      store_preq(j, j & 1, S);
    else
      quant_write(j, S, [](int) {});
  };
  // Step jq's A from S into LDS buffer jq&1, and the A of step jl requested into
  // S: piece by piece for bf16 A, so that the loads spread over the VALU work.
  // Pre-quantised, at step j = jq - 1 with phase PH = j % 4: step j+1 comes from
  // set ((j+1)/2)%2 (sets 0, 1, 1, 0 for PH 0..3), and odd steps request pair
  // (j+3)/2 into set ((j+3)/2)%2 (set 0 at PH 1, set 1 at PH 3) once both halves
  // of the pair it held have been stored.
  auto quant_then_load = [&](auto ph, int jq, int jl, AStage& S) {
    if constexpr (PREQ) {
      constexpr int PH = decltype(ph)::value;
      (void)S;
      store_preq(jq, jq & 1, (PH == 0 || PH == 3) ? s0 : s1);
      if constexpr (PH == 1) load_pair((jq + 2) >> 1, s0);
      if constexpr (PH == 3) load_pair((jq + 2) >> 1, s1);
    } else {
      quant_write(jq, S, [&](int h) { load_a_piece(jl, S, h); });
    }
  };
  __amdgpu_buffer_rsrc_t brs[2], bss[2];  // per packed tile: code units, scale dwords
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int t32 = t0 + t;
    const bool ok = t32 < d.NT32;  // past the packed N: empty resource, loads give 0
    brs[t] = make_rsrc(p.Bunit + (int64_t)t32 * d.KU * 1024, ok ? (int64_t)d.KU * 1024 : 0);
    bss[t] = make_rsrc(p.Bscale + (int64_t)t32 * d.KG * 64, ok ? (int64_t)d.KG * 256 : 0);
  }
  // B of step jj into ring stage st: units 2jj (ks 0) and 2jj+1 (ks 1) of this
  // wave's 2 packed tiles, and the tiles' scale dwords. The unit sits in the
  // per-lane offset, so a unit past K (odd K/64) or a tile past N reads as zeros
  // by the range check alone. Six buffer loads.
  // Load p (< 6) of those: code unit (t, ks) = (p/2, p%2) for p < 4, else the
  // scale dwords of tile p-4.
  auto dma_part = [&](int jj, int st, int p) {
    uint8_t* const base = ring + st * kRingStage + wave * kRingWave;
    if (p < 4) {
      const int t = p >> 1, ks = p & 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(brs[t], (lds_void*)(base + (2 * t + ks) * 1024), 16,
                                               (int)((uint32_t)l * 16 + (uint32_t)(2 * jj + ks) * 1024), 0, 0, 0);
    } else if (p < 6) {
      const int t = p - 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(bss[t], (lds_void*)(base + 4096 + t * 256), 4,
                                               (int)((uint32_t)l * 4 + (uint32_t)(jj >> 1) * 256), 0, 0, 0);
    }
  };
  auto dma_b = [&](int jj, int st, int parts) {
#pragma unroll
    for (int p = 0; p < 6; ++p)
      if (p < parts) dma_part(jj, st, p);
  };
  const uint32_t rlane = lds_addr(ring + wave * kRingWave) + (uint32_t)l * 16;
  const uint32_t rlane_sc = lds_addr(ring + wave * kRingWave + 4096) + (uint32_t)l * 4;
  // Step j's 16 matrix instructions on B from ring stage st (whose buffer loads
  // the caller has waited for). B and the first 64-k half of A are read and
  // waited for; the second half's A reads are issued before the first matrix
  // instruction and land behind the first half's.
  uint32_t sck[2] = {0u, 0u};  // B scale dwords of the current pair of steps
  auto compute = [&](auto odd, int j, int st, auto&& after_pair) {
    const int buf = j & 1;
    uint4 a0[4], a1[4];
    const uint32_t so = (uint32_t)(st * kRingStage);
    u32x4v b00 = ring_read16<0>(rlane + so), b01 = ring_read16<2048>(rlane + so);
    u32x4v b10 = ring_read16<1024>(rlane + so), b11 = ring_read16<3072>(rlane + so);
    uint32_t sc0, sc1;
    if constexpr (!decltype(odd)::value) {
      sc0 = ring_read4<0>(rlane_sc + so);
      sc1 = ring_read4<256>(rlane_sc + so);
    }
    const uint32_t sa0 = sm.as[buf][0][l];
    const int sl0 = slot32(l, 0) * 4, sl1 = slot32(l, 1) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) a0[i] = *reinterpret_cast<const uint4*>(&sm.a[buf][0][i][sl0]);
    // Every LDS read so far has landed; binding the ring registers to this wait
    // keeps each of their uses below it.
    if constexpr (!decltype(odd)::value) {
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(b00), "+v"(b01), "+v"(b10), "+v"(b11), "+v"(sc0), "+v"(sc1)
                   :
                   : "memory");
      sck[0] = sc0;
      sck[1] = sc1;
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(b00), "+v"(b01), "+v"(b10), "+v"(b11) : : "memory");
      sc0 = sck[0];
      sc1 = sck[1];
    }
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t sa1 = sm.as[buf][1][l];
    const uint4 b[2][2] = {{__builtin_bit_cast(uint4, b00), __builtin_bit_cast(uint4, b01)},
                           {__builtin_bit_cast(uint4, b10), __builtin_bit_cast(uint4, b11)}};
    const uint32_t sc[2] = {sc0, sc1};
    auto mfma_pair = [&](int ks, int i, const uint4& av, uint32_t sa) {
      const int bsh = 8 * ((2 * j + ks) & 3);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t sb = sc[t] >> bsh;
        switch (i) {  // A scale byte = 32-row tile; folds once unrolled
          case 0: acc[i][t] = mx::mfma32_fp4<0, 0>(av, b[ks][t], acc[i][t], sa, sb); break;
          case 1: acc[i][t] = mx::mfma32_fp4<1, 0>(av, b[ks][t], acc[i][t], sa, sb); break;
          case 2: acc[i][t] = mx::mfma32_fp4<2, 0>(av, b[ks][t], acc[i][t], sa, sb); break;
          default: acc[i][t] = mx::mfma32_fp4<3, 0>(av, b[ks][t], acc[i][t], sa, sb); break;
        }
      }
    };
    // First 64-k half; the second half's A operand i is requested behind the
    // first half's pair i, four pairs ahead of its use, in the registers that
    // pair has finished with. after_pair(p) runs behind matrix pair p (< 8).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mfma_pair(0, i, a0[i], sa0);
      __builtin_amdgcn_sched_barrier(0);
      a1[i] = *reinterpret_cast<const uint4*>(&sm.a[buf][1][i][sl1]);
      after_pair(i);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mfma_pair(1, i, a1[i], sa1);
      __builtin_amdgcn_sched_barrier(0);
      after_pair(4 + i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Buffer loads a wave issues per A step: 4 (bf16 A), or on average 2 for
  // pre-quantised A (4 on odd steps: a pair's codes and scale bytes, none on
  // even steps; any two consecutive steps hold exactly one odd one), and per B
  // step 6 for an even step (4 code units, 2 scale dwords) and 4 for an odd one
  // (a scale dword covers two steps: the odd step reuses the dwords its even
  // predecessor read). The waits below count the loads issued after a ring
  // stage's.
  constexpr int kLa = PREQ ? 2 : 4, kDb = 6;
  // K step j. Every step requests B(j+2) into the ring stage read at step j-1,
  // one load behind each of its first six matrix pairs, and the A of step j+3
  // into the registers S, piece by piece as the quantisation of A(j+1) from S
  // (into the other LDS buffer) empties them: spread over the step, the loads
  // keep the address unit busy without stalling a wave on a full queue. Past
  // the end of K the loads are clamped (A) or read zeros (B) and the quantised
  // A lands in a buffer no step reads, so every step is the same code and the
  // waits are fixed counts. The two waves that share a SIMD (w and w+4) take
  // the matrix and the quantisation phases in opposite orders, so that one
  // wave's MFMAs run while the other wave's VALU quantisation runs. Loads
  // issued after B(j)'s, at B(j)'s use: matrix-first A(j+1), B(j+1), A(j+2);
  // quantisation-first A(j+2), B(j+1), A(j+3).
  auto step = [&](auto mfma_first, auto odd, auto ph, int j, int st, AStage& S) {
    constexpr bool kOdd = decltype(odd)::value;
    const int st2 = st == 0 ? 2 : st - 1;
    const int jb = j + 2 < d.KT ? j + 2 : d.KT - 1;
    // B(j+2) has the parity of j: odd steps load no scale dwords (the even step
    // before them read the dword both share).
    auto dma_hook = [&](int p) {
      if (!kOdd || p < 4) dma_part(jb, st2, p);
    };
    // Loads issued after B(j)'s include B(j+1): 4 loads if j+1 is odd, else 6.
    constexpr int kDbNext = kOdd ? kDb : kDb - 2;
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();  // A(j) is complete; every wave is past its reads of the other buffer
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(mfma_first)::value) {
      wait_vm<2 * kLa + kDbNext>();
      compute(odd, j, st, dma_hook);
      __builtin_amdgcn_sched_barrier(0);
      quant_then_load(ph, j + 1, j + 3, S);
    } else {
      quant_then_load(ph, j + 1, j + 3, S);
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<2 * kLa + kDbNext>();
      compute(odd, j, st, dma_hook);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Steps two at a time (the register sets alternate: even steps quantise from
  // s1), then an odd last step. Step j reads ring stage j % 3.
  // (Pre-quantised A takes its register set by the step's phase modulo 4, so
  // its loop runs four steps at a time.)
  using Ph0 = std::integral_constant<int, 0>;
  using Ph1 = std::integral_constant<int, 1>;
  using Ph2 = std::integral_constant<int, 2>;
  using Ph3 = std::integral_constant<int, 3>;
  auto run = [&](auto mfma_first) {
    int j = 0, st = 0;
    auto next = [](int x) { return x == 2 ? 0 : x + 1; };
    if constexpr (PREQ) {
      for (; j + 3 < d.KT; j += 4) {
        step(mfma_first, std::false_type{}, Ph0{}, j, st, s1);
        st = next(st);
        step(mfma_first, std::true_type{}, Ph1{}, j + 1, st, s0);
        st = next(st);
        step(mfma_first, std::false_type{}, Ph2{}, j + 2, st, s1);
        st = next(st);
        step(mfma_first, std::true_type{}, Ph3{}, j + 3, st, s0);
        st = next(st);
      }
      if (j < d.KT) step(mfma_first, std::false_type{}, Ph0{}, j, st, s1);
      st = next(st);
      if (j + 1 < d.KT) step(mfma_first, std::true_type{}, Ph1{}, j + 1, st, s0);
      st = next(st);
      if (j + 2 < d.KT) step(mfma_first, std::false_type{}, Ph2{}, j + 2, st, s1);
    } else {
      for (; j + 1 < d.KT; j += 2) {
        step(mfma_first, std::false_type{}, Ph0{}, j, st, s1);
        st = next(st);
        step(mfma_first, std::true_type{}, Ph1{}, j + 1, st, s0);
        st = next(st);
      }
      if (j < d.KT) step(mfma_first, std::false_type{}, Ph0{}, j, st, s1);
    }
    // No buffer-to-LDS load may still be in flight when the workgroup's LDS is
    // released. Draining inside each branch also keeps the compiler's wait
    // analysis from carrying one order's loads into the other order's loop (its
    // structurised control flow links the two); the two waits differ in their
    // LDS field so that they are not merged behind the join.
    if constexpr (decltype(mfma_first)::value)
      __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8));  // vmcnt(0) lgkmcnt(0)
    else
      wait_vm<0>();
  };

  // Prologue: B(0), B(1) and A(0..2) requested (pre-quantised: step pairs 0 and
  // 1), A(0) quantised into buffer 0.
  dma_b(0, 0, 6);
  dma_b(d.KT > 1 ? 1 : 0, 1, 4);
  if constexpr (PREQ) {
    load_pair(0, s0);
    load_pair(1, s1);
    store_preq(0, 0, s0);
  } else {
    load_a(0, s0);
    quant_store(0, s0);
    load_a(1, s1);
    load_a(2, s0);
  }
  // Enter the loops with nothing in flight: the compiler's wait analysis would
  // otherwise carry the prologue's loads into the loop and wait on them there.
  wait_vm<0>();
  if (wave < kTWaves / 2)  // uniform; each order is its own loop
    run(std::true_type{});
  else
    run(std::false_type{});

  // Epilogue. acc[i][t] register r of lane l holds row 32i + 8(r/4) + 4(l/32) + r%4,
  // column 32t + l%32 of this wave's 128 x 64 block. Per 32-row tile i: lane pairs
  // (l, l^1) trade halves of their packed bf16 pairs so that each lane holds two
  // adjacent columns of one row, the wave writes the 32 x 64 bf16 block to its
  // LDS staging area, reads it back by rows and stores 16 bytes per lane.
  uint32_t* const cst = sm.cst[wave];
  const int odd = l & 1;
  const int n0 = t0 * 32;  // first column of this wave's block
  const bool vec = ((reinterpret_cast<uintptr_t>(p.C) & 15u) == 0) && ((p.ldc & 7) == 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t pk = mx::pack_bf16x2(acc[i][t][2 * k], acc[i][t][2 * k + 1]);
        const uint32_t q = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pk, 0xB1, 0xF, 0xF, false);  // lane l^1
        const uint32_t w = odd ? ((q >> 16) | (pk & 0xffff0000u)) : ((pk & 0xffffu) | (q << 16));
        const int row = 8 * (k >> 1) + 4 * (l >> 5) + 2 * (k & 1) + odd;
        cst[cst_at(row, 16 * t + ((l & 31) >> 1))] = w;
      }
    // LDS operations of one wave complete in order: the reads below see the writes.
#pragma unroll
    for (int qr = 0; qr < 4; ++qr) {
      const int row = 8 * qr + (l >> 3), c8 = (l & 7) * 8;
      const uint4 v = *reinterpret_cast<const uint4*>(&cst[cst_at(row, c8 / 2)]);
      const int grow = m0 + 32 * i + row, gcol = n0 + c8;
      if (grow < p.M) {
        uint16_t* const dst = p.C + (int64_t)grow * p.ldc + gcol;
        if (vec && gcol + 8 <= d.N) {
          // Non-temporal: C is written once and not read back here (measured 4 % faster).
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(dst));
        } else {
          const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (gcol + e < d.N) dst[e] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

template <bool PREQ, bool DUMP>
__global__ __launch_bounds__(kTThreads) void gemm_tiled_kernel(Operand p, Dims d, int ntiles_n) {
  __shared__ __align__(16) TiledSmem sm;
  __shared__ __align__(16) uint8_t ring[kRingBytes];
  const int v = xcd_remap(blockIdx.x, gridDim.x);
  tiled_tile<PREQ, DUMP>(p, d, v / ntiles_n, v % ntiles_n, sm, ring);
}

// Grouped GEMM. A group of at most kGsMaxM rows is an HBM-bound problem (its B
// is read once for very few rows): it takes small tiles of one to four 16-row
// sub-tiles x 128 columns over the whole K, the workgroup's 8 waves splitting K
// (the skinny tile), so that its B spreads over many CUs; a 128 x 512 tile
// would give it one CU per 512 columns and leave the matrix cores of that CU
// computing 128 rows for a few. The host picks the fewest sub-tiles per tile
// at which the launch fits one round of workgroups, else all of the group's
// rows (each B byte then loaded once). Groups of up to a few hundred rows take
// the same skinny tiles (several row tiles per column) when the host's model
// (pick_small_max) estimates the launch faster so: few such groups leave most
// CUs idle on 128 x 512 tiles.
// Larger groups take the 128 x 512 tiled tiles. The large tiles take the first
// workgroup ids, so the hardware starts them first (they run longest), and the
// small tiles fill the other CUs beside them and whatever frees up. Each range
// is remapped for the XCDs on its own (the large range padded to a multiple of
// 8 ids with idle workgroups), and a small group's row tiles of one column tile
// are adjacent (they share that B in one XCD's L2).
constexpr int kGsMaxM = 64, kGsNB = 8;

struct GroupedArgs {
  Operand g[MXFP4_MAX_GROUPS];
  int tile_start[MXFP4_MAX_GROUPS + 1];  // prefix sums of the entries' tile counts, in launch order
  int order[MXFP4_MAX_GROUPS];           // group of launch entry e: large groups, then small ones
  int rows[MXFP4_MAX_GROUPS];            // row tiles of entry e
  int mt[MXFP4_MAX_GROUPS];              // 16-row sub-tiles of a small entry's tile
  int small_from;                        // first entry of a small group
  int nlarge, nlarge_pad;                // large tiles, and their id range rounded up to a multiple of 8
  int G;
  int ntiles_n;                          // 512-column tiles of a large group
};

template <bool DUMP>
__global__ __launch_bounds__(kTThreads) void gemm_grouped_kernel(GroupedArgs a, Dims d) {
  const int b = blockIdx.x;
  int v;
  if (b < a.nlarge_pad) {
    if (b >= a.nlarge) return;  // padding: the whole workgroup leaves
    v = xcd_remap(b, a.nlarge);
  } else {
    v = a.nlarge + xcd_remap(b - a.nlarge_pad, (int)gridDim.x - a.nlarge_pad);
  }
  int e = 0;
  while (e + 1 < a.G && a.tile_start[e + 1] <= v) ++e;
  const int local = v - a.tile_start[e];
  const Operand& p = a.g[a.order[e]];
  // The tiled tile's operand tiles and its B ring stay two LDS objects: the
  // compiler then knows that the ring's buffer-to-LDS loads do not write the
  // tiles it reads, and adds no wait for them. The skinny tile (no such loads)
  // lives in the ring's bytes.
  __shared__ __align__(16) TiledSmem sm;
  __shared__ __align__(16) uint8_t ring[kRingBytes];
  static_assert(sizeof(SkinnySmem<kTWaves, kGsNB, 4>) <= sizeof(ring), "skinny tile LDS");
  if (e >= a.small_from) {
    const int c = local / a.rows[e], r = local - c * a.rows[e];
    if (a.mt[e] == 1)
      skinny_tile<kTWaves, 16, kGsNB, 2, DUMP>(p, d, r * 16, c * kGsNB, c,
                                               *reinterpret_cast<SkinnySmem<kTWaves, kGsNB, 1>*>(ring));
    else if (a.mt[e] == 2)
      skinny_tile<kTWaves, 32, kGsNB, 1, DUMP>(p, d, r * 32, c * kGsNB, c,
                                               *reinterpret_cast<SkinnySmem<kTWaves, kGsNB, 2>*>(ring));
    else if (a.mt[e] == 3)
      skinny_tile<kTWaves, 48, kGsNB, 1, DUMP>(p, d, r * 48, c * kGsNB, c,
                                               *reinterpret_cast<SkinnySmem<kTWaves, kGsNB, 3>*>(ring));
    else
      skinny_tile<kTWaves, 64, kGsNB, 1, DUMP>(p, d, r * 64, c * kGsNB, c,
                                               *reinterpret_cast<SkinnySmem<kTWaves, kGsNB, 4>*>(ring));
  } else {
    tiled_tile<false, DUMP>(p, d, local / a.ntiles_n, local % a.ntiles_n, sm, ring);
  }
}

// A grouped launch of small groups only whose 16-row tiles all fit one round of
// workgroups: the tiles of the skinny kernel, 16 rows x 16*NB columns with K
// split over 16 waves (faster than the 8-wave tiles above), 64 columns when
// 128-column tiles would fill at most half a round. Entries and rows as for
// gemm_grouped_kernel with every mt 1; the whole grid is remapped for the XCDs.
template <int NB, bool DUMP>
__global__ __launch_bounds__(kSkWaves * 64) void gemm_grouped_small_kernel(GroupedArgs a, Dims d) {
  __shared__ __align__(16) SkinnySmem<kSkWaves, NB> sm;
  const int v = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  int e = 0;
  while (e + 1 < a.G && a.tile_start[e + 1] <= v) ++e;
  const int local = v - a.tile_start[e];
  const int c = local / a.rows[e], r = local - c * a.rows[e];
  skinny_tile<kSkWaves, 16, NB, NB == 4 ? 2 : 1, DUMP>(a.g[a.order[e]], d, r * 16, c * NB, c, sm);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// Per-problem list of grouped_gemm_a4w4_mnk: every group contributes L
// problems with their own (M, N, K); tile_start holds the prefix sums of the
// problems' output tiles. As in the grouped kernel, a problem of at most
// kGsMaxM rows (or of a few hundred, by pick_small_max) takes skinny tiles of mt
// 16-row sub-tiles x 128 columns (rows tiles per column), a larger one 128 x 512
// tiled tiles; the large problems come first and take the first workgroup ids.
struct MnkProblem {
  const uint16_t* A;
  int64_t lda;
  const uint8_t* Bunit;
  const uint32_t* Bscale;
  uint16_t* C;
  int64_t ldc;
  int M, N, K;
  int mt;    // 0: tiled tiles; 1..4: skinny tiles of mt 16-row sub-tiles
  int rows;  // skinny row tiles per column tile
};
struct MnkArgs {
  MnkProblem p[MXFP4_MAX_GROUPS];
  int tile_start[MXFP4_MAX_GROUPS + 1];
  int P;
  int nlarge, nlarge_pad;  // large-problem tiles, and their id range rounded up to a multiple of 8
};

__global__ __launch_bounds__(kTThreads) void gemm_grouped_mnk_kernel(MnkArgs a) {
  const int b = blockIdx.x;
  int v;
  if (b < a.nlarge_pad) {
    if (b >= a.nlarge) return;  // padding: the whole workgroup leaves
    v = xcd_remap(b, a.nlarge);
  } else {
    v = a.nlarge + xcd_remap(b - a.nlarge_pad, (int)gridDim.x - a.nlarge_pad);
  }
  int g = 0;
  while (g + 1 < a.P && a.tile_start[g + 1] <= v) ++g;
  const int local = v - a.tile_start[g];
  const MnkProblem& q = a.p[g];
  Operand o{};
  o.A = q.A;
  o.lda = q.lda;
  o.Bunit = q.Bunit;
  o.Bscale = q.Bscale;
  o.C = q.C;
  o.ldc = q.ldc;
  o.M = q.M;
  const int ku = (q.K + 63) / 64;
  const Dims d{q.N, q.K, (q.K + 127) / 128, ku, (q.N + 31) / 32, (ku + 3) / 4};
  __shared__ __align__(16) TiledSmem sm;
  __shared__ __align__(16) uint8_t ring[kRingBytes];
  if (q.mt > 0) {
    const int c = local / q.rows, r = local - c * q.rows;
    if (q.mt == 1)
      skinny_tile<kTWaves, 16, kGsNB, 2, false>(o, d, r * 16, c * kGsNB, c,
                                                *reinterpret_cast<SkinnySmem<kTWaves, kGsNB, 1>*>(ring));
    else if (q.mt == 2)
      skinny_tile<kTWaves, 32, kGsNB, 1, false>(o, d, r * 32, c * kGsNB, c,
                                                *reinterpret_cast<SkinnySmem<kTWaves, kGsNB, 2>*>(ring));
    else if (q.mt == 3)
      skinny_tile<kTWaves, 48, kGsNB, 1, false>(o, d, r * 48, c * kGsNB, c,
                                                *reinterpret_cast<SkinnySmem<kTWaves, kGsNB, 3>*>(ring));
    else
      skinny_tile<kTWaves, 64, kGsNB, 1, false>(o, d, r * 64, c * kGsNB, c,
                                                *reinterpret_cast<SkinnySmem<kTWaves, kGsNB, 4>*>(ring));
  } else {
    const int ntn = (q.N + kTBN - 1) / kTBN;
    tiled_tile<false>(o, d, local / ntn, local % ntn, sm, ring);
  }
}

Dims make_dims(int64_t N, int64_t K) {
  const mxh::PackedGeom g(N, K);
  return Dims{(int)N, (int)K, (int)mxh::cdiv(K, 128), (int)g.KU, (int)g.NT, (int)g.KG};
}

Operand make_operand(const void* A, int64_t lda, const void* Bp, void* C, int64_t ldc, int64_t M, int64_t N,
                     int64_t K) {
  const mxh::PackedGeom g(N, K);
  Operand o{};
  o.A = (const uint16_t*)A;
  o.lda = lda;
  o.Bunit = (const uint8_t*)Bp;
  o.Bscale = (const uint32_t*)((const uint8_t*)Bp + g.code_bytes);
  o.C = (uint16_t*)C;
  o.ldc = ldc;
  o.M = (int)M;
  return o;
}

Operand make_operand_q(const void* Aq, int64_t ldaq, const void* As, int64_t ldas, const void* Bp, void* C, int64_t ldc,
                       int64_t M, int64_t N, int64_t K) {
  Operand o = make_operand(nullptr, 0, Bp, C, ldc, M, N, K);
  o.Aq = (const uint8_t*)Aq;
  o.ldaq = ldaq;
  o.As = (const uint8_t*)As;
  o.ldas = ldas;
  return o;
}

// The kernels address A and packed B through buffer resources with 32-bit
// offsets: an A window spans at most kTBM rows from its base row, and one packed
// 32-column tile of B spans ceil(K/64) KB. Both must stay below 2^31 bytes, or
// the range check would silently clip in-range elements.
bool offsets_fit(int64_t ld_elems, int64_t K) {
  return (kTBM * ld_elems + K) * 2 < ((int64_t)1 << 31) && mxh::cdiv(K, 64) * 1024 < ((int64_t)1 << 31);
}

int check_problem(const void* A, int64_t lda, const void* Bp, const void* C, int64_t ldc, int64_t M, int64_t N,
                  int64_t K) {
  if (!A || !Bp || !C) return MXFP4_ERR_NULL;
  if (M < 1 || N < 1 || K < 32 || K % 32 != 0 || M > mxh::kMaxDim || N > mxh::kMaxDim || K > mxh::kMaxDim)
    return MXFP4_ERR_SHAPE;
  if (lda < K || ldc < N) return MXFP4_ERR_SHAPE;
  if (!offsets_fit(lda, K)) return MXFP4_ERR_SHAPE;
  if (!mxh::aligned(A, 16) || (lda * 2) % 16 != 0 || !mxh::aligned(Bp, 16) || !mxh::aligned(C, 2))
    return MXFP4_ERR_ALIGN;
  return MXFP4_OK;
}

template <int MS, int NB, int PF>
hipError_t launch_skinny(const Operand& o, const Dims& d, int64_t M, bool dump, hipStream_t st, bool preq = false) {
  Operand op = o;
  Dims dd = d;
  int rows = (int)mxh::cdiv(M, MS);
  void* args[] = {&op, &dd, &rows};
  const int64_t grid = mxh::cdiv(mxh::cdiv(d.N, 16), NB) * rows;
  const void* kern = preq   ? (const void*)gemm_skinny_kernel<MS, NB, PF, false, true>
                     : dump ? (const void*)gemm_skinny_kernel<MS, NB, PF, true>
                            : (const void*)gemm_skinny_kernel<MS, NB, PF, false>;
  return hipLaunchKernel(kern, dim3((unsigned)grid), dim3(kSkWaves * 64), args, 0, st);
}

// Skinny tile shape (rows MS x 16*NB columns per workgroup). Every workgroup
// reads its MS rows of bf16 A over the whole K plus its columns of packed B, and
// the busiest CU sets the time; pick the shape with the fewest bytes on it,
// counting 256 CUs with one 1024-thread workgroup each at a time.
struct SkinnyShape {
  int MS, NB;
};
SkinnyShape choose_skinny(int64_t M, int64_t N, int64_t K) {
  // {16, 8}: 128 columns, 145 KB of LDS (the 16 partial tiles), one workgroup per CU.
  static const SkinnyShape cand[] = {{4, 1}, {4, 2}, {4, 4}, {8, 1}, {8, 2}, {8, 4}, {16, 1}, {16, 2}, {16, 4}, {16, 8}};
  SkinnyShape best = {16, 1};
  double best_cost = -1.0;
  for (const SkinnyShape& c : cand) {
    if (c.MS > 4 && M <= c.MS / 2) continue;  // do not pad M by more than 2x
    const int64_t wgs = mxh::cdiv(mxh::cdiv(N, 16), c.NB) * mxh::cdiv(M, c.MS);
    const double per_wg = (double)c.MS * K * 2.0 + (double)c.NB * 16 * K / 2.0;
    const double cost = (double)mxh::cdiv(wgs, 256) * per_wg;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

// Split-K geometry for M <= 16: 64-column tiles, and as many K splits as make
// about one workgroup per CU (tiles x splits ~ 256), with at most kSpMaxSteps K
// steps per split. The workspace holds the complemented fp32 partials of all
// splits but the owner; it is all zero between calls.
struct SplitGeom {
  int MT = 0, T = 0, S = 0;
  size_t part_bytes = 0;
  double t_us = 0.0;  // the model's time for the chosen S
  bool ok = false;
  size_t total() const { return part_bytes; }
};
SplitGeom split_geom(int64_t M, int64_t N, int64_t K) {
  SplitGeom g;
  if (M < 1 || M > 16 || N < 1 || K < 32) return g;
  const int64_t KT = mxh::cdiv(K, 128);
  const int64_t T = mxh::cdiv(mxh::cdiv(N, 16), kSpW);
  const int64_t smin = mxh::cdiv(KT, kSpMaxSteps);
  if (smin > kSpMaxSplits || T * kSpMaxSplits > INT32_MAX) return g;
  // Pick S by a simple time model: a workgroup's loads take a latency plus its
  // bytes at one CU's streaming rate, rounds of more workgroups than CUs add up,
  // and splitting adds one device-scope hand-off to the owners, plus one more
  // poll round trip for every further batch of kSpBatch partials. (Measured at
  // M16 K7168, N 264..2112: 5.5-6.2 us with one batch, +0.6-1 us per batch.)
  int64_t S = smin;
  double best = -1.0;
  for (int64_t s = smin; s <= std::min<int64_t>(KT, kSpMaxSplits); ++s) {
    const double steps = (double)mxh::cdiv(KT, s);
    const double bytes = steps * (16.0 * 128 * 2 + kSpW * 1024.0 + kSpW * 256.0);  // A, B codes, B scales
    const double rounds = (double)mxh::cdiv(T * s, 256);
    const double batches = (double)mxh::cdiv(s - 1, kSpBatch);
    const double t = rounds * (1.0 + bytes / 25e3) + (s > 1 ? 1.5 * batches : 0.0);  // microseconds
    if (best < 0 || t < best - 1e-9) {
      best = t;
      S = s;
    }
  }
  g.MT = 1;
  g.T = (int)T;
  g.S = (int)S;
  g.part_bytes = (size_t)T * (size_t)(S - 1) * kSpW * g.MT * 64 * 16;
  g.t_us = best;
  g.ok = true;
  return g;
}

// Kernel of a fused call with M <= 16: the split-K kernel, unless its best
// split needs a hand-off (S > 1) and the skinny kernel (no hand-off: one
// workgroup's waves split K) is estimated at least 20 % faster (the two
// models are rough; near a tie the split-K kernel measured faster). The skinny estimate counts
// rounds of 256 workgroups, each a latency plus its bf16 A rows at the rate a
// CU reaches when every workgroup reads the same A from L2 (~60 GB/s) plus its
// packed B at one CU's HBM streaming rate (~25 GB/s). Wide N favours it
// (measured, split-K against skinny: M1 N4096 K7168 8.3 / 6.3 us, M16 N7168
// K2048 6.5 / 5.5 us), long K over few columns favours split-K (M16 N2112
// K7168 6.7 / 9.3 us, M16 N264 K7168 6.2 / 6.6 us).
bool fused_splitk(int64_t M, int64_t N, int64_t K, const SplitGeom& g) {
  if (!g.ok) return false;
  if (g.S == 1) return true;
  const SkinnyShape sh = choose_skinny(M, N, K);
  const int64_t wgs = mxh::cdiv(mxh::cdiv(N, 16), sh.NB) * mxh::cdiv(M, sh.MS);
  const double a_bytes = (double)sh.MS * (double)K * 2.0, b_bytes = (double)sh.NB * 16.0 * (double)K * 17.0 / 32.0;
  const double t = (double)mxh::cdiv(wgs, 256) * (1.0 + a_bytes / 60e3 + b_bytes / 25e3);
  return t >= 0.8 * g.t_us;
}

hipError_t launch_splitk(const Operand& o, const Dims& d, const SplitGeom& g, void* ws, bool preq, bool dump,
                         hipStream_t st) {
  Operand op = o;
  Dims dd = d;
  SplitArgs sa{};
  sa.part = (uint32_t*)ws;
  sa.S = g.S;
  void* args[] = {&op, &dd, &sa};
  const void* k = preq ? (const void*)gemm_splitk_kernel<1, true, false>
                  : dump ? (const void*)gemm_splitk_kernel<1, false, true>
                         : (const void*)gemm_splitk_kernel<1, false, false>;
  return hipLaunchKernel(k, dim3((unsigned)(g.T * g.S)), dim3(kSpT), args, 0, st);
}

hipError_t launch_tiled(const Operand& o, const Dims& d, int64_t M, int64_t N, bool preq, bool dump, hipStream_t st) {
  Operand op = o;
  Dims dd = d;
  int ntn = (int)mxh::cdiv(N, kTBN);
  void* args[] = {&op, &dd, &ntn};
  const int64_t tiles = mxh::cdiv(M, kTBM) * ntn;
  const void* k = preq ? (const void*)gemm_tiled_kernel<true, false>
                  : dump ? (const void*)gemm_tiled_kernel<false, true>
                         : (const void*)gemm_tiled_kernel<false, false>;
  return hipLaunchKernel(k, dim3((unsigned)tiles), dim3(kTThreads), args, 0, st);
}

// CUs counted by the host's kernel-choice models (the MI355X's), so that the
// choices they make, and the verification dump's layout, depend on the shapes
// alone.
constexpr int kModelCUs = 256;

// 16-row sub-tiles per small tile of the grouped kernel: a small problem with
// sub[i] sub-tiles and cols[i] 128-column tiles (times its batches) takes tiles
// of min(cap, sub[i]) sub-tiles. cap is the smallest count at which the launch
// (large_tiles besides) fits one round of workgroups on the device's CUs: more
// CUs stream each B, and each reads fewer A rows. When no count fits, every
// tile takes four sub-tiles (all rows of a group of at most 64), so fewer
// workgroups load each B byte.
int small_tile_cap(int64_t large_tiles, const int64_t* sub, const int64_t* cols, int n, int cus) {
  for (int c = 1; c < kGsMaxM / 16; ++c) {
    int64_t t = large_tiles;
    for (int i = 0; i < n; ++i) t += mxh::cdiv(sub[i], c) * cols[i];
    if (t <= cus) return c;
  }
  return kGsMaxM / 16;
}

// 16-column tiles per small tile of a grouped launch: kGsNB (128 columns), or
// half when every group is small and their 16 x 128 tiles fill at most half a
// round of kModelCUs workgroups (twice the workgroups, each reading half the B,
// as choose_skinny does for one problem). Counted on the model's CUs, so the
// dump layout depends on the shapes alone.
int small_nb(const int64_t* M, int n, int64_t N, int64_t small_max) {
  int64_t t = 0;
  for (int i = 0; i < n; ++i) {
    if (M[i] > small_max) return kGsNB;
    t += mxh::cdiv(M[i], 16) * mxh::cdiv(N, 16 * kGsNB);
  }
  return 2 * t <= kModelCUs ? kGsNB / 2 : kGsNB;
}

// Kernel of the single fused call for M > 64. The 128 x 512 tiled tile loads
// the fewest bytes per output, but a problem of a few hundred rows has few of
// them (M = 128, N = 4096: 8 tiles for 256 CUs), each bound by one CU's load
// rate. Skinny tiles spread such a problem over all CUs. Each option is
// estimated as rounds of workgroups on kModelCUs CUs, each round a fixed cost
// plus one workgroup's bytes (its bf16 A rows and packed B columns over the
// whole K) at one CU's rate, fitted to measurements at M 65..1024,
// N 1024..7168, K 1024..7168 (cold operands, graph replay):
//   tiled kernel (8 waves, 128 x 512)                  9.0 us + bytes / 70.4 KB/us
//   skinny kernel (16 waves, choose_skinny's tile)     3.2 us + bytes / 55.6 KB/us
//   grouped kernel's skinny tiles (8 waves, mt 16-row
//     sub-tiles x 128 columns, small_tile_cap's mt)    5.0 us + bytes / 53.0 KB/us
// The tiled kernel stays unless another is estimated at least 15 % faster. The
// model counts the MI355X's 256 CUs whatever the device, so the choice (and
// with it the verification dump's layout) depends on M, N and K alone.
enum class MidPath { kTiled, kSkinny, kRows };
constexpr int64_t kMidMaxM = 4096;  // larger M always takes the tiled kernel
// One workgroup's time (us) in the model: a tiled tile, a skinny-kernel tile of
// MS rows x 16*NB columns, a grouped-kernel skinny tile of mt sub-tiles.
double tiled_tile_us(int64_t K) { return 9.0 + (2.0 * kTBM + kTBN * 17.0 / 32.0) * (double)K / 70.4e3; }
double skinny_kernel_tile_us(int MS, int NB, int64_t K) {
  return 3.2 + (2.0 * MS + 16.0 * NB * 17.0 / 32.0) * (double)K / 55.6e3;
}
double skinny_tile_us(int64_t mt, int64_t K) {
  return 5.0 + (32.0 * mt + 16.0 * kGsNB * 17.0 / 32.0) * (double)K / 53.0e3;
}

struct MidTimes {
  double tiled, skinny, rows;
};
MidTimes mid_times(int64_t M, int64_t N, int64_t K) {
  const auto rounds = [](int64_t wgs) { return (double)mxh::cdiv(wgs, kModelCUs); };
  MidTimes t;
  t.tiled = rounds(mxh::cdiv(M, kTBM) * mxh::cdiv(N, kTBN)) * tiled_tile_us(K);
  const SkinnyShape sh = choose_skinny(M, N, K);
  t.skinny =
      rounds(mxh::cdiv(mxh::cdiv(N, 16), sh.NB) * mxh::cdiv(M, sh.MS)) * skinny_kernel_tile_us(sh.MS, sh.NB, K);
  const int64_t sub = mxh::cdiv(M, 16), cols = mxh::cdiv(N, 16 * kGsNB);
  const int64_t mt = std::min<int64_t>(small_tile_cap(0, &sub, &cols, 1, kModelCUs), sub);
  t.rows = rounds(mxh::cdiv(M, 16 * mt) * cols) * skinny_tile_us(mt, K);
  return t;
}

MidPath mid_path(int64_t M, int64_t N, int64_t K) {
  if (M <= 64 || M > kMidMaxM) return MidPath::kTiled;
  const MidTimes mtm = mid_times(M, N, K);
  const double t_tiled = mtm.tiled, t_sk = mtm.skinny, t_rows = mtm.rows;
  MidPath best = MidPath::kTiled;
  double t = 0.85 * t_tiled;
  if (t_sk < t) {
    t = t_sk;
    best = MidPath::kSkinny;
  }
  if (t_rows < t) best = MidPath::kRows;
  return best;
}

// gemm_a4w4 (pre-quantised A) past 16 rows: the skinny kernel up to 64 rows and
// where mid_path's estimate puts it at least 15 % ahead of the tiled kernel
// (there is no pre-quantised form of the grouped kernel's tiles), else tiled.
bool a4w4_skinny(int64_t M, int64_t N, int64_t K) {
  if (M <= 64) return true;
  if (M > kMidMaxM) return false;
  const MidTimes t = mid_times(M, N, K);
  return t.skinny < 0.85 * t.tiled;
}

// Which groups of a grouped launch take skinny tiles: those of at most
// small_max rows. small_max is 64, or the M of a group of at most
// kMidGroupMaxM rows when the model estimates that launch at least 15 % faster
// (a few mid-size groups leave most 128 x 512 tiles' CUs idle, as in mid_path).
// A launch is estimated as the longer of its longest tile and its rounds of
// kModelCUs workgroups times the mean tile time (exact for tiles of one
// length, which run in whole rounds). Problem p has M[p] rows, cols[p]
// 128-column tiles and big[p] 128 x 512 tiles (both times its batches) and K[p].
constexpr int64_t kMidGroupMaxM = 512;
double launch_us(const int64_t* M, const int64_t* cols, const int64_t* big, const int64_t* K, int n,
                 int64_t small_max) {
  int64_t large = 0, sub[MXFP4_MAX_GROUPS], scols[MXFP4_MAX_GROUPS], tiles = 0;
  int ns = 0;
  double total = 0.0, longest = 0.0;
  for (int p = 0; p < n; ++p) {
    if (M[p] <= small_max) {
      sub[ns] = mxh::cdiv(M[p], 16);
      scols[ns++] = cols[p];
    } else {
      large += big[p];
      tiles += big[p];
      total += (double)big[p] * tiled_tile_us(K[p]);
      longest = std::max(longest, tiled_tile_us(K[p]));
    }
  }
  const int64_t cap = small_tile_cap(large, sub, scols, ns, kModelCUs);
  for (int p = 0; p < n; ++p) {
    if (M[p] > small_max) continue;
    const int64_t mt = std::min(cap, mxh::cdiv(M[p], 16));
    const double t = skinny_tile_us(mt, K[p]);
    const int64_t n_p = mxh::cdiv(M[p], 16 * mt) * cols[p];
    tiles += n_p;
    total += (double)n_p * t;
    longest = std::max(longest, t);
  }
  if (tiles == 0) return 0.0;
  return std::max(longest, (double)mxh::cdiv(tiles, kModelCUs) * total / (double)tiles);
}
int64_t pick_small_max(const int64_t* M, const int64_t* cols, const int64_t* big, const int64_t* K, int n) {
  int64_t cand[MXFP4_MAX_GROUPS];
  int nc = 0;
  for (int p = 0; p < n; ++p)
    if (M[p] > kGsMaxM && M[p] <= kMidGroupMaxM) cand[nc++] = M[p];
  std::sort(cand, cand + nc);  // ascending: of equal estimates the smallest wins
  int64_t best = kGsMaxM;
  double t = 0.85 * launch_us(M, cols, big, K, n, kGsMaxM);
  for (int c = 0; c < nc; ++c) {
    const double tc = launch_us(M, cols, big, K, n, cand[c]);
    if (tc < t) {
      t = tc;
      best = cand[c];
    }
  }
  return best;
}
int64_t grouped_small_max(const mxfp4_group* groups, int G, int64_t N, int64_t K) {
  int64_t M[MXFP4_MAX_GROUPS], cols[MXFP4_MAX_GROUPS], big[MXFP4_MAX_GROUPS], Ks[MXFP4_MAX_GROUPS];
  for (int g = 0; g < G; ++g) {
    M[g] = groups[g].M;
    cols[g] = mxh::cdiv(N, 16 * kGsNB);
    big[g] = mxh::cdiv(M[g], kTBM) * mxh::cdiv(N, kTBN);
    Ks[g] = K;
  }
  return pick_small_max(M, cols, big, Ks, G);
}

int grouped_call(const mxfp4_group* groups, int G, int64_t N, int64_t K, void* dump, size_t dump_bytes, void* stream,
                 int64_t small_max);

// The skinny kernel with choose_skinny's tile, on bf16 A or (preq) pre-quantised A.
hipError_t launch_skinny_for(const Operand& o, const Dims& d, int64_t M, int64_t N, int64_t K, bool dump, bool preq,
                             hipStream_t st) {
  const SkinnyShape sh = choose_skinny(M, N, K);
  switch (sh.MS * 16 + sh.NB) {
    case 4 * 16 + 1: return launch_skinny<4, 1, 4>(o, d, M, dump, st, preq);
    case 4 * 16 + 2: return launch_skinny<4, 2, 4>(o, d, M, dump, st, preq);
    case 4 * 16 + 4: return launch_skinny<4, 4, 2>(o, d, M, dump, st, preq);
    case 8 * 16 + 1: return launch_skinny<8, 1, 4>(o, d, M, dump, st, preq);
    case 8 * 16 + 2: return launch_skinny<8, 2, 4>(o, d, M, dump, st, preq);
    case 8 * 16 + 4: return launch_skinny<8, 4, 2>(o, d, M, dump, st, preq);
    case 16 * 16 + 1: return launch_skinny<16, 1, 2>(o, d, M, dump, st, preq);
    case 16 * 16 + 2: return launch_skinny<16, 2, 2>(o, d, M, dump, st, preq);
    case 16 * 16 + 8: return launch_skinny<16, 8, 1>(o, d, M, dump, st, preq);
    default: return launch_skinny<16, 4, 2>(o, d, M, dump, st, preq);
  }
}

hipError_t launch_gemm(const Operand& o, const Dims& d, int64_t M, int64_t N, int64_t K, bool dump, hipStream_t st) {
  if (M <= 64 || mid_path(M, N, K) == MidPath::kSkinny) return launch_skinny_for(o, d, M, N, K, dump, false, st);
  return launch_tiled(o, d, M, N, false, dump, st);
}

// Copies of the quantised A that the fused call computes (one per N-tile of
// the kernel it runs): the leading dimension of the verification dump.
int64_t dump_copies(int64_t M, int64_t N, int64_t K) {
  const SplitGeom g = split_geom(M, N, K);
  if (fused_splitk(M, N, K, g)) return g.T;
  const MidPath mp = mid_path(M, N, K);
  if (M <= 64 || mp == MidPath::kSkinny) return mxh::cdiv(mxh::cdiv(N, 16), choose_skinny(M, N, K).NB);
  if (mp == MidPath::kRows) return mxh::cdiv(N, 16 * small_nb(&M, 1, N, M));
  return mxh::cdiv(N, kTBN);
}
size_t dump_bytes_of(int64_t M, int64_t N, int64_t K) {
  return (size_t)(dump_copies(M, N, K) * M * (K / 2 + K / 32));
}

}  // namespace

extern "C" int gemm_a4w4_fused_path(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 32 || K % 32 != 0 || M > mxh::kMaxDim || N > mxh::kMaxDim || K > mxh::kMaxDim) return 0;
  if (!offsets_fit(K, K)) return 0;  // rejected even with the smallest lda
  const SplitGeom g = split_geom(M, N, K);
  if (fused_splitk(M, N, K, g)) return MXFP4_PATH_SPLITK;
  if (M <= 64) return MXFP4_PATH_SKINNY;
  switch (mid_path(M, N, K)) {
    case MidPath::kSkinny: return MXFP4_PATH_SKINNY;
    case MidPath::kRows: return MXFP4_PATH_SKINNY_TILES;
    default: return MXFP4_PATH_TILED;
  }
}

extern "C" size_t gemm_a4w4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 32 || K % 32 != 0 || M > mxh::kMaxDim || N > mxh::kMaxDim || K > mxh::kMaxDim) return 0;
  const SplitGeom g = split_geom(M, N, K);
  // The split-K partials (gemm_a4w4 always runs that kernel for M <= 16; the
  // fused call may run the skinny kernel instead and then uses none of it).
  return g.ok ? g.total() : 0;  // larger M: every output tile is reduced inside one workgroup
}

namespace {
int fused_call(const void* A, int64_t lda, const void* Bp, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
               void* workspace, size_t workspace_bytes, void* dump, size_t dump_bytes, void* stream) {
  const int st = check_problem(A, lda, Bp, C, ldc, M, N, K);
  if (st != MXFP4_OK) return st;
  if (mxh::cdiv(M, kTBM) * mxh::cdiv(N, kTBN) > INT32_MAX) return MXFP4_ERR_SHAPE;
  if (mid_path(M, N, K) == MidPath::kRows) {  // one small group of the grouped kernel
    const mxfp4_group g{A, lda, Bp, C, ldc, M};
    return grouped_call(&g, 1, N, K, dump, dump_bytes, stream, M);
  }
  Operand o = make_operand(A, lda, Bp, C, ldc, M, N, K);
  if (dump) {
    if (dump_bytes < dump_bytes_of(M, N, K)) return MXFP4_ERR_BUFFER;
    if (!mxh::aligned(dump, 16)) return MXFP4_ERR_ALIGN;
    o.dq = (uint8_t*)dump;
    o.ds = (uint8_t*)dump + dump_copies(M, N, K) * M * (K / 2);
  }
  const Dims d = make_dims(N, K);
  const SplitGeom g = split_geom(M, N, K);
  if (fused_splitk(M, N, K, g)) {
    if (g.total() > 0) {
      if (!workspace || workspace_bytes < g.total()) return MXFP4_ERR_WORKSPACE;
      if (!mxh::aligned(workspace, 256)) return MXFP4_ERR_ALIGN;
    }
    return mxh::launch_status(launch_splitk(o, d, g, workspace, false, dump != nullptr, (hipStream_t)stream));
  }
  return mxh::launch_status(launch_gemm(o, d, M, N, K, dump != nullptr, (hipStream_t)stream));
}
}  // namespace

extern "C" int gemm_a4w4_fused(const void* A, int64_t lda, const void* Bp, void* C, int64_t ldc, int64_t M, int64_t N,
                               int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  return fused_call(A, lda, Bp, C, ldc, M, N, K, workspace, workspace_bytes, nullptr, 0, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free form of gemm_a4w4_fused, for callers that cannot allocate.
// ---------------------------------------------------------------------------
// The split-K partial slots (M <= 16) live in this fixed array instead of a
// caller workspace. Each GPU the library runs on holds its own copy for the
// life of the process; it is zero at load, and every completed call leaves the
// slots it used zero again (the tile owners clear them), so no call has to
// clear it first. Host code must not pass `scratch` itself to a kernel (that is
// a host-side stand-in): its device address comes from hipGetSymbolAddress,
// taken once per device with that device current.
static __device__ __align__(256) uint8_t scratch[MXFP4_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device a stream runs on (the current device for the null stream), and
// the current device.
int stream_device(void* stream, int* dev, int* cur) {
  if (hipGetDevice(cur) != hipSuccess) return MXFP4_ERR_HIP;
  *dev = *cur;
  if (stream) {
    hipDevice_t d = 0;
    if (hipStreamGetDevice((hipStream_t)stream, &d) != hipSuccess) return MXFP4_ERR_HIP;
    *dev = (int)d;
  }
  return *dev >= 0 && *dev < kMaxDevices ? MXFP4_OK : MXFP4_ERR_HIP;
}

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream), looked up once per device.
int scratch_address(void* stream, void** out) {
  int cur = 0, dev = 0;
  const int st = stream_device(stream, &dev, &cur);
  if (st != MXFP4_OK) return st;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return MXFP4_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return MXFP4_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MXFP4_OK;
}

// Compute units of the stream's device, read once per device.
std::atomic<int> g_cus[kMaxDevices];
int device_cus(void* stream, int* cus) {
  int cur = 0, dev = 0;
  const int st = stream_device(stream, &dev, &cur);
  if (st != MXFP4_OK) return st;
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return MXFP4_ERR_HIP;
    g_cus[dev].store(n, std::memory_order_relaxed);
  }
  *cus = n;
  return MXFP4_OK;
}
}  // namespace

extern "C" int gemm_a4w4_fused_noalloc(const void* A, int64_t lda, const void* Bp, void* C, int64_t ldc, int64_t M,
                                       int64_t N, int64_t K, void* stream) {
  const int st = check_problem(A, lda, Bp, C, ldc, M, N, K);
  if (st != MXFP4_OK) return st;
  const SplitGeom g = split_geom(M, N, K);
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (fused_splitk(M, N, K, g) && g.total() > 0) {
    if (g.total() > (size_t)MXFP4_NOALLOC_SCRATCH_BYTES) return MXFP4_ERR_WORKSPACE;  // beyond the fixed scratch
    const int s2 = scratch_address(stream, &ws);
    if (s2 != MXFP4_OK) return s2;
    ws_bytes = MXFP4_NOALLOC_SCRATCH_BYTES;
  }
  return fused_call(A, lda, Bp, C, ldc, M, N, K, ws, ws_bytes, nullptr, 0, stream);
}

extern "C" size_t gemm_a4w4_fused_dump_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 32 || K % 32 != 0 || M > mxh::kMaxDim || N > mxh::kMaxDim || K > mxh::kMaxDim) return 0;
  return dump_bytes_of(M, N, K);
}

extern "C" int gemm_a4w4_fused_dump(const void* A, int64_t lda, const void* Bp, void* C, int64_t ldc, int64_t M,
                                    int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* dump,
                                    size_t dump_bytes, void* stream) {
  if (!dump) return MXFP4_ERR_NULL;
  return fused_call(A, lda, Bp, C, ldc, M, N, K, workspace, workspace_bytes, dump, dump_bytes, stream);
}

extern "C" int gemm_a4w4(const void* Aq, int64_t ldaq, const void* As, int64_t ldas, const void* Bp, void* C,
                         int64_t ldc, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (!Aq || !As || !Bp || !C) return MXFP4_ERR_NULL;
  if (M < 1 || N < 1 || K < 32 || K % 32 != 0 || M > mxh::kMaxDim || N > mxh::kMaxDim || K > mxh::kMaxDim)
    return MXFP4_ERR_SHAPE;
  if (ldaq < K / 2 || ldas < K / 32 || ldc < N) return MXFP4_ERR_SHAPE;
  if (ldaq > (int64_t)1 << 24 || ldas > (int64_t)1 << 24) return MXFP4_ERR_SHAPE;  // 32-bit buffer offsets over 128 rows
  if (!offsets_fit(0, K)) return MXFP4_ERR_SHAPE;                                  // one packed B tile below 2^31 bytes
  if (!mxh::aligned(Aq, 16) || ldaq % 16 != 0 || !mxh::aligned(Bp, 16) || !mxh::aligned(C, 2)) return MXFP4_ERR_ALIGN;
  if (mxh::cdiv(M, kTBM) * mxh::cdiv(N, kTBN) > INT32_MAX) return MXFP4_ERR_SHAPE;
  const Operand o = make_operand_q(Aq, ldaq, As, ldas, Bp, C, ldc, M, N, K);
  const Dims d = make_dims(N, K);
  const SplitGeom g = split_geom(M, N, K);
  if (g.ok) {
    if (g.total() > 0) {
      if (!workspace || workspace_bytes < g.total()) return MXFP4_ERR_WORKSPACE;
      if (!mxh::aligned(workspace, 256)) return MXFP4_ERR_ALIGN;
    }
    return mxh::launch_status(launch_splitk(o, d, g, workspace, true, false, (hipStream_t)stream));
  }
  if (a4w4_skinny(M, N, K))
    return mxh::launch_status(launch_skinny_for(o, d, M, N, K, false, true, (hipStream_t)stream));
  return mxh::launch_status(launch_tiled(o, d, M, N, true, false, (hipStream_t)stream));
}

extern "C" size_t grouped_gemm_a4w4_workspace_bytes(const mxfp4_group* groups, int G, int64_t N, int64_t K) {
  (void)groups;
  (void)G;
  (void)N;
  (void)K;
  return 0;
}

namespace {
// Copies of a group's quantised A in the verification dump: one per column tile
// of the tile kind the group takes.
int64_t grouped_copies(int64_t M, int64_t N, int64_t small_max, int nb) {
  return M <= small_max ? mxh::cdiv(N, 16 * nb) : mxh::cdiv(N, kTBN);
}
int grouped_nb(const mxfp4_group* groups, int G, int64_t N, int64_t small_max) {
  int64_t M[MXFP4_MAX_GROUPS];
  for (int g = 0; g < G; ++g) M[g] = groups[g].M;
  return small_nb(M, G, N, small_max);
}

// Verification dump of the grouped call: group g's block (its copies, codes
// then scales, as for the single call) follows group g-1's.
size_t grouped_dump_bytes_of(const mxfp4_group* groups, int G, int64_t N, int64_t K, int64_t small_max) {
  const int nb = grouped_nb(groups, G, N, small_max);
  size_t t = 0;
  for (int g = 0; g < G; ++g)
    t += (size_t)(grouped_copies(groups[g].M, N, small_max, nb) * groups[g].M * (K / 2 + K / 32));
  return t;
}

// Groups of at most small_max rows take skinny tiles; small_max < 0 picks it
// by grouped_small_max (the grouped calls). The single fused call routes one
// group of any M here with small_max = M.
int grouped_call(const mxfp4_group* groups, int G, int64_t N, int64_t K, void* dump, size_t dump_bytes, void* stream,
                 int64_t small_max) {
  if (!groups) return MXFP4_ERR_NULL;
  if (G < 1 || G > MXFP4_MAX_GROUPS) return MXFP4_ERR_TOO_MANY_GROUPS;
  GroupedArgs a{};
  const int64_t ntn = mxh::cdiv(N, kTBN);
  for (int g = 0; g < G; ++g) {
    const mxfp4_group& q = groups[g];
    const int st = check_problem(q.A, q.lda, q.Bp, q.C, q.ldc, q.M, N, K);
    if (st != MXFP4_OK) return st;
    a.g[g] = make_operand(q.A, q.lda, q.Bp, q.C, q.ldc, q.M, N, K);
  }
  if (small_max < 0) small_max = grouped_small_max(groups, G, N, K);
  // A small group's tiles: 16-row sub-tiles x 128 columns, as many sub-tiles
  // per tile as small_tile_cap allows.
  int64_t large_tiles = 0, sub[MXFP4_MAX_GROUPS], cols[MXFP4_MAX_GROUPS];
  int nsmall = 0;
  for (int g = 0; g < G; ++g) {
    const int64_t M = groups[g].M;
    if (M <= small_max) {
      sub[nsmall] = mxh::cdiv(M, 16);
      cols[nsmall++] = mxh::cdiv(N, 16 * kGsNB);
    } else {
      large_tiles += mxh::cdiv(M, kTBM) * ntn;
    }
  }
  // 64-column small tiles (nb 4) only with 16-row tiles on the 16-wave kernel.
  const int nb = grouped_nb(groups, G, N, small_max);
  int64_t cap = kGsMaxM / 16;
  if (nb < kGsNB) {
    cap = 1;
  } else if (nsmall > 0) {
    int cus = 0;
    const int st = device_cus(stream, &cus);
    if (st != MXFP4_OK) return st;
    cap = small_tile_cap(large_tiles, sub, cols, nsmall, cus);
  }
  // Launch entries: the large groups in their order, then the small ones.
  int64_t total = 0;
  int e = 0;
  for (int small = 0; small < 2; ++small) {
    if (small) {
      a.small_from = e;
      a.nlarge = (int)total;
      a.nlarge_pad = (int)mxh::cdiv(total, 8) * 8;
    }
    for (int g = 0; g < G; ++g) {
      const int64_t M = groups[g].M;
      if ((M <= small_max) != (small != 0)) continue;
      const int64_t mt = std::min(cap, mxh::cdiv(M, 16));  // 16-row sub-tiles of a small tile
      const int64_t rows = small ? mxh::cdiv(M, 16 * mt) : mxh::cdiv(M, kTBM);
      a.order[e] = g;
      a.rows[e] = (int)rows;
      a.mt[e] = small ? (int)mt : 0;
      a.tile_start[e] = (int)total;
      total += rows * (small ? mxh::cdiv(N, 16 * nb) : ntn);
      if (total > INT32_MAX) return MXFP4_ERR_SHAPE;
      ++e;
    }
  }
  if (dump) {
    if (dump_bytes < grouped_dump_bytes_of(groups, G, N, K, small_max)) return MXFP4_ERR_BUFFER;
    if (!mxh::aligned(dump, 16)) return MXFP4_ERR_ALIGN;
    uint8_t* at = (uint8_t*)dump;
    for (int g = 0; g < G; ++g) {
      const int64_t copies = grouped_copies(groups[g].M, N, small_max, nb);
      a.g[g].dq = at;
      a.g[g].ds = at + copies * groups[g].M * (K / 2);
      at += copies * groups[g].M * (K / 2 + K / 32);
    }
  }
  a.tile_start[G] = (int)total;
  a.G = G;
  a.ntiles_n = (int)ntn;
  const int64_t grid = total + (a.nlarge_pad - a.nlarge);
  if (grid > INT32_MAX) return MXFP4_ERR_SHAPE;
  Dims d = make_dims(N, K);
  void* args[] = {&a, &d};
  if (large_tiles == 0 && cap == 1) {  // small groups only, 16-row tiles in one round
    const void* kern = nb < kGsNB ? (dump ? (const void*)gemm_grouped_small_kernel<kGsNB / 2, true>
                                          : (const void*)gemm_grouped_small_kernel<kGsNB / 2, false>)
                                  : (dump ? (const void*)gemm_grouped_small_kernel<kGsNB, true>
                                          : (const void*)gemm_grouped_small_kernel<kGsNB, false>);
    return mxh::launch_status(
        hipLaunchKernel(kern, dim3((unsigned)grid), dim3(kSkWaves * 64), args, 0, (hipStream_t)stream));
  }
  return mxh::launch_status(hipLaunchKernel(
      dump ? (const void*)gemm_grouped_kernel<true> : (const void*)gemm_grouped_kernel<false>, dim3((unsigned)grid),
      dim3(kTThreads), args, 0, (hipStream_t)stream));
}
}  // namespace

extern "C" int grouped_gemm_a4w4(const mxfp4_group* groups, int G, int64_t N, int64_t K, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  return grouped_call(groups, G, N, K, nullptr, 0, stream, -1);
}

namespace {
bool dump_shape_ok(const mxfp4_group* groups, int G, int64_t N, int64_t K) {
  if (!groups || G < 1 || G > MXFP4_MAX_GROUPS || N < 1 || N > mxh::kMaxDim || K < 32 || K % 32 != 0 ||
      K > mxh::kMaxDim)
    return false;
  for (int g = 0; g < G; ++g)
    if (groups[g].M < 1 || groups[g].M > mxh::kMaxDim) return false;
  return true;
}
}  // namespace

extern "C" size_t grouped_gemm_a4w4_dump_bytes(const mxfp4_group* groups, int G, int64_t N, int64_t K) {
  if (!dump_shape_ok(groups, G, N, K)) return 0;
  return grouped_dump_bytes_of(groups, G, N, K, grouped_small_max(groups, G, N, K));
}

extern "C" int64_t grouped_gemm_a4w4_dump_copies(const mxfp4_group* groups, int G, int64_t N, int64_t K, int g) {
  if (!dump_shape_ok(groups, G, N, K) || g < 0 || g >= G) return 0;
  const int64_t small_max = grouped_small_max(groups, G, N, K);
  return grouped_copies(groups[g].M, N, small_max, grouped_nb(groups, G, N, small_max));
}

extern "C" int grouped_gemm_a4w4_dump(const mxfp4_group* groups, int G, int64_t N, int64_t K, void* workspace,
                                      size_t workspace_bytes, void* dump, size_t dump_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!dump) return MXFP4_ERR_NULL;
  return grouped_call(groups, G, N, K, dump, dump_bytes, stream, -1);
}

extern "C" int grouped_gemm_a4w4_mnk(const mxfp4_group_mnk* groups, int G, void* stream) {
  if (!groups) return MXFP4_ERR_NULL;
  if (G < 1) return MXFP4_ERR_TOO_MANY_GROUPS;
  MnkArgs a{};
  int P = 0;
  // Every group is at most MXFP4_MAX_GROUPS problems, so G is at most that too.
  int64_t gM[MXFP4_MAX_GROUPS], gcols[MXFP4_MAX_GROUPS], gbig[MXFP4_MAX_GROUPS], gK[MXFP4_MAX_GROUPS];
  for (int g = 0; g < G; ++g) {
    const mxfp4_group_mnk& q = groups[g];
    if (q.L < 1) return MXFP4_ERR_SHAPE;
    if (q.L > MXFP4_MAX_GROUPS - P) return MXFP4_ERR_TOO_MANY_GROUPS;
    P += (int)q.L;
    const int st = check_problem(q.A, q.lda, q.Bp, q.C, q.ldc, q.M, q.N, q.K);
    if (st != MXFP4_OK) return st;
    const mxh::PackedGeom pg(q.N, q.K);
    if (q.L > 1) {  // batches: C slices must not overlap; every slice keeps the alignment rules
      if (q.strideA < 0 || q.strideB < (int64_t)pg.total() || q.strideC < q.M * q.ldc) return MXFP4_ERR_SHAPE;
      if ((q.strideA * 2) % 16 != 0 || q.strideB % 16 != 0) return MXFP4_ERR_ALIGN;
    }
    gM[g] = q.M;
    gcols[g] = q.L * mxh::cdiv(q.N, 16 * kGsNB);
    gbig[g] = q.L * mxh::cdiv(q.M, kTBM) * mxh::cdiv(q.N, kTBN);
    gK[g] = q.K;
  }
  // Problems of at most small_max rows take skinny tiles (as in the grouped call).
  const int64_t small_max = pick_small_max(gM, gcols, gbig, gK, G);
  int64_t large_tiles = 0, sub[MXFP4_MAX_GROUPS], cols[MXFP4_MAX_GROUPS];
  int nsmall = 0;
  for (int g = 0; g < G; ++g) {
    if (gM[g] <= small_max) {
      sub[nsmall] = mxh::cdiv(gM[g], 16);
      cols[nsmall++] = gcols[g];
    } else {
      large_tiles += gbig[g];
    }
  }
  // Small problems: tiles of min(cap, M/16) 16-row sub-tiles x 128 columns.
  int64_t cap = kGsMaxM / 16;
  if (nsmall > 0) {
    int cus = 0;
    const int st = device_cus(stream, &cus);
    if (st != MXFP4_OK) return st;
    cap = small_tile_cap(large_tiles, sub, cols, nsmall, cus);
  }
  P = 0;
  int64_t total = 0;
  for (int small = 0; small < 2; ++small) {
    if (small) {
      a.nlarge = (int)total;
      a.nlarge_pad = (int)mxh::cdiv(total, 8) * 8;
    }
    for (int g = 0; g < G; ++g) {
      const mxfp4_group_mnk& q = groups[g];
      if ((q.M <= small_max) != (small != 0)) continue;
      const mxh::PackedGeom pg(q.N, q.K);
      const int64_t mt = small ? std::min(cap, mxh::cdiv(q.M, 16)) : 0;
      const int64_t rows = small ? mxh::cdiv(q.M, 16 * mt) : 0;
      const int64_t tiles =
          small ? rows * mxh::cdiv(q.N, 16 * kGsNB) : mxh::cdiv(q.M, kTBM) * mxh::cdiv(q.N, kTBN);
      for (int64_t l = 0; l < q.L; ++l) {
        MnkProblem& o = a.p[P];
        o.A = (const uint16_t*)q.A + l * q.strideA;
        o.lda = q.lda;
        o.Bunit = (const uint8_t*)q.Bp + l * q.strideB;
        o.Bscale = (const uint32_t*)(o.Bunit + pg.code_bytes);
        o.C = (uint16_t*)q.C + l * q.strideC;
        o.ldc = q.ldc;
        o.M = (int)q.M;
        o.N = (int)q.N;
        o.K = (int)q.K;
        o.mt = (int)mt;
        o.rows = (int)rows;
        a.tile_start[P] = (int)total;
        total += tiles;
        if (total > INT32_MAX) return MXFP4_ERR_SHAPE;
        ++P;
      }
    }
  }
  a.tile_start[P] = (int)total;
  a.P = P;
  const int64_t grid = total + (a.nlarge_pad - a.nlarge);
  if (grid > INT32_MAX) return MXFP4_ERR_SHAPE;
  void* args[] = {&a};
  return mxh::launch_status(hipLaunchKernel((const void*)gemm_grouped_mnk_kernel, dim3((unsigned)grid),
                                            dim3(kTThreads), args, 0, (hipStream_t)stream));
}
