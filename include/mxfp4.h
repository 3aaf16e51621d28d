/*
 * mxfp4.h -- C ABI of libmxfp4.so: dynamic MXFP4 quantisation of a bf16
 * activation fused with a block-scaled FP4 GEMM, for MI355X (gfx950).
 *
 * Format (MXFP4, OCP Microscaling Formats v1.0): each element is an E2M1 code
 * (bit 3 sign, bits 0-2 magnitude index into {0, 0.5, 1, 1.5, 2, 3, 4, 6}),
 * two codes per byte with the first (even k) element in the low nibble; one
 * E8M0 scale byte s per 32 consecutive elements along K, value 2^(s-127).
 * Quantisation rule: scale exponent floor(log2(amax)) - 2 clamped to
 * [-127, 127], byte 127 for an all-zero block; each element x/2^e rounded to
 * the nearest E2M1 value, ties to the even code, saturating at +-6; the sign of
 * zero is kept. Sources: kernelbot amd-mxfp4-mm submission 517169 (module
 * docstring: E2M1 grid, per-1x32 scales, low nibble first; the fused
 * quant + GEMM plan), submission 683203 (docstring: scale byte 127 = 2^0,
 * allocation-free hot path). The pages state the shared exponent four
 * different ways (517169's docstring, its scale helper's docstring and its
 * code, and 683203's call into a helper whose body is absent) and round ties
 * upward; the rule taken here instead is the conversion rule of the OCP MX
 * v1.0 specification with round-to-nearest-even, the reading this library is
 * built and tested to.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless stated otherwise; the caller owns
 *    all memory. The library allocates nothing and holds no device state.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *    is enqueued on it asynchronously; no call synchronises.
 *  - All arguments are validated before any HIP call. On a validation error
 *    the call returns a non-zero status, launches nothing and leaves every
 *    output untouched. A failed launch returns MXFP4_ERR_HIP. Faults inside a
 *    kernel surface at the caller's next synchronising HIP call.
 *  - bf16 tensors are row-major with a row stride in ELEMENTS; byte tensors
 *    (packed fp4x2, E8M0 scales) have row strides in BYTES.
 *  - Inputs must be finite; NaN or Inf input gives unspecified output.
 */
#ifndef MXFP4_H
#define MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXFP4_OK = 0,
  MXFP4_ERR_NULL = 1,            /* a required pointer is NULL                          */
  MXFP4_ERR_SHAPE = 2,           /* M, N or K < 1, K % 32 != 0, a stride < row length,   */
                                 /* or a size beyond the supported range                */
  MXFP4_ERR_ALIGN = 3,           /* a pointer or row stride breaks the stated alignment  */
  MXFP4_ERR_WORKSPACE = 4,       /* workspace NULL or smaller than *_workspace_bytes()   */
  MXFP4_ERR_TOO_MANY_GROUPS = 5, /* G < 1 or G > MXFP4_MAX_GROUPS                        */
  MXFP4_ERR_HIP = 6,             /* the HIP runtime rejected a launch                    */
  MXFP4_ERR_BUFFER = 7,          /* an output buffer is smaller than the size required   */
  MXFP4_ERR_ARG = 8              /* a scalar argument is out of range (e.g. eps <= 0)    */
} mxfp4_status;

/* Static, human-readable name of a status code (never NULL). */
const char* mxfp4_status_str(int status);

/* ---------------------------------------------------------------------------
 * mxfp4_quant -- quantise a bf16 matrix X[M, K] to MXFP4 along K.
 * The standalone form of the quantisation steps of the fused path (page
 * 683203, ``_quant_shuffled``: one program per tile of A writing fp4x2 and
 * E8M0 bytes; here the scales are stored row-major, not shuffled).
 *   x : bf16 [M, K], row stride ldx elements (ldx >= K). x and ldx*2 must be
 *       multiples of 16 bytes.
 *   q : out, fp4x2 [M, K/2], row stride ldq bytes (ldq >= K/2). q and ldq
 *       must be multiples of 16 bytes.
 *   s : out, E8M0 [M, K/32], row stride lds bytes (lds >= K/32), no alignment.
 *   K % 32 == 0, M >= 1, K >= 32.
 * ------------------------------------------------------------------------- */
int mxfp4_quant(const void* x, int64_t ldx, void* q, int64_t ldq, void* s, int64_t lds,
                int64_t M, int64_t K, void* stream);

/* ---------------------------------------------------------------------------
 * mxfp4_rmsnorm_quant -- RMSNorm of each row of a bf16 matrix X[M, K] followed
 * by MXFP4 quantisation along K, in one launch: the fused RMSNorm + MXFP4
 * quantisation that page 683203 names (docstring trick 1, and the comment above
 * ``_quant_shuffled``) as the step before the GEMM in a transformer layer; the
 * pages print none of its arithmetic, so the norm is the standard one:
 *   ss  = sum_k x[k]^2, the exact sum taken in float64; the library adds the
 *         (exact) squares in one fixed order (64 lane sums per wave, lane t
 *         adding k = 512c + 8t + e over the wave's 512-element passes c in
 *         order and e = 0..7; a halving tree over the lanes; for K <= 8192
 *         the row's passes are split over four waves in order and their sums
 *         added in wave order), so results are reproducible bit for
 *         bit, and ss is within (K-1)*2^-53 relative of the exact sum; inv
 *         below differs from the value the exact sum (rounded once) gives only
 *         when that difference crosses an fp32 rounding boundary of inv;
 *   inv = fp32(1 / sqrt(ss / K + eps)), float64 steps;
 *   y   = bf16(fp32(fp32(x * inv) * w)), rounding to nearest even;
 *   (q, s) = the MXFP4 quantisation of y, exactly as mxfp4_quant.
 *   x   : bf16 [M, K], row stride ldx elements (ldx >= K); x and ldx*2 must be
 *         multiples of 16 bytes.
 *   w   : bf16 [K], 16-byte aligned.
 *   eps : finite, > 0; otherwise MXFP4_ERR_ARG.
 *   q   : out, fp4x2 [M, K/2], row stride ldq bytes (ldq >= K/2); q and ldq
 *         multiples of 4 bytes.
 *   s   : out, E8M0 [M, K/32], row stride lds bytes (lds >= K/32).
 *   K % 32 == 0, M >= 1, 32 <= K <= 2^29.
 * ------------------------------------------------------------------------- */
int mxfp4_rmsnorm_quant(const void* x, int64_t ldx, const void* w, float eps, void* q, int64_t ldq,
                        void* s, int64_t lds, int64_t M, int64_t K, void* stream);

/* ---------------------------------------------------------------------------
 * mxfp4_pack_B -- one-time, offline repacking of a quantised weight B[N, K]
 * into the library's MFMA-fragment layout (the idea of page 683203's scale
 * shuffle and page 496271's pre-arranged scale layout: lay the data out the way
 * the matrix instruction's lanes consume it, so that each wave fetches its
 * operand with one coalesced load).
 *   bq  : fp4x2 [N, K/2], contiguous (row stride K/2 bytes), 16-byte aligned.
 *   bs  : E8M0 [N, K/32], contiguous (row stride K/32 bytes).
 *   out : mxfp4_pack_B_bytes(N, K) bytes, 16-byte aligned; out_bytes is its
 *         size. Padding (N up to a multiple of 32, K up to a multiple of 64)
 *         holds code 0 and scale byte 127.
 * Layout of `out` (opaque to callers; stated for completeness):
 *   NT = ceil(N/32), KU = ceil(K/64), KG = ceil(KU/4).
 *   Codes: unit (t, u), t < NT, u < KU, is 1024 bytes at ((t*KU + u)*1024):
 *     bytes [16*l, 16*l+16) hold row 32t + l%32, elements
 *     k in [64u + 32(l/32), +32), for lane l = 0..63.
 *   Scales, at offset NT*KU*1024: dword (t, g, l) at ((t*KG + g)*64 + l)*4
 *     holds in byte i the scale of row 32t + l%32, 32-element chunk
 *     2(4g+i) + l/32.
 * ------------------------------------------------------------------------- */
size_t mxfp4_pack_B_bytes(int64_t N, int64_t K);
int mxfp4_pack_B(const void* bq, const void* bs, int64_t N, int64_t K, void* out, size_t out_bytes,
                 void* stream);

/* ---------------------------------------------------------------------------
 * gemm_a4w4_fused -- C[M, N] = Q(A) . B^T in one launch: A is quantised to
 * MXFP4 per 1x32 block along K inside the GEMM kernel (the quantised A never
 * reaches global memory), multiplied with the packed MXFP4 B on the scaled
 * FP4 matrix cores with fp32 accumulation, and rounded to bf16 (nearest,
 * ties to even). Page 517169 module docstring (the fused plan: load a bf16
 * tile, quantise on chip, dot against B, fp32 accumulate, bf16 store).
 *   A  : bf16 [M, K], row stride lda elements (lda >= K); A and lda*2 must be
 *        multiples of 16 bytes.
 *   Bp : output of mxfp4_pack_B(N, K).
 *   C  : out, bf16 [M, N], row stride ldc elements (ldc >= N), 2-byte aligned.
 *   workspace : device scratch of at least gemm_a4w4_workspace_bytes(M, N, K)
 *        bytes (may be NULL when that size is 0), 256-byte aligned, ZEROED BY
 *        THE CALLER ONCE after allocation; every call leaves it zeroed again.
 *        Calls that may run concurrently need distinct workspaces. It is used
 *        for M <= 16 when K is split over workgroups (page 683203, direct
 *        GEMM call: its split-K argument) and each tile's last split sums the
 *        others' fp32 partials, which pass through the workspace. For M <= 16
 *        with wide N the call may instead split K over the waves of one
 *        workgroup (faster there, no workspace used); the size above is
 *        always enough. Larger M needs none. Too small or NULL when needed:
 *        MXFP4_ERR_WORKSPACE; not 256-byte aligned: MXFP4_ERR_ALIGN.
 *   The kernel follows from (M, N, K) alone (gemm_a4w4_fused_path): for
 *   M <= 16 the split-K or the skinny kernel, for 16 < M <= 64 the skinny
 *   kernel, for larger M the tiled kernel (128 x 512 tiles), or, where that
 *   would leave most CUs idle (M up to a few hundred rows), the skinny kernel
 *   or the grouped kernel's skinny tiles.
 * ------------------------------------------------------------------------- */
size_t gemm_a4w4_workspace_bytes(int64_t M, int64_t N, int64_t K);
int gemm_a4w4_fused(const void* A, int64_t lda, const void* Bp, void* C, int64_t ldc, int64_t M,
                    int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * gemm_a4w4_fused_path -- the kernel that gemm_a4w4_fused (and its _noalloc
 * and _dump forms) runs for a shape: a pure function of (M, N, K), computed on
 * the host without a GPU. MXFP4_PATH_SPLITK: K split over workgroups (M <= 16).
 * MXFP4_PATH_SKINNY: MS rows x 16*NB columns per 1024-thread workgroup, K split
 * over its 16 waves. MXFP4_PATH_SKINNY_TILES: the skinny tiles that
 * grouped_gemm_a4w4 gives small groups (16 to 64 rows x 128 columns, K split
 * over 8 waves), for M > 64. MXFP4_PATH_TILED: 128 x 512 tiles. 0 for a shape
 * the call rejects (as MXFP4_ERR_SHAPE). Calls that run the same kernel on the
 * same operands give bit-identical C (gemm_a4w4's kernel choice is stated
 * with it). Not an operation of the pages: a query for callers and tests.
 * ------------------------------------------------------------------------- */
#define MXFP4_PATH_SPLITK 1
#define MXFP4_PATH_SKINNY 2
#define MXFP4_PATH_SKINNY_TILES 3
#define MXFP4_PATH_TILED 4
int gemm_a4w4_fused_path(int64_t M, int64_t N, int64_t K);

/* ---------------------------------------------------------------------------
 * gemm_a4w4_fused_noalloc -- gemm_a4w4_fused without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same kernels, tiling and arithmetic, so C equals
 * gemm_a4w4_fused's bit for bit. The split-K partials (M <= 16) go to a fixed
 * device array of MXFP4_NOALLOC_SCRATCH_BYTES bytes inside the library, one
 * per GPU, held until the process ends; a call that would run the split-K
 * kernel with more partials than that (gemm_a4w4_workspace_bytes(M, N, K) >
 * MXFP4_NOALLOC_SCRATCH_BYTES, e.g. M16 N1088 K65536) returns
 * MXFP4_ERR_WORKSPACE and launches nothing.
 * Every call on one GPU shares that GPU's array: calls that may overlap on one
 * GPU (different streams, or concurrent host threads) race and must not be
 * issued; use gemm_a4w4_fused with distinct workspaces for those. The first
 * call on a device looks up the array's device address (a HIP call, no
 * allocation); it runs on the device of `stream` (the current device for
 * NULL). Other arguments and errors as for gemm_a4w4_fused.
 * ------------------------------------------------------------------------- */
#define MXFP4_NOALLOC_SCRATCH_BYTES (4u << 20)
int gemm_a4w4_fused_noalloc(const void* A, int64_t lda, const void* Bp, void* C, int64_t ldc, int64_t M,
                            int64_t N, int64_t K, void* stream);

/* ---------------------------------------------------------------------------
 * gemm_a4w4_fused_dump -- verification form of gemm_a4w4_fused: the same
 * call (same kernel choice, tiling, arithmetic and C), whose kernels also
 * write the quantised A they compute on chip, so that it can be compared byte
 * for byte with the quantisation rule (page 517169 module docstring, step
 * "quantise on chip"; the fused path otherwise never stores it). Every N-tile
 * of the kernel quantises the whole of A again; each writes its own copy.
 *   dump : device buffer of at least gemm_a4w4_fused_dump_bytes(M, N, K)
 *          bytes, 16-byte aligned. With C = the number of copies (that size
 *          divided by M*(K/2 + K/32)), it receives codes [C][M][K/2] (fp4x2,
 *          rows contiguous) followed by scale bytes [C][M][K/32]. A scale
 *          byte is the one the matrix instruction receives: as mxfp4_quant's,
 *          except that an all-zero block (codes all 0 or 8) gets 0 instead of
 *          127, which gives the same (zero) products.
 *   Too small: MXFP4_ERR_BUFFER; NULL: MXFP4_ERR_NULL; misaligned:
 *   MXFP4_ERR_ALIGN. Every other argument as for gemm_a4w4_fused. Slower than
 *   gemm_a4w4_fused (the extra stores); meant for tests, not the hot path.
 * ------------------------------------------------------------------------- */
size_t gemm_a4w4_fused_dump_bytes(int64_t M, int64_t N, int64_t K);
int gemm_a4w4_fused_dump(const void* A, int64_t lda, const void* Bp, void* C, int64_t ldc, int64_t M,
                         int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* dump,
                         size_t dump_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * gemm_a4w4 -- C[M, N] = A_q . B^T with A ALREADY quantised (for example by
 * mxfp4_quant): the unfused pipeline of page 683203's anatomy (quantise A in
 * one launch, then run the block-scaled GEMM on A_q and its scales), kept as
 * a comparator for the fused call. Same arithmetic as gemm_a4w4_fused (exact
 * products of the same codes and scales, fp32 accumulation, bf16 rounding).
 * Kernel: split-K for M <= 16; past 16 rows the skinny kernel (pre-quantised
 * form) up to 64 rows and where the fused call's cost model estimates it at
 * least 15 % faster than the tiled kernel, else the tiled kernel. On the bytes
 * mxfp4_quant(A) produces it gives the fused call's C bit for bit where both
 * run the same kernel: for M <= 16 where gemm_a4w4_fused_path reports
 * MXFP4_PATH_SPLITK, for M > 16 where it reports MXFP4_PATH_SKINNY or
 * MXFP4_PATH_TILED.
 *   Aq : fp4x2 [M, K/2], row stride ldaq bytes (ldaq >= K/2, ldaq <= 2^24);
 *        Aq and ldaq must be multiples of 16 bytes.
 *   As : E8M0 [M, K/32], row stride ldas bytes (K/32 <= ldas <= 2^24).
 *   Bp, C, ldc, M, N, K, workspace : as for gemm_a4w4_fused, including the
 *        workspace size (gemm_a4w4_workspace_bytes(M, N, K)).
 * ------------------------------------------------------------------------- */
int gemm_a4w4(const void* Aq, int64_t ldaq, const void* As, int64_t ldas, const void* Bp, void* C, int64_t ldc,
              int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * grouped_gemm_a4w4 -- G independent fused problems C_g = Q(A_g) . B_g^T that
 * share N and K, in ONE launch (page 496271, ``custom_kernel``: a list of
 * per-group problems; there one launch per group, here a single launch whose
 * workgroups are spread over all groups' output tiles). A group of at most 64
 * rows takes output tiles of 16 to 64 rows x 128 columns (its B spread over
 * many CUs), a larger one 128 x 512 tiles. Groups of up to 512 rows take the
 * small tiles too when a cost model of the whole launch (a function of the
 * groups' M, N and K only) estimates it at least 15 % faster: a few such groups
 * leave most CUs idle on 128 x 512 tiles. The C of a group of at most 64 rows
 * is the same whatever the other groups are; a larger group's tile kind (and
 * so its fp32 summation order) can depend on them.
 *   groups : HOST array of G descriptors, read during the call only. Per
 *            group the same rules as gemm_a4w4_fused apply to A, lda, Bp, C,
 *            ldc; M >= 1.
 *   1 <= G <= MXFP4_MAX_GROUPS.
 *   workspace : as for gemm_a4w4_fused, sized by
 *            grouped_gemm_a4w4_workspace_bytes().
 * ------------------------------------------------------------------------- */
#define MXFP4_MAX_GROUPS 32
typedef struct {
  const void* A;
  int64_t lda;
  const void* Bp;
  void* C;
  int64_t ldc;
  int64_t M;
} mxfp4_group;

size_t grouped_gemm_a4w4_workspace_bytes(const mxfp4_group* groups, int G, int64_t N, int64_t K);
int grouped_gemm_a4w4(const mxfp4_group* groups, int G, int64_t N, int64_t K, void* workspace,
                      size_t workspace_bytes, void* stream);

/* grouped_gemm_a4w4_dump -- verification form of grouped_gemm_a4w4 (same
 * launch and C), also writing each group's on-chip quantised A as
 * gemm_a4w4_fused_dump does: group g's block (C_g copies, one per column tile
 * of the group's tile kind: codes [C_g][M_g][K/2], then scale bytes
 * [C_g][M_g][K/32]) follows group g-1's.
 * dump: at least grouped_gemm_a4w4_dump_bytes(groups, G, N, K) bytes,
 * 16-byte aligned.
 * grouped_gemm_a4w4_dump_copies(groups, G, N, K, g) gives C_g: ceil(N/128) for a
 * group on skinny tiles (ceil(N/64) when only small groups share the launch and
 * 128-column tiles would leave most CUs idle), ceil(N/512) for one on tiled
 * tiles; it depends on the whole list (see grouped_gemm_a4w4). 0 for an invalid
 * list, N, K or g. */
size_t grouped_gemm_a4w4_dump_bytes(const mxfp4_group* groups, int G, int64_t N, int64_t K);
int64_t grouped_gemm_a4w4_dump_copies(const mxfp4_group* groups, int G, int64_t N, int64_t K, int g);
int grouped_gemm_a4w4_dump(const mxfp4_group* groups, int G, int64_t N, int64_t K, void* workspace,
                           size_t workspace_bytes, void* dump, size_t dump_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * grouped_gemm_a4w4_mnk -- G groups of fused problems with their OWN (M, N, K)
 * and a batch count L each, in ONE launch: page 496271's problem form
 * (``custom_kernel``: a list of groups, each with its problem size (m, n, k, l)
 * and tensors carrying a batch index l; there one launch per group and per l,
 * here one launch over every problem's output tiles). Batch l of group g is
 *   C_l = Q(A_l) . B_l^T,  A_l = A + l*strideA (elements), B_l = Bp + l*strideB
 *   (bytes, each an mxfp4_pack_B(N, K) image), C_l = C + l*strideC (elements).
 *   Per batch the rules of gemm_a4w4_fused apply to A, lda, B, C, ldc, M, N, K
 *   (each batch row-major with unit stride along K; page 496271's layout with
 *   the batch index innermost is transposed by the caller).
 *   L >= 1. For L > 1: strideA >= 0 with strideA*2 a multiple of 16; strideB >=
 *   mxfp4_pack_B_bytes(N, K), a multiple of 16; strideC >= M*ldc (the C slices
 *   do not overlap); otherwise MXFP4_ERR_SHAPE / MXFP4_ERR_ALIGN.
 *   The sum of L over the groups is at most MXFP4_MAX_GROUPS
 *   (else MXFP4_ERR_TOO_MANY_GROUPS). No workspace. A problem takes skinny or
 *   128 x 512 tiled tiles by the same rule as a group of grouped_gemm_a4w4 (its
 *   model counts every problem's own N and K).
 *   groups : HOST array of G descriptors, read during the call only.
 * ------------------------------------------------------------------------- */
typedef struct {
  const void* A;
  int64_t lda;
  int64_t strideA;
  const void* Bp;
  int64_t strideB;
  void* C;
  int64_t ldc;
  int64_t strideC;
  int64_t M, N, K, L;
} mxfp4_group_mnk;

int grouped_gemm_a4w4_mnk(const mxfp4_group_mnk* groups, int G, void* stream);

/* ---------------------------------------------------------------------------
 * grouped_gemm_nvfp4 -- the NVFP4 block-scaled GEMM of page 496271
 * (kernelbot nvfp4-group-gemm: module docstring, constants block,
 * ``nvfp4_gemm_kernel``, ``custom_kernel``) for G groups with their own
 * (M, N, K) and batch count L, in ONE launch. Both operands arrive quantised:
 *   C_l[m, n] = sum_k deq(A_l)[m, k] * deq(B_l)[n, k],   deq(X)[r, k] =
 *     E2M1(code of element k of row r) * E4M3(Xs[r, k / 16]),
 * accumulated in fp32 and stored as float16 (round to nearest even; overflow
 * gives infinity). No per-tensor scale (the page applies none).
 *   Aq : E2M1 codes [M, K/2], two per byte, element 2j in the low nibble of
 *        byte j, sign in bit 3 (the MXFP4 nibble order); row stride lda bytes,
 *        8-byte aligned, lda a multiple of 8, lda >= K/2.
 *   As : E4M3 (OCP FP8 E4M3: bias 7, no infinities, 0x7F/0xFF NaN) scale bytes
 *        [M, K/16] row-major (the page's reordered layout is not used), row
 *        stride ldas >= K/16 bytes, any alignment.
 *   Bq, ldb, Bs, ldbs : the same for B [N, K].
 *   C  : float16 [M, N], row stride ldc >= N elements, 2-byte aligned.
 *   M, N >= 1; K >= 16 with K % 16 == 0 (else MXFP4_ERR_SHAPE). Code bytes of
 *   elements past K in a row are ignored (any value); scale bytes past K/16
 *   are ignored. A NaN scale inside K makes the affected C entries NaN.
 *   (M + 128) * lda, (M + 128) * ldas, (N + 128) * ldb and (N + 128) * ldbs
 *   must stay below 2^31 (else MXFP4_ERR_SHAPE).
 *   Batch l uses Aq + l*strideA, As + l*strideAs, Bq + l*strideB,
 *   Bs + l*strideBs (bytes) and C + l*strideC (elements). L >= 1; for L > 1
 *   the strides are >= 0, strideA and strideB multiples of 8
 *   (MXFP4_ERR_ALIGN), strideC >= M*ldc (MXFP4_ERR_SHAPE).
 *   The sum of L over the groups is at most MXFP4_MAX_GROUPS
 *   (else MXFP4_ERR_TOO_MANY_GROUPS). No workspace.
 *   groups : HOST array of G descriptors, read during the call only.
 * ------------------------------------------------------------------------- */
typedef struct {
  const void* Aq;
  int64_t lda;
  int64_t strideA;
  const void* As;
  int64_t ldas;
  int64_t strideAs;
  const void* Bq;
  int64_t ldb;
  int64_t strideB;
  const void* Bs;
  int64_t ldbs;
  int64_t strideBs;
  void* C;
  int64_t ldc;
  int64_t strideC;
  int64_t M, N, K, L;
} nvfp4_group;

int grouped_gemm_nvfp4(const nvfp4_group* groups, int G, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
