/*
 * mmq.h -- C ABI of the block-quantized int8 MMQ library for AMD MI355X
 * (gfx950).
 *
 * The operation ("When the Product Won't Collapse: A Negative Result on int8
 * Tensor-Core MMQ", section 2, the displayed contraction):
 *
 *     out[m,n] = sum over 32-element k-blocks b of
 *                (activation scale[m,b] * weight scale[n,b]) * I[m,n,b],
 *     I[m,n,b] = exact int32 dot of the 32 activation codes of row m and the
 *                32 weight codes of row n inside block b.
 *
 * For Q4_K weights the block term is the affine identity of "When Does a
 * Kernel Win Surface?" (section 6.2): d*sc * xs * I - dmin*m * xsum, with
 * (sc, m) the 6-bit scale and min of the weight sub-block and xsum the
 * activation block-sum field of q8_1.  Activations are quantized to q8_1 once
 * per GEMM input by a separate pass ("13 . r7-r8 raw-byte MMQ kernel",
 * section 3.2, quantize pass; the same page's section 1 keeps it a pass of
 * its own).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or synchronises; work is enqueued on `stream`
 *    (a hipStream_t passed as void*; NULL is the null stream) and runs
 *    asynchronously.
 *  - Return value: 1 = launched; 0 = refused.  A refusal enqueues nothing and
 *    writes no output byte; the reason is returned by mmq_last_error() and
 *    printed to stderr.  The library never falls back silently: a caller that
 *    wants a fallback decides it ("13 . r7-r8 raw-byte MMQ kernel", section
 *    3.3: a launch that fails must be reported, never mistaken for success).
 *  - Refusal causes, all checked on the host before any device work: null
 *    pointer, M/N/K < 1, K not a multiple of the format's block, a pointer not
 *    16-byte aligned (4-byte for `out`/`dots`), sizes beyond int32 tile
 *    indexing, no HIP device or a device that is not gfx950, a launch plan
 *    whose LDS exceeds the device's per-workgroup maximum, and any launch
 *    error reported by hipGetLastError().
 *  - Faults that happen asynchronously on the device surface at the caller's
 *    next synchronisation and are outside this contract.
 *  - Inputs must be finite; non-finite activations give unspecified codes.
 *  - Thread safety: entry points may be called from several host threads; the
 *    only global state is a per-device limits cache and a thread-local error
 *    string.
 *
 * Byte layouts (little-endian, blocks packed back to back, row-major over
 * blocks):
 *  - q8_1 activation block, 36 B per 32 values: fp16 d @0, fp16 s @2 where
 *    s = fp16(d * sum of codes), 32 x int8 codes @4.
 *  - Q8_0 weight block, 34 B per 32 values: fp16 d @0, 32 x int8 codes @2.
 *  - Q4_K weight super-block, 144 B per 256 values: fp16 d @0, fp16 dmin @2,
 *    12 B of packed 6-bit sub-block scales and mins @4 (GGUF K-quant packing),
 *    128 B of 4-bit codes @16 where code byte 32*g + i holds element 64*g + i
 *    in its low nibble and element 64*g + 32 + i in its high nibble.
 */
#ifndef MMQ_H
#define MMQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MMQ_FMT_Q8_0 0
#define MMQ_FMT_Q4_K 1
#define MMQ_FMT_Q5_K 2
#define MMQ_FMT_Q6_K 3

/* Quantize fp32 activations to q8_1 ("13 . r7-r8 raw-byte MMQ kernel",
 * section 3.2; q8_1 fields from "When Does a Kernel Win Surface?", 6.2).
 *   x: M x K fp32, row-major (leading dimension K), 16-byte aligned.
 *   y: M x (K/32) q8_1 blocks (36 B each), row-major, 16-byte aligned.
 * Per block: amax = max |x|, d = amax/127 (fp32, correctly rounded),
 * code = round-half-away(x * (1/d)) clamped to [-127, 127] (d = 0, or a d
 * so small that 1/d overflows fp32, gives all codes 0), s = fp16(d * sum of
 * codes).  Requires K % 32 == 0. */
int mmq_quantize_q8_1(const float *x, void *y, int64_t M, int64_t K, void *stream);

/* q8_1 activations x Q8_0 weights -> fp32 ("When the Product Won't
 * Collapse", section 2).
 *   x_q8_1: M x (K/32) q8_1 blocks; w_q8_0: N x (K/32) Q8_0 blocks;
 *   out: M x N fp32 row-major (leading dimension N), fully overwritten.
 * Per block the weight scale multiplies the integer dot first (one
 * rounding) and the activation scale is then fused into the fp32 running
 * sum, blocks in ascending order from 0.  Requires K % 32 == 0 (any whole
 * number of Q8_0 blocks).
 * Shapes with too few 128 x 128 output tiles to occupy the device are split
 * along K into two slices (mmq_plan_describe reports split_k): the library
 * first zeroes `out` with a kernel on `stream`, then each slice adds its
 * partial sums with fp32 atomics.  A two-term sum onto an exact zero rounds
 * the same in either order, so the result is the same on every run, but it
 * is not the single ascending-order sum (a few ulp apart; Q8_0 is then not
 * bit-identical to the one-pass order).  mmq_gemm_multi_ws splits such
 * shapes further through a caller workspace, also reproducibly.
 * M <= 8 (decode; "When Does a Kernel Win Surface?", sections 2 and 8: the
 * matvec contraction, bound by the weight stream) runs a matrix-vector
 * kernel instead: each weight row is read once for all M activation rows
 * and its blocks are summed per lane and then across the 64 lanes of a
 * wave, a fixed order (the same on every run) other than ascending.
 * mmq_plan_describe reports kernel=mv for such shapes.  The large decode
 * launches (N >= 16384 or K > 8192) take the batch-decode kernel below from
 * the M where it measured faster: M >= 4 for Q8_0, M >= 4 (wide) or 7
 * (long K) for Q6_K, M >= 6 for the long-K launches of Q4_K and Q5_K.
 * 9 <= M <= 32 (batched decode) runs a matrix-core kernel of 32 weight rows
 * per workgroup instead (kernel=sm): one int8 MFMA per block with the
 * activation rows as its other operand, the per-block scale arithmetic
 * above (the K-quant min term on the matrix core too: two blocks per fp32
 * MFMA), four K-slices each summed in ascending order and then added in
 * slice order; narrow shapes split K over two workgroups more, added into
 * the zeroed output by fp32 atomics as above.  The same kernel takes
 * 33 <= M <= 192 in blocks of 32 activation rows when N has fewer 128-wide
 * tiles than the device has compute units.  The result is the same on every
 * run. */
int mmq_gemm_q8_0(const void *x_q8_1, const void *w_q8_0, float *out,
                  int64_t M, int64_t N, int64_t K, void *stream);

/* Tile-packed Q8_0 weights: the bytes of an N x K Q8_0 matrix (the
 * contraction's weight operand, "When the Product Won't Collapse", section
 * 2) reordered once, on the device, into the order in which the GEMM kernel
 * stages them, so that each k-step's weight codes reach LDS by DMA with no
 * register or VALU work.  The layout is this library's own: for every
 * 128-column tile and every step of 4 blocks, 17408 bytes -- the 4 x 128
 * blocks' 32 code bytes as [block][column][32 bytes], the two 16-byte
 * halves swapped for the columns c (within the tile) whose bits 2 and 3
 * differ, then their fp16 scales [block][column] -- with columns past N
 * and blocks past K/32 zero.  No
 * byte of the weights is converted; the scales are decoded in the GEMM, as
 * for the row-major form.
 * mmq_packed_bytes_q8_0: the packed size for N x K (N >= 1, K a multiple of
 * 32 in 32..8388608), or -1 (reason in mmq_last_error).
 * mmq_pack_q8_0: w_q8_0 (N x (K/32) Q8_0 blocks, 16-byte aligned, caller
 * owned, read only) -> packed (at least mmq_packed_bytes_q8_0(N, K) bytes,
 * 16-byte aligned, caller owned, every byte of the packed form written),
 * one kernel on `stream`.  Refuses (0) a short buffer or a bad shape. */
int64_t mmq_packed_bytes_q8_0(int64_t N, int64_t K);
int mmq_pack_q8_0(const void *w_q8_0, int64_t N, int64_t K, void *packed, int64_t packed_bytes,
                  void *stream);

/* mmq_gemm_q8_0 on weights packed by mmq_pack_q8_0 for the same N and K:
 * the same arithmetic in the same order, so out is bit-identical to
 * mmq_gemm_q8_0's on every shape the tile kernel runs.  Every M runs the
 * tile kernel (the decode kernels read the row-major form), with the same
 * split-K rule and its atomics.  w_packed: mmq_packed_bytes_q8_0(N, K)
 * bytes, 16-byte aligned; x_q8_1, out and the refusals as for
 * mmq_gemm_q8_0. */
int mmq_gemm_q8_0_packed(const void *x_q8_1, const void *w_packed, float *out,
                         int64_t M, int64_t N, int64_t K, void *stream);

/* q8_1 activations x Q4_K weights -> fp32 ("When Does a Kernel Win
 * Surface?", section 6.2, affine identity with the min term folded in
 * through the q8_1 block-sum field).
 *   x_q8_1: M x (K/32) q8_1 blocks; w_q4_K: N x (K/256) super-blocks;
 *   out: M x N fp32 row-major, fully overwritten.  Requires K % 256 == 0.
 * Split-K and M <= 8 shapes behave as for mmq_gemm_q8_0, except that with
 * K <= 8192 and either M = 8 or 3 <= M and N >= 16384 the few rows run on
 * the matrix core instead (mmq_plan_describe reports mv_mfma=1): one int8
 * MFMA per block over 32 weight rows, the activation rows as its other
 * operand, each output summed by one lane over a quarter of the blocks in
 * ascending order and the four quarters then added in order.  9 <= M <= 32
 * as for mmq_gemm_q8_0. */
int mmq_gemm_q4_K(const void *x_q8_1, const void *w_q4_K, float *out,
                  int64_t M, int64_t N, int64_t K, void *stream);

/* q8_1 activations x Q5_K weights -> fp32 (a K-quant family "When Does a
 * Kernel Win Surface?" names in section 2; block term: the Q4_K affine
 * identity of its section 6.2 with 5-bit codes).
 *   x_q8_1: M x (K/32) q8_1 blocks; w_q5_K: N x (K/256) super-blocks of
 *   176 B (fp16 d @0, fp16 dmin @2, 12 B of 6-bit scales/mins @4 packed as
 *   for Q4_K, 32 B of high bits @16, 128 B of low nibbles @48 in the Q4_K
 *   order; the code of element e is its nibble + 16 * bit (e/32) of
 *   high-bit byte e%32); out: M x N fp32 row-major, fully overwritten.
 *   Requires K % 256 == 0.  Split-K, M <= 8 and 9 <= M <= 32 shapes behave
 *   as for mmq_gemm_q8_0. */
int mmq_gemm_q5_K(const void *x_q8_1, const void *w_q5_K, float *out,
                  int64_t M, int64_t N, int64_t K, void *stream);

/* q8_1 activations x Q6_K weights -> fp32 (a K-quant the pages name with
 * 16-element scale groups and 6-bit codes centred at 32: "When Does a Kernel
 * Win Surface?", section 4.1).
 *   x_q8_1: M x (K/32) q8_1 blocks; w_q6_K: N x (K/256) super-blocks of
 *   210 B (128 B of low four bits @0, 64 B of high two bits @128, 16 int8
 *   scales @192, fp16 d @208; element e, with h = e/128, q = (e%128)/32 and
 *   l = e%32, takes nibble q/2 of byte 64h + 32(q%2) + l and bits 2q, 2q+1 of
 *   byte 128 + 32h + l, and the scale byte 192 + e/16); out: M x N fp32
 *   row-major, fully overwritten.  Requires K % 256 == 0.
 * Per 16-element group (two per 32-block, in order) the weight scale d*sc
 * multiplies the exact integer dot of the activation codes with the centred
 * codes (code - 32) first (one rounding), and the activation scale of the
 * block is then fused into the running sum: the same arithmetic, in the
 * same order, as a single pass over the groups, so unsplit tile-kernel
 * shapes are bit-identical to it.  Split-K, M <= 8 (the matrix-vector
 * kernel, one term per 16-element group) and 9 <= M <= 32 (one term per
 * 16-element group as here, in four K-slices) as for mmq_gemm_q8_0. */
int mmq_gemm_q6_K(const void *x_q8_1, const void *w_q6_K, float *out,
                  int64_t M, int64_t N, int64_t K, void *stream);

/* Several GEMMs of one format that read the same q8_1 activations (the
 * layer pipeline of "13 . r7-r8 raw-byte MMQ kernel": quantize once per
 * distinct input, e.g. the q, k and v projections, or gate and up), computed
 * by one launch whose grid covers the column tiles of all of them (for
 * M <= 8, the output rows of all of them, in the matrix-vector kernel; in
 * the batch-decode kernel, their groups of 32 output rows, a group never
 * holding rows of two of them).
 *   fmt: MMQ_FMT_Q8_0, MMQ_FMT_Q4_K, MMQ_FMT_Q5_K or MMQ_FMT_Q6_K; count: 1..8;
 *   x_q8_1: M x (K/32) q8_1 blocks, shared;
 *   w[g]: N[g] x K weights of format fmt; out[g]: M x N[g] fp32 row-major,
 *   fully overwritten; the arrays w, out and N are host memory (read during
 *   the call), the tensors device memory.
 * Each out[g] equals what mmq_gemm_q8_0 / _q4_K / _q5_K / _q6_K would write
 * for (x, w[g], N[g]), except that split-K, for M <= 8 the choice between
 * the two few-row kernels (Q4_K, Q5_K), and for 33 <= M <= 192 the choice
 * between the batch-decode and the tile kernel, are decided for the set as
 * a whole (the summation order, and so the last bits, can then differ from
 * the member's own launch).
 * Refused (nothing launched) when any member would be refused. */
int mmq_gemm_multi(int fmt, const void *x_q8_1, int count, const void *const *w, float *const *out,
                   const int64_t *N, int64_t M, int64_t K, void *stream);

/* Bytes of device workspace mmq_gemm_multi_ws needs for this GEMM set on the
 * current device: 0 when its plan does not split K (then the workspace may be
 * NULL), else 4 bytes per output tile of arrival counters (padded to 256 B)
 * plus split_k x 64 KiB of fp32 partial sums per 128 x 128 output tile: at
 * most 2 x (compute units) x 64 KiB plus the counters (32 MiB on MI355X,
 * whose 256 CUs hold two workgroups each).  -1 when the
 * set would be refused (reason in mmq_last_error()).  The size depends on the
 * device (its compute-unit count), so query it on the device that runs the
 * GEMMs. */
int64_t mmq_gemm_workspace_bytes(int fmt, int count, const int64_t *N, int64_t M, int64_t K);

/* mmq_gemm_multi with a split-K workspace ("When Does a Kernel Win Surface?",
 * section 4.5, on occupying the device when the output has few tiles): the
 * same GEMMs, but shapes with few output tiles may be split into more than
 * two K slices.  Each slice stores its partial tile in the workspace; the
 * last slice of a tile to finish (an arrival counter per tile, zeroed by a
 * kernel on `stream` before the GEMM) sums the partials in slice order
 * 0, 1, ... and writes the tile, so the result is the same on every run.
 * mmq_plan_describe reports the split as ws_split_k.
 *   workspace: device memory of workspace_bytes >= mmq_gemm_workspace_bytes
 *   for the same arguments, 16-byte aligned, owned by the caller; its
 *   contents need no preparation and are clobbered.  NULL with 0 bytes
 *   behaves as mmq_gemm_multi.  Two calls that run at the same time must not
 *   share a workspace.
 * Refused, in addition to mmq_gemm_multi's causes, when the workspace is
 * smaller than the plan needs or misaligned. */
int mmq_gemm_multi_ws(int fmt, const void *x_q8_1, int count, const void *const *w, float *const *out,
                      const int64_t *N, int64_t M, int64_t K, void *workspace, int64_t workspace_bytes,
                      void *stream);

/* Bytes of device workspace mmq_moe_gemm needs for T tokens routed to topk
 * experts each among n_experts: a 32-byte header, a tile table (16 B per
 * possible 128-row tile, floor(T*topk/128) + min(n_experts, T*topk) of
 * them), a list of small remainders (16 B per expert) and the routed row ids
 * sorted by expert (4 B each, rounded up to 16 B).  -1 for arguments
 * mmq_moe_gemm refuses outright (topk outside 1..64, n_experts outside
 * 1..2048, T < 0). */
int64_t mmq_moe_workspace_bytes(int64_t T, int topk, int n_experts);

/* Indexed-MoE GEMM ("When Does a Kernel Win Surface?", section 4.5, the fused
 * indexed-MoE prefill GEMM): each token's q8_1 activation row is multiplied
 * by the weights of each of the topk experts it was routed to, all in one
 * launch, with every 128-row tile holding rows of a single expert.
 *   x_q8_1: T x (K/32) q8_1 blocks (device);
 *   fmt: MMQ_FMT_Q8_0, MMQ_FMT_Q4_K, MMQ_FMT_Q5_K or MMQ_FMT_Q6_K;
 *   w: n_experts weight matrices of format fmt stored one after another,
 *      each N x K (N rows of K/32 Q8_0 blocks or K/256 Q4_K / Q5_K
 *      super-blocks, the layout the dense GEMMs take) (device);
 *   ids: int32 [T][topk] expert ids (device); routed row r = t*topk + j is
 *      token t times expert ids[r];
 *   out: (T*topk) x N fp32 row-major (device); row r is routed row r.
 *   workspace: at least mmq_moe_workspace_bytes(T, topk, n_experts) bytes of
 *      16-byte aligned device memory, caller-owned; its contents on entry do
 *      not matter and on return are the routing tables.
 * An expert's routed rows fill 128-row tiles of the tile kernel, except a
 * last partial tile of at most 32 rows, which a second launch computes one
 * wave per 32 weight rows over the whole of K (so a decode-sized call, at
 * most 32 rows per expert, runs on that launch alone).  Both compute every
 * output element with the tile kernel's per-block arithmetic in ascending
 * block order, so row r of out equals the tiled dense GEMM's row for token
 * t and expert ids[r]'s matrix, bit-identical for Q8_0 and Q6_K (for Q4_K
 * and Q5_K the min term is added per k-step on the matrix core in the
 * tiles and per sub-block in the second launch: equal within rounding).
 * A routed row whose id is outside [0, n_experts) is not computed and its
 * row of out is left as it was.  The routing runs on the device (a kernel
 * on `stream` before the GEMM launches): the ids never visit the host.
 * Requires K % 32 == 0 (Q8_0) or K % 256 == 0 (K-quants), 1 <= topk <= 64,
 * 1 <= n_experts <= 2048, T*topk < 2^31 and x under 2 GiB.  Two calls on
 * one stream may share a workspace; calls that overlap in time may not. */
int mmq_moe_gemm(int fmt, const void *x_q8_1, const void *w, int n_experts, const int32_t *ids, int topk,
                 float *out, int64_t T, int64_t N, int64_t K, void *workspace, int64_t workspace_bytes,
                 void *stream);

/* The indexed-MoE GEMM on the routing tables an earlier mmq_moe_gemm left in
 * `workspace` (no ids, no routing kernel): for a second expert GEMM of the
 * same routed rows, e.g. the down projection after gate/up, whose input has
 * one row per routed row (pass T' = T*topk, topk' = 1: routed row r is then
 * input row r, grouped into the same expert tiles).  Arguments as for
 * mmq_moe_gemm.  Refused (nothing launched) unless the last mmq_moe_gemm
 * call of this process that was given this workspace on the current device
 * routed the same number of routed rows (T*topk) and n_experts; the library
 * remembers the last 1024 workspaces it routed.  As a second guard the GEMM
 * kernel uses the tables only if the header the routing kernel wrote
 * records the same sizes, so a workspace the caller overwrote after routing
 * computes nothing and leaves `out` as it was.  Tables routed for other ids
 * of the same sizes are used as they are: keeping the ids and the workspace
 * together is the caller's part. */
int mmq_moe_gemm_routed(int fmt, const void *x_q8_1, const void *w, int n_experts, int topk, float *out,
                        int64_t T, int64_t N, int64_t K, void *workspace, int64_t workspace_bytes, void *stream);

/* The indexed-MoE GEMM of mmq_moe_gemm for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same routing and GEMM kernels, with the
 * routing tables in a static device array of the library (about 592 KiB per
 * device, held until the process ends) instead of a caller workspace.
 * Arguments, layouts and results as for mmq_moe_gemm, without the workspace.
 * Refused when T*topk exceeds MMQ_MOE_NOALLOC_MAX_ROUTED.  Calls no
 * allocating routine.  Every call on a device shares that device's array,
 * which keeps the last call's tables: calls that overlap in time on one
 * device (several streams or host threads) race and must not be made;
 * calls in order on one stream are safe.  The tables are not offered to
 * mmq_moe_gemm_routed. */
#define MMQ_MOE_NOALLOC_MAX_ROUTED 131072
int mmq_moe_gemm_noalloc(int fmt, const void *x_q8_1, const void *w, int n_experts, const int32_t *ids, int topk,
                         float *out, int64_t T, int64_t N, int64_t K, void *stream);

/* Test entry: the exact int32 block dots I[m,n,b] through the same staging
 * and matrix-core code as the tiled GEMM of format `fmt` (MMQ_FMT_Q8_0,
 * MMQ_FMT_Q4_K or MMQ_FMT_Q5_K; always the tile kernel, whatever M),
 * written to dots[(m*N + n)*(K/32) + b].  MMQ_FMT_Q6_K gives one dot per
 * 16-element scale group instead, with the codes centred (code - 32):
 * dots[(m*N + n)*(K/16) + g].  Same refusal rules as the GEMM. */
int mmq_debug_block_dots(int fmt, const void *x_q8_1, const void *w, int32_t *dots,
                         int64_t M, int64_t N, int64_t K, void *stream);

/* Reason for the calling thread's last refusal ("" if none). Static storage. */
const char *mmq_last_error(void);

/* Describe the launch plan the GEMM of `fmt` would use on the current device
 * (kernel=mmq for the 128 x 128 tile kernel or kernel=mv for the M <= 8
 * matrix-vector kernel, tile, LDS bytes, grid, split-K, skip_idle_waves:
 * whether waves whose 32 rows all lie past M skip their MFMAs, and
 * mv_rows_per_wave: the matrix-vector kernel's output rows per wave, 0 for
 * the tiled kernel; wg_per_cu and vgprs: the launched kernel's resident
 * workgroups per CU and registers per lane, read from the device with
 * hipFuncGetAttributes) into buf (NUL-terminated).  Returns 1 if the plan
 * would launch, 0 if it would be refused (reason in buf). */
int mmq_plan_describe(int fmt, int64_t M, int64_t N, int64_t K, char *buf, int64_t len);

/* Pure host planning with explicit device limits and kernel attributes, so
 * that the guard can be checked without a GPU ("13 . r7-r8 raw-byte MMQ
 * kernel", sections 3.3 and 6: every capacity a launch depends on is checked
 * before it).  lds_limit_bytes: the per-workgroup LDS limit, taken as the
 * CU's LDS as well (both 160 KiB on gfx950).  kernel_vgprs: registers per
 * lane of the kernel the plan launches (<= 0: the 128 the kernels are built
 * for); kernel_scratch_bytes: its scratch bytes per lane.  On a device the
 * library reads both with hipFuncGetAttributes before planning: the
 * workgroups resident per CU (reported as wg_per_cu, and used by the split-K
 * decision) follow from them and the plan's LDS, and a kernel that needs
 * scratch (a register spill) or fits no workgroup per CU is refused.  Same
 * return convention as mmq_plan_describe. */
int mmq_plan_for_limits(int fmt, int64_t M, int64_t N, int64_t K, int64_t lds_limit_bytes,
                        int cu_count, int kernel_vgprs, int64_t kernel_scratch_bytes, char *buf, int64_t len);

/* Test hook: add `extra_bytes` to the LDS every GEMM plan requests from now
 * on (0 restores normal plans).  Used to check that an over-capacity plan is
 * refused before launch.  Process-wide; not for production use. */
void mmq_debug_set_extra_lds(int64_t extra_bytes);

/* Library version string. */
const char *mmq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MMQ_H */
