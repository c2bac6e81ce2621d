// mmq_plan.hpp -- launch planning and the capacity guard (pure host C++).
//
// "13 . r7-r8 raw-byte MMQ kernel", sections 3.3 and 6: a tile whose shared
// memory exceeds the device's cap must be refused by the launcher before
// launch, loudly, instead of failing silently and leaving the output
// unwritten.  Every refusal decision of the library lives here, in code with
// no HIP calls, so that it can be exercised without a GPU.
#pragma once

#include <cstdint>
#include <cstdio>
#include <cstring>

namespace mmq {

enum Fmt : int { FMT_Q8_0 = 0, FMT_Q4_K = 1, FMT_Q5_K = 2, FMT_Q6_K = 3 };

// Super-block formats with an affine min term (Q4_K, Q5_K); Q6_K's codes are
// centred instead and it has none.
constexpr bool has_min(int fmt) { return fmt == FMT_Q4_K || fmt == FMT_Q5_K; }

// Bytes of one weight row of K values (Q8_0: 34-byte blocks of 32; Q4_K /
// Q5_K / Q6_K: 144- / 176- / 210-byte super-blocks of 256).
constexpr int64_t weight_row_bytes(int fmt, int64_t K) {
    return fmt == FMT_Q8_0 ? (K / 32) * 34 : (K / 256) * (fmt == FMT_Q4_K ? 144 : fmt == FMT_Q5_K ? 176 : 210);
}

// Geometry of the GEMM kernel (must match the kernel's compile-time tile).
constexpr int kTileM = 128;        // output rows per workgroup
constexpr int kTileN = 128;        // output columns per workgroup
constexpr int kThreads = 512;      // eight wave64s, a 4 x 2 grid of 32 x 64 wave tiles
constexpr int kBlocksPerStage = 4; // 32-blocks staged per k-step (half a Q4_K super-block)
// Tile-packed Q8_0 weights (mmq_pack_q8_0): the same bytes as the Q8_0
// blocks, ordered as the tile kernel stages them.  For every 128-column tile
// and every k-step of kBlocksPerStage blocks, one image of kPackImg bytes:
// the 4 x 128 blocks' 32 code bytes in the kernel's LDS order (kPackCodes
// bytes: [block][column][32 bytes], the two 16-byte halves of a column
// swapped where the LDS swizzle swaps them), then their fp16 scales as
// [block][column].  Columns past N and blocks past K/32 are zero (scale 0).
constexpr int64_t kPackCodes = int64_t(kBlocksPerStage) * kTileN * 32;
constexpr int64_t kPackImg = kPackCodes + int64_t(kBlocksPerStage) * kTileN * 2;
// Bytes of the packed form of an N x K Q8_0 matrix (K a multiple of 32), or
// -1 for a shape the GEMMs refuse.
inline int64_t packed_bytes_q8_0(int64_t N, int64_t K) {
    if (N < 1 || K < 32 || K % 32 != 0 || N > INT32_MAX || K > (int64_t(1) << 23)) return -1;
    const int64_t tiles = (N + kTileN - 1) / kTileN, steps = (K / 32 + kBlocksPerStage - 1) / kBlocksPerStage;
    // a tile's images are addressed with 32-bit offsets
    if (steps * kPackImg > INT32_MAX) return -1;
    return tiles * steps * kPackImg;
}

// Workgroups resident per CU are derived from the launched kernel's own
// register and LDS use (kernel_wg_per_cu below); the kernels are built for
// two (at most 128 VGPRs, four waves per SIMD).
constexpr int kBuiltVgprs = 128;
// Split-K policy, measured on the 7B layer shapes: split only when the output
// tiles fill at most half of the resident workgroup slots, and then into
// about one workgroup per CU (more slices cost more in fp32 atomics than
// they gain), each slice keeping at least four k-steps; with fewer tiles
// than CUs, into up to two per CU when each slice keeps eight k-steps.
constexpr int kMinStepsPerSplit = 4;   // k-steps a split-K slice keeps at least
constexpr int kSplitBelow = 2;         // split when tiles * kSplitBelow <= resident slots
constexpr int kSplitSlots = 1;         // workgroups per CU a split aims for ...
constexpr int kMinStepsPerSplit2 = 8;  // ... or two per CU, for slices this long
// Without a workspace the slices add into a zeroed output with fp32 atomics,
// and only two of them: a sum of two terms onto an exact zero rounds the
// same in either order, so the result does not change from run to run.  With
// a caller workspace any number of slices store their partial tiles there and
// the last slice of a tile to finish sums them in slice order (also the same
// on every run).
constexpr int kMaxSplitAtomic = 2;
// (measured at M = 512: the down projection, 112 tiles of 148 k-steps, 143 ->
// 123 us with 4 slices instead of 3; the q+k+v set, 144 tiles of 28, 62 -> 55
// us with 3 instead of 2; o, 112 tiles of 28, slower with 4 slices of 7; 256
// tiles of 28 split in two, slower than one per CU)

// LDS bytes for the kernel's layouts: two k-step buffers, each with codes
// block-major (32 B per block per row, no padding), the activation block
// headers [row][4] as dwords, and the weight scale pairs [4][col] as two fp32
// (Q6_K: its eight 16-element group scales [8][col], one fp32 each, the same
// bytes); Q4_K and Q5_K add the split min operand [col][2][4] fp16 and come
// to exactly 80 KiB, so two workgroups share a CU's 160 KiB.
constexpr int64_t lds_bytes_for(int fmt) {
    int64_t step = int64_t(kTileM + kTileN) * 32 * kBlocksPerStage + int64_t(kTileM) * kBlocksPerStage * 4 +
                   int64_t(kBlocksPerStage) * kTileN * 8;
    if (has_min(fmt)) step += int64_t(kTileN) * 2 * kBlocksPerStage * 2;
    return 2 * step;
}

// Few activation rows (decode): a matrix-vector kernel streams each weight
// row once for all of them (mv_rows_per_wave(M) output rows per wave, four
// waves per workgroup) instead of a 128-row tile that would be almost empty.
enum Kernel : int { KERNEL_MMQ = 0, KERNEL_MV = 1, KERNEL_SM = 2 };
constexpr int kMvMaxM = 8;          // activation rows the matvec kernel takes at most
constexpr int kMvThreads = 256;
constexpr int kMvWaves = kMvThreads / 64;
// Output rows per wave: two for M >= 5, where the activation loads (one
// 72-byte block pair per unit, activation row and output row, served from
// the caches) weigh most and a wave's rows share each of them; one below.
// Measured on the 7B decode layer at M = 8: Q4_K 150 -> 119 us, Q5_K 157 ->
// 128 us, Q8_0 168 -> 159 us; four or eight rows per wave were slower than
// one (fewer resident waves), and at M = 3-4 two rows gained nothing.
constexpr int mv_rows_per_wave(int64_t M) { return M >= 5 ? 2 : 1; }
// Q4_K and Q5_K few-row shapes on the matrix core (k_mmvq: 32 weight rows
// per workgroup, one MFMA per block): its time hardly grows with M, the
// dot-product matvec's does, but it has a latency floor of ~9.5 us.
// Measured on the 7B decode shapes (Q4_K, us, dot matvec -> matrix core):
// 37888 rows x 3584 at M = 3: 33.0 -> 28.6, M = 4: 39.6 -> 28.6, M = 8:
// 55.0 -> 30.8; 4608 rows at M = 5: 9.6 -> 9.7, M = 6: 10.6 -> 9.8; 3584
// rows at M = 6: 8.6 -> 9.7, M = 8: 10.3 -> 9.6; at M = 2 it lost everywhere
// (25.9 -> 29.1 on the 37888 rows).  K is capped: four K-slices per 32
// weight rows leave a long-K launch with few rows too few waves (3584 x
// 18944 at M = 8: 27.7 -> 30.6).
constexpr int64_t kMvqMaxK = 8192;
constexpr int kMvqRows = 32;   // weight rows per k_mmvq workgroup
constexpr int kMvqSlices = 4;  // its waves, one K-slice each
constexpr int64_t kMvqLds = int64_t(kMvqSlices) * 4 * 64 * 4;   // the slices' partial sums
inline bool mv_on_mfma(int fmt, int64_t M, int64_t N, int64_t K) {
    if (fmt != FMT_Q4_K && fmt != FMT_Q5_K) return false;
    if (K > kMvqMaxK) return false;
    return M >= 8 || (M >= 3 && N >= 16384);
}

// Batch-decode sizes (kMvMaxM < M <= kSmMaxM): k_mmsm, the matrix-core
// kernel of 32 weight rows per workgroup, one int8 MFMA per block with the
// activation rows as A (16 or 32 of them staged, sm_act_rows).  Its four
// waves take a K-slice each, staging their operands into LDS of their own by
// DMA in chunks of 4 blocks (or whole super-blocks, sm_cb), two stages deep,
// and add their partial sums in wave order at the end.  A 128-row tile would leave 3 of its 4 wave rows
// idle here and give too few workgroups for the narrow GEMMs.
// Above 32 rows the kernel takes the activations in blocks of 32 rows, one
// workgroup per (32 weight rows, row block), up to kSmMaxM rows, for GEMMs
// (sets) whose 128-column tiles would be fewer than the CUs: there the tile
// kernel has too few workgroups, while on wider GEMMs it is faster (the 7B
// layer at M = 64, Q4_K, us, tile kernel -> this one: gate+up 78.0 -> 85.3;
// q+k+v 34.4 -> 18.8, o 31.1 -> 15.4, down 128.7 -> 42.8; at M = 128 gate+up
// 94.4 -> 150.7, down 123.8 -> 72.6).  The layer with the narrow GEMMs on
// this kernel: M = 160 347 -> 311 us, M = 192 352 -> 320, M = 256 351 ->
// 353 (Q4_K); Q8_0 M = 192 333 -> 306.
constexpr int kSmMaxM = 192;
constexpr int kSmRowBlock = 32;
// At decode sizes (M <= 8) the batch-decode kernel also replaces the
// matvecs on the large launches where it was measured faster (the 7B layer,
// µs, matvec -> batch decode): Q8_0 from M = 4 on the wide (N >= 16384) and
// long-K launches (gate+up at M = 4 47.8 -> 39.7, M = 8 69.7 -> 42.4; down
// at M = 8 37.7 -> 23.1; at M = 3 down lost, 22.1 -> 24.4); Q6_K gate+up from
// M = 4 (52.7 -> 46.5) and its long-K down from M = 7 (M = 6 31.0 -> 33.0,
// M = 8 36.0 -> 32.5); Q4_K and Q5_K long-K launches (where the matrix-core
// matvec does not go) from M = 6 (Q4_K down at M = 8 27.6 -> 21.6, Q5_K 30.2
// -> 27.1).  The narrow launches (q+k+v, o) stay on the matvecs, which win
// there (Q8_0 q+k+v at M = 5 13.1 against 16.1).
inline bool sm_few_rows(int fmt, int64_t M, int64_t N, int64_t K) {
    const bool wide = N >= 16384, long_k = K > kMvqMaxK;
    if (fmt == FMT_Q8_0) return M >= 4 && (wide || long_k);
    if (fmt == FMT_Q6_K) return (M >= 4 && wide) || (M >= 7 && long_k);
    return M >= 6 && long_k;
}
inline bool sm_takes(int fmt, int64_t M, int64_t N, int64_t K, int cu_count) {
    if (M <= kMvMaxM) return M >= 1 && sm_few_rows(fmt, M, N, K);
    return M <= kSmMaxM && (M <= kSmRowBlock || (N + kTileN - 1) / kTileN < cu_count);
}
constexpr int kSmRows = 32;      // weight rows per workgroup
constexpr int kSmWaves = 4;      // its waves, one K-slice each
constexpr int kSmThreads = 64 * kSmWaves;
// Two stages: three (92 KiB of LDS at Q4_K, 16 rows) or four measured
// slower on the 7B layer at M = 16 and 32 (gate+up, Q4_K at M = 16: 38.2 us
// with two, 41.9 with three, 54.6 with four): the workgroups a CU holds
// fall with the LDS, and the extra chunk in flight per wave does not make
// up for the waves lost.
constexpr int kSmStages = 2;
constexpr int sm_act_rows(int64_t M) { return M <= 16 ? 16 : 32; }
// 16-byte units of one weight row's 4-block chunk (Q8_0: 136 bytes from the
// dword below the first; K-quants: the super-block header and the chunk's
// code half; Q6_K: low bits, high bits, scales and d of the half)
constexpr int sm_w_units(int fmt) { return fmt == FMT_Q8_0 ? 9 : fmt == FMT_Q4_K ? 5 : fmt == FMT_Q5_K ? 7 : 10; }
// ... of a whole K-quant super-block (Q6_K: 210 bytes from the dword below
// the first)
constexpr int sm_w_units_sb(int fmt) { return fmt == FMT_Q4_K ? 9 : fmt == FMT_Q5_K ? 11 : 14; }
// Blocks per chunk: 4, or whole super-blocks (one contiguous 144-byte span
// per weight row, ~1.6 times the bytes per cache line the two half chunks
// touch) for Q4_K with 16 staged rows.  Measured on the 7B layer (us per
// layer, 4 -> 8 blocks): Q4_K M = 16 96.4 -> 89.9 (gate+up 38.1 -> 33.2);
// slower wherever the larger stage costs workgroups per CU: Q4_K M = 32
// 126.5 -> 146.7, Q5_K M = 16 gate+up 42.5 -> 49.0, Q6_K M = 16 122.8 ->
// 140.5.
constexpr int sm_cb(int fmt, int ar) { return fmt == FMT_Q4_K && ar == 16 ? 8 : 4; }
// one wave's stage: activation codes (32 B per row and block) and headers
// (4 B per row and block), then the 32 weight rows' units padded to whole
// 64-lane DMA instructions of 16 bytes
constexpr int64_t sm_wave_stage_bytes(int fmt, int ar) {
    return int64_t(ar) * sm_cb(fmt, ar) * 36 +
           1024 * ((32 * (sm_cb(fmt, ar) == 8 ? sm_w_units_sb(fmt) : sm_w_units(fmt)) + 63) / 64);
}
constexpr int64_t sm_lds_bytes(int fmt, int ar) { return int64_t(kSmStages) * kSmWaves * sm_wave_stage_bytes(fmt, ar); }
// Split K over two workgroups (grid z, fp32 atomics into a zeroed output)
// when the workgroups fill at most half of the resident slots, and K is
// long (at least kSmSplitLongKb blocks) or the workgroups are fewer than
// half the CUs with every wave keeping two 4-block chunks.  Measured on the
// 7B layer's K = 3584 launches (us, split -> not): q+k+v (144 workgroups)
// at M = 16 11.5 -> 10.4, at M = 32 15.2 -> 14.2; o (112) at M = 16 9.7 ->
// 10.0, at M = 32 12.4 -> 13.9; at M = 64 (224 and 288 workgroups in two
// row blocks) o 14.8 -> 14.2.
constexpr int kSmMinChunksPerWave = 2;
constexpr int kSmSplitLongKb = 256;
#ifndef MMQ_SM_MIN_MFMA
#define MMQ_SM_MIN_MFMA 1
#endif
constexpr bool kSmMinMfma = MMQ_SM_MIN_MFMA;

// gfx950 register file: 512 registers per lane per SIMD (arch and
// accumulation VGPRs together), allocated in granules of 8; at most 8 waves
// per SIMD; 4 SIMDs per CU.
constexpr int kRegsPerSimdLane = 512, kVgprGranule = 8, kMaxWavesPerSimd = 8, kSimdsPerCu = 4;

// What the capacity guard needs to know of the kernel a plan launches (read
// from the device with hipFuncGetAttributes; a pure-host caller passes it).
struct KernelFit {
    int vgprs = kBuiltVgprs;     // registers per lane
    int64_t scratch = 0;         // private (scratch) bytes per lane: register spills
};

// Workgroups of `threads` threads using `vgprs` registers per lane and
// `lds` bytes of LDS that fit one CU at once (0: none fits).
inline int kernel_wg_per_cu(int vgprs, int64_t lds, int64_t lds_per_cu, int threads) {
    const int waves = (threads + 63) / 64;
    const int per_simd = (waves + kSimdsPerCu - 1) / kSimdsPerCu;
    const int regs = ((vgprs < 1 ? 1 : vgprs) + kVgprGranule - 1) / kVgprGranule * kVgprGranule;
    int waves_per_simd = kRegsPerSimdLane / regs;
    if (waves_per_simd > kMaxWavesPerSimd) waves_per_simd = kMaxWavesPerSimd;
    int wg = waves_per_simd / per_simd;
    if (lds > 0) {
        const int64_t by_lds = lds_per_cu / lds;
        if (by_lds < wg) wg = int(by_lds);
    }
    return wg;
}

struct Plan {
    int fmt = 0;
    int kernel = KERNEL_MMQ;
    bool packed = false;   // Q8_0 weights in the tile-packed form (kPackImg images)
    int tile_m = kTileM, tile_n = kTileN, threads = kThreads, blocks_per_stage = kBlocksPerStage;
    int64_t lds_bytes = 0;
    int64_t grid_x = 0, grid_y = 0;   // x: column tiles, y: row tiles
    int64_t k_steps = 0;
    // Split K: grid z = split_k slices of steps_per_split k-steps each (the
    // last may be shorter).  split_ws: the slices' partial tiles go to the
    // caller's workspace and are summed there in slice order; otherwise
    // (split_k <= kMaxSplitAtomic) they are added into a zeroed output with
    // fp32 atomics.
    int64_t split_k = 1, steps_per_split = 0;
    bool split_ws = false;
    // Waves whose 32 rows all lie past M skip their MFMAs and epilogues.
    // Q8_0 whenever any wave row is idle; the K-quants only when at least
    // 1/kSkipShare of the launch's wave rows are idle (measured: a gain of
    // 11-17 % with 1-3 of 4 wave rows idle, a small loss with 1 of 8).  The
    // skipping instantiation runs full tiles 1-2 % slower in both formats.
    bool skip_idle_waves = false;
    // Q8_0 with K % 128 != 0: the last k-step holds fewer than
    // kBlocksPerStage blocks (a kernel variant of its own)
    bool tail = false;
    int mv_rows_per_wave = 0;   // matvec kernel: output rows per wave
    bool mv_mfma = false;       // ... on the matrix core (k_mmvq: kMvqRows weight rows per workgroup)
    int wg_per_cu = 0;          // workgroups of the launched kernel resident per CU
    int kernel_vgprs = 0;       // its registers per lane
};
constexpr int kSkipShare = 4;   // K-quants skip when idle wave rows >= 1/kSkipShare of all

inline bool fmt_ok(int fmt) { return fmt == FMT_Q8_0 || fmt == FMT_Q4_K || fmt == FMT_Q5_K || fmt == FMT_Q6_K; }
inline const char *fmt_name(int fmt) {
    return fmt == FMT_Q8_0 ? "Q8_0" : fmt == FMT_Q4_K ? "Q4_K" : fmt == FMT_Q5_K ? "Q5_K" : fmt == FMT_Q6_K ? "Q6_K" : "?";
}

// Shape checks shared by the quantize pass.  Returns nullptr when fine.
inline const char *check_quantize_shape(int64_t M, int64_t K) {
    if (M < 1 || K < 1) return "M and K must be >= 1";
    if (K % 32 != 0) return "K must be a multiple of 32 (whole q8_1 blocks)";
    if (M > (int64_t(1) << 40) / K) return "M*K too large";
    return nullptr;
}

// Build the GEMM plan or explain the refusal.  `extra_lds` is the test hook;
// `fit` describes the kernel the plan launches (registers, scratch), and
// `lds_limit` is both the per-workgroup LDS limit and the CU's LDS (the same
// 160 KiB on gfx950).  A kernel that spills to scratch is refused (the
// kernels are built to need none, so a spill means a build that misses its
// register budget), and the resident workgroups per CU that split-K plans
// with come from the kernel's own registers and LDS.
inline bool make_plan(int fmt, int64_t M, int64_t N, int64_t K, int64_t lds_limit, int cu_count,
                      int64_t extra_lds, Plan *p, char *why, size_t why_len, bool allow_mv = true,
                      const KernelFit &fit = KernelFit(), bool workspace = false) {
    auto fail = [&](const char *msg) {
        if (why && why_len) std::snprintf(why, why_len, "%s", msg);
        return false;
    };
    auto check_fit = [&](Plan &q) {
        q.kernel_vgprs = fit.vgprs;
        q.wg_per_cu = kernel_wg_per_cu(fit.vgprs, q.lds_bytes, lds_limit, q.threads);
        if (fit.scratch > 0) {
            if (why && why_len)
                std::snprintf(why, why_len, "the %s kernel uses %lld B of scratch per lane (register spills): refused",
                              q.kernel == KERNEL_MV ? "matvec" : q.kernel == KERNEL_SM ? "batch-decode" : "GEMM",
                              (long long)fit.scratch);
            return false;
        }
        if (q.wg_per_cu < 1) {
            if (why && why_len)
                std::snprintf(why, why_len, "no workgroup of the kernel fits a CU (%d VGPRs per lane, %lld B of LDS): refused",
                              fit.vgprs, (long long)q.lds_bytes);
            return false;
        }
        return true;
    };
    if (!fmt_ok(fmt)) return fail("unknown weight format");
    if (M < 1 || N < 1 || K < 1) return fail("M, N and K must be >= 1");
    // Q8_0: any whole number of 32-blocks (the last k-step of the tile kernel
    // may hold fewer than kBlocksPerStage of them); K-quants: whole 256-value
    // super-blocks
    if (fmt == FMT_Q8_0 ? K % 32 != 0 : K % 256 != 0)
        return fail(fmt != FMT_Q8_0 ? "K must be a multiple of 256 (whole K-quant super-blocks)"
                                    : "K must be a multiple of 32 (whole Q8_0 blocks)");
    if (M > INT32_MAX || N > INT32_MAX) return fail("M and N must fit in int32");
    // byte offsets inside one 128-row tile are 32-bit buffer offsets
    if (K > (int64_t(1) << 23)) return fail("K must be at most 8388608 (32-bit offsets within a tile)");
    // Every byte offset the kernels form must fit in int64 comfortably.
    if (M > (int64_t(1) << 50) / N || M > (int64_t(1) << 45) / (K / 32))
        return fail("problem too large for 64-bit offsets");
    if (cu_count < 1) return fail("device reports no compute units");
    Plan q;
    q.fmt = fmt;
    if (allow_mv && sm_takes(fmt, M, N, K, cu_count)) {
        q.kernel = KERNEL_SM;
        q.tile_m = sm_act_rows(M);
        q.tile_n = kSmRows;
        q.threads = kSmThreads;
        q.blocks_per_stage = sm_cb(fmt, q.tile_m);
        q.lds_bytes = sm_lds_bytes(fmt, q.tile_m) + extra_lds;
        q.grid_x = (N + kSmRows - 1) / kSmRows;
        if (M > kSmRowBlock)   // row blocks of 32; the groups padded to whole groups of 8
            q.grid_x = (q.grid_x + 7) / 8 * 8 * ((M + kSmRowBlock - 1) / kSmRowBlock);
        q.grid_y = 1;
        q.k_steps = (K / 32 + q.blocks_per_stage - 1) / q.blocks_per_stage;   // chunks (Q8_0: the last may be partial)
        q.steps_per_split = q.k_steps;
        if (q.grid_x > INT32_MAX) return fail("too many output rows");
        if (q.lds_bytes > lds_limit) return fail("plan needs more LDS per workgroup than the device allows: refused");
        if (!check_fit(q)) return false;
        if (2 * q.grid_x <= int64_t(q.wg_per_cu) * cu_count &&
            (K / 32 >= kSmSplitLongKb ||
             (2 * q.grid_x <= cu_count && K / 32 >= 4 * 2 * kSmWaves * kSmMinChunksPerWave))) {
            q.split_k = 2;
            q.steps_per_split = (q.k_steps + 1) / 2;
        }
        *p = q;
        return true;
    }
    if (allow_mv && M <= kMvMaxM) {
        q.kernel = KERNEL_MV;
        q.tile_m = int(M);
        q.tile_n = 1;
        q.threads = kMvThreads;
        q.blocks_per_stage = 2;
        q.mv_mfma = mv_on_mfma(fmt, M, N, K);
        q.lds_bytes = (q.mv_mfma ? kMvqLds : 0) + extra_lds;
        const int64_t rows_per_wg = q.mv_mfma ? kMvqRows : int64_t(kMvWaves) * mv_rows_per_wave(M);
        q.grid_x = (N + rows_per_wg - 1) / rows_per_wg;
        q.mv_rows_per_wave = q.mv_mfma ? 0 : mv_rows_per_wave(M);
        q.grid_y = 1;
        q.k_steps = (K / 32 + 1) / 2;   // block pairs per row (an odd last block is a unit of its own)
        q.steps_per_split = q.k_steps;
        if (q.grid_x > INT32_MAX) return fail("too many output rows");
        if (q.lds_bytes > lds_limit) return fail("plan needs more LDS per workgroup than the device allows: refused");
        if (!check_fit(q)) return false;
        *p = q;
        return true;
    }
    q.lds_bytes = lds_bytes_for(fmt) + extra_lds;
    q.grid_x = (N + kTileN - 1) / kTileN;
    q.grid_y = (M + kTileM - 1) / kTileM;
    q.k_steps = (K / 32 + kBlocksPerStage - 1) / kBlocksPerStage;   // the last one may be partial (Q8_0)
    if (q.grid_y > 65535) return fail("too many row tiles for the launch grid (M too large)");
    // Too few output tiles to occupy the device (at most half of the
    // resident workgroup slots): split K into slices of at least
    // kMinStepsPerSplit k-steps, about one workgroup per CU in all, or into
    // up to two per CU when the slices still keep kMinStepsPerSplit2.
    q.steps_per_split = q.k_steps;
    if (q.lds_bytes > lds_limit) {
        if (why && why_len)
            std::snprintf(why, why_len,
                          "plan needs %lld B of LDS per workgroup, device allows %lld B: refused",
                          (long long)q.lds_bytes, (long long)lds_limit);
        return false;
    }
    if (!check_fit(q)) return false;
    const int64_t tiles = q.grid_x * q.grid_y, slots = int64_t(q.wg_per_cu) * cu_count;
    if (tiles * kSplitBelow <= slots) {
        // about one workgroup per CU, slices of at least kMinStepsPerSplit ...
        int64_t s = (int64_t(kSplitSlots) * cu_count + tiles - 1) / tiles;
        if (s > q.k_steps / kMinStepsPerSplit) s = q.k_steps / kMinStepsPerSplit;
        // ... or, with fewer tiles than CUs, up to two per CU where the
        // slices keep kMinStepsPerSplit2
        if (tiles < cu_count) {
            int64_t s2 = (2 * int64_t(cu_count)) / tiles;
            if (s2 > q.k_steps / kMinStepsPerSplit2) s2 = q.k_steps / kMinStepsPerSplit2;
            if (s2 > s) s = s2;
        }
        if (!workspace && s > kMaxSplitAtomic) s = kMaxSplitAtomic;
        if (s > 1) {
            q.steps_per_split = (q.k_steps + s - 1) / s;
            q.split_k = (q.k_steps + q.steps_per_split - 1) / q.steps_per_split;
            q.split_ws = workspace && q.split_k > 1;
        }
    }
    {
        // the skipping kernel costs 1-2 % on full tiles (both formats): Q8_0
        // takes it whenever a wave row is idle, the K-quants from a quarter on
        const int64_t rows = q.grid_y * kTileM, idle_wave_rows = (rows - M) / 32;
        q.skip_idle_waves = fmt == FMT_Q8_0 ? idle_wave_rows > 0 : idle_wave_rows * 32 * kSkipShare >= rows;
    }
    q.tail = fmt == FMT_Q8_0 && (K / 32) % kBlocksPerStage != 0;
    if (q.grid_x > INT32_MAX) return fail("too many column tiles");
    *p = q;
    return true;
}

// Several GEMMs of one format that read the same activations (M x K), one
// launch: the column tiles of all of them form one grid row, GEMM g owning
// tiles [tile_start[g], tile_start[g+1]).  Planned as one GEMM of
// N = 128 * (total column tiles); every N[g] must itself plan.
constexpr int kMaxGemms = 8;

inline bool make_plan_multi(int fmt, int64_t M, int count, const int64_t *Ns, int64_t K, int64_t lds_limit,
                            int cu_count, int64_t extra_lds, Plan *p, int *tile_start, char *why,
                            size_t why_len, bool allow_mv = true, const KernelFit &fit = KernelFit(),
                            bool workspace = false) {
    auto fail = [&](const char *msg) {
        if (why && why_len) std::snprintf(why, why_len, "%s", msg);
        return false;
    };
    if (count < 1 || count > kMaxGemms) return fail("count must be 1..8 GEMMs");
    if (!Ns) return fail("null N array");
    // tile units: 128-column tiles for the MMQ kernel, single rows for the
    // matvec kernel, 32-row groups for the batch-decode kernel (a group never
    // holds rows of two GEMMs)
    // the batch-decode kernel's choice for the set as a whole, on the N the
    // final plan below receives (whole 32-row groups per member)
    int64_t rows32 = 0;
    for (int g = 0; g < count; g++) rows32 += (Ns[g] > 0 ? (Ns[g] + kSmRows - 1) / kSmRows : 0) * kSmRows;
    const bool sm = allow_mv && sm_takes(fmt, M, rows32, K, cu_count);
    const bool mv = allow_mv && !sm && M >= 1 && M <= kMvMaxM;
    int64_t tiles = 0;
    for (int g = 0; g < count; g++) {
        Plan one;
        if (!make_plan(fmt, M, Ns[g], K, lds_limit, cu_count, extra_lds, &one, why, why_len, allow_mv, fit))
            return false;
        tile_start[g] = int(tiles);
        tiles += mv ? Ns[g] : sm ? (Ns[g] + kSmRows - 1) / kSmRows : (Ns[g] + kTileN - 1) / kTileN;
        if (tiles > (int64_t(1) << 30)) return fail("too many output columns in the GEMM set");
    }
    tile_start[count] = int(tiles);
    return make_plan(fmt, M, mv ? tiles : tiles * (sm ? kSmRows : kTileN), K, lds_limit, cu_count, extra_lds, p, why,
                     why_len, allow_mv, fit, workspace);
}

// Split-K workspace of a plan: one 32-bit arrival counter per output tile
// (padded to kSplitCountBytesAlign), then every slice's fp32 partial tile,
// [tile][slice][128 x 128 values in the kernel's register order].
constexpr int64_t kSplitCountBytesAlign = 256;
inline int64_t split_counter_bytes(const Plan &p) {
    const int64_t tiles = p.grid_x * p.grid_y;
    return (4 * tiles + kSplitCountBytesAlign - 1) / kSplitCountBytesAlign * kSplitCountBytesAlign;
}
inline int64_t split_workspace_bytes(const Plan &p) {
    if (p.kernel != KERNEL_MMQ || !p.split_ws) return 0;
    return split_counter_bytes(p) + p.grid_x * p.grid_y * p.split_k * int64_t(kTileM) * kTileN * 4;
}

// Indexed MoE ("When Does a Kernel Win Surface?", section 4.5, the fused
// indexed-MoE prefill GEMM): routed row r = t * topk + j multiplies token t's activations
// by the weights of expert ids[r].  The routed rows are grouped by expert
// into 128-row tiles; every non-empty expert leaves at most one partial tile,
// so floor(R / 128) + min(E, R) row tiles always suffice, and that is the
// tile launch's grid y.  An expert's last partial tile of at most
// kMoeSmallRows rows is not a row tile: those rows go to the small-remainder
// launch (32 weight rows per wave over the whole of K), whose grid y is E.
// The workspace holds a header, the tile table (one int4 per row tile:
// expert, first sorted row, end of the tile's rows, unused), the remainder
// list (one int4 per expert with a small remainder, in no particular order:
// expert, first and end sorted row, unused; their count is in the header)
// and the routed-row ids sorted by expert (int32 [R]).
constexpr int kMoeMaxExperts = 2048;   // the routing kernel keeps its per-expert tables in LDS
constexpr int kMoeMaxTopk = 64;
constexpr int kMoeSmallRows = 32;      // the rows of one MFMA operand

constexpr int64_t moe_max_tiles(int64_t R, int64_t E) { return R / kTileM + (E < R ? E : R); }

// Workspace: a 32-byte header ((kMoeMagic, R, E, row tiles filled), then
// (small remainders listed, 0, 0, 0)) that the routing kernel writes last,
// so that a later launch can check that the tables it reuses were built for
// the same routed rows and experts; then the tile table; then the remainder
// list; then the sorted routed-row ids.
constexpr int kMoeMagic = 0x4d6f4532;   // "MoE2"
constexpr int64_t kMoeHeaderBytes = 32;

constexpr int64_t moe_small_table_bytes(int64_t E) { return 16 * E; }

constexpr int64_t moe_workspace_bytes(int64_t R, int64_t E) {
    if (R < 0 || E < 0) return -1;
    return kMoeHeaderBytes + 16 * moe_max_tiles(R, E) + moe_small_table_bytes(E) + ((4 * R + 15) / 16) * 16;
}

// The allocation-free MoE entry point keeps its routing tables in a static
// device array sized for this many routed rows (T * topk) and the most
// experts: about 592 KiB per device.
constexpr int64_t kNoAllocMaxRouted = 131072;
constexpr int64_t kNoAllocScratchBytes = moe_workspace_bytes(kNoAllocMaxRouted, kMoeMaxExperts);

inline bool make_plan_moe(int fmt, int64_t T, int topk, int n_experts, int64_t N, int64_t K, int64_t lds_limit,
                          int cu_count, int64_t extra_lds, Plan *p, char *why, size_t why_len,
                          const KernelFit &fit = KernelFit()) {
    auto fail = [&](const char *msg) {
        if (why && why_len) std::snprintf(why, why_len, "%s", msg);
        return false;
    };
    if (n_experts < 1 || n_experts > kMoeMaxExperts) return fail("n_experts must be 1..2048");
    if (topk < 1 || topk > kMoeMaxTopk) return fail("topk must be 1..64");
    if (T < 1) return fail("T (tokens) must be >= 1");
    if (T > INT32_MAX / topk) return fail("T * topk (routed rows) must fit in int32");
    Plan q;
    if (!make_plan(fmt, T, N, K, lds_limit, cu_count, extra_lds, &q, why, why_len, false, fit)) return false;
    // the gathered activation rows are addressed by 32-bit byte offsets
    // from the start of x
    if (T * (K / 32) * 36 > int64_t(0x7fffffff)) return fail("activations must be under 2 GiB (32-bit offsets)");
    const int64_t R = T * topk;
    q.grid_y = moe_max_tiles(R, n_experts);
    if (q.grid_y > 65535) return fail("too many row tiles for the launch grid (T * topk too large)");
    q.split_k = 1;
    q.steps_per_split = q.k_steps;
    *p = q;
    return true;
}

// `ws`: the plan of the same call given a split-K workspace (appended as
// ws_split_k, ws_steps_per_split and ws_bytes), or null.
inline void describe(const Plan &p, const Plan *ws, char *buf, size_t len) {
    int n = std::snprintf(buf, len,
                          "kernel=%s fmt=%s tile=%dx%d threads=%d blocks_per_stage=%d lds=%lld grid=%lldx%lld "
                          "k_steps=%lld split_k=%lld steps_per_split=%lld skip_idle_waves=%d mv_rows_per_wave=%d "
                          "wg_per_cu=%d vgprs=%d tail=%d split_ws=%d mv_mfma=%d packed=%d",
                          p.kernel == KERNEL_MV ? "mv" : p.kernel == KERNEL_SM ? "sm" : "mmq", fmt_name(p.fmt), p.tile_m, p.tile_n, p.threads,
                          p.blocks_per_stage, (long long)p.lds_bytes, (long long)p.grid_x, (long long)p.grid_y,
                          (long long)p.k_steps, (long long)p.split_k, (long long)p.steps_per_split,
                          int(p.skip_idle_waves), p.mv_rows_per_wave, p.wg_per_cu, p.kernel_vgprs, int(p.tail),
                          int(p.split_ws), int(p.mv_mfma), int(p.packed));
    if (ws && n > 0 && size_t(n) < len)
        std::snprintf(buf + n, len - size_t(n), " ws_split_k=%lld ws_steps_per_split=%lld ws_bytes=%lld",
                      (long long)ws->split_k, (long long)ws->steps_per_split, (long long)split_workspace_bytes(*ws));
}

}  // namespace mmq
