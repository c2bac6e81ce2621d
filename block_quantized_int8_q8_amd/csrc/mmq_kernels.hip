// mmq_kernels.hip -- gfx950 kernels of the block-quantized int8 MMQ library.
//
//   k_quantize_q8_1   fp32 -> q8_1, one pass over the activations (HBM-bound)
//   k_mmq<FMT, DOTS, MOE, SKIP, TAIL>
//                     q8_1 x {Q8_0, Q4_K, Q5_K, Q6_K} -> fp32 (or the raw int32 block
//                     dots when DOTS), int8 MFMA with the per-block scale
//                     applied in registers on the MFMA accumulator layout;
//                     MOE gathers the rows of each expert's routed tokens;
//                     SKIP lets waves with no rows left skip their compute;
//                     TAIL handles a last k-step of fewer than 4 blocks
//   k_moe_route       expert routing for the MOE launch (counts, scan, scatter)
//   k_mmv<FMT>        the same contraction for a few activation rows
//                     (decode): VALU int8 dot products at the HBM roofline
//   k_mmvq<FMT>       K-quant decode (M <= 8) on the matrix core
//   k_mmsm<FMT, AR>   batch decode (9 <= M <= 32) on the matrix core
//   k_moe_small<FMT>  the indexed MoE's small expert remainders
//
// The operation is the block-scaled contraction of "When the Product Won't
// Collapse" (section 2) and, for Q4_K, the affine identity of "When Does a
// Kernel Win Surface?" (section 6.2).  The structure follows what those pages
// establish (raw quantized bytes staged, integer products inside one block,
// the float scale applied once per block boundary in register, never through
// a shared-memory round trip) but the tiling, data layout and scale
// arithmetic are gfx950-specific and described beside each piece.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "mmq_plan.hpp"

namespace mmq {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return __half2float(__ushort_as_half((unsigned short)(bits16 & 0xffffu)));
}

// Lane exchanges inside a 16-lane row by DPP (a VALU operand modifier; no LDS
// round trip as with ds_bpermute): every lane reads the lane the pattern
// names, which is always a lane of its own row.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141; // lane i of each 8 <-> lane 7 - i
constexpr int kDppMirror = 0x140;     // lane i of each 16 <-> lane 15 - i
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

// ---------------------------------------------------------------------------
// Quantize: fp32 -> q8_1 ("13 . r7-r8 raw-byte MMQ kernel", section 3.2).
//
// Four lanes share one 32-value block, eight values (two 16-byte loads) each,
// so a wave64 reads 1 KiB of contiguous activations per load instruction
// with two of them in flight per lane, and writes 16 x 36 contiguous bytes.
// amax and the code sum are reduced across the four lanes with
// xor-shuffles; max is exact in any association order (same page, section
// 3.1) so the tree reduction cannot change d.  One block per lane group per
// launch (the grid covers every block): measured 6.0 against 7.1-7.3 us at
// 2048 x 3584 for eight lanes per block with one load each on a grid capped
// at 16 workgroups per CU, bytes identical.
// ---------------------------------------------------------------------------
constexpr int kQuantLanes = 4;                                // lanes per 32-value block
constexpr int kQuantBlocksPerWg = 256 / kQuantLanes;

__global__ __launch_bounds__(256) void k_quantize_q8_1(const float *__restrict__ x,
                                                       uint32_t *__restrict__ y, int64_t nblocks) {
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const int sub = threadIdx.x % kQuantLanes;
    const int64_t first = int64_t(blockIdx.x) * kQuantBlocksPerWg + threadIdx.x / kQuantLanes;
    const int64_t step = int64_t(gridDim.x) * kQuantBlocksPerWg;
    for (int64_t blk = first; blk < nblocks; blk += step) {
        const f32x4v *p = reinterpret_cast<const f32x4v *>(x) + blk * 8 + sub * 2;
        const f32x4v a = p[0], b = p[1];
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++) am = fmaxf(am, fabsf(v[i]));
        am = fmaxf(am, __shfl_xor(am, 1, kQuantLanes));
        am = fmaxf(am, __shfl_xor(am, 2, kQuantLanes));
        const float d = am / 127.0f;                    // correctly rounded fp32 divide
        // id = 1/d; a zero block, or one so small that 1/d overflows fp32,
        // quantizes to all-zero codes (its fp16 scale is 0 as well)
        float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        if (__builtin_isinf(id)) id = 0.0f;
        // round half away from zero (roundf), then clamp to the symmetric range
        int s = 0;
        uint32_t packed[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            uint32_t pk = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                int q = (int)roundf(v[4 * h + i] * id);
                q = min(127, max(-127, q));
                s += q;
                pk |= (uint32_t(q) & 0xffu) << (8 * i);
            }
            packed[h] = pk;
        }
        s += __shfl_xor(s, 1, kQuantLanes);
        s += __shfl_xor(s, 2, kQuantLanes);
        uint32_t *yb = y + blk * 9;                     // 36 bytes = 9 dwords per block
        yb[1 + 2 * sub] = packed[0];
        yb[2 + 2 * sub] = packed[1];
        if (sub == 0) {
            const uint32_t dh = __half_as_ushort(__float2half_rn(d));
            // s = fp16(fp32(d * sum)): keep the fp32 product a value of its own so
            // that the compiler cannot fold it into a single-rounding mixed FMA
            float ds = d * (float)s;
            asm volatile("" : "+v"(ds));
            const uint32_t sh = __half_as_ushort(__float2half_rn(ds));
            yb[0] = dh | (sh << 16);
        }
    }
}

// ---------------------------------------------------------------------------
// MMQ kernel.
//
// Workgroup: 512 threads (8 wave64s) compute a 128 x 128 output tile as a
// 4 x 2 grid of 32 x 64 wave tiles; each wave holds two 32 x 32 sub-tiles.
// Each k-step covers 4 consecutive 32-blocks (half a Q4_K super-block).
// LDS holds two k-steps: while the waves compute step ks from one buffer,
// step ks+1 is brought into the other (activations by DMA, weights through
// registers), so a step costs one barrier.  The kernel is held to 128
// VGPRs so that two workgroups -- four waves per SIMD -- share a CU: the
// per-block scale epilogue is VALU work that only other waves can overlap
// with a wave's MFMA and LDS latency.
//
// Matrix core: v_mfma_i32_32x32x32_i8 takes exactly one 32-block as its K,
// so every MFMA result is one exact block dot I (the block-boundary rule of
// "When the Product Won't Collapse", section 2).  A = activation codes (rows
// m), B = weight codes (columns n).  Lane l feeds row/column l%32 with the 16
// codes of k-half l/32; D holds column l%32 and rows
// 8*(r/4) + 4*(l/32) + r%4 in register r (the exposed accumulator map the
// same page's section 4 asks for).
//
// Scale epilogue, per block and output element, two fp32 FMAs in registers:
//   the MFMA accumulates onto srcC = 0x4B400000 (1.5 * 2^23) so that the
//   int32 result, read as a float, is exactly 1.5*2^23 + I (|I| < 2^22);
//   t   = fma(D_f, ws, -1.5*2^23*ws) = round(ws * I)      (ws = weight scale,
//         one value per lane: its column's scale; the product 1.5*2^23*ws is
//         exact, so t is the singly-rounded ws*I)
//   acc = fma(xs, t, acc)                                 (xs = activation
//         scale of the element's row)
// For Q8_0 this is the same arithmetic, in the same block order, as the
// oracle, so the output is bit-identical.
//
// Q4_K ("When Does a Kernel Win Surface?", 6.2): ws = d*sc_j (exact in fp32);
// the packed 4-bit codes are unpacked once per workgroup while staging (low
// nibbles = even sub-block, high nibbles = odd sub-block of a 32-byte
// group); and the min term  -sum_j dmin*m_j * s_j  of the step's four
// sub-blocks is added by one fp16 MFMA per 32x32 sub-tile that accumulates
// straight into the fp32 accumulator: A = the four activation block sums s_j
// (fp16, as stored), B = -dmin*m_j split exactly into an fp16 high and low
// part (k = 0..3 high parts, k = 4..7 low parts, each against the same s_j).
// ---------------------------------------------------------------------------
constexpr uint32_t kMagicBits = 0x4B400000u;   // 12582912.0f
constexpr float kMagic = 12582912.0f;
constexpr int KB = kBlocksPerStage;            // 32-blocks per k-step

// LDS layout of one k-step buffer.  Codes (activations, and weights of either
// format once unpacked to one int8 code per byte) are block-major: [block of
// the step][row][32 bytes].  A fragment read (32 consecutive rows, one
// 16-byte k-half) covers 16 bytes of every 32 in a 1 KiB span, and every
// fragment address is a per-lane base plus a compile-time offset for the
// block and sub-tile.  (Swapping the k-halves of every other group of four
// rows, which would spread an 8-lane phase over 128 contiguous bytes, was
// measured slower on gfx950.)
//
// Activation block headers (fp16 d and s) are copied as they are, [row][block]
// as one dword each; a lane widens the one activation scale it needs per block
// itself.  Weight scales are widened to fp32 at staging (v_fma_mix_f32, which
// would take the fp16 form in the FMA, issues at half the rate of v_fmac_f32
// on gfx950) and stored [block][column] as the pair (ws, -1.5*2^23*ws), so
// the epilogue's two constants arrive in one LDS read.
//
// An output register r of lane l needs the scale of row 8(r/4) + 4(l/32) +
// r%4, so a lane needs 16 different row scales per block.  Instead of
// reading them from LDS (4 KiB per wave and block) each lane reads one:
// lane l holds the scale of row 8(k/4) + k%4 + 4(l/32), k = l%16, and the
// DPP broadcast row_newbcast:r (every lane of a 16-lane row takes lane r of
// that row) hands each lane the scale of its register r inside the FMA
// itself (v_fmac_f32 with a DPP source): lanes 0-31 see rows with l/32 = 0
// and lanes 32-63 rows with l/32 = 1, as needed.
constexpr int kBlockBytes = kTileM * 32;   // one block of codes for the tile's 128 rows
constexpr int kWavesN = 2;           // wave grid: 4 along rows x 2 along columns
constexpr int kWaveN = kTileN / kWavesN;
constexpr int kNSub = kWaveN / 32;   // 32-column sub-tiles per wave
#ifndef MMQ_PREFETCH_B
#define MMQ_PREFETCH_B 1
#endif
constexpr int kPfB = MMQ_PREFETCH_B; // sub-steps of B-fragment prefetch

// Codes in LDS: block b, row r (activation row or weight column), k-half h
// (16 bytes each).  A fragment read gives lane l row l%32 and half l/32, so
// rows r and r+8 of one half would share banks (32-byte rows) and every
// 16-byte read would conflict two ways; the two halves of a row therefore
// trade places when bit 2 xor bit 3 of r is set, which makes any 8 or 16
// consecutive lanes of a read touch distinct banks.  Measured: LDS bank
// conflicts halved (Q8_0 9.2 -> 4.4 M, Q4_K 64 -> 38 M cycles per launch at
// the 7B shapes), Q4_K 1-2 % faster, Q8_0 unchanged.
__device__ __forceinline__ int half_swz(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }
__device__ __forceinline__ int code_off(int b, int row, int half) {
    return b * kBlockBytes + row * 32 + 16 * (half ^ half_swz(row));
}

// acc[R0+i] += (xsv of lane R0+i of this lane's 16-lane row) * t[R0+i], i =
// 0..7, as v_fmac_f32_dpp row_newbcast (the compiler does not fold a
// row_newbcast move into an FMA by itself).  DPP reads a VGPR at least two
// wait states after a VALU write to it: the leading s_nop covers the VALU
// instructions just before the block (the t values), and nothing inside the
// block writes a register that a later DPP instruction of the block reads.
#define MMQ_FMAC_BCAST(R, A, T) "v_fmac_f32_dpp %" #A ", %16, %" #T " row_newbcast:" #R " row_mask:0xf bank_mask:0xf\n"
template <int R0>
__device__ __forceinline__ void fmac_row_bcast8(f32x16 &acc, const f32x16 &t, float xsv) {
    float a0 = acc[R0 + 0], a1 = acc[R0 + 1], a2 = acc[R0 + 2], a3 = acc[R0 + 3];
    float a4 = acc[R0 + 4], a5 = acc[R0 + 5], a6 = acc[R0 + 6], a7 = acc[R0 + 7];
    if constexpr (R0 == 0) {
        asm volatile("s_nop 1\n"
                     MMQ_FMAC_BCAST(0, 0, 8) MMQ_FMAC_BCAST(1, 1, 9) MMQ_FMAC_BCAST(2, 2, 10)
                     MMQ_FMAC_BCAST(3, 3, 11) MMQ_FMAC_BCAST(4, 4, 12) MMQ_FMAC_BCAST(5, 5, 13)
                     MMQ_FMAC_BCAST(6, 6, 14) MMQ_FMAC_BCAST(7, 7, 15)
                     : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                     : "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]), "v"(t[4]), "v"(t[5]), "v"(t[6]),
                       "v"(t[7]), "v"(xsv));
    } else {
        asm volatile("s_nop 1\n"
                     MMQ_FMAC_BCAST(8, 0, 8) MMQ_FMAC_BCAST(9, 1, 9) MMQ_FMAC_BCAST(10, 2, 10)
                     MMQ_FMAC_BCAST(11, 3, 11) MMQ_FMAC_BCAST(12, 4, 12) MMQ_FMAC_BCAST(13, 5, 13)
                     MMQ_FMAC_BCAST(14, 6, 14) MMQ_FMAC_BCAST(15, 7, 15)
                     : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                     : "v"(t[8]), "v"(t[9]), "v"(t[10]), "v"(t[11]), "v"(t[12]), "v"(t[13]), "v"(t[14]),
                       "v"(t[15]), "v"(xsv));
    }
    acc[R0 + 0] = a0; acc[R0 + 1] = a1; acc[R0 + 2] = a2; acc[R0 + 3] = a3;
    acc[R0 + 4] = a4; acc[R0 + 5] = a5; acc[R0 + 6] = a6; acc[R0 + 7] = a7;
}
#undef MMQ_FMAC_BCAST

// One k-step buffer of the tile kernel is two LDS variables: A, the
// activation codes and headers (written by DMA), and B, the weight codes,
// scales and mins (written by the threads' stores); offsets are within each
// variable.  Q6_K keeps one variable per buffer (B after A): split, its
// kernel spilled.
template <int FMT>
struct Lds {
    static constexpr bool SPLIT = FMT != FMT_Q6_K;
    static constexpr int A_CODES = KB * kBlockBytes;
    static constexpr int A_HDR = kTileM * KB * 4;                               // [row][4] (d, s) fp16 pairs
    static constexpr int B_CODES = KB * kBlockBytes;
    // [4][col] (ws, cs) fp32 pairs; Q6_K: [8][col] ws of its 16-element groups
    static constexpr int B_SCALE = KB * kTileN * 8;
    static constexpr int B_MIN = has_min(FMT) ? kTileN * 2 * KB * 2 : 0;     // [col][g][4] fp16
    static constexpr int OFF_A_HDR = A_CODES;
    static constexpr int A_BYTES = OFF_A_HDR + A_HDR;
    static constexpr int OFF_B_CODES = SPLIT ? 0 : A_BYTES;
    static constexpr int OFF_B_SCALE = OFF_B_CODES + B_CODES;
    static constexpr int OFF_B_MIN = OFF_B_SCALE + B_SCALE;
    static constexpr int B_BYTES = OFF_B_MIN + B_MIN - OFF_B_CODES;
    static constexpr int STEP = A_BYTES + B_BYTES;     // one k-step buffer
    static constexpr int TOTAL = 2 * STEP;
};
static_assert(KB == 4 && kTileM == 128 && kTileN == 128 && kThreads == 512 && kNSub == 2 && kBlockBytes == 4096,
              "the staging maps below assume 4 blocks per k-step, a 128 x 128 tile and 512 threads");
static_assert(Lds<FMT_Q8_0>::TOTAL == lds_bytes_for(FMT_Q8_0), "plan and kernel LDS disagree");
static_assert(Lds<FMT_Q4_K>::TOTAL == lds_bytes_for(FMT_Q4_K), "plan and kernel LDS disagree");
static_assert(Lds<FMT_Q5_K>::TOTAL == lds_bytes_for(FMT_Q5_K), "plan and kernel LDS disagree");
static_assert(Lds<FMT_Q6_K>::TOTAL == lds_bytes_for(FMT_Q6_K), "plan and kernel LDS disagree");
static_assert(Lds<FMT_Q4_K>::A_BYTES % 16 == 0 && Lds<FMT_Q4_K>::OFF_B_MIN % 16 == 0 &&
              Lds<FMT_Q4_K>::B_BYTES % 16 == 0 && Lds<FMT_Q8_0>::OFF_B_SCALE % 16 == 0 &&
              Lds<FMT_Q8_0>::B_BYTES % 16 == 0 && Lds<FMT_Q6_K>::B_BYTES % 16 == 0,
              "LDS regions must stay 16-byte aligned");

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// A raw buffer over the rows of one tile: reads past `bytes` return zero in
// hardware, which is how rows beyond M or N are zero-filled (codes 0,
// scales 0: they add nothing and are never stored) without a single VALU
// instruction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t *base, int64_t bytes) {
    const int n = bytes > 0x7fffffffLL ? 0x7fffffff : int(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, n, 0x00020000);
}

// A raw buffer over weight bytes that may start 2 bytes off the dword grid
// (Q8_0 rows, or MoE experts' matrices, when K/32 is odd): the descriptor
// starts at the dword below the first byte, `shift` (0 or 2) is added to
// every offset, and the length is rounded up to whole dwords.  The range
// check is per dword, so a last dword the exact length covered only in part
// would read as zero; the <= 3 bytes added share a dword with the last byte
// of the range, so they never reach another page.
struct WBuf {
    __amdgpu_buffer_rsrc_t r;
    int shift;
};

__device__ __forceinline__ WBuf weight_rsrc(const uint8_t *base, int64_t bytes) {
    WBuf w;
    w.shift = int(reinterpret_cast<uintptr_t>(base) & 3);
    w.r = tile_rsrc(base - w.shift, bytes > 0 ? (bytes + w.shift + 3) & ~int64_t(3) : 0);
    return w;
}

// Activations go from global memory to LDS by DMA (buffer_load ... lds): a
// wave's DMA instruction writes 64 consecutive LDS slots of its size, slot i
// from lane i's address, so choosing each lane's source realises any layout
// of whole 16-byte (codes) or 4-byte (headers) units with no registers and no
// VALU work.  A wave moves two 1 KiB slices of codes (slice s = block s/4,
// rows 32(s%4)..32(s%4)+31) and one 256-byte slice of headers (rows
// 16w..16w+15) per k-step.  Each lane's offsets are fixed for the whole kernel; the k-step
// enters as the scalar offset.
typedef __attribute__((address_space(3))) void lds_void;

struct ActDma {
    int code_off[2];   // per slice: byte offset in x of this lane's 16 code bytes at k-step 0
    int hdr_off;       // byte offset of this lane's block header at k-step 0
};

__device__ __forceinline__ ActDma act_dma_offsets(int kb, int wv, int lane) {
    ActDma o;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int s = 2 * wv + i, b = s >> 2;
        // lane -> slot (b, row, stored half lane & 1) = code_off(b, row, half)
        const int row = 32 * (s & 3) + (lane >> 1), half = (lane & 1) ^ half_swz(row);
        o.code_off[i] = row * kb * 36 + b * 36 + 4 + 16 * half;
    }
    o.hdr_off = (16 * wv + (lane >> 2)) * kb * 36 + (lane & 3) * 36;
    return o;
}

// The same slots for a gathered tile (indexed MoE): tile row i is sorted
// routed row rbeg + i, whose activations are those of its token
// (routed row / topk).  Rows at or past rend belong to no routed row: they
// read token 0, which is in bounds, and are never stored.  Offsets stay
// 32-bit: the launcher refuses activations of 2 GiB or more.
__device__ __forceinline__ int gathered_row(const int32_t *__restrict__ sorted, int rbeg, int rend, int topk,
                                            int i) {
    const int p = rbeg + i;
    return p < rend ? sorted[p] / topk : 0;
}

__device__ __forceinline__ ActDma act_dma_offsets_gather(int kb, int wv, int lane, const int32_t *__restrict__ sorted,
                                                         int rbeg, int rend, int topk) {
    ActDma o;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int s = 2 * wv + i, b = s >> 2;
        const int row = 32 * (s & 3) + (lane >> 1);
        const int tok = gathered_row(sorted, rbeg, rend, topk, row);
        o.code_off[i] = tok * kb * 36 + b * 36 + 4 + 16 * ((lane & 1) ^ half_swz(row));
    }
    const int tok = gathered_row(sorted, rbeg, rend, topk, 16 * wv + (lane >> 2));
    o.hdr_off = tok * kb * 36 + (lane & 3) * 36;
    return o;
}

// VOFF: the k-step's offset goes into the lane offset instead of the scalar
// one, so that the buffer's range check covers it: kernels whose last k-step
// may hold fewer than KB blocks (the bytes past a row's last block then lie
// past the activations' end for the last row, and read as zero).
template <int FMT, bool VOFF = false>
__device__ __forceinline__ void dma_activations(__amdgpu_buffer_rsrc_t rx, const ActDma &o, int ks, uint8_t *buf,
                                                int wv, int piece) {
    // piece 0, 1: the wave's two code slices; 2: its header slice; -1: all
    using L = Lds<FMT>;
    const int koff = ks * KB * 36;
    const int soff = VOFF ? 0 : koff, voff = VOFF ? koff : 0;
#pragma unroll
    for (int i = 0; i < 2; i++)
        if (piece < 0 || piece == i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(buf + (2 * wv + i) * 1024), 16,
                                                     o.code_off[i] + voff, soff, 0, 0);
    if (piece < 0 || piece == 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(buf + L::OFF_A_HDR + wv * 256), 4, o.hdr_off + voff,
                                                 soff, 0, 0);
}

// Weights pass through registers instead (fetched one k-step ahead, stored
// at the end of a step): Q8_0 codes sit two bytes off the dword grid and Q4_K
// codes are unpacked, so neither can be copied as it is.  Each of the 512
// threads moves one unit per step.
//
// Q8_0: thread -> (column, block b of the step), b = 2*(u%2) + wave%2, so a
// lane pair covers four consecutive blocks of one column.  A 34-byte block
// starts on a 2-byte boundary: at byte 4j of the dword grid when its index
// (column * kb + block) is even, at 4j + 2 when it is odd (every row starts
// on a 4-byte boundary when kb is even, every other row when kb is odd).  The
// thread loads the 9 dwords [4j, 4j + 36) that hold it and realigns the codes
// with v_perm, whose byte selector takes the lane's own offset.  Blocks past
// the row's last one (the partial last k-step when K % 128 != 0) are staged
// with weight scale 0, so whatever codes the load returned add nothing.
struct Q80Regs {
    uint32_t first;   // dword 0 of the window: the scale, in its low or high half
    u32x4 v0, v1;     // dwords 1..8
};

__device__ __forceinline__ void q80_unit(int tid, int &col, int &b) {
    const int u = (tid >> 7) * 64 + (tid & 63);
    col = u >> 1;
    b = 2 * (u & 1) + ((tid >> 6) & 1);
}

// Byte offset of block blk of tile column col in the tile's weight buffer.
__device__ __forceinline__ int q80_off(int wshift, int kb, int col, int blk) { return wshift + (col * kb + blk) * 34; }

__device__ __forceinline__ void load_q8_0(__amdgpu_buffer_rsrc_t rw, int wshift, int kb, int ks, int tid,
                                          Q80Regs &r) {
    int col, b;
    q80_unit(tid, col, b);
    const int a = q80_off(wshift, kb, col, ks * KB + b) & ~3;   // the dword holding the block's first byte
    r.first = __builtin_amdgcn_raw_buffer_load_b32(rw, a, 0, 0);
    r.v0 = __builtin_amdgcn_raw_buffer_load_b128(rw, a + 4, 0, 0);
    r.v1 = __builtin_amdgcn_raw_buffer_load_b128(rw, a + 20, 0, 0);
}

__device__ __forceinline__ void store_q8_0(const Q80Regs &r, uint8_t *buf, int wshift, int kb, int ks, int tid) {
    using L = Lds<FMT_Q8_0>;
    uint8_t *sB = buf + L::OFF_B_CODES;
    float2 *sW = reinterpret_cast<float2 *>(buf + L::OFF_B_SCALE);
    int col, b;
    q80_unit(tid, col, b);
    const int blk = ks * KB + b;
    const bool odd = q80_off(wshift, kb, col, blk) & 2;   // block starts 2 bytes into its first dword
    // bytes 2..5 of (dword i+1 : dword i), or all of dword i+1
    const uint32_t sel = odd ? 0x07060504u : 0x05040302u;
    const uint32_t w[9] = {r.first, r.v0.x, r.v0.y, r.v0.z, r.v0.w, r.v1.x, r.v1.y, r.v1.z, r.v1.w};
    u32x4 c0, c1;
    c0.x = __builtin_amdgcn_perm(w[1], w[0], sel);
    c0.y = __builtin_amdgcn_perm(w[2], w[1], sel);
    c0.z = __builtin_amdgcn_perm(w[3], w[2], sel);
    c0.w = __builtin_amdgcn_perm(w[4], w[3], sel);
    c1.x = __builtin_amdgcn_perm(w[5], w[4], sel);
    c1.y = __builtin_amdgcn_perm(w[6], w[5], sel);
    c1.z = __builtin_amdgcn_perm(w[7], w[6], sel);
    c1.w = __builtin_amdgcn_perm(w[8], w[7], sel);
    *reinterpret_cast<u32x4 *>(sB + code_off(b, col, 0)) = c0;
    *reinterpret_cast<u32x4 *>(sB + code_off(b, col, 1)) = c1;
    const float ws = blk < kb ? h2f(odd ? r.first >> 16 : r.first) : 0.0f;
    sW[b * kTileN + col] = make_float2(ws, -kMagic * ws);   // exact: 11 x 2 bits
}

// Byte k (0..11) of the packed scale/min field held in three dwords.
template <int k>
__device__ __forceinline__ uint32_t sbyte(const u32x4 &h) {
    const uint32_t w = k < 4 ? h.y : (k < 8 ? h.z : h.w);
    return (w >> (8 * (k & 3))) & 0xffu;
}

// Sub-block J (0..7) of a Q4_K super-block: 6-bit scale and min from the 12
// packed bytes (GGUF K-quant packing).  J < 4 uses the low six bits of bytes J
// and J+4; J >= 4 takes its low four bits from byte J+4 (scale: low nibble,
// min: high nibble) and its top two bits from the spare top bits of bytes J-4
// (scale) and J (min).  Writes d*sc_J and -dmin*m_J split into fp16 high and
// low parts, for block J%4 of the step.
template <int J>
__device__ __forceinline__ void q4k_subblock(const u32x4 &h, int col, float2 *sW, _Float16 *sMin) {
    uint32_t sc, mn;
    if constexpr (J < 4) {
        sc = sbyte<J>(h) & 63u;
        mn = sbyte<J + 4>(h) & 63u;
    } else {
        sc = (sbyte<J + 4>(h) & 15u) | ((sbyte<J - 4>(h) >> 6) << 4);
        mn = (sbyte<J + 4>(h) >> 4) | ((sbyte<J>(h) >> 6) << 4);
    }
    const float d = h2f(h.x), dmin = h2f(h.x >> 16);
    constexpr int jb = J % KB;                              // block of the step
    const float ws = d * (float)sc;                         // exact: 11 x 6 bits
    sW[jb * kTileN + col] = make_float2(ws, -kMagic * ws);  // exact: 17 x 2 bits
    const float neg = -(dmin * (float)mn);                  // exact
    const _Float16 hi = (_Float16)neg;
    const _Float16 lo = (_Float16)(neg - (float)hi);        // exact remainder
    sMin[(col * 2 + 0) * KB + jb] = hi;
    sMin[(col * 2 + 1) * KB + jb] = lo;
}

// Q4_K, half `ks & 1` of super-block `ks / 2`.  Codes: thread -> (column,
// packed chunk c = 4*half + cl) by q4k_code_unit: the 16 code bytes 16c..16c+15
// belong to 32-byte group c/2 and k-half c%2; their low nibbles are codes of
// sub-block 2*(c/2), their high nibbles of sub-block 2*(c/2)+1 (the layout
// reading in the header).  They are unpacked at store time, once per
// workgroup, into the same one-code-per-byte layout as Q8_0, so the MFMA loop
// reads both formats alike.  Header: thread -> (column = 64*(wave/4) + lane,
// sub-block 4*half + wave%4), so the sub-block index is wave-uniform and a
// compile-time constant inside each case of the switch.
struct Q4KRegs {
    u32x4 v;
    u32x4 h;
};

// Q5_K: the header as for Q4_K (its scales use the same packing).  Codes:
// byte l of the high-bit plane carries the fifth bit of element l of every
// sub-block j in bit j, so a thread takes the same 8 byte positions
// l = 8*cl .. 8*cl+7 (cl = tid % 4) of both 32-byte code groups of the step
// and the 8 high-bit bytes at those positions, which serve both groups:
// 6 registers of codes and high bits where 16-byte chunks per group would
// need 8 (the kernel is at its register limit).
struct Q5KRegs {
    uint2 v0, v1;   // code bytes 8cl.. of groups 2*half and 2*half+1
    uint2 qh;       // high-bit bytes 8cl..
    u32x4 h;
};

// Q4_K codes: thread -> (column 16*wave + lane%16, chunk lane/16 of the
// half), so 16 consecutive lanes store 16 consecutive columns of one block
// and k-half, which the swizzled code rows spread over distinct banks (four
// lanes per column wrote four blocks, 4 KiB apart, into the same banks).  A
// wave instruction still reads 16 columns x 64 contiguous bytes.  Measured
// 1-2 % faster on Q4_K, output unchanged; Q5_K keeps four lanes per column,
// since its 8-byte loads lose more coalescing than its stores gain (6 %
// slower).
__device__ __forceinline__ void q4k_code_unit(int tid, int &col, int &cl) {
    col = 16 * (tid >> 6) + (tid & 15);
    cl = (tid >> 4) & 3;
}

__device__ __forceinline__ void load_q4_K(__amdgpu_buffer_rsrc_t rw, int nsb, int ks, int tid, Q4KRegs &r) {
    const int sb = ks >> 1, half = ks & 1;
    int col, cl;
    q4k_code_unit(tid, col, cl);
    const int c = 4 * half + cl;
    r.v = __builtin_amdgcn_raw_buffer_load_b128(rw, (col * nsb + sb) * 144 + 16 + 16 * c, 0, 0);
    const int hcol = (tid >> 8) * 64 + (tid & 63);
    r.h = __builtin_amdgcn_raw_buffer_load_b128(rw, (hcol * nsb + sb) * 144, 0, 0);
}

__device__ __forceinline__ void load_q5_K(__amdgpu_buffer_rsrc_t rw, int nsb, int ks, int tid, Q5KRegs &r) {
    const int sb = ks >> 1, half = ks & 1;
    const int col = tid >> 2, cl = tid & 3;
    const int base = (col * nsb + sb) * 176;
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(rw, base + 48 + 64 * half + 8 * cl, 0, 0);
    const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(rw, base + 48 + 64 * half + 32 + 8 * cl, 0, 0);
    const u32x2 q = __builtin_amdgcn_raw_buffer_load_b64(rw, base + 16 + 8 * cl, 0, 0);
    r.v0 = make_uint2(a.x, a.y);
    r.v1 = make_uint2(b.x, b.y);
    r.qh = make_uint2(q.x, q.y);
    const int hcol = (tid >> 8) * 64 + (tid & 63);
    r.h = __builtin_amdgcn_raw_buffer_load_b128(rw, (hcol * nsb + sb) * 176, 0, 0);
}

template <int FMT, typename Regs>
__device__ __forceinline__ void store_kquant(const Regs &r, uint8_t *buf, int ks, int tid) {
    using L = Lds<FMT>;
    uint8_t *sB = buf + L::OFF_B_CODES;
    float2 *sW = reinterpret_cast<float2 *>(buf + L::OFF_B_SCALE);
    _Float16 *sMin = reinterpret_cast<_Float16 *>(buf + L::OFF_B_MIN);
    if constexpr (FMT == FMT_Q5_K) {
        const int col = tid >> 2, cl = tid & 3;
        // element positions 8cl..8cl+7: k-half cl/2 of each block, bytes 8*(cl%2).. of it
        const int off = code_off(0, col, cl >> 1) + 8 * (cl & 1);
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const uint2 v = i ? r.v1 : r.v0;
            const int g = 2 * (ks & 1) + i;             // group of the super-block
            uint2 lo = make_uint2(v.x & 0x0F0F0F0Fu, v.y & 0x0F0F0F0Fu);
            uint2 hi = make_uint2((v.x >> 4) & 0x0F0F0F0Fu, (v.y >> 4) & 0x0F0F0F0Fu);
            lo.x |= ((r.qh.x >> (2 * g)) & 0x01010101u) << 4;
            lo.y |= ((r.qh.y >> (2 * g)) & 0x01010101u) << 4;
            hi.x |= ((r.qh.x >> (2 * g + 1)) & 0x01010101u) << 4;
            hi.y |= ((r.qh.y >> (2 * g + 1)) & 0x01010101u) << 4;
            // sub-blocks 2g and 2g+1 are blocks 2i and 2i+1 of this step
            *reinterpret_cast<uint2 *>(sB + off + (2 * i) * kBlockBytes) = lo;
            *reinterpret_cast<uint2 *>(sB + off + (2 * i + 1) * kBlockBytes) = hi;
        }
    } else {
        int col, cl;                                 // cl: chunk within this half
        q4k_code_unit(tid, col, cl);
        const u32x4 lo = r.v & 0x0F0F0F0Fu;
        const u32x4 hi = (r.v >> 4) & 0x0F0F0F0Fu;
        // sub-blocks 2*(c/2) and 2*(c/2)+1 are blocks 2*(cl/2) and 2*(cl/2)+1 of this step
        const int gl = cl >> 1, kh = cl & 1;
        *reinterpret_cast<u32x4 *>(sB + code_off(2 * gl, col, kh)) = lo;
        *reinterpret_cast<u32x4 *>(sB + code_off(2 * gl + 1, col, kh)) = hi;
    }
    const int hcol = (tid >> 8) * 64 + (tid & 63);
    switch ((ks & 1) * 4 + ((tid >> 6) & 3)) {   // wave-uniform
    case 0: q4k_subblock<0>(r.h, hcol, sW, sMin); break;
    case 1: q4k_subblock<1>(r.h, hcol, sW, sMin); break;
    case 2: q4k_subblock<2>(r.h, hcol, sW, sMin); break;
    case 3: q4k_subblock<3>(r.h, hcol, sW, sMin); break;
    case 4: q4k_subblock<4>(r.h, hcol, sW, sMin); break;
    case 5: q4k_subblock<5>(r.h, hcol, sW, sMin); break;
    case 6: q4k_subblock<6>(r.h, hcol, sW, sMin); break;
    default: q4k_subblock<7>(r.h, hcol, sW, sMin); break;
    }
}

// Q6_K ("When Does a Kernel Win Surface?", section 4.1: 6-bit codes centred
// at 32, one scale per 16 elements), half `ks & 1` of super-block `ks / 2`:
// 64 low-bit bytes (two rows of 32), 32 high-bit bytes, 8 scales and d.
// Thread -> (column tid/4, t = tid%4): element positions l = 8t..8t+7 of all
// four 32-element quarters q of the half, which take byte l of low-bit row
// q%2 (its nibble q/2) and bits 2q, 2q+1 of high-bit byte l; and the two
// scales of quarter t.  A 210-byte super-block starts 2 bytes off the dword
// grid when its index is odd, so each 8-byte field is loaded as the three
// dwords around it and realigned with v_perm; the codes are centred to
// signed int8 (c - 32) at store time, once per workgroup, so the MFMA takes
// them as they are and the term needs no bias.
struct Q6KRegs {
    uint32_t lo0[3], lo1[3], hi[3];   // low-bit rows 0 and 1, high bits: the dword windows
    uint32_t sc, d;                   // the dwords holding the two scales and d
};

__device__ __forceinline__ int q6k_base(int wshift, int nsb, int col, int sb) { return wshift + (col * nsb + sb) * 210; }

__device__ __forceinline__ void load_q6_K(__amdgpu_buffer_rsrc_t rw, int wshift, int nsb, int ks, int tid,
                                          Q6KRegs &r) {
    const int col = tid >> 2, t = tid & 3, half = ks & 1;
    const int o = q6k_base(wshift, nsb, col, ks >> 1);
    typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
    const u32x3 a = __builtin_amdgcn_raw_buffer_load_b96(rw, (o + 64 * half + 8 * t) & ~3, 0, 0);
    const u32x3 b = __builtin_amdgcn_raw_buffer_load_b96(rw, (o + 64 * half + 32 + 8 * t) & ~3, 0, 0);
    const u32x3 c = __builtin_amdgcn_raw_buffer_load_b96(rw, (o + 128 + 32 * half + 8 * t) & ~3, 0, 0);
    r.lo0[0] = a.x; r.lo0[1] = a.y; r.lo0[2] = a.z;
    r.lo1[0] = b.x; r.lo1[1] = b.y; r.lo1[2] = b.z;
    r.hi[0] = c.x; r.hi[1] = c.y; r.hi[2] = c.z;
    r.sc = __builtin_amdgcn_raw_buffer_load_b32(rw, (o + 192 + 8 * half + 2 * t) & ~3, 0, 0);
    r.d = __builtin_amdgcn_raw_buffer_load_b32(rw, (o + 208) & ~3, 0, 0);
}

// 8 bytes starting `sh` (0 or 2) bytes into the 3-dword window w.
__device__ __forceinline__ uint2 q6k_field(const uint32_t *w, int sh) {
    const uint32_t sel = sh ? 0x05040302u : 0x03020100u;
    return make_uint2(__builtin_amdgcn_perm(w[1], w[0], sel), __builtin_amdgcn_perm(w[2], w[1], sel));
}

// c - 32 in every byte of c (6-bit codes 0..63): set bit 7 so that the
// subtraction cannot borrow across bytes, subtract, then flip bit 7 back.
__device__ __forceinline__ uint32_t q6k_centre(uint32_t c) { return ((c | 0x80808080u) - 0x20202020u) ^ 0x80808080u; }

__device__ __forceinline__ void store_q6_K(const Q6KRegs &r, uint8_t *buf, int wshift, int nsb, int ks, int tid) {
    using L = Lds<FMT_Q6_K>;
    uint8_t *sB = buf + L::OFF_B_CODES;
    float *sW = reinterpret_cast<float *>(buf + L::OFF_B_SCALE);
    const int col = tid >> 2, t = tid & 3, half = ks & 1;
    const int o = q6k_base(wshift, nsb, col, ks >> 1);
    const int sh = o & 2;   // every 8-byte field sits at o + a multiple of 4
    const uint2 l0 = q6k_field(r.lo0, sh), l1 = q6k_field(r.lo1, sh), hb = q6k_field(r.hi, sh);
    // positions 8t..8t+7: k-half t/2 of each block, bytes 8*(t%2).. of it
    const int off = code_off(0, col, t >> 1) + 8 * (t & 1);
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const uint2 lb = (q & 1) ? l1 : l0;
        const int ns = 4 * (q >> 1);
        uint2 c;
        c.x = ((lb.x >> ns) & 0x0F0F0F0Fu) | (((hb.x >> (2 * q)) & 0x03030303u) << 4);
        c.y = ((lb.y >> ns) & 0x0F0F0F0Fu) | (((hb.y >> (2 * q)) & 0x03030303u) << 4);
        *reinterpret_cast<uint2 *>(sB + off + q * kBlockBytes) = make_uint2(q6k_centre(c.x), q6k_centre(c.y));
    }
    // scales 2t, 2t+1 of the half: the groups of block t
    const uint32_t sv = r.sc >> (8 * ((o + 192 + 8 * half + 2 * t) & 2));
    const float d = h2f(r.d >> (8 * ((o + 208) & 2)));
    sW[(2 * t) * kTileN + col] = d * (float)(int8_t)(sv & 0xffu);             // exact: 11 x 8 bits
    sW[(2 * t + 1) * kTileN + col] = d * (float)(int8_t)((sv >> 8) & 0xffu);
}

template <int FMT>
struct WRegs;
template <>
struct WRegs<FMT_Q8_0> { Q80Regs r; };
template <>
struct WRegs<FMT_Q4_K> { Q4KRegs r; };
template <>
struct WRegs<FMT_Q5_K> { Q5KRegs r; };
template <>
struct WRegs<FMT_Q6_K> { Q6KRegs r; };

// One int8 MFMA at this point of the program.  The empty asm statements
// redefine the operands just before it and its result just after it, so the
// MFMA can move neither above nor below its neighbours in the software
// pipeline (left free, the compiler may hoist all of a k-step's MFMAs ahead
// of their epilogues and run out of registers).
__device__ __forceinline__ i32x16 mfma_at(i32x4 &a, i32x4 &b, const i32x16 &c) {
    asm volatile("" : "+v"(a), "+v"(b));
    i32x16 d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
    asm volatile("" : "+v"(d));
    return d;
}

// Q6_K: one 16-element scale group, K = 16 (v_mfma_i32_32x32x16_i8: lane l
// feeds row/column l%32 with the 8 codes 8*(l/32).. of the group).
__device__ __forceinline__ i32x16 mfma16_at(long &a, long &b, const i32x16 &c) {
    asm volatile("" : "+v"(a), "+v"(b));
    i32x16 d = __builtin_amdgcn_mfma_i32_32x32x16_i8(a, b, c, 0, 0, 0);
    asm volatile("" : "+v"(d));
    return d;
}

// acc[r] += xs(row of register r) * round(ws * I[r]) for the 16 registers:
// all sixteen t first (compiler-visible, so the MFMA-to-VALU wait states are
// the compiler's), then the row-broadcast FMAs.
__device__ __forceinline__ void scale_epilogue(f32x16 &acc, const i32x16 &D, float ws, float cs, float xsv) {
    f32x16 t;
#pragma unroll
    for (int r = 0; r < 16; r++) t[r] = __builtin_fmaf(__int_as_float(D[r]), ws, cs);
    fmac_row_bcast8<0>(acc, t, xsv);
    fmac_row_bcast8<8>(acc, t, xsv);
}

// Output tile of this workgroup.  Workgroups reach the eight XCDs (each with
// its own L2) round-robin by linear id, so neighbouring ids share no L2.
// XCD k is therefore given a contiguous run of the tile sequence (k-th
// eighth, linear id = 8q + k -> run position q), and the sequence walks
// groups of kGroupRows row tiles column by column: an XCD's run is a compact
// rectangle of tiles (4 x 14 at 2048 x 3584) whose A rows and B columns its
// L2 serves to all of them.  Measured: Q4_K 2-3 % faster with it; Q8_0 at
// 2048 x 3584 x 3584 1.4 % faster, with 29 % fewer bytes fetched past L2.
// The indexed-MoE launch takes the same order over the row tiles its routing
// filled (tile_in_rows).
constexpr int kXcds = 8, kGroupRows = 4;
// The same order over the first `gy` row tiles of the grid (the indexed MoE:
// the row tiles its routing filled; the table's spare entries follow them).
// Returns false for a workgroup past them, which has nothing to do: their
// linear ids are the grid's last, so the real tiles still spread evenly over
// the XCDs.
__device__ __forceinline__ bool tile_in_rows(int gy, int &tx, int &ty) {
    const int gx = gridDim.x, T = gx * gy;
    const int L = blockIdx.y * gx + blockIdx.x;
    if (L >= T) return false;
    const int k = L % kXcds, q = L / kXcds;
    const int base = T / kXcds, rem = T % kXcds;
    const int n = k * base + min(k, rem) + q;          // bijective on [0, T)
    const int group = n / (kGroupRows * gx);
    const int rows = min(kGroupRows, gy - group * kGroupRows);
    const int idx = n - group * kGroupRows * gx;
    ty = group * kGroupRows + idx % rows;
    tx = idx / rows;
    return true;
}

template <bool REMAP>
__device__ __forceinline__ void tile_of_workgroup(int &tx, int &ty) {
    if constexpr (!REMAP) {
        tx = blockIdx.x;
        ty = blockIdx.y;
        return;
    }
    const int gx = gridDim.x, gy = gridDim.y, T = gx * gy;
    const int L = blockIdx.y * gx + blockIdx.x;
    const int k = L % kXcds, q = L / kXcds;
    const int base = T / kXcds, rem = T % kXcds;
    const int n = k * base + min(k, rem) + q;          // bijective on [0, T)
    const int group = n / (kGroupRows * gx);
    const int rows = min(kGroupRows, gy - group * kGroupRows);
    const int idx = n - group * kGroupRows * gx;
    ty = group * kGroupRows + idx % rows;
    tx = idx / rows;
}

template <int P>
struct Parity {
    static constexpr int value = P;
};

// The GEMMs of one launch (a single GEMM is a set of one): they share the
// activations and K; GEMM g owns column tiles [tile_start[g], tile_start[g+1])
// of the grid's x dimension.  Passed by value in the kernel arguments.
struct GemmSet {
    int count;
    int tile_start[kMaxGemms + 1];
    int N[kMaxGemms];
    const uint8_t *w[kMaxGemms];
    void *out[kMaxGemms];
    // split K through a workspace (null otherwise): the slices' partial
    // tiles, [tile][slice][8][512 threads] float4, and one arrival counter
    // per tile, zeroed before the launch
    float *part;
    uint32_t *cnt;
};

// The GEMM of the set that holds grid unit t (column tile, 32-row group or
// row), and the units of the whole set.  The launcher pads tile_start past
// the set's count with the set's total, so both read fixed entries: one
// scalar load brings them all, where a loop up to the count (or an index by
// it) waits for each load in turn before the kernel's first memory access.
// A unit past the total maps to the last GEMM of the set.
__device__ __forceinline__ int set_member(const GemmSet &set, int t) {
    int g = 0;
#pragma unroll
    for (int i = 1; i < kMaxGemms; i++)
        if (t >= set.tile_start[i]) g = i;
    return min(g, set.count - 1);
}
__device__ __forceinline__ int set_total(const GemmSet &set) { return set.tile_start[kMaxGemms]; }

// Indexed MoE: the row tiles come from the routing kernel's table instead of
// from blockIdx.y alone (row tile y = tiles[y]: expert, first sorted row, end
// of the expert's sorted rows; expert -1 marks a spare tile), the activation
// rows are gathered through the sorted routed-row ids, the weights are those
// of the tile's expert (expert_bytes apart) and output row i of the tile is
// routed row sorted[first + i].
struct MoeArgs {
    const int4 *header;   // (kMoeMagic, R, E, row tiles filled) when the tables below are this launch's
    const int4 *tiles;
    const int4 *small;    // small remainders (expert, first and end sorted row), header[1].x of them
    const int32_t *sorted;
    int topk;
    int R, E;
    int64_t expert_bytes;
};

// SKIP: waves whose 32 rows all lie past the tile's last row skip their
// MFMAs and epilogues (see wave_live below).  The MoE launch always skips.
// On full tiles the branch costs 1-2 % (measured on both formats), so the
// launcher uses the skipping instantiation only when the plan marks waves
// as idle (Q8_0: any; K-quants: at least a quarter of the wave rows).
// TAIL: the last k-step may hold fewer than KB blocks (Q8_0 with
// K % 128 != 0); without it the per-block check of that case (2 % of the
// step) is compiled out.
// Q8_0 runs each k-step's last epilogue after the step's barrier (DEFER
// below): the next step's first fragment reads are issued first, so their
// LDS latency is spent on that epilogue instead of stalling the step's
// first MFMA, and the last MFMA's latency is spent at the barrier.
// PK: Q8_0 weights in the tile-packed form (kPackImg images, mmq_pack_q8_0).
// Their codes are already in the LDS order, so they go to LDS by DMA like
// the activations (no registers, no VALU); each thread fetches one fp16
// scale a k-step ahead and stores its fp32 pair, the same values as the
// unpacked staging, so the output is bit-identical to it.
template <int FMT, bool DOTS, bool MOE, bool SKIP, bool TAIL, bool PK = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(DOTS ? 2 : 4)))
void k_mmq(const uint8_t *__restrict__ xq, const GemmSet set, int M, int K, int steps_per_split, const MoeArgs moe) {
    static_assert(!PK || (FMT == FMT_Q8_0 && !DOTS && !MOE), "the packed form is a Q8_0 GEMM layout");
    static_assert(!(MOE && DOTS), "the block-dot output exists for plain GEMMs only");
    static_assert(!(DOTS && SKIP) && (!MOE || SKIP), "block dots never skip; the MoE launch always does");
    static_assert(!TAIL || FMT == FMT_Q8_0, "only Q8_0 k-steps can be partial");
    constexpr bool DEFER = FMT == FMT_Q8_0 && !DOTS;
    using L = Lds<FMT>;
    // The two k-step buffers are LDS variables of their own, each in two
    // (A: activations, B: weights), not offsets into one array: the compiler
    // then knows that the DMA into one buffer cannot write what the fragment
    // reads of the other return (it would make every LDS read wait for the
    // DMA in flight), and that the weight stores into B cannot write what the
    // activation DMA into A writes (it orders an LDS store after an LDS DMA
    // it may alias: with one variable per buffer the weight stores waited for
    // every DMA piece of the step).  The step loop is unrolled by two so that
    // each copy names its buffers at compile time.  PK: the weight scale
    // pairs are variables of their own as well, apart from the codes' DMA.
    static_assert(FMT != FMT_Q8_0 || L::OFF_B_SCALE + L::B_SCALE == L::B_BYTES, "Q8_0 scale pairs end B");
    constexpr bool kSplitAB = L::SPLIT;
    constexpr int kBBytes = PK ? L::OFF_B_SCALE : L::B_BYTES;
    __shared__ __attribute__((aligned(16))) uint8_t lds0[kSplitAB ? L::A_BYTES : L::STEP];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[kSplitAB ? L::A_BYTES : L::STEP];
    __shared__ __attribute__((aligned(16))) float2 pks0[PK ? KB * kTileN : 1];
    __shared__ __attribute__((aligned(16))) float2 pks1[PK ? KB * kTileN : 1];
    __shared__ __attribute__((aligned(16))) uint8_t ldsb0_[kSplitAB ? kBBytes : 1];
    __shared__ __attribute__((aligned(16))) uint8_t ldsb1_[kSplitAB ? kBBytes : 1];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wr = wv >> 1, wc = wv & 1;          // wave tile: rows 32*wr.., columns 64*wc..
    const int g = lane >> 5, l32 = lane & 31;
    int tx = 0, ty = 0;
    int4 mh = {0, 0, 0, 0};
    if constexpr (MOE) {
        // tables built for other routed rows or experts (or never built):
        // nothing is computed and nothing written
        mh = *moe.header;
        if (mh.x != kMoeMagic || mh.y != moe.R || mh.z != moe.E) return;
        // XCD-aware order over the row tiles the routing filled (their count
        // is the header's last field): an XCD's workgroups share the gathered
        // activation rows of a group of row tiles and the experts' weight
        // columns in its L2
        if (!tile_in_rows(min(mh.w, int(gridDim.y)), tx, ty)) return;
    } else {
        tile_of_workgroup<true>(tx, ty);
    }
    // which GEMM of the set this column tile belongs to (workgroup-uniform)
    // (a loop, not set_member: the workgroup runs long enough that its
    // load latency does not matter, and the eight boundaries set_member
    // holds in scalar registers made the Q6_K kernel spill)
    int gi = 0;
    for (int i = 1; i < set.count; i++)
        if (tx >= set.tile_start[i]) gi = i;
    const uint8_t *__restrict__ wq = set.w[gi];
    void *__restrict__ outp = set.out[gi];
    const int N = set.N[gi];
    int4 mt = {0, 0, 0, 0};   // MoE row tile: expert, first sorted row, end of the expert's rows
    if constexpr (MOE) {
        mt = moe.tiles[ty];
        if (mt.x < 0) return;   // a spare row tile (workgroup-uniform)
        wq += int64_t(mt.x) * moe.expert_bytes;
    }
    const int n0 = (tx - set.tile_start[gi]) * kTileN, m0 = MOE ? 0 : ty * kTileM;
    // K-quants: whole super-blocks, so whole k-steps; Q8_0: the last k-step
    // may hold fewer than KB blocks (see nvalid below)
    const int kb = K >> 5, nsteps = (kb + KB - 1) / KB;
    // this workgroup's k-steps: [ks0, ks0 + nloc) (all of them unless K is split)
    const int ks0 = blockIdx.z * steps_per_split;
    const int nloc = min(steps_per_split, nsteps - ks0);

    // Buffers over this tile's rows of x and w (reads past M / N return 0).
    const int64_t xrow = int64_t(kb) * 36;
    const int64_t wrow = weight_row_bytes(FMT, K);
    const __amdgpu_buffer_rsrc_t rx = tile_rsrc(xq + int64_t(m0) * xrow, int64_t(M - m0) * xrow);
    const WBuf rwb = weight_rsrc(wq + int64_t(n0) * wrow, int64_t(N - n0) * wrow);
    const __amdgpu_buffer_rsrc_t rw = rwb.r;
    // PK: this column tile's images, one per k-step
    const __amdgpu_buffer_rsrc_t rpk =
        PK ? tile_rsrc(wq + int64_t(n0 / kTileN) * nsteps * kPackImg, int64_t(nsteps) * kPackImg) : rw;

    const int b_col0 = kWaveN * wc + l32;            // this lane's B column in sub-tile 0
    const int a_lane = code_off(0, 32 * wr + l32, g); // fragment bases; blocks and sub-tiles
    const int b_lane = code_off(0, b_col0, g);        // are compile-time offsets from here
    // Q6_K: 8-byte fragments of each 16-element group h (k-half h), lane
    // group g taking its bytes 8g..8g+7; the two halves of a 32-byte row
    // differ in bit 4 of the offset only
    const int a6 = code_off(0, 32 * wr + l32, 0) + 8 * g;
    const int b6 = code_off(0, b_col0, 0) + 8 * g;
    // the activation row whose scale this lane holds for the row broadcasts
    const int xs_row = 32 * wr + 8 * ((lane & 15) >> 2) + (lane & 3) + 4 * g;
    const ActDma adma = MOE ? act_dma_offsets_gather(kb, wv, lane, moe.sorted, mt.y, mt.z, moe.topk)
                            : act_dma_offsets(kb, wv, lane);

    i32x16 srcC;
#pragma unroll
    for (int r = 0; r < 16; r++) srcC[r] = DOTS ? 0 : int(kMagicBits);
    // an opaque value: kept in registers instead of being rebuilt from
    // scalar registers before every MFMA
    asm volatile("" : "+v"(srcC));

    f32x16 acc[kNSub];
#pragma unroll
    for (int c = 0; c < kNSub; c++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[c][r] = 0.0f;
    // DEFER: the last MFMA of the previous k-step and the scales of its
    // epilogue (sub-tile kNSub-1 of block KB-1)
    i32x16 pendD;
    float2 pendW = make_float2(0.0f, 0.0f);
    float pendX = 0.0f;
    bool pending = false;   // wave-uniform
    auto run_pending = [&]() {
        if constexpr (DEFER) {
            if (pending) {
                scale_epilogue(acc[kNSub - 1], pendD, pendW.x, pendW.y, pendX);
                asm volatile("" : "+v"(acc[kNSub - 1]));
                pending = false;
            }
        }
    };

    WRegs<FMT> wr_;
    // PK: the fp16 scale of (block tid / 128, column tid % 128) of a k-step,
    // kept as the loaded 16-bit value (widened where it is used, so the load
    // is not waited for when it is issued)
    unsigned short pk_d = 0;
    auto load_w = [&](int k) {
        if constexpr (PK)
            pk_d = __builtin_amdgcn_raw_buffer_load_b16(rpk, k * int(kPackImg) + int(kPackCodes) + 2 * tid, 0, 0);
        else if constexpr (FMT == FMT_Q8_0)
            load_q8_0(rw, rwb.shift, kb, k, tid, wr_.r);
        else if constexpr (FMT == FMT_Q6_K)
            load_q6_K(rw, rwb.shift, K >> 8, k, tid, wr_.r);
        else if constexpr (FMT == FMT_Q4_K)
            load_q4_K(rw, K >> 8, k, tid, wr_.r);
        else
            load_q5_K(rw, K >> 8, k, tid, wr_.r);
    };
    // PK: the 16 KiB of codes, two 1 KiB DMA pieces per wave, and the
    // thread's scale pair (from the fp16 scale load_w fetched)
    auto pk_codes = [&](int k, uint8_t *buf) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int c = wv + 8 * i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rpk, (lds_void *)(buf + L::OFF_B_CODES + 1024 * c), 16,
                                                     k * int(kPackImg) + 1024 * c + 16 * lane, 0, 0, 0);
        }
    };
    auto pk_scale = [&](uint8_t *buf) {
        const float ws = __half2float(__ushort_as_half(pk_d));
        (buf == ldsb0_ ? pks0 : pks1)[tid] = make_float2(ws, -kMagic * ws);   // exact
    };
    auto store_w = [&](int k, uint8_t *buf) {
        if constexpr (PK) {
            pk_codes(k, buf);
            pk_scale(buf);
        } else if constexpr (FMT == FMT_Q8_0)
            store_q8_0(wr_.r, buf, rwb.shift, kb, k, tid);
        else if constexpr (FMT == FMT_Q6_K)
            store_q6_K(wr_.r, buf, rwb.shift, K >> 8, k, tid);
        else
            store_kquant<FMT>(wr_.r, buf, k, tid);
    };

    // Pipeline: step ks computes from buffer ks%2 (lds0/ldsb0 or lds1/ldsb1).  Meanwhile the DMA fills
    // the other buffer with step ks+1's activations, and the weight
    // registers, fetched one step earlier, are stored into it; after the
    // barrier they fetch step ks+2.
    // Buffer (ks+1)%2 was last read by step ks-1, which every wave finished
    // before the previous barrier.
    dma_activations<FMT, TAIL || DOTS>(rx, adma, ks0, lds0, wv, -1);
    load_w(ks0);
    if constexpr (kSplitAB)
        store_w(ks0, ldsb0_);
    else
        store_w(ks0, lds0);   // B offsets count from the buffer's start
    if (nloc > 1) load_w(ks0 + 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the DMA has landed in LDS
    __syncthreads();

    // A wave whose 32 rows lie past the tile's last row (rows at or past M in
    // the last row tile of a GEMM; past its expert's last routed row in a MoE
    // tile) has nothing to compute: it only takes its part in staging, which
    // leaves the SIMD's VALU to the other waves.
    bool wave_live = true;
    if constexpr (MOE)
        wave_live = __builtin_amdgcn_readfirstlane(int(mt.y + 32 * wr < mt.z)) != 0;
    else if constexpr (SKIP)
        wave_live = __builtin_amdgcn_readfirstlane(int(m0 + 32 * wr < M)) != 0;

    auto step = [&](auto parity, int j) {
        constexpr int P = decltype(parity)::value;
        const int ks = ks0 + j;                   // the k-step; j is its place in this workgroup's range
        uint8_t *const buf = P ? lds1 : lds0;     // local step j (j % 2 == P): activations
        uint8_t *const nxt = P ? lds0 : lds1;     // local step j + 1
        // the same steps' weights (B offsets count from here)
        uint8_t *const bufb = [&]() -> uint8_t * {
            if constexpr (kSplitAB) return P ? ldsb1_ : ldsb0_;
            else return buf;
        }();
        uint8_t *const nxtb = [&]() -> uint8_t * {
            if constexpr (kSplitAB) return P ? ldsb0_ : ldsb1_;
            else return nxt;
        }();
        // Q8_0: an idle wave takes this path of its own (staging only).  The
        // K-quants skip the same work by guarding the fragment reads, MFMAs
        // and epilogues below instead: with a second copy of the staging code
        // their register allocation spilled inside the k-loop.
        if constexpr (SKIP && FMT == FMT_Q8_0) {
            if (!wave_live) {
                if (j + 1 < nloc) {
#pragma unroll
                    for (int piece = 0; piece < 3; piece++)
                        dma_activations<FMT, TAIL || DOTS>(rx, adma, ks + 1, nxt, wv, piece);
                    store_w(ks + 1, nxtb);
                }
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                if (j + 2 < nloc) load_w(ks + 2);
                return;
            }
        }
        const unsigned short *sHdr = reinterpret_cast<const unsigned short *>(buf + L::OFF_A_HDR);
        const uint8_t *sB = bufb + L::OFF_B_CODES;
        const float2 *sW = PK ? (P ? pks1 : pks0) : reinterpret_cast<const float2 *>(bufb + L::OFF_B_SCALE);

        // Sub-step st = (block b = st/2, sub-tile c = st%2).  B fragments are
        // read from LDS kPfB sub-steps ahead, A fragments one block ahead.
        constexpr int kSteps = KB * kNSub;
        constexpr int kRing = kPfB + 1;
        i32x4 fa[2];
        float xsv[2];
        i32x4 fb[kRing];
        // Q8_0 reads the (ws, cs) pair; Q4_K, short of registers, reads ws
        // alone and forms cs with one multiply (exact); Q6_K reads the ws of
        // each 16-element group just before its MFMA
        using WsT = typename std::conditional<FMT == FMT_Q8_0, float2, float>::type;
        WsT fw[kRing];
        // Blocks of this step that exist (Q8_0 with K % 128 != 0: the last
        // step has 1-3).  A block past the row's end holds whatever the loads
        // returned; its weight scale was staged as 0, so t = 0, and its
        // activation scale is taken as 0 here, so the epilogue adds
        // fma(0, 0, acc) = acc whatever those bytes were.
        const int nvalid = kb - ks * KB;   // wave-uniform, >= KB except in that last step
        auto load_a = [&](int b) {
            if constexpr (FMT == FMT_Q6_K) {
                const uint2 f0 = *reinterpret_cast<const uint2 *>(buf + a6 + b * kBlockBytes);
                const uint2 f1 = *reinterpret_cast<const uint2 *>(buf + (a6 ^ 16) + b * kBlockBytes);
                fa[b & 1] = i32x4{int(f0.x), int(f0.y), int(f1.x), int(f1.y)};
            } else {
                fa[b & 1] = *reinterpret_cast<const i32x4 *>(buf + a_lane + b * kBlockBytes);
            }
            if constexpr (!DOTS) {
                const float xs = h2f(sHdr[(xs_row * KB + b) * 2]);
                if constexpr (TAIL)
                    xsv[b & 1] = (b == 0 || b < nvalid) ? xs : 0.0f;
                else
                    xsv[b & 1] = xs;
            }
        };
        auto load_b = [&](int st) {
            const int b = st / kNSub, c = st % kNSub;
            if constexpr (FMT == FMT_Q6_K) {
                const uint2 f0 = *reinterpret_cast<const uint2 *>(sB + b6 + b * kBlockBytes + c * 32 * 32);
                const uint2 f1 = *reinterpret_cast<const uint2 *>(sB + (b6 ^ 16) + b * kBlockBytes + c * 32 * 32);
                fb[st % kRing] = i32x4{int(f0.x), int(f0.y), int(f1.x), int(f1.y)};
            } else {
                fb[st % kRing] = *reinterpret_cast<const i32x4 *>(sB + b_lane + b * kBlockBytes + c * 32 * 32);
            }
            if constexpr (!DOTS) {
                if constexpr (FMT == FMT_Q8_0) {
                    fw[st % kRing] = sW[b * kTileN + b_col0 + 32 * c];
                } else if constexpr (FMT == FMT_Q6_K) {
                    // read where it is used (registers)
                } else {
                    fw[st % kRing] = sW[b * kTileN + b_col0 + 32 * c].x;
                }
            }
        };
        const bool live = !SKIP || FMT == FMT_Q8_0 || wave_live;   // wave-uniform
        if (live) {
            load_a(0);
#pragma unroll
            for (int st = 0; st < kPfB; st++) load_b(st);
        }
        // the previous step's last epilogue, while those reads are in flight
        run_pending();
#pragma unroll
        for (int st = 0; st < kSteps; st++) {
            const int b = st / kNSub, c = st % kNSub;
            if (live) {
                if (st + kPfB < kSteps) load_b(st + kPfB);
                if (c == 0 && b + 1 < KB) load_a(b + 1);
            }
            // The LDS writes for step ks+1 are spread over the sub-steps (the
            // three DMA pieces at 1, 3 and 5, the weight stores at 6): issued
            // together at the top or bottom of the step they were measured to
            // cost 8-10 % more.
            // The DMA pieces are issued on every step, the last one included
            // (it copies its own k-step again into the buffer no one reads
            // any more): issued on some paths only, they leave the compiler
            // unable to count them, and the weight registers' wait at the
            // stores then drains every load in flight (Q8_0 2048 x 3584 x
            // 18944: 429 -> 398 us).  Q6_K keeps the guarded form (unguarded,
            // its kernel spilled), and so does PK, which has no weight
            // registers to wait for (1.7 % slower unguarded).
            // PK: the codes' DMA at sub-step 2 (measured 10 % faster than at
            // 6 and 7 % faster than at 3); the scale pairs are stored after
            // the step, below.
            if constexpr (FMT == FMT_Q6_K || PK) {
                if (j + 1 < nloc) {
                    if ((st & 1) && st < 6) dma_activations<FMT, TAIL || DOTS>(rx, adma, ks + 1, nxt, wv, st >> 1);
                    if constexpr (PK) {
                        if (st == 2) pk_codes(ks + 1, nxtb);
                    } else {
                        if (st == 6) store_w(ks + 1, nxtb);
                    }
                }
            } else {
                const int kn = j + 1 < nloc ? ks + 1 : ks;   // the k-step the DMA stages into the other buffer
                if ((st & 1) && st < 6) dma_activations<FMT, TAIL || DOTS>(rx, adma, kn, nxt, wv, st >> 1);
                if (st == 6 && j + 1 < nloc) store_w(ks + 1, nxtb);
            }
            if (!live) continue;
            const int col = b_col0 + 32 * c;
            if constexpr (FMT == FMT_Q6_K) {
                // the block's two 16-element groups, each with its own scale
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    float ws = 0.0f;
                    if constexpr (!DOTS) ws = reinterpret_cast<const float *>(sW)[(2 * b + h) * kTileN + col];
                    long fa6 = __builtin_bit_cast(long, make_uint2(uint32_t(fa[b & 1][2 * h]), uint32_t(fa[b & 1][2 * h + 1])));
                    long fb6 = __builtin_bit_cast(long, make_uint2(uint32_t(fb[st % kRing][2 * h]),
                                                                   uint32_t(fb[st % kRing][2 * h + 1])));
                    const i32x16 D6 = mfma16_at(fa6, fb6, srcC);
                    if constexpr (DOTS) {
                        int32_t *dots = reinterpret_cast<int32_t *>(outp);
                        const int n = n0 + col;
#pragma unroll
                        for (int r = 0; r < 16; r++) {
                            const int m = m0 + 32 * wr + 8 * (r >> 2) + 4 * g + (r & 3);
                            if (m < M && n < N)
                                dots[(int64_t(m) * N + n) * (2 * kb) + 2 * (int64_t(ks) * KB + b) + h] = D6[r];
                        }
                    } else {
                        scale_epilogue(acc[c], D6, ws, -kMagic * ws, xsv[b & 1]);
                        asm volatile("" : "+v"(acc[c]));
                    }
                }
            } else {
            const i32x16 D = mfma_at(fa[b & 1], fb[st % kRing], srcC);
            if constexpr (DEFER) {
                if (st == kSteps - 1) {   // its epilogue runs after the barrier
                    pendD = D;
                    pendW = fw[st % kRing];
                    pendX = xsv[b & 1];
                    pending = true;
                    continue;
                }
            }
            if constexpr (DOTS) {
                int32_t *dots = reinterpret_cast<int32_t *>(outp);
                const int n = n0 + col;
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int m = m0 + 32 * wr + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (m < M && n < N && b < nvalid)
                        dots[(int64_t(m) * N + n) * kb + int64_t(ks) * KB + b] = D[r];
                }
            } else {
                if constexpr (FMT == FMT_Q8_0)
                    scale_epilogue(acc[c], D, fw[st % kRing].x, fw[st % kRing].y, xsv[b & 1]);
                else
                    scale_epilogue(acc[c], D, fw[st % kRing], -kMagic * fw[st % kRing], xsv[b & 1]);
                // the epilogue happens here, not sunk to the end of the step
                asm volatile("" : "+v"(acc[c]));
            }
            }
        }
        if constexpr (has_min(FMT) && !DOTS) if (live) {
            // the min term of this step's four sub-blocks
            const _Float16 *sMin = reinterpret_cast<const _Float16 *>(bufb + L::OFF_B_MIN);
            // A = the four block sums s (high halves of the row's headers)
            const u32x4 h = *reinterpret_cast<const u32x4 *>(buf + L::OFF_A_HDR + (32 * wr + l32) * KB * 4);
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 sp = {__builtin_amdgcn_perm(h.y, h.x, 0x07060302u), __builtin_amdgcn_perm(h.w, h.z, 0x07060302u)};
            const f16x4 sa = __builtin_bit_cast(f16x4, sp);
            // the accumulators were last written by the asm FMAs, which the
            // compiler's hazard tracking does not see: wait states before an
            // MFMA reads them as its C operand
            asm volatile("s_nop 4" ::: "memory");
#pragma unroll
            for (int c = 0; c < kNSub; c++) {
                const f16x4 mb = *reinterpret_cast<const f16x4 *>(sMin + ((b_col0 + 32 * c) * 2 + g) * KB);
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x8f16(sa, mb, acc[c], 0, 0, 0);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // step ks+1's DMA has landed
        // PK: the scale pairs of step ks+1, stored where every load has
        // landed anyway (anywhere inside the step the compiler makes the
        // store wait for all loads in flight, the DMA pieces included)
        if constexpr (PK)
            if (j + 1 < nloc) pk_scale(nxtb);
        __syncthreads();
        if (j + 2 < nloc) load_w(ks + 2);
    };
    for (int j = 0; j < nloc; j += 2) {
        step(Parity<0>{}, j);
        if (j + 1 < nloc) step(Parity<1>{}, j + 1);
    }
    run_pending();

    if constexpr (MOE) {
        // scatter: tile row i -> routed row sorted[first + i]
        float *out = reinterpret_cast<float *>(outp);
        int64_t orow[16];
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int p = mt.y + 32 * wr + 8 * (r >> 2) + 4 * g + (r & 3);
            orow[r] = p < mt.z ? int64_t(moe.sorted[p]) * N : -1;
        }
#pragma unroll
        for (int c = 0; c < kNSub; c++) {
            const int n = n0 + b_col0 + 32 * c;
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (orow[r] >= 0 && n < N) out[orow[r] + n] = acc[c][r];
        }
    } else if constexpr (!DOTS) {
        float *out = reinterpret_cast<float *>(outp);
        bool split = gridDim.z > 1;   // partial sums: added into the zeroed output
        if (split && set.cnt) {
            // Split through the workspace: every slice stores its partial
            // tile; the slice that finds the tile's counter at S-1 on arrival
            // is the last, and it sums the S partials in slice order 0..S-1
            // (its own from registers) and stores the result.  No slice waits
            // for another, and the sum's order does not depend on which one
            // finishes last.
            // Coherence across the XCDs' separate L2 caches: the partials
            // are written and read with agent-scope coherent accesses (cache
            // policy sc1, what an agent-scope atomic load or store uses), and
            // each wave waits for its stores to complete before the
            // workgroup's arrival is counted; the counter is a relaxed
            // agent-scope atomic.  An agent-scope release/acquire fence pair
            // would do the same by writing back and invalidating the whole
            // L2, which slowed the concurrent workgroups' weight reads
            // (measured: the 512-token layer 0.48 -> 0.70 ms).
            constexpr int kCoherent = 16;   // sc1
            const int S = gridDim.z, me = blockIdx.z;
            const int64_t t = int64_t(ty) * gridDim.x + tx;
            const __amdgpu_buffer_rsrc_t rp = tile_rsrc(reinterpret_cast<const uint8_t *>(set.part) + t * S * 65536,
                                                        int64_t(S) * 65536);
            // float4 i of this thread in slice sl: byte ((sl * 8 + i) * 512 + tid) * 16
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int c = i >> 2, r = (i & 3) * 4;
                const u32x4 v = {__float_as_uint(acc[c][r]), __float_as_uint(acc[c][r + 1]),
                                 __float_as_uint(acc[c][r + 2]), __float_as_uint(acc[c][r + 3])};
                __builtin_amdgcn_raw_buffer_store_b128(v, rp, ((me * 8 + i) * kThreads + tid) * 16, 0, kCoherent);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's partial is in place
            __syncthreads();   // also: no wave reads either LDS buffer any more
            int *last = reinterpret_cast<int *>(lds0);
            if (tid == 0)
                *last = __hip_atomic_fetch_add(set.cnt + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                        uint32_t(S - 1);
            __syncthreads();
            if (!*last) return;   // workgroup-uniform
            f32x16 sum[kNSub];
            for (int sl = 0; sl < S; sl++) {
                f32x16 v[kNSub];
                if (sl == me) {
#pragma unroll
                    for (int c = 0; c < kNSub; c++) v[c] = acc[c];
                } else {
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(
                            rp, ((sl * 8 + i) * kThreads + tid) * 16, 0, kCoherent);
                        const int c = i >> 2, r = (i & 3) * 4;
                        v[c][r] = __uint_as_float(q.x);
                        v[c][r + 1] = __uint_as_float(q.y);
                        v[c][r + 2] = __uint_as_float(q.z);
                        v[c][r + 3] = __uint_as_float(q.w);
                    }
                }
#pragma unroll
                for (int c = 0; c < kNSub; c++) sum[c] = sl == 0 ? v[c] : sum[c] + v[c];
            }
#pragma unroll
            for (int c = 0; c < kNSub; c++) acc[c] = sum[c];
            split = false;
        }
#pragma unroll
        for (int c = 0; c < kNSub; c++) {
            const int n = n0 + b_col0 + 32 * c;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = m0 + 32 * wr + 8 * (r >> 2) + 4 * g + (r & 3);
                if (m < M && n < N) {
                    if (split)
                        unsafeAtomicAdd(out + int64_t(m) * N + n, acc[c][r]);
                    else
                        out[int64_t(m) * N + n] = acc[c][r];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Matrix-vector kernel for a few activation rows (decode, M <= kMvMaxM): the
// matvec contraction of "When Does a Kernel Win Surface?" (section 2; its
// section 8 puts decode at the HBM roofline).  Every weight byte is read
// once from HBM and used for all M rows, so the kernel is bound by the
// weight stream, and its arithmetic is VALU int8 dot products
// (v_dot4_i32_i8), not a matrix core: a wave computes one output row (all M
// rows of x against one weight row), or two for M >= 5 (see
// mv_rows_per_wave), at a time.  The lanes of the wave stride
// over the row in units of two 32-blocks (Q8_0: a 68-byte block pair, 17
// dwords; Q4_K: one 32-byte code group of a super-block, i.e. two sub-blocks,
// plus the super-block's 16-byte header), each lane keeping one fp32 partial
// sum per activation row in ascending unit order; the 64 partials are then
// summed by a butterfly.  The q8_1 activations (at most 8 x 21 KiB here) are
// read per unit straight from the caches.  The per-block arithmetic is the
// oracle's (t = fl(ws * I), then fma(xs, t, acc); Q4_K with its min term
// per sub-block); only the order of the sum over blocks differs.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int dot4x4(const uint32_t *a, const uint32_t *b) {
    int acc = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) acc = __builtin_amdgcn_sdot4(int(a[i]), int(b[i]), acc, false);
    return acc;
}

__device__ __forceinline__ int dot8(const uint32_t *a, const uint32_t *b) {
    int acc = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) acc = __builtin_amdgcn_sdot4(int(a[i]), int(b[i]), acc, false);
    return acc;
}

// The q8_1 block pair starting at block b of activation row m: headers and codes.
struct XPair {
    uint32_t h0, h1;
    uint32_t c0[8], c1[8];
};

__device__ __forceinline__ XPair load_x_pair(__amdgpu_buffer_rsrc_t rx, int off) {
    XPair x;
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16, 0, 0);
    const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rx, off + 32, 0, 0);
    const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(rx, off + 48, 0, 0);
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 e = __builtin_amdgcn_raw_buffer_load_b64(rx, off + 64, 0, 0);
    // dwords 0..17: [h0][c0 x 8][h1][c1 x 8]
    x.h0 = a.x;
    x.c0[0] = a.y; x.c0[1] = a.z; x.c0[2] = a.w; x.c0[3] = b.x;
    x.c0[4] = b.y; x.c0[5] = b.z; x.c0[6] = b.w; x.c0[7] = c.x;
    x.h1 = c.y;
    x.c1[0] = c.z; x.c1[1] = c.w; x.c1[2] = d.x; x.c1[3] = d.y;
    x.c1[4] = d.z; x.c1[5] = d.w; x.c1[6] = e.x; x.c1[7] = e.y;
    return x;
}

// The sum over a wave (all 64 lanes active).  Measured on the decode layers
// against a six-step xor butterfly through ds_bpermute: 3 % faster at M = 1
// (Q4_K 51.5 -> 49.8 us, Q8_0 71.6 -> 69.2), 5 % at M = 8 (Q8_0 107 -> 101.6,
// Q6_K 119.5 -> 113.5).  (The quantize pass's four-lane reductions measured
// 2 % slower through DPP and keep the shuffles.)
__device__ __forceinline__ float wave_sum(float v) {
    // butterfly inside each 16-lane row (every lane ends with its row's sum),
    // then the four row sums, read as wave-uniform values
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
}

// One weight unit (two 32-blocks) of one output row, ready for the dot
// products: one int8 code per byte, the weight scales and (K-quants) the
// min terms dmin * m of its two sub-blocks.
struct WUnit {
    uint32_t w0[8], w1[8];
    float ws0, ws1, dm0, dm1;
    float ws2, ws3;   // Q6_K: ws0..ws3 are the scales of the unit's four 16-element groups
};

// K-quant unit u of a row: one 32-byte code group of super-block u/4 (low
// nibbles: sub-block 2*grp, high nibbles: sub-block 2*grp+1) and the
// super-block's header; Q5_K adds the fifth bits from its high-bit plane.
template <int FMT>
__device__ __forceinline__ WUnit mv_load_kquant(__amdgpu_buffer_rsrc_t rw, int u) {
    WUnit r;
    const int sb = u >> 2, grp = u & 3;   // super-block, 32-byte code group
    constexpr int SB = FMT == FMT_Q4_K ? 144 : 176, QS = FMT == FMT_Q4_K ? 16 : 48;
    const u32x4 h = __builtin_amdgcn_raw_buffer_load_b128(rw, SB * sb, 0, 0);
    const u32x4 q0 = __builtin_amdgcn_raw_buffer_load_b128(rw, SB * sb + QS + 32 * grp, 0, 0);
    const u32x4 q1 = __builtin_amdgcn_raw_buffer_load_b128(rw, SB * sb + QS + 16 + 32 * grp, 0, 0);
    const uint32_t q[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        r.w0[i] = q[i] & 0x0f0f0f0fu;
        r.w1[i] = (q[i] >> 4) & 0x0f0f0f0fu;
    }
    if constexpr (FMT == FMT_Q5_K) {
        // fifth bits: byte l of the high-bit plane holds element l of
        // sub-block j in bit j (here j = 2*grp and 2*grp+1)
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rw, SB * sb + 16, 0, 0);
        const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rw, SB * sb + 32, 0, 0);
        const uint32_t qh[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; i++) {
            r.w0[i] |= ((qh[i] >> (2 * grp)) & 0x01010101u) << 4;
            r.w1[i] |= ((qh[i] >> (2 * grp + 1)) & 0x01010101u) << 4;
        }
    }
    // 6-bit scale and min of sub-blocks j = 2*grp + {0, 1} (the K-quant
    // packing: j < 4 in the low six bits of bytes j and j+4; j >= 4 low four
    // bits from byte j+4, top two bits from the spare top bits of bytes j-4
    // and j)
    const float d = h2f(h.x), dmin = h2f(h.x >> 16);
    float sc[2], mn[2];
#pragma unroll
    for (int t = 0; t < 2; t++) {
        const int j = 2 * grp + t, sh = 8 * (j & 3);
        const uint32_t b0 = (h.y >> sh) & 0xffu, b1 = (h.z >> sh) & 0xffu, b2 = (h.w >> sh) & 0xffu;
        const uint32_t sv = j < 4 ? (b0 & 63u) : ((b2 & 15u) | ((b0 >> 6) << 4));
        const uint32_t mv = j < 4 ? (b1 & 63u) : ((b2 >> 4) | ((b1 >> 6) << 4));
        sc[t] = (float)sv;
        mn[t] = (float)mv;
    }
    r.ws0 = d * sc[0];     // exact (11 x 6 bits)
    r.ws1 = d * sc[1];
    r.dm0 = dmin * mn[0];  // exact
    r.dm1 = dmin * mn[1];
    return r;
}

// Q6_K unit u of a row (blocks 2u, 2u+1 = quarters 2p, 2p+1 of half n of
// super-block u/4, p = u%2, n = (u/2)%2): low bits from nibble p of both
// 32-byte low-bit rows of the half (row 0 for quarter 2p, row 1 for 2p+1),
// high bits from bit pairs 2q of the half's 32 high-bit bytes, the four
// group scales 192 + 8n + 4p.. and d.  The super-block starts `sh` (0 or 2)
// bytes past the dword grid plus 2 bytes per odd index: each 32-byte field
// is loaded as the 9 dwords around it and realigned with v_perm.
__device__ __forceinline__ void q6k_window32(__amdgpu_buffer_rsrc_t rw, int f, uint32_t *out) {
    const int a = f & ~3;
    const u32x4 v0 = __builtin_amdgcn_raw_buffer_load_b128(rw, a, 0, 0);
    const u32x4 v1 = __builtin_amdgcn_raw_buffer_load_b128(rw, a + 16, 0, 0);
    const uint32_t v8 = __builtin_amdgcn_raw_buffer_load_b32(rw, a + 32, 0, 0);
    const uint32_t w[9] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w, v8};
    const uint32_t sel = (f & 2) ? 0x05040302u : 0x03020100u;
#pragma unroll
    for (int i = 0; i < 8; i++) out[i] = __builtin_amdgcn_perm(w[i + 1], w[i], sel);
}

__device__ __forceinline__ WUnit mv_load_q6k(__amdgpu_buffer_rsrc_t rw, int sh, int u) {
    WUnit r;
    const int sb = u >> 2, p = u & 1, n = (u >> 1) & 1;
    const int o = sh + sb * 210;
    uint32_t l0[8], l1[8], qh[8];
    q6k_window32(rw, o + 64 * n, l0);
    q6k_window32(rw, o + 64 * n + 32, l1);
    q6k_window32(rw, o + 128 + 32 * n, qh);
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const int fs = o + 192 + 8 * n + 4 * p, fd = o + 208;
    const u32x2 sv = __builtin_amdgcn_raw_buffer_load_b64(rw, fs & ~3, 0, 0);
    const uint32_t scw = __builtin_amdgcn_perm(sv.y, sv.x, (fs & 2) ? 0x05040302u : 0x03020100u);
    const uint32_t dw = __builtin_amdgcn_raw_buffer_load_b32(rw, fd & ~3, 0, 0);
    const float d = h2f((fd & 2) ? dw >> 16 : dw);
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t c0 = ((l0[i] >> (4 * p)) & 0x0F0F0F0Fu) | (((qh[i] >> (4 * p)) & 0x03030303u) << 4);
        const uint32_t c1 = ((l1[i] >> (4 * p)) & 0x0F0F0F0Fu) | (((qh[i] >> (4 * p + 2)) & 0x03030303u) << 4);
        r.w0[i] = ((c0 | 0x80808080u) - 0x20202020u) ^ 0x80808080u;   // c - 32 per byte
        r.w1[i] = ((c1 | 0x80808080u) - 0x20202020u) ^ 0x80808080u;
    }
    r.ws0 = d * (float)(int8_t)(scw & 0xffu);           // exact: 11 x 8 bits
    r.ws1 = d * (float)(int8_t)((scw >> 8) & 0xffu);
    r.ws2 = d * (float)(int8_t)((scw >> 16) & 0xffu);
    r.ws3 = d * (float)(int8_t)(scw >> 24);
    r.dm0 = r.dm1 = 0.0f;
    return r;
}

// One Q8_0 block from the 9 dwords at src, starting `off` (0 or 2) bytes in:
// scale in the low or high half of dword 0, codes realigned by v_perm (bytes
// 2..5 of each dword pair, or the upper dword whole).
__device__ __forceinline__ float mv_block_q8_0(const uint32_t *src, int off, uint32_t *w) {
    uint32_t v[9];
#pragma unroll
    for (int i = 0; i < 9; i++) v[i] = src[i];
    const uint32_t sel = off ? 0x07060504u : 0x05040302u;
#pragma unroll
    for (int i = 0; i < 8; i++) w[i] = __builtin_amdgcn_perm(v[i + 1], v[i], sel);
    return h2f(off ? v[0] >> 16 : v[0]);
}

// Q8_0 unit from LDS: its 68 bytes start `sh` bytes (0 or 2, the row's
// offset from the dword grid) past src.  Block 0 is read from dwords 0..8 at
// byte offset sh, block 1 from dwords 8 + sh/2 .. 16 + sh/2 at byte offset
// 2 - sh.  `pair` false: the row's odd last block, alone in its unit (block
// 1 gets scale 0 and is skipped by the caller).
__device__ __forceinline__ WUnit mv_unit_q8_0(const uint32_t *src, int sh, bool pair) {
    WUnit r;
    r.ws0 = mv_block_q8_0(src, sh, r.w0);
    r.ws1 = mv_block_q8_0(src + 8 + (sh >> 1), 2 - sh, r.w1);
    if (!pair) r.ws1 = 0.0f;
    r.dm0 = r.dm1 = 0.0f;
    return r;
}

// `pair` false (Q8_0 with an odd number of blocks, the row's last unit):
// only block 0 exists; the activation pair's second block is the next row's
// first (or zeros past the end) and is not added.
template <int FMT, int MR, int RW>
__device__ __forceinline__ void mv_unit_terms(__amdgpu_buffer_rsrc_t rx, int M, int kb, int u, const WUnit *wu,
                                              float (*acc)[MR], bool pair) {
#pragma unroll
    for (int m = 0; m < MR; m++) {
        if (m < M) {
            const XPair x = load_x_pair(rx, (m * kb + 2 * u) * 36);
            const float xs0 = h2f(x.h0), xs1 = h2f(x.h1);
            if constexpr (FMT == FMT_Q6_K) {
                // one term per 16-element group, in order, each with its own scale
#pragma unroll
                for (int r = 0; r < RW; r++) {
                    acc[r][m] = __builtin_fmaf(xs0, wu[r].ws0 * (float)dot4x4(wu[r].w0, x.c0), acc[r][m]);
                    acc[r][m] = __builtin_fmaf(xs0, wu[r].ws1 * (float)dot4x4(wu[r].w0 + 4, x.c0 + 4), acc[r][m]);
                    acc[r][m] = __builtin_fmaf(xs1, wu[r].ws2 * (float)dot4x4(wu[r].w1, x.c1), acc[r][m]);
                    acc[r][m] = __builtin_fmaf(xs1, wu[r].ws3 * (float)dot4x4(wu[r].w1 + 4, x.c1 + 4), acc[r][m]);
                }
                continue;
            }
#pragma unroll
            for (int r = 0; r < RW; r++) {
                const float t0 = wu[r].ws0 * (float)dot8(wu[r].w0, x.c0);
                const float t1 = wu[r].ws1 * (float)dot8(wu[r].w1, x.c1);
                acc[r][m] = __builtin_fmaf(xs0, t0, acc[r][m]);
                if constexpr (FMT != FMT_Q8_0) acc[r][m] = __builtin_fmaf(-wu[r].dm0, h2f(x.h0 >> 16), acc[r][m]);
                if (FMT != FMT_Q8_0 || pair) acc[r][m] = __builtin_fmaf(xs1, t1, acc[r][m]);
                if constexpr (FMT != FMT_Q8_0) acc[r][m] = __builtin_fmaf(-wu[r].dm1, h2f(x.h1 >> 16), acc[r][m]);
            }
        }
    }
}

// MR: activation rows compiled for (M <= MR).  RW: output rows per wave
// (mv_rows_per_wave(M), the planner's choice): with several activation rows
// the activation loads, served from the caches, cost more than the weight
// stream, and RW rows per wave divide them by RW.
template <int FMT, int MR>
__global__ __launch_bounds__(kMvThreads) void k_mmv(const uint8_t *__restrict__ xq, const GemmSet set, int M, int K) {
    constexpr int RW = mv_rows_per_wave(MR);
    const int lane = threadIdx.x & 63;
    // this wave's first output row over all GEMMs of the set; read as a
    // wave-uniform (scalar) value, so that the weight rows' buffer
    // descriptors live in scalar registers (a descriptor in vector registers
    // makes every load a loop over the lanes' distinct values)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row0 = (blockIdx.x * kMvWaves + wave) * RW;
    const int total = set_total(set);
    if (row0 >= total) return;
    const int kb = K >> 5;
    const int64_t wrow = weight_row_bytes(FMT, K);
    // row r of the wave: GEMM gi[r] of the set, its row n[r]; a row past the
    // last one reads through an empty buffer (zeros) and is not stored
    // (a Q8_0 row starts 2 bytes off the dword grid when its first block
    // index n*kb is odd: sh[r] = 2)
    __amdgpu_buffer_rsrc_t rw[RW];
    int gi[RW], n[RW], sh[RW];
#pragma unroll
    for (int r = 0; r < RW; r++) {
        const int row = row0 + r;
        const int g = set_member(set, row);
        gi[r] = g;
        n[r] = row - set.tile_start[g];
        const WBuf b = weight_rsrc(set.w[g] + int64_t(n[r]) * wrow, row < total ? wrow : 0);
        rw[r] = b.r;
        sh[r] = b.shift;
    }
    const __amdgpu_buffer_rsrc_t rx = tile_rsrc(xq, int64_t(M) * kb * 36);
    // block pairs (Q8_0) / sub-block pairs (K-quants) in a row; a Q8_0 row of
    // an odd number of blocks ends with a unit of one block
    const int units = (kb + 1) >> 1;

    float acc[RW][MR];
#pragma unroll
    for (int r = 0; r < RW; r++)
#pragma unroll
        for (int m = 0; m < MR; m++) acc[r][m] = 0.0f;

    // Q8_0 rows are read in 64-unit chunks (4352 bytes) with contiguous
    // 16-byte pieces per lane (each load instruction covers 1 KiB) into this
    // wave's own LDS area, and each lane then takes its 68-byte unit from
    // there: 68-byte units loaded straight by each lane touch ~34 cache lines
    // per instruction, and were measured 15-30 % slower.  K-quant units (a
    // 16-byte header and 32 code bytes, both 16-byte aligned) load straight:
    // the staged form was 10-13 % slower there.
    constexpr int kQ8Chunk = 64 * 68;
    constexpr int kQ8Pieces = kQ8Chunk / 16 + 1;   // one more for a row 2 bytes off the grid
    for (int u0 = 0; u0 < units; u0 += 64) {
        const int u = u0 + lane;
        const bool pair = 2 * u + 1 < kb;
        WUnit wu[RW];
        if constexpr (FMT == FMT_Q8_0) {
            __shared__ __attribute__((aligned(16))) uint8_t stage[kMvWaves][kQ8Pieces * 16];
            uint8_t *my = stage[wave];
#pragma unroll
            for (int r = 0; r < RW; r++) {
                // pieces past the row end read as zero
#pragma unroll
                for (int i = 0; i < (kQ8Pieces + 63) / 64; i++) {
                    const int piece = lane + 64 * i;
                    if (piece < kQ8Pieces)
                        *reinterpret_cast<u32x4 *>(my + 16 * piece) =
                            __builtin_amdgcn_raw_buffer_load_b128(rw[r], u0 * 68 + 16 * piece, 0, 0);
                }
                // the area is this wave's alone and LDS serves a wave's
                // accesses in order; the barriers only keep the compiler from
                // moving the unit reads above the other lanes' piece writes
                // (or the next row's writes above these reads)
                __builtin_amdgcn_wave_barrier();
                if (u < units) wu[r] = mv_unit_q8_0(reinterpret_cast<const uint32_t *>(my + 68 * lane), sh[r], pair);
                __builtin_amdgcn_wave_barrier();
            }
        } else if (u < units) {
#pragma unroll
            for (int r = 0; r < RW; r++) {
                if constexpr (FMT == FMT_Q6_K)
                    wu[r] = mv_load_q6k(rw[r], sh[r], u);
                else
                    wu[r] = mv_load_kquant<FMT>(rw[r], u);
            }
        }
        if (u < units) mv_unit_terms<FMT, MR, RW>(rx, M, kb, u, wu, acc, pair);
    }
#pragma unroll
    for (int r = 0; r < RW; r++) {
        if (row0 + r < total) {
            float *out = reinterpret_cast<float *>(set.out[gi[r]]);
            const int N = set.N[gi[r]];
#pragma unroll
            for (int m = 0; m < MR; m++) {
                if (m < M) {
                    const float v = wave_sum(acc[r][m]);
                    if (lane == 0) out[int64_t(m) * N + n[r]] = v;
                }
            }
        }
    }
}

// K-quant decode on the matrix core (the planner's choice for 2 <= M <= 8):
// the matvec above spends 16 dot instructions per unit and activation row on
// the VALU, so at M = 8 the VALU, not the weight stream, bounds it.  Here
// one int8 MFMA per 32-block takes the activation rows as A (rows m, 8 of
// its 32 used) and 32 weight rows as B: lane l holds weight row l%32 as its
// D column, so its weight scale and min are single values, and D rows
// 4(l/32) + r of registers r = 0..3 are the activation rows (the other 12
// registers hold rows >= 8 and are never read).  The epilogue is the
// oracle's per block (t = fl(ws * I), fma with the row's activation scale,
// then the min term), a lane summing its rows' blocks in ascending order.
// A workgroup of four waves takes 32 weight rows; wave w takes the w-th
// quarter of the super-blocks, and the four partial sums are added in wave
// order through LDS.
template <int FMT>
__global__ __launch_bounds__(kMvThreads) void k_mmvq(const uint8_t *__restrict__ xq, const GemmSet set, int M,
                                                     int K) {
    static_assert(FMT == FMT_Q4_K || FMT == FMT_Q5_K, "K-quant super-blocks with a min term");
    static_assert(kMvThreads == 64 * kMvqSlices, "one K-slice per wave");
    __shared__ float part[kMvqSlices][4][64];
    static_assert(sizeof(part) == kMvqLds, "plan and kernel LDS disagree");
    const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int total = set_total(set);
    const int row = int(blockIdx.x) * 32 + l32;   // this lane's weight row over the set
    const bool live = row < total;
    const int gi = set_member(set, row);
    const int n = row - set.tile_start[gi];
    constexpr int SB = FMT == FMT_Q4_K ? 144 : 176, QS = FMT == FMT_Q4_K ? 16 : 48;
    const int nsb = K >> 8, kb = K >> 5;
    const uint8_t *wrow = set.w[gi] + int64_t(live ? n : 0) * nsb * SB;
    const __amdgpu_buffer_rsrc_t rx = tile_rsrc(xq, int64_t(M) * kb * 36);   // rows >= M read as zero
    const int s0 = (nsb * wave) / kMvqSlices, s1 = (nsb * (wave + 1)) / kMvqSlices;
    i32x16 srcC;
#pragma unroll
    for (int r = 0; r < 16; r++) srcC[r] = int(kMagicBits);
    asm volatile("" : "+v"(srcC));
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const u32x4 zero = {0, 0, 0, 0};
    for (int sb = s0; sb < s1; sb++) {
        // every load of the super-block first (8 activation fragments and
        // headers, 4 weight code chunks), then its 8 MFMAs and epilogues
        const uint8_t *blk = wrow + int64_t(sb) * SB;
        const u32x4 hd = live ? *reinterpret_cast<const u32x4 *>(blk) : zero;
        u32x4 hb = zero;   // Q5_K: high-bit bytes 16h..16h+15 (element positions of this lane's k-half)
        if constexpr (FMT == FMT_Q5_K) hb = live ? *reinterpret_cast<const u32x4 *>(blk + 16 + 16 * h) : zero;
        u32x4 v[4];
#pragma unroll
        for (int grp = 0; grp < 4; grp++) v[grp] = live ? *reinterpret_cast<const u32x4 *>(blk + QS + 32 * grp + 16 * h) : zero;
        i32x4 A[8];
        uint32_t xh[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int b = 8 * sb + j;
            A[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (l32 * kb + b) * 36 + 4 + 16 * h, 0, 0));
            xh[j] = __builtin_amdgcn_raw_buffer_load_b32(rx, (l32 * kb + b) * 36, 0, 0);
        }
        const float d = h2f(hd.x), dmin = h2f(hd.x >> 16);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int grp = j >> 1, t = j & 1;
            i32x4 Bt;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                uint32_t c = t ? (v[grp][i] >> 4) & 0x0F0F0F0Fu : v[grp][i] & 0x0F0F0F0Fu;
                if constexpr (FMT == FMT_Q5_K) c |= ((hb[i] >> j) & 0x01010101u) << 4;
                Bt[i] = int(c);
            }
            // 6-bit scale and min of sub-block j (the K-quant packing)
            const int sh = 8 * (j & 3);
            const uint32_t b0 = (hd.y >> sh) & 0xffu, b1 = (hd.z >> sh) & 0xffu, b2 = (hd.w >> sh) & 0xffu;
            const uint32_t sc = j < 4 ? (b0 & 63u) : ((b2 & 15u) | ((b0 >> 6) << 4));
            const uint32_t mn = j < 4 ? (b1 & 63u) : ((b2 >> 4) | ((b1 >> 6) << 4));
            const float ws = d * (float)sc, dm = dmin * (float)mn;   // exact
            const i32x16 D = mfma_at(A[j], Bt, srcC);
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const uint32_t hr = uint32_t(__shfl(int(xh[j]), 4 * h + r, 64));   // row 4h + r's header
                const float tv = __builtin_fmaf(__int_as_float(D[r]), ws, -kMagic * ws);   // fl(ws * I)
                acc[r] = __builtin_fmaf(h2f(hr), tv, acc[r]);
                acc[r] = __builtin_fmaf(-dm, h2f(hr >> 16), acc[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; r++) part[wave][r][lane] = acc[r];
    __syncthreads();
    if (wave == 0 && live) {
        float *out = reinterpret_cast<float *>(set.out[gi]);
        const int N = set.N[gi];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int m = 4 * h + r;
            float v = part[0][r][lane];
#pragma unroll
            for (int w = 1; w < kMvqSlices; w++) v += part[w][r][lane];
            if (m < M) out[int64_t(m) * N + n] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Small remainders of the indexed MoE: the routed rows of an expert past its
// last full 128-row tile when there are at most kMoeSmallRows (32) of them.
// As a row tile such a remainder holds a workgroup slot about as long as a
// full tile (the weight staging and barriers of every k-step run for one
// live wave of eight).  Here a workgroup of four waves takes 128 weight rows
// of the expert over the whole of K, each wave 32 of them as the B operand
// of a 32 x 32 x 32 int8 MFMA per block, the remainder's (gathered)
// activation rows as A.
//
// Staging.  A vector load costs about one cycle per cache line its lanes
// touch (measured on gfx950, cache-resident: ~57 cycles for 64 lanes over 32
// rows, ~16 for 8 rows x 128 B or 1 KiB contiguous), so operands are not
// loaded lane = row as the MFMA wants them: every 16-byte load takes 8
// consecutive lanes along one row, by DMA into LDS (buffer_load ... lds),
// and the fragments are read back from LDS.
//   * activations, shared by the four waves: the 16-byte code halves of the
//     k-chunk's 4 blocks for 32 rows, 8 units per row, unit (block j, half
//     h) of row r in slot 8r + ((2j + h) xor (r mod 8)) (fragment reads of
//     consecutive rows hit distinct banks), then the rows' block headers;
//   * weights, per wave: the raw bytes of each of its 32 rows' k-chunk, as
//     W_UNITS 16-byte units from the dword below the first byte (Q8_0 and
//     Q6_K rows start 0 or 2 bytes off the dword grid; the fragment reads
//     realign them with v_perm), row stride 16 * W_UNITS bytes, the wave's
//     region padded to whole 64-lane DMA instructions.
// K is walked in chunks of 4 blocks (128 values); two LDS stages alternate,
// the next chunk's DMA issued before the current chunk's MFMAs.
//
// Grid: x = groups of 128 weight rows, y = the routing's list of small
// remainders (workgroups past the list's length exit at once).  Listed
// remainders, not experts, index the grid so that the live workgroups take
// its first positions and spread evenly over the CUs.
//
// Epilogue.  Lane l's output register r holds remainder row 8(r/4) +
// 4(l/32) + r%4, so register group r/4 holds rows 8(r/4)..8(r/4)+7: only
// the ceil(cnt/8) groups that hold routed rows get the scale epilogue.
//
// The arithmetic and its order are the tile kernel's: t = fl(ws * I), the
// row-broadcast FMA of the activation scale, blocks in ascending order (Q6_K:
// a 32 x 32 x 16 MFMA per 16-element group), so Q8_0 and Q6_K rows are
// bit-identical wherever the routing puts them.  The K-quants add their min
// term per sub-block as the oracle does (fma(-dm, s, acc), again by row
// broadcast), where the tile kernel adds it per k-step on a matrix core.
// ---------------------------------------------------------------------------
constexpr int kSmallThreads = 256, kSmallRowsPerWg = 128;

template <int FMT>
struct SmallLds {
    // 16-byte units of one weight row's k-chunk
    static constexpr int W_UNITS = FMT == FMT_Q8_0 ? 9 : FMT == FMT_Q4_K ? 5 : FMT == FMT_Q5_K ? 7 : 10;
    static constexpr int W_ROW = 16 * W_UNITS;
    static constexpr int W_DMA = (32 * W_UNITS + 63) / 64;   // DMA instructions per wave
    static constexpr int W_WAVE = 1024 * W_DMA;              // a wave's rows, padded to whole instructions
    static constexpr int A_CODES = 32 * 4 * 32;   // 32 rows x 4 blocks x 32 code bytes
    static constexpr int OFF_HDR = A_CODES;       // 32 rows x 4 block headers
    static constexpr int OFF_W = A_CODES + 32 * 4 * 4;
    static constexpr int BYTES = OFF_W + 4 * W_WAVE;
};
static_assert(2 * SmallLds<FMT_Q6_K>::BYTES * 3 <= 160 * 1024 && 2 * SmallLds<FMT_Q8_0>::BYTES * 3 <= 160 * 1024,
              "three small-remainder workgroups per CU");

// Byte offset (from the workgroup's weight buffer) of 16-byte unit p of
// weight row `row`'s k-chunk u, and that row's shift off the dword grid.
template <int FMT>
__device__ __forceinline__ int small_w_unit(int wshift, int kb, int row, int u, int p) {
    if constexpr (FMT == FMT_Q8_0) {
        return ((wshift + (row * kb + 4 * u) * 34) & ~3) + 16 * p;
    } else if constexpr (FMT == FMT_Q6_K) {
        const int a = (wshift + (row * (kb >> 3) + (u >> 1)) * 210) & ~3, hh = u & 1;
        // low bits (64 B of half hh), high bits (32 B), then scales and d
        return p < 5 ? a + 64 * hh + 16 * p : p < 8 ? a + 128 + 32 * hh + 16 * (p - 5) : a + 192 + 16 * (p - 8);
    } else {
        constexpr int SB = FMT == FMT_Q4_K ? 144 : 176, QS = FMT == FMT_Q4_K ? 16 : 48;
        const int base = (row * (kb >> 3) + (u >> 1)) * SB, hs = u & 1;
        if (p == 0) return base;                                            // d, dmin, scales
        if (FMT == FMT_Q5_K && p < 3) return base + 16 + 16 * (p - 1);      // high bits
        return base + QS + 64 * hs + 16 * (p - (FMT == FMT_Q5_K ? 3 : 1));  // code groups 2hs, 2hs+1
    }
}

// Issue the DMA of k-chunk u into buffer buf: every thread one activation
// code unit, every wave 64 block headers (waves 2 and 3 repeat waves 0 and
// 1: the same bytes into the same slots), every wave its 32 weight rows (the
// lanes past them reload the last unit into the padding).  Every DMA
// instruction has all lanes active and every wave issues kSmallDmaOps of
// them: the compiler's wait counts (and the pipeline's) rely on that count.
// The weight units' source offsets are returned in wo: the caller keeps them
// live until its compute is issued (a register the compute reused for an
// LDS read would make the compiler wait for the DMA first).
template <int FMT>
struct SmallDmaOffs {
    static constexpr int N = SmallLds<FMT>::W_DMA;
    int v[N];
};
template <int FMT>
constexpr int kSmallDmaOps = 2 + SmallDmaOffs<FMT>::N;


template <int FMT>
__device__ __forceinline__ void small_dma(__amdgpu_buffer_rsrc_t rx, int xcode, int xhdr,
                                          __amdgpu_buffer_rsrc_t rw, int wshift, int kb, int wave, int lane,
                                          int u, uint8_t *buf, SmallDmaOffs<FMT> &wo) {
    using L = SmallLds<FMT>;
    // the chunk's 4 blocks, in the lane offset: the buffer's range check
    // covers it (a Q8_0 row's last chunk may reach past the last token)
    const int cu = u * 4 * 36;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(buf + 1024 * wave), 16, xcode + cu, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(buf + L::OFF_HDR + 256 * (wave & 1)), 4, xhdr + cu, 0,
                                             0, 0);
    constexpr int kUnits = 32 * L::W_UNITS;
#pragma unroll
    for (int i = 0; i < SmallDmaOffs<FMT>::N; i++) {
        const int f = min(64 * i + lane, kUnits - 1);
        wo.v[i] = small_w_unit<FMT>(wshift, kb, 32 * wave + f / L::W_UNITS, u, f % L::W_UNITS);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(buf + L::OFF_W + wave * L::W_WAVE + 1024 * i), 16,
                                                 wo.v[i], 0, 0, 0);
    }
}

// acc[R0 + i] += (xsv of lane R0 + i of this lane's 16-lane row) * t_i,
// i = 0..3: one register group of the row-broadcast FMA (see
// fmac_row_bcast8; the leading s_nop covers the VALU writes just before).
#define MMQ_FMAC_BCAST4(R, A, T) "v_fmac_f32_dpp %" #A ", %8, %" #T " row_newbcast:" #R " row_mask:0xf bank_mask:0xf\n"
template <int R0>
__device__ __forceinline__ void fmac_row_bcast4(f32x16 &acc, float t0, float t1, float t2, float t3, float xsv) {
    float a0 = acc[R0 + 0], a1 = acc[R0 + 1], a2 = acc[R0 + 2], a3 = acc[R0 + 3];
#define MMQ_BCAST4_ASM(R0_, R1_, R2_, R3_)                                                                         \
    asm volatile("s_nop 1\n" MMQ_FMAC_BCAST4(R0_, 0, 4) MMQ_FMAC_BCAST4(R1_, 1, 5) MMQ_FMAC_BCAST4(R2_, 2, 6)       \
                     MMQ_FMAC_BCAST4(R3_, 3, 7)                                                                  \
                 : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3)                                                        \
                 : "v"(t0), "v"(t1), "v"(t2), "v"(t3), "v"(xsv))
    if constexpr (R0 == 0)
        MMQ_BCAST4_ASM(0, 1, 2, 3);
    else if constexpr (R0 == 4)
        MMQ_BCAST4_ASM(4, 5, 6, 7);
    else if constexpr (R0 == 8)
        MMQ_BCAST4_ASM(8, 9, 10, 11);
    else
        MMQ_BCAST4_ASM(12, 13, 14, 15);
#undef MMQ_BCAST4_ASM
    acc[R0 + 0] = a0; acc[R0 + 1] = a1; acc[R0 + 2] = a2; acc[R0 + 3] = a3;
}
#undef MMQ_FMAC_BCAST4

// The scale epilogue (t = fl(ws * I), acc += xs * t) of register group G.
template <int G>
__device__ __forceinline__ void small_epi_group(f32x16 &acc, const i32x16 &D, float ws, float cs, float xsv) {
    fmac_row_bcast4<4 * G>(acc, __builtin_fmaf(__int_as_float(D[4 * G]), ws, cs),
                           __builtin_fmaf(__int_as_float(D[4 * G + 1]), ws, cs),
                           __builtin_fmaf(__int_as_float(D[4 * G + 2]), ws, cs),
                           __builtin_fmaf(__int_as_float(D[4 * G + 3]), ws, cs), xsv);
}

// The scale epilogue of the first ng register groups (ng wave-uniform).
__device__ __forceinline__ void small_epilogue(f32x16 &acc, const i32x16 &D, float ws, float cs, float xsv, int ng) {
    small_epi_group<0>(acc, D, ws, cs, xsv);
    if (ng > 1) small_epi_group<1>(acc, D, ws, cs, xsv);
    if (ng > 2) small_epi_group<2>(acc, D, ws, cs, xsv);
    if (ng > 3) small_epi_group<3>(acc, D, ws, cs, xsv);
}

// The K-quant min term of the first ng groups: acc[r] += s(row of r) * c,
// the row's block sum s arriving by the same row broadcast as the scale.
__device__ __forceinline__ void small_min(f32x16 &acc, float c, float sv, int ng) {
    fmac_row_bcast4<0>(acc, c, c, c, c, sv);
    if (ng > 1) fmac_row_bcast4<4>(acc, c, c, c, c, sv);
    if (ng > 2) fmac_row_bcast4<8>(acc, c, c, c, c, sv);
    if (ng > 3) fmac_row_bcast4<12>(acc, c, c, c, c, sv);
}

// LDS reads of the small kernel are written as one byte offset from the
// buffer's base: the compiler's LDS lowering gives a read the alias scope of
// its buffer only through a few levels of address arithmetic, and a read
// without one waits for every LDS DMA in flight (the next chunk's included).
template <typename T>
__device__ __forceinline__ T lds_at(const uint8_t *buf, int off) {
    return *reinterpret_cast<const T *>(buf + off);
}

__device__ __forceinline__ void lds_at_store(uint8_t *buf, int off, float v) { *reinterpret_cast<float *>(buf + off) = v; }

// 8 bytes starting at byte b (even) of buf, from the three dwords around them.
__device__ __forceinline__ uint2 lds_field8(const uint8_t *buf, int b) {
    const int a = b & ~3;
    const uint32_t sel = (b & 2) ? 0x05040302u : 0x03020100u;
    const uint32_t w0 = lds_at<uint32_t>(buf, a), w1 = lds_at<uint32_t>(buf, a + 4), w2 = lds_at<uint32_t>(buf, a + 8);
    return make_uint2(__builtin_amdgcn_perm(w1, w0, sel), __builtin_amdgcn_perm(w2, w1, sel));
}

// The MFMAs and epilogues of k-chunk u from buffer buf, for one wave's 32
// weight rows: activation code units at a0 (AR rows staged, 16 or 32),
// their block headers at h0 (16 bytes per row), the weight rows' windows at
// w0; wrow is this lane's weight row counted from the weight buffer's start.
// With AR = 16 the lanes of rows 16-31 read rows 0-15 again: their D rows lie
// in register groups 2 and 3, which the epilogue of ng <= 2 never reads.
//
// CB = 8 (K-quants only): the stage holds 8-block chunks (whole
// super-blocks), the weight window of a row is its raw super-block and the
// activation rows hold 16 code units (XOR-swizzled by row % 16) and 8
// headers; `sub` picks the chunk's half computed here and u is the 4-block
// unit index of that half.
//
// MINMFMA (K-quants): the min term of the half chunk as two fp32 MFMAs
// (32 x 32 x 2, two blocks each: A = the activation rows' block sums, B =
// -dmin * m of the weight rows' sub-blocks) into the accumulator, instead of
// one row-broadcast FMA per register group and block; its sums are then in
// the matrix core's order, not the oracle's.
template <int FMT, int AR = 32, int CB = 4, bool MINMFMA = false>
__device__ __forceinline__ void small_compute(const uint8_t *buf, int a0, int h0, int w0, int wrow, f32x16 &acc,
                                              const i32x16 &srcC, int wshift, int kb, int lane, int u, int ng,
                                              int sub = 0) {
    static_assert(AR == 16 || AR == 32, "16 or 32 staged activation rows");
    static_assert(CB == 4 || (CB == 8 && FMT != FMT_Q8_0), "4-block chunks, or whole super-blocks");
    constexpr int W_ROW = CB == 4 ? SmallLds<FMT>::W_ROW : 16 * sm_w_units_sb(FMT);
    const int l32 = lane & 31, g = lane >> 5, ar = l32 & (AR - 1);
    // the row whose header this lane broadcasts
    const int xr = (8 * ((lane & 15) >> 2) + (lane & 3) + 4 * g) & (AR - 1);
    const int wr = w0 + l32 * W_ROW;                // this lane's weight row
    const int hdr = h0 + 4 * CB * xr + 16 * sub;    // its 4 block headers of the half
    auto a_unit = [&](int j, int h) {
        return a0 + 16 * (2 * CB * ar + ((2 * (4 * sub + j) + h) ^ (ar & (2 * CB - 1))));
    };
    if constexpr (FMT == FMT_Q8_0) {
        const int sh = (wshift + wrow * kb * 34 + u * 4 * 34) & 3;   // the row's chunk start, 0 or 2
#pragma unroll
        for (int j = 0; j < 4; j++) {
            if (4 * u + j >= kb) break;   // wave-uniform: the row's last chunk may hold 1-3 blocks
            const int b0 = wr + sh + 34 * j;   // the block's first byte
            const float ws = h2f(lds_at<unsigned short>(buf, b0));
            const uint2 c0 = lds_field8(buf, b0 + 2 + 16 * g), c1 = lds_field8(buf, b0 + 10 + 16 * g);
            i32x4 bf = {int(c0.x), int(c0.y), int(c1.x), int(c1.y)};
            i32x4 af = lds_at<i32x4>(buf, a_unit(j, g));
            const i32x16 D = mfma_at(af, bf, srcC);
            small_epilogue(acc, D, ws, -kMagic * ws, h2f(lds_at<uint32_t>(buf, hdr + 4 * j)), ng);
            asm volatile("" : "+v"(acc));
        }
    } else if constexpr (FMT == FMT_Q6_K) {
        const int hh = u & 1;
        const int w6 = wr + ((wshift + (wrow * (kb >> 3) + (u >> 1)) * 210) & 3);
        // window offsets (CB = 4): low bits at 0, high bits at 80, scales at
        // 128, d at 144 (each from its dword); the raw super-block (CB = 8):
        // low bits of the half at 64 hh, its high bits at 128 + 32 hh,
        // scales at 192, d at 208
        constexpr int SC = CB == 4 ? 128 : 192, DO = CB == 4 ? 144 : 208;
        const int LO = CB == 4 ? 0 : 64 * hh, HI = CB == 4 ? 80 : 128 + 32 * hh;
        const float d = h2f(lds_at<unsigned short>(buf, w6 + DO));
        const uint2 hb[2] = {lds_field8(buf, w6 + HI + 8 * g), lds_field8(buf, w6 + HI + 16 + 8 * g)};
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const float xs = h2f(lds_at<uint32_t>(buf, hdr + 4 * q));
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const uint2 lb = lds_field8(buf, w6 + LO + 32 * (q & 1) + 16 * h + 8 * g);
                const int ns = 4 * (q >> 1);
                const uint32_t c0 = ((lb.x >> ns) & 0x0F0F0F0Fu) | (((hb[h].x >> (2 * q)) & 0x03030303u) << 4);
                const uint32_t c1 = ((lb.y >> ns) & 0x0F0F0F0Fu) | (((hb[h].y >> (2 * q)) & 0x03030303u) << 4);
                long b6 = __builtin_bit_cast(long, make_uint2(q6k_centre(c0), q6k_centre(c1)));
                long a6 = lds_at<long>(buf, a_unit(q, h) + 8 * g);
                // scale of group 2q + h of the half: byte 192 + 8hh + 2q + h of the super-block
                const float ws = d * (float)lds_at<int8_t>(buf, w6 + SC + 8 * hh + 2 * q + h);
                const i32x16 D6 = mfma16_at(a6, b6, srcC);
                small_epilogue(acc, D6, ws, -kMagic * ws, xs, ng);
                asm volatile("" : "+v"(acc));
            }
        }
    } else {
        const int hs = u & 1;
        const u32x4 hd = lds_at<u32x4>(buf, wr);
        const float d = h2f(hd.x), dmin = h2f(hd.x >> 16);
        // the code groups' place in the row's window (the raw super-block:
        // those of half hs)
        const int C0 = (FMT == FMT_Q5_K ? 48 : 16) + (CB == 8 ? 64 * hs : 0);
        // this lane's k-half of the row, an opaque offset: the high-bit and
        // code reads would otherwise share address arithmetic deep enough to
        // lose their alias scope (Q5_K)
        int wq = wr + 16 * g;
        asm volatile("" : "+v"(wq));
        u32x4 qh = {0, 0, 0, 0};
        if constexpr (FMT == FMT_Q5_K) qh = lds_at<u32x4>(buf, wq + 16);
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
            const int j = 4 * hs + jj;   // the sub-block within its super-block
            const u32x4 v = lds_at<u32x4>(buf, wq + C0 + 32 * (jj >> 1));
            i32x4 bf;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                uint32_t c = (jj & 1) ? (v[i] >> 4) & 0x0F0F0F0Fu : v[i] & 0x0F0F0F0Fu;
                if constexpr (FMT == FMT_Q5_K) c |= ((qh[i] >> j) & 0x01010101u) << 4;
                bf[i] = int(c);
            }
            // 6-bit scale and min of sub-block j (the K-quant packing)
            const int s8 = 8 * (j & 3);
            const uint32_t b0 = (hd.y >> s8) & 0xffu, b1 = (hd.z >> s8) & 0xffu, b2 = (hd.w >> s8) & 0xffu;
            const uint32_t sc = j < 4 ? (b0 & 63u) : ((b2 & 15u) | ((b0 >> 6) << 4));
            const uint32_t mn = j < 4 ? (b1 & 63u) : ((b2 >> 4) | ((b1 >> 6) << 4));
            const float ws = d * (float)sc, dm = dmin * (float)mn;   // exact
            i32x4 af = lds_at<i32x4>(buf, a_unit(jj, g));
            const uint32_t xh = lds_at<uint32_t>(buf, hdr + 4 * jj);
            const i32x16 D = mfma_at(af, bf, srcC);
            small_epilogue(acc, D, ws, -kMagic * ws, h2f(xh), ng);
            asm volatile("" : "+v"(acc));
            if constexpr (!MINMFMA) {
                small_min(acc, -dm, h2f(xh >> 16), ng);
                asm volatile("" : "+v"(acc));
            }
        }
        if constexpr (MINMFMA) {
            // lane l: A row l % 32 (activation row ar) and B column l % 32
            // (weight row l32) at k = l / 32 = g: blocks g and 2 + g of the
            // half chunk, one MFMA each pair
            const int xrow = h0 + 4 * CB * ar + 16 * sub;
            const float sa0 = h2f(lds_at<uint32_t>(buf, xrow + 4 * g) >> 16);
            const float sa1 = h2f(lds_at<uint32_t>(buf, xrow + 8 + 4 * g) >> 16);
            auto neg_dm = [&](int jj) {
                const int j = 4 * hs + jj, s8 = 8 * (j & 3);
                const uint32_t b0 = (hd.y >> s8) & 0xffu, b1 = (hd.z >> s8) & 0xffu, b2 = (hd.w >> s8) & 0xffu;
                const uint32_t mn = j < 4 ? (b1 & 63u) : ((b2 >> 4) | ((b1 >> 6) << 4));
                return -(dmin * (float)mn);
            };
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sa0, neg_dm(g), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sa1, neg_dm(2 + g), acc, 0, 0, 0);
            asm volatile("" : "+v"(acc));
        }
    }
}

template <int FMT>
__global__ __launch_bounds__(kSmallThreads) void k_moe_small(const uint8_t *__restrict__ xq,
                                                             const uint8_t *__restrict__ w, float *__restrict__ out,
                                                             int T, int N, int K, const MoeArgs moe) {
    static_assert(kSmallThreads == 64 * (kSmallRowsPerWg / 32) && kMoeSmallRows == 32, "one wave per 32 weight rows");
    using L = SmallLds<FMT>;
    // The two stages as two variables, so that the compiler knows the DMA
    // into one cannot write what the reads of the other return (see k_mmq).
    __shared__ __attribute__((aligned(16))) uint8_t lds0[L::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[L::BYTES];
    // tables built for other routed rows or experts (or never built):
    // nothing is computed and nothing written
    const int4 mh = moe.header[0];
    if (mh.x != kMoeMagic || mh.y != moe.R || mh.z != moe.E) return;
    // the listed remainders take the grid's first rows, so that their
    // workgroups spread evenly over the CUs; the rest exit (workgroup-
    // uniform, before any barrier)
    if (int(blockIdx.y) >= moe.header[1].x) return;
    const int4 se = moe.small[blockIdx.y];
    const int e = se.x;
    const int2 rr = make_int2(se.y, se.z);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = int(blockIdx.x) * kSmallRowsPerWg;   // the workgroup's first weight row
    const int kb = K >> 5;
    const int64_t wrow = weight_row_bytes(FMT, K);
    // weight rows past N read as zero (scale 0) and are never stored
    const WBuf rwb = weight_rsrc(w + int64_t(e) * moe.expert_bytes + int64_t(n0) * wrow, int64_t(N - n0) * wrow);
    const __amdgpu_buffer_rsrc_t rx = tile_rsrc(xq, int64_t(T) * kb * 36);
    // this thread's activation DMA sources at chunk 0 (rows past the
    // remainder read token 0 and are never stored)
    int xcode, xhdr;
    {
        const int r = tid >> 3, q = (tid & 7) ^ (r & 7);
        xcode = gathered_row(moe.sorted, rr.x, rr.y, moe.topk, r) * kb * 36 + (q >> 1) * 36 + 4 + 16 * (q & 1);
        const int hi = 64 * ((tid >> 6) & 1) + lane;   // header slot: row hi / 4, block hi % 4
        xhdr = gathered_row(moe.sorted, rr.x, rr.y, moe.topk, hi >> 2) * kb * 36 + (hi & 3) * 36;
    }
    const bool live = n0 + 32 * wave < N;   // wave-uniform: the wave has weight rows to compute
    const int ng = (rr.y - rr.x + 7) >> 3;  // register groups holding routed rows (1..4)

    i32x16 srcC;
#pragma unroll
    for (int r = 0; r < 16; r++) srcC[r] = int(kMagicBits);
    asm volatile("" : "+v"(srcC));
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; r++) acc[r] = 0.0f;

    // Two LDS stages: chunk u computes from stage u % 2 while the DMA of
    // chunk u + 1 is in flight; at its end the wave waits for that DMA and
    // the barrier makes every wave's part of it visible and frees stage
    // u % 2 for chunk u + 2.  Every chunk issues its DMA and the loop runs an
    // even number of chunks, the DMA index clamped to the last chunk (a
    // reload from the cache into a stage nothing reads) and the compute
    // skipped past it: with the DMA behind a branch the compiler's wait
    // counts, unable to tell how many DMA were in flight, waited for the
    // next chunk's too before reading the current one.  (Three stages, the
    // DMA two chunks ahead, measured slower.)
    const int nunits = (kb + 3) >> 2, last = nunits - 1;
    {
        SmallDmaOffs<FMT> wo;
        small_dma<FMT>(rx, xcode, xhdr, rwb.r, rwb.shift, kb, wave, lane, 0, lds0, wo);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    auto chunk = [&](auto parity, int u) {
        constexpr int P = decltype(parity)::value;
        uint8_t *const cur = P ? lds1 : lds0;
        uint8_t *const nxt = P ? lds0 : lds1;
        SmallDmaOffs<FMT> wo;
        small_dma<FMT>(rx, xcode, xhdr, rwb.r, rwb.shift, kb, wave, lane, min(u + 1, last), nxt, wo);
        if (live && u < nunits)
            small_compute<FMT>(cur, 0, L::OFF_HDR, L::OFF_W + wave * L::W_WAVE, 32 * wave + (lane & 31), acc, srcC,
                               rwb.shift, kb, lane, u, ng);
#pragma unroll
        for (int i = 0; i < SmallDmaOffs<FMT>::N; i++) asm volatile("" ::"v"(wo.v[i]));
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // chunk u + 1 has landed
        __syncthreads();                                    // and no wave reads chunk u any more
    };
    for (int u = 0; u < nunits; u += 2) {
        chunk(Parity<0>{}, u);
        chunk(Parity<1>{}, u + 1);
    }
    if (!live) return;

    // scatter: row m of the remainder -> routed row sorted[first + m] (the
    // 16 ids loaded together, rows past the remainder clamped to its last)
    const int g = lane >> 5, n = n0 + 32 * wave + (lane & 31), cnt = rr.y - rr.x;
    int orow[16];
#pragma unroll
    for (int r = 0; r < 16; r++) orow[r] = moe.sorted[rr.x + min(8 * (r >> 2) + 4 * g + (r & 3), cnt - 1)];
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int m = 8 * (r >> 2) + 4 * g + (r & 3);
        if (m < cnt && n < N) out[int64_t(orow[r]) * N + n] = acc[r];
    }
}

// ---------------------------------------------------------------------------
// Batch decode (9 <= M <= 32 activation rows): the matrix-core step of the
// small-remainder kernel above, for dense GEMMs and GEMM sets.  A workgroup
// takes 32 weight rows (one set member's: the grid's x counts 32-row groups
// per member) as the B operand of a 32 x 32 x 32 int8 MFMA per block, the
// activation rows as A (AR = 16 or 32 staged; rows past M read as zero
// through the buffer's range check and are never stored).  A 128-row tile
// kernel would leave 3 of its 4 wave rows idle at these sizes and give
// narrow GEMMs (N = 3584 at K = 18944: 28 tiles) a small fraction of the
// CUs; here the same GEMM has 112 workgroups of four waves.
//
// Each wave takes a K-slice of the 32 rows: slice q = 4 * blockIdx.z + wave
// of S = 4 * gridDim.z holds chunks [nunits * q / S, nunits * (q + 1) / S) of
// CB blocks (4, or a whole super-block for Q4_K with 16 staged rows: one
// contiguous span per weight row).  The waves share nothing while they run: each stages its own
// activation codes and headers and its rows' weight windows (the layouts of
// the small-remainder kernel) into LDS of its own by DMA, two stages deep,
// with no barrier.  At the end the four partial sums are added in wave
// order through LDS (wave w adds register group w, the output rows
// 8w..8w+7) and stored; with gridDim.z = 2 the two workgroups of a row group
// add theirs into the zeroed output with fp32 atomics (two terms onto an
// exact zero: the same result in either order).
//
// Every DMA offset is in the lane's offset register, never the scalar one,
// so that the buffer's range check sees the whole offset (the last chunk of
// a Q8_0 row with K % 128 != 0 reaches past the row's end).
// ---------------------------------------------------------------------------
template <int FMT, int AR, int CB = sm_cb(FMT, AR)>
struct SmLds {
    static_assert(SmallLds<FMT>::W_UNITS == sm_w_units(FMT), "plan and kernel weight windows disagree");
    static constexpr int W_UNITS = CB == 4 ? sm_w_units(FMT) : sm_w_units_sb(FMT);
    static constexpr int W_DMA = (32 * W_UNITS + 63) / 64;   // weight DMA instructions per wave
    static constexpr int A = 0;                      // AR rows x 2 CB code units of 16 bytes
    static constexpr int H = AR * CB * 32;           // AR rows x CB block headers
    static constexpr int W = H + AR * CB * 4;        // the 32 weight rows' windows
    static constexpr int WAVE = W + 1024 * W_DMA;    // one wave's stage
    static constexpr int STAGE = kSmWaves * WAVE;
    static constexpr int NC = AR * CB * 2 / 64, NH = AR * CB / 64;   // activation DMA instructions
};
static_assert(kSmStages * SmLds<FMT_Q8_0, 32>::STAGE == sm_lds_bytes(FMT_Q8_0, 32) &&
                  kSmStages * SmLds<FMT_Q4_K, 16>::STAGE == sm_lds_bytes(FMT_Q4_K, 16) &&
                  kSmStages * SmLds<FMT_Q5_K, 32>::STAGE == sm_lds_bytes(FMT_Q5_K, 32) &&
                  kSmStages * SmLds<FMT_Q6_K, 16>::STAGE == sm_lds_bytes(FMT_Q6_K, 16) && kSmStages >= 2 &&
                  kSmStages <= 4,
              "plan and kernel LDS disagree");

template <int N>
struct DmaOffs {
    int v[N];
};

// A lane's activation DMA sources at chunk 0: code unit f = 64 i + lane is
// slot f of the stage (row f / 8, unit (2j + h) = (f % 8) xor (row % 8)),
// header slot 64 i + lane is row (64 i + lane) / 4, block lane % 4.
template <int FMT, int AR>
struct SmActOffs {
    int code[SmLds<FMT, AR>::NC];
    int hdr[SmLds<FMT, AR>::NH];
};

// Source offset of 16-byte unit p of weight row `row`'s chunk u (CB = 8: its
// super-block u, from the dword below its first byte).
template <int FMT, int CB>
__device__ __forceinline__ int sm_w_unit(int wshift, int kb, int row, int u, int p) {
    if constexpr (CB == 4) {
        return small_w_unit<FMT>(wshift, kb, row, u, p);
    } else if constexpr (FMT == FMT_Q6_K) {
        return ((wshift + (row * (kb >> 3) + u) * 210) & ~3) + 16 * p;
    } else {
        return (row * (kb >> 3) + u) * (FMT == FMT_Q4_K ? 144 : 176) + 16 * p;
    }
}

template <int FMT, int AR>
__device__ __forceinline__ void sm_dma(__amdgpu_buffer_rsrc_t rx, const SmActOffs<FMT, AR> &xo,
                                       __amdgpu_buffer_rsrc_t rw, int wshift, int kb, int lane, int u, uint8_t *buf,
                                       int base, DmaOffs<SmLds<FMT, AR>::W_DMA> &wo) {
    using S = SmLds<FMT, AR>;
    constexpr int CB = sm_cb(FMT, AR);
    const int cu = u * CB * 36;   // the chunk's CB blocks
#pragma unroll
    for (int i = 0; i < S::NC; i++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(buf + base + S::A + 1024 * i), 16, xo.code[i] + cu,
                                                 0, 0, 0);
#pragma unroll
    for (int i = 0; i < S::NH; i++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(buf + base + S::H + 256 * i), 4, xo.hdr[i] + cu, 0,
                                                 0, 0);
    constexpr int kUnits = 32 * S::W_UNITS;
#pragma unroll
    for (int i = 0; i < S::W_DMA; i++) {
        const int f = min(64 * i + lane, kUnits - 1);
        wo.v[i] = sm_w_unit<FMT, CB>(wshift, kb, f / S::W_UNITS, u, f % S::W_UNITS);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(buf + base + S::W + 1024 * i), 16, wo.v[i], 0, 0,
                                                 0);
    }
}

template <int FMT, int AR>
__global__ __launch_bounds__(kSmThreads) void k_mmsm(const uint8_t *__restrict__ xq, const GemmSet set, int M,
                                                     int K) {
    static_assert(kSmRows == 32 && kSmThreads == 256, "four waves over 32 weight rows");
    using S = SmLds<FMT, AR>;
    static_assert(S::STAGE >= kSmWaves * 16 * 64 * 4, "the partial sums fit one stage");
    // the stages as variables of their own (see k_moe_small), each holding
    // the four waves' regions
    constexpr int NST = kSmStages;
    __shared__ __attribute__((aligned(16))) uint8_t lds0[S::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[S::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds2[NST > 2 ? S::STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t lds3[NST > 3 ? S::STAGE : 16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // M > 32: the workgroup's 32-row group bx and activation row block yb
    // (rows 32 yb .. 32 yb + 31).  The Y row blocks of a group are 8 ids
    // apart, so that they run on one XCD at about the same time and the
    // later ones find the weight rows in its L2 (ids go to the XCDs in turn);
    // ids past the last group (the grid is padded to whole groups of 8) exit.
    static_assert(kSmRowBlock == 32, "row blocks of one MFMA operand");
    int bx = int(blockIdx.x), yb = 0;
    if (AR == 32 && M > kSmRowBlock) {
        const int Y = (M + 31) >> 5, r = bx % (8 * Y);
        bx = bx / (8 * Y) * 8 + (r & 7);
        yb = r >> 3;
        if (bx >= set_total(set)) return;
    }
    const int gi = set_member(set, bx);
    const int N = set.N[gi], n0 = (bx - set.tile_start[gi]) * kSmRows;
    const int kb = K >> 5;
    const int64_t wrow = weight_row_bytes(FMT, K);
    // weight rows past N read as zero (scale 0) and are never stored
    const WBuf rwb = weight_rsrc(set.w[gi] + int64_t(n0) * wrow, int64_t(N - n0) * wrow);
    const int m0 = 32 * yb, Mb = min(M - m0, AR);   // the block's activation rows
    const __amdgpu_buffer_rsrc_t rx = tile_rsrc(xq + int64_t(m0) * kb * 36, int64_t(Mb) * kb * 36);
    constexpr int CB = sm_cb(FMT, AR);
    SmActOffs<FMT, AR> xo;
#pragma unroll
    for (int i = 0; i < S::NC; i++) {
        const int f = 64 * i + lane, r = f / (2 * CB), q = (f % (2 * CB)) ^ (r & (2 * CB - 1));
        xo.code[i] = r * kb * 36 + (q >> 1) * 36 + 4 + 16 * (q & 1);
    }
#pragma unroll
    for (int i = 0; i < S::NH; i++) {
        const int hi = 64 * i + lane;
        xo.hdr[i] = (hi / CB) * kb * 36 + (hi % CB) * 36;
    }
    // register groups holding activation rows: 2 (M <= 16), else 3 or 4 (a
    // select of constants, so the epilogue's first two group tests fold; a
    // last row block of at most 16 rows computes one group of zero rows)
    const int ng = AR == 16 ? 2 : (Mb > 24 ? 4 : 3);
    const int nunits = CB == 4 ? (kb + 3) >> 2 : kb >> 3, slices = kSmWaves * int(gridDim.z);
    const int sq = int(blockIdx.z) * kSmWaves + wave;
    const int c0 = nunits * sq / slices, c1 = nunits * (sq + 1) / slices;
    const int base = wave * S::WAVE;

    i32x16 srcC;
#pragma unroll
    for (int r = 0; r < 16; r++) srcC[r] = int(kMagicBits);
    asm volatile("" : "+v"(srcC));
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; r++) acc[r] = 0.0f;

    auto stage = [&](auto p) -> uint8_t * {
        constexpr int P = decltype(p)::value % NST;
        if constexpr (P == 0) return lds0;
        else if constexpr (P == 1) return lds1;
        else if constexpr (P == 2) return lds2;
        else return lds3;
    };
    if (c1 > c0) {   // wave-uniform: a K-slice with chunks
        // the first NST - 1 chunks (clamped to the slice)
        {
            DmaOffs<S::W_DMA> wo;
            sm_dma<FMT, AR>(rx, xo, rwb.r, rwb.shift, kb, lane, c0, stage(Parity<0>{}), base, wo);
            if constexpr (NST > 2) sm_dma<FMT, AR>(rx, xo, rwb.r, rwb.shift, kb, lane, min(c0 + 1, c1 - 1),
                                                   stage(Parity<1>{}), base, wo);
            if constexpr (NST > 3) sm_dma<FMT, AR>(rx, xo, rwb.r, rwb.shift, kb, lane, min(c0 + 2, c1 - 1),
                                                   stage(Parity<2>{}), base, wo);
        }
        // Chunk u computes from stage u % NST while the DMA of chunks up to
        // u + NST - 1 fill the others (the compiler's wait before the first
        // read of a stage leaves the later DMA in flight).  Every chunk
        // issues its DMA, the index clamped to the slice's last chunk, and
        // the loop runs a multiple of NST chunks with the compute skipped
        // past the slice: the wait counts rely on every iteration issuing
        // the same DMA instructions.
        auto chunk = [&](auto parity, int u) {
            constexpr int P = decltype(parity)::value;
            DmaOffs<S::W_DMA> wo;
            // the reads of chunk u - 1 from the stage refilled here have returned
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            sm_dma<FMT, AR>(rx, xo, rwb.r, rwb.shift, kb, lane, min(u + NST - 1, c1 - 1),
                            stage(Parity<P + NST - 1>{}), base, wo);
            if (u < c1) {
#pragma unroll
                for (int sub = 0; sub < CB / 4; sub++)
                    small_compute<FMT, AR, CB, kSmMinMfma>(stage(parity), base + S::A, base + S::H, base + S::W,
                                                           lane & 31, acc, srcC, rwb.shift, kb, lane,
                                                           (CB / 4) * u + sub, ng, sub);
            }
#pragma unroll
            for (int i = 0; i < S::W_DMA; i++) asm volatile("" ::"v"(wo.v[i]));
        };
        for (int u = c0; u < c1; u += NST) {
            chunk(Parity<0>{}, u);
            chunk(Parity<1>{}, u + 1);
            if constexpr (NST > 2) chunk(Parity<2>{}, u + 2);
            if constexpr (NST > 3) chunk(Parity<3>{}, u + 3);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();   // every wave is done with both stages
    // partial sums [wave][register][lane] in stage 0
#pragma unroll
    for (int r = 0; r < 16; r++)
        if (r < 4 * ng) lds_at_store(lds0, 4 * ((wave * 16 + r) * 64 + lane), acc[r]);
    __syncthreads();
    if (wave >= ng) return;
    // wave w: register group w (output rows 8w + 4(l/32) + i), the slices
    // added in order
    float *out = reinterpret_cast<float *>(set.out[gi]);
    const int n = n0 + (lane & 31), g = lane >> 5;
    const bool split = gridDim.z > 1;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int r = 4 * wave + i;
        float v = lds_at<float>(lds0, 4 * (r * 64 + lane));
#pragma unroll
        for (int w = 1; w < kSmWaves; w++) v += lds_at<float>(lds0, 4 * ((w * 16 + r) * 64 + lane));
        const int m = 8 * wave + 4 * g + i;
        if (m < Mb && n < N) {
            if (split)
                unsafeAtomicAdd(out + int64_t(m0 + m) * N + n, v);
            else
                out[int64_t(m0 + m) * N + n] = v;
        }
    }
}

// Routing of the indexed MoE GEMM, one workgroup: count the routed rows of
// each expert, scan the counts into row and tile offsets, scatter the routed
// row ids into expert order and write the tile table (spare tiles: expert
// -1) and the table of small remainders.  Rows with an id outside [0, E) join no expert.  Within an expert the
// order of rows depends on atomic timing; the GEMM's result does not (every
// output row is computed on its own, in the same arithmetic wherever it sits).
//
// The kernel is latency-bound (16 K ids are 64 KiB): each thread loads its
// kRouteIds ids of a chunk with independent loads before it uses any, so a
// chunk costs one memory latency, and the scan runs in registers within each
// wave (row broadcasts by shuffle) with one LDS exchange of wave totals.
constexpr int kRouteThreads = 1024, kRouteWaves = kRouteThreads / 64, kRouteIds = 16;
static_assert(kMoeMaxExperts <= 2 * kRouteThreads, "each routing thread owns two experts");

// Ids of one chunk of routed rows (kRouteIds per thread, strided by the
// block size so that the loads coalesce); -1 past the end.
__device__ __forceinline__ void load_ids(const int32_t *__restrict__ ids, int R, int base, int *e) {
#pragma unroll
    for (int j = 0; j < kRouteIds; j++) {
        const int i = base + j * kRouteThreads + int(threadIdx.x);
        e[j] = i < R ? ids[i] : -1;
    }
}

__global__ __launch_bounds__(kRouteThreads) void k_moe_route(const int32_t *__restrict__ ids, int R, int E,
                                                             int max_tiles, int4 *__restrict__ header,
                                                             int4 *__restrict__ tiles, int4 *__restrict__ small,
                                                             int32_t *__restrict__ sorted) {
    __shared__ int cnt[kMoeMaxExperts];
    __shared__ int nsmall;
    __shared__ int cursor[kMoeMaxExperts];
    __shared__ int row_off[kMoeMaxExperts + 1];
    __shared__ int tile_off[kMoeMaxExperts + 1];
    __shared__ long long wave_sum[kRouteWaves];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    constexpr int kChunk = kRouteThreads * kRouteIds;
    // the first chunk's ids stay in registers for both passes (all of them
    // when R <= 16 Ki, the usual case); they are requested before anything
    // else so that their latency overlaps the clearing of the counters
    int e0[kRouteIds];
    load_ids(ids, R, 0, e0);
    for (int e = tid; e < E; e += kRouteThreads) cnt[e] = 0;
    if (tid == 0) nsmall = 0;
    __syncthreads();
    auto valid = [&](int e) { return e >= 0 && e < E; };
#pragma unroll
    for (int j = 0; j < kRouteIds; j++)
        if (valid(e0[j])) atomicAdd(&cnt[e0[j]], 1);
    for (int base = kChunk; base < R; base += kChunk) {
        int e[kRouteIds];
        load_ids(ids, R, base, e);
#pragma unroll
        for (int j = 0; j < kRouteIds; j++)
            if (valid(e[j])) atomicAdd(&cnt[e[j]], 1);
    }
    __syncthreads();
    // exclusive scan of (rows, row tiles) per expert, packed as rows + tiles
    // * 2^32 (rows <= R < 2^31, so the low half never carries); thread t owns
    // experts 2t and 2t + 1.  A last partial tile of at most kMoeSmallRows
    // rows is no row tile: it goes to the remainder table.
    long long own[2], v = 0;
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int e = 2 * tid + j;
        const int c = e < E ? cnt[e] : 0;
        const int nt = c / kTileM + (c % kTileM > kMoeSmallRows ? 1 : 0);
        own[j] = (long long)c + ((long long)nt << 32);
        v += own[j];
    }
    long long inc = v;   // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const long long a = __shfl_up(inc, off, 64);
        if (lane >= off) inc += a;
    }
    if (lane == 63) wave_sum[wv] = inc;
    __syncthreads();
    long long ex = inc - v;
    for (int w = 0; w < wv; w++) ex += wave_sum[w];
    int my_row[2], my_tile[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int e = 2 * tid + j;
        my_row[j] = int(ex & 0xffffffffLL);
        my_tile[j] = int(ex >> 32);
        if (e < E) {
            row_off[e] = my_row[j];
            tile_off[e] = my_tile[j];
            cursor[e] = my_row[j];
        }
        ex += own[j];
    }
    if (tid == kRouteThreads - 1) {   // ex is now the total over all experts
        row_off[E] = int(ex & 0xffffffffLL);
        tile_off[E] = int(ex >> 32);
    }
    // the tile table and the remainder list need only this thread's own
    // offsets and counts (the list's order follows the LDS atomics; each
    // entry is computed on its own, so the output does not depend on it)
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int e = 2 * tid + j;
        const int c = int(own[j] & 0xffffffffLL), nt = int(own[j] >> 32);
        if (e < E) {
            for (int t = 0; t < nt; t++)
                tiles[my_tile[j] + t] =
                    make_int4(e, my_row[j] + kTileM * t, my_row[j] + min(c, kTileM * (t + 1)), 0);
            const int rem = c - kTileM * nt;   // 0..kMoeSmallRows rows left over
            if (rem > 0) small[atomicAdd(&nsmall, 1)] = make_int4(e, my_row[j] + c - rem, my_row[j] + c, 0);
        }
    }
    __syncthreads();
    for (int t = tile_off[E] + tid; t < max_tiles; t += kRouteThreads) tiles[t] = make_int4(-1, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < kRouteIds; j++)
        if (valid(e0[j])) sorted[atomicAdd(&cursor[e0[j]], 1)] = j * kRouteThreads + tid;
    for (int base = kChunk; base < R; base += kChunk) {
        int e[kRouteIds];
        load_ids(ids, R, base, e);
#pragma unroll
        for (int j = 0; j < kRouteIds; j++)
            if (valid(e[j])) sorted[atomicAdd(&cursor[e[j]], 1)] = base + j * kRouteThreads + tid;
    }
    // last: the header, with the number of row tiles the table fills and
    // the number of small remainders listed
    if (tid == 0) {
        header[1] = make_int4(nsmall, 0, 0, 0);
        header[0] = make_int4(kMoeMagic, R, E, tile_off[E]);
    }
}

// Zero an fp32 array (the output of a split-K launch, before the slices add
// into it; or, as 32-bit words, the arrival counters of a split through a
// workspace).  A kernel rather than a memset node, so that the launch
// sequence stays capturable as plain kernels.
__global__ __launch_bounds__(256) void k_zero_fill(float *__restrict__ p, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) p[i] = 0.0f;
}

// The same for the M x N[g] outputs of every GEMM of a set, in one launch
// (grid y = the set's members): a launch per member costs more than the
// zeroing itself on the short launches of decode-sized sets.
__global__ __launch_bounds__(256) void k_zero_fill_set(const GemmSet set, int64_t M) {
    const int g = int(blockIdx.y);
    float *__restrict__ p = reinterpret_cast<float *>(set.out[g]);
    const int64_t n = M * set.N[g];
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) p[i] = 0.0f;
}

// ---------------------------------------------------------------------------
// Tile-packed Q8_0 weights (mmq_pack_q8_0): a permutation of the Q8_0 bytes
// into the order the tile kernel stages them, kPackImg bytes per 128-column
// tile and k-step (layout at kPackCodes).  One thread per output dword; a
// Q8_0 block is 17 16-bit units (the scale, then the codes), so the dword's
// four code bytes, or its two scales, are read as 16-bit values.  Columns
// past N and blocks past K/32 are written as zero.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pack_q8_0(const uint16_t *__restrict__ w, int N, int kb, int nsteps,
                                                   uint32_t *__restrict__ packed, int64_t ndw) {
    constexpr int kImgDw = int(kPackImg / 4), kCodeDw = int(kPackCodes / 4), kBlockDw = kBlockBytes / 4;
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t d = int64_t(blockIdx.x) * 256 + threadIdx.x; d < ndw; d += stride) {
        const int64_t img = d / kImgDw;   // image = (column tile, k-step)
        const int o = int(d - img * kImgDw);
        const int t = int(img / nsteps), s = int(img - int64_t(t) * nsteps);
        uint32_t v = 0;
        if (o < kCodeDw) {
            // the inverse of code_off: block b, column col, stored half, dword i of the half
            const int b = o / kBlockDw, r = o - b * kBlockDw;
            const int col = r >> 3, half = ((r >> 2) & 1) ^ half_swz(col);
            const int byte0 = 16 * half + 4 * (r & 3);
            const int n = t * kTileN + col, blk = s * KB + b;
            if (n < N && blk < kb) {
                const int64_t h = (int64_t(n) * kb + blk) * 17 + 1 + byte0 / 2;
                v = uint32_t(w[h]) | (uint32_t(w[h + 1]) << 16);
            }
        } else {
            // scales [block][column], two per dword
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int u = 2 * (o - kCodeDw) + j, b = u / kTileN, col = u - b * kTileN;
                const int n = t * kTileN + col, blk = s * KB + b;
                if (n < N && blk < kb) v |= uint32_t(w[(int64_t(n) * kb + blk) * 17]) << (16 * j);
            }
        }
        packed[d] = v;
    }
}

hipError_t launch_pack_q8_0(const void *w, int64_t N, int64_t K, void *packed, int cu_count, hipStream_t stream) {
    const int kb = int(K / 32), nsteps = (kb + KB - 1) / KB;
    const int64_t ndw = packed_bytes_q8_0(N, K) / 4;
    int64_t grid = (ndw + 255) / 256;
    if (grid > int64_t(cu_count) * 32) grid = int64_t(cu_count) * 32;   // the kernel strides over the rest
    hipLaunchKernelGGL(k_pack_q8_0, dim3((unsigned)grid), dim3(256), 0, stream, reinterpret_cast<const uint16_t *>(w),
                       int(N), kb, nsteps, reinterpret_cast<uint32_t *>(packed), ndw);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free MoE entry point: the routing tables of one
// call (header, tile table, sorted routed-row ids: kNoAllocScratchBytes for
// up to kNoAllocMaxRouted routed rows and kMoeMaxExperts experts) in a
// file-scope device array instead of a caller workspace.  Each device holds
// its own copy for the life of the process; every call on a device shares
// it, so calls that overlap in time on one device race.  The routing kernel
// rewrites everything the GEMM reads (header last) on every call, so
// nothing needs clearing between calls.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
static_assert(kNoAllocScratchBytes % 16 == 0, "the tables are read as 16-byte units");

// The device address of this device's copy of `scratch`, looked up once per
// device with that device current (in host code the array's name is only a
// stand-in for the symbol, never a device address).
hipError_t noalloc_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static void *addr[kMaxDevices] = {};
    static std::mutex mu;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// Host-side launchers (declared in mmq_launch.hpp).
hipError_t launch_quantize(const float *x, void *y, int64_t M, int64_t K, int cu_count,
                           hipStream_t stream) {
    (void)cu_count;
    const int64_t nblocks = M * (K / 32);
    int64_t grid = (nblocks + kQuantBlocksPerWg - 1) / kQuantBlocksPerWg;
    if (grid > (int64_t(1) << 30)) grid = int64_t(1) << 30;   // the kernel strides over the rest
    hipLaunchKernelGGL(k_quantize_q8_1, dim3((unsigned)grid), dim3(256), 0, stream, x,
                       reinterpret_cast<uint32_t *>(y), nblocks);
    return hipGetLastError();
}

static hipError_t launch_mv(const Plan &p, const GemmSet &set, const uint8_t *xb, int64_t M, int64_t K,
                            hipStream_t stream) {
    const dim3 grid((unsigned)p.grid_x), block(kMvThreads);
    static_assert(kMvMaxM == 8, "the matvec launches below cover M = 1, 2, 3-4, 5-8");
    if (p.mv_mfma) {
        if (p.fmt == FMT_Q4_K)
            hipLaunchKernelGGL((k_mmvq<FMT_Q4_K>), grid, block, 0, stream, xb, set, int(M), int(K));
        else if (p.fmt == FMT_Q5_K)
            hipLaunchKernelGGL((k_mmvq<FMT_Q5_K>), grid, block, 0, stream, xb, set, int(M), int(K));
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    auto go = [&](auto mr) {
        constexpr int MR = decltype(mr)::value;
        if (p.fmt == FMT_Q8_0)
            hipLaunchKernelGGL((k_mmv<FMT_Q8_0, MR>), grid, block, 0, stream, xb, set, int(M), int(K));
        else if (p.fmt == FMT_Q4_K)
            hipLaunchKernelGGL((k_mmv<FMT_Q4_K, MR>), grid, block, 0, stream, xb, set, int(M), int(K));
        else if (p.fmt == FMT_Q5_K)
            hipLaunchKernelGGL((k_mmv<FMT_Q5_K, MR>), grid, block, 0, stream, xb, set, int(M), int(K));
        else
            hipLaunchKernelGGL((k_mmv<FMT_Q6_K, MR>), grid, block, 0, stream, xb, set, int(M), int(K));
    };
    if (M == 1)
        go(std::integral_constant<int, 1>{});
    else if (M == 2)
        go(std::integral_constant<int, 2>{});
    else if (M <= 4)
        go(std::integral_constant<int, 4>{});
    else
        go(std::integral_constant<int, 8>{});
    return hipGetLastError();
}

// The kernel a plan launches: launch_gemm and launch_moe below launch
// exactly this one, and the capacity guard reads its attributes.
template <int F, bool DOTS, bool MOE, bool SKIP, bool TAIL, bool PK = false>
static const void *kmmq() {
    return reinterpret_cast<const void *>(&k_mmq<F, DOTS, MOE, SKIP, TAIL, PK>);
}

const void *plan_kernel(const Plan &p, bool dots, bool moe) {
    auto pick = [&](auto fmt) -> const void * {
        constexpr int F = decltype(fmt)::value;
        if (p.kernel == KERNEL_MV) {
            if constexpr (F == FMT_Q4_K || F == FMT_Q5_K)
                if (p.mv_mfma) return reinterpret_cast<const void *>(&k_mmvq<F>);
            if (p.tile_m == 1) return reinterpret_cast<const void *>(&k_mmv<F, 1>);
            if (p.tile_m == 2) return reinterpret_cast<const void *>(&k_mmv<F, 2>);
            if (p.tile_m <= 4) return reinterpret_cast<const void *>(&k_mmv<F, 4>);
            return reinterpret_cast<const void *>(&k_mmv<F, 8>);
        }
        if (p.kernel == KERNEL_SM && !dots)
            return p.tile_m == 16 ? reinterpret_cast<const void *>(&k_mmsm<F, 16>)
                                  : reinterpret_cast<const void *>(&k_mmsm<F, 32>);
        if (dots) return kmmq<F, true, false, false, false>();   // partial steps: the store mask
        if constexpr (F == FMT_Q8_0) {
            if (p.packed) {
                if (p.skip_idle_waves)
                    return p.tail ? kmmq<F, false, false, true, true, true>() : kmmq<F, false, false, true, false, true>();
                return p.tail ? kmmq<F, false, false, false, true, true>() : kmmq<F, false, false, false, false, true>();
            }
            if (moe) return p.tail ? kmmq<F, false, true, true, true>() : kmmq<F, false, true, true, false>();
            if (p.skip_idle_waves)
                return p.tail ? kmmq<F, false, false, true, true>() : kmmq<F, false, false, true, false>();
            return p.tail ? kmmq<F, false, false, false, true>() : kmmq<F, false, false, false, false>();
        } else {
            if (moe) return kmmq<F, false, true, true, false>();
            return p.skip_idle_waves ? kmmq<F, false, false, true, false>() : kmmq<F, false, false, false, false>();
        }
    };
    if (p.fmt == FMT_Q8_0) return pick(std::integral_constant<int, FMT_Q8_0>{});
    if (p.fmt == FMT_Q4_K) return pick(std::integral_constant<int, FMT_Q4_K>{});
    if (p.fmt == FMT_Q5_K) return pick(std::integral_constant<int, FMT_Q5_K>{});
    return pick(std::integral_constant<int, FMT_Q6_K>{});
}

// The small-remainder kernel of the indexed MoE for a weight format.
const void *small_kernel(int fmt) {
    if (fmt == FMT_Q8_0) return reinterpret_cast<const void *>(&k_moe_small<FMT_Q8_0>);
    if (fmt == FMT_Q4_K) return reinterpret_cast<const void *>(&k_moe_small<FMT_Q4_K>);
    if (fmt == FMT_Q5_K) return reinterpret_cast<const void *>(&k_moe_small<FMT_Q5_K>);
    return reinterpret_cast<const void *>(&k_moe_small<FMT_Q6_K>);
}

hipError_t launch_gemm(const Plan &p, const int *tile_start, int count, const void *x, const void *const *w,
                       void *const *out, const int64_t *N, int64_t M, int64_t K, bool dots, void *workspace,
                       hipStream_t stream) {
    GemmSet set{};
    set.count = count;
    for (int g = 0; g < count; g++) {
        set.tile_start[g] = tile_start[g];
        set.N[g] = int(N[g]);
        set.w[g] = reinterpret_cast<const uint8_t *>(w[g]);
        set.out[g] = out[g];
    }
    for (int g = count; g <= kMaxGemms; g++) set.tile_start[g] = tile_start[count];   // set_member, set_total
    if (p.kernel == KERNEL_MV) return launch_mv(p, set, reinterpret_cast<const uint8_t *>(x), M, K, stream);
    set.part = nullptr;
    set.cnt = nullptr;
    if (p.split_k > 1 && !dots && p.split_ws) {
        // the arrival counters start at zero (a kernel, not a memset: the
        // launch may be captured into a graph)
        set.cnt = reinterpret_cast<uint32_t *>(workspace);
        set.part = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(workspace) + split_counter_bytes(p));
        const int64_t words = split_counter_bytes(p) / 4;
        hipLaunchKernelGGL(k_zero_fill, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                           reinterpret_cast<float *>(workspace), words);
    } else if (p.split_k > 1 && !dots) {
        int64_t nmax = 0;
        for (int g = 0; g < count; g++) nmax = std::max<int64_t>(nmax, M * N[g]);
        const int64_t blocks = std::min<int64_t>((nmax + 255) / 256, 8192);
        hipLaunchKernelGGL(k_zero_fill_set, dim3((unsigned)blocks, (unsigned)count), dim3(256), 0, stream, set, M);
    }
    const dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y, (unsigned)p.split_k);
    const dim3 block(p.threads);
    // the kernel the plan names (the one whose attributes the guard read);
    // its LDS is static (checked by the plan)
    const uint8_t *xb = reinterpret_cast<const uint8_t *>(x);
    int Mi = int(M), Ki = int(K), sps = int(p.steps_per_split);
    MoeArgs noMoe{};
    void *args[] = {&xb, &set, &Mi, &Ki, &sps, &noMoe};
    void *sm_args[] = {&xb, &set, &Mi, &Ki};
    const hipError_t e = hipLaunchKernel(plan_kernel(p, dots, false), grid, block,
                                         p.kernel == KERNEL_SM ? sm_args : args, 0, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

hipError_t launch_moe(const Plan &p, const void *x, const void *w, const int32_t *ids, int topk, int n_experts,
                      float *out, int64_t T, int64_t N, int64_t K, void *workspace, hipStream_t stream) {
    const int64_t R = T * topk;
    const int max_tiles = int(p.grid_y);
    int4 *header = reinterpret_cast<int4 *>(workspace);
    int4 *tiles = reinterpret_cast<int4 *>(reinterpret_cast<uint8_t *>(workspace) + kMoeHeaderBytes);
    int4 *small = reinterpret_cast<int4 *>(reinterpret_cast<uint8_t *>(tiles) + 16 * int64_t(max_tiles));
    int32_t *sorted = reinterpret_cast<int32_t *>(reinterpret_cast<uint8_t *>(small) + moe_small_table_bytes(n_experts));
    if (ids)   // else: the tables a previous launch left in the workspace
        hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(kRouteThreads), 0, stream, ids, int(R), n_experts, max_tiles,
                           header, tiles, small, sorted);
    GemmSet set{};
    set.count = 1;
    set.tile_start[0] = 0;
    for (int g = 1; g <= kMaxGemms; g++) set.tile_start[g] = int(p.grid_x);   // set_member, set_total
    set.N[0] = int(N);
    set.w[0] = reinterpret_cast<const uint8_t *>(w);
    set.out[0] = out;
    set.part = nullptr;
    set.cnt = nullptr;
    MoeArgs moe;
    moe.header = header;
    moe.tiles = tiles;
    moe.small = small;
    moe.sorted = sorted;
    moe.topk = topk;
    moe.R = int(R);
    moe.E = n_experts;
    moe.expert_bytes = N * weight_row_bytes(p.fmt, K);
    const dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y, 1);
    const dim3 block(p.threads);
    const uint8_t *xb = reinterpret_cast<const uint8_t *>(x);
    int Ti = int(T), Ki = int(K), sps = int(p.steps_per_split);
    void *args[] = {&xb, &set, &Ti, &Ki, &sps, &moe};
    hipError_t e = hipLaunchKernel(plan_kernel(p, false, true), grid, block, args, 0, stream);
    if (e != hipSuccess) return e;
    // the small remainders: every expert may hold one
    const dim3 sgrid((unsigned)((N + kSmallRowsPerWg - 1) / kSmallRowsPerWg), (unsigned)n_experts, 1);
    const uint8_t *wb = reinterpret_cast<const uint8_t *>(w);
    int Ni = int(N);
    void *sargs[] = {&xb, &wb, &out, &Ti, &Ni, &Ki, &moe};
    e = hipLaunchKernel(small_kernel(p.fmt), sgrid, dim3(kSmallThreads), sargs, 0, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace mmq
