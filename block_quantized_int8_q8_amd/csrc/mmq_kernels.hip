// mmq_kernels.hip -- gfx950 kernels of the block-quantized int8 MMQ library.
//
//   k_quantize_q8_1   fp32 -> q8_1, one pass over the activations (HBM-bound)
//   k_mmq<FMT, DOTS>  q8_1 x {Q8_0, Q4_K} -> fp32 (or the raw int32 block
//                     dots when DOTS), int8 MFMA with the per-block scale
//                     applied in registers on the MFMA accumulator layout.
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

#include "mmq_plan.hpp"

namespace mmq {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return __half2float(__ushort_as_half((unsigned short)(bits16 & 0xffffu)));
}

// ---------------------------------------------------------------------------
// Quantize: fp32 -> q8_1 ("13 . r7-r8 raw-byte MMQ kernel", section 3.2).
//
// Eight lanes share one 32-value block, four values (one 16-byte load) each,
// so a wave64 reads 1 KiB of contiguous activations per instruction and
// writes 8 x 36 contiguous bytes.  amax and the code sum are reduced across
// the eight lanes with xor-shuffles; max is exact in any association order
// (same page, section 3.1) so the tree reduction cannot change d.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quantize_q8_1(const float *__restrict__ x,
                                                       uint32_t *__restrict__ y, int64_t nblocks) {
    const int sub = threadIdx.x & 7;
    const int64_t first = int64_t(blockIdx.x) * (blockDim.x >> 3) + (threadIdx.x >> 3);
    const int64_t step = int64_t(gridDim.x) * (blockDim.x >> 3);
    for (int64_t blk = first; blk < nblocks; blk += step) {
        const float4 v = reinterpret_cast<const float4 *>(x)[blk * 8 + sub];
        float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        am = fmaxf(am, __shfl_xor(am, 1, 8));
        am = fmaxf(am, __shfl_xor(am, 2, 8));
        am = fmaxf(am, __shfl_xor(am, 4, 8));
        const float d = am / 127.0f;                    // correctly rounded fp32 divide
        // id = 1/d; a zero block, or one so small that 1/d overflows fp32,
        // quantizes to all-zero codes (its fp16 scale is 0 as well)
        float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        if (__builtin_isinf(id)) id = 0.0f;
        // round half away from zero (roundf), then clamp to the symmetric range
        int q0 = (int)roundf(v.x * id), q1 = (int)roundf(v.y * id);
        int q2 = (int)roundf(v.z * id), q3 = (int)roundf(v.w * id);
        q0 = min(127, max(-127, q0));
        q1 = min(127, max(-127, q1));
        q2 = min(127, max(-127, q2));
        q3 = min(127, max(-127, q3));
        const uint32_t packed = (uint32_t(q0) & 0xffu) | ((uint32_t(q1) & 0xffu) << 8) |
                                ((uint32_t(q2) & 0xffu) << 16) | ((uint32_t(q3) & 0xffu) << 24);
        int s = q0 + q1 + q2 + q3;
        s += __shfl_xor(s, 1, 8);
        s += __shfl_xor(s, 2, 8);
        s += __shfl_xor(s, 4, 8);
        uint32_t *yb = y + blk * 9;                     // 36 bytes = 9 dwords per block
        yb[1 + sub] = packed;
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
// Workgroup: 256 threads (4 wave64s) compute a 128 x 128 output tile; wave w
// owns rows 32w..32w+31 and all 128 columns as four 32x32 sub-tiles.  Each
// k-step stages 4 consecutive 32-blocks (half a Q4_K super-block) into LDS;
// a step's LDS (36-44 KiB) lets three or four workgroups share a CU, so that
// every SIMD has several waves to switch between while one waits on LDS,
// the matrix core or a barrier.
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
//         scale of the element's row, fp16 widened exactly inside the FMA)
// For Q8_0 this is the same arithmetic, in the same block order, as the
// oracle, so the output is bit-identical.
//
// Q4_K ("When Does a Kernel Win Surface?", 6.2): ws = d*sc_j (exact in fp32);
// the packed 4-bit codes are unpacked once per workgroup while staging (low
// nibbles = even sub-block, high nibbles = odd sub-block of a 32-byte
// group); and the min term  -sum_j dmin*m_j * s_j  of a whole super-block is
// added by one fp16 MFMA per 32x32 sub-tile that accumulates straight into
// the fp32 accumulator: A = the eight activation block sums s_j (fp16, as
// stored), B = -dmin*m_j split exactly into an fp16 high and low part
// (k = 0..7 high parts, k = 8..15 low parts, each multiplied by the same s_j).
// ---------------------------------------------------------------------------
constexpr uint32_t kMagicBits = 0x4B400000u;   // 12582912.0f
constexpr float kMagic = 12582912.0f;
constexpr int KB = kBlocksPerStage;            // 32-blocks per k-step

// LDS layouts.  Codes (activations, and weights of either format once
// unpacked to one int8 code per byte) are row-major, 128 bytes per row = 8
// chunks of 16 bytes (block b of the step, k-half g -> chunk 2b+g), with the
// chunk index XOR-swizzled by row%8.  A fragment read (32 consecutive rows,
// one chunk) then touches eight distinct 16-byte bank groups per 8-lane
// phase, and staging writes are at worst 2-way conflicted, with no padding.
//
// Activation scales stay fp16 as stored in q8_1 and are consumed by
// v_fma_mix_f32 (exact widening inside the FMA).  They are kept per block in
// accumulator-fragment order: within each 32-row group, lane half g needs the
// scales of rows 8q + 4g + i (q, i = 0..3) for its registers r = 4q + i, so
// position 16g + 4q + i holds row 8q + 4g + i and a lane reads its 16 scales
// as two contiguous 16-byte words.  Planes are 272 bytes apart (16-byte
// aligned, 4 banks apart).  Weight scales are fp32 [block][column] planes of
// 132 floats (staging writes of one column's blocks land on distinct banks);
// Q4_K keeps all eight planes of a super-block, written at its first step.
constexpr int kRowBytes = KB * 32;   // codes per row per step
constexpr int kPlaneH = 136;         // halves per activation-scale plane
constexpr int kPlane = 132;          // floats per weight-scale plane

__device__ __forceinline__ int chunk_off(int row, int j) { return row * kRowBytes + ((j ^ (row & 7)) << 4); }
__device__ __forceinline__ int xs_pos(int row) {
    return (row & ~31) + (((row >> 2) & 1) << 4) + (((row >> 3) & 3) << 2) + (row & 3);
}

template <int FMT>
struct Lds {
    static constexpr int A_CODES = kTileM * kRowBytes;
    static constexpr int A_SCALE = KB * kPlaneH * 2;
    static constexpr int B_CODES = kTileN * kRowBytes;
    static constexpr int B_SCALE = (FMT == FMT_Q8_0 ? KB : 8) * kPlane * 4;
    static constexpr int B_MIN = (FMT == FMT_Q4_K) ? kTileN * 2 * 8 * 2 : 0;   // [col][g][8] fp16
    static constexpr int A_SUM = (FMT == FMT_Q4_K) ? kTileM * 8 * 2 : 0;       // [row][8] fp16
    static constexpr int OFF_A_SCALE = A_CODES;
    static constexpr int OFF_B_CODES = OFF_A_SCALE + A_SCALE;
    static constexpr int OFF_B_SCALE = OFF_B_CODES + B_CODES;
    static constexpr int OFF_B_MIN = OFF_B_SCALE + B_SCALE;
    static constexpr int OFF_A_SUM = OFF_B_MIN + B_MIN;
    static constexpr int TOTAL = OFF_A_SUM + A_SUM;
};
static_assert(KB == 4, "the staging maps below assume 4 blocks per k-step");
static_assert(Lds<FMT_Q8_0>::TOTAL == lds_bytes_for(FMT_Q8_0), "plan and kernel LDS disagree");
static_assert(Lds<FMT_Q4_K>::TOTAL == lds_bytes_for(FMT_Q4_K), "plan and kernel LDS disagree");
static_assert(Lds<FMT_Q4_K>::OFF_B_CODES % 16 == 0 && Lds<FMT_Q4_K>::OFF_B_MIN % 16 == 0 &&
              Lds<FMT_Q4_K>::OFF_A_SUM % 16 == 0 && Lds<FMT_Q8_0>::OFF_B_SCALE % 16 == 0,
              "LDS regions must stay 16-byte aligned");

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// A raw buffer over the rows of one tile: reads past `bytes` return zero in
// hardware, which is how rows beyond M or N are zero-filled (codes 0,
// scales 0: they add nothing and are never stored) without a single VALU
// instruction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t *base, int64_t bytes) {
    const int n = bytes > 0x7fffffffLL ? 0x7fffffff : int(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, n, 0x00020000);
}

// Staging is split into a load half (global memory -> registers, issued one
// k-step ahead so that its latency hides behind the current step's MFMAs)
// and a store half (registers -> LDS after the step's barrier).

// Activations: unit u -> (row = u/4, block = u%4): four consecutive threads
// read one row's 144 contiguous bytes of this step.
struct ActRegs {
    uint32_t w0[2];
    u32x4 lo[2], hi[2];
};

__device__ __forceinline__ void load_activations(__amdgpu_buffer_rsrc_t rx, int kb, int ks, int tid,
                                                 ActRegs &r) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int u = tid + kThreads * i;
        const int row = u >> 2, b = u & 3;
        const int off = (row * kb + ks * KB + b) * 36;
        r.w0[i] = __builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 0);
        r.lo[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, off + 4, 0, 0);
        r.hi[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, off + 20, 0, 0);
    }
}

template <int FMT>
__device__ __forceinline__ void store_activations(const ActRegs &r, uint8_t *smem, int ks, int tid) {
    using L = Lds<FMT>;
    unsigned short *sXh = reinterpret_cast<unsigned short *>(smem + L::OFF_A_SCALE);
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int u = tid + kThreads * i;
        const int row = u >> 2, b = u & 3;
        *reinterpret_cast<u32x4 *>(smem + chunk_off(row, 2 * b)) = r.lo[i];
        *reinterpret_cast<u32x4 *>(smem + chunk_off(row, 2 * b + 1)) = r.hi[i];
        sXh[b * kPlaneH + xs_pos(row)] = (unsigned short)(r.w0[i] & 0xffffu);
        if constexpr (FMT == FMT_Q4_K) {
            unsigned short *sSum = reinterpret_cast<unsigned short *>(smem + L::OFF_A_SUM);
            sSum[row * 8 + (ks & 1) * KB + b] = (unsigned short)(r.w0[i] >> 16);   // sub-block of its super-block
        }
    }
}

// Q8_0: thread -> (row = tid/2, block pair p = tid%2).  A pair of 34-byte
// blocks is 68 bytes = 17 dwords starting on a 4-byte boundary (K % 256 == 0
// makes every row an even number of blocks); the even block's codes sit two
// bytes off the dword grid and are realigned with v_alignbyte.
struct Q80Regs {
    u32x4 v[4];
    uint32_t last;
};

__device__ __forceinline__ void load_q8_0(__amdgpu_buffer_rsrc_t rw, int kb, int ks, int tid, Q80Regs &r) {
    const int row = tid >> 1, p = tid & 1;
    const int off = (row * kb + ks * KB + 2 * p) * 34;
#pragma unroll
    for (int q = 0; q < 4; q++) r.v[q] = __builtin_amdgcn_raw_buffer_load_b128(rw, off + 16 * q, 0, 0);
    r.last = __builtin_amdgcn_raw_buffer_load_b32(rw, off + 64, 0, 0);
}

__device__ __forceinline__ void store_q8_0(const Q80Regs &r, uint8_t *smem, int tid) {
    using L = Lds<FMT_Q8_0>;
    uint8_t *sB = smem + L::OFF_B_CODES;
    float *sWd = reinterpret_cast<float *>(smem + L::OFF_B_SCALE);
    const int row = tid >> 1, p = tid & 1;
    const uint32_t w[17] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w, r.v[1].x, r.v[1].y,
                            r.v[1].z, r.v[1].w, r.v[2].x, r.v[2].y, r.v[2].z, r.v[2].w,
                            r.v[3].x, r.v[3].y, r.v[3].z, r.v[3].w, r.last};
    u32x4 c0, c1;
    c0.x = __builtin_amdgcn_alignbyte(w[1], w[0], 2);
    c0.y = __builtin_amdgcn_alignbyte(w[2], w[1], 2);
    c0.z = __builtin_amdgcn_alignbyte(w[3], w[2], 2);
    c0.w = __builtin_amdgcn_alignbyte(w[4], w[3], 2);
    c1.x = __builtin_amdgcn_alignbyte(w[5], w[4], 2);
    c1.y = __builtin_amdgcn_alignbyte(w[6], w[5], 2);
    c1.z = __builtin_amdgcn_alignbyte(w[7], w[6], 2);
    c1.w = __builtin_amdgcn_alignbyte(w[8], w[7], 2);
    *reinterpret_cast<u32x4 *>(sB + chunk_off(row, 4 * p + 0)) = c0;
    *reinterpret_cast<u32x4 *>(sB + chunk_off(row, 4 * p + 1)) = c1;
    *reinterpret_cast<u32x4 *>(sB + chunk_off(row, 4 * p + 2)) = u32x4{w[9], w[10], w[11], w[12]};
    *reinterpret_cast<u32x4 *>(sB + chunk_off(row, 4 * p + 3)) = u32x4{w[13], w[14], w[15], w[16]};
    sWd[(2 * p) * kPlane + row] = h2f(w[0]);
    sWd[(2 * p + 1) * kPlane + row] = h2f(w[8] >> 16);
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
// low parts.
template <int J>
__device__ __forceinline__ void q4k_subblock(const u32x4 &h, float d, float dmin, int row, float *sWd,
                                             _Float16 *sMin) {
    uint32_t sc, mn;
    if constexpr (J < 4) {
        sc = sbyte<J>(h) & 63u;
        mn = sbyte<J + 4>(h) & 63u;
    } else {
        sc = (sbyte<J + 4>(h) & 15u) | ((sbyte<J - 4>(h) >> 6) << 4);
        mn = (sbyte<J + 4>(h) >> 4) | ((sbyte<J>(h) >> 6) << 4);
    }
    sWd[J * kPlane + row] = d * (float)sc;                 // exact: 11 x 6 bits
    const float neg = -(dmin * (float)mn);                  // exact
    const _Float16 hi = (_Float16)neg;
    const _Float16 lo = (_Float16)(neg - (float)hi);        // exact remainder
    sMin[(row * 2 + 0) * 8 + J] = hi;
    sMin[(row * 2 + 1) * 8 + J] = lo;
}

// Q4_K, half `ks & 1` of super-block `ks / 2`, for the tile's 128 columns.
// Unit u -> (row = u/4, packed chunk c = 4*half + u%4): the 16 code bytes
// 16c..16c+15 belong to 32-byte group c/2 and k-half c%2; their low nibbles
// are codes of sub-block 2*(c/2), their high nibbles of sub-block 2*(c/2)+1
// (the layout reading in the header).  They are unpacked at store time, once
// per workgroup, into the same one-code-per-byte layout as Q8_0, so the MFMA
// loop reads both formats alike.  At the first half the header is decoded
// too: waves 0-1 turn sub-blocks 0..3 of row tid%128 into d*sc_j and the
// split min operand, waves 2-3 sub-blocks 4..7 (a wave-uniform branch; every
// sub-block index a compile-time constant).
struct Q4KRegs {
    u32x4 v[2];
    u32x4 h;
};

__device__ __forceinline__ void load_q4_K(__amdgpu_buffer_rsrc_t rw, int nsb, int ks, int tid, Q4KRegs &r) {
    const int sb = ks >> 1, half = ks & 1;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int u = tid + kThreads * i;
        const int row = u >> 2, c = 4 * half + (u & 3);
        r.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, (row * nsb + sb) * 144 + 16 + 16 * c, 0, 0);
    }
    if (half == 0)
        r.h = __builtin_amdgcn_raw_buffer_load_b128(rw, ((tid & (kTileN - 1)) * nsb + sb) * 144, 0, 0);
}

__device__ __forceinline__ void store_q4_K(const Q4KRegs &r, uint8_t *smem, int ks, int tid) {
    using L = Lds<FMT_Q4_K>;
    uint8_t *sB = smem + L::OFF_B_CODES;
    float *sWd = reinterpret_cast<float *>(smem + L::OFF_B_SCALE);
    _Float16 *sMin = reinterpret_cast<_Float16 *>(smem + L::OFF_B_MIN);
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int u = tid + kThreads * i;
        const int row = u >> 2, cl = u & 3;          // cl: chunk within this half
        const u32x4 lo = r.v[i] & 0x0F0F0F0Fu;
        const u32x4 hi = (r.v[i] >> 4) & 0x0F0F0F0Fu;
        // sub-blocks 2*(c/2) and 2*(c/2)+1 are blocks 2*(cl/2) and 2*(cl/2)+1 of this step
        const int gl = cl >> 1, kh = cl & 1;
        *reinterpret_cast<u32x4 *>(sB + chunk_off(row, 4 * gl + kh)) = lo;
        *reinterpret_cast<u32x4 *>(sB + chunk_off(row, 4 * gl + 2 + kh)) = hi;
    }
    if ((ks & 1) == 0) {
        const int row = tid & (kTileN - 1);
        const float d = h2f(r.h.x), dmin = h2f(r.h.x >> 16);
        if (tid < kTileN) {
            q4k_subblock<0>(r.h, d, dmin, row, sWd, sMin);
            q4k_subblock<1>(r.h, d, dmin, row, sWd, sMin);
            q4k_subblock<2>(r.h, d, dmin, row, sWd, sMin);
            q4k_subblock<3>(r.h, d, dmin, row, sWd, sMin);
        } else {
            q4k_subblock<4>(r.h, d, dmin, row, sWd, sMin);
            q4k_subblock<5>(r.h, d, dmin, row, sWd, sMin);
            q4k_subblock<6>(r.h, d, dmin, row, sWd, sMin);
            q4k_subblock<7>(r.h, d, dmin, row, sWd, sMin);
        }
    }
}

template <int FMT>
struct WRegs;
template <>
struct WRegs<FMT_Q8_0> { Q80Regs r; };
template <>
struct WRegs<FMT_Q4_K> { Q4KRegs r; };

template <int FMT, bool DOTS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(DOTS ? 1 : (FMT == FMT_Q8_0 ? 2 : 3))))
void k_mmq(const uint8_t *__restrict__ xq, const uint8_t *__restrict__ wq, void *__restrict__ outp,
           int M, int N, int K) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using L = Lds<FMT>;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int n0 = blockIdx.x * kTileN, m0 = blockIdx.y * kTileM;
    const int kb = K >> 5, nsteps = kb / KB;

    const _Float16 *sXh = reinterpret_cast<const _Float16 *>(smem + L::OFF_A_SCALE);
    const uint8_t *sB = smem + L::OFF_B_CODES;
    const float *sWd = reinterpret_cast<const float *>(smem + L::OFF_B_SCALE);

    // Buffers over this tile's rows of x and w (reads past M / N return 0).
    const int64_t xrow = int64_t(kb) * 36;
    const int64_t wrow = FMT == FMT_Q8_0 ? int64_t(kb) * 34 : int64_t(K >> 8) * 144;
    const __amdgpu_buffer_rsrc_t rx = tile_rsrc(xq + int64_t(m0) * xrow, int64_t(M - m0) * xrow);
    const __amdgpu_buffer_rsrc_t rw = tile_rsrc(wq + int64_t(n0) * wrow, int64_t(N - n0) * wrow);

    const int a_row = (32 * wv + l32) * kRowBytes;   // this lane's A row (fragment row l32 of wave wv)
    const int b_row = l32 * kRowBytes;                // this lane's B column within a 32-column sub-tile

    i32x16 srcC;
#pragma unroll
    for (int r = 0; r < 16; r++) srcC[r] = DOTS ? 0 : int(kMagicBits);

    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; c++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[c][r] = 0.0f;

    // Q8_0 software-pipelines its staging (the registers hold step ks+1 while
    // step ks computes); Q4_K, held to 168 VGPRs for three waves per SIMD,
    // has no room for the prefetch registers and loads each step just before
    // storing it.
    constexpr bool kPrefetch = FMT == FMT_Q8_0;
    ActRegs ar;
    WRegs<FMT> wr;
    auto load_step = [&](int k) {
        load_activations(rx, kb, k, tid, ar);
        if constexpr (FMT == FMT_Q8_0)
            load_q8_0(rw, kb, k, tid, wr.r);
        else
            load_q4_K(rw, K >> 8, k, tid, wr.r);
    };
    if constexpr (kPrefetch) load_step(0);

    for (int ks = 0; ks < nsteps; ks++) {
        if constexpr (!kPrefetch) load_step(ks);
        store_activations<FMT>(ar, smem, ks, tid);
        if constexpr (FMT == FMT_Q8_0)
            store_q8_0(wr.r, smem, tid);
        else
            store_q4_K(wr.r, smem, ks, tid);
        __syncthreads();
        if (kPrefetch && ks + 1 < nsteps) load_step(ks + 1);

        // Q4_K weight-scale planes hold the whole super-block: this step's
        // blocks are sub-blocks 4*(ks&1) .. 4*(ks&1)+3
        const int wplane = FMT == FMT_Q8_0 ? 0 : (ks & 1) * KB;
#pragma unroll
        for (int b = 0; b < KB; b++) {
            // swizzled chunk of (block b, k-half g) for this lane's rows and
            // columns: all of them are == l32 (mod 8)
            const int sw = ((2 * b + g) ^ (l32 & 7)) << 4;
            const i32x4 a = *reinterpret_cast<const i32x4 *>(smem + a_row + sw);
            f16x8 xs0, xs1;   // activation scales of this lane's 16 accumulator rows
            if constexpr (!DOTS) {
                xs0 = *reinterpret_cast<const f16x8 *>(sXh + b * kPlaneH + 32 * wv + 16 * g);
                xs1 = *reinterpret_cast<const f16x8 *>(sXh + b * kPlaneH + 32 * wv + 16 * g + 8);
            }
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int col = 32 * c + l32;
                const i32x4 bq = *reinterpret_cast<const i32x4 *>(sB + b_row + sw + c * 32 * kRowBytes);
                const i32x16 D = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq, srcC, 0, 0, 0);
                if constexpr (DOTS) {
                    int32_t *dots = reinterpret_cast<int32_t *>(outp);
                    const int n = n0 + col;
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int m = m0 + 32 * wv + 8 * (r >> 2) + 4 * g + (r & 3);
                        if (m < M && n < N)
                            dots[(int64_t(m) * N + n) * kb + int64_t(ks) * KB + b] = D[r];
                    }
                } else {
                    const float ws = sWd[(wplane + b) * kPlane + col];
                    const float cs = -kMagic * ws;   // exact
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const float t = __builtin_fmaf(__int_as_float(D[r]), ws, cs);
                        const float xr = (float)(r < 8 ? xs0[r & 7] : xs1[r & 7]);   // exact widening
                        acc[c][r] = __builtin_fmaf(xr, t, acc[c][r]);
                    }
                }
                // One MFMA result in flight per wave: the matrix core and the
                // VALU do not overlap within a SIMD here, so the other waves
                // of the SIMD hide this wave's MFMA latency, and the register
                // budget allows three (Q4_K) or four (Q8_0) waves per SIMD.
                // Only LDS reads may be hoisted across.
                __builtin_amdgcn_sched_barrier(0x0100);
            }
        }
        if constexpr (FMT == FMT_Q4_K && !DOTS) {
            if (ks & 1) {   // end of a super-block: its min term
                const unsigned short *sSum = reinterpret_cast<const unsigned short *>(smem + L::OFF_A_SUM);
                const _Float16 *sMin = reinterpret_cast<const _Float16 *>(smem + L::OFF_B_MIN);
                const f16x8 sa = *reinterpret_cast<const f16x8 *>(sSum + (32 * wv + l32) * 8);
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    const f16x8 mb = *reinterpret_cast<const f16x8 *>(sMin + ((32 * c + l32) * 2 + g) * 8);
                    acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(sa, mb, acc[c], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    if constexpr (!DOTS) {
        float *out = reinterpret_cast<float *>(outp);
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const int n = n0 + 32 * c + l32;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = m0 + 32 * wv + 8 * (r >> 2) + 4 * g + (r & 3);
                if (m < M && n < N) out[int64_t(m) * N + n] = acc[c][r];
            }
        }
    }
}

// Host-side launchers (declared in mmq_launch.hpp).
hipError_t launch_quantize(const float *x, void *y, int64_t M, int64_t K, int cu_count,
                           hipStream_t stream) {
    const int64_t nblocks = M * (K / 32);
    const int64_t groups_per_wg = 256 / 8;
    int64_t grid = (nblocks + groups_per_wg - 1) / groups_per_wg;
    const int64_t cap = int64_t(cu_count) * 16;   // enough resident waves to saturate HBM
    if (grid > cap) grid = cap;
    hipLaunchKernelGGL(k_quantize_q8_1, dim3((unsigned)grid), dim3(256), 0, stream, x,
                       reinterpret_cast<uint32_t *>(y), nblocks);
    return hipGetLastError();
}

hipError_t launch_gemm(const Plan &p, const void *x, const void *w, void *out, int64_t M, int64_t N,
                       int64_t K, bool dots, hipStream_t stream) {
    const dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y);
    const dim3 block(p.threads);
    const auto *xb = reinterpret_cast<const uint8_t *>(x);
    const auto *wb = reinterpret_cast<const uint8_t *>(w);
    const size_t lds = size_t(p.lds_bytes);
    if (p.fmt == FMT_Q8_0) {
        if (dots)
            hipLaunchKernelGGL((k_mmq<FMT_Q8_0, true>), grid, block, lds, stream, xb, wb, out, int(M), int(N), int(K));
        else
            hipLaunchKernelGGL((k_mmq<FMT_Q8_0, false>), grid, block, lds, stream, xb, wb, out, int(M), int(N), int(K));
    } else {
        if (dots)
            hipLaunchKernelGGL((k_mmq<FMT_Q4_K, true>), grid, block, lds, stream, xb, wb, out, int(M), int(N), int(K));
        else
            hipLaunchKernelGGL((k_mmq<FMT_Q4_K, false>), grid, block, lds, stream, xb, wb, out, int(M), int(N), int(K));
    }
    return hipGetLastError();
}

}  // namespace mmq
