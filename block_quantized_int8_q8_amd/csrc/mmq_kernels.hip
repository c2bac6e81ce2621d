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
// k-step stages 8 consecutive 32-blocks (one Q4_K super-block) into LDS.
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
// Q4_K ("When Does a Kernel Win Surface?", 6.2): ws = d*sc_j (exact in fp32),
// the 4-bit codes are unpacked from the raw packed bytes in registers
// (low nibbles = even sub-block, high nibbles = odd sub-block of a 32-byte
// group), and the min term  -sum_j dmin*m_j * s_j  of a whole super-block is
// added by one fp16 MFMA per 32x32 sub-tile that accumulates straight into
// the fp32 accumulator: A = the eight activation block sums s_j (fp16, as
// stored), B = -dmin*m_j split exactly into an fp16 high and low part
// (k = 0..7 high parts, k = 8..15 low parts, each multiplied by the same s_j).
// ---------------------------------------------------------------------------
constexpr uint32_t kMagicBits = 0x4B400000u;   // 12582912.0f
constexpr float kMagic = 12582912.0f;

template <int FMT>
struct Lds {
    static constexpr int A_CODES = kBlocksPerStage * 2 * kTileM * 16;   // [b][g][row][16]
    static constexpr int A_SCALE = kBlocksPerStage * kTileM * 4;        // [b][row] fp32
    static constexpr int B_CODES = (FMT == FMT_Q8_0 ? kBlocksPerStage : 4) * 2 * kTileN * 16;
    static constexpr int B_SCALE = kBlocksPerStage * kTileN * 4;        // [b][col] fp32
    static constexpr int B_MIN = (FMT == FMT_Q4_K) ? kTileN * 2 * 8 * 2 : 0;   // [col][g][8] fp16
    static constexpr int A_SUM = (FMT == FMT_Q4_K) ? kTileM * 8 * 2 : 0;       // [row][8] fp16
    static constexpr int OFF_A_SCALE = A_CODES;
    static constexpr int OFF_B_CODES = OFF_A_SCALE + A_SCALE;
    static constexpr int OFF_B_SCALE = OFF_B_CODES + B_CODES;
    static constexpr int OFF_B_MIN = OFF_B_SCALE + B_SCALE;
    static constexpr int OFF_A_SUM = OFF_B_MIN + B_MIN;
    static constexpr int TOTAL = OFF_A_SUM + A_SUM;
};
static_assert(Lds<FMT_Q8_0>::TOTAL == lds_bytes_for(FMT_Q8_0), "plan and kernel LDS disagree");
static_assert(Lds<FMT_Q4_K>::TOTAL == lds_bytes_for(FMT_Q4_K), "plan and kernel LDS disagree");

// Stage the 8 q8_1 blocks of k-step `ks` for the tile's 128 rows.
// Unit u -> (row = u/8, block = u%8): eight consecutive threads read one
// row's 288 contiguous bytes.  Rows past M are zero-filled (codes and scale 0,
// so they add nothing and are never stored).
template <int FMT>
__device__ __forceinline__ void stage_activations(const uint8_t *__restrict__ xq, uint8_t *smem,
                                                  int M, int kb, int m0, int ks, int tid) {
    using L = Lds<FMT>;
    float *sXd = reinterpret_cast<float *>(smem + L::OFF_A_SCALE);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int u = tid + kThreads * i;
        const int row = u >> 3, b = u & 7;
        const int m = m0 + row;
        uint32_t w[9];
        if (m < M) {
            const uint32_t *src = reinterpret_cast<const uint32_t *>(
                xq + (int64_t(m) * kb + int64_t(ks) * kBlocksPerStage + b) * 36);
#pragma unroll
            for (int j = 0; j < 9; j++) w[j] = src[j];
        } else {
#pragma unroll
            for (int j = 0; j < 9; j++) w[j] = 0;
        }
        *reinterpret_cast<uint4 *>(smem + ((b * 2 + 0) * kTileM + row) * 16) = make_uint4(w[1], w[2], w[3], w[4]);
        *reinterpret_cast<uint4 *>(smem + ((b * 2 + 1) * kTileM + row) * 16) = make_uint4(w[5], w[6], w[7], w[8]);
        sXd[b * kTileM + row] = h2f(w[0]);
        if constexpr (FMT == FMT_Q4_K) {
            unsigned short *sSum = reinterpret_cast<unsigned short *>(smem + L::OFF_A_SUM);
            sSum[row * 8 + b] = (unsigned short)(w[0] >> 16);
        }
    }
}

// Stage Q8_0: unit u -> (row = u/4, block pair p = u%4).  A pair of 34-byte
// blocks is 68 bytes = 17 dwords starting on a 4-byte boundary (K % 256 == 0
// makes every row an even number of blocks); the even block's codes sit two
// bytes off the dword grid and are realigned with v_alignbyte.
__device__ __forceinline__ void stage_q8_0(const uint8_t *__restrict__ wq, uint8_t *smem, int N,
                                           int kb, int n0, int ks, int tid) {
    using L = Lds<FMT_Q8_0>;
    uint8_t *sB = smem + L::OFF_B_CODES;
    float *sWd = reinterpret_cast<float *>(smem + L::OFF_B_SCALE);
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int u = tid + kThreads * i;
        const int row = u >> 2, p = u & 3;
        const int n = n0 + row;
        uint32_t w[17];
        if (n < N) {
            const uint32_t *src = reinterpret_cast<const uint32_t *>(
                wq + (int64_t(n) * kb + int64_t(ks) * kBlocksPerStage + 2 * p) * 34);
#pragma unroll
            for (int j = 0; j < 17; j++) w[j] = src[j];
        } else {
#pragma unroll
            for (int j = 0; j < 17; j++) w[j] = 0;
        }
        uint32_t c[8];
#pragma unroll
        for (int j = 0; j < 8; j++) c[j] = __builtin_amdgcn_alignbyte(w[j + 1], w[j], 2);
        const int b0 = 2 * p, b1 = 2 * p + 1;
        *reinterpret_cast<uint4 *>(sB + ((b0 * 2 + 0) * kTileN + row) * 16) = make_uint4(c[0], c[1], c[2], c[3]);
        *reinterpret_cast<uint4 *>(sB + ((b0 * 2 + 1) * kTileN + row) * 16) = make_uint4(c[4], c[5], c[6], c[7]);
        *reinterpret_cast<uint4 *>(sB + ((b1 * 2 + 0) * kTileN + row) * 16) = make_uint4(w[9], w[10], w[11], w[12]);
        *reinterpret_cast<uint4 *>(sB + ((b1 * 2 + 1) * kTileN + row) * 16) = make_uint4(w[13], w[14], w[15], w[16]);
        sWd[b0 * kTileN + row] = h2f(w[0]);
        sWd[b1 * kTileN + row] = h2f(w[8] >> 16);
    }
}

// Sub-block j (0..7) 6-bit scale and min from the 12 packed bytes (GGUF
// K-quant packing): j < 4 uses the low six bits of bytes j and j+4; j >= 4
// takes its low four bits from byte j+4 and its top two from the spare top
// bits of bytes j-4 (scale) and j (min).
__device__ __forceinline__ void q4k_scale_min(const uint8_t *s, int j, int &sc, int &mn) {
    if (j < 4) {
        sc = s[j] & 63;
        mn = s[j + 4] & 63;
    } else {
        sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        mn = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

// Stage Q4_K super-block `ks` for the tile's 128 columns: 9 units of 16 bytes
// per row (one header, eight code chunks), consecutive threads on consecutive
// 16-byte chunks.  The codes stay packed (two 4-bit codes per byte) in LDS;
// the header is decoded once here into d*sc_j and the split min operand.
__device__ __forceinline__ void stage_q4_K(const uint8_t *__restrict__ wq, uint8_t *smem, int N,
                                           int nsb, int n0, int ks, int tid) {
    using L = Lds<FMT_Q4_K>;
    uint8_t *sB = smem + L::OFF_B_CODES;
    float *sWd = reinterpret_cast<float *>(smem + L::OFF_B_SCALE);
    _Float16 *sMin = reinterpret_cast<_Float16 *>(smem + L::OFF_B_MIN);
    for (int u = tid; u < kTileN * 9; u += kThreads) {
        const int row = u / 9, part = u - 9 * (u / 9);
        const int n = n0 + row;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n < N)
            v = reinterpret_cast<const uint4 *>(wq + (int64_t(n) * nsb + ks) * 144)[part];
        if (part == 0) {
            const float d = h2f(v.x), dmin = h2f(v.x >> 16);
            uint8_t s[12];
            const uint32_t sw[3] = {v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 12; j++) s[j] = uint8_t(sw[j >> 2] >> (8 * (j & 3)));
#pragma unroll
            for (int j = 0; j < 8; j++) {
                int sc, mn;
                q4k_scale_min(s, j, sc, mn);
                sWd[j * kTileN + row] = d * (float)sc;               // exact: 11 x 6 bits
                const float neg = -(dmin * (float)mn);               // exact
                const _Float16 hi = (_Float16)neg;
                const _Float16 lo = (_Float16)(neg - (float)hi);     // exact remainder
                sMin[(row * 2 + 0) * 8 + j] = hi;
                sMin[(row * 2 + 1) * 8 + j] = lo;
            }
        } else {
            const int c = part - 1;                  // code bytes 16c .. 16c+15
            const int grp = c >> 1, half = c & 1;    // 32-byte group, k-half within it
            *reinterpret_cast<uint4 *>(sB + ((grp * 2 + half) * kTileN + row) * 16) = v;
        }
    }
}

template <int FMT, bool DOTS>
__global__ __launch_bounds__(kThreads) void k_mmq(const uint8_t *__restrict__ xq,
                                                  const uint8_t *__restrict__ wq,
                                                  void *__restrict__ outp, int M, int N, int K) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using L = Lds<FMT>;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int n0 = blockIdx.x * kTileN, m0 = blockIdx.y * kTileM;
    const int kb = K >> 5, nsteps = K >> 8;

    const float *sXd = reinterpret_cast<const float *>(smem + L::OFF_A_SCALE);
    const uint8_t *sB = smem + L::OFF_B_CODES;
    const float *sWd = reinterpret_cast<const float *>(smem + L::OFF_B_SCALE);

    i32x16 srcC;
#pragma unroll
    for (int r = 0; r < 16; r++) srcC[r] = DOTS ? 0 : int(kMagicBits);

    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; c++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[c][r] = 0.0f;

    for (int ks = 0; ks < nsteps; ks++) {
        stage_activations<FMT>(xq, smem, M, kb, m0, ks, tid);
        if constexpr (FMT == FMT_Q8_0)
            stage_q8_0(wq, smem, N, kb, n0, ks, tid);
        else
            stage_q4_K(wq, smem, N, K >> 8, n0, ks, tid);
        __syncthreads();

#pragma unroll
        for (int b = 0; b < kBlocksPerStage; b++) {
            const i32x4 a = *reinterpret_cast<const i32x4 *>(smem + ((b * 2 + g) * kTileM + 32 * wv + l32) * 16);
            float xs[16];
            if constexpr (!DOTS) {
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const float4 t4 = *reinterpret_cast<const float4 *>(sXd + b * kTileM + 32 * wv + 8 * q + 4 * g);
                    xs[4 * q + 0] = t4.x;
                    xs[4 * q + 1] = t4.y;
                    xs[4 * q + 2] = t4.z;
                    xs[4 * q + 3] = t4.w;
                }
            }
#pragma unroll
            for (int c = 0; c < 4; c++) {
                i32x4 bq;
                if constexpr (FMT == FMT_Q8_0) {
                    bq = *reinterpret_cast<const i32x4 *>(sB + ((b * 2 + g) * kTileN + 32 * c + l32) * 16);
                } else {
                    const i32x4 raw = *reinterpret_cast<const i32x4 *>(sB + (((b >> 1) * 2 + g) * kTileN + 32 * c + l32) * 16);
                    bq = (b & 1) ? ((raw >> 4) & 0x0F0F0F0F) : (raw & 0x0F0F0F0F);
                }
                const i32x16 D = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq, srcC, 0, 0, 0);
                if constexpr (DOTS) {
                    int32_t *dots = reinterpret_cast<int32_t *>(outp);
                    const int n = n0 + 32 * c + l32;
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int m = m0 + 32 * wv + 8 * (r >> 2) + 4 * g + (r & 3);
                        if (m < M && n < N)
                            dots[(int64_t(m) * N + n) * kb + int64_t(ks) * kBlocksPerStage + b] = D[r];
                    }
                } else {
                    const float ws = sWd[b * kTileN + 32 * c + l32];
                    const float cs = -kMagic * ws;   // exact
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const float t = __builtin_fmaf(__int_as_float(D[r]), ws, cs);
                        acc[c][r] = __builtin_fmaf(xs[r], t, acc[c][r]);
                    }
                }
            }
        }
        if constexpr (FMT == FMT_Q4_K && !DOTS) {
            const unsigned short *sSum = reinterpret_cast<const unsigned short *>(smem + L::OFF_A_SUM);
            const _Float16 *sMin = reinterpret_cast<const _Float16 *>(smem + L::OFF_B_MIN);
            const f16x8 sa = *reinterpret_cast<const f16x8 *>(sSum + (32 * wv + l32) * 8);
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const f16x8 mb = *reinterpret_cast<const f16x8 *>(sMin + ((32 * c + l32) * 2 + g) * 8);
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(sa, mb, acc[c], 0, 0, 0);
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
