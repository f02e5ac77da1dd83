// gemm.hip — prefill W4A16 linear layer (m > 16) for gfx950.
//
//   y[m][n] = sum_g S[n][g] * sum_{k in g} x[m][k] * (u[n][k] - z[n][g])
//
// Large-batch prefill is compute-bound ("LLM Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV
// Cache (7/10)", §Batch와 Context에 따라 속도가 달라진다), so this is a dense MFMA
// contraction with the dequantization fused into the tile loads (path A of
// §Kernel이 없으면 압축 이점이 사라진다).
//
// Tiles.  A workgroup of 4 waves computes a 256 x 128 block of y (256 activation rows x
// 128 weight rows); wave w owns rows [64w, 64w+64) x all 128 columns as 2 x 4 tiles of
// v_mfma_f32_32x32x16 (bf16 or fp16 inputs, fp32 accumulation).  The K loop walks 32
// columns per stage through double-buffered LDS: while the MFMAs of stage s run, the
// packed words and activations of stage s+1 are already in registers, and are
// dequantized and parked in the other LDS buffer afterwards (one barrier per stage).
//
// Exactness.  The weight operand is the exact small integer u - z (|u - z| <= 15, exact
// in bf16 and fp16), so every product is exact and every sum is fp32.  The per-group
// scale is applied without a second set of accumulators: within group g the accumulator
// is kept in units of S[n][g]; entering group g it is multiplied by S[n][g-1] / S[n][g],
// and the epilogue multiplies by the last group's scale.  Zero stays exactly zero.
//
// Placement.  Consecutive workgroups land on consecutive XCDs (8 per MI355X), so block b
// takes activation block b % mtiles first: with 8 row blocks (m = 2048) each XCD's L2
// keeps one 4 MB activation block while the packed weights stream through.
#include "q4_device.h"

namespace {

constexpr int BM = 256, BN = 128, BK = 32;
constexpr int NTHREADS = 256;
constexpr int XS = BK + 8;  // LDS row stride in 16-bit elements (80 bytes: conflict-free)
constexpr int kOOB = 0x40000000;

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32_bf16(q4::u32x4 a, q4::u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(q4::bf16x8, a),
                                                   __builtin_bit_cast(q4::bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f16(q4::u32x4 a, q4::u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(q4::f16x8, a),
                                                  __builtin_bit_cast(q4::f16x8, b), c, 0, 0, 0);
}

// 8 codes of one packed word minus z, as exact 16-bit floats in natural column order
// (elements 0..7 = columns 8j..8j+7).  Bytes 128 + u - z (no borrow between bytes), then
// XOR 0x80 gives u - z as signed bytes, converted exactly to fp32 and narrowed by keeping
// the upper half (bf16) or converting (fp16; small integers are exact either way).
template <bool XF16>
__device__ __forceinline__ q4::u32x4 dequant_word(uint32_t w, uint32_t zrep) {
    const uint32_t lo = (((w & 0x0F0F0F0Fu) | 0x80808080u) - zrep) ^ 0x80808080u;         // cols 0,2,4,6
    const uint32_t hi = ((((w >> 4) & 0x0F0F0F0Fu) | 0x80808080u) - zrep) ^ 0x80808080u;  // cols 1,3,5,7
    q4::u32x4 r;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const float e = (float)(int8_t)((lo >> (8 * b)) & 0xFF);  // column 2b
        const float o = (float)(int8_t)((hi >> (8 * b)) & 0xFF);  // column 2b+1
        if constexpr (XF16) {
            const q4::f16x2 v = {(_Float16)e, (_Float16)o};
            r[b] = __builtin_bit_cast(uint32_t, v);
        } else {
            r[b] = (__builtin_bit_cast(uint32_t, e) >> 16) | (__builtin_bit_cast(uint32_t, o) & 0xFFFF0000u);
        }
    }
    return r;
}

template <int G, bool SYM, bool XF16>
__global__ __launch_bounds__(NTHREADS, 2) void gemm_kernel(const uint16_t* __restrict__ x, int M,
                                                          const uint32_t* __restrict__ qweight,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint32_t* __restrict__ zeros,
                                                          int N, int K, float* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) uint16_t a_lds[2][BM * XS];
    __shared__ __attribute__((aligned(16))) uint16_t b_lds[2][BN * XS];
    __shared__ float s_lds[2][BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int mtiles = (M + BM - 1) / BM;
    const int mt = blockIdx.x % mtiles, nt = blockIdx.x / mtiles;  // XCD-friendly order
    const int m0 = mt * BM, n0 = nt * BN;
    const int KW = K / 8;
    const int n_groups = K / G;
    const int zwords = (n_groups + 7) >> 3;
    constexpr int SPG = G / BK;  // stages per group
    const int stages = K / BK;

    const int arows = M - m0 < BM ? M - m0 : BM;
    const int brows = N - n0 < BN ? N - n0 : BN;
    const q4::rsrc rx = q4::make_rsrc(x + (int64_t)m0 * K, (uint32_t)arows * K * 2u);
    const q4::rsrc rq = q4::make_rsrc(qweight + (int64_t)n0 * KW, (uint32_t)brows * KW * 4u);
    const q4::rsrc rs = q4::make_rsrc(scales + (int64_t)n0 * n_groups, (uint32_t)brows * n_groups * 2u);
    const q4::rsrc rz = q4::make_rsrc(zeros + (int64_t)n0 * zwords, (uint32_t)brows * zwords * 4u);

    // loader roles per stage: activations, 256 rows x 64 bytes, thread t loads row t
    // (4 x 16 B); weights, 128 rows x 16 words, thread t loads 2 words of row t/2 (half
    // t%2) plus, at a group start, that row's scale and zero-point word.
    const int xoff = tid < arows ? tid * K * 2 : kOOB;
    const int wr = tid >> 1, wh = tid & 1;
    const int woff = wr < brows ? (wr * KW + 2 * wh) * 4 : kOOB;
    const int soff = wr < brows ? wr * n_groups * 2 : kOOB;
    const int zoff = wr < brows ? wr * zwords * 4 : kOOB;

    q4::u32x4 xa[4];
    q4::u32x2 wq;
    uint32_t zword = 0, sraw = 0;
    auto gload = [&](int s) {
        const int k0 = s * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) xa[i] = q4::buf_load_x4(rx, xoff, (k0 + 8 * i) * 2);
        wq = q4::buf_load_x2(rq, woff, k0 / 2);
        if (s % SPG == 0) {
            const int g = k0 / G;
            sraw = q4::buf_load_u16(rs, soff, g * 2);
            if constexpr (!SYM) zword = q4::buf_load_x1(rz, zoff, (g >> 3) * 4);
        }
    };
    auto park = [&](int s, int buf) {
        const int g = (s * BK) / G;
        q4::u32x4* ap = reinterpret_cast<q4::u32x4*>(&a_lds[buf][tid * XS]);
#pragma unroll
        for (int i = 0; i < 4; ++i) ap[i] = xa[i];
        int z = 8;
        if constexpr (!SYM) z = (int)((zword >> (4 * (g & 7))) & 0xFu);
        const uint32_t zrep = (uint32_t)z * 0x01010101u;
        // A group whose scale is zero contributes exactly nothing: its weights are parked
        // as zeros and the accumulator keeps the previous group's units (rows past N read
        // scale 0 from outside the buffer and take the same path).
        const uint32_t keep = (sraw & 0x7FFFu) != 0 ? 0xFFFFFFFFu : 0u;
        q4::u32x4* bp = reinterpret_cast<q4::u32x4*>(&b_lds[buf][wr * XS + 16 * wh]);
        bp[0] = dequant_word<XF16>(wq[0], zrep) & keep;
        bp[1] = dequant_word<XF16>(wq[1], zrep) & keep;
        if (s % SPG == 0 && wh == 0) s_lds[(s / SPG) & 1][wr] = q4::f16_bits_to_float((uint16_t)sraw);
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int col = lane & 31, half = lane >> 5;
    float s_cur[4] = {1.f, 1.f, 1.f, 1.f};

    gload(0);
    park(0, 0);
    __syncthreads();
    for (int s = 0; s < stages; ++s) {
        const int buf = s & 1;
        if (s + 1 < stages) gload(s + 1);
        if (s % SPG == 0) {  // entering a group: rescale to its units
            const float* sl = s_lds[(s / SPG) & 1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float sn = sl[32 * j + col];
                const float ratio = sn != 0.0f ? s_cur[j] / sn : 1.0f;
                if (sn != 0.0f) s_cur[j] = sn;
                if (s != 0) {
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[i][j][r] *= ratio;
                }
            }
        }
        const uint16_t* al = a_lds[buf];
        const uint16_t* bl = b_lds[buf];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            q4::u32x4 af[2], bf[4];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const q4::u32x4*>(&al[(wave * 64 + 32 * i + col) * XS + 16 * kk + 8 * half]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const q4::u32x4*>(&bl[(32 * j + col) * XS + 16 * kk + 8 * half]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (XF16)
                        acc[i][j] = mfma32_f16(af[i], bf[j], acc[i][j]);
                    else
                        acc[i][j] = mfma32_bf16(af[i], bf[j], acc[i][j]);
                }
        }
        if (s + 1 < stages) park(s + 1, buf ^ 1);
        __syncthreads();
    }

    // epilogue: back to true units, store.  Lane (col, half), register r of a 32x32 tile
    // holds row (r & 3) + 4*half + 8*(r >> 2), column col.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int nn = n0 + 32 * j + col;
        if (nn >= N) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int mm = m0 + wave * 64 + 32 * i + (r & 3) + 4 * half + 8 * (r >> 2);
                if (mm < M) y[(int64_t)mm * N + nn] = acc[i][j][r] * s_cur[j];
            }
    }
}

template <int G, bool SYM>
hipError_t launch(const void* x, int xd, int m, const uint32_t* qw, const uint16_t* sc,
                  const uint32_t* zr, int n, int k, float* y, hipStream_t st, const char** kname) {
    const int mtiles = (m + BM - 1) / BM, ntiles = (n + BN - 1) / BN;
    const dim3 grid((unsigned)(mtiles * ntiles)), block(NTHREADS);
    const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
    if (xd == 1) {
        *kname = "q4_gemm_mfma_f16";
        hipLaunchKernelGGL((gemm_kernel<G, SYM, true>), grid, block, 0, st, xp, m, qw, sc, zr, n, k, y);
    } else {
        *kname = "q4_gemm_mfma_bf16";
        hipLaunchKernelGGL((gemm_kernel<G, SYM, false>), grid, block, 0, st, xp, m, qw, sc, zr, n, k, y);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t q4k_gemm(const void* x, int x_dtype, int64_t m, const uint32_t* qweight,
                    const uint16_t* scales, const uint32_t* zeros, int64_t n, int64_t k, int g,
                    int sym, float* y, hipStream_t stream, const char** kname) {
    const int mi = (int)m, ni = (int)n, ki = (int)k;
    switch (g * 2 + (sym ? 1 : 0)) {
    case 64: return launch<32, false>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, stream, kname);
    case 65: return launch<32, true>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, stream, kname);
    case 128: return launch<64, false>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, stream, kname);
    case 129: return launch<64, true>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, stream, kname);
    case 256: return launch<128, false>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, stream, kname);
    default: return launch<128, true>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, stream, kname);
    }
}
