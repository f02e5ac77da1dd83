// gemm.hip — prefill W4A16 linear layer (m > 16) for gfx950.
//
//   y[m][n] = sum_g S[n][g] * sum_{k in g} x[m][k] * (u[n][k] - z[n][g])
//
// Large-batch prefill is compute-bound ("LLM Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV
// Cache (7/10)", §Batch와 Context에 따라 속도가 달라진다), so this is a dense MFMA
// contraction.  Each workgroup dequantizes a tile of packed weights into LDS as exact
// small integers u - z (bf16 or fp16, matching the activations), stages the activation
// tile next to it, and runs v_mfma_f32_16x16x32 over the tile.  The per-group scale is
// applied to fp32 partial sums at every group boundary, so every product is exact and
// every sum is fp32 (path A of §Kernel이 없으면 압축 이점이 사라진다).
//
// Tile: 128 activation rows x 128 weight rows, 32 columns per step; 4 waves in a 2x2
// arrangement, 64x64 outputs (4x4 MFMA tiles) per wave.
#include "q4_device.h"

namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDS_STRIDE = BK + 8;  // 16-bit elements per LDS row (pad spreads banks)

template <int G, bool SYM, bool XF16>
__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t* __restrict__ x, int M,
                                                   const uint32_t* __restrict__ qweight,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint32_t* __restrict__ zeros, int N,
                                                   int K, float* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) uint16_t a_lds[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t b_lds[BN * LDS_STRIDE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int col = lane & 15, c = lane >> 4;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int KW = K / 8;
    const int n_groups = K / G;
    const int zwords = (n_groups + 7) >> 3;

    // loader roles: row r of both tiles, half h (16 columns)
    const int lr = tid >> 1, lh = tid & 1;
    const int xm = m0 + lr, wn_row = n0 + lr;
    const bool xok = xm < M, wok = wn_row < N;

    q4::f32x4 acc[4][4], part[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[i][j] = q4::f32x4{0.f, 0.f, 0.f, 0.f};
            part[i][j] = q4::f32x4{0.f, 0.f, 0.f, 0.f};
        }

    for (int k0 = 0; k0 < K; k0 += BK) {
        const int gidx = k0 / G;
        // ---- stage activations
        q4::u32x4 xv0 = {0u, 0u, 0u, 0u}, xv1 = {0u, 0u, 0u, 0u};
        if (xok) {
            const q4::u32x4* p =
                reinterpret_cast<const q4::u32x4*>(x + (int64_t)xm * K + k0 + 16 * lh);
            xv0 = p[0];
            xv1 = p[1];
        }
        // ---- dequantize two packed words (16 weights) of one weight row
        q4::u32x4 wv0 = {0u, 0u, 0u, 0u}, wv1 = {0u, 0u, 0u, 0u};
        if (wok) {
            const q4::u32x2 pw =
                *reinterpret_cast<const q4::u32x2*>(qweight + (int64_t)wn_row * KW + k0 / 8 + 2 * lh);
            int z = 8;
            if constexpr (!SYM)
                z = (int)((zeros[(int64_t)wn_row * zwords + (gidx >> 3)] >> (4 * (gidx & 7))) & 0xFu);
            uint16_t e[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int d = (int)((pw[i >> 3] >> (4 * (i & 7))) & 0xFu) - z;
                if constexpr (XF16)
                    e[i] = __builtin_bit_cast(uint16_t, (_Float16)(float)d);
                else
                    e[i] = __builtin_bit_cast(uint16_t, (__bf16)(float)d);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                wv0[i] = (uint32_t)e[2 * i] | ((uint32_t)e[2 * i + 1] << 16);
                wv1[i] = (uint32_t)e[8 + 2 * i] | ((uint32_t)e[8 + 2 * i + 1] << 16);
            }
        }
        __syncthreads();  // previous step's MFMAs are done reading LDS
        *reinterpret_cast<q4::u32x4*>(&a_lds[lr * LDS_STRIDE + 16 * lh]) = xv0;
        *reinterpret_cast<q4::u32x4*>(&a_lds[lr * LDS_STRIDE + 16 * lh + 8]) = xv1;
        *reinterpret_cast<q4::u32x4*>(&b_lds[lr * LDS_STRIDE + 16 * lh]) = wv0;
        *reinterpret_cast<q4::u32x4*>(&b_lds[lr * LDS_STRIDE + 16 * lh + 8]) = wv1;
        __syncthreads();

        q4::u32x4 af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            af[i] = *reinterpret_cast<const q4::u32x4*>(&a_lds[(wm * 64 + 16 * i + col) * LDS_STRIDE + 8 * c]);
            bf[i] = *reinterpret_cast<const q4::u32x4*>(&b_lds[(wn * 64 + 16 * i + col) * LDS_STRIDE + 8 * c]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (XF16)
                    part[i][j] = q4::mfma_f16(af[i], bf[j], part[i][j]);
                else
                    part[i][j] = q4::mfma_bf16(af[i], bf[j], part[i][j]);
            }

        if ((k0 + BK) % G == 0) {  // group boundary: acc += S * partial
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int nn = n0 + wn * 64 + 16 * j + col;
                nn = nn < N ? nn : N - 1;
                const float s = q4::f16_bits_to_float(scales[(int64_t)nn * n_groups + gidx]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        acc[i][j][r] += s * part[i][j][r];
                        part[i][j][r] = 0.f;
                    }
            }
        }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int nn = n0 + wn * 64 + 16 * j + col;
            if (nn >= N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int mm = m0 + wm * 64 + 16 * i + 4 * c + r;
                if (mm < M) y[(int64_t)mm * N + nn] = acc[i][j][r];
            }
        }
}

template <int G, bool SYM>
hipError_t launch(const void* x, int xd, int m, const uint32_t* qw, const uint16_t* sc,
                  const uint32_t* zr, int n, int k, float* y, hipStream_t st, const char** kname) {
    const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM)), block(256);
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
