// gptq.hip — GPTQ-style error-feedback quantization into the packed INT4 format, gfx950.
//
// "Quantization Algorithms 단권화", GPTQ chapter (§Hessian 정의, §OBQ single-step 수식,
// §GPTQ block-wise, §알고리즘 개요): columns are quantized in order and each column's
// quantization error is carried into the columns not yet quantized, weighted by the
// calibration Hessian H = 2 X^T X (dampened).  The group quantizers (scale, zero point)
// are those of RTN on the original weights, fixed before the sweep; the sweep only chooses
// the codes.
//
// Formulation.  The pages carry the error with L, the upper Cholesky factor of H^-1:
// err_j = (w'_j - w_hat_j) / L_jj, w'_l -= err_j L_jl.  Here the same updates come from the
// upper factor U of H itself (H = U U^T), with no inverse: column j is quantized at
//   w'_j = w_j + (sum_{i<j} d_i U_ij) / U_jj,   d_i = w_i - w_hat_i
// (w the original weights, w_hat the dequantized codes).  Both give the one-step optimal
// update: for two coupled features, w'_1 = w_1 + d_0 H_01 / H_11.  U is the lower Cholesky
// factor of H with rows and columns reversed, so the Hessian is written reversed
// (A[a][b] = H[k-1-a][k-1-b]) and factored in place: U_ij = A[k-1-i][k-1-j].
//
// Steps, all on the caller's stream:
//   1. RTN quantize/pack: the static group scales and zero points (codes overwritten).
//   2. A = reversed H, lower triangle, fp32: 2 sum_t x_t x_t^T; a zero diagonal becomes 1;
//      the diagonal is scaled by 1 + damp.
//   3. In-place blocked Cholesky of A (64-wide panels): factor the diagonal block in LDS,
//      solve the rows below against it, subtract the panel's outer product from the
//      trailing lower triangle.
//   4. C = 0 (n x k accumulators of sum_{i<j} d_i U_ij).  For each block of 64 columns:
//      the sweep (one lane per weight row, the block's 64 columns in order) writes the
//      codes and the errors d of the block (column-major); the update adds d_block * U[block, later] to
//      the accumulators of every later column.
// Everything is fp32; the codes are the sweep's decisions in fp32 (the oracle's in fp64
// may differ where a value falls within rounding of a code boundary).
#include "q4_launch.h"

namespace {

constexpr int NB = 64;  // panel and block width

// ------------------------------------------------------------ 64 x 64 fp32 tile products
// out[r][c] (r, c < 64) += sum_{s < 64} X[s][r] * Y[s][c], with X and Y in LDS k-major
// ([64][64]: a row of 64 values per s).  Thread t of 256 owns rows 4 (t / 16) .. +3 and
// columns 4 (t % 16) .. +3: per s one 16-byte read of X (shared by 16 threads) and one of Y
// (16 consecutive threads read 64 consecutive floats) feed 16 FMAs.
typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void tile_fma(const float (*X)[NB], const float (*Y)[NB], float (&acc)[4][4]) {
    const int t = threadIdx.x;
    const int r0 = 4 * (t >> 4), c0 = 4 * (t & 15);
#pragma unroll 8
    for (int s = 0; s < NB; ++s) {
        const f32x4v xv = *reinterpret_cast<const f32x4v*>(&X[s][r0]);
        const f32x4v yv = *reinterpret_cast<const f32x4v*>(&Y[s][c0]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(xv[i], yv[j], acc[i][j]);
    }
}

// out[r][c] (r, c < 64) += sum_{s < 64} X[r][s] * Y[c][s], with X and Y in LDS row-major at a
// row stride of RS floats.  Thread t owns rows t / 16 + 16 i and columns t % 16 + 16 j
// (i, j < 4): per 4 values of s, four 16-byte reads of X (4 addresses per wave, broadcast)
// and four of Y (16 addresses per wave, RS apart: every bank once) feed 64 FMAs.
constexpr int RS = NB + 4;

__device__ __forceinline__ void tile_fma_rows(const float (*X)[RS], const float (*Y)[RS], float (&acc)[4][4]) {
    const int t = threadIdx.x;
    const int r = t >> 4, c = t & 15;
#pragma unroll 2
    for (int s = 0; s < NB; s += 4) {
        f32x4v xv[4], yv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[i] = *reinterpret_cast<const f32x4v*>(&X[r + 16 * i][s]);
#pragma unroll
        for (int j = 0; j < 4; ++j) yv[j] = *reinterpret_cast<const f32x4v*>(&Y[c + 16 * j][s]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(xv[i][q], yv[j][q], acc[i][j]);
    }
}

template <bool XF16>
__device__ __forceinline__ float half_to_float(uint16_t h) {
    if constexpr (XF16) return (float)__builtin_bit_cast(_Float16, h);
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// ------------------------------------------------------------ step 2: reversed Hessian
// Workgroup (I, J), I >= J, computes the 64 x 64 tile A[64 I ..][64 J ..] over all tokens.
template <bool XF16>
__global__ __launch_bounds__(256) void hessian_kernel(const uint16_t* __restrict__ x, int tokens, int k,
                                                      float damp, float* __restrict__ A) {
    const int tiles = (k + NB - 1) / NB;
    const int I = blockIdx.x / tiles, J = blockIdx.x % tiles;
    if (J > I) return;  // upper tiles: not needed (uniform)
    __shared__ __attribute__((aligned(16))) float Xs[NB][NB], Ys[NB][NB];
    const int t = threadIdx.x;
    float acc[4][4] = {};
    for (int t0 = 0; t0 < tokens; t0 += NB) {
        // token slice [t0, t0 + 64): Xs[s][a] = x[t0 + s][k-1-(64 I + a)], Ys likewise for J
        for (int e = t; e < NB * NB; e += 256) {
            const int s = e / NB, a = e % NB;
            const int tok = t0 + s;
            const int fa = k - 1 - (NB * I + a), fb = k - 1 - (NB * J + a);
            Xs[s][a] = tok < tokens && fa >= 0 ? half_to_float<XF16>(x[(int64_t)tok * k + fa]) : 0.f;
            Ys[s][a] = tok < tokens && fb >= 0 ? half_to_float<XF16>(x[(int64_t)tok * k + fb]) : 0.f;
        }
        __syncthreads();
        tile_fma(Xs, Ys, acc);
        __syncthreads();
    }
    const int r0 = 4 * (t >> 4), c0 = 4 * (t & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int a = NB * I + r0 + i, b = NB * J + c0 + j;
            if (a >= k || b > a) continue;
            float h = 2.0f * acc[i][j];
            if (a == b) {
                if (h == 0.0f) h = 1.0f;  // a feature never active
                h = h + damp * h;
            }
            A[(int64_t)a * k + b] = h;
        }
}

// ------------------------------------------------------------ step 3: blocked Cholesky
// Factor the diagonal block A[j0 .. j0+bw)^2 (lower) in place, in LDS.
__global__ __launch_bounds__(256) void chol_diag_kernel(float* __restrict__ A, int k, int j0, int bw) {
    __shared__ float T[NB][NB + 1];
    const int t = threadIdx.x;
    for (int e = t; e < NB * NB; e += 256) {
        const int r = e / NB, c = e % NB;
        T[r][c] = r < bw && c <= r ? A[(int64_t)(j0 + r) * k + j0 + c] : 0.f;
    }
    __syncthreads();
    // thread t updates row r = t % 64, columns s = t / 64, +4, ... of the trailing block
    const int ur = t & 63, us = t >> 6;
    for (int c = 0; c < bw; ++c) {
        const float d = sqrtf(T[c][c]);  // every thread: no barrier between the root and its use
        __syncthreads();                 // all have read T[c][c] before it is overwritten
        if (t == c) T[c][c] = d;
        if (t > c && t < bw) T[t][c] = T[t][c] / d;
        __syncthreads();
        if (ur > c && ur < bw) {
            const float lr = T[ur][c];
            for (int s2 = c + 1 + ((us - (c + 1)) & 3); s2 <= ur; s2 += 4)
                T[ur][s2] = __builtin_fmaf(-lr, T[s2][c], T[ur][s2]);
        }
        __syncthreads();
    }
    for (int e = t; e < NB * NB; e += 256) {
        const int r = e / NB, c = e % NB;
        if (r < bw && c <= r) A[(int64_t)(j0 + r) * k + j0 + c] = T[r][c];
    }
}

// Rows r >= j0 + bw: L[r][j0 + c] = (A[r][j0 + c] - sum_{s<c} L[r][j0+s] L[j0+c][j0+s]) / L[j0+c][j0+c].
__global__ __launch_bounds__(256) void chol_trsm_kernel(float* __restrict__ A, int k, int j0, int bw) {
    __shared__ float D[NB][NB + 1];
    const int t = threadIdx.x;
    for (int e = t; e < NB * NB; e += 256) {
        const int r = e / NB, c = e % NB;
        D[r][c] = r < bw && c <= r ? A[(int64_t)(j0 + r) * k + j0 + c] : 0.f;
    }
    __syncthreads();
    const int r = j0 + bw + (int)blockIdx.x * 256 + t;
    if (r >= k) return;
    float* row = A + (int64_t)r * k + j0;
    float v[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) v[c] = c < bw ? row[c] : 0.f;
#pragma unroll
    for (int c = 0; c < NB; ++c) {
        if (c < bw) {
            float s = v[c];
#pragma unroll
            for (int q = 0; q < c; ++q) s = __builtin_fmaf(-v[q], D[c][q], s);
            v[c] = s / D[c][c];
        }
    }
#pragma unroll
    for (int c = 0; c < NB; ++c)
        if (c < bw) row[c] = v[c];
}

// Trailing update: A[a][b] -= sum_{s<bw} L[a][j0+s] L[b][j0+s] for j0+bw <= b <= a < k, in 64 x 64
// tiles (I, J) of the trailing part, I >= J.
__global__ __launch_bounds__(256) void chol_update_kernel(float* __restrict__ A, int k, int j0, int bw) {
    const int base = j0 + bw;
    const int tiles = (k - base + NB - 1) / NB;
    const int I = blockIdx.x / tiles, J = blockIdx.x % tiles;
    if (J > I) return;  // uniform
    __shared__ __attribute__((aligned(16))) float Xs[NB][RS], Ys[NB][RS];
    const int t = threadIdx.x;
    for (int e = t; e < NB * NB; e += 256) {
        const int r = e / NB, s = e % NB;
        const int a = base + NB * I + r, b = base + NB * J + r;
        Xs[r][s] = a < k && s < bw ? A[(int64_t)a * k + j0 + s] : 0.f;
        Ys[r][s] = b < k && s < bw ? A[(int64_t)b * k + j0 + s] : 0.f;
    }
    __syncthreads();
    float acc[4][4] = {};
    tile_fma_rows(Xs, Ys, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int a = base + NB * I + (t >> 4) + 16 * i, b = base + NB * J + (t & 15) + 16 * j;
            if (a < k && b <= a) A[(int64_t)a * k + b] -= acc[i][j];
        }
}

// ------------------------------------------------------------ step 4: sweep and update
__global__ void fill_zero_kernel(float* __restrict__ p, int64_t count) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

template <int DT>
__device__ __forceinline__ float load_w(const void* w, int64_t idx) {
    if constexpr (DT == 0) return reinterpret_cast<const float*>(w)[idx];
    else return half_to_float<DT == 1>(reinterpret_cast<const uint16_t*>(w)[idx]);
}

// One lane per weight row; the block's columns j0 .. j0+bw-1 (bw = 64 or 32) in order.
// U[i][j] for i, j in the block is A[k-1-(j0+i)][k-1-(j0+j)], staged transposed in LDS.
template <int DT, bool SYM>
__global__ __launch_bounds__(64) void sweep_kernel(const void* __restrict__ w, int n, int k, int g,
                                                   const float* __restrict__ A, const float* __restrict__ C,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint32_t* __restrict__ zeros,
                                                   uint32_t* __restrict__ qweight, float* __restrict__ Dout,
                                                   int j0, int bw) {
    __shared__ float UT[NB][NB + 1];  // UT[j][i] = U_ij (i <= j), zero elsewhere
    const int t = threadIdx.x;
    for (int e = t; e < NB * NB; e += 64) {
        const int j = e / NB, i = e % NB;
        UT[j][i] = i <= j && j < bw ? A[(int64_t)(k - 1 - (j0 + i)) * k + (k - 1 - (j0 + j))] : 0.f;
    }
    __syncthreads();
    const int row = (int)blockIdx.x * 64 + t;
    if (row >= n) return;
    const int n_groups = k / g, zwords = (n_groups + 7) / 8;
    // the row's slice of C and of the weights for the block, in 16-byte loads (k is a multiple
    // of 32 and the rows of w are 16-byte aligned)
    float cv[NB], wv[NB];
    const float* crow = C + (int64_t)row * k + j0;
#pragma unroll
    for (int q = 0; q < NB / 4; ++q) {
        const f32x4v v = 4 * q < bw ? *reinterpret_cast<const f32x4v*>(crow + 4 * q) : f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) cv[4 * q + e] = v[e];
    }
    if constexpr (DT == 0) {
        const float* wrow = reinterpret_cast<const float*>(w) + (int64_t)row * k + j0;
#pragma unroll
        for (int q = 0; q < NB / 4; ++q) {
            const f32x4v v = 4 * q < bw ? *reinterpret_cast<const f32x4v*>(wrow + 4 * q) : f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) wv[4 * q + e] = v[e];
        }
    } else {
        typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
        const uint16_t* wrow = reinterpret_cast<const uint16_t*>(w) + (int64_t)row * k + j0;
#pragma unroll
        for (int q = 0; q < NB / 8; ++q) {
            const u32x4v v = 8 * q < bw ? *reinterpret_cast<const u32x4v*>(wrow + 8 * q) : u32x4v{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                wv[8 * q + e] = half_to_float<DT == 1>((uint16_t)(v[e / 2] >> (16 * (e % 2))));
        }
    }
    float d[NB];
    uint32_t words[NB / 8];
#pragma unroll
    for (int q = 0; q < NB / 8; ++q) words[q] = 0u;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        d[j] = 0.f;
        if (j < bw) {
            const int col = j0 + j, gi = col / g;
            const float S = (float)__builtin_bit_cast(_Float16, scales[(int64_t)row * n_groups + gi]);
            const float z = SYM ? 8.f : (float)((zeros[(int64_t)row * zwords + gi / 8] >> (4 * (gi % 8))) & 0xFu);
            // sum_{i<j} d_i U_ij in four interleaved partial sums (a shorter dependency chain)
            float p[4] = {cv[j], 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < j; ++i) p[i & 3] = __builtin_fmaf(d[i], UT[j][i], p[i & 3]);
            const float sum = (p[0] + p[1]) + (p[2] + p[3]);
            const float wp = wv[j] + sum / UT[j][j];
            const float u = fminf(fmaxf(rintf(wp / S) + z, 0.f), 15.f);
            d[j] = wv[j] - S * (u - z);
            words[j / 8] |= (uint32_t)u << (4 * (j % 8));
        }
    }
#pragma unroll
    for (int q = 0; q < NB / 8; ++q)
        if (8 * q < bw) qweight[(int64_t)row * (k / 8) + j0 / 8 + q] = words[q];
#pragma unroll
    for (int j = 0; j < NB; ++j)
        if (j < bw) Dout[(int64_t)j * n + row] = d[j];
}

// C[r][l] += sum_{i<bw} D[i][r] U_{j0+i, l} for the later columns l >= j0 + bw, in 64 x 64
// tiles (row tile R, column tile L); D holds the block's errors column-major ([64][n]) and
// U_{j0+i, l} = A[k-1-(j0+i)][k-1-l].
__global__ __launch_bounds__(256) void gptq_update_kernel(const float* __restrict__ A, const float* __restrict__ D,
                                                          float* __restrict__ C, int n, int k, int j0, int bw) {
    const int base = j0 + bw;
    const int ctiles = (k - base + NB - 1) / NB;
    const int R = blockIdx.x / ctiles, Lt = blockIdx.x % ctiles;
    __shared__ __attribute__((aligned(16))) float Xs[NB][NB], Ys[NB][NB];
    const int t = threadIdx.x;
    for (int e = t; e < NB * NB; e += 256) {
        // D is column-major ([64][n]) and U[j0 + s][col] has reversed, contiguous addresses
        // along col: consecutive threads take consecutive rows, columns
        const int s = e / NB, c = e % NB;
        const int row = NB * R + c, col = base + NB * Lt + c;
        Xs[s][c] = row < n && s < bw ? D[(int64_t)s * n + row] : 0.f;
        Ys[s][c] = col < k && s < bw ? A[(int64_t)(k - 1 - (j0 + s)) * k + (k - 1 - col)] : 0.f;
    }
    __syncthreads();
    float acc[4][4] = {};
    tile_fma(Xs, Ys, acc);
    const int r0 = 4 * (t >> 4), c0 = 4 * (t & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = NB * R + r0 + i, col = base + NB * Lt + c0 + j;
            if (row < n && col < k) C[(int64_t)row * k + col] += acc[i][j];
        }
}

template <int DT, bool SYM>
hipError_t sweep_all(const void* w, int n, int k, int g, const float* A, float* C, const uint16_t* sc,
                     const uint32_t* zr, uint32_t* qw, float* D, hipStream_t st) {
    for (int j0 = 0; j0 < k; j0 += NB) {
        const int bw = k - j0 < NB ? k - j0 : NB;
        hipLaunchKernelGGL((sweep_kernel<DT, SYM>), dim3((n + 63) / 64), dim3(64), 0, st, w, n, k, g, A, C, sc,
                           zr, qw, D, j0, bw);
        if (j0 + bw < k) {
            const int ctiles = (k - j0 - bw + NB - 1) / NB;
            hipLaunchKernelGGL(gptq_update_kernel, dim3(((n + NB - 1) / NB) * ctiles), dim3(256), 0, st, A, D, C,
                               n, k, j0, bw);
        }
    }
    return hipGetLastError();
}

}  // namespace

int64_t q4k_gptq_workspace_floats(int64_t n, int64_t k) {
    return k * k + n * k + n * NB;  // A, C, D
}

hipError_t q4k_gptq(const void* w, int w_dtype, int64_t n, int64_t k, const void* x, int x_dtype,
                    int64_t tokens, int g, int sym, float damp, uint32_t* qweight, uint16_t* scales,
                    uint32_t* zeros, float* workspace, hipStream_t st, const char** kname) {
    // 1. static group quantizers (and RTN codes, overwritten below)
    hipError_t e = q4k_quant_pack(w, w_dtype, n, k, g, sym, qweight, scales, zeros, st, kname);
    if (e != hipSuccess) return e;
    float* A = workspace;
    float* C = A + k * k;
    float* D = C + n * k;
    const int ki = (int)k, ni = (int)n;
    // 2. reversed Hessian, lower triangle
    const int tiles = (ki + NB - 1) / NB;
    const uint16_t* xs = reinterpret_cast<const uint16_t*>(x);
    if (x_dtype == 1)
        hipLaunchKernelGGL(hessian_kernel<true>, dim3(tiles * tiles), dim3(256), 0, st, xs, (int)tokens, ki, damp, A);
    else
        hipLaunchKernelGGL(hessian_kernel<false>, dim3(tiles * tiles), dim3(256), 0, st, xs, (int)tokens, ki, damp, A);
    // 3. Cholesky in place
    for (int j0 = 0; j0 < ki; j0 += NB) {
        const int bw = ki - j0 < NB ? ki - j0 : NB;
        hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), 0, st, A, ki, j0, bw);
        const int below = ki - j0 - bw;
        if (below > 0) {
            hipLaunchKernelGGL(chol_trsm_kernel, dim3((below + 255) / 256), dim3(256), 0, st, A, ki, j0, bw);
            const int tt = (below + NB - 1) / NB;
            hipLaunchKernelGGL(chol_update_kernel, dim3(tt * tt), dim3(256), 0, st, A, ki, j0, bw);
        }
    }
    // 4. sweep
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, st, C, n * k);
    switch (w_dtype * 2 + (sym ? 1 : 0)) {
    case 0: e = sweep_all<0, false>(w, ni, ki, g, A, C, scales, zeros, qweight, D, st); break;
    case 1: e = sweep_all<0, true>(w, ni, ki, g, A, C, scales, zeros, qweight, D, st); break;
    case 2: e = sweep_all<1, false>(w, ni, ki, g, A, C, scales, zeros, qweight, D, st); break;
    case 3: e = sweep_all<1, true>(w, ni, ki, g, A, C, scales, zeros, qweight, D, st); break;
    case 4: e = sweep_all<2, false>(w, ni, ki, g, A, C, scales, zeros, qweight, D, st); break;
    default: e = sweep_all<2, true>(w, ni, ki, g, A, C, scales, zeros, qweight, D, st); break;
    }
    static const char* names[3] = {"q4_gptq_f32", "q4_gptq_f16", "q4_gptq_bf16"};
    *kname = names[w_dtype];
    return e;
}
