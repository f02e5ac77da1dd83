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
//      codes and the errors d of the block; the update adds d_block * U[block, later] to
//      the accumulators of every later column.
// Everything is fp32; the codes are the sweep's decisions in fp32 (the oracle's in fp64
// may differ where a value falls within rounding of a code boundary).
#include "q4_launch.h"

namespace {

constexpr int NB = 64;  // panel and block width

// ------------------------------------------------------------ 64 x 64 fp32 tile products
// out[r][c] (r, c < 64) += sum_{s < 64} X[r][s] * Y[c][s], with X and Y in LDS as [64][65]
// (padded rows: conflict-free column reads).  Thread t of 256 owns rows 4 (t / 16) .. +3
// and columns 4 (t % 16) .. +3.
__device__ __forceinline__ void tile_fma(const float (*X)[65], const float (*Y)[65], float (&acc)[4][4]) {
    const int t = threadIdx.x;
    const int r0 = 4 * (t >> 4), c0 = 4 * (t & 15);
#pragma unroll 4
    for (int s = 0; s < NB; ++s) {
        float xv[4], yv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xv[i] = X[r0 + i][s];
            yv[i] = Y[c0 + i][s];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(xv[i], yv[j], acc[i][j]);
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
    __shared__ float Xs[NB][65], Ys[NB][65];
    const int t = threadIdx.x;
    float acc[4][4] = {};
    for (int t0 = 0; t0 < tokens; t0 += NB) {
        // token slice [t0, t0 + 64): Xs[a][s] = x[t0 + s][k-1-(64 I + a)], Ys likewise for J
        for (int e = t; e < NB * NB; e += 256) {
            const int s = e / NB, a = e % NB;
            const int tok = t0 + s;
            const int fa = k - 1 - (NB * I + a), fb = k - 1 - (NB * J + a);
            Xs[a][s] = tok < tokens && fa >= 0 ? half_to_float<XF16>(x[(int64_t)tok * k + fa]) : 0.f;
            Ys[a][s] = tok < tokens && fb >= 0 ? half_to_float<XF16>(x[(int64_t)tok * k + fb]) : 0.f;
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
    for (int c = 0; c < bw; ++c) {
        if (t == 0) T[c][c] = sqrtf(T[c][c]);
        __syncthreads();
        const float d = T[c][c];
        for (int r = c + 1 + t; r < bw; r += 256) T[r][c] = T[r][c] / d;
        __syncthreads();
        // T[r][s] -= T[r][c] T[s][c] for c < s <= r < bw
        const int m = bw - c - 1;
        for (int e = t; e < m * m; e += 256) {
            const int r = c + 1 + e / m, s = c + 1 + e % m;
            if (s <= r) T[r][s] = __builtin_fmaf(-T[r][c], T[s][c], T[r][s]);
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
    __shared__ float Xs[NB][65], Ys[NB][65];
    const int t = threadIdx.x;
    for (int e = t; e < NB * NB; e += 256) {
        const int r = e / NB, s = e % NB;
        const int a = base + NB * I + r, b = base + NB * J + r;
        Xs[r][s] = a < k && s < bw ? A[(int64_t)a * k + j0 + s] : 0.f;
        Ys[r][s] = b < k && s < bw ? A[(int64_t)b * k + j0 + s] : 0.f;
    }
    __syncthreads();
    float acc[4][4] = {};
    tile_fma(Xs, Ys, acc);
    const int r0 = 4 * (t >> 4), c0 = 4 * (t & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int a = base + NB * I + r0 + i, b = base + NB * J + c0 + j;
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
            const float wj = load_w<DT>(w, (int64_t)row * k + col);
            float s = C[(int64_t)row * k + col];
#pragma unroll
            for (int i = 0; i < j; ++i) s = __builtin_fmaf(d[i], UT[j][i], s);
            const float wp = wj + s / UT[j][j];
            const float u = fminf(fmaxf(rintf(wp / S) + z, 0.f), 15.f);
            d[j] = wj - S * (u - z);
            words[j / 8] |= (uint32_t)u << (4 * (j % 8));
        }
    }
#pragma unroll
    for (int q = 0; q < NB / 8; ++q)
        if (8 * q < bw) qweight[(int64_t)row * (k / 8) + j0 / 8 + q] = words[q];
#pragma unroll
    for (int j = 0; j < NB; ++j)
        if (j < bw) Dout[(int64_t)row * NB + j] = d[j];
}

// C[r][l] += sum_{i<bw} D[r][i] U_{j0+i, l} for the later columns l >= j0 + bw, in 64 x 64
// tiles (row tile R, column tile L); U_{j0+i, l} = A[k-1-(j0+i)][k-1-l].
__global__ __launch_bounds__(256) void gptq_update_kernel(const float* __restrict__ A, const float* __restrict__ D,
                                                          float* __restrict__ C, int n, int k, int j0, int bw) {
    const int base = j0 + bw;
    const int ctiles = (k - base + NB - 1) / NB;
    const int R = blockIdx.x / ctiles, Lt = blockIdx.x % ctiles;
    __shared__ float Xs[NB][65], Ys[NB][65];
    const int t = threadIdx.x;
    for (int e = t; e < NB * NB; e += 256) {
        const int r = e / NB, s = e % NB;
        const int row = NB * R + r, col = base + NB * Lt + r;
        Xs[r][s] = row < n && s < bw ? D[(int64_t)row * NB + s] : 0.f;
        Ys[r][s] = col < k && s < bw ? A[(int64_t)(k - 1 - (j0 + s)) * k + (k - 1 - col)] : 0.f;
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
