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
//   2. A = reversed H, lower triangle, fp32: 2 sum_t x_t x_t^T (128 x 128 tiles); a zero
//      diagonal becomes 1; the diagonal is scaled by 1 + damp.
//   3. In-place blocked Cholesky of A (64-wide panels): factor the diagonal block in
//      registers (and invert the factor), multiply the rows below by the inverse's
//      transpose, subtract the panel's outer product from the trailing lower triangle.
//   4. C = 0 (n x k accumulators of sum_{i<j} d_i U_ij).  For each block of 64 columns:
//      the sweep (one lane per weight row, the block's 64 columns in order) writes the
//      codes and the errors d of the block (column-major); updates add d * U[block, later]
//      to the accumulators of later columns, lazily in super-blocks of 256 columns (see
//      sweep_all).
// Everything is fp32; the codes are the sweep's decisions in fp32 (the oracle's in fp64
// may differ where a value falls within rounding of a code boundary).
#include "q4_launch.h"

namespace {

constexpr int NB = 64;   // panel and block width
constexpr int SB = 256;  // super-block width of the lazy updates (a multiple of NB)

// ------------------------------------------------------------ 64 x 64 fp32 tile products
// On the fp32 matrix cores (v_mfma_f32_32x32x2_f32).  Four waves split the 64 x 64 output:
// wave w computes rows 32 (w / 2) .. +31 and columns 32 (w % 2) .. +31.  Per MFMA, lane l
// gives the A value of row l % 32 and the B value of column l % 32, both at inner index
// s + l / 32; its 16 results are rows (e & 3) + 4 (l / 32) + 8 (e / 4) (e < 16) of
// column l % 32 of the quadrant (tile_row / tile_col below).
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
constexpr int RS = NB + 1;   // row stride of row-major LDS tiles (lanes of a read: all banks)
constexpr int KS = NB;  // row stride of k-major LDS tiles (unpadded: occupancy over a 2-way read conflict)

__device__ __forceinline__ int tile_row(int e) {
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    return 32 * (w >> 1) + (e & 3) + 4 * (l >> 5) + 8 * (e >> 2);
}
__device__ __forceinline__ int tile_col() {
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    return 32 * (w & 1) + (l & 31);
}

// acc += X^T Y over s < 64, with X and Y in LDS k-major (X[s][r], Y[s][c]) at stride KS.
__device__ __forceinline__ void tile_mfma(const float (*X)[KS], const float (*Y)[KS], f32x16& acc) {
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int rb = 32 * (w >> 1) + (l & 31), cb = 32 * (w & 1) + (l & 31), h = l >> 5;
#pragma unroll 8
    for (int s = 0; s < NB; s += 2) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(X[s + h][rb], Y[s + h][cb], acc, 0, 0, 0);
}

// acc += X Y^T over s < 64, with X and Y in LDS row-major (X[r][s], Y[c][s]) at stride RS.
__device__ __forceinline__ void tile_mfma_rows(const float (*X)[RS], const float (*Y)[RS], f32x16& acc) {
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int rb = 32 * (w >> 1) + (l & 31), cb = 32 * (w & 1) + (l & 31), h = l >> 5;
#pragma unroll 8
    for (int s = 0; s < NB; s += 2) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(X[rb][s + h], Y[cb][s + h], acc, 0, 0, 0);
}

template <bool XF16>
__device__ __forceinline__ float half_to_float(uint16_t h) {
    if constexpr (XF16) return (float)__builtin_bit_cast(_Float16, h);
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// ------------------------------------------------------------ step 2: reversed Hessian
// Workgroup (I, J), I >= J, computes the 128 x 128 tile A[128 I ..][128 J ..] over all
// tokens; wave w computes the 64 x 64 quadrant (w / 2, w % 2) as 2 x 2 MFMA tiles.  The
// tiles are twice the panel width so that the activations are read half as often (each
// token slice of a tile pair is staged once per 128 x 128 outputs).
constexpr int HB = 128;

// With PERM, position p of the sweep is feature perm[p] (act-order): the tile is the
// Hessian of the permuted features, A[a][b] = H[perm[k-1-a]][perm[k-1-b]], gathered from
// the activations one 16-bit value at a time.
template <bool XF16, bool PERM>
__global__ __launch_bounds__(256) void hessian_kernel(const uint16_t* __restrict__ x, int tokens, int k,
                                                      float damp, const int* __restrict__ perm,
                                                      float* __restrict__ A) {
    const int tiles = (k + HB - 1) / HB;
    const int I = blockIdx.x / tiles, J = blockIdx.x % tiles;
    if (J > I) return;  // upper tiles: not needed (uniform)
    // token slice [t0, t0 + 64): Xs[s][a] = x[t0 + s][k-1-(128 I + a)], Ys likewise for J
    __shared__ __attribute__((aligned(16))) float Xs[NB][HB], Ys[NB][HB];
    __shared__ int pX[PERM ? HB : 1], pY[PERM ? HB : 1];  // features of this tile's positions
    const int t = threadIdx.x;
    const int l = t & 63, w = t >> 6, h = l >> 5, li = l & 31;
    if constexpr (PERM) {
        // position k-1-(HB I + a) holds feature pX[a] (0 past the last position)
        if (t < HB) {
            const int pa = k - 1 - (HB * I + t);
            pX[t] = pa >= 0 ? perm[pa] : 0;
        } else {
            const int pb = k - 1 - (HB * J + (t - HB));
            pY[t - HB] = pb >= 0 ? perm[pb] : 0;
        }
        __syncthreads();
    }
    const int rb = 64 * (w >> 1), cb = 64 * (w & 1);
    f32x16 acc[2][2] = {};
    // This thread's 16 feature pairs of a slice (one 32-bit word each: features a and a+1
    // are adjacent, reversed, in the row) are loaded a slice ahead, so the next slice's
    // loads are in flight while the current one's products run.  k is even and a row
    // starts 4-byte aligned, so the pair (k-1-(128 I + a) - 1, k-1-(128 I + a)) is one word.
    constexpr int PP = NB * HB / 2 / 256;
    const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
    uint32_t xr[PP], yr[PP];
    auto fetch = [&](int t0) {
#pragma unroll
        for (int r = 0; r < PP; ++r) {
            const int e = t + 256 * r, s = e / (HB / 2), a = 2 * (e % (HB / 2));
            const int tok = t0 + s;
            const int fa = k - 1 - (HB * I + a), fb = k - 1 - (HB * J + a);
            if constexpr (PERM) {
                // positions fa and fa - 1 (fa is odd) are pX[a] and pX[a + 1]
                const uint16_t* xt = x + (int64_t)tok * k;
                xr[r] = tok < tokens && fa >= 0 ? ((uint32_t)xt[pX[a]] << 16) | (uint32_t)xt[pX[a + 1]] : 0u;
                yr[r] = tok < tokens && fb >= 0 ? ((uint32_t)xt[pY[a]] << 16) | (uint32_t)xt[pY[a + 1]] : 0u;
            } else {
                xr[r] = tok < tokens && fa >= 0 ? x32[((int64_t)tok * k + fa - 1) / 2] : 0u;
                yr[r] = tok < tokens && fb >= 0 ? x32[((int64_t)tok * k + fb - 1) / 2] : 0u;
            }
        }
    };
    fetch(0);
    for (int t0 = 0; t0 < tokens; t0 += NB) {
        __syncthreads();  // the previous slice's products have read the tiles
#pragma unroll
        for (int r = 0; r < PP; ++r) {
            const int e = t + 256 * r, s = e / (HB / 2), a = 2 * (e % (HB / 2));
            // the high half is feature a (x[fa]), the low half feature a + 1 (x[fa - 1])
            Xs[s][a] = half_to_float<XF16>((uint16_t)(xr[r] >> 16));
            Xs[s][a + 1] = half_to_float<XF16>((uint16_t)(xr[r] & 0xFFFFu));
            Ys[s][a] = half_to_float<XF16>((uint16_t)(yr[r] >> 16));
            Ys[s][a + 1] = half_to_float<XF16>((uint16_t)(yr[r] & 0xFFFFu));
        }
        __syncthreads();
        if (t0 + NB < tokens) fetch(t0 + NB);
#pragma unroll 4
        for (int s = 0; s < NB; s += 2) {
            const float a0 = Xs[s + h][rb + li], a1 = Xs[s + h][rb + 32 + li];
            const float b0 = Ys[s + h][cb + li], b1 = Ys[s + h][cb + 32 + li];
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int a = HB * I + rb + 32 * i + (e & 3) + 4 * h + 8 * (e >> 2);
                const int b = HB * J + cb + 32 * j + li;
                if (a >= k || b > a) continue;
                float hv = 2.0f * acc[i][j][e];
                if (a == b) {
                    if (hv == 0.0f) hv = 1.0f;  // a feature never active
                    hv = hv + damp * hv;
                }
                A[(int64_t)a * k + b] = hv;
            }
}

// ------------------------------------------------------------ step 3: blocked Cholesky
// Factor the diagonal block A[j0 .. j0+bw)^2 (lower) in place, and store the inverse of the
// factor, Linv = L^-1 (lower), by its strict lower part transposed into the block's upper
// triangle, which nothing else uses: A[j0+s][j0+c] = Linv[c][s] for s < c.  (Linv's
// diagonal is 1/L[c][c].)  Rows and columns past bw are an identity.
//
// Thread t holds row r = t % 64 of both matrices at the columns s = DW i + t/64 (i < 64/DW)
// in registers; each of the DW waves owns one residue class of columns.  Step c, for
// c = 0 .. 63:
//   - the wave owning column c takes the root of its diagonal entry (lane c), scales the
//     column and writes it to col[c] (each column once: no second barrier);
//   - after the barrier every thread subtracts col[c][r] * col[c][s] from its entries s > c
//     (right-looking factorization);
//   - the inverse by forward substitution, one step behind: the rows of Linv below row c-1
//     subtract L[r][c-1] * Linv[c-1][s], then row c divides by L[c][c] and goes to inv[c].
// Sixteen waves keep each step's per-wave work short: the steps are a serial chain.
constexpr int DW = 16, DPER = NB / DW;

__global__ __launch_bounds__(64 * DW) void chol_diag_kernel(float* __restrict__ A, int k, int j0, int bw) {
    __shared__ float col[NB][NB];  // col[c][r] = L[r][c] (0 above the diagonal)
    __shared__ float inv[NB][NB];  // inv[c][s] = Linv[c][s] (0 right of the diagonal)
    const int t = threadIdx.x;
    // w stays a vector value: as a scalar, the column predicates of a step would live in
    // scalar register pairs and spill
    const int r = t & 63, w = t >> 6;
    float T[DPER], X[DPER];
#pragma unroll
    for (int i = 0; i < DPER; ++i) {
        const int s = DW * i + w;
        T[i] = r < bw && s <= r ? A[(int64_t)(j0 + r) * k + j0 + s] : (r == s ? 1.f : 0.f);
        X[i] = r == s ? 1.f : 0.f;
    }
    // fully unrolled: T[c / DW] must be a fixed register
#pragma clang loop unroll(full)
    for (int c = 0; c < NB; ++c) {
        if (w == c % DW) {
            const float v = T[c / DW];  // this lane's row, column c
            const float dg = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), c));
            const float d = sqrtf(dg);
            const float l = r == c ? d : (r > c ? v / d : 0.f);
            T[c / DW] = l;
            col[c][r] = l;
        }
        __syncthreads();
        // every read up front (broadcasts, always in range), then the updates as selects
        float cs[DPER], is[DPER];
#pragma unroll
        for (int i = 0; i < DPER; ++i) {
            cs[i] = col[c][DW * i + w];
            is[i] = c > 0 ? inv[c - 1][DW * i + w] : 0.f;
        }
        const float lr = col[c][r];
        const float lx = c > 0 ? col[c - 1][r] : 0.f;
#pragma unroll
        for (int i = 0; i < DPER; ++i) {
            const int s = DW * i + w;
            const float tv = __builtin_fmaf(-lr, cs[i], T[i]);
            T[i] = s > c && s <= r ? tv : T[i];
            const float xv = __builtin_fmaf(-lx, is[i], X[i]);
            X[i] = c > 0 && r >= c && s <= c - 1 ? xv : X[i];
        }
        if (r == c) {
            const float dinv = 1.0f / col[c][c];
#pragma unroll
            for (int i = 0; i < DPER; ++i) {
                X[i] = DW * i + w <= c ? X[i] * dinv : 0.f;
                inv[c][DW * i + w] = X[i];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < DPER; ++i) {
        const int s = DW * i + w;
        if (r < bw && s <= r) A[(int64_t)(j0 + r) * k + j0 + s] = T[i];
        if (r < bw && s < r) A[(int64_t)(j0 + s) * k + j0 + r] = X[i];
    }
}

// Rows below the diagonal block, 64 per workgroup: L21 = A21 Linv^T, a 64 x 64 tile product
// with the inverse stored by chol_diag_kernel (Y[c][s] = Linv[c][s]).
__global__ __launch_bounds__(256) void chol_trsm_kernel(float* __restrict__ A, int k, int j0, int bw) {
    __shared__ __attribute__((aligned(16))) float Xs[NB][RS], Ys[NB][RS];
    const int t = threadIdx.x;
    const int base = j0 + bw + (int)blockIdx.x * NB;
    for (int e = t; e < NB * NB; e += 256) {
        const int a = e / NB, b = e % NB;
        Xs[a][b] = base + a < k && b < bw ? A[(int64_t)(base + a) * k + j0 + b] : 0.f;
        // Ys[c][s] = Linv[c][s], stored transposed in the block's upper triangle
        // (A[j0+s][j0+c], s < c): consecutive threads take consecutive c, contiguous in A
        const int s = e / NB, c = e % NB;
        float v = 0.f;
        if (c < bw && s < bw) {
            if (s < c) v = A[(int64_t)(j0 + s) * k + j0 + c];
            else if (s == c) v = 1.0f / A[(int64_t)(j0 + c) * k + j0 + c];
        }
        Ys[c][s] = v;
    }
    __syncthreads();
    f32x16 acc = {};
    tile_mfma_rows(Xs, Ys, acc);
    const int cc = tile_col();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int a = base + tile_row(e);
        if (a < k && cc < bw) A[(int64_t)a * k + j0 + cc] = acc[e];
    }
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
    f32x16 acc = {};
    tile_mfma_rows(Xs, Ys, acc);
    const int b = base + NB * J + tile_col();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int a = base + NB * I + tile_row(e);
        if (a < k && b <= a) A[(int64_t)a * k + b] -= acc[e];
    }
}

// ------------------------------------------------------------ step 4: sweep and update
__global__ void fill_zero_kernel(float* __restrict__ p, int64_t count) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

// ------------------------------------------------------------ act-order
// The sweep order of act-order ("Quantization Algorithms 단권화", GPTQ chapter, §설정 grid:
// the columns whose activations carry the most energy first): features by descending
// e_i = sum_t x_ti^2, equal energies by the lower index.
//
// Energies in two passes with a fixed summation order: slice s of `slice` tokens sums
// sequentially into part[s][i] (one lane per feature, a wave per 64 features and slice),
// then key[i] = sum_s part[s][i] in order of s.
template <bool XF16>
__global__ __launch_bounds__(64) void energy_kernel(const uint16_t* __restrict__ x, int tokens, int k, int slice,
                                                    float* __restrict__ part) {
    const int i = (int)blockIdx.x * 64 + (int)threadIdx.x;
    const int s = (int)blockIdx.y;
    if (i >= k) return;
    const int t0 = s * slice, t1 = tokens - t0 < slice ? tokens : t0 + slice;
    float acc = 0.f;
    for (int t = t0; t < t1; ++t) {
        const float v = half_to_float<XF16>(x[(int64_t)t * k + i]);
        acc = acc + v * v;
    }
    part[(int64_t)s * k + i] = acc;
}

__global__ void energy_sum_kernel(const float* __restrict__ part, int slices, int k, float* __restrict__ key,
                                  int* __restrict__ rank) {
    const int i = (int)blockIdx.x * blockDim.x + (int)threadIdx.x;
    if (i >= k) return;
    float acc = 0.f;
    for (int s = 0; s < slices; ++s) acc = acc + part[(int64_t)s * k + i];
    key[i] = acc;
    rank[i] = 0;
}

// rank[i] += #{j in this block's chunk of 1024 : e_j > e_i, or e_j == e_i and j < i}.
// The energies are compared as their bit patterns: for non-negative floats that is their
// order, and it stays a strict total order (with the index) whatever the values, so the
// ranks are a permutation.  Integer counts: the order of the atomic additions is immaterial.
__global__ __launch_bounds__(256) void rank_kernel(const float* __restrict__ key, int k, int* __restrict__ rank) {
    __shared__ uint32_t kb[1024];
    const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
    const int c0 = (int)blockIdx.y * 1024;
    const int cn = k - c0 < 1024 ? k - c0 : 1024;
    for (int e = threadIdx.x; e < cn; e += 256) kb[e] = __builtin_bit_cast(uint32_t, key[c0 + e]);
    __syncthreads();
    if (i >= k) return;
    const uint32_t mine = __builtin_bit_cast(uint32_t, key[i]);
    int cnt = 0;
    for (int e = 0; e < cn; ++e) {
        const uint32_t o = kb[e];
        cnt += (o > mine) | ((o == mine) & (c0 + e < i));
    }
    if (cnt) atomicAdd(rank + i, cnt);
}

__global__ void scatter_order_kernel(const int* __restrict__ rank, int k, int* __restrict__ perm) {
    const int i = (int)blockIdx.x * blockDim.x + (int)threadIdx.x;
    if (i < k) perm[rank[i]] = i;
}

// qweight[r][c / 8] from the byte codes codes[r][c] (column order), eight per word.
__global__ void pack_codes_kernel(const uint8_t* __restrict__ codes, int64_t words, uint32_t* __restrict__ qweight) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t c = reinterpret_cast<const uint64_t*>(codes)[i];
        uint32_t wv = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) wv |= (uint32_t)((c >> (8 * e)) & 0xFu) << (4 * e);
        qweight[i] = wv;
    }
}

template <int DT>
__device__ __forceinline__ float load_w(const void* w, int64_t idx) {
    if constexpr (DT == 0) return reinterpret_cast<const float*>(w)[idx];
    else return half_to_float<DT == 1>(reinterpret_cast<const uint16_t*>(w)[idx]);
}

// Four lanes per weight row (a quad of consecutive lanes); the block's columns j0 .. j0+bw-1
// (bw = 64 or 32) in order.  Lane q of the quad holds the errors d_i of the columns
// i = 4m + q and sums their share of sum_{i<j} d_i U_ij; the quad adds its four shares, so
// every lane holds the same total and takes the same quantization decision for column j
// (the errors of columns not yet reached are still zero, so the shares need no bounds).
// U's block is staged transposed in LDS: UT[j][i] = U_ij (i <= j), zero elsewhere.
// Lane q loads the block's C and weights for columns 16q .. 16q+15; column j's pair comes
// from lane j / 16 of the quad by a lane broadcast.
template <int SRC>
__device__ __forceinline__ float quad_bcast_from(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), SRC * 0x55, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_bcast(float v, int src) {  // src folds to a constant in the unrolled sweep
    switch (src) {
    case 0: return quad_bcast_from<0>(v);
    case 1: return quad_bcast_from<1>(v);
    case 2: return quad_bcast_from<2>(v);
    default: return quad_bcast_from<3>(v);
    }
}
__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));  // lane ^ 1
    return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));  // lane ^ 2
}

//
// With PERM (act-order) position j0 + j is column perm[j0 + j]: its weight and its group's
// scale and zero point are gathered per column (lane q holds those of its 16 columns, like
// C), and its code goes to byte codes[row][perm[j0 + j]]; pack_codes_kernel packs them.
template <int DT, bool SYM, bool PERM>
__global__ __launch_bounds__(256) void sweep_kernel(const void* __restrict__ w, int n, int k, int g,
                                                    const float* __restrict__ A, const float* __restrict__ C,
                                                    const uint16_t* __restrict__ scales,
                                                    const uint32_t* __restrict__ zeros,
                                                    uint32_t* __restrict__ qweight, float* __restrict__ Dout,
                                                    int j0, int bw, const int* __restrict__ perm,
                                                    uint8_t* __restrict__ codes) {
    __shared__ float UT[NB][NB + 1];  // UT[j][i] = U_ij (i <= j), zero elsewhere
    __shared__ float rU[NB];          // 1 / U_jj
    const int t = threadIdx.x;
    for (int e = t; e < NB * NB; e += 256) {
        // consecutive threads take consecutive j: one row of A, contiguous (reversed) addresses
        const int i = e / NB, j = e % NB;
        UT[j][i] = i <= j && j < bw ? A[(int64_t)(k - 1 - (j0 + i)) * k + (k - 1 - (j0 + j))] : 0.f;
    }
    if (t < NB) rU[t] = t < bw ? 1.0f / A[(int64_t)(k - 1 - (j0 + t)) * k + (k - 1 - (j0 + t))] : 0.f;
    __syncthreads();
    const int q = t & 3;
    const int row = (int)blockIdx.x * 64 + (t >> 2);
    if (row >= n) return;  // whole quads together; nothing below waits for other lanes
    const int n_groups = k / g, zwords = (n_groups + 7) / 8;
    // columns 16q .. 16q+15 of the row's C and weights, in 16-byte loads (k is a multiple of
    // 32 and the rows of w are 16-byte aligned)
    float cv[16], wv[16];
    const int c0 = 16 * q;
    const float* crow = C + (int64_t)row * k + j0 + c0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const f32x4v x = c0 + 4 * v < bw ? *reinterpret_cast<const f32x4v*>(crow + 4 * v) : f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) cv[4 * v + e] = x[e];
    }
    // act-order: the fp16 scale (low half) and zero point (bits 16..19) of each column
    uint32_t szv[PERM ? 16 : 1];
    if constexpr (PERM) {
        const int n_groups_ = k / g, zwords_ = (n_groups_ + 7) / 8;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const bool in = c0 + e < bw;
            const int col = in ? perm[j0 + c0 + e] : 0;
            const int gi = col / g;
            wv[e] = in ? load_w<DT>(w, (int64_t)row * k + col) : 0.f;
            const uint32_t zc = SYM ? 8u : (zeros[(int64_t)row * zwords_ + gi / 8] >> (4 * (gi % 8))) & 0xFu;
            szv[e] = (uint32_t)scales[(int64_t)row * n_groups_ + gi] | (zc << 16);
        }
    } else if constexpr (DT == 0) {
        const float* wrow = reinterpret_cast<const float*>(w) + (int64_t)row * k + j0 + c0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const f32x4v x = c0 + 4 * v < bw ? *reinterpret_cast<const f32x4v*>(wrow + 4 * v) : f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) wv[4 * v + e] = x[e];
        }
    } else {
        typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
        const uint16_t* wrow = reinterpret_cast<const uint16_t*>(w) + (int64_t)row * k + j0 + c0;
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const u32x4v x = c0 + 8 * v < bw ? *reinterpret_cast<const u32x4v*>(wrow + 8 * v) : u32x4v{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                wv[8 * v + e] = half_to_float<DT == 1>((uint16_t)(x[e / 2] >> (16 * (e % 2))));
        }
    }
    float dl[NB / 4];  // d_i for i = 4m + q (zero until column i is quantized)
#pragma unroll
    for (int m = 0; m < NB / 4; ++m) dl[m] = 0.f;
    uint32_t words[NB / 8];
#pragma unroll
    for (int m = 0; m < NB / 8; ++m) words[m] = 0u;
    uint32_t cu[PERM ? 16 : 1];  // codes of this lane's 16 columns (act-order)
#pragma unroll
    for (int e = 0; e < (PERM ? 16 : 1); ++e) cu[e] = 0u;
    // The column loop is a serial chain: the divisions by U_jj and by the scale are
    // multiplications by reciprocals taken once per block and once per group, and the
    // lane's share of each dot product runs in two interleaved sums.
    float S = 1.f, rS = 1.f, z = 8.f;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        if (j < bw) {
            if constexpr (PERM) {
                const uint32_t sz = __builtin_bit_cast(uint32_t, quad_bcast(__builtin_bit_cast(float, szv[j % 16]), j / 16));
                S = (float)__builtin_bit_cast(_Float16, (uint16_t)(sz & 0xFFFFu));
                rS = 1.0f / S;
                z = (float)(sz >> 16);
            } else {
                const int col = j0 + j, gi = col / g;
                if (j == 0 || col % g == 0) {  // a new group (uniform)
                    S = (float)__builtin_bit_cast(_Float16, scales[(int64_t)row * n_groups + gi]);
                    rS = 1.0f / S;
                    if constexpr (!SYM) z = (float)((zeros[(int64_t)row * zwords + gi / 8] >> (4 * (gi % 8))) & 0xFu);
                }
            }
            const float cj = quad_bcast(cv[j % 16], j / 16);
            const float wj = quad_bcast(wv[j % 16], j / 16);
            // this lane's share of sum_{i<j} d_i U_ij (entries with i >= j are zero)
            float p0 = 0.f, p1 = 0.f;
#pragma unroll
            for (int m = 0; m < (j + 3) / 4; ++m) {
                if (m % 2 == 0) p0 = __builtin_fmaf(dl[m], UT[j][4 * m + q], p0);
                else p1 = __builtin_fmaf(dl[m], UT[j][4 * m + q], p1);
            }
            const float sum = quad_sum(p0 + p1) + cj;
            const float wp = __builtin_fmaf(sum, rU[j], wj);
            const float u = fminf(fmaxf(rintf(wp * rS) + z, 0.f), 15.f);
            const float dj = wj - S * (u - z);
            dl[j / 4] = q == (j & 3) ? dj : dl[j / 4];
            if constexpr (PERM) cu[j % 16] = q == j / 16 ? (uint32_t)u : cu[j % 16];
            else words[j / 8] |= (uint32_t)u << (4 * (j % 8));
        }
    }
    if constexpr (PERM) {
        // lane q stores the codes of its 16 columns at their own positions
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (c0 + e < bw) codes[(int64_t)row * k + perm[j0 + c0 + e]] = (uint8_t)cu[e];
    } else {
        // lane q stores code words 2q, 2q+1 (columns 16q .. 16q+15)
#pragma unroll
        for (int m = 0; m < NB / 8; ++m)
            if (m / 2 == q && 8 * m < bw) qweight[(int64_t)row * (k / 8) + j0 / 8 + m] = words[m];
    }
    // and its own errors
#pragma unroll
    for (int m = 0; m < NB / 4; ++m)
        if (4 * m + q < bw) Dout[(int64_t)(4 * m + q) * n + row] = dl[m];
}

// C[r][l] += sum_{i < inner} D[i][r] U_{j0+i, l} for the columns col0 <= l < col1, in 64 x 64
// tiles (row tile R, column tile L), the inner sum in chunks of 64 staged in LDS.  D holds
// errors column-major ([inner][n], row i = weight column j0 + i) and
// U_{j0+i, l} = A[k-1-(j0+i)][k-1-l].
__global__ __launch_bounds__(256) void gptq_update_kernel(const float* __restrict__ A, const float* __restrict__ D,
                                                          float* __restrict__ C, int n, int k, int j0, int inner,
                                                          int col0, int col1) {
    const int ctiles = (col1 - col0 + NB - 1) / NB;
    const int R = blockIdx.x / ctiles, Lt = blockIdx.x % ctiles;
    __shared__ __attribute__((aligned(16))) float Xs[NB][KS], Ys[NB][KS];
    const int t = threadIdx.x;
    f32x16 acc = {};
    // this thread's 16 elements of a chunk in registers: the next chunk's loads are in
    // flight while the current chunk's products run
    constexpr int PER = NB * NB / 256;
    float xr[PER], yr[PER];
    auto fetch = [&](int ch) {
        const int cw = inner - ch < NB ? inner - ch : NB;
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            // D is column-major and U[j0 + ch + s][col] has reversed, contiguous addresses
            // along col: consecutive threads take consecutive rows, columns
            const int e = t + 256 * r, s = e / NB, c = e % NB;
            const int row = NB * R + c, col = col0 + NB * Lt + c;
            xr[r] = row < n && s < cw ? D[(int64_t)(ch + s) * n + row] : 0.f;
            yr[r] = col < col1 && s < cw ? A[(int64_t)(k - 1 - (j0 + ch + s)) * k + (k - 1 - col)] : 0.f;
        }
    };
    fetch(0);
    for (int ch = 0; ch < inner; ch += NB) {
        __syncthreads();  // the previous chunk's products have read the tiles
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int e = t + 256 * r;
            Xs[e / NB][e % NB] = xr[r];
            Ys[e / NB][e % NB] = yr[r];
        }
        __syncthreads();
        if (ch + NB < inner) fetch(ch + NB);
        tile_mfma(Xs, Ys, acc);
    }
    const int col = col0 + NB * Lt + tile_col();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int row = NB * R + tile_row(e);
        if (row < n && col < col1) C[(int64_t)row * k + col] += acc[e];
    }
}

void update(const float* A, const float* D, float* C, int n, int k, int j0, int inner, int col0, int col1,
            hipStream_t st) {
    if (col0 >= col1) return;
    const int ctiles = (col1 - col0 + NB - 1) / NB;
    hipLaunchKernelGGL(gptq_update_kernel, dim3(((n + NB - 1) / NB) * ctiles), dim3(256), 0, st, A, D, C, n, k, j0,
                       inner, col0, col1);
    q4k_record("q4_gptq_update");
}

// Lazy updates at two levels.  Blocks of 64 columns are swept in order inside super-blocks
// of SB columns.  After a block, only the later columns of its super-block take its
// errors; after a super-block, every column beyond it takes the errors of all its blocks
// in one update with an inner size of SB.  The accumulator traffic falls by about SB / 64
// against updating every later column after every block; the sums are the same.
template <int DT, bool SYM, bool PERM>
hipError_t sweep_all(const void* w, int n, int k, int g, const float* A, float* C, const uint16_t* sc,
                     const uint32_t* zr, uint32_t* qw, float* D, const int* perm, uint8_t* codes,
                     hipStream_t st) {
    for (int s0 = 0; s0 < k; s0 += SB) {
        const int s1 = k - s0 < SB ? k : s0 + SB;
        for (int j0 = s0; j0 < s1; j0 += NB) {
            const int bw = s1 - j0 < NB ? s1 - j0 : NB;
            float* Db = D + (int64_t)(j0 - s0) * n;  // this block's rows of the super-block's errors
            hipLaunchKernelGGL((sweep_kernel<DT, SYM, PERM>), dim3((n + 63) / 64), dim3(256), 0, st, w, n, k, g, A,
                               C, sc, zr, qw, Db, j0, bw, perm, codes);
            q4k_record("q4_gptq_sweep");
            update(A, Db, C, n, k, j0, bw, j0 + bw, s1, st);   // the rest of the super-block
        }
        update(A, D, C, n, k, s0, s1 - s0, s1, k, st);        // every column beyond it
    }
    return hipGetLastError();
}

template <bool PERM>
hipError_t sweep_dispatch(int w_dtype, int sym, const void* w, int n, int k, int g, const float* A, float* C,
                          const uint16_t* sc, const uint32_t* zr, uint32_t* qw, float* D, const int* perm,
                          uint8_t* codes, hipStream_t st) {
    switch (w_dtype * 2 + (sym ? 1 : 0)) {
    case 0: return sweep_all<0, false, PERM>(w, n, k, g, A, C, sc, zr, qw, D, perm, codes, st);
    case 1: return sweep_all<0, true, PERM>(w, n, k, g, A, C, sc, zr, qw, D, perm, codes, st);
    case 2: return sweep_all<1, false, PERM>(w, n, k, g, A, C, sc, zr, qw, D, perm, codes, st);
    case 3: return sweep_all<1, true, PERM>(w, n, k, g, A, C, sc, zr, qw, D, perm, codes, st);
    case 4: return sweep_all<2, false, PERM>(w, n, k, g, A, C, sc, zr, qw, D, perm, codes, st);
    default: return sweep_all<2, true, PERM>(w, n, k, g, A, C, sc, zr, qw, D, perm, codes, st);
    }
}

// Tokens per energy slice: 32, or more so that the slices' partial sums (one row of k per
// slice) fit the k x k Hessian area they are staged in.
int energy_slice(int64_t tokens, int64_t k) {
    const int64_t per = (tokens + 31) / 32;
    return (int)(32 * ((per + k - 1) / k));
}

}  // namespace

int64_t q4k_gptq_workspace_floats(int64_t n, int64_t k) {
    return k * k + n * k + n * SB;  // A, C, D
}

int64_t q4k_gptq_act_order_workspace_floats(int64_t n, int64_t k) {
    // then the energies, the ranks, the order, and n x k byte codes
    return q4k_gptq_workspace_floats(n, k) + 3 * k + n * k / 4;
}

hipError_t q4k_gptq(const void* w, int w_dtype, int64_t n, int64_t k, const void* x, int x_dtype,
                    int64_t tokens, int g, int sym, float damp, uint32_t* qweight, uint16_t* scales,
                    uint32_t* zeros, float* workspace, int act_order, hipStream_t st, const char** kname) {
    // 1. static group quantizers (and RTN codes, overwritten below)
    hipError_t e = q4k_quant_pack(w, w_dtype, n, k, g, sym, qweight, scales, zeros, st, kname);
    if (e != hipSuccess) return e;
    float* A = workspace;
    float* C = A + k * k;
    float* D = C + n * k;
    float* key = D + n * SB;
    int* rank = reinterpret_cast<int*>(key + k);
    int* perm = act_order ? rank + k : nullptr;
    uint8_t* codes = act_order ? reinterpret_cast<uint8_t*>(rank + 2 * k) : nullptr;
    const int ki = (int)k, ni = (int)n;
    const uint16_t* xs = reinterpret_cast<const uint16_t*>(x);
    // 1b. act-order: the sweep order from the activation energies (partials staged in A)
    if (act_order) {
        const int slice = energy_slice(tokens, k);
        const int slices = (int)((tokens + slice - 1) / slice);
        const dim3 eg((unsigned)((ki + 63) / 64), (unsigned)slices);
        if (x_dtype == 1)
            hipLaunchKernelGGL(energy_kernel<true>, eg, dim3(64), 0, st, xs, (int)tokens, ki, slice, A);
        else
            hipLaunchKernelGGL(energy_kernel<false>, eg, dim3(64), 0, st, xs, (int)tokens, ki, slice, A);
        hipLaunchKernelGGL(energy_sum_kernel, dim3((ki + 255) / 256), dim3(256), 0, st, A, slices, ki, key, rank);
        hipLaunchKernelGGL(rank_kernel, dim3((ki + 255) / 256, (ki + 1023) / 1024), dim3(256), 0, st, key, ki, rank);
        hipLaunchKernelGGL(scatter_order_kernel, dim3((ki + 255) / 256), dim3(256), 0, st, rank, ki, perm);
        q4k_record("q4_gptq_energy");
        q4k_record("q4_gptq_energy_sum");
        q4k_record("q4_gptq_rank");
        q4k_record("q4_gptq_order");
    }
    // 2. reversed Hessian, lower triangle (of the permuted features with act-order)
    const int tiles = (ki + HB - 1) / HB;
    const dim3 hg(tiles * tiles);
    if (x_dtype == 1 && act_order)
        hipLaunchKernelGGL((hessian_kernel<true, true>), hg, dim3(256), 0, st, xs, (int)tokens, ki, damp, perm, A);
    else if (x_dtype == 1)
        hipLaunchKernelGGL((hessian_kernel<true, false>), hg, dim3(256), 0, st, xs, (int)tokens, ki, damp, perm, A);
    else if (act_order)
        hipLaunchKernelGGL((hessian_kernel<false, true>), hg, dim3(256), 0, st, xs, (int)tokens, ki, damp, perm, A);
    else
        hipLaunchKernelGGL((hessian_kernel<false, false>), hg, dim3(256), 0, st, xs, (int)tokens, ki, damp, perm, A);
    q4k_record("q4_gptq_hessian");
    // 3. Cholesky in place
    for (int j0 = 0; j0 < ki; j0 += NB) {
        const int bw = ki - j0 < NB ? ki - j0 : NB;
        hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(64 * DW), 0, st, A, ki, j0, bw);
        q4k_record("q4_gptq_chol_diag");
        const int below = ki - j0 - bw;
        if (below > 0) {
            hipLaunchKernelGGL(chol_trsm_kernel, dim3((below + NB - 1) / NB), dim3(256), 0, st, A, ki, j0, bw);
            const int tt = (below + NB - 1) / NB;
            hipLaunchKernelGGL(chol_update_kernel, dim3(tt * tt), dim3(256), 0, st, A, ki, j0, bw);
            q4k_record("q4_gptq_chol_panel");
            q4k_record("q4_gptq_chol_update");
        }
    }
    // 4. sweep
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, st, C, n * k);
    q4k_record("q4_gptq_fill_zero");
    if (act_order) {
        e = sweep_dispatch<true>(w_dtype, sym, w, ni, ki, g, A, C, scales, zeros, qweight, D, perm, codes, st);
        if (e != hipSuccess) return e;
        const int64_t words = n * k / 8;
        hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)((words + 255) / 256 < 4096 ? (words + 255) / 256 : 4096)),
                           dim3(256), 0, st, codes, words, qweight);
        q4k_record("q4_gptq_pack_codes");
        e = hipGetLastError();
    } else {
        e = sweep_dispatch<false>(w_dtype, sym, w, ni, ki, g, A, C, scales, zeros, qweight, D, nullptr, nullptr, st);
    }
    static const char* names[2][3] = {{"q4_gptq_f32", "q4_gptq_f16", "q4_gptq_bf16"},
                                      {"q4_gptq_act_order_f32", "q4_gptq_act_order_f16", "q4_gptq_act_order_bf16"}};
    *kname = names[act_order ? 1 : 0][w_dtype];
    return e;
}
