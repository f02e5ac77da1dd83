// gemv_tile.h — decode W4A16 tile kernel (m <= 4) for gfx950, any group size in {32, 64, 128}.
//
//   y[m][n] = sum_g S[n][g] * sum_{k in g} x[m][k] * (u[n][k] - z[n][g])
//
// Path A of "LLM Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV Cache (7/10)"
// (§Kernel이 없으면 압축 이점이 사라진다), for the bandwidth-bound decode case
// (§Batch와 Context에 따라 속도가 달라진다): the packed weights are streamed once,
// dequantized in registers and multiplied with fp32 accumulation.
//
// One 16-row tile per workgroup; its S waves split K into slices of UPW 128-column units,
// wave w taking units [w*UPW, w*UPW + nu) with nu = min(UPW, units - w*UPW), so only the
// last wave may be short.  A wave issues every load it needs at once, in wait order: its
// slice of the activations, the scales and zero points of its groups (straight into
// registers: lane l needs those of row l%16 only), then its packed weights; slots past nu
// read nothing (an offset past the buffer) and are masked out of the sums.  The activation
// slice goes to a wave-private LDS region in the decoder's slot order, so no barrier
// precedes the arithmetic; only the cross-wave sum of the tile's partial results meets at
// one.  Activation rows past m feed MFMA rows whose outputs are never stored, so lane l
// reads row min(l%16, m-1) and no zero padding is staged.  Unit offsets are compile-time
// constants, so loads and LDS reads carry them as immediates.
//
// Weights.  Lane l (row r = l%16, lane row c = l/16) loads the 16 bytes of words 4c..4c+3
// of each unit: 16 rows x 64 bytes per wave-wide load for every group size.  A 16x16x32
// MFMA takes one word from each lane row, and its product can only be scaled afterwards if
// those four words share a group.  At g = 128 they do; at g = 64 one v_permlane32_swap per
// register pair moves the second group's words into the upper registers; at g = 32 a
// further v_permlane16_swap per pair completes the 4x4 transpose so that register a holds
// word c of group a.  The activation vectors are read in the matching order:
//   g = 128: register a, lane row c -> unit word 4c + a
//   g = 64:  register a, lane row c -> unit word 8(a/2) + a%2 + 4(c%2) + 2(c/2)
//   g = 32:  register a, lane row c -> unit word 4a + c
//
// Dequantization as in the streaming kernel: the weight operand is the exact small integer
// u - z (q4_device.h), in natural column order for bf16 activations and in (i, i+4) pairs
// for fp16 ones, whose activation vectors are permuted to match.  Products are exact and
// the fp32 sums carry the only rounding.
//
// LDS (16-byte vectors): S x [m][UPW*16] activation slices | S x 64 x MQ partial sums.
#pragma once

#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>

#include "q4_device.h"

int q4k_device_cus();

namespace q4t {

constexpr int kOOB = 0x40000000;             // a buffer offset past every load resource: reads 0
constexpr uint32_t kStoreOOB = 0xFFFFFFF0u;  // a store offset past the y resource: dropped
constexpr int kLdsBudget = 96 * 1024;        // LDS per workgroup

constexpr int gcd8(int v) { return (v & 7) == 0 ? 8 : ((v & 3) == 0 ? 4 : ((v & 1) == 0 ? 2 : 1)); }

// NV consecutive dwords at byte offset off of resource rs (chunks of 4, 2, 1).  The whole
// offset is per-lane, so the range check covers every chunk (the last slice of the last
// row may reach past the buffer: those dwords read zero).
template <int NV>
__device__ __forceinline__ void load_dwords(q4::rsrc rs, int off, uint32_t (&v)[NV]) {
#pragma unroll
    for (int j = 0; j < NV / 4; ++j) {
        const q4::u32x4 t = q4::buf_load_x4(rs, off + 16 * j, 0);
        v[4 * j] = t[0];
        v[4 * j + 1] = t[1];
        v[4 * j + 2] = t[2];
        v[4 * j + 3] = t[3];
    }
    if constexpr (NV % 4 >= 2) {
        const q4::u32x2 t = q4::buf_load_x2(rs, off + 16 * (NV / 4), 0);
        v[NV / 4 * 4] = t[0];
        v[NV / 4 * 4 + 1] = t[1];
    }
    if constexpr (NV % 2 == 1) v[NV - 1] = q4::buf_load_x1(rs, off + 4 * (NV - 1), 0);
}

// Vector loads that load_dwords<nv> issues.
constexpr int dword_loads(int nv) { return nv / 4 + (nv % 4 >= 2 ? 1 : 0) + nv % 2; }

__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
    const auto t = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = t[0];
    b = t[1];
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
    const auto t = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = t[0];
    b = t[1];
}

template <int G, bool SYM, bool XF16, int UPW, int MQ, bool GROUPED>
__global__ __launch_bounds__(MQ == 1 ? 1024 : 512) void gemv_tile_kernel(const q4::GemvBatch bt, int M, int K) {
    constexpr int NG = 128 / G;                // groups per unit
    constexpr int RPG = 4 / NG;                // MFMAs (registers) per group
    constexpr int GPS = UPW * NG;              // groups per slice
    constexpr int XV = UPW >= 4 ? UPW / 4 : 1;  // activation vectors per lane per row of the slice
    constexpr int SV = GPS / 2;                // scale dwords per lane (two fp16 each)
    constexpr int ZOFF = GPS % 8 == 0 ? 0 : 8 - gcd8(GPS);  // largest nibble offset of a slice
    constexpr int ZV = (ZOFF + GPS + 7) / 8;   // zero-point words a slice can span
    constexpr int SLICE = UPW * 16;            // activation vectors per row of the slice
    extern __shared__ q4::u32x4 lds[];
    int pi = 0;
    if constexpr (GROUPED) {
#pragma unroll
        for (int i = 1; i < q4::kMaxGroup; ++i)
            if (i < bt.count && (int)blockIdx.x >= bt.p[i].tile0) pi = i;
    }
    const uint16_t* __restrict__ x = reinterpret_cast<const uint16_t*>(bt.p[pi].x);
    const uint32_t* __restrict__ qweight = bt.p[pi].qweight;
    const uint16_t* __restrict__ scales = bt.p[pi].scales;
    const uint32_t* __restrict__ zeros = bt.p[pi].zeros;
    void* __restrict__ y = bt.p[pi].y;
    const int ydt = bt.ydt;
    const int N = bt.p[pi].n;
    const int n0 = ((int)blockIdx.x - bt.p[pi].tile0) * 16;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int S = blockDim.x >> 6;
    const int r = lane & 15, c = lane >> 4;
    const int KW = K >> 3, units = K >> 7, ng = K / G, zw = (ng + 7) >> 3;
    const int rows = N - n0 < 16 ? N - n0 : 16;
    const int U0 = w * UPW;  // this wave's first unit
    const int G0 = U0 * NG;  // ... and first group
    const int nu = units - U0 < UPW ? units - U0 : UPW;

    // ---- prologue: every load of the wave, in the order it is waited for
    q4::u32x4 xv[MQ][XV];
    {
        const q4::rsrc rx = q4::make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
#pragma unroll
        for (int m = 0; m < MQ; ++m)
#pragma unroll
            for (int j = 0; j < XV; ++j) {
                // a two-unit slice has 32 vectors per row: lanes 32..63 repeat 0..31
                const int v = UPW >= 4 ? j * 64 + lane : (lane & 31);
                const int off = (m * K + U0 * 128 + v * 8) * 2;
                xv[m][j] = q4::buf_load_x4(rx, m < M ? off : kOOB, 0);
            }
    }
    uint32_t sv[SV];
    {
        const q4::rsrc rs = q4::make_rsrc(scales + (int64_t)n0 * ng, (uint32_t)rows * ng * 2u);
        load_dwords<SV>(rs, r < rows ? (r * ng + G0) * 2 : kOOB, sv);
    }
    uint32_t zv[ZV] = {};
    if constexpr (!SYM) {
        const q4::rsrc rz = q4::make_rsrc(zeros + (int64_t)n0 * zw, (uint32_t)rows * zw * 4u);
        load_dwords<ZV>(rz, r < rows ? (r * zw + (G0 >> 3)) * 4 : kOOB, zv);
    }
    q4::u32x4 wv[UPW];
    {
        const q4::rsrc rq = q4::make_rsrc(qweight + (int64_t)n0 * KW, (uint32_t)rows * KW * 4u);
        const int qo = r < rows ? r * KW * 4 + c * 16 : kOOB;
#pragma unroll
        for (int u = 0; u < UPW; ++u) wv[u] = q4::buf_load_x4(rq, u < nu ? qo : kOOB, (U0 + u) * 64);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- operand route.  fp16 activations use the exact fp16 decode.  bf16 activations
    // use the split fp16 decode when the nonzero exponents of the wave's slice span at most
    // 25 binades (q4_device.h): the slice is staged as exact fp16 values (x * 2^xs, the odd
    // columns of each word divided by 16 more) and the wave's sums are scaled back by
    // 2^-xs.  Otherwise (a wider range, subnormal or non-finite values) the wave takes the
    // exact bf16 decode.  Both routes multiply exact operands.
    bool f16r = XF16;
    int xs = 0;
    if constexpr (!XF16) {
        // rows past m read zeros, which leave both extremes alone
        q4::u16x2 hi = {0, 0}, lo = {0xFFFF, 0xFFFF};
#pragma unroll
        for (int m = 0; m < MQ; ++m)
#pragma unroll
            for (int j = 0; j < XV; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) q4::bf16_mag_range(xv[m][j][e], hi, lo);
        // largest magnitude in the low half, 0xFFFF - (smallest nonzero magnitude - 1) in
        // the high half: one maximum over the wave gives both
        const uint32_t hm = hi[0] > hi[1] ? hi[0] : hi[1];
        const uint32_t lm = lo[0] < lo[1] ? lo[0] : lo[1];
        const uint32_t red = q4::wave_max_u16x2(hm | ((0xFFFFu - lm) << 16));
        const int rr = __builtin_amdgcn_readfirstlane((int)red);
        const int emax = (rr & 0xFFFF) >> 7;                              // 0: every value is zero
        const int emin = (int)((0xFFFFu - ((uint32_t)rr >> 16)) + 1u) >> 7;  // smallest nonzero
        // bitwise, not short-circuit: no branch may split the block the loads sit in
        f16r = (emax == 0) | ((emax <= 254) & (emin >= 1) & (emax - emin <= 25));
        xs = f16r && emax != 0 ? 142 - emax : 0;  // the bf16 route leaves x unscaled
    }

    // ---- this wave's activation slice into its LDS region, in the decoder's slot order.
    // Rows m..MQ-1 (zeros) go to this wave's partial-sum slots, which it overwrites later:
    // no store (and so no load) sits behind a branch.  The fp16 form is computed either
    // way and selected: a branch here would let the compiler sink the weight loads issued
    // above below it, behind the wait for the activations and the range reduction.
    q4::u32x4* xw = lds + w * (M * SLICE);
    q4::u32x4* spare = lds + S * M * SLICE + w * 64 + lane;
#pragma unroll
    for (int m = 0; m < MQ; ++m)
#pragma unroll
        for (int j = 0; j < XV; ++j) {
            q4::u32x4* dst = xw + m * SLICE + (UPW >= 4 ? j * 64 + lane : (lane & 31));
            q4::u32x4 v = xv[m][j];
            if constexpr (XF16) {
                v = q4::pair_perm(v);
            } else {
                const q4::u32x4 h = q4::bf16_to_f16_split(v, xs);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = f16r ? h[e] : v[e];
            }
            *(m == 0 || m < M ? dst : spare) = v;
        }

    // zero points of the slice's groups from nibble 0 on (a slice may start mid-word)
    uint32_t zs[ZV];
#pragma unroll
    for (int j = 0; j < ZV; ++j) zs[j] = zv[j];
    if constexpr (!SYM && ZOFF != 0) {
        const uint32_t sh = 4u * (uint32_t)(G0 & 7);
#pragma unroll
        for (int j = 0; j + 1 < ZV; ++j) zs[j] = __builtin_amdgcn_alignbit(zv[j + 1], zv[j], sh);
        zs[ZV - 1] = zv[ZV - 1] >> sh;
    }

    // ---- dequantize and multiply, one unit at a time, as the loads land
    const int mrow = r < M ? r : M - 1;
    const int lb = G == 128 ? 4 * c : (G == 64 ? 4 * (c & 1) + 2 * (c >> 1) : c);
    const q4::u32x4* xr = xw + mrow * SLICE + lb;
    float acc[MQ];
#pragma unroll
    for (int q = 0; q < MQ; ++q) acc[q] = 0.f;
    const uint32_t kMask = q4::vreg_const(0x000F000Fu);
    const uint32_t kMaskHi = q4::vreg_const(0x00F000F0u);
    const uint32_t kMagic = q4::vreg_const(0x64006400u);
    auto slice = [&](auto route) {
    constexpr bool F16 = decltype(route)::value;
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
        const bool valid = u < nu;
        uint32_t wq[4] = {wv[u][0], wv[u][1], wv[u][2], wv[u][3]};
        if constexpr (G <= 64) {
            swap32(wq[0], wq[2]);
            swap32(wq[1], wq[3]);
        }
        if constexpr (G == 32) {
            swap16(wq[0], wq[1]);
            swap16(wq[2], wq[3]);
        }
        q4::u32x4 xa[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int imm = G == 128 ? a : (G == 64 ? 8 * (a >> 1) + (a & 1) : 4 * a);
            xa[a] = xr[u * 16 + imm];
        }
#pragma unroll
        for (int h = 0; h < NG; ++h) {
            const int gi = u * NG + h;  // group within the slice
            const uint32_t sw = sv[gi >> 1];
            const float s = q4::f16_bits_to_float((uint16_t)((gi & 1) ? (sw >> 16) : sw));
            int z = 8;
            if constexpr (!SYM) z = (int)((zs[gi >> 3] >> (4 * (gi & 7))) & 0xFu);
            q4::f32x4 dv = {0.f, 0.f, 0.f, 0.f};
            if constexpr (XF16) {
                const q4::f16x2 bias = q4::f16_bias_pair((uint32_t)z);
#pragma unroll
                for (int t = 0; t < RPG; ++t) {
                    const int a = h * RPG + t;
                    dv = q4::mfma_f16(xa[a], q4::decode_f16_exact(wq[a], bias, kMask, kMagic), dv);
                }
            } else if constexpr (F16) {
                const q4::f16x2 bias_lo = q4::f16_bias_pair((uint32_t)z);
                const q4::f16x2 bias_hi = q4::f16_bias_pair((uint32_t)z << 4);
#pragma unroll
                for (int t = 0; t < RPG; ++t) {
                    const int a = h * RPG + t;
                    dv = q4::mfma_f16(xa[a], q4::decode_f16_split(wq[a], bias_lo, bias_hi, kMask, kMaskHi, kMagic), dv);
                }
            } else {
                const uint32_t zb = q4::bf16_zero_bias(z);
#pragma unroll
                for (int t = 0; t < RPG; ++t) {
                    const int a = h * RPG + t;
                    dv = q4::mfma_bf16(xa[a], q4::decode_bf16_exact(wq[a], zb), dv);
                }
            }
#pragma unroll
            for (int q = 0; q < MQ; ++q) acc[q] = valid ? acc[q] + s * dv[q] : acc[q];
        }
    }
    };
    if constexpr (XF16) {
        slice(std::true_type{});
    } else {
        if (f16r)
            slice(std::true_type{});
        else
            slice(std::false_type{});
#pragma unroll
        for (int q = 0; q < MQ; ++q) acc[q] = __builtin_amdgcn_ldexpf(acc[q], -xs);
    }

    // ---- cross-wave sum (lanes 0..15 hold rows m = 0..MQ-1 of the tile's 16 columns)
    float* red = reinterpret_cast<float*>(lds + S * M * SLICE);
#pragma unroll
    for (int q = 0; q < MQ; ++q) red[(w * 64 + lane) * MQ + q] = acc[q];
    __syncthreads();
    if (w == 0) {
        float sum[MQ];
#pragma unroll
        for (int q = 0; q < MQ; ++q) sum[q] = 0.f;
        for (int v = 0; v < S; ++v)
#pragma unroll
            for (int q = 0; q < MQ; ++q) sum[q] += red[(v * 64 + lane) * MQ + q];
        const q4::rsrc ry = q4::make_rsrc(y, (uint32_t)M * (uint32_t)N * q4::y_bytes(ydt));
#pragma unroll
        for (int q = 0; q < MQ; ++q) {
            const bool st = lane < 16 && q < M && r < rows;
            const uint32_t off = st ? ((uint32_t)q * (uint32_t)N + (uint32_t)(n0 + r)) * q4::y_bytes(ydt) : kStoreOOB;
            q4::store_y(ry, off, sum[q], ydt);
        }
    }
}

// Wide tile kernel: m <= 16 (4 < m, and the m <= 4 shapes the tile kernel cannot take).
// Same tiles, slices and metadata as the tile kernel; the activations, m x K of which do
// not fit in LDS for the larger projections, stream through a small wave-private LDS ring
// instead.  The wave keeps two batches of D units in flight: per unit, MR/4 direct-to-LDS
// loads of its activations (MR = 4, 8 or 16 rows; rows past m read nothing) and one load
// of its packed words into registers.  Each direct load moves 4 whole rows x 256 bytes
// (coalesced): lane l writes row 4a + l/16, position l%16 of that row, and fetches chunk
// (l%16) ^ row into it, so that the MFMA-layout reads afterwards (16 rows at one chunk
// index) hit 16 different bank groups.  Before a batch is read the wave waits for its
// loads with a fixed count (the next batch's loads stay in flight); once it is computed,
// its slots take the batch two ahead.  All 16 MFMA rows are activation rows (rows past m
// read row m-1 and are never stored), so every lane holds four outputs.
template <int G, bool SYM, bool XF16, int UPW, int MR, int D, int T, bool GROUPED>
__global__ __launch_bounds__(512) void gemv_wide_kernel(const q4::GemvBatch bt, int M, int K) {
    constexpr int NB = UPW / D;     // batches per slice (at least two)
    constexpr int NG = 128 / G, RPG = 4 / NG, GPS = UPW * NG, SV = GPS / 2;
    constexpr int ZOFF = GPS % 8 == 0 ? 0 : 8 - gcd8(GPS);
    constexpr int ZV = (ZOFF + GPS + 7) / 8;
    constexpr int XR = MR / 4;                   // direct loads per unit
    constexpr int UNIT_LDS = MR * 256;           // bytes of one unit's activations
    constexpr int WAVE_LDS = 2 * D * UNIT_LDS;   // this wave's ring
    constexpr int PER_BATCH = D * (XR + T);      // vector loads per batch
    constexpr int WAIT_NEXT = (PER_BATCH & 15) | ((PER_BATCH >> 4) << 14) | (0x7 << 4) | (0xF << 8);
    constexpr int WAIT_ALL = (0x7 << 4) | (0xF << 8);   // vmcnt(0)
    constexpr int WAIT_LDS = 0xF | (0x3 << 14) | (0x7 << 4);  // lgkmcnt(0)
    static_assert(T * 1024 <= WAVE_LDS, "partial sums fit the ring");
    extern __shared__ q4::u32x4 lds[];
    int pi = 0;
    if constexpr (GROUPED) {
#pragma unroll
        for (int i = 1; i < q4::kMaxGroup; ++i)
            if (i < bt.count && (int)blockIdx.x >= bt.p[i].tile0) pi = i;
    }
    const uint16_t* __restrict__ x = reinterpret_cast<const uint16_t*>(bt.p[pi].x);
    const uint32_t* __restrict__ qweight = bt.p[pi].qweight;
    const uint16_t* __restrict__ scales = bt.p[pi].scales;
    const uint32_t* __restrict__ zeros = bt.p[pi].zeros;
    void* __restrict__ y = bt.p[pi].y;
    const int ydt = bt.ydt;
    const int N = bt.p[pi].n;
    const int n0 = ((int)blockIdx.x - bt.p[pi].tile0) * 16 * T;  // T tiles of 16 rows
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int S = blockDim.x >> 6;
    const int r = lane & 15, c = lane >> 4;
    const int KW = K >> 3, units = K >> 7, ng = K / G, zw = (ng + 7) >> 3;
    const int rows = N - n0 < 16 * T ? N - n0 : 16 * T;  // rows of the workgroup
    const int U0 = w * UPW, G0 = U0 * NG;
    const int nu = units - U0 < UPW ? units - U0 : UPW;
    uint8_t* ring = reinterpret_cast<uint8_t*>(lds) + w * WAVE_LDS;

    // ---- metadata of the slice, per tile (waited for before the first unit)
    uint32_t sv[T][SV];
    uint32_t zv[T][ZV] = {};
    {
        const q4::rsrc rs = q4::make_rsrc(scales + (int64_t)n0 * ng, (uint32_t)rows * ng * 2u);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int rr = 16 * t + r;
            load_dwords<SV>(rs, rr < rows ? (rr * ng + G0) * 2 : kOOB, sv[t]);
        }
        if constexpr (!SYM) {
            const q4::rsrc rz = q4::make_rsrc(zeros + (int64_t)n0 * zw, (uint32_t)rows * zw * 4u);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int rr = 16 * t + r;
                load_dwords<ZV>(rz, rr < rows ? (rr * zw + (G0 >> 3)) * 4 : kOOB, zv[t]);
            }
        }
    }

    // ---- loads of a batch: per unit the activation rows into the ring slot, then the
    // unit's packed words of each tile
    const q4::rsrc rx = q4::make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    uint32_t doff[XR];
#pragma unroll
    for (int a = 0; a < XR; ++a) {
        const int R = 4 * a + (lane >> 4);
        doff[a] = R < M ? (uint32_t)(R * K + 8 * ((lane & 15) ^ R)) * 2u : (uint32_t)kOOB;
    }
    const q4::rsrc rq = q4::make_rsrc(qweight + (int64_t)n0 * KW, (uint32_t)rows * KW * 4u);
    uint32_t qo[T];
#pragma unroll
    for (int t = 0; t < T; ++t) qo[t] = 16 * t + r < rows ? (uint32_t)((16 * t + r) * KW * 4 + c * 16) : (uint32_t)kOOB;
    q4::u32x4 wb[2][D][T];
    auto load_batch = [&](int b, q4::u32x4 (&ws)[D][T]) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int u = b * D + j;
            // slots past the slice read nothing: the mask goes into the per-lane offset
            const uint32_t pm = u < nu ? 0u : (uint32_t)kOOB;
            uint8_t* slot = ring + ((b & 1) * D + j) * UNIT_LDS;
#pragma unroll
            for (int a = 0; a < XR; ++a)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(slot + a * 1024),
                                                         16, (int)(doff[a] | pm), (U0 + u) * 256, 0, 0);
#pragma unroll
            for (int t = 0; t < T; ++t) ws[j][t] = q4::buf_load_x4(rq, (int)(qo[t] | pm), (U0 + u) * 64);
        }
    };
    // the metadata, batch 0 and batch 1 are issued in this order: the fixed wait counts
    // below depend on it
    __builtin_amdgcn_sched_barrier(0);
    load_batch(0, wb[0]);
    __builtin_amdgcn_sched_barrier(0);
    load_batch(1, wb[1]);
    __builtin_amdgcn_sched_barrier(0);

    uint32_t zs[T][ZV];
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int j = 0; j < ZV; ++j) zs[t][j] = zv[t][j];
        if constexpr (!SYM && ZOFF != 0) {
            const uint32_t sh = 4u * (uint32_t)(G0 & 7);
#pragma unroll
            for (int j = 0; j + 1 < ZV; ++j) zs[t][j] = __builtin_amdgcn_alignbit(zv[t][j + 1], zv[t][j], sh);
            zs[t][ZV - 1] = zv[t][ZV - 1] >> sh;
        }
    }

    // read addresses: row min(l%16, m-1), chunk lb + imm(a) at its swizzled position
    const int mrow = r < M ? r : M - 1;
    const int lb = G == 128 ? 4 * c : (G == 64 ? 4 * (c & 1) + 2 * (c >> 1) : c);
    uint32_t xaddr[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int imm = G == 128 ? a : (G == 64 ? 8 * (a >> 1) + (a & 1) : 4 * a);
        xaddr[a] = (uint32_t)(mrow * 256 + (((lb + imm) ^ mrow) << 4));
    }

    const uint32_t kMask = q4::vreg_const(0x000F000Fu);
    const uint32_t kMagic = q4::vreg_const(0x64006400u);
    float acc[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[t][q] = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int slot = b & 1;
        // this batch's loads have landed (the next batch's stay in flight)
        if (b + 1 < NB)
            __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
        else
            __builtin_amdgcn_s_waitcnt(WAIT_ALL);
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int u = b * D + j;
            const bool valid = u < nu;
            const uint8_t* sb = ring + (slot * D + j) * UNIT_LDS;
            q4::u32x4 xa[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const q4::u32x4 v = *reinterpret_cast<const q4::u32x4*>(sb + xaddr[a]);
                xa[a] = XF16 ? q4::pair_perm(v) : v;
            }
#pragma unroll
            for (int t = 0; t < T; ++t) {
                uint32_t wq[4] = {wb[slot][j][t][0], wb[slot][j][t][1], wb[slot][j][t][2], wb[slot][j][t][3]};
                if constexpr (G <= 64) {
                    swap32(wq[0], wq[2]);
                    swap32(wq[1], wq[3]);
                }
                if constexpr (G == 32) {
                    swap16(wq[0], wq[1]);
                    swap16(wq[2], wq[3]);
                }
#pragma unroll
                for (int h = 0; h < NG; ++h) {
                    const int gi = u * NG + h;
                    const uint32_t sw = sv[t][gi >> 1];
                    const float s = q4::f16_bits_to_float((uint16_t)((gi & 1) ? (sw >> 16) : sw));
                    int z = 8;
                    if constexpr (!SYM) z = (int)((zs[t][gi >> 3] >> (4 * (gi & 7))) & 0xFu);
                    q4::f32x4 dv = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (XF16) {
                        const q4::f16x2 bias = q4::f16_bias_pair((uint32_t)z);
#pragma unroll
                        for (int e = 0; e < RPG; ++e) {
                            const int a = h * RPG + e;
                            dv = q4::mfma_f16(xa[a], q4::decode_f16_exact(wq[a], bias, kMask, kMagic), dv);
                        }
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[t][q] = valid ? acc[t][q] + s * dv[q] : acc[t][q];
                    } else {
                        const uint32_t zb = q4::bf16_zero_bias(z);
#pragma unroll
                        for (int e = 0; e < RPG; ++e) {
                            const int a = h * RPG + e;
                            dv = q4::mfma_bf16(xa[a], q4::decode_bf16_exact(wq[a], zb), dv);
                        }
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[t][q] = valid ? acc[t][q] + s * dv[q] : acc[t][q];
                    }
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // refill these slots with the batch two ahead once every read of them has returned
        if (b + 2 < NB) {
            __builtin_amdgcn_s_waitcnt(WAIT_LDS);
            load_batch(b + 2, wb[slot]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- cross-wave sum: lane l holds rows m = 4(l/16)..+3 of column l%16 of each tile.
    // Each wave writes into its own ring (its loads have all landed and been read).
    __builtin_amdgcn_s_waitcnt(WAIT_LDS);
    float* red = reinterpret_cast<float*>(ring);
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[(t * 64 + lane) * 4 + q] = acc[t][q];
    __syncthreads();
    if (w == 0) {
        const q4::rsrc ry = q4::make_rsrc(y, (uint32_t)M * (uint32_t)N * q4::y_bytes(ydt));
#pragma unroll
        for (int t = 0; t < T; ++t) {
            float sum[4] = {0.f, 0.f, 0.f, 0.f};
            for (int v = 0; v < S; ++v) {
                const float* rv = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(lds) + v * WAVE_LDS);
#pragma unroll
                for (int q = 0; q < 4; ++q) sum[q] += rv[(t * 64 + lane) * 4 + q];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = 4 * c + q;
                const bool st = m < M && 16 * t + r < rows;
                const uint32_t off = st ? ((uint32_t)m * (uint32_t)N + (uint32_t)(n0 + 16 * t + r)) * q4::y_bytes(ydt) : kStoreOOB;
                q4::store_y(ry, off, sum[q], ydt);
            }
        }
    }
}

// Resident kernel (8 < m <= 16, all m x K activations within the LDS budget, at least two
// tiles per workgroup): persistent workgroups.  Each workgroup stages the whole of x into
// LDS once, with direct-to-LDS loads of 4 whole rows x 256 bytes swizzled exactly as in the
// wide kernel's ring (unit u, row R: chunk c at position c ^ R), and then serves tiles
// b, b + P, b + 2P, ... of the batch (P workgroups).  Per tile, wave w takes units
// [w*UPW, w*UPW + nu) of the tile's 16 rows as in the tile kernel.  Before computing a tile
// it issues every load of its slice of the next one (into a second register set; offsets
// past the buffers when there is no next tile, so the wait counts never depend on a
// branch), which keeps one tile's weights in flight per wave.  The cross-wave sums of
// consecutive tiles alternate between two LDS regions, so one barrier per tile orders
// them.  Each staged activation byte feeds every tile the workgroup serves, where the wide
// kernel stages all of x again for each 16-row tile: at m = 16 the wide kernel moves four
// activation bytes through each CU's memory pipeline per weight byte.  With one tile per
// workgroup, or m <= 8, the wide kernel measured faster (the staging is not shared, or is
// small, and one workgroup per CU hides less latency than the wide kernel's two).
template <int G, bool SYM, bool XF16, int UPW, bool GROUPED>
__global__ __launch_bounds__(512) void gemv_resident_kernel(const q4::GemvBatch bt, int M, int K, int tiles) {
    constexpr int NG = 128 / G, RPG = 4 / NG, GPS = UPW * NG, SV = GPS / 2;
    constexpr int ZOFF = GPS % 8 == 0 ? 0 : 8 - gcd8(GPS);
    constexpr int ZV = (ZOFF + GPS + 7) / 8;
    constexpr int MR = 16;              // activation rows staged per unit (rows past m read nothing)
    constexpr int UNIT_LDS = MR * 256;  // bytes of one unit's activation rows
    // vector loads per tile and wave, in issue order: scales, zero points, packed words
    constexpr int nvec = dword_loads(SV) + (SYM ? 0 : dword_loads(ZV)) + UPW;
    static_assert(nvec < 64, "vmcnt range");
    constexpr int WAIT_TILE = (nvec & 15) | ((nvec >> 4) << 14) | (0x7 << 4) | (0xF << 8);  // vmcnt(nvec)
    constexpr int WAIT_ALL = (0x7 << 4) | (0xF << 8);                                         // vmcnt(0)
    extern __shared__ q4::u32x4 lds[];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int S = blockDim.x >> 6;
    const int P = gridDim.x;
    const int r = lane & 15, c = lane >> 4;
    const int KW = K >> 3, units = K >> 7, ng = K / G, zw = (ng + 7) >> 3;
    const int U0 = w * UPW, G0 = U0 * NG;
    const int nu = units - U0 < UPW ? units - U0 : UPW;
    uint8_t* xs = reinterpret_cast<uint8_t*>(lds);
    float* red = reinterpret_cast<float*>(xs + units * UNIT_LDS);  // 2 regions of S x 64 x 4

    // ---- every activation row of the batch's shared x into LDS: units * MR/4 loads of 1 KB,
    // dealt round-robin to the waves.  Rows past m read nothing (and are never read back).
    {
        const q4::rsrc rx = q4::make_rsrc(bt.p[0].x, (uint32_t)M * (uint32_t)K * 2u);
        const int nl = units * (MR / 4);
        for (int j = w; j < nl; j += S) {
            const int u = j / (MR / 4), a = j % (MR / 4);
            const int R = 4 * a + (lane >> 4);
            const uint32_t off = R < M ? (uint32_t)(R * K + u * 128 + 8 * ((lane & 15) ^ R)) * 2u : (uint32_t)kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void*)(xs + u * UNIT_LDS + a * 1024), 16, (int)off, 0, 0, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    struct Set {
        uint32_t sv[SV];
        uint32_t zv[ZV];
        q4::u32x4 wv[UPW];
    };
    // problem and first row of tile t (t < tiles)
    auto locate = [&](int t, int& pi, int& n0) {
        pi = 0;
        if constexpr (GROUPED) {
#pragma unroll
            for (int i = 1; i < q4::kMaxGroup; ++i)
                if (i < bt.count && t >= bt.p[i].tile0) pi = i;
        }
        n0 = (t - bt.p[pi].tile0) * 16;
    };
    // every load of this wave's slice of tile t; nothing is read when t >= tiles
    auto issue = [&](int t, Set& s) {
        const bool live = t < tiles;
        int pi, n0;
        locate(live ? t : 0, pi, n0);
        const int N = bt.p[pi].n;
        const int rows = N - n0 < 16 ? N - n0 : 16;
        const bool lr = live && r < rows;
        const q4::rsrc rs = q4::make_rsrc(bt.p[pi].scales + (int64_t)n0 * ng, (uint32_t)rows * ng * 2u);
        load_dwords<SV>(rs, lr ? (r * ng + G0) * 2 : kOOB, s.sv);
        if constexpr (!SYM) {
            const q4::rsrc rz = q4::make_rsrc(bt.p[pi].zeros + (int64_t)n0 * zw, (uint32_t)rows * zw * 4u);
            load_dwords<ZV>(rz, lr ? (r * zw + (G0 >> 3)) * 4 : kOOB, s.zv);
        } else {
#pragma unroll
            for (int j = 0; j < ZV; ++j) s.zv[j] = 0;
        }
        const q4::rsrc rq = q4::make_rsrc(bt.p[pi].qweight + (int64_t)n0 * KW, (uint32_t)rows * KW * 4u);
        const int qo = lr ? r * KW * 4 + c * 16 : kOOB;
#pragma unroll
        for (int u = 0; u < UPW; ++u) s.wv[u] = q4::buf_load_x4(rq, u < nu ? qo : kOOB, (U0 + u) * 64);
    };

    // read addresses: row min(l%16, m-1), chunk lb + imm(a) at its swizzled position
    const int mrow = r < M ? r : M - 1;
    const int lb = G == 128 ? 4 * c : (G == 64 ? 4 * (c & 1) + 2 * (c >> 1) : c);
    uint32_t xaddr[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int imm = G == 128 ? a : (G == 64 ? 8 * (a >> 1) + (a & 1) : 4 * a);
        xaddr[a] = (uint32_t)(mrow * 256 + (((lb + imm) ^ mrow) << 4));
    }
    const uint32_t kMask = q4::vreg_const(0x000F000Fu);
    const uint32_t kMagic = q4::vreg_const(0x64006400u);

    // dequantize, multiply and sum tile t from set s; cross-wave sum in region par
    auto compute = [&](int t, Set& s, int par) {
        uint32_t zs[ZV];
#pragma unroll
        for (int j = 0; j < ZV; ++j) zs[j] = s.zv[j];
        if constexpr (!SYM && ZOFF != 0) {
            const uint32_t sh = 4u * (uint32_t)(G0 & 7);
#pragma unroll
            for (int j = 0; j + 1 < ZV; ++j) zs[j] = __builtin_amdgcn_alignbit(s.zv[j + 1], s.zv[j], sh);
            zs[ZV - 1] = s.zv[ZV - 1] >> sh;
        }
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < UPW; ++u) {
            const bool valid = u < nu;
            // slots past the slice read a staged unit (their products are discarded)
            const uint8_t* sb = xs + (valid ? U0 + u : 0) * UNIT_LDS;
            q4::u32x4 xa[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const q4::u32x4 v = *reinterpret_cast<const q4::u32x4*>(sb + xaddr[a]);
                xa[a] = XF16 ? q4::pair_perm(v) : v;
            }
            uint32_t wq[4] = {s.wv[u][0], s.wv[u][1], s.wv[u][2], s.wv[u][3]};
            if constexpr (G <= 64) {
                swap32(wq[0], wq[2]);
                swap32(wq[1], wq[3]);
            }
            if constexpr (G == 32) {
                swap16(wq[0], wq[1]);
                swap16(wq[2], wq[3]);
            }
#pragma unroll
            for (int h = 0; h < NG; ++h) {
                const int gi = u * NG + h;
                const uint32_t sw = s.sv[gi >> 1];
                const float sc = q4::f16_bits_to_float((uint16_t)((gi & 1) ? (sw >> 16) : sw));
                int z = 8;
                if constexpr (!SYM) z = (int)((zs[gi >> 3] >> (4 * (gi & 7))) & 0xFu);
                q4::f32x4 dv = {0.f, 0.f, 0.f, 0.f};
                if constexpr (XF16) {
                    const q4::f16x2 bias = q4::f16_bias_pair((uint32_t)z);
#pragma unroll
                    for (int e = 0; e < RPG; ++e) {
                        const int a = h * RPG + e;
                        dv = q4::mfma_f16(xa[a], q4::decode_f16_exact(wq[a], bias, kMask, kMagic), dv);
                    }
                } else {
                    const uint32_t zb = q4::bf16_zero_bias(z);
#pragma unroll
                    for (int e = 0; e < RPG; ++e) {
                        const int a = h * RPG + e;
                        dv = q4::mfma_bf16(xa[a], q4::decode_bf16_exact(wq[a], zb), dv);
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] = valid ? acc[q] + sc * dv[q] : acc[q];
            }
        }
        // lane l holds rows m = 4(l/16)..+3 of the tile's column l%16
        float* rd = red + par * (S * 256);
#pragma unroll
        for (int q = 0; q < 4; ++q) rd[(w * 64 + lane) * 4 + q] = acc[q];
        __syncthreads();
        if (w == 0) {
            int pi, n0;
            locate(t, pi, n0);
            const int N = bt.p[pi].n;
            const int rows = N - n0 < 16 ? N - n0 : 16;
            float sum[4] = {0.f, 0.f, 0.f, 0.f};
            for (int v = 0; v < S; ++v)
#pragma unroll
                for (int q = 0; q < 4; ++q) sum[q] += rd[(v * 64 + lane) * 4 + q];
            const q4::rsrc ry = q4::make_rsrc(bt.p[pi].y, (uint32_t)M * (uint32_t)N * q4::y_bytes(bt.ydt));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = 4 * c + q;
                const bool st = m < M && r < rows;
                const uint32_t off = st ? ((uint32_t)m * (uint32_t)N + (uint32_t)(n0 + r)) * q4::y_bytes(bt.ydt) : kStoreOOB;
                q4::store_y(ry, off, sum[q], bt.ydt);
            }
        }
    };

    // Tiles t0, t0 + P, ... of this workgroup, in pairs: while one tile is computed the
    // next one's loads are in flight.  The loop body has no exit, so the loads pending at its
    // back edge are always exactly one register set's (a loop that could leave between the
    // two halves makes the compiler wait for every load at its top, and then only one tile
    // at a time is in flight).  Keeping more tiles in flight (two groups of two sets) was
    // measured slower: the weights of later tiles queue in the memory pipeline ahead of the
    // current one's.
    const int nt = (tiles - (int)blockIdx.x + P - 1) / P;
    Set A, B;
    int t = blockIdx.x;
    issue(t, A);
    __builtin_amdgcn_sched_barrier(0);
    // the activations (issued first) have landed once at most this tile's loads are
    // outstanding; the barrier makes every wave's share visible
    __builtin_amdgcn_s_waitcnt(WAIT_TILE);
    __syncthreads();
    for (int i = 0; i + 1 < nt; i += 2) {
        issue(t + P, B);
        __builtin_amdgcn_sched_barrier(0);
        compute(t, A, 0);
        t += P;
        issue(t + P, A);  // past the last tile when nt is even: reads nothing
        __builtin_amdgcn_sched_barrier(0);
        compute(t, B, 1);
        t += P;
    }
    if (nt & 1) compute(t, A, 0);
    // loads past the buffers retire before the wave ends
    __builtin_amdgcn_s_waitcnt(WAIT_ALL);
}

// LDS of the resident kernel: the staged activations (units x 16 rows x 256 bytes) and two
// regions of cross-wave sums.
inline size_t resident_lds(int k, int waves) { return (size_t)(k / 128) * 16 * 256 + (size_t)2 * waves * 64 * 16; }
constexpr size_t kResidentLdsMax = 160 * 1024;  // LDS per workgroup on gfx950
// The resident kernel's shape: 8 < m <= 16; slices of 4 or 8 units over at most 8 waves
// (the shape nearest eight waves); K a multiple of 128 with an even number of groups per
// row; the activations within the LDS budget; and at least two tiles for every workgroup
// the CUs hold at that LDS size.
inline bool resident_shape(int g, int m, int k, int tiles, int num_cus, int* upw, int* waves) {
    if (m <= 8 || m > 16 || k % 128 != 0 || (k / g) % 2 != 0) return false;
    const int units = k / 128;
    *upw = 0;
    for (int u : {4, 8}) {
        const int sw = (units + u - 1) / u;
        if (sw > 8) continue;
        if (*upw == 0 || (8 - sw) * 4096 + (sw * u - units) < (8 - *waves) * 4096 + (*waves * *upw - units)) {
            *upw = u;
            *waves = sw;
        }
    }
    if (*upw == 0) return false;
    const size_t lds = resident_lds(k, *waves);
    if (lds > kResidentLdsMax) return false;
    const int slots = (num_cus > 0 ? num_cus : 256) * (int)(kResidentLdsMax / lds);
    return tiles >= 2 * slots;
}

// LDS of the wide kernel per workgroup: each wave's ring of two batches of D units.
constexpr int wide_rows(int m) { return m <= 4 ? 4 : (m <= 8 ? 8 : 16); }
constexpr int wide_batch(int m) { return m <= 8 ? 2 : 1; }
inline size_t wide_lds(int m, int waves) { return (size_t)waves * 2 * wide_batch(m) * wide_rows(m) * 256; }
// Two tiles per workgroup when the halved grid still holds two tiles per CU.
inline bool wide_pair(int tiles, int num_cus) { return tiles >= 4 * (num_cus > 0 ? num_cus : 256); }

// Slice widths per group size (the g = 32 and g = 64 metadata registers grow with the
// slice; these stay within the launch bounds' register budgets).
constexpr int kMaxUpw128 = 16, kMaxUpw64 = 12, kMaxUpw32 = 8;

// The tile kernel's shape: S slices of UPW units (UPW in {2, 4, 8, 12, 16} up to the group
// size's maximum; S = ceil(units / UPW) waves, at most 16 for m = 1 and 8 otherwise, the
// kernel's launch bound), K a multiple of 128, an even number of groups per row (scales are
// read as dwords) and activations within the LDS budget.  Among the shapes that fit, the
// one nearest the target wave count wins, then the one with fewer idle slots.  The target
// is eight waves while one round of eight-wave workgroups holds every tile (the arithmetic
// of a tile spreads over more SIMDs and the tail after the last load is short), four when
// the tiles need several rounds (more loads in flight per wave, less per-workgroup
// overhead per byte).  Returns false when no shape fits.
inline bool tile_shape(int g, int m, int k, int tiles, int num_cus, int* upw, int* waves) {
    if (m > 4 || k % 128 != 0 || (k / g) % 2 != 0) return false;
    const int units = k / 128, mq = m <= 1 ? 1 : 4, max_waves = mq == 1 ? 16 : 8;
    const int max_upw = g == 128 ? kMaxUpw128 : (g == 64 ? kMaxUpw64 : kMaxUpw32);
    const int target = tiles > 4 * (num_cus > 0 ? num_cus : 256) ? 4 : 8;
    *upw = 0;
    auto key = [&](int uu, int ww) {  // smaller is better
        return (ww > target ? ww - target : target - ww) * 4096 + (ww * uu - units);
    };
    for (int u : {2, 4, 8, 12, 16}) {
        const int sw = (units + u - 1) / u;
        if (u > max_upw || sw > max_waves ||
            (size_t)m * sw * u * 256 + (size_t)sw * 64 * mq * 4 > (size_t)kLdsBudget)
            continue;
        if (*upw == 0 || key(u, sw) < key(*upw, *waves)) {
            *upw = u;
            *waves = sw;
        }
    }
    return *upw != 0;
}

// The wide kernel's shape (m <= 16; it serves 4 < m and the m <= 4 shapes the tile kernel
// cannot take): slices of 4, 8, 12 or 16 units, S = ceil(units / UPW) <= 8 waves, K a
// multiple of 128 and an even number of groups per row; the shape nearest eight waves with
// the fewest idle slots.
inline bool wide_shape(int g, int m, int k, int* upw, int* waves) {
    if (m < 1 || m > 16 || k % 128 != 0 || (k / g) % 2 != 0) return false;
    const int units = k / 128;
    *upw = 0;
    for (int u : {4, 8, 12, 16}) {
        const int sw = (units + u - 1) / u;
        if (sw > 8) continue;
        auto key = [&](int uu, int ww) { return (8 - ww) * 4096 + (ww * uu - units); };
        if (*upw == 0 || key(u, sw) < key(*upw, *waves)) {
            *upw = u;
            *waves = sw;
        }
    }
    return *upw != 0;
}

template <int G, bool SYM, bool XF16, bool GR, int U>
hipError_t launch_upw(int mq, dim3 grid, dim3 block, size_t lds, hipStream_t st,
                      const q4::GemvBatch& bt, int m, int k) {
    if (mq == 1)
        hipLaunchKernelGGL((gemv_tile_kernel<G, SYM, XF16, U, 1, GR>), grid, block, lds, st, bt, m, k);
    else
        hipLaunchKernelGGL((gemv_tile_kernel<G, SYM, XF16, U, 4, GR>), grid, block, lds, st, bt, m, k);
    return q4k_launched(XF16 ? "q4_gemv_tile_f16" : "q4_gemv_tile_bf16");
}

template <int G, bool SYM, bool XF16, bool GR>
hipError_t launch_x(int upw, int mq, dim3 grid, dim3 block, size_t lds, hipStream_t st,
                    const q4::GemvBatch& bt, int m, int k) {
    switch (upw) {
    case 2: return launch_upw<G, SYM, XF16, GR, 2>(mq, grid, block, lds, st, bt, m, k);
    case 4: return launch_upw<G, SYM, XF16, GR, 4>(mq, grid, block, lds, st, bt, m, k);
    case 8: return launch_upw<G, SYM, XF16, GR, 8>(mq, grid, block, lds, st, bt, m, k);
    case 12:
        if constexpr (G >= 64) return launch_upw<G, SYM, XF16, GR, 12>(mq, grid, block, lds, st, bt, m, k);
        break;
    case 16:
        if constexpr (G == 128) return launch_upw<G, SYM, XF16, GR, 16>(mq, grid, block, lds, st, bt, m, k);
        break;
    default: break;
    }
    return hipErrorInvalidValue;
}

template <int G, bool SYM, bool XF16, bool GR, int MR, int T>
hipError_t launch_wide_rows(int upw, dim3 grid, dim3 block, size_t lds, hipStream_t st,
                            const q4::GemvBatch& bt, int m, int k) {
    constexpr int D = MR <= 8 ? 2 : 1;
    static_assert(D == wide_batch(MR), "ring shape");
#define Q4_WIDE(U)                                                                                          \
    if (upw == U) {                                                                                         \
        hipLaunchKernelGGL((gemv_wide_kernel<G, SYM, XF16, U, MR, D, T, GR>), grid, block, lds, st, bt, m, k); \
        return q4k_launched(XF16 ? "q4_gemv_wide_f16" : "q4_gemv_wide_bf16");                               \
    }
    Q4_WIDE(4) Q4_WIDE(8) Q4_WIDE(12) Q4_WIDE(16)
#undef Q4_WIDE
    return hipErrorInvalidValue;
}

template <int G, bool SYM, bool XF16, bool GR>
hipError_t launch_wide(int upw, int pair, dim3 grid, dim3 block, size_t lds, hipStream_t st,
                       const q4::GemvBatch& bt, int m, int k) {
    switch (wide_rows(m) * 2 + pair) {
    case 8: return launch_wide_rows<G, SYM, XF16, GR, 4, 1>(upw, grid, block, lds, st, bt, m, k);
    case 9: return launch_wide_rows<G, SYM, XF16, GR, 4, 2>(upw, grid, block, lds, st, bt, m, k);
    case 16: return launch_wide_rows<G, SYM, XF16, GR, 8, 1>(upw, grid, block, lds, st, bt, m, k);
    case 17: return launch_wide_rows<G, SYM, XF16, GR, 8, 2>(upw, grid, block, lds, st, bt, m, k);
    case 32: return launch_wide_rows<G, SYM, XF16, GR, 16, 1>(upw, grid, block, lds, st, bt, m, k);
    default: return launch_wide_rows<G, SYM, XF16, GR, 16, 2>(upw, grid, block, lds, st, bt, m, k);
    }
}

// Workgroups of kernel kern resident per CU at (threads, LDS bytes), looked up once per
// (device, kernel, threads, LDS bytes).
template <typename Kern>
int resident_per_cu(Kern kern, int threads, size_t lds) {
    static std::mutex mu;
    static std::map<std::tuple<int, const void*, int, size_t>, int> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const auto key = std::make_tuple(dev, reinterpret_cast<const void*>(kern), threads, lds);
    std::lock_guard<std::mutex> lock(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kern, threads, lds) != hipSuccess || v < 1) v = 1;
    cache.emplace(key, v);
    return v;
}

// The resident kernel for a shape from resident_shape: P persistent workgroups, as few as
// give every workgroup the same number of tiles (give or take one) within one round.
template <int G, bool SYM, bool XF16, bool GR>
hipError_t launch_resident(int upw, int m, int k, int waves, const q4::GemvBatch& bt, int tiles, hipStream_t st) {
    const size_t lds = resident_lds(k, waves);
    const int threads = 64 * waves;
    const char* name = XF16 ? "q4_gemv_resident_f16" : "q4_gemv_resident_bf16";
    auto run = [&](auto kern) {
        const int cus = q4k_device_cus();
        const int slots = (cus > 0 ? cus : 256) * resident_per_cu(kern, threads, lds);
        const int per = (tiles + slots - 1) / slots;
        const int grid = (tiles + per - 1) / per;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3((unsigned)threads), lds, st, bt, m, k, tiles);
        return q4k_launched(name);
    };
    if (upw == 4) return run(gemv_resident_kernel<G, SYM, XF16, 4, GR>);
    if (upw == 8) return run(gemv_resident_kernel<G, SYM, XF16, 8, GR>);
    return hipErrorInvalidValue;
}

// Launch for a shape from tile_shape (wide == 0), wide_shape (wide == 1: one workgroup of
// 64 * waves threads per tile; wide == 2: per two tiles) or resident_shape (wide == 3:
// persistent workgroups over the batch's tiles, its problems sharing one x).
template <int G>
hipError_t launch_tile(int sym, int xd, int m, int k, int upw, int waves, int wide,
                       const q4::GemvBatch& bt, int tiles, hipStream_t st, const char** kname) {
    if (wide == 3) {
        const bool gr = bt.count > 1;
        *kname = xd == 1 ? "q4_gemv_resident_f16" : "q4_gemv_resident_bf16";
        if (sym) {
            if (xd == 1)
                return gr ? launch_resident<G, true, true, true>(upw, m, k, waves, bt, tiles, st)
                          : launch_resident<G, true, true, false>(upw, m, k, waves, bt, tiles, st);
            return gr ? launch_resident<G, true, false, true>(upw, m, k, waves, bt, tiles, st)
                      : launch_resident<G, true, false, false>(upw, m, k, waves, bt, tiles, st);
        }
        if (xd == 1)
            return gr ? launch_resident<G, false, true, true>(upw, m, k, waves, bt, tiles, st)
                      : launch_resident<G, false, true, false>(upw, m, k, waves, bt, tiles, st);
        return gr ? launch_resident<G, false, false, true>(upw, m, k, waves, bt, tiles, st)
                  : launch_resident<G, false, false, false>(upw, m, k, waves, bt, tiles, st);
    }
    if (wide) {  // wide kernel: each wave's activation ring (its partial sums reuse it)
        // Two 16-row tiles per workgroup (sharing every activation unit) while that still
        // leaves two tiles per CU; the problems' first workgroups are recounted for it.
        const int pair = wide == 2 ? 1 : 0;
        q4::GemvBatch bp = bt;
        int groups = tiles;
        if (pair) {
            groups = 0;
            for (int i = 0; i < bp.count; ++i) {
                bp.p[i].tile0 = groups;
                groups += (int)((bp.p[i].n + 31) / 32);
            }
        }
        const size_t lds = wide_lds(m, waves);
        const dim3 grid(groups), block(64 * waves);
        const bool gr = bt.count > 1;
        *kname = xd == 1 ? "q4_gemv_wide_f16" : "q4_gemv_wide_bf16";
        if (sym) {
            if (xd == 1)
                return gr ? launch_wide<G, true, true, true>(upw, pair, grid, block, lds, st, bp, m, k)
                          : launch_wide<G, true, true, false>(upw, pair, grid, block, lds, st, bp, m, k);
            return gr ? launch_wide<G, true, false, true>(upw, pair, grid, block, lds, st, bp, m, k)
                      : launch_wide<G, true, false, false>(upw, pair, grid, block, lds, st, bp, m, k);
        }
        if (xd == 1)
            return gr ? launch_wide<G, false, true, true>(upw, pair, grid, block, lds, st, bp, m, k)
                      : launch_wide<G, false, true, false>(upw, pair, grid, block, lds, st, bp, m, k);
        return gr ? launch_wide<G, false, false, true>(upw, pair, grid, block, lds, st, bp, m, k)
                  : launch_wide<G, false, false, false>(upw, pair, grid, block, lds, st, bp, m, k);
    }
    const int mq = m <= 1 ? 1 : 4;
    const size_t lds = (size_t)m * waves * upw * 256 + (size_t)waves * 64 * mq * 4;
    const dim3 grid(tiles), block(64 * waves);
    const bool gr = bt.count > 1;
    *kname = xd == 1 ? "q4_gemv_tile_f16" : "q4_gemv_tile_bf16";
    if (sym) {
        if (xd == 1)
            return gr ? launch_x<G, true, true, true>(upw, mq, grid, block, lds, st, bt, m, k)
                      : launch_x<G, true, true, false>(upw, mq, grid, block, lds, st, bt, m, k);
        return gr ? launch_x<G, true, false, true>(upw, mq, grid, block, lds, st, bt, m, k)
                  : launch_x<G, true, false, false>(upw, mq, grid, block, lds, st, bt, m, k);
    }
    if (xd == 1)
        return gr ? launch_x<G, false, true, true>(upw, mq, grid, block, lds, st, bt, m, k)
                  : launch_x<G, false, true, false>(upw, mq, grid, block, lds, st, bt, m, k);
    return gr ? launch_x<G, false, false, true>(upw, mq, grid, block, lds, st, bt, m, k)
              : launch_x<G, false, false, false>(upw, mq, grid, block, lds, st, bt, m, k);
}

}  // namespace q4t
