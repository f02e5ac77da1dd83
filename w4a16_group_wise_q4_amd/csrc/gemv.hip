// gemv.hip — decode W4A16 linear layer, m <= 16, for gfx950.
//
//   y[m][n] = sum_g S[n][g] * sum_{k in g} x[m][k] * (u[n][k] - z[n][g])
//
// Path A of "LLM Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV Cache (7/10)"
// (§Kernel이 없으면 압축 이점이 사라진다): packed INT4 weights are loaded, dequantized
// in registers and multiplied with higher-precision (fp32) accumulation.  Decode is
// bandwidth-bound (§Batch와 Context에 따라 속도가 달라진다), so the kernel is built
// around streaming the packed weights once at HBM speed.
//
// Mapping.  Work is split into tiles of 16 output rows.  Lane l handles row n0 + l%16 and
// k-slot block c = l/16 of a 16x16x32 MFMA: the 16 rows are the MFMA's N columns, the
// (zero-padded) activation rows are its M rows, so m = 1..16 costs the same.  The waves
// of a workgroup split the K range of a tile into contiguous slices of 128-column units;
// partial tiles are summed through LDS, so y is written once, without atomics, in a
// fixed order.  Workgroups are persistent: each takes tiles blockIdx.x, +gridDim.x, ...
// and stages the activations in LDS once for all of them (when they fit; otherwise one
// tile per workgroup and the activations are staged in column chunks).
//
// Memory.  All global reads are raw buffer loads (SGPR resource, per-lane row offset,
// scalar unit offset; reads past a resource's end return zero, which pads rows past N
// without branches).  The packed weights are the only stream on the hot path: per
// wave-wide load they touch 16 rows x 64 bytes.  A tile's scales and zero points are
// copied to LDS once per tile with coalesced loads, and the activations live in LDS,
// already permuted into the decoder's slot order, with an all-zero row feeding the
// MFMA's padding rows.  The packed weights stream through registers in double-buffered
// batches of kDepth units.  Per group and lane the loads are g/32 consecutive packed
// words (one dwordx4 at g = 128): lane block c holds words [GW*h + LW*c, +LW) of a group
// of GW = g/8 words, so the 32 k-slots of each MFMA lie in one group and the group's
// scale applies to the MFMA result.
//
// Dequantization.  The weight operand is the exact small integer u - z.  bf16
// activations: the nibbles plus 128 - z per byte, XOR 0x80, give u - z as signed bytes,
// converted exactly to fp32 and narrowed to bf16 by keeping the upper half (natural column
// order, so the activations are staged as loaded).  fp16 activations: 1024 + u in fp16
// minus (1024 + z) with one packed fp16 subtraction gives the exact u - z (pairs of
// columns i, i+4; the staged activations are permuted to match).  Either way products are
// exact and only the fp32 sums round, so the error of a group's dot product is relative to
// sum |x| |u - z|.
#include "q4_device.h"
#include "gemv_tile.h"
#include "q4_launch.h"

#include <map>
#include <tuple>

namespace {

constexpr int kMaxWaves = 8;           // waves per workgroup (all on one 16-row tile)
constexpr int kDepth = 4;              // 128-column units per batch (two batches in flight)
constexpr int kLdsBudget = 96 * 1024;  // LDS per workgroup (activations + metadata + sums)
constexpr int kStage = 4;              // activation vectors per thread per staging pass
constexpr int kMS = 4;                 // scale entries per thread per tile (chunked kernel)
constexpr int kMZ = 2;                 // zero-point words per thread per tile (chunked kernel)
constexpr int kPS = 8;                 // scale entries per thread per tile (streaming kernel)
constexpr int kPZ = 2;                 // zero-point dwords per thread per tile (streaming kernel)
constexpr int kOOB = 0x40000000;       // a buffer offset past every load resource: reads 0
constexpr uint32_t kStoreOOB = 0xFFFFFFF0u;  // a store offset past the y resource: dropped

using GemvBatch = q4::GemvBatch;

// One lane's share of one 128-column unit: 4 packed words (one per MFMA).
struct Unit {
    uint32_t w[4];
};

// Dequantize-and-multiply of one 128-column unit for one lane, accumulated into acc.
// xs: this lane's activation row in LDS (16-byte vectors, chunk-relative), s_row / z_row:
// this lane's row of the tile metadata in LDS, gbase: index of the unit's first group
// relative to that metadata, valid_groups: how many of the unit's NH groups exist.
template <int G, bool SYM, bool XF16>
__device__ __forceinline__ void unit_mac(q4::f32x4& acc, const Unit& d, const q4::u32x4* xs,
                                         int wrel, const uint16_t* s_row,
                                         const uint32_t* z_row, int gbase, bool ok0, int c,
                                         int KWrem, uint32_t kMask, uint32_t kMagic) {
    constexpr int GW = G / 8, LW = G / 32, NH = 4 / LW;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const bool ok = ok0 && (GW * h < KWrem);  // a short last unit has fewer groups
        const int hh = GW * h < KWrem ? h : 0;    // keep every index inside the row
        const int gl = gbase + hh;
        q4::u32x4 xa[LW];
#pragma unroll
        for (int a = 0; a < LW; ++a) xa[a] = xs[wrel + GW * hh + LW * c + a];
        const float s = q4::f16_bits_to_float(s_row[gl]);
        int z = 8;
        if constexpr (!SYM) z = (int)((z_row[gl >> 3] >> (4 * (gl & 7))) & 0xFu);
        q4::f32x4 dv = {0.f, 0.f, 0.f, 0.f};
        if constexpr (XF16) {
            const q4::f16x2 bias = q4::f16_bias_pair((uint32_t)z);
#pragma unroll
            for (int a = 0; a < LW; ++a)
                dv = q4::mfma_f16(xa[a], q4::decode_f16_exact(d.w[hh * LW + a], bias, kMask, kMagic), dv);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = ok ? acc[i] + s * dv[i] : acc[i];
        } else {
            const uint32_t zb = q4::bf16_zero_bias(z);
#pragma unroll
            for (int a = 0; a < LW; ++a) dv = q4::mfma_bf16(xa[a], q4::decode_bf16_exact(d.w[hh * LW + a], zb), dv);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = ok ? acc[i] + s * dv[i] : acc[i];
        }
    }
}

// Loads one lane's packed words of unit u (clamped inside the row).
template <int G>
__device__ __forceinline__ void unit_load(Unit& d, q4::rsrc rq, int qoff, int u, int KW) {
    constexpr int GW = G / 8, LW = G / 32, NH = 4 / LW;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        int wbase = u * 16 + GW * h;
        wbase = wbase < KW ? wbase : KW - GW;
        if constexpr (LW == 4) {
            const q4::u32x4 t = q4::buf_load_x4(rq, qoff, wbase * 4);
            d.w[0] = t[0]; d.w[1] = t[1]; d.w[2] = t[2]; d.w[3] = t[3];
        } else if constexpr (LW == 2) {
            const q4::u32x2 t = q4::buf_load_x2(rq, qoff, wbase * 4);
            d.w[2 * h] = t[0]; d.w[2 * h + 1] = t[1];
        } else {
            d.w[h] = q4::buf_load_x1(rq, qoff, wbase * 4);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Streaming kernel (the activations fit in LDS): persistent workgroups, each wave runs one
// continuous stream of D-unit batches over (tile, its K slice) with R batches in flight,
// so the next tile's weights are in flight while the current one is computed and reduced.
//
// The hardware counts outstanding loads in issue order and a wait names how many may
// remain in flight, so the stream stays overlapped only if every wait the compiler emits
// is a static count.  Hence: no load and no LDS store of loaded data sits behind a
// branch (lanes or batches with nothing to load use an offset past the buffer's end and
// read zeros; lanes with nothing to store write a private spare slot), the batches of a
// tile are a whole number of ring turns (nb % R == 0) so ring slots are static, and y
// is written with buffer stores that every wave issues (off the end when not its turn).
//
// LDS (16-byte vectors): activations [(M+1)][RS] | metadata x2 (each with a spare area
// of one dword per thread) | partial sums x2 ([S][64] each).
template <int G, bool SYM, bool XF16, int R, int D, int MAXT, int MINW, bool MULTI>
__global__ __launch_bounds__(MAXT, MINW) void gemv_stream_kernel(const GemvBatch bt, int M, int K) {
    constexpr int LW = G / 32;
    extern __shared__ q4::u32x4 lds[];
    // this workgroup's problem (wave-uniform; MULTI launches carry a single problem)
    int pi = 0;
#pragma unroll
    for (int i = 1; i < q4::kMaxGroup; ++i)
        if (i < bt.count && (int)blockIdx.x >= bt.p[i].tile0) pi = i;
    const uint16_t* __restrict__ x = reinterpret_cast<const uint16_t*>(bt.p[pi].x);
    const uint32_t* __restrict__ qweight = bt.p[pi].qweight;
    const uint16_t* __restrict__ scales = bt.p[pi].scales;
    const uint32_t* __restrict__ zeros = bt.p[pi].zeros;
    void* __restrict__ y = bt.p[pi].y;
    const int ydt = bt.ydt;
    const int N = bt.p[pi].n;
    const int bx = (int)blockIdx.x - bt.p[pi].tile0;  // tile index within the problem
    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int S = nthreads >> 6;
    const int col = lane & 15, c = lane >> 4;
    const int KW = K / 8, n_groups = K / G, zwords = (n_groups + 7) >> 3;
    const int tiles = (N + 15) / 16;
    const int RS = KW + 1;
    const int xs_end = (M + 1) * RS;
    const int s_ent = 16 * n_groups;       // scale entries of a tile (16 rows, contiguous)
    const int s_dw = 8 * n_groups;         // ... in dwords (the zero block starts after them)
    const int z_dw = SYM ? 0 : 16 * zwords;
    const int meta_vec = (s_dw + z_dw + 3) / 4;
    const int mbuf = meta_vec + nthreads / 4;  // one metadata copy plus its spare dwords
    uint32_t* meta0 = reinterpret_cast<uint32_t*>(lds + xs_end);
    q4::f32x4* red0 = reinterpret_cast<q4::f32x4*>(lds + xs_end + 2 * mbuf);
    const q4::u32x4* xs = lds + (col < M ? col : M) * RS;  // padding lanes: zero row
    const uint32_t kMask = q4::vreg_const(0x000F000Fu);
    const uint32_t kMagic = q4::vreg_const(0x64006400u);

    const int units = (K + 127) / 128;
    const int per = (units + S - 1) / S;
    const int u0 = wave * per;
    const int u1 = u0 + per < units ? u0 + per : units;
    const int ulast = u1 > u0 ? u1 - 1 : 0;
    const int nb = R * ((per + D * R - 1) / (D * R));  // batches per tile, whole ring turns
    // grid <= tiles; MULTI == false means grid == tiles (one tile per workgroup)
    const int ntiles = MULTI ? (tiles - 1 - bx) / (int)gridDim.x + 1 : 1;

    auto tile_n0 = [&](int tl) { return (bx + tl * (int)gridDim.x) * 16; };

    // metadata of tile ordinal tl (none for tl >= ntiles: every offset off the end): scales
    // block (16*n_groups fp16, copied entry by entry so no load straddles the end of the
    // array) then zero block (16*zwords dwords)
    auto meta_load = [&](int tl, uint32_t (&mv)[kPS + kPZ]) {
        const int n0 = tile_n0(tl);
        int rows = N - n0 < 16 ? N - n0 : 16;
        rows = tl < ntiles ? rows : 0;
        const q4::rsrc rs = q4::make_rsrc(scales + (int64_t)(tl < ntiles ? n0 : 0) * n_groups,
                                          (uint32_t)rows * n_groups * 2u);
#pragma unroll
        for (int j = 0; j < kPS; ++j) {
            const int e = j * nthreads + tid;
            mv[j] = q4::buf_load_u16(rs, e < s_ent ? e * 2 : kOOB, 0);
        }
#pragma unroll
        for (int j = 0; j < kPZ; ++j) {
            if constexpr (SYM) {
                mv[kPS + j] = 0u;
            } else {
                const q4::rsrc rz = q4::make_rsrc(zeros + (int64_t)(tl < ntiles ? n0 : 0) * zwords,
                                                  (uint32_t)rows * zwords * 4u);
                const int e = j * nthreads + tid;
                mv[kPS + j] = q4::buf_load_x1(rz, e < z_dw ? e * 4 : kOOB, 0);
            }
        }
    };
    auto meta_store = [&](uint32_t* dst, const uint32_t (&mv)[kPS + kPZ]) {
        uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);
        const int spare = 4 * meta_vec + tid;  // this thread's spare dword
#pragma unroll
        for (int j = 0; j < kPS; ++j) {
            const int e = j * nthreads + tid;
            d16[e < s_ent ? e : 2 * spare] = (uint16_t)mv[j];
        }
#pragma unroll
        for (int j = 0; j < kPZ; ++j) {
            const int e = j * nthreads + tid;
            dst[e < z_dw ? s_dw + e : spare] = mv[kPS + j];
        }
    };
    // issue batch b of tile ordinal tl (a batch past the end of the stream reads nothing)
    auto batch_load = [&](Unit (&bf)[D], int tl, int b) {
        const int n0 = tile_n0(tl < ntiles ? tl : 0);
        const int rows = N - n0 < 16 ? N - n0 : 16;
        const q4::rsrc rq = q4::make_rsrc(qweight + (int64_t)n0 * KW, (uint32_t)rows * KW * 4u);
        const int qoff = col < rows && tl < ntiles ? col * KW * 4 + c * LW * 4 : kOOB;
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int u = u0 + b * D + j;
            unit_load<G>(bf[j], rq, u < u1 ? qoff : kOOB, u < u1 ? u : ulast, KW);
        }
    };

    q4::f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto batch_compute = [&](const Unit (&bf)[D], int b, const uint32_t* meta) {
        const uint16_t* s_row = reinterpret_cast<const uint16_t*>(meta) + col * n_groups;
        const uint32_t* z_row = meta + s_dw + col * zwords;
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int u = u0 + b * D + j;
            const bool ok = u < u1;
            const int ue = ok ? u : ulast;
            unit_mac<G, SYM, XF16>(acc, bf[j], xs, ue * 16, s_row, z_row, ue * (4 / LW), ok,
                                   c, KW - ue * 16, kMask, kMagic);
        }
    };

    // ---- prologue: activations, first tile's metadata, first R batches
    Unit buf[R][D];
    {
        q4::u32x4 xv[kStage];
        const q4::rsrc rx = q4::make_rsrc(x, (uint32_t)M * K * 2u);
#pragma unroll
        for (int j = 0; j < kStage; ++j) {
            const int v = j * nthreads + tid;
            const int m = v / RS, jj = v - m * RS;
            const bool real = v < xs_end && m < M && jj < KW;
            xv[j] = q4::buf_load_x4(rx, real ? (m * K + 8 * jj) * 2 : kOOB, 0);
        }
        // issue order is wait order: activations (cache-hot), metadata, then the weight
        // ring, so staging the first two never waits for the weights
        __builtin_amdgcn_sched_barrier(0);
        uint32_t mv[kPS + kPZ];
        meta_load(0, mv);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < R; ++r) batch_load(buf[r], 0, r);  // R <= nb
        __builtin_amdgcn_sched_barrier(0);
        q4::u32x4* spare = reinterpret_cast<q4::u32x4*>(red0) + tid;  // unused until tile 0 ends
#pragma unroll
        for (int j = 0; j < kStage; ++j) {
            const int v = j * nthreads + tid;
            *(v < xs_end ? lds + v : spare) = XF16 ? q4::pair_perm(xv[j]) : xv[j];
        }
        for (int v0 = kStage * nthreads; v0 < xs_end; v0 += nthreads) {  // larger m*k only
            const int v = v0 + tid;
            const int m = v / RS, jj = v - m * RS;
            const bool real = v < xs_end && m < M && jj < KW;
            const q4::u32x4 t = q4::buf_load_x4(rx, real ? (m * K + 8 * jj) * 2 : kOOB, 0);
            *(v < xs_end ? lds + v : spare) = XF16 ? q4::pair_perm(t) : t;
        }
        meta_store(meta0, mv);
    }
    __syncthreads();

    const q4::rsrc ry = q4::make_rsrc(y, (uint32_t)M * (uint32_t)N * q4::y_bytes(ydt));
    for (int tl = 0; tl < ntiles; ++tl) {
        uint32_t mnext[kPS + kPZ];
        // next tile's metadata.  Its loads sit behind the ring's, so the first wait of the
        // tile also covers them; a one-tile grid has nothing to fetch and skips them.
        if constexpr (MULTI) meta_load(tl + 1, mnext);
        const uint32_t* meta = meta0 + (tl & 1) * 4 * mbuf;
        int b = 0;
        do {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                batch_compute(buf[r], b + r, meta);
                const int nx = b + r + R;          // the batch that refills this slot
                const bool wrap = nx >= nb;
                batch_load(buf[r], wrap ? tl + 1 : tl, wrap ? nx - nb : nx);
                // keep the refill right behind the compute that frees its registers, so
                // loads are issued as early as the ring allows
                __builtin_amdgcn_sched_barrier(0);
            }
            b += R;
        } while (b < nb);
        // tile done: publish partial sums and the next tile's metadata; one barrier
        q4::f32x4* red = red0 + (tl & 1) * 64 * S;
        red[wave * 64 + lane] = acc;
        acc = q4::f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (MULTI) meta_store(meta0 + ((tl + 1) & 1) * 4 * mbuf, mnext);
        __syncthreads();
        const int n0 = tile_n0(tl);
        const bool fin = wave == tl % S;  // rotating finisher wave
        float sum[4] = {0.f, 0.f, 0.f, 0.f};  // a plain array: see f32_bits
        if (fin) {
            for (int w = 0; w < S; ++w) {
                const q4::f32x4 t = red[w * 64 + lane];
                sum[0] += t.x;
                sum[1] += t.y;
                sum[2] += t.z;
                sum[3] += t.w;
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = 4 * c + q;
            const bool st = fin && m < M && n0 + col < N;
            const uint32_t off = st ? ((uint32_t)m * (uint32_t)N + (uint32_t)(n0 + col)) * q4::y_bytes(ydt) : kStoreOOB;
            q4::store_y(ry, off, sum[q], ydt);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Chunked kernel (the activations do not fit in LDS): one tile per workgroup, activations
// staged in column chunks.
// LDS layout (16-byte vectors):
//   [0, (M+1)*RS)        activation chunk: row m at m*RS, row M all zeros
//   [xs_end, +META)      tile metadata: scales [16][cg] fp16, then zero words [16][czw]
//   [.., + waves*64)     cross-wave partial sums
template <int G, bool SYM, bool XF16>
__global__ __launch_bounds__(512) void gemv_chunk_kernel(const uint16_t* __restrict__ x, int M,
                                                         const uint32_t* __restrict__ qweight,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint32_t* __restrict__ zeros, int N,
                                                         int K, int KC, void* __restrict__ y, int ydt) {
    constexpr int LW = G / 32;  // words per lane per group (one MFMA per word)
    constexpr int NH = 4 / LW;  // groups per 128-column unit
    extern __shared__ q4::u32x4 lds[];

    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int S = nthreads >> 6;
    const int col = lane & 15;
    const int c = lane >> 4;
    const int KW = K / 8;
    const int n_groups = K / G;
    const int zwords = (n_groups + 7) >> 3;
    const int RS = KC / 8 + 1;                   // LDS activation row stride (vectors)
    const int cg = (KC + G - 1) / G;             // groups per chunk (KC is a multiple of 8*G)
    const int czw = (cg + 7) >> 3;               // zero words per chunk row
    const int xs_end = (M + 1) * RS;
    uint16_t* meta_s = reinterpret_cast<uint16_t*>(lds + xs_end);
    uint32_t* meta_z = reinterpret_cast<uint32_t*>(lds + xs_end) + (16 * cg + 1) / 2;
    const int meta_vec = ((16 * cg + 1) / 2 + 16 * czw + 3) / 4;
    q4::f32x4* red = reinterpret_cast<q4::f32x4*>(lds + xs_end + meta_vec);
    const q4::u32x4* xs = lds + (col < M ? col : M) * RS;  // padding lanes: zero row

    const q4::rsrc rx = q4::make_rsrc(x, (uint32_t)M * K * 2u);
    const uint32_t kMask = q4::vreg_const(0x000F000Fu);
    const uint32_t kMagic = q4::vreg_const(0x64006400u);

    const int tile = blockIdx.x;
    const int n0 = tile * 16;
    const int rows = N - n0 < 16 ? N - n0 : 16;
    const q4::rsrc rq = q4::make_rsrc(qweight + (int64_t)n0 * KW, (uint32_t)rows * KW * 4u);
    const q4::rsrc rs = q4::make_rsrc(scales + (int64_t)n0 * n_groups, (uint32_t)rows * n_groups * 2u);
    const q4::rsrc rz = q4::make_rsrc(zeros + (int64_t)n0 * zwords, (uint32_t)rows * zwords * 4u);
    const int qoff = col < rows ? col * KW * 4 + c * LW * 4 : kOOB;

    q4::f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    Unit bufA[kDepth], bufB[kDepth];
    auto load_batch = [&](Unit(&bf)[kDepth], int ub, int u1, int ulast) {
#pragma unroll
        for (int i = 0; i < kDepth; ++i) unit_load<G>(bf[i], rq, qoff, ub + i < u1 ? ub + i : ulast, KW);
    };
    // padding units (past the wave's range) were loaded from ulast and are computed as
    // ulast, so every index stays inside the chunk; their result is not added
    auto compute_batch = [&](const Unit(&bf)[kDepth], int ub, int u1, int ulast, int cb) {
#pragma unroll
        for (int i = 0; i < kDepth; ++i) {
            const bool ok = ub + i < u1;
            const int ue = ok ? ub + i : ulast;
            unit_mac<G, SYM, XF16>(acc, bf[i], xs, ue * 16 - cb / 8, meta_s + col * cg,
                                   meta_z + col * czw, ue * NH - cb / G, ok, c, KW - ue * 16,
                                   kMask, kMagic);
        }
    };

    for (int cb = 0; cb < K; cb += KC) {
        const int ce = cb + KC < K ? cb + KC : K;
        const int cu0 = cb / 128, cu1 = (ce + 127) / 128;
        const int per = (cu1 - cu0 + S - 1) / S;  // units per wave (the last may have fewer)
        const int u0 = cu0 + wave * per;
        const int u1 = u0 + per < cu1 ? u0 + per : cu1;
        const int ulast = u1 > u0 ? u1 - 1 : cu0;  // in-range unit to point idle loads at
        const int nb = (per + kDepth - 1) / kDepth;  // batches of kDepth units

        // 1. issue the activation chunk, the chunk's metadata, the first two weight batches
        const int vpr = (ce - cb) / 8;
        const int nvec = xs_end;
        q4::u32x4 xv[kStage];
#pragma unroll
        for (int j = 0; j < kStage; ++j) {
            const int v = j * nthreads + tid;
            const int m = v / RS, jj = v - m * RS;
            const bool real = v < nvec && m < M && jj < vpr;
            xv[j] = q4::buf_load_x4(rx, real ? (m * K + cb + 8 * jj) * 2 : kOOB, 0);
        }
        const int gc0 = cb / G, ngc = (ce - cb + G - 1) / G, zc0 = gc0 >> 3;
        const int nzc = (ngc + 7) >> 3;
        uint32_t sv[kMS], zv[kMZ];
#pragma unroll
        for (int j = 0; j < kMS; ++j) {
            const int e = j * nthreads + tid;  // scale entry (row r, chunk group g)
            const int r = e / cg, g = e - r * cg;
            const bool real = r < 16 && g < ngc;
            sv[j] = q4::buf_load_u16(rs, real ? (r * n_groups + gc0 + g) * 2 : kOOB, 0);
        }
#pragma unroll
        for (int j = 0; j < kMZ; ++j) {
            const int e = j * nthreads + tid;  // zero word entry (row r, chunk word q)
            const int r = e / czw, q = e - r * czw;
            const bool real = !SYM && r < 16 && q < nzc;
            zv[j] = SYM ? 0u : q4::buf_load_x1(rz, real ? (r * zwords + zc0 + q) * 4 : kOOB, 0);
        }
        load_batch(bufA, u0, u1, ulast);
        if (nb > 1) load_batch(bufB, u0 + kDepth, u1, ulast);

        if (cb > 0) __syncthreads();  // LDS free for reuse
        // 2. park activations and metadata in LDS
#pragma unroll
        for (int j = 0; j < kStage; ++j) {
            const int v = j * nthreads + tid;
            if (v < nvec) lds[v] = XF16 ? q4::pair_perm(xv[j]) : xv[j];
        }
        for (int v0 = kStage * nthreads; v0 < nvec; v0 += nthreads) {
            const int v = v0 + tid;
            const int m = v / RS, jj = v - m * RS;
            const bool real = v < nvec && m < M && jj < vpr;
            const q4::u32x4 t = q4::buf_load_x4(rx, real ? (m * K + cb + 8 * jj) * 2 : kOOB, 0);
            if (v < nvec) lds[v] = XF16 ? q4::pair_perm(t) : t;
        }
#pragma unroll
        for (int j = 0; j < kMS; ++j) {
            const int e = j * nthreads + tid;
            if (e < 16 * cg) meta_s[e] = (uint16_t)sv[j];
        }
#pragma unroll
        for (int j = 0; j < kMZ; ++j) {
            const int e = j * nthreads + tid;
            if (e < 16 * czw) meta_z[e] = zv[j];
        }
        __syncthreads();
        // 3. double-buffered batches: batch b+2 is requested once batch b is consumed
        for (int b = 0; b < nb; b += 2) {
            compute_batch(bufA, u0 + b * kDepth, u1, ulast, cb);
            if (b + 2 < nb) load_batch(bufA, u0 + (b + 2) * kDepth, u1, ulast);
            if (b + 1 < nb) {
                compute_batch(bufB, u0 + (b + 1) * kDepth, u1, ulast, cb);
                if (b + 3 < nb) load_batch(bufB, u0 + (b + 3) * kDepth, u1, ulast);
            }
        }
    }

    // 4. cross-wave sum of the tile, written once
    red[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave == 0 && col < rows) {
        q4::f32x4 t = red[lane];
        for (int w = 1; w < S; ++w) {
            const q4::f32x4 r = red[w * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) t[i] += r[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * c + i;
            if (m < M) q4::store_y(y, (int64_t)m * N + n0 + col, t[i], ydt);
        }
    }
}

// One problem (batch == nullptr) or a batch of problems whose tiles add up to n rows.
template <int G, bool SYM>
hipError_t launch(const void* x, int xd, int m, const uint32_t* qw, const uint16_t* sc,
                  const uint32_t* zr, int n, int k, void* y, int ydt, hipStream_t st, const char** kname,
                  const GemvBatch* batch = nullptr, int batch_tiles = 0) {
    const int num_cus = q4k_device_cus();
    // Workgroup shape.  With tiles to spare (at least two per CU): 4-wave workgroups,
    // several resident per CU, two batches in flight per wave.  With at most one tile per
    // CU the whole matrix is requested at once and the time after the data arrives
    // dominates, so the tile is spread over up to 16 waves of 2-unit batches.  Otherwise
    // 8 waves of 2-unit batches.
    const int units_k = (k + 127) / 128;
    const int tiles = batch != nullptr ? batch_tiles : (n + 15) / 16;
    {
        // the tile kernel reads scales as dwords: every scale array 4-byte aligned
        bool sc4 = true;
        if (batch != nullptr) {
            for (int i = 0; i < batch->count; ++i) sc4 = sc4 && ((uintptr_t)batch->p[i].scales & 3) == 0;
        } else {
            sc4 = ((uintptr_t)sc & 3) == 0;
        }
        // the resident kernel stages one x for every problem of the launch (8 < m <= 16)
        bool one_x = true;
        if (batch != nullptr)
            for (int i = 1; i < batch->count; ++i) one_x = one_x && batch->p[i].x == batch->p[0].x;
        int upw = 0, tw = 0, wide = 0;
        bool fits = false;
        if (sc4 && one_x && q4t::resident_shape(G, m, k, tiles, num_cus, &upw, &tw)) {
            fits = true;
            wide = 3;
        } else if (sc4 && m >= 2 && tiles <= 4 * num_cus && q4t::wide_shape(G, m, k, &upw, &tw)) {
            // 2 <= m <= 4 with at most four tiles per CU: the wide kernel, whose waves
            // stream their activations unit by unit, measured faster than the tile kernel,
            // whose waves wait for their whole activation slice before any arithmetic
            // (8.15 against 9.68 us on 4096x11008 at m = 2; 10.6 against 12.2 on 8192x8192
            // at m = 4).  With more tiles, and at m = 1, the tile kernel is faster.
            fits = true;
            wide = q4t::wide_pair(tiles, num_cus) ? 2 : 1;
        } else {
            fits = sc4 && (q4t::tile_shape(G, m, k, tiles, num_cus, &upw, &tw) ||
                           (wide = q4t::wide_shape(G, m, k, &upw, &tw)));
            if (wide && q4t::wide_pair(tiles, num_cus)) wide = 2;
        }
        if (fits) {
            GemvBatch one{};
            if (batch == nullptr) {
                one.p[0] = q4::GemvProblem{x, qw, sc, zr, y, n, 0};
                one.count = 1;
                one.ydt = ydt;
            }
            const GemvBatch& bt = batch != nullptr ? *batch : one;
            if constexpr (G == 32) return q4k_gemv_tile_g32(SYM, xd, m, k, upw, tw, wide, bt, tiles, st, kname);
            if constexpr (G == 64) return q4k_gemv_tile_g64(SYM, xd, m, k, upw, tw, wide, bt, tiles, st, kname);
            return q4k_gemv_tile_g128(SYM, xd, m, k, upw, tw, wide, bt, tiles, st, kname);
        }
    }
    int shape;  // 0: up to 8 waves   1: up to 4 waves   2: up to 16 waves
    int waves;
    if (tiles >= 2 * num_cus) {
        shape = 1;
        waves = (units_k + 3) / 4;
        waves = waves < 1 ? 1 : (waves > 4 ? 4 : waves);
    } else if (tiles <= num_cus && units_k >= 16 && G >= 64) {
        shape = 2;
        waves = (units_k + 1) / 2;
        waves = waves > 16 ? 16 : waves;
    } else {
        shape = 0;
        waves = (units_k + 3) / 4;
        waves = waves < 1 ? 1 : (waves > kMaxWaves ? kMaxWaves : waves);
    }
    const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
    const int ng = k / G, zw = (ng + 7) / 8;
    // streaming kernel when the activations (plus zero row), two metadata copies and two
    // sets of partial sums fit, and a tile's metadata fits the per-thread copy
    const int meta_vec = (8 * ng + (SYM ? 0 : 16 * zw) + 3) / 4;
    auto stream_lds = [&](int w) {  // activations, 2 x (metadata + spare dwords), 2 x partial sums
        return (size_t)((m + 1) * (k / 8 + 1) + 2 * (meta_vec + 16 * w) + 2 * w * 64) * 16;
    };
    auto stream_fits = [&](int w) {
        return stream_lds(w) <= (size_t)kLdsBudget && 16 * ng <= kPS * 64 * w &&
               16 * zw <= kPZ * 64 * w;
    };
    if (shape == 2 && !stream_fits(waves)) {  // too much LDS for 16 waves: 8-wave shape
        shape = 0;
        waves = (units_k + 3) / 4;
        waves = waves < 1 ? 1 : (waves > kMaxWaves ? kMaxWaves : waves);
    }
    const bool stream = stream_fits(waves);
    if (!stream && batch != nullptr) return hipErrorNotSupported;  // one by one instead
    if (!stream && waves > kMaxWaves) waves = kMaxWaves;  // the chunked kernel's bound
    const int threads = 64 * waves;
    const size_t lds_stream = stream_lds(waves);
    if (stream) {
        // Workgroups resident per CU for a kernel at this shape, cached per thread on
        // (device, kernel, threads, LDS bytes).  When every tile gets its own workgroup the
        // one-tile form runs (no metadata prefetch for a next tile); otherwise persistent
        // workgroups take turns.
        auto per_cu = [&](auto kern) {
            thread_local std::map<std::tuple<int, const void*, int, size_t>, int> cache;
            int dev = 0;
            (void)hipGetDevice(&dev);
            const auto key = std::make_tuple(dev, reinterpret_cast<const void*>(kern), threads, lds_stream);
            const auto it = cache.find(key);
            if (it != cache.end()) return it->second;
            int v = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kern, threads, lds_stream) != hipSuccess || v < 1)
                v = 1;
            cache.emplace(key, v);
            return v;
        };
        auto run = [&](auto k_multi, auto k_one, const char* name) {
            *kname = name;
            if (batch != nullptr) {  // several problems: one workgroup per tile
                hipLaunchKernelGGL(k_one, dim3(tiles), dim3(threads), lds_stream, st, *batch, m, k);
                return q4k_launched(name);
            }
            GemvBatch one{};
            one.p[0] = q4::GemvProblem{x, qw, sc, zr, y, n, 0};
            one.count = 1;
            one.ydt = ydt;
            const int cap = num_cus * per_cu(k_multi);
            if (tiles <= cap)
                hipLaunchKernelGGL(k_one, dim3(tiles), dim3(threads), lds_stream, st, one, m, k);
            else
                hipLaunchKernelGGL(k_multi, dim3(cap), dim3(threads), lds_stream, st, one, m, k);
            return q4k_launched(name);
        };
        // A tile's batches are whole ring turns (D units per batch, R batches in flight);
        // pick the batch size that leaves the fewest idle unit slots in a wave's slice.
        const int per = (units_k + waves - 1) / waves;
        const bool wide = 8 * ((per + 7) / 8) - per <= 4 * ((per + 3) / 4) - per;
        if (shape == 1) {
            if (wide) {
                if (xd == 1) return run(gemv_stream_kernel<G, SYM, true, 2, 4, 256, 2, true>,
                                        gemv_stream_kernel<G, SYM, true, 2, 4, 256, 2, false>, "q4_gemv_mfma_f16");
                return run(gemv_stream_kernel<G, SYM, false, 2, 4, 256, 2, true>,
                           gemv_stream_kernel<G, SYM, false, 2, 4, 256, 2, false>, "q4_gemv_mfma_bf16");
            }
            if (xd == 1) return run(gemv_stream_kernel<G, SYM, true, 2, 2, 256, 2, true>,
                                    gemv_stream_kernel<G, SYM, true, 2, 2, 256, 2, false>, "q4_gemv_mfma_f16");
            return run(gemv_stream_kernel<G, SYM, false, 2, 2, 256, 2, true>,
                       gemv_stream_kernel<G, SYM, false, 2, 2, 256, 2, false>, "q4_gemv_mfma_bf16");
        }
        if constexpr (G >= 64) {
            if (shape == 2) {  // tiles <= CUs: always one tile per workgroup
                if (xd == 1) return run(gemv_stream_kernel<G, SYM, true, 1, 2, 1024, 1, true>,
                                        gemv_stream_kernel<G, SYM, true, 1, 2, 1024, 1, false>, "q4_gemv_mfma_f16");
                return run(gemv_stream_kernel<G, SYM, false, 1, 2, 1024, 1, true>,
                           gemv_stream_kernel<G, SYM, false, 1, 2, 1024, 1, false>, "q4_gemv_mfma_bf16");
            }
        }
        if (xd == 1) return run(gemv_stream_kernel<G, SYM, true, 2, 2, 512, 1, true>,
                                gemv_stream_kernel<G, SYM, true, 2, 2, 512, 1, false>, "q4_gemv_mfma_f16");
        return run(gemv_stream_kernel<G, SYM, false, 2, 2, 512, 1, true>,
                   gemv_stream_kernel<G, SYM, false, 2, 2, 512, 1, false>, "q4_gemv_mfma_bf16");
    }
    auto lds_bytes = [&](int kc) {
        const int cg = (kc + G - 1) / G, czw = (cg + 7) / 8;
        const int mv = ((16 * cg + 1) / 2 + 16 * czw + 3) / 4;
        return (size_t)((m + 1) * (kc / 8 + 1) + mv + waves * 64) * 16;
    };
    auto fits = [&](int kc) {
        const int cg = (kc + G - 1) / G, czw = (cg + 7) / 8;
        return lds_bytes(kc) <= (size_t)kLdsBudget && 16 * cg <= kMS * threads &&
               16 * czw <= kMZ * threads;
    };
    // activation chunk: the largest multiple of 8 groups (and of 128 columns) that fits
    const int step = 8 * G > 128 ? 8 * G : 128;
    int kc = step;
    while (kc + step < k && fits(kc + step)) kc += step;
    if (kc > k) kc = k;
    const size_t lds = lds_bytes(kc);
    if (xd == 1) {
        *kname = "q4_gemv_mfma_f16";
        hipLaunchKernelGGL((gemv_chunk_kernel<G, SYM, true>), dim3(tiles), dim3(threads), lds, st, xp, m,
                           qw, sc, zr, n, k, kc, y, ydt);
    } else {
        *kname = "q4_gemv_mfma_bf16";
        hipLaunchKernelGGL((gemv_chunk_kernel<G, SYM, false>), dim3(tiles), dim3(threads), lds, st, xp, m,
                           qw, sc, zr, n, k, kc, y, ydt);
    }
    return q4k_launched(*kname);
}

}  // namespace

hipError_t q4k_gemv(const void* x, int x_dtype, int m, const uint32_t* qweight,
                    const uint16_t* scales, const uint32_t* zeros, int64_t n, int64_t k, int g,
                    int sym, void* y, int ydt, hipStream_t stream, const char** kname) {
    const int ni = (int)n, ki = (int)k;
    switch (g * 2 + (sym ? 1 : 0)) {
    case 64: return launch<32, false>(x, x_dtype, m, qweight, scales, zeros, ni, ki, y, ydt, stream, kname);
    case 65: return launch<32, true>(x, x_dtype, m, qweight, scales, zeros, ni, ki, y, ydt, stream, kname);
    case 128: return launch<64, false>(x, x_dtype, m, qweight, scales, zeros, ni, ki, y, ydt, stream, kname);
    case 129: return launch<64, true>(x, x_dtype, m, qweight, scales, zeros, ni, ki, y, ydt, stream, kname);
    case 256: return launch<128, false>(x, x_dtype, m, qweight, scales, zeros, ni, ki, y, ydt, stream, kname);
    default: return launch<128, true>(x, x_dtype, m, qweight, scales, zeros, ni, ki, y, ydt, stream, kname);
    }
}

hipError_t q4k_gemv_grouped(const q4::GemvProblem* problems, int count, int x_dtype, int m,
                            int64_t k, int g, int sym, int ydt, hipStream_t stream, const char** kname) {
    if (count < 1 || count > q4::kMaxGroup) return hipErrorInvalidValue;
    GemvBatch batch{};
    int tiles = 0;
    for (int i = 0; i < count; ++i) {
        batch.p[i] = problems[i];
        batch.p[i].tile0 = tiles;
        tiles += (problems[i].n + 15) / 16;
    }
    batch.count = count;
    batch.ydt = ydt;
    const int ki = (int)k, rows = 16 * tiles;
    const void* x = problems[0].x;
    switch (g * 2 + (sym ? 1 : 0)) {
    case 64: return launch<32, false>(x, x_dtype, m, nullptr, nullptr, nullptr, rows, ki, nullptr, ydt, stream, kname, &batch, tiles);
    case 65: return launch<32, true>(x, x_dtype, m, nullptr, nullptr, nullptr, rows, ki, nullptr, ydt, stream, kname, &batch, tiles);
    case 128: return launch<64, false>(x, x_dtype, m, nullptr, nullptr, nullptr, rows, ki, nullptr, ydt, stream, kname, &batch, tiles);
    case 129: return launch<64, true>(x, x_dtype, m, nullptr, nullptr, nullptr, rows, ki, nullptr, ydt, stream, kname, &batch, tiles);
    case 256: return launch<128, false>(x, x_dtype, m, nullptr, nullptr, nullptr, rows, ki, nullptr, ydt, stream, kname, &batch, tiles);
    default: return launch<128, true>(x, x_dtype, m, nullptr, nullptr, nullptr, rows, ki, nullptr, ydt, stream, kname, &batch, tiles);
    }
}

