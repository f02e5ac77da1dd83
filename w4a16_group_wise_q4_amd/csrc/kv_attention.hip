// kv_attention.hip — decode attention over an INT4 group-quantized KV cache, for gfx950.
//
//   o[h] = sum_t softmax_t(scale * q[h] . K_hat[h][t]) * V_hat[h][t],
//   K_hat[h][t][i] = S_K[h][t][i/g] * (u_K[h][t][i] - z_K[h][t][i/g])   (and V alike)
//
// The KV-cache chapter of "Quantization Algorithms 단권화" (§INT4 group scheme, §asym 선택
// 이유, §Attention에서의 결합): asymmetric INT4 groups of g along the head dimension, one
// fp16 scale and one zero point per (token, head, group), recomputed for every new token,
// and the dequantization fused into the attention matmuls so that the cache is read once,
// at 4 bits.  The cache is head-major: token t of head h is row h * t_cap + t of the same
// packed layout as a weight matrix with k = d.
//
// Split over tokens (decode has one query per head, so one head alone cannot fill the
// chip): workgroup (h, c) takes chunk c of head h, CH = 4 waves x NL loads x 2048/d
// tokens, computes their scores, a reference m_c (each wave's largest score of its first
// batch, moved up only when a later score passes it by more than 40; the softmax is the
// same for any reference that keeps the exponentials in range), l_c = sum exp(s - m_c)
// and the unnormalized o_c = sum exp(s - m_c) * V_hat, and writes (m_c, l_c, o_c) to the
// workspace.  NL (1, 2, 4 or 8 loads per wave) is the largest that still gives 512
// workgroups.  A second kernel combines the chunks of each head in chunk order:
// M = max m_c, o = sum o_c e^(m_c - M) / sum l_c e^(m_c - M).
//
// Lanes: each lane owns 32 consecutive head dimensions (one 16-byte load of codes per
// token, inside one group since g >= 32); d/32 lanes share a token, so a wave-wide load
// covers 2048/d consecutive tokens.  The loads of the whole chunk (K and V codes, scales,
// zero words) are issued first; HBM latency is covered by the bytes in flight.  Scores:
// the lane's partial sum_i q_i u_i - z * sum_i q_i, times the group scale, summed over the
// token's lanes.  Values: the lane accumulates p_t S_t u_i for its 32 dimensions and
// p_t S_t z separately.  Everything is fp32; no fp32 addition chain is longer than
// chunks + 32 terms (at most 8 tokens per lane, 3 levels within a row of lanes, 16 rows of
// the workgroup, the chunks, the rest).
#include "q4_launch.h"

#include <mutex>

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr uint32_t kOff = 0xFFFFFFF0u;

// Lane exchanges without LDS: DPP within rows of 16 lanes, v_permlane16/32_swap across
// rows.  xor1/xor2 swap neighbours inside a quad; ror4/ror8 rotate a row; across16/32
// give each lane the value of lane ^ 16 / lane ^ 32.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float xor1(float v) { return dpp<0xB1>(v); }   // quad_perm 1,0,3,2
__device__ __forceinline__ float xor2(float v) { return dpp<0x4E>(v); }   // quad_perm 2,3,0,1
__device__ __forceinline__ float ror4(float v) { return dpp<0x124>(v); }  // row_ror:4
__device__ __forceinline__ float ror8(float v) { return dpp<0x128>(v); }  // row_ror:8
__device__ __forceinline__ float across16(float v) {
    const auto t = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v), false, false);
    const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    return __builtin_bit_cast(float, (lane & 16) ? t[0] : t[1]);
}
__device__ __forceinline__ float across32(float v) {
    const auto t = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v), false, false);
    const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    return __builtin_bit_cast(float, (lane & 32) ? t[0] : t[1]);
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, xor1(v));
    v = fmaxf(v, xor2(v));
    v = fmaxf(v, ror4(v));
    v = fmaxf(v, ror8(v));
    v = fmaxf(v, across16(v));
    return fmaxf(v, across32(v));
}
// Sum over the LPT consecutive lanes of one token (lanes tl * LPT .. + LPT - 1).
template <int LPT>
__device__ __forceinline__ float token_sum(float v) {
    if constexpr (LPT >= 2) v += xor1(v);
    if constexpr (LPT >= 4) v += xor2(v);
    if constexpr (LPT >= 8) v += __shfl_xor(v, 4, 64);
    return v;
}
// Sum over the tokens of one row of 16 lanes: afterwards lane r * 16 + j (j < LPT) holds
// the row's sum for dimensions block j.
template <int LPT>
__device__ __forceinline__ float row_dim_sum(float v) {
    if constexpr (LPT <= 2) v += xor2(v);
    if constexpr (LPT <= 4) v += ror4(v);
    return v + ror8(v);
}

// 8 codes of a packed word as floats (column order 0..7): two masks, then one
// v_cvt_f32_ubyteN per code (written as asm: the compiler folds the byte masks into
// bit-field extracts and loses the byte conversions)
template <int B>
__device__ __forceinline__ float ubyte(uint32_t x) {
    float f;
    if constexpr (B == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(x));
    if constexpr (B == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(x));
    if constexpr (B == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(x));
    if constexpr (B == 3) asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(x));
    return f;
}
__device__ __forceinline__ void unpack8(uint32_t w, float (&f)[8]) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    f[0] = ubyte<0>(lo);
    f[1] = ubyte<0>(hi);
    f[2] = ubyte<1>(lo);
    f[3] = ubyte<1>(hi);
    f[4] = ubyte<2>(lo);
    f[5] = ubyte<2>(hi);
    f[6] = ubyte<3>(lo);
    f[7] = ubyte<3>(hi);
}

struct KvArgs {
    const void* q;
    const uint32_t* kq;
    const uint16_t* ks;
    const uint32_t* kz;
    const uint32_t* vq;
    const uint16_t* vs;
    const uint32_t* vz;
    float* ws;           // [heads][chunks][d + 2]: m, l, o[d]
    int t, t_cap, chunks;
    float scale;
};

// o[h][i] = sum_c o_c[i] e^(m_c - M) / sum_c l_c e^(m_c - M), M = max_c m_c, the sums
// taken in chunk order; one workgroup of 256 threads per head.  The chunks' maxima and the
// partials of the first kTile chunks are loaded together (independent loads: one memory
// round trip in all for up to kTile chunks), later tiles one round trip each; each
// thread i < D walks a tile's chunks in order from LDS.
constexpr int kTile = 32;

template <int D>
__global__ __launch_bounds__(256) void kv_combine_kernel(const float* __restrict__ ws, int chunks,
                                                         float* __restrict__ o) {
    constexpr int ROW = D + 2;
    constexpr int PER = (kTile * ROW + 255) / 256;  // floats per thread per tile
    __shared__ float tile[kTile * ROW];
    __shared__ float ec[kTile];
    __shared__ float red[4];
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const float* base = ws + (int64_t)h * chunks * ROW;
    const q4::rsrc rall = q4::make_rsrc(base, (uint32_t)(chunks * ROW) * 4u);

    float v[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) v[e] = __builtin_bit_cast(float, q4::buf_load_x1(rall, (e * 256 + tid) * 4, 0));
    float mx = -INFINITY;
    for (int c = tid; c < chunks; c += 256)
        mx = fmaxf(mx, __builtin_bit_cast(float, q4::buf_load_x1(rall, c * ROW * 4, 0)));
    mx = wave_max(mx);
    if (lane == 0) red[w] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

    float acc = 0.f, lsum = 0.f;
    for (int c0 = 0; c0 < chunks; c0 += kTile) {
        const int nc = chunks - c0 < kTile ? chunks - c0 : kTile;
        if (c0 > 0) {
            const q4::rsrc r = q4::make_rsrc(base + (int64_t)c0 * ROW, (uint32_t)(nc * ROW) * 4u);
#pragma unroll
            for (int e = 0; e < PER; ++e) v[e] = __builtin_bit_cast(float, q4::buf_load_x1(r, (e * 256 + tid) * 4, 0));
            __syncthreads();  // the previous tile is no longer read
        }
#pragma unroll
        for (int e = 0; e < PER; ++e)
            if (e * 256 + tid < kTile * ROW) tile[e * 256 + tid] = v[e];
        __syncthreads();
        if (tid < nc) ec[tid] = expf(tile[tid * ROW] - M);
        __syncthreads();
        if (tid < D) {
            for (int c = 0; c < nc; ++c) acc = __builtin_fmaf(tile[c * ROW + 2 + tid], ec[c], acc);
        }
        if (tid == 0) {
            for (int c = 0; c < nc; ++c) lsum = __builtin_fmaf(tile[c * ROW + 1], ec[c], lsum);
        }
    }
    if (tid == 0) red[0] = lsum;
    __syncthreads();
    if (tid < D) o[(int64_t)h * D + tid] = acc / red[0];
}

// Workgroup (h, c) of 4 waves; wave w's l-th load covers the TPL consecutive tokens
// (l * 4 + w) * TPL .. + TPL - 1 of the chunk (CH = 4 * TPL * NL tokens), lane
// tl * LPT + j holding token tl's dimensions [32j, 32j + 32).  Every K and V load of the
// chunk is issued before any arithmetic (K_0, V_0, K_1, V_1, ...), so a wave keeps 2 NL
// 16-byte loads per lane in flight, and works on each batch as soon as it has arrived
// (scores, weights against a wave-wide reference maximum, weighted values); the tokens of
// each row of 16 lanes are summed with DPP, and the rows and waves (rescaled by
// e^(m_wave - m_chunk)) through LDS, once, at the end.
template <int D, int G, bool SYM, bool XF16, int NL>
__global__ __launch_bounds__(kThreads) void kv_partial_kernel(const KvArgs a) {
    constexpr int LPT = D / 32;               // lanes per token
    constexpr int TPL = 64 / LPT;             // tokens per wave-wide load
    constexpr int CH = kWaves * TPL * NL;     // tokens per chunk
    constexpr int NG = D / G;                 // groups per token
    constexpr int ZW = (NG + 7) / 8;          // zero-point words per token
    const int h = blockIdx.x / a.chunks, c = blockIdx.x - h * a.chunks;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int j = lane % LPT;
    const int tl = lane / LPT;
    const int grp = (32 * j) / G;
    const int t_begin = c * CH;
    const int ntok = a.t - t_begin < CH ? a.t - t_begin : CH;
    const int64_t row0 = (int64_t)h * a.t_cap + t_begin;

    const q4::rsrc rk = q4::make_rsrc(a.kq + row0 * (D / 8), (uint32_t)ntok * (D / 2));
    const q4::rsrc rks = q4::make_rsrc(a.ks + row0 * NG, (uint32_t)ntok * NG * 2u);
    const q4::rsrc rkz = q4::make_rsrc(SYM ? (const void*)a.ks : (const void*)(a.kz + row0 * ZW),
                                       SYM ? 0u : (uint32_t)ntok * ZW * 4u);
    const q4::rsrc rv = q4::make_rsrc(a.vq + row0 * (D / 8), (uint32_t)ntok * (D / 2));
    const q4::rsrc rvs = q4::make_rsrc(a.vs + row0 * NG, (uint32_t)ntok * NG * 2u);
    const q4::rsrc rvz = q4::make_rsrc(SYM ? (const void*)a.vs : (const void*)(a.vz + row0 * ZW),
                                       SYM ? 0u : (uint32_t)ntok * ZW * 4u);

    // the query's 32 values of this lane (first: the scores need them first)
    q4::u32x4 qw[4];
    {
        // one descriptor for the head's row (uniform), the lane's 64 bytes by offset
        const q4::rsrc rqv = q4::make_rsrc(reinterpret_cast<const uint16_t*>(a.q) + (int64_t)h * D, 2u * D);
#pragma unroll
        for (int v = 0; v < 4; ++v) qw[v] = q4::buf_load_x4(rqv, 64 * j + 16 * v, 0);
    }
    // every load of the chunk; a token past the end reads as zero (offset past the range)
    q4::u32x4 kc[NL], vc[NL];
    uint32_t ksc[NL], vsc[NL], kzw[NL], vzw[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l) {
        const int tt = (l * kWaves + w) * TPL + tl;
        const bool live = tt < ntok;
        const int co = live ? (tt * (D / 8) + 4 * j) * 4 : (int)kOff;
        const int so = live ? (tt * NG + grp) * 2 : (int)kOff;
        const int zo = live ? (tt * ZW + grp / 8) * 4 : (int)kOff;
        kc[l] = q4::buf_load_x4(rk, co, 0);
        ksc[l] = q4::buf_load_u16(rks, so, 0);
        kzw[l] = SYM ? 0u : q4::buf_load_x1(rkz, zo, 0);
        vc[l] = q4::buf_load_x4(rv, co, 0);
        vsc[l] = q4::buf_load_u16(rvs, so, 0);
        vzw[l] = SYM ? 0u : q4::buf_load_x1(rvz, zo, 0);
        // loads retire in issue order: keep each batch's loads together and in batch
        // order, and keep the scheduler from sinking them towards their uses
        __builtin_amdgcn_sched_barrier(0);
    }

    float qv[32];
    float qsum = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t wd = qw[v][e];
            if constexpr (XF16) {
                qv[8 * v + 2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd & 0xFFFFu));
                qv[8 * v + 2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd >> 16));
            } else {
                qv[8 * v + 2 * e] = __builtin_bit_cast(float, wd << 16);
                qv[8 * v + 2 * e + 1] = __builtin_bit_cast(float, wd & 0xFFFF0000u);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) qsum += qv[i];

    // ---- each batch as soon as its K and V have arrived: scores, weights against the
    // wave's reference m_w, weighted values.  Per lane acc_i = sum p S u_i over its tokens,
    // accz = sum p S z, lsum = sum p.  m_w is the first batch's maximum score; softmax only
    // needs the exponents in range, so m_w moves (and the sums are rescaled) only when a
    // score exceeds it by more than 40 (e^40 keeps every sum far from fp32 overflow).
    float m_w = -INFINITY;
    float lsum = 0.f, accz = 0.f;
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;
#pragma unroll
    for (int l = 0; l < NL; ++l) {
        const int tt = (l * kWaves + w) * TPL + tl;
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float f[8];
            unpack8(kc[l][e], f);
#pragma unroll
            for (int i = 0; i < 8; ++i) dot = __builtin_fmaf(qv[8 * e + i], f[i], dot);
        }
        const uint32_t zk = SYM ? 8u : (kzw[l] >> (4 * (grp % 8))) & 0xFu;
        float sc = token_sum<LPT>(q4::f16_bits_to_float((uint16_t)ksc[l]) * (dot - (float)zk * qsum));
        sc = tt < ntok ? sc * a.scale : -INFINITY;
        if (l == 0) {
            m_w = wave_max(sc);  // -inf only for a wave without live tokens: then every p is 0
        } else if (__any(sc > m_w + 40.f)) {
            const float m_new = wave_max(fmaxf(sc, m_w));
            const float f = expf(m_w - m_new);
            lsum *= f;
            accz *= f;
#pragma unroll
            for (int i = 0; i < 32; ++i) acc[i] *= f;
            m_w = m_new;
        }
        const float p = sc == -INFINITY ? 0.f : expf(sc - m_w);
        lsum += p;
        const uint32_t zv = SYM ? 8u : (vzw[l] >> (4 * (grp % 8))) & 0xFu;
        const float ps = p * q4::f16_bits_to_float((uint16_t)vsc[l]);
        accz = __builtin_fmaf(ps, (float)zv, accz);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float f[8];
            unpack8(vc[l][e], f);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[8 * e + i] = __builtin_fmaf(ps, f[i], acc[8 * e + i]);
        }
    }

    // ---- sums over each row's tokens (DPP), row leaders to LDS: per (wave, row, j) the
    // 32 dimension sums, the z term and the weight sum; the wave maxima beside them
    constexpr int REC = 34;                         // floats per (wave, row, j) record
    __shared__ float red[kWaves * 4 * LPT * REC];
    __shared__ float wmax[kWaves];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = row_dim_sum<LPT>(acc[i]);
    accz = row_dim_sum<LPT>(accz);
    lsum = row_dim_sum<LPT>(lsum);
    if ((lane & 15) < LPT) {
        float* r = red + ((w * 4 + (lane >> 4)) * LPT + j) * REC;
#pragma unroll
        for (int i = 0; i < 32; ++i) r[i] = acc[i];
        r[32] = accz;
        r[33] = lsum;
    }
    if (lane == 0) wmax[w] = m_w;
    __syncthreads();

    // ---- merge the waves and rows (in order) and write the chunk's (m_c, l_c, o_c)
    float m_c = wmax[0];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) m_c = fmaxf(m_c, wmax[v]);
    float fw[kWaves];
#pragma unroll
    for (int v = 0; v < kWaves; ++v) fw[v] = wmax[v] == -INFINITY ? 0.f : expf(wmax[v] - m_c);
    float* out = a.ws + ((int64_t)h * a.chunks + c) * (D + 2);
    for (int i = threadIdx.x; i < D; i += kThreads) {
        const int jj = i / 32, ii = i % 32;
        float sv = 0.f, sz = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float* rec = red + ((v * 4 + r) * LPT + jj) * REC;
                sv = __builtin_fmaf(rec[ii], fw[v], sv);
                sz = __builtin_fmaf(rec[32], fw[v], sz);
            }
        }
        out[2 + i] = sv - sz;
    }
    if (threadIdx.x == 0) {
        float sl = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sl = __builtin_fmaf(red[((v * 4 + r) * LPT) * REC + 33], fw[v], sl);
        }
        out[0] = m_c;
        out[1] = sl;
    }
}

template <int D, int G, bool SYM, bool XF16>
hipError_t launch_nl(const KvArgs& a, int nl, int heads, hipStream_t st) {
    const dim3 grid(heads * a.chunks), block(kThreads);
    switch (nl) {
    case 1: hipLaunchKernelGGL((kv_partial_kernel<D, G, SYM, XF16, 1>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((kv_partial_kernel<D, G, SYM, XF16, 2>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((kv_partial_kernel<D, G, SYM, XF16, 4>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((kv_partial_kernel<D, G, SYM, XF16, 8>), grid, block, 0, st, a); break;
    }
    return q4k_launched(XF16 ? "q4_kv_partial_f16" : "q4_kv_partial_bf16");
}

template <int D, int G, bool SYM>
hipError_t launch_d(const KvArgs& a, int xd, int nl, int heads, hipStream_t st) {
    return xd == 1 ? launch_nl<D, G, SYM, true>(a, nl, heads, st)
                   : launch_nl<D, G, SYM, false>(a, nl, heads, st);
}

template <int D>
hipError_t launch_g(const KvArgs& a, int xd, int g, int sym, int nl, int heads, hipStream_t st) {
    if constexpr (D >= 32) {
        if (g == 32) return sym ? launch_d<D, 32, true>(a, xd, nl, heads, st) : launch_d<D, 32, false>(a, xd, nl, heads, st);
    }
    if constexpr (D >= 64) {
        if (g == 64) return sym ? launch_d<D, 64, true>(a, xd, nl, heads, st) : launch_d<D, 64, false>(a, xd, nl, heads, st);
    }
    if constexpr (D >= 128) {
        if (g == 128) return sym ? launch_d<D, 128, true>(a, xd, nl, heads, st) : launch_d<D, 128, false>(a, xd, nl, heads, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// ---------------------------------------------------------------------------------------
// Scratch for callers that cannot allocate (q4_kv_attention_noalloc): the per-chunk
// partials go to this fixed array instead of a caller workspace.  Every GPU the library
// runs on holds its own copy until the process ends.  Host code never uses the array's
// name as an address (on the host it is a stand-in, not device memory): the device
// address comes from hipGetSymbolAddress, once per device, with that device current.
// The array has external linkage: the runtime finds a device variable by its symbol in
// the code object, and an internal-linkage (static) one is emitted as a local symbol it
// cannot look up.
__device__ __align__(256) unsigned char q4_kv_noalloc_scratch[kKvScratchBytes];
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t q4k_kv_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(q4_kv_noalloc_scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

void q4k_kv_attention_shape(int64_t heads, int64_t d, int64_t n_tok, int* chunks, int* loads) {
    // the most loads per wave (longest chunks) that still give at least 512 workgroups
    // (two per CU of a 256-CU chip), at least one load; depends on the sizes alone, so
    // the summation order does too
    const int64_t tpl = 64 / (d / 32);
    int nl = 8;
    while (nl > 1 && heads * ((n_tok + kWaves * tpl * nl - 1) / (kWaves * tpl * nl)) < 512) nl /= 2;
    *loads = nl;
    *chunks = (int)((n_tok + kWaves * tpl * nl - 1) / (kWaves * tpl * nl));
}

int64_t q4k_kv_max_chunks(int64_t d, int64_t n_tok) {
    return (n_tok * d + 8191) / 8192;  // chunks of one load per wave: the most there can be
}

hipError_t q4k_kv_attention(const void* q, int xd, const uint32_t* kq, const uint16_t* ks,
                            const uint32_t* kz, const uint32_t* vq, const uint16_t* vs,
                            const uint32_t* vz, int64_t heads, int64_t d, int64_t t, int64_t t_cap,
                            int g, int sym, float scale, float* out, float* workspace, int chunks,
                            int loads, hipStream_t st, const char** kname) {
    KvArgs a{q, kq, ks, kz, vq, vs, vz, workspace, (int)t, (int)t_cap, chunks, scale};
    hipError_t e;
    switch (d) {
    case 64: e = launch_g<64>(a, xd, g, sym, loads, (int)heads, st); break;
    case 128: e = launch_g<128>(a, xd, g, sym, loads, (int)heads, st); break;
    default: e = launch_g<256>(a, xd, g, sym, loads, (int)heads, st); break;
    }
    if (e != hipSuccess) return e;
    const dim3 cg((unsigned)heads), cb(256);
    if (d == 64)
        hipLaunchKernelGGL(kv_combine_kernel<64>, cg, cb, 0, st, workspace, chunks, out);
    else if (d == 128)
        hipLaunchKernelGGL(kv_combine_kernel<128>, cg, cb, 0, st, workspace, chunks, out);
    else
        hipLaunchKernelGGL(kv_combine_kernel<256>, cg, cb, 0, st, workspace, chunks, out);
    *kname = xd == 1 ? "q4_kv_attention_f16" : "q4_kv_attention_bf16";
    return q4k_launched("q4_kv_combine");
}
