// quant_pack.hip — RTN quantize-and-pack of W [n][k] into the canonical packed format
// for gfx950.
//
// Method: the affine quantizer q = clamp(round(w/s) + z, q_min, q_max) of
// "LLM Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV Cache (7/10)" (blog.ruahverce.com),
// §Affine Quantization, with per-group statistics (§Per-group: g consecutive weights
// share one scale) and the symmetric / asymmetric scale and zero point of
// §Symmetric과 Asymmetric; INT4 code ranges [-8,7] / [0,15] from
// "Quantization Algorithms 단권화" §Signed ↔ Unsigned; round-to-nearest as the
// calibration-free RTN baseline of the same page (§Calibration-free).
//
// Work mapping (2 or 4 bytes read and 0.5 byte written per weight; the exact arithmetic
// makes the kernel about as much VALU-bound as HBM-bound):
//   one wave task = one row x 16 consecutive groups = two 32-bit zero-point words;
//   lane l handles E = g/4 consecutive weights of group l/4; the 4 lanes of a group
//   reduce min/max (or max|w|) with two xor shuffles; each lane then packs its E codes
//   (E/8 words) and the wave writes a contiguous run of 8*g bytes of qweight.  Each half
//   wave OR-combines the 8 zero points of its word.  Four lanes per group (rather than
//   eight) halve the per-weight cost of the group's scale, zero point and reciprocal,
//   which every lane of the group computes.
//
// Arithmetic is IEEE fp32 in the order written (no contraction, correctly rounded
// divisions for the scale and zero point, round-half-to-even), so codes, scales and zero
// points are bit-identical to the plain CPU definition.  The per-weight quotient w/S of
// 16-bit weights comes from a reciprocal and one FMA correction whose rounded value equals
// that of the IEEE quotient for every reachable (w, S) pair, a property checked
// exhaustively by the test suite; fp32 weights use the IEEE division itself.
#include "quant_common.h"

#pragma clang fp contract(off)

namespace {

using namespace q4q;

// Persistent waves over the (row, zero-word pair) tasks of every problem of the launch, one
// problem after another.  For a problem with Z = min(zero-word pairs per row, waves) and
// R = min(waves / Z, n), wave gw starts at (row r0, pair z0) = (gw / Z, gw % Z) and steps
// by R rows and Z pairs, so every task is done exactly once and consecutive matrices of a
// grouped launch form one stream.
template <int G, bool SYM, int DT>
__global__ __launch_bounds__(256) void quant_pack_kernel(const q4::QuantBatch bt) {
    constexpr int ZT = 2;                   // zero-point words per task
    constexpr int E = G * ZT / 8;           // weights per lane
    constexpr int LPG = G / E;              // lanes per group
    constexpr uint32_t EB = DT == 0 ? 4 : 2;  // bytes per weight
    constexpr uint32_t kOff = 0xFFFFFFF0u;   // an offset past every resource
    const int lane = threadIdx.x & 63;
    const int waves = (int)gridDim.x * (int)(blockDim.x >> 6);
    const int gw = (int)blockIdx.x * (int)(blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane / LPG;             // group within the task
    const int t = lane % LPG;
    for (int pi = 0; pi < bt.count; ++pi) {
        const void* __restrict__ w = bt.p[pi].w;
        uint32_t* __restrict__ qweight = bt.p[pi].qweight;
        uint16_t* __restrict__ scales = bt.p[pi].scales;
        uint32_t* __restrict__ zeros = bt.p[pi].zeros;
        const int n = bt.p[pi].n, k = bt.p[pi].k;
        const int heads = bt.p[pi].heads, t_cap = bt.p[pi].t_cap, t0 = bt.p[pi].t0;
        const int n_groups = k / G;
        const int zwords = (n_groups + 7) >> 3;
        const int zpairs = (zwords + ZT - 1) / ZT;
        const int Z = zpairs < waves ? zpairs : waves;
        const int R = waves / Z < n ? waves / Z : n;
        const int r0 = gw / Z, z0 = gw - r0 * Z;
        if (r0 >= R) continue;  // wave-uniform: the waves past R * Z sit this problem out

        // one task's weights (none past the last row: an offset past the resource)
        auto issue = [&](int rr, int zz, float (&dst)[E]) {
            const bool live = rr < n;
            const q4::rsrc rw = q4::make_rsrc(reinterpret_cast<const char*>(w) + (int64_t)(live ? rr : 0) * k * EB,
                                              (uint32_t)k * EB);
            const int gi = zz * 8 * ZT + grp;
            const uint32_t el = (uint32_t)gi * G + (uint32_t)t * E;
            load_slice<E, DT>(rw, live && gi < n_groups ? el * EB : kOff, dst);
        };
        // tasks in order (row, zero word), the next task's weights loaded before this
        // task's arithmetic so that one load is always in flight behind the compute
        int row = r0, zw = z0;
        float vn[E];
        issue(row, zw, vn);
        while (row < n) {
            float v[E];
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = vn[e];
            int nrow = row, nzw = zw + Z;
            if (nzw >= zpairs) {
                nzw = z0;
                nrow = row + R;
            }
            issue(nrow, nzw, vn);
            {
                // output row: the same row, or the (head, token) slot of a KV cache
                const int64_t orow = heads > 0 ? (int64_t)(row % heads) * t_cap + t0 + row / heads : row;
                const q4::rsrc rq = q4::make_rsrc(qweight + orow * (k / 8), (uint32_t)k / 2u);
                const q4::rsrc rs = q4::make_rsrc(scales + orow * n_groups, (uint32_t)n_groups * 2u);
                const q4::rsrc rz = q4::make_rsrc(zeros + orow * zwords, (uint32_t)zwords * 4u);
                const int gidx = zw * 8 * ZT + grp;
                const bool valid = gidx < n_groups;
                const uint32_t elem = (uint32_t)gidx * G + (uint32_t)t * E;  // within the row

                uint16_t s16;
                int zi;
                uint32_t packed[(E + 7) / 8];
                quant_group<G, SYM, DT>(v, s16, zi, packed);

                // codes: E/2 bytes per lane, contiguous across the wave
                const uint32_t qoff = valid ? elem / 2u : kOff;
                if constexpr (E == 32) {
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(q4::u32x4, q4::u32x4{packed[0], packed[1], packed[2], packed[3]}), rq,
                        (int)qoff, 0, 0);
                } else if constexpr (E == 16) {
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(q4::u32x2, q4::u32x2{packed[0], packed[1]}),
                                                          rq, (int)qoff, 0, 0);
                } else {  // E == 8
                    __builtin_amdgcn_raw_buffer_store_b32(packed[0], rq, (int)qoff, 0, 0);
                }
                __builtin_amdgcn_raw_buffer_store_b16(s16, rs, (int)(valid && t == 0 ? (uint32_t)gidx * 2u : kOff), 0, 0);
                if constexpr (!SYM) {
                    // the 8 groups of each zero word sit in one half wave (lanes 32 h ..)
                    uint32_t zn = valid ? ((uint32_t)zi << (4 * (grp & 7))) : 0u;
#pragma unroll
                    for (int m = LPG; m < 32; m <<= 1) zn |= __shfl_xor(zn, m, 64);
                    const int word = zw * ZT + (lane >> 5);
                    const bool head = (lane & 31) == 0 && word < zwords;
                    __builtin_amdgcn_raw_buffer_store_b32(zn, rz, (int)(head ? (uint32_t)word * 4u : kOff), 0, 0);
                }
            }
            row = nrow;
            zw = nzw;
        }
    }
}

// KV-cache rows (head_dim d dividing 512, at most 8 groups): one wave task is 512/d
// consecutive tokens of one head (input rows t*heads + h, 512 weights), and lane l
// quantizes weights 8l .. 8l+7 of it: token 8l / d of the task, g/8 lanes per group, a
// row's d/8 lanes loading its d contiguous elements.  Tasks are numbered head-major and
// consecutive waves take consecutive tasks, so a workgroup's codes, scales and zero words
// land in consecutive cache slots of one head: contiguous runs, where tasks of consecutive
// input rows would spread each wave's small stores over every head's region.  Each wave
// keeps P tasks' loads in flight when there are tasks to spare.  The arithmetic is
// quant_group's, so the codes, scales and zero points are those of the row kernel.
template <int G, bool SYM, int DT>
__global__ __launch_bounds__(256) void kv_quant_kernel(const void* __restrict__ kv, int rows, int d, int heads,
                                                       int t_cap, int t0, uint32_t* __restrict__ qc,
                                                       uint16_t* __restrict__ sc, uint32_t* __restrict__ zc) {
    constexpr int E = 8, P = 4, LPG = G / E;
    constexpr uint32_t EB = DT == 0 ? 4 : 2;
    constexpr uint32_t kOff = 0xFFFFFFF0u;
    const int lane = threadIdx.x & 63;
    const int waves = (int)gridDim.x * (int)(blockDim.x >> 6);
    const int gw = (int)blockIdx.x * (int)(blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rpt = 512 / d;                  // tokens per task
    const int ro = (8 * lane) / d;            // this lane's token within the task
    const int el = 8 * lane - ro * d;         // its first element within the row
    const int gr = el / G;                    // its group within the row
    const int lpr = d / 8;                    // lanes per row
    const int t_new = rows / heads;
    const int tbn = (t_new + rpt - 1) / rpt;  // tasks per head
    const int tasks = heads * tbn;
    const q4::rsrc rw = q4::make_rsrc(kv, (uint32_t)rows * (uint32_t)d * EB);
    for (int b = gw; b < tasks; b += P * waves) {
        float v[P][E];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int tk = b + p * waves;
            const int h = tk / tbn, t = (tk - h * tbn) * rpt + ro;
            const bool live = tk < tasks && t < t_new;
            load_slice<E, DT>(rw, live ? ((uint32_t)(t * heads + h) * (uint32_t)d + (uint32_t)el) * EB : kOff, v[p]);
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int tk = b + p * waves;
            if (tk >= tasks) break;  // wave-uniform
            const int h = tk / tbn, t = (tk - h * tbn) * rpt + ro;
            uint16_t s16;
            int zi;
            uint32_t packed[1];
            quant_group<G, SYM, DT, E>(v[p], s16, zi, packed);
            // the row's zero word: the nibbles of its groups, OR-ed over the row's lanes
            uint32_t zn = (uint32_t)zi << (4 * gr);
#pragma unroll
            for (int m = LPG; m < 64; m <<= 1)
                if (m < lpr) zn |= __shfl_xor(zn, m, 64);
            if (t < t_new) {
                const int64_t orow = (int64_t)h * t_cap + t0 + t;
                qc[orow * (d / 8) + el / 8] = packed[0];
                if (el % G == 0) sc[orow * (d / G) + gr] = s16;
                if (!SYM && el == 0) zc[orow * ((d / G + 7) / 8)] = zn;
            }
        }
    }
}

template <int G, bool SYM>
hipError_t launch_dt(const q4::QuantBatch& bt, int dt, hipStream_t st, const char** kname) {
    const int num_cus = q4k_device_cus();
    // enough waves to keep every SIMD busy (8 per SIMD), no more than the largest problem
    // has tasks
    const int64_t cap = (int64_t)num_cus * 32;
    int64_t tasks = 0;
    for (int i = 0; i < bt.count; ++i) {
        const int64_t t = (int64_t)bt.p[i].n * (((bt.p[i].k / G + 7) / 8 + 1) / 2);  // zero-word pairs
        tasks = t > tasks ? t : tasks;
    }
    const int64_t waves = tasks < cap ? tasks : cap;
    const int64_t blocks = (waves + 3) / 4;
    static const char* names[3] = {"q4_quant_pack_f32", "q4_quant_pack_f16", "q4_quant_pack_bf16"};
    *kname = names[dt];
    const dim3 grid((unsigned)blocks), block(256);
    if (dt == 0)
        hipLaunchKernelGGL((quant_pack_kernel<G, SYM, 0>), grid, block, 0, st, bt);
    else if (dt == 1)
        hipLaunchKernelGGL((quant_pack_kernel<G, SYM, 1>), grid, block, 0, st, bt);
    else
        hipLaunchKernelGGL((quant_pack_kernel<G, SYM, 2>), grid, block, 0, st, bt);
    return q4k_launched(*kname);
}

hipError_t launch_batch(const q4::QuantBatch& bt, int w_dtype, int g, int sym, hipStream_t st,
                        const char** kname) {
    switch (g * 2 + (sym ? 1 : 0)) {
    case 64: return launch_dt<32, false>(bt, w_dtype, st, kname);
    case 65: return launch_dt<32, true>(bt, w_dtype, st, kname);
    case 128: return launch_dt<64, false>(bt, w_dtype, st, kname);
    case 129: return launch_dt<64, true>(bt, w_dtype, st, kname);
    case 256: return launch_dt<128, false>(bt, w_dtype, st, kname);
    default: return launch_dt<128, true>(bt, w_dtype, st, kname);
    }
}

}  // namespace

hipError_t q4k_quant_pack(const void* w, int w_dtype, int64_t n, int64_t k, int g, int sym,
                          uint32_t* qweight, uint16_t* scales, uint32_t* zeros,
                          hipStream_t stream, const char** kname) {
    q4::QuantBatch bt{};
    bt.p[0] = q4::QuantProblem{w, qweight, scales, zeros, (int)n, (int)k};
    bt.count = 1;
    return launch_batch(bt, w_dtype, g, sym, stream, kname);
}

namespace {
template <int G, bool SYM>
hipError_t launch_kv(const void* kv, int dt, int rows, int d, int heads, int t_cap, int t0, uint32_t* qc,
                     uint16_t* sc, uint32_t* zc, hipStream_t st) {
    const int64_t tasks = (int64_t)heads * ((rows / heads + 512 / d - 1) / (512 / d));
    const int64_t cap = (int64_t)q4k_device_cus() * 32;
    const int64_t waves = tasks < cap ? tasks : cap;  // one task per wave while they last
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (dt == 0)
        hipLaunchKernelGGL((kv_quant_kernel<G, SYM, 0>), grid, block, 0, st, kv, rows, d, heads, t_cap, t0, qc, sc, zc);
    else if (dt == 1)
        hipLaunchKernelGGL((kv_quant_kernel<G, SYM, 1>), grid, block, 0, st, kv, rows, d, heads, t_cap, t0, qc, sc, zc);
    else
        hipLaunchKernelGGL((kv_quant_kernel<G, SYM, 2>), grid, block, 0, st, kv, rows, d, heads, t_cap, t0, qc, sc, zc);
    static const char* names[3] = {"q4_kv_quant_f32", "q4_kv_quant_f16", "q4_kv_quant_bf16"};
    return q4k_launched(names[dt]);
}
}  // namespace

hipError_t q4k_kv_quantize(const void* kv, int dtype, int64_t t_new, int64_t heads, int64_t d, int g,
                           int sym, int64_t t_cap, int64_t t0, uint32_t* qcache, uint16_t* scache,
                           uint32_t* zcache, hipStream_t stream, const char** kname) {
    static const char* names[3] = {"q4_kv_quant_f32", "q4_kv_quant_f16", "q4_kv_quant_bf16"};
    const int64_t in_bytes = t_new * heads * d * (dtype == 0 ? 4 : 2);
    // rows that divide a 512-weight task and hold at most one zero-point word
    if (512 % d == 0 && d / g <= 8 && in_bytes < ((int64_t)1 << 31)) {
        const int rows = (int)(t_new * heads), di = (int)d, hi = (int)heads, tc = (int)t_cap, t0i = (int)t0;
        hipError_t e;
        switch (g * 2 + (sym ? 1 : 0)) {
        case 64: e = launch_kv<32, false>(kv, dtype, rows, di, hi, tc, t0i, qcache, scache, zcache, stream); break;
        case 65: e = launch_kv<32, true>(kv, dtype, rows, di, hi, tc, t0i, qcache, scache, zcache, stream); break;
        case 128: e = launch_kv<64, false>(kv, dtype, rows, di, hi, tc, t0i, qcache, scache, zcache, stream); break;
        case 129: e = launch_kv<64, true>(kv, dtype, rows, di, hi, tc, t0i, qcache, scache, zcache, stream); break;
        case 256: e = launch_kv<128, false>(kv, dtype, rows, di, hi, tc, t0i, qcache, scache, zcache, stream); break;
        default: e = launch_kv<128, true>(kv, dtype, rows, di, hi, tc, t0i, qcache, scache, zcache, stream); break;
        }
        *kname = names[dtype];
        return e;
    }
    q4::QuantBatch bt{};
    bt.p[0] = q4::QuantProblem{kv, qcache, scache, zcache, (int)(t_new * heads), (int)d,
                               (int)heads, (int)t_cap, (int)t0};
    bt.count = 1;
    const hipError_t e = launch_batch(bt, dtype, g, sym, stream, kname);
    *kname = names[dtype];
    return e;
}

hipError_t q4k_quant_pack_grouped(const q4::QuantProblem* problems, int count, int w_dtype, int g,
                                  int sym, hipStream_t stream, const char** kname) {
    if (count < 1 || count > q4::kMaxGroup) return hipErrorInvalidValue;
    q4::QuantBatch bt{};
    for (int i = 0; i < count; ++i) bt.p[i] = problems[i];
    bt.count = count;
    return launch_batch(bt, w_dtype, g, sym, stream, kname);
}
