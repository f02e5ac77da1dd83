// gemm.hip — prefill W4A16 linear layer (m > 16) for gfx950.
//
//   y[m][n] = sum_g S[n][g] * sum_{k in g} x[m][k] * (u[n][k] - z[n][g])
//
// Large-batch prefill is compute-bound ("LLM Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV
// Cache (7/10)", §Batch와 Context에 따라 속도가 달라진다), so this is a dense MFMA
// contraction with the dequantization fused into the operand path (path A of
// §Kernel이 없으면 압축 이점이 사라진다).
//
// Tiles.  A workgroup of 4 waves computes a 128 x 256 block of y (128 activation rows x
// 256 weight rows); wave w owns all 128 rows x weight rows [64w, 64w+64) as 4 x 2 tiles
// of v_mfma_f32_32x32x16 (bf16 or fp16 inputs, fp32 accumulation).  The K loop walks 64
// columns per stage.
//
// Operands.  Activations are shared by the 4 waves: they go from HBM/L2 straight into a
// three-stage LDS ring with buffer-to-LDS loads (no registers), two stages ahead of the
// MFMAs, in an XOR-swizzled layout (16-byte chunk c of row r at position c ^ (r & 7)) that
// makes both the 1 KB loads and the operand reads bank-conflict free.  Weights are not
// shared: each lane of the 32x32x16 MFMA's weight operand needs 8 consecutive k of one
// weight row, which is exactly one packed word, so every lane loads its own words (and
// the scale and zero point of its row) into registers two stages ahead and dequantizes
// them right before the MFMA.  Every stage issues the same loads in the same order, so
// each wait is a fixed count and the two stages in flight stay in flight.
//
// k slots.  An MFMA consumes 16 k: lanes 0-31 supply 8 and lanes 32-63 another 8.  With
// g >= 64 lane half h takes words 4h..4h+3 of the stage (one 16-byte load) and MFMA kk
// uses word 4h+kk; with g = 32 the halves interleave (words 2h, 2h+1, 4+2h, 5+2h) so each
// MFMA stays inside one group.  The activation operand reads the matching chunks.
//
// Exactness.  The weight operand is the exact small integer u - z (|u - z| <= 15, exact
// in bf16 and fp16), so every product is exact and every sum is fp32.  The per-group
// scale is applied without a second set of accumulators: within group g the accumulator
// is kept in units of S[n][g]; entering group g it is multiplied by S[n][g-1] / S[n][g],
// and the epilogue multiplies by the last group's scale.  A group with S = 0 contributes
// nothing (its operand is zeroed and the units stay those of the previous group).
//
// Placement.  Consecutive workgroups land on consecutive XCDs (8 per MI355X), so block b
// takes activation block b % mtiles: with 16 row blocks (m = 2048) each XCD's L2 holds
// two 2 MB activation blocks while the packed weights stream through.
#include "q4_launch.h"

namespace {

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int NTHREADS = 256;
constexpr int RING = 3;                   // LDS stages of activations
constexpr int A_STAGE = BM * BK * 2;      // bytes of one activation stage (16 KB)
constexpr uint32_t kOOB = 0x80000000u;    // an offset past every resource: reads 0

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ f32x16 mfma32_bf16(q4::u32x4 a, q4::u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(q4::bf16x8, a),
                                                   __builtin_bit_cast(q4::bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f16(q4::u32x4 a, q4::u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(q4::f16x8, a),
                                                  __builtin_bit_cast(q4::f16x8, b), c, 0, 0, 0);
}

// 8 codes of one packed word minus z, as exact 16-bit floats in natural k order
// (elements 0..7 = k 8j..8j+7).  Bytes 128 + u - z (no borrow between bytes), then XOR 0x80
// gives u - z as signed bytes, converted exactly to fp32 and narrowed by keeping the upper
// half (bf16) or converting (fp16; small integers are exact either way).
template <bool XF16>
__device__ __forceinline__ q4::u32x4 dequant_word(uint32_t w, uint32_t zrep) {
    const uint32_t lo = (((w & 0x0F0F0F0Fu) | 0x80808080u) - zrep) ^ 0x80808080u;         // k 0,2,4,6
    const uint32_t hi = ((((w >> 4) & 0x0F0F0F0Fu) | 0x80808080u) - zrep) ^ 0x80808080u;  // k 1,3,5,7
    q4::u32x4 r;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const float e = (float)(int8_t)((lo >> (8 * b)) & 0xFF);
        const float o = (float)(int8_t)((hi >> (8 * b)) & 0xFF);
        if constexpr (XF16) {
            const q4::f16x2 v = {(_Float16)e, (_Float16)o};
            r[b] = __builtin_bit_cast(uint32_t, v);
        } else {
            // upper halves of the two fp32 values: bytes 2,3 of e then bytes 2,3 of o
            r[b] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, o), __builtin_bit_cast(uint32_t, e), 0x07060302u);
        }
    }
    return r;
}

// word of the stage (0..7) that lane half h feeds to MFMA kk
template <int G>
__device__ __forceinline__ constexpr int word_of(int kk, int h) {
    return G >= 64 ? 4 * h + kk : (kk & 1) + 2 * h + 4 * (kk >> 1);
}

// Per-lane weight-side registers of one stage: the lane's 4 words for each of its two
// 32-row blocks, the scales of the stage's groups (1, or 2 when g = 32) and the zero word.
template <int G>
struct BStage {
    static constexpr int NGS = G == 32 ? 2 : 1;
    uint32_t w[2][4];
    uint32_t s[2][NGS];
    uint32_t z[2];
};

template <int G, bool SYM, bool XF16>
__global__ __launch_bounds__(NTHREADS, 2) void gemm_kernel(const uint16_t* __restrict__ x, int M,
                                                          const uint32_t* __restrict__ qweight,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint32_t* __restrict__ zeros,
                                                          int N, int K, void* __restrict__ y, int ydt) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // RING x A_STAGE
    constexpr int NGS = BStage<G>::NGS;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int mtiles = (M + BM - 1) / BM;
    const int mt = (int)blockIdx.x % mtiles, nt = (int)blockIdx.x / mtiles;  // XCD-friendly order
    const int m0 = mt * BM, n0 = nt * BN;
    const int KW = K / 8;
    const int n_groups = K / G;
    const int zwords = (n_groups + 7) >> 3;
    const int stages = (K + BK - 1) / BK;

    // activations of this row block
    const int arows = __builtin_amdgcn_readfirstlane(M - m0 < BM ? M - m0 : BM);
    const q4::rsrc rx = q4::make_rsrc(x + (int64_t)m0 * K, (uint32_t)arows * (uint32_t)K * 2u);
    // this wave's 64 weight rows
    const int wn0 = n0 + 64 * wave;
    int wrows = N - wn0;
    wrows = wrows < 0 ? 0 : (wrows > 64 ? 64 : wrows);
    // uniform values computed with vector instructions: pin them to scalars, or every load
    // through the resources below becomes a waterfall loop
    wrows = __builtin_amdgcn_readfirstlane(wrows);
    const int wbase = __builtin_amdgcn_readfirstlane(wrows > 0 ? wn0 : 0);
    const q4::rsrc rq = q4::make_rsrc(qweight + (int64_t)wbase * KW, (uint32_t)wrows * (uint32_t)KW * 4u);
    const q4::rsrc rs = q4::make_rsrc(scales + (int64_t)wbase * n_groups, (uint32_t)wrows * (uint32_t)n_groups * 2u);
    const q4::rsrc rz = q4::make_rsrc(zeros + (int64_t)wbase * zwords, (uint32_t)wrows * (uint32_t)zwords * 4u);

    const int col = lane & 31, h = lane >> 5;

    // Per-lane parts of the load offsets; the per-stage part is a uniform scalar offset.
    // Rows past the end of a block read nothing (their per-lane offset carries kOOB), and
    // so do the loads for the two stages after the last one (issued by the pipeline, never
    // used): every mask goes into the per-lane offset.  The k tail (k % 64 == 32): the
    // activation chunks past k are read as zeros, so whatever the weight words past the
    // end of a row hold meets a zero.
    const int ca = (lane & 7) ^ ((lane >> 3) & 7);  // activation chunk this lane moves (DMA rows are 8-aligned)
    uint32_t aoff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        aoff[q] = ((uint32_t)(32 * wave + 8 * q + (lane >> 3)) * (uint32_t)K + 8u * ca) * 2u;
    const int tail_chunks = (K % BK) / 8;  // valid chunks of a short last stage (0: none short)
    const uint32_t tail_mask = tail_chunks != 0 && ca >= tail_chunks ? kOOB : 0u;
    uint32_t qoff[2], soff[2], zoff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t row = (uint32_t)(32 * j + col);
        const uint32_t rowmask = (int)row < wrows ? 0u : kOOB;
        qoff[j] = (row * (uint32_t)KW * 4u + (G >= 64 ? 16u : 8u) * h) | rowmask;
        soff[j] = (row * (uint32_t)n_groups * 2u) | rowmask;
        zoff[j] = (row * (uint32_t)zwords * 4u) | rowmask;
    }

    // ---- loads of one stage (fixed count and order: 4 activation DMAs, then per block j
    //      the words, the scales and the zero word)
    auto load_a = [&](int s) {  // rows [32 wave, +32) of stage s into ring slot s % RING
        const uint32_t tm = s >= stages ? kOOB : (s == stages - 1 ? tail_mask : 0u);
        const int so = __builtin_amdgcn_readfirstlane(2 * s * BK);
        uint8_t* slot = smem + (s % RING) * A_STAGE;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr)(slot + (32 * wave + 8 * q) * (BK * 2)), 16,
                                                     (int)(aoff[q] | tm), so, 0, 0);
    };
    auto load_b = [&](BStage<G>& b, int s) {
        const int wso = __builtin_amdgcn_readfirstlane(4 * s * (BK / 8));  // the stage's first word
        const int g0 = G == 128 ? (s >> 1) : (G == 64 ? s : 2 * s);        // its first group
        const int sso = __builtin_amdgcn_readfirstlane(2 * g0);
        const int zso = __builtin_amdgcn_readfirstlane(4 * (g0 >> 3));
        const uint32_t pm = s >= stages ? kOOB : 0u;  // past the last stage: read nothing
        // a short last stage (k % 64 == 32) holds words 0..3 and one group: the words and the
        // scale past the row read nothing
        const bool short_stage = s == stages - 1 && (K % BK) != 0;
        const uint32_t hm = short_stage && (G == 32 || h == 1) ? kOOB : 0u;  // words 4..7
        const uint32_t sm = short_stage ? kOOB : 0u;                         // second group
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if constexpr (G >= 64) {
                const q4::u32x4 t = q4::buf_load_x4(rq, (int)(qoff[j] | pm | hm), wso);
                b.w[j][0] = t[0]; b.w[j][1] = t[1]; b.w[j][2] = t[2]; b.w[j][3] = t[3];
            } else {
                const q4::u32x2 ta = q4::buf_load_x2(rq, (int)(qoff[j] | pm), wso);
                const q4::u32x2 tb = q4::buf_load_x2(rq, (int)(qoff[j] | pm | hm), wso + 16);
                b.w[j][0] = ta[0]; b.w[j][1] = ta[1]; b.w[j][2] = tb[0]; b.w[j][3] = tb[1];
            }
#pragma unroll
            for (int q = 0; q < NGS; ++q)
                b.s[j][q] = q4::buf_load_u16(rs, (int)(soff[j] | pm | (q == 1 ? sm : 0u)), sso + 2 * q);
            if constexpr (!SYM)
                b.z[j] = q4::buf_load_x1(rz, (int)(zoff[j] | pm), zso);
            else
                b.z[j] = 0u;
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    float s_cur[2] = {1.f, 1.f};
    int g_cur = -1;

    // LDS operand addresses: row 32i + col of the slot, chunk word_of(kk, h) at its swizzled
    // position ((32i + col) & 7 == col & 7, so one address per kk; i goes in the offset)
    uint32_t apos[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        apos[kk] = (uint32_t)col * (BK * 2) + ((uint32_t)(word_of<G>(kk, h) ^ (col & 7)) << 4);

    // ---- compute of one stage
    auto compute = [&](const BStage<G>& b, int s) {
        const uint8_t* slot = smem + (s % RING) * A_STAGE;
        float sn[NGS][2], ratio[NGS][2];
        uint32_t zrep[NGS][2];
        bool fresh[NGS], zmask[NGS];
#pragma unroll
        for (int q = 0; q < NGS; ++q) {  // the stage's groups (one, or two when g = 32)
            const int gk = G == 128 ? (s >> 1) : (G == 64 ? s : 2 * s + q);
            bool zs = false;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                sn[q][j] = q4::f16_bits_to_float((uint16_t)b.s[j][q]);
                zs = zs || sn[q][j] == 0.0f;
                const int z = SYM ? 8 : (int)((b.z[j] >> (4 * (gk & 7))) & 0xFu);
                zrep[q][j] = (uint32_t)z * 0x01010101u;
            }
            zmask[q] = __builtin_amdgcn_ballot_w64(zs) != 0;  // a zero scale anywhere in the wave
            // entering a new group (wave-uniform): the accumulator moves to its units
            fresh[q] = gk != g_cur;
#pragma unroll
            for (int j = 0; j < 2; ++j) ratio[q][j] = 1.0f;
            if (fresh[q]) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    ratio[q][j] = sn[q][j] != 0.0f && g_cur >= 0 ? s_cur[j] / sn[q][j] : 1.0f;
                    if (sn[q][j] != 0.0f) s_cur[j] = sn[q][j];
                }
                g_cur = gk;
            }
        }
        // g = 128: the activation operands of two MFMA k-slots are read from LDS ahead of
        // their MFMAs (32 registers), so each MFMA waits for a read issued long before.  At
        // g = 32 and 64 (a group boundary every stage or two per stage, with its rescale) the
        // extra registers would spill: one read per MFMA, as it is needed.
        constexpr int AP = G == 128 ? 2 : 1;
        q4::u32x4 aop[AP][4];
        q4::u32x4 bnext[2];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if constexpr (AP == 2) {
                if ((kk & 1) == 0) {
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            aop[k2][i] = *reinterpret_cast<const q4::u32x4*>(slot + apos[kk + k2] + i * 32 * (BK * 2));
                }
            }
            const int q = G == 32 ? (kk >> 1) : 0;  // group slot of this MFMA
            const bool rescale = fresh[q] && (G == 32 ? (kk & 1) == 0 : kk == 0);
            q4::u32x4 bop[2];
            if constexpr (G == 64) {
                // decoded one k-slot ahead: slot kk + 1's words while slot kk's MFMAs run
                // (see the schedule below)
                if (kk == 0) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) bnext[j] = dequant_word<XF16>(b.w[j][0], zrep[q][j]);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    bop[j] = bnext[j];
                    // zero-scale groups (rare) get a zero operand; a select, so no branch
                    // splits the slot's code
                    const uint32_t keep = zmask[q] && sn[q][j] == 0.0f ? 0u : 0xFFFFFFFFu;
                    bop[j] &= keep;
                }
                if (kk < 3) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) bnext[j] = dequant_word<XF16>(b.w[j][kk + 1 < 4 ? kk + 1 : 3], zrep[0][j]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) bop[j] = dequant_word<XF16>(b.w[j][kk], zrep[q][j]);
                if (zmask[q]) {  // rare: zero the operand of zero-scale groups
#pragma unroll
                    for (int j = 0; j < 2; ++j) bop[j] &= sn[q][j] != 0.0f ? 0xFFFFFFFFu : 0u;
                }
            }
            const uint8_t* ab = slot + apos[kk];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const q4::u32x4 a = AP == 2 ? aop[(kk & 1) % AP][i]
                                            : *reinterpret_cast<const q4::u32x4*>(ab + i * 32 * (BK * 2));
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    // each 32x32 tile moves to the new group's units right before its own MFMA,
                    // so the multiplies issue while the MFMAs of the other tiles run
                    if (rescale) {
#pragma unroll
                        for (int e = 0; e < 16; ++e) acc[i][j][e] *= ratio[q][j];
                    }
                    if constexpr (XF16)
                        acc[i][j] = mfma32_f16(a, bop[j], acc[i][j]);
                    else
                        acc[i][j] = mfma32_bf16(a, bop[j], acc[i][j]);
                }
            }
            // g = 64, a slot without a group change: each MFMA followed by five VALU
            // instructions (the next slot's decode), so the decode issues while the matrix
            // cores work.  On the 70B prefill this takes g = 64 from 571 to 823 TFLOP/s
            // (its register pressure falls with it); at g = 128 and g = 32 the early decode
            // and the forced order were 1-3% slower than the compiler's own, so they keep it.
            if constexpr (G == 64) {
                if (!rescale) {
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // five VALU
                    }
                }
            }
        }
    };

    // ---- pipeline: stages s and s+1 are in flight when stage s starts
    constexpr int LOADS = 4 + 2 * ((G >= 64 ? 1 : 2) + NGS + (SYM ? 0 : 1));  // vector loads per stage
    constexpr int WAIT = (LOADS & 15) | ((LOADS >> 4) << 14) | (0x7 << 4) | (0xF << 8);  // vmcnt(LOADS)
    BStage<G> bs[3];
    load_a(0);
    load_b(bs[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(1);
    load_b(bs[1], 1);
    __builtin_amdgcn_sched_barrier(0);
    auto step = [&](int s, BStage<G>& cur, BStage<G>& nxt2) {
        // This wave's loads of stage s have landed (those of stage s+1 stay in flight); the
        // barrier then makes every wave's activation DMA visible and frees slot s-1.  A plain
        // s_barrier: __syncthreads() would also wait for the DMA of stage s+1.
        __builtin_amdgcn_s_waitcnt(WAIT);
        asm volatile("s_barrier" ::: "memory");
        load_a(s + 2);                     // (past the last stage: offsets off the end)
        load_b(nxt2, s + 2);
        __builtin_amdgcn_sched_barrier(0);
        compute(cur, s);
    };
    int s = 0;
    for (; s + 3 <= stages; s += 3) {
        step(s, bs[0], bs[2]);
        step(s + 1, bs[1], bs[0]);
        step(s + 2, bs[2], bs[1]);
    }
    if (s < stages) step(s, bs[0], bs[2]);
    if (s + 1 < stages) step(s + 1, bs[1], bs[0]);

    // epilogue: back to true units, store.  Lane (col, h), register r of a 32x32 tile holds
    // row (r & 3) + 4h + 8(r >> 2), column col.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int nn = wn0 + 32 * j + col;
        if (nn >= N) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int mm = m0 + 32 * i + (r & 3) + 4 * h + 8 * (r >> 2);
                if (mm < M) q4::store_y(y, (int64_t)mm * N + nn, acc[i][j][r] * s_cur[j], ydt);
            }
    }
}

template <int G, bool SYM>
hipError_t launch(const void* x, int xd, int m, const uint32_t* qw, const uint16_t* sc,
                  const uint32_t* zr, int n, int k, void* y, int ydt, hipStream_t st, const char** kname) {
    const int mtiles = (m + BM - 1) / BM, ntiles = (n + BN - 1) / BN;
    const dim3 grid((unsigned)(mtiles * ntiles)), block(NTHREADS);
    const size_t lds = (size_t)RING * A_STAGE;
    const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
    if (xd == 1) {
        *kname = "q4_gemm_mfma_f16";
        hipLaunchKernelGGL((gemm_kernel<G, SYM, true>), grid, block, lds, st, xp, m, qw, sc, zr, n, k, y, ydt);
    } else {
        *kname = "q4_gemm_mfma_bf16";
        hipLaunchKernelGGL((gemm_kernel<G, SYM, false>), grid, block, lds, st, xp, m, qw, sc, zr, n, k, y, ydt);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t q4k_gemm(const void* x, int x_dtype, int64_t m, const uint32_t* qweight,
                    const uint16_t* scales, const uint32_t* zeros, int64_t n, int64_t k, int g,
                    int sym, void* y, int ydt, hipStream_t stream, const char** kname) {
    const int mi = (int)m, ni = (int)n, ki = (int)k;
    switch (g * 2 + (sym ? 1 : 0)) {
    case 64: return launch<32, false>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, ydt, stream, kname);
    case 65: return launch<32, true>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, ydt, stream, kname);
    case 128: return launch<64, false>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, ydt, stream, kname);
    case 129: return launch<64, true>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, ydt, stream, kname);
    case 256: return launch<128, false>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, ydt, stream, kname);
    default: return launch<128, true>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, ydt, stream, kname);
    }
}
