// gemm.hip — prefill W4A16 linear layer (m > 16) for gfx950.
//
//   y[m][n] = sum_g S[n][g] * sum_{k in g} x[m][k] * (u[n][k] - z[n][g])
//
// Large-batch prefill is compute-bound ("LLM Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV
// Cache (7/10)", §Batch와 Context에 따라 속도가 달라진다), so this is a dense MFMA
// contraction with the dequantization fused into the operand path (path A of
// §Kernel이 없으면 압축 이점이 사라진다).
//
// Tiles.  A workgroup of 4 waves computes a 32 MI x 128 NJ block of y (activation rows x
// weight rows); every wave owns all 32 MI activation rows and 32 NJ weight rows as MI x NJ
// tiles of v_mfma_f32_32x32x16 (bf16 or fp16 inputs, fp32 accumulation): 128 x 256
// (MI = 4, NJ = 2), 128 x 128 (4, 1) or 256 x 128 (8, 1, where each decoded weight word
// feeds 8 MFMAs).  The K loop walks 64 columns per stage.
//
// Operands.  Activations are shared by the 4 waves: they go from HBM/L2 straight into an
// LDS ring with buffer-to-LDS loads (no registers), in an XOR-swizzled layout (16-byte
// chunk c of row r at position c ^ (r & 7)) that makes both the 1 KB loads and the operand
// reads bank-conflict free: three stages of 128 rows loaded two ahead, or two stages of
// 256 rows loaded one ahead.  Weights are not shared: each lane of the 32x32x16 MFMA's
// weight operand needs 8 consecutive k of one weight row, which is exactly one packed word,
// so every lane loads its own words (and the scale and zero point of its row) into
// registers with its stage's activations and dequantizes them right before the MFMA.
// Every stage issues the same loads in the same order, so each wait is a fixed count and
// the stages in flight stay in flight.
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
#include <type_traits>

#include "q4_launch.h"

namespace {

constexpr int BK = 64;  // k per stage of a workgroup tile
constexpr int NTHREADS = 256;
// MI: 32-row activation blocks per wave (the workgroup tile has 32 MI activation rows).
// The activation ring holds 3 stages of 128 rows (loads two stages ahead) or 2 stages of
// 256 rows (one stage ahead; its stages take twice as long), 48 or 64 KB: two workgroups
// per CU either way.
constexpr int ring_of(int mi) { return mi == 8 ? 2 : 3; }
constexpr int a_stage_of(int mi) { return 32 * mi * BK * 2; }  // bytes of one activation stage
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
// half (bf16) or converting (fp16; small integers are exact either way).  nm is the nibble
// mask 0x0F0F0F0F, or 0 together with zrep = 0 for a group whose scale is zero: every
// element is then 0, so such a group adds nothing without a branch of its own.
template <bool XF16>
__device__ __forceinline__ q4::u32x4 dequant_word(uint32_t w, uint32_t zrep, uint32_t nm) {
    const uint32_t lo = (((w & nm) | 0x80808080u) - zrep) ^ 0x80808080u;         // k 0,2,4,6
    const uint32_t hi = ((((w >> 4) & nm) | 0x80808080u) - zrep) ^ 0x80808080u;  // k 1,3,5,7
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
template <int G, int NJ>
struct BStage {
    static constexpr int NGS = G == 32 ? 2 : 1;
    uint32_t w[NJ][4];
    uint32_t s[NJ][NGS];
    uint32_t z[NJ];
};

// NJ: 32-row weight blocks per wave, MI: 32-row activation blocks per wave (the workgroup
// tile is 32 MI x 128 NJ).  With per > 0 the K range is split: the blocks of split s
// (blockIdx.x / tiles) take stages [s per, (s + 1) per) and write their fp32 partial sums
// to part[s][M][N] instead of y.
template <int G, bool SYM, bool XF16, int NJ, int MI>
__global__ __launch_bounds__(NTHREADS, 2) void gemm_kernel(const uint16_t* __restrict__ x, int M,
                                                          const uint32_t* __restrict__ qweight,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint32_t* __restrict__ zeros,
                                                          int N, int K, void* __restrict__ y, int ydt,
                                                          int per, float* __restrict__ part) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // RING x A_STAGE
    constexpr int BM = 32 * MI, BN = 128 * NJ;
    constexpr int RING = ring_of(MI), AHEAD = RING - 1;  // stages in the ring, loaded ahead
    constexpr int A_STAGE = a_stage_of(MI);
    constexpr int WROWS = 8 * MI;  // activation rows each wave moves into a stage
    constexpr int NGS = BStage<G, NJ>::NGS;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int mtiles = (M + BM - 1) / BM;
    const int tiles = mtiles * ((N + BN - 1) / BN);
    const int split = (int)blockIdx.x / tiles, tile = (int)blockIdx.x - split * tiles;
    const int mt = tile % mtiles, nt = tile / mtiles;  // XCD-friendly order
    const int m0 = mt * BM, n0 = nt * BN;
    const int KW = K / 8;
    const int n_groups = K / G;
    const int zwords = (n_groups + 7) >> 3;
    const int stages = (K + BK - 1) / BK;
    // this block's stages [sb, se)
    const int sb = per > 0 ? split * per : 0;
    const int se = per > 0 && sb + per < stages ? sb + per : stages;

    // activations of this row block
    const int arows = __builtin_amdgcn_readfirstlane(M - m0 < BM ? M - m0 : BM);
    const q4::rsrc rx = q4::make_rsrc(x + (int64_t)m0 * K, (uint32_t)arows * (uint32_t)K * 2u);
    // this wave's 32 NJ weight rows
    const int wn0 = n0 + 32 * NJ * wave;
    int wrows = N - wn0;
    wrows = wrows < 0 ? 0 : (wrows > 32 * NJ ? 32 * NJ : wrows);
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
    // so do the loads for the stages after the last one (issued by the pipeline, never
    // used): every mask goes into the per-lane offset.  The k tail (k % 64 == 32): the
    // activation chunks past k are read as zeros, so whatever the weight words past the
    // end of a row hold meets a zero.
    const int ca = (lane & 7) ^ ((lane >> 3) & 7);  // activation chunk this lane moves (DMA rows are 8-aligned)
    uint32_t aoff[MI];
#pragma unroll
    for (int q = 0; q < MI; ++q)
        aoff[q] = ((uint32_t)(WROWS * wave + 8 * q + (lane >> 3)) * (uint32_t)K + 8u * ca) * 2u;
    const int tail_chunks = (K % BK) / 8;  // valid chunks of a short last stage (0: none short)
    const uint32_t tail_mask = tail_chunks != 0 && ca >= tail_chunks ? kOOB : 0u;
    uint32_t qoff[NJ], soff[NJ], zoff[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const uint32_t row = (uint32_t)(32 * j + col);
        const uint32_t rowmask = (int)row < wrows ? 0u : kOOB;
        qoff[j] = (row * (uint32_t)KW * 4u + (G >= 64 ? 16u : 8u) * h) | rowmask;
        soff[j] = (row * (uint32_t)n_groups * 2u) | rowmask;
        zoff[j] = (row * (uint32_t)zwords * 4u) | rowmask;
    }

    // ---- loads of one stage (fixed count and order: MI activation DMAs, then per block j
    //      the words, the scales and the zero word)
    auto load_a = [&](int s) {  // rows [WROWS wave, +WROWS) of stage s into ring slot s % RING
        const uint32_t tm = s >= se ? kOOB : (s == stages - 1 ? tail_mask : 0u);
        const int so = __builtin_amdgcn_readfirstlane(2 * s * BK);
        uint8_t* slot = smem + (s % RING) * A_STAGE;
#pragma unroll
        for (int q = 0; q < MI; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr)(slot + (WROWS * wave + 8 * q) * (BK * 2)), 16,
                                                     (int)(aoff[q] | tm), so, 0, 0);
    };
    auto load_b = [&](BStage<G, NJ>& b, int s) {
        const int wso = __builtin_amdgcn_readfirstlane(4 * s * (BK / 8));  // the stage's first word
        const int g0 = G == 128 ? (s >> 1) : (G == 64 ? s : 2 * s);        // its first group
        const int sso = __builtin_amdgcn_readfirstlane(2 * g0);
        const int zso = __builtin_amdgcn_readfirstlane(4 * (g0 >> 3));
        const uint32_t pm = s >= se ? kOOB : 0u;  // past the block's last stage: read nothing
        // a short last stage (k % 64 == 32) holds words 0..3 and one group: the words and the
        // scale past the row read nothing
        const bool short_stage = s == stages - 1 && (K % BK) != 0;
        const uint32_t hm = short_stage && (G == 32 || h == 1) ? kOOB : 0u;  // words 4..7
        const uint32_t sm = short_stage ? kOOB : 0u;                         // second group
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
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

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    float s_cur[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) s_cur[j] = 1.f;
    int g_cur = -1;

    // LDS operand addresses: row 32i + col of the slot, chunk word_of(kk, h) at its swizzled
    // position ((32i + col) & 7 == col & 7, so one address per kk; i goes in the offset)
    uint32_t apos[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        apos[kk] = (uint32_t)col * (BK * 2) + ((uint32_t)(word_of<G>(kk, h) ^ (col & 7)) << 4);

    // ---- compute of one stage.  FRESH (a compile-time tag): the stage opens a group (every
    // stage when g <= 64; at g = 128 the caller picks the variant per stage), so its MFMAs
    // move the accumulators to the new group's units first.  Both variants are straight-line
    // code, which leaves the scheduler free to interleave decodes, rescales and MFMAs.
    auto compute = [&](const BStage<G, NJ>& b, int s, auto fresh_tag) {
        constexpr bool FRESH = decltype(fresh_tag)::value;
        const uint8_t* slot = smem + (s % RING) * A_STAGE;
        float ratio[NGS][NJ];
        uint32_t zrep[NGS][NJ], nm[NGS][NJ];
#pragma unroll
        for (int q = 0; q < NGS; ++q) {  // the stage's groups (one, or two when g = 32)
            const int gk = G == 128 ? (s >> 1) : (G == 64 ? s : 2 * s + q);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float sn = q4::f16_bits_to_float((uint16_t)b.s[j][q]);
                const bool live = sn != 0.0f;  // a zero scale: the group's operand is zero
                const int z = SYM ? 8 : (int)((b.z[j] >> (4 * (gk & 7))) & 0xFu);
                zrep[q][j] = live ? (uint32_t)z * 0x01010101u : 0u;
                nm[q][j] = live ? 0x0F0F0F0Fu : 0u;
                ratio[q][j] = 1.0f;
                if constexpr (FRESH) {
                    // the units stay those of the previous group across a zero scale
                    ratio[q][j] = live && g_cur >= 0 ? s_cur[j] / sn : 1.0f;
                    if (live) s_cur[j] = sn;
                }
            }
            if constexpr (FRESH) g_cur = gk;
        }
        // g = 128 with 128-row tiles: the activation operands of two MFMA k-slots are read
        // from LDS ahead of their MFMAs (32 registers), so each MFMA waits for a read issued
        // long before.  At g = 32 and 64 (a group boundary every stage or two per stage, with
        // its rescale) and with 256-row tiles the extra registers would spill: one read per
        // MFMA, as it is needed.
        constexpr int AP = G == 128 && MI == 4 ? 2 : 1;
        q4::u32x4 aop[AP][MI];
        q4::u32x4 bnext[NJ];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if constexpr (AP == 2) {
                if ((kk & 1) == 0) {
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                        for (int i = 0; i < MI; ++i)
                            aop[k2][i] = *reinterpret_cast<const q4::u32x4*>(slot + apos[kk + k2] + i * 32 * (BK * 2));
                }
            }
            const int q = G == 32 ? (kk >> 1) : 0;  // group slot of this MFMA
            const bool rescale = FRESH && (G == 32 ? (kk & 1) == 0 : kk == 0);
            q4::u32x4 bop[NJ];
            if constexpr (G == 64) {
                // decoded one k-slot ahead: slot kk + 1's words while slot kk's MFMAs run
                if (kk == 0) {
#pragma unroll
                    for (int j = 0; j < NJ; ++j) bnext[j] = dequant_word<XF16>(b.w[j][0], zrep[q][j], nm[q][j]);
                }
#pragma unroll
                for (int j = 0; j < NJ; ++j) bop[j] = bnext[j];
                if (kk < 3) {
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        bnext[j] = dequant_word<XF16>(b.w[j][kk + 1 < 4 ? kk + 1 : 3], zrep[0][j], nm[0][j]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < NJ; ++j) bop[j] = dequant_word<XF16>(b.w[j][kk], zrep[q][j], nm[q][j]);
            }
            const uint8_t* ab = slot + apos[kk];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const q4::u32x4 a = AP == 2 ? aop[(kk & 1) % AP][i]
                                            : *reinterpret_cast<const q4::u32x4*>(ab + i * 32 * (BK * 2));
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
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
        }
    };

    // ---- pipeline: stages s .. s + AHEAD - 1 are in flight when stage s starts
    constexpr int LOADS = MI + NJ * ((G >= 64 ? 1 : 2) + NGS + (SYM ? 0 : 1));  // vector loads per stage
    constexpr int WN = LOADS * (AHEAD - 1);  // loads left in flight once stage s has landed
    static_assert(WN < 64, "vmcnt holds 6 bits");
    constexpr int WAIT = (WN & 15) | ((WN >> 4) << 14) | (0x7 << 4) | (0xF << 8);  // vmcnt(WN)
    BStage<G, NJ> bs[AHEAD + 1];
#pragma unroll
    for (int a = 0; a < AHEAD; ++a) {
        load_a(sb + a);
        load_b(bs[a], sb + a);
        __builtin_amdgcn_sched_barrier(0);
    }
    auto step = [&](int s, BStage<G, NJ>& cur, BStage<G, NJ>& nxt, auto fresh_tag) {
        // This wave's loads of stage s have landed (those of the stages after it stay in
        // flight); the barrier then makes every wave's activation DMA visible and frees the
        // slot of stage s - 1.  A plain s_barrier: __syncthreads() would also wait for the
        // loads still in flight.
        __builtin_amdgcn_s_waitcnt(WAIT);
        asm volatile("s_barrier" ::: "memory");
        load_a(s + AHEAD);                 // (past the last stage: offsets off the end)
        load_b(nxt, s + AHEAD);
        __builtin_amdgcn_sched_barrier(0);
        compute(cur, s, fresh_tag);
    };
    // The loop is unrolled over the register ring (AHEAD + 1 stages) and, at g = 128, over
    // the group's two stages, so that whether a stage opens a group is known at compile time
    // (a branch between two compute variants makes the compiler copy the accumulators at
    // the join).  A split starts on an even stage (plan() keeps per even).
    constexpr std::true_type kFresh{};
    constexpr std::integral_constant<bool, G != 128> kOdd{};  // a stage at an odd index
    int s = sb;
    if constexpr (AHEAD == 1) {  // register ring of 2: the unroll by 2 covers both
        for (; s + 2 <= se; s += 2) {
            step(s, bs[0], bs[1], kFresh);
            step(s + 1, bs[1], bs[0], kOdd);
        }
        if (s < se) step(s, bs[0], bs[1], kFresh);
    } else if constexpr (G == 128) {
        for (; s + 6 <= se; s += 6) {
            step(s, bs[0], bs[2], kFresh);
            step(s + 1, bs[1], bs[0], kOdd);
            step(s + 2, bs[2], bs[1], kFresh);
            step(s + 3, bs[0], bs[2], kOdd);
            step(s + 4, bs[1], bs[0], kFresh);
            step(s + 5, bs[2], bs[1], kOdd);
        }
        if (s < se) step(s, bs[0], bs[2], kFresh);
        if (s + 1 < se) step(s + 1, bs[1], bs[0], kOdd);
        if (s + 2 < se) step(s + 2, bs[2], bs[1], kFresh);
        if (s + 3 < se) step(s + 3, bs[0], bs[2], kOdd);
        if (s + 4 < se) step(s + 4, bs[1], bs[0], kFresh);
    } else {
        for (; s + 3 <= se; s += 3) {
            step(s, bs[0], bs[2], kFresh);
            step(s + 1, bs[1], bs[0], kFresh);
            step(s + 2, bs[2], bs[1], kFresh);
        }
        if (s < se) step(s, bs[0], bs[2], kFresh);
        if (s + 1 < se) step(s + 1, bs[1], bs[0], kFresh);
    }

    // epilogue: back to true units, store (y, or this split's fp32 partial sums).  Lane
    // (col, h), register r of a 32x32 tile holds row (r & 3) + 4h + 8(r >> 2), column col.
    float* pp = part != nullptr ? part + (int64_t)split * M * N : nullptr;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int nn = wn0 + 32 * j + col;
        if (nn >= N) continue;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int mm = m0 + 32 * i + (r & 3) + 4 * h + 8 * (r >> 2);
                if (mm >= M) continue;
                const float v = acc[i][j][r] * s_cur[j];
                if (pp != nullptr)
                    pp[(int64_t)mm * N + nn] = v;
                else
                    q4::store_y(y, (int64_t)mm * N + nn, v, ydt);
            }
    }
}

// y[i] = the sum over the splits of part[s][i], in order of s (one rounding per addition,
// the same order every call), stored as ydt.
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int splits, int64_t count,
                                     void* __restrict__ y, int ydt) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x) {
        float acc = part[i];
        for (int sp = 1; sp < splits; ++sp) acc = acc + part[(int64_t)sp * count + i];
        q4::store_y(y, i, acc, ydt);
    }
}

// The tile and split for a product.  From m = 512 on, the 256 x 128 tile (each decoded
// weight word feeds 8 MFMAs instead of 4) while it gives at least one workgroup per CU;
// otherwise the 128 x 256 tile while that does; otherwise the 128 x 128 tile, and, when a
// workspace is given and that still leaves CUs idle, the K range split so that the
// workgroups cover every CU (each split at least 8 stages, at most 16 splits).
struct GemmPlan {
    int nj;     // 32-row weight blocks per wave: 2 (128 x 256 tile) or 1
    int mi;     // 32-row activation blocks per wave: 8 (256 x 128 tile) or 4
    int per;    // stages per split (0: no split)
    int splits;
};
GemmPlan plan(int64_t m, int64_t n, int64_t k, int num_cus, bool may_split) {
    const int cus = num_cus > 0 ? num_cus : 256;
    const int64_t mtiles = (m + 127) / 128;
    const int64_t stages = (k + BK - 1) / BK;
    if (m >= 512 && ((m + 255) / 256) * ((n + 127) / 128) >= cus) return {1, 8, 0, 1};
    if (mtiles * ((n + 255) / 256) >= cus) return {2, 4, 0, 1};
    const int64_t tiles = mtiles * ((n + 127) / 128);
    if (!may_split || tiles >= cus) return {1, 4, 0, 1};
    int64_t splits = (cus + tiles - 1) / tiles;
    if (splits > 16) splits = 16;
    if (splits > stages / 8) splits = stages / 8;
    if (splits < 2) return {1, 4, 0, 1};
    // per even: every split starts on the first stage of a g = 128 group
    const int64_t per = ((stages + splits - 1) / splits + 1) & ~(int64_t)1;
    return {1, 4, (int)per, (int)((stages + per - 1) / per)};
}

template <int G, bool SYM, int NJ, int MI>
void launch_tile(const void* x, int xd, int m, const uint32_t* qw, const uint16_t* sc, const uint32_t* zr,
                 int n, int k, void* y, int ydt, int per, int splits, float* part, hipStream_t st) {
    const int mtiles = (m + 32 * MI - 1) / (32 * MI), ntiles = (n + 128 * NJ - 1) / (128 * NJ);
    const dim3 grid((unsigned)(mtiles * ntiles * splits)), block(NTHREADS);
    const size_t lds = (size_t)ring_of(MI) * a_stage_of(MI);
    const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
    if (xd == 1)
        hipLaunchKernelGGL((gemm_kernel<G, SYM, true, NJ, MI>), grid, block, lds, st, xp, m, qw, sc, zr, n, k, y,
                           ydt, per, part);
    else
        hipLaunchKernelGGL((gemm_kernel<G, SYM, false, NJ, MI>), grid, block, lds, st, xp, m, qw, sc, zr, n, k, y,
                           ydt, per, part);
}

template <int G, bool SYM>
hipError_t launch(const void* x, int xd, int m, const uint32_t* qw, const uint16_t* sc,
                  const uint32_t* zr, int n, int k, void* y, int ydt, float* ws, int64_t ws_floats,
                  hipStream_t st, const char** kname) {
    GemmPlan pl = plan(m, n, k, q4k_device_cus(), ws != nullptr);
    if (pl.splits > 1 && (int64_t)pl.splits * m * n > ws_floats) pl = {1, 4, 0, 1};
    float* part = pl.splits > 1 ? ws : nullptr;
    *kname = xd == 1 ? "q4_gemm_mfma_f16" : "q4_gemm_mfma_bf16";
    if (pl.mi == 8)
        launch_tile<G, SYM, 1, 8>(x, xd, m, qw, sc, zr, n, k, y, ydt, 0, 1, nullptr, st);
    else if (pl.nj == 2)
        launch_tile<G, SYM, 2, 4>(x, xd, m, qw, sc, zr, n, k, y, ydt, 0, 1, nullptr, st);
    else
        launch_tile<G, SYM, 1, 4>(x, xd, m, qw, sc, zr, n, k, y, ydt, pl.per, pl.splits, part, st);
    hipError_t e = q4k_launched(*kname);
    if (e != hipSuccess || part == nullptr) return e;
    const int64_t count = (int64_t)m * n;
    const int64_t blocks = (count + 255) / 256 < 4096 ? (count + 255) / 256 : 4096;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st, part, pl.splits, count, y,
                       ydt);
    return q4k_launched("q4_gemm_splitk_reduce");
}

}  // namespace

int64_t q4k_gemm_workspace_floats(int64_t m, int64_t n, int64_t k) {
    const GemmPlan pl = plan(m, n, k, q4k_device_cus(), true);
    return pl.splits > 1 ? (int64_t)pl.splits * m * n : 0;
}

hipError_t q4k_gemm(const void* x, int x_dtype, int64_t m, const uint32_t* qweight,
                    const uint16_t* scales, const uint32_t* zeros, int64_t n, int64_t k, int g,
                    int sym, void* y, int ydt, float* workspace, int64_t workspace_floats,
                    hipStream_t stream, const char** kname) {
    const int mi = (int)m, ni = (int)n, ki = (int)k;
    float* ws = workspace;
    const int64_t wf = workspace_floats;
    switch (g * 2 + (sym ? 1 : 0)) {
    case 64: return launch<32, false>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, ydt, ws, wf, stream, kname);
    case 65: return launch<32, true>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, ydt, ws, wf, stream, kname);
    case 128: return launch<64, false>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, ydt, ws, wf, stream, kname);
    case 129: return launch<64, true>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, ydt, ws, wf, stream, kname);
    case 256: return launch<128, false>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, ydt, ws, wf, stream, kname);
    default: return launch<128, true>(x, x_dtype, mi, qweight, scales, zeros, ni, ki, y, ydt, ws, wf, stream, kname);
    }
}
