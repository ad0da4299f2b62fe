// Fused attention forward for wide heads whose values are the first d_v
// columns of the keys (d_qk = 576, d_v = 512, one K/V head shared by the query
// heads, V given as that view of K), over one range of the keys: the split-KV
// form of the V-in-K kernel for workloads with few query rows per head.
//
// Each workgroup owns 64 query rows of one (batch, head) and one range of
// keys and writes that range's attention of its rows, O / l in fp32 and the
// logsumexp, to a workspace; attn_split_merge_wide combines the ranges exactly
// (the running maximum and normalizer recurrence of "Distilling a 4.5 hour
// CUDA talk", section 7, carried across ranges). Against the 32-row kernel,
// a K tile copied into LDS serves twice the rows (half the copy volume and
// half the LDS reads of Vᵀ per row), and splitting the keys keeps one
// workgroup on every CU.
//
// gfx950 mapping (8 waves, two per SIMD):
//  * Score waves 0..3, w = 2 rg + kh, own keys 16 kh .. 16 kh + 15 of each
//    32-key tile for rows 32 rg .. 32 rg + 31: two 16 x 16 blocks (row
//    blocks rb = 0, 1) computed whole (Sᵀ = K·Qᵀ, 18 k-steps of
//    v_mfma_f32_16x16x32_bf16 each, both blocks' Q in registers), so every K
//    fragment read feeds two MFMAs. They apply the mask and the exponential
//    and write P (bf16) to LDS.
//  * Value waves 4..7 (vw = w - 4) read the tile's P and accumulate output
//    columns 128 vw .. 128 vw + 127 for all 64 rows (two 32-row blocks),
//    their Vᵀ fragments read once from the K tile for both blocks. At the
//    start of each period they also copy a K tile into LDS (LDS-DMA, a
//    quarter each), three tiles ahead, and wait for it at the period's end:
//    an LDS-DMA holds its issuing wave for tens of cycles, and the value
//    waves' path through a period is the shorter one.
//  * Per tile the score waves' MFMAs for tile T + 1 and the value waves' for
//    tile T share each SIMD's matrix pipe (36 16x16 + 16 32x32 MFMAs).
//  * K tiles in a four-stage ring; P double-buffered; one barrier per tile.
//  * The per-row reference m is the maximum over the range's first tile;
//    if a row's normalizer leaves [0, 2^32] the workgroup finds the exact row
//    maxima of its range and runs the range again.
#pragma once

#include "attn_fwd_wide_vk_kernel.hpp"
#include "attn_split_kernel.hpp"
#include "tile.hpp"

namespace attn {

template <int DQK, int DV>
struct WideVkSplitCfg {
    static constexpr int TQ = 64;  // query rows per workgroup
    static constexpr int TK = 32;  // keys per tile
    static constexpr int NWAVE = 8;
    static constexpr int NT = 64 * NWAVE;
    static constexpr int NSW = 4;
    static constexpr int KCH = DQK / 8;  // 16-byte chunks per K row
    static constexpr int KROW_B = 2 * DQK;
    static constexpr int KTILE_B = TK * KROW_B;
    static constexpr int NSTAGE = 4;
    static constexpr int NKS = DQK / 32;           // k-steps of a 16x16 score block
    static constexpr int PROW_B = 2 * TK + 16;     // P row: 32 bf16 + 16 bytes of padding
    static constexpr int PBUF_B = TQ * PROW_B;     // one P buffer
    static constexpr int POFF = NSTAGE * KTILE_B;  // P buffers after the ring
    static constexpr int SOFF = POFF + 2 * PBUF_B; // row statistics: [2 key halves][64 rows] + m[64]
    static constexpr int LDS_BYTES = SOFF + 3 * TQ * 4;
    static constexpr int KWIN_W = KTILE_B / 1024 / (NWAVE - NSW);  // 1 KB copies per value wave per tile
    static constexpr int CBW = DV / 32 / (NWAVE - NSW);  // 32-column blocks of O per value wave
    static_assert(NKS == 18 && KWIN_W == 9, "the score block is written for 18 k-steps; 9 copies per wave");
    static_assert(KCH % 8 == 0, "the swizzle permutes aligned groups of 8 chunks");
    static_assert(CBW == 4 && DV <= DQK, "value columns 128 vw .. 128 vw + 127");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// ---- the score block ------------------------------------------------------
// As the 32-row kernel's (wide_vk_qk): K fragments stream through a ring of 6
// register quads the compiler does not allocate, here v[232:255]; fragment ks
// (slot ks % 6) is read six k-steps ahead, right after the two MFMAs of step
// ks - 6 took the slot's old contents at issue, and waited for with a count of
// this block's own ds_read_b128s (they complete in order). Each k-step runs
// one MFMA per row block, s0 (rows 0..15 of the wave's 32) and s1 (16..31),
// two independent chains. The block ends with the wait states a VALU read of
// an MFMA result needs (the compiler does not see the MFMA latency through the
// statement).
#define WVKS_CLOBBERS "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255"
#define WVKS_KR0 "ds_read_b128 v[232:235], %[kb0] offset:0\n\t"
#define WVKS_KR1 "ds_read_b128 v[236:239], %[kb1] offset:0\n\t"
#define WVKS_KR2 "ds_read_b128 v[240:243], %[kb0] offset:128\n\t"
#define WVKS_KR3 "ds_read_b128 v[244:247], %[kb1] offset:128\n\t"
#define WVKS_KR4 "ds_read_b128 v[248:251], %[kb0] offset:256\n\t"
#define WVKS_KR5 "ds_read_b128 v[252:255], %[kb1] offset:256\n\t"
#define WVKS_KR6 "ds_read_b128 v[232:235], %[kb0] offset:384\n\t"
#define WVKS_KR7 "ds_read_b128 v[236:239], %[kb1] offset:384\n\t"
#define WVKS_KR8 "ds_read_b128 v[240:243], %[kb0] offset:512\n\t"
#define WVKS_KR9 "ds_read_b128 v[244:247], %[kb1] offset:512\n\t"
#define WVKS_KR10 "ds_read_b128 v[248:251], %[kb0] offset:640\n\t"
#define WVKS_KR11 "ds_read_b128 v[252:255], %[kb1] offset:640\n\t"
#define WVKS_KR12 "ds_read_b128 v[232:235], %[kb0] offset:768\n\t"
#define WVKS_KR13 "ds_read_b128 v[236:239], %[kb1] offset:768\n\t"
#define WVKS_KR14 "ds_read_b128 v[240:243], %[kb0] offset:896\n\t"
#define WVKS_KR15 "ds_read_b128 v[244:247], %[kb1] offset:896\n\t"
#define WVKS_KR16 "ds_read_b128 v[248:251], %[kb0] offset:1024\n\t"
#define WVKS_KR17 "ds_read_b128 v[252:255], %[kb1] offset:1024\n\t"
#define WVKS_MM0 "s_waitcnt lgkmcnt(0)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[232:235], %[qa0], 0\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[232:235], %[qb0], 0\n\t"
#define WVKS_MM1 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[236:239], %[qa1], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[236:239], %[qb1], %[s1]\n\t"
#define WVKS_MM2 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[240:243], %[qa2], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[240:243], %[qb2], %[s1]\n\t"
#define WVKS_MM3 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[244:247], %[qa3], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[244:247], %[qb3], %[s1]\n\t"
#define WVKS_MM4 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[248:251], %[qa4], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[248:251], %[qb4], %[s1]\n\t"
#define WVKS_MM5 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[252:255], %[qa5], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[252:255], %[qb5], %[s1]\n\t"
#define WVKS_MM6 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[232:235], %[qa6], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[232:235], %[qb6], %[s1]\n\t"
#define WVKS_MM7 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[236:239], %[qa7], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[236:239], %[qb7], %[s1]\n\t"
#define WVKS_MM8 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[240:243], %[qa8], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[240:243], %[qb8], %[s1]\n\t"
#define WVKS_MM9 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[244:247], %[qa9], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[244:247], %[qb9], %[s1]\n\t"
#define WVKS_MM10 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[248:251], %[qa10], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[248:251], %[qb10], %[s1]\n\t"
#define WVKS_MM11 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[252:255], %[qa11], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[252:255], %[qb11], %[s1]\n\t"
#define WVKS_MM12 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[232:235], %[qa12], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[232:235], %[qb12], %[s1]\n\t"
#define WVKS_MM13 "s_waitcnt lgkmcnt(4)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[236:239], %[qa13], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[236:239], %[qb13], %[s1]\n\t"
#define WVKS_MM14 "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[240:243], %[qa14], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[240:243], %[qb14], %[s1]\n\t"
#define WVKS_MM15 "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[244:247], %[qa15], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[244:247], %[qb15], %[s1]\n\t"
#define WVKS_MM16 "s_waitcnt lgkmcnt(1)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[248:251], %[qa16], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[248:251], %[qb16], %[s1]\n\t"
#define WVKS_MM17 "s_waitcnt lgkmcnt(0)\n\tv_mfma_f32_16x16x32_bf16 %[s0], v[252:255], %[qa17], %[s0]\n\tv_mfma_f32_16x16x32_bf16 %[s1], v[252:255], %[qb17], %[s1]\n\t"
#define WVKS_BODY WVKS_MM0 WVKS_KR6 WVKS_MM1 WVKS_KR7 WVKS_MM2 WVKS_KR8 WVKS_MM3 WVKS_KR9 WVKS_MM4 WVKS_KR10 WVKS_MM5 WVKS_KR11 WVKS_MM6 WVKS_KR12 WVKS_MM7 WVKS_KR13 WVKS_MM8 WVKS_KR14 WVKS_MM9 WVKS_KR15 WVKS_MM10 WVKS_KR16 WVKS_MM11 WVKS_KR17 WVKS_MM12 WVKS_MM13 WVKS_MM14 WVKS_MM15 WVKS_MM16 WVKS_MM17
#define WVKS_Q_IN [qa0] "v"(qa[0]), [qa1] "v"(qa[1]), [qa2] "v"(qa[2]), [qa3] "v"(qa[3]), [qa4] "v"(qa[4]), [qa5] "v"(qa[5]), [qa6] "v"(qa[6]), [qa7] "v"(qa[7]), [qa8] "v"(qa[8]), [qa9] "v"(qa[9]), [qa10] "v"(qa[10]), [qa11] "v"(qa[11]), [qa12] "v"(qa[12]), [qa13] "v"(qa[13]), [qa14] "v"(qa[14]), [qa15] "v"(qa[15]), [qa16] "v"(qa[16]), [qa17] "v"(qa[17]), [qb0] "v"(qb[0]), [qb1] "v"(qb[1]), [qb2] "v"(qb[2]), [qb3] "v"(qb[3]), [qb4] "v"(qb[4]), [qb5] "v"(qb[5]), [qb6] "v"(qb[6]), [qb7] "v"(qb[7]), [qb8] "v"(qb[8]), [qb9] "v"(qb[9]), [qb10] "v"(qb[10]), [qb11] "v"(qb[11]), [qb12] "v"(qb[12]), [qb13] "v"(qb[13]), [qb14] "v"(qb[14]), [qb15] "v"(qb[15]), [qb16] "v"(qb[16]), [qb17] "v"(qb[17])


__device__ __forceinline__ void wvks_kreads0(uint32_t kb0, uint32_t kb1) {
    asm volatile(WVKS_KR0 WVKS_KR1 WVKS_KR2 WVKS_KR3 WVKS_KR4 WVKS_KR5
                 :
                 : [kb0] "v"(kb0), [kb1] "v"(kb1)
                 : WVKS_CLOBBERS, "memory");
}

__device__ __forceinline__ void wvks_qk(const bf16x8 (&qa)[18], const bf16x8 (&qb)[18], uint32_t kb0,
                                        uint32_t kb1, f32x4 &r0, f32x4 &r1) {
    f32x4 s0, s1;
    asm volatile(WVKS_BODY "s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : [s0] "=&v"(s0), [s1] "=&v"(s1)
                 : [kb0] "v"(kb0), [kb1] "v"(kb1), WVKS_Q_IN
                 : WVKS_CLOBBERS, "memory");
    r0 = s0;
    r1 = s1;
}

template <int DQK, int DV>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
__attribute__((amdgpu_num_vgpr(232)))  // v232 .. v255: the K fragment ring of the score block
attn_fwd_wide_vk_split_kernel(const SplitArgs sa) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    using C = WideVkSplitCfg<DQK, DV>;
    constexpr int TK = C::TK, CBW = C::CBW;
    const KernelArgs &a = sa.a;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool sw = w < C::NSW;                  // a score wave (else a value wave)
    const int l32 = lane & 31, g = lane >> 5;    // 32x32 fragments (P·V)
    const int l16 = lane & 15, G = lane >> 4;    // 16x16 fragments (scores)
    const int kh = w & 1, rg = (w >> 1) & 1;     // a score wave's keys and 32-row group
    const int vw = (w - C::NSW) & 3;             // a value wave's index
    // k-group of this lane's 8 contraction elements in a k-step (the order
    // that keeps the K fragment reads free of bank conflicts with the row
    // swizzle); Q uses the same assignment
    const int kg = (0x9C >> (2 * G)) & 3;

    // ---- work item: split s of (batch, head, 64-row tile); consecutive
    // workgroups take consecutive splits, so with as many XCDs as a multiple
    // of the split count each XCD streams one range of K ------------------
    const int BH = a.B * a.Hq;
    const uint32_t wid = work_index(blockIdx.x, gridDim.x);
    const int s = (int)(wid % (uint32_t)sa.n_splits);
    const int item = (int)(wid / (uint32_t)sa.n_splits);
    const int bh = item % BH, qt = item / BH;
    const int b = bh / a.Hq, h = bh % a.Hq, hk = h / a.group;
    const __bf16 *__restrict__ Qp = (const __bf16 *)a.q + b * a.q_sb + h * a.q_sh;
    const __bf16 *__restrict__ Kp = (const __bf16 *)a.k + b * a.k_sb + hk * a.k_sh;

    const int q0 = qt * C::TQ;
    const int k_begin = s * sa.split_len;                 // a multiple of TK
    const int k_end = min(a.Nkv, k_begin + sa.split_len);
    const int n_tiles = k_end > k_begin ? (k_end - k_begin + TK - 1) / TK : 0;
    const int T0 = k_begin / TK;                          // first tile of the range
    // partial outputs of this split: row r of (b, h) is row (b H_q + h) N_q + r
    const int64_t prow0 = ((int64_t)b * a.Hq + h) * a.Nq;
    float *const opart = sa.opart + (int64_t)s * BH * a.Nq * DV;
    float *const lpart = sa.lpart + (int64_t)s * BH * a.Nq;

    if (n_tiles == 0) {
        // an empty range: weight zero in the merge
        if (tid < C::TQ && q0 + tid < a.Nq) lpart[prow0 + q0 + tid] = -INFINITY;
        for (int i = tid; i < C::TQ * DV / 4; i += C::NT) {
            const int r = i / (DV / 4), c = i % (DV / 4);
            if (q0 + r < a.Nq) *(f32x4 *)(opart + (prow0 + q0 + r) * DV + 4 * c) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        return;
    }

    auto lds_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    float *stat = (float *)(lds + C::SOFF);  // [kh][64] per-half row values, then m[64]

    // ---- K copies (value waves): in the period that computes P·V of range
    // tile t, value wave cw = w - 4 moves pieces 4 u + cw (1 KB each) of
    // range tile t + 3 and waits for them at the period's end.
    const int cw = w & 3;
    auto copy_offsets = [&](uint32_t (&koff)[C::KWIN_W]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < C::KWIN_W; ++u) {
            const int p = (4 * u + cw) * 64 + lane;
            const int r = p / C::KCH, c = wide_vk_chunk(r, p % C::KCH);
            koff[u] = (uint32_t)r * (uint32_t)a.k_sn * 2u + 16u * (uint32_t)c;
        }
    };
    // buffer resource over tile t of the range (absolute tile T0 + t), ending
    // at the last key of the whole K (rows past it read as zeros)
    auto tile_rsrc = [&](int t) __attribute__((always_inline)) {
        const int T = T0 + t;
        const int rem = a.Nkv - T * TK;  // keys left, >= 1
        u32x4 rk = buffer_rsrc(Kp + (int64_t)T * TK * a.k_sn,
                               (uint32_t)(((int64_t)(rem - 1) * a.k_sn + DQK) * 2));
#pragma unroll
        for (int i = 0; i < 4; ++i) rk[i] = __builtin_amdgcn_readfirstlane(rk[i]);
        return rk;
    };
    auto dma_tile = [&](const uint32_t (&koff)[C::KWIN_W], int t, int stage) __attribute__((always_inline)) {
        const u32x4 rk = tile_rsrc(t);
        unsigned char *st = lds + stage * C::KTILE_B;
        perturb_pause();
#pragma unroll
        for (int u = 0; u < C::KWIN_W; ++u) dma16_buf_to_lds(rk, koff[u], st + (4 * u + cw) * 1024);
    };
    // the end of a period in which this wave copied: its copies have landed
    // (vmcnt(0): a partial count did not order the LDS-DMA writes), then the
    // barrier publishes them
    auto copy_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // the first three tiles of the range (copied by the value waves, koff
    // non-null), landed and published
    auto prologue = [&](const uint32_t (*koff)[C::KWIN_W]) __attribute__((always_inline)) {
        __syncthreads();
        if (koff)
            for (int t = 0; t < 3 && t < n_tiles; ++t) dma_tile(*koff, t, t);
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    };

    // ---- P layout: row-major 80-byte rows, keys of each 16-key chunk at the
    // positions the P·V operand reads as one 16-byte piece (as in the 32-row
    // kernel); score wave (rg, kh) writes rows 32 rg + 16 rb + l16
    const uint32_t p_wr0 = (uint32_t)(32 * rg + l16) * C::PROW_B + 2 * (16 * kh + 8 * (G & 1) + 4 * (G >> 1));
    const uint32_t p_rd = (uint32_t)l32 * C::PROW_B + 2 * 8 * g;

    // combine a per-row value of the two key halves: score waves give v0 (row
    // block 0) and v1 (block 1) of their rows, every wave takes part in the
    // barrier; returns the combined values for the score wave's two rows
    auto combine_halves = [&](float v0, float v1, bool is_max, float &r0, float &r1) __attribute__((always_inline)) {
        if (sw && G == 0) {
            stat[64 * kh + 32 * rg + l16] = v0;
            stat[64 * kh + 32 * rg + 16 + l16] = v1;
        }
        lds_barrier();
        const int ra = 32 * rg + l16, rb = ra + 16;
        r0 = is_max ? fmaxf(stat[ra], stat[64 + ra]) : stat[ra] + stat[64 + ra];
        r1 = is_max ? fmaxf(stat[rb], stat[64 + rb]) : stat[rb] + stat[64 + rb];
    };
    // every wave gets l and m of rows l32 and 32 + l32 (the epilogue's rows)
    auto finish_stats = [&](float lp0, float lp1, float m0, float m1, float (&l_out)[2], float (&m_out)[2])
                            __attribute__((always_inline)) {
        float x0 = lp0, x1 = lp1;
        x0 += __shfl_xor(x0, 16);
        x0 += __shfl_xor(x0, 32);
        x1 += __shfl_xor(x1, 16);
        x1 += __shfl_xor(x1, 32);
        __syncthreads();
        if (sw && G == 0) {
            stat[64 * kh + 32 * rg + l16] = x0;
            stat[64 * kh + 32 * rg + 16 + l16] = x1;
            if (kh == 0) {
                stat[128 + 32 * rg + l16] = m0;
                stat[128 + 32 * rg + 16 + l16] = m1;
            }
        }
        __syncthreads();
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            l_out[rb] = stat[32 * rb + l32] + stat[64 + 32 * rb + l32];
            m_out[rb] = stat[128 + 32 * rb + l32];
        }
    };
    constexpr float kMaxL = 4294967296.0f;
    auto needs_exact = [&](const float (&l_row)[2]) __attribute__((always_inline)) {
        return __builtin_amdgcn_ballot_w64(!(l_row[0] <= kMaxL) || !(l_row[1] <= kMaxL)) != 0;
    };

    // The two roles run separate code with the same sequence of barriers:
    //   pass: prologue, [reference: one], after P(0): one, then one per tile
    //   t < n_tiles - 1; stats: two; if some row needs exact maxima: the max
    //   pass (prologue, one per tile), one, the pass again, stats again.
    if (sw) {
        // ================= score waves =================
        uint32_t kb[2];
        {
            const int r = 16 * kh + l16;
            const int t = (r >> 1) & 7, sz = t ^ ((t & 1) << 2);
            const uint32_t base = (uint32_t)(uintptr_t)(lds_void *)lds + (uint32_t)(r * C::KROW_B + 16 * (kg ^ (sz & 3)));
            kb[0] = base + 64 * (0 ^ (sz >> 2));
            kb[1] = base + 64 * (1 ^ (sz >> 2));
        }
        const int srow0 = q0 + 32 * rg + l16, srow1 = srow0 + 16;  // this lane's rows in the two blocks
        bf16x8 qa[C::NKS], qb[C::NKS];
        auto load_q = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) {
                u32x4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
                if (srow0 < a.Nq) v0 = load8_bf16(Qp + (int64_t)srow0 * a.q_sn + 32 * ks + 8 * kg);
                if (srow1 < a.Nq) v1 = load8_bf16(Qp + (int64_t)srow1 * a.q_sn + 32 * ks + 8 * kg);
                qa[ks] = u32x4_as_bf16x8(v0);
                qb[ks] = u32x4_as_bf16x8(v1);
            }
        };
        float m0 = 0.f, m1 = 0.f;  // references of rows srow0, srow1 (score*c units)
        float l0 = 0.f, l1 = 0.f;  // normalizers over this lane's keys
        auto kreads0 = [&](int stage) __attribute__((always_inline)) {
            const uint32_t so = stage * C::KTILE_B;
            wvks_kreads0(kb[0] + so, kb[1] + so);
        };
        // the score blocks of range tile t (first K reads issued)
        auto scores = [&](int t, int stage, float (&sv0)[4], float (&sv1)[4]) __attribute__((always_inline)) {
            const uint32_t so = stage * C::KTILE_B;
            f32x4 s0, s1;
            wvks_qk(qa, qb, kb[0] + so, kb[1] + so, s0, s1);
#pragma unroll
            for (int i = 0; i < 4; ++i) sv0[i] = s0[i], sv1[i] = s1[i];
            const int key0 = (T0 + t) * TK + 16 * kh + 4 * G;
            if (key0 + 4 > a.Nkv) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (key0 + i >= a.Nkv) sv0[i] = -INFINITY, sv1[i] = -INFINITY;
            }
        };
        auto block_row_max = [&](const float (&sv)[4]) __attribute__((always_inline)) {
            float x = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            x = fmaxf(x, __shfl_xor(x, 16));
            x = fmaxf(x, __shfl_xor(x, 32));
            return x;
        };
        auto block_p = [&](int t, const float (&sv0)[4], const float (&sv1)[4]) __attribute__((always_inline)) {
            unsigned char *pb = lds + C::POFF + (t & 1) * C::PBUF_B;
            {
                const float negm = -m0;
                const float e0 = exp2_hw(fmaf(sv0[0], a.c, negm)), e1 = exp2_hw(fmaf(sv0[1], a.c, negm));
                const float e2 = exp2_hw(fmaf(sv0[2], a.c, negm)), e3 = exp2_hw(fmaf(sv0[3], a.c, negm));
                const uint32_t p01 = pack_bf16x2(e0, e1), p23 = pack_bf16x2(e2, e3);
                l0 = sum_bf16x2(p23, sum_bf16x2(p01, l0));
                *(u32x2 *)(pb + p_wr0) = u32x2{p01, p23};
            }
            {
                const float negm = -m1;
                const float e0 = exp2_hw(fmaf(sv1[0], a.c, negm)), e1 = exp2_hw(fmaf(sv1[1], a.c, negm));
                const float e2 = exp2_hw(fmaf(sv1[2], a.c, negm)), e3 = exp2_hw(fmaf(sv1[3], a.c, negm));
                const uint32_t p01 = pack_bf16x2(e0, e1), p23 = pack_bf16x2(e2, e3);
                l1 = sum_bf16x2(p23, sum_bf16x2(p01, l1));
                *(u32x2 *)(pb + p_wr0 + 16 * C::PROW_B) = u32x2{p01, p23};
            }
        };
        auto pass = [&](bool set_m) __attribute__((always_inline)) {
            l0 = 0.f, l1 = 0.f;
            load_q();
            prologue(nullptr);
            kreads0(0);
            {
                float sv0[4], sv1[4];
                scores(0, 0, sv0, sv1);
                if (n_tiles > 1) kreads0(1);  // tile 1 landed in the prologue
                if (set_m) {
                    float mx0, mx1;
                    combine_halves(block_row_max(sv0), block_row_max(sv1), true, mx0, mx1);
                    mx0 *= a.c, mx1 *= a.c;
                    m0 = (mx0 == -INFINITY) ? 0.f : mx0;
                    m1 = (mx1 == -INFINITY) ? 0.f : mx1;
                }
                block_p(0, sv0, sv1);
                lds_barrier();  // P(0) written; tile 1 landed in the prologue
            }
            // the first fragments of tile t + 2 are read right after the score
            // block of tile t + 1 (that tile landed a period earlier, and the
            // register ring is free), so the next block starts on them
            for (int t = 0; t + 1 < n_tiles; ++t) {
                float sv0[4], sv1[4];
                scores(t + 1, (t + 1) & 3, sv0, sv1);
                if (t + 2 < n_tiles) kreads0((t + 2) & 3);
                block_p(t + 1, sv0, sv1);
                lds_barrier();
            }
        };
        auto max_pass = [&](float &M0, float &M1) __attribute__((always_inline)) {
            M0 = -INFINITY, M1 = -INFINITY;
            load_q();
            prologue(nullptr);
            kreads0(0);
            for (int t = 0; t < n_tiles; ++t) {
                float sv0[4], sv1[4];
                scores(t, t & 3, sv0, sv1);
                M0 = fmaxf(M0, block_row_max(sv0) * a.c);
                M1 = fmaxf(M1, block_row_max(sv1) * a.c);
                lds_barrier();
                if (t + 1 < n_tiles) kreads0((t + 1) & 3);
            }
        };
        pass(true);
        float l_row[2], m_row[2];
        finish_stats(l0, l1, m0, m1, l_row, m_row);
        if (needs_exact(l_row)) {
            float M0, M1;
            max_pass(M0, M1);
            __syncthreads();
            float c0, c1;
            combine_halves(M0, M1, true, c0, c1);
            m0 = (c0 == -INFINITY) ? 0.f : c0;
            m1 = (c1 == -INFINITY) ? 0.f : c1;
            pass(false);
            finish_stats(l0, l1, m0, m1, l_row, m_row);
        }
    } else {
        // ================= value waves =================
        uint32_t koff[C::KWIN_W];
        copy_offsets(koff);
        uint32_t vtb[2][CBW];
        {
            const int i16 = lane & 15;
#pragma unroll
            for (int hr = 0; hr < 2; ++hr)
#pragma unroll
                for (int i = 0; i < CBW; ++i) {
                    const int vr = 8 * hr + 4 * g + (i16 >> 2);
                    const int col = 32 * (CBW * vw + i) + 16 * (G & 1) + 4 * (i16 & 3);
                    vtb[hr][i] = (uint32_t)(uintptr_t)(lds_void *)lds +
                                 (uint32_t)(vr * C::KROW_B + 16 * wide_vk_chunk(vr, col >> 3) + 2 * (col & 7));
                }
        }
        auto vt_frag_k = [&](uint32_t stage_off, int i, int kc) __attribute__((always_inline)) {
            i16x4 hv[2];
#pragma unroll
            for (int hr = 0; hr < 2; ++hr) {
                const uint32_t addr = vtb[hr][i] + stage_off + 16 * C::KROW_B * kc;
                hv[hr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(uintptr_t)addr);
            }
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7));
        };
        f32x16 oacc[2][CBW];  // [row block][column block]
        auto pv_tile = [&](int t) __attribute__((always_inline)) {
            const unsigned char *pb = lds + C::POFF + (t & 1) * C::PBUF_B;
            const uint32_t stage_off = (t & 3) * C::KTILE_B;
            bf16x8 pf[2][2], vf[2][CBW];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc)
                    pf[rb][kc] = *(const bf16x8 *)(pb + p_rd + 32 * rb * C::PROW_B + 32 * kc);
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int i = 0; i < CBW; ++i) vf[kc][i] = vt_frag_k(stage_off, i, kc);
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int i = 0; i < CBW; ++i)
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) oacc[rb][i] = mfma_32x32x16(vf[kc][i], pf[rb][kc], oacc[rb][i]);
        };
        auto pass = [&](bool set_m) __attribute__((always_inline)) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < CBW; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[rb][i][r] = 0.f;
            prologue(&koff);
            if (set_m) {
                float d0, d1;
                combine_halves(0.f, 0.f, true, d0, d1);  // the score waves' reference barrier
            }
            lds_barrier();  // P(0) written
            for (int t = 0; t < n_tiles; ++t) {
                if (t + 3 < n_tiles) dma_tile(koff, t + 3, (t + 3) & 3);
                pv_tile(t);
                if (t + 1 < n_tiles) copy_barrier();
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no copy outlives the pass
        };
        auto max_pass = [&]() __attribute__((always_inline)) {
            prologue(&koff);
            for (int t = 0; t < n_tiles; ++t) {
                if (t + 3 < n_tiles) dma_tile(koff, t + 3, (t + 3) & 3);
                copy_barrier();
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        };
        pass(true);
        float l_row[2], m_row[2];
        finish_stats(0.f, 0.f, 0.f, 0.f, l_row, m_row);
        if (needs_exact(l_row)) {
            max_pass();
            __syncthreads();
            float d0, d1;
            combine_halves(0.f, 0.f, true, d0, d1);
            pass(false);
            finish_stats(0.f, 0.f, 0.f, 0.f, l_row, m_row);
        }

        // ---- this range's O / l (fp32) and logsumexp, per row -----------------
        // Through LDS (every wave is past the statistics' barriers and every
        // copy has landed; the staged blocks end below the P buffers and the
        // statistics): each lane writes its rows' runs of four columns to this
        // wave's 64-row block (rows padded by 16 bytes), then each store
        // covers two rows' 512 contiguous bytes instead of 16 bytes in each of
        // 32 rows.
        constexpr int SRB = 4 * 32 * CBW + 16;
        static_assert((C::NWAVE - C::NSW) * C::TQ * SRB <= C::POFF, "the staged O stays in the K ring");
        unsigned char *const stg = lds + vw * C::TQ * SRB;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const float inv_l = 1.0f / l_row[rb];
#pragma unroll
            for (int i = 0; i < CBW; ++i)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int col = 32 * i + acc_row(4 * rr, g);
                    *(f32x4 *)(stg + (32 * rb + l32) * SRB + 4 * col) =
                        f32x4{oacc[rb][i][4 * rr] * inv_l, oacc[rb][i][4 * rr + 1] * inv_l,
                              oacc[rb][i][4 * rr + 2] * inv_l, oacc[rb][i][4 * rr + 3] * inv_l};
                }
            const int row = q0 + 32 * rb + l32;
            if (vw == 0 && g == 0 && row < a.Nq)
                lpart[prow0 + row] = (m_row[rb] + log2f(l_row[rb])) * 0.69314718055994531f;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int rl = lane >> 5, cl = lane & 31;  // 32 lanes x 16 bytes per row
#pragma unroll
        for (int it = 0; it < C::TQ / 2; ++it) {
            const int r = 2 * it + rl;
            const f32x4 v = *(const f32x4 *)(stg + r * SRB + 16 * cl);
            if (q0 + r < a.Nq) *(f32x4 *)(opart + (prow0 + q0 + r) * DV + 32 * CBW * vw + 4 * cl) = v;
        }
    }
#endif
}

// Merge of the ranges for wide rows: thread-wise over (row, 4 columns) in a
// grid-stride loop, each thread forming its row's weights from the ranges'
// logsumexps itself (the same few values for every thread of the row, served
// by the caches): lse = ln Σ_s exp(lse_s), largest term factored out, and
// O = Σ_s exp(lse_s - lse) O_s. Written for the handful of ranges the wide
// path uses; one memory pass over the partial outputs.
template <int D>
__global__ void __launch_bounds__(256) attn_split_merge_wide(const float *__restrict__ opart,
                                                             const float *__restrict__ lpart, int32_t n_splits,
                                                             int64_t n_rows, KernelArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int CG = D / 4;
    const int64_t items = n_rows * CG;
    for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items;
         it += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = it / CG;
        const int c = (int)(it % CG);
        float mx = -INFINITY;
        for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, lpart[(int64_t)s * n_rows + row]);
        const float mref = (mx == -INFINITY) ? 0.f : mx;
        float wsum = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < n_splits; ++s) {
            const float ls = lpart[(int64_t)s * n_rows + row];
            const float wgt = exp2_hw((ls - mref) * 1.4426950408889634f);
            wsum += wgt;
            if (wgt > 0.f) acc += wgt * *(const f32x4 *)(opart + ((int64_t)s * n_rows + row) * D + 4 * c);
        }
        const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
        const int64_t i = row % a.Nq, bh = row / a.Nq;
        const int64_t h = bh % a.Hq, b = bh / a.Hq;
        __bf16 *orow = (__bf16 *)a.o + b * a.o_sb + h * a.o_sh + i * a.o_sn + 4 * c;
        store4(orow, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
        if (c == 0 && a.lse)
            a.lse[row] = wsum > 0.f ? mref + log2f(wsum) * 0.69314718055994531f : -INFINITY;
    }
#endif
}

}  // namespace attn
