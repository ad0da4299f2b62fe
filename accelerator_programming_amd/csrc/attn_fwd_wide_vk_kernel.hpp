// Fused attention forward for wide heads whose values are the first d_v
// columns of the keys (d_qk = 576, d_v = 512: the latent-attention layout,
// one K/V head shared by every query head), with V given as that view of K.
//
// Same method as the other kernels (disjoint output tiles, "Distilling a 4.5
// hour CUDA talk", section 5; K/V streamed through LDS with the row softmax
// carried by a per-row reference and normalizer, section 7). What differs is
// how the 4 waves of a workgroup share the work of one 32-row query tile and
// a 32-key tile:
//  * Scores: wave w = 2 rh + kh owns the 16 x 16 block of keys
//    16 kh .. 16 kh + 15 and rows 16 rh .. 16 rh + 15 and computes it whole
//    (Sᵀ = K·Qᵀ, 18 k-steps of v_mfma_f32_16x16x32_bf16; it holds its 16
//    rows of Q in registers). It applies the mask and the exponential to its
//    block only and writes P (bf16) to LDS.
//  * Values: after one barrier every wave reads all of P and accumulates
//    output columns 128 w .. 128 w + 127 for all 32 rows (O = P·V split over
//    the value columns), reading its Vᵀ fragments from the K tile.
//  So no MFMA or exponential is repeated across waves (per tile a wave does
//  18 16x16 and 8 32x32 MFMAs and 4 exponentials per lane), and the only
//  per-tile exchange is the 2 KB of P.
//  * Row statistics: the reference m of a row (the maximum over the first 32
//    keys) and, at the end, its normalizer l are the two key halves' values
//    combined through LDS.
//  * K tiles (32 keys x 1152 bytes) sit in a four-stage LDS ring, filled by
//    LDS-DMA (buffer_load ... lds): after tile T's barrier each wave copies
//    its quarter of tile T + 3, and tile T + 2's barrier waits for it, which
//    leaves two tiles of time for the copies. One barrier per tile: P of
//    tile T is written to a double-buffered area before it and read after it.
//  * K rows are 72 16-byte chunks. Chunk c of row r is stored at
//    c ^ s(r), s(r) = t ^ 4 (t & 1), t = (r / 2) % 8: the 16 rows of a
//    fragment read (ds_read_b128) fall in 16 distinct bank groups, and so do
//    the 4 x 4 row/column pieces of a transposed Vᵀ read (ds_read_b64_tr_b16).
//  * Software pipeline: after the barrier of tile T a wave issues the LDS
//    reads of P·V(T) and the 18 K fragment reads of tile T + 1's scores (into
//    registers the compiler does not allocate, v184 .. v255), then the score
//    MFMAs of T + 1 (one assembly block that waits for each read in turn),
//    then the P·V MFMAs of T, then P of T + 1 and the barrier. So the read
//    latencies overlap MFMA work instead of following a barrier. (Left to
//    itself the compiler issues each K read right before its MFMA.)
//  * Softmax in base 2 with the per-row reference fixed by the first 32
//    keys, exact O = acc / l and lse, and a slow pass with exact row maxima
//    when some row's normalizer leaves [0, 2^32] (as in the main kernel).
#pragma once

#include "tile.hpp"

namespace attn {

template <int DQK, int DV>
struct WideVkCfg {
    static constexpr int TQ = 32;  // query rows per workgroup
    static constexpr int TK = 32;  // keys per tile
    static constexpr int NWAVE = 4;
    static constexpr int NT = 64 * NWAVE;
    static constexpr int KCH = DQK / 8;  // 16-byte chunks per K row
    static constexpr int KROW_B = 2 * DQK;
    static constexpr int KTILE_B = TK * KROW_B;
    static constexpr int NSTAGE = 4;
    static constexpr int NKS = DQK / 32;           // k-steps of a 16x16 score block
    static constexpr int PROW_B = 2 * TK + 16;     // P row: 32 bf16 + 16 bytes of padding
    static constexpr int PBUF_B = TQ * PROW_B;     // one P buffer
    static constexpr int POFF = NSTAGE * KTILE_B;  // P buffers after the ring
    static constexpr int SOFF = POFF + 2 * PBUF_B; // row statistics: [2 key halves][32 rows] + m[32]
    static constexpr int LDS_BYTES = SOFF + 3 * TQ * 4;
    static constexpr int KWIN_W = KTILE_B / 1024 / NWAVE;  // 1 KB pieces per wave per tile
    static constexpr int CBW = DV / 32 / NWAVE;            // 32-column blocks of O per wave
    static_assert(KTILE_B % (1024 * NWAVE) == 0, "tile pieces must split over the waves");
    static_assert(NKS == 18, "the score block is written for 18 k-steps");
    static_assert(KCH % 8 == 0, "the swizzle permutes aligned groups of 8 chunks");
    static_assert(DV % (32 * NWAVE) == 0 && DV <= DQK, "value columns");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Physical chunk of logical chunk c in K row r (an involution in c).
__device__ __forceinline__ int wide_vk_chunk(int r, int c) {
    const int t = (r >> 1) & 7;
    return c ^ (t ^ ((t & 1) << 2));
}

// ---- the score block ----------------------------------------------------------
// K fragment ks (k-step ks, ks = 0..17) sits in v[184 + 4 ks : 187 + 4 ks].
// wide_vk_kreads reads fragment 2 j + b from kb_b + 128 j (kb0, kb1: this
// lane's addresses of fragments 0 and 1 in the stage); wide_vk_qk waits for
// read ks with lgkmcnt(min(17 - ks, 15)): LDS operations finish in order and
// a wave never has more than 15 in flight, so later LDS traffic only makes
// that wait stricter. The block ends with enough wait states for VALU, LDS
// or memory reads of the accumulator (the compiler does not see the MFMA
// latency through an asm statement).
#define WIDE_VK_S(x) #x
#define WIDE_VK_STR(x) WIDE_VK_S(x)
#define WIDE_VK_KREAD(KS, B, J)                                                                       \
    "ds_read_b128 v[" WIDE_VK_STR(184 + 4 * KS) ":" WIDE_VK_STR(187 + 4 * KS) "], %[kb" #B "] offset:" \
    WIDE_VK_STR(128 * J) "\n\t"
#define WIDE_VK_CLOBBERS                                                                              \
    "v184", "v185", "v186", "v187", "v188", "v189", "v190", "v191", "v192", "v193", "v194", "v195", \
        "v196", "v197", "v198", "v199", "v200", "v201", "v202", "v203", "v204", "v205", "v206",     \
        "v207", "v208", "v209", "v210", "v211", "v212", "v213", "v214", "v215", "v216", "v217",     \
        "v218", "v219", "v220", "v221", "v222", "v223", "v224", "v225", "v226", "v227", "v228",     \
        "v229", "v230", "v231", "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239",     \
        "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250",     \
        "v251", "v252", "v253", "v254", "v255"

__device__ __forceinline__ void wide_vk_kreads(uint32_t kb0, uint32_t kb1) {
    asm volatile(WIDE_VK_KREAD(0, 0, 0) WIDE_VK_KREAD(1, 1, 0) WIDE_VK_KREAD(2, 0, 1)
                 WIDE_VK_KREAD(3, 1, 1) WIDE_VK_KREAD(4, 0, 2) WIDE_VK_KREAD(5, 1, 2)
                 WIDE_VK_KREAD(6, 0, 3) WIDE_VK_KREAD(7, 1, 3) WIDE_VK_KREAD(8, 0, 4)
                 WIDE_VK_KREAD(9, 1, 4) WIDE_VK_KREAD(10, 0, 5) WIDE_VK_KREAD(11, 1, 5)
                 WIDE_VK_KREAD(12, 0, 6) WIDE_VK_KREAD(13, 1, 6) WIDE_VK_KREAD(14, 0, 7)
                 WIDE_VK_KREAD(15, 1, 7) WIDE_VK_KREAD(16, 0, 8) WIDE_VK_KREAD(17, 1, 8)
                 :
                 : [kb0] "v"(kb0), [kb1] "v"(kb1)
                 : WIDE_VK_CLOBBERS, "memory");
}

#define WIDE_VK_STEP(WAIT, KS, C)                                                                   \
    "s_waitcnt lgkmcnt(" WIDE_VK_STR(WAIT) ")\n\t"                                                  \
    "v_mfma_f32_16x16x32_bf16 %[s], v[" WIDE_VK_STR(184 + 4 * KS) ":" WIDE_VK_STR(187 + 4 * KS) "], " \
    "%[q" #KS "], " C "\n\t"

__device__ __forceinline__ f32x4 wide_vk_qk(const bf16x8 (&q)[18]) {
    f32x4 s;
    asm volatile(WIDE_VK_STEP(15, 0, "0") WIDE_VK_STEP(15, 1, "%[s]") WIDE_VK_STEP(15, 2, "%[s]")
                 WIDE_VK_STEP(14, 3, "%[s]") WIDE_VK_STEP(13, 4, "%[s]") WIDE_VK_STEP(12, 5, "%[s]")
                 WIDE_VK_STEP(11, 6, "%[s]") WIDE_VK_STEP(10, 7, "%[s]") WIDE_VK_STEP(9, 8, "%[s]")
                 WIDE_VK_STEP(8, 9, "%[s]") WIDE_VK_STEP(7, 10, "%[s]") WIDE_VK_STEP(6, 11, "%[s]")
                 WIDE_VK_STEP(5, 12, "%[s]") WIDE_VK_STEP(4, 13, "%[s]") WIDE_VK_STEP(3, 14, "%[s]")
                 WIDE_VK_STEP(2, 15, "%[s]") WIDE_VK_STEP(1, 16, "%[s]") WIDE_VK_STEP(0, 17, "%[s]")
                 "s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : [s] "=&a"(s)
                 : [q0] "v"(q[0]), [q1] "v"(q[1]), [q2] "v"(q[2]), [q3] "v"(q[3]), [q4] "v"(q[4]),
                   [q5] "v"(q[5]), [q6] "v"(q[6]), [q7] "v"(q[7]), [q8] "v"(q[8]), [q9] "v"(q[9]),
                   [q10] "v"(q[10]), [q11] "v"(q[11]), [q12] "v"(q[12]), [q13] "v"(q[13]),
                   [q14] "v"(q[14]), [q15] "v"(q[15]), [q16] "v"(q[16]), [q17] "v"(q[17])
                 : "memory");
    return s;
}

template <int DQK, int DV, bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
__attribute__((amdgpu_num_vgpr(184)))  // v184 .. v255: the K fragments of the asm blocks
attn_fwd_wide_vk_kernel(const KernelArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    using C = WideVkCfg<DQK, DV>;
    constexpr int TK = C::TK, CBW = C::CBW;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;    // 32x32 fragments (P·V)
    const int l16 = lane & 15, G = lane >> 4;    // 16x16 fragments (scores)
    const int kh = w & 1, rh = w >> 1;           // this wave's score block
    // k-group of this lane's 8 contraction elements in a k-step: quarter G
    // takes group (G % 2) * 2 + G / 2, so that the two quarters whose LDS
    // reads are served together (lanes i and i + 32) read chunks 4 ks + x and
    // 4 ks + x + 1 (x even): with the row swizzle below the 16 lanes of such a
    // pass then hit distinct banks. Q uses the same assignment.
    const int kg = ((G & 1) << 1) | (G >> 1);

    // ---- work item ----------------------------------------------------------
    const int BH = a.B * a.Hq;
    const int bh = blockIdx.x % BH;
    int qt = blockIdx.x / BH;
    if (CAUSAL) qt = a.n_qtiles - 1 - qt;
    const int b = bh / a.Hq, h = bh % a.Hq, hk = h / a.group;
    const __bf16 *__restrict__ Qp = (const __bf16 *)a.q + b * a.q_sb + h * a.q_sh;
    const __bf16 *__restrict__ Kp = (const __bf16 *)a.k + b * a.k_sb + hk * a.k_sh;
    __bf16 *__restrict__ Op = (__bf16 *)a.o + b * a.o_sb + h * a.o_sh;

    const int q0 = qt * C::TQ;
    const int row = q0 + l32;             // this lane's row in P·V and the epilogue
    const int srow = q0 + 16 * rh + l16;  // this lane's row in the score block
    const int kv_end = CAUSAL ? min(a.Nkv, q0 + C::TQ) : a.Nkv;
    const int n_tiles = (kv_end + TK - 1) / TK;  // >= 1
    // tiles from this index on need the causal or key-range mask
    const int first_masked = CAUSAL ? min(q0 / TK, a.Nkv / TK) : a.Nkv / TK;

    // ---- Q of the block's 16 rows (B operands), resident throughout ---------
    bf16x8 qf[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
        u32x4 v = {0, 0, 0, 0};
        if (srow < a.Nq) v = load8_bf16(Qp + (int64_t)srow * a.q_sn + 32 * ks + 8 * kg);
        qf[ks] = u32x4_as_bf16x8(v);
    }

    // ---- K staging: piece u of wave w is the 1 KB at (4u + w) KB of the tile;
    // lane i moves its 16-byte unit 64 (4u + w) + i, which holds the logical
    // chunk the swizzle puts there. The byte offsets inside a tile are the
    // same for every tile; the copies go through a buffer resource that ends
    // at the last key, so rows past it read as zeros (finite, masked). -----
    uint32_t koff[C::KWIN_W];
#pragma unroll
    for (int u = 0; u < C::KWIN_W; ++u) {
        const int p = (C::NWAVE * u + w) * 64 + lane;
        const int r = p / C::KCH, c = wide_vk_chunk(r, p % C::KCH);
        koff[u] = (uint32_t)r * (uint32_t)a.k_sn * 2u + 16u * (uint32_t)c;
    }
    // LDS-DMA of tile T into a stage: 9 buffer_load ... lds per wave, each
    // 1 KB, counted by vmcnt (nothing else in the loop uses it).
    auto dma_tile = [&](int T, int stage) __attribute__((always_inline)) {
        const int rem = a.Nkv - T * TK;  // keys left, >= 1
        const u32x4 rk = buffer_rsrc(Kp + (int64_t)T * TK * a.k_sn,
                                     (uint32_t)(((int64_t)(rem - 1) * a.k_sn + DQK) * 2));
        unsigned char *st = lds + stage * C::KTILE_B;
#pragma unroll
        for (int u = 0; u < C::KWIN_W; ++u) dma16_buf_to_lds(rk, koff[u], st + (C::NWAVE * u + w) * 1024);
    };
    // this wave's LDS accesses are done, then every wave reaches this point;
    // DMAs stay in flight (also a compiler memory barrier)
    auto lds_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // the same, after this wave's DMAs but the newest tile's (9) have landed:
    // each wave waits for its own share, the barrier covers all shares
    auto dma_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    // ---- K fragment addresses: key row r = 16 kh + l16, chunk 4 ks + kg. With
    // s = the row's swizzle, (4 ks + kg) ^ s = 4 (ks ^ s/4) + (kg ^ s%4), and
    // s/4 < 2 only flips ks's low bit: fragment 2 j + b is at kb_b + 128 j. --
    uint32_t kb[2];
    {
        const int r = 16 * kh + l16;
        const int t = (r >> 1) & 7, s = t ^ ((t & 1) << 2);
        const uint32_t base = (uint32_t)(uintptr_t)(lds_void *)lds + (uint32_t)(r * C::KROW_B + 16 * (kg ^ (s & 3)));
        kb[0] = base + 64 * (0 ^ (s >> 2));
        kb[1] = base + 64 * (1 ^ (s >> 2));
    }
    auto kreads = [&](int stage) __attribute__((always_inline)) {
        wide_vk_kreads(kb[0] + stage * C::KTILE_B, kb[1] + stage * C::KTILE_B);
    };

    // ---- P layout: row-major, 80-byte rows (conflict-free 16-byte reads of 16
    // rows); within each 16-key chunk key 4 q + i (q < 4, i < 4) sits at
    // position 8 (q % 2) + 4 (q / 2) + i, so that the 8 keys a P·V operand
    // lane needs (4g + i and 8 + 4g + i, the 32x32 accumulator's key order)
    // are one 16-byte piece. ----------------------------------------------
    const uint32_t p_wr = (uint32_t)(l16 + 16 * rh) * C::PROW_B + 2 * (16 * kh + 8 * (G & 1) + 4 * (G >> 1));
    const uint32_t p_rd = (uint32_t)l32 * C::PROW_B + 2 * 8 * g;

    // ---- state -------------------------------------------------------------
    f32x16 oacc[CBW];
    float m = 0.f;  // reference of row srow (score*c units), same in both key halves
    float l;        // normalizer of row srow over this lane's keys
    float *stat = (float *)(lds + C::SOFF);  // [kh][32] per-half row values, then m[32]

    // ---- Vᵀ fragments (value columns 32 db .. 32 db + 31, keys 16 kc ..
    // 16 kc + 15, db = 4w + i): two transposed reads (key halves hr) of the K
    // tile, whose rows begin with the values. Lane (4 g + i16 / 4 + 8 hr + 16 kc,
    // column 32 db + 16 (G % 2) + 4 (i16 % 4)) reads 4 values. The row's
    // swizzle s does not depend on kc, and XOR-ing the chunk 4 db + x (x < 4)
    // with s gives 4 (db ^ s/4) + (x ^ s%4): the address of (i, kc, hr) is
    // vtb[hr][i % 2] + 128 (i / 2) + 16 rows (kc). -------------------------
    static_assert(CBW == 4, "column blocks 4w + i, i < 4");
    uint32_t vtb[2][2];
    {
        const int i16 = lane & 15;
#pragma unroll
        for (int hr = 0; hr < 2; ++hr)
#pragma unroll
            for (int ip = 0; ip < 2; ++ip) {
                const int vr = 8 * hr + 4 * g + (i16 >> 2);
                const int col = 32 * (CBW * w + ip) + 16 * (G & 1) + 4 * (i16 & 3);
                vtb[hr][ip] = (uint32_t)(uintptr_t)(lds_void *)lds +
                              (uint32_t)(vr * C::KROW_B + 16 * wide_vk_chunk(vr, col >> 3) + 2 * (col & 7));
            }
    }
    auto vt_frag_k = [&](uint32_t stage_off, int i, int kc) __attribute__((always_inline)) {
        i16x4 hv[2];
#pragma unroll
        for (int hr = 0; hr < 2; ++hr) {
            const uint32_t addr = vtb[hr][i & 1] + stage_off + 128 * (i >> 1) + 16 * C::KROW_B * kc;
            hv[hr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(uintptr_t)addr);
        }
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // P·V of a tile in two parts: the LDS reads (P and the Vᵀ fragments) and
    // the MFMAs, so that the next tile's score block can go between them
    auto pv_reads = [&](const unsigned char *pb, int stage, bf16x8 (&pf)[2], bf16x8 (&vf)[2][CBW])
                        __attribute__((always_inline)) {
        const uint32_t stage_off = stage * C::KTILE_B;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) pf[kc] = *(const bf16x8 *)(pb + p_rd + 32 * kc);
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int i = 0; i < CBW; ++i) vf[kc][i] = vt_frag_k(stage_off, i, kc);
    };
    auto pv_mma = [&](const bf16x8 (&pf)[2], const bf16x8 (&vf)[2][CBW]) __attribute__((always_inline)) {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int i = 0; i < CBW; ++i) oacc[i] = mfma_32x32x16(vf[kc][i], pf[kc], oacc[i]);
    };
    // maximum of this lane's block row over the 4 lanes that share it
    auto block_row_max = [&](const float (&sv)[4]) __attribute__((always_inline)) {
        float x = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        x = fmaxf(x, __shfl_xor(x, 16));
        x = fmaxf(x, __shfl_xor(x, 32));
        return x;
    };
    // combine a per-row value of the two key halves: both halves' waves get
    // v(half 0) op v(half 1) (one barrier); returns it for row srow
    auto combine_halves = [&](float v, bool is_max) __attribute__((always_inline)) {
        if (G == 0) stat[32 * kh + 16 * rh + l16] = v;
        lds_barrier();
        const float v0 = stat[16 * rh + l16], v1 = stat[32 + 16 * rh + l16];
        return is_max ? fmaxf(v0, v1) : v0 + v1;
    };
    // the score block of tile T (its K fragments already read), masked
    auto scores = [&](int T, float (&sv)[4]) __attribute__((always_inline)) {
        const f32x4 sacc = wide_vk_qk(qf);
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[i] = sacc[i];
        if (T >= first_masked) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = T * TK + 16 * kh + 4 * G + i;
                if ((CAUSAL && key > srow) || key >= a.Nkv) sv[i] = -INFINITY;
            }
        }
    };
    // P of the block (bf16) into tile T's P buffer, and l
    auto block_p = [&](int T, const float (&sv)[4]) __attribute__((always_inline)) {
        const float negm = -m;
        const float e0 = exp2_hw(fmaf(sv[0], a.c, negm)), e1 = exp2_hw(fmaf(sv[1], a.c, negm));
        const float e2 = exp2_hw(fmaf(sv[2], a.c, negm)), e3 = exp2_hw(fmaf(sv[3], a.c, negm));
        const uint32_t p01 = pack_bf16x2(e0, e1), p23 = pack_bf16x2(e2, e3);
        l = sum_bf16x2(p23, sum_bf16x2(p01, l));
        *(u32x2 *)(lds + C::POFF + (T & 1) * C::PBUF_B + p_wr) = u32x2{p01, p23};
    };
    // tiles 0, 1, 2 into stages 0, 1, 2; tile 0 landed everywhere; its K
    // fragment reads issued
    auto prologue = [&]() __attribute__((always_inline)) {
        __syncthreads();  // the ring, the P buffers and the statistics are free
        dma_tile(0, 0);
        dma_tile(min(1, n_tiles - 1), 1);
        dma_tile(min(2, n_tiles - 1), 2);
        asm volatile("s_waitcnt vmcnt(18)\n\ts_barrier" ::: "memory");
        kreads(0);
    };

    // ---- one pass over the keys: O and l (set_m: the reference from tile 0)
    // Tile T's stage is T % 4. Software pipeline, one barrier per tile:
    //   [P·V reads of T] [K reads of T + 1] [copy of T + 3] [scores of T + 1]
    //   [P·V MFMAs of T] [P of T + 1] barrier
    // The barrier that publishes P of T + 1 also waits for this wave's copy
    // of tile T + 2 (two tiles old); the copy of T + 3 goes into the stage of
    // tile T - 1, which every wave finished before the previous barrier. The
    // copies are unconditional (past the last tile a free stage gets the last
    // tile again), so every vmcnt(9) is exact.
    auto pass = [&](bool set_m) __attribute__((always_inline)) {
        l = 0.f;
#pragma unroll
        for (int i = 0; i < CBW; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
        prologue();
        {
            float sv[4];
            scores(0, sv);
            if (set_m) {
                // reference: the row maximum over tile 0 (an extra barrier,
                // the same in every wave)
                const float mx = combine_halves(block_row_max(sv), true) * a.c;
                m = (mx == -INFINITY) ? 0.f : mx;
            }
            block_p(0, sv);
            dma_barrier();
        }
        for (int T = 0; T < n_tiles; ++T) {
            const bool more = T + 1 < n_tiles;
            bf16x8 pf[2], vf[2][CBW];
            pv_reads(lds + C::POFF + (T & 1) * C::PBUF_B, T & 3, pf, vf);
            if (more) kreads((T + 1) & 3);
            dma_tile(min(T + 3, n_tiles - 1), (T + 3) & 3);
            float sv[4];
            if (more) scores(T + 1, sv);
            pv_mma(pf, vf);
            if (more) {
                block_p(T + 1, sv);
                dma_barrier();
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no copy outlives the pass
    };
    // exact row maxima (in score*c units, combined over the key halves
    // later), no P·V; one barrier per tile as above
    auto max_pass = [&]() __attribute__((always_inline)) {
        float M = -INFINITY;
        prologue();
        for (int T = 0; T < n_tiles; ++T) {
            float sv[4];
            scores(T, sv);
            M = fmaxf(M, block_row_max(sv) * a.c);
            dma_barrier();
            dma_tile(min(T + 3, n_tiles - 1), (T + 3) & 3);
            if (T + 1 < n_tiles) kreads((T + 1) & 3);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return M;
    };

    // per-row l of the whole row (both halves, all lanes), for row l32 of the
    // epilogue; m of row l32 likewise
    auto finish_stats = [&](float &l_out, float &m_out) __attribute__((always_inline)) {
        float x = l;
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        __syncthreads();  // the statistics area is free
        if (G == 0) {
            stat[32 * kh + 16 * rh + l16] = x;
            if (kh == 0) stat[64 + 16 * rh + l16] = m;
        }
        __syncthreads();
        l_out = stat[l32] + stat[32 + l32];
        m_out = stat[64 + l32];
    };

    constexpr float kMaxL = 4294967296.0f;  // 2^32: every p <= 2^32 when l <= 2^32
    pass(true);
    float l_row, m_row;
    finish_stats(l_row, m_row);
    // every wave holds the same 32 rows' normalizers
    const bool bad = __builtin_amdgcn_ballot_w64(!(l_row <= kMaxL)) != 0;
    if (bad) {
        // exact row maxima, then the pass again (rare)
        float M = max_pass();
        __syncthreads();
        M = combine_halves(M, true);
        m = (M == -INFINITY) ? 0.f : M;
        pass(false);
        finish_stats(l_row, m_row);
    }

    // ---- O = Oᵀ / l (one reciprocal per row), logsumexp ---------------------
    const float inv_l = 1.0f / l_row;
    if (row < a.Nq) {
        __bf16 *orow = Op + (int64_t)row * a.o_sn;
#pragma unroll
        for (int i = 0; i < CBW; ++i)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int col = 32 * (CBW * w + i) + acc_row(4 * rr, g);
                store4(orow + col, oacc[i][4 * rr] * inv_l, oacc[i][4 * rr + 1] * inv_l,
                       oacc[i][4 * rr + 2] * inv_l, oacc[i][4 * rr + 3] * inv_l);
            }
        if (w == 0 && g == 0 && a.lse)
            a.lse[((int64_t)b * a.Hq + h) * a.Nq + row] = (m_row + log2f(l_row)) * 0.69314718055994531f;
    }
#endif
}

}  // namespace attn
