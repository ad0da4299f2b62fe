// Fused attention forward for wide heads whose values are the first d_v
// columns of the keys (d_qk = 576, d_v = 512: the latent-attention layout,
// one K/V head shared by every query head), with V given as that view of K.
//
// Same method as the other kernels (disjoint output tiles, "Distilling a 4.5
// hour CUDA talk", section 5; K/V streamed through LDS with the row softmax
// carried by a per-row reference and normalizer, section 7). What differs is
// how the 8 waves of a workgroup (two per SIMD) share the work of one 32-row
// query tile and a 32-key tile:
//  * Score waves 0..3, w = 2 rh + kh, each own the 16 x 16 block of keys
//    16 kh .. 16 kh + 15 and rows 16 rh .. 16 rh + 15 and compute it whole
//    (Sᵀ = K·Qᵀ, 18 k-steps of v_mfma_f32_16x16x32_bf16, their 16 rows of Q
//    held in registers), apply the mask and the exponential to it and write
//    P (bf16) to LDS. They also move the K tiles into LDS (LDS-DMA), one
//    copy after each score MFMA, inside the score block.
//  * Value waves 4..7 (vw = w - 4), after the barrier that publishes a
//    tile's P, read all of it and accumulate output columns 128 vw ..
//    128 vw + 127 for all 32 rows (O = P·V split over the value columns),
//    reading their Vᵀ fragments from the K tile.
//  Each SIMD holds one score wave and one value wave: in each tile period
//  the score wave's MFMAs for tile T + 1 and the value wave's for tile T
//  share the SIMD's matrix pipe (18 16x16 + 8 32x32 MFMAs), and each wave's
//  LDS waits, exponentials and copies run beside the other's MFMAs. No MFMA
//  or exponential is repeated; the only per-tile exchange is the 2 KB of P.
//  The two roles run separate code, so that each keeps only its own
//  registers live (the Q fragments, or the O accumulators).
//  * Row statistics: the reference m of a row (the maximum over the first 32
//    keys) and, at the end, its normalizer l are the two key halves' values
//    combined through LDS.
//  * K tiles (32 keys x 1152 bytes) sit in a four-stage LDS ring: in the
//    period after tile T's barrier one pair of score waves issues tile T + 3
//    (the pairs take turns), and the barrier two tiles later waits for it.
//  * Software pipeline, one barrier per tile: after the barrier that
//    publishes P of tile T, the score waves read K of tile T + 1 and run its
//    score MFMAs (the copying pair issuing the copy of tile T + 3 between
//    them), then write its P; the value waves read P and Vᵀ of tile T and
//    run its P·V MFMAs.
//  * K rows are 72 16-byte chunks. Chunk c of row r is stored at
//    c ^ s(r), s(r) = t ^ 4 (t & 1), t = (r / 2) % 8; with the k-group
//    order below the 16 lanes served together by a fragment read
//    (ds_read_b128) or a transposed Vᵀ read (ds_read_b64_tr_b16) hit distinct
//    banks.
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
    static constexpr int NWAVE = 8;
    static constexpr int NT = 64 * NWAVE;
    static constexpr int NSW = 4;  // score waves (0..3), which also copy; the others do P·V
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
    static constexpr int KWIN_W = KTILE_B / 1024 / 2;  // 1 KB copies per copying wave per copied tile
    static constexpr int CBW = DV / 32 / (NWAVE - NSW);            // 32-column blocks of O per value wave
    static_assert(NSW == 4 && NWAVE - NSW == 4, "four score waves (two copy pairs), four value waves");
    static_assert(KTILE_B % 2048 == 0, "tile pieces must split over a pair of copying waves");
    static_assert(NKS == 18, "the score block is written for 18 k-steps");
    static_assert(KCH % 8 == 0, "the swizzle permutes aligned groups of 8 chunks");
    static_assert(CBW == 4 && DV <= DQK, "value columns 128 vw .. 128 vw + 127");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Physical chunk of logical chunk c in K row r (an involution in c).
__device__ __forceinline__ int wide_vk_chunk(int r, int c) {
    const int t = (r >> 1) & 7;
    return c ^ (t ^ ((t & 1) << 2));
}

// ---- the score block ----------------------------------------------------------
// K fragments go through a ring of 6 register quads in v[176:199], which the
// compiler does not allocate: fragment ks (k-step ks, ks = 0..17) uses slot
// ks % 6, v[176 + 4 (ks % 6) : 179 + 4 (ks % 6)]. Fragment 2 j + b is at
// kb_b + 128 j (kb0, kb1: this lane's addresses of fragments 0 and 1 in the
// stage). wide_vk_kreads0 reads fragments 0..5; wide_vk_qk first waits for
// every LDS access of the wave (lgkmcnt(0): the reads of fragments 0..5 and
// whatever the compiler issued before them; completion order across
// different LDS read instructions is not relied on), then issues read ks + 6
// into slot ks % 6 right after the MFMA of step ks (which took its operand
// at issue) and waits for read ks (ks >= 1) with lgkmcnt(min(5, 17 - ks)),
// counting only its own ds_read_b128s, which complete in order. Even
// k-steps accumulate into s and odd ones into t, two independent chains
// instead of one chain of 18 dependent MFMAs (C5 +1.4 %); the block returns
// s + t. It ends with enough wait states for VALU, LDS or memory reads of
// the accumulators (the compiler does not see the MFMA latency through an
// asm statement).
#define WIDE_VK_CLOBBERS                                                                              \
    "v176", "v177", "v178", "v179", "v180", "v181", "v182", "v183", "v184", "v185", "v186", "v187", \
        "v188", "v189", "v190", "v191", "v192", "v193", "v194", "v195", "v196", "v197", "v198", "v199"
// read of fragment ks: slot ks % 6, base kb(ks % 2), offset 128 (ks / 2)
#define WIDE_VK_KR0 "ds_read_b128 v[176:179], %[kb0] offset:0\n\t"
#define WIDE_VK_KR1 "ds_read_b128 v[180:183], %[kb1] offset:0\n\t"
#define WIDE_VK_KR2 "ds_read_b128 v[184:187], %[kb0] offset:128\n\t"
#define WIDE_VK_KR3 "ds_read_b128 v[188:191], %[kb1] offset:128\n\t"
#define WIDE_VK_KR4 "ds_read_b128 v[192:195], %[kb0] offset:256\n\t"
#define WIDE_VK_KR5 "ds_read_b128 v[196:199], %[kb1] offset:256\n\t"
#define WIDE_VK_KR6 "ds_read_b128 v[176:179], %[kb0] offset:384\n\t"
#define WIDE_VK_KR7 "ds_read_b128 v[180:183], %[kb1] offset:384\n\t"
#define WIDE_VK_KR8 "ds_read_b128 v[184:187], %[kb0] offset:512\n\t"
#define WIDE_VK_KR9 "ds_read_b128 v[188:191], %[kb1] offset:512\n\t"
#define WIDE_VK_KR10 "ds_read_b128 v[192:195], %[kb0] offset:640\n\t"
#define WIDE_VK_KR11 "ds_read_b128 v[196:199], %[kb1] offset:640\n\t"
#define WIDE_VK_KR12 "ds_read_b128 v[176:179], %[kb0] offset:768\n\t"
#define WIDE_VK_KR13 "ds_read_b128 v[180:183], %[kb1] offset:768\n\t"
#define WIDE_VK_KR14 "ds_read_b128 v[184:187], %[kb0] offset:896\n\t"
#define WIDE_VK_KR15 "ds_read_b128 v[188:191], %[kb1] offset:896\n\t"
#define WIDE_VK_KR16 "ds_read_b128 v[192:195], %[kb0] offset:1024\n\t"
#define WIDE_VK_KR17 "ds_read_b128 v[196:199], %[kb1] offset:1024\n\t"
// MFMA of step ks after waiting for its read; C: the accumulator input
#define WIDE_VK_MM0 "s_waitcnt lgkmcnt(0)\n\tv_mfma_f32_16x16x32_bf16 %[s], v[176:179], %[q0], " "0" "\n\t"
#define WIDE_VK_MM1 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[t], v[180:183], %[q1], " "0" "\n\t"
#define WIDE_VK_MM2 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s], v[184:187], %[q2], " "%[s]" "\n\t"
#define WIDE_VK_MM3 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[t], v[188:191], %[q3], " "%[t]" "\n\t"
#define WIDE_VK_MM4 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s], v[192:195], %[q4], " "%[s]" "\n\t"
#define WIDE_VK_MM5 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[t], v[196:199], %[q5], " "%[t]" "\n\t"
#define WIDE_VK_MM6 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s], v[176:179], %[q6], " "%[s]" "\n\t"
#define WIDE_VK_MM7 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[t], v[180:183], %[q7], " "%[t]" "\n\t"
#define WIDE_VK_MM8 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s], v[184:187], %[q8], " "%[s]" "\n\t"
#define WIDE_VK_MM9 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[t], v[188:191], %[q9], " "%[t]" "\n\t"
#define WIDE_VK_MM10 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s], v[192:195], %[q10], " "%[s]" "\n\t"
#define WIDE_VK_MM11 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[t], v[196:199], %[q11], " "%[t]" "\n\t"
#define WIDE_VK_MM12 "s_waitcnt lgkmcnt(5)\n\tv_mfma_f32_16x16x32_bf16 %[s], v[176:179], %[q12], " "%[s]" "\n\t"
#define WIDE_VK_MM13 "s_waitcnt lgkmcnt(4)\n\tv_mfma_f32_16x16x32_bf16 %[t], v[180:183], %[q13], " "%[t]" "\n\t"
#define WIDE_VK_MM14 "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_16x16x32_bf16 %[s], v[184:187], %[q14], " "%[s]" "\n\t"
#define WIDE_VK_MM15 "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_16x16x32_bf16 %[t], v[188:191], %[q15], " "%[t]" "\n\t"
#define WIDE_VK_MM16 "s_waitcnt lgkmcnt(1)\n\tv_mfma_f32_16x16x32_bf16 %[s], v[192:195], %[q16], " "%[s]" "\n\t"
#define WIDE_VK_MM17 "s_waitcnt lgkmcnt(0)\n\tv_mfma_f32_16x16x32_bf16 %[t], v[196:199], %[q17], " "%[t]" "\n\t"

__device__ __forceinline__ void wide_vk_kreads0(uint32_t kb0, uint32_t kb1) {
    asm volatile(WIDE_VK_KR0 WIDE_VK_KR1 WIDE_VK_KR2 WIDE_VK_KR3 WIDE_VK_KR4 WIDE_VK_KR5
                 :
                 : [kb0] "v"(kb0), [kb1] "v"(kb1)
                 : WIDE_VK_CLOBBERS, "memory");
}

__device__ __forceinline__ f32x4 wide_vk_qk(const bf16x8 (&q)[18], uint32_t kb0, uint32_t kb1) {
    f32x4 s, t;
    asm volatile(WIDE_VK_MM0 WIDE_VK_KR6 WIDE_VK_MM1 WIDE_VK_KR7 WIDE_VK_MM2 WIDE_VK_KR8
                 WIDE_VK_MM3 WIDE_VK_KR9 WIDE_VK_MM4 WIDE_VK_KR10 WIDE_VK_MM5 WIDE_VK_KR11
                 WIDE_VK_MM6 WIDE_VK_KR12 WIDE_VK_MM7 WIDE_VK_KR13 WIDE_VK_MM8 WIDE_VK_KR14
                 WIDE_VK_MM9 WIDE_VK_KR15 WIDE_VK_MM10 WIDE_VK_KR16 WIDE_VK_MM11 WIDE_VK_KR17
                 WIDE_VK_MM12 WIDE_VK_MM13 WIDE_VK_MM14 WIDE_VK_MM15 WIDE_VK_MM16 WIDE_VK_MM17
                 "s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : [s] "=&v"(s), [t] "=&v"(t)
                 : [kb0] "v"(kb0), [kb1] "v"(kb1),
                   [q0] "v"(q[0]), [q1] "v"(q[1]), [q2] "v"(q[2]), [q3] "v"(q[3]), [q4] "v"(q[4]),
                   [q5] "v"(q[5]), [q6] "v"(q[6]), [q7] "v"(q[7]), [q8] "v"(q[8]), [q9] "v"(q[9]),
                   [q10] "v"(q[10]), [q11] "v"(q[11]), [q12] "v"(q[12]), [q13] "v"(q[13]),
                   [q14] "v"(q[14]), [q15] "v"(q[15]), [q16] "v"(q[16]), [q17] "v"(q[17])
                 : WIDE_VK_CLOBBERS, "memory");
    return s + t;
}

// The same score block with the LDS-DMA of one K tile's share of a copying
// wave (18 x 1 KB) interleaved: DMA u right after the MFMA of k-step u, so
// that the copies reach the memory pipeline at the pace it takes them
// instead of as a burst that would stall the wave (about 16 cycles per 1 KB
// copy per CU). DMA u lands at LDS byte address mb + 2048 u; M0 is written
// inside the statement, each DMA followed by a wait state before the next
// M0 write. The copies are counted by vmcnt only, so the lgkmcnt waits of
// the block are unchanged.
#define WIDE_VK_DMA0 "s_add_u32 m0, %[mb], 0\n\tbuffer_load_dwordx4 %[o0], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA1 "s_add_u32 m0, %[mb], 2048\n\tbuffer_load_dwordx4 %[o1], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA2 "s_add_u32 m0, %[mb], 4096\n\tbuffer_load_dwordx4 %[o2], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA3 "s_add_u32 m0, %[mb], 6144\n\tbuffer_load_dwordx4 %[o3], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA4 "s_add_u32 m0, %[mb], 8192\n\tbuffer_load_dwordx4 %[o4], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA5 "s_add_u32 m0, %[mb], 10240\n\tbuffer_load_dwordx4 %[o5], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA6 "s_add_u32 m0, %[mb], 12288\n\tbuffer_load_dwordx4 %[o6], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA7 "s_add_u32 m0, %[mb], 14336\n\tbuffer_load_dwordx4 %[o7], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA8 "s_add_u32 m0, %[mb], 16384\n\tbuffer_load_dwordx4 %[o8], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA9 "s_add_u32 m0, %[mb], 18432\n\tbuffer_load_dwordx4 %[o9], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA10 "s_add_u32 m0, %[mb], 20480\n\tbuffer_load_dwordx4 %[o10], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA11 "s_add_u32 m0, %[mb], 22528\n\tbuffer_load_dwordx4 %[o11], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA12 "s_add_u32 m0, %[mb], 24576\n\tbuffer_load_dwordx4 %[o12], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA13 "s_add_u32 m0, %[mb], 26624\n\tbuffer_load_dwordx4 %[o13], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA14 "s_add_u32 m0, %[mb], 28672\n\tbuffer_load_dwordx4 %[o14], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA15 "s_add_u32 m0, %[mb], 30720\n\tbuffer_load_dwordx4 %[o15], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA16 "s_add_u32 m0, %[mb], 32768\n\tbuffer_load_dwordx4 %[o16], %[rk], 0 offen lds\n\ts_nop 0\n\t"
#define WIDE_VK_DMA17 "s_add_u32 m0, %[mb], 34816\n\tbuffer_load_dwordx4 %[o17], %[rk], 0 offen lds\n\ts_nop 0\n\t"

__device__ __forceinline__ f32x4 wide_vk_qk_copy(const bf16x8 (&q)[18], uint32_t kb0, uint32_t kb1,
                                                 const uint32_t (&o)[18], u32x4 rk, uint32_t mb) {
    f32x4 s, t;
    asm volatile(WIDE_VK_MM0 WIDE_VK_DMA0 WIDE_VK_KR6 WIDE_VK_MM1 WIDE_VK_DMA1 WIDE_VK_KR7
                 WIDE_VK_MM2 WIDE_VK_DMA2 WIDE_VK_KR8 WIDE_VK_MM3 WIDE_VK_DMA3 WIDE_VK_KR9
                 WIDE_VK_MM4 WIDE_VK_DMA4 WIDE_VK_KR10 WIDE_VK_MM5 WIDE_VK_DMA5 WIDE_VK_KR11
                 WIDE_VK_MM6 WIDE_VK_DMA6 WIDE_VK_KR12 WIDE_VK_MM7 WIDE_VK_DMA7 WIDE_VK_KR13
                 WIDE_VK_MM8 WIDE_VK_DMA8 WIDE_VK_KR14 WIDE_VK_MM9 WIDE_VK_DMA9 WIDE_VK_KR15
                 WIDE_VK_MM10 WIDE_VK_DMA10 WIDE_VK_KR16 WIDE_VK_MM11 WIDE_VK_DMA11 WIDE_VK_KR17
                 WIDE_VK_MM12 WIDE_VK_DMA12 WIDE_VK_MM13 WIDE_VK_DMA13 WIDE_VK_MM14 WIDE_VK_DMA14
                 WIDE_VK_MM15 WIDE_VK_DMA15 WIDE_VK_MM16 WIDE_VK_DMA16 WIDE_VK_MM17 WIDE_VK_DMA17
                 "s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : [s] "=&v"(s), [t] "=&v"(t)
                 : [kb0] "v"(kb0), [kb1] "v"(kb1),
                   [q0] "v"(q[0]), [q1] "v"(q[1]), [q2] "v"(q[2]), [q3] "v"(q[3]), [q4] "v"(q[4]),
                   [q5] "v"(q[5]), [q6] "v"(q[6]), [q7] "v"(q[7]), [q8] "v"(q[8]), [q9] "v"(q[9]),
                   [q10] "v"(q[10]), [q11] "v"(q[11]), [q12] "v"(q[12]), [q13] "v"(q[13]),
                   [q14] "v"(q[14]), [q15] "v"(q[15]), [q16] "v"(q[16]), [q17] "v"(q[17]),
                   [mb] "s"(mb), [rk] "s"(rk),
                   [o0] "v"(o[0]), [o1] "v"(o[1]), [o2] "v"(o[2]), [o3] "v"(o[3]), [o4] "v"(o[4]),
                   [o5] "v"(o[5]), [o6] "v"(o[6]), [o7] "v"(o[7]), [o8] "v"(o[8]), [o9] "v"(o[9]),
                   [o10] "v"(o[10]), [o11] "v"(o[11]), [o12] "v"(o[12]), [o13] "v"(o[13]),
                   [o14] "v"(o[14]), [o15] "v"(o[15]), [o16] "v"(o[16]), [o17] "v"(o[17])
                 : WIDE_VK_CLOBBERS, "memory", "scc");
    return s + t;
}

template <int DQK, int DV, bool CAUSAL>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
__attribute__((amdgpu_num_vgpr(176)))  // v176 .. v199: the K fragment ring of the asm blocks
attn_fwd_wide_vk_kernel(const KernelArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    using C = WideVkCfg<DQK, DV>;
    constexpr int TK = C::TK, CBW = C::CBW;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool sw = w < C::NSW;                  // a score wave (else a value wave)
    const int l32 = lane & 31, g = lane >> 5;    // 32x32 fragments (P·V)
    const int l16 = lane & 15, G = lane >> 4;    // 16x16 fragments (scores)
    const int kh = w & 1, rh = (w >> 1) & 1;     // a score wave's block
    const int vw = (w - C::NSW) & 3;             // a value wave's index
    // k-group of this lane's 8 contraction elements in a k-step: quarter G
    // takes group 0, 3, 1, 2 for G = 0..3. With the row swizzle this order
    // makes every K fragment read free of LDS bank conflicts (measured with
    // SQ_LDS_BANK_CONFLICT over the candidate orders: the natural order 0..3
    // costs 4 extra cycles per read). Q uses the same assignment.
    const int kg = (0x9C >> (2 * G)) & 3;

    // ---- work item ----------------------------------------------------------
    const int BH = a.B * a.Hq;
    const uint32_t wid = work_index(blockIdx.x, gridDim.x);
    const int bh = wid % BH;
    int qt = wid / BH;
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

    // this wave's LDS accesses are done, then every wave reaches this point
    // (also a compiler memory barrier)
    auto lds_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    float *stat = (float *)(lds + C::SOFF);  // [kh][32] per-half row values, then m[32]

    // ---- K copies (score waves): waves 0, 1 copy the even tiles, 2, 3 the
    // odd ones, so that a pair's copies of a tile are its only ones in flight
    // when it waits for them (vmcnt(0)) two tiles later. Piece u of pair
    // member cm is the 1 KB at (2u + cm) KB of the tile; lane i moves its
    // 16-byte unit 64 (2u + cm) + i, which holds the logical chunk the
    // swizzle puts there. The byte offsets inside a tile are the same for
    // every tile; the copies go through a buffer resource that ends at the
    // last key, so rows past it read as zeros (finite, masked). ----------
    const int cpair = (w >> 1) & 1, cm = w & 1;  // score waves' copy pair
    auto copy_offsets = [&](uint32_t (&koff)[C::KWIN_W]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < C::KWIN_W; ++u) {
            const int p = (2 * u + cm) * 64 + lane;
            const int r = p / C::KCH, c = wide_vk_chunk(r, p % C::KCH);
            koff[u] = (uint32_t)r * (uint32_t)a.k_sn * 2u + 16u * (uint32_t)c;
        }
    };
    // LDS-DMA of tile T into a stage by the pair T % 2 (score waves): 18
    // buffer_load ... lds per wave, each 1 KB, counted by vmcnt (nothing else
    // in the loop uses it). T is uniform; the resource is made explicitly so
    // (readfirstlane), as the instruction takes it in scalar registers.
    auto tile_rsrc = [&](int T) __attribute__((always_inline)) {
        const int rem = a.Nkv - T * TK;  // keys left, >= 1
        u32x4 rk = buffer_rsrc(Kp + (int64_t)T * TK * a.k_sn,
                               (uint32_t)(((int64_t)(rem - 1) * a.k_sn + DQK) * 2));
#pragma unroll
        for (int i = 0; i < 4; ++i) rk[i] = __builtin_amdgcn_readfirstlane(rk[i]);
        return rk;
    };
    auto dma_tile = [&](const uint32_t (&koff)[C::KWIN_W], int T, int stage) __attribute__((always_inline)) {
        if ((T & 1) != cpair) return;
        const u32x4 rk = tile_rsrc(T);
        unsigned char *st = lds + stage * C::KTILE_B;
        perturb_pause();
#pragma unroll
        for (int u = 0; u < C::KWIN_W; ++u) dma16_buf_to_lds(rk, koff[u], st + (2 * u + cm) * 1024);
    };
    // the end of a tile for a score wave: the pair that copied tile Tw first
    // waits for all its copies (vmcnt(0): a partial count did not order the
    // LDS-DMA writes); the barrier then publishes tile Tw to every wave
    auto copy_barrier = [&](int Tw) __attribute__((always_inline)) {
        if ((Tw & 1) == cpair)
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else
            lds_barrier();
    };
    // tiles 0, 1, 2 into stages 0, 1, 2 (score waves), landed everywhere
    auto prologue = [&](const uint32_t(&koff)[C::KWIN_W], bool copies) __attribute__((always_inline)) {
        __syncthreads();  // the ring, the P buffers and the statistics are free
        if (copies)
            for (int T = 0; T < 3 && T < n_tiles; ++T) dma_tile(koff, T, T);
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    };

    // ---- P layout: row-major, 80-byte rows (conflict-free 16-byte reads of 16
    // rows); within each 16-key chunk key 4 q + i (q < 4, i < 4) sits at
    // position 8 (q % 2) + 4 (q / 2) + i, so that the 8 keys a P·V operand
    // lane needs (4g + i and 8 + 4g + i, the 32x32 accumulator's key order)
    // are one 16-byte piece. ----------------------------------------------
    const uint32_t p_wr = (uint32_t)(l16 + 16 * rh) * C::PROW_B + 2 * (16 * kh + 8 * (G & 1) + 4 * (G >> 1));
    const uint32_t p_rd = (uint32_t)l32 * C::PROW_B + 2 * 8 * g;

    // combine a per-row value of the two key halves (score waves give it; one
    // barrier for all waves); returns v(half 0) op v(half 1) for row srow
    auto combine_halves = [&](float v, bool is_max) __attribute__((always_inline)) {
        if (sw && G == 0) stat[32 * kh + 16 * rh + l16] = v;
        lds_barrier();
        const float v0 = stat[16 * rh + l16], v1 = stat[32 + 16 * rh + l16];
        return is_max ? fmaxf(v0, v1) : v0 + v1;
    };
    // per-row l of the whole row (both halves), for row l32 of the epilogue,
    // and m of that row: score waves give their l_part and m, every wave gets
    // the results
    auto finish_stats = [&](float l_part, float m_srow, float &l_out, float &m_out)
                            __attribute__((always_inline)) {
        float x = l_part;
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        __syncthreads();  // the statistics area is free
        if (sw && G == 0) {
            stat[32 * kh + 16 * rh + l16] = x;
            if (kh == 0) stat[64 + 16 * rh + l16] = m_srow;
        }
        __syncthreads();
        l_out = stat[l32] + stat[32 + l32];
        m_out = stat[64 + l32];
    };
    constexpr float kMaxL = 4294967296.0f;  // 2^32: every p <= 2^32 when l <= 2^32
    // every wave holds the same 32 rows' normalizers, so the whole workgroup
    // takes the same decision
    auto needs_exact = [&](float l_row) __attribute__((always_inline)) {
        return __builtin_amdgcn_ballot_w64(!(l_row <= kMaxL)) != 0;
    };

    // The two roles run separate code from here on (so that each keeps only
    // its own registers live), with the same sequence of barriers:
    //   pass: prologue barrier, [tile-0 reference: one barrier], the barrier
    //   after P(0), then one barrier per tile T < n_tiles - 1;
    //   stats: two; if some row needs exact maxima: the max pass (prologue,
    //   one per tile), one, the pass again, stats again.
    // Per tile T the score waves compute the scores of tile T + 1, write its
    // P and copy tile T + 3 while the value waves run P·V of tile T; on each
    // SIMD one wave of each kind, so the MFMAs of the two overlap.
    if (sw) {
        // ================= score waves =================
        // K fragment addresses: key row r = 16 kh + l16, chunk 4 ks + kg.
        // With s = the row's swizzle, (4 ks + kg) ^ s = 4 (ks ^ s/4) +
        // (kg ^ s%4), and s/4 < 2 only flips ks's low bit: fragment 2 j + b
        // is at kb_b + 128 j.
        uint32_t kb[2];
        {
            const int r = 16 * kh + l16;
            const int t = (r >> 1) & 7, s = t ^ ((t & 1) << 2);
            const uint32_t base = (uint32_t)(uintptr_t)(lds_void *)lds + (uint32_t)(r * C::KROW_B + 16 * (kg ^ (s & 3)));
            kb[0] = base + 64 * (0 ^ (s >> 2));
            kb[1] = base + 64 * (1 ^ (s >> 2));
        }
        uint32_t koff[C::KWIN_W];  // this wave's byte offsets of its copies in a tile
        copy_offsets(koff);
        // Q of the block's 16 rows (B operands), loaded at the start of each
        // pass so that it is live in this role's code only
        bf16x8 qf[C::NKS];
        auto load_q = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) {
                u32x4 v = {0, 0, 0, 0};
                if (srow < a.Nq) v = load8_bf16(Qp + (int64_t)srow * a.q_sn + 32 * ks + 8 * kg);
                qf[ks] = u32x4_as_bf16x8(v);
            }
        };
        float m = 0.f;  // reference of row srow (score*c units), same in both key halves
        float l = 0.f;  // normalizer of row srow over this lane's keys
        auto kreads0 = [&](int stage) __attribute__((always_inline)) {
            const uint32_t so = stage * C::KTILE_B;
            wide_vk_kreads0(kb[0] + so, kb[1] + so);
        };
        // the score block of tile T (its first K fragment reads issued), masked
        // with Tc >= 0 this wave's share of the copy of tile Tc (into its
        // stage) goes between the MFMAs
        auto scores = [&](int T, int stage, float (&sv)[4], int Tc) __attribute__((always_inline)) {
            const uint32_t so = stage * C::KTILE_B;
            f32x4 sacc;
            if (Tc >= 0) {
                const u32x4 rk = tile_rsrc(Tc);
                const uint32_t mb = __builtin_amdgcn_readfirstlane(
                    lds_addr(lds + (Tc & 3) * C::KTILE_B + cm * 1024));
                perturb_pause();
                sacc = wide_vk_qk_copy(qf, kb[0] + so, kb[1] + so, koff, rk, mb);
            } else {
                sacc = wide_vk_qk(qf, kb[0] + so, kb[1] + so);
            }
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
        // maximum of this lane's block row over the 4 lanes that share it
        auto block_row_max = [&](const float (&sv)[4]) __attribute__((always_inline)) {
            float x = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            x = fmaxf(x, __shfl_xor(x, 16));
            x = fmaxf(x, __shfl_xor(x, 32));
            return x;
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
        auto pass = [&](bool set_m) __attribute__((always_inline)) {
            l = 0.f;
            load_q();
            prologue(koff, true);
            kreads0(0);
            {
                float sv[4];
                scores(0, 0, sv, -1);
                if (set_m) {
                    // reference: the row maximum over tile 0
                    const float mx = combine_halves(block_row_max(sv), true) * a.c;
                    m = (mx == -INFINITY) ? 0.f : mx;
                }
                block_p(0, sv);
                lds_barrier();  // P(0) written; tile 1 landed in the prologue
            }
            for (int T = 0; T + 1 < n_tiles; ++T) {
                float sv[4];
                kreads0((T + 1) & 3);
                // this pair's copy of tile T + 3 rides on the score block
                const bool copies = T + 3 < n_tiles && ((T + 3) & 1) == cpair;
                scores(T + 1, (T + 1) & 3, sv, copies ? T + 3 : -1);
                block_p(T + 1, sv);
                copy_barrier(T + 2);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no copy outlives the pass
        };
        // exact row maxima (in score*c units), no P·V; one barrier per tile
        auto max_pass = [&]() __attribute__((always_inline)) {
            float M = -INFINITY;
            load_q();
            prologue(koff, true);
            kreads0(0);
            for (int T = 0; T < n_tiles; ++T) {
                float sv[4];
                scores(T, T & 3, sv, -1);
                M = fmaxf(M, block_row_max(sv) * a.c);
                if (T + 3 < n_tiles) dma_tile(koff, T + 3, (T + 3) & 3);
                copy_barrier(T + 1);
                if (T + 1 < n_tiles) kreads0((T + 1) & 3);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            return M;
        };
        pass(true);
        float l_row, m_row;
        finish_stats(l, m, l_row, m_row);
        if (needs_exact(l_row)) {
            float M = max_pass();
            __syncthreads();
            M = combine_halves(M, true);
            m = (M == -INFINITY) ? 0.f : M;
            pass(false);
            finish_stats(l, m, l_row, m_row);
        }
    } else {
        // ================= value waves =================
        const uint32_t koff[C::KWIN_W] = {};
        // Vᵀ fragments (value columns 32 db .. 32 db + 31, db = 4 vw + i, keys
        // 16 kc .. 16 kc + 15): two transposed reads (key halves hr) of the K
        // tile, whose rows begin with the values. Lane (4 g + i16 / 4 + 8 hr +
        // 16 kc, column 32 db + 16 (G % 2) + 4 (i16 % 4)) reads 4 values; the
        // row's swizzle does not depend on kc, so (i, kc, hr) is at
        // vtb[hr][i] + 16 rows (kc).
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
        f32x16 oacc[CBW];
        // O += P·V of tile T: P from its buffer, V from its stage
        auto pv_tile = [&](int T) __attribute__((always_inline)) {
            const unsigned char *pb = lds + C::POFF + (T & 1) * C::PBUF_B;
            const uint32_t stage_off = (T & 3) * C::KTILE_B;
            bf16x8 pf[2], vf[2][CBW];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) pf[kc] = *(const bf16x8 *)(pb + p_rd + 32 * kc);
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int i = 0; i < CBW; ++i) vf[kc][i] = vt_frag_k(stage_off, i, kc);
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int i = 0; i < CBW; ++i) oacc[i] = mfma_32x32x16(vf[kc][i], pf[kc], oacc[i]);
        };
        auto pass = [&](bool set_m) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < CBW; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
            prologue(koff, false);
            if (set_m) combine_halves(0.f, true);  // the score waves' reference barrier
            lds_barrier();                         // P(0) written
            for (int T = 0; T < n_tiles; ++T) {
                pv_tile(T);
                if (T + 1 < n_tiles) lds_barrier();
            }
        };
        auto max_pass = [&]() __attribute__((always_inline)) {
            prologue(koff, false);
            for (int T = 0; T < n_tiles; ++T) lds_barrier();
        };
        pass(true);
        float l_row, m_row;
        finish_stats(0.f, 0.f, l_row, m_row);
        if (needs_exact(l_row)) {
            max_pass();
            __syncthreads();
            combine_halves(0.f, true);
            pass(false);
            finish_stats(0.f, 0.f, l_row, m_row);
        }

        // ---- O = Oᵀ / l (one reciprocal per row), logsumexp -----------------
        // Through LDS (every copy has landed and every wave is past the
        // statistics' barriers; the staged blocks end below the P buffers):
        // each lane writes its row's runs of four columns to this wave's
        // block, then each store covers four rows' 256 contiguous bytes
        // instead of 8 bytes in each of 32 rows. Rows are unpadded: a run's
        // 16-byte chunk is XORed with row bits 0..3 and its 8-byte half with
        // row bit 4, so the 32 lanes of a write pass reach every bank once.
        const float inv_l = 1.0f / l_row;
        constexpr int SRB = 2 * 32 * CBW;
        static_assert((C::NWAVE - C::NSW) * C::TQ * SRB <= C::POFF, "the staged O stays in the K ring");
        static_assert(SRB == 256, "16 chunks a row");
        unsigned char *const stg = lds + vw * C::TQ * SRB;
#pragma unroll
        for (int i = 0; i < CBW; ++i)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int ch = (4 * i + rr) ^ (l32 & 15), hf = g ^ ((l32 >> 4) & 1);
                *(u32x2 *)(stg + l32 * SRB + 16 * ch + 8 * hf) =
                    u32x2{pack_bf16x2(oacc[i][4 * rr] * inv_l, oacc[i][4 * rr + 1] * inv_l),
                          pack_bf16x2(oacc[i][4 * rr + 2] * inv_l, oacc[i][4 * rr + 3] * inv_l)};
            }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int rl = lane >> 4, cl = lane & 15;  // 16 lanes x 16 bytes per row
#pragma unroll
        for (int it = 0; it < C::TQ / 4; ++it) {
            const int r = 4 * it + rl;
            u32x4 v = *(const u32x4 *)(stg + r * SRB + 16 * (cl ^ (r & 15)));
            if ((r >> 4) & 1) v = u32x4{v[2], v[3], v[0], v[1]};
            if (q0 + r < a.Nq) *(u32x4 *)(Op + (int64_t)(q0 + r) * a.o_sn + 32 * CBW * vw + 8 * cl) = v;
        }
        if (row < a.Nq && vw == 0 && g == 0 && a.lse)
            a.lse[((int64_t)b * a.Hq + h) * a.Nq + row] = (m_row + log2f(l_row)) * 0.69314718055994531f;
    }
#endif
}

}  // namespace attn
