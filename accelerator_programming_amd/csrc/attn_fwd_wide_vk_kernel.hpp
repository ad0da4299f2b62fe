// Fused attention forward for wide heads whose values are the first d_v
// columns of the keys (d_qk = 576, d_v = 512: the latent-attention layout,
// one K/V head shared by every query head), with V given as that view of K.
//
// Same method as the other kernels (disjoint output tiles, "Distilling a 4.5
// hour CUDA talk", section 5; K/V streamed through LDS with the row softmax
// carried by a per-row reference and normalizer, section 7). What differs is
// how the 4 waves of a workgroup share the work of one 32-row query tile:
//  * The score tile Sᵀ = K·Qᵀ (32 keys x 32 rows, contraction over 576) is
//    split over the contraction: wave w multiplies its 144-wide slice of K
//    and Q (9 k-steps of v_mfma_f32_32x32x16_bf16; it holds only that slice
//    of Q in registers). The four partial tiles go through LDS and every wave
//    adds them up in the same order, so all waves hold the same scores, the
//    same reference and the same P without a second exchange.
//  * Wave w accumulates output columns 128w .. 128w + 127 (O = P·V split over
//    the value columns), reading its Vᵀ fragments from the K tile.
//  So no MFMA work is repeated across waves (a wave does 9 + 8 MFMAs per
//  tile), and each K tile is staged into LDS once and read once for S and
//  once for V.
//  * K tiles (32 keys x 1152 bytes) sit in a three-stage LDS ring, filled
//    through registers: each wave loads its quarter of tile T + 4 after it has
//    written tile T + 2, which leaves two tiles of time for the global loads.
//    One barrier per tile: the partial scores of tile T are written to a
//    double-buffered exchange area before it, read after it; a stage is
//    rewritten only after every wave has passed the next tile's barrier.
//  * K rows are 72 16-byte chunks. Chunk c of row r is stored at
//    c ^ s(r), s(r) = t ^ 4 (t & 1), t = (r / 2) % 8: the 16 rows of a
//    fragment read (ds_read_b128) fall in 16 distinct bank groups, and so do
//    the 4 x 4 row/column pieces of a transposed Vᵀ read (ds_read_b64_tr_b16).
//  * The 9 K fragment reads of a tile's partial scores are issued right after
//    the previous tile's barrier, into registers the compiler does not
//    allocate (v220 .. v255), so their latency overlaps that tile's softmax
//    and P·V; the 9 MFMAs are one assembly block that waits for each read in
//    turn. (Left to itself the compiler issues each read right before its
//    MFMA.)
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
    static constexpr int NSTAGE = 3;
    static constexpr int XPART_B = 64 * 16 * 4;       // one wave's 32x32 fp32 partial
    static constexpr int XBUF_B = NWAVE * XPART_B;    // one exchange buffer
    static constexpr int XOFF = NSTAGE * KTILE_B;     // exchange buffers after the ring
    static constexpr int LDS_BYTES = XOFF + 2 * XBUF_B;
    static constexpr int KWIN_W = KTILE_B / 1024 / NWAVE;  // 1 KB pieces per wave per tile
    static constexpr int NKC = DQK / 16;                   // k-steps of Sᵀ = K·Qᵀ
    static constexpr int KCW = NKC / NWAVE;                // k-steps per wave
    static constexpr int CBW = DV / 32 / NWAVE;            // 32-column blocks of O per wave
    static_assert(KTILE_B % (1024 * NWAVE) == 0, "tile pieces must split over the waves");
    static_assert(NKC % NWAVE == 0, "the contraction must split over the waves");
    static_assert(NKC / NWAVE == 9, "the partial-score block is written for 9 k-steps");
    static_assert(KCH % 8 == 0, "the swizzle permutes aligned groups of 8 chunks");
    static_assert(DV % (32 * NWAVE) == 0 && DV <= DQK, "value columns");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Physical chunk of logical chunk c in K row r (an involution in c).
__device__ __forceinline__ int wide_vk_chunk(int r, int c) {
    const int t = (r >> 1) & 7;
    return c ^ (t ^ ((t & 1) << 2));
}

// ---- the partial-score block ----------------------------------------------
// Nine K fragments (k-steps 4j + w, j = 0..8, of this wave w) sit in
// v[220:255], fragment j in v[220 + 4j : 223 + 4j]. They are read by
// wide_vk_kreads from kb + 128 j (kb: this lane's fragment address in the
// stage for k-step w) and consumed by wide_vk_qk, which waits for read j
// with lgkmcnt(8 - j): LDS operations finish in order, so later LDS traffic
// only makes that wait stricter. The block ends with enough wait states for
// VALU, LDS or memory reads of the accumulator (the compiler does not see
// the MFMA latency through an asm statement).
#define WIDE_VK_S(x) #x
#define WIDE_VK_STR(x) WIDE_VK_S(x)
#define WIDE_VK_KREAD(J, R0, R1) "ds_read_b128 v[" WIDE_VK_STR(R0) ":" WIDE_VK_STR(R1) "], %[kb] offset:" WIDE_VK_STR(J) "*128\n\t"
#define WIDE_VK_CLOBBERS                                                                              \
    "v220", "v221", "v222", "v223", "v224", "v225", "v226", "v227", "v228", "v229", "v230", "v231", \
        "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", "v242",     \
        "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253",     \
        "v254", "v255"

__device__ __forceinline__ void wide_vk_kreads(uint32_t kb) {
    asm volatile(WIDE_VK_KREAD(0, 220, 223) WIDE_VK_KREAD(1, 224, 227) WIDE_VK_KREAD(2, 228, 231)
                 WIDE_VK_KREAD(3, 232, 235) WIDE_VK_KREAD(4, 236, 239) WIDE_VK_KREAD(5, 240, 243)
                 WIDE_VK_KREAD(6, 244, 247) WIDE_VK_KREAD(7, 248, 251) WIDE_VK_KREAD(8, 252, 255)
                 :
                 : [kb] "v"(kb)
                 : WIDE_VK_CLOBBERS, "memory");
}

#define WIDE_VK_STEP(WAIT, R0, R1, Q, C) \
    "s_waitcnt lgkmcnt(" WIDE_VK_STR(WAIT) ")\n\t" \
    "v_mfma_f32_32x32x16_bf16 %[sp], v[" WIDE_VK_STR(R0) ":" WIDE_VK_STR(R1) "], %[" Q "], " C "\n\t"

__device__ __forceinline__ f32x16 wide_vk_qk(const bf16x8 (&q)[9]) {
    f32x16 sp;
    asm volatile(WIDE_VK_STEP(8, 220, 223, "q0", "0") WIDE_VK_STEP(7, 224, 227, "q1", "%[sp]")
                 WIDE_VK_STEP(6, 228, 231, "q2", "%[sp]") WIDE_VK_STEP(5, 232, 235, "q3", "%[sp]")
                 WIDE_VK_STEP(4, 236, 239, "q4", "%[sp]") WIDE_VK_STEP(3, 240, 243, "q5", "%[sp]")
                 WIDE_VK_STEP(2, 244, 247, "q6", "%[sp]") WIDE_VK_STEP(1, 248, 251, "q7", "%[sp]")
                 WIDE_VK_STEP(0, 252, 255, "q8", "%[sp]")
                 "s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : [sp] "=&a"(sp)
                 : [q0] "v"(q[0]), [q1] "v"(q[1]), [q2] "v"(q[2]), [q3] "v"(q[3]), [q4] "v"(q[4]),
                   [q5] "v"(q[5]), [q6] "v"(q[6]), [q7] "v"(q[7]), [q8] "v"(q[8])
                 : "memory");
    return sp;
}

template <int DQK, int DV, bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
__attribute__((amdgpu_num_vgpr(220)))  // v220 .. v255: the K fragments of the asm blocks
attn_fwd_wide_vk_kernel(const KernelArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    using C = WideVkCfg<DQK, DV>;
    constexpr int TK = C::TK, KCW = C::KCW, CBW = C::CBW;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;

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
    const int row = q0 + l32;  // this lane's query row
    const int kv_end = CAUSAL ? min(a.Nkv, q0 + C::TQ) : a.Nkv;
    const int n_tiles = (kv_end + TK - 1) / TK;  // >= 1
    // tiles from this index on need the causal or key-range mask
    const int first_masked = CAUSAL ? min(q0 / TK, a.Nkv / TK) : a.Nkv / TK;

    // ---- Q at this wave's k-steps 4j + w (B operands), resident throughout ---
    bf16x8 qf[KCW];
#pragma unroll
    for (int j = 0; j < KCW; ++j) {
        u32x4 v = {0, 0, 0, 0};
        if (row < a.Nq) v = load8_bf16(Qp + (int64_t)row * a.q_sn + 16 * (C::NWAVE * j + w) + 8 * g);
        qf[j] = u32x4_as_bf16x8(v);
    }

    // ---- K staging: piece u of wave w is the 1 KB at (4u + w) KB of the tile;
    // lane i moves its 16-byte unit 64 (4u + w) + i, which holds the logical
    // chunk the swizzle puts there. Rows past the last key repeat the last
    // key (finite values, masked). -----------------------------------------
    auto load_tile = [&](int T, u32x4 (&kr)[C::KWIN_W]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < C::KWIN_W; ++u) {
            const int p = (C::NWAVE * u + w) * 64 + lane;
            const int r = p / C::KCH, c = wide_vk_chunk(r, p % C::KCH);
            const int key = min(T * TK + r, a.Nkv - 1);
            kr[u] = load8_bf16(Kp + (int64_t)key * a.k_sn + 8 * c);
        }
    };
    auto store_tile = [&](int stage, const u32x4 (&kr)[C::KWIN_W]) __attribute__((always_inline)) {
        unsigned char *st = lds + stage * C::KTILE_B;
#pragma unroll
        for (int u = 0; u < C::KWIN_W; ++u) *(u32x4 *)(st + (C::NWAVE * u + w) * 1024 + 16 * lane) = kr[u];
    };
    // this wave's LDS accesses are done, then every wave reaches this point;
    // global loads stay in flight (also a compiler memory barrier)
    auto lds_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    // ---- K fragment addresses: key row l32, chunk 2 kc + g. With s = the
    // row's swizzle, (2 kc + g) ^ s = 2 (kc ^ s/2) + (g ^ s%2), and s/2 < 4
    // only touches kc's low two bits: four per-lane bases, + 128 (kc / 4). --
    // This wave's k-steps are 4j + w: the fragment of k-step 4j + w is at
    // kb0 + 128 j (+ the stage's offset). --------------------------------------
    uint32_t kb0;
    {
        const int t = (l32 >> 1) & 7, s = t ^ ((t & 1) << 2);
        kb0 = (uint32_t)(uintptr_t)(lds_void *)lds +
              (uint32_t)(l32 * C::KROW_B + 16 * (g ^ (s & 1)) + 32 * (w ^ (s >> 1)));
    }

    // ---- state -------------------------------------------------------------
    f32x16 oacc[CBW];
    float m = 0.f;  // per-row reference (score*c units), same in all waves
    float l;        // normalizer, partial over this lane half

    // write the partial, barrier, add the four partials in wave order (the
    // same sum in every wave)
    auto exchange = [&](const f32x16 &sp, int T, f32x16 &s) __attribute__((always_inline)) {
        unsigned char *xb = lds + C::XOFF + (T & 1) * C::XBUF_B;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *(f32x4 *)(xb + w * C::XPART_B + j * 1024 + 16 * lane) =
                f32x4{sp[4 * j], sp[4 * j + 1], sp[4 * j + 2], sp[4 * j + 3]};
        lds_barrier();
        // all four partials, this wave's included, in one batch of reads
        f32x4 x[C::NWAVE][4];
#pragma unroll
        for (int v = 0; v < C::NWAVE; ++v)
#pragma unroll
            for (int j = 0; j < 4; ++j) x[v][j] = *(const f32x4 *)(xb + v * C::XPART_B + j * 1024 + 16 * lane);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[4 * j + e] = ((x[0][j][e] + x[1][j][e]) + x[2][j][e]) + x[3][j][e];
    };
    auto masked_scores = [&](bool masked, const f32x16 &sacc, float (&sv)[16], int T)
                             __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = sacc[r];
        if (masked) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = T * TK + acc_row(r, g);
                if ((CAUSAL && key > row) || key >= a.Nkv) sv[r] = -INFINITY;
            }
        }
    };
    auto row_max = [&](const float (&sv)[16]) __attribute__((always_inline)) {
        float x = fmaxf(sv[0], sv[1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) x = fmaxf(x, fmaxf(sv[r], sv[r + 1]));
        return xhalf_max(x) * a.c;
    };
    // Vᵀ fragment (32 value columns from 32 db, keys 16 kc .. 16 kc + 15):
    // transposed reads of the K tile, whose rows begin with the values
    auto vt_frag_k = [&](const __bf16 *Ks, int db, int kc) __attribute__((always_inline)) {
        const int G = lane >> 4, i16 = lane & 15;
        i16x4 hv[2];
#pragma unroll
        for (int hr = 0; hr < 2; ++hr) {
            const int vr = 16 * kc + 8 * hr + 4 * g + (i16 >> 2);
            const int col = 32 * db + 16 * (G & 1) + 4 * (i16 & 3);
            const __bf16 *src = Ks + vr * DQK + 8 * wide_vk_chunk(vr, col >> 3) + (col & 7);
            hv[hr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(src));
        }
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto pv = [&](const uint32_t (&pk)[8], int stage) __attribute__((always_inline)) {
        const __bf16 *Ks = (const __bf16 *)(lds + stage * C::KTILE_B);
        bf16x8 vf[2][CBW];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int i = 0; i < CBW; ++i) vf[kc][i] = vt_frag_k(Ks, CBW * w + i, kc);
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const bf16x8 pf = u32x4_as_bf16x8(u32x4{pk[4 * kc], pk[4 * kc + 1], pk[4 * kc + 2], pk[4 * kc + 3]});
#pragma unroll
            for (int i = 0; i < CBW; ++i) oacc[i] = mfma_32x32x16(vf[kc][i], pf, oacc[i]);
        }
    };

    // ---- one pass over the keys ---------------------------------------------
    // mode 0: reference from the first tile, then O and l;
    // mode 1: O and l for the given reference m;
    // mode 2: exact row maxima only (returned)
    u32x4 kr0[C::KWIN_W], kr1[C::KWIN_W];
    auto pass = [&](int mode) __attribute__((always_inline)) {
        float M = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int i = 0; i < CBW; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
        __syncthreads();  // the ring and the exchange buffers are free
        load_tile(0, kr0);
        if (n_tiles > 1) load_tile(1, kr1);
        store_tile(0, kr0);
        if (n_tiles > 1) store_tile(1, kr1);
        if (n_tiles > 2) load_tile(2, kr0);
        if (n_tiles > 3) load_tile(3, kr1);
        lds_barrier();
        wide_vk_kreads(kb0);  // tile 0, stage 0

        // tile T reads stage T % 3; at its end this wave writes tile T + 2
        // (held in kr[T % 2]) into stage (T + 2) % 3, the stage of tile T - 1,
        // which every wave finished before this tile's barrier, then loads
        // tile T + 4 into the same registers
        auto tile = [&](int T, int stage, u32x4 (&kr)[C::KWIN_W]) __attribute__((always_inline)) {
            f32x16 s;
            const f32x16 sp = wide_vk_qk(qf);
            exchange(sp, T, s);
            // tile T + 1 was written before this barrier
            if (T + 1 < n_tiles) wide_vk_kreads(kb0 + (stage == 2 ? 0 : (stage + 1) * C::KTILE_B));
            float sv[16];
            masked_scores(T >= first_masked, s, sv, T);
            if (mode == 2) {
                M = fmaxf(M, row_max(sv));
            } else {
                if (mode == 0 && T == 0) {
                    const float mx = row_max(sv);
                    m = (mx == -INFINITY) ? 0.f : mx;
                }
                const float negm = -m;
                uint32_t pk[8];
                float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float e0 = exp2_hw(fmaf(sv[2 * j], a.c, negm));
                    const float e1 = exp2_hw(fmaf(sv[2 * j + 1], a.c, negm));
                    pk[j] = pack_bf16x2(e0, e1);
                    ls[j & 3] = sum_bf16x2(pk[j], ls[j & 3]);
                }
                l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
                pv(pk, stage);
            }
            if (T + 2 < n_tiles) {
                store_tile(stage == 0 ? 2 : stage - 1, kr);
                if (T + 4 < n_tiles) load_tile(T + 4, kr);
            }
        };
        int stage = 0;
        for (int T = 0; T < n_tiles; T += 2) {
            tile(T, stage, kr0);
            stage = stage == 2 ? 0 : stage + 1;
            if (T + 1 < n_tiles) {
                tile(T + 1, stage, kr1);
                stage = stage == 2 ? 0 : stage + 1;
            }
        }
        return M;
    };

    constexpr float kMaxL = 4294967296.0f;  // 2^32: every p <= 2^32 when l <= 2^32
    pass(0);
    float l_row = xhalf_sum(l);
    // every wave holds the same rows' normalizers; decide once for the group
    __shared__ int wave_bad[C::NWAVE];
    if (lane == 0) wave_bad[w] = __builtin_amdgcn_ballot_w64(!(l_row <= kMaxL)) != 0;
    __syncthreads();
    bool wg_bad = false;
#pragma unroll
    for (int i = 0; i < C::NWAVE; ++i) wg_bad |= wave_bad[i] != 0;
    if (wg_bad) {
        // exact row maxima, then the pass again (rare)
        const float M = pass(2);
        m = (M == -INFINITY) ? 0.f : M;
        pass(1);
        l_row = xhalf_sum(l);
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
            a.lse[((int64_t)b * a.Hq + h) * a.Nq + row] = (m + log2f(l_row)) * 0.69314718055994531f;
    }
#endif
}

}  // namespace attn
