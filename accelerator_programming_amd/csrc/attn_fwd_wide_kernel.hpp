// Fused attention forward for wide heads (d_qk = 576, d_v = 512, the
// latent-attention shape: one shared K/V head, values a prefix of the keys).
//
// Same method as the main kernel (disjoint output tiles, "Distilling a 4.5
// hour CUDA talk", section 5; streaming K/V through LDS with the row softmax
// carried by a per-row reference and normalizer, section 7), laid out for a
// head too wide to keep a 64-row output tile in one wave:
//  * A workgroup owns TQ = 32 query rows of one (batch, head); 4 waves, one
//    per SIMD. Wave w accumulates output columns 128w .. 128w + 127
//    (4 blocks of 32x32 fp32 = 64 VGPRs) and holds the rows' whole Q slab
//    (32 x 576 bf16 = 144 VGPRs) as MFMA B operands.
//  * Each wave computes the full 32-key x 32-row score tile itself
//    (Sᵀ = K·Qᵀ, 36 k-steps of v_mfma_f32_32x32x16_bf16), so the softmax and
//    P stay in registers and no wave waits for another's scores.
//  * K/V tiles of 32 keys stream through a two-stage LDS ring by LDS-DMA
//    (buffer_load ... lds through a resource that ends at the last key, so
//    rows past it read as zeros). K rows are 72 16-byte chunks: the chunk
//    XOR (r / 2) % 8 stays inside each aligned group of 8 chunks and makes
//    the 16 rows of a fragment read land in 16 distinct bank groups. V rows
//    are 64 chunks with the main kernel's V swizzle (XOR < 16).
//  * Softmax in base 2 with the per-row reference fixed by the first 32
//    keys, exact O = acc / l and lse, and a slow pass with exact row maxima
//    when some row's normalizer leaves [0, 2^32] (as in the main kernel).
#pragma once

#include "tile.hpp"

namespace attn {

template <int DQK, int DV>
struct WideCfg {
    static constexpr int TQ = 32;  // query rows per workgroup
    static constexpr int TK = 32;  // keys per tile
    static constexpr int NWAVE = 4;
    static constexpr int NT = 64 * NWAVE;
    static constexpr int KCH = DQK / 8, VCH = DV / 8;  // 16-byte chunks per row
    static constexpr int KROW_B = 2 * DQK, VROW_B = 2 * DV;
    static constexpr int KTILE_B = TK * KROW_B, VTILE_B = TK * VROW_B;
    static constexpr int STAGE_B = KTILE_B + VTILE_B;
    static constexpr int LDS_BYTES = 2 * STAGE_B;
    static constexpr int KWIN_W = KTILE_B / 1024 / NWAVE;  // 1 KB DMA windows per wave
    static constexpr int VWIN_W = VTILE_B / 1024 / NWAVE;
    static constexpr int NKC = DQK / 16;        // k-steps of Sᵀ = K·Qᵀ
    static constexpr int CBW = DV / 32 / NWAVE;  // 32-column blocks of O per wave
    static_assert(KTILE_B % (1024 * NWAVE) == 0 && VTILE_B % (1024 * NWAVE) == 0,
                  "tile windows must split over the waves");
    static_assert(KCH % 8 == 0, "the K swizzle permutes aligned groups of 8 chunks");
    static_assert(VCH == 64, "one V row per DMA window");
    static_assert(NKC % 4 == 0, "K fragment addresses repeat every 4 k-steps");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Physical chunk of logical chunk c in K row r (an involution).
__device__ __forceinline__ int wide_k_chunk(int r, int c) { return c ^ ((r >> 1) & 7); }

template <int DQK, int DV, bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_fwd_wide_kernel(const KernelArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    using C = WideCfg<DQK, DV>;
    constexpr int TQ = C::TQ, TK = C::TK, NKC = C::NKC, CBW = C::CBW;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;

    // ---- work item ----------------------------------------------------------
    const int BH = a.B * a.Hq;
    const uint32_t wid = work_index(blockIdx.x, gridDim.x);
    const int bh = wid % BH;
    int qt = wid / BH;
    if (CAUSAL) qt = a.n_qtiles - 1 - qt;
    const int b = bh / a.Hq, h = bh % a.Hq, hk = h / a.group;
    const __bf16 *__restrict__ Qp = (const __bf16 *)a.q + b * a.q_sb + h * a.q_sh;
    const __bf16 *__restrict__ Kp = (const __bf16 *)a.k + b * a.k_sb + hk * a.k_sh;
    const __bf16 *__restrict__ Vp = (const __bf16 *)a.v + b * a.v_sb + hk * a.v_sh;
    __bf16 *__restrict__ Op = (__bf16 *)a.o + b * a.o_sb + h * a.o_sh;

    const int q0 = qt * TQ;
    const int row = q0 + l32;  // this lane's query row
    const int kv_end = CAUSAL ? min(a.Nkv, q0 + TQ) : a.Nkv;
    const int n_tiles = (kv_end + TK - 1) / TK;  // >= 1
    // tiles from this index on need the causal or key-range mask
    const int first_masked = CAUSAL ? min(q0 / TK, a.Nkv / TK) : a.Nkv / TK;

    // ---- Q fragments (B operands), resident for the whole loop --------------
    bf16x8 qf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
        u32x4 v = {0, 0, 0, 0};
        if (row < a.Nq) v = load8_bf16(Qp + (int64_t)row * a.q_sn + 16 * kc + 8 * g);
        qf[kc] = u32x4_as_bf16x8(v);
    }

    // ---- LDS-DMA: wave w fills the 1 KB windows w, w + 4, ... of each tile;
    // lane i of a window lands at 16-byte unit 64 win + i of the tile and
    // fetches the logical chunk the swizzle puts there. The byte offsets
    // inside a tile are the same for every tile. ---------------------------
    uint32_t koff[C::KWIN_W], voff[C::VWIN_W];
#pragma unroll
    for (int u = 0; u < C::KWIN_W; ++u) {
        const int p = (C::NWAVE * u + w) * 64 + lane;
        const int r = p / C::KCH, c = wide_k_chunk(r, p % C::KCH);
        const int64_t off = ((int64_t)r * a.k_sn + 8 * c) * 2;
        koff[u] = off < 0xFFFFFFF0ll ? (uint32_t)off : 0xFFFFFFF0u;
    }
#pragma unroll
    for (int u = 0; u < C::VWIN_W; ++u) {
        const int r = C::NWAVE * u + w;  // one row per window
        const int c = v_chunk<DV>(r, lane);
        const int64_t off = ((int64_t)r * a.v_sn + 8 * c) * 2;
        voff[u] = off < 0xFFFFFFF0ll ? (uint32_t)off : 0xFFFFFFF0u;
    }
    auto issue = [&](int T, int stage) __attribute__((always_inline)) {
        const int rem = a.Nkv - T * TK;  // keys left, >= 1
        const u32x4 rk = buffer_rsrc(Kp + (int64_t)T * TK * a.k_sn,
                                     (uint32_t)(((int64_t)(rem - 1) * a.k_sn + DQK) * 2));
        const u32x4 rv = buffer_rsrc(Vp + (int64_t)T * TK * a.v_sn,
                                     (uint32_t)(((int64_t)(rem - 1) * a.v_sn + DV) * 2));
        unsigned char *st = lds + stage * C::STAGE_B;
        perturb_pause();
#pragma unroll
        for (int u = 0; u < C::KWIN_W; ++u) dma16_buf_to_lds(rk, koff[u], st + (C::NWAVE * u + w) * 1024);
#pragma unroll
        for (int u = 0; u < C::VWIN_W; ++u)
            dma16_buf_to_lds(rv, voff[u], st + C::KTILE_B + (C::NWAVE * u + w) * 1024);
    };

    // ---- K fragment addresses: key row l32, chunk 2 kc + g. With s = the
    // row's swizzle, (2 kc + g) ^ s = 2 (kc ^ s/2) + (g ^ s%2), and s/2 < 4
    // only touches kc's low two bits: four per-lane bases, + 128 (kc / 4). --
    uint32_t kaddr[4];
    {
        const int s = (l32 >> 1) & 7;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            kaddr[j] = (uint32_t)(l32 * C::KROW_B + 16 * (g ^ (s & 1)) + 32 * (j ^ (s >> 1)));
    }

    // ---- state -------------------------------------------------------------
    f32x16 oacc[CBW];
    float m = 0.f;  // per-row reference (score*c units), same in all waves
    float l;        // normalizer, partial over this lane half

    auto scores = [&](f32x16 &sacc, int stage) __attribute__((always_inline)) {
        const unsigned char *ks = lds + stage * C::STAGE_B;
        auto kread = [&](int kc) __attribute__((always_inline)) {
            return *(const bf16x8 *)(ks + kaddr[kc & 3] + 128 * (kc >> 2));
        };
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
        bf16x8 kf[NKC];
        kf[0] = kread(0);
        kf[1] = kread(1);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            if (kc + 2 < NKC) kf[kc + 2] = kread(kc + 2);
            sacc = mfma_32x32x16(kf[kc], qf[kc], sacc);
            asm volatile("" ::);  // keeps the reads two steps ahead, not all hoisted
        }
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
    auto pv = [&](const uint32_t (&pk)[8], int stage) __attribute__((always_inline)) {
        const __bf16 *Vs = (const __bf16 *)(lds + stage * C::STAGE_B + C::KTILE_B);
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const bf16x8 pf = u32x4_as_bf16x8(u32x4{pk[4 * kc], pk[4 * kc + 1], pk[4 * kc + 2], pk[4 * kc + 3]});
            bf16x8 vf[CBW];
#pragma unroll
            for (int i = 0; i < CBW; ++i) vf[i] = vt_frag<DV>(Vs, CBW * w + i, kc, lane);
#pragma unroll
            for (int i = 0; i < CBW; ++i) oacc[i] = mfma_32x32x16(vf[i], pf, oacc[i]);
        }
    };

    // ---- one pass over the keys: O, l for the reference m --------------------
    auto pass = [&](bool set_m) __attribute__((always_inline)) {
        l = 0.f;
#pragma unroll
        for (int i = 0; i < CBW; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
        issue(0, 0);
        __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
        __syncthreads();
        if (set_m) {
            f32x16 sacc;
            scores(sacc, 0);
            float sv[16];
            masked_scores(0 >= first_masked, sacc, sv, 0);
            const float mx = row_max(sv);
            m = (mx == -INFINITY) ? 0.f : mx;
        }
        for (int T = 0; T < n_tiles; ++T) {
            const int stage = T & 1;
            if (T + 1 < n_tiles) issue(T + 1, stage ^ 1);
            f32x16 sacc;
            scores(sacc, stage);
            float sv[16];
            masked_scores(T >= first_masked, sacc, sv, T);
            uint32_t pk[8];
            float ls = 0.f;
#pragma unroll
            for (int r = 0; r < 16; r += 2) exp_pair(sv[r], sv[r + 1], a.c, -m, ls, pk[r / 2]);
            l += ls;
            pv(pk, stage);
            __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's DMAs landed
            __syncthreads();
        }
    };

    constexpr float kMaxL = 4294967296.0f;  // 2^32: every p <= 2^32 when l <= 2^32
    pass(true);
    float l_row = xhalf_sum(l);
    // every wave holds the same rows' normalizers; decide once for the group
    __shared__ int wave_bad[C::NWAVE];
    // the ballot runs in every lane (inside `lane == 0` it would see lane 0's
    // row only); lane 0 then publishes the wave's verdict
    const bool any_bad = __builtin_amdgcn_ballot_w64(!(l_row <= kMaxL)) != 0;
    if (lane == 0) wave_bad[w] = any_bad;
    __syncthreads();
    bool wg_bad = false;
#pragma unroll
    for (int i = 0; i < C::NWAVE; ++i) wg_bad |= wave_bad[i] != 0;
    if (wg_bad) {
        // exact row maxima, then the pass again (rare)
        float M = -INFINITY;
        for (int T = 0; T < n_tiles; ++T) {
            __syncthreads();  // stage 0 is no longer read
            issue(T, 0);
            __builtin_amdgcn_s_waitcnt(0x3f70);
            __syncthreads();
            f32x16 sacc;
            scores(sacc, 0);
            float sv[16];
            masked_scores(true, sacc, sv, T);
            M = fmaxf(M, row_max(sv));
        }
        __syncthreads();
        m = (M == -INFINITY) ? 0.f : M;
        pass(false);
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
