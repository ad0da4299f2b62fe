// Fused attention forward kernel for gfx950.
//
// One workgroup owns one (batch, query head, tile of TQ = 256 query rows) and
// writes that tile of O and logsumexp; no workgroup talks to another: the
// disjoint-output-tile decomposition of "Distilling a 4.5 hour CUDA talk",
// section 5. Inside it, the FlashAttention-2 structure of the same page's
// section 7: the query tile stays in registers while K/V tiles stream through
// on-chip memory (LDS), and the row softmax is carried across key tiles with
// a per-row reference and a normalizer.
//
// gfx950 mapping
//  * 8 waves, two per SIMD. Waves p and p + 4 form a pair on SIMD p and share
//    query rows q0 + 64p .. q0 + 64p + 63 (two 32-row blocks). In each 64-key
//    tile, role r = 0 / 1 (wave p / p + 4) scores keys 32r .. 32r + 31 and
//    accumulates O columns 64r .. 64r + 63 (d = 128; half of d in general).
//    Every K or V fragment read from LDS feeds the MFMAs of both row blocks.
//  * Why pairs: on gfx950 a wave's VALU work does not overlap its own MFMAs,
//    while VALU and MFMA work of two waves on one SIMD do overlap. The two
//    roles run their period in different orders (role 0: P·V, scores,
//    softmax; role 1: scores, softmax, P·V), so each one's exponentials run
//    while the other's MFMAs execute: compute never idle, as the pages ask
//    ("CS149 L11: Programming Specialized Hardware", section 4, slide 35),
//    with the producer / consumer split of "Distilling a 4.5 hour CUDA talk",
//    section 12, becoming a score / value split between two waves.
//  * Scores are computed transposed, Sᵀ = K·Qᵀ, with 32x32x16 bf16 MFMAs:
//    A = a 32-key slab of K read from LDS, B = the block's Q fragment held in
//    VGPRs for the whole loop. In the accumulator every lane holds one query
//    row (l % 32) and 16 keys, so the softmax row work is in-lane.
//  * Oᵀ += Vᵀ·Pᵀ: Pᵀ is the score accumulator converted to bf16 in place. The
//    keys a lane holds come in runs of four (rows 8*(r/4) + 4g + r%4), so the
//    MFMA k index 8g + e names key 8*(e/4) + 4g + e%4 of each 16-key chunk.
//    The Vᵀ operand is read from the row-major V tile with the LDS transpose
//    read (ds_read_b64_tr_b16) in exactly that key order. Each role writes its
//    P to LDS in register order; both roles read both halves back.
//  * Softmax in base 2 with log2(e) folded into the scale on the host, and
//    one reciprocal per row at the end ("Distilling a 4.5 hour CUDA talk",
//    section 2 on the base-2 exponential and on reciprocal reuse; section 7
//    on folding log2(e) into the temperature). Each row's exponent reference
//    m is fixed from its first 32 keys: O = acc / l and lse = m + log2 l are
//    exact in real arithmetic for any m, so nothing is rescaled in the loop.
//    If some row's l leaves [0, 2^32] (a later key outscored the first ones by
//    a wide margin) the workgroup recomputes with exact row maxima.
//  * K/V staging: role-1 waves are also the loaders: they issue LDS-DMA
//    (global_load_lds_dwordx4, no VGPRs) for K(T+1) and V(T) at the start of
//    period T into two-stage rings; "my loads landed" (s_waitcnt vmcnt(0))
//    plus one barrier close each period. LDS-DMA writes 16 bytes per lane at
//    consecutive addresses, so bank-conflict avoidance is an XOR swizzle of the
//    16-byte chunks of a row, applied by choosing which global chunk each lane
//    fetches ("Distilling a 4.5 hour CUDA talk", section 8).
#pragma once
#include <type_traits>

#include "tile.hpp"

namespace attn {

struct KernelArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int64_t q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;  // batch / head strides (elements)
    int32_t q_sn, k_sn, v_sn, o_sn;                          // row strides (elements)
    int32_t B, Hq, Hkv, Nq, Nkv, group;                      // group = Hq / Hkv
    int32_t n_qtiles;
    float c;         // softmax scale * log2(e)
    int32_t v_in_k;  // V is the first d_v columns of K's rows (same pointer and strides)
};

template <int D>
struct TileCfg {
    static constexpr int TQ = 256;          // query rows per workgroup
    static constexpr int TK = 64;           // keys per tile (one 32-key half per role)
    static constexpr int NWAVE = 8;
    static constexpr int NT = 64 * NWAVE;   // threads per workgroup
    static constexpr int CPR = D / 8;       // 16-byte chunks per K or V row
    static constexpr int TILE = TK * D;     // elements of one K or V tile
    static constexpr int P_BYTES = 4096;    // one wave's P: 64 rows x 32 keys bf16
    static constexpr int P_SLOT = NWAVE * P_BYTES;
    static constexpr int KV_BYTES = 4 * TILE * 2;  // two K stages, two V stages
    static constexpr int LDS_BYTES = KV_BYTES + 2 * P_SLOT;
    static constexpr int ROWS_PER_DMA = 64 / CPR;                 // rows per wave-wide DMA
    static constexpr int DMA_PER_LOADER = TK / ROWS_PER_DMA / 4;  // per tile, tensor and loader wave
    static constexpr int NKC = D / 16;      // k-steps of Sᵀ = K·Qᵀ
    static constexpr int NDB = D / 64;      // 32-column blocks of O per role
    static_assert(TK % (ROWS_PER_DMA * 4) == 0, "tile rows must split over the loader waves");
    static_assert(D % 64 == 0, "each role owns a multiple of 32 output columns");
};

template <int N>
using IC = std::integral_constant<int, N>;

template <int D, bool CAUSAL, typename TIn>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(const KernelArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    using C = TileCfg<D>;
    constexpr int TQ = C::TQ, TK = C::TK, CPR = C::CPR, NKC = C::NKC, NDB = C::NDB;
    constexpr int DPL = C::DMA_PER_LOADER;
    __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[C::LDS_BYTES];
    __bf16 *const Kst = (__bf16 *)lds_raw;             // two K stages
    __bf16 *const Vst = Kst + 2 * C::TILE;             // two V stages
    unsigned char *const Pst = lds_raw + C::KV_BYTES;  // two P slots

    const int tid = threadIdx.x;
    int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = w & 3, role = w >> 2;
    int l32 = lane & 31, g = lane >> 5;

    // ---- work item: heaviest causal tiles are dispatched first. Workgroups
    // go to the 8 XCDs round-robin by index; when the kv-head groups split
    // evenly over them, each XCD takes whole groups and runs the query heads
    // of a group on the same q-tile side by side, so they read the same K/V
    // tiles through that XCD's L2. ------------------------------------------
    int b, h, qt;
    {
        const int n_groups = a.B * a.Hkv;
        const int bid = blockIdx.x;
        if (n_groups % 8 == 0) {
            const int xcd = bid % 8, idx = bid / 8;
            const int per_round = (n_groups / 8) * a.group;  // WGs of one q-tile on one XCD
            const int qt_rank = idx / per_round, r = idx % per_round;
            const int grp = xcd + 8 * (r / a.group);
            b = grp / a.Hkv;
            h = (grp % a.Hkv) * a.group + r % a.group;
            qt = qt_rank;
        } else {
            const int BH = a.B * a.Hq;
            b = (bid % BH) / a.Hq;
            h = (bid % BH) % a.Hq;
            qt = bid / BH;
        }
        if (CAUSAL) qt = a.n_qtiles - 1 - qt;
    }
    const int hk = h / a.group;
    const TIn *__restrict__ Qp = (const TIn *)a.q + b * a.q_sb + h * a.q_sh;
    const TIn *__restrict__ Kp = (const TIn *)a.k + b * a.k_sb + hk * a.k_sh;
    const TIn *__restrict__ Vp = (const TIn *)a.v + b * a.v_sb + hk * a.v_sh;
    TIn *__restrict__ Op = (TIn *)a.o + b * a.o_sb + h * a.o_sh;

    const int q0 = qt * TQ;
    const int prow0 = q0 + 64 * pair;  // first query row of this pair
    const int kv_end = CAUSAL ? min(a.Nkv, q0 + TQ) : a.Nkv;
    const int n_tiles = (kv_end + TK - 1) / TK;  // >= 1
    // 32-key half-tiles from this index on need the causal or key-range mask;
    // tiles below n_plain have none
    const int first_masked_sub = CAUSAL ? min(q0 / 32, a.Nkv / 32) : a.Nkv / 32;
    const int n_plain = min(n_tiles, first_masked_sub / 2);

    // ---- Q fragments: B operands of Sᵀ = K·Qᵀ, resident for the whole loop --
    bf16x8 qf[2][NKC];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = prow0 + 32 * rb + l32;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            u32x4 v = {0, 0, 0, 0};
            if (row < a.Nq) v = load8_bf16(Qp + (int64_t)row * a.q_sn + 16 * kc + 8 * g);
            qf[rb][kc] = u32x4_as_bf16x8(v);
        }
    }

    // ---- LDS stages; PAR is the tile index parity (a compile-time constant
    // in the unrolled loop, so stage offsets are instruction immediates) ----
    auto kstage = [&](auto PAR) __attribute__((always_inline)) {
        return Kst + decltype(PAR)::value * C::TILE;
    };
    auto vstage = [&](auto PAR) __attribute__((always_inline)) {
        return Vst + decltype(PAR)::value * C::TILE;
    };
    // P of wave (pair, rl) for a tile of parity PAR, in register order:
    // 16-byte chunk j of lane l at byte 16 * (64 j + l), conflict-free
    auto pslot = [&](auto PAR, int rl) __attribute__((always_inline)) {
        return Pst + decltype(PAR)::value * C::P_SLOT + (pair + 4 * rl) * C::P_BYTES;
    };

    // ---- LDS-DMA of one K or V tile by the four loader (role-1) waves. A
    // window is 64 lanes x 16 bytes = ROWS_PER_DMA rows; loader `pair` fills
    // windows pair, pair + 4, ...; lane i of a window lands at chunk i and
    // fetches the global chunk that the swizzle puts there. bf16 inputs go
    // through a buffer resource that ends at the last key, so rows past the
    // end read as zeros (finite, and masked). -----------------------------
    int dma_r = lane / CPR;  // row within the window
    int dma_p = lane % CPR;  // physical chunk this lane fills
    auto issue = [&](auto PAR, bool is_v, int tile) __attribute__((always_inline)) {
        __bf16 *dst = is_v ? vstage(PAR) : kstage(PAR);
        const TIn *base = is_v ? Vp : Kp;
        const int32_t sn = is_v ? a.v_sn : a.k_sn;
        if constexpr (sizeof(TIn) == 2) {
            const int rem = a.Nkv - tile * TK;  // keys left, >= 1
            const uint32_t bytes = (uint32_t)(((int64_t)(rem - 1) * sn + D) * 2);
            const u32x4 rsrc = buffer_rsrc(base + (int64_t)tile * TK * sn, bytes);
#pragma unroll
            for (int u = 0; u < DPL; ++u) {
                const int win_id = 4 * u + pair;
                const int r = win_id * C::ROWS_PER_DMA + dma_r;  // tile row
                const int chunk = is_v ? v_chunk<D>(r, dma_p) : k_chunk<D>(r, dma_p);
                const int64_t off = ((int64_t)r * sn + 8 * chunk) * 2;
                const uint32_t voff = off < (int64_t)bytes ? (uint32_t)off : 0xFFFFFFF0u;
                dma16_buf_to_lds(rsrc, voff, dst + win_id * 64 * 8);
            }
        } else {
            // fp32 inputs: rounded to bf16 in registers, same LDS placement
#pragma unroll
            for (int u = 0; u < DPL; ++u) {
                const int win_id = 4 * u + pair;
                const int r = win_id * C::ROWS_PER_DMA + dma_r;
                const int key = min(tile * TK + r, a.Nkv - 1);  // clamped: a finite, masked row
                const int chunk = is_v ? v_chunk<D>(r, dma_p) : k_chunk<D>(r, dma_p);
                *(u32x4 *)(dst + win_id * 64 * 8 + 8 * lane) =
                    load8_bf16(base + (int64_t)key * sn + 8 * chunk);
            }
        }
    };

    // ---- state -------------------------------------------------------------
    f32x16 oacc[2][NDB];  // O columns 32 * (NDB * role + db) .. of both row blocks
    float m[2] = {0.f, 0.f};  // per-row reference of the exponentials (score*c units)
    float l[2];               // normalizer, partial over this wave's keys and lane half

    // Sᵀ of one 32-key half-tile (rows kq_row0.. of K stage Kq), both row blocks
    auto scores = [&](f32x16 (&sacc)[2], const __bf16 *Kq, int kq_row0)
                      __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[rb][r] = 0.f;
        bf16x8 kf[NKC];
        kf[0] = k_frag<D>(Kq, kq_row0 + l32, 0, g);
        kf[1] = k_frag<D>(Kq, kq_row0 + l32, 1, g);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            if (kc + 2 < NKC) kf[kc + 2] = k_frag<D>(Kq, kq_row0 + l32, kc + 2, g);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) sacc[rb] = mfma_32x32x16(kf[kc], qf[rb][kc], sacc[rb]);
            // a scheduling boundary: keeps the fragment reads two steps ahead
            // rather than all hoisted (registers are the limit in this kernel)
            asm volatile("" ::);
        }
    };
    // scores of half-tile js as floats, with the causal / key-range mask
    auto masked_scores = [&](bool masked, const f32x16 (&sacc)[2], float (&sv)[2][16], int js)
                             __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sv[rb][r] = sacc[rb][r];
        if (masked) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int row = prow0 + 32 * rb + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 32 * js + acc_row(r, g);
                    if ((CAUSAL && key > row) || key >= a.Nkv) sv[rb][r] = -INFINITY;
                }
            }
        }
    };
    // row maxima of score * c over a half-tile (both wave halves)
    auto row_max = [&](const float (&sv)[2][16], float (&mx)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            float x = fmaxf(sv[rb][0], sv[rb][1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) x = fmaxf(x, fmaxf(sv[rb][r], sv[rb][r + 1]));
            mx[rb] = xhalf_max(x) * a.c;
        }
    };
    // this wave's half of tile T: scores, p = 2^(s·c - m) (Map(exp)), the
    // partial row sums (Reduce(+)), P to LDS
    auto score_softmax = [&](auto ROLE, auto PAR, int T, bool masked) __attribute__((always_inline)) {
        constexpr int R = decltype(ROLE)::value;
        f32x16 sacc[2];
        scores(sacc, kstage(PAR), 32 * R);
        float sv[2][16];
        masked_scores(masked, sacc, sv, 2 * T + R);
        // p = 2^(s·c - m) rounded to bf16; the row sums add the rounded p
        // (what P·V multiplies) two at a time with v_dot2_f32_bf16, in
        // independent partial sums so no instruction waits on the previous
        uint32_t pk[2][8];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const float negm = -m[rb];
            float e[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) e[r] = exp2_hw(__builtin_fmaf(sv[rb][r], a.c, negm));
#pragma unroll
            for (int j = 0; j < 8; ++j) pk[rb][j] = pack_bf16x2(e[2 * j], e[2 * j + 1]);
            float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 8; ++j) ls[j & 3] = sum_bf16x2(pk[rb][j], ls[j & 3]);
            l[rb] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
        }
        unsigned char *dst = pslot(PAR, R);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                *(u32x4 *)(dst + 16 * (64 * (2 * rb + hh) + lane)) =
                    u32x4{pk[rb][4 * hh], pk[rb][4 * hh + 1], pk[rb][4 * hh + 2], pk[rb][4 * hh + 3]};
    };
    // O (own columns) += P·V for the tile of parity PAR, P of both roles read
    // back from LDS
    auto pv = [&](auto ROLE, auto PAR) __attribute__((always_inline)) {
        constexpr int R = decltype(ROLE)::value;
        const __bf16 *Vs = vstage(PAR);
        bf16x8 pf[2][4];  // [rb][16-key chunk of the tile]
#pragma unroll
        for (int rl = 0; rl < 2; ++rl) {
            const unsigned char *src = pslot(PAR, rl);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    pf[rb][2 * rl + hh] = *(const bf16x8 *)(src + 16 * (64 * (2 * rb + hh) + lane));
        }
        constexpr int NFV = 4 * NDB;  // Vᵀ fragments: 4 key chunks x NDB column blocks
        bf16x8 vf[NFV];
        vf[0] = vt_frag<D>(Vs, NDB * R + 0 % NDB, 0 / NDB, lane);
        vf[1] = vt_frag<D>(Vs, NDB * R + 1 % NDB, 1 / NDB, lane);
#pragma unroll
        for (int f = 0; f < NFV; ++f) {
            if (f + 2 < NFV) vf[f + 2] = vt_frag<D>(Vs, NDB * R + (f + 2) % NDB, (f + 2) / NDB, lane);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
                oacc[rb][f % NDB] = mfma_32x32x16(vf[f], pf[rb][f / NDB], oacc[rb][f % NDB]);
            asm volatile("" ::);
        }
    };

    // ---- one pass over the keys: O, l for the references m ------------------
    // With set_m, m is first fixed from each row's first 32 keys (both roles
    // compute the same value); otherwise m already holds the exact row maxima.
    // Period T: the loaders bring K(T+1) and V(T); role 0 runs P·V(T-1), then
    // its half of tile T; role 1 its half of tile T, then P·V(T-1).
    auto pass = [&](auto ROLE, bool set_m) __attribute__((always_inline)) {
        constexpr int R = decltype(ROLE)::value;
        // an opaque copy of the lane index: the per-lane LDS and global
        // offsets derived from it are then computed inside this role's branch
        // and are not hoisted above it, where both roles' sets would be live
        const int saved[5] = {lane, l32, g, dma_r, dma_p};
        asm volatile("" : "+v"(lane), "+v"(l32), "+v"(g), "+v"(dma_r), "+v"(dma_p));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            l[rb] = 0.f;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[rb][db][r] = 0.f;
        }
        if (R == 1) issue(IC<0>{}, false, 0);
        __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
        __syncthreads();
        if (set_m) {
            f32x16 sacc[2];
            scores(sacc, kstage(IC<0>{}), 0);
            float sv[2][16], mx[2];
            masked_scores(0 >= first_masked_sub, sacc, sv, 0);
            row_max(sv, mx);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) m[rb] = (mx[rb] == -INFINITY) ? 0.f : mx[rb];
        }
        auto period = [&](auto PAR, int T) __attribute__((always_inline)) {
            constexpr int P = decltype(PAR)::value;
            const bool masked = T >= n_plain;
            if constexpr (R == 0) {
                if (T > 0) pv(ROLE, IC<P ^ 1>{});
                score_softmax(ROLE, PAR, T, masked);
            } else {
                if (T + 1 < n_tiles) issue(IC<P ^ 1>{}, false, T + 1);
                issue(PAR, true, T);
                score_softmax(ROLE, PAR, T, masked);
                if (T > 0) pv(ROLE, IC<P ^ 1>{});
            }
            __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's DMAs landed
            __syncthreads();
        };
        for (int T = 0; T < n_tiles; T += 2) {
            period(IC<0>{}, T);
            if (T + 1 < n_tiles) period(IC<1>{}, T + 1);
        }
        if ((n_tiles - 1) & 1)
            pv(ROLE, IC<1>{});
        else
            pv(ROLE, IC<0>{});
        lane = saved[0], l32 = saved[1], g = saved[2], dma_r = saved[3], dma_p = saved[4];
    };
    // normalizer of each row = this lane's part + the other lane half + partner
    __shared__ float l_share[C::NWAVE][2][32];
    __shared__ int wave_bad[C::NWAVE];
    float l_row[2];
    auto combine_l = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            l_row[rb] = xhalf_sum(l[rb]);
            if (g == 0) l_share[w][rb][l32] = l_row[rb];
        }
        __syncthreads();
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) l_row[rb] += l_share[w ^ 4][rb][l32];
    };

    // ---- fast pass with m fixed by each row's first 32 keys; if some row's
    // normalizer leaves [0, 2^32] (every p <= 2^32 when it does not), the
    // exact row maxima are found and the pass runs again (rare) -----------
    constexpr float kMaxL = 4294967296.0f;
    for (bool exact = false;; exact = true) {
        if (role == 0)
            pass(IC<0>{}, !exact);
        else
            pass(IC<1>{}, !exact);
        combine_l();
        if (exact) break;
        bool bad = false;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) bad |= !(l_row[rb] <= kMaxL);  // also catches inf and NaN
        if (lane == 0) wave_bad[w] = __builtin_amdgcn_ballot_w64(bad) != 0;
        __syncthreads();
        bool wg_bad = false;
#pragma unroll
        for (int i = 0; i < C::NWAVE; ++i) wg_bad |= wave_bad[i] != 0;
        if (!wg_bad) break;
        float M[2] = {-INFINITY, -INFINITY};
        for (int T = 0; T < n_tiles; ++T) {
            __syncthreads();  // the previous tile's K stage is no longer read
            if (role == 1) issue(IC<0>{}, false, T);
            __builtin_amdgcn_s_waitcnt(0x3f70);
            __syncthreads();
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f32x16 sacc[2];
                scores(sacc, kstage(IC<0>{}), 32 * half);
                float sv[2][16], mx[2];
                masked_scores(true, sacc, sv, 2 * T + half);
                row_max(sv, mx);
                M[0] = fmaxf(M[0], mx[0]);
                M[1] = fmaxf(M[1], mx[1]);
            }
        }
        __syncthreads();  // K stage 0 and l_share are free again
        m[0] = (M[0] == -INFINITY) ? 0.f : M[0];
        m[1] = (M[1] == -INFINITY) ? 0.f : M[1];
    }

    // ---- O = Oᵀ / l (one reciprocal per row), logsumexp ---------------------
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = prow0 + 32 * rb + l32;
        const float inv_l = 1.0f / l_row[rb];
        if (row < a.Nq) {
            TIn *orow = Op + (int64_t)row * a.o_sn;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int col = 32 * (NDB * role + db) + acc_row(4 * rr, g);
                    store4(orow + col, oacc[rb][db][4 * rr] * inv_l, oacc[rb][db][4 * rr + 1] * inv_l,
                           oacc[rb][db][4 * rr + 2] * inv_l, oacc[rb][db][4 * rr + 3] * inv_l);
                }
            if (role == 0 && g == 0 && a.lse)
                a.lse[((int64_t)b * a.Hq + h) * a.Nq + row] = (m[rb] + log2f(l_row[rb])) * 0.69314718055994531f;
        }
    }
#endif
}

}  // namespace attn
