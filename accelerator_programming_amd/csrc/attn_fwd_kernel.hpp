// Fused attention forward kernel for gfx950.
//
// One workgroup owns one (batch, query head, tile of TQ = 256 query rows) and
// writes that tile of O and logsumexp; no workgroup talks to another: the
// disjoint-output-tile decomposition of "Distilling a 4.5 hour CUDA talk",
// section 5. Inside it, the FlashAttention-2 structure of the same page's
// section 7: the query tile stays in registers while K/V tiles stream through
// on-chip memory (here a three-stage LDS ring), and the row softmax is carried
// online with a running max m and normalizer l.
//
// gfx950 mapping
//  * 4 waves of 64 lanes, one per SIMD; wave w owns query rows
//    q0 + 64w .. q0 + 64w + 63 as two 32-row blocks (rb = 0, 1). Every K or V
//    fragment read from LDS feeds the MFMAs of both blocks, so a CU reads each
//    tile four times per 256 rows and LDS bandwidth (about 128 bytes per
//    clock per CU) stays well below what the MFMA pipe consumes.
//  * Scores are computed transposed, Sᵀ = K·Qᵀ, with 32x32x16 bf16 MFMAs:
//    A = a 32-key slab of K read from LDS, B = the block's Q fragment held in
//    VGPRs for the whole loop. In the accumulator every lane then holds one
//    query row (l % 32) and 16 keys, so the row max and row sum are in-lane,
//    plus one swap with lane l ^ 32 for the max.
//  * Oᵀ += Vᵀ·Pᵀ: Pᵀ is the score accumulator converted to bf16 in place.
//    The keys a lane holds come in runs of four (rows 8*(r/4) + 4g + r%4), so
//    the MFMA k index 8g + e names key 8*(e/4) + 4g + e%4 of each 16-key
//    chunk. The Vᵀ operand is read from the row-major V tile with the LDS
//    transpose read (ds_read_b64_tr_b16) in exactly that key order: P needs no
//    data movement, V no transposing store. (The pages' P·V operand is
//    likewise transposed at load time.)
//  * Softmax in base 2 with log2(e) folded into the scale on the host, and
//    one reciprocal per row at the end ("Distilling a 4.5 hour CUDA talk",
//    section 2 on the base-2 exponential and on reciprocal reuse; section 7
//    on folding log2(e) into the temperature). Each row's exponent reference
//    m is fixed from its first 32 keys: O = acc / l and lse = m + log2 l are
//    exact in real arithmetic for any m, so no rescaling happens inside the
//    loop. If some row's l leaves [0, 2^32] (a later key outscored the first
//    ones by a wide margin) the workgroup recomputes with exact row maxima.
//  * Per 32-key sub-tile: the Sᵀ MFMAs, then the P·V MFMAs of the previous
//    sub-tile with the exponentials of this one placed between them.
//  * K/V staging: LDS-DMA (global_load_lds_dwordx4, no VGPRs) into a
//    three-stage ring per tensor. In 64-key tile T the waves issue K(T+2) and
//    V(T+1) and read K(T), K(T+1), V(T-1), V(T); "my loads landed"
//    (s_waitcnt vmcnt(0)) plus one barrier per tile close the tile. LDS-DMA
//    writes 16 bytes per lane at consecutive addresses, so bank-conflict
//    avoidance is an XOR swizzle of the 16-byte chunks of a row, applied by
//    choosing which global chunk each lane fetches.
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
    float c;  // softmax scale * log2(e)
};

template <int D>
struct TileCfg {
    static constexpr int TQ = 256;          // query rows per workgroup
    static constexpr int TK = 64;           // keys per LDS tile (two 32-key sub-tiles)
    static constexpr int NWAVE = 4;
    static constexpr int NT = 64 * NWAVE;   // threads per workgroup
    static constexpr int NSTAGE = 3;        // LDS ring depth for K and for V
    static constexpr int CPR = D / 8;       // 16-byte chunks per K or V row
    static constexpr int TILE = TK * D;     // elements of one K or V tile
    static constexpr int LDS_ELEMS = 2 * NSTAGE * TILE;
    static constexpr int LDS_BYTES = LDS_ELEMS * 2;
    static constexpr int ROWS_PER_DMA = 64 / CPR;                   // rows per wave-wide DMA
    static constexpr int DMA_PER_WAVE = TK / ROWS_PER_DMA / NWAVE;  // per tile per tensor
    static constexpr int NKC = D / 16;      // k-steps of Sᵀ = K·Qᵀ
    static constexpr int NDB = D / 32;      // 32-column blocks of O
    static_assert(TK % (ROWS_PER_DMA * NWAVE) == 0, "tile rows must split over the waves");
};

// Two 32-row blocks x two 16-key chunks of bf16 Pᵀ operands.
struct PTile {
    bf16x8 v[2][2];
};

template <int D, bool CAUSAL, typename TIn>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_fwd_kernel(const KernelArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    using C = TileCfg<D>;
    constexpr int TQ = C::TQ, TK = C::TK, CPR = C::CPR, NKC = C::NKC, NDB = C::NDB;
    __shared__ __attribute__((aligned(1024))) __bf16 lds[C::LDS_ELEMS];
    __bf16 *const Kst = lds;                        // K stages
    __bf16 *const Vst = lds + C::NSTAGE * C::TILE;  // V stages

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;

    // ---- work item: heaviest causal tiles are dispatched first -------------
    const int BH = a.B * a.Hq;
    const int bh = blockIdx.x % BH;
    int qt = blockIdx.x / BH;
    if (CAUSAL) qt = a.n_qtiles - 1 - qt;
    const int b = bh / a.Hq, h = bh % a.Hq, hk = h / a.group;
    const TIn *__restrict__ Qp = (const TIn *)a.q + b * a.q_sb + h * a.q_sh;
    const TIn *__restrict__ Kp = (const TIn *)a.k + b * a.k_sb + hk * a.k_sh;
    const TIn *__restrict__ Vp = (const TIn *)a.v + b * a.v_sb + hk * a.v_sh;
    TIn *__restrict__ Op = (TIn *)a.o + b * a.o_sb + h * a.o_sh;

    const int q0 = qt * TQ;
    const int wrow0 = q0 + 64 * w;  // first query row of this wave
    const int kv_end = CAUSAL ? min(a.Nkv, q0 + TQ) : a.Nkv;
    const int n_tiles = (kv_end + TK - 1) / TK;  // >= 1
    // 32-key sub-tiles from this index on need the causal or key-range mask
    const int first_masked_sub = CAUSAL ? min(q0 / 32, a.Nkv / 32) : a.Nkv / 32;

    // ---- Q fragments: B operands of Sᵀ = K·Qᵀ, resident for the whole loop --
    bf16x8 qf[2][NKC];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = wrow0 + 32 * rb + l32;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            u32x4 v = {0, 0, 0, 0};
            if (row < a.Nq) v = load8_bf16(Qp + (int64_t)row * a.q_sn + 16 * kc + 8 * g);
            qf[rb][kc] = u32x4_as_bf16x8(v);
        }
    }

    // ---- LDS-DMA of one K or V tile: each wave fills DMA_PER_WAVE windows
    // of 64 lanes x 16 bytes; lane i of a window lands at chunk i. ----------
    const int dma_r = lane / CPR;  // row within the window
    const int dma_p = lane % CPR;  // physical chunk this lane fills
    auto issue = [&](const TIn *base, int32_t sn, int tile, __bf16 *dst, bool is_v)
                     __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < C::DMA_PER_WAVE; ++u) {
            const int r = (w * C::DMA_PER_WAVE + u) * C::ROWS_PER_DMA + dma_r;  // tile row
            const int key = min(tile * TK + r, a.Nkv - 1);  // clamped: a finite, masked row
            const int chunk = is_v ? v_chunk<D>(r, dma_p) : k_chunk<D>(r, dma_p);
            const TIn *src = base + (int64_t)key * sn + 8 * chunk;
            __bf16 *win = dst + (w * C::DMA_PER_WAVE + u) * 64 * 8;
            if constexpr (sizeof(TIn) == 2) {
                dma16_to_lds(src, win);
            } else {
                // fp32 inputs: round to bf16 in registers, same LDS placement
                *(u32x4 *)(win + 8 * lane) = load8_bf16(src);
            }
        }
    };
    // ring slots; tile indices are never negative here (callers pass T + NSTAGE - 1 for T - 1)
    auto kstage = [&](int tile) __attribute__((always_inline)) { return Kst + (tile % C::NSTAGE) * C::TILE; };
    auto vstage = [&](int tile) __attribute__((always_inline)) { return Vst + (tile % C::NSTAGE) * C::TILE; };

    // ---- state -------------------------------------------------------------
    f32x16 oacc[2][NDB];
    float m[2];  // per-row reference of the exponentials (base 2, score*c units)
    float l[2];  // normalizer, partial over this lane's keys
    PTile pA, pB;

    // Sᵀ of one 32-key sub-tile (rows kq_row0.. of K stage Kq) for both row
    // blocks: 2*NKC MFMAs in two independent chains sharing each K fragment.
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
    // scores of sub-tile js as floats, with the causal / key-range mask
    auto masked_scores = [&](auto masked, const f32x16 (&sacc)[2], float (&sv)[2][16], int js)
                             __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sv[rb][r] = sacc[rb][r];
        if (decltype(masked)::value) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int row = wrow0 + 32 * rb + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 32 * js + acc_row(r, g);
                    if ((CAUSAL && key > row) || key >= a.Nkv) sv[rb][r] = -INFINITY;
                }
            }
        }
    };
    // row maxima of score * c over a sub-tile (both wave halves)
    auto row_max = [&](const float (&sv)[2][16], float (&mx)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            float x = fmaxf(sv[rb][0], sv[rb][1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) x = fmaxf(x, fmaxf(sv[rb][r], sv[rb][r + 1]));
            mx[rb] = xhalf_max(x) * a.c;
        }
    };

    // ---- one pipeline step (32-key sub-tile js) ----------------------------
    // 1. Sᵀ(js) = K·Qᵀ.
    // 2. Oᵀ += Vᵀ(js-1)·Pᵀ(js-1) (pin, V chunks pv_kc0.. of stage Vs) on the
    //    MFMA pipe, issued slot by slot together with the exponentials of S(js)
    //    into pout: p = 2^(s·c - m), with m the row's fixed reference.
    // set_m: this is the first sub-tile of the pass and fixes m from its max.
    auto step = [&](auto masked, bool set_m, PTile &pout, const __bf16 *Kq, int kq_row0,
                    const PTile &pin, const __bf16 *Vs, int pv_kc0, int js)
                    __attribute__((always_inline)) {
        f32x16 sacc[2];
        scores(sacc, Kq, kq_row0);
        float sv[2][16];
        masked_scores(masked, sacc, sv, js);
        if (set_m) {
            float mx[2];
            row_max(sv, mx);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) m[rb] = (mx[rb] == -INFINITY) ? 0.f : mx[rb];
        }
        const float negm[2] = {-m[0], -m[1]};
        float ls[2] = {0.f, 0.f};
        constexpr int NFV = 2 * NDB;       // Vᵀ fragments, each feeding two MFMAs
        constexpr int NSLOT = 2 * NFV;     // MFMAs
        constexpr int PAIRS = 16 / NSLOT;  // score pairs per slot (1 for d=128, 2 for d=64)
        uint32_t pk[2][8];
        bf16x8 vf[NFV];
        vf[0] = vt_frag<D>(Vs, 0, pv_kc0, lane);
        vf[1] = vt_frag<D>(Vs, 1 % NDB, pv_kc0 + 1 / NDB, lane);
#pragma unroll
        for (int f = 0; f < NFV; ++f) {
            if (f + 2 < NFV) vf[f + 2] = vt_frag<D>(Vs, (f + 2) % NDB, pv_kc0 + (f + 2) / NDB, lane);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int slot = 2 * f + rb;
                oacc[rb][f % NDB] = mfma_32x32x16(vf[f], pin.v[rb][f / NDB], oacc[rb][f % NDB]);
#pragma unroll
                for (int q = 0; q < PAIRS; ++q) {
                    const int pp = PAIRS * slot + q, srb = pp / 8, r = 2 * (pp % 8);
                    exp_pair(sv[srb][r], sv[srb][r + 1], a.c, negm[srb], ls[srb], pk[srb][r / 2]);
                }
            }
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                pout.v[rb][hh] = u32x4_as_bf16x8(
                    u32x4{pk[rb][4 * hh], pk[rb][4 * hh + 1], pk[rb][4 * hh + 2], pk[rb][4 * hh + 3]});
            l[rb] += ls[rb];
        }
    };

    // ---- one pass over the keys: O, l for the current references m ----------
    // With set_m_first, m is fixed from each row's first 32 keys; otherwise m
    // must already hold the exact row maxima.
    auto pass = [&](bool set_m_first) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            l[rb] = 0.f;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[rb][db][r] = 0.f;
            // P of "sub-tile -1": zero, so the first step's P·V adds nothing
            // (it reads V(0), which holds finite values)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) pB.v[rb][hh] = u32x4_as_bf16x8(u32x4{0, 0, 0, 0});
        }
        // prologue: K(0), K(1), V(0) in flight
        issue(Kp, a.k_sn, 0, kstage(0), false);
        if (n_tiles > 1) issue(Kp, a.k_sn, 1, kstage(1), false);
        issue(Vp, a.v_sn, 0, vstage(0), true);
        __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's DMA landed
        __syncthreads();
        auto tile = [&](int T, auto masked) __attribute__((always_inline)) {
            if (T + 2 < n_tiles) issue(Kp, a.k_sn, T + 2, kstage(T + 2), false);
            if (T + 1 < n_tiles) issue(Vp, a.v_sn, T + 1, vstage(T + 1), true);
            // sub-tile 2T: first half of K(T); P·V of sub-tile 2T-1 (second half
            // of V(T-1)) with pB; exponentials into pA
            const __bf16 *Vprev = T > 0 ? vstage(T + C::NSTAGE - 1) : vstage(0);
            step(masked, set_m_first && T == 0, pA, kstage(T), 0, pB, Vprev, 2, 2 * T);
            // sub-tile 2T+1: second half of K(T); P·V of sub-tile 2T (first half
            // of V(T)) with pA; exponentials into pB
            step(masked, false, pB, kstage(T), 32, pA, vstage(T), 0, 2 * T + 1);
            __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's DMAs of K(T+2), V(T+1) landed
            __syncthreads();
        };
        // tiles whose keys all precede every row of the workgroup need no mask
        const int n_plain = min(n_tiles, first_masked_sub / 2);
        for (int T = 0; T < n_plain; ++T) tile(T, std::integral_constant<bool, false>{});
        for (int T = n_plain; T < n_tiles; ++T) tile(T, std::integral_constant<bool, true>{});
        // P·V of the last sub-tile
        const __bf16 *Vl = vstage(n_tiles - 1);
#pragma unroll
        for (int kc2 = 0; kc2 < 2; ++kc2)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const bf16x8 vf = vt_frag<D>(Vl, db, 2 + kc2, lane);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    oacc[rb][db] = mfma_32x32x16(vf, pB.v[rb][kc2], oacc[rb][db]);
            }
    };

    // ---- fast pass: reference m fixed by each row's first 32 keys ------------
    // Exact in real arithmetic for any m (O = acc / l, lse = m + log2 l); it
    // only has to stay in range: p <= 2^32 is guaranteed when l <= 2^32.
    pass(true);
    constexpr float kMaxL = 4294967296.0f;  // 2^32
    bool bad = false;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) bad |= !(xhalf_sum(l[rb]) <= kMaxL);  // also catches inf/NaN
    __shared__ int wave_bad[C::NWAVE];
    if (lane == 0) wave_bad[w] = __builtin_amdgcn_ballot_w64(bad) != 0;
    __syncthreads();
    const bool wg_bad = wave_bad[0] | wave_bad[1] | wave_bad[2] | wave_bad[3];
    if (wg_bad) {
        // ---- slow pass (rare: a later key outscored a row's first keys by
        // more than 2^32): exact row maxima first, then the pass again ------
        float M[2] = {-INFINITY, -INFINITY};
        for (int T = 0; T < n_tiles; ++T) {
            issue(Kp, a.k_sn, T, kstage(0), false);
            __builtin_amdgcn_s_waitcnt(0x3f70);
            __syncthreads();
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f32x16 sacc[2];
                scores(sacc, kstage(0), 32 * half);
                float sv[2][16], mx[2];
                masked_scores(std::integral_constant<bool, true>{}, sacc, sv, 2 * T + half);
                row_max(sv, mx);
                M[0] = fmaxf(M[0], mx[0]);
                M[1] = fmaxf(M[1], mx[1]);
            }
            __syncthreads();
        }
        m[0] = (M[0] == -INFINITY) ? 0.f : M[0];
        m[1] = (M[1] == -INFINITY) ? 0.f : M[1];
        pass(false);
    }

    // ---- O = Oᵀ / l (one reciprocal per row), logsumexp ---------------------
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = wrow0 + 32 * rb + l32;
        const float l_row = xhalf_sum(l[rb]);
        const float inv_l = 1.0f / l_row;
        if (row < a.Nq) {
            TIn *orow = Op + (int64_t)row * a.o_sn;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int col = 32 * db + acc_row(4 * rr, g);
                    store4(orow + col, oacc[rb][db][4 * rr] * inv_l, oacc[rb][db][4 * rr + 1] * inv_l,
                           oacc[rb][db][4 * rr + 2] * inv_l, oacc[rb][db][4 * rr + 3] * inv_l);
                }
            if (g == 0 && a.lse)
                a.lse[((int64_t)b * a.Hq + h) * a.Nq + row] = (m[rb] + log2f(l_row)) * 0.69314718055994531f;
        }
    }
#endif
}

}  // namespace attn
