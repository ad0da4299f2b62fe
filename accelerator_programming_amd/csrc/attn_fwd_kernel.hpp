// Fused attention forward kernel for gfx950.
//
// One workgroup owns one (batch, query head, tile of TQ query rows) and writes
// that tile of O and logsumexp; no workgroup talks to another. This is the
// disjoint-output-tile decomposition of "Distilling a 4.5 hour CUDA talk",
// section 5. Inside it, the FlashAttention-2 structure of the same page's
// section 7: the query tile stays in registers while K/V tiles stream through
// on-chip memory (here LDS, double buffered), and the row softmax is carried
// online with a running max m and normalizer l.
//
// gfx950 mapping
//  * 4 waves of 64 lanes; wave w owns query rows q0 + 32w .. q0 + 32w + 31.
//  * Scores are computed transposed, Sᵀ = K·Qᵀ, with 32x32x16 bf16 MFMAs:
//    A = a 32-key slab of K read from LDS, B = the wave's Q fragment held in
//    VGPRs for the whole loop. In the accumulator every lane then holds one
//    query row (l % 32) and 16 keys, so the row max and row sum are in-lane,
//    plus one swap with lane l ^ 32 per tile for the max.
//  * Oᵀ += Vᵀ·Pᵀ: Pᵀ is the score accumulator converted to bf16 in place.
//    The keys a lane holds come in runs of four (rows 8*(r/4) + 4g + r%4), so
//    the MFMA k index 8g + e names key 8*(e/4) + 4g + e%4 of each 16-key
//    chunk. The Vᵀ operand is read from the row-major V tile with the LDS
//    transpose read (ds_read_b64_tr_b16), two reads of four keys each, in
//    exactly that key order: P needs no data movement, V no transposing
//    store. (The pages' P·V operand is likewise transposed at load time.)
//  * Softmax in base 2 with log2(e) folded into the scale on the host, and
//    one reciprocal per row at the end ("Distilling a 4.5 hour CUDA talk",
//    section 2 on the base-2 exponential and on reciprocal reuse; section 7
//    on folding log2(e) into the temperature). The running max is raised
//    lazily: O and l are rescaled only when some row's tile max exceeds its
//    running max by more than 2^kLazy, which keeps every p <= 2^kLazy and
//    leaves O = acc / l and lse = m + log2 l exact in real arithmetic.
//  * K/V staging: every wave issues LDS-DMA loads (global_load_lds_dwordx4,
//    no VGPRs) for its share of tile t+1 into the other LDS buffer before it
//    computes tile t; then "my loads landed" (s_waitcnt vmcnt(0)) and one
//    barrier per tile ("everyone's loads landed, nobody reads the old
//    buffer") close the iteration. LDS-DMA writes 16 bytes per lane at
//    consecutive addresses, so bank-conflict avoidance is an XOR swizzle of
//    the 16-byte chunks of a row, applied by choosing which global chunk each
//    lane fetches (XOR layouts: "Distilling a 4.5 hour CUDA talk", section 8).
#pragma once
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
    static constexpr int TQ = 128;          // query rows per workgroup
    static constexpr int TK = 64;           // keys per streamed tile
    static constexpr int NWAVE = 4;
    static constexpr int NT = 64 * NWAVE;   // threads per workgroup
    static constexpr int CPR = D / 8;       // 16-byte chunks per K or V row
    static constexpr int TILE_ELEMS = TK * D;
    static constexpr int STAGE = 2 * TILE_ELEMS;             // K tile then V tile
    static constexpr int LDS_BYTES = 2 * STAGE * 2;          // two stages, bf16
    static constexpr int ROWS_PER_DMA = 64 / CPR;            // rows one wave-wide DMA covers
    static constexpr int DMA_PER_WAVE = TK / ROWS_PER_DMA / NWAVE;  // per tile per K (or V)
    static_assert(TK % (ROWS_PER_DMA * NWAVE) == 0, "tile rows must split over the waves");
};

// Two workgroups per CU (two waves per SIMD): the register budget per wave is
// therefore 256, and one wave's softmax can issue while the other's MFMAs run.
template <int D, bool CAUSAL, typename TIn>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(const KernelArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    using C = TileCfg<D>;
    constexpr int TQ = C::TQ, TK = C::TK, CPR = C::CPR;
    constexpr float kLazy = 8.0f;
    __shared__ __attribute__((aligned(1024))) __bf16 lds[2 * C::STAGE];

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
    const int wrow0 = q0 + 32 * w;  // first query row of this wave
    const int row = wrow0 + l32;    // this lane's query row
    const int kv_end = CAUSAL ? min(a.Nkv, q0 + TQ) : a.Nkv;
    const int n_tiles = (kv_end + TK - 1) / TK;

    // ---- Q fragment: B operand of Sᵀ = K·Qᵀ, resident for the whole loop ---
    bf16x8 qf[D / 16];
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
        u32x4 v = {0, 0, 0, 0};
        if (row < a.Nq) v = load8_bf16(Qp + (int64_t)row * a.q_sn + 16 * kc + 8 * g);
        qf[kc] = u32x4_as_bf16x8(v);
    }

    // ---- LDS-DMA of one K/V tile: each wave fills DMA_PER_WAVE windows of
    // 64 lanes x 16 bytes in each tile; lane i of a window lands at chunk i. --
    const int dma_r = lane / CPR;          // row within the window
    const int dma_p = lane % CPR;          // physical chunk this lane fills
    auto issue_tile = [&](int t, int s) {
        __bf16 *Ks = lds + s * C::STAGE;
        __bf16 *Vs = Ks + C::TILE_ELEMS;
#pragma unroll
        for (int u = 0; u < C::DMA_PER_WAVE; ++u) {
            const int r = (w * C::DMA_PER_WAVE + u) * C::ROWS_PER_DMA + dma_r;  // tile row
            const int key = min(t * TK + r, a.Nkv - 1);  // clamped: a finite, masked row
            const TIn *kg = Kp + (int64_t)key * a.k_sn + 8 * k_chunk<D>(r, dma_p);
            const TIn *vg = Vp + (int64_t)key * a.v_sn + 8 * v_chunk<D>(r, dma_p);
            const int win = (w * C::DMA_PER_WAVE + u) * 64 * 8;  // elements
            if constexpr (sizeof(TIn) == 2) {
                __builtin_amdgcn_global_load_lds(kg, (lds_void *)(Ks + win), 16, 0, 0);
                __builtin_amdgcn_global_load_lds(vg, (lds_void *)(Vs + win), 16, 0, 0);
            } else {
                // fp32 inputs: round to bf16 in registers, same LDS placement
                *(u32x4 *)(Ks + win + 8 * lane) = load8_bf16(kg);
                *(u32x4 *)(Vs + win + 8 * lane) = load8_bf16(vg);
            }
        }
    };

    // ---- online softmax state (per lane = per query row) -------------------
    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m = -INFINITY;  // running max of score * c (base-2 domain), raised lazily
    float l = 0.f;        // running normalizer, partial over this lane's keys

    if (n_tiles > 0) issue_tile(0, 0);
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's DMA landed
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        const int s = t & 1;
        if (t + 1 < n_tiles) issue_tile(t + 1, s ^ 1);

        const int kb0 = t * TK;
        {
            // (A wave whose rows see no key of this tile still runs it: the
            // mask zeroes its p, and a uniform path keeps the accumulators in
            // place; such tiles are under 1% of a long causal sweep.)
            const __bf16 *Ks = lds + s * C::STAGE;
            const __bf16 *Vs = Ks + C::TILE_ELEMS;

            // Sᵀ = K·Qᵀ for the 64 keys of this tile, two 32-key slabs
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
                const int kr = 32 * kb + l32;
#pragma unroll
                for (int kc = 0; kc < D / 16; ++kc) {
                    sacc[kb] = mfma_32x32x16(k_frag<D>(Ks, kr, kc, g), qf[kc], sacc[kb]);
                }
            }

            // causal mask on diagonal tiles, key-range mask on the ragged tail
            const bool need_mask = (CAUSAL && kb0 + TK - 1 > wrow0) || (kb0 + TK > a.Nkv);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kb0 + 32 * kb + acc_row(r, g);
                        if ((CAUSAL && key > row) || key >= a.Nkv) sacc[kb][r] = -INFINITY;
                    }
            }

            // row max: in-lane over 32 keys, then across the two wave halves
            float mx = fmaxf(sacc[0][0], sacc[0][1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[0][r], sacc[0][r + 1]));
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[1][r], sacc[1][r + 1]));
            mx = xhalf_max(mx) * a.c;

            // lazy rescale: only when some row's max grew by more than 2^kLazy
            if (__builtin_amdgcn_ballot_w64(mx > m + kLazy)) {
                const float m_new = fmaxf(m, mx);
                const float alpha = (m_new == -INFINITY) ? 1.f : exp2_hw(m - m_new);
                l *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                m = m_new;
            }
            const float m_sub = (m == -INFINITY) ? 0.f : m;

            // p = 2^(s·c - m): Map(exp); partial row sum: Reduce(+);
            // Pᵀ as bf16 B operands: 16-key chunk 2*kb + hh is registers 8hh..8hh+7
            bf16x8 pf[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    float p[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        p[e] = exp2_hw(fmaf(sacc[kb][8 * hh + e], a.c, -m_sub));
                        l += p[e];
                    }
                    u32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
                    pf[2 * kb + hh] = u32x4_as_bf16x8(v);
                }

            // Oᵀ += Vᵀ·Pᵀ, Vᵀ fragments by transpose reads of the row-major V tile
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int kc = 0; kc < TK / 16; ++kc)
                    oacc[db] = mfma_32x32x16(vt_frag<D>(Vs, db, kc, lane), pf[kc], oacc[db]);
        }

        __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's DMA of tile t+1 landed
        __syncthreads();
    }

    // ---- epilogue: O = Oᵀ / l (one reciprocal per row), logsumexp ---------
    const float l_row = xhalf_sum(l);
    const float inv_l = 1.0f / l_row;
    if (row < a.Nq) {
        TIn *orow = Op + (int64_t)row * a.o_sn;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int col = 32 * db + acc_row(4 * rr, g);
                store4(orow + col, oacc[db][4 * rr] * inv_l, oacc[db][4 * rr + 1] * inv_l,
                       oacc[db][4 * rr + 2] * inv_l, oacc[db][4 * rr + 3] * inv_l);
            }
        if (g == 0 && a.lse)
            a.lse[((int64_t)b * a.Hq + h) * a.Nq + row] = (m + log2f(l_row)) * 0.69314718055994531f;
    }
#endif
}

}  // namespace attn
