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
//    A = a 32-key slab of K from LDS, B = the wave's Q fragment held in VGPRs.
//    In the accumulator every lane then holds one query row (l % 32) and 16
//    keys, so the row max and row sum are in-lane, plus one swap with lane
//    l ^ 32 per tile for the max.
//  * Oᵀ += Vᵀ·Pᵀ: Pᵀ is the score accumulator converted to bf16 in place.
//    The keys a lane holds come in runs of four (rows 8*(r/4) + 4g + r%4), so
//    the MFMA k index 8g + e names key 8*(e/4) + 4g + e%4 of each 16-key
//    chunk: bits 2 and 3 swapped. Vᵀ is written to LDS with its keys in that
//    same order, which makes P·V correct with no data movement for P.
//  * Softmax in base 2 with log2(e) folded into the scale on the host, and
//    one reciprocal per row at the end ("Distilling a 4.5 hour CUDA talk",
//    section 2 on the base-2 exponential and on reciprocal reuse; section 7
//    on folding log2(e) into the temperature).
//  * K/V staging: every wave loads a share of tile t+1 into VGPRs before it
//    computes tile t, then writes it to the other LDS buffer; one barrier per
//    tile separates "buffer full" from "buffer free". K keeps row-major order
//    with rows padded by 16 bytes; V is transposed on its way into LDS
//    (the transpose happens at load time, as the pages describe for the
//    P·V operand), rows padded by 16 bytes.
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
    static constexpr int PK = D + 8;        // K row pitch in LDS (elements)
    static constexpr int PV = TK + 8;       // Vᵀ row pitch in LDS (elements)
    static constexpr int K_ELEMS = TK * PK;
    static constexpr int V_ELEMS = D * PV;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int LDS_BYTES = 2 * STAGE * 2;
    static constexpr int KCH = TK * D / 8 / NT;   // 16-byte K chunks per thread
    static constexpr int VITEMS = (TK / 4) * (D / 8);  // 4-key x 8-column V items
    static_assert(TK * D / 8 % NT == 0, "K tile must split evenly over the threads");
    static_assert(VITEMS <= NT, "one V item per thread at most");
};

// Position in the LDS Vᵀ row of key `key` (0..TK-1): bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int key) {
    return (key & ~0xC) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// Two workgroups per CU (two waves per SIMD): the register budget per wave is
// therefore 256, and one wave's softmax can issue while the other's MFMAs run.
template <int D, bool CAUSAL, typename TIn>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(const KernelArgs a) {
    using C = TileCfg<D>;
    constexpr int TQ = C::TQ, TK = C::TK, NT = C::NT, PK = C::PK, PV = C::PV;
    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
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

    // ---- staging registers for the next K/V tile ---------------------------
    u32x4 kreg[C::KCH];
    u32x4 vreg[4];
    const int v_kq = tid % (TK / 4);  // which 4-key group of the tile
    const int v_do = tid / (TK / 4);  // which 8-column group of V
    const bool v_active = tid < C::VITEMS;

    auto load_tile = [&](int t) {
        const int kb0 = t * TK;
#pragma unroll
        for (int u = 0; u < C::KCH; ++u) {
            const int ch = tid + NT * u;
            const int r = ch / (D / 8), c8 = ch % (D / 8);
            const int key = kb0 + r;
            kreg[u] = u32x4{0, 0, 0, 0};
            if (key < a.Nkv) kreg[u] = load8_bf16(Kp + (int64_t)key * a.k_sn + 8 * c8);
        }
        if (v_active) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = kb0 + 4 * v_kq + j;
                vreg[j] = u32x4{0, 0, 0, 0};
                if (key < a.Nkv) vreg[j] = load8_bf16(Vp + (int64_t)key * a.v_sn + 8 * v_do);
            }
        }
    };
    auto store_tile = [&](int s) {
        __bf16 *Ks = lds + s * C::STAGE;
        __bf16 *Vs = Ks + C::K_ELEMS;
#pragma unroll
        for (int u = 0; u < C::KCH; ++u) {
            const int ch = tid + NT * u;
            const int r = ch / (D / 8), c8 = ch % (D / 8);
            *(u32x4 *)(Ks + r * PK + 8 * c8) = kreg[u];
        }
        if (v_active) {
            // 4 keys x 8 columns in registers -> 8 Vᵀ rows x 4 keys in LDS
            const int pos = vt_pos(4 * v_kq);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int p = i >> 1;
                const bool hi = i & 1;
                const uint32_t k01 = pick_halves(vreg[0][p], vreg[1][p], hi);
                const uint32_t k23 = pick_halves(vreg[2][p], vreg[3][p], hi);
                *(u32x2 *)(Vs + (8 * v_do + i) * PV + pos) = u32x2{k01, k23};
            }
        }
    };

    // ---- online softmax state (per lane = per query row) -------------------
    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m = -INFINITY;  // running max of score * c (base-2 domain)
    float l = 0.f;        // running normalizer, partial over this lane's keys

    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        const int s = t & 1;
        if (t + 1 < n_tiles) load_tile(t + 1);

        const int kb0 = t * TK;
        const bool wave_active = !CAUSAL || kb0 <= wrow0 + 31;
        if (wave_active) {
            const __bf16 *Ks = lds + s * C::STAGE;
            const __bf16 *Vs = Ks + C::K_ELEMS;

            // Sᵀ = K·Qᵀ for the 64 keys of this tile, two 32-key slabs
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
                for (int kc = 0; kc < D / 16; ++kc) {
                    const bf16x8 kf = *(const bf16x8 *)(Ks + (32 * kb + l32) * PK + 16 * kc + 8 * g);
                    sacc[kb] = mfma_32x32x16(kf, qf[kc], sacc[kb]);
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
            float mx = sacc[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = xhalf_max(mx);
            const float m_new = fmaxf(m, mx * a.c);
            const float m_sub = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = exp2_hw(m - m_sub);
            m = m_new;

            // p = 2^(s·c - m): Map(exp); partial row sum: Reduce(+)
            float ls = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = exp2_hw(fmaf(sacc[kb][r], a.c, -m_sub));
                    sacc[kb][r] = p;
                    ls += p;
                }
            l = alpha * l + ls;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

            // Pᵀ as bf16 B operands: 16-key chunk 2*kb + hh is registers 8hh..8hh+7
            bf16x8 pf[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    u32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = pack_bf16x2(sacc[kb][8 * hh + 2 * e], sacc[kb][8 * hh + 2 * e + 1]);
                    pf[2 * kb + hh] = u32x4_as_bf16x8(v);
                }

            // Oᵀ += Vᵀ·Pᵀ
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int kc = 0; kc < TK / 16; ++kc) {
                    const bf16x8 vf = *(const bf16x8 *)(Vs + (32 * db + l32) * PV + 16 * kc + 8 * g);
                    oacc[db] = mfma_32x32x16(vf, pf[kc], oacc[db]);
                }
        }

        if (t + 1 < n_tiles) store_tile(s ^ 1);
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
}

}  // namespace attn
