// Split-KV attention forward for few query rows per head (decode-like shapes),
// and the merge of the splits' partial results.
//
// Same method as the main kernel (disjoint output tiles, "Distilling a 4.5
// hour CUDA talk", section 5; K/V streamed through LDS with the row softmax
// carried by a running max and normalizer, section 7), decomposed for shapes
// where the query rows of a kv head are few (rows = group x N_q <= 64) and
// the keys many. Such a problem is bound by reading K and V once from HBM:
//  * One workgroup per (key split, batch, kv head) takes all query rows of
//    the kv head's group (row r = query head h0 + r / N_q, query r % N_q, up
//    to 64 rows in two 32-row blocks) against the split's keys, so every K/V
//    byte is read from HBM once; the splits make enough workgroups to keep
//    every CU streaming.
//  * 4 waves (two workgroups share a CU); wave w = 2 rb + kh takes row block rb and key half
//    kh of each 64-key tile: Sᵀ = K·Qᵀ (32x32x16 bf16 MFMA), the online
//    softmax (running max per row, rescale of O when it grows, as the
//    FlashAttention-2 recurrence states), Oᵀ += Vᵀ·Pᵀ with P from registers
//    and Vᵀ by transposed LDS reads. At the end the two key halves of a row
//    block are combined through LDS.
//  * K/V tiles (64 keys) in a two-stage LDS ring (64 KB at d = 128), copied
//    by LDS-DMA, so that two workgroups share a CU: while one waits for its
//    copies or at its barrier the other computes (measured: 1.45x the
//    bandwidth of one workgroup per CU with four tiles in flight). Wave T % 4
//    copies tile T one tile ahead and waits (vmcnt(0)) for it before the
//    barrier that opens tile T: its only copies in flight.
//  * The workgroup writes its rows' O / l (fp32) and logsumexp for the split
//    to a caller-provided workspace; the merge kernel combines the splits:
//    lse = ln Σ_s exp(lse_s), O = Σ_s exp(lse_s - lse) O_s.
#pragma once

#include "attn_fwd_kernel.hpp"

namespace attn {

template <int D>
struct SplitCfg {
    static constexpr int ROWS = 64;  // query rows per workgroup (two 32-row blocks)
    static constexpr int TK = 64;    // keys per tile (one 32-key half per wave)
    static constexpr int NWAVE = 4;
    static constexpr int NT = 64 * NWAVE;
    static constexpr int CPR = D / 8;            // 16-byte chunks per K or V row
    static constexpr int TILE = TK * D;          // elements of one K or V tile
    static constexpr int STAGE_B = 2 * TILE * 2; // K and V of one tile
    static constexpr int NSTAGE = 2;  // tile T computed while tile T + 1 is copied
    static constexpr int LDS_BYTES = NSTAGE * STAGE_B;
    static constexpr int ROWS_PER_DMA = 64 / CPR;
    static constexpr int WIN = TK / ROWS_PER_DMA;  // 1 KB copies per tensor per tile
    static constexpr int NKC = D / 16;             // k-steps of Sᵀ = K·Qᵀ
    static constexpr int NCB = D / 32;             // 32-column blocks of O
    static constexpr int XCH_B = NCB * 16 * 64 * 4;  // one wave's O accumulator
    static_assert(D == 64 || D == 128, "head dimension");
    static_assert(LDS_BYTES >= 2 * XCH_B + 4 * 64 * 4, "the combine reuses the ring");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert(NSTAGE - 1 <= NWAVE, "one copy in flight per wave");
    static_assert(2 * LDS_BYTES <= 160 * 1024, "two workgroups per CU");
};

struct SplitArgs {
    KernelArgs a;
    float *opart;     // [n_splits][B][H_q][N_q][D] fp32: O / l of each split
    float *lpart;     // [n_splits][B][H_q][N_q]: logsumexp of each split (-inf if empty)
    int32_t n_splits;
    int32_t split_len;  // keys per split, a multiple of the tile
    int32_t rows;       // group * N_q (<= 64)
};

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_split_kernel(const SplitArgs sa) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    using C = SplitCfg<D>;
    constexpr int TK = C::TK, NKC = C::NKC, NCB = C::NCB;
    const KernelArgs &a = sa.a;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int kh = w & 1, rb = w >> 1;

    // ---- work item: blockIdx = (split, batch, kv head), kv head fastest ----
    const int n_groups = a.B * a.Hkv;
    const uint32_t wid = work_index(blockIdx.x, gridDim.x);
    const int split = wid / n_groups;
    const int b = (wid % n_groups) / a.Hkv, hk = (wid % n_groups) % a.Hkv;
    const int k_begin = split * sa.split_len;
    const int k_end = min(a.Nkv, k_begin + sa.split_len);
    const int n_tiles = k_end > k_begin ? (k_end - k_begin + TK - 1) / TK : 0;
    const __bf16 *__restrict__ Kp = (const __bf16 *)a.k + b * a.k_sb + hk * a.k_sh;
    const __bf16 *__restrict__ Vp = (const __bf16 *)a.v + b * a.v_sb + hk * a.v_sh;

    // this lane's row (P·V, epilogue, score column): row r of the group
    const int r = 32 * rb + l32;
    const bool row_ok = r < sa.rows;
    const int h = hk * a.group + (row_ok ? r / a.Nq : 0), qi = row_ok ? r % a.Nq : 0;

    // ---- Q fragments of the row block (B operands), resident -------------
    bf16x8 qf[NKC];
    {
        const __bf16 *qrow = (const __bf16 *)a.q + b * a.q_sb + h * a.q_sh + (int64_t)qi * a.q_sn;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            u32x4 v = {0, 0, 0, 0};
            if (row_ok) v = load8_bf16(qrow + 16 * kc + 8 * g);
            qf[kc] = u32x4_as_bf16x8(v);
        }
    }

    // ---- K/V copies: the tile of loop step T into stage T % 2 by wave
    // T % 4: window u of a tensor covers rows ROWS_PER_DMA u .. of the
    // tile; lane i of a window lands at chunk i % CPR of row i / CPR and
    // fetches the global chunk the swizzle puts there; a buffer resource that
    // ends at the split's last key makes rows past it read as zeros. --------
    // Loop step T works on tile phys(T) of the split: each workgroup starts
    // at its own tile and wraps around, so that the workgroups, whose key
    // ranges lie at equal power-of-two strides, do not all read the same
    // offsets of their ranges at the same time (measured: +11 % bandwidth
    // on 512 workgroups of 32 tiles). The softmax takes the keys in any order.
    const int rot = n_tiles > 0 ? (int)(wid % (uint32_t)n_tiles) : 0;
    auto phys = [&](int T) { const int t = T + rot; return t >= n_tiles ? t - n_tiles : t; };
    const int dma_r = lane / C::CPR, dma_p = lane % C::CPR;
    auto copy_tile = [&](int T, int stage) __attribute__((always_inline)) {
        if (T >= n_tiles || (T & 3) != w) return;
        unsigned char *st = lds + stage * C::STAGE_B;
        perturb_pause();
        const int key0 = k_begin + phys(T) * TK;
        const int rem = k_end - key0;  // >= 1
#pragma unroll
        for (int is_v = 0; is_v < 2; ++is_v) {
            const __bf16 *base = is_v ? Vp : Kp;
            const int32_t sn = is_v ? a.v_sn : a.k_sn;
            const uint32_t bytes = (uint32_t)(((int64_t)(rem - 1) * sn + D) * 2);
            const u32x4 rsrc = buffer_rsrc(base + (int64_t)key0 * sn, bytes);
            unsigned char *dst = st + is_v * C::TILE * 2;
#pragma unroll
            for (int u = 0; u < C::WIN; ++u) {
                const int row = u * C::ROWS_PER_DMA + dma_r;
                const int chunk = is_v ? v_chunk<D>(row, dma_p) : k_chunk<D>(row, dma_p);
                const int64_t off = ((int64_t)row * sn + 8 * chunk) * 2;
                const uint32_t voff = off < (int64_t)bytes ? (uint32_t)off : 0xFFFFFFF0u;
                dma16_buf_to_lds(rsrc, voff, dst + u * 1024);
            }
        }
    };

    // ---- online softmax state of this wave's rows over its keys -----------
    f32x16 oacc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[cb][i] = 0.f;
    float m = -INFINITY;  // running max of score * c (row l32, both lane halves)
    float l = 0.f;        // normalizer, this lane half's keys

    auto tile_step = [&](int T, int stage) __attribute__((always_inline)) {
        const __bf16 *Ks = (const __bf16 *)(lds + stage * C::STAGE_B);
        const __bf16 *Vs = Ks + C::TILE;
        // Sᵀ = K·Qᵀ over keys 32 kh .. 32 kh + 31 of the tile
        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
        bf16x8 kf[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) kf[kc] = k_frag<D>(Ks, 32 * kh + l32, kc, g);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) sacc = mfma_32x32x16(kf[kc], qf[kc], sacc);
        // mask keys past the split's end, scale to base 2
        const int key0 = k_begin + phys(T) * TK + 32 * kh;
        float t[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            t[i] = (key0 + acc_row(i, g) < k_end) ? sacc[i] * a.c : -INFINITY;
            tmax = fmaxf(tmax, t[i]);
        }
        tmax = xhalf_max(tmax);
        // running max; O and l rescaled when it grows
        const float m_new = fmaxf(m, tmax);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // all masked so far
        const float alpha = exp2_hw(m - m_use);                  // 0 while m = -inf
        m = m_new;
        uint32_t pk[8];
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pk[j] = pack_bf16x2(exp2_hw(t[2 * j] - m_use), exp2_hw(t[2 * j + 1] - m_use));
            ls[j & 3] = sum_bf16x2(pk[j], ls[j & 3]);
        }
        l = l * alpha + ((ls[0] + ls[1]) + (ls[2] + ls[3]));
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[cb][i] *= alpha;
        // Oᵀ += Vᵀ·Pᵀ over the wave's 32 keys (two 16-key chunks)
        const __bf16 *Vh = Vs + 32 * kh * D;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const bf16x8 pf = u32x4_as_bf16x8(u32x4{pk[4 * kc], pk[4 * kc + 1], pk[4 * kc + 2], pk[4 * kc + 3]});
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) oacc[cb] = mfma_32x32x16(vt_frag<D>(Vh, cb, kc, lane), pf, oacc[cb]);
        }
    };

    // prologue: tile 0 copied; each tile's copier waits for its own copy
    // (vmcnt(0): its only copies in flight) before the barrier that opens it
#pragma unroll
    for (int T = 0; T < C::NSTAGE - 1; ++T) copy_tile(T, T);
    int stage = 0;  // T % NSTAGE
    for (int T = 0; T < n_tiles; ++T) {
        if ((T & 3) == w) __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
        __syncthreads();  // tile T landed; every wave is done with tile T - 1
        copy_tile(T + C::NSTAGE - 1, stage == 0 ? C::NSTAGE - 1 : stage - 1);  // the stage of tile T - 1
        // a row block without query rows (group x N_q <= 32) keeps only its
        // copy duty and the barriers
        if (32 * rb < sa.rows) tile_step(T, stage);
        stage = stage == C::NSTAGE - 1 ? 0 : stage + 1;
    }
    __builtin_amdgcn_s_waitcnt(0x3f70);  // no copy outlives the loop
    __syncthreads();                      // the ring is free for the combine

    // ---- combine the two key halves of each row block, write the split ----
    float *mx = (float *)(lds + 2 * C::XCH_B);  // [4 waves][32 rows]
    float *lx = mx + 4 * 32;                    // [4 waves][32 rows]
    const float l_row = xhalf_sum(l);
    if (g == 0) {
        mx[32 * w + l32] = m;
        lx[32 * w + l32] = l_row;
    }
    __syncthreads();
    const float m_other = mx[32 * (w ^ 1) + l32];
    const float M = fmaxf(m, m_other);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    const float f_self = exp2_hw(m - M_use), f_other = exp2_hw(m_other - M_use);
    float *xo = (float *)(lds + rb * C::XCH_B);  // the kh = 1 wave's O of row block rb
    if (kh == 1) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *(f32x4 *)(xo + 4 * (64 * (4 * cb + q) + lane)) =
                    f32x4{oacc[cb][4 * q], oacc[cb][4 * q + 1], oacc[cb][4 * q + 2], oacc[cb][4 * q + 3]};
    }
    __syncthreads();
    if (kh == 0) {
        const float L = l_row * f_self + lx[32 * (w ^ 1) + l32] * f_other;
        const float inv = L > 0.f ? 1.0f / L : 0.f;
        const int64_t prow = (((int64_t)split * a.B + b) * a.Hq + h) * a.Nq + qi;
        if (row_ok) {
            float *orow = sa.opart + prow * D;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 o2 = *(const f32x4 *)(xo + 4 * (64 * (4 * cb + q) + lane));
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (oacc[cb][4 * q + e] * f_self + o2[e] * f_other) * inv;
                    *(f32x4 *)(orow + 32 * cb + acc_row(4 * q, g)) = v;
                }
            if (g == 0)
                sa.lpart[prow] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
        }
    }
#endif
}

// Merge of the splits, one workgroup per (b, h, i) row. Every thread loads
// its share of the splits' partial rows at once (thread t: columns
// 4 (t % (D/4)) .. + 3 of splits t / (D/4), + 256 / (D/4), ...), while wave 0
// forms the weights from the splits' logsumexps: lse = ln Σ_s exp(lse_s)
// (largest term factored out), w_s = exp(lse_s - lse); then each thread sums
// w_s O_s over its splits and the split slots are added through LDS. One
// memory round trip per row, whatever the split count.
template <int D>
__global__ void __launch_bounds__(256) attn_split_merge(const float *__restrict__ opart,
                                                        const float *__restrict__ lpart, int32_t n_splits,
                                                        int64_t n_rows, KernelArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int CG = D / 4;         // float4 column groups of a row
    constexpr int SLOTS = 256 / CG;   // split slots
    constexpr int PER = 64 / SLOTS;   // splits per slot (at most 64 splits)
    __shared__ float wsh[64];
    __shared__ f32x4 red[SLOTS][CG];
    const int t = threadIdx.x;
    const int c = t % CG, j = t / CG;
    const int64_t row = work_index(blockIdx.x, gridDim.x);
    f32x4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int s = j + SLOTS * i;
        v[i] = s < n_splits ? *(const f32x4 *)(opart + ((int64_t)s * n_rows + row) * D + 4 * c)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (t < 64) {
        const float ls = t < n_splits ? lpart[(int64_t)t * n_rows + row] : -INFINITY;
        float mxv = ls;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) mxv = fmaxf(mxv, __shfl_xor(mxv, off));
        const float mref = (mxv == -INFINITY) ? 0.f : mxv;
        const float wgt = t < n_splits ? exp2_hw((ls - mref) * 1.4426950408889634f) : 0.f;
        float sum = wgt;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
        const float inv = sum > 0.f ? 1.0f / sum : 0.f;
        wsh[t] = wgt * inv;
        if (t == 0 && a.lse) a.lse[row] = sum > 0.f ? mref + log2f(sum) * 0.69314718055994531f : -INFINITY;
    }
    __syncthreads();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int s = j + SLOTS * i;
        if (s < n_splits) acc += wsh[s] * v[i];
    }
    red[j][c] = acc;
    __syncthreads();
    if (t < CG) {
        f32x4 o = red[0][t];
#pragma unroll
        for (int q = 1; q < SLOTS; ++q) o += red[q][t];
        // row -> (b, h, i)
        const int64_t i = row % a.Nq, bh = row / a.Nq;
        const int64_t h = bh % a.Hq, b = bh / a.Hq;
        __bf16 *orow = (__bf16 *)a.o + b * a.o_sb + h * a.o_sh + i * a.o_sn + 4 * t;
#pragma unroll
        for (int e = 0; e < 4; ++e) orow[e] = (__bf16)o[e];
    }
#endif
}

}  // namespace attn
