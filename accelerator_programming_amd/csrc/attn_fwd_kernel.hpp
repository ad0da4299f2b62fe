// Fused attention forward kernel for gfx950.
//
// One workgroup owns one (batch, query head, tile of TQ = 256 query rows) at a
// time and writes that tile of O and logsumexp; no workgroup talks to
// another: the disjoint-output-tile decomposition of "Distilling a 4.5 hour
// CUDA talk", section 5. Where the items split evenly over the 256 CUs the
// grid is one workgroup per CU, each taking its items in turn (no launch
// between items on a CU). Inside it, the FlashAttention-2 structure of the same page's
// section 7: the query tile stays in registers while K/V tiles stream through
// on-chip memory (LDS), and the row softmax is carried across key tiles with
// a per-row reference and a normalizer.
//
// gfx950 mapping
//  * 8 waves, two per SIMD (waves p and p + 4 share SIMD p). Wave w owns the
//    32 query rows q0 + 32w .. q0 + 32w + 31 over every key and every output
//    column, so a wave's softmax, P and O never leave its registers; the
//    waves share only the K/V tiles in LDS.
//  * Why two phase orders: on gfx950 a wave's VALU work does not overlap its
//    own MFMAs, while the VALU and MFMA work of two waves on one SIMD do. In
//    each period (one 64-key tile) wave p (role 0) runs its MFMAs first, the
//    scores of this tile and P·V of the previous one, then its softmax; wave
//    p + 4 (role 1) runs its softmax first, on scores it computed at the end
//    of the previous period, then P·V and the next tile's scores. Each wave's
//    exponentials run while its SIMD partner's MFMAs execute: compute never
//    idle, as the pages ask ("CS149 L11: Programming Specialized Hardware",
//    section 4, slide 35), the two-group alternation that "Distilling a 4.5
//    hour CUDA talk", section 12, describes for its consumers.
//  * Scores are computed transposed, Sᵀ = K·Qᵀ, with 32x32x16 bf16 MFMAs:
//    A = a 32-key slab of K read from LDS, B = the wave's Q fragment held in
//    VGPRs for the whole loop. In the accumulator every lane holds one query
//    row (l % 32) and 16 keys, so the softmax row work is in-lane.
//  * Oᵀ += Vᵀ·Pᵀ: Pᵀ is the score accumulator converted to bf16 in place. The
//    keys a lane holds come in runs of four (rows 8*(r/4) + 4g + r%4), so the
//    MFMA k index 8g + e names key 8*(e/4) + 4g + e%4 of each 16-key chunk.
//    The Vᵀ operand is read from the row-major V tile with the LDS transpose
//    read (ds_read_b64_tr_b16) in exactly that key order.
//  * Softmax in base 2 with log2(e) folded into the scale on the host, and
//    one reciprocal per row at the end ("Distilling a 4.5 hour CUDA talk",
//    section 2 on the base-2 exponential and on reciprocal reuse; section 7
//    on folding log2(e) into the temperature). Each row's exponent reference
//    m is fixed from its first 32 keys: O = acc / l and lse = m + log2 l are
//    exact in real arithmetic for any m, so nothing is rescaled in the loop.
//    If some row's l leaves [0, 2^32] (a later key outscored the first ones by
//    a wide margin) the workgroup recomputes with exact row maxima.
//  * K/V staging: four-stage rings of K and of V, filled by LDS-DMA
//    (buffer_load ... lds, no VGPRs). Two copy groups (the four role-0 waves,
//    the four role-1 waves) take turns: in period T the group T % 2 copies
//    K(T+3) and V(T+2), one LDS-DMA after every fourth MFMA of its two MFMA
//    chains (the copy engine accepts them at about that pace; a burst would
//    stall the issuing wave), and waits for them (s_waitcnt vmcnt(0)) at the
//    end of period T+1. At d = 64 (half the MFMAs per period) the role-1
//    waves instead issue every copy, all of them at the start of their
//    period, during their softmax, and wait for them at its end, so the role-0
//    waves are never held by the copy issue. One barrier closes each period.
//    LDS-DMA writes 16
//    bytes per lane at consecutive addresses, so bank-conflict avoidance is
//    an XOR swizzle of the 16-byte chunks of a row, applied by choosing which
//    global chunk each lane fetches ("Distilling a 4.5 hour CUDA talk",
//    section 8).
//  * Causal: a wave stops computing after the last tile any of its rows
//    sees and only keeps its copy duty and the barriers until the
//    workgroup's last period.
#pragma once
#include <type_traits>

#include "rope.hpp"
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
    // dropout (kernels instantiated with DROP only): drop probability
    // drop_thr / 256, generator key (seed_lo, seed_hi), drop_scale =
    // 256 / (256 - drop_thr)
    uint32_t drop_thr, seed_lo, seed_hi;
    float drop_scale;
    // RoPE of Q at load (kernels instantiated with ROPE only): log2(base)
    double rope_log2_base;
    // main kernel: 0 (one work item per workgroup), or the number of items
    // each workgroup takes in turn (gridDim.x a multiple of 8)
    int32_t persist_rounds;
};

typedef short i16x2 __attribute__((ext_vector_type(2)));

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11): ten rounds of two 32x32 -> 64-bit products whose
// high halves are xored with the other two words and the key, the key
// advanced by the Weyl constants between rounds. Counter-based: the output
// depends only on (ctr, key), so any element's random bits can be produced
// where that element is.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // the full 64-bit products: one v_mad_u64_u32 each, where a high and
        // a low 32-bit multiply would take two slow-rate instructions
        const uint64_t p0 = (uint64_t)c[0] * 0xD2511F53u, p1 = (uint64_t)c[2] * 0xCD9E8D57u;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
    }
}

template <int D>
struct TileCfg {
    static constexpr int TQ = 256;           // query rows per workgroup
    static constexpr int TK = 64;            // keys per tile
    static constexpr int NWAVE = 8;
    static constexpr int ROWS = TQ / NWAVE;  // query rows per wave
    static constexpr int NT = 64 * NWAVE;    // threads per workgroup
    static constexpr int CPR = D / 8;        // 16-byte chunks per K or V row
    static constexpr int TILE = TK * D;      // elements of one K or V tile
    static constexpr int NSTAGE = 4;         // depth of the K ring and of the V ring
    static constexpr int LDS_BYTES = 2 * NSTAGE * TILE * 2;
    static constexpr int ROWS_PER_DMA = 64 / CPR;                 // rows per wave-wide DMA
    static constexpr int DMA_PER_COPIER = TK / ROWS_PER_DMA / 4;  // per tile, tensor and copying wave
    static constexpr int NKC = D / 16;       // k-steps of Sᵀ = K·Qᵀ
    static constexpr int NDB = D / 32;       // 32-column blocks of O
    static_assert(ROWS == 32, "one 32-row MFMA block per wave");
    static_assert(TK % (ROWS_PER_DMA * 4) == 0, "tile rows must split over a copy group");
    static_assert(LDS_BYTES <= 160 * 1024, "the rings must fit in LDS");
    static_assert(4 * DMA_PER_COPIER == 4 * NDB && 4 * DMA_PER_COPIER == 2 * NKC,
                  "one copy per four MFMAs of each chain");
};

template <int N>
using IC = std::integral_constant<int, N>;

template <int D, bool CAUSAL, typename TIn, bool DROP = false, bool ROPE = false>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(const KernelArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    using C = TileCfg<D>;
    constexpr int TQ = C::TQ, TK = C::TK, CPR = C::CPR, NKC = C::NKC, NDB = C::NDB;
    constexpr int NS = C::NSTAGE, DPC = C::DMA_PER_COPIER;
    // LDS fragment reads run PF MFMAs ahead of their use: enough that one
    // wave's chain is not held up by the LDS latency
    constexpr int PF = 4;
    __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[C::LDS_BYTES];
    __shared__ int wave_bad[C::NWAVE];
    __bf16 *const Kst = (__bf16 *)lds_raw;   // K ring
    __bf16 *const Vst = Kst + NS * C::TILE;  // V ring

    const int tid = threadIdx.x;
    int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int role = w >> 2, cw = w & 3;  // cw: this wave's share of its group's copies
    int l32 = lane & 31, g = lane >> 5;

    // ---- work item: heaviest causal tiles are dispatched first. Workgroups
    // go to the 8 XCDs round-robin by index; when the kv-head groups split
    // evenly over them, each XCD takes whole groups and runs the query heads
    // of a group on the same q-tile side by side, so they read the same K/V
    // tiles through that XCD's L2. ------------------------------------------
    // Persistent rounds: in round rnd the workgroups of an XCD take its next
    // gridDim / 8 items, in reversed order every other round, so that heavy
    // and light causal tiles pair up and every workgroup gets the same work.
    // (Not with RoPE, whose Q load needs the registers the loop would keep.)
    const int n_rounds = (!ROPE && a.persist_rounds > 0) ? a.persist_rounds : 1;
    const uint32_t n_items = gridDim.x * (uint32_t)n_rounds;
    for (int rnd = 0; rnd < n_rounds; ++rnd) {
    int b, h, qt;
    {
        const int n_groups = a.B * a.Hkv;
        uint32_t vbid = blockIdx.x;
        if (n_rounds > 1) {
            const uint32_t per_xcd = gridDim.x / 8, j = blockIdx.x / 8;
            const uint32_t jj = (rnd & 1) ? per_xcd - 1 - j : j;
            vbid = blockIdx.x % 8 + 8 * ((uint32_t)rnd * per_xcd + jj);
        }
        const int bid = work_index(vbid, n_items);
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
    const int wrow0 = q0 + C::ROWS * w;  // first query row of this wave
    const int row = wrow0 + l32;         // the query row of this lane
    const int kv_end = CAUSAL ? min(a.Nkv, q0 + TQ) : a.Nkv;
    const int n_tiles = (kv_end + TK - 1) / TK;  // >= 1; the workgroup's periods
    // tiles this wave computes: under the causal mask, tiles past its last
    // row hold no key any of its rows sees
    const int n_live = CAUSAL ? min(n_tiles, (wrow0 + C::ROWS - 1) / TK + 1) : n_tiles;
    // 32-key halves from this index on need the causal or key-range mask for
    // this wave's rows; tiles below n_plain have none
    const int first_masked_sub = CAUSAL ? min(wrow0 / 32, a.Nkv / 32) : a.Nkv / 32;
    const int n_plain = min(n_tiles, first_masked_sub / 2);

    // ---- Q fragment: B operand of Sᵀ = K·Qᵀ, resident for the whole loop ---
    bf16x8 qf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
        u32x4 v = {0, 0, 0, 0};
        if (row < a.Nq) v = load8_bf16(Qp + (int64_t)row * a.q_sn + 16 * kc + 8 * g);
        // RoPE on the way in: the chunk's four pairs start at pair 8kc + 4g
        // of the row, whose position is its index
        if constexpr (ROPE) v = rope_chunk(v, row, 8 * kc + 4 * g, D, a.rope_log2_base);
        qf[kc] = u32x4_as_bf16x8(v);
    }

    // ---- ring stages; S is a compile-time constant in the unrolled loop, so
    // stage offsets are instruction immediates ---------------------------------
    auto kst = [&](auto S) __attribute__((always_inline)) { return Kst + decltype(S)::value * C::TILE; };
    auto vst = [&](auto S) __attribute__((always_inline)) { return Vst + decltype(S)::value * C::TILE; };
    auto lds_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    auto wait_copies = [&]() __attribute__((always_inline)) {
        // a partial vmcnt does not order LDS-DMA writes; only zero is used
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    // ---- LDS-DMA of one K or V tile by one copy group. A window is 64 lanes
    // x 16 bytes = ROWS_PER_DMA rows; the group's wave cw fills windows cw,
    // cw + 4, ...; lane i of a window lands at chunk i and fetches the global
    // chunk that the swizzle puts there. bf16 inputs go through a buffer
    // resource that ends at the last key, so rows past the end read as zeros
    // (finite, and masked). ---------------------------------------------------
    int dma_r = lane / CPR;  // row within the window
    int dma_p = lane % CPR;  // physical chunk this lane fills
    // this lane's byte offset, within a tile, of window u of its share
    // (bf16 inputs); formed once per pass, like the LDS read addresses
    uint32_t voff_k[DPC], voff_v[DPC];
    auto form_copy_offsets = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < DPC; ++u) {
            const uint32_t r = (4 * u + cw) * C::ROWS_PER_DMA + dma_r;  // tile row
            voff_k[u] = (r * (uint32_t)a.k_sn + 8u * k_chunk<D>(r, dma_p)) * 2u;
            voff_v[u] = (r * (uint32_t)a.v_sn + 8u * v_chunk<D>(r, dma_p)) * 2u;
            asm volatile("" : "+v"(voff_k[u]), "+v"(voff_v[u]));
        }
    };
    // window u (0 .. DPC-1) of this wave's share of one tile
    // LDS byte address of the K and V rings (uniform)
    const uint32_t lds_k0 = __builtin_amdgcn_readfirstlane(lds_addr(Kst));
    const uint32_t lds_v0 = __builtin_amdgcn_readfirstlane(lds_addr(Vst));
    const int last_tile = (a.Nkv - 1) / TK;
    // Buffer resource over the rows of K or V tile `tile` that exist: a load
    // at a byte offset past the last existing row returns zeros. A tile past
    // the last one is replaced by the last tile (its copy lands in a stage
    // nobody reads before it is refilled). Scalar arithmetic only.
    auto tile_rsrc = [&](bool is_v, int tile) __attribute__((always_inline)) {
        const int32_t sn = is_v ? a.v_sn : a.k_sn;
        const int t = min(tile, last_tile);
        const uint32_t rows = (uint32_t)min(a.Nkv - t * TK, TK);
        const uint64_t gb = (uint64_t)(uintptr_t)(is_v ? Vp : Kp) +
                            (uint64_t)(uint32_t)t * ((uint64_t)(uint32_t)sn * (TK * 2));
        return u32x4{(uint32_t)gb, (uint32_t)(gb >> 32), rows * (uint32_t)sn * 2u, 0x00020000u};
    };
    // window u of this wave's share of a tile into the stage at LDS byte
    // offset stage_off of the K or V ring
    auto dma_one = [&](const u32x4 rsrc, bool is_v, uint32_t stage_off, int u) __attribute__((always_inline)) {
        // formed right here from one live register, not kept per copy
        uint32_t m0 = lds_k0 + (uint32_t)cw * 1024u;
        asm volatile("" : "+s"(m0));
        m0 += (is_v ? NS * C::TILE * 2 : 0) + stage_off + (uint32_t)(4 * u) * 1024u;
        // M0 (the LDS destination) is written inside the statement, and the
        // DMA is followed by a wait state (see dma16_buf_to_lds)
        perturb_pause();
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_nop 0"
                     :
                     : "s"(m0), "v"(is_v ? voff_v[u] : voff_k[u]), "s"(rsrc)
                     : "memory");
    };
    auto issue_one = [&](__bf16 *dst, bool is_v, int tile, int u) __attribute__((always_inline)) {
        const TIn *base = is_v ? Vp : Kp;
        const int32_t sn = is_v ? a.v_sn : a.k_sn;
        if constexpr (sizeof(TIn) == 2) {
            dma_one(tile_rsrc(is_v, tile), is_v,
                    (uint32_t)((char *)dst - (char *)(is_v ? Vst : Kst)), u);
        } else {
            // fp32 inputs: rounded to bf16 in registers, same LDS placement
            {
                const int win_id = 4 * u + cw;
                const int r = win_id * C::ROWS_PER_DMA + dma_r;
                const int key = min(tile * TK + r, a.Nkv - 1);  // clamped: a finite, masked row
                const int chunk = is_v ? v_chunk<D>(r, dma_p) : k_chunk<D>(r, dma_p);
                *(u32x4 *)(dst + win_id * 64 * 8 + 8 * lane) =
                    load8_bf16(base + (int64_t)key * sn + 8 * chunk);
            }
        }
    };
    auto issue = [&](__bf16 *dst, bool is_v, int tile) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < DPC; ++u) issue_one(dst, is_v, tile, u);
    };

    // ---- state -------------------------------------------------------------
    f32x16 oacc[NDB];  // Oᵀ: columns 32db + acc_row(r, g) of this lane's row
    float m = 0.f;     // the row's reference of the exponentials (score*c units)
    float l = 0.f;     // normalizer, partial over this lane's keys

    // LDS byte addresses of this lane's fragment reads in stage 0: K rows
    // l32 (and 32 + l32 at +32 rows) for each k-step, V transpose reads for
    // each column block. They are made opaque where they are formed (inside
    // the role branch), so that the compiler keeps these NKC + NDB registers
    // and puts every stage / row / key-chunk offset in the instruction's
    // 16-bit immediate instead of materialising an address per offset (the
    // V ring lies beyond 64 KiB).
    uint32_t kaddr[NKC], vaddr[NDB];
    auto form_addresses = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            kaddr[kc] = lds_addr(&k_frag_ptr<D>(Kst, l32, 2 * kc + g));
            asm volatile("" : "+v"(kaddr[kc]));
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            vaddr[db] = lds_addr(vt_read_ptr<D>(Vst, db, lane));
            asm volatile("" : "+v"(vaddr[db]));
        }
    };

    auto no_hook = [](int) {};
    // Sᵀ of one 64-key tile (K stage S): s[js] holds keys 32js .. 32js + 31
    auto scores = [&](f32x16 (&s)[2], auto S, auto hook) __attribute__((always_inline)) {
        constexpr uint32_t so = decltype(S)::value * C::TILE * 2;
#pragma unroll
        for (int js = 0; js < 2; ++js)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[js][r] = 0.f;
        constexpr int NF = 2 * NKC;  // fragment f: k-step f / 2 of half f % 2
        bf16x8 kf[NF];
        auto kread = [&](int f) __attribute__((always_inline)) {
            return lds_read_b128(kaddr[f >> 1] + so + (f & 1) * 32 * D * 2);
        };
#pragma unroll
        for (int f = 0; f < PF; ++f) kf[f] = kread(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (f + PF < NF) kf[f + PF] = kread(f + PF);
            s[f & 1] = mfma_32x32x16(kf[f], qf[f >> 1], s[f & 1]);
            // a scheduling boundary: keeps the fragment reads PF steps ahead
            // rather than all hoisted
            asm volatile("" ::);
            hook(f);
        }
        // at d = 64 (half the MFMAs per fragment read of d = 128) the
        // compiler is also told the order: PF reads, then one read after each
        // MFMA (measured +2-4 % on d = 64; at d = 128 the same order cost 2 %)
        if constexpr (D == 64 && sizeof(TIn) == 2) {
            __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);  // DS reads
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // an MFMA
                if (f + PF < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
    };
    // the causal / key-range mask on the scores of tile T: key j of this
    // lane's row is visible iff j < lim = min(row + 1, Nkv) (Nkv without
    // the causal mask). With j = 64T + 32js + acc_row(r, g) and acc_row(r, g)
    // = acc_row(r, 0) + 4g, one threshold per half and one compare against a
    // constant per element.
    auto mask = [&](f32x16 (&s)[2], int T) __attribute__((always_inline)) {
        const int lim = CAUSAL ? min(row + 1, a.Nkv) : a.Nkv;
#pragma unroll
        for (int js = 0; js < 2; ++js) {
            const int t = lim - (TK * T + 32 * js + 4 * g);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (acc_row(r, 0) >= t) s[js][r] = -INFINITY;
        }
    };
    // m from the row's first 32 keys (tile 0, masked)
    auto fix_m = [&](f32x16 (&s)[2]) __attribute__((always_inline)) {
        mask(s, 0);
        float x = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) x = fmaxf(x, fmaxf(s[0][r], s[0][r + 1]));
        x = xhalf_max(x) * a.c;
        m = (x == -INFINITY) ? 0.f : x;
    };
    // Dropout of the rounded P of tile T, after its row sum (the normalizer is
    // that of the softmax before dropout): element (row, key j) is kept when
    // its byte of Philox4x32-10 is >= drop_thr, with key (seed_lo, seed_hi),
    // counter (row, 2 (j / 32) + (j / 4) mod 2, b H_q + h, 0) and the byte
    // t = j mod 4 of output word (j / 8) mod 4. A lane's 16 keys of one
    // 32-key half are 8q + 4g + t (q, t < 4): one counter, all 16 bytes.
    // The kept values are scaled by 256 / (256 - drop_thr) at the end.
    const i16x2 thr2 = {(short)a.drop_thr, (short)a.drop_thr};
    auto drop = [&](uint32_t (&pk)[2][8], int T) __attribute__((always_inline)) {
#pragma unroll
        for (int js = 0; js < 2; ++js) {
            uint32_t w[4] = {(uint32_t)row, (uint32_t)(2 * (2 * T + js) + g),
                             (uint32_t)(b * a.Hq + h), 0u};
            philox4x32_10(w, a.seed_lo, a.seed_hi);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // elements 2j, 2j + 1: word j / 2, bytes 2 (j % 2) and 2 (j % 2) + 1,
                // moved to the two 16-bit halves; byte - thr < 0 (drop) sets
                // the half's sign, which the shift spreads over the half
                const uint32_t sel = (j & 1) ? 0x0C030C02u : 0x0C010C00u;
                const uint32_t bytes = __builtin_amdgcn_perm(0u, w[j >> 1], sel);
                const i16x2 diff = __builtin_bit_cast(i16x2, bytes) - thr2;
                const uint32_t drop_mask = __builtin_bit_cast(uint32_t, (i16x2)(diff >> (short)15));
                pk[js][j] &= ~drop_mask;
            }
        }
    };
    // p = 2^(s·c - m) (Map(exp)) rounded to bf16 into pk, and the partial row
    // sum of the rounded p (what P·V multiplies; Reduce(+)), two at a time
    // with v_dot2_f32_bf16 in independent partial sums
    auto softmax = [&](f32x16 (&s)[2], uint32_t (&pk)[2][8], int T, bool masked)
                       __attribute__((always_inline)) {
        if (masked) mask(s, T);
        const float negm = -m;
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int js = 0; js < 2; ++js) {
            float e[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) e[r] = exp2_hw(__builtin_fmaf(s[js][r], a.c, negm));
#pragma unroll
            for (int j = 0; j < 8; ++j) pk[js][j] = pack_bf16x2(e[2 * j], e[2 * j + 1]);
#pragma unroll
            for (int j = 0; j < 8; ++j) ls[j & 3] = sum_bf16x2(pk[js][j], ls[j & 3]);
        }
        l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
        if constexpr (DROP) drop(pk, T);
    };
    // Oᵀ += Vᵀ·Pᵀ over one tile (V stage at byte offset so); the 16-key chunk
    // kch of Pᵀ is pk[kch / 2][4 (kch % 2) .. + 3]
    // hook(f) runs after MFMA f (the copies issued between them)
    auto pv = [&](const uint32_t (&pk)[2][8], uint32_t so, auto hook) __attribute__((always_inline)) {
        constexpr int NF = 4 * NDB;  // fragment f: key chunk f / NDB, column block f % NDB
        bf16x8 vf[NF];
        auto vread = [&](int f) __attribute__((always_inline)) {
            return vt_frag_at<D>(vaddr[f % NDB] + so, f / NDB);
        };
#pragma unroll
        for (int f = 0; f < PF; ++f) vf[f] = vread(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (f + PF < NF) vf[f + PF] = vread(f + PF);
            const int kch = f / NDB;
            const u32x4 p = {pk[kch >> 1][4 * (kch & 1)], pk[kch >> 1][4 * (kch & 1) + 1],
                             pk[kch >> 1][4 * (kch & 1) + 2], pk[kch >> 1][4 * (kch & 1) + 3]};
            oacc[f % NDB] = mfma_32x32x16(vf[f], u32x4_as_bf16x8(p), oacc[f % NDB]);
            asm volatile("" ::);
            hook(f);
        }
        if constexpr (D == 64 && sizeof(TIn) == 2) {  // as in the scores: two reads per fragment
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 1);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                if (f + PF < NF) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
            }
        }
    };

    // ---- one pass over the keys: O, l for the references m ------------------
    // With set_m, m is first fixed from each row's first 32 keys; otherwise m
    // already holds the exact row maxima.
    auto pass = [&](auto ROLE, bool set_m) __attribute__((always_inline)) {
        constexpr int R = decltype(ROLE)::value;
        // an opaque copy of the lane index: the per-lane LDS and global
        // offsets derived from it are then computed inside this role's branch
        // and are not hoisted above it, where both roles' sets would be live
        const int saved[5] = {lane, l32, g, dma_r, dma_p};
        asm volatile("" : "+v"(lane), "+v"(l32), "+v"(g), "+v"(dma_r), "+v"(dma_p));
        form_addresses();
        if constexpr (sizeof(TIn) == 2) form_copy_offsets();
        l = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
        // prologue copies: group 0 brings K(0), V(0), K(2); group 1 K(1), V(1)
        if (R == 0) {
            issue(kst(IC<0>{}), false, 0);
            issue(vst(IC<0>{}), true, 0);
            if (n_tiles > 2) issue(kst(IC<2>{}), false, 2);
        } else if (n_tiles > 1) {
            issue(kst(IC<1>{}), false, 1);
            issue(vst(IC<1>{}), true, 1);
        }
        wait_copies();
        lds_barrier();
        f32x16 snext[2];       // role 1: scores of its next tile, across the period boundary
        uint32_t pprev[2][8];  // role 0: P of its previous tile, across the period boundary
        if (R == 1) {
            scores(snext, IC<0>{}, no_hook);
            if (set_m) fix_m(snext);
        }
        // period T (T < n_live, a tile this wave computes): role 0 runs
        // scores(T), P·V(T-1), softmax(T); role 1 softmax(T), P·V(T),
        // scores(T+1). Copies of K(T+3) and V(T+2): at d = 128 by group
        // T % 2, one LDS-DMA per four MFMAs of the period's two chains, so
        // that the copy engine is fed at its own pace instead of stalling a
        // wave on a burst, waited for at the end of period T+1; at d = 64 by
        // the role-1 waves in every period, all at its start (their softmax
        // has slack there), waited for at its end (measured: C2 +3-4 %, C4
        // and C3 -1.6 % with the same scheme).
        constexpr bool BURST = D == 64;
        auto copy_job = [&](auto PAR, int T, int j, const u32x4 &rk, const u32x4 &rv) __attribute__((always_inline)) {
            constexpr int P = decltype(PAR)::value;
            // window j of K(T+3) (j < DPC), else of V(T+2); no branch on
            // whether the tile exists (see tile_rsrc)
            if constexpr (sizeof(TIn) == 2) {
                if (j < DPC)
                    dma_one(rk, false, (P + 3) % NS * C::TILE * 2, j);
                else
                    dma_one(rv, true, (P + 2) % NS * C::TILE * 2, j - DPC);
            } else {
                if (j < DPC)
                    issue_one(kst(IC<(P + 3) % NS>{}), false, T + 3, j);
                else
                    issue_one(vst(IC<(P + 2) % NS>{}), true, T + 2, j - DPC);
            }
        };
        auto period = [&](auto PAR, int T) __attribute__((always_inline)) {
            constexpr int P = decltype(PAR)::value;          // T % NS
            constexpr bool copier = !BURST && (P & 1) == R;  // copies between the MFMAs
            const bool masked = T >= n_plain;
            u32x4 rk = {0, 0, 0, 0}, rv = {0, 0, 0, 0};
            if constexpr (copier && sizeof(TIn) == 2) rk = tile_rsrc(false, T + 3), rv = tile_rsrc(true, T + 2);
            if constexpr (BURST && R == 1) {
                if constexpr (sizeof(TIn) == 2) rk = tile_rsrc(false, T + 3), rv = tile_rsrc(true, T + 2);
#pragma unroll
                for (int j = 0; j < 2 * DPC; ++j) copy_job(PAR, T, j, rk, rv);
            }
            // P·V: jobs 0 .. DPC-1; scores: jobs DPC .. 2 DPC-1
            auto pv_hook = [&](int f) __attribute__((always_inline)) {
                if constexpr (copier)
                    if ((f & 3) == 3) copy_job(PAR, T, f >> 2, rk, rv);
            };
            auto sc_hook = [&](int f) __attribute__((always_inline)) {
                if constexpr (copier)
                    if ((f & 3) == 3) copy_job(PAR, T, DPC + (f >> 2), rk, rv);
            };
            if constexpr (R == 0) {
                // scores first, so that their results have drained from the
                // MFMA pipe (behind P·V) when the softmax reads them
                f32x16 s[2];
                scores(s, PAR, sc_hook);
                if (P != 0 || T > 0) {
                    pv(pprev, (P + NS - 1) % NS * C::TILE * 2, pv_hook);
                } else if constexpr (copier) {
#pragma unroll
                    for (int j = 0; j < DPC; ++j) copy_job(PAR, T, j, rk, rv);
                }
                if (T == 0 && set_m) fix_m(s);
                softmax(s, pprev, T, masked);
                // P and l complete before the barrier: the softmax overlaps
                // role 1's MFMAs of this period, not the next period's start
#pragma unroll
                for (int js = 0; js < 2; ++js)
                    asm volatile("" : "+v"(pprev[js][0]), "+v"(pprev[js][1]), "+v"(pprev[js][2]),
                                 "+v"(pprev[js][3]), "+v"(pprev[js][4]), "+v"(pprev[js][5]),
                                 "+v"(pprev[js][6]), "+v"(pprev[js][7]));
                asm volatile("" : "+v"(l));
            } else {
                uint32_t pk[2][8];
                softmax(snext, pk, T, masked);
                pv(pk, P * C::TILE * 2, pv_hook);
                // the next tile's scores; unused when that tile is not live
                // (its stage then holds finite stale data or zeros)
                scores(snext, IC<(P + 1) % NS>{}, sc_hook);
            }
            // at d = 128 the other group's copies of the previous period; at
            // d = 64 role 1's copies of this one
            if constexpr (BURST ? R == 1 : !copier) wait_copies();
            lds_barrier();
        };
        // period T >= n_live (causal: no key of the tile is visible to this
        // wave's rows): copy duty only, and role 0's P·V of its last tile
        auto tail_period = [&](auto PAR, int T) __attribute__((always_inline)) {
            constexpr int P = decltype(PAR)::value;
            constexpr bool copier = BURST ? R == 1 : (P & 1) == R;
            if (R == 0 && T == n_live) pv(pprev, (P + NS - 1) % NS * C::TILE * 2, no_hook);
            if constexpr (copier) {
                u32x4 rk = {0, 0, 0, 0}, rv = {0, 0, 0, 0};
                if constexpr (sizeof(TIn) == 2) rk = tile_rsrc(false, T + 3), rv = tile_rsrc(true, T + 2);
#pragma unroll
                for (int j = 0; j < 2 * DPC; ++j) copy_job(PAR, T, j, rk, rv);
            }
            if constexpr (BURST ? R == 1 : !copier) wait_copies();
            lds_barrier();
        };
        for (int T = 0; T < n_live; T += NS) {
            period(IC<0>{}, T);
            if (T + 1 < n_live) period(IC<1>{}, T + 1);
            if (T + 2 < n_live) period(IC<2>{}, T + 2);
            if (T + 3 < n_live) period(IC<3>{}, T + 3);
        }
        for (int T = n_live & ~(NS - 1); T < n_tiles; T += NS) {
            if (T >= n_live) tail_period(IC<0>{}, T);
            if (T + 1 >= n_live && T + 1 < n_tiles) tail_period(IC<1>{}, T + 1);
            if (T + 2 >= n_live && T + 2 < n_tiles) tail_period(IC<2>{}, T + 2);
            if (T + 3 >= n_live && T + 3 < n_tiles) tail_period(IC<3>{}, T + 3);
        }
        if (R == 0 && n_live == n_tiles) pv(pprev, (n_tiles - 1) % NS * C::TILE * 2, no_hook);
        wait_copies();  // no copy outlives the pass
        lane = saved[0], l32 = saved[1], g = saved[2], dma_r = saved[3], dma_p = saved[4];
    };

    // ---- fast pass with m fixed by each row's first 32 keys; if some row's
    // normalizer leaves [0, 2^32] (every p <= 2^32 when it does not), the
    // exact row maxima are found and the pass runs again (rare) -----------
    constexpr float kMaxL = 4294967296.0f;
    float l_row;
    for (bool exact = false;; exact = true) {
        if (role == 0)
            pass(IC<0>{}, !exact);
        else
            pass(IC<1>{}, !exact);
        l_row = xhalf_sum(l);
        if (exact) {
            lds_barrier();  // every wave is done with the rings (the epilogue reuses them)
            break;
        }
        const bool bad = !(l_row <= kMaxL);  // also catches inf and NaN
        // the ballot runs in every lane (inside `lane == 0` it would see
        // lane 0's row only); lane 0 then publishes the wave's verdict
        const bool any_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
        if (lane == 0) wave_bad[w] = any_bad;
        lds_barrier();
        bool wg_bad = false;
#pragma unroll
        for (int i = 0; i < C::NWAVE; ++i) wg_bad |= wave_bad[i] != 0;
        if (!wg_bad) break;
        float M = -INFINITY;
        form_addresses();
        for (int T = 0; T < n_tiles; ++T) {
            lds_barrier();  // the previous tile's K stage is no longer read
            if (role == 0) issue(kst(IC<0>{}), false, T);
            wait_copies();
            lds_barrier();
            if (T < n_live) {
                f32x16 s[2];
                scores(s, IC<0>{}, no_hook);
                mask(s, T);
                float x = -INFINITY;
#pragma unroll
                for (int js = 0; js < 2; ++js)
#pragma unroll
                    for (int r = 0; r < 16; ++r) x = fmaxf(x, s[js][r]);
                M = fmaxf(M, xhalf_max(x) * a.c);
            }
        }
        lds_barrier();  // K stage 0 and wave_bad are free again
        m = (M == -INFINITY) ? 0.f : M;
    }

    // ---- O = Oᵀ / l (one reciprocal per row), logsumexp ---------------------
    const float inv_l = DROP ? a.drop_scale / l_row : 1.0f / l_row;
    if constexpr (sizeof(TIn) == 2) {
        // Through LDS (every wave is past its last read of the rings): each
        // lane writes its row's 4-column runs to this wave's 32-row block,
        // then each store covers whole rows (D / 8 lanes x 16 bytes a row)
        // instead of 8 bytes in each of 32 rows. Rows are unpadded; the
        // 16-byte chunk of a run is XORed with row bits (1..3 at D = 64, 0..3
        // at D = 128) and its 8-byte half with row bit 4, so the 32 lanes of
        // a write pass reach every bank once and a row's chunks stay a
        // permutation for the reads.
        constexpr int CPRS = D / 8;                        // 16-byte chunks per row
        auto swz = [](int r) { return D >= 128 ? (r & 15) : ((r >> 1) & 7); };
        static_assert(C::NWAVE * C::ROWS * D * 2 <= C::LDS_BYTES, "the staged O fits in the rings");
        __bf16 *const stg = Kst + w * C::ROWS * D;
        // opaque copies of the lane index: the staging addresses are formed
        // here, not hoisted out of the item loop to stay live through it
        int el = lane;
        asm volatile("" : "+v"(el));
        const int el32 = el & 31, eg = el >> 5;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int ch = (4 * db + rr) ^ swz(el32), hf = eg ^ ((el32 >> 4) & 1);
                *(u32x2 *)(stg + el32 * D + 8 * ch + 4 * hf) =
                    u32x2{pack_bf16x2(oacc[db][4 * rr] * inv_l, oacc[db][4 * rr + 1] * inv_l),
                          pack_bf16x2(oacc[db][4 * rr + 2] * inv_l, oacc[db][4 * rr + 3] * inv_l)};
            }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        constexpr int RPI = 64 / CPRS;  // rows per store
        const int rl = el / CPRS, cl = el % CPRS;
#pragma unroll
        for (int i = 0; i < C::ROWS / RPI; ++i) {
            const int r = i * RPI + rl;
            u32x4 v = *(const u32x4 *)(stg + r * D + 8 * (cl ^ swz(r)));
            if ((r >> 4) & 1) v = u32x4{v[2], v[3], v[0], v[1]};
            if (wrow0 + r < a.Nq) *(u32x4 *)(Op + (int64_t)(wrow0 + r) * a.o_sn + 8 * cl) = v;
        }
        if (row < a.Nq && g == 0 && a.lse)
            a.lse[((int64_t)b * a.Hq + h) * a.Nq + row] = (m + log2f(l_row)) * 0.69314718055994531f;
        if (rnd + 1 < n_rounds) lds_barrier();  // the next item's first copies reuse the rings
    } else if (row < a.Nq) {
        TIn *orow = Op + (int64_t)row * a.o_sn;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int col = 32 * db + acc_row(4 * rr, g);
                store4(orow + col, oacc[db][4 * rr] * inv_l, oacc[db][4 * rr + 1] * inv_l,
                       oacc[db][4 * rr + 2] * inv_l, oacc[db][4 * rr + 3] * inv_l);
            }
        if (g == 0 && a.lse)
            a.lse[((int64_t)b * a.Hq + h) * a.Nq + row] = (m + log2f(l_row)) * 0.69314718055994531f;
    }
    // the next item's prologue copies overwrite the ring: every wave is past
    // the fallback check's barrier, after its last read of this item's tiles
    }  // work items
#endif
}

}  // namespace attn
