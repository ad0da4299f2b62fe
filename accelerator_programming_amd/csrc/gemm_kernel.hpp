// bf16 GEMM C = A·Bᵀ for gfx950 on the attention kernel's tile layer.
//
// A is [M, K] and B is [N, K], both row-major with K contiguous (the layout
// of activations and of [out, in] weights, so the Q/K/V and O projections on
// either side of attention are C = X·Wᵀ); C is [M, N] row-major bf16, with
// fp32 accumulation and one round-to-nearest-even at the end.
//
// Decomposition ("Distilling a 4.5 hour CUDA talk", section 5, blocking):
// every workgroup owns a disjoint 256 x 256 tile of C and privately streams
// the slabs of A and B it needs, so no two workgroups touch the same output
// and nothing synchronizes between them; the tile is as large as the
// workgroup's accumulators and LDS ring allow (output work grows with the
// tile's area, input traffic with its perimeter). The same passage's super-blocked
// launch order is used for L2 reuse: each XCD (own L2) takes a contiguous run
// of tiles, walked in groups of 8 tile-rows so that neighbouring workgroups
// share slabs of A and of B. The K loop is the inner loop of the
// matrix-multiply metapipeline of "CS149 L11: Programming Specialized
// Hardware" (slides 51-53): a slab of A and a slab of B are staged on chip,
// multiplied into the accumulators, and the next slabs stream in meanwhile.
//
// gfx950 mapping
//  * 8 waves, two per SIMD, so that one wave's barrier and LDS waits are
//    covered by the other's MFMAs; wave (wm, wn) owns C rows 128wm .. +127
//    and columns 64wn .. +63 of the tile as 2 x 4 accumulators of 32 x 32
//    (128 registers). With one wave per SIMD and 128 x 128 per wave the
//    kernel ran 2-4 % slower on the projection shapes.
//  * Cᵀ blocks are computed, Cᵀ = B·Aᵀ, with v_mfma_f32_32x32x16_bf16: the A
//    operand is a 32-row slab of B, the B operand a 32-row slab of A, both
//    read from LDS as 16 contiguous bytes per lane. A lane then holds one row
//    of C and runs of four consecutive columns. When C's rows allow 16-byte
//    stores, each wave writes its 128 x 64 block into the idle LDS ring
//    first and stores 8 rows of 128 contiguous bytes per instruction (16
//    bytes in each of 32 rows otherwise).
//  * K steps of 32: A and B slabs (256 x 32 bf16 = 16 KB each) go through a
//    four-stage LDS ring (128 KB) by LDS-DMA (buffer_load ... lds). Two copy
//    groups (waves 0-3, waves 4-7) alternate: in step t the group t mod 2
//    copies the slabs of step t+3, one LDS-DMA after every second MFMA, and
//    waits for them (vmcnt(0)) at the end of step t+1; one barrier per step.
//  * LDS rows are 64 bytes (4 chunks of 16); chunk c of row r is stored at
//    c XOR ((r / 4) mod 4), so the 16 lanes a ds_read_b128 serves per pass
//    (16 consecutive rows, one chunk) hit 16 distinct 16-byte bank groups.
//  * Ragged edges: the buffer resources end at the last existing row of the
//    slab, so rows past M or N read as zeros; K chunks past K are given an
//    out-of-range offset, so they read as zeros too; stores are guarded.
#pragma once
#include <type_traits>

#include "tile.hpp"

namespace attn {

template <int N>
using GIC = std::integral_constant<int, N>;

struct GemmArgs {
    const __bf16 *a, *b;
    __bf16 *c;
    int32_t M, N, K;
    int32_t lda, ldb, ldc;  // row strides in elements
    int32_t tiles_m, tiles_n;
    int32_t stage_c;  // C rows 16-byte aligned (ldc % 8 == 0, C % 16 == 0): stores go through LDS
};

struct GemmCfg {
    static constexpr int BM = 256, BN = 256, BK = 32;
    static constexpr int NWAVE = 8, NT = 64 * NWAVE;
    static constexpr int WM = 128, WN = 64;        // per-wave C tile
    static constexpr int NB = WN / 32;             // 32-column blocks per wave
    static constexpr int NSTAGE = 4;
    static constexpr int SLAB = BM * BK;           // elements of one A (or B) slab
    static constexpr int STAGE_BYTES = 2 * SLAB * 2;
    static constexpr int RING_BYTES = NSTAGE * STAGE_BYTES;  // 128 KB
    // the epilogue stages each wave's 128 x 64 block of C in LDS (the ring is
    // idle by then), 128-byte rows
    static constexpr int CROW_B = 2 * 64;
    static constexpr int STAGE_C_BYTES = NWAVE * 128 * CROW_B;
    static constexpr int LDS_BYTES = RING_BYTES > STAGE_C_BYTES ? RING_BYTES : STAGE_C_BYTES;
    // LDS-DMA windows of 64 lanes x 16 B = 16 rows of 64 B; a slab is 16
    // windows, so one step's A and B slabs are 32 windows, 16 per wave of the
    // copying group
    static constexpr int WIN_PER_SLAB = BM * BK * 2 / 1024;
    static constexpr int DMA_PER_WAVE = 2 * WIN_PER_SLAB / (NWAVE / 2);
    static_assert(BM == BN, "A and B slabs share one shape");
    static_assert(LDS_BYTES <= 160 * 1024, "the ring must fit in LDS");
};

// physical 16-byte chunk of logical chunk c (0..3) in slab row r
__device__ __forceinline__ int gemm_chunk(int r, int c) { return c ^ ((r >> 2) & 3); }

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_bf16_nt_kernel(const GemmArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = GemmCfg;
    constexpr int BM = C::BM, BK = C::BK, NS = C::NSTAGE, DPW = C::DMA_PER_WAVE;
    __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[C::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w & 1, wn = w >> 1;  // wn 0..3
    const int l32 = lane & 31, g = lane >> 5;

    // ---- tile of this workgroup: XCD-contiguous runs, 8-row super-blocks ----
    int tm, tn;
    {
        const int T = a.tiles_m * a.tiles_n;
        const int bid = work_index(blockIdx.x, gridDim.x);
        int t = bid;
        if (T % 8 == 0) t = (bid % 8) * (T / 8) + bid / 8;
        constexpr int GM = 8;
        const int per_group = GM * a.tiles_n;
        const int first_m = (t / per_group) * GM;
        const int gsize = min(a.tiles_m - first_m, GM);
        const int r = t % per_group;
        tm = first_m + r % gsize;
        tn = r / gsize;
    }
    const int m0 = tm * BM, n0 = tn * C::BN;

    // ---- copy set-up: buffer resources over the slab rows that exist ----
    const int rows_a = min(a.M - m0, BM), rows_b = min(a.N - n0, BM);
    const uint64_t abase = (uint64_t)(uintptr_t)(a.a + (int64_t)m0 * a.lda);
    const uint64_t bbase = (uint64_t)(uintptr_t)(a.b + (int64_t)n0 * a.ldb);
    const uint32_t abytes = ((uint32_t)(rows_a - 1) * (uint32_t)a.lda + (uint32_t)a.K) * 2u;
    const uint32_t bbytes = ((uint32_t)(rows_b - 1) * (uint32_t)a.ldb + (uint32_t)a.K) * 2u;
    const int n_steps = (a.K + BK - 1) / BK;
    const int cw = w & 3;        // this wave's quarter of its group's windows
    const int group = w >> 2;    // copy group: copies in steps t with t % 2 == group
    // lane i of a window fills slab row 16 * win + i / 4 at physical chunk
    // i % 4, fetching the logical chunk the swizzle puts there
    const int dr = lane >> 2, dp = lane & 3;
    uint32_t voff[DPW];  // byte offset within the slab, per window of this wave
    int kch[DPW];        // element offset in K of the fetched chunk
#pragma unroll
    for (int u = 0; u < DPW; ++u) {
        const int win = 4 * u + cw;                    // 0..31: A windows 0..15, B 16..31
        const int row = 16 * (win & 15) + dr;
        const int c = gemm_chunk(row, dp);
        const int ld = win < 16 ? a.lda : a.ldb;
        voff[u] = ((uint32_t)row * (uint32_t)ld + 8u * c) * 2u;
        kch[u] = 8 * c;
    }
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_raw));
    // slabs of step t into stage t mod NS; K chunks past K get an offset past
    // every resource, so they read as zeros
    auto copy_one = [&](int t, int u) __attribute__((always_inline)) {
        const int win = 4 * u + cw;
        const bool is_b = win >= 16;
        const uint32_t k0 = (uint32_t)t * BK;
        const uint64_t base = (is_b ? bbase : abase) + (uint64_t)k0 * 2u;
        const uint32_t nrec = (is_b ? bbytes : abytes) - min(k0 * 2u, is_b ? bbytes : abytes);
        // uniform values, held in scalar registers for the resource
        const u32x4 rsrc = {(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base),
                            (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)),
                            (uint32_t)__builtin_amdgcn_readfirstlane(nrec), 0x00020000u};
        const uint32_t off = ((int)k0 + kch[u] < a.K) ? voff[u] : 0x80000000u;
        uint32_t m0v = lds0 + (uint32_t)(t % NS) * C::STAGE_BYTES;
        asm volatile("" : "+s"(m0v));
        m0v = __builtin_amdgcn_readfirstlane(m0v + (uint32_t)win * 1024u);
        // M0 (the LDS destination) is written inside the statement, and the
        // DMA is followed by a wait state (see dma16_buf_to_lds in tile.hpp)
        perturb_pause();
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_nop 0"
                     :
                     : "s"(m0v), "v"(off), "s"(rsrc)
                     : "memory");
    };
    auto wait_copies = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    auto barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- fragment addresses: B rows (A operand) and A rows (B operand) ----
    // block i of this wave's 128 rows, k-substep kk: row 32i + l32, chunk 2kk + g
    constexpr int NB = C::NB;
    uint32_t fa[4][2], fb[NB][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int ra = C::WM * wm + 32 * i + l32;
            fa[i][kk] = lds0 + (uint32_t)(ra * 64 + 16 * gemm_chunk(ra, 2 * kk + g));
        }
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int rb = C::WN * wn + 32 * i + l32;
            fb[i][kk] = lds0 + (uint32_t)(C::SLAB * 2 + rb * 64 + 16 * gemm_chunk(rb, 2 * kk + g));
        }

    f32x16 acc[NB][4];  // acc[nb][mb]: Cᵀ block of columns 32nb.., rows 32mb..
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // ---- prologue: group 0 copies steps 0 and 2, group 1 step 1 ----
    if (group == 0) {
#pragma unroll
        for (int u = 0; u < DPW; ++u) copy_one(0, u);
        if (n_steps > 2)
#pragma unroll
            for (int u = 0; u < DPW; ++u) copy_one(2, u);
    } else if (n_steps > 1) {
#pragma unroll
        for (int u = 0; u < DPW; ++u) copy_one(1, u);
    }
    wait_copies();
    barrier();

    // ---- K loop. The fragments of a k-substep are read one substep ahead
    // (two register sets), and those of the next step's first substep at the
    // end of this step: that stage was published by the barrier of the step
    // before, so only the copy ring needs the barrier that closes a step.
    // Two steps per iteration, so that whether this wave copies in a step is
    // known at compile time (COPIER). Past the last step the copy re-reads
    // the last step's slabs (the same bytes) into that step's stage.
    bf16x8 xa[2][4], xb[2][NB];
    auto load = [&](int set, uint32_t so, int kk) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xa[set][i] = lds_read_b128(fa[i][kk] + so);
#pragma unroll
        for (int i = 0; i < NB; ++i) xb[set][i] = lds_read_b128(fb[i][kk] + so);
    };
    auto mma = [&](int set, int tc, int kk, auto COPIER) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[i][j] = mfma_32x32x16(xb[set][i], xa[set][j], acc[i][j]);
                if constexpr (decltype(COPIER)::value)
                    if ((j & 1) == 1) copy_one(tc, 4 * kk + 2 * i + (j >> 1));
            }
    };
    auto step = [&](int t, auto COPIER) __attribute__((always_inline)) {
        const uint32_t so = (uint32_t)(t % NS) * C::STAGE_BYTES;
        const uint32_t so_next = (uint32_t)((t + 1) % NS) * C::STAGE_BYTES;
        const int tc = min(t + 3, n_steps - 1);
        load(1, so, 1);
        __builtin_amdgcn_sched_barrier(0);
        mma(0, tc, 0, COPIER);
        __builtin_amdgcn_sched_barrier(0);
        load(0, so_next, 0);  // unused after the last step (a finite stage)
        __builtin_amdgcn_sched_barrier(0);
        mma(1, tc, 1, COPIER);
        if constexpr (!decltype(COPIER)::value) wait_copies();  // this group's copies of step t-1
        barrier();
    };
    auto k_loop = [&](auto G) __attribute__((always_inline)) {
        constexpr int GR = decltype(G)::value;
        load(0, 0, 0);
        for (int t = 0; t < n_steps; t += 2) {
            step(t, std::integral_constant<bool, GR == 0>{});
            if (t + 1 < n_steps) step(t + 1, std::integral_constant<bool, GR == 1>{});
        }
    };
    if (group == 0)
        k_loop(GIC<0>{});
    else
        k_loop(GIC<1>{});
    wait_copies();  // no copy outlives the workgroup

    // ---- epilogue -------------------------------------------------------------
    if (a.stage_c) {
        // Through LDS, once every wave's copies have landed (the barrier):
        // each lane writes its row's runs of four columns to this wave's
        // 128-row block, then each store covers 8 rows of 128 contiguous bytes
        // instead of 16 bytes in each of 32 rows.
        barrier();
        static_assert(C::WM == 128 && C::WN == 64, "the staged block is 128 x 64");
        // the 16-byte chunk of a run is XORed with row bits 1..3 and its
        // 8-byte half with row bit 4: the 32 lanes of a write pass reach
        // every bank once, and a row's chunks stay a permutation for the reads
        auto swz = [](int r) { return (r >> 1) & 7; };
        unsigned char *const stg = lds_raw + w * 128 * C::CROW_B;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int r = 32 * j + l32;
                    const int ch = (4 * i + rr) ^ swz(r), hf = g ^ ((r >> 4) & 1);
                    *(u32x2 *)(stg + r * C::CROW_B + 16 * ch + 8 * hf) =
                        u32x2{pack_bf16x2(acc[i][j][4 * rr], acc[i][j][4 * rr + 1]),
                              pack_bf16x2(acc[i][j][4 * rr + 2], acc[i][j][4 * rr + 3])};
                }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int rl = lane >> 3, cl = lane & 7;  // 8 lanes x 16 bytes per row
        const int col = n0 + C::WN * wn + 8 * cl;
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int r = 8 * it + rl;
            u32x4 v = *(const u32x4 *)(stg + r * C::CROW_B + 16 * (cl ^ swz(r)));
            if ((r >> 4) & 1) v = u32x4{v[2], v[3], v[0], v[1]};
            const int row = m0 + C::WM * wm + r;
            if (row < a.M && col < a.N) {
                __bf16 *p = a.c + (int64_t)row * a.ldc + col;
                if (col + 8 <= a.N)
                    *(u32x4 *)p = v;
                else
                    *(u32x2 *)p = u32x2{v[0], v[1]};  // N is a multiple of 4
            }
        }
    } else {
    // C row m0 + 128wm + 32mb + l32, columns in runs of four
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = m0 + C::WM * wm + 32 * j + l32;
        if (row >= a.M) continue;
        __bf16 *crow = a.c + (int64_t)row * a.ldc;
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int col = n0 + C::WN * wn + 32 * i + acc_row(4 * rr, g);
                if (col < a.N)
                    store4(crow + col, acc[i][j][4 * rr], acc[i][j][4 * rr + 1],
                           acc[i][j][4 * rr + 2], acc[i][j][4 * rr + 3]);
            }
    }
    }
#endif
}

}  // namespace attn
