// Tile layer for gfx950 (CDNA4): bf16 MFMA fragments, wave64 row reductions,
// bf16 packing, and the global/LDS moves the attention kernel is built from.
//
// The pages treat a small matrix tile as the primitive type and name the two
// contractions attention needs, A·Bᵀ for Q·Kᵀ and A·B for P·V with V read in
// transposed form ("Distilling a 4.5 hour CUDA talk", section 10, register
// tiles). On gfx950 the native shape is the 32x32x16 bf16 MFMA with fp32
// accumulation, so that is the tile here; the operands live in VGPRs.
//
// Fragment layout of v_mfma_f32_32x32x16_bf16 (wave64), for C = A·B with A
// 32xK16, B K16x32, lane l, half g = l / 32:
//   A operand: 8 bf16 of row (l % 32), k = 8g .. 8g+7 (the same k numbering
//              as B, so any consistent in-lane k order contracts correctly);
//   B operand: 8 bf16 of column (l % 32), the same k range;
//   C (16 fp32): column (l % 32), rows 8*(r/4) + 4g + (r%4) for r = 0..15.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// C += A·B on one 32x32x16 bf16 tile, fp32 accumulate.
__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8 a, const bf16x8 b, const f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// C += A·B on one 16x16x32 bf16 tile, fp32 accumulate. Lane l, quarter
// G = l / 16: A = 8 bf16 of row (l % 16), k = 8G .. 8G+7; B = 8 bf16 of
// column (l % 16), the same k range; C (4 fp32) = column (l % 16), rows
// 4G .. 4G+3.
__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8 a, const bf16x8 b, const f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator held in register r by a lane of half g.
__device__ __forceinline__ constexpr int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// Combine a value with the one held by lane l ^ 32 (the other half of the
// wave): one v_permlane32_swap, no LDS traffic.
__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x on the transcendental unit (v_exp_f32). exp2(-inf) = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16, round to nearest even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// acc + lo + hi of a packed bf16 pair, in fp32 (one v_dot2_f32_bf16 with 1, 1).
__device__ __forceinline__ float sum_bf16x2(uint32_t pair, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

__device__ __forceinline__ bf16x8 u32x4_as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight consecutive elements starting at p, as bf16 (16 bytes). fp32 inputs
// are rounded to bf16 here, once, on their way on chip.
__device__ __forceinline__ u32x4 load8_bf16(const __bf16 *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ u32x4 load8_bf16(const float *p) {
    const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
    return u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                 pack_bf16x2(b[2], b[3])};
}

// Stores of four consecutive output values.
__device__ __forceinline__ void store4(__bf16 *p, float a, float b, float c, float d) {
    *(u32x2 *)p = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
    *(f32x4 *)p = f32x4{a, b, c, d};
}

// ---------------------------------------------------------------------------
// LDS tile layouts. K and V tiles are row-major, D bf16 per row, no padding;
// the 16-byte chunks of each row are XOR-permuted ("Distilling a 4.5 hour CUDA
// talk", section 8: a swizzle is an invertible permutation within a row that
// spreads the accesses a layout sees across banks, XOR being its own inverse).
// ---------------------------------------------------------------------------

// Physical chunk of logical chunk c in K row r. LDS has 64 banks of 4 bytes,
// so 16-byte chunk p of row r lands in bank group (r * D / 8 + p) mod 16, and
// a ds_read_b128 serves 16 lanes at a time: the 16 rows an A-fragment read
// touches in one pass must fill the 16 groups. At D = 128 a row is one whole
// 256-byte bank line and the XOR with r mod 16 does that. At D = 64 two rows
// share a line (group 8 (r mod 2) + p), so the XOR takes (r / 2) mod 8: rows of
// one parity then get 8 different chunks (r mod 8 would give rows r and r + 8
// the same group). Rows r and r + 32 always get the same XOR.
template <int D>
__device__ __forceinline__ int k_chunk(int r, int c) {
    constexpr int rows_per_line = (D >= 128) ? 1 : 128 / D;
    return c ^ ((r / rows_per_line) & (D / 8 - 1));
}

// Physical chunk of logical chunk c in V row r. A transpose read covers four
// consecutive rows x 32 bytes per 16 lanes (x 64 bytes per 32 lanes); the XOR
// value 2q + 8*parity(q), q = r % 4, keeps both windows conflict-free.
template <int D>
__device__ __forceinline__ int v_chunk(int r, int c) {
    const int q = r & 3;
    const int f = (D >= 128) ? (2 * q + 8 * ((q ^ (q >> 1)) & 1)) : 2 * q;
    return c ^ f;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

// A operand of Sᵀ = K·Qᵀ: K row kr, d = 16kc + 8g .. +7 (one ds_read_b128).
template <int D>
__device__ __forceinline__ bf16x8 k_frag(const __bf16 *Ks, int kr, int kc, int g) {
    return *(const bf16x8 *)(Ks + kr * D + 8 * k_chunk<D>(kr, 2 * kc + g));
}

// Where k_frag(Ks, kr, 0, g) reads: the first 16 bytes of that fragment.
template <int D>
__device__ __forceinline__ const __bf16 &k_frag_ptr(const __bf16 *Ks, int kr, int g) {
    return Ks[kr * D + 8 * k_chunk<D>(kr, g)];
}

// A operand of Oᵀ = Vᵀ·Pᵀ for output columns 32db .. 32db+31 and the 16-key
// chunk kc: lane l gets column 32db + l%32 at keys 16kc + 8(e/4) + 4g + e%4,
// e = 0..7 (the Pᵀ key order), from two ds_read_b64_tr_b16. Within each
// 16-lane group that instruction returns, to lane i, element i%4 of the
// 8-byte reads of lanes i/4, i/4+4, i/4+8, i/4+12; so lane s of the group
// points at row 4(s/4)-block, columns 4(s%4) .. +3.
template <int D>
__device__ __forceinline__ bf16x8 vt_frag(const __bf16 *Vs, int db, int kc, int lane) {
    const int G = lane >> 4, i16 = lane & 15, g = lane >> 5;
    i16x4 half[2];
#pragma unroll
    for (int hr = 0; hr < 2; ++hr) {
        const int vr = 16 * kc + 8 * hr + 4 * g + (i16 >> 2);
        const int col = 32 * db + 16 * (G & 1) + 4 * (i16 & 3);
        const __bf16 *src = Vs + vr * D + 8 * v_chunk<D>(vr, col >> 3) + (col & 7);
        half[hr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(src));
    }
    const i16x8 v8 = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v8);
}

// Where the first of vt_frag(Vs, db, 0, lane)'s transpose reads points.
template <int D>
__device__ __forceinline__ const __bf16 *vt_read_ptr(const __bf16 *Vs, int db, int lane) {
    const int G = lane >> 4, i16 = lane & 15, g = lane >> 5;
    const int vr = 4 * g + (i16 >> 2);
    const int col = 32 * db + 16 * (G & 1) + 4 * (i16 & 3);
    return Vs + vr * D + 8 * v_chunk<D>(vr, col >> 3) + (col & 7);
}

// LDS byte address of an LDS location (the 32-bit address DS instructions take).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(lds_void *)p;
}

// 16 bytes from LDS byte address a (one ds_read_b128).
__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t a) {
    return *(const __attribute__((address_space(3))) bf16x8 *)(uintptr_t)a;
}

// vt_frag(Vs, db, kc, lane) from the address p = vt_read_ptr(Vs, db, lane) as
// an LDS byte address: the key chunk only moves the address by whole rows.
template <int D>
__device__ __forceinline__ bf16x8 vt_frag_at(uint32_t p, int kc) {
    i16x4 half[2];
#pragma unroll
    for (int hr = 0; hr < 2; ++hr)
        half[hr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(uintptr_t)(p + (16 * kc + 8 * hr) * D * 2));
    const i16x8 v8 = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v8);
}

// ---------------------------------------------------------------------------
// Timing perturbation, for test builds only. A library compiled with
// -DATTN_PERTURB=<seed> runs every kernel with its workgroups taking their
// work items in a seeded permuted order and with a pseudo-random pause of up
// to 7 s_sleeps before every LDS-DMA of the main kernel and the GEMM, and
// before every tile copy (a burst of DMAs) of the wide-head and split-KV
// kernels (one pause per DMA there raised the V-in-K kernel above its
// register budget). Arithmetic and data placement are
// unchanged, so such a build must reproduce the normal build's outputs bit
// for bit; it exists so that the parity tests also run with the copies,
// waits and barriers pulled out of their usual timing.
// ---------------------------------------------------------------------------
#ifdef ATTN_PERTURB
// work item of workgroup bid: (bid * p + seed) mod grid with p a prime above
// 2^32, so a bijection of [0, grid) for every grid size
__device__ __forceinline__ uint32_t work_index(uint32_t bid, uint32_t grid) {
    return (uint32_t)(((uint64_t)bid * 4294967311ull + (uint64_t)(ATTN_PERTURB)) % (uint64_t)grid);
}
__device__ __forceinline__ void perturb_pause() {
    uint32_t h = __builtin_amdgcn_readfirstlane(blockIdx.x * 0x9E3779B9u ^ (threadIdx.x >> 6) * 0x85EBCA6Bu) ^
                 (uint32_t)__builtin_amdgcn_s_memtime();
    h ^= h >> 16;
    h *= 0x7FEB352Du;
    h ^= h >> 15;
    h *= 0x846CA68Bu;
    h ^= h >> 16;
    const uint32_t n = __builtin_amdgcn_readfirstlane(h & 7u);
    for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(2);
}
#else
__device__ __forceinline__ uint32_t work_index(uint32_t bid, uint32_t) { return bid; }
__device__ __forceinline__ void perturb_pause() {}
#endif

// LDS-DMA: 16 bytes from gptr (per lane) into LDS at lds_base + 16 * lane,
// lds_base wave-uniform (it goes through M0). Issued as inline assembly so
// that the compiler does not treat it as a store that every later LDS read
// might alias (which would put a vmcnt(0) wait in front of those reads); the
// caller owns the ordering: s_waitcnt vmcnt(0) and a barrier before any wave
// reads the destination.
// M0 carries the LDS destination. The compiler reserves M0 (it never keeps a
// value of its own there, and warns when M0 is named as a clobber), so the
// statement writes it itself. The DMA reads M0 after it issues: with M0
// bound as an operand instead, the compiler put the next DMA's M0 write
// directly after the previous DMA and that DMA landed elsewhere in LDS
// (wrong attention outputs on MI355X, different from run to run). So every
// DMA statement here ends with a wait state (s_nop 0), and the next M0
// write is always at least two instructions later.
__device__ __forceinline__ void dma16_to_lds(const void *gptr, const void *lds_base) {
    const uint32_t addr =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_nop 0"
                 :
                 : "s"(addr), "v"(gptr)
                 : "memory");
}

// The lane index, recomputed (v_mbcnt) at each call and opaque to the
// compiler, so that values derived from it are formed where they are used
// instead of being hoisted out of loops as long-lived registers.
__device__ __forceinline__ int fresh_lane() {
    int x;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
    return x;
}

// Raw buffer resource over [base, base + bytes): loads at byte offsets
// >= bytes return zeros instead of touching memory (gfx9 range checking
// applies to the VGPR offset; the SGPR offset is kept 0).
__device__ __forceinline__ u32x4 buffer_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32), bytes, 0x00020000u};
}

// The same LDS-DMA from a buffer resource: lane i fetches 16 bytes at byte
// offset voff (zeros when out of range) into lds_base + 16 * i.
__device__ __forceinline__ void dma16_buf_to_lds(u32x4 rsrc, uint32_t voff, const void *lds_base) {
    const uint32_t addr =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_nop 0"
                 :
                 : "s"(addr), "v"(voff), "s"(rsrc)
                 : "memory");
}

// Softmax work for one MFMA slot of the P·V / softmax overlap, as an
// instruction group the compiler keeps in place (it is placed between two
// MFMAs): the exponentials of NPAIR pairs of scores,
//   p = 2^(s·c - m), ls += p, pk = bf16x2(p0, p1),
// i.e. Map(exp) and Reduce(+) of the softmax. Every v_exp result is consumed
// at least one instruction later (the transcendental forwarding hazard).
__device__ __forceinline__ void exp_pair(float s0, float s1, float c, float negm, float &ls,
                                         uint32_t &pk) {
    float t0, t1;
    asm volatile(
        "v_fma_f32 %[t0], %[s0], %[c], %[nm]\n\t"
        "v_fma_f32 %[t1], %[s1], %[c], %[nm]\n\t"
        "v_exp_f32 %[t0], %[t0]\n\t"
        "v_exp_f32 %[t1], %[t1]\n\t"
        "v_add_f32 %[ls], %[ls], %[t0]\n\t"
        "v_add_f32 %[ls], %[ls], %[t1]\n\t"
        "v_cvt_pk_bf16_f32 %[pk], %[t0], %[t1]"
        : [t0] "=&v"(t0), [t1] "=&v"(t1), [ls] "+v"(ls), [pk] "=v"(pk)
        : [s0] "v"(s0), [s1] "v"(s1), [c] "s"(c), [nm] "v"(negm));
}


}  // namespace attn
