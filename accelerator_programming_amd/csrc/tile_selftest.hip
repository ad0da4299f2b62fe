// Probes of the tile layer, one wave each, for the GPU unit tests: the MFMA
// fragment layout, the cross-half wave reductions, the swizzled K fragment
// path of Q·Kᵀ, the transposed V fragment path of P·V, and the lane layout of
// the LDS transpose read, the shader clock under load, and the sustained
// MFMA rate of the chip on data that toggles like real operands. They
// check the primitives the attention kernel is built from, separately from it
// ("Distilling a 4.5 hour CUDA talk", section 9: unit tests over every
// load/store/layout/MMA combination).
#include <hip/hip_runtime.h>

#include "attn_fwd_kernel.hpp"

using namespace attn;

namespace {

// C (32x32, row-major fp32) = A (32x16, row-major bf16) · B (16x32, row-major bf16)
__global__ void __launch_bounds__(64) mfma_probe(const __bf16 *A, const __bf16 *B, float *Cm) {
    const int lane = threadIdx.x, l32 = lane & 31, g = lane >> 5;
    bf16x8 a, b;
    for (int e = 0; e < 8; ++e) {
        a[e] = A[l32 * 16 + 8 * g + e];
        b[e] = B[(8 * g + e) * 32 + l32];
    }
    f32x16 c;
    for (int r = 0; r < 16; ++r) c[r] = 0.f;
    c = mfma_32x32x16(a, b, c);
    for (int r = 0; r < 16; ++r) Cm[acc_row(r, g) * 32 + l32] = c[r];
}

// C (16x16, row-major fp32) = A (16x32, row-major bf16) · B (32x16, row-major bf16)
__global__ void __launch_bounds__(64) mfma16_probe(const __bf16 *A, const __bf16 *B, float *Cm) {
    const int lane = threadIdx.x, l16 = lane & 15, G = lane >> 4;
    bf16x8 a, b;
    for (int e = 0; e < 8; ++e) {
        a[e] = A[l16 * 32 + 8 * G + e];
        b[e] = B[(8 * G + e) * 16 + l16];
    }
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    c = mfma_16x16x32(a, b, c);
    for (int i = 0; i < 4; ++i) Cm[(4 * G + i) * 16 + l16] = c[i];
}

__global__ void __launch_bounds__(64) xhalf_probe(const float *x, float *mx, float *sm) {
    const int lane = threadIdx.x;
    mx[lane] = xhalf_max(x[lane]);
    sm[lane] = xhalf_sum(x[lane]);
}

// Sᵀ = K·Qᵀ through the kernel's fragment path: K (32 keys x D, row-major
// bf16) is written to LDS in the swizzled K layout, Q (32 rows x D) is read
// into B fragments as the kernel does. St is 32 keys x 32 queries, fp32.
template <int D>
__global__ void __launch_bounds__(64) qk_probe(const __bf16 *Kg, const __bf16 *Qg, float *St) {
    __shared__ __attribute__((aligned(16))) __bf16 ks[32 * D];
    const int lane = threadIdx.x, l32 = lane & 31, g = lane >> 5;
    for (int ch = lane; ch < 32 * D / 8; ch += 64) {
        const int r = ch / (D / 8), c = ch % (D / 8);
        *(u32x4 *)(ks + r * D + 8 * k_chunk<D>(r, c)) = *(const u32x4 *)(Kg + r * D + 8 * c);
    }
    __syncthreads();
    f32x16 s;
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    for (int kc = 0; kc < D / 16; ++kc) {
        const bf16x8 qf = u32x4_as_bf16x8(*(const u32x4 *)(Qg + l32 * D + 16 * kc + 8 * g));
        s = mfma_32x32x16(k_frag<D>(ks, l32, kc, g), qf, s);
    }
    for (int r = 0; r < 16; ++r) St[acc_row(r, g) * 32 + l32] = s[r];
}

// Oᵀ = Vᵀ·Pᵀ through the kernel's fragment path: scores St (64 keys x 32
// queries, fp32) are taken in accumulator layout and packed to bf16 Pᵀ
// operands as the kernel does; V (64 keys x D, row-major bf16) is written to
// LDS in the swizzled V layout and read with transpose reads. O is
// 32 queries x D, fp32.
template <int D>
__global__ void __launch_bounds__(64) pv_probe(const float *St, const __bf16 *Vg, float *O) {
    __shared__ __attribute__((aligned(16))) __bf16 vs[64 * D];
    const int lane = threadIdx.x, l32 = lane & 31, g = lane >> 5;
    for (int ch = lane; ch < 64 * D / 8; ch += 64) {
        const int r = ch / (D / 8), c = ch % (D / 8);
        *(u32x4 *)(vs + r * D + 8 * v_chunk<D>(r, c)) = *(const u32x4 *)(Vg + r * D + 8 * c);
    }
    __syncthreads();
    bf16x8 pf[4];
    for (int kb = 0; kb < 2; ++kb)
        for (int hh = 0; hh < 2; ++hh) {
            u32x4 v;
            for (int e = 0; e < 4; ++e) {
                const float lo = St[(32 * kb + acc_row(8 * hh + 2 * e, g)) * 32 + l32];
                const float hi = St[(32 * kb + acc_row(8 * hh + 2 * e + 1, g)) * 32 + l32];
                v[e] = pack_bf16x2(lo, hi);
            }
            pf[2 * kb + hh] = u32x4_as_bf16x8(v);
        }
    for (int db = 0; db < D / 32; ++db) {
        f32x16 o;
        for (int r = 0; r < 16; ++r) o[r] = 0.f;
        for (int kc = 0; kc < 4; ++kc) o = mfma_32x32x16(vt_frag<D>(vs, db, kc, lane), pf[kc], o);
        for (int r = 0; r < 16; ++r) O[l32 * D + 32 * db + acc_row(r, g)] = o[r];
    }
}

// ds_read_b64_tr_b16: LDS holds n 16-bit values equal to their index; lane l
// reads at byte offset off[l] (host-checked: 8-byte aligned, in bounds).
__global__ void __launch_bounds__(64) tr16_probe(const int *off, int n, short *out) {
    __shared__ __attribute__((aligned(16))) short buf[4096];
    for (int i = threadIdx.x; i < n; i += 64) buf[i] = (short)i;
    __syncthreads();
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)((__attribute__((address_space(3))) char *)buf +
                                                    off[threadIdx.x]));
    for (int e = 0; e < 4; ++e) out[threadIdx.x * 4 + e] = r[e];
}

// The shader clock a CU runs at while it carries other work: one wave per
// workgroup reads the shader-cycle counter (s_memtime) and the constant-rate
// counter (s_memrealtime), sleeps until the latter has advanced by `ticks`
// (at most `max_iter` sleeps, so every wave ends), reads both again and
// stores the two differences (cycles, ticks) for its workgroup.
__global__ void __launch_bounds__(64) clock_probe(uint64_t *out, uint32_t ticks, uint32_t max_iter) {
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    uint64_t r = r0;
    for (uint32_t i = 0; i < max_iter && r - r0 < ticks; ++i) {
        __builtin_amdgcn_s_sleep(2);
        r = __builtin_amdgcn_s_memrealtime();
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = t1 - t0;
        out[2 * blockIdx.x + 1] = r - r0;
    }
}

// The sustained dense bf16 MFMA rate of the chip: 8 waves per workgroup (two
// per SIMD), one workgroup per CU (96 KB of LDS each), every wave issuing
// `iters` x 16 v_mfma_f32_32x32x16_bf16 back to back. Both operands come from
// LDS through a ring of eight fragment registers read four MFMAs ahead (A is
// this MFMA's fragment, B the previous one), and LDS holds hashed bf16 values
// in [-2, 2), so the operand bits toggle as with real data; constant operands
// let the chip hold a much higher clock. The whole loop is one assembly
// statement that ends with every fragment read complete. Each wave stores its
// shader cycles (s_memtime) and constant-rate ticks (s_memrealtime).
#define MR_RD(q, o) "ds_read_b128 %[" #q "], %[ad] offset:" #o "\n\t"
#define MR_MF(c, a, b) "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 %[" #c "], %[" #a "], %[" #b "], %[" #c "]\n\t"
constexpr int kRateLdsBytes = 96 * 1024;
__global__ void __launch_bounds__(512) mfma_rate_probe(uint64_t *out, uint32_t iters) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kRateLdsBytes];
    for (int i = threadIdx.x; i < 16384 / 2; i += blockDim.x) {
        uint32_t x = (uint32_t)i * 2654435761u + 0x9E3779B9u;
        x ^= x >> 15;
        x *= 2246822519u;
        x ^= x >> 13;
        ((__bf16 *)lds)[i] = (__bf16)((float)(x & 0xffffu) * (1.0f / 16384.0f) - 2.0f);
    }
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const uint32_t ad = lds_addr(lds) + 16u * (uint32_t)lane;  // fragment reads stay below 16 KB
    f32x16 c0, c1;
    for (int r = 0; r < 16; ++r) c0[r] = c1[r] = 0.f;
    u32x4 q0, q1, q2, q3, q4, q5, q6, q7;
    uint32_t n;
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    asm volatile(
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_mov_b32 %[n], %[iters]\n\t"
        MR_RD(q7, 7168) "s_waitcnt lgkmcnt(0)\n\t"
        MR_RD(q0, 0) MR_RD(q1, 1024) MR_RD(q2, 2048) MR_RD(q3, 3072)
        ".Lmfma_rate_loop%=:\n\t"
        MR_MF(c0, q0, q7) MR_RD(q4, 4096) MR_MF(c1, q1, q0) MR_RD(q5, 5120)
        MR_MF(c0, q2, q1) MR_RD(q6, 6144) MR_MF(c1, q3, q2) MR_RD(q7, 7168)
        MR_MF(c0, q4, q3) MR_RD(q0, 8192) MR_MF(c1, q5, q4) MR_RD(q1, 9216)
        MR_MF(c0, q6, q5) MR_RD(q2, 10240) MR_MF(c1, q7, q6) MR_RD(q3, 11264)
        MR_MF(c0, q0, q7) MR_RD(q4, 12288) MR_MF(c1, q1, q0) MR_RD(q5, 13312)
        MR_MF(c0, q2, q1) MR_RD(q6, 14336) MR_MF(c1, q3, q2) MR_RD(q7, 15360)
        MR_MF(c0, q4, q3) MR_RD(q0, 0) MR_MF(c1, q5, q4) MR_RD(q1, 1024)
        MR_MF(c0, q6, q5) MR_RD(q2, 2048) MR_MF(c1, q7, q6) MR_RD(q3, 3072)
        "s_sub_u32 %[n], %[n], 1\n\t"
        "s_cmp_lg_u32 %[n], 0\n\t"
        "s_cbranch_scc1 .Lmfma_rate_loop%=\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
        : [c0] "+v"(c0), [c1] "+v"(c1), [q0] "=&v"(q0), [q1] "=&v"(q1), [q2] "=&v"(q2),
          [q3] "=&v"(q3), [q4] "=&v"(q4), [q5] "=&v"(q5), [q6] "=&v"(q6), [q7] "=&v"(q7),
          [n] "=&s"(n)
        : [iters] "s"(iters), [ad] "v"(ad)
        : "scc", "memory");
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    float sink = 0.f;
    for (int r = 0; r < 16; ++r) sink += c0[r] + c1[r];
    const int wave = threadIdx.x >> 6;
    if (lane == 0) {
        out[2 * (8 * blockIdx.x + wave)] = t1 - t0;
        out[2 * (8 * blockIdx.x + wave) + 1] = r1 - r0;
    }
    // keeps the accumulators live; the sum of finite products is never NaN
    if (sink != sink) out[0] = 0;
}
#undef MR_RD
#undef MR_MF

}  // namespace

extern "C" {

int tile_selftest_mfma(const void *A, const void *B, void *C, void *stream) {
    hipLaunchKernelGGL(mfma_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (const __bf16 *)A,
                       (const __bf16 *)B, (float *)C);
    return (int)hipGetLastError();
}

int tile_selftest_mfma16(const void *A, const void *B, void *C, void *stream) {
    hipLaunchKernelGGL(mfma16_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (const __bf16 *)A,
                       (const __bf16 *)B, (float *)C);
    return (int)hipGetLastError();
}

int tile_selftest_xhalf(const void *x, void *mx, void *sm, void *stream) {
    hipLaunchKernelGGL(xhalf_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (const float *)x,
                       (float *)mx, (float *)sm);
    return (int)hipGetLastError();
}

int tile_selftest_qk(int d, const void *K, const void *Q, void *St, void *stream) {
    if (d == 64)
        hipLaunchKernelGGL(qk_probe<64>, dim3(1), dim3(64), 0, (hipStream_t)stream,
                           (const __bf16 *)K, (const __bf16 *)Q, (float *)St);
    else if (d == 128)
        hipLaunchKernelGGL(qk_probe<128>, dim3(1), dim3(64), 0, (hipStream_t)stream,
                           (const __bf16 *)K, (const __bf16 *)Q, (float *)St);
    else
        return -1;
    return (int)hipGetLastError();
}

int tile_selftest_pv(int d, const void *St, const void *V, void *O, void *stream) {
    if (d == 64)
        hipLaunchKernelGGL(pv_probe<64>, dim3(1), dim3(64), 0, (hipStream_t)stream,
                           (const float *)St, (const __bf16 *)V, (float *)O);
    else if (d == 128)
        hipLaunchKernelGGL(pv_probe<128>, dim3(1), dim3(64), 0, (hipStream_t)stream,
                           (const float *)St, (const __bf16 *)V, (float *)O);
    else
        return -1;
    return (int)hipGetLastError();
}

// n_blocks workgroups of the clock probe; out: 2 * n_blocks uint64 (device)
int tile_selftest_clock(void *out, int n_blocks, unsigned ticks, unsigned max_iter, void *stream) {
    if (!out || n_blocks < 1 || n_blocks > 65536) return -1;
    hipLaunchKernelGGL(clock_probe, dim3(n_blocks), dim3(64), 0, (hipStream_t)stream, (uint64_t *)out,
                       (uint32_t)ticks, (uint32_t)max_iter);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// rate of the counter s_memrealtime reads, in kHz (0 if unknown)
int tile_selftest_wallclock_khz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}

// n_blocks workgroups of the MFMA rate probe, each wave `iters` x 16 MFMAs;
// out: 16 * n_blocks uint64 (device): per wave its shader cycles, then its
// s_memrealtime ticks. Returns -1 without launching on a bad argument.
int tile_selftest_mfma_rate(void *out, int n_blocks, unsigned iters, void *stream) {
    if (!out || n_blocks < 1 || n_blocks > 4096 || iters < 1 || iters > 10000000u) return -1;
    hipLaunchKernelGGL(mfma_rate_probe, dim3(n_blocks), dim3(512), 0, (hipStream_t)stream,
                       (uint64_t *)out, (uint32_t)iters);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// offsets: 64 device ints; n: number of 16-bit values in LDS (<= 4096).
// Returns -1 without launching if n is out of range; the caller checks the
// offsets against n on the host before the call.
int tile_selftest_tr16(const void *offsets, int n, void *out, void *stream) {
    if (n < 1 || n > 4096) return -1;
    hipLaunchKernelGGL(tr16_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (const int *)offsets,
                       n, (short *)out);
    return (int)hipGetLastError();
}

}  // extern "C"
