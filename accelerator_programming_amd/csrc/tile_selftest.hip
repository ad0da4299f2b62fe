// Probes of the tile layer, one wave each, for the GPU unit tests: the MFMA
// fragment layout, the cross-half wave reductions, the Vᵀ key order used by
// the P·V contraction, and the lane layout of the LDS transpose read. They
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

__global__ void __launch_bounds__(64) xhalf_probe(const float *x, float *mx, float *sm) {
    const int lane = threadIdx.x;
    mx[lane] = xhalf_max(x[lane]);
    sm[lane] = xhalf_sum(x[lane]);
}

// Pᵀ·V through the kernel's own path: scores Sᵀ (32 keys x 32 queries,
// supplied already in accumulator layout by the host as a row-major 32x32
// matrix), converted to bf16 Pᵀ operands, times V (32 keys x 32 columns,
// row-major bf16) staged to LDS in the permuted Vᵀ order. Output O is 32
// queries x 32 columns, row-major fp32.
__global__ void __launch_bounds__(64) pv_probe(const float *St, const __bf16 *Vg, float *O) {
    constexpr int PV = 32 + 8;
    __shared__ __attribute__((aligned(16))) __bf16 vt[32 * PV];
    const int lane = threadIdx.x, l32 = lane & 31, g = lane >> 5;
    // stage: lanes 0..31 each handle keys 4*(lane%8) .. +3, columns 8*(lane/8) .. +7
    if (lane < 32) {
        const int kq = lane % 8, d8 = lane / 8;
        u32x4 vr[4];
        for (int j = 0; j < 4; ++j) vr[j] = *(const u32x4 *)(Vg + (4 * kq + j) * 32 + 8 * d8);
        const int pos = vt_pos(4 * kq);
        for (int i = 0; i < 8; ++i) {
            const int p = i >> 1;
            const bool hi = i & 1;
            *(u32x2 *)(vt + (8 * d8 + i) * PV + pos) =
                u32x2{pick_halves(vr[0][p], vr[1][p], hi), pick_halves(vr[2][p], vr[3][p], hi)};
        }
    }
    __syncthreads();
    f32x16 s;
    for (int r = 0; r < 16; ++r) s[r] = St[acc_row(r, g) * 32 + l32];
    bf16x8 pf[2];
    for (int hh = 0; hh < 2; ++hh) {
        u32x4 v;
        for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(s[8 * hh + 2 * e], s[8 * hh + 2 * e + 1]);
        pf[hh] = u32x4_as_bf16x8(v);
    }
    f32x16 o;
    for (int r = 0; r < 16; ++r) o[r] = 0.f;
    for (int kc = 0; kc < 2; ++kc) {
        const bf16x8 vf = *(const bf16x8 *)(vt + l32 * PV + 16 * kc + 8 * g);
        o = mfma_32x32x16(vf, pf[kc], o);
    }
    // o holds Oᵀ: row = output column, column = query
    for (int r = 0; r < 16; ++r) O[l32 * 32 + acc_row(r, g)] = o[r];
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

}  // namespace

extern "C" {

int tile_selftest_mfma(const void *A, const void *B, void *C, void *stream) {
    hipLaunchKernelGGL(mfma_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (const __bf16 *)A,
                       (const __bf16 *)B, (float *)C);
    return (int)hipGetLastError();
}

int tile_selftest_xhalf(const void *x, void *mx, void *sm, void *stream) {
    hipLaunchKernelGGL(xhalf_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (const float *)x,
                       (float *)mx, (float *)sm);
    return (int)hipGetLastError();
}

int tile_selftest_pv(const void *St, const void *V, void *O, void *stream) {
    hipLaunchKernelGGL(pv_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (const float *)St,
                       (const __bf16 *)V, (float *)O);
    return (int)hipGetLastError();
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
