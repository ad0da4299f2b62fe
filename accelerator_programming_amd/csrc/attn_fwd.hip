// C ABI of the gfx950 attention forward library: plan creation (host-only
// validation and variant choice), launch, and teardown. The declarations and
// their contracts are in include/attn_fwd.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <new>

#include "../../include/attn_fwd.h"
#include "attn_fwd_kernel.hpp"
#include "attn_fwd_wide_kernel.hpp"
#include "attn_fwd_wide_vk_kernel.hpp"
#include "attn_fwd_wide_vk_split_kernel.hpp"
#include "attn_split_kernel.hpp"

using attn::KernelArgs;
using attn::TileCfg;
using attn::WideCfg;

namespace {

enum Variant : int32_t {
    V_D64_BF16 = 0,
    V_D128_BF16 = 1,
    V_D64_FP32 = 2,
    V_D576_BF16 = 3,  // d_qk = 576, d_v = 512
};

}  // namespace

struct attn_fwd_plan {
    attn_fwd_params p;  // strides filled in
    int32_t variant;
    int32_t tile_q, tile_k, block, lds_bytes;
    int64_t n_qtiles, grid;   // grid: work items (query tiles x heads x batch)
    int32_t persist_rounds;   // main kernel: 0, or items per workgroup of a kPersistGrid launch
    float c;  // scale * log2(e)
};

namespace {

constexpr int64_t kMaxSlab = ((int64_t)1 << 31) - 1;
// one main-kernel workgroup per CU of an MI355X (256 CUs in 8 XCDs)
constexpr int64_t kPersistGrid = 256;

bool fill_strides(int64_t s[3], int64_t H, int64_t N, int64_t d, int64_t row_min,
                  int64_t align_elems) {
    if (s[0] == 0 && s[1] == 0 && s[2] == 0) {
        s[2] = d;
        s[1] = N * d;
        s[0] = H * N * d;
    }
    for (int i = 0; i < 3; ++i)
        if (s[i] < 0 || s[i] % align_elems != 0) return false;
    if (s[2] < row_min) return false;
    // every element offset inside one [N, d] slab must fit in 31 bits
    if ((N - 1) * s[2] + d > kMaxSlab) return false;
    return true;
}

attn_status validate(const attn_fwd_params *in, attn_fwd_plan *out) {
    attn_fwd_params p = *in;
    if (p.N_kv == 0) p.N_kv = p.N;
    if (p.d_v == 0) p.d_v = p.d;
    if (p.B < 1 || p.H_q < 1 || p.H_kv < 1 || p.N < 1 || p.d < 1 || p.N_kv < 1 || p.d_v < 1)
        return ATTN_ERR_INVALID;
    if (p.H_q % p.H_kv != 0) return ATTN_ERR_INVALID;
    if (p.causal != 0 && p.causal != 1) return ATTN_ERR_INVALID;
    if (p.causal && p.N_kv != p.N) return ATTN_ERR_INVALID;
    if (!std::isfinite(p.scale) || !(p.scale > 0.f)) return ATTN_ERR_INVALID;
    if (p.dtype != ATTN_BF16 && p.dtype != ATTN_FP32) return ATTN_ERR_INVALID;
    // grid and index arithmetic run in 32 bits inside the kernel
    if (p.B * p.H_q > ((int64_t)1 << 30) || p.N > ((int64_t)1 << 30) || p.N_kv > ((int64_t)1 << 30))
        return ATTN_ERR_UNSUPPORTED;

    const int64_t align = (p.dtype == ATTN_BF16) ? 8 : 4;
    if (!fill_strides(p.q_strides, p.H_q, p.N, p.d, p.d, align)) return ATTN_ERR_INVALID;
    if (!fill_strides(p.k_strides, p.H_kv, p.N_kv, p.d, p.d, align)) return ATTN_ERR_INVALID;
    if (!fill_strides(p.v_strides, p.H_kv, p.N_kv, p.d_v, p.d_v, align)) return ATTN_ERR_INVALID;
    if (!fill_strides(p.o_strides, p.H_q, p.N, p.d_v, p.d_v, align)) return ATTN_ERR_INVALID;

    int32_t variant;
    if (p.d == 64 && p.d_v == 64 && p.dtype == ATTN_BF16) variant = V_D64_BF16;
    else if (p.d == 128 && p.d_v == 128 && p.dtype == ATTN_BF16) variant = V_D128_BF16;
    else if (p.d == 64 && p.d_v == 64 && p.dtype == ATTN_FP32) variant = V_D64_FP32;
    else if (p.d == 576 && p.d_v == 512 && p.dtype == ATTN_BF16) variant = V_D576_BF16;
    else return ATTN_ERR_UNSUPPORTED;

    out->p = p;
    out->variant = variant;
    if (variant == V_D576_BF16) {
        out->tile_q = WideCfg<576, 512>::TQ;
        out->tile_k = WideCfg<576, 512>::TK;
        out->block = WideCfg<576, 512>::NT;
        out->lds_bytes = WideCfg<576, 512>::LDS_BYTES;
    } else if (variant == V_D128_BF16) {
        out->tile_q = TileCfg<128>::TQ;
        out->tile_k = TileCfg<128>::TK;
        out->block = TileCfg<128>::NT;
        out->lds_bytes = TileCfg<128>::LDS_BYTES;
    } else {
        out->tile_q = TileCfg<64>::TQ;
        out->tile_k = TileCfg<64>::TK;
        out->block = TileCfg<64>::NT;
        out->lds_bytes = TileCfg<64>::LDS_BYTES;
    }
    out->n_qtiles = (p.N + out->tile_q - 1) / out->tile_q;
    out->grid = out->n_qtiles * p.B * p.H_q;
    if (out->grid > 0x7fffffff) return ATTN_ERR_UNSUPPORTED;
    // the main kernel runs persistent workgroups, one per CU, when its items
    // fill at least two whole rounds of them and its kv-head groups split
    // evenly over the 8 XCDs (the work order keeps each group on one XCD)
    out->persist_rounds = 0;
    if (variant != V_D576_BF16 && (p.B * p.H_kv) % 8 == 0 && out->grid % kPersistGrid == 0 &&
        out->grid >= 2 * kPersistGrid)
        out->persist_rounds = (int32_t)(out->grid / kPersistGrid);
    out->c = (float)((double)p.scale * 1.4426950408889634074);
    return ATTN_OK;
}

template <int D, bool CAUSAL, typename T, bool DROP = false, bool ROPE = false>
hipError_t launch(const attn_fwd_plan *pl, const KernelArgs &a0, hipStream_t stream) {
    KernelArgs a = a0;
    a.persist_rounds = ROPE ? 0 : pl->persist_rounds;
    const int64_t grid = a.persist_rounds > 0 ? kPersistGrid : pl->grid;
    hipLaunchKernelGGL((attn::attn_fwd_kernel<D, CAUSAL, T, DROP, ROPE>), dim3((uint32_t)grid),
                       dim3(pl->block), 0, stream, a);
    return hipGetLastError();
}

// RoPE launch over a [B, H, N, d] bf16 tensor (strides in elements, innermost 1)
hipError_t launch_rope(const void *X, void *Y, int64_t B, int64_t H, int64_t N, int64_t d,
                       const int64_t xs[3], const int64_t ys[3], double log2_base,
                       hipStream_t stream) {
    attn::RopeArgs r;
    r.x = (const __bf16 *)X;
    r.y = (__bf16 *)Y;
    r.x_sb = xs[0]; r.x_sh = xs[1]; r.x_sn = xs[2];
    r.y_sb = ys[0]; r.y_sh = ys[1]; r.y_sn = ys[2];
    r.H = (int32_t)H;
    r.N = (int32_t)N;
    r.d = (int32_t)d;
    r.row_blocks = (int32_t)((N + attn::ROPE_ROWS - 1) / attn::ROPE_ROWS);
    r.log2_base = log2_base;
    const int64_t blocks = B * H * r.row_blocks;
    hipLaunchKernelGGL(attn::rope_bf16_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, r);
    return hipGetLastError();
}

bool rope_base_ok(float base) { return std::isfinite(base) && base > 1.0f; }

// Wide heads: V given as the first d_v columns of K's rows takes the kernel
// that stages only K (512 threads); any other V takes the general one (the
// plan's block). Both use 32-row tiles, so the grid is the same.
template <bool CAUSAL>
hipError_t launch_wide(const attn_fwd_plan *pl, const KernelArgs &a, hipStream_t stream) {
    static_assert(attn::WideVkCfg<576, 512>::TQ == WideCfg<576, 512>::TQ, "one grid for both wide kernels");
    if (a.v_in_k)
        hipLaunchKernelGGL((attn::attn_fwd_wide_vk_kernel<576, 512, CAUSAL>), dim3((uint32_t)pl->grid),
                           dim3(attn::WideVkCfg<576, 512>::NT), 0, stream, a);
    else
        hipLaunchKernelGGL((attn::attn_fwd_wide_kernel<576, 512, CAUSAL>), dim3((uint32_t)pl->grid),
                           dim3(pl->block), 0, stream, a);
    return hipGetLastError();
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Kernel arguments of a plan and a set of device pointers.
KernelArgs make_args(const attn_fwd_plan *plan, const void *Q, const void *K, const void *V, void *O,
                     float *lse) {
    const attn_fwd_params &p = plan->p;
    KernelArgs a;
    a.persist_rounds = 0;
    a.q = Q;
    a.k = K;
    a.v = V;
    a.o = O;
    a.lse = lse;
    a.q_sb = p.q_strides[0];
    a.q_sh = p.q_strides[1];
    a.q_sn = (int32_t)p.q_strides[2];
    a.k_sb = p.k_strides[0];
    a.k_sh = p.k_strides[1];
    a.k_sn = (int32_t)p.k_strides[2];
    a.v_sb = p.v_strides[0];
    a.v_sh = p.v_strides[1];
    a.v_sn = (int32_t)p.v_strides[2];
    a.o_sb = p.o_strides[0];
    a.o_sh = p.o_strides[1];
    a.o_sn = (int32_t)p.o_strides[2];
    a.B = (int32_t)p.B;
    a.Hq = (int32_t)p.H_q;
    a.Hkv = (int32_t)p.H_kv;
    a.Nq = (int32_t)p.N;
    a.Nkv = (int32_t)p.N_kv;
    a.group = (int32_t)(p.H_q / p.H_kv);
    a.n_qtiles = (int32_t)plan->n_qtiles;
    a.c = plan->c;
    a.v_in_k = (V == K && p.v_strides[0] == p.k_strides[0] && p.v_strides[1] == p.k_strides[1] &&
                p.v_strides[2] == p.k_strides[2]) ? 1 : 0;
    a.drop_thr = 0;
    a.seed_lo = a.seed_hi = 0;
    a.drop_scale = 1.0f;
    a.rope_log2_base = 0.0;
    return a;
}

// ---- split-KV path (few query rows per kv head, non-causal) ----------------
constexpr int32_t kMaxSplits = 64;  // the merge holds one split per lane

using WVS = attn::WideVkSplitCfg<576, 512>;

// wide heads (d_qk 576, d_v 512) with V inside K: 64-row tiles of each
// (batch, head) over key ranges (the V-in-K check needs the pointers and is
// made at run time)
bool wide_split(const attn_fwd_plan *pl) { return pl->variant == V_D576_BF16; }

bool split_supported(const attn_fwd_plan *pl) {
    const attn_fwd_params &p = pl->p;
    if (p.causal) return false;
    if (wide_split(pl)) {
        // one 512-thread workgroup per (range, batch, head, 64-row tile): at
        // the most ranges the launch stays below 2^32 work-items
        const int64_t items = p.B * p.H_q * ((p.N + WVS::TQ - 1) / WVS::TQ);
        return items * kMaxSplits * WVS::NT < ((int64_t)1 << 32);
    }
    // one 256-thread workgroup per (split, batch, kv head) and one per merged
    // row (at most 64 per (batch, kv head)): each launch stays below 2^32
    // work-items
    return (pl->variant == V_D64_BF16 || pl->variant == V_D128_BF16) &&
           (p.H_q / p.H_kv) * p.N <= attn::SplitCfg<64>::ROWS && (int64_t)p.B * p.H_kv <= (1 << 18);
}

// about two workgroups per CU (256 CUs), at least one 64-key tile per split;
// wide heads: about one 512-thread workgroup per CU, at least one 32-key tile
int32_t auto_splits(const attn_fwd_plan *pl) {
    const attn_fwd_params &p = pl->p;
    int64_t n, tiles;
    if (wide_split(pl)) {
        const int64_t items = p.B * p.H_q * ((p.N + WVS::TQ - 1) / WVS::TQ);
        tiles = (p.N_kv + WVS::TK - 1) / WVS::TK;
        n = (256 + items - 1) / items;
    } else {
        const int64_t groups = p.B * p.H_kv;
        tiles = (p.N_kv + 63) / 64;
        n = (512 + groups - 1) / groups;
    }
    if (n > tiles) n = tiles;
    if (n > kMaxSplits) n = kMaxSplits;
    return (int32_t)(n < 1 ? 1 : n);
}

// workspace: n_splits partial outputs [n][B][H_q][N][d_v] fp32, then their
// logsumexps [n][B][H_q][N] fp32
int64_t split_workspace(const attn_fwd_plan *pl, int32_t n) {
    const attn_fwd_params &p = pl->p;
    return (int64_t)n * p.B * p.H_q * p.N * (p.d_v + 1) * 4;
}

template <int D>
hipError_t launch_split(const attn_fwd_plan *pl, const KernelArgs &a, int32_t n, float *ws,
                        hipStream_t stream) {
    using SC = attn::SplitCfg<D>;
    const attn_fwd_params &p = pl->p;
    const int64_t rows = p.B * p.H_q * p.N;
    attn::SplitArgs sa;
    sa.a = a;
    sa.opart = ws;
    sa.lpart = ws + (int64_t)n * rows * D;
    sa.n_splits = n;
    const int64_t tiles = (p.N_kv + SC::TK - 1) / SC::TK;
    sa.split_len = (int32_t)(((tiles + n - 1) / n) * SC::TK);
    sa.rows = (int32_t)((p.H_q / p.H_kv) * p.N);
    hipLaunchKernelGGL((attn::attn_split_kernel<D>), dim3((uint32_t)(n * p.B * p.H_kv)), dim3(SC::NT), 0,
                       stream, sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn::attn_split_merge<D>), dim3((uint32_t)rows), dim3(256), 0, stream,
                       (const float *)sa.opart, (const float *)sa.lpart, n, rows, a);
    return hipGetLastError();
}

hipError_t launch_wide_split(const attn_fwd_plan *pl, KernelArgs a, int32_t n, float *ws, hipStream_t stream) {
    const attn_fwd_params &p = pl->p;
    const int64_t rows = p.B * p.H_q * p.N;
    a.n_qtiles = (int32_t)((p.N + WVS::TQ - 1) / WVS::TQ);
    attn::SplitArgs sa;
    sa.a = a;
    sa.opart = ws;
    sa.lpart = ws + (int64_t)n * rows * 512;
    sa.n_splits = n;
    const int64_t tiles = (p.N_kv + WVS::TK - 1) / WVS::TK;
    sa.split_len = (int32_t)(((tiles + n - 1) / n) * WVS::TK);
    sa.rows = 0;
    const int64_t grid = (int64_t)n * p.B * p.H_q * a.n_qtiles;
    hipLaunchKernelGGL((attn::attn_fwd_wide_vk_split_kernel<576, 512>), dim3((uint32_t)grid), dim3(WVS::NT), 0,
                       stream, sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = rows * (512 / 4);
    const int64_t mgrid = items / 256 < 2048 ? (items + 255) / 256 : 2048;
    hipLaunchKernelGGL((attn::attn_split_merge_wide<512>), dim3((uint32_t)mgrid), dim3(256), 0, stream,
                       (const float *)sa.opart, (const float *)sa.lpart, n, rows, a);
    return hipGetLastError();
}

// ---- static scratch of attn_fwd_run_split_noalloc --------------------------
// One buffer per GPU (each device holds its own copy of a __device__ array).
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address is looked up with hipGetSymbolAddress once per device, with
// that device current, and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[ATTN_SPLIT_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];

// Device address of `scratch` on the device `stream` belongs to.
hipError_t scratch_address(hipStream_t stream, void **out) {
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t e2 = (cur != dev) ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (e2 != hipSuccess) return e2;
        if (!p || ((uintptr_t)p & 255u)) return hipErrorInvalidValue;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

attn_status attn_fwd_create_ex(const attn_fwd_params *params, attn_fwd_plan **plan) {
    if (!plan) return ATTN_ERR_INVALID;
    *plan = nullptr;
    if (!params) return ATTN_ERR_INVALID;
    attn_fwd_plan tmp;
    const attn_status st = validate(params, &tmp);
    if (st != ATTN_OK) return st;
    attn_fwd_plan *p = new (std::nothrow) attn_fwd_plan(tmp);
    if (!p) return ATTN_ERR_NOMEM;
    *plan = p;
    return ATTN_OK;
}

attn_status attn_fwd_create(attn_fwd_plan **plan, int64_t B, int64_t H_q, int64_t H_kv, int64_t N,
                            int64_t d, int32_t causal, float scale) {
    attn_fwd_params p = {};
    p.B = B;
    p.H_q = H_q;
    p.H_kv = H_kv;
    p.N = N;
    p.d = d;
    p.causal = causal;
    p.scale = scale;
    p.dtype = ATTN_BF16;
    return attn_fwd_create_ex(&p, plan);
}

attn_status attn_fwd_run(const attn_fwd_plan *plan, const void *Q, const void *K, const void *V,
                         void *O, float *lse, void *stream) {
    if (!plan || !Q || !K || !V || !O) return ATTN_ERR_INVALID;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) ||
        (lse && ((uintptr_t)lse & 3u)))
        return ATTN_ERR_INVALID;
    const attn_fwd_params &p = plan->p;
    const KernelArgs a = make_args(plan, Q, K, V, O, lse);

    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    switch (plan->variant) {
        case V_D64_BF16:
            e = p.causal ? launch<64, true, __bf16>(plan, a, s) : launch<64, false, __bf16>(plan, a, s);
            break;
        case V_D128_BF16:
            e = p.causal ? launch<128, true, __bf16>(plan, a, s) : launch<128, false, __bf16>(plan, a, s);
            break;
        case V_D64_FP32:
            e = p.causal ? launch<64, true, float>(plan, a, s) : launch<64, false, float>(plan, a, s);
            break;
        case V_D576_BF16:
            e = p.causal ? launch_wide<true>(plan, a, s) : launch_wide<false>(plan, a, s);
            break;
        default:
            return ATTN_ERR_INVALID;
    }
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_fwd_run_dropout(const attn_fwd_plan *plan, const void *Q, const void *K,
                                 const void *V, void *O, float *lse, float p_drop, uint64_t seed,
                                 void *stream) {
    if (!plan || !Q || !K || !V || !O) return ATTN_ERR_INVALID;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) ||
        (lse && ((uintptr_t)lse & 3u)))
        return ATTN_ERR_INVALID;
    if (!(p_drop >= 0.0f && p_drop < 1.0f)) return ATTN_ERR_INVALID;  // also NaN
    if (plan->variant == V_D576_BF16) return ATTN_ERR_UNSUPPORTED;
    // the drop probability is taken in steps of 1/256
    const uint32_t thr = (uint32_t)((double)p_drop * 256.0);
    if (thr == 0) return attn_fwd_run(plan, Q, K, V, O, lse, stream);
    const attn_fwd_params &p = plan->p;
    KernelArgs a = make_args(plan, Q, K, V, O, lse);
    a.drop_thr = thr;
    a.seed_lo = (uint32_t)seed;
    a.seed_hi = (uint32_t)(seed >> 32);
    a.drop_scale = (float)(256.0 / (256.0 - (double)thr));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    switch (plan->variant) {
        case V_D64_BF16:
            e = p.causal ? launch<64, true, __bf16, true>(plan, a, s)
                         : launch<64, false, __bf16, true>(plan, a, s);
            break;
        case V_D128_BF16:
            e = p.causal ? launch<128, true, __bf16, true>(plan, a, s)
                         : launch<128, false, __bf16, true>(plan, a, s);
            break;
        case V_D64_FP32:
            e = p.causal ? launch<64, true, float, true>(plan, a, s)
                         : launch<64, false, float, true>(plan, a, s);
            break;
        default:
            return ATTN_ERR_INVALID;
    }
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_rope_bf16(const void *X, void *Y, int64_t B, int64_t H, int64_t N, int64_t d,
                           const int64_t x_strides[3], const int64_t y_strides[3], float base,
                           void *stream) {
    if (B < 0 || H < 0 || N < 0 || d < 8 || d % 8 != 0) return ATTN_ERR_INVALID;
    if (!rope_base_ok(base)) return ATTN_ERR_INVALID;
    if (B == 0 || H == 0 || N == 0) return ATTN_OK;
    // one workgroup per (b, h, 64 rows); a row's chunks fit one workgroup
    if (N >= ((int64_t)1 << 31) || d > 2048 ||
        B * H * ((N + attn::ROPE_ROWS - 1) / attn::ROPE_ROWS) >= ((int64_t)1 << 31))
        return ATTN_ERR_INVALID;
    if (!X || !Y || !aligned16(X) || !aligned16(Y)) return ATTN_ERR_INVALID;
    int64_t xs[3], ys[3];
    for (int i = 0; i < 3; ++i) {
        xs[i] = x_strides ? x_strides[i] : 0;
        ys[i] = y_strides ? y_strides[i] : 0;
    }
    if (!fill_strides(xs, H, N, d, d, 8) || !fill_strides(ys, H, N, d, d, 8)) return ATTN_ERR_INVALID;
    return launch_rope(X, Y, B, H, N, d, xs, ys, std::log2((double)base), (hipStream_t)stream) ==
                   hipSuccess
               ? ATTN_OK
               : ATTN_ERR_HIP;
}

int64_t attn_fwd_rope_workspace_bytes(const attn_fwd_plan *plan) {
    if (!plan || (plan->variant != V_D64_BF16 && plan->variant != V_D128_BF16)) return -1;
    const attn_fwd_params &p = plan->p;
    return p.B * p.H_kv * p.N_kv * p.d * 2;
}

attn_status attn_fwd_run_rope(const attn_fwd_plan *plan, const void *Q, const void *K, const void *V,
                              void *O, float *lse, float base, void *k_rot, int64_t k_rot_bytes,
                              void *stream) {
    if (!plan || !Q || !K || !V || !O || !k_rot) return ATTN_ERR_INVALID;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(k_rot) ||
        (lse && ((uintptr_t)lse & 3u)))
        return ATTN_ERR_INVALID;
    if (!rope_base_ok(base)) return ATTN_ERR_INVALID;
    if (plan->variant != V_D64_BF16 && plan->variant != V_D128_BF16) return ATTN_ERR_UNSUPPORTED;
    const attn_fwd_params &p = plan->p;
    if (k_rot_bytes < attn_fwd_rope_workspace_bytes(plan)) return ATTN_ERR_INVALID;
    const double log2_base = std::log2((double)base);
    hipStream_t s = (hipStream_t)stream;
    // K rotated once per kv head into the workspace ([B, H_kv, N_kv, d], contiguous)
    int64_t ks[3] = {p.k_strides[0], p.k_strides[1], p.k_strides[2]};
    int64_t rs[3] = {p.H_kv * p.N_kv * p.d, p.N_kv * p.d, p.d};
    if (launch_rope(K, k_rot, p.B, p.H_kv, p.N_kv, p.d, ks, rs, log2_base, s) != hipSuccess)
        return ATTN_ERR_HIP;
    KernelArgs a = make_args(plan, Q, k_rot, V, O, lse);
    a.k_sb = rs[0];
    a.k_sh = rs[1];
    a.k_sn = (int32_t)rs[2];
    a.v_in_k = 0;
    a.rope_log2_base = log2_base;
    hipError_t e = p.d == 64 ? (p.causal ? launch<64, true, __bf16, false, true>(plan, a, s)
                                         : launch<64, false, __bf16, false, true>(plan, a, s))
                             : (p.causal ? launch<128, true, __bf16, false, true>(plan, a, s)
                                         : launch<128, false, __bf16, false, true>(plan, a, s));
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

void attn_fwd_destroy(attn_fwd_plan *plan) { delete plan; }

const char *attn_status_str(attn_status status) {
    switch (status) {
        case ATTN_OK: return "ATTN_OK";
        case ATTN_ERR_INVALID: return "ATTN_ERR_INVALID";
        case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
        case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
        case ATTN_ERR_NOMEM: return "ATTN_ERR_NOMEM";
        case ATTN_ERR_TOO_LARGE: return "ATTN_ERR_TOO_LARGE";
    }
    return "ATTN_ERR_UNKNOWN";
}

int32_t attn_fwd_split_count(const attn_fwd_plan *plan) {
    if (!plan || !split_supported(plan)) return 0;
    return auto_splits(plan);
}

int64_t attn_fwd_split_workspace_bytes(const attn_fwd_plan *plan, int32_t n_splits) {
    if (!plan || !split_supported(plan)) return -1;
    if (n_splits <= 0) n_splits = auto_splits(plan);
    if (n_splits > kMaxSplits) return -1;
    return split_workspace(plan, n_splits);
}

attn_status attn_fwd_run_split(const attn_fwd_plan *plan, const void *Q, const void *K, const void *V,
                               void *O, float *lse, int32_t n_splits, void *workspace,
                               int64_t workspace_bytes, void *stream) {
    if (!plan || !Q || !K || !V || !O || !workspace) return ATTN_ERR_INVALID;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(workspace) ||
        (lse && ((uintptr_t)lse & 3u)))
        return ATTN_ERR_INVALID;
    if (!split_supported(plan)) return ATTN_ERR_UNSUPPORTED;
    if (n_splits <= 0) n_splits = auto_splits(plan);
    if (n_splits > kMaxSplits) return ATTN_ERR_INVALID;
    if (workspace_bytes < split_workspace(plan, n_splits)) return ATTN_ERR_INVALID;
    const KernelArgs a = make_args(plan, Q, K, V, O, lse);
    if (wide_split(plan) && !a.v_in_k) return ATTN_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    const hipError_t e = wide_split(plan) ? launch_wide_split(plan, a, n_splits, (float *)workspace, s)
                         : plan->variant == V_D128_BF16 ? launch_split<128>(plan, a, n_splits, (float *)workspace, s)
                                                        : launch_split<64>(plan, a, n_splits, (float *)workspace, s);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_fwd_run_split_noalloc(const attn_fwd_plan *plan, const void *Q, const void *K,
                                       const void *V, void *O, float *lse, int32_t n_splits,
                                       void *stream) {
    // every argument check comes before the first HIP call
    if (!plan || !Q || !K || !V || !O) return ATTN_ERR_INVALID;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) ||
        (lse && ((uintptr_t)lse & 3u)))
        return ATTN_ERR_INVALID;
    if (!split_supported(plan)) return ATTN_ERR_UNSUPPORTED;
    if (n_splits <= 0) n_splits = auto_splits(plan);
    if (n_splits > kMaxSplits) return ATTN_ERR_INVALID;
    const int64_t need = split_workspace(plan, n_splits);
    if (need > ATTN_SPLIT_SCRATCH_BYTES) return ATTN_ERR_TOO_LARGE;
    const KernelArgs a = make_args(plan, Q, K, V, O, lse);
    if (wide_split(plan) && !a.v_in_k) return ATTN_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    void *ws = nullptr;
    if (scratch_address(s, &ws) != hipSuccess) return ATTN_ERR_HIP;
    const hipError_t e = wide_split(plan) ? launch_wide_split(plan, a, n_splits, (float *)ws, s)
                         : plan->variant == V_D128_BF16 ? launch_split<128>(plan, a, n_splits, (float *)ws, s)
                                                        : launch_split<64>(plan, a, n_splits, (float *)ws, s);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_fwd_plan_info(const attn_fwd_plan *plan, int64_t *grid, int32_t *block,
                               int32_t *tile_q, int32_t *tile_k, int32_t *lds_bytes) {
    if (!plan) return ATTN_ERR_INVALID;
    if (grid) *grid = plan->grid;
    if (block) *block = plan->block;
    if (tile_q) *tile_q = plan->tile_q;
    if (tile_k) *tile_k = plan->tile_k;
    if (lds_bytes) *lds_bytes = plan->lds_bytes;
    return ATTN_OK;
}

}  // extern "C"
