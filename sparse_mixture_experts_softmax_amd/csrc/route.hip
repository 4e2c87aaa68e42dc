// moe_route: router linear (fp32 logits on the matrix cores), softmax over
// all experts, top-k in torch.topk order and optional renormalisation.
//
// Two kernels. router_logits_kernel: one workgroup per (16 tokens, 16*NTW
// experts) tile, the H dimension split in four contiguous slices over the
// workgroup's four waves; each wave issues its slice's 16-byte loads in
// batches of eight k-steps and accumulates with v_mfma_f32_16x16x32_bf16;
// the four partials are summed in LDS in a fixed order, so the logits do not
// depend on scheduling. Small batches use one expert tile per workgroup (many
// workgroups pull the router weight in parallel); large ones use eight, so
// the activation rows are re-read less often. route_topk_kernel: one wave
// per token; each lane holds up to four of the token's logits, and the
// softmax max, the softmax sum and each of the k arg-max rounds are wave
// reductions. Selection uses the fp32 logits, so it is exact given them.
#include "abi_util.h"
#include "moe_common.h"

namespace moe {

constexpr int kRouteTokens = 16;  // tokens per logits tile (the MFMA M size)
constexpr int kRouteSlices = 4;   // waves per logits workgroup = slices of H
constexpr int kTopkWaves = 4;     // tokens per top-k workgroup

template <int NTW>
__global__ __launch_bounds__(kRouteSlices* kWave) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                                            const uint16_t* __restrict__ wr,
                                                                            const float* __restrict__ bias,
                                                                            float* __restrict__ logits, int64_t T,
                                                                            int H, int E) {
    constexpr int U = 8;  // k-steps per batch of loads
    constexpr int COLS = 16 * NTW;
    __shared__ float part[kRouteSlices][kRouteTokens][COLS + 1];
    const int lane = threadIdx.x % kWave, slice = threadIdx.x / kWave;
    const int64_t t0 = (int64_t)blockIdx.x * kRouteTokens;
    const int e0 = blockIdx.y * COLS;
    const int row = lane % 16, koff = (lane / 16) * 8;
    const bool row_ok = t0 + row < T;
    // unconditional loads from clamped rows: rows past T are zeroed, experts
    // past E only feed logits that are never stored
    const uint16_t* xrow = x + (row_ok ? (t0 + row) * (int64_t)H : 0) + koff;
    const uint16_t* wrow[NTW];
#pragma unroll
    for (int n = 0; n < NTW; ++n) wrow[n] = wr + (int64_t)min(e0 + n * 16 + row, E - 1) * H + koff;
    f32x4 acc[NTW];
#pragma unroll
    for (int n = 0; n < NTW; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int ksteps = H / 32;
    const int per = (ksteps + kRouteSlices - 1) / kRouteSlices;
    const int s_lo = slice * per, s_hi = min(ksteps, s_lo + per);
    int s = s_lo;
    for (; s + U <= s_hi; s += U) {
        u32x4 a[U], b[U][NTW];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            a[u] = sel(row_ok, ld16(xrow + (s + u) * 32));
#pragma unroll
            for (int n = 0; n < NTW; ++n) b[u][n] = ld16(wrow[n] + (s + u) * 32);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int n = 0; n < NTW; ++n) acc[n] = mfma16x16x32(a[u], b[u][n], acc[n]);
    }
    for (; s < s_hi; ++s) {
        const u32x4 a = sel(row_ok, ld16(xrow + s * 32));
#pragma unroll
        for (int n = 0; n < NTW; ++n) acc[n] = mfma16x16x32(a, ld16(wrow[n] + s * 32), acc[n]);
    }
    // D layout: lane holds rows 4*(lane/16)+i, column lane%16 of each tile
#pragma unroll
    for (int n = 0; n < NTW; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[slice][(lane / 16) * 4 + i][n * 16 + lane % 16] = acc[n][i];
    __syncthreads();
    for (int idx = threadIdx.x; idx < kRouteTokens * COLS; idx += blockDim.x) {
        const int r = idx / COLS, c = idx % COLS;
        const int e = e0 + c;
        if (t0 + r >= T || e >= E) continue;
        float v = part[0][r][c];
#pragma unroll
        for (int w = 1; w < kRouteSlices; ++w) v += part[w][r][c];
        if (bias) v += bias[e];
        logits[(t0 + r) * E + e] = v;
    }
}

struct ArgMax {
    float v;
    int i;
};

__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b) {
    // larger value first; equal values -> lower expert index first
    return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

__global__ __launch_bounds__(kTopkWaves* kWave) void route_topk_kernel(const float* __restrict__ logits,
                                                                       int32_t* __restrict__ topk_ids,
                                                                       float* __restrict__ topk_w, int64_t T, int E,
                                                                       int k, int norm) {
    const int lane = threadIdx.x % kWave;
    const int64_t t = (int64_t)blockIdx.x * kTopkWaves + threadIdx.x / kWave;
    if (t >= T) return;
    const float* row = logits + t * E;
    float v[4];
    bool live[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + i * kWave;
        live[i] = e < E;
        v[i] = live[i] ? row[e] : -INFINITY;
        mx = fmaxf(mx, v[i]);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, wave_shfl_xor(mx, m));
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) z += live[i] ? expf(v[i] - mx) : 0.f;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) z += wave_shfl_xor(z, m);

    int my_id = 0;
    float my_val = 0.f;
    for (int j = 0; j < k; ++j) {
        ArgMax best{-INFINITY, 0x7fffffff};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (live[i]) best = better(best, ArgMax{v[i], lane + i * kWave});
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            ArgMax o{wave_shfl_xor(best.v, m), wave_shfl_xor(best.i, m)};
            best = better(best, o);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + i * kWave == best.i) live[i] = false;
        if (lane == j) {
            my_id = best.i;
            my_val = best.v;
        }
    }
    const float ex = lane < k ? expf(my_val - mx) : 0.f;
    float denom = z;
    if (norm) {
        float sel_sum = ex;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) sel_sum += wave_shfl_xor(sel_sum, m);
        denom = sel_sum;
    }
    if (lane < k) {
        topk_ids[t * k + lane] = my_id;
        topk_w[t * k + lane] = ex / denom;
    }
}

}  // namespace moe

extern "C" int moe_route(const void* x, const void* w_router, const float* router_bias, float* logits,
                         int32_t* topk_ids, float* topk_weights, int64_t T, int32_t H, int32_t E, int32_t k,
                         int32_t norm_topk_prob, void* stream) {
    using namespace moe;
    clear_error();
    if (x == nullptr) {
        // logits are an input; H is not used
        if (T < 0 || E < 0 || k < 0) return set_error(MOE_ERR_INVALID, "moe_route: negative size");
        if (E < 1 || E > kMaxExperts) return set_error(MOE_ERR_UNSUPPORTED, "moe_route: E=%d outside [1, 256]", E);
        if (k < 1 || k > E || k > kMaxTopK) return set_error(MOE_ERR_UNSUPPORTED, "moe_route: k=%d invalid", k);
        if (T * (int64_t)k >= ((int64_t)1 << 31)) return set_error(MOE_ERR_UNSUPPORTED, "moe_route: T*k too large");
    } else {
        int rc = check_shape("moe_route", T, H, E, k, -1);
        if (rc) return rc;
        if (!w_router) return set_error(MOE_ERR_INVALID, "moe_route: w_router is NULL");
    }
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_weights)
        return set_error(MOE_ERR_INVALID, "moe_route: logits/topk_ids/topk_weights must not be NULL");
    if (x && (((uintptr_t)x | (uintptr_t)w_router) & 15))
        return set_error(MOE_ERR_INVALID, "moe_route: x and w_router must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    if (x) {
        const int64_t tblocks = (T + kRouteTokens - 1) / kRouteTokens;
        const int ntiles = (E + 15) / 16;
        if (tblocks >= ((int64_t)1 << 31)) return set_error(MOE_ERR_UNSUPPORTED, "moe_route: T too large");
        if (T <= 256 || ntiles < 8) {
            hipLaunchKernelGGL(router_logits_kernel<1>, dim3((unsigned)tblocks, (unsigned)ntiles),
                               dim3(kRouteSlices * kWave), 0, s, (const uint16_t*)x, (const uint16_t*)w_router,
                               router_bias, logits, T, (int)H, (int)E);
        } else {
            hipLaunchKernelGGL(router_logits_kernel<8>, dim3((unsigned)tblocks, (unsigned)((ntiles + 7) / 8)),
                               dim3(kRouteSlices * kWave), 0, s, (const uint16_t*)x, (const uint16_t*)w_router,
                               router_bias, logits, T, (int)H, (int)E);
        }
        int rc = check_launch("moe_route (logits)");
        if (rc) return rc;
    }
    const int64_t blocks = (T + kTopkWaves - 1) / kTopkWaves;
    if (blocks >= ((int64_t)1 << 31)) return set_error(MOE_ERR_UNSUPPORTED, "moe_route: T too large");
    hipLaunchKernelGGL(route_topk_kernel, dim3((unsigned)blocks), dim3(kTopkWaves * kWave), 0, s, logits, topk_ids,
                       topk_weights, T, (int)E, (int)k, (int)(norm_topk_prob != 0));
    return check_launch("moe_route (top-k)");
}
