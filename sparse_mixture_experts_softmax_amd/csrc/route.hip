// moe_route: router linear (fp32 logits on the matrix cores), softmax over
// all experts, top-k in torch.topk order and optional renormalisation.
//
// One workgroup owns 16 tokens. Phase 1 computes their [16, E] logits with
// v_mfma_f32_16x16x32_bf16, the H dimension split across the workgroup's
// waves (each wave streams every expert's router row over its share of H,
// so many independent 16-byte loads are in flight), then sums the per-wave
// partials in LDS in a fixed order. Phase 2 gives each token to one wave:
// every lane holds up to four of the token's logits, and the softmax max,
// the softmax sum and each of the k arg-max rounds are wave reductions.
#include "abi_util.h"
#include "moe_common.h"

namespace moe {

constexpr int kRouteTokens = 16;  // tokens per workgroup (the MFMA M size)
constexpr int kRouteWaves = 4;

struct ArgMax {
    float v;
    int i;
};

__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b) {
    // larger value first; equal values -> lower expert index first
    return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

// NT = 16-expert tiles covered (experts >= E read as zero rows).
template <int NT>
__global__ __launch_bounds__(kRouteWaves* kWave) void route_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, int64_t T, int H, int E,
    int k, int norm, int compute_logits) {
    __shared__ float part[kRouteWaves][kRouteTokens][kMaxExperts + 1];
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int64_t t0 = (int64_t)blockIdx.x * kRouteTokens;
    float* lg = &part[0][0][0];  // final [16][E] logits reuse the first partial slab

    if (compute_logits) {
        f32x4 acc[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int row = lane % 16;
        const int koff = (lane / 16) * 8;
        const bool row_ok = t0 + row < T;
        const uint16_t* xrow = x + (row_ok ? (t0 + row) * (int64_t)H : 0) + koff;
        const uint16_t* wrow[NT];
        bool e_ok[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int e = n * 16 + row;
            e_ok[n] = e < E;
            wrow[n] = wr + (e_ok[n] ? (int64_t)e * H : 0) + koff;
        }
        // this wave's contiguous share of the k-steps
        const int ksteps = H / 32;
        const int per = (ksteps + kRouteWaves - 1) / kRouteWaves;
        const int s_lo = wave * per, s_hi = min(ksteps, s_lo + per);
#pragma unroll 2
        for (int s = s_lo; s < s_hi; ++s) {
            // unconditional loads from clamped rows: rows past T are zeroed,
            // experts past E only feed logits that are never read
            const u32x4 a = sel(row_ok, ld16(xrow + s * 32));
            u32x4 b[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) b[n] = ld16(wrow[n] + s * 32);
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[n] = mfma16x16x32(a, b[n], acc[n]);
        }
        // D layout: lane holds rows 4*(lane/16)+i, column lane%16 of each tile
#pragma unroll
        for (int n = 0; n < NT; ++n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) part[wave][(lane / 16) * 4 + i][n * 16 + lane % 16] = acc[n][i];
        }
        __syncthreads();
        // fixed-order reduction over waves, + bias, store logits
        for (int idx = threadIdx.x; idx < kRouteTokens * E; idx += blockDim.x) {
            const int r = idx / E, e = idx % E;
            float s = part[0][r][e];
#pragma unroll
            for (int w = 1; w < kRouteWaves; ++w) s += part[w][r][e];
            if (bias) s += bias[e];
            part[0][r][e] = s;
            if (t0 + r < T) logits[(t0 + r) * E + e] = s;
        }
    } else {
        for (int idx = threadIdx.x; idx < kRouteTokens * E; idx += blockDim.x) {
            const int r = idx / E, e = idx % E;
            part[0][r][e] = t0 + r < T ? logits[(t0 + r) * E + e] : 0.f;
        }
    }
    __syncthreads();

    for (int r = wave; r < kRouteTokens; r += kRouteWaves) {
        const int64_t t = t0 + r;
        if (t >= T) break;
        const float* row = lg + r * (kMaxExperts + 1);
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
            float sel = ex;
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) sel += wave_shfl_xor(sel, m);
            denom = sel;
        }
        if (lane < k) {
            topk_ids[t * k + lane] = my_id;
            topk_w[t * k + lane] = ex / denom;
        }
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
    const int64_t blocks = (T + kRouteTokens - 1) / kRouteTokens;
    const int ntiles = (E + 15) / 16;
    auto kern = ntiles <= 1 ? route_kernel<1>
              : ntiles <= 2 ? route_kernel<2>
              : ntiles <= 4 ? route_kernel<4>
              : ntiles <= 8 ? route_kernel<8>
                            : route_kernel<16>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kRouteWaves * kWave), 0, (hipStream_t)stream,
                       (const uint16_t*)x, (const uint16_t*)w_router, router_bias, logits, topk_ids, topk_weights, T,
                       (int)H, (int)E, (int)k, (int)(norm_topk_prob != 0), (int)(x != nullptr));
    return check_launch("moe_route");
}
