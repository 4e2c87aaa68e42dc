// moe_combine: out[t, :] = sum_j w[t, j] * y[t*k + j, :] in fp32 (y is fp16
// or fp32).
//
// The k rows of a token are adjacent in y (token, slot order), so each
// thread streams eight elements (16 bytes of fp16, two 16-byte chunks of
// fp32) of those rows and writes 8 outputs: fully coalesced, HBM-bound. One workgroup per token, 256 threads; a
// thread covers hidden positions 8*tid + 2048*m.
#include "abi_util.h"
#include "moe_common.h"

namespace moe {

constexpr int kCombineThreads = 256;
constexpr int kCombineBatch = 8;  // rows of a token loaded together

// Eight consecutive elements of y as fp32. y is read once, so the loads
// are non-temporal (skewed and large: 115 -> 101 us).
template <bool Y16>
__device__ __forceinline__ void load_y8(const void* y, int64_t idx, float (&v)[8]) {
    if constexpr (Y16) {
        const u32x4 p = __builtin_nontemporal_load((const u32x4*)((const _Float16*)y + idx));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[2 * q] = (float)__builtin_bit_cast(_Float16, (uint16_t)(p[q] & 0xffffu));
            v[2 * q + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(p[q] >> 16));
        }
    } else {
        const f32x4 a = __builtin_nontemporal_load((const f32x4*)((const float*)y + idx));
        const f32x4 b = __builtin_nontemporal_load((const f32x4*)((const float*)y + idx + 4));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[q] = a[q];
            v[4 + q] = b[q];
        }
    }
}

template <bool Y16, bool OUT_F32>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const void* __restrict__ y,
                                                                  const float* __restrict__ w, int k, int H,
                                                                  void* __restrict__ out) {
    const int64_t t = blockIdx.x;
    const int64_t yt = t * k * (int64_t)H;
    const float* wt = w + t * k;
    for (int h = threadIdx.x * 8; h < H; h += kCombineThreads * 8) {
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.f;
        // The k rows are taken kCombineBatch at a time with every load of a
        // batch issued before any is used (one load per trip of a loop over
        // k waits for each row in turn). Slots past k re-read row k-1 and
        // are left out of the sum by a select, so a non-finite y there
        // cannot reach it; each kept row adds wj * y in row order as before.
        for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
            float wj[kCombineBatch], v[kCombineBatch][8];
#pragma unroll
            for (int u = 0; u < kCombineBatch; ++u) {
                const int j = min(j0 + u, k - 1);
                wj[u] = wt[j];
                load_y8<Y16>(y, yt + (int64_t)j * H + h, v[u]);
            }
#pragma unroll
            for (int u = 0; u < kCombineBatch; ++u) {
                const bool use = j0 + u < k;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float sum = acc[q] + wj[u] * v[u][q];
                    acc[q] = use ? sum : acc[q];
                }
            }
        }
        if (OUT_F32) {
            float* o = (float*)out + t * H + h;
            *(f32x4*)o = f32x4{acc[0], acc[1], acc[2], acc[3]};
            *(f32x4*)(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
        } else {
            u32x4 p;
#pragma unroll
            for (int q = 0; q < 4; ++q) p[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
            *(u32x4*)((uint16_t*)out + t * H + h) = p;
        }
    }
}

}  // namespace moe

extern "C" int moe_combine(const void* y, int32_t y_dtype, const float* topk_weights, int64_t T, int32_t k,
                           int32_t H, void* out, int32_t out_dtype, void* stream) {
    using namespace moe;
    clear_error();
    if (T < 0 || k < 0 || H < 0) return set_error(MOE_ERR_INVALID, "moe_combine: negative size");
    if (k < 1 || k > kMaxTopK) return set_error(MOE_ERR_UNSUPPORTED, "moe_combine: k=%d outside [1, 32]", k);
    if (H == 0 || H % 64) return set_error(MOE_ERR_UNSUPPORTED, "moe_combine: H=%d is not a positive multiple of 64", H);
    if (y_dtype != MOE_DTYPE_FP16 && y_dtype != MOE_DTYPE_FP32)
        return set_error(MOE_ERR_INVALID, "moe_combine: y_dtype=%d is neither fp16 (2) nor fp32 (1)", y_dtype);
    if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_FP32)
        return set_error(MOE_ERR_INVALID, "moe_combine: out_dtype=%d is neither bf16 (0) nor fp32 (1)", out_dtype);
    if (T * (int64_t)k >= ((int64_t)1 << 31)) return set_error(MOE_ERR_UNSUPPORTED, "moe_combine: T*k too large");
    if (T == 0) return MOE_OK;
    if (!y || !topk_weights || !out) return set_error(MOE_ERR_INVALID, "moe_combine: required pointer is NULL");
    if (((uintptr_t)y | (uintptr_t)out) & 15)
        return set_error(MOE_ERR_INVALID, "moe_combine: y and out must be 16-byte aligned");
    if (T >= ((int64_t)1 << 31)) return set_error(MOE_ERR_UNSUPPORTED, "moe_combine: T too large");
    const dim3 grid((unsigned)T), block(kCombineThreads);
    hipStream_t s = (hipStream_t)stream;
    const bool y16 = y_dtype == MOE_DTYPE_FP16, o32 = out_dtype == MOE_OUT_FP32;
    if (y16 && o32)
        hipLaunchKernelGGL((combine_kernel<true, true>), grid, block, 0, s, y, topk_weights, (int)k, (int)H, out);
    else if (y16)
        hipLaunchKernelGGL((combine_kernel<true, false>), grid, block, 0, s, y, topk_weights, (int)k, (int)H, out);
    else if (o32)
        hipLaunchKernelGGL((combine_kernel<false, true>), grid, block, 0, s, y, topk_weights, (int)k, (int)H, out);
    else
        hipLaunchKernelGGL((combine_kernel<false, false>), grid, block, 0, s, y, topk_weights, (int)k, (int)H, out);
    return check_launch("moe_combine");
}
