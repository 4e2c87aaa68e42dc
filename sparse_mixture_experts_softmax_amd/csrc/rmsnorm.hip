// moe_fused_add_rmsnorm: the residual add and RMSNorm that precede the MoE
// layer, fused into one pass over the hidden state (in place):
//   with a residual:  residual <- bf16(residual + x), x <- rmsnorm(residual)
//   without (first layer): residual <- x,          x <- rmsnorm(x)
//   rmsnorm(r) = bf16(w * bf16(r / sqrt(mean(r^2) + eps)))
// One workgroup per row; each thread owns 8-element chunks (16-byte vectors)
// and keeps the new residual in registers between the sum of squares and
// the scaling, so the row is read once and written once per tensor.
#include "abi_util.h"
#include "moe_common.h"

namespace moe {

constexpr int kNormThreads = 256;

template <int NCH>  // 8-element chunks per thread: H <= NCH * 2048
__global__ __launch_bounds__(kNormThreads) void fused_add_rmsnorm_kernel(uint16_t* __restrict__ x,
                                                                         uint16_t* __restrict__ residual,
                                                                         const uint16_t* __restrict__ w, int H,
                                                                         float eps, int has_residual) {
    __shared__ float wave_sum[kNormThreads / kWave];
    const int64_t base = (int64_t)blockIdx.x * H;
    const int tid = threadIdx.x;
    float r[NCH][8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int h = (c * kNormThreads + tid) * 8;
        if (h >= H) continue;
        const u32x4 xv = *(const u32x4*)(x + base + h);
        u32x4 rv;
        if (has_residual) {
            const u32x4 ov = *(const u32x4*)(residual + base + h);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo = __uint_as_float(ov[q] << 16) + __uint_as_float(xv[q] << 16);
                const float hi = __uint_as_float(ov[q] & 0xffff0000u) + __uint_as_float(xv[q] & 0xffff0000u);
                rv[q] = pack_bf16x2(lo, hi);
            }
        } else {
            rv = xv;
        }
        *(u32x4*)(residual + base + h) = rv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            r[c][2 * q] = __uint_as_float(rv[q] << 16);
            r[c][2 * q + 1] = __uint_as_float(rv[q] & 0xffff0000u);
            ss += r[c][2 * q] * r[c][2 * q] + r[c][2 * q + 1] * r[c][2 * q + 1];
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += wave_shfl_xor(ss, m);
    if (tid % kWave == 0) wave_sum[tid / kWave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kNormThreads / kWave; ++i) tot += wave_sum[i];
    const float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int h = (c * kNormThreads + tid) * 8;
        if (h >= H) continue;
        const u32x4 wv = *(const u32x4*)(w + h);
        u32x4 ov;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float n0 = bf16_to_f32(f32_to_bf16(r[c][2 * q] * inv));
            const float n1 = bf16_to_f32(f32_to_bf16(r[c][2 * q + 1] * inv));
            ov[q] = pack_bf16x2(__uint_as_float(wv[q] << 16) * n0, __uint_as_float(wv[q] & 0xffff0000u) * n1);
        }
        *(u32x4*)(x + base + h) = ov;
    }
}

}  // namespace moe

extern "C" int moe_fused_add_rmsnorm(void* x, void* residual, const void* weight, int64_t T, int32_t H, float eps,
                                     int32_t has_residual, void* stream) {
    using namespace moe;
    clear_error();
    if (T < 0 || H < 0) return set_error(MOE_ERR_INVALID, "moe_fused_add_rmsnorm: negative size");
    if (H == 0 || H % 8 || H > 8 * 2048)
        return set_error(MOE_ERR_UNSUPPORTED, "moe_fused_add_rmsnorm: H=%d must be a multiple of 8 in [8, 16384]", H);
    if (!(eps >= 0.f)) return set_error(MOE_ERR_INVALID, "moe_fused_add_rmsnorm: eps must be >= 0");
    if (T == 0) return MOE_OK;
    if (!x || !residual || !weight) return set_error(MOE_ERR_INVALID, "moe_fused_add_rmsnorm: NULL pointer");
    if (((uintptr_t)x | (uintptr_t)residual | (uintptr_t)weight) & 15)
        return set_error(MOE_ERR_INVALID, "moe_fused_add_rmsnorm: pointers must be 16-byte aligned");
    if (x == residual) return set_error(MOE_ERR_INVALID, "moe_fused_add_rmsnorm: x and residual must not alias");
    if (T >= ((int64_t)1 << 31)) return set_error(MOE_ERR_UNSUPPORTED, "moe_fused_add_rmsnorm: T too large");
    const int nch = (H + 2047) / 2048;
    auto kern = nch <= 1 ? fused_add_rmsnorm_kernel<1>
              : nch <= 2 ? fused_add_rmsnorm_kernel<2>
              : nch <= 4 ? fused_add_rmsnorm_kernel<4>
                         : fused_add_rmsnorm_kernel<8>;
    hipLaunchKernelGGL(kern, dim3((unsigned)T), dim3(kNormThreads), 0, (hipStream_t)stream, (uint16_t*)x,
                       (uint16_t*)residual, (const uint16_t*)weight, (int)H, eps, (int)(has_residual != 0));
    return check_launch("moe_fused_add_rmsnorm");
}
