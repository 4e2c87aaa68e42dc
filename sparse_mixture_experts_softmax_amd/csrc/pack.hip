// moe_pack_weights: rewrite row-major expert weights [E, N, K] into the
// fragment layout the grouped GEMMs stream.
//
// The rows of each expert are cut into 16-row bands and each band into
// 32-column k-steps. One (band, k-step) block is the B operand of one
// v_mfma_f32_16x16x32_bf16 and is stored as 512 contiguous bf16 (1 KB):
// lane l of a wave owns elements [8l, 8l+8), which hold row l%16 of the band,
// columns 8*(l/16) .. 8*(l/16)+7 of the k-step. Blocks are stored band-major,
// k-step-minor, so a wave streaming one band reads 1 KB contiguous per load
// instruction. For a merged gate/up weight (gated) the gate bands and up
// bands are interleaved (gate band b, up band b, gate band b+1, ...), so the
// gate and up rows that feed the same output columns form one contiguous
// run. The packed tensor has the same size as the row-major one.
#include "abi_util.h"
#include "moe_common.h"

namespace moe {

constexpr int kPackThreads = 256;

__global__ __launch_bounds__(kPackThreads) void pack_kernel(const uint16_t* __restrict__ src,
                                                            uint16_t* __restrict__ dst, int64_t chunks, int N, int K,
                                                            int gated) {
    const int64_t c = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;  // 16-byte chunk of dst
    if (c >= chunks) return;
    const int lane = (int)(c % 64);
    const int64_t blk = c / 64;  // (e, band, kstep) block
    const int ksteps = K / 32, bands = N / 16;
    const int s = (int)(blk % ksteps);
    const int64_t eb = blk / ksteps;
    const int band = (int)(eb % bands);
    const int64_t e = eb / bands;
    int src_band = band;
    if (gated) src_band = (band % 2 == 0) ? band / 2 : bands / 2 + band / 2;  // gate rows first, then up rows
    const int64_t row = (int64_t)src_band * 16 + lane % 16;
    const int64_t col = (int64_t)s * 32 + (lane / 16) * 8;
    *(u32x4*)(dst + c * 8) = *(const u32x4*)(src + (e * N + row) * K + col);
}

}  // namespace moe

extern "C" size_t moe_packed_weight_bytes(int32_t E, int32_t N, int32_t K) {
    if (E < 1 || N < 16 || K < 32 || N % 16 || K % 32) return 0;
    return (size_t)E * (size_t)N * (size_t)K * 2;
}

extern "C" int moe_pack_weights(const void* w, void* w_packed, int32_t E, int32_t N, int32_t K, int32_t gated,
                                void* stream) {
    using namespace moe;
    clear_error();
    if (E < 0 || N < 0 || K < 0) return set_error(MOE_ERR_INVALID, "moe_pack_weights: negative size");
    if (E < 1 || N < 16 || K < 32 || N % 16 || K % 32)
        return set_error(MOE_ERR_UNSUPPORTED, "moe_pack_weights: need E >= 1, N %% 16 == 0, K %% 32 == 0 (E=%d N=%d K=%d)",
                         E, N, K);
    if (gated && N % 32)
        return set_error(MOE_ERR_UNSUPPORTED, "moe_pack_weights: gated weight needs N = 2I with I %% 16 == 0 (N=%d)", N);
    if (!w || !w_packed) return set_error(MOE_ERR_INVALID, "moe_pack_weights: NULL pointer");
    if (((uintptr_t)w | (uintptr_t)w_packed) & 15)
        return set_error(MOE_ERR_INVALID, "moe_pack_weights: pointers must be 16-byte aligned");
    if (w == w_packed) return set_error(MOE_ERR_INVALID, "moe_pack_weights: packing cannot be done in place");
    const int64_t chunks = (int64_t)E * N * K / 8;
    const int64_t grid = (chunks + kPackThreads - 1) / kPackThreads;
    if (grid >= ((int64_t)1 << 31)) return set_error(MOE_ERR_UNSUPPORTED, "moe_pack_weights: tensor too large");
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)grid), dim3(kPackThreads), 0, (hipStream_t)stream,
                       (const uint16_t*)w, (uint16_t*)w_packed, chunks, (int)N, (int)K, (int)(gated != 0));
    return check_launch("moe_pack_weights");
}
