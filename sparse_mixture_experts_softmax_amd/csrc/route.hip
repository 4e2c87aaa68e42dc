// moe_route: router linear (fp32 logits on the matrix cores), softmax over
// all experts, top-k in torch.topk order and optional renormalisation.
//
// Two kernels. router_logits_kernel: one workgroup per (16 tokens, 16*NTW
// experts) tile, the H dimension split in four contiguous slices over the
// workgroup's four waves; each wave issues its slice's 16-byte loads in
// batches of k-steps (16 for small batches, 8 for large) and accumulates
// with v_mfma_f32_16x16x32_bf16;
// the four partials are summed in LDS in a fixed order, so the logits do not
// depend on scheduling. Small batches use one expert tile per workgroup (many
// workgroups pull the router weight in parallel); large ones use eight, so
// the activation rows are re-read less often. Top-k: for k <= 16,
// route_topk_row_kernel gives each token one 16-lane row of a wave; above,
// route_topk_kernel gives it a whole wave (each lane holding up to four of
// the token's logits). Each of the k arg-max rounds and the softmax sums are
// reductions on DPP lane permutations (no LDS). Selection uses the fp32
// logits, so it is exact given them.
#include "abi_util.h"
#include "moe_common.h"

namespace moe {

constexpr int kRouteTokens = 16;  // tokens per logits tile (the MFMA M size)
constexpr int kRouteSlices = 4;   // waves per logits workgroup = slices of H
constexpr int kTopkWaves = 4;     // tokens per top-k workgroup

// The residual add + RMSNorm that precedes the layer, fused into the
// router's read of x (moe_fused_add_rmsnorm_route): the router kernels then
// read x and the residual, form the new residual r = bf16(residual + x) (or
// x for the first layer), the row's inv = 1 / sqrt(mean(r^2) + eps) and the
// normalized row bf16(w * bf16(r * inv)), multiply that with the router
// weight, and the workgroups of the first expert tile write r and the
// normalized row out. Every router workgroup of a token block reads the
// block's rows, so the outputs go to other buffers than the inputs.
struct NormArgs {
    const uint16_t* res;  // [T, H] residual in (ignored without has_res)
    const uint16_t* w;    // [H] norm weight
    uint16_t* x_out;      // [T, H] normalized x
    uint16_t* res_out;    // [T, H] new residual
    float eps;
    int has_res;
};

// New residual of one 16-byte chunk: bf16(fp32(res) + fp32(x)), or x.
__device__ __forceinline__ u32x4 new_residual(u32x4 xv, u32x4 rv, int has_res) {
    if (!has_res) return xv;
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float lo = __uint_as_float(rv[q] << 16) + __uint_as_float(xv[q] << 16);
        const float hi = __uint_as_float(rv[q] & 0xffff0000u) + __uint_as_float(xv[q] & 0xffff0000u);
        o[q] = pack_bf16x2(lo, hi);
    }
    return o;
}

// Adds the squares of a chunk's eight values to ss, in element order.
__device__ __forceinline__ float add_squares(float ss, u32x4 r) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float lo = __uint_as_float(r[q] << 16), hi = __uint_as_float(r[q] & 0xffff0000u);
        ss += lo * lo;
        ss += hi * hi;
    }
    return ss;
}

// bf16(w * bf16(r * inv)) of one chunk (the weight product of two bf16
// values is exact in fp32 and rounded once).
__device__ __forceinline__ u32x4 normalized(u32x4 r, u32x4 w, float inv) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float n0 = bf16_to_f32(f32_to_bf16(__uint_as_float(r[q] << 16) * inv));
        const float n1 = bf16_to_f32(f32_to_bf16(__uint_as_float(r[q] & 0xffff0000u) * inv));
        o[q] = pack_bf16x2(__uint_as_float(w[q] << 16) * n0, __uint_as_float(w[q] & 0xffff0000u) * n1);
    }
    return o;
}

// Sum of a lane's squares over the four lanes holding the same row (lanes
// l, l^16, l^32, l^48): every lane receives its row's total.
__device__ __forceinline__ float row_total(float ss) {
    ss += wave_shfl_xor(ss, 16);
    ss += wave_shfl_xor(ss, 32);
    return ss;
}

// NORM: 0 = plain router; 1 = fused norm re-reading x and the residual in
// the second pass; 2 = fused norm keeping the new residual rows in LDS
// between the passes (16 x (H + 8) bf16, plus the norm weight: dynamic LDS)
// and fetching the first batch of router fragments during the first pass.
template <int NTW, int U, int NORM>
__global__ __launch_bounds__(kRouteSlices* kWave) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                                            const uint16_t* __restrict__ wr,
                                                                            const float* __restrict__ bias,
                                                                            float* __restrict__ logits, int64_t T,
                                                                            int H, int E, NormArgs na) {
    // U: k-steps per batch of loads (all loads of a batch are issued before
    // the first MFMA: one memory wait per batch)
    constexpr int COLS = 16 * NTW;
    __shared__ float part[kRouteSlices][kRouteTokens][COLS + 1];
    __shared__ float part_ss[kRouteSlices][kRouteTokens];
    extern __shared__ __attribute__((aligned(16))) char norm_lds[];
    const int lane = threadIdx.x % kWave, slice = threadIdx.x / kWave;
    const int64_t t0 = (int64_t)blockIdx.x * kRouteTokens;
    const int e0 = blockIdx.y * COLS;
    const int row = lane % 16, koff = (lane / 16) * 8;
    const bool row_ok = t0 + row < T;
    // unconditional loads from clamped rows: rows past T are zeroed, experts
    // past E only feed logits that are never stored
    const int64_t xoff = (row_ok ? (t0 + row) * (int64_t)H : 0) + koff;
    const uint16_t* xrow = x + xoff;
    const uint16_t* wrow[NTW];
#pragma unroll
    for (int n = 0; n < NTW; ++n) wrow[n] = wr + (int64_t)min(e0 + n * 16 + row, E - 1) * H + koff;
    f32x4 acc[NTW];
#pragma unroll
    for (int n = 0; n < NTW; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int ksteps = H / 32;
    const int per = (ksteps + kRouteSlices - 1) / kRouteSlices;
    const int s_lo = slice * per, s_hi = min(ksteps, s_lo + per);

    float inv = 0.f;
    const uint16_t* rrow = nullptr;
    const bool writer = NORM && blockIdx.y == 0 && row_ok;
    const int rstride = H + 8;  // LDS row stride of the staged residual (16-byte pad against bank conflicts)
    uint16_t* r_lds = (uint16_t*)norm_lds;
    uint16_t* w_lds = r_lds + kRouteTokens * rstride;
    u32x4 b0[U][NTW];  // NORM == 2: the first batch of router fragments, fetched during pass 1
    if constexpr (NORM == 2) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int n = 0; n < NTW; ++n) b0[u][n] = ld16(wrow[n] + min(s_lo + u, ksteps - 1) * 32);
        for (int h = (int)threadIdx.x * 8; h < H; h += kRouteSlices * kWave * 8) *(u32x4*)(w_lds + h) = ld16(na.w + h);
    }
    if constexpr (NORM != 0) {
        // pass 1: the row's sum of squares of the new residual (this wave's
        // slice, k-step by k-step, then the four lanes of a row, then the
        // four slices in order)
        rrow = na.has_res ? na.res + xoff : xrow;
        constexpr int U1 = NORM == 2 ? 8 : U;
        float ss = 0.f;
        auto take = [&](u32x4 xv, u32x4 rv, int s_) {
            const u32x4 r = new_residual(xv, rv, na.has_res);
            if constexpr (NORM == 2) *(u32x4*)(r_lds + row * rstride + s_ * 32 + koff) = r;
            ss = add_squares(ss, r);
        };
        int s = s_lo;
        for (; s + U1 <= s_hi; s += U1) {
            u32x4 xv[U1], rv[U1];
#pragma unroll
            for (int u = 0; u < U1; ++u) {
                xv[u] = ld16(xrow + (s + u) * 32);
                rv[u] = ld16(rrow + (s + u) * 32);
            }
#pragma unroll
            for (int u = 0; u < U1; ++u) take(xv[u], rv[u], s + u);
        }
        for (; s < s_hi; ++s) take(ld16(xrow + s * 32), ld16(rrow + s * 32), s);
        ss = row_total(ss);
        if (lane < 16) part_ss[slice][row] = ss;
        __syncthreads();  // also publishes the staged residual rows and norm weight
        float tot = 0.f;
#pragma unroll
        for (int sl = 0; sl < kRouteSlices; ++sl) tot += part_ss[sl][row];
        inv = 1.0f / sqrtf(tot / (float)H + na.eps);
    }
    // A operand of k-step s: the x chunk, or (fused norm) its normalized
    // value, written out with the new residual by the first expert tile
    auto a_chunk = [&](u32x4 xv, u32x4 rv, u32x4 wv, int s_) -> u32x4 {
        if constexpr (NORM == 0) {
            return sel(row_ok, xv);
        } else {
            const u32x4 r = NORM == 2 ? *(const u32x4*)(r_lds + row * rstride + s_ * 32 + koff)
                                      : new_residual(xv, rv, na.has_res);
            const u32x4 xn = normalized(r, NORM == 2 ? *(const u32x4*)(w_lds + s_ * 32 + koff) : wv, inv);
            if (writer) {
                *(u32x4*)(na.res_out + xoff + s_ * 32) = r;
                *(u32x4*)(na.x_out + xoff + s_ * 32) = xn;
            }
            return sel(row_ok, xn);
        }
    };
    if constexpr (NORM == 2) {
        // pass 2 from LDS: only the router fragments come from memory, the
        // first batch already in flight
        for (int s = s_lo; s < s_hi; s += U) {
            u32x4 b[U][NTW];
            if (s == s_lo) {
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int n = 0; n < NTW; ++n) b[u][n] = b0[u][n];
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int n = 0; n < NTW; ++n) b[u][n] = ld16(wrow[n] + min(s + u, ksteps - 1) * 32);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (s + u >= s_hi) break;
                const u32x4 zero{0u, 0u, 0u, 0u};
                const u32x4 au = a_chunk(zero, zero, zero, s + u);
#pragma unroll
                for (int n = 0; n < NTW; ++n) acc[n] = mfma16x16x32(au, b[u][n], acc[n]);
            }
        }
    } else {
        int s = s_lo;
        for (; s + U <= s_hi; s += U) {
            u32x4 a[U], b[U][NTW], rv[U], wv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                a[u] = ld16(xrow + (s + u) * 32);
                if constexpr (NORM == 1) {
                    rv[u] = ld16(rrow + (s + u) * 32);
                    wv[u] = ld16(na.w + (s + u) * 32 + koff);
                }
#pragma unroll
                for (int n = 0; n < NTW; ++n) b[u][n] = ld16(wrow[n] + (s + u) * 32);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const u32x4 au = a_chunk(a[u], NORM ? rv[u] : a[u], NORM ? wv[u] : a[u], s + u);
#pragma unroll
                for (int n = 0; n < NTW; ++n) acc[n] = mfma16x16x32(au, b[u][n], acc[n]);
            }
        }
        for (; s < s_hi; ++s) {
            const u32x4 xv = ld16(xrow + s * 32);
            const u32x4 a = a_chunk(xv, NORM ? ld16(rrow + s * 32) : xv, NORM ? ld16(na.w + s * 32 + koff) : xv, s);
#pragma unroll
            for (int n = 0; n < NTW; ++n) acc[n] = mfma16x16x32(a, ld16(wrow[n] + s * 32), acc[n]);
        }
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

// Large batches: a workgroup covers 64 tokens (one 16-token MFMA tile per
// wave) x 16*ET experts, so the router weight is read once per 64 tokens
// instead of once per 16. Both operands go global -> LDS by direct copies
// (global_load_lds_dwordx4, lane l of a copy lands at base + 16*l, i.e. as
// an MFMA fragment), in chunks of RC k-steps through a ring of NB chunk
// buffers with NB-1 chunks in flight: the router fragments of a chunk are
// copied once and read by all four waves, each wave copies its own
// activation fragments. The sums follow router_logits_kernel exactly: H is
// cut into the same four slices, each slice accumulated k-step by k-step
// into its own accumulator, the four slice sums added in order, then the
// bias; a token's logits are the same bits whichever kernel and batch size
// computed them. Needs the slice length (H/32/4 k-steps) to be a multiple
// of RC.
constexpr int kRouteWideTokens = 64;
constexpr int kRouteChunk = 4;  // k-steps per chunk (RC)

// s_waitcnt until at most `later` chunks of OPS copies each remain in
// flight (later <= L; only the waits that can occur are instantiated).
template <int L, int OPS>
__device__ __forceinline__ void wait_for_later(int later) {
    if constexpr (L > 0) {
        if (later >= L) {
            vm_wait<L * OPS>();
            return;
        }
        wait_for_later<L - 1, OPS>(later);
    } else {
        vm_wait<0>();
    }
}

// With NORM (the fused residual add + RMSNorm), each chunk also holds the
// wave's residual fragments next to its activation fragments, and the norm
// weight is staged in LDS (H*2 bytes after the ring) once per workgroup.
template <int ET, int NB_, bool NORM = false>
struct RouteWide {
    static constexpr int RC = kRouteChunk, NB = NB_, D = NB - 1;
    static constexpr int W_COPIES = ET * RC / kRouteSlices;  // router fragments per wave per chunk
    static constexpr int X_COPIES = RC * (NORM ? 2 : 1);     // activation (+ residual) fragments per wave per chunk
    static constexpr int OPS = W_COPIES + X_COPIES;
    static constexpr int W_BYTES = ET * RC * 1024;
    static constexpr int X_BYTES = kRouteSlices * RC * 1024;
    static constexpr int CHUNK_BYTES = W_BYTES + X_BYTES * (NORM ? 2 : 1);
    static_assert((ET * RC) % kRouteSlices == 0, "router fragments split evenly over the waves");
    static_assert(OPS * (D - 1) < 64, "vmcnt range");
    static_assert(NB * CHUNK_BYTES <= 160 * 1024, "LDS");
};

template <int ET, int NB_, bool NORM>
__global__ __launch_bounds__(kRouteSlices* kWave) void router_logits_wide_kernel(const uint16_t* __restrict__ x,
                                                                                 const uint16_t* __restrict__ wr,
                                                                                 const float* __restrict__ bias,
                                                                                 float* __restrict__ logits,
                                                                                 int64_t T, int H, int E, NormArgs na) {
    using C = RouteWide<ET, NB_, NORM>;
    constexpr int RC = C::RC, NB = C::NB, D = C::D;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int64_t t0 = (int64_t)blockIdx.x * kRouteWideTokens + wave * kRouteTokens;
    const int e0 = blockIdx.y * 16 * ET;
    const int row = lane % 16, koff = (lane / 16) * 8;
    // unconditional copies from clamped rows: rows past T are never stored,
    // experts past E only feed logits that are never stored
    const int64_t xoff = min(t0 + row, T - 1) * (int64_t)H + koff;
    const uint16_t* xsrc = x + xoff;
    const uint16_t* rsrc = NORM ? (na.has_res ? na.res + xoff : xsrc) : nullptr;
    const bool writer = NORM && blockIdx.y == 0 && t0 + row < T;
    // Copies of 8 rows x 2 k-steps (128 contiguous bytes of each row): copy
    // lane l fetches piece (l%8) ^ (l/8) of row l/8 (a piece is 8 elements;
    // pieces 0-3 are the first k-step), so piece p of row r lands in slot
    // r*8 + (p ^ r), which keeps the fragment reads of 8 consecutive rows on
    // distinct banks. Copy index: (16-row tile, 8-row half, k-step pair).
    const int crow = lane / 8, cpiece = (lane % 8) ^ (lane / 8);
    const uint16_t* wsrc[C::W_COPIES];
#pragma unroll
    for (int j = 0; j < C::W_COPIES; ++j) {
        const int f = wave * C::W_COPIES + j;
        const int pr = f % (RC / 2), half = (f / (RC / 2)) % 2, tile = f / RC;
        wsrc[j] = wr + (int64_t)min(e0 + 16 * tile + 8 * half + crow, E - 1) * H + pr * 64 + cpiece * 8;
    }
    const uint16_t* xcp[2];
    const uint16_t* rcp[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int64_t off = min(t0 + 8 * half + crow, T - 1) * (int64_t)H + cpiece * 8;
        xcp[half] = x + off;
        rcp[half] = NORM ? (na.has_res ? na.res + off : x + off) : nullptr;
    }
    // slot of this lane's fragment (row lane%16, k offset koff) of k-step s
    // within the copies of its 8-row half
    auto frag_slot = [&](int s) { return ((lane % 8) * 8 + (((s % 2) * 4 + lane / 16) ^ (lane % 8))) * 16; };
    const int ksteps = H / 32, per = ksteps / kRouteSlices, nchunk = ksteps / RC;
    auto issue = [&](int c) {
        char* buf = smem + (c % NB) * C::CHUNK_BYTES;
#pragma unroll
        for (int j = 0; j < C::W_COPIES; ++j) lds_dma16(wsrc[j] + c * RC * 32, buf + (wave * C::W_COPIES + j) * 1024);
#pragma unroll
        for (int q = 0; q < RC; ++q) {
            const int pr = q % (RC / 2), half = q / (RC / 2);
            lds_dma16(xcp[half] + c * RC * 32 + pr * 64, buf + C::W_BYTES + (wave * RC + q) * 1024);
        }
        if constexpr (NORM) {
#pragma unroll
            for (int q = 0; q < RC; ++q) {
                const int pr = q % (RC / 2), half = q / (RC / 2);
                lds_dma16(rcp[half] + c * RC * 32 + pr * 64, buf + C::W_BYTES + C::X_BYTES + (wave * RC + q) * 1024);
            }
        }
    };
    f32x4 acc[kRouteSlices][ET];
#pragma unroll
    for (int sl = 0; sl < kRouteSlices; ++sl)
#pragma unroll
        for (int j = 0; j < ET; ++j) acc[sl][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c = 0; c < D && c < nchunk; ++c) issue(c);
    float inv = 0.f;
    uint16_t* w_lds = (uint16_t*)(smem + NB * C::CHUNK_BYTES);
    if constexpr (NORM) {
        // the norm weight, once, into LDS
        for (int h = tid * 8; h < H; h += kRouteSlices * kWave * 8) *(u32x4*)(w_lds + h) = ld16(na.w + h);
        // the row's sum of squares of the new residual, per slice of H and
        // in the small-batch kernel's order (k-step by k-step in a lane, the
        // four lanes of a row, then the slices in order), so both kernels
        // normalize a row with the same inv
        float tot = 0.f;
        for (int sl = 0; sl < kRouteSlices; ++sl) {
            float ss = 0.f;
            constexpr int B8 = 8;
            int s = sl * per;
            for (; s + B8 <= (sl + 1) * per; s += B8) {
                u32x4 xv[B8], rv[B8];
#pragma unroll
                for (int u = 0; u < B8; ++u) {
                    xv[u] = ld16(xsrc + (s + u) * 32);
                    rv[u] = ld16(rsrc + (s + u) * 32);
                }
#pragma unroll
                for (int u = 0; u < B8; ++u) ss = add_squares(ss, new_residual(xv[u], rv[u], na.has_res));
            }
            for (; s < (sl + 1) * per; ++s)
                ss = add_squares(ss, new_residual(ld16(xsrc + s * 32), ld16(rsrc + s * 32), na.has_res));
            tot += row_total(ss);
        }
        inv = 1.0f / sqrtf(tot / (float)H + na.eps);
        __syncthreads();  // the norm weight is in LDS
    }
    int c = 0;
#pragma unroll
    for (int sl = 0; sl < kRouteSlices; ++sl) {
        for (int cc = 0; cc < per / RC; ++cc, ++c) {
            // this wave's copies of chunk c are done once at most the ops of
            // the later chunks already issued remain; the barrier publishes
            // the chunk and frees the buffer of chunk c - 1
            const int later = min(D - 1, nchunk - 1 - c);
            static_assert(D <= 5, "wait ladder covers up to four later chunks");
            wait_for_later<D - 1, C::OPS>(later);
            __builtin_amdgcn_s_barrier();
            if (c + D < nchunk) issue(c + D);
            const char* buf = smem + (c % NB) * C::CHUNK_BYTES;
#pragma unroll
            for (int s = 0; s < RC; ++s) {
                // this lane's 8-row half and k-step pair
                const int xq = (row / 8) * (RC / 2) + s / 2;
                u32x4 a = *(const u32x4*)(buf + C::W_BYTES + (wave * RC + xq) * 1024 + frag_slot(s));
                if constexpr (NORM) {
                    const int ks = c * RC + s;
                    const u32x4 rv =
                        *(const u32x4*)(buf + C::W_BYTES + C::X_BYTES + (wave * RC + xq) * 1024 + frag_slot(s));
                    const u32x4 r = new_residual(a, rv, na.has_res);
                    a = normalized(r, *(const u32x4*)(w_lds + ks * 32 + koff), inv);
                    if (writer) {
                        *(u32x4*)(na.res_out + xoff + ks * 32) = r;
                        *(u32x4*)(na.x_out + xoff + ks * 32) = a;
                    }
                }
#pragma unroll
                for (int j = 0; j < ET; ++j)
                    acc[sl][j] = mfma16x16x32(a, *(const u32x4*)(buf + (j * RC + xq) * 1024 + frag_slot(s)), acc[sl][j]);
            }
        }
    }
    // D layout: lane holds rows 4*(lane/16)+i, column lane%16 of each tile
#pragma unroll
    for (int j = 0; j < ET; ++j) {
        const int e = e0 + 16 * j + lane % 16;
        const float b = (bias && e < E) ? bias[e] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = t0 + (lane / 16) * 4 + i;
            float v = acc[0][j][i];
#pragma unroll
            for (int sl = 1; sl < kRouteSlices; ++sl) v += acc[sl][j][i];
            if (bias) v += b;
            if (t < T && e < E) logits[t * E + e] = v;
        }
    }
}

// Wave-wide reductions without LDS traffic: DPP lane permutations inside
// each row of 16 lanes (xor 1, xor 2, mirror within 8, mirror within 16)
// leave every lane holding its row's result; the four row results are then
// read with v_readlane and combined in a fixed order.
constexpr int kDppXor1 = 0xB1;         // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;         // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within each 8
constexpr int kDppMirror = 0x140;      // lane i <- 15 - i within each 16

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ uint64_t max_dpp(uint64_t v) {
    const uint64_t o = ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
    return o > v ? o : v;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), lane) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_dpp<kDppXor1>(v);
    v = max_dpp<kDppXor2>(v);
    v = max_dpp<kDppHalfMirror>(v);
    v = max_dpp<kDppMirror>(v);
    uint64_t m = readlane_u64(v, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const uint64_t o = readlane_u64(v, 16 * r);
        m = o > m ? o : m;
    }
    return m;
}

template <int CTRL>
__device__ __forceinline__ float add_dpp(float v) {
    return v + __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

__device__ __forceinline__ float wave_sum(float v) {
    v = add_dpp<kDppXor1>(v);
    v = add_dpp<kDppXor2>(v);
    v = add_dpp<kDppHalfMirror>(v);
    v = add_dpp<kDppMirror>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// Selection key of (logit, expert): the logit's bits mapped to an unsigned
// integer of the same order in the high word (-0 taken as +0), the
// complemented expert index in the low word, so the largest key is the
// largest logit and, among equal logits, the lowest expert. NaN logits rank
// below every number (high word 0); key 0 marks an expert already taken or
// past E.
__device__ __forceinline__ uint64_t select_key(float v, int e) {
    const uint32_t u = v == 0.f ? 0u : __float_as_uint(v);
    const uint32_t ord = (u & 0x7fffffffu) > 0x7f800000u ? 0u : ((u & 0x80000000u) ? ~u : (u | 0x80000000u));
    return ((uint64_t)ord << 32) | (uint32_t)~e;
}

__device__ __forceinline__ float key_logit(uint64_t key) {
    const uint32_t ord = (uint32_t)(key >> 32);
    return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
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
    uint64_t key[4];
    // all loads are issued before any is used; keys past E are masked
    // without a branch (a branch per key made each load wait for the last)
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = row[min(lane + i * kWave, E - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + i * kWave;
        key[i] = select_key(v[i], e) & (0ull - (uint64_t)(e < E));
    }
    // k rounds of a wave arg-max; lane j keeps the j-th pick
    int my_id = 0;
    float my_val = 0.f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        const int e = (int)~(uint32_t)best;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + i * kWave == e) key[i] = 0;
        if (lane == j) {
            my_id = e;
            my_val = key_logit(best);
        }
    }
    // softmax: the largest logit is the first pick
    const float mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_val), 0));
    const float ex = lane < k ? expf(my_val - mx) : 0.f;
    float denom;
    if (norm) {
        denom = wave_sum(ex);
    } else {
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) z += lane + i * kWave < E ? expf(v[i] - mx) : 0.f;
        denom = wave_sum(z);
    }
    if (lane < k) {
        topk_ids[t * k + lane] = my_id;
        topk_w[t * k + lane] = ex / denom;
    }
}

// The same selection with 16 lanes (one DPP row) per token, four tokens per
// wave, for k <= 16: every reduction stays inside a row, so no v_readlane,
// and a quarter of the waves. Lane r of a row holds experts r, r+16, ...
// (PER of them) and keeps pick r. With norm the weights are the same bits
// as route_topk_kernel's (the same four DPP steps over the same values).
constexpr int kTopkRowTokens = 16;  // tokens per workgroup (4 waves x 4 rows)

__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
    v = max_dpp<kDppXor1>(v);
    v = max_dpp<kDppXor2>(v);
    v = max_dpp<kDppHalfMirror>(v);
    return max_dpp<kDppMirror>(v);
}

__device__ __forceinline__ float row_sum(float v) {
    v = add_dpp<kDppXor1>(v);
    v = add_dpp<kDppXor2>(v);
    v = add_dpp<kDppHalfMirror>(v);
    return add_dpp<kDppMirror>(v);
}

template <int PER>
__global__ __launch_bounds__(kTopkWaves* kWave) void route_topk_row_kernel(const float* __restrict__ logits,
                                                                           int32_t* __restrict__ topk_ids,
                                                                           float* __restrict__ topk_w, int64_t T,
                                                                           int E, int k, int norm) {
    const int r = threadIdx.x % 16;
    const int64_t t = (int64_t)blockIdx.x * kTopkRowTokens + threadIdx.x / 16;
    if (t >= T) return;  // the whole row leaves together
    const float* row = logits + t * E;
    float v[PER];
    uint64_t key[PER];
    // as above: every load in flight at once, keys past E masked
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = row[min(r + 16 * i, E - 1)];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = r + 16 * i;
        key[i] = select_key(v[i], e) & (0ull - (uint64_t)(e < E));
    }
    int my_id = 0;
    float my_val = 0.f, mx = 0.f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < PER; ++i) best = key[i] > best ? key[i] : best;
        best = row_max_u64(best);
        const int e = (int)~(uint32_t)best;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (r + 16 * i == e) key[i] = 0;
        const float lv = key_logit(best);
        if (j == 0) mx = lv;  // softmax: the largest logit is the first pick
        if (r == j) {
            my_id = e;
            my_val = lv;
        }
    }
    const float ex = r < k ? expf(my_val - mx) : 0.f;
    float denom;
    if (norm) {
        denom = row_sum(ex);
    } else {
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) z += r + 16 * i < E ? expf(v[i] - mx) : 0.f;
        denom = row_sum(z);
    }
    if (r < k) {
        topk_ids[t * k + r] = my_id;
        topk_w[t * k + r] = ex / denom;
    }
}

template <int ET, int NB, bool NORM>
static int launch_route_wide(const void* x, const void* w_router, const float* bias, float* logits, int64_t T,
                             int32_t H, int32_t E, int ntiles, const NormArgs& na, hipStream_t s) {
    using C = RouteWide<ET, NB, NORM>;
    const dim3 grid((unsigned)((T + kRouteWideTokens - 1) / kRouteWideTokens), (unsigned)((ntiles + ET - 1) / ET));
    const int lds = C::NB * C::CHUNK_BYTES + (NORM ? H * 2 : 0);
    if (lds > 160 * 1024) return set_error(MOE_ERR_UNSUPPORTED, "moe_route: H=%d too large for the fused norm", H);
    static std::atomic<uint64_t> lds_set{0};
    const int rc = ensure_dynamic_lds((const void*)router_logits_wide_kernel<ET, NB, NORM>,
                                      NORM ? 160 * 1024 : lds, lds_set, "moe_route");
    if (rc) return rc;
    hipLaunchKernelGGL((router_logits_wide_kernel<ET, NB, NORM>), grid, dim3(kRouteSlices * kWave), lds, s,
                       (const uint16_t*)x, (const uint16_t*)w_router, bias, logits, T, (int)H, (int)E, na);
    return MOE_OK;
}

// Router logits (a1), optionally with the residual add + RMSNorm fused into
// the read of x (na != nullptr), then the softmax / top-k (a2). Arguments
// are checked by the callers.
template <bool NORM>
static int route_logits(const void* x, const void* w_router, const float* router_bias, float* logits, int64_t T,
                        int32_t H, int32_t E, const NormArgs& na, hipStream_t s) {
    const int64_t tblocks = (T + kRouteTokens - 1) / kRouteTokens;
    const int ntiles = (E + 15) / 16;
    if (tblocks >= ((int64_t)1 << 31)) return set_error(MOE_ERR_UNSUPPORTED, "moe_route: T too large");
    const int ksteps = H / 32;
    if (T > 256 && ksteps % (kRouteSlices * kRouteChunk) == 0) {
        // Each workgroup re-reads its 64 activation rows once per group of
        // 16*ET experts, so ET is as large as still gives a full round of
        // workgroups on the 256 CUs (one per CU, the deepest ring); below
        // that, ET = 2 with a shallower ring, two per CU. With the fused
        // norm each chunk also carries the residual, so the rings are one
        // or two chunks shallower.
        const int64_t tg = (T + kRouteWideTokens - 1) / kRouteWideTokens;
        int rc;
        if (tg * ((ntiles + 7) / 8) >= 256)
            rc = launch_route_wide<8, NORM ? 2 : 3, NORM>(x, w_router, router_bias, logits, T, H, E, ntiles, na, s);
        else if (tg * ((ntiles + 3) / 4) >= 256)
            rc = launch_route_wide<4, NORM ? 2 : 4, NORM>(x, w_router, router_bias, logits, T, H, E, ntiles, na, s);
        else if (tg * ((ntiles + 1) / 2) <= 256)
            rc = launch_route_wide<2, NORM ? 3 : 6, NORM>(x, w_router, router_bias, logits, T, H, E, ntiles, na, s);
        else
            rc = launch_route_wide<2, 3, NORM>(x, w_router, router_bias, logits, T, H, E, ntiles, na, s);
        if (rc) return rc;
    } else if (T <= 256 || ntiles < 8) {
        // one batch of loads per slice at H = 2048 (16 k-steps). With the
        // fused norm and H <= 4096 the new residual rows stay in LDS between
        // the passes; above, the second pass re-reads x and the residual
        // (batches of 8, as it also holds their chunks and the norm weight's).
        const dim3 grid((unsigned)tblocks, (unsigned)ntiles), block(kRouteSlices * kWave);
        if (!NORM) {
            hipLaunchKernelGGL((router_logits_kernel<1, 16, 0>), grid, block, 0, s, (const uint16_t*)x,
                               (const uint16_t*)w_router, router_bias, logits, T, (int)H, (int)E, na);
        } else if (H <= 4096) {
            const int lds = (kRouteTokens * (H + 8) + H) * 2;
            static std::atomic<uint64_t> lds_set{0};
            const int rc = ensure_dynamic_lds((const void*)router_logits_kernel<1, 16, 2>, 160 * 1024 - 8192,
                                              lds_set, "moe_route");
            if (rc) return rc;
            hipLaunchKernelGGL((router_logits_kernel<1, 16, 2>), grid, block, lds, s, (const uint16_t*)x,
                               (const uint16_t*)w_router, router_bias, logits, T, (int)H, (int)E, na);
        } else {
            hipLaunchKernelGGL((router_logits_kernel<1, 8, 1>), grid, block, 0, s, (const uint16_t*)x,
                               (const uint16_t*)w_router, router_bias, logits, T, (int)H, (int)E, na);
        }
    } else {
        hipLaunchKernelGGL((router_logits_kernel<8, NORM ? 4 : 8, NORM ? 1 : 0>),
                           dim3((unsigned)tblocks, (unsigned)((ntiles + 7) / 8)), dim3(kRouteSlices * kWave), 0, s,
                           (const uint16_t*)x, (const uint16_t*)w_router, router_bias, logits, T, (int)H, (int)E, na);
    }
    return check_launch("moe_route (logits)");
}

static int route_topk(const float* logits, int32_t* topk_ids, float* topk_weights, int64_t T, int32_t E, int32_t k,
                      int32_t norm_topk_prob, hipStream_t s) {
    const int64_t blocks = (T + kTopkWaves - 1) / kTopkWaves;
    if (blocks >= ((int64_t)1 << 31)) return set_error(MOE_ERR_UNSUPPORTED, "moe_route: T too large");
    if (k <= 16) {
        const dim3 grid((unsigned)((T + kTopkRowTokens - 1) / kTopkRowTokens)), block(kTopkWaves * kWave);
        if (E <= 128)
            hipLaunchKernelGGL((route_topk_row_kernel<8>), grid, block, 0, s, logits, topk_ids, topk_weights, T, (int)E,
                               (int)k, (int)(norm_topk_prob != 0));
        else
            hipLaunchKernelGGL((route_topk_row_kernel<16>), grid, block, 0, s, logits, topk_ids, topk_weights, T,
                               (int)E, (int)k, (int)(norm_topk_prob != 0));
        return check_launch("moe_route (top-k)");
    }
    hipLaunchKernelGGL(route_topk_kernel, dim3((unsigned)blocks), dim3(kTopkWaves * kWave), 0, s, logits, topk_ids,
                       topk_weights, T, (int)E, (int)k, (int)(norm_topk_prob != 0));
    return check_launch("moe_route (top-k)");
}

// Checks of the (x, w_router, ..., k) arguments shared by both entry points.
static int check_route_args(const char* fn, const void* x, const void* w_router, const float* logits,
                            const int32_t* topk_ids, const float* topk_weights, int64_t T, int32_t H, int32_t E,
                            int32_t k) {
    if (x == nullptr) {
        // logits are an input; H is not used
        if (T < 0 || E < 0 || k < 0) return set_error(MOE_ERR_INVALID, "%s: negative size", fn);
        if (E < 1 || E > kMaxExperts) return set_error(MOE_ERR_UNSUPPORTED, "%s: E=%d outside [1, 256]", fn, E);
        if (k < 1 || k > E || k > kMaxTopK) return set_error(MOE_ERR_UNSUPPORTED, "%s: k=%d invalid", fn, k);
        if (T * (int64_t)k >= ((int64_t)1 << 31)) return set_error(MOE_ERR_UNSUPPORTED, "%s: T*k too large", fn);
    } else {
        int rc = check_shape(fn, T, H, E, k, -1);
        if (rc) return rc;
        if (!w_router) return set_error(MOE_ERR_INVALID, "%s: w_router is NULL", fn);
    }
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_weights)
        return set_error(MOE_ERR_INVALID, "%s: logits/topk_ids/topk_weights must not be NULL", fn);
    if (x && (((uintptr_t)x | (uintptr_t)w_router) & 15))
        return set_error(MOE_ERR_INVALID, "%s: x and w_router must be 16-byte aligned", fn);
    return MOE_OK;
}

}  // namespace moe

extern "C" int moe_route(const void* x, const void* w_router, const float* router_bias, float* logits,
                         int32_t* topk_ids, float* topk_weights, int64_t T, int32_t H, int32_t E, int32_t k,
                         int32_t norm_topk_prob, void* stream) {
    using namespace moe;
    clear_error();
    int rc = check_route_args("moe_route", x, w_router, logits, topk_ids, topk_weights, T, H, E, k);
    if (rc || T == 0) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (x) {
        rc = route_logits<false>(x, w_router, router_bias, logits, T, H, E, NormArgs{}, s);
        if (rc) return rc;
    }
    return route_topk(logits, topk_ids, topk_weights, T, E, k, norm_topk_prob, s);
}

extern "C" int moe_fused_add_rmsnorm_route(const void* x, const void* residual, const void* norm_weight, float eps,
                                           int32_t has_residual, void* x_out, void* residual_out,
                                           const void* w_router, const float* router_bias, float* logits,
                                           int32_t* topk_ids, float* topk_weights, int64_t T, int32_t H, int32_t E,
                                           int32_t k, int32_t norm_topk_prob, void* stream) {
    using namespace moe;
    clear_error();
    const char* fn = "moe_fused_add_rmsnorm_route";
    if (!x) return set_error(MOE_ERR_INVALID, "%s: x is NULL", fn);
    int rc = check_route_args(fn, x, w_router, logits, topk_ids, topk_weights, T, H, E, k);
    if (rc) return rc;
    if (H > 16384) return set_error(MOE_ERR_UNSUPPORTED, "%s: H=%d above 16384", fn, H);
    if (!(eps >= 0.f)) return set_error(MOE_ERR_INVALID, "%s: eps must be >= 0", fn);
    if (T == 0) return MOE_OK;
    if (!norm_weight || !x_out || !residual_out || (has_residual && !residual))
        return set_error(MOE_ERR_INVALID, "%s: required pointer is NULL", fn);
    if (((uintptr_t)norm_weight | (uintptr_t)x_out | (uintptr_t)residual_out |
         (uintptr_t)(has_residual ? residual : nullptr)) & 15)
        return set_error(MOE_ERR_INVALID, "%s: pointers must be 16-byte aligned", fn);
    // every router workgroup of a token block reads the block's rows while
    // the first expert tile writes the outputs: they must be other memory
    const char* in_lo[2] = {(const char*)x, (const char*)(has_residual ? residual : x)};
    const char* out_lo[2] = {(const char*)x_out, (const char*)residual_out};
    const size_t bytes = (size_t)T * H * 2;
    for (const char* o : out_lo)
        for (const char* i : in_lo)
            if (o < i + bytes && i < o + bytes)
                return set_error(MOE_ERR_INVALID, "%s: x_out and residual_out must not overlap x or residual", fn);
    if (out_lo[0] < out_lo[1] + bytes && out_lo[1] < out_lo[0] + bytes)
        return set_error(MOE_ERR_INVALID, "%s: x_out and residual_out must not overlap", fn);
    hipStream_t s = (hipStream_t)stream;
    const NormArgs na{(const uint16_t*)residual, (const uint16_t*)norm_weight, (uint16_t*)x_out,
                      (uint16_t*)residual_out, eps, has_residual ? 1 : 0};
    rc = route_logits<true>(x, w_router, router_bias, logits, T, H, E, na, s);
    if (rc) return rc;
    return route_topk(logits, topk_ids, topk_weights, T, E, k, norm_topk_prob, s);
}
