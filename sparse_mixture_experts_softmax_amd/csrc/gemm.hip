// Grouped expert GEMMs on the matrix cores (bf16 operands, fp32
// accumulation), one launch for all experts.
//
//   gate/up:  act[r, c] = silu(x[t] . w13[e, c]) * (x[t] . w13[e, I + c])
//   down:     y[i, h]   = act[r] . w2[e, h]      (fp32 accumulation; y stored fp16 or fp32)
//
// with r a row of the expert-grouped permutation, i = sorted_ids[r] the flat
// (token, slot) index, t = i / k its token and e = block_expert[r / BM] the
// expert owning the row block. Activations are row-major; weights come in
// the fragment layout of moe_pack_weights (16-row bands x 32-column k-steps,
// each a contiguous 1 KB MFMA B operand; gate and up bands interleaved), so
// every weight load instruction reads 1 KB contiguous.
//
// Three kernels, chosen by the row-block size block_m:
//   16       grouped_gemm_skinny_kernel (weight streaming, decode-sized)
//   32       grouped_gemm_kernel        (16x16x32 MFMA, LDS-staged)
//   64, 128  grouped_gemm_wide_kernel   (32x32x16 MFMA, direct-to-LDS copies;
//   and 256  256-row blocks as two 128-row tiles)
// The skinny and general kernels launch one workgroup per (row block, N
// tile) of the capacity and blocks past num_padded (read on the device)
// return at once; the wide kernel launches one persistent workgroup per CU
// that walks the real tiles. Either way no host sync is needed.
//
// General kernel (row blocks of 32): each workgroup stages BMxBK
// activation rows (gathered through sorted_ids for gate/up) in padded
// row-major LDS and the tile's BN/16 weight bands (BK/32 fragments each) in
// fragment-major LDS, double-buffered: the next K tile is loaded into
// registers while the current one feeds the MFMAs. For gate/up an N tile
// holds BN/2 gate rows and the BN/2 matching up rows, so each wave owns the
// gate and up accumulators of the same output columns and applies
// silu(g) * u in registers.
#include "abi_util.h"
#include "moe_common.h"

namespace moe {

// ----------------------------------------------------------------------------
// Weighted combine fused into the down projection (moe_grouped_gemm_down_combine)
//
// A token's k expert outputs come from k different row blocks, computed by
// different workgroups on different XCDs, so the sum is taken by whichever
// workgroup finishes a token's last slot: after storing its y rows, a
// workgroup makes them visible device-wide (release fence: L2 write-back),
// then counts one arrival per (token, 128-column group) it covered on a
// device-scope counter; the workgroup whose arrival is the k-th for a
// (token, group) acquires (L2 invalidate) and forms
//   out[t, c] = sum_j topk_weights[t, j] * y[t*k + j, c],  j = 0, 1, ... in order
// for the group's columns, exactly as moe_combine does, then puts the
// counter back to zero. Which workgroup sums a group does not change its
// bits, so the result is deterministic. Column tiles start on multiples of
// 128 and cover whole groups, so every (row, group) is counted once.
struct CombineArgs {
    const float* w;      // [T, k] routing weights
    int32_t* cnt;        // [T, G] arrival counters, zero on entry and on exit
    void* out;           // [T, N_out] bf16 or fp32
    int G;               // 128-column groups: ceil(N_out / 128)
};

constexpr int kCombineGroup = 128;

// Called by every thread of the workgroup after its y stores. row_id(r) is
// the flat index of row r of the tile (or anything outside [0, n_pairs) for
// a pad row); list points to LDS for nrows * groups int64 entries plus an
// int counter.
template <bool Y16, int OUTF, int THREADS, class RowId>
__device__ __forceinline__ void combine_completed(RowId row_id, int nrows, int col0, int cols, int k, int64_t n_pairs,
                                                  int N_out, const void* __restrict__ y, const CombineArgs& ca,
                                                  int64_t* list, int* n_list, int tid) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (tid == 0) *n_list = 0;
    __syncthreads();
    const int gpt = cols / kCombineGroup;
    for (int i = tid; i < nrows * gpt; i += THREADS) {
        const int r = i / gpt, g = col0 / kCombineGroup + i % gpt;
        const int64_t id = row_id(r);
        if (id < 0 || id >= n_pairs || g * kCombineGroup >= N_out) continue;
        const int64_t e = (id / k) * ca.G + g;
        if (__hip_atomic_fetch_add(ca.cnt + e, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == k - 1)
            list[atomicAdd(n_list, 1)] = e;
    }
    __syncthreads();
    const int n = *n_list;
    if (n == 0) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // 32 threads per completed (token, group), four columns each
    for (int q = tid / 32; q < n; q += THREADS / 32) {
        const int64_t e = list[q];
        const int64_t t = e / ca.G;
        const int c = (int)(e % ca.G) * kCombineGroup + (tid % 32) * 4;
        if (c < N_out) {
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
            float v[kMaxTopK > 8 ? 8 : kMaxTopK][4];
            for (int j0 = 0; j0 < k; j0 += 8) {
                float wj[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = min(j0 + u, k - 1);
                    wj[u] = ca.w[t * k + j];
                    const int64_t idx = (t * k + j) * N_out + c;
                    if constexpr (Y16) {
                        const uint32_t* p = (const uint32_t*)((const _Float16*)y + idx);
                        const uint32_t lo = p[0], hi = p[1];
                        v[u][0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(lo & 0xffffu));
                        v[u][1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(lo >> 16));
                        v[u][2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hi & 0xffffu));
                        v[u][3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hi >> 16));
                    } else {
                        const f32x4 a = *(const f32x4*)((const float*)y + idx);
#pragma unroll
                        for (int m = 0; m < 4; ++m) v[u][m] = a[m];
                    }
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const bool use = j0 + u < k;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const float sum = acc[m] + wj[u] * v[u][m];
                        acc[m] = use ? sum : acc[m];
                    }
                }
            }
            if constexpr (OUTF == 2) {
                *(f32x4*)((float*)ca.out + t * N_out + c) = f32x4{acc[0], acc[1], acc[2], acc[3]};
            } else {
                uint32_t* o = (uint32_t*)((uint16_t*)ca.out + t * N_out + c);
                o[0] = pack_bf16x2(acc[0], acc[1]);
                o[1] = pack_bf16x2(acc[2], acc[3]);
            }
        }
        if (tid % 32 == 0) ca.cnt[e] = 0;
    }
}

template <int BM_, int BN_, bool GATED_>
struct GemmCfg {
    static constexpr int BM = BM_;
    static constexpr int BN = BN_;
    static constexpr bool GATED = GATED_;
    static constexpr int BK = 64;
    static constexpr int THREADS = 256;
    static constexpr int WAVES = THREADS / kWave;
    static constexpr int WAVES_M = BM >= 32 ? 2 : 1;
    static constexpr int WAVES_N = WAVES / WAVES_M;
    static constexpr int WTM = BM / WAVES_M;
    static constexpr int WTN = BN / WAVES_N;
    static constexpr int MT = WTM / 16;
    static constexpr int NT = WTN / 16;
    static constexpr int STRIDE = BK + 8;  // A: LDS row stride in elements (16-byte pad)
    static constexpr int KS = BK / 32;     // k-steps (fragments per band) per K tile
    static constexpr int A_CHUNKS = BM * BK / 8;
    static constexpr int B_CHUNKS = BN * BK / 8;
    static constexpr int A_PER_T = (A_CHUNKS + THREADS - 1) / THREADS;
    static constexpr int B_PER_T = (B_CHUNKS + THREADS - 1) / THREADS;
    static_assert(MT >= 1 && NT >= 1, "tile too small");
    static_assert(!GATED || NT % 2 == 0, "gated tile needs gate and up halves");
};

template <class C, bool Y16, int OUTF = 0>
__global__ __launch_bounds__(C::THREADS) void grouped_gemm_kernel(
    const uint16_t* __restrict__ a_src, const uint16_t* __restrict__ w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded, int k, int64_t n_pairs,
    int K, int N_out, int n_tiles, void* __restrict__ out, CombineArgs ca) {
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, STRIDE = C::STRIDE;
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];  // [band][k-step][512]
    __shared__ int64_t row_src[BM];  // gate/up: x row offset (-1 = zero row); down: y row (-1 = skip)

    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave;
    const int mb = blockIdx.x / n_tiles;
    const int tn = blockIdx.x % n_tiles;
    if ((int64_t)mb * BM >= (int64_t)*num_padded) return;
    const int e = block_expert[mb];
    if (e < 0) return;

    // weights: gate/up W13[e] is [2*N_out, K]; down W2[e] is [N_out, K]
    const int64_t w_rows = C::GATED ? 2 * (int64_t)N_out : (int64_t)N_out;
    const uint16_t* we = w + (int64_t)e * w_rows * K;

    for (int i = tid; i < BM; i += C::THREADS) {
        const int32_t id = sorted_ids[(int64_t)mb * BM + i];
        const bool real = id >= 0 && (int64_t)id < n_pairs;
        if (C::GATED) row_src[i] = real ? (int64_t)(id / k) * K : -1;
        else row_src[i] = real ? (int64_t)id : -1;
    }
    __syncthreads();

    // Global source of each thread's chunks (fixed across K tiles).
    const uint16_t* a_ptr[C::A_PER_T];
    bool a_ok[C::A_PER_T];
#pragma unroll
    for (int j = 0; j < C::A_PER_T; ++j) {
        const int c = tid + j * C::THREADS;
        const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
        a_ok[j] = c < C::A_CHUNKS;
        if (C::GATED) {
            const int64_t src = a_ok[j] ? row_src[row] : -1;
            a_ok[j] = a_ok[j] && src >= 0;
            a_ptr[j] = a_src + (src >= 0 ? src : 0) + kc;
        } else {
            a_ptr[j] = a_src + frag_index((int64_t)mb * BM + (a_ok[j] ? row : 0), kc, K);
        }
    }
    // B chunk c of a K tile: band-in-tile c / (KS*64), k-step (c / 64) % KS,
    // lane c % 64. Bands past the weight (ragged N) are clamped to the last
    // band: their columns are never stored.
    const int bands = (int)(w_rows / 16);
    const int ksteps = K / 32;
    const uint16_t* b_ptr[C::B_PER_T];
#pragma unroll
    for (int j = 0; j < C::B_PER_T; ++j) {
        const int c = min(tid + j * C::THREADS, C::B_CHUNKS - 1);
        const int band = min(tn * (BN / 16) + c / (C::KS * 64), bands - 1);
        b_ptr[j] = we + (int64_t)band * 16 * K + ((c / 64) % C::KS) * 512 + (c % 64) * 8;
    }

    // Unconditional loads from clamped addresses; values outside the operand
    // (sentinel rows, the K tail) are zeroed with sel(). B rows past N_out
    // are clamped to row 0: their columns are never stored. When K % 64 ==
    // 32 the second half of the last K tile lies past the operand: those
    // chunks load from k-step 0 of the same row or band instead (a_ptr and
    // b_ptr already include the chunk's k-step offset within the tile, which
    // there points past the row band or the weight), and sel() drops them.
    u32x4 ra[C::A_PER_T], rb[C::B_PER_T];
    auto load_tile = [&](int kt, auto once) {
        const int k0 = kt * BK;
#pragma unroll
        for (int j = 0; j < C::A_PER_T; ++j) {
            const int kc = ((tid + j * C::THREADS) % (BK / 8)) * 8;
            const bool in = k0 + kc < K;
            // gathered x rows: columns k0.. are k0 elements on (K = H is a
            // multiple of 64, so always in); act fragments: columns k0.. of a
            // row sit k0 / 32 blocks of 512 on, and column kc itself (kc / 32)
            // blocks on, which is undone when out of range
            const int64_t off = C::GATED ? (in ? k0 : 0) : (in ? (int64_t)k0 * 16 : -(int64_t)(kc >> 5) * 512);
            ra[j] = sel(a_ok[j] && in, ld16(a_ptr[j] + off));
        }
#pragma unroll
        for (int j = 0; j < C::B_PER_T; ++j) {
            const int ks = ((tid + j * C::THREADS) / 64) % C::KS;
            const bool in = kt * C::KS + ks < ksteps;
            const uint16_t* bq = b_ptr[j] + (in ? (int64_t)kt * C::KS * 512 : -(int64_t)ks * 512);
            u32x4 v;
            if constexpr (decltype(once)::value) v = __builtin_nontemporal_load((const u32x4*)bq);
            else v = ld16(bq);
            rb[j] = sel(in, v);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int j = 0; j < C::A_PER_T; ++j) {
            const int c = tid + j * C::THREADS;
            if (c < C::A_CHUNKS) *(u32x4*)&sA[buf][(c / (BK / 8)) * STRIDE + (c % (BK / 8)) * 8] = ra[j];
        }
#pragma unroll
        for (int j = 0; j < C::B_PER_T; ++j) {
            const int c = tid + j * C::THREADS;
            if (c < C::B_CHUNKS) *(u32x4*)&sB[buf][c * 8] = rb[j];
        }
    };

    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    f32x4 acc[C::MT][C::NT];
#pragma unroll
    for (int i = 0; i < C::MT; ++i)
#pragma unroll
        for (int j = 0; j < C::NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // band (within the N tile) that wave-tile column block j reads: gate/up
    // bands are interleaved, so gate tile g of output columns c.. is band
    // 2*(c/16) and its up tile the next band
    auto b_band = [&](int j) {
        if (C::GATED) {
            constexpr int HALF_NT = C::NT / 2;
            const int g = j % HALF_NT;
            return 2 * (wn * (C::WTN / 32) + g) + (j < HALF_NT ? 0 : 1);
        }
        return wn * (C::WTN / 16) + j;
    };

    const int nk = (K + BK - 1) / BK;
    auto run = [&](auto once) {
        load_tile(0, once);
        store_tile(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int buf = kt & 1;
            if (kt + 1 < nk) load_tile(kt + 1, once);
#pragma unroll
            for (int ks = 0; ks < BK / 32; ++ks) {
                const int kof = ks * 32 + (lane / 16) * 8;
                u32x4 fa[C::MT], fb[C::NT];
#pragma unroll
                for (int i = 0; i < C::MT; ++i)
                    fa[i] = *(const u32x4*)&sA[buf][(wm * C::WTM + i * 16 + lane % 16) * STRIDE + kof];
#pragma unroll
                for (int j = 0; j < C::NT; ++j) fb[j] = *(const u32x4*)&sB[buf][(b_band(j) * C::KS + ks) * 512 + lane * 8];
#pragma unroll
                for (int i = 0; i < C::MT; ++i)
#pragma unroll
                    for (int j = 0; j < C::NT; ++j) acc[i][j] = mfma16x16x32(fa[i], fb[j], acc[i][j]);
            }
            if (kt + 1 < nk) store_tile(buf ^ 1);
            __syncthreads();
        }
    };
    // weights read by no other row block of this launch (the expert's only
    // block) are loaded non-temporally, as in the skinny kernel
    const int n_blocks = gridDim.x / n_tiles;
    if ((mb == 0 || block_expert[mb - 1] != e) && (mb + 1 >= n_blocks || block_expert[mb + 1] != e))
        run(std::true_type{});
    else
        run(std::false_type{});

    // Epilogue. Lane holds rows 4*(lane/16)+q, column lane%16 of each 16x16 tile.
    if (C::GATED) {
        constexpr int HALF_NT = C::NT / 2;
#pragma unroll
        for (int i = 0; i < C::MT; ++i) {
#pragma unroll
            for (int g = 0; g < HALF_NT; ++g) {
                const int col = tn * (BN / 2) + wn * (C::WTN / 2) + g * 16 + lane % 16;
                if (col >= N_out) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row = wm * C::WTM + i * 16 + (lane / 16) * 4 + q;
                    const float v = silu(acc[i][g][q]) * acc[i][g + HALF_NT][q];
                    ((uint16_t*)out)[frag_index((int64_t)mb * BM + row, col, N_out)] = f32_to_bf16(v);
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < C::MT; ++i) {
#pragma unroll
            for (int j = 0; j < C::NT; ++j) {
                const int col = tn * BN + wn * C::WTN + j * 16 + lane % 16;
                if (col >= N_out) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row = wm * C::WTM + i * 16 + (lane / 16) * 4 + q;
                    const int64_t dst = row_src[row];
                    if (dst >= 0) store_y<Y16>(out, dst * N_out + col, acc[i][j][q]);
                }
            }
        }
        if constexpr (OUTF != 0) {
            // the stages are free after the k loop's last barrier
            int64_t* list = (int64_t*)&sA[0][0];
            int* n_list = (int*)&sB[0][0];
            static_assert(BM * (BN / kCombineGroup) * 8 <= (int)sizeof(sA[0]), "combine list");
            combine_completed<Y16, OUTF, C::THREADS>([&](int r) { return row_src[r]; }, BM, tn * BN, BN, k, n_pairs,
                                                     N_out, out, ca, list, n_list, tid);
        }
    }
}

// Wide variant for row blocks of 64 or 128 (tens to thousands of rows per
// expert, as in prefill): matrix-core bound, so it runs on
// v_mfma_f32_32x32x16_bf16 (half the MFMA instructions of the 16x16x32 form
// for the same work, which leaves issue slots to the copies and fragment
// reads) with 64x128 wave tiles (2x4 accumulator tiles of 32x32, 128
// accumulator registers); the workgroup covers BM rows x 512 weight rows
// with (BM/64) x 4 waves, two waves per SIMD.
//
// Operands reach LDS by direct global->LDS copies (global_load_lds_dwordx4,
// no registers), S stages deep (128-row blocks: 4 stages of 40 KB, all of
// LDS): stage kt holds
// the activation rows' columns [32kt, 32kt+32) and one packed 1 KB block per
// weight band. The A rows are stored 64 bytes apart with their four 16-byte
// chunks XOR-swizzled by (row/4)%4 so that fragment reads are free of bank
// conflicts; B blocks are stored as packed. Each copy instruction costs the
// issuing wave time, so its address is a uniform SGPR base plus a 32-bit
// lane offset. Each wave waits only for its own copies of the stage it needs
// (explicit vmcnt), then a bare s_barrier publishes the stage to all waves
// and frees the oldest one for the next copy.
//
// Tiles are ordered so each XCD (workgroups go to the 8 XCDs round robin)
// takes a contiguous share of the real (row block, N tile) pairs, row-block
// major: the row blocks of one expert run together on one XCD and share its
// L2 for the weight tile. For gate/up the weights are the MFMA's first
// operand, so each lane's accumulators hold runs of four consecutive output
// columns of one row and act is stored straight from the registers; the
// down projection's y rows go through LDS (see its epilogue).
template <bool GATED_, int BM_, int STAGES_, int WAVES_N_ = 4, int TM_ = 2, int WTN_ = 128, int MINB_ = 1>
struct WideCfg {
    static constexpr bool GATED = GATED_;
    static constexpr int MINB = MINB_;           // workgroups per CU (LDS permitting)
    static constexpr int BM = BM_;
    static constexpr int TM = TM_;               // 32-row accumulator tiles per wave
    static constexpr int WAVES_N = WAVES_N_;
    static constexpr int WAVES_M = BM / (32 * TM);
    static constexpr int THREADS = WAVES_M * WAVES_N * kWave;
    static constexpr int WTN = WTN_;             // weight rows per wave
    static constexpr int TN = WTN / 32;          // 32-column accumulator tiles per wave
    static constexpr int BN = WAVES_N * WTN;     // weight rows per workgroup
    static constexpr int COLS = GATED ? BN / 2 : BN;  // output columns per workgroup
    static constexpr int STAGES = STAGES_;
    static constexpr int A_BYTES = BM * 64;      // one stage of A: BM rows x 32 columns
    static constexpr int B_BYTES = BN * 64;      // BN/16 packed blocks of 1 KB
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int COPIES = (BM + BN) / 16;  // 1 KB copies per stage
    static constexpr int COPIES_PER_WAVE = COPIES / (WAVES_M * WAVES_N);
    static_assert(COPIES % (WAVES_M * WAVES_N) == 0, "copies must split evenly over the waves");
    static_assert(STAGES >= 2 && STAGES <= 6, "stages");
    static_assert((STAGES - 1) * COPIES_PER_WAVE < 64, "vmcnt range");
    static_assert(MINB * STAGES * STAGE_BYTES <= 160 * 1024, "LDS");
    static_assert(THREADS >= BM, "one row id per thread");
    // the down epilogue reuses the stages: 1 KB of row ids, then 32 rows of
    // the fp32 y tile at a time
    static_assert(GATED || 1024 + 32 * COLS * 4 <= STAGES * STAGE_BYTES, "epilogue staging");
};

// Quarter-width tiles of the down projection's 128-row blocks (128 output
// columns, eight waves as 4 x 2 with 32x64 wave tiles): the last, partial
// round of tiles of an XCD is handed out as four of these per tile, so it
// takes about a third of a full tile's time instead of a whole one. Same
// MFMA and the same k order per element, so the same bits.
template <int BM_>
using WideQuarterCfg = WideCfg<false, BM_, 6, 2, 1, 64>;

// One tile of the wide GEMM: the workgroup's C::BM rows of row block mb
// (expert e) against C::BN weight rows from band band0 on, written to the
// output columns from col0 on. smem holds the stages (and, after the k loop,
// the epilogue's staging); the caller synchronises before reusing it.
template <class C, bool Y16, int OUTF = 0>
__device__ __forceinline__ void wide_tile(const uint16_t* __restrict__ a_src, const uint16_t* __restrict__ w,
                                          const int32_t* __restrict__ sorted_ids, int e, int mb, int band0,
                                          int col0, int k, int64_t n_pairs, int K, int N_out,
                                          void* __restrict__ out, char* smem, int tid, int lane, int wave,
                                          const CombineArgs& ca) {
    constexpr int BM = C::BM, S = C::STAGES;
    const int64_t w_rows = C::GATED ? 2 * (int64_t)N_out : (int64_t)N_out;
    const int bands = (int)(w_rows / 16);
    const uint16_t* we = w + (int64_t)e * w_rows * K;

    const int32_t* ids_blk = sorted_ids + (int64_t)mb * BM;
    auto real_row = [&](int32_t id) { return id >= 0 && (int64_t)id < n_pairs; };
    const int32_t my_id = tid < BM ? ids_blk[tid] : 0;  // row ids for the down epilogue (C::THREADS >= BM)
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    int32_t rid[C::TM];  // gate/up: the flat (token, slot) index of this lane's row in each row block
#pragma unroll
    for (int i = 0; i < C::TM; ++i) rid[i] = ids_blk[wm * (32 * C::TM) + i * 32 + lane % 32];

    // This wave's copies: index q over [A rows 16q.. | B band q - BM/16],
    // each a uniform base (the activations or this expert's weights) plus a
    // 32-bit per-lane byte offset (operands are under 4 GiB, checked on the
    // host), so the copies use the SGPR-base form and take half the address
    // registers of 64-bit pointers.
    typedef uint32_t copy_off_t;
    const char* const base_a = (const char*)a_src;
    const char* const base_b = (const char*)we;
    copy_off_t soff[C::COPIES_PER_WAVE];
    int dst[C::COPIES_PER_WAVE];  // byte offset inside a stage (wave-uniform)
#pragma unroll
    for (int j = 0; j < C::COPIES_PER_WAVE; ++j) {
        const int q = wave * C::COPIES_PER_WAVE + j;
        if (q < BM / 16) {
            if (C::GATED) {
                // 16 gathered x rows, 64 bytes each
                const int row = q * 16 + lane / 4;
                const int chunk = (lane % 4) ^ ((row >> 2) & 3);  // LDS slot lane%4 holds this chunk
                const int32_t id = ids_blk[row];
                const int64_t base = real_row(id) ? (int64_t)(id / k) * K : 0;  // sentinel rows: any valid row
                soff[j] = (copy_off_t)((base + chunk * 8) * 2);
            } else {
                // one 1 KB act fragment block (16 rows x 32 columns)
                soff[j] = (copy_off_t)(((int64_t)(mb * (BM / 16) + q) * (K / 32) * 512 + lane * 8) * 2);
            }
            dst[j] = q * 1024;
        } else {
            const int bt = q - BM / 16;
            const int band = min(band0 + bt, bands - 1);
            soff[j] = (copy_off_t)(((int64_t)band * 16 * K + lane * 8) * 2);
            dst[j] = C::A_BYTES + bt * 1024;
        }
    }
    const int nkt = K / 32;
    auto issue = [&](int kt) {
        char* stage = smem + (kt % S) * C::STAGE_BYTES;
#pragma unroll
        for (int j = 0; j < C::COPIES_PER_WAVE; ++j) {
            const int q = wave * C::COPIES_PER_WAVE + j;
            const bool is_a = q < BM / 16;
            // gathered rows: 32 columns (64 bytes) on; fragment blocks: the next 1 KB block
            const copy_off_t step = (is_a && C::GATED) ? 64 : 1024;
            lds_dma16((is_a ? base_a : base_b) + (soff[j] + (copy_off_t)kt * step), stage + dst[j]);
        }
    };

    // B band pairs (32 weight rows) of each accumulator column tile
    int band_lo[C::TN], band_hi[C::TN];
#pragma unroll
    for (int t = 0; t < C::TN; ++t) {
        if (C::GATED) {
            const int g = t % (C::TN / 2);
            const int cb = wn * (C::WTN / 32) + g * 2;  // output column block (16 wide) within the tile
            const int up = t < C::TN / 2 ? 0 : 1;
            band_lo[t] = 2 * cb + up;
            band_hi[t] = 2 * (cb + 1) + up;
        } else {
            band_lo[t] = wn * (C::WTN / 16) + 2 * t;
            band_hi[t] = band_lo[t] + 1;
        }
    }
    f32x16 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int t = 0; t < C::TN; ++t) acc[i][t] = f32x16{};

    // One k-step: this wave's fragments of stage kt (both 16-column halves)
    // are read first, then (do_issue) the copies of stage kt+S-1 are issued,
    // then the 16 MFMAs; the compiler overlaps the second half's reads and
    // the copies with the first half's MFMAs. Every row is computed, pad rows
    // included (the epilogue drops them): branches around the MFMAs cost more
    // than skipping pad-only accumulator tiles saves.
    auto kstep = [&](int kt, auto do_issue) {
        const char* stage = smem + (kt % S) * C::STAGE_BYTES;
        u32x4 fa[2][C::TM], fb[2][C::TN];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int chunk = 2 * ks + lane / 32;
#pragma unroll
            for (int i = 0; i < C::TM; ++i) {
                const int r = wm * (32 * C::TM) + i * 32 + lane % 32;
                // gathered rows: swizzled row-major; act: fragment blocks
                const int off = C::GATED ? r * 64 + ((chunk ^ ((r >> 2) & 3)) * 16)
                                         : (r / 16) * 1024 + (chunk * 16 + r % 16) * 16;
                fa[ks][i] = *(const u32x4*)(stage + off);
            }
#pragma unroll
            for (int t = 0; t < C::TN; ++t) {
                const int band = (lane % 32) < 16 ? band_lo[t] : band_hi[t];
                fb[ks][t] = *(const u32x4*)(stage + C::A_BYTES + band * 1024 + (chunk * 16 + lane % 16) * 16);
            }
        }
        if constexpr (decltype(do_issue)::value) issue(kt + S - 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int t = 0; t < C::TN; ++t)
                    acc[i][t] = C::GATED ? mfma32x32x16(fb[ks][t], fa[ks][i], acc[i][t])
                                         : mfma32x32x16(fa[ks][i], fb[ks][t], acc[i][t]);
    };

    // Prologue: the first S-1 stages (when K has fewer k-steps, the extra
    // stages repeat the last one into buffers that are never read).
#pragma unroll
    for (int p = 0; p < S - 1; ++p) issue(min(p, nkt - 1));
    if (nkt >= S - 1) {
        // Steady state: wait for this wave's copies of stage kt (those of the
        // S-2 later stages stay in flight), publish it with a bare barrier,
        // and refill the buffer every wave finished with at the previous step.
        int kt = 0;
        for (; kt < nkt - (S - 1); ++kt) {
            vm_wait<(S - 2) * C::COPIES_PER_WAVE>();
            __builtin_amdgcn_s_barrier();
            kstep(kt, std::true_type{});
        }
        // The last S-1 stages: no more copies, so fewer remain in flight.
        static_for<0, S - 1>([&](auto j) {
            vm_wait<(S - 2 - decltype(j)::value) * C::COPIES_PER_WAVE>();
            __builtin_amdgcn_s_barrier();
            kstep(kt + decltype(j)::value, std::false_type{});
        });
    } else {
        vm_wait<0>();
        __builtin_amdgcn_s_barrier();
        for (int kt = 0; kt < nkt; ++kt) kstep(kt, std::false_type{});
    }

    if constexpr (C::GATED) {
        // Straight from the accumulators, no LDS. With the weights as the
        // MFMA's first operand, element q of accumulator tile (i, g) is
        // output column 8*(q/4) + 4*(lane/32) + q%4 of 32-column block g and
        // row lane%32 of 32-row block i: for each q/4 a lane holds four
        // consecutive columns of one row, and lanes l and l+32 together one
        // 8-column chunk. In act's fragment blocks (16 rows x 32 columns,
        // 1 KB) chunk q/4 of row R sits at chunk*16 + R%16, so each store
        // instruction writes two runs of 256 contiguous bytes.
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
            const int64_t R = (int64_t)mb * BM + wm * (32 * C::TM) + i * 32 + lane % 32;  // act row
            const bool real = real_row(rid[i]);  // pad rows are written as zeros
#pragma unroll
            for (int g = 0; g < C::TN / 2; ++g) {
                const int cb = col0 + wn * (C::WTN / 2) + g * 32;  // 32-column block (N_out % 32 == 0)
                if (cb >= N_out) continue;
                uint16_t* blk = (uint16_t*)out + ((R / 16) * (N_out / 32) + cb / 32) * 512 + (R % 16) * 8 +
                                4 * (lane / 32);
#pragma unroll
                for (int c8 = 0; c8 < 4; ++c8) {
                    float v[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int q = 4 * c8 + u;
                        v[u] = real ? silu(acc[i][g][q]) * acc[i][g + C::TN / 2][q] : 0.f;
                    }
                    const u32x2 p = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                    __builtin_nontemporal_store(p, (u32x2*)(blk + c8 * 128));
                }
            }
        }
    } else {
        // y rows are whole 1 KB (fp16) or 2 KB (fp32) runs of scattered rows,
        // so they are staged: the stages are free once every wave is done
        // with the last one, and hold the block's row ids (first 1 KB) and
        // 32 rows of the tile at a time, each row then stored 16 bytes per
        // lane (straight from the accumulators each lane would write 16-byte
        // pieces of 32 rows: 2.8x slower at prefill)
        __syncthreads();
        int32_t* ids_s = (int32_t*)smem;
        char* stile = smem + 1024;
        if (tid < BM) ids_s[tid] = my_id;
        __syncthreads();
        // 32-row passes (one accumulator tile row of the waves of one wm)
        constexpr int ES = Y16 ? 2 : 4;
        constexpr int CPR = C::COLS * ES / 16;  // 16-byte chunks per row
#pragma unroll
        for (int pass = 0; pass < BM / 32; ++pass) {
            const int pm = pass / C::TM, pi = pass % C::TM;
            if (wm == pm) {
#pragma unroll
                for (int t = 0; t < C::TN; ++t) {
                    const int col = wn * C::WTN + t * 32 + lane % 32;
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const int row = 8 * (q / 4) + 4 * (lane / 32) + q % 4;
                        const float v = acc[pi][t][q];
                        if constexpr (Y16)
                            ((_Float16*)stile)[row * C::COLS + col] = (_Float16)v;
                        else
                            ((float*)stile)[row * C::COLS + col] = v;
                    }
                }
            }
            __syncthreads();
            for (int ci = tid; ci < 32 * CPR; ci += C::THREADS) {
                const int r = ci / CPR, col = col0 + (ci % CPR) * (16 / ES);
                const int32_t id = ids_s[pass * 32 + r];
                const u32x4 v = *(const u32x4*)(stile + ci * 16);
                if (real_row(id) && col < N_out)
                    __builtin_nontemporal_store(v, (u32x4*)((char*)out + ((int64_t)id * N_out + col) * ES));
            }
            __syncthreads();
        }
        if constexpr (OUTF != 0) {
            static_assert(C::COLS % kCombineGroup == 0, "column tiles cover whole combine groups");
            static_assert(1024 + 16 + BM * (C::COLS / kCombineGroup) * 8 <= C::STAGES * C::STAGE_BYTES, "list");
            combine_completed<Y16, OUTF, C::THREADS>([&](int r) { return (int64_t)ids_s[r]; }, BM, col0, C::COLS,
                                                     k, n_pairs, N_out, out, ca, (int64_t*)(stile + 16),
                                                     (int*)stile, tid);
        }
    }
}

// The persistent grid: the gridDim.x/8 workgroups of an XCD (workgroups go
// to the 8 XCDs round robin) walk the XCD's contiguous share of the real
// (row block, N tile) tiles in steps of gridDim.x/8, so at any time they
// hold consecutive tiles (the row blocks of one expert together) and a
// workgroup's stores drain while it starts its next tile. When SPLIT and the
// last round of an XCD holds at most a quarter as many tiles as it has
// workgroups, those tiles are computed as four quarter-width tiles each
// (WideQuarterCfg), on four workgroups.
//
// AM: grouping blocks per tile row block. With block_m 256 the grouping pads
// each expert to 256 rows and every 256-row block is computed as two 128-row
// tiles (AM = 2) of the same expert, so the row block of tile mb is mb / AM.
template <class C, bool Y16, bool SPLIT, int AM = 1, int OUTF = 0>
__global__ __launch_bounds__(C::THREADS, C::MINB* C::THREADS / 256) void grouped_gemm_wide_kernel(
    const uint16_t* __restrict__ a_src, const uint16_t* __restrict__ w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded, int k, int64_t n_pairs,
    int K, int N_out, int n_tiles, void* __restrict__ out, CombineArgs ca) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: copy bases and LDS slots in SGPRs
    const int m_real = *num_padded / C::BM;
    const int64_t real = (int64_t)m_real * n_tiles;
    const int64_t share = (real + 7) / 8;
    const int xcd = blockIdx.x % 8, g = gridDim.x / 8, wg = blockIdx.x / 8;
    const int64_t t_begin = (int64_t)xcd * share;
    const int64_t n_x = max((int64_t)0, min(t_begin + share, real) - t_begin);
    constexpr int QS = SPLIT ? C::BN / WideQuarterCfg<C::BM>::BN : 1;
    const int64_t rem = n_x % g;
    const bool split = SPLIT && rem > 0 && rem * QS <= g;
    const int64_t n_full = split ? n_x - rem : n_x;
    for (int64_t l = wg; l < n_full; l += g) {
        const int64_t logical = t_begin + l;
        const int tn = (int)(logical % n_tiles), mb = (int)(logical / n_tiles);
        const int e = block_expert[mb / AM];
        if (e < 0) continue;
        wide_tile<C, Y16, OUTF>(a_src, w, sorted_ids, e, mb, tn * (C::BN / 16), tn * C::COLS, k, n_pairs, K, N_out,
                                out, smem, tid, lane, wave, ca);
        __syncthreads();  // the next tile's copies reuse the staging memory
    }
    if constexpr (SPLIT) {
        using CQ = WideQuarterCfg<C::BM>;
        static_assert(!C::GATED && CQ::THREADS == C::THREADS && CQ::BM == C::BM, "quarter tiles of the same block");
        static_assert(CQ::STAGES * CQ::STAGE_BYTES <= C::STAGES * C::STAGE_BYTES, "quarter tiles fit the stages");
        if (split && wg < rem * QS) {
            const int64_t logical = t_begin + n_full + wg / QS;
            const int sub = wg % QS;
            const int tn = (int)(logical % n_tiles), mb = (int)(logical / n_tiles);
            const int e = block_expert[mb / AM];
            if (e >= 0)
                wide_tile<CQ, Y16, OUTF>(a_src, w, sorted_ids, e, mb, tn * (C::BN / 16) + sub * (CQ::BN / 16),
                                         tn * C::COLS + sub * CQ::COLS, k, n_pairs, K, N_out, out, smem, tid, lane,
                                         wave, ca);
        }
    }
}

template <class C, bool Y16, int AM = 1, int OUTF = 0>
static int launch_wide(const void* a, const void* w, const int32_t* sorted_ids, const int32_t* block_expert,
                       const int32_t* num_padded, int k, int64_t n_pairs, int K, int N_out, int64_t cap, void* out,
                       hipStream_t s, const char* what, const CombineArgs& ca = CombineArgs{}) {
    const int n_tiles = (N_out + C::COLS - 1) / C::COLS;
    // The copies take 32-bit offsets: the activation rows they address
    // (gathered x rows, T = n_pairs / k of them, for gate/up; the act rows of
    // the capacity for down) and one expert's weights must be under 4 GiB.
    const int64_t a_bytes = (C::GATED ? n_pairs / k : cap) * (int64_t)K * 2;
    const int64_t w_bytes = (C::GATED ? 2 : 1) * (int64_t)N_out * K * 2;  // one expert's weights
    if (a_bytes >= ((int64_t)1 << 32) || w_bytes >= ((int64_t)1 << 32))
        return set_error(MOE_ERR_UNSUPPORTED,
                         "%s: block_m=%d needs the activations (%lld bytes) and one expert's weights (%lld bytes) "
                         "under 4 GiB; split the batch",
                         what, C::BM, (long long)a_bytes, (long long)w_bytes);
    // C::MINB workgroups per compute unit at most (160 KB of LDS between
    // them), a multiple of 8 so that every XCD gets the same number
    const int cus = device_cu_count(what);
    if (cus < 0) return cus;
    int64_t grid = (cap / C::BM) * n_tiles;
    grid = (grid + 7) / 8 * 8;
    grid = min(grid, (int64_t)max(8, cus / 8 * 8) * C::MINB);
    if (grid >= ((int64_t)1 << 31)) return set_error(MOE_ERR_UNSUPPORTED, "%s: grid too large", what);
    const size_t lds = (size_t)C::STAGES * C::STAGE_BYTES;
    // quarter tiles for the down projection's last round (one workgroup per CU)
    constexpr bool SPLIT = !C::GATED && C::MINB == 1;
    static std::atomic<uint64_t> lds_set{0};
    const int rc =
        ensure_dynamic_lds((const void*)grouped_gemm_wide_kernel<C, Y16, SPLIT, AM, OUTF>, (int)lds, lds_set, what);
    if (rc) return rc;
    hipLaunchKernelGGL((grouped_gemm_wide_kernel<C, Y16, SPLIT, AM, OUTF>), dim3((unsigned)grid), dim3(C::THREADS),
                       lds, s, (const uint16_t*)a, (const uint16_t*)w, sorted_ids, block_expert, num_padded, k,
                       n_pairs, K, N_out, n_tiles, out, ca);
    return check_launch(what);
}

// Skinny variant for 16-row blocks (a handful of rows per expert, as in
// decode): the work is streaming each touched expert's weights once, so the
// weights bypass LDS. Each wave owns NTILE packed 16-row bands (gate/up:
// NTILE/2 gate bands and the NTILE/2 matching up bands, i.e. 8*NTILE output
// columns; down: NTILE bands, 16*NTILE output columns) and streams them from
// HBM straight into MFMA B-fragments, 1 KB contiguous per load, U k-steps per
// stage, two stages in flight. The gathered activation rows (A-fragments) are re-read from L2
// (the activation matrix is small in this regime). When the row block is its
// expert's only one, nothing reads those weights again in this launch and
// they are loaded non-temporally (decode: gate/up 128 -> 118 us, down 72 ->
// 65 us); an expert with more row blocks shares them through the caches and
// keeps ordinary loads (non-temporal there: 13-15% slower at 20 rows per
// expert).
template <bool GATED, int NW, int NTILE, int U, bool Y16, int OUTF = 0>
__global__ __launch_bounds__(NW* kWave) void grouped_gemm_skinny_kernel(
    const uint16_t* __restrict__ a_src, const uint16_t* __restrict__ w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded, int k, int64_t n_pairs,
    int K, int N_out, int n_tiles, void* __restrict__ out, CombineArgs ca) {
    constexpr int BM = 16;
    constexpr int COLS = GATED ? 8 * NTILE : 16 * NTILE;  // output columns per wave
    static_assert(!GATED || NTILE % 2 == 0, "gate/up needs gate and up tiles in pairs");
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int mb = blockIdx.x / n_tiles;
    const int tn = blockIdx.x % n_tiles;
    if ((int64_t)mb * BM >= (int64_t)*num_padded) return;
    const int e = block_expert[mb];
    if (e < 0) return;
    const int64_t w_rows = GATED ? 2 * (int64_t)N_out : (int64_t)N_out;
    const uint16_t* we = w + (int64_t)e * w_rows * K;
    const int c0 = (tn * NW + wave) * COLS;  // first output column of this wave
    const int r16 = lane % 16, koff = (lane / 16) * 8;

    // A: row r16 of the block
    const int32_t id = sorted_ids[(int64_t)mb * BM + r16];
    const bool a_ok = id >= 0 && (int64_t)id < n_pairs;
    // gate/up: gathered x rows (a k-step is 32 columns on); down: the row
    // block's act fragments (a k-step is the next 512-element block)
    const uint16_t* ap;
    if (GATED) ap = a_src + (a_ok ? (int64_t)(id / k) * K : 0) + koff;  // sentinel -> row 0, zeroed
    else ap = a_src + (int64_t)mb * (K / 32) * 512 + lane * 8;
    constexpr int A_STEP = GATED ? 32 : 512;
    const bool a_live = GATED ? a_ok : true;

    // B: NTILE packed bands of 16 weight rows (gate/up: gate band 2c, up
    // band 2c+1 for output columns 16c..16c+15). Bands past the weight are
    // clamped to the last band: their columns are never stored.
    const int bands = (int)(w_rows / 16);
    const uint16_t* bp[NTILE];
#pragma unroll
    for (int j = 0; j < NTILE; ++j) {
        int band;
        if (GATED) band = 2 * (c0 / 16 + j % (NTILE / 2)) + (j < NTILE / 2 ? 0 : 1);
        else band = c0 / 16 + j;
        bp[j] = we + (int64_t)min(band, bands - 1) * 16 * K + lane * 8;
    }

    f32x4 acc[NTILE];
#pragma unroll
    for (int j = 0; j < NTILE; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 ra[2][U], rb[2][NTILE][U];
    // weight loads: non-temporal when this is the expert's only row block
    auto ldw = [&](const uint16_t* p, auto once) -> u32x4 {
        if constexpr (decltype(once)::value) return __builtin_nontemporal_load((const u32x4*)p);
        else return ld16(p);
    };
    // Loads are unconditional: rows outside the operand were clamped to a
    // valid row above (their columns are never stored) and sentinel A rows
    // are zeroed by sel() so pad rows of act come out as zeros.
    auto load = [&](int st, int s0, auto once) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            ra[st][u] = sel(a_live, ld16(ap + (s0 + u) * A_STEP));
#pragma unroll
            for (int j = 0; j < NTILE; ++j) rb[st][j][u] = ldw(bp[j] + (s0 + u) * 512, once);
        }
    };
    auto compute = [&](int st) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < NTILE; ++j) acc[j] = mfma16x16x32(ra[st][u], rb[st][j][u], acc[j]);
    };
    const int ksteps = K / 32;
    const int nstage = ksteps / U;  // full stages; the ksteps % U tail follows
    auto stream = [&](auto once) {
        if (nstage > 0) load(0, 0, once);
        for (int c = 0; c < nstage; c += 2) {
            if (c + 1 < nstage) load(1, (c + 1) * U, once);
            compute(0);
            if (c + 2 < nstage) load(0, (c + 2) * U, once);
            if (c + 1 < nstage) compute(1);
        }
        for (int s = nstage * U; s < ksteps; ++s) {
            const u32x4 a = sel(a_live, ld16(ap + s * A_STEP));
#pragma unroll
            for (int j = 0; j < NTILE; ++j) acc[j] = mfma16x16x32(a, ldw(bp[j] + s * 512, once), acc[j]);
        }
    };
    // the expert's only row block: its neighbours (if any) belong to other
    // experts or are past the padded rows (-1)
    const int n_blocks = gridDim.x / n_tiles;
    const bool only_block = (mb == 0 || block_expert[mb - 1] != e) && (mb + 1 >= n_blocks || block_expert[mb + 1] != e);
    if (only_block) stream(std::true_type{});
    else stream(std::false_type{});

    // Epilogue: lane holds rows 4*(lane/16)+q, column lane%16 of each tile.
    if (GATED) {
#pragma unroll
        for (int g = 0; g < NTILE / 2; ++g) {
            const int col = c0 + g * 16 + r16;
            if (col >= N_out) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = (lane / 16) * 4 + q;
                const float v = silu(acc[g][q]) * acc[g + NTILE / 2][q];
                ((uint16_t*)out)[frag_index((int64_t)mb * BM + row, col, N_out)] = f32_to_bf16(v);
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = (lane / 16) * 4 + q;
            const int32_t dst = sorted_ids[(int64_t)mb * BM + row];
            if (dst < 0 || (int64_t)dst >= n_pairs) continue;
#pragma unroll
            for (int j = 0; j < NTILE; ++j) {
                const int col = c0 + j * 16 + r16;
                if (col < N_out) store_y<Y16>(out, (int64_t)dst * N_out + col, acc[j][q]);
            }
        }
        if constexpr (OUTF != 0) {
            constexpr int WG_COLS = NW * COLS;
            static_assert(WG_COLS % kCombineGroup == 0, "column tiles cover whole combine groups");
            __shared__ int64_t list[BM * (WG_COLS / kCombineGroup)];
            __shared__ int n_list;
            const int32_t* ids = sorted_ids + (int64_t)mb * BM;
            combine_completed<Y16, OUTF, NW * kWave>([&](int r) { return (int64_t)ids[r]; }, BM, tn * WG_COLS,
                                                     WG_COLS, k, n_pairs, N_out, out, ca, list, &n_list,
                                                     (int)threadIdx.x);
        }
    }
}

template <bool GATED, int NW, int NTILE, int U, bool Y16, int OUTF>
static int launch_skinny_cfg(const void* a, const void* w, const int32_t* sorted_ids, const int32_t* block_expert,
                             const int32_t* num_padded, int k, int64_t n_pairs, int K, int N_out, int64_t cap,
                             void* out, hipStream_t s, const char* what, const CombineArgs& ca) {
    const int cols_per_wg = NW * (GATED ? 8 * NTILE : 16 * NTILE);
    const int n_tiles = (N_out + cols_per_wg - 1) / cols_per_wg;
    const int64_t grid = (cap / 16) * n_tiles;
    if (grid >= ((int64_t)1 << 31)) return set_error(MOE_ERR_UNSUPPORTED, "%s: grid too large", what);
    hipLaunchKernelGGL((grouped_gemm_skinny_kernel<GATED, NW, NTILE, U, Y16, OUTF>), dim3((unsigned)grid),
                       dim3(NW * kWave), 0, s, (const uint16_t*)a, (const uint16_t*)w, sorted_ids, block_expert,
                       num_padded, k, n_pairs, K, N_out, n_tiles, out, ca);
    return check_launch(what);
}

template <bool GATED, bool Y16, int OUTF>
static int launch_skinny(const void* a, const void* w, const int32_t* sorted_ids, const int32_t* block_expert,
                         const int32_t* num_padded, int k, int64_t n_pairs, int K, int N_out, int64_t cap, void* out,
                         hipStream_t s, const char* what, const CombineArgs& ca) {
    // Chosen by sweeps on the decode-shaped layer: single-wave workgroups
    // (finest load balance) for gate/up; the down shape is insensitive.
    if (GATED)
        return launch_skinny_cfg<true, 1, 2, 8, false, 0>(a, w, sorted_ids, block_expert, num_padded, k, n_pairs, K,
                                                          N_out, cap, out, s, what, ca);
    return launch_skinny_cfg<false, 4, 4, 4, Y16, OUTF>(a, w, sorted_ids, block_expert, num_padded, k, n_pairs, K,
                                                        N_out, cap, out, s, what, ca);
}

template <class C, bool Y16, int OUTF>
static int launch_gemm(const void* a, const void* w, const int32_t* sorted_ids, const int32_t* block_expert,
                       const int32_t* num_padded, int k, int64_t n_pairs, int K, int N_out, int64_t cap, void* out,
                       hipStream_t s, const char* what, const CombineArgs& ca) {
    const int n_cols = C::GATED ? C::BN / 2 : C::BN;
    const int n_tiles = (N_out + n_cols - 1) / n_cols;
    const int64_t m_blocks = cap / C::BM;
    const int64_t grid = m_blocks * n_tiles;
    if (grid >= ((int64_t)1 << 31)) return set_error(MOE_ERR_UNSUPPORTED, "%s: grid too large", what);
    hipLaunchKernelGGL((grouped_gemm_kernel<C, Y16, OUTF>), dim3((unsigned)grid), dim3(C::THREADS), 0, s,
                       (const uint16_t*)a, (const uint16_t*)w, sorted_ids, block_expert, num_padded, k, n_pairs, K,
                       N_out, n_tiles, out, ca);
    return check_launch(what);
}

// OUTF: 0 = plain projection (y only); 1 / 2 = the weighted combine fused in,
// out bf16 / fp32 (down projection only).
template <bool GATED, bool Y16, int OUTF = 0>
static int dispatch_gemm(int32_t block_m, const void* a, const void* w, const int32_t* sorted_ids,
                         const int32_t* block_expert, const int32_t* num_padded, int k, int64_t n_pairs, int K,
                         int N_out, int64_t cap, void* out, hipStream_t s, const char* what,
                         const CombineArgs& ca = CombineArgs{}) {
    switch (block_m) {
        case 16:
            return launch_skinny<GATED, Y16, OUTF>(a, w, sorted_ids, block_expert, num_padded, k, n_pairs, K, N_out,
                                                   cap, out, s, what, ca);
        case 32:
            return launch_gemm<GemmCfg<32, 128, GATED>, Y16, OUTF>(a, w, sorted_ids, block_expert, num_padded, k,
                                                                   n_pairs, K, N_out, cap, out, s, what, ca);
        case 64:
            // 64x256 tiles, four waves of 32x128, four 20 KB stages, two
            // workgroups per CU: at 32 rows per expert (weight streaming)
            // gate/up -9% and down -7% against 64x512 tiles with one
            // workgroup per CU (same-process probe, outputs identical)
            return launch_wide<WideCfg<GATED, 64, 4, 2, 1, 128, 2>, Y16, 1, OUTF>(
                a, w, sorted_ids, block_expert, num_padded, k, n_pairs, K, N_out, cap, out, s, what, ca);
        case 128:
            // 4 stages for both projections (down: -1 to -2.5% against 3 in
            // same-box A/B runs on prefill, skewed and large); 3 stages for
            // gate/up were 6% faster at prefill but need 32 bytes/lane of
            // scratch, which this library does not allow
            return launch_wide<WideCfg<GATED, 128, 4>, Y16, 1, OUTF>(a, w, sorted_ids, block_expert, num_padded, k,
                                                                     n_pairs, K, N_out, cap, out, s, what, ca);
        case 256:  // two 128-row tiles per grouping block: the same bits as block_m 128 for every row
            return launch_wide<WideCfg<GATED, 128, 4>, Y16, 2, OUTF>(a, w, sorted_ids, block_expert, num_padded, k,
                                                                     n_pairs, K, N_out, cap, out, s, what, ca);
    }
    return set_error(MOE_ERR_UNSUPPORTED, "%s: block_m=%d not in {16,32,64,128,256}", what, block_m);
}

static int check_gemm_args(const char* fn, const void* a, const void* w, const int32_t* sorted_ids,
                           const int32_t* block_expert, const int32_t* num_padded, int64_t T, int32_t k, int32_t H,
                           int32_t I, int32_t E, int32_t block_m, int64_t cap, const void* out) {
    int rc = check_shape(fn, T, H, E, k, I);
    if (rc) return rc;
    if (!valid_block_m(block_m))
        return set_error(MOE_ERR_UNSUPPORTED, "%s: block_m=%d not in {16,32,64,128,256}", fn, block_m);
    if (T == 0) return MOE_OK;
    if (!a || !w || !sorted_ids || !block_expert || !num_padded || !out)
        return set_error(MOE_ERR_INVALID, "%s: required pointer is NULL", fn);
    if (((uintptr_t)a | (uintptr_t)w | (uintptr_t)out) & 15)
        return set_error(MOE_ERR_INVALID, "%s: activation, weight and output pointers must be 16-byte aligned", fn);
    const int64_t need = moe_align_capacity(T, k, E, block_m);
    if (cap < need)
        return set_error(MOE_ERR_WORKSPACE, "%s: cap=%lld below moe_align_capacity=%lld", fn, (long long)cap,
                         (long long)need);
    if (cap % block_m) return set_error(MOE_ERR_INVALID, "%s: cap must be a multiple of block_m", fn);
    return MOE_OK;
}

}  // namespace moe

extern "C" int moe_grouped_gemm_gate_up_silu(const void* x, const void* w13, const int32_t* sorted_ids,
                                             const int32_t* block_expert, const int32_t* num_padded, int64_t T,
                                             int32_t k, int32_t H, int32_t I, int32_t E, int32_t block_m, int64_t cap,
                                             void* act, void* stream) {
    using namespace moe;
    clear_error();
    const char* fn = "moe_grouped_gemm_gate_up_silu";
    int rc = check_gemm_args(fn, x, w13, sorted_ids, block_expert, num_padded, T, k, H, I, E, block_m, cap, act);
    if (rc || T == 0) return rc;
    return dispatch_gemm<true, false>(block_m, x, w13, sorted_ids, block_expert, num_padded, k, T * k, H, I, cap,
                                      act, (hipStream_t)stream, fn);
}

extern "C" int moe_grouped_gemm_down(const void* act, const void* w2, const int32_t* sorted_ids,
                                     const int32_t* block_expert, const int32_t* num_padded, int64_t T, int32_t k,
                                     int32_t H, int32_t I, int32_t E, int32_t block_m, int64_t cap, void* y,
                                     int32_t y_dtype, void* stream) {
    using namespace moe;
    clear_error();
    const char* fn = "moe_grouped_gemm_down";
    if (y_dtype != MOE_DTYPE_FP16 && y_dtype != MOE_DTYPE_FP32)
        return set_error(MOE_ERR_INVALID, "%s: y_dtype=%d is neither fp16 (2) nor fp32 (1)", fn, y_dtype);
    int rc = check_gemm_args(fn, act, w2, sorted_ids, block_expert, num_padded, T, k, H, I, E, block_m, cap, y);
    if (rc || T == 0) return rc;
    if (y_dtype == MOE_DTYPE_FP16)
        return dispatch_gemm<false, true>(block_m, act, w2, sorted_ids, block_expert, num_padded, k, T * k, I, H, cap,
                                          y, (hipStream_t)stream, fn);
    return dispatch_gemm<false, false>(block_m, act, w2, sorted_ids, block_expert, num_padded, k, T * k, I, H, cap, y,
                                       (hipStream_t)stream, fn);
}

extern "C" int64_t moe_combine_counter_count(int64_t T, int32_t H) {
    if (T < 0 || H <= 0) return -1;
    return T * ((H + moe::kCombineGroup - 1) / moe::kCombineGroup);
}

extern "C" int moe_grouped_gemm_down_combine(const void* act, const void* w2, const int32_t* sorted_ids,
                                             const int32_t* block_expert, const int32_t* num_padded,
                                             const float* topk_weights, int64_t T, int32_t k, int32_t H, int32_t I,
                                             int32_t E, int32_t block_m, int64_t cap, void* y, int32_t y_dtype,
                                             int32_t* counters, void* out, int32_t out_dtype, void* stream) {
    using namespace moe;
    clear_error();
    const char* fn = "moe_grouped_gemm_down_combine";
    if (y_dtype != MOE_DTYPE_FP16 && y_dtype != MOE_DTYPE_FP32)
        return set_error(MOE_ERR_INVALID, "%s: y_dtype=%d is neither fp16 (2) nor fp32 (1)", fn, y_dtype);
    if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_FP32)
        return set_error(MOE_ERR_INVALID, "%s: out_dtype=%d is neither bf16 (0) nor fp32 (1)", fn, out_dtype);
    int rc = check_gemm_args(fn, act, w2, sorted_ids, block_expert, num_padded, T, k, H, I, E, block_m, cap, y);
    if (rc || T == 0) return rc;
    if (!topk_weights || !counters || !out) return set_error(MOE_ERR_INVALID, "%s: required pointer is NULL", fn);
    if ((uintptr_t)out & 15) return set_error(MOE_ERR_INVALID, "%s: out must be 16-byte aligned", fn);
    const CombineArgs ca{topk_weights, counters, out, (H + kCombineGroup - 1) / kCombineGroup};
    hipStream_t s = (hipStream_t)stream;
    const bool y16 = y_dtype == MOE_DTYPE_FP16, o32 = out_dtype == MOE_OUT_FP32;
    if (y16 && o32)
        return dispatch_gemm<false, true, 2>(block_m, act, w2, sorted_ids, block_expert, num_padded, k, T * k, I, H, cap,
                                             y, s, fn, ca);
    if (y16)
        return dispatch_gemm<false, true, 1>(block_m, act, w2, sorted_ids, block_expert, num_padded, k, T * k, I, H, cap,
                                             y, s, fn, ca);
    if (o32)
        return dispatch_gemm<false, false, 2>(block_m, act, w2, sorted_ids, block_expert, num_padded, k, T * k, I, H,
                                              cap, y, s, fn, ca);
    return dispatch_gemm<false, false, 1>(block_m, act, w2, sorted_ids, block_expert, num_padded, k, T * k, I, H, cap,
                                          y, s, fn, ca);
}

extern "C" int32_t moe_pick_block_m(int64_t T, int32_t k, int32_t E) {
    if (T < 0 || k < 1 || E < 1) return -1;
    // Crossovers of the whole layer's step time between block sizes, measured
    // at the Qwen3-30B-A3B shape (H 2048, I 768, E 128, k 8) with near-uniform
    // routing, T from 64 to 4096 (rows per expert = T * k / E on average):
    // 16 (weight streaming, skinny kernel) below 16 rows per expert (239 vs
    // 242 us at 15; at 16 the busier experts need a second 16-row block: 248
    // vs 242); 64 (64x256 tiles, two workgroups per CU) up to 60 (284 vs 285
    // at 60, 278 vs 286 at 56; at 64 rows: 298 vs 287), where it streams each
    // expert's weights once for its one or two blocks and beats the 32-row
    // kernel at every size (257 vs 248 us at 20 rows, 349 vs 251 at 32); 128
    // above.
    const double rows_per_expert = (double)T * k / E;
    if (rows_per_expert < 16) return 16;
    if (rows_per_expert <= 60) return 64;
    return 128;
}
