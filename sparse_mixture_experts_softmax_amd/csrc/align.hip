// moe_align_by_expert: group (token, slot) pairs by expert, each group
// padded to the GEMM row tile, stable (ascending flat index inside a group)
// and deterministic.
//
// The flat pairs are cut into tiles of 1024, 2048 or 4096 entries (the
// smallest giving at most 32 tiles, since every tile's workgroup reads all
// tiles' counts); each thread loads its (at most 16) ids of the tile at once,
// so a kernel waits for memory once. Kernel 1 counts
// each tile's pairs per expert into the workspace (LDS atomics: the counts do
// not depend on their order). Kernel 2 runs one workgroup per tile: it reads
// every tile's counts, forms the expert totals, the padded exclusive scan and
// the number of pairs of each expert in earlier tiles, then scatters its own
// tile in rounds of 256 entries. Inside a round a pair's rank among the
// earlier pairs of the same expert comes from wave ballots over the bits of
// the expert id (the same-expert lane mask) plus per-wave counts in LDS, so
// positions follow flat-index order exactly. Each workgroup also writes the
// sentinel into the pad rows and the block owners of its share of the
// capacity. When all pairs fit one tile, kernel 2 counts them itself and
// kernel 1 is skipped; up to kAlignFusedMaxPairs pairs (ids 16-byte
// aligned) every workgroup of kernel 2 counts all pairs itself, the earlier
// tiles' separately, and kernel 1 is skipped as well.
#include <mutex>

#include "abi_util.h"
#include "moe_common.h"

namespace moe {

constexpr int kAlignMaxTiles = 32;
constexpr int kAlignThreads = 256;
constexpr int kAlignWaves = kAlignThreads / kWave;

// Entry q of this thread in tile `tile` (PT entries per thread): flat index
// tile*PT*256 + q*256 + tid. All PT loads are issued before any is used;
// entries past n read entry n-1 and are marked -1.
template <int PT>
__device__ __forceinline__ void load_tile_ids(const int32_t* __restrict__ ids, int64_t n, int E, int tile,
                                              int (&e)[PT]) {
    const int64_t start = (int64_t)tile * PT * kAlignThreads + threadIdx.x;
#pragma unroll
    for (int q = 0; q < PT; ++q) {
        const int64_t i = start + q * kAlignThreads;
        e[q] = ids[min(i, n - 1)];
    }
#pragma unroll
    for (int q = 0; q < PT; ++q) {
        const int64_t i = start + q * kAlignThreads;
        if (i >= n || (unsigned)e[q] >= (unsigned)E) e[q] = -1;
    }
}

template <int PT>
__global__ __launch_bounds__(kAlignThreads) void align_hist_kernel(const int32_t* __restrict__ ids, int64_t n, int E,
                                                                   int32_t* __restrict__ ws) {
    __shared__ int cnt[kMaxExperts];
    int my[PT];
    load_tile_ids<PT>(ids, n, E, blockIdx.x, my);
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PT; ++q)
        if (my[q] >= 0) atomicAdd(&cnt[my[q]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) ws[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// Inclusive scan over the workgroup's first kMaxExperts threads (values of
// threads >= E count as 0): a shuffle scan inside each wave, then the wave
// totals. Every thread of the workgroup must call it.
__device__ int block_inclusive_scan(int v, int* wave_tot, int E) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    int x = tid < E ? v : 0;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    if (lane == kWave - 1) wave_tot[wave] = x;
    __syncthreads();
    int add = 0;
    for (int w = 0; w < wave; ++w) add += wave_tot[w];
    __syncthreads();
    return x + add;
}

template <int PT>
__global__ __launch_bounds__(kAlignThreads) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int BM, int64_t cap, int ntiles,
    const int32_t* __restrict__ ws, int fused_hist, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ counts_out, int32_t* __restrict__ num_padded) {
    __shared__ int total[kMaxExperts];    // c_e
    __shared__ int base[kMaxExperts];     // next position of this tile's pairs of expert e (relative to off)
    __shared__ int off[kMaxExperts + 1];  // padded exclusive scan; off[E] = num_padded
    __shared__ int scan_buf[kAlignWaves];
    __shared__ int wcnt[kAlignWaves][kMaxExperts];
    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave;
    const int tile = blockIdx.x;
    const int64_t start = (int64_t)tile * PT * kAlignThreads;
    int my[PT];
    load_tile_ids<PT>(ids, n, E, tile, my);

    if (fused_hist == 1) {
        // the only tile: its own pairs are all pairs
        for (int e = tid; e < kMaxExperts; e += blockDim.x) total[e] = 0;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < PT; ++q)
            if (my[q] >= 0) atomicAdd(&total[my[q]], 1);
        __syncthreads();
        if (tid < E) base[tid] = 0;
    } else if (fused_hist == 2) {
        // every workgroup counts all n pairs itself (16-byte loads, ids
        // 16-byte aligned), and separately those of the earlier tiles: no
        // histogram kernel and no workspace round trip
        for (int e = tid; e < kMaxExperts; e += blockDim.x) {
            total[e] = 0;
            base[e] = 0;
        }
        __syncthreads();
        auto count = [&](int64_t i, int e) {
            if ((unsigned)e < (unsigned)E) {
                atomicAdd(&total[e], 1);
                if (i < start) atomicAdd(&base[e], 1);
            }
        };
        const int64_t n4 = n / 4;
        constexpr int B = 16;  // 16-byte loads in flight per thread
        for (int64_t v0 = tid; v0 < n4; v0 += (int64_t)B * kAlignThreads) {
            int4 q[B];
#pragma unroll
            for (int u = 0; u < B; ++u) q[u] = ((const int4*)ids)[min(v0 + (int64_t)u * kAlignThreads, n4 - 1)];
#pragma unroll
            for (int u = 0; u < B; ++u) {
                const int64_t v = v0 + (int64_t)u * kAlignThreads;
                if (v < n4) {
                    count(4 * v, q[u].x);
                    count(4 * v + 1, q[u].y);
                    count(4 * v + 2, q[u].z);
                    count(4 * v + 3, q[u].w);
                }
            }
        }
        for (int64_t i = 4 * n4 + tid; i < n; i += kAlignThreads) count(i, ids[i]);
        __syncthreads();
    } else if (tid < E) {
        // every tile's count of expert tid, 32 loads in flight at a time
        int tot = 0, pre = 0;
        for (int t0 = 0; t0 < ntiles; t0 += kAlignMaxTiles) {
            int h[kAlignMaxTiles];
#pragma unroll
            for (int u = 0; u < kAlignMaxTiles; ++u) h[u] = ws[(int64_t)min(t0 + u, ntiles - 1) * E + tid];
#pragma unroll
            for (int u = 0; u < kAlignMaxTiles; ++u) {
                const int t = t0 + u;
                if (t < ntiles) {
                    if (t < tile) pre += h[u];
                    tot += h[u];
                }
            }
        }
        total[tid] = tot;
        base[tid] = pre;
    }
    for (int i = tid; i < kAlignWaves * kMaxExperts; i += blockDim.x) (&wcnt[0][0])[i] = 0;
    __syncthreads();

    const int padded = tid < E ? (total[tid] + BM - 1) / BM * BM : 0;
    const int incl = block_inclusive_scan(padded, scan_buf, E);
    if (tid < E) off[tid] = incl - padded;
    if (tid == E - 1) off[E] = incl;
    __syncthreads();
    const int npad = off[E];
    if (tile == 0) {
        if (tid < E) counts_out[tid] = total[tid];
        if (tid == 0) *num_padded = npad;
    }

    // Pad rows (sentinel) and block owners. Expert e's share is done by
    // workgroup e % ntiles (thread e / ntiles); rows from num_padded to cap
    // are split over all workgroups.
    for (int e = tile + (int)(tid * ntiles); e < E; e += (int)(blockDim.x * ntiles)) {
        const int o = off[e], c = total[e], p = off[e + 1] - o;
        for (int r = o + c; r < o + p; ++r) sorted_ids[r] = (int32_t)n;
        for (int b = o / BM; b < (o + p) / BM; ++b) block_expert[b] = e;
    }
    {
        const int64_t rest = cap - npad;
        const int64_t per = (rest + ntiles - 1) / ntiles;
        const int64_t lo = npad + (int64_t)tile * per, hi = min(cap, lo + per);
        for (int64_t r = lo + tid; r < hi; r += blockDim.x) {
            sorted_ids[r] = (int32_t)n;
            if (r % BM == 0) block_expert[r / BM] = -1;
        }
    }

    // Stable scatter of this tile's pairs, 256 per round; rounds that start
    // past the last pair (a short single tile) are skipped by the whole
    // workgroup.
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int q = 0; q < PT; ++q) {
        if (start + q * kAlignThreads >= n) break;
        const int64_t i = start + q * kAlignThreads + tid;
        const int e = my[q];
        const bool valid = e >= 0;
        unsigned long long same = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const unsigned long long m = __ballot(valid && ((e >> b) & 1));
            same &= ((e >> b) & 1) ? m : ~m;
        }
        const int rank = __popcll(same & below);
        if (valid && rank == 0) wcnt[wave][e] = __popcll(same);
        __syncthreads();
        if (valid) {
            int pos = off[e] + base[e] + rank;
            for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
            sorted_ids[pos] = (int32_t)i;
        }
        __syncthreads();
        if (tid < E) {
            int s = 0;
#pragma unroll
            for (int w = 0; w < kAlignWaves; ++w) {
                s += wcnt[w][tid];
                wcnt[w][tid] = 0;
            }
            base[tid] += s;
        }
        __syncthreads();
    }
}

// Entries per thread (tile = 256 * that): 4, 8 or 16, the smallest giving at
// most kAlignMaxTiles tiles.
static int align_per_thread(int64_t T, int32_t k) {
    const int64_t n = T * k;
    for (int pt = 4; pt < 16; pt *= 2)
        if ((n + pt * kAlignThreads - 1) / (pt * kAlignThreads) <= kAlignMaxTiles) return pt;
    return 16;
}
static int64_t align_ntiles(int64_t T, int32_t k) {
    const int64_t ts = (int64_t)align_per_thread(T, k) * kAlignThreads;
    return (T * k + ts - 1) / ts;
}

// Up to this many pairs (and with 16-byte aligned ids) every workgroup of
// the scatter kernel counts all pairs itself instead of reading the
// histogram kernel's per-tile counts: one launch and no workspace round
// trip. Grouping step (events) at 4096 pairs: 14.4 -> 11.5 us; at 32768
// pairs each of the 32 workgroups reading all ids made it slower (17.3 ->
// 20.9 us), so larger groupings keep the histogram kernel.
constexpr int64_t kAlignFusedMaxPairs = 8192;

template <int PT>
static void launch_align(const int32_t* ids, int64_t n, int E, int BM, int64_t cap, int64_t ntiles, int32_t* ws,
                         int32_t* sorted_ids, int32_t* block_expert, int32_t* counts, int32_t* num_padded,
                         hipStream_t s) {
    const int fused = ntiles <= 1 ? 1 : (n <= kAlignFusedMaxPairs && ((uintptr_t)ids & 15) == 0) ? 2 : 0;
    if (!fused)
        hipLaunchKernelGGL(align_hist_kernel<PT>, dim3((unsigned)ntiles), dim3(kAlignThreads), 0, s, ids, n, E, ws);
    hipLaunchKernelGGL(align_scatter_kernel<PT>, dim3((unsigned)ntiles), dim3(kAlignThreads), 0, s, ids, n, E, BM, cap,
                       (int)ntiles, (const int32_t*)ws, fused, sorted_ids, block_expert, counts, num_padded);
}

// Workspace of moe_align_by_expert_noalloc: the per-tile histograms live in
// this file-scope device array instead of a caller buffer (each device holds
// its own copy for the life of the process). Host code must not pass the
// array's name to a kernel (on the host it is only a stand-in symbol): its
// device address comes from hipGetSymbolAddress, taken once per device.
constexpr int64_t kAlignScratchInts = MOE_ALIGN_NOALLOC_MAX_WORKSPACE_BYTES / sizeof(int32_t);  // ntiles * E counts
static __device__ __align__(256) int32_t scratch[kAlignScratchInts];

constexpr int kMaxDevices = 64;
static std::atomic<int32_t*> g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up once per
// device; nullptr (with the error set) on failure.
static int32_t* scratch_on_current_device(const char* fn) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) {
        set_error(MOE_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(err));
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        set_error(MOE_ERR_UNSUPPORTED, "%s: device %d beyond the %d this library tracks", fn, dev, kMaxDevices);
        return nullptr;
    }
    int32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p) return p;
    err = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || p == nullptr) {
        set_error(MOE_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(err));
        return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace moe

extern "C" int64_t moe_align_capacity(int64_t T, int32_t k, int32_t E, int32_t block_m) {
    if (T < 0 || k < 1 || E < 1 || !moe::valid_block_m(block_m)) return -1;
    const int64_t n = T * k;
    const int64_t c = n + (n < E ? n : E) * (int64_t)(block_m - 1);
    return (c + block_m - 1) / block_m * block_m;
}

extern "C" size_t moe_align_workspace_bytes(int64_t T, int32_t k, int32_t E, int32_t block_m) {
    if (T < 0 || k < 1 || E < 1 || !moe::valid_block_m(block_m)) return 0;
    const int64_t ntiles = moe::align_ntiles(T, k);
    return ntiles <= 1 ? 0 : (size_t)ntiles * (size_t)E * sizeof(int32_t);
}

namespace moe {

// Checks shared by both align entry points; MOE_OK with T > 0 means launch.
static int check_align_args(const char* fn, const int32_t* topk_ids, int64_t T, int32_t k, int32_t E,
                            int32_t block_m, const int32_t* sorted_ids, const int32_t* block_expert,
                            const int32_t* expert_counts, const int32_t* num_padded) {
    if (T < 0 || k < 0 || E < 0) return set_error(MOE_ERR_INVALID, "%s: negative size", fn);
    if (E < 1 || E > kMaxExperts) return set_error(MOE_ERR_UNSUPPORTED, "%s: E=%d outside [1, 256]", fn, E);
    if (k < 1 || k > E || k > kMaxTopK) return set_error(MOE_ERR_UNSUPPORTED, "%s: k=%d invalid", fn, k);
    if (!valid_block_m(block_m))
        return set_error(MOE_ERR_UNSUPPORTED, "%s: block_m=%d not in {16,32,64,128,256}", fn, block_m);
    if (T * (int64_t)k >= ((int64_t)1 << 31)) return set_error(MOE_ERR_UNSUPPORTED, "%s: T*k too large", fn);
    if (T == 0) return MOE_OK;
    if (!topk_ids || !sorted_ids || !block_expert || !expert_counts || !num_padded)
        return set_error(MOE_ERR_INVALID, "%s: required pointer is NULL", fn);
    return MOE_OK;
}

static int run_align(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t block_m, int32_t* sorted_ids,
                     int32_t* block_expert, int32_t* expert_counts, int32_t* num_padded, int32_t* ws,
                     hipStream_t s, const char* fn) {
    const int64_t ntiles = align_ntiles(T, k);
    const int64_t cap = moe_align_capacity(T, k, E, block_m);
    const int64_t n = T * k;
    switch (align_per_thread(T, k)) {
        case 4:
            launch_align<4>(topk_ids, n, E, block_m, cap, ntiles, ws, sorted_ids, block_expert, expert_counts,
                            num_padded, s);
            break;
        case 8:
            launch_align<8>(topk_ids, n, E, block_m, cap, ntiles, ws, sorted_ids, block_expert, expert_counts,
                            num_padded, s);
            break;
        default:
            launch_align<16>(topk_ids, n, E, block_m, cap, ntiles, ws, sorted_ids, block_expert, expert_counts,
                             num_padded, s);
    }
    return check_launch(fn);
}

}  // namespace moe

extern "C" int moe_align_by_expert(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t block_m,
                                   int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_counts,
                                   int32_t* num_padded, void* workspace, size_t workspace_bytes, void* stream) {
    using namespace moe;
    clear_error();
    const char* fn = "moe_align_by_expert";
    int rc = check_align_args(fn, topk_ids, T, k, E, block_m, sorted_ids, block_expert, expert_counts, num_padded);
    if (rc || T == 0) return rc;
    const size_t need = moe_align_workspace_bytes(T, k, E, block_m);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return set_error(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                         workspace_bytes);
    return run_align(topk_ids, T, k, E, block_m, sorted_ids, block_expert, expert_counts, num_padded,
                     (int32_t*)workspace, (hipStream_t)stream, fn);
}

extern "C" int moe_align_by_expert_noalloc(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E,
                                           int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                                           int32_t* expert_counts, int32_t* num_padded, void* stream) {
    using namespace moe;
    clear_error();
    const char* fn = "moe_align_by_expert_noalloc";
    int rc = check_align_args(fn, topk_ids, T, k, E, block_m, sorted_ids, block_expert, expert_counts, num_padded);
    if (rc || T == 0) return rc;
    const size_t need = moe_align_workspace_bytes(T, k, E, block_m);
    if (need > (size_t)MOE_ALIGN_NOALLOC_MAX_WORKSPACE_BYTES)
        return set_error(MOE_ERR_UNSUPPORTED,
                         "%s: T*k=%lld pairs over E=%d experts need %zu bytes of per-tile histograms, beyond the "
                         "%d-byte static scratch; use moe_align_by_expert with a workspace",
                         fn, (long long)(T * k), E, need, MOE_ALIGN_NOALLOC_MAX_WORKSPACE_BYTES);
    int32_t* ws = nullptr;
    if (need > 0) {
        // every entry the scatter kernel reads is first written by the
        // histogram kernel of the same call, so the scratch needs no clearing
        ws = scratch_on_current_device(fn);
        if (!ws) return MOE_ERR_HIP;
    }
    return run_align(topk_ids, T, k, E, block_m, sorted_ids, block_expert, expert_counts, num_padded, ws,
                     (hipStream_t)stream, fn);
}


