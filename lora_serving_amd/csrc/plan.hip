// Stable counting sort of small integer keys on the GPU (the token-mapping plan).
//
// "Multi-LoRA Serving Explained" (sevydevy.com) sorts the batch's tokens by slot before the
// shrink and expand kernels, so that one adapter's tokens form one group; its six-token script
// does it with a stable argsort.  Here keys are slot ids (or tile ids, for the prefill path's
// tile plan), -1 entries are dropped, and ties keep their input order.  Exactly one output is
// correct, so the result is bit-exact.
//
// Small maps (up to 8192 entries, up to 1000 keys): one launch, sort_wave (one wave, up to 512
// entries) or sort_small (below).  Otherwise three launches:
//   sort_count   one wave per unit of SORT_UNIT consecutive entries: per-key counts (LDS)
//   sort_scan    one workgroup: exclusive scan of the counts in key-major order, which gives
//                every (key, unit) its first output position; then the segment table
//   sort_scatter one wave per unit: walks its entries in order, 64 at a time, ranks equal keys
//                inside the wave with one ballot per key bit, and writes each entry's index
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace mlora {

__global__ __launch_bounds__(64) void sort_count(const int32_t *__restrict__ keys, int64_t n,
                                                 int32_t nkeys, int32_t *__restrict__ cnt,
                                                 int32_t nu)
{
    extern __shared__ int32_t hist[];
    const int lane = threadIdx.x;
    const int u = blockIdx.x;
    for (int k = lane; k < nkeys; k += 64)
        hist[k] = 0;
    __syncthreads();
    const int64_t p0 = (int64_t)u * SORT_UNIT;
    const int64_t p1 = min(p0 + (int64_t)SORT_UNIT, n);
    for (int64_t p = p0 + lane; p < p1; p += 64) {
        const int32_t k = keys[p];
        if (k >= 0)
            atomicAdd(&hist[k], 1);
    }
    __syncthreads();
    for (int k = lane; k < nkeys; k += 64)
        cnt[(int64_t)k * nu + u] = hist[k];
}

// Exclusive scan across a 1024-thread block.
__device__ int block_exclusive_scan(int v, int *total, int *wsum)
{
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    int wtot;
    const int ex = wave_exclusive_scan(v, &wtot);
    if (lane == 0)
        wsum[w] = wtot;
    __syncthreads();
    int base = 0, all = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
        const int s = wsum[i];
        if (i < w)
            base += s;
        all += s;
    }
    __syncthreads();
    *total = all;
    return base + ex;
}

__global__ __launch_bounds__(1024) void sort_scan(int32_t *__restrict__ cnt, int64_t len,
                                                  int32_t nkeys, int32_t nu,
                                                  int32_t *__restrict__ seg_key,
                                                  int32_t *__restrict__ seg_start,
                                                  int32_t *__restrict__ seg_len,
                                                  int32_t *__restrict__ counts)
{
    __shared__ int wsum[16];
    int carry = 0;
    for (int64_t base = 0; base < len; base += blockDim.x) {
        const int64_t i = base + threadIdx.x;
        const int v = i < len ? cnt[i] : 0;
        int tot;
        const int ex = block_exclusive_scan(v, &tot, wsum);
        if (i < len)
            cnt[i] = carry + ex;
        carry += tot;
    }
    const int total = carry;
    __syncthreads();
    int g = 0;
    for (int base = 0; base < nkeys; base += blockDim.x) {
        const int k = base + threadIdx.x;
        int start = 0, n = 0;
        if (k < nkeys && nu > 0) {
            start = cnt[(int64_t)k * nu];
            const int end = (k + 1 < nkeys) ? cnt[(int64_t)(k + 1) * nu] : total;
            n = end - start;
        }
        const int flag = n > 0;
        int tot;
        const int ex = block_exclusive_scan(flag, &tot, wsum);
        if (flag) {
            seg_key[g + ex] = k;
            seg_start[g + ex] = start;
            seg_len[g + ex] = n;
        }
        g += tot;
    }
    if (threadIdx.x == 0) {
        counts[0] = g;
        counts[1] = total;
    }
}

__global__ __launch_bounds__(64) void sort_scatter(const int32_t *__restrict__ keys, int64_t n,
                                                   int32_t nkeys, int32_t nbits,
                                                   const int32_t *__restrict__ off, int32_t nu,
                                                   int32_t *__restrict__ perm)
{
    extern __shared__ int32_t running[];
    const int lane = threadIdx.x;
    const int u = blockIdx.x;
    for (int k = lane; k < nkeys; k += 64)
        running[k] = 0;
    __syncthreads();
    const int64_t p0 = (int64_t)u * SORT_UNIT;
    const int64_t p1 = min(p0 + (int64_t)SORT_UNIT, n);
    const uint64_t below = (1ull << lane) - 1ull;
    for (int64_t w = p0; w < p1; w += 64) {
        const int64_t p = w + lane;
        const int32_t k = p < p1 ? keys[p] : -1;
        const bool part = k >= 0;
        const uint64_t same = match_key((uint32_t)(k + 1), nbits) & ballot64(part);
        const int rank = __popcll(same & below);
        if (part)
            perm[off[(int64_t)k * nu + u] + running[k] + rank] = (int32_t)p;
        __syncthreads();
        if (part && rank == 0)
            running[k] += __popcll(same);
        __syncthreads();
    }
}

// One-workgroup form for small index maps (n <= SORT_SMALL_MAX_N, nkeys <= SORT_SMALL_MAX_KEYS),
// one launch instead of three: wave w owns the contiguous range [w U, (w + 1) U) of the entries
// (U a multiple of 64), its keys held in registers.  The per-(key, wave) counts sit in LDS (each
// wave adds one ballot-matched group of equal keys at a time to its own column); their
// exclusive scan in key-major, wave-minor order gives every (key, wave) its first output
// position, which is the stable order because the waves' ranges follow each other.  Each wave
// then walks its range 64 entries at a time, ranking equal keys with ballots, and advances its
// own positions (a column of the table no other wave touches).
constexpr int SORT_SMALL_WAVES = 16;
constexpr int SORT_SMALL_PER_LANE = 8;    // beyond 8 steps per wave the three kernels are faster
constexpr int64_t SORT_SMALL_MAX_N = (int64_t)SORT_SMALL_WAVES * 64 * SORT_SMALL_PER_LANE;
constexpr int SORT_SMALL_MAX_KEYS = 1000;   // the table fits the 64 KB of static LDS

__global__ __launch_bounds__(1024) void sort_small(const int32_t *__restrict__ keys, int32_t n,
                                                   int32_t nkeys, int32_t nbits,
                                                   int32_t *__restrict__ perm,
                                                   int32_t *__restrict__ seg_key,
                                                   int32_t *__restrict__ seg_start,
                                                   int32_t *__restrict__ seg_len,
                                                   int32_t *__restrict__ counts)
{
    __shared__ int32_t tab[SORT_SMALL_MAX_KEYS * SORT_SMALL_WAVES];   // [key][wave]
    __shared__ int wsum[16];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int len = nkeys * SORT_SMALL_WAVES;
    for (int i = threadIdx.x; i < len; i += blockDim.x)
        tab[i] = 0;
    const int U = ((n + 1023) >> 10) * 64;          // entries per wave, a multiple of 64
    const int p0 = w * U;
    int kk[SORT_SMALL_PER_LANE];
#pragma unroll
    for (int i = 0; i < SORT_SMALL_PER_LANE; ++i) {
        const int p = p0 + i * 64 + lane;
        kk[i] = (i * 64 < U && p < n) ? keys[p] : -1;
    }
    __syncthreads();
    // counts: the first lane of each group of equal keys adds the group's size (runs of one
    // key, as in prefill batches, would otherwise make 64 atomics on one address per step)
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < SORT_SMALL_PER_LANE; ++i) {
        if (i * 64 >= U)
            break;                                   // the same for every wave
        const int k = kk[i];
        const uint64_t same = match_key((uint32_t)(k + 1), nbits) & ballot64(k >= 0);
        if (k >= 0 && __popcll(same & below) == 0)
            tab[k * SORT_SMALL_WAVES + w] += __popcll(same);
    }
    __syncthreads();

    int carry = 0;
    for (int base = 0; base < len; base += blockDim.x) {
        const int i = base + threadIdx.x;
        const int v = i < len ? tab[i] : 0;
        int tot;
        const int ex = block_exclusive_scan(v, &tot, wsum);
        if (i < len)
            tab[i] = carry + ex;
        carry += tot;
    }
    const int total = carry;
    __syncthreads();
    int g = 0;
    for (int base = 0; base < nkeys; base += blockDim.x) {
        const int k = base + threadIdx.x;
        int start = 0, cnt = 0;
        if (k < nkeys) {
            start = tab[k * SORT_SMALL_WAVES];
            const int end = k + 1 < nkeys ? tab[(k + 1) * SORT_SMALL_WAVES] : total;
            cnt = end - start;
        }
        const int flag = cnt > 0;
        int tot;
        const int ex = block_exclusive_scan(flag, &tot, wsum);
        if (flag) {
            seg_key[g + ex] = k;
            seg_start[g + ex] = start;
            seg_len[g + ex] = cnt;
        }
        g += tot;
    }
    if (threadIdx.x == 0) {
        counts[0] = g;
        counts[1] = total;
    }

#pragma unroll
    for (int i = 0; i < SORT_SMALL_PER_LANE; ++i) {
        if (i * 64 >= U)
            break;
        const int k = kk[i];
        const bool part = k >= 0;
        const uint64_t same = match_key((uint32_t)(k + 1), nbits) & ballot64(part);
        const int rank = __popcll(same & below);
        if (part) {
            const int at = tab[k * SORT_SMALL_WAVES + w];
            perm[at + rank] = p0 + i * 64 + lane;
            if (rank == 0)
                tab[k * SORT_SMALL_WAVES + w] = at + __popcll(same);
        }
    }
}

// One-wave form for the smallest maps (n <= SORT_WAVE_MAX_N): a single wave holds every entry
// in registers (up to 8 a lane) and the per-key table in LDS, so no step needs a barrier (one
// wave's LDS operations complete in order).  Counts: the first lane of each ballot-matched group
// of equal keys adds the group's size; the exclusive scan over the keys, 64 at a time, gives
// each key its first output position and, compacted with a ballot, the segment table; then the
// entries are placed in input order, equal keys ranked by lane.  Same output as the kernels
// above, with a sixteenth of the waves and none of their barriers.
constexpr int SORT_WAVE_MAX_N = 64 * SORT_SMALL_PER_LANE;

__global__ __launch_bounds__(64) void sort_wave(const int32_t *__restrict__ keys, int32_t n,
                                                int32_t nkeys, int32_t nbits,
                                                int32_t *__restrict__ perm,
                                                int32_t *__restrict__ seg_key,
                                                int32_t *__restrict__ seg_start,
                                                int32_t *__restrict__ seg_len,
                                                int32_t *__restrict__ counts)
{
    __shared__ int32_t tab[SORT_SMALL_MAX_KEYS];
    const int lane = threadIdx.x;
    const int steps = (n + 63) >> 6;
    int kk[SORT_SMALL_PER_LANE];
#pragma unroll
    for (int i = 0; i < SORT_SMALL_PER_LANE; ++i) {
        const int p = i * 64 + lane;
        kk[i] = p < n ? keys[p] : -1;
    }
    for (int k = lane; k < nkeys; k += 64)
        tab[k] = 0;
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < SORT_SMALL_PER_LANE; ++i) {
        if (i >= steps)
            break;
        const int k = kk[i];
        const uint64_t same = match_key((uint32_t)(k + 1), nbits) & ballot64(k >= 0);
        if (k >= 0 && __popcll(same & below) == 0)
            tab[k] += __popcll(same);
    }
    int carry = 0, g = 0;
    for (int k0 = 0; k0 < nkeys; k0 += 64) {
        const int k = k0 + lane;
        const int c = k < nkeys ? tab[k] : 0;
        int tot;
        const int start = carry + wave_exclusive_scan(c, &tot);
        const uint64_t used = ballot64(c > 0);
        if (c > 0) {
            const int at = g + __popcll(used & below);
            seg_key[at] = k;
            seg_start[at] = start;
            seg_len[at] = c;
        }
        if (k < nkeys)
            tab[k] = start;
        carry += tot;
        g += __popcll(used);
    }
    if (lane == 0) {
        counts[0] = g;
        counts[1] = carry;
    }
#pragma unroll
    for (int i = 0; i < SORT_SMALL_PER_LANE; ++i) {
        if (i >= steps)
            break;
        const int k = kk[i];
        const bool part = k >= 0;
        const uint64_t same = match_key((uint32_t)(k + 1), nbits) & ballot64(part);
        const int rank = __popcll(same & below);
        if (part) {
            const int at = tab[k];
            perm[at + rank] = i * 64 + lane;
            if (rank == 0)
                tab[k] = at + __popcll(same);
        }
    }
}

static int key_bits(int32_t nkeys)
{
    int b = 0;
    while ((1ll << b) < (int64_t)nkeys + 1)
        ++b;
    return b;
}

size_t sort_workspace_bytes(int64_t n, int32_t nkeys)
{
    const int64_t nu = (n + SORT_UNIT - 1) / SORT_UNIT;
    return (size_t)(nu * (int64_t)nkeys) * sizeof(int32_t);
}

hipError_t launch_stable_sort(const int32_t *keys, int64_t n, int32_t nkeys, int32_t *perm,
                              int32_t *seg_key, int32_t *seg_start, int32_t *seg_len,
                              int32_t *counts, int32_t *cnt_ws, hipStream_t stream)
{
    if (n <= SORT_WAVE_MAX_N && nkeys <= SORT_SMALL_MAX_KEYS) {
        hipLaunchKernelGGL(sort_wave, dim3(1), dim3(64), 0, stream, keys, (int32_t)n, nkeys,
                           key_bits(nkeys), perm, seg_key, seg_start, seg_len, counts);
        return hipGetLastError();
    }
    if (n <= SORT_SMALL_MAX_N && nkeys <= SORT_SMALL_MAX_KEYS) {
        hipLaunchKernelGGL(sort_small, dim3(1), dim3(1024), 0, stream, keys, (int32_t)n, nkeys,
                           key_bits(nkeys), perm, seg_key, seg_start, seg_len, counts);
        return hipGetLastError();
    }
    const int64_t nu64 = (n + SORT_UNIT - 1) / SORT_UNIT;
    const int32_t nu = (int32_t)nu64;
    const size_t lds = (size_t)nkeys * sizeof(int32_t);
    if (nu > 0)
        hipLaunchKernelGGL(sort_count, dim3(nu), dim3(64), lds, stream, keys, n, nkeys, cnt_ws,
                           nu);
    hipLaunchKernelGGL(sort_scan, dim3(1), dim3(1024), 0, stream, cnt_ws, nu64 * nkeys, nkeys, nu,
                       seg_key, seg_start, seg_len, counts);
    if (nu > 0)
        hipLaunchKernelGGL(sort_scatter, dim3(nu), dim3(64), lds, stream, keys, n, nkeys,
                           key_bits(nkeys), cnt_ws, nu, perm);
    return hipGetLastError();
}

}  // namespace mlora
