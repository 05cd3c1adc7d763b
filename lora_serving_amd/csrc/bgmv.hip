// BGMV ("batched gather matrix-vector") shrink and expand: every (token, slot) pair fetches its
// own adapter's rows by slot index.
//
// Sources: "Multi-LoRA Serving Explained" (sevydevy.com), six-token batching example, gather
// variant (the slot id of a token selects the matrices it is multiplied with; -1 selects
// none); vLLM learning book, chapter "04. LoRA Serving", section 6 (the shrink to a rank-wide
// scaled intermediate and the expand that adds it back through B); "[RFC]: Per-request
// activation of multiple LoRA adapters with static scales", Proposed Change, step 4 (a token's
// K slots handled in one kernel pass, as both kernels here do).
//
// shrink: one workgroup (4 waves) per (pair, block of RB rows of the pair's n_slices * R rows),
//   RB = 16, 8, 4, 2 or 1 so that small batches still spread over many workgroups.  Lanes
//   walk n_in in 16-byte chunks (A rows read fully coalesced), two chunks of loads issued
//   before any is used, keep the RB rows' partial dot products in registers, fold them with a
//   wave "transpose reduction" (every lane ends with one row's sum) and then across the 4
//   waves through LDS in a fixed order (deterministic).
// expand: one workgroup per (token, block of output rows).  Lanes walk the contiguous
//   B[a][rows][0..R) block 16 bytes at a time, so each lane holds 8 rank entries of one row;
//   the R/8 lanes of a row finish the dot product with xor shuffles over the rank dimension.
//   Slot widths up to 32 have a kernel of their own with the row width fixed at compile time.
// These kernels are bound by latency at decode sizes: a launch and one round trip to HBM that
// waits for a slot id are most of their time, and every instruction on a wave's path counts,
// so everything that does not depend on a slot id is loaded before it is read, masked loads
// read a static zero block instead of branching, and the index arithmetic stays 32-bit where
// the grid allows.
#include "common.h"
#include "kernels.h"

namespace mlora {

__device__ __forceinline__ float dot8_bf16(const u32x4 a, const float xf[8])
{
    float s = 0.f;
    s += bf16_lo(a.x) * xf[0];
    s += bf16_hi(a.x) * xf[1];
    s += bf16_lo(a.y) * xf[2];
    s += bf16_hi(a.y) * xf[3];
    s += bf16_lo(a.z) * xf[4];
    s += bf16_hi(a.z) * xf[5];
    s += bf16_lo(a.w) * xf[6];
    s += bf16_hi(a.w) * xf[7];
    return s;
}

// RB per-lane values -> every lane ends with the wave-wide sum of value number row_of(lane):
// log2(RB) halving rounds (xor 32, 16, ...: a lane keeps the half its lane bit selects and adds
// its partner's), then plain xor sums over the remaining lane bits.  row_of(lane) is read off
// the lane bits 5, 4, ... used by the halving rounds.
template <int RB>
__device__ __forceinline__ float transpose_reduce(float (&acc)[RB])
{
    const int lane = lane_id();
#pragma unroll
    for (int half = RB / 2, bit = 5; half >= 1; half >>= 1, --bit) {
        const bool hi = (lane >> bit) & 1;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float keep = hi ? acc[half + i] : acc[i];
            const float send = hi ? acc[i] : acc[half + i];
            acc[i] = keep + __shfl_xor(send, 1 << bit, 64);
        }
    }
    float r1 = acc[0];
#pragma unroll
    for (int bit = 5 - __builtin_ctz(RB); bit >= 0; --bit)
        r1 += __shfl_xor(r1, 1 << bit, 64);
    return r1;
}

template <int RB>
__device__ __forceinline__ int transpose_row(int lane)
{
    int row = 0;
#pragma unroll
    for (int l = 0; (1 << l) < RB; ++l)
        row = row * 2 + ((lane >> (5 - l)) & 1);
    return row;
}

// Masked loads read this static block instead: the choice is made on the address, so a load
// is always issued and no branch or select waits for anything when it is.
__device__ __attribute__((aligned(16))) float vzero[4];   // never written: zeros

// Workgroup = (pair p = (token blockIdx.x, slot blockIdx.z), rows r0 .. r0 + RB - 1 of the
// pair's n_slices * R rows of v, r0 = RB blockIdx.y).  The loads that do not depend on the slot id (x, the pair's scale)
// are issued before it is read, the adapter's factor right after it, so the chain of dependent
// round trips is the slot id, the rank (only with a rank table) and the A rows.
template <int RB>
__global__ __launch_bounds__(256) void shrink_rows_kernel(const uint16_t *__restrict__ x,
                                                          int64_t T, int64_t n_in, SlotGeom g,
                                                          const int32_t *__restrict__ idx,
                                                          int32_t K,
                                                          const float *__restrict__ scale,
                                                          float *__restrict__ v, int pieces)
{
    __shared__ float red[4 * RB];
    const u32x4 *zero = (const u32x4 *)vzero;
    const int wd = g.n_slices * g.R;
    const int64_t t = blockIdx.x;
    const int j = blockIdx.z;
    const int64_t p = t * K + j;
    const int r0 = (int)blockIdx.y * RB;
    const int nr = min(RB, wd - r0);
    // v [K][T][wd] (scaled), or the decode finish's shrink pieces of one split: per 64-token
    // chunk c a block [K][Tc][wd] (Tc its tokens), blocks K 64 wd apart, unscaled
    const int64_t tc = t >> 6, tl = t & 63, Tc = min((int64_t)64, T - (tc << 6));
    float *out = pieces ? v + (tc * K * 64 + (int64_t)j * Tc + tl) * wd + r0
                        : v + ((int64_t)j * T + t) * wd + r0;
    const uint16_t *xt = x + t * n_in;
    const int64_t step = (int64_t)blockDim.x * 8;
    const int64_t kt = (int64_t)threadIdx.x * 8;
    u32x4 xv0[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        xv0[h] = *(kt + h * step < n_in ? (const u32x4 *)(xt + kt + h * step) : zero);
    const float sc = scale ? scale[p] : 1.f;
    const int a = idx[p];
    const float fa = a >= 0 ? g.factor[a] : 0.f;
    // rows of this block below the adapter's rank (rounded to 8); the others are zero padding,
    // neither read nor multiplied (R is a power of two)
    const int r8 = a >= 0 ? slot_rank8(g.rank, a, g.R) : 0;
    uint32_t live = 0;
#pragma unroll
    for (int r = 0; r < RB; ++r)
        live |= (r < nr && ((r0 + r) & (g.R - 1)) < r8 ? 1u : 0u) << r;
    if (live == 0) {
        if ((int)threadIdx.x < nr)
            out[threadIdx.x] = 0.f;
        return;
    }
    const uint16_t *Aa = g.A + ((int64_t)a * wd + r0) * n_in;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;

    float acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
        acc[r] = 0.f;
    // one round: two 16-byte chunks per lane, the live rows' A chunks all in flight, then the
    // products in chunk order
    auto round = [&](int64_t k0, const u32x4 (&xv)[2]) {
        u32x4 av[2][RB];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t k = k0 + h * step;
#pragma unroll
            for (int r = 0; r < RB; ++r)
                av[h][r] = *(k < n_in && (live >> r & 1u)
                                 ? (const u32x4 *)(Aa + (int64_t)r * n_in + k)
                                 : zero);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float xf[8] = {bf16_lo(xv[h].x), bf16_hi(xv[h].x), bf16_lo(xv[h].y),
                                 bf16_hi(xv[h].y), bf16_lo(xv[h].z), bf16_hi(xv[h].z),
                                 bf16_lo(xv[h].w), bf16_hi(xv[h].w)};
#pragma unroll
            for (int r = 0; r < RB; ++r)
                acc[r] += dot8_bf16(av[h][r], xf);
        }
    };
    round(kt, xv0);
    for (int64_t k0 = kt + 2 * step; k0 < n_in; k0 += 2 * step) {
        u32x4 xv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            xv[h] = *(k0 + h * step < n_in ? (const u32x4 *)(xt + k0 + h * step) : zero);
        round(k0, xv);
    }
    const float s = transpose_reduce<RB>(acc);
    if ((lane & (64 / RB - 1)) == 0)
        red[wave * RB + transpose_row<RB>(lane)] = s;
    __syncthreads();
    if ((int)threadIdx.x < nr) {
        const int rr = threadIdx.x;
        const float tot = ((red[rr] + red[RB + rr]) + red[2 * RB + rr]) + red[3 * RB + rr];
        out[rr] = pieces ? tot : (sc * fa) * tot;
    }
}

hipError_t launch_shrink_pairs(const uint16_t *x, int64_t T, int64_t n_in, const SlotGeom &g,
                               const int32_t *idx, int32_t K, const float *scale, float *v,
                               hipStream_t stream, bool pieces)
{
    const int64_t P = T * K;
    if (P == 0)
        return hipSuccess;
    if (T >= 2147483647LL)                 // tokens along the grid's x dimension
        return hipErrorInvalidValue;
    const int wd = g.n_slices * g.R;
    // rows per workgroup: the most (16, 8, 4, 2, 1) that still gives SHRINK_MIN_WG workgroups,
    // so small batches spread over many more workgroups than the chip has CUs
    constexpr int64_t SHRINK_MIN_WG = 2048;
    int RB = 16;
    while (RB > 1 && P * ((wd + RB - 1) / RB) < SHRINK_MIN_WG)
        RB >>= 1;
    const dim3 grid((unsigned)T, (unsigned)((wd + RB - 1) / RB), (unsigned)K);
    switch (RB) {
    case 16:
        hipLaunchKernelGGL(shrink_rows_kernel<16>, grid, dim3(256), 0, stream, x, T, n_in, g,
                           idx, K, scale, v, pieces ? 1 : 0);
        break;
    case 8:
        hipLaunchKernelGGL(shrink_rows_kernel<8>, grid, dim3(256), 0, stream, x, T, n_in, g, idx,
                           K, scale, v, pieces ? 1 : 0);
        break;
    case 4:
        hipLaunchKernelGGL(shrink_rows_kernel<4>, grid, dim3(256), 0, stream, x, T, n_in, g, idx,
                           K, scale, v, pieces ? 1 : 0);
        break;
    case 2:
        hipLaunchKernelGGL(shrink_rows_kernel<2>, grid, dim3(256), 0, stream, x, T, n_in, g, idx,
                           K, scale, v, pieces ? 1 : 0);
        break;
    default:
        hipLaunchKernelGGL(shrink_rows_kernel<1>, grid, dim3(256), 0, stream, x, T, n_in, g, idx,
                           K, scale, v, pieces ? 1 : 0);
        break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// output rows per workgroup: 1024 (256 threads x 4), or 256 when that leaves too few
// workgroups for the chip (small batches)
constexpr int EXPAND_MIN_WG = 1024;
constexpr int EXPAND_GROUP = 8;     // 16-byte B loads a thread keeps in flight

__device__ __forceinline__ int slice_of(const SlotGeom &g, int64_t n)
{
    int s = 0;
    while (s + 1 < g.n_slices && n >= g.slice_start[s + 1])
        ++s;
    return s;
}

// One workgroup per (token t = blockIdx.x, block of ER output rows from ER blockIdx.y):
//   delta[n] = sum_j sum_rho B[a_j][n][rho] v[j][t][slice(n)*R+rho],  y[t][n] = bf16(y + delta)
// Rows of a token whose slots are all -1 are left untouched.  The loads that do not depend on
// the slot ids (this thread's rows of y, v of the token's first slot, the ids themselves) are
// issued first, so the only dependent round trip before the products is the B rows (and the
// rank, with a rank table and R above 32).
template <int ER>
__global__ __launch_bounds__(256) void expand_tokens_kernel(const float *__restrict__ v,
                                                            int64_t T, int64_t n_out, SlotGeom g,
                                                            const int32_t *__restrict__ idx,
                                                            int32_t K, uint16_t *__restrict__ y)
{
    __shared__ float delta[ER];
    __shared__ float vs[MLORA_MAX_SLICES_DEV * MLORA_MAX_RANK_DEV];
    const int64_t t = blockIdx.x;
    const int64_t n0 = (int64_t)blockIdx.y * ER;
    const int nrows = (int)min((int64_t)ER, n_out - n0);
    const int R = g.R;
    const int wd = g.n_slices * R;
    const int lane = threadIdx.x & 63;
    const int r4 = threadIdx.x * 4;       // first of this thread's 4 output rows
    const bool vec = ((n_out & 3) == 0) && r4 + 3 < nrows;

    // lane j of every wave holds slot j's id
    const int my = lane < K ? idx[t * K + lane] : -1;
    u32x2 yv = {0u, 0u};
    if (vec)
        yv = *(const u32x2 *)(y + t * n_out + n0 + r4);
    // slot 0's v, 4 entries a thread (wd is a multiple of 8; up to 2048 entries)
    constexpr int VPRE = MLORA_MAX_SLICES_DEV * MLORA_MAX_RANK_DEV / 1024;
    f32x4 vpre[VPRE];
#pragma unroll
    for (int q = 0; q < VPRE; ++q)
        vpre[q] = *(const f32x4 *)(r4 + q * 1024 < wd ? v + t * wd + r4 + q * 1024 : vzero);
    if (__ballot(my >= 0) == 0)
        return;   // no adapter: the rows are left untouched (the same test in every wave)

    // the first slot with an adapter stores its row sums, later ones add theirs (a row's sum
    // is always written by the same thread)
    bool first = true;
    const int64_t step = (int64_t)blockDim.x * 8;
    for (int j = 0; j < K; ++j) {
        const int a = __builtin_amdgcn_readlane(my, j);
        if (a < 0)
            continue;
        // this adapter's columns: the smallest power of two at or above its rank (rounded to
        // 8), never above R; the columns past it are zero padding and are not read.  Up to
        // R = 32 a row is at most 64 bytes, inside one cache line that is fetched whole either
        // way: all R columns are walked then, and the rank's load stays off the B loads' path
        const int r8 = R <= 32 ? R : slot_rank8(g.rank, a, R);
        int lw = 3;                                     // log2 of the columns walked per row
        while ((1 << lw) < r8)
            ++lw;
        const int RW = 1 << lw;
        const int G = RW >> 3;                          // lanes per output row
        const int total = nrows << lw;                  // elements of the block walked
        const uint16_t *Bb = g.B + ((int64_t)a * n_out + n0) * R;
        for (int e0 = 0; e0 < total; e0 += (int)step * EXPAND_GROUP) {
            // B loads of this group first, then (first group only) v of this slot into LDS
            u32x4 bv[EXPAND_GROUP];
#pragma unroll
            for (int u = 0; u < EXPAND_GROUP; ++u) {
                const int e = e0 + u * (int)step + (int)threadIdx.x * 8;
                const int row = e >> lw;
                bv[u] = e < total ? *(const u32x4 *)(Bb + (int64_t)row * R + (e & (RW - 1)))
                                  : u32x4{0u, 0u, 0u, 0u};
            }
            if (e0 == 0) {
                if (!first)
                    lds_barrier();                      // the previous slot's reads are done
#pragma unroll
                for (int q = 0; q < VPRE; ++q) {
                    const int c = r4 + q * 1024;
                    if (c < wd)
                        *(f32x4 *)(vs + c) =
                            j == 0 ? vpre[q] : *(const f32x4 *)(v + ((int64_t)j * T + t) * wd + c);
                }
                lds_barrier();
            }
#pragma unroll
            for (int u = 0; u < EXPAND_GROUP; ++u) {
                const int e = e0 + u * (int)step + (int)threadIdx.x * 8;
                float ps = 0.f;
                int row = 0;
                if (e < total) {
                    row = e >> lw;
                    const int rho0 = e & (RW - 1);
                    const float *vv = vs + slice_of(g, n0 + row) * R + rho0;
                    ps += bf16_lo(bv[u].x) * vv[0];
                    ps += bf16_hi(bv[u].x) * vv[1];
                    ps += bf16_lo(bv[u].y) * vv[2];
                    ps += bf16_hi(bv[u].y) * vv[3];
                    ps += bf16_lo(bv[u].z) * vv[4];
                    ps += bf16_hi(bv[u].z) * vv[5];
                    ps += bf16_lo(bv[u].w) * vv[6];
                    ps += bf16_hi(bv[u].w) * vv[7];
                }
                for (int off = 1; off < G; off <<= 1)
                    ps += __shfl_xor(ps, off, 64);
                if (e < total && (lane & (G - 1)) == 0)
                    delta[row] = first ? ps : delta[row] + ps;
            }
        }
        first = false;
    }
    lds_barrier();

    if (r4 < nrows) {
        uint16_t *yo = y + t * n_out + n0 + r4;
        if (vec) {
            const uint32_t lo = pack_bf16x2(bf16_lo(yv.x) + delta[r4], bf16_hi(yv.x) + delta[r4 + 1]);
            const uint32_t hi =
                pack_bf16x2(bf16_lo(yv.y) + delta[r4 + 2], bf16_hi(yv.y) + delta[r4 + 3]);
            *(u32x2 *)yo = u32x2{lo, hi};
        } else {
            for (int q = 0; q < 4 && r4 + q < nrows; ++q)
                yo[q] = f32_to_bf16(bf16_to_f32(yo[q]) + delta[r4 + q]);
        }
    }
}

// Slot width R = RC in {8, 16, 32}: every row of B is at most 64 bytes, one cache line read
// whole either way, so the rank table is not consulted and the row width is known at compile
// time.  One workgroup per (token t = blockIdx.x, 256 output rows from 256 blockIdx.y); lane
// pieces of 8 columns as in the kernel above (RC / 8 lanes per row, RC / 8 pieces a thread),
// the v rows of all K slots staged in LDS at once, the row sums kept in registers across the
// slots, then gathered in LDS so that each thread rounds 4 consecutive rows.  The only
// dependent round trip before the products is the B rows.
template <int RC>
__global__ __launch_bounds__(256) void expand_narrow_kernel(const float *__restrict__ v,
                                                            int64_t T, int n_out, SlotGeom g,
                                                            const int32_t *__restrict__ idx,
                                                            int32_t K, uint16_t *__restrict__ y)
{
    constexpr int U = RC / 8;             // 16-byte pieces a thread (and lanes a row)
    __shared__ float vs[MLORA_MAX_K_DEV * MLORA_MAX_SLICES_DEV * RC];
    __shared__ float delta[256];
    const u32x4 *zero = (const u32x4 *)vzero;
    const int64_t t = blockIdx.x;
    const int n0 = (int)blockIdx.y * 256;
    const int nrows = min(256, n_out - n0);
    const int wd = g.n_slices * RC;
    const int lane = threadIdx.x & 63;
    const int r4 = threadIdx.x * 4;
    uint16_t *yt = y + t * n_out + n0;
    const bool vec = ((n_out & 3) == 0) && r4 + 3 < nrows;

    // independent loads first: the slot ids (lane j of every wave holds slot j's), v of every
    // slot (wave w loads slots w and w + 4, 4 entries a lane; wd <= 128), this thread's rows
    // of y
    const int my = lane < K ? idx[t * K + lane] : -1;
    const int wave = threadIdx.x >> 6;
    const int l4 = lane * 4;
    const bool vl0 = wave < K && l4 < wd, vl1 = wave + 4 < K && l4 < wd;
    const float *vrow = v + ((int64_t)wave * T + t) * wd + l4;
    const f32x4 vq0 = *(const f32x4 *)(vl0 ? vrow : vzero);
    const f32x4 vq1 = *(const f32x4 *)(vl1 ? vrow + 4 * T * wd : vzero);
    u32x2 yv = {0u, 0u};
    if (vec)
        yv = *(const u32x2 *)(yt + r4);
    if (vl0)
        *(f32x4 *)(vs + wave * wd + l4) = vq0;
    if (vl1)
        *(f32x4 *)(vs + (wave + 4) * wd + l4) = vq1;
    if (__ballot(my >= 0) == 0)
        return;   // no adapter: the rows are left untouched (the same test in every wave)
    lds_barrier();

    // piece u of this thread: element e = 2048 u + 8 threadIdx.x of the block's [256][RC]
    // B rows (row e / RC, columns e % RC .. + 8)
    const int total = nrows * RC;
    const int rho0 = ((int)threadIdx.x * 8) % RC;
    int sg[U] = {};
    if (g.n_slices > 1) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int n = n0 + (u * 2048 + (int)threadIdx.x * 8) / RC;
            sg[u] = (n >= g.slice_start[1]) + (n >= g.slice_start[2]) + (n >= g.slice_start[3]);
        }
    }
    float acc[U] = {};
    bool first = true;
    for (int j = 0; j < K; ++j) {
        const int a = __builtin_amdgcn_readlane(my, j);
        if (a < 0)
            continue;
        const uint16_t *Bb = g.B + ((int64_t)a * n_out + n0) * RC;
        u32x4 bv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = u * 2048 + (int)threadIdx.x * 8;
            bv[u] = *(e < total ? (const u32x4 *)(Bb + e) : zero);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float *vv = vs + j * wd + sg[u] * RC + rho0;
            float ps = 0.f;
            ps += bf16_lo(bv[u].x) * vv[0];
            ps += bf16_hi(bv[u].x) * vv[1];
            ps += bf16_lo(bv[u].y) * vv[2];
            ps += bf16_hi(bv[u].y) * vv[3];
            ps += bf16_lo(bv[u].z) * vv[4];
            ps += bf16_hi(bv[u].z) * vv[5];
            ps += bf16_lo(bv[u].w) * vv[6];
            ps += bf16_hi(bv[u].w) * vv[7];
#pragma unroll
            for (int off = 1; off < U; off <<= 1)
                ps += __shfl_xor(ps, off, 64);
            acc[u] = first ? ps : acc[u] + ps;
        }
        first = false;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int e = u * 2048 + (int)threadIdx.x * 8;
        if (e < total && (lane & (U - 1)) == 0)
            delta[e / RC] = acc[u];
    }
    lds_barrier();

    if (vec) {
        const uint32_t lo = pack_bf16x2(bf16_lo(yv.x) + delta[r4], bf16_hi(yv.x) + delta[r4 + 1]);
        const uint32_t hi = pack_bf16x2(bf16_lo(yv.y) + delta[r4 + 2], bf16_hi(yv.y) + delta[r4 + 3]);
        *(u32x2 *)(yt + r4) = u32x2{lo, hi};
    } else {
        for (int q = 0; q < 4 && r4 + q < nrows; ++q)
            yt[r4 + q] = f32_to_bf16(bf16_to_f32(yt[r4 + q]) + delta[r4 + q]);
    }
}

hipError_t launch_expand_tokens(const float *v, int64_t T, int64_t n_out, const SlotGeom &g,
                                const int32_t *idx, int32_t K, uint16_t *y, hipStream_t stream)
{
    if (T == 0 || n_out == 0)
        return hipSuccess;
    // grid: tokens along x (up to 2^31 - 1), row blocks along y (up to 65535)
    const int64_t nblk1k = (n_out + 1023) / 1024, nblk256 = (n_out + 255) / 256;
    if (T >= 2147483647LL || nblk256 > 65535)
        return hipErrorInvalidValue;
    if (g.R <= 32) {
        const dim3 grid((unsigned)T, (unsigned)nblk256);
        if (g.R == 8)
            hipLaunchKernelGGL(expand_narrow_kernel<8>, grid, dim3(256), 0, stream, v, T,
                               (int)n_out, g, idx, K, y);
        else if (g.R == 16)
            hipLaunchKernelGGL(expand_narrow_kernel<16>, grid, dim3(256), 0, stream, v, T,
                               (int)n_out, g, idx, K, y);
        else
            hipLaunchKernelGGL(expand_narrow_kernel<32>, grid, dim3(256), 0, stream, v, T,
                               (int)n_out, g, idx, K, y);
    } else if (T * nblk1k >= EXPAND_MIN_WG)
        hipLaunchKernelGGL(expand_tokens_kernel<1024>, dim3((unsigned)T, (unsigned)nblk1k),
                           dim3(256), 0, stream, v, T, n_out, g, idx, K, y);
    else
        hipLaunchKernelGGL(expand_tokens_kernel<256>, dim3((unsigned)T, (unsigned)nblk256),
                           dim3(256), 0, stream, v, T, n_out, g, idx, K, y);
    return hipGetLastError();
}

}  // namespace mlora
