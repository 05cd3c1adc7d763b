// Prefill path: tiled bf16 MFMA GEMM with the LoRA delta folded in as extra K-steps (SGMV).
//
// "Multi-LoRA Serving Explained" (sevydevy.com): the segmented method groups the tokens of one
// adapter together so each adapter's matrices are read once per group, not once per token
// (the six-token script's segmented variant; SGMV in the multi-tenant serving paper it cites),
// and the shared base product stays one big matrix multiplication.  The vLLM RFC on per-request
// composition (Semantics; Testing) notes that k-slot composition equals a rank-concatenated
// ("cat-merged") virtual adapter; here every 256-token tile gets exactly that, built on the fly:
//
//  1. tile plan (one workgroup per tile of PF_BM tokens): the distinct adapters used by the
//     tile's (token, slot) pairs, ascending, and each adapter's number of tokens;
//  2. SGMV shrink: V[token][col(s, d, rho)] = c_t * sum_i A[a][s][rho][i] x[t][i] on the
//     matrix cores (a tile with few adapters: one product of its x with the stacked A rows,
//     n_in split across workgroups and the parts added in order by a second small kernel; a
//     tile with many: each adapter's tokens gathered),
//     c_t = sum over the token's slots holding a of s[t][j] * f[a].  V is kept as two bf16
//     halves, hi = bf16(v) and lo = bf16(v - hi) (about 16 significant bits: a single bf16
//     rounding of v breaks the layer's tolerance when s*f is large, e.g. rsLoRA at rank 64),
//     in one column block of width 2R per adapter and slice, zeros where a token does not use it;
//  3. GEMM: y = bf16( x W^T + V B_cat^T ), where B_cat[n][col(s, d, h, rho)] = B[a_d][n][rho]
//     for both halves h if row n belongs to slice s, else 0.  The main K loop walks n_in, the
//     extra K loop walks the tile's V columns (only the slices the output tile touches), so the
//     expand costs one K-block of 64 per 32/R adapters and the output is rounded once.
//
// GEMM tile: PF_BN = 256 rows of W x PF_BM = 256 tokens x 64 columns, 8 waves (4 along W rows x
// 2 along tokens, 64 x 128 each), v_mfma_f32_16x16x32_bf16 with W rows as the A operand so each
// lane ends up with 4 consecutive outputs of one token (one 8-byte store).  LDS is double
// buffered (2 x 64 KB); 16-byte chunks are XOR-swizzled by row so the operand reads are
// conflict-free.  Workgroups walk the output tiles in groups of 8 n-tiles per m-tile so that
// workgroups running together share x and W panels in L2.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace mlora {

constexpr int PF_BM = 256;   // tokens per tile
constexpr int PF_BN = 256;   // rows of W per tile
constexpr int PF_BK = 64;    // column granule of a tile's V block (its width is a multiple)

// Masked loads read this static block instead of choosing zero after the load: the choice is
// made on the address, so nothing waits for a load right after it is issued.
__device__ __attribute__((aligned(64))) uint32_t pf_zero16[16];   // never written: zeros

// One 16-byte copy per lane from global memory straight into LDS (64 lanes: 1 KB contiguous
// at lds).
__device__ __forceinline__ void pf_dma(const void *g, uint16_t *lds)
{
    __builtin_amdgcn_global_load_lds(g, (void __attribute__((address_space(3))) *)lds, 16, 0, 0);
}

// ------------------------------------------------------------------------------------------
// 1. tile plan
// ------------------------------------------------------------------------------------------
// A tile is "scattered" when its stacked adapters would add more than n_in / 2 k-columns per
// slice to the GEMM (e.g. 256 decode tokens over 64 adapters): its shrink and expand then run per
// adapter over that adapter's tokens only (sgmv_shrink_kernel's group items, sc_expand_kernel),
// and the GEMM leaves fp32 sums for it instead of extra k-steps.
__device__ __forceinline__ bool tile_scattered(int D, int R, int n_in)
{
    return D > 0 && (int64_t)D * 2 * R > n_in / 2;
}

// Width of one adapter's half of a tile's V block: the smallest power of two at or above the
// largest true rank (rounded to 8) among the tile's adapters, never above R.  Columns past an
// adapter's rank would multiply its zero padding, so they are left out of the extra k-steps.
__device__ __forceinline__ int tile_vwidth(int r8max, int R)
{
    int w = 8;
    while (w < r8max)
        w <<= 1;
    return min(w, R);
}

// Token i (0..15) of a group record's token bytes.
__device__ __forceinline__ int grp_token(const int4 &gt, int i)
{
    const int w = i >> 2;
    const uint32_t v = (uint32_t)(w == 0 ? gt.x : w == 1 ? gt.y : w == 2 ? gt.z : gt.w);
    return (int)((v >> ((i & 3) * 8)) & 255u);
}

// Exclusive scan of two values over the 256 threads of a workgroup; ws holds 8 ints.
__device__ __forceinline__ void block_scan2(int v1, int v2, int *ws, int &ex1, int &ex2, int &all1,
                                            int &all2)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int t1, t2;
    const int e1 = wave_exclusive_scan(v1, &t1);
    const int e2 = wave_exclusive_scan(v2, &t2);
    if (lane == 0) {
        ws[wv] = t1;
        ws[4 + wv] = t2;
    }
    __syncthreads();
    int b1 = 0, b2 = 0;
    all1 = 0;
    all2 = 0;
    for (int w = 0; w < 4; ++w) {
        b1 += w < wv ? ws[w] : 0;
        b2 += w < wv ? ws[4 + w] : 0;
        all1 += ws[w];
        all2 += ws[4 + w];
    }
    __syncthreads();
    ex1 = b1 + e1;
    ex2 = b2 + e2;
}

// One workgroup of 256 threads per tile.  For a scattered tile it also lists, per adapter of
// the tile (list order), the tile-local tokens that use it (entries toff[d] .. toff[d+1] of the
// tile's list, built in LDS), in groups of 16 numbered by gpre[d] = sum over d' < d of
// ceil(count / 16), and writes one record per group: {position d, adapter, the tile's V
// columns per slice, tokens | the adapter's rank rounded to 8 << 8 | log2 of the tile's V width
// << 20}, then the group's up to 16 tile-local token numbers as bytes, so that a consumer has
// the group's tokens and where its V goes after one load.  The order of the tokens inside a
// list is whatever the atomics give; each token's results do not depend on it.
static_assert(PF_BM == 256, "tile_plan_kernel: one thread per token of a tile");
__global__ __launch_bounds__(256) void tile_plan_kernel(const int32_t *__restrict__ idx, int T,
                                                        int K, int S, int R, int n_slices, int n_in,
                                                        const int32_t *__restrict__ rank,
                                                        int list_stride, int32_t *tile_D,
                                                        int32_t *tile_w,
                                                        int32_t *tile_list, int32_t *tile_toff,
                                                        int32_t *tile_gpre, int4 *tile_grp,
                                                        int grp_stride, int force_scatter)
{
    // bits[(S+31)/32], cnt[S], r8[S], lst[list_stride], tok[256 K] bytes
    extern __shared__ uint32_t plan_lds[];
    const int nw = (S + 31) / 32;
    uint32_t *bits = plan_lds;
    int *cnt = (int *)(plan_lds + nw);
    int *r8 = cnt + S;
    int *lst = r8 + S;
    uint8_t *tok = (uint8_t *)(lst + list_stride);
    __shared__ int wsum[8];
    const int m = blockIdx.x;
    const int t0 = m * PF_BM;
    const int nt = min(PF_BM, T - t0);
    // thread tl holds token tl's slot ids (256 threads, 256 tokens a tile), distinct ids only
    // (a repeated id is -1 here), loaded before the LDS is cleared so that the slot map and
    // the slots' ranks are read in one round trip
    const int tl = threadIdx.x;
    int ids[MLORA_MAX_K_DEV];
#pragma unroll
    for (int j = 0; j < MLORA_MAX_K_DEV; ++j)
        ids[j] = j < K && tl < nt ? idx[(int64_t)(t0 + tl) * K + j] : -1;
    for (int i = threadIdx.x; i < nw; i += blockDim.x)
        bits[i] = 0u;
    for (int i = threadIdx.x; i < S; i += blockDim.x) {
        cnt[i] = 0;
        r8[i] = slot_rank8(rank, i, R);
    }
#pragma unroll
    for (int j = 1; j < MLORA_MAX_K_DEV; ++j) {
        bool dup = false;
#pragma unroll
        for (int jj = 0; jj < j; ++jj)
            dup |= ids[jj] == ids[j];
        if (dup)
            ids[j] = -1;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < MLORA_MAX_K_DEV; ++j) {
        const int a = ids[j];
        if (a >= 0) {
            atomicOr(&bits[a >> 5], 1u << (a & 31));
            atomicAdd(&cnt[a], 1);
        }
    }
    __syncthreads();
    // ascending list of the set bits: exclusive scan of per-word popcounts
    int base = 0;
    for (int w0 = 0; w0 < nw; w0 += blockDim.x) {
        const int w = w0 + threadIdx.x;
        const uint32_t b = w < nw ? bits[w] : 0u;
        int ex, unused, all, unused2;
        block_scan2(__popc(b), 0, wsum, ex, unused, all, unused2);
        int pos = base + ex;
        uint32_t bb = b;
        while (bb) {
            const int bit = __ffs(bb) - 1;
            bb &= bb - 1;
            const int a = w * 32 + bit;
            tile_list[(int64_t)m * list_stride + pos] = a;
            lst[pos] = a;
            ++pos;
        }
        base += all;
    }
    if (threadIdx.x == 0)
        tile_D[m] = base;
    const int D = base;
    __syncthreads();                              // lst complete
    // the tile's V width: largest rounded rank among its adapters (block maximum via wsum)
    int r8max = 0;
    for (int d = threadIdx.x; d < D; d += blockDim.x)
        r8max = max(r8max, r8[lst[d]]);
    for (int off = 32; off >= 1; off >>= 1)
        r8max = max(r8max, __shfl_xor(r8max, off, 64));
    if ((threadIdx.x & 63) == 0)
        wsum[threadIdx.x >> 6] = r8max;
    __syncthreads();
    r8max = max(max(wsum[0], wsum[1]), max(wsum[2], wsum[3]));
    const int VW = tile_vwidth(r8max, R);
    if (threadIdx.x == 0)
        tile_w[m] = VW;
    __syncthreads();                              // wsum free again
    if (force_scatter || tile_scattered(D, R, n_in)) {
        int32_t *toff = tile_toff + (int64_t)m * (list_stride + 1);
        int32_t *gpre = tile_gpre + (int64_t)m * (list_stride + 1);
        int obase = 0, gbase = 0;
        int my_o0 = 0, my_o1 = 0, my_g0 = 0;     // list range and first group of adapter tid
        for (int d0 = 0; d0 < D; d0 += blockDim.x) {
            const int d = d0 + threadIdx.x;
            const int c = d < D ? cnt[lst[d]] : 0;
            int oex, gex, oall, gall;
            block_scan2(c, (c + 15) >> 4, wsum, oex, gex, oall, gall);
            if (d < D) {
                toff[d] = obase + oex;
                gpre[d] = gbase + gex;
                cnt[lst[d]] = obase + oex;        // now the next free place of adapter lst[d]
                if (d0 == 0) {
                    my_o0 = obase + oex;
                    my_o1 = my_o0 + c;
                    my_g0 = gbase + gex;
                }
            }
            obase += oall;
            gbase += gall;
        }
        if (threadIdx.x == 0) {
            toff[D] = obase;
            gpre[D] = gbase;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < MLORA_MAX_K_DEV; ++j)
            if (ids[j] >= 0)
                tok[atomicAdd(&cnt[ids[j]], 1)] = (uint8_t)tl;
        __syncthreads();                          // the lists complete
        int4 *grp = tile_grp + (int64_t)m * grp_stride * 2;
        // the tile's V block geometry goes into every record, so that a consumer needs no
        // other load before its V reads: columns per slice, and log2 of the V width
        const int kxs = ((D * 2 * VW + PF_BK - 1) / PF_BK) * PF_BK;
        const int lvw = 31 - __clz(VW);
        for (int d = threadIdx.x; d < D; d += blockDim.x) {
            // the first 256 adapters' ranges are still in registers; the rest are read back
            // (the stores above are this workgroup's own, ordered by the barrier)
            const bool mine = d == (int)threadIdx.x;
            const int o0 = mine ? my_o0 : toff[d], o1 = mine ? my_o1 : toff[d + 1];
            const int g0 = mine ? my_g0 : gpre[d];
            for (int o = o0; o < o1; o += 16) {
                const int n = min(16, o1 - o);
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                for (int i = 0; i < n; ++i)
                    w[i >> 2] |= (uint32_t)tok[o + i] << ((i & 3) * 8);
                const int gi = g0 + (o - o0) / 16;
                grp[2 * gi] = int4{d, lst[d], kxs, n | (r8[lst[d]] << 8) | (lvw << 20)};
                grp[2 * gi + 1] = int4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            }
        }
    }
    // (the V block's columns past 2 D VW, up to the 64-column k-step, are never written: the
    // GEMM copies zeros in their place)
}

// ------------------------------------------------------------------------------------------
// 2. SGMV shrink into V
// ------------------------------------------------------------------------------------------
// The tile's D adapters are stacked into one "cat" matrix A_cat (D * n_slices * VW rows: each
// slice's first VW rows, VW the tile's V width, the power of two at or above its largest rank),
// so the shrink of a tile is one dense product V_tile = X_tile A_cat^T; a token that does not
// use adapter d gets coefficient 0 for d's columns (the zeros the GEMM's extra K-steps expect).
// Rows past an adapter's own rank are copied from the zero block, not read.
//
// Dense item = (tile m, 128-row block rb of A_cat, part kp of n_in split in ks parts): all 256
// tokens of the tile against the block's rows over the part's columns.  Operands are copied
// straight into LDS (global_load_lds_dwordx4) in stages of 64 columns whose rows are 128 bytes
// (whole cache lines per request), three stages deep (two in flight while one is multiplied);
// wave w multiplies tokens 64w .. 64w+63 against the 128 rows.  With ks = 1 the item applies
// the coefficients and writes V; with ks > 1 it writes its fp32 partial block and
// shrink_reduce_kernel adds the parts in order.  ks is chosen in the kernel (every workgroup
// computes the same value) so that there are about SD_TARGET items and the partial blocks fit
// their workspace region.
// Scattered tiles have group items instead (below).  The items of all tiles are numbered
// through a prefix over the tiles and shared out to a persistent grid.
constexpr int SH_THREADS = 256;
constexpr int SH_MAX_TILES = 4096;   // tiles whose item prefix fits LDS
constexpr int SD_ROWS = 128;         // A_cat rows of a dense item
constexpr int SD_KS = 64;            // columns per stage
constexpr int SD_STAGE_ELEMS = (PF_BM + SD_ROWS) * SD_KS;   // bf16: 256 x rows, then A rows
constexpr int SD_STAGE_BYTES = SD_STAGE_ELEMS * 2;          // 48 KB
constexpr int SD_KS_MAX = 16;        // most parts of n_in
constexpr int SD_TARGET = 256;       // dense items aimed for
constexpr int SD_PART_ELEMS = PF_BM * SD_ROWS;              // fp32 partial block of an item
constexpr int SD_TABLE_BYTES = 9;    // LDS per tile for the item tables (pre, pbase, grouped)

struct ShrinkArgs {
    const uint16_t *x;
    int T, n_in, K;
    SlotGeom g;
    const int32_t *idx;
    const float *scale;
    int n_mtiles, list_stride;
    const int32_t *tile_D, *tile_list;
    const int32_t *tile_w;   // V width of each tile (tile plan)
    uint16_t *vcat;
    int64_t vcat_tile_elems;
    int32_t *tile_ord;    // out: ordinal of a scattered tile (< sc_cap), else -1
    int32_t *sc_tiles;    // out: [sc_cap] tile of each ordinal, then their count
    int sc_cap;
    const int32_t *tile_toff, *tile_gpre;   // scattered tiles: list offsets (tile plan)
    const int4 *tile_grp;                   // scattered tiles: group records, 2 x int4 each
    int grp_stride;
    int32_t *sc_pre;      // out: [sc_cap + 1] expand items before each scattered ordinal, total
    int n_chunks;         // output row chunks of an expand item
    float *sd_part;       // [sd_cap_slots][256][128] fp32 partial blocks (ks > 1)
    int sd_cap_slots;
    int32_t *tile_pbase;  // out: first partial slot / SD block of a dense tile, -1 otherwise
    int32_t *sd_ks;       // out: ks of this launch
    int stages;           // dense item stages in LDS (2 or 3)
    int skip_groups;      // 1: the GEMM's helper workgroups run the group items instead
    int force_scatter;    // 1: every tile takes the scattered route (grouped decode)
};

// Coefficient of adapter a for token t: the sum of s[t][j] * f[a] over the slots j holding a.
__device__ __forceinline__ float sh_coef(const ShrinkArgs &P, int t, int a)
{
    const int32_t *it = P.idx + (int64_t)t * P.K;
    float cf = 0.f;
    for (int j = 0; j < P.K; ++j)
        if (it[j] == a)
            cf += (P.scale ? P.scale[(int64_t)t * P.K + j] : 1.f) * P.g.factor[a];
    return cf;
}

// v as the pair hi = bf16(v), lo = bf16(v - hi), R columns apart
__device__ __forceinline__ void sh_store_v(uint16_t *vp, int R, float v)
{
    const uint16_t vh = f32_to_bf16(v);
    vp[0] = vh;
    vp[R] = f32_to_bf16(v - bf16_to_f32(vh));
}

// The k-columns [kb, kend) of this wave: n_in split in 4, each part a multiple of 32 wide (the
// last may be short).
__device__ __forceinline__ void sh_wave_cols(int n_in, int wave, int &kb, int &kend, int &nsteps)
{
    const int kq = ((n_in + 4 * 32 - 1) / (4 * 32)) * 32;
    kb = wave * kq;
    kend = min(n_in, kb + kq);
    nsteps = kend > kb ? (kend - kb + 31) / 32 : 0;
}

// The n_in split of the dense items: ks parts of kc columns (a multiple of SD_KS), for
// total_rb 128-row blocks over all dense tiles.  The same on every workgroup and in the reduce.
__device__ __forceinline__ void sd_split(int total_rb, int n_in, int cap_slots, int &ks, int &kc)
{
    int k0 = 1;
    if (total_rb > 0) {
        k0 = min(SD_KS_MAX, (SD_TARGET + total_rb - 1) / total_rb);
        k0 = min(k0, cap_slots / total_rb);
        k0 = min(k0, n_in / 256);
        k0 = max(k0, 1);
    }
    kc = ((n_in + k0 - 1) / k0 + SD_KS - 1) / SD_KS * SD_KS;
    ks = (n_in + kc - 1) / kc;
}

// Copies of stage q (columns c0 .. c0+63) into the stage buffer sb: wave w copies its 64 token
// rows (8 instructions of 8 rows x 128 bytes) and A rows 32w .. 32w+31 (4 instructions).
// Chunk c of row r sits at position c ^ (r & 7) of its row.
__device__ __forceinline__ void sd_issue(uint16_t *sb, const uint16_t *const (&xr)[8],
                                         const uint16_t *const (&ar)[4], uint32_t rmask, int c0,
                                         int kend, int wave, int lane)
{
    const int c = ((lane & 7) ^ (lane >> 3)) * 8;
    const bool ok = c0 + c < kend;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        pf_dma(ok && (rmask >> i & 1u) ? (const void *)(xr[i] + c0 + c) : (const void *)pf_zero16,
               sb + (wave * 64 + i * 8) * SD_KS);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        pf_dma(ok && (rmask >> (8 + i) & 1u) ? (const void *)(ar[i] + c0 + c)
                                             : (const void *)pf_zero16,
               sb + (PF_BM + wave * 32 + i * 8) * SD_KS);
}

// MFMAs of one stage (two k-steps of 32): the wave's 4 token groups x ni row groups of 16.
__device__ __forceinline__ void sd_compute(const uint16_t *sb, int wave, int r, int gq, int ni,
                                           f32x4 (&acc)[8][4])
{
    const uint16_t *sx = sb, *sa = sb + PF_BM * SD_KS;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
        const int pos = (k2 * 4 + gq) ^ (r & 7);
        bf16x8 xf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            xf[j] = *(const bf16x8 *)(sx + ((wave * 64 + j * 16 + r) * 8 + pos) * 8);
        bf16x8 af[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            af[i] = *(const bf16x8 *)(sa + ((i * 16 + r) * 8 + pos) * 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i < ni) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], xf[j], acc[i][j],
                                                                        0, 0, 0);
            }
        }
    }
}

__device__ __forceinline__ void sh_dense_item(const ShrinkArgs &P, int m, int rb, int kp, int ks,
                                              int kc, int slot, uint16_t *lds)
{
    const SlotGeom &g = P.g;
    const int R = g.R, wd = g.n_slices * R;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, gq = lane >> 4;
    const int D = P.tile_D[m];
    const int32_t *list = P.tile_list + (int64_t)m * P.list_stride;
    const int VW = P.tile_w[m], wv = g.n_slices * VW;   // A_cat rows per adapter
    const int rows_cat = D * wv;
    const int row0 = rb * SD_ROWS;
    const int ni = min(8, (rows_cat - row0 + 15) / 16);   // row groups with a row of A_cat
    const int kbeg = kp * kc, kend = min(P.n_in, kbeg + kc);
    const int nst = (kend - kbeg + SD_KS - 1) / SD_KS;

    // row pointers of this lane's copies, and which of them are real rows (bit i: x row i,
    // bit 8 + i: A row i; the others are copied from the zero block).  Rows past their
    // adapter's rank (zero padding) are not read.
    const int rr = lane >> 3;
    const uint16_t *xr[8], *ar[4];
    uint32_t rmask = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int t = m * PF_BM + wave * 64 + i * 8 + rr;
        xr[i] = P.x + (int64_t)min(t, P.T - 1) * P.n_in;
        rmask |= (t < P.T ? 1u : 0u) << i;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int a_row = row0 + wave * 32 + i * 8 + rr;
        const int ac = min(a_row, rows_cat - 1);
        const int d = ac / wv, rin = ac - d * wv, sg = rin / VW, rho = rin - sg * VW;
        const bool ok = a_row < rows_cat && rho < slot_rank8(g.rank, list[d], R);
        ar[i] = g.A + ((int64_t)list[d] * wd + sg * R + rho) * P.n_in;
        rmask |= (ok ? 1u : 0u) << (8 + i);
    }

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // stages: issue up to S - 1 ahead; before multiplying stage q, wait for this wave's copies
    // of it (12 per stage, in order) and publish them with a barrier; stage q + S - 1 then goes
    // into the buffer stage q - 1 used, which every wave has finished with
    const int S = P.stages;
    for (int q = 0; q < S - 1 && q < nst; ++q)
        sd_issue(lds + q * SD_STAGE_ELEMS, xr, ar, rmask, kbeg + q * SD_KS, kend, wave, lane);
    for (int q = 0; q < nst; ++q) {
        const int ahead = min(S - 2, nst - 1 - q);    // stages issued after q
        if (ahead >= 1)
            asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        if (q + S - 1 < nst)
            sd_issue(lds + ((q + S - 1) % S) * SD_STAGE_ELEMS, xr, ar, rmask,
                     kbeg + (q + S - 1) * SD_KS, kend, wave, lane);
        sd_compute(lds + (q % S) * SD_STAGE_ELEMS, wave, r, gq, ni, acc);
    }
    __syncthreads();   // the stage buffers are free for the next item

    // lane holds rows row0 + 16i + 4gq + e (e = 0..3) of token wave*64 + 16j + r
    if (ks > 1) {
        float *pb = P.sd_part + (int64_t)slot * SD_PART_ELEMS;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i < ni) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *(float4 *)(pb + (wave * 64 + j * 16 + r) * SD_ROWS + i * 16 + gq * 4) =
                        float4{acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
            }
        }
        return;
    }
    const int kxs = ((D * 2 * VW + PF_BK - 1) / PF_BK) * PF_BK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tl = wave * 64 + j * 16 + r;
        const int t = m * PF_BM + tl;
        if (t >= P.T)
            continue;
        uint16_t *vrow = P.vcat + (int64_t)m * P.vcat_tile_elems + (int64_t)tl * (g.n_slices * kxs);
        int dprev = -1;
        float cf = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int a_row = row0 + i * 16 + gq * 4 + e;
                if (i >= ni || a_row >= rows_cat)
                    continue;
                const int d = a_row / wv;
                if (d != dprev) {
                    cf = sh_coef(P, t, list[d]);
                    dprev = d;
                }
                const int rin = a_row - d * wv, sg = rin / VW, rho = rin - sg * VW;
                sh_store_v(vrow + sg * kxs + d * 2 * VW + rho, VW, cf * acc[i][j][e]);
            }
        }
    }
}

// Group item of a scattered tile (token group gidx of one adapter, 32-row block rb of that
// adapter's n_slices * R rows of A): only the up to 16 tokens that use the adapter, gathered
// as the MFMA's token columns, against 32 rows; SG_ST k-steps of loads in flight.
constexpr int SG_ROWS = 32;
constexpr int SG_ST = 4;

__device__ __forceinline__ void sg_load(const uint16_t *const (&ap)[2], const bool (&aok)[2],
                                        const uint16_t *xp, bool xok, int col, int kend,
                                        u32x4 (&af)[2], u32x4 &xf)
{
    const int off = ((threadIdx.x & 63) >> 4) * 8;
    const bool ok = col + off < kend;
    af[0] = *(const u32x4 *)(ok && aok[0] ? (const void *)(ap[0] + col) : (const void *)pf_zero16);
    af[1] = *(const u32x4 *)(ok && aok[1] ? (const void *)(ap[1] + col) : (const void *)pf_zero16);
    xf = *(const u32x4 *)(ok && xok ? (const void *)(xp + col) : (const void *)pf_zero16);
}

// tid: the thread's index among the item's 256 threads (its wave is tid / 64); red: 8 KB of
// LDS for the item.  Every thread of the workgroup meets exactly two barriers.
__device__ __forceinline__ void sh_group_item(const ShrinkArgs &P, int m, int local, float4 *red,
                                              int tid)
{
    const SlotGeom &g = P.g;
    const int R = g.R, wd = g.n_slices * R;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, gq = lane >> 4;
    const int RB = (wd + SG_ROWS - 1) / SG_ROWS;
    const int gidx = local / RB, rb = local - gidx * RB;
    const int4 *rec = P.tile_grp + ((int64_t)m * P.grp_stride + gidx) * 2;
    // {d, adapter, V columns per slice, tokens | rank rounded to 8 << 8 | log2 VW << 20},
    // then the token bytes
    const int4 gr = rec[0], gt = rec[1];
    const int d = gr.x, a = gr.y, ng = gr.w & 0xff;
    // rows past the adapter's rank (zero padding) are neither read nor multiplied: their
    // fragments come from the zero block, and a block with no row below the rank skips the loop
    const int rk = (gr.w >> 8) & 0xfff;
    const uint16_t *ap[2];
    bool aok[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int row = rb * SG_ROWS + f * 16 + r;
        aok[f] = row < wd && row % R < rk;
        ap[f] = g.A + ((int64_t)a * wd + min(row, wd - 1)) * P.n_in + gq * 8;
    }
    const bool any_row = __ballot(aok[0] || aok[1]) != 0ull;
    const bool xok = r < ng && any_row;
    const uint16_t *xp = P.x + ((int64_t)m * PF_BM + (r < ng ? grp_token(gt, r) : 0)) * P.n_in + gq * 8;
    int kb, kend, nsteps;
    sh_wave_cols(P.n_in, wave, kb, kend, nsteps);
    if (!any_row)
        nsteps = 0;

    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    u32x4 af[SG_ST][2], xf[SG_ST];
#pragma unroll
    for (int s = 0; s < SG_ST; ++s)
        sg_load(ap, aok, xp, xok, kb + s * 32, kend, af[s], xf[s]);
    for (int st = 0; st < nsteps; st += SG_ST) {
#pragma unroll
        for (int s = 0; s < SG_ST; ++s) {
#pragma unroll
            for (int f = 0; f < 2; ++f)
                acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, af[s][f]), __builtin_bit_cast(bf16x8, xf[s]), acc[f],
                    0, 0, 0);
            sg_load(ap, aok, xp, xok, kb + (st + s + SG_ST) * 32, kend, af[s], xf[s]);
        }
    }

    // lane holds rows rb*32 + 16f + 4gq + e of gathered token r
#pragma unroll
    for (int f = 0; f < 2; ++f)
        red[(wave * 2 + f) * 64 + lane] = float4{acc[f][0], acc[f][1], acc[f][2], acc[f][3]};
    __syncthreads();
    // thread: gathered token j = tid % 16, rows 2 * (tid / 16) and the next
    const int j = tid & 15, rp = (tid >> 4) * 2;
    if (j < ng) {
        const int tl = grp_token(gt, j);
        const float cf = sh_coef(P, m * PF_BM + tl, a);
        const int VW = 1 << (gr.w >> 20), kxs = gr.z;
        uint16_t *vrow = P.vcat + (int64_t)m * P.vcat_tile_elems + (int64_t)tl * (g.n_slices * kxs) +
                         d * 2 * VW;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int rl = rp + e, row = rb * SG_ROWS + rl;
            if (row >= wd)
                break;
            const int f = rl >> 4, rr = rl & 15;
            const int ln = j + 16 * (rr >> 2), comp = rr & 3;
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float4 v4 = red[(w * 2 + f) * 64 + ln];
                sum += comp == 0 ? v4.x : comp == 1 ? v4.y : comp == 2 ? v4.z : v4.w;
            }
            const int sg = row / R, rho = row - sg * R;
            if (rho < VW)
                sh_store_v(vrow + sg * kxs + rho, VW, cf * sum);
        }
    }
    __syncthreads();
}

// 128-row blocks of tile m's A_cat (D adapters, n_slices * VW rows each)
__device__ __forceinline__ int sd_row_blocks(const ShrinkArgs &P, int m, int D)
{
    return (D * P.g.n_slices * P.tile_w[m] + SD_ROWS - 1) / SD_ROWS;
}

constexpr int SG_RED_BYTES = 4 * 2 * 64 * 16;   // a group item's reduction space (8 KB)

// GO (groups only): every tile scattered (the grouped decode), so no dense item code, few
// registers and 8 KB of LDS: the kernel can share CUs with the decode GEMM it runs beside.
template <bool GO>
__global__ __launch_bounds__(SH_THREADS) void sgmv_shrink_kernel(ShrinkArgs P)
{
    extern __shared__ __attribute__((aligned(16))) float sh_lds[];
    // stage buffers of the dense items (the group items' reduction space shares them), then
    // the item tables
    uint16_t *stages = (uint16_t *)sh_lds;
    float4 *red = (float4 *)sh_lds;                           // [4 waves][16][64] float4
    const size_t tbl_off = GO ? (size_t)SG_RED_BYTES : (size_t)P.stages * SD_STAGE_BYTES;
    int *pre = (int *)((uint8_t *)sh_lds + tbl_off);          // item prefix
    int *pbase = pre + P.n_mtiles;                            // first 128-row block of a tile
    uint8_t *grouped = (uint8_t *)(pbase + P.n_mtiles);       // 1: group items
    __shared__ int wsum[8];
    const int wd = P.g.n_slices * P.g.R;
    const int RBg = (wd + SG_ROWS - 1) / SG_ROWS;

    // Pass 1: which tiles take group items (a scattered tile whose ordinal is below sc_cap),
    // and the 128-row blocks of the others; workgroup 0 also numbers the scattered tiles and
    // the expand's items (each kept tile's 16-token groups x the output row chunks).
    int rb_base = 0, sc_base = 0, ei_base = 0;
    for (int m0 = 0; m0 < P.n_mtiles; m0 += SH_THREADS) {
        const int m = m0 + threadIdx.x;
        const int Dm = m < P.n_mtiles ? P.tile_D[m] : 0;
        const int scm =
            m < P.n_mtiles && (P.force_scatter || tile_scattered(Dm, P.g.R, P.n_in)) ? 1 : 0;
        int sc_ex, sc_all, u0, u1;
        block_scan2(scm, 0, wsum, sc_ex, u0, sc_all, u1);
        const int ord = sc_base + sc_ex;
        const bool kept = scm && ord < P.sc_cap;
        const int rbs = kept || m >= P.n_mtiles ? 0 : sd_row_blocks(P, m, Dm);
        // expand items of a kept scattered tile (its 16-token groups x the row chunks)
        const int eit = kept ? P.tile_gpre[(int64_t)m * (P.list_stride + 1) + Dm] * P.n_chunks : 0;
        int rb_ex, rb_all, ei_ex, ei_all;
        block_scan2(rbs, eit, wsum, rb_ex, ei_ex, rb_all, ei_all);
        if (m < P.n_mtiles) {
            grouped[m] = kept ? 1 : 0;
            pbase[m] = rbs > 0 ? rb_base + rb_ex : -1;
        }
        if (blockIdx.x == 0 && m < P.n_mtiles) {
            P.tile_ord[m] = kept ? ord : -1;
            if (kept) {
                P.sc_tiles[ord] = m;
                P.sc_pre[ord] = ei_base + ei_ex;
            }
        }
        rb_base += rb_all;
        sc_base += sc_all;
        ei_base += ei_all;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        P.sc_tiles[P.sc_cap] = min(sc_base, P.sc_cap);
        P.sc_pre[P.sc_cap] = ei_base;
    }
    int ks, kc;
    sd_split(rb_base, P.n_in, P.sd_cap_slots, ks, kc);
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int m = threadIdx.x; m < P.n_mtiles; m += SH_THREADS)
            P.tile_pbase[m] = pbase[m] >= 0 ? pbase[m] * ks : -1;
        if (threadIdx.x == 0)
            *P.sd_ks = ks;
    }

    // Pass 2: items of tile m: group items, or ks parts of each 128-row block
    int base = 0;
    for (int m0 = 0; m0 < P.n_mtiles; m0 += SH_THREADS) {
        const int m = m0 + threadIdx.x;
        int cnt = 0;
        if (m < P.n_mtiles) {
            const int Dm = P.tile_D[m];
            cnt = grouped[m] ? (P.skip_groups ? 0
                                              : P.tile_gpre[(int64_t)m * (P.list_stride + 1) + Dm] *
                                                    RBg)
                             : (GO ? 0 : sd_row_blocks(P, m, Dm) * ks);
        }
        int ex, all, u0, u1;
        block_scan2(cnt, 0, wsum, ex, u0, all, u1);
        if (m < P.n_mtiles)
            pre[m] = base + ex;
        base += all;
    }
    const int total = base;
    __syncthreads();

    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        // tile: last m with pre[m] <= item
        int lo = 0, hi = P.n_mtiles - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= item)
                lo = mid;
            else
                hi = mid - 1;
        }
        const int local = item - pre[lo];
        if (grouped[lo]) {
            sh_group_item(P, lo, local, red, threadIdx.x);
        } else if constexpr (!GO) {
            const int rb = local / ks, kp = local - rb * ks;
            sh_dense_item(P, lo, rb, kp, ks, kc, (pbase[lo] + rb) * ks + kp, stages);
        }
    }
}

// Adds the ks partial blocks of the dense tiles in part order, applies each token's
// coefficients and writes V (bf16 hi/lo halves).  One workgroup per (tile, 16 tokens); each
// thread takes 4 consecutive rows of A_cat for one token (one adapter and slice: R is a
// multiple of 4), so its partials are float4 loads and its V halves 8-byte stores.  The
// tokens' slot ids and scales, and the tile's adapter ids and factors (the first SR_D of them;
// more are read from global memory), are staged in LDS first.  Nothing to do when the launch
// used ks = 1 (the items wrote V themselves) or for group-item tiles.
constexpr int SR_TOK = 16;
constexpr int SR_D = 1024;

__global__ __launch_bounds__(256) void shrink_reduce_kernel(ShrinkArgs P)
{
    __shared__ int s_idx[SR_TOK * MLORA_MAX_K_DEV];
    __shared__ float s_sc[SR_TOK * MLORA_MAX_K_DEV];
    __shared__ int s_a[SR_D];
    __shared__ float s_f[SR_D];
    const int m = blockIdx.x / (PF_BM / SR_TOK);
    const int t0l = (blockIdx.x % (PF_BM / SR_TOK)) * SR_TOK;
    const int ks = *P.sd_ks;
    const int pb = P.tile_pbase[m];
    const int nt = min(SR_TOK, P.T - (m * PF_BM + t0l));
    if (ks <= 1 || pb < 0 || nt <= 0)
        return;
    const SlotGeom &g = P.g;
    const int K = P.K;
    const int D = P.tile_D[m];
    const int32_t *list = P.tile_list + (int64_t)m * P.list_stride;
    const int64_t tb = (int64_t)m * PF_BM + t0l;   // first token of the block
    for (int i = threadIdx.x; i < nt * K; i += 256) {
        s_idx[i] = P.idx[tb * K + i];
        s_sc[i] = P.scale ? P.scale[tb * K + i] : 1.f;
    }
    for (int d = threadIdx.x; d < min(D, SR_D); d += 256) {
        const int a = list[d];
        s_a[d] = a;
        s_f[d] = g.factor[a];
    }
    __syncthreads();
    const int VW = P.tile_w[m], wv = g.n_slices * VW;   // A_cat rows per adapter
    const int rows4 = D * wv / 4;                  // groups of 4 rows
    const int kxs = ((D * 2 * VW + PF_BK - 1) / PF_BK) * PF_BK;
    for (int e = threadIdx.x; e < nt * rows4; e += 256) {
        const int tt = e / rows4, a_row = (e - tt * rows4) * 4;
        const int tl = t0l + tt;
        const int rb = a_row / SD_ROWS, rl = a_row - rb * SD_ROWS;
        const float *src = P.sd_part + ((int64_t)(pb + rb * ks) * PF_BM + tl) * SD_ROWS + rl;
        float4 pv[SD_KS_MAX];
#pragma unroll
        for (int kp = 0; kp < SD_KS_MAX; ++kp)
            if (kp < ks)
                pv[kp] = *(const float4 *)(src + (int64_t)kp * SD_PART_ELEMS);
        float4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < SD_KS_MAX; ++kp) {
            if (kp < ks) {
                sum.x += pv[kp].x;
                sum.y += pv[kp].y;
                sum.z += pv[kp].z;
                sum.w += pv[kp].w;
            }
        }
        const int d = a_row / wv;
        const int a = d < SR_D ? s_a[d] : list[d];
        const float f = d < SR_D ? s_f[d] : g.factor[a];
        float cf = 0.f;
        for (int j = 0; j < K; ++j)
            if (s_idx[tt * K + j] == a)
                cf += s_sc[tt * K + j] * f;
        const int rin = a_row - d * wv, sg = rin / VW, rho = rin - sg * VW;
        uint16_t *vp = P.vcat + (int64_t)m * P.vcat_tile_elems + (int64_t)tl * (g.n_slices * kxs) +
                       sg * kxs + d * 2 * VW + rho;
        const float v[4] = {cf * sum.x, cf * sum.y, cf * sum.z, cf * sum.w};
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            hi[i] = f32_to_bf16(v[i]);
            lo[i] = f32_to_bf16(v[i] - bf16_to_f32(hi[i]));
        }
        *(u32x2 *)vp = u32x2{(uint32_t)hi[0] | (uint32_t)hi[1] << 16,
                             (uint32_t)hi[2] | (uint32_t)hi[3] << 16};
        *(u32x2 *)(vp + VW) = u32x2{(uint32_t)lo[0] | (uint32_t)lo[1] << 16,
                                   (uint32_t)lo[2] | (uint32_t)lo[3] << 16};
    }
}

// ------------------------------------------------------------------------------------------
// 3. GEMM with the LoRA K-extension
// ------------------------------------------------------------------------------------------
struct GemmArgs {
    const uint16_t *x, *W;
    uint16_t *y;
    int T, n_in, n_out;
    int n_mtiles, n_ntiles;
    int lora;
    SlotGeom g;
    const uint16_t *vcat;
    int64_t vcat_tile_elems;
    const int32_t *tile_D, *tile_list;
    const int32_t *tile_w;     // V width of each tile
    int list_stride;
    const int32_t *tile_ord;   // scattered tile ordinal (sgmv_shrink_kernel), or -1
    float *part_sc;            // fp32 [sc_cap][256][n_out] sums of scattered tiles
    int n_rg, n_kb;            // packed W: row groups of 16, column blocks of 32
    ShrinkArgs sh;             // for the helper workgroups (group items of scattered tiles)
};

// Workgroups past the GEMM's tiles (launched only while the tiles leave CUs idle) run the
// scattered tiles' shrink group items, which the shrink kernel then skips: nothing in the GEMM
// reads a scattered tile's V, only the expand after it.  Two items at a time, waves 0-3 and
// 4-7, each half with 8 KB of the stage LDS; a half without an item meets the other half's
// two barriers.
__device__ void pf_group_helper(const GemmArgs &P, int n_tiles, uint16_t *lds)
{
    const ShrinkArgs &S = P.sh;
    const int n_sc = S.sc_tiles[S.sc_cap];
    const int wd = S.g.n_slices * S.g.R;
    const int RBg = (wd + SG_ROWS - 1) / SG_ROWS;
    auto items_of = [&](int o) {
        const int m = S.sc_tiles[o];
        return S.tile_gpre[(int64_t)m * (S.list_stride + 1) + S.tile_D[m]] * RBg;
    };
    int total = 0;
    for (int o = 0; o < n_sc; ++o)
        total += items_of(o);
    const int h = blockIdx.x - n_tiles, nh = gridDim.x - n_tiles;
    const int half = threadIdx.x >> 8, tid = threadIdx.x & 255;
    float4 *red = (float4 *)lds + half * 512;
    for (int base = 0; base < total; base += 2 * nh) {
        const int item = base + 2 * h + half;
        if (item < total) {
            int o = 0, pre = 0;
            while (item >= pre + items_of(o)) {
                pre += items_of(o);
                ++o;
            }
            sh_group_item(S, S.sc_tiles[o], item - pre, red, tid);
        } else {
            __syncthreads();
            __syncthreads();
        }
    }
}

// GEMM: 256 W rows x 256 tokens per workgroup, 8 waves (4 along W rows x 2 along tokens,
// 64 x 128 each), k-steps of 64 columns.  Operand tiles go from global memory straight into
// LDS (global_load_lds_dwordx4, no register staging), double buffered (2 stages of 64 KB), one
// stage ahead of the MFMAs; each wave waits for its own copies of the next stage and a barrier
// (LDS only) publishes them.  A stage holds W[256][64] and X[256][64], 128 bytes a row: one
// copy instruction fills a contiguous 1 KB block (lane L writes bytes 16 L..16 L+15: 8 rows,
// 8 lanes per row), so every request to L2 is a whole 128-byte line.  (With 64-byte rows the
// copies were bound by the CU's outstanding L2 requests, each carrying half a line.)  The
// 16-byte chunk c of row r sits at position c ^ (r & 7) of its row; with that swizzle the
// operand reads (16 rows x 16 bytes per lane group) measured free of LDS bank conflicts.
// Chunks past n_in, masked B rows and padding are copied from a static block of zeros.
constexpr int PF_KS = 64;                  // columns per stage
constexpr int PF_STAGES = 2;
constexpr int PF_STAGE_BYTES = 2 * 256 * PF_KS * 2;

// Issues this wave's copies of stage q (k-step q: base columns q*64 while q < nk_main, then
// the LoRA extra steps) into buffer `st`: 4 blocks of 8 W rows and 4 of 8 tokens per wave.
// With a packed W (PW) the W side of a stage is 32 fragments of 16 rows x 32 columns in lane
// order instead (4 per wave), for the base steps and the LoRA steps alike.
template <bool PW, bool BASE_ONLY = false>
__device__ __forceinline__ void pf_issue(const GemmArgs &P, uint16_t *st, int q, int nk_main,
                                         int nk_extra, int m0, int n0, const uint16_t *vtile,
                                         int D, int kxs, int VW, int sg_lo, int kb_per_slice,
                                         const int *slist, int wave, int lane)
{
    const int rr = lane >> 3;                       // row within the 8-row block
    const int c = (lane & 7) ^ rr;                  // chunk this lane's position holds
    uint16_t *sw = st, *sx = st + 256 * PF_KS;
    if (BASE_ONLY || q < nk_main) {
        const int k = q * PF_KS + c * 8;
        const bool ok = k < P.n_in;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int row = (wave * 4 + b) * 8 + rr;
            if constexpr (PW) {
                const int f = wave * 4 + b, rg = (n0 >> 4) + (f >> 1), kb = 2 * q + (f & 1);
                const uint16_t *gw = P.W + (((int64_t)min(rg, P.n_rg - 1) * P.n_kb +
                                             min(kb, P.n_kb - 1)) * 64 + lane) * 8;
                pf_dma(rg < P.n_rg && kb < P.n_kb ? (const void *)gw : (const void *)pf_zero16,
                       sw + f * 512);
            } else {
                const uint16_t *gw = P.W + (int64_t)min(n0 + row, P.n_out - 1) * P.n_in + k;
                pf_dma(ok ? (const void *)gw : (const void *)pf_zero16, sw + (wave * 4 + b) * 8 * PF_KS);
            }
            const uint16_t *gx = P.x + (int64_t)min(m0 + row, P.T - 1) * P.n_in + k;
            pf_dma(ok ? (const void *)gx : (const void *)pf_zero16, sx + (wave * 4 + b) * 8 * PF_KS);
        }
    } else if constexpr (!BASE_ONLY) {
        const int R = P.g.R;
        const int ke = min(q - nk_main, nk_extra - 1);
        const int sg = sg_lo + ke / kb_per_slice;
        const int kk0 = (ke % kb_per_slice) * PF_KS;          // first column of the step
        const int kk = kk0 + c * 8;                           // column within the slice block
        const int dd = kk / (2 * VW);
        const int rho = (kk - dd * 2 * VW) & (VW - 1);
        // the step's 64 columns meet at most four adapters (2 VW >= 16): dd0 .. dd0 + 3.  Their
        // ids are read with scalar loads (constant address space), which wait on the scalar
        // counter only: a vector load here would also wait for every copy in flight.
        const int dd0 = __builtin_amdgcn_readfirstlane(kk0 / (2 * VW));
        const __attribute__((address_space(4))) int *cl =
            (const __attribute__((address_space(4))) int *)slist;
        const int a0 = cl[min(dd0, D - 1)];
        const int a1 = cl[min(dd0 + 1, D - 1)];
        const int a2 = cl[min(dd0 + 2, D - 1)];
        const int a3 = cl[min(dd0 + 3, D - 1)];
        const int e = dd - dd0;
        const int a = e == 0 ? a0 : e == 1 ? a1 : e == 2 ? a2 : a3;
        const int s_lo = P.g.slice_start[sg], s_hi = P.g.slice_start[sg + 1];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int row = (wave * 4 + b) * 8 + rr;
            if constexpr (PW) {
                // fragment layout: this lane holds row f/2*16 + lane%16, chunk (f%2)*4 + lane/16
                const int f = wave * 4 + b;
                const int bn = n0 + (f >> 1) * 16 + (lane & 15);
                const int bkk = kk0 + ((f & 1) * 4 + (lane >> 4)) * 8;
                const int bdd = bkk / (2 * VW);
                const int brho = (bkk - bdd * 2 * VW) & (VW - 1);
                const int be = bdd - dd0;
                const int ba = be == 0 ? a0 : be == 1 ? a1 : be == 2 ? a2 : a3;
                const bool bok = bdd < D && bn >= s_lo && bn < s_hi;
                const uint16_t *gb = P.g.B + ((int64_t)ba * P.n_out + min(bn, P.n_out - 1)) * R + brho;
                pf_dma(bok ? (const void *)gb : (const void *)pf_zero16, sw + f * 512);
            } else {
                const int n = n0 + row;
                const bool ok = dd < D && n >= s_lo && n < s_hi;   // s_hi <= n_out
                const uint16_t *gb = P.g.B + ((int64_t)a * P.n_out + min(n, P.n_out - 1)) * R + rho;
                pf_dma(ok ? (const void *)gb : (const void *)pf_zero16, sw + (wave * 4 + b) * 8 * PF_KS);
            }
            const uint16_t *gv = vtile + (int64_t)row * (P.g.n_slices * kxs) + sg * kxs + kk;
            // columns past the tile's adapters (up to the step's end) are not written: zeros
            pf_dma(kk < D * 2 * VW ? (const void *)gv : (const void *)pf_zero16,
                   sx + (wave * 4 + b) * 8 * PF_KS);
        }
    }
}

// MFMAs of one stage (two k-steps of 32): wave (wn, wm) owns W rows wn*64 .. +64 and tokens
// wm*128 .. +128.  The operand reads run one group ahead of the MFMAs (a group: one k-step's two
// 16-token fragments against the four W fragments), so a wave never waits for the LDS right
// after issuing its reads; each accumulator still takes k-step 0, then 1.
template <bool PW>
__device__ __forceinline__ bf16x8 pf_rd_a(const uint16_t *st, int wn, int r, int gq, int ks, int i)
{
    const uint16_t *sw = st;
    const int pos = (ks * 4 + gq) ^ (r & 7);
    if constexpr (PW)
        return *(const bf16x8 *)(sw + (((wn * 4 + i) * 2 + ks) * 64 + gq * 16 + r) * 8);
    else
        return *(const bf16x8 *)(sw + ((wn * 64 + i * 16 + r) * 8 + pos) * 8);
}

__device__ __forceinline__ bf16x8 pf_rd_b(const uint16_t *st, int wm, int r, int gq, int ks, int j)
{
    const uint16_t *sx = st + 256 * PF_KS;
    const int pos = (ks * 4 + gq) ^ (r & 7);
    return *(const bf16x8 *)(sx + ((wm * 128 + j * 16 + r) * 8 + pos) * 8);
}

// The first MFMA group's operands of a stage (k-step 0: the four W fragments and token
// fragments 0, 1), read as soon as the stage is published, ahead of the copy issue.
template <bool PW>
__device__ __forceinline__ void pf_prefetch(const uint16_t *st, int wn, int wm, int r, int gq,
                                            bf16x8 (&a0)[4], bf16x8 (&b0)[2])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a0[i] = pf_rd_a<PW>(st, wn, r, gq, 0, i);
    b0[0] = pf_rd_b(st, wm, r, gq, 0, 0);
    b0[1] = pf_rd_b(st, wm, r, gq, 0, 1);
}

// MFMAs of one stage (two k-steps of 32): wave (wn, wm) owns W rows wn*64 .. +64 and tokens
// wm*128 .. +128.  The operand reads run one group ahead of the MFMAs (a group: one k-step's two
// 16-token fragments against the four W fragments; the first group's come from pf_prefetch), so
// a wave never waits for the LDS right after issuing its reads; each accumulator still takes
// k-step 0, then 1.
template <bool PW>
__device__ __forceinline__ void pf_compute(const uint16_t *st, int wn, int wm, int r, int gq,
                                           const bf16x8 (&a0)[4], const bf16x8 (&b0)[2],
                                           f32x4 (&acc)[4][8])
{
    bf16x8 af[2][4], bv[2][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        af[0][i] = a0[i];
    bv[0][0] = b0[0];
    bv[0][1] = b0[1];
#pragma unroll
    for (int g = 0; g < 8; ++g) {              // group g: k-step g / 4, fragments 2 (g % 4) + 0, 1
        const int ks = g >> 2, jp = g & 3, cur = g & 1;
        if (g + 1 < 8) {
            const int nks = (g + 1) >> 2, njp = (g + 1) & 3;
            if (njp == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    af[nks][i] = pf_rd_a<PW>(st, wn, r, gq, nks, i);
            }
            bv[cur ^ 1][0] = pf_rd_b(st, wm, r, gq, nks, 2 * njp);
            bv[cur ^ 1][1] = pf_rd_b(st, wm, r, gq, nks, 2 * njp + 1);
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i][2 * jp + jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    af[ks][i], bv[cur][jj], acc[i][2 * jp + jj], 0, 0, 0);
    }
    // keep that order in the schedule: for every group the next group's reads (2, or 6 where
    // the next k-step's W fragments start) before its 8 MFMAs
#define PF_SG(ds) __builtin_amdgcn_sched_group_barrier(0x100, ds, 0); \
                  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    PF_SG(2) PF_SG(2) PF_SG(2) PF_SG(6) PF_SG(2) PF_SG(2) PF_SG(2)
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
#undef PF_SG
}

template <bool PW>
__global__ __launch_bounds__(512) void prefill_gemm_kernel(GemmArgs P)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t pf_lds[];
    // [stage][W 256 x 32 | X 256 x 32], then the tile's adapter list
    const int nwg = P.n_mtiles * P.n_ntiles;
    if ((int)blockIdx.x >= nwg) {
        pf_group_helper(P, nwg, pf_lds);
        return;
    }

    // Workgroups are dealt to the 8 XCDs round robin (their own L2 each): give every XCD a
    // contiguous run of logical tiles, ordered in groups of 8 n-tiles per m-tile, so the
    // tiles an XCD runs together share their x and W panels in its L2.  Any bijection is
    // correct; this one only decides which tiles meet in which cache.
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int lt = xcd * (nwg >> 3) + min(xcd, nwg & 7) + slot;
    const int GN = 8;
    const int per_group = GN * P.n_mtiles;
    const int grp = lt / per_group;
    const int rem = lt - grp * per_group;
    const int gn = min(GN, P.n_ntiles - grp * GN);
    const int mt = rem / gn;
    const int nt = grp * GN + (rem - mt * gn);
    const int m0 = mt * PF_BM, n0 = nt * PF_BN;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wn = wave & 3, wm = wave >> 2;
    const int r = lane & 15, gq = lane >> 4;

    const int nk_main = (P.n_in + PF_KS - 1) / PF_KS;
    int D = 0, kxs = 0, VW = 8, sg_lo = 0, sg_hi = -1, kb_per_slice = 1;
    // a scattered tile gets no extra k-steps: its fp32 sums go to part_sc for the expand kernel
    const int ord = P.lora ? P.tile_ord[mt] : -1;
    if (P.lora && ord < 0) {
        D = P.tile_D[mt];
        VW = P.tile_w[mt];
        kxs = ((D * 2 * VW + PF_BK - 1) / PF_BK) * PF_BK;
        if (D > 0) {
            kb_per_slice = kxs / PF_KS;
            const int nlast = min(n0 + PF_BN, P.n_out) - 1;
            while (sg_lo + 1 < P.g.n_slices && n0 >= P.g.slice_start[sg_lo + 1])
                ++sg_lo;
            sg_hi = sg_lo;
            while (sg_hi + 1 < P.g.n_slices && nlast >= P.g.slice_start[sg_hi + 1])
                ++sg_hi;
        }
    }
    const int nk_extra = D > 0 ? (sg_hi - sg_lo + 1) * kb_per_slice : 0;
    const int nk = nk_main + nk_extra;
    const uint16_t *vtile = P.vcat + (int64_t)mt * P.vcat_tile_elems;
    const int *slist = P.tile_list + (int64_t)mt * P.list_stride;

    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // the second prologue stage repeats the first when there is only one (never read), so the
    // count of the first wait below stays exact
#pragma unroll
    for (int q = 0; q < PF_STAGES; ++q)
        pf_issue<PW>(P, pf_lds + q * (PF_STAGE_BYTES / 2), min(q, nk - 1), nk_main, nk_extra, m0, n0,
                 vtile, D, kxs, VW, sg_lo, kb_per_slice, slist, wave, lane);
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");    // stage 0 (8 copies per stage)
    lds_barrier();
    bf16x8 a0[4], b0[2];
    pf_prefetch<PW>(pf_lds, wn, wm, r, gq, a0, b0);
    // two loops: while the stage after next is a base stage the copies need no adapter ids
    // (no scalar loads in the loop, so the LDS waits can count exactly); then the rest
    int q = 0;
    for (; q + PF_STAGES < nk_main; ++q) {
        uint16_t *st = pf_lds + (q & 1) * (PF_STAGE_BYTES / 2);
        pf_compute<PW>(st, wn, wm, r, gq, a0, b0, acc);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // stage q+1
        lds_barrier();                                      // also: stage q fully read
        // stage q+1's first operands, then the copies into the buffer stage q used
        pf_prefetch<PW>(pf_lds + ((q + 1) & 1) * (PF_STAGE_BYTES / 2), wn, wm, r, gq, a0, b0);
        pf_issue<PW, true>(P, st, q + PF_STAGES, nk_main, nk_extra, m0, n0, vtile, D, kxs, VW,
                           sg_lo, kb_per_slice, slist, wave, lane);
    }
    for (; q < nk; ++q) {
        uint16_t *st = pf_lds + (q & 1) * (PF_STAGE_BYTES / 2);
        pf_compute<PW>(st, wn, wm, r, gq, a0, b0, acc);
        if (q + 1 == nk)
            break;                                          // nothing left to publish or copy
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // stage q+1
        lds_barrier();
        pf_prefetch<PW>(pf_lds + ((q + 1) & 1) * (PF_STAGE_BYTES / 2), wn, wm, r, gq, a0, b0);
        // copies only for stages that exist: the waits in this loop are vmcnt(0), so the
        // number in flight need not be the same every iteration, and the tile's stores no
        // longer wait behind copies of a stage nobody reads
        if (q + PF_STAGES < nk)
            pf_issue<PW>(P, st, q + PF_STAGES, nk_main, nk_extra, m0, n0, vtile, D, kxs, VW,
                         sg_lo, kb_per_slice, slist, wave, lane);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");       // no copy outlives the workgroup

    // lane holds rows n0 + wn*64 + i*16 + 4*gq + (0..3) of token m0 + wm*128 + j*16 + r
    if (ord >= 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int tl = wm * 128 + j * 16 + r;
            if (m0 + tl >= P.T)
                continue;
            float *po = P.part_sc + ((int64_t)ord * PF_BM + tl) * P.n_out;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = n0 + wn * 64 + i * 16 + gq * 4;
                if (n + 3 < P.n_out && (P.n_out & 3) == 0) {
                    *(float4 *)(po + n) = float4{acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                } else {
                    for (int e = 0; e < 4; ++e)
                        if (n + e < P.n_out)
                            po[n + e] = acc[i][j][e];
                }
            }
        }
        // and the bf16 base product below, which stays the output of tokens with no adapter
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int t = m0 + wm * 128 + j * 16 + r;
        if (t >= P.T)
            continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = n0 + wn * 64 + i * 16 + gq * 4;
            uint16_t *yo = P.y + (int64_t)t * P.n_out + n;
            if (n + 3 < P.n_out && (P.n_out & 3) == 0) {
                const uint32_t lo = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
                const uint32_t hi = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
                *(u32x2 *)yo = u32x2{lo, hi};
            } else {
                for (int e = 0; e < 4; ++e)
                    if (n + e < P.n_out)
                        yo[e] = f32_to_bf16(acc[i][j][e]);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// 4. expand of the scattered tiles, per adapter
// ------------------------------------------------------------------------------------------
// Item = (scattered tile, token group of one adapter, 256-row chunk of the output): B[a]'s rows
// are the MFMA's A operand, the gathered tokens' V columns (hi and lo halves, one MFMA each) the
// B operand; 4 waves of 64 rows, 16 tokens.  Pass p (one launch each, p < K) adds, for every
// token, the adapter that is its p-th distinct one in ascending id order: the token's last
// adapter writes y = bf16(sum), an earlier one writes the fp32 sum back for the next pass, so
// every output is summed in one fixed order.  Tokens with no adapter keep the bf16 base product
// the GEMM wrote for them.
struct ScArgs {
    int T, n_out, K, pass;
    SlotGeom g;
    const int32_t *idx;
    const int32_t *tile_D, *tile_list;
    const int32_t *tile_w;
    int list_stride;
    const int4 *tile_grp;     // group records, 2 x int4 each (tile plan)
    int grp_stride;
    const uint16_t *vcat;
    int64_t vcat_tile_elems;
    const int32_t *sc_tiles;  // [sc_cap] tile of each scattered ordinal, then their count
    const int32_t *sc_pre;    // [sc_cap] first item of each ordinal, then the item total
    int sc_cap, n_chunks;
    float *part_sc;
    uint16_t *y;
};

constexpr int SC_ROWS = 256;   // output rows of an expand item

__device__ __forceinline__ int sc_slice(const SlotGeom &g, int n)
{
    int sg = 0;
    while (sg + 1 < g.n_slices && n >= g.slice_start[sg + 1])
        ++sg;
    return sg;
}

// The group record of an item: (tile m, group local / n_chunks).
__device__ __forceinline__ const int4 *sc_record(const ScArgs &P, int m, int local)
{
    return P.tile_grp + ((int64_t)m * P.grp_stride + local / P.n_chunks) * 2;
}

// gr, gt: the item's group record (loaded by the caller, ahead of the item)
__device__ __forceinline__ void sc_expand_item(const ScArgs &P, int ord, int m, int local,
                                               const int4 gr, const int4 gt)
{
    const SlotGeom &g = P.g;
    const int R = g.R;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, gq = lane >> 4;
    const int gidx = local / P.n_chunks, nc = local - gidx * P.n_chunks;
    const int n0 = nc * SC_ROWS + wave * 64;
    if (n0 >= P.n_out)
        return;
    // {d, adapter, V columns per slice, tokens | rank rounded to 8 << 8 | log2 VW << 20},
    // then the token bytes
    const int d = gr.x, a = gr.y, ng = gr.w & 0xff;
    const bool tok_ok = r < ng;
    const int tl = tok_ok ? grp_token(gt, r) : 0;
    const int t = m * PF_BM + tl;

    // this pass's adapter of the token: its rank among the token's distinct ids, and their
    // count (one slot per token: the group's adapter is the token's only one)
    int below = 0, n_dist = 1;
    if (tok_ok && P.K > 1) {
        n_dist = 0;
        const int32_t *it = P.idx + (int64_t)t * P.K;
        for (int j = 0; j < P.K; ++j) {
            const int b = it[j];
            bool dup = b < 0;
            for (int jj = 0; jj < j; ++jj)
                dup |= it[jj] == b;
            if (!dup) {
                ++n_dist;
                below += b < a ? 1 : 0;
            }
        }
    }
    const bool act = tok_ok && below == P.pass;
    const bool last = below == n_dist - 1;
    const int rk = (gr.w >> 8) & 0xfff;
    const int VW = 1 << (gr.w >> 20), kxs = gr.z;
    const uint16_t *vrow = P.vcat + (int64_t)m * P.vcat_tile_elems + (int64_t)tl * (g.n_slices * kxs) +
                           d * 2 * VW + gq * 8;
    const uint16_t *brow0 = g.B + (int64_t)a * P.n_out * R + gq * 8;
    float *po = P.part_sc + ((int64_t)ord * PF_BM + tl) * P.n_out;

    // the fp32 sums of this lane's outputs, loaded first
    f32x4 acc[4], prt[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int n = n0 + f * 16 + gq * 4;
        acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (n + 3 < P.n_out && (P.n_out & 3) == 0) {
            const float4 v = *(const float4 *)(act ? (const void *)(po + n) : (const void *)pf_zero16);
            prt[f] = f32x4{v.x, v.y, v.z, v.w};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                prt[f][e] = act && n + e < P.n_out ? po[n + e] : 0.f;
        }
    }
    // B rows of the 4 row groups (lane row nb[f]) and their slices; a batch of 64 columns
    // issues the V halves and all 4 groups' B fragments together, then its MFMAs.  Per group
    // the sums run over (slice, column) in ascending order; a group outside the slice, rows
    // past n_out and columns past the rank multiply zeros (B columns past the rank are zero).
    int nb[4], sgb[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        nb[f] = n0 + f * 16 + r;
        sgb[f] = nb[f] < P.n_out ? sc_slice(g, nb[f]) : -1;
    }
    const int sg_lo = sc_slice(g, n0), sg_hi = sc_slice(g, min(n0 + 63, P.n_out - 1));
    for (int sg = sg_lo; sg <= sg_hi; ++sg) {
        for (int k0 = 0; k0 < rk; k0 += 64) {
            u32x4 vh[2], vl[2], bv[4][2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = k0 + h * 32;
                const bool kok = k + gq * 8 < rk;
                const uint16_t *vp = vrow + sg * kxs + k;
                vh[h] = *(const u32x4 *)(tok_ok && kok ? (const void *)vp : (const void *)pf_zero16);
                vl[h] = *(const u32x4 *)(tok_ok && kok ? (const void *)(vp + VW) : (const void *)pf_zero16);
#pragma unroll
                for (int f = 0; f < 4; ++f)
                    bv[f][h] = *(const u32x4 *)(sgb[f] == sg && kok
                                                    ? (const void *)(brow0 + (int64_t)nb[f] * R + k)
                                                    : (const void *)pf_zero16);
            }
            // all 12 loads in flight before the first MFMA (left alone, the compiler moves
            // each load down to its MFMA)
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, bv[f][h]), __builtin_bit_cast(bf16x8, vh[h]),
                        acc[f], 0, 0, 0);
                    acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, bv[f][h]), __builtin_bit_cast(bf16x8, vl[h]),
                        acc[f], 0, 0, 0);
                }
        }
    }
    if (!act)
        return;
    // lane holds rows n0 + 16f + 4gq + e of token t
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int n = n0 + f * 16 + gq * 4;
        if (n >= P.n_out)
            break;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = prt[f][e] + acc[f][e];
        if (n + 3 < P.n_out && (P.n_out & 3) == 0) {
            if (last)
                *(u32x2 *)(P.y + (int64_t)t * P.n_out + n) =
                    u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            else
                *(float4 *)(po + n) = float4{o[0], o[1], o[2], o[3]};
        } else {
            for (int e = 0; e < 4; ++e) {
                if (n + e >= P.n_out)
                    break;
                if (last)
                    P.y[(int64_t)t * P.n_out + n + e] = f32_to_bf16(o[e]);
                else
                    po[n + e] = o[e];
            }
        }
    }
}

__global__ __launch_bounds__(256) void sc_expand_kernel(ScArgs P)
{
    // the scattered tiles and their first items (numbered by sgmv_shrink_kernel), in LDS
    extern __shared__ int sc_pre[];           // [sc_cap] item prefix, then [sc_cap] tiles
    int *sc_m = sc_pre + P.sc_cap;
    // the tables are read whole (sc_cap entries; those past the scattered tiles' count are
    // never used), in the same round trip as the counts
    const int n_sc = P.sc_tiles[P.sc_cap];
    const int total = P.sc_pre[P.sc_cap];
    for (int o = threadIdx.x; o < P.sc_cap; o += 256) {
        sc_pre[o] = P.sc_pre[o];
        sc_m[o] = P.sc_tiles[o];
    }
    __syncthreads();
    // scattered tile of an item: last o with sc_pre[o] <= item
    auto find = [&](int item) {
        int lo = 0, hi = n_sc - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sc_pre[mid] <= item)
                lo = mid;
            else
                hi = mid - 1;
        }
        return lo;
    };
    // each item's group record is loaded one item ahead, so that an item's first dependent
    // round trip overlaps the previous item
    int item = blockIdx.x;
    if (item >= total)
        return;
    int o = find(item);
    const int4 *rec = sc_record(P, sc_m[o], item - sc_pre[o]);
    int4 gr = rec[0], gt = rec[1];
    while (true) {
        const int next = item + gridDim.x;
        int on = 0;
        int4 grn = gr, gtn = gt;
        if (next < total) {
            on = find(next);
            const int4 *rn = sc_record(P, sc_m[on], next - sc_pre[on]);
            grn = rn[0];
            gtn = rn[1];
        }
        sc_expand_item(P, o, sc_m[o], item - sc_pre[o], gr, gt);
        if (next >= total)
            break;
        item = next;
        o = on;
        gr = grn;
        gt = gtn;
    }
}

// ------------------------------------------------------------------------------------------
PrefillCfg prefill_config(int64_t T, int32_t K, int64_t n_in, int64_t n_out, int32_t S, int32_t R,
                          int32_t n_slices)
{
    PrefillCfg c;
    c.n_mtiles = (int)((T + PF_BM - 1) / PF_BM);
    c.n_ntiles = (int)((n_out + PF_BN - 1) / PF_BN);
    c.list_stride = (int)std::min<int64_t>((int64_t)PF_BM * K, S);
    const int64_t kxs_max = ((int64_t)c.list_stride * 2 * R + PF_BK - 1) / PF_BK * PF_BK;
    c.vcat_tile_elems = (int64_t)PF_BM * n_slices * kxs_max;
    // fp32 sums of up to sc_cap scattered tiles, within 64 MiB (at least one tile)
    c.n_out = n_out;
    c.tok_stride = PF_BM * K;
    c.grp_stride = PF_BM * K / 16 + c.list_stride;   // 16-token groups of a scattered tile
    c.sc_cap = (int)std::min<int64_t>(
        c.n_mtiles, std::max<int64_t>(1, (64ll << 20) / ((int64_t)PF_BM * n_out * 4)));
    // a tile holds at most list_stride adapters: when even that many stay within the
    // scattered-tile limit (tile_scattered), no tile is scattered and the expand launches
    // after the GEMM would find no work
    c.may_scatter = (int64_t)c.list_stride * 2 * R > n_in / 2;
    // fp32 partial blocks of the dense shrink items: within 64 MiB, and no more than the most
    // the launch can use (every tile dense with list_stride adapters, SD_KS_MAX parts)
    const int64_t rbs_max = ((int64_t)c.list_stride * n_slices * R + SD_ROWS - 1) / SD_ROWS;
    c.sd_cap_slots = (int)std::min<int64_t>(
        (64ll << 20) / ((int64_t)SD_PART_ELEMS * 4), (int64_t)c.n_mtiles * rbs_max * SD_KS_MAX);
    return c;
}

// Workspace regions of the tiled path, each 256-byte aligned, in this order.
struct PrefillLayout {
    size_t tile_w, tile_D, tile_list, tile_toff, tile_gpre, sc_pre, tile_ord, sc_tiles, part_sc, vcat,
        tile_pbase, sd_ks, sd_part, tile_grp, total;
};

static size_t al256(size_t v) { return (v + 255) / 256 * 256; }

static PrefillLayout prefill_layout(const PrefillCfg &c)
{
    PrefillLayout L;
    const size_t lists = al256((size_t)c.n_mtiles * c.list_stride * sizeof(int32_t));
    const size_t offs = al256((size_t)c.n_mtiles * (c.list_stride + 1) * sizeof(int32_t));
    L.tile_w = 0;
    L.tile_D = L.tile_w + al256((size_t)c.n_mtiles * sizeof(int32_t));
    L.tile_list = L.tile_D + al256((size_t)c.n_mtiles * sizeof(int32_t));
    L.tile_toff = L.tile_list + lists;
    L.tile_gpre = L.tile_toff + offs;
    L.sc_pre = L.tile_gpre + offs;
    L.tile_ord = L.sc_pre + al256(((size_t)c.sc_cap + 1) * sizeof(int32_t));
    L.sc_tiles = L.tile_ord + al256((size_t)c.n_mtiles * sizeof(int32_t));
    L.part_sc = L.sc_tiles + al256(((size_t)c.sc_cap + 1) * sizeof(int32_t));
    L.vcat = L.part_sc + al256((size_t)c.sc_cap * PF_BM * (size_t)c.n_out * sizeof(float));
    L.tile_pbase = L.vcat + al256((size_t)c.n_mtiles * c.vcat_tile_elems * sizeof(uint16_t));
    L.sd_ks = L.tile_pbase + al256((size_t)c.n_mtiles * sizeof(int32_t));
    L.sd_part = L.sd_ks + 256;
    L.tile_grp = L.sd_part + al256((size_t)c.sd_cap_slots * SD_PART_ELEMS * sizeof(float));
    L.total = L.tile_grp + (size_t)c.n_mtiles * c.grp_stride * 2 * sizeof(int4);
    return L;
}

size_t prefill_workspace_bytes(const PrefillCfg &c) { return prefill_layout(c).total; }

// Grouping pays where the per-(token, slot) reads of the decode kernels (each pair's A rows
// and B columns, padded slot width) would dwarf the base weight and take long in themselves:
// at least 128 tokens, that gather above four times W's bytes and above 200 MB.  Below it the
// group kernels (five launches, items of a few tokens bound by their latency) lose to the
// gather: measured at 256 tokens, rank 16 at 4096 -> 512 (38 MB of gather) 17.8 against 45.1
// us, rank 32 at 4096 -> 4096 (134 MB) 51.6 against 62.3 us; with 268 MB or more the grouped
// decode won (rank 64 at 4096 -> 4096: 64.7 against 79.9 us; at 512 tokens 94.6 against 152.9).
bool grouped_decode_worth_it(int64_t T, int32_t K, int64_t n_in, int64_t n_out, int32_t wd,
                             int32_t R)
{
    const double gather = (double)T * K * ((double)wd * n_in + (double)n_out * R);
    return T >= 128 && gather > 4.0 * (double)n_out * n_in && 2.0 * gather >= 200.0e6;
}

bool prefill_worth_it(int64_t T, int64_t n_in, int64_t n_out, int32_t K, int32_t wd)
{
    // Estimated times of the two paths (us), fitted to their rates measured on MI355X (64 to
    // 4096 tokens; 4096 -> 512, 1024, 4096 and 11008, 512 and 11008 -> 4096):
    //  decode: launches of up to 512 tokens; each takes about 10 us, 6 us per round of its
    //    (64-token chunk, 64-row tile, split) items over the CUs, 10 us more where the shrink
    //    runs apart, and the split partials written and read (8 bytes per split, token and
    //    output at about 6 TB/s);
    //  tiled: 25 us for the plan, shrink and expand kernels, and per round of 256 x 256 output
    //    tiles over the CUs about 45 us plus 85 us per 4096 columns of n_in, times 1.15 for
    //    batches whose adapters spread over many tiles (the index map is not read here; tiles
    //    of random maps took 1.1 to 1.6 times those of contiguous ones; 1.8 when a tile's fp32
    //    sums exceed the 64 MiB kept for the per-adapter expand, so that such tiles take the
    //    extra k-steps of all their adapters).
    // wd: rows of a slot (n_slices R), 0 for the base alone.
    const int64_t n_cus = device_cu_count();
    double dec = 0.0;
    for (int64_t t0 = 0; t0 < T; t0 += 512) {
        const int64_t Tc = std::min<int64_t>(512, T - t0);
        const DecodeCfg c = decode_config(Tc, n_in, n_out);
        const int64_t items = (Tc + 63) / 64 * c.n_tiles * c.sk;
        const bool apart = wd > 0 && decode_shrink_apart(Tc, K, n_out, wd);
        dec += 10.0 + 6.0 * (double)((items + n_cus - 1) / n_cus) + (apart ? 10.0 : 0.0) +
               8.0 * (double)c.sk * (double)Tc * (double)n_out / 6.0e6;
    }
    const int64_t tiles = ((T + PF_BM - 1) / PF_BM) * ((n_out + PF_BN - 1) / PF_BN);
    const double spread = (int64_t)PF_BM * n_out * 4 > (64ll << 20) ? 1.8 : 1.15;
    const double til = 25.0 + spread * (double)((tiles + n_cus - 1) / n_cus) *
                                  (45.0 + 85.0 * (double)n_in / 4096.0);
    return til < dec;
}

// The tiled path's workspace regions of one call.
struct PrefillPtrs {
    int32_t *tile_D, *tile_w, *tile_list, *tile_toff, *tile_gpre, *sc_pre, *tile_ord, *sc_tiles;
    float *part_sc;
    uint16_t *vcat;
    int32_t *tile_pbase, *sd_ks;
    float *sd_part;
    int4 *tile_grp;
};

static PrefillPtrs prefill_ptrs(const PrefillCfg &c, void *ws)
{
    uint8_t *p = (uint8_t *)ws;
    const PrefillLayout WL = prefill_layout(c);
    PrefillPtrs q;
    q.tile_D = (int32_t *)(p + WL.tile_D);
    q.tile_w = (int32_t *)(p + WL.tile_w);
    q.tile_list = (int32_t *)(p + WL.tile_list);
    q.tile_toff = (int32_t *)(p + WL.tile_toff);
    q.tile_gpre = (int32_t *)(p + WL.tile_gpre);
    q.sc_pre = (int32_t *)(p + WL.sc_pre);
    q.tile_ord = (int32_t *)(p + WL.tile_ord);
    q.sc_tiles = (int32_t *)(p + WL.sc_tiles);
    q.part_sc = (float *)(p + WL.part_sc);
    q.vcat = (uint16_t *)(p + WL.vcat);
    q.tile_pbase = (int32_t *)(p + WL.tile_pbase);
    q.sd_ks = (int32_t *)(p + WL.sd_ks);
    q.sd_part = (float *)(p + WL.sd_part);
    q.tile_grp = (int4 *)(p + WL.tile_grp);
    return q;
}

// Tile plan, then the shrink kernels into the tiles' V blocks.  skip_groups: the GEMM's helper
// workgroups take the scattered tiles' group items; force_scatter: every tile is scattered.
static hipError_t plan_and_shrink(const uint16_t *x, int64_t T, int64_t n_in, int64_t n_out,
                                  const SlotGeom &g, const int32_t *idx, int32_t K,
                                  const float *scale, const PrefillCfg &c, const PrefillPtrs &q,
                                  int skip_groups, int force_scatter, hipStream_t stream,
                                  ShrinkArgs &s)
{
    if (c.n_mtiles > SH_MAX_TILES)
        return hipErrorInvalidValue;   // callers split larger batches
    const size_t lds = (size_t)((g.S + 31) / 32) * 4 + (size_t)g.S * 8 +
                       (size_t)c.list_stride * 4 + (size_t)c.tok_stride;
    if (hipError_t e = ensure_dynamic_lds((const void *)tile_plan_kernel, lds); e != hipSuccess)
        return e;
    hipLaunchKernelGGL(tile_plan_kernel, dim3(c.n_mtiles), dim3(256), lds, stream, idx, (int)T,
                       K, g.S, g.R, g.n_slices, (int)n_in, g.rank, c.list_stride, q.tile_D,
                       q.tile_w, q.tile_list, q.tile_toff, q.tile_gpre, q.tile_grp, c.grp_stride,
                       force_scatter);
    s = ShrinkArgs{};
    s.x = x;
    s.T = (int)T;
    s.n_in = (int)n_in;
    s.K = K;
    s.g = g;
    s.idx = idx;
    s.scale = scale;
    s.n_mtiles = c.n_mtiles;
    s.list_stride = c.list_stride;
    s.tile_D = q.tile_D;
    s.tile_w = q.tile_w;
    s.tile_list = q.tile_list;
    s.vcat = q.vcat;
    s.vcat_tile_elems = c.vcat_tile_elems;
    s.tile_ord = q.tile_ord;
    s.sc_tiles = q.sc_tiles;
    s.sc_cap = c.sc_cap;
    s.tile_toff = q.tile_toff;
    s.tile_gpre = q.tile_gpre;
    s.sc_pre = q.sc_pre;
    s.n_chunks = (int)((n_out + SC_ROWS - 1) / SC_ROWS);
    s.tile_grp = q.tile_grp;
    s.grp_stride = c.grp_stride;
    s.sd_part = q.sd_part;
    s.sd_cap_slots = c.sd_cap_slots;
    s.tile_pbase = q.tile_pbase;
    s.sd_ks = q.sd_ks;
    s.skip_groups = skip_groups;
    s.force_scatter = force_scatter;
    const size_t tables = (size_t)c.n_mtiles * SD_TABLE_BYTES;
    if (force_scatter) {
        // group items only: 8 KB of reduction space and the tables; up to two workgroups per CU
        // (the items are bound by their latency), fewer when there are fewer items
        const void *kf = (const void *)sgmv_shrink_kernel<true>;
        const size_t sh_lds = (size_t)SG_RED_BYTES + tables;
        if (sh_lds + kernel_static_lds(kf) > LDS_BYTES)
            return hipErrorInvalidValue;
        if (hipError_t e = ensure_dynamic_lds(kf, sh_lds); e != hipSuccess)
            return e;
        const int wd = g.n_slices * g.R;
        const int64_t items = (int64_t)c.n_mtiles * c.grp_stride * ((wd + SG_ROWS - 1) / SG_ROWS);
        const unsigned grid = (unsigned)std::max<int64_t>(
            1, std::min<int64_t>(items, 2 * (int64_t)device_cu_count()));
        hipLaunchKernelGGL(sgmv_shrink_kernel<true>, dim3(grid), dim3(SH_THREADS), sh_lds, stream,
                           s);
        return hipGetLastError();
    }
    // three dense stages while the item tables and the kernel's own __shared__ arrays leave
    // room in the 160 KB of LDS, else two
    const void *kf = (const void *)sgmv_shrink_kernel<false>;
    const size_t st_lds = kernel_static_lds(kf);
    s.stages = 3 * (size_t)SD_STAGE_BYTES + tables + st_lds <= LDS_BYTES ? 3 : 2;
    const size_t sh_lds = (size_t)s.stages * SD_STAGE_BYTES + tables;
    if (sh_lds + st_lds > LDS_BYTES)
        return hipErrorInvalidValue;   // more tiles than SH_MAX_TILES allows
    if (hipError_t e = ensure_dynamic_lds(kf, sh_lds); e != hipSuccess)
        return e;
    // one workgroup per CU (the stages take most of its LDS), items shared out in the kernel:
    // every workgroup then runs the kernel's item numbering once, all in one round
    hipLaunchKernelGGL(sgmv_shrink_kernel<false>, dim3((unsigned)device_cu_count()),
                       dim3(SH_THREADS), sh_lds, stream, s);
    hipLaunchKernelGGL(shrink_reduce_kernel, dim3((unsigned)c.n_mtiles * (PF_BM / SR_TOK)),
                       dim3(256), 0, stream, s);
    return hipGetLastError();
}

// The scattered tiles' LoRA delta per adapter group, added to their fp32 sums and rounded
// into y, one launch per slot rank (K).
static hipError_t expand_scattered(int64_t T, int64_t n_out, const SlotGeom &g,
                                   const int32_t *idx, int32_t K, uint16_t *y,
                                   const PrefillCfg &c, const PrefillPtrs &q, hipStream_t stream)
{
    ScArgs x2{};
    x2.T = (int)T;
    x2.n_out = (int)n_out;
    x2.K = K;
    x2.g = g;
    x2.idx = idx;
    x2.tile_D = q.tile_D;
    x2.tile_w = q.tile_w;
    x2.tile_list = q.tile_list;
    x2.list_stride = c.list_stride;
    x2.sc_pre = q.sc_pre;
    x2.tile_grp = q.tile_grp;
    x2.grp_stride = c.grp_stride;
    x2.vcat = q.vcat;
    x2.vcat_tile_elems = c.vcat_tile_elems;
    x2.sc_tiles = q.sc_tiles;
    x2.sc_cap = c.sc_cap;
    x2.n_chunks = (int)((n_out + SC_ROWS - 1) / SC_ROWS);
    x2.part_sc = q.part_sc;
    x2.y = y;
    const size_t xl = (size_t)2 * c.sc_cap * sizeof(int32_t);
    // items per scattered tile: at most (256 K / 16 + list_stride) groups x n_chunks
    // (a grid of workgroups that all fit at once: one wave of 1024 with a second partial one
    // behind it was 1 us slower at the mixed batch, 21.0 against 19.8 us)
    const int64_t items = (int64_t)c.sc_cap * (PF_BM * K / 16 + c.list_stride) * x2.n_chunks;
    const int64_t resident =
        (int64_t)kernel_resident_blocks((const void *)sc_expand_kernel, 256, xl) * device_cu_count();
    const unsigned grid = (unsigned)std::min<int64_t>(items, resident);
    hipError_t e = hipSuccess;
    for (int pass = 0; pass < K && e == hipSuccess; ++pass) {
        x2.pass = pass;
        hipLaunchKernelGGL(sc_expand_kernel, dim3(grid), dim3(256), xl, stream, x2);
        e = hipGetLastError();
    }
    return e;
}

hipError_t launch_prefill(const uint16_t *x, const uint16_t *W, bool packed, int64_t T,
                          int64_t n_in, int64_t n_out, const SlotGeom *g, const int32_t *idx,
                          int32_t K, const float *scale, uint16_t *y, const PrefillCfg &c,
                          void *ws, hipStream_t stream)
{
    const PrefillPtrs q = prefill_ptrs(c, ws);
    // helper workgroups after the GEMM's tiles take the scattered tiles' shrink group items
    // while the tiles leave CUs idle (one workgroup per CU: 128 KB of LDS each)
    const int n_tiles = c.n_mtiles * c.n_ntiles;
    const int n_cus = device_cu_count();
    const int n_helpers = g != nullptr && c.may_scatter && n_tiles < n_cus ? n_cus - n_tiles : 0;
    ShrinkArgs s{};
    if (g != nullptr) {
        if (hipError_t e = plan_and_shrink(x, T, n_in, n_out, *g, idx, K, scale, c, q,
                                           n_helpers > 0 ? 1 : 0, 0, stream, s);
            e != hipSuccess)
            return e;
    }
    GemmArgs a{};
    a.x = x;
    a.W = W;
    a.y = y;
    a.T = (int)T;
    a.n_in = (int)n_in;
    a.n_out = (int)n_out;
    a.n_mtiles = c.n_mtiles;
    a.n_ntiles = c.n_ntiles;
    a.lora = g != nullptr;
    if (g != nullptr)
        a.g = *g;
    a.vcat = q.vcat;
    a.vcat_tile_elems = c.vcat_tile_elems;
    a.tile_D = q.tile_D;
    a.tile_w = q.tile_w;
    a.tile_list = q.tile_list;
    a.list_stride = c.list_stride;
    a.tile_ord = q.tile_ord;
    a.part_sc = q.part_sc;
    a.n_rg = (int)((n_out + 15) / 16);
    a.n_kb = (int)((n_in + 31) / 32);
    a.sh = s;
    const size_t lds = (size_t)PF_STAGES * PF_STAGE_BYTES;                // 128 KB of stages
    const void *kfn = packed ? (const void *)prefill_gemm_kernel<true>
                             : (const void *)prefill_gemm_kernel<false>;
    if (hipError_t e = ensure_dynamic_lds(kfn, lds); e != hipSuccess)
        return e;
    trace_mark(stream, true);
    if (packed)
        hipLaunchKernelGGL(prefill_gemm_kernel<true>, dim3((unsigned)(n_tiles + n_helpers)),
                           dim3(512), lds, stream, a);
    else
        hipLaunchKernelGGL(prefill_gemm_kernel<false>, dim3((unsigned)(n_tiles + n_helpers)),
                           dim3(512), lds, stream, a);
    hipError_t e = hipGetLastError();
    trace_mark(stream, false);
    if (e == hipSuccess && g != nullptr && c.may_scatter)
        e = expand_scattered(T, n_out, *g, idx, K, y, c, q, stream);
    return e;
}

PrefillCfg grouped_config(int64_t T, int32_t K, int64_t n_in, int64_t n_out, int32_t S, int32_t R,
                          int32_t n_slices)
{
    PrefillCfg c = prefill_config(T, K, n_in, n_out, S, R, n_slices);
    c.sd_cap_slots = 0;   // every tile scattered: no dense item, no partial blocks
    return c;
}

bool grouped_decode_fits(const PrefillCfg &c)
{
    return c.n_mtiles <= c.sc_cap && c.n_mtiles <= SH_MAX_TILES;
}

hipError_t launch_grouped_shrink(const uint16_t *x, int64_t T, int64_t n_in, int64_t n_out,
                                 const SlotGeom &g, const int32_t *idx, int32_t K,
                                 const float *scale, const PrefillCfg &c, void *ws,
                                 hipStream_t stream)
{
    if (!grouped_decode_fits(c))
        return hipErrorInvalidValue;
    ShrinkArgs s;
    return plan_and_shrink(x, T, n_in, n_out, g, idx, K, scale, c, prefill_ptrs(c, ws), 0, 1,
                           stream, s);
}

float *grouped_base_sums(const PrefillCfg &c, void *ws)
{
    return prefill_ptrs(c, ws).part_sc;
}

hipError_t launch_grouped_expand(int64_t T, int64_t n_out, const SlotGeom &g, const int32_t *idx,
                                 int32_t K, uint16_t *y, const PrefillCfg &c, void *ws,
                                 hipStream_t stream)
{
    if (!grouped_decode_fits(c))
        return hipErrorInvalidValue;
    return expand_scattered(T, n_out, g, idx, K, y, c, prefill_ptrs(c, ws), stream);
}

}  // namespace mlora
