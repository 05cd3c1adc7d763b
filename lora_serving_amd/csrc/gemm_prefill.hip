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
//  2. SGMV shrink: for each (tile, adapter) the tokens that use it are gathered, and
//     V[token][col(s, d, rho)] = c_t * sum_i A[a][s][rho][i] x[t][i] runs on the matrix cores,
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
constexpr int PF_BK = 64;    // columns per K-step
constexpr int PF_THREADS = 512;

__device__ __forceinline__ int pf_swz(int row, int c) { return c ^ (row & 7); }

// ------------------------------------------------------------------------------------------
// 1. tile plan
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tile_plan_kernel(const int32_t *__restrict__ idx, int T,
                                                        int K, int S, int R, int n_slices,
                                                        int list_stride, int32_t *tile_D,
                                                        int32_t *tile_list, int32_t *tile_cnt,
                                                        uint16_t *vcat, int64_t vcat_tile_elems)
{
    extern __shared__ uint32_t plan_lds[];         // bits[(S+31)/32] then cnt[S]
    const int nw = (S + 31) / 32;
    uint32_t *bits = plan_lds;
    int *cnt = (int *)(plan_lds + nw);
    const int m = blockIdx.x;
    const int t0 = m * PF_BM;
    const int nt = min(PF_BM, T - t0);
    for (int i = threadIdx.x; i < nw; i += blockDim.x)
        bits[i] = 0u;
    for (int i = threadIdx.x; i < S; i += blockDim.x)
        cnt[i] = 0;
    __syncthreads();
    for (int tl = threadIdx.x; tl < nt; tl += blockDim.x) {
        const int32_t *it = idx + (int64_t)(t0 + tl) * K;
        for (int j = 0; j < K; ++j) {
            const int a = it[j];
            if (a < 0)
                continue;
            bool dup = false;
            for (int jj = 0; jj < j; ++jj)
                dup |= it[jj] == a;
            if (dup)
                continue;
            atomicOr(&bits[a >> 5], 1u << (a & 31));
            atomicAdd(&cnt[a], 1);
        }
    }
    __syncthreads();
    // ascending list of the set bits: exclusive scan of per-word popcounts
    __shared__ int wsum[4];
    int base = 0;
    for (int w0 = 0; w0 < nw; w0 += blockDim.x) {
        const int w = w0 + threadIdx.x;
        const uint32_t b = w < nw ? bits[w] : 0u;
        const int pc = __popc(b);
        int tot;
        const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
        int ex = wave_exclusive_scan(pc, &tot);
        if (lane == 0)
            wsum[wv] = tot;
        __syncthreads();
        int before = 0, all = 0;
        for (int i = 0; i < 4; ++i) {
            if (i < wv)
                before += wsum[i];
            all += wsum[i];
        }
        __syncthreads();
        int pos = base + before + ex;
        uint32_t bb = b;
        while (bb) {
            const int bit = __ffs(bb) - 1;
            bb &= bb - 1;
            const int a = w * 32 + bit;
            tile_list[(int64_t)m * list_stride + pos] = a;
            tile_cnt[(int64_t)m * list_stride + pos] = cnt[a];
            ++pos;
        }
        base += all;
    }
    if (threadIdx.x == 0)
        tile_D[m] = base;
    // zero the padding columns [2*D*R, KXs) of every slice block of this tile's V
    const int D = base;
    const int kxs = ((D * 2 * R + PF_BK - 1) / PF_BK) * PF_BK;
    const int pad = kxs - D * 2 * R;
    if (pad > 0) {
        const int pitch = n_slices * kxs;
        uint16_t *vt = vcat + (int64_t)m * vcat_tile_elems;
        const int per_row = n_slices * pad;
        for (int e = threadIdx.x; e < PF_BM * per_row; e += blockDim.x) {
            const int row = e / per_row;
            const int rem = e - row * per_row;
            const int sg = rem / pad;
            const int c = D * 2 * R + (rem - sg * pad);
            vt[(int64_t)row * pitch + sg * kxs + c] = 0;
        }
    }
}

// ------------------------------------------------------------------------------------------
// 2. SGMV shrink into V
// ------------------------------------------------------------------------------------------
struct ShrinkArgs {
    const uint16_t *x;
    int T, n_in, K;
    SlotGeom g;
    const int32_t *idx;
    const float *scale;
    int n_mtiles, list_stride, n_wb;
    const int32_t *tile_D, *tile_list, *tile_cnt;
    uint16_t *vcat;
    int64_t vcat_tile_elems;
};

// item = (m, d, c, wb): tile m, its d-th adapter, tokens [64c, 64c+64) of that adapter's
// gathered tokens, A rows [64 wb, 64 wb + 64) of the adapter's n_slices*R rows
__global__ __launch_bounds__(256) void sgmv_shrink_kernel(ShrinkArgs P)
{
    __shared__ int s_tok[PF_BM];
    __shared__ float s_coef[PF_BM];
    __shared__ int s_n;
    __shared__ int wsum[4];
    __shared__ __attribute__((aligned(16))) uint16_t sa[64 * 64];   // A rows x 64 columns
    __shared__ __attribute__((aligned(16))) uint16_t sx[64 * 64];   // gathered x rows
    const SlotGeom &g = P.g;
    const int R = g.R;
    const int wd = g.n_slices * R;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n_items = (int64_t)P.n_mtiles * P.list_stride * (PF_BM / 64) * P.n_wb;

    for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
        int64_t rest = item;
        const int wb = (int)(rest % P.n_wb);
        rest /= P.n_wb;
        const int c = (int)(rest % (PF_BM / 64));
        rest /= (PF_BM / 64);
        const int d = (int)(rest % P.list_stride);
        const int m = (int)(rest / P.list_stride);
        const int D = P.tile_D[m];
        if (d >= D)
            continue;
        const int ntok_a = P.tile_cnt[(int64_t)m * P.list_stride + d];
        if (c * 64 >= ntok_a && c > 0)
            continue;
        const int a = P.tile_list[(int64_t)m * P.list_stride + d];
        const int t0 = m * PF_BM;
        const int nt = min(PF_BM, P.T - t0);
        const float fa = g.factor[a];

        // gather the tile's tokens that use a (in token order) and their coefficients
        int use = 0;
        float coef = 0.f;
        const int tl = threadIdx.x;      // PF_BM == blockDim.x
        if (tl < nt) {
            const int32_t *it = P.idx + (int64_t)(t0 + tl) * P.K;
            for (int j = 0; j < P.K; ++j)
                if (it[j] == a) {
                    use = 1;
                    coef += (P.scale ? P.scale[(int64_t)(t0 + tl) * P.K + j] : 1.f) * fa;
                }
        }
        int tot;
        const int ex = wave_exclusive_scan(use, &tot);
        if (lane == 0)
            wsum[wave] = tot;
        __syncthreads();
        int before = 0;
        for (int i = 0; i < wave; ++i)
            before += wsum[i];
        if (threadIdx.x == 0)
            s_n = wsum[0] + wsum[1] + wsum[2] + wsum[3];
        if (use) {
            s_tok[before + ex] = tl;
            s_coef[before + ex] = coef;
        }
        __syncthreads();
        const int n_use = s_n;
        const int kxs = ((D * 2 * R + PF_BK - 1) / PF_BK) * PF_BK;
        const int pitch = g.n_slices * kxs;
        uint16_t *vt = P.vcat + (int64_t)m * P.vcat_tile_elems;
        const int ar0 = wb * 64;                    // first A row of this item
        const int nar = min(64, wd - ar0);

        // chunk 0 also writes the zeros of the tokens (and tile rows) that do not use a
        if (c == 0) {
            const int row = threadIdx.x;   // tile row
            if (!use) {
                for (int q = 0; q < nar; ++q) {
                    const int ar = ar0 + q;
                    const int sg = ar / R;
                    uint16_t *vp = vt + (int64_t)row * pitch + sg * kxs + d * 2 * R + (ar - sg * R);
                    vp[0] = 0;
                    vp[R] = 0;
                }
            }
        }
        const int r0 = c * 64;
        const int nrow = min(64, n_use - r0);
        if (nrow <= 0)
            continue;

        // D[ar][row] = sum_k A[a][ar][k] x[tok_row][k]: wave w owns A rows 16w..16w+15,
        // 4 token tiles of 16
        f32x4 acc[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint16_t *Aa = g.A + ((int64_t)a * wd + ar0) * P.n_in;
        for (int k0 = 0; k0 < P.n_in; k0 += 64) {
            // stage A rows (64 x 64) and gathered x rows (64 x 64): 512 + 512 chunks
            for (int e = threadIdx.x; e < 1024; e += 256) {
                const int isx = e >= 512;
                const int ee = e & 511;
                const int row = ee >> 3, cc = ee & 7;
                const int k = k0 + cc * 8;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (!isx) {
                    if (row < nar && k < P.n_in)
                        v = *(const u32x4 *)(Aa + (int64_t)row * P.n_in + k);
                    *(u32x4 *)(sa + (row * 8 + pf_swz(row, cc)) * 8) = v;
                } else {
                    if (row < nrow && k < P.n_in)
                        v = *(const u32x4 *)(P.x + (int64_t)(t0 + s_tok[r0 + row]) * P.n_in + k);
                    *(u32x4 *)(sx + (row * 8 + pf_swz(row, cc)) * 8) = v;
                }
            }
            __syncthreads();
            const int r = lane & 15, gq = lane >> 4;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int cch = ks * 4 + gq;
                const int arow = wave * 16 + r;
                const bf16x8 av = *(const bf16x8 *)(sa + (arow * 8 + pf_swz(arow, cch)) * 8);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int xrow = q * 16 + r;
                    const bf16x8 bv = *(const bf16x8 *)(sx + (xrow * 8 + pf_swz(xrow, cch)) * 8);
                    acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[q], 0, 0, 0);
                }
            }
            __syncthreads();
        }
        // lane holds A rows 16*wave + 4*(lane/16) + e of token column 16q + lane%16
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = q * 16 + (lane & 15);
            if (row >= nrow)
                continue;
            const int tok = s_tok[r0 + row];
            const float cf = s_coef[r0 + row];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int arl = wave * 16 + (lane >> 4) * 4 + e;
                if (arl >= nar)
                    continue;
                const int ar = ar0 + arl;
                const int sg = ar / R;
                const float v = cf * acc[q][e];
                const uint16_t hi = f32_to_bf16(v);
                const uint16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
                uint16_t *vp = vt + (int64_t)tok * pitch + sg * kxs + d * 2 * R + (ar - sg * R);
                vp[0] = hi;
                vp[R] = lo;
            }
        }
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
    int list_stride;
};

// Loads this thread's 4 + 4 chunks of k-tile kt (main or extra) into registers.
struct PfLoad {
    u32x4 w[4], x[4];
};

__device__ __forceinline__ void pf_load(const GemmArgs &P, int m0, int n0, int kt, int nk_main,
                                        int m, int D, int kxs, int sg_lo, int kb_per_slice,
                                        PfLoad &L)
{
    const int R = P.g.R;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = threadIdx.x + i * PF_THREADS;   // 0..2047
        const int row = e >> 3, cc = e & 7;
        u32x4 wv = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
        const int n = n0 + row;
        const int t = m0 + row;
        if (kt < nk_main) {
            const int k = kt * PF_BK + cc * 8;
            if (n < P.n_out && k < P.n_in)
                wv = *(const u32x4 *)(P.W + (int64_t)n * P.n_in + k);
            if (t < P.T && k < P.n_in)
                xv = *(const u32x4 *)(P.x + (int64_t)t * P.n_in + k);
        } else {
            const int ke = kt - nk_main;
            const int sg = sg_lo + ke / kb_per_slice;
            const int kk = (ke % kb_per_slice) * PF_BK + cc * 8;   // column within the slice block
            // V side: tile row `row`, column sg*kxs + kk
            if (t < P.T)
                xv = *(const u32x4 *)(P.vcat + (int64_t)m * P.vcat_tile_elems +
                                      (int64_t)row * (P.g.n_slices * kxs) + sg * kxs + kk);
            // B side: B[a_d][n][rho..rho+8) (for the hi and the lo half) when row n is in slice sg
            const int dd = kk / (2 * R);
            if (n < P.n_out && dd < D && n >= P.g.slice_start[sg] && n < P.g.slice_start[sg + 1]) {
                const int a = P.tile_list[(int64_t)m * P.list_stride + dd];
                const int rho = (kk - dd * 2 * R) % R;
                wv = *(const u32x4 *)(P.g.B + ((int64_t)a * P.n_out + n) * R + rho);
            }
        }
        L.w[i] = wv;
        L.x[i] = xv;
    }
}

__device__ __forceinline__ void pf_store(uint16_t *sw, uint16_t *sx, const PfLoad &L)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = threadIdx.x + i * PF_THREADS;
        const int row = e >> 3, cc = e & 7;
        *(u32x4 *)(sw + (row * 8 + pf_swz(row, cc)) * 8) = L.w[i];
        *(u32x4 *)(sx + (row * 8 + pf_swz(row, cc)) * 8) = L.x[i];
    }
}

__global__ __launch_bounds__(PF_THREADS) void prefill_gemm_kernel(GemmArgs P)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t pf_lds[];
    // [buf][W tile 256 x 64 | x tile 256 x 64]
    uint16_t *sw0 = pf_lds, *sx0 = pf_lds + PF_BN * PF_BK;
    uint16_t *sw1 = pf_lds + 2 * PF_BN * PF_BK, *sx1 = sw1 + PF_BN * PF_BK;

    // tile order: groups of 8 n-tiles per m-tile, m fastest inside a group
    const int GN = 8;
    const int per_group = GN * P.n_mtiles;
    const int grp = blockIdx.x / per_group;
    const int rem = blockIdx.x - grp * per_group;
    const int gn = min(GN, P.n_ntiles - grp * GN);
    const int mt = rem / gn;
    const int nt = grp * GN + (rem - mt * gn);
    const int m0 = mt * PF_BM, n0 = nt * PF_BN;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wn = wave & 3, wm = wave >> 2;
    const int r = lane & 15, gq = lane >> 4;

    const int nk_main = (P.n_in + PF_BK - 1) / PF_BK;
    int D = 0, kxs = 0, sg_lo = 0, sg_hi = -1, kb_per_slice = 1;
    if (P.lora) {
        D = P.tile_D[mt];
        kxs = ((D * 2 * P.g.R + PF_BK - 1) / PF_BK) * PF_BK;
        if (D > 0) {
            kb_per_slice = kxs / PF_BK;
            const int nlast = min(n0 + PF_BN, P.n_out) - 1;
            while (sg_lo + 1 < P.g.n_slices && n0 >= P.g.slice_start[sg_lo + 1])
                ++sg_lo;
            sg_hi = sg_lo;
            while (sg_hi + 1 < P.g.n_slices && nlast >= P.g.slice_start[sg_hi + 1])
                ++sg_hi;
        }
    }
    const int nk = nk_main + (D > 0 ? (sg_hi - sg_lo + 1) * kb_per_slice : 0);

    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    PfLoad L;
    pf_load(P, m0, n0, 0, nk_main, mt, D, kxs, sg_lo, kb_per_slice, L);
    pf_store(sw0, sx0, L);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more)
            pf_load(P, m0, n0, kt + 1, nk_main, mt, D, kxs, sg_lo, kb_per_slice, L);
        const uint16_t *sw = (kt & 1) ? sw1 : sw0;
        const uint16_t *sx = (kt & 1) ? sx1 : sx0;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int cch = ks * 4 + gq;
            bf16x8 af[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wn * 64 + i * 16 + r;
                af[i] = *(const bf16x8 *)(sw + (row * 8 + pf_swz(row, cch)) * 8);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int row = wm * 128 + j * 16 + r;
                const bf16x8 bv = *(const bf16x8 *)(sx + (row * 8 + pf_swz(row, cch)) * 8);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bv, acc[i][j], 0,
                                                                        0, 0);
            }
        }
        if (more)
            pf_store((kt & 1) ? sw0 : sw1, (kt & 1) ? sx0 : sx1, L);
        __syncthreads();
    }

    // lane holds rows n0 + wn*64 + i*16 + 4*gq + (0..3) of token m0 + wm*128 + j*16 + r
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
PrefillCfg prefill_config(int64_t T, int32_t K, int64_t n_in, int64_t n_out, int32_t S, int32_t R,
                          int32_t n_slices)
{
    PrefillCfg c;
    c.n_mtiles = (int)((T + PF_BM - 1) / PF_BM);
    c.n_ntiles = (int)((n_out + PF_BN - 1) / PF_BN);
    c.list_stride = (int)std::min<int64_t>((int64_t)PF_BM * K, S);
    const int64_t kxs_max = ((int64_t)c.list_stride * 2 * R + PF_BK - 1) / PF_BK * PF_BK;
    c.vcat_tile_elems = (int64_t)PF_BM * n_slices * kxs_max;
    (void)n_in;
    return c;
}

size_t prefill_workspace_bytes(const PrefillCfg &c)
{
    const size_t lists = (size_t)c.n_mtiles * c.list_stride * sizeof(int32_t);
    return ((size_t)c.n_mtiles * sizeof(int32_t) + 255) / 256 * 256 + 2 * ((lists + 255) / 256 * 256) +
           (size_t)c.n_mtiles * c.vcat_tile_elems * sizeof(uint16_t);
}

bool prefill_worth_it(int64_t T, int64_t n_out)
{
    const int64_t tiles = ((T + PF_BM - 1) / PF_BM) * ((n_out + PF_BN - 1) / PF_BN);
    return T >= 512 && tiles >= 128;
}

hipError_t launch_prefill(const uint16_t *x, const uint16_t *W, int64_t T, int64_t n_in,
                          int64_t n_out, const SlotGeom *g, const int32_t *idx, int32_t K,
                          const float *scale, uint16_t *y, const PrefillCfg &c, void *ws,
                          hipStream_t stream)
{
    uint8_t *p = (uint8_t *)ws;
    int32_t *tile_D = (int32_t *)p;
    p += ((size_t)c.n_mtiles * sizeof(int32_t) + 255) / 256 * 256;
    const size_t lists = ((size_t)c.n_mtiles * c.list_stride * sizeof(int32_t) + 255) / 256 * 256;
    int32_t *tile_list = (int32_t *)p;
    p += lists;
    int32_t *tile_cnt = (int32_t *)p;
    p += lists;
    uint16_t *vcat = (uint16_t *)p;

    if (g != nullptr) {
        const size_t lds = (size_t)((g->S + 31) / 32) * 4 + (size_t)g->S * 4;
        static size_t lds_allowed = 64 * 1024;
        if (lds > lds_allowed) {
            hipError_t e = hipFuncSetAttribute((const void *)tile_plan_kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess)
                return e;
            lds_allowed = lds;
        }
        hipLaunchKernelGGL(tile_plan_kernel, dim3(c.n_mtiles), dim3(256), lds, stream, idx,
                           (int)T, K, g->S, g->R, g->n_slices, c.list_stride, tile_D, tile_list,
                           tile_cnt, vcat, c.vcat_tile_elems);
        ShrinkArgs s{};
        s.x = x;
        s.T = (int)T;
        s.n_in = (int)n_in;
        s.K = K;
        s.g = *g;
        s.idx = idx;
        s.scale = scale;
        s.n_mtiles = c.n_mtiles;
        s.list_stride = c.list_stride;
        s.n_wb = (g->n_slices * g->R + 63) / 64;
        s.tile_D = tile_D;
        s.tile_list = tile_list;
        s.tile_cnt = tile_cnt;
        s.vcat = vcat;
        s.vcat_tile_elems = c.vcat_tile_elems;
        hipLaunchKernelGGL(sgmv_shrink_kernel, dim3(1024), dim3(256), 0, stream, s);
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
    a.vcat = vcat;
    a.vcat_tile_elems = c.vcat_tile_elems;
    a.tile_D = tile_D;
    a.tile_list = tile_list;
    a.list_stride = c.list_stride;
    const size_t lds = (size_t)4 * PF_BN * PF_BK * sizeof(uint16_t);   // 128 KB
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)prefill_gemm_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
        attr = true;
    }
    trace_mark(stream, true);
    hipLaunchKernelGGL(prefill_gemm_kernel, dim3((unsigned)(c.n_mtiles * c.n_ntiles)),
                       dim3(PF_THREADS), lds, stream, a);
    const hipError_t e = hipGetLastError();
    trace_mark(stream, false);
    return e;
}

}  // namespace mlora
