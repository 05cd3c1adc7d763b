// Decode path (T <= 64 per launch), first kernel: skinny base GEMM and LoRA shrink in one pass
// over W.
//
// "Multi-LoRA Serving Explained" (sevydevy.com): every token of the batch is multiplied by the
// shared base weight in one product, then each token's side path (shrink by its own A, expand
// by its own B, found through its slot id) is added.  At decode sizes the base product reads W
// (n_out x n_in bf16) once and is bound by HBM bandwidth, so this kernel is built to stream W:
//
//  - a workgroup owns 64 rows of W ("tile") and one split of n_in (up to 8 x 128 columns)
//    and has 8 waves; wave w owns the w-th 128 columns of the split for all 64 rows;
//  - each lane first loads its share of x (all T tokens of the wave's 128 columns, read once
//    per workgroup with whole cache lines per instruction), then the A rows of its
//    workgroup's share of the LoRA shrink, then all of its W fragments (16 x 16 bytes); vmcnt
//    is in order, so the x and A data are usable while W streams in.  x is moved into the
//    MFMA operand layout through the wave's own 16 KB of LDS (XOR-swizzled, conflict-free);
//  - the products run on the matrix cores (v_mfma_f32_16x16x32_bf16: W rows = A operand,
//    16-token tiles of x = B operand).  The order in which a lane's bytes map onto the MFMA's
//    k positions is a permutation shared by both operands, which a sum allows;
//  - the shrink of a (token, slot) pair is the same kind of product with A[a]'s rows in place
//    of W's: one extra MFMA per 32 columns against the x fragments already in registers,
//    keeping the pair's token column;
//  - the 8 waves' partial tiles are added in LDS in a fixed order (deterministic) and the
//    split's partial tile goes to fp32 scratch.
// Launches with many more (chunk, tile, split) items than CUs (vocabulary-wide outputs, several
// chunks) take a persistent variant of the same kernel (below): each workgroup keeps its x and
// walks W.  The finish kernel (decode_finish.hip) then adds the splits in order, adds the LoRA
// delta and rounds y once.  Partial tiles are stored tile-contiguous ([split][tile][token][64 rows]) so
// that the finish kernel reads whole cache lines.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace mlora {

constexpr int DEC_ROWS = 64;    // rows of W per workgroup
constexpr int DEC_CHUNK = 64;   // tokens of one chunk (several chunks may share a launch)
constexpr int DEC_WK = 128;     // columns of n_in per wave
constexpr int DEC_WAVES = 8;

// 16 bytes at row + c when ok, else 16 zero bytes read from a static block: the choice is
// made on the address, so the load's result is used as is (no select that would wait for the
// load right after issuing it) and no branch splits the load stream.
__device__ __attribute__((aligned(64))) uint32_t dec_zero16[16];   // never written: zeros

__device__ __forceinline__ u32x4 dec_ld16(const uint16_t *row, int c, bool ok)
{
    return *(const u32x4 *)(ok ? row + c : (const uint16_t *)dec_zero16);
}

// The same for W, which every launch reads exactly once: a non-temporal load (nt), so the
// stream does not displace x, A and the split partials from the caches.  Measured: the
// T = 64 step 17.8 -> 16.6 us, the LM head 252 -> 243 us.
__device__ __forceinline__ u32x4 dec_ld16_stream(const uint16_t *p, bool ok)
{
    return __builtin_nontemporal_load((const u32x4 *)(ok ? p : (const uint16_t *)dec_zero16));
}

// Shrink piece of pair p, A rows r0..r0+15: D[16 rows][16 tokens] = A rows x (the token tile
// holding t), one MFMA per 32 columns on fragments already in registers; the pair's token
// column is summed over the 8 waves (fixed order) and written to upart[s][j][t][r0..].
template <int TT>
__device__ __forceinline__ void decode_shrink_piece(const u32x4 (&xf)[TT][4], const u32x4 (&af)[4],
                                                    int p, int r0, int K, int T, int wd, int s,
                                                    int wave, int r, int gq,
                                                    float (*sred)[16], float *upart)
{
    const int t = p / K;
    const int tt = t >> 4;
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
    // uniform branch per token tile with compile-time indices: a runtime index into xf would
    // put the fragments in scratch memory
#pragma unroll
    for (int q = 0; q < TT; ++q) {
        if (q == tt) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[ks]),
                                                            __builtin_bit_cast(bf16x8, xf[q][ks]),
                                                            d, 0, 0, 0);
        }
    }
    if (r == (t & 15)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sred[wave][gq * 4 + i] = d[i];
    }
    lds_barrier();
    if (threadIdx.x < 16 && r0 + (int)threadIdx.x < wd) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w)
            sum += sred[w][threadIdx.x];
        const int j = p - t * K;
        float *dst = upart + (((int64_t)s * K + j) * T + t) * wd + r0 + threadIdx.x;
        *dst = sum;
    }
    lds_barrier();
}

struct DecodeArgs {
    const uint16_t *x, *W;
    int T, n_in, n_out, n_tiles, ks_cols, sk;
    SlotGeom g;
    const int32_t *idx;
    int K;
    const float *scale;
    float *part;       // per chunk of 64 tokens: [sk][n_tiles][Tc][64]
    float *upart;      // per chunk: [sk][K][Tc][wd], or nullptr (no LoRA)
    int n_pairs;       // (token, slot) pairs of one chunk: T * K when there is one chunk
    int n_rg, n_kb;    // packed W: row groups of 16, column blocks of 32
    int n_chunks;      // chunks of DEC_CHUNK tokens in this launch (T is their total)
};

template <int TT, bool PW, bool MC>
__global__ __launch_bounds__(512) void decode_gemm_kernel(DecodeArgs P)
{
    extern __shared__ __attribute__((aligned(16))) float red[];   // [8][4][TT][64] float4
    __shared__ float sred[DEC_WAVES][16];
    const uint16_t *__restrict__ W = P.W;
    const int n_in = P.n_in, n_out = P.n_out, n_tiles = P.n_tiles, K = P.K;
    const SlotGeom &g = P.g;
    const int wd = g.n_slices * g.R;
    // Workgroup -> (token chunk, row tile, split).  With several chunks in one launch every XCD
    // (workgroups are dealt to the 8 XCDs round robin) runs a contiguous range of (tile, split)
    // pairs with the chunks innermost, so the chunks of one W slice run back to back on one XCD
    // and read it from that XCD's L2 after the first.
    // (MC: several chunks; the one-chunk kernel keeps the plain mapping and base pointers)
    int chunk = 0, tile, s;
    if constexpr (!MC) {
        tile = blockIdx.x % n_tiles;
        s = blockIdx.x / n_tiles;
    } else {
        const int nwg = gridDim.x, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        const int lt = xcd * (nwg >> 3) + min(xcd, nwg & 7) + slot;
        chunk = lt % P.n_chunks;
        const int pg = lt / P.n_chunks;
        tile = pg % n_tiles;
        s = pg / n_tiles;
    }
    int T = P.T, n_pairs = P.n_pairs;   // one chunk: straight from the arguments
    const uint16_t *__restrict__ x = P.x;
    const int32_t *idx = P.idx;
    float *part = P.part, *upart = P.upart;
    if constexpr (MC) {
        T = min(DEC_CHUNK, P.T - chunk * DEC_CHUNK);
        n_pairs = T * K;
        x += (int64_t)chunk * DEC_CHUNK * n_in;
        if (idx != nullptr)
            idx += (int64_t)chunk * DEC_CHUNK * K;
        part += (int64_t)chunk * P.sk * n_tiles * DEC_CHUNK * DEC_ROWS;
        if (upart != nullptr)
            upart += (int64_t)chunk * P.sk * K * DEC_CHUNK * wd;
    }
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;     // row (A operand) / token (B operand) within a 16-tile
    const int gq = lane >> 4;    // which 16-byte chunk group of the k-step this lane supplies
    const int kw = s * P.ks_cols + wave * DEC_WK;      // first column of this wave
    const bool wave_on = kw < n_in && wave * DEC_WK < P.ks_cols;

    // slot id of this workgroup's first shrink pair, read first (the A addresses wait for it)
    int a0 = -1;
    if (upart != nullptr && tile < n_pairs)
        a0 = idx[tile];

    // column of the chunk this lane supplies at k-step ks: the 4 lanes of a row read 64
    // contiguous bytes per instruction (16 cache lines per wave instruction)
    auto col = [&](int ks) { return kw + (ks * 4 + gq) * 8; };

    // ---- x: the wave's T x 128 slice, loaded line-friendly (lane l reads 16 bytes of row
    //      tt*16 + ks*4 + l/16 at chunk l%16: 8 full cache lines per instruction), then moved
    //      through this wave's own 16 KB of LDS into the MFMA layout (fragment (tt, ks): token
    //      tt*16 + r, chunk ks*4 + gq).  LDS chunk (row, c) is stored at c ^ (row & 15).
    uint16_t *xl = (uint16_t *)(red + wave * (4 * TT * 64 * 4));   // [16*TT rows][16 chunks]
    u32x4 xf[TT][4];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int row = tt * 16 + ks * 4 + gq;
            const int c = kw + r * 8;
            xf[tt][ks] = dec_ld16(x + (int64_t)min(row, T - 1) * n_in, c,
                                  wave_on && row < T && c < n_in);
        }
    // ---- the A rows of the first shrink piece of this workgroup: pair p = tile, rows 0..15 of
    //      A[a] (used after the base products; summed over the waves with the base tiles)
    u32x4 af[4];
    {
        // issued whether or not the pair has an adapter (slot 0's rows then, or x's first row
        // without LoRA; unused either way).  The slot's rank is not consulted here: it would
        // put a second dependent scalar load in front of the W stream (rows past the rank are
        // zero in memory, so reading them is exact).
        const int arow = min(r, max(wd, 1) - 1);
        const uint16_t *ap = upart != nullptr ? g.A + ((int64_t)max(a0, 0) * wd + arow) * n_in : x;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c = col(ks);
            af[ks] = dec_ld16(ap, c, a0 >= 0 && wave_on && c < n_in && r < wd);
        }
    }

    // ---- W fragments: row tile rt, k-step ks, issued in k-step order so that the MFMAs of a
    //      k-step can start as soon as its data is in
    u32x4 wf[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            if constexpr (PW) {
                // packed W: the fragment (row group, column block) is 1 KB in lane order
                const int rg = tile * 4 + rt, kb = (kw >> 5) + ks;
                const bool ok = wave_on && rg < P.n_rg && kb < P.n_kb;
                const uint16_t *wp = W + (((int64_t)min(rg, P.n_rg - 1) * P.n_kb + min(kb, P.n_kb - 1)) * 64 + lane) * 8;
                wf[rt][ks] = dec_ld16_stream(wp, ok);
            } else {
                const int row = tile * DEC_ROWS + rt * 16 + r;
                const uint16_t *wrow = W + (int64_t)min(row, n_out - 1) * n_in;
                const int c = col(ks);
                wf[rt][ks] = dec_ld16_stream(wrow + c, wave_on && c < n_in && row < n_out);
            }
        }
    }
    // every load of the workgroup's slice is in flight before the first wait below (keeps the
    // scheduler from hoisting the x transpose, and its waits, between the W loads)
    asm volatile("" ::: "memory");

#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int row = tt * 16 + ks * 4 + gq;
            *(u32x4 *)(xl + (row * 16 + (r ^ (row & 15))) * 8) = xf[tt][ks];
        }
    // the reads below take other lanes' writes: complete them and keep the compiler from
    // moving the reads above them (LDS executes one wave's operations in order)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int row = tt * 16 + r;
            const int c = ks * 4 + gq;
            xf[tt][ks] = *(const u32x4 *)(xl + (row * 16 + (c ^ (row & 15))) * 8);
        }

    // ---- base products
    f32x4 acc[4][TT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
            acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
                acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, wf[rt][ks]), __builtin_bit_cast(bf16x8, xf[tt][ks]),
                    acc[rt][tt], 0, 0, 0);

    // ---- first shrink piece: its token's column goes to sred and is summed over the waves
    //      together with the base tiles below (no barrier of its own)
    const int t0p = tile / K;
    if (a0 >= 0) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < TT; ++q) {
            if (q == (t0p >> 4)) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, af[ks]), __builtin_bit_cast(bf16x8, xf[q][ks]), d,
                        0, 0, 0);
            }
        }
        if (r == (t0p & 15)) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sred[wave][gq * 4 + i] = d[i];
        }
    }

    // ---- add the 8 waves' tiles in a fixed order and store the split's partial tile
    float4 *red4 = (float4 *)red;
    constexpr int SLOTS = 4 * TT * 64;   // float4 outputs of the workgroup
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
            red4[wave * SLOTS + (rt * TT + tt) * 64 + lane] =
                float4{acc[rt][tt][0], acc[rt][tt][1], acc[rt][tt][2], acc[rt][tt][3]};
    lds_barrier();
    if (a0 >= 0 && threadIdx.x < 16 && (int)threadIdx.x < wd) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w)
            sum += sred[w][threadIdx.x];
        upart[(((int64_t)s * K + (tile - t0p * K)) * T + t0p) * wd + threadIdx.x] = sum;
    }
    for (int sl = threadIdx.x; sl < SLOTS; sl += 512) {
        float4 sum = red4[sl];
#pragma unroll
        for (int w = 1; w < DEC_WAVES; ++w) {
            const float4 v = red4[w * SLOTS + sl];
            sum.x += v.x;
            sum.y += v.y;
            sum.z += v.z;
            sum.w += v.w;
        }
        const int ln = sl & 63;
        const int rt = sl / (64 * TT);
        const int tt = (sl / 64) % TT;
        const int tok = tt * 16 + (ln & 15);
        const int rloc = rt * 16 + (ln >> 4) * 4;   // row within the tile
        if (tok < T)
            *(float4 *)(part + (((int64_t)s * n_tiles + tile) * T + tok) * DEC_ROWS + rloc) = sum;
    }

    // ---- remaining shrink pieces (other row groups, other pairs of this tile); sred is
    //      reused once every wave is past the reads above
    if (upart != nullptr) {
        bool synced = false;
        for (int p = tile; p < n_pairs; p += n_tiles) {
            const int a = idx[p];
            if (a < 0)
                continue;
            const int r8 = slot_rank8(g.rank, a, g.R);
            for (int r0 = (p == tile ? 16 : 0); r0 < wd; r0 += 16) {
                if (g.R >= 16 && r0 % g.R >= r8) {
                    // all 16 rows of the piece past the adapter's rank: exact zeros, no loads
                    const int t = p / K;
                    if (threadIdx.x < 16)
                        upart[(((int64_t)s * K + (p - t * K)) * T + t) * wd + r0 + threadIdx.x] = 0.f;
                    continue;
                }
                if (!synced) {
                    lds_barrier();
                    synced = true;
                }
                u32x4 afr[4];
                const int arow = r0 + r;
                const uint16_t *ap = g.A + ((int64_t)a * wd + min(arow, wd - 1)) * n_in;
                // rows past the adapter's rank (zero padding) come from the zero block
                const bool rok = arow < wd && arow % g.R < r8;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int c = col(ks);
                    afr[ks] = dec_ld16(ap, c, rok && wave_on && c < n_in);
                }
                decode_shrink_piece<TT>(xf, afr, p, r0, K, T, wd, s, wave, r, gq, sred, upart);
            }
        }
    }
}
// Many more (chunk, tile, split) items than CUs (vocabulary-wide outputs, or several 64-token
// chunks): a persistent grid of one workgroup per CU.  A workgroup keeps one (chunk, split s of
// n_in) and walks row tiles l, l + L, l + 2L, ...: x's slice is loaded and moved into the MFMA
// layout once, and each next tile's A rows and W fragments are issued right after the current
// tile's MFMAs, so they stream in while its 8-wave reduction, partial store and remaining
// shrink pieces run.  With one chunk, workgroup b takes s = b % sk and l = b / sk (L = grid /
// sk).  With several, the workgroups of one XCD (b mod 8) hold every chunk of the same (s, l)
// pairs, chunk innermost, so the chunks' copies of a tile's W meet in that XCD's L2.  Per tile
// the arithmetic and its order are those of the kernel above (same output bits).
template <int TT, bool PW, bool MC>
__global__ __launch_bounds__(512) void decode_gemm_ps_kernel(DecodeArgs P, int n_lanes)
{
    extern __shared__ __attribute__((aligned(16))) float red[];   // [8][4][TT][64] float4
    __shared__ float sred[DEC_WAVES][16];
    const uint16_t *__restrict__ W = P.W;
    const int n_in = P.n_in, n_out = P.n_out, n_tiles = P.n_tiles, K = P.K;
    const SlotGeom &g = P.g;
    const int wd = g.n_slices * g.R;
    int s, tile, tstep, chunk = 0;
    if constexpr (!MC) {
        s = blockIdx.x % P.sk;
        tile = blockIdx.x / P.sk;
        tstep = gridDim.x / P.sk;                // the grid is a multiple of sk
    } else {
        // per XCD: (grid / 8) slots = n_chunks x (its share of the (s, l) pairs)
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        const int per_xcd = (gridDim.x >> 3) / P.n_chunks;
        chunk = slot % P.n_chunks;
        const int q = xcd * per_xcd + slot / P.n_chunks;   // (s, l) pair; 8 per_xcd of them
        if (q >= n_lanes * P.sk)
            return;                               // past the last whole lane (sk need not divide)
        s = q % P.sk;
        tile = q / P.sk;
        tstep = n_lanes;                          // 8 per_xcd / sk, set by the host
    }
    int T = P.T, n_pairs = P.n_pairs;
    const uint16_t *__restrict__ x = P.x;
    const int32_t *idx = P.idx;
    float *part = P.part, *upart = P.upart;
    if constexpr (MC) {
        T = min(DEC_CHUNK, P.T - chunk * DEC_CHUNK);
        n_pairs = T * K;
        x += (int64_t)chunk * DEC_CHUNK * n_in;
        if (idx != nullptr)
            idx += (int64_t)chunk * DEC_CHUNK * K;
        part += (int64_t)chunk * P.sk * n_tiles * DEC_CHUNK * DEC_ROWS;
        if (upart != nullptr)
            upart += (int64_t)chunk * P.sk * K * DEC_CHUNK * wd;
    }
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int gq = lane >> 4;
    const int kw = s * P.ks_cols + wave * DEC_WK;
    const bool wave_on = kw < n_in && wave * DEC_WK < P.ks_cols;
    auto col = [&](int ks) { return kw + (ks * 4 + gq) * 8; };

    int a0 = -1;
    if (upart != nullptr && tile < n_pairs)
        a0 = idx[tile];

    // x: as in the kernel above, once for all the workgroup's tiles
    uint16_t *xl = (uint16_t *)(red + wave * (4 * TT * 64 * 4));
    u32x4 xf[TT][4];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int row = tt * 16 + ks * 4 + gq;
            const int c = kw + r * 8;
            xf[tt][ks] = dec_ld16(x + (int64_t)min(row, T - 1) * n_in, c,
                                  wave_on && row < T && c < n_in);
        }
    // A rows of a tile's first shrink piece (pair p = tile) and its W fragments
    u32x4 af[4], wf[4][4];
    auto load_a = [&](int a) {
        const int arow = min(r, max(wd, 1) - 1);
        const uint16_t *ap = upart != nullptr ? g.A + ((int64_t)max(a, 0) * wd + arow) * n_in : x;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c = col(ks);
            af[ks] = dec_ld16(ap, c, a >= 0 && wave_on && c < n_in && r < wd);
        }
    };
    auto load_w = [&](int tl) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                if constexpr (PW) {
                    const int rg = tl * 4 + rt, kb = (kw >> 5) + ks;
                    const bool ok = wave_on && rg < P.n_rg && kb < P.n_kb;
                    const uint16_t *wp = W + (((int64_t)min(rg, P.n_rg - 1) * P.n_kb + min(kb, P.n_kb - 1)) * 64 + lane) * 8;
                    wf[rt][ks] = dec_ld16_stream(wp, ok);
                } else {
                    const int row = tl * DEC_ROWS + rt * 16 + r;
                    const uint16_t *wrow = W + (int64_t)min(row, n_out - 1) * n_in;
                    const int c = col(ks);
                    wf[rt][ks] = dec_ld16_stream(wrow + c, wave_on && c < n_in && row < n_out);
                }
            }
        }
    };
    load_a(a0);
    load_w(tile);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int row = tt * 16 + ks * 4 + gq;
            *(u32x4 *)(xl + (row * 16 + (r ^ (row & 15))) * 8) = xf[tt][ks];
        }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int row = tt * 16 + r;
            const int c = ks * 4 + gq;
            xf[tt][ks] = *(const u32x4 *)(xl + (row * 16 + (c ^ (row & 15))) * 8);
        }
    // every wave is past its transpose reads before the first tile's sums reuse the LDS
    lds_barrier();

    while (true) {
        const int next = tile + tstep;
        const bool more = next < n_tiles;
        // the next tile's slot id, early: its A rows wait for it
        int a0n = -1;
        if (more && upart != nullptr && next < n_pairs)
            a0n = idx[next];

        f32x4 acc[4][TT];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
                acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
                    acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, wf[rt][ks]), __builtin_bit_cast(bf16x8, xf[tt][ks]),
                        acc[rt][tt], 0, 0, 0);
        const int t0p = tile / K;
        if (a0 >= 0) {
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < TT; ++q) {
                if (q == (t0p >> 4)) {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, af[ks]), __builtin_bit_cast(bf16x8, xf[q][ks]),
                            d, 0, 0, 0);
                }
            }
            if (r == (t0p & 15)) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sred[wave][gq * 4 + i] = d[i];
            }
        }
        // the next tile's loads, in flight during this tile's reduction and stores
        if (more) {
            load_a(a0n);
            load_w(next);
        }

        float4 *red4 = (float4 *)red;
        constexpr int SLOTS = 4 * TT * 64;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
                red4[wave * SLOTS + (rt * TT + tt) * 64 + lane] =
                    float4{acc[rt][tt][0], acc[rt][tt][1], acc[rt][tt][2], acc[rt][tt][3]};
        lds_barrier();
        if (a0 >= 0 && threadIdx.x < 16 && (int)threadIdx.x < wd) {
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < DEC_WAVES; ++w)
                sum += sred[w][threadIdx.x];
            upart[(((int64_t)s * K + (tile - t0p * K)) * T + t0p) * wd + threadIdx.x] = sum;
        }
        for (int sl = threadIdx.x; sl < SLOTS; sl += 512) {
            float4 sum = red4[sl];
#pragma unroll
            for (int w = 1; w < DEC_WAVES; ++w) {
                const float4 v = red4[w * SLOTS + sl];
                sum.x += v.x;
                sum.y += v.y;
                sum.z += v.z;
                sum.w += v.w;
            }
            const int ln = sl & 63;
            const int rt = sl / (64 * TT);
            const int tt = (sl / 64) % TT;
            const int tok = tt * 16 + (ln & 15);
            const int rloc = rt * 16 + (ln >> 4) * 4;
            if (tok < T)
                *(float4 *)(part + (((int64_t)s * n_tiles + tile) * T + tok) * DEC_ROWS + rloc) = sum;
        }

        // remaining shrink pieces of this tile (as in the kernel above)
        if (upart != nullptr) {
            bool synced = false;
            for (int p = tile; p < n_pairs; p += n_tiles) {
                const int a = idx[p];
                if (a < 0)
                    continue;
                const int r8 = slot_rank8(g.rank, a, g.R);
                for (int r0 = (p == tile ? 16 : 0); r0 < wd; r0 += 16) {
                    if (g.R >= 16 && r0 % g.R >= r8) {
                        const int t = p / K;
                        if (threadIdx.x < 16)
                            upart[(((int64_t)s * K + (p - t * K)) * T + t) * wd + r0 + threadIdx.x] = 0.f;
                        continue;
                    }
                    if (!synced) {
                        lds_barrier();
                        synced = true;
                    }
                    u32x4 afr[4];
                    const int arow = r0 + r;
                    const uint16_t *ap = g.A + ((int64_t)a * wd + min(arow, wd - 1)) * n_in;
                    const bool rok = arow < wd && arow % g.R < r8;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const int c = col(ks);
                        afr[ks] = dec_ld16(ap, c, rok && wave_on && c < n_in);
                    }
                    decode_shrink_piece<TT>(xf, afr, p, r0, K, T, wd, s, wave, r, gq, sred, upart);
                }
            }
        }
        if (!more)
            break;
        tile = next;
        a0 = a0n;
        lds_barrier();   // this tile's reads of red and sred are done before the next one's writes
    }
}

DecodeCfg decode_config(int64_t T, int64_t n_in, int64_t n_out)
{
    DecodeCfg c;
    c.tt = T <= 16 ? 1 : T <= 32 ? 2 : 4;   // more than 64 tokens: chunks of 64
    c.n_tiles = (int)((n_out + DEC_ROWS - 1) / DEC_ROWS);
    const int64_t wblocks = (n_in + DEC_WK - 1) / DEC_WK;          // 128-column blocks
    // each workgroup takes up to 8 blocks (one per wave); split further, down to 4 blocks a
    // workgroup, while the grid (all the launch's 64-token chunks) is smaller than the
    // device's CUs.  Finer splits measured slower: they leave most waves of a workgroup
    // without columns and make the finish add more partials (64 tokens at 4096 -> 512: 21.3
    // us at 32 splits, 13.8 at 8; 256 tokens at 512 -> 4096: 31.9 us at 4 splits, 18.6 at 1)
    const int n_cus = device_cu_count();
    const int64_t n_chunks = (T + DEC_CHUNK - 1) / DEC_CHUNK;
    int per = DEC_WAVES;
    while (per > DEC_WAVES / 2 && n_chunks * c.n_tiles * ((wblocks + per - 1) / per) < n_cus)
        per >>= 1;
    c.kr = per * DEC_WK;
    c.sk = (int)((n_in + c.kr - 1) / c.kr);
    return c;
}

// The GEMM's workgroups of one row tile share out the shrink pieces of the pairs assigned to
// that tile (pair p of a 64-token chunk to tile p mod n_tiles), each pair's n_slices R rows in
// blocks of 16, one piece after another, each a dependent chain (A rows, MFMAs, the 8 waves'
// sums); the first rides in the main pass.  Where a tile gets 2 or more pairs and 4 or more
// pieces (8 when the launch has several chunks, whose workgroups take two or more rounds of
// the CUs and so hide part of the chains), the shrink runs apart (the per-pair kernel, in the
// pieces' layout with one split) before a GEMM of the base alone.  Measured at 64 tokens:
// 4096 -> 512 13.3 against 19.8 us, 4096 -> 1024 13.8 against 15.2, merged QKV 4096 -> 1536
// (3 pairs, 3 blocks a pair) 17.0 against 22.6; kept fused: 4096 -> 2048 (2 pieces) 14.4
// against 15.6, rank 64 slots at 4096 -> 4096 (1 pair, 4 blocks) 27.7 against 28.8, 512
// tokens at 4096 -> 1024 (4 pieces, 8 chunks) 35.7 against 40.9.
bool decode_shrink_apart(int64_t T, int32_t K, int64_t n_out, int32_t wd)
{
    const int64_t n_tiles = (n_out + DEC_ROWS - 1) / DEC_ROWS;
    const int64_t pairs = (std::min<int64_t>(T, DEC_CHUNK) * K + n_tiles - 1) / n_tiles;
    const int64_t pieces = pairs * ((wd + 15) / 16);
    const bool chunks = T > DEC_CHUNK;
    return pairs >= 2 && pieces >= (chunks ? 8 : 4);
}

size_t decode_partial_bytes(int64_t T, int64_t n_in, int64_t n_out)
{
    const DecodeCfg c = decode_config(T, n_in, n_out);
    const int64_t n_chunks = (T + DEC_CHUNK - 1) / DEC_CHUNK;
    const int64_t per = n_chunks > 1 ? DEC_CHUNK : T;           // token stride of a chunk
    return (size_t)n_chunks * c.sk * c.n_tiles * (size_t)per * DEC_ROWS * sizeof(float);
}

// When the launch takes the persistent grid (decode_gemm_ps_kernel): one chunk with more
// (tile, split) items than CUs (one workgroup per item would take a second, partial round:
// 64 tokens at 4096 -> 6144 22.8 -> 21.6 us, merged QKV 29.9 -> 25.7 us with the grid from
// there rather than from twice the CUs); several chunks when every XCD can hold all chunks of
// whole (split, tile-lane) groups (the (split, lane) slots past the last whole lane stay idle:
// 256 tokens at 11008 -> 4096, 11 splits over 64 slots, 107 -> 93 us) and each workgroup
// walks at least two tiles.
static bool ps_one_chunk(const DecodeCfg &c)
{
    const int n_cus = device_cu_count();
    return (int64_t)c.n_tiles * c.sk > (int64_t)n_cus && c.sk <= n_cus;
}

static bool ps_several_chunks(int n_chunks, const DecodeCfg &c)
{
    const int per_xcd = (device_cu_count() / 8) / n_chunks;
    const int n_lanes = 8 * per_xcd / c.sk;
    return n_lanes >= 1 && c.n_tiles >= 2 * n_lanes;
}

bool decode_gemm_persistent(int64_t T, int64_t n_in, int64_t n_out)
{
    const DecodeCfg c = decode_config(T, n_in, n_out);
    const int n_chunks = (int)((T + DEC_CHUNK - 1) / DEC_CHUNK);
    return n_chunks > 1 ? (c.tt == 4 && ps_several_chunks(n_chunks, c)) : ps_one_chunk(c);
}

template <int TT, bool PW, bool MC>
static hipError_t launch_tfm(DecodeArgs &a, const DecodeCfg &c, hipStream_t stream)
{
    const size_t lds = (size_t)DEC_WAVES * 4 * TT * 64 * sizeof(float4);
    if (hipError_t e = ensure_dynamic_lds((const void *)decode_gemm_kernel<TT, PW, MC>, lds);
        e != hipSuccess)
        return e;
    const dim3 grid((unsigned)(a.n_chunks * c.n_tiles * c.sk)), block(512);
    hipLaunchKernelGGL((decode_gemm_kernel<TT, PW, MC>), grid, block, lds, stream, a);
    return hipGetLastError();
}

template <int TT, bool PW>
static hipError_t launch_tf(DecodeArgs &a, const DecodeCfg &c, hipStream_t stream)
{
    if constexpr (TT == 4) {   // only full 64-token chunks come before the last one
        if (a.n_chunks > 1) {
            // the persistent grid when every XCD can hold all chunks of whole (split, lane)
            // groups and each workgroup gets at least two tiles
            const int n_cus = device_cu_count();
            const int per_xcd = (n_cus / 8) / a.n_chunks;          // (s, l) pairs per XCD
            const int n_lanes = 8 * per_xcd / c.sk;                 // whole lanes of sk splits
            if (ps_several_chunks(a.n_chunks, c)) {
                const size_t lds = (size_t)DEC_WAVES * 4 * TT * 64 * sizeof(float4);
                if (hipError_t e =
                        ensure_dynamic_lds((const void *)decode_gemm_ps_kernel<TT, PW, true>, lds);
                    e != hipSuccess)
                    return e;
                const dim3 grid((unsigned)(8 * per_xcd * a.n_chunks)), block(512);
                hipLaunchKernelGGL((decode_gemm_ps_kernel<TT, PW, true>), grid, block, lds, stream,
                                   a, n_lanes);
                return hipGetLastError();
            }
            return launch_tfm<TT, PW, true>(a, c, stream);
        }
    }
    // one chunk with at least twice as many (tile, split) items as CUs: the persistent grid
    const int n_cus = device_cu_count();
    if (ps_one_chunk(c)) {
        const size_t lds = (size_t)DEC_WAVES * 4 * TT * 64 * sizeof(float4);
        if (hipError_t e = ensure_dynamic_lds((const void *)decode_gemm_ps_kernel<TT, PW, false>, lds);
            e != hipSuccess)
            return e;
        const dim3 grid((unsigned)((n_cus / c.sk) * c.sk)), block(512);
        hipLaunchKernelGGL((decode_gemm_ps_kernel<TT, PW, false>), grid, block, lds, stream, a, 0);
        return hipGetLastError();
    }
    return launch_tfm<TT, PW, false>(a, c, stream);
}

hipError_t launch_decode_gemm(const uint16_t *x, const uint16_t *W, bool packed, int64_t T,
                              int64_t n_in, int64_t n_out, float *part, const DecodeCfg &c,
                              const SlotGeom *g, const int32_t *idx, int32_t K, float *upart,
                              hipStream_t stream)
{
    DecodeArgs a{};
    a.x = x;
    a.W = W;
    a.T = (int)T;
    a.n_in = (int)n_in;
    a.n_out = (int)n_out;
    a.n_tiles = c.n_tiles;
    a.ks_cols = c.kr;
    a.sk = c.sk;
    a.idx = idx;
    a.K = K;
    a.part = part;
    a.n_chunks = (int)((T + DEC_CHUNK - 1) / DEC_CHUNK);
    if (g != nullptr && upart != nullptr) {
        a.g = *g;
        a.upart = upart;
        a.n_pairs = (int)(std::min<int64_t>(T, DEC_CHUNK) * K);
    }
    a.n_rg = (int)((n_out + 15) / 16);
    a.n_kb = (int)((n_in + 31) / 32);
    switch (c.tt * 2 + (packed ? 1 : 0)) {
    case 2: return launch_tf<1, false>(a, c, stream);
    case 3: return launch_tf<1, true>(a, c, stream);
    case 4: return launch_tf<2, false>(a, c, stream);
    case 5: return launch_tf<2, true>(a, c, stream);
    case 8: return launch_tf<4, false>(a, c, stream);
    case 9: return launch_tf<4, true>(a, c, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mlora
