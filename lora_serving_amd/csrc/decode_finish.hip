// Decode path, second kernel: y = bf16(sum of the base GEMM's split-K partials + LoRA delta).
//
// "Multi-LoRA Serving Explained" (sevydevy.com): the base product of the whole batch plus each
// token's own side path B[a] (A[a] x), found through its slot id (-1 = base only).  Learning
// book chapter "04. LoRA Serving", section 6: the scale multiplies the shrink output (v) and
// the expand adds B v into y.  The first kernel (gemm_decode.hip) leaves the base product as
// split-K partial sums and the shrink as split-K pieces; this one finishes both.
//
// The base partials are stored tile-contiguous by the GEMM ([split][64-row tile][token][64]).
// Two kernels: slots up to 32 wide and the base alone take one workgroup per (tile, 8 tokens),
// two rows a thread; wider slots one workgroup per (tile, 16 tokens), four rows a thread.  In
// both, every load that does not depend on another is issued at once, v = s * f * (pieces
// summed in split order) is staged in LDS, then the B rows of each (token, slot) are read and
// the expand added.  Sums run in a fixed order, so the output bits do not depend on
// scheduling.
#include "common.h"
#include "kernels.h"

namespace mlora {

constexpr int DF_ROWS = 64;       // rows of a tile (the GEMM's tile)
constexpr int DF_TOK = 16;        // tokens per workgroup
constexpr int DF_THREADS = 256;   // 16 tokens x 16 groups of 4 rows
constexpr int DF_CHUNK = 64;      // tokens of one chunk of the GEMM (one launch may hold several)

// Masked loads read this static block instead (the choice is made on the address, so no
// select waits for a load right after it is issued).
__device__ __attribute__((aligned(64))) float df_zero[16];   // never written: zeros

// 8 bf16 (packed) times 8 fp32, summed in order
__device__ __forceinline__ float dot8(const u32x4 b, const float *v)
{
    float d = 0.f;
    d += bf16_lo(b.x) * v[0];
    d += bf16_hi(b.x) * v[1];
    d += bf16_lo(b.y) * v[2];
    d += bf16_hi(b.y) * v[3];
    d += bf16_lo(b.z) * v[4];
    d += bf16_hi(b.z) * v[5];
    d += bf16_lo(b.w) * v[6];
    d += bf16_hi(b.w) * v[7];
    return d;
}

// Loads the split partials of this thread's 4 rows (up to DF_PQ in flight; more splits are
// added in further groups) without waiting for them.
constexpr int DF_PQ = 8;

// v of one (slot j, slice sg) for the block's tokens: element e0..e0+3 of the [DF_TOK][R]
// block, the pieces of the sk splits (zeros for a -1 slot) loaded into pv.
__device__ __forceinline__ void df_vload(const float *upart, int sk, int64_t pstride, int K, int T,
                                         int wd, int R, int t0, int j, int sg, int e0,
                                         const int *sidx, const float *scale, const float *factor,
                                         float4 (&pv)[DF_PQ], float &sc, float &fa)
{
    const int tt = e0 / R, c = e0 - tt * R;
    const int a = sidx[tt * K + j];
    const float *src = upart + ((int64_t)j * T + t0 + tt) * wd + sg * R + c;
#pragma unroll
    for (int sp = 0; sp < DF_PQ; ++sp)
        pv[sp] = *(const float4 *)(a >= 0 && sp < sk ? src + sp * pstride : df_zero);
    sc = *(scale ? scale + (t0 + tt) * K + j : df_zero + 1);    // df_zero[1] stands for "no scale"
    fa = *(a >= 0 ? factor + a : df_zero);
}

// Slots wider than 32 (R >= 64): each thread reads its own 4 rows of B, the columns up to the
// adapter's rank (rounded to 8).
template <bool MC>
__global__ __launch_bounds__(DF_THREADS) void decode_finish_wide_kernel(
    const float *__restrict__ part, int sk, int n_tiles, const float *__restrict__ upart, int usk,
    const float *__restrict__ scale, int T_all, int n_out, SlotGeom g,
    const int32_t *__restrict__ idx, int K, uint16_t *__restrict__ y, float *__restrict__ ysum)
{
    extern __shared__ __attribute__((aligned(16))) float vl[];   // [DF_TOK][R] of one (slot, slice)
    __shared__ int sidx[DF_TOK * MLORA_MAX_K_DEV];
    // chunks of DF_CHUNK tokens (the GEMM's chunks): this workgroup's chunk and its inputs
    // (MC: several chunks; one chunk keeps the plain mapping and base pointers)
    const int n_tg = ((MC ? DF_CHUNK : T_all) + DF_TOK - 1) / DF_TOK;
    const int chunk = MC ? blockIdx.x / (n_tiles * n_tg) : 0;
    const unsigned bl = blockIdx.x - chunk * (n_tiles * n_tg);
    const int T = MC ? min(DF_CHUNK, T_all - chunk * DF_CHUNK) : T_all;
    if constexpr (MC) {
        const int wd0 = g.n_slices * g.R;
        part += (int64_t)chunk * sk * n_tiles * DF_CHUNK * DF_ROWS;
        if (upart != nullptr)
            upart += (int64_t)chunk * usk * K * DF_CHUNK * wd0;
        if (idx != nullptr)
            idx += (int64_t)chunk * DF_CHUNK * K;
        if (scale != nullptr)
            scale += (int64_t)chunk * DF_CHUNK * K;
        y += (int64_t)chunk * DF_CHUNK * n_out;
        if (ysum != nullptr)
            ysum += (int64_t)chunk * DF_CHUNK * n_out;
    }
    const int tile = bl / n_tg;
    const int t0 = (bl - tile * n_tg) * DF_TOK;
    const int nt = min(DF_TOK, T - t0);
    const int tl = threadIdx.x >> 4, g4 = threadIdx.x & 15;
    const int t = t0 + tl;
    const int row0 = tile * DF_ROWS;
    const int n = row0 + g4 * 4;                  // first of this thread's 4 rows
    const bool lora = upart != nullptr;
    const int R = g.R, wd = g.n_slices * R;
    const int64_t pstride = (int64_t)K * T * wd;

    // ---- phase 1: the slot map and the first DF_PQ split partials, all in flight
    const bool has_idx = lora && (int)threadIdx.x < nt * K;
    const int32_t my_idx = *(has_idx ? idx + t0 * K + threadIdx.x : (const int32_t *)df_zero);
    const float *psrc = part + ((int64_t)tile * T + min(t, T - 1)) * DF_ROWS + g4 * 4;
    const int64_t sstride = (int64_t)n_tiles * T * DF_ROWS;
    // the partials are read exactly once: non-temporal loads (nt), which leave the caches to
    // the B rows and v (the step at T = 64 went 16.65 -> 16.55 us)
    float4 pq[DF_PQ];
#pragma unroll
    for (int sp = 0; sp < DF_PQ; ++sp) {
        const f32x4 q =
            __builtin_nontemporal_load((const f32x4 *)(sp < sk ? psrc + sp * sstride : df_zero));
        pq[sp] = float4{q[0], q[1], q[2], q[3]};
    }
    asm volatile("" ::: "memory");

    float d4[4] = {0.f, 0.f, 0.f, 0.f};
    if (lora) {
        // ---- phase 2: the slot map in LDS
        if (has_idx)
            sidx[threadIdx.x] = my_idx;
        lds_barrier();
        // ---- phase 3: the first round's pieces
        int rsg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ni = min(n + i, n_out - 1);
            int sg = 0;
            while (sg + 1 < g.n_slices && ni >= g.slice_start[sg + 1])
                ++sg;
            rsg[i] = sg;
        }
        const int nv = nt * R;                     // a multiple of 8
        const int e0 = threadIdx.x * 4;
        float4 pv[DF_PQ];
        float sc = 0.f, fa = 0.f;
        if (e0 < nv)
            df_vload(upart, usk, pstride, K, T, wd, R, t0, 0, 0, e0, sidx, scale, g.factor, pv, sc,
                     fa);
        asm volatile("" ::: "memory");

        // ---- phase 4: v in LDS one (slot, slice) round at a time, then the expand
        for (int j = 0; j < K; ++j) {
            for (int sg = 0; sg < g.n_slices; ++sg) {
                if (j + sg > 0)
                    lds_barrier();                 // the previous round's reads are done
                for (int e = e0; e < nv; e += DF_THREADS * 4) {
                    if (j + sg > 0 || e != e0)
                        df_vload(upart, usk, pstride, K, T, wd, R, t0, j, sg, e, sidx, scale,
                                 g.factor, pv, sc, fa);
                    const int tt = e / R;
                    const int a = sidx[tt * K + j];
                    float4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int sp = 0; sp < DF_PQ; ++sp) {
                        sum.x += pv[sp].x;
                        sum.y += pv[sp].y;
                        sum.z += pv[sp].z;
                        sum.w += pv[sp].w;
                    }
                    // splits past DF_PQ (rare): added in split order after the first ones
                    for (int sp = DF_PQ; sp < usk; ++sp) {
                        const float4 o = *(const float4 *)(a >= 0 ? upart + ((int64_t)j * T + t0 + tt) * wd +
                                                                        sg * R + (e - tt * R) + sp * pstride
                                                                  : df_zero);
                        sum.x += o.x;
                        sum.y += o.y;
                        sum.z += o.z;
                        sum.w += o.w;
                    }
                    const float cf = a >= 0 ? (scale ? sc : 1.f) * fa : 0.f;
                    *(float4 *)(vl + e) = float4{sum.x * cf, sum.y * cf, sum.z * cf, sum.w * cf};
                }
                lds_barrier();
                const int a = tl < nt ? sidx[tl * K + j] : -1;
                if (a < 0)
                    continue;
                const float *vv = vl + tl * R;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (rsg[i] != sg)
                        continue;
                    // the row's columns up to the adapter's rank (rounded to 8; the rest
                    // multiply zero padding)
                    float dj = 0.f;
                    const uint16_t *brow = g.B + ((int64_t)a * n_out + min(n + i, n_out - 1)) * R;
                    const int r8 = slot_rank8(g.rank, a, R);
                    for (int rho = 0; rho < r8; rho += 8)
                        dj += dot8(*(const u32x4 *)(brow + rho), vv + rho);
                    d4[i] += dj;
                }
            }
        }
    }

    // ---- base: the split partials in split order
    float4 base = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < DF_PQ; ++sp) {
        base.x += pq[sp].x;
        base.y += pq[sp].y;
        base.z += pq[sp].z;
        base.w += pq[sp].w;
    }
    for (int sp = DF_PQ; sp < sk; ++sp) {
        const float4 o = *(const float4 *)(psrc + sp * sstride);
        base.x += o.x;
        base.y += o.y;
        base.z += o.z;
        base.w += o.w;
    }
    if (tl >= nt)
        return;
    const float o4[4] = {base.x + d4[0], base.y + d4[1], base.z + d4[2], base.w + d4[3]};
    uint16_t *yo = y + (int64_t)t * n_out + n;
    float *so = ysum != nullptr ? ysum + (int64_t)t * n_out + n : nullptr;
    if (n + 3 < n_out && (n_out & 3) == 0) {
        *(u32x2 *)yo = u32x2{pack_bf16x2(o4[0], o4[1]), pack_bf16x2(o4[2], o4[3])};
        if (so != nullptr)
            *(float4 *)so = float4{o4[0], o4[1], o4[2], o4[3]};
    } else {
        for (int i = 0; i < 4; ++i) {
            if (n + i < n_out) {
                yo[i] = f32_to_bf16(o4[i]);
                if (so != nullptr)
                    so[i] = o4[i];
            }
        }
    }
}

// Two rows a thread, 8 tokens a workgroup (twice the workgroups of the kernel above, each
// thread with half the rows: more loads in flight per CU and shorter per-wave chains), for
// slot widths R = RC in {8, 16, 32} and for the base alone (RC = 0, no LoRA).  Every load that
// does not depend on a slot id is issued first: the split partials, this thread's token's
// first slot id, and (threads that own a 4-entry quad of v) the quad's shrink pieces, scale
// and slot id.  Then the B rows of the thread's 2 rows and the quad's factor; v = s * f *
// (pieces summed in split order) goes through LDS, one barrier per slot.  The row sums follow
// the kernel above's order (8-column dot products, pieces added pairwise, slots in order).
typedef float f32x2 __attribute__((ext_vector_type(2)));
constexpr int DF2_TOK = 8;

template <bool MC, int RC>
__global__ __launch_bounds__(DF_THREADS) void decode_finish_kernel(
    const float *__restrict__ part, int sk, int n_tiles, const float *__restrict__ upart, int usk,
    const float *__restrict__ scale, int T_all, int n_out, SlotGeom g,
    const int32_t *__restrict__ idx, int K, uint16_t *__restrict__ y, float *__restrict__ ysum)
{
    __shared__ __attribute__((aligned(16))) float vl[DF2_TOK * MLORA_MAX_SLICES_DEV * (RC > 0 ? RC : 4)];
    const int n_tg = ((MC ? DF_CHUNK : T_all) + DF2_TOK - 1) / DF2_TOK;
    const int chunk = MC ? blockIdx.x / (n_tiles * n_tg) : 0;
    const unsigned bl = blockIdx.x - chunk * (n_tiles * n_tg);
    const int T = MC ? min(DF_CHUNK, T_all - chunk * DF_CHUNK) : T_all;
    if constexpr (MC) {
        const int wd0 = g.n_slices * RC;
        part += (int64_t)chunk * sk * n_tiles * DF_CHUNK * DF_ROWS;
        if (RC > 0) {
            upart += (int64_t)chunk * usk * K * DF_CHUNK * wd0;
            idx += (int64_t)chunk * DF_CHUNK * K;
            if (scale != nullptr)
                scale += (int64_t)chunk * DF_CHUNK * K;
        }
        y += (int64_t)chunk * DF_CHUNK * n_out;
        if (ysum != nullptr)
            ysum += (int64_t)chunk * DF_CHUNK * n_out;
    }
    const int tile = bl / n_tg;
    const int t0 = (bl - tile * n_tg) * DF2_TOK;
    const int nt = min(DF2_TOK, T - t0);
    const int tl = threadIdx.x >> 5, g2 = threadIdx.x & 31;
    const int t = t0 + tl;
    const int n = tile * DF_ROWS + g2 * 2;          // first of this thread's 2 rows

    // ---- independent loads: the split partials (read once: non-temporal)
    const float *psrc = part + ((int64_t)tile * T + min(t, T - 1)) * DF_ROWS + g2 * 2;
    const int64_t sstride = (int64_t)n_tiles * T * DF_ROWS;
    f32x2 pq[DF_PQ];
#pragma unroll
    for (int sp = 0; sp < DF_PQ; ++sp)
        pq[sp] = __builtin_nontemporal_load((const f32x2 *)(sp < sk ? psrc + sp * sstride : df_zero));

    float acc[2] = {0.f, 0.f};
    if constexpr (RC > 0) {
        constexpr int CP = RC / 8;                  // 16-byte pieces of a row
        const int wd = g.n_slices * RC, wq = wd / 4;
        const int64_t pstride = (int64_t)K * T * wd;
        // this thread's quad of v: token tq, entries e4 .. e4 + 3 (nt * wd / 4 <= 256 quads)
        const int tq = threadIdx.x / wq, e4 = (threadIdx.x - tq * wq) * 4;
        const bool has_q = tq < nt;
        int my_a = *(tl < nt ? idx + (int64_t)t * K : (const int32_t *)df_zero);
        int sg[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ni = min(n + i, n_out - 1);
            sg[i] = (ni >= g.slice_start[1]) + (ni >= g.slice_start[2]) + (ni >= g.slice_start[3]);
        }
        for (int j = 0; j < K; ++j) {
            // pieces, scale and slot id of this thread's quad (no slot id needed to load them)
            f32x4 pv[DF_PQ];
            const float *qsrc = upart + ((int64_t)j * T + t0 + tq) * wd + e4;
#pragma unroll
            for (int sp = 0; sp < DF_PQ; ++sp)
                pv[sp] = *(const f32x4 *)(has_q && sp < usk ? qsrc + sp * pstride : df_zero);
            const int aq = has_q ? idx[(int64_t)(t0 + tq) * K + j] : -1;
            const float sc = has_q && scale ? scale[(int64_t)(t0 + tq) * K + j] : 1.f;
            if (j > 0) {
                my_a = tl < nt ? idx[(int64_t)t * K + j] : -1;
                lds_barrier();                      // the previous slot's reads of vl are done
            }
            const int a = tl < nt ? my_a : -1;
            // this thread's 2 rows of B[a] (RC columns each), then the quad's factor
            u32x4 bq[2][CP];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint16_t *brow = g.B + ((int64_t)max(a, 0) * n_out + min(n + i, n_out - 1)) * RC;
#pragma unroll
                for (int c = 0; c < CP; ++c)
                    bq[i][c] = *(const u32x4 *)(a >= 0 ? (const void *)(brow + c * 8) : (const void *)df_zero);
            }
            const float fa = *(aq >= 0 ? g.factor + aq : df_zero);
            if (has_q) {
                f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sp = 0; sp < DF_PQ; ++sp)
                    sum += pv[sp];
                for (int sp = DF_PQ; sp < usk; ++sp)
                    sum += *(const f32x4 *)(qsrc + sp * pstride);
                const float cf = aq >= 0 ? (scale ? sc : 1.f) * fa : 0.f;
                *(f32x4 *)(vl + tq * wd + e4) = sum * cf;
            }
            lds_barrier();
            if (a < 0)
                continue;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float *vv = vl + tl * wd + sg[i] * RC;
                float d[CP];
#pragma unroll
                for (int c = 0; c < CP; ++c)
                    d[c] = dot8(bq[i][c], vv + c * 8);
                float sp;
                if constexpr (CP == 1)
                    sp = d[0];
                else if constexpr (CP == 2)
                    sp = d[0] + d[1];
                else
                    sp = (d[0] + d[1]) + (d[2] + d[3]);
                acc[i] += sp;
            }
        }
    }

    // ---- base: the split partials in split order
    f32x2 base = {0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < DF_PQ; ++sp)
        base += pq[sp];
    for (int sp = DF_PQ; sp < sk; ++sp)
        base += *(const f32x2 *)(psrc + sp * sstride);
    if (t >= t0 + nt || n >= n_out)
        return;
    const float o0 = base[0] + acc[0], o1 = base[1] + acc[1];
    uint16_t *yo = y + (int64_t)t * n_out + n;
    float *so = ysum != nullptr ? ysum + (int64_t)t * n_out + n : nullptr;
    if (n + 1 < n_out && (n_out & 1) == 0) {
        *(uint32_t *)yo = pack_bf16x2(o0, o1);
        if (so != nullptr)
            *(f32x2 *)so = f32x2{o0, o1};
    } else {
        yo[0] = f32_to_bf16(o0);
        if (so != nullptr)
            so[0] = o0;
        if (n + 1 < n_out) {
            yo[1] = f32_to_bf16(o1);
            if (so != nullptr)
                so[1] = o1;
        }
    }
}

hipError_t launch_decode_finish(const float *part, int32_t sk, int32_t n_tiles, const float *upart,
                                int32_t usk, const float *scale, int64_t T, int64_t n_out,
                                const SlotGeom *g, const int32_t *idx, int32_t K, uint16_t *y,
                                float *ysum, hipStream_t stream)
{
    SlotGeom gg{};
    size_t lds = 0;
    if (g != nullptr && upart != nullptr) {
        gg = *g;
        lds = (size_t)DF_TOK * g->R * sizeof(float);
    } else {
        upart = nullptr;
        K = 1;
    }
    const int64_t n_chunks = (T + DF_CHUNK - 1) / DF_CHUNK;
    const int rc = upart != nullptr ? (gg.R == 8 || gg.R == 16 || gg.R == 32 ? gg.R : -1) : 0;
    const bool mc = n_chunks > 1;
    if (rc >= 0) {
        // two rows a thread: the base alone, or LoRA with slots up to 32 wide
        const unsigned grid2 = (unsigned)(n_chunks * n_tiles *
                                          ((std::min<int64_t>(T, DF_CHUNK) + DF2_TOK - 1) / DF2_TOK));
#define DF2_LAUNCH(M, C)                                                                           \
    hipLaunchKernelGGL((decode_finish_kernel<M, C>), dim3(grid2), dim3(DF_THREADS), 0, stream,   \
                       part, sk, n_tiles, upart, usk, scale, (int)T, (int)n_out, gg, idx, K, y, \
                       ysum)
        switch (rc * 2 + (mc ? 1 : 0)) {
        case 0: DF2_LAUNCH(false, 0); break;
        case 1: DF2_LAUNCH(true, 0); break;
        case 16: DF2_LAUNCH(false, 8); break;
        case 17: DF2_LAUNCH(true, 8); break;
        case 32: DF2_LAUNCH(false, 16); break;
        case 33: DF2_LAUNCH(true, 16); break;
        case 64: DF2_LAUNCH(false, 32); break;
        default: DF2_LAUNCH(true, 32); break;
        }
#undef DF2_LAUNCH
        return hipGetLastError();
    }
    // wider slots: four rows a thread, each thread reading its own rows of B
    const unsigned grid =
        (unsigned)(n_chunks * n_tiles * ((std::min<int64_t>(T, DF_CHUNK) + DF_TOK - 1) / DF_TOK));
#define DF_LAUNCH(M)                                                                               \
    hipLaunchKernelGGL((decode_finish_wide_kernel<M>), dim3(grid), dim3(DF_THREADS), lds, stream,   \
                       part, sk, n_tiles, upart, usk, scale, (int)T, (int)n_out, gg, idx, K, y, \
                       ysum)
    if (mc)
        DF_LAUNCH(true);
    else
        DF_LAUNCH(false);
#undef DF_LAUNCH
    return hipGetLastError();
}

}  // namespace mlora
