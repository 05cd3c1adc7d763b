// Decode path, second kernel: y = bf16(sum of the base GEMM's split-K partials + LoRA delta).
//
// "Multi-LoRA Serving Explained" (sevydevy.com): the base product of the whole batch plus each
// token's own side path B[a] (A[a] x), found through its slot id (-1 = base only).  Learning
// book chapter "04. LoRA Serving", section 6: the scale multiplies the shrink output (v) and
// the expand adds B v into y.  The first kernel (gemm_decode.hip) leaves the base product as
// split-K partial sums and the shrink as split-K pieces; this one finishes both.
//
// One workgroup per (64-row tile, 16 tokens); each thread finishes 4 consecutive rows of one
// token.  Every load that does not depend on another is issued at once: the slot map, the base
// partials (stored tile-contiguous by the GEMM: 4 KB contiguous per split and workgroup) and
// the shrink pieces; v = s * f * (pieces summed in split order) is staged in LDS, then the B
// rows of each (token, slot) are read (4 rows x 2R contiguous bytes) and the expand added.
// Sums run in a fixed order, so the output bits do not depend on scheduling.
#include "common.h"
#include "kernels.h"

namespace mlora {

constexpr int DF_ROWS = 64;       // rows of a tile (the GEMM's tile)
constexpr int DF_TOK = 16;        // tokens per workgroup
constexpr int DF_THREADS = 256;   // 16 tokens x 16 groups of 4 rows
constexpr int DF_BPRE_R = 16;     // ranks up to which slot 0's B rows are prefetched

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

__global__ __launch_bounds__(DF_THREADS) void decode_finish_kernel(
    const float *__restrict__ part, int sk, int n_tiles, const float *__restrict__ upart,
    const float *__restrict__ scale, int T, int n_out, SlotGeom g, const int32_t *__restrict__ idx,
    int K, uint16_t *__restrict__ y)
{
    extern __shared__ __attribute__((aligned(16))) float vl[];   // [DF_TOK][R] of one (slot, slice)
    __shared__ int sidx[DF_TOK * MLORA_MAX_K_DEV];
    const int n_tg = (T + DF_TOK - 1) / DF_TOK;
    const int tile = blockIdx.x / n_tg;
    const int t0 = (blockIdx.x - tile * n_tg) * DF_TOK;
    const int nt = min(DF_TOK, T - t0);
    const int tl = threadIdx.x >> 4, g4 = threadIdx.x & 15;
    const int t = t0 + tl;
    const int row0 = tile * DF_ROWS;
    const int n = row0 + g4 * 4;                  // first of this thread's 4 rows
    const bool lora = upart != nullptr;
    const int R = g.R, wd = g.n_slices * R;

    if (lora && threadIdx.x < nt * K)
        sidx[threadIdx.x] = idx[t0 * K + threadIdx.x];

    // base: split partials of this thread's 4 rows, in split order
    float4 base = {0.f, 0.f, 0.f, 0.f};
    if (tl < nt) {
        const float *src = part + ((int64_t)tile * T + t) * DF_ROWS + g4 * 4;
        const int64_t sstride = (int64_t)n_tiles * T * DF_ROWS;
#pragma unroll 4
        for (int sp = 0; sp < sk; ++sp) {
            const float4 o = *(const float4 *)(src + sp * sstride);
            base.x += o.x;
            base.y += o.y;
            base.z += o.z;
            base.w += o.w;
        }
    }

    // LoRA delta, one (slot j, slice sg) at a time: v[j][t0 + tt][sg*R .. sg*R + R) =
    // coef * (pieces summed in split order), zero for -1 slots, staged in LDS.  For small
    // ranks the B rows of slot 0 are loaded before the staging, so the two loads overlap.
    float d4[4] = {0.f, 0.f, 0.f, 0.f};
    if (lora) {
        lds_barrier();   // sidx visible
        int rsg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ni = min(n + i, n_out - 1);
            int sg = 0;
            while (sg + 1 < g.n_slices && ni >= g.slice_start[sg + 1])
                ++sg;
            rsg[i] = sg;
        }
        const bool pre = R <= DF_BPRE_R;
        u32x4 bp[4][DF_BPRE_R / 8];
        if (pre) {
            const int a = tl < nt ? sidx[tl * K] : -1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint16_t *brow = g.B + ((int64_t)max(a, 0) * n_out + min(n + i, n_out - 1)) * R;
#pragma unroll
                for (int u = 0; u < DF_BPRE_R / 8; ++u)
                    bp[i][u] = (a >= 0 && u * 8 < R) ? *(const u32x4 *)(brow + u * 8)
                                                     : u32x4{0u, 0u, 0u, 0u};
            }
        }
        const int64_t pstride = (int64_t)K * T * wd;
        const int nv = nt * R;                    // a multiple of 8
        for (int j = 0; j < K; ++j) {
            for (int sg = 0; sg < g.n_slices; ++sg) {
                if (j + sg > 0)
                    lds_barrier();                // the previous round's reads are done
                for (int e0 = threadIdx.x * 4; e0 < nv; e0 += DF_THREADS * 4) {
                    const int tt = e0 / R, c = e0 - tt * R;
                    const int a = sidx[tt * K + j];
                    float4 sum = {0.f, 0.f, 0.f, 0.f};
                    if (a >= 0) {
                        const float *src = upart + ((int64_t)j * T + t0 + tt) * wd + sg * R + c;
#pragma unroll 4
                        for (int sp = 0; sp < sk; ++sp) {
                            const float4 o = *(const float4 *)(src + sp * pstride);
                            sum.x += o.x;
                            sum.y += o.y;
                            sum.z += o.z;
                            sum.w += o.w;
                        }
                        const float cf = (scale ? scale[(t0 + tt) * K + j] : 1.f) * g.factor[a];
                        sum.x *= cf;
                        sum.y *= cf;
                        sum.z *= cf;
                        sum.w *= cf;
                    }
                    *(float4 *)(vl + e0) = sum;
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
                    float dj = 0.f;
                    if (pre && j == 0) {
#pragma unroll
                        for (int u = 0; u < DF_BPRE_R / 8; ++u)
                            if (u * 8 < R)
                                dj += dot8(bp[i][u], vv + u * 8);
                    } else {
                        const uint16_t *brow = g.B + ((int64_t)a * n_out + min(n + i, n_out - 1)) * R;
                        for (int rho = 0; rho < R; rho += 8)
                            dj += dot8(*(const u32x4 *)(brow + rho), vv + rho);
                    }
                    d4[i] += dj;
                }
            }
        }
    }
    const float4 delta = {d4[0], d4[1], d4[2], d4[3]};
    if (tl >= nt)
        return;
    const float o4[4] = {base.x + delta.x, base.y + delta.y, base.z + delta.z, base.w + delta.w};
    uint16_t *yo = y + (int64_t)t * n_out + n;
    if (n + 3 < n_out && (n_out & 3) == 0) {
        *(u32x2 *)yo = u32x2{pack_bf16x2(o4[0], o4[1]), pack_bf16x2(o4[2], o4[3])};
    } else {
        for (int i = 0; i < 4; ++i)
            if (n + i < n_out)
                yo[i] = f32_to_bf16(o4[i]);
    }
}

hipError_t launch_decode_finish(const float *part, int32_t sk, int32_t n_tiles, const float *upart,
                                const float *scale, int64_t T, int64_t n_out, const SlotGeom *g,
                                const int32_t *idx, int32_t K, uint16_t *y, hipStream_t stream)
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
    const unsigned grid = (unsigned)(n_tiles * ((T + DF_TOK - 1) / DF_TOK));
    hipLaunchKernelGGL(decode_finish_kernel, dim3(grid), dim3(DF_THREADS), lds, stream, part, sk,
                       n_tiles, upart, scale, (int)T, (int)n_out, gg, idx, K, y);
    return hipGetLastError();
}

}  // namespace mlora
