// Skinny base GEMM for decode batches (T <= 128): part[s][t][n] = sum_{i in split s} x[t][i] W[n][i].
//
// "Multi-LoRA Serving Explained" (sevydevy.com): the server multiplies every token of the batch
// by the shared base weight in one big product and adds each token's side path afterwards.  At
// decode sizes that product reads W (n_out x n_in bf16) once and is bound by HBM bandwidth, so
// the kernel is built to stream W at full rate:
//  - a workgroup owns 64 rows of W and one slice of n_in (the split), 4 waves x 16 rows;
//  - every lane issues ALL of its W loads (up to 8 x 64 contiguous bytes) before touching any
//    of them, so each CU keeps ~128 KB of HBM reads in flight;
//  - x[0:T, slice] is copied once into LDS and shared by the 4 waves;
//  - the product runs on the matrix cores (v_mfma_f32_16x16x32_bf16): W rows are the A
//    operand, 16-token tiles of x the B operand.  The order in which a lane's 64 bytes map onto
//    the MFMA's k positions is a permutation shared by both operands, which a sum allows;
//  - partial sums of the n_in splits go to fp32 scratch and are added, in split order, by the
//    expand kernel that also adds the LoRA delta and rounds y once.
// Workgroups past the GEMM grid run the per-pair LoRA shrink instead (no dependency between the
// two, so one launch covers both).
#include <algorithm>

#include "bgmv_dev.h"

namespace mlora {

constexpr int DEC_ROWS = 64;      // rows of W per workgroup
constexpr int DEC_KB = 128;       // n_in per block of loads
constexpr int DEC_NI = 8;         // blocks per workgroup at most (kr <= 1024)

template <int TT>
__global__ __launch_bounds__(256) void decode_gemm_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, int T, int n_in, int n_out,
    float *__restrict__ part, int kr, int n_tiles, int sk, SlotGeom g,
    const int32_t *__restrict__ idx, int32_t K, const float *__restrict__ scale,
    float *__restrict__ v)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
    const int n_gemm = n_tiles * sk;
    if ((int)blockIdx.x >= n_gemm) {
        __shared__ float red[64];
        shrink_one_pair(x, T, n_in, g, idx, K, scale, v, (int64_t)blockIdx.x - n_gemm, red);
        return;
    }
    const int tile = blockIdx.x % n_tiles;
    const int s = blockIdx.x / n_tiles;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int gq = lane >> 4;
    const int k0 = s * kr;
    const int klen = min(kr, n_in - k0);
    const int pitch = kr + 8;

    // 1) every W load of this lane, issued up front
    const int row = tile * DEC_ROWS + wave * 16 + r;
    const bool row_ok = row < n_out;
    const uint16_t *wrow = W + (int64_t)(row_ok ? row : 0) * n_in + k0;
    u32x4 wreg[DEC_NI][4];
#pragma unroll
    for (int ib = 0; ib < DEC_NI; ++ib)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int kk = ib * DEC_KB + gq * 32 + q * 8;
            wreg[ib][q] = (row_ok && kk < klen) ? __builtin_nontemporal_load((const u32x4 *)(wrow + kk))
                                                : u32x4{0u, 0u, 0u, 0u};
        }

    // 2) x[0:16*TT, k0:k0+klen) -> LDS (zeros past T and past klen)
    const int c8n = kr >> 3;
    for (int e = threadIdx.x; e < 16 * TT * c8n; e += 256) {
        const int tt = e / c8n;
        const int c8 = e - tt * c8n;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (tt < T && c8 * 8 < klen)
            val = *(const u32x4 *)(x + (int64_t)tt * n_in + k0 + c8 * 8);
        *(u32x4 *)(xs + tt * pitch + c8 * 8) = val;
    }
    __syncthreads();

    // 3) products
    f32x4 acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
        acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ib = 0; ib < DEC_NI; ++ib) {
        if (ib * DEC_KB < klen) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bf16x8 av = __builtin_bit_cast(bf16x8, wreg[ib][q]);
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    const bf16x8 bv = *(const bf16x8 *)(xs + (tt * 16 + r) * pitch + ib * DEC_KB +
                                                        gq * 32 + q * 8);
                    acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[tt], 0, 0, 0);
                }
            }
        }
    }

    // 4) partial sums: lane holds rows 4*gq..4*gq+3 (of the wave's 16) of token column r
    const int nb = tile * DEC_ROWS + wave * 16 + gq * 4;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int tok = tt * 16 + r;
        if (tok < T) {
            float *dst = part + ((int64_t)s * T + tok) * n_out + nb;
            if (nb + 3 < n_out && (n_out & 3) == 0) {
                *(float4 *)dst = float4{acc[tt][0], acc[tt][1], acc[tt][2], acc[tt][3]};
            } else {
                for (int q = 0; q < 4; ++q)
                    if (nb + q < n_out)
                        dst[q] = acc[tt][q];
            }
        }
    }
}

DecodeCfg decode_config(int64_t T, int64_t n_in, int64_t n_out)
{
    DecodeCfg c;
    c.tt = T <= 16 ? 1 : T <= 32 ? 2 : T <= 64 ? 4 : 8;
    const int kr_max = c.tt == 8 ? 512 : 1024;
    c.n_tiles = (int)((n_out + DEC_ROWS - 1) / DEC_ROWS);
    const int64_t kblocks = (n_in + DEC_KB - 1) / DEC_KB;
    int64_t sk = std::max<int64_t>((256 + c.n_tiles - 1) / c.n_tiles,
                                   (n_in + kr_max - 1) / kr_max);
    sk = std::min<int64_t>(sk, kblocks);
    sk = std::max<int64_t>(sk, 1);
    c.kr = (int)(((kblocks + sk - 1) / sk) * DEC_KB);
    c.sk = (int)((n_in + c.kr - 1) / c.kr);
    return c;
}

size_t decode_partial_bytes(int64_t T, int64_t n_in, int64_t n_out)
{
    const DecodeCfg c = decode_config(T, n_in, n_out);
    return (size_t)c.sk * (size_t)T * (size_t)n_out * sizeof(float);
}

template <int TT>
static hipError_t launch_tt(const uint16_t *x, const uint16_t *W, int64_t T, int64_t n_in,
                            int64_t n_out, float *part, const DecodeCfg &c, const SlotGeom &g,
                            int64_t n_pairs, const int32_t *idx, int32_t K, const float *scale,
                            float *v, hipStream_t stream)
{
    const size_t lds = (size_t)16 * TT * (c.kr + 8) * sizeof(uint16_t);
    if (lds > 160 * 1024 - 1024)
        return hipErrorInvalidValue;
    static size_t lds_allowed = 64 * 1024;   // raised on demand, per instantiation
    if (lds > lds_allowed) {
        hipError_t e = hipFuncSetAttribute((const void *)decode_gemm_kernel<TT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
        lds_allowed = lds;
    }
    const unsigned grid = (unsigned)(c.n_tiles * c.sk + n_pairs);
    hipLaunchKernelGGL(decode_gemm_kernel<TT>, dim3(grid), dim3(256), lds, stream, x, W, (int)T,
                       (int)n_in, (int)n_out, part, c.kr, c.n_tiles, c.sk, g, idx, K, scale, v);
    return hipGetLastError();
}

hipError_t launch_decode_gemm(const uint16_t *x, const uint16_t *W, int64_t T, int64_t n_in,
                              int64_t n_out, float *part, const DecodeCfg &cfg,
                              const SlotGeom *g, const int32_t *idx, int32_t K,
                              const float *scale, float *v, hipStream_t stream)
{
    SlotGeom gg{};
    int64_t n_pairs = 0;
    if (g != nullptr && v != nullptr) {
        gg = *g;
        n_pairs = T * K;
    }
    switch (cfg.tt) {
    case 1: return launch_tt<1>(x, W, T, n_in, n_out, part, cfg, gg, n_pairs, idx, K, scale, v, stream);
    case 2: return launch_tt<2>(x, W, T, n_in, n_out, part, cfg, gg, n_pairs, idx, K, scale, v, stream);
    case 4: return launch_tt<4>(x, W, T, n_in, n_out, part, cfg, gg, n_pairs, idx, K, scale, v, stream);
    default: return launch_tt<8>(x, W, T, n_in, n_out, part, cfg, gg, n_pairs, idx, K, scale, v, stream);
    }
}

}  // namespace mlora
