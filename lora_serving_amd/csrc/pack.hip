// Packed weight layout for the matrix cores.
//
// The v_mfma_f32_16x16x32_bf16 A operand takes, in lane l, 8 values of row l % 16 at k-chunk
// l / 16 of a 16 x 32 block.  Read straight from a row-major W, one load instruction for such
// a fragment touches 16 rows with 64 bytes each; in the packed layout the fragment is 1 KB
// contiguous in lane order, so the same instruction reads 8 whole cache lines.  Packing is a
// one-time relayout of a static weight (done when the weight is loaded), not part of the
// layer's computation:
//   Wp[rg][kb][lane][e] = W[16 rg + lane % 16][32 kb + 8 (lane / 16) + e]
// with rg < ceil(n_out / 16), kb < ceil(n_in / 32), zeros past n_out and n_in.
#include "common.h"
#include "kernels.h"

namespace mlora {

int64_t packed_weight_elems(int64_t n_out, int64_t n_in)
{
    return ((n_out + 15) / 16) * 16 * ((n_in + 31) / 32) * 32;
}

// one thread per 16-byte chunk of the packed buffer
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint16_t *__restrict__ W,
                                                          int64_t n_out, int64_t n_in,
                                                          int64_t n_kb, int64_t n_chunks,
                                                          uint16_t *__restrict__ Wp)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n_chunks; q += stride) {
        const int lane = (int)(q & 63);
        const int64_t frag = q >> 6;                  // rg * n_kb + kb
        const int64_t rg = frag / n_kb, kb = frag - rg * n_kb;
        const int64_t n = rg * 16 + (lane & 15);
        const int64_t k = kb * 32 + (lane >> 4) * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (n < n_out && k < n_in)                    // n_in is a multiple of 8: whole chunks
            v = *(const u32x4 *)(W + n * n_in + k);
        *(u32x4 *)(Wp + q * 8) = v;
    }
}

hipError_t launch_pack_weight(const uint16_t *W, int64_t n_out, int64_t n_in, uint16_t *Wp,
                              hipStream_t stream)
{
    const int64_t n_kb = (n_in + 31) / 32;
    const int64_t n_chunks = packed_weight_elems(n_out, n_in) / 8;
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n_chunks + 255) / 256, 8192));
    hipLaunchKernelGGL(pack_weight_kernel, dim3(grid), dim3(256), 0, stream, W, n_out, n_in, n_kb,
                       n_chunks, Wp);
    return hipGetLastError();
}

}  // namespace mlora
