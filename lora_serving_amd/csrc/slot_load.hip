// Slot activation: the zero padding of an adapter loaded into a slot of width R.
//
// "Multi-LoRA Serving Explained" (sevydevy.com), memory script and padding example: every
// resident slot is sized for max_lora_rank R, and an adapter of rank r < R occupies the first
// r rows of the slot's A (per slice) and the first r columns of its B, the rest being zero, so
// that the padded product equals the unpadded one.  The copies of the r rows / columns are
// plain asynchronous copies issued by the host; this kernel writes the zeros around them and
// the slot's scale factor.
#include "common.h"
#include "kernels.h"

namespace mlora {

// Zeroes A rows [r, R) of every slice ([n_slices][R][n_in] from A_slot) and B columns [r, R)
// of every row ([n_out][R] from B_slot); thread 0 writes *factor = f.  Grid-stride loop over
// the padding elements (A part first, then B).
__global__ __launch_bounds__(256) void slot_pad_kernel(uint16_t *A_slot, uint16_t *B_slot,
                                                       float *factor, int R, int r, int n_slices,
                                                       int64_t n_in, int64_t n_out, float f)
{
    const int64_t pad = R - r;
    const int64_t na = (int64_t)n_slices * pad * n_in;   // contiguous per slice: pad * n_in
    const int64_t nb = n_out * pad;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < na + nb; e += stride) {
        if (e < na) {
            const int64_t s = e / (pad * n_in);
            const int64_t rest = e - s * pad * n_in;
            A_slot[(s * R + r) * n_in + rest] = 0;
        } else {
            const int64_t b = e - na;
            const int64_t n = b / pad;
            B_slot[n * R + r + (b - n * pad)] = 0;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *factor = f;
}

hipError_t launch_slot_pad(uint16_t *A_slot, uint16_t *B_slot, float *factor, int32_t R,
                           int32_t r, int32_t n_slices, int64_t n_in, int64_t n_out, float f,
                           hipStream_t stream)
{
    const int64_t n = (int64_t)n_slices * (R - r) * n_in + n_out * (R - r);
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 2048));
    hipLaunchKernelGGL(slot_pad_kernel, dim3(grid), dim3(256), 0, stream, A_slot, B_slot, factor,
                       (int)R, (int)r, (int)n_slices, n_in, n_out, f);
    return hipGetLastError();
}

}  // namespace mlora
