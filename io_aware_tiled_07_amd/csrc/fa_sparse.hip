// Block-sparse attention: the caller's block mask (one byte per 128 x 128
// block of the score matrix, nonzero = computed) packed into bit rows and bit
// columns, the form the attention kernels walk (fa_device.h, BlockWalk).
//
// The block-sparse extension is named by the michaelc-yu summary of Dao et
// al. (abstract) without a definition; the reading taken: the same exact
// attention with every pair (i, j) whose block is not kept masked out, so a
// kernel skips the dropped blocks' tiles entirely.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

// One wave per 64-bit word, one lane per bit: word w of row r of mask m
// collects blocks (r, 64 w + lane); word w of column r collects blocks
// (64 w + lane, r). Every lane issues its one byte load at once, so a word
// costs one memory latency.
__global__ __launch_bounds__(256) void mask_bits_kernel(const uint8_t* __restrict__ mask, int64_t head_stride,
                                                        int nm, int nb, int W, uint64_t* __restrict__ rows,
                                                        uint64_t* __restrict__ cols) {
    const int64_t per = (int64_t)nb * W;  // words per mask
    const int64_t t = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (t >= 2 * nm * per) return;  // whole waves leave together
    const bool col = t >= nm * per;
    const int64_t u = col ? t - nm * per : t;
    const int64_t m = u / per;
    const int r = (int)((u % per) / W), x = (int)(u % W) * 64 + lane;
    const uint8_t* __restrict__ base = mask + m * head_stride;
    bool keep = false;
    if (x < nb) keep = (col ? base[(int64_t)x * nb + r] : base[(int64_t)r * nb + x]) != 0;
    const uint64_t bits = __ballot(keep);
    if (lane == 0) (col ? cols : rows)[u] = bits;
}

}  // namespace

hipError_t sparse_mask_bits(const uint8_t* mask, int64_t head_stride, int nm, int nb, uint64_t* rows, uint64_t* cols,
                            hipStream_t stream) {
    const int W = (nb + 63) / 64;
    const int64_t words = 2 * (int64_t)nm * nb * W;  // one wave each, four per workgroup
    const dim3 grid((unsigned)((words + 3) / 4));
    hipLaunchKernelGGL(mask_bits_kernel, grid, dim3(256), 0, stream, mask, head_stride, nm, nb, W, rows, cols);
    return hipGetLastError();
}

}  // namespace fa
