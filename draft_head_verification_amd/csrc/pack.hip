// pack.hip -- one-off layout conversion of the Markov head's right factor.
//
// The pages describe the head as a rank-r factorisation of a token-to-token bias (QbitAI "DSpark
// in 10 concepts", section "Cheaper serial module: the Markov head"): bias = U[prev] . W with W
// of shape r x V.  The drafting and verifying kernels read W as [V][r] (row v = column v of the
// r x V factor), the layout of an output-projection weight, so that both matrix-core operands
// are contiguous along r.  W is a weight: a caller that holds it as r x V converts it once,
// when the weights are loaded, with dspark_pack_w, not per round.
//
// Tiled transpose through LDS: a workgroup moves a 64 x 64 tile, reading 64 consecutive
// vocabulary entries of 64 rank rows (coalesced along V) and writing 64 consecutive rank
// entries of 64 vocabulary rows (coalesced along r); the tile is padded by one element per
// row so that the transposed reads hit distinct banks.
#include "dspark_common.hpp"

namespace dspark {

constexpr int kPackTile = 64;

template <typename T>
__global__ __launch_bounds__(256) void pack_w_kernel(const T *__restrict__ src, T *__restrict__ dst,
                                                     int r, int V) {
    __shared__ T tile[kPackTile][kPackTile + 1];
    const int v0 = blockIdx.x * kPackTile, i0 = blockIdx.y * kPackTile;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4 threads
    for (int i = ty; i < kPackTile; i += 4) {
        const int ri = i0 + i, v = v0 + tx;
        if (ri < r && v < V) tile[i][tx] = src[(size_t)ri * V + v];
    }
    __syncthreads();
    for (int j = ty; j < kPackTile; j += 4) {
        const int v = v0 + j, ri = i0 + tx;
        if (v < V && ri < r) dst[(size_t)v * r + ri] = tile[tx][j];
    }
}

hipError_t launch_pack_w(const void *w_rv, void *w_vr, int r, int V, int dtype, hipStream_t s) {
    const dim3 grid((unsigned)((V + kPackTile - 1) / kPackTile),
                    (unsigned)((r + kPackTile - 1) / kPackTile));
    if (dtype == DSPARK_BF16)
        pack_w_kernel<uint16_t><<<grid, 256, 0, s>>>(reinterpret_cast<const uint16_t *>(w_rv),
                                                    reinterpret_cast<uint16_t *>(w_vr), r, V);
    else
        pack_w_kernel<float><<<grid, 256, 0, s>>>(reinterpret_cast<const float *>(w_rv),
                                                 reinterpret_cast<float *>(w_vr), r, V);
    return hipGetLastError();
}

}  // namespace dspark
