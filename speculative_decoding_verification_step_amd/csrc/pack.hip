// Packing of bf16 weights into the MFMA-tiled layout.
//
// The verification forward is bound by streaming the weights from HBM once
// per step.  In row-major order, the 16 weight rows that one matrix-core
// operand needs are 16 separate 64-byte pieces per load instruction; in the
// tiled layout each 16 x 32 operand block is one contiguous KiB, stored in the
// exact lane order of the v_mfma_f32_16x16x32_bf16 A operand, so every wave
// load is a single contiguous KiB.
//
// Layout of a [rows, cols] matrix (cols % 32 == 0), rows padded with zeros to
// a multiple of 16:  tile (rt, s) for rt < ceil(rows/16), s < cols/32 starts at
// element (rt * cols/32 + s) * 512; lane l = r + 16 q (r < 16, q < 4) holds
// elements l*8 .. l*8+7 of the tile = W[rt*16 + r][s*32 + 8q + e], e = 0..7.
#include "common.hpp"
#include "kernels.hpp"

namespace sv {

namespace {

__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ src,
                                                   uint16_t* __restrict__ dst, int rows, int cols,
                                                   size_t chunks_per_matrix) {
    const size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    const size_t mat = blockIdx.y;
    if (t >= chunks_per_matrix) return;
    const int S = cols / 32;
    const size_t tile = t / 64;
    const int lane = (int)(t % 64);
    const size_t rt = tile / S;
    const int s = (int)(tile % S);
    const size_t row = rt * 16 + (lane & 15);
    const int col = s * 32 + 8 * (lane >> 4);
    const size_t in_elems = (size_t)rows * cols;
    const size_t out_elems = chunks_per_matrix * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < (size_t)rows)
        v = *reinterpret_cast<const u32x4*>(src + mat * in_elems + row * cols + col);
    *reinterpret_cast<u32x4*>(dst + mat * out_elems + t * 8) = v;
}

}  // namespace

size_t tiled_elems(int rows, int cols) { return (size_t)((rows + 15) / 16) * 16 * cols; }

hipError_t launch_pack(const uint16_t* src, uint16_t* dst, int rows, int cols, int count,
                       hipStream_t stream) {
    if (rows <= 0 || count <= 0) return hipSuccess;
    const size_t chunks = tiled_elems(rows, cols) / 8;
    const dim3 grid((unsigned)((chunks + 255) / 256), (unsigned)count);
    ProfScope prof("pack_weights", stream, 2.0 * count * (double)rows * cols * 2, 0.0);
    SV_LAUNCH(prof, pack_kernel, grid, 256, stream, src, dst, rows, cols, chunks);
    return hipGetLastError();
}

}  // namespace sv
