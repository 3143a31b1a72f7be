// moe_dequant: the 4-bit affine decode of the GEMM kernels (dequant8_bf16),
// applied to a whole matrix.  Inspection and test export only -- the layer
// itself never writes decoded weights to memory (Lily pages: the 4-bit
// weights are unpacked tile by tile inside the matrix multiply, page
// "Perplexity's Lily Beats MLX-LM by 1.35x Running Qwen3.6 on Apple
// Silicon", section "Prefill optimizations").
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// one thread per 8 consecutive codes (one dword, inside one group)
__global__ void dequant_kernel(moe_qmat m, int rows, int cols, int G, uint16_t *__restrict__ out)
{
    const int64_t per_row = cols >> 3;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)rows * per_row) return;
    const int64_t n = i / per_row;
    const int c8 = (int)(i - n * per_row) * 8;
    const uint32_t v = reinterpret_cast<const uint32_t *>(m.q + n * (cols >> 1))[c8 >> 3];
    const int64_t gi = n * (cols / G) + c8 / G;
    uint32_t o[4];
    dequant8_bf16(v, bf16_to_f32(m.s[gi]), bf16_to_f32(m.b[gi]), o);
    *reinterpret_cast<uint4 *>(out + n * cols + c8) = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_dequant(const moe_qmat &m, int rows, int cols, int G, uint16_t *out, hipStream_t s)
{
    const int64_t n = (int64_t)rows * (cols >> 3);
    if (n == 0) return hipSuccess;
    const int threads = 256;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((n + threads - 1) / threads)), dim3(threads), 0,
                       s, m, rows, cols, G, out);
    return hipGetLastError();
}

}  // namespace moe
