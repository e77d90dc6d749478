// tables.hip -- fp32 cos/sin tables for RoPE, angles formed in fp64.
//
// Row p, column i holds cos(a) and sin(a) with a = (p / pos_div) theta_i and
// theta_i = base^(-2i/rot_dim) ("Write Triton Rope Kernel", "Correctness
// requirements"; the fp64 angle follows "RoPE and FlashAttention: relative
// positions and online softmax", section 2, and pos_div > 1 is the position
// interpolation of its section 3).  Each value is rounded once, fp64 -> fp32.
// This runs once per (base, rot_dim, max_pos, pos_div), off the hot path.
#include "common.hpp"

namespace {

__global__ __launch_bounds__(256) void tables_kernel(double base, int rot_dim, double pos_div, int64_t n,
                                                     float *__restrict__ cos_out,
                                                     float *__restrict__ sin_out)
{
    const int half = rot_dim / 2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += stride) {
        const int64_t p = idx / half;
        const int i = (int)(idx - p * half);
        const double theta = pow(base, -2.0 * (double)i / (double)rot_dim);
        const double ang = ((double)p / pos_div) * theta;
        double s, c;
        sincos(ang, &s, &c);
        cos_out[idx] = (float)c;
        sin_out[idx] = (float)s;
    }
}

}  // namespace

int rope_launch_tables(double base, int rot_dim, int64_t max_pos, double pos_div, float *cos_out,
                       float *sin_out, hipStream_t stream)
{
    const int64_t n = max_pos * (rot_dim / 2);
    const int threads = 256;
    int64_t blocks = (n + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;   // grid-stride loop covers the rest
    hipLaunchKernelGGL(tables_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, base,
                       rot_dim, pos_div, n, cos_out, sin_out);
    return hipGetLastError() == hipSuccess ? ROPE_LAUNCH_OK : ROPE_LAUNCH_ERR;
}
