// SwiGLU between the gate_up and down matrices of a layer.
//
// The pages do not spell out the layer's non-GEMM steps; the round's shapes
// do: the fused gate_up matrix has N = 2 F outputs and the down matrix takes
// K = F (34816 = 2 x 17408).  The plainest reading is the gated MLP of the
// model family: h = silu(gate) * up with silu(g) = g / (1 + exp(-g)), gate
// the first F outputs and up the second.  With it, down consumes what gate_up
// produced, so the two GEMMs of a round are a dependent chain as in a real
// forward pass ("Ignis" README, "The decode round").
//
// Precision: each h is computed in fp64 from the bf16 inputs and rounded once
// to bf16 (nearest, ties to even, no intermediate fp32), so the result is the
// correctly rounded value except when fp64 rounding error moves it across a
// bf16 rounding boundary (relative distance 2^-52 against 2^-9).
#include "swiglu_device.h"

namespace nvfp4 {

// h[m][j] = silu(gu[m][j]) * gu[m][F + j]; one thread per output.
__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t* __restrict__ gu,
                                                     uint16_t* __restrict__ h, int M, int F) {
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    if (t >= (long long)M * F) return;
    const int m = (int)(t / F), j = (int)(t - (long long)m * F);
    h[(size_t)m * F + j] = swiglu_bf16(gu[(size_t)m * 2 * F + j], gu[(size_t)m * 2 * F + F + j]);
}

int launch_swiglu(const uint16_t* gu, uint16_t* h, int M, int F, hipStream_t s) {
    const long long n = (long long)M * F;
    hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, gu, h,
                       M, F);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" int nvfp4_swiglu(const uint16_t* gate_up_dev, int M, int F, uint16_t* out_dev,
                            void* stream) {
    clear_error();
    if (M < 1) return set_error(NVFP4_EINVAL, "M: %d < 1", M);
    if (F < 1) return set_error(NVFP4_EINVAL, "F: %d < 1", F);
    if ((long long)M * 2 * F > 0x7FFFFFFF)
        return set_error(NVFP4_EINVAL, "M * 2F: more than 2^31 - 1 elements");
    if (!gate_up_dev) return set_error(NVFP4_EINVAL, "gate_up: NULL");
    if (!out_dev) return set_error(NVFP4_EINVAL, "out: NULL");
    if (((uintptr_t)gate_up_dev | (uintptr_t)out_dev) & 1)
        return set_error(NVFP4_EINVAL, "gate_up/out: not 2-byte aligned");
    return launch_swiglu(gate_up_dev, out_dev, M, F, (hipStream_t)stream);
}
