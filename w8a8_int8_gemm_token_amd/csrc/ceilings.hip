// ceilings.hip -- measurement kernels for the benchmark, built into
// libq8_ceilings.so beside the library.  They compute nothing of the layer;
// they measure what this board sustains, so that the layer's kernels can be
// compared with a ceiling measured in the same run as well as with the
// datasheet peaks (INT8 dense MFMA, HBM bandwidth):
//
//  q8c_mfma_i8_loop  -- back-to-back v_mfma_i32_32x32x32_i8 from registers,
//                       no memory traffic.  With `random` set the operands
//                       are 8 distinct fragments per wave filled from a
//                       counter-based hash, and every MFMA takes a different
//                       one, so the matrix core sees changing data as it does
//                       in a GEMM (the board's clock depends on it); with
//                       `random` clear every operand is zero.
//  q8c_stream_read   -- a plain coalesced read of a buffer with 16-byte
//                       non-temporal loads (the weight-streaming kernels'
//                       load form), one running xor per thread written out so
//                       the loads are kept.
//
// Both take a stream and return the HIP launch status; they allocate
// nothing.  Timing is the caller's (events around the launches).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    // a 32-bit finalizer (multiply-xorshift); only its spread matters here
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// Each wave: 4 independent accumulator chains, NF operand fragments in
// registers; step j issues 4 MFMAs, chain c on fragments (j + c) % NF and
// (j + c + 1) % NF.  About 100 registers: four waves per SIMD stay resident.
template <int NF>
__global__ __launch_bounds__(256) void mfma_i8_loop_kernel(int iters, int random, int* out) {
    v4i f[NF];
    const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 131u;
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) f[j][e] = random ? (int)mix32(seed + 4u * j + e) : 0;
    v16i acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = v16i{};
    for (int i = 0; i < iters; i += NF) {
#pragma unroll
        for (int j = 0; j < NF; ++j) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[(j + c) % NF], f[(j + c + 1) % NF], acc[c], 0,
                                                               0, 0);
        }
    }
    int s = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) s ^= acc[c][e];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

// The same loop on v_mfma_i32_16x16x64_i8 (the prefill GEMM's form): eight
// independent chains, each MFMA 16 x 16 x 64.
template <int NF>
__global__ __launch_bounds__(256) void mfma_i8_loop16_kernel(int iters, int random, int* out) {
    v4i f[NF];
    const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 131u;
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) f[j][e] = random ? (int)mix32(seed + 4u * j + e) : 0;
    v4i acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = v4i{};
    for (int i = 0; i < iters; i += NF) {
#pragma unroll
        for (int j = 0; j < NF; ++j) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
                acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f[(j + c) % NF], f[(j + c + 1) % NF], acc[c], 0,
                                                               0, 0);
        }
    }
    int s = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) s ^= acc[c][e];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void stream_read_kernel(const v4i* __restrict__ p, int64_t n16,
                                                          int* out) {
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    v4i a = v4i{0, 0, 0, 0};
    int64_t i = tid;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const v4i x0 = __builtin_nontemporal_load(p + i);
        const v4i x1 = __builtin_nontemporal_load(p + i + stride);
        const v4i x2 = __builtin_nontemporal_load(p + i + 2 * stride);
        const v4i x3 = __builtin_nontemporal_load(p + i + 3 * stride);
        a ^= x0 ^ x1 ^ x2 ^ x3;
    }
    for (; i < n16; i += stride) a ^= __builtin_nontemporal_load(p + i);
    out[tid] = a[0] ^ a[1] ^ a[2] ^ a[3];
}

}  // namespace

extern "C" {

// MFMA loop: `blocks` workgroups of 4 waves (256 threads), each wave
// `iters` steps of 4 MFMAs (iters a multiple of 8).  One MFMA is
// 2 * 32 * 32 * 32 = 65,536 int8 operations.  out: int32 [blocks * 256].
int q8c_mfma_i8_loop(int blocks, int iters, int random, int* out, void* stream) {
    if (blocks <= 0 || iters <= 0 || iters % 8 != 0 || !out) return 1;
    hipLaunchKernelGGL((mfma_i8_loop_kernel<8>), dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters,
                       random, out);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

// Streaming read of `bytes` bytes at p (16-byte aligned, bytes a multiple
// of 16) by `blocks` workgroups of 256 threads.  out: int32 [blocks * 256].
// iters 16x16x64 MFMAs on each of 8 chains per wave
int q8c_mfma_i8_loop16(int blocks, int iters, int random, int* out, void* stream) {
    if (blocks <= 0 || iters <= 0 || iters % 8 != 0 || !out) return 1;
    hipLaunchKernelGGL((mfma_i8_loop16_kernel<8>), dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters,
                       random, out);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

int q8c_stream_read(const void* p, int64_t bytes, int blocks, int* out, void* stream) {
    if (!p || !out || bytes <= 0 || bytes % 16 != 0 || blocks <= 0 || ((uintptr_t)p & 15) != 0) return 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const v4i*>(p), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
