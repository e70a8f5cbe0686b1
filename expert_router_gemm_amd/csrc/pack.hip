// pack.hip -- row-major weight matrices -> the fragment layout (frag_offset).
//
// A one-time conversion when expert weights are loaded: the expert GEMMs
// then read every 16-row x 64-byte MFMA operand tile as one contiguous 1 KB
// (see gemm_stream.hip).  A pure permutation of 16-byte units: thread u
// writes destination unit u (coalesced) and reads the source unit that
// frag_offset maps there.
#include "kernels.h"

namespace moe {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void pack_frag_kernel(const u32x4_t *__restrict__ src,
                                                        u32x4_t *__restrict__ dst, long units,
                                                        long mat_units, int row_units) {
    const int frags_per_row = row_units / 4;  // 64-byte K chunks per row
    for (long u = (long)blockIdx.x * blockDim.x + threadIdx.x; u < units;
         u += (long)gridDim.x * blockDim.x) {
        const long m = u / mat_units, w = u - m * mat_units;
        const long f = w >> 6;  // fragment within the matrix
        const int l = (int)(w & 63);
        const long i = f / frags_per_row;  // 16-row group
        const int j = (int)(f - i * frags_per_row);
        const long row = i * 16 + (l & 15);
        const int unit = j * 4 + (l >> 4);  // 16-byte unit within the row
        dst[u] = src[m * mat_units + row * row_units + unit];
    }
}

}  // namespace

hipError_t launch_pack_frag(const void *src, void *dst, long n_mats, int rows, int row_bytes,
                            hipStream_t s) {
    if (n_mats <= 0) return hipSuccess;
    if (rows <= 0 || rows % 16 || row_bytes <= 0 || row_bytes % 64) return hipErrorInvalidValue;
    const long mat_units = (long)rows * (row_bytes / 16);
    const long units = n_mats * mat_units;
    long blocks = (units + 255) / 256;
    if (blocks > 8192) blocks = 8192;  // grid-stride beyond 2M units
    hipLaunchKernelGGL(pack_frag_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const u32x4_t *>(src), reinterpret_cast<u32x4_t *>(dst),
                       units, mat_units, row_bytes / 16);
    return hipGetLastError();
}

}  // namespace moe
