// Test entry point: whole matrices decoded through the same device path as the projections
// (decode8 + the exact LDS tables), written in natural K order.
#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, int E,
                                                      int N, int K, const uint8_t* table_id,
                                                      TableArgs ta, uint16_t* __restrict__ out) {
    extern __shared__ u32x4 tab[];
    build_decode_tables(ta, tab);
    const size_t dw_per_row = (size_t)K / 8;
    const size_t total = (size_t)E * N * dw_per_row;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const size_t row = i / dw_per_row;
        const int dd = (int)(i % dw_per_row);
        const int e = (int)(row / N);
        const int tsel = table_id[e];
        const uint32_t c = *reinterpret_cast<const uint32_t*>(codes + row * (K / 2) + dd * 4);
        const int s = scales[row * (K / 32) + dd / 4];
        u32x4 v;
        if (tsel >= ta.n) {
            v = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
        } else {
            v = pair_join(decode8(c, tab[tsel * 256 + s]));
        }
        *reinterpret_cast<u32x4*>(out + row * K + (size_t)dd * 8) = v;
    }
}

void launch_dequant(const uint8_t* codes, const uint8_t* scales, int E, int N, int K,
                    const uint8_t* table_id, const TableArgs& ta, uint16_t* out, int blocks,
                    hipStream_t stream) {
    const size_t lds = (size_t)ta.n * 256 * sizeof(u32x4);
    hipLaunchKernelGGL(dequant_kernel, dim3(blocks), dim3(256), lds, stream, codes, scales, E, N,
                       K, table_id, ta, out);
}

}  // namespace moeq
