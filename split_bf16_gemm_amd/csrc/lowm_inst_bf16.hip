// Kernels of one output kind (bf16) of the low-M split-K bf16 GEMM: each output
// kind is its own translation unit so that the library compiles in parallel.
#include "lowm_kernels.cuh"

namespace lowm {
void fill_table_bf16(Table& t) { fill_out<__bf16>(t, kOutBf16); }
}  // namespace lowm
