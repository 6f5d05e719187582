// Kernels of one output kind (f32) of the low-M split-K bf16 GEMM: each output
// kind is its own translation unit so that the library compiles in parallel.
#include "lowm_kernels.cuh"

namespace lowm {
void fill_table_f32(Table& t) { fill_out<float>(t, kOutF32); }
}  // namespace lowm
