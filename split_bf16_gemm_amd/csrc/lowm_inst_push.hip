// Kernels of one output kind (push) of the low-M split-K bf16 GEMM: each output
// kind is its own translation unit so that the library compiles in parallel.
#include "lowm_kernels.cuh"

namespace lowm {
void fill_table_push(Table& t) { fill_out<PushBf16>(t, kOutPush); }
}  // namespace lowm
