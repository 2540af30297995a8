// The binary16-activation instances of the matrix-vector kernels, compiled
// apart from the bf16 ones (swq_gemv.hip) so that the two build in parallel.
#define SWQ_GEMV_ACT 1
#include "swq_gemv.hip"
