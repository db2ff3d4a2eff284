// Definitions of the GEMM kernels with E4M3 A and E5M2 B operands (tiled, few-rows and
// packed-segment kernels); the other translation units only declare them.
#define DG_DEFINE_FMT_45
#include "gemm_f16mma.hpp"
#include "gemm_skinny.hpp"
#include "gemm_sharedb.hpp"
