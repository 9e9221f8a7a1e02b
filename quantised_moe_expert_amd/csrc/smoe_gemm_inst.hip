// Instantiation unit for the matrix-core stage; compiled once per (bits,
// scale type) with -DSMOE_INST_BITS and -DSMOE_INST_ST.

#include "smoe_gemm.hpp"

#ifndef SMOE_INST_BITS
#error "SMOE_INST_BITS not set"
#endif

namespace smoe {

template hipError_t launch_gm<SMOE_INST_BITS, SMOE_INST_ST>(const GemvArgs&, bool, int, int,
                                                            dim3, unsigned, hipStream_t);
template hipError_t launch_gm_ks<SMOE_INST_BITS, SMOE_INST_ST>(const GemvArgs&, bool, dim3,
                                                               hipStream_t);

}  // namespace smoe
