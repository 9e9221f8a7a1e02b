// Instantiation unit for the expert GEMV launchers. The build compiles this
// file several times with -DSMOE_INST_BITS=<2|4> -DSMOE_INST_ST=<float|_Float16>
// -DSMOE_INST_VLO=<n> -DSMOE_INST_VHI=<n> so the instantiations compile in
// parallel.

#include "smoe_gemv.hpp"

#ifndef SMOE_INST_BITS
#error "SMOE_INST_BITS not set"
#endif

namespace smoe {

#define SMOE_INST(n)                                                                      \
  template hipError_t launch_gu<SMOE_INST_BITS, SMOE_INST_ST, n>(const GemvArgs&, int,    \
                                                                 dim3, unsigned,          \
                                                                 hipStream_t);            \
  template hipError_t launch_dn<SMOE_INST_BITS, SMOE_INST_ST, n>(const GemvArgs&, dim3,   \
                                                                 unsigned, hipStream_t);

#if SMOE_INST_VLO <= 1 && 1 <= SMOE_INST_VHI
SMOE_INST(1)
#endif
#if SMOE_INST_VLO <= 2 && 2 <= SMOE_INST_VHI
SMOE_INST(2)
#endif
#if SMOE_INST_VLO <= 3 && 3 <= SMOE_INST_VHI
SMOE_INST(3)
#endif
#if SMOE_INST_VLO <= 4 && 4 <= SMOE_INST_VHI
SMOE_INST(4)
#endif
#if SMOE_INST_VLO <= 5 && 5 <= SMOE_INST_VHI
SMOE_INST(5)
#endif
#if SMOE_INST_VLO <= 6 && 6 <= SMOE_INST_VHI
SMOE_INST(6)
#endif
#if SMOE_INST_VLO <= 7 && 7 <= SMOE_INST_VHI
SMOE_INST(7)
#endif
#if SMOE_INST_VLO <= 8 && 8 <= SMOE_INST_VHI
SMOE_INST(8)
#endif
#if SMOE_INST_VLO <= 9 && 9 <= SMOE_INST_VHI
SMOE_INST(9)
#endif
#if SMOE_INST_VLO <= 10 && 10 <= SMOE_INST_VHI
SMOE_INST(10)
#endif
#if SMOE_INST_VLO <= 11 && 11 <= SMOE_INST_VHI
SMOE_INST(11)
#endif
#if SMOE_INST_VLO <= 12 && 12 <= SMOE_INST_VHI
SMOE_INST(12)
#endif
#if SMOE_INST_VLO <= 13 && 13 <= SMOE_INST_VHI
SMOE_INST(13)
#endif
#if SMOE_INST_VLO <= 14 && 14 <= SMOE_INST_VHI
SMOE_INST(14)
#endif
#if SMOE_INST_VLO <= 15 && 15 <= SMOE_INST_VHI
SMOE_INST(15)
#endif
#if SMOE_INST_VLO <= 16 && 16 <= SMOE_INST_VHI
SMOE_INST(16)
#endif

}  // namespace smoe
