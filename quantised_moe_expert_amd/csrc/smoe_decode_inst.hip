// Instantiation unit for the batch-1 layer kernels; compiled once per (bits,
// scale type) with -DSMOE_INST_BITS and -DSMOE_INST_ST.

#include "smoe_decode.hpp"
#include "smoe_small.hpp"

#ifndef SMOE_INST_BITS
#error "SMOE_INST_BITS not set"
#endif

namespace smoe {

#define SMOE_DEC_INST_G(vg)                                                                  \
  template hipError_t launch_dec_gate_up<SMOE_INST_BITS, SMOE_INST_ST, vg, false>(           \
      const DecodeArgs&, int, hipStream_t);                                                   \
  template hipError_t launch_dec_gate_up<SMOE_INST_BITS, SMOE_INST_ST, vg, true>(            \
      const DecodeArgs&, int, hipStream_t);                                                   \
  template hipError_t launch_sb_gate_up<SMOE_INST_BITS, SMOE_INST_ST, vg, false>(            \
      const SmallArgs&, int, hipStream_t);                                                    \
  template hipError_t launch_sb_gate_up<SMOE_INST_BITS, SMOE_INST_ST, vg, true>(             \
      const SmallArgs&, int, hipStream_t);
#define SMOE_DEC_INST_D(vd)                                                                  \
  template hipError_t launch_dec_down<SMOE_INST_BITS, SMOE_INST_ST, vd>(const DecodeArgs&,  \
                                                                         int, hipStream_t); \
  template hipError_t launch_sb_down<SMOE_INST_BITS, SMOE_INST_ST, vd>(const SmallDownArgs&, \
                                                                        int, hipStream_t);

#if SMOE_INST_BITS == 4
SMOE_DEC_Q4_VG(SMOE_DEC_INST_G)
SMOE_DEC_Q4_VD(SMOE_DEC_INST_D)
#else
SMOE_DEC_Q2_VG(SMOE_DEC_INST_G)
SMOE_DEC_Q2_VD(SMOE_DEC_INST_D)
#endif

}  // namespace smoe
