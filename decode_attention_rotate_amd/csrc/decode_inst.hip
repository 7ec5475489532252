// One instantiation unit of the split-K decode kernel: head_dim KVQ_INST_D and
// K width KVQ_INST_KB (set by the build), every V width and 1..8 query heads
// per KV-head chunk, plus the chunked-prefill variant per V width.  Split
// across units so the build compiles in parallel.
#include "decode_kernels.hpp"

#ifndef KVQ_INST_D
#error "KVQ_INST_D must be defined"
#endif
#ifndef KVQ_INST_KB
#error "KVQ_INST_KB must be defined"
#endif

#define KVQ_CAT2(a, b, c) a##_##b##_##c
#define KVQ_CAT(a, b, c) KVQ_CAT2(a, b, c)
#define KVQ_TABLE KVQ_CAT(kvq_decode_table, KVQ_INST_D, KVQ_INST_KB)
#define KVQ_PF_TABLE KVQ_CAT(kvq_prefill_table, KVQ_INST_D, KVQ_INST_KB)

namespace kvq {

#define KVQ_ROW(VB)                                                                \
  {launch_decode_split<KVQ_INST_D, KVQ_INST_KB, VB, 1>,                            \
   launch_decode_split<KVQ_INST_D, KVQ_INST_KB, VB, 2>,                            \
   launch_decode_split<KVQ_INST_D, KVQ_INST_KB, VB, 3>,                            \
   launch_decode_split<KVQ_INST_D, KVQ_INST_KB, VB, 4>,                            \
   launch_decode_split<KVQ_INST_D, KVQ_INST_KB, VB, 5>,                            \
   launch_decode_split<KVQ_INST_D, KVQ_INST_KB, VB, 6>,                            \
   launch_decode_split<KVQ_INST_D, KVQ_INST_KB, VB, 7>,                            \
   launch_decode_split<KVQ_INST_D, KVQ_INST_KB, VB, 8>}

DecodeLauncher KVQ_TABLE[4][8] = {KVQ_ROW(4), KVQ_ROW(5), KVQ_ROW(6), KVQ_ROW(8)};

// chunked prefill, indexed by v_bits 4/5/6/8
DecodeLauncher KVQ_PF_TABLE[4] = {launch_decode_split<KVQ_INST_D, KVQ_INST_KB, 4, 8, true>,
                                  launch_decode_split<KVQ_INST_D, KVQ_INST_KB, 5, 8, true>,
                                  launch_decode_split<KVQ_INST_D, KVQ_INST_KB, 6, 8, true>,
                                  launch_decode_split<KVQ_INST_D, KVQ_INST_KB, 8, 8, true>};

}  // namespace kvq
