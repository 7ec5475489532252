// One instantiation unit of the split-K decode kernel: head_dim KVQ_INST_D,
// K width KVQ_INST_KB and K block kind KVQ_INST_KM (1: scale-and-min), set by
// the build; every V format and 1..8 query heads per KV-head chunk, plus the
// chunked-prefill variant per V format.  Split across units so the build
// compiles in parallel.
#include "decode_kernels.hpp"

#ifndef KVQ_INST_D
#error "KVQ_INST_D must be defined"
#endif
#ifndef KVQ_INST_KB
#error "KVQ_INST_KB must be defined"
#endif
#ifndef KVQ_INST_KM
#error "KVQ_INST_KM must be defined"
#endif

#define KVQ_CAT2(a, b, c, d) a##_##b##_##c##_##d
#define KVQ_CAT(a, b, c, d) KVQ_CAT2(a, b, c, d)

namespace kvq {

constexpr bool kKM = KVQ_INST_KM != 0;

// head_dim 256 builds the contiguous and the paged layouts as separate
// kernels (KVQ_INST_PAGED selects the paged tables); other sizes decide the
// layout at run time.
#if KVQ_INST_D == 256
#ifdef KVQ_INST_PAGED
constexpr int kPGM = kPagePaged;
#define KVQ_TABLE KVQ_CAT(kvq_decode_ptable, KVQ_INST_D, KVQ_INST_KB, KVQ_INST_KM)
#define KVQ_PF_TABLE KVQ_CAT(kvq_prefill_ptable, KVQ_INST_D, KVQ_INST_KB, KVQ_INST_KM)
#else
constexpr int kPGM = kPageFlat;
#endif
#else
constexpr int kPGM = kPageAny;
#endif
#ifndef KVQ_TABLE
#define KVQ_TABLE KVQ_CAT(kvq_decode_table, KVQ_INST_D, KVQ_INST_KB, KVQ_INST_KM)
#define KVQ_PF_TABLE KVQ_CAT(kvq_prefill_table, KVQ_INST_D, KVQ_INST_KB, KVQ_INST_KM)
#endif

#define KVQ_L(VB, VM, G) launch_decode_split<KVQ_INST_D, KVQ_INST_KB, VB, G, false, kKM, VM, kPGM>
#define KVQ_ROW(VB, VM) \
  {KVQ_L(VB, VM, 1), KVQ_L(VB, VM, 2), KVQ_L(VB, VM, 3), KVQ_L(VB, VM, 4), \
   KVQ_L(VB, VM, 5), KVQ_L(VB, VM, 6), KVQ_L(VB, VM, 7), KVQ_L(VB, VM, 8)}

// V formats in the order q4_0, q5_0, q6_0, q8_0, q4_1, q5_1
DecodeLauncher KVQ_TABLE[6][8] = {KVQ_ROW(4, false), KVQ_ROW(5, false), KVQ_ROW(6, false),
                                  KVQ_ROW(8, false), KVQ_ROW(4, true), KVQ_ROW(5, true)};

// outlier-channel kernels (head_dim 128, absmax K and V): V q4_0..q8_0
#if KVQ_INST_D == 128 && KVQ_INST_KM == 0
#define KVQ_OTABLE KVQ_CAT(kvq_decode_otable, KVQ_INST_D, KVQ_INST_KB, KVQ_INST_KM)
#define KVQ_LO(VB, G) launch_decode_split<KVQ_INST_D, KVQ_INST_KB, VB, G, false, false, false, kPGM, true>
#define KVQ_OROW(VB) \
  {KVQ_LO(VB, 1), KVQ_LO(VB, 2), KVQ_LO(VB, 3), KVQ_LO(VB, 4), \
   KVQ_LO(VB, 5), KVQ_LO(VB, 6), KVQ_LO(VB, 7), KVQ_LO(VB, 8)}
DecodeLauncher KVQ_OTABLE[4][8] = {KVQ_OROW(4), KVQ_OROW(5), KVQ_OROW(6), KVQ_OROW(8)};
#endif

// chunked prefill, same V order
#define KVQ_P(VB, VM) launch_decode_split<KVQ_INST_D, KVQ_INST_KB, VB, 8, true, kKM, VM, kPGM>
DecodeLauncher KVQ_PF_TABLE[6] = {KVQ_P(4, false), KVQ_P(5, false), KVQ_P(6, false),
                                  KVQ_P(8, false), KVQ_P(4, true), KVQ_P(5, true)};

}  // namespace kvq
