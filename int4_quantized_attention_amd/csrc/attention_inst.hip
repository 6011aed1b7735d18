// One (head dimension, kv step) instance of the K2 kernels: compiled once per pair
// with -DATT_D=<64|128> -DATT_KVB=<16..256>, so that the instances build in parallel.
#include "attention_impl.h"

namespace ra {
template hipError_t launch_s<ATT_D, ATT_KVB>(const AttnArgs& a, bool dbg, hipStream_t st);
}  // namespace ra
