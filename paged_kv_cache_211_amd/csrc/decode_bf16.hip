// Vector-ALU decode kernels for bf16 key/value caches.
#include "decode_valu.h"

namespace pkv {
namespace valu {
template int launch_valu<PKV_BF16>(const DecodeArgs&, bool, hipStream_t);
template int valu_heads_per_wg<PKV_BF16>(const DecodeArgs&);
template int launch_valu_sk<PKV_BF16>(const DecodeArgs&, bool, hipStream_t);
template int valu_sk_workers<PKV_BF16>(const DecodeArgs&);
}  // namespace valu
}  // namespace pkv
