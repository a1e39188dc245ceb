// Vector-ALU decode kernels for f32 key/value caches.
#include "decode_valu.h"

namespace pkv {
namespace valu {
template int launch_valu<PKV_F32>(const DecodeArgs&, bool, hipStream_t);
template int valu_heads_per_wg<PKV_F32>(const DecodeArgs&);
template int launch_valu_sk<PKV_F32>(const DecodeArgs&, bool, hipStream_t);
template int valu_sk_workers<PKV_F32>(const DecodeArgs&);
}  // namespace valu
}  // namespace pkv
