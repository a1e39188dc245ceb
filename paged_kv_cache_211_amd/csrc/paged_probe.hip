// Paged read probe (a measurement aid): the vector-ALU split-K decode's
// memory reads without its arithmetic (shapes the matrix-core kernel serves
// go to its own probe, decode_mfma.hip).  Same grid, same workgroup order,
// same item mapping (locate), same block-table walk and tile ring
// (tile_loop): every key and value tile the decode reads is read here, and
// only folded into a checksum.  Timing it gives the rate this access
// pattern -- 1 KiB-contiguous loads of scattered blocks through the block
// table -- reaches on the device, the ceiling of a decode kernel that
// streams the cache this way ("Memory Systems" notes, core idea 1: judge an
// HBM-bound kernel by the bytes it moves).

#include "decode_valu.h"

namespace pkv {
namespace {

using namespace dec;

template <int KV, int D, int BS, int HPW, int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) void paged_read_probe_kernel(const DecodeArgs a,
                                                                   uint32_t* __restrict__ sink) {
  using Gm = valu::Geo<KV, D, BS>;
  constexpr int NLOAD = Gm::NLOAD, TILE = Gm::TILE;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nhg = a.Hkv * (a.Hq / a.Hkv / HPW);
  const Work wk = locate<true, BS>(a, HPW, lane, blockIdx.x / nhg, blockIdx.x % nhg);
  bool bad = wk.bad;
  const int32_t* __restrict__ tbl = a.tables + (size_t)wk.s * a.max_blocks;
  const size_t head_off = (size_t)wk.hkv * TILE;
  uint32_t acc = 0;
  tile_loop<NBUF, NLOAD, NW>(tbl, wk.t0 / BS + w, wk.jend, a.nb,
                             (const uint8_t*)a.kc + head_off + lane * 16,
                             (const uint8_t*)a.vc + head_off + lane * 16, (size_t)a.Hkv * TILE,
                             lane, bad, [&](int, const u32x4* kr, const u32x4* vr) {
#pragma unroll
                               for (int l = 0; l < NLOAD; ++l)
                                 acc ^= kr[l].x ^ kr[l].y ^ kr[l].z ^ kr[l].w ^ vr[l].x ^
                                        vr[l].y ^ vr[l].z ^ vr[l].w;
                             });
  // a store only on a checksum nobody expects: the loads cannot be dropped
  if (acc == 0x9e3779b9u && !bad) sink[0] = acc;
}

template <int KV>
int launch_probe_t(const DecodeArgs& a, uint32_t* sink, hipStream_t st) {
  return valu::with_shape<KV>(a, [&](auto d, auto bs, auto h) {
    constexpr int D = decltype(d)::value, BS = decltype(bs)::value, HPW = decltype(h)::value;
    constexpr int NBUF = valu_bufs<HPW, valu::Geo<KV, D, BS>::TILE>();
    const int groups = a.Hq / a.Hkv / HPW;
    dim3 block(kWaves * 64), grid(a.total_parts * a.Hkv * groups);
    hipLaunchKernelGGL((paged_read_probe_kernel<KV, D, BS, HPW, kWaves, NBUF>), grid, block, 0, st,
                       a, sink);
    return (int)hipGetLastError();
  });
}

}  // namespace

int launch_paged_read_probe(const DecodeArgs& a, uint32_t* sink, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (decode_mfma_eligible(a)) return launch_paged_read_probe_mfma(a, sink, stream);
  switch (a.kv_dtype) {
    case PKV_F32: return launch_probe_t<PKV_F32>(a, sink, st);
    case PKV_BF16: return launch_probe_t<PKV_BF16>(a, sink, st);
    default: return launch_probe_t<PKV_FP8_E4M3>(a, sink, st);
  }
}

}  // namespace pkv
