// kvc_compact: gather the kept K and V rows into a dense per-head cache.
//
// Keyformer blog page, prompt-phase paragraph: the kept tokens form the new,
// smaller cache; KVzap news page: the cache is (2, L, H, T, D).  The copy is of
// raw bf16 bytes.  Each lane moves 16 bytes, so a 128-dim row is 16 lanes and
// a wave copies 4 full rows per instruction (coalesced 256-byte segments); K
// and V are two planes of the same grid.
#include "common.h"

namespace kvc {
namespace {

__global__ __launch_bounds__(256) void compact_kernel(const uint16_t* k, const uint16_t* v, int S, int D,
                                                       int64_t khs, int64_t vhs, const int32_t* idx,
                                                       int budget, uint16_t* ko, uint16_t* vo) {
  const int g = blockIdx.y;
  const bool isv = blockIdx.z != 0;
  const uint16_t* src = (isv ? v : k) + g * (isv ? vhs : khs);
  uint16_t* dst = (isv ? vo : ko) + (int64_t)g * budget * D;
  const int32_t* ix = idx + (int64_t)g * budget;
  const int chunks = D >> 3;
  const int64_t total = (int64_t)budget * chunks;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int t = (int)(e / chunks), ch = (int)(e - (int64_t)t * chunks);
    const int j = ix[t];
    u32x4 val;
    if (j >= 0 && j < S)
      val = *reinterpret_cast<const u32x4*>(src + (int64_t)j * D + ch * 8);
    else
      val = u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    *reinterpret_cast<u32x4*>(dst + (int64_t)t * D + ch * 8) = val;
  }
}

}  // namespace
}  // namespace kvc

extern "C" kvc_status kvc_compact(const void* k, const void* v, int32_t Hkv, int32_t S, int32_t D,
                                  int64_t k_head_stride, int64_t v_head_stride, const int32_t* indices,
                                  int32_t budget, void* k_out, void* v_out, void* stream) {
  using namespace kvc;
  if (Hkv < 1 || S < 1 || budget < 0 || D < 8 || D > 1024 || (D & 7)) return KVC_E_ARG;
  if (Hkv > 65535) return KVC_E_SHAPE;
  if (!k || !k_out || (budget > 0 && !indices)) return KVC_E_ARG;
  if ((v == nullptr) != (v_out == nullptr)) return KVC_E_ARG;
  if (k_head_stride < (int64_t)S * D || (v && v_head_stride < (int64_t)S * D)) return KVC_E_SHAPE;
  if ((k_head_stride & 7) || (v && (v_head_stride & 7))) return KVC_E_ARG;
  if (!aligned16(k) || !aligned16(k_out) || (v && (!aligned16(v) || !aligned16(v_out)))) return KVC_E_ARG;
  if (reinterpret_cast<uintptr_t>(indices) & 3) return KVC_E_ARG;
  if (budget == 0) return KVC_OK;
  const int64_t total = (int64_t)budget * (D / 8);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipStream_t s = static_cast<hipStream_t>(stream);
  KVC_LAUNCH("compact", compact_kernel, dim3((unsigned)blocks, Hkv, v ? 2 : 1), dim3(256), s,
             static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), S, D, k_head_stride,
             v_head_stride, indices, budget, static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out));
  return KVC_OK;
}
