// kvc_compact: gather the kept K and V rows into a dense per-head cache.
// kvc_compact_ragged: the same for per-head kept counts that vary (packed
// heads, as the threshold selection writes them).  kvc_compact_layers: every
// layer in one launch, each with its own budget read on the device.
//
// Keyformer blog page, prompt-phase paragraph: the kept tokens form the new,
// smaller cache; KVzap news page: the cache is (2, L, H, T, D).  The copy is of
// raw bf16 bytes.  Each lane moves 16-byte chunks, consecutive lanes on
// consecutive chunks of a row (coalesced 256-byte segments for D = 128), 4 rows
// per thread so that 4 loads are in flight; K and V are two planes of one
// grid.
#include "common.h"

namespace kvc {
namespace {

// One 16-byte chunk per lane, consecutive lanes on consecutive chunks of a row
// (a 128-dim row is 16 lanes: coalesced 256-byte segments), and kRPT rows per
// thread, kRPT independent loads in flight.  kChunks = D / 8 divides 256.
template <int kRPT>
__global__ __launch_bounds__(256) void compact_rows(const uint16_t* k, const uint16_t* v, int S, int D,
                                                     int64_t khs, int64_t vhs, const int32_t* idx,
                                                     int budget, uint16_t* ko, uint16_t* vo) {
  const int g = blockIdx.y;
  const bool isv = blockIdx.z != 0;
  const uint16_t* src = (isv ? v : k) + g * (isv ? vhs : khs);
  uint16_t* dst = (isv ? vo : ko) + (int64_t)g * budget * D;
  const int32_t* ix = idx + (int64_t)g * budget;
  const int chunks = D >> 3, rpp = 256 / chunks;   // rows per pass of the workgroup
  const int ch = threadIdx.x % chunks;
  const int r0 = blockIdx.x * rpp * kRPT + threadIdx.x / chunks;
  int j[kRPT];
#pragma unroll
  for (int q = 0; q < kRPT; ++q) {
    const int t = r0 + q * rpp;
    j[q] = t < budget ? ix[t] : -1;
  }
  u32x4 val[kRPT];
#pragma unroll
  for (int q = 0; q < kRPT; ++q) {
    const bool ok = j[q] >= 0 && j[q] < S;
    val[q] = *reinterpret_cast<const u32x4*>(src + (int64_t)(ok ? j[q] : 0) * D + ch * 8);
    if (!ok) val[q] = u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  }
#pragma unroll
  for (int q = 0; q < kRPT; ++q) {
    const int t = r0 + q * rpp;
    if (t < budget) *reinterpret_cast<u32x4*>(dst + (int64_t)t * D + ch * 8) = val[q];
  }
}

// Any D % 8 == 0: one chunk per thread.
__global__ __launch_bounds__(256) void compact_chunks(const uint16_t* k, const uint16_t* v, int S, int D,
                                                       int64_t khs, int64_t vhs, const int32_t* idx,
                                                       int budget, uint16_t* ko, uint16_t* vo) {
  const int g = blockIdx.y;
  const bool isv = blockIdx.z != 0;
  const uint16_t* src = (isv ? v : k) + g * (isv ? vhs : khs);
  uint16_t* dst = (isv ? vo : ko) + (int64_t)g * budget * D;
  const int32_t* ix = idx + (int64_t)g * budget;
  const int chunks = D >> 3;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int t = e / chunks;
  if (t >= budget) return;
  const int ch = e - t * chunks;
  const int j = ix[t];
  const bool ok = j >= 0 && j < S;
  u32x4 val = *reinterpret_cast<const u32x4*>(src + (int64_t)(ok ? j : 0) * D + ch * 8);
  if (!ok) val = u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  *reinterpret_cast<u32x4*>(dst + (int64_t)t * D + ch * 8) = val;
}

// Packed heads: head g's rows are [offsets[g], offsets[g + 1]) of indices and
// of the outputs.  grid (row blocks, Hkv, planes); a workgroup strides over
// its head's rows (the counts live on the device).  Every access is bounded
// by max_rows and [0, S) whatever the offsets hold.
template <int kRPT>
__global__ __launch_bounds__(256) void compact_ragged_rows(const uint16_t* k, const uint16_t* v, int S, int D,
                                                            int64_t khs, int64_t vhs, const int32_t* idx,
                                                            const int32_t* offsets, int max_rows,
                                                            uint16_t* ko, uint16_t* vo) {
  const int g = blockIdx.y;
  const bool isv = blockIdx.z != 0;
  const uint16_t* src = (isv ? v : k) + g * (isv ? vhs : khs);
  uint16_t* dst = isv ? vo : ko;
  const int a = offsets[g], b = offsets[g + 1];
  const int lo = max(a, 0), hi = min(b, max_rows);
  const int chunks = D >> 3, rpp = 256 / chunks;
  const int ch = threadIdx.x % chunks;
  const int step = gridDim.x * rpp * kRPT;
  for (int r0 = lo + blockIdx.x * rpp * kRPT + threadIdx.x / chunks; r0 - (int)(threadIdx.x / chunks) < hi;
       r0 += step) {
    int j[kRPT];
#pragma unroll
    for (int q = 0; q < kRPT; ++q) {
      const int t = r0 + q * rpp;
      j[q] = t < hi ? idx[t] : -1;
    }
    u32x4 val[kRPT];
#pragma unroll
    for (int q = 0; q < kRPT; ++q) {
      const bool ok = j[q] >= 0 && j[q] < S;
      val[q] = *reinterpret_cast<const u32x4*>(src + (int64_t)(ok ? j[q] : 0) * D + ch * 8);
      if (!ok) val[q] = u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    }
#pragma unroll
    for (int q = 0; q < kRPT; ++q) {
      const int t = r0 + q * rpp;
      if (t < hi) *reinterpret_cast<u32x4*>(dst + (int64_t)t * D + ch * 8) = val[q];
    }
  }
}

// Layers in one launch: grid (row blocks, Hkv * L, planes).  Layer l's block
// of indices and outputs starts at row Hkv * (budgets[0] + ... + budgets[l-1]),
// head g's rows at g * budgets[l] within it; a workgroup strides over its
// head's rows.  A layer whose block would pass out_rows rows writes nothing.
template <int kRPT>
__global__ __launch_bounds__(256) void compact_layers_rows(const uint16_t* k, const uint16_t* v, int S, int D,
                                                            int Hkv, int64_t khs, int64_t kls, int64_t vhs,
                                                            int64_t vls, const int32_t* budgets, int64_t out_rows,
                                                            const int32_t* idx, uint16_t* ko, uint16_t* vo) {
  const int hl = blockIdx.y, layer = hl / Hkv, g = hl - layer * Hkv;
  const bool isv = blockIdx.z != 0;
  int64_t before = 0;
  for (int i = 0; i < layer; ++i) before += budgets[i];
  const int B = budgets[layer];
  const int64_t base = (int64_t)Hkv * before + (int64_t)g * B;
  if (B <= 0 || before < 0 || base + B > out_rows) return;
  const uint16_t* src = isv ? v + layer * vls + g * vhs : k + layer * kls + g * khs;
  uint16_t* dst = (isv ? vo : ko) + base * D;
  const int32_t* ix = idx + base;
  const int chunks = D >> 3, rpp = 256 / chunks;
  const int ch = threadIdx.x % chunks;
  const int step = gridDim.x * rpp * kRPT;
  for (int r0 = blockIdx.x * rpp * kRPT + threadIdx.x / chunks; r0 - (int)(threadIdx.x / chunks) < B; r0 += step) {
    int j[kRPT];
#pragma unroll
    for (int q = 0; q < kRPT; ++q) {
      const int t = r0 + q * rpp;
      j[q] = t < B ? ix[t] : -1;
    }
    u32x4 val[kRPT];
#pragma unroll
    for (int q = 0; q < kRPT; ++q) {
      const bool ok = j[q] >= 0 && j[q] < S;
      val[q] = *reinterpret_cast<const u32x4*>(src + (int64_t)(ok ? j[q] : 0) * D + ch * 8);
      if (!ok) val[q] = u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    }
#pragma unroll
    for (int q = 0; q < kRPT; ++q) {
      const int t = r0 + q * rpp;
      if (t < B) *reinterpret_cast<u32x4*>(dst + (int64_t)t * D + ch * 8) = val[q];
    }
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
  if ((int64_t)budget * (D / 8) > 0x7FFFFFFF - 256) return KVC_E_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 block(256);
  const uint16_t *kp = static_cast<const uint16_t*>(k), *vp = static_cast<const uint16_t*>(v);
  uint16_t *kop = static_cast<uint16_t*>(k_out), *vop = static_cast<uint16_t*>(v_out);
  const int planes = v ? 2 : 1;
  const int chunks = D / 8;
  if (256 % chunks == 0) {   // 4 rows per thread
    constexpr int kRPT = 4;
    const int rows_per_wg = 256 / chunks * kRPT;
    KVC_LAUNCH("compact", compact_rows<kRPT>, dim3((budget + rows_per_wg - 1) / rows_per_wg, Hkv, planes), block, s,
               kp, vp, S, D, k_head_stride, v_head_stride, indices, budget, kop, vop);
  } else {
    const int threads = budget * chunks;
    KVC_LAUNCH("compact", compact_chunks, dim3((threads + 255) / 256, Hkv, planes), block, s, kp, vp, S, D,
               k_head_stride, v_head_stride, indices, budget, kop, vop);
  }
  return KVC_OK;
}

extern "C" kvc_status kvc_compact_ragged(const void* k, const void* v, int32_t Hkv, int32_t S, int32_t D,
                                         int64_t k_head_stride, int64_t v_head_stride, const int32_t* indices,
                                         const int32_t* offsets, int32_t max_rows, void* k_out, void* v_out,
                                         void* stream) {
  using namespace kvc;
  if (Hkv < 1 || S < 1 || max_rows < 0 || D < 8 || D > 1024 || (D & 7)) return KVC_E_ARG;
  if (256 % (D / 8)) return KVC_E_UNSUPPORTED;
  if (Hkv > 65535) return KVC_E_SHAPE;
  if (!k || !k_out || !offsets || (max_rows > 0 && !indices)) return KVC_E_ARG;
  if ((v == nullptr) != (v_out == nullptr)) return KVC_E_ARG;
  if (k_head_stride < (int64_t)S * D || (v && v_head_stride < (int64_t)S * D)) return KVC_E_SHAPE;
  if ((k_head_stride & 7) || (v && (v_head_stride & 7))) return KVC_E_ARG;
  if (!aligned16(k) || !aligned16(k_out) || (v && (!aligned16(v) || !aligned16(v_out)))) return KVC_E_ARG;
  if ((reinterpret_cast<uintptr_t>(indices) & 3) || (reinterpret_cast<uintptr_t>(offsets) & 3)) return KVC_E_ARG;
  if (max_rows == 0) return KVC_OK;
  if ((int64_t)max_rows * (D / 8) > 0x7FFFFFFF - 256) return KVC_E_SHAPE;
  constexpr int kRPT = 4;
  const int rows_per_wg = 256 / (D / 8) * kRPT;
  // rows per head are known only on the device: enough workgroups for an even
  // share of max_rows per head, at most 256 per head, striding beyond that
  int64_t per_head = ((int64_t)max_rows + Hkv - 1) / Hkv;
  int gx = (int)((per_head + rows_per_wg - 1) / rows_per_wg);
  gx = gx < 1 ? 1 : (gx > 256 ? 256 : gx);
  hipStream_t s = static_cast<hipStream_t>(stream);
  KVC_LAUNCH("compact_ragged", compact_ragged_rows<kRPT>, dim3(gx, Hkv, v ? 2 : 1), dim3(256), s,
             static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), S, D, k_head_stride,
             v_head_stride, indices, offsets, max_rows, static_cast<uint16_t*>(k_out),
             static_cast<uint16_t*>(v_out));
  return KVC_OK;
}

extern "C" kvc_status kvc_compact_layers(const void* k, const void* v, int32_t L, int32_t Hkv, int32_t S, int32_t D,
                                         int64_t k_head_stride, int64_t k_layer_stride, int64_t v_head_stride,
                                         int64_t v_layer_stride, const int32_t* budgets, int32_t total_budget,
                                         const int32_t* indices, void* k_out, void* v_out, void* stream) {
  using namespace kvc;
  if (L < 1 || Hkv < 1 || S < 1 || total_budget < 0 || D < 8 || D > 1024 || (D & 7)) return KVC_E_ARG;
  if (256 % (D / 8)) return KVC_E_UNSUPPORTED;
  if ((int64_t)Hkv * L > 65535) return KVC_E_SHAPE;
  if (!k || !k_out || !budgets || !indices) return KVC_E_ARG;
  if ((v == nullptr) != (v_out == nullptr)) return KVC_E_ARG;
  if (k_head_stride < (int64_t)S * D || (v && v_head_stride < (int64_t)S * D)) return KVC_E_SHAPE;
  if (L > 1 && (k_layer_stride < Hkv * k_head_stride || (v && v_layer_stride < Hkv * v_head_stride)))
    return KVC_E_SHAPE;
  if ((k_head_stride | k_layer_stride) & 7 || (v && ((v_head_stride | v_layer_stride) & 7))) return KVC_E_ARG;
  if (!aligned16(k) || !aligned16(k_out) || (v && (!aligned16(v) || !aligned16(v_out)))) return KVC_E_ARG;
  if ((reinterpret_cast<uintptr_t>(indices) | reinterpret_cast<uintptr_t>(budgets)) & 3) return KVC_E_ARG;
  const int64_t rows = (int64_t)Hkv * total_budget;
  if (rows == 0) return KVC_OK;
  if (rows * (D / 8) > 0x7FFFFFFF - 256) return KVC_E_SHAPE;
  constexpr int kRPT = 4;
  const int rows_per_wg = 256 / (D / 8) * kRPT;
  // a layer's budget is known only on the device: enough workgroups for 4x the
  // mean per-layer budget, striding beyond that
  int64_t mean = ((int64_t)total_budget + L - 1) / L;
  int gx = (int)((4 * mean + rows_per_wg - 1) / rows_per_wg);
  gx = gx < 1 ? 1 : (gx > 64 ? 64 : gx);
  KVC_LAUNCH("compact_layers", compact_layers_rows<kRPT>, dim3(gx, Hkv * L, v ? 2 : 1), dim3(256),
             static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), S,
             D, Hkv, k_head_stride, k_layer_stride, v_head_stride, v_layer_stride, budgets, rows, indices,
             static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out));
  return KVC_OK;
}
