// kvc_channel_prune / kvc_channel_prune_query: ThinK key-channel pruning.
//
// ThinK page (papercache summary of arXiv 2407.21018): magnitude-based pruning
// keeps, per head, the T = floor((1 - lambda) D) key channels with the largest
// l_p norm over tokens; query-driven pruning keeps the T channels with the
// largest ||Q[-S_obs:, j] K[:, j]^T||_F = ||Q[:, j]|| ||K[:, j]|| (rank-1
// outer product) over the observation-window queries; THINK's implementation
// section: recent keys are not pruned and a binary mask records the pruned
// channels.  The key norms here run over the non-recent kept rows (the rows
// that get pruned); a KV head's query side stacks its G query heads' windows.
//
// Design (D = 128):
//  * think_partial: grid (row chunks of 256, heads); 16 lanes cover one
//    256-byte row with 16-byte loads and each thread issues its 16 rows'
//    loads together (addresses clamped, tail masked); per-lane fp32 sums of
//    |x|^p, folded over the 16 row lanes in a fixed order -> partial[g, chunk, d].
//  * think_qpartial (query-driven only): grid (G, heads), the same row layout
//    over one query head's w window rows -> per-channel sums of q^2.
//  * think_select: one workgroup per head, 8 groups of 128 threads, group i
//    folding chunks i, i+8, ... (loads in flight), then the 8 group sums in a
//    fixed order (times the folded query sums, query-driven: ||Q|| ||K|| and
//    its square rank alike); channels ranked by (score desc, index asc), kept
//    channels written ascending, and the mask.
//  * think_gather: a wave takes 8 rows at a time (8 loads in flight); lane l
//    holds bf16 channels 2l, 2l+1 of a row and an output channel takes its
//    value with one cross-lane read from lane channels[c]/2.  With T even and
//    a 4-byte aligned output, lane c/2 packs output channels c, c+1 into one
//    4-byte store; otherwise 2-byte stores.
#include "common.h"

namespace kvc {
namespace {

constexpr int kD = 128;
constexpr int kChunkRows = 256;
constexpr int kRowsPerThread = kChunkRows / 16;
constexpr int kSelGroups = 8;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__global__ __launch_bounds__(256) void think_partial(const uint16_t* kc, int budget, int rows, int p,
                                                    int nchunk, float* part) {
  __shared__ float red[16][kD + 1];
  const int chunk = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int cg = tid & 15, rl = tid >> 4;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  const int r0 = chunk * kChunkRows;
  const uint16_t* base = kc + (int64_t)g * budget * kD + cg * 8;
  if (rows > 0) {
    u32x4 x[kRowsPerThread];
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
      const int r = r0 + rl + 16 * i;
      x[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)(r < rows ? r : rows - 1) * kD);
    }
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
      if (r0 + rl + 16 * i >= rows) continue;
      const uint32_t wv[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = bf16_lo(wv[e]), b = bf16_hi(wv[e]);
        if (p == 2) {
          acc[2 * e] = fmaf(a, a, acc[2 * e]);
          acc[2 * e + 1] = fmaf(b, b, acc[2 * e + 1]);
        } else {
          acc[2 * e] += fabsf(a);
          acc[2 * e + 1] += fabsf(b);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rl][cg * 8 + e] = acc[e];
  __syncthreads();
  if (tid < kD) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += red[i][tid];
    part[((int64_t)g * nchunk + chunk) * kD + tid] = s;
  }
}

__global__ __launch_bounds__(256) void think_qpartial(const uint16_t* q, int64_t q_hs, int G, int w,
                                                     float* qpart) {
  __shared__ float red[16][kD + 1];
  const int hh = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int cg = tid & 15, rl = tid >> 4;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  const uint16_t* base = q + (int64_t)(g * G + hh) * q_hs + cg * 8;
  for (int r = rl; r < w; r += 16) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(base + (int64_t)r * kD);
    const uint32_t wv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf16_lo(wv[e]), b = bf16_hi(wv[e]);
      acc[2 * e] = fmaf(a, a, acc[2 * e]);
      acc[2 * e + 1] = fmaf(b, b, acc[2 * e + 1]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rl][cg * 8 + e] = acc[e];
  __syncthreads();
  if (tid < kD) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += red[i][tid];
    qpart[((int64_t)g * G + hh) * kD + tid] = s;
  }
}

// qpart == nullptr: magnitude score; else the query-driven score (squared).
__global__ __launch_bounds__(kD * kSelGroups) void think_select(const float* part, int nchunk, const float* qpart,
                                                               int G, int T, int32_t* channels, uint8_t* mask) {
  __shared__ float red[kSelGroups][kD];
  __shared__ float sm[kD];
  __shared__ int ssel[kD];
  const int g = blockIdx.x, d = threadIdx.x & (kD - 1), grp = threadIdx.x / kD;
  const float* pp = part + (int64_t)g * nchunk * kD + d;
  // chunks grp + 8i go to sum i % 4 (four loads in flight), joined in order
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  int c = grp;
  for (; c + 3 * kSelGroups < nchunk; c += 4 * kSelGroups) {
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] += pp[(int64_t)(c + j * kSelGroups) * kD];
  }
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (c + j * kSelGroups < nchunk) a[j] += pp[(int64_t)(c + j * kSelGroups) * kD];
  red[grp][d] = (a[0] + a[1]) + (a[2] + a[3]);
  __syncthreads();
  // group 0 (threads 0..127) ranks; every thread still meets every barrier
  float M = 0.f;
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < kSelGroups; ++i) M += red[i][d];
    if (qpart) {
      float qn = 0.f;
      for (int hh = 0; hh < G; ++hh) qn += qpart[((int64_t)g * G + hh) * kD + d];
      M *= qn;
    }
    sm[d] = M;
  }
  __syncthreads();
  bool sel = false;
  if (grp == 0) {
    int rank = 0;
    for (int e = 0; e < kD; ++e) {
      const float o = sm[e];
      rank += (o > M || (o == M && e < d)) ? 1 : 0;
    }
    sel = rank < T;
    ssel[d] = sel ? 1 : 0;
  }
  __syncthreads();
  if (grp != 0) return;
  int pos = 0;
  for (int e = 0; e < d; ++e) pos += ssel[e];
  if (sel && pos < T) channels[(int64_t)g * T + pos] = d;   // pos < T unless norms are NaN
  if (mask) mask[(int64_t)g * kD + d] = sel ? 1 : 0;
}

// kPairs: T even and the output 4-byte aligned (lane l < T/2 stores output
// channels 2l and 2l+1 as one 4-byte word); else lanes l and l+64 store one
// bf16 each.
template <bool kPairs>
__global__ __launch_bounds__(256) void think_gather(const uint16_t* kc, int budget, int rows, int T,
                                                   const int32_t* channels, uint16_t* out) {
  constexpr int kRows = 8;   // rows per wave per step, loads in flight
  const int g = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int32_t* ch = channels + (int64_t)g * T;
  int s0, s1;
  bool w0, w1;
  if (kPairs) {
    w0 = 2 * lane < T;
    w1 = false;
    s0 = w0 ? ch[2 * lane] : 0;
    s1 = w0 ? ch[2 * lane + 1] : 0;
  } else {
    w0 = lane < T;
    w1 = lane + 64 < T;
    s0 = w0 ? ch[lane] : 0;
    s1 = w1 ? ch[lane + 64] : 0;
  }
  const uint32_t* src = reinterpret_cast<const uint32_t*>(kc + (int64_t)g * budget * kD);
  uint16_t* dst = out + (int64_t)g * rows * T;
  const int step = gridDim.x * 4 * kRows;
  for (int r0 = (blockIdx.x * 4 + wave) * kRows; r0 < rows; r0 += step) {
    uint32_t x[kRows];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      const int r = r0 + j < rows ? r0 + j : rows - 1;
      x[j] = src[(int64_t)r * (kD / 2) + lane];
    }
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      const int r = r0 + j;
      const uint32_t y0 = __shfl(x[j], s0 >> 1);
      const uint32_t y1 = __shfl(x[j], s1 >> 1);
      const uint32_t v0 = (s0 & 1) ? (y0 >> 16) : (y0 & 0xFFFFu);
      const uint32_t v1 = (s1 & 1) ? (y1 >> 16) : (y1 & 0xFFFFu);
      if (r >= rows) continue;
      if (kPairs) {
        if (w0) reinterpret_cast<uint32_t*>(dst + (int64_t)r * T)[lane] = v0 | (v1 << 16);
      } else {
        if (w0) dst[(int64_t)r * T + lane] = (uint16_t)v0;
        if (w1) dst[(int64_t)r * T + lane + 64] = (uint16_t)v1;
      }
    }
  }
}

}  // namespace
}  // namespace kvc

namespace kvc {
namespace {

size_t think_chunks(int32_t budget) {
  const size_t nchunk = ((size_t)budget + kChunkRows - 1) / kChunkRows;
  return nchunk ? nchunk : 1;
}

// Shared body of both entry points; q == nullptr selects the magnitude score.
kvc_status channel_prune(const void* k_c, const void* q, int32_t G, int32_t w, int64_t q_hs, int32_t Hkv,
                         int32_t budget, int32_t D, int32_t recent, double lambda, int32_t p, int32_t* channels,
                         uint8_t* mask, void* k_pruned, void* ws, size_t ws_bytes, size_t need, void* stream) {
  if (Hkv < 1 || budget < 0 || recent < 0 || recent > budget) return KVC_E_ARG;
  if (!(lambda >= 0.0 && lambda < 1.0) || (p != 1 && p != 2)) return KVC_E_ARG;
  if (D != kD) return KVC_E_UNSUPPORTED;
  if (Hkv > 65535) return KVC_E_SHAPE;
  const int T = kvc_think_channels(D, lambda);
  if (T < 1) return KVC_E_ARG;
  const int rows = budget - recent;
  if (!k_c || !channels || (rows > 0 && !k_pruned)) return KVC_E_ARG;
  if (!aligned16(k_c) || (reinterpret_cast<uintptr_t>(channels) & 3) ||
      (reinterpret_cast<uintptr_t>(k_pruned) & 1))
    return KVC_E_ARG;
  if (!ws || ws_bytes < need || !aligned16(ws)) return KVC_E_WORKSPACE;
  const int nchunk = (int)think_chunks(rows);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(ws);
  float* qpart = q ? part + align_up(think_chunks(budget) * Hkv * kD, 64) : nullptr;
  const uint16_t* kcp = static_cast<const uint16_t*>(k_c);
  KVC_LAUNCH("think_partial", think_partial, dim3(nchunk, Hkv), dim3(256), s, kcp, budget, rows, q ? 2 : p,
             nchunk, part);
  if (q)
    KVC_LAUNCH("think_qpartial", think_qpartial, dim3(G, Hkv), dim3(256), s, static_cast<const uint16_t*>(q),
               q_hs, G, w, qpart);
  KVC_LAUNCH("think_select", think_select, dim3(Hkv), dim3(kD * kSelGroups), s, part, nchunk, qpart, G, T,
             channels, mask);
  if (rows > 0) {
    int gx = (rows + 31) / 32;   // 4 waves x 8 rows per workgroup step
    if (gx > 1024) gx = 1024;
    uint16_t* kp = static_cast<uint16_t*>(k_pruned);
    if ((T & 1) == 0 && (reinterpret_cast<uintptr_t>(k_pruned) & 3) == 0)
      KVC_LAUNCH("think_gather", think_gather<true>, dim3(gx, Hkv), dim3(256), s, kcp, budget, rows, T, channels,
                 kp);
    else
      KVC_LAUNCH("think_gather", think_gather<false>, dim3(gx, Hkv), dim3(256), s, kcp, budget, rows, T, channels,
                 kp);
  }
  return KVC_OK;
}

}  // namespace
}  // namespace kvc

extern "C" size_t kvc_channel_prune_workspace_size(int32_t Hkv, int32_t budget, int32_t D) {
  if (Hkv < 1 || budget < 0 || D != kvc::kD) return 0;
  return kvc::align_up(kvc::think_chunks(budget) * Hkv * kvc::kD * sizeof(float), 256);
}

extern "C" kvc_status kvc_channel_prune(const void* k_c, int32_t Hkv, int32_t budget, int32_t D,
                                        int32_t recent, double lambda, int32_t p, int32_t* channels,
                                        uint8_t* mask, void* k_pruned, void* ws, size_t ws_bytes,
                                        void* stream) {
  return kvc::channel_prune(k_c, nullptr, 0, 0, 0, Hkv, budget, D, recent, lambda, p, channels, mask, k_pruned,
                            ws, ws_bytes, kvc_channel_prune_workspace_size(Hkv, budget, D), stream);
}

extern "C" size_t kvc_channel_prune_query_workspace_size(int32_t Hkv, int32_t G, int32_t budget, int32_t D) {
  if (Hkv < 1 || G < 1 || budget < 0 || D != kvc::kD) return 0;
  const size_t keys = kvc::align_up(kvc::think_chunks(budget) * Hkv * kvc::kD, 64);
  return kvc::align_up((keys + (size_t)Hkv * G * kvc::kD) * sizeof(float), 256);
}

extern "C" kvc_status kvc_channel_prune_query(const void* k_c, const void* q_obs, int32_t Hkv, int32_t G,
                                              int32_t w, int64_t q_head_stride, int32_t budget, int32_t D,
                                              int32_t recent, double lambda, int32_t* channels, uint8_t* mask,
                                              void* k_pruned, void* ws, size_t ws_bytes, void* stream) {
  using namespace kvc;
  if (G < 1 || w < 1 || !q_obs || !aligned16(q_obs)) return KVC_E_ARG;
  if ((int64_t)Hkv * G > 65535) return KVC_E_SHAPE;
  if (q_head_stride < (int64_t)w * D || (q_head_stride & 7)) return KVC_E_SHAPE;
  return channel_prune(k_c, q_obs, G, w, q_head_stride, Hkv, budget, D, recent, lambda, 2, channels, mask,
                       k_pruned, ws, ws_bytes, kvc_channel_prune_query_workspace_size(Hkv, G, budget, D), stream);
}
