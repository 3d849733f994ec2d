// kvc_select_threshold: KVzap's threshold rule with a sliding window.
//
// KVzap news page, inference section: entries whose score falls below a
// threshold are removed and a window of the most recent tokens is kept, so
// the kept count (the compression ratio) follows the prompt.  Candidates are
// [0, c), c = min(S - w, S - recent); a candidate is kept when its fp32 score
// is >= theta (NaN never); each head's kept positions are written ascending,
// followed by its recent window, and the heads are packed one after another
// (offsets[g] .. offsets[g + 1]).
//
// Design: two launches over the grid (chunk of 4096 candidates, head), 4 waves
// per workgroup, each wave on 1024 contiguous candidates with 16 coalesced
// loads per lane (load i of lane l reads candidate base + 64 i + l, so the
// candidate order is (i, lane)).
//  * threshold_count: per chunk, the number kept (wave ballots, popcounts).
//  * threshold_emit: the chunk's output offset is the sum of the counts of
//    every earlier chunk (head-major) plus the earlier heads' recent windows;
//    a lane's position inside the chunk is the popcount of the wave's earlier
//    ballots plus its rank in the current one (mbcnt), plus the earlier waves'
//    totals.  The last chunk of a head appends the recent window and writes
//    offsets[g + 1]; integer sums, so the output is deterministic.
#include "common.h"

namespace kvc {
namespace {

constexpr int kThrThreads = 256;
constexpr int kThrWaves = kThrThreads / kWave;
constexpr int kThrLoads = 16;                              // loads per lane
constexpr int kThrChunk = kThrWaves * kThrLoads * kWave;   // 4096 candidates per workgroup

struct ThrArgs {
  const float* s;
  int64_t hs;
  int c, S, recent, nchunk;
  float theta;
  uint32_t* counts;   // [Hkv * nchunk]
  int32_t* out;
  int32_t* offsets;   // [Hkv + 1]
};

// The 16 keep-ballots of this wave's candidates (uniform across the wave).
__device__ __forceinline__ void chunk_ballots(const ThrArgs& a, int g, int chunk, uint64_t (&m)[kThrLoads],
                                              int& first) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  first = chunk * kThrChunk + wave * (kThrLoads * kWave);
  const float* row = a.s + (int64_t)g * a.hs;
  float x[kThrLoads];
#pragma unroll
  for (int i = 0; i < kThrLoads; ++i) x[i] = 0.f;
  if (a.c > 0) {
    // unconditional loads from clamped addresses (c >= 1), masked below
#pragma unroll
    for (int i = 0; i < kThrLoads; ++i) {
      const int j = first + kWave * i + lane;
      x[i] = row[j < a.c ? j : a.c - 1];
    }
  }
#pragma unroll
  for (int i = 0; i < kThrLoads; ++i) {
    const int j = first + kWave * i + lane;
    m[i] = __ballot(a.c > 0 && j < a.c && x[i] >= a.theta);
  }
}

__global__ __launch_bounds__(kThrThreads) void threshold_count(ThrArgs a) {
  __shared__ uint32_t wtot[kThrWaves];
  const int chunk = blockIdx.x, g = blockIdx.y;
  uint64_t m[kThrLoads];
  int first;
  chunk_ballots(a, g, chunk, m, first);
  uint32_t n = 0;
#pragma unroll
  for (int i = 0; i < kThrLoads; ++i) n += (uint32_t)__popcll(m[i]);
  if ((threadIdx.x & 63) == 0) wtot[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kThrWaves; ++w) t += wtot[w];
    a.counts[(int64_t)g * a.nchunk + chunk] = t;
  }
}

__global__ __launch_bounds__(kThrThreads) void threshold_emit(ThrArgs a) {
  __shared__ uint32_t wred[kThrWaves], wtot[kThrWaves];
  const int chunk = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  // output offset of this chunk: every earlier chunk's count (head-major)
  const int64_t me = (int64_t)g * a.nchunk + chunk;
  uint32_t p = 0;
  for (int64_t i = tid; i < me; i += kThrThreads) p += a.counts[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) p += __shfl_xor(p, o);
  if (lane == 0) wred[wave] = p;

  uint64_t m[kThrLoads];
  int first;
  chunk_ballots(a, g, chunk, m, first);
  uint32_t n = 0;
#pragma unroll
  for (int i = 0; i < kThrLoads; ++i) n += (uint32_t)__popcll(m[i]);
  if (lane == 0) wtot[wave] = n;
  __syncthreads();
  uint32_t prefix = (uint32_t)g * (uint32_t)a.recent, before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kThrWaves; ++w) {
    prefix += wred[w];
    before += w < wave ? wtot[w] : 0u;
    total += wtot[w];
  }
  uint32_t pos = prefix + before;
#pragma unroll
  for (int i = 0; i < kThrLoads; ++i) {
    const uint32_t lo = (uint32_t)m[i], hi = (uint32_t)(m[i] >> 32);
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
    if ((m[i] >> lane) & 1ull) a.out[pos + rank] = first + kWave * i + lane;
    pos += (uint32_t)__popcll(m[i]);
  }
  if (chunk == a.nchunk - 1) {
    const uint32_t end = prefix + total;   // head g's kept candidates end here
    for (int t = tid; t < a.recent; t += kThrThreads) a.out[end + t] = a.S - a.recent + t;
    if (tid == 0) a.offsets[g + 1] = (int32_t)(end + (uint32_t)a.recent);
  }
  if (g == 0 && chunk == 0 && tid == 0) a.offsets[0] = 0;
}

int thr_chunks(int c) { return c > 0 ? (c + kThrChunk - 1) / kThrChunk : 1; }

}  // namespace
}  // namespace kvc

extern "C" size_t kvc_select_threshold_workspace_size(int32_t Hkv, int32_t S, int32_t w, int32_t recent) {
  if (Hkv < 1 || S < 2 || w < 1 || w >= S || recent < 0 || recent > S) return 0;
  const int32_t n = S - w;
  const int32_t c = n < S - recent ? n : S - recent;
  return kvc::align_up((size_t)Hkv * kvc::thr_chunks(c) * sizeof(uint32_t), 256);
}

extern "C" kvc_status kvc_select_threshold(const float* scores, int64_t score_head_stride, int32_t Hkv,
                                           int32_t S, int32_t w, int32_t recent, float threshold,
                                           int32_t* indices, int32_t* offsets, void* ws, size_t ws_bytes,
                                           void* stream) {
  using namespace kvc;
  if (Hkv < 1 || S < 2 || w < 1 || w >= S || recent < 0 || recent > S) return KVC_E_ARG;
  if (threshold != threshold) return KVC_E_ARG;   // NaN
  const int32_t n = S - w;
  const int32_t c = n < S - recent ? n : S - recent;
  if (score_head_stride < n && Hkv > 1) return KVC_E_SHAPE;
  if (Hkv > 65535 || (int64_t)Hkv * ((int64_t)c + recent) > 0x7FFFFFFF) return KVC_E_SHAPE;
  if (!indices || !offsets || (!scores && c > 0)) return KVC_E_ARG;
  if ((reinterpret_cast<uintptr_t>(scores) & 3) || (reinterpret_cast<uintptr_t>(indices) & 3) ||
      (reinterpret_cast<uintptr_t>(offsets) & 3))
    return KVC_E_ARG;
  const int nchunk = thr_chunks(c);
  if (!ws || ws_bytes < (size_t)Hkv * nchunk * sizeof(uint32_t) || (reinterpret_cast<uintptr_t>(ws) & 3))
    return KVC_E_WORKSPACE;
  ThrArgs a;
  a.s = scores;
  a.hs = score_head_stride;
  a.c = c;
  a.S = S;
  a.recent = recent;
  a.nchunk = nchunk;
  a.theta = threshold;
  a.counts = static_cast<uint32_t*>(ws);
  a.out = indices;
  a.offsets = offsets;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(nchunk, Hkv);
  KVC_LAUNCH("threshold_count", threshold_count, grid, dim3(kThrThreads), s, a);
  KVC_LAUNCH("threshold_emit", threshold_emit, grid, dim3(kThrThreads), s, a);
  return KVC_OK;
}
