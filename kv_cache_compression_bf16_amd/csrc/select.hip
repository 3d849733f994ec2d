// kvc_select_topk: per-head top-k of the importance plus the recent window.
//
// Selection rule (ZigZagKV blog page, SnapKV and token-selection sections;
// Keyformer blog page, prompt phase): candidates are positions [0, c),
// c = min(S - w, S - recent); the k_top = budget - recent candidates first in
// (importance descending, position ascending) order are kept together with
// every position of [S - recent, S); kept positions are written ascending.
//
// Design: one 1024-thread workgroup per head runs an exact MSB-first radix
// select on order-preserving 32-bit keys of the fp32 scores (digits of 11, 11
// and 10 bits, histograms in LDS with integer atomics, which are exact and
// order-independent).  That yields the k-th key T and how many T-valued
// candidates must be taken; a final ordered pass keeps every key > T and the
// first such T-valued candidates by position.  Each thread owns a contiguous
// run of 64 candidates held in registers, so the ascending output needs only
// two workgroup prefix sums per 32768 candidates and no sort.
#include "common.h"

namespace kvc {
namespace {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kBins = 2048;
constexpr int kBPT = kBins / kSelThreads;   // histogram bins per thread in the scan

// fp32 -> uint32 with the same order (-0 folded onto +0).
__device__ __forceinline__ uint32_t order_key(uint32_t b) {
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive prefix sum over the workgroup; *total receives the sum of all x.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const uint32_t s = wsum[i];
    before += (i < wid) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + v - x;
}

// Scores are processed in rounds of kSelThreads * kVPT candidates; thread t owns
// the contiguous segment [round_base + t*kVPT, round_base + (t+1)*kVPT), so the
// ordered emission needs only two workgroup scans per round.  When the
// candidates fit in one round they are loaded once and stay in registers for
// every radix level.
constexpr int kVPT = 64;
constexpr int kRound = kSelThreads * kVPT;

__device__ __forceinline__ void load_segment(const uint32_t* v, int c, int base, uint32_t (&key)[kVPT]) {
  const int j0 = base + (int)threadIdx.x * kVPT;
  if (j0 + kVPT <= c) {
    const u32x4* p = reinterpret_cast<const u32x4*>(v + j0);
    const bool al = (reinterpret_cast<uintptr_t>(v + j0) & 15u) == 0;
    if (al) {
#pragma unroll
      for (int i = 0; i < kVPT / 4; ++i) {
        const u32x4 x = p[i];
        key[4 * i + 0] = order_key(x.x);
        key[4 * i + 1] = order_key(x.y);
        key[4 * i + 2] = order_key(x.z);
        key[4 * i + 3] = order_key(x.w);
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < kVPT; ++i) key[i] = (j0 + i < c) ? order_key(v[j0 + i]) : 0u;
}

__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(const float* imp, int64_t hs, int c,
                                                                 int k_top, int S, int recent, int budget,
                                                                 int32_t* out) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t wsum[kSelWaves];
  __shared__ uint32_t s_digit, s_above;

  const int g = blockIdx.x, tid = threadIdx.x;
  const uint32_t* v = reinterpret_cast<const uint32_t*>(imp + (int64_t)g * hs);
  int32_t* o = out + (int64_t)g * budget;

  for (int t = tid; t < recent; t += kSelThreads) o[k_top + t] = S - recent + t;
  if (k_top == 0) return;
  if (k_top >= c) {
    for (int j = tid; j < c; j += kSelThreads) o[j] = j;
    return;
  }

  const int rounds = (c + kRound - 1) / kRound;
  uint32_t key[kVPT];
  if (rounds == 1) load_segment(v, c, 0, key);
  const int seg0 = tid * kVPT;

  // ---- radix select of the k_top-th largest key (11, 11, 10-bit digits)
  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)k_top;
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t width_mask = (pass == 2) ? 0x3FFu : 0x7FFu;
    for (int b = tid; b < kBins; b += kSelThreads) hist[b] = 0;
    if (tid == 0) {
      s_digit = 0;
      s_above = 0;
    }
    __syncthreads();
    for (int r = 0; r < rounds; ++r) {
      if (rounds > 1) load_segment(v, c, r * kRound, key);
      const int j0 = r * kRound + seg0;
#pragma unroll
      for (int i = 0; i < kVPT; ++i)
        if (j0 + i < c && (key[i] & pmask) == prefix) atomicAdd(&hist[(key[i] >> sh) & width_mask], 1u);
    }
    __syncthreads();
    // suffix counts: thread tid owns bins [kBPT*rt, kBPT*rt + kBPT), rt = last - tid
    const int rt = kSelThreads - 1 - tid;
    uint32_t hb[kBPT], a = 0;
#pragma unroll
    for (int i = 0; i < kBPT; ++i) {
      hb[i] = hist[kBPT * rt + i];
      a += hb[i];
    }
    uint32_t tot;
    const uint32_t incl = block_excl_scan(a, wsum, &tot) + a;   // = count of bins >= kBPT*rt
    uint32_t below = 0;
#pragma unroll
    for (int i = 0; i < kBPT; ++i) {
      const uint32_t suf = incl - below;                          // = count of bins >= kBPT*rt + i
      if (suf >= krem && suf - hb[i] < krem) {
        s_digit = kBPT * rt + i;
        s_above = suf - hb[i];
      }
      below += hb[i];
    }
    __syncthreads();
    prefix |= s_digit << sh;
    pmask |= width_mask << sh;
    krem -= s_above;
    __syncthreads();
  }
  const uint32_t T = prefix;   // k_top-th largest key; take krem of the keys equal to T

  // ---- ordered emission: keys > T, then the first krem keys == T by position
  uint32_t eq_carry = 0, out_carry = 0;
  for (int r = 0; r < rounds; ++r) {
    if (rounds > 1) load_segment(v, c, r * kRound, key);
    const int j0 = r * kRound + seg0;
    uint32_t n_eq = 0, n_gt = 0;
#pragma unroll
    for (int i = 0; i < kVPT; ++i) {
      const bool in = j0 + i < c;
      n_eq += (in && key[i] == T) ? 1u : 0u;
      n_gt += (in && key[i] > T) ? 1u : 0u;
    }
    uint32_t eq_tot;
    const uint32_t eq_before = block_excl_scan(n_eq, wsum, &eq_tot) + eq_carry;
    // T-valued keys of this thread that still fit in the quota
    const uint32_t eq_room = krem > eq_before ? krem - eq_before : 0u;
    const uint32_t n_take = n_gt + (n_eq < eq_room ? n_eq : eq_room);
    uint32_t take_tot;
    uint32_t pos = block_excl_scan(n_take, wsum, &take_tot) + out_carry;
    uint32_t eq_seen = 0;
#pragma unroll
    for (int i = 0; i < kVPT; ++i) {
      const bool in = j0 + i < c;
      const bool eq = in && key[i] == T;
      const bool take = (in && key[i] > T) || (eq && eq_seen < eq_room);
      eq_seen += eq ? 1u : 0u;
      if (take && pos < (uint32_t)k_top) o[pos] = j0 + i;
      pos += take ? 1u : 0u;
    }
    eq_carry += eq_tot;
    out_carry += take_tot;
  }
}

}  // namespace
}  // namespace kvc

extern "C" size_t kvc_select_topk_workspace_size(int32_t Hkv, int32_t n) {
  (void)Hkv;
  (void)n;
  return 0;
}

extern "C" kvc_status kvc_select_topk(const float* importance, int64_t imp_head_stride, int32_t Hkv,
                                      int32_t S, int32_t w, int32_t recent, int32_t budget,
                                      int32_t* indices, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (Hkv < 1 || S < 2 || w < 1 || w >= S || recent < 0 || recent > S) return KVC_E_ARG;
  const int32_t n = S - w;
  const int32_t c = n < S - recent ? n : S - recent;
  if (budget < recent || budget - recent > c) return KVC_E_ARG;
  if (imp_head_stride < n && Hkv > 1) return KVC_E_SHAPE;
  if (!indices || (!importance && budget > recent)) return KVC_E_ARG;
  if ((reinterpret_cast<uintptr_t>(importance) & 3) || (reinterpret_cast<uintptr_t>(indices) & 3))
    return KVC_E_ARG;
  if (budget == 0) return KVC_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  KVC_LAUNCH("select_topk", kvc::select_topk_kernel, dim3(Hkv), dim3(kvc::kSelThreads), s, importance,
             imp_head_stride, c, budget - recent, S, recent, budget, indices);
  return KVC_OK;
}
