// kvc_select_topk: per-head top-k of the importance plus the recent window.
//
// Selection rule (ZigZagKV blog page, SnapKV and token-selection sections;
// Keyformer blog page, prompt phase): candidates are positions [0, c),
// c = min(S - w, S - recent); the k_top = budget - recent candidates first in
// (importance descending, position ascending) order are kept together with
// every position of [S - recent, S); kept positions are written ascending.
//
// Both designs below run an exact MSB-first radix select on order-preserving
// 32-bit keys of the fp32 scores with LDS histograms and integer atomics
// (exact and order-independent), then write the kept positions in order, so
// the output is ascending without a sort and bit-reproducible.
//
//  * Up to 32768 candidates per head (one launch): one 1024-thread workgroup
//    per head keeps all keys in registers; its levels work on key - min, each
//    taking the next (up to) 11 bits below the top set bit of max - min, so
//    scores of similar magnitude still spread over the bins.  As soon as the
//    bin holding the k_top-th key has at most 256 keys, those are gathered in
//    LDS and ranked directly (usually after the first level).  Emission: each
//    wave owns a contiguous span of candidates, so ballots and mbcnt within
//    the wave plus per-wave counts give every kept candidate its slot.
//  * More candidates (four launches, each ordered after the previous one on
//    the stream): every head is cut into chunks of at most 4096 and each
//    (chunk, head) gets a 256-thread workgroup.  Levels of 11, 11 and 10 bits;
//    level L's workgroups first resolve level L-1's digit by a binary search
//    over the per-chunk inclusive suffix counts the previous launch stored
//    (11 sums over the chunks), histogram their chunk, and store its suffix
//    counts; the last launch resolves T, counts the kept candidates of the
//    earlier chunks from their suffix counts and emits its chunk.  Launches
//    cost several microseconds each, so this only pays off where one
//    workgroup per head would leave most of the chip idle for long.
#include "common.h"

namespace kvc {
namespace {

constexpr int kBins = 2048;

// fp32 -> uint32 with the same order (-0 folded onto +0).
__device__ __forceinline__ uint32_t order_key(uint32_t b) {
  // sign set: all bits flipped; clear: the sign bit set.  -0 lands on
  // 0x7FFFFFFF (no other input does) and is moved onto +0's key.
  const uint32_t k = b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
  return k == 0x7FFFFFFFu ? 0x80000000u : k;
}

// Exclusive prefix sum over a workgroup of kThreadsT threads; *total receives
// the sum of all x.
template <int kThreadsT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* wsum, uint32_t* total) {
  constexpr int kWavesT = kThreadsT / kWave;
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
  for (int i = 0; i < kWavesT; ++i) {
    const uint32_t s = wsum[i];
    before += (i < wid) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + v - x;
}

// ======================================================== one workgroup per head
namespace one {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kBPT = kBins / kSelThreads;   // histogram bins per thread in the scan

// Workgroup-wide (min, max); every thread receives the result.
// Within each 16-lane row, DPP moves (xor 1, xor 2, half-row mirror, row
// mirror) leave every lane with the row's (min, max); lanes 0, 16, 32 and 48
// are then read into scalar registers.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kCtrl, 0xF, 0xF, false);
}
__device__ __forceinline__ void wave_min_max(uint32_t& lo, uint32_t& hi) {
  lo = min(lo, dpp_u32<0xB1>(lo));
  hi = max(hi, dpp_u32<0xB1>(hi));
  lo = min(lo, dpp_u32<0x4E>(lo));
  hi = max(hi, dpp_u32<0x4E>(hi));
  lo = min(lo, dpp_u32<0x141>(lo));
  hi = max(hi, dpp_u32<0x141>(hi));
  lo = min(lo, dpp_u32<0x140>(lo));
  hi = max(hi, dpp_u32<0x140>(hi));
  lo = min(min((uint32_t)__builtin_amdgcn_readlane((int)lo, 0), (uint32_t)__builtin_amdgcn_readlane((int)lo, 16)),
           min((uint32_t)__builtin_amdgcn_readlane((int)lo, 32), (uint32_t)__builtin_amdgcn_readlane((int)lo, 48)));
  hi = max(max((uint32_t)__builtin_amdgcn_readlane((int)hi, 0), (uint32_t)__builtin_amdgcn_readlane((int)hi, 16)),
           max((uint32_t)__builtin_amdgcn_readlane((int)hi, 32), (uint32_t)__builtin_amdgcn_readlane((int)hi, 48)));
}

__device__ __forceinline__ void block_min_max(uint32_t& lo, uint32_t& hi, uint32_t* wlo, uint32_t* whi) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  wave_min_max(lo, hi);
  if (lane == 0) {
    wlo[wid] = lo;
    whi[wid] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    lo = min(lo, wlo[i]);
    hi = max(hi, whi[i]);
  }
  __syncthreads();
}

// Up to kRound = 32768 candidates: wave w owns the contiguous range
// [w*kSpan, (w+1)*kSpan) and lane l holds candidates w*kSpan + 64*i + l
// (i < kVPL), so every load instruction reads 256 contiguous bytes and a lane
// keeps kVPL loads in flight.  The keys are loaded once and stay in registers
// for every radix level and the emission.  They come back as bits ^ 2^31,
// which is order_key for every value whose sign bit is clear (scores of
// softmax means always are); the caller redoes them with order_key when a
// candidate's sign bit is set.
constexpr int kVPL = 32768 / kSelThreads;          // candidates per lane per round
constexpr int kSpan = kVPL * kWave;                 // candidates per wave per round
constexpr int kRound = kSelWaves * kSpan;

__device__ __forceinline__ void load_round(const uint32_t* v, int c, int r, uint32_t (&key)[kVPL]) {
  const int base = r * kRound + (int)(threadIdx.x >> 6) * kSpan + (int)(threadIdx.x & 63);
  uint32_t raw[kVPL];
  if (r * kRound + (int)(threadIdx.x >> 6) * kSpan + kSpan <= c) {
    // a wave whose whole span is candidates: one base address and immediate
    // offsets, no range test
    const uint32_t* vb = v + base;
#pragma unroll
    for (int i = 0; i < kVPL; ++i) raw[i] = vb[64 * i];
#pragma unroll
    for (int i = 0; i < kVPL; ++i) key[i] = raw[i] ^ 0x80000000u;
    return;
  }
  // Unconditional loads from a clamped address (then masked): a guarded load
  // would be a branch, and the wait at each branch merge would serialize them.
#pragma unroll
  for (int i = 0; i < kVPL; ++i) {
    const int j = base + 64 * i;
    raw[i] = v[j < c ? j : c - 1];
  }
#pragma unroll
  for (int i = 0; i < kVPL; ++i) key[i] = (base + 64 * i < c) ? raw[i] ^ 0x80000000u : 0u;
}

// Keys of the threshold bin are ranked directly once a level leaves at most
// this many of them.
constexpr int kLiveMax = 256;

// Layers in one launch (budgets != null): grid (Hkv, L); layer l keeps
// budgets[l] tokens per head and its block of the output starts at
// Hkv * (budgets[0] + ... + budgets[l-1]) (head g's rows at g * budgets[l]), the
// layout of per-layer calls on one flat buffer.  A layer whose budget is out
// of range, or whose block would pass out_cap entries, writes nothing.
// Candidate counts above kRound are never launched here with 0 < k_top < c.
__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(const float* imp, int64_t hs, int64_t ls, int c,
                                                                 int k_top, int S, int recent, int budget,
                                                                 const int32_t* budgets, int64_t out_cap,
                                                                 int32_t* out) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t wsum[kSelWaves], wsum2[kSelWaves];
  __shared__ uint32_t s_digit, s_above, s_count, s_live, s_T, s_krem;
  __shared__ __attribute__((aligned(16))) uint32_t live[kLiveMax];

  const int g = blockIdx.x, layer = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int64_t obase = (int64_t)g * budget;
  if (budgets) {
    int64_t before = 0;
    for (int i = 0; i < layer; ++i) before += budgets[i];
    budget = budgets[layer];
    k_top = budget - recent;
    obase = (int64_t)gridDim.x * before + (int64_t)g * budget;
    if (k_top < 0 || k_top > c || before < 0 || obase < 0 || obase + budget > out_cap) return;
  }
  const uint32_t* v = reinterpret_cast<const uint32_t*>(imp + layer * ls + (int64_t)g * hs);
  int32_t* o = out + obase;

  for (int t = tid; t < recent; t += kSelThreads) o[k_top + t] = S - recent + t;
  if (k_top == 0) return;
  if (k_top >= c) {
    for (int j = tid; j < c; j += kSelThreads) o[j] = j;
    return;
  }
  if (c > kRound) return;

  uint32_t key[kVPL];
  load_round(v, c, 0, key);
  const int lbase = wave * kSpan + lane;   // candidate of key[0]

  // Waves are full (every slot a candidate), partial (the one holding c - 1)
  // or empty (uniform per wave); empty waves skip every per-key loop.
  const bool wave_full = wave * kSpan + kSpan <= c, wave_empty = wave * kSpan >= c;

  // the first level's histogram and flags are cleared here, while the loads
  // are in flight; the range reduction's barriers publish them
  for (int b = tid; b < kBins; b += kSelThreads) hist[b] = 0;
  if (tid == 0) {
    s_digit = 0;
    s_above = 0;
    s_count = 0;
    s_live = 0;
  }

  // ---- key range of the candidates (slots past them hold key 0: no effect
  // on the max; the min skips them)
  uint32_t kmin, kmax;
  auto key_range = [&] {
    kmin = 0xFFFFFFFFu;
    kmax = 0u;
    if (wave_full) {
#pragma unroll
      for (int i = 0; i < kVPL; i += 2) {
        kmin = min(kmin, min(key[i], key[i + 1]));
        kmax = max(kmax, max(key[i], key[i + 1]));
      }
    } else if (!wave_empty) {
#pragma unroll
      for (int i = 0; i < kVPL; ++i) {
        kmin = min(kmin, lbase + 64 * i < c ? key[i] : 0xFFFFFFFFu);
        kmax = max(kmax, key[i]);
      }
    }
    block_min_max(kmin, kmax, wsum, wsum2);
  };
  key_range();
  if (kmin < 0x80000000u) {
    // a candidate's sign bit is set (a negative value, -0 or a negative
    // NaN): the full order key, and the range again
    if (wave_full) {
#pragma unroll
      for (int i = 0; i < kVPL; ++i) key[i] = order_key(key[i] ^ 0x80000000u);
    } else if (!wave_empty) {
#pragma unroll
      for (int i = 0; i < kVPL; ++i) key[i] = lbase + 64 * i < c ? order_key(key[i] ^ 0x80000000u) : 0u;
    }
    key_range();
  }
  // From here on key[i] holds d = key - kmin.  The partial wave's slots past
  // the candidates take d = 0: they follow every candidate in position order
  // and no candidate is smaller, so they are never kept (ties are taken in
  // position order and the candidates alone hold k_top keys >= T) and need
  // no range test.
  if (wave_full) {
#pragma unroll
    for (int i = 0; i < kVPL; ++i) key[i] -= kmin;
  } else {
#pragma unroll
    for (int i = 0; i < kVPL; ++i) key[i] = lbase + 64 * i < c ? key[i] - kmin : 0u;
  }

  // ---- radix select on d, MSB first.  Bits [top, 32) of the k_top-th
  // largest d are known (= hi); each level resolves up to 11 more.
  // Once the keys sharing the resolved bits are few, they are ranked directly.
  int top = 32 - __clz(kmax - kmin);   // 0 when every candidate has the same key
  uint32_t hi = 0, krem = (uint32_t)k_top;
  uint32_t T;
  bool first = true;   // the first level counts every key: all d < 2^top
  while (true) {
    if (top == 0) {
      T = hi;   // every bit resolved: take krem of the keys equal to T
      break;
    }
    const int width = top < 11 ? top : 11;
    const int sh = top - width;
    const uint32_t dmask = (1u << width) - 1u;
    const uint32_t hmask = top >= 32 ? 0u : (0xFFFFFFFFu << top);   // bits already resolved
    const uint32_t hval = top >= 32 ? 0u : (hi << top);
    if (!first) {   // the first level's were cleared before the range reduction
      for (int b = tid; b < kBins; b += kSelThreads) hist[b] = 0;
      if (tid == 0) {
        s_digit = 0;
        s_above = 0;
        s_count = 0;
        s_live = 0;
      }
      __syncthreads();
    }
    if (wave_empty) {
    } else if (first) {
#pragma unroll
      for (int i = 0; i < kVPL; ++i) atomicAdd(&hist[(key[i] >> sh) & dmask], 1u);
    } else {
#pragma unroll
      for (int i = 0; i < kVPL; ++i) {
        const uint32_t d = key[i];
        if ((d & hmask) == hval) atomicAdd(&hist[(d >> sh) & dmask], 1u);
      }
    }
    first = false;
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
    const uint32_t incl = block_excl_scan<kSelThreads>(a, wsum, &tot) + a;   // = count of bins >= kBPT*rt
    uint32_t below = 0;
#pragma unroll
    for (int i = 0; i < kBPT; ++i) {
      const uint32_t suf = incl - below;                          // = count of bins >= kBPT*rt + i
      if (suf >= krem && suf - hb[i] < krem) {
        s_digit = kBPT * rt + i;
        s_above = suf - hb[i];
        s_count = hb[i];
      }
      below += hb[i];
    }
    __syncthreads();
    hi = (hi << width) | s_digit;
    krem -= s_above;
    top = sh;
    const uint32_t count = s_count;   // keys whose bits [top, 32) of d equal hi
    if (top > 0 && count <= (uint32_t)kLiveMax) {
      // gather those keys (any order; count of them, so the slots stay below kLiveMax) ...
      if (!wave_empty) {
#pragma unroll
        for (int i = 0; i < kVPL; ++i) {
          const uint32_t d = key[i];
          if ((d >> top) == hi) {
            const uint32_t slot = atomicAdd(&s_live, 1u);
            if (slot < (uint32_t)kLiveMax) live[slot] = d;
          }
        }
      }
      __syncthreads();
      // ... and the one whose rank (keys greater, keys equal) covers krem is T
      // (16-byte broadcast reads, 8 in flight; slots past count hold no key)
      if (tid < (int)count) {
        const uint32_t x = live[tid];
        uint32_t gt = 0, eq = 0;
        const uint4* l4 = reinterpret_cast<const uint4*>(live);
        for (int j0 = 0; j0 < (int)count; j0 += 32) {
          uint4 y[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) y[u] = l4[j0 / 4 + u];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const uint32_t yy[4] = {y[u].x, y[u].y, y[u].z, y[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool ok = j0 + 4 * u + e < (int)count;
              gt += ok && yy[e] > x ? 1u : 0u;
              eq += ok && yy[e] == x ? 1u : 0u;
            }
          }
        }
        if (gt < krem && krem <= gt + eq) {   // every such thread holds the same x
          s_T = x;
          s_krem = krem - gt;
        }
      }
      __syncthreads();
      T = s_T;
      krem = s_krem;
      break;
    }
    __syncthreads();
  }

  // ---- ordered emission.  Wave w owns candidates [w*kSpan, (w+1)*kSpan) and
  // its lane l holds the one at offset 64i + l, so (wave, i, lane) is position
  // order.  A kept candidate's output slot is (keys > T before it) +
  // min(keys == T before it, krem): per-wave counts give the earlier waves'
  // share, ballots and mbcnt the rest.  Output is ascending without a sort.
  // When every key equal to T is kept (the usual case), the kept keys are
  // exactly those >= T and one ballot per step suffices.
  // per-wave counts of keys >= T and == T: per-lane counts summed over the
  // wave (vector adds and one xor tree, no ballot-to-scalar round trips)
  uint32_t n_ge = 0, n_eq = 0;
  if (!wave_empty) {
#pragma unroll
    for (int i = 0; i < kVPL; ++i) {
      n_ge += key[i] >= T ? 1u : 0u;
      n_eq += key[i] == T ? 1u : 0u;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      n_ge += (uint32_t)__shfl_xor((int)n_ge, o);
      n_eq += (uint32_t)__shfl_xor((int)n_eq, o);
    }
  }
  if (lane == 0) {
    wsum[wave] = n_ge;
    wsum2[wave] = n_eq;
  }
  __syncthreads();
  // positions are recomputed here from an opaque copy of lbase: otherwise the
  // compiler keeps the 32 positions of the range test alive (in scratch)
  int pos0 = lbase;
  asm volatile("" : "+v"(pos0));
  uint32_t ge_run = 0, eq_run = 0, eq_all = 0;
  for (int u = 0; u < kSelWaves; ++u) {
    ge_run += u < wave ? wsum[u] : 0u;
    eq_run += u < wave ? wsum2[u] : 0u;
    eq_all += wsum2[u];
  }
  if (wave_empty) return;
  if (eq_all <= krem) {   // then the keys >= T number exactly k_top
#pragma unroll
    for (int i = 0; i < kVPL; ++i) {
      const bool ge = key[i] >= T;
      const uint64_t b = __ballot(ge);
      const uint32_t slot = ge_run + __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
      if (ge && slot < (uint32_t)k_top) o[slot] = pos0 + 64 * i;   // < k_top by construction; checked anyway
      ge_run += (uint32_t)__popcll(b);
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }
  uint32_t gt_run = ge_run - eq_run;
#pragma unroll
  for (int i = 0; i < kVPL; ++i) {
    const bool gt = key[i] > T, eq = key[i] == T;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    const uint32_t below_g = __builtin_amdgcn_mbcnt_hi((uint32_t)(bg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bg, 0u));
    const uint32_t below_e = __builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0u));
    const uint32_t er = eq_run + below_e;
    const uint32_t slot = gt_run + below_g + min(er, krem);   // < k_top by construction; checked anyway
    if ((gt || (eq && er < krem)) && slot < (uint32_t)k_top) o[slot] = pos0 + 64 * i;
    gt_run += (uint32_t)__popcll(bg);
    eq_run += (uint32_t)__popcll(be);
    __builtin_amdgcn_sched_barrier(0);
  }
}


}  // namespace one

// ================================================= several workgroups per head
namespace many {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kBPT = kBins / kThreads;           // histogram bins per thread in a scan
constexpr int kMaxChunk = 4096;                  // candidates per workgroup
constexpr int kSegment = kMaxChunk / kThreads;   // candidates per thread in the emission
constexpr int kTargetGroups = 256;               // workgroups aimed for over all heads

// Level L: digit = (key >> level_shift(L)) & level_mask(L).
__host__ __device__ constexpr int level_shift(int L) { return L == 0 ? 21 : (L == 1 ? 10 : 0); }
__host__ __device__ constexpr uint32_t level_mask(int L) { return L == 2 ? 0x3FFu : 0x7FFu; }

// Per-head state passed between launches: resolved digits and the rank of T
// still to place after each level.
enum : int { kD0 = 0, kD1 = 1, kKrem1 = 2, kKrem2 = 3, kStateWords = 4 };

struct SelArgs {
  const uint32_t* imp;   // fp32 bit patterns
  int64_t hs;            // head stride (elements)
  int c, k_top, S, recent, budget;
  int chunk, nchunk;     // candidates per chunk, chunks per head
  int32_t* out;          // [Hkv, budget]
  uint32_t* suf;         // [3][Hkv][nchunk][kBins]: inclusive suffix counts per chunk
  uint32_t* state;       // [Hkv][kStateWords]
};

__device__ __forceinline__ const uint32_t* chunk_suffix(const SelArgs& a, int L, int g, int q) {
  return a.suf + (((int64_t)L * gridDim.y + g) * a.nchunk + q) * kBins;
}

// Level L's digit: the largest d with total suffix count >= krem (the count
// at bin 0, all live keys, is >= krem), and the count above it.  The totals
// are non-increasing in d, so two steps find it: the 32 coarse bins 64c,
// then the 64 bins of the chosen coarse interval.  Each step sums its bins
// over the chunks with every load in flight at once (integer sums: the order
// does not matter).  Both steps end in barriers, which also publish LDS
// writes made before the call.
constexpr int kCoarse = kBins / 64;                                // 32 coarse bins
static_assert(kThreads % kCoarse == 0 && kThreads % 64 == 0, "resolve_digit thread split");
__device__ __forceinline__ void resolve_digit(const SelArgs& a, int L, int g, uint32_t krem, uint32_t* wsum,
                                              uint32_t& digit, uint32_t& above) {
  (void)wsum;
  __shared__ uint32_t rs_part[kThreads];
  __shared__ uint32_t rs_tot[64];
  const int tid = threadIdx.x;
  const uint32_t* base = chunk_suffix(a, L, g, 0);
  // coarse step: totals at bins 64c; thread tid sums chunks q = tid / 32 (mod 8) of bin 64 (tid % 32)
  {
    constexpr int kGroups = kThreads / kCoarse;
    const int c = tid % kCoarse;
    uint32_t x = 0;
    for (int q = tid / kCoarse; q < a.nchunk; q += kGroups) x += base[(int64_t)q * kBins + 64 * c];
    rs_part[tid] = x;
    __syncthreads();
    if (tid < kCoarse) {
      uint32_t t = 0;
#pragma unroll
      for (int i = 0; i < kGroups; ++i) t += rs_part[i * kCoarse + tid];
      rs_tot[tid] = t;
    }
    __syncthreads();
  }
  int cstar = 0;
  for (int c = 1; c < kCoarse; ++c)
    if (rs_tot[c] >= krem) cstar = c;
  const uint32_t next_coarse = cstar + 1 < kCoarse ? rs_tot[cstar + 1] : 0u;
  __syncthreads();   // every thread has read rs_tot before the fine step reuses it
  // fine step: totals at bins 64 cstar + i, i < 64
  {
    constexpr int kGroups = kThreads / 64;
    const int i = tid % 64;
    uint32_t x = 0;
    for (int q = tid / 64; q < a.nchunk; q += kGroups) x += base[(int64_t)q * kBins + 64 * cstar + i];
    rs_part[tid] = x;
    __syncthreads();
    if (tid < 64) {
      uint32_t t = 0;
#pragma unroll
      for (int k = 0; k < kGroups; ++k) t += rs_part[k * 64 + tid];
      rs_tot[tid] = t;
    }
    __syncthreads();
  }
  int istar = 0;
  for (int i = 1; i < 64; ++i)
    if (rs_tot[i] >= krem) istar = i;
  digit = (uint32_t)(64 * cstar + istar);
  above = istar + 1 < 64 ? rs_tot[istar + 1] : next_coarse;
  __syncthreads();   // rs_tot is read by every thread before any later reuse
}

template <int kLevel>
__global__ __launch_bounds__(kThreads) void select_level(SelArgs a) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t wsum[kWaves];
  const int p = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  uint32_t* st = a.state + g * kStateWords;

  // the chunk (<= kMaxChunk candidates) with every load in flight at once,
  // from clamped addresses (entries past j1 are not counted); issued before
  // the digit resolution, whose round trips they overlap
  const int j0 = p * a.chunk, j1 = min(a.c, j0 + a.chunk);
  const uint32_t* v = a.imp + (int64_t)g * a.hs;
  uint32_t raw[kSegment];
#pragma unroll
  for (int e = 0; e < kSegment; ++e) raw[e] = v[min(j0 + tid + e * kThreads, j1 - 1)];
  for (int b = tid; b < kBins; b += kThreads) h[b] = 0u;

  // digits resolved so far: (key & pmask) == prefix marks the keys still live
  uint32_t prefix = 0, pmask = 0;
  if (kLevel >= 1) {
    const uint32_t krem = kLevel == 1 ? (uint32_t)a.k_top : st[kKrem1];
    if (kLevel == 2) {
      prefix = st[kD0] << level_shift(0);
      pmask = level_mask(0) << level_shift(0);
    }
    uint32_t d, above;
    resolve_digit(a, kLevel - 1, g, krem, wsum, d, above);
    prefix |= d << level_shift(kLevel - 1);
    pmask |= level_mask(kLevel - 1) << level_shift(kLevel - 1);
    if (p == 0 && tid == 0) {
      st[kLevel == 1 ? kD0 : kD1] = d;
      st[kLevel == 1 ? kKrem1 : kKrem2] = krem - above;
    }
  }
  __syncthreads();   // the cleared histogram
#pragma unroll
  for (int e = 0; e < kSegment; ++e) {
    const uint32_t key = order_key(raw[e]);
    if (j0 + tid + e * kThreads < j1 && (key & pmask) == prefix)
      atomicAdd(&h[(key >> level_shift(kLevel)) & level_mask(kLevel)], 1u);
  }
  __syncthreads();

  // inclusive suffix counts: the thread owns kBPT bins from base = kBPT*(last - tid)
  const int base = kBPT * (kThreads - 1 - tid);
  uint32_t hb[kBPT], sum = 0;
#pragma unroll
  for (int i = 0; i < kBPT; ++i) {
    hb[i] = h[base + i];
    sum += hb[i];
  }
  uint32_t tot;
  uint32_t s = block_excl_scan<kThreads>(sum, wsum, &tot);   // count in bins >= base + kBPT
  uint32_t* my = a.suf + (((int64_t)kLevel * gridDim.y + g) * a.nchunk + p) * kBins;
#pragma unroll
  for (int i = kBPT - 1; i >= 0; --i) {
    s += hb[i];
    my[base + i] = s;
  }
}

__global__ __launch_bounds__(kThreads) void select_emit(SelArgs a) {
  __shared__ uint32_t keys[kMaxChunk + kMaxChunk / 64];   // candidate j at j + j/64
  __shared__ uint32_t wsum[kWaves];
  const int p = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const uint32_t* st = a.state + g * kStateWords;
  int32_t* o = a.out + (int64_t)g * a.budget;
  if (p == 0)
    for (int t = tid; t < a.recent; t += kThreads) o[a.k_top + t] = a.S - a.recent + t;
  const int j0 = p * a.chunk, cnt = min(a.c, j0 + a.chunk) - j0;
  const uint32_t* v = a.imp + (int64_t)g * a.hs + j0;
  {
    uint32_t raw[kSegment];   // every load in flight at once, clamped addresses
#pragma unroll
    for (int e = 0; e < kSegment; ++e) raw[e] = v[min(tid + e * kThreads, cnt - 1)];
#pragma unroll
    for (int e = 0; e < kSegment; ++e) {
      const int j = tid + e * kThreads;
      if (j < cnt) keys[j + (j >> 6)] = order_key(raw[e]);
    }
  }

  // T = the k_top-th key; krem of the T-valued candidates are taken
  const uint32_t d0 = st[kD0], d1 = st[kD1], krem2 = st[kKrem2];
  uint32_t d2, above2;
  resolve_digit(a, 2, g, krem2, wsum, d2, above2);   // its barriers also publish `keys`
  const uint32_t T = (d0 << level_shift(0)) | (d1 << level_shift(1)) | d2;
  const uint32_t krem = krem2 - above2;

  // candidates kept before this chunk, from the earlier chunks' suffix counts
  uint32_t gt_q = 0, eq_q = 0;
  for (int q = tid; q < p; q += kThreads) {
    const uint32_t* s0 = chunk_suffix(a, 0, g, q);
    const uint32_t* s1 = chunk_suffix(a, 1, g, q);
    const uint32_t* s2 = chunk_suffix(a, 2, g, q);
    const uint32_t up0 = d0 + 1 < (uint32_t)kBins ? s0[d0 + 1] : 0u;
    const uint32_t up1 = d1 + 1 < (uint32_t)kBins ? s1[d1 + 1] : 0u;
    const uint32_t up2 = d2 + 1 < (uint32_t)kBins ? s2[d2 + 1] : 0u;
    gt_q += up0 + up1 + up2;
    eq_q += s2[d2] - up2;
  }
  uint32_t gt_before, eq_before;
  (void)block_excl_scan<kThreads>(gt_q, wsum, &gt_before);
  (void)block_excl_scan<kThreads>(eq_q, wsum, &eq_before);
  const uint32_t eq_room = krem > eq_before ? krem - eq_before : 0u;
  const uint32_t out0 = gt_before + (eq_before < krem ? eq_before : krem);

  // this chunk: the thread owns candidates [kSegment*tid, kSegment*tid + kSegment)
  const int seg = tid * kSegment;
  const int valid = min(kSegment, max(0, cnt - seg));
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int e = 0; e < kSegment; ++e) {
    const int j = seg + e;
    const uint32_t k = e < valid ? keys[j + (j >> 6)] : 0u;
    n_gt += (e < valid && k > T) ? 1u : 0u;
    n_eq += (e < valid && k == T) ? 1u : 0u;
  }
  uint32_t eq_tot, take_tot;
  const uint32_t eqx = block_excl_scan<kThreads>(n_eq, wsum, &eq_tot);
  const uint32_t room = eq_room > eqx ? eq_room - eqx : 0u;
  uint32_t eq_left = n_eq < room ? n_eq : room;   // T-valued candidates this thread keeps
  uint32_t pos = out0 + block_excl_scan<kThreads>(n_gt + eq_left, wsum, &take_tot);
#pragma unroll
  for (int e = 0; e < kSegment; ++e) {
    const int j = seg + e;
    const uint32_t k = e < valid ? keys[j + (j >> 6)] : 0u;
    const bool eq = e < valid && k == T && eq_left > 0;
    const bool take = (e < valid && k > T) || eq;
    eq_left -= eq ? 1u : 0u;
    if (take && pos < (uint32_t)a.k_top) o[pos] = j0 + j;
    pos += take ? 1u : 0u;
  }
}

// Chunking of c candidates over Hkv heads: about kTargetGroups workgroups, in
// chunks of 256..4096 candidates (multiples of 256).
void plan_chunks(int32_t Hkv, int32_t c, int* chunk, int* nchunk) {
  const int goal = (kTargetGroups + Hkv - 1) / Hkv;
  int ch = (c + goal - 1) / goal;
  ch = (ch + kThreads - 1) / kThreads * kThreads;
  ch = ch < kThreads ? kThreads : (ch > kMaxChunk ? kMaxChunk : ch);
  *chunk = ch;
  *nchunk = c > 0 ? (c + ch - 1) / ch : 1;
}

// Workspace words for nchunk chunks per head.
size_t workspace_words(int32_t Hkv, int nchunk) {
  return (size_t)3 * Hkv * nchunk * kBins + (size_t)Hkv * kStateWords;
}

// Most chunks any c <= n is cut into: at most the target count while the
// chunk size is free to grow, else n / 4096 rounded up.
int max_chunks(int32_t Hkv, int32_t n) {
  const int goal = (kTargetGroups + Hkv - 1) / Hkv;
  const int big = (n + kMaxChunk - 1) / kMaxChunk;
  return goal > big ? goal : big;
}

}  // namespace many

// Candidate counts up to one round of the single-workgroup kernel use it.
bool use_one_workgroup(int c) { return c <= one::kRound; }

}  // namespace
}  // namespace kvc

// Enough for every call with Hkv heads and at most n candidates.
extern "C" size_t kvc_select_topk_workspace_size(int32_t Hkv, int32_t n) {
  if (Hkv < 1 || n < 1) return 0;
  if (kvc::use_one_workgroup(n)) return 0;
  return kvc::many::workspace_words(Hkv, kvc::many::max_chunks(Hkv, n)) * sizeof(uint32_t);
}

extern "C" kvc_status kvc_select_topk(const float* importance, int64_t imp_head_stride, int32_t Hkv,
                                      int32_t S, int32_t w, int32_t recent, int32_t budget,
                                      int32_t* indices, void* ws, size_t ws_bytes, void* stream) {
  using namespace kvc;
  if (Hkv < 1 || S < 2 || w < 1 || w >= S || recent < 0 || recent > S) return KVC_E_ARG;
  const int32_t n = S - w;
  const int32_t c = n < S - recent ? n : S - recent;
  if (budget < recent || budget - recent > c) return KVC_E_ARG;
  if (imp_head_stride < n && Hkv > 1) return KVC_E_SHAPE;
  if (!indices || (!importance && budget > recent)) return KVC_E_ARG;
  if ((reinterpret_cast<uintptr_t>(importance) & 3) || (reinterpret_cast<uintptr_t>(indices) & 3))
    return KVC_E_ARG;
  if (Hkv > 65535) return KVC_E_SHAPE;
  if (budget == 0) return KVC_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int k_top = budget - recent;
  if (use_one_workgroup(c) || k_top == 0 || k_top >= c) {
    KVC_LAUNCH("select_topk", one::select_topk_kernel, dim3(Hkv), dim3(one::kSelThreads), s, importance,
               imp_head_stride, (int64_t)0, c, k_top, S, recent, budget, (const int32_t*)nullptr,
               (int64_t)Hkv * budget, indices);
    return KVC_OK;
  }

  int chunk, nchunk;
  many::plan_chunks(Hkv, c, &chunk, &nchunk);
  if (!ws || ws_bytes < many::workspace_words(Hkv, nchunk) * sizeof(uint32_t) ||
      (reinterpret_cast<uintptr_t>(ws) & 3))
    return KVC_E_WORKSPACE;
  many::SelArgs a;
  a.imp = reinterpret_cast<const uint32_t*>(importance);
  a.hs = imp_head_stride;
  a.c = c;
  a.k_top = k_top;
  a.S = S;
  a.recent = recent;
  a.budget = budget;
  a.chunk = chunk;
  a.nchunk = nchunk;
  a.out = indices;
  a.suf = static_cast<uint32_t*>(ws);
  a.state = a.suf + (size_t)3 * Hkv * nchunk * kBins;
  const dim3 grid(nchunk, Hkv);
  KVC_LAUNCH("select_level0", many::select_level<0>, grid, dim3(many::kThreads), s, a);
  KVC_LAUNCH("select_level1", many::select_level<1>, grid, dim3(many::kThreads), s, a);
  KVC_LAUNCH("select_level2", many::select_level<2>, grid, dim3(many::kThreads), s, a);
  KVC_LAUNCH("select_emit", many::select_emit, grid, dim3(many::kThreads), s, a);
  return KVC_OK;
}

extern "C" kvc_status kvc_select_topk_layers(const float* importance, int64_t imp_head_stride,
                                             int64_t imp_layer_stride, int32_t L, int32_t Hkv, int32_t S,
                                             int32_t w, int32_t recent, const int32_t* budgets,
                                             int32_t total_budget, int32_t* indices, void* stream) {
  using namespace kvc;
  if (L < 1 || Hkv < 1 || S < 2 || w < 1 || w >= S || recent < 0 || recent > S || total_budget < 0)
    return KVC_E_ARG;
  const int32_t n = S - w;
  const int32_t c = n < S - recent ? n : S - recent;
  if (!use_one_workgroup(c)) return KVC_E_UNSUPPORTED;
  if (Hkv > 65535 || L > 65535) return KVC_E_SHAPE;
  if ((imp_head_stride < n && Hkv > 1) || (imp_layer_stride < (int64_t)Hkv * imp_head_stride && L > 1))
    return KVC_E_SHAPE;
  if (!importance || !budgets || !indices) return KVC_E_ARG;
  if ((reinterpret_cast<uintptr_t>(importance) | reinterpret_cast<uintptr_t>(budgets) |
       reinterpret_cast<uintptr_t>(indices)) & 3)
    return KVC_E_ARG;
  if (total_budget == 0) return KVC_OK;
  KVC_LAUNCH("select_topk_layers", one::select_topk_kernel, dim3(Hkv, L), dim3(one::kSelThreads),
             static_cast<hipStream_t>(stream), importance, imp_head_stride, imp_layer_stride, c, 0, S, recent, 0,
             budgets, (int64_t)Hkv * total_budget, indices);
  return KVC_OK;
}
