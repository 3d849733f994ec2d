// kvc_decode_init_scores / kvc_keyformer_decode_step: Keyformer's decode phase.
//
// Keyformer blog page, closing paragraphs on the two phases: decoding runs on
// the reduced cache and each step's score is added to the score carried from
// before; the cache keeps the w most recent tokens and the other tokens with
// the highest score.  The step score is the Gumbel-noised tempered softmax of
// the Gumbel-distribution and temperature sections, summed over the query
// heads of a KV head.  One step: the new token (position t) attends over the B
// slots and itself; every slot's accumulated score grows by its step score;
// among the entries outside the recent window (positions <= t - recent) the
// lowest accumulated score leaves (ties: the smaller position, then the
// smaller slot) and the new token's key, value, position and step score take
// its slot.
//
// Design: two launches.  decode_logits, grid (chunks of 256 keys, KV heads):
// 16 lanes cover a 256-byte key row with 16-byte loads (8 rows per lane in
// flight) and dot it with the group's G queries (registers, kernel templated
// on G <= 8), 4 xor-shuffles finishing each product; then every thread adds
// the noise (keyed by the key's position, as in the prompt phase) and the
// temperature to its own entries, giving logits in log2 units, written to the
// workspace with the chunk's (max, sum of 2^(y - max)) per query head.
// decode_update, one workgroup of 16 waves per KV head: folds the chunk
// statistics in a fixed order into each head's softmax constants, then
// accumulates the step scores, finds the lowest (score, position, slot)
// outside the recent window with a two-stage 64-bit argmin and writes the new
// token there.  Every reduction runs in a fixed order: bit-reproducible.
#include "common.h"
#include "philox.h"

namespace kvc {
namespace {

constexpr int kD = 128;
constexpr int kDecThreads = 1024;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kMaxG = 8;

struct DecodeArgs {
  const uint16_t* q;        // [Hkv * G][D], head stride q_hs
  int64_t q_hs;
  const uint16_t* k_new;    // [Hkv][D]
  const uint16_t* v_new;
  uint16_t* kc;             // [Hkv][B][D]
  uint16_t* vc;
  int32_t* pos;             // [Hkv][B]
  float* acc;               // [Hkv][B]
  int32_t* evicted;         // [Hkv] or null
  int G, B, t, recent;
  float c;                  // scale * log2(e)
  float inv_tau;            // 1 / tau, 0 for tau = +inf
  uint32_t seed_lo, seed_hi;
};

__device__ __forceinline__ uint64_t block_min_u64(uint64_t v, uint64_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t u = __shfl_xor(v, o);
    v = u < v ? u : v;
  }
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint64_t m = red[0];
#pragma unroll
  for (int i = 1; i < kDecWaves; ++i) m = red[i] < m ? red[i] : m;
  return m;
}

constexpr int kChunkKeys = 256;            // keys per decode_logits workgroup
constexpr int kLogitThreads = 256;

template <int kWaves>
__device__ __forceinline__ float wg_max(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) m = fmaxf(m, red[i]);
  return m;
}

template <int kWaves>
__device__ __forceinline__ float wg_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) s += red[i];
  return s;
}

// kGmax: a power of two >= G (query registers and loop bounds sized for it).
// y[(g * G + hh) * N + j] in log2 units; stats[(g * nchunk + chunk) * G + hh].
template <int kGmax>
__global__ __launch_bounds__(kLogitThreads) void decode_logits(DecodeArgs a, float* y, float2* stats, int nchunk) {
  constexpr int kWaves = kLogitThreads / kWave;
  __shared__ float ys[kGmax][kChunkKeys];
  __shared__ float red[kWaves];
  const int chunk = blockIdx.x, g = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane & 15;
  const int N = a.B + 1, j_lo = chunk * kChunkKeys, nk = min(kChunkKeys, N - j_lo);
  const uint16_t* kg = a.kc + (int64_t)g * a.B * kD;
  const int32_t* pg = a.pos + (int64_t)g * a.B;

  float qv[kGmax][8];
#pragma unroll
  for (int hh = 0; hh < kGmax; ++hh) {
    if (hh < a.G) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(a.q + (int64_t)(g * a.G + hh) * a.q_hs + sub * 8);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[hh][2 * e] = __uint_as_float(ww[e] << 16);
        qv[hh][2 * e + 1] = __uint_as_float(ww[e] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[hh][e] = 0.f;
    }
  }

  // dot products: local key jl = 16 u + 4 wave + lane / 16, all 16 rows of a
  // lane in flight at once
  constexpr int kU = kChunkKeys / 16;
  for (int u0 = 0; u0 < kChunkKeys / 16; u0 += kU) {
    u32x4 w[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = j_lo + 16 * (u0 + u) + 4 * wave + (lane >> 4);
      const uint16_t* row = j < a.B ? kg + (int64_t)j * kD : a.k_new + (int64_t)g * kD;   // j >= B: new key
      w[u] = *reinterpret_cast<const u32x4*>(row + sub * 8);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int jl = 16 * (u0 + u) + 4 * wave + (lane >> 4);
      const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
      float kv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv[2 * e] = __uint_as_float(ww[e] << 16);
        kv[2 * e + 1] = __uint_as_float(ww[e] & 0xFFFF0000u);
      }
#pragma unroll
      for (int hh = 0; hh < kGmax; ++hh) {
        if (hh >= a.G) break;
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(kv[e], qv[hh][e], d);
        d += __shfl_xor(d, 8);
        d += __shfl_xor(d, 4);
        d += __shfl_xor(d, 2);
        d += __shfl_xor(d, 1);
        if (sub == 0) ys[hh][jl] = d;
      }
    }
  }
  __syncthreads();
  // noise and temperature with every lane busy: y = (x c + zeta log2 e) / tau
  for (int i = tid; i < a.G * nk; i += kLogitThreads) {
    const int hh = i / nk, jl = i - hh * nk, j = j_lo + jl;
    float v = 0.f;   // tau = +inf: uniform
    if (a.inv_tau != 0.f) {
      const int p = j < a.B ? pg[j] : a.t;
      const uint32_t h = (uint32_t)(g * a.G + hh);
      const u32x4 x = philox4x32_10(u32x4{(uint32_t)p >> 2, (uint32_t)a.t, h, 0u}, a.seed_lo, a.seed_hi);
      const uint32_t word = (p & 3) == 0 ? x.x : (p & 3) == 1 ? x.y : (p & 3) == 2 ? x.z : x.w;
      v = fmaf(ys[hh][jl], a.c, gumbel_log2_from_word(word)) * a.inv_tau;
    }
    ys[hh][jl] = v;
    y[((int64_t)g * a.G + hh) * N + j] = v;
  }
  __syncthreads();
  for (int hh = 0; hh < a.G; ++hh) {
    const float m = wg_max<kWaves>(tid < nk ? ys[hh][tid] : -INFINITY, red);
    const float l = wg_sum<kWaves>(tid < nk ? __builtin_amdgcn_exp2f(ys[hh][tid] - m) : 0.f, red);
    if (tid == 0) stats[((int64_t)g * nchunk + chunk) * a.G + hh] = float2{m, l};
  }
}

// kSlots > 0: the head's slots are held in registers, kSlots per thread
// (B <= kSlots * kDecThreads), and every independent load (chunk statistics,
// the thread's logits, scores and positions, the new token's logits and rows)
// is issued at the start, so the step pays one round trip to memory; the
// scores are written once, after the evicted slot is known.  kSlots = 0:
// strided loops over the slots, for any B.
template <int kGmax, int kSlots>
__global__ __launch_bounds__(kDecThreads) void decode_update(DecodeArgs a, const float* y, const float2* stats,
                                                             int nchunk) {
  __shared__ float red[kDecWaves];
  __shared__ uint64_t red64[kDecWaves];
  const int g = blockIdx.x, tid = threadIdx.x;
  const int N = a.B + 1;
  const int32_t* pg = a.pos + (int64_t)g * a.B;
  const float* yg = y + (int64_t)g * a.G * N;
  float* ag = a.acc + (int64_t)g * a.B;
  const int cut = a.t - a.recent;   // positions <= cut may leave

  // register path: this thread's slots j = tid + kDecThreads * s (clamped
  // addresses; slots past B are never used), the new token's logits and rows
  constexpr int kS = kSlots > 0 ? kSlots : 1;
  float yv[kS][kGmax], av[kS], ynew[kGmax];
  int pv[kS];
  u32x4 kn{}, vn{};
  if constexpr (kSlots > 0) {
#pragma unroll
    for (int s2 = 0; s2 < kSlots; ++s2) {
      const int j = min(tid + kDecThreads * s2, a.B - 1);
      av[s2] = ag[j];
      pv[s2] = pg[j];
#pragma unroll
      for (int hh = 0; hh < kGmax; ++hh) yv[s2][hh] = hh < a.G ? yg[(int64_t)hh * N + j] : 0.f;
    }
#pragma unroll
    for (int hh = 0; hh < kGmax; ++hh) ynew[hh] = hh < a.G ? yg[(int64_t)hh * N + a.B] : 0.f;
    if (tid < 16) {
      kn = *reinterpret_cast<const u32x4*>(a.k_new + (int64_t)g * kD + tid * 8);
      vn = *reinterpret_cast<const u32x4*>(a.v_new + (int64_t)g * kD + tid * 8);
    }
  }

  // each query head's softmax constants from the chunk statistics (fixed
  // order; with nchunk <= kDecThreads a thread holds at most one chunk)
  float m_h[kGmax], il_h[kGmax];
  float2 st[kGmax];
#pragma unroll
  for (int hh = 0; hh < kGmax; ++hh)
    st[hh] = (hh < a.G && tid < nchunk) ? stats[((int64_t)g * nchunk + tid) * a.G + hh] : float2{-INFINITY, 0.f};
  // Up to 64 chunks: wave 0 folds them alone and hands the constants over
  // through LDS (one barrier).  Its xor trees are those of the workgroup-wide
  // fold below, whose other waves would only add -inf to the max and +0 to
  // the sum, so both give the same bits.
  __shared__ float s_m[kGmax], s_il[kGmax];
  const bool one_wave = nchunk <= kWave;
  if (one_wave) {
    if (tid < kWave) {
#pragma unroll
      for (int hh = 0; hh < kGmax; ++hh) {
        if (hh >= a.G) break;
        float m = st[hh].x;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        float l = tid < nchunk ? st[hh].y * __builtin_amdgcn_exp2f(st[hh].x - m) : 0.f;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
        if (tid == 0) {
          s_m[hh] = m;
          s_il[hh] = 1.0f / l;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < kGmax; ++hh) {
      m_h[hh] = hh < a.G ? s_m[hh] : 0.f;
      il_h[hh] = hh < a.G ? s_il[hh] : 0.f;
    }
  }
#pragma unroll
  for (int hh = 0; hh < kGmax; ++hh) {
    if (one_wave || hh >= a.G) break;
    const float2* sh = stats + (int64_t)g * nchunk * a.G + hh;
    float mx = st[hh].x;
    for (int c = tid + kDecThreads; c < nchunk; c += kDecThreads) mx = fmaxf(mx, sh[(int64_t)c * a.G].x);
    const float m = wg_max<kDecWaves>(mx, red);
    float sm = tid < nchunk ? st[hh].y * __builtin_amdgcn_exp2f(st[hh].x - m) : 0.f;
    for (int c = tid + kDecThreads; c < nchunk; c += kDecThreads) {
      const float2 s1 = sh[(int64_t)c * a.G];
      sm += s1.y * __builtin_amdgcn_exp2f(s1.x - m);
    }
    const float l = wg_sum<kDecWaves>(sm, red);
    m_h[hh] = m;
    il_h[hh] = 1.0f / l;
  }
  // step score of an entry from its G logits (query heads in order)
  auto score_of = [&](const float* yy) {
    float sc = 0.f;
#pragma unroll
    for (int hh = 0; hh < kGmax; ++hh) {
      if (hh >= a.G) break;
      sc += __builtin_amdgcn_exp2f(yy[hh] - m_h[hh]) * il_h[hh];
    }
    return sc;
  };
  auto step_score = [&](int j) {
    float yy[kGmax];
#pragma unroll
    for (int hh = 0; hh < kGmax; ++hh) yy[hh] = hh < a.G ? yg[(int64_t)hh * N + j] : 0.f;
    return score_of(yy);
  };

  if constexpr (kSlots > 0) {
    // accumulate and find the lowest (score, position, slot) outside the
    // recent window: one workgroup reduction of (key, slot) pairs
    __shared__ uint32_t red_slot[kDecWaves];
    float nv[kSlots];
    uint64_t best = ~0ull;
    uint32_t bslot = ~0u;
#pragma unroll
    for (int s2 = 0; s2 < kSlots; ++s2) {
      nv[s2] = av[s2] + score_of(yv[s2]);
      if (tid + kDecThreads * s2 < a.B && pv[s2] <= cut) {
        const uint64_t key = ((uint64_t)__float_as_uint(nv[s2]) << 32) | (uint32_t)pv[s2];   // scores >= 0
        if (key < best) {   // slots ascend with s2: an equal key keeps the smaller slot
          best = key;
          bslot = (uint32_t)(tid + kDecThreads * s2);
        }
      }
    }
    auto take = [&](uint64_t k2, uint32_t s3) {
      if (k2 < best || (k2 == best && s3 < bslot)) {
        best = k2;
        bslot = s3;
      }
    };
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t k2 = __shfl_xor(best, o);
      const uint32_t s3 = (uint32_t)__shfl_xor((int)bslot, o);
      take(k2, s3);
    }
    if ((tid & (kWave - 1)) == 0) {
      red64[tid >> 6] = best;
      red_slot[tid >> 6] = bslot;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kDecWaves; ++i) take(red64[i], red_slot[i]);
    const int e = best == ~0ull ? -1 : (int)bslot;   // -1: nothing may leave, no eviction
    const float snew = score_of(ynew);
#pragma unroll
    for (int s2 = 0; s2 < kSlots; ++s2) {
      const int j = tid + kDecThreads * s2;
      if (j < a.B) ag[j] = j == e ? snew : nv[s2];
      if (j == e) a.pos[(int64_t)g * a.B + e] = a.t;
    }
    if (tid == 0 && a.evicted) a.evicted[g] = e;
    if (e >= 0 && tid < 16) {
      *reinterpret_cast<u32x4*>(a.kc + ((int64_t)g * a.B + e) * kD + tid * 8) = kn;
      *reinterpret_cast<u32x4*>(a.vc + ((int64_t)g * a.B + e) * kD + tid * 8) = vn;
    }
    return;
  }

  // any B: strided loops
  uint64_t best = ~0ull;
  for (int j = tid; j < a.B; j += kDecThreads) {
    const float nv = ag[j] + step_score(j);
    ag[j] = nv;
    const int p = pg[j];
    if (p <= cut) {
      const uint64_t key = ((uint64_t)__float_as_uint(nv) << 32) | (uint32_t)p;   // scores >= 0
      best = key < best ? key : best;
    }
  }
  best = block_min_u64(best, red64);
  uint64_t slot = ~0ull;
  if (best != ~0ull)
    for (int j = tid; j < a.B; j += kDecThreads) {
      const uint64_t key = ((uint64_t)__float_as_uint(ag[j]) << 32) | (uint32_t)pg[j];
      if (pg[j] <= cut && key == best) slot = (uint64_t)j < slot ? (uint64_t)j : slot;
    }
  slot = block_min_u64(slot, red64);
  if (slot == ~0ull) {   // nothing may leave (positions not below t - recent): no eviction
    if (tid == 0 && a.evicted) a.evicted[g] = -1;
    return;
  }
  const int e = (int)slot;
  // the new token takes slot e
  if (tid < 16) {
    const u32x4 k1 = *reinterpret_cast<const u32x4*>(a.k_new + (int64_t)g * kD + tid * 8);
    const u32x4 v1 = *reinterpret_cast<const u32x4*>(a.v_new + (int64_t)g * kD + tid * 8);
    *reinterpret_cast<u32x4*>(a.kc + ((int64_t)g * a.B + e) * kD + tid * 8) = k1;
    *reinterpret_cast<u32x4*>(a.vc + ((int64_t)g * a.B + e) * kD + tid * 8) = v1;
  }
  if (tid == 0) {
    ag[e] = step_score(a.B);
    a.pos[(int64_t)g * a.B + e] = a.t;
    if (a.evicted) a.evicted[g] = e;
  }
}

__global__ __launch_bounds__(256) void decode_init_scores(const float* imp, int64_t hs, const int32_t* idx,
                                                          int budget, int n, float* acc) {
  const int g = blockIdx.y, t = blockIdx.x * 256 + threadIdx.x;
  if (t >= budget) return;
  const int j = idx[(int64_t)g * budget + t];
  acc[(int64_t)g * budget + t] = (j >= 0 && j < n) ? imp[(int64_t)g * hs + j] : 0.f;
}

}  // namespace
}  // namespace kvc

extern "C" kvc_status kvc_decode_init_scores(const float* importance, int64_t imp_head_stride,
                                             const int32_t* indices, int32_t Hkv, int32_t budget, int32_t n,
                                             float* acc, void* stream) {
  using namespace kvc;
  if (Hkv < 1 || budget < 0 || n < 0) return KVC_E_ARG;
  if (Hkv > 65535) return KVC_E_SHAPE;
  if (Hkv > 1 && imp_head_stride < n) return KVC_E_SHAPE;
  if (budget == 0) return KVC_OK;
  if (!importance || !indices || !acc) return KVC_E_ARG;
  if ((reinterpret_cast<uintptr_t>(importance) | reinterpret_cast<uintptr_t>(indices) |
       reinterpret_cast<uintptr_t>(acc)) & 3)
    return KVC_E_ARG;
  KVC_LAUNCH("decode_init_scores", decode_init_scores, dim3((budget + 255) / 256, Hkv), dim3(256),
             static_cast<hipStream_t>(stream), importance, imp_head_stride, indices, budget, n, acc);
  return KVC_OK;
}

namespace kvc {
namespace {

struct DecodeWs {
  size_t y, stats, total;
  int nchunk;
};

DecodeWs decode_ws(int Hkv, int G, int B) {
  DecodeWs w{};
  w.nchunk = (B + 1 + kChunkKeys - 1) / kChunkKeys;
  w.y = 0;
  w.stats = align_up((size_t)Hkv * G * (B + 1) * sizeof(float), 256);
  w.total = w.stats + align_up((size_t)Hkv * w.nchunk * G * sizeof(float2), 256);
  return w;
}

}  // namespace
}  // namespace kvc

extern "C" size_t kvc_keyformer_decode_step_workspace_size(int32_t Hkv, int32_t G, int32_t B) {
  if (Hkv < 1 || G < 1 || G > kvc::kMaxG || B < 2) return 0;
  return kvc::decode_ws(Hkv, G, B).total;
}

extern "C" kvc_status kvc_keyformer_decode_step(const void* q, int64_t q_head_stride, const void* k_new,
                                                const void* v_new, void* k_cache, void* v_cache, int32_t* pos,
                                                float* acc, int32_t Hkv, int32_t G, int32_t B, int32_t D,
                                                int32_t t, int32_t recent, float scale, float tau,
                                                uint64_t seed, int32_t* evicted, void* workspace,
                                                size_t workspace_bytes, void* stream) {
  using namespace kvc;
  if (Hkv < 1 || G < 1 || B < 2 || t < 0 || recent < 1 || recent >= B) return KVC_E_ARG;
  if (!(scale > 0.f && scale < INFINITY) || !(tau > 0.f)) return KVC_E_ARG;   // tau = +inf allowed
  if (D != kD) return KVC_E_UNSUPPORTED;
  if (G > kMaxG) return KVC_E_UNSUPPORTED;
  if (Hkv > 65535 || (int64_t)Hkv * G > 65535 || B > (1 << 28)) return KVC_E_SHAPE;
  if (q_head_stride < D || (q_head_stride & 7)) return KVC_E_SHAPE;
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !pos || !acc) return KVC_E_ARG;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return KVC_E_ARG;
  if ((reinterpret_cast<uintptr_t>(pos) | reinterpret_cast<uintptr_t>(acc) |
       reinterpret_cast<uintptr_t>(evicted)) & 3)
    return KVC_E_ARG;
  const DecodeWs W = decode_ws(Hkv, G, B);
  if (!workspace || workspace_bytes < W.total || !aligned16(workspace)) return KVC_E_WORKSPACE;
  float* y = reinterpret_cast<float*>(static_cast<char*>(workspace) + W.y);
  float2* stats = reinterpret_cast<float2*>(static_cast<char*>(workspace) + W.stats);
  DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.q_hs = q_head_stride;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.kc = static_cast<uint16_t*>(k_cache);
  a.vc = static_cast<uint16_t*>(v_cache);
  a.pos = pos;
  a.acc = acc;
  a.evicted = evicted;
  a.G = G;
  a.B = B;
  a.t = t;
  a.recent = recent;
  a.c = scale * kLog2e;
  a.inv_tau = tau == INFINITY ? 0.f : 1.0f / tau;
  a.seed_lo = (uint32_t)(seed & 0xFFFFFFFFull);
  a.seed_hi = (uint32_t)(seed >> 32);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 lg(W.nchunk, Hkv);
  // slots per thread of the update's register path (0: strided loops); 8 only
  // for G <= 4 (with 8 query heads the 64 logits of 8 slots would spill)
  const int slots = B <= 4 * kDecThreads ? 4 : (B <= 8 * kDecThreads && G <= 4 ? 8 : 0);
#define KVC_UPDATE(GM, NS)                                                                                    \
  KVC_LAUNCH("keyformer_decode_update", (decode_update<GM, NS>), dim3(Hkv), dim3(kDecThreads), s, a,         \
             static_cast<const float*>(y), static_cast<const float2*>(stats), W.nchunk)
#define KVC_DECODE(GM)                                                                                        \
  do {                                                                                                        \
    KVC_LAUNCH("keyformer_decode_logits", decode_logits<GM>, lg, dim3(kLogitThreads), s, a, y, stats, W.nchunk); \
    if (slots == 4)                                                                                           \
      KVC_UPDATE(GM, 4);                                                                                      \
    else if (slots == 8)                                                                                      \
      KVC_UPDATE(GM, (GM <= 4 ? 8 : 0));                                                                      \
    else                                                                                                      \
      KVC_UPDATE(GM, 0);                                                                                      \
  } while (0)
  if (G == 1)
    KVC_DECODE(1);
  else if (G == 2)
    KVC_DECODE(2);
  else if (G <= 4)
    KVC_DECODE(4);
  else
    KVC_DECODE(8);
#undef KVC_DECODE
#undef KVC_UPDATE
  return KVC_OK;
}
