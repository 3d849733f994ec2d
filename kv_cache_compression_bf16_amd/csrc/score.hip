// kvc_score: observation-window importance on gfx950.
//
// What is computed (ZigZagKV blog page, SnapKV section; ThinK page, query-driven
// pruning; Keyformer blog page, Gumbel-distribution section): for every KV
// head g the G*w window query rows of its query heads are scored against the
// n = S - w prefix keys, each row is softmax-normalised over the prefix, and
// the normalised rows are summed into a per-key importance (times 1/w).
//
// Design (two passes over the keys, same grid):
//  * A workgroup owns 256 consecutive prefix keys of one KV head (4 waves x
//    64 keys).  Each wave holds its 64 keys in registers, already in the A
//    operand layout of v_mfma_f32_32x32x16_bf16, for the whole kernel: K is
//    read from HBM exactly once per pass, straight into VGPRs.
//  * The G*w query rows of the group stream through LDS in blocks of 32 rows
//    (8.5 KB, double-buffered, rows padded by 16 bytes so the MFMA B-operand
//    reads are bank-conflict free and need no per-block address math).
//  * The tile is computed as K x Q^T, so a lane owns ONE query row and 16 keys
//    of each 32x32 tile: row statistics (pass 1) and the per-row softmax
//    constant (pass 2) are per-lane scalars, and column sums over query rows
//    accumulate in registers across all query blocks; the 32-lane reduction
//    happens once per workgroup at the end.  Every key column has a single
//    owner, so no atomics are used and results are bit-reproducible.
//  * Pass 1 writes per-(row, workgroup) partials (max, sum of exp2) in log2
//    units; a combine kernel folds them per row in a fixed order into
//    rowc = m + log2(l); pass 2 recomputes the logits and accumulates
//    exp2(t - rowc).
//  * Keyformer noise: lane values come in groups of 4 consecutive, 4-aligned
//    keys, which is exactly one Philox4x32-10 block, so every Philox call is
//    fully used.
#include <math.h>

#include <type_traits>

#include "common.h"


namespace kvc {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kTiles = 2;                              // 32-key tiles per wave
constexpr int kKeysPerWave = 32 * kTiles;
constexpr int kKeysPerBlock = kKeysPerWave * kWaves;   // 256
constexpr int kQRows = 32;
constexpr int kThreads = kWaves * kWave;
// LDS row pitch of a staged query row: 256 bytes + 16 bytes of padding, so the
// 16 lanes that read one 16-byte chunk of 16 different rows hit 16 distinct
// bank groups, and the 8 chunk reads of a lane are one base + immediates.
constexpr int kRowPitch = kD * 2 + 16;
constexpr int kQBlockBytes = kQRows * kRowPitch;

struct ScoreParams {
  const uint16_t* q;
  const uint16_t* k;
  int64_t q_hs, q_ls, k_hs, k_ls;
  float* imp;        // [L, Hkv, n]
  float2* part;      // [L, Hkv, nblk, R] (max, sum) in log2 units
  float* rowc;       // [L, Hkv, R]
  const float* layer_scales;
  float scale;
  float inv_tau;     // 1 / tau, 0 for tau = +inf
  float inv_w;
  uint32_t seed_lo, seed_hi;
  int L, Hkv, G, w, S, n, R, nblk, nqb;
};

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// multiply-high/low S-box on words 0 and 2 with the key bumped by the Weyl
// constants between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 x, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * x.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x.z;
    u32x4 y;
    y.x = (uint32_t)(p1 >> 32) ^ x.y ^ k0;
    y.y = (uint32_t)p1;
    y.z = (uint32_t)(p0 >> 32) ^ x.w ^ k1;
    y.w = (uint32_t)p0;
    x = y;
  }
  return x;
}

// Gumbel(0,1) noise from one 32-bit word, in log2 units: u = (2*(X>>9)+1) * 2^-24
// (exact in fp32) and zeta * log2(e) = -log2(-ln u) = -log2(-log2 u) - log2(ln 2).
// The hardware log2 is within 1.2e-7 relative of the exact value on every u of
// this grid, u -> 1 included, so the noise is good to about 1e-6 absolute.
__device__ __forceinline__ float gumbel_log2_from_word(uint32_t x) {
  const float u = (float)(((x >> 9) << 1) | 1u) * 0x1p-24f;
  return -__builtin_amdgcn_logf(-__builtin_amdgcn_logf(u)) + 0.52876637f;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool kPass2, bool kGumbel>
__global__ __launch_bounds__(kThreads) void score_pass(ScoreParams p) {
  __shared__ __attribute__((aligned(16))) char qs[2][kQBlockBytes];   // 2 x 8.5 KB
  __shared__ float2 red[2][kWaves][64];   // [.., 32 + col] is the unused half-wave copy

  const int blk = blockIdx.x, g = blockIdx.y, layer = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hb = lane >> 5, col = lane & 31;
  const int key0 = blk * kKeysPerBlock + wave * kKeysPerWave;
  const bool tail = blk * kKeysPerBlock + kKeysPerBlock > p.n;
  // w % 32 == 0: a 32-row query block never straddles two query heads and is
  // never partial, so its head / window offset are block-uniform scalars.
  const bool w32 = (p.w & 31) == 0;
  const float alpha = p.layer_scales ? p.layer_scales[layer] : p.scale;
  const float c = alpha * kLog2e;
  const int64_t head_row0 = ((int64_t)layer * p.Hkv + g) * p.R;

  // ---- K fragments: lane holds key (col) of tile t, 16-byte chunk (2s + hb).
  bf16x8 kf[kTiles][8];
  {
    const uint16_t* kb = p.k + layer * p.k_ls + g * p.k_hs;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      int j = key0 + t * 32 + col;
      j = j < p.n ? j : p.n - 1;   // clamp: keys past the prefix are masked in pass 1
      const bf16x8* row = reinterpret_cast<const bf16x8*>(kb + (int64_t)j * kD);
#pragma unroll
      for (int s = 0; s < 8; ++s) kf[t][s] = row[2 * s + hb];
    }
  }

  // ---- Q block staging: 512 16-byte chunks per 32-row block, 2 per thread
  // (rows tid/16 and tid/16 + 16, chunk tid%16), coalesced 256-byte rows.
  const uint16_t* qg = p.q + layer * p.q_ls + (int64_t)g * p.G * p.q_hs;
  const int q_toff = (tid >> 4) * kD + (tid & 15) * 8;           // element offset in a block
  const int st_off = (tid >> 4) * kRowPitch + (tid & 15) * 16;    // LDS byte offset, row tid/16
  const int rd_off = col * kRowPitch + hb * 16;                   // LDS byte offset of chunk hb
  // Blocks are loaded strictly in order, so with w % 32 == 0 the (query head,
  // window offset) of the next block to load is a running scalar pair: no
  // integer division (which the compiler would expand on the VALU).
  int ld_hh = 0, ld_i0 = 0;
  auto load_q = [&](int qb, u32x4 (&regs)[2]) {
    const int r0 = qb * kQRows;
    if (w32) {
      const uint16_t* src = qg + (ld_hh * p.q_hs + (int64_t)ld_i0 * kD) + q_toff;
      regs[0] = *reinterpret_cast<const u32x4*>(src);
      regs[1] = *reinterpret_cast<const u32x4*>(src + 16 * kD);
      ld_i0 += kQRows;
      if (ld_i0 == p.w) {
        ld_i0 = 0;
        ++ld_hh;
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = r0 + (tid >> 4) + 16 * u;
      if (r < p.R) {
        const int hh = r / p.w, i = r - hh * p.w;
        regs[u] = *reinterpret_cast<const u32x4*>(qg + hh * p.q_hs + (int64_t)i * kD + (tid & 15) * 8);
      } else {
        regs[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_q = [&](int buf, const u32x4 (&regs)[2]) {
    *reinterpret_cast<u32x4*>(qs[buf] + st_off) = regs[0];
    *reinterpret_cast<u32x4*>(qs[buf] + st_off + 16 * kRowPitch) = regs[1];
  };
  auto load_rc = [&](int qb) -> float {
    const int r = qb * kQRows + col;
    return (w32 || r < p.R) ? p.rowc[head_row0 + r] : INFINITY;
  };
  // Pass 1: wave 0 folds the 4 waves' statistics of block qb into one partial.
  auto store_partial = [&](int qb) {
    if (wave == 0 && hb == 0) {
      const int b = qb & 1;
      float m = -INFINITY;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) m = fmaxf(m, red[b][v][col].x);
      const float ms = (m == -INFINITY) ? 0.f : m;
      float l = 0.f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float2 a = red[b][v][col];
        l += a.y * fast_exp2(a.x - ms);
      }
      const int r = qb * kQRows + col;
      if (w32 || r < p.R) p.part[(head_row0 * p.nblk) + (int64_t)blk * p.R + r] = float2{m, l};
    }
  };
  // B operands from LDS, 8 k-steps x kTiles MFMAs: acc[t][r] = <K[key], Q[row]> with
  // key = key0 + 32t + 8(r/4) + 4hb + (r%4), row = 32qb + col.
  auto mfma_block = [&](int buf, f32x16 (&acc)[kTiles]) {
    const char* qsb = qs[buf] + rd_off;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) acc[t] = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 qf = *reinterpret_cast<const bf16x8*>(qsb + 32 * s);
#pragma unroll
      for (int t = 0; t < kTiles; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t][s], qf, acc[t], 0, 0, 0);
    }
  };
  // Keyformer path: t = (alpha x + zeta) * log2(e) / tau, in place.
  int ep_hh = 0, ep_i0 = 0;   // running (head, offset) of the block in the epilogue (w32 path)
  auto noisy = [&](f32x16 (&acc)[kTiles], int qb) {
    const int r = qb * kQRows + col;
    int hh, i;
    if (w32) {
      hh = ep_hh;
      i = ep_i0 + col;
      ep_i0 += kQRows;
      if (ep_i0 == p.w) {
        ep_i0 = 0;
        ++ep_hh;
      }
    } else {
      hh = r / p.w;
      i = r - hh * p.w;
    }
    const uint32_t h = (uint32_t)(g * p.G + hh);
    const uint32_t pos = (uint32_t)(p.S - p.w + i);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const uint32_t j0 = (uint32_t)(key0 + t * 32 + 8 * r4 + 4 * hb);
        const u32x4 x = philox4x32_10(u32x4{j0 >> 2, pos, h, 0u}, p.seed_lo, p.seed_hi);
        acc[t][4 * r4 + 0] = fmaf(acc[t][4 * r4 + 0], c, gumbel_log2_from_word(x.x)) * p.inv_tau;
        acc[t][4 * r4 + 1] = fmaf(acc[t][4 * r4 + 1], c, gumbel_log2_from_word(x.y)) * p.inv_tau;
        acc[t][4 * r4 + 2] = fmaf(acc[t][4 * r4 + 2], c, gumbel_log2_from_word(x.z)) * p.inv_tau;
        acc[t][4 * r4 + 3] = fmaf(acc[t][4 * r4 + 3], c, gumbel_log2_from_word(x.w)) * p.inv_tau;
      }
    }
  };

  f32x16 colacc[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) colacc[t] = f32x16{};

  // VALU half of one query block (other waves' MFMAs run meanwhile).
  auto epilogue = [&](auto clean_c, int qb, f32x16 (&acc)[kTiles], float rc) {
    constexpr bool kClean = decltype(clean_c)::value;
    if (kGumbel) noisy(acc, qb);
    // logit -> log2 units is fmaf(v, cc, -ref); the Keyformer path is already there
    const float cc = kGumbel ? 1.0f : c;
    if (!kPass2) {
      if (!kClean) {
        const bool row_ok = qb * kQRows + col < p.R;
#pragma unroll
        for (int t = 0; t < kTiles; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + t * 32 + 8 * (r >> 2) + 4 * hb + (r & 3);
            if (key >= p.n || !row_ok) acc[t][r] = -INFINITY;
          }
      }
      float mx = acc[0][0];
#pragma unroll
      for (int t = 0; t < kTiles; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[t][r]);
      const float mt = mx * cc;
      const float mts = (mx == -INFINITY) ? 0.f : mt;
      float l = 0.f;
#pragma unroll
      for (int t = 0; t < kTiles; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) l += fast_exp2(fmaf(acc[t][r], cc, -mts));
      // fold with the other half-wave (same query row, the other keys of each group)
      const float mo = __shfl_xor(mt, 32), lo = __shfl_xor(l, 32);
      const float m2 = fmaxf(mt, mo);
      const float m2s = (m2 == -INFINITY) ? 0.f : m2;
      const float l2 = l * fast_exp2(mt - m2s) + lo * fast_exp2(mo - m2s);
      red[qb & 1][wave][lane] = float2{m2, l2};   // lanes col and 32+col hold the same pair
    } else {
#pragma unroll
      for (int t = 0; t < kTiles; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) colacc[t][r] += fast_exp2(fmaf(acc[t][r], cc, -rc));
    }
  };

  u32x4 qreg[2];
  float rc_cur = 0.f;
  // The whole block loop, specialised for "clean" workgroups (no key past the
  // prefix, query blocks never partial: no masking code at all) and the rest.
  auto run = [&](auto clean_c) {
    load_q(0, qreg);
    store_q(0, qreg);
    if (p.nqb > 1) {
      load_q(1, qreg);
      store_q(1, qreg);
    }
    if (kPass2) rc_cur = load_rc(0);
    __syncthreads();
    // Plain loop: MFMAs then epilogue per block; latency is hidden across waves.
    for (int qb = 0; qb < p.nqb; ++qb) {
      const bool has_next2 = qb + 2 < p.nqb;
      if (has_next2) load_q(qb + 2, qreg);
      f32x16 acc[kTiles];
      mfma_block(qb & 1, acc);
      epilogue(clean_c, qb, acc, rc_cur);
      if (kPass2 && qb + 1 < p.nqb) rc_cur = load_rc(qb + 1);
      __syncthreads();                          // every wave is done with buffer qb & 1
      if (!kPass2) store_partial(qb);
      if (has_next2) store_q(qb & 1, qreg);     // visible after the next iteration's barrier
    }
  };
  if (!tail && w32)
    run(std::true_type{});
  else
    run(std::false_type{});

  if (!kPass2) return;

  // ---- pass 2: sum each key column over the 32 query lanes of its half-wave.
  float* out = p.imp + ((int64_t)layer * p.Hkv + g) * p.n;
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    float mine = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = colacc[t][r];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 1);
      if (col == r) mine = v;
    }
    if (col < 16) {
      const int key = key0 + t * 32 + 8 * (col >> 2) + 4 * hb + (col & 3);
      if (key < p.n) out[key] = mine * p.inv_w;
    }
  }
}

// Fold the per-workgroup partials of each query row into
// rowc = m + log2(sum_b l_b * 2^(m_b - m)).  A workgroup takes 32 consecutive
// rows of one head; its 8 thread groups each fold every 8th key block online
// (coalesced 256-byte reads), and the 8 group results are folded in a fixed
// order, so the result is bit-reproducible.
constexpr int kCombRows = 32, kCombGroups = 8;
__global__ __launch_bounds__(256) void score_combine(ScoreParams p, int heads) {
  __shared__ float2 sg[kCombGroups][kCombRows];
  const int rr = threadIdx.x & (kCombRows - 1), q = threadIdx.x / kCombRows;
  const int tiles = (p.R + kCombRows - 1) / kCombRows;
  const int head = blockIdx.x / tiles, r = (blockIdx.x - head * tiles) * kCombRows + rr;
  float m = -INFINITY, l = 0.f;
  if (head < heads && r < p.R) {
    const float2* pp = p.part + (int64_t)head * p.nblk * p.R + r;
#pragma unroll 4
    for (int b = q; b < p.nblk; b += kCombGroups) {
      const float2 a = pp[(int64_t)b * p.R];
      const float mn = fmaxf(m, a.x);
      const float ms = (mn == -INFINITY) ? 0.f : mn;
      l = l * fast_exp2(m - ms) + a.y * fast_exp2(a.x - ms);
      m = mn;
    }
  }
  sg[q][rr] = float2{m, l};
  __syncthreads();
  if (q == 0 && head < heads && r < p.R) {
    float mm = -INFINITY;
#pragma unroll
    for (int i = 0; i < kCombGroups; ++i) mm = fmaxf(mm, sg[i][rr].x);
    const float ms = (mm == -INFINITY) ? 0.f : mm;
    float ll = 0.f;
#pragma unroll
    for (int i = 0; i < kCombGroups; ++i) ll += sg[i][rr].y * fast_exp2(sg[i][rr].x - ms);
    p.rowc[(int64_t)head * p.R + r] = (ll > 0.f) ? mm + log2f(ll) : INFINITY;
  }
}

struct Plan {
  int n, G, R, nblk, nqb;
  size_t part_bytes, rowc_bytes, total;
};

kvc_status plan(const kvc_score_args* a, Plan* pl) {
  if (!a) return KVC_E_ARG;
  if (a->L < 1 || a->H < 1 || a->Hkv < 1 || a->w < 1 || a->S < 2 || a->D < 1) return KVC_E_ARG;
  if (a->H % a->Hkv) return KVC_E_SHAPE;
  if (a->w >= a->S) return KVC_E_SHAPE;
  if (a->D != kD) return KVC_E_UNSUPPORTED;
  if (a->L > 65535 || a->Hkv > 65535) return KVC_E_SHAPE;
  const int64_t G = a->H / a->Hkv;
  if (G * a->w > 65536) return KVC_E_SHAPE;
  if (a->q_head_stride < (int64_t)a->w * kD || a->k_head_stride < (int64_t)a->S * kD) return KVC_E_SHAPE;
  if (a->L > 1 && (a->q_layer_stride < a->H * a->q_head_stride ||
                   a->k_layer_stride < a->Hkv * a->k_head_stride))
    return KVC_E_SHAPE;
  if ((a->q_head_stride | a->k_head_stride | a->q_layer_stride | a->k_layer_stride) & 7) return KVC_E_ARG;
  if (!a->layer_scales && !(a->scale > 0.f && isfinite(a->scale))) return KVC_E_ARG;
  if (a->gumbel && !(a->tau > 0.f)) return KVC_E_ARG;   // rejects NaN; +inf allowed
  pl->n = a->S - a->w;
  pl->G = (int)G;
  pl->R = (int)(G * a->w);
  pl->nblk = (pl->n + kKeysPerBlock - 1) / kKeysPerBlock;
  pl->nqb = (pl->R + kQRows - 1) / kQRows;
  const size_t rows = (size_t)a->L * a->Hkv * pl->R;
  pl->part_bytes = align_up(rows * pl->nblk * sizeof(float2), 256);
  pl->rowc_bytes = align_up(rows * sizeof(float), 256);
  pl->total = pl->part_bytes + pl->rowc_bytes;
  return KVC_OK;
}

}  // namespace
}  // namespace kvc

extern "C" size_t kvc_score_workspace_size(const kvc_score_args* args) {
  kvc::Plan pl;
  return kvc::plan(args, &pl) == KVC_OK ? pl.total : 0;
}

extern "C" kvc_status kvc_score(const kvc_score_args* a, const void* q_obs, const void* k,
                                float* importance, void* ws, size_t ws_bytes, void* stream) {
  using namespace kvc;
  Plan pl;
  kvc_status st = plan(a, &pl);
  if (st != KVC_OK) return st;
  if (!q_obs || !k || !importance) return KVC_E_ARG;
  if (!aligned16(q_obs) || !aligned16(k) || (reinterpret_cast<uintptr_t>(importance) & 3)) return KVC_E_ARG;
  if (!ws || ws_bytes < pl.total || !aligned16(ws)) return KVC_E_WORKSPACE;

  ScoreParams p;
  p.q = static_cast<const uint16_t*>(q_obs);
  p.k = static_cast<const uint16_t*>(k);
  p.q_hs = a->q_head_stride;
  p.q_ls = a->q_layer_stride;
  p.k_hs = a->k_head_stride;
  p.k_ls = a->k_layer_stride;
  p.imp = importance;
  p.part = reinterpret_cast<float2*>(ws);
  p.rowc = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.part_bytes);
  p.layer_scales = a->layer_scales;
  p.scale = a->scale;
  p.inv_tau = a->gumbel ? (isinf(a->tau) ? 0.f : 1.0f / a->tau) : 0.f;
  p.inv_w = 1.0f / (float)a->w;
  p.seed_lo = (uint32_t)(a->seed & 0xFFFFFFFFull);
  p.seed_hi = (uint32_t)(a->seed >> 32);
  p.L = a->L;
  p.Hkv = a->Hkv;
  p.G = pl.G;
  p.w = a->w;
  p.S = a->S;
  p.n = pl.n;
  p.R = pl.R;
  p.nblk = pl.nblk;
  p.nqb = pl.nqb;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(pl.nblk, a->Hkv, a->L), block(kThreads);
  const int heads = a->L * a->Hkv;
  const dim3 comb_grid(heads * ((pl.R + kCombRows - 1) / kCombRows));
  if (a->gumbel) {
    KVC_LAUNCH("score_pass1_gumbel", (score_pass<false, true>), grid, block, s, p);
    KVC_LAUNCH("score_combine", score_combine, comb_grid, dim3(256), s, p, heads);
    KVC_LAUNCH("score_pass2_gumbel", (score_pass<true, true>), grid, block, s, p);
  } else {
    KVC_LAUNCH("score_pass1", (score_pass<false, false>), grid, block, s, p);
    KVC_LAUNCH("score_combine", score_combine, comb_grid, dim3(256), s, p, heads);
    KVC_LAUNCH("score_pass2", (score_pass<true, false>), grid, block, s, p);
  }
  return KVC_OK;
}
