// kvc_score: observation-window importance on gfx950.
//
// What is computed (ZigZagKV blog page, SnapKV section; ThinK page, query-driven
// pruning; Keyformer blog page, Gumbel-distribution section): for every KV
// head g the G*w window query rows of its query heads are scored against the
// n = S - w prefix keys, each row is softmax-normalised over the prefix, and
// the normalised rows are summed into a per-key importance (times 1/w).
//
// Design (two passes over the keys):
//  * Work is split into units of 32*kW*kT consecutive prefix keys of one KV
//    head.  A persistent grid (as many workgroups as fit on the device) gives
//    each workgroup a contiguous range of units.  Each wave holds its 32*kT
//    keys of the unit in registers, already in the A operand layout of
//    v_mfma_f32_32x32x16_bf16: K is read from HBM exactly once per pass,
//    straight into VGPRs.
//  * The G*w query rows of the unit's group are staged in LDS in chunks of up
//    to 32*cb rows (rows padded by 16 bytes so the MFMA B-operand reads are
//    bank-conflict free) and stay there for the next unit of the same head.
//    After the staging barrier every wave walks the query blocks on its own:
//    no barrier and no shared state inside the block loop.  A block's 8 query
//    fragments are read before its MFMA chains, so LDS latency is paid once
//    per block.  With kT = 2 each wave runs two independent MFMA chains.
//  * The tile is computed as K x Q^T, so a lane owns ONE query row and 16 keys
//    of each 32x32 tile: row statistics (pass 1) and the per-row softmax
//    constant (pass 2) are per-lane scalars, and column sums over query rows
//    accumulate in registers across all query blocks; the 32-lane reduction
//    happens once per unit.  Every key column has a single owner, so no
//    atomics are used and results are bit-reproducible.
//  * Pass 1 keeps each half-wave's per-row (max, sum of exp2) in registers and
//    folds the waves in a fixed order, 4 query blocks at a time through a
//    small LDS strip, into per-(row, unit) partials in log2 units; a combine
//    kernel folds those per row into rowc = m + log2(l); pass 2 recomputes
//    the logits and accumulates exp2(t - rowc).
//  * Keyformer noise: lane values come in groups of 4 consecutive, 4-aligned
//    keys, which is exactly one Philox4x32-10 block, so every Philox call is
//    fully used.
#include <limits.h>
#include <math.h>

#include <mutex>
#include <type_traits>

#include "common.h"
#include "philox.h"

// Scratch of kvc_score_noalloc: the scoring workspace (row-statistics partials
// and row constants) for callers that cannot allocate.  Every device the
// library runs on holds one copy, at its own address, until the process ends.
// Host code never passes this name to a kernel: it is a host-side stand-in;
// the device address comes from hipGetSymbolAddress (score_scratch_ptr).
static constexpr size_t kScoreScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kScoreScratchBytes];


namespace kvc {
namespace {

constexpr int kD = 128;
// LDS row pitch of a staged query row: 256 bytes + 16 bytes of padding, so the
// 16 lanes that read one 16-byte chunk of 16 different rows hit 16 distinct
// bank groups, and the 8 chunk reads of a lane are one base + immediates.
constexpr int kRowPitch = kD * 2 + 16;

// Shape of a scoring workgroup: kw waves, kt 32-key tiles per wave, and up to
// 32*cb staged query rows per chunk.  A unit of work is 32*kw*kt consecutive
// prefix keys of one KV head.
//  * R > 256: 8 waves x 2 tiles, 512-row chunks (one workgroup per CU, 2 waves
//    per SIMD, each with two independent MFMA chains);
//  * R <= 256: 4 waves x 2 tiles, chunks of up to 256 rows;
//  * Keyformer noise: 4 waves x 1 tile, 128-row chunks (Philox needs the
//    registers).
struct Shape {
  int kw, kt, cb;
};
inline Shape score_shape(int R, bool gumbel) {
  if (gumbel) return {4, 1, 4};
  if (R > 256) return {8, 2, 16};
  return {4, 2, 8};
}
inline int score_chunk_rows(int R, const Shape& sh) { return min((R + 31) / 32 * 32, 32 * sh.cb); }
inline size_t score_lds_bytes(int rows, int kw, bool pass2) {
  // staged rows, then the row constants (pass 2) or the 4-block fold strip (pass 1)
  return (size_t)rows * kRowPitch + (pass2 ? (size_t)rows * sizeof(float) : (size_t)4 * 32 * kw * 2 * sizeof(float2));
}


// Most units per head for which pass 2 folds the row constants itself: one
// step of loads per row.  Beyond it the fold's chain of round trips to
// memory, which pass 2 must wait for, costs more than the combine launch.
constexpr int kFuseRowcUnits = 32;
// Most segment partials per row that the segment passes' pass 2 folds itself
// (kFuseRowcUnits loads in flight per step).
constexpr int kFuseRowcSegments = 64;

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
  int L, Hkv, G, w, S, n, R, nblk, chunk_rows;
  int causal_unit;   // causal scoring: keys per unit (row r sees units b <= pos(r) / causal_unit); else 0
  int fuse_rowc;     // pass 2 folds the partials into the row constants itself (no combine launch)
  int seg_grid;      // > 0: pass 1 wrote one partial per (head, workgroup segment) and ran on
                     // this many workgroups (score_pass_seg); 0: one partial per (head, unit)
};

// Workgroup i runs on XCD i % 8.  With the grid a multiple of 8, the 8-wave
// segment passes number their workgroups XCD-major, so each XCD takes a
// contiguous eighth of the units: its L2 then holds the query rows and row
// partials of about an eighth of the heads (on the 32K-token GQA layer each
// XCD's workgroups load one head's 128 KB of rows instead of all eight), and
// a workgroup of pass 2 still finds the keys the same-numbered workgroup of
// pass 1 read last in its own L2.  The 4-wave passes keep the plain order,
// which measured faster there (131K-token layer, 64 rows per head).
__device__ inline int xcd_major_block(int nwg) {
  const int b = (int)blockIdx.x;
  return (nwg & 7) == 0 ? (b & 7) * (nwg >> 3) + (b >> 3) : b;
}

// Contiguous unit ranges over a grid of `grid` workgroups: the workgroup that
// owns unit u (every workgroup owns per or per + 1 consecutive units).
__host__ __device__ inline int unit_owner(int u, int total, int grid) {
  const int per = total / grid, extra = total % grid;
  const int big = extra * (per + 1);
  return u < big ? u / (per + 1) : extra + (u - big) / per;
}
// Partials of head h in segment mode: one per workgroup whose range meets the
// head's units [h*nblk, (h+1)*nblk), indexed from the first of them.
__host__ __device__ inline int head_segments(int h, int nblk, int total, int grid) {
  return unit_owner((h + 1) * nblk - 1, total, grid) - unit_owner(h * nblk, total, grid) + 1;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// For each of the 16 values v[e] of a lane, the sum over the 32 lanes of its
// half-wave, as a butterfly of DPP moves (no LDS round trip).  Four steps
// within each 16-lane row -- row mirror, half-row mirror, quad xor 2, quad
// xor 1 -- each pair two lanes that hold the same set of partial values; each
// lane keeps the half of the set its position selects and adds its partner's
// copy of that half, so position i of a row ends with the row sum of value i.
// One exchange between the two rows of the half-wave completes the sum.  Lane
// col of a half-wave returns the total of value col & 15.  A fixed order:
// bit-reproducible.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float half_wave_sum16_dpp(const f32x16& v, int col) {
  const int i = col & 15;
  const bool k1 = i & 8, k2 = i & 4, k3 = i & 2, k4 = i & 1;
  // keep + partner's copy of it: the partner (opposite selector) sends what
  // this lane keeps.  The selects act on the operands, before the move, so
  // every lane runs every move.
  auto step = [](bool k, float a, float b, auto ctrl_c) {
    const float keep = k ? b : a, send = k ? a : b;
    return keep + dpp_f32<decltype(ctrl_c)::value>(send);
  };
  using Mirror = std::integral_constant<int, 0x140>;      // row mirror: lane i with 15 - i
  using HalfMirror = std::integral_constant<int, 0x141>;  // half-row mirror: i with 7 - i in each half
  using Xor2 = std::integral_constant<int, 0x4E>;         // quad_perm [2,3,0,1]
  using Xor1 = std::integral_constant<int, 0xB1>;         // quad_perm [1,0,3,2]
  float w[8], x[4], y[2];
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = step(k1, v[e], v[e + 8], Mirror{});
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = step(k2, w[e], w[e + 4], HalfMirror{});
#pragma unroll
  for (int e = 0; e < 2; ++e) y[e] = step(k3, x[e], x[e + 2], Xor2{});
  const float z = step(k4, y[0], y[1], Xor1{});
  return z + __shfl_xor(z, 16);
}

// kCausal: keys [0, S) and window row i (position S - w + i) sees the keys at
// positions <= its own; w % 32 == 0, so no 32-row query block spans two heads.
// kPF: tiles of the next unit's keys prefetched during this unit (0..kT).
template <bool kPass2, bool kGumbel, bool kCausal, int kW, int kT, int kCB, int kPF>
__global__ __launch_bounds__(kW * kWave, kGumbel ? 3 : 1) void score_pass(ScoreParams p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int kThreads = kW * kWave;
  constexpr int kKeysPerWave = 32 * kT;
  constexpr int kKeysPerUnit = kKeysPerWave * kW;
  constexpr int kFoldBlocks = 4;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hb = lane >> 5, col = lane & 31;
  const int rows_alloc = p.chunk_rows;
  float* rcs = reinterpret_cast<float*>(lds + (size_t)rows_alloc * kRowPitch);    // pass 2: [rows]
  float2* fold = reinterpret_cast<float2*>(lds + (size_t)rows_alloc * kRowPitch); // pass 1: [kW][128][2]

  // row r -> (query head r / w, window offset r % w): a float estimate of the
  // quotient, then one exact integer correction (r < 2^16 + 32, so the
  // estimate is off by at most one).
  const float inv_w = 1.0f / (float)p.w;
  auto split_row = [&](int r, int& hh, int& ii) {
    hh = (int)((float)r * inv_w);
    ii = r - hh * p.w;
    if (ii < 0) { --hh; ii += p.w; }
    if (ii >= p.w) { ++hh; ii -= p.w; }
  };
  // prompt position of window row r (row past R: past every key)
  auto row_pos = [&](int r) {
    if (r >= p.R) return p.S;
    int hh, ii;
    split_row(r, hh, ii);
    return p.S - p.w + ii;
  };

  // This workgroup's units u = (layer*Hkv + g)*nblk + blk: a contiguous range,
  // or (causal: a unit's work shrinks with blk) every gridDim.x-th unit of the
  // order (blk, head), so each workgroup gets a mix and the costly ones first.
  const int heads = p.L * p.Hkv;
  const int total = heads * p.nblk;
  const int per = total / (int)gridDim.x, extra = total % (int)gridDim.x;
  const int u_first = (int)blockIdx.x * per + min((int)blockIdx.x, extra);
  const int n_units = kCausal ? (total - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x
                              : per + ((int)blockIdx.x < extra ? 1 : 0);
  auto unit_at = [&](int it) {
    // pass 2 walks its range backwards: it starts on the keys pass 1 read
    // last, which the same workgroup index may still find in its XCD's L2
    if (!kCausal) return kPass2 ? u_first + n_units - 1 - it : u_first + it;
    const int v = (int)blockIdx.x + it * (int)gridDim.x;
    const int blk = v / heads, head = v - blk * heads;
    return head * p.nblk + blk;
  };

  // K fragments of unit u: lane holds key (32t + col) of its wave's tiles,
  // 16-byte chunk (2s + hb), already in the MFMA A-operand layout; tiles
  // [t0, t0 + kN) into dst[0 .. kN).
  auto load_tiles = [&](int u, int t0, auto n_c, bf16x8 (*dst)[8]) {
    constexpr int kN = decltype(n_c)::value;
    const int head = u / p.nblk, blk = u - head * p.nblk;
    const int layer = head / p.Hkv, g = head - layer * p.Hkv;
    const uint16_t* kb = p.k + layer * p.k_ls + g * p.k_hs;
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int t = t0 + i;
      const int j = min(blk * kKeysPerUnit + wave * kKeysPerWave + t * 32 + col, p.n - 1);   // clamp; masked
      const bf16x8* row = reinterpret_cast<const bf16x8*>(kb + (int64_t)j * kD);
#pragma unroll
      for (int s = 0; s < 8; ++s) dst[i][s] = row[2 * s + hb];
    }
  };
  auto load_k = [&](int u, bf16x8 (&dst)[kT][8]) {
    const int head = u / p.nblk, blk = u - head * p.nblk;
    const int layer = head / p.Hkv, g = head - layer * p.Hkv;
    const uint16_t* kb = p.k + layer * p.k_ls + g * p.k_hs;
#pragma unroll
    for (int t = 0; t < kT; ++t) {
      const int j = min(blk * kKeysPerUnit + wave * kKeysPerWave + t * 32 + col, p.n - 1);   // clamp; masked
      const bf16x8* row = reinterpret_cast<const bf16x8*>(kb + (int64_t)j * kD);
#pragma unroll
      for (int s = 0; s < 8; ++s) dst[t][s] = row[2 * s + hb];
    }
  };

  // The first kPF tiles of the next unit are loaded during this one (after any
  // staging, unconditionally -- the last unit reloads itself -- so the count
  // of outstanding loads is the same on every path and the block loop never
  // waits for them).
  bf16x8 kf[kT][8];
  bf16x8 kn[kPF > 0 ? kPF : 1][8];
  if (n_units > 0) load_k(unit_at(0), kf);
  int staged = -1;   // head whose query rows are in LDS (single-chunk case)
  for (int it = 0; it < n_units; ++it) {
    const int u = unit_at(it);
    const int head = u / p.nblk, blk = u - head * p.nblk;
    const int layer = head / p.Hkv, g = head - layer * p.Hkv;
    if (it != 0) {
      if (kPF > 0) {
#pragma unroll
        for (int t = 0; t < kPF; ++t)
#pragma unroll
          for (int s2 = 0; s2 < 8; ++s2) kf[t][s2] = kn[t][s2];
      }
      if (kPF < kT) load_tiles(u, kPF, std::integral_constant<int, kT - kPF>{}, kf + kPF);
    }

    const int key0 = blk * kKeysPerUnit + wave * kKeysPerWave;
    const bool wave_full = key0 + kKeysPerWave <= p.n;   // no key of this wave past the prefix
    const float alpha = p.layer_scales ? p.layer_scales[layer] : p.scale;
    const float c = alpha * kLog2e;
    // logit -> log2 units is fmaf(v, cc, -ref); the Keyformer path is already there
    const float cc = kGumbel ? 1.0f : c;
    const int64_t head_row0 = (int64_t)head * p.R;
    const uint16_t* qg = p.q + layer * p.q_ls + (int64_t)g * p.G * p.q_hs;

    // stage query rows [c0, c0 + nrows) into LDS (zero rows past R), 8
    // independent 16-byte loads in flight per thread, addresses clamped.
    auto stage = [&](int c0, int nrows) {
      const int tot = nrows * 16;
      for (int base = 0; base < tot; base += 8 * kThreads) {
        u32x4 v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = base + e * kThreads + tid;
          const int r = min(c0 + (i >> 4), p.R - 1);
          int hh, ii;
          split_row(r, hh, ii);
          v[e] = *reinterpret_cast<const u32x4*>(qg + hh * p.q_hs + (int64_t)ii * kD + (i & 15) * 8);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = base + e * kThreads + tid;
          if (i < tot) {
            const bool ok = c0 + (i >> 4) < p.R;
            *reinterpret_cast<u32x4*>(lds + (i >> 4) * kRowPitch + (i & 15) * 16) = ok ? v[e] : u32x4{0u, 0u, 0u, 0u};
          }
        }
      }
      constexpr bool kCanFuse = kPass2 && !kGumbel && !kCausal;   // the Keyformer shape has no registers to spare
      if (kPass2 && !(kCanFuse && p.fuse_rowc))
        for (int i = tid; i < nrows; i += kThreads) {
          const int r = c0 + i;
          rcs[i] = r < p.R ? p.rowc[head_row0 + r] : INFINITY;
        }
      if (kCanFuse && p.fuse_rowc)
        // rowc = m + log2(sum_b l_b 2^(m_b - m)) over the head's units, one
        // thread per row, kFuseStep units per step in order (loads from a
        // clamped unit index, so none waits on a branch)
        for (int i = tid; i < nrows; i += kThreads) {
          constexpr int kFuseStep = kFuseRowcUnits;   // one step: every unit's load in flight at once
          const int r = min(c0 + i, p.R - 1);
          const float2* pp = p.part + head_row0 * p.nblk + r;
          float m = -INFINITY, l = 0.f;
          for (int b0 = 0; b0 < p.nblk; b0 += kFuseStep) {
            float2 a[kFuseStep];
#pragma unroll
            for (int e = 0; e < kFuseStep; ++e) a[e] = pp[(int64_t)min(b0 + e, p.nblk - 1) * p.R];
            float mn = m;
#pragma unroll
            for (int e = 0; e < kFuseStep; ++e) mn = fmaxf(mn, b0 + e < p.nblk ? a[e].x : -INFINITY);
            const float ms = (mn == -INFINITY) ? 0.f : mn;
            float acc = l * fast_exp2(m - ms);
#pragma unroll
            for (int e = 0; e < kFuseStep; ++e) acc += b0 + e < p.nblk ? a[e].y * fast_exp2(a[e].x - ms) : 0.f;
            m = mn;
            l = acc;
          }
          rcs[i] = (c0 + i < p.R && l > 0.f) ? m + log2f(l) : INFINITY;
        }
    };
    // A operands from registers, B operand (32 query rows) from LDS:
    // acc[t][e] = <K[key], Q[row]>, key = key0 + 32t + 8(e/4) + 4hb + (e%4), row = 32qb + col.
    // All 8 fragments of the block are read first, so the LDS latency is paid
    // once per block rather than once per k-step.
    auto mfma_block = [&](int qb, f32x16 (&acc)[kT]) {
      const char* qsb = lds + (qb * 32 + col) * kRowPitch + hb * 16;
      bf16x8 qf[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qsb + 32 * s);
#pragma unroll
      for (int t = 0; t < kT; ++t) acc[t] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int t = 0; t < kT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t][s], qf[s], acc[t], 0, 0, 0);
    };
    // Keyformer path: t = (alpha x + zeta) * log2(e) / tau, in place, for row r.
    auto noisy = [&](f32x16 (&acc)[kT], int r) {
      int hh, i;
      split_row(r, hh, i);
      const uint32_t h = (uint32_t)(g * p.G + hh);
      const uint32_t pos = (uint32_t)(p.S - p.w + i);
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const uint32_t j0 = (uint32_t)(key0 + 32 * t + 8 * r4 + 4 * hb);
          const u32x4 x = philox4x32_10(u32x4{j0 >> 2, pos, h, 0u}, p.seed_lo, p.seed_hi);
          acc[t][4 * r4 + 0] = fmaf(acc[t][4 * r4 + 0], c, gumbel_log2_from_word(x.x)) * p.inv_tau;
          acc[t][4 * r4 + 1] = fmaf(acc[t][4 * r4 + 1], c, gumbel_log2_from_word(x.y)) * p.inv_tau;
          acc[t][4 * r4 + 2] = fmaf(acc[t][4 * r4 + 2], c, gumbel_log2_from_word(x.z)) * p.inv_tau;
          acc[t][4 * r4 + 3] = fmaf(acc[t][4 * r4 + 3], c, gumbel_log2_from_word(x.w)) * p.inv_tau;
        }
    };
    // Pass 1, one query block: (max, sum of exp2) of the lane's row over the
    // lane's own keys; the two half-waves (the same rows, other keys) are
    // folded later with the other waves.
    auto row_stats = [&](auto clean_c, f32x16 (&acc)[kT], int r) -> float2 {
      constexpr bool kClean = decltype(clean_c)::value;
      if (!kClean) {
        const int rpos = kCausal ? row_pos(r) : 0;
#pragma unroll
        for (int t = 0; t < kT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = key0 + 32 * t + 8 * (e >> 2) + 4 * hb + (e & 3);
            if (key >= p.n || r >= p.R || (kCausal && key > rpos)) acc[t][e] = -INFINITY;
          }
      }
      float mx = acc[0][0];
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[t][e]);
      const float mt = mx * cc;
      const float mts = (mx == -INFINITY) ? 0.f : mt;
      float l = 0.f;
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) l += fast_exp2(fmaf(acc[t][e], cc, -mts));
      return float2{mt, l};
    };

    f32x16 colacc[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) colacc[t] = f32x16{};
    for (int c0 = 0; c0 < p.R; c0 += rows_alloc) {
      const int nrows = min(rows_alloc, (p.R - c0 + 31) / 32 * 32);
      const int nb = nrows / 32;
      const bool rows_full = c0 + nrows <= p.R;
      // causal: positions of the chunk's rows; skip a chunk no row of which
      // sees this unit (uniform over the workgroup), and take the unmasked
      // path only where every key of this wave is visible to every row
      bool causal_clean = true;
      if (kCausal) {
        int h0, i0, h1, i1;
        split_row(c0, h0, i0);
        split_row(min(c0 + nrows, p.R) - 1, h1, i1);
        const int pmin = h0 == h1 ? p.S - p.w + i0 : p.S - p.w;
        const int pmax = h0 == h1 ? p.S - p.w + i1 : p.S - 1;
        if (pmax < blk * kKeysPerUnit) continue;
        causal_clean = pmin >= key0 + kKeysPerWave - 1;
      }
      if (p.R > rows_alloc || head != staged) {
        __syncthreads();   // every wave is done with the previous rows
        stage(c0, nrows);
        __syncthreads();
        staged = head;
      }
      if (kPF > 0) {
        // this unit's K tiles and staged rows are in (the first MFMA needs
        // them anyway); then the next unit's first kPF tiles, which nothing
        // in the block loop waits for
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        load_tiles(unit_at(min(it + 1, n_units - 1)), 0, std::integral_constant<int, (kPF > 0 ? kPF : 1)>{}, kn);
      }
      if (!kPass2) {
        float2 st[kCB];   // per-block partials stay in registers until the chunk is done
        auto blocks = [&](auto clean_c) {
#pragma unroll
          for (int qb = 0; qb < kCB; ++qb) {
            st[qb] = float2{-INFINITY, 0.f};
            if (qb < nb) {
              f32x16 acc[kT];
              mfma_block(qb, acc);
              const int r = c0 + qb * 32 + col;
              if (kGumbel) noisy(acc, r);
              st[qb] = row_stats(clean_c, acc, r);
            }
          }
        };
        if (wave_full && rows_full && causal_clean)
          blocks(std::true_type{});
        else
          blocks(std::false_type{});
        // fold the waves, kFoldBlocks query blocks at a time, in a fixed order
#pragma unroll
        for (int f0 = 0; f0 < kCB; f0 += kFoldBlocks) {
          if (f0 < nb) {
#pragma unroll
            for (int qq = 0; qq < kFoldBlocks; ++qq)
              if (f0 + qq < kCB && f0 + qq < nb) fold[((wave * kFoldBlocks + qq) * 32 + col) * 2 + hb] = st[f0 + qq];
            __syncthreads();
            {
              // kTPR adjacent threads per row, each folding kPer of its 2*kW
              // entries, then an xor tree over the kTPR (a fixed order; every
              // thread of the row ends with the same value)
              constexpr int kTPR = kThreads / (kFoldBlocks * 32);
              constexpr int kPer = 2 * kW / kTPR;
              static_assert(kTPR * kFoldBlocks * 32 == kThreads && kPer * kTPR == 2 * kW, "fold split");
              const int i = tid / kTPR, j = tid % kTPR;
              const int rr = f0 * 32 + i, r = c0 + rr;
              float2 e[kPer];
#pragma unroll
              for (int k = 0; k < kPer; ++k) {
                const int v = j * kPer + k;
                e[k] = fold[(v >> 1) * kFoldBlocks * 64 + i * 2 + (v & 1)];
              }
              float m = e[0].x;
#pragma unroll
              for (int k = 1; k < kPer; ++k) m = fmaxf(m, e[k].x);
              const float ms = (m == -INFINITY) ? 0.f : m;
              float l = 0.f;
#pragma unroll
              for (int k = 0; k < kPer; ++k) l += e[k].y * fast_exp2(e[k].x - ms);
#pragma unroll
              for (int o = 1; o < kTPR; o <<= 1) {
                const float mo = __shfl_xor(m, o), lo = __shfl_xor(l, o);
                const float m2 = fmaxf(m, mo);
                const float m2s = (m2 == -INFINITY) ? 0.f : m2;
                l = l * fast_exp2(m - m2s) + lo * fast_exp2(mo - m2s);
                m = m2;
              }
              if (j == 0 && rr < nrows && r < p.R) p.part[head_row0 * p.nblk + (int64_t)blk * p.R + r] = float2{m, l};
            }
            __syncthreads();
          }
        }
      } else {
        for (int qb = 0; qb < nb; ++qb) {
          f32x16 acc[kT];
          mfma_block(qb, acc);
          if (kGumbel) noisy(acc, c0 + qb * 32 + col);
          if (kCausal && !causal_clean) {
            const int rpos = row_pos(c0 + qb * 32 + col);
#pragma unroll
            for (int t = 0; t < kT; ++t)
#pragma unroll
              for (int e = 0; e < 16; ++e)
                if (key0 + 32 * t + 8 * (e >> 2) + 4 * hb + (e & 3) > rpos) acc[t][e] = -INFINITY;
          }
          const float rc = rcs[qb * 32 + col];   // +inf for rows past R: adds 0
#pragma unroll
          for (int t = 0; t < kT; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) colacc[t][e] += fast_exp2(fmaf(acc[t][e], cc, -rc));
        }
      }
    }

    if (kPass2) {
      // sum each key column over the 32 query lanes of its half-wave (lane
      // col receives the total of value col & 15; the first row stores it)
      float* out = p.imp + (int64_t)head * p.n;
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        const float mine = half_wave_sum16_dpp(colacc[t], col);
        if (col < 16) {
          const int e = col;
          const int key = key0 + 32 * t + 8 * (e >> 2) + 4 * hb + (e & 3);
          if (key < p.n) out[key] = mine * p.inv_w;
        }
      }
    }
  }
}

// ---- window passes for 256 < G*w <= 512: statistics kept per segment -------
//
// The same tiling as score_pass's 8-wave shape (8 waves x 2 tiles of 32 keys,
// K in registers, the head's rows staged once in LDS), with three changes:
//  * Pass 1 keeps each lane's (max, sum) per query block across all of the
//    workgroup's units of a head and folds them once per head segment (not
//    once per unit), with a lazy reference: a block's exponentials are taken
//    against the row's running maximum; only when no maximum exists yet, or
//    the block would overflow it (a key far above it), is the block's own
//    maximum taken and the sum rescaled.  Partials are indexed by workgroup
//    segment (seg_grid mode), so a head has as many as workgroups meet it.
//  * Pass 2 folds those few partials into the row constants while staging
//    the rows, so no combine kernel runs between the passes.
//  * The next unit's key tiles that do not fit a prefetch register set are
//    loaded straight into the key registers once the last block's MFMAs have
//    read them, and the query fragments of the next block are read during
//    the current block's exponentials.
// (A barrier-synchronised ping-pong of the two waves of each SIMD -- one in
// its MFMAs while the other does exponentials -- measured slower than
// leaving the waves free.)

// f(integral_constant<int, Q>) for Q = I .. N-1, unrolled at compile time
// (register arrays indexed by Q stay in registers whatever the body's size).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// kPreQ: read the next block's query fragments during the current block's
// exponentials (else at the start of each block, which frees their registers
// for a deeper key prefetch).  kTag only separates the instantiation that the
// ThinK value path runs for row constants alone (its own name in profiles).
template <bool kPass2, int kW, int kT, int kCB, int kPF, bool kPreQ, int kTag>
__global__ __launch_bounds__(kW * kWave, 1) void score_pass_seg(ScoreParams p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int kThreads = kW * kWave;
  constexpr int kKeysPerWave = 32 * kT, kKeysPerUnit = kKeysPerWave * kW, kFoldBlocks = 4;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hb = lane >> 5, col = lane & 31;
  const int rows_alloc = p.chunk_rows;   // >= R: one chunk
  const int nb = (p.R + 31) / 32;
  float* rcs = reinterpret_cast<float*>(lds + (size_t)rows_alloc * kRowPitch);
  float2* fold = reinterpret_cast<float2*>(lds + (size_t)rows_alloc * kRowPitch);

  const float inv_w = 1.0f / (float)p.w;
  auto split_row = [&](int r, int& hh, int& ii) {
    hh = (int)((float)r * inv_w);
    ii = r - hh * p.w;
    if (ii < 0) { --hh; ii += p.w; }
    if (ii >= p.w) { ++hh; ii -= p.w; }
  };
  const int heads = p.L * p.Hkv;
  const int total = heads * p.nblk;
  // the 8-wave pass 2 numbers its workgroups like the query-stationary pass 1
  const int nwg = (int)gridDim.x, bid = kW == 8 ? xcd_major_block(nwg) : (int)blockIdx.x;
  const int per = total / nwg, extra = total % nwg;
  const int u_first = bid * per + min(bid, extra);
  const int n_units = per + (bid < extra ? 1 : 0);
  // pass 2 walks its range backwards: its first keys are the ones pass 1 read last
  auto unit_at = [&](int it) { return kPass2 ? u_first + n_units - 1 - it : u_first + it; };

  auto load_tiles = [&](int u, int t0, auto n_c, bf16x8 (*dst)[8]) {
    constexpr int kN = decltype(n_c)::value;
    const int head = u / p.nblk, blk = u - head * p.nblk;
    const int layer = head / p.Hkv, g = head - layer * p.Hkv;
    const uint16_t* kb = p.k + layer * p.k_ls + g * p.k_hs;
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int j = min(blk * kKeysPerUnit + wave * kKeysPerWave + (t0 + i) * 32 + col, p.n - 1);   // clamp; masked
      const bf16x8* row = reinterpret_cast<const bf16x8*>(kb + (int64_t)j * kD);
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) dst[i][s2] = row[2 * s2 + hb];
    }
  };
  bf16x8 kf[kT][8];
  bf16x8 kn[kPF > 0 ? kPF : 1][8];
  bf16x8 qf[8];
  auto read_q = [&](int qb) {
    const char* qsb = lds + (qb * 32 + col) * kRowPitch + hb * 16;
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) qf[s2] = *reinterpret_cast<const bf16x8*>(qsb + 32 * s2);
  };
  auto mfma_block = [&](f32x16 (&acc)[kT]) {
#pragma unroll
    for (int t = 0; t < kT; ++t) acc[t] = f32x16{};
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
#pragma unroll
      for (int t = 0; t < kT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t][s2], qf[s2], acc[t], 0, 0, 0);
  };

  // stage the head's rows (zero rows past R) and, in pass 2, its row constants
  auto stage = [&](int head) {
    const int layer = head / p.Hkv, g = head - layer * p.Hkv;
    const uint16_t* qg = p.q + layer * p.q_ls + (int64_t)g * p.G * p.q_hs;
    const int nrows = nb * 32, tot = nrows * 16;
    for (int base = 0; base < tot; base += 8 * kThreads) {
      u32x4 v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = base + e * kThreads + tid;
        const int r = min(i >> 4, p.R - 1);
        int hh, ii;
        split_row(r, hh, ii);
        v[e] = *reinterpret_cast<const u32x4*>(qg + hh * p.q_hs + (int64_t)ii * kD + (i & 15) * 8);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = base + e * kThreads + tid;
        if (i < tot) *reinterpret_cast<u32x4*>(lds + (i >> 4) * kRowPitch + (i & 15) * 16) =
            (i >> 4) < p.R ? v[e] : u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (kPass2) {
      const int64_t head_row0 = (int64_t)head * p.R;
      if (!p.fuse_rowc) {
        for (int i = tid; i < nrows; i += kThreads) rcs[i] = i < p.R ? p.rowc[head_row0 + i] : INFINITY;
      } else {
        // rowc = m + log2(sum_s l_s 2^(m_s - m)) over the head's segments, one
        // thread per row, kFuseRowcUnits segment loads in flight per step, the
        // steps folded in order
        const int nseg = head_segments(head, p.nblk, total, p.seg_grid);
        for (int i = tid; i < nrows; i += kThreads) {
          const int r = min(i, p.R - 1);
          const float2* pp = p.part + head_row0 * p.nblk + r;
          float m = -INFINITY, l = 0.f;
          for (int b0 = 0; b0 < nseg; b0 += kFuseRowcUnits) {
            float2 a[kFuseRowcUnits];
#pragma unroll
            for (int e = 0; e < kFuseRowcUnits; ++e) a[e] = pp[(int64_t)min(b0 + e, nseg - 1) * p.R];
            float mn = m;
#pragma unroll
            for (int e = 0; e < kFuseRowcUnits; ++e) mn = fmaxf(mn, b0 + e < nseg ? a[e].x : -INFINITY);
            const float ms = (mn == -INFINITY) ? 0.f : mn;
            float acc = l * fast_exp2(m - ms);
#pragma unroll
            for (int e = 0; e < kFuseRowcUnits; ++e) acc += b0 + e < nseg ? a[e].y * fast_exp2(a[e].x - ms) : 0.f;
            m = mn;
            l = acc;
          }
          rcs[i] = (i < p.R && l > 0.f) ? m + log2f(l) : INFINITY;
        }
      }
    }
  };

  // per query block (reference, sum) of the lane's row (the blocks are
  // unrolled, so every index is a constant)
  using stvec = float __attribute__((ext_vector_type(kCB)));
  stvec stm, stl;
  f32x16 colacc[kT];
  int cur = -1;
  float cc = 0.f;
  // pass 1: fold each lane's per-block (max, sum) over the 2*kW half-waves of
  // every row, kFoldBlocks query blocks at a time through LDS, in a fixed order
  auto flush = [&](int head) {
    const int seg = bid - unit_owner(head * p.nblk, total, nwg);
    const int64_t base = ((int64_t)head * p.nblk + seg) * p.R;
#pragma unroll
    for (int f0 = 0; f0 < kCB; f0 += kFoldBlocks) {
      if (f0 < nb) {
#pragma unroll
        for (int qq = 0; qq < kFoldBlocks; ++qq) fold[((wave * kFoldBlocks + qq) * 32 + col) * 2 + hb] = float2{stm[f0 + qq], stl[f0 + qq]};
        __syncthreads();
        {
          constexpr int kTPR = kThreads / (kFoldBlocks * 32);
          constexpr int kPer = 2 * kW / kTPR;
          const int i = tid / kTPR, j = tid % kTPR;
          const int r = f0 * 32 + i;
          float2 e[kPer];
#pragma unroll
          for (int k = 0; k < kPer; ++k) {
            const int v = j * kPer + k;
            e[k] = fold[(v >> 1) * kFoldBlocks * 64 + i * 2 + (v & 1)];
          }
          float m = e[0].x;
#pragma unroll
          for (int k = 1; k < kPer; ++k) m = fmaxf(m, e[k].x);
          const float ms = (m == -INFINITY) ? 0.f : m;
          float l = 0.f;
#pragma unroll
          for (int k = 0; k < kPer; ++k) l += e[k].y * fast_exp2(e[k].x - ms);
#pragma unroll
          for (int o = 1; o < kTPR; o <<= 1) {
            const float mo = __shfl_xor(m, o), lo = __shfl_xor(l, o);
            const float m2 = fmaxf(m, mo);
            const float m2s = (m2 == -INFINITY) ? 0.f : m2;
            l = l * fast_exp2(m - m2s) + lo * fast_exp2(mo - m2s);
            m = m2;
          }
          if (j == 0 && r < p.R) p.part[base + r] = float2{m, l};
        }
        __syncthreads();
      }
    }
  };
  // pass 1, one block: add the lane's exponentials against the running
  // reference st.x (log2 units); take the block maximum only where no
  // reference exists yet or the block would overflow it
  auto stats = [&](bool clean, f32x16 (&acc)[kT], int key0, int r, float2& s) {
    if (!clean) {
      // wave-uniform branch: keys past the prefix and rows past R take -inf.
      // Element (t, e) is key key0 + 4hb + off(t, e) with a constant offset;
      // it is masked when off >= lim (every element of a row past R)
      const int lim = r < p.R ? p.n - key0 - 4 * hb : INT_MIN;
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * t + 8 * (e >> 2) + (e & 3) >= lim) acc[t][e] = -INFINITY;
    }
    const float mref = s.x;
    const float mrs = (mref == -INFINITY) ? 0.f : mref;
    // every lane sums against its own reference, also while other lanes of
    // the wave have none (rows past R never get one); a lane without one, or
    // whose sum leaves fp32 range, redoes the block against its maximum
    float l = 0.f;
#pragma unroll
    for (int t = 0; t < kT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) l += fast_exp2(fmaf(acc[t][e], cc, -mrs));
    const bool redo = mref == -INFINITY || !(l < 0x1p64f);
    if (__ballot(redo)) {
      if (redo) {
        float mx = acc[0][0];
#pragma unroll
        for (int t = 0; t < kT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[t][e]);
        const float m2 = fmaxf(mref, mx * cc);
        const float m2s = (m2 == -INFINITY) ? 0.f : m2;
        l = 0.f;
#pragma unroll
        for (int t = 0; t < kT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) l += fast_exp2(fmaf(acc[t][e], cc, -m2s));
        if (mref != -INFINITY) s.y *= fast_exp2(mrs - m2s);   // (s.y = 0 while no reference exists)
        s.x = m2;
      }
    }
    s.y += l;
  };

  if (n_units > 0) load_tiles(unit_at(0), 0, std::integral_constant<int, kT>{}, kf);
#pragma unroll 1
  for (int it = 0; it < n_units; ++it) {
    const int u = unit_at(it);
    const int head = u / p.nblk, blk = u - head * p.nblk;
    const int layer = head / p.Hkv;
    if (head != cur) {
      if (!kPass2 && cur >= 0) flush(cur);
      __syncthreads();   // every wave is done with the previous rows
      stage(head);
      __syncthreads();
      cur = head;
      const float alpha = p.layer_scales ? p.layer_scales[layer] : p.scale;
      cc = alpha * kLog2e;
      if (!kPass2) {
#pragma unroll
        for (int qb = 0; qb < kCB; ++qb) {
          stm[qb] = -INFINITY;
          stl[qb] = 0.f;
        }
      }
    }
    if (it != 0 && kPF > 0) {
#pragma unroll
      for (int t = 0; t < kPF; ++t)
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) kf[t][s2] = kn[t][s2];
    }
    // this unit's tiles are in (tiles [kPF, kT) were loaded into kf during the
    // previous unit's last block); the next unit's first kPF tiles go in
    // flight (unconditionally -- the last unit reloads itself -- so nothing
    // below waits on them)
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if (kPF > 0)
      load_tiles(unit_at(min(it + 1, n_units - 1)), 0, std::integral_constant<int, (kPF > 0 ? kPF : 1)>{}, kn);
    // once the last block's MFMAs have read this unit's tiles, tiles [kPF, kT)
    // of the next unit are loaded into their registers (the next unit's wait
    // above covers them)
    auto tail_prefetch = [&] {
      if (it + 1 < n_units) load_tiles(unit_at(it + 1), kPF, std::integral_constant<int, kT - kPF>{}, kf + kPF);
    };
    const int key0 = blk * kKeysPerUnit + wave * kKeysPerWave;
    const bool wave_full = key0 + kKeysPerWave <= p.n;
    if (kPreQ) read_q(0);
    if (!kPass2) {
      const bool clean = wave_full && nb * 32 == p.R;
      auto block1 = [&](int qb, bool last) {
        f32x16 acc[kT];
        if (!kPreQ) read_q(qb);
        mfma_block(acc);
        if (last)
          tail_prefetch();
        else if (kPreQ)
          read_q(qb + 1);
        float2 sq = float2{stm[qb], stl[qb]};
        stats(clean, acc, key0, qb * 32 + col, sq);
        stm[qb] = sq.x;
        stl[qb] = sq.y;
      };
      static_for<0, kCB>([&](auto qb_c) {
        constexpr int qb = decltype(qb_c)::value;
        if (qb < nb) block1(qb, qb == nb - 1);
      });
    } else {
#pragma unroll
      for (int t = 0; t < kT; ++t) colacc[t] = f32x16{};
      // the last block is peeled: its vector phase issues the tail prefetch,
      // and a load issued inside the loop would make the compiler wait for
      // the outstanding prefetches before the loop's MFMAs
      auto block2 = [&](int qb, bool last) {
        f32x16 acc[kT];
        if (!kPreQ) read_q(qb);
        mfma_block(acc);
        const float rc = rcs[qb * 32 + col];   // +inf for rows past R: adds 0
        if (last)
          tail_prefetch();
        else if (kPreQ)
          read_q(qb + 1);
#pragma unroll
        for (int t = 0; t < kT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) colacc[t][e] += fast_exp2(fmaf(acc[t][e], cc, -rc));
      };
#pragma unroll 1
      for (int qb = 0; qb < nb - 1; ++qb) block2(qb, false);
      block2(nb - 1, true);
      // sum each key column over the 32 query lanes of its half-wave (lane
      // col receives the total of value col & 15; the first row stores it)
      float* out = p.imp + (int64_t)head * p.n;
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        const float mine = half_wave_sum16_dpp(colacc[t], col);
        if (col < 16) {
          const int e = col;
          const int key = key0 + 32 * t + 8 * (e >> 2) + 4 * hb + (e & 3);
          if (key < p.n) out[key] = mine * p.inv_w;
        }
      }
    }
  }
  if (!kPass2 && cur >= 0) flush(cur);
}

// Pass 1, query-stationary form (8 waves, R <= 512): wave w keeps query rows
// [64w, 64w + 64) of the head in registers as two B-operand blocks, so each
// lane carries the statistics of just two rows, in fixed registers, for the
// whole segment.  The keys stream through LDS: half-units of 256 keys (8
// tiles of 32) are copied by global_load_lds_dwordx4 into a two-buffer ring,
// one buffer filling while the other is read, one barrier per half-unit.  A
// key row's 16-byte chunk c lands at position c ^ (row & 15) of its 256-byte
// LDS row, so the A-operand reads of 8 or 16 consecutive keys hit distinct
// banks.  Per tile a wave runs 16 MFMAs (2 row blocks x 8 depth steps).  At
// the end of a head's segment each row's two half-wave (reference, sum) pairs
// are merged with one lane exchange; no cross-wave fold, so the segment's
// partials are written without LDS or barriers.
constexpr int kQsHalfKeys = 256;                           // keys per ring buffer
constexpr int kQsTiles = kQsHalfKeys / 32;                 // 32-key tiles per buffer
constexpr int kQsBufBytes = kQsHalfKeys * kD * 2;          // 64 KB
constexpr int kQsLds = 2 * kQsBufBytes;

template <int kTag>
__global__ __launch_bounds__(512, 1) void score_pass1_qs(ScoreParams p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int kThreads = 512, kKeysPerUnit = 512;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hb = lane >> 5, col = lane & 31;
  const int heads = p.L * p.Hkv, total = heads * p.nblk;
  const int nwg = (int)gridDim.x, bid = xcd_major_block(nwg);
  const int per = total / nwg, extra = total % nwg;
  const int u_first = bid * per + min(bid, extra);
  const int n_units = per + (bid < extra ? 1 : 0);
  if (n_units <= 0) return;   // uniform over the workgroup: no barrier is skipped by part of it
  const int n_half = 2 * n_units;
  const float inv_w = 1.0f / (float)p.w;
  auto split_row = [&](int r, int& hh, int& ii) {
    hh = (int)((float)r * inv_w);
    ii = r - hh * p.w;
    if (ii < 0) { --hh; ii += p.w; }
    if (ii >= p.w) { ++hh; ii -= p.w; }
  };

  // copy half-unit h (keys key0 .. key0 + 255 of its head) into ring buffer
  // h & 1: copy instruction i of wave w moves the KB holding keys
  // 32i + 4w .. 32i + 4w + 3 (tile i), so a lane's key row differs between
  // its instructions by 32 and its chunk (lane & 15) ^ (row & 15) not at all;
  // the key base and LDS slot are uniform
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int cp_row = 4 * wave_u + (lane >> 4);                 // + 32 i
  const int cp_off = (cp_row * kD + (((lane & 15) ^ (cp_row & 15)) * 8)) * 2;   // bytes
  auto issue_copy = [&](int h) {
    const int u = u_first + (h >> 1);
    const int head = u / p.nblk, blk = u - head * p.nblk;
    const int layer = head / p.Hkv, g = head - layer * p.Hkv;
    const int key0 = blk * kKeysPerUnit + (h & 1) * kQsHalfKeys;
    const uint16_t* kb = p.k + layer * p.k_ls + g * p.k_hs + (int64_t)key0 * kD;
    // a buffer over the half-unit's keys inside the prefix: rows past it
    // read as zeros (the statistics mask them)
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)kb, 0, min(kQsHalfKeys, p.n - key0) * kD * 2, 0x00020000);
    char* buf = lds + (h & 1) * kQsBufBytes + wave_u * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(buf + i * 8192), 16,
                                               cp_off + i * 32 * kD * 2, 0, 0, 0);
  };

  // A-operand byte offsets within a tile: lane (col, hb) reads logical chunk
  // 2 s2 + hb of key row col, stored at position (2 s2 + hb) ^ (col & 15)
  int aoff[8];
#pragma unroll
  for (int s2 = 0; s2 < 8; ++s2) aoff[s2] = col * 256 + (((2 * s2) | hb) ^ (col & 15)) * 16;

  bf16x8 qf[2][8];
  float stm[2], stl[2];
  int cur = -1;
  float cc = 0.f;
  const int row0 = wave * 64;   // this wave's first query row

  auto load_q = [&](int head) {
    const int layer = head / p.Hkv, g = head - layer * p.Hkv;
    const uint16_t* qg = p.q + layer * p.q_ls + (int64_t)g * p.G * p.q_hs;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int r = min(row0 + 32 * b + col, p.R - 1);
      int hh, ii;
      split_row(r, hh, ii);
      const bf16x8* src = reinterpret_cast<const bf16x8*>(qg + hh * p.q_hs + (int64_t)ii * kD) + hb;
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) qf[b][s2] = src[2 * s2];
    }
  };
  // merge the two half-waves' (reference, sum) of each row and write the
  // segment's partial for rows < R
  auto flush = [&](int head) {
    const int seg = bid - unit_owner(head * p.nblk, total, nwg);
    const int64_t base = ((int64_t)head * p.nblk + seg) * p.R;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float m = stm[b], l = stl[b];
      const float mo = __shfl_xor(m, 32), lo = __shfl_xor(l, 32);
      const float m2 = fmaxf(m, mo);
      const float m2s = (m2 == -INFINITY) ? 0.f : m2;
      const float l2 = (m == -INFINITY ? 0.f : l * fast_exp2(m - m2s)) + (mo == -INFINITY ? 0.f : lo * fast_exp2(mo - m2s));
      const int r = row0 + 32 * b + col;
      if (hb == 0 && r < p.R) p.part[base + r] = float2{m2, l2};
    }
  };
  // one tile's statistics for both row blocks, against each lane's running
  // reference (log2 units).  stats_sum is branch-free: every lane sums
  // against its own references, also while other lanes of the wave have none
  // (rows past R never get one); stats_fix lets a block take its own maximum
  // where the lane has no reference yet or the sum left fp32 range
  auto stats_sum = [&](const f32x16 (&acc)[2], float (&l)[2], bool& redo) {
    redo = false;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float mrs = (stm[b] == -INFINITY) ? 0.f : stm[b];
      float s0 = fast_exp2(fmaf(acc[b][0], cc, -mrs)), s1 = fast_exp2(fmaf(acc[b][1], cc, -mrs));
#pragma unroll
      for (int e = 2; e < 16; e += 2) {
        s0 += fast_exp2(fmaf(acc[b][e], cc, -mrs));
        s1 += fast_exp2(fmaf(acc[b][e + 1], cc, -mrs));
      }
      l[b] = s0 + s1;
      redo = redo || stm[b] == -INFINITY || !(l[b] < 0x1p64f);
    }
  };
  auto stats_fix = [&](const f32x16 (&acc)[2], float (&l)[2], bool redo) {
    if (__ballot(redo)) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (stm[b] == -INFINITY || !(l[b] < 0x1p64f)) {
          float mx = acc[b][0];
#pragma unroll
          for (int e = 1; e < 16; ++e) mx = fmaxf(mx, acc[b][e]);
          const float mref = stm[b];
          const float m2 = fmaxf(mref, mx * cc);
          const float m2s = (m2 == -INFINITY) ? 0.f : m2;
          float s0 = fast_exp2(fmaf(acc[b][0], cc, -m2s)), s1 = fast_exp2(fmaf(acc[b][1], cc, -m2s));
#pragma unroll
          for (int e = 2; e < 16; e += 2) {
            s0 += fast_exp2(fmaf(acc[b][e], cc, -m2s));
            s1 += fast_exp2(fmaf(acc[b][e + 1], cc, -m2s));
          }
          l[b] = s0 + s1;
          if (mref != -INFINITY) stl[b] *= fast_exp2(mref - m2s);   // (no reference: the sum is 0)
          stm[b] = m2;
        }
      }
    }
    stl[0] += l[0];
    stl[1] += l[1];
  };
  auto stats = [&](f32x16 (&acc)[2]) {
    float l[2];
    bool redo;
    stats_sum(acc, l, redo);
    stats_fix(acc, l, redo);
  };
  auto load_tile = [&](bf16x8 (&kf)[8], const char* tp) {
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) kf[s2] = *reinterpret_cast<const bf16x8*>(tp + aoff[s2]);
  };
  auto mfma_tile = [&](f32x16 (&acc)[2], const bf16x8 (&kf)[8]) {
    acc[0] = f32x16{};
    acc[1] = f32x16{};
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s2], qf[b][s2], acc[b], 0, 0, 0);
  };

  // Half-units whose 256 keys are all in the prefix run as a software
  // pipeline: each step issues tile t's MFMAs (into acc2[t & 1]), the LDS
  // reads of tile t + 1 and the statistics of tile t - 1, with no branch
  // between them but the rare redo, so the MFMAs run under the vector work.
  // The last tile's statistics are pending into the next half-unit (pend).
  // Rows past R need no mask: their query rows are copies of row R - 1 and
  // flush skips them.
  f32x16 acc2[2][2];
  bf16x8 kf2[2][8];
  bool pend = false;
  auto drain = [&] {
    if (pend) stats(acc2[1]);
    pend = false;
  };
  auto step = [&](auto t_c, auto pend_c, const char* buf) {
    constexpr int t = decltype(t_c)::value, c = t & 1, o = c ^ 1;
    constexpr bool kPend = decltype(pend_c)::value;
    if (t + 1 < kQsTiles) load_tile(kf2[o], buf + (t + 1) * 32 * 256);
    mfma_tile(acc2[c], kf2[c]);
    if (kPend) stats(acc2[o]);
  };

  auto set_head = [&](int head) {
    load_q(head);
    cur = head;
    const int layer = head / p.Hkv;
    cc = (p.layer_scales ? p.layer_scales[layer] : p.scale) * kLog2e;
    stm[0] = stm[1] = -INFINITY;
    stl[0] = stl[1] = 0.f;
  };
  set_head(u_first / p.nblk);
  issue_copy(0);
#pragma unroll 1
  for (int h = 0; h < n_half; ++h) {
    const int u = u_first + (h >> 1);
    const int head = u / p.nblk, blk = u - head * p.nblk;
    if (head != cur) {
      drain();
      flush(cur);
      set_head(head);
    }
    // this wave's part of half-unit h (and the head's rows) have landed; the
    // barrier makes every wave's part visible and ends every wave's reads of
    // the other buffer, which the next copy then refills
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    if (h + 1 < n_half) issue_copy(h + 1);
    const char* buf = lds + (h & 1) * kQsBufBytes;
    const int key_h = blk * kKeysPerUnit + (h & 1) * kQsHalfKeys;
    if (key_h + kQsHalfKeys <= p.n) {
      load_tile(kf2[0], buf);
      if (pend)
        step(std::integral_constant<int, 0>{}, std::true_type{}, buf);
      else
        step(std::integral_constant<int, 0>{}, std::false_type{}, buf);
      static_for<1, kQsTiles>([&](auto t_c) { step(t_c, std::true_type{}, buf); });
      pend = true;
    } else {
      // the head's last, part-filled half-unit, tile by tile: keys past the
      // prefix take -inf
      drain();
      static_for<0, kQsTiles>([&](auto t_c) {
        constexpr int t = decltype(t_c)::value;
        const int key_t = key_h + 32 * t;
        if (key_t < p.n) {
          bf16x8 kfr[8];
          load_tile(kfr, buf + t * 32 * 256);
          f32x16 acc[2];
          mfma_tile(acc, kfr);
          if (key_t + 32 > p.n) {
            const int lim = p.n - key_t - 4 * hb;   // element (e) is key key_t + 4hb + 8(e/4) + e%4
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
              for (int e = 0; e < 16; ++e)
                if (8 * (e >> 2) + (e & 3) >= lim) acc[b][e] = -INFINITY;
          }
          stats(acc);
        }
      });
    }
  }
  drain();
  flush(cur);
}

// Fold the per-unit partials of each query row into
// rowc = m + log2(sum_b l_b * 2^(m_b - m)).  A workgroup takes kRows
// consecutive rows of one head; its 256/kRows thread groups each fold every
// (256/kRows)-th unit online (coalesced reads along the rows), and the group
// results are folded in a fixed order, so the result is bit-reproducible.
// Rows with many units use 8 rows x 32 groups, the rest 32 rows x 8 groups.
// kTag only separates the ThinK value path's row-constant fold (its own name
// in profiles).
template <int kRows, int kTag = 0>
__global__ __launch_bounds__(256) void score_combine(ScoreParams p, int heads) {
  constexpr int kGroups = 256 / kRows;
  __shared__ float2 sg[kGroups][kRows];
  const int rr = threadIdx.x % kRows, q = threadIdx.x / kRows;
  const int tiles = (p.R + kRows - 1) / kRows;
  const int head = blockIdx.x / tiles, r = (blockIdx.x - head * tiles) * kRows + rr;
  float m = -INFINITY, l = 0.f;
  if (head < heads && r < p.R) {
    const float2* pp = p.part + (int64_t)head * p.nblk * p.R + r;
    // causal: only the units this row's position can see were scored for it;
    // segment mode: one partial per workgroup segment of the head
    const int nb_row = p.seg_grid ? head_segments(head, p.nblk, heads * p.nblk, p.seg_grid)
                       : p.causal_unit ? min(p.nblk, (p.S - p.w + r % p.w) / p.causal_unit + 1) : p.nblk;
#pragma unroll 4
    for (int b = q; b < nb_row; b += kGroups) {
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
    for (int i = 0; i < kGroups; ++i) mm = fmaxf(mm, sg[i][rr].x);
    const float ms = (mm == -INFINITY) ? 0.f : mm;
    float ll = 0.f;
#pragma unroll
    for (int i = 0; i < kGroups; ++i) ll += sg[i][rr].y * fast_exp2(sg[i][rr].x - ms);
    p.rowc[(int64_t)head * p.R + r] = (ll > 0.f) ? mm + log2f(ll) : INFINITY;
  }
}

struct Plan {
  int n, G, R, nblk, chunk_rows;
  Shape shape;
  size_t part_bytes, rowc_bytes, total;
};

kvc_status plan(const kvc_score_args* a, Plan* pl, bool causal = false) {
  if (!a) return KVC_E_ARG;
  if (a->L < 1 || a->H < 1 || a->Hkv < 1 || a->w < 1 || a->S < 2 || a->D < 1) return KVC_E_ARG;
  if (a->H % a->Hkv) return KVC_E_SHAPE;
  if (causal ? (a->w > a->S || (a->w & 31)) : a->w >= a->S) return KVC_E_SHAPE;
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
  pl->n = causal ? a->S : a->S - a->w;
  // units of work (at least 128 keys each) are counted in 32-bit integers
  if ((int64_t)a->L * a->Hkv * ((pl->n + 127) / 128) > INT32_MAX) return KVC_E_SHAPE;
  pl->G = (int)G;
  pl->R = (int)(G * a->w);
  pl->shape = score_shape(pl->R, a->gumbel != 0);
  const int unit = 32 * pl->shape.kw * pl->shape.kt;
  pl->nblk = (pl->n + unit - 1) / unit;
  pl->chunk_rows = score_chunk_rows(pl->R, pl->shape);
  const size_t rows = (size_t)a->L * a->Hkv * pl->R;
  pl->part_bytes = align_up(rows * pl->nblk * sizeof(float2), 256);
  pl->rowc_bytes = align_up(rows * sizeof(float), 256);
  pl->total = pl->part_bytes + pl->rowc_bytes;
  return KVC_OK;
}

// Persistent grid for one scoring pass: as many workgroups as fit on the
// device at once (occupancy x CUs), at most one per unit.
template <typename K>
kvc_status score_grid(K kernel, int threads, size_t lds, int units, int* grid) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess || per_cu < 1)
    return KVC_E_DEVICE;
  const int cus = device_cu_count();
  if (cus < 1) return KVC_E_DEVICE;
  *grid = units < per_cu * cus ? units : per_cu * cus;
  return KVC_OK;
}

// Pass 1, combine and (unless only the row constants are wanted) pass 2 on one
// stream.
// Prefetch depth: every tile where the registers allow it (the 8-wave pass 2)
// and for the 4-wave shape when a workgroup walks many units of >= 4 query
// blocks (R >= 128; there it beats a second workgroup per CU, which a deeper
// prefetch costs); one tile otherwise; none for the Keyformer shape (3 waves
// per SIMD, no registers to spare) nor for the causal 8-wave pass 1 (its
// masking path leaves no registers for it).
template <bool kGumbel, bool kCausal, int kW, int kT, int kCB, int kPF1, int kPF2>
kvc_status launch_score(ScoreParams p, const Plan& pl, hipStream_t s, bool pass2 = true) {
  p.causal_unit = kCausal ? 32 * kW * kT : 0;
  constexpr int kThreads = kW * kWave;
  const int units = p.L * p.Hkv * pl.nblk;
  const int heads = p.L * p.Hkv;
  const bool wide = pl.nblk >= 128;   // many units per row: more groups per row
  const int comb_rows = wide ? 8 : 32;
  const dim3 comb_grid(heads * ((pl.R + comb_rows - 1) / comb_rows));
  auto kc = wide ? score_combine<8> : score_combine<32>;
  const size_t lds1 = score_lds_bytes(pl.chunk_rows, kW, false), lds2 = score_lds_bytes(pl.chunk_rows, kW, true);
  auto k1 = score_pass<false, kGumbel, kCausal, kW, kT, kCB, kPF1>;
  auto k2 = score_pass<true, kGumbel, kCausal, kW, kT, kCB, kPF2>;
  int g1 = 0, g2 = 0;
  kvc_status st = score_grid(k1, kThreads, lds1, units, &g1);
  if (st != KVC_OK) return st;
  st = score_grid(k2, kThreads, lds2, units, &g2);
  if (st != KVC_OK) return st;
  if (!pass2) {   // row constants only (ThinK value scores): named apart from the scoring pass
    KVC_LAUNCH_SHM("think_rowc_pass1", k1, dim3(g1), dim3(kThreads), lds1, s, p);
    KVC_LAUNCH("think_rowc_combine", wide ? (score_combine<8, 1>) : (score_combine<32, 1>), comb_grid, dim3(256),
               s, p, heads);
    return KVC_OK;
  }
  KVC_LAUNCH_SHM(kCausal ? (kGumbel ? "score_causal_pass1_gumbel" : "score_causal_pass1")
                         : (kGumbel ? "score_pass1_gumbel" : "score_pass1"),
                 k1, dim3(g1), dim3(kThreads), lds1, s, p);
  if (!p.fuse_rowc) KVC_LAUNCH("score_combine", kc, comb_grid, dim3(256), s, p, heads);
  KVC_LAUNCH_SHM(kCausal ? (kGumbel ? "score_causal_pass2_gumbel" : "score_causal_pass2")
                         : (kGumbel ? "score_pass2_gumbel" : "score_pass2"),
                 k2, dim3(g2), dim3(kThreads), lds2, s, p);
  return KVC_OK;
}

// Window scoring whose G*w rows fit one staged chunk: the segment passes.
// Pass 2 folds the segment partials itself while staging when every head has
// at most kFuseRowcUnits segments; otherwise the combine kernel runs.
// pass2 == false: pass 1 and the row constants only (the ThinK value path),
// from an instantiation of its own (kTag 1).
template <int kW, int kT, int kCB, int kPF1, bool kPreQ1, int kPF2, bool kPreQ2>
kvc_status launch_score_seg(ScoreParams p, const Plan& pl, hipStream_t s, bool pass2 = true) {
  constexpr int kThreads = kW * kWave;
  const int units = p.L * p.Hkv * pl.nblk;
  const int heads = p.L * p.Hkv;
  // the 8-wave shape's pass 1 is the query-stationary kernel (same units,
  // segments and partials; kPF1 and kPreQ1 do not apply to it)
  constexpr bool kQs = kW == 8;
  const size_t lds1 = kQs ? (size_t)kQsLds : score_lds_bytes(pl.chunk_rows, kW, false);
  const size_t lds2 = score_lds_bytes(pl.chunk_rows, kW, true);
  auto pick_pass1 = [pass2]() {
    if constexpr (kQs)
      return pass2 ? score_pass1_qs<0> : score_pass1_qs<1>;
    else
      return pass2 ? score_pass_seg<false, kW, kT, kCB, kPF1, kPreQ1, 0> : score_pass_seg<false, kW, kT, kCB, kPF1, kPreQ1, 1>;
  };
  auto k1 = pick_pass1();
  auto k2 = score_pass_seg<true, kW, kT, kCB, kPF2, kPreQ2, 0>;
  int g1 = 0, g2 = 0;
  kvc_status st = score_grid(k1, kThreads, lds1, units, &g1);
  if (st != KVC_OK) return st;
  st = score_grid(k2, kThreads, lds2, units, &g2);
  if (st != KVC_OK) return st;
  p.causal_unit = 0;
  p.seg_grid = g1;
  int nseg_max = 0;
  for (int h = 0; h < heads; ++h) nseg_max = max(nseg_max, head_segments(h, pl.nblk, units, g1));
  p.fuse_rowc = (pass2 && nseg_max <= kFuseRowcSegments) ? 1 : 0;
  const dim3 comb_grid(heads * ((pl.R + 31) / 32));
  if (!pass2) {
    KVC_LAUNCH_SHM("think_rowc_pass1", k1, dim3(g1), dim3(kThreads), lds1, s, p);
    KVC_LAUNCH("think_rowc_combine", (score_combine<32, 1>), comb_grid, dim3(256), s, p, heads);
    return KVC_OK;
  }
  KVC_LAUNCH_SHM("score_pass1", k1, dim3(g1), dim3(kThreads), lds1, s, p);
  if (!p.fuse_rowc) KVC_LAUNCH("score_combine", score_combine<32>, comb_grid, dim3(256), s, p, heads);
  KVC_LAUNCH_SHM("score_pass2", k2, dim3(g2), dim3(kThreads), lds2, s, p);
  return KVC_OK;
}

}  // namespace
}  // namespace kvc

extern "C" size_t kvc_score_workspace_size(const kvc_score_args* args) {
  kvc::Plan pl;
  return kvc::plan(args, &pl) == KVC_OK ? pl.total : 0;
}

namespace kvc {
namespace {

kvc_status score_entry(const kvc_score_args* a, const void* q_obs, const void* k, float* importance, void* ws,
                       size_t ws_bytes, void* stream, bool causal) {
  Plan pl;
  kvc_status st = plan(a, &pl, causal);
  if (st != KVC_OK) return st;
  if (!q_obs || !k || !importance) return KVC_E_ARG;
  if (!aligned16(q_obs) || !aligned16(k) || (reinterpret_cast<uintptr_t>(importance) & 3)) return KVC_E_ARG;
  if (!ws || ws_bytes < pl.total || !aligned16(ws)) return KVC_E_WORKSPACE;

  ScoreParams p{};
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
  p.chunk_rows = pl.chunk_rows;
  // A workgroup stages a head's rows once when they fit one chunk; with few
  // units per row, folding them there is cheaper than a combine launch.
  p.fuse_rowc = (!causal && !a->gumbel && pl.R <= pl.chunk_rows && pl.nblk <= kFuseRowcUnits) ? 1 : 0;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (causal) {
    if (a->gumbel) return launch_score<true, true, 4, 1, 4, 0, 0>(p, pl, s);
    if (pl.shape.kw == 8) return launch_score<false, true, 8, 2, 16, 0, 1>(p, pl, s);
    return launch_score<false, true, 4, 2, 8, 1, 1>(p, pl, s);
  }
  if (a->gumbel) return launch_score<true, false, 4, 1, 4, 0, 0>(p, pl, s);
  if (pl.shape.kw == 8 && pl.R <= pl.chunk_rows) return launch_score_seg<8, 2, 16, 0, true, 1, true>(p, pl, s);
  if (pl.shape.kw == 8) return launch_score<false, false, 8, 2, 16, 1, 2>(p, pl, s);
  return launch_score_seg<4, 2, 8, 1, true, 1, true>(p, pl, s);
}

}  // namespace
}  // namespace kvc

extern "C" kvc_status kvc_score(const kvc_score_args* a, const void* q_obs, const void* k, float* importance,
                                void* ws, size_t ws_bytes, void* stream) {
  return kvc::score_entry(a, q_obs, k, importance, ws, ws_bytes, stream, false);
}

extern "C" size_t kvc_score_causal_workspace_size(const kvc_score_args* args) {
  kvc::Plan pl;
  return kvc::plan(args, &pl, true) == KVC_OK ? pl.total : 0;
}

extern "C" kvc_status kvc_score_causal(const kvc_score_args* a, const void* q_obs, const void* k,
                                       float* importance, void* ws, size_t ws_bytes, void* stream) {
  return kvc::score_entry(a, q_obs, k, importance, ws, ws_bytes, stream, true);
}

namespace kvc {

// Row constants of softmax(scale * q k^T) over the first n rows of each KV head
// of k (pass 1 and the combine of the scoring path, no importance): rowc[g*R + r]
// = max + log2(sum) in log2 units, R = G*w rows per KV head.  k's rows past n
// are never read, so k may hold fewer than n + w rows.
static kvc_score_args rowc_args(int Hkv, int G, int w, int n, int64_t q_hs, float scale) {
  kvc_score_args a{};
  a.L = 1;
  a.H = Hkv * G;
  a.Hkv = Hkv;
  a.w = w;
  a.S = n + w;
  a.D = kD;
  a.q_head_stride = q_hs;
  a.k_head_stride = (int64_t)(n + w) * kD;   // validation only: the kernels read rows [0, n)
  a.scale = scale;
  return a;
}

size_t score_rowc_workspace_size(int Hkv, int G, int w, int n, int64_t q_hs) {
  if (n < 1) return 0;
  const kvc_score_args a = rowc_args(Hkv, G, w, n, q_hs, 1.0f);
  Plan pl;
  return plan(&a, &pl) == KVC_OK ? pl.total : 0;
}

kvc_status score_rowc(const uint16_t* q, int64_t q_hs, const uint16_t* k, int64_t k_hs, int Hkv, int G, int w,
                      int n, float scale, void* ws, size_t ws_bytes, const float** rowc, hipStream_t s) {
  const kvc_score_args a = rowc_args(Hkv, G, w, n, q_hs, scale);
  Plan pl;
  kvc_status st = plan(&a, &pl);
  if (st != KVC_OK) return st;
  if (k_hs < (int64_t)n * kD || (k_hs & 7)) return KVC_E_SHAPE;
  if (!ws || ws_bytes < pl.total || !aligned16(ws)) return KVC_E_WORKSPACE;
  ScoreParams p{};
  p.q = q;
  p.k = k;
  p.q_hs = q_hs;
  p.k_hs = k_hs;
  p.imp = nullptr;
  p.part = reinterpret_cast<float2*>(ws);
  p.rowc = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.part_bytes);
  p.scale = scale;
  p.inv_w = 1.0f / (float)w;
  p.L = 1;
  p.Hkv = Hkv;
  p.G = pl.G;
  p.w = w;
  p.S = n + w;
  p.n = pl.n;
  p.R = pl.R;
  p.nblk = pl.nblk;
  p.chunk_rows = pl.chunk_rows;
  *rowc = p.rowc;
  if (pl.shape.kw == 8 && pl.R <= pl.chunk_rows) return launch_score_seg<8, 2, 16, 0, true, 1, true>(p, pl, s, false);
  if (pl.shape.kw == 8) return launch_score<false, false, 8, 2, 16, 1, 2>(p, pl, s, false);
  return launch_score_seg<4, 2, 8, 1, true, 1, true>(p, pl, s, false);
}

}  // namespace kvc

namespace kvc {
namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's copy of `scratch`, looked up once per
// device (with that device current) and kept.
kvc_status score_scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return KVC_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVC_E_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVC_OK;
}

}  // namespace
}  // namespace kvc

extern "C" size_t kvc_score_noalloc_max_workspace(void) { return kScoreScratchBytes; }

extern "C" kvc_status kvc_score_noalloc(const kvc_score_args* a, const void* q_obs, const void* k, float* importance,
                                        void* stream) {
  kvc::Plan pl;
  kvc_status st = kvc::plan(a, &pl);
  if (st != KVC_OK) return st;
  if (pl.total > kScoreScratchBytes) return KVC_E_WORKSPACE;   // checked before any device call
  if (stream) {
    // the scratch is the current device's: the kernels must run there
    hipDevice_t sdev = -1;
    int cur = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess || hipGetDevice(&cur) != hipSuccess)
      return KVC_E_DEVICE;
    if (sdev != cur) return KVC_E_ARG;
  }
  void* ws = nullptr;
  st = kvc::score_scratch_ptr(&ws);
  if (st != KVC_OK) return st;
  return kvc::score_entry(a, q_obs, k, importance, ws, kScoreScratchBytes, stream, false);
}
