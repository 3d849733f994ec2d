// kvc_channel_prune / kvc_channel_prune_query: ThinK key-channel pruning;
// kvc_channel_prune_value: ThinK value-channel pruning.
//
// ThinK page (papercache summary of arXiv 2407.21018): magnitude-based pruning
// keeps, per head, the T = floor((1 - lambda) D) key channels with the largest
// l_p norm over tokens; query-driven pruning keeps the T channels with the
// largest ||Q[-S_obs:, j] K[:, j]^T||_F = ||Q[:, j]|| ||K[:, j]|| (rank-1
// outer product) over the observation-window queries; THINK's implementation
// section: recent keys are not pruned and a binary mask records the pruned
// channels.  The key norms here run over the non-recent kept rows (the rows
// that get pruned); a KV head's query side stacks its G query heads' windows.
// The page's supplementary value-pruning section scores value channel j by
// ||softmax(Q[-S_obs:] K^T / sqrt(D)) V[:, j]||_F; here K and V are the same
// non-recent kept rows U, each stacked query row's softmax is normalised over
// U, and the T top-scoring value channels are kept.
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
//  * value pruning: the scoring path's pass 1 and combine give each stacked
//    query row's softmax constant over U (score_rowc); think_vpartial, grid
//    (key splits of 512, heads, groups of 4 query blocks), stages each 32-key
//    tile of K (padded rows) and of V transposed (keys contiguous per channel)
//    in LDS; each wave keeps its 32 query rows' fragments in registers, takes
//    S = K Q^T with MFMA, P = 2^(S c - rowc) split exactly into bf16 hi + lo,
//    and accumulates O^T += V^T P^T with MFMA, P used straight from the
//    accumulator layout as the B operand (the keys of each 16-key step are
//    permuted the same way in both operands).  think_vnorm folds the splits
//    in a fixed order and sums O^2 over 8 rows per workgroup; think_select and
//    think_gather (on V) finish as for keys.
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
// kTag only separates the value path's instantiation (its own name in
// profiles).
template <int kTag>
__global__ __launch_bounds__(kD * kSelGroups) void think_select(const float* part, int nchunk, const float* qpart,
                                                               int G, int T, int32_t* channels, uint8_t* mask) {
  __shared__ float red[kSelGroups][kD];
  __shared__ float sm[kD];
  __shared__ int ssel[kD];
  const int g = blockIdx.x, d = threadIdx.x & (kD - 1), grp = threadIdx.x / kD;
  const float* pp = part + (int64_t)g * nchunk * kD + d;
  // chunks grp + 8i go to sum i % 4, joined in order.  Up to 16 chunks per
  // group every load is in flight at once (missing chunks add +0, which
  // leaves the non-negative sums unchanged); beyond, four at a time.
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  constexpr int kOnce = 16;
  if (nchunk <= kOnce * kSelGroups) {
    float v[kOnce];
#pragma unroll
    for (int i = 0; i < kOnce; ++i) {
      const int c1 = grp + i * kSelGroups;
      v[i] = pp[(int64_t)min(c1, nchunk - 1) * kD];
      if (c1 >= nchunk) v[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < kOnce; ++i) a[i % 4] += v[i];
  } else {
    int c = grp;
    for (; c + 3 * kSelGroups < nchunk; c += 4 * kSelGroups) {
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] += pp[(int64_t)(c + j * kSelGroups) * kD];
    }
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (c + j * kSelGroups < nchunk) a[j] += pp[(int64_t)(c + j * kSelGroups) * kD];
  }
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
// bf16 each.  kTag as for think_select.
template <bool kPairs, int kTag>
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


// ---- value pruning
constexpr int kVWaves = 4;                // query blocks (waves) per workgroup
constexpr int kVSplit = 512;              // keys per workgroup
constexpr int kKPitch = kD * 2 + 16;      // bytes per staged key row
constexpr int kVNormRows = 8;             // query rows per think_vnorm workgroup


__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {   // finite x
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Query blocks per workgroup for R rows (1, 2 or 4); the other waves take
// further 32-key tiles of each staging step ("key phases").
__host__ __device__ inline int vq_per_wg(int R) {
  const int nqb = (R + 31) / 32;
  return nqb >= 4 ? 4 : (nqb >= 2 ? 2 : 1);
}

__global__ __launch_bounds__(kVWaves * kWave) void think_vpartial(const uint16_t* q, int64_t q_hs, int G, int w,
                                                                 const uint16_t* kc, const uint16_t* vc,
                                                                 int budget, int rows, const float* rowc,
                                                                 float cc, int nsplit, float* opart) {
  // staging: K rows (kVWaves*32 x 272 B) then V^T (128 x (64 kp + 8) B); after
  // the key loop the same bytes hold the key phases' partial O for the fold
  __shared__ __attribute__((aligned(16))) char smem[kVWaves * 32 * kKPitch + kD * (kVWaves * 64 + 8)];
  const int split = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hb = lane >> 5, col = lane & 31;
  const int R = G * w;
  const int qpw = vq_per_wg(R), kp = kVWaves / qpw;
  const int phase = wave / qpw;              // which 32-key tile of a staging step
  const int qb = blockIdx.z * qpw + wave % qpw;
  const int row = qb * 32 + col;             // this lane's query row
  const bool wave_on = qb * 32 < R;
  const int vt_pitch = 64 * kp + 8;          // bytes per staged V^T row (32 kp keys + padding)
  char* ks = smem;
  char* vt = smem + kVWaves * 32 * kKPitch;
  // B operand of S = K Q^T: lane holds Q[row][16 s + 8 hb .. +8]
  bf16x8 qf[8];
  float rc = INFINITY;                       // rows past R: P = 0
  if (row < R) {
    const int hh = row / w, ii = row - hh * w;
    const uint16_t* qr = q + (int64_t)(g * G + hh) * q_hs + (int64_t)ii * kD + 8 * hb;
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qr + 16 * st);
    rc = rowc[(int64_t)g * R + row];
  } else {
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = bf16x8{};
  }
  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  const int key_lo = split * kVSplit;
  const int key_hi = min(key_lo + kVSplit, rows);
  const uint16_t* kb = kc + (int64_t)g * budget * kD;
  const uint16_t* vb = vc + (int64_t)g * budget * kD;
  const int nkeys = 32 * kp;                 // keys per staging step
  // a thread stages 4 consecutive keys of one 8-channel chunk per item (at
  // most two items): 4 K rows as 16-byte writes, and per channel the 4 keys'
  // values as one 8-byte V^T write.  The next step's items are loaded into
  // registers while this step computes.
  constexpr int kItems = (32 * kVWaves * 4) / (kVWaves * kWave);
  u32x4 pk[kItems][4], pv[kItems][4];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int i = tid + it * kVWaves * kWave;
      const int kr0 = (i >> 4) * 4, ch = i & 15;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // clamped address; keys past key_hi are zeroed when staged
        const int kk = min(t0 + kr0 + r, key_hi - 1);
        pk[it][r] = *reinterpret_cast<const u32x4*>(kb + (int64_t)kk * kD + ch * 8);
        pv[it][r] = *reinterpret_cast<const u32x4*>(vb + (int64_t)kk * kD + ch * 8);
      }
    }
  };
  auto put = [&](int t0) {
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int i = tid + it * kVWaves * kWave;
      if (i >= nkeys * 4) continue;
      const int kr0 = (i >> 4) * 4, ch = i & 15;
      uint32_t vwd[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = t0 + kr0 + r < key_hi;
        const u32x4 kv = ok ? pk[it][r] : u32x4{0u, 0u, 0u, 0u};
        const u32x4 vv = ok ? pv[it][r] : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(ks + (kr0 + r) * kKPitch + ch * 16) = kv;
        vwd[r][0] = vv.x;
        vwd[r][1] = vv.y;
        vwd[r][2] = vv.z;
        vwd[r][3] = vv.w;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {   // channels ch*8 + 2j (low halves) and ch*8 + 2j + 1 (high halves)
        const uint2 lo = uint2{(vwd[0][j] & 0xFFFFu) | (vwd[1][j] << 16), (vwd[2][j] & 0xFFFFu) | (vwd[3][j] << 16)};
        const uint2 hi = uint2{(vwd[0][j] >> 16) | (vwd[1][j] & 0xFFFF0000u),
                               (vwd[2][j] >> 16) | (vwd[3][j] & 0xFFFF0000u)};
        *reinterpret_cast<uint2*>(vt + (ch * 8 + 2 * j) * vt_pitch + kr0 * 2) = lo;
        *reinterpret_cast<uint2*>(vt + (ch * 8 + 2 * j + 1) * vt_pitch + kr0 * 2) = hi;
      }
    }
  };
  if (key_lo < key_hi) fetch(key_lo);
  for (int t0 = key_lo; t0 < key_hi; t0 += nkeys) {
    __syncthreads();   // every wave is done with the previous step
    put(t0);
    if (t0 + nkeys < key_hi) fetch(t0 + nkeys);   // uniform over the workgroup
    __syncthreads();
    const int tb = t0 + 32 * phase;          // this wave's 32-key tile
    if (!wave_on || tb >= key_hi) continue;
    // S[key][row]: lane holds row = col, key = tb + 8 (e / 4) + 4 hb + e % 4
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const bf16x8 kf =
          *reinterpret_cast<const bf16x8*>(ks + (32 * phase + col) * kKPitch + (16 * st + 8 * hb) * 2);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], sacc, 0, 0, 0);
    }
    // P = 2^(S c - rowc) (0 past the split's keys), as bf16 hi + lo; element
    // i of operand `half` is e = 8 half + i
    uint32_t ph[2][4], pl[2][4];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      uint32_t hbits[2], lbits[2];
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int ee = e + k2;
        const int key = tb + 8 * (ee >> 2) + 4 * hb + (ee & 3);
        const float pv = key < key_hi ? __builtin_amdgcn_exp2f(fmaf(sacc[ee], cc, -rc)) : 0.f;
        hbits[k2] = bf16_rne_bits(pv);
        lbits[k2] = bf16_rne_bits(pv - __uint_as_float(hbits[k2] << 16));
      }
      ph[e >> 3][(e & 7) >> 1] = hbits[0] | (hbits[1] << 16);
      pl[e >> 3][(e & 7) >> 1] = lbits[0] | (lbits[1] << 16);
    }
    // O^T[d][row] += sum over the tile's keys of V^T[d][key] P[row][key]
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const bf16x8 bh = __builtin_bit_cast(bf16x8, u32x4{ph[half][0], ph[half][1], ph[half][2], ph[half][3]});
      const bf16x8 bl = __builtin_bit_cast(bf16x8, u32x4{pl[half][0], pl[half][1], pl[half][2], pl[half][3]});
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const char* vr = vt + (32 * db + col) * vt_pitch + 64 * phase;
        const uint2 a0 = *reinterpret_cast<const uint2*>(vr + (16 * half + 4 * hb) * 2);
        const uint2 a1 = *reinterpret_cast<const uint2*>(vr + (16 * half + 8 + 4 * hb) * 2);
        const bf16x8 af = __builtin_bit_cast(bf16x8, u32x4{a0.x, a0.y, a1.x, a1.y});
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bh, oacc[db], 0, 0, 0);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bl, oacc[db], 0, 0, 0);
      }
    }
  }
  // fold the key phases of each query block in phase order through LDS
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);   // [(phase - 1) * qpw + block][64 lanes][64]
  if (phase > 0) {
    float* dst = red + ((int64_t)((phase - 1) * qpw + wave % qpw) * 64 + lane) * 64;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) dst[db * 16 + e] = oacc[db][e];
  }
  __syncthreads();
  if (phase != 0 || !wave_on || row >= R) return;
  for (int ph2 = 1; ph2 < kp; ++ph2) {
    const float* src = red + ((int64_t)((ph2 - 1) * qpw + wave % qpw) * 64 + lane) * 64;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] += src[db * 16 + e];
  }
  // O^T layout: lane holds row = col and d = 32 db + 8 (e / 4) + 4 hb + e % 4
  float* op = opart + (((int64_t)g * nsplit + split) * R + row) * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4)
      *reinterpret_cast<f32x4*>(op + 32 * db + 8 * e4 + 4 * hb) =
          f32x4{oacc[db][4 * e4], oacc[db][4 * e4 + 1], oacc[db][4 * e4 + 2], oacc[db][4 * e4 + 3]};
}

// vpart[g, rg, d] = sum over rows r in [8 rg, 8 rg + 8) of (sum over splits of
// opart[g, split, r, d])^2, every sum in a fixed order.
__global__ __launch_bounds__(kD * kVNormRows) void think_vnorm(const float* opart, int nsplit, int R,
                                                              float* vpart) {
  __shared__ float red[kVNormRows][kD];
  const int rg = blockIdx.x, g = blockIdx.y, d = threadIdx.x & (kD - 1), rr = threadIdx.x / kD;
  const int r = rg * kVNormRows + rr;
  float o2 = 0.f;
  if (r < R) {
    const float* pp = opart + ((int64_t)g * nsplit * R + r) * kD + d;
    const int64_t st = (int64_t)R * kD;
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 3 < nsplit; s += 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] += pp[(s + j) * st];
    }
    for (; s < nsplit; ++s) a[0] += pp[s * st];
    const float o = (a[0] + a[1]) + (a[2] + a[3]);
    o2 = o * o;
  }
  red[rr][d] = o2;
  __syncthreads();
  if (rr == 0) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < kVNormRows; ++i) t += red[i][d];
    vpart[((int64_t)g * gridDim.x + rg) * kD + d] = t;
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
  KVC_LAUNCH("think_select", think_select<0>, dim3(Hkv), dim3(kD * kSelGroups), s, part, nchunk, qpart, G, T,
             channels, mask);
  if (rows > 0) {
    int gx = (rows + 31) / 32;   // 4 waves x 8 rows per workgroup step
    if (gx > 1024) gx = 1024;
    uint16_t* kp = static_cast<uint16_t*>(k_pruned);
    if ((T & 1) == 0 && (reinterpret_cast<uintptr_t>(k_pruned) & 3) == 0)
      KVC_LAUNCH("think_gather", (think_gather<true, 0>), dim3(gx, Hkv), dim3(256), s, kcp, budget, rows, T, channels,
                 kp);
    else
      KVC_LAUNCH("think_gather", (think_gather<false, 0>), dim3(gx, Hkv), dim3(256), s, kcp, budget, rows, T, channels,
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

namespace kvc {
namespace {

struct ValueWs {
  size_t rowc, opart, vpart, total;
  int nsplit, nrg;
};

ValueWs value_ws(int Hkv, int G, int w, int budget, int recent) {
  ValueWs v{};
  const int rows = budget - recent, R = G * w;
  v.nsplit = rows > 0 ? (rows + kVSplit - 1) / kVSplit : 0;
  v.nrg = (R + kVNormRows - 1) / kVNormRows;
  const size_t rs = rows > 0 ? score_rowc_workspace_size(Hkv, G, w, rows, (int64_t)w * kD) : 0;
  v.rowc = 0;
  v.opart = align_up(rs, 256);
  v.vpart = v.opart + align_up((size_t)Hkv * v.nsplit * R * kD * sizeof(float), 256);
  v.total = v.vpart + align_up((size_t)Hkv * v.nrg * kD * sizeof(float), 256);
  return v;
}

}  // namespace
}  // namespace kvc

extern "C" size_t kvc_channel_prune_value_workspace_size(int32_t Hkv, int32_t G, int32_t w, int32_t budget,
                                                         int32_t recent, int32_t D) {
  if (Hkv < 1 || G < 1 || w < 1 || budget < 0 || recent < 0 || recent > budget || D != kvc::kD) return 0;
  if ((int64_t)G * w > 65536) return 0;
  return kvc::value_ws(Hkv, G, w, budget, recent).total;
}

extern "C" kvc_status kvc_channel_prune_value(const void* k_c, const void* v_c, const void* q_obs, int32_t Hkv,
                                              int32_t G, int32_t w, int64_t q_head_stride, int32_t budget,
                                              int32_t D, int32_t recent, double lambda, float scale,
                                              int32_t* channels, uint8_t* mask, void* v_pruned, void* ws,
                                              size_t ws_bytes, void* stream) {
  using namespace kvc;
  if (Hkv < 1 || G < 1 || w < 1 || budget < 0 || recent < 0 || recent > budget) return KVC_E_ARG;
  if (!(lambda >= 0.0 && lambda < 1.0) || !(scale > 0.f && scale < INFINITY)) return KVC_E_ARG;
  if (D != kD) return KVC_E_UNSUPPORTED;
  if (Hkv > 65535 || (int64_t)Hkv * G > 65535 || (int64_t)G * w > 65536) return KVC_E_SHAPE;
  if (q_head_stride < (int64_t)w * D || (q_head_stride & 7)) return KVC_E_SHAPE;
  const int T = kvc_think_channels(D, lambda);
  if (T < 1) return KVC_E_ARG;
  const int rows = budget - recent, R = G * w;
  if (!k_c || !v_c || !q_obs || !channels || (rows > 0 && !v_pruned)) return KVC_E_ARG;
  if (!aligned16(k_c) || !aligned16(v_c) || !aligned16(q_obs) || (reinterpret_cast<uintptr_t>(channels) & 3) ||
      (reinterpret_cast<uintptr_t>(v_pruned) & 1))
    return KVC_E_ARG;
  const ValueWs L = value_ws(Hkv, G, w, budget, recent);
  if (!ws || ws_bytes < L.total || !aligned16(ws)) return KVC_E_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  float* opart = reinterpret_cast<float*>(base + L.opart);
  float* vpart = reinterpret_cast<float*>(base + L.vpart);
  const uint16_t* qp = static_cast<const uint16_t*>(q_obs);
  const uint16_t* kp = static_cast<const uint16_t*>(k_c);
  const uint16_t* vp = static_cast<const uint16_t*>(v_c);
  if (rows > 0) {
    const float* rowc = nullptr;
    kvc_status st = score_rowc(qp, q_head_stride, kp, (int64_t)budget * kD, Hkv, G, w, rows, scale, base + L.rowc,
                               L.opart - L.rowc, &rowc, s);
    if (st != KVC_OK) return st;
    const int qpw = vq_per_wg(R);
    const int nqg = ((R + 31) / 32 + qpw - 1) / qpw;
    KVC_LAUNCH("think_vpartial", think_vpartial, dim3(L.nsplit, Hkv, nqg), dim3(kVWaves * kWave), s, qp,
               q_head_stride, G, w, kp, vp, budget, rows, rowc, scale * kLog2e, L.nsplit, opart);
  }
  KVC_LAUNCH("think_vnorm", think_vnorm, dim3(L.nrg, Hkv), dim3(kD * kVNormRows), s, opart, L.nsplit, R, vpart);
  KVC_LAUNCH("think_select_v", think_select<1>, dim3(Hkv), dim3(kD * kSelGroups), s, vpart, L.nrg, nullptr, 0, T,
             channels, mask);
  if (rows > 0) {
    int gx = (rows + 31) / 32;
    if (gx > 1024) gx = 1024;
    uint16_t* out = static_cast<uint16_t*>(v_pruned);
    if ((T & 1) == 0 && (reinterpret_cast<uintptr_t>(v_pruned) & 3) == 0)
      KVC_LAUNCH("think_gather_v", (think_gather<true, 1>), dim3(gx, Hkv), dim3(256), s, vp, budget, rows, T, channels,
                 out);
    else
      KVC_LAUNCH("think_gather_v", (think_gather<false, 1>), dim3(gx, Hkv), dim3(256), s, vp, budget, rows, T, channels,
                 out);
  }
  return KVC_OK;
}
