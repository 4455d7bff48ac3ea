// Channel statistics, K smoothing and the INT8 / FP8 quantisation kernels.
//
// These are HBM-bound scans: every kernel reads each input element once per
// pass with 16-byte coalesced loads (a token row of one head is d contiguous
// 16-bit values in both layouts) and writes codes with 8/16-byte stores.
//
// Arithmetic is kept bit-compatible with a plain IEEE reading of the method:
// fp64 channel sums, correctly rounded fp32 divides, separate (never fused)
// subtract and multiply, round-half-to-even to integers.
#include <algorithm>

#include "sage_device.h"
#include "sage_launch.h"

#pragma clang fp contract(off)

namespace sage {


// Per (b, kv-head, 256-token chunk): fp64 sums of K over tokens per channel and,
// optionally, fp32 max |V| per channel. Partials go to [B*H][chunks][D] in a
// fixed order (no atomics), so the result does not depend on scheduling.
// Packed batches (seq set): b is the sequence and its keys are the range
// [k0, k0 + nk) of the packed tensor.
template <typename T, int D, bool WITH_K, bool WITH_V>
__global__ __launch_bounds__(256) void channel_stats_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, TensorGeom geo, int H, int N,
    int chunks, double* __restrict__ ksum_part, float* __restrict__ vmax_part, const SeqSpan* __restrict__ seq) {
  constexpr int TPR = D / 8;        // threads per token row (8 values each)
  constexpr int RPI = 256 / TPR;    // token rows per iteration
  __shared__ double red_k[RPI][D];
  __shared__ float red_v[RPI][D];
  const int tid = threadIdx.x;
  const int col = (tid % TPR) * 8;
  const int r0 = tid / TPR;
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh % H;
  int64_t base = (int64_t)b * geo.batch_stride + (int64_t)h * geo.head_stride + col;
  int n = N;
  if (seq) {
    n = seq[b].nk;
    base += (int64_t)seq[b].k0 * geo.tok_stride;
  }
  const int t_begin = blockIdx.x * kStatChunk;
  const int t_end = min(n, t_begin + kStatChunk);

  double ks[8];
  float vm[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { ks[e] = 0.0; vm[e] = 0.0f; }
  // All of the thread's rows are loaded before any is used, so every load is
  // in flight at once (16 rows of 16 bytes per tensor). Rows past the end
  // re-read the chunk's first row and add -0.0 to the sums (an exact
  // identity) or 0 to the maxima. (A chunk wholly past a packed sequence's
  // keys loads nothing and writes zero partials.)
  constexpr int ROWS = kStatChunk / RPI;
  i32x4 rk[WITH_K ? ROWS : 1], rv[WITH_V ? ROWS : 1];
  if (t_begin < t_end) {
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
      const int t = t_begin + r0 + i * RPI;
      const int64_t off = base + (int64_t)(t < t_end ? t : t_begin) * geo.tok_stride;
      if (WITH_K) rk[i] = *reinterpret_cast<const i32x4*>(k + off);
      if (WITH_V) rv[i] = *reinterpret_cast<const i32x4*>(v + off);
    }
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
      const bool live = t_begin + r0 + i * RPI < t_end;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (WITH_K) {
          const uint16_t bits = (uint16_t)(((uint32_t)rk[i][e / 2]) >> (16 * (e & 1)));
          ks[e] += live ? (double)T::to_f32(bits) : -0.0;
        }
        if (WITH_V) {
          const uint16_t bits = (uint16_t)(((uint32_t)rv[i][e / 2]) >> (16 * (e & 1)));
          vm[e] = fmaxf(vm[e], live ? fabsf(T::to_f32(bits)) : 0.0f);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (WITH_K) red_k[r0][col + e] = ks[e];
    if (WITH_V) red_v[r0][col + e] = vm[e];
  }
  __syncthreads();
  if (tid < D) {
    const int64_t o = ((int64_t)bh * chunks + blockIdx.x) * D + tid;
    if (WITH_K) {
      double s = 0.0;
      for (int r = 0; r < RPI; ++r) s += red_k[r][tid];
      ksum_part[o] = s;
    }
    if (WITH_V) {
      float m = 0.0f;
      for (int r = 0; r < RPI; ++r) m = fmaxf(m, red_v[r][tid]);
      vmax_part[o] = m;
    }
  }
}

// Per (b, kv-head, channel): mu = fp32(sum / N) (fp64 divide, one rounding to
// fp32); s_v = a_v / 448 and 448 / a_v (both correctly rounded fp32 divides).
// (packed batches: the token count is the sequence's; a sequence without keys
// gets a zero mean)
// kFinalizeThreads threads per (b, kv-head): P = kFinalizeThreads / D threads
// per channel, thread p folding chunks p, p + P, ... with eight independent
// accumulators (eight loads in flight each), the P results combined in a
// fixed order through LDS, so the result does not depend on timing.
constexpr int kFinalizeThreads = 512;
template <int D, bool WITH_K, bool WITH_V>
__global__ __launch_bounds__(kFinalizeThreads) void channel_finalize_kernel(
    int N, int chunks, const double* __restrict__ ksum_part, const float* __restrict__ vmax_part,
    float* __restrict__ k_mean, float* __restrict__ v_scale, float* __restrict__ v_inv, int H,
    const SeqSpan* __restrict__ seq) {
  constexpr int P = kFinalizeThreads / D;
  constexpr int U = 8;
  __shared__ double part_k[WITH_K ? P : 1][D];
  __shared__ float part_v[WITH_V ? P : 1][D];
  const int bh = blockIdx.x, c = threadIdx.x % D, pi = threadIdx.x / D;
  const int n = seq ? seq[bh / H].nk : N;
  const int64_t p = (int64_t)bh * chunks * D + c;
  if (WITH_K) {
    double s[U] = {};
    int i = pi;
    for (; i + (U - 1) * P < chunks; i += U * P)
#pragma unroll
      for (int u = 0; u < U; ++u) s[u] += ksum_part[p + (int64_t)(i + u * P) * D];
    for (; i < chunks; i += P) s[0] += ksum_part[p + (int64_t)i * D];
    part_k[pi][c] = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
  }
  if (WITH_V) {
    float a[U] = {};
    int i = pi;
    for (; i + (U - 1) * P < chunks; i += U * P)
#pragma unroll
      for (int u = 0; u < U; ++u) a[u] = fmaxf(a[u], vmax_part[p + (int64_t)(i + u * P) * D]);
    for (; i < chunks; i += P) a[0] = fmaxf(a[0], vmax_part[p + (int64_t)i * D]);
    part_v[pi][c] = fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])), fmaxf(fmaxf(a[4], a[5]), fmaxf(a[6], a[7])));
  }
  __syncthreads();
  if (threadIdx.x >= D) return;
  if (WITH_K) {
    double total = part_k[0][c];
#pragma unroll
    for (int q = 1; q < P; ++q) total += part_k[q][c];
    k_mean[bh * D + c] = n > 0 ? (float)(total / (double)n) : 0.0f;
  }
  if (WITH_V) {
    float m = part_v[0][c];
#pragma unroll
    for (int q = 1; q < P; ++q) m = fmaxf(m, part_v[q][c]);
    v_scale[bh * D + c] = m / kE4m3Max;
    v_inv[bh * D + c] = m > 0.0f ? kE4m3Max / m : 0.0f;
  }
}

// INT8 quantisation per (b, head, block of BLK tokens): optional smoothing
// x - mu[c], block absmax a, s = a/127, codes = rne(x * (127/a)).
// Thread tid of pass `it` holds the 16-byte chunk (it*256 + tid) of the
// work-group's token rows, so a block is G = BLK * D/8 consecutive chunks.
// Blocks of G >= 256 chunks take one work-group each (reduction over the
// whole group); smaller blocks share 64-token work-groups, and each pass
// reduces its 256/G blocks over lane groups of G (in-wave butterflies up to
// 64 lanes, one LDS exchange between waves above).
// Packed batches (seq set): b is the sequence, its tokens are the range given
// by the span's query (side 0) or key (side 1) pair, codes go to
// [H][total][D], and nblk is the per-sequence scale stride. Work-groups past
// the sequence's end leave at once: the attention kernel reads a Q scale only
// for rows that exist and a K scale past the keys only for masked scores.
// Threads per work-group: 512 for blocks of at least 2048 chunks (128 tokens
// at d = 128), so that each thread holds 4 chunks instead of 8 and the kernel
// keeps 8 waves per SIMD; 256 otherwise.
template <int D, int BLK>
struct QuantThreads {
  static constexpr int value = BLK * (D / 8) >= 2048 ? 512 : 256;
};

template <typename T, int D, int BLK, bool SMOOTH>
__global__ __launch_bounds__((QuantThreads<D, BLK>::value)) void quant_int8_kernel(
    const uint16_t* __restrict__ x, TensorGeom geo, int H, int N, int nblk,
    const float* __restrict__ mean, int8_t* __restrict__ codes, float* __restrict__ scale,
    const SeqSpan* __restrict__ seq, int side, int total) {
  constexpr int NT = QuantThreads<D, BLK>::value;
  constexpr int TPR = D / 8;
  constexpr int G = BLK * TPR;                   // chunks per block
  constexpr bool WHOLE = G >= NT;                // one block per work-group
  constexpr int TOKS = WHOLE ? BLK : 64;         // token rows per work-group
  constexpr int ITER = TOKS * TPR / NT;          // 16-byte chunks per thread
  static_assert(ITER * NT == TOKS * TPR, "token rows must tile the work-group");
  static_assert(WHOLE ? G % NT == 0 : NT % G == 0, "blocks must tile the passes");
  __shared__ float red[NT / 64];
  const int tid = threadIdx.x;
  const int col = (tid % TPR) * 8;        // NT % TPR == 0: fixed per thread
  // Work-groups run in reverse launch order. For K the statistics pass has just
  // read the tensor front to back, so its tail is the part the last-level cache
  // still holds; for Q the order makes no difference.
  const int bh = gridDim.y - 1 - blockIdx.y;
  const int b = bh / H, h = bh % H;
  int64_t base = (int64_t)b * geo.batch_stride + (int64_t)h * geo.head_stride + col;
  int8_t* out = codes + (int64_t)bh * N * D + col;
  if (seq) {
    const int32_t* sp = &seq[b].q0 + 2 * side;   // (q0, nq) or (k0, nk)
    N = sp[1];
    base += (int64_t)sp[0] * geo.tok_stride;
    out = codes + ((int64_t)h * total + sp[0]) * D + col;
  }

  float mu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = SMOOTH ? mean[bh * D + col + e] : 0.0f;

  // One pass per TOKS-token tile. Work-group i takes the tiles ntiles-1-i,
  // ntiles-1-i-G, ... (G = gridDim.x): a dense launch has kQuantTilesPerWg of
  // them per work-group; a packed batch's grid covers about the average
  // sequence, and its work-groups stride over the tiles of longer ones (rather
  // than launching the longest sequence's tile count for every sequence,
  // mostly empty). The next tile's loads are issued before the current tile's
  // reduction, so they are in flight during its barrier and its stores.
  const int ntiles = (N + TOKS - 1) / TOKS;
  auto load_tile = [&](int bx, i32x4 (&raw)[ITER]) {
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int t = bx * TOKS + (it * NT + tid) / TPR;
      raw[it] = t < N ? *reinterpret_cast<const i32x4*>(x + base + (int64_t)t * geo.tok_stride) : i32x4{0, 0, 0, 0};
    }
  };
  const int g = (int)gridDim.x;
  i32x4 cur[ITER], nxt[ITER];
  if ((int)blockIdx.x < ntiles) load_tile(ntiles - 1 - (int)blockIdx.x, cur);
  for (int idx = blockIdx.x; idx < ntiles; idx += g) {
    const int bx = ntiles - 1 - idx;
    const int t0 = bx * TOKS;
    if (idx + g < ntiles) load_tile(ntiles - 1 - idx - g, nxt);
    else
#pragma unroll
      for (int it = 0; it < ITER; ++it) nxt[it] = i32x4{0, 0, 0, 0};
    float val[ITER][8];
    float amax[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int t = t0 + (it * NT + tid) / TPR;
      amax[it] = 0.0f;
      if (t < N) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint16_t bits = (uint16_t)(((uint32_t)cur[it][e / 2]) >> (16 * (e & 1)));
          float f = T::to_f32(bits);
          if (SMOOTH) f = f - mu[e];
          val[it][e] = f;
          amax[it] = fmaxf(amax[it], fabsf(f));
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) val[it][e] = 0.0f;
      }
    }
    float inv[ITER];
    if constexpr (WHOLE) {
      float a = 0.0f;
#pragma unroll
      for (int it = 0; it < ITER; ++it) a = fmaxf(a, amax[it]);
      a = wave_max(a);
      if ((tid & 63) == 0) red[tid >> 6] = a;
      __syncthreads();
      a = red[0];
#pragma unroll
      for (int w = 1; w < NT / 64; ++w) a = fmaxf(a, red[w]);
      if (tid == 0) scale[(int64_t)bh * nblk + bx] = a / 127.0f;
#pragma unroll
      for (int it = 0; it < ITER; ++it) inv[it] = a > 0.0f ? 127.0f / a : 0.0f;
      __syncthreads();                   // red is rewritten by the next pass
    } else {
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        float a = amax[it];
#pragma unroll
        for (int o = 1; o < (G < 64 ? G : 64); o <<= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
        if constexpr (G > 64) {
          // the G/64 waves of each block exchange their maxima
          if ((tid & 63) == 0) red[tid >> 6] = a;
          __syncthreads();
          const int w0 = (tid >> 6) & ~(G / 64 - 1);
#pragma unroll
          for (int w = 0; w < G / 64; ++w) a = fmaxf(a, red[w0 + w]);
          __syncthreads();               // red is rewritten by the next pass
        }
        const int blk = (t0 + (it * NT + tid) / TPR) / BLK;
        if (tid % G == 0 && blk < nblk) scale[(int64_t)bh * nblk + blk] = a / 127.0f;
        inv[it] = a > 0.0f ? 127.0f / a : 0.0f;
      }
    }

#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int t = t0 + (it * NT + tid) / TPR;
      if (t < N) {
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float prod = val[it][e] * inv[it];
          const int q = (int)__builtin_rintf(prod);
          w[e / 4] |= ((uint32_t)(q & 0xff)) << (8 * (e & 3));
        }
        *reinterpret_cast<i32x2*>(out + (int64_t)t * D) = i32x2{(int)w[0], (int)w[1]};
      }
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) cur[it] = nxt[it];
  }
}

// Work-groups along the token axis for `units` slots of `per_unit` tokens: one
// per slot, or, for a packed batch, about the average sequence's slot count
// (the kernels then stride over the slots of longer sequences).
// Tiles per work-group of a dense quantisation launch. One: same machine, the
// whole quantisation took 0.328 ms with one tile per work-group and 0.339,
// 0.346, 0.359, 0.365 ms with 2, 4, 8, 16 (fewer work-groups in flight).
constexpr int kQuantTilesPerWg = 1;
static int token_wgs(int units, int per_unit, const SeqSpan* seq, int B, int total) {
  if (!seq) return (units + kQuantTilesPerWg - 1) / kQuantTilesPerWg;
  const int64_t per = (int64_t)B * per_unit;
  return (int)std::max<int64_t>(1, std::min<int64_t>(units, ((int64_t)total + per - 1) / per));
}

// Launch of quant_int8_kernel over N tokens of B*H heads.
// (N: the token count, or the longest sequence of a packed batch)
template <typename T, int D, int BLK, bool SMOOTH>
static void launch_quant_int8(const void* x, TensorGeom geo, int BH, int H, int N, const float* mean,
                              int8_t* codes, float* scale, const SeqSpan* seq, int side, int total,
                              hipStream_t st) {
  constexpr int NT = QuantThreads<D, BLK>::value;
  constexpr int TOKS = BLK * (D / 8) >= NT ? BLK : 64;
  const int nblk = (N + BLK - 1) / BLK;
  const int wgs = token_wgs((N + TOKS - 1) / TOKS, TOKS, seq, BH / H, total);
  hipLaunchKernelGGL((quant_int8_kernel<T, D, BLK, SMOOTH>), dim3(wgs, BH), dim3(NT), 0, st,
                     (const uint16_t*)x, geo, H, N, nblk, mean, codes, scale, seq, side, total);
}

// V transposed to [D][Nk_pad] with keys contiguous per channel, in 64-token
// tiles, kQuantTilesPerWg of them per work-group of a (b, kv-head). FP8: e4m3(v * (448/a_v[c]));
// otherwise the 16-bit values are copied. Tokens >= N are written as 0.
// Packed batches (seq set): b is the sequence, its keys [k0, k0 + nk) go to the
// columns [kp0, kp0 + nk rounded up to the KV tile) of rows [H][D][n_pad].
template <typename T, int D, bool FP8>
__global__ __launch_bounds__(256) void transpose_v_kernel(
    const uint16_t* __restrict__ v, TensorGeom geo, int H, int N, int n_pad,
    const float* __restrict__ v_inv, void* __restrict__ out, const SeqSpan* __restrict__ seq) {
  constexpr int EB = FP8 ? 1 : 2;               // output bytes per element
  constexpr int ROWB = 64 * EB;                 // bytes per channel row of the tile
  constexpr int UNITS = (64 / 4) * (D / 8);     // 4 tokens x 8 channels per unit
  __shared__ __attribute__((aligned(16))) uint8_t tile[D * ROWB];
  static_assert(UNITS <= 256, "one unit per thread at most");
  const int tid = threadIdx.x;
  // reverse launch order, as in quant_int8_kernel (V's statistics pass ran just before)
  const int bh = gridDim.y - 1 - blockIdx.y;
  const int b = bh / H, h = bh % H;
  int64_t base = (int64_t)b * geo.batch_stride + (int64_t)h * geo.head_stride;
  int64_t dst0 = (int64_t)bh * D * n_pad;
  int ntiles = n_pad / 64;
  if (seq) {
    const SeqSpan sp = seq[b];
    ntiles = (sp.nk + kVPad - 1) / kVPad * (kVPad / 64);   // this sequence's padded keys
    N = sp.nk;
    base += (int64_t)sp.k0 * geo.tok_stride;
    dst0 = (int64_t)h * D * n_pad + sp.kp0;
  }
  const bool has_unit = tid < UNITS;
  const int c0 = (tid % (D / 8)) * 8;
  const int tt = (tid / (D / 8)) * 4;           // first token of the unit inside the tile
  // Work-group i takes the tiles ntiles-1-i, ntiles-1-i-G, ... (G = gridDim.x),
  // with the next tile's loads in flight while the current one is converted,
  // transposed through LDS and stored.
  auto load_tile = [&](int t0, i32x4 (&raw)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + tt + j;
      raw[j] = has_unit && t < N ? *reinterpret_cast<const i32x4*>(v + base + (int64_t)t * geo.tok_stride + c0)
                                 : i32x4{0, 0, 0, 0};   // +0.0 in both dtypes and in e4m3
    }
  };
  const int g = (int)gridDim.x;
  i32x4 cur[4], nxt[4];
  if ((int)blockIdx.x < ntiles) load_tile((ntiles - 1 - (int)blockIdx.x) * 64, cur);
  for (int idx = blockIdx.x; idx < ntiles; idx += g) {
    const int t0 = (ntiles - 1 - idx) * 64;
    if (idx + g < ntiles) load_tile((ntiles - 1 - idx - g) * 64, nxt);
    else
#pragma unroll
      for (int j = 0; j < 4; ++j) nxt[j] = i32x4{0, 0, 0, 0};
    if (has_unit) {
      uint32_t raw16[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) raw16[j][e] = (((uint32_t)cur[j][e / 2]) >> (16 * (e & 1))) & 0xffffu;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = c0 + e;
        if (FP8) {
          const float s = v_inv[bh * D + c];
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(T::to_f32((uint16_t)raw16[0][e]) * s,
                                                  T::to_f32((uint16_t)raw16[1][e]) * s, 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(T::to_f32((uint16_t)raw16[2][e]) * s,
                                              T::to_f32((uint16_t)raw16[3][e]) * s, w, true);
          *reinterpret_cast<int*>(tile + c * ROWB + tt) = w;
        } else {
          const uint32_t lo = raw16[0][e] | (raw16[1][e] << 16);
          const uint32_t hi = raw16[2][e] | (raw16[3][e] << 16);
          *reinterpret_cast<i32x2*>(tile + c * ROWB + tt * 2) = i32x2{(int)lo, (int)hi};
        }
      }
    }
    __syncthreads();
    uint8_t* dst = reinterpret_cast<uint8_t*>(out) + (dst0 + t0) * EB;
    constexpr int CHUNKS = D * ROWB / 16;
    for (int ci = tid; ci < CHUNKS; ci += 256) {
      const int c = ci / (ROWB / 16), j = ci % (ROWB / 16);
      *reinterpret_cast<i32x4*>(dst + (int64_t)c * n_pad * EB + j * 16) =
          *reinterpret_cast<const i32x4*>(tile + c * ROWB + j * 16);
    }
    __syncthreads();                         // the tile is rewritten by the next pass
#pragma unroll
    for (int j = 0; j < 4; ++j) cur[j] = nxt[j];
  }
}

// Per-sequence spans of a packed batch from the caller's cu_seqlens (B + 1
// non-decreasing offsets each), and the attention work list: entry i of
// qp_owner names the sequence of the i-th query pair (256 queries), the pairs
// of sequence b being entries [qp0, qp0 + ceil(nq/256)), -1 after the last.
// One work-group walks the sequences 256 at a time with LDS prefix sums for
// the padded V^T column starts and the work-list starts. Every range is
// clamped into the packed tensors and the longest-sequence bounds; a sequence
// whose padded keys would pass n_pad, or whose query pairs would pass the
// work list (both possible only for a malformed table), loses its keys or the
// pairs past the end, so no later kernel can index out of bounds.
__global__ __launch_bounds__(256) void varlen_plan_kernel(const int32_t* __restrict__ cu_q,
                                                          const int32_t* __restrict__ cu_k, int B, int total_q,
                                                          int total_k, int max_q, int max_k, int n_pad,
                                                          SeqSpan* __restrict__ out, int32_t* __restrict__ qp_owner,
                                                          int n_owner) {
  __shared__ int part[256];          // <= 256 * 2^20: fits
  __shared__ int partq[256];
  __shared__ int64_t carry, carryq;  // a malformed table can pass 2^31
  const int tid = threadIdx.x;
  if (tid == 0) {
    carry = 0;
    carryq = 0;
  }
  __syncthreads();
  for (int b0 = 0; b0 < B; b0 += 256) {
    const int b = b0 + tid;
    SeqSpan sp{};
    int padded = 0, pairs = 0;
    if (b < B) {
      const int q0 = min(max(cu_q[b], 0), total_q), q1 = min(max(cu_q[b + 1], q0), total_q);
      const int k0 = min(max(cu_k[b], 0), total_k), k1 = min(max(cu_k[b + 1], k0), total_k);
      sp.q0 = q0;
      sp.nq = min(q1 - q0, max_q);
      sp.k0 = k0;
      sp.nk = min(k1 - k0, max_k);
      padded = (sp.nk + kVPad - 1) / kVPad * kVPad;
      pairs = (sp.nq + 255) / 256;
    }
    part[tid] = padded;
    partq[tid] = pairs;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {          // inclusive scans
      const int add = tid >= o ? part[tid - o] : 0;
      const int addq = tid >= o ? partq[tid - o] : 0;
      __syncthreads();
      part[tid] += add;
      partq[tid] += addq;
      __syncthreads();
    }
    if (b < B) {
      const int64_t kp0 = carry + part[tid] - padded;   // padded keys of the earlier sequences
      if (kp0 + padded > n_pad) {
        sp.nk = 0;
        sp.kp0 = 0;
      } else {
        sp.kp0 = (int)kp0;
      }
      const int64_t qp0 = carryq + partq[tid] - pairs;
      sp.qp0 = (int)min(qp0, (int64_t)n_owner);
      for (int64_t i = qp0; i < qp0 + pairs && i < n_owner; ++i) qp_owner[i] = b;
      out[b] = sp;
    }
    __syncthreads();
    if (tid == 0) {
      carry += part[255];
      carryq += partq[255];
    }
    __syncthreads();
  }
  for (int64_t i = carryq + tid; i < n_owner; i += 256) qp_owner[i] = -1;
}

// ---------------------------------------------------------------- host launchers
hipError_t launch_varlen_plan(const int32_t* cu_q, const int32_t* cu_k, int B, int total_q, int total_k, int max_q,
                              int max_k, int n_pad, SeqSpan* out, int32_t* qp_owner, int n_owner, hipStream_t st) {
  hipLaunchKernelGGL(varlen_plan_kernel, dim3(1), dim3(256), 0, st, cu_q, cu_k, B, total_q, total_k, max_q, max_k,
                     n_pad, out, qp_owner, n_owner);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_qk_t(const QuantQKArgs& a, hipStream_t st) {
  const int chunks = (a.Nk + kStatChunk - 1) / kStatChunk;
  const int bhk = a.B * a.Hkv;
  if (a.Nk > 0) {
    hipLaunchKernelGGL((channel_stats_kernel<T, D, true, false>), dim3(chunks, bhk), dim3(256), 0, st,
                       (const uint16_t*)a.k, (const uint16_t*)nullptr, a.kgeo, a.Hkv, a.Nk, chunks,
                       a.ksum_part, (float*)nullptr, a.seq);
    hipLaunchKernelGGL((channel_finalize_kernel<D, true, false>), dim3(bhk), dim3(kFinalizeThreads), 0, st,
                       a.Nk, chunks, a.ksum_part, (const float*)nullptr, a.k_mean, (float*)nullptr,
                       (float*)nullptr, a.Hkv, a.seq);
    if (a.fine)
      launch_quant_int8<T, D, kFineBlkK, true>(a.k, a.kgeo, bhk, a.Hkv, a.Nk, a.k_mean, a.k_codes, a.k_scale,
                                               a.seq, 1, a.total_k, st);
    else
      launch_quant_int8<T, D, kBlkK, true>(a.k, a.kgeo, bhk, a.Hkv, a.Nk, a.k_mean, a.k_codes, a.k_scale,
                                           a.seq, 1, a.total_k, st);
  }
  if (a.Nq > 0) {
    const int bhq = a.B * a.Hq;
    if (a.fine)
      launch_quant_int8<T, D, kFineBlkQ, false>(a.q, a.qgeo, bhq, a.Hq, a.Nq, nullptr, a.q_codes, a.q_scale,
                                                a.seq, 0, a.total_q, st);
    else
      launch_quant_int8<T, D, kBlkQ, false>(a.q, a.qgeo, bhq, a.Hq, a.Nq, nullptr, a.q_codes, a.q_scale,
                                            a.seq, 0, a.total_q, st);
  }
  return hipGetLastError();
}

hipError_t launch_quant_qk(const QuantQKArgs& a, hipStream_t st) {
  if (a.bf16) return a.D == 64 ? launch_qk_t<BF16, 64>(a, st) : launch_qk_t<BF16, 128>(a, st);
  return a.D == 64 ? launch_qk_t<F16, 64>(a, st) : launch_qk_t<F16, 128>(a, st);
}

template <typename T, int D>
static hipError_t launch_k_mean_t(const void* k, TensorGeom kgeo, int B, int Hkv, int Nk, double* ksum_part,
                                  float* k_mean, hipStream_t st, const SeqSpan* seq) {
  const int chunks = (Nk + kStatChunk - 1) / kStatChunk;
  const int bhk = B * Hkv;
  hipLaunchKernelGGL((channel_stats_kernel<T, D, true, false>), dim3(chunks, bhk), dim3(256), 0, st,
                     (const uint16_t*)k, (const uint16_t*)nullptr, kgeo, Hkv, Nk, chunks, ksum_part, (float*)nullptr,
                     seq);
  hipLaunchKernelGGL((channel_finalize_kernel<D, true, false>), dim3(bhk), dim3(kFinalizeThreads), 0, st, Nk, chunks,
                     ksum_part, (const float*)nullptr, k_mean, (float*)nullptr, (float*)nullptr, Hkv, seq);
  return hipGetLastError();
}

hipError_t launch_k_mean(const void* k, TensorGeom kgeo, int B, int Hkv, int Nk, int D, bool bf16, double* ksum_part,
                         float* k_mean, hipStream_t st, const SeqSpan* seq) {
  if (Nk <= 0) return hipSuccess;
  if (bf16)
    return D == 64 ? launch_k_mean_t<BF16, 64>(k, kgeo, B, Hkv, Nk, ksum_part, k_mean, st, seq)
                   : launch_k_mean_t<BF16, 128>(k, kgeo, B, Hkv, Nk, ksum_part, k_mean, st, seq);
  return D == 64 ? launch_k_mean_t<F16, 64>(k, kgeo, B, Hkv, Nk, ksum_part, k_mean, st, seq)
                 : launch_k_mean_t<F16, 128>(k, kgeo, B, Hkv, Nk, ksum_part, k_mean, st, seq);
}

template <typename T, int D>
static hipError_t launch_v_t(const QuantVArgs& a, hipStream_t st) {
  const int bhk = a.B * a.Hkv;
  // (packed batches: n_pad is the padded-key bound of all sequences; a
  //  sequence spans at most the longest one rounded up to the tile)
  const int tiles = ((a.seq ? (a.Nk + kVPad - 1) / kVPad * kVPad : a.n_pad) / 64 + kQuantTilesPerWg - 1) /
                    kQuantTilesPerWg;
  if (a.fp8) {
    const int chunks = (a.Nk + kStatChunk - 1) / kStatChunk;
    hipLaunchKernelGGL((channel_stats_kernel<T, D, false, true>), dim3(chunks, bhk), dim3(256), 0, st,
                       (const uint16_t*)nullptr, (const uint16_t*)a.v, a.vgeo, a.Hkv, a.Nk, chunks,
                       (double*)nullptr, a.vmax_part, a.seq);
    hipLaunchKernelGGL((channel_finalize_kernel<D, false, true>), dim3(bhk), dim3(kFinalizeThreads), 0, st,
                       a.Nk, chunks, (const double*)nullptr, a.vmax_part, (float*)nullptr, a.v_scale,
                       a.v_inv, a.Hkv, a.seq);
    hipLaunchKernelGGL((transpose_v_kernel<T, D, true>), dim3(tiles, bhk), dim3(256), 0, st,
                       (const uint16_t*)a.v, a.vgeo, a.Hkv, a.Nk, a.n_pad, (const float*)a.v_inv, a.out, a.seq);
  } else {
    hipLaunchKernelGGL((transpose_v_kernel<T, D, false>), dim3(tiles, bhk), dim3(256), 0, st,
                       (const uint16_t*)a.v, a.vgeo, a.Hkv, a.Nk, a.n_pad, (const float*)nullptr, a.out, a.seq);
  }
  return hipGetLastError();
}

hipError_t launch_quant_v(const QuantVArgs& a, hipStream_t st) {
  if (a.bf16) return a.D == 64 ? launch_v_t<BF16, 64>(a, st) : launch_v_t<BF16, 128>(a, st);
  return a.D == 64 ? launch_v_t<F16, 64>(a, st) : launch_v_t<F16, 128>(a, st);
}

}  // namespace sage
