// The FP4 microscaling variant: MXFP4 quantisation of Q, K (smoothed) and V,
// and the fused attention kernel on the block-scaled FP4 matrix cores.
//
// SageAttention3 brings FP4 microscaling to the method (heatdrop.ai review,
// "Key highlights"; cnnetsun.cn guide, 序列长度优化技巧); the pages name it
// without a format. The format here is OCP MXFP4: E2M1 elements, one E8M0
// power-of-two scale per 32 elements along the contraction axis of each
// product, which is the operand format of gfx950's block-scaled
// v_mfma_scale_f32_32x32x64_f8f6f4. Q and the smoothed K are blocked per token
// and 32 channels, V per channel and 32 keys, P~ per query row and 32 keys of
// its tile. Shared exponent of a block: floor(log2 amax) - 2 (the exponent of
// E2M1's largest value), clamped to E8M0; elements x / 2^exponent rounded half
// to even, saturating at 6. Q is scaled by c = sm_scale * log2(e) before it
// is quantised, so the product yields log2-domain scores with no per-score
// multiply (the power-of-two block scales cannot carry c).
//
// Layouts (codes two per byte, element 2i in the low nibble):
//   q_codes [B*Hq][Nq][D/2]    q_scale [B*Hq][Nq][D/32]       (E8M0 bytes; of Q * c)
//   k_codes [B*Hkv][Nk][D/2]   k_scale [B*Hkv][Nk][D/32]
//   v_codes [B*Hkv][D][n_pad/2] (V^T, keys contiguous, zero past Nk)
//   v_scale [B*Hkv][n_pad/128][D][4] (per 128-key tile: each channel's four
//           32-key blocks, so one tile's scales are one contiguous run)
// Packed variable-length batches (tokens of all sequences concatenated): the
// codes and their scales are [H][total][.], k_mean [sequence][Hkv][D], and V^T
// [Hkv][D][n_pad/2] with each sequence's keys from column kp0 of its span (a
// multiple of 128), so its tiles and their scale runs never straddle two
// sequences.
#include <type_traits>

#include "attn_schedule.h"
#include "sage_device.h"
#include "sage_launch.h"

#pragma clang fp contract(off)

namespace sage {
namespace fp4 {

constexpr int kMx = 32;            // elements per MX block
constexpr int kBq = 128;           // queries per group
constexpr int kBlocks = kBkv / 32; // 32-key S^T blocks per tile
constexpr int kWaves = 8;

// E8M0 byte of a block with largest magnitude `amax` (>= 0): floor(log2 amax)
// - 2 + 127, clamped at 0 (zero, subnormal and tiny blocks). amax's exponent
// field is floor(log2 amax) + 127 for normal values.
__device__ __forceinline__ int mx_scale_byte(float amax) {
  const int e = (int)(__builtin_bit_cast(uint32_t, amax) >> 23);
  return e > 2 ? e - 2 : 0;
}

// Eight values (x / 2^(byte - 127)) to E2M1, packed into one dword (value 2i
// in the low nibble of byte i). The multiply by a power of two is exact
// wherever the result can round to a nonzero code; the conversion rounds half
// to even and saturates at 6.
__device__ __forceinline__ uint32_t pack8(const float (&x)[8], int byte) {
  const int sh = 127 - byte;
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = __builtin_ldexpf(x[e], sh);
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

// ----------------------------------------------------------------- quantisation
// Q or K rows: thread = one 16-byte chunk (8 channels) of one token row; the
// four threads of a 32-channel block are adjacent lanes. Chunks are numbered
// over [B*H][N][D/8] (the codes' order), ITER per thread.
// Packed batches (seq set, K only): the rows are [H][total_k] and a token's
// smoothing mean is its sequence's (the last span starting at or before it).
template <typename T, int D, bool SMOOTH>
__global__ __launch_bounds__(256) void quant_rows_fp4_kernel(const uint16_t* __restrict__ x, TensorGeom geo, int H,
                                                             int N, int64_t total_chunks,
                                                             const float* __restrict__ mean, float mul,
                                                             uint32_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scale,
                                                             const SeqSpan* __restrict__ seq, int n_seq) {
  constexpr int CPR = D / 8;      // chunks per row
  constexpr int ITER = 4;
  // (a work-group covers whole 4-chunk blocks: 256 is a multiple of 4, and a
  //  block past the end is past it in all four lanes)
  // The ITER chunk loads of a pass (and, for K, the chunks' smoothing means)
  // are issued together, then converted. Chunks past the end read as zero and
  // are not stored.
  for (int64_t c0 = (int64_t)blockIdx.x * (256 * ITER) + threadIdx.x; c0 < total_chunks;
       c0 += (int64_t)gridDim.x * (256 * ITER)) {
    i32x4 raw[ITER];
    f32x4 mu[ITER][2];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int64_t ci = c0 + it * 256;
      const bool live = ci < total_chunks;
      const int64_t row = ci / CPR;
      const int col = (int)(ci % CPR) * 8;
      const int64_t bh = row / N;
      const int t = (int)(row % N);
      const int b = (int)(bh / H), h = (int)(bh % H);
      raw[it] = live ? *reinterpret_cast<const i32x4*>(x + (int64_t)b * geo.batch_stride +
                                                       (int64_t)h * geo.head_stride + (int64_t)t * geo.tok_stride + col)
                     : i32x4{0, 0, 0, 0};
      if (SMOOTH) {
        int64_t mrow = bh;                             // row of the smoothing mean
        if (seq && live) {
          int lo = 0, hi = n_seq - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (seq[mid].k0 <= t) lo = mid; else hi = mid - 1;
          }
          mrow = (int64_t)lo * H + h;
        }
        const f32x4* mp = reinterpret_cast<const f32x4*>(mean + mrow * D + col);
        mu[it][0] = live ? mp[0] : f32x4{0.f, 0.f, 0.f, 0.f};
        mu[it][1] = live ? mp[1] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int64_t ci = c0 + it * 256;
      if (ci >= total_chunks) break;
      const int64_t row = ci / CPR;
      const int col = (int)(ci % CPR) * 8;
      float v[8];
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float f = T::to_f32((uint16_t)(((uint32_t)raw[it][e / 2]) >> (16 * (e & 1))));
        if (SMOOTH) f = f - mu[it][e / 4][e % 4];      // K: smoothed
        else f = f * mul;                              // Q: times the score factor
        v[e] = f;
        amax = fmaxf(amax, fabsf(f));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      const int byte = mx_scale_byte(amax);
      codes[ci] = pack8(v, byte);
      if ((col & 31) == 0) scale[row * (D / kMx) + col / kMx] = (uint8_t)byte;
    }
  }
}

// V: one work-group per (b*Hkv, 128-key tile). The tile's 16-bit values are
// staged in LDS; each thread then quantises one (channel, 32-key block) run
// (lanes = consecutive channels: conflict-free column reads), and the codes
// leave as 64-byte channel rows of V^T and one 4*D-byte run of scales.
// (packed batches, seq set: blockIdx.y is (sequence, kv head); the
//  sequence's tiles go to its columns from kp0, tiles past its keys exit)
template <typename T, int D>
__global__ __launch_bounds__(256) void quant_v_fp4_kernel(const uint16_t* __restrict__ v, TensorGeom geo, int H,
                                                          int N, int n_pad, uint8_t* __restrict__ vt,
                                                          uint8_t* __restrict__ vscale,
                                                          const SeqSpan* __restrict__ seq) {
  constexpr int ROWS = kBkv;
  constexpr int CROW = 80;                     // bytes per staged code row (64 + 16: spreads the writes)
  __shared__ __attribute__((aligned(16))) uint16_t tile[ROWS * D];
  __shared__ __attribute__((aligned(16))) uint8_t ctile[D * CROW];
  __shared__ __attribute__((aligned(16))) uint8_t stile[D * 4];
  const int tid = threadIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh % H;
  const int tt = blockIdx.x;                   // tile
  const int t0 = tt * kBkv;
  int64_t base = (int64_t)b * geo.batch_stride + (int64_t)h * geo.head_stride;
  int n = N;
  int64_t vrow = bh;                           // V^T row block and the first column of this tile
  int64_t col0 = t0, tile0 = tt;
  if (seq) {
    const SeqSpan sp = seq[b];
    n = sp.nk;
    if (t0 >= n) return;                       // (the whole work-group)
    base += (int64_t)sp.k0 * geo.tok_stride;
    vrow = h;
    col0 = sp.kp0 + t0;
    tile0 = sp.kp0 / kBkv + tt;
  }
  // every chunk load of the tile in flight before the first LDS store
  constexpr int LOADS = ROWS * D / 8 / 256;
  static_assert(LOADS * 256 == ROWS * D / 8, "the tile's chunks tile the work-group");
  i32x4 raw[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int ci = tid + 256 * i;
    const int r = ci / (D / 8), c = (ci % (D / 8)) * 8;
    const int t = t0 + r;
    raw[i] = t < n ? *reinterpret_cast<const i32x4*>(v + base + (int64_t)t * geo.tok_stride + c) : i32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int ci = tid + 256 * i;
    const int r = ci / (D / 8), c = (ci % (D / 8)) * 8;
    *reinterpret_cast<i32x4*>(tile + r * D + c) = raw[i];
  }
  __syncthreads();
  for (int p = tid; p < D * 4; p += 256) {
    const int c = p % D, j = p / D;            // channel, 32-key block of the tile
    float x[32];
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      x[r] = T::to_f32(tile[(32 * j + r) * D + c]);
      amax = fmaxf(amax, fabsf(x[r]));
    }
    const int byte = mx_scale_byte(amax);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = x[8 * q + e];
      w[q] = pack8(y, byte);
    }
    *reinterpret_cast<i32x4*>(ctile + c * CROW + 16 * j) = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    stile[c * 4 + j] = (uint8_t)byte;
  }
  __syncthreads();
  uint8_t* dst = vt + vrow * D * (n_pad / 2) + col0 / 2;
  for (int ci = tid; ci < D * 4; ci += 256) {
    const int c = ci / 4, j = ci % 4;
    *reinterpret_cast<i32x4*>(dst + (int64_t)c * (n_pad / 2) + 16 * j) =
        *reinterpret_cast<const i32x4*>(ctile + c * CROW + 16 * j);
  }
  uint8_t* sdst = vscale + (vrow * (n_pad / kBkv) + tile0) * (D * 4);
  for (int ci = tid; ci < D * 4 / 16; ci += 256)
    *reinterpret_cast<i32x4*>(sdst + 16 * ci) = *reinterpret_cast<const i32x4*>(stile + 16 * ci);
}

// ----------------------------------------------------------------- attention
// LDS layouts. K tile: [128 keys][D/2 bytes]; a lane group of 16 reads rows
// key_perm(b, 0..15) (or 16..31) of one 16-byte chunk column, which the
// swizzle spreads over the 16 slots of a 256-byte span. V^T tile: [D
// channels][64 bytes]; a lane group reads 16 consecutive rows of one chunk
// column. Scale tiles: K [128 keys][D/32], V [D][4], unswizzled (their
// 4-byte reads touch 32 distinct banks).
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  if constexpr (D == 128) return ((row >> 2) & 1) | (((row >> 5) & 1) << 1);   // 4 chunks per row
  else return (row >> 5) & 1;                                                  // 2 chunks per row
}
template <int D>
__device__ __forceinline__ int k_lds_off(int row, int chunk) {
  return row * (D / 2) + ((chunk ^ k_swz<D>(row)) << 4);
}
__device__ __forceinline__ int v_lds_off(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

// Row m of S^T block b holds key key_perm(b, m): then every lane's 32 P values
// for one PV instruction (blocks 2u and 2u+1, lane half g) are the 32
// consecutive keys 64u + 32g + 0..31, one MX block of P, in element order, and
// V needs no permutation. Lane half g of block b holds the keys
// 32g + kb(b) + 0..15 of the tile, kb(b) = 64(b/2) + 16(b%2).
__device__ __forceinline__ int key_perm(int b, int m) {
  return 64 * (b >> 1) + 32 * ((m >> 2) & 1) + 16 * (b & 1) + 4 * (m >> 3) + (m & 3);
}
__device__ __forceinline__ constexpr int key_base(int b) { return 64 * (b >> 1) + 16 * (b & 1); }

template <int D>
struct Stage {
  static constexpr int kKRowB = D / 2;
  static constexpr int kKBytes = kBkv * kKRowB;
  static constexpr int kVBytes = D * (kBkv / 2);
  static constexpr int kSBytes = kBkv * (D / kMx);   // K scale tile == V scale tile bytes (4 D)
  static constexpr int kPass = 4 * 1024;              // one group's 16-byte-per-lane pass
  static constexpr int kKLoads = kKBytes / kPass;
  static constexpr int kVLoads = kVBytes / kPass;
  static constexpr int kSWaves = kSBytes / 256;       // waves that load a scale tile, 4 bytes per lane
  static_assert(kKLoads >= 1 && kVLoads >= 1 && kSWaves >= 1, "every load instruction is whole");
  static_assert(kPass / kKRowB >= 64 && kPass / 64 >= 16, "swizzle bits stay below the pass stride");

  static __device__ __forceinline__ void init(uint32_t& koff, uint32_t& voff, int w, int lane, int n_pad) {
    const int slot = w * 64 + lane;
    const int krow = slot / (kKRowB / 16), kchunk = slot % (kKRowB / 16);
    koff = (uint32_t)krow * kKRowB + ((kchunk ^ k_swz<D>(krow)) << 4);
    const int vrow = slot / 4, vchunk = slot % 4;
    voff = (uint32_t)vrow * (n_pad / 2) + ((vchunk ^ ((vrow >> 2) & 3)) << 4);
  }
  // K pass i of tile t: its own resource from the pass's first byte to the end
  // of the head's codes (the range check covers only the per-lane offset).
  static __device__ __forceinline__ void k_pass(const uint8_t* kbase, uint32_t kbytes, uint32_t koff, int w, int t,
                                                uint8_t* sk, int i) {
    const uint32_t start = (uint32_t)t * kKBytes + i * kPass;
    const auto r = make_rsrc(kbase + start, tail_bytes(kbytes, start));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(sk + (i * 4 + w) * 1024),
                                            16, koff, 0, 0, 0);
  }
  static __device__ __forceinline__ void k_scales(const uint8_t* ksbase, uint32_t ksbytes, int w, int lane, int t,
                                                  uint8_t* sks) {
    if (w < kSWaves) {
      const uint32_t start = (uint32_t)t * kSBytes;
      const auto r = make_rsrc(ksbase + start, tail_bytes(ksbytes, start));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(sks + w * 256), 4,
                                              (uint32_t)(w * 64 + lane) * 4, 0, 0, 0);
    }
  }
  // V^T rows are padded to whole tiles: every load lies inside its rows, and
  // the tile and pass offsets ride in the scalar offset.
  static __device__ __forceinline__ void v_pass(__amdgpu_buffer_rsrc_t rv, uint32_t voff, int w, int t, int n_pad,
                                                uint8_t* sv, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(sv + (i * 4 + w) * 1024),
                                            16, voff, t * 64 + i * 64 * (n_pad / 2), 0, 0);
  }
  static __device__ __forceinline__ void v_scales(__amdgpu_buffer_rsrc_t rvs, int w, int lane, int t, uint8_t* svs) {
    if (w < kSWaves)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rvs, (__attribute__((address_space(3))) void*)(svs + w * 256), 4,
                                              (uint32_t)(w * 64 + lane) * 4, t * kSBytes, 0, 0);
  }
};

__device__ __forceinline__ i32x4 lds16(const void* p) { return *reinterpret_cast<const i32x4*>(p); }
__device__ __forceinline__ i32x8 widen(i32x4 x) { return i32x8{x[0], x[1], x[2], x[3], 0, 0, 0, 0}; }

// D(32x32) += A(32x64) B(64x32), both MXFP4; the scale of each lane's 32
// elements is byte SA of sa (A) and byte SB of sb (B).
template <int SA, int SB>
__device__ __forceinline__ f32x16 mfma_fp4(i32x4 a, i32x4 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(a), widen(b), c, 4, 4, SA, sa, SB, sb);
}

// S^T for the 128 keys of the staged tile against this wave's 32 queries.
// qsc: this lane's Q scale bytes, its half's block of each 64-channel step in
// bytes 0 and 2 (bytes 0 only at D = 64).
// Every product chain starts from c0 (minus the running row max, one value
// per lane), so the result is S2 - m.
template <int D>
__device__ __forceinline__ void qk_tile(const uint8_t* sk, const uint8_t* sks, const i32x4* qreg, int qsc, int lane,
                                        f32x16* s, const f32x16& c0) {
  const int g = lane >> 5, m = lane & 31;
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) {
    const int row = key_perm(b, m);
    int ksc;
    if constexpr (D == 128) ksc = (int)(*reinterpret_cast<const uint32_t*>(sks + row * 4) >> (8 * g));
    else ksc = (int)(*reinterpret_cast<const uint16_t*>(sks + row * 2) >> (8 * g));
    const i32x4 k0 = lds16(sk + k_lds_off<D>(row, g));
    s[b] = mfma_fp4<0, 0>(k0, qreg[0], c0, ksc, qsc);
    if constexpr (D == 128) {
      const i32x4 k1 = lds16(sk + k_lds_off<D>(row, 2 + g));
      s[b] = mfma_fp4<2, 2>(k1, qreg[1], s[b], ksc, qsc);
    }
  }
}

template <int D>
struct RowState {
  f32x16 o[D / 32];
  float m;
  float l;
};

// P of one tile as the PV product consumes it: pk[u] = the lane's 32 E2M1
// codes of keys 64u + 32g + 0..31, psc = their E8M0 bytes (byte u).
struct PTile {
  i32x4 pk[2];
  int psc;
  float alpha;
};

// Softmax phase of one KV tile (vector ALU work only): mask, online softmax in
// the log2 domain, P~ to MXFP4. The scores arrive as S2 - m (the product chain
// started from -m, m the running row max; 0 on the first tile), so while no
// row of the wave raises its max, P~ = exp2 of them directly. A row whose max
// rises by delta takes P~ = exp2(x - delta), alpha = exp2(-delta), m += delta,
// and the chain start of the next tiles moves with it; the subtraction runs
// only on tiles where some row of the wave moved (a wave-uniform branch).
template <bool CAUSAL, bool MASK>
__device__ __forceinline__ void softmax_phase(f32x16* s, int lane, int k0, int qi, int nk, bool first, float& m,
                                              f32x16& c0, PTile& pt) {
  const int g = lane >> 5;
  if (MASK) {
    const int lim = (CAUSAL ? min(nk, qi + 1) : nk) - k0 - 32 * g;
#pragma unroll
    for (int b = 0; b < kBlocks; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (key_base(b) + e >= lim) s[b][e] = -INFINITY;
  }
  // Maximum of each 32-key P block (blocks 2u and 2u+1 of this lane): two
  // chains of 3-input maxima.
  float bm[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    float a0 = fmaxf(s[2 * u][0], s[2 * u + 1][0]);
    float a1 = fmaxf(s[2 * u][1], s[2 * u + 1][1]);
#pragma unroll
    for (int e = 2; e < 16; e += 2) {
      a0 = fmaxf(a0, fmaxf(s[2 * u][e], s[2 * u + 1][e]));
      pin(a0);
      a1 = fmaxf(a1, fmaxf(s[2 * u][e + 1], s[2 * u + 1][e + 1]));
      pin(a1);
    }
    bm[u] = fmaxf(a0, a1);
  }
  const float mt = pair_max(fmaxf(bm[0], bm[1]));        // the tile's row max, relative to m
  const float delta = first ? mt : fmaxf(mt, 0.0f);
  pt.alpha = first ? 0.0f : fast_exp2(-delta);           // (O and l are still zero on the first tile)
  // (the chain start is rewritten on every tile: kept inside the branch, its
  //  sixteen registers become a merge of two values and cost more than the
  //  moves)
  m = (first ? 0.0f : m) + delta;
#pragma unroll
  for (int e = 0; e < 16; ++e) c0[e] = -m;
  if (__builtin_amdgcn_ballot_w64(delta != 0.0f) != 0) {
#pragma unroll
    for (int b = 0; b < kBlocks; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[b][e] -= delta;
  }
  // Each block's scale from its largest P~ (the same expression as that
  // element's own P~: the block holding the row max gets exactly 1)
  int sb[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float pmax = fast_exp2(bm[u] - delta);
    const int e = mx_scale_byte(pmax);
    sb[u] = e > 1 ? e : 1;          // (a block of zeros: any scale; keep the conversion's scale normal)
  }
#pragma unroll
  for (int b = 0; b < kBlocks; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[b][e] = fast_exp2(s[b][e]);
  // E2M1 codes: dword w of pk[u] holds elements 8w..8w+7 = block 2u + w/2,
  // entries 8(w%2)..+7; the conversion divides by 2^floor(log2 scale).
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float scale = __builtin_bit_cast(float, (uint32_t)sb[u] << 23);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int b = 2 * u + (w >> 1), e0 = 8 * (w & 1);
      // (all four bytes are written: start from an input's register, which
      //  needs no clearing)
      uint32_t d = __builtin_bit_cast(uint32_t, s[b][e0 + 0]);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, s[b][e0 + 0], s[b][e0 + 1], scale, 0);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, s[b][e0 + 2], s[b][e0 + 3], scale, 1);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, s[b][e0 + 4], s[b][e0 + 5], scale, 2);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, s[b][e0 + 6], s[b][e0 + 7], scale, 3);
      pt.pk[u][w] = (int)d;
    }
  }
  pt.psc = sb[0] | (sb[1] << 8);
  pin(pt.pk[0]);
  pin(pt.pk[1]);
  pin(pt.psc);
  pin(pt.alpha);
  pin(m);
  pin(c0);
}

template <int D>
__device__ __forceinline__ void rescale_o(float alpha, RowState<D>& st) {
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) st.o[cb][e] *= alpha;
  }
}

struct NoHook {
  __device__ __forceinline__ void operator()(int) const {}
};

// PV phase of one KV tile (matrix-core work): the row sum of the quantised P,
// then O = alpha O + V^T P^T, each instruction summing 64 keys (level 1) into
// the fp32 accumulator O (level 2).
template <int D, typename Hook = NoHook>
__device__ __forceinline__ void pv_phase(const uint8_t* sv, const uint8_t* svs, int lane, const PTile& pt,
                                         RowState<D>& st, const Hook& hook = Hook{}) {
  constexpr int NT = D / 32;
  const int g = lane >> 5, n = lane & 31;
  const float alpha = pt.alpha;
  auto load_v = [&](int cb, i32x4* va, int& vsc) {
    const int row = cb * 32 + n;
    va[0] = lds16(sv + v_lds_off(row, g));
    va[1] = lds16(sv + v_lds_off(row, 2 + g));
    vsc = (int)(*reinterpret_cast<const uint32_t*>(svs + row * 4) >> (8 * g));
  };
  i32x4 va[NT][2];
  int vsc[NT];
  load_v(0, va[0], vsc[0]);
  {
    // Row sum of the quantised P: an all-ones A operand (E2M1 1.0, scale 2^0)
    // makes every row of the product the sum over the tile's keys.
    constexpr int kOnes = 0x22222222;
    const i32x4 ones = {kOnes, kOnes, kOnes, kOnes};
    f32x16 ls = mfma_fp4<0, 0>(ones, pt.pk[0], f32x16{}, 127, pt.psc);
    ls = mfma_fp4<0, 1>(ones, pt.pk[1], ls, 127, pt.psc);
    st.l = __builtin_fmaf(alpha, st.l, ls[0]);
  }
  rescale_o<D>(alpha, st);
#pragma unroll
  for (int cb = 0; cb < NT; ++cb) {
    if (cb + 1 < NT) load_v(cb + 1, va[cb + 1], vsc[cb + 1]);
    st.o[cb] = mfma_fp4<0, 0>(va[cb][0], pt.pk[0], st.o[cb], vsc[cb], pt.psc);
    hook(2 * cb);
    st.o[cb] = mfma_fp4<2, 1>(va[cb][1], pt.pk[1], st.o[cb], vsc[cb], pt.psc);
    hook(2 * cb + 1);
  }
#pragma unroll
  for (int cb = 0; cb < NT; ++cb) pin(st.o[cb]);
  pin(st.l);
}

template <int D, bool CAUSAL, typename T>
__global__ __launch_bounds__(512, 1) void attn_fp4_kernel(Fp4AttnArgs a) {
  constexpr int NT = D / 32;
  using St = Stage<D>;
  constexpr int kK = St::kKBytes, kV = St::kVBytes, kS = St::kSBytes;
  // [K0 | K1 | V0 | V1 | KS0 | KS1 | VS0 | VS1]
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kK + 2 * kV + 4 * kS];
  uint8_t* const sks0 = smem + 2 * kK + 2 * kV;
  uint8_t* const svs0 = sks0 + 2 * kS;

  // Work decomposition, as in the INT8 kernel. Dense batches: XCD-contiguous
  // (head, query pair) ranges, causal pairs longest first. Packed batches: XCD
  // x takes heads [x Hq/8, (x+1) Hq/8) of every sequence and walks the work
  // list of query pairs (sequence by sequence, each from its longest pair).
  int bh, qp;
  if (a.seq) {
    int heads = a.Hq, h0 = 0, j = blockIdx.x;
    if ((a.Hq & 7) == 0) {
      heads = a.Hq >> 3;
      h0 = (blockIdx.x & 7) * heads;
      j = blockIdx.x >> 3;
    }
    const int qpi = j / heads;
    const int sb = qpi < a.n_owner ? a.qp_owner[qpi] : -1;
    if (sb < 0) return;                                          // past the work list
    qp = (a.seq[sb].nq + 2 * kBq - 1) / (2 * kBq) - 1 - (qpi - a.seq[sb].qp0);
    bh = sb * a.Hq + h0 + j % heads;
  } else {
    const int n_qp = (a.Nq + 2 * kBq - 1) / (2 * kBq);
    const int total = n_qp * a.B * a.Hq;
    int id = blockIdx.x;
    if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
    bh = id / n_qp;
    qp = id % n_qp;
    if (CAUSAL) qp = n_qp - 1 - qp;
  }
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int bhk = b * a.Hkv + hk;
  // Rows of this work-group's queries and keys in the codes ([B*H][N] or, packed,
  // [H][total] from the sequence's first token), its V^T column and scale-tile
  // offsets, and its first output token.
  int nq = a.Nq, nk = a.Nk;
  int64_t q_row = (int64_t)bh * a.Nq, k_row = (int64_t)bhk * a.Nk;
  int64_t v_off = (int64_t)bhk * a.D * (a.n_pad / 2), v_len = (int64_t)a.D * (a.n_pad / 2);
  int64_t vs_tile = (int64_t)bhk * (a.n_pad / kBkv), vs_tiles = a.n_pad / kBkv;
  int64_t o_tok = 0;
  if (a.seq) {
    const SeqSpan sp = a.seq[b];
    nq = sp.nq;
    nk = sp.nk;
    if (2 * qp * kBq >= nq) return;                              // no rows of this sequence here
    q_row = (int64_t)h * a.total_q + sp.q0;
    k_row = (int64_t)hk * a.total_k + sp.k0;
    v_off = (int64_t)hk * a.D * (a.n_pad / 2) + sp.kp0 / 2;
    v_len = (int64_t)a.D * (a.n_pad / 2) - sp.kp0 / 2;
    vs_tile = (int64_t)hk * (a.n_pad / kBkv) + sp.kp0 / kBkv;
    vs_tiles = a.n_pad / kBkv - sp.kp0 / kBkv;
    o_tok = sp.q0;
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);
  const int wv4 = __builtin_amdgcn_readfirstlane(wave & 3);
  const int g = lane >> 5;
  const int qt = 2 * qp + grp;
  const int qi = qt * kBq + (wave & 3) * 32 + (lane & 31);

  // Q operand: the lane's query row, channels 64kk + 32g + 0..31; its scale
  // bytes (blocks 2kk + g) shifted into bytes 0 and 2.
  i32x4 qreg[D / 64];
  int qsc;
  {
    const auto rq = make_rsrc(a.q4 + q_row * (D / 2), (uint32_t)nq * (D / 2));
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) qreg[kk] = buf_load16(rq, (uint32_t)qi * (D / 2) + 32 * kk + 16 * g);
    const auto rqs = make_rsrc(a.q_sc + q_row * (D / kMx), (uint32_t)nq * (D / kMx));
    if constexpr (D == 128) qsc = __builtin_amdgcn_raw_buffer_load_b32(rqs, (uint32_t)qi * 4, 0, 0) >> (8 * g);
    else qsc = (__builtin_amdgcn_raw_buffer_load_b16(rqs, (uint32_t)qi * 2, 0, 0) >> (8 * g)) & 0xff;
  }
  auto tiles_for = [&](int q_tile) {
    const int kv_end = CAUSAL ? min(nk, (q_tile + 1) * kBq) : nk;
    return (kv_end + kBkv - 1) / kBkv;
  };
  const bool grp_live = qt * kBq < nq;
  const int n_g = grp_live ? tiles_for(qt) : 0;
  const int n_wg = ((2 * qp + 1) * kBq < nq) ? tiles_for(2 * qp + 1) : tiles_for(2 * qp);

  const uint8_t* kbase = a.k4 + k_row * (D / 2);
  const uint32_t kbytes = (uint32_t)nk * (D / 2);
  const uint8_t* ksbase = a.k_sc + k_row * (D / kMx);
  // The K scales are staged in 4-byte words. At d = 64 a key has two scale
  // bytes, so with an odd key count the last key shares its word with two bytes
  // past the range, and a range check on that word would return it as zero:
  // the range is rounded up to whole words (the two extra bytes land in the
  // slot of key nk, which is masked; the buffers hold them, see sage.h).
  const uint32_t ksbytes = ((uint32_t)nk * (D / kMx) + 3u) & ~3u;
  const auto rv = make_rsrc(a.v4 + v_off, (uint32_t)v_len);
  const auto rvs = make_rsrc(a.v_sc + vs_tile * (kBkv * D / kMx), (uint32_t)(vs_tiles * (kBkv * D / kMx)));
  uint32_t koff, voff;
  St::init(koff, voff, wv4, lane, a.n_pad);

  // Group 0 stages K(0) before the first phase.
  if (grp == 0 && n_wg > 0) {
#pragma unroll
    for (int i = 0; i < St::kKLoads; ++i) St::k_pass(kbase, kbytes, koff, wv4, 0, smem, i);
    St::k_scales(ksbase, ksbytes, wv4, lane, 0, sks0);
  }
  wait_loads_barrier();

  RowState<D> st;
#pragma unroll
  for (int cb = 0; cb < NT; ++cb) st.o[cb] = f32x16{};
  st.m = 0.0f;
  st.l = 0.0f;
  f32x16 s[kBlocks];
  PTile pt;
  // The start of every product chain, -m (opaque, so that it is not rebuilt
  // per tile).
  f32x16 c0 = {};
  pin(c0);

  auto kbuf = [&](int p) { return smem + p * kK; };
  auto vbuf = [&](int p) { return smem + 2 * kK + p * kV; };
  auto ksbuf = [&](int p) { return sks0 + p * kS; };
  auto vsbuf = [&](int p) { return svs0 + p * kS; };

  auto loads_k = [&](auto par, int t) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    if (t + 1 < n_wg) {
#pragma unroll
      for (int i = 0; i < St::kKLoads; ++i) St::k_pass(kbase, kbytes, koff, wv4, t + 1, kbuf(1 - P), i);
      St::k_scales(ksbase, ksbytes, wv4, lane, t + 1, ksbuf(1 - P));
    }
  };
  auto loads_v = [&](auto par, int t) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    if (t < n_wg) {
#pragma unroll
      for (int i = 0; i < St::kVLoads; ++i) St::v_pass(rv, voff, wv4, t, a.n_pad, vbuf(P), i);
      St::v_scales(rvs, wv4, lane, t, vsbuf(P));
    }
  };
  auto loads_k_rt = [&](int t) __attribute__((always_inline)) {
    if (t & 1) loads_k(std::integral_constant<int, 1>{}, t); else loads_k(std::integral_constant<int, 0>{}, t);
  };
  auto loads_v_rt = [&](int t) __attribute__((always_inline)) {
    if (t & 1) loads_v(std::integral_constant<int, 1>{}, t); else loads_v(std::integral_constant<int, 0>{}, t);
  };
  auto x_bufs = [&](int P, bool do_pv, bool do_qk, const auto& hook) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    if (do_pv) pv_phase<D>(vbuf(1 - P), vsbuf(1 - P), lane, pt, st, hook);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    if (do_qk) qk_tile<D>(kbuf(P), ksbuf(P), qreg, qsc, lane, s, c0);
  };
  auto x_phase = [&](auto par, int t, bool do_pv, bool do_qk) __attribute__((always_inline)) {
    x_bufs(decltype(par)::value, do_pv, do_qk, NoHook{});
  };
  // Steady pairs: this group's loads issued one after each PV product.
  auto x_phase_loading = [&](auto par, int t) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    auto hook = [&](int j) __attribute__((always_inline)) {
      if (grp == 0) {
        if (t + 1 < n_wg) {
          if (j < St::kKLoads) St::k_pass(kbase, kbytes, koff, wv4, t + 1, kbuf(1 - P), j);
          if (j == St::kKLoads) St::k_scales(ksbase, ksbytes, wv4, lane, t + 1, ksbuf(1 - P));
        }
      } else {
        if (t < n_wg) {
          if (j < St::kVLoads) St::v_pass(rv, voff, wv4, t, a.n_pad, vbuf(P), j);
          if (j == St::kVLoads) St::v_scales(rvs, wv4, lane, t, vsbuf(P));
        }
      }
    };
    x_bufs(P, true, true, hook);
  };
  auto x_phase_rt = [&](int t, bool do_pv, bool do_qk) __attribute__((always_inline)) {
    x_bufs(t & 1, do_pv, do_qk, NoHook{});
  };
  auto y_phase = [&](int t, auto masked) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(0);
    softmax_phase<CAUSAL, decltype(masked)::value>(s, lane, t * kBkv, qi, nk, t == 0, st.m, c0, pt);
  };
  static_assert(2 * NT >= St::kKLoads + 1 && 2 * NT >= St::kVLoads + 1, "one PV product per load instruction");
  run_pingpong(grp, n_g, n_wg, x_phase, x_phase_loading, x_phase_rt, y_phase, loads_k, loads_v, loads_k_rt,
               loads_v_rt);
  __builtin_amdgcn_s_setprio(0);

  // Epilogue: normalise, round, store in the caller's layout (the block scales
  // entered the products; no V scale is left to apply).
  if (qi < nq) {
    const float l = st.l;
    const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.o) + (int64_t)b * a.ogeo.batch_stride +
                     (int64_t)h * a.ogeo.head_stride + (o_tok + qi) * a.ogeo.tok_stride;
#pragma unroll
    for (int cb = 0; cb < NT; ++cb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = cb * 32 + 8 * j + 4 * g;
        uint32_t w[2];
#pragma unroll
        for (int i = 0; i < 4; i += 2)
          w[i / 2] = (uint32_t)T::from_f32(st.o[cb][4 * j + i] * inv_l) |
                     ((uint32_t)T::from_f32(st.o[cb][4 * j + i + 1] * inv_l) << 16);
        *reinterpret_cast<i32x2*>(orow + ch) = i32x2{(int)w[0], (int)w[1]};
      }
    }
  }
}

}  // namespace fp4

// ----------------------------------------------------------------- launchers
// Work-groups of the row quantisation: one per 1024 chunks, capped (the kernel
// strides over the rest).
static unsigned row_wgs(int64_t chunks) {
  const int64_t n = (chunks + 1023) / 1024;
  return (unsigned)(n < (int64_t(1) << 20) ? n : (int64_t(1) << 20));
}

// Packed batches (a.seq set): the Q and K rows are quantised as one [H][total]
// batch (K's mean looked up per token), V per (sequence, kv head) over the
// longest sequence's tiles.
template <typename T, int D>
static hipError_t launch_quant_fp4_t(const Fp4QuantArgs& a, hipStream_t st) {
  hipError_t e = hipSuccess;
  const bool packed = a.seq != nullptr;
  if (a.Nk > 0 && (!packed || a.total_k > 0)) {
    e = launch_k_mean(a.k, a.kgeo, a.B, a.Hkv, a.Nk, a.D, a.bf16, a.ksum_part, a.k_mean, st, a.seq);
    if (e != hipSuccess) return e;
    const int kn = packed ? a.total_k : a.Nk;
    const int64_t kchunks = (int64_t)(packed ? 1 : a.B) * a.Hkv * kn * (D / 8);
    hipLaunchKernelGGL((fp4::quant_rows_fp4_kernel<T, D, true>), dim3(row_wgs(kchunks)),
                       dim3(256), 0, st, (const uint16_t*)a.k, a.kgeo, a.Hkv, kn, kchunks, a.k_mean, 1.0f,
                       (uint32_t*)a.k_codes, a.k_scale, a.seq, a.B);
  }
  if (a.Nq > 0 && (!packed || a.total_q > 0)) {
    const int qn = packed ? a.total_q : a.Nq;
    const int64_t qchunks = (int64_t)(packed ? 1 : a.B) * a.Hq * qn * (D / 8);
    hipLaunchKernelGGL((fp4::quant_rows_fp4_kernel<T, D, false>), dim3(row_wgs(qchunks)),
                       dim3(256), 0, st, (const uint16_t*)a.q, a.qgeo, a.Hq, qn, qchunks, (const float*)nullptr,
                       a.q_mul, (uint32_t*)a.q_codes, a.q_scale, (const SeqSpan*)nullptr, 0);
  }
  const int v_tiles = !packed ? a.n_pad / kBkv : a.total_k > 0 ? (a.Nk + kBkv - 1) / kBkv : 0;
  if (v_tiles > 0)
    hipLaunchKernelGGL((fp4::quant_v_fp4_kernel<T, D>), dim3(v_tiles, a.B * a.Hkv), dim3(256), 0, st,
                       (const uint16_t*)a.v, a.vgeo, a.Hkv, a.Nk, a.n_pad, a.v_codes, a.v_scale, a.seq);
  return hipGetLastError();
}

hipError_t launch_quant_fp4(const Fp4QuantArgs& a, hipStream_t st) {
  if (a.bf16) return a.D == 64 ? launch_quant_fp4_t<BF16, 64>(a, st) : launch_quant_fp4_t<BF16, 128>(a, st);
  return a.D == 64 ? launch_quant_fp4_t<F16, 64>(a, st) : launch_quant_fp4_t<F16, 128>(a, st);
}

template <int D, bool CAUSAL, typename T>
static hipError_t launch_attn_fp4_t(const Fp4AttnArgs& a, hipStream_t st) {
  const int n_qp = (a.Nq + 2 * fp4::kBq - 1) / (2 * fp4::kBq);
  const int grid = a.seq ? a.n_owner * a.Hq : n_qp * a.B * a.Hq;   // packed: the work list per head
  hipLaunchKernelGGL((fp4::attn_fp4_kernel<D, CAUSAL, T>), dim3(grid), dim3(64 * fp4::kWaves), 0, st, a);
  return hipGetLastError();
}

template <int D, typename T>
static hipError_t launch_attn_fp4_c(const Fp4AttnArgs& a, hipStream_t st) {
  return a.causal ? launch_attn_fp4_t<D, true, T>(a, st) : launch_attn_fp4_t<D, false, T>(a, st);
}

hipError_t launch_attn_fp4(const Fp4AttnArgs& a, hipStream_t st) {
  if (a.Nq == 0) return hipSuccess;
  if (a.bf16) return a.D == 64 ? launch_attn_fp4_c<64, BF16>(a, st) : launch_attn_fp4_c<128, BF16>(a, st);
  return a.D == 64 ? launch_attn_fp4_c<64, F16>(a, st) : launch_attn_fp4_c<128, F16>(a, st);
}

}  // namespace sage
